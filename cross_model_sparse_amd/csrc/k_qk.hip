// Compression from the sender's Q and K, without a dense map.
//
// MapFlow's compressor computes block statistics and then picks blocks
// without first laying out the complete dense attention matrix (article
// aitest123.com/news/zaoi86, third section, first component).  The sender's
// causal map is the softmax of its scores, so with the per-row log-sum-exp
//     A[h][i][j] = exp(scale[h] * q_h,i . k_h,j - lse[h][i]),   j <= i,
// and the block masses and the kept tiles follow from Q, K and lse:
//   * k_lse_*      lse[h][i] (online maximum and sum over the causal keys);
//   * k_mass_qk_*  per-head fp32 sums of A over (16-row tile, column block),
//                  into a workspace; k_mass_reduce adds tiles and heads in
//                  fp64 in a fixed order and divides by H_s;
//   * k_gather_qk_* the kept tiles, recomputed and rounded once.
// Exponentials run in base 2 on scores pre-multiplied by log2(e).
//
// Matrix-core kernels (fp16/bf16, d in {64, 128}; block mass and gather also
// need B >= 32): a 32 x 32 score tile is S^T = K Q^T on MFMA 32x32x16 with K
// rows as the A operand (m = key, k = head dim) and Q rows as the B operand
// (k = head dim, n = query row), so both load straight from their row-major
// layout and each lane owns one query row: lane l holds row l%32 and the keys
// 8(e/4) + 4(l/32) + e%4, e = 0..15, of the tile.  Plain kernels cover every
// other case (fp32, d = 64/128 with B = 16).
#include "mf_internal.h"

#include <algorithm>
#include <type_traits>

namespace {

using namespace mfd;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kRT = 16;                         // rows per partial tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;

// 2^x with the hardware instruction alone: results below 2^-126 may flush to
// zero, which is harmless inside a sum of terms that include a 1 (log-sum-exp),
// in probabilities compared at 1e-5 relative (block mass) and in stored tile
// values (an absolute error below 2^-126)
__device__ __forceinline__ float exp2_sum(float x) { return __builtin_amdgcn_exp2f(x); }

// x of lane l ^ 32 (the other half of the wavefront), by one register swap
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ f16x8 as_f16x8(const u32x4& v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

template <bool kBF16>
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  if constexpr (kBF16)
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a), as_f16x8(b), c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// plain kernels
// ---------------------------------------------------------------------------

template <class TT>
__device__ __forceinline__ float dot_row(const typename TT::S* a, const typename TT::S* b, int d) {
  float s = 0.f;
  for (int t = 0; t < d; ++t) s += TT::tof(a[t]) * TT::tof(b[t]);
  return s;
}

// one thread per (head, row)
template <class TT>
__global__ __launch_bounds__(256) void k_lse_plain(
    const typename TT::S* __restrict__ Q, const typename TT::S* __restrict__ K, int H_s,
    int H_ks, int N, int d, const float* __restrict__ scale, float* __restrict__ lse) {
  const int h = blockIdx.y;
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= N) return;
  const int g = h / (H_s / H_ks);
  const typename TT::S* q = Q + ((int64_t)h * N + i) * d;
  const typename TT::S* kb = K + (int64_t)g * N * d;
  const float sc = scale[h] * kLog2e;
  float m = -INFINITY, l = 0.f;
  for (int j = 0; j <= i; ++j) {
    const float x = dot_row<TT>(q, kb + (int64_t)j * d, d) * sc;
    if (x > m) { l = l * exp2f(m - x) + 1.f; m = x; }
    else l += exp2f(x - m);
  }
  lse[(int64_t)h * N + i] = (m + log2f(l)) * kLn2;
}

// one workgroup per (16-row tile, head); thread t sums column blocks t, t+256, ...
template <class TT>
__global__ __launch_bounds__(256) void k_mass_qk_plain(
    const typename TT::S* __restrict__ Q, const typename TT::S* __restrict__ K, int H_s,
    int H_ks, int N, int d, int B, const float* __restrict__ scale,
    const float* __restrict__ lse, float* __restrict__ part) {
  const int rt = blockIdx.x, h = blockIdx.y;
  const int T = (N + B - 1) / B;
  const int NRT = (N + kRT - 1) / kRT;
  const int g = h / (H_s / H_ks);
  const int i0 = rt * kRT, i1 = min(N, i0 + kRT);
  const int I = i0 / B;
  const float sc = scale[h] * kLog2e;
  for (int J = threadIdx.x; J <= I; J += 256) {
    float acc = 0.f;
    for (int i = i0; i < i1; ++i) {
      const typename TT::S* q = Q + ((int64_t)h * N + i) * d;
      const float l2 = lse[(int64_t)h * N + i] * kLog2e;
      const int j1 = min(min(N, (J + 1) * B), i + 1);
      for (int j = J * B; j < j1; ++j)
        acc += exp2f(dot_row<TT>(q, K + ((int64_t)g * N + j) * d, d) * sc - l2);
    }
    part[((int64_t)h * NRT + rt) * T + J] = acc;
  }
}

// mass[I][J] = (1/H_s) sum_h sum_{tiles of I} part, fp64 in a fixed order.
// Workgroup (I, 64-column chunk); thread (c = t % 64, q = t / 64) adds, for
// column J = 64 chunk + c, heads q, q+4, q+8, ... and every 16-row tile of
// block row I in (head, tile) order; the four partial sums are then added in
// the order q = 0, 1, 2, 3.  The result depends on nothing but the inputs.
__global__ __launch_bounds__(256) void k_mass_reduce(const float* __restrict__ part, int H_s,
                                                     int N, int B, float* __restrict__ mass) {
  __shared__ double red[4][64];
  const int T = (N + B - 1) / B;
  const int NRT = (N + kRT - 1) / kRT;
  const int I = blockIdx.x;
  const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int J = blockIdx.y * 64 + c;
  const int rt0 = I * (B / kRT), rt1 = min(NRT, (I + 1) * (B / kRT));
  double s = 0.0;
  if (J <= I && J < T)
    for (int h = q; h < H_s; h += 4)
      for (int rt = rt0; rt < rt1; ++rt) s += (double)part[((int64_t)h * NRT + rt) * T + J];
  red[q][c] = s;
  __syncthreads();
  if (q == 0 && J < T) {
    const double t = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
    mass[(int64_t)I * T + J] = J <= I ? (float)(t / (double)H_s) : 0.f;
  }
}

// Per-head block sums from the (m, e) pairs of k_lse_mfma<.., true>:
//   sums[h][I(I+1)/2 + J] = sum_{i in I} e 2^(m - lse2_i).
// Workgroup (head, block row I), heaviest rows first, eight wavefronts;
// wavefront w takes columns J = w, w + 8, ..., two at a time so that their
// loads overlap.  Lane t holds the pairs t, t + 64 of the block's B rows
// (contiguous loads); the lanes' terms are added by a fixed fp32 butterfly
// (at most 128 terms, each at most B: relative error about 2^-21), so the
// result is bit-reproducible.  launch_block_mass_heads then adds the heads in
// fp64 in a fixed order.
constexpr int kMfpThreads = 512;
__global__ __launch_bounds__(kMfpThreads) void k_mass_from_partials(const float2* __restrict__ part,
                                                                    const float* __restrict__ lse,
                                                                    int H_s, int N, int B,
                                                                    float* __restrict__ sums) {
  constexpr int kW = kMfpThreads / 64;
  const int T = (N + B - 1) / B;
  const int h = blockIdx.x % H_s;
  const int I = T - 1 - (int)(blockIdx.x / H_s);
  const int rows = min(B, N - I * B);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* lh = lse + (int64_t)h * N + (int64_t)I * B;
  // pair t of a block is row t; lane takes t = lane and t = lane + 64
  constexpr int NP = 2;
  float l2[NP];
  bool ok[NP];
#pragma unroll
  for (int k = 0; k < NP; ++k) {
    const int r = lane + 64 * k;
    ok[k] = r < rows;
    l2[k] = ok[k] ? lh[r] * kLog2e : 0.f;
  }
  const float2* ph = part + (int64_t)h * B * T * (T + 1) / 2 + (int64_t)B * I * (I + 1) / 2;
  float* out = sums + (int64_t)h * T * (T + 1) / 2 + (int64_t)I * (I + 1) / 2;
  auto term = [&](const float2& v, int k) {
    return (ok[k] && v.x > -INFINITY) ? v.y * exp2_sum(v.x - l2[k]) : 0.f;
  };
  auto tree = [](float s) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
    return s;
  };
  for (int J = wave; J <= I; J += 2 * kW) {
    const int J2 = J + kW;
    const bool has2 = J2 <= I;
    const float2* p1 = ph + (int64_t)J * B;
    const float2* p2 = ph + (int64_t)(has2 ? J2 : J) * B;
    float2 a[NP], b[NP];
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      a[k] = ok[k] ? p1[lane + 64 * k] : make_float2(-INFINITY, 0.f);
      b[k] = ok[k] ? p2[lane + 64 * k] : make_float2(-INFINITY, 0.f);
    }
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int k = 0; k < NP; ++k) {
      s1 += term(a[k], k);
      s2 += term(b[k], k);
    }
    s1 = tree(s1);
    s2 = tree(s2);
    if (lane == 0) {
      out[J] = s1;
      if (has2) out[J2] = s2;
    }
  }
}

// block row of kept block k: the last I with row_ptr[I] <= k
__device__ __forceinline__ int row_of(const int32_t* row_ptr, int T, int64_t k) {
  int lo = 0, hi = T - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if ((int64_t)row_ptr[mid] <= k) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// grid-stride over (kept block, head); one thread per tile element
template <class TT>
__global__ __launch_bounds__(256) void k_gather_qk_plain(
    const typename TT::S* __restrict__ Q, const typename TT::S* __restrict__ K, int H_s,
    int H_ks, int N, int d, int B, const float* __restrict__ scale,
    const float* __restrict__ lse, const int32_t* __restrict__ row_ptr,
    const int32_t* __restrict__ kept, int64_t cap, int32_t* __restrict__ col_idx,
    typename TT::S* __restrict__ vals) {
  const int T = (N + B - 1) / B;
  const int64_t nnzb = row_ptr[T];
  if (nnzb > cap) return;
  const int G = H_s / H_ks;
  for (int64_t u = blockIdx.x; u < nnzb * H_s; u += gridDim.x) {
    const int64_t k = u / H_s;
    const int h = (int)(u - k * H_s);
    const int I = row_of(row_ptr, T, k);
    const int J = kept[(int64_t)I * T + (k - row_ptr[I])];
    if (h == 0 && threadIdx.x == 0) col_idx[k] = J;
    const float sc = scale[h] * kLog2e;
    for (int e = threadIdx.x; e < B * B; e += 256) {
      const int r = e / B, c = e % B;
      const int i = I * B + r, j = J * B + c;
      float v = 0.f;
      if (i < N && j <= i) {
        const float x = dot_row<TT>(Q + ((int64_t)h * N + i) * d,
                                    K + ((int64_t)(h / G) * N + j) * d, d) * sc;
        v = exp2f(x - lse[(int64_t)h * N + i] * kLog2e);
      }
      vals[((k * H_s + h) * B + r) * B + c] = TT::fromf(v);
    }
  }
}

// ---------------------------------------------------------------------------
// matrix-core kernels
// ---------------------------------------------------------------------------

constexpr int kQkHalfWaves = 4;                 // wavefronts per half workgroup
constexpr int kQkHalf = 64 * kQkHalfWaves;      // threads per half
constexpr int kQkThreads = 2 * kQkHalf;
constexpr int kQkRows = 32 * kQkHalfWaves;      // query rows per workgroup

// LDS K tile: 32 key rows of D elements, each row padded by 16 bytes so that
// 16-byte reads of 16 consecutive rows hit distinct banks.
template <int D>
struct KTile {
  static constexpr int kRowBytes = D * 2 + 16;
  static constexpr int kBytes = 32 * kRowBytes;
};

// Shared walk of lse and mass over one group of kQkRows query rows of head h.
// The workgroup's two halves take the same rows (wavefront w of a half: rows
// q0 = R0 + 32w .. +31) and split the causal key tiles: half 0 walks tiles
// [0, nfirst), half 1 tiles [nfirst, nkt), with nfirst a multiple of `align`,
// so the longest walk is half as long.  K tiles of 32 keys are staged through
// LDS in two buffers per half, loaded from a uniform base with fixed
// per-thread offsets.
//
// Software pipeline: while a wavefront exponentiates the scores of tile kt,
// it issues the MFMA chain of tile kt+1, one MFMA between each group of
// exponentials (body(kt, c, mf) must call mf(0) .. mf(NKS-1) once each, in
// order), so the matrix cores and the vector ALU work at the same time
// within one wavefront.  At step kt the MFMAs read tile kt+1 from one buffer
// and tile kt+2 is stored into the other, whose last reader (tile kt) was
// done before the previous barrier; tile kt+3 is in flight in registers.
// With `negate` the query operand's signs are flipped, so that a negative
// score scale becomes a non-negative one on negated products.
template <bool kBF16, int D, class Body>
__device__ __forceinline__ void qk_walk(const unsigned short* __restrict__ Q,
                                        const unsigned short* __restrict__ K, int h, int g,
                                        int N, int R0, int align, bool negate,
                                        unsigned char* smem, Body&& body) {
  constexpr int NKS = D / 16;                   // MFMA K steps
  constexpr int kRowU4 = D / 8;                 // 16-byte pieces per row
  constexpr int NP = 32 * kRowU4 / kQkHalf;     // pieces of a tile per thread
  static_assert(NP * kQkHalf == 32 * kRowU4, "tile pieces must divide evenly");
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int hf = wave / kQkHalfWaves;           // half of the workgroup
  const int ht = threadIdx.x % kQkHalf;         // thread within the half
  const int q0 = R0 + 32 * (wave % kQkHalfWaves);
  unsigned char* hs = smem + hf * 2 * KTile<D>::kBytes;
  // B operand: this lane's query row (clamped), head-dim chunks 8(l/32) + 16s
  u32x4 qop[NKS];
  {
    const int row = min(q0 + (lane & 31), N - 1);
    const unsigned short* qr = Q + ((int64_t)h * N + row) * D + 8 * (lane >> 5);
    const unsigned flip = negate ? 0x80008000u : 0u;   // sign bits of both 16-bit halves
#pragma unroll
    for (int s = 0; s < NKS; ++s) {
      qop[s] = *reinterpret_cast<const u32x4*>(qr + 16 * s);
      qop[s] ^= flip;
    }
  }
  const int last_row = min(N, R0 + kQkRows) - 1;
  const int nkt = last_row / 32 + 1;            // key tiles 0..nkt-1
  const int nfirst = min(nkt, ((nkt + 1) / 2 + align - 1) / align * align);
  const int t0 = hf ? nfirst : 0;
  const int cnt = hf ? nkt - nfirst : nfirst;   // tiles of this half
  const int nit = nfirst;                       // steps of both halves (nfirst >= nkt - nfirst)
  // piece pc = ht + kQkHalf * n: key row pc / kRowU4, 16-byte chunk pc % kRowU4;
  // per-thread offsets are fixed, the tile base is uniform
  const unsigned short* Kg = K + (int64_t)g * N * D;
  auto load_tile = [&](int kt, u32x4* v) {
    if (kt * 32 + 31 < N) {
      const unsigned short* base = Kg + (int64_t)kt * 32 * D;
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        const int pc = ht + kQkHalf * n;
        v[n] = *reinterpret_cast<const u32x4*>(base + (pc / kRowU4) * D + 8 * (pc % kRowU4));
      }
    } else {                                     // last, partial tile: clamp the key row
#pragma unroll
      for (int n = 0; n < NP; ++n) {
        const int pc = ht + kQkHalf * n;
        const int key = min(kt * 32 + pc / kRowU4, N - 1);
        v[n] = *reinterpret_cast<const u32x4*>(Kg + (int64_t)key * D + 8 * (pc % kRowU4));
      }
    }
  };
  auto store_tile = [&](int buf, const u32x4* v) {
#pragma unroll
    for (int n = 0; n < NP; ++n) {
      const int pc = ht + kQkHalf * n;
      *reinterpret_cast<u32x4*>(hs + buf * KTile<D>::kBytes + (pc / kRowU4) * KTile<D>::kRowBytes +
                                16 * (pc % kRowU4)) = v[n];
    }
  };
  // this lane's K operand piece s (row lane%32, chunk 16(lane/32) + 32 s) of buffer b
  auto read_k = [&](int buf, int s) -> u32x4 {
    const unsigned char* kb = hs + buf * KTile<D>::kBytes + (lane & 31) * KTile<D>::kRowBytes + 16 * (lane >> 5);
    return *reinterpret_cast<const u32x4*>(kb + 32 * s);
  };
  // tile to load for step it of this half (any valid tile once the half is done)
  auto tile_at = [&](int it) { return min(t0 + min(it, max(cnt - 1, 0)), nkt - 1); };
  // step it (P = it % 2): cur holds the scores of tile t0+it; the MFMAs of
  // tile t0+it+1 (buffer P^1) go into nxt while body exponentiates cur; sa
  // holds tile it+2 (stored into buffer P at the end), tile it+3 is loaded
  // into sb.  Loads are issued on every step so that the wait before the LDS
  // store counts only the older tile's loads.  Steps alternate register sets
  // and buffers, so nothing is copied and LDS offsets are fixed; both halves
  // take the same number of barriers.  The MFMAs of a tile past the half's
  // end read a valid buffer and are unused.
  auto step = [&](auto pc, int it, const f32x16& cur, f32x16& nxt, u32x4* sa, u32x4* sb) {
    constexpr int P = decltype(pc)::value;
    const int kt = t0 + it;
    load_tile(tile_at(it + 3), sb);
    // the K operand pieces go through two registers, each read one MFMA ahead
    u32x4 kc = read_k(P ^ 1, 0);
    nxt = f32x16{};
    auto mf = [&](int s) {
      const u32x4 kn = s + 1 < NKS ? read_k(P ^ 1, s + 1) : kc;
      nxt = mfma32<kBF16>(kc, qop[s], nxt);
      kc = kn;
    };
    if (it < cnt && kt * 32 <= q0 + 31 && q0 < N) {   // some key of the tile is causal for these rows
      body(kt, cur, mf);
    } else {
#pragma unroll
      for (int s = 0; s < NKS; ++s) mf(s);
    }
    if (it + 1 < nit) {
      store_tile(P, sa);
      __syncthreads();
    }
  };
  u32x4 stage_a[NP], stage_b[NP];
  load_tile(tile_at(0), stage_a);
  store_tile(0, stage_a);
  load_tile(tile_at(1), stage_a);
  store_tile(1, stage_a);
  load_tile(tile_at(2), stage_a);
  __syncthreads();
  f32x16 ca = {}, cb;
#pragma unroll
  for (int s = 0; s < NKS; ++s) ca = mfma32<kBF16>(read_k(0, s), qop[s], ca);
  __syncthreads();                              // buffer 0 is refilled in step 0
  for (int it = 0; it < nit; it += 2) {
    step(std::integral_constant<int, 0>{}, it, ca, cb, stage_a, stage_b);
    if (it + 1 < nit) step(std::integral_constant<int, 1>{}, it + 1, cb, ca, stage_b, stage_a);
  }
}

// Work item of a workgroup of the lse / mass kernels: row group grp of head
// h.  The longest groups (most causal key tiles) of every head come first, so
// the workgroups that share a CU mix long and short walks; workgroups with
// equal b mod 8 (one XCD) take the same heads and share their K rows in L2.
__device__ __forceinline__ void qk_item(int ngrp, int H_s, int& h, int& grp) {
  const int b = blockIdx.x;
  h = b % H_s;
  grp = ngrp - 1 - b / H_s;
}

// key of output element e of this lane within a tile
__device__ __forceinline__ int tile_key(int lane, int e) { return 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3); }

// The MFMA calls and exponential groups of a fully causal tile alternate as
// written: sched_barrier keeps the compiler from gathering the MFMAs.
#define MF_PIN() __builtin_amdgcn_sched_barrier(0)

// kMass: the same walk also leaves, for every row i and causal column block J,
// the pair (m, e) with e = sum over the block's keys j of 2^(x_ij - m) and m
// the row's running maximum after the block (log2 units), in
// part[h][B (I(I+1)/2 + J) + i - I B], I = i / B (rows fastest, so a
// wavefront's 32 rows store one contiguous run).  The block's share of
// the softmax row is then e 2^(m - lse2_i), and k_mass_from_partials forms
// the block masses from these pairs and lse without a second pass over the
// scores.  Both halves of the workgroup split the key tiles at a column-block
// boundary, so each block's pair comes from one half.
template <bool kBF16, int D, bool kMass>
__global__ __launch_bounds__(kQkThreads, 4) void k_lse_mfma(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K, int H_s,
    int H_ks, int N, const float* __restrict__ scale, float* __restrict__ lse, int B,
    float2* __restrict__ part) {
  constexpr int NKS = D / 16;
  constexpr int EPS = 16 / NKS;                  // scores per MFMA step
  __shared__ __align__(16) unsigned char smem[4 * KTile<D>::kBytes];
  __shared__ float2 half1[kQkRows];              // (max, sum) of half 1 per row
  const int ngrp = (N + kQkRows - 1) / kQkRows;
  int h, grp;
  qk_item(ngrp, H_s, h, grp);
  const int g = h / (H_s / H_ks);
  const float sc_raw = scale[h] * kLog2e;
  const bool neg = sc_raw < 0.f;                 // products negated by the walk
  const float sc = fabsf(sc_raw);
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int R0 = grp * kQkRows;
  const int q0 = R0 + 32 * (wave % kQkHalfWaves);
  const int row = q0 + (lane & 31);
  float m = -INFINITY, l = 0.f;                  // running maximum and sum, log2 units
  float lb = 0.f;                                // kMass: this block's sum, relative to m
  const int tpb = kMass ? B / 32 : 1;            // key tiles per column block
  // kMass: store the pair of block J.  Lanes l and l+32 hold the same row over
  // different keys; their pairs are merged through one half-wave register
  // swap (v_permlane32_swap, no LDS round trip).  This wavefront's rows all
  // lie in block row I (B >= 32, q0 a multiple of 32); the address is formed
  // here from a wave-uniform base and a 32-bit lane offset, so no pointer
  // stays live across the walk.
  auto emit = [&](int J) {
    const float m2 = other_half(m), e2 = other_half(lb);
    const float mm = fmaxf(m, m2);
    const float e = (m > -INFINITY ? lb * exp2_sum(m - mm) : 0.f) +
                    (m2 > -INFINITY ? e2 * exp2_sum(m2 - mm) : 0.f);
    const int I = __builtin_amdgcn_readfirstlane(q0 / B);
    const int T = (N + B - 1) / B;
    const int64_t base = (int64_t)h * B * T * (T + 1) / 2 + (int64_t)B * I * (I + 1) / 2;
    if (lane < 32 && row < N) part[base + (unsigned)(J * B + row - I * B)] = make_float2(mm, e);
    lb = 0.f;
  };
  qk_walk<kBF16, D>(Q, K, h, g, N, R0, tpb, neg, smem, [&](int kt, const f32x16& c, auto&& mf) {
    if (kt * 32 + 31 <= q0 && q0 + 31 < N) {    // every key of the tile is causal for every row
      // sc >= 0: the maximum of sc * c is sc times the maximum of c
      float r = c[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) r = fmaxf(r, c[e]);
      const float mx = fmaxf(m, r * sc);
      if constexpr (kMass) {
        const float f = exp2_sum(m - mx);
        float t = 0.f;
#pragma unroll
        for (int k = 0; k < NKS; ++k) {
          MF_PIN();
          mf(k);
          MF_PIN();
#pragma unroll
          for (int e = k * EPS; e < (k + 1) * EPS; ++e) t += exp2_sum(fmaf(c[e], sc, -mx));
        }
        MF_PIN();
        l = fmaf(l, f, t);
        lb = fmaf(lb, f, t);
      } else {
        float s = l * exp2_sum(m - mx);
#pragma unroll
        for (int k = 0; k < NKS; ++k) {
          MF_PIN();
          mf(k);
          MF_PIN();
#pragma unroll
          for (int e = k * EPS; e < (k + 1) * EPS; ++e) s += exp2_sum(fmaf(c[e], sc, -mx));
        }
        MF_PIN();
        l = s;
      }
      m = mx;
    } else {
#pragma unroll
      for (int k = 0; k < NKS; ++k) mf(k);
      float x[16];
      float mx = m;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = kt * 32 + tile_key(lane, e);
        x[e] = (j <= row && j < N) ? c[e] * sc : -INFINITY;
        mx = fmaxf(mx, x[e]);
      }
      if (mx > -INFINITY) {
        if constexpr (kMass) {
          const float f = exp2_sum(m - mx);
          float t = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) t += exp2_sum(x[e] - mx);
          l = fmaf(l, f, t);
          lb = fmaf(lb, f, t);
        } else {
          float s = l * exp2_sum(m - mx);
#pragma unroll
          for (int e = 0; e < 16; ++e) s += exp2_sum(x[e] - mx);
          l = s;
        }
        m = mx;
      }
    }
    if constexpr (kMass) {
      // the block's last tile, or the last tile these rows reach
      if (kt % tpb == tpb - 1 || (kt + 1) * 32 > q0 + 31 || (kt + 1) * 32 >= N) emit(kt / tpb);
    }
  });
  // merge (max, sum) pairs: lanes l and l+32 of a wavefront hold the same row,
  // then the two halves (half 0 merges in half 1's pair)
  auto merge = [](float& m, float& l, float m2, float l2) {
    const float mm = fmaxf(m, m2);
    l = (m > -INFINITY ? l * exp2_sum(m - mm) : 0.f) + (m2 > -INFINITY ? l2 * exp2_sum(m2 - mm) : 0.f);
    m = mm;
  };
  merge(m, l, __shfl_xor(m, 32), __shfl_xor(l, 32));
  const int r = row - R0;
  if (wave >= kQkHalfWaves && lane < 32) half1[r] = make_float2(m, l);
  __syncthreads();
  if (wave < kQkHalfWaves && lane < 32 && row < N) {
    const float2 o = half1[r];
    merge(m, l, o.x, o.y);
    lse[(int64_t)h * N + row] = (m + log2f(l)) * kLn2;
  }
}

template <bool kBF16, int D>
__global__ __launch_bounds__(kQkThreads, 4) void k_mass_qk_mfma(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K, int H_s,
    int H_ks, int N, int B, const float* __restrict__ scale, const float* __restrict__ lse,
    float* __restrict__ part) {
  constexpr int NKS = D / 16;
  constexpr int EPS = 16 / NKS;                  // scores per MFMA step
  __shared__ __align__(16) unsigned char smem[4 * KTile<D>::kBytes];
  const int T = (N + B - 1) / B;
  const int NRT = (N + kRT - 1) / kRT;
  const int ngrp = (N + kQkRows - 1) / kQkRows;
  int h, grp;
  qk_item(ngrp, H_s, h, grp);
  const int g = h / (H_s / H_ks);
  const float sc_raw = scale[h] * kLog2e;
  const bool neg = sc_raw < 0.f;                 // products negated by the walk
  const float sc = fabsf(sc_raw);
  const int lane = threadIdx.x & 63;
  const int tpb = B / 32;                        // key tiles per column block
  const int R0 = grp * kQkRows;
  const int q0 = R0 + 32 * ((threadIdx.x >> 6) % kQkHalfWaves);
  const int row = q0 + (lane & 31);
  const float l2 = row < N ? lse[(int64_t)h * N + row] * kLog2e : 0.f;
  float acc = 0.f;
  // sums of the lanes of one 16-row tile: lanes {0..15, 32..47} and {16..31, 48..63}
  auto flush = [&](int J) {
    float v = acc;
    v += __shfl_xor(v, 1);
    v += __shfl_xor(v, 2);
    v += __shfl_xor(v, 4);
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 32);
    const int rt = q0 / kRT + ((lane >> 4) & 1);
    if ((lane == 0 || lane == 16) && rt * kRT < N) part[((int64_t)h * NRT + rt) * T + J] = v;
    acc = 0.f;
  };
  // halves split at a column-block boundary: each block's partials come from one half
  qk_walk<kBF16, D>(Q, K, h, g, N, R0, tpb, neg, smem, [&](int kt, const f32x16& c, auto&& mf) {
    if (kt * 32 + 31 <= q0 && q0 + 31 < N) {    // every key of the tile is causal for every row
#pragma unroll
      for (int k = 0; k < NKS; ++k) {
        MF_PIN();
        mf(k);
        MF_PIN();
#pragma unroll
        for (int e = k * EPS; e < (k + 1) * EPS; ++e) acc += exp2_sum(fmaf(c[e], sc, -l2));
      }
      MF_PIN();
    } else {
#pragma unroll
      for (int k = 0; k < NKS; ++k) mf(k);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int j = kt * 32 + tile_key(lane, e);
        acc += (j <= row && j < N && row < N) ? exp2_sum(fmaf(c[e], sc, -l2)) : 0.f;
      }
    }
    const int J = kt / tpb;
    // the block's last tile, or the last tile these rows reach
    if (kt % tpb == tpb - 1 || (kt + 1) * 32 > q0 + 31 || (kt + 1) * 32 >= N) flush(J);
  });
}

#undef MF_PIN

// two values rounded to the storage type (RNE), packed low first
template <bool kBF16>
__device__ __forceinline__ unsigned pack2(float a, float b) {
  if constexpr (kBF16)
    return (unsigned)__builtin_bit_cast(unsigned short, (__bf16)a) |
           ((unsigned)__builtin_bit_cast(unsigned short, (__bf16)b) << 16);
  else
    return (unsigned)f32_to_f16(a) | ((unsigned)f32_to_f16(b) << 16);
}

// one wavefront per (kept block, head).  The block's NSUB = B/32 key
// sub-tiles are loaded once; for each 32-row sub-tile the NSUB score tiles
// are independent MFMA chains (their latencies overlap), then exponentiated,
// rounded and stored, 8 bytes (4 keys) per lane and tile row.
template <bool kBF16, int D, int NSUB>
__global__ __launch_bounds__(256) void k_gather_qk_mfma(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K, int H_s,
    int H_ks, int N, const float* __restrict__ scale, const float* __restrict__ lse,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ kept, int64_t cap,
    int32_t* __restrict__ col_idx, unsigned short* __restrict__ vals) {
  constexpr int NKS = D / 16;
  constexpr int B = 32 * NSUB;
  const int T = (N + B - 1) / B;
  const int64_t nnzb = row_ptr[T];
  if (nnzb > cap) return;
  const int G = H_s / H_ks;
  const int lane = threadIdx.x & 63;
  const int64_t items = nnzb * H_s;
  for (int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); u < items; u += (int64_t)gridDim.x * 4) {
    const int64_t k = u / H_s;
    const int h = (int)(u - k * H_s);
    const int I = row_of(row_ptr, T, k);
    const int J = kept[(int64_t)I * T + (k - row_ptr[I])];
    if (h == 0 && lane == 0) col_idx[k] = J;
    const float sc = scale[h] * kLog2e;
    unsigned short* tile = vals + (k * H_s + h) * (int64_t)B * B;
    // A operands: key rows J*B + 32 ks + l%32 (clamped), head-dim chunks 8(l/32) + 16 s
    u32x4 kop[NSUB][NKS];
#pragma unroll
    for (int ks = 0; ks < NSUB; ++ks) {
      const unsigned short* kr = K + ((int64_t)(h / G) * N + min(J * B + ks * 32 + (lane & 31), N - 1)) * D + 8 * (lane >> 5);
#pragma unroll
      for (int s = 0; s < NKS; ++s) kop[ks][s] = *reinterpret_cast<const u32x4*>(kr + 16 * s);
    }
    for (int qs = 0; qs < NSUB; ++qs) {
      const int row = I * B + qs * 32 + (lane & 31);
      const bool row_ok = row < N;
      u32x4 qop[NKS];
      const unsigned short* qr = Q + ((int64_t)h * N + min(row, N - 1)) * D + 8 * (lane >> 5);
#pragma unroll
      for (int s = 0; s < NKS; ++s) qop[s] = *reinterpret_cast<const u32x4*>(qr + 16 * s);
      // rows past N: an infinite shift makes every value exactly 0
      const float l2 = row_ok ? lse[(int64_t)h * N + row] * kLog2e : INFINITY;
      f32x16 c[NSUB];
#pragma unroll
      for (int ks = 0; ks < NSUB; ++ks) c[ks] = f32x16{};
#pragma unroll
      for (int s = 0; s < NKS; ++s)
#pragma unroll
        for (int ks = 0; ks < NSUB; ++ks) c[ks] = mfma32<kBF16>(kop[ks][s], qop[s], c[ks]);
      // lane: row qs*32 + l%32 of the tile, keys ks*32 + 8(e/4) + 4(l/32) + e%4.
      // Below the diagonal block every key is causal for every row.
      const bool diag = J == I;
#pragma unroll
      for (int ks = 0; ks < NSUB; ++ks) {
        const int key0 = J * B + ks * 32;
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int e = 4 * e4 + t;
            v[t] = exp2_sum(fmaf(c[ks][e], sc, -l2));
            if (diag && key0 + tile_key(lane, e) > row) v[t] = 0.f;
          }
          const int col = ks * 32 + 8 * e4 + 4 * (lane >> 5);
          *reinterpret_cast<u32x2*>(tile + (int64_t)(qs * 32 + (lane & 31)) * B + col) =
              u32x2{pack2<kBF16>(v[0], v[1]), pack2<kBF16>(v[2], v[3])};
        }
      }
    }
  }
}

// Kept tiles for B = 64 and 128: a workgroup of four wavefronts takes up to
// kGC consecutive kept blocks (in BSR order, so mostly of one block row) of
// one head.  The query operand of each wavefront (32 rows of the block row)
// stays in registers while the row does not change.  Per block, the K block
// (B contiguous rows) comes into LDS through coalesced 16-byte loads issued
// one block ahead; each wavefront computes NSUB*NSUB/4 score sub-tiles of
// 32 x 32, exponentiates and rounds them into an LDS copy of the output tile;
// the tile (B*B contiguous elements) then leaves with coalesced 16-byte
// stores.  Workgroup (x, y): head x (the heads that one XCD serves share
// their Q and K rows in its L2), block group y, y + gridDim.y, ...
constexpr int kGC = 8;                           // kept blocks per block group

template <bool kBF16, int D, int NSUB>
__global__ __launch_bounds__(256) void k_gather_qk_rows(
    const unsigned short* __restrict__ Q, const unsigned short* __restrict__ K, int H_s,
    int H_ks, int N, const float* __restrict__ scale, const float* __restrict__ lse,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ kept, int64_t cap,
    int32_t* __restrict__ col_idx, unsigned short* __restrict__ vals) {
  constexpr int B = 32 * NSUB;
  constexpr int NKS = D / 16;                    // MFMA K steps
  constexpr int kRowU4 = D / 8;                  // 16-byte pieces per K row
  constexpr int KROW = D * 2 + 16;               // LDS bytes per K row (padded)
  constexpr int OROW = B * 2 + 16;               // LDS bytes per output row (padded)
  constexpr int NPK = B * kRowU4 / 256;          // K pieces per thread
  constexpr int kOutU4 = B / 8;                  // 16-byte pieces per output row
  constexpr int NPO = B * kOutU4 / 256;          // output pieces per thread
  constexpr int KPW = NSUB * NSUB / 4;           // score sub-tiles per wavefront
  static_assert(NPK * 256 == B * kRowU4 && NPO * 256 == B * kOutU4, "pieces must divide evenly");
  __shared__ __align__(16) unsigned char k_lds[B * KROW];
  __shared__ __align__(16) unsigned char o_lds[B * OROW];
  const int T = (N + B - 1) / B;
  const int64_t nnzb = row_ptr[T];
  if (nnzb > cap) return;
  const int h = blockIdx.x;
  const int g = h / (H_s / H_ks);
  const float sc = scale[h] * kLog2e;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qs = wave * KPW / NSUB;              // this wavefront's 32-row sub-tile
  const unsigned short* Kg = K + (int64_t)g * N * D;
  // K block J: uniform base and fixed per-thread offsets; only the last,
  // partial block clamps its key rows
  auto load_k = [&](int J, u32x4* v) {
    if (J * B + B <= N) {
      const unsigned short* base = Kg + (int64_t)J * B * D;
#pragma unroll
      for (int n = 0; n < NPK; ++n) {
        const int pc = tid + 256 * n;
        v[n] = *reinterpret_cast<const u32x4*>(base + (pc / kRowU4) * D + 8 * (pc % kRowU4));
      }
    } else {
#pragma unroll
      for (int n = 0; n < NPK; ++n) {
        const int pc = tid + 256 * n;
        const int key = min(J * B + pc / kRowU4, N - 1);
        v[n] = *reinterpret_cast<const u32x4*>(Kg + (int64_t)key * D + 8 * (pc % kRowU4));
      }
    }
  };
  for (int64_t k0 = (int64_t)blockIdx.y * kGC; k0 < nnzb; k0 += (int64_t)gridDim.y * kGC) {
    const int64_t k1 = min(nnzb, k0 + kGC);
    int I = row_of(row_ptr, T, k0);
    int In = I;                                  // row of the prefetched block
    int Iq = -1;                                 // row whose queries are in qop
    u32x4 qop[NKS];
    float l2 = 0.f;
    u32x4 kst[NPK];
    load_k(kept[(int64_t)I * T + (k0 - row_ptr[I])], kst);
    for (int64_t k = k0; k < k1; ++k) {
      I = In;
      const int J = kept[(int64_t)I * T + (k - row_ptr[I])];
      if (h == 0 && tid == 0) col_idx[k] = J;
      // K block of k into LDS, then the next block's loads
#pragma unroll
      for (int n = 0; n < NPK; ++n) {
        const int pc = tid + 256 * n;
        *reinterpret_cast<u32x4*>(k_lds + (pc / kRowU4) * KROW + 16 * (pc % kRowU4)) = kst[n];
      }
      if (k + 1 < k1) {
        while (row_ptr[In + 1] <= k + 1) ++In;
        load_k(kept[(int64_t)In * T + (k + 1 - row_ptr[In])], kst);
      }
      const int row = I * B + qs * 32 + (lane & 31);
      if (I != Iq) {                             // B operand: query rows of this row block
        const unsigned short* qr = Q + ((int64_t)h * N + min(row, N - 1)) * D + 8 * (lane >> 5);
#pragma unroll
        for (int s = 0; s < NKS; ++s) qop[s] = *reinterpret_cast<const u32x4*>(qr + 16 * s);
        // rows past N: an infinite shift makes every value exactly 0
        l2 = row < N ? lse[(int64_t)h * N + row] * kLog2e : INFINITY;
        Iq = I;
      }
      __syncthreads();                           // K block in LDS; the previous tile has left
      // lane: row qs*32 + l%32 of the tile, keys ks*32 + 8(e/4) + 4(l/32) + e%4.
      // Below the diagonal block every key is causal for every row.
      const bool diag = J == I;
#pragma unroll
      for (int i = 0; i < KPW; ++i) {
        const int ks = (wave * KPW + i) % NSUB;
        const unsigned char* kb = k_lds + (ks * 32 + (lane & 31)) * KROW + 16 * (lane >> 5);
        f32x16 c = {};
#pragma unroll
        for (int s = 0; s < NKS; ++s)
          c = mfma32<kBF16>(*reinterpret_cast<const u32x4*>(kb + 32 * s), qop[s], c);
        const int key0 = J * B + ks * 32;
        unsigned char* ob = o_lds + (qs * 32 + (lane & 31)) * OROW + 2 * (ks * 32 + 4 * (lane >> 5));
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
          float v[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int e = 4 * e4 + t;
            v[t] = exp2_sum(fmaf(c[e], sc, -l2));
            if (diag && key0 + tile_key(lane, e) > row) v[t] = 0.f;
          }
          *reinterpret_cast<u32x2*>(ob + 16 * e4) = u32x2{pack2<kBF16>(v[0], v[1]), pack2<kBF16>(v[2], v[3])};
        }
      }
      __syncthreads();                           // output tile complete in LDS
      unsigned short* tile = vals + (k * H_s + h) * (int64_t)B * B;
#pragma unroll
      for (int n = 0; n < NPO; ++n) {
        const int pc = tid + 256 * n;
        const u32x4 v = *reinterpret_cast<const u32x4*>(o_lds + (pc / kOutU4) * OROW + 16 * (pc % kOutU4));
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(tile + (pc / kOutU4) * B + 8 * (pc % kOutU4)));
      }
    }
    __syncthreads();                             // LDS is reused by the next block group
  }
}

bool qk_mfma(int dt, int d, const void* Q, const void* K) {
  return dt != MF_F32 && (d == 64 || d == 128) &&
         (reinterpret_cast<uintptr_t>(Q) & 15) == 0 && (reinterpret_cast<uintptr_t>(K) & 15) == 0;
}

template <class TT>
hipError_t lse_plain(const void* Q, const void* K, int H_s, int H_ks, int N, int d,
                     const float* scale, float* lse, hipStream_t st) {
  using S = typename TT::S;
  hipLaunchKernelGGL((k_lse_plain<TT>), dim3((N + 255) / 256, H_s), dim3(256), 0, st,
                     reinterpret_cast<const S*>(Q), reinterpret_cast<const S*>(K), H_s, H_ks,
                     N, d, scale, lse);
  return hipGetLastError();
}

template <class TT>
hipError_t mass_plain(const void* Q, const void* K, int H_s, int H_ks, int N, int d, int B,
                      const float* scale, const float* lse, float* part, hipStream_t st) {
  using S = typename TT::S;
  hipLaunchKernelGGL((k_mass_qk_plain<TT>), dim3((N + kRT - 1) / kRT, H_s), dim3(256), 0, st,
                     reinterpret_cast<const S*>(Q), reinterpret_cast<const S*>(K), H_s, H_ks,
                     N, d, B, scale, lse, part);
  return hipGetLastError();
}

template <class TT>
hipError_t gather_plain(const void* Q, const void* K, int H_s, int H_ks, int N, int d, int B,
                        const float* scale, const float* lse, const int32_t* row_ptr,
                        const int32_t* kept, int64_t cap, int32_t* col_idx, void* vals,
                        hipStream_t st) {
  using S = typename TT::S;
  const int T = mf::blocks_of(N, B);
  const int64_t ub = std::min<int64_t>(cap, (int64_t)T * (T + 1) / 2) * H_s;
  if (ub <= 0) return hipSuccess;
  hipLaunchKernelGGL((k_gather_qk_plain<TT>), dim3((int)std::min<int64_t>(ub, 8192)), dim3(256), 0,
                     st, reinterpret_cast<const S*>(Q), reinterpret_cast<const S*>(K), H_s, H_ks,
                     N, d, B, scale, lse, row_ptr, kept, cap, col_idx, reinterpret_cast<S*>(vals));
  return hipGetLastError();
}

// part == nullptr: lse only; otherwise also the (m, e) pairs of block size B
template <bool kBF16>
hipError_t lse_mfma(const void* Q, const void* K, int H_s, int H_ks, int N, int d,
                    const float* scale, float* lse, hipStream_t st, int B = 32,
                    float2* part = nullptr) {
  auto q = reinterpret_cast<const unsigned short*>(Q);
  auto k = reinterpret_cast<const unsigned short*>(K);
  const dim3 grid(H_s * ((N + kQkRows - 1) / kQkRows));
#define MF_LSE(D_, M_) \
  hipLaunchKernelGGL((k_lse_mfma<kBF16, D_, M_>), grid, dim3(kQkThreads), 0, st, q, k, H_s, H_ks, N, \
                     scale, lse, B, part)
  if (part) {
    if (d == 128) MF_LSE(128, true); else MF_LSE(64, true);
  } else {
    if (d == 128) MF_LSE(128, false); else MF_LSE(64, false);
  }
#undef MF_LSE
  return hipGetLastError();
}

template <bool kBF16>
hipError_t mass_mfma(const void* Q, const void* K, int H_s, int H_ks, int N, int d, int B,
                     const float* scale, const float* lse, float* part, hipStream_t st) {
  auto q = reinterpret_cast<const unsigned short*>(Q);
  auto k = reinterpret_cast<const unsigned short*>(K);
  const dim3 grid(H_s * ((N + kQkRows - 1) / kQkRows));
  if (d == 128) hipLaunchKernelGGL((k_mass_qk_mfma<kBF16, 128>), grid, dim3(kQkThreads), 0, st, q, k, H_s, H_ks, N, B, scale, lse, part);
  else hipLaunchKernelGGL((k_mass_qk_mfma<kBF16, 64>), grid, dim3(kQkThreads), 0, st, q, k, H_s, H_ks, N, B, scale, lse, part);
  return hipGetLastError();
}

template <bool kBF16>
hipError_t gather_mfma(const void* Q, const void* K, int H_s, int H_ks, int N, int d, int B,
                       const float* scale, const float* lse, const int32_t* row_ptr,
                       const int32_t* kept, int64_t cap, int32_t* col_idx, void* vals,
                       hipStream_t st) {
  const int T = mf::blocks_of(N, B);
  const int64_t ub = std::min<int64_t>(cap, (int64_t)T * (T + 1) / 2) * H_s;
  if (ub <= 0) return hipSuccess;
  const dim3 grid((unsigned)std::min<int64_t>((ub + 3) / 4, 16384));
  auto q = reinterpret_cast<const unsigned short*>(Q);
  auto k = reinterpret_cast<const unsigned short*>(K);
  auto v = reinterpret_cast<unsigned short*>(vals);
#define MF_GQ(D_, NS_) \
  hipLaunchKernelGGL((k_gather_qk_mfma<kBF16, D_, NS_>), grid, dim3(256), 0, st, q, k, H_s, H_ks, N, \
                     scale, lse, row_ptr, kept, cap, col_idx, v)
  if (B == 32 || (reinterpret_cast<uintptr_t>(vals) & 15) != 0) {   // per-wavefront tiles, 8-byte stores
    if (d == 128) {
      if (B == 32) MF_GQ(128, 1); else if (B == 64) MF_GQ(128, 2); else MF_GQ(128, 4);
    } else {
      if (B == 32) MF_GQ(64, 1); else if (B == 64) MF_GQ(64, 2); else MF_GQ(64, 4);
    }
#undef MF_GQ
    return hipGetLastError();
  }
  const int64_t groups = (std::min<int64_t>(cap, (int64_t)T * (T + 1) / 2) + kGC - 1) / kGC;
  const dim3 grid_rows(H_s, (unsigned)std::min<int64_t>(groups, 65535));
#define MF_GR(D_, NS_) \
  hipLaunchKernelGGL((k_gather_qk_rows<kBF16, D_, NS_>), grid_rows, dim3(256), 0, st, q, k, H_s, H_ks, \
                     N, scale, lse, row_ptr, kept, cap, col_idx, v)
  if (d == 128) {
    if (B == 64) MF_GR(128, 2); else MF_GR(128, 4);
  } else {
    if (B == 64) MF_GR(64, 2); else MF_GR(64, 4);
  }
#undef MF_GR
  return hipGetLastError();
}

}  // namespace

namespace mf {

hipError_t launch_row_lse(const void* Q, const void* K, int dt, int H_s, int H_ks, int N, int d,
                          const float* scale, float* lse, hipStream_t st) {
  if (qk_mfma(dt, d, Q, K))
    return dt == MF_BF16 ? lse_mfma<true>(Q, K, H_s, H_ks, N, d, scale, lse, st)
                         : lse_mfma<false>(Q, K, H_s, H_ks, N, d, scale, lse, st);
  if (dt == MF_F32) return lse_plain<mfd::TF32>(Q, K, H_s, H_ks, N, d, scale, lse, st);
  if (dt == MF_F16) return lse_plain<mfd::TF16>(Q, K, H_s, H_ks, N, d, scale, lse, st);
  return lse_plain<mfd::TBF16>(Q, K, H_s, H_ks, N, d, scale, lse, st);
}

size_t block_mass_qk_workspace_bytes(int H_s, int N, int B) {
  return (size_t)H_s * (size_t)((N + kRT - 1) / kRT) * (size_t)blocks_of(N, B) * sizeof(float);
}

hipError_t launch_block_mass_qk(const void* Q, const void* K, const float* scale, const float* lse,
                                int dt, int H_s, int H_ks, int N, int d, int B, float* mass,
                                void* workspace, hipStream_t st) {
  float* part = reinterpret_cast<float*>(workspace);
  hipError_t e;
  if (qk_mfma(dt, d, Q, K) && B >= 32)
    e = dt == MF_BF16 ? mass_mfma<true>(Q, K, H_s, H_ks, N, d, B, scale, lse, part, st)
                      : mass_mfma<false>(Q, K, H_s, H_ks, N, d, B, scale, lse, part, st);
  else if (dt == MF_F32) e = mass_plain<mfd::TF32>(Q, K, H_s, H_ks, N, d, B, scale, lse, part, st);
  else if (dt == MF_F16) e = mass_plain<mfd::TF16>(Q, K, H_s, H_ks, N, d, B, scale, lse, part, st);
  else e = mass_plain<mfd::TBF16>(Q, K, H_s, H_ks, N, d, B, scale, lse, part, st);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_mass_reduce, dim3(blocks_of(N, B), (blocks_of(N, B) + 63) / 64), dim3(256), 0,
                     st, part, H_s, N, B, mass);
  return hipGetLastError();
}

// workspace of the one-pass form: the (m, e) pairs, then the per-head block sums
static size_t lse_pairs_bytes(int H_s, int N, int B) {
  const size_t T = (size_t)blocks_of(N, B);
  return ((size_t)H_s * (size_t)B * (T * (T + 1) / 2) * sizeof(float2) + 255) & ~(size_t)255;
}

size_t lse_block_mass_qk_workspace_bytes(int H_s, int N, int B) {
  const size_t T = (size_t)blocks_of(N, B);
  const size_t one = lse_pairs_bytes(H_s, N, B) + (size_t)H_s * (T * (T + 1) / 2) * sizeof(float);
  return std::max(one, block_mass_qk_workspace_bytes(H_s, N, B));
}

hipError_t launch_lse_block_mass_qk(const void* Q, const void* K, const float* scale, int dt,
                                    int H_s, int H_ks, int N, int d, int B, float* lse,
                                    float* mass, void* workspace, hipStream_t st) {
  if (!(qk_mfma(dt, d, Q, K) && B >= 32)) {      // two passes: lse, then the masses
    const hipError_t e = launch_row_lse(Q, K, dt, H_s, H_ks, N, d, scale, lse, st);
    if (e != hipSuccess) return e;
    return launch_block_mass_qk(Q, K, scale, lse, dt, H_s, H_ks, N, d, B, mass, workspace, st);
  }
  float2* part = reinterpret_cast<float2*>(workspace);
  float* sums = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(workspace) +
                                         lse_pairs_bytes(H_s, N, B));
  const int T = blocks_of(N, B);
  hipError_t e = dt == MF_BF16 ? lse_mfma<true>(Q, K, H_s, H_ks, N, d, scale, lse, st, B, part)
                               : lse_mfma<false>(Q, K, H_s, H_ks, N, d, scale, lse, st, B, part);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_mass_from_partials, dim3(H_s * T), dim3(kMfpThreads), 0, st, part, lse, H_s, N, B,
                     sums);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_block_mass_heads(sums, H_s, T, mass, st);
}

hipError_t launch_gather_qk(const void* Q, const void* K, const float* scale, const float* lse,
                            int dt, int H_s, int H_ks, int N, int d, int B,
                            const int32_t* row_ptr, const int32_t* kept, int64_t cap,
                            int32_t* col_idx, void* vals, hipStream_t st) {
  if (qk_mfma(dt, d, Q, K) && B >= 32 && (reinterpret_cast<uintptr_t>(vals) & 7) == 0)
    return dt == MF_BF16
               ? gather_mfma<true>(Q, K, H_s, H_ks, N, d, B, scale, lse, row_ptr, kept, cap, col_idx, vals, st)
               : gather_mfma<false>(Q, K, H_s, H_ks, N, d, B, scale, lse, row_ptr, kept, cap, col_idx, vals, st);
  if (dt == MF_F32)
    return gather_plain<mfd::TF32>(Q, K, H_s, H_ks, N, d, B, scale, lse, row_ptr, kept, cap, col_idx, vals, st);
  if (dt == MF_F16)
    return gather_plain<mfd::TF16>(Q, K, H_s, H_ks, N, d, B, scale, lse, row_ptr, kept, cap, col_idx, vals, st);
  return gather_plain<mfd::TBF16>(Q, K, H_s, H_ks, N, d, B, scale, lse, row_ptr, kept, cap, col_idx, vals, st);
}

}  // namespace mf
