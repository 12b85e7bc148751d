// Fused head-mapped BSR retrieval.
//
// MapFlow's retrieval kernel reads only the kept sparse blocks, linearly
// combines the sender heads into each receiver head on chip and immediately
// multiplies by the receiver's own values, accumulating the output; no dense
// receiver map is ever written (article aitest123.com/news/zaoi86, third
// section, third component; paper page montaan.com/papers/2610.14688,
// "Practical Implementation Details" and highlight 4).  Per kept block
// k = (I, J) and receiver head r:
//     Ahat_k[r] = sum_s W[r][s] * vals[k][s]
//     O[I*B+i][r][:] += sum_c Ahat_k[r][i][c] * V[J*B+c][r/G][:]
//
// Kernels:
//
// k_prep_values   once per call: V (fp16/bf16, rows of stride ldV) becomes an
//                 fp16 copy in the MFMA B-operand layout Vp[g][key/8][d][8]
//                 (eight consecutive keys of one head-dim column are 16
//                 contiguous bytes).  Each 32-key chunk of each KV head gets a
//                 power-of-two scale 2^-e (e >= 0, e = 0 unless |V| reaches
//                 2^15) that keeps the fp16 copy in range; the matching 2^e is
//                 folded into the mixed map before it is rounded to fp16.
//
// k_retrieve_mfma (fp16/bf16, d = 128, B in {32,64,128}, H_r <= 32, H_s <= 56)
//   Work item = (block row I, 16-row slice); one 256-thread workgroup owns all
//   receiver heads and all of d for its 16 query rows, so every kept tile
//   element leaves HBM once.  The row's kept blocks are walked in 32-column
//   chunks through a software pipeline:
//   * the chunk's [H_s][16][32] tile slice is copied HBM -> LDS with the
//     gfx950 direct-to-LDS 16-byte loads into a double buffer: chunk u+2
//     streams in while chunk u is computed, with no registers spent on it;
//   * head mix on MFMA 16x16x32 (M = receiver heads, K = sender heads,
//     N = 16 tile positions).  B operands come from LDS as 16-byte runs of
//     8 sender heads and are transposed in registers (v_perm_b32).  bf16 tiles
//     use bf16 MFMA with W split into hi + lo bf16 halves, so W is exact and
//     the tiles need no conversion; the lo half of a partly filled K step
//     rides in its empty K slots.  fp16 tiles use fp16 MFMA with W in fp16;
//   * the fp32 mixed map is rounded to fp16 into LDS (the round trip is also
//     the re-layout to "query rows across lanes, key columns along K");
//   * Ahat . V on fp16 MFMA (M = 16 query rows, K = 32 keys, N = 16 head-dim
//     columns); V operands are single 16-byte loads from the prepared copy,
//     issued before the head mix so their latency is hidden; one V operand
//     serves every receiver head of its KV group;
//   * accumulators (16 rows x 8 heads x 128 d per wavefront) stay in AGPRs
//     for the whole row; O is written once through an LDS transpose as
//     16-byte stores.
//   The 16-row slices of one block row go to one XCD (shared V tiles in its
//   L2); block rows are issued from the last to the first.
//
// k_retrieve_simple (every other supported case, including fp32)
//   One workgroup per (block row, receiver head): the mixed tile is built in
//   LDS in fp32, then multiplied with V by plain fp32 FMAs.
#include <algorithm>
#include <type_traits>

#include "mf_internal.h"

namespace {

using namespace mfd;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kThreads = 256;
constexpr int kD = 128;          // head dim of the MFMA kernel
constexpr int kRows = 16;        // query rows per work item
constexpr int kCB = 32;          // key columns per pipeline chunk
constexpr int kMaxRecv = 32;     // receiver heads of the MFMA kernel
constexpr int kMaxHs = 56;       // sender heads of the MFMA kernel
constexpr int kSlotBytes = kRows * kCB * 2;             // one head of one chunk
constexpr int kAP = kCB + 8;     // LDS pitch (halves) of the mixed map rows
constexpr int kAhatBytes = kMaxRecv * kRows * kAP * 2;

__device__ __forceinline__ f16x8 as_f16x8(const u32x4& v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// 8x8 transpose of 16-bit elements held as 8 rows of 8 (u32x4 each):
// out[t] element j = in[j] element t.
__device__ __forceinline__ void transpose8x8(const u32x4 (&x)[8], u32x4 (&y)[8]) {
  constexpr unsigned kLo = 0x05040100u;  // low halves of (src1, src0)
  constexpr unsigned kHi = 0x07060302u;  // high halves of (src1, src0)
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const unsigned sel = (t & 1) ? kHi : kLo;
#pragma unroll
    for (int m = 0; m < 4; ++m)
      y[t][m] = __builtin_amdgcn_perm(x[2 * m + 1][t >> 1], x[2 * m][t >> 1], sel);
  }
}

// s_waitcnt vmcnt(n) with the other counters left alone (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// The retrieval loop issues its vector-memory traffic through these wrappers
// and waits on it explicitly.  Loads return in issue order, so "at most n
// newer operations outstanding" identifies exactly which data has landed; the
// compiler, unaware of these operations, adds no conservative waits of its own.
__device__ __forceinline__ void dma16(const void* g, unsigned lds_base) {
  // 16 bytes per lane from HBM straight into LDS at lds_base + 16 * lane
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(g) : "memory", "m0");
}
__device__ __forceinline__ u32x4 gload16(const void* p) {
  u32x4 r;
  asm volatile("global_load_dwordx4 %0, %1, off" : "=v"(r) : "v"(p));
  return r;
}
// Waits until at most N vector-memory operations are outstanding; the 16
// operands tie the V operand registers to the wait so no use precedes it.
template <int N>
__device__ __forceinline__ void wait_vop(u32x4 (&v)[2][8]) {
  asm volatile("s_waitcnt vmcnt(%16)"
               : "+v"(v[0][0]), "+v"(v[0][1]), "+v"(v[0][2]), "+v"(v[0][3]),
                 "+v"(v[0][4]), "+v"(v[0][5]), "+v"(v[0][6]), "+v"(v[0][7]),
                 "+v"(v[1][0]), "+v"(v[1][1]), "+v"(v[1][2]), "+v"(v[1][3]),
                 "+v"(v[1][4]), "+v"(v[1][5]), "+v"(v[1][6]), "+v"(v[1][7])
               : "n"(N));
}
// Workgroup barrier for LDS traffic only (outstanding HBM loads stay in flight).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p);
}

__device__ __forceinline__ unsigned short bf16_bits(float f) {
  return __builtin_bit_cast(unsigned short, (__bf16)f);  // RNE
}

// ---------------------------------------------------------------------------
// V preparation
// ---------------------------------------------------------------------------

template <bool kBF16>
__global__ __launch_bounds__(kThreads) void k_prep_values(
    const unsigned short* __restrict__ V, int N, int H_kv, int64_t ldV, int nchunk,
    unsigned short* __restrict__ Vp, int* __restrict__ escale, int* __restrict__ eflag) {
  __shared__ float tile[kCB][kD + 1];
  __shared__ float red[kThreads / 64];
  const int ch = blockIdx.x;
  const int tid = threadIdx.x;
  int any = 0;
  for (int g = 0; g < H_kv; ++g) {
    float mx = 0.f;
    for (int e = tid; e < kCB * kD; e += kThreads) {
      const int c = e / kD, dd = e % kD;
      const int64_t key = (int64_t)ch * kCB + c;
      float v = 0.f;
      if (key < N) {
        const unsigned short h = V[key * ldV + (int64_t)g * kD + dd];
        v = kBF16 ? bf16_to_f32(h) : f16_to_f32(h);
      }
      tile[c][dd] = v;
      mx = fmaxf(mx, fabsf(v));
    }
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    if ((tid & 63) == 0) red[tid >> 6] = mx;
    __syncthreads();
    mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    int ex = 0;
    if (kBF16 && mx >= 32768.f) {
      int x;
      frexpf(mx, &x);            // mx < 2^x
      ex = min(x - 15, 120);
    }
    any |= ex;
    // Vp[g][key/8][d][8]: thread -> (8-key group, d)
    for (int e = tid; e < (kCB / 8) * kD; e += kThreads) {
      const int c8 = e / kD, dd = e % kD;
      u32x4 pk;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float a = __builtin_ldexpf(tile[8 * c8 + 2 * j][dd], -ex);
        const float b = __builtin_ldexpf(tile[8 * c8 + 2 * j + 1][dd], -ex);
        pk[j] = pack_f16x2(a, b);
      }
      const int64_t row8 = (int64_t)g * (nchunk * (kCB / 8)) + (int64_t)ch * (kCB / 8) + c8;
      *reinterpret_cast<u32x4*>(Vp + (row8 * kD + dd) * 8) = pk;
    }
    if (tid == 0) escale[(int64_t)ch * H_kv + g] = ex;
    __syncthreads();
  }
  if (tid == 0) eflag[ch] = any;
}

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------

__device__ __forceinline__ int item_of(int b, int subs, int T, int* I, int* sub) {
  const int xcd = b & 7;
  const int local = b >> 3;
  const int row_slot = (local / subs) * 8 + xcd;
  if (row_slot >= T) return 0;
  *I = T - 1 - row_slot;
  *sub = local % subs;
  return 1;
}

// Head-mix K-step plan.  Sender heads come in NCH chunks of 8.
//  fp16: operand b covers chunks 4b..4b+3 (lane group q -> chunk 4b+q), W in fp16.
//  bf16: W = hi + lo (both bf16).  Full groups of 4 chunks use one B operand
//        twice (W_hi, then W_lo).  A remainder of R <= 2 chunks fits in one
//        K step: lane groups 0..R-1 carry the chunks with W_hi, R..2R-1 the same
//        chunks with W_lo.  A remainder of 3 is a full-style pair.
template <bool kBF16, int NCH>
struct HmPlan {
  static constexpr int F = NCH / 4;
  static constexpr int R = NCH % 4;
  static constexpr int NBOP = kBF16 ? F + (R ? 1 : 0) : (NCH + 3) / 4;
  // number of W operands used with B operand b
  static constexpr __host__ __device__ int nw(int b) {
    return !kBF16 ? 1 : (b < F ? 2 : (R == 3 ? 2 : 1));
  }
  // chunk carried by lane group q in B operand b (-1: zero)
  static __device__ __forceinline__ int chunk(int b, int q) {
    if (!kBF16) { const int c = 4 * b + q; return c < NCH ? c : -1; }
    if (b < F || R == 3) { const int c = 4 * b + q; return c < NCH ? c : -1; }
    return q < 2 * R ? 4 * F + (q % R) : -1;
  }
  // which half of W lane group q uses with (b, w): 0 = hi/plain, 1 = lo
  static __device__ __forceinline__ int half(int b, int w, int q) {
    if (!kBF16) return 0;
    if (b < F || R == 3) return w;
    return q < R ? 0 : 1;
  }
};

// RPW receiver heads per wavefront (H_r = 4 * RPW); GS consecutive receivers
// share one KV group inside a wavefront (GS = G when a wavefront spans two
// groups, GS = RPW when it lies inside one), so the group of local receiver rl
// is rl / GS.
template <bool kBF16, int NCH, int RPW, int GS>
__global__ __launch_bounds__(kThreads, 1) void k_retrieve_mfma(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const unsigned short* __restrict__ vals, int64_t nnzb, int H_s, int N,
    int B, const float* __restrict__ W, int H_r,
    const unsigned short* __restrict__ Vp, const int* __restrict__ escale,
    const int* __restrict__ eflag, int nchunk, int H_kv,
    unsigned short* __restrict__ O, int64_t ldO) {
  using Plan = HmPlan<kBF16, NCH>;
  constexpr int NBOP = Plan::NBOP;
  constexpr int MT = RPW > 4 ? 2 : 1;             // 16-receiver M tiles of the head mix
  static_assert(RPW % GS == 0 && RPW / GS <= 2, "at most two KV groups per wavefront");
  constexpr int NDMA = 2 * NCH;  // direct-to-LDS copies per wave per chunk (8*NCH heads / 4 waves)
  constexpr int kStageBytes = 8 * NCH * kSlotBytes;   // one chunk, head slots 0..8*NCH-1
  constexpr int kSmem = 2 * kStageBytes + kAhatBytes > 4 * kRows * kD * 2
                            ? 2 * kStageBytes + kAhatBytes : 4 * kRows * kD * 2;
  __shared__ __align__(16) unsigned char smem[kSmem];
  unsigned short* stage0 = reinterpret_cast<unsigned short*>(smem);
  unsigned short* Ahs = reinterpret_cast<unsigned short*>(smem + 2 * kStageBytes);

  const int T = (N + B - 1) / B;
  const int subs = B / kRows;
  int I, sub;
  if (!item_of(blockIdx.x, subs, T, &I, &sub)) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15;
  const int q = lane >> 4;

  // head slots H_s..8*NCH-1 of both stage buffers are never copied into: zero them
  for (int e = threadIdx.x; e < 2 * (8 * NCH - H_s) * (kSlotBytes / 16); e += kThreads) {
    const int per = (8 * NCH - H_s) * (kSlotBytes / 16);
    const int bsel = e / per, rem = e % per;
    *reinterpret_cast<u32x4*>(smem + bsel * kStageBytes + H_s * kSlotBytes + rem * 16) =
        u32x4{0u, 0u, 0u, 0u};
  }

  // ---- head-map operands: row r = 16*mt + n; K slot (q, j) per the plan ----
  u32x4 wop[NBOP][2][MT];
#pragma unroll
  for (int b = 0; b < NBOP; ++b)
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const int r = 16 * mt + n;
        const int c = Plan::chunk(b, q);
        const int hf = Plan::half(b, w, q);
        unsigned short hv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int s = 8 * c + j;
          float x = (w < Plan::nw(b) && c >= 0 && r < H_r && s < H_s) ? W[(int64_t)r * H_s + s] : 0.f;
          if (kBF16) {
            const unsigned short hi = bf16_bits(x);
            hv[j] = hf == 0 ? hi : bf16_bits(x - bf16_to_f32(hi));
          } else {
            hv[j] = f32_to_f16(x);
          }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) wop[b][w][mt][j] = (unsigned)hv[2 * j] | ((unsigned)hv[2 * j + 1] << 16);
      }

  f32x4 acc[RPW][8];
#pragma unroll
  for (int rl = 0; rl < RPW; ++rl)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[rl][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int G = H_r / H_kv;
  const int rbeg = wave * RPW;
  int64_t kb = row_ptr[I], ke = row_ptr[I + 1];
  kb = kb < 0 ? 0 : (kb > nnzb ? nnzb : kb);
  ke = ke < kb ? kb : (ke > nnzb ? nnzb : ke);
  const int ncc = B / kCB;
  const int nchunks = (int)(ke - kb) * ncc;
  const int64_t nkey8 = (int64_t)nchunk * (kCB / 8);

  // direct-to-LDS copy of chunk u's [H_s][16][32] slice into stage buffer u&1
  const int64_t tile_elems = (int64_t)B * B;
  const int lane_off = (sub * kRows + (lane >> 2)) * B + (lane & 3) * 8;
  auto issue_stage = [&](int u) {
    const int64_t k = kb + u / ncc;
    const int cc = u % ncc;
    const unsigned buf = lds_addr(smem + (u & 1) * kStageBytes);
    const unsigned short* src0 = vals + k * H_s * tile_elems + lane_off + cc * kCB;
#pragma unroll
    for (int m = 0; m < NDMA; ++m) {
      int s = wave + 4 * m;
      s = s < H_s ? s : H_s - 1;  // duplicate copies of the last head are harmless
      dma16(src0 + s * tile_elems, buf + s * kSlotBytes);
    }
  };

  if (nchunks > 0) issue_stage(0);
  if (nchunks > 1) issue_stage(1);

  for (int u = 0; u < nchunks; ++u) {
    const int64_t k = kb + u / ncc;
    const int cc = u % ncc;
    const int J = col_idx[k];
    const bool jok = (J >= 0 && J < T);
    const int chunk = jok ? (J * B + cc * kCB) / kCB : 0;   // global 32-key chunk

    // Stage u landed: its copies were issued before chunk u-1's V loads,
    // which the previous iteration waited for (u = 0: wait here).
    if (u == 0) { if (nchunks > 1) wait_vmcnt<NDMA>(); else wait_vmcnt<0>(); }
    lds_barrier();

    // V operands for this chunk: this wave's (at most two) KV groups
    const int g0 = rbeg / G;
    const int g1 = (rbeg + RPW - 1) / G;
    u32x4 vop[2][8];
#pragma unroll
    for (int gi = 0; gi < 2; ++gi) {
      const int g = gi == 0 ? g0 : g1;
      const unsigned short* base = Vp + (((int64_t)g * nkey8 + (int64_t)chunk * (kCB / 8) + q) * kD + n) * 8;
#pragma unroll
      for (int t = 0; t < 8; ++t) vop[gi][t] = gload16(base + 16 * t * 8);
    }

    // ---- head mix: rows 4w..4w+3, columns 0..31 of the chunk -----------
    // Two halves of 4 tile columns each keep the live registers down; the
    // 16-byte LDS runs are simply read again for the second half.
    {
      const unsigned short* buf = reinterpret_cast<const unsigned short*>(smem + (u & 1) * kStageBytes);
      const int il = wave * 4 + (n >> 2);          // row within the slice
      const int cg = (n & 3) * 8;                  // column group within the chunk
      const bool scaled = jok && eflag[chunk] != 0;
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        f32x4 c[4][MT];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) c[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NBOP; ++b) {
          // lane groups without a chunk read chunk 0; their W slots are zero
          const int ch = Plan::chunk(b, q) < 0 ? 0 : Plan::chunk(b, q);
          u32x4 x[8], y[8];
#pragma unroll
          for (int uu = 0; uu < 8; ++uu)
            x[uu] = *reinterpret_cast<const u32x4*>(buf + ((8 * ch + uu) * kRows + il) * kCB + cg);
          transpose8x8(x, y);
#pragma unroll
          for (int w = 0; w < Plan::nw(b); ++w)
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
              for (int mt = 0; mt < MT; ++mt) {
                if constexpr (kBF16)
                  c[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                      as_bf16x8(wop[b][w][mt]), as_bf16x8(y[4 * th + t]), c[t][mt], 0, 0, 0);
                else
                  c[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                      as_f16x8(wop[b][w][mt]), as_f16x8(y[4 * th + t]), c[t][mt], 0, 0, 0);
              }
        }
        // lane (n, q) holds Ahat[16mt + 4q + a][row il][cg + 4th + t]
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int r = 16 * mt + 4 * q + a;
            if (r < H_r) {
              uint2 pk;
              if (scaled) {
                const int ex = escale[(int64_t)chunk * H_kv + r / G];
                pk.x = pack_f16x2(__builtin_ldexpf(c[0][mt][a], ex), __builtin_ldexpf(c[1][mt][a], ex));
                pk.y = pack_f16x2(__builtin_ldexpf(c[2][mt][a], ex), __builtin_ldexpf(c[3][mt][a], ex));
              } else {
                pk.x = pack_f16x2(c[0][mt][a], c[1][mt][a]);
                pk.y = pack_f16x2(c[2][mt][a], c[3][mt][a]);
              }
              *reinterpret_cast<uint2*>(&Ahs[(r * kRows + il) * kAP + cg + 4 * th]) = pk;
            }
          }
      }
    }
    lds_barrier();

    if (u + 2 < nchunks) issue_stage(u + 2);

    // ---- Ahat . V: this wave's receiver heads, all 16 rows --------------
    if (u + 2 < nchunks) wait_vop<NDMA>(vop); else wait_vop<0>(vop);
    if (jok) {
#pragma unroll
      for (int rl = 0; rl < RPW; ++rl) {
        const int r = rbeg + rl;
        const u32x4 a4 = *reinterpret_cast<const u32x4*>(&Ahs[(r * kRows + n) * kAP + 8 * q]);
#pragma unroll
        for (int t = 0; t < 8; ++t)
          acc[rl][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              as_f16x8(a4), as_f16x8(vop[rl / GS][t]), acc[rl][t], 0, 0, 0);
      }
    }
  }

  // ---- store through LDS: lane (n, q) holds O[row 4q+a][r][d = 16t + n] ----
  unsigned short* ot = reinterpret_cast<unsigned short*>(smem) + wave * (kRows * kD);
#pragma unroll
  for (int rl = 0; rl < RPW; ++rl) {
    const int r = rbeg + rl;
    lds_barrier();
    {
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float v = acc[rl][t][a];
          ot[(4 * q + a) * kD + 16 * t + n] = kBF16 ? bf16_bits(v) : f32_to_f16(v);
        }
    }
    lds_barrier();
    {
      // each lane stores 16 contiguous bytes: row lane/16 + 4*pass, d = 8*(lane%16)
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        const int i = 4 * pass + (lane >> 4);
        const int64_t grow = (int64_t)I * B + sub * kRows + i;
        const u32x4 v = *reinterpret_cast<const u32x4*>(&ot[i * kD + 8 * n]);
        if (grow < N) *reinterpret_cast<u32x4*>(O + grow * ldO + (int64_t)r * kD + 8 * n) = v;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Plain kernel
// ---------------------------------------------------------------------------

template <class TT, int BB, int D>
__global__ __launch_bounds__(kThreads) void k_retrieve_simple(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const typename TT::S* __restrict__ vals, int64_t nnzb, int H_s, int N,
    const float* __restrict__ W, int H_r, const typename TT::S* __restrict__ V,
    int H_kv, int64_t ldV, typename TT::S* __restrict__ O, int64_t ldO) {
  constexpr int RPP = kThreads / D;        // query rows per pass
  constexpr int NACC = BB / RPP;           // rows per thread
  __shared__ float ahat[BB * BB];
  __shared__ float wrow[64];
  const int T = (N + BB - 1) / BB;
  const int I = T - 1 - (int)blockIdx.x;
  const int r = blockIdx.y;
  const int g = r / (H_r / H_kv);
  const int tid = threadIdx.x;
  const int dcol = tid % D;
  const int i0 = tid / D;
  if (tid < H_s) wrow[tid] = W[(int64_t)r * H_s + tid];
  float acc[NACC];
#pragma unroll
  for (int m = 0; m < NACC; ++m) acc[m] = 0.f;
  int64_t kb = row_ptr[I], ke = row_ptr[I + 1];
  kb = kb < 0 ? 0 : (kb > nnzb ? nnzb : kb);
  ke = ke < kb ? kb : (ke > nnzb ? nnzb : ke);
  __syncthreads();
  for (int64_t k = kb; k < ke; ++k) {
    const int J = col_idx[k];
    if (J < 0 || J >= T) continue;
    const typename TT::S* blk = vals + k * H_s * BB * BB;
    for (int e = tid; e < BB * BB; e += kThreads) {
      float s = 0.f;
      for (int h = 0; h < H_s; ++h) s += wrow[h] * TT::tof(blk[(int64_t)h * BB * BB + e]);
      ahat[e] = s;
    }
    __syncthreads();
    const int cols = min(BB, N - J * BB);
    for (int c = 0; c < cols; ++c) {
      const float v = TT::tof(V[((int64_t)J * BB + c) * ldV + (int64_t)g * D + dcol]);
#pragma unroll
      for (int m = 0; m < NACC; ++m) acc[m] += ahat[(i0 + m * RPP) * BB + c] * v;
    }
    __syncthreads();
  }
#pragma unroll
  for (int m = 0; m < NACC; ++m) {
    const int64_t grow = (int64_t)I * BB + i0 + m * RPP;
    if (grow < N) O[grow * ldO + (int64_t)r * D + dcol] = TT::fromf(acc[m]);
  }
}

template <class TT, int BB, int D>
int launch_simple_t(const int32_t* row_ptr, const int32_t* col_idx, const void* vals,
                    int64_t nnzb, int H_s, int N, const float* W, int H_r,
                    const void* V, int H_kv, int64_t ldV, void* O, int64_t ldO,
                    hipStream_t st) {
  using S = typename TT::S;
  const int T = mf::blocks_of(N, BB);
  hipLaunchKernelGGL((k_retrieve_simple<TT, BB, D>), dim3(T, H_r), dim3(kThreads),
                     0, st, row_ptr, col_idx, reinterpret_cast<const S*>(vals),
                     nnzb, H_s, N, W, H_r, reinterpret_cast<const S*>(V), H_kv,
                     ldV, reinterpret_cast<S*>(O), ldO);
  return mf::hip_check(hipGetLastError(), "k_retrieve_simple launch");
}

template <class TT, int D>
int launch_simple_d(int B, const int32_t* row_ptr, const int32_t* col_idx,
                    const void* vals, int64_t nnzb, int H_s, int N, const float* W,
                    int H_r, const void* V, int H_kv, int64_t ldV, void* O,
                    int64_t ldO, hipStream_t st) {
  switch (B) {
    case 16: return launch_simple_t<TT, 16, D>(row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
    case 32: return launch_simple_t<TT, 32, D>(row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
    case 64: return launch_simple_t<TT, 64, D>(row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
    default: return launch_simple_t<TT, 128, D>(row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
  }
}

template <class TT>
int launch_simple(int B, int d, const int32_t* row_ptr, const int32_t* col_idx,
                  const void* vals, int64_t nnzb, int H_s, int N, const float* W,
                  int H_r, const void* V, int H_kv, int64_t ldV, void* O,
                  int64_t ldO, hipStream_t st) {
  if (d == 64)
    return launch_simple_d<TT, 64>(B, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
  return launch_simple_d<TT, 128>(B, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

// Workspace layout of the MFMA path: Vp | escale | eflag (each 256-byte aligned).
struct WsLayout {
  size_t vp, es, ef, total;
  int nchunk;
};
inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
inline WsLayout ws_layout(int N, int B, int H_kv) {
  WsLayout L;
  const int T = mf::blocks_of(N, B);
  L.nchunk = T * B / kCB;
  L.vp = 0;
  L.es = up256((size_t)H_kv * L.nchunk * kCB * kD * 2);
  L.ef = L.es + up256((size_t)L.nchunk * H_kv * 4);
  L.total = L.ef + up256((size_t)L.nchunk * 4);
  return L;
}

template <bool kBF16, int RPW, int GS>
int launch_mfma_g(int NCH, dim3 grid, hipStream_t st, const int32_t* row_ptr,
                  const int32_t* col_idx, const unsigned short* vals, int64_t nnzb,
                  int H_s, int N, int B, const float* W, int H_r,
                  const unsigned short* Vp, const int* es, const int* ef, int nchunk,
                  int H_kv, unsigned short* O, int64_t ldO) {
#define MF_CASE(NCH_)                                                                     \
  case NCH_:                                                                              \
    hipLaunchKernelGGL((k_retrieve_mfma<kBF16, NCH_, RPW, GS>), grid, dim3(kThreads), 0, \
                       st, row_ptr, col_idx, vals, nnzb, H_s, N, B, W, H_r, Vp, es, ef,   \
                       nchunk, H_kv, O, ldO);                                             \
    break;
  switch (NCH) {
    MF_CASE(1) MF_CASE(2) MF_CASE(3) MF_CASE(4) MF_CASE(5) MF_CASE(6) MF_CASE(7)
    default: return mf::fail(MF_ERR_UNSUPPORTED, "k_retrieve_mfma: H_s out of range");
  }
#undef MF_CASE
  return mf::hip_check(hipGetLastError(), "k_retrieve_mfma launch");
}

// (receivers per wavefront, receivers per KV-group segment) pairs that are built
inline int mfma_group_split(int H_r, int H_kv) {
  if (H_r % 4 != 0) return 0;
  const int rpw = H_r / 4, G = H_r / H_kv;
  if (rpw != 2 && rpw != 4 && rpw != 6 && rpw != 8) return 0;
  if (rpw % G == 0 && rpw / G <= 2) return G;   // whole groups, one or two of them
  if (G % rpw == 0) return rpw;                  // inside one group
  return 0;
}

template <bool kBF16>
int launch_mfma(int NCH, int RPW, int GS, dim3 grid, hipStream_t st, const int32_t* row_ptr,
                const int32_t* col_idx, const unsigned short* vals, int64_t nnzb, int H_s,
                int N, int B, const float* W, int H_r, const unsigned short* Vp,
                const int* es, const int* ef, int nchunk, int H_kv, unsigned short* O,
                int64_t ldO) {
#define MF_G(R_, S_)                                                                    \
  if (RPW == R_ && GS == S_)                                                            \
    return launch_mfma_g<kBF16, R_, S_>(NCH, grid, st, row_ptr, col_idx, vals, nnzb,   \
                                        H_s, N, B, W, H_r, Vp, es, ef, nchunk, H_kv, O, \
                                        ldO);
  MF_G(8, 4) MF_G(8, 8) MF_G(6, 3) MF_G(6, 6) MF_G(4, 2) MF_G(4, 4) MF_G(2, 1) MF_G(2, 2)
#undef MF_G
  return mf::fail(MF_ERR_UNSUPPORTED, "k_retrieve_mfma: receiver/KV-head split not built");
}

}  // namespace

namespace mf {

bool retrieve_uses_mfma(int dt, int H_s, int B, int H_r, int H_kv, int d, const void* vals,
                        const void* O, int64_t ldO) {
  return dt != MF_F32 && d == kD && B >= 32 && H_r <= kMaxRecv && H_s <= kMaxHs &&
         mfma_group_split(H_r, H_kv) > 0 && aligned16(vals) && aligned16(O) &&
         (ldO % 8) == 0;
}

size_t retrieve_workspace_bytes(int N, int B, int H_kv, int d, int dt) {
  if (dt == MF_F32 || d != kD || B < 32) return 0;
  return ws_layout(N, B, H_kv).total;
}

int launch_retrieve(const int32_t* row_ptr, const int32_t* col_idx,
                    const void* vals, int64_t nnzb, int dt, int H_s, int N,
                    int B, const float* W, int H_r, const void* V, int H_kv,
                    int d, int64_t ldV, void* O, int64_t ldO, void* workspace,
                    size_t workspace_bytes, hipStream_t st) {
  if (retrieve_uses_mfma(dt, H_s, B, H_r, H_kv, d, vals, O, ldO) && workspace &&
      workspace_bytes >= ws_layout(N, B, H_kv).total) {
    const WsLayout L = ws_layout(N, B, H_kv);
    unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
    auto Vp = reinterpret_cast<unsigned short*>(ws + L.vp);
    auto es = reinterpret_cast<int*>(ws + L.es);
    auto ef = reinterpret_cast<int*>(ws + L.ef);
    auto Vs = reinterpret_cast<const unsigned short*>(V);
    if (dt == MF_BF16)
      hipLaunchKernelGGL(k_prep_values<true>, dim3(L.nchunk), dim3(kThreads), 0, st, Vs, N,
                         H_kv, ldV, L.nchunk, Vp, es, ef);
    else
      hipLaunchKernelGGL(k_prep_values<false>, dim3(L.nchunk), dim3(kThreads), 0, st, Vs, N,
                         H_kv, ldV, L.nchunk, Vp, es, ef);
    int rc = hip_check(hipGetLastError(), "k_prep_values launch");
    if (rc != MF_OK) return rc;
    const int T = blocks_of(N, B);
    const dim3 grid(((T + 7) / 8) * 8 * (B / kRows));
    const int NCH = (H_s + 7) / 8;
    const int RPW = H_r / 4, GS = mfma_group_split(H_r, H_kv);
    auto vp = reinterpret_cast<const unsigned short*>(vals);
    auto Op = reinterpret_cast<unsigned short*>(O);
    if (dt == MF_BF16)
      return launch_mfma<true>(NCH, RPW, GS, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, W, H_r, Vp, es, ef, L.nchunk, H_kv, Op, ldO);
    return launch_mfma<false>(NCH, RPW, GS, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, W, H_r, Vp, es, ef, L.nchunk, H_kv, Op, ldO);
  }
  if (dt == MF_F32)
    return launch_simple<mfd::TF32>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
  if (dt == MF_F16)
    return launch_simple<mfd::TF16>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
  return launch_simple<mfd::TBF16>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
}

}  // namespace mf
