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
//                 fp16 copy in the matrix-core operand layout
//                 Vp[g][key/8][d][8] (eight consecutive keys of one head-dim
//                 column are 16 contiguous bytes).  Each 16-key chunk of each
//                 KV head gets a power-of-two scale 2^-e (e >= 0; e = 0 unless
//                 |V| reaches 2^15) that keeps the copy in fp16 range; the
//                 matching 2^e is folded into the mixed map before it is
//                 rounded to fp16.
//
// k_retrieve_mfma (fp16/bf16, d = 128, B in {32,64,128}, H_r = 4*{2,4,6,8},
//                  H_s <= 48, H_kv <= 8)
//   Work item = (block row I, 16-row slice); one 256-thread workgroup owns all
//   receiver heads and all of d for its 16 query rows, so every kept tile
//   element leaves HBM once.  The row's kept blocks are walked in 16-key
//   chunks through a software pipeline in which every operand reaches the
//   matrix cores from LDS:
//   * per chunk, the [H_s][16][16] tile slice (triple buffered) and the
//     [H_kv][16 keys][128] slice of the prepared V (double buffered) are
//     copied HBM/L2 -> LDS with the gfx950 direct-to-LDS 16-byte loads, two
//     chunks ahead, through asm wrappers with explicit counter waits: loads
//     complete in issue order, so one wait per chunk (for the V slice about
//     to be used) also covers the next tile slice, and no barrier drains the
//     prefetch;
//   * head mix on MFMA 16x16x32 (M = 16 receiver heads, K = sender heads,
//     N = 16 tile positions); each wavefront owns one M tile and 8 rows.  B
//     operands are 16-byte LDS runs of 8 sender heads, transposed in
//     registers (v_perm_b32).  bf16 tiles use bf16 MFMA with W split into
//     hi + lo bf16 halves (W enters exactly, tiles need no conversion; the lo
//     half of a partly filled K step rides in its empty K slots); fp16 tiles
//     use fp16 MFMA with W in fp16;
//   * the fp32 mixed map is rounded to fp16 into a swizzled LDS tile, which is
//     also the re-layout to "query rows across lanes, keys along K";
//   * Ahat . V on MFMA 32x32x16 f16 with M = two receiver heads of one KV
//     group x 16 rows (16x16x16 when receivers cannot be paired inside a
//     group), N = 32 head-dim columns, K = the chunk's 16 keys;
//   * accumulators (16 rows x RPW heads x 128 d per wavefront) stay in AGPRs
//     for the whole row; O is written once through an LDS transpose as
//     16-byte stores.
//   Blocks of consecutive rows go to one XCD, so the V slices of their shared
//   band columns stay in that XCD's L2.
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
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kD = 128;          // head dim of the MFMA kernel
constexpr int kRows = 16;        // query rows per work item
constexpr int kCB = 16;          // keys per pipeline chunk
constexpr int kMaxRecv = 32;     // receiver heads of the MFMA kernel
constexpr int kMaxHs = 48;       // sender heads of the MFMA kernel
constexpr int kMaxKV = 8;        // KV heads of the MFMA kernel
constexpr int kHeadSlot = kRows * kCB * 2;        // bytes: one head of one chunk
constexpr int kVSlot = kMaxKV * kCB * kD * 2;     // bytes: V slice of one chunk
constexpr int kAhatBytes = kMaxRecv * kRows * kCB * 2;
constexpr int kVDma = kVSlot / 1024 / 4;          // V copies per wavefront per chunk

__device__ __forceinline__ f16x8 as_f16x8(const u32x4& v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ f16x4 as_f16x4(const uint2& v) { return __builtin_bit_cast(f16x4, v); }

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

// The retrieval loop issues its vector-memory traffic through these wrappers
// and waits on it explicitly.  Loads return in issue order, so "at most n
// newer operations outstanding" identifies exactly which data has landed; the
// compiler, unaware of these operations, adds no conservative waits of its own.
__device__ __forceinline__ void dma16(const void* g, unsigned lds_base) {
  // 16 bytes per lane from memory straight into LDS at lds_base + 16 * lane
  asm volatile("s_mov_b32 m0, %0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(g) : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}
// Workgroup barrier for LDS traffic only (outstanding memory loads stay in flight).
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
// V preparation: one workgroup per (64 keys, KV head)
// ---------------------------------------------------------------------------

template <bool kBF16, bool kVec>
__global__ __launch_bounds__(kThreads) void k_prep_values(
    const unsigned short* __restrict__ V, int N, int H_kv, int64_t ldV, int nkey8,
    unsigned short* __restrict__ Vp, int* __restrict__ escale) {
  __shared__ unsigned short tile[64][kD + 2];
  const int k0 = blockIdx.x * 64;
  const int g = blockIdx.y;
  const int tid = threadIdx.x;
  const int key = k0 + (tid >> 2);      // one key per 4 threads, 32 d each
  const int dq = (tid & 3) * 32;
  float v[32];
  if (key < N) {
    const unsigned short* src = V + (int64_t)key * ldV + (int64_t)g * kD + dq;
    if constexpr (kVec) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(src + 8 * j);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const unsigned short lo = w[e] & 0xffffu, hi = w[e] >> 16;
          v[8 * j + 2 * e] = kBF16 ? bf16_to_f32(lo) : f16_to_f32(lo);
          v[8 * j + 2 * e + 1] = kBF16 ? bf16_to_f32(hi) : f16_to_f32(hi);
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) v[e] = kBF16 ? bf16_to_f32(src[e]) : f16_to_f32(src[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 32; ++e) v[e] = 0.f;
  }
  // per 16-key chunk (= one wavefront) range scale
  float mx = 0.f;
#pragma unroll
  for (int e = 0; e < 32; ++e) mx = fmaxf(mx, fabsf(v[e]));
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  int ex = 0;
  if (kBF16 && mx >= 32768.f) {
    int x;
    frexpf(mx, &x);                     // mx < 2^x
    ex = min(x - 15, 120);
  }
#pragma unroll
  for (int e = 0; e < 32; ++e) tile[tid >> 2][dq + e] = f32_to_f16(__builtin_ldexpf(v[e], -ex));
  if ((tid & 63) == 0) escale[(int64_t)(k0 / kCB + (tid >> 6)) * H_kv + g] = ex;
  __syncthreads();
  // Vp[g][key/8][d][8]: thread -> (8-key group, d), 4 per thread
#pragma unroll
  for (int rep = 0; rep < 4; ++rep) {
    const int e = tid + rep * kThreads;
    const int c8 = e >> 7, dd = e & (kD - 1);
    u32x4 pk;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      pk[j] = (unsigned)tile[8 * c8 + 2 * j][dd] | ((unsigned)tile[8 * c8 + 2 * j + 1][dd] << 16);
    const int64_t row8 = (int64_t)g * nkey8 + k0 / 8 + c8;
    *reinterpret_cast<u32x4*>(Vp + (row8 * kD + dd) * 8) = pk;
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------

// Work item of workgroup b: blocks of RG consecutive block rows are dealt to
// the 8 XCDs in turn (workgroups go to XCDs round-robin by index), so rows
// that share band columns share an L2; within an XCD rows are taken from the
// last to the first.
__device__ __forceinline__ int item_of(int b, int subs, int T, int RG, int* I, int* sub) {
  const int xcd = b & 7;
  const int local = b >> 3;
  const int lrow = local / subs;                 // row index within this XCD's list
  const int grp = (lrow / RG) * 8 + xcd;         // global row group
  const int row_slot = grp * RG + lrow % RG;
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
  static constexpr __host__ __device__ int nw(int b) {
    return !kBF16 ? 1 : (b < F ? 2 : (R == 3 ? 2 : 1));
  }
  static __device__ __forceinline__ int chunk(int b, int q) {
    if (!kBF16) { const int c = 4 * b + q; return c < NCH ? c : -1; }
    if (b < F || R == 3) { const int c = 4 * b + q; return c < NCH ? c : -1; }
    return q < 2 * R ? 4 * F + (q % R) : -1;
  }
  static __device__ __forceinline__ int half(int b, int w, int q) {
    if (!kBF16) return 0;
    if (b < F || R == 3) return w;
    return q < R ? 0 : 1;
  }
};

// RPW receiver heads per wavefront (H_r = 4 * RPW); GS consecutive receivers
// share one KV group inside a wavefront (GS = G when a wavefront spans two
// groups, GS = RPW when it lies inside one): local receiver rl reads group
// g0 + rl / GS.  With GS even, receivers are paired for the 32x32 A.V.
template <bool kBF16, int NCH, int RPW, int GS>
__global__ __launch_bounds__(kThreads, 1) void k_retrieve_mfma(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const unsigned short* __restrict__ vals, int64_t nnzb, int H_s, int N,
    int B, const float* __restrict__ W, int H_r,
    const unsigned short* __restrict__ Vp, const int* __restrict__ escale,
    int nkey8, int H_kv, unsigned short* __restrict__ O, int64_t ldO, int RG) {
  using Plan = HmPlan<kBF16, NCH>;
  constexpr int NBOP = Plan::NBOP;
  constexpr int MT = RPW > 4 ? 2 : 1;             // 16-receiver M tiles of the head mix
  constexpr bool kPairs = (GS % 2) == 0;          // 32x32x16 A.V on receiver pairs
  constexpr int NSTG = 3;                         // tile-slice buffers in flight
  constexpr int kStage = 8 * NCH * kHeadSlot;     // one tile slice: head slots 0..8*NCH-1
  constexpr int NDV = NCH;                        // tile-slice copies per wavefront per chunk
  constexpr int kSmem = NSTG * kStage + 2 * kVSlot + kAhatBytes;
  static_assert(kSmem <= 160 * 1024, "LDS budget");
  static_assert(RPW % GS == 0 && RPW / GS <= 2, "at most two KV groups per wavefront");
  __shared__ __align__(16) unsigned char smem[kSmem];
  unsigned char* vstage = smem + NSTG * kStage;
  unsigned short* Ahs = reinterpret_cast<unsigned short*>(smem + NSTG * kStage + 2 * kVSlot);

  const int T = (N + B - 1) / B;
  const int subs = B / kRows;
  int I, sub;
  if (!item_of(blockIdx.x, subs, T, RG, &I, &sub)) return;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15;
  const int q = lane >> 4;

  // ---- head mix role: M tile hm_mt, tile rows 8*(wave&1)..+7 -------------
  const int hm_mt = wave >> 1;
  const bool hm_on = hm_mt < MT;
  u32x4 wop[NBOP][2];
#pragma unroll
  for (int b = 0; b < NBOP; ++b)
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int r = 16 * hm_mt + n;
      const int c = Plan::chunk(b, q);
      const int hf = Plan::half(b, w, q);
      unsigned short hv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = 8 * c + j;
        const float x = (w < Plan::nw(b) && c >= 0 && r < H_r && s < H_s) ? W[(int64_t)r * H_s + s] : 0.f;
        if (kBF16) {
          const unsigned short hi = bf16_bits(x);
          hv[j] = hf == 0 ? hi : bf16_bits(x - bf16_to_f32(hi));
        } else {
          hv[j] = f32_to_f16(x);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) wop[b][w][j] = (unsigned)hv[2 * j] | ((unsigned)hv[2 * j + 1] << 16);
    }

  // ---- accumulators ---------------------------------------------------------
  constexpr int NACC = kPairs ? RPW / 2 : RPW;
  constexpr int NDT = kPairs ? 4 : 8;
  using AccT = typename std::conditional<kPairs, f32x16, f32x4>::type;
  AccT acc[NACC][NDT];
#pragma unroll
  for (int p = 0; p < NACC; ++p)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[p][dt] = AccT{};

  const int G = H_r / H_kv;
  const int rbeg = wave * RPW;
  const int g0 = rbeg / G;
  int64_t kb = row_ptr[I], ke = row_ptr[I + 1];
  kb = kb < 0 ? 0 : (kb > nnzb ? nnzb : kb);
  ke = ke < kb ? kb : (ke > nnzb ? nnzb : ke);
  const int ncc = B / kCB;
  const int nchunks = (int)(ke - kb) * ncc;
  const int64_t tile_elems = (int64_t)B * B;

  // chunk u -> (kept block k, 16-key column chunk cc, global 16-key chunk of V)
  auto chunk_of = [&](int u, int64_t* k, int* cc, int* vch, bool* ok) {
    *k = kb + u / ncc;
    *cc = u % ncc;
    const int J = col_idx[*k];
    *ok = (J >= 0 && J < T);
    *vch = *ok ? (J * B + *cc * kCB) / kCB : 0;
  };
  // tile slice: [H_s][16 rows][16 keys]; one copy = 2 heads x 16 rows x 32 bytes
  const int lane_row = (lane & 31) >> 1;
  const int lane_off = (sub * kRows + lane_row) * B + (lane & 1) * 8;
  auto issue_vals = [&](int u) {
    int64_t k; int cc, vch; bool ok;
    chunk_of(u, &k, &cc, &vch, &ok);
    const unsigned base = lds_addr(smem + (u % NSTG) * kStage);
    const unsigned short* src0 = vals + k * H_s * tile_elems + lane_off + cc * kCB;
#pragma unroll
    for (int m = 0; m < NDV; ++m) {
      const int pair = wave + 4 * m;                    // heads 2*pair, 2*pair+1
      int s = 2 * pair + (lane >> 5);
      s = s < H_s ? s : H_s - 1;                        // padding slots get a real head (zero weight)
      dma16(src0 + s * tile_elems, base + pair * 1024);
    }
  };
  // V slice: [g][2 x 8 keys][128][8] = 4 KB per KV head, copied in 1 KB pieces
  auto issue_v = [&](int u) {
    int64_t k; int cc, vch; bool ok;
    chunk_of(u, &k, &cc, &vch, &ok);
    const unsigned base = lds_addr(vstage + (u & 1) * kVSlot);
#pragma unroll
    for (int m = 0; m < kVDma; ++m) {
      const int piece = wave + 4 * m;                   // 0..31
      int g = piece >> 2;
      g = g < H_kv ? g : H_kv - 1;
      const unsigned short* src =
          Vp + ((int64_t)g * nkey8 + (int64_t)vch * 2) * kD * 8 + (piece & 3) * 512 + lane * 8;
      dma16(src, base + piece * 1024);
    }
  };

  constexpr int NDMA = NDV + kVDma;
  // prologue: vals(0), vals(1), V(0), vals(2), V(1)  (the steady-state order)
  if (nchunks > 0) issue_vals(0);
  if (nchunks > 1) issue_vals(1);
  if (nchunks > 0) issue_v(0);
  if (nchunks > 2) issue_vals(2);
  if (nchunks > 1) issue_v(1);
  if (nchunks > 0) {
    // vals(0) must have landed before the first head mix
    if (nchunks > 2) wait_vm<2 * NDV + 2 * kVDma>();
    else if (nchunks > 1) wait_vm<NDV + 2 * kVDma>();
    else wait_vm<kVDma>();
    lds_barrier();
  }

  const int hrow = 8 * (wave & 1) + (n >> 1);          // head-mix tile row of this lane
  const int hcg = n & 1;                               // 8-key half of the chunk
  for (int u = 0; u < nchunks; ++u) {
    int64_t k; int cc, vch; bool jok;
    chunk_of(u, &k, &cc, &vch, &jok);

    // ---- head mix: M tile hm_mt, rows hrow, 16 keys -------------------------
    if (hm_on) {
      const unsigned short* buf = reinterpret_cast<const unsigned short*>(smem + (u % NSTG) * kStage);
      f32x4 c[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) c[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int b = 0; b < NBOP; ++b) {
        // lane groups without a chunk read chunk 0; their W slots are zero
        const int ch = Plan::chunk(b, q) < 0 ? 0 : Plan::chunk(b, q);
        u32x4 x[8], y[8];
#pragma unroll
        for (int uu = 0; uu < 8; ++uu)
          x[uu] = *reinterpret_cast<const u32x4*>(buf + ((8 * ch + uu) * kRows + hrow) * kCB + hcg * 8);
        transpose8x8(x, y);
#pragma unroll
        for (int w = 0; w < Plan::nw(b); ++w)
#pragma unroll
          for (int t = 0; t < 8; ++t) {
            if constexpr (kBF16)
              c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wop[b][w]), as_bf16x8(y[t]), c[t], 0, 0, 0);
            else
              c[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(wop[b][w]), as_f16x8(y[t]), c[t], 0, 0, 0);
          }
      }
      // lane (n, q) holds Ahat[16 hm_mt + 4q + a][hrow][8 hcg + t]; rows of Ahs
      // are 32 bytes, their two 16-byte halves swapped on rows 8..15
      // a block with an invalid column contributes nothing: its mixed map is
      // zeroed (the A.V below runs unconditionally on a valid V slice)
      int scale_any = 0;
      if (jok)
        for (int g = 0; g < H_kv; ++g) scale_any |= escale[(int64_t)vch * H_kv + g];
      const float zero_if_bad = jok ? 1.f : 0.f;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int r = 16 * hm_mt + 4 * q + a;
        if (r < H_r) {
          const float sc = scale_any ? __builtin_ldexpf(1.f, escale[(int64_t)vch * H_kv + r / G])
                                     : zero_if_bad;
          u32x4 pk;
#pragma unroll
          for (int j = 0; j < 4; ++j) pk[j] = pack_f16x2(c[2 * j][a] * sc, c[2 * j + 1][a] * sc);
          *reinterpret_cast<u32x4*>(&Ahs[(r * kRows + hrow) * kCB + 8 * (hcg ^ (hrow >> 3))]) = pk;
        }
      }
    }
    // V(u) landed (and, being issued later, vals(u+1) too)
    if (u + 2 < nchunks) wait_vm<NDV + kVDma>();
    else if (u + 1 < nchunks) wait_vm<kVDma>();
    else wait_vm<0>();
    lds_barrier();
    if (u + 3 < nchunks) issue_vals(u + 3);

    // ---- Ahat . V -------------------------------------------------------------
    {
      const unsigned char* vb = vstage + (u & 1) * kVSlot;
      if constexpr (kPairs) {
        const int m = lane & 31, hh = lane >> 5;
        const int rp = m >> 4, i = m & 15;
        u32x4 bop[2][4];
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          const int g = min(g0 + gi, H_kv - 1);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
            bop[gi][dt] = *reinterpret_cast<const u32x4*>(vb + ((g * 2 + hh) * kD + 32 * dt + m) * 16);
        }
#pragma unroll
        for (int p = 0; p < NACC; ++p) {
          const int r = rbeg + 2 * p + rp;
          const u32x4 a4 = *reinterpret_cast<const u32x4*>(&Ahs[(r * kRows + i) * kCB + 8 * (hh ^ (i >> 3))]);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
            acc[p][dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                as_f16x8(a4), as_f16x8(bop[(2 * p) / GS][dt]), acc[p][dt], 0, 0, 0);
        }
      } else {
        uint2 bop[2][8];
#pragma unroll
        for (int gi = 0; gi < 2; ++gi) {
          const int g = min(g0 + gi, H_kv - 1);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            bop[gi][dt] = *reinterpret_cast<const uint2*>(
                vb + ((g * 2 + (q >> 1)) * kD + 16 * dt + n) * 16 + (q & 1) * 8);
        }
#pragma unroll
        for (int rl = 0; rl < RPW; ++rl) {
          const int r = rbeg + rl;
          const uint2 a2 = *reinterpret_cast<const uint2*>(
              &Ahs[(r * kRows + n) * kCB + 8 * ((q >> 1) ^ (n >> 3)) + 4 * (q & 1)]);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
            acc[rl][dt] = __builtin_amdgcn_mfma_f32_16x16x16f16(
                as_f16x4(a2), as_f16x4(bop[rl / GS][dt]), acc[rl][dt], 0, 0, 0);
        }
      }
    }
    lds_barrier();
    if (u + 2 < nchunks) issue_v(u + 2);
  }

  // ---- store through LDS: one receiver head at a time per wavefront --------
  unsigned short* ot = reinterpret_cast<unsigned short*>(smem) + wave * (kRows * kD);
#pragma unroll
  for (int rl = 0; rl < RPW; ++rl) {
    const int r = rbeg + rl;
    lds_barrier();
    if constexpr (kPairs) {
      // acc[rl/2][dt][e]: row m = 8(e>>2) + 4(lane>>5) + (e&3) of the pair,
      // receiver m>>4, tile row m&15, column d = 32 dt + (lane&31)
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if ((m >> 4) == (rl & 1)) {
            const float v = acc[rl >> 1][dt][e];
            ot[(m & 15) * kD + 32 * dt + (lane & 31)] = kBF16 ? bf16_bits(v) : f32_to_f16(v);
          }
        }
    } else {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const float v = acc[rl][dt][a];
          ot[(4 * q + a) * kD + 16 * dt + n] = kBF16 ? bf16_bits(v) : f32_to_f16(v);
        }
    }
    lds_barrier();
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

// Workspace layout of the MFMA path: Vp | escale (each 256-byte aligned).
struct WsLayout {
  size_t vp, es, total;
  int nkey8;      // 8-key rows of Vp per KV head (covers T*B keys, a multiple of 64)
};
inline size_t up256(size_t x) { return (x + 255) & ~(size_t)255; }
inline WsLayout ws_layout(int N, int B, int H_kv) {
  WsLayout L;
  const int T = mf::blocks_of(N, B);
  const int keys = ((T * B + 63) / 64) * 64;
  L.nkey8 = keys / 8;
  L.vp = 0;
  L.es = up256((size_t)H_kv * keys * kD * 2);
  L.total = L.es + up256((size_t)(keys / kCB) * H_kv * 4);
  return L;
}

template <bool kBF16, int RPW, int GS>
int launch_mfma_g(int NCH, dim3 grid, hipStream_t st, const int32_t* row_ptr,
                  const int32_t* col_idx, const unsigned short* vals, int64_t nnzb,
                  int H_s, int N, int B, const float* W, int H_r,
                  const unsigned short* Vp, const int* es, int nkey8, int H_kv,
                  unsigned short* O, int64_t ldO, int RG) {
#define MF_CASE(NCH_)                                                                     \
  case NCH_:                                                                              \
    hipLaunchKernelGGL((k_retrieve_mfma<kBF16, NCH_, RPW, GS>), grid, dim3(kThreads), 0, \
                       st, row_ptr, col_idx, vals, nnzb, H_s, N, B, W, H_r, Vp, es,       \
                       nkey8, H_kv, O, ldO, RG);                                          \
    break;
  switch (NCH) {
    MF_CASE(1) MF_CASE(2) MF_CASE(3) MF_CASE(4) MF_CASE(5) MF_CASE(6)
    default: return mf::fail(MF_ERR_UNSUPPORTED, "k_retrieve_mfma: H_s out of range");
  }
#undef MF_CASE
  return mf::hip_check(hipGetLastError(), "k_retrieve_mfma launch");
}

// Receiver split per wavefront: returns GS (receivers per KV-group segment
// inside a wavefront) for the built (RPW, GS) pairs, 0 otherwise.
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
                const int* es, int nkey8, int H_kv, unsigned short* O, int64_t ldO, int RG) {
#define MF_G(R_, S_)                                                                    \
  if (RPW == R_ && GS == S_)                                                            \
    return launch_mfma_g<kBF16, R_, S_>(NCH, grid, st, row_ptr, col_idx, vals, nnzb,   \
                                        H_s, N, B, W, H_r, Vp, es, nkey8, H_kv, O, ldO, \
                                        RG);
  MF_G(8, 4) MF_G(8, 8) MF_G(6, 3) MF_G(6, 6) MF_G(4, 2) MF_G(4, 4) MF_G(2, 1) MF_G(2, 2)
#undef MF_G
  return mf::fail(MF_ERR_UNSUPPORTED, "k_retrieve_mfma: receiver/KV-head split not built");
}

}  // namespace

namespace mf {

bool retrieve_uses_mfma(int dt, int H_s, int B, int H_r, int H_kv, int d, const void* vals,
                        const void* O, int64_t ldO) {
  return dt != MF_F32 && d == kD && B >= 32 && H_r <= kMaxRecv && H_s <= kMaxHs &&
         H_kv <= kMaxKV && mfma_group_split(H_r, H_kv) > 0 && aligned16(vals) &&
         aligned16(O) && (ldO % 8) == 0;
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
    auto Vs = reinterpret_cast<const unsigned short*>(V);
    const bool vec = aligned16(V) && (ldV % 8) == 0;
    const dim3 pgrid(L.nkey8 / 8, H_kv);
    if (dt == MF_BF16) {
      if (vec) hipLaunchKernelGGL((k_prep_values<true, true>), pgrid, dim3(kThreads), 0, st, Vs, N, H_kv, ldV, L.nkey8, Vp, es);
      else hipLaunchKernelGGL((k_prep_values<true, false>), pgrid, dim3(kThreads), 0, st, Vs, N, H_kv, ldV, L.nkey8, Vp, es);
    } else {
      if (vec) hipLaunchKernelGGL((k_prep_values<false, true>), pgrid, dim3(kThreads), 0, st, Vs, N, H_kv, ldV, L.nkey8, Vp, es);
      else hipLaunchKernelGGL((k_prep_values<false, false>), pgrid, dim3(kThreads), 0, st, Vs, N, H_kv, ldV, L.nkey8, Vp, es);
    }
    int rc = hip_check(hipGetLastError(), "k_prep_values launch");
    if (rc != MF_OK) return rc;
    const int T = blocks_of(N, B);
    const int RG = std::max(1, T / 16);
    const int groups = (T + RG - 1) / RG;
    const int rows_per_xcd = ((groups + 7) / 8) * RG;
    const dim3 grid(rows_per_xcd * 8 * (B / kRows));
    const int NCH = (H_s + 7) / 8;
    const int RPW = H_r / 4, GS = mfma_group_split(H_r, H_kv);
    auto vp = reinterpret_cast<const unsigned short*>(vals);
    auto Op = reinterpret_cast<unsigned short*>(O);
    if (dt == MF_BF16)
      return launch_mfma<true>(NCH, RPW, GS, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, W, H_r, Vp, es, L.nkey8, H_kv, Op, ldO, RG);
    return launch_mfma<false>(NCH, RPW, GS, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, W, H_r, Vp, es, L.nkey8, H_kv, Op, ldO, RG);
  }
  if (dt == MF_F32)
    return launch_simple<mfd::TF32>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
  if (dt == MF_F16)
    return launch_simple<mfd::TF16>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
  return launch_simple<mfd::TBF16>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
}

}  // namespace mf
