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
// k_retrieve_mfma (fp16/bf16, d = 128, B in {16,32,64,128}, H_r in
//                  {8,16,24,32}, H_s <= 48, each wavefront's receivers in
//                  one KV group)
//   Work item = (block row I, 16-row slice); one 512-thread workgroup (eight
//   wavefronts, two per SIMD) owns all receiver heads and all of d for its 16
//   query rows, so every kept tile element leaves HBM once.  The row's kept
//   blocks are walked in 16-key chunks.  Phase u of the loop, between two
//   workgroup barriers, does
//     * A.V of chunk u: MFMA 32x32x16 with M = two receiver heads x 16 rows,
//       N = 32 head-dim columns, K = the chunk's 16 keys, accumulating in
//       registers for the whole row (wavefront w owns receivers
//       [w*H_r/8, (w+1)*H_r/8), which share one KV head);
//     * head mix of chunk u+1: MFMA 16x16x32 with M = 16 receiver heads,
//       K = sender heads, N = 16 (row, key) positions; each wavefront owns one
//       M tile and 4 rows; the fp32 result goes to a double-buffered LDS tile
//       in the A.V operand layout;
//     * loads: the V rows of chunk u+1, each wavefront copying its own KV
//       head's 16 x 128 block into its own LDS slot (read back at the start
//       of the next phase with 8-byte LDS reads and transposed in registers
//       so that each lane holds eight consecutive keys of four head-dim
//       columns), then the [H_s][16 rows][16 keys] tile slice of chunk u+3,
//       both with the gfx950 direct-to-LDS 16-byte loads; the slice copies
//       sit between the A.V MFMAs (three slices in flight).
//   Loads return in issue order, so one counter wait per phase ("all but the
//   newest tile slice") covers both V and the slice needed next; no barrier
//   drains the prefetch.
//   bf16: the head mix runs on bf16 MFMA with W split into hi + lo bf16 halves
//   (W enters exactly); the fp32 mixed map is split the same way into hi + lo
//   bf16 planes, and A.V runs on bf16 MFMA for both planes against the bf16 V
//   as stored, so nothing is rounded except the mixed map's hi + lo split
//   (16 significant bits).  fp16: W and the mixed map are rounded to fp16, V
//   is used as stored.
//   Blocks of consecutive rows go to one XCD, and every row walks its kept
//   blocks as a rotation of their ascending order chosen so that rows of
//   equal length meet each band column at the same step (the four 16-row
//   slices of a row take the block's 16-key chunks in staggered order): the
//   V rows of a shared band column are then read by all of that XCD's
//   workgroups within a few phases and come from L2, not HBM.  The output is
//   written once with non-temporal stores.
//
// k_retrieve_simple (every other supported case, including fp32)
//   One workgroup per (block row, receiver head): the mixed tile is built in
//   LDS in fp32, then multiplied with V by plain fp32 FMAs.
//
// Packed batches (chunked prefill and paged caches are what the pages' serving
// integration has to live with: paper page, "Practical Implementation
// Details"): both kernels also take a batch of sequences in one launch.  The
// block rows of all sequences are numbered globally (sequence s owns rows
// cu_rows[s] .. cu_rows[s+1]-1 of row_ptr) and V, O are packed by token
// (sequence s starts at token cu_seqlens[s]); a work item finds its sequence
// by binary search and then runs exactly as for a single sequence.  An
// optional block table names, for each kept block, its page in a tile pool,
// so the compressed state of many sequences (or layers) can live in one
// allocation; a page outside the pool contributes nothing.
#include <algorithm>
#include <type_traits>

#include "mf_internal.h"

namespace {

using namespace mfd;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;          // MFMA kernel workgroup
constexpr int kSimpleThreads = 256;            // plain kernel workgroup
constexpr int kD = 128;                        // head dim of the MFMA kernel
constexpr int kRows = 16;                      // query rows per work item
constexpr int kCB = 16;                        // keys per pipeline chunk
constexpr int kMaxRecv = 32;                   // receiver heads of the MFMA kernel
constexpr int kMaxHs = 48;                     // sender heads of the MFMA kernel
constexpr int kHeadSlot = kRows * kCB * 2;     // bytes: one head of one tile slice
constexpr int kPlane = kMaxRecv * kRows * kCB * 2;  // bytes: one mixed-map plane
constexpr int kOutSlot = 2 * kRows * kD * 2;   // bytes: a receiver pair's output rows
constexpr int kVSlot = kCB * kD * 2;           // bytes: one KV head's V rows of one chunk

__device__ __forceinline__ f16x8 as_f16x8(const u32x4& v) { return __builtin_bit_cast(f16x8, v); }
__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) { return __builtin_bit_cast(bf16x8, v); }

// 8x4 transpose of 16-bit elements held as 8 rows of 4 (u32x2 each):
// out[t] element j = in[j] element t.
__device__ __forceinline__ void transpose8x4(const u32x2 (&x)[8], u32x4 (&y)[4]) {
  constexpr unsigned kLo = 0x05040100u;  // low halves of (src1, src0)
  constexpr unsigned kHi = 0x07060302u;  // high halves of (src1, src0)
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      y[t][m] = __builtin_amdgcn_perm(x[2 * m + 1][t >> 1], x[2 * m][t >> 1], (t & 1) ? kHi : kLo);
}

// The retrieval loop issues its vector-memory traffic through these wrappers
// and waits on it explicitly.  Loads return in issue order, so "at most n
// newer operations outstanding" identifies exactly which data has landed; the
// compiler, unaware of these operations, adds no conservative waits of its own.
// Hazards the compiler does not see through inline asm, handled inside each
// statement: an SGPR written by a VALU instruction (v_readfirstlane) needs 5
// wait states before a vector-memory instruction reads it (s_nop 4), and M0
// written by SALU needs 1 before an LDS DMA reads it (s_nop 0).
__device__ __forceinline__ void dma16(const void* g, unsigned lds_base) {
  // 16 bytes per lane from memory straight into LDS at lds_base + 16 * lane
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               :: "s"(lds_base), "v"(g) : "memory", "m0");
}
// A wave-uniform pointer, guaranteed to live in scalar registers.
__device__ __forceinline__ const void* sgpr_ptr(const void* p) {
  const unsigned long long v = reinterpret_cast<unsigned long long>(p);
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)v);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  return reinterpret_cast<const void*>(((unsigned long long)hi << 32) | lo);
}
// Same copy with a wave-uniform base address and a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16s(unsigned voff, const void* sbase, unsigned lds_base) {
  asm volatile("s_nop 4\n\ts_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_base), "v"(voff), "s"(sgpr_ptr(sbase)) : "memory", "m0");
}
// The same copy with a base computed by scalar instructions only: no VALU
// write of it to wait for (the static checks confirm it).
__device__ __forceinline__ void dma16b(unsigned voff, const void* sbase, unsigned lds_base) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_base), "v"(voff), "s"(sbase) : "memory", "m0");
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
// Packed batches
// ---------------------------------------------------------------------------

// One receiver of a sender's BSR state: its head map, values and output.
struct Recv {
  const float* W;
  const void* V;
  void* O;
  int64_t ldV, ldO;
  int H_r, RPW, G;
};
constexpr int kMaxRecvSets = 4;

// The general form of a launch: a packed batch of sequences (cu_rows null:
// one sequence of N tokens whose block rows are the whole row_ptr), tiles
// optionally read through a block table, and up to kMaxRecvSets receivers fed
// from the same BSR state.  Kernels take it with kVar = true; with kVar =
// false they see one sequence and one receiver (the kernel arguments) and the
// batch fields are not read.
struct Batch {
  const int32_t* cu_rows;      // [S+1] first global block row of each sequence
  const int32_t* cu_seqlens;   // [S+1] first token of each sequence in V and O
  const int32_t* block_table;  // [nnzb] pool page of each kept block, or nullptr
  int64_t n_pages;             // tiles in the pool (bounds block_table entries)
  int S;
  int n_recv;                  // receivers; more than 1: recv[] replaces W, V, O
  Recv recv[kMaxRecvSets];
};
// The kernels take the batch's index arrays (cu_rows, cu_seqlens,
// block_table) again as separate read-only, non-aliased arguments: read
// through the struct they become vector loads, each followed by a wait on
// every outstanding tile copy; as restrict arguments they are scalar loads.

// The sequence of global block row Ig: its local row I, block rows T, tokens
// N and first token tok0.  False when the row holds no query row.
struct RowView {
  int I, T, N;
  int64_t tok0;
};
template <bool kVar>
__device__ __forceinline__ bool row_view(const Batch& bt, const int32_t* __restrict__ cu_rows,
                                         const int32_t* __restrict__ cu_seqlens, int Ig, int N,
                                         int B, RowView& rv) {
  if (!kVar || cu_rows == nullptr) {
    rv.I = Ig;
    rv.N = N;
    rv.T = (N + B - 1) / B;
    rv.tok0 = 0;
    return true;
  }
  int lo = 0, hi = bt.S - 1;                     // last s with cu_rows[s] <= Ig
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_rows[mid] <= Ig) lo = mid; else hi = mid - 1;
  }
  rv.I = Ig - cu_rows[lo];
  rv.T = cu_rows[lo + 1] - cu_rows[lo];
  rv.tok0 = cu_seqlens[lo];
  rv.N = cu_seqlens[lo + 1] - cu_seqlens[lo];
  return rv.I >= 0 && rv.I < rv.T && (int64_t)rv.I * B < rv.N;
}
// Table entry of kept block k (k itself without a table), unchecked: the
// retrieval loop loads it a phase before it checks it with page_ok, so that
// the load's latency stays off the copy issue.  The load is issued either way
// (from col_idx, a valid address for every k < nnzb, when there is no table):
// a load inside a branch gets a wait of its own at the branch's end.
template <bool kVar>
__device__ __forceinline__ int64_t page_raw(const int32_t* __restrict__ block_table,
                                            const int32_t* __restrict__ col_idx, int64_t k) {
  if (!kVar) return k;
  const int64_t v = (block_table ? block_table : col_idx)[k];
  return block_table ? v : k;
}
__device__ __forceinline__ bool page_ok(const Batch& bt, int64_t p) { return p >= 0 && p < bt.n_pages; }
// Pool page of kept block k, or -1 when the table points outside the pool.
template <bool kVar>
__device__ __forceinline__ int64_t page_of(const Batch& bt, const int32_t* __restrict__ block_table,
                                           int64_t k) {
  if (!kVar || block_table == nullptr) return k;
  const int64_t p = block_table[k];
  return page_ok(bt, p) ? p : -1;
}

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------

// Work item of workgroup b: blocks of RG consecutive block rows are dealt to
// the 8 XCDs (workgroups go to XCDs round-robin by index, whatever their
// load), so rows that share band columns share an L2; the deal runs forward
// and backward in turn over the XCDs, so that rows of unequal length even out
// across them; within an XCD rows are taken from the last to the first.
__device__ __forceinline__ int item_of(int b, int subs, int T, int RG, int* I, int* sub) {
  const int xcd = b & 7;
  const int local = b >> 3;
  const int lrow = local / subs;                 // row index within this XCD's list
  const int rnd = lrow / RG;                     // deal round
  const int grp = rnd * 8 + ((rnd & 1) ? 7 - xcd : xcd);   // global row group
  const int row_slot = grp * RG + lrow % RG;
  if (row_slot >= T) return 0;
  *I = T - 1 - row_slot;
  *sub = local % subs;
  return 1;
}

// Block rows per group dealt to one XCD.  Groups of 16 rows (a sixteenth of
// the rows) left the long-context layer, whose rows keep 1 to 66 blocks, with
// one XCD doing four times the work of another; groups of R/64 rows dealt in
// alternating order even that out and lose nothing on the other layers.
inline int row_group(int R) { return R / 64 > 1 ? R / 64 : 1; }

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
    return q < 2 * R ? 4 * F + (q % (R ? R : 1)) : -1;
  }
  static __device__ __forceinline__ int half(int b, int w, int q) {
    if (!kBF16) return 0;
    if (b < F || R == 3) return w;
    return q < R ? 0 : 1;
  }
};

// NPAIR = ceil(RPW / 2) receiver pairs per wavefront, RPW = H_r / 8 receivers
// (a pair's second receiver past RPW is computed from valid data and never
// stored).  lg_ncc = log2(B / 16).
template <bool kBF16, int NCH, int NPAIR, bool kVar>
__global__ __launch_bounds__(kThreads, 1) void k_retrieve_mfma(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const unsigned short* __restrict__ vals, int64_t nnzb, int H_s, int N, int B,
    int lg_ncc, const float* __restrict__ W, int H_r, int RPW, int G,
    const unsigned short* __restrict__ V, int64_t ldV,
    unsigned short* __restrict__ O, int64_t ldO, int RG, Batch bt,
    const int32_t* __restrict__ cu_rows, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ block_table, int R) {
  using Plan = HmPlan<kBF16, NCH>;
  constexpr int NBOP = Plan::NBOP;
  constexpr int NPL = kBF16 ? 2 : 1;               // mixed-map planes (hi, lo)
  constexpr int NSTG = (kBF16 && NCH == 6) ? 2 : 3;  // tile-slice buffers (LDS budget)
  constexpr int kStage = 8 * NCH * kHeadSlot;      // one tile slice: head slots 0..8*NCH-1
  constexpr int NPR = 4 * NCH;                     // 1 KB copies per tile slice
  constexpr int NDV = (NPR + kWaves - 1) / kWaves; // copies per wavefront per slice
  constexpr int kAhatOff = NSTG * kStage;
  constexpr int kAhatBuf = NPL * kPlane;
  constexpr int kVOff = kAhatOff + 2 * kAhatBuf;   // per-wavefront V slots
  constexpr int kUsed = kVOff + kWaves * kVSlot;
  constexpr int kSmem = kUsed > kWaves * kOutSlot ? kUsed : kWaves * kOutSlot;
  static_assert(kSmem <= 160 * 1024, "LDS budget");
  static_assert(NPAIR == 1 || NPAIR == 2, "receiver pairs per wavefront");
  __shared__ __align__(16) unsigned char smem[kSmem];

  const int subs = B / kRows;
  int bid = blockIdx.x;
  if constexpr (kVar) {
    // several receivers: the work items of one (row, slice) for each receiver
    // are consecutive among the workgroups one XCD receives (index b, b+8,
    // b+16, ...), so they run together and read the row's tiles from that
    // XCD's L2 after the first one has fetched them
    if (bt.n_recv > 1) {
      const int local = bid >> 3;
      const Recv& rc = bt.recv[local % bt.n_recv];
      bid = (bid & 7) | ((local / bt.n_recv) << 3);
      W = rc.W;
      H_r = rc.H_r;
      RPW = rc.RPW;
      G = rc.G;
      V = reinterpret_cast<const unsigned short*>(rc.V);
      ldV = rc.ldV;
      O = reinterpret_cast<unsigned short*>(rc.O);
      ldO = rc.ldO;
    }
  }
  int Ig, sub;                                   // global block row, 16-row slice
  if (!item_of(bid, subs, R, RG, &Ig, &sub)) return;
  RowView rv;
  if (!row_view<kVar>(bt, cu_rows, cu_seqlens, Ig, N, B, rv)) return;
  const int I = rv.I;                            // block row within its sequence
  const int T = rv.T;
  N = rv.N;
  V += rv.tok0 * ldV;
  O += rv.tok0 * ldO;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int n = lane & 15;
  const int q = lane >> 4;

  // ---- head-mix role: M tile hm_mt (receivers 16 hm_mt..+15), rows 4 rq..+3
  const int hm_mt = wave >> 2;
  const int rq = wave & 3;
  u32x4 wop[NBOP][2];
#pragma unroll
  for (int b = 0; b < NBOP; ++b)
#pragma unroll
    for (int w = 0; w < Plan::nw(b); ++w) {
      const int r = 16 * hm_mt + n;
      const int c = Plan::chunk(b, q);
      const int hf = Plan::half(b, w, q);
      unsigned short hv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int s = 8 * c + j;
        const bool ok = c >= 0 && r < H_r && s < H_s;
        const float x = W[ok ? r * H_s + s : 0];       // unconditional: all loads in flight together
        const float xv = ok ? x : 0.f;
        if constexpr (kBF16) {
          const unsigned short hi = bf16_bits(xv);
          hv[j] = hf == 0 ? hi : bf16_bits(xv - bf16_to_f32(hi));
        } else {
          hv[j] = f32_to_f16(xv);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) wop[b][w][j] = (unsigned)hv[2 * j] | ((unsigned)hv[2 * j + 1] << 16);
    }
  // the W loads must have landed before the first counted asm load is issued
#pragma unroll
  for (int b = 0; b < NBOP; ++b) asm volatile("" :: "v"(wop[b][0]));

  // ---- accumulators ---------------------------------------------------------
  f32x16 acc[NPAIR][4];
#pragma unroll
  for (int p = 0; p < NPAIR; ++p)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[p][dt] = f32x16{};

  const int rbeg = wave * RPW;
  const int g = rbeg / G;
  int64_t kb = row_ptr[Ig], ke = row_ptr[Ig + 1];
  kb = kb < 0 ? 0 : (kb > nnzb ? nnzb : kb);
  ke = ke < kb ? kb : (ke > nnzb ? nnzb : ke);
  const int ncc_mask = (1 << lg_ncc) - 1;
  const int cnt = (int)(ke - kb);
  const int n_chunks = cnt << lg_ncc;
  const int64_t tile = (int64_t)B * B;
  // The row's kept blocks are walked as a rotation of their ascending order
  // starting at position (cnt - 1 - I) mod cnt: a row whose list ends in the
  // band of diagonal columns then meets column J at step J mod cnt, the same
  // step as every other row of equal length, so neighbouring rows on one XCD
  // read each band column's V rows at about the same time and share them in
  // L2 instead of re-fetching them.
  const int rot = cnt > 0 ? cnt - 1 - I % cnt : 0;
  auto block_of = [&](int x) -> int64_t {       // kept block of chunk x (clamped)
    x = x < n_chunks ? x : n_chunks - 1;
    const int t = (x >> lg_ncc) + rot;
    return kb + (t >= cnt ? t - cnt : t);
  };
  auto col_ok = [&](int J) { return J >= 0 && J < T; };
  // valid keys at the start of chunk x of column J: 16, fewer in the chunk
  // that reaches past N, 0 for an invalid column
  auto kvalid_of = [&](int x, int J) -> int {
    if (!col_ok(J)) return 0;
    const int xc = x < n_chunks ? x : n_chunks - 1;
    const int rem = N - (J * B + ((xc + sub) & ncc_mask) * kCB);
    return rem < kCB ? (rem < 0 ? 0 : rem) : kCB;
  };
  // column of chunk x's block; -1 (never valid) when its page is outside the pool
  auto col_of = [&](int x) -> int {
    const int64_t k = block_of(x);
    if constexpr (!kVar) return col_idx[k];
    else return page_of<kVar>(bt, block_table, k) >= 0 ? col_idx[k] : -1;
  };

  // tile-slice copy d of this wavefront: 1 KB piece pr = wave + 8d (heads 2pr,
  // 2pr+1), issued only for pr < NPR, so wavefronts issue NDV or NDV-1 copies;
  // lane -> (head 2pr + lane/32, tile row (lane%32)/2, 16-byte half lane%2)
  const int ndv_w = (NPR - wave + kWaves - 1) / kWaves;  // copies of this wavefront
  const int64_t lane_off = (int64_t)(sub * kRows + ((lane & 31) >> 1)) * B + (lane & 1) * 8;
  unsigned head_off[NDV];                        // byte offset of this lane's 16 bytes in a block
#pragma unroll
  for (int d = 0; d < NDV; ++d) {
    int s = 2 * (wave + kWaves * d) + (lane >> 5);
    s = s < H_s ? s : H_s - 1;                  // padding slots get a real head (zero weight)
    head_off[d] = (unsigned)((s * tile + lane_off) * 2);
  }
  const unsigned smem_lds = lds_addr(smem);
  // chunk x covers keys 16 * ((x + sub) mod B/16) of its block: the row
  // slices of one block row take the block's chunks in staggered order
  // (with a block table the page of chunk x is passed in: the loop loads it
  // one phase ahead, so its latency stays out of the copy issue)
  auto vals_src = [&](int x, int64_t pg = 0) -> const unsigned short* {
    const int xc = x < n_chunks ? x : n_chunks - 1;
    if constexpr (!kVar) return vals + block_of(x) * H_s * tile + ((xc + sub) & ncc_mask) * kCB;
    return vals + (page_ok(bt, pg) ? pg : 0) * H_s * tile + ((xc + sub) & ncc_mask) * kCB;
  };
  auto copy_piece = [&](const unsigned short* src, int slot, int d) {
    if (d < ndv_w) dma16s(head_off[d], src, smem_lds + slot * kStage + (wave + kWaves * d) * 1024);
  };
  auto issue_vals = [&](int x, int slot) {
    const unsigned short* src = vals_src(x, page_of<kVar>(bt, block_table, block_of(x)));
#pragma unroll
    for (int d = 0; d < NDV; ++d) copy_piece(src, slot, d);
  };
  // s_waitcnt vmcnt(n) for a wave-uniform n in [0, 2 NDV]
  auto wait_vm_n = [&](int n) {
    switch (n) {
      case 0: wait_vm<0>(); break;
      case 1: wait_vm<1>(); break;
      case 2: wait_vm<2>(); break;
      case 3: wait_vm<3>(); break;
      case 4: wait_vm<4>(); break;
      case 5: wait_vm<5>(); break;
      default: wait_vm<6>(); break;
    }
  };
  static_assert(NDV <= 3, "copies per wavefront per slice");

  // V rows of chunk x for this wavefront's KV head g: 16 keys x 128 columns,
  // copied as four 1 KB pieces (lane -> key 4m + lane/16, columns
  // 8*(lane%16)..+7) into the wavefront's own LDS slot [16 keys][128].  A chunk
  // that reaches past row N (only the last one of a partial block) copies row
  // N-1 instead, whose weight is zero.
  const unsigned vslot = smem_lds + kVOff + wave * kVSlot;
  const unsigned v_off = (unsigned)(((int64_t)(lane >> 4) * ldV + g * kD + (lane & 15) * 8) * 2);
  const unsigned short* vlane = V + (int64_t)g * kD + (lane & 15) * 8;
  auto issue_v = [&](int x, int J) {
    const int xc = x < n_chunks ? x : n_chunks - 1;
    const int key0 = (col_ok(J) ? J : 0) * B + ((xc + sub) & ncc_mask) * kCB;
    if (key0 + kCB <= N) {
#pragma unroll
      for (int m = 0; m < 4; ++m) dma16s(v_off, V + (int64_t)(key0 + 4 * m) * ldV, vslot + m * 1024);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int key = key0 + 4 * m + (lane >> 4);
        dma16(vlane + (int64_t)(key < N ? key : N - 1) * ldV, vslot + m * 1024);
      }
    }
  };
  // A.V B operand from the slot: lane -> keys 8*(lane/32)..+7, columns
  // 4*(lane%32)..+3, transposed to vt[dt] = 8 keys of column 4*(lane%32)+dt
  const unsigned char* vsl = smem + kVOff + wave * kVSlot + 8 * (lane & 31) + 2048 * (lane >> 5);
  auto read_vt = [&](u32x4 (&vt)[4]) {
    u32x2 xv[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) xv[j] = *reinterpret_cast<const u32x2*>(vsl + j * 256);
    transpose8x4(xv, vt);
  };

  // head mix of chunk x from tile slot `slot` into mixed-map buffer `ab`;
  // `kvalid` = number of valid keys at the start of the chunk (0: invalid
  // column or padding chunk); the mixed map is zero from there on, selected
  // rather than multiplied, so whatever the skipped tile positions hold
  // (padding past N, a block outside the row's columns) never reaches O
  const int hrow = 4 * rq + (n >> 2);            // tile row of this lane
  const int hkq = n & 3;                         // 4-key quarter of the chunk
  const int hm_off = hrow * 32 + (((hkq >> 1) ^ ((hrow >> 2) & 1)) * 16) + (hkq & 1) * 8;
  auto key_ok = [&](int kvalid, int t) { return 4 * hkq + t < kvalid; };
  auto head_mix = [&](int slot, int kvalid, int ab) {
    const unsigned char* st = smem + slot * kStage + hrow * 32 + hkq * 8;
    f32x4 c[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < NBOP; ++b) {
      // lane groups without a chunk read chunk 0; their W slots are zero
      const int ch = Plan::chunk(b, q) < 0 ? 0 : Plan::chunk(b, q);
      u32x2 x[8];
      u32x4 y[4];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        x[j] = *reinterpret_cast<const u32x2*>(st + (8 * ch + j) * kHeadSlot);
      transpose8x4(x, y);
#pragma unroll
      for (int w = 0; w < Plan::nw(b); ++w)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if constexpr (kBF16)
            c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wop[b][w]), as_bf16x8(y[t]), c[t], 0, 0, 0);
          else
            c[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(wop[b][w]), as_f16x8(y[t]), c[t], 0, 0, 0);
        }
    }
    // lane (n, q) holds Ahat[16 hm_mt + 4q + a][hrow][4 hkq + t]; a plane is
    // [32 receivers][16 rows][16 keys], its rows' two 16-byte halves swapped
    // when bit 2 of the row is set
    unsigned char* dst = smem + kAhatOff + ab * kAhatBuf + hm_off;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int r = 16 * hm_mt + 4 * q + a;
      const f32x2 v01 = {key_ok(kvalid, 0) ? c[0][a] : 0.f, key_ok(kvalid, 1) ? c[1][a] : 0.f};
      const f32x2 v23 = {key_ok(kvalid, 2) ? c[2][a] : 0.f, key_ok(kvalid, 3) ? c[3][a] : 0.f};
      if constexpr (kBF16) {
        const unsigned h01 = __builtin_bit_cast(unsigned, __builtin_convertvector(v01, bf16x2));
        const unsigned h23 = __builtin_bit_cast(unsigned, __builtin_convertvector(v23, bf16x2));
        const f32x2 r01 = {v01[0] - __uint_as_float(h01 << 16), v01[1] - __uint_as_float(h01 & 0xffff0000u)};
        const f32x2 r23 = {v23[0] - __uint_as_float(h23 << 16), v23[1] - __uint_as_float(h23 & 0xffff0000u)};
        const unsigned l01 = __builtin_bit_cast(unsigned, __builtin_convertvector(r01, bf16x2));
        const unsigned l23 = __builtin_bit_cast(unsigned, __builtin_convertvector(r23, bf16x2));
        *reinterpret_cast<u32x2*>(dst + r * 512) = u32x2{h01, h23};
        *reinterpret_cast<u32x2*>(dst + kPlane + r * 512) = u32x2{l01, l23};
      } else {
        *reinterpret_cast<u32x2*>(dst + r * 512) =
            u32x2{pack_f16x2(v01[0], v01[1]), pack_f16x2(v23[0], v23[1])};
      }
    }
  };

  // A.V operand addressing
  const int am = lane & 31;
  const int a_off = (am & 15) * 32 + (((lane >> 5) ^ ((am >> 2) & 1)) * 16);

  // One phase's compute, in an explicit order that keeps the matrix cores fed:
  // head-mix operand reads, head-mix MFMAs with the next operand's transpose
  // between them, then the A.V MFMAs with the packing of the head-mix result
  // between them.  sched_barrier stops the compiler from regrouping the parts.
  auto compute = [&](int slot, int kvalid, int ab_hm, int ab_av, const u32x4 (&vt)[4], auto&& mid_copy, auto&& step_copy) {
    const unsigned char* st = smem + slot * kStage + hrow * 32 + hkq * 8;
    f32x4 c[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x2 x[8];
    {
      const int ch = Plan::chunk(0, q) < 0 ? 0 : Plan::chunk(0, q);
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = *reinterpret_cast<const u32x2*>(st + (8 * ch + j) * kHeadSlot);
    }
    __builtin_amdgcn_sched_barrier(0);
    mid_copy();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < NBOP; ++b) {
      u32x4 y[4];
      transpose8x4(x, y);
      if (b + 1 < NBOP) {
        const int ch = Plan::chunk(b + 1, q) < 0 ? 0 : Plan::chunk(b + 1, q);
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = *reinterpret_cast<const u32x2*>(st + (8 * ch + j) * kHeadSlot);
      }
#pragma unroll
      for (int w = 0; w < Plan::nw(b); ++w)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          if constexpr (kBF16)
            c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wop[b][w]), as_bf16x8(y[t]), c[t], 0, 0, 0);
          else
            c[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(wop[b][w]), as_f16x8(y[t]), c[t], 0, 0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
    }
    // A.V operands
    const unsigned char* asrc = smem + kAhatOff + ab_av * kAhatBuf + a_off;
    unsigned char* dst = smem + kAhatOff + ab_hm * kAhatBuf + hm_off;
#pragma unroll
    for (int p = 0; p < NPAIR; ++p) {
      const int r = rbeg + 2 * p + (am >> 4);
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) {
        const u32x4 a4 = *reinterpret_cast<const u32x4*>(asrc + pl * kPlane + r * 512);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          if constexpr (kBF16)
            acc[p][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a4), as_bf16x8(vt[dt]), acc[p][dt], 0, 0, 0);
          else
            acc[p][dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a4), as_f16x8(vt[dt]), acc[p][dt], 0, 0, 0);
        }
        // pack receiver row a = 2p + pl of the head-mix result between the MFMAs
        constexpr int kSteps = NPAIR * NPL;
#pragma unroll
        for (int a = (p * NPL + pl) * 4 / kSteps; a < (p * NPL + pl + 1) * 4 / kSteps; ++a) {
          const int rr = 16 * hm_mt + 4 * q + a;
          const f32x2 v01 = {key_ok(kvalid, 0) ? c[0][a] : 0.f, key_ok(kvalid, 1) ? c[1][a] : 0.f};
          const f32x2 v23 = {key_ok(kvalid, 2) ? c[2][a] : 0.f, key_ok(kvalid, 3) ? c[3][a] : 0.f};
          if constexpr (kBF16) {
            const unsigned h01 = __builtin_bit_cast(unsigned, __builtin_convertvector(v01, bf16x2));
            const unsigned h23 = __builtin_bit_cast(unsigned, __builtin_convertvector(v23, bf16x2));
            const f32x2 r01 = {v01[0] - __uint_as_float(h01 << 16), v01[1] - __uint_as_float(h01 & 0xffff0000u)};
            const f32x2 r23 = {v23[0] - __uint_as_float(h23 << 16), v23[1] - __uint_as_float(h23 & 0xffff0000u)};
            const unsigned l01 = __builtin_bit_cast(unsigned, __builtin_convertvector(r01, bf16x2));
            const unsigned l23 = __builtin_bit_cast(unsigned, __builtin_convertvector(r23, bf16x2));
            *reinterpret_cast<u32x2*>(dst + rr * 512) = u32x2{h01, h23};
            *reinterpret_cast<u32x2*>(dst + kPlane + rr * 512) = u32x2{l01, l23};
          } else {
            *reinterpret_cast<u32x2*>(dst + rr * 512) =
                u32x2{pack_f16x2(v01[0], v01[1]), pack_f16x2(v23[0], v23[1])};
          }
        }
        step_copy(p * NPL + pl);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- pipeline ---------------------------------------------------------------
  // Phase u: V(u) from the wavefront's slot into registers; head-mix operand
  // reads; copy V(u+1) into the (now read) slot; head mix(u+1); A.V(u) with the
  // copies of tile slice u+NSTG issued between its MFMAs, so that the copies
  // drain through the vector-memory path while the matrix cores work; wait for
  // V(u+1) and slice u+2; barrier.  Each wavefront copies and reads only its own
  // V slot; tile slices are shared through the barrier.
  constexpr int kSteps = NPAIR * NPL;            // A.V steps that can carry a copy
  int J1 = 0;                                    // column of chunk u+1
  int slot = 0;                                  // u % NSTG
  if (n_chunks > 0) {
    const int J0 = col_of(0);
    J1 = col_of(1);
    issue_v(0, J0);
#pragma unroll
    for (int st = 0; st < NSTG; ++st) issue_vals(st, st);
    wait_vm_n((NSTG - 1) * ndv_w);               // V(0) and slice 0 landed
    lds_barrier();
    head_mix(0, kvalid_of(0, J0), 0);
    wait_vm_n((NSTG - 2) * ndv_w);               // slice 1 landed
    lds_barrier();
  }
  int64_t pg_n = 0;                              // table entry of chunk u + NSTG
  if constexpr (kVar)
    if (n_chunks > 0) pg_n = page_raw<kVar>(block_table, col_idx, block_of(NSTG));
  for (int u = 0; u < n_chunks; ++u) {
    // column (and, with a table, page) of chunk u+2: loaded now, combined
    // after this phase's barrier, so neither load waits inside the phase
    const int64_t kn = block_of(u + 2);
    const int Jn_col = col_idx[kn];
    int64_t pg_J = 0;
    if constexpr (kVar) pg_J = page_raw<kVar>(block_table, col_idx, kn);
    u32x4 vt[4];
    read_vt(vt);
    const unsigned short* vsrc = vals_src(u + NSTG, pg_n);
    if constexpr (kVar) pg_n = page_raw<kVar>(block_table, col_idx, block_of(u + NSTG + 1));
    const int cur = slot;
    const int s1 = slot + 1 == NSTG ? 0 : slot + 1;
    auto mid_copy = [&]() {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slot read before it is refilled
      issue_v(u + 1, J1);
    };
    auto step_copy = [&](int step) {
      // tile-slice copies spread over the A.V steps; the last step takes the rest
#pragma unroll
      for (int d = 0; d < NDV; ++d)
        if ((d * kSteps) / NDV == step || (step == kSteps - 1 && (d * kSteps) / NDV >= kSteps))
          copy_piece(vsrc, cur, d);
    };
    compute(s1, u + 1 < n_chunks ? kvalid_of(u + 1, J1) : 0, (u + 1) & 1, u & 1, vt, mid_copy, step_copy);
    wait_vm_n((NSTG - 2) * ndv_w);               // V(u+1) and slice u+2 landed
    lds_barrier();
    J1 = (!kVar || page_ok(bt, pg_J)) ? Jn_col : -1;
    slot = s1;
  }
  wait_vm<0>();
  lds_barrier();

  // ---- store through LDS: one receiver pair at a time per wavefront ---------
  unsigned short* ot = reinterpret_cast<unsigned short*>(smem + wave * kOutSlot);  // [16 rows][2][128]
#pragma unroll
  for (int p = 0; p < NPAIR; ++p) {
    if (p) lds_barrier();
    // acc[p][dt][e]: row m = 8(e>>2) + 4(lane>>5) + (e&3) of the pair (receiver
    // m>>4, tile row m&15), head-dim column 4 (lane&31) + dt
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      unsigned short h[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) h[dt] = kBF16 ? bf16_bits(acc[p][dt][e]) : f32_to_f16(acc[p][dt][e]);
      *reinterpret_cast<u32x2*>(ot + ((m & 15) * 2 + (m >> 4)) * kD + 4 * am) =
          u32x2{(unsigned)h[0] | ((unsigned)h[1] << 16), (unsigned)h[2] | ((unsigned)h[3] << 16)};
    }
    lds_barrier();
    // 16 rows x 2 receivers x 256 bytes, 16 contiguous bytes per lane
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int c16 = pass * 64 + lane;
      const int i = c16 >> 5, rp = (c16 >> 4) & 1, d8 = (c16 & 15) * 8;
      const int64_t grow = (int64_t)I * B + sub * kRows + i;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ot + (i * 2 + rp) * kD + d8);
      if (2 * p + rp < RPW && grow < N)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(O + grow * ldO + (int64_t)(rbeg + 2 * p + rp) * kD + d8));
    }
  }
}

// ---------------------------------------------------------------------------
// MFMA kernel, pair-stage form (B >= 32)
// ---------------------------------------------------------------------------
//
// The same work items, head-mix plan and A.V tiling as k_retrieve_mfma, with
// the memory traffic reorganised:
//   * tile slices are copied as key pairs: one 1 KB copy moves one sender
//     head's [16 rows][32 keys], i.e. 64 contiguous bytes of each tile row
//     (half a 128-byte line instead of a quarter), into one of two pair
//     stages [head slot][16 rows][32 keys]; a pair serves two consecutive
//     16-key phases;
//   * the V rows of the next chunk come straight into registers (eight 8-byte
//     loads per lane, issued at the start of the phase before their use), so
//     LDS holds only tile pairs and the two mixed-map buffers;
//   * the head mix reads its B operands out of the stage with the gfx950
//     transposing LDS read (ds_read_b64_tr_b16), which hands each lane four
//     sender heads of one (row, key) position, instead of reading head rows
//     and transposing them in registers; for that, MFMA t of a chunk covers
//     keys 4t..4t+3 of four rows, the mixed map is stored with the chunk's
//     keys in the order 0,4,8,12,1,5,9,13,2,6,10,14,3,7,11,15, and V is
//     loaded in the same order, so A.V pairs the same keys on both sides;
//   * V and tile bases are computed by scalar instructions only, one 64-bit
//     product per chunk and a row stride per load.
// Pair P goes into stage P % 2 once the head mix of the previous occupant's
// last chunk has passed a barrier: its copies are issued between the A.V
// MFMAs of phase 2P-3 (behind that phase's V loads) and waited for at the end
// of phase 2P-2.

// Split rows.  When a few long block rows would set the time of a launch (the
// rows of a near-dense map run from 1 to T kept blocks), every row with more
// than P kept blocks is cut into ceil(cnt / P) parts of balanced length.  The
// work items are then the rows from the last to the first, each row's parts in
// order; a part writes its fp32 partial output to the workspace, and
// k_split_combine adds a row's partials in part order, so the output is the
// same bit for bit on every run.  Rows of at most P blocks write O directly.
struct Split {
  float* part;            // [item][slice][16 rows][H_r][128] fp32 partials
  int32_t* first_item;    // [T] item index of part 0 of each split row
  int P;                  // longest part, in kept blocks
};
__device__ __forceinline__ int split_parts(int64_t cnt, int P) {
  return cnt > P ? (int)((cnt + P - 1) / P) : 1;
}
// Item j of the split list -> block row I, part index, part count; false when
// j is past the last item.  All 512 threads of the workgroup take part; `buf`
// is LDS for 8 + 4 ints.
__device__ bool split_item(const int32_t* __restrict__ row_ptr, int64_t nnzb, int T, int P, int j,
                           int* buf, int& I, int& part, int& parts) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int per = (T + kThreads - 1) / kThreads;  // item-order rows per thread
  const int i0 = tid * per;
  auto row_cnt = [&](int i) -> int64_t {          // kept blocks of the i-th row in item order
    const int r = T - 1 - i;
    int64_t kb = row_ptr[r], ke = row_ptr[r + 1];
    kb = kb < 0 ? 0 : (kb > nnzb ? nnzb : kb);
    ke = ke < kb ? kb : (ke > nnzb ? nnzb : ke);
    return ke - kb;
  };
  int mine = 0;
  for (int i = i0; i < i0 + per && i < T; ++i) mine += split_parts(row_cnt(i), P);
  int incl = mine;                                // inclusive scan within the wavefront
  for (int off = 1; off < 64; off <<= 1) {
    const int v = __shfl_up(incl, off, 64);
    if (lane >= off) incl += v;
  }
  if (lane == 63) buf[wave] = incl;
  __syncthreads();
  int base = 0, total = 0;
  for (int w = 0; w < kWaves; ++w) {
    const int v = buf[w];
    base += w < wave ? v : 0;
    total += v;
  }
  const int excl = base + incl - mine;
  if (j >= excl && j < excl + mine) {             // this thread's rows hold item j
    int k = excl;
    for (int i = i0; i < i0 + per && i < T; ++i) {
      const int np = split_parts(row_cnt(i), P);
      if (j < k + np) {
        buf[kWaves] = T - 1 - i;
        buf[kWaves + 1] = j - k;
        buf[kWaves + 2] = np;
        break;
      }
      k += np;
    }
  }
  __syncthreads();
  I = buf[kWaves];
  part = buf[kWaves + 1];
  parts = buf[kWaves + 2];
  __syncthreads();                                // buf is reused by the caller
  return j < total;
}

// 8 bytes per lane from memory into a register pair: a per-lane address, or
// a wave-uniform base computed by scalar instructions (no VALU write of it to
// wait for; the static checks confirm it) and a 32-bit per-lane byte offset.
// The registers receive the data asynchronously; they are read only after
// wait_vm_regs() has retired the load.
__device__ __forceinline__ void vld8(u32x2& dst, const void* g) {
  asm volatile("global_load_dwordx2 %0, %1, off" : "=v"(dst) : "v"(g) : "memory");
}
__device__ __forceinline__ void vld8b(u32x2& dst, unsigned voff, const void* sbase) {
  asm volatile("global_load_dwordx2 %0, %1, %2"
               : "=v"(dst) : "v"(voff), "s"(sbase) : "memory");
}
// s_waitcnt vmcnt(N) that the eight V registers depend on, so that no read of
// them is scheduled above the wait.
template <int N>
__device__ __forceinline__ void wait_vm_regs(u32x2 (&x)[8]) {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%8)"
               : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]), "+v"(x[4]), "+v"(x[5]),
                 "+v"(x[6]), "+v"(x[7])
               : "n"(N) : "memory");
}

template <bool kBF16, int NCH, int NPAIR, bool kVar, bool kSplit = false>
__global__ __launch_bounds__(kThreads, 1) void k_retrieve_pair(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const unsigned short* __restrict__ vals, int64_t nnzb, int H_s, int N, int B,
    int lg_ncc, const float* __restrict__ W, int H_r, int RPW, int G,
    const unsigned short* __restrict__ V, int64_t ldV,
    unsigned short* __restrict__ O, int64_t ldO, int RG, Batch bt,
    const int32_t* __restrict__ cu_rows, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ block_table, int R, Split sp) {
  static_assert(!(kSplit && kVar), "split rows: one sequence, one receiver");
  using Plan = HmPlan<kBF16, NCH>;
  constexpr int NBOP = Plan::NBOP;
  constexpr int NPL = kBF16 ? 2 : 1;               // mixed-map planes (hi, lo)
  constexpr int kPieces = 8 * NCH;                 // 1 KB copies per pair: one per head slot
  constexpr int kHeadPair = 1024;                  // bytes: one head of one pair stage
  constexpr int kStage = kPieces * kHeadPair;      // [head slot][16 rows][32 keys]
  constexpr int kAhatOff = 2 * kStage;
  constexpr int kAhatBuf = NPL * kPlane;
  constexpr int kUsed = kAhatOff + 2 * kAhatBuf;
  constexpr int kSmem = kUsed > kWaves * kOutSlot ? kUsed : kWaves * kOutSlot;
  static_assert(kSmem <= 160 * 1024, "LDS budget");
  static_assert(NPAIR == 1 || NPAIR == 2, "receiver pairs per wavefront");
  static_assert(NCH <= 6, "copies per wavefront per pair");
  __shared__ __align__(16) unsigned char smem[kSmem];

  const int subs = B / kRows;
  int bid = blockIdx.x;
  if constexpr (kVar) {
    if (bt.n_recv > 1) {
      const int local = bid >> 3;
      const Recv& rc = bt.recv[local % bt.n_recv];
      bid = (bid & 7) | ((local / bt.n_recv) << 3);
      W = rc.W;
      H_r = rc.H_r;
      RPW = rc.RPW;
      G = rc.G;
      V = reinterpret_cast<const unsigned short*>(rc.V);
      ldV = rc.ldV;
      O = reinterpret_cast<unsigned short*>(rc.O);
      ldO = rc.ldO;
    }
  }
  int Ig, sub;
  int part = 0, parts = 1, item = 0;             // split rows: this item's part of its row
  if constexpr (kSplit) {
    // items dealt to the XCDs in turn, the slices of one item on one XCD
    const int local = bid >> 3;
    sub = local % subs;
    item = (local / subs) * 8 + (bid & 7);
    if (!split_item(row_ptr, nnzb, R, sp.P, item, reinterpret_cast<int*>(smem), Ig, part, parts))
      return;
  } else {
    if (!item_of(bid, subs, R, RG, &Ig, &sub)) return;
  }
  RowView rv;
  if (!row_view<kVar>(bt, cu_rows, cu_seqlens, Ig, N, B, rv)) return;
  const int I = rv.I;
  const int T = rv.T;
  N = rv.N;
  V += rv.tok0 * ldV;
  O += rv.tok0 * ldO;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;
  const int q = lane >> 4;

  // ---- head-mix role and W operands (as in k_retrieve_mfma) ----------------
  // The head map's loads go first, so that their round trip overlaps those of
  // row_ptr and of the first column; the conversion follows both.
  const int hm_mt = wave >> 2;
  const int rq = wave & 3;
  float wraw[NBOP][2][8];
#pragma unroll
  for (int b = 0; b < NBOP; ++b)
#pragma unroll
    for (int w = 0; w < Plan::nw(b); ++w)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 16 * hm_mt + n;
        const int c = Plan::chunk(b, q);
        const int s = 8 * c + j;
        const bool ok = c >= 0 && r < H_r && s < H_s;
        const float x = W[ok ? r * H_s + s : 0];
        wraw[b][w][j] = ok ? x : 0.f;
      }
  // ---- the row's kept blocks ------------------------------------------------
  int64_t kb = row_ptr[Ig], ke = row_ptr[Ig + 1];
  kb = kb < 0 ? 0 : (kb > nnzb ? nnzb : kb);
  ke = ke < kb ? kb : (ke > nnzb ? nnzb : ke);
  if constexpr (kSplit) {
    if (parts > 1) {                             // this part's balanced share of the row
      const int64_t len = (ke - kb + parts - 1) / parts;
      const int64_t k0 = kb + part * len;
      ke = k0 + len < ke ? k0 + len : ke;
      kb = k0 < ke ? k0 : ke;
      if (part == 0 && sub == 0 && threadIdx.x == 0) sp.first_item[Ig] = item;
    }
  }
  const int lg_npb = lg_ncc - 1;                 // pairs per block: B / 32
  const int npb_mask = (1 << lg_npb) - 1;
  const int cnt = (int)(ke - kb);
  const int n_chunks = cnt << lg_ncc;
  const int64_t tile = (int64_t)B * B;
  const int rot = (cnt > 0 && parts == 1) ? cnt - 1 - I % cnt : 0;
  auto block_of = [&](int x) -> int64_t {        // kept block of chunk x (clamped)
    x = x < n_chunks ? x : n_chunks - 1;
    const int t = (x >> lg_ncc) + rot;
    return kb + (t >= cnt ? t - cnt : t);
  };
  auto col_ok = [&](int J) { return J >= 0 && J < T; };
  // key offset of chunk x in its block: the pair's staggered position, then
  // the chunk's half of it (the row slices of one block row take the block's
  // pairs in staggered order)
  auto key_off = [&](int x) -> int {
    x = x < n_chunks ? x : n_chunks - 1;
    return ((((x >> 1) + sub) & npb_mask) << 5) + ((x & 1) << 4);
  };
  auto kvalid_of = [&](int x, int J) -> int {
    if (!col_ok(J)) return 0;
    const int rem = N - (J * B + key_off(x));
    return rem < kCB ? (rem < 0 ? 0 : rem) : kCB;
  };
  auto col_of = [&](int x) -> int {
    const int64_t k = block_of(x);
    if constexpr (!kVar) return col_idx[k];
    else return page_of<kVar>(bt, block_table, k) >= 0 ? col_idx[k] : -1;
  };
  // column of chunks 0 and 1 (one block: a block holds B/16 >= 2 chunks)
  const int J0 = n_chunks > 0 ? col_of(0) : 0;
  u32x4 wop[NBOP][2];
#pragma unroll
  for (int b = 0; b < NBOP; ++b)
#pragma unroll
    for (int w = 0; w < Plan::nw(b); ++w) {
      const int hf = Plan::half(b, w, q);
      unsigned short hv[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float xv = wraw[b][w][j];
        if constexpr (kBF16) {
          const unsigned short hi = bf16_bits(xv);
          hv[j] = hf == 0 ? hi : bf16_bits(xv - bf16_to_f32(hi));
        } else {
          hv[j] = f32_to_f16(xv);
        }
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) wop[b][w][j] = (unsigned)hv[2 * j] | ((unsigned)hv[2 * j + 1] << 16);
    }
#pragma unroll
  for (int b = 0; b < NBOP; ++b) asm volatile("" :: "v"(wop[b][0]));

  f32x16 acc[NPAIR][4];
#pragma unroll
  for (int p = 0; p < NPAIR; ++p)
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) acc[p][dt] = f32x16{};

  const int rbeg = wave * RPW;
  const int g = rbeg / G;

  // Pair-stage layout: head slot hs holds 16 rows of 64 bytes; the four
  // 16-byte quarters of each row sit in the order quarter ^ (hs % 4), so that
  // a transposing head-mix read (four heads x four rows, 8 bytes each, per
  // 16 lanes) meets every bank once.
  auto swz = [](int hs) { return hs & 3; };
  // tile-pair copy d of this wavefront: head slot hs = wave + 8d; lane -> the
  // 16 bytes at LDS offset 16*lane of the slot, i.e. tile row lane/4 and
  // quarter (lane%4) ^ swz
  unsigned head_off[NCH];
#pragma unroll
  for (int d = 0; d < NCH; ++d) {
    const int hs = wave + kWaves * d;
    const int s = hs < H_s ? hs : H_s - 1;      // padding slots get a real head (zero weight)
    const int row = lane >> 2;
    const int quarter = (lane & 3) ^ swz(hs);
    head_off[d] = (unsigned)((s * tile + (int64_t)(sub * kRows + row) * B + quarter * 8) * 2);
  }
  const unsigned smem_lds = lds_addr(smem);
  // copies of pair P (its first chunk 2P) into stage P % 2; with a block table
  // the page is passed in (loaded a phase ahead)
  auto issue_pair = [&](int P, int64_t pg, int d) {
    const int x = 2 * P;
    const unsigned short* src;
    if constexpr (!kVar) src = vals + block_of(x) * H_s * tile + key_off(x);
    else src = vals + (page_ok(bt, pg) ? pg : 0) * H_s * tile + key_off(x);
    dma16b(head_off[d], src, smem_lds + (P & 1) * kStage + (wave + kWaves * d) * kHeadPair);
  };
  auto pair_page = [&](int P) -> int64_t {
    if constexpr (!kVar) return 0;
    else return page_of<kVar>(bt, block_table, block_of(2 * P));
  };

  // V rows of chunk x for this wavefront's KV head g, straight into registers:
  // lane -> keys kperm(j) + 2*(lane/32) (j = 0..7) of columns 4*(lane%32)..+3.
  // The keys of a chunk are taken in the order 0,4,8,12,1,5,9,13 | 2,6,10,
  // 14,3,7,11,15 on both sides of A.V (the mixed map is stored in that
  // order, see pack_row).  A chunk reaching past row N (only the last of a
  // partial block) reads row N-1 for the missing keys; their mixed-map
  // weights are zero.
  auto kperm = [](int j) { return 4 * (j & 3) + (j >> 2); };
  const unsigned v_off = (unsigned)(((int64_t)(2 * (lane >> 5)) * ldV + g * kD + 4 * (lane & 31)) * 2);
  const unsigned short* vlane = V + (int64_t)g * kD + 4 * (lane & 31);
  const int64_t ldV2 = ldV * 2;                  // bytes per V row
  u32x2 xv[2][8];                                // raw V of the even and the odd chunks
  // loads j0 <= j < j1 of V(x) into xd
  auto issue_v_part = [&](int x, int J, u32x2 (&xd)[8], int j0, int j1) {
    const int key0 = (col_ok(J) ? J : 0) * B + key_off(x);
    if (key0 + kCB <= N) {
      // one 64-bit product per chunk, then a row stride per key
      const char* vb = reinterpret_cast<const char*>(V + (int64_t)key0 * ldV);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (j >= j0 && j < j1) vld8b(xd[j], v_off, vb + kperm(j) * ldV2);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int key = key0 + 2 * (lane >> 5) + kperm(j);
        if (j >= j0 && j < j1) vld8(xd[j], vlane + (int64_t)(key < N ? key : N - 1) * ldV);
      }
    }
  };
  auto issue_v = [&](int x, int J, u32x2 (&xd)[8]) { issue_v_part(x, J, xd, 0, 8); };

  // ---- head mix ---------------------------------------------------------------
  const int hrow = 4 * rq + (n >> 2);
  const int hkq = n & 3;
  const int hm_off = hrow * 32 + (((hkq >> 1) ^ ((hrow >> 2) & 1)) * 16) + (hkq & 1) * 8;
  // MFMA t of the head mix covers keys 4t + (position % 4): c[t] of this
  // lane is key 4t + hkq
  auto key_ok = [&](int kvalid, int t) { return 4 * t + hkq < kvalid; };
  // operand base of chunk x: its pair's stage and this lane's row; the
  // quarter (16-key half of the pair, 8-key half of that) is placed by
  // read_hm, which knows the sender group
  auto hm_base = [&](int x) -> const unsigned char* {
    return smem + ((x >> 1) & 1) * kStage;
  };
  auto pack_row = [&](unsigned char* dst, const f32x4 (&c)[4], int a, int kvalid) {
    const int rr = 16 * hm_mt + 4 * q + a;
    const f32x2 v01 = {key_ok(kvalid, 0) ? c[0][a] : 0.f, key_ok(kvalid, 1) ? c[1][a] : 0.f};
    const f32x2 v23 = {key_ok(kvalid, 2) ? c[2][a] : 0.f, key_ok(kvalid, 3) ? c[3][a] : 0.f};
    if constexpr (kBF16) {
      const unsigned h01 = __builtin_bit_cast(unsigned, __builtin_convertvector(v01, bf16x2));
      const unsigned h23 = __builtin_bit_cast(unsigned, __builtin_convertvector(v23, bf16x2));
      const f32x2 r01 = {v01[0] - __uint_as_float(h01 << 16), v01[1] - __uint_as_float(h01 & 0xffff0000u)};
      const f32x2 r23 = {v23[0] - __uint_as_float(h23 << 16), v23[1] - __uint_as_float(h23 & 0xffff0000u)};
      const unsigned l01 = __builtin_bit_cast(unsigned, __builtin_convertvector(r01, bf16x2));
      const unsigned l23 = __builtin_bit_cast(unsigned, __builtin_convertvector(r23, bf16x2));
      *reinterpret_cast<u32x2*>(dst + rr * 512) = u32x2{h01, h23};
      *reinterpret_cast<u32x2*>(dst + kPlane + rr * 512) = u32x2{l01, l23};
    } else {
      *reinterpret_cast<u32x2*>(dst + rr * 512) =
          u32x2{pack_f16x2(v01[0], v01[1]), pack_f16x2(v23[0], v23[1])};
    }
  };
  auto hm_mfmas = [&](const u32x4 (&y)[4], int b, f32x4 (&c)[4]) {
#pragma unroll
    for (int w = 0; w < Plan::nw(b); ++w)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        if constexpr (kBF16)
          c[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(wop[b][w]), as_bf16x8(y[t]), c[t], 0, 0, 0);
        else
          c[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_f16x8(wop[b][w]), as_f16x8(y[t]), c[t], 0, 0, 0);
      }
  };
  // B operands of group b for chunk half xh (x & 1), straight from the
  // stage with the transposing LDS read: for MFMA t, position n = 4r + e of
  // this 16-lane group is (row 4rq + r, key 4t + e), and its 8 sender heads
  // come from two reads in which source lane 4h + r points at keys 4t..4t+3
  // of head h (then h + 4) of that row.
  const int tr_h = (lane & 15) >> 2;
  const int tr_row = 4 * rq + (lane & 3);
  auto read_hm = [&](const unsigned char* st, int xh, int b, u32x4 (&y)[4]) {
    const int ch = Plan::chunk(b, q) < 0 ? 0 : Plan::chunk(b, q);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      unsigned w[4];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int slot = 8 * ch + 4 * hh + tr_h;
        const int quarter = ((xh << 1) | (t >> 1)) ^ swz(slot);
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
        const unsigned char* pa = st + slot * kHeadPair + tr_row * 64 + quarter * 16 + (t & 1) * 8;
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4*)(__attribute__((address_space(3))) unsigned char*)(pa));
        const u32x2 u = __builtin_bit_cast(u32x2, v);
        w[2 * hh] = u[0];
        w[2 * hh + 1] = u[1];
      }
      y[t] = u32x4{w[0], w[1], w[2], w[3]};
    }
  };
  // prologue form: head mix of chunk x into mixed-map buffer ab
  auto head_mix = [&](int x, int kvalid, int ab) {
    const unsigned char* st = hm_base(x);
    f32x4 c[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int b = 0; b < NBOP; ++b) {
      u32x4 y[4];
      read_hm(st, x & 1, b, y);
      hm_mfmas(y, b, c);
    }
    unsigned char* dst = smem + kAhatOff + ab * kAhatBuf + hm_off;
#pragma unroll
    for (int a = 0; a < 4; ++a) pack_row(dst, c, a, kvalid);
  };

  const int am = lane & 31;
  const int a_off = (am & 15) * 32 + (((lane >> 5) ^ ((am >> 2) & 1)) * 16);
  constexpr int kSteps = NPAIR * NPL;            // A.V steps that can carry a copy

  // One phase: head-mix operand reads and MFMAs of chunk x1 (next operand's
  // reads between them), the current chunk's V operands (prep_v), then its
  // A.V MFMAs with the packing of the head-mix result and the phase's loads
  // (step_copy) between them.
  auto compute = [&](int x1, int kvalid, int ab_hm, int ab_av, auto&& prep_v, auto&& step_copy) {
    const unsigned char* st = hm_base(x1);
    f32x4 c[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) c[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    u32x4 y[4];
    read_hm(st, x1 & 1, 0, y);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int b = 0; b < NBOP; ++b) {
      u32x4 yn[4];
      if (b + 1 < NBOP) read_hm(st, x1 & 1, b + 1, yn);
      hm_mfmas(y, b, c);
      if (b + 1 < NBOP) {
#pragma unroll
        for (int t = 0; t < 4; ++t) y[t] = yn[t];
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    u32x4 vt[4];
    prep_v(vt);
    const unsigned char* asrc = smem + kAhatOff + ab_av * kAhatBuf + a_off;
    unsigned char* dst = smem + kAhatOff + ab_hm * kAhatBuf + hm_off;
#pragma unroll
    for (int p = 0; p < NPAIR; ++p) {
      const int r = rbeg + 2 * p + (am >> 4);
#pragma unroll
      for (int pl = 0; pl < NPL; ++pl) {
        const u32x4 a4 = *reinterpret_cast<const u32x4*>(asrc + pl * kPlane + r * 512);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          if constexpr (kBF16)
            acc[p][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a4), as_bf16x8(vt[dt]), acc[p][dt], 0, 0, 0);
          else
            acc[p][dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16x8(a4), as_f16x8(vt[dt]), acc[p][dt], 0, 0, 0);
        }
#pragma unroll
        for (int a = (p * NPL + pl) * 4 / kSteps; a < (p * NPL + pl + 1) * 4 / kSteps; ++a)
          pack_row(dst, c, a, kvalid);
        step_copy(p * NPL + pl);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // ---- pipeline ---------------------------------------------------------------
  int J1 = 0;                                    // column of chunk u+1
  int64_t pg_next = 0;                           // table page of the next pair to copy
  if (n_chunks > 0) {
    J1 = J0;
    // pair 0 needs only row_ptr, V(0) the first column: pair 0 goes first, and
    // V(0) sits between the pairs so that one wait covers pair 0 and V(0)
    const int64_t pg0 = pair_page(0), pg1 = pair_page(1);
#pragma unroll
    for (int d = 0; d < NCH; ++d) issue_pair(0, pg0, d);
    issue_v(0, J0, xv[0]);
#pragma unroll
    for (int d = 0; d < NCH; ++d) issue_pair(1, pg1, d);
    wait_vm_regs<NCH>(xv[0]);                    // pair 0 and V(0) landed (pair 1 in flight)
    lds_barrier();
    head_mix(0, kvalid_of(0, J0), 0);
    lds_barrier();
    pg_next = pair_page(2);
  }
  // Two phases per iteration (n_chunks is even for B >= 32), so that which
  // loads each phase issues and how many each wait leaves in flight are
  // fixed in the code.  Phase u waits for V(u) and transposes it after its
  // head mix, right before its A.V MFMAs.
  // - Even phase: no tile copies.  V(u+1) is loaded in parts, one behind the
  //   transpose and one behind each A.V step, so that the eight wavefronts'
  //   V loads do not reach the texture path at once and stall their issue.
  //   At its end it waits only for the pair copied in the previous phase.
  // - Odd phase: V(u+1) at its start, then pair (u+3)/2 into the stage whose
  //   last chunk was head-mixed in the previous phase, its copies spread over
  //   the A.V steps (loads return in issue order, so V goes first and the
  //   copies do not queue ahead of it); the pair has until the end of the
  //   next phase.  It ends with no wait: the next head mix reads the second
  //   chunk of a pair that has landed, and V(u+1) stays in flight across the
  //   loop's back edge (the static checks confirm that no instruction reads
  //   or writes those registers before the wait that retires them).
  auto phase = [&](int u, auto odd_tag) {
    constexpr bool kOdd = decltype(odd_tag)::value;
    const int64_t kn = block_of(u + 2);          // column of chunk u+2: used after the barrier
    const int Jn_col = col_idx[kn];
    int64_t pg_J = 0;
    if constexpr (kVar) pg_J = page_raw<kVar>(block_table, col_idx, kn);
    if constexpr (kOdd) issue_v(u + 1, J1, xv[0]);
    const int P = (u + 3) >> 1;
    auto step_copy = [&](int st) {
      if constexpr (!kOdd) {
        issue_v_part(u + 1, J1, xv[1], (st + 1) * 8 / (kSteps + 1), (st + 2) * 8 / (kSteps + 1));
      } else {
#pragma unroll
        for (int d = 0; d < NCH; ++d)
          if (d * kSteps / NCH == st) issue_pair(P, pg_next, d);
      }
    };
    auto prep_v = [&](u32x4 (&vt)[4]) {
      if constexpr (kOdd) {
        wait_vm_regs<8>(xv[1]);                  // V(u): only V(u+1) was issued after it
        transpose8x4(xv[1], vt);
      } else {
        wait_vm_regs<NCH>(xv[0]);                // V(u): the copies of a pair were issued after it
        transpose8x4(xv[0], vt);
        issue_v_part(u + 1, J1, xv[1], 0, 8 / (kSteps + 1));
      }
    };
    compute(u + 1, u + 1 < n_chunks ? kvalid_of(u + 1, J1) : 0, (u + 1) & 1, u & 1, prep_v, step_copy);
    if constexpr (kOdd) {
      if constexpr (kVar) pg_next = pair_page(P + 1);
    } else {
      wait_vm<8>();                              // the pair copied last phase (V(u+1) stays in flight)
    }
    lds_barrier();
    J1 = (!kVar || page_ok(bt, pg_J)) ? Jn_col : -1;
  };
  for (int u = 0; u < n_chunks; u += 2) {
    phase(u, std::false_type{});
    phase(u + 1, std::true_type{});
  }
  wait_vm_regs<0>(xv[0]);                        // no V load in flight past the loop
  wait_vm_regs<0>(xv[1]);
  lds_barrier();

  // ---- a part of a split row: fp32 partials, 16 bytes (4 head-dim columns) per lane
  if constexpr (kSplit) {
    if (parts > 1) {
      float* pp = sp.part + (int64_t)(item * subs + sub) * kRows * H_r * kD;
#pragma unroll
      for (int p = 0; p < NPAIR; ++p)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
          if (2 * p + (m >> 4) < RPW)
            *reinterpret_cast<f32x4*>(pp + ((m & 15) * H_r + rbeg + 2 * p + (m >> 4)) * kD + 4 * am) =
                f32x4{acc[p][0][e], acc[p][1][e], acc[p][2][e], acc[p][3][e]};
        }
      return;
    }
  }

  // ---- store through LDS (as in k_retrieve_mfma) ------------------------------
  unsigned short* ot = reinterpret_cast<unsigned short*>(smem + wave * kOutSlot);
#pragma unroll
  for (int p = 0; p < NPAIR; ++p) {
    if (p) lds_barrier();
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int m = 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
      unsigned short h[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) h[dt] = kBF16 ? bf16_bits(acc[p][dt][e]) : f32_to_f16(acc[p][dt][e]);
      *reinterpret_cast<u32x2*>(ot + ((m & 15) * 2 + (m >> 4)) * kD + 4 * am) =
          u32x2{(unsigned)h[0] | ((unsigned)h[1] << 16), (unsigned)h[2] | ((unsigned)h[3] << 16)};
    }
    lds_barrier();
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int c16 = pass * 64 + lane;
      const int i = c16 >> 5, rp = (c16 >> 4) & 1, d8 = (c16 & 15) * 8;
      const int64_t grow = (int64_t)I * B + sub * kRows + i;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ot + (i * 2 + rp) * kD + d8);
      if (2 * p + rp < RPW && grow < N)
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(O + grow * ldO + (int64_t)(rbeg + 2 * p + rp) * kD + d8));
    }
  }
}

// O rows of the split block rows: the sum of the row's part partials in part
// order, rounded once to the output type.  One workgroup per (block row,
// 16-row slice); rows kept whole return at once.
template <bool kBF16>
__global__ __launch_bounds__(256) void k_split_combine(
    const int32_t* __restrict__ row_ptr, int64_t nnzb, int T, int N, int B, int H_r,
    unsigned short* __restrict__ O, int64_t ldO, Split sp) {
  const int I = blockIdx.x, sub = blockIdx.y;
  const int subs = B / kRows;
  int64_t kb = row_ptr[I], ke = row_ptr[I + 1];
  kb = kb < 0 ? 0 : (kb > nnzb ? nnzb : kb);
  ke = ke < kb ? kb : (ke > nnzb ? nnzb : ke);
  const int parts = split_parts(ke - kb, sp.P);
  if (parts == 1) return;
  const int j0 = sp.first_item[I];
  const int64_t slot = (int64_t)kRows * H_r * kD;     // floats per (item, slice)
  const int n4 = (int)(slot / 4);
  for (int e4 = threadIdx.x; e4 < n4; e4 += 256) {
    const int e = 4 * e4;
    const int row = e / (H_r * kD);
    const int64_t grow = (int64_t)I * B + sub * kRows + row;
    if (grow >= N) continue;
    f32x4 s = *reinterpret_cast<const f32x4*>(sp.part + (int64_t)(j0 * subs + sub) * slot + e);
    for (int p = 1; p < parts; ++p) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(sp.part + (int64_t)((j0 + p) * subs + sub) * slot + e);
      s[0] += v[0]; s[1] += v[1]; s[2] += v[2]; s[3] += v[3];
    }
    const int rc = e - row * H_r * kD;            // receiver * 128 + column
    unsigned short h[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) h[t] = kBF16 ? bf16_bits(s[t]) : f32_to_f16(s[t]);
    *reinterpret_cast<u32x2*>(O + grow * ldO + rc) =
        u32x2{(unsigned)h[0] | ((unsigned)h[1] << 16), (unsigned)h[2] | ((unsigned)h[3] << 16)};
  }
}

// ---------------------------------------------------------------------------
// Plain kernel
// ---------------------------------------------------------------------------

template <class TT, int BB, int D, bool kVar>
__global__ __launch_bounds__(kSimpleThreads) void k_retrieve_simple(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const typename TT::S* __restrict__ vals, int64_t nnzb, int H_s, int N,
    const float* __restrict__ W, int H_r, const typename TT::S* __restrict__ V,
    int H_kv, int64_t ldV, typename TT::S* __restrict__ O, int64_t ldO, Batch bt,
    const int32_t* __restrict__ cu_rows, const int32_t* __restrict__ cu_seqlens,
    const int32_t* __restrict__ block_table, int R) {
  constexpr int RPP = kSimpleThreads / D;        // query rows per pass
  constexpr int NACC = BB / RPP;           // rows per thread
  __shared__ float ahat[BB * BB];
  __shared__ float wrow[64];
  const int Ig = R - 1 - (int)blockIdx.x;        // global block row, last first
  RowView rv;
  if (!row_view<kVar>(bt, cu_rows, cu_seqlens, Ig, N, BB, rv)) return;
  const int T = rv.T;
  const int I = rv.I;
  N = rv.N;
  V += rv.tok0 * ldV;
  O += rv.tok0 * ldO;
  const int r = blockIdx.y;
  const int g = r / (H_r / H_kv);
  const int tid = threadIdx.x;
  const int dcol = tid % D;
  const int i0 = tid / D;
  if (tid < H_s) wrow[tid] = W[(int64_t)r * H_s + tid];
  float acc[NACC];
#pragma unroll
  for (int m = 0; m < NACC; ++m) acc[m] = 0.f;
  int64_t kb = row_ptr[Ig], ke = row_ptr[Ig + 1];
  kb = kb < 0 ? 0 : (kb > nnzb ? nnzb : kb);
  ke = ke < kb ? kb : (ke > nnzb ? nnzb : ke);
  __syncthreads();
  for (int64_t k = kb; k < ke; ++k) {
    const int J = col_idx[k];
    const int64_t pg = page_of<kVar>(bt, block_table, k);
    if (J < 0 || J >= T || pg < 0) continue;
    const typename TT::S* blk = vals + pg * H_s * BB * BB;
    for (int e = tid; e < BB * BB; e += kSimpleThreads) {
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
                    const Batch& bt, int R, hipStream_t st) {
  using S = typename TT::S;
  if (R <= 0) return MF_OK;
  if (bt.cu_rows)
    hipLaunchKernelGGL((k_retrieve_simple<TT, BB, D, true>), dim3(R, H_r), dim3(kSimpleThreads),
                       0, st, row_ptr, col_idx, reinterpret_cast<const S*>(vals),
                       nnzb, H_s, N, W, H_r, reinterpret_cast<const S*>(V), H_kv,
                       ldV, reinterpret_cast<S*>(O), ldO, bt, bt.cu_rows, bt.cu_seqlens,
                       bt.block_table, R);
  else
    hipLaunchKernelGGL((k_retrieve_simple<TT, BB, D, false>), dim3(R, H_r), dim3(kSimpleThreads),
                       0, st, row_ptr, col_idx, reinterpret_cast<const S*>(vals),
                       nnzb, H_s, N, W, H_r, reinterpret_cast<const S*>(V), H_kv,
                       ldV, reinterpret_cast<S*>(O), ldO, bt, bt.cu_rows, bt.cu_seqlens,
                       bt.block_table, R);
  return mf::hip_check(hipGetLastError(), "k_retrieve_simple launch");
}

template <class TT, int D>
int launch_simple_d(int B, const int32_t* row_ptr, const int32_t* col_idx,
                    const void* vals, int64_t nnzb, int H_s, int N, const float* W,
                    int H_r, const void* V, int H_kv, int64_t ldV, void* O,
                    int64_t ldO, const Batch& bt, int R, hipStream_t st) {
  switch (B) {
    case 16: return launch_simple_t<TT, 16, D>(row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, bt, R, st);
    case 32: return launch_simple_t<TT, 32, D>(row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, bt, R, st);
    case 64: return launch_simple_t<TT, 64, D>(row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, bt, R, st);
    default: return launch_simple_t<TT, 128, D>(row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, bt, R, st);
  }
}

template <class TT>
int launch_simple(int B, int d, const int32_t* row_ptr, const int32_t* col_idx,
                  const void* vals, int64_t nnzb, int H_s, int N, const float* W,
                  int H_r, const void* V, int H_kv, int64_t ldV, void* O,
                  int64_t ldO, const Batch& bt, int R, hipStream_t st) {
  if (d == 64)
    return launch_simple_d<TT, 64>(B, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, bt, R, st);
  return launch_simple_d<TT, 128>(B, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, bt, R, st);
}

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// kGeneral: always the batch instantiation (several receivers); otherwise the
// batch instantiation exactly when bt describes a packed batch.
template <bool kBF16, int NPAIR, bool kGeneral = false>
int launch_mfma_p(int NCH, dim3 grid, hipStream_t st, const int32_t* row_ptr,
                  const int32_t* col_idx, const unsigned short* vals, int64_t nnzb,
                  int H_s, int N, int B, int lg_ncc, const float* W, int H_r, int RPW,
                  int G, const unsigned short* V, int64_t ldV, unsigned short* O,
                  int64_t ldO, int RG, const Batch& bt, int R) {
#define MF_CASE(NCH_)                                                                            \
  case NCH_:                                                                                     \
    if (kGeneral || bt.cu_rows)                                                                  \
      hipLaunchKernelGGL((k_retrieve_mfma<kBF16, NCH_, NPAIR, true>), grid, dim3(kThreads), 0, st, \
                         row_ptr, col_idx, vals, nnzb, H_s, N, B, lg_ncc, W, H_r, RPW, G,        \
                         V, ldV, O, ldO, RG, bt, bt.cu_rows, bt.cu_seqlens, bt.block_table, R);   \
    else                                                                                         \
      hipLaunchKernelGGL((k_retrieve_mfma<kBF16, NCH_, NPAIR, false>), grid, dim3(kThreads), 0, st, \
                         row_ptr, col_idx, vals, nnzb, H_s, N, B, lg_ncc, W, H_r, RPW, G,        \
                         V, ldV, O, ldO, RG, bt, bt.cu_rows, bt.cu_seqlens, bt.block_table, R);   \
    break;
  switch (NCH) {
    MF_CASE(1) MF_CASE(2) MF_CASE(3) MF_CASE(4) MF_CASE(5) MF_CASE(6)
    default: return mf::fail(MF_ERR_UNSUPPORTED, "k_retrieve_mfma: H_s out of range");
  }
#undef MF_CASE
  return mf::hip_check(hipGetLastError(), "k_retrieve_mfma launch");
}

// The pair-stage kernel, B >= 32 (same arguments and cases as launch_mfma_p).
template <bool kBF16, int NPAIR, bool kGeneral = false>
int launch_pair_p(int NCH, dim3 grid, hipStream_t st, const int32_t* row_ptr,
                  const int32_t* col_idx, const unsigned short* vals, int64_t nnzb,
                  int H_s, int N, int B, int lg_ncc, const float* W, int H_r, int RPW,
                  int G, const unsigned short* V, int64_t ldV, unsigned short* O,
                  int64_t ldO, int RG, const Batch& bt, int R) {
#define MF_CASE(NCH_)                                                                            \
  case NCH_:                                                                                     \
    if (kGeneral || bt.cu_rows)                                                                  \
      hipLaunchKernelGGL((k_retrieve_pair<kBF16, NCH_, NPAIR, true>), grid, dim3(kThreads), 0, st, \
                         row_ptr, col_idx, vals, nnzb, H_s, N, B, lg_ncc, W, H_r, RPW, G,        \
                         V, ldV, O, ldO, RG, bt, bt.cu_rows, bt.cu_seqlens, bt.block_table, R, Split{}); \
    else                                                                                         \
      hipLaunchKernelGGL((k_retrieve_pair<kBF16, NCH_, NPAIR, false>), grid, dim3(kThreads), 0, st, \
                         row_ptr, col_idx, vals, nnzb, H_s, N, B, lg_ncc, W, H_r, RPW, G,        \
                         V, ldV, O, ldO, RG, bt, bt.cu_rows, bt.cu_seqlens, bt.block_table, R, Split{}); \
    break;
  switch (NCH) {
    MF_CASE(1) MF_CASE(2) MF_CASE(3) MF_CASE(4) MF_CASE(5)
    default: return mf::fail(MF_ERR_UNSUPPORTED, "k_retrieve_pair: H_s out of range");
  }
#undef MF_CASE
  return mf::hip_check(hipGetLastError(), "k_retrieve_pair launch");
}

// The matrix-core kernel for block size B: pair stages for B >= 32.
template <bool kBF16, int NPAIR, bool kGeneral = false>
int launch_mfma_any(int NCH, dim3 grid, hipStream_t st, const int32_t* row_ptr,
                    const int32_t* col_idx, const unsigned short* vals, int64_t nnzb,
                    int H_s, int N, int B, int lg_ncc, const float* W, int H_r, int RPW,
                    int G, const unsigned short* V, int64_t ldV, unsigned short* O,
                    int64_t ldO, int RG, const Batch& bt, int R) {
  // 41-48 sender heads (NCH = 6) keep the first form: with pair stages its
  // register set no longer fits without spilling
  if (B >= 32 && NCH <= 5)
    return launch_pair_p<kBF16, NPAIR, kGeneral>(NCH, grid, st, row_ptr, col_idx, vals, nnzb, H_s, N, B,
                                                 lg_ncc, W, H_r, RPW, G, V, ldV, O, ldO, RG, bt, R);
  return launch_mfma_p<kBF16, NPAIR, kGeneral>(NCH, grid, st, row_ptr, col_idx, vals, nnzb, H_s, N, B,
                                               lg_ncc, W, H_r, RPW, G, V, ldV, O, ldO, RG, bt, R);
}

}  // namespace

namespace mf {

// The MFMA kernel covers fp16/bf16 with d = 128, B in {16, 32, 64, 128},
// H_r in {8, 16, 24, 32}, H_s <= 48, the H_r/8 receivers of every wavefront
// inside one KV group (G % (H_r/8) == 0), 16-byte aligned vals and O rows and
// 8-byte aligned V rows.
bool retrieve_uses_mfma(int dt, int H_s, int B, int H_r, int H_kv, int d, const void* vals,
                        const void* V, int64_t ldV, const void* O, int64_t ldO) {
  if (dt == MF_F32 || d != kD || H_s > kMaxHs) return false;
  if (B != 16 && B != 32 && B != 64 && B != 128) return false;
  if (H_r % 8 != 0 || H_r > kMaxRecv) return false;
  const int G = H_r / H_kv, RPW = H_r / 8;
  if (G % RPW != 0) return false;
  return aligned(vals, 16) && aligned(O, 16) && ldO % 8 == 0 && aligned(V, 16) && ldV % 8 == 0 &&
         ldV <= (int64_t)1 << 26;   // per-lane V offsets are 32-bit
}

size_t retrieve_workspace_bytes(int, int, int, int, int) { return 0; }

namespace {
int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1)
    return 256;
  return n;
}
size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
}  // namespace

int split_part_len(int64_t nnzb, int B) {
  const int64_t work = nnzb * (B / kRows);        // (kept block, 16-row slice) units
  const int64_t cus = device_cus();
  const int64_t P = (work + cus - 1) / cus;
  return (int)std::max<int64_t>(1, std::min<int64_t>(P, 1 << 20));
}

// Splitting pays when the average row is longer than half the per-CU share P:
// then there are too few items per CU for the longest rows to even out.
bool split_applies(int dt, int H_s, int N, int B, int H_r, int H_kv, int d, int64_t nnzb) {
  if (dt == MF_F32 || d != kD || B < 32 || (H_s + 7) / 8 > 5 || H_r % 8 != 0 || H_r > kMaxRecv) return false;
  const int G = H_r / H_kv, RPW = H_r / 8;
  if (G % RPW != 0 || nnzb <= 0) return false;
  const int T = blocks_of(N, B);
  return 2 * nnzb > (int64_t)split_part_len(nnzb, B) * T;
}

size_t split_workspace_bytes(int dt, int H_s, int N, int B, int H_r, int H_kv, int d, int64_t nnzb) {
  if (!split_applies(dt, H_s, N, B, H_r, H_kv, d, nnzb)) return 0;
  const int T = blocks_of(N, B);
  const int64_t items = T + nnzb / split_part_len(nnzb, B);
  return align256((size_t)items * (B / kRows) * kRows * H_r * kD * sizeof(float)) +
         align256((size_t)T * sizeof(int32_t));
}

namespace {

// R block rows (all sequences of bt); N is the single sequence's length when
// bt.cu_rows is null.
// Split-row launch (one sequence, one receiver, pair kernel): the retrieval
// over the split work list, then the partial sums of the split rows.
int launch_split(const int32_t* row_ptr, const int32_t* col_idx, const void* vals, int64_t nnzb,
                 int dt, int H_s, int N, int B, const float* W, int H_r, const void* V, int H_kv,
                 int64_t ldV, void* O, int64_t ldO, void* workspace, hipStream_t st) {
  const int T = blocks_of(N, B);
  const int subs = B / kRows;
  const int P = split_part_len(nnzb, B);
  const int64_t items = T + nnzb / P;
  const size_t part_bytes = align256((size_t)items * subs * kRows * H_r * kD * sizeof(float));
  Split sp{reinterpret_cast<float*>(workspace),
           reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + part_bytes), P};
  const Batch bt{nullptr, nullptr, nullptr, nnzb, 1, 1, {}};
  const dim3 grid((unsigned)(((items + 7) / 8) * 8 * subs));
  const int NCH = (H_s + 7) / 8;
  const int RPW = H_r / 8, G = H_r / H_kv;
  const int lg_ncc = B == 32 ? 1 : B == 64 ? 2 : 3;
  auto vp = reinterpret_cast<const unsigned short*>(vals);
  auto Vs = reinterpret_cast<const unsigned short*>(V);
  auto Op = reinterpret_cast<unsigned short*>(O);
  const bool bf = dt == MF_BF16;
#define MF_SPLIT(BF_, NP_, NCH_)                                                                   \
  hipLaunchKernelGGL((k_retrieve_pair<BF_, NCH_, NP_, false, true>), grid, dim3(kThreads), 0, st,  \
                     row_ptr, col_idx, vp, nnzb, H_s, N, B, lg_ncc, W, H_r, RPW, G, Vs, ldV, Op,  \
                     ldO, 1, bt, nullptr, nullptr, nullptr, T, sp)
#define MF_SPLIT_NCH(BF_, NP_)                                                                    \
  switch (NCH) {                                                                                \
    case 1: MF_SPLIT(BF_, NP_, 1); break;                                                       \
    case 2: MF_SPLIT(BF_, NP_, 2); break;                                                       \
    case 3: MF_SPLIT(BF_, NP_, 3); break;                                                       \
    case 4: MF_SPLIT(BF_, NP_, 4); break;                                                       \
    default: MF_SPLIT(BF_, NP_, 5); break;                                                      \
  }
  if (bf) {
    if (RPW > 2) { MF_SPLIT_NCH(true, 2) } else { MF_SPLIT_NCH(true, 1) }
  } else {
    if (RPW > 2) { MF_SPLIT_NCH(false, 2) } else { MF_SPLIT_NCH(false, 1) }
  }
#undef MF_SPLIT_NCH
#undef MF_SPLIT
  int r = mf::hip_check(hipGetLastError(), "k_retrieve_pair (split rows) launch");
  if (r != MF_OK) return r;
  if (bf)
    hipLaunchKernelGGL(k_split_combine<true>, dim3(T, subs), dim3(256), 0, st, row_ptr, nnzb, T, N, B,
                       H_r, Op, ldO, sp);
  else
    hipLaunchKernelGGL(k_split_combine<false>, dim3(T, subs), dim3(256), 0, st, row_ptr, nnzb, T, N, B,
                       H_r, Op, ldO, sp);
  return mf::hip_check(hipGetLastError(), "k_split_combine launch");
}

int retrieve_impl(const int32_t* row_ptr, const int32_t* col_idx, const void* vals,
                  int64_t nnzb, int dt, int H_s, int N, int B, const float* W, int H_r,
                  const void* V, int H_kv, int d, int64_t ldV, void* O, int64_t ldO,
                  const Batch& bt, int R, hipStream_t st, void* workspace = nullptr,
                  size_t workspace_bytes = 0) {
  if (R <= 0) return MF_OK;
  if (bt.cu_rows == nullptr && bt.n_recv == 1 && workspace != nullptr &&
      retrieve_uses_mfma(dt, H_s, B, H_r, H_kv, d, vals, V, ldV, O, ldO) &&
      split_applies(dt, H_s, N, B, H_r, H_kv, d, nnzb) &&
      workspace_bytes >= split_workspace_bytes(dt, H_s, N, B, H_r, H_kv, d, nnzb))
    return launch_split(row_ptr, col_idx, vals, nnzb, dt, H_s, N, B, W, H_r, V, H_kv, ldV, O, ldO,
                        workspace, st);
  if (retrieve_uses_mfma(dt, H_s, B, H_r, H_kv, d, vals, V, ldV, O, ldO)) {
    const int RG = row_group(R);
    const int groups = (R + RG - 1) / RG;
    const int rows_per_xcd = ((groups + 7) / 8) * RG;
    const dim3 grid(rows_per_xcd * 8 * (B / kRows));
    const int NCH = (H_s + 7) / 8;
    const int RPW = H_r / 8, G = H_r / H_kv;
    const int lg_ncc = B == 16 ? 0 : B == 32 ? 1 : B == 64 ? 2 : 3;
    auto vp = reinterpret_cast<const unsigned short*>(vals);
    auto Vs = reinterpret_cast<const unsigned short*>(V);
    auto Op = reinterpret_cast<unsigned short*>(O);
    const bool bf = dt == MF_BF16;
    if (RPW > 2)
      return bf ? launch_mfma_any<true, 2>(NCH, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, lg_ncc, W, H_r, RPW, G, Vs, ldV, Op, ldO, RG, bt, R)
                : launch_mfma_any<false, 2>(NCH, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, lg_ncc, W, H_r, RPW, G, Vs, ldV, Op, ldO, RG, bt, R);
    return bf ? launch_mfma_any<true, 1>(NCH, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, lg_ncc, W, H_r, RPW, G, Vs, ldV, Op, ldO, RG, bt, R)
              : launch_mfma_any<false, 1>(NCH, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, lg_ncc, W, H_r, RPW, G, Vs, ldV, Op, ldO, RG, bt, R);
  }
  if (dt == MF_F32)
    return launch_simple<mfd::TF32>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, bt, R, st);
  if (dt == MF_F16)
    return launch_simple<mfd::TF16>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, bt, R, st);
  return launch_simple<mfd::TBF16>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, bt, R, st);
}

}  // namespace

int launch_retrieve(const int32_t* row_ptr, const int32_t* col_idx,
                    const void* vals, int64_t nnzb, int dt, int H_s, int N,
                    int B, const float* W, int H_r, const void* V, int H_kv,
                    int d, int64_t ldV, void* O, int64_t ldO, void* workspace,
                    size_t workspace_bytes, hipStream_t st) {
  const Batch bt{nullptr, nullptr, nullptr, nnzb, 1, 1, {}};
  return retrieve_impl(row_ptr, col_idx, vals, nnzb, dt, H_s, N, B, W, H_r, V, H_kv, d, ldV,
                       O, ldO, bt, blocks_of(N, B), st, workspace, workspace_bytes);
}

int launch_retrieve_multi(const int32_t* row_ptr, const int32_t* col_idx, const void* vals,
                          int64_t nnzb, int dt, int H_s, int N, int B, int n_recv,
                          const float* const* W, const int* H_r, const void* const* V,
                          const int* H_kv, int d, const int64_t* ldV, void* const* O,
                          const int64_t* ldO, hipStream_t st) {
  bool together = n_recv > 1 && n_recv <= kMaxRecvSets;
  for (int i = 0; i < n_recv && together; ++i)
    together = retrieve_uses_mfma(dt, H_s, B, H_r[i], H_kv[i], d, vals, V[i], ldV[i], O[i], ldO[i]);
  if (!together) {                               // one launch per receiver, same arithmetic
    for (int i = 0; i < n_recv; ++i) {
      const int r = launch_retrieve(row_ptr, col_idx, vals, nnzb, dt, H_s, N, B, W[i], H_r[i], V[i],
                                    H_kv[i], d, ldV[i], O[i], ldO[i], nullptr, 0, st);
      if (r != MF_OK) return r;
    }
    return MF_OK;
  }
  Batch bt{nullptr, nullptr, nullptr, nnzb, 1, n_recv, {}};
  int max_rpw = 0;
  for (int i = 0; i < n_recv; ++i) {
    bt.recv[i] = Recv{W[i], V[i], O[i], ldV[i], ldO[i], H_r[i], H_r[i] / 8, H_r[i] / H_kv[i]};
    max_rpw = std::max(max_rpw, H_r[i] / 8);
  }
  const int R = blocks_of(N, B);
  const int RG = row_group(R);
  const int groups = (R + RG - 1) / RG;
  const int rows_per_xcd = ((groups + 7) / 8) * RG;
  const dim3 grid(rows_per_xcd * 8 * (B / kRows) * n_recv);
  const int NCH = (H_s + 7) / 8;
  const int lg_ncc = B == 16 ? 0 : B == 32 ? 1 : B == 64 ? 2 : 3;
  auto vp = reinterpret_cast<const unsigned short*>(vals);
  const Recv& r0 = bt.recv[0];
  auto V0 = reinterpret_cast<const unsigned short*>(r0.V);
  auto O0 = reinterpret_cast<unsigned short*>(r0.O);
  const bool bf = dt == MF_BF16;
  if (max_rpw > 2)
    return bf ? launch_mfma_any<true, 2, true>(NCH, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, lg_ncc, r0.W, r0.H_r, r0.RPW, r0.G, V0, r0.ldV, O0, r0.ldO, RG, bt, R)
              : launch_mfma_any<false, 2, true>(NCH, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, lg_ncc, r0.W, r0.H_r, r0.RPW, r0.G, V0, r0.ldV, O0, r0.ldO, RG, bt, R);
  return bf ? launch_mfma_any<true, 1, true>(NCH, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, lg_ncc, r0.W, r0.H_r, r0.RPW, r0.G, V0, r0.ldV, O0, r0.ldO, RG, bt, R)
            : launch_mfma_any<false, 1, true>(NCH, grid, st, row_ptr, col_idx, vp, nnzb, H_s, N, B, lg_ncc, r0.W, r0.H_r, r0.RPW, r0.G, V0, r0.ldV, O0, r0.ldO, RG, bt, R);
}

int launch_retrieve_varlen(int S, int R, const int32_t* cu_seqlens, const int32_t* cu_rows,
                           const int32_t* row_ptr, const int32_t* col_idx,
                           const int32_t* block_table, const void* vals, int64_t n_pages,
                           int64_t nnzb, int dt, int H_s, int B, const float* W, int H_r,
                           const void* V, int H_kv, int d, int64_t ldV, void* O, int64_t ldO,
                           hipStream_t st) {
  const Batch bt{cu_rows, cu_seqlens, block_table, block_table ? n_pages : nnzb, S, 1, {}};
  return retrieve_impl(row_ptr, col_idx, vals, nnzb, dt, H_s, 0, B, W, H_r, V, H_kv, d, ldV,
                       O, ldO, bt, R, st);
}

}  // namespace mf
