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
// Two kernels:
//
// k_retrieve_mfma  (fp16 / bf16 inputs, d = 128, B in {32,64,128}, H_r <= 32)
//   Work item = (block row I, 16-row slice of it); one 256-thread workgroup
//   owns all receiver heads and all of d for its 16 query rows, so every kept
//   tile element leaves HBM exactly once.  Per kept block and 64-column chunk:
//   * head mix on MFMA (v_mfma_f32_16x16x32_f16): M = receiver heads,
//     K = sender heads, N = tile positions.  Each lane loads 16-byte runs of a
//     tile row for 8 sender heads straight from HBM and transposes them in
//     registers (v_perm_b32) into B operands, so the H_s-major tile layout
//     needs no LDS staging.  bf16 tiles are converted to fp16 on the way.
//   * the fp32 mixed map is rounded to fp16 and written to LDS once; that
//     round trip is also the re-layout from "positions across lanes" to
//     "query rows across lanes, key columns along K" that the second
//     contraction needs.
//   * Ahat . V on MFMA: M = 16 query rows, K = 32 key columns, N = 16 head-dim
//     columns.  Each wavefront owns a quarter of the receiver heads; V rows
//     are read as 16-byte runs along d and transposed in registers, and one V
//     operand serves every receiver head of its KV group.
//   * accumulation stays in registers across all kept blocks of the row; O is
//     written once, rounded to the storage dtype.
//   Work items are dealt out so that the slices of one block row land on one
//   XCD (they share V tiles in that XCD's L2) and block rows are handed out
//   from the last (longest candidate list) to the first.
//
// k_retrieve_simple  (every other supported case, including fp32)
//   One workgroup per (block row, receiver head): the mixed tile is built in
//   LDS in fp32, then multiplied with V by plain fp32 FMAs.
#include "mf_internal.h"

namespace {

using namespace mfd;

// ---------------------------------------------------------------------------
// MFMA kernel
// ---------------------------------------------------------------------------

constexpr int kThreads = 256;
constexpr int kD = 128;       // head dim handled by the MFMA kernel
constexpr int kRowsPerItem = 16;
constexpr int kMaxRecv = 32;  // receiver heads handled by the MFMA kernel
constexpr int kRPW = kMaxRecv / 4;  // receiver heads per wavefront

__device__ __forceinline__ f16x8 as_f16x8(const u32x4& v) {
  return __builtin_bit_cast(f16x8, v);
}

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

template <bool kBF16>
__device__ __forceinline__ void to_f16(u32x4& v) {
  if constexpr (kBF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j) v[j] = bf16x2_to_f16x2(v[j]);
  }
}

// Maps a workgroup index to a work item: the `subs` slices of a block row go
// to one XCD (workgroups are dealt to XCDs round-robin), block rows are
// interleaved across XCDs and issued from the last row to the first.
__device__ __forceinline__ int item_of(int b, int subs, int T, int* I, int* sub) {
  const int xcd = b & 7;
  const int local = b >> 3;
  const int row_slot = (local / subs) * 8 + xcd;
  if (row_slot >= T) return 0;
  *I = T - 1 - row_slot;
  *sub = local % subs;
  return 1;
}

template <bool kBF16, int CB, int KS, int MT>
__global__ __launch_bounds__(kThreads, 1) void k_retrieve_mfma(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const unsigned short* __restrict__ vals, int64_t nnzb, int H_s, int N,
    int B, const float* __restrict__ W, int H_r,
    const unsigned short* __restrict__ V, int H_kv, int64_t ldV,
    unsigned short* __restrict__ O, int64_t ldO) {
  constexpr int CPR = CB / 8;    // 16-byte column runs per tile row in a chunk
  constexpr int RPS = 16 / CPR;  // tile rows covered by one head-mix row set
  constexpr int NRS = 4 / RPS;   // row sets per wavefront (4 rows each wave)
  constexpr int KK = CB / 32;    // K steps of the A.V contraction per chunk
  constexpr int AP = CB + 8;     // LDS row pitch (halves) of the mixed map
  __shared__ __align__(16) unsigned short Ahs[kMaxRecv * kRowsPerItem * AP];

  const int T = (N + B - 1) / B;
  const int subs = B / kRowsPerItem;
  int I, sub;
  if (!item_of(blockIdx.x, subs, T, &I, &sub)) return;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n = lane & 15;
  const int q = lane >> 4;

  // Head-map operand (A of the head mix): row r = 16*mt + n, K slot (q, j)
  // is sender head 32*ks + 8*q + j.
  f16x8 wop[MT][KS];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int r = 16 * mt + n, s = 32 * ks + 8 * q + j;
        const float w = (r < H_r && s < H_s) ? W[(int64_t)r * H_s + s] : 0.f;
        wop[mt][ks][j] = (_Float16)w;
      }

  f32x4 acc[kRPW][8];
#pragma unroll
  for (int rl = 0; rl < kRPW; ++rl)
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[rl][t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int G = H_r / H_kv;
  const int rpw = (H_r + 3) / 4;  // receiver heads per wavefront
  const int rbeg = wave * rpw;
  int64_t kb = row_ptr[I], ke = row_ptr[I + 1];
  kb = kb < 0 ? 0 : (kb > nnzb ? nnzb : kb);
  ke = ke < kb ? kb : (ke > nnzb ? nnzb : ke);

  for (int64_t k = kb; k < ke; ++k) {
    const int J = col_idx[k];
    if (J < 0 || J >= T) continue;
    for (int cc = 0; cc < B / CB; ++cc) {
      // ---- head mix: this wave's 4 tile rows, all receiver heads ----------
#pragma unroll
      for (int rs = 0; rs < NRS; ++rs) {
        const int il = wave * 4 + rs * RPS + n / CPR;  // row within the slice
        const int row = sub * kRowsPerItem + il;       // row within the tile
        const int col = cc * CB + (n % CPR) * 8;       // column within the tile
        f32x4 c[8][MT];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
          for (int mt = 0; mt < MT; ++mt) c[t][mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 x[8], y[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int s = 32 * ks + 8 * q + u;
            if (s < H_s) {
              x[u] = *reinterpret_cast<const u32x4*>(
                  vals + (((k * H_s + s) * B + row) * B + col));
              to_f16<kBF16>(x[u]);
            } else {
              x[u] = u32x4{0u, 0u, 0u, 0u};
            }
          }
          transpose8x8(x, y);
#pragma unroll
          for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
              c[t][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  wop[mt][ks], as_f16x8(y[t]), c[t][mt], 0, 0, 0);
        }
        // lane (n, q) holds Ahat[16mt + 4q + a][row il][col .. col+7]
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int r = 16 * mt + 4 * q + a;
            if (r < H_r) {
              u32x4 pk;
#pragma unroll
              for (int j = 0; j < 4; ++j)
                pk[j] = pack_f16x2(c[2 * j][mt][a], c[2 * j + 1][mt][a]);
              *reinterpret_cast<u32x4*>(&Ahs[(r * kRowsPerItem + il) * AP +
                                             (n % CPR) * 8]) = pk;
            }
          }
      }
      __syncthreads();
      // ---- Ahat . V: this wave's receiver heads, all 16 rows --------------
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int64_t key0 = (int64_t)J * B + cc * CB + 32 * kk + 8 * q;
        int gcur = -1;
        u32x4 vt[8];
#pragma unroll
        for (int rl = 0; rl < kRPW; ++rl) {
          const int r = rbeg + rl;
          if (rl < rpw && r < H_r) {
            const int g = r / G;
            if (g != gcur) {
              u32x4 x[8];
#pragma unroll
              for (int u = 0; u < 8; ++u) {
                const int64_t key = key0 + u;
                if (key < N) {
                  x[u] = *reinterpret_cast<const u32x4*>(V + key * ldV +
                                                         (int64_t)g * kD + 8 * n);
                  to_f16<kBF16>(x[u]);
                } else {
                  x[u] = u32x4{0u, 0u, 0u, 0u};
                }
              }
              transpose8x8(x, vt);
              gcur = g;
            }
            const u32x4 a4 = *reinterpret_cast<const u32x4*>(
                &Ahs[(r * kRowsPerItem + n) * AP + 32 * kk + 8 * q]);
#pragma unroll
            for (int t = 0; t < 8; ++t)
              acc[rl][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                  as_f16x8(a4), as_f16x8(vt[t]), acc[rl][t], 0, 0, 0);
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- store: lane (n, q) holds O[row 4q + a][r][d = 8n .. 8n+7] ----------
#pragma unroll
  for (int rl = 0; rl < kRPW; ++rl) {
    const int r = rbeg + rl;
    if (rl < rpw && r < H_r) {
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int64_t grow = (int64_t)I * B + sub * kRowsPerItem + 4 * q + a;
        if (grow < N) {
          u32x4 pk;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float lo = acc[rl][2 * j][a], hi = acc[rl][2 * j + 1][a];
            if constexpr (kBF16)
              pk[j] = (unsigned)f32_to_bf16(lo) | ((unsigned)f32_to_bf16(hi) << 16);
            else
              pk[j] = pack_f16x2(lo, hi);
          }
          *reinterpret_cast<u32x4*>(O + grow * ldO + (int64_t)r * kD + 8 * n) = pk;
        }
      }
    }
  }
}

template <bool kBF16, int CB>
int launch_mfma_cb(int KS, int MT, const int32_t* row_ptr, const int32_t* col_idx,
                   const void* vals, int64_t nnzb, int H_s, int N, int B,
                   const float* W, int H_r, const void* V, int H_kv,
                   int64_t ldV, void* O, int64_t ldO, hipStream_t st) {
  const int T = mf::blocks_of(N, B);
  const int subs = B / kRowsPerItem;
  const int grid = ((T + 7) / 8) * 8 * subs;
  auto vp = reinterpret_cast<const unsigned short*>(vals);
  auto Vp = reinterpret_cast<const unsigned short*>(V);
  auto Op = reinterpret_cast<unsigned short*>(O);
#define MF_LAUNCH(KS_, MT_)                                                    \
  hipLaunchKernelGGL((k_retrieve_mfma<kBF16, CB, KS_, MT_>), dim3(grid),       \
                     dim3(kThreads), 0, st, row_ptr, col_idx, vp, nnzb, H_s,  \
                     N, B, W, H_r, Vp, H_kv, ldV, Op, ldO)
  if (KS == 1 && MT == 1) MF_LAUNCH(1, 1);
  else if (KS == 1) MF_LAUNCH(1, 2);
  else if (MT == 1) MF_LAUNCH(2, 1);
  else MF_LAUNCH(2, 2);
#undef MF_LAUNCH
  return mf::hip_check(hipGetLastError(), "k_retrieve_mfma launch");
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

}  // namespace

namespace mf {

// Whether the MFMA kernel serves this call (otherwise the plain kernel does).
bool retrieve_uses_mfma(int dt, int H_s, int B, int H_r, int d, const void* vals,
                        const void* V, int64_t ldV, const void* O, int64_t ldO) {
  return dt != MF_F32 && d == kD && B >= 32 && H_r <= kMaxRecv && H_s <= 64 &&
         aligned16(vals) && aligned16(V) && aligned16(O) && (ldV % 8) == 0 &&
         (ldO % 8) == 0;
}

int launch_retrieve(const int32_t* row_ptr, const int32_t* col_idx,
                    const void* vals, int64_t nnzb, int dt, int H_s, int N,
                    int B, const float* W, int H_r, const void* V, int H_kv,
                    int d, int64_t ldV, void* O, int64_t ldO, hipStream_t st) {
  if (retrieve_uses_mfma(dt, H_s, B, H_r, d, vals, V, ldV, O, ldO)) {
    const int KS = H_s <= 32 ? 1 : 2;
    const int MT = H_r <= 16 ? 1 : 2;
    if (B == 32) {
      if (dt == MF_BF16)
        return launch_mfma_cb<true, 32>(KS, MT, row_ptr, col_idx, vals, nnzb, H_s, N, B, W, H_r, V, H_kv, ldV, O, ldO, st);
      return launch_mfma_cb<false, 32>(KS, MT, row_ptr, col_idx, vals, nnzb, H_s, N, B, W, H_r, V, H_kv, ldV, O, ldO, st);
    }
    if (dt == MF_BF16)
      return launch_mfma_cb<true, 64>(KS, MT, row_ptr, col_idx, vals, nnzb, H_s, N, B, W, H_r, V, H_kv, ldV, O, ldO, st);
    return launch_mfma_cb<false, 64>(KS, MT, row_ptr, col_idx, vals, nnzb, H_s, N, B, W, H_r, V, H_kv, ldV, O, ldO, st);
  }
  if (dt == MF_F32)
    return launch_simple<mfd::TF32>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
  if (dt == MF_F16)
    return launch_simple<mfd::TF16>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
  return launch_simple<mfd::TBF16>(B, d, row_ptr, col_idx, vals, nnzb, H_s, N, W, H_r, V, H_kv, ldV, O, ldO, st);
}

}  // namespace mf
