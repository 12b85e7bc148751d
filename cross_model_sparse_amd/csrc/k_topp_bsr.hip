// Block-level Top-p selection and Block Sparse Row build.
//
// MapFlow keeps, per block row, the blocks needed to reach a cumulative
// attention probability p (paper page montaan.com/papers/2610.14688,
// highlight 3) and stores them as BSR with regular 2-D blocks ("Practical
// Implementation Details"); different rows keep different numbers of blocks
// (article aitest123.com/news/zaoi86, third section, second component).
//
// Three launches on the caller's stream:
//  1. k_select  one workgroup per block row: sort of the row's causal
//               candidates in LDS by (mass descending, column ascending) (rank
//               counting up to 512 candidates, a bitonic network above), then
//               a single-lane fp64 walk over the masses staged in LDS (row total in column order, running
//               sum in sorted order) that stops at the first running sum
//               >= p * total, then a compaction of the kept columns into
//               ascending order (wavefront ballots up to 256 candidates, an
//               LDS scan above).  Sequential sums keep the decision exactly
//               reproducible and independent of the launch shape.
//  2. k_scan    one workgroup: exclusive scan of the per-row counts -> row_ptr.
//  3. k_gather  grid-stride over (kept block, group of 8 heads): writes
//               col_idx and copies the kept tiles into vals with full-width
//               coalesced loads/stores (16-byte pieces also where map rows
//               start off a 16-byte boundary), zero-padding rows/columns >= N.  It
//               reads nnzb = row_ptr[T] on the device and does nothing when
//               nnzb exceeds the caller's capacity, so no host round trip is
//               needed between the launches.
#include "mf_internal.h"

namespace {

using namespace mfd;

constexpr int kMaxT = 4096;
constexpr int kSelThreads = 256;

__device__ __forceinline__ unsigned long long desc_key(float m, int J) {
  // Monotone map of IEEE floats to unsigned (ascending), then complemented so
  // that larger masses sort first; ties fall back to the column index.
  unsigned u = __float_as_uint(m);
  unsigned asc = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((unsigned long long)(~asc) << 32) | (unsigned)J;
}

__global__ __launch_bounds__(kSelThreads) void k_select(
    const float* __restrict__ mass, int T, float p, int32_t* __restrict__ kept,
    int32_t* __restrict__ count) {
  __shared__ unsigned long long keys[kMaxT];
  __shared__ float mv[kMaxT];                    // the row's masses, for the fp64 walk
  __shared__ unsigned char flag[kMaxT];
  __shared__ int scan_buf[kSelThreads];
  __shared__ int k_sh;
  const int I = blockIdx.x;
  const int tid = threadIdx.x;
  const int ncand = I + 1;
  const float* mrow = mass + (int64_t)I * T;

  if (p >= 1.0f) {
    for (int J = tid; J < ncand; J += kSelThreads) kept[(int64_t)I * T + J] = J;
    if (tid == 0) count[I] = ncand;
    return;
  }
  int n = 1;
  while (n < ncand) n <<= 1;
  for (int j = tid; j < n; j += kSelThreads) {
    const float m = j < ncand ? mrow[j] : 0.f;
    keys[j] = (j < ncand) ? desc_key(m, j) : ~0ull;
    if (j < ncand) {
      mv[j] = m;
      flag[j] = 0;
    }
  }
  __syncthreads();
  if (ncand <= 2 * kSelThreads) {
    // Rank sort, ascending keys: keys are distinct (the column is in the low
    // bits), so the number of smaller keys is each key's sorted position; no
    // barrier between steps, unlike the bitonic network below.
    const bool h0 = tid < ncand, h1 = tid + kSelThreads < ncand;
    const unsigned long long k0 = h0 ? keys[tid] : 0ull;
    const unsigned long long k1 = h1 ? keys[tid + kSelThreads] : 0ull;
    int r0 = 0, r1 = 0;
    for (int i = 0; i < ncand; ++i) {
      const unsigned long long ki = keys[i];
      r0 += ki < k0;
      r1 += ki < k1;
    }
    __syncthreads();
    if (h0) keys[r0] = k0;
    if (h1) keys[r1] = k1;
    __syncthreads();
  } else {
    // Bitonic sort, ascending keys.
    for (int size = 2; size <= n; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < (n >> 1); t += kSelThreads) {
          const int lo = 2 * t - (t & (stride - 1));
          const int hi = lo + stride;
          const bool up = ((lo & size) == 0);
          unsigned long long a = keys[lo], b = keys[hi];
          if ((a > b) == up) {
            keys[lo] = b;
            keys[hi] = a;
          }
        }
        __syncthreads();
      }
    }
  }
  if (tid == 0) {
    double total = 0.0;
    for (int J = 0; J < ncand; ++J) total += (double)mv[J];
    const double thr = (double)p * total;
    double cum = 0.0;
    int k = 0;
    while (k < ncand) {
      const int J = (int)(keys[k] & 0xffffffffu);
      cum += (double)mv[J];
      flag[J] = 1;
      ++k;
      if (cum >= thr) break;
    }
    k_sh = k;
  }
  __syncthreads();
  // Compact flagged columns in ascending order.
  if (ncand <= kSelThreads) {
    // one candidate per thread: position = kept columns below it, counted by
    // wavefront ballots
    const bool f = tid < ncand && flag[tid];
    const unsigned long long b = __ballot(f);
    const int lane = tid & 63, w = tid >> 6;
    if (lane == 0) scan_buf[w] = __popcll(b);
    __syncthreads();
    int pos = __popcll(b & ((1ull << lane) - 1ull));
    for (int q = 0; q < w; ++q) pos += scan_buf[q];
    if (f) kept[(int64_t)I * T + pos] = tid;
    if (tid == 0) count[I] = k_sh;
    return;
  }
  const int chunk = (ncand + kSelThreads - 1) / kSelThreads;
  const int j0 = tid * chunk, j1 = min(ncand, j0 + chunk);
  int c = 0;
  for (int j = j0; j < j1; ++j) c += flag[j];
  scan_buf[tid] = c;
  __syncthreads();
  for (int off = 1; off < kSelThreads; off <<= 1) {
    int v = (tid >= off) ? scan_buf[tid - off] : 0;
    __syncthreads();
    scan_buf[tid] += v;
    __syncthreads();
  }
  int pos = scan_buf[tid] - c;
  for (int j = j0; j < j1; ++j)
    if (flag[j]) kept[(int64_t)I * T + pos++] = j;
  if (tid == 0) count[I] = k_sh;
}

constexpr int kScanThreads = 256;

__global__ __launch_bounds__(kScanThreads) void k_scan(
    const int32_t* __restrict__ count, int T, int32_t* __restrict__ row_ptr) {
  __shared__ int buf[kScanThreads];
  const int tid = threadIdx.x;
  const int per = (T + kScanThreads - 1) / kScanThreads;
  const int i0 = tid * per, i1 = min(T, i0 + per);
  int s = 0;
  for (int i = i0; i < i1; ++i) s += count[i];
  buf[tid] = s;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    int v = (tid >= off) ? buf[tid - off] : 0;
    __syncthreads();
    buf[tid] += v;
    __syncthreads();
  }
  int run = buf[tid] - s;
  if (tid == 0) row_ptr[0] = 0;
  for (int i = i0; i < i1; ++i) {
    run += count[i];
    row_ptr[i + 1] = run;
  }
}

constexpr int kGatherThreads = 256;
constexpr int kHeadsPerUnit = 8;

// kRagged: map rows start off a VEC-byte boundary (N*e not a multiple of VEC,
// or A off one): pieces are read with loads aligned only to the element size,
// and the piece that straddles column N (last column block only) is put
// together element by element, zero past N.
template <class TT, int VEC, bool kRagged>
__global__ __launch_bounds__(kGatherThreads) void k_gather(
    const typename TT::S* __restrict__ A, int H_s, int N, int B,
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ kept,
    int64_t cap, int32_t* __restrict__ col_idx, typename TT::S* __restrict__ vals) {
  using S = typename TT::S;
  using Vt = typename VecT<VEC>::T;
  constexpr int EPV = VEC / (int)sizeof(S);
  const int T = (N + B - 1) / B;
  const int64_t nnzb = row_ptr[T];
  if (nnzb > cap) return;
  const int HG = (H_s + kHeadsPerUnit - 1) / kHeadsPerUnit;
  const int64_t units = nnzb * HG;
  const int CPJ = B / EPV;
  const int tid = threadIdx.x;
  for (int64_t u = blockIdx.x; u < units; u += gridDim.x) {
    const int64_t k = u / HG;
    const int hg = (int)(u - k * HG);
    // Block row of k: the last I with row_ptr[I] <= k.
    int lo = 0, hi = T - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)row_ptr[mid] <= k) lo = mid; else hi = mid - 1;
    }
    const int I = lo;
    const int J = kept[(int64_t)I * T + (k - row_ptr[I])];
    if (hg == 0 && tid == 0) col_idx[k] = J;
    const int h0 = hg * kHeadsPerUnit;
    const int nh = min(kHeadsPerUnit, H_s - h0);
    const int rows_valid = min(B, N - I * B);
    const int cols_valid = min(B, N - J * B);
    const int total = nh * B * CPJ;
    int f = tid;
    for (; f < total; f += 8 * kGatherThreads) {
      Vt v[8];
      int64_t dst[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int ff = f + w * kGatherThreads;
        dst[w] = -1;
        if (ff < total) {
          const int chk = ff % CPJ;
          const int rest = ff / CPJ;
          const int i = rest % B;
          const int h = h0 + rest / B;
          const int c = chk * EPV;
          dst[w] = (((k * H_s + h) * B + i) * B + c);
          if (i < rows_valid && c < cols_valid) {
            const S* src = A + ((int64_t)h * N + (int64_t)I * B + i) * N + (int64_t)J * B + c;
            if constexpr (kRagged) {
              if (c + EPV <= cols_valid) {
                v[w] = load_any<VEC>(src);
              } else {
                S e[EPV];
#pragma unroll
                for (int t = 0; t < EPV; ++t) e[t] = t < cols_valid - c ? src[t] : S{};
                __builtin_memcpy(&v[w], e, VEC);
              }
            } else {
              v[w] = *reinterpret_cast<const Vt*>(src);
            }
          } else {
            v[w] = Vt{};
          }
        }
      }
#pragma unroll
      for (int w = 0; w < 8; ++w)
        if (dst[w] >= 0) *reinterpret_cast<Vt*>(vals + dst[w]) = v[w];
    }
  }
}

template <class TT, int VEC, bool kRagged = false>
hipError_t launch_gather(const void* A, int H_s, int N, int B,
                         const int32_t* row_ptr, const int32_t* kept,
                         int64_t cap, int32_t* col_idx, void* vals,
                         hipStream_t st) {
  const int T = mf::blocks_of(N, B);
  const int64_t ub = std::min<int64_t>(cap, (int64_t)T * (T + 1) / 2);
  const int HG = (H_s + kHeadsPerUnit - 1) / kHeadsPerUnit;
  const int64_t units = ub * HG;
  if (units <= 0) return hipSuccess;
  const int grid = (int)std::min<int64_t>(units, 8192);
  hipLaunchKernelGGL((k_gather<TT, VEC, kRagged>), dim3(grid), dim3(kGatherThreads), 0,
                     st, reinterpret_cast<const typename TT::S*>(A), H_s, N, B,
                     row_ptr, kept, cap, col_idx,
                     reinterpret_cast<typename TT::S*>(vals));
  return hipGetLastError();
}

template <class TT>
hipError_t launch_gather_t(int vec, const void* A, int H_s, int N, int B,
                           const int32_t* row_ptr, const int32_t* kept,
                           int64_t cap, int32_t* col_idx, void* vals,
                           hipStream_t st) {
  if (vec < 0) return launch_gather<TT, 16, true>(A, H_s, N, B, row_ptr, kept, cap, col_idx, vals, st);
  if (vec >= 16) return launch_gather<TT, 16>(A, H_s, N, B, row_ptr, kept, cap, col_idx, vals, st);
  if (vec >= 8) return launch_gather<TT, 8>(A, H_s, N, B, row_ptr, kept, cap, col_idx, vals, st);
  if (vec >= 4 || sizeof(typename TT::S) == 4)
    return launch_gather<TT, 4>(A, H_s, N, B, row_ptr, kept, cap, col_idx, vals, st);
  return launch_gather<TT, 2>(A, H_s, N, B, row_ptr, kept, cap, col_idx, vals, st);
}

}  // namespace

namespace mf {

hipError_t launch_select_scan(const float* mass, int N, int B, float p, int32_t* row_ptr,
                              void* workspace, hipStream_t st) {
  const int T = blocks_of(N, B);
  int32_t* kept = reinterpret_cast<int32_t*>(workspace);
  int32_t* count = kept + (int64_t)T * T;
  hipLaunchKernelGGL(k_select, dim3(T), dim3(kSelThreads), 0, st, mass, T, p,
                     kept, count);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(kScanThreads), 0, st, count, T,
                     row_ptr);
  return hipGetLastError();
}

hipError_t launch_topp_bsr(const float* mass, const void* A, int dt, int H_s,
                           int N, int B, float p, int32_t* row_ptr,
                           int32_t* col_idx, void* vals, int64_t cap_nnzb,
                           void* workspace, hipStream_t st) {
  const int32_t* kept = reinterpret_cast<const int32_t*>(workspace);
  hipError_t e = launch_select_scan(mass, N, B, p, row_ptr, workspace, st);
  if (e != hipSuccess) return e;
  int vec = row_vec_bytes(A, N, B, dtype_bytes(dt));
  // rows off a 16-byte boundary into a 16-byte aligned vals: the ragged
  // variant (vec = -1) keeps 16-byte pieces
  if (vec < 16 && ragged_rows_ok(A, N, dtype_bytes(dt)) && (reinterpret_cast<uintptr_t>(vals) % 16) == 0)
    vec = -1;
  while (vec > dtype_bytes(dt) && (reinterpret_cast<uintptr_t>(vals) % vec) != 0) vec >>= 1;
  if (dt == MF_F32)
    return launch_gather_t<mfd::TF32>(vec, A, H_s, N, B, row_ptr, kept, cap_nnzb, col_idx, vals, st);
  if (dt == MF_F16)
    return launch_gather_t<mfd::TF16>(vec, A, H_s, N, B, row_ptr, kept, cap_nnzb, col_idx, vals, st);
  return launch_gather_t<mfd::TBF16>(vec, A, H_s, N, B, row_ptr, kept, cap_nnzb, col_idx, vals, st);
}

}  // namespace mf
