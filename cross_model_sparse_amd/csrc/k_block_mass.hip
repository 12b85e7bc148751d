// Block-mass reduction over the causal tiles of a sender attention map.
//
// MapFlow's compressor first computes a statistic per block, then picks the
// blocks to keep (article aitest123.com/news/zaoi86, third section, first
// component); the pick is driven by cumulative attention probability (paper
// page montaan.com/papers/2610.14688, highlight 3).  The statistic here is
// the head-averaged attention mass of a block tile:
//   mass[I][J] = (1/H_s) * sum_h sum_{i in I} sum_{j in J} A[h][i][j],  J <= I.
//
// Design (HBM-bound scan, read-once):
//  * One workgroup owns block row I and a run of JPC consecutive column
//    blocks.  Along a map row those JPC tiles are contiguous in memory, so
//    every wavefront load is a run of whole cache lines; the workgroup walks
//    all H_s * B rows of its strip.
//  * Each lane keeps one fixed 16-byte column chunk (hence one fixed J) for
//    the whole walk, sums the chunk in fp32 (at most 8 elements) and adds the
//    partial into an fp64 accumulator, so the result carries no order-
//    dependent drift.  Eight independent loads per lane are kept in flight.
//  * The per-J combine runs over LDS in a fixed order: the result is
//    bit-reproducible run to run.
//  * The same workgroup writes the zeros of its strip above the diagonal, so
//    mass[T][T] is written completely without a separate fill.
#include "mf_internal.h"

namespace {

using namespace mfd;

constexpr int kThreads = 256;

template <class TT, int VEC>
__global__ __launch_bounds__(kThreads) void k_block_mass(
    const typename TT::S* __restrict__ A, int H_s, int N, int B, int JPC,
    float* __restrict__ mass) {
  using S = typename TT::S;
  using V = typename VecT<VEC>::T;
  constexpr int EPV = VEC / (int)sizeof(S);  // elements per vector
  const int T = (N + B - 1) / B;
  const int I = blockIdx.x;
  const int J0 = blockIdx.y * JPC;
  const int tid = threadIdx.x;
  const int Jend = min(T, J0 + JPC);  // strip columns this group owns
  if (J0 >= T) return;
  if (J0 > I) {  // strip entirely above the diagonal
    if (tid < Jend - J0) mass[(int64_t)I * T + J0 + tid] = 0.f;
    return;
  }
  const int J1 = min(I + 1, Jend);          // causal columns [J0, J1)
  const int CPJ = B / EPV;                  // chunks per column block
  const int CPR = JPC * CPJ;                // chunks per strip row (<= 256)
  const int RPI = kThreads / CPR;           // strip rows per pass
  const int ch = tid % CPR;
  const int r0 = tid / CPR;
  const int col = J0 * B + ch * EPV;
  const int col_end = min(N, J1 * B);
  const int rows = min(B, N - I * B);

  double acc = 0.0;
  if (col < col_end) {
    for (int h = 0; h < H_s; ++h) {
      const S* base = A + ((int64_t)h * N + (int64_t)I * B) * N + col;
      int i = r0;
      for (; i + 7 * RPI < rows; i += 8 * RPI) {
        V v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u)
          v[u] = *reinterpret_cast<const V*>(base + (int64_t)(i + u * RPI) * N);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += (double)vec_sum<TT, VEC>(v[u]);
      }
      for (; i < rows; i += RPI) {
        V v = *reinterpret_cast<const V*>(base + (int64_t)i * N);
        acc += (double)vec_sum<TT, VEC>(v);
      }
    }
  }

  __shared__ double part[kThreads];
  part[tid] = acc;
  __syncthreads();
  const int nj = Jend - J0;
  if (tid < nj) {
    const int jl = tid;
    float out = 0.f;
    if (J0 + jl <= I) {
      double s = 0.0;
      for (int rr = 0; rr < RPI; ++rr)
        for (int c = jl * CPJ; c < (jl + 1) * CPJ; ++c) s += part[rr * CPR + c];
      out = (float)(s / (double)H_s);
    }
    mass[(int64_t)I * T + J0 + jl] = out;
  }
}

template <class TT, int VEC>
hipError_t launch_t(const void* A, int H_s, int N, int B, float* mass,
                    hipStream_t st) {
  const int esz = (int)sizeof(typename TT::S);
  const int T = mf::blocks_of(N, B);
  const int limit = min(1024, kThreads * VEC);     // strip row bytes
  const int JPC = max(1, limit / (B * esz));
  dim3 grid(T, (T + JPC - 1) / JPC);
  hipLaunchKernelGGL((k_block_mass<TT, VEC>), grid, dim3(kThreads), 0, st,
                     reinterpret_cast<const typename TT::S*>(A), H_s, N, B, JPC,
                     mass);
  return hipGetLastError();
}

}  // namespace

namespace mf {

hipError_t launch_block_mass(const void* A, int dt, int H_s, int N, int B,
                             float* mass, hipStream_t st) {
  const int esz = dtype_bytes(dt);
  const int vec = row_vec_bytes(A, N, B, esz);
  if (dt == MF_F32) {
    if (vec >= 16) return launch_t<mfd::TF32, 16>(A, H_s, N, B, mass, st);
    if (vec >= 8) return launch_t<mfd::TF32, 8>(A, H_s, N, B, mass, st);
    return launch_t<mfd::TF32, 4>(A, H_s, N, B, mass, st);
  }
  if (dt == MF_F16) {
    if (vec >= 16) return launch_t<mfd::TF16, 16>(A, H_s, N, B, mass, st);
    if (vec >= 8) return launch_t<mfd::TF16, 8>(A, H_s, N, B, mass, st);
    if (vec >= 4) return launch_t<mfd::TF16, 4>(A, H_s, N, B, mass, st);
    return launch_t<mfd::TF16, 2>(A, H_s, N, B, mass, st);
  }
  if (vec >= 16) return launch_t<mfd::TBF16, 16>(A, H_s, N, B, mass, st);
  if (vec >= 8) return launch_t<mfd::TBF16, 8>(A, H_s, N, B, mass, st);
  if (vec >= 4) return launch_t<mfd::TBF16, 4>(A, H_s, N, B, mass, st);
  return launch_t<mfd::TBF16, 2>(A, H_s, N, B, mass, st);
}

}  // namespace mf
