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
//  * Rows that start off a 16-byte boundary (ragged N) keep 16-byte chunks,
//    read with loads aligned only to the element size.
#include "mf_internal.h"

namespace {

using namespace mfd;

constexpr int kThreads = 256;

// kRagged: map rows start off a VEC-byte boundary (N*e not a multiple of VEC,
// or A off one).  Chunks are read with loads aligned only to the element
// size; the one chunk that straddles column N (last column block) is summed
// element by element.
template <class TT, int VEC, bool kRagged>
__global__ __launch_bounds__(kThreads) void k_block_mass(
    const typename TT::S* __restrict__ A, int H_s, int N, int B, int JPC,
    float* __restrict__ mass) {
  using S = typename TT::S;
  using V = typename VecT<VEC>::T;
  constexpr int EPV = VEC / (int)sizeof(S);  // elements per vector
  auto ld = [](const S* q) -> V {
    if constexpr (kRagged) return load_any<VEC>(q);
    else return *reinterpret_cast<const V*>(q);
  };
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
  if (col < col_end && (!kRagged || col + EPV <= col_end)) {
    for (int h = 0; h < H_s; ++h) {
      const S* base = A + ((int64_t)h * N + (int64_t)I * B) * N + col;
      int i = r0;
      for (; i + 7 * RPI < rows; i += 8 * RPI) {
        V v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = ld(base + (int64_t)(i + u * RPI) * N);
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += (double)vec_sum<TT, VEC>(v[u]);
      }
      for (; i < rows; i += RPI) acc += (double)vec_sum<TT, VEC>(ld(base + (int64_t)i * N));
    }
  } else if (kRagged && col < col_end) {
    // the chunk straddling column N: its col_end - col valid elements
    const int nv = col_end - col;
    for (int h = 0; h < H_s; ++h) {
      const S* base = A + ((int64_t)h * N + (int64_t)I * B) * N + col;
      for (int i = r0; i < rows; i += RPI) {
        float t = 0.f;
        for (int e = 0; e < nv; ++e) t += TT::tof(base[(int64_t)i * N + e]);
        acc += (double)t;
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

template <class TT, int VEC, bool kRagged = false>
hipError_t launch_t(const void* A, int H_s, int N, int B, float* mass,
                    hipStream_t st) {
  const int esz = (int)sizeof(typename TT::S);
  const int T = mf::blocks_of(N, B);
  const int limit = min(1024, kThreads * VEC);     // strip row bytes
  const int JPC = max(1, limit / (B * esz));
  dim3 grid(T, (T + JPC - 1) / JPC);
  hipLaunchKernelGGL((k_block_mass<TT, VEC, kRagged>), grid, dim3(kThreads), 0, st,
                     reinterpret_cast<const typename TT::S*>(A), H_s, N, B, JPC,
                     mass);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Row-streaming variant (needs a workspace)
// ---------------------------------------------------------------------------
//
// A workgroup owns one (head h, block row I): it streams the causal part of
// the block row's map rows, columns [0, min(N, (I+1)B)), as whole contiguous
// rows (a scan of the map in column strips reads 1 KB pieces of rows N*e
// bytes apart and reaches about 80% of the rate of whole rows).  Columns go in
// chunks of at most NPT * kRowThreads 16-byte pieces; within a chunk every
// thread owns NPT fixed pieces (so fixed column blocks) of RPP rows per pass,
// sums their elements in fp32 and accumulates in fp64, with UNR rows in
// flight.  Each chunk's per-J totals are formed over LDS in a fixed order and
// stored, once rounded to fp32, as part[h][I(I+1)/2 + J] (the causal
// triangle); a second kernel adds the heads in a fixed order in fp64.
// Workgroups go longest row first, consecutive ones on different heads of the
// same block row.
// kRagged (N*e not a multiple of VEC, or A off a VEC-byte boundary): rows
// start off a VEC-byte boundary, so pieces are read with loads aligned only
// to the element size, and the last block row's final N mod EPV columns are
// summed one element at a time per row and added to their column block.
constexpr int kRowThreads = 512;

template <class TT, int VEC, int UNR, bool kRagged>
__global__ __launch_bounds__(kRowThreads) void k_block_mass_rows(
    const typename TT::S* __restrict__ A, int H_s, int N, int B, float* __restrict__ part) {
  using S = typename TT::S;
  using V = typename VecT<VEC>::T;
  constexpr int EPV = VEC / (int)sizeof(S);      // elements per piece
  constexpr int NPT = 2;                         // pieces per thread in a wide chunk
  __shared__ double red[NPT * kRowThreads];
  __shared__ double tail[kRagged ? 128 : 1];     // per-row sum of the ragged columns
  auto ld = [](const S* q) -> V {
    if constexpr (kRagged) return load_any<VEC>(q);
    else return *reinterpret_cast<const V*>(q);
  };
  const int T = (N + B - 1) / B;
  const int h = blockIdx.x % H_s;
  const int I = T - 1 - (int)(blockIdx.x / H_s);
  const int tid = threadIdx.x;
  const int rows = min(B, N - I * B);
  const int cols = min(N, (I + 1) * B);          // causal columns of these rows
  const int P = cols / EPV;                      // whole pieces per row (>= 1: N >= EPV)
  const int CPJ = B / EPV;                       // pieces per column block
  const int64_t tri = (int64_t)T * (T + 1) / 2;
  float* out = part + (int64_t)h * tri + (int64_t)I * (I + 1) / 2;
  const S* rowbase = A + ((int64_t)h * N + (int64_t)I * B) * N;
  // ragged columns [P EPV, cols) (last block row only): column block Jt
  const int tailn = kRagged ? cols - P * EPV : 0;
  const int Jt = (P * EPV) / B;
  if (kRagged && tailn > 0 && tid < rows) {
    const S* q = rowbase + (int64_t)tid * N + (int64_t)P * EPV;
    float t = 0.f;
    for (int e = 0; e < tailn; ++e) t += TT::tof(q[e]);
    tail[tid] = (double)t;
  }
  for (int c0 = 0; c0 < P; c0 += NPT * kRowThreads) {
    const int CW = min(P - c0, NPT * kRowThreads);  // pieces in this chunk
    // narrow chunk (CW <= kRowThreads): one piece per thread, RPP rows per
    // pass; wide chunk: pieces c and c + kRowThreads of every row (the second
    // clamped into the chunk and masked, so that both loads are unconditional)
    const int W = min(CW, kRowThreads);
    const int RPP = kRowThreads / W;             // rows per pass
    const int rr = tid / W, c = tid % W;
    double acc0 = 0.0, acc1 = 0.0;
    if (CW <= kRowThreads) {
      if (rr < RPP) {
        const S* p = rowbase + (int64_t)rr * N + (int64_t)(c0 + c) * EPV;
        const int64_t step = (int64_t)RPP * N;
        int r = rr;
        for (; r + (UNR - 1) * RPP < rows; r += UNR * RPP) {
          V v[UNR];
#pragma unroll
          for (int u = 0; u < UNR; ++u) v[u] = ld(p + u * step);
#pragma unroll
          for (int u = 0; u < UNR; ++u) acc0 += (double)vec_sum<TT, VEC>(v[u]);
          p += UNR * step;
        }
        for (; r < rows; r += RPP, p += step) acc0 += (double)vec_sum<TT, VEC>(ld(p));
      }
    } else {
      const bool has1 = c + kRowThreads < CW;
      const int c1 = has1 ? c + kRowThreads : CW - 1;
      const S* p0 = rowbase + (int64_t)(c0 + c) * EPV;
      const S* p1 = rowbase + (int64_t)(c0 + c1) * EPV;
      constexpr int U2 = UNR / 2;
      int r = 0;
      for (; r + U2 - 1 < rows; r += U2) {
        V v0[U2], v1[U2];
#pragma unroll
        for (int u = 0; u < U2; ++u) {
          v0[u] = ld(p0 + (int64_t)(r + u) * N);
          v1[u] = ld(p1 + (int64_t)(r + u) * N);
        }
#pragma unroll
        for (int u = 0; u < U2; ++u) {
          acc0 += (double)vec_sum<TT, VEC>(v0[u]);
          const double s1 = (double)vec_sum<TT, VEC>(v1[u]);
          acc1 += has1 ? s1 : 0.0;
        }
      }
      for (; r < rows; ++r) {
        acc0 += (double)vec_sum<TT, VEC>(ld(p0 + (int64_t)r * N));
        const double s1 = (double)vec_sum<TT, VEC>(ld(p1 + (int64_t)r * N));
        acc1 += has1 ? s1 : 0.0;
      }
    }
    red[tid] = acc0;
    red[kRowThreads + tid] = acc1;
    __syncthreads();
    // column blocks of this chunk, J = (c0 + x) / CPJ for x < CW; piece x is
    // held by threads (x % W) + W q, q < RPP, in slot k = x / W.  Chunks start
    // at multiples of NPT * kRowThreads, which CPJ (a power of two <= 128)
    // divides, so no column block spans two chunks.
    // The ragged columns join the last chunk: their block Jt is the chunk's
    // last one, or the next one when they start a block of their own (xb = xe).
    const int j0 = c0 / CPJ;
    int j1 = (c0 + CW - 1) / CPJ;
    if (kRagged && tailn > 0 && c0 + CW == P) j1 = max(j1, Jt);
    for (int jj = tid; jj <= j1 - j0; jj += kRowThreads) {
      const int J = j0 + jj;
      const int xb = J * CPJ - c0, xe = min((J + 1) * CPJ, c0 + CW) - c0;
      double s = 0.0;
      for (int x = xb; x < xe; ++x) {
        const int k = x / W, cc = x - k * W;
        for (int q = 0; q < RPP; ++q) s += red[k * kRowThreads + q * W + cc];
      }
      if (kRagged && tailn > 0 && J == Jt)
        for (int r = 0; r < rows; ++r) s += tail[r];
      out[J] = (float)s;
    }
    __syncthreads();
  }
}

// mass[I][J] = (1/H_s) sum_h part[h][I(I+1)/2 + J] in fp64, head order fixed;
// J > I is 0.  Workgroup (I, 64 columns); thread (column, head group q of 4)
// adds heads q, q+4, ...; the four partials are added in the order 0..3.
__global__ __launch_bounds__(256) void k_block_mass_heads(const float* __restrict__ part, int H_s,
                                                          int T, float* __restrict__ mass) {
  __shared__ double red[4][64];
  const int I = blockIdx.y;
  const int c = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int J = blockIdx.x * 64 + c;
  const int64_t tri = (int64_t)T * (T + 1) / 2;
  const int64_t o = (int64_t)I * (I + 1) / 2 + J;
  double s = 0.0;
  if (J <= I)
    for (int h = q; h < H_s; h += 4) s += (double)part[(int64_t)h * tri + o];
  red[q][c] = s;
  __syncthreads();
  if (q == 0 && J < T)
    mass[(int64_t)I * T + J] = J <= I ? (float)((((red[0][c] + red[1][c]) + red[2][c]) + red[3][c]) / (double)H_s) : 0.f;
}

template <class TT, int VEC, bool kRagged = false>
hipError_t launch_rows_t(const void* A, int H_s, int N, int B, float* mass, float* part,
                         hipStream_t st) {
  const int T = mf::blocks_of(N, B);
  const auto* a = reinterpret_cast<const typename TT::S*>(A);
  hipLaunchKernelGGL((k_block_mass_rows<TT, VEC, 8, kRagged>), dim3(H_s * T), dim3(kRowThreads), 0, st,
                     a, H_s, N, B, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_block_mass_heads, dim3((T + 63) / 64, T), dim3(256), 0, st, part, H_s, T, mass);
  return hipGetLastError();
}

}  // namespace

namespace mf {

size_t block_mass_rows_workspace_bytes(int H_s, int N, int B) {
  const int64_t T = blocks_of(N, B);
  return (size_t)H_s * (size_t)(T * (T + 1) / 2) * sizeof(float);
}

hipError_t launch_block_mass_heads(const float* part, int H_s, int T, float* mass, hipStream_t st) {
  hipLaunchKernelGGL(k_block_mass_heads, dim3((T + 63) / 64, T), dim3(256), 0, st, part, H_s, T, mass);
  return hipGetLastError();
}

hipError_t launch_block_mass_rows(const void* A, int dt, int H_s, int N, int B, float* mass,
                                  void* workspace, hipStream_t st) {
  float* part = reinterpret_cast<float*>(workspace);
  const int esz = dtype_bytes(dt);
  const int vec = row_vec_bytes(A, N, B, esz);
  if (vec < 16 && ragged_rows_ok(A, N, esz)) {
    // rows off a 16-byte boundary: 16-byte pieces all the same, ragged end apart
    if (dt == MF_F32) return launch_rows_t<mfd::TF32, 16, true>(A, H_s, N, B, mass, part, st);
    if (dt == MF_F16) return launch_rows_t<mfd::TF16, 16, true>(A, H_s, N, B, mass, part, st);
    return launch_rows_t<mfd::TBF16, 16, true>(A, H_s, N, B, mass, part, st);
  }
  if (dt == MF_F32) {
    if (vec >= 16) return launch_rows_t<mfd::TF32, 16>(A, H_s, N, B, mass, part, st);
    if (vec >= 8) return launch_rows_t<mfd::TF32, 8>(A, H_s, N, B, mass, part, st);
    return launch_rows_t<mfd::TF32, 4>(A, H_s, N, B, mass, part, st);
  }
  if (dt == MF_F16) {
    if (vec >= 16) return launch_rows_t<mfd::TF16, 16>(A, H_s, N, B, mass, part, st);
    if (vec >= 8) return launch_rows_t<mfd::TF16, 8>(A, H_s, N, B, mass, part, st);
    if (vec >= 4) return launch_rows_t<mfd::TF16, 4>(A, H_s, N, B, mass, part, st);
    return launch_rows_t<mfd::TF16, 2>(A, H_s, N, B, mass, part, st);
  }
  if (vec >= 16) return launch_rows_t<mfd::TBF16, 16>(A, H_s, N, B, mass, part, st);
  if (vec >= 8) return launch_rows_t<mfd::TBF16, 8>(A, H_s, N, B, mass, part, st);
  if (vec >= 4) return launch_rows_t<mfd::TBF16, 4>(A, H_s, N, B, mass, part, st);
  return launch_rows_t<mfd::TBF16, 2>(A, H_s, N, B, mass, part, st);
}

hipError_t launch_block_mass(const void* A, int dt, int H_s, int N, int B,
                             float* mass, hipStream_t st) {
  const int esz = dtype_bytes(dt);
  const int vec = row_vec_bytes(A, N, B, esz);
  if (vec < 16 && ragged_rows_ok(A, N, esz)) {
    if (dt == MF_F32) return launch_t<mfd::TF32, 16, true>(A, H_s, N, B, mass, st);
    if (dt == MF_F16) return launch_t<mfd::TF16, 16, true>(A, H_s, N, B, mass, st);
    return launch_t<mfd::TBF16, 16, true>(A, H_s, N, B, mass, st);
  }
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
