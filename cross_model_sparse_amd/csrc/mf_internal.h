// Internal declarations shared by the libmapflow translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "mapflow.h"

namespace mf {

// Records a message for mf_last_error() and returns `st`.
int fail(int st, const std::string& msg);
// Checks a HIP status after a launch or runtime call.
int hip_check(hipError_t e, const char* what);

inline int blocks_of(int N, int B) { return (N + B - 1) / B; }
inline int dtype_bytes(int dt) { return dt == MF_F32 ? 4 : 2; }

// Largest load width in bytes (16, 8, 4 or the element size) such that every
// row segment of a block tile starts on that alignment.
int row_vec_bytes(const void* base, int N, int B, int esize);
// True when map rows that miss row_vec_bytes' 16 bytes can still be read in
// 16-byte pieces with element-aligned loads: A element-aligned and a row at
// least 16 bytes long (so every block row has a whole piece).
bool ragged_rows_ok(const void* base, int N, int esize);

// Kernel launchers (one per translation unit); arguments already validated.
// Row-streaming block mass: per-(head, block row) workgroups into an fp32
// workspace of block_mass_rows_workspace_bytes, then a fixed-order head sum.
size_t block_mass_rows_workspace_bytes(int H_s, int N, int B);
// mass[I][J] = (1/H_s) sum_h part[h][I(I+1)/2 + J] in fp64, head order fixed;
// zeros above the diagonal (part: H_s * T(T+1)/2 fp32 per-head block sums)
hipError_t launch_block_mass_heads(const float* part, int H_s, int T, float* mass, hipStream_t st);
hipError_t launch_block_mass_rows(const void* A, int dt, int H_s, int N, int B, float* mass,
                                  void* workspace, hipStream_t st);
hipError_t launch_block_mass(const void* A, int dt, int H_s, int N, int B,
                             float* mass, hipStream_t st);
hipError_t launch_topp_bsr(const float* mass, const void* A, int dt, int H_s,
                           int N, int B, float p, int32_t* row_ptr,
                           int32_t* col_idx, void* vals, int64_t cap_nnzb,
                           void* workspace, hipStream_t st);
// Top-p selection and row_ptr scan only (kept[T][T] and counts in workspace).
hipError_t launch_select_scan(const float* mass, int N, int B, float p, int32_t* row_ptr,
                              void* workspace, hipStream_t st);
// Compression from Q and K (k_qk.hip).
hipError_t launch_row_lse(const void* Q, const void* K, int dt, int H_s, int H_ks, int N, int d,
                          const float* scale, float* lse, hipStream_t st);
size_t block_mass_qk_workspace_bytes(int H_s, int N, int B);
// lse and block masses in one pass over the scores ((m, e) pairs per row and
// column block in the workspace, then a fixed-order reduction)
size_t lse_block_mass_qk_workspace_bytes(int H_s, int N, int B);
hipError_t launch_lse_block_mass_qk(const void* Q, const void* K, const float* scale, int dt,
                                    int H_s, int H_ks, int N, int d, int B, float* lse,
                                    float* mass, void* workspace, hipStream_t st);
hipError_t launch_block_mass_qk(const void* Q, const void* K, const float* scale, const float* lse,
                                int dt, int H_s, int H_ks, int N, int d, int B, float* mass,
                                void* workspace, hipStream_t st);
// Kept tiles recomputed from Q, K, lse; row_ptr and kept[T][T] from launch_select_scan.
hipError_t launch_gather_qk(const void* Q, const void* K, const float* scale, const float* lse,
                            int dt, int H_s, int H_ks, int N, int d, int B,
                            const int32_t* row_ptr, const int32_t* kept, int64_t cap,
                            int32_t* col_idx, void* vals, hipStream_t st);
int launch_retrieve(const int32_t* row_ptr, const int32_t* col_idx,
                    const void* vals, int64_t nnzb, int dt, int H_s, int N,
                    int B, const float* W, int H_r, const void* V, int H_kv,
                    int d, int64_t ldV, void* O, int64_t ldO, void* workspace,
                    size_t workspace_bytes, hipStream_t st);
// Several receivers (host arrays of n_recv entries) fed from one BSR state.
int launch_retrieve_multi(const int32_t* row_ptr, const int32_t* col_idx, const void* vals,
                          int64_t nnzb, int dt, int H_s, int N, int B, int n_recv,
                          const float* const* W, const int* H_r, const void* const* V,
                          const int* H_kv, int d, const int64_t* ldV, void* const* O,
                          const int64_t* ldO, hipStream_t st);
// One launch over a packed batch of S sequences (R block rows in total).
int launch_retrieve_varlen(int S, int R, const int32_t* cu_seqlens, const int32_t* cu_rows,
                           const int32_t* row_ptr, const int32_t* col_idx,
                           const int32_t* block_table, const void* vals, int64_t n_pages,
                           int64_t nnzb, int dt, int H_s, int B, const float* W, int H_r,
                           const void* V, int H_kv, int d, int64_t ldV, void* O, int64_t ldO,
                           hipStream_t st);
size_t retrieve_workspace_bytes(int N, int B, int H_kv, int d, int dt);
// Workspace that lets launch_retrieve split long block rows (0 when splitting
// does not apply to these shapes); split_part_len is the longest part.
size_t split_workspace_bytes(int dt, int H_s, int N, int B, int H_r, int H_kv, int d, int64_t nnzb);
int split_part_len(int64_t nnzb, int B);
// True when launch_retrieve runs the matrix-core kernel for these arguments.
bool retrieve_uses_mfma(int dt, int H_s, int B, int H_r, int H_kv, int d, const void* vals,
                        const void* V, int64_t ldV, const void* O, int64_t ldO);

}  // namespace mf

// ---- device helpers -------------------------------------------------------

namespace mfd {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __uint_as_float(((unsigned)h) << 16);
}
__device__ __forceinline__ float f16_to_f32(unsigned short h) {
  return (float)__builtin_bit_cast(_Float16, h);
}
// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ unsigned short f32_to_bf16(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (unsigned short)((u >> 16) | 0x40);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}
// fp32 -> fp16 bits, round to nearest even.
__device__ __forceinline__ unsigned short f32_to_f16(float f) {
  return __builtin_bit_cast(unsigned short, (_Float16)f);
}
__device__ __forceinline__ unsigned pack_f16x2(float lo, float hi) {
  return (unsigned)f32_to_f16(lo) | ((unsigned)f32_to_f16(hi) << 16);
}
// Two bf16 values packed in a dword -> two fp16 values (RNE).
__device__ __forceinline__ unsigned bf16x2_to_f16x2(unsigned v) {
  return pack_f16x2(__uint_as_float(v << 16), __uint_as_float(v & 0xffff0000u));
}

// Storage-type tags: S is the element type in memory.
struct TF32 {
  using S = float;
  static __device__ __forceinline__ float tof(S x) { return x; }
  static __device__ __forceinline__ S fromf(float f) { return f; }
};
struct TF16 {
  using S = unsigned short;
  static __device__ __forceinline__ float tof(S x) { return f16_to_f32(x); }
  static __device__ __forceinline__ S fromf(float f) { return f32_to_f16(f); }
};
struct TBF16 {
  using S = unsigned short;
  static __device__ __forceinline__ float tof(S x) { return bf16_to_f32(x); }
  static __device__ __forceinline__ S fromf(float f) { return f32_to_bf16(f); }
};

// Vector of VEC bytes used for global loads and stores.
template <int VEC> struct VecT;
template <> struct VecT<16> { using T = uint4; };
template <> struct VecT<8> { using T = uint2; };
template <> struct VecT<4> { using T = unsigned; };
template <> struct VecT<2> { using T = unsigned short; };

// VEC bytes from an address aligned only to the element size.  The HSA
// target runs with unaligned global access enabled, so this is still one
// vector load (the memory path splits it where it crosses a line); it serves
// map rows that do not start on a VEC-byte boundary (N*e not a multiple of
// VEC, as in ragged sequence lengths).
template <int VEC, class S>
__device__ __forceinline__ typename VecT<VEC>::T load_any(const S* p) {
  typename VecT<VEC>::T v;
  __builtin_memcpy(&v, p, VEC);
  return v;
}

// Sum, in fp32, of the elements packed in one vector.
template <class TT, int VEC>
__device__ __forceinline__ float vec_sum(const typename VecT<VEC>::T& v) {
  constexpr int ES = sizeof(typename TT::S);
  constexpr int NE = VEC / ES;
  const typename TT::S* e = reinterpret_cast<const typename TT::S*>(&v);
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < NE; ++j) s += TT::tof(e[j]);
  return s;
}

}  // namespace mfd
