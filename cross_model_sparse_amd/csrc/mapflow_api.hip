// C boundary of libmapflow: argument validation, status codes and error text.
// Every entry point checks its arguments on the host before touching the GPU.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>

#include "mf_internal.h"

// Fixed scratch of mf_topp_select_bsr_noalloc: the selection's kept[T][T] and
// count[T] int32 arrays for up to kNoAllocMaxT block rows.  Each GPU the
// library runs on holds its own copy for the life of the process.  Host code
// never uses this name as an address: the per-device address comes from
// hipGetSymbolAddress (noalloc_scratch below).
namespace {
constexpr int kNoAllocMaxT = 1024;
constexpr size_t kNoAllocScratchBytes = ((size_t)kNoAllocMaxT * kNoAllocMaxT + kNoAllocMaxT) * 4;
}  // namespace
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace mf {

namespace {
thread_local std::string g_last_error;
}

int fail(int st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

int hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return MF_OK;
  return fail(MF_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

int row_vec_bytes(const void* base, int N, int B, int esize) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(base);
  for (int v = 16; v > esize; v >>= 1) {
    if ((a % v) == 0 && ((int64_t)N * esize) % v == 0 && ((int64_t)B * esize) % v == 0)
      return v;
  }
  return esize;
}

bool ragged_rows_ok(const void* base, int N, int esize) {
  return (reinterpret_cast<uintptr_t>(base) % esize) == 0 && (int64_t)N * esize >= 16;
}

}  // namespace mf

namespace {

bool valid_dtype(int dt) { return dt == MF_F32 || dt == MF_F16 || dt == MF_BF16; }
bool valid_block(int B) { return B == 16 || B == 32 || B == 64 || B == 128; }

std::string fmt(const char* f, long long a, long long b = 0) {
  char buf[256];
  snprintf(buf, sizeof buf, f, a, b);
  return buf;
}

// Shared checks of the map geometry; returns MF_OK or records the error.
int check_geom(const char* fn, int dtype, int H_s, int N, int B) {
  using mf::fail;
  std::string f = std::string(fn) + ": ";
  if (!valid_dtype(dtype)) return fail(MF_ERR_INVALID, f + fmt("unknown dtype code %lld", dtype));
  if (N < 1) return fail(MF_ERR_INVALID, f + fmt("N must be >= 1 (got %lld)", N));
  if (!valid_block(B)) return fail(MF_ERR_INVALID, f + fmt("B must be 16, 32, 64 or 128 (got %lld)", B));
  if (H_s < 1 || H_s > 64) return fail(MF_ERR_INVALID, f + fmt("H_s must be in [1, 64] (got %lld)", H_s));
  return MF_OK;
}

}  // namespace

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of `scratch` on the calling thread's current device, looked
// up once per device and cached.
int noalloc_scratch(const char* fn, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mf::hip_check(e, fn);
  if (dev < 0 || dev >= kMaxDevices)
    return mf::fail(MF_ERR_UNSUPPORTED, std::string(fn) + fmt(": device index %lld >= 64", dev));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return mf::hip_check(e != hipSuccess ? e : hipErrorInvalidSymbol,
                           (std::string(fn) + " scratch address").c_str());
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return MF_OK;
}

}  // namespace

extern "C" {

int mf_abi_version(void) { return MF_ABI_VERSION; }

const char* mf_status_string(int status) {
  switch (status) {
    case MF_OK: return "MF_OK";
    case MF_ERR_INVALID: return "MF_ERR_INVALID: invalid argument";
    case MF_ERR_UNSUPPORTED: return "MF_ERR_UNSUPPORTED: valid arguments, combination not built";
    case MF_ERR_CAPACITY: return "MF_ERR_CAPACITY: BSR larger than the given capacity";
    case MF_ERR_HIP: return "MF_ERR_HIP: HIP runtime error";
    default: return "unknown mapflow status";
  }
}

const char* mf_last_error(void) { return mf::g_last_error.c_str(); }

size_t mf_block_mass_ws_bytes(int H_s, int N, int B) {
  if (H_s < 1 || N < 1 || B < 1) return 0;
  return mf::block_mass_rows_workspace_bytes(H_s, N, B);
}

int mf_block_mass_ws(const void* A, int dtype, int H_s, int N, int B, float* mass,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mf_block_mass_ws";
  int st = check_geom(fn, dtype, H_s, N, B);
  if (st != MF_OK) return st;
  if (!A || !mass || !workspace) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  const size_t need = mf::block_mass_rows_workspace_bytes(H_s, N, B);
  if (workspace_bytes < need)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": workspace of %lld bytes < %lld required",
                                                          (long long)workspace_bytes, (long long)need));
  return mf::hip_check(mf::launch_block_mass_rows(A, dtype, H_s, N, B, mass, workspace,
                                                  (hipStream_t)stream),
                       "mf_block_mass_ws launch");
}

int mf_block_mass(const void* A, int dtype, int H_s, int N, int B, float* mass,
                  void* stream) {
  int st = check_geom("mf_block_mass", dtype, H_s, N, B);
  if (st != MF_OK) return st;
  if (!A || !mass) return mf::fail(MF_ERR_INVALID, "mf_block_mass: null pointer");
  return mf::hip_check(
      mf::launch_block_mass(A, dtype, H_s, N, B, mass, (hipStream_t)stream),
      "mf_block_mass launch");
}

size_t mf_topp_workspace_bytes(int N, int B) {
  if (N < 1 || B < 1) return 0;
  const size_t T = (size_t)mf::blocks_of(N, B);
  const size_t bytes = (T * T + T) * sizeof(int32_t);
  return (bytes + 255) & ~(size_t)255;
}

int mf_topp_select_bsr(const float* mass, const void* A, int dtype, int H_s,
                       int N, int B, float p, int32_t* row_ptr,
                       int32_t* col_idx, void* vals, int64_t cap_nnzb,
                       int64_t* nnzb_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  const char* fn = "mf_topp_select_bsr";
  int st = check_geom(fn, dtype, H_s, N, B);
  if (st != MF_OK) return st;
  if (!mass || !A || !row_ptr || !workspace)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  if (cap_nnzb < 0) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": cap_nnzb < 0");
  if (cap_nnzb > 0 && (!col_idx || !vals))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null col_idx/vals with cap_nnzb > 0");
  if (!(p > 0.0f && p <= 1.0f))  // also rejects NaN
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": p must be in (0, 1]");
  const int T = mf::blocks_of(N, B);
  if (T > 4096)
    return mf::fail(MF_ERR_UNSUPPORTED, std::string(fn) + fmt(": T = %lld block rows > 4096", T));
  if (workspace_bytes < mf_topp_workspace_bytes(N, B))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": workspace of %lld bytes < %lld required",
                                                          (long long)workspace_bytes,
                                                          (long long)mf_topp_workspace_bytes(N, B)));
  hipStream_t s = (hipStream_t)stream;
  st = mf::hip_check(mf::launch_topp_bsr(mass, A, dtype, H_s, N, B, p, row_ptr,
                                         col_idx, vals, cap_nnzb, workspace, s),
                     "mf_topp_select_bsr launch");
  if (st != MF_OK || !nnzb_out) return st;
  int32_t nnzb = 0;
  st = mf::hip_check(hipMemcpyAsync(&nnzb, row_ptr + T, sizeof nnzb,
                                    hipMemcpyDeviceToHost, s),
                     "mf_topp_select_bsr nnzb read-back");
  if (st != MF_OK) return st;
  st = mf::hip_check(hipStreamSynchronize(s), "mf_topp_select_bsr synchronise");
  if (st != MF_OK) return st;
  *nnzb_out = nnzb;
  if (nnzb > cap_nnzb)
    return mf::fail(MF_ERR_CAPACITY, std::string(fn) + fmt(": nnzb = %lld exceeds cap_nnzb = %lld",
                                                           nnzb, cap_nnzb));
  return MF_OK;
}

int mf_topp_select_bsr_noalloc(const float* mass, const void* A, int dtype, int H_s, int N, int B,
                               float p, int32_t* row_ptr, int32_t* col_idx, void* vals,
                               int64_t cap_nnzb, void* stream) {
  const char* fn = "mf_topp_select_bsr_noalloc";
  int st = check_geom(fn, dtype, H_s, N, B);
  if (st != MF_OK) return st;
  if (!mass || !A || !row_ptr) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  if (cap_nnzb < 0) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": cap_nnzb < 0");
  if (cap_nnzb > 0 && (!col_idx || !vals))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null col_idx/vals with cap_nnzb > 0");
  if (!(p > 0.0f && p <= 1.0f))  // also rejects NaN
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": p must be in (0, 1]");
  const int T = mf::blocks_of(N, B);
  if (T > kNoAllocMaxT)
    return mf::fail(MF_ERR_UNSUPPORTED,
                    std::string(fn) + fmt(": T = %lld block rows exceeds the %lld that the fixed scratch "
                                          "holds (use mf_topp_select_bsr with a workspace)",
                                          T, kNoAllocMaxT));
  void* ws = nullptr;
  st = noalloc_scratch(fn, &ws);
  if (st != MF_OK) return st;
  return mf::hip_check(mf::launch_topp_bsr(mass, A, dtype, H_s, N, B, p, row_ptr, col_idx, vals,
                                           cap_nnzb, ws, (hipStream_t)stream),
                       "mf_topp_select_bsr_noalloc launch");
}

// Shape checks shared by the calls that read Q and K.
static int check_qk(const char* fn, int dtype, int H_s, int H_ks, int N, int d, int B) {
  int st = check_geom(fn, dtype, H_s, N, B);
  if (st != MF_OK) return st;
  if (H_ks < 1 || H_s % H_ks != 0)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": H_ks = %lld does not divide H_s", H_ks));
  if (d != 64 && d != 128) return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": d must be 64 or 128 (got %lld)", d));
  return MF_OK;
}

int mf_row_lse(const void* Q, const void* K, int dtype, int H_s, int H_ks, int N, int d,
               const float* scale, float* lse, void* stream) {
  const char* fn = "mf_row_lse";
  // any valid block size passes the shared geometry check
  int st = check_qk(fn, dtype, H_s, H_ks, N, d, 16);
  if (st != MF_OK) return st;
  if (!Q || !K || !scale || !lse) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  return mf::hip_check(mf::launch_row_lse(Q, K, dtype, H_s, H_ks, N, d, scale, lse,
                                          (hipStream_t)stream), "mf_row_lse launch");
}

size_t mf_block_mass_qk_workspace_bytes(int H_s, int N, int B) {
  if (H_s < 1 || H_s > 64 || N < 1 || !valid_block(B)) return 0;
  return mf::block_mass_qk_workspace_bytes(H_s, N, B);
}

size_t mf_lse_block_mass_qk_workspace_bytes(int H_s, int N, int B) {
  if (H_s < 1 || H_s > 64 || N < 1 || !valid_block(B)) return 0;
  return mf::lse_block_mass_qk_workspace_bytes(H_s, N, B);
}

int mf_lse_block_mass_qk(const void* Q, const void* K, const float* scale, int dtype, int H_s,
                         int H_ks, int N, int d, int B, float* lse, float* mass,
                         void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mf_lse_block_mass_qk";
  int st = check_qk(fn, dtype, H_s, H_ks, N, d, B);
  if (st != MF_OK) return st;
  if (!Q || !K || !scale || !lse || !mass || !workspace)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  const size_t need = mf::lse_block_mass_qk_workspace_bytes(H_s, N, B);
  if (workspace_bytes < need)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": workspace of %lld bytes < %lld required",
                                                          (long long)workspace_bytes, (long long)need));
  return mf::hip_check(mf::launch_lse_block_mass_qk(Q, K, scale, dtype, H_s, H_ks, N, d, B, lse, mass,
                                                    workspace, (hipStream_t)stream),
                       "mf_lse_block_mass_qk launch");
}

int mf_block_mass_qk(const void* Q, const void* K, const float* scale, const float* lse,
                     int dtype, int H_s, int H_ks, int N, int d, int B, float* mass,
                     void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mf_block_mass_qk";
  int st = check_qk(fn, dtype, H_s, H_ks, N, d, B);
  if (st != MF_OK) return st;
  if (!Q || !K || !scale || !lse || !mass || !workspace)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  const size_t need = mf::block_mass_qk_workspace_bytes(H_s, N, B);
  if (workspace_bytes < need)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": workspace of %lld bytes < %lld required",
                                                          (long long)workspace_bytes, (long long)need));
  return mf::hip_check(mf::launch_block_mass_qk(Q, K, scale, lse, dtype, H_s, H_ks, N, d, B, mass,
                                                workspace, (hipStream_t)stream),
                       "mf_block_mass_qk launch");
}

int mf_topp_select_bsr_qk(const float* mass, const void* Q, const void* K,
                          const float* scale, const float* lse, int dtype, int H_s,
                          int H_ks, int N, int d, int B, float p, int32_t* row_ptr,
                          int32_t* col_idx, void* vals, int64_t cap_nnzb,
                          int64_t* nnzb_out, void* workspace, size_t workspace_bytes,
                          void* stream) {
  const char* fn = "mf_topp_select_bsr_qk";
  int st = check_qk(fn, dtype, H_s, H_ks, N, d, B);
  if (st != MF_OK) return st;
  if (!mass || !Q || !K || !scale || !lse || !row_ptr || !workspace)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  if (cap_nnzb < 0) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": cap_nnzb < 0");
  if (cap_nnzb > 0 && (!col_idx || !vals))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null col_idx/vals with cap_nnzb > 0");
  if (!(p > 0.0f && p <= 1.0f))  // also rejects NaN
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": p must be in (0, 1]");
  const int T = mf::blocks_of(N, B);
  if (T > 4096)
    return mf::fail(MF_ERR_UNSUPPORTED, std::string(fn) + fmt(": T = %lld block rows > 4096", T));
  if (workspace_bytes < mf_topp_workspace_bytes(N, B))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": workspace of %lld bytes < %lld required",
                                                          (long long)workspace_bytes,
                                                          (long long)mf_topp_workspace_bytes(N, B)));
  hipStream_t s = (hipStream_t)stream;
  st = mf::hip_check(mf::launch_select_scan(mass, N, B, p, row_ptr, workspace, s),
                     "mf_topp_select_bsr_qk selection launch");
  if (st != MF_OK) return st;
  st = mf::hip_check(mf::launch_gather_qk(Q, K, scale, lse, dtype, H_s, H_ks, N, d, B, row_ptr,
                                          reinterpret_cast<const int32_t*>(workspace), cap_nnzb,
                                          col_idx, vals, s),
                     "mf_topp_select_bsr_qk gather launch");
  if (st != MF_OK || !nnzb_out) return st;
  int32_t nnzb = 0;
  st = mf::hip_check(hipMemcpyAsync(&nnzb, row_ptr + T, sizeof nnzb, hipMemcpyDeviceToHost, s),
                     "mf_topp_select_bsr_qk nnzb read-back");
  if (st != MF_OK) return st;
  st = mf::hip_check(hipStreamSynchronize(s), "mf_topp_select_bsr_qk synchronise");
  if (st != MF_OK) return st;
  *nnzb_out = nnzb;
  if (nnzb > cap_nnzb)
    return mf::fail(MF_ERR_CAPACITY, std::string(fn) + fmt(": nnzb = %lld exceeds cap_nnzb = %lld",
                                                           nnzb, cap_nnzb));
  return MF_OK;
}

size_t mf_retrieve_workspace_bytes(int N, int B, int H_kv, int d, int dtype) {
  if (N < 1 || !valid_block(B) || H_kv < 1 || !valid_dtype(dtype)) return 0;
  return mf::retrieve_workspace_bytes(N, B, H_kv, d, dtype);
}

size_t mf_retrieve_split_workspace_bytes(int64_t nnzb, int dtype, int H_s, int N, int B, int H_r,
                                         int H_kv, int d) {
  if (nnzb <= 0 || N < 1 || !valid_block(B) || !valid_dtype(dtype) || H_s < 1 || H_s > 64 ||
      H_r < 1 || H_r > 64 || H_kv < 1 || H_r % H_kv != 0)
    return 0;
  return mf::split_workspace_bytes(dtype, H_s, N, B, H_r, H_kv, d, nnzb);
}

// Shape and stride checks shared by mf_retrieve_fused and mf_retrieve_kernel.
static int check_retrieve_shape(const char* fn, int dtype, int H_s, int N, int B, int H_r,
                                int H_kv, int d, int64_t ldV, int64_t ldO) {
  int st = check_geom(fn, dtype, H_s, N, B);
  if (st != MF_OK) return st;
  if (H_r < 1 || H_r > 64) return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": H_r must be in [1, 64] (got %lld)", H_r));
  if (H_kv < 1 || H_r % H_kv != 0)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": H_r = %lld is not a multiple of H_kv = %lld", H_r, H_kv));
  if (d != 64 && d != 128) return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": d must be 64 or 128 (got %lld)", d));
  if (ldV < (int64_t)H_kv * d) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": ldV < H_kv*d");
  if (ldO < (int64_t)H_r * d) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": ldO < H_r*d");
  return MF_OK;
}

int mf_retrieve_kernel(int dtype, int H_s, int N, int B, int H_r, int H_kv, int d,
                       const void* vals, const void* V, int64_t ldV, const void* O,
                       int64_t ldO) {
  const int st = check_retrieve_shape("mf_retrieve_kernel", dtype, H_s, N, B, H_r, H_kv, d, ldV, ldO);
  if (st != MF_OK) return -st;
  return mf::retrieve_uses_mfma(dtype, H_s, B, H_r, H_kv, d, vals, V, ldV, O, ldO) ? 1 : 0;
}

int mf_retrieve_fused(const int32_t* row_ptr, const int32_t* col_idx,
                      const void* vals, int64_t nnzb, int dtype, int H_s,
                      int N, int B, const float* W, int H_r, const void* V,
                      int H_kv, int d, int64_t ldV, void* O, int64_t ldO,
                      void* workspace, size_t workspace_bytes, void* stream) {
  const char* fn = "mf_retrieve_fused";
  int st = check_geom(fn, dtype, H_s, N, B);
  if (st != MF_OK) return st;
  if (!row_ptr || !W || !V || !O) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  if (nnzb < 0) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": nnzb < 0");
  if (nnzb > 0 && (!col_idx || !vals))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null col_idx/vals with nnzb > 0");
  if (H_r < 1 || H_r > 64) return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": H_r must be in [1, 64] (got %lld)", H_r));
  if (H_kv < 1 || H_r % H_kv != 0)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": H_r = %lld is not a multiple of H_kv = %lld", H_r, H_kv));
  if (d != 64 && d != 128) return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": d must be 64 or 128 (got %lld)", d));
  if (ldV < (int64_t)H_kv * d) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": ldV < H_kv*d");
  if (ldO < (int64_t)H_r * d) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": ldO < H_r*d");
  const size_t need = mf::retrieve_workspace_bytes(N, B, H_kv, d, dtype);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": workspace of %lld bytes < %lld required",
                                                          workspace ? (long long)workspace_bytes : 0LL,
                                                          (long long)need));
  return mf::launch_retrieve(row_ptr, col_idx, vals, nnzb, dtype, H_s, N, B, W,
                             H_r, V, H_kv, d, ldV, O, ldO, workspace, workspace_bytes,
                             (hipStream_t)stream);
}

int mf_retrieve_fused_multi(const int32_t* row_ptr, const int32_t* col_idx, const void* vals,
                            int64_t nnzb, int dtype, int H_s, int N, int B, int n_recv,
                            const float* const* W, const int* H_r, const void* const* V,
                            const int* H_kv, int d, const int64_t* ldV, void* const* O,
                            const int64_t* ldO, void* stream) {
  const char* fn = "mf_retrieve_fused_multi";
  if (n_recv < 1 || n_recv > 4)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": n_recv must be in [1, 4] (got %lld)", n_recv));
  if (!W || !H_r || !V || !H_kv || !ldV || !O || !ldO)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null receiver array");
  if (!row_ptr) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  if (nnzb < 0) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": nnzb < 0");
  if (nnzb > 0 && (!col_idx || !vals))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null col_idx/vals with nnzb > 0");
  for (int i = 0; i < n_recv; ++i) {
    const std::string fi = std::string(fn) + fmt(" (receiver %lld)", i);
    const int st = check_retrieve_shape(fi.c_str(), dtype, H_s, N, B, H_r[i], H_kv[i], d, ldV[i], ldO[i]);
    if (st != MF_OK) return st;
    if (!W[i] || !V[i] || !O[i]) return mf::fail(MF_ERR_INVALID, fi + ": null pointer");
    for (int j = 0; j < i; ++j)
      if (O[j] == O[i]) return mf::fail(MF_ERR_INVALID, fi + ": output shared with another receiver");
  }
  return mf::launch_retrieve_multi(row_ptr, col_idx, vals, nnzb, dtype, H_s, N, B, n_recv, W, H_r, V,
                                   H_kv, d, ldV, O, ldO, (hipStream_t)stream);
}

int mf_retrieve_fused_varlen(int S, int R, const int32_t* cu_seqlens, const int32_t* cu_rows,
                             const int32_t* row_ptr, const int32_t* col_idx,
                             const int32_t* block_table, const void* vals, int64_t n_pages,
                             int64_t nnzb, int dtype, int H_s, int B, const float* W, int H_r,
                             const void* V, int H_kv, int d, int64_t ldV, void* O, int64_t ldO,
                             void* stream) {
  const char* fn = "mf_retrieve_fused_varlen";
  if (S < 1) return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt(": S must be >= 1 (got %lld)", S));
  if (R < 0) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": R < 0");
  // N = 1 stands in for the per-sequence lengths, which live on the device
  const int st = check_retrieve_shape(fn, dtype, H_s, 1, B, H_r, H_kv, d, ldV, ldO);
  if (st != MF_OK) return st;
  if (!cu_seqlens || !cu_rows || !row_ptr || !W || !V || !O)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  if (nnzb < 0) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": nnzb < 0");
  if (nnzb > 0 && (!col_idx || !vals))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null col_idx/vals with nnzb > 0");
  if (block_table && n_pages < 0) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": n_pages < 0");
  return mf::launch_retrieve_varlen(S, R, cu_seqlens, cu_rows, row_ptr, col_idx, block_table, vals,
                                    n_pages, nnzb, dtype, H_s, B, W, H_r, V, H_kv, d, ldV, O, ldO,
                                    (hipStream_t)stream);
}

}  // extern "C"
