// Block Manager: the prefix-hash index of cached BSR block rows.
//
// MapFlow keeps its compressed attention state in a cache organised by a
// Block Manager that indexes it with prefix hashes, each carrying the
// information of all preceding context (paper page, "Practical Implementation
// Details"; article, third section, second component).  Block row I of a
// sender layer's causal map depends on tokens 0 .. (I+1)B-1 and nothing else,
// so it is cached under the chained hash of exactly that prefix:
//     h_0 = seed,  h_{c+1} = FNV-1a-64( h_c as 8 little-endian bytes,
//                                       tokens cB .. cB+B-1 as 4 little-endian bytes each )
// and block row I is keyed by (layer, h_{I+1}).  An entry stores the row's
// kept columns and, for each kept block, the page of a device tile pool that
// holds its [H_s][B][B] tiles; it also stores the parent hash h_I and the
// chunk's tokens, and a lookup compares both, so a hash collision can only
// make a row look absent, never wrong.  Only full chunks are cached (a partial
// last block row depends on the sequence length).
//
// Pages are handed out smallest index first; when none is free, rows that no
// lookup holds (reference count 0) are evicted least recently used first.
// Every operation on one manager takes its mutex, so a manager can be shared
// by host threads.  The tiles themselves move with mf_pool_store (a device
// copy kernel below); the manager is host bookkeeping only.
#include <cstring>
#include <map>
#include <mutex>
#include <set>
#include <unordered_map>
#include <vector>

#include "mf_internal.h"

namespace {

constexpr uint64_t kFnvOffset = 14695981039346656037ull;
constexpr uint64_t kFnvPrime = 1099511628211ull;

inline uint64_t fnv_bytes(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

// h_{c+1} from h_c and chunk tokens (byte order fixed to little-endian)
uint64_t chain(uint64_t parent, const int32_t* tok, int B) {
  unsigned char buf[8];
  for (int i = 0; i < 8; ++i) buf[i] = (unsigned char)(parent >> (8 * i));
  uint64_t h = fnv_bytes(kFnvOffset, buf, 8);
  for (int t = 0; t < B; ++t) {
    const uint32_t v = (uint32_t)tok[t];
    unsigned char b[4] = {(unsigned char)v, (unsigned char)(v >> 8), (unsigned char)(v >> 16),
                          (unsigned char)(v >> 24)};
    h = fnv_bytes(h, b, 4);
  }
  return h;
}

struct Row {
  uint64_t parent;
  std::vector<int32_t> tokens;   // the chunk, for verification
  std::vector<int32_t> cols;     // kept column blocks, ascending
  std::vector<int32_t> pages;    // pool page of each kept block
  int64_t refs = 0;
  uint64_t stamp = 0;            // last use (logical clock)
};

struct Key {
  int layer;
  uint64_t h;
  bool operator==(const Key& o) const { return layer == o.layer && h == o.h; }
};
struct KeyHash {
  size_t operator()(const Key& k) const { return (size_t)(k.h ^ ((uint64_t)k.layer * 0x9e3779b97f4a7c15ull)); }
};

}  // namespace

struct mf_block_manager {
  int B, n_layers;
  int64_t n_pages;
  uint64_t seed;
  std::mutex mu;
  std::unordered_map<Key, Row, KeyHash> rows;
  std::set<int32_t> free_pages;                       // smallest first
  std::map<uint64_t, Key> lru;                        // stamp -> key, rows with refs == 0
  uint64_t clock = 0;
  int64_t hits = 0, misses = 0, evictions = 0, inserted = 0;
};

namespace {

std::string fmt2(const char* f, long long a, long long b = 0) {
  char buf[256];
  snprintf(buf, sizeof buf, f, a, b);
  return buf;
}

void touch(mf_block_manager* m, const Key& k, Row& r) {
  if (r.refs == 0) m->lru.erase(r.stamp);
  r.stamp = ++m->clock;
  if (r.refs == 0) m->lru.emplace(r.stamp, k);
}

// frees pages by evicting least recently used unreferenced rows until `need`
// pages are free; false (and nothing evicted) when even evicting every
// unreferenced row would not free enough
bool make_room(mf_block_manager* m, int64_t need) {
  int64_t avail = (int64_t)m->free_pages.size();
  for (auto it = m->lru.begin(); it != m->lru.end() && avail < need; ++it)
    avail += (int64_t)m->rows.find(it->second)->second.pages.size();
  if (avail < need) return false;
  while ((int64_t)m->free_pages.size() < need) {
    if (m->lru.empty()) return false;
    auto it = m->lru.begin();
    const Key k = it->second;
    m->lru.erase(it);
    auto rit = m->rows.find(k);
    for (int32_t p : rit->second.pages) m->free_pages.insert(p);
    m->rows.erase(rit);
    ++m->evictions;
  }
  return true;
}

}  // namespace

extern "C" {

int mf_prefix_hashes(const int32_t* tokens, int64_t n_tokens, int B, uint64_t seed,
                     uint64_t* hashes) {
  if (B < 1) return mf::fail(MF_ERR_INVALID, fmt2("mf_prefix_hashes: B must be >= 1 (got %lld)", B));
  if (n_tokens < 0) return mf::fail(MF_ERR_INVALID, "mf_prefix_hashes: n_tokens < 0");
  const int64_t n = n_tokens / B;
  if (n > 0 && (!tokens || !hashes)) return mf::fail(MF_ERR_INVALID, "mf_prefix_hashes: null pointer");
  uint64_t h = seed;
  for (int64_t c = 0; c < n; ++c) {
    h = chain(h, tokens + c * B, B);
    hashes[c] = h;
  }
  return MF_OK;
}

mf_block_manager* mf_bm_create(int B, int n_layers, int64_t n_pages, uint64_t seed) {
  if (B < 1 || n_layers < 1 || n_pages < 0 || n_pages > INT32_MAX) {
    mf::fail(MF_ERR_INVALID, "mf_bm_create: need B >= 1, n_layers >= 1, 0 <= n_pages <= 2^31-1");
    return nullptr;
  }
  auto* m = new (std::nothrow) mf_block_manager();
  if (!m) {
    mf::fail(MF_ERR_INVALID, "mf_bm_create: out of host memory");
    return nullptr;
  }
  m->B = B;
  m->n_layers = n_layers;
  m->n_pages = n_pages;
  m->seed = seed;
  for (int64_t p = 0; p < n_pages; ++p) m->free_pages.insert(m->free_pages.end(), (int32_t)p);
  return m;
}

void mf_bm_destroy(mf_block_manager* m) { delete m; }

int mf_bm_lookup(mf_block_manager* m, int layer, const int32_t* tokens, int64_t n_tokens,
                 int max_rows, int* n_rows, int32_t* row_ptr, int32_t* col_idx, int32_t* pages,
                 int64_t cap) {
  const char* fn = "mf_bm_lookup";
  if (!m || !n_rows || !row_ptr) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  std::lock_guard<std::mutex> lk(m->mu);
  if (layer < 0 || layer >= m->n_layers)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt2(": layer %lld outside [0, %lld)", layer, m->n_layers));
  if (n_tokens < 0 || max_rows < 0) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": negative size");
  if (n_tokens > 0 && !tokens) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null tokens");
  if (cap < 0 || (cap > 0 && (!col_idx || !pages)))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": cap < 0 or null col_idx/pages");
  const int64_t chunks = std::min<int64_t>(n_tokens / m->B, max_rows);
  // first pass: the cached prefix and its size
  std::vector<Row*> hit;
  std::vector<Key> keys;
  uint64_t h = m->seed;
  int64_t nnz = 0;
  for (int64_t c = 0; c < chunks; ++c) {
    const int32_t* tok = tokens + c * m->B;
    const uint64_t hn = chain(h, tok, m->B);
    auto it = m->rows.find(Key{layer, hn});
    if (it == m->rows.end() || it->second.parent != h ||
        memcmp(it->second.tokens.data(), tok, sizeof(int32_t) * m->B) != 0)
      break;
    hit.push_back(&it->second);
    keys.push_back(Key{layer, hn});
    nnz += (int64_t)it->second.cols.size();
    h = hn;
  }
  if (nnz > cap) {
    *n_rows = (int)hit.size();
    row_ptr[0] = 0;
    return mf::fail(MF_ERR_CAPACITY, std::string(fn) + fmt2(": %lld cached blocks exceed cap %lld", nnz, cap));
  }
  int64_t k = 0;
  row_ptr[0] = 0;
  for (size_t i = 0; i < hit.size(); ++i) {
    Row& r = *hit[i];
    for (size_t j = 0; j < r.cols.size(); ++j, ++k) {
      col_idx[k] = r.cols[j];
      pages[k] = r.pages[j];
    }
    row_ptr[i + 1] = (int32_t)k;
    touch(m, keys[i], r);
    if (r.refs++ == 0) m->lru.erase(r.stamp);
  }
  *n_rows = (int)hit.size();
  m->hits += (int64_t)hit.size();
  m->misses += chunks - (int64_t)hit.size();
  return MF_OK;
}

int mf_bm_release(mf_block_manager* m, int layer, const int32_t* tokens, int64_t n_tokens,
                  int n_rows) {
  const char* fn = "mf_bm_release";
  if (!m) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null manager");
  std::lock_guard<std::mutex> lk(m->mu);
  if (layer < 0 || layer >= m->n_layers)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt2(": layer %lld outside [0, %lld)", layer, m->n_layers));
  if (n_rows < 0 || (int64_t)n_rows * m->B > n_tokens || (n_rows > 0 && !tokens))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": n_rows needs n_rows * B tokens");
  // validate first, then release: all rows must be held
  std::vector<std::pair<Key, Row*>> rs;
  uint64_t h = m->seed;
  for (int c = 0; c < n_rows; ++c) {
    const uint64_t hn = chain(h, tokens + (int64_t)c * m->B, m->B);
    auto it = m->rows.find(Key{layer, hn});
    if (it == m->rows.end() || it->second.refs <= 0)
      return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt2(": row %lld is not held", c));
    rs.emplace_back(Key{layer, hn}, &it->second);
    h = hn;
  }
  for (auto& [key, r] : rs)
    if (--r->refs == 0) m->lru.emplace(r->stamp, key);
  return MF_OK;
}

int mf_bm_insert(mf_block_manager* m, int layer, const int32_t* tokens, int64_t n_tokens,
                 int row0, int n_rows, const int32_t* row_ptr, const int32_t* col_idx,
                 int32_t* pages_out) {
  const char* fn = "mf_bm_insert";
  if (!m || !row_ptr || !pages_out) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  std::lock_guard<std::mutex> lk(m->mu);
  if (layer < 0 || layer >= m->n_layers)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt2(": layer %lld outside [0, %lld)", layer, m->n_layers));
  if (row0 < 0 || n_rows < 0 || ((int64_t)row0 + n_rows) * m->B > n_tokens || (n_tokens > 0 && !tokens))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": rows need (row0 + n_rows) * B tokens (full chunks)");
  const int64_t nnz = row_ptr[n_rows] - row_ptr[0];
  if (row_ptr[0] != 0 || nnz < 0 || (nnz > 0 && !col_idx))
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": row_ptr must start at 0 and be monotone");
  for (int i = 0; i < n_rows; ++i) {
    if (row_ptr[i + 1] < row_ptr[i]) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": row_ptr not monotone");
    for (int32_t k = row_ptr[i]; k < row_ptr[i + 1]; ++k)
      if (col_idx[k] < 0 || col_idx[k] > row0 + i || (k > row_ptr[i] && col_idx[k] <= col_idx[k - 1]))
        return mf::fail(MF_ERR_INVALID, std::string(fn) + ": columns must be ascending and causal");
  }
  // hashes of the rows, and which of them are new
  std::vector<uint64_t> hs(row0 + n_rows + 1);
  hs[0] = m->seed;
  for (int c = 0; c < row0 + n_rows; ++c) hs[c + 1] = chain(hs[c], tokens + (int64_t)c * m->B, m->B);
  // rows already cached under their key are left as they are (their blocks
  // get page -1); a key taken by another prefix (a hash collision) is left
  // alone too, so that prefix's row simply stays uncached
  int64_t need = 0;
  std::vector<bool> fresh(n_rows);
  std::vector<std::pair<Key, Row*>> kept_rows;
  for (int i = 0; i < n_rows; ++i) {
    const Key key{layer, hs[row0 + i + 1]};
    auto it = m->rows.find(key);
    fresh[i] = it == m->rows.end();
    if (fresh[i]) need += row_ptr[i + 1] - row_ptr[i];
    else kept_rows.emplace_back(key, &it->second);
  }
  // the existing rows of the range are used again now: hold them while room is
  // made, so that eviction cannot take them
  for (auto& [key, r] : kept_rows) {
    touch(m, key, *r);
    if (r->refs++ == 0) m->lru.erase(r->stamp);
  }
  const bool room = make_room(m, need);
  for (auto& [key, r] : kept_rows)
    if (--r->refs == 0) m->lru.emplace(r->stamp, key);
  if (!room)
    return mf::fail(MF_ERR_CAPACITY, std::string(fn) + fmt2(": %lld pages needed, %lld free or evictable",
                                                            need, (long long)m->free_pages.size()));
  for (int i = 0; i < n_rows; ++i) {
    const int32_t k0 = row_ptr[i], k1 = row_ptr[i + 1];
    if (!fresh[i]) {
      for (int32_t k = k0; k < k1; ++k) pages_out[k] = -1;   // already cached
      continue;
    }
    const int c = row0 + i;
    Row r;
    r.parent = hs[c];
    r.tokens.assign(tokens + (int64_t)c * m->B, tokens + (int64_t)(c + 1) * m->B);
    r.cols.assign(col_idx + k0, col_idx + k1);
    for (int32_t k = k0; k < k1; ++k) {
      const int32_t p = *m->free_pages.begin();
      m->free_pages.erase(m->free_pages.begin());
      r.pages.push_back(p);
      pages_out[k] = p;
    }
    r.stamp = ++m->clock;
    const Key key{layer, hs[c + 1]};
    m->lru.emplace(r.stamp, key);
    m->rows.emplace(key, std::move(r));
    ++m->inserted;
  }
  return MF_OK;
}

int mf_bm_stats(mf_block_manager* m, int64_t* out) {
  if (!m || !out) return mf::fail(MF_ERR_INVALID, "mf_bm_stats: null pointer");
  std::lock_guard<std::mutex> lk(m->mu);
  int64_t held = 0;
  for (auto& kv : m->rows) held += kv.second.refs > 0;
  out[0] = (int64_t)m->free_pages.size();
  out[1] = (int64_t)m->rows.size();
  out[2] = held;
  out[3] = m->hits;
  out[4] = m->misses;
  out[5] = m->evictions;
  out[6] = m->inserted;
  return MF_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Tile copies into the pool
// ---------------------------------------------------------------------------

namespace {

// pool[pages[k]] = vals[k] for every k with pages[k] in [0, n_pages).
// Workgroup (segment, block k): 64 KB of the tile (4096 pieces of 16 bytes),
// each thread moving 16 pieces; a whole segment issues all 16 loads
// unconditionally before its stores, a partial last segment goes four at a
// time under bounds checks (a tile is H_s * B * B elements, a multiple of 16
// bytes for every supported B and dtype).
constexpr int kSegU4 = 4096;
typedef unsigned pool_u4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void k_pool_store(const pool_u4* __restrict__ vals, int64_t nnzb,
                                                    const int32_t* __restrict__ pages,
                                                    pool_u4* __restrict__ pool, int64_t n_pages,
                                                    int64_t tile_u4) {
  const int64_t seg0 = (int64_t)blockIdx.x * kSegU4;
  for (int64_t k = blockIdx.y; k < nnzb; k += gridDim.y) {
    const int64_t p = pages[k];
    if (p < 0 || p >= n_pages) continue;
    const pool_u4* src = vals + k * tile_u4 + seg0;
    pool_u4* dst = pool + p * tile_u4 + seg0;
    const int64_t n = tile_u4 - seg0 < kSegU4 ? tile_u4 - seg0 : kSegU4;
    if (n == kSegU4) {
      // whole segment: every load unconditional, all 16 in flight at once
      constexpr int kPer = kSegU4 / 256;
      pool_u4 v[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) v[j] = src[threadIdx.x + j * 256];
#pragma unroll
      for (int j = 0; j < kPer; ++j) dst[threadIdx.x + j * 256] = v[j];
      continue;
    }
    for (int64_t i = threadIdx.x; i < n; i += 4 * 256) {
      pool_u4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i + j * 256 < n) v[j] = src[i + j * 256];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (i + j * 256 < n) __builtin_nontemporal_store(v[j], dst + i + j * 256);
    }
  }
}

}  // namespace

extern "C" int mf_pool_store(const void* vals, int64_t nnzb, const int32_t* pages, void* pool,
                             int64_t n_pages, int dtype, int H_s, int B, void* stream) {
  const char* fn = "mf_pool_store";
  if (dtype != MF_F32 && dtype != MF_F16 && dtype != MF_BF16)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt2(": unknown dtype code %lld", dtype));
  if (B != 16 && B != 32 && B != 64 && B != 128)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + fmt2(": B must be 16, 32, 64 or 128 (got %lld)", B));
  if (H_s < 1 || H_s > 64) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": H_s must be in [1, 64]");
  if (nnzb < 0 || n_pages < 0) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": negative size");
  if (nnzb == 0) return MF_OK;
  if (!vals || !pages || !pool) return mf::fail(MF_ERR_INVALID, std::string(fn) + ": null pointer");
  if ((reinterpret_cast<uintptr_t>(vals) | reinterpret_cast<uintptr_t>(pool)) & 15)
    return mf::fail(MF_ERR_INVALID, std::string(fn) + ": vals and pool must be 16-byte aligned");
  const int64_t tile_bytes = (int64_t)H_s * B * B * (dtype == MF_F32 ? 4 : 2);
  const int64_t tile_u4 = tile_bytes / 16;
  const dim3 grid((unsigned)((tile_u4 + kSegU4 - 1) / kSegU4), (unsigned)std::min<int64_t>(nnzb, 65535));
  hipLaunchKernelGGL(k_pool_store, grid, dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<const pool_u4*>(vals), nnzb, pages, reinterpret_cast<pool_u4*>(pool),
                     n_pages, tile_u4);
  return mf::hip_check(hipGetLastError(), "k_pool_store launch");
}
