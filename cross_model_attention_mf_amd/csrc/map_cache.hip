// Prefix cache of compressed maps (MapFlow page, section "让复用真正省时…",
// paragraph "第二": a cache managed by shared prefix, so requests that share
// a prefix share the sender's compressed state for it).
//
// Host side: FNV-1a chained block hashes, an index hash -> (entry, block),
// a first-fit allocator over the caller's device pool, pins and LRU eviction.
// Device side: one gather kernel that copies a table of byte segments (CSR
// row ranges of col_idx and values) in a single launch.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <list>
#include <map>
#include <unordered_map>
#include <vector>

#include "errors.h"
#include "mapflow.h"

using mf::fail;

namespace {

constexpr uint64_t kFnvBasis = 0xcbf29ce484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001b3ull;

inline uint64_t fnv_bytes(uint64_t h, const unsigned char* p, size_t n) {
  for (size_t i = 0; i < n; ++i) {
    h ^= p[i];
    h *= kFnvPrime;
  }
  return h;
}

inline size_t align256(size_t x) { return (x + 255) / 256 * 256; }

struct Segment {
  uint64_t src, dst, bytes;
  uint64_t first;  // index of the segment's first chunk in the launch
};

constexpr uint64_t kChunk = 64 * 1024;  // bytes per workgroup
constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 4;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per 64 KB chunk of the segment list, so a few long value
// ranges still spread over the whole chip.  The chunk's segment is found by
// a binary search over the segments' first-chunk indices (uniform across the
// workgroup).  16-byte copies when source, destination and length allow,
// else 4-byte (col_idx ranges), else bytes; each thread issues its loads
// before its stores.
__global__ void __launch_bounds__(kGatherThreads) gather_segments(const Segment* __restrict__ segs, int nseg) {
  const uint64_t g = blockIdx.x;
  int lo = 0, hi = nseg - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (segs[mid].first <= g) lo = mid;
    else hi = mid - 1;
  }
  const Segment sg = segs[lo];
  const uint64_t off = (g - sg.first) * kChunk;
  if (off >= sg.bytes) return;
  const uint64_t n = sg.bytes - off < kChunk ? sg.bytes - off : kChunk;
  const char* __restrict__ src = reinterpret_cast<const char*>(sg.src) + off;
  char* __restrict__ dst = reinterpret_cast<char*>(sg.dst) + off;
  const int tid = threadIdx.x;
  if (((sg.src | sg.dst | sg.bytes) & 15) == 0) {
    constexpr uint64_t kStep = (uint64_t)kGatherThreads * 16 * kGatherUnroll;
    for (uint64_t base = 0; base < n; base += kStep) {
      u32x4 r[kGatherUnroll];
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const uint64_t o = base + ((uint64_t)u * kGatherThreads + tid) * 16;
        if (o < n) r[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + o));
      }
#pragma unroll
      for (int u = 0; u < kGatherUnroll; ++u) {
        const uint64_t o = base + ((uint64_t)u * kGatherThreads + tid) * 16;
        if (o < n) __builtin_nontemporal_store(r[u], reinterpret_cast<u32x4*>(dst + o));
      }
    }
  } else if (((sg.src | sg.dst | sg.bytes) & 3) == 0) {
    for (uint64_t o = (uint64_t)tid * 4; o < n; o += kGatherThreads * 4)
      *reinterpret_cast<uint32_t*>(dst + o) = *reinterpret_cast<const uint32_t*>(src + o);
  } else {
    for (uint64_t o = tid; o < n; o += kGatherThreads) dst[o] = src[o];
  }
}

struct Entry {
  int32_t nblocks = 0;
  size_t off = 0, bytes = 0;      // allocation in the pool
  size_t val_off = 0;             // values start, relative to off
  std::vector<int32_t> counts;    // [L][H][nblocks] kept blocks per row
  std::vector<int64_t> lh_first;  // [L*H + 1] first entry of each (layer, head)
  std::vector<uint64_t> hashes;
  int32_t pins = 0;
  uint64_t last_use = 0;
};

}  // namespace

struct mf_map_cache {
  mf_map_cache_desc d;
  char* pool = nullptr;
  size_t pool_bytes = 0;
  size_t table_bytes = 0;           // segment table at the start of the pool
  size_t elem = 2;
  std::map<size_t, size_t> free_ranges;  // offset -> size, coalesced
  std::list<Entry> entries;
  // hash of blocks [0, i] -> every entry holding block i (at position i)
  std::unordered_map<uint64_t, std::vector<Entry*>> index;
  uint64_t clock = 0;
  mf_map_cache_stats st{};
  std::vector<Segment> segs;
  std::vector<int32_t> rp;          // a spliced row_ptr, built on the host
  // pinned host staging of the segment table and row_ptr, so the copies to
  // the device are asynchronous; `staged` marks when they have been read
  char* hstage = nullptr;
  size_t hstage_bytes = 0;
  hipEvent_t staged = nullptr;
  bool in_flight = false;

  ~mf_map_cache() {
    if (in_flight) (void)hipEventSynchronize(staged);
    if (staged) (void)hipEventDestroy(staged);
    if (hstage) (void)hipHostFree(hstage);
  }

  bool alloc(size_t bytes, size_t* off) {
    for (auto it = free_ranges.begin(); it != free_ranges.end(); ++it) {
      if (it->second >= bytes) {
        *off = it->first;
        const size_t rest = it->second - bytes;
        const size_t next = it->first + bytes;
        free_ranges.erase(it);
        if (rest) free_ranges[next] = rest;
        return true;
      }
    }
    return false;
  }
  void release_range(size_t off, size_t bytes) {
    auto it = free_ranges.emplace(off, bytes).first;
    auto nx = std::next(it);
    if (nx != free_ranges.end() && it->first + it->second == nx->first) {
      it->second += nx->second;
      free_ranges.erase(nx);
    }
    if (it != free_ranges.begin()) {
      auto pv = std::prev(it);
      if (pv->first + pv->second == it->first) {
        pv->second += it->second;
        free_ranges.erase(it);
      }
    }
  }
  void evict(std::list<Entry>::iterator e) {
    for (uint64_t h : e->hashes) {
      auto f = index.find(h);
      if (f == index.end()) continue;
      auto& v = f->second;
      for (size_t i = 0; i < v.size(); ++i)
        if (v[i] == &*e) {
          v.erase(v.begin() + i);
          break;
        }
      if (v.empty()) index.erase(f);
    }
    release_range(e->off, e->bytes);
    st.bytes_used -= (int64_t)e->bytes;
    st.entries -= 1;
    st.evictions += 1;
    entries.erase(e);
  }
  // least recently used unpinned entry, or end()
  std::list<Entry>::iterator victim() {
    auto best = entries.end();
    for (auto it = entries.begin(); it != entries.end(); ++it)
      if (it->pins == 0 && (best == entries.end() || it->last_use < best->last_use)) best = it;
    return best;
  }
  // an entry holding blocks [0, m) of this chain, a pinned one if any
  Entry* holder(const uint64_t* hashes, int32_t m, bool want_pinned = false) {
    if (m < 1) return nullptr;
    auto f = index.find(hashes[m - 1]);
    if (f == index.end()) return nullptr;
    Entry* any = nullptr;
    for (Entry* e : f->second) {
      if (e->nblocks < m || e->hashes[m - 1] != hashes[m - 1]) continue;
      if (!want_pinned || e->pins > 0) return e;
      if (!any) any = e;
    }
    return want_pinned ? nullptr : any;
  }
  // The staging area may be rewritten once the previous call's host-to-device
  // copies have read it.
  mf_status stage_room(size_t need, const char* fn) {
    hipError_t e = hipSuccess;
    if (in_flight) {
      e = hipEventSynchronize(staged);
      in_flight = false;
    }
    if (e == hipSuccess && !staged) e = hipEventCreateWithFlags(&staged, hipEventDisableTiming);
    if (e == hipSuccess && need > hstage_bytes) {
      const size_t want = need > 2 * hstage_bytes ? need : 2 * hstage_bytes;
      if (hstage) e = hipHostFree(hstage);
      hstage = nullptr;
      hstage_bytes = 0;
      if (e == hipSuccess) e = hipHostMalloc((void**)&hstage, want, hipHostMallocDefault);
      if (e == hipSuccess) hstage_bytes = want;
    }
    if (e != hipSuccess) return fail(MF_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    return MF_OK;
  }
  // Stream-ordered: the segment table (and a row_ptr for rp_dst) go through
  // the pinned staging area to the device, then one gather launch copies
  // every segment.  Nothing waits for the device.
  mf_status run_segments(void* stream, const char* fn, int32_t* rp_dst = nullptr) {
    const size_t bytes = segs.size() * sizeof(Segment);
    if (bytes > table_bytes) return fail(MF_ERR_UNSUPPORTED, "%s: %zu copy segments exceed the table", fn, segs.size());
    uint64_t chunks = 0;
    for (Segment& sg : segs) {
      sg.first = chunks;
      chunks += (sg.bytes + kChunk - 1) / kChunk;
    }
    if (chunks > 0x7fffffffull) return fail(MF_ERR_UNSUPPORTED, "%s: %llu bytes to copy in one call", fn,
                                            (unsigned long long)(chunks * kChunk));
    const size_t rp_bytes = rp_dst ? rp.size() * sizeof(int32_t) : 0;
    const size_t rp_off = align256(bytes);
    if (chunks == 0 && rp_bytes == 0) return MF_OK;
    mf_status st = stage_room(rp_off + rp_bytes, fn);
    if (st) return st;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    if (chunks) {
      memcpy(hstage, segs.data(), bytes);
      e = hipMemcpyAsync(pool, hstage, bytes, hipMemcpyHostToDevice, s);
    }
    if (e == hipSuccess && rp_bytes) {
      memcpy(hstage + rp_off, rp.data(), rp_bytes);
      e = hipMemcpyAsync(rp_dst, hstage + rp_off, rp_bytes, hipMemcpyHostToDevice, s);
    }
    if (e == hipSuccess) e = hipEventRecord(staged, s);
    if (e == hipSuccess) in_flight = true;
    if (e == hipSuccess && chunks) {
      hipLaunchKernelGGL(gather_segments, dim3((unsigned)chunks), dim3(kGatherThreads), 0, s,
                         reinterpret_cast<const Segment*>(pool), (int)segs.size());
      e = hipGetLastError();
    }
    if (e != hipSuccess) return fail(MF_ERR_HIP, "%s: %s", fn, hipGetErrorString(e));
    return MF_OK;
  }
};

extern "C" {

int64_t mf_prefix_block_hashes(const int32_t* tokens, int64_t n_tokens, int32_t B, uint64_t parent,
                               uint64_t* hashes_out) {
  if (!tokens || !hashes_out || n_tokens < 0 || B < 1) return -1;
  const int64_t nb = n_tokens / B;
  uint64_t h = parent;
  for (int64_t i = 0; i < nb; ++i) {
    unsigned char buf[8];
    for (int k = 0; k < 8; ++k) buf[k] = (unsigned char)(h >> (8 * k));
    uint64_t x = fnv_bytes(kFnvBasis, buf, 8);
    for (int32_t t = 0; t < B; ++t) {
      const uint32_t v = (uint32_t)tokens[i * B + t];
      unsigned char tb[4] = {(unsigned char)v, (unsigned char)(v >> 8), (unsigned char)(v >> 16),
                             (unsigned char)(v >> 24)};
      x = fnv_bytes(x, tb, 4);
    }
    hashes_out[i] = h = x;
  }
  return nb;
}

mf_status mf_map_cache_create(const mf_map_cache_desc* desc, void* pool, size_t pool_bytes, mf_map_cache** out) {
  mf::clear_error();
  const char* fn = "mf_map_cache_create";
  if (!desc || !pool || !out) return fail(MF_ERR_INVALID, "%s: NULL argument", fn);
  if (desc->dtype != MF_F32 && desc->dtype != MF_BF16) return fail(MF_ERR_INVALID, "%s: unknown dtype", fn);
  if (desc->num_layers < 1 || desc->num_layers > MF_MAX_LAYERS || desc->H_s < 1 || desc->H_s > 64 || desc->B < 1)
    return fail(MF_ERR_INVALID, "%s: num_layers, H_s or B out of range", fn);
  if ((uintptr_t)pool % 256) return fail(MF_ERR_INVALID, "%s: pool is not 256-byte aligned", fn);
  const size_t table = align256((size_t)4 * desc->num_layers * desc->H_s * sizeof(Segment));
  if (pool_bytes <= table) return fail(MF_ERR_CAPACITY, "%s: pool of %zu bytes holds no entry", fn, pool_bytes);
  mf_map_cache* c = new mf_map_cache();
  c->d = *desc;
  c->pool = static_cast<char*>(pool);
  c->pool_bytes = pool_bytes;
  c->table_bytes = table;
  c->elem = desc->dtype == MF_BF16 ? 2 : 4;
  const size_t usable = (pool_bytes - table) / 256 * 256;
  c->free_ranges[table] = usable;
  c->st.bytes_capacity = (int64_t)usable;
  *out = c;
  return MF_OK;
}

void mf_map_cache_destroy(mf_map_cache* cache) { delete cache; }

mf_status mf_map_cache_insert(mf_map_cache* c, const uint64_t* hashes, int32_t n_blocks, const int32_t* row_ptr_host,
                              int32_t total_rb, int32_t rb_first, const int32_t* col_idx, const void* values,
                              void* stream) {
  mf::clear_error();
  const char* fn = "mf_map_cache_insert";
  if (!c || !hashes || !row_ptr_host) return fail(MF_ERR_INVALID, "%s: NULL argument", fn);
  if (n_blocks < 1 || rb_first < 0 || total_rb < 1 || rb_first + n_blocks > total_rb)
    return fail(MF_ERR_INVALID, "%s: rows [%d, %d) outside %d row-blocks", fn, rb_first, rb_first + n_blocks, total_rb);
  if (Entry* held = c->holder(hashes, n_blocks)) {
    held->last_use = ++c->clock;
    return MF_OK;
  }
  const int L = c->d.num_layers, H = c->d.H_s, B = c->d.B;
  Entry e;
  e.nblocks = n_blocks;
  e.counts.resize((size_t)L * H * n_blocks);
  e.lh_first.resize((size_t)L * H + 1);
  int64_t total = 0;
  for (int lh = 0; lh < L * H; ++lh) {
    e.lh_first[lh] = total;
    const int64_t row0 = (int64_t)lh * total_rb + rb_first;
    for (int i = 0; i < n_blocks; ++i) {
      const int32_t n = row_ptr_host[row0 + i + 1] - row_ptr_host[row0 + i];
      if (n < 0) return fail(MF_ERR_INVALID, "%s: row_ptr decreases at row %lld", fn, (long long)(row0 + i));
      e.counts[(size_t)lh * n_blocks + i] = n;
      total += n;
    }
  }
  e.lh_first[(size_t)L * H] = total;
  if (total > 0 && (!col_idx || !values)) return fail(MF_ERR_INVALID, "%s: col_idx or values is NULL", fn);
  const size_t vbytes_per = (size_t)B * B * c->elem;
  e.val_off = align256((size_t)total * 4);
  e.bytes = align256(e.val_off + (size_t)total * vbytes_per);
  if (e.bytes == 0) e.bytes = 256;
  while (!c->alloc(e.bytes, &e.off)) {
    auto v = c->victim();
    if (v == c->entries.end())
      return fail(MF_ERR_CAPACITY, "%s: %zu bytes do not fit beside the pinned entries", fn, e.bytes);
    c->evict(v);
  }
  // copy every (layer, head)'s rows: one col_idx and one values segment each
  c->segs.clear();
  char* base = c->pool + e.off;
  for (int lh = 0; lh < L * H; ++lh) {
    const int64_t row0 = (int64_t)lh * total_rb + rb_first;
    const int64_t src0 = row_ptr_host[row0];
    const int64_t n = e.lh_first[lh + 1] - e.lh_first[lh];
    if (n == 0) continue;
    c->segs.push_back({(uint64_t)(uintptr_t)(col_idx + src0), (uint64_t)(uintptr_t)(base + e.lh_first[lh] * 4),
                       (uint64_t)n * 4});
    c->segs.push_back({(uint64_t)(uintptr_t)(static_cast<const char*>(values) + src0 * vbytes_per),
                       (uint64_t)(uintptr_t)(base + e.val_off + e.lh_first[lh] * vbytes_per), (uint64_t)n * vbytes_per});
  }
  mf_status s = c->run_segments(stream, fn);
  if (s) {
    c->release_range(e.off, e.bytes);
    return s;
  }
  e.hashes.assign(hashes, hashes + n_blocks);
  e.last_use = ++c->clock;
  c->entries.push_back(std::move(e));
  Entry* ep = &c->entries.back();
  for (int32_t i = 0; i < n_blocks; ++i) c->index[hashes[i]].push_back(ep);
  c->st.entries += 1;
  c->st.bytes_used += (int64_t)ep->bytes;
  return MF_OK;
}

int32_t mf_map_cache_lookup(mf_map_cache* c, const uint64_t* hashes, int32_t n) {
  if (!c || !hashes || n < 1) return 0;
  int32_t m = 0;
  for (int32_t i = n; i >= 1; --i) {
    if (c->holder(hashes, i)) {
      m = i;
      break;
    }
  }
  c->st.blocks_hit += m;
  c->st.blocks_missed += n - m;
  if (m > 0) {
    Entry* e = c->holder(hashes, m);
    if (e->pins++ == 0) c->st.pinned_entries += 1;
    e->last_use = ++c->clock;
  }
  return m;
}

void mf_map_cache_release(mf_map_cache* c, const uint64_t* hashes, int32_t m) {
  if (!c || !hashes || m < 1) return;
  Entry* e = c->holder(hashes, m, true);
  if (e && --e->pins == 0) c->st.pinned_entries -= 1;
}

mf_status mf_map_cache_splice(mf_map_cache* c, const uint64_t* hashes, int32_t m, int32_t n_blocks,
                              const int32_t* suffix_row_ptr_host, int32_t suffix_total_rb, int32_t suffix_rb_first,
                              const int32_t* suffix_col_idx, const void* suffix_values, int32_t* row_ptr_out,
                              int32_t* col_idx_out, void* values_out, int64_t capacity_blocks, int64_t* nnz_out,
                              void* stream) {
  mf::clear_error();
  const char* fn = "mf_map_cache_splice";
  if (!c || !nnz_out || !row_ptr_out) return fail(MF_ERR_INVALID, "%s: NULL argument", fn);
  if (m < 0 || n_blocks < 1 || m > n_blocks) return fail(MF_ERR_INVALID, "%s: m = %d, n_blocks = %d", fn, m, n_blocks);
  if (m > 0 && !hashes) return fail(MF_ERR_INVALID, "%s: hashes is NULL", fn);
  const int32_t ns = n_blocks - m;   // suffix row-blocks
  if (ns > 0 && (!suffix_row_ptr_host || suffix_rb_first < 0 || suffix_rb_first + ns > suffix_total_rb))
    return fail(MF_ERR_INVALID, "%s: suffix rows outside its CSR", fn);
  Entry* e = m > 0 ? c->holder(hashes, m, true) : nullptr;
  if (m > 0 && !e) return fail(MF_ERR_INVALID, "%s: the first %d blocks are not pinned in the cache", fn, m);
  const int L = c->d.num_layers, H = c->d.H_s, B = c->d.B;
  const size_t vbytes_per = (size_t)B * B * c->elem;
  // row_ptr of the spliced CSR
  c->rp.assign((size_t)L * H * n_blocks + 1, 0);
  int64_t total = 0;
  for (int lh = 0; lh < L * H; ++lh) {
    for (int32_t i = 0; i < n_blocks; ++i) {
      int64_t n;
      if (i < m) {
        n = e->counts[(size_t)lh * e->nblocks + i];
      } else {
        const int64_t r = (int64_t)lh * suffix_total_rb + suffix_rb_first + (i - m);
        n = suffix_row_ptr_host[r + 1] - suffix_row_ptr_host[r];
        if (n < 0) return fail(MF_ERR_INVALID, "%s: suffix row_ptr decreases", fn);
      }
      c->rp[(size_t)lh * n_blocks + i] = (int32_t)total;
      total += n;
    }
  }
  c->rp[(size_t)L * H * n_blocks] = (int32_t)total;
  *nnz_out = total;
  if (total > capacity_blocks) return fail(MF_ERR_CAPACITY, "%s: %lld entries > capacity %lld", fn, (long long)total,
                                           (long long)capacity_blocks);
  if (total > 0 && (!col_idx_out || !values_out)) return fail(MF_ERR_INVALID, "%s: output col_idx or values is NULL", fn);
  c->segs.clear();
  for (int lh = 0; lh < L * H; ++lh) {
    const int64_t dst0 = c->rp[(size_t)lh * n_blocks];
    int64_t ncache = 0;
    if (m > 0) {
      ncache = (int64_t)c->rp[(size_t)lh * n_blocks + m] - dst0;
      if (ncache > 0) {
        const char* base = c->pool + e->off;
        const int64_t s0 = e->lh_first[lh];
        c->segs.push_back({(uint64_t)(uintptr_t)(base + s0 * 4), (uint64_t)(uintptr_t)(col_idx_out + dst0),
                           (uint64_t)ncache * 4});
        c->segs.push_back({(uint64_t)(uintptr_t)(base + e->val_off + s0 * vbytes_per),
                           (uint64_t)(uintptr_t)(static_cast<char*>(values_out) + dst0 * vbytes_per),
                           (uint64_t)ncache * vbytes_per});
      }
    }
    if (ns > 0) {
      const int64_t r0 = (int64_t)lh * suffix_total_rb + suffix_rb_first;
      const int64_t src0 = suffix_row_ptr_host[r0];
      const int64_t nsuf = suffix_row_ptr_host[r0 + ns] - src0;
      if (nsuf > 0) {
        if (!suffix_col_idx || !suffix_values) return fail(MF_ERR_INVALID, "%s: suffix col_idx or values is NULL", fn);
        c->segs.push_back({(uint64_t)(uintptr_t)(suffix_col_idx + src0),
                           (uint64_t)(uintptr_t)(col_idx_out + dst0 + ncache), (uint64_t)nsuf * 4});
        c->segs.push_back({(uint64_t)(uintptr_t)(static_cast<const char*>(suffix_values) + src0 * vbytes_per),
                           (uint64_t)(uintptr_t)(static_cast<char*>(values_out) + (dst0 + ncache) * vbytes_per),
                           (uint64_t)nsuf * vbytes_per});
      }
    }
  }
  if (e) e->last_use = ++c->clock;
  return c->run_segments(stream, fn, row_ptr_out);
}

mf_status mf_map_cache_get_stats(const mf_map_cache* c, mf_map_cache_stats* out) {
  if (!c || !out) return fail(MF_ERR_INVALID, "mf_map_cache_get_stats: NULL argument");
  *out = c->st;
  return MF_OK;
}

}  // extern "C"
