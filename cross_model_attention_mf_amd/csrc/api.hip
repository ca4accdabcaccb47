// C-ABI entry points: validate every argument on the host, then launch the
// gfx950 kernels on the caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>

#include <atomic>
#include <mutex>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "errors.h"
#include "internal.h"
#include "mapflow.h"

using mf::fail;

namespace mf {

static std::atomic<uint32_t> g_forced_portable{0};

uint32_t forced_portable() { return g_forced_portable.load(std::memory_order_relaxed); }

}  // namespace mf

namespace {

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

mf_status hip_fail(int err, const char* what) {
  return fail(MF_ERR_HIP, "%s: %s", what, hipGetErrorString((hipError_t)err));
}

mf_status check_batch(const mf_batch* b, int B, const char* fn) {
  if (!b) return fail(MF_ERR_INVALID, "%s: batch is NULL", fn);
  const mf_plan_info& in = b->info;
  if (in.block != B) return fail(MF_ERR_INVALID, "%s: batch planned for B = %d, call uses B = %d", fn, in.block, B);
  if (in.num_seqs < 0 || in.total_rowblocks < 0 || in.max_colblocks < 0 || in.total_q < 0 || in.total_k < 0)
    return fail(MF_ERR_INVALID, "%s: negative size in batch info", fn);
  if (in.plan_len != in.num_seqs + 1 + in.total_rowblocks)
    return fail(MF_ERR_INVALID, "%s: batch info is inconsistent (plan_len)", fn);
  if (in.max_k_len > MF_MAX_KEYS) return fail(MF_ERR_UNSUPPORTED, "%s: %d keys > MF_MAX_KEYS", fn, in.max_k_len);
  if (in.total_rowblocks > 0 && (!b->cu_seqlens_q || !b->cu_seqlens_k || !b->plan))
    return fail(MF_ERR_INVALID, "%s: batch device arrays are NULL", fn);
  return MF_OK;
}

mf_status check_common(mf_dtype dt, int L, int H, int Hkv, int d, int B, const char* fn) {
  if (dt != MF_F32 && dt != MF_BF16) return fail(MF_ERR_INVALID, "%s: unknown dtype %d", fn, (int)dt);
  if (L < 0) return fail(MF_ERR_INVALID, "%s: num_layers = %d < 0", fn, L);
  if (B != 32 && B != 64 && B != 128) return fail(MF_ERR_UNSUPPORTED, "%s: B = %d not in {32, 64, 128}", fn, B);
  if (d != 64 && d != 128) return fail(MF_ERR_UNSUPPORTED, "%s: d = %d not in {64, 128}", fn, d);
  if (H < 1 || H > 64) return fail(MF_ERR_UNSUPPORTED, "%s: %d heads not in [1, 64]", fn, H);
  if (Hkv < 1 || H % Hkv) return fail(MF_ERR_INVALID, "%s: %d kv heads do not divide %d heads", fn, Hkv, H);
  return MF_OK;
}

mf_status check_sender(const mf_sender_desc* s, const mf_batch* b, const char* fn) {
  if (!s) return fail(MF_ERR_INVALID, "%s: desc is NULL", fn);
  mf_status st = check_common(s->dtype, s->num_layers, s->H_s, s->H_kv_s, s->d, s->B, fn);
  if (st) return st;
  st = check_batch(b, s->B, fn);
  if (st) return st;
  if (!(s->sm_scale >= 0.f) || isinf(s->sm_scale)) return fail(MF_ERR_INVALID, "%s: sm_scale must be finite and >= 0", fn);
  if (s->num_layers > 1) {
    if (s->layer_stride_q < (int64_t)b->info.total_q * s->H_s * s->d ||
        s->layer_stride_k < (int64_t)b->info.total_k * s->H_kv_s * s->d)
      return fail(MF_ERR_INVALID, "%s: layer strides smaller than one layer", fn);
  }
  return MF_OK;
}

mf::BatchArgs batch_args(const mf_batch* b) {
  mf::BatchArgs a;
  a.cu_q = b->cu_seqlens_q;
  a.cu_k = b->cu_seqlens_k;
  a.q_pos0 = b->q_pos0;
  a.plan = b->plan;
  a.num_seqs = b->info.num_seqs;
  a.total_rb = b->info.total_rowblocks;
  a.max_cb = b->info.max_colblocks;
  a.total_q = b->info.total_q;
  a.total_k = b->info.total_k;
  return a;
}

double scale_of(const mf_sender_desc* s) { return s->sm_scale > 0.f ? (double)s->sm_scale : 1.0 / sqrt((double)s->d); }

size_t device_lds_limit() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 65536;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return 65536;
  return (size_t)v;
}

struct WorkspaceLayout {
  size_t counts, bits, total, bytes;
  int words;
};

WorkspaceLayout workspace_layout(const mf_sender_desc* s, const mf_batch* b) {
  WorkspaceLayout w;
  const size_t nrows = (size_t)s->num_layers * s->H_s * b->info.total_rowblocks;
  w.words = (b->info.max_colblocks + 31) / 32;
  w.counts = 0;
  w.bits = align256(nrows * 4);
  w.total = w.bits + align256(nrows * (size_t)w.words * 4);
  w.bytes = w.total + 256;
  return w;
}

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  return n;
}

}  // namespace

extern "C" {

const char* mf_status_string(mf_status s) {
  switch (s) {
    case MF_OK: return "MF_OK";
    case MF_ERR_INVALID: return "MF_ERR_INVALID";
    case MF_ERR_UNSUPPORTED: return "MF_ERR_UNSUPPORTED";
    case MF_ERR_CAPACITY: return "MF_ERR_CAPACITY";
    case MF_ERR_HIP: return "MF_ERR_HIP";
    case MF_ERR_WORKSPACE: return "MF_ERR_WORKSPACE";
  }
  return "MF_ERR_UNKNOWN";
}

const char* mf_last_error_message(void) { return mf::error_buffer(); }

const char* mf_version(void) { return "mapflow-mi355x 0.2"; }

mf_status mf_mfma_probe(float* out, int nblocks, int iters, int with_vector, void* stream) {
  mf::clear_error();
  if (!out || nblocks < 1 || iters < 1) return fail(MF_ERR_INVALID, "mf_mfma_probe: out NULL or nblocks, iters < 1");
  const int e = mf::launch_mfma_probe(out, nblocks, iters, with_vector != 0, stream);
  return e ? hip_fail(e, "mf_mfma_probe") : MF_OK;
}

uint32_t mf_debug_force_portable(uint32_t mask) {
  const uint32_t all = MF_FORCE_PORTABLE_STATS | MF_FORCE_PORTABLE_SELECT | MF_FORCE_PORTABLE_EXTRACT |
                       MF_FORCE_PORTABLE_MAPPED;
  return mf::g_forced_portable.exchange(mask & all);
}

size_t mf_block_stats_workspace_size(const mf_sender_desc* desc, const mf_batch* batch) {
  if (!desc || !batch) return 0;
  if (!mf::stats_fast_path(desc->dtype, desc->B, desc->d)) return 0;
  const int cus = device_cu_count();
  if (cus <= 0) return 0;
  return mf::stats_workspace_layout(desc->B, batch->info.max_colblocks, batch->info.total_rowblocks,
                                    mf::stats_slots(cus)).bytes;
}

mf_status mf_block_stats(const mf_sender_desc* desc, const mf_batch* batch, const void* q, const void* k,
                         float* row_lse, float* block_mass, void* workspace, size_t workspace_bytes,
                         void* stream) {
  mf::clear_error();
  const char* fn = "mf_block_stats";
  mf_status st = check_sender(desc, batch, fn);
  if (st) return st;
  if (desc->num_layers == 0 || batch->info.total_rowblocks == 0) return MF_OK;
  if (!q || !k || !row_lse || !block_mass) return fail(MF_ERR_INVALID, "%s: a tensor pointer is NULL", fn);
  mf::StatsArgs a;
  a.b = batch_args(batch);
  a.q = q; a.k = k; a.row_lse = row_lse; a.block_mass = block_mass;
  a.lsq = desc->layer_stride_q; a.lsk = desc->layer_stride_k;
  a.L = desc->num_layers; a.H = desc->H_s; a.Hkv = desc->H_kv_s; a.d = desc->d; a.B = desc->B;
  a.scale = scale_of(desc);
  a.ws = nullptr;
  if (mf::stats_fast_path(desc->dtype, desc->B, desc->d)) {
    const int cus = device_cu_count();
    if (cus <= 0) return fail(MF_ERR_HIP, "%s: cannot query the device's compute units", fn);
    a.wsl = mf::stats_workspace_layout(desc->B, batch->info.max_colblocks, batch->info.total_rowblocks,
                                       mf::stats_slots(cus));
    if (!workspace || workspace_bytes < a.wsl.bytes)
      return fail(MF_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, a.wsl.bytes, workspace_bytes);
    a.ws = workspace;
  } else {
    const size_t lds = mf::block_stats_lds_bytes(desc->B, batch->info.max_colblocks);
    if (lds > device_lds_limit())
      return fail(MF_ERR_UNSUPPORTED, "%s: %zu bytes of LDS needed, device allows %zu", fn, lds, device_lds_limit());
  }
  const int e = mf::launch_block_stats(a, desc->dtype, stream);
  return e ? hip_fail(e, fn) : MF_OK;
}

size_t mf_compress_workspace_size(const mf_sender_desc* desc, const mf_batch* batch) {
  if (!desc || !batch) return 0;
  return workspace_layout(desc, batch).bytes;
}

}  // extern "C"

namespace {

mf_status compress_impl(const mf_sender_desc* desc, const mf_batch* batch, const void* q, const void* k,
                        const float* row_lse, const float* block_mass, float tau, int32_t* row_ptr,
                        int32_t* col_idx, void* values, int64_t capacity_blocks, int64_t* nnz_out,
                        void* workspace, size_t workspace_bytes, void* stream, const char* fn) {
  mf_status st = check_sender(desc, batch, fn);
  if (st) return st;
  if (!(tau > 0.f && tau <= 1.f)) return fail(MF_ERR_INVALID, "%s: tau = %g not in (0, 1]", fn, (double)tau);
  if (capacity_blocks < 0) return fail(MF_ERR_INVALID, "%s: capacity_blocks < 0", fn);
  if (!row_ptr) return fail(MF_ERR_INVALID, "%s: row_ptr is NULL", fn);
  if (capacity_blocks > 0 && !col_idx) return fail(MF_ERR_INVALID, "%s: col_idx is NULL", fn);
  const int64_t nrows = (int64_t)desc->num_layers * desc->H_s * batch->info.total_rowblocks;
  if (nrows > INT32_MAX - 1) return fail(MF_ERR_UNSUPPORTED, "%s: too many CSR rows", fn);
  if (nrows > 0 && (!q || !k || !row_lse || !block_mass)) return fail(MF_ERR_INVALID, "%s: a tensor pointer is NULL", fn);
  const WorkspaceLayout wl = workspace_layout(desc, batch);
  if (!workspace || workspace_bytes < wl.bytes)
    return fail(MF_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, wl.bytes, workspace_bytes);
  if (mf::select_lds_bytes(batch->info.max_colblocks) > device_lds_limit())
    return fail(MF_ERR_UNSUPPORTED, "%s: too many column blocks for the selection sort", fn);
  char* ws = static_cast<char*>(workspace);
  int32_t* counts = reinterpret_cast<int32_t*>(ws + wl.counts);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + wl.bits);
  long long* total = reinterpret_cast<long long*>(ws + wl.total);
  const mf::BatchArgs ba = batch_args(batch);

  if (nrows > 0) {
    mf::SelectArgs s;
    s.b = ba; s.block_mass = block_mass; s.counts = counts; s.keep_bits = bits; s.words = wl.words;
    s.L = desc->num_layers; s.H = desc->H_s; s.B = desc->B; s.tau = (double)tau;
    int e = mf::launch_select(s, stream);
    if (e) return hip_fail(e, fn);
  }
  mf::ScanArgs sc;
  sc.counts = counts; sc.row_ptr = row_ptr; sc.total = total; sc.n = nrows;
  int e = mf::launch_scan(sc, stream);
  if (e) return hip_fail(e, fn);
  if (nnz_out) {
    long long nnz = 0;
    e = (int)hipMemcpyAsync(&nnz, total, sizeof(nnz), hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (!e) e = (int)hipStreamSynchronize((hipStream_t)stream);
    if (e) return hip_fail(e, fn);
    *nnz_out = nnz;
    if (capacity_blocks == 0 && !col_idx) return MF_OK;  // count only
    if (nnz > capacity_blocks)
      return fail(MF_ERR_CAPACITY, "%s: %lld kept blocks exceed capacity %lld", fn, nnz, (long long)capacity_blocks);
  }
  if (nrows == 0 || capacity_blocks == 0) return MF_OK;
  mf::ExtractArgs x;
  x.b = ba; x.q = q; x.k = k; x.row_lse = row_lse; x.row_ptr = row_ptr; x.keep_bits = bits; x.words = wl.words;
  x.col_idx = col_idx; x.values = values; x.capacity = capacity_blocks;
  x.lsq = desc->layer_stride_q; x.lsk = desc->layer_stride_k;
  x.L = desc->num_layers; x.H = desc->H_s; x.Hkv = desc->H_kv_s; x.d = desc->d; x.B = desc->B;
  x.scale = scale_of(desc);
  e = mf::launch_extract(x, desc->dtype, stream);
  return e ? hip_fail(e, fn) : MF_OK;
}

// The no-allocation variant's scratch: one array per device, holding the
// selection's per-row counts and keep bits and the scan's total.  Host code
// reaches it only through the address hipGetSymbolAddress returns on each
// device (the array's name is a host-side stand-in).
constexpr size_t kStaticScratchBytes = (size_t)MF_STATIC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// the scratch's device address on the current device (set up once per device)
mf_status static_scratch(void** out, const char* fn) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail((int)e, fn);
  if (dev < 0 || dev >= kMaxDevices) return fail(MF_ERR_UNSUPPORTED, "%s: device %d beyond %d", fn, dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol, fn);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MF_OK;
}

}  // namespace

extern "C" {

mf_status mf_compress_blocks(const mf_sender_desc* desc, const mf_batch* batch, const void* q, const void* k,
                             const float* row_lse, const float* block_mass, float tau, int32_t* row_ptr,
                             int32_t* col_idx, void* values, int64_t capacity_blocks, int64_t* nnz_out,
                             void* workspace, size_t workspace_bytes, void* stream) {
  mf::clear_error();
  return compress_impl(desc, batch, q, k, row_lse, block_mass, tau, row_ptr, col_idx, values, capacity_blocks,
                       nnz_out, workspace, workspace_bytes, stream, "mf_compress_blocks");
}

mf_status mf_compress_blocks_noalloc(const mf_sender_desc* desc, const mf_batch* batch, const void* q,
                                     const void* k, const float* row_lse, const float* block_mass, float tau,
                                     int32_t* row_ptr, int32_t* col_idx, void* values, int64_t capacity_blocks,
                                     int64_t* nnz_out, void* stream) {
  mf::clear_error();
  const char* fn = "mf_compress_blocks_noalloc";
  mf_status st = check_sender(desc, batch, fn);
  if (st) return st;
  const size_t need = workspace_layout(desc, batch).bytes;
  if (need > kStaticScratchBytes)
    return fail(MF_ERR_WORKSPACE, "%s: needs %zu bytes of scratch, the static scratch holds %zu", fn, need,
                kStaticScratchBytes);
  void* ws = nullptr;
  st = static_scratch(&ws, fn);
  if (st) return st;
  return compress_impl(desc, batch, q, k, row_lse, block_mass, tau, row_ptr, col_idx, values, capacity_blocks,
                       nnz_out, ws, kStaticScratchBytes, stream, fn);
}

}  // extern "C"

namespace {

// Validation of one receiver descriptor and its tensors (MF_OK when the call
// has work or is an empty no-op; *empty tells which).
mf_status check_receiver(const mf_receiver_desc* desc, const mf_batch* batch, const int32_t* row_ptr,
                         const int32_t* col_idx, const void* values, const float* W, const void* v, void* o,
                         const char* fn, bool* empty) {
  *empty = false;
  if (!desc) return fail(MF_ERR_INVALID, "%s: desc is NULL", fn);
  mf_status st = check_common(desc->dtype, desc->num_layers, desc->H_r, desc->H_kv_r, desc->d, desc->B, fn);
  if (st) return st;
  st = check_batch(batch, desc->B, fn);
  if (st) return st;
  if (desc->H_s < 1 || desc->H_s > 64) return fail(MF_ERR_UNSUPPORTED, "%s: H_s = %d not in [1, 64]", fn, desc->H_s);
  if (desc->num_layers > MF_MAX_LAYERS) return fail(MF_ERR_UNSUPPORTED, "%s: more than %d layers", fn, MF_MAX_LAYERS);
  if (desc->sender_layers < 1 && desc->num_layers > 0) return fail(MF_ERR_INVALID, "%s: sender_layers < 1", fn);
  if (desc->num_layers > 0 && !desc->layer_map) return fail(MF_ERR_INVALID, "%s: layer_map is NULL", fn);
  for (int l = 0; l < desc->num_layers; ++l)
    if (desc->layer_map[l] < 0 || desc->layer_map[l] >= desc->sender_layers)
      return fail(MF_ERR_INVALID, "%s: layer_map[%d] = %d outside [0, %d)", fn, l, desc->layer_map[l], desc->sender_layers);
  if (desc->block_table) {
    if (desc->page_size < 1 || desc->max_pages < 1 || desc->num_pages < 1)
      return fail(MF_ERR_INVALID, "%s: paged values need page_size, max_pages, num_pages >= 1", fn);
    if ((int64_t)desc->max_pages * desc->page_size < batch->info.max_k_len)
      return fail(MF_ERR_INVALID, "%s: max_pages * page_size < longest key range", fn);
  }
  if (desc->num_layers > 1) {
    const int64_t vrows = desc->block_table ? desc->num_pages * desc->page_size : (int64_t)batch->info.total_k;
    if (desc->layer_stride_v < vrows * desc->H_kv_r * desc->d ||
        desc->layer_stride_o < (int64_t)batch->info.total_q * desc->H_r * desc->d)
      return fail(MF_ERR_INVALID, "%s: layer strides smaller than one layer", fn);
  }
  if (desc->csr_capacity < 0) return fail(MF_ERR_INVALID, "%s: csr_capacity < 0", fn);
  if (desc->num_layers == 0 || batch->info.total_rowblocks == 0) {
    *empty = true;
    return MF_OK;
  }
  if (!row_ptr || !W || !v || !o || (desc->csr_capacity > 0 && (!col_idx || !values)))
    return fail(MF_ERR_INVALID, "%s: a tensor pointer is NULL", fn);
  return MF_OK;
}

mf::MappedRecv receiver_args(const mf_receiver_desc* desc, const mf_batch* batch, const float* W, const void* v,
                             void* o, int group0) {
  mf::MappedRecv r;
  memset(&r, 0, sizeof(r));
  r.W = W; r.v = v; r.o = o;
  r.lsv = desc->layer_stride_v; r.lso = desc->layer_stride_o;
  r.block_table = desc->block_table; r.page_size = desc->page_size; r.max_pages = desc->max_pages;
  r.num_pages = desc->num_pages;
  r.Hr = desc->H_r; r.Hkv = desc->H_kv_r;
  r.group0 = group0;
  r.vrows = desc->block_table ? desc->num_pages * desc->page_size : (int64_t)batch->info.total_k;
  return r;
}

// shared fields from desc, receiver 0 from (desc, W, v, o)
mf::MappedArgs mapped_args(const mf_receiver_desc* desc, const mf_batch* batch, const int32_t* row_ptr,
                           const int32_t* col_idx, const void* values, const float* W, const void* v, void* o) {
  mf::MappedArgs a;
  memset(&a, 0, sizeof(a));
  a.b = batch_args(batch);
  a.row_ptr = row_ptr; a.col_idx = col_idx; a.values = values; a.W = W; a.v = v; a.o = o;
  a.lsv = desc->layer_stride_v; a.lso = desc->layer_stride_o;
  a.block_table = desc->block_table; a.page_size = desc->page_size; a.max_pages = desc->max_pages;
  a.num_pages = desc->num_pages; a.csr_capacity = desc->csr_capacity;
  a.L = desc->num_layers; a.Ls = desc->sender_layers; a.Hs = desc->H_s; a.Hr = desc->H_r; a.Hkv = desc->H_kv_r;
  a.d = desc->d; a.B = desc->B;
  for (int l = 0; l < desc->num_layers; ++l) a.layer_map[l] = desc->layer_map[l];
  a.nrecv = 1;
  a.rx[0] = receiver_args(desc, batch, W, v, o, 0);
  return a;
}

bool allow_fast_mapped() { return !(mf::forced_portable() & MF_FORCE_PORTABLE_MAPPED); }

}  // namespace

extern "C" {

mf_status mf_mapped_attn_v(const mf_receiver_desc* desc, const mf_batch* batch, const int32_t* row_ptr,
                           const int32_t* col_idx, const void* values, const float* W, const void* v, void* o,
                           void* stream) {
  mf::clear_error();
  const char* fn = "mf_mapped_attn_v";
  bool empty = false;
  mf_status st = check_receiver(desc, batch, row_ptr, col_idx, values, W, v, o, fn, &empty);
  if (st || empty) return st;
  const mf::MappedArgs a = mapped_args(desc, batch, row_ptr, col_idx, values, W, v, o);
  const int e = mf::launch_mapped(a, desc->dtype, stream, allow_fast_mapped(), device_lds_limit());
  return e ? hip_fail(e, fn) : MF_OK;
}

size_t mf_mapped_split_workspace_size(const mf_receiver_desc* desc, const mf_batch* batch) {
  mf::clear_error();
  if (!desc || !batch || desc->num_layers < 0 || desc->num_layers > MF_MAX_LAYERS || (desc->num_layers > 0 && !desc->layer_map))
    return 0;
  const mf::MappedArgs a = mapped_args(desc, batch, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr);
  return mf::mapped_split_workspace_bytes(a, mf::mapped_splits(a, desc->dtype, allow_fast_mapped(), device_lds_limit()));
}

mf_status mf_mapped_attn_v_split(const mf_receiver_desc* desc, const mf_batch* batch, const int32_t* row_ptr,
                                 const int32_t* col_idx, const void* values, const float* W, const void* v, void* o,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  mf::clear_error();
  const char* fn = "mf_mapped_attn_v_split";
  bool empty = false;
  mf_status st = check_receiver(desc, batch, row_ptr, col_idx, values, W, v, o, fn, &empty);
  if (st || empty) return st;
  const mf::MappedArgs a = mapped_args(desc, batch, row_ptr, col_idx, values, W, v, o);
  const size_t need = mf::mapped_split_workspace_bytes(a, mf::mapped_splits(a, desc->dtype, allow_fast_mapped(),
                                                                            device_lds_limit()));
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MF_ERR_WORKSPACE, "%s: workspace of %zu bytes, %zu needed", fn, workspace ? workspace_bytes : (size_t)0,
                need);
  if (need > 0 && ((uintptr_t)workspace & 255u))
    return fail(MF_ERR_INVALID, "%s: workspace not 256-byte aligned", fn);
  const int e = mf::launch_mapped_split(a, desc->dtype, workspace, stream, allow_fast_mapped(), device_lds_limit());
  return e ? hip_fail(e, fn) : MF_OK;
}

mf_status mf_mapped_attn_v_multi(const mf_receiver_desc* const* descs, int n_receivers, const mf_batch* batch,
                                 const int32_t* row_ptr, const int32_t* col_idx, const void* values,
                                 const float* const* W, const void* const* v, void* const* o, void* stream) {
  mf::clear_error();
  const char* fn = "mf_mapped_attn_v_multi";
  if (!descs || !W || !v || !o) return fail(MF_ERR_INVALID, "%s: a receiver array is NULL", fn);
  if (n_receivers < 1 || n_receivers > MF_MAX_RECEIVERS)
    return fail(MF_ERR_INVALID, "%s: n_receivers = %d not in [1, %d]", fn, n_receivers, MF_MAX_RECEIVERS);
  bool empty = false;
  for (int k = 0; k < n_receivers; ++k) {
    mf_status st = check_receiver(descs[k], batch, row_ptr, col_idx, values, W[k], v[k], o[k], fn, &empty);
    if (st) return st;
  }
  const mf_receiver_desc* d0 = descs[0];
  for (int k = 1; k < n_receivers; ++k) {
    const mf_receiver_desc* dk = descs[k];
    bool same = dk->dtype == d0->dtype && dk->num_layers == d0->num_layers && dk->sender_layers == d0->sender_layers &&
                dk->H_s == d0->H_s && dk->d == d0->d && dk->B == d0->B && dk->csr_capacity == d0->csr_capacity;
    for (int l = 0; same && l < d0->num_layers; ++l) same = dk->layer_map[l] == d0->layer_map[l];
    if (!same)
      return fail(MF_ERR_INVALID, "%s: receiver %d differs from receiver 0 in a shared field "
                  "(dtype, layers, layer_map, sender layers, H_s, d, B or csr_capacity)", fn, k);
  }
  if (empty) return MF_OK;   // no layers or no row-blocks: every receiver is empty alike
  mf::MappedArgs a = mapped_args(d0, batch, row_ptr, col_idx, values, W[0], v[0], o[0]);
  int groups = 0;
  for (int k = 0; k < n_receivers; ++k) {
    a.rx[k] = receiver_args(descs[k], batch, W[k], v[k], o[k], groups);
    groups += (descs[k]->H_r + 7) / 8;
  }
  a.nrecv = n_receivers;
  const int e = mf::launch_mapped_multi(a, d0->dtype, stream, allow_fast_mapped(), device_lds_limit());
  return e ? hip_fail(e, fn) : MF_OK;
}

}  // extern "C"

namespace {

mf_status check_headmix(const mf_headmix_desc* d, const char* fn) {
  if (!d) return fail(MF_ERR_INVALID, "%s: desc is NULL", fn);
  if (d->dtype != MF_F32 && d->dtype != MF_BF16) return fail(MF_ERR_INVALID, "%s: unknown dtype %d", fn, (int)d->dtype);
  if (d->B != 32 && d->B != 64 && d->B != 128) return fail(MF_ERR_UNSUPPORTED, "%s: B = %d not in {32, 64, 128}", fn, d->B);
  if (d->H_s < 1 || d->H_s > 64 || d->H_r < 1 || d->H_r > 64)
    return fail(MF_ERR_UNSUPPORTED, "%s: H_s = %d, H_r = %d not in [1, 64]", fn, d->H_s, d->H_r);
  if (d->num_layers < 0 || d->num_layers > MF_MAX_LAYERS)
    return fail(MF_ERR_INVALID, "%s: num_layers = %d not in [0, %d]", fn, d->num_layers, MF_MAX_LAYERS);
  if (d->num_layers > 0 && !d->layer_map) return fail(MF_ERR_INVALID, "%s: layer_map is NULL", fn);
  for (int l = 0; l < d->num_layers; ++l)
    if (d->layer_map[l] < 0 || d->layer_map[l] >= d->sender_layers)
      return fail(MF_ERR_INVALID, "%s: layer_map[%d] = %d outside [0, %d)", fn, l, d->layer_map[l], d->sender_layers);
  if (d->sender_capacity < 0 || d->receiver_capacity < 0) return fail(MF_ERR_INVALID, "%s: negative capacity", fn);
  return MF_OK;
}

}  // namespace

extern "C" {

size_t mf_headmix_workspace_size(const mf_headmix_desc* desc, const mf_batch* batch) {
  if (!desc || !batch || desc->num_layers < 0 || desc->H_s < 1 || desc->H_s > 64 || desc->H_r < 1 || desc->H_r > 64 ||
      batch->info.total_rowblocks < 0)
    return 0;
  return align256(mf::headmix_partial_bytes(desc->num_layers, batch->info.total_rowblocks, desc->H_s, desc->H_r));
}

mf_status mf_headmix_gram(const mf_headmix_desc* desc, const mf_batch* batch, const int32_t* s_row_ptr,
                          const int32_t* s_col_idx, const void* s_values, const int32_t* r_row_ptr,
                          const int32_t* r_col_idx, const void* r_values, double* gram, double* cross,
                          void* workspace, size_t workspace_bytes, void* stream) {
  mf::clear_error();
  const char* fn = "mf_headmix_gram";
  mf_status st = check_headmix(desc, fn);
  if (st) return st;
  st = check_batch(batch, desc->B, fn);
  if (st) return st;
  if (desc->num_layers == 0) return MF_OK;
  if (!gram || !cross) return fail(MF_ERR_INVALID, "%s: gram or cross is NULL", fn);
  const int R = batch->info.total_rowblocks;
  if (R > 0) {
    if (!s_row_ptr || !r_row_ptr) return fail(MF_ERR_INVALID, "%s: a row_ptr is NULL", fn);
    if (desc->sender_capacity > 0 && (!s_col_idx || !s_values))
      return fail(MF_ERR_INVALID, "%s: sender col_idx or values is NULL", fn);
    if (desc->receiver_capacity > 0 && (!r_col_idx || !r_values))
      return fail(MF_ERR_INVALID, "%s: receiver col_idx or values is NULL", fn);
    if ((uintptr_t)s_values % 16 || (uintptr_t)r_values % 16)
      return fail(MF_ERR_INVALID, "%s: values must be 16-byte aligned", fn);
    if ((int64_t)desc->sender_layers * desc->H_s * R > INT32_MAX - 1 || (int64_t)desc->num_layers * desc->H_r * R > INT32_MAX - 1)
      return fail(MF_ERR_UNSUPPORTED, "%s: too many CSR rows", fn);
  }
  const size_t need = mf_headmix_workspace_size(desc, batch);
  if (R > 0 && (!workspace || workspace_bytes < need))
    return fail(MF_ERR_WORKSPACE, "%s: workspace needs %zu bytes, got %zu", fn, need, workspace_bytes);
  if (mf::headmix_gram_lds_bytes(desc->H_s, desc->H_r) > device_lds_limit())
    return fail(MF_ERR_UNSUPPORTED, "%s: staging does not fit in LDS", fn);
  mf::HeadmixArgs a;
  a.b = batch_args(batch);
  a.s_row_ptr = s_row_ptr; a.s_col = s_col_idx; a.s_val = s_values; a.s_cap = desc->sender_capacity;
  a.r_row_ptr = r_row_ptr; a.r_col = r_col_idx; a.r_val = r_values; a.r_cap = desc->receiver_capacity;
  a.partial = static_cast<double*>(workspace);
  a.L = desc->num_layers; a.Hs = desc->H_s; a.Hr = desc->H_r; a.B = desc->B;
  for (int l = 0; l < desc->num_layers; ++l) a.layer_map[l] = desc->layer_map[l];
  const int e = mf::launch_headmix_gram(a, desc->dtype, gram, cross, stream);
  return e ? hip_fail(e, fn) : MF_OK;
}

mf_status mf_headmix_solve(const mf_headmix_desc* desc, const double* gram, const double* cross, double lambda,
                           float* W, int32_t* dropped, void* stream) {
  mf::clear_error();
  const char* fn = "mf_headmix_solve";
  if (!desc) return fail(MF_ERR_INVALID, "%s: desc is NULL", fn);
  if (desc->H_s < 1 || desc->H_s > 64 || desc->H_r < 1 || desc->H_r > 64)
    return fail(MF_ERR_UNSUPPORTED, "%s: H_s = %d, H_r = %d not in [1, 64]", fn, desc->H_s, desc->H_r);
  if (desc->num_layers < 0 || desc->num_layers > MF_MAX_LAYERS)
    return fail(MF_ERR_INVALID, "%s: num_layers = %d not in [0, %d]", fn, desc->num_layers, MF_MAX_LAYERS);
  if (!(lambda >= 0.0) || isinf(lambda)) return fail(MF_ERR_INVALID, "%s: lambda must be finite and >= 0", fn);
  if (desc->num_layers == 0) return MF_OK;
  if (!gram || !cross || !W) return fail(MF_ERR_INVALID, "%s: gram, cross or W is NULL", fn);
  const int e = mf::launch_headmix_solve(gram, cross, lambda, desc->num_layers, desc->H_s, desc->H_r, W, dropped, stream);
  return e ? hip_fail(e, fn) : MF_OK;
}

}  // extern "C"
