// Internal interface between the C-ABI layer and the kernel launchers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "mapflow.h"

namespace mf {

// Fields of a packed batch every kernel needs.
struct BatchArgs {
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* q_pos0;   // may be null
  const int32_t* plan;
  int32_t num_seqs;
  int32_t total_rb;
  int32_t max_cb;
  int32_t total_q;
  int32_t total_k;
};

struct StatsWorkspace {
  size_t hdr, table, escratch, bytes;  // byte offsets inside the workspace
  int32_t slots;                       // persistent workgroups
};

struct StatsArgs {
  BatchArgs b;
  const void* q;
  const void* k;
  float* row_lse;
  float* block_mass;
  int64_t lsq, lsk;        // layer strides (elements)
  int32_t L, H, Hkv, d, B;
  double scale;            // logit scale
  void* ws;                // MFMA path workspace (null: portable kernel)
  StatsWorkspace wsl;
};

struct SelectArgs {
  BatchArgs b;
  const float* block_mass;
  int32_t* counts;         // [L*H*total_rb]
  uint32_t* keep_bits;     // [L*H*total_rb][words]
  int32_t words;
  int32_t L, H, B;
  double tau;
};

struct ScanArgs {
  const int32_t* counts;
  int32_t* row_ptr;
  long long* total;        // device int64
  int64_t n;
};

struct ExtractArgs {
  BatchArgs b;
  const void* q;
  const void* k;
  const float* row_lse;
  const int32_t* row_ptr;
  const uint32_t* keep_bits;
  int32_t words;
  int32_t* col_idx;
  void* values;            // may be null
  int64_t capacity;
  int64_t lsq, lsk;
  int32_t L, H, Hkv, d, B;
  double scale;
};

// One receiver of the fused step: its head mapping, values, output and value
// layout, and the first of its groups of 8 receiver heads in a launch that
// serves several receivers.
struct MappedRecv {
  const float* W;
  const void* v;
  void* o;
  int64_t lsv, lso;
  const int32_t* block_table;
  int32_t page_size, max_pages;
  int64_t num_pages;
  int32_t Hr, Hkv;
  int32_t group0;
  int64_t vrows;           // value rows of one layer (tokens, or pages x page size)
};

struct MappedArgs {
  BatchArgs b;
  const int32_t* row_ptr;
  const int32_t* col_idx;
  const void* values;
  // the receiver of a single-receiver launch (portable kernel, and rx[0])
  const float* W;
  const void* v;
  void* o;
  int64_t lsv, lso;
  const int32_t* block_table;
  int32_t page_size, max_pages;
  int64_t num_pages;
  int64_t csr_capacity;
  int32_t L, Ls, Hs, Hr, Hkv, d, B;
  int32_t layer_map[MF_MAX_LAYERS];
  // every receiver of the launch (the MFMA kernel reads these)
  int32_t nrecv;
  MappedRecv rx[MF_MAX_RECEIVERS];
  // union splits (MFMA kernel, one receiver): up to nsplit workgroups share a
  // unit's union walk, each over a column range, and write fp32 partial
  // outputs that a second kernel sums; 0 or 1: no splits
  int32_t nsplit;
  float* partial;           // [unit x group][nsplit][64 rows][8 heads][d]
  int32_t* split_count;     // [unit x group]: the splits a unit took
};

// Least-squares fit of the head mix: the two CSRs, the layer pairing and
// the per-row-block partial products (workspace).
struct HeadmixArgs {
  BatchArgs b;
  const int32_t* s_row_ptr;
  const int32_t* s_col;
  const void* s_val;
  int64_t s_cap;
  const int32_t* r_row_ptr;
  const int32_t* r_col;
  const void* r_val;
  int64_t r_cap;
  double* partial;          // [L][total_rb][H_s + H_r][H_s]
  int32_t L, Hs, Hr, B;
  int32_t layer_map[MF_MAX_LAYERS];
};

// The matrix-pipe probe (mf_mfma_probe).
int launch_mfma_probe(float* out, int nblocks, int iters, bool with_vector, void* stream);

// Mask of stages forced onto their portable twins (mf_debug_force_portable).
uint32_t forced_portable();

// Launchers: return 0 on success, a hipError_t value otherwise.
int launch_block_stats(const StatsArgs& a, mf_dtype dt, void* stream);
size_t block_stats_lds_bytes(int B, int max_cb);
bool stats_fast_path(mf_dtype dt, int B, int d);
StatsWorkspace stats_workspace_layout(int B, int max_cb, int total_rb, int slots);
int stats_slots(int num_cus);
int launch_select(const SelectArgs& a, void* stream);
int launch_scan(const ScanArgs& a, void* stream);
int launch_extract(const ExtractArgs& a, mf_dtype dt, void* stream);
int launch_mapped(const MappedArgs& a, mf_dtype dt, void* stream, bool allow_fast, size_t lds_limit);
// the union-split launch of one receiver: the splits it would use (1: none)
// and the workspace they need, and the launch itself (the plain launch when
// no split applies)
int mapped_splits(const MappedArgs& a, mf_dtype dt, bool allow_fast, size_t lds_limit);
size_t mapped_split_workspace_bytes(const MappedArgs& a, int nsplit);
int launch_mapped_split(MappedArgs a, mf_dtype dt, void* ws, void* stream, bool allow_fast, size_t lds_limit);
// several receivers on one CSR: one launch when the MFMA kernel covers them
// all, else one launch per receiver
int launch_mapped_multi(const MappedArgs& a, mf_dtype dt, void* stream, bool allow_fast, size_t lds_limit);
size_t select_lds_bytes(int max_cb);
size_t headmix_partial_bytes(int L, int total_rb, int Hs, int Hr);
size_t headmix_gram_lds_bytes(int Hs, int Hr);
int launch_headmix_gram(const HeadmixArgs& a, mf_dtype dt, double* gram, double* cross, void* stream);
int launch_headmix_solve(const double* gram, const double* cross, double lam, int L, int Hs, int Hr, float* W,
                         int32_t* dropped, void* stream);

}  // namespace mf
