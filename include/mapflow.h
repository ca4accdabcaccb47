/*
 * mapflow.h - C ABI of the MapFlow hot path on AMD Instinct MI355X (gfx950).
 *
 * MapFlow lets a receiver model reuse a sender model's attention map for the
 * same context instead of recomputing its own (MapFlow page, 163.com,
 * section "从内部表示,走向 token 之间的依赖关系").  This library runs the
 * data-parallel part of that path on one GPU:
 *
 *   mf_block_stats      first stage of the staged compression: per query
 *                       row-block, the attention probability mass of every
 *                       causal B x B block, straight from the sender's Q and
 *                       K, without forming the dense map (section
 *                       "让复用真正省时…", paragraph "第一").
 *   mf_compress_blocks  second stage: per (layer, sender head, row-block) keep
 *                       the blocks needed to reach cumulative probability tau
 *                       and extract their probabilities into a block-sparse
 *                       CSR (same paragraph; kept counts differ per layer and
 *                       position, paragraph "第二").
 *   mf_mapped_attn_v    the fused step: read the kept blocks of every sender
 *                       head, form the learned linear head combination on
 *                       chip, multiply by the receiver's own V and accumulate
 *                       the output, with no dense receiver map (paragraph
 *                       "第三"); mf_mapped_attn_v_multi serves several
 *                       receivers of one compressed map in one launch.
 *
 * Around it: a prefix cache of compressed maps (mf_prefix_block_hashes,
 * mf_map_cache_*; paragraph "第二"), and the offline least-squares fit of the
 * head mapping W from compressed maps (mf_headmix_*; section "从内部表示…").
 *
 * Conventions shared by every entry point
 *   - Pointers marked DEVICE are GPU memory, HOST are CPU memory.  The caller
 *     owns and allocates every device buffer; the library allocates no device
 *     memory.  The prefix cache keeps its index in host memory and a small
 *     pinned host buffer for its copy tables.
 *   - Calls are asynchronous on `stream` (a hipStream_t, NULL = default
 *     stream).  mf_compress_blocks with a non-NULL nnz_out synchronises
 *     `stream` once to read the kept-block count; a prefix-cache insert or
 *     splice waits on the host only until the previous such call's small
 *     table copies have left the pinned buffer.
 *   - Every argument is validated on the host before anything is launched;
 *     a failing call returns a status other than MF_OK, launches nothing and
 *     records a message for mf_last_error_message().  No exceptions or aborts
 *     cross the ABI.
 *   - Layouts are token-major: Q [T, H, d], K [T, H_kv, d], V [T, H_kv_r, d],
 *     O [T, H_r, d], d contiguous.  Sequences of a batch are packed one after
 *     another (varlen); a batch may hold prefill chunks, whose first query row
 *     sits at position q_pos0 of its sequence while its keys cover the whole
 *     prefix (chunked prefill, MapFlow page, paragraph "第三" and the closing
 *     paragraph of that section on vLLM support for PagedAttention, chunked
 *     prefill and varlen packing).
 *   - Supported shapes: B in {32, 64, 128}; d in {64, 128}; 1 <= H <= 64 with
 *     H_kv dividing H; dtype fp32 or bf16; chunk starts multiple of B; keys
 *     of a sequence per call <= MF_MAX_KEYS.
 *   - Thread safety: calls on distinct streams may run concurrently, except
 *     calls that share a workspace or a prefix cache; the compressed CSR is
 *     read-only for mf_mapped_attn_v, so any number of receivers may read one
 *     sender state at once (paragraph "第二": one sender state serves several
 *     downstream models).  Error messages are kept per host thread.
 */
#ifndef MAPFLOW_H
#define MAPFLOW_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MF_OK = 0,
  MF_ERR_INVALID = 1,      /* null pointer, negative size, inconsistent layout */
  MF_ERR_UNSUPPORTED = 2,  /* well-formed but outside the supported shapes */
  MF_ERR_CAPACITY = 3,     /* more kept blocks than capacity_blocks (see below) */
  MF_ERR_HIP = 4,          /* a HIP runtime call failed */
  MF_ERR_WORKSPACE = 5     /* workspace missing or too small */
} mf_status;

typedef enum { MF_F32 = 0, MF_BF16 = 1 } mf_dtype;

/* Longest key range of one sequence: the per-(row, column-block) statistics
 * of one row-block live in on-chip LDS (about 4 bytes per key). */
#define MF_MAX_KEYS 40448

/* ------------------------------------------------------------------------ */
/* Batch layout (varlen + chunked prefill)                                  */
/* ------------------------------------------------------------------------ */

/* Sizes of a packed batch, filled by mf_plan. */
typedef struct {
  int32_t num_seqs;
  int32_t block;            /* B the plan was made for */
  int32_t total_rowblocks;  /* sum over sequences of ceil(q_len / B) */
  int32_t max_colblocks;    /* max over sequences of ceil(k_len / B) */
  int32_t total_q;          /* packed query rows */
  int32_t total_k;          /* packed keys (= value rows) */
  int32_t max_k_len;
  int32_t plan_len;         /* int32 words of the device plan: num_seqs + 1 + total_rowblocks */
} mf_plan_info;

/* Host-only.  Validates a packed batch and writes its row-block plan.
 *   h_cu_seqlens_q  HOST [num_seqs+1]  query row offsets, non-decreasing, [0] = 0
 *   h_cu_seqlens_k  HOST [num_seqs+1]  key offsets
 *   h_q_pos0        HOST [num_seqs] or NULL  position of each chunk's first
 *                   query row inside its sequence (multiple of B); NULL = 0
 *   h_plan          HOST [plan_capacity] int32 or NULL: receives the plan, a
 *                   prefix of row-block offsets per sequence (num_seqs + 1
 *                   words) followed by the sequence of every row-block.  The
 *                   caller copies it to the device and passes it in mf_batch.
 * Requires k_len >= q_pos0 + q_len per sequence.  With h_plan NULL or
 * plan_capacity < info->plan_len only `info` is filled and the call returns
 * MF_ERR_CAPACITY, so a caller can size the buffer first. */
mf_status mf_plan(const int32_t* h_cu_seqlens_q, const int32_t* h_cu_seqlens_k,
                  const int32_t* h_q_pos0, int32_t num_seqs, int32_t B,
                  int32_t* h_plan, int64_t plan_capacity, mf_plan_info* info);

/* A packed batch as the kernels see it. */
typedef struct {
  mf_plan_info info;            /* from mf_plan */
  const int32_t* cu_seqlens_q;  /* DEVICE [num_seqs+1] */
  const int32_t* cu_seqlens_k;  /* DEVICE [num_seqs+1] */
  const int32_t* q_pos0;        /* DEVICE [num_seqs] or NULL (all zero) */
  const int32_t* plan;          /* DEVICE [info.plan_len] copy of mf_plan's h_plan */
} mf_batch;

/* ------------------------------------------------------------------------ */
/* Sender side: staged block compression                                    */
/* ------------------------------------------------------------------------ */

typedef struct {
  mf_dtype dtype;           /* of Q, K and the packed block values */
  int32_t num_layers;       /* sender layers compressed in one call */
  int32_t H_s, H_kv_s;      /* query heads, key heads (H_kv_s divides H_s) */
  int32_t d, B;             /* head dim, block size */
  float sm_scale;           /* logit scale; 0 means 1/sqrt(d) */
  int64_t layer_stride_q;   /* elements between layers of q (>= total_q*H_s*d) */
  int64_t layer_stride_k;   /* elements between layers of k (>= total_k*H_kv_s*d) */
} mf_sender_desc;

/* Stage 1: block statistics.
 *   q          DEVICE [num_layers][total_q][H_s][d]   (layer stride as above)
 *   k          DEVICE [num_layers][total_k][H_kv_s][d]
 *   row_lse    DEVICE fp32 [num_layers][H_s][total_q]: log sum_c exp(s_rc)
 *              over the causal keys of each query row, s = sm_scale * q.k
 *   block_mass DEVICE fp32 [num_layers][H_s][total_rowblocks][max_colblocks]:
 *              m[i][j] = (sum of the softmax probabilities of block (i, j)) /
 *              (valid rows of row-block i), so each row-block's masses sum to
 *              1; entries past the row-block's causal range are 0.
 * Row-block i of a sequence covers query positions [q_pos0 + iB, ...); its
 * causal column blocks are 0 .. (position of its last row) / B. */
mf_status mf_block_stats(const mf_sender_desc* desc, const mf_batch* batch,
                         const void* q, const void* k,
                         float* row_lse, float* block_mass,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes mf_block_stats needs for this batch on the current device
 * (0 when the shapes take the path without scratch; then workspace may be
 * NULL).  workspace: DEVICE, at least this many bytes, owned by the caller;
 * its contents on entry do not matter and are scratch afterwards (per-block
 * log masses of the row-blocks in flight, the work queue of the persistent
 * grid).  Calls that overlap in time need distinct workspaces.  Too small a
 * workspace returns MF_ERR_WORKSPACE before anything is launched. */
size_t mf_block_stats_workspace_size(const mf_sender_desc* desc, const mf_batch* batch);

/* Workspace bytes mf_compress_blocks needs for this batch. */
size_t mf_compress_workspace_size(const mf_sender_desc* desc, const mf_batch* batch);

/* Stage 2: selection and extraction.
 * For every (layer l, sender head h, row-block i), sort its causal blocks by
 * mass (descending; equal masses by ascending column block), and keep the
 * shortest prefix whose cumulative mass (summed in fp64) reaches tau; tau = 1
 * keeps every causal block.  The kept blocks form CSR row
 * (l * H_s + h) * total_rowblocks + i:
 *   row_ptr  DEVICE int32 [num_layers * H_s * total_rowblocks + 1]
 *   col_idx  DEVICE int32 [capacity_blocks], ascending within a row
 *   values   DEVICE [capacity_blocks][B][B] in dtype, or NULL (count only),
 *            key-major: values[e][c][r] = exp(s_rc - row_lse_r) for key
 *            column c and query row r of the block, exactly the sender's
 *            probabilities (not renormalised), 0 where c is past row r or
 *            past the sequence.  Key-major rows let the fused kernel stage a
 *            block with plain 16-byte copies.
 * nnz_out HOST or NULL.  Non-NULL: the call synchronises `stream`, stores the
 * number of kept blocks, and returns MF_ERR_CAPACITY (row_ptr valid,
 * col_idx/values untouched) when it exceeds capacity_blocks; with col_idx
 * NULL and capacity_blocks 0 it only counts (row_ptr and nnz) and succeeds.  NULL: nothing
 * blocks; entries past capacity_blocks are dropped on the device, and
 * row_ptr[last] always holds the true count, so a caller can check it later.
 * tau must be in (0, 1].  workspace: DEVICE, at least
 * mf_compress_workspace_size() bytes. */
mf_status mf_compress_blocks(const mf_sender_desc* desc, const mf_batch* batch,
                             const void* q, const void* k,
                             const float* row_lse, const float* block_mass, float tau,
                             int32_t* row_ptr, int32_t* col_idx, void* values,
                             int64_t capacity_blocks, int64_t* nnz_out,
                             void* workspace, size_t workspace_bytes, void* stream);

/* mf_compress_blocks for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without the workspace, whose role a static
 * device array of MF_STATIC_SCRATCH_BYTES per GPU takes (held by each GPU the
 * library runs on until the process ends).  It calls no allocator.  A batch
 * whose mf_compress_workspace_size() exceeds MF_STATIC_SCRATCH_BYTES returns
 * MF_ERR_WORKSPACE before anything is launched.  Every call on one GPU shares
 * that GPU's array, so calls that overlap in time on one GPU race; calls in
 * one stream, or separated by synchronisation, do not.  The array's contents
 * on entry do not matter. */
#define MF_STATIC_SCRATCH_BYTES (16u << 20)
mf_status mf_compress_blocks_noalloc(const mf_sender_desc* desc, const mf_batch* batch,
                                     const void* q, const void* k,
                                     const float* row_lse, const float* block_mass, float tau,
                                     int32_t* row_ptr, int32_t* col_idx, void* values,
                                     int64_t capacity_blocks, int64_t* nnz_out, void* stream);

/* ------------------------------------------------------------------------ */
/* Receiver side: fused mapped attention . V                                */
/* ------------------------------------------------------------------------ */

#define MF_MAX_LAYERS 256

typedef struct {
  mf_dtype dtype;             /* of the block values, V and O */
  int32_t num_layers;         /* receiver mapped layers in this call */
  int32_t sender_layers;      /* layers in the CSR (its num_layers) */
  const int32_t* layer_map;   /* HOST [num_layers]: CSR layer each receiver layer
                                 reads (layer mapping matches depths, section
                                 "从内部表示…") */
  int32_t H_s;                /* sender heads in the CSR */
  int32_t H_r, H_kv_r;        /* receiver heads, value heads (H_kv_r divides H_r) */
  int32_t d, B;
  int64_t layer_stride_v;     /* elements between layers of v */
  int64_t layer_stride_o;     /* elements between layers of o */
  /* Paged values (PagedAttention).  block_table NULL: v is packed
     [total_k][H_kv_r][d] per layer.  Otherwise v is a page pool
     [num_pages][page_size][H_kv_r][d] per layer, and token t of sequence s
     lives in page block_table[s * max_pages + t / page_size]. */
  const int32_t* block_table; /* DEVICE [num_seqs][max_pages] or NULL */
  int32_t page_size, max_pages;
  int64_t num_pages;          /* pages per layer of the pool; page ids are clamped to it */
  int64_t csr_capacity;       /* entries of col_idx / values; CSR entries past it are ignored */
} mf_receiver_desc;

/* O_r[i] = sum over blocks j kept by any sender head of
 *          (sum_{h keeps j} W[r][h] * P_h[i][j]) . V_{g(r)}[j]
 * for every receiver layer, row-block i and receiver head r, where P_h are the
 * packed values of CSR layer layer_map[l] and g(r) = r / (H_r / H_kv_r).
 *   row_ptr, col_idx, values  DEVICE, as written by mf_compress_blocks
 *   W    DEVICE fp32 [num_layers][H_r][H_s]  learned head mapping
 *   v    DEVICE values (packed or paged, see above)
 *   o    DEVICE [num_layers][total_q][H_r][d] in dtype; overwritten
 * The CSR must come from a compression of the same batch layout. */
mf_status mf_mapped_attn_v(const mf_receiver_desc* desc, const mf_batch* batch,
                           const int32_t* row_ptr, const int32_t* col_idx,
                           const void* values, const float* W, const void* v,
                           void* o, void* stream);

/* mf_mapped_attn_v for launches too small to fill the GPU (few row-blocks
 * and layers, such as a single 4K layer), where the time is that of the
 * longest row-block's walk over its union of kept blocks.  Same arguments
 * and output as mf_mapped_attn_v (paragraph "第三": the output is a sum over
 * the kept blocks, with no renormalisation), plus a workspace: the union of a
 * long row-block is cut into up to 8 column ranges walked by separate
 * workgroups, each writing an fp32 partial output, and a second kernel sums
 * the partials in range order into O.  O therefore equals mf_mapped_attn_v's
 * up to fp32 summation order (the same tolerance against the definition),
 * and repeated calls give the same bits.  When the launch is large enough,
 * or the shape runs on the portable kernel, no split is made, the workspace
 * is not touched and the result is mf_mapped_attn_v's bit for bit.
 *   workspace  DEVICE, 256-byte aligned, at least
 *              mf_mapped_split_workspace_size() bytes (may be NULL when that
 *              is 0); calls that overlap in time need distinct workspaces
 * Errors: as mf_mapped_attn_v, plus MF_ERR_WORKSPACE (missing or too small)
 * and MF_ERR_INVALID (misaligned workspace). */
size_t mf_mapped_split_workspace_size(const mf_receiver_desc* desc, const mf_batch* batch);
mf_status mf_mapped_attn_v_split(const mf_receiver_desc* desc, const mf_batch* batch,
                                 const int32_t* row_ptr, const int32_t* col_idx,
                                 const void* values, const float* W, const void* v,
                                 void* o, void* workspace, size_t workspace_bytes,
                                 void* stream);

#define MF_MAX_RECEIVERS 4

/* Several receivers reuse one sender state in one launch (one sender state
 * serving several downstream models, section "让复用真正省时…", paragraph
 * "第二").  Receiver k is described by descs[k], W[k], v[k] and o[k] exactly as
 * in mf_mapped_attn_v, and gets the same output.  All descriptors must share
 * dtype, num_layers, the layer_map contents, sender_layers, H_s, d, B and
 * csr_capacity; each has its own H_r, H_kv_r, value layout (packed or paged)
 * and strides.  The head groups of every receiver for one row-block and
 * layer run back to back on one XCD, so the kept values they all read are
 * fetched from HBM about once instead of once per receiver.
 *   descs, W, v, o  HOST arrays of n_receivers (1 <= n <= MF_MAX_RECEIVERS)
 *                   pointers; the tensors they point to are DEVICE
 *   o[k] must not overlap another receiver's o or any input.
 * Errors: MF_ERR_INVALID for a NULL array or a descriptor that differs in a
 * shared field, plus everything mf_mapped_attn_v reports per receiver. */
mf_status mf_mapped_attn_v_multi(const mf_receiver_desc* const* descs, int n_receivers,
                                 const mf_batch* batch, const int32_t* row_ptr,
                                 const int32_t* col_idx, const void* values,
                                 const float* const* W, const void* const* v,
                                 void* const* o, void* stream);

/* ------------------------------------------------------------------------ */
/* Offline calibration of the head mix                                      */
/* ------------------------------------------------------------------------ */

/* The head mapping W is a learned linear combination of sender heads,
 * trained once by offline calibration with both models frozen (section
 * "从内部表示…").  These calls fit it by least squares from compressed maps:
 * for receiver layer l, paired with sender CSR layer layer_map[l], W[l]
 * minimises
 *     sum_r sum_(i, j) || A_r[i][j] - sum_h W[r][h] Pt_h[i][j] ||_F^2
 *     + lambda ||W[l]||_F^2
 * over the blocks (i, j) of the union of the sender heads' kept sets, where
 * Pt_h[i][j] is sender head h's kept block (0 where h does not keep j; the
 * operand mf_mapped_attn_v mixes) and A_r[i][j] is receiver head r's block
 * from the receiver's own compressed map (0 where r does not keep j).  Blocks
 * outside the union add a constant and are left out.  The minimiser solves
 *     (G + lambda I) w_r = b_r,  G[h][h'] = sum <Pt_h, Pt_h'>,
 *                                b_r[h]   = sum <A_r, Pt_h>
 * (inner products over the B x B entries of a block). */
typedef struct {
  mf_dtype dtype;             /* of both CSRs' values */
  int32_t B;
  int32_t num_layers;         /* receiver layers fitted = layers of the receiver CSR */
  int32_t sender_layers;      /* layers of the sender CSR */
  const int32_t* layer_map;   /* HOST [num_layers]: sender layer of each receiver layer */
  int32_t H_s, H_r;           /* heads of the sender CSR and of the receiver CSR, each in [1, 64] */
  int64_t sender_capacity;    /* entries of the sender col_idx / values; entries past it are ignored */
  int64_t receiver_capacity;  /* same for the receiver CSR */
} mf_headmix_desc;

/* Workspace bytes of mf_headmix_gram: one partial product matrix per
 * (receiver layer, row-block), 8 (H_s + H_r) H_s bytes each. */
size_t mf_headmix_workspace_size(const mf_headmix_desc* desc, const mf_batch* batch);

/* G and b of the normal equations, summed in fp64 (bf16 and fp32 products are
 * exact in fp64; the sum over row-blocks runs in a fixed order, so results
 * repeat bit for bit).
 *   s_row_ptr, s_col_idx, s_values  DEVICE sender CSR as mf_compress_blocks
 *                                   writes it (sender_layers x H_s rows per
 *                                   row-block of `batch`)
 *   r_row_ptr, r_col_idx, r_values  DEVICE receiver CSR of the same batch
 *                                   layout (num_layers x H_r heads), e.g.
 *                                   mf_compress_blocks on the receiver's Q/K
 *   gram   DEVICE fp64 [num_layers][H_s][H_s], overwritten
 *   cross  DEVICE fp64 [num_layers][H_r][H_s]: cross[l][r][h] = b_r[h]
 *   workspace  DEVICE, at least mf_headmix_workspace_size() bytes
 * Both CSRs must use the same B and dtype; both values arrays must be 16-byte
 * aligned (MF_ERR_INVALID otherwise). */
mf_status mf_headmix_gram(const mf_headmix_desc* desc, const mf_batch* batch,
                          const int32_t* s_row_ptr, const int32_t* s_col_idx, const void* s_values,
                          const int32_t* r_row_ptr, const int32_t* r_col_idx, const void* r_values,
                          double* gram, double* cross, void* workspace, size_t workspace_bytes,
                          void* stream);

/* W[l] from gram[l] and cross[l]: a Cholesky factorisation of G + lambda I
 * in fp64, column by column; head k is dropped when its pivot falls to at
 * most 1e-12 of its diagonal (a head that keeps nothing, or whose maps lie in
 * the span of earlier heads) and gets weight 0, the others being the fit
 * without it.  Then a forward and a back substitution per receiver head.
 *   gram, cross  DEVICE as written by mf_headmix_gram
 *   lambda       ridge weight, finite and >= 0
 *   W            DEVICE fp32 [num_layers][H_r][H_s], ready for mf_mapped_attn_v
 *   dropped      DEVICE int32 [num_layers][H_s] or NULL: 1 for a dropped head */
mf_status mf_headmix_solve(const mf_headmix_desc* desc, const double* gram, const double* cross,
                           double lambda, float* W, int32_t* dropped, void* stream);

/* ------------------------------------------------------------------------ */
/* Prefix cache of compressed maps                                          */
/* ------------------------------------------------------------------------ */
/* Requests that share a token prefix share the sender's compressed rows for
 * it (a cache managed by shared prefix, section "让复用真正省时…", paragraph
 * "第二").  In a causal sender, row-block i of a sequence depends only on
 * tokens [0, (i+1) B), so its CSR rows (every layer and sender head) are keyed
 * by a chained hash of the first i + 1 blocks of tokens.
 *
 * Row numbering used below: in a CSR written by mf_compress_blocks for a batch
 * of R row-blocks, the row of (layer l, sender head h, row-block r) is
 * (l * H_s + h) * R + r. */

/* FNV-1a 64-bit (offset basis 0xcbf29ce484222325, prime 0x100000001b3),
 * chained over blocks: hash[i] is FNV-1a over the 8 bytes of hash[i - 1]
 * (little-endian; `parent` for i = 0, 0 at a sequence start) followed by the
 * B tokens of block i (int32 little-endian).  tokens and hashes_out are HOST
 * arrays; one hash per full block (n_tokens / B) is written.  Returns that
 * count, or -1 for a NULL pointer, n_tokens < 0 or B < 1. */
int64_t mf_prefix_block_hashes(const int32_t* tokens, int64_t n_tokens, int32_t B,
                               uint64_t parent, uint64_t* hashes_out);

typedef struct mf_map_cache mf_map_cache;

typedef struct {
  mf_dtype dtype;             /* of the block values */
  int32_t num_layers;         /* CSR layers an entry holds */
  int32_t H_s;                /* sender heads */
  int32_t B;
} mf_map_cache_desc;

typedef struct {
  int64_t entries, pinned_entries;
  int64_t bytes_used, bytes_capacity;   /* of the device pool */
  int64_t blocks_hit, blocks_missed;    /* by mf_map_cache_lookup */
  int64_t evictions;
} mf_map_cache_stats;

/* An entry holds the CSR rows of row-blocks [0, n) of one sequence for every
 * layer and head, in `pool` (DEVICE, pool_bytes, owned by the caller; it must
 * outlive the cache).  The index stays on the host.  Entries not pinned by a
 * lookup are evicted least recently used first when an insert needs room.
 * One caller at a time, and every call on one stream (or synchronised
 * between streams): the cache reuses a small table area in the pool.
 *
 * Insert and splice are stream-ordered and return before their copies run:
 * their device sources must stay unchanged, and their outputs are ready, only
 * once `stream` has passed the call.  So a fetch of cached rows can overlap
 * other work on another stream (the receiver recomputing its early layers
 * while the maps are fetched: the MapFlow page, paragraph "第二").  A call
 * waits on the host only for the previous call's small host-to-device table
 * copies; the cache keeps a pinned host staging buffer for them (allocated at
 * the first copying call, grown when a larger row_ptr needs it, freed by
 * mf_map_cache_destroy, which first waits for those copies). */
mf_status mf_map_cache_create(const mf_map_cache_desc* desc, void* pool, size_t pool_bytes,
                              mf_map_cache** out);
void mf_map_cache_destroy(mf_map_cache* cache);

/* Copies the CSR rows of the first n_blocks row-blocks of one sequence into a
 * new entry keyed by hashes[0..n_blocks) (HOST).  The sequence's rows must
 * start at token 0 and occupy rows rb_first .. rb_first + n_blocks - 1 of a
 * CSR with total_rb row-blocks per (layer, head); row_ptr_host is a HOST copy
 * of that CSR's row_ptr, col_idx and values are DEVICE.  Nothing is copied
 * when hashes[n_blocks - 1] is already cached.  MF_ERR_CAPACITY when the pool
 * cannot hold the entry even after evicting every unpinned entry. */
mf_status mf_map_cache_insert(mf_map_cache* cache, const uint64_t* hashes, int32_t n_blocks,
                              const int32_t* row_ptr_host, int32_t total_rb, int32_t rb_first,
                              const int32_t* col_idx, const void* values, void* stream);

/* Number m of leading hashes[0..n) (HOST) the cache holds.  A nonzero m pins
 * the entry holding them until mf_map_cache_release(cache, hashes, m). */
int32_t mf_map_cache_lookup(mf_map_cache* cache, const uint64_t* hashes, int32_t n);
void mf_map_cache_release(mf_map_cache* cache, const uint64_t* hashes, int32_t m);

/* Writes the CSR mf_compress_blocks would write for one sequence of n_blocks
 * row-blocks (a single-sequence batch from token 0): row-blocks [0, m) from
 * the pinned entry of hashes[0..m), row-blocks [m, n_blocks) from a CSR of
 * the same sequence compressed as a chunk that starts at row m * B.  That
 * suffix CSR has suffix_total_rb row-blocks per (layer, head), the sequence
 * at rows suffix_rb_first .. + n_blocks - m - 1; suffix_row_ptr_host is HOST,
 * its col_idx and values DEVICE.  Outputs are DEVICE: row_ptr_out
 * [num_layers * H_s * n_blocks + 1], col_idx_out and values_out with room for
 * capacity_blocks entries; *nnz_out (HOST) receives the entry count.
 * MF_ERR_CAPACITY when it exceeds capacity_blocks (nothing is written then);
 * MF_ERR_INVALID when hashes[0..m) are not all held by one pinned entry. */
mf_status mf_map_cache_splice(mf_map_cache* cache, const uint64_t* hashes, int32_t m,
                              int32_t n_blocks, const int32_t* suffix_row_ptr_host,
                              int32_t suffix_total_rb, int32_t suffix_rb_first,
                              const int32_t* suffix_col_idx, const void* suffix_values,
                              int32_t* row_ptr_out, int32_t* col_idx_out, void* values_out,
                              int64_t capacity_blocks, int64_t* nnz_out, void* stream);

mf_status mf_map_cache_get_stats(const mf_map_cache* cache, mf_map_cache_stats* out);

/* ------------------------------------------------------------------------ */
/* Diagnostics                                                              */
/* ------------------------------------------------------------------------ */

const char* mf_status_string(mf_status s);
/* Message of the last failing call on this thread ("" if none). */
const char* mf_last_error_message(void);
/* Library version, e.g. "mapflow-mi355x 0.2". */
const char* mf_version(void);

/* Matrix-pipe probe: what the bf16 MFMA pipe of this GPU sustains, to set
 * the statistics kernel's measured rate beside a measured ceiling as well as
 * beside the nominal peak.  Each of nblocks workgroups of 4 waves issues
 * 4 * iters independent MFMA 32x32x16 bf16 operations per wave (32768 flop
 * each, so 524288 * nblocks * iters flop in all); with_vector != 0 adds the
 * vector work the statistics kernel does per MFMA (two exp2 sums, three
 * vector instructions each).  out: DEVICE float [nblocks * 256], overwritten
 * with values that only keep the work from being optimised away.  Time the
 * launch on `stream`.  Errors: MF_ERR_INVALID for NULL out, nblocks or
 * iters < 1. */
mf_status mf_mfma_probe(float* out, int nblocks, int iters, int with_vector, void* stream);

/* Cross-check hook for tests.  Every fast kernel has a portable twin that
 * computes the same results with plain code (no MFMA, no async copies).  A
 * set bit makes later calls, on every thread, take the twin of that stage;
 * the calls' results are otherwise unchanged.  Returns the previous mask.
 * The mask is process-wide and 0 by default: production callers never set
 * it, and a change does not affect launches already queued. */
#define MF_FORCE_PORTABLE_STATS   0x1u  /* mf_block_stats */
#define MF_FORCE_PORTABLE_SELECT  0x2u  /* selection sort of mf_compress_blocks */
#define MF_FORCE_PORTABLE_EXTRACT 0x4u  /* extraction of mf_compress_blocks */
#define MF_FORCE_PORTABLE_MAPPED  0x8u  /* mf_mapped_attn_v, mf_mapped_attn_v_multi */
uint32_t mf_debug_force_portable(uint32_t mask);

#ifdef __cplusplus
}
#endif

#endif /* MAPFLOW_H */
