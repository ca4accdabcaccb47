// Host-only planning of a packed (varlen, chunked) batch into query
// row-blocks: the block grid restarts in every sequence and is aligned to
// absolute positions, so a prefill chunk must start on a block edge.
#include <stdint.h>
#include <string.h>

#include "mapflow.h"
#include "errors.h"

extern "C" mf_status mf_plan(const int32_t* h_cu_q, const int32_t* h_cu_k, const int32_t* h_q_pos0,
                             int32_t num_seqs, int32_t B, int32_t* h_plan, int64_t plan_capacity,
                             mf_plan_info* info) {
  using mf::fail;
  mf::clear_error();
  if (!info) return fail(MF_ERR_INVALID, "mf_plan: info is NULL");
  memset(info, 0, sizeof(*info));
  if (num_seqs < 0) return fail(MF_ERR_INVALID, "mf_plan: num_seqs = %d < 0", num_seqs);
  if (num_seqs > 0 && (!h_cu_q || !h_cu_k))
    return fail(MF_ERR_INVALID, "mf_plan: cu_seqlens arrays are NULL");
  if (B != 32 && B != 64 && B != 128) return fail(MF_ERR_UNSUPPORTED, "mf_plan: B = %d not in {32, 64, 128}", B);
  if (num_seqs > 0 && (h_cu_q[0] != 0 || h_cu_k[0] != 0))
    return fail(MF_ERR_INVALID, "mf_plan: cu_seqlens must start at 0");
  int64_t total_rb = 0;
  int32_t max_k = 0;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t qlen = (int64_t)h_cu_q[s + 1] - h_cu_q[s];
    const int64_t klen = (int64_t)h_cu_k[s + 1] - h_cu_k[s];
    const int64_t p0 = h_q_pos0 ? h_q_pos0[s] : 0;
    if (qlen < 0 || klen < 0) return fail(MF_ERR_INVALID, "mf_plan: sequence %d has negative length", s);
    if (p0 < 0) return fail(MF_ERR_INVALID, "mf_plan: q_pos0[%d] = %lld < 0", s, (long long)p0);
    if (p0 % B) return fail(MF_ERR_UNSUPPORTED, "mf_plan: q_pos0[%d] = %lld is not a multiple of B = %d", s, (long long)p0, B);
    if (klen < p0 + qlen)
      return fail(MF_ERR_INVALID, "mf_plan: sequence %d: keys (%lld) do not cover positions up to %lld", s,
                  (long long)klen, (long long)(p0 + qlen));
    if (klen > MF_MAX_KEYS)
      return fail(MF_ERR_UNSUPPORTED, "mf_plan: sequence %d has %lld keys > MF_MAX_KEYS = %d", s, (long long)klen, MF_MAX_KEYS);
    total_rb += (qlen + B - 1) / B;
    if (klen > max_k) max_k = (int32_t)klen;
  }
  if (total_rb + num_seqs + 1 > INT32_MAX) return fail(MF_ERR_UNSUPPORTED, "mf_plan: batch too large");
  info->num_seqs = num_seqs;
  info->block = B;
  info->total_rowblocks = (int32_t)total_rb;
  info->max_colblocks = (max_k + B - 1) / B;
  info->total_q = num_seqs ? h_cu_q[num_seqs] : 0;
  info->total_k = num_seqs ? h_cu_k[num_seqs] : 0;
  info->max_k_len = max_k;
  info->plan_len = (int32_t)(num_seqs + 1 + total_rb);
  if (!h_plan || plan_capacity < info->plan_len)
    return fail(MF_ERR_CAPACITY, "mf_plan: plan buffer needs %d int32 words", info->plan_len);
  int32_t rb = 0;
  for (int s = 0; s < num_seqs; ++s) {
    h_plan[s] = rb;
    const int32_t qlen = h_cu_q[s + 1] - h_cu_q[s];
    const int32_t n = (qlen + B - 1) / B;
    for (int32_t i = 0; i < n; ++i) h_plan[num_seqs + 1 + rb + i] = s;
    rb += n;
  }
  h_plan[num_seqs] = rb;
  return MF_OK;
}
