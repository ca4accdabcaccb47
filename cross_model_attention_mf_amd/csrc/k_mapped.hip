// Fused mapped attention . V (MapFlow page, section "让复用真正省时…",
// paragraph "第三"): read the kept sparse blocks of every sender head, form
// the learned linear head combination on chip, multiply by the receiver's own
// values and accumulate the output; the receiver's dense map never exists.
//
// Portable kernel (any dtype, B, d): one workgroup per (receiver layer,
// row-block, receiver head).  Wave 0 merges the sender heads' sorted column
// lists into their union, one block at a time; the mixed block
// A = sum_h W[r][h] P_h is formed in LDS (fp32) and multiplied by the V tile.
#include "device_common.h"
#include "internal.h"

namespace mf {

namespace {

constexpr int kMapThreads = 256;

template <typename T, int B, int D>
__global__ void __launch_bounds__(kMapThreads) mapped_generic_kernel(MappedArgs a) {
  constexpr int NO = B * D / kMapThreads;   // outputs per thread
  constexpr int QSTEP = kMapThreads / D;    // rows between a thread's outputs
  __shared__ float A[B * B];
  __shared__ float Wr[64];
  __shared__ int64_t vptr[64];
  __shared__ int j_s;
  __shared__ unsigned long long mask_s;

  const int rb = blockIdx.x, r = blockIdx.y, l = blockIdx.z;
  const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, B, rb);
  const int sl = a.layer_map[l];
  const int g = r / (a.Hr / a.Hkv);
  const int tid = threadIdx.x, lane = tid & 63;
  if (tid < a.Hs) Wr[tid] = a.W[((size_t)l * a.Hr + r) * a.Hs + tid];

  int64_t ptr = 0, end = 0;
  if (tid < 64 && lane < a.Hs) {
    const size_t row = ((size_t)sl * a.Hs + lane) * a.b.total_rb + rb;
    ptr = min((int64_t)a.row_ptr[row], a.csr_capacity);
    end = min((int64_t)a.row_ptr[row + 1], a.csr_capacity);
  }
  const T* __restrict__ vals = reinterpret_cast<const T*>(a.values);
  const T* __restrict__ vbase = reinterpret_cast<const T*>(a.v) + (size_t)l * a.lsv;
  const int n = tid % D;
  const int q0 = tid / D;
  float o[NO];
#pragma unroll
  for (int u = 0; u < NO; ++u) o[u] = 0.f;

  for (;;) {
    if (tid < 64) {
      const int cur = (lane < a.Hs && ptr < end) ? a.col_idx[ptr] : 0x7FFFFFFF;
      int jm = cur;
      for (int off = 32; off > 0; off >>= 1) jm = min(jm, __shfl_xor(jm, off, 64));
      const unsigned long long m = __ballot(cur == jm && cur != 0x7FFFFFFF);
      if (cur == jm && cur != 0x7FFFFFFF) {
        vptr[lane] = ptr;
        ++ptr;
      }
      if (lane == 0) { j_s = jm; mask_s = m; }
    }
    __syncthreads();
    const int j = j_s;
    if (j == 0x7FFFFFFF) break;
    const unsigned long long mask = mask_s;
    for (int pos = tid; pos < B * B; pos += kMapThreads) {
      float acc = 0.f;
      unsigned long long mm = mask;
      while (mm) {
        const int h = __builtin_ctzll(mm);
        mm &= mm - 1;
        acc += Wr[h] * to_f32(vals[(size_t)vptr[h] * B * B + pos]);
      }
      A[pos] = acc;
    }
    __syncthreads();
    for (int c = 0; c < B; ++c) {
      const int key = j * B + c;
      if (key >= ri.klen) break;
      const T* vrow;
      if (a.block_table) {
        int64_t page = a.block_table[(size_t)ri.seq * a.max_pages + key / a.page_size];
        page = page < 0 ? 0 : (page >= a.num_pages ? a.num_pages - 1 : page);
        vrow = vbase + (((size_t)page * a.page_size + key % a.page_size) * a.Hkv + g) * D;
      } else {
        vrow = vbase + ((size_t)(ri.k0 + key) * a.Hkv + g) * D;
      }
      const float vv = to_f32(vrow[n]);
#pragma unroll
      for (int u = 0; u < NO; ++u) o[u] += A[(q0 + QSTEP * u) * B + c] * vv;
    }
    __syncthreads();
  }

  T* __restrict__ obase = reinterpret_cast<T*>(a.o) + (size_t)l * a.lso;
#pragma unroll
  for (int u = 0; u < NO; ++u) {
    const int qr = q0 + QSTEP * u;
    if (qr < ri.rows) obase[((size_t)(ri.q0 + qr) * a.Hr + r) * D + n] = from_f32<T>(o[u]);
  }
}

template <typename T, int B, int D>
int launch_g(const MappedArgs& a, void* stream) {
  dim3 grid(a.b.total_rb, a.Hr, a.L);
  hipLaunchKernelGGL((mapped_generic_kernel<T, B, D>), grid, dim3(kMapThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

template <typename T>
int launch_gd(const MappedArgs& a, void* stream) {
  switch (a.B * 1000 + a.d) {
    case 32064: return launch_g<T, 32, 64>(a, stream);
    case 32128: return launch_g<T, 32, 128>(a, stream);
    case 64064: return launch_g<T, 64, 64>(a, stream);
    case 64128: return launch_g<T, 64, 128>(a, stream);
    case 128064: return launch_g<T, 128, 64>(a, stream);
    case 128128: return launch_g<T, 128, 128>(a, stream);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_mapped(const MappedArgs& a, mf_dtype dt, void* stream) {
  if (a.b.total_rb == 0 || a.L == 0) return 0;
  return dt == MF_BF16 ? launch_gd<bf16>(a, stream) : launch_gd<float>(a, stream);
}

}  // namespace mf
