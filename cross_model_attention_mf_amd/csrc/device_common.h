// Device helpers shared by the gfx950 kernels: MFMA operand types, row
// reductions inside 16-lane DPP rows, and the row-block lookup of a packed
// (varlen, chunked) batch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mf {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2 = 0.6931471805599453;
constexpr double kLog2eD = 1.4426950408889634;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// ---------------------------------------------------------------------------
// Reductions over the 16 lanes of a DPP row (lanes 16g .. 16g+15).  After the
// call every lane of the row holds the same result (max and + are
// commutative, so each lane combines the same operands).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp_f<0xB1>(x));
  x = fmaxf(x, dpp_f<0x4E>(x));
  x = fmaxf(x, dpp_f<0x141>(x));
  x = fmaxf(x, dpp_f<0x140>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x = x + dpp_f<0xB1>(x);
  x = x + dpp_f<0x4E>(x);
  x = x + dpp_f<0x141>(x);
  x = x + dpp_f<0x140>(x);
  return x;
}

// ---------------------------------------------------------------------------
// Packed batch: row-block rb of the plan -> sequence, rows, positions.
// plan = [rb_start[0..S], rb_seq[0..total_rb)].
// ---------------------------------------------------------------------------
struct RowBlockInfo {
  int seq;      // packed sequence
  int q0;       // first packed query row of the block
  int rows;     // valid rows (<= B)
  int pos0;     // absolute position of the first row
  int k0;       // first packed key of the sequence
  int klen;     // keys of the sequence
  int ncand;    // causal column blocks: 0 .. (pos0 + rows - 1) / B
};

__device__ __forceinline__ RowBlockInfo rowblock_info(const int32_t* __restrict__ plan, int num_seqs,
                                                      const int32_t* __restrict__ cu_q,
                                                      const int32_t* __restrict__ cu_k,
                                                      const int32_t* __restrict__ q_pos0, int B, int rb) {
  RowBlockInfo r;
  const int s = plan[num_seqs + 1 + rb];
  const int local = rb - plan[s];
  const int qs = cu_q[s], qe = cu_q[s + 1];
  r.seq = s;
  r.q0 = qs + local * B;
  r.rows = min(B, qe - r.q0);
  r.pos0 = (q_pos0 ? q_pos0[s] : 0) + local * B;
  r.k0 = cu_k[s];
  r.klen = cu_k[s + 1] - r.k0;
  r.ncand = (r.pos0 + r.rows - 1) / B + 1;
  return r;
}

// ---------------------------------------------------------------------------
// XCD-aware work order.  Workgroups are dealt round-robin to the 8 XCDs
// (linear id n runs on XCD n % 8), and each XCD has its own L2.  Work items
// (rb fastest, then h, then l) are cut into 8 contiguous ranges, one per XCD,
// so the row-blocks of one (layer, head) run together on one XCD and share
// its L2 for K.  Linear ids past the end of the work return l = L (exit).
// ---------------------------------------------------------------------------
constexpr int kXcds = 8;

__host__ __device__ inline unsigned xcd_grid(int nrb, int H, int L) {
  const long long n = (long long)nrb * H * L;
  const long long per = (n + kXcds - 1) / kXcds;
  return (unsigned)(per * kXcds);
}

__device__ __forceinline__ void xcd_unflatten(unsigned bid, int nrb, int H, int L, int& rb, int& h, int& l) {
  const long long n = (long long)nrb * H * L;
  const long long per = (n + kXcds - 1) / kXcds;
  const long long item = (long long)(bid % kXcds) * per + bid / kXcds;
  if (item >= n) { rb = 0; h = 0; l = L; return; }
  rb = (int)(item % nrb);
  const long long t = item / nrb;
  h = (int)(t % H);
  l = (int)(t / H);
}

// ---------------------------------------------------------------------------
// MFMA score tile: S[16 rows x 16 cols] = Q_rows . K_cols^T over D.
// Lane L of a wave supplies row/col L%16 and the k-slice selected by L/16;
// the output holds S[4*(L/16)+i][L%16] in element i (checked on gfx950).
// ---------------------------------------------------------------------------
template <typename T, int D> struct QFrag;

template <int D> struct QFrag<bf16, D> {
  static constexpr int KS = D / 32;
  bf16x8 a[KS];
  __device__ __forceinline__ void load(const bf16* __restrict__ row, int lane) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      a[ks] = *reinterpret_cast<const bf16x8*>(row + 32 * ks + 8 * (lane >> 4));
  }
  __device__ __forceinline__ f32x4 dot(const bf16* __restrict__ krow, int lane, f32x4 acc) const {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 b = *reinterpret_cast<const bf16x8*>(krow + 32 * ks + 8 * (lane >> 4));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ks], b, acc, 0, 0, 0);
    }
    return acc;
  }
};

template <int D> struct QFrag<float, D> {
  static constexpr int KS = D / 4;
  float a[KS];
  __device__ __forceinline__ void load(const float* __restrict__ row, int lane) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) a[ks] = row[4 * ks + (lane >> 4)];
  }
  __device__ __forceinline__ f32x4 dot(const float* __restrict__ krow, int lane, f32x4 acc) const {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[ks], krow[4 * ks + (lane >> 4)], acc, 0, 0, 0);
    return acc;
  }
};

}  // namespace mf
