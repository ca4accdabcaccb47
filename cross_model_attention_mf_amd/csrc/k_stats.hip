// Stage 1 of the staged block compression: block-level attention statistics
// straight from the sender's Q and K (MapFlow page, section "让复用真正省时…",
// paragraph "第一": statistics first, then extraction, never the dense map).
//
// One workgroup per (layer, sender head, query row-block of B rows), B/16
// waves, each wave owning 16 query rows.  The row-block's causal column
// blocks are visited once, diagonal block first, then 0 .. diag-1:
//   S = Q_rows K_cols^T           bf16 MFMA 16x16x32 (fp32: 16x16x4), fp32 acc
//   m_run = running row max       (m_ref = max of the diagonal block)
//   s_rj  = sum_c exp2((S - m_run) * c2)        c2 = scale * log2(e)
//   E[r][j] = log2(s_rj) + (m_run - m_ref) * c2  (log2 mass relative to m_ref)
//   l_run = online sum of the s_rj (fp64)
// E lives in LDS (B x ncand floats).  Epilogue: per row
//   lse2_r = (m_run - m_ref) * c2 + log2(l_run)     (fp64)
//   row_lse_r = scale * m_ref + ln2 * lse2_r
// and per column block, in fp64, mass_j = sum_r exp2(E[r][j] - lse2_r) / R.
// Keeping E relative to the diagonal block's maximum keeps the important
// blocks' log-masses small in magnitude, so fp32 holds them to ~1e-7.
#include "device_common.h"
#include "internal.h"

namespace mf {

namespace {

template <typename T, int B, int D>
__global__ void __launch_bounds__(B * 4)
block_stats_kernel(StatsArgs a) {
  constexpr int NT = B / 16;  // 16-column tiles per column block
  extern __shared__ __align__(16) char smem[];
  const int ecols = a.b.max_cb | 1;  // odd row stride: no bank conflicts
  float* E = reinterpret_cast<float*>(smem);
  double* LSE = reinterpret_cast<double*>(smem + ((size_t)B * ecols * 4 + 15) / 16 * 16);

  int rbi, h, l;
  xcd_unflatten(blockIdx.x, a.b.total_rb, a.H, a.L, rbi, h, l);
  if (l >= a.L) return;
  // heaviest (latest) row-blocks first: causal work grows with position
  const int rb = a.b.total_rb - 1 - rbi;
  const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, B, rb);
  const int hk = h / (a.H / a.Hkv);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int lr = lane & 15, lg = lane >> 4;

  const T* __restrict__ qbase = reinterpret_cast<const T*>(a.q) + (size_t)l * a.lsq;
  const T* __restrict__ kbase = reinterpret_cast<const T*>(a.k) + (size_t)l * a.lsk +
                                (size_t)ri.k0 * a.Hkv * D + (size_t)hk * D;
  const size_t kstride = (size_t)a.Hkv * D;

  QFrag<T, D> qf;
  {
    const int r = min(16 * w + lr, ri.rows - 1);
    qf.load(qbase + ((size_t)(ri.q0 + r) * a.H + h) * D, lane);
  }

  const float c2 = (float)(a.scale * kLog2eD);
  const double c2d = a.scale * kLog2eD;
  const int diag = ri.ncand - 1;
  int rowl[4];
  bool rowok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rowl[i] = 16 * w + 4 * lg + i;
    rowok[i] = rowl[i] < ri.rows;
  }
  float m_ref[4], m_run[4];
  double l_run[4];

  for (int t = 0; t < ri.ncand; ++t) {
    const int j = (t == 0) ? diag : t - 1;
    f32x4 acc[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int c = min(j * B + 16 * nt + lr, ri.klen - 1);
      acc[nt] = qf.dot(kbase + (size_t)c * kstride, lane, acc[nt]);
    }
    // causal mask: only the diagonal block can hold keys past a row
    bool valid[NT][4];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        valid[nt][i] = rowok[i] && (j * B + 16 * nt + lr <= ri.pos0 + rowl[i]);

    float Ev[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float mx = -INFINITY;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) mx = valid[nt][i] ? fmaxf(mx, acc[nt][i]) : mx;
      mx = row16_max(mx);
      const float m_new = (t == 0) ? mx : fmaxf(m_run[i], mx);
      float s = 0.f;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) s += valid[nt][i] ? exp2f((acc[nt][i] - m_new) * c2) : 0.f;
      s = row16_sum(s);
      if (t == 0) {
        m_ref[i] = m_new;
        l_run[i] = (double)s;
        Ev[i] = log2f(s);
      } else {
        if (m_new > m_run[i]) l_run[i] *= (double)exp2f((m_run[i] - m_new) * c2);
        l_run[i] += (double)s;
        Ev[i] = log2f(s) + (float)(((double)m_new - (double)m_ref[i]) * c2d);
      }
      m_run[i] = m_new;
    }
    // lane lr (< 4) of each 16-lane row writes row 4*lg + lr of the wave
    if (lr < 4) {
      const float ev = lr == 0 ? Ev[0] : lr == 1 ? Ev[1] : lr == 2 ? Ev[2] : Ev[3];
      E[(16 * w + 4 * lg + lr) * ecols + j] = ev;
    }
  }

  const size_t lh = (size_t)l * a.H + h;
  if (lr < 4) {
    const int i = lr;
    const float mr = i == 0 ? m_ref[0] : i == 1 ? m_ref[1] : i == 2 ? m_ref[2] : m_ref[3];
    const float mu = i == 0 ? m_run[0] : i == 1 ? m_run[1] : i == 2 ? m_run[2] : m_run[3];
    const double lr_ = i == 0 ? l_run[0] : i == 1 ? l_run[1] : i == 2 ? l_run[2] : l_run[3];
    const int row = 16 * w + 4 * lg + i;
    if (row < ri.rows) {
      const double lse2 = ((double)mu - (double)mr) * c2d + log2(lr_);
      LSE[row] = lse2;
      a.row_lse[lh * a.b.total_q + ri.q0 + row] = (float)((double)mr * a.scale + lse2 * kLn2);
    }
  }
  __syncthreads();

  float* __restrict__ bm = a.block_mass + (lh * a.b.total_rb + rb) * (size_t)a.b.max_cb;
  for (int j = threadIdx.x; j < a.b.max_cb; j += B * 4) {
    float out = 0.f;
    if (j < ri.ncand) {
      double accm = 0.0;
      for (int r = 0; r < ri.rows; ++r)
        accm += (double)exp2f((float)((double)E[r * ecols + j] - LSE[r]));
      out = (float)(accm / ri.rows);
    }
    bm[j] = out;
  }
}

template <typename T, int B, int D>
int launch_t(const StatsArgs& a, void* stream) {
  const size_t lds = block_stats_lds_bytes(B, a.b.max_cb);
  auto kern = block_stats_kernel<T, B, D>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return (int)e;
  dim3 grid(xcd_grid(a.b.total_rb, a.H, a.L));
  hipLaunchKernelGGL(kern, grid, dim3(B * 4), lds, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

template <typename T>
int launch_d(const StatsArgs& a, void* stream) {
  switch (a.B * 1000 + a.d) {
    case 32064: return launch_t<T, 32, 64>(a, stream);
    case 32128: return launch_t<T, 32, 128>(a, stream);
    case 64064: return launch_t<T, 64, 64>(a, stream);
    case 64128: return launch_t<T, 64, 128>(a, stream);
    case 128064: return launch_t<T, 128, 64>(a, stream);
    case 128128: return launch_t<T, 128, 128>(a, stream);
  }
  return (int)hipErrorInvalidValue;
}

}  // namespace

size_t block_stats_lds_bytes(int B, int max_cb) {
  const size_t ecols = (size_t)(max_cb | 1);
  return ((size_t)B * ecols * 4 + 15) / 16 * 16 + (size_t)B * 8;
}

int launch_block_stats(const StatsArgs& a, mf_dtype dt, void* stream) {
  if (a.b.total_rb == 0 || a.L == 0) return 0;
  return dt == MF_BF16 ? launch_d<bf16>(a, stream) : launch_d<float>(a, stream);
}

}  // namespace mf
