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
#include <stdlib.h>

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

// ---------------------------------------------------------------------------
// bf16, B = 64: transposed score tiles on MFMA 32x32x16.
//
// A workgroup owns up to SQ = 4 consecutive row-blocks of one (layer, head)
// of one sequence, one wave per row-block (64 query rows, Q kept in registers
// as MFMA B operands).  The K column blocks the group needs are streamed
// once through LDS (async global_load_lds, SNST-deep ring, 16-byte chunks
// XOR-swizzled per key row) and read by all four waves, from the group's
// highest diagonal block down to block 0; a wave joins at its own diagonal,
// which is therefore its first block and sets m_ref, as in the portable
// kernel.  Scores are computed transposed, S^T = K Q^T: lane L then holds
// query L % 32 of each 32-query half and 16 keys of each 32-key tile, so a
// row max / row sum over a 64-key block is an in-lane reduction plus one
// v_permlane32_swap with lane L ^ 32.  Only the diagonal block takes a row
// max: it is the exponent reference of every later block of the row, whose
// sums are taken against it directly (a block that would overflow that
// reference is re-taken against its own maximum).  Each block's log2 mass relative to
// m_ref goes to a per-slot scratch table in HBM ([block][row], one coalesced
// 256-byte store per wave and block); the epilogue reads it back through LDS
// transposes and sums the masses in fp64.  The grid is persistent: slot b
// runs on XCD b % 8, takes (layer, head) pairs p = XCD, XCD + 8, ... from
// its XCD's queue (heaviest row-block groups of a pair first), so the K of a
// head stays in one XCD's L2.
// ---------------------------------------------------------------------------
constexpr int SQ = 4;        // row-blocks (waves) per workgroup
constexpr int SNST = 4;      // K ring depth
constexpr int SEPITCH = 65;  // floats per row of an epilogue transpose

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void copy16_to_lds(const void* gsrc, char* lds_generic_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)((uintptr_t)lds_generic_base), 16, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// a copy of a lane value the compiler cannot see through
__device__ __forceinline__ int opaque_int(int x) {
  int y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}

__device__ __forceinline__ float swap32_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Group leaders: row-block rb leads a group when it is the first, fifth, ...
// row-block of its sequence.  One workgroup of 1024 threads writes the
// leaders in ascending order, their count, and clears the per-XCD queues.
__global__ void __launch_bounds__(1024) stats_groups_kernel(BatchArgs b, int32_t* hdr, int32_t* table) {
  __shared__ int wcount[16];
  __shared__ int base;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int c0 = 0; c0 < b.total_rb; c0 += 1024) {
    const int rb = c0 + tid;
    bool lead = false;
    if (rb < b.total_rb) {
      const int s = b.plan[b.num_seqs + 1 + rb];
      lead = ((rb - b.plan[s]) % SQ) == 0;
    }
    const unsigned long long m = __ballot(lead);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wcount[w] = __popcll(m);
    __syncthreads();
    int off = base;
    for (int i = 0; i < w; ++i) off += wcount[i];
    if (lead) table[off + before] = rb;
    __syncthreads();
    if (tid == 0) {
      int t = 0;
      for (int i = 0; i < 16; ++i) t += wcount[i];
      base += t;
    }
    __syncthreads();
  }
  if (tid < kXcds) hdr[tid] = 0;
  if (tid == 0) hdr[kXcds] = base;
}

template <int D>
__global__ void __launch_bounds__(SQ * 64, 2)
stats_mfma_kernel(StatsArgs a, int32_t* hdr, const int32_t* __restrict__ table, float* __restrict__ escratch) {
  constexpr int KS = D / 16;            // MFMA k-steps over the head dim
  constexpr int ROWB = D * 2;           // bytes per key row
  constexpr int CPR = D / 8;            // 16-byte chunks per key row
  constexpr int STAGE = 64 * ROWB;      // one 64-key column block
  constexpr int CPW = STAGE / 1024 / SQ;  // copy instructions per wave per block
  static_assert(CPW >= 1, "stage too small");
  extern __shared__ __align__(16) char smem[];
  __shared__ int item_sh;

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int xcd = blockIdx.x % kXcds;
  const int ngroups = hdr[kXcds];
  const long long pairs = (long long)a.L * a.H;
  const long long npx = pairs > xcd ? (pairs - xcd + kXcds - 1) / kXcds : 0;
  const long long nitems = npx * ngroups;
  const float c2 = (float)(a.scale * kLog2eD);
  const double c2d = a.scale * kLog2eD;
  float* __restrict__ ew = escratch + ((size_t)blockIdx.x * SQ + w) * 64 * a.b.max_cb;  // [block][row]
  const size_t kstride = (size_t)a.Hkv * D;

  for (;;) {
    if (threadIdx.x == 0) item_sh = atomicAdd(&hdr[xcd], 1);
    __syncthreads();
    // wave-uniform: every lane read the same word (readfirstlane lets the
    // compiler keep the item's addresses and block offsets in scalar registers)
    const long long item = __builtin_amdgcn_readfirstlane(item_sh);
    __syncthreads();
    if (item >= nitems) break;
    const long long p = xcd + (long long)kXcds * (item / ngroups);
    const int lead = table[ngroups - 1 - (int)(item % ngroups)];
    const int l = (int)(p / a.H), h = (int)(p % a.H);
    const int hk = h / (a.H / a.Hkv);
    const int seq = a.b.plan[a.b.num_seqs + 1 + lead];
    const int last_rb = min(lead + SQ - 1, a.b.plan[seq + 1] - 1);
    const RowBlockInfo rlast = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, 64, last_rb);
    const int jtop = rlast.ncand - 1;
    const int rb = lead + w;
    const bool valid = rb <= last_rb;
    const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, 64,
                                          valid ? rb : last_rb);
    const int diag = valid ? ri.ncand - 1 : -1;

    const bf16* __restrict__ kbase = reinterpret_cast<const bf16*>(a.k) + (size_t)l * a.lsk +
                                     (size_t)rlast.k0 * kstride + (size_t)hk * D;
    const int klast = rlast.klen - 1;

    // copies of column block jtop - t into ring slot t % SNST (steps past the
    // end re-read block 0 so every wave issues the same number of copies)
    // copy slot i of this wave: key kkey[i] of the block, source chunk
    // csrc[i]; its source for block jb is kptr[i] + jb * 64 rows
    const bf16* kptr[CPW];
    int kkey[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int pidx = (i * SQ + w) * 64 + lane;  // 16-byte chunk index in the stage
      const int key = pidx / CPR, cc = pidx % CPR;
      const int src_chunk = cc ^ (key & (CPR - 1));
      kkey[i] = key;
      kptr[i] = kbase + (size_t)key * kstride + src_chunk * 8;
    }
    auto issue = [&](int t) {
      const int jb = max(jtop - t, 0);
      char* stage = smem + (t % SNST) * STAGE;
      if (jb * 64 + 63 <= klast) {
        const size_t step = (size_t)jb * 64 * kstride;
#pragma unroll
        for (int i = 0; i < CPW; ++i) copy16_to_lds(kptr[i] + step, stage + (i * SQ + w) * 1024);
      } else {
        // block reaching past the last key: clamp rows to the last key
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
          const int over = max(jb * 64 + kkey[i] - klast, 0);
          copy16_to_lds(kptr[i] + ((size_t)jb * 64 - over) * kstride, stage + (i * SQ + w) * 1024);
        }
      }
    };
#pragma unroll
    for (int t = 0; t < SNST - 1; ++t) issue(t);

    // Q of this wave's 64 rows as B operands: lane L -> row 32 qt + L % 32,
    // head-dim slice 16 ks + 8 (L / 32) .. + 7
    bf16x8 qf[2][KS];
    {
      const bf16* __restrict__ qbase = reinterpret_cast<const bf16*>(a.q) + (size_t)l * a.lsq;
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int r = 32 * qt + l32;
        const bool ok = valid && r < ri.rows;
        const bf16* src = qbase + ((size_t)(ri.q0 + (ok ? r : 0)) * a.H + h) * D + 8 * hi;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          bf16x8 v = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
          if (!ok) v = bf16x8{};
          qf[qt][ks] = v;
        }
      }
    }

    float m_ref[2] = {0.f, 0.f}, m_run[2] = {0.f, 0.f};
    // (m_run - m_ref) c2 in log2 units, rounded once from fp64; it changes
    // only when a block overflows the reference
    float eoff[2] = {0.f, 0.f};
    double l_run[2] = {1.0, 1.0};

    for (int t = 0; t <= jtop; ++t) {
      switch (min(t, SNST - 1)) {
        case 0: wait_vmcnt<(SNST - 2) * CPW + 0>(); break;
        case 1: wait_vmcnt<(SNST - 2) * CPW + 1>(); break;
        case 2: wait_vmcnt<(SNST - 2) * CPW + 2>(); break;
        default: wait_vmcnt<(SNST - 2) * CPW + 3>(); break;
      }
      __syncthreads();
      issue(t + SNST - 1);
      const int jb = jtop - t;
      float ev = 0.f;
      if (jb <= diag) {
        const char* stage = smem + (t % SNST) * STAGE;
        f32x16 acc[2][2];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) acc[kt][qt] = f32x16{};
        // K fragment (kt, ks) of lane L: key 32 kt + L % 32, head-dim slice
        // 16 ks + 8 (L / 32); read two fragments ahead of the MFMAs using them
        auto kfrag = [&](int idx) {
          const int kt = idx & 1, ks = idx >> 1;
          const int key = 32 * kt + l32;
          const int chunk = (2 * ks + hi) ^ (key & (CPR - 1));
          return *reinterpret_cast<const bf16x8*>(stage + key * ROWB + chunk * 16);
        };
        bf16x8 kf0 = kfrag(0), kf1 = kfrag(1);
#pragma unroll
        for (int idx = 0; idx < 2 * KS; ++idx) {
          const int kt = idx & 1, ks = idx >> 1;
          const bf16x8 kf2 = idx + 2 < 2 * KS ? kfrag(idx + 2) : kf0;
          acc[kt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[0][ks], acc[kt][0], 0, 0, 0);
          acc[kt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf0, qf[1][ks], acc[kt][1], 0, 0, 0);
          kf0 = kf1;
          kf1 = kf2;
        }
        // per row: its sum over the block relative to the reference m_run,
        // both 32-key halves (in-lane) and both lane halves (one swap)
        auto block_sum = [&](int qt, float nb) {
          float s0 = 0.f, s1 = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            s0 += __builtin_amdgcn_exp2f(fmaf(acc[0][qt][e], c2, -nb));
            s1 += __builtin_amdgcn_exp2f(fmaf(acc[1][qt][e], c2, -nb));
          }
          return swap32_sum(s0 + s1);
        };
        auto block_max = [&](int qt) {
          float mx = acc[0][qt][0];
#pragma unroll
          for (int e = 1; e < 16; ++e) mx = fmaxf(mx, acc[0][qt][e]);
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[1][qt][e]);
          return swap32_max(mx);
        };
        float evq[2];
        if (jb == diag) {
          asm volatile("");  // a real branch: this runs once per row-block
          // causal mask inside the diagonal block, key index > query index:
          // tile (kt = 1, qt = 0) lies wholly above the diagonal, (0, 1)
          // wholly below; in the two diagonal tiles register e holds key
          // 8 (e / 4) + 4 (L / 32) + e % 4 against query L % 32.  The lane
          // offset is re-derived here so the 32 predicates are not hoisted
          // out of the block loop.
          const int t = opaque_int(l32 - 4 * hi);
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const bool masked = 8 * (e >> 2) + (e & 3) > t;
            acc[0][0][e] = masked ? -INFINITY : acc[0][0][e];
            acc[1][1][e] = masked ? -INFINITY : acc[1][1][e];
            acc[1][0][e] = -INFINITY;
          }
          // the diagonal block's maximum is the reference of the row's
          // log2 masses; s lies in [1, 64], where the hardware log2 is
          // exact to an ulp
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            const float mx = block_max(qt);
            const float s = block_sum(qt, mx * c2);
            m_ref[qt] = m_run[qt] = mx;
            eoff[qt] = 0.f;
            l_run[qt] = (double)s;
            evq[qt] = __builtin_amdgcn_logf(s);
          }
        } else {
          // Off the diagonal the exponent reference stays m_run; no block
          // maximum is needed unless a score exceeds it so far that the
          // sum leaves [0, 2^64) (overflow, or NaN from an infinite score).
          // Then the wave re-takes the block with its maximum folded in.
          float s[2];
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) s[qt] = block_sum(qt, m_run[qt] * c2);
          const bool big = !(s[0] < 0x1p64f) || !(s[1] < 0x1p64f);
          if (__builtin_expect(__ballot(big) != 0, 0)) {
            asm volatile("");
#pragma unroll
            for (int qt = 0; qt < 2; ++qt) {
              const float m_new = fmaxf(m_run[qt], block_max(qt));
              l_run[qt] *= (double)__builtin_amdgcn_exp2f((m_run[qt] - m_new) * c2);
              m_run[qt] = m_new;
              eoff[qt] = (float)(((double)m_new - (double)m_ref[qt]) * c2d);
              s[qt] = block_sum(qt, m_new * c2);
            }
          }
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            l_run[qt] += (double)s[qt];
            evq[qt] = __builtin_amdgcn_logf(s[qt]) + eoff[qt];
          }
        }
        ev = hi ? evq[1] : evq[0];
      }
      ew[(size_t)jb * 64 + lane] = ev;  // row `lane` of block jb (unused when inactive)
    }

    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the K ring: LDS becomes the transposes
    if (valid) {
      // lane L keeps query row L: half L / 32 of the wave's two 32-row halves
      const float mr = hi ? m_ref[1] : m_ref[0];
      const float mu = hi ? m_run[1] : m_run[0];
      const double lr = hi ? l_run[1] : l_run[0];
      const double lse2 = ((double)mu - (double)mr) * c2d + log2(lr);
      const size_t lh = (size_t)l * a.H + h;
      if (lane < ri.rows)
        a.row_lse[lh * a.b.total_q + ri.q0 + lane] = (float)((double)mr * a.scale + lse2 * kLn2);
      float* tr = reinterpret_cast<float*>(smem) + w * 64 * SEPITCH;
      float* __restrict__ bm = a.block_mass + (lh * a.b.total_rb + rb) * (size_t)a.b.max_cb;
      for (int j0 = 0; j0 < ri.ncand; j0 += 64) {
        const int nj = min(64, ri.ncand - j0);
        // the scratch rows were written by this wave on this CU and its
        // stores have completed: plain loads see them.  Eight in flight.
        for (int jj = 0; jj < nj; jj += 8) {
          float e[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) e[u] = ew[(size_t)min(j0 + jj + u, ri.ncand - 1) * 64 + lane];
#pragma unroll
          for (int u = 0; u < 8; ++u)
            if (jj + u < nj) tr[(jj + u) * SEPITCH + lane] = lane < ri.rows ? exp2f((float)((double)e[u] - lse2)) : 0.f;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        if (lane < nj) {
          double accm = 0.0;
          for (int r = 0; r < ri.rows; ++r) accm += (double)tr[lane * SEPITCH + r];
          bm[j0 + lane] = (float)(accm / ri.rows);
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      }
      for (int j = ri.ncand + lane; j < a.b.max_cb; j += 64) bm[j] = 0.f;
    }
  }
}

}  // namespace

size_t block_stats_lds_bytes(int B, int max_cb) {
  const size_t ecols = (size_t)(max_cb | 1);
  return ((size_t)B * ecols * 4 + 15) / 16 * 16 + (size_t)B * 8;
}

bool stats_fast_path(mf_dtype dt, int B, int d) {
  if (dt != MF_BF16 || B != 64 || (d != 64 && d != 128)) return false;
  const char* env = getenv("MF_PORTABLE_STATS");
  return !(env && env[0] == '1');
}

static size_t stats_mfma_lds_bytes(int d) {
  const size_t ring = (size_t)SNST * 64 * d * 2;
  const size_t tr = (size_t)SQ * 64 * SEPITCH * 4;
  return ring > tr ? ring : tr;
}

StatsWorkspace stats_workspace_layout(int B, int max_cb, int total_rb, int slots) {
  StatsWorkspace w;
  w.hdr = 0;
  w.table = 256;
  w.escratch = w.table + ((size_t)total_rb * 4 + 255) / 256 * 256;
  w.slots = slots;
  w.bytes = w.escratch + (size_t)slots * SQ * B * (size_t)max_cb * 4;
  return w;
}

int stats_slots(int num_cus) { return 2 * num_cus; }

int launch_block_stats(const StatsArgs& a, mf_dtype dt, void* stream) {
  if (a.b.total_rb == 0 || a.L == 0) return 0;
  if (a.ws) {
    char* ws = static_cast<char*>(a.ws);
    int32_t* hdr = reinterpret_cast<int32_t*>(ws + a.wsl.hdr);
    int32_t* table = reinterpret_cast<int32_t*>(ws + a.wsl.table);
    float* escr = reinterpret_cast<float*>(ws + a.wsl.escratch);
    hipLaunchKernelGGL(stats_groups_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, a.b, hdr, table);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const size_t lds = stats_mfma_lds_bytes(a.d);
    auto kern = a.d == 128 ? stats_mfma_kernel<128> : stats_mfma_kernel<64>;
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(kern, dim3(a.wsl.slots), dim3(SQ * 64), lds, (hipStream_t)stream, a, hdr, table, escr);
    return (int)hipGetLastError();
  }
  return dt == MF_BF16 ? launch_d<bf16>(a, stream) : launch_d<float>(a, stream);
}

}  // namespace mf
