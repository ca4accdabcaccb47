// Stage 1 of the staged block compression: block-level attention statistics
// straight from the sender's Q and K (MapFlow page, section "让复用真正省时…",
// paragraph "第一": statistics first, then extraction, never the dense map).
//
// One workgroup per (layer, sender head, query row-block of B rows), B/16
// waves, each wave owning 16 query rows.  The row-block's causal column
// blocks are visited once, diagonal block first, then 0 .. diag-1:
//   S = Q_rows K_cols^T           bf16 MFMA 16x16x32 (fp32: 16x16x4), fp32 acc
//   m_run = running row max
//   s_rj  = sum_c exp2((S - m_run) * c2)        c2 = scale * log2(e)
//   E[r][j] = log2(s_rj) + (m_run - m_ref) * c2  (log2 mass relative to m_ref)
//   l_run = online sum of the s_rj (fp64)
// m_ref starts as the diagonal block's maximum; when m_run passes it by more
// than kRebase log2 units the row's stored E move to m_ref = m_run (in fp64).
// E thus stays below log2(B) + kRebase in magnitude wherever the mass is not
// negligible, where the fp32 E (and the hardware log2) are good to ~1e-6
// relative in the mass.  E lives in LDS (B x ncand floats).  Epilogue: per row
//   lse2_r = (m_run - m_ref) * c2 + log2(l_run)     (fp64)
//   row_lse_r = scale * m_ref + ln2 * lse2_r
// and per column block, in fp64, mass_j = sum_r exp2(E[r][j] - lse2_r) / R.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace mf {

namespace {

template <int N>
using IC = std::integral_constant<int, N>;

constexpr double kRebase = 8.0;

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
        double off = ((double)m_new - (double)m_ref[i]) * c2d;
        if (off > kRebase) {
          // the row's earlier blocks (the diagonal, then 0 .. j - 1), written
          // by this lane, move to the new reference
          if (lr == i && rowok[i]) {
            float* Er = E + (size_t)rowl[i] * ecols;
            for (int tp = 0; tp < t; ++tp) {
              float* e = Er + (tp == 0 ? diag : tp - 1);
              *e = (float)((double)*e - off);
            }
          }
          m_ref[i] = m_new;
          off = 0.0;
        }
        Ev[i] = log2f(s) + (float)off;
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
// max: it is the exponent reference m_run of every later block of the row,
// whose sums are taken against it directly; a 32-key half with a score more
// than 13 log2 units above it moves m_run to the half's maximum and is taken
// again.  Off the diagonal a block runs in two 32-key halves, software-
// pipelined so that the matrix pipe computes one half's scores while the
// vector pipe sums the half before it.  Each block's log2 mass relative to
// m_run goes to a per-slot scratch table in HBM ([block][row], one coalesced
// 256-byte store per wave and block; when m_run moves, the wave shifts the
// entries it already stored, in fp64); the epilogue reads it back through
// LDS transposes and sums the masses in fp64.  The grid is persistent: slot b
// runs on XCD b % 8, takes (layer, head) pairs p = XCD, XCD + 8, ... from
// its XCD's queue (heaviest row-block groups of a pair first), so the K of a
// head stays in one XCD's L2.
// ---------------------------------------------------------------------------
constexpr int SQ = 4;        // row-blocks (waves) per workgroup
// K rows of one sequence are addressed by 32-bit byte offsets from its first
// key row (at most MF_MAX_KEYS keys of at most 64 heads x 128 dims, bf16)
static_assert((unsigned long long)MF_MAX_KEYS * 64 * 128 * 2 < (1ull << 32), "32-bit K row offsets");
constexpr int SNST = 4;      // K ring depth
constexpr int SEPITCH = 65;  // floats per row of an epilogue transpose

typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ void copy16_to_lds(const void* gsrc, char* lds_generic_base) {
  __builtin_amdgcn_global_load_lds(gsrc, (lds_void_t*)((uintptr_t)lds_generic_base), 16, 0, 0);
}
// 16 bytes per lane from a scalar base plus a 32-bit lane offset into LDS at
// m0 + 16 * lane.  Inline assembly (the compiler neither counts it nor
// orders LDS accesses against it beyond the memory clobber: the kernel's own
// counted waits and barriers do); one wait state between the M0 write and
// the copy reading it.
__device__ __forceinline__ void copy16_saddr(unsigned voff, const void* sbase, unsigned m0) {
  // the base is uniform; pin it in scalar registers (a value the compiler
  // keeps in vector registers is not moved for an "s" operand by itself)
  const uint64_t v = (uint64_t)(uintptr_t)sbase;
  // (readfirstlane returns int: through unsigned, so the low word does not
  // sign-extend into the high one)
  const uint64_t lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)v);
  const uint64_t hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  const void* sb = reinterpret_cast<const void*>((uintptr_t)((hi << 32) | lo));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(sb), "s"(m0)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ unsigned lds_addr(const char* lds_generic) {
  return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_generic);
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

// Group leaders over 64-row units (unit u is half u % sub of row-block
// u / sub; sub = B / 64): unit u leads a group when it is the first, fifth,
// ... unit of its sequence.  One workgroup of 1024 threads writes the leaders
// in ascending order, their count, and clears the per-XCD queues.
__global__ void __launch_bounds__(1024) stats_groups_kernel(BatchArgs b, int sub, int32_t* hdr, int32_t* table) {
  __shared__ int wcount[16];
  __shared__ int base;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  if (tid == 0) base = 0;
  __syncthreads();
  const int nunits = b.total_rb * sub;
  for (int c0 = 0; c0 < nunits; c0 += 1024) {
    const int rb = c0 + tid;
    bool lead = false;
    if (rb < nunits) {
      const int s = b.plan[b.num_seqs + 1 + rb / sub];
      lead = ((rb - sub * b.plan[s]) % SQ) == 0;
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

// 64-row unit u of a batch of SUB * 64-row row-blocks: half u % SUB of
// row-block u / SUB, with its own rows, positions and 64-key causal range
// (rows = 0 for the empty second half of a short last row-block)
template <int SUB>
__device__ __forceinline__ RowBlockInfo unit_info(const BatchArgs& b, int u) {
  RowBlockInfo r = rowblock_info(b.plan, b.num_seqs, b.cu_q, b.cu_k, b.q_pos0, 64 * SUB, u / SUB);
  if constexpr (SUB > 1) {
    const int half = u % SUB;
    r.q0 += 64 * half;
    r.pos0 += 64 * half;
    r.rows = max(0, min(64, r.rows - 64 * half));
    r.ncand = r.rows > 0 ? (r.pos0 + r.rows - 1) / 64 + 1 : 0;
  }
  return r;
}

template <int D, int SUB>
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
  const int max_cb64 = a.b.max_cb * SUB;   // 64-key blocks
  float* __restrict__ ew = escratch + ((size_t)blockIdx.x * SQ + w) * 64 * max_cb64;  // [block][row]
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
    const int seq = a.b.plan[a.b.num_seqs + 1 + lead / SUB];
    int last_rb = min(lead + SQ - 1, SUB * a.b.plan[seq + 1] - 1);
    RowBlockInfo rlast = unit_info<SUB>(a.b, last_rb);
    if (SUB > 1 && rlast.rows == 0) rlast = unit_info<SUB>(a.b, --last_rb);   // empty second half
    const int jtop = rlast.ncand - 1;
    const int rb = lead + w;
    const bool valid = rb <= last_rb;
    const RowBlockInfo ri = unit_info<SUB>(a.b, valid ? rb : last_rb);
    const int diag = valid ? ri.ncand - 1 : -1;

    const bf16* __restrict__ kbase = reinterpret_cast<const bf16*>(a.k) + (size_t)l * a.lsk +
                                     (size_t)rlast.k0 * kstride + (size_t)hk * D;
    const int klast = rlast.klen - 1;

    // copies of column block jtop - t into ring slot t % SNST (steps past the
    // end re-read block 0 so every wave issues the same number of copies).
    // Copy i of this wave: key kkey[i] of the block, source chunk
    // cc ^ (key % CPR) at byte offset koff[i] from the block's first key row,
    // whose address is scalar.
    unsigned koff[CPW];
    int kkey[CPW];
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int pidx = (i * SQ + w) * 64 + lane;  // 16-byte chunk index in the stage
      const int key = pidx / CPR, cc = pidx % CPR;
      const int src_chunk = cc ^ (key & (CPR - 1));
      kkey[i] = key;
      koff[i] = (unsigned)(((size_t)key * kstride + src_chunk * 8) * 2);
    }
    const char* kbytes = reinterpret_cast<const char*>(kbase);
    auto issue = [&](int t) {
      const int jb = max(jtop - t, 0);
      const char* src = kbytes + (size_t)jb * 64 * kstride * 2;
      const unsigned m0 = lds_addr(smem + (t % SNST) * STAGE + w * 1024);
      if (jb * 64 + 63 <= klast) {
#pragma unroll
        for (int i = 0; i < CPW; ++i) copy16_saddr(koff[i], src, m0 + i * SQ * 1024);
      } else {
        // block reaching past the last key: each row's key clamped to the
        // last key, addressed from the sequence's first key row (scalar)
#pragma unroll
        for (int i = 0; i < CPW; ++i) {
          const unsigned chb = koff[i] - (unsigned)((size_t)kkey[i] * kstride * 2);   // the chunk's byte offset in its row
          const int kk = min(jb * 64 + kkey[i], klast);
          // below 2^32: a sequence has at most MF_MAX_KEYS keys of at most 64 heads x 128 dims
          copy16_saddr((unsigned)((size_t)kk * kstride * 2) + chb, kbytes, m0 + i * SQ * 1024);
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
    double l_run[2] = {1.0, 1.0};

    // K fragment (kt, ks) of lane L in the block staged at `stage`: key
    // 32 kt + L % 32, head-dim slice 16 ks + 8 (L / 32), at kfo[ks] +
    // 32 kt ROWB (key % CPR, which picks the chunk swizzle, is the same for
    // both kt), so with the stage's slot known at compile time each read is
    // one LDS instruction with an immediate offset
    // (opaque, so that the compiler keeps the KS sums instead of re-adding
    // their common part at every read)
    typedef __attribute__((address_space(3))) const char lds_char;
    int kfo[KS];   // LDS byte addresses
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kfo[ks] = opaque_int((int)lds_addr(smem) + l32 * ROWB + (((2 * ks + hi) ^ (l32 & (CPR - 1))) * 16));
    // soff: the stage's byte offset in the ring
    auto kfrag = [&](int soff, int kt, int ks) {
      lds_char* p = reinterpret_cast<lds_char*>((uintptr_t)(unsigned)kfo[ks]);
      return *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(p + soff + 32 * kt * ROWB);
    };
    // transposed scores of the 32-key half kt of a block:
    // acc[kt][qt] = K[32 kt .. + 31] Q[32 qt .. + 31]^T
    f32x16 acc[2][2];
    auto mfma_half = [&](int soff, int kt) __attribute__((always_inline)) {
      bf16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) kf[ks] = kfrag(soff, kt, ks);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        acc[kt][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[0][ks], ks ? acc[kt][0] : f32x16{}, 0, 0, 0);
        acc[kt][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[1][ks], ks ? acc[kt][1] : f32x16{}, 0, 0, 0);
      }
    };
    // in-lane sums of exp2(s c2 - nb) over half kt's 16 keys of each query
    // tile (the lane's partner L ^ 32 holds the other 16)
    auto half_sum = [&](int kt, const float (&nb)[2], float (&part)[2]) __attribute__((always_inline)) {
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float a0 = __builtin_amdgcn_exp2f(fmaf(acc[kt][qt][0], c2, -nb[qt]));
        float a1 = __builtin_amdgcn_exp2f(fmaf(acc[kt][qt][1], c2, -nb[qt]));
#pragma unroll
        for (int e = 2; e < 16; e += 2) {
          a0 += __builtin_amdgcn_exp2f(fmaf(acc[kt][qt][e], c2, -nb[qt]));
          a1 += __builtin_amdgcn_exp2f(fmaf(acc[kt][qt][e + 1], c2, -nb[qt]));
        }
        part[qt] = a0 + a1;
      }
    };
    // The MFMAs of half km of the block at ring offset soff on the matrix
    // pipe while the vector pipe sums half kv of the scores already in acc.
    // The work runs in 2 KS scheduling groups plus LEAD: group g issues MFMA
    // g - LEAD (k-step (g - LEAD) / 2, query tile (g - LEAD) % 2) and the
    // fma, exp2 and add of the g-th 16 / KS of the other half's scores, so
    // the vector work leads by LEAD groups and covers the first K reads.  A
    // scheduling barrier after each group keeps that order.  K fragments are
    // read KA k-steps ahead through a shift register that starts from kin;
    // with NEXT the last k-steps read the first KA fragments of half 1 into
    // kout.  The sums run in half_sum's order, so both give the same bits.
    constexpr int KA = 2;     // K fragments read this many k-steps ahead of their MFMAs
    constexpr int LEAD = 1;   // groups the vector work leads the matrix work by
    auto pipe_half = [&](int soff, int km, int kv, const float (&nb)[2], float (&part)[2], const bf16x8 (&kin)[KA],
                         bf16x8 (&kout)[KA], auto NEXT) __attribute__((always_inline)) {
      constexpr bool next = decltype(NEXT)::value != 0;
      constexpr int SPG = 16 / KS;   // scores summed per group
      constexpr int NM = 2 * KS;     // MFMAs of the half
      static_assert(SPG * KS == 16 && SPG % 2 == 0, "two sum chains per query tile");
      bf16x8 kw[KA + 1];
#pragma unroll
      for (int i = 0; i < KA; ++i) kw[i] = kin[i];
      float a[2][2];
#pragma unroll
      for (int g = 0; g < NM + LEAD; ++g) {
        const int m = g - LEAD;
        if (m >= 0 && m < NM) {
          const int ks = m >> 1, qt = m & 1;
          if (qt == 0)
            kw[KA] = ks + KA < KS ? kfrag(soff, km, ks + KA) : (next ? kfrag(soff, 1, ks + KA - KS) : kw[0]);
          acc[km][qt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kw[0], qf[qt][ks], ks ? acc[km][qt] : f32x16{}, 0, 0, 0);
          if (qt == 1) {
#pragma unroll
            for (int i = 0; i < KA; ++i) kw[i] = kw[i + 1];
          }
        }
        if (g < NM) {
          const int qs = (SPG * g) >> 4;   // the query tile of this group's scores
#pragma unroll
          for (int u = 0; u < SPG; ++u) {
            const int e = (SPG * g + u) & 15;
            const float x = __builtin_amdgcn_exp2f(fmaf(acc[kv][qs][e], c2, -nb[qs]));
            a[qs][u & 1] = e < 2 ? x : a[qs][u & 1] + x;
          }
          // this query tile's sums so far are due here: an empty asm that
          // takes them in place (ordered against the scheduling barrier;
          // pure arithmetic alone is not)
          asm volatile("" : "+v"(a[qs][0]), "+v"(a[qs][1]));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int i = 0; i < KA; ++i) kout[i] = kw[i];
      part[0] = a[0][0] + a[0][1];
      part[1] = a[1][0] + a[1][1];
    };
    // The log2 mass of a block, log2 of its sum, is kept relative to the
    // running reference m_run of the moment; the last one's (sjb, sev) may
    // still be in a register.
    int sjb = 0;
    float sev = 0.f;
    // A half whose in-lane sum left [0, 2^13) (a score more than 13 log2
    // units above the reference, an overflow, or NaN from an infinite
    // score): the running reference moves to the half's maximum,
    // rescaling the row's sum so far and `other`, the block's half taken
    // against the old reference; the half is taken again, and the log masses
    // of the blocks jdone .. diag already finished move to the new reference
    // (in fp64, so that they keep their precision however far it moves).
    auto retake = [&](int kt, int jdone, float (&part)[2], float (&other)[2]) __attribute__((always_inline)) {
      double dl[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        float mx = acc[kt][qt][0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, acc[kt][qt][e]);
        const float m_new = fmaxf(m_run[qt], swap32_max(mx));
        const float f = __builtin_amdgcn_exp2f((m_run[qt] - m_new) * c2);
        l_run[qt] *= (double)f;
        other[qt] *= f;
        dl[qt] = ((double)m_new - (double)m_run[qt]) * c2d;
        m_run[qt] = m_new;
      }
      const float nb[2] = {m_run[0] * c2, m_run[1] * c2};
      half_sum(kt, nb, part);
      const double d = hi ? dl[1] : dl[0];
      sev = (float)((double)sev - d);
      // this wave's earlier stores of those rows have landed before they
      // are read back, and the rewrites before the loop goes on
      wait_vmcnt<0>();
      for (int j = jdone; j <= diag; ++j) {
        float* e = ew + (size_t)j * 64 + lane;
        *e = (float)((double)*e - d);
      }
      wait_vmcnt<0>();
    };
    auto escaped = [](const float (&part)[2]) {
      return __ballot(!(part[0] < 0x1p13f) || !(part[1] < 0x1p13f)) != 0;
    };
    // a block's log2 mass relative to m_run from its two halves' sums
    auto finish = [&](const float (&s0)[2], const float (&s1)[2]) __attribute__((always_inline)) {
      float evq[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const float s = swap32_sum(s0[qt] + s1[qt]);
        l_run[qt] += (double)s;
        evq[qt] = __builtin_amdgcn_logf(s);
      }
      return hi ? evq[1] : evq[0];
    };

    // Off the diagonal each block runs in two halves, software-pipelined:
    // its first half's MFMAs overlap the sums of the previous block's second
    // half, its second half's MFMAs the sums of its own first half.  Every
    // iteration stores one log mass (of the block it finished, or again the
    // last one), so the counted waits see one store per iteration.
    float p0[2] = {0.f, 0.f}, p1[2] = {0.f, 0.f};
    bool pend = false;          // block jb + 1 still needs its second half summed
    static_assert(SNST == 4, "the block loop is unrolled by the ring depth");
    // one block step; the ring slot is a compile-time constant, so the K
    // reads take it as an immediate offset
    auto step = [&](const int t, auto SLOT) __attribute__((always_inline)) {
      switch (min(t, SNST - 1)) {
        case 0: wait_vmcnt<(SNST - 2) * CPW + 0>(); break;
        case 1: wait_vmcnt<(SNST - 2) * CPW + 1>(); break;
        case 2: wait_vmcnt<(SNST - 2) * CPW + 2>(); break;
        default: wait_vmcnt<(SNST - 2) * CPW + 3>(); break;
      }
      __syncthreads();
      issue(t + SNST - 1);
      const int jb = jtop - t;
      constexpr int soff = decltype(SLOT)::value * STAGE;
      if (jb > diag) {
        sjb = jb;   // outside the wave's causal range: a slot nothing reads
        sev = 0.f;
      } else if (jb == diag) {
        asm volatile("");  // a real branch: this runs once per row-block
        mfma_half(soff, 0);
        mfma_half(soff, 1);
        // causal mask inside the diagonal block, key index > query index:
        // tile (kt = 1, qt = 0) lies wholly above the diagonal, (0, 1)
        // wholly below; in the two diagonal tiles register e holds key
        // 8 (e / 4) + 4 (L / 32) + e % 4 against query L % 32.  The lane
        // offset is re-derived here so the 32 predicates are not hoisted
        // out of the block loop.
        const int tq = opaque_int(l32 - 4 * hi);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const bool masked = 8 * (e >> 2) + (e & 3) > tq;
          acc[0][0][e] = masked ? -INFINITY : acc[0][0][e];
          acc[1][1][e] = masked ? -INFINITY : acc[1][1][e];
          acc[1][0][e] = -INFINITY;
        }
        // the diagonal block's maximum is the reference of the row's log2
        // masses; its sum lies in [1, 64], where the hardware log2 is exact
        // to an ulp
        float nb[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          float mx = acc[0][qt][0];
#pragma unroll
          for (int e = 1; e < 16; ++e) mx = fmaxf(mx, acc[0][qt][e]);
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, acc[1][qt][e]);
          mx = swap32_max(mx);
          m_ref[qt] = m_run[qt] = mx;
          nb[qt] = mx * c2;
        }
        half_sum(0, nb, p0);
        half_sum(1, nb, p1);
        float evq[2];
#pragma unroll
        for (int qt = 0; qt < 2; ++qt) {
          const float s = swap32_sum(p0[qt] + p1[qt]);
          l_run[qt] = (double)s;
          evq[qt] = __builtin_amdgcn_logf(s);
        }
        sjb = jb;
        sev = hi ? evq[1] : evq[0];
      } else {
        bf16x8 kh0[KA], kh1[KA];   // first K fragments of the block's halves 0 and 1
#pragma unroll
        for (int i = 0; i < KA; ++i) kh0[i] = kfrag(soff, 0, i);
        {
          // block jb + 1's second half (unused right after the diagonal);
          // the empty asm keeps its sums here, beside the MFMAs
          const float nb[2] = {m_run[0] * c2, m_run[1] * c2};
          pipe_half(soff, 0, 1, nb, p1, kh0, kh1, IC<1>{});
          asm volatile("" : "+v"(p1[0]), "+v"(p1[1]));
        }
        if (pend) {
          if (__builtin_expect(escaped(p1), 0)) {
            asm volatile("");
            retake(1, jb + 2, p1, p0);
          }
          sjb = jb + 1;
          sev = finish(p0, p1);
        }
        {
          const float nb[2] = {m_run[0] * c2, m_run[1] * c2};
          pipe_half(soff, 1, 0, nb, p0, kh1, kh0, IC<0>{});
        }
        if (__builtin_expect(escaped(p0), 0)) {
          asm volatile("");
          float none[2] = {0.f, 0.f};
          retake(0, jb + 1, p0, none);
        }
        pend = true;
      }
      // row `lane` of block sjb; non-temporal: written once, read once by
      // the epilogue, it should not evict the K blocks other groups re-read
      __builtin_nontemporal_store(sev, ew + (size_t)sjb * 64 + lane);
    };
    for (int t = 0; t <= jtop; t += SNST) {
      step(t, IC<0>{});
      if (t + 1 > jtop) break;
      step(t + 1, IC<1>{});
      if (t + 2 > jtop) break;
      step(t + 2, IC<2>{});
      if (t + 3 > jtop) break;
      step(t + 3, IC<3>{});
    }
    if (pend) {
      // the second half of the last block, block 0
      const float nb[2] = {m_run[0] * c2, m_run[1] * c2};
      half_sum(1, nb, p1);
      if (escaped(p1)) retake(1, 1, p1, p0);
      __builtin_nontemporal_store(finish(p0, p1), ew + lane);
    }

    wait_vmcnt<0>();
    __syncthreads();  // every wave is done with the K ring: LDS becomes the transposes
    // 128-row blocks: row sums of each 64-key block of the wave's half, in
    // LDS after the transposes, combined below by the first half's wave
    float* const hsum = reinterpret_cast<float*>(smem) + SQ * 64 * SEPITCH + (size_t)w * max_cb64;
    if (valid) {
      // lane L keeps query row L: half L / 32 of the wave's two 32-row halves
      const float mr = hi ? m_ref[1] : m_ref[0];
      const float mu = hi ? m_run[1] : m_run[0];
      const double lr = hi ? l_run[1] : l_run[0];
      // the row's log2 normaliser relative to m_run (the reference of every
      // stored log mass) and to m_ref
      const double lrun2 = log2(lr);
      const double lse2 = ((double)mu - (double)mr) * c2d + lrun2;
      const size_t lh = (size_t)l * a.H + h;
      if (lane < ri.rows)
        a.row_lse[lh * a.b.total_q + ri.q0 + lane] = (float)((double)mr * a.scale + lse2 * kLn2);
      float* tr = reinterpret_cast<float*>(smem) + w * 64 * SEPITCH;
      float* __restrict__ bm = a.block_mass + (lh * a.b.total_rb + rb) * (size_t)a.b.max_cb;   // SUB == 1
      for (int j0 = 0; j0 < ri.ncand; j0 += 64) {
        const int nj = min(64, ri.ncand - j0);
        // the scratch rows were written by this wave on this CU and its
        // stores have completed: plain loads see them.  32 in flight (the
        // loop's registers are free now): the read-back is latency-bound.
        for (int jj = 0; jj < nj; jj += 32) {
          float e[32];
#pragma unroll
          for (int u = 0; u < 32; ++u) e[u] = __builtin_nontemporal_load(ew + (size_t)min(j0 + jj + u, ri.ncand - 1) * 64 + lane);
#pragma unroll
          for (int u = 0; u < 32; ++u)
            if (jj + u < nj) tr[(jj + u) * SEPITCH + lane] = lane < ri.rows ? exp2f((float)((double)e[u] - lrun2)) : 0.f;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        if (lane < nj) {
          double accm = 0.0;
          for (int r = 0; r < ri.rows; ++r) accm += (double)tr[lane * SEPITCH + r];
          if constexpr (SUB == 1) bm[j0 + lane] = (float)(accm / ri.rows);
          else hsum[j0 + lane] = (float)accm;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      }
      if constexpr (SUB == 1)
        for (int j = ri.ncand + lane; j < a.b.max_cb; j += 64) bm[j] = 0.f;
    }
    if constexpr (SUB == 2) {
      // a half's sums past its own causal range are 0 (the first half sees
      // one 64-key block fewer of the diagonal 128-key block, an empty half none)
      if (valid)
        for (int j = ri.ncand + lane; j < max_cb64; j += 64) hsum[j] = 0.f;
      __syncthreads();
      if ((w & 1) == 0 && valid) {
        // the row-block's masses: both halves' sums over both 64-key halves
        // of each 128-key block, over the row-block's rows
        const int rb128 = rb / 2;
        const bool second = rb + 1 <= last_rb;
        const RowBlockInfo r2 = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, 128, rb128);
        const size_t lh = (size_t)l * a.H + h;
        float* __restrict__ bm = a.block_mass + (lh * a.b.total_rb + rb128) * (size_t)a.b.max_cb;
        const float* hs2 = hsum + max_cb64;
        for (int J = lane; J < a.b.max_cb; J += 64) {
          float m = 0.f;
          if (J < r2.ncand) {
            double t = (double)hsum[2 * J] + (double)hsum[2 * J + 1];
            if (second) t += (double)hs2[2 * J] + (double)hs2[2 * J + 1];
            m = (float)(t / r2.rows);
          }
          bm[J] = m;
        }
      }
      __syncthreads();   // the sums are read before the next item's ring overwrites LDS
    }
  }
}

}  // namespace

size_t block_stats_lds_bytes(int B, int max_cb) {
  const size_t ecols = (size_t)(max_cb | 1);
  return ((size_t)B * ecols * 4 + 15) / 16 * 16 + (size_t)B * 8;
}

bool stats_fast_path(mf_dtype dt, int B, int d) {
  if (dt != MF_BF16 || (B != 64 && B != 128) || (d != 64 && d != 128)) return false;
  return !(forced_portable() & MF_FORCE_PORTABLE_STATS);
}

static size_t stats_mfma_lds_bytes(int d, int B, int max_cb) {
  const size_t ring = (size_t)SNST * 64 * d * 2;
  // 128-row blocks: the halves' row sums per 64-key block beside the transposes
  const size_t tr = (size_t)SQ * 64 * SEPITCH * 4 + (B == 128 ? (size_t)SQ * 2 * max_cb * 4 : 0);
  return ring > tr ? ring : tr;
}

StatsWorkspace stats_workspace_layout(int B, int max_cb, int total_rb, int slots) {
  // 64-row units: B / 64 per row-block, each with B / 64 times the 64-key blocks
  const size_t sub = (size_t)B / 64;
  StatsWorkspace w;
  w.hdr = 0;
  w.table = 256;
  w.escratch = w.table + ((size_t)total_rb * sub * 4 + 255) / 256 * 256;
  w.slots = slots;
  w.bytes = w.escratch + (size_t)slots * SQ * 64 * (size_t)max_cb * sub * 4;
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
    const int sub = a.B / 64;
    hipLaunchKernelGGL(stats_groups_kernel, dim3(1), dim3(1024), 0, (hipStream_t)stream, a.b, sub, hdr, table);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
    const size_t lds = stats_mfma_lds_bytes(a.d, a.B, a.b.max_cb);
    auto kern = sub == 2 ? (a.d == 128 ? stats_mfma_kernel<128, 2> : stats_mfma_kernel<64, 2>)
                         : (a.d == 128 ? stats_mfma_kernel<128, 1> : stats_mfma_kernel<64, 1>);
    e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(kern, dim3(a.wsl.slots), dim3(SQ * 64), lds, (hipStream_t)stream, a, hdr, table, escr);
    return (int)hipGetLastError();
  }
  return dt == MF_BF16 ? launch_d<bf16>(a, stream) : launch_d<float>(a, stream);
}

}  // namespace mf
