// Stage 2 of the staged block compression: keep, per (layer, sender head,
// row-block), the blocks needed to reach cumulative attention probability
// tau, then extract their probabilities (MapFlow page, section
// "让复用真正省时…", paragraph "第一").
//
//   select:  one workgroup per CSR row.  Keys (mass desc, column asc) are
//            bitonic-sorted in LDS; the sorted masses are prefix-summed in
//            fp64; the cut is the first prefix reaching tau.  Output: kept
//            count and a bitmask over column blocks.
//   scan:    one workgroup turns the counts into row_ptr (exclusive scan).
//   extract: one workgroup per CSR row recomputes S = Q K^T for its kept
//            blocks only (MFMA), P = exp(S * scale - row_lse), and writes
//            each B x B block key-major (values[e][key][query]) through LDS
//            so every store is a full 16-byte vector.
#include <type_traits>

#include "device_common.h"
#include "internal.h"

namespace mf {

namespace {

constexpr int kSelThreads = 256;

__global__ void __launch_bounds__(kSelThreads) select_kernel(SelectArgs a, int n2) {
  extern __shared__ __align__(16) char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);                 // [n2]
  double* tsum = reinterpret_cast<double*>(keys + n2);                // [kSelThreads]
  uint32_t* bits = reinterpret_cast<uint32_t*>(tsum + kSelThreads);   // [words]
  __shared__ int kstar_s;

  const int rb = blockIdx.x, h = blockIdx.y, l = blockIdx.z;
  const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, a.B, rb);
  const size_t row = ((size_t)l * a.H + h) * a.b.total_rb + rb;
  const float* __restrict__ m = a.block_mass + row * (size_t)a.b.max_cb;
  const int n = ri.ncand;
  const int tid = threadIdx.x;

  for (int t = tid; t < n2; t += kSelThreads) {
    uint64_t key = ~0ull;
    if (t < n) key = ((uint64_t)(0xFFFFFFFFu - __float_as_uint(m[t])) << 32) | (uint32_t)t;
    keys[t] = key;
  }
  for (int t = tid; t < a.words; t += kSelThreads) bits[t] = 0u;
  if (tid == 0) kstar_s = n;
  __syncthreads();

  // bitonic sort, ascending keys = mass descending, column ascending
  for (int k = 2; k <= n2; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int t = tid; t < n2; t += kSelThreads) {
        const int p = t ^ jj;
        if (p > t) {
          const uint64_t x = keys[t], y = keys[p];
          const bool up = (t & k) == 0;
          if ((x > y) == up) { keys[t] = y; keys[p] = x; }
        }
      }
      __syncthreads();
    }
  }

  // fp64 prefix sums of the sorted masses: contiguous chunk per thread
  const int per = (n2 + kSelThreads - 1) / kSelThreads;
  const int t0 = tid * per;
  double local = 0.0;
  for (int t = t0; t < min(t0 + per, n); ++t)
    local += (double)__uint_as_float(0xFFFFFFFFu - (uint32_t)(keys[t] >> 32));
  tsum[tid] = local;
  __syncthreads();
  if (a.tau < 1.0) {
    double before = 0.0;
    for (int u = 0; u < tid; ++u) before += tsum[u];
    double c = before;
    for (int t = t0; t < min(t0 + per, n); ++t) {
      c += (double)__uint_as_float(0xFFFFFFFFu - (uint32_t)(keys[t] >> 32));
      if (c >= a.tau) { atomicMin(&kstar_s, t + 1); break; }
    }
  }
  __syncthreads();
  const int kstar = kstar_s;
  for (int t = tid; t < kstar; t += kSelThreads) {
    const uint32_t j = (uint32_t)(keys[t] & 0xFFFFFFFFu);
    atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  __syncthreads();
  uint32_t* __restrict__ out = a.keep_bits + row * (size_t)a.words;
  for (int t = tid; t < a.words; t += kSelThreads) out[t] = bits[t];
  if (tid == 0) a.counts[row] = kstar;
}

// One wave per CSR row for rows of at most 64 * E candidates: the keys sit
// in registers (element e of lane L is sorted position L + 64 e), the bitonic
// network exchanges across lanes with shuffles and inside a lane for strides
// of 64 and up, the fp64 cumulative sum is a wave scan per element, and the
// kept set is every key at or before the cut key, so the bit words come
// straight from ballots over the unsorted keys.
constexpr int kSelWaves = 4;

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int mask) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, mask, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), mask, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ uint64_t shfl_u64(uint64_t x, int src) {
  const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)x, src, 64);
  const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(x >> 32), src, 64);
  return ((uint64_t)hi << 32) | lo;
}
__device__ __forceinline__ double key_mass(uint64_t key) {
  return (double)__uint_as_float(0xFFFFFFFFu - (uint32_t)(key >> 32));
}

template <int E>
__global__ void __launch_bounds__(kSelWaves * 64) select_wave_kernel(SelectArgs a, long long nrows) {
  const int lane = threadIdx.x & 63;
  const long long row = (long long)blockIdx.x * kSelWaves + (threadIdx.x >> 6);
  if (row >= nrows) return;  // uniform per wave
  const int rb = (int)(row % a.b.total_rb);
  const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, a.B, rb);
  const int n = ri.ncand;
  const float* __restrict__ m = a.block_mass + row * (long long)a.b.max_cb;

  uint64_t orig[E], key[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int t = lane + 64 * e;
    orig[e] = t < n ? ((uint64_t)(0xFFFFFFFFu - __float_as_uint(m[t])) << 32) | (uint32_t)t : ~0ull;
    key[e] = orig[e];
  }
  // bitonic sort, ascending keys = mass descending, column ascending
#pragma unroll
  for (int k = 2; k <= 64 * E; k <<= 1) {
#pragma unroll
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      if (jj >= 64) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const int f = e ^ (jj >> 6);
          if (f > e) {
            const bool up = ((lane + 64 * e) & k) == 0;
            const uint64_t x = key[e], y = key[f];
            const uint64_t lo = x < y ? x : y, hi = x < y ? y : x;
            key[e] = up ? lo : hi;
            key[f] = up ? hi : lo;
          }
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const uint64_t y = shfl_xor_u64(key[e], jj);
          const bool lower = (lane & jj) == 0;
          const bool up = ((lane + 64 * e) & k) == 0;
          const uint64_t x = key[e];
          key[e] = (lower == up) ? (x < y ? x : y) : (x < y ? y : x);
        }
      }
    }
  }
  // shortest sorted prefix whose fp64 cumulative mass reaches tau
  int kstar = n;
  if (a.tau < 1.0) {
    double run = 0.0;
    bool found = false;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const bool valid = lane + 64 * e < n;
      double c = valid ? key_mass(key[e]) : 0.0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(c, off, 64);
        if (lane >= off) c += y;
      }
      c += run;
      run = __shfl(c, 63, 64);
      const unsigned long long hit = __ballot(valid && c >= a.tau);
      if (!found && hit) {
        kstar = 64 * e + __ffsll((long long)hit);
        found = true;
      }
    }
  }
  // kept = every candidate whose key is at or before the cut key
  uint64_t cut = 0;
  if (kstar > 0) {
    const int r = kstar - 1;
    uint64_t src = key[0];
#pragma unroll
    for (int e = 1; e < E; ++e)
      if ((r >> 6) == e) src = key[e];
    cut = shfl_u64(src, r & 63);
  }
  uint32_t* __restrict__ out = a.keep_bits + row * (long long)a.words;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const unsigned long long bal = __ballot(kstar > 0 && orig[e] <= cut);
    if (lane == 0) {
      if (2 * e < a.words) out[2 * e] = (uint32_t)bal;
      if (2 * e + 1 < a.words) out[2 * e + 1] = (uint32_t)(bal >> 32);
    }
  }
  if (lane == 0) a.counts[row] = kstar;
}

// Exclusive scan of the per-row counts into row_ptr by one workgroup: tiles
// of 1024 x 32 counts, each thread scanning 32 consecutive counts in
// registers, then one wave-and-LDS scan of the 1024 thread totals per tile.
constexpr int kScanThreads = 1024;
constexpr int kScanPer = 32;

__global__ void __launch_bounds__(kScanThreads) scan_kernel(ScanArgs a) {
  __shared__ long long wsum[kScanThreads / 64];
  __shared__ long long carry_s;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  if (tid == 0) carry_s = 0;
  __syncthreads();
  // a thread's 32 counts are 128 contiguous bytes: whole chunks move as
  // 16-byte vectors when both arrays are 16-byte aligned
  const bool aligned = ((reinterpret_cast<uintptr_t>(a.counts) | reinterpret_cast<uintptr_t>(a.row_ptr)) & 15) == 0;
  for (int64_t base = 0; base < a.n; base += (int64_t)kScanThreads * kScanPer) {
    const int64_t i0 = base + (int64_t)tid * kScanPer;
    const bool vec = aligned && i0 + kScanPer <= a.n;
    int32_t x[kScanPer];
    long long tot = 0;
    if (vec) {
      const int4* src = reinterpret_cast<const int4*>(a.counts + i0);
#pragma unroll
      for (int u = 0; u < kScanPer / 4; ++u) {
        const int4 c = src[u];
        x[4 * u] = c.x;
        x[4 * u + 1] = c.y;
        x[4 * u + 2] = c.z;
        x[4 * u + 3] = c.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kScanPer; ++u) x[u] = i0 + u < a.n ? a.counts[i0 + u] : 0;
    }
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) tot += x[u];
    long long v = tot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = __shfl_up(v, off, 64);
      if (lane >= off) v += y;
    }
    if (lane == 63) wsum[w] = v;
    __syncthreads();
    long long pre = carry_s;
    for (int u = 0; u < w; ++u) pre += wsum[u];
    long long run = pre + v - tot;
    if (vec) {
      int4* dst = reinterpret_cast<int4*>(a.row_ptr + i0);
#pragma unroll
      for (int u = 0; u < kScanPer / 4; ++u) {
        int4 o;
        o.x = (int32_t)run;
        run += x[4 * u];
        o.y = (int32_t)run;
        run += x[4 * u + 1];
        o.z = (int32_t)run;
        run += x[4 * u + 2];
        o.w = (int32_t)run;
        run += x[4 * u + 3];
        dst[u] = o;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kScanPer; ++u) {
        if (i0 + u < a.n) a.row_ptr[i0 + u] = (int32_t)run;
        run += x[u];
      }
    }
    __syncthreads();
    if (tid == kScanThreads - 1) carry_s = run;
    __syncthreads();
  }
  if (tid == 0) {
    a.row_ptr[a.n] = (int32_t)carry_s;
    *a.total = carry_s;
  }
}

template <typename T, int B, int D>
__global__ void __launch_bounds__(B * 4) extract_kernel(ExtractArgs a) {
  constexpr int NT = B / 16;
  constexpr int VEC = 16 / sizeof(T);          // elements per 16-byte store
  constexpr int PITCH = B + VEC;               // LDS row pitch (elements)
  // the block, key-major: tile[c][q]
  __shared__ __align__(16) T tile[B * PITCH];

  int rb, h, l;
  xcd_unflatten(blockIdx.x, a.b.total_rb, a.H, a.L, rb, h, l);
  if (l >= a.L) return;
  const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, B, rb);
  const size_t lh = (size_t)l * a.H + h;
  const size_t row = lh * a.b.total_rb + rb;
  const int64_t base = a.row_ptr[row];
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
  // exp(s - lse) with s = scale * S: scale split in two floats so the
  // product keeps ~48 bits before the subtraction
  const float s_hi = (float)a.scale;
  const float s_lo = (float)(a.scale - (double)s_hi);
  float lse[4];
  int rowl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rowl[i] = 16 * w + 4 * lg + i;
    lse[i] = rowl[i] < ri.rows ? a.row_lse[lh * a.b.total_q + ri.q0 + rowl[i]] : 0.f;
  }
  const uint32_t* __restrict__ kb = a.keep_bits + row * (size_t)a.words;
  T* __restrict__ vals = reinterpret_cast<T*>(a.values);

  int64_t e = base;
  for (int wd = 0; wd < a.words; ++wd) {
    uint32_t bitsw = kb[wd];
    while (bitsw) {
      const int j = wd * 32 + __builtin_ctz(bitsw);
      bitsw &= bitsw - 1;
      if (e < a.capacity) {
        if (threadIdx.x == 0) a.col_idx[e] = j;
        if (vals) {
          f32x4 acc[NT];
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            acc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
            const int c = min(j * B + 16 * nt + lr, ri.klen - 1);
            acc[nt] = qf.dot(kbase + (size_t)c * kstride, lane, acc[nt]);
          }
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int c = j * B + 16 * nt + lr;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              float p = 0.f;
              if (rowl[i] < ri.rows && c <= ri.pos0 + rowl[i]) {
                float x = fmaf(acc[nt][i], s_hi, -lse[i]);
                x = fmaf(acc[nt][i], s_lo, x);
                p = exp2f(x * kLog2e);
              }
              tile[(16 * nt + lr) * PITCH + rowl[i]] = from_f32<T>(p);
            }
          }
          __syncthreads();
          // B key rows of B queries each -> global, 16 bytes per store
          T* __restrict__ dst = vals + (size_t)e * B * B;
          constexpr int CH = B * B / VEC;
          for (int c = threadIdx.x; c < CH; c += B * 4) {
            const int r = c / (B / VEC), col = (c % (B / VEC)) * VEC;
            *reinterpret_cast<uint4*>(dst + (size_t)r * B + col) =
                *reinterpret_cast<const uint4*>(tile + r * PITCH + col);
          }
          __syncthreads();
        }
      }
      ++e;
    }
  }
}

// ---------------------------------------------------------------------------
// bf16, B = 64: one workgroup of four waves per CSR row.  The row's kept
// column blocks are listed in LDS; their K tiles stream once through an
// LDS ring (async global_load_lds, 16-byte chunks XOR-swizzled per key row)
// shared by the four waves, and wave w computes quadrant (row half w & 1,
// key half w >> 1) of every block on MFMA 32x32x16 (A = Q rows kept in
// registers, B = K keys from LDS).  Lane L then holds key 32 kh + L % 32 and
// the four consecutive rows 8 (e / 4) + 4 (L / 32) + 0..3 of register group
// e / 4, so exp2(s c2 - lse2) of four rows packs into one 8-byte bf16 LDS
// write of the key-major tile; the workgroup then stores the 8 KB tile with
// 16-byte vector stores.  The ring has two slots and the tile is written
// into the slot whose K the block just consumed: at most 32 KB of LDS and 128
// VGPRs let four workgroups share a CU, and that occupancy hides the K
// fetches better than a deeper ring.
// ---------------------------------------------------------------------------
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
constexpr int XNST = 2;                 // K ring depth
// Output tile [64 keys][64 rows] bf16, 128 bytes per key row, 16-byte chunk c
// of key k stored at chunk c ^ ((k / 2) % 8).  A write instruction (32 keys x
// 8 bytes per half-wave) then spreads over every bank, and so does a
// read-back quarter-wave (two key rows of 128 bytes, in opposite bank halves).
constexpr int XPITCH = 64 * 2;
__device__ __forceinline__ int xtile_off(int key, int byte) {   // byte < 128
  return key * XPITCH + ((((byte >> 4) ^ ((key >> 1) & 7))) << 4) + (byte & 15);
}
constexpr int kXMaxCb = (MF_MAX_KEYS + 63) / 64;   // column blocks of the longest sequence
// K rows of one sequence are addressed by 32-bit byte offsets from its first
// key row (at most MF_MAX_KEYS keys of at most 64 heads x 128 dims, bf16)
static_assert((unsigned long long)MF_MAX_KEYS * 64 * 128 * 2 < (1ull << 32), "32-bit K row offsets");

// Async 16-byte-per-lane copy HBM -> LDS (lane L lands at base + 16 L).
// Issued as inline assembly so the compiler does not track it: it would
// otherwise drain every copy in flight (vmcnt(0)) before any later LDS
// access, including the output tile, which no copy ever writes.  The kernel
// waits for the copies itself (counted vmcnt) before the barrier that opens
// a ring slot.  The instruction writes no VGPR.
__device__ __forceinline__ void xcopy16(const void* gsrc, char* lds_generic_base) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_generic_base);
  // one wait state between the M0 write and the copy that reads it
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gsrc), "s"(base)
               : "memory", "m0");
}

// The same copy from a scalar base plus a 32-bit lane offset; m0 is the LDS
// destination of lane 0.
__device__ __forceinline__ void xcopy16s(unsigned voff, const void* sbase, unsigned m0) {
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
__device__ __forceinline__ unsigned xlds_addr(const char* lds_generic) {
  return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_generic);
}
// a copy of a lane value the compiler cannot see through
__device__ __forceinline__ int opaque_int(int x) {
  int y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}
template <int N>
using IC = std::integral_constant<int, N>;

template <int N>
__device__ __forceinline__ void xwait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// two floats to bf16 (round to nearest even) in one 32-bit word, lo in the
// low half: one two-source conversion instruction
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  typedef float f32x2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(unsigned, v);
}

template <int D>
__global__ void __launch_bounds__(256, 4) extract_mfma_kernel(ExtractArgs a) {
  constexpr int KS = D / 16;
  constexpr int ROWB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int STAGE = 64 * ROWB;
  constexpr int CPW = STAGE / 1024 / 4;
  constexpr int OT = 64 * XPITCH;       // one output tile
  // the K ring; each output tile goes into the slot whose K its block just
  // consumed
  extern __shared__ __align__(16) char ring[];
  __shared__ int jlist[kXMaxCb];
  __shared__ int nkept;

  int rb, h, l;
  xcd_unflatten(blockIdx.x, a.b.total_rb, a.H, a.L, rb, h, l);
  if (l >= a.L) return;
  const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, 64, rb);
  const size_t lh = (size_t)l * a.H + h;
  const size_t row = lh * a.b.total_rb + rb;
  const int64_t base = a.row_ptr[row];
  const int hk = h / (a.H / a.Hkv);
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qh = w & 1, kh = w >> 1;

  // Q rows 32 qh + L % 32 as A operands and lse2 of the lane's 16 output
  // rows: independent of the kept set, so their loads go out first
  bf16x8 qf[KS];
  {
    const int r = 32 * qh + l32;
    const bf16* src = reinterpret_cast<const bf16*>(a.q) + (size_t)l * a.lsq +
                      ((size_t)(ri.q0 + (r < ri.rows ? r : 0)) * a.H + h) * D + 8 * hi;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
  }
  const float c2 = (float)(a.scale * kLog2eD);
  float lse2[16];
  {
    const float* __restrict__ lrow = a.row_lse + lh * a.b.total_q + ri.q0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = 32 * qh + 8 * (e >> 2) + 4 * hi + (e & 3);
      const float v = lrow[r < ri.rows ? r : 0];
      lse2[e] = r < ri.rows ? v * kLog2e : INFINITY;
    }
  }

  // kept column blocks of the row, ascending, and their col_idx entries:
  // wave 0, one keep-bit word per lane (a row has at most 64 words), an
  // exclusive prefix of the words' counts places each lane's columns
  if (w == 0) {
    const uint32_t bw = lane < a.words ? a.keep_bits[row * (size_t)a.words + lane] : 0u;
    const int cnt = __popc(bw);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    int pos = incl - cnt;
    uint32_t bits = bw;
    while (bits) {
      const int j = lane * 32 + __builtin_ctz(bits);
      bits &= bits - 1;
      if (base + pos < a.capacity) a.col_idx[base + pos] = j;
      jlist[pos++] = j;
    }
    if (lane == 63) {
      const int64_t room = a.capacity - base;
      nkept = a.values ? (int)(room < 0 ? 0 : (room < incl ? room : incl)) : 0;
    }
  }
  __syncthreads();
  const int n = __builtin_amdgcn_readfirstlane(nkept);
  if (n == 0) return;

  const bf16* __restrict__ kbase = reinterpret_cast<const bf16*>(a.k) + (size_t)l * a.lsk +
                                   (size_t)ri.k0 * a.Hkv * D + (size_t)hk * D;
  const size_t kstride = (size_t)a.Hkv * D;
  const int klast = ri.klen - 1;
  // copy i of this wave: key kkey[i] of the block, source chunk
  // cc ^ (key % CPR) at byte offset koff[i] from the block's first key row,
  // whose address is scalar
  unsigned koff[CPW];
  int kkey[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int pidx = (i * 4 + w) * 64 + lane;
    const int key = pidx / CPR, cc = pidx % CPR;
    kkey[i] = key;
    koff[i] = (unsigned)(((size_t)key * kstride + (cc ^ (key & (CPR - 1))) * 8) * 2);
  }
  const char* kbytes = reinterpret_cast<const char*>(kbase);
  auto issue = [&](int t, int slot) __attribute__((always_inline)) {
    const int j = __builtin_amdgcn_readfirstlane(jlist[t < n ? t : n - 1]);
    const char* src = kbytes + (size_t)j * 64 * kstride * 2;
    const unsigned m0 = xlds_addr(ring + slot * STAGE + w * 1024);
    if (j * 64 + 63 <= klast) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) xcopy16s(koff[i], src, m0 + i * 4 * 1024);
    } else {
      // block reaching past the last key: each row's key clamped to the last
      // key, addressed from the sequence's first key row
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const unsigned chb = koff[i] - (unsigned)((size_t)kkey[i] * kstride * 2);   // the chunk's byte offset in its row
        const int kk = min(j * 64 + kkey[i], klast);
        // below 2^32: a sequence has at most MF_MAX_KEYS keys of at most 64 heads x 128 dims
        xcopy16s((unsigned)((size_t)kk * kstride * 2) + chb, kbytes, m0 + i * 4 * 1024);
      }
    }
  };
  issue(0, 0);

  const int diag = ri.ncand - 1;
  const char* __restrict__ vbytes = reinterpret_cast<const char*>(a.values);
  // per-lane LDS byte addresses, kept opaque so that the compiler holds the
  // sums rather than re-adding their parts, and every access of a step (its
  // ring slot known at compile time) is one instruction with an immediate
  // offset: the K fragment of k-step ks (key 32 kh + L % 32, head-dim slice
  // 16 ks + 8 (L / 32)), the tile write of row group g, the tile read of
  // store c
  typedef __attribute__((address_space(3))) char lds_char;
  const int key = 32 * kh + l32;
  const int ring0 = (int)xlds_addr(ring);
  int kfo[KS], two[4], tro[2];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kfo[ks] = opaque_int(ring0 + key * ROWB + (((2 * ks + hi) ^ (key & (CPR - 1))) * 16));
#pragma unroll
  for (int g = 0; g < 4; ++g) two[g] = opaque_int(ring0 + xtile_off(key, (32 * qh + 8 * g + 4 * hi) * 2));
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int ch = c * 256 + tid;           // 16-byte chunk: key ch / 8, rows 8 (ch % 8) ..
    tro[c] = opaque_int(ring0 + xtile_off(ch >> 3, (ch & 7) * 16));
  }
  auto lds = [](int addr) { return reinterpret_cast<lds_char*>((uintptr_t)(unsigned)addr); };

  // one kept block t in ring slot SLOT: the next block's K goes into the
  // other slot, the value tile into this one once its K is consumed
  auto step = [&](const int t, auto SLOT) __attribute__((always_inline)) {
    constexpr int slot = decltype(SLOT)::value;
    constexpr int soff = slot * STAGE;
    if (t == 0) xwait_vmcnt<0>();
    else xwait_vmcnt<2>();   // this slot's copies: only the previous block's two stores are younger
    __syncthreads();
    issue(t + 1, slot ^ 1);
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kf = *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(lds(kfo[ks]) + soff);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[ks], kf, acc, 0, 0, 0);
    }
    const bool dg = __builtin_amdgcn_readfirstlane(jlist[t]) == diag;
    __syncthreads();       // every wave is done reading K from the slot
    // causal mask (diagonal block only) and rows past the row-block: lse2 = inf
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * g + i;
        p[i] = __builtin_amdgcn_exp2f(fmaf(acc[e], c2, -lse2[e]));
      }
      if (dg) {
        asm volatile("");  // a real branch: at most one block per row-block
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key > 32 * qh + 8 * g + 4 * hi + i) p[i] = 0.f;
      }
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(lds(two[g]) + soff) = pk;
    }
    __syncthreads();
    // non-temporal stores: the values are read only by a later kernel, and
    // streaming them past L2 keeps the K blocks the row-blocks of this head
    // share resident there
    const char* dst = vbytes + (size_t)(base + t) * 64 * 64 * 2;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int ch = c * 256 + tid;
      const u32x4 v = *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(lds(tro[c]) + soff);
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(const_cast<char*>(dst) + ((ch >> 3) * 64 + (ch & 7) * 8) * 2));
    }
  };
  static_assert(XNST == 2 && STAGE >= OT, "two ring slots, each holding an output tile");
  for (int t = 0; t < n; t += 2) {
    step(t, IC<0>{});
    if (t + 1 >= n) break;
    step(t + 1, IC<1>{});
  }
  xwait_vmcnt<0>();   // the copy issued past the last block has landed before the LDS is released
}

// 128-row blocks: the same scheme over 64-key halves.  A workgroup walks its
// row-block's kept 128-key blocks one 64-key half at a time (the K ring holds
// 64-key stages); for each half, wave w computes rows 64 a + 32 (w % 2) ..
// + 31 against keys 32 (w / 2) .. + 31 of the half for both 64-row halves a,
// so every K fragment feeds two MFMA chains.  The half's 64 keys x 128 rows
// go through a key-major LDS tile to 256-byte rows of the value block.
// 128-row output tile: 256 bytes per key row, chunk c of key k at c ^ (k % 16)
constexpr int XPITCH2 = 128 * 2;
__device__ __forceinline__ int xtile2_off(int key, int byte) {   // byte < 256
  return key * XPITCH2 + ((((byte >> 4) ^ (key & 15))) << 4) + (byte & 15);
}

template <int D>
__global__ void __launch_bounds__(256, 2) extract_mfma128_kernel(ExtractArgs a) {
  constexpr int KS = D / 16;
  constexpr int ROWB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int STAGE = 64 * ROWB;
  constexpr int CPW = STAGE / 1024 / 4;
  constexpr int BB = 128;
  extern __shared__ __align__(16) char ring[];
  __shared__ __align__(16) char otile[64 * XPITCH2];
  __shared__ int jlist[kXMaxCb];
  __shared__ int nkept;

  int rb, h, l;
  xcd_unflatten(blockIdx.x, a.b.total_rb, a.H, a.L, rb, h, l);
  if (l >= a.L) return;
  const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, BB, rb);
  const size_t lh = (size_t)l * a.H + h;
  const size_t row = lh * a.b.total_rb + rb;
  const int64_t base = a.row_ptr[row];
  const int hk = h / (a.H / a.Hkv);
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qh = w & 1, kh = w >> 1;

  // Q rows 64 a + 32 qh + L % 32 as A operands and lse2 of the lane's output
  // rows of both halves
  const float c2 = (float)(a.scale * kLog2eD);
  bf16x8 qf[2][KS];
  float lse2[2][16];
  {
    const float* __restrict__ lrow = a.row_lse + lh * a.b.total_q + ri.q0;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int r = 64 * hf + 32 * qh + l32;
      const bf16* src = reinterpret_cast<const bf16*>(a.q) + (size_t)l * a.lsq +
                        ((size_t)(ri.q0 + (r < ri.rows ? r : 0)) * a.H + h) * D + 8 * hi;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[hf][ks] = *reinterpret_cast<const bf16x8*>(src + 16 * ks);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int rr = 64 * hf + 32 * qh + 8 * (e >> 2) + 4 * hi + (e & 3);
        const float v = lrow[rr < ri.rows ? rr : 0];
        lse2[hf][e] = rr < ri.rows ? v * kLog2e : INFINITY;
      }
    }
  }

  // kept column blocks, as in the 64-row kernel
  if (w == 0) {
    const uint32_t bw = lane < a.words ? a.keep_bits[row * (size_t)a.words + lane] : 0u;
    const int cnt = __popc(bw);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off, 64);
      if (lane >= off) incl += y;
    }
    int pos = incl - cnt;
    uint32_t bits = bw;
    while (bits) {
      const int j = lane * 32 + __builtin_ctz(bits);
      bits &= bits - 1;
      if (base + pos < a.capacity) a.col_idx[base + pos] = j;
      jlist[pos++] = j;
    }
    if (lane == 63) {
      const int64_t room = a.capacity - base;
      nkept = a.values ? (int)(room < 0 ? 0 : (room < incl ? room : incl)) : 0;
    }
  }
  __syncthreads();
  const int n = __builtin_amdgcn_readfirstlane(nkept);
  if (n == 0) return;

  const bf16* __restrict__ kbase = reinterpret_cast<const bf16*>(a.k) + (size_t)l * a.lsk +
                                   (size_t)ri.k0 * a.Hkv * D + (size_t)hk * D;
  const size_t kstride = (size_t)a.Hkv * D;
  const int klast = ri.klen - 1;
  // copy i of this wave: key kkey[i] of the stage, byte offset koff[i] from
  // the stage's first key row (scalar), as in the 64-row kernel
  unsigned koff[CPW];
  int kkey[CPW];
#pragma unroll
  for (int i = 0; i < CPW; ++i) {
    const int pidx = (i * 4 + w) * 64 + lane;
    const int key = pidx / CPR, cc = pidx % CPR;
    kkey[i] = key;
    koff[i] = (unsigned)(((size_t)key * kstride + (cc ^ (key & (CPR - 1))) * 8) * 2);
  }
  const char* kbytes = reinterpret_cast<const char*>(kbase);
  // stage t: key half t % 2 of kept block t / 2, into ring slot t % 2
  auto issue = [&](int t) __attribute__((always_inline)) {
    const int tt = t < 2 * n ? t : 2 * n - 1;
    const int j = __builtin_amdgcn_readfirstlane(jlist[tt >> 1]);
    const int k0 = j * BB + 64 * (tt & 1);
    const char* src = kbytes + (size_t)k0 * kstride * 2;
    const unsigned m0 = xlds_addr(ring + (t % XNST) * STAGE + w * 1024);
    if (k0 + 63 <= klast) {
#pragma unroll
      for (int i = 0; i < CPW; ++i) xcopy16s(koff[i], src, m0 + i * 4 * 1024);
    } else {
      // rows past the last key (the second half may start past it): each
      // row's key clamped to the last key, addressed from the sequence's
      // first key row
#pragma unroll
      for (int i = 0; i < CPW; ++i) {
        const unsigned chb = koff[i] - (unsigned)((size_t)kkey[i] * kstride * 2);   // the chunk's byte offset in its row
        const int kk = min(k0 + kkey[i], klast);
        // below 2^32: a sequence has at most MF_MAX_KEYS keys of at most 64 heads x 128 dims
        xcopy16s((unsigned)((size_t)kk * kstride * 2) + chb, kbytes, m0 + i * 4 * 1024);
      }
    }
  };
  issue(0);

  const int diag = ri.ncand - 1;
  const char* __restrict__ vbytes = reinterpret_cast<const char*>(a.values);
  // per-lane LDS byte addresses (opaque, as in the 64-row kernel): K
  // fragment ks of key 32 kh + L % 32 in slot 0, the tile write of (half
  // hf, row group g), the tile read of store c
  typedef __attribute__((address_space(3))) char lds_char;
  const int key = 32 * kh + l32;
  const int ring0 = (int)xlds_addr(ring), tile0 = (int)xlds_addr(otile);
  int kfo[KS], two[2][4], tro[4];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) kfo[ks] = opaque_int(ring0 + key * ROWB + (((2 * ks + hi) ^ (key & (CPR - 1))) * 16));
#pragma unroll
  for (int hf = 0; hf < 2; ++hf)
#pragma unroll
    for (int g = 0; g < 4; ++g) two[hf][g] = opaque_int(tile0 + xtile2_off(key, (64 * hf + 32 * qh + 8 * g + 4 * hi) * 2));
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ch = c * 256 + tid;          // 16-byte chunk: key ch / 16, rows 8 (ch % 16) ..
    tro[c] = opaque_int(tile0 + xtile2_off(ch >> 4, (ch & 15) * 16));
  }
  auto lds = [](int addr) { return reinterpret_cast<lds_char*>((uintptr_t)(unsigned)addr); };

  // stage t (key half KB = t % 2, the ring slot too) of kept block t / 2
  auto step = [&](const int t, auto KBC) __attribute__((always_inline)) {
    constexpr int kb = decltype(KBC)::value;
    constexpr int soff = kb * STAGE;
    if (t == 0) xwait_vmcnt<0>();
    else xwait_vmcnt<4>();   // this slot's copies: only the previous stage's four stores are younger
    __syncthreads();
    issue(t + 1);
    f32x16 acc[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 kf = *reinterpret_cast<__attribute__((address_space(3))) const bf16x8*>(lds(kfo[ks]) + soff);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[0][ks], kf, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf[1][ks], kf, acc[1], 0, 0, 0);
    }
    // causal mask (diagonal block only: key 64 kb + key against row 64 a + r)
    // and rows past the row-block (lse2 = inf)
    const bool dg = __builtin_amdgcn_readfirstlane(jlist[t >> 1]) == diag;
    const int kr = 64 * kb + key;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int e = 4 * g + i;
          p[i] = __builtin_amdgcn_exp2f(fmaf(acc[hf][e], c2, -lse2[hf][e]));
        }
        if (dg) {
          asm volatile("");  // a real branch: at most one block per row-block
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kr > 64 * hf + 32 * qh + 8 * g + 4 * hi + i) p[i] = 0.f;
        }
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 pk = {pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3])};
        *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(lds(two[hf][g])) = pk;
      }
    __syncthreads();
    // 64 key rows of 256 bytes: key 64 kb + kk of value block t / 2
    const char* dst = vbytes + ((size_t)(base + (t >> 1)) * BB * BB + (size_t)(64 * kb) * BB) * 2;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int ch = c * 256 + tid;
      const u32x4 v = *reinterpret_cast<__attribute__((address_space(3))) const u32x4*>(lds(tro[c]));
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(const_cast<char*>(dst) + ((ch >> 4) * BB + (ch & 15) * 8) * 2));
    }
  };
  static_assert(XNST == 2, "two ring slots, one per key half");
  for (int t = 0; t < 2 * n; t += 2) {
    step(t, IC<0>{});
    step(t + 1, IC<1>{});
  }
  xwait_vmcnt<0>();   // the copy issued past the last stage has landed before the LDS is released
}

template <typename T, int B, int D>
int launch_ex(const ExtractArgs& a, void* stream) {
  dim3 grid(xcd_grid(a.b.total_rb, a.H, a.L));
  hipLaunchKernelGGL((extract_kernel<T, B, D>), grid, dim3(B * 4), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

template <typename T>
int launch_ex_d(const ExtractArgs& a, void* stream) {
  switch (a.B * 1000 + a.d) {
    case 32064: return launch_ex<T, 32, 64>(a, stream);
    case 32128: return launch_ex<T, 32, 128>(a, stream);
    case 64064: return launch_ex<T, 64, 64>(a, stream);
    case 64128: return launch_ex<T, 64, 128>(a, stream);
    case 128064: return launch_ex<T, 128, 64>(a, stream);
    case 128128: return launch_ex<T, 128, 128>(a, stream);
  }
  return (int)hipErrorInvalidValue;
}

int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

}  // namespace

size_t select_lds_bytes(int max_cb) {
  const int n2 = next_pow2(max_cb < 1 ? 1 : max_cb);
  return (size_t)n2 * 8 + kSelThreads * 8 + (size_t)((max_cb + 31) / 32) * 4;
}

int launch_select(const SelectArgs& a, void* stream) {
  if (a.b.total_rb == 0 || a.L == 0) return 0;
  const int n2 = next_pow2(a.b.max_cb < 1 ? 1 : a.b.max_cb);
  if (n2 <= 256 && !(forced_portable() & MF_FORCE_PORTABLE_SELECT)) {
    const long long nrows = (long long)a.L * a.H * a.b.total_rb;
    const dim3 grid((unsigned)((nrows + kSelWaves - 1) / kSelWaves));
    auto kern = n2 <= 64 ? select_wave_kernel<1> : n2 <= 128 ? select_wave_kernel<2> : select_wave_kernel<4>;
    hipLaunchKernelGGL(kern, grid, dim3(kSelWaves * 64), 0, (hipStream_t)stream, a, nrows);
    return (int)hipGetLastError();
  }
  const size_t lds = select_lds_bytes(a.b.max_cb);
  hipError_t e = hipFuncSetAttribute((const void*)select_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return (int)e;
  dim3 grid(a.b.total_rb, a.H, a.L);
  hipLaunchKernelGGL(select_kernel, grid, dim3(kSelThreads), lds, (hipStream_t)stream, a, n2);
  return (int)hipGetLastError();
}

int launch_scan(const ScanArgs& a, void* stream) {
  hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

bool extract_fast_path(mf_dtype dt, int B, int d) {
  if (dt != MF_BF16 || (B != 64 && B != 128) || (d != 64 && d != 128)) return false;
  return !(forced_portable() & MF_FORCE_PORTABLE_EXTRACT);
}

size_t extract_mfma_lds_bytes(int d) { return (size_t)XNST * 64 * d * 2; }

int launch_extract(const ExtractArgs& a, mf_dtype dt, void* stream) {
  if (a.b.total_rb == 0 || a.L == 0) return 0;
  if (a.values && a.words <= 64 && extract_fast_path(dt, a.B, a.d)) {
    const size_t lds = extract_mfma_lds_bytes(a.d);
    auto kern = a.B == 128 ? (a.d == 128 ? extract_mfma128_kernel<128> : extract_mfma128_kernel<64>)
                           : (a.d == 128 ? extract_mfma_kernel<128> : extract_mfma_kernel<64>);
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(kern, dim3(xcd_grid(a.b.total_rb, a.H, a.L)), dim3(256), lds, (hipStream_t)stream, a);
    return (int)hipGetLastError();
  }
  return dt == MF_BF16 ? launch_ex_d<bf16>(a, stream) : launch_ex_d<float>(a, stream);
}

}  // namespace mf
