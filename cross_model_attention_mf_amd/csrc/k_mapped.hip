// Fused mapped attention . V (MapFlow page, section "让复用真正省时…",
// paragraph "第三"): read the kept sparse blocks of every sender head, form
// the learned linear head combination on chip, multiply by the receiver's own
// values and accumulate the output; the receiver's dense map never exists.
//
// Portable kernel (any dtype, B, d): one workgroup per (receiver layer,
// row-block, receiver head).  Wave 0 merges the sender heads' sorted column
// lists into their union, one block at a time; the mixed block
// A = sum_h W[r][h] P_h is formed in LDS (fp32) and multiplied by the V tile.
#include <type_traits>

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
    // values are key-major: element (query q, key c) of a block sits at c*B + q
    for (int pos = tid; pos < B * B; pos += kMapThreads) {
      float acc = 0.f;
      unsigned long long mm = mask;
      while (mm) {
        const int h = __builtin_ctzll(mm);
        mm &= mm - 1;
        acc += Wr[h] * to_f32(vals[(size_t)vptr[h] * B * B + pos]);
      }
      A[(pos % B) * B + pos / B] = acc;
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

// ---------------------------------------------------------------------------
// MFMA kernel (bf16, B = 64 or 128).  One workgroup of 8 waves per (receiver
// layer, row-block, 64-row half of a 128-row block, group of 8 receiver
// heads).  The union of the sender heads' kept blocks is walked in 4-key
// stages; for every stage:
//
//   head mix (MFMA 16x16x32, K = sender heads, 32 per chunk):
//     A^T[(c, q)][r] = sum_h P_h[c][q] W[r][h]
//     wave w mixes key 4 s + w / 2 for queries 32 (w & 1) .. + 31; the 16
//     positions of one MFMA are 16 consecutive queries of one key (the
//     transposing LDS read hands lane t the sender heads of query t), the
//     16 columns are the group's receiver heads (8, padded to 16).  Each lane
//     then holds four consecutive queries of one receiver head and stores
//     them as one 8-byte write into the mixed-map buffer A[r][key][q].
//   P.V (MFMA 32x32x16, K = 16 keys): wave w owns receiver head 8 g + w for
//     all 64 rows and d, O_r[q][n] += A_r[q][c] V_r[c][n], once every four
//     stages, over the 16 keys the four stages mixed.
//
// So every staged value of P, of the mixed map and of V is read from LDS
// exactly once per workgroup, and the mixed map never leaves the chip.
//
// Memory pipeline: kept values (key-major rows of 64 queries, 128 bytes) and
// V rows move HBM -> LDS with global_load_lds (16 bytes per lane, no
// registers).  P stages sit in an NS-slot ring; the copies of stage s + NS - 1
// are issued right after the barrier that opens stage s, into the slot stage
// s - 1 consumed.  V rows of a 16-key step arrive in one of NVB buffers: with
// two, step t's rows are issued at its first stage and P.V of step t runs
// spread over the four stages of step t + 1 (one 32-wide n tile per stage);
// with one, they are issued at the second stage of step t and P.V of step t
// runs whole at the first stage of step t + 1.  One counted vmcnt wait plus
// one barrier per stage: every wave issues its P copies last, so the wait
// covers the rows of the stage about to be mixed and every older copy.
// Sender heads that do not keep a block issue no copy: their rows in the
// ring keep finite values of an earlier block (or the initial zeros) and meet
// a zero weight.  Keys past the sequence read a valid V row whose finite
// values meet zero probabilities.  The union merge runs on wave 0, two
// blocks ahead, with the next column of each sender head arriving through an
// async copy.  The copies are inline assembly, which the compiler does not
// track, so it inserts no drain of the ring before LDS accesses; the kernel's
// own waits and barriers order them.
//
// LDS swizzles (16-byte chunks, 64 banks of 4 bytes):
//   P ring [head][4 keys][64 q]: head h keeps its key rows in pair order
//     flipped by gp(h) and its chunks XOR fp(h), so the 16 heads one
//     transposing read touches spread over both bank halves;
//   A [r][16 keys][64 q], head stride 16 * 128 + 32 bytes: chunks XOR sa(key);
//   V [value head][16 keys][d]: chunks XOR sv(key).
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x4 tr_read(const char* lds_generic, unsigned byte_off) {
  auto p = (__attribute__((address_space(3))) i16x4*)((__attribute__((address_space(3))) char*)
           ((uintptr_t)lds_generic) + byte_off);
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p);
  return __builtin_bit_cast(bf16x4, v);
}

// Async copies HBM -> LDS; lane L lands at base + size * L.  Inline assembly
// (one wait state between the M0 write and the copy reading it); the copy
// writes no VGPR.
__device__ __forceinline__ void async_copy16(const void* gsrc, char* lds_generic_base) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_generic_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(gsrc), "s"(base)
               : "memory", "m0");
}
__device__ __forceinline__ void async_copy4(const void* gsrc, char* lds_generic_base) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_generic_base);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" : : "v"(gsrc), "s"(base)
               : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// N copies of 16 bytes per lane whose LDS destinations lie 8 KB apart (one
// M0 write, then increments).  P: a 64-bit address per copy.  V: one 32-bit
// lane offset against a per-copy scalar base.
template <int N>
__device__ __forceinline__ void copy_p(const bf16* const (&src)[N], unsigned m0);
template <>
__device__ __forceinline__ void copy_p<1>(const bf16* const (&src)[1], unsigned m0) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off" : : "v"(src[0]), "s"(m0)
               : "memory", "m0");
}
template <>
__device__ __forceinline__ void copy_p<2>(const bf16* const (&src)[2], unsigned m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off\n\t"
               "s_add_u32 m0, m0, 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off"
               : : "v"(src[0]), "v"(src[1]), "s"(m0) : "memory", "m0", "scc");
}
template <>
__device__ __forceinline__ void copy_p<3>(const bf16* const (&src)[3], unsigned m0) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off\n\t"
               "s_add_u32 m0, m0, 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
               "s_add_u32 m0, m0, 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off"
               : : "v"(src[0]), "v"(src[1]), "v"(src[2]), "s"(m0) : "memory", "m0", "scc");
}
template <>
__device__ __forceinline__ void copy_p<4>(const bf16* const (&src)[4], unsigned m0) {
  asm volatile("s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off\n\t"
               "s_add_u32 m0, m0, 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
               "s_add_u32 m0, m0, 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\t"
               "s_add_u32 m0, m0, 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, off"
               : : "v"(src[0]), "v"(src[1]), "v"(src[2]), "v"(src[3]), "s"(m0) : "memory", "m0", "scc");
}
template <int N>
__device__ __forceinline__ void copy_v(unsigned voff, const char* const (&base)[N], unsigned m0);
template <>
__device__ __forceinline__ void copy_v<1>(unsigned voff, const char* const (&base)[1], unsigned m0) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" : : "v"(voff), "s"(base[0]), "s"(m0)
               : "memory", "m0");
}
template <>
__device__ __forceinline__ void copy_v<2>(unsigned voff, const char* const (&base)[2], unsigned m0) {
  asm volatile("s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
               "s_add_u32 m0, m0, 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
               : : "v"(voff), "s"(base[0]), "s"(base[1]), "s"(m0) : "memory", "m0", "scc");
}
template <>
__device__ __forceinline__ void copy_v<4>(unsigned voff, const char* const (&base)[4], unsigned m0) {
  asm volatile("s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1\n\t"
               "s_add_u32 m0, m0, 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2\n\t"
               "s_add_u32 m0, m0, 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %3\n\t"
               "s_add_u32 m0, m0, 0x2000\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %4"
               : : "v"(voff), "s"(base[0]), "s"(base[1]), "s"(base[2]), "s"(base[3]), "s"(m0)
               : "memory", "m0", "scc");
}
__device__ __forceinline__ unsigned lds_addr(const char* lds_generic) {
  return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)lds_generic);
}

// chunk / row swizzles (see above)
__host__ __device__ constexpr int fp_swz(int h) { return 2 * ((h & 1) | (((h >> 3) & 1) << 1)); }
__host__ __device__ constexpr int gp_swz(int h) { return (h >> 1) & 1; }
__host__ __device__ constexpr int sa_swz(int key) { return 4 * (((key >> 1) ^ (key >> 3)) & 1); }
template <int D>
__host__ __device__ constexpr int sv_swz(int key) {
  return D == 128 ? 4 * ((key & 3) ^ ((key >> 2) & 3)) : 4 * (((key >> 1) ^ (key >> 3)) & 1);
}

struct alignas(16) UnionInfo {
  int j;
  int pad;
  unsigned long long mask;
  int vidx[64];
  int page[128];
};

constexpr int kUnionSlots = 3;
constexpr int kSplitBlocks = 4;   // kept blocks of a unit's longest head per split
constexpr size_t kMapMeta = kUnionSlots * sizeof(UnionInfo) + 64 * sizeof(int) + 8 * 64 * sizeof(float);
constexpr int kMapWaves = 8;
constexpr int kMapRows = 64;   // query rows per workgroup

// LDS plan of the MFMA kernel
template <int B, int D, int HP, int KVC, int NS, int NVB>
struct MapCfg {
  static_assert(B == 64 || B == 128, "64- or 128-row blocks");
  static_assert(HP % 16 == 0 && HP >= 16 && HP <= 64, "sender heads padded to 16");
  static_assert(NS >= 2 && NS <= 8 && (NVB == 1 || NVB == 2), "ring plan");
  static constexpr int QH = B / kMapRows;            // workgroups per row-block
  static constexpr int SPB = B / 4;                  // 4-key stages per block
  static constexpr int SB = B / 16;                  // 16-key steps per block
  static constexpr int PROW = kMapRows * 2;          // bytes of one key row of P (64 queries)
  static constexpr int SLOT = HP * 4 * PROW;         // one stage: HP heads x 4 keys
  static constexpr int VROW = D * 2;
  static constexpr int VCPR = VROW / 16;             // 16-byte chunks per V row
  static constexpr int VRPI = 1024 / VROW;           // V rows per copy instruction
  static constexpr int VB = KVC * 16 * VROW;         // V rows of one 16-key step
  static constexpr int VC = KVC * 16 / VRPI / kMapWaves;   // V copy instructions per wave and step
  static constexpr int AHS = 12 * PROW + 32;         // mixed map, keys 4..15 of a step, per receiver head
  static constexpr int AB = 8 * AHS;
  static constexpr int SHS = 8 * PROW + 32;          // keys 0..3 of a step, two step parities, per receiver head
  static constexpr int SB2 = 8 * SHS;
  static constexpr int VOFF = NS * SLOT;
  static constexpr int AOFF = VOFF + NVB * VB;
  static constexpr int SOFF = AOFF + AB;
  static constexpr int DOFF = SOFF + SB2;            // writes nothing reads: padded mix lanes, dummy copies
  static constexpr int MAIN = DOFF + 2048;
  static constexpr int OST = kMapRows * 8 * D * 2;   // output staging (aliases the buffers above)
  static constexpr int MAINX = ((MAIN > OST ? MAIN : OST) + 15) / 16 * 16;
  static constexpr size_t LDS = (size_t)MAINX + kMapMeta;
  static constexpr int PCW = HP / 16;                // P copy instructions (head pairs) per wave and stage
  static constexpr int NKC = (HP + 31) / 32;         // 16x16x32 chunks of sender heads (the last may be half)
  static constexpr int NT = D / 32;                  // 32-wide n tiles of d
  static constexpr int VPART = NVB == 2 ? 0 : 1;     // stage of a step that issues the step's V rows
  static_assert(16 % VRPI == 0 && VC * VRPI * kMapWaves == KVC * 16, "V rows fill whole copy instructions");
  // copies one wave issues at stage p of a step (P copies, V rows, and the
  // union merge's copies, real on wave 0 at a block's first step and dummies
  // otherwise, so that every wave issues the same count), and how many may
  // still be in flight when stage p opens: those of the NS - 2 stages issued
  // after the copies of stage p
  static constexpr int MC = 1 + B / 64;              // union-merge copies (next columns, page ids)
  static constexpr int ops(int p) { return PCW + (p == VPART ? VC : 0) + (p == 1 ? MC : 0); }
  static constexpr int allow_p(int p) {
    int n = 0;
    for (int b = 1; b <= NS - 2; ++b) n += ops((p - b + 8) & 3);
    return n;
  }
  // The first stage of a step also reads the previous step's V rows, issued
  // at its stage VPART before that stage's merge copies and P: those and every
  // later stage's copies may be in flight.
  static constexpr int allow_v() {
    int n = (VPART == 1 ? MC : 0) + PCW;
    for (int q = VPART + 1; q <= 3; ++q) n += ops(q);
    return n;
  }
  static constexpr int allow(int p) { return p == 0 && allow_v() < allow_p(0) ? allow_v() : allow_p(p); }
};

size_t map_lds_bytes(int B, int D, int HP, int KVC, int NS, int NVB) {
  const size_t prow = 128, slot = (size_t)HP * 4 * prow, vb = (size_t)KVC * 16 * D * 2;
  const size_t ab = 8 * (12 * prow + 32), sb = 8 * (8 * prow + 32);
  const size_t main = NS * slot + NVB * vb + ab + sb + 2048;
  const size_t ost = (size_t)kMapRows * 8 * D * 2;
  const size_t mainx = ((main > ost ? main : ost) + 15) / 16 * 16;
  (void)B;
  return mainx + kMapMeta;
}

// value heads one group of 8 receiver heads reads, at most over the groups
int group_value_heads(int Hr, int Hkv) {
  const int ratio = Hr / Hkv;
  int mx = 0;
  for (int r0 = 0; r0 < Hr; r0 += 8) {
    const int r1 = r0 + 7 < Hr - 1 ? r0 + 7 : Hr - 1;
    const int n = r1 / ratio - r0 / ratio + 1;
    mx = n > mx ? n : mx;
  }
  return mx;
}

// First position in [lo, hi) of an ascending column list whose column is
// >= c (hi if none): eight-way probes while more than eight entries remain,
// so a list of n entries takes about log8(n) + 1 rounds of loads.
__device__ __forceinline__ int64_t lower_col(const int32_t* __restrict__ col, int64_t lo, int64_t hi, int c) {
  while (hi - lo > 8) {
    const int64_t step = (hi - lo + 7) >> 3;
    int k = 0;
#pragma unroll
    for (int t = 1; t < 8; ++t) {
      const int64_t p = lo + t * step;
      k += (p < hi && col[p] < c) ? 1 : 0;
    }
    // probes 1 .. k lie below c: the answer is in (lo + k step, lo + (k + 1) step]
    const int64_t nhi = min(hi, lo + (k + 1) * step);
    lo = k == 0 ? lo : lo + k * step + 1;
    hi = nhi;
  }
  int below = 0;
#pragma unroll
  for (int t = 0; t < 8; ++t) below += (lo + t < hi && col[lo + t] < c) ? 1 : 0;
  return lo + below;
}

// column of an exhausted sender head (the merge copies it instead of a
// col_idx entry)
__device__ const int kNoColumn = 0x7FFFFFFF;

template <int N>
using IC = std::integral_constant<int, N>;

template <int B, int D, int HP, int KVC, int NS, int NVB>
__global__ void __launch_bounds__(kMapWaves * 64)
mapped_mfma_kernel(MappedArgs a, int ngroups) {
  using C = MapCfg<B, D, HP, KVC, NS, NVB>;
  extern __shared__ __align__(16) char smem[];
  char* const ring = smem;
  char* const vbuf = smem + C::VOFF;
  UnionInfo* UI = reinterpret_cast<UnionInfo*>(smem + C::MAINX);
  int* curcol = reinterpret_cast<int*>(UI + kUnionSlots);   // next column of each sender head
  float* Wsh = reinterpret_cast<float*>(curcol + 64);        // [8 receiver heads][64 sender heads]

  // ---- work item.  A unit is one (row-block part, receiver layer); its head
  // groups (those of every receiver of the launch) run back to back on one
  // XCD (workgroup b runs on XCD b % 8), so they share that XCD's L2 for the
  // kept values.  Units are dealt to the XCDs in turn, latest row-blocks
  // first: a row-block's union (and work) grows with its causal range, and
  // the short ones then fill the tail.
  // With union splits, the nsplit workgroups of a unit's head group each
  // walk one column range of its union (split sp), the ranges of one split
  // index following each other group by group.
  const int nitems = a.b.total_rb * C::QH;
  const int nsplit = a.nsplit > 1 ? a.nsplit : 1;
  int item, grp, l, sp;
  {
    const long long nu = (long long)nitems * a.L;
    const long long pos = blockIdx.x / kXcds;
    const long long per = (long long)ngroups * nsplit;
    const long long u = (long long)(blockIdx.x % kXcds) + (long long)kXcds * (pos / per);
    if (u >= nu) return;
    grp = (int)(pos % per % ngroups);
    sp = (int)(pos % per / ngroups);
    item = nitems - 1 - (int)(u / a.L);
    l = (int)(u % a.L);
  }
  // the unit's head group in the split bookkeeping
  const long long ug = ((long long)item * a.L + l) * ngroups + grp;
  // the receiver this group belongs to, and the group's index in it
  int rk = 0;
  for (int k = 1; k < a.nrecv; ++k) rk = grp >= a.rx[k].group0 ? k : rk;
  const MappedRecv R = a.rx[rk];
  grp -= R.group0;
  const int rb = item / C::QH, qoff = (item % C::QH) * kMapRows;
  const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, B, rb);
  const int sl = a.layer_map[l];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lg = lane >> 4, l16 = lane & 15, lh = lane >> 5;
  const bool paged = R.block_table != nullptr;

  // ---- clear the ring and the V / mixed-map buffers (finite values for
  // rows no copy writes), load the group's W rows
  for (int o = tid * 16; o < C::MAIN; o += kMapWaves * 64 * 16)
    *reinterpret_cast<uint4*>(smem + o) = make_uint4(0, 0, 0, 0);
  for (int t = tid; t < 8 * 64; t += kMapWaves * 64) {
    const int rl = t >> 6, h = t & 63, r = 8 * grp + rl;
    Wsh[t] = (h < a.Hs && r < R.Hr) ? R.W[((size_t)l * R.Hr + r) * a.Hs + h] : 0.f;
  }

  // ---- union merge state (wave 0): lane h walks sender head h's sorted list
  int64_t mptr = 0, mend = 0;
  if (wave == 0) {
    int c0 = kNoColumn;
    if (lane < a.Hs) {
      const size_t row = ((size_t)sl * a.Hs + lane) * a.b.total_rb + rb;
      mptr = min((int64_t)a.row_ptr[row], a.csr_capacity);
      mend = min((int64_t)a.row_ptr[row + 1], a.csr_capacity);
    }
    // splits this unit takes: about kSplitBlocks kept blocks of its longest
    // head per split (known from row_ptr alone, so the workgroups of splits
    // past them leave after one round of loads)
    int su = 1;
    if (nsplit > 1) {
      int mx = lane < a.Hs ? (int)(mend - mptr) : 0;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) mx = max(mx, __shfl_xor(mx, off, 64));
      su = max(1, min(nsplit, (mx + kSplitBlocks - 1) / kSplitBlocks));
      if (lane == 0) UI[0].pad = su;
    }
    if (nsplit > 1 && sp < su && su > 1) {
      // The union's columns are gathered as a bitmap in LDS (the merge slot
      // UI[1], unused until the walk starts); split sp walks the union
      // positions [sp U / su, (sp + 1) U / su), that is the columns
      // [c_lo, c_hi) of every head's list.
      unsigned* ubits = reinterpret_cast<unsigned*>(UI[1].vidx);
      const int nw = (ri.ncand + 31) >> 5;   // <= 20 words: 632 column blocks at most
      if (lane < nw) ubits[lane] = 0u;
      if (lane < a.Hs) {
        for (int64_t e0 = mptr; e0 < mend; e0 += 16) {
          int c[16];
#pragma unroll
          for (int t = 0; t < 16; ++t) c[t] = e0 + t < mend ? a.col_idx[e0 + t] : -1;
#pragma unroll
          for (int t = 0; t < 16; ++t)
            if (c[t] >= 0) atomicOr(&ubits[c[t] >> 5], 1u << (c[t] & 31));
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
      const unsigned word = lane < nw ? ubits[lane] : 0u;
      const int pc = __popc(word);
      int incl = pc;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      const int U = __shfl(incl, 63, 64);   // >= the longest head's count, so >= su
      {
        // column of union position k: the owning word's (k - before)-th set bit
        auto column_at = [&](int k) {
          const int before = incl - pc;
          const bool mine = k >= before && k < incl;
          int col = 0;
          if (mine) {
            unsigned wd = word;
            for (int r = k - before; r > 0; --r) wd &= wd - 1u;
            col = 32 * lane + __builtin_ctz(wd);
          }
          return __shfl(col, __builtin_ctzll(__ballot(mine)), 64);
        };
        const int clo = sp == 0 ? 0 : column_at((int)((long long)sp * U / su));
        const int chi = sp == su - 1 ? ri.ncand : column_at((int)((long long)(sp + 1) * U / su));
        if (lane < a.Hs) {
          const int64_t lo = lower_col(a.col_idx, mptr, mend, clo);
          mend = lower_col(a.col_idx, lo, mend, chi);
          mptr = lo;
        }
      }
    }
    // the union's first two blocks, merged from each head's first three
    // columns (one round of plain loads) instead of merge()'s copies
    if (sp >= su) mend = mptr;   // a split past the unit's: nothing to load
    int c1 = kNoColumn, c2 = kNoColumn;
    if (mptr < mend) c0 = a.col_idx[mptr];
    if (mptr + 1 < mend) c1 = a.col_idx[mptr + 1];
    if (mptr + 2 < mend) c2 = a.col_idx[mptr + 2];
    int adv = 0;   // columns this head has given to the two blocks
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      UnionInfo* out = &UI[u];
      const int cur = adv == 0 ? c0 : c1;
      int jm = cur;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) jm = min(jm, __shfl_xor(jm, off, 64));
      const bool take = (cur == jm) && (cur != kNoColumn);
      const unsigned long long m = __ballot(take);
      if (take) {
        out->vidx[lane] = (int)mptr;
        ++mptr;
        ++adv;
      }
      if (lane == 0) { out->j = jm; out->mask = m; }
      // the block's page ids (paged values); the loop's merges fetch the rest
      if (paged && jm != kNoColumn)
        for (int k0 = 0; k0 < B; k0 += 64) {
          const int key = min(jm * B + k0 + lane, ri.klen - 1);
          async_copy4(R.block_table + (size_t)ri.seq * R.max_pages + key / R.page_size,
                      reinterpret_cast<char*>(out->page + k0));
        }
    }
    curcol[lane] = adv == 0 ? c0 : (adv == 1 ? c1 : c2);
  }
  // wave 0: next block of the union and the heads that keep it; the heads'
  // next columns and the block's page ids arrive asynchronously in LDS
  auto merge = [&](UnionInfo* out) {
    const int mcur = curcol[lane];
    int jm = mcur;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) jm = min(jm, __shfl_xor(jm, off, 64));
    const bool take = (mcur == jm) && (mcur != kNoColumn);
    const unsigned long long m = __ballot(take);
    if (take) {
      out->vidx[lane] = (int)mptr;
      ++mptr;
    }
    // every lane copies: the next column of a head that advanced, its current
    // column otherwise, the sentinel once its list is exhausted
    const int* src = mptr < mend ? a.col_idx + mptr : &kNoColumn;
    async_copy4(src, reinterpret_cast<char*>(curcol));
    if (lane == 0) { out->j = jm; out->mask = m; }
    // always B / 64 page copies (dummies when unpaged), so the count is fixed
    const bool pg = paged && jm != kNoColumn;
    for (int k0 = 0; k0 < B; k0 += 64) {
      const int key = pg ? min(jm * B + k0 + lane, ri.klen - 1) : 0;
      async_copy4(pg ? R.block_table + (size_t)ri.seq * R.max_pages + key / R.page_size : &kNoColumn,
                  pg ? reinterpret_cast<char*>(out->page + k0) : smem + C::DOFF);
    }
  };
  // the same number of copies, into the dump area
  auto merge_dummy = [&]() {
#pragma unroll
    for (int c = 0; c < C::MC; ++c) async_copy4(&kNoColumn, smem + C::DOFF);
  };
  wait_vmcnt<0>();   // page ids of the first two blocks
  __syncthreads();
  // splits past the ones this unit takes have nothing to do
  const int su = nsplit > 1 ? __builtin_amdgcn_readfirstlane(UI[0].pad) : 1;
  if (sp >= su) return;

  f32x16 O[2][C::NT];
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) O[qt][nt] = f32x16{};

  if (UI[0].j != kNoColumn) {
    const bf16* __restrict__ vals = reinterpret_cast<const bf16*>(a.values);
    const char* __restrict__ vlayer = reinterpret_cast<const char*>(R.v) + (size_t)l * R.lsv * 2;

    // ---- P copies.  Every wave issues PCW copies per stage.  Instruction
    // (wave, i) copies head pair c = wave + 8 i: lane L writes head
    // 2c + L / 32, physical key row (L / 8) % 4, chunk L % 8 of the stage,
    // which hold logical key row ^ gp(h) and query chunk (L % 8) ^ fp(h).
    // A head that does not keep the block (or does not exist) copies the rows
    // of its partner, else of the block's first keeping head: finite values
    // the mix gives zero weight, fetched from L2 by the copy of their owner.
    const bf16* pcur[C::PCW];      // source of each instruction's next copy
    unsigned pconst[C::PCW];       // the lane's element offset inside a kept block
    {
      const int kp = (lane >> 3) & 3, pc = lane & 7;
#pragma unroll
      for (int i = 0; i < C::PCW; ++i) {
        const int h = 2 * (wave + kMapWaves * i) + lh;
        pconst[i] = (unsigned)((kp ^ gp_swz(h)) * B + qoff + 8 * (pc ^ fp_swz(h)));
      }
    }
    auto prep_p = [&](const UnionInfo* ui) {
      const unsigned long long mk = ui->mask;
      const int h0 = __builtin_ctzll(mk);
#pragma unroll
      for (int i = 0; i < C::PCW; ++i) {
        const int h = 2 * (wave + kMapWaves * i) + lh, hp = h ^ 1;
        const bool mine = h < a.Hs && ((mk >> h) & 1ull);
        const bool partner = hp < a.Hs && ((mk >> hp) & 1ull);
        const int e = ui->vidx[mine ? h : (partner ? hp : h0)];
        pcur[i] = vals + (size_t)e * B * B + pconst[i];
      }
    };
    // issue cursor: stage psi of the block in union slot prot.  Past the
    // union it keeps copying the last block's first stage into slots no stage
    // reads again.
    int psi = 0, prot = 0;
    bool pdone = false;
    auto issue_p = [&](int slot) {
      copy_p<C::PCW>(pcur, lds_addr(ring + (size_t)slot * C::SLOT + (size_t)wave * 1024));
      if (!pdone) {
        if (++psi < C::SPB) {
#pragma unroll
          for (int i = 0; i < C::PCW; ++i) pcur[i] += 4 * B;
        } else {
          psi = 0;
          prot = prot == kUnionSlots - 1 ? 0 : prot + 1;
          const UnionInfo* nx = &UI[prot];
          if (__builtin_amdgcn_readfirstlane(nx->j) == kNoColumn) {
            pdone = true;
#pragma unroll
            for (int i = 0; i < C::PCW; ++i) pcur[i] -= (C::SPB - 1) * 4 * B;
          } else {
            prep_p(nx);
          }
        }
      }
    };

    // ---- V copies.  The group's receiver heads read nkv consecutive value
    // heads kv0 .. kv0 + nkv - 1 (grouped-query attention: ratio receivers
    // per value head), staged once per value head.  Row rho = 16 kvl + key of
    // the buffer holds value head kv0 + kvl at key 16 st + key of the block;
    // lane L of instruction k = wave + 8 i writes row k VRPI + L / VCPR, chunk
    // L % VCPR, which holds d chunk (L % VCPR) ^ sv(key).  A lane's key is the
    // same for every i and the value head steps by KVS, so one lane offset
    // (its token's row) serves every instruction against a scalar base per
    // value head.  Value heads past nkv copy head nkv - 1, and keys past the
    // sequence the sequence's last key: valid rows that nothing reads or that
    // meet zero probabilities.
    const int ratio = R.Hr / R.Hkv;
    const int kv0 = (8 * grp) / ratio;
    const int nkv = min(8 * grp + 7, R.Hr - 1) / ratio - kv0 + 1;
    constexpr int KVS = 8 * C::VRPI / 16;
    const int vrho = wave * C::VRPI + lane / C::VCPR;
    const int vkk = vrho & 15;
    const int kvlw = __builtin_amdgcn_readfirstlane(vrho >> 4);
    const unsigned vchunk = 16u * (unsigned)((lane % C::VCPR) ^ sv_swz<D>(vkk));
    const unsigned vrowb = (unsigned)R.Hkv * D * 2;
    const char* vsb[C::VC];
#pragma unroll
    for (int i = 0; i < C::VC; ++i)
      vsb[i] = vlayer + (size_t)(kv0 + min(kvlw + KVS * i, nkv - 1)) * D * 2;
    // the rows of step st_ of block j (union slot ui); dummies past the union
    auto issue_v = [&](const UnionInfo* ui, int jr, int st_, char* dst, bool real) {
      const int j = real ? jr : 0;
      unsigned tok;
      if (!paged) {
        tok = (unsigned)ri.k0 + (real ? (unsigned)min(j * B + 16 * st_ + vkk, ri.klen - 1) : 0u);
      } else {
        // page ids of keys past the sequence repeat its last key's page
        const int kl = 16 * st_ + vkk;
        int64_t page = real ? ui->page[kl] : 0;
        page = page < 0 ? 0 : (page >= R.num_pages ? R.num_pages - 1 : page);
        const int key = real ? min(j * B + kl, ri.klen - 1) : 0;
        tok = (unsigned)page * (unsigned)R.page_size + (unsigned)(key % R.page_size);
      }
      copy_v<C::VC>(tok * vrowb + vchunk, vsb, lds_addr(dst + (size_t)wave * 1024));
    };

    // ---- this wave's roles
    // mix: key mkey of each stage, queries mq0 .. mq0 + 31; per-lane
    // transposing-read offsets inside a ring slot for (chunk kc, head quad
    // hh, query tile qi), and whether the quad is staged (HP is a multiple
    // of 16, so a 16-lane group's four heads are all staged or all not)
    const int mkey = wave >> 1;
    const int mq0 = 32 * (wave & 1);
    unsigned moff[C::NKC][2][2];
    bool mstaged[C::NKC][2];
#pragma unroll
    for (int kc = 0; kc < C::NKC; ++kc)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int h0 = 32 * kc + 8 * lg + 4 * hh;
        mstaged[kc][hh] = h0 < HP;
        const int h = (h0 < HP ? h0 : 0) + (l16 >> 2);
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) {
          const int q = mq0 + 16 * qi + 4 * (l16 & 3);
          moff[kc][hh][qi] = (unsigned)(h * 4 * C::PROW + (mkey ^ gp_swz(h)) * C::PROW + (((q >> 3) ^ fp_swz(h)) << 4) +
                                        (q & 7) * 2);
        }
      }
    // mixed-map writes: lane (lg, r) stores queries mq0 + 16 qi + 4 lg + 0..3
    // of receiver head r.  Keys 0..3 of a step go to S (two step parities,
    // 512 bytes apart), keys 4..15 to A (stage p at +512 (p - 1)); lanes of
    // the padding heads r >= 8 write the dump area.
    auto chunk_off = [](int q, int swz) { return (((q >> 3) ^ swz) << 4) + (q & 7) * 2; };
    unsigned wS[2], wA[2][2];
#pragma unroll
    for (int qi = 0; qi < 2; ++qi) {
      const int qq = mq0 + 16 * qi + 4 * lg;
      const unsigned dump = (unsigned)(C::DOFF + 8 * (8 * lg + (l16 & 7)));
      wS[qi] = l16 < 8 ? (unsigned)(C::SOFF + l16 * C::SHS + mkey * C::PROW + chunk_off(qq, sa_swz(mkey))) : dump;
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2)
        wA[qi][h2] = l16 < 8 ? (unsigned)(C::AOFF + l16 * C::AHS + mkey * C::PROW +
                                          chunk_off(qq, sa_swz(8 * h2 + mkey)))
                             : dump;
    }
    // P.V: receiver head 8 grp + wave, its value head in the V buffer.  The
    // A operand of query tile qt: lane L takes queries 32 qt + L % 32 and keys
    // 8 (L / 32) + 0..7, two transposing reads (keys +0..3 from S or A,
    // +4..7 from A).
    const int kvl = min((8 * grp + wave) / ratio - kv0, KVC - 1);
    unsigned ao0[2], ao1[2];
    const unsigned aopar = lh == 0 ? 4 * C::PROW : 0;   // S's second parity
#pragma unroll
    for (int qt = 0; qt < 2; ++qt) {
      const int q = 32 * qt + 16 * (lg & 1) + 4 * (l16 & 3);
      const int k0 = 8 * lh + (l16 >> 2), k1 = k0 + 4;
      ao0[qt] = lh == 0 ? (unsigned)(C::SOFF + wave * C::SHS + k0 * C::PROW + chunk_off(q, sa_swz(k0)))
                        : (unsigned)(C::AOFF + wave * C::AHS + (k0 - 4) * C::PROW + chunk_off(q, sa_swz(k0)));
      ao1[qt] = (unsigned)(C::AOFF + wave * C::AHS + (k1 - 4) * C::PROW + chunk_off(q, sa_swz(k1)));
    }
    unsigned voff[C::NT][2];
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int key = 8 * lh + 4 * hh + (l16 >> 2);
        const int n = 32 * nt + 16 * (lg & 1) + 4 * (l16 & 3);
        voff[nt][hh] = (unsigned)(C::VOFF + (kvl * 16 + key) * C::VROW + (((n >> 3) ^ sv_swz<D>(key)) << 4) + (n & 7) * 2);
      }

    // W of the current block as the mix's B operand: lane L supplies receiver
    // head L % 16 (zero past the group's 8 and past Hr) and sender heads
    // 32 kc + 8 (L / 16) + e; heads that do not keep the block (or do not
    // exist) weigh 0
    bf16x8 Wk[C::NKC];
    auto prep_w = [&](const UnionInfo* ui) {
      const unsigned long long mk = ui->mask;
      const float* wrow = Wsh + (l16 & 7) * 64 + 8 * lg;
#pragma unroll
      for (int kc = 0; kc < C::NKC; ++kc) {
        const f32x4 w0 = *reinterpret_cast<const f32x4*>(wrow + 32 * kc);
        const f32x4 w1 = *reinterpret_cast<const f32x4*>(wrow + 32 * kc + 4);
        const unsigned bits = l16 < 8 ? (unsigned)(mk >> (32 * kc + 8 * lg)) & 0xffu : 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          Wk[kc][e] = (bf16)(((bits >> e) & 1u) ? (e < 4 ? w0[e] : w1[e - 4]) : 0.f);
      }
    };

    prep_p(&UI[0]);
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) issue_p(t);

    bf16x8 Aop[2];
    int st = 0, crot = 0, jcur = 0;       // step in block, its UI slot and column block
    int mslot = 0, pslot = NS - 1;        // ring slots mixed / filled (rings of other than 4 slots)
    bool mixing = true, pvv = false;      // this step mixes; the previous one did (its P.V runs now)
    // one stage p of a step of parity PAR
    auto stage = [&](auto PP, auto PAR) -> bool {
      constexpr int p = decltype(PP)::value;
      constexpr int par = decltype(PAR)::value;
      // the wave's copies of this stage and everything older have landed
      wait_vmcnt<C::allow(p)>();
      __syncthreads();
      if constexpr (p == 0) {
        if (mixing && st == 0) {
          jcur = __builtin_amdgcn_readfirstlane(UI[crot].j);
          if (jcur == kNoColumn) mixing = false;
        }
        if (!mixing && !pvv) return false;
      }
      const int ms = NS == 4 ? p : mslot;
      const int is = NS == 4 ? (p + 3) & 3 : pslot;
      // ---- LDS reads first: the mix operands, the previous step's mixed map
      // (stage 0), the V rows of this stage's P.V
      bf16x4 mp[2][C::NKC][2];
      if (mixing) {
#pragma unroll
        for (int qi = 0; qi < 2; ++qi)
#pragma unroll
          for (int kc = 0; kc < C::NKC; ++kc)
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
              // a transposing read hands each lane values from rows other
              // lanes of its 16-lane group address, so it never runs under a
              // partial exec mask: unstaged quads read heads 0..3 and take a
              // zero operand
              const bf16x4 v = tr_read(smem, moff[kc][hh][qi] + (unsigned)(ms * C::SLOT));
              mp[qi][kc][hh] = mstaged[kc][hh] ? v : bf16x4{};
            }
      }
      if constexpr (p == 0) {
        if (pvv) {
#pragma unroll
          for (int qt = 0; qt < 2; ++qt) {
            const bf16x4 lo = tr_read(smem, ao0[qt] + (par == 0 ? aopar : 0u));   // previous step: parity par ^ 1
            const bf16x4 hi = tr_read(smem, ao1[qt]);
            Aop[qt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
      }
      constexpr int vpar = NVB == 2 ? (par ^ 1) : 0;     // V buffer of the previous step
      constexpr int NTS = NVB == 2 ? 1 : C::NT;           // n tiles of P.V at this stage
      constexpr int nt0 = NVB == 2 ? p : 0;
      constexpr bool pv_here = NVB == 2 ? p < C::NT : p == 0;
      bf16x8 vop[NTS];
      if constexpr (pv_here) {
        if (pvv) {
#pragma unroll
          for (int t = 0; t < NTS; ++t) {
            const bf16x4 lo = tr_read(smem, voff[nt0 + t][0] + vpar * C::VB);
            const bf16x4 hi = tr_read(smem, voff[nt0 + t][1] + vpar * C::VB);
            vop[t] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
      }
      if constexpr (p == 0)
        if (mixing && st == 0) prep_w(&UI[crot]);

      // ---- copies: the step's V rows, the union two blocks ahead, P of the
      // stage NS - 1 ahead
      if constexpr (p == C::VPART)
        issue_v(&UI[crot], jcur, st, vbuf + (size_t)(NVB == 2 ? par : 0) * C::VB, mixing);
      if constexpr (p == 1) {
        if (mixing && st == 0 && wave == 0) merge(&UI[crot == 0 ? 2 : crot - 1]);
        else merge_dummy();
      }
      issue_p(is);
      if constexpr (NS != 4) {
        mslot = mslot + 1 == NS ? 0 : mslot + 1;
        pslot = pslot + 1 == NS ? 0 : pslot + 1;
      }

      // ---- head mix of this stage (key 4 p + mkey, queries mq0 .. mq0 + 31),
      // then P.V of the previous step on the matrix pipe while the mix's
      // results are converted and stored
      f32x4 acc[2];
      if (mixing) {
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) {
          acc[qi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kc = 0; kc < C::NKC; ++kc) {
            const bf16x8 op = __builtin_shufflevector(mp[qi][kc][0], mp[qi][kc][1], 0, 1, 2, 3, 4, 5, 6, 7);
            acc[qi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(op, Wk[kc], acc[qi], 0, 0, 0);
          }
        }
      }
      if constexpr (pv_here) {
        if (pvv) {
#pragma unroll
          for (int t = 0; t < NTS; ++t)
#pragma unroll
            for (int qt = 0; qt < 2; ++qt)
              O[qt][nt0 + t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Aop[qt], vop[t], O[qt][nt0 + t], 0, 0, 0);
        }
      }
      if (mixing) {
#pragma unroll
        for (int qi = 0; qi < 2; ++qi) {
          bf16x4 o4;
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = (bf16)acc[qi][i];
          const unsigned off = p == 0 ? wS[qi] + par * 4 * C::PROW : wA[qi][p >> 1] + (p - 1) * 4 * C::PROW;
          *reinterpret_cast<bf16x4*>(smem + off) = o4;
        }
      }
      return true;
    };
    auto end_step = [&]() {
      pvv = mixing;
      if (mixing && ++st == C::SB) {
        st = 0;
        crot = crot == kUnionSlots - 1 ? 0 : crot + 1;
      }
    };
    for (;;) {
      if (!stage(IC<0>{}, IC<0>{})) break;
      stage(IC<1>{}, IC<0>{});
      stage(IC<2>{}, IC<0>{});
      stage(IC<3>{}, IC<0>{});
      end_step();
      if (!stage(IC<0>{}, IC<1>{})) break;
      stage(IC<1>{}, IC<1>{});
      stage(IC<2>{}, IC<1>{});
      stage(IC<3>{}, IC<1>{});
      end_step();
    }
  }

  // ---- output: stage [q][8 heads][d] in LDS, then 16-byte stores of whole rows
  wait_vmcnt<0>();
  if (nsplit > 1 && sp == 0 && tid == 0) a.split_count[ug] = su;
  if (su > 1) {
    // a split's fp32 partial, [q][8 heads][d], straight from the registers
    // (lanes 0-31 and 32-63 each write 128 contiguous bytes of a row)
    float* __restrict__ pd = a.partial + ((size_t)ug * nsplit + sp) * (size_t)(kMapRows * 8 * D);
#pragma unroll
    for (int qt = 0; qt < 2; ++qt)
#pragma unroll
      for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int qq = 32 * qt + 8 * (i >> 2) + 4 * lh + (i & 3);
          pd[((size_t)qq * 8 + wave) * D + 32 * nt + (lane & 31)] = O[qt][nt][i];
        }
    return;
  }
  __syncthreads();
  bf16* stage = reinterpret_cast<bf16*>(smem);
#pragma unroll
  for (int qt = 0; qt < 2; ++qt)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int qq = 32 * qt + 8 * (i >> 2) + 4 * lh + (i & 3);
        stage[((size_t)qq * 8 + wave) * D + 32 * nt + (lane & 31)] = (bf16)O[qt][nt][i];
      }
  __syncthreads();
  bf16* __restrict__ obase = reinterpret_cast<bf16*>(R.o) + (size_t)l * R.lso;
  const int heads_here = min(8, R.Hr - 8 * grp);
  constexpr int CPQ = 8 * D * 2 / 16;                  // 16-byte chunks per query row
  for (int c = tid; c < kMapRows * CPQ; c += kMapWaves * 64) {
    const int qq = c / CPQ, k = c % CPQ;
    const int hl = (k * 8) / D;
    if (qoff + qq < ri.rows && hl < heads_here) {
      bf16* dst = obase + ((size_t)(ri.q0 + qoff + qq) * R.Hr + 8 * grp) * D + (size_t)k * 8;
      // non-temporal: O is not read again here, and the kept values and V
      // rows other workgroups still read stay in L2
      const u32x4 ov = *reinterpret_cast<const u32x4*>(stage + (size_t)qq * 8 * D + (size_t)k * 8);
      __builtin_nontemporal_store(ov, reinterpret_cast<u32x4*>(dst));
    }
  }
}

// Largest ring / V-buffer plan whose LDS fits, preferring a 4-slot ring with
// two V buffers.  Returns false if none fits.
bool map_plan(int B, int D, int HP, int KVC, size_t lds_limit, int* ns, int* nvb) {
  static const int plans[][2] = {{4, 2}, {4, 1}, {3, 2}, {3, 1}, {2, 1}};
  for (const auto& p : plans)
    if (map_lds_bytes(B, D, HP, KVC, p[0], p[1]) <= lds_limit) {
      *ns = p[0];
      *nvb = p[1];
      return true;
    }
  return false;
}

template <int B, int D, int HP, int KVC, int NS, int NVB>
int launch_fast_cfg(const MappedArgs& a, void* stream) {
  using C = MapCfg<B, D, HP, KVC, NS, NVB>;
  // plans past the 160 KB of LDS are never chosen (map_plan); none is built
  if constexpr (C::LDS > 163840) {
    return (int)hipErrorInvalidValue;
  } else {
  auto kern = mapped_mfma_kernel<B, D, HP, KVC, NS, NVB>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)C::LDS);
  if (e != hipSuccess) return (int)e;
  int ngroups = 0;
  for (int k = 0; k < a.nrecv; ++k) ngroups += (a.rx[k].Hr + 7) / 8;
  const long long nu = (long long)a.b.total_rb * C::QH * a.L;
  const long long per_xcd = (nu + kXcds - 1) / kXcds * ngroups * (a.nsplit > 1 ? a.nsplit : 1);
  hipLaunchKernelGGL(kern, dim3((unsigned)(per_xcd * kXcds)), dim3(kMapWaves * 64), C::LDS, (hipStream_t)stream,
                     a, ngroups);
  return (int)hipGetLastError();
  }
}

template <int B, int D, int HP, int KVC>
int launch_fast_p(const MappedArgs& a, void* stream, int ns, int nvb) {
  if (ns == 4 && nvb == 2) return launch_fast_cfg<B, D, HP, KVC, 4, 2>(a, stream);
  if (ns == 4 && nvb == 1) return launch_fast_cfg<B, D, HP, KVC, 4, 1>(a, stream);
  if (ns == 3 && nvb == 2) return launch_fast_cfg<B, D, HP, KVC, 3, 2>(a, stream);
  if (ns == 3 && nvb == 1) return launch_fast_cfg<B, D, HP, KVC, 3, 1>(a, stream);
  return launch_fast_cfg<B, D, HP, KVC, 2, 1>(a, stream);
}

template <int B, int D, int KVC>
int launch_fast_k(const MappedArgs& a, void* stream, int ns, int nvb) {
  switch ((a.Hs + 15) / 16) {
    case 1: return launch_fast_p<B, D, 16, KVC>(a, stream, ns, nvb);
    case 2: return launch_fast_p<B, D, 32, KVC>(a, stream, ns, nvb);
    case 3: return launch_fast_p<B, D, 48, KVC>(a, stream, ns, nvb);
    case 4: return launch_fast_p<B, D, 64, KVC>(a, stream, ns, nvb);
  }
  return (int)hipErrorInvalidValue;
}

// V buffers sized for 4 value heads per group when the grouped-query
// layout allows, else for 8
static int max_group_value_heads(const MappedArgs& a) {
  int m = 0;
  for (int k = 0; k < a.nrecv; ++k) {
    const int g = group_value_heads(a.rx[k].Hr, a.rx[k].Hkv);
    m = g > m ? g : m;
  }
  return m;
}

template <int B, int D>
int launch_fast(const MappedArgs& a, void* stream, int kvc, int ns, int nvb) {
  return kvc <= 4 ? launch_fast_k<B, D, 4>(a, stream, ns, nvb) : launch_fast_k<B, D, 8>(a, stream, ns, nvb);
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

// Sum of a unit's split partials (in split order, so repeated calls give the
// same bits) into its bf16 output rows.  Workgroup (unit head group ug, row
// slice z) covers kRedRows query rows x 8 receiver heads x d: each thread
// issues the loads of all its chunks' partials at once, then adds them.
// Units that took one split wrote their output themselves.
constexpr int kRedRows = 4;
template <int D>
__global__ void __launch_bounds__(256) mapped_split_reduce_kernel(MappedArgs a, int ngroups, int qh) {
  constexpr int SL = kMapRows / kRedRows;        // row slices per unit head group
  constexpr int NC = kRedRows * 8 * D / 4 / 256; // 16-byte chunks per thread
  const long long ug = blockIdx.x / SL;
  const int z = blockIdx.x % SL;
  const int su = a.split_count[ug];
  if (su <= 1) return;
  const int grp = (int)(ug % ngroups);
  const long long t = ug / ngroups;
  const int l = (int)(t % a.L), item = (int)(t / a.L);
  const int rb = item / qh, qoff = (item % qh) * kMapRows + kRedRows * z;
  const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, a.B, rb);
  const int heads_here = min(8, a.Hr - 8 * grp);
  constexpr int PER = kMapRows * 8 * D;          // floats of one split's partial
  const float* __restrict__ src = a.partial + (size_t)ug * a.nsplit * PER + (size_t)kRedRows * z * 8 * D;
  bf16* __restrict__ obase = reinterpret_cast<bf16*>(a.o) + (size_t)l * a.lso;
  f32x4 v[NC][8];
#pragma unroll
  for (int k = 0; k < NC; ++k)
#pragma unroll
    for (int s2 = 0; s2 < 8; ++s2)
      if (s2 < su) v[k][s2] = *reinterpret_cast<const f32x4*>(src + (size_t)s2 * PER + 4 * (threadIdx.x + 256 * k));
#pragma unroll
  for (int k = 0; k < NC; ++k) {
    const int idx = 4 * (threadIdx.x + 256 * k);
    const int row = idx / (8 * D), hd = (idx / D) % 8, d0 = idx % D;
    f32x4 acc = v[k][0];
#pragma unroll
    for (int s2 = 1; s2 < 8; ++s2)
      if (s2 < su) {
        acc[0] += v[k][s2][0]; acc[1] += v[k][s2][1]; acc[2] += v[k][s2][2]; acc[3] += v[k][s2][3];
      }
    if (qoff + row < ri.rows && hd < heads_here) {
      bf16x4 o4;
#pragma unroll
      for (int i = 0; i < 4; ++i) o4[i] = (bf16)acc[i];
      *reinterpret_cast<bf16x4*>(obase + ((size_t)(ri.q0 + qoff + row) * a.Hr + 8 * grp + hd) * D + d0) = o4;
    }
  }
}

}  // namespace

// The MFMA kernel's plan for these shapes (false: the portable kernel runs)
static bool mapped_mfma_plan(const MappedArgs& a, mf_dtype dt, bool allow_fast, size_t lds_limit, int* kvc, int* ns,
                             int* nvb) {
  if (dt != MF_BF16 || !allow_fast || (a.B != 64 && a.B != 128) || (a.d != 64 && a.d != 128)) return false;
  // V rows are addressed by 32-bit byte offsets inside one layer
  for (int k = 0; k < a.nrecv; ++k)
    if ((uint64_t)a.rx[k].vrows * (uint64_t)a.rx[k].Hkv * (uint64_t)a.d * 2u > 0xFFFFFFFFull) return false;
  *kvc = max_group_value_heads(a) <= 4 ? 4 : 8;
  const int hp = (a.Hs + 15) / 16 * 16;
  return map_plan(a.B, a.d, hp, *kvc, lds_limit, ns, nvb);
}

int launch_mapped(const MappedArgs& a, mf_dtype dt, void* stream, bool allow_fast, size_t lds_limit) {
  if (a.b.total_rb == 0 || a.L == 0) return 0;
  int kvc = 0, ns = 0, nvb = 0;
  if (mapped_mfma_plan(a, dt, allow_fast, lds_limit, &kvc, &ns, &nvb)) {
    switch (a.B * 1000 + a.d) {
      case 64064: return launch_fast<64, 64>(a, stream, kvc, ns, nvb);
      case 64128: return launch_fast<64, 128>(a, stream, kvc, ns, nvb);
      case 128064: return launch_fast<128, 64>(a, stream, kvc, ns, nvb);
      case 128128: return launch_fast<128, 128>(a, stream, kvc, ns, nvb);
    }
  }
  return dt == MF_BF16 ? launch_gd<bf16>(a, stream) : launch_gd<float>(a, stream);
}

// Union splits for a launch too small to fill the chip: enough that the
// launch has about kSplitTarget workgroups, at most 8 per unit (a unit takes
// fewer when its heads keep few blocks).  One receiver, MFMA kernel only.
constexpr long long kSplitTarget = 1024;

int mapped_splits(const MappedArgs& a, mf_dtype dt, bool allow_fast, size_t lds_limit) {
  if (a.b.total_rb == 0 || a.L == 0 || a.nrecv != 1) return 1;
  int kvc = 0, ns = 0, nvb = 0;
  if (!mapped_mfma_plan(a, dt, allow_fast, lds_limit, &kvc, &ns, &nvb)) return 1;
  const long long wg = (long long)a.b.total_rb * (a.B / kMapRows) * a.L * ((a.Hr + 7) / 8);
  const long long s = (kSplitTarget + wg - 1) / wg;
  return (int)(s < 1 ? 1 : (s > 8 ? 8 : s));
}

size_t mapped_split_workspace_bytes(const MappedArgs& a, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t ug = (size_t)a.b.total_rb * (a.B / kMapRows) * a.L * ((a.Hr + 7) / 8);
  return (ug * 4 + 255) / 256 * 256 + ug * nsplit * (size_t)kMapRows * 8 * a.d * 4;
}

int launch_mapped_split(MappedArgs a, mf_dtype dt, void* ws, void* stream, bool allow_fast, size_t lds_limit) {
  const int ns = mapped_splits(a, dt, allow_fast, lds_limit);
  if (ns <= 1) {
    a.nsplit = 0;
    return launch_mapped(a, dt, stream, allow_fast, lds_limit);
  }
  const size_t ug = (size_t)a.b.total_rb * (a.B / kMapRows) * a.L * ((a.Hr + 7) / 8);
  a.nsplit = ns;
  a.split_count = reinterpret_cast<int32_t*>(ws);
  a.partial = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (ug * 4 + 255) / 256 * 256);
  int e = launch_mapped(a, dt, stream, allow_fast, lds_limit);
  if (e) return e;
  const int ngroups = (a.Hr + 7) / 8;
  const dim3 grid((unsigned)(ug * (kMapRows / kRedRows)));
  auto reduce = a.d == 128 ? mapped_split_reduce_kernel<128> : mapped_split_reduce_kernel<64>;
  hipLaunchKernelGGL(reduce, grid, dim3(256), 0, (hipStream_t)stream, a, ngroups, a.B / kMapRows);
  return (int)hipGetLastError();
}

int launch_mapped_multi(const MappedArgs& a, mf_dtype dt, void* stream, bool allow_fast, size_t lds_limit) {
  if (a.b.total_rb == 0 || a.L == 0) return 0;
  int kvc = 0, ns = 0, nvb = 0;
  if (mapped_mfma_plan(a, dt, allow_fast, lds_limit, &kvc, &ns, &nvb))
    return launch_mapped(a, dt, stream, allow_fast, lds_limit);
  // one launch per receiver
  for (int k = 0; k < a.nrecv; ++k) {
    MappedArgs one = a;
    const MappedRecv& r = a.rx[k];
    one.W = r.W; one.v = r.v; one.o = r.o; one.lsv = r.lsv; one.lso = r.lso;
    one.block_table = r.block_table; one.page_size = r.page_size; one.max_pages = r.max_pages;
    one.num_pages = r.num_pages; one.Hr = r.Hr; one.Hkv = r.Hkv;
    one.nrecv = 1;
    one.rx[0] = r;
    one.rx[0].group0 = 0;
    const int e = launch_mapped(one, dt, stream, allow_fast, lds_limit);
    if (e) return e;
  }
  return 0;
}

}  // namespace mf
