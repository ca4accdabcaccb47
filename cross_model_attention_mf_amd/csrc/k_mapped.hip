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
// MFMA kernel (bf16).  One workgroup per (receiver layer, row-block, 64-row
// half of a 128-row block, group of 8 receiver heads); 2 x RQ/16 waves, wave
// (hq, qt) owning receiver heads 4hq..4hq+3 of the group and query rows
// 16qt..16qt+15.  Each block j of the union of the sender heads' kept sets is
// walked in 32-key steps; a step is 4 stages g2 = 0..3, and stage g2 stages
// the 8 keys 32cb + 8 g2 + e (e = 0..7) of every sender head in LDS.
//
//   head mix (MFMA 16x16x32, K = sender heads, W block-diagonal in the key
//   group):  C_e[(g, r)][q] += sum_h [g == g2] W[r][h] P_h[32cb + 8 g2 + e][q]
//   so lane (g, q) holds, for e = 0..7, the mixed map A_r[q][32cb + 8g + e]:
//   exactly the A operand (8 keys per lane group) of the P.V MFMA, and the
//   mixed map never leaves registers.
//   P.V (MFMA 16x16x32, K = keys): O_r[q][n] += A_r[q][c] V_r[c][n].
//
// Two memory pipelines; key-major block rows (RQ contiguous queries) are
// copied HBM -> LDS with global_load_lds (16 bytes per lane, no registers).
//
// Half-stage ring (when the sender heads, padded to a multiple of 16, leave
// room for five 4-key slots beside a 32-key V buffer): stage s mixes the
// half-stages 2s and 2s+1 and, right after the barrier that opens it, issues
// 2s+3 and 2s+4 into the slots stage s-1 consumed, so one and a half stages
// are in flight.  A slot holds 4 key rows per head, unpadded; odd heads hold
// each key pair swapped, so a transpose read of one key meets neighbouring
// heads in opposite bank halves.  One copy covers a pair of heads.  The V
// rows of a 32-key step arrive at its first stage, and P.V runs once per
// step, after stage 3, over all 32 keys.
//
// Stage ring (other shapes): a 3-slot ring of 8-key stages (2 when the
// sender heads leave LDS for only two), each head's rows padded by 128 bytes:
// the copies of stage s + 2 are issued at stage s.  Key groups not yet mixed
// are still zero, so P.V runs twice per step, after stages 1 and 3, each
// time over the 16 keys whose V rows are in LDS.  The V rows of a 16-key
// half arrive in their own buffer, issued at the half's first stage and used
// after its second (or one half ahead with two buffers).  V rows are staged once per
// value head the group's receiver heads read (grouped-query receivers share
// them), not once per receiver head.  Only sender heads that keep the block
// issue P copies; the slot of an absent head keeps finite values from an
// earlier block (or the initial zeros), which meet a zero weight.  Every
// stage issues its P copies last, so one counted wait at the top of each
// stage (vmcnt = the wave's newest P copies, a wave-uniform count; 0 with a
// 2-slot ring) covers the rows the stage reads and the V rows of its step.  The copies are issued as inline
// assembly, which the compiler does not track, so it inserts no drain of the
// ring before LDS accesses; the kernel's own waits and barriers order them.
// The column lists of the sender heads and the page ids of paged values also
// arrive through async LDS copies.  Keys past the sequence read a valid row
// whose finite values meet zero probabilities.  Operands are read
// with ds_read_tr16_b64 (lane t of a 16-lane group gets column t of a 4-row
// tile) from rows whose 16-byte chunks are XOR-swizzled.
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
// wait until at most n (wave-uniform, 0 <= n <= M) vector memory operations
// of this wave are outstanding
template <int M>
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  static_assert(M <= 15, "wait range");
  switch (n < M ? n : M) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<M>(); break;
  }
}

// A copy of a lane value the compiler cannot see through: per-stage address
// math derived from it is recomputed in place (a few VALU ops) instead of
// being hoisted out of the stage loop and pinned in registers.
__device__ __forceinline__ int opaque(int x) {
  int y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}

// P rows of one head (8 keys x RQ queries) sit in a group padded by 128
// bytes, so heads of opposite parity start half an LDS bank cycle apart, and
// each head's 16-byte chunks are XOR-swizzled by swz_p(h): the 16 heads one
// transpose read touches (4 per 16-lane group, 32 bytes each) then cover all
// 64 banks.  V rows (one key, D values) are swizzled by swz_v(row), which
// gives the 8 rows read together 8 distinct chunk pairs.
__host__ __device__ constexpr int swz_p(int h) { return 2 * (((h >> 1) & 1) | (((h >> 3) & 1) << 1)); }
__device__ __forceinline__ int swz_v(int row, int cpr) { return (2 * ((row & 3) | (((row >> 3) & 1) << 2))) & (cpr - 1); }

struct alignas(16) UnionInfo {
  int j;
  int pad;
  unsigned long long mask;
  int vidx[64];
  int page[128];
};

constexpr size_t kMapMeta = 2 * sizeof(UnionInfo) + 64 * sizeof(int) + 8 * 64 * sizeof(float);

template <int B, int D, int HP8, int KVC>
struct MapCfg {
  static_assert(B >= 64, "the MFMA kernel covers 64-row query tiles");
  static constexpr int RQ = 64;                        // query rows per workgroup
  static constexpr int NQT = RQ / 16;                  // query tiles
  static constexpr int NW = 2 * NQT;                   // waves
  static constexpr int NT = D / 16;                    // 16-wide n tiles of d
  static constexpr int CB = B / 32;                    // 32-key steps per block
  static constexpr int SPU = 4 * CB;                   // 8-key stages per block
  static constexpr int QH = B / RQ;                    // workgroups per row-block
  static constexpr int PROW = RQ * 2;                  // bytes per P row (one key, RQ queries)
  static constexpr int HSTR = 8 * PROW + 128;          // bytes per head group of 8 P rows
  static constexpr int VROW = D * 2;                   // bytes per V row
  static constexpr int VCPR = VROW / 16;
  static constexpr int VB = KVC * 16 * VROW;           // one V buffer: KVC value heads x 16 keys
  static constexpr int HPAD = 8 * HP8;
  static constexpr int SBYTES = HPAD * HSTR;           // one stage: 8 keys x all heads
  static constexpr bool fits(int ns, int nv) { return (size_t)ns * SBYTES + (size_t)nv * VB + kMapMeta <= 163840; }
  static constexpr int NSLOT = fits(3, 2) || fits(3, 1) ? 3 : 2;  // P ring slots
  static constexpr int NVB = fits(NSLOT, 2) ? 2 : 1;   // V buffers
  static constexpr int VBYTES = NVB * VB;
  static constexpr int AHEAD = NSLOT - 1;              // stages issued ahead of the mix
  static constexpr int PW = HPAD / NW;                 // P copy instructions (heads) per wave per stage
  static constexpr int RPI = 1024 / VROW;              // V rows per copy instruction
  static_assert(HPAD % NW == 0, "P copies must split evenly over the waves");
  static_assert(16 % RPI == 0, "a value head's 16 rows fill whole copy instructions");
  // half-stage ring: NHS slots of 4 key rows per head, unpadded, beside a
  // V buffer of 32 keys (P.V then covers 32 live keys)
  static constexpr int NHS = 5;
  static constexpr int HSB = HPAD * 4 * PROW;          // one half-slot
  static constexpr int VB32 = KVC * 32 * VROW;
  static constexpr bool HALF = (HPAD / 2) % NW == 0 && (size_t)NHS * HSB + (size_t)VB32 + kMapMeta <= 163840;
  static constexpr int PWH = HPAD / 2 / NW;            // head-pair copies per wave per half-stage
  static constexpr int HPU = B / 4;                    // half-stages per block
  static constexpr int RING = HALF ? NHS * HSB : NSLOT * SBYTES;
  static constexpr int VK = HALF ? 32 : 16;            // keys per V buffer
  static constexpr int VBUF = HALF ? VB32 : VB;
  static constexpr int VTOT = HALF ? VB32 : VBYTES;
};

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

size_t mapped_mfma_lds_bytes(int B, int D, int Hs, int kvc) {
  if (B < 64) return (size_t)1 << 40;                  // no MFMA kernel for 32-row blocks
  const size_t hpad = (size_t)(Hs + 7) / 8 * 8;
  const size_t stage = hpad * (8 * 128 + 128);
  const size_t vb = (size_t)kvc * 16 * D * 2;
  auto fits = [&](size_t ns, size_t nv) { return ns * stage + nv * vb + kMapMeta <= 163840; };
  const size_t nslot = fits(3, 2) || fits(3, 1) ? 3 : 2;
  const size_t nvb = fits(nslot, 2) ? 2 : 1;
  const size_t obytes = (size_t)64 * 8 * D * 2;       // output staging (aliases the ring and V)
  size_t main = nslot * stage + nvb * vb;
  const size_t hsb = hpad * 4 * 128, vb32 = (size_t)kvc * 32 * D * 2;
  if (hpad % 16 == 0 && 5 * hsb + vb32 + kMapMeta <= 163840) main = 5 * hsb + vb32;
  if (obytes > main) main = obytes;
  return main + kMapMeta;
}

// column of an exhausted sender head (the merge copies it instead of a
// col_idx entry)
__device__ const int kNoColumn = 0x7FFFFFFF;

template <int B, int D, int HP8, int KVC>
__global__ void __launch_bounds__(((B < 64 ? B : 64) / 16) * 2 * 64)
mapped_mfma_kernel(MappedArgs a, int ngroups) {
  using C = MapCfg<B, D, HP8, KVC>;
  constexpr int hpad = C::HPAD;
  extern __shared__ __align__(16) char smem[];
  char* ring = smem;
  char* Vs = smem + C::RING;
  size_t main_bytes = C::RING + C::VTOT;
  if ((size_t)C::RQ * 8 * D * 2 > main_bytes) main_bytes = (size_t)C::RQ * 8 * D * 2;
  UnionInfo* UI = reinterpret_cast<UnionInfo*>(smem + main_bytes);
  int* curcol = reinterpret_cast<int*>(UI + 2);        // next column of each sender head
  float* Wsh = reinterpret_cast<float*>(curcol + 64);   // [8 receiver heads][64 sender heads]

  // ---- work item.  A unit is one (row-block part, receiver layer); its head
  // groups (those of every receiver of the launch) run back to back on one
  // XCD (workgroup b runs on XCD b % 8), so they share that XCD's L2 for the
  // kept values.  Units are dealt to the
  // XCDs in turn, latest row-blocks first: a row-block's union (and work)
  // grows with its causal range, and the short ones then fill the tail.
  const int nitems = a.b.total_rb * C::QH;
  int item, grp, l;
  {
    const long long nu = (long long)nitems * a.L;
    const long long pos = blockIdx.x / kXcds;
    const long long u = (long long)(blockIdx.x % kXcds) + (long long)kXcds * (pos / ngroups);
    if (u >= nu) return;
    grp = (int)(pos % ngroups);
    item = nitems - 1 - (int)(u / a.L);
    l = (int)(u % a.L);
  }
  // the receiver this group belongs to, and the group's index in it
  int rk = 0;
  for (int k = 1; k < a.nrecv; ++k) rk = grp >= a.rx[k].group0 ? k : rk;
  const MappedRecv R = a.rx[rk];
  grp -= R.group0;
  const int rb = item / C::QH, qoff = (item % C::QH) * C::RQ;
  const RowBlockInfo ri = rowblock_info(a.b.plan, a.b.num_seqs, a.b.cu_q, a.b.cu_k, a.b.q_pos0, B, rb);
  const int sl = a.layer_map[l];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hq = wave / C::NQT, qt = wave % C::NQT;
  const int lg = lane >> 4, lr = lane & 15;
  const bool paged = R.block_table != nullptr;

  // ---- zero the ring and V rows, load the group's W rows
  for (size_t o = (size_t)tid * 16; o < main_bytes; o += (size_t)C::NW * 64 * 16)
    *reinterpret_cast<uint4*>(smem + o) = make_uint4(0, 0, 0, 0);
  for (int t = tid; t < 8 * 64; t += C::NW * 64) {
    const int rl = t >> 6, h = t & 63, r = 8 * grp + rl;
    Wsh[t] = (h < a.Hs && r < R.Hr) ? R.W[((size_t)l * R.Hr + r) * a.Hs + h] : 0.f;
  }

  // ---- union merge state (wave 0): lane h walks sender head h's sorted list
  int64_t mptr = 0, mend = 0;
  if (wave == 0) {
    int c0 = 0x7FFFFFFF;
    if (lane < a.Hs) {
      const size_t row = ((size_t)sl * a.Hs + lane) * a.b.total_rb + rb;
      mptr = min((int64_t)a.row_ptr[row], a.csr_capacity);
      mend = min((int64_t)a.row_ptr[row + 1], a.csr_capacity);
      if (mptr < mend) c0 = a.col_idx[mptr];
    }
    curcol[lane] = c0;
  }
  // wave 0: next block of the union and the heads that keep it; the heads'
  // next columns and the block's page ids arrive asynchronously in LDS
  auto merge = [&](UnionInfo* out) {
    int copies = 1;
    const int mcur = curcol[lane];
    int jm = mcur;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) jm = min(jm, __shfl_xor(jm, off, 64));
    const bool take = (mcur == jm) && (mcur != 0x7FFFFFFF);
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
    if (paged && jm != 0x7FFFFFFF) {
      for (int k0 = 0; k0 < B; k0 += 64) {
        const int key = min(jm * B + k0 + lane, ri.klen - 1);
        async_copy4(R.block_table + (size_t)ri.seq * R.max_pages + key / R.page_size,
                    reinterpret_cast<char*>(out->page + k0));
        ++copies;
      }
    }
    return copies;
  };
  __syncthreads();
  if (wave == 0) merge(&UI[0]);
  wait_vmcnt<0>();
  __syncthreads();

  const bf16* __restrict__ vals = reinterpret_cast<const bf16*>(a.values);
  const bf16* __restrict__ vbase = reinterpret_cast<const bf16*>(R.v) + (size_t)l * R.lsv;

  // P copies: instruction (wave, i) copies head h = wave + i NW, lane L row
  // e = L / 8 (key 8 si + e of the block), chunk L % 8 from source chunk
  // (L % 8) ^ swz_p(h).  Sources are prepared once per union block, so a
  // stage adds one offset.  Heads that do not keep the block issue no copy:
  // their slot keeps an earlier block's finite values (or the initial
  // zeros), which meet a zero weight in the head mix.
  const bf16* pbase[C::PW];
  unsigned plive = 0;   // bit i: copy slot i of this wave reads a kept block
  auto prep_p = [&](const UnionInfo* ui) {
    const unsigned long long mk = ui ? ui->mask : 0ull;
    const int e = lane >> 3, pc = lane & 7;
    unsigned bits = 0;
#pragma unroll
    for (int i = 0; i < C::PW; ++i) {
      const int h = wave + i * C::NW;
      const int sc = pc ^ swz_p(h);
      const bool live = h < a.Hs && ((mk >> h) & 1ull);
      pbase[i] = live ? vals + (size_t)ui->vidx[h] * B * B + (size_t)e * B + qoff + 8 * sc : vals;
      bits |= live ? 1u << i : 0u;
    }
    plive = __builtin_amdgcn_readfirstlane(bits);
  };
  auto issue_p = [&](int si, char* buf) {
#pragma unroll
    for (int i = 0; i < C::PW; ++i)
      if ((plive >> i) & 1u)
        async_copy16(pbase[i] + (size_t)si * 8 * B, buf + (size_t)(wave + i * C::NW) * C::HSTR);
    return __builtin_popcount(plive);
  };
  // Half-stage copies: instruction (wave, i) copies head pair c = wave + i NW,
  // lane L head 2c + L / 32, row r = (L / 8) % 4, chunk L % 8.  Row r of
  // head h holds key r ^ (h & 1) of the half-stage (odd heads swap key
  // pairs, which puts the same key of neighbouring heads in opposite bank
  // halves), chunk from source chunk (L % 8) ^ swz_p(h).  A pair issues a
  // copy when either head keeps the block; the lanes of a head that does not
  // keep it read rows of the first stored block instead (finite values that
  // meet a zero weight).
  const bf16* hbase[C::HALF ? C::PWH : 1];
  unsigned hlive = 0;
  auto prep_h = [&](const UnionInfo* ui) {
    const unsigned long long mk = ui ? ui->mask : 0ull;
    const int r = (lane >> 3) & 3, pc = lane & 7;
    unsigned bits = 0;
#pragma unroll
    for (int i = 0; i < C::PWH; ++i) {
      const int c = wave + i * C::NW, h = 2 * c + (lane >> 5);
      const int sc = pc ^ swz_p(h);
      const bool live = h < a.Hs && ((mk >> h) & 1ull);
      const bool plv = ((mk >> (2 * c)) & 3ull) != 0ull && 2 * c < a.Hs;
      hbase[i] = vals + (live ? (size_t)ui->vidx[h] * B * B : (size_t)0) + (size_t)(r ^ (h & 1)) * B + qoff + 8 * sc;
      bits |= plv ? 1u << i : 0u;
    }
    hlive = __builtin_amdgcn_readfirstlane(bits);
  };
  auto issue_h = [&](int hsi, char* slot) {
#pragma unroll
    for (int i = 0; i < C::PWH; ++i)
      if ((hlive >> i) & 1u)
        async_copy16(hbase[i] + (size_t)hsi * 4 * B, slot + (size_t)(wave + i * C::NW) * 1024);
    return __builtin_popcount(hlive);
  };
  // The group's receiver heads read nkv consecutive value heads kv0 ..
  // kv0 + nkv - 1 (grouped-query attention: ratio receivers per value head).
  // V rows of the VK-key part hh of the block (16 keys with the stage ring,
  // 32 with the half-stage ring), staged once per value head -> Vs, row
  // VK kvl + key
  const int ratio = R.Hr / R.Hkv;
  const int kv0 = (8 * grp) / ratio;
  const int nkv = min(8 * grp + 7, R.Hr - 1) / ratio - kv0 + 1;
  auto issue_v = [&](const UnionInfo* ui, int hh, int buf) {
    const int ln = opaque(lane);
    const int ninst = nkv * (C::VK / C::RPI);
    char* vdst = Vs + (size_t)buf * C::VBUF;
#pragma unroll 1
    for (int k = wave; k < ninst; k += C::NW) {
      const int rho = k * C::RPI + ln / C::VCPR;
      const int p = ln % C::VCPR;
      const int kvl = rho / C::VK, cl = rho % C::VK;
      const int kl = C::VK * hh + cl;                  // key inside the block
      const int key = ui->j * B + kl;
      const bool live = key < ri.klen;
      const int g = kv0 + kvl;
      const int lc = p ^ swz_v(rho, C::VCPR);
      size_t tok;
      if (paged) {
        int64_t page = live ? ui->page[kl] : 0;
        page = page < 0 ? 0 : (page >= R.num_pages ? R.num_pages - 1 : page);
        tok = live ? (size_t)page * R.page_size + key % R.page_size : 0;
      } else {
        tok = (size_t)ri.k0 + (live ? key : 0);
      }
      async_copy16(vbase + (tok * R.Hkv + g) * D + 8 * lc, vdst + (size_t)k * 1024);
    }
    return wave < ninst ? (ninst - 1 - wave) / C::NW + 1 : 0;
  };

  f32x4 O[4][C::NT];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt) O[i][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // per-lane transpose-read offsets inside a ring slot: key e of heads
  // h = 32 hk + 8 lg + (lr >> 2) and h + 4, queries q .. q + 3 (the key adds
  // e * PROW, an immediate)
  const int q = 16 * qt + 4 * (lr & 3);
  const int pch = q >> 3, pwithin = (q & 7) * 2;
  unsigned moff[2][2];
#pragma unroll
  for (int hk = 0; hk < 2; ++hk)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int h = 32 * hk + 8 * lg + (lr >> 2) + 4 * t;
      moff[hk][t] = (unsigned)(h * (C::HALF ? 4 * C::PROW : C::HSTR) + ((pch ^ swz_p(h)) << 4) + pwithin);
    }
  const float* wrow = Wsh + (4 * hq + (lr & 3)) * 64;
  const unsigned ppar = ((lr >> 2) & 1) * C::PROW;     // this lane's heads are odd: key pairs swapped

  if (UI[0].j != 0x7FFFFFFF) {
    // stages are numbered over the whole walk: stage s is stage s % SPU of
    // union block s / SPU (half-stage t is half-stage t % HPU of block
    // t / HPU).  Copies outstanding at the top of a stage:
    //  - half-stage ring: the prologue issues half-stages 0..2 and stage s
    //    issues 2s+3 and 2s+4, so only 2s+2, the previous stage's last
    //    copies, may still be in flight; the V rows of a step (and the
    //    merge's copies), issued before the P copies of its first stage, have
    //    landed by its second;
    //  - stage ring, two V buffers: every copy is needed two stages after
    //    the one that issued it at the earliest, so all of the previous
    //    stage's copies may still be in flight;
    //  - stage ring, one V buffer: the V rows issued at a half's first stage
    //    (and the merge's copies, issued before them) are needed at its
    //    second, so only the previous stage's P copies, always its last, may
    //    be;
    //  - 2-slot stage ring: everything is waited for.
    int ops_prev = 0, p_prev = 0;
    if constexpr (C::HALF) {
      prep_h(&UI[0]);
#pragma unroll
      for (int t = 0; t < 3; ++t) p_prev = issue_h(t, ring + (size_t)t * C::HSB);
    } else {
      prep_p(&UI[0]);
      if (C::NVB == 2) issue_v(&UI[0], 0, 0);
#pragma unroll
      for (int t = 0; t < C::AHEAD; ++t) p_prev = issue_p(t, ring + (size_t)t * C::SBYTES);
    }
    ops_prev = p_prev;
    bf16x8 Wk[2];
    f32x4 Cacc[8];
#pragma unroll
    for (int ee = 0; ee < 8; ++ee) Cacc[ee] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0;; ++s) {
      // P rows of stage s and the V rows of its half have landed (only the
      // P copies issued at stage s - 1, the wave's latest, may still be in
      // flight)
      if (C::HALF) {
        // half-stages 2s and 2s+1 have landed; only 2s+2, issued last at
        // stage s-1, may be in flight
        wait_vmcnt_upto<C::PWH>(p_prev);
      } else if (C::AHEAD == 1) {
        wait_vmcnt<0>();
      } else if (C::NVB == 1) {
        wait_vmcnt_upto<C::PW>(p_prev);
      } else {
        wait_vmcnt_upto<15>(ops_prev);
      }
      __syncthreads();
      const int u = s / C::SPU, si = s % C::SPU;
      const UnionInfo* ui = &UI[u & 1];
      if (si == 0 && ui->j == 0x7FFFFFFF) break;
      const int g2 = si & 3;
      int ops = 0;
      if (si == 0) {
        if (wave == 0) ops += merge(&UI[(u + 1) & 1]);
        // W of this union block: sender heads that do not keep j get weight 0
        const unsigned long long mk = ui->mask;
#pragma unroll
        for (int hk = 0; hk < 2; ++hk)
#pragma unroll
          for (int ee = 0; ee < 8; ++ee) {
            const int h = 32 * hk + 8 * lg + ee;
            Wk[hk][ee] = (bf16)(((mk >> h) & 1ull) ? wrow[h] : 0.f);
          }
      }
      // V rows: with two buffers, those of the next half at the last stage of
      // this one (into the other buffer); with one, those of this half at
      // its first stage
      if (C::HALF) {
        // V rows of this 32-key step, needed at its last stage
        if (g2 == 0) ops += issue_v(ui, si >> 2, 0);
      } else if (C::NVB == 2) {
        if (g2 & 1) {
          const int s1 = s + 1;
          const UnionInfo* ui1 = &UI[(s1 / C::SPU) & 1];
          if (ui1->j != 0x7FFFFFFF) {
            ops += issue_v(ui1, (s1 % C::SPU) >> 1, (s1 >> 1) & 1);
          }
        }
      } else if ((g2 & 1) == 0) {
        ops += issue_v(ui, si >> 1, 0);
      }
      // ---- P copies of stage s + AHEAD (dummy rows past the last block)
      if constexpr (C::HALF) {
        // half-stages 2s+3 and 2s+4, into the slots stage s-1 consumed
#pragma unroll
        for (int k = 3; k <= 4; ++k) {
          const int t = 2 * s + k, u2 = t / C::HPU, hsi = t % C::HPU;
          if (hsi == 0) {
            const UnionInfo* ui2 = &UI[u2 & 1];
            prep_h(ui2->j != 0x7FFFFFFF ? ui2 : nullptr);
          }
          p_prev = issue_h(hsi, ring + (size_t)(t % C::NHS) * C::HSB);
          ops += p_prev;
        }
      } else {
        const int s2 = s + C::AHEAD, u2 = s2 / C::SPU, si2 = s2 % C::SPU;
        if (si2 == 0) {
          const UnionInfo* ui2 = &UI[u2 & 1];
          prep_p(ui2->j != 0x7FFFFFFF ? ui2 : nullptr);
        }
        p_prev = issue_p(si2, ring + (size_t)(s2 % C::NSLOT) * C::SBYTES);
        ops += p_prev;
      }
      ops_prev = ops;

      // ---- head mix over the 8 keys of key group g2: lanes of key group g2
      // take W, the others zero (block-diagonal)
      const char* cur = ring + (size_t)(s % C::NSLOT) * C::SBYTES;
      const char* curA = ring + (size_t)((2 * s) % C::NHS) * C::HSB;
      const char* curB = ring + (size_t)((2 * s + 1) % C::NHS) * C::HSB;
      const bf16x8 zero8 = {};
#pragma unroll
      for (int hk = 0; hk < 2; ++hk) {
        if (32 * hk < hpad) {
          const bf16x8 wop = ((lr >> 2) == g2) ? Wk[hk] : zero8;
          const bool hv = 32 * hk + 8 * lg < hpad;
          // A transposing read gives each lane data from rows other lanes
          // address, so it never runs under a partial exec mask: every lane
          // reads (lanes past the padded heads at head 0's rows) and the
          // lanes past the heads take zeros afterwards.
          const unsigned o0 = hv ? moff[hk][0] : moff[0][0];
          const unsigned o1 = hv ? moff[hk][1] : moff[0][1];
          // all eight operands first, then the MFMAs
          bf16x8 pop[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            bf16x4 lo, hi;
            if constexpr (C::HALF) {
              const char* hs = e < 4 ? curA : curB;
              const int ep = e & 3;
              const unsigned kofs = (ep & 1) ? (ep - 1) * C::PROW + (C::PROW - ppar) : ep * C::PROW + ppar;
              lo = tr_read(hs, o0 + kofs);
              hi = tr_read(hs, o1 + kofs);
            } else {
              lo = tr_read(cur, o0 + e * C::PROW);
              hi = tr_read(cur, o1 + e * C::PROW);
            }
            const bf16x8 pv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            pop[e] = hv ? pv : zero8;
          }
#pragma unroll
          for (int e = 0; e < 8; ++e)
            Cacc[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wop, pop[e], Cacc[e], 0, 0, 0);
        }
      }
      if (C::HALF ? g2 == 3 : (g2 & 1) != 0) {
        // ---- P.V over the 16 keys of this half: A_r[q][32cb + 8lg + e] =
        // Cacc[e][i]; lane groups of the other half hold zeros, and their V
        // rows (any finite row of the buffer) add nothing
        bf16x8 Aop[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int ee = 0; ee < 8; ++ee) Aop[i][ee] = (bf16)Cacc[ee][i];
        const int nlo = 4 * (lr & 3);
        const char* Vh = Vs + (size_t)(!C::HALF && C::NVB == 2 ? (s >> 1) & 1 : 0) * C::VBUF;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // value head of receiver 8 grp + 4 hq + i, local to the group (a
          // padding receiver past Hr reads some staged row: its mixed map is 0)
          const int kvl = min((8 * grp + 4 * hq + i) / ratio - kv0, KVC - 1);
          const int rho0 = kvl * C::VK + 8 * (C::HALF ? lg : (lg & 1)) + (lr >> 2);
          const int sw0 = swz_v(rho0, C::VCPR);         // same for rho0 + 4
#pragma unroll
          for (int nt = 0; nt < C::NT; ++nt) {
            const int n = 16 * nt + nlo;
            const int lc = n >> 3, within = (n & 7) * 2;
            const unsigned off = (unsigned)(rho0 * C::VROW + ((lc ^ sw0) << 4) + within);
            const bf16x4 lo = tr_read(Vh, off);
            const bf16x4 hi = tr_read(Vh, off + 4 * C::VROW);
            const bf16x8 vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            O[i][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(Aop[i], vop, O[i][nt], 0, 0, 0);
          }
        }
#pragma unroll
        for (int ee = 0; ee < 8; ++ee) Cacc[ee] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  }

  // ---- output: stage [q][8 heads][d] in LDS, then 16-byte stores of whole rows
  wait_vmcnt<0>();
  __syncthreads();
  bf16* stage = reinterpret_cast<bf16*>(smem);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int nt = 0; nt < C::NT; ++nt)
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int qq = 16 * qt + 4 * lg + ii;
        stage[((size_t)qq * 8 + 4 * hq + i) * D + 16 * nt + lr] = (bf16)O[i][nt][ii];
      }
  __syncthreads();
  bf16* __restrict__ obase = reinterpret_cast<bf16*>(R.o) + (size_t)l * R.lso;
  const int heads_here = min(8, R.Hr - 8 * grp);
  constexpr int CPQ = 8 * D * 2 / 16;                  // 16-byte chunks per query row
  for (int c = tid; c < C::RQ * CPQ; c += C::NW * 64) {
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

template <int B, int D, int HP8, int KVC>
int launch_fast_h(const MappedArgs& a, void* stream) {
  using C = MapCfg<B, D, HP8, KVC>;
  const size_t lds = mapped_mfma_lds_bytes(B, D, a.Hs, KVC);
  auto kern = mapped_mfma_kernel<B, D, HP8, KVC>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return (int)e;
  int ngroups = 0;
  for (int k = 0; k < a.nrecv; ++k) ngroups += (a.rx[k].Hr + 7) / 8;
  const long long nu = (long long)a.b.total_rb * C::QH * a.L;
  const long long per_xcd = (nu + kXcds - 1) / kXcds * ngroups;
  hipLaunchKernelGGL(kern, dim3((unsigned)(per_xcd * kXcds)), dim3(C::NW * 64), lds, (hipStream_t)stream, a, ngroups);
  return (int)hipGetLastError();
}

template <int B, int D, int KVC>
int launch_fast_k(const MappedArgs& a, void* stream) {
  switch ((a.Hs + 7) / 8) {
    case 1: return launch_fast_h<B, D, 1, KVC>(a, stream);
    case 2: return launch_fast_h<B, D, 2, KVC>(a, stream);
    case 3: return launch_fast_h<B, D, 3, KVC>(a, stream);
    case 4: return launch_fast_h<B, D, 4, KVC>(a, stream);
    case 5: return launch_fast_h<B, D, 5, KVC>(a, stream);
    case 6: return launch_fast_h<B, D, 6, KVC>(a, stream);
    case 7: return launch_fast_h<B, D, 7, KVC>(a, stream);
    case 8: return launch_fast_h<B, D, 8, KVC>(a, stream);
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
int launch_fast(const MappedArgs& a, void* stream) {
  return max_group_value_heads(a) <= 4 ? launch_fast_k<B, D, 4>(a, stream) : launch_fast_k<B, D, 8>(a, stream);
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

bool mapped_mfma_covers(int B, int d, int Hs, int kv_heads_per_group, size_t lds_limit) {
  return mapped_mfma_lds_bytes(B, d, Hs, kv_heads_per_group <= 4 ? 4 : 8) <= lds_limit;
}

int launch_mapped(const MappedArgs& a, mf_dtype dt, void* stream, bool allow_fast, size_t lds_limit) {
  if (a.b.total_rb == 0 || a.L == 0) return 0;
  if (dt == MF_BF16 && allow_fast && mapped_mfma_covers(a.B, a.d, a.Hs, max_group_value_heads(a), lds_limit)) {
    switch (a.B * 1000 + a.d) {
      case 64064: return launch_fast<64, 64>(a, stream);
      case 64128: return launch_fast<64, 128>(a, stream);
      case 128064: return launch_fast<128, 64>(a, stream);
      case 128128: return launch_fast<128, 128>(a, stream);
    }
  }
  return dt == MF_BF16 ? launch_gd<bf16>(a, stream) : launch_gd<float>(a, stream);
}

int launch_mapped_multi(const MappedArgs& a, mf_dtype dt, void* stream, bool allow_fast, size_t lds_limit) {
  if (a.b.total_rb == 0 || a.L == 0) return 0;
  if (dt == MF_BF16 && allow_fast && mapped_mfma_covers(a.B, a.d, a.Hs, max_group_value_heads(a), lds_limit) &&
      (a.B == 64 || a.B == 128) && (a.d == 64 || a.d == 128))
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
