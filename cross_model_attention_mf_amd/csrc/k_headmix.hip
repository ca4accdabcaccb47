// Offline calibration of the head mix W by least squares (MapFlow page,
// section "从内部表示,走向 token 之间的依赖关系": the head mapping is a learned
// linear combination of sender heads, fitted once offline with both models
// frozen).  For each receiver layer the fit solves the normal equations
//   (G + lambda I) w_r = b_r,  G[h][h'] = sum <Pt_h, Pt_h'>,  b_r[h] = sum <A_r, Pt_h>
// over the blocks (i, j) of the union of the sender heads' kept sets, with
// Pt_h the kept block of sender head h (0 where h does not keep j) and A_r
// the receiver head's own block (0 where it does not keep j).
//
// headmix_gram_kernel: one workgroup per (receiver layer, row-block).  Wave 0
// merges the sender heads' sorted column lists (lane h walks head h) and
// moves each receiver head's list (lane r) up to the union block; the kept
// blocks of every sender and receiver head are then staged through LDS, 64
// entries at a time (16-byte loads of the next 128 in flight while the current
// ones are multiplied; two LDS buffers, one barrier per step), transposed to
// [entry][head] in fp32.  The products are a dense contraction over the
// entries, [sender + receiver heads] x [sender heads], on fp64 MFMA
// (16 x 16 x 4; bf16 and fp32 values are exact in fp64, and so are their
// products), 16 x 16 output tiles dealt to the four waves.  Each workgroup
// writes its partial products, and headmix_reduce_kernel adds them over the
// row-blocks in order, so results do not depend on scheduling.
// headmix_solve_kernel: one workgroup per layer, Cholesky of G + lambda I in
// LDS with the drop rule (a pivot at most 1e-12 of its diagonal drops the
// head: weight 0), then forward and back substitution per receiver head.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "device_common.h"
#include "internal.h"

namespace mf {
namespace {

constexpr int kHmThreads = 256;
constexpr int kHmChunk = 64;   // block entries staged per step
constexpr int kNoCol = 0x7FFFFFFF;

constexpr int kHmItems = 4;   // staging items per thread: up to (64 + 64) heads x 8 parts / 256 threads

// eight consecutive block entries, as loaded (16 bytes of bf16, 32 of fp32)
template <typename T> struct Raw8;
template <> struct Raw8<__hip_bfloat16> { uint4 w; };
template <> struct Raw8<float> { uint4 w[2]; };

__device__ __forceinline__ Raw8<__hip_bfloat16> load8(const __hip_bfloat16* p) {
  return Raw8<__hip_bfloat16>{*reinterpret_cast<const uint4*>(p)};
}
__device__ __forceinline__ Raw8<float> load8(const float* p) {
  const uint4* q = reinterpret_cast<const uint4*>(p);
  return Raw8<float>{{q[0], q[1]}};
}
__device__ __forceinline__ void unpack8(const Raw8<__hip_bfloat16>& r, float* x) {
  const unsigned w[4] = {r.w.x, r.w.y, r.w.z, r.w.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void unpack8(const Raw8<float>& r, float* x) {
  const unsigned w[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w, r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = __uint_as_float(w[e]);
}

// A copy of a lane value the compiler cannot see through, so address math
// derived from it is redone in place each step instead of being hoisted out of
// the loop and held in registers.
__device__ __forceinline__ int opaque(int x) {
  int y;
  asm volatile("v_mov_b32 %0, %1" : "=v"(y) : "v"(x));
  return y;
}

typedef double f64x4 __attribute__((ext_vector_type(4)));

constexpr int kHmMaxTiles = 8;   // 16 x 16 output tiles per wave: (128 / 16) x (64 / 16) / 4 waves

// heads staged per entry (sender then receiver, padded to whole 16-row
// tiles) and the LDS pitch of one entry: the first count >= that which is 16
// mod 32, so the 4 entries one MFMA operand read touches (16 consecutive
// heads each) fall on 4 disjoint quarters of the 64 banks
__host__ __device__ inline int hm_rows(int Hs, int Hr) { return (Hs + Hr + 15) / 16 * 16; }
// staged heads per entry as a power of two (>= hm_rows), so the staging index
// splits into (head, part) with a mask and a shift
__host__ __device__ inline int hm_slots_log2(int Hs, int Hr) {
  int lg = 4;
  while ((1 << lg) < hm_rows(Hs, Hr)) ++lg;
  return lg;
}
__host__ __device__ inline int hm_pitch(int Hs, int Hr) { return (1 << hm_slots_log2(Hs, Hr)) + 16; }

template <typename T, int MT>
__global__ void __launch_bounds__(kHmThreads) headmix_gram_kernel(HeadmixArgs a) {
  extern __shared__ __align__(16) char smem[];
  const int NA = a.Hs + a.Hr;
  const int NAP = hm_rows(a.Hs, a.Hr);                 // heads in whole 16-row tiles
  const int SL = hm_slots_log2(a.Hs, a.Hr);            // staged heads per entry: 1 << SL
  const int P = hm_pitch(a.Hs, a.Hr);                  // floats per staged entry
  float* stage = reinterpret_cast<float*>(smem);      // 2 x [kHmChunk][P]
  __shared__ int j_sh;
  __shared__ unsigned long long smask_sh, rmask_sh;
  __shared__ int svidx[64], rvidx[64];

  const int R = a.b.total_rb;
  const int l = blockIdx.x / R, i = blockIdx.x % R;
  const int s = a.layer_map[l];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // output tiles: 16 x 16 blocks of [staged heads] x [sender heads]; wave w
  // takes tiles w, w + 4, ...
  const int CT = (a.Hs + 15) / 16, T16 = (NAP / 16) * CT;
  const int BB = a.B * a.B;
  const T* __restrict__ sval = reinterpret_cast<const T*>(a.s_val);
  const T* __restrict__ rval = reinterpret_cast<const T*>(a.r_val);

  f64x4 acc[MT];   // this wave's tiles (MT >= its tile count)
#pragma unroll
  for (int m = 0; m < MT; ++m) acc[m] = f64x4{0.0, 0.0, 0.0, 0.0};

  // merge state (wave 0): sender list of head `lane`, receiver list of head `lane`
  int sp = 0, se = 0, rp = 0, re = 0;   // CSR entries (int32 row_ptr)
  int scol = kNoCol, rcol = kNoCol;
  if (wave == 0) {
    if (lane < a.Hs) {
      const size_t row = ((size_t)s * a.Hs + lane) * R + i;
      sp = (int)min((long long)a.s_row_ptr[row], (long long)a.s_cap);
      se = (int)min((long long)a.s_row_ptr[row + 1], (long long)a.s_cap);
      if (sp < se) scol = a.s_col[sp];
    }
    if (lane < a.Hr) {
      const size_t row = ((size_t)l * a.Hr + lane) * R + i;
      rp = (int)min((long long)a.r_row_ptr[row], (long long)a.r_cap);
      re = (int)min((long long)a.r_row_ptr[row + 1], (long long)a.r_cap);
      if (rp < re) rcol = a.r_col[rp];
    }
  }

  for (;;) {
    if (wave == 0) {
      int jm = scol;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) jm = min(jm, __shfl_xor(jm, off, 64));
      if (jm != kNoCol) {
        // receiver heads skip their blocks outside the sender union
        while (rcol < jm) {
          ++rp;
          rcol = rp < re ? a.r_col[rp] : kNoCol;
        }
      }
      const bool take_s = scol == jm && jm != kNoCol;
      const bool take_r = rcol == jm && jm != kNoCol;
      const unsigned long long sm = __ballot(take_s), rm = __ballot(take_r);
      if (take_s) svidx[lane] = sp;
      if (take_r) rvidx[lane] = rp;
      if (lane == 0) {
        j_sh = jm;
        smask_sh = sm;
        rmask_sh = rm;
      }
      if (take_s) {
        ++sp;
        scol = sp < se ? a.s_col[sp] : kNoCol;
      }
      if (take_r) {
        ++rp;
        rcol = rp < re ? a.r_col[rp] : kNoCol;
      }
    }
    __syncthreads();
    if (j_sh == kNoCol) break;
    const unsigned long long sm = smask_sh, rm = rmask_sh;
    // this thread's staging items: (head slot, 8-entry part); the 16-byte
    // loads of chunk c + 1 are in flight while chunk c is multiplied
    const T* isrc[kHmItems];
#pragma unroll
    for (int t = 0; t < kHmItems; ++t) {
      const int idx = tid + t * kHmThreads;
      const int slot = idx & ((1 << SL) - 1), part = idx >> SL;   // consecutive lanes, consecutive heads
      const T* src = nullptr;
      if (part < kHmChunk / 8) {
        if (slot < a.Hs) {
          if ((sm >> slot) & 1ull) src = sval + (size_t)svidx[slot] * BB + 8 * part;
        } else if (slot < NA) {
          const int r = slot - a.Hs;
          if ((rm >> r) & 1ull) src = rval + (size_t)rvidx[r] * BB + 8 * part;
        }
      }
      isrc[t] = src;
    }
    // two chunks of loads in flight: chunk c + 2 is issued into the registers
    // chunk c was just staged from
    Raw8<T> preA[kHmItems], preB[kHmItems];
    auto load = [&](Raw8<T>* pre, int k0) {
#pragma unroll
      for (int t = 0; t < kHmItems; ++t) pre[t] = isrc[t] ? load8(isrc[t] + k0) : Raw8<T>{};
    };
    const int nch = BB / kHmChunk;   // even: B * B / 64 for B in {32, 64, 128}
    auto step = [&](Raw8<T>* pre, int c) {
      float* st = stage + (size_t)(c & 1) * kHmChunk * P;
#pragma unroll
      for (int t = 0; t < kHmItems; ++t) {
        const int idx = opaque(tid + t * kHmThreads);
        const int slot = idx & ((1 << SL) - 1), part = idx >> SL;
        if (part < kHmChunk / 8) {
          float x[8];
          unpack8(pre[t], x);
          float* q = st + 8 * part * P + slot;
#pragma unroll
          for (int e = 0; e < 8; ++e) q[e * P] = x[e];
        }
      }
      __syncthreads();
      if (c + 2 < nch) load(pre, (c + 2) * kHmChunk);
      // MFMA 16x16x4 fp64: lane L supplies A[L % 16][L / 16] (head 16 ra +
      // L % 16, entry 4 kk + L / 16) and B[L / 16][L % 16] (sender head
      // 16 cb + L % 16, same entry)
      const float* col = st + (lane >> 4) * P + (lane & 15);
#pragma unroll 2
      for (int kk = 0; kk < kHmChunk / 4; ++kk) {
        const float* rowk = col + 4 * kk * P;
#pragma unroll
        for (int m = 0; m < MT; ++m) {
          const int t = wave + 4 * m;
          if (t < T16) {
            const int ra = t / CT, cb = t % CT;
            const double av = (double)rowk[16 * ra];
            const double bv = (double)rowk[16 * cb];
            acc[m] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[m], 0, 0, 0);
          }
        }
      }
    };
    load(preA, 0);
    load(preB, kHmChunk);
    for (int c = 0; c < nch; c += 2) {
      step(preA, c);
      step(preB, c + 1);
    }
  }

  // this row-block's partial products: element j of lane L is row 4 j + L / 16,
  // column L % 16 of its tile (the fp64 MFMA's output layout)
  double* out = a.partial + (size_t)blockIdx.x * NA * a.Hs;
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int t = wave + 4 * m;
    if (t < T16) {
      const int ra = t / CT, cb = t % CT;
      const int cc = 16 * cb + (lane & 15);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 16 * ra + 4 * j + (lane >> 4);
        if (rr < NA && cc < a.Hs) out[(size_t)rr * a.Hs + cc] = acc[m][j];
      }
    }
  }
}

// gram[l] / cross[l] = sum over row-blocks i (in order) of the partials
__global__ void __launch_bounds__(kHmThreads) headmix_reduce_kernel(HeadmixArgs a, double* gram, double* cross) {
  const int NA = a.Hs + a.Hr;
  const int e = blockIdx.x * kHmThreads + threadIdx.x, l = blockIdx.y;
  if (e >= NA * a.Hs) return;
  const size_t per = (size_t)NA * a.Hs;
  const double* p = a.partial + (size_t)l * a.b.total_rb * per + e;
  double t = 0.0;
  for (int i = 0; i < a.b.total_rb; ++i) t += p[(size_t)i * per];
  const int row = e / a.Hs, c = e % a.Hs;
  if (row < a.Hs) gram[((size_t)l * a.Hs + row) * a.Hs + c] = t;
  else cross[((size_t)l * a.Hr + (row - a.Hs)) * a.Hs + c] = t;
}

constexpr double kDropTol = 1e-12;

__global__ void __launch_bounds__(64) headmix_solve_kernel(const double* __restrict__ gram,
                                                           const double* __restrict__ cross, double lam, int Hs,
                                                           int Hr, float* __restrict__ W, int32_t* __restrict__ dropped) {
  __shared__ double M[64][65];   // G + lam I, overwritten by its Cholesky factor (lower)
  __shared__ double Y[64][65];   // per receiver head: y, then w
  __shared__ double diag0[64];
  __shared__ int drop[64];
  const int l = blockIdx.x, t = threadIdx.x;
  for (int r = 0; r < Hs; ++r)
    if (t < Hs) M[r][t] = gram[((size_t)l * Hs + r) * Hs + t] + (r == t ? lam : 0.0);
  __syncthreads();
  if (t < Hs) diag0[t] = M[t][t];
  __syncthreads();
  for (int k = 0; k < Hs; ++k) {
    if (t == 0) {
      double piv = M[k][k];
      for (int p = 0; p < k; ++p) piv -= M[k][p] * M[k][p];
      const bool dk = !(diag0[k] > 0.0) || piv <= kDropTol * diag0[k];
      drop[k] = dk;
      M[k][k] = dk ? 0.0 : sqrt(piv);
    }
    __syncthreads();
    const int i = k + 1 + t;
    if (i < Hs) {
      if (drop[k]) {
        M[i][k] = 0.0;
      } else {
        double v = M[i][k];
        for (int p = 0; p < k; ++p) v -= M[i][p] * M[k][p];
        M[i][k] = v / M[k][k];
      }
    }
    __syncthreads();
  }
  if (t < Hr) {
    const double* b = cross + ((size_t)l * Hr + t) * Hs;
    for (int k = 0; k < Hs; ++k) {
      double v = 0.0;
      if (!drop[k]) {
        v = b[k];
        for (int p = 0; p < k; ++p) v -= M[k][p] * Y[t][p];
        v /= M[k][k];
      }
      Y[t][k] = v;
    }
    for (int k = Hs - 1; k >= 0; --k) {
      double v = 0.0;
      if (!drop[k]) {
        v = Y[t][k];
        for (int p = k + 1; p < Hs; ++p) v -= M[p][k] * Y[t][p];
        v /= M[k][k];
      }
      Y[t][k] = v;   // entries above k already hold w
    }
    for (int k = 0; k < Hs; ++k) W[((size_t)l * Hr + t) * Hs + k] = (float)Y[t][k];
  }
  if (dropped && t < Hs) dropped[(size_t)l * Hs + t] = drop[t];
}

}  // namespace

size_t headmix_partial_bytes(int L, int total_rb, int Hs, int Hr) {
  return (size_t)L * total_rb * (size_t)(Hs + Hr) * Hs * sizeof(double);
}

size_t headmix_gram_lds_bytes(int Hs, int Hr) {
  return (size_t)2 * kHmChunk * hm_pitch(Hs, Hr) * sizeof(float);
}

int launch_headmix_gram(const HeadmixArgs& a, mf_dtype dt, double* gram, double* cross, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int NA = a.Hs + a.Hr;
  if (a.L == 0) return 0;
  if (a.b.total_rb > 0) {
    const size_t lds = headmix_gram_lds_bytes(a.Hs, a.Hr);
    const int tiles = (hm_rows(a.Hs, a.Hr) / 16) * ((a.Hs + 15) / 16);
    const int per_wave = (tiles + 3) / 4;
    const bool bf = dt == MF_BF16;
    auto kern = per_wave <= 1 ? (bf ? headmix_gram_kernel<__hip_bfloat16, 1> : headmix_gram_kernel<float, 1>)
              : per_wave <= 2 ? (bf ? headmix_gram_kernel<__hip_bfloat16, 2> : headmix_gram_kernel<float, 2>)
              : per_wave <= 4 ? (bf ? headmix_gram_kernel<__hip_bfloat16, 4> : headmix_gram_kernel<float, 4>)
                              : (bf ? headmix_gram_kernel<__hip_bfloat16, kHmMaxTiles>
                                    : headmix_gram_kernel<float, kHmMaxTiles>);
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return (int)e;
    hipLaunchKernelGGL(kern, dim3((unsigned)(a.L * a.b.total_rb)), dim3(kHmThreads), lds, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return (int)e;
  }
  hipLaunchKernelGGL(headmix_reduce_kernel, dim3((unsigned)((NA * a.Hs + kHmThreads - 1) / kHmThreads), (unsigned)a.L),
                     dim3(kHmThreads), 0, s, a, gram, cross);
  return (int)hipGetLastError();
}

int launch_headmix_solve(const double* gram, const double* cross, double lam, int L, int Hs, int Hr, float* W,
                         int32_t* dropped, void* stream) {
  if (L == 0) return 0;
  hipLaunchKernelGGL(headmix_solve_kernel, dim3((unsigned)L), dim3(64), 0, (hipStream_t)stream, gram, cross, lam, Hs,
                     Hr, W, dropped);
  return (int)hipGetLastError();
}

}  // namespace mf
