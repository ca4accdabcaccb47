// Matrix-pipe probe: the bf16 MFMA rate this GPU sustains, alone and with
// the vector work of the block statistics beside it (per MFMA 32x32x16, two
// exp2 sums of three vector instructions each, as a 64 x 64 block of scores
// costs 32 MFMAs and 64 fma + exp2 + add per lane).  The nominal figure the
// rooflines divide by is the vendor's dense bf16 peak; this measures what the
// pipe delivers under the GPU's power and clock limits.
#include "device_common.h"
#include "internal.h"

namespace mf {

namespace {

template <bool VEC>
__global__ void __launch_bounds__(256) mfma_probe_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (bf16)(1e-3f * (float)(lane + i));
    b[i] = (bf16)(1e-3f * (float)(63 - lane + i));
  }
  // four independent accumulators: each chain's next MFMA issues four later,
  // past the result latency of the one before
  f32x16 c0 = f32x16{}, c1 = f32x16{}, c2 = f32x16{}, c3 = f32x16{};
  float x0 = -1e-3f * (float)lane, x1 = -0.5f - 1e-3f * (float)lane, s0 = 0.f, s1 = 0.f;
  const float dx = 1e-7f;
  for (int it = 0; it < iters; ++it) {
#define MF_PROBE_STEP(C)                                            \
    C = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, C, 0, 0, 0); \
    if constexpr (VEC) {                                            \
      x0 += dx; x1 += dx;                                           \
      s0 += __builtin_amdgcn_exp2f(x0);                             \
      s1 += __builtin_amdgcn_exp2f(x1);                             \
    }
    MF_PROBE_STEP(c0)
    MF_PROBE_STEP(c1)
    MF_PROBE_STEP(c2)
    MF_PROBE_STEP(c3)
#undef MF_PROBE_STEP
  }
  float r = s0 + s1;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = r;
}

}  // namespace

int launch_mfma_probe(float* out, int nblocks, int iters, bool with_vector, void* stream) {
  if (with_vector)
    hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3(nblocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3(nblocks), dim3(256), 0, (hipStream_t)stream, out, iters);
  return (int)hipGetLastError();
}

}  // namespace mf
