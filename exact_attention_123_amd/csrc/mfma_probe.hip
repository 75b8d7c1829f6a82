// Matrix-core throughput probe for AMD Instinct MI355X (gfx950), behind the
// C ABI of include/attn_probe.h: the rate the chip sustains on bf16 MFMA
// alone (no memory traffic, no other instructions), the measured ceiling
// that the attention kernels' throughput is compared with next to the
// published dense peak.
//
// Each wave runs independent accumulation chains of one MFMA shape on
// register operands whose bits come from a hash of the thread index (random
// signs and mantissas, exponents near 1, so the products stay finite and the
// operand bits toggle like real data), rotating through four A and four B
// operands so that consecutive MFMAs read different registers.  Four waves
// per workgroup, one per SIMD; the caller sizes the grid (several
// workgroups per CU keep every SIMD's matrix core fed).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "attn_probe.h"
#include "tiles.h"

namespace {

using namespace attn_tiles;

__device__ __forceinline__ unsigned mix(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352dU;
  x ^= x >> 15;
  x *= 0x846ca68bU;
  x ^= x >> 16;
  return x;
}

// Eight bf16 values: random sign and 7-bit mantissa, exponent 126..128.
__device__ __forceinline__ bf16x8_t operand(unsigned seed) {
  u32x4_t u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const unsigned x = mix(seed * 4 + i);
    const unsigned lo = (x & 0x807fU) | ((126U + (x >> 8) % 3U) << 7);
    const unsigned hi = ((x >> 16) & 0x807fU) | ((126U + (x >> 24) % 3U) << 7);
    u[i] = lo | (hi << 16);
  }
  return __builtin_bit_cast(bf16x8_t, u);
}

typedef float f32x4v_t __attribute__((ext_vector_type(4)));

template <int SHAPE>
__global__ __launch_bounds__(256) void attn_probe_mfma_kernel(float* __restrict__ sink,
                                                              int iters) {
  const unsigned gid = blockIdx.x * blockDim.x + threadIdx.x;
  bf16x8_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = operand(gid * 8 + i);
    b[i] = operand(gid * 8 + 4 + i);
  }
  float total = 0.0f;
  if constexpr (SHAPE == 0) {  // v_mfma_f32_32x32x16_bf16: 16 per trip
    f32x16_t c[4] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int x = 0; x < 4; ++x)
          c[x] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(i + x) & 3], b[(i + 2 * x) & 3],
                                                         c[x], 0, 0, 0);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int r = 0; r < 16; ++r) total += c[x][r];
  } else {  // v_mfma_f32_16x16x32_bf16: 32 per trip
    f32x4v_t c[8] = {};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int x = 0; x < 8; ++x)
          c[x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[(i + x) & 3], b[(i + 3 * x) & 3],
                                                         c[x], 0, 0, 0);
    }
#pragma unroll
    for (int x = 0; x < 8; ++x)
#pragma unroll
      for (int r = 0; r < 4; ++r) total += c[x][r];
  }
  sink[gid] = total;  // keeps the chains live
}

}  // namespace

extern "C" {

double attn_probe_mfma_flops(int shape, int64_t workgroups, int64_t iters) {
  if ((shape != 0 && shape != 1) || workgroups < 1 || iters < 1) return 0.0;
  // per wave and trip: 16 MFMAs of 32x32x16 or 32 of 16x16x32, 2 m n k each
  const double per_trip = shape == 0 ? 16.0 * 2 * 32 * 32 * 16 : 32.0 * 2 * 16 * 16 * 32;
  return per_trip * (double)iters * (double)workgroups * 4.0;
}

attn_status attn_probe_mfma(int shape, int64_t workgroups, int64_t iters, float* sink,
                            hipStream_t stream) {
  if (shape != 0 && shape != 1) return ATTN_ERR_ARG;
  if (workgroups < 1 || workgroups > (int64_t(1) << 20) || iters < 1 || iters > INT32_MAX)
    return ATTN_ERR_SHAPE;
  if (!sink) return ATTN_ERR_NULL;
  if ((uintptr_t)sink & 3u) return ATTN_ERR_ALIGN;
  int it = (int)iters;
  void* args[] = {(void*)&sink, (void*)&it};
  const void* k = shape == 0 ? (const void*)attn_probe_mfma_kernel<0>
                             : (const void*)attn_probe_mfma_kernel<1>;
  if (hipLaunchKernel(k, dim3((unsigned)workgroups), dim3(256), args, 0, stream) != hipSuccess)
    return ATTN_ERR_LAUNCH;
  return ATTN_OK;
}

}  // extern "C"
