// Materialised attention: the unfused three-kernel forward that writes the
// T x T score and probability matrices to device memory and reads them back,
// for AMD Instinct MI355X (gfx950), behind the C ABI of include/attn.h.
//
// This is the naive pattern the pages contrast with the fused kernel ("Why
// Attention Is Difficult to Optimize", Figure 2; "FlashAttention -- avoid
// writing the giant intermediate", the materialized path of its flowchart):
//   1. scores : S = scale Q K^T with the causal mask, written to memory
//   2. softmax: each row of S read back, P = rowsoftmax(S) written, with LSE
//   3. output : P read back, O = P V
// It exists to measure, with the same inputs and hardware, the time and the
// device-memory traffic the fused forward avoids.  S is stored in fp32: at
// the score spread of the benchmark workload (|S| up to ~60) a bf16 score
// would carry an absolute error of up to 0.125 into the exponent.  P is
// stored in bf16, the precision the fused kernel's P V contraction uses.
//
// Under the causal mask only the visible part is touched: kernel 1 writes
// the 64-key tiles at or below the diagonal of each 128-query block, kernel 2
// reads each row's visible prefix and writes P up to the end of its 128-query
// block (zeros after the diagonal), kernel 3 reads those tiles.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "attn.h"
#include "device.h"
#include "tiles.h"

namespace {

using namespace attn_tiles;
using attn_internal::check_device;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;  // query rows per workgroup (kernels 1, 3)
constexpr int kTile = 64;           // keys per staged K or V tile

// Keys a row of query block qb may touch: up to the end of the block under
// the causal mask, all of them otherwise.
__device__ __forceinline__ int block_keys(int T, int qb, bool causal) {
  return causal ? min(T, (qb + 1) * kRows) : T;
}

// ---------------------------------------------------------------------------
// 1. scores: S[q][k] = scale * (Q K^T)[q][k], -inf where k > q (causal), fp32.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_mat_scores_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, float* __restrict__ S, int T,
    int nqb, float scale) {
  using C = RowTile<D>;
  constexpr int NDS = C::NDS, RB = C::RB;
  __shared__ __attribute__((aligned(1024))) char sK0[kTile * RB];
  __shared__ __attribute__((aligned(1024))) char sK1[kTile * RB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, h = lane >> 5;
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const size_t head = (size_t)bh * T * D;
  const int qg = qb * kRows + 32 * wave + j;

  bf16x8_t qf[NDS];
  {
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Q + head, T * RB);
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8_t, buf_load16(rQ, qg * RB + (16 * s + 8 * h) * 2));
  }
  TileAddr<D> ad;
  ad.init(lane);
  TileDma<D, kTile, kWaves> dma;
  dma.init(wave, lane);
  const int nkt = block_keys(T, qb, CAUSAL) / kTile;
  float* srow = S + ((size_t)bh * T + qg) * T;

  auto tile = [&](const char* kt, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      f32x16_t sc = f32x16_t{};
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row(kt, 32 * u * RB + ad.row[s]),
                                                     qf[s], sc, 0, 0, 0);
      // register 8 a + e: key t * 64 + 32 u + 16 a + 8 h + e of query qg
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int key0 = t * kTile + 32 * u + 16 * a + 8 * h;
        f32x4_t lo, hi;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          lo[e] = (CAUSAL && key0 + e > qg) ? -INFINITY : sc[8 * a + e] * scale;
          hi[e] = (CAUSAL && key0 + 4 + e > qg) ? -INFINITY : sc[8 * a + 4 + e] * scale;
        }
        *reinterpret_cast<f32x4_t*>(srow + key0) = lo;
        *reinterpret_cast<f32x4_t*>(srow + key0 + 4) = hi;
      }
    }
  };

  dma.load(sK0, K + head, T, 0, wave);
  __syncthreads();
  for (int t = 0; t < nkt; t += 2) {
    if (t + 1 < nkt) dma.load(sK1, K + head, T, (t + 1) * kTile, wave);
    tile(sK0, t);
    __syncthreads();
    if (t + 1 >= nkt) break;
    if (t + 2 < nkt) dma.load(sK0, K + head, T, (t + 2) * kTile, wave);
    tile(sK1, t + 1);
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// 2. softmax: one wave per row.  Reads S[q][0 .. n) (n = q + 1 causal, T
// otherwise) three times (max, sum, write), writes P[q][0 .. lim) in bf16
// (lim = end of the row's 128-query block under the mask, zeros past n) and
// LSE = max + ln(sum).
// ---------------------------------------------------------------------------
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_mat_softmax_kernel(
    const float* __restrict__ S, __bf16* __restrict__ P, float* __restrict__ LSE, int T,
    int64_t rows) {
  const int64_t row = (int64_t)blockIdx.x * kWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const int q = (int)(row % T);
  const int n = CAUSAL ? q + 1 : T;
  const int lim = CAUSAL ? min(T, (q / kRows + 1) * kRows) : T;
  const float* s = S + row * T;
  __bf16* p = P + row * T;
  // lane handles 4 consecutive entries per 256-entry stride
  float m = -INFINITY;
  for (int i = 4 * lane; i < n; i += 256) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(s + i);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i + e < n) m = fmaxf(m, v[e]);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  float l = 0.0f;
  for (int i = 4 * lane; i < n; i += 256) {
    const f32x4_t v = *reinterpret_cast<const f32x4_t*>(s + i);
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (i + e < n) l += exp2_hw((v[e] - m) * kLog2e);
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
  const float inv = 1.0f / l;
  for (int i = 4 * lane; i < lim; i += 256) {
    f32x4_t v = f32x4_t{};
    if (i < n) v = *reinterpret_cast<const f32x4_t*>(s + i);
    __bf16 w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(i + e < n ? exp2_hw((v[e] - m) * kLog2e) * inv
                                                          : 0.0f);
    u32x2_t bits;
    std::memcpy(&bits, w, 8);
    *reinterpret_cast<u32x2_t*>(p + i) = bits;
  }
  if (lane == 0) LSE[row] = m + log2_hw(l) * kLn2;
}

// ---------------------------------------------------------------------------
// 3. output: O = P V; per wave 32 query rows, O^T += V^T P^T with V tiles
// in LDS (transposing reads) and P^T read from memory as the B operand,
// divided by the row sum of the bf16 P it used.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_mat_pv_kernel(
    const __bf16* __restrict__ P, const __bf16* __restrict__ V, __bf16* __restrict__ O, int T,
    int nqb) {
  using C = RowTile<D>;
  constexpr int NDT = C::NDT, RB = C::RB;
  __shared__ __attribute__((aligned(1024))) char sV0[kTile * RB];
  __shared__ __attribute__((aligned(1024))) char sV1[kTile * RB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, h = lane >> 5;
  const int bh = blockIdx.x / nqb, qb = blockIdx.x % nqb;
  const size_t head = (size_t)bh * T * D;
  const int qg = qb * kRows + 32 * wave + j;
  const __bf16* prow = P + ((size_t)bh * T + qg) * T;
  TileAddr<D> ad;
  ad.init(lane);
  TileDma<D, kTile, kWaves> dma;
  dma.init(wave, lane);
  const int nkt = block_keys(T, qb, CAUSAL) / kTile;

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
  // Sum of the bf16 probabilities the contraction uses (lane-partial): O is
  // divided by it, so that O stays a convex combination of V rows although
  // the stored row of P sums to 1 only up to its bf16 rounding.
  float wsum = 0.0f;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  auto tile = [&](const char* vt, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int r0 = 32 * u + 16 * a;
        const bf16x8_t pb =
            *reinterpret_cast<const bf16x8_t*>(prow + t * kTile + r0 + 8 * h);
        wsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), one2, wsum,
                                               false);
        wsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), one2, wsum,
                                               false);
        wsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), one2, wsum,
                                               false);
        wsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), one2, wsum,
                                               false);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_tr(vt, r0 * RB + ad.tr[0][dt], r0 * RB + ad.tr[1][dt]), pb, oacc[dt], 0, 0,
              0);
      }
  };

  dma.load(sV0, V + head, T, 0, wave);
  __syncthreads();
  for (int t = 0; t < nkt; t += 2) {
    if (t + 1 < nkt) dma.load(sV1, V + head, T, (t + 1) * kTile, wave);
    tile(sV0, t);
    __syncthreads();
    if (t + 1 >= nkt) break;
    if (t + 2 < nkt) dma.load(sV0, V + head, T, (t + 2) * kTile, wave);
    tile(sV1, t + 1);
    __syncthreads();
  }
  wsum += __shfl_xor(wsum, 32);
  store_rows<D>(O + head, oacc, 1.0f / wsum, qg, T, h);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

template <int D>
const void* scores_kernel(int causal) {
  return causal ? (const void*)attn_mat_scores_kernel<D, true>
                : (const void*)attn_mat_scores_kernel<D, false>;
}
template <int D>
const void* pv_kernel(int causal) {
  return causal ? (const void*)attn_mat_pv_kernel<D, true>
                : (const void*)attn_mat_pv_kernel<D, false>;
}

}  // namespace

extern "C" {

attn_status attn_fwd_materialized(const void* q, const void* k, const void* v, void* o,
                                  float* lse, float* s_buf, void* p_buf, int64_t B, int64_t H,
                                  int64_t T, int64_t d, int causal, float scale,
                                  hipStream_t stream) {
  if (B < 0 || H < 0 || T < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (B == 0 || H == 0 || T == 0) return ATTN_OK;
  if (T % kRows != 0) return ATTN_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !lse || !s_buf || !p_buf) return ATTN_ERR_NULL;
  if (T > 32768) return ATTN_ERR_SHAPE;  // a head's T x T fp32 scores stay under 4 GiB
  if (B > (int64_t(1) << 31) / H) return ATTN_ERR_SHAPE;
  const int64_t BH = B * H;
  if (BH > (INT32_MAX / (T / kRows)) || BH > (INT64_MAX / 8) / (T * T * 4))
    return ATTN_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)s_buf |
       (uintptr_t)p_buf) & 15u)
    return ATTN_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return ATTN_ERR_ALIGN;
  const int64_t nb = BH * T * d * 2, lb = BH * T * 4, sb = BH * T * T * 4, pb = BH * T * T * 2;
  const void* bufs[7] = {q, k, v, o, lse, s_buf, p_buf};
  const int64_t sz[7] = {nb, nb, nb, nb, lb, sb, pb};
  for (int a = 3; a < 7; ++a)  // outputs and scratch against everything else
    for (int b = 0; b < 7; ++b)
      if (a != b && overlaps(bufs[a], sz[a], bufs[b], sz[b])) return ATTN_ERR_ARG;
  attn_status st = check_device();
  if (st != ATTN_OK) return st;

  int t = (int)T, nqb = (int)(T / kRows);
  const dim3 grid((unsigned)(BH * nqb));
  {
    void* args[] = {(void*)&q, (void*)&k, (void*)&s_buf, (void*)&t, (void*)&nqb, (void*)&scale};
    const void* kern = d == 64 ? scores_kernel<64>(causal) : scores_kernel<128>(causal);
    if (hipLaunchKernel(kern, grid, dim3(kThreads), args, 0, stream) != hipSuccess)
      return ATTN_ERR_LAUNCH;
  }
  {
    int64_t rows = BH * T;
    const float* sc = s_buf;
    void* args[] = {(void*)&sc, (void*)&p_buf, (void*)&lse, (void*)&t, (void*)&rows};
    const void* kern = causal ? (const void*)attn_mat_softmax_kernel<true>
                              : (const void*)attn_mat_softmax_kernel<false>;
    if (hipLaunchKernel(kern, dim3((unsigned)((rows + kWaves - 1) / kWaves)), dim3(kThreads),
                        args, 0, stream) != hipSuccess)
      return ATTN_ERR_LAUNCH;
  }
  {
    const void* pc = p_buf;
    void* args[] = {(void*)&pc, (void*)&v, (void*)&o, (void*)&t, (void*)&nqb};
    const void* kern = d == 64 ? pv_kernel<64>(causal) : pv_kernel<128>(causal);
    if (hipLaunchKernel(kern, grid, dim3(kThreads), args, 0, stream) != hipSuccess)
      return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

}  // extern "C"
