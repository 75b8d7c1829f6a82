// Decode: attention of a few new queries over a long key/value cache, for
// AMD Instinct MI355X (gfx950), behind the C ABI of include/attn.h.
//
// What is computed: for each (batch, query head) the Tq new queries sit at
// positions Tk - Tq .. Tk - 1 of a cached sequence of Tk keys and values;
// query i sees key j iff j <= Tk - Tq + i under the causal mask (all keys
// without it); O = softmax(scale Q K^T) V and LSE per query row, exactly as
// the forward.  "FlashAttention -- avoid writing the giant intermediate"
// separates this short-input decode from long-input prefill and stresses the
// key/value state kept across steps.
//
// Why a separate path.  With one or a few queries per head the work is
// reading the cache once: 4 Tk d bytes per key/value head against 4 Tq G Tk d
// FLOPs, about one FLOP per byte, far below the MFMA ridge.  The forward's
// one-workgroup-per-256-queries grid would give B*H workgroups, each reading
// its whole cache alone.  Here:
//   - the G query heads that share a key/value head (grouped-query
//     attention) are processed together, so the cache is read once per
//     group: the Tq G query rows form one MFMA column block (up to 32
//     rows; more rows take one workgroup per 32-row chunk, which read the
//     same keys from L2);
//   - the keys are split across workgroups (split-KV) so that the grid
//     fills all 256 CUs, and inside a workgroup each wave streams its own
//     32-key blocks, no workgroup barrier in the loop: K straight into
//     registers (it is the A operand of the score MFMA as loaded), V
//     direct-to-LDS (its transposing read needs LDS), both one block ahead.
//     With only V in LDS (16 KiB per wave) two workgroups fit on a CU, so
//     eight waves keep loads in flight;
//   - partial results (running max, normalisers, output accumulator) of the
//     4 waves merge in LDS with the rescaling of the online softmax; partial
//     results of the splits merge in a second small kernel:
//     LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
//     ("Attention Mechanism: Computation & Memory Patterns", section 3: the
//     running max and sum let partial results over key blocks be rescaled
//     and combined; the same algebra at workgroup and grid level.)

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "attn.h"
#include "device.h"
#include "fwd_cache.h"
#include "rows.h"
#include "tiles.h"

namespace {

using namespace attn_tiles;
using attn_internal::check_device;
using attn_rows::kBlk;
using attn_rows::kMaxRows;
using attn_rows::kThreads;
using attn_rows::kWaves;

// Key split: about kTargetGroups workgroups (one round at two per CU), each
// split at least kMinSplitKeys long: short splits cost a prologue, an LDS
// merge and partial results each (measured on MI355X, us per call of one
// 131072-key sequence with 32 query / 8 key-value heads: 32 splits of 4096
// keys 97.9, 64 of 2048 100.1, 128 of 1024 109.0; a target of 256 instead
// of 512 costs 3% on 16 sequences of 32768 keys).
constexpr int kMinSplitKeys = 4096;
constexpr int kTargetGroups = 512;

// One workgroup per (row chunk, key/value head, key split); see
// attn_rows::row_chunk_attention.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_decode_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, float* __restrict__ part_o,
    float* __restrict__ part_lse, int Tq, int Tk, int Tcap, int G, int nsplit, int kps,
    int NR, int nwg, float c) {
  attn_rows::row_chunk_attention<D, CAUSAL>(Q, K, V, O, LSE, part_o, part_lse, Tq, Tk, Tcap, G,
                                            nsplit, kps, NR, nwg, c);
}

// Merge of the splits: one wave per query row, D / 64 columns per lane.
// The row's log-sum-exp over the splits, lse = ln sum_s exp(lse_s), comes
// from wave reductions over lanes that each hold splits lane, lane + 64, ...
// (the first 64 in a register, read once); then O = sum_s exp(lse_s - lse)
// O_s, with kCombineUnroll splits' partial rows loaded at a time and each
// split's weight read from the lane that holds it.  The first group of
// partial rows is loaded before the reductions, which it does not depend
// on, so that a merge of up to kCombineUnroll splits waits for one memory
// round trip.  (A loop over the splits one load at a time is a chain of
// 3 nsplit dependent memory round trips: 20 us for 32 splits.)
constexpr int kCombineUnroll = 16;

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

template <int D>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, __bf16* __restrict__ O,
    float* __restrict__ LSE, int NR, int nsplit) {
  constexpr int CPL = D / 64;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // one per wave
  const int lane = threadIdx.x & 63;
  if (row >= NR) return;  // the whole wave
  const float* src = part_o + (size_t)row * D + lane * CPL;
  const size_t split_stride = (size_t)NR * D;
  auto load = [&](float (&v)[kCombineUnroll][CPL], int s, int n) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < kCombineUnroll; ++k)
#pragma unroll
      for (int u = 0; u < CPL; ++u)
        v[k][u] = k < n ? src[(size_t)(s + k) * split_stride + u] : 0.0f;
  };
  float v[kCombineUnroll][CPL];
  load(v, 0, min(kCombineUnroll, nsplit));

  const float x0 = lane < nsplit ? part_lse[(size_t)lane * NR + row] : -INFINITY;
  float mx = x0;
  for (int s = lane + 64; s < nsplit; s += 64) mx = fmaxf(mx, part_lse[(size_t)s * NR + row]);
  const float M = wave_max(mx);
  float L = exp2_hw((x0 - M) * kLog2e);  // exp2(-inf) = 0 past the last split
  for (int s = lane + 64; s < nsplit; s += 64)
    L += exp2_hw((part_lse[(size_t)s * NR + row] - M) * kLog2e);
  const float lse = M + log2_hw(wave_sum(L)) * kLn2;

  float o[CPL] = {};
  for (int s0 = 0; s0 < nsplit; s0 += 64) {
    // weight of split s0 + lane
    const int sl = s0 + lane;
    const float x = s0 == 0 ? x0 : sl < nsplit ? part_lse[(size_t)sl * NR + row] : -INFINITY;
    const float w = exp2_hw((x - lse) * kLog2e);
    const int n = min(64, nsplit - s0);
    for (int i = 0; i < n; i += kCombineUnroll) {
      if (s0 + i > 0) load(v, s0 + i, n - i);
#pragma unroll
      for (int k = 0; k < kCombineUnroll; ++k) {
        // lanes i + k < 64 always (i < n <= 64, and the weight of a lane
        // past the last split is 0)
        const float wk = __builtin_bit_cast(
            float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), (i + k) & 63));
#pragma unroll
        for (int u = 0; u < CPL; ++u) o[u] = fmaf(wk, v[k][u], o[u]);
      }
    }
  }
#pragma unroll
  for (int u = 0; u < CPL; ++u) O[(size_t)row * D + lane * CPL + u] = (__bf16)o[u];
  if (lane == 0) LSE[row] = lse;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int64_t kMaxHeadBytes = (int64_t(1) << 31) - 1;

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// Workgroups per (key/value head, split): one per 32 query rows.
int64_t row_chunks(int64_t Tq, int64_t G) { return (Tq * G + kMaxRows - 1) / kMaxRows; }

// With many query rows per key/value head the work is the contractions,
// not reading the cache; when in addition the forward kernel's grid (of
// 128-row workgroups) fills the device, that kernel (software pipelined, K and V tiles shared by its
// 8 or 4 waves) runs them over the cache instead of the row-chunk kernel.
// Measured on MI355X (us, forward / row-chunk): B = 2, 16 heads, Tq =
// 1024, Tk = 4096, d = 128 91 / 145; but 32 query / 8 key-value heads,
// Tq = 64, Tk = 8192 143 / 44 and 8 heads, Tq = 2048, Tk = 16384, d = 64
// 208 / 142 (grids below one 128-row workgroup per CU).
constexpr int64_t kFwdMinRows = 256;
bool over_forward(int64_t B, int64_t H, int64_t H_kv, int64_t Tq) {
  return Tq * (H / H_kv) >= kFwdMinRows && attn_internal::fwd_fills_device(B, H, Tq);
}


// Split of the keys: about kTargetGroups workgroups over the B*H_kv groups
// (times their row chunks),
// each split at least kMinSplitKeys keys (fewer splits when the cache is
// short) and a multiple of the 4 waves' 32-key blocks.  Returns nsplit and
// sets *kps.
int64_t choose_split(int64_t BHkv, int64_t Tk, int64_t* kps) {
  int64_t want = (kTargetGroups + BHkv - 1) / BHkv;
  int64_t most = (Tk + kMinSplitKeys - 1) / kMinSplitKeys;
  int64_t n = want < most ? want : most;
  if (n < 1) n = 1;
  const int64_t unit = kBlk * kWaves;
  int64_t per = (Tk + n - 1) / n;
  per = (per + unit - 1) / unit * unit;
  *kps = per;
  return (Tk + per - 1) / per;
}

// Key splits of a call (one when the forward kernel runs it).
int64_t splits_for(int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk, int64_t* kps) {
  if (over_forward(B, H, H_kv, Tq)) {
    *kps = Tk;
    return 1;
  }
  return choose_split(B * H_kv * row_chunks(Tq, H / H_kv), Tk, kps);
}

attn_status validate(const void* q, const void* k, const void* v, const void* o,
                     const void* lse, int64_t B, int64_t H, int64_t H_kv, int64_t Tq,
                     int64_t Tk, int64_t Tk_cap, int64_t d, int causal, float scale,
                     bool& empty) {
  empty = false;
  if (B < 0 || H < 0 || H_kv < 0 || Tq < 0 || Tk < 0 || Tk_cap < Tk) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if ((H_kv == 0) != (H == 0) || (H_kv > 0 && H % H_kv != 0)) return ATTN_ERR_SHAPE;
  if (B == 0 || H == 0 || Tq == 0) {
    empty = true;
    return ATTN_OK;
  }
  // the new queries are the last Tq positions of the cache; a query needs at
  // least one key
  if (Tk < 1 || (causal && Tk < Tq)) return ATTN_ERR_SHAPE;
  // row and grid indices are 32-bit: Tq G rows per key/value head, their
  // 32-row chunks over all heads, B H Tq output rows
  if (Tq * (H / H_kv) > (int64_t(1) << 30)) return ATTN_ERR_SHAPE;
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if ((Tk_cap + 64) * d * 2 > kMaxHeadBytes) return ATTN_ERR_SHAPE;
  if (B > (int64_t(1) << 31) / H) return ATTN_ERR_SHAPE;
  if (B * H > (INT64_MAX / 8) / (Tk_cap * d * 2)) return ATTN_ERR_SHAPE;
  if (B * H_kv * row_chunks(Tq, H / H_kv) > (int64_t(1) << 30)) return ATTN_ERR_SHAPE;
  if (B * H * Tq > INT32_MAX) return ATTN_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return ATTN_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return ATTN_ERR_ALIGN;
  const int64_t qb = B * H * Tq * d * 2, kb = B * H_kv * Tk_cap * d * 2, lb = B * H * Tq * 4;
  if (overlaps(o, qb, q, qb) || overlaps(o, qb, k, kb) || overlaps(o, qb, v, kb) ||
      overlaps(lse, lb, q, qb) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) ||
      overlaps(lse, lb, o, qb))
    return ATTN_ERR_ARG;
  return ATTN_OK;
}

template <int D>
const void* decode_kernel(int causal) {
  return causal ? (const void*)attn_decode_kernel<D, true>
                : (const void*)attn_decode_kernel<D, false>;
}

// Both decode entry points after validation: ws (ws_bytes) holds the split
// partial results when there is more than one split.
attn_status decode_launch(const void* q, const void* k, const void* v, void* o, float* lse,
                          void* ws, int64_t ws_bytes, int64_t B, int64_t H, int64_t H_kv,
                          int64_t Tq, int64_t Tk, int64_t Tk_cap, int64_t d, int causal,
                          float scale, hipStream_t stream) {
  int64_t kps;
  const int64_t nchunk = row_chunks(Tq, H / H_kv);
  const int64_t nsplit = splits_for(B, H, H_kv, Tq, Tk, &kps);
  const int64_t NR = B * H * Tq;
  const int64_t need = nsplit > 1 ? nsplit * NR * (d + 1) * 4 : 0;
  float* part_o = nullptr;
  float* part_lse = nullptr;
  if (need > 0) {
    if (!ws || ws_bytes < need) return ATTN_ERR_WORKSPACE;
    if ((uintptr_t)ws & 15u) return ATTN_ERR_ALIGN;
    const int64_t qb = NR * d * 2, kb = B * H_kv * Tk_cap * d * 2, lb = NR * 4;
    if (overlaps(ws, need, q, qb) || overlaps(ws, need, k, kb) || overlaps(ws, need, v, kb) ||
        overlaps(ws, need, o, qb) || overlaps(ws, need, lse, lb))
      return ATTN_ERR_ARG;
    part_o = (float*)ws;
    part_lse = part_o + nsplit * NR * d;
  }
  attn_status st;
  if ((st = check_device()) != ATTN_OK) return st;
  if (over_forward(B, H, H_kv, Tq))
    return attn_internal::fwd_over_cache(q, k, v, o, lse, B, H, H_kv, Tq, Tk, Tk_cap, d, causal,
                                         scale, stream);

  int tq = (int)Tq, tk = (int)Tk, tcap = (int)Tk_cap, g = (int)(H / H_kv), ns = (int)nsplit,
      kp = (int)kps, nr = (int)NR, nwg = (int)(B * H_kv * nsplit);
  float c = scale * kLog2e;
  void* args[] = {(void*)&q,  (void*)&k,  (void*)&v,    (void*)&o,  (void*)&lse,
                  (void*)&part_o, (void*)&part_lse, (void*)&tq, (void*)&tk, (void*)&tcap,
                  (void*)&g,  (void*)&ns, (void*)&kp,   (void*)&nr, (void*)&nwg, (void*)&c};
  const void* kern = d == 64 ? decode_kernel<64>(causal) : decode_kernel<128>(causal);
  const dim3 grid((unsigned)(nwg * nchunk));
  if (hipLaunchKernel(kern, grid, dim3(kThreads), args, 0, stream) != hipSuccess)
    return ATTN_ERR_LAUNCH;
  if (nsplit > 1) {
    const float* po = part_o;
    const float* pl = part_lse;
    void* cargs[] = {(void*)&po, (void*)&pl, (void*)&o, (void*)&lse, (void*)&nr, (void*)&ns};
    const void* ck = d == 64 ? (const void*)attn_decode_combine_kernel<64>
                             : (const void*)attn_decode_combine_kernel<128>;
    if (hipLaunchKernel(ck, dim3((unsigned)((NR + 3) / 4)), dim3(256), cargs, 0, stream) !=
        hipSuccess)
      return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

// Device scratch of attn_decode_noalloc (the split partial results), for
// callers that cannot allocate.  Each device the library runs on holds its
// own copy from the time the library's code object is loaded on it until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// device memory: its device address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is ever passed to
// a kernel.
constexpr int64_t kScratchBytes = ATTN_DECODE_NOALLOC_MAX_BYTES;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch (looked up on the first
// call on each device).
attn_status scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ATTN_ERR_DEVICE;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int64_t attn_decode_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk,
                                    int64_t d) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || Tq <= 0 || Tk <= 0 || (d != 64 && d != 128)) return 0;
  if (H % H_kv != 0) return 0;
  int64_t kps;
  const int64_t n = splits_for(B, H, H_kv, Tq, Tk, &kps);
  return n > 1 ? n * B * H * Tq * (d + 1) * 4 : 0;
}

attn_status attn_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                        void* ws, int64_t ws_bytes, int64_t B, int64_t H, int64_t H_kv,
                        int64_t Tq, int64_t Tk, int64_t Tk_cap, int64_t d, int causal,
                        float scale, hipStream_t stream) {
  bool empty;
  attn_status st = validate(q, k, v, o, lse, B, H, H_kv, Tq, Tk, Tk_cap, d, causal, scale,
                            empty);
  if (st != ATTN_OK || empty) return st;
  return decode_launch(q, k, v, o, lse, ws, ws_bytes, B, H, H_kv, Tq, Tk, Tk_cap, d, causal,
                       scale, stream);
}

attn_status attn_decode_noalloc(const void* q, const void* k, const void* v, void* o,
                                float* lse, int64_t B, int64_t H, int64_t H_kv, int64_t Tq,
                                int64_t Tk, int64_t Tk_cap, int64_t d, int causal, float scale,
                                hipStream_t stream) {
  bool empty;
  attn_status st = validate(q, k, v, o, lse, B, H, H_kv, Tq, Tk, Tk_cap, d, causal, scale,
                            empty);
  if (st != ATTN_OK || empty) return st;
  if (attn_decode_workspace_bytes(B, H, H_kv, Tq, Tk, d) > kScratchBytes)
    return ATTN_ERR_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_address(&ws)) != ATTN_OK) return st;
  return decode_launch(q, k, v, o, lse, ws, kScratchBytes, B, H, H_kv, Tq, Tk, Tk_cap, d, causal,
                       scale, stream);
}

const char* attn_decode_kernel_name_for(int64_t B, int64_t H, int64_t H_kv, int64_t Tq,
                                        int64_t Tk, int64_t d, int causal) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || Tq <= 0 || Tk <= 0 || H % H_kv != 0) return nullptr;
  if ((d != 64 && d != 128) || (causal != 0 && causal != 1)) return nullptr;
  if (B > (int64_t(1) << 31) / H || Tq > (int64_t(1) << 30)) return nullptr;
  if (check_device() != ATTN_OK) return nullptr;
  if (over_forward(B, H, H_kv, Tq))
    return attn_internal::fwd_over_cache_kernel_name(B, H, Tq, d, causal);
  static const char* names[2][2] = {
      {"attn_decode_bf16_d64_full_w4_blk32", "attn_decode_bf16_d64_causal_w4_blk32"},
      {"attn_decode_bf16_d128_full_w4_blk32", "attn_decode_bf16_d128_causal_w4_blk32"}};
  return names[d == 128 ? 1 : 0][causal];
}

int64_t attn_decode_splits(int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || Tq <= 0 || Tk <= 0 || H % H_kv != 0) return 0;
  int64_t kps;
  return splits_for(B, H, H_kv, Tq, Tk, &kps);
}

}  // extern "C"
