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
#include <cstring>

#include "attn.h"
#include "tiles.h"

namespace {

using namespace attn_tiles;

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlk = 32;            // keys per block (one MFMA score tile)
constexpr int kMaxRows = 32;        // query rows of one workgroup (one MFMA column block)
constexpr int kMaxChunks = 8;       // Tq * G <= 256 query rows per key/value head
// Key split: about kTargetGroups workgroups (one round at two per CU), each
// split at least kMinSplitKeys long: short splits cost a prologue, an LDS
// merge and partial results each (measured: 32 splits of 4096 keys read a
// 131072-key cache at 4.7 TB/s, 128 splits of 1024 keys at 3.3 TB/s).
constexpr int kMinSplitKeys = 4096;
constexpr int kTargetGroups = 512;
// Running-max threshold (log2 units), as in the forward: the max is raised
// only when a block's max exceeds it by more than this, so weights stay
// below 2^64 and sums of at most 2^17 of them far inside fp32.
constexpr float kLazyRescale = 64.0f;
constexpr float kMinusHuge = -1e38f;

__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Workgroup (row chunk, kv head bhkv, split s) over keys
// [s kps, min(Tk, (s + 1) kps)).  Row r < R = Tq G of the group is member
// r / Tq (query head bhkv G + r / Tq), new query r % Tq; the chunk holds rows
// 32 chunk .. 32 chunk + 31.  part_o / part_lse: when nsplit > 1,
// the split's normalised output and natural-log LSE per query row
// (row index (bhq Tq + qi), NR rows), else unused and O, LSE written.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads, 2) void attn_decode_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, float* __restrict__ part_o,
    float* __restrict__ part_lse, int Tq, int Tk, int Tcap, int G, int nsplit, int kps,
    int NR, int nwg, float c) {
  using C = RowTile<D>;
  constexpr int NDS = C::NDS, NDT = C::NDT, RB = C::RB;
  constexpr int TB = kBlk * RB;  // bytes of one K or V block
  // Two V stages per wave, each stage its own object so that the compiler
  // can tell the loads into one from the reads of the other.
  __shared__ __attribute__((aligned(1024))) char sV0[kWaves][TB];
  __shared__ __attribute__((aligned(1024))) char sV1[kWaves][TB];
  __shared__ float sM[kWaves][kMaxRows], sL[kWaves][kMaxRows], sW[kWaves][kMaxRows];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, h = lane >> 5;
  // Workgroup id: row chunk outermost (nwg = B H_kv nsplit workgroups per
  // chunk), so the chunks reading the same keys share an XCD when nwg is a
  // multiple of 8.
  const int id = blockIdx.x;
  const int chunk = id / nwg, rest = id % nwg;
  const int bhkv = rest / nsplit, split = rest % nsplit;
  const int R = Tq * G;             // query rows of the group
  const int r0 = kMaxRows * chunk;  // this workgroup's first row
  const bool row_ok = r0 + j < R;
  const int qi = (r0 + j) % Tq;
  const size_t qrow = ((size_t)bhkv * G + (r0 + j) / Tq) * Tq + qi;  // global query row
  const int pos = Tk - Tq + qi;                                      // its position

  // Q fragment: B operand [d][query] of S^T = K Q^T.  The contraction
  // over d takes k-step s of lane half h from d = 8 (NDS h + s) .. + 8, so
  // that a lane's K operand over all steps is one contiguous run of its row.
  bf16x8_t qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    qf[s] = bf16x8_t{};
    if (row_ok)
      qf[s] = *reinterpret_cast<const bf16x8_t*>(Q + qrow * D + 8 * (NDS * h + s));
  }

  const int k_lo = split * kps, k_hi = min(Tk, k_lo + kps);
  const int nblk = (k_hi - k_lo + kBlk - 1) / kBlk;
  const int nmine = nblk > wave ? (nblk - wave + kWaves - 1) / kWaves : 0;
  const __bf16* Kh = K + (size_t)bhkv * Tcap * D;
  const __bf16* Vh = V + (size_t)bhkv * Tcap * D;

  TileAddr<D> ad;
  ad.init(lane);
  TileDma<D, kBlk, 1> dma;
  dma.init(0, lane);
  constexpr int PER = TileDma<D, kBlk, 1>::PER;  // V load instructions per block
  // K operand of lane (j, h): row row_perm(j) of the block, d from
  // 8 NDS h on (see qf).  Keys >= k_hi read as zero (and are masked below).
  const int krow = row_perm(j) * RB + 16 * NDS * h;
  auto load = [&](bf16x8_t (&kr)[NDS], char* vt, int i) __attribute__((always_inline)) {
    const int kb0 = k_lo + kBlk * (wave + kWaves * i);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kh + (size_t)kb0 * D, max(k_hi - kb0, 0) * RB);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      kr[s] = __builtin_bit_cast(bf16x8_t, buf_load16(rk, krow + 16 * s));
    dma.load(vt, Vh, k_hi, kb0, 0);
  };

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = kMinusHuge, l_run = 0.0f, w_run = 0.0f;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  // One block: scores, mask, online softmax, O^T += V^T P^T.
  auto block = [&](const bf16x8_t (&kr)[NDS], const char* vt, int i)
      __attribute__((always_inline)) {
    const int kb0 = k_lo + kBlk * (wave + kWaves * i);
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[s], qf[s], sc, 0, 0, 0);
    // scores in log2 units (any sign of the scale); register 8 a + e holds
    // key kb0 + 16 a + 8 h + e of query row j
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] *= c;
    if (kb0 + kBlk > k_hi || (CAUSAL && kb0 + kBlk - 1 > Tk - Tq)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + 16 * (r >> 3) + 8 * h + (r & 7);
        if (key >= k_hi || (CAUSAL && key > pos)) sc[r] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sc[r]);
    const float mt = pair_max(mx);
    const bool grow = mt > m_run + kLazyRescale;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
      const float alpha = grow ? exp2_hw(m_run - mt) : 1.0f;
      l_run *= alpha;
      w_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
      m_run = grow ? mt : m_run;
    }
    bf16x8_t pb[2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = exp2_hw(sc[8 * a + e] - m_run);
        l_run += p;
        pb[a][e] = (__bf16)p;
      }
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      // the normaliser of O sums exactly the bf16 weights the MFMA uses
      w_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 0, 1), one2,
                                             w_run, false);
      w_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 2, 3), one2,
                                             w_run, false);
      w_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 4, 5), one2,
                                             w_run, false);
      w_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 6, 7), one2,
                                             w_run, false);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            lds_tr(vt, 16 * a * RB + ad.tr[0][dt], 16 * a * RB + ad.tr[1][dt]), pb[a],
            oacc[dt], 0, 0, 0);
    }
  };
  // Waits until at most n of this wave's loads are in flight (loads
  // complete in issue order; a direct-to-LDS load has written LDS when it
  // completes).
  auto wait_loads = [&](auto n) __attribute__((always_inline)) {
    constexpr int N = decltype(n)::value;
    static_assert(N < 64, "vmcnt field");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
    asm volatile("" ::: "memory");
  };
  using Zero = std::integral_constant<int, 0>;
  using Next = std::integral_constant<int, NDS + PER>;  // one block's loads

  bf16x8_t k0[NDS], k1[NDS];
  if (nmine > 0) load(k0, sV0[wave], 0);
  for (int i = 0; i < nmine; i += 2) {
    if (i + 1 < nmine) {
      load(k1, sV1[wave], i + 1);
      wait_loads(Next{});
    } else {
      wait_loads(Zero{});
    }
    block(k0, sV0[wave], i);
    if (i + 1 >= nmine) break;
    if (i + 2 < nmine) {
      load(k0, sV0[wave], i + 2);
      wait_loads(Next{});
    } else {
      wait_loads(Zero{});
    }
    block(k1, sV1[wave], i + 1);
  }

  // Merge the four waves' partial results for each query row.
  l_run += __shfl_xor(l_run, 32);
  w_run += __shfl_xor(w_run, 32);
  __syncthreads();  // every wave is done with its LDS stages
  // Wave w's 32 x D fp32 accumulator goes to half (w & 1) of sV0 (w < 2)
  // or sV1 (w >= 2): each V stage holds exactly two of them.
  static_assert(sizeof(sV0) == 2 * sizeof(float) * kMaxRows * D, "merge buffer");
  auto part = [&](int w) __attribute__((always_inline)) -> float* {
    return reinterpret_cast<float*>(w < 2 ? &sV0[0][0] : &sV1[0][0]) + (w & 1) * kMaxRows * D;
  };
  {
    float* mine = part(wave);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t v4;
#pragma unroll
        for (int u = 0; u < 4; ++u) v4[u] = oacc[dt][4 * g + u];
        *reinterpret_cast<f32x4_t*>(&mine[j * D + 32 * dt + 8 * g + 4 * h]) = v4;
      }
  }
  if (h == 0) {
    sM[wave][j] = m_run;
    sL[wave][j] = l_run;
    sW[wave][j] = w_run;
  }
  __syncthreads();

  // 8 threads per query row, D / 8 columns each.
  constexpr int CPT = D / 8;
  const int row = tid >> 3, c0 = (tid & 7) * CPT;
  if (r0 + row >= R) return;
  float M = sM[0][row];
#pragma unroll
  for (int w = 1; w < kWaves; ++w) M = fmaxf(M, sM[w][row]);
  float a[kWaves], Lt = 0.0f, Wt = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    a[w] = exp2_hw(sM[w][row] - M);
    Lt += a[w] * sL[w][row];
    Wt += a[w] * sW[w][row];
  }
  // A row with no visible key in this split (causal, split past its
  // position) has Wt = 0: output 0, LSE -inf, weight 0 in the merge.
  const float inv = Wt > 0.0f ? 1.0f / Wt : 0.0f;
  float o[CPT];
#pragma unroll
  for (int u = 0; u < CPT; ++u) {
    float acc = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      acc = fmaf(a[w], part(w)[row * D + c0 + u], acc);
    o[u] = acc * inv;
  }
  const float lse = Lt > 0.0f ? (M + log2_hw(Lt)) * kLn2 : -INFINITY;
  const size_t orow = ((size_t)bhkv * G + (r0 + row) / Tq) * Tq + (r0 + row) % Tq;
  if (nsplit == 1) {
#pragma unroll
    for (int u = 0; u < CPT; u += 4) {
      __bf16 b4[4];
#pragma unroll
      for (int x = 0; x < 4; ++x) b4[x] = (__bf16)o[u + x];
      u32x2_t bits;
      std::memcpy(&bits, b4, 8);
      *reinterpret_cast<u32x2_t*>(O + orow * D + c0 + u) = bits;
    }
    if (c0 == 0) LSE[orow] = lse;
  } else {
    float* dst = part_o + ((size_t)split * NR + orow) * D + c0;
#pragma unroll
    for (int u = 0; u < CPT; u += 4)
      *reinterpret_cast<f32x4_t*>(dst + u) = f32x4_t{o[u], o[u + 1], o[u + 2], o[u + 3]};
    if (c0 == 0) part_lse[(size_t)split * NR + orow] = lse;
  }
}

// Merge of the splits: one wave per query row, D / 64 columns per lane.
template <int D>
__global__ __launch_bounds__(256) void attn_decode_combine_kernel(
    const float* __restrict__ part_o, const float* __restrict__ part_lse, __bf16* __restrict__ O,
    float* __restrict__ LSE, int NR, int nsplit) {
  constexpr int CPL = D / 64;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= NR) return;
  float M = -INFINITY;
  for (int s = 0; s < nsplit; ++s) M = fmaxf(M, part_lse[(size_t)s * NR + row]);
  float L = 0.0f;
  for (int s = 0; s < nsplit; ++s)
    L += exp2_hw((part_lse[(size_t)s * NR + row] - M) * kLog2e);
  const float lse = M + log2_hw(L) * kLn2;
  float o[CPL] = {};
  for (int s = 0; s < nsplit; ++s) {
    const float wgt = exp2_hw((part_lse[(size_t)s * NR + row] - lse) * kLog2e);
    const float* src = part_o + ((size_t)s * NR + row) * D + lane * CPL;
#pragma unroll
    for (int u = 0; u < CPL; ++u) o[u] = fmaf(wgt, src[u], o[u]);
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

attn_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
  return std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? ATTN_OK : ATTN_ERR_DEVICE;
}

// Workgroups per (key/value head, split): one per 32 query rows.
int64_t row_chunks(int64_t Tq, int64_t G) { return (Tq * G + kMaxRows - 1) / kMaxRows; }

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
  if (Tq * (H / H_kv) > kMaxRows * kMaxChunks) return ATTN_ERR_UNSUPPORTED;
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  if ((Tk_cap + 64) * d * 2 > kMaxHeadBytes) return ATTN_ERR_SHAPE;
  if (B > (int64_t(1) << 31) / H) return ATTN_ERR_SHAPE;
  if (B * H > (INT64_MAX / 8) / (Tk_cap * d * 2)) return ATTN_ERR_SHAPE;
  if (B * H_kv * kTargetGroups * kMaxChunks > INT32_MAX) return ATTN_ERR_SHAPE;
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

}  // namespace

extern "C" {

int64_t attn_decode_workspace_bytes(int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk,
                                    int64_t d) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || Tq <= 0 || Tk <= 0 || (d != 64 && d != 128)) return 0;
  if (H % H_kv != 0) return 0;
  int64_t kps;
  const int64_t n = choose_split(B * H_kv * row_chunks(Tq, H / H_kv), Tk, &kps);
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
  int64_t kps;
  const int64_t nchunk = row_chunks(Tq, H / H_kv);
  const int64_t nsplit = choose_split(B * H_kv * nchunk, Tk, &kps);
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
  if ((st = check_device()) != ATTN_OK) return st;

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

int64_t attn_decode_splits(int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || Tq <= 0 || Tk <= 0 || H % H_kv != 0) return 0;
  int64_t kps;
  return choose_split(B * H_kv * row_chunks(Tq, H / H_kv), Tk, &kps);
}

}  // extern "C"
