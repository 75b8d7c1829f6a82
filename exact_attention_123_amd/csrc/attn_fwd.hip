// Fused, I/O-aware forward pass of exact scaled dot-product attention for
// AMD Instinct MI355X (gfx950, CDNA4), behind the C ABI of include/attn.h.
//
// What is computed, per (batch, head): S = scale * Q K^T, an optional causal
// mask (key j visible to query i iff j <= i), a row softmax and O = P V,
// plus LSE_i = ln sum_j exp(S_ij).  ("Attention Mechanism: Computation &
// Memory Patterns", section 1; "Why Attention Is Difficult to Optimize",
// "The Attention Computation Flow" and Figure 1.)
//
// How.  One workgroup owns BR consecutive query rows of one head and walks
// the key/value tiles it needs; S and P only ever exist as MFMA accumulator
// tiles in registers, so no T x T array touches HBM ("Attention Mechanism",
// sections 3-4: tiling, fusion, online softmax).  Each key/value tile is
// loaded once per workgroup from global memory with 16-byte coalesced loads
// into LDS (double-buffered: the loads of tile t+1 are in flight while
// tile t is computed) and read from LDS by all waves of the workgroup.
//
// Per wave (32 query rows), per tile of BC keys:
//   1. S^T = K Q^T on MFMA 32x32x16 bf16 (fp32 accumulate).  Computing the
//      transpose puts one query in each lane column, so a row's scores live
//      in one lane pair (l, l+32): the row max is 31 in-register max ops and
//      one cross-lane exchange, and the accumulator layout is already the
//      B-operand layout of the second contraction (no LDS round trip for P).
//   2. scale, mask (only on tiles that straddle the diagonal or the ragged
//      end of the sequence), online softmax in the log2 domain: running max
//      m, running normaliser l (lane-partial, combined at the end) and the
//      fp32 output accumulator rescaled by exp2(m_old - m_new) ("FlashAttention
//      -- avoid writing the giant intermediate", "Tiling and an incremental
//      normalization").
//   3. O^T += V^T P^T on MFMA 32x32x16 bf16, P rounded to bf16 (RNE).
// Epilogue: O = acc / l (bf16 RNE), LSE = ln2 * (m + log2 l).
//
// The workgroup order is heavy-first for causal masks (the last query
// blocks need the most key tiles and are dispatched first), and consecutive
// workgroup ids walk the heads so that all blocks of one head land on the
// same XCD (workgroups are dispatched round-robin over the 8 XCDs), which
// keeps a head's K and V in that XCD's L2.

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "attn.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // 4 waves of 64 lanes
constexpr int kBR = 128;       // query rows per workgroup (32 per wave)
constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Raw buffer descriptor over `bytes` bytes at `base`.  Loads through it whose
// byte range lies past `bytes` return zero instead of touching memory, which
// is how the ragged end of the sequence (keys or queries >= T) is read as
// zero without branches.  Word 3 (0x00020000) is the raw-buffer format word
// of the gfx9 family.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// Row of the 32-row MFMA operand tile that lane row i feeds with key
// (swap bits 2 and 3 of i).  With this order the accumulator registers
// r = 8a..8a+7 of lane half h hold keys 16a + 8h + 0..7, i.e. eight
// consecutive keys, which is what one B-operand slot of the PV MFMA wants.
__device__ __forceinline__ int key_row_perm(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// Key offset (within a 32-key block) held by accumulator register r of lane
// half h, for the bf16 kernel (permuted rows) and the fp32 kernel (plain).
__host__ __device__ constexpr int acc_key_perm(int r, int h) {
  return 16 * (r / 8) + 8 * h + 4 * ((r / 4) & 1) + (r & 3);
}
__host__ __device__ constexpr int acc_key_plain(int r, int h) {
  return 8 * (r / 4) + 4 * h + (r & 3);
}

// Workgroup id -> (head index bh, query block qb).  Heavy-first: the
// highest query blocks (most key tiles under a causal mask) get the lowest
// ids.  Within a block index, ids walk the heads, so id and id + BH*k fall
// on the same XCD whenever BH is a multiple of 8.
__device__ __forceinline__ void block_coords(int BH, int nqb, int& bh, int& qb) {
  const int id = blockIdx.x;
  qb = nqb - 1 - id / BH;
  bh = id % BH;
}

// Max of x over the lane pair (l, l ^ 32) that holds one query's scores.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Rescaling threshold of the running max, in log2 units.  The running max m
// is only raised when a tile's max exceeds it by more than this, so p =
// exp2(c*s - m) stays below 2^kLazyRescale and the output accumulator and
// normaliser are rescaled only on those (rare, wave-uniform) occasions.  The
// result is the same softmax: the common factor cancels in acc / l.
constexpr float kLazyRescale = 8.0f;

// Online-softmax update for one wave's tile of scores ("FlashAttention --
// avoid writing the giant intermediate", "Tiling and an incremental
// normalization"; "Attention Mechanism", section 3, online softmax).
//   s   : NKT accumulator tiles of scores, masked entries = -inf; the score
//         in log2 units is cm * s
//   m   : running max in log2 units (same value in both lane halves)
//   l, w: lane-partial running normalisers, relative to m
//   o   : NDT output accumulator tiles, relative to m
// On return s holds p = exp2(cm * s - m); l, w and o are rescaled when m
// rises, and the caller adds the tile's p to l and w.
template <int NKT, int NDT>
__device__ __forceinline__ void online_softmax_update(f32x16_t (&s)[NKT], float cm, float& m,
                                                      float& l, float& w, f32x16_t (&o)[NDT]) {
  float mx = s[0][0];
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kt][r]);
  const float mt = pair_max(mx) * cm;
  // Raise a row's running max only when the tile's max outgrows it by more
  // than the threshold (m = -inf on the first tile always does).  The
  // decision is per row, so a row's result never depends on other rows; the
  // wave only skips the rescaling loop when no row needs it (alpha = 1 is
  // exact for the rows that do not).
  const bool grow = mt > m + kLazyRescale;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float alpha = !grow ? 1.0f : (m == -INFINITY) ? 0.0f : exp2_hw(m - mt);
    l *= alpha;
    w *= alpha;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
    m = grow ? mt : m;
  }
  // A row with no visible key so far keeps m = -inf; subtract 0 instead so
  // that its terms are exp2(-inf) = 0 rather than NaN.
  const float base = (m == -INFINITY) ? 0.0f : m;
#pragma unroll
  for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kt][r] = exp2_hw(fmaf(s[kt][r], cm, -base));
}

// ---------------------------------------------------------------------------
// bf16 kernel
// ---------------------------------------------------------------------------
template <int D>
struct Bf16Tile {
  static constexpr int BC = 64;              // keys per tile
  static constexpr int NKT = BC / 32;        // 32-key accumulator tiles
  static constexpr int NDS = D / 16;         // k-steps of the QK^T MFMA
  static constexpr int NDT = D / 32;         // 32-row d tiles of O^T
  static constexpr int KS = D + 8;           // K row stride in LDS (elements)
  static constexpr int VS = BC + 8;          // V^T row stride in LDS (elements)
  static constexpr int KCH = BC * D / 8 / kThreads;  // 16-byte K chunks per thread
  static constexpr int KPT = BC * D / 8 / kThreads;  // keys per thread (V transpose)
  static constexpr int NKB = BC / KPT;       // key blocks per tile (V transpose)
  static constexpr int DCH = D / 8;          // 16-byte chunks per row
};

// PRESCALE: multiply the scores by c before the softmax (any sign of c);
// otherwise (c > 0) the multiply is folded into the exponent's fma and the
// max is taken over the raw scores.
template <int D, bool CAUSAL, bool PRESCALE>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int T, int BH, int nqb, float c) {
  using C = Bf16Tile<D>;
  constexpr int BC = C::BC, NKT = C::NKT, NDS = C::NDS, NDT = C::NDT;
  constexpr int KS = C::KS, VS = C::VS, KCH = C::KCH, KPT = C::KPT, DCH = C::DCH;
  constexpr int NKB = C::NKB;
  constexpr int ROWB = D * 2;  // bytes per row of Q, K, V, O
  static_assert(KCH * kThreads * 8 == BC * D, "K tile split");
  static_assert(NKB * (D / 8) == kThreads, "V tile split");

  __shared__ __attribute__((aligned(16))) __bf16 sK[2][BC * KS];
  __shared__ __attribute__((aligned(16))) __bf16 sV[2][D * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  int bh, qb;
  block_coords(BH, nqb, bh, qb);
  const size_t head = (size_t)bh * (size_t)T * D;
  const int head_bytes = T * ROWB;
  const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Q + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(K + head, head_bytes);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(V + head, head_bytes);
  const int q0 = qb * kBR;
  const int q0w = q0 + wave * 32;
  const int qg = q0w + j;

  // Q fragment: B operand of S^T = K Q^T; lane (j, h) holds
  // Q[qg][16 s + 8 h .. +8] for every k-step s.  Rows >= T read as zero.
  bf16x8_t qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s)
    qf[s] = __builtin_bit_cast(bf16x8_t, buf_load16(rQ, qg * ROWB + (16 * s + 8 * h) * 2));

  const int kv_end = CAUSAL ? min(T, q0 + kBR) : T;
  const int ntiles = (kv_end + BC - 1) / BC;
  // Tiles below n_full need no mask: every key is < T and, when causal, no
  // later than the workgroup's first query.
  const int n_full = (CAUSAL ? min(q0 + 1, T) : T) / BC;

  // Staging registers for the next tile's global loads.
  u32x4_t kreg[KCH], vreg[KPT];
  // V transpose: each thread owns 8 d x KPT keys; the 16 (or 32) lanes of a
  // group take consecutive key blocks of one d block, so that each V^T row
  // they store is one contiguous, bank-conflict-free run.
  const int vkb = tid % NKB, vdb = tid / NKB;
  auto gload = [&](int t) {
    const int kv0 = t * BC;
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = i * kThreads + tid;
      kreg[i] = buf_load16(rK, (kv0 + ch / DCH) * ROWB + (ch % DCH) * 16);
    }
#pragma unroll
    for (int i = 0; i < KPT; ++i) vreg[i] = buf_load16(rV, (kv0 + vkb * KPT + i) * ROWB + vdb * 16);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const int ch = i * kThreads + tid;
      *reinterpret_cast<u32x4_t*>(&sK[buf][(ch / DCH) * KS + (ch % DCH) * 8]) = kreg[i];
    }
    // Transpose 8 d x KPT keys in registers and store rows d of V^T.
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int w = e >> 1, sh = (e & 1) * 16;
      unsigned int packed[KPT / 2];
#pragma unroll
      for (int i = 0; i < KPT / 2; ++i) {
        const unsigned int lo = (vreg[2 * i][w] >> sh) & 0xffffu;
        const unsigned int hi = (vreg[2 * i + 1][w] >> sh) & 0xffffu;
        packed[i] = lo | (hi << 16);
      }
      __bf16* dst = &sV[buf][(vdb * 8 + e) * VS + vkb * KPT];
      if constexpr (KPT == 4) {
        *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{packed[0], packed[1]};
      } else {
        *reinterpret_cast<unsigned int*>(dst) = packed[0];
      }
    }
  };

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f, w_run = 0.0f;
  const int krow = key_row_perm(j);

  // One tile: S^T = K Q^T, scale and mask, online softmax, O^T += V^T P^T.
  auto compute = [&](int buf, int kv0, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    f32x16_t x[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) x[kt] = f32x16_t{};
    const __bf16* kb = sK[buf];
#pragma unroll
    for (int s = 0; s < NDS; ++s)
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(kb + (kt * 32 + krow) * KS + 16 * s + 8 * h);
        x[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], x[kt], 0, 0, 0);
      }
    if constexpr (PRESCALE) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[kt][r] *= c;
    }
    if constexpr (MASK) {
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + kt * 32 + acc_key_perm(r, h);
          if (key >= T || (CAUSAL && key > qg)) x[kt][r] = -INFINITY;
        }
    }
    online_softmax_update<NKT, NDT>(x, PRESCALE ? 1.0f : c, m_run, l_run, w_run, oacc);
    const __bf16* vb = sV[buf];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        bf16x8_t pb;
#pragma unroll
        for (int u = 0; u < 8; ++u) pb[u] = (__bf16)x[kt][8 * a + u];
        // Two normalisers: l_run sums the fp32 weights (it gives LSE), and
        // w_run sums exactly the bf16 weights the PV MFMA uses, so that O =
        // sum p'v / sum p' is a convex combination of V rows (bf16 rounding
        // of a dominant weight then cancels instead of scaling O).
        const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int u = 0; u < 8; ++u) l_run += x[kt][8 * a + u];
        w_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 0, 1), one2, w_run, false);
        w_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 2, 3), one2, w_run, false);
        w_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 4, 5), one2, w_run, false);
        w_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb, pb, 6, 7), one2, w_run, false);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const bf16x8_t vv = *reinterpret_cast<const bf16x8_t*>(
              vb + (dt * 32 + j) * VS + kt * 32 + 16 * a + 8 * h);
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb, oacc[dt], 0, 0, 0);
        }
      }
  };

  gload(0);
  lstore(0);
  __syncthreads();
  int t = 0;
  for (; t < n_full; ++t) {
    if (t + 1 < ntiles) gload(t + 1);
    compute(t & 1, t * BC, std::false_type{});
    if (t + 1 < ntiles) lstore((t + 1) & 1);
    __syncthreads();
  }
  for (; t < ntiles; ++t) {
    if (t + 1 < ntiles) gload(t + 1);
    const int kv0 = t * BC;
    // Under a causal mask a wave skips tiles that start after its last query.
    if (!CAUSAL || kv0 <= q0w + 31) compute(t & 1, kv0, std::true_type{});
    if (t + 1 < ntiles) lstore((t + 1) & 1);
    __syncthreads();
  }

  // Epilogue: combine the two lane halves' partial normalisers.
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float w_tot = w_run + __shfl_xor(w_run, 32);
  if (qg < T) {
    const float inv = 1.0f / w_tot;
    __bf16* orow = O + head + (size_t)qg * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // registers 4g..4g+3 hold d = dt*32 + 8g + 4h + 0..3
        __bf16 ov[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) ov[u] = (__bf16)(oacc[dt][4 * g + u] * inv);
        u32x2_t w;
        std::memcpy(&w, ov, 8);
        *reinterpret_cast<u32x2_t*>(orow + dt * 32 + 8 * g + 4 * h) = w;
      }
    if (h == 0) LSE[(size_t)bh * T + qg] = (m_run + log2_hw(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// fp32 kernel: same structure on MFMA 32x32x2 f32.  Each lane feeds one
// element per MFMA, so V needs no transpose and K no row permutation.
// ---------------------------------------------------------------------------
template <int D>
struct F32Tile {
  static constexpr int BC = 32;
  static constexpr int NDS = D / 2;
  static constexpr int NDT = D / 32;
  static constexpr int KS = D + 1;           // odd stride: column reads spread banks
  static constexpr int VS = D;
  static constexpr int CH = BC * D / 4 / kThreads;  // 16-byte chunks per thread
  static constexpr int DCH = D / 4;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int T, int BH, int nqb, float c) {
  using C = F32Tile<D>;
  constexpr int BC = C::BC, NDS = C::NDS, NDT = C::NDT, KS = C::KS, VS = C::VS;
  constexpr int CH = C::CH, DCH = C::DCH;
  static_assert(CH * kThreads * 4 == BC * D, "tile split");

  __shared__ float sK[2][BC * KS];
  __shared__ __attribute__((aligned(16))) float sV[2][BC * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  int bh, qb;
  block_coords(BH, nqb, bh, qb);
  const size_t head = (size_t)bh * (size_t)T * D;
  const float* Qh = Q + head;
  const float* Kh = K + head;
  const float* Vh = V + head;
  const int q0 = qb * kBR;
  const int q0w = q0 + wave * 32;
  const int qg = q0w + j;

  float qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) qf[s] = qg < T ? Qh[(size_t)qg * D + 2 * s + h] : 0.0f;

  const int kv_end = CAUSAL ? min(T, q0 + kBR) : T;
  const int ntiles = (kv_end + BC - 1) / BC;

  f32x4_t kreg[CH], vreg[CH];
  auto gload = [&](int t) {
    const int kv0 = t * BC;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ch = i * kThreads + tid;
      const int row = ch / DCH, col = ch % DCH;
      const int key = kv0 + row;
      const bool ok = key < T;
      kreg[i] = ok ? *reinterpret_cast<const f32x4_t*>(Kh + (size_t)key * D + col * 4)
                   : f32x4_t{};
      vreg[i] = ok ? *reinterpret_cast<const f32x4_t*>(Vh + (size_t)key * D + col * 4)
                   : f32x4_t{};
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int ch = i * kThreads + tid;
      const int row = ch / DCH, col = ch % DCH;
#pragma unroll
      for (int u = 0; u < 4; ++u) sK[buf][row * KS + col * 4 + u] = kreg[i][u];
      *reinterpret_cast<f32x4_t*>(&sV[buf][row * VS + col * 4]) = vreg[i];
    }
  };

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  gload(0);
  lstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) gload(t + 1);
    const int kv0 = t * BC;
    const bool active = !CAUSAL || kv0 <= q0w + 31;
    if (active) {
      f32x16_t x[1] = {f32x16_t{}};
      const float* kb = sK[buf];
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        x[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(kb[j * KS + 2 * s + h], qf[s], x[0], 0, 0, 0);
#pragma unroll
      for (int r = 0; r < 16; ++r) x[0][r] *= c;
      const bool need_mask = (kv0 + BC > T) || (CAUSAL && kv0 + BC - 1 > q0w);
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kv0 + acc_key_plain(r, h);
          if (key >= T || (CAUSAL && key > qg)) x[0][r] = -INFINITY;
        }
      }
      float unused = 0.0f;  // fp32 P is not rounded: one normaliser serves O and LSE
      online_softmax_update<1, NDT>(x, 1.0f, m_run, l_run, unused, oacc);
#pragma unroll
      for (int r = 0; r < 16; ++r) l_run += x[0][r];
      const float* vb = sV[buf];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = acc_key_plain(r, h);
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vb[key * VS + dt * 32 + j], x[0][r],
                                                         oacc[dt], 0, 0, 0);
      }
    }
    if (t + 1 < ntiles) lstore((t + 1) & 1);
    __syncthreads();
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qg < T) {
    const float inv = 1.0f / l_tot;
    float* orow = O + head + (size_t)qg * D;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4_t w;
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = oacc[dt][4 * g + u] * inv;
        *reinterpret_cast<f32x4_t*>(orow + dt * 32 + 8 * g + 4 * h) = w;
      }
    if (h == 0) LSE[(size_t)bh * T + qg] = (m_run + log2_hw(l_tot)) * kLn2;
  }
}

// ---------------------------------------------------------------------------
// Host side: validation, device check, launch.
// ---------------------------------------------------------------------------

// Per-head byte offsets are 32-bit (buffer descriptors), so one head of a
// tensor, plus a tile of overhang at the ragged end, must stay below 2 GiB.
constexpr int64_t kMaxHeadBytes = (int64_t(1) << 31) - 1;

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

attn_status validate(const void* q, const void* k, const void* v, const void* o, const void* lse,
                     int64_t B, int64_t H, int64_t T, int64_t d, int causal, float scale,
                     int64_t elem, bool& empty) {
  empty = false;
  if (B < 0 || H < 0 || T < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if (B == 0 || H == 0 || T == 0) {
    empty = true;
    return ATTN_OK;
  }
  if (!q || !k || !v || !o || !lse) return ATTN_ERR_NULL;
  // sizes: a head fits 32-bit byte offsets, the grid fits in 2^31-1, and
  // total byte sizes fit in int64.
  if ((T + 256) * d * elem > kMaxHeadBytes) return ATTN_ERR_SHAPE;
  if (B > (int64_t(1) << 31) / H) return ATTN_ERR_SHAPE;
  const int64_t BH = B * H;
  const int64_t nqb = (T + kBR - 1) / kBR;
  if (BH > INT32_MAX / nqb) return ATTN_ERR_SHAPE;
  if (BH > (INT64_MAX / 8) / (T * d * elem)) return ATTN_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o) & 15u) return ATTN_ERR_ALIGN;
  if ((uintptr_t)lse & 3u) return ATTN_ERR_ALIGN;
  const int64_t nb = BH * T * d * elem, lb = BH * T * 4;
  if (overlaps(o, nb, q, nb) || overlaps(o, nb, k, nb) || overlaps(o, nb, v, nb) ||
      overlaps(lse, lb, q, nb) || overlaps(lse, lb, k, nb) || overlaps(lse, lb, v, nb) ||
      overlaps(lse, lb, o, nb))
    return ATTN_ERR_ARG;
  return ATTN_OK;
}

// Per-device cache of "is this a gfx950": 0 unknown, 1 yes, 2 no.
std::atomic<int> g_arch_ok[64];

attn_status check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_DEVICE;
  if (dev < 0 || dev >= 64) return ATTN_ERR_DEVICE;
  int s = g_arch_ok[dev].load(std::memory_order_relaxed);
  if (s == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
    s = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_ok[dev].store(s, std::memory_order_relaxed);
  }
  return s == 1 ? ATTN_OK : ATTN_ERR_DEVICE;
}

template <typename Elem>
attn_status launch(const void* kernel, const Elem* q, const Elem* k, const Elem* v, Elem* o,
                   float* lse, int64_t B, int64_t H, int64_t T, float scale, hipStream_t stream) {
  int t = (int)T, bh = (int)(B * H), nqb = (int)((T + kBR - 1) / kBR);
  float c = scale * kLog2e;
  void* args[] = {(void*)&q, (void*)&k, (void*)&v, (void*)&o, (void*)&lse,
                  (void*)&t, (void*)&bh,  (void*)&nqb, (void*)&c};
  const dim3 grid((unsigned)(bh * nqb)), block(kThreads);
  if (hipLaunchKernel(kernel, grid, block, args, 0, stream) != hipSuccess) return ATTN_ERR_LAUNCH;
  return ATTN_OK;
}

template <bool PRESCALE>
const void* bf16_kernel_p(int64_t d, int causal) {
  if (d == 64) return causal ? (const void*)attn_fwd_bf16_kernel<64, true, PRESCALE>
                             : (const void*)attn_fwd_bf16_kernel<64, false, PRESCALE>;
  return causal ? (const void*)attn_fwd_bf16_kernel<128, true, PRESCALE>
                : (const void*)attn_fwd_bf16_kernel<128, false, PRESCALE>;
}

const void* bf16_kernel(int64_t d, int causal, float scale) {
  return scale > 0.0f ? bf16_kernel_p<false>(d, causal) : bf16_kernel_p<true>(d, causal);
}

const void* f32_kernel(int64_t d, int causal) {
  if (d == 64) return causal ? (const void*)attn_fwd_f32_kernel<64, true>
                             : (const void*)attn_fwd_f32_kernel<64, false>;
  return causal ? (const void*)attn_fwd_f32_kernel<128, true>
                : (const void*)attn_fwd_f32_kernel<128, false>;
}

}  // namespace

extern "C" {

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                     int64_t H, int64_t T, int64_t d, int causal, float scale,
                     hipStream_t stream) {
  bool empty;
  attn_status st = validate(q, k, v, o, lse, B, H, T, d, causal, scale, 2, empty);
  if (st != ATTN_OK || empty) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  return launch<__bf16>(bf16_kernel(d, causal, scale), (const __bf16*)q, (const __bf16*)k,
                        (const __bf16*)v, (__bf16*)o, lse, B, H, T, scale, stream);
}

attn_status attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                         int64_t B, int64_t H, int64_t T, int64_t d, int causal, float scale,
                         hipStream_t stream) {
  bool empty;
  attn_status st = validate(q, k, v, o, lse, B, H, T, d, causal, scale, 4, empty);
  if (st != ATTN_OK || empty) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  return launch<float>(f32_kernel(d, causal), q, k, v, o, lse, B, H, T, scale, stream);
}

const char* attn_status_string(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL: return "null pointer for a non-empty problem";
    case ATTN_ERR_SHAPE: return "B, H or T negative, or sizes exceed the supported limits";
    case ATTN_ERR_UNSUPPORTED: return "unsupported head dimension (d must be 64 or 128)";
    case ATTN_ERR_SCALE: return "scale is not finite";
    case ATTN_ERR_ALIGN: return "q/k/v/o must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_ERR_ARG: return "causal must be 0 or 1 and outputs must not overlap any buffer";
    case ATTN_ERR_DEVICE: return "current device is not an AMD gfx950 GPU";
    case ATTN_ERR_LAUNCH: return "kernel launch failed";
  }
  return "unknown status";
}

const char* attn_kernel_name(int is_f32, int64_t d, int causal) {
  if (d != 64 && d != 128) return nullptr;
  if (causal != 0 && causal != 1) return nullptr;
  static const char* names[2][2][2] = {
      {{"attn_fwd_bf16_d64_full_br128_bc64_w4", "attn_fwd_bf16_d64_causal_br128_bc64_w4"},
       {"attn_fwd_bf16_d128_full_br128_bc64_w4", "attn_fwd_bf16_d128_causal_br128_bc64_w4"}},
      {{"attn_fwd_f32_d64_full_br128_bc32_w4", "attn_fwd_f32_d64_causal_br128_bc32_w4"},
       {"attn_fwd_f32_d128_full_br128_bc32_w4", "attn_fwd_f32_d128_causal_br128_bc32_w4"}}};
  return names[is_f32 ? 1 : 0][d == 128 ? 1 : 0][causal];
}

}  // extern "C"
