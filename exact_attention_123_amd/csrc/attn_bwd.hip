// Backward pass of exact scaled dot-product attention for AMD Instinct
// MI355X (gfx950), behind the C ABI of include/attn.h.
//
// What is computed, per (batch, head), for the forward S = scale Q K^T
// (causal mask optional), P = rowsoftmax(S), O = P V and an upstream
// gradient dO of O:
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - Delta),  Delta_i = dO_i . O_i,
//   dQ = scale dS K,  dK = scale dS^T Q.
// The pages state that this pass recomputes the scores the forward never
// stored rather than reading them back ("Attention Mechanism: Computation &
// Memory Patterns", section 4, "Computational Pattern"; its conclusion): P
// is rebuilt tile by tile from Q, K and the forward's saved log-sum-exp,
// P_ij = exp(S_ij - LSE_i), so no T x T matrix reaches device memory here
// either.
//
// Three kernels, in stream order:
//   1. prep : -Delta_i = -sum_c dO_ic O_ic and the log-sum-exp (as -LSE_i /
//             scale, or -LSE_i log2(e)) per query row, into the caller's
//             workspace.
//   2. dkdv : one workgroup of 8 waves per 256 keys of a head (32 per
//             wave), K of those keys staged in LDS and V held in
//             registers; it walks 64-query tiles of Q and dO (staged in
//             LDS) and accumulates dV^T += dO^T P and dK^T += Q^T dS in
//             registers.  When the 256-key blocks of the problem are fewer
//             than the device's CUs (under the causal mask, than twice the
//             CUs, or at most four times with T <= 4096): 128 keys per
//             workgroup, two waves per 32 keys, each taking one half of
//             every query tile, their sums added at the end.
//   3. dq   : one workgroup per 128 queries (32 per wave), Q and dO in
//             registers; it walks 64-key tiles of K and V (staged in LDS)
//             and accumulates dQ^T += K^T dS^T.  When the 128-query blocks
//             are fewer than twice the CUs (under the causal mask, at most
//             twice): two waves per 32 queries, each taking one half of
//             every key tile.
// dkdv and dq each recompute S and dP for their tiles; neither needs
// atomics or a second pass, and every output element is written by exactly
// one lane (the result does not depend on scheduling).
//
// All four contractions of a tile run on v_mfma_f32_32x32x16_bf16 (fp32
// accumulate).  P and dS are rounded to bf16 (nearest-even) as MFMA
// operands; S, P, dP, dS, Delta and the log-sum-exp stay fp32.

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "attn.h"
#include "device.h"
#include "tiles.h"

namespace {

using namespace attn_tiles;
using attn_internal::check_device;
using attn_internal::device_cus;

constexpr int kThreads = 256;  // 4 waves
constexpr int kWaves = 4;
// dkdv: 8 waves per workgroup, 32 keys per wave (256 keys), or two waves
// per 32 keys (128 keys) for grids of few 256-key blocks (see dkdv_paired)
constexpr int kDkdvWaves = 8;
constexpr int kBK = 32 * kDkdvWaves;  // keys per dkdv workgroup (unpaired)
constexpr int kBQ = 128;       // queries per dq workgroup
constexpr int kTile = 64;      // rows of a staged Q/dO (dkdv) or K/V (dq) tile
// Heads an XCD works on side by side in the dq kernel (see its workgroup
// order): two read as fast as all four of an XCD's heads and fetch half the
// device memory (0.40 against 0.81 GB per call at B H = 32, T = 8192).
constexpr int kHeadsInFlight = 2;

template <int D>
struct BwdTile : RowTile<D> {
  static constexpr int TBYTES = kTile * 2 * D;  // one staged tile
};

// ---------------------------------------------------------------------------
// 1. prep: -Delta_i = -sum_c dO_ic O_ic (fp32) and the row's log-sum-exp in
// the form the kernels start from, one row per D / 8 lanes.  ws[0 .. n) =
// -Delta, ws[n .. 2 n) = -LSE / scale when the scale is folded into the
// score accumulator (see the dK/dV kernel), else -LSE * log2(e); n = B H T.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_prep_kernel(
    const __bf16* __restrict__ O, const __bf16* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ ws, int64_t n, float lse_mult) {
  constexpr int LPR = D / 8;  // lanes per row
  const int64_t row = (int64_t)blockIdx.x * (kThreads / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  float acc = 0.0f;
  if (row < n) {
    const bf16x8_t o = *reinterpret_cast<const bf16x8_t*>(O + row * D + 8 * sub);
    const bf16x8_t g = *reinterpret_cast<const bf16x8_t*>(dO + row * D + 8 * sub);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int m = LPR / 2; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
  if (row < n && sub == 0) {
    ws[row] = -acc;
    ws[n + row] = LSE[row] * lse_mult;
  }
}

// ---------------------------------------------------------------------------
// 2. dkdv
// ---------------------------------------------------------------------------
// FOLD: the score accumulator starts from -LSE_i / scale, so that the
// exponent c (S_ij + v_i) = scale log2(e) S_ij - LSE_i log2(e) needs one
// multiply per element and no per-element row statistic beside the
// accumulator (the dP accumulator likewise starts from -Delta_i).  Used for
// |scale| >= 2^-32, where -LSE / scale is finite; otherwise (scale 0
// included) the exponent is fma(S_ij, c, -LSE_i log2(e)) on a zero-started
// accumulator.  The fp32 error of the folded exponent is about 2^-24
// |LSE log2(e)|, against 2^-9 for the bf16 rounding of P that follows.
//
// 8 waves, two per SIMD (at most 256 registers per lane, so that the
// matrix results stay in VGPRs where the softmax reads them): the block's
// 256 keys are staged in LDS once, each wave holds V of its 32 keys and
// its dK, dV accumulators in registers, and the staged Q and dO tiles serve
// all 256 keys.  PAIR (128 keys, two waves per 32 keys) for problems with
// few 256-key blocks (see dkdv_paired): there the heaviest block's walk over
// every query tile sets the time; a 128-key block halves the walk and the
// pair's split of every tile halves each wave's share again.  Measured on MI355X
// (us per call of the whole backward, paired / 4 waves of 32 keys per
// 128-key block, dQ likewise paired / not): B H = 8, T = 2048, causal,
// d = 64 65.0 / 83.0, d = 128 99.9 / 119.9; no mask, d = 64 64.2 / 82.7;
// B H = 8, T = 4096, d = 128 199.8 / 225.0.
template <int D, bool CAUSAL, bool FOLD, bool PAIR>
__global__ __launch_bounds__(64 * kDkdvWaves, 1) void attn_bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ ws, __bf16* __restrict__ dK,
    __bf16* __restrict__ dV, int T, int BHkv, int G, int nkb, float c, float scale) {
  using C = BwdTile<D>;
  constexpr int NDS = C::NDS, NDT = C::NDT, RB = C::RB;
  constexpr int NW = kDkdvWaves;
  constexpr int BK = PAIR ? 16 * NW : 32 * NW;  // keys per workgroup

  // Two stages, each operand and stage its own object: the compiler then
  // tells the direct-to-LDS loads into one stage from the reads of the
  // other and does not wait for the loads in flight before reading.  The
  // stages must lie below 64 KiB, where their fixed offsets fit the LDS
  // instructions' immediate field: aligned to their own size, they are laid
  // out ahead of the block's keys (the layout orders by alignment) at no
  // cost in padding.
  __shared__ __attribute__((aligned(C::TBYTES))) char sQ0[C::TBYTES];
  __shared__ __attribute__((aligned(C::TBYTES))) char sQ1[C::TBYTES];
  __shared__ __attribute__((aligned(C::TBYTES))) char sG0[C::TBYTES];  // dO
  __shared__ __attribute__((aligned(C::TBYTES))) char sG1[C::TBYTES];
  __shared__ __attribute__((aligned(16))) float sL0[kTile];       // LSE statistic
  __shared__ __attribute__((aligned(16))) float sL1[kTile];
  __shared__ __attribute__((aligned(16))) float sD0[kTile];       // -Delta
  __shared__ __attribute__((aligned(16))) float sD1[kTile];
  __shared__ __attribute__((aligned(1024))) char sK[BK * RB];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, h = lane >> 5;
  // Workgroups are dispatched round-robin over the 8 XCDs (id % 8), each
  // with its own L2.  When the key/value heads split evenly over the XCDs,
  // XCD x takes its heads x, x + 8, ... one after the other, each head's key
  // blocks heavy-first (under a causal mask the first key blocks see the
  // most query tiles), and consecutive heads of an XCD walk their query
  // tiles in opposite directions (`up`).  A CU that finishes the lightest
  // block of one head then takes the next head's heaviest, so the CUs pair
  // blocks kb and nkb - 1 - kb (equal work), and the blocks of a head that
  // run side by side read the same Q and dO tile at the same time and share
  // it in L2.  Otherwise ids walk all heads within each key block.
  const int id = blockIdx.x;
  int kb, bhkv;
  bool up = false;
  if (BHkv % 8 == 0) {
    const int r = id / 8;
    kb = r % nkb;
    bhkv = id % 8 + 8 * (r / nkb);
    up = (r / nkb) & 1;
  } else {
    kb = id / BHkv;
    bhkv = id % BHkv;
  }
  const size_t head = (size_t)bhkv * (size_t)T * D;
  // Waves w and w + 4 share a SIMD; they take key groups w and 7 - w (256
  // keys) or w and 3 - w (PAIR: 128 keys, each group's two waves taking
  // the first (w < 4) and the second 32 queries of every staged tile), so
  // that under a causal mask every SIMD skips the same number of sub-tiles
  // on the diagonal.
  const int kg = wave < 4 ? wave : (PAIR ? 7 : 11) - wave;
  const int u_mine = wave >> 2;  // PAIR: the wave's half of each tile
  const int k0 = kb * BK, kw0 = k0 + 32 * kg;
  const int64_t n = (int64_t)BHkv * G * T;

  // The block's keys, rows k0 .. k0 + BK - 1 (rows >= T read as zero).
  {
    TileDma<D, BK, NW> kdma;
    kdma.init(wave, lane);
    kdma.load(sK, K + head, T, k0, wave);
  }
  // V of the wave's 32 keys: B operand [d][key] of dP = dO V^T; lane (j, h)
  // holds row kw0 + j, d = 16 s + 8 h .. + 8.
  bf16x8_t vf[NDS];
  {
    const __amdgpu_buffer_rsrc_t rV = make_rsrc(V + head, T * RB);
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      vf[s] = __builtin_bit_cast(bf16x8_t, buf_load16(rV, (kw0 + j) * RB + (16 * s + 8 * h) * 2));
  }
  // K of the same keys from LDS, as the B operand [d][key] of S = Q K^T:
  // lane (j, h) reads row 32 kg + j, chunk 2 s + h (swizzled).
  const char* tk = sK + 32 * kg * RB;
  int kaddr[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) kaddr[s] = j * RB + 16 * ((2 * s + h) ^ swz<D>(j));

  TileAddr<D> ad;
  ad.init(lane);
  TileDma<D, kTile, NW> dma;
  dma.init(wave, lane);
  // Query tile `qt` of member `m` of the group (query head bhkv G + m):
  // part 0 its Q rows, part 1 its dO rows and row statistics, part 2 all.
  // Row statistics: one dword per lane of wave 0 (LSE) and wave 1 (-Delta),
  // lane L landing at 4 L; rows >= T read as zero.
  auto stage = [&](char* tq, char* tg, float* tl, float* td, int m, int qt, int part)
      __attribute__((always_inline)) {
    const size_t bhq = (size_t)bhkv * G + m;
    const size_t qhead = bhq * (size_t)T * D;
    const int row0 = qt * kTile;
    if (part != 1) dma.load(tq, Q + qhead, T, row0, wave);
    if (part == 0) return;
    dma.load(tg, dO + qhead, T, row0, wave);
    if (wave < 2) {
      const float* src = ws + (wave == 0 ? n : 0) + bhq * T + row0;
      const __amdgpu_buffer_rsrc_t r = make_rsrc(src, max(T - row0, 0) * 4);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(wave == 0 ? tl : td), 4,
                                               lane * 4, 0, 0, 0);
    }
  };

  f32x16_t dk[NDT], dv[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    dk[dt] = f32x16_t{};
    dv[dt] = f32x16_t{};
  }

  // The walk: for each of the G query heads of the group, the query tiles
  // from the last one down to the block's first visible one.  Every key
  // block of a head starts at the last tile, so the workgroups of a head
  // that run side by side (one XCD) read the same Q and dO tile at the same
  // time and share it in that XCD's L2; walking up from each block's own
  // first tile, they would read different tiles at every step.
  const int qt0 = CAUSAL ? k0 / kTile : 0;
  const int nqt = (T + kTile - 1) / kTile;
  const int per = nqt - qt0;  // > 0: k0 < T
  const int nit = G * per;
  // query tile at position r of a member's walk
  auto qt_at = [&](int r) __attribute__((always_inline)) {
    return up ? qt0 + r : nqt - 1 - r;
  };
  // Query tile qt, staged in (tq, tg, tl, td).  When st is set, the next
  // tile's loads (member nm, tile nq_t, into (nq, ng, nl, nd)) are issued
  // half before each sub-tile, rather than all at once when the waves leave
  // the barrier.
  auto tile = [&](const char* tq, const char* tg, const float* tl, const float* td, int qt,
                  bool st, char* nq, char* ng, float* nl, float* nd, int nm, int nq_t)
      __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int i0 = qt * kTile + 32 * u;
      if (st) stage(nq, ng, nl, nd, nm, nq_t, u);
      __builtin_amdgcn_sched_barrier(0);
      if (PAIR && u != u_mine) continue;
      // Nothing to add when every query of the sub-tile precedes every key
      // of the wave (causal) or lies past the end of the sequence (its Q
      // and dO rows read as zero).  Without a branch here the non-causal
      // kernels need more registers than they have and spill.
      if (CAUSAL ? i0 + 31 < kw0 : i0 >= T) continue;
      // Register 8 a + e of lane (j, h) holds query i0 + 16 a + 8 h + e and
      // key kw0 + j.  The accumulators start from the row statistics: dP
      // from -Delta, S from -LSE / scale (FOLD) or zero.
      f32x16_t S, dP;
      float p[16];
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int q8 = 32 * u + 16 * a + 8 * h;
        const f32x4_t d0 = *reinterpret_cast<const f32x4_t*>(&td[q8]);
        const f32x4_t d1 = *reinterpret_cast<const f32x4_t*>(&td[q8 + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          dP[8 * a + e] = d0[e];
          dP[8 * a + 4 + e] = d1[e];
        }
        if constexpr (FOLD) {
          const f32x4_t l0 = *reinterpret_cast<const f32x4_t*>(&tl[q8]);
          const f32x4_t l1 = *reinterpret_cast<const f32x4_t*>(&tl[q8 + 4]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            S[8 * a + e] = l0[e];
            S[8 * a + 4 + e] = l1[e];
          }
        }
      }
      if constexpr (!FOLD) S = f32x16_t{};
      // S before dP, so that the exponentials of S overlap dP's MFMAs
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row(tq, 32 * u * RB + ad.row[s]),
                                                    lds_row(tk, kaddr[s]), S, 0, 0, 0);
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row(tg, 32 * u * RB + ad.row[s]), vf[s],
                                                     dP, 0, 0, 0);
      if constexpr (FOLD) {
#pragma unroll
        for (int r = 0; r < 16; ++r) p[r] = exp2_hw(S[r] * c);
      } else {
#pragma unroll
        for (int a = 0; a < 2; ++a) {
          const int q8 = 32 * u + 16 * a + 8 * h;
          const f32x4_t l0 = *reinterpret_cast<const f32x4_t*>(&tl[q8]);
          const f32x4_t l1 = *reinterpret_cast<const f32x4_t*>(&tl[q8 + 4]);
#pragma unroll
          for (int e = 0; e < 8; ++e)
            p[8 * a + e] = exp2_hw(fmaf(S[8 * a + e], c, e < 4 ? l0[e] : l1[e - 4]));
        }
      }
      // The mask (keys past the end of the sequence, and causal keys after
      // the query) only on sub-tiles that need it: the empty asm keeps this
      // a branch; as a select the compiler would apply it to every tile.
      if ((CAUSAL && i0 < kw0 + 31) || kw0 + 31 >= T) {
        asm volatile("" ::: "memory");
        // key kw0 + j is masked for query i0 + 16 a + 8 h + e iff
        // 16 a + e < lim (every query when the key is past the end)
        const int key = kw0 + j;
        const int lim = key >= T ? 64 : (CAUSAL ? key - i0 - 8 * h : -1);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * (r >> 3) + (r & 7) < lim) p[r] = 0.0f;
      }
      bf16x8_t pb[2], db[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[a][e] = (__bf16)p[8 * a + e];
          db[a][e] = (__bf16)(p[8 * a + e] * dP[8 * a + e]);
        }
      // dV^T += dO^T P, then dK^T += Q^T dS, over the sub-tile's 32 queries
      // (dS is formed while the dV MFMAs run)
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int ro = (32 * u + 16 * a) * RB;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_tr(tg, ro + ad.tr[0][dt], ro + ad.tr[1][dt]), pb[a], dv[dt], 0, 0, 0);
      }
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int ro = (32 * u + 16 * a) * RB;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_tr(tq, ro + ad.tr[0][dt], ro + ad.tr[1][dt]), db[a], dk[dt], 0, 0, 0);
      }
      // one sub-tile at a time: bounds the registers live at once
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  stage(sQ0, sG0, sL0, sD0, 0, qt_at(0), 2);
  __syncthreads();
  // Two tiles per trip, alternating the stages: the loads of the next tile
  // run while this one is computed; the barrier after each tile waits for
  // them (and frees the stage just read).  No instruction is scheduled
  // across the tiles (sched_barrier), which keeps the register pressure of
  // one tile.  (r, m): walk position and member of the tile computed, and
  // (rn, mn) of the next one, advanced without divisions.
  int r = 0, m = 0;
  for (int it = 0; it < nit; it += 2) {
    int rn = r + 1, mn = m;
    if (rn == per) rn = 0, ++mn;
    ATTN_DEBUG_SYNC();
    tile(sQ0, sG0, sL0, sD0, qt_at(r), it + 1 < nit, sQ1, sG1, sL1, sD1, mn, qt_at(rn));
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (it + 1 >= nit) break;
    r = rn, m = mn;
    if (++rn == per) rn = 0, ++mn;
    ATTN_DEBUG_SYNC();
    tile(sQ1, sG1, sL1, sD1, qt_at(r), it + 2 < nit, sQ0, sG0, sL0, sD0, mn, qt_at(rn));
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    r = rn, m = mn;
  }

  if constexpr (PAIR) {
    // The two waves of a key group add their sums, the second half's into
    // the first's (a fixed order), through the stages, which every wave is
    // done with (the walk ends at a barrier): one stage of 64 lanes x 16 NDT
    // floats per group, dK then dV.
    static_assert(C::TBYTES == NDT * 16 * 64 * 4, "merge buffer");
    float* buf = reinterpret_cast<float*>(kg == 0 ? sQ0 : kg == 1 ? sQ1 : kg == 2 ? sG0 : sG1);
    auto merge = [&](f32x16_t (&acc)[NDT]) __attribute__((always_inline)) {
      if (u_mine == 1) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) buf[(16 * dt + r) * 64 + lane] = acc[dt][r];
      }
      __syncthreads();
      if (u_mine == 0) {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[dt][r] += buf[(16 * dt + r) * 64 + lane];
      }
      __syncthreads();
    };
    merge(dk);
    merge(dv);
    if (u_mine == 1) return;
  }
  store_rows<D>(dK + head, dk, scale, kw0 + j, T, h);
  store_rows<D>(dV + head, dv, 1.0f, kw0 + j, T, h);
}

// ---------------------------------------------------------------------------
// 3. dq
// ---------------------------------------------------------------------------
// PAIR: 8 waves, two per 32 queries, taking the first (waves 0-3) and the
// second 32 keys of every staged tile; for grids of fewer workgroups than
// twice the CUs, where the heaviest block's walk over every key tile sets
// the time.
template <int D, bool CAUSAL, bool PAIR>
__global__ __launch_bounds__(PAIR ? 2 * kThreads : kThreads, PAIR ? 1 : 2) void
attn_bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                   const __bf16* __restrict__ V, const __bf16* __restrict__ dO,
                   const float* __restrict__ ws, __bf16* __restrict__ dQ, int T, int BH, int nqb,
                   int G, float c, float cw, float scale) {
  using C = BwdTile<D>;
  constexpr int NDS = C::NDS, NDT = C::NDT, RB = C::RB;
  constexpr int NW = PAIR ? 2 * kWaves : kWaves;

  // Two stages, each operand and stage its own object (see the dK/dV kernel).
  __shared__ __attribute__((aligned(1024))) char sK0[C::TBYTES];
  __shared__ __attribute__((aligned(1024))) char sK1[C::TBYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[C::TBYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[C::TBYTES];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave & (kWaves - 1);  // the wave's 32 queries
  const int u_mine = wave >> 2;        // PAIR: the wave's half of each tile
  const int j = lane & 31, h = lane >> 5;
  // Heavy-first: the last query blocks see the most key tiles.  Head slot
  // hid is member hid / NKV of key/value group hid % NKV, so that the query
  // heads of one group share an XCD (as in the forward).  When the head
  // slots split evenly over the 8 XCDs (dispatch is round-robin, id % 8) in
  // groups of kHeadsInFlight, XCD x takes its slots x, x + 8, ... in such
  // groups, so that its CUs walk the K and V tiles of few heads at a time
  // and share them in L2; otherwise ids walk all heads within each block
  // index.
  const int id = blockIdx.x;
  int qb, hid;
  if (BH % (8 * kHeadsInFlight) == 0) {
    const int r = id / 8, s = r % (kHeadsInFlight * nqb);
    qb = nqb - 1 - s / kHeadsInFlight;
    hid = id % 8 + 8 * (kHeadsInFlight * (r / (kHeadsInFlight * nqb)) + s % kHeadsInFlight);
  } else {
    qb = nqb - 1 - id / BH;
    hid = id % BH;
  }
  const int nkv = BH / G, bhkv = hid % nkv, bh = bhkv * G + hid / nkv;
  const size_t head = (size_t)bh * (size_t)T * D;
  const size_t kvhead = (size_t)bhkv * (size_t)T * D;
  const int q0 = qb * kBQ, qw0 = q0 + 32 * rg, qg = qw0 + j;
  const int64_t n = (int64_t)BH * T;

  // Q and dO of the wave's 32 queries: B operands [d][query] of S^T = K Q^T
  // and dP^T = V dO^T.
  bf16x8_t qf[NDS], gf[NDS];
  {
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Q + head, T * RB);
    const __amdgpu_buffer_rsrc_t rG = make_rsrc(dO + head, T * RB);
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      qf[s] = __builtin_bit_cast(bf16x8_t, buf_load16(rQ, qg * RB + (16 * s + 8 * h) * 2));
      gf[s] = __builtin_bit_cast(bf16x8_t, buf_load16(rG, qg * RB + (16 * s + 8 * h) * 2));
    }
  }
  // -Delta and -LSE log2(e) of the lane's query (cw: the factor that turns
  // the workspace's form of the log-sum-exp into the latter)
  const float nd = qg < T ? ws[(size_t)bh * T + qg] : 0.0f;
  const float nl = qg < T ? cw * ws[n + (size_t)bh * T + qg] : 0.0f;
  // Every dP^T accumulator starts from -Delta of the lane's query, so that
  // dP - Delta comes out of the contraction (16 registers held throughout;
  // the non-causal d = 128 kernel has none to spare and subtracts instead).
  constexpr bool kFoldDelta = CAUSAL || D == 64;
  f32x16_t dP0;
#pragma unroll
  for (int r = 0; r < 16; ++r) dP0[r] = kFoldDelta ? nd : 0.0f;

  TileAddr<D> ad;
  ad.init(lane);
  TileDma<D, kTile, NW> dma;
  dma.init(wave, lane);
  auto stage = [&](char* tk, char* tv, int t) __attribute__((always_inline)) {
    dma.load(tk, K + kvhead, T, t * kTile, wave);
    dma.load(tv, V + kvhead, T, t * kTile, wave);
  };

  f32x16_t dq[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) dq[dt] = f32x16_t{};

  const int kv_end = CAUSAL ? min(T, q0 + kBQ) : T;
  const int nkt = (kv_end + kTile - 1) / kTile;
  // Key tile t, staged in (tk, tv).
  auto tile = [&](const char* tk, const char* tv, int t) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int kv0 = t * kTile + 32 * u;
      if (PAIR && u != u_mine) continue;
      // every key of the sub-tile follows every query of the wave
      if (CAUSAL && kv0 > qw0 + 31) continue;
      f32x16_t S = f32x16_t{}, dP = dP0;
      // S^T before dP^T, so that the exponentials overlap dP^T's MFMAs
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        S = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row(tk, 32 * u * RB + ad.row[s]), qf[s],
                                                    S, 0, 0, 0);
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        dP = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_row(tv, 32 * u * RB + ad.row[s]), gf[s],
                                                     dP, 0, 0, 0);
      // Register 8 a + e of lane (j, h) holds key kv0 + 16 a + 8 h + e and
      // query qg.
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = exp2_hw(fmaf(S[r], c, nl));
      // The mask only on sub-tiles that need it (a branch, as in the dK/dV
      // kernel): key kv0 + 16 a + 8 h + e is masked iff 16 a + e >= lim.
      if ((CAUSAL && kv0 + 31 > qw0) || kv0 + 31 >= T) {
        asm volatile("" ::: "memory");
        const int lim = min(T, CAUSAL ? qg + 1 : T) - kv0 - 8 * h;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (16 * (r >> 3) + (r & 7) >= lim) p[r] = 0.0f;
      }
      bf16x8_t db[2];
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          db[a][e] = (__bf16)(p[8 * a + e] * (kFoldDelta ? dP[8 * a + e] : dP[8 * a + e] + nd));
      // dQ^T += K^T dS^T over the sub-tile's 32 keys.
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        const int ro = (32 * u + 16 * a) * RB;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          dq[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              lds_tr(tk, ro + ad.tr[0][dt], ro + ad.tr[1][dt]), db[a], dq[dt], 0, 0, 0);
      }
      // one sub-tile at a time: bounds the registers live at once
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  if (nkt > 0) stage(sK0, sV0, 0);
  __syncthreads();
  // Two tiles per trip, alternating the stages (see the dK/dV kernel).
  for (int t = 0; t < nkt; t += 2) {
    if (t + 1 < nkt) stage(sK1, sV1, t + 1);
    ATTN_DEBUG_SYNC();
    tile(sK0, sV0, t);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
    if (t + 1 >= nkt) break;
    if (t + 2 < nkt) stage(sK0, sV0, t + 2);
    ATTN_DEBUG_SYNC();
    tile(sK1, sV1, t + 1);
    __syncthreads();
    __builtin_amdgcn_sched_barrier(0);
  }

  if constexpr (PAIR) {
    // The two waves of 32 queries add their sums, the second half's into
    // the first's (a fixed order), through the stages, which every wave is
    // done with (the walk ends at a barrier): one stage of 64 lanes x 16 NDT
    // floats per query group.
    static_assert(C::TBYTES == NDT * 16 * 64 * 4, "merge buffer");
    float* buf = reinterpret_cast<float*>(rg == 0 ? sK0 : rg == 1 ? sK1 : rg == 2 ? sV0 : sV1);
    if (u_mine == 1) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) buf[(16 * dt + r) * 64 + lane] = dq[dt][r];
    }
    __syncthreads();
    if (u_mine == 1) return;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) dq[dt][r] += buf[(16 * dt + r) * 64 + lane];
  }
  store_rows<D>(dQ + head, dq, scale, qg, T, h);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int64_t kMaxHeadBytes = (int64_t(1) << 31) - 1;

bool overlaps(const void* a, int64_t na, const void* b, int64_t nb) {
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

template <int D, bool FOLD, bool PAIR>
const void* dkdv_kernel(int causal) {
  return causal ? (const void*)attn_bwd_dkdv_kernel<D, true, FOLD, PAIR>
                : (const void*)attn_bwd_dkdv_kernel<D, false, FOLD, PAIR>;
}
template <int D, bool PAIR>
const void* dkdv_kernel(int causal, bool fold) {
  return fold ? dkdv_kernel<D, true, PAIR>(causal) : dkdv_kernel<D, false, PAIR>(causal);
}
template <int D>
const void* dkdv_kernel(int causal, bool fold, bool pair) {
  return pair ? dkdv_kernel<D, true>(causal, fold) : dkdv_kernel<D, false>(causal, fold);
}

// Paired waves (128 keys per workgroup, two waves per 32 keys) when the
// 256-key blocks of all key/value heads are fewer than the CUs, or, under
// the causal mask, fewer than twice the CUs: there the heaviest block's
// walk over every query tile sets the time (under the mask the first block
// of a head walks every tile, the last one a few, and one or two rounds of
// blocks cannot even that out), and a 128-key block with the tiles' halves
// split between two waves shortens each wave's walk to a quarter.
// Measured on MI355X (us per call of the backward, causal, d = 128; paired
// below 2 / below 1 CU count): 32 query over 8 key/value heads, T = 8192
// (256 blocks, each walking 4 query heads) 1655.8 / 2109.3; B H = 8,
// T = 8192 492.5 / 595.1; B H = 48, T = 2048 (384 blocks) 231.1 / 245.8;
// B H = 12, T = 8192 678.6 / 686.3; 512 blocks (B H = 16, T = 8192) the
// same; unmasked, 256 blocks (32 over 8 heads, T = 8192) 3329 against 3235
// paired, so without the mask only grids below the CU count pair (pairing
// costs 4-7% where the blocks are equal: more Q/dO staging per FLOP; B H =
// 64, T = 4096 1734.6 / 1616.0, B H = 32, T = 4096, d = 64 483.1 / 462.3).
// Under the mask short sequences (T <= 4096, walks of at most 64 query
// tiles, where the finer blocks even out the unequal causal work by more
// than the pairing costs) pair up to four times the CU count: B H = 32, T = 4096 459.4 / 513.2 (d = 128), 276.3 / 321.0
// (d = 64); B H = 64, T = 2048 286.0 / 303.8 and 178.2 / 190.8; B H = 48,
// T = 4096 696.0 / 719.9 and 395.6 / 424.4; B H = 64, T = 4096 (1024
// blocks) 920.7 / 935.1 and 518.7 / 551.0; B H = 128, T = 2048 570.5 /
// 559.7 and 320.2 / 332.4.  Longer sequences keep the larger blocks: the
// T = 8192 workload (1024 blocks) 1740.7 paired / 1666.1, B H = 8,
// T = 65536 25103 / 24216, B H = 16, T = 8192 (512 blocks) 847.3 / 823.4.
bool dkdv_paired(int64_t BHkv, int64_t T, int causal) {
  const int64_t blocks = BHkv * ((T + kBK - 1) / kBK), cus = device_cus();
  if (!causal) return blocks < cus;
  return blocks < 2 * cus || (T <= 4096 && blocks <= 4 * cus);
}
template <int D, bool PAIR>
const void* dq_kernel(int causal) {
  return causal ? (const void*)attn_bwd_dq_kernel<D, true, PAIR>
                : (const void*)attn_bwd_dq_kernel<D, false, PAIR>;
}
template <int D>
const void* dq_kernel(int causal, bool pair) {
  return pair ? dq_kernel<D, true>(causal) : dq_kernel<D, false>(causal);
}

// Paired waves in the dQ kernel (8 per 128 queries) when its 128-query
// blocks are fewer than twice the CUs (the unpaired kernel's two
// workgroups per CU), or, under the causal mask, exactly twice as many (one
// round whose blocks the mask makes unequal).  Measured on MI355X (us per
// call of the backward, paired below 2 / 1 CU count): B H = 16, T = 2048,
// causal, d = 64 65.9 / 70.8, d = 128 103.5 / 111.7; B H = 8, T = 4096,
// d = 128 183.7 / 201.4; B H = 24, T = 2048, d = 128 131.7 / 140.2; at 512
// blocks, causal (paired / not): B H = 32, T = 2048, d = 128 163.0 / 177.5,
// d = 64 98.8 / 109.0; B H = 8, T = 8192 444.5 / 480.4; at 768 the same.
bool dq_paired(int64_t BH, int64_t T, int causal) {
  return BH * ((T + kBQ - 1) / kBQ) < 2 * device_cus() + (causal ? 1 : 0);
}

}  // namespace

extern "C" {

attn_status attn_bwd_gqa(const void* q, const void* k, const void* v, const void* o,
                         const void* dout, const float* lse, void* dq, void* dk, void* dv,
                         float* ws, int64_t B, int64_t H, int64_t H_kv, int64_t T, int64_t d,
                         int causal, float scale, hipStream_t stream) {
  if (B < 0 || H < 0 || T < 0 || H_kv < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  if ((H_kv == 0) != (H == 0) || (H_kv > 0 && H % H_kv != 0)) return ATTN_ERR_SHAPE;
  if (B == 0 || H == 0 || T == 0) return ATTN_OK;
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !ws) return ATTN_ERR_NULL;
  if ((T + 256) * d * 2 > kMaxHeadBytes) return ATTN_ERR_SHAPE;
  if (B > (int64_t(1) << 31) / H) return ATTN_ERR_SHAPE;
  const int64_t BH = B * H, BHkv = B * H_kv;
  const int64_t nblk = (T + 127) / 128;
  if (BH > INT32_MAX / nblk) return ATTN_ERR_SHAPE;
  if (BH > (INT64_MAX / 8) / (T * d * 2)) return ATTN_ERR_SHAPE;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)o | (uintptr_t)dout |
       (uintptr_t)dq | (uintptr_t)dk | (uintptr_t)dv) & 15u)
    return ATTN_ERR_ALIGN;
  if (((uintptr_t)lse | (uintptr_t)ws) & 3u) return ATTN_ERR_ALIGN;
  const int64_t nb = BH * T * d * 2, kb = BHkv * T * d * 2, lb = BH * T * 4, wb = 2 * lb;
  const void* ins[6] = {q, k, v, o, dout, lse};
  const int64_t in_bytes[6] = {nb, kb, kb, nb, nb, lb};
  void* outs[4] = {dq, dk, dv, ws};
  const int64_t out_bytes[4] = {nb, kb, kb, wb};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlaps(outs[a], out_bytes[a], ins[b], in_bytes[b])) return ATTN_ERR_ARG;
    for (int b = a + 1; b < 4; ++b)
      if (overlaps(outs[a], out_bytes[a], outs[b], out_bytes[b])) return ATTN_ERR_ARG;
  }
  attn_status st = check_device();
  if (st != ATTN_OK) return st;

  const int t = (int)T, bh = (int)BH, bhkv = (int)BHkv, g = (int)(H / H_kv);
  const int64_t n = BH * T;
  const float c = scale * kLog2e;
  // Fold the scale into the dK/dV kernel's score accumulator where
  // -LSE / scale stays finite (see attn_bwd_dkdv_kernel).
  const bool fold = std::fabs(scale) >= 0x1p-32f;
  const float lse_mult = fold ? -1.0f / scale : -kLog2e;
  const float cw = fold ? c : 1.0f;
  {
    const int rows_per_block = kThreads / (int)(d / 8);
    const dim3 grid((unsigned)((n + rows_per_block - 1) / rows_per_block));
    const __bf16* ob = (const __bf16*)o;
    const __bf16* gb = (const __bf16*)dout;
    void* args[] = {(void*)&ob, (void*)&gb, (void*)&lse, (void*)&ws, (void*)&n,
                    (void*)&lse_mult};
    const void* kern = d == 64 ? (const void*)attn_bwd_prep_kernel<64>
                               : (const void*)attn_bwd_prep_kernel<128>;
    if (hipLaunchKernel(kern, grid, dim3(kThreads), args, 0, stream) != hipSuccess)
      return ATTN_ERR_LAUNCH;
  }
  const __bf16 *qb = (const __bf16*)q, *kb_ = (const __bf16*)k, *vb = (const __bf16*)v,
               *gb = (const __bf16*)dout;
  const float* wsc = ws;
  {
    const bool pair = dkdv_paired(BHkv, T, causal);
    const int bk = pair ? kBK / 2 : kBK;
    int nkb = (int)((T + bk - 1) / bk);
    __bf16 *dkb = (__bf16*)dk, *dvb = (__bf16*)dv;
    void* args[] = {(void*)&qb,  (void*)&kb_, (void*)&vb, (void*)&gb,  (void*)&wsc,
                    (void*)&dkb, (void*)&dvb, (void*)&t,  (void*)&bhkv, (void*)&g,
                    (void*)&nkb, (void*)&c,   (void*)&scale};
    const void* kern =
        d == 64 ? dkdv_kernel<64>(causal, fold, pair) : dkdv_kernel<128>(causal, fold, pair);
    if (hipLaunchKernel(kern, dim3((unsigned)(bhkv * nkb)), dim3(64 * kDkdvWaves), args, 0,
                        stream) !=
        hipSuccess)
      return ATTN_ERR_LAUNCH;
  }
  {
    int nqb = (int)((T + kBQ - 1) / kBQ);
    __bf16* dqb = (__bf16*)dq;
    void* args[] = {(void*)&qb, (void*)&kb_, (void*)&vb,  (void*)&gb, (void*)&wsc,
                    (void*)&dqb, (void*)&t,  (void*)&bh,  (void*)&nqb, (void*)&g,
                    (void*)&c,  (void*)&cw, (void*)&scale};
    const bool pair = dq_paired(BH, T, causal);
    const void* kern = d == 64 ? dq_kernel<64>(causal, pair) : dq_kernel<128>(causal, pair);
    if (hipLaunchKernel(kern, dim3((unsigned)(bh * nqb)), dim3(pair ? 2 * kThreads : kThreads),
                        args, 0, stream) != hipSuccess)
      return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o,
                     const void* dout, const float* lse, void* dq, void* dk, void* dv, float* ws,
                     int64_t B, int64_t H, int64_t T, int64_t d, int causal, float scale,
                     hipStream_t stream) {
  return attn_bwd_gqa(q, k, v, o, dout, lse, dq, dk, dv, ws, B, H, H, T, d, causal, scale,
                      stream);
}

const char* attn_bwd_kernel_name(int64_t d, int causal, int which) {
  if ((d != 64 && d != 128) || (causal != 0 && causal != 1) || which < 0 || which > 2)
    return nullptr;
  static const char* names[2][2][3] = {
      {{"attn_bwd_prep_d64", "attn_bwd_dkdv_bf16_d64_full_bk256_bq64_w8",
        "attn_bwd_dq_bf16_d64_full_bq128_bk64_w4"},
       {"attn_bwd_prep_d64", "attn_bwd_dkdv_bf16_d64_causal_bk256_bq64_w8",
        "attn_bwd_dq_bf16_d64_causal_bq128_bk64_w4"}},
      {{"attn_bwd_prep_d128", "attn_bwd_dkdv_bf16_d128_full_bk256_bq64_w8",
        "attn_bwd_dq_bf16_d128_full_bq128_bk64_w4"},
       {"attn_bwd_prep_d128", "attn_bwd_dkdv_bf16_d128_causal_bk256_bq64_w8",
        "attn_bwd_dq_bf16_d128_causal_bq128_bk64_w4"}}};
  return names[d == 128 ? 1 : 0][causal][which];
}

const char* attn_bwd_kernel_name_for(int64_t B, int64_t H, int64_t H_kv, int64_t T, int64_t d,
                                     int causal, int which) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || T <= 0 || H % H_kv != 0) return nullptr;
  const char* name = attn_bwd_kernel_name(d, causal, which);
  if (name == nullptr || check_device() != ATTN_OK) return nullptr;
  if (which == 1 && dkdv_paired(B * H_kv, T, causal)) {
    static const char* small[2][2] = {
        {"attn_bwd_dkdv_bf16_d64_full_bk128_bq64_w8",
         "attn_bwd_dkdv_bf16_d64_causal_bk128_bq64_w8"},
        {"attn_bwd_dkdv_bf16_d128_full_bk128_bq64_w8",
         "attn_bwd_dkdv_bf16_d128_causal_bk128_bq64_w8"}};
    return small[d == 128 ? 1 : 0][causal];
  }
  if (which == 2 && dq_paired(B * H, T, causal)) {
    static const char* small[2][2] = {
        {"attn_bwd_dq_bf16_d64_full_bq128_bk64_w8", "attn_bwd_dq_bf16_d64_causal_bq128_bk64_w8"},
        {"attn_bwd_dq_bf16_d128_full_bq128_bk64_w8",
         "attn_bwd_dq_bf16_d128_causal_bq128_bk64_w8"}};
    return small[d == 128 ? 1 : 0][causal];
  }
  return name;
}

}  // extern "C"
