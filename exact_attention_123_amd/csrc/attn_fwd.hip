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
// into LDS, ahead of its use (bf16: three stages, direct-to-LDS; fp32: two
// stages through registers), and read from LDS by all waves of the
// workgroup.
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

#include <cmath>
#include <cstdint>
#include <cstring>
#include <type_traits>

#include "attn.h"
#include "device.h"
#include "fwd_cache.h"
#include "rows.h"
#include "tiles.h"

namespace {

using namespace attn_tiles;
using attn_internal::check_device;
using attn_internal::device_cus;

// fp32 kernel: 4 waves, 128 query rows per workgroup (32 per wave).
constexpr int kThreads = 256;
constexpr int kBR = 128;
// bf16 kernel: 8 waves, 256 query rows per workgroup (32 per wave), or 4
// waves and 128 rows when the 8-wave grid has fewer workgroups than the GPU
// has CUs (see pick_plan, which sends the smallest problems to the
// row-chunk kernel instead).

// Key offset (within a 32-key block) held by accumulator register r of lane
// half h, for the bf16 kernel (K rows fed in attn_tiles::row_perm order, so
// that registers 8a..8a+7 of lane half h hold eight consecutive keys, one
// B-operand slot of the PV MFMA) and the fp32 kernel (plain order).
__host__ __device__ constexpr int acc_key_perm(int r, int h) {
  return 16 * (r / 8) + 8 * h + 4 * ((r / 4) & 1) + (r & 3);
}
__host__ __device__ constexpr int acc_key_plain(int r, int h) {
  return 8 * (r / 4) + 4 * h + (r & 3);
}

// Head slots an XCD works on side by side (see block_coords).  Measured
// on MI355X at B H = 32, T = 8192, causal (us per launch, one box): all four
// of an XCD's heads interleaved 535.5, two at a time 536.3, one at a time
// 549.4 (the heavy blocks of one head end together and leave CUs idle);
// two at a time halves the number of heads whose K and V compete for an
// XCD's L2 at no cost in time.
constexpr int kHeadsInFlight = 2;

// Workgroup id -> (query head bhq, key/value head bhkv, query block qb).
// Workgroups are dispatched round-robin over the 8 XCDs (id % 8), each
// with its own L2.  When the head slots split evenly over the XCDs in
// groups of kHeadsInFlight, XCD x takes its slots x, x + 8, ... in groups
// of kHeadsInFlight, each group's query blocks heavy-first (the highest
// blocks, most key tiles under a causal mask, first) with the group's
// heads alternating; otherwise ids walk all heads within each block index,
// heavy-first.  Either way all blocks of one head run on one XCD and share
// its L2.  With grouped key/value heads (G query heads per key/value head,
// "FlashAttention -- avoid writing the giant intermediate", the closing note
// on grouped-query attention), head slot hid maps to member hid / NKV of
// group hid % NKV, so the G query heads that read one key/value head also
// share an XCD whenever NKV = BH / G is a multiple of 8.  G = 1 is the
// identity.
__device__ __forceinline__ void block_coords(int BH, int nqb, int G, int& bhq, int& bhkv,
                                             int& qb) {
  const int id = blockIdx.x;
  int hid;
  if (BH % (8 * kHeadsInFlight) == 0) {
    const int r = id / 8, s = r % (kHeadsInFlight * nqb);
    qb = nqb - 1 - s / kHeadsInFlight;
    hid = id % 8 + 8 * (kHeadsInFlight * (r / (kHeadsInFlight * nqb)) + s % kHeadsInFlight);
  } else {
    qb = nqb - 1 - id / BH;
    hid = id % BH;
  }
  const int nkv = BH / G;
  bhkv = hid % nkv;
  bhq = bhkv * G + hid / nkv;
}

// Lazy running max of the large-grid bf16 kernel.  Bound on a lane's sum of
// one sub-tile's weights (see
// its softmax): above it the running max is raised.  kRegrow: once some lane
// passed the bound, every row whose sub-tile max exceeds its running max by
// more than this gets the sub-tile max as its new running max (a row that
// reached the bound always does: its largest weight is then above 2^60).
// At 0 each such event brings every row of the wave up to date, which makes
// the next one as late as possible (the event costs the wave the same
// whatever number of rows it raises).
constexpr float kMaxLaneSum = 18446744073709551616.0f;  // 2^64
constexpr float kRegrow = 0.0f;

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

template <int D, int NW_ = 8>
struct Bf16Tile {
  static constexpr int NW = NW_;            // waves per workgroup
  static constexpr int BC = 64;             // keys per tile
  static constexpr int NST = 3;             // LDS stages per operand
  static constexpr int NDS = D / 16;        // 16-wide d steps of the QK MFMA
  static constexpr int NDT = D / 32;        // 32-row d tiles of O^T
  static constexpr int RB = D * 2;          // bytes per row of Q, K, V, O
  static constexpr int NCH = D / 8;         // 16-byte chunks per row
  // K tile in LDS: unpadded rows, the 16-byte chunk c of row r at chunk
  // c ^ attn_tiles::swz<D>(r), which is one-to-one on 16 consecutive rows:
  // the 16 rows that one 16-lane phase of a 128-bit LDS read touches (one
  // chunk each) fall in 16 different bank groups.
  static constexpr int KBYTES = BC * RB;
  static constexpr int KDMA = KBYTES / 1024;  // 1 KiB direct-to-LDS blocks
  static constexpr int KPER = KDMA / NW;      // load instructions per wave
  // V tile in LDS: unpadded rows with an XOR swizzle of the 16-byte chunks
  // (see v_chunk_swizzle), 1 KiB blocks of RPK rows.
  static constexpr int VBYTES = BC * RB;
  static constexpr int VDMA = VBYTES / 1024;
  static constexpr int VPER = VDMA / NW;
  static constexpr int RPK = 1024 / RB;
  static constexpr int RPB = 256 / RB;      // rows per 256-byte bank cycle
  static_assert(KDMA % NW == 0 && VDMA % NW == 0 && VPER <= 4, "tile split");
  static_assert(NST * (KBYTES + VBYTES) <= 160 * 1024, "LDS");
};

// XOR applied to the 16-byte chunk index of V row r.  The transposing LDS
// read of the PV operand makes each half-wave read 4 consecutive rows x 4
// consecutive chunks; flipping chunk bits 2-3 by the row's position within
// 4 rows (counted in 256-byte bank cycles) puts those 16 chunks in 16
// different bank groups.
template <int D>
__host__ __device__ constexpr int v_chunk_swizzle(int r) {
  using C = Bf16Tile<D>;
  return 4 * ((r / C::RPB) % (C::NCH / 4));
}

// Exact sum of the lane's fp32 values in four independent chains.
template <int N>
__device__ __forceinline__ float sum_tree(const float* x) {
  float a = x[0], b = x[1], c = x[2], d = x[3];
#pragma unroll
  for (int i = 4; i < N; i += 4) {
    a += x[i];
    b += x[i + 1];
    c += x[i + 2];
    d += x[i + 3];
  }
  return (a + b) + (c + d);
}

// One wave owns 32 query rows; the workgroup (NWAVES = 8 waves, or 4 for
// grids smaller than the GPU) 32 NWAVES rows of one head.
// Key/value tiles of 64 keys stream through three LDS stages per operand,
// written by direct-to-LDS buffer loads (no staging registers) three tiles
// (K) and two tiles (V) ahead of their use, so a load has two tile periods
// to land.
//
// The online softmax runs on score sub-tiles of 32 keys, software-pipelined
// per wave: while the VALU computes the softmax of sub-tile k, the matrix
// cores compute S_{k+1} = K_{k+1} Q^T and O^T += V_{k-1}^T P_{k-1}^T, all
// in one straight-line block.  The running max is raised lazily (see
// kLazyRescale), so the accumulator rescale is a rare, wave-uniform branch
// between blocks (after P_{k-1} V_{k-1} is in, before P_k V_k).
//
// PRESCALE: multiply the scores by c before the softmax (any sign of c);
// otherwise (c > 0) the multiply is folded into the exponent's fma and the
// max is taken over the raw scores.
template <int D, bool CAUSAL, bool PRESCALE, int NWAVES>
__global__ __launch_bounds__(64 * NWAVES, 1) void attn_fwd_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int T, int Tk, int Tcap, int off, int BH, int nqb, int G,
    float c) {
  using C = Bf16Tile<D, NWAVES>;
  constexpr int BR = 32 * NWAVES;  // query rows per workgroup
  constexpr int NW = C::NW, BC = C::BC, NDS = C::NDS, NDT = C::NDT;
  constexpr int RB = C::RB, NCH = C::NCH;
  constexpr int KPER = C::KPER, VPER = C::VPER, RPK = C::RPK;
  static_assert(BC == 64, "two 32-key score sub-tiles per LDS tile");

  // LDS: three K and three V stages, separate objects so that the compiler
  // can tell the direct-to-LDS writes into one stage from reads of another.
  // The K stages, aligned to their size (no padding), are laid out first
  // (the layout orders by alignment), then the V stages: at d = 128 the
  // second and third V stages start at 64 and 80 KiB, past the 16-bit
  // immediate offset of the LDS instructions (see vhi below).
  __shared__ __attribute__((aligned(C::KBYTES))) char sK0[C::KBYTES];
  __shared__ __attribute__((aligned(C::KBYTES))) char sK1[C::KBYTES];
  __shared__ __attribute__((aligned(C::KBYTES))) char sK2[C::KBYTES];
  __shared__ __attribute__((aligned(1024))) char sV0[C::VBYTES];
  __shared__ __attribute__((aligned(1024))) char sV1[C::VBYTES];
  __shared__ __attribute__((aligned(1024))) char sV2[C::VBYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, h = lane >> 5;
  int bh, bhkv, qb;
  block_coords(BH, nqb, G, bh, bhkv, qb);
  // T query rows per head (Q, O, LSE); Tk keys per key/value head, stored
  // with a row stride of Tcap rows per head; query row i sits at key
  // position i + off (off = 0 for the square forward, Tk - T for new
  // queries appended to a cache).
  const size_t head = (size_t)bh * (size_t)T * D;
  const size_t kvhead = (size_t)bhkv * (size_t)Tcap * D;
  const int head_bytes = T * RB;
  const __bf16* Kh = K + kvhead;
  const __bf16* Vh = V + kvhead;
  const int q0 = qb * BR;
  // Row group of the wave: with 8 waves, waves w and w + 4 share a SIMD,
  // and under a causal mask a row group's work in the block's last
  // (diagonal) tiles grows with its index, so the pair takes groups w and
  // 7 - w.
  const int rg = NW == 8 && wave >= 4 ? 11 - wave : wave;
  const int qg = q0 + rg * 32 + j;
  // Under a causal mask the last score sub-tile (32 keys) with a key visible
  // to some row of the wave is klast = (off + q0 + 32 rg + 31) / 32 (for
  // the square forward q0 / 32 + rg); from iteration tskip on
  // (sub-steps k >= 2 tskip + 1 > klast + 1: nothing left to accumulate)
  // the wave only loads its share of the tiles and joins the barriers.
  const int tskip = CAUSAL ? ((off + q0 + 32 * rg + 31) / 32) / 2 + 1 : INT32_MAX;

  // Q fragment: B operand of S^T = K Q^T; lane (j, h) holds
  // Q[qg][16 s + 8 h .. +8] for every k-step s.  Rows >= T read as zero.
  bf16x8_t qf[NDS];
  {
    const __amdgpu_buffer_rsrc_t rQ = make_rsrc(Q + head, head_bytes);
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      qf[s] = __builtin_bit_cast(bf16x8_t, buf_load16(rQ, qg * RB + (16 * s + 8 * h) * 2));
  }

  const int kv_end = CAUSAL ? min(Tk, off + q0 + BR) : Tk;
  const int ntiles = (kv_end + BC - 1) / BC;
  const int kv_bytes = kv_end * RB;
  // Score sub-tiles (32 keys) below nfs need no mask: every key is < Tk
  // and, when causal, no later than the workgroup's first query.
  const int nfs = (CAUSAL ? min(off + q0 + 1, Tk) : Tk) / 32;

  // Direct-to-LDS loads.  A 1 KiB block is written by one wave instruction,
  // lane L's 16 bytes landing at block offset 16 L; each lane picks the
  // global chunk that belongs there.  K: block b holds rows RPK b ..
  // RPK b + RPK - 1, swizzled; wave w writes blocks w, w + NW, ...
  int koff[KPER];
#pragma unroll
  for (int n = 0; n < KPER; ++n) {
    const int r = RPK * (wave + NW * n) + lane / NCH;
    const int pc = lane % NCH;
    koff[n] = r * RB + 16 * (pc ^ attn_tiles::swz<D>(r));
  }
  // V: wave w writes blocks VPER w .. VPER w + VPER - 1 (block b holds rows
  // RPK b .. RPK b + RPK - 1).
  int voff;
  {
    const int r = RPK * VPER * wave + lane / NCH;
    const int pc = lane % NCH;
    voff = r * RB + 16 * (pc ^ v_chunk_swizzle<D>(r));
  }
  // Both are issued for every tile index, also past the last tile: keys at
  // or past kv_end read as zero without touching memory (the descriptor's
  // size ends there), so the count of loads per wave and tile is fixed.
  auto dma_k = [&](char* buf, int t) __attribute__((always_inline)) {
    const int kv0 = t * BC;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(Kh + (size_t)kv0 * D, max(kv_bytes - kv0 * RB, 0));
#pragma unroll
    for (int n = 0; n < KPER; ++n) {
      // (a plain local: host-side template instantiation drops the kernel
      // when an array element is passed to this builtin directly)
      const int off = koff[n];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void_t*)(buf + 1024 * (wave + NW * n)), 16,
                                               off, 0, 0, 0);
    }
  };
  auto dma_v = [&](char* buf, int t) __attribute__((always_inline)) {
    const int kv0 = t * BC;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(Vh + (size_t)kv0 * D, max(kv_bytes - kv0 * RB, 0));
    // The instruction offset (1024 n) advances both the global and the LDS
    // address; voffset only moves the global one.
    lds_void_t* dst = (lds_void_t*)(buf + 1024 * VPER * wave);
    auto block = [&](auto n) __attribute__((always_inline)) {
      constexpr int N = decltype(n)::value;
      if constexpr (N < VPER)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 1024 * N, 0);
    };
    block(std::integral_constant<int, 0>{});
    block(std::integral_constant<int, 1>{});
    block(std::integral_constant<int, 2>{});
    block(std::integral_constant<int, 3>{});
  };
  // Workgroup barrier for the LDS stages.  __syncthreads() would also wait
  // for every load in flight, including the direct-to-LDS loads of the next
  // stages; this waits only for this wave's LDS reads (lgkmcnt) and keeps the
  // compiler from moving memory accesses across it.  The stage loads that
  // must have landed are waited for explicitly (wait_dma) before it.
  auto stage_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // Waits until at most n of this wave's direct-to-LDS loads are still in
  // flight (they complete in issue order).
  auto wait_dma = [&](auto n) __attribute__((always_inline)) {
    constexpr int N = decltype(n)::value;
    static_assert(N < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0F70 | N);
  };

  // LDS read addresses.  K (A operand of the QK MFMA): lane (j, h) reads row
  // 32 half + perm(j), chunk 2 s + h (stored at chunk (2 s + h) ^ swz; the
  // swizzle has period 16 in the row, so the half adds a plain offset).
  int kaddr[NDS];
  {
    const int r = row_perm(j);
    const int f = attn_tiles::swz<D>(r);
#pragma unroll
    for (int s = 0; s < NDS; ++s) kaddr[s] = r * RB + 16 * ((2 * s + h) ^ f);
  }
  // V (A operand of the PV MFMA, V^T): ds_read_b64_tr_b16 gives lane i of a
  // 16-lane group element (i % 4) of the 8 bytes read by lane 4 e + i / 4 of
  // the group, in slot e.  Lane l of group g reads V[row][d .. d + 3] with
  // row = 8 (g / 2) + l / 4 (+ 16 kc + 4 half) and d = 32 dt + 16 (g % 2) +
  // 4 (l % 4), so lane i of the group receives V[row0 + e][32 dt + 16 (g % 2)
  // + i] for e = 0..3: four consecutive keys of one d, i.e. V^T.  The
  // swizzle only flips chunk bits 2-3, i.e. the dt field, so the address of
  // tile dt is vaddr0 ^ (64 dt).
  int vaddr[NDT];
  {
    const int g = lane >> 4, l = lane & 15;
    const int r = 8 * (g >> 1) + (l >> 2);
    const int ch = 2 * (g & 1) + ((l >> 1) & 1);
    const int vaddr0 = r * RB + 16 * (ch ^ v_chunk_swizzle<D>(r)) + 8 * (l & 1);
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) vaddr[dt] = vaddr0 ^ (64 * dt);
  }
  // For the V stages at 64 KiB and beyond: the same addresses plus 64 KiB,
  // kept opaque, so that a read of such a stage is one register plus an
  // immediate (the stage's offset past 64 KiB); the compiler would otherwise
  // fold the 64 KiB back into the offset and add it on every read.
  int vhi[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) {
    vhi[dt] = vaddr[dt] + 65536;
    asm volatile("" : "+v"(vhi[dt]));
  }

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
  // The running max starts at kMinusHuge (see attn_tiles): the first visible
  // sub-tile always raises it, and masked scores (-inf) give weight 0.
  float m_run = kMinusHuge, l_run = 0.0f, w_run = 0.0f;
  const float cm = PRESCALE ? 1.0f : c;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  // S^T of the 32-key half `half` of the K tile in `kb`.
  auto qk = [&](const char* kb, int half, f32x16_t& sn) __attribute__((always_inline)) {
    sn = f32x16_t{};
    const char* base = kb + half * 32 * RB;
#pragma unroll
    for (int s = 0; s < NDS; ++s) {
      const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(base + kaddr[s]);
      sn = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[s], sn, 0, 0, 0);
    }
  };

  // O^T += V^T P^T for the 32-key half `half` of the V tile in `vb`; HI:
  // the stage lies at 64 KiB or beyond (the address is still formed from the
  // stage, so that the compiler knows which stage a read touches).
  auto pv = [&](auto hi, const char* vb, int half, const bf16x8_t (&pb)[2])
                __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const char* base = decltype(hi)::value ? vb + (vhi[dt] - 65536) : vb + vaddr[dt];
        const int off = (32 * half + 16 * a) * RB;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + off));
        const i16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + off + 4 * RB));
        const bf16x8_t vv = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vv, pb[a], oacc[dt], 0, 0, 0);
      }
  };

  // Online softmax of one 32-key score sub-tile x ("FlashAttention -- avoid
  // writing the giant intermediate", "Tiling and an incremental
  // normalization"; "Attention Mechanism", section 3), in two parts.
  //
  // softmax (every sub-tile, inside the MFMA block): the weights
  // p = exp2(cm x - m) against the current running max m, their bf16
  // rounding pb, the lane's partial sums ls (fp32) and ws (of the bf16
  // weights), and whether any lane of the wave has ls above 2^64.  Below
  // that bound every weight is at most 2^64 and m may stay where it is (the
  // common factor cancels in acc / l): no row max is needed.
  //
  // regrow (only when some lane's sum passed the bound; the workgroup's
  // first sub-tile, where m is still -1e38, goes straight to it): the
  // row max over the sub-tile (the two lane halves holding a query's scores
  // exchange theirs) becomes the running max of the rows whose max outgrew
  // m by more than kRegrow, the accumulator and normalisers of those rows
  // are multiplied by exp2(m_old - m_new), and the weights are recomputed.
  // The decision is per row, so a row's result never depends on other rows.
  auto softmax = [&](const f32x16_t& x, bf16x8_t(&pb)[2], float& ls,
                     float& ws) __attribute__((always_inline)) -> bool {
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = exp2_hw(fmaf(x[r], cm, -m_run));
    ls = sum_tree<16>(p);
    ws = 0.0f;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int u = 0; u < 8; ++u) pb[a][u] = (__bf16)p[8 * a + u];
      // ws sums exactly the bf16 weights the PV MFMA uses, so that O =
      // sum p'v / sum p' is a convex combination of V rows.
      ws = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 0, 1), one2, ws,
                                           false);
      ws = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 2, 3), one2, ws,
                                           false);
      ws = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 4, 5), one2, ws,
                                           false);
      ws = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 6, 7), one2, ws,
                                           false);
    }
    // Keep every softmax instruction in the MFMA block: without this the
    // compiler may sink them past the branch that follows.
    asm volatile("" ::"v"(ls), "v"(ws), "v"(pb[0]), "v"(pb[1]));
    return __builtin_amdgcn_ballot_w64(!(ls <= kMaxLaneSum)) != 0;
  };

  auto rescale = [&](float alpha) __attribute__((always_inline)) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[dt][r] *= alpha;
  };

  // first: the workgroup's first sub-tile, where nothing has been
  // accumulated yet: the row max becomes the running max directly (it stays
  // -1e38 for a row whose scores are all masked) and nothing is rescaled.
  auto regrow = [&](auto first, const f32x16_t& x, bf16x8_t(&pb)[2], float& ls,
                    float& ws) __attribute__((always_inline)) {
    float mx = x[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, x[r]);
    const float mt = pair_max(mx) * cm;
    if constexpr (decltype(first)::value) {
      m_run = mt > m_run ? mt : m_run;
    } else {
      const bool grow = mt > m_run + kRegrow;
      const float alpha = grow ? exp2_hw(m_run - mt) : 1.0f;  // exp2(-huge) = 0
      m_run = grow ? mt : m_run;
      l_run *= alpha;
      w_run *= alpha;
      rescale(alpha);
    }
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) p[r] = exp2_hw(fmaf(x[r], cm, -m_run));
    ls = sum_tree<16>(p);
    ws = 0.0f;
#pragma unroll
    for (int a = 0; a < 2; ++a) {
#pragma unroll
      for (int u = 0; u < 8; ++u) pb[a][u] = (__bf16)p[8 * a + u];
      ws = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 0, 1), one2, ws,
                                           false);
      ws = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 2, 3), one2, ws,
                                           false);
      ws = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 4, 5), one2, ws,
                                           false);
      ws = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pb[a], pb[a], 6, 7), one2, ws,
                                           false);
    }
  };

  // Interleave the block's MFMAs with its LDS reads and VALU work; the LDS
  // reads run a few MFMAs ahead of their use so that their latency is hidden.
  auto interleave = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 0);  // DS reads ahead
#pragma unroll
    for (int i = 0; i < 2 * NDS; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // VALU
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // DS reads
    }
  };

  // Scale-then-mask of sub-tile k's scores (keys 32 k ..): keys past the end
  // of the sequence and, when causal, keys after the query get -inf.  Only
  // sub-tiles k >= nfs need it.
  auto mask = [&](f32x16_t& x, int k) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 32 * k + acc_key_perm(r, h);
      if (key >= Tk || (CAUSAL && key > qg + off)) x[r] = -INFINITY;
    }
  };

  // Score tiles and bf16 weights of consecutive sub-tiles alternate between
  // the X (even k) and Y (odd k) registers, so the pipeline never copies.
  f32x16_t sX, sY;
  bf16x8_t pX[2], pY[2];

  // One sub-step for score sub-tile k: S_k is in scur, P_{k-1} in pprev;
  // computes S_{k+1} from K half kh of kb and accumulates P_{k-1} V_{k-1}
  // from V half vh of vb.
  auto substep = [&](auto has_pv, auto vhi_stage, const char* kb, int kh, const char* vb, int vh,
                     f32x16_t& scur,
                     f32x16_t& snext, const bf16x8_t(&pprev)[2], bf16x8_t(&pcur)[2],
                     int k) __attribute__((always_inline)) {
    if constexpr (PRESCALE) {
#pragma unroll
      for (int r = 0; r < 16; ++r) scur[r] *= c;
    }
    if (k >= nfs) mask(scur, k);
    qk(kb, kh, snext);
    float ls, ws;
    if constexpr (decltype(has_pv)::value) {
      pv(vhi_stage, vb, vh, pprev);
      const bool over = softmax(scur, pcur, ls, ws);
      interleave();
      if (over) regrow(std::false_type{}, scur, pcur, ls, ws);
    } else {
      // the first sub-tile (no P V yet): straight to the row max
      regrow(std::true_type{}, scur, pcur, ls, ws);
    }
    l_run += ls;
    w_run += ws;
  };

  // Iteration tau: sub-steps k = 2 tau + 1 and 2 tau + 2.  K_{tau+1} and V_tau
  // are in LDS (stages (tau+1)%3 and tau%3); K_{tau+3} and V_{tau+2} are
  // loaded into the stages freed by the previous iteration.  At the end the
  // loads of the previous iteration (K_{tau+2}, V_{tau+1}) must have landed.
  auto iteration = [&](auto stage, int tau) __attribute__((always_inline)) {
    constexpr int R = decltype(stage)::value;  // tau % 3
    // V stage R (laid out after the three K stages) past 64 KiB?
    using VHi = std::integral_constant<bool, 3 * C::KBYTES + R * C::VBYTES >= 65536>;
    char* kcur = R == 0 ? sK1 : R == 1 ? sK2 : sK0;
    char* kfree = R == 0 ? sK0 : R == 1 ? sK1 : sK2;
    char* vcur = R == 0 ? sV0 : R == 1 ? sV1 : sV2;
    char* vfree = R == 0 ? sV2 : R == 1 ? sV0 : sV1;
    dma_k(kfree, tau + 3);
    dma_v(vfree, tau + 2);
    ATTN_DEBUG_SYNC();
    if (tau < tskip) {
      substep(std::true_type{}, VHi{}, kcur, 0, vcur, 0, sY, sX, pX, pY, 2 * tau + 1);
      substep(std::true_type{}, VHi{}, kcur, 1, vcur, 1, sX, sY, pY, pX, 2 * tau + 2);
    }
    ATTN_DEBUG_SYNC();
    // Every wave issued KPER + VPER loads this iteration: waiting down to
    // that many in flight means K_{tau+2} and V_{tau+1} have landed.
    wait_dma(std::integral_constant<int, KPER + VPER>{});
    // The barrier makes every wave's landed writes visible and frees the
    // stages read in this iteration.
    stage_barrier();
  };

  // Prologue: K_0, V_0, K_1, V_1, K_2 into LDS, S_0, then sub-step 0 (no
  // P V yet).
  dma_k(sK0, 0);
  dma_v(sV0, 0);
  dma_k(sK1, 1);
  dma_v(sV1, 1);
  dma_k(sK2, 2);
  wait_dma(std::integral_constant<int, 0>{});
  __syncthreads();
  qk(sK0, 0, sX);
  substep(std::false_type{}, std::false_type{}, sK0, 1, sV0, 0, sX, sY, pY, pX, 0);
  // K_0's stage receives K_3 in iteration 0: every wave must be done
  // reading it first.
  __syncthreads();

  // Sub-tiles past the last tile's keys (k = 2 ntiles) are fully masked, so
  // their softmax leaves the running state unchanged.
  for (int tau = 0; tau < ntiles; tau += 3) {
    iteration(std::integral_constant<int, 0>{}, tau);
    if (tau + 1 >= ntiles) break;
    iteration(std::integral_constant<int, 1>{}, tau + 1);
    if (tau + 2 >= ntiles) break;
    iteration(std::integral_constant<int, 2>{}, tau + 2);
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
    float* __restrict__ O, float* __restrict__ LSE, int T, int BH, int nqb, int G, float c) {
  using C = F32Tile<D>;
  constexpr int BC = C::BC, NDS = C::NDS, NDT = C::NDT, KS = C::KS, VS = C::VS;
  constexpr int CH = C::CH, DCH = C::DCH;
  static_assert(CH * kThreads * 4 == BC * D, "tile split");

  __shared__ float sK[2][BC * KS];
  __shared__ __attribute__((aligned(16))) float sV[2][BC * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  int bh, bhkv, qb;
  block_coords(BH, nqb, G, bh, bhkv, qb);
  const size_t head = (size_t)bh * (size_t)T * D;
  const size_t kvhead = (size_t)bhkv * (size_t)T * D;
  const float* Qh = Q + head;
  const float* Kh = K + kvhead;
  const float* Vh = V + kvhead;
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
// fp32 kernel for grids far smaller than the GPU (d = 64): one workgroup per
// 32 query rows, the rows' visible keys split over the 4 waves in 32-key
// blocks (wave w takes blocks w, w + 4, ...), the waves' partial results
// merged in LDS with the online-softmax rescaling ("Attention Mechanism",
// section 3).  The time of the 128-row kernel is one wave's chain of fp32
// MFMAs over all keys of the longest query block; here it is a quarter of
// that.  The problem is tiny, so each lane reads its K and V operands
// straight from memory (bounded buffer loads: rows >= T read as zero), one
// block ahead.
// ---------------------------------------------------------------------------
template <bool CAUSAL>
__global__ __launch_bounds__(kThreads) void attn_fwd_f32_rows_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int T, int BH, int nqb, int G, float c) {
  constexpr int D = 64, NDS = D / 2, NDT = D / 32, NW = kThreads / 64, BLK = 32;
  __shared__ float sAcc[NW][32 * D];
  __shared__ float sM[NW][32], sL[NW][32];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int j = lane & 31, h = lane >> 5;
  int bh, bhkv, qb;
  block_coords(BH, nqb, G, bh, bhkv, qb);
  const size_t head = (size_t)bh * (size_t)T * D;
  const size_t kvhead = (size_t)bhkv * (size_t)T * D;
  const int r0 = qb * 32;
  const int qg = r0 + j;

  // Q: B operand of S^T = K Q^T, lane (j, h) holds Q[qg][2 s + h].
  float qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) qf[s] = qg < T ? Q[head + (size_t)qg * D + 2 * s + h] : 0.0f;

  const int kv_end = CAUSAL ? min(T, r0 + 32) : T;
  const int nblk = (kv_end + BLK - 1) / BLK;
  const int nmine = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;
  const __amdgpu_buffer_rsrc_t rK = make_rsrc(K + kvhead, T * D * 4);
  const __amdgpu_buffer_rsrc_t rV = make_rsrc(V + kvhead, T * D * 4);

  // Operands of block kb0: K[kb0 + j][2 s + h] (A of the score MFMA) and
  // V[kb0 + acc_key_plain(r, h)][32 dt + j] (A of the P V MFMA).
  auto load = [&](float (&kv)[NDS], float (&vv)[16 * NDT], int kb0) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      kv[s] = __uint_as_float(
          __builtin_amdgcn_raw_buffer_load_b32(rK, ((kb0 + j) * D + 2 * s + h) * 4, 0, 0));
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        vv[r * NDT + dt] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
            rV, ((kb0 + acc_key_plain(r, h)) * D + 32 * dt + j) * 4, 0, 0));
  };

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.0f;

  auto block = [&](const float (&kv)[NDS], const float (&vv)[16 * NDT], int kb0)
      __attribute__((always_inline)) {
    f32x16_t x[1] = {f32x16_t{}};
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      x[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[s], qf[s], x[0], 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 16; ++r) x[0][r] *= c;
    if (kb0 + BLK > T || (CAUSAL && kb0 + BLK - 1 > r0)) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kb0 + acc_key_plain(r, h);
        if (key >= T || (CAUSAL && key > qg)) x[0][r] = -INFINITY;
      }
    }
    float unused = 0.0f;  // fp32 P is not rounded: one normaliser serves O and LSE
    online_softmax_update<1, NDT>(x, 1.0f, m_run, l_run, unused, oacc);
#pragma unroll
    for (int r = 0; r < 16; ++r) l_run += x[0][r];
#pragma unroll
    for (int r = 0; r < 16; ++r)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vv[r * NDT + dt], x[0][r], oacc[dt], 0,
                                                        0, 0);
  };

  float k0[NDS], k1[NDS], v0[16 * NDT], v1[16 * NDT];
  if (nmine > 0) load(k0, v0, BLK * wave);
  for (int i = 0; i < nmine; i += 2) {
    if (i + 1 < nmine) load(k1, v1, BLK * (wave + NW * (i + 1)));
    block(k0, v0, BLK * (wave + NW * i));
    if (i + 1 >= nmine) break;
    if (i + 2 < nmine) load(k0, v0, BLK * (wave + NW * (i + 2)));
    block(k1, v1, BLK * (wave + NW * (i + 1)));
  }

  // Merge the waves' partial results per query row: each wave's
  // accumulator (relative to its own running max) into LDS, then 8 threads
  // per row combine them.
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4_t w;
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = oacc[dt][4 * g + u];
      *reinterpret_cast<f32x4_t*>(&sAcc[wave][j * D + 32 * dt + 8 * g + 4 * h]) = w;
    }
  if (h == 0) {
    sM[wave][j] = m_run;
    sL[wave][j] = l_run;
  }
  __syncthreads();
  constexpr int CPT = D / 8;
  const int row = tid >> 3, c0 = (tid & 7) * CPT;
  const int q = r0 + row;
  if (q >= T) return;
  float M = sM[0][row];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, sM[w][row]);
  float a[NW], Lt = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    a[w] = sM[w][row] == -INFINITY ? 0.0f : exp2_hw(sM[w][row] - M);
    Lt += a[w] * sL[w][row];
  }
  const float inv = 1.0f / Lt;
  float* orow = O + head + (size_t)q * D + c0;
#pragma unroll
  for (int u = 0; u < CPT; u += 4) {
    f32x4_t w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float acc = 0.0f;
#pragma unroll
      for (int ww = 0; ww < NW; ++ww) acc = fmaf(a[ww], sAcc[ww][row * D + c0 + u + e], acc);
      w[e] = acc * inv;
    }
    *reinterpret_cast<f32x4_t*>(orow + u) = w;
  }
  if (c0 == 0) LSE[(size_t)bh * T + q] = (M + log2_hw(Lt)) * kLn2;
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
                     int64_t B, int64_t H, int64_t Hkv, int64_t T, int64_t d, int causal,
                     float scale, int64_t elem, bool& empty) {
  empty = false;
  if (B < 0 || H < 0 || T < 0 || Hkv < 0) return ATTN_ERR_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_UNSUPPORTED;
  if (causal != 0 && causal != 1) return ATTN_ERR_ARG;
  if (!std::isfinite(scale)) return ATTN_ERR_SCALE;
  // H is a whole number of groups of query heads per key/value head
  if ((Hkv == 0) != (H == 0) || (Hkv > 0 && H % Hkv != 0)) return ATTN_ERR_SHAPE;
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
  const int64_t nb = BH * T * d * elem, kb = B * Hkv * T * d * elem, lb = BH * T * 4;
  if (overlaps(o, nb, q, nb) || overlaps(o, nb, k, kb) || overlaps(o, nb, v, kb) ||
      overlaps(lse, lb, q, nb) || overlaps(lse, lb, k, kb) || overlaps(lse, lb, v, kb) ||
      overlaps(lse, lb, o, nb))
    return ATTN_ERR_ARG;
  return ATTN_OK;
}

// Kernel of the bf16 forward for these sizes on the current device (after
// check_device).  Problems whose grid of 256-row workgroups is smaller than
// the device are bound by the latency of their longest query block, which
// one wave walks key tile after key tile:
//  - the row-chunk kernel (32 query rows per workgroup, their keys split
//    over its 4 waves: a quarter of that chain, 8x the workgroups of the
//    8-wave kernel, with a software pipeline between the two contractions
//    only at d = 128) when the 4-wave grid, counted in d = 64 units, fits
//    the CUs once;
//  - else the 4-wave kernel (128 rows, one wave per SIMD) when the 8-wave
//    grid has fewer workgroups than the device has CUs (or, causal with
//    T >= 2048 at d = 128, T >= 4096 at d = 64, as many);
//  - else the 8-wave kernel.
// Measured on MI355X (average launch, bf16): the row-chunk kernel takes
// 16 us against 37 us (4-wave) at B H = 8, T = 2048, d = 64, causal, 167
// against 282 us at B H = 1, T = 16384, d = 128, causal, but 112 against
// 83 us at B H = 8, T = 4096, d = 128, causal, where the 4-wave grid
// already fills the CUs twice in d = 64 units.
enum class FwdPlan { kWaves8, kWaves4, kRows };

// The 4-wave instance also takes one full round of 256-row blocks under the
// causal mask from T = 2048 on at d = 128 and T = 4096 at d = 64: there a
// head's last block walks every key tile and its first a few, the heaviest
// sets the time, and the 128-row blocks halve it.  Measured on MI355X (us
// per launch, 4-wave / 8-wave, B H ceil(T / 256) = 256, causal): d = 128,
// T = 2048 55.4-55.6 / 58.0-58.8, T = 4096 91.4 / 105.9, T = 8192
// 167.7 / 199.5, T = 32768 625.7 / 760.4; d = 64, T = 4096 63.2 / 74.0;
// but d = 64, T = 2048 44.5 / 41.2, d = 128, T = 1024 46.3 / 36.7; and at
// 384 blocks (one and a half rounds) 267.5 / 222.9.
FwdPlan pick_plan(int64_t B, int64_t H, int64_t T, int64_t d, int causal) {
  const int64_t cus = device_cus();
  if (B * H * ((T + 127) / 128) * (d / 64) <= cus) return FwdPlan::kRows;
  const int64_t blocks = B * H * ((T + 255) / 256);
  const bool one_round = causal && blocks == cus && T >= (d == 128 ? 2048 : 4096);
  return blocks < cus || one_round ? FwdPlan::kWaves4 : FwdPlan::kWaves8;
}

// The fp32 forward takes the row-chunk kernel (32 rows per workgroup, keys
// split over 4 waves) at d = 64 when its 128-row grid has fewer workgroups
// than the device has CUs.
bool f32_rows(int64_t B, int64_t H, int64_t T, int64_t d) {
  const int64_t cus = device_cus();
  return d == 64 && B * H * ((T + kBR - 1) / kBR) < cus;
}

// K through LDS in the row-chunk forward (see attn_rows::row_chunk_attention),
// except at d = 128 with 8 waves, where the K stages would not fit LDS next
// to V's.  Measured on MI355X (us per launch, K in LDS / in registers):
// B H = 8, T = 2048, causal: d = 64 16.3 / 20.1, d = 128 29.8 / 37.4; no
// mask, d = 64 19.0 / 24.9.
template <int D, int NW>
constexpr bool kRowsKLds = D == 64 || NW == 4;
// The software-pipelined block loop where a wave has its SIMD to itself
// (d = 128, 4 waves, one workgroup per CU).  Measured on MI355X (us per
// launch, pipelined / plain, bit-identical outputs): B H = 8, T = 2048,
// causal, d = 128 25.7 / 27.6; the d = 64 instances, two workgroups per CU,
// lose with it (d = 64 15.0 / 14.7).
template <int D, int NW>
constexpr bool kRowsPipe = D == 128 && NW == 4;

// Square forward on the row-chunk kernel: Tq = Tk = T, one key split (the
// chunk's keys are cut only between its NW waves), O and LSE written
// directly.
// Two workgroups per CU at d = 64; at d = 128 the K and V stages of one
// 4-wave workgroup take 128 KiB of LDS, so one.
template <int D, bool CAUSAL, int NW>
__global__ __launch_bounds__(64 * NW, NW == 4 && D == 64 ? 2 : 1) void attn_fwd_rows_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int T, int G, int NR, int nwg, float c) {
  attn_rows::row_chunk_attention<D, CAUSAL, NW, kRowsKLds<D, NW>, kRowsPipe<D, NW>>(
      Q, K, V, O, LSE, nullptr, nullptr, T, T, T, G, 1, T, NR, nwg, c);
}

template <int NW>
const void* rows_kernel(int64_t d, int causal) {
  if (d == 64) return causal ? (const void*)attn_fwd_rows_kernel<64, true, NW>
                             : (const void*)attn_fwd_rows_kernel<64, false, NW>;
  return causal ? (const void*)attn_fwd_rows_kernel<128, true, NW>
                : (const void*)attn_fwd_rows_kernel<128, false, NW>;
}

// Waves of the row-chunk kernel: 4, or 8 for sequences of at least 4096
// keys.  More waves shorten each wave's chain of key blocks, but fewer
// workgroups then fit a CU (registers, LDS); only long key ranges gain.
// Measured on MI355X with K in registers (us per launch, 8 / 4 waves):
// B H = 1, T = 16384, d = 128, causal 167 / 217; B H = 4, T = 4096,
// d = 128, causal 55 / 61; B H = 8, T = 4096, d = 64, causal 56 / 56; but
// B H = 8, T = 2048, d = 64, causal 24 / 20 and B H = 16, T = 1024,
// d = 128, no mask 35 / 28 (with K in LDS at d = 64, 8 waves for every
// length: 18.2 against 16.3 us at T = 2048).
int rows_waves(int64_t T) { return T >= 4096 ? 8 : 4; }

attn_status launch_rows(int64_t d, int causal, const void* q, const void* k, const void* v,
                        void* o, float* lse, int64_t B, int64_t H, int64_t Hkv, int64_t T,
                        float scale, hipStream_t stream) {
  const int nw = rows_waves(T);
  const void* kern = nw == 8 ? rows_kernel<8>(d, causal) : rows_kernel<4>(d, causal);
  const int64_t G = H / Hkv;
  const int64_t nchunk = (T * G + attn_rows::kMaxRows - 1) / attn_rows::kMaxRows;
  int t = (int)T, g = (int)G, nr = (int)(B * H * T), nwg = (int)(B * Hkv);
  float c = scale * kLog2e;
  void* args[] = {(void*)&q, (void*)&k,  (void*)&v,   (void*)&o,   (void*)&lse,
                  (void*)&t, (void*)&g,  (void*)&nr,  (void*)&nwg, (void*)&c};
  const dim3 grid((unsigned)(B * Hkv * nchunk)), block(64 * nw);
  if (hipLaunchKernel(kern, grid, block, args, 0, stream) != hipSuccess) return ATTN_ERR_LAUNCH;
  return ATTN_OK;
}

// Launches one workgroup of `threads` threads per `rows` query rows of each
// query head; G query heads share one key/value head.
template <typename Elem>
attn_status launch(const void* kernel, int threads, int rows, const Elem* q, const Elem* k,
                   const Elem* v, Elem* o, float* lse, int64_t B, int64_t H, int64_t Hkv,
                   int64_t T, float scale, hipStream_t stream) {
  int t = (int)T, bh = (int)(B * H), nqb = (int)((T + rows - 1) / rows), g = (int)(H / Hkv);
  float c = scale * kLog2e;
  void* args[] = {(void*)&q, (void*)&k,   (void*)&v, (void*)&o, (void*)&lse,
                  (void*)&t, (void*)&bh,  (void*)&nqb, (void*)&g, (void*)&c};
  const dim3 grid((unsigned)(bh * nqb)), block(threads);
  if (hipLaunchKernel(kernel, grid, block, args, 0, stream) != hipSuccess) return ATTN_ERR_LAUNCH;
  return ATTN_OK;
}

template <bool PRESCALE, int NW>
const void* bf16_kernel_p(int64_t d, int causal) {
  if (d == 64) return causal ? (const void*)attn_fwd_bf16_kernel<64, true, PRESCALE, NW>
                             : (const void*)attn_fwd_bf16_kernel<64, false, PRESCALE, NW>;
  return causal ? (const void*)attn_fwd_bf16_kernel<128, true, PRESCALE, NW>
                : (const void*)attn_fwd_bf16_kernel<128, false, PRESCALE, NW>;
}

const void* bf16_kernel(int64_t d, int causal, float scale, int nw) {
  if (nw == 4)
    return scale > 0.0f ? bf16_kernel_p<false, 4>(d, causal) : bf16_kernel_p<true, 4>(d, causal);
  return scale > 0.0f ? bf16_kernel_p<false, 8>(d, causal) : bf16_kernel_p<true, 8>(d, causal);
}

// Launches the bf16 kernel with `nw` waves (32 nw query rows per
// workgroup) over T query rows per head and Tk keys per key/value head
// stored with a stride of Tcap rows; query row i sits at key position
// i + off.
attn_status launch_bf16(int nw, int64_t d, int causal, float scale, const void* q, const void* k,
                        const void* v, void* o, float* lse, int64_t B, int64_t H, int64_t Hkv,
                        int64_t T, int64_t Tk, int64_t Tcap, int64_t off, hipStream_t stream) {
  const void* kernel = bf16_kernel(d, causal, scale, nw);
  const int rows = 32 * nw;
  int t = (int)T, tk = (int)Tk, tcap = (int)Tcap, of = (int)off, bh = (int)(B * H),
      nqb = (int)((T + rows - 1) / rows), g = (int)(H / Hkv);
  float c = scale * kLog2e;
  void* args[] = {(void*)&q,  (void*)&k,   (void*)&v,  (void*)&o,   (void*)&lse,
                  (void*)&t,  (void*)&tk,  (void*)&tcap, (void*)&of, (void*)&bh,
                  (void*)&nqb, (void*)&g,  (void*)&c};
  const dim3 grid((unsigned)(bh * nqb)), block(64 * nw);
  if (hipLaunchKernel(kernel, grid, block, args, 0, stream) != hipSuccess) return ATTN_ERR_LAUNCH;
  return ATTN_OK;
}

const void* f32_kernel(int64_t d, int causal) {
  if (d == 64) return causal ? (const void*)attn_fwd_f32_kernel<64, true>
                             : (const void*)attn_fwd_f32_kernel<64, false>;
  return causal ? (const void*)attn_fwd_f32_kernel<128, true>
                : (const void*)attn_fwd_f32_kernel<128, false>;
}

// Name of the 4-wave (128-row) bf16 instance.
const char* w4_kernel_name(int64_t d, int causal) {
  static const char* w4[2][2] = {
      {"attn_fwd_bf16_d64_full_br128_bc64_w4", "attn_fwd_bf16_d64_causal_br128_bc64_w4"},
      {"attn_fwd_bf16_d128_full_br128_bc64_w4", "attn_fwd_bf16_d128_causal_br128_bc64_w4"}};
  return w4[d == 128 ? 1 : 0][causal ? 1 : 0];
}

}  // namespace

namespace attn_internal {

bool fwd_fills_device(int64_t B, int64_t H, int64_t Tq) {
  return B * H * ((Tq + 127) / 128) >= device_cus();
}

attn_status fwd_over_cache(const void* q, const void* k, const void* v, void* o, float* lse,
                           int64_t B, int64_t H, int64_t H_kv, int64_t Tq, int64_t Tk,
                           int64_t Tk_cap, int64_t d, int causal, float scale,
                           hipStream_t stream) {
  if (check_device() != ATTN_OK) return ATTN_ERR_DEVICE;
  const int nw = pick_plan(B, H, Tq, d, 0) == FwdPlan::kWaves8 ? 8 : 4;
  return launch_bf16(nw, d, causal, scale, q, k, v, o, lse, B, H, H_kv, Tq, Tk, Tk_cap,
                     causal ? Tk - Tq : 0, stream);
}

const char* fwd_over_cache_kernel_name(int64_t B, int64_t H, int64_t Tq, int64_t d, int causal) {
  if (check_device() != ATTN_OK) return nullptr;
  if (pick_plan(B, H, Tq, d, 0) == FwdPlan::kWaves8) return attn_kernel_name(0, d, causal);
  return w4_kernel_name(d, causal);
}

}  // namespace attn_internal

extern "C" {

attn_status attn_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                         int64_t B, int64_t H, int64_t H_kv, int64_t T, int64_t d, int causal,
                         float scale, hipStream_t stream) {
  bool empty;
  attn_status st = validate(q, k, v, o, lse, B, H, H_kv, T, d, causal, scale, 2, empty);
  if (st != ATTN_OK || empty) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  const FwdPlan plan = pick_plan(B, H, T, d, causal);
  if (plan == FwdPlan::kRows)
    return launch_rows(d, causal, q, k, v, o, lse, B, H, H_kv, T, scale, stream);
  const int nw = plan == FwdPlan::kWaves4 ? 4 : 8;
  return launch_bf16(nw, d, causal, scale, q, k, v, o, lse, B, H, H_kv, T, T, T, 0, stream);
}

attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                     int64_t H, int64_t T, int64_t d, int causal, float scale,
                     hipStream_t stream) {
  return attn_fwd_gqa(q, k, v, o, lse, B, H, H, T, d, causal, scale, stream);
}

attn_status attn_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                         int64_t B, int64_t H, int64_t T, int64_t d, int causal, float scale,
                         hipStream_t stream) {
  bool empty;
  attn_status st = validate(q, k, v, o, lse, B, H, H, T, d, causal, scale, 4, empty);
  if (st != ATTN_OK || empty) return st;
  if ((st = check_device()) != ATTN_OK) return st;
  if (f32_rows(B, H, T, d))
    return launch<float>(causal ? (const void*)attn_fwd_f32_rows_kernel<true>
                                : (const void*)attn_fwd_f32_rows_kernel<false>,
                         kThreads, 32, q, k, v, o, lse, B, H, H, T, scale, stream);
  return launch<float>(f32_kernel(d, causal), kThreads, kBR, q, k, v, o, lse, B, H, H, T, scale,
                       stream);
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
    case ATTN_ERR_WORKSPACE: return "workspace missing or smaller than required";
  }
  return "unknown status";
}

const char* attn_fwd_kernel_name_for(int64_t B, int64_t H, int64_t T, int64_t d, int causal) {
  if (B <= 0 || H <= 0 || T <= 0 || (d != 64 && d != 128) || (causal != 0 && causal != 1))
    return nullptr;
  if (B > (int64_t(1) << 31) / H || T > (int64_t(1) << 31)) return nullptr;
  if (check_device() != ATTN_OK) return nullptr;
  const FwdPlan plan = pick_plan(B, H, T, d, causal);
  if (plan == FwdPlan::kWaves8) return attn_kernel_name(0, d, causal);
  static const char* rows[2][2][2] = {
      {{"attn_fwd_rows_bf16_d64_full_br32_bc32_w4", "attn_fwd_rows_bf16_d64_causal_br32_bc32_w4"},
       {"attn_fwd_rows_bf16_d128_full_br32_bc32_w4",
        "attn_fwd_rows_bf16_d128_causal_br32_bc32_w4"}},
      {{"attn_fwd_rows_bf16_d64_full_br32_bc32_w8", "attn_fwd_rows_bf16_d64_causal_br32_bc32_w8"},
       {"attn_fwd_rows_bf16_d128_full_br32_bc32_w8",
        "attn_fwd_rows_bf16_d128_causal_br32_bc32_w8"}}};
  if (plan == FwdPlan::kRows) return rows[rows_waves(T) == 8 ? 1 : 0][d == 128 ? 1 : 0][causal];
  return w4_kernel_name(d, causal);
}

const char* attn_fwd_f32_kernel_name_for(int64_t B, int64_t H, int64_t T, int64_t d,
                                         int causal) {
  if (B <= 0 || H <= 0 || T <= 0 || (d != 64 && d != 128) || (causal != 0 && causal != 1))
    return nullptr;
  if (B > (int64_t(1) << 31) / H || T > (int64_t(1) << 31)) return nullptr;
  if (check_device() != ATTN_OK) return nullptr;
  if (!f32_rows(B, H, T, d)) return attn_kernel_name(1, d, causal);
  return causal ? "attn_fwd_f32_rows_d64_causal_br32_bc32_w4"
                : "attn_fwd_f32_rows_d64_full_br32_bc32_w4";
}

const char* attn_kernel_name(int is_f32, int64_t d, int causal) {
  if (d != 64 && d != 128) return nullptr;
  if (causal != 0 && causal != 1) return nullptr;
  static const char* names[2][2][2] = {
      {{"attn_fwd_bf16_d64_full_br256_bc64_w8", "attn_fwd_bf16_d64_causal_br256_bc64_w8"},
       {"attn_fwd_bf16_d128_full_br256_bc64_w8", "attn_fwd_bf16_d128_causal_br256_bc64_w8"}},
      {{"attn_fwd_f32_d64_full_br128_bc32_w4", "attn_fwd_f32_d64_causal_br128_bc32_w4"},
       {"attn_fwd_f32_d128_full_br128_bc32_w4", "attn_fwd_f32_d128_causal_br128_bc32_w4"}}};
  return names[is_f32 ? 1 : 0][d == 128 ? 1 : 0][causal];
}

}  // extern "C"
