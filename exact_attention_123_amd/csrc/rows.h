// Row-chunk attention for AMD Instinct MI355X (gfx950): one workgroup takes
// up to 32 query rows (one MFMA column block) and a range of keys, which its
// waves (4 or 8) split between them: each wave streams its own 32-key blocks,
// with no workgroup barrier in the loop -- K straight into registers (the A
// operand of the score MFMA as loaded) or direct-to-LDS, V direct-to-LDS
// (its transposing read needs LDS), both one block ahead, and with one wave
// per SIMD the next block's scores computed during this block's softmax --
// and the waves' partial results
// (running max, normalisers, output accumulator) merge in LDS at the end
// with the rescaling of the online softmax ("Attention Mechanism:
// Computation & Memory Patterns", section 3: the running max and sum let
// partial results over key blocks be rescaled and combined).
//
// Rows are (query head, query) pairs of the G query heads that share one
// key/value head: row r is member r / Tq, query r % Tq, and the Tq queries
// sit at positions Tk - Tq .. Tk - 1 of the Tk keys (query i sees key j iff
// j <= Tk - Tq + i under the causal mask).  With Tq = Tk this is the square
// forward; with a few queries over a long cache it is decode.  Under the
// causal mask a workgroup visits only the keys its rows can see, and the
// chunks are ordered heavy-first (most keys first).
//
// Used by the decode kernel (key splits over workgroups, merged by a second
// kernel) and by the forward for grids too small to fill the GPU with
// 256-row workgroups (one split: the keys of a chunk are cut only between
// its waves, so the critical path is 1 / NW of the longest key range).
#ifndef ATTN_ROWS_H_
#define ATTN_ROWS_H_

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "tiles.h"

namespace attn_rows {

using namespace attn_tiles;

constexpr int kWaves = 4;  // waves per workgroup unless the caller picks NW
constexpr int kThreads = 64 * kWaves;
constexpr int kBlk = 32;      // keys per block (one MFMA score tile)
constexpr int kMaxRows = 32;  // query rows of one workgroup (one MFMA column block)
// The running max follows the max-threshold rule of attn_tiles
// (kLazyRescale).

// Body of a kernel of 64 NW threads (NW waves share the keys of the
// chunk).  Workgroup (row chunk, kv head
// bhkv, split s) over keys [s kps, min(Tk, (s + 1) kps)); the grid holds
// nwg = (key/value heads) x nsplit workgroups per chunk, chunk outermost.
// The chunk holds rows 32 chunk .. 32 chunk + 31 of the R = Tq G rows of
// its group.  part_o / part_lse: when nsplit > 1, the split's normalised
// output and natural-log LSE per query row (row index (bhq Tq + qi), NR
// rows), else unused and O, LSE written.
// KLDS: K goes through LDS like V (coalesced direct-to-LDS loads, swizzled
// row reads) instead of straight into registers.  Loading K in MFMA operand
// order makes every load instruction touch 64 partial cache lines, which
// costs the vector memory pipeline four times the work of a coalesced load:
// the right trade when the kernel streams a long cache from HBM (decode),
// not when it re-reads short key ranges from L2 (forward on small grids).
// PIPE: software-pipelined block loop (see below), for instances with one
// wave per SIMD, whose own chain no other wave hides; with two waves per
// SIMD the plain loop is as fast and needs fewer registers.
template <int D, bool CAUSAL, int NW = kWaves, bool KLDS = false, bool PIPE = false>
__device__ __forceinline__ void row_chunk_attention(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, float* __restrict__ part_o,
    float* __restrict__ part_lse, int Tq, int Tk, int Tcap, int G, int nsplit, int kps,
    int NR, int nwg, float c) {
  using C = RowTile<D>;
  constexpr int NDS = C::NDS, NDT = C::NDT, RB = C::RB;
  constexpr int TB = kBlk * RB;  // bytes of one K or V block
  // Two V stages per wave, each stage its own object so that the compiler
  // can tell the loads into one from the reads of the other.
  static_assert(NW % 2 == 0 && (64 * NW) % kMaxRows == 0, "wave count");
  __shared__ __attribute__((aligned(1024))) char sV0[NW][TB];
  __shared__ __attribute__((aligned(1024))) char sV1[NW][TB];
  __shared__ __attribute__((aligned(1024))) char sK0[KLDS ? NW : 1][KLDS ? TB : 16];
  __shared__ __attribute__((aligned(1024))) char sK1[KLDS ? NW : 1][KLDS ? TB : 16];
  __shared__ float sM[NW][kMaxRows], sL[NW][kMaxRows], sW[NW][kMaxRows];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int j = lane & 31, h = lane >> 5;
  // Workgroup id: row chunk outermost (nwg workgroups per chunk), so the
  // chunks reading the same keys share an XCD when nwg is a multiple of 8;
  // the last chunk first (under the causal mask it has the most keys).
  const int id = blockIdx.x;
  const int nchunk = (int)gridDim.x / nwg;
  const int chunk = nchunk - 1 - id / nwg, rest = id % nwg;
  const int bhkv = rest / nsplit, split = rest % nsplit;
  const int R = Tq * G;             // query rows of the group
  const int r0 = kMaxRows * chunk;  // this workgroup's first row
  const bool row_ok = r0 + j < R;
  const int qi = (r0 + j) % Tq;
  const size_t qrow = ((size_t)bhkv * G + (r0 + j) / Tq) * Tq + qi;  // global query row
  const int pos = Tk - Tq + qi;                                      // its position

  // Q fragment: B operand [d][query] of S^T = K Q^T.  The contraction
  // over d takes k-step s of lane half h from d = 8 (NDS h + s) .. + 8, so
  // that a lane's K operand over all steps is one contiguous run of its row
  // (K from LDS: d = 8 (2 s + h) .. + 8, the order of the swizzled row
  // reads).
  bf16x8_t qf[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) {
    qf[s] = bf16x8_t{};
    const int d0 = KLDS ? 8 * (2 * s + h) : 8 * (NDS * h + s);
    if (row_ok) qf[s] = *reinterpret_cast<const bf16x8_t*>(Q + qrow * D + d0);
  }

  const int k_lo = split * kps;
  int k_hi = min(Tk, k_lo + kps);
  // Under the causal mask the chunk's rows see keys up to Tk - Tq + (their
  // largest query index), and keys below k_all are visible to all of them
  // (a chunk that wraps from one member's last queries to the next one's
  // first holds both ends of the query range).
  int k_all = k_hi;
  if (CAUSAL) {
    const int r_last = min(r0 + kMaxRows, R) - 1;
    const bool one_member = r0 / Tq == r_last / Tq;
    const int qi_max = one_member ? r_last % Tq : Tq - 1;
    const int qi_min = one_member ? r0 % Tq : 0;
    k_hi = min(k_hi, Tk - Tq + qi_max + 1);
    k_all = Tk - Tq + qi_min + 1;
  }
  const int nblk = (k_hi - k_lo + kBlk - 1) / kBlk;
  const int nmine = nblk > wave ? (nblk - wave + NW - 1) / NW : 0;
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
  // Loads of the wave's i-th block (keys kb0 ..): K into registers kr or
  // LDS stage kt, V into LDS stage vt.  (No load into a stage may move
  // above the reads of the block that stage held before.)
  auto load_k = [&](bf16x8_t (&kr)[NDS], char* kt, int i) __attribute__((always_inline)) {
    const int kb0 = k_lo + kBlk * (wave + NW * i);
    asm volatile("" ::: "memory");
    if constexpr (KLDS) {
      dma.load(kt, Kh, k_hi, kb0, 0);
    } else {
      const __amdgpu_buffer_rsrc_t rk =
          make_rsrc(Kh + (size_t)kb0 * D, max(k_hi - kb0, 0) * RB);
#pragma unroll
      for (int s = 0; s < NDS; ++s)
        kr[s] = __builtin_bit_cast(bf16x8_t, buf_load16(rk, krow + 16 * s));
    }
  };
  auto load_v = [&](char* vt, int i) __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    dma.load(vt, Vh, k_hi, k_lo + kBlk * (wave + NW * i), 0);
  };

  f32x16_t oacc[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; ++dt) oacc[dt] = f32x16_t{};
  float m_run = kMinusHuge, l_run = 0.0f, w_run = 0.0f;
  const bf16x2_t one2 = {(__bf16)1.0f, (__bf16)1.0f};

  // The steps of one block (keys kb0 ..):
  // scores S^T = K Q^T;
  auto qk = [&](const bf16x8_t (&kr)[NDS], const char* kt, f32x16_t& sc)
      __attribute__((always_inline)) {
    sc = f32x16_t{};
#pragma unroll
    for (int s = 0; s < NDS; ++s)
      sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(KLDS ? lds_row(kt, ad.row[s]) : kr[s], qf[s],
                                                   sc, 0, 0, 0);
  };
  // the scores in log2 units (any sign of the scale; register 8 a + e holds
  // key kb0 + 16 a + 8 h + e of query row j), the mask, the row max and,
  // where it outgrew the running max by more than the threshold, the
  // rescaling of the accumulator and normalisers;
  auto rescale = [&](f32x16_t& sc, int i) __attribute__((always_inline)) {
    const int kb0 = k_lo + kBlk * (wave + NW * i);
#pragma unroll
    for (int r = 0; r < 16; ++r) sc[r] *= c;
    if (kb0 + kBlk > k_hi || (CAUSAL && kb0 + kBlk > k_all)) {
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
  };
  // the weights and their bf16 rounding, with both normalisers;
  auto weights = [&](const f32x16_t& sc, bf16x8_t (&pb)[2]) __attribute__((always_inline)) {
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
    }
  };
  // O^T += V^T P^T.
  auto pv = [&](const char* vt, const bf16x8_t (&pb)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            lds_tr(vt, 16 * a * RB + ad.tr[0][dt], 16 * a * RB + ad.tr[1][dt]), pb[a],
            oacc[dt], 0, 0, 0);
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
  constexpr int PERK = KLDS ? PER : NDS;  // load instructions of one K block
  using Zero = std::integral_constant<int, 0>;
  using WaitV = std::integral_constant<int, PER>;
  using WaitKV = std::integral_constant<int, PER + PERK>;

  bf16x8_t k0[NDS], k1[NDS];
#pragma unroll
  for (int s = 0; s < NDS; ++s) k0[s] = k1[s] = bf16x8_t{};
  char* kt0 = KLDS ? sK0[KLDS ? wave : 0] : nullptr;
  char* kt1 = KLDS ? sK1[KLDS ? wave : 0] : nullptr;
  if constexpr (!PIPE) {
    // Plain loop: block i's K and V in stage i % 2, the next block's loads
    // issued before the block's steps run one after the other.
    auto block = [&](const bf16x8_t (&kr)[NDS], const char* kt, const char* vt, int i)
        __attribute__((always_inline)) {
      f32x16_t sc;
      bf16x8_t pb[2];
      qk(kr, kt, sc);
      rescale(sc, i);
      weights(sc, pb);
      pv(vt, pb);
    };
    if (nmine > 0) {
      load_k(k0, kt0, 0);
      load_v(sV0[wave], 0);
    }
    for (int i = 0; i < nmine; i += 2) {
      if (i + 1 < nmine) {
        load_k(k1, kt1, i + 1);
        load_v(sV1[wave], i + 1);
        wait_loads(WaitKV{});
      } else {
        wait_loads(Zero{});
      }
      block(k0, kt0, sV0[wave], i);
      if (i + 1 >= nmine) break;
      if (i + 2 < nmine) {
        load_k(k0, kt0, i + 2);
        load_v(sV0[wave], i + 2);
        wait_loads(WaitKV{});
      } else {
        wait_loads(Zero{});
      }
      block(k1, kt1, sV1[wave], i + 1);
    }
  } else {
    // Software pipeline over the wave's blocks, two stages each of K and V:
    // step i issues V_i and K_{i+2}, then (once K_{i+1} and V_{i-1} have
    // landed) accumulates P_{i-1} V_{i-1} while it takes the row max of S_i,
    // and computes S_{i+1} while it takes the weights of S_i, so that each
    // wave's matrix work overlaps its own softmax.  Block i uses K stage i % 2
    // and V stage i % 2; score tiles and weights alternate between the X
    // (even i) and Y (odd i) registers.  At the last step S_{i+1} comes from
    // a stage that holds no new block and is never used.
    f32x16_t sX, sY;
    bf16x8_t pX[2], pY[2];
    auto step = [&](auto odd, int i) __attribute__((always_inline)) {
      constexpr bool O = decltype(odd)::value;  // i % 2
      char* vfree = O ? sV1[wave] : sV0[wave];  // V_i's stage (V_{i-2} read at step i - 1)
      const char* vprev = O ? sV0[wave] : sV1[wave];
      if (i + 2 < nmine) {
        load_v(vfree, i);
        load_k(O ? k1 : k0, O ? kt1 : kt0, i + 2);  // K_i's stage, read at step i - 1
        wait_loads(WaitKV{});
      } else {
        load_v(vfree, i);
        wait_loads(WaitV{});
      }
      pv(vprev, O ? pX : pY);
      rescale(O ? sY : sX, i);
      qk(O ? k0 : k1, O ? kt0 : kt1, O ? sX : sY);
      weights(O ? sY : sX, O ? pY : pX);
    };
    using Even = std::false_type;
    using Odd = std::true_type;
    if (nmine > 0) {
      load_k(k0, kt0, 0);
      if (nmine > 1) {
        load_k(k1, kt1, 1);
        wait_loads(std::integral_constant<int, PERK>{});
      } else {
        wait_loads(Zero{});
      }
      qk(k0, kt0, sX);
      // step 0, with no P V yet: V_0 and K_2 (into K_0's stage, which S_0 has
      // read), then S_1 once K_1 has landed
      load_v(sV0[wave], 0);
      if (nmine > 2) {
        load_k(k0, kt0, 2);
        wait_loads(WaitKV{});
      } else {
        wait_loads(WaitV{});
      }
      rescale(sX, 0);
      qk(k1, kt1, sY);
      weights(sX, pX);
      for (int i = 1; i < nmine; i += 2) {
        step(Odd{}, i);
        if (i + 1 >= nmine) break;
        step(Even{}, i + 1);
      }
      wait_loads(Zero{});
      pv((nmine & 1) ? sV0[wave] : sV1[wave], (nmine & 1) ? pX : pY);
    }
  }

  // Merge the waves' partial results for each query row.
  l_run += __shfl_xor(l_run, 32);
  w_run += __shfl_xor(w_run, 32);
  __syncthreads();  // every wave is done with its LDS stages
  // Wave w's 32 x D fp32 accumulator goes to slot w % (NW / 2) of sV0
  // (w < NW / 2) or sV1: each V stage holds exactly NW / 2 of them.
  static_assert(sizeof(sV0) == NW / 2 * sizeof(float) * kMaxRows * D, "merge buffer");
  auto part = [&](int w) __attribute__((always_inline)) -> float* {
    return reinterpret_cast<float*>(w < NW / 2 ? &sV0[0][0] : &sV1[0][0]) +
           (w % (NW / 2)) * kMaxRows * D;
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

  // TPR threads per query row, CPT columns each.
  constexpr int TPR = 64 * NW / kMaxRows;  // threads per query row
  constexpr int CPT = D / TPR;             // columns per thread
  static_assert(CPT % 4 == 0, "columns per thread");
  const int row = tid / TPR, c0 = (tid % TPR) * CPT;
  if (r0 + row >= R) return;
  float M = sM[0][row];
#pragma unroll
  for (int w = 1; w < NW; ++w) M = fmaxf(M, sM[w][row]);
  float a[NW], Lt = 0.0f, Wt = 0.0f;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
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
    for (int w = 0; w < NW; ++w)
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

}  // namespace attn_rows

#endif  // ATTN_ROWS_H_
