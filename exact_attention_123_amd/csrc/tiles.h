// Device helpers shared by every kernel of the library: vector types,
// constants, hardware exp2/log2, raw buffer descriptors, the lane-pair max
// and lazy-max constants of the online softmax, and a swizzled LDS layout
// for tiles of D-wide bf16 rows that are read both row-wise (A operand of a
// score MFMA) and column-wise with the transposing LDS read (A operand of a
// contraction over the rows).
#ifndef ATTN_TILES_H_
#define ATTN_TILES_H_

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>

// Race check.  Built with -DATTN_DEBUG_BARRIERS, the kernels add full
// workgroup barriers (every wave's loads, stores and LDS operations
// complete, then all waves meet) at points that every wave of a workgroup
// reaches: after each key/value tile's loads are issued and after its
// compute.  A correct kernel gives bitwise the same results either way
// (same arithmetic, same order); a missing wait shows as a difference.
#ifdef ATTN_DEBUG_BARRIERS
#define ATTN_DEBUG_SYNC() __syncthreads()
#else
#define ATTN_DEBUG_SYNC() \
  do {                     \
  } while (0)
#endif

namespace attn_tiles {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;

constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }

// Max of x over the lane pair (l, l ^ 32) that holds one query's scores in
// the transposed score tile of a 32x32 MFMA.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Lazy running max of the online softmax, max-threshold form (the row-chunk
// and fp32 kernels; the large-grid bf16 forward bounds each lane's weight
// sum instead): the running max m (log2 units) is raised only when a
// block's max exceeds it by more than kLazyRescale, so every weight
// exp2(s - m) stays below 2^64, a normaliser of at most 2^17 such weights
// far inside fp32, and the accumulators are rescaled only on those rare,
// wave-uniform occasions.  The common factor cancels in acc / l.
constexpr float kLazyRescale = 64.0f;
// Initial running max: finite and far below any score in log2 units, so
// the first visible block always raises it (exp2(-huge - x) = 0 rescales an
// empty accumulator) while masked scores (-inf) still give weight 0.
constexpr float kMinusHuge = -1e38f;

// Raw buffer descriptor over `bytes` bytes at `base`: loads past the end
// return zero without touching memory (ragged ends of the sequence).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(__amdgpu_buffer_rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}

// Row order of the A operand of a score-like MFMA (swap bits 2 and 3 of the
// row index within 32).  With it, accumulator registers 8a .. 8a + 7 of lane
// half h hold rows 16 a + 8 h + 0..7 of the tile: eight consecutive rows,
// which is one B-operand slot of the MFMA that contracts over those rows.
__device__ __forceinline__ int row_perm(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// LDS tile of rows of D bf16: rows are unpadded, and the 16-byte chunk c of
// row r sits at chunk c ^ swz(r).  The tile is read two ways: row-wise, 16
// bytes per lane (A operand of a score MFMA; 16 lanes read 16 rows of one
// chunk), and column-wise with ds_read_b64_tr_b16 (A operand of a
// contraction over the rows; 32 lanes read 4 rows x 4 chunks).  swz makes
// both conflict-free: it is one-to-one on 16 consecutive rows, and on 4
// aligned rows it moves the 4-chunk group by the row within the four and the
// chunk within the group by the row's 4-row block.  It depends only on
// r mod 16.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

template <int D>
struct RowTile {
  static constexpr int RB = 2 * D;    // bytes per row
  static constexpr int NCH = D / 8;   // 16-byte chunks per row
  static constexpr int NDS = D / 16;  // k-steps over d
  static constexpr int NDT = D / 32;  // 32-wide d tiles
  static constexpr int RPK = 1024 / RB;  // rows per 1 KiB block
};

// Per-lane LDS addresses of the two read patterns (see swz).
//  row read: lane (j, h) reads row row_perm(j) (+ 32 u), chunk 2 s + h.
//  transposed read: ds_read_b64_tr_b16 hands lane i of a 16-lane group
//  element (i % 4) of the 8 bytes read by lane 4 e + i / 4 of the group, in
//  slot e.  Lane l of group g reads row 8 (g / 2) + l / 4 (+ 4 for the
//  second read), bytes 8 (l % 2) of chunk 4 dt + 2 (g % 2) + (l / 2) % 2, so
//  lane i of group g receives rows 8 (g / 2) + e (+ 4) of column
//  32 dt + 16 (g % 2) + i: for the wave, lane (j, h) gets rows 8 h + 0..7
//  of column 32 dt + j, the A operand [d][row] of a contraction over rows.
//  Offsets by multiples of 16 rows keep both patterns (swz has period 16).
template <int D>
struct TileAddr {
  using C = RowTile<D>;
  int row[C::NDS];
  int tr[2][C::NDT];
  __device__ __forceinline__ void init(int lane) {
    const int j = lane & 31, h = lane >> 5;
    const int r = row_perm(j);
    const int f = swz<D>(r);
#pragma unroll
    for (int s = 0; s < C::NDS; ++s) row[s] = r * C::RB + 16 * ((2 * s + h) ^ f);
    const int g = lane >> 4, l = lane & 15;
#pragma unroll
    for (int hi = 0; hi < 2; ++hi) {
      const int rr = 8 * (g >> 1) + (l >> 2) + 4 * hi;
      const int cc = 2 * (g & 1) + ((l >> 1) & 1);
#pragma unroll
      for (int dt = 0; dt < C::NDT; ++dt)
        tr[hi][dt] = rr * C::RB + 16 * ((4 * dt + cc) ^ swz<D>(rr)) + 8 * (l & 1);
    }
  }
};

// 16 bytes at a byte address of an LDS tile.
__device__ __forceinline__ bf16x8_t lds_row(const char* base, int off) {
  return *reinterpret_cast<const bf16x8_t*>(base + off);
}
// A operand (8 consecutive rows of one column) by two transposing reads.
__device__ __forceinline__ bf16x8_t lds_tr(const char* base, int off_lo, int off_hi) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + off_lo));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(base + off_hi));
  return __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Direct-to-LDS load of rows [row0, row0 + ROWS) of one head's [T][D] array
// into a tile, shared by NW waves.  Wave w writes 1 KiB blocks
// PER w .. PER w + PER - 1; a block is written by one instruction, lane L's
// 16 bytes landing at block offset 16 L = (row RPK b + L / NCH, chunk
// L % NCH), so the lane loads the global chunk that the swizzle puts there.
// Rows >= T read as zero.
template <int D, int ROWS, int NW>
struct TileDma {
  using C = RowTile<D>;
  static constexpr int NBLK = ROWS * C::RB / 1024;
  static constexpr int PER = NBLK / NW;
  static_assert(PER * NW == NBLK, "tile split");
  int off[PER];
  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      const int r = C::RPK * (PER * wave + n) + lane / C::NCH;
      const int p = lane % C::NCH;
      off[n] = r * C::RB + 16 * (p ^ swz<D>(r));
    }
  }
  __device__ __forceinline__ void load(char* tile, const __bf16* head, int T, int row0,
                                       int wave) const {
    const int rem = max(T - row0, 0) * C::RB;
    const __amdgpu_buffer_rsrc_t r = make_rsrc(head + (size_t)row0 * D, rem);
#pragma unroll
    for (int n = 0; n < PER; ++n) {
      // (a plain local: passing an array element to the builtin directly
      // makes the host-side instantiation drop the kernel)
      const int o = off[n];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (lds_void_t*)(tile + 1024 * (PER * wave + n)), 16, o, 0, 0, 0);
    }
  }
};

// Stores the 32 x D tile held as D / 32 transposed accumulators acc[dt]
// (lane (j, h): row j, columns 32 dt + 8 g + 4 h + 0..3 in registers
// 4 g .. 4 g + 3), times mul, as bf16 to out[row][.] if row < T.
template <int D>
__device__ __forceinline__ void store_rows(__bf16* out, const f32x16_t (&acc)[D / 32], float mul,
                                           int row, int T, int h) {
  if (row >= T) return;
  __bf16* dst = out + (size_t)row * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      __bf16 w[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) w[u] = (__bf16)(acc[dt][4 * g + u] * mul);
      u32x2_t bits;
      std::memcpy(&bits, w, 8);
      *reinterpret_cast<u32x2_t*>(dst + 32 * dt + 8 * g + 4 * h) = bits;
    }
}

}  // namespace attn_tiles

#endif  // ATTN_TILES_H_
