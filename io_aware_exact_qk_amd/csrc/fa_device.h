// fa_device.h — CDNA4 (gfx950) building blocks shared by the attention kernels.
//
// Matrix-core conventions (v_mfma_f32_32x32x16_{bf16,f16}, one wave of 64 lanes):
//   lane l, g = l / 32 (0 or 1), r = l % 32.
//   A operand (32 x 16): lane l holds row r, 8 contraction elements.
//   B operand (16 x 32): lane l holds column r, 8 contraction elements.
//   C/D (32 x 32 f32):   lane l holds column r, element i at row
//                        8*(i/4) + 4*g + (i%4).
// Which contraction index each (g, element) pair stands for is up to the
// caller as long as A and B agree.  Two assignments are used here:
//   * "natural":   element e of group g is k = 8*g + e within a 16-wide chunk,
//                  i.e. 16 contiguous bytes of a row (one ds_read_b128);
//   * "acc-order": element e of group g is k = 8*(e/4) + 4*g + (e%4), which is
//                  exactly the row order of a C fragment, so 8 consecutive
//                  accumulator elements of a fragment can be fed back as a B
//                  operand without moving data between lanes.
// A operands whose contraction runs along LDS rows (V^T, K^T, Q^T, dO^T) are
// read in acc-order with ds_read_b64_tr_b16: within each 16-lane group the
// four 8-byte fetches of lanes 4r..4r+3 form row r of a 4x16 tile and lane i
// receives column i of that tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fa_host.h"

namespace fa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

enum { DT_F16 = 0, DT_BF16 = 1 };

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Online softmax: how far (log2 units) a row max may exceed the exponent
// reference before the accumulators are rescaled.
constexpr float kRescaleSlack = 8.0f;

// ---------------------------------------------------------------- MFMA ----
// 32 x 32 x 64 product of fp8 (OCP e4m3) operands, float32 accumulate: each
// lane holds 32 contraction elements of its row (A) or column (B) as bytes;
// the hardware pairs byte j of A lane (i, half g) with byte j of B lane
// (n, half g), so any assignment of contraction indices to (g, j) that A and
// B share gives the same product.  Zero block scales select the unscaled
// instruction.
__device__ __forceinline__ f32x16 mfma32_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  if constexpr (DT == DT_BF16) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
}

// Two float32 -> one dword of two 16-bit values, round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2 v = {lo, hi};
  if constexpr (DT == DT_BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2_t));
  }
}

template <int DT>
__device__ __forceinline__ float to_f32(uint16_t h) {
  if constexpr (DT == DT_BF16) {
    return __builtin_bit_cast(float, (uint32_t)h << 16);
  } else {
    return (float)__builtin_bit_cast(_Float16, h);
  }
}

// Elements 8*half .. 8*half+7 of an accumulator fragment, rounded to 16 bits
// and packed as a B operand in acc-order.
template <int DT>
__device__ __forceinline__ u32x4 pack_frag_half(const f32x16& c, int half) {
  u32x4 r;
  const int o = 8 * half;
  r[0] = pack2<DT>(c[o + 0], c[o + 1]);
  r[1] = pack2<DT>(c[o + 2], c[o + 3]);
  r[2] = pack2<DT>(c[o + 4], c[o + 5]);
  r[3] = pack2<DT>(c[o + 6], c[o + 7]);
  return r;
}

// Row of element i of a C fragment held by a lane of group g.
__device__ __forceinline__ int frag_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// ------------------------------------------------------------- LDS tiles --
// A tile is ROWS x D 16-bit elements stored row-major; its 16-byte chunks are
// permuted within each row by an XOR with swz<D>(row).  The LDS returns 256
// bytes per clock: a ds_read_b128 is served 16 lanes at a time and a
// ds_read_b64_tr_b16 32 lanes at a time, and two addresses in the same clock
// conflict when they fall in the same 16-byte slot of a 256-byte line.  The
// permutation is chosen so that
//  * 16 consecutive rows read at one logical chunk (natural-order operands)
//    land in 16 different slots, and
//  * the 4 rows x 4 chunks of one half-wave transposed read (rows 4m..4m+3,
//    chunks 4n..4n+3) land in 16 different slots.
// D = 128 (16 chunks, one row per line): the low two row bits pick which
// aligned group of 4 chunks, the next two permute inside it.  D = 256 (32
// chunks, two lines per row): the same permutation inside each line.  D = 64
// (8 chunks, two rows per line, row parity picks the half line): row bit 1
// picks the group of 4 chunks, row bits 2-3 permute inside it.  D = 32
// (4 chunks, four rows per line, the low two row bits pick the quarter
// line): row bits 2-3 permute the 4 chunks.  In every case
// swz(row + 8) = swz(row) ^ 2 and swz depends on row % 16 only.
template <int D>
__device__ __forceinline__ uint32_t swz(int row) {
  static_assert(D == 32 || D == 64 || D == 128 || D == 256, "head dim");
  if constexpr (D >= 128) {
    return (uint32_t)(((row & 3) << 2) | ((row >> 2) & 3));
  } else if constexpr (D == 64) {
    return (uint32_t)((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
  } else {
    return (uint32_t)((row >> 2) & 3);
  }
}

template <int D>
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return (uint32_t)row * (D * 2) + (((uint32_t)chunk ^ swz<D>(row)) << 4);
}

// Byte offset of element (row, col) where col is a multiple of 4.
template <int D>
__device__ __forceinline__ uint32_t tile_off_elem4(int row, int col) {
  return tile_off<D>(row, col >> 3) + ((col & 7) << 1);
}

__device__ __forceinline__ u32x4 lds_read128(const char* smem, uint32_t off) {
  return *reinterpret_cast<const u32x4*>(smem + off);
}

__device__ __forceinline__ void lds_write128(char* smem, uint32_t off, u32x4 v) {
  *reinterpret_cast<u32x4*>(smem + off) = v;
}

__device__ __forceinline__ u32x2 lds_read_tr(const char* smem, uint32_t off) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(smem + off));
  return __builtin_bit_cast(u32x2, v);
}

// A operand (32 x 16) whose 32 rows are tile columns col0 .. col0+31 and whose
// contraction runs over tile rows row0 .. row0+15 in acc-order.
template <int D>
__device__ __forceinline__ u32x4 lds_read_At(const char* smem, int row0, int col0, int lane) {
  const int grp = lane >> 4;        // 16-lane group 0..3
  const int i = lane & 15;
  const int g = grp >> 1;           // which half of the wave (acc-order group)
  const int col = col0 + 16 * (grp & 1) + 4 * (i & 3);
  const int r = row0 + 4 * g + (i >> 2);
  u32x2 lo = lds_read_tr(smem, tile_off_elem4<D>(r, col));
  u32x2 hi = lds_read_tr(smem, tile_off_elem4<D>(r + 8, col));
  u32x4 out = {lo[0], lo[1], hi[0], hi[1]};
  return out;
}

// Natural-order operand: 8 contiguous elements of tile row `row`, chunk `chunk`.
template <int D>
__device__ __forceinline__ u32x4 lds_read_nat(const char* smem, int row, int chunk) {
  return lds_read128(smem, tile_off<D>(row, chunk));
}

// Offsets in XOR form.  Because row * 2D has no bits inside the chunk field,
//   tile_off(row, k) = row_base(row) ^ (k << 4),
// and swz depends on row % 16 only, so for R0 a multiple of 16
//   row_base(R0 + r) = R0 * 2D + row_base(r).
// A kernel therefore keeps one per-lane base and forms each LDS address with
// one XOR against a compile-time constant.
template <int D>
__device__ __forceinline__ uint32_t row_base(int row) {
  return (uint32_t)row * (D * 2) + (swz<D>(row) << 4);
}

// A value the compiler must treat as redefined at this point.  Loop bodies
// pass their per-lane LDS offsets through it once per iteration, so the
// per-read XORs below are recomputed in the loop (one VALU each) instead of
// being hoisted into one live register per read.
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// Natural-order operand offset of a lane: row r = lane % 32 of a 32-row block,
// chunk half g = lane / 32 folded in.
template <int D>
__device__ __forceinline__ uint32_t nat_base(int lane) {
  return row_base<D>(lane & 31) ^ ((uint32_t)(lane >> 5) << 4);
}

// Step c (16 contraction elements: chunks 2c and 2c + 1) of a natural-order
// operand whose 32 rows start at `tile` (16-row aligned within its tile);
// nb = the lane's nat_base.  Addresses stay derived from the __shared__ array
// (no integer-to-pointer casts), so the compiler can tell a read of one stage
// buffer from a DMA into the other and does not wait for that DMA.
__device__ __forceinline__ u32x4 lds_nat(const char* tile, uint32_t nb, int c) {
  return lds_read128(tile, nb ^ ((uint32_t)c << 5));
}

// Transposed (acc-order) operand offset of a lane for lds_At: byte offset,
// relative to a 16-row-aligned row0, of the 4-element piece it fetches from
// row 4g'+(i/4) (g' = lane/32, i = lane%16), columns 16*((lane/16)%2) + 4*(i%4)
// of a 32-column block.  The piece 8 rows below sits at (offset ^ 32) + 16D:
// swz(rr + 8) = swz(rr) ^ 2 for both tile widths.
template <int D>
__device__ __forceinline__ uint32_t tr_base(int lane) {
  const int grp = lane >> 4, i = lane & 15;
  const int rr = 4 * (grp >> 1) + (i >> 2);
  const int col = 16 * (grp & 1) + 4 * (i & 3);
  return (row_base<D>(rr) ^ ((uint32_t)(col >> 3) << 4)) | ((uint32_t)(col & 7) << 1);
}

// A operand (32 x 16) whose 32 rows are tile columns 32d .. 32d+31 and whose
// contraction runs over the 16 tile rows starting at `tile` (16-row aligned);
// tb = the lane's tr_base.
template <int D>
__device__ __forceinline__ u32x4 lds_At(const char* tile, uint32_t tb, int d) {
  const uint32_t lo = tb ^ ((uint32_t)d << 6);  // column block d = chunks 4d .. 4d+3
  const u32x2 x = lds_read_tr(tile, lo);
  const u32x2 y = lds_read_tr(tile + 8 * (D * 2), lo ^ 32u);
  u32x4 out = {x[0], x[1], y[0], y[1]};
  return out;
}

// ----------------------------------------------------- global -> LDS DMA --
// buffer_load_dword{,x4} ... lds: every lane fetches 4 or 16 bytes from
// base + soffset + its own voffset and the hardware writes lane l's bytes to
// LDS at lds_block + size * l, so one x4 instruction fills one contiguous 1 KB
// block without passing through VGPRs.  Completion is tracked by vmcnt.
//
// The buffer (MUBUF) form is used rather than global_load_lds: the compiler
// models the FLAT-encoded global form as an access that may also count on
// lgkmcnt, and while one is in flight it turns every LDS-read wait into
// lgkmcnt(0), which drains the operand rings the kernels keep a few reads
// ahead.  With the buffer form the waits stay exact (lgkmcnt(n)).
//
// The resource covers [base, base + 4 GB) with stride 0 (raw offsets) and the
// gfx9 default format word; callers keep every offset non-negative and far
// below 4 GB by rebasing on the first row a call touches.
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ buf_rsrc make_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, -1, 0x00020000);
}

__device__ __forceinline__ void dma16(buf_rsrc r, uint32_t voff, uint32_t soff, char* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_block, 16, voff, soff, 0, 0);
}

// 4-byte variant: lane l's dword lands at lds_block + 4 * l.
__device__ __forceinline__ void dma4(buf_rsrc r, uint32_t voff, char* lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_block, 4, voff, 0, 0, 0);
}

// Wait until every DMA (and global load) this wave issued has landed.
// Encoding: vmcnt = 0, expcnt and lgkmcnt left at their maxima.
__device__ __forceinline__ void dma_wait() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// s_waitcnt immediate that waits until at most n (< 64) vector-memory
// operations of this wave are outstanding (vmcnt split over bits 3:0 and
// 15:14), leaving expcnt and lgkmcnt at their maxima.
constexpr int vmcnt_imm(int n) { return ((n >> 4) << 14) | 0x0F70 | (n & 15); }

// Rows [row0, row0 + ROWS) of a row-major 16-bit matrix with D columns and a
// row stride of `rstride` elements, copied into an LDS tile laid out as
// tile_off<D>.  The 1 KB blocks of the tile are dealt to the NWAVES waves
// (w must be wave-uniform); lane l of a block writes physical chunk
// l % (D/8) of its row, so it loads the logical chunk that the swizzle maps
// there.  When every row is in range the source address is a wave-uniform
// base (scalar arithmetic) plus a 32-bit lane offset that does not change
// between tiles; otherwise rows at or past `nrows` (>= 1) re-read row
// nrows - 1 (valid memory) and callers mask those rows.  FAST = false always
// takes the clamped form (fewer live values, for kernels at the VGPR limit).
// DG < D: rows hold DG elements in memory and are padded to D on chip; the
// lanes of logical chunks >= DG / 8 copy nothing (those slots are zeroed
// once by zero_pad and never written again).
template <int D, int ROWS, int NWAVES, bool FAST = true, int DG = D>
__device__ __forceinline__ void dma_tile(char* tile, const uint16_t* base, int64_t rstride, int row0,
                                         int nrows, int w, int lane) {
  constexpr int NCH = D / 8, RPB = 64 / NCH, NBLK = ROWS / RPB;
  // more waves than 1 KB blocks (narrow tiles): the extra waves copy nothing
  constexpr int PER = (NBLK + NWAVES - 1) / NWAVES;
  static_assert(NBLK % NWAVES == 0 || NBLK < NWAVES, "tile blocks must divide among the waves");
  if (NBLK < NWAVES && w >= NBLK) return;
  const int rin = lane / NCH, pch = lane % NCH;
  if (FAST && row0 + ROWS <= nrows) {
    // resource at row row0; block offsets are wave-uniform (soffset)
    const buf_rsrc rs = make_rsrc(base + (int64_t)row0 * rstride);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk = i * NWAVES + w;
      const int row = blk * RPB + rin;
      // re-derived per call: keeping one offset per block live across the
      // tile loop would cost a VGPR each
      const uint32_t loff = opaque((uint32_t)(rin * rstride + ((pch ^ (int)swz<D>(row)) << 3)) * 2u);
      const uint32_t soff = (uint32_t)(blk * RPB) * (uint32_t)rstride * 2u;
      if (DG == D || (pch ^ (int)swz<D>(row)) < DG / 8) dma16(rs, loff, soff, tile + blk * 1024);
    }
  } else {
    // resource at the first row this call reads (row0 may lie past the last
    // row, whose copy is then read), so every lane offset is >= 0
    const int rb = min(row0, nrows - 1);
    const buf_rsrc rs = make_rsrc(base + (int64_t)rb * rstride);
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int blk = i * NWAVES + w;
      const int row = blk * RPB + rin;
      const int lch = pch ^ (int)swz<D>(row);
      const int grow = min(row0 + row, nrows - 1);
      const uint32_t voff = (uint32_t)((grow - rb) * (int)rstride + lch * 8) * 2u;
      if (DG == D || lch < DG / 8) dma16(rs, voff, 0u, tile + blk * 1024);
    }
  }
}

// Zero the 16-byte slots of a ROWS x D tile that hold logical chunks
// >= DG / 8 (a head dim DG < D padded to D on chip).  The DMA never writes
// them, so one pass before the first barrier keeps them zero for good.
template <int D, int ROWS, int DG>
__device__ __forceinline__ void zero_pad(char* tile, int tid, int nthreads) {
  if constexpr (DG < D) {
    constexpr int PAD = D / 8 - DG / 8;
    for (int i = tid; i < ROWS * PAD; i += nthreads) {
      const int row = i / PAD, lch = DG / 8 + i % PAD;
      lds_write128(tile, tile_off<D>(row, lch), u32x4{0, 0, 0, 0});
    }
  }
}

// ------------------------------------------------------------ wave utils --
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// Max / sum of x over lanes l and l ^ 32 with v_permlane32_swap (a VALU
// exchange, no LDS round trip).  Swapping x with itself leaves the low half
// of x in both halves of one result and the high half in both halves of the
// other, so every lane holds the pair {x[l], x[l ^ 32]}; both operations are
// symmetric, hence bitwise equal to x op xor32(x).
__device__ __forceinline__ float pair_max32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

// tanh from the identity tanh(y) = 1 - 2 / (1 + e^{2y}); its absolute error is
// a few float32 ulps of 1 for every y (e^{2y} overflowing to +inf gives 1,
// underflowing to 0 gives -1).
__device__ __forceinline__ float tanh_exp(float y) {
  const float e = fast_exp2(y * (2.0f * kLog2e));
  return 1.0f - 2.0f * fast_rcp(1.0f + e);
}

// 16-byte global load / store helpers.
__device__ __forceinline__ u32x4 gload128(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void gstore128(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ void gstore64(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// ---------------------------------------------------------- mask logic ----
// Visibility of key j to query row i (aligned position ip = i + Sk - Sq):
//   j < Sk, j >= ip - wl (wl >= 0), j <= ip + wr (wr >= 0).  Causal is folded
// into wr = 0 by the host.
struct MaskSpec {
  int wl, wr;  // -1 = unbounded
};

// Bitwise (not short-circuit) operators keep this a few VALU compares and no
// branches when it is evaluated per element.
__device__ __forceinline__ bool visible(int ip, int j, int Sk, MaskSpec m) {
  return (j < Sk) & ((m.wl < 0) | (j >= ip - m.wl)) & ((m.wr < 0) | (j <= ip + m.wr));
}

// The same mask in range form, for the elements of one lane: the visible
// values of the coordinate that varies along a lane's accumulator elements
// (keys for a query row, or query rows for a key) form one interval
// [lo, hi], empty when hi < lo.  Element i of a 32 x 32 block whose
// coordinate is base + frag_row(i, g) = (base + 4 g) + frag_c(i) is then
// visible iff (uint32)(base + 4 g - lo + frag_c(i)) <= (uint32)(hi - lo):
// an add with a constant, a compare and a select per element, instead of
// the three compares and the lane-mask logic of visible().
struct LaneRange {
  int lo, hi;
};

// Keys visible to query position ip (none when !row_ok).
__device__ __forceinline__ LaneRange keys_for_row(bool row_ok, int ip, int Sk, MaskSpec m) {
  const int lo = m.wl >= 0 ? max(ip - m.wl, 0) : 0;
  const int hi = m.wr >= 0 ? min(ip + m.wr, Sk - 1) : Sk - 1;
  return {lo, row_ok ? hi : lo - 1};
}

// Query rows (within the sequence, below Sq) that see key j, where query
// row r sits at position r + off (none when !key_ok).
__device__ __forceinline__ LaneRange rows_for_key(bool key_ok, int j, int Sq, int off, MaskSpec m) {
  const int lo = m.wr >= 0 ? max(j - m.wr - off, 0) : 0;
  const int hi = m.wl >= 0 ? min(j + m.wl - off, Sq - 1) : Sq - 1;
  return {lo, key_ok ? hi : lo - 1};
}

struct RangeTest {
  uint32_t a, w;
};

// base: the coordinate of element frag_c = 0 of this lane (block base + 4 g).
__device__ __forceinline__ RangeTest range_test(LaneRange r, int base) {
  if (r.hi < r.lo) return {0x80000000u, 0u};
  return {(uint32_t)(base - r.lo), (uint32_t)(r.hi - r.lo)};
}

// frag_row(i, g) - 4 g: the element's offset that does not depend on the lane
__device__ __forceinline__ constexpr int frag_c(int i) { return 8 * (i >> 2) + (i & 3); }

__device__ __forceinline__ bool in_range(RangeTest t, int i) { return t.a + (uint32_t)frag_c(i) <= t.w; }

// Block-level classification for query positions [ip0, ip1] and keys [j0, j1].
// Returns 0 = nothing visible, 1 = partially visible, 2 = everything visible.
__device__ __forceinline__ int classify(int ip0, int ip1, int j0, int j1, int Sk, MaskSpec m) {
  if (j0 >= Sk) return 0;
  if (m.wr >= 0 && j0 > ip1 + m.wr) return 0;
  if (m.wl >= 0 && j1 < ip0 - m.wl) return 0;
  const bool full = (j1 < Sk) && (m.wr < 0 || j1 <= ip0 + m.wr) && (m.wl < 0 || j0 >= ip1 - m.wl);
  return full ? 2 : 1;
}

// ------------------------------------------------------------- dropout ----
// Dropout on the attention weights.  The keep decision of (query row i, key
// j) of one (batch entry, query head) bh comes from the counter-based
// generator Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror,
// D. E. Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011): one
// call per 4 x 4 block of pairs, counter (j/4, i/4, bh, offset), key = the
// 64-bit seed; word i%4 of the result holds the block's row i, byte j%4 of
// that word the pair (i, j), which is kept when the byte is >= t.  Kept
// weights are scaled by 256 / (256 - t), applied once to the accumulated
// products.
// (DropSpec, the parameters, is declared with the host helpers.)

__device__ __forceinline__ u32x4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                               uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return u32x4{c0, c1, c2, c3};
}

// 4 x 4 transpose across the four lanes of every quad: word w of lane q
// becomes word q of lane w.  Stage 1 exchanges lane bit 0 with word bit 0
// (DPP quad_perm [1,0,3,2]), stage 2 lane bit 1 with word bit 1
// (quad_perm [2,3,0,1]).
__device__ __forceinline__ void quad_transpose(uint32_t (&x)[4], int lane) {
  const bool b0 = (lane & 1) != 0, b1 = (lane & 2) != 0;
#pragma unroll
  for (int w = 0; w < 4; w += 2) {
    const uint32_t send = b0 ? x[w] : x[w + 1];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0xB1, 0xF, 0xF, false);
    if (b0) x[w] = recv;
    else x[w + 1] = recv;
  }
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t send = b1 ? x[w] : x[w + 2];
    const uint32_t recv = (uint32_t)__builtin_amdgcn_mov_dpp((int)send, 0x4E, 0xF, 0xF, false);
    if (b1) x[w] = recv;
    else x[w + 2] = recv;
  }
}

// 4 x 4 byte transpose inside one lane: byte c of word a becomes byte a of
// word c.  v_perm_b32 picks each result byte from the 8 bytes {s0 : s1}
// (s1 = bytes 0..3, s0 = bytes 4..7).
__device__ __forceinline__ void byte_transpose(uint32_t (&x)[4]) {
  const uint32_t a0 = __builtin_amdgcn_perm(x[1], x[0], 0x06020400u);  // x0.0 x1.0 x0.2 x1.2
  const uint32_t a1 = __builtin_amdgcn_perm(x[1], x[0], 0x07030501u);  // x0.1 x1.1 x0.3 x1.3
  const uint32_t c0 = __builtin_amdgcn_perm(x[3], x[2], 0x06020400u);  // x2.0 x3.0 x2.2 x3.2
  const uint32_t c1 = __builtin_amdgcn_perm(x[3], x[2], 0x07030501u);  // x2.1 x3.1 x2.3 x3.3
  x[0] = __builtin_amdgcn_perm(c0, a0, 0x05040100u);
  x[1] = __builtin_amdgcn_perm(c1, a1, 0x05040100u);
  x[2] = __builtin_amdgcn_perm(c0, a0, 0x07060302u);
  x[3] = __builtin_amdgcn_perm(c1, a1, 0x07060302u);
}

// Keep words of a 32 x 32 block in MFMA accumulator layout.  A lane owns one
// index `own` along the accumulator's columns (a query, or a key) and the
// runs R = 0..3 of four consecutive indices 8 R + 4 g + 0..3 along its rows,
// counted from `first`.  The four lanes of a quad own four consecutive
// indices (own % 4 = lane % 4); lane q computes the generator call of run q.
// Queries along the columns: the call's word own % 4 is the lane's, so the
// quad transpose hands lane q word q of every run's call.  Keys along the
// columns: the call of run R holds the four queries as words and the quad's
// keys as bytes; a byte transpose first gathers byte (own % 4) of the four
// words.  Either way x[R] byte c keeps the pair at row 8 R + 4 g + c.
template <bool KEY_COLUMNS>
__device__ __forceinline__ void drop_words(const DropSpec& ds, uint32_t bh, int own, int first, int lane,
                                           uint32_t (&x)[4]) {
  const int run = lane & 3, g = (lane >> 5) & 1;
  const uint32_t row4 = (uint32_t)(first + 8 * run + 4 * g) >> 2;
  const uint32_t own4 = (uint32_t)own >> 2;
  // counter = (key / 4, query / 4, bh, offset)
  const u32x4 w = KEY_COLUMNS ? philox4x32_10(own4, row4, bh, ds.off, ds.k0, ds.k1)
                              : philox4x32_10(row4, own4, bh, ds.off, ds.k0, ds.k1);
#pragma unroll
  for (int e = 0; e < 4; ++e) x[e] = w[e];
  if constexpr (KEY_COLUMNS) byte_transpose(x);
  quad_transpose(x, lane);
}

// Element e (0..15) of the lane's accumulator fragment: kept?
__device__ __forceinline__ bool drop_keep(const uint32_t (&x)[4], int e, uint32_t t) {
  return ((x[e >> 2] >> (8 * (e & 3))) & 0xFFu) >= t;
}

}  // namespace fa
