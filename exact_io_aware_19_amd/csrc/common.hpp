// Device building blocks for the gfx950 attention kernels: MFMA fragments, LDS
// swizzles, wave-half exchanges, bf16 packing.  CDNA4 only (wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace fa355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded in
// the source (no reliance on the unroller, whose size limits long schedules exceed).
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------------------------
// MFMA 32x32x16 bf16 -> fp32.  Fragment layout (checked on gfx950 with a probe):
//   A (32 x 16): lane l supplies row (l % 32), k-slots 8*(l/32) .. +7
//   B (16 x 32): lane l supplies column (l % 32), the same k-slots
//   C (32 x 32): lane l, register r holds row 8*(r/4) + 4*(l/32) + (r%4), column l%32
// Only the pairing of A and B k-slots matters for the product, so any consistent
// assignment of the contraction index to (l/32, j) is valid.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ f32x16 mfma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// The same product with the accumulator in ordinary vector registers and B read from
// accumulation registers, as inline assembly.  The compiler picks one accumulator form
// per kernel; where it keeps accumulators in accumulation registers, VALU code that
// reads a product (v_accvgpr_read) while other products run is slow, so products whose
// results feed VALU code use these.  The compiler does not know these are MFMAs: a VALU
// read of the result must come at least kMfmaValuWait wait states after the product
// (callers insert them with mfma_valu_wait()); a following product may accumulate into
// the result directly.  Nor does it insert the wait states a product needs after a VALU
// write of its B operand: b_acc must be a value that lives in accumulation registers
// (loaded there once, as the dK/dV pass's K and V fragments are).  A B operand computed
// by VALU code (measured: K with its sign bits changed by an AND and an XOR) is kept in
// vector registers and copied into accumulation registers right before each product,
// which then reads stale values.
constexpr int kMfmaValuWait = 12;  // 32x32x16 bf16 result -> VALU read, gfx950
__device__ __forceinline__ f32x16 mfma32_vz(const u32x4& a, const u32x4& b_acc) {  // C = 0
  f32x16 d;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b_acc));
  return d;
}
__device__ __forceinline__ void mfma32_vacc(f32x16& d, const u32x4& a, const u32x4& b_acc) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b_acc));
}
__device__ __forceinline__ void mfma_valu_wait() { asm volatile("s_nop 7\n\ts_nop 3" ::: "memory"); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Round-to-nearest-even pack of two fp32 values into one dword of two bf16
// (lo = a, hi = b); lowers to v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// v_permlane32_swap: after the swap lane l < 32 holds (own x, x of lane l+32) and lane
// l >= 32 holds (x of lane l-32, own x), so both results together are the two halves.
__device__ __forceinline__ float half_max(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)p[0]), __builtin_bit_cast(float, (uint32_t)p[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  uint32_t u = __builtin_bit_cast(uint32_t, x);
  auto p = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)p[0]) + __builtin_bit_cast(float, (uint32_t)p[1]);
}

// Max / sum of the 16*NB values of NB C fragments as balanced trees (depth log2, not
// a serial chain).
// The max tree takes three inputs per node (v_max3_f32): about half the instructions of
// a binary tree.
template <int NB>
__device__ __forceinline__ float tree_max(const f32x16 (&v)[NB]) {
  constexpr int NV = 16 * NB;
  float t[NV];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 16; ++i) t[16 * b + i] = v[b][i];
  int n = NV;
#pragma unroll
  for (int lvl = 0; lvl < 8; ++lvl) {
    if (n == 1) break;
    const int m = (n + 2) / 3;  // nodes of this level; the last one may take 1 or 2 inputs
#pragma unroll
    for (int i = 0; i < m; ++i) {
      const int a = 3 * i;
      if (a + 2 < n) t[i] = __builtin_fmaxf(__builtin_fmaxf(t[a], t[a + 1]), t[a + 2]);
      else if (a + 1 < n) t[i] = __builtin_fmaxf(t[a], t[a + 1]);
      else t[i] = t[a];
    }
    n = m;
  }
  return t[0];
}
template <int NB>
__device__ __forceinline__ float tree_sum(const f32x16 (&v)[NB]) {
  float t[8 * NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
#pragma unroll
    for (int i = 0; i < 8; ++i) t[8 * b + i] = v[b][2 * i] + v[b][2 * i + 1];
#pragma unroll
  for (int n = 4 * NB; n >= 1; n >>= 1)
#pragma unroll
    for (int i = 0; i < n; ++i) t[i] = t[i] + t[i + n];
  return t[0];
}

// Byte-select helpers for the 4x4 bf16 register transpose (v_perm_b32).
__device__ __forceinline__ uint32_t lo16_pair(uint32_t a, uint32_t b) {  // (a.lo16, b.lo16)
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t hi16_pair(uint32_t a, uint32_t b) {  // (a.hi16, b.hi16)
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Workgroup order.  Workgroups are dispatched round-robin over the 8 XCDs (workgroup i
// on XCD i % 8), each with its own L2.  HEAD_MAJOR (when B*H is a multiple of 8): every
// XCD works through whole heads, so the workgroups streaming one head's tiles share one
// L2 and HBM traffic drops to about the algorithmic bytes (measured: 2.5x less).
// Otherwise block-major: block `blk` of all heads before block blk+1, which runs the
// heaviest causal blocks first (measured faster for causal masks, where block costs
// differ; for equal-cost blocks both orders take the same time).
template <bool HEAD_MAJOR>
__device__ __forceinline__ void block_order(int i, int nblk, int BH, int& blk, int& bh) {
  if (HEAD_MAJOR && (BH & 7) == 0) {
    const int xcd = i & 7, slot = i >> 3;
    blk = slot % nblk;
    bh = (slot / nblk) * 8 + xcd;
  } else {
    blk = i / BH;
    bh = i % BH;
  }
}

// ---------------------------------------------------------------------------------
// LDS access helpers (explicit LDS address space so the compiler emits ds_* ops).
// ---------------------------------------------------------------------------------
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) u32x2 lds_u32x2;
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ __forceinline__ u32x4 lds_read128(const unsigned char* base, uint32_t byte) {
  return *(const lds_u32x4*)((const __attribute__((address_space(3))) unsigned char*)base + byte);
}
__device__ __forceinline__ void lds_write64(unsigned char* base, uint32_t byte, u32x2 v) {
  *(lds_u32x2*)((__attribute__((address_space(3))) unsigned char*)base + byte) = v;
}
__device__ __forceinline__ void lds_write128(unsigned char* base, uint32_t byte, u32x4 v) {
  *(lds_u32x4*)((__attribute__((address_space(3))) unsigned char*)base + byte) = v;
}

// Direct global -> LDS copy of 16 bytes per lane: lane l's 16 bytes land at
// lds_wave_base + 16*l (M0-relative; checked on gfx950 with a probe).
__device__ __forceinline__ void g2lds16(const void* gptr, unsigned char* lds_wave_base) {
  __builtin_amdgcn_global_load_lds((const void*)gptr,
                                   (__attribute__((address_space(3))) void*)(
                                       (__attribute__((address_space(3))) unsigned char*)lds_wave_base),
                                   16, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier that completes this wave's LDS operations but leaves its global
// loads (register loads and direct-to-LDS copies) in flight; __syncthreads() also waits
// for those.  Data copied into LDS must be waited for (wait_vmem) before a barrier that
// publishes it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------------
// Buffer-resource loads.  One resource per head matrix ([N][D] bf16, at most 16 MiB):
// the tile offset travels in the scalar soffset operand and each lane's offset inside
// the tile is loop-invariant, so a tile load costs no VALU address arithmetic.
// ---------------------------------------------------------------------------------
typedef __amdgpu_buffer_rsrc_t buf_rsrc;
constexpr int kBufWord3 = 0x00020000;  // raw (unformatted, unswizzled) dword access
__device__ __forceinline__ buf_rsrc make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufWord3);
}
// 16 bytes per lane straight into LDS at lds_wave_base + 16*lane
__device__ __forceinline__ void buf2lds16(buf_rsrc r, uint32_t voff, uint32_t soff, unsigned char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) unsigned char*)lds_wave_base),
      16, voff, soff, 0, 0);
}
// 4 bytes per lane straight into LDS at lds_wave_base + 4*lane (a buffer load: unlike a
// global one it counts only in the vector-memory wait counter, so waits for earlier LDS
// reads can stay partial)
__device__ __forceinline__ void buf2lds4(buf_rsrc r, uint32_t voff, uint32_t soff, unsigned char* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) unsigned char*)lds_wave_base),
      4, voff, soff, 0, 0);
}
__device__ __forceinline__ u32x2 buf_load64(buf_rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// ---------------------------------------------------------------------------------
// LDS tiles, "blocked chunk-major" layout.
//
// A tile is a matrix of R rows, each NCH 16-byte chunks long (8 bf16 per chunk).  The
// 16-byte unit holding chunk ch of row r sits at
//     unit(r, ch) = (r / 16) * 16 * NCH  +  ch * 16  +  (r % 16)
// i.e. blocks of 16 rows, chunk-major inside a block.  MFMA operand reads have 16
// lanes take 16 consecutive rows at one chunk: 16 consecutive units, one per 16-byte
// bank group, so they never conflict; and moving to another chunk or another 16-row
// block adds a compile-time constant, so every fragment address is one per-lane base
// plus an immediate offset.
//
// Natural tile: a [ROWS][D] slice of a row-major [N][D] matrix (NCH = D/8), filled
// with direct global->LDS copies (each wave instruction fills 64 consecutive units:
// 16 rows x 4 chunks).
// Transposed tile: the same slice stored as [D][ROWS] (row = head-dim index, NCH =
// ROWS/8: 8 consecutive slice rows per chunk), filled through registers with 4x4 bf16
// blocks transposed by v_perm.
// ---------------------------------------------------------------------------------
template <int NCH>
__device__ __forceinline__ constexpr uint32_t bcm_unit(uint32_t row, uint32_t ch) {
  return (row >> 4) * (16 * NCH) + ch * 16 + (row & 15);
}
template <int NCH>
__device__ __forceinline__ constexpr uint32_t bcm_byte(uint32_t row, uint32_t ch) {
  return bcm_unit<NCH>(row, ch) * 16;
}
// Transposed tiles additionally XOR the in-block row slot with (row / 16) % 4.  The
// register-path stores write, per instruction, rows d = 4*q + j over many q; without
// the XOR those rows occupy only 4 of the 16 bank groups (12 conflict cycles per store,
// measured); with it all 16 are used.  Reads keep 16 consecutive rows of one 16-row
// block, which the XOR only permutes.
template <int NCH>
__device__ __forceinline__ constexpr uint32_t bcm_tr_byte(uint32_t row, uint32_t ch) {
  return ((row >> 4) * (16 * NCH) + ch * 16 + ((row & 15) ^ ((row >> 4) & 3))) * 16;
}

// Row of a 32-row block that lane c feeds as the A operand: bits 2 and 3 of c swapped.
// With it, C register r of lane l belongs to block row 16*(r/8) + 8*(l/32) + (r%8), so
// each lane's eight consecutive C registers are eight consecutive rows -- the k-slots
// that lane feeds when the result is used as the B operand of the next product.
__device__ __forceinline__ uint32_t row_perm(uint32_t c) { return (c & ~12u) | ((c & 4u) << 1) | ((c & 8u) >> 1); }
// Block row held by C register r of a lane in half h (inverse view of row_perm).
__device__ __forceinline__ constexpr int c_row(int r, int h) { return 16 * (r >> 3) + 8 * h + (r & 7); }

// Direct copy of rows [row0, row0+ROWS) of a [N][D] bf16 matrix (buffer resource `r`)
// into a natural tile.  Rows at or past N are clamped to N-1: callers pass the number of
// rows that may be read (the matrix length, or the key-padding limit), so rows beyond it
// are never read and whatever they hold cannot reach a result (callers mask them).
template <int ROWS, int D, int NWAVES>
__device__ __forceinline__ void load_nat_tile(buf_rsrc r, int row0, int N, unsigned char* tile, int w, int l) {
  constexpr int NCH = D / 8;
  constexpr int UNITS = ROWS * NCH;
  constexpr int PER_WAVE = UNITS / (NWAVES * 64);
  static_assert(PER_WAVE * NWAVES * 64 == UNITS, "tile must split evenly over the waves");
  const uint32_t soff = (uint32_t)row0 * (D * 2);
  if (row0 + ROWS <= N) {  // uniform branch: the common case needs no clamping at all
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int pos = (i * NWAVES + w) * 64 + l;  // unit index written by this lane
      const int blk = pos / (16 * NCH), rem = pos % (16 * NCH);
      const int ch = rem >> 4, row = blk * 16 + (rem & 15);
      buf2lds16(r, (uint32_t)(row * (D * 2) + ch * 16), soff, tile + (size_t)(i * NWAVES + w) * 64 * 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int pos = (i * NWAVES + w) * 64 + l;
      const int blk = pos / (16 * NCH), rem = pos % (16 * NCH);
      const int ch = rem >> 4, row = min(blk * 16 + (rem & 15), N - 1 - row0);
      buf2lds16(r, (uint32_t)(row * (D * 2) + ch * 16), soff, tile + (size_t)(i * NWAVES + w) * 64 * 16);
    }
  }
}

// Per-lane base byte offsets of MFMA A-operand fragments.
//  natural tile [R][D]: lane (h, c) reads row 32*blk + row_perm(c), chunk 2*kk + h
//      -> nat_base + blk * NAT_BLK + kk * NAT_KK
//  transposed tile [D][R]: lane (h, c) reads row d = 32*db + c, chunk 4*rb + 2*sb + h
//      -> tr_base + db * TR_DB + (4*rb + 2*sb) * TR_CH
template <int D>
struct NatFrag {
  static constexpr int NCH = D / 8;
  static constexpr uint32_t BLK = 2 * 16 * NCH * 16;  // 32 rows
  static constexpr uint32_t KK = 2 * 16 * 16;         // 2 chunks
  __device__ __forceinline__ static uint32_t base(int c, int h) { return bcm_byte<NCH>(row_perm(c), h); }
};
template <int R>
struct TrFrag {
  static constexpr int NCH = R / 8;
  static constexpr uint32_t DB = 2 * 16 * NCH * 16;  // 32 head-dim rows
  static constexpr uint32_t CH = 16 * 16;            // one chunk (8 tile rows)
  // the slot XOR depends on (d / 16) % 4 = (2*db + c/16) % 4, i.e. on the parity of db:
  // base(c, h, db & 1) + db * DB + (4*rb + 2*sb) * CH
  __device__ __forceinline__ static uint32_t base(int c, int h, int dbpar) {
    return bcm_tr_byte<NCH>(c + 32 * dbpar, h) - dbpar * DB;
  }
};

// ---------------------------------------------------------------------------------
// Swizzled tiles.  The blocked chunk-major arrangement above with the in-block row slot
// XORed by (ch % 4) | 12 * ((row / 16) % 2):
//     unit(r, ch) = (r/16)*16*NCH + ch*16 + ((r%16) ^ ((ch%4) | 12*((r/16)%2)))
// Chosen by measurement (SQ_LDS_BANK_CONFLICT on gfx950 for each access pattern): a
// 128-bit LDS read is served in four 16-lane phases that are not plain lane ranges,
// and with this XOR the MFMA operand reads (natural and transposed tiles) and the
// reads and writes of the 8x8 transposition below are all conflict-free; an XOR by 4
// * ((r/16) % 2) alone, the obvious choice for 16-lane phases 0-15, 16-31, ..., costs
// a second cycle on every operand read.  Within 8 consecutive rows 8a .. 8a+7 of one
// chunk the slot is 8*b + (j ^ x) for a lane-constant b, x < 8, so the byte address of
// row 8a + j is addr(8a) ^ (16 j).
// ---------------------------------------------------------------------------------
template <int NCH>
__device__ __forceinline__ constexpr uint32_t swz_unit(uint32_t row, uint32_t ch) {
  return (row >> 4) * (16 * NCH) + ch * 16 + ((row & 15) ^ ((ch & 3) | (((row >> 4) & 1) * 12)));
}

// Second swizzle, for tiles that are also read transposed with ds_read_b64_tr_b16: the
// in-block slot XORed by 4 * (ch % 4).  Measured conflict-free on gfx950 for the MFMA
// operand reads (16 rows of one block at one chunk) and for transposed reads of 4
// rows x 16 columns per 16-lane group; the swizzle above conflicts on the latter.
template <int NCH>
__device__ __forceinline__ constexpr uint32_t swz4_unit(uint32_t row, uint32_t ch) {
  return (row >> 4) * (16 * NCH) + ch * 16 + ((row & 15) ^ (4 * (ch & 3)));
}

// 8 bytes per lane with the gfx950 16-bit transpose read: within each group of 16
// lanes, lane i receives element i % 4 of the 8-byte pieces addressed by lanes
// 4j + i / 4, j = 0..3 (checked with a probe).  A lane group that addresses rows
// k0 + s / 4, columns c0 + 4 (s % 4) .. +3 of a row-major bf16 matrix thus receives
// column c0 + i, rows k0 .. k0+3.
__device__ __forceinline__ u32x2 lds_read_tr16(const unsigned char* base, uint32_t byte) {
  typedef short v4i16 __attribute__((ext_vector_type(4)));
  const v4i16 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16*)((__attribute__((address_space(3))) unsigned char*)base + byte));
  return __builtin_bit_cast(u32x2, v);
}

// Direct copy of rows [row0, row0+ROWS) of a [N][D] bf16 matrix into a swizzled tile
// (swz_unit, or swz4_unit if SWZ4), one wave instruction (1 KB) at a time: instruction ii of wave w fills the 64
// consecutive 16-byte units starting at unit 64*(ii*NWAVES + w); the lane filling unit
// u fetches the (row, chunk) that the swizzle places there.  Rows at or past N are clamped
// to N-1 (callers pass the number of rows that may be read; rows beyond are never read
// and get zero weight).
template <int ROWS, int D, int NWAVES, bool SWZ4 = false>
struct SwzCopy {
  static constexpr int NCH = D / 8;
  static constexpr int PER_WAVE = ROWS * NCH / (NWAVES * 64);  // instructions per wave
  static_assert(PER_WAVE * NWAVES * 64 == ROWS * NCH, "tile must split evenly over the waves");
  __device__ __forceinline__ static void issue(buf_rsrc r, int row0, int N, unsigned char* tile, int w, int l,
                                               int ii) {
    const int u = (ii * NWAVES + w) * 64 + l;
    const int blk = u / (16 * NCH), ch = (u % (16 * NCH)) >> 4, slot = u & 15;
    const int x = SWZ4 ? 4 * (ch & 3) : ((ch & 3) | ((blk & 1) * 12));
    const int row = min(blk * 16 + (slot ^ x), N - 1 - row0);
    buf2lds16(r, (uint32_t)(row * (D * 2) + ch * 16), (uint32_t)row0 * (D * 2),
              tile + (size_t)(ii * NWAVES + w) * 64 * 16);
  }
};


// Transposition of one 8x8 bf16 block between swizzled tiles: rows 8*rc .. 8*rc+7,
// chunk dc of a natural [R][D] tile become rows 8*dc .. 8*dc+7, chunk rc of the
// transposed [D][R] tile.  rd = byte address of (row 8*rc, chunk dc) in the natural tile,
// wr = byte address of (row 8*dc, chunk rc) in the transposed one.
__device__ __forceinline__ void transpose8x8(const unsigned char* nat, uint32_t rd, unsigned char* tr, uint32_t wr) {
  u32x4 x[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = lds_read128(nat, rd ^ (16u * j));
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    // output row jj holds element jj of the 8 input rows; dword p = rows 2p, 2p+1
    u32x4 y;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      y[p] = (jj & 1) ? hi16_pair(x[2 * p][jj >> 1], x[2 * p + 1][jj >> 1])
                      : lo16_pair(x[2 * p][jj >> 1], x[2 * p + 1][jj >> 1]);
    lds_write128(tr, wr ^ (16u * jj), y);
  }
}

// Store a C fragment holding X^T (rows = head-dim d, column = this lane's row `row`)
// as fp32 row `row` of a [N][D] matrix, scaled by `mul`.
template <int D>
__device__ __forceinline__ void store_ct_rows_f32(float* g, int row, const f32x16 (&acc)[D / 32], float mul, int h) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = 32 * db + 8 * gq + 4 * h;
      const f32x4 out = {acc[db][4 * gq + 0] * mul, acc[db][4 * gq + 1] * mul, acc[db][4 * gq + 2] * mul,
                         acc[db][4 * gq + 3] * mul};
      *(f32x4*)(g + (size_t)row * D + d0) = out;
    }
}
// The same as bf16 (round to nearest even).
template <int D>
__device__ __forceinline__ void store_ct_rows(uint16_t* g, int row, const f32x16 (&acc)[D / 32], float mul, int h) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int d0 = 32 * db + 8 * gq + 4 * h;
      u32x2 out;
      out[0] = pack_bf16x2(acc[db][4 * gq + 0] * mul, acc[db][4 * gq + 1] * mul);
      out[1] = pack_bf16x2(acc[db][4 * gq + 2] * mul, acc[db][4 * gq + 3] * mul);
      *(u32x2*)(g + (size_t)row * D + d0) = out;
    }
}

// ---------------------------------------------------------------------------------
// Forward-pass V^T tiles.
// ---------------------------------------------------------------------------------
// Register-staged transposition of one half of a V tile (rows [BN/2 * part, +BN/2)) by
// the 256 threads of one wave group: each thread moves one 4x4 bf16 block (4 keys x 4
// head-dim columns) into the transposed [D][BN] tile, one 8-byte column at a time.
template <int BN, int D>
struct VtHalf {
  static_assert((BN / 2 / 4) * (D / 4) == 256, "one 4x4 block per thread of a wave group");
  u32x2 r[4];
  int k0, dq, kc, hsel;
  __device__ __forceinline__ void init(int t, int part) {
    hsel = t & 1;
    dq = (t >> 1) % (D / 4);
    kc = part * (BN / 16) + (t >> 1) / (D / 4);
    k0 = kc * 8 + hsel * 4;
  }
  // kend: one past the last admissible key; rows at or past it repeat row kend-1, so
  // padded rows are never read (whatever they hold, their P is 0 and they add 0)
  __device__ __forceinline__ void fetch(buf_rsrc rs, int row0, int kend) {
#pragma unroll
    for (int j = 0; j < 4; ++j) fetch_one(rs, row0, kend, j);
  }
  // row k0 + j of the block (one 8-byte load per lane)
  __device__ __forceinline__ void fetch_one(buf_rsrc rs, int row0, int kend, int j) {
    const int lim = kend - 1 - row0;
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)row0 * (D * 2));  // wave-uniform
    r[j] = buf_load64(rs, (uint32_t)(min(k0 + j, lim) * (D * 2) + dq * 8), soff);
  }
  // column j of the block: (V[k0 .. k0+3][4*dq + j])
  __device__ __forceinline__ void store(unsigned char* tile, int j) const {
    const int half = j >> 1;
    u32x2 out;
    if (j & 1) {
      out[0] = hi16_pair(r[0][half], r[1][half]);
      out[1] = hi16_pair(r[2][half], r[3][half]);
    } else {
      out[0] = lo16_pair(r[0][half], r[1][half]);
      out[1] = lo16_pair(r[2][half], r[3][half]);
    }
    lds_write64(tile, bcm_tr_byte<BN / 8>(dq * 4 + j, kc) + hsel * 8, out);
  }
};

}  // namespace fa355
