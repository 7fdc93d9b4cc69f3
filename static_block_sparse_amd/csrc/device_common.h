// Device-side helpers shared by the radial attention kernels (gfx950).
//
// MFMA conventions used throughout (v_mfma_f32_32x32x16_bf16, wave64):
//   * lane l has column c = l % 32 and k-group g = l / 32;
//   * A operand (32 x 16, M x K): lane l holds row c, 8 bf16 along K;
//   * B operand (16 x 32, K x N): lane l holds column c, 8 bf16 along K;
//   * C/D (32 x 32 fp32): lane l holds column c, register r is row
//     8 * (r / 4) + 4 * g + (r % 4).
// The product sums over K, so any one-to-one assignment of the 16 K indices
// to (g, element) gives the same result as long as A and B use the same
// assignment.  The kernels pick, per 16-wide K step,
//   element e of k-group g  <->  k = 8 * (e / 4) + 4 * g + (e % 4),
// which is exactly the row set a C fragment's registers 0..7 (or 8..15,
// shifted by 16) hold.  That lets an fp32 C fragment be rounded to bf16 and
// fed back as an A or B operand without moving data between lanes: the
// fragment's column index stays the lane's column and its rows become the
// contraction index.  Operands loaded from memory with that assignment read
// two runs of 4 consecutive elements: [4g, 4g+4) and [8+4g, 8+4g+4).
// Operands whose K index is contiguous in memory (the head dimension D of
// Q, K, V, dO rows) use the plain assignment k = 8 * g + e instead; both
// operands of such a product are loaded that way.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace radial {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.f;
  return z;
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = bf16(0.f);
  return z;
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 lo, bf16x4 hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 8 bf16 from the permuted K assignment: p[0..3] and p[8..11].
__device__ __forceinline__ bf16x8 ld_perm(const bf16 *p) {
  return cat(*reinterpret_cast<const bf16x4 *>(p), *reinterpret_cast<const bf16x4 *>(p + 8));
}

__device__ __forceinline__ bf16x8 ld8(const bf16 *p) {
  return *reinterpret_cast<const bf16x8 *>(p);
}

__device__ __forceinline__ void st4(bf16 *p, bf16x4 v) {
  *reinterpret_cast<bf16x4 *>(p) = v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Swizzled element offset of 16-byte block `ch` of row `row` in a row-major
// [rows][D] bf16 LDS tile (no padding): the block index is XORed with f(row).
// LDS has 64 banks of 4 bytes.  A 16-byte read serves 16 lanes per pass: at
// D = 128 they read one block of 16 consecutive rows (256-byte rows, one bank
// line each), at D = 64 one block of 16 rows two to a bank line.  A
// transposing 8-byte read serves 32 lanes per pass, which read 4 consecutive
// rows x 4 consecutive blocks (lane groups 0-15 and 16-31 take the two
// 16-column halves of the same rows).  f is chosen so both kinds of pass
// touch every bank once:
//   D = 128: f = 4 (row % 4) + (row / 4) % 4 -- the 4 rows of a pass get
//            XOR masks in distinct 4-block groups, and 16 consecutive rows
//            get all 16 masks;
//   D = 64:  f = 4 ((row / 2) % 2) + (row / 4) % 4 -- two rows share a bank
//            line (one per half); the rows of a transposing pass that share
//            a half get masks in distinct 4-block groups, and the 8 rows of
//            one half among 16 consecutive rows get all 8 masks.
template <int D>
__device__ __forceinline__ int swz_f(int row) {
  static_assert(D == 64 || D == 128, "head dim");
  if constexpr (D == 128) return 4 * (row % 4) + (row / 4) % 4;
  return 4 * ((row / 2) % 2) + (row / 4) % 4;
}

template <int D>
__device__ __forceinline__ int swz(int row, int ch) {
  return row * D + 8 * (ch ^ swz_f<D>(row));
}

// max / sum of x over the lane pair (l, l ^ 32) (gfx950 v_permlane32_swap)
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i supplies the address of 4 consecutive bf16 of row r0 + i / 4 at
// columns c0 + 4 (i % 4) (a 4 x 16 block); lane i receives column c0 + i of
// rows r0 .. r0 + 3.
__device__ __forceinline__ bf16x4 ld_tr(const bf16 *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(p));
}

// Raw buffer resource over `bytes` bytes at p (gfx9 data-format word).
// Loads at offsets >= bytes return zeros, which is how rows past the end of
// a sequence are padded without branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, bytes, 0x00020000);
}

__device__ __forceinline__ bf16x8 buf_ld8(__amdgpu_buffer_rsrc_t r, int byte_off) {
  typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
  return __builtin_bit_cast(bf16x8, v);
}

typedef __attribute__((address_space(3))) void lds_void;

// Direct global-to-LDS copy (gfx950 buffer_load_dwordx4 ... lds): lane l
// copies the 16 bytes at `byte_off` of the buffer to LDS address
// lds_block + 16 * l; lanes past the end of the buffer write zeros.  The
// data is visible to other waves after s_waitcnt vmcnt(0) and a barrier.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, bf16 *lds_block, int byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_block, 16, byte_off, 0, 0, 0);
}

typedef __attribute__((ext_vector_type(4))) unsigned u32x4;

// The four words of a raw buffer resource over `bytes` bytes at p, in
// scalar registers (p and bytes must be wave-uniform).  Same layout as
// make_rsrc: base, base high bits (stride 0), record count, format word.
__device__ __forceinline__ u32x4 rsrc_words(const void *p, int bytes) {
  const unsigned long long a = (unsigned long long)p;
  u32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((unsigned)a);
  r[1] = __builtin_amdgcn_readfirstlane((unsigned)(a >> 32) & 0xffffu);
  r[2] = __builtin_amdgcn_readfirstlane((unsigned)bytes);
  r[3] = 0x00020000u;
  return r;
}

// LDS offset of a generic pointer into LDS: the low 32 bits of a flat
// address inside the LDS aperture (the aperture base has zero low bits).
// Unlike an address-space cast this needs no null check; p must point into
// LDS.
__device__ __forceinline__ unsigned lds_offset(const void *p) {
  return (unsigned)(unsigned long long)p;
}

// dma16 issued from inline assembly.  The compiler does not see this copy,
// so it adds no vmcnt waits of its own before LDS reads that it cannot prove
// disjoint from the copy's destination (it cannot for the transposing reads,
// and would otherwise make every copy complete before the next V^T read).
// The caller therefore owns the wait: s_waitcnt vmcnt(0) (wait_vmem) and a
// barrier before anyone reads the destination.  The instruction writes LDS
// only (no register results).  M0 carries the LDS address.  M0 is a register
// the compiler reserves, so listing it as clobbered does not oblige the
// compiler to preserve it (it warns about exactly that): a kernel that uses
// these copies must not have compiler-generated code that relies on M0.
// The backward kernels have none (they use no compiler-issued copy to LDS);
// a CPU test checks their compiled code for any M0 access outside these
// statements.
__device__ __forceinline__ void dma16_async(u32x4 r, const bf16 *lds_block, int byte_off) {
  const unsigned lds_addr = __builtin_amdgcn_readfirstlane(lds_offset(lds_block));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(byte_off), "s"(r)
      : "m0");
}

// The 4-byte form of dma16_async: lane l writes LDS bytes [4 l, 4 l + 4) of
// lds_block from byte offset byte_off of the resource.
__device__ __forceinline__ void dma4_async(u32x4 r, const void *lds_block, int byte_off) {
  const unsigned lds_addr = __builtin_amdgcn_readfirstlane(lds_offset(lds_block));
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "buffer_load_dword %1, %2, 0 offen lds"
      :
      : "s"(lds_addr), "v"(byte_off), "s"(r)
      : "m0");
}

// Copies a ROWS x D bf16 tile (row-major at `src`, `valid` rows before the
// end of the sequence) into a row-major, swizzled LDS tile, NW waves sharing
// the work: copy jj of wave w fills LDS bytes [(w*NDMA + jj) * 1024, +1024);
// lane l writes element e = blk*512 + 8l, i.e. row e / D and physical 16-byte
// block (e % D) / 8, which holds logical block (physical ^ swz_f(row)) of the
// row.  Rows at or past `valid` read as zeros.
template <int D, int ROWS, int NW>
struct TileCopier {
  static constexpr int NDMA = ROWS * D * 2 / 1024 / NW;  // copies per wave
  static_assert(NDMA >= 1 && ROWS * D * 2 % (1024 * NW) == 0, "tile split");
  int off[NDMA];
  __device__ __forceinline__ void init(int wave, int lane);
  // issued with dma16_async (the caller waits with wait_vmem)
  __device__ __forceinline__ void copy_async(bf16 *dst, const bf16 *src, int valid,
                                             int wave) const;
};

// Scheduling order for a run of NP matrix products whose operands come from
// LDS reads, RPP reads per product: the first RA reads, then each product
// followed by the reads of the product RA / RPP places later (group ID as
// __builtin_amdgcn_sched_group_barrier).
template <int ID, int RA, int NP, int RPP>
__device__ __forceinline__ void read_ahead_order() {
  static_assert(RA % RPP == 0 && RA / RPP <= NP, "read-ahead");
  __builtin_amdgcn_sched_group_barrier(0x100, RA, ID);  // DS reads
#pragma unroll
  for (int i = 0; i < NP - RA / RPP; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, ID);  // one product
    __builtin_amdgcn_sched_group_barrier(0x100, RPP, ID);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, RA / RPP, ID);
}

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt left at their maximum)
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int D, int ROWS, int NW>
__device__ __forceinline__ void TileCopier<D, ROWS, NW>::init(int wave, int lane) {
#pragma unroll
  for (int jj = 0; jj < NDMA; ++jj) {
    const int e = (wave * NDMA + jj) * 512 + 8 * lane;
    const int row = e / D, pblk = (e % D) / 8;
    off[jj] = row * D * 2 + 16 * (pblk ^ swz_f<D>(row));
  }
}

template <int D, int ROWS, int NW>
__device__ __forceinline__ void TileCopier<D, ROWS, NW>::copy_async(bf16 *dst, const bf16 *src,
                                                                    int valid, int wave) const {
  // the resource covers this tile's rows only (at most ROWS, so the byte
  // count stays small whatever the sequence length)
  const int rows = valid < ROWS ? valid : ROWS;
  const u32x4 r = rsrc_words(src, rows * D * 2);
#pragma unroll
  for (int jj = 0; jj < NDMA; ++jj) dma16_async(r, dst + (wave * NDMA + jj) * 512, off[jj]);
}

// s_waitcnt vmcnt(n) for a compile-time n < 16
template <int n>
__device__ __forceinline__ void wait_vmem_n() {
  static_assert(n >= 0 && n < 16, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | n);
}

// Token predicate of the mask as runs (used inside the tiles a token-exact
// layout marks partial).  For a query at in-frame position a of frame i, the
// allowed keys of frame j are one run of positions: all of frame 0 with the
// sink; else, with delta = |i - j|, the shifted distance
// e = max(delta - d + 1, 1) for the central band d, and the band's half
// width w, the positions b with |a - b| < w, or below unit width (w == 0)
// the single position a on frame distances that are a multiple of the
// band's period (review Step 2-A..C and Step 4; paper §4.2 Fig.5, Eq.8;
// the central band and width scale of the rebuttal's ablations; the
// harmonic-series width of review Appx C.3).  The radial decay's w and
// period depend on r = floor(log2 e) only and come from a 32-entry table;
// the harmonic decay's are w = s / e and period = ceil(e / s).
// key_run returns the run as [lo, lo + len) in absolute key index (len 0
// when empty).  The predicate is symmetric in (i, a) and (j, b) except for
// the sink, which is a key-frame condition: query_run gives the allowed
// queries of query frame i for the key at position b of frame j.
struct BandCtx {
  int s, frames, central;
  bool sink, harmonic;
  const int *rtab;  // width of band r at [r], period at [32 + r]
  int kshift;       // scale 2^kshift: width s >> (kshift r) directly; else -1
  unsigned long long smagic;  // x / s == (x * smagic) >> sshift, 0 <= x < 2^31
  int sshift;
  __device__ __forceinline__ int div_s(int x) const {
    return (int)(((unsigned long long)(unsigned)x * smagic) >> sshift);
  }
};
__device__ __forceinline__ BandCtx make_band_ctx(const MaskGeom &mg, const int *rtab) {
  return BandCtx{mg.s,     mg.frames,     mg.central,  mg.sink != 0, mg.decay == 1,
                 rtab,     mg.pow2_shift, mg.s_magic,  mg.s_shift};
}
__device__ __forceinline__ void band_run(const BandCtx &c, int delta, int pos, int frame,
                                         int &lo, unsigned &len) {
  const int e = delta - c.central + 1 > 1 ? delta - c.central + 1 : 1;
  int w, r = 0;
  if (c.harmonic) {
    w = c.s / e;
  } else {
    r = 31 - __builtin_clz(e);
    if (c.kshift >= 0) {
      const int sh = c.kshift * r;
      w = sh < 31 ? (c.s >> sh) : 0;
    } else {
      w = c.rtab[r];
    }
  }
  if (w >= 1) {
    const int b0 = pos >= w ? pos - w + 1 : 0;
    const int b1 = w < c.s - pos ? pos + w : c.s;
    lo = frame * c.s + b0;
    len = (unsigned)(b1 - b0);
  } else {  // below unit width: the sampled diagonal
    const int period = c.harmonic ? c.div_s(e - 1) + 1 : c.rtab[32 + r];
    lo = frame * c.s + pos;
    len = (delta % period == 0) ? 1u : 0u;
  }
}
__device__ __forceinline__ void key_run(const BandCtx &c, int qi, int qa, int j, int &lo,
                                        unsigned &len) {
  if (c.sink && j == 0) {
    lo = 0;
    len = (unsigned)c.s;
    return;
  }
  band_run(c, qi > j ? qi - j : j - qi, qa, j, lo, len);
}
__device__ __forceinline__ void query_run(const BandCtx &c, int kj, int kb, int i, int &lo,
                                          unsigned &len) {
  if (c.sink && kj == 0) {
    lo = i * c.s;
    len = (unsigned)c.s;
    return;
  }
  band_run(c, kj > i ? kj - i : i - kj, kb, i, lo, len);
}

// x in [lo, lo + len)
__device__ __forceinline__ bool in_run(int x, int lo, unsigned len) {
  return (unsigned)(x - lo) < len;
}

// Allowed-pair bits of one lane over NB 32-wide blocks of a 32 x 32 product
// result, in the result's register layout: bit 16 kb + r stands for index
// x0 + 32 kb + 8 (r / 4) + 4 g + r % 4 of the span (g = lane / 32).  The
// span may cross any number of frames (frames shorter than the span), so
// the runs of every frame it touches are tested; indices past the last
// frame get 0.  lane_key_bits: the lane is query (qi, qa), the span is keys;
// lane_query_bits: the lane is key (kj, kb), the span is queries.
// Bits of the lane elements whose offset is below y (see lane_pair_bits):
// 4 per 8 offsets, i.e. 4 floor(y / 8) + min(y % 8, 4) of them.
template <int NB>
__device__ __forceinline__ unsigned rank_mask(int y) {
  y = y < 0 ? 0 : (y > 32 * NB ? 32 * NB : y);
  const int k = 4 * (y >> 3) + ((y & 7) < 4 ? (y & 7) : 4);
  return k >= 32 ? ~0u : (1u << k) - 1u;
}
template <int NB, bool QUERIES>
__device__ __forceinline__ unsigned lane_pair_bits(const BandCtx &c, int fi, int pos, int x0,
                                                   int g) {
  static_assert(NB >= 1 && NB <= 2, "at most 32 bits");
  const int f0 = c.div_s(x0);
  int f1 = c.div_s(x0 + 32 * NB - 1);
  f1 = f1 < c.frames - 1 ? f1 : c.frames - 1;
  unsigned ok = 0;
  for (int f = f0; f <= f1; ++f) {
    int lo;
    unsigned len;
    if constexpr (QUERIES)
      query_run(c, fi, pos, f, lo, len);
    else
      key_run(c, fi, pos, f, lo, len);
    // the lane's elements sit at offsets 32 kb + 8 (r / 4) + r % 4 from
    // x0 + 4 g, ascending with the bit index, so a run covers the bits
    // between the counts of elements below its two ends
    const int b = x0 + 4 * g;
    ok |= rank_mask<NB>(lo + (int)len - b) & ~rank_mask<NB>(lo - b);
  }
  return ok;
}
template <int NB>
__device__ __forceinline__ unsigned lane_key_bits(const BandCtx &c, int qi, int qa, int key0,
                                                  int g) {
  return lane_pair_bits<NB, false>(c, qi, qa, key0, g);
}
__device__ __forceinline__ unsigned lane_query_bits(const BandCtx &c, int kj, int kb, int row0,
                                                    int g) {
  return lane_pair_bits<1, true>(c, kj, kb, row0, g);
}

// s[kb][r] = -inf where bit 16 kb + r of ok is clear (register r of block kb
// is the lane's element of that bit, see lane_pair_bits).  Each element
// takes its bit sign-extended (all ones or zero) as a bit-select mask: two
// vector instructions per element and no compare, so no condition register
// per element (compare results held in scalar register pairs overflowed the
// scalar register file where several masks meet).
template <int NB>
__device__ __forceinline__ void mask_elems(f32x16 (&s)[NB], unsigned ok) {
  const float ninf = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < NB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int m;
      asm("v_bfe_i32 %0, %1, %2, 1" : "=v"(m) : "v"(ok), "i"(16 * kb + r));
      asm("v_bfi_b32 %0, %1, %0, %2" : "+v"(s[kb][r]) : "v"(m), "v"(ninf));
    }
}

// A running maximum that starts finite: a row whose first chunks are fully
// masked (token-exact layouts) then exponentiates -inf - m = -inf to 0
// instead of -inf + inf = NaN.
constexpr float kNoMax = -1e30f;

// Work-item order for a launch of n workgroups whose work items are
// numbered head-major (query tile fastest).  The hardware hands workgroups to
// the 8 XCDs round robin (workgroup b runs on XCD b % 8).  Work is dealt to
// the XCDs in blocks of `blk` consecutive items: XCD x takes blocks
// x, x + 8, x + 16, ... in order.  At any moment the XCDs then work on 8
// neighbouring blocks of the same head, so the key/value tiles in use across
// the chip are those of about one head (they stay in the memory-side cache)
// and the workgroups sharing one XCD's L2 work on neighbouring query tiles.
// Items past the last full round of 8 blocks keep their own index.
// Bijective on [0, n).  blk == 0: XCD x takes one contiguous range.
__device__ __forceinline__ int xcd_remap(int b, int n, int blk) {
  constexpr int X = 8;
  if (blk == 0) {
    const int q = n / X, r = n % X;
    const int x = b % X, k = b / X;
    return (x < r) ? x * (q + 1) + k : r * (q + 1) + (x - r) * q + k;
  }
  const int main_part = n / (X * blk) * (X * blk);
  if (b >= main_part) return b;
  const int x = b % X, k = b / X;
  return ((k / blk) * X + x) * blk + k % blk;
}


}  // namespace radial
