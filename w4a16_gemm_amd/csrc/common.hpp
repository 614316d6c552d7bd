// Device-side helpers shared by the gfx950 kernels: vector types, MFMA wrappers,
// nibble unpacking and the exact int4 -> fp16 dequantization.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4 {

typedef _Float16 half_t;
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef int int4_t __attribute__((ext_vector_type(4)));
typedef int int16_t_ __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- MFMA
// v_mfma_f32_16x16x32_f16: D[16x16] += A[16x32] * B[32x16].  Lane l holds A row
// (l % 16), B column (l % 16), and 8 K-elements (a K-slot) each; the same K-slot
// assignment is used for A and B, so any consistent mapping of real k indices to
// (lane / 16, element) gives the same product.  D: lane l holds column l % 16,
// rows 4 * (l / 16) + r, r = 0..3.
__device__ __forceinline__ float4_t mfma16(half8_t a, half8_t b, float4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_f16: D[32x32] += A[32x16] * B[16x32].  Lane l holds A row
// (l % 32), B column (l % 32), 8 K-elements each.  D: lane l holds column l % 32,
// rows 8 * (r / 4) + 4 * (l / 32) + (r % 4), r = 0..15.
__device__ __forceinline__ float16_t mfma32(half8_t a, half8_t b, float16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// int8: v_mfma_i32_16x16x64_i8 (16 K-bytes per lane) and v_mfma_i32_32x32x32_i8.
__device__ __forceinline__ int4_t mfma16_i8(int4_t a, int4_t b, int4_t c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int16_t_ mfma32_i8(int4_t a, int4_t b, int16_t_ c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

// 16-byte load of data read exactly once per call (the packed weights of the decode
// kernels), marked non-temporal: it streams through L2 and the Infinity Cache without
// displacing what the other workgroups re-read (X, scales, zero points).  A read-only
// stream of the decode weights' sizes runs 4-10 % faster with the hint.
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// ----------------------------------------------------- tiled weight layout
// Packed weights are stored in 1 KB blocks of 16 rows x 128 k (one group): block
// (n / 16, g) holds, for slot = 0..3 (32 k each) and row r = n % 16, the four words
// 4 slot .. 4 slot + 3 of that row's group at word offset 64 slot + 4 r.  The array is
// int32 [ceil(N/16), K/128, 4, 16, 4]; one wave reading lane l -> chunk l reads a
// contiguous 1 KB block (rows l % 16, slot l / 16).  Returns the word offset of the
// 16-byte chunk (row n, group g, slot); ng = K / 128.
__device__ __forceinline__ int64_t tiled_chunk(int n, int g, int slot, int ng) {
  return ((int64_t)((n >> 4) * ng + g) * 4 + slot) * 64 + (n & 15) * 4;
}

// ------------------------------------------------------ nibble unpacking
// A W4A16 code word holds 8 consecutive elements e_0..e_7 split by parity: e_0, e_2,
// e_4, e_6 in nibbles 0..3 (the low half-word), e_1, e_3, e_5, e_7 in nibbles 4..7.
// Masking the word with 0x000f000f puts e_0 and e_1 each in the low mantissa bits of
// one half; ORing in 0x6400 (fp16 1024, unit steps) makes them fp16 1024 + e exactly.
// Masking with 0x00f000f0 puts e_2 and e_3 in mantissa bits 4..7, which under fp16 64
// (0x5400, steps of 1/16) are worth 64 + e exactly.  The word shifted right by 8 gives
// e_4, e_5 and e_6, e_7 the same way: four registers of fp16 pairs in natural element
// order, (1024 + e_0, 1024 + e_1), (64 + e_2, 64 + e_3), (1024 + e_4, 1024 + e_5),
// (64 + e_6, 64 + e_7), in one shift and four v_and_or_b32.
// (x & mask) | bits in one v_and_or_b32.  VOP3 encodings on gfx9 take no literal
// constants, so with literal operands the expression compiles to a separate v_and_b32
// and v_or_b32.  The constants are therefore passed through vreg(), an empty asm that
// hides their value: the compiler then keeps them in registers (hoisted out of loops)
// and selects v_and_or_b32 itself.  The instruction stays compiler-generated, so the
// hazard checks around in-flight MFMAs (a VALU write to an MFMA source needs wait
// states) apply to it; hand-written VALU asm would escape them.
__device__ __forceinline__ uint32_t vreg(uint32_t c) {
  asm("" : "+v"(c));
  return c;
}
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t bits) {
  return (x & mask) | bits;
}

// The magic constants of the expansion, held in registers: masks 0x000f000f (mlo),
// 0x00f000f0 (mhi), fp16 pairs 1024 (e1024) and 64 (e64).
struct Magic {
  uint32_t mlo, mhi, e1024, e64;
};
__device__ __forceinline__ Magic magic_regs() {
  return Magic{vreg(0x000f000fu), vreg(0x00f000f0u), vreg(0x64006400u), vreg(0x54005400u)};
}
__device__ __forceinline__ u32x4 expand_word(uint32_t w, const Magic& c) {
  const uint32_t w8 = w >> 8;
  u32x4 r;
  r[0] = and_or(w, c.mlo, c.e1024);   // 1024 + e0, 1024 + e1
  r[1] = and_or(w, c.mhi, c.e64);     //   64 + e2,   64 + e3
  r[2] = and_or(w8, c.mlo, c.e1024);  // 1024 + e4, 1024 + e5
  r[3] = and_or(w8, c.mhi, c.e64);    //   64 + e6,   64 + e7
  return r;
}

// Exact dequantization of one word: ((1024 + q) - (1024 + z)) and ((64 + q) - (64 + z))
// are the exact integer q - z in fp16, then one multiply by the fp16 scale: a single
// rounding per element.  c1024 = -(1024 + z) and c64 = -(64 + z) in both halves (bit
// patterns 0xE400 | z and 0xD400 | 16 z), s2 = scale in both halves.
__device__ __forceinline__ half8_t dequant8(uint32_t w, const Magic& c, half2_t c1024, half2_t c64, half2_t s2) {
  const u32x4 r = expand_word(w, c);
  half2_t p0 = __builtin_bit_cast(half2_t, (uint32_t)r[0]);
  half2_t p1 = __builtin_bit_cast(half2_t, (uint32_t)r[1]);
  half2_t p2 = __builtin_bit_cast(half2_t, (uint32_t)r[2]);
  half2_t p3 = __builtin_bit_cast(half2_t, (uint32_t)r[3]);
  p0 = (p0 + c1024) * s2;
  p1 = (p1 + c64) * s2;
  p2 = (p2 + c1024) * s2;
  p3 = (p3 + c64) * s2;
  return half8_t{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}
// -(1024 + z) and -(64 + z) in both halves of a register, and s twice, as bit patterns.
__device__ __forceinline__ half2_t neg1024z2(uint32_t z) {
  return __builtin_bit_cast(half2_t, (0xE400u | z) * 0x00010001u);
}
__device__ __forceinline__ half2_t neg64z2(uint32_t z) {
  return __builtin_bit_cast(half2_t, (0xD400u | (z << 4)) * 0x00010001u);
}
__device__ __forceinline__ half2_t scale2(uint32_t sbits) {
  return __builtin_bit_cast(half2_t, sbits * 0x00010001u);
}

__device__ __forceinline__ half2_t splat2(half_t h) { return half2_t{h, h}; }

// W4A8 code words hold 8 biased nibbles b = q + 8 split by halves: elements e_0..e_3 in
// nibbles 0, 2, 4, 6 and e_4..e_7 in nibbles 1, 3, 5, 7.
//
// Biased int4 -> 16 * q as int8 bytes, natural order: b ^ 8 is the 4-bit two's
// complement of q, and placed in the high nibble of a byte it is the int8 value 16 q
// exactly.  Shifting the even nibbles up (and masking) gives e_0..e_3 as bytes, masking
// the odd ones in place gives e_4..e_7: four VALU operations, no byte permutation.
__device__ __forceinline__ void unpack_i4x16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t t = w ^ 0x88888888u;
  lo = (t << 4) & 0xf0f0f0f0u;  // bytes 16 q0, 16 q1, 16 q2, 16 q3
  hi = t & 0xf0f0f0f0u;         // bytes 16 q4, 16 q5, 16 q6, 16 q7
}

// Biased int4 times a per-group int8 scale s -> int8 bytes q * s (|q s| <= 127 is
// guaranteed by the weight rule), natural order, as two words (elements 0..3, 4..7).
// The products are formed in 16-bit lanes: (b * s + (-8 s)) mod 2^16 is q * s as int16,
// whose low byte is the int8 value; the nibble pairs (0, 4), (1, 5), (2, 6), (3, 7) of
// the word hold elements (0, 2), (4, 6), (1, 3), (5, 7).  Pairs (2, 6) and (3, 7) are
// masked in place at bits 8..11 of each half (256 b): (256 b s + 256 (-8 s)) mod 2^16 is
// 256 ((q s) mod 256), so their products land in the high byte of each 16-bit lane with
// no shift.  One v_perm_b32 per half then gathers the low bytes of one product word and
// the high bytes of the other (11 VALU operations per word).  sp = (s, s),
// cp = (-8 s, -8 s) as u16 pairs.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void unpack_i4_scaled(uint32_t w, u16x2 sp, u16x2 cp, uint32_t& lo, uint32_t& hi) {
  const uint32_t ws = w >> 4;
  const u16x2 cp8 = cp << (unsigned short)8;                       // 256 (-8 s) mod 2^16
  const u16x2 e0 = __builtin_bit_cast(u16x2, w & 0x000f000fu);     // b0, b2
  const u16x2 e1 = __builtin_bit_cast(u16x2, ws & 0x000f000fu);    // b4, b6
  const u16x2 e2 = __builtin_bit_cast(u16x2, w & 0x0f000f00u);     // 256 b1, 256 b3
  const u16x2 e3 = __builtin_bit_cast(u16x2, ws & 0x0f000f00u);    // 256 b5, 256 b7
  const uint32_t r0 = __builtin_bit_cast(uint32_t, (u16x2)(e0 * sp + cp));
  const uint32_t r1 = __builtin_bit_cast(uint32_t, (u16x2)(e1 * sp + cp));
  const uint32_t r2 = __builtin_bit_cast(uint32_t, (u16x2)(e2 * sp + cp8));
  const uint32_t r3 = __builtin_bit_cast(uint32_t, (u16x2)(e3 * sp + cp8));
  lo = __builtin_amdgcn_perm(r2, r0, 0x07020500u);  // p0 p1 p2 p3
  hi = __builtin_amdgcn_perm(r3, r1, 0x07020500u);  // p4 p5 p6 p7
}

// ------------------------------------------------------------ reductions
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// --------------------------------------- per-column values in the MFMA layout
// Per-column values (scales, zero points, group scales) of a workgroup's T 16-column
// n-tiles are loaded once per 64 columns (a column per lane) and moved to the MFMA
// output layout with lane swaps; kChunks<T> such loads cover T n-tiles.
template <int T>
constexpr int kChunks = (T + 3) / 4;

// Column (within the workgroup's 16 T) whose scale and zero point lane `lane` loads in
// chunk c: 64 c + lane for T >= 3 (past column 16 T - 1 the values are never used); for
// T = 1, 2 the 16 T columns repeat over the lanes.
template <int T>
__device__ __forceinline__ int chunk_col(int c, int lane) {
  return 64 * c + (lane & (T == 1 ? 15 : T == 2 ? 31 : 63));
}

// v holds, in 16-lane row r of chunk c, the value of n-tile 4 c + r (rows repeat for
// T < 4); w[t] gets n-tile t's values in every row (lane l: column 16 t + l % 16).
// v_permlane32_swap of two copies gives rows (0,1,0,1) and (2,3,2,3); v_permlane16_swap
// of two copies of each gives a row repeated four times in each result.
template <int T>
__device__ __forceinline__ void rows_to_tiles(const uint32_t (&v)[kChunks<T>], uint32_t (&w)[T]) {
  if constexpr (T == 1) {
    w[0] = v[0];
  } else if constexpr (T == 2) {
    const auto p = __builtin_amdgcn_permlane16_swap(v[0], v[0], false, false);
    w[0] = p[0];
    w[1] = p[1];
  } else {
#pragma unroll
    for (int c = 0; c < kChunks<T>; ++c) {
      const auto h = __builtin_amdgcn_permlane32_swap(v[c], v[c], false, false);
      const auto p = __builtin_amdgcn_permlane16_swap(h[0], h[0], false, false);
      const auto q = __builtin_amdgcn_permlane16_swap(h[1], h[1], false, false);
      // (T not a multiple of 4: the last chunk's rows past tile T - 1 are dropped)
      w[4 * c] = p[0];
      if (4 * c + 1 < T) w[4 * c + 1] = p[1];
      if (4 * c + 2 < T) w[4 * c + 2] = q[0];
      if (4 * c + 3 < T) w[4 * c + 3] = q[1];
    }
  }
}

// Workgroup -> tile remapping for 8 XCDs.  Workgroups are handed to the XCDs round
// robin (id % 8); this returns a logical id such that the workgroups one XCD runs are
// consecutive logical ids, so neighbouring tiles share that XCD's L2.
__device__ __forceinline__ int xcd_remap(int id, int total) {
  const int per = total / 8;
  if (per == 0 || id >= per * 8) return id;
  return (id % 8) * per + id / 8;
}

}  // namespace w4
