// Device-side decode arithmetic of the packed Trellis code stream (gfx950).
//
// Method: web page "mlx-bun 0.2.0 -> 0.4.0" (npm diff, page 57), section
// src/model/trellis-wide-prefill.ts, kernel body: 12-bit cyclic window at
// stream bit (255 - t)*k of the weight's 256-weight block (LSB-first words,
// the block's first word follows its last), 1MAD hash, byte sum minus 510,
// float32 reciprocal refinement by C = 147.800537109375, per-row scale, bf16.
//
// Three equivalent ways to reach the bf16 weight live here:
//   * trellis_value(): the refinement exactly as the page orders it; used to
//     build the per-workgroup 4096-entry window -> value table and by the
//     materialising decode kernel;
//   * the table path: value = table[window], weight = bf16(value * scale);
//   * the ALU path: weight = bf16(float(code) * q), q = float32(scale * r),
//     r = float32(1/C). For every code in [-510, 510] and every bf16 scale
//     mantissa this gives the same bf16 as the page's chain (checked
//     exhaustively on the CPU and, for the GPU, by the decode tests); scaling
//     by a power of two commutes with every rounding involved as long as all
//     intermediates stay normal, which holds for 2^-110 <= |scale| <= 2^110.
//     Rows whose scale lies outside that range (or is not finite) use the
//     table path only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace trellis {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kC = 147.800537109375f;
constexpr float kR = 1.0f / kC;  // IEEE division folded at compile time

// 1MAD hash of a 12-bit window: win * 34038481 + 76625530 (mod 2^32).
// 34038481 = 2*2^24 + 0x0762D1, so for win < 2^24 the product is one
// 24-bit multiply-add plus (win << 25): two full-rate VALU ops instead of a
// quarter-rate 32-bit multiply.
__device__ __forceinline__ uint32_t hash_1mad(uint32_t win) {
  uint32_t t, z;
  asm("v_mad_u32_u24 %0, %1, %2, %3" : "=v"(t) : "v"(win), "s"(0x0762D1u), "v"(76625530u));
  asm("v_lshl_add_u32 %0, %1, 25, %2" : "=v"(z) : "v"(win), "v"(t));
  return z;
}

// Byte sum of the hash minus 510. v_sad_u8(z, 0, acc) adds the four bytes of
// z to acc; acc = -510 (mod 2^32) yields the signed code.
__device__ __forceinline__ int code_of(uint32_t win) {
  return (int)__builtin_amdgcn_sad_u8(hash_1mad(win), 0u, 0xFFFFFE02u);
}

// 1.5*2^23 + code as a float: v_sad_u8 adds the byte sum to the bit pattern
// 0x4B3FFE02 = bits(1.5*2^23) - 510, and 1.5*2^23 + code stays inside the
// binade [2^23, 2^24) where the float spacing is 1.
__device__ __forceinline__ float code_plus_magic(uint32_t win) {
  return __uint_as_float(__builtin_amdgcn_sad_u8(hash_1mad(win), 0u, 0x4B3FFE02u));
}
constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23

// ALU-path row constants: q = float32(s * r) rounded to the nearest multiple
// of 4 units in its last place, so K = -1.5*2^23 * q is exact and
// fma(1.5*2^23 + code, q, K) rounds code*q exactly once. For every code and
// every bf16 scale mantissa (either sign) bf16(code * q) equals the page's
// weight (zero weights may differ in sign only).
__device__ __forceinline__ void alu_row_constants(float s, float &q, float &k) {
  q = __uint_as_float((__float_as_uint(s * kR) + 2u) & ~3u);
  k = -kMagic * q;
}

// (v >> 16) & m in one VALU op (SDWA word select on the first operand).
__device__ __forceinline__ uint32_t and_hi16(uint32_t v, uint32_t m) {
  uint32_t r;
  asm("v_and_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1 src1_sel:DWORD"
      : "=v"(r)
      : "v"(v), "v"(m));
  return r;
}

// The page's normalisation: a = c*r, residual = fma(-a, C, c), a + residual*r.
__device__ __forceinline__ float trellis_value(int code) {
  const float c = (float)code;
  const float a = c * kR;
  const float residual = __builtin_fmaf(-a, kC, c);
  return __builtin_fmaf(residual, kR, a);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Scales for which the ALU path is exact (see the file comment).
__device__ __forceinline__ bool alu_scale_ok(float s) {
  const float a = __builtin_fabsf(s);
  return a == 0.0f || (a >= 0x1p-110f && a <= 0x1p110f);
}

// ---- window extraction from a lane's registers ----------------------------
// D[] holds consecutive code words of one block (LSB-first); O is the bit
// offset of the window's lowest bit inside D (compile-time).

// The 12-bit window itself.
template <int O, int N>
__device__ __forceinline__ uint32_t win12(const uint32_t (&D)[N]) {
  constexpr int w = O >> 5, b = O & 31;
  static_assert(w < N, "window start outside the lane's words");
  if constexpr (b + 12 <= 32) {
    return __builtin_amdgcn_ubfe(D[w], b, 12);
  } else {
    static_assert(w + 1 < N, "straddling window needs the next word");
    return __builtin_amdgcn_alignbit(D[w + 1], D[w], b) & 0xFFFu;
  }
}

// The window times 2^SH: the byte address of its entry in a table of
// 2^SH-byte entries (SH = 2: float values, SH = 1: float16 codes).
template <int O, int SH, int N>
__device__ __forceinline__ uint32_t win_xa(const uint32_t (&D)[N]) {
  constexpr int w = O >> 5, b = O & 31;
  constexpr uint32_t m = 0xFFFu << SH;
  static_assert(w < N, "window start outside the lane's words");
  if constexpr (b >= SH) {
    if constexpr (b + 12 <= 32) {
      return (D[w] >> (b - SH)) & m;
    } else {
      static_assert(w + 1 < N, "straddling window needs the next word");
      return __builtin_amdgcn_alignbit(D[w + 1], D[w], b - SH) & m;
    }
  } else {
    return (D[w] << (SH - b)) & m;
  }
}

// Table byte addresses (window * 2^SH) of the four windows whose lowest
// bits are at O0, O0+16, O0+32 and O0+48: two words holding stream bits
// [O0-SH, O0-SH+64) are built once, and each address is one mask of their
// low or high halves (mask = 0xFFF << SH in a register, for the SDWA form).
template <int O0, int SH, int N>
__device__ __forceinline__ void quad_xa(const uint32_t (&D)[N], uint32_t mask, uint32_t (&a)[4]) {
  constexpr int sh = O0 - SH;
  constexpr uint32_t m = 0xFFFu << SH;
  uint32_t lo, hi;
  if constexpr (sh < 0) {
    static_assert(sh >= -2, "unexpected window offset");
    lo = D[0] << (-sh);
    hi = __builtin_amdgcn_alignbit(D[1], D[0], 32 + sh);
  } else {
    constexpr int w = sh >> 5, r = sh & 31;
    if constexpr (r == 0) {
      static_assert(w + 1 < N, "quad outside the lane's words");
      lo = D[w];
      hi = D[w + 1];
    } else {
      static_assert(w + 2 < N, "quad outside the lane's words");
      lo = __builtin_amdgcn_alignbit(D[w + 1], D[w], r);
      hi = __builtin_amdgcn_alignbit(D[w + 2], D[w + 1], r);
    }
  }
  a[0] = lo & m;
  a[1] = and_hi16(lo, mask);
  a[2] = hi & m;
  a[3] = and_hi16(hi, mask);
}

// ---- float16 code table -----------------------------------------------------
// Entries 2p and 2p + 1 of the 4096-entry window -> code table as one word
// (every code in [-510, 510] is exact in float16).
__device__ __forceinline__ uint32_t code_entry_pair(uint32_t p) {
  const float lo = (float)code_of(2 * p), hi = (float)code_of(2 * p + 1);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// ---- k = 2 pair table -------------------------------------------------------
// For k = 2 the windows of weights idx and idx + 1 (idx even) overlap in 10
// bits: the 14 stream bits from the lower window's start hold both. A
// 16384-entry table indexed by those 14 bits gives both codes at once, as
// two float16 values (every code in [-510, 510] is exact in float16): the
// high half holds the code of the upper 12 bits (weight idx), the low half
// that of the lower 12 bits (weight idx + 1).
__device__ __forceinline__ uint32_t pair_entry(uint32_t p) {
  const float hi = (float)code_of(p >> 2), lo = (float)code_of(p & 0xFFFu);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

// Table byte addresses (pair * 4) of the two 14-bit pair fields whose lowest
// bits are at O0 and O0 + 16: one word holding stream bits [O0-2, O0+30) is
// built, and each address is one mask of its low or high half.
template <int O0, int N>
__device__ __forceinline__ void pair_x4(const uint32_t (&D)[N], uint32_t mask, uint32_t (&a)[2]) {
  constexpr int sh = O0 - 2;
  uint32_t w;
  if constexpr (sh < 0) {
    static_assert(sh == -2, "unexpected pair offset");
    w = D[0] << 2;
  } else {
    constexpr int wi = sh >> 5, r = sh & 31;
    if constexpr (r == 0) {
      w = D[wi];
    } else {
      static_assert(wi + 1 < N, "pair outside the lane's words");
      w = __builtin_amdgcn_alignbit(D[wi + 1], D[wi], r);
    }
  }
  a[0] = w & 0xFFFCu;
  a[1] = and_hi16(w, mask);
}

// float32(code * q) from the low or high float16 half of a pair entry, one
// fused multiply-add of mixed precision (the code converts exactly).
__device__ __forceinline__ float mix_lo(uint32_t h2, float q) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h2), "v"(q));
  return r;
}
__device__ __forceinline__ float mix_hi(uint32_t h2, float q) {
  float r;
  asm("v_fma_mix_f32 %0, %1, %2, 0 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(h2), "v"(q));
  return r;
}

}  // namespace trellis
