// Packed Trellis-quantized linear layer for narrow-batch prefill, gfx950.
//
// Method: web page "mlx-bun 0.2.0 -> 0.4.0" (npm diff, page 57), section
// src/model/trellis-wide-prefill.ts -- Metal kernel body (window extraction,
// 1MAD hash, byte sum, reciprocal-refinement normalisation, per-row scale,
// bf16 rounding, narrow-M dot product) and host wrapper (shape checks). The
// materialising decode is the "expand" mode of page "mlx-bun 0.4.0 -> 0.5.0"
// (npm diff, page 26), section src/model/trellis-linear.ts. The fused gate/up
// tail follows page "mlx-bun 0.0.4" (npm, page 62), section
// src/model/minicpm5.ts (MLP forward).
//
// CDNA4 design (not a translation of the Metal kernel):
//   * one persistent workgroup of 16 waves per CU; the work is a list of
//     units (16-row tile x one 256-weight block), split evenly over
//     workgroups and then into 16 contiguous pieces whose lengths differ by at
//     most one unit per SIMD (stream-K); waves rank themselves by the work
//     they have left;
//   * x is staged once per workgroup in LDS (a K panel of it when all of x
//     does not fit), read and written through per-row pointers so packed
//     inputs need no copy;
//   * each lane reads the code words of 64 consecutive weights of one row
//     through a buffer descriptor and decodes them in registers, part of them
//     through an LDS table (window -> value, window -> float16 code, or for
//     k = 2 a 14-bit pair of windows -> two codes) and part with ALU
//     arithmetic, so LDS and VALU work in parallel;
//   * bf16 MFMA 16x16x32: A = x (rows past M repeat row M-1 and feed output
//     rows that are never stored), B = W^T (16 rows);
//   * tiles shared by pieces of one workgroup are summed through LDS, tiles
//     shared with other workgroups through a workspace, in a fixed order
//     either way, the last contributor (per-tile counter) writing bf16;
//   * the fused gate/up variant decodes each block of both matrices against
//     the same x into two accumulators, so the wave that completes a tile
//     writes the elementwise tail itself.
//
// Build flags that matter for exactness: -ffp-contract=off.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <map>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <thread>
#include <utility>
#include <vector>

#include "decode.hpp"
#include "trellis.h"
#include "trellis_testing.h"

namespace trellis {
namespace {

constexpr int kWave = 64;
constexpr int kMaxRows = 16;               // row-pointer slots (m <= 15)
constexpr int kRowTableBytes = kMaxRows * 8;  // LDS copy of the output row pointers
constexpr int kWaves = 16;                 // waves per prefill workgroup (4 per SIMD)
constexpr int kWgThreads = kWave * kWaves;
// LDS decode tables: window -> float value (4096 x 4 bytes), window ->
// float16 code (4096 x 2 bytes), or for k = 2 a 14-bit pair of windows ->
// two float16 codes (16384 x 4 bytes).
enum TableKind { kValueTable = 0, kCodeTable = 1, kPairTable = 2 };
constexpr int table_bytes(int tab) { return tab == kPairTable ? 16384 * 4 : tab == kCodeTable ? 4096 * 2 : 4096 * 4; }
constexpr int kMaxLds = 160 * 1024;        // gfx950 LDS per workgroup
constexpr int kMinLds = 82 * 1024;         // > half the LDS: one workgroup per CU
constexpr int kStageRegs = 10;             // x-staging vectors (16 B) per thread
constexpr int kCombineBytes = kWaves * 2 * kWave * 16;  // LDS partial tiles of the end-of-kernel combine
                                                        // (per matrix: twice that for gate and up)
constexpr int kCombineCounters = kWaves * 4;             // LDS counters of the barrier-free combine
static_assert(kStageRegs * kWgThreads * 16 >= kMaxLds - table_bytes(kCodeTable), "x staging must cover the largest panel");
static_assert(kStageRegs * kWgThreads <= 32 << 9, "staged x vector indices divide by the row length with 9-bit quotients");

// ---------------------------------------------------------------------------
// trellis_decode: W[N, K] bf16. One thread per 8 consecutive weights of one
// row, one 16-byte store each. Weights t = 8q .. 8q+7 of a block start at
// stream bits (255 - t)*BITS; weight 8q+7 is the lowest, at (248 - 8q)*BITS,
// and the eight windows span 7*BITS + 12 <= 40 bits, inside the 64-bit pair
// of the start word and the next word of the same block (cyclic).
// ---------------------------------------------------------------------------
template <int BITS>
__global__ __launch_bounds__(256) void decode_kernel(const uint32_t *__restrict__ codes,
                                                     const uint16_t *__restrict__ scales, int n, int k,
                                                     uint16_t *__restrict__ w) {
  constexpr int wpb = 8 * BITS;
  const int groups_per_row = k >> 3;
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= (int64_t)n * groups_per_row) return;
  const int row = (int)(gid / groups_per_row);
  const int c8 = (int)(gid - (int64_t)row * groups_per_row);
  const int q = c8 & 31;
  const uint32_t *bw = codes + (int64_t)row * (k >> 8) * wpb + (int64_t)(c8 >> 5) * wpb;
  const int start = (248 - 8 * q) * BITS;
  const int d = start >> 5, off = start & 31;
  const uint64_t f = ((uint64_t)bw[d + 1 == wpb ? 0 : d + 1] << 32) | (uint64_t)bw[d];
  const float scale = bf16_bits_to_f32(scales[row]);
  bf16x8 v;
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const uint32_t win = (uint32_t)(f >> (off + (7 - s) * BITS)) & 0xFFFu;
    v[s] = (__bf16)(trellis_value(code_of(win)) * scale);
  }
  *reinterpret_cast<bf16x8 *>(w + (int64_t)row * k + (int64_t)c8 * 8) = v;
}

// ---------------------------------------------------------------------------
// trellis_prefill
// ---------------------------------------------------------------------------

// Rows of x and of the output, one pointer each: row i of x is
// x[i][0 .. K), row i of the output out[i][0 .. N). Rows of one
// array are consecutive for a plain call; packed calls gather rows of
// several arrays. Entries past m are unused.
struct RowPtrs {
  const uint16_t *x[kMaxRows];
  uint16_t *out[kMaxRows];
};

// Work partition, computed on the host and re-derived by every wave.
struct Plan {
  int32_t m, n, k;
  int32_t tiles;     // ceil(N / 16)
  int32_t panels;    // K panels (x panel staged per workgroup)
  int32_t kp;        // 256-weight blocks per panel
  int32_t groups;    // workgroups per panel
  int32_t maxc;      // contributor slots per (tile, panel) in the workspace
  int32_t x_stride;  // bytes per staged x row
  int32_t lds_bytes;
  int32_t units;     // tiles * kp (per panel), < 2^28; with two matrices a unit is the
                     // same block of both
  int32_t cq;        // units / groups: every workgroup gets cq or cq + 1 units
  int32_t cr;        // units % groups: the first cr workgroups get cq + 1
  uint32_t xmul, xshift;  // row of a staged x vector idx: ((idx >> 5) * xmul) >> xshift
  int32_t x_contiguous;  // 1: x row i is at row 0 + i * K (plain calls); 0: per-row pointers
  int32_t slots_off;     // > 0: byte offset of dedicated partial-tile slots after x (LDS combine
                         // without barriers); 0: slots reuse the x region after a barrier
  // Multipliers for exact division (div_by) by the divisors that locating a
  // unit's piece needs: [0] cq + 1, [1] cq, [2] base + 1 and [3] base of a
  // workgroup with cq + 1 units, [4] and [5] the same with cq units; and by
  // [6] panels and [7] kp (a workgroup's panel, a unit's tile).
  uint32_t dm[8];
  uint32_t dl, dl2;  // their shifts l, 5 bits each, [0..5] and [6..7] (l = 0: the divisor is 1)
  // Tile t's counter is word t << cshift of the counter array: 64 bytes
  // apart for allocated workspaces, so the atomics on different tiles at the
  // end of a launch do not queue behind each other on one cache line
  // (measured 0.2 us per launch at M = 15, K = 17408), and packed (0) in the
  // fixed scratch of the no-allocation entry point.
  int32_t cshift;
};

// n / d (unsigned, any 32-bit n) for a divisor whose multiplier the host
// computed as m = floor(2^32 (2^l - d) / d) + 1 with l = ceil(log2 d): with
// t = umulhi(n, m), n / d = (t + ((n - t) >> 1)) >> (l - 1). The round-up
// multiplier method (Granlund and Montgomery, "Division by invariant
// integers using multiplication", 1994): a multiply-high, a subtract and
// three shifts and adds on the scalar unit, where a division by a runtime
// value would be a chain of about twenty instructions through the VALU's
// reciprocal.
__device__ __forceinline__ uint32_t div_magic(uint32_t n, uint32_t m, uint32_t l) {
  const uint32_t t = __umulhi(n, m);
  return l == 0 ? n : (t + ((n - t) >> 1)) >> ((l - 1) & 31u);
}
template <int I>
__device__ __forceinline__ uint32_t div_by(uint32_t n, const Plan &pl) {
  return div_magic(n, pl.dm[I], ((I < 6 ? pl.dl : pl.dl2) >> (5 * (I % 6))) & 31u);
}

// Split of a workgroup's contiguous units [u0, u0 + len) into s <= 16
// pieces, one per wave. Wave slot w decodes the piece at position
// w / 2 when w is even and s - 1 - w / 2 when w is odd: the lowest slots --
// which a SIMD serves first -- take both ends of the range, where the tiles
// shared with other workgroups lie. Slots 0 .. r-1 (r = len % s) get one unit
// more than the others; consecutive slots sit on different SIMDs, so every
// SIMD's load is within one unit of the others'. In position order the
// lengths are base + 1 for [0, ce), base for [ce, s - h) and base + 1 for
// [s - h, s), with ce = ceil(r / 2) and h = floor(r / 2).
struct CuSplit {
  int u0, len, s, base, ce, h;
};

__device__ __forceinline__ CuSplit cu_split(int c, const Plan &pl) {
  CuSplit q;
  q.u0 = c * pl.cq + (c < pl.cr ? c : pl.cr);
  q.len = pl.cq + (c < pl.cr ? 1 : 0);
  q.s = q.len < kWaves ? q.len : kWaves;
  q.base = q.s == kWaves ? (int)((uint32_t)q.len / kWaves) : q.len > 0 ? 1 : 0;  // len / s
  const int r = q.len - q.base * q.s;
  q.ce = (r + 1) >> 1;
  q.h = r >> 1;
  return q;
}

// First unit of the piece at position p (0 <= p <= s).
__device__ __forceinline__ int piece_start(const CuSplit &q, int p) {
  const int tail = p - (q.s - q.h);
  return q.u0 + p * q.base + (p < q.ce ? p : q.ce) + (tail > 0 ? tail : 0);
}

// Position of the piece holding unit q.u0 + o (0 <= o < q.len) in the split q
// of workgroup c: pieces of base + 1 units (the first ce and the last h) and
// of base units.
__device__ __forceinline__ int piece_in(const CuSplit &q, int c, int o, const Plan &pl) {
  const int x1 = q.ce * (q.base + 1), x2 = x1 + (q.s - q.h - q.ce) * q.base;
  // this workgroup's base + 1 and base (the divisors differ with its length)
  const bool lng = c < pl.cr;
  const uint32_t m1 = lng ? pl.dm[2] : pl.dm[4], l1 = (pl.dl >> (lng ? 10 : 20)) & 31u;
  const uint32_t m0 = lng ? pl.dm[3] : pl.dm[5], l0 = (pl.dl >> (lng ? 15 : 25)) & 31u;
  if (o < x1) return (int)div_magic((uint32_t)o, m1, l1);
  if (o < x2) return q.ce + (int)div_magic((uint32_t)(o - x1), m0, l0);
  return q.s - q.h + (int)div_magic((uint32_t)(o - x2), m1, l1);
}

// Global index (workgroup * 16 + position) of the piece holding unit u;
// consecutive pieces in unit order have consecutive indices.
__device__ __forceinline__ int piece_of(int u, const Plan &pl) {
  const int cut = pl.cr * (pl.cq + 1);
  const int c = u < cut ? (int)div_by<0>((uint32_t)u, pl) : pl.cr + (int)div_by<1>((uint32_t)(u - cut), pl);
  const CuSplit q = cu_split(c, pl);
  return c * kWaves + piece_in(q, c, u - q.u0, pl);
}

// Lane (j, g) of a wave: j = row of the 16-row tile (B column) and x row (A
// row); g = k-group. For each block the lane owns stream bits
// [64*BITS*g, 64*BITS*(g+1)) -- words [2*BITS*g, 2*BITS*(g+1)) -- plus the
// next word of the block (cyclic) for the windows that run past its range.
// Those are the windows of weights t = 192 - 64g + idx, idx = 0..63: weight
// idx sits at local bit (63 - idx)*BITS. MFMA group u (0..7) takes
// idx = 8u .. 8u+7 for both A and B, so x and W meet at the same k.
template <int BITS>
struct LaneWords {
  uint32_t d[2 * BITS + 1];
};

// Code words are read through a buffer resource whose base is the unit's
// block in the tile's first row and whose size ends at the last valid row:
// every lane's offset is then a per-lane constant (j * row bytes + its word
// range), the unit's position is scalar, and the rows past N of the last
// tile fall outside the range, which the hardware reads as zero.
constexpr int kRawBufferWord3 = 0x00020000;  // gfx9 raw-buffer descriptor word 3

template <int BITS>
__device__ __forceinline__ void load_words(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t off_next,
                                           LaneWords<BITS> &L) {
  if constexpr (BITS == 4) {
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    const auto b = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16, 0, 0);
    L.d[0] = a[0]; L.d[1] = a[1]; L.d[2] = a[2]; L.d[3] = a[3];
    L.d[4] = b[0]; L.d[5] = b[1]; L.d[6] = b[2]; L.d[7] = b[3];
  } else if constexpr (BITS == 3) {
    const auto a = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    const auto b = __builtin_amdgcn_raw_buffer_load_b64(r, off + 8, 0, 0);
    const auto c = __builtin_amdgcn_raw_buffer_load_b64(r, off + 16, 0, 0);
    L.d[0] = a[0]; L.d[1] = a[1]; L.d[2] = b[0]; L.d[3] = b[1]; L.d[4] = c[0]; L.d[5] = c[1];
  } else {
    const auto a = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    L.d[0] = a[0]; L.d[1] = a[1]; L.d[2] = a[2]; L.d[3] = a[3];
  }
  L.d[2 * BITS] = __builtin_amdgcn_raw_buffer_load_b32(r, off_next, 0, 0);
}

// A weight from one table entry (byte address a): the value table gives
// value(window) * s, the code table float32(code * q) -- the same bf16
// weight for every scale in the ALU path's exact range.
template <int TAB> struct TableRead;
template <> struct TableRead<kValueTable> {
  static constexpr int kShift = 2;  // log2 of the entry size
  static __device__ __forceinline__ uint32_t raw(const unsigned char *table, uint32_t a) {
    return *reinterpret_cast<const uint32_t *>(table + a);
  }
  static __device__ __forceinline__ float from_raw(uint32_t r, float s, float) { return __uint_as_float(r) * s; }
  static __device__ __forceinline__ float weight(const unsigned char *table, uint32_t a, float s, float q) {
    return from_raw(raw(table, a), s, q);
  }
};
template <> struct TableRead<kCodeTable> {
  static constexpr int kShift = 1;
  static __device__ __forceinline__ uint32_t raw(const unsigned char *table, uint32_t a) {
    return *reinterpret_cast<const uint16_t *>(table + a);
  }
  static __device__ __forceinline__ float from_raw(uint32_t r, float, float q) { return mix_lo(r, q); }
  static __device__ __forceinline__ float weight(const unsigned char *table, uint32_t a, float s, float q) {
    return from_raw(raw(table, a), s, q);
  }
};

template <int BITS, int TAB, int U, int... S>
__device__ __forceinline__ bf16x8 group_table(const LaneWords<BITS> &L, const unsigned char *table, float s,
                                              float q, std::integer_sequence<int, S...>) {
  using R = TableRead<TAB>;
  const float f[8] = {R::weight(table, win_xa<(63 - 8 * U - S) * BITS, R::kShift>(L.d), s, q)...};
  bf16x8 w;
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = (__bf16)f[i];
  return w;
}

template <int BITS, int U, int... S>
__device__ __forceinline__ bf16x8 group_alu(const LaneWords<BITS> &L, float q, float k,
                                            std::integer_sequence<int, S...>) {
  const float f[8] = {__builtin_fmaf(code_plus_magic(win12<(63 - 8 * U - S) * BITS>(L.d)), q, k)...};
  bf16x8 w;
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = (__bf16)f[i];
  return w;
}

// Table-path groups sharing window extraction. Windows 16 bits apart come
// out of one pair of shifted words (quad_xa): for k = 4 they are 4 weights
// apart, so groups (U, U+1) share four quads; for k = 2 they are 8 weights
// apart, so groups U..U+3 share eight quads.
template <int BITS, int TAB, int U>
__device__ __forceinline__ void table_span(const LaneWords<BITS> &L, const unsigned char *table, float s,
                                           float q, uint32_t mask, bf16x8 *w) {
  using R = TableRead<TAB>;
  constexpr int SH = R::kShift;
  static_assert(BITS == 4 || BITS == 2, "spans exist for k = 4 and k = 2");
  constexpr int G = BITS == 4 ? 2 : 4;  // groups in the span
  constexpr int Q = 8 * G / 4;          // quads in the span
  float f[G][8];
#pragma unroll
  for (int i = 0; i < Q; ++i) {
    uint32_t a[4];
    if constexpr (BITS == 4) {
      // idx = 8U + s' + {12, 8, 4, 0}, s' = i (0..3): (group U+1, slot 4+s'),
      // (U+1, s'), (U, 4+s'), (U, s')
      switch (i) {
        case 0: quad_xa<(63 - (8 * U + 12 + 0)) * 4, SH>(L.d, mask, a); break;
        case 1: quad_xa<(63 - (8 * U + 12 + 1)) * 4, SH>(L.d, mask, a); break;
        case 2: quad_xa<(63 - (8 * U + 12 + 2)) * 4, SH>(L.d, mask, a); break;
        default: quad_xa<(63 - (8 * U + 12 + 3)) * 4, SH>(L.d, mask, a); break;
      }
      f[1][4 + i] = R::weight(table, a[0], s, q);
      f[1][i] = R::weight(table, a[1], s, q);
      f[0][4 + i] = R::weight(table, a[2], s, q);
      f[0][i] = R::weight(table, a[3], s, q);
    } else {
      // idx = 8U + s' + {24, 16, 8, 0}, s' = i (0..7): groups U+3, U+2, U+1, U at slot s'
      switch (i) {
        case 0: quad_xa<(63 - (8 * U + 24 + 0)) * 2, SH>(L.d, mask, a); break;
        case 1: quad_xa<(63 - (8 * U + 24 + 1)) * 2, SH>(L.d, mask, a); break;
        case 2: quad_xa<(63 - (8 * U + 24 + 2)) * 2, SH>(L.d, mask, a); break;
        case 3: quad_xa<(63 - (8 * U + 24 + 3)) * 2, SH>(L.d, mask, a); break;
        case 4: quad_xa<(63 - (8 * U + 24 + 4)) * 2, SH>(L.d, mask, a); break;
        case 5: quad_xa<(63 - (8 * U + 24 + 5)) * 2, SH>(L.d, mask, a); break;
        case 6: quad_xa<(63 - (8 * U + 24 + 6)) * 2, SH>(L.d, mask, a); break;
        default: quad_xa<(63 - (8 * U + 24 + 7)) * 2, SH>(L.d, mask, a); break;
      }
      f[3][i] = R::weight(table, a[0], s, q);
      f[2][i] = R::weight(table, a[1], s, q);
      f[1][i] = R::weight(table, a[2], s, q);
      f[0][i] = R::weight(table, a[3], s, q);
    }
  }
#pragma unroll
  for (int gidx = 0; gidx < G; ++gidx)
#pragma unroll
    for (int e = 0; e < 8; ++e) w[gidx][e] = (__bf16)f[gidx][e];
}

// Decode-path choice per MFMA group: bit u of MASK set = table path.
// Spans (k = 4: aligned pairs, k = 2: aligned quads) whose groups all use
// the table path share window extraction.
template <int BITS, int MASK, int U>
constexpr bool span_start() {
  if constexpr (BITS == 4) return U % 2 == 0 && ((MASK >> U) & 3) == 3;
  else if constexpr (BITS == 2) return U % 4 == 0 && ((MASK >> U) & 15) == 15;
  else return false;
}
template <int BITS, int MASK, int U>
constexpr bool in_span() {
  if constexpr (BITS == 4) return span_start<BITS, MASK, U - U % 2>();
  else if constexpr (BITS == 2) return span_start<BITS, MASK, U - U % 4>();
  else return false;
}

// k = 2 with the pair table: groups (U, U + 1), U even, share four pair
// fields per 8 weights each (16 bits apart: pair i of group U + 1 in the low
// half of a shifted word, pair i of group U in its high half).
template <int U, int N>
__device__ __forceinline__ void pair_span(const uint32_t (&D)[N], const unsigned char *table, float q,
                                          uint32_t mask, bf16x8 (&w)[2]) {
  float f[2][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t a[2];
    switch (i) {
      case 0: pair_x4<108 - 16 * U - 0>(D, mask, a); break;
      case 1: pair_x4<108 - 16 * U - 4>(D, mask, a); break;
      case 2: pair_x4<108 - 16 * U - 8>(D, mask, a); break;
      default: pair_x4<108 - 16 * U - 12>(D, mask, a); break;
    }
    const uint32_t g1 = *reinterpret_cast<const uint32_t *>(table + a[0]);
    const uint32_t g0 = *reinterpret_cast<const uint32_t *>(table + a[1]);
    f[1][2 * i] = mix_hi(g1, q);
    f[1][2 * i + 1] = mix_lo(g1, q);
    f[0][2 * i] = mix_hi(g0, q);
    f[0][2 * i + 1] = mix_lo(g0, q);
  }
#pragma unroll
  for (int gidx = 0; gidx < 2; ++gidx)
#pragma unroll
    for (int e = 0; e < 8; ++e) w[gidx][e] = (__bf16)f[gidx][e];
}

// The pages' arithmetic on the ALU (window, hash, byte sum, reciprocal
// refinement, scale): the exact fallback of the code- and pair-table kernels
// for rows whose scale is outside the range where code * q is exact.
template <int BITS, int U, int... S>
__device__ __forceinline__ bf16x8 group_exact(const LaneWords<BITS> &L, float s, std::integer_sequence<int, S...>) {
  const float f[8] = {(trellis_value(code_of(win12<(63 - 8 * U - S) * BITS>(L.d))) * s)...};
  bf16x8 w;
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = (__bf16)f[i];
  return w;
}

template <int BITS, int MASK, int TAB, bool EXACT, int U>
__device__ __forceinline__ void unit_group(const LaneWords<BITS> &L, const unsigned char *table,
                                           const unsigned char *xa, float s, float q, float k, uint32_t mask,
                                           f32x4 &acc) {
  if constexpr (EXACT) {
    const bf16x8 w = group_exact<BITS, U>(L, s, std::make_integer_sequence<int, 8>{});
    const bf16x8 xv = *reinterpret_cast<const bf16x8 *>(xa + 16 * U);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, w, acc, 0, 0, 0);
  } else if constexpr (TAB == kPairTable) {
    static_assert(BITS == 2, "the pair table is for k = 2");
    constexpr bool span = ((MASK >> (U - U % 2)) & 3) == 3;
    if constexpr (span && U % 2 == 0) {
      bf16x8 w[2];
      pair_span<U>(L.d, table, q, mask, w);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const bf16x8 xv = *reinterpret_cast<const bf16x8 *>(xa + 16 * (U + i));
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, w[i], acc, 0, 0, 0);
      }
    } else if constexpr (!span) {
      static_assert(((MASK >> U) & 1) == 0, "pair-table groups come in aligned pairs");
      const bf16x8 w = group_alu<BITS, U>(L, q, k, std::make_integer_sequence<int, 8>{});
      const bf16x8 xv = *reinterpret_cast<const bf16x8 *>(xa + 16 * U);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, w, acc, 0, 0, 0);
    }
  } else if constexpr (span_start<BITS, MASK, U>()) {
    constexpr int G = BITS == 4 ? 2 : 4;
    bf16x8 w[G];
    table_span<BITS, TAB, U>(L, table, s, q, mask, w);
#pragma unroll
    for (int i = 0; i < G; ++i) {
      const bf16x8 xv = *reinterpret_cast<const bf16x8 *>(xa + 16 * (U + i));
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, w[i], acc, 0, 0, 0);
    }
  } else if constexpr (!in_span<BITS, MASK, U>()) {
    bf16x8 w;
    if constexpr ((MASK >> U) & 1)
      w = group_table<BITS, TAB, U>(L, table, s, q, std::make_integer_sequence<int, 8>{});
    else
      w = group_alu<BITS, U>(L, q, k, std::make_integer_sequence<int, 8>{});
    const bf16x8 xv = *reinterpret_cast<const bf16x8 *>(xa + 16 * U);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, w, acc, 0, 0, 0);
  }
}

// k = 4 with groups 0, 1 and 4, 5 on the table and 2, 3, 6, 7 on the ALU,
// in two phases. Scheduling barriers keep the compiler from pulling the
// phases together: left to itself it consumes the gathers right after
// issuing them (and reuses their registers one gather at a time), so each
// wave waits out the LDS latency. The phased order was measured 2% faster
// per launch (the same treatment of the k = 3 and k = 2 mixes gained
// nothing). The LDS wait counter saturates past 15 outstanding reads, so
// each phase waits once, after its ALU work. Within a phase the 16 gathers
// go out four at a time between quarters of the ALU work rather than in one
// burst: with 16 waves sharing the LDS, bursts queue behind each other, and
// spreading them was measured 2-2.5% faster per launch at k = 4.
template <int TAB, int U, int Q0 = 0, int Q1 = 4>
__device__ __forceinline__ void span4_issue(const LaneWords<4> &L, const unsigned char *table, uint32_t mask,
                                            uint32_t (&r)[2][8]) {
  using R = TableRead<TAB>;
  constexpr int SH = R::kShift;
#pragma unroll
  for (int i = Q0; i < Q1; ++i) {
    uint32_t a[4];
    switch (i) {
      case 0: quad_xa<(63 - (8 * U + 12 + 0)) * 4, SH>(L.d, mask, a); break;
      case 1: quad_xa<(63 - (8 * U + 12 + 1)) * 4, SH>(L.d, mask, a); break;
      case 2: quad_xa<(63 - (8 * U + 12 + 2)) * 4, SH>(L.d, mask, a); break;
      default: quad_xa<(63 - (8 * U + 12 + 3)) * 4, SH>(L.d, mask, a); break;
    }
    r[1][4 + i] = R::raw(table, a[0]);
    r[1][i] = R::raw(table, a[1]);
    r[0][4 + i] = R::raw(table, a[2]);
    r[0][i] = R::raw(table, a[3]);
  }
}
template <int TAB>
__device__ __forceinline__ bf16x8 span4_weights(const uint32_t (&r)[8], float s, float q) {
  using R = TableRead<TAB>;
  bf16x8 w;
#pragma unroll
  for (int e = 0; e < 8; ++e) w[e] = (__bf16)R::from_raw(r[e], s, q);
  return w;
}
// ALU-path weights S of group U (float32, before the bf16 rounding).
template <int U, int... S>
__device__ __forceinline__ void alu4_part(const LaneWords<4> &L, float q, float k, float (&f)[8],
                                          std::integer_sequence<int, S...>) {
  ((f[S] = __builtin_fmaf(code_plus_magic(win12<(63 - 8 * U - S) * 4>(L.d)), q, k)), ...);
}
__device__ __forceinline__ bf16x8 pack8(const float (&f)[8]) {
  bf16x8 w;
#pragma unroll
  for (int i = 0; i < 8; ++i) w[i] = (__bf16)f[i];
  return w;
}
// One ALU group of k = 4 in two quarters of the phase, each after a quad of
// gathers (the gathers of quads Q and Q + 1 of the phase's table span).
template <int TAB, int SPAN, int U, int Q>
__device__ __forceinline__ bf16x8 alu4_between_gathers(const LaneWords<4> &L, const unsigned char *table,
                                                       uint32_t mask, uint32_t (&r)[2][8], float q, float k) {
  float f[8];
  span4_issue<TAB, SPAN, Q, Q + 1>(L, table, mask, r);
  __builtin_amdgcn_sched_barrier(0);
  alu4_part<U>(L, q, k, f, std::integer_sequence<int, 0, 1, 2, 3>{});
  __builtin_amdgcn_sched_barrier(0);
  span4_issue<TAB, SPAN, Q + 1, Q + 2>(L, table, mask, r);
  __builtin_amdgcn_sched_barrier(0);
  alu4_part<U>(L, q, k, f, std::integer_sequence<int, 4, 5, 6, 7>{});
  const bf16x8 w = pack8(f);
  __builtin_amdgcn_sched_barrier(0);
  return w;
}
// A workgroup barrier for data in LDS only: the wave's LDS accesses are
// complete when it arrives, while its global loads may still be in flight
// (the compiler's barrier waits for those too).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }
__device__ __forceinline__ bf16x8 xop(const unsigned char *xa, int u) {
  return *reinterpret_cast<const bf16x8 *>(xa + 16 * u);
}
__device__ __forceinline__ void mfma(bf16x8 xv, bf16x8 w, f32x4 &acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xv, w, acc, 0, 0, 0);
}
template <int TAB>
__device__ __forceinline__ void unit4_phase2(const LaneWords<4> &L, const unsigned char *table,
                                             const unsigned char *xa, float s, float q, float k, uint32_t mask,
                                             f32x4 &acc) {
  uint32_t r[2][8];
  const bf16x8 x3 = xop(xa, 3), x7 = xop(xa, 7), x4 = xop(xa, 4), x5 = xop(xa, 5);
  const bf16x8 w3 = alu4_between_gathers<TAB, 4, 3, 0>(L, table, mask, r, q, k);
  const bf16x8 w7 = alu4_between_gathers<TAB, 4, 7, 2>(L, table, mask, r, q, k);
  mfma(x3, w3, acc);
  mfma(x7, w7, acc);
  mfma(x4, span4_weights<TAB>(r[0], s, q), acc);
  mfma(x5, span4_weights<TAB>(r[1], s, q), acc);
}
template <int TAB>
__device__ __forceinline__ void unit4_phased(const LaneWords<4> &L, const unsigned char *table,
                                             const unsigned char *xa, float s, float q, float k, uint32_t mask,
                                             f32x4 &acc) {
  uint32_t r[2][8];
  // Two phases: the x operands of the phase are read, the gathers of one
  // table span go out a quad at a time between the quarters of two ALU
  // groups, and only then are the gathered entries turned into weights.
  {
    const bf16x8 x2 = xop(xa, 2), x6 = xop(xa, 6), x0 = xop(xa, 0), x1 = xop(xa, 1);
    const bf16x8 w2 = alu4_between_gathers<TAB, 0, 2, 0>(L, table, mask, r, q, k);
    const bf16x8 w6 = alu4_between_gathers<TAB, 0, 6, 2>(L, table, mask, r, q, k);
    mfma(x2, w2, acc);
    mfma(x6, w6, acc);
    mfma(x0, span4_weights<TAB>(r[0], s, q), acc);
    mfma(x1, span4_weights<TAB>(r[1], s, q), acc);
  }
  __builtin_amdgcn_sched_barrier(0);
  unit4_phase2<TAB>(L, table, xa, s, q, k, mask, acc);
}
// The first phase's weights alone (groups 2, 6, 0, 1, in the order the
// phase multiplies them), for a unit decoded before its x operands are in
// LDS.
template <int TAB>
__device__ __forceinline__ void unit4_phase1_weights(const LaneWords<4> &L, const unsigned char *table, float s,
                                                     float q, float k, uint32_t mask, bf16x8 (&w)[4]) {
  uint32_t r[2][8];
  w[0] = alu4_between_gathers<TAB, 0, 2, 0>(L, table, mask, r, q, k);
  w[1] = alu4_between_gathers<TAB, 0, 6, 2>(L, table, mask, r, q, k);
  w[2] = span4_weights<TAB>(r[0], s, q);
  w[3] = span4_weights<TAB>(r[1], s, q);
}

// k = 2 with groups 0, 1 and 4, 5 on the table (windows of groups U and
// U + 1 at one slot are 16 bits apart: one shifted word, two masks) and
// 2, 3, 6, 7 on the ALU, in the two phases and quad-by-quad gather issue of
// k = 4. Against groups 4..7 on the table in one span, compiled freely,
// this was measured 1.5% faster per launch at M = 15, K = 5120.
template <int O0, int SH, int N>
__device__ __forceinline__ void half_quad_xa(const uint32_t (&D)[N], uint32_t mask, uint32_t (&a)[2]) {
  constexpr int sh = O0 - SH;
  constexpr uint32_t m = 0xFFFu << SH;
  static_assert(sh >= 0, "unexpected window offset");
  constexpr int w = sh >> 5, r = sh & 31;
  static_assert(w + (r != 0) < N, "pair of windows outside the lane's words");
  uint32_t lo;
  if constexpr (r == 0) lo = D[w];
  else lo = __builtin_amdgcn_alignbit(D[w + 1], D[w], r);
  a[0] = lo & m;
  a[1] = and_hi16(lo, mask);
}
template <int TAB, int U, int Q0, int Q1>
__device__ __forceinline__ void span2_issue(const LaneWords<2> &L, const unsigned char *table, uint32_t mask,
                                            uint32_t (&r)[2][8]) {
  using R = TableRead<TAB>;
  constexpr int SH = R::kShift;
#pragma unroll
  for (int i = 2 * Q0; i < 2 * Q1; ++i) {
    uint32_t a[2];
    switch (i) {
      case 0: half_quad_xa<(63 - 8 * (U + 1) - 0) * 2, SH>(L.d, mask, a); break;
      case 1: half_quad_xa<(63 - 8 * (U + 1) - 1) * 2, SH>(L.d, mask, a); break;
      case 2: half_quad_xa<(63 - 8 * (U + 1) - 2) * 2, SH>(L.d, mask, a); break;
      case 3: half_quad_xa<(63 - 8 * (U + 1) - 3) * 2, SH>(L.d, mask, a); break;
      case 4: half_quad_xa<(63 - 8 * (U + 1) - 4) * 2, SH>(L.d, mask, a); break;
      case 5: half_quad_xa<(63 - 8 * (U + 1) - 5) * 2, SH>(L.d, mask, a); break;
      case 6: half_quad_xa<(63 - 8 * (U + 1) - 6) * 2, SH>(L.d, mask, a); break;
      default: half_quad_xa<(63 - 8 * (U + 1) - 7) * 2, SH>(L.d, mask, a); break;
    }
    r[1][i] = R::raw(table, a[0]);
    r[0][i] = R::raw(table, a[1]);
  }
}
template <int U, int... S>
__device__ __forceinline__ void alu2_part(const LaneWords<2> &L, float q, float k, float (&f)[8],
                                          std::integer_sequence<int, S...>) {
  ((f[S] = __builtin_fmaf(code_plus_magic(win12<(63 - 8 * U - S) * 2>(L.d)), q, k)), ...);
}
template <int TAB, int SPAN, int U, int Q>
__device__ __forceinline__ bf16x8 alu2_between_gathers(const LaneWords<2> &L, const unsigned char *table,
                                                       uint32_t mask, uint32_t (&r)[2][8], float q, float k) {
  float f[8];
  span2_issue<TAB, SPAN, Q, Q + 1>(L, table, mask, r);
  __builtin_amdgcn_sched_barrier(0);
  alu2_part<U>(L, q, k, f, std::integer_sequence<int, 0, 1, 2, 3>{});
  __builtin_amdgcn_sched_barrier(0);
  span2_issue<TAB, SPAN, Q + 1, Q + 2>(L, table, mask, r);
  __builtin_amdgcn_sched_barrier(0);
  alu2_part<U>(L, q, k, f, std::integer_sequence<int, 4, 5, 6, 7>{});
  const bf16x8 w = pack8(f);
  __builtin_amdgcn_sched_barrier(0);
  return w;
}
template <int TAB>
__device__ __forceinline__ void unit2_phase2(const LaneWords<2> &L, const unsigned char *table,
                                             const unsigned char *xa, float s, float q, float k, uint32_t mask,
                                             f32x4 &acc) {
  uint32_t r[2][8];
  const bf16x8 x3 = xop(xa, 3), x7 = xop(xa, 7), x4 = xop(xa, 4), x5 = xop(xa, 5);
  const bf16x8 w3 = alu2_between_gathers<TAB, 4, 3, 0>(L, table, mask, r, q, k);
  const bf16x8 w7 = alu2_between_gathers<TAB, 4, 7, 2>(L, table, mask, r, q, k);
  mfma(x3, w3, acc);
  mfma(x7, w7, acc);
  mfma(x4, span4_weights<TAB>(r[0], s, q), acc);
  mfma(x5, span4_weights<TAB>(r[1], s, q), acc);
}
template <int TAB>
__device__ __forceinline__ void unit2_phased(const LaneWords<2> &L, const unsigned char *table,
                                             const unsigned char *xa, float s, float q, float k, uint32_t mask,
                                             f32x4 &acc) {
  uint32_t r[2][8];
  {
    const bf16x8 x2 = xop(xa, 2), x6 = xop(xa, 6), x0 = xop(xa, 0), x1 = xop(xa, 1);
    const bf16x8 w2 = alu2_between_gathers<TAB, 0, 2, 0>(L, table, mask, r, q, k);
    const bf16x8 w6 = alu2_between_gathers<TAB, 0, 6, 2>(L, table, mask, r, q, k);
    mfma(x2, w2, acc);
    mfma(x6, w6, acc);
    mfma(x0, span4_weights<TAB>(r[0], s, q), acc);
    mfma(x1, span4_weights<TAB>(r[1], s, q), acc);
  }
  __builtin_amdgcn_sched_barrier(0);
  unit2_phase2<TAB>(L, table, xa, s, q, k, mask, acc);
}
template <int TAB>
__device__ __forceinline__ void unit2_phase1_weights(const LaneWords<2> &L, const unsigned char *table, float s,
                                                     float q, float k, uint32_t mask, bf16x8 (&w)[4]) {
  uint32_t r[2][8];
  w[0] = alu2_between_gathers<TAB, 0, 2, 0>(L, table, mask, r, q, k);
  w[1] = alu2_between_gathers<TAB, 0, 6, 2>(L, table, mask, r, q, k);
  w[2] = span4_weights<TAB>(r[0], s, q);
  w[3] = span4_weights<TAB>(r[1], s, q);
}

template <int BITS, int MASK, int TAB, bool EXACT, int... U>
__device__ __forceinline__ void unit(const LaneWords<BITS> &L, const unsigned char *table, const unsigned char *xa,
                                     float s, float q, float k, uint32_t mask, f32x4 &acc,
                                     std::integer_sequence<int, U...>) {
  (unit_group<BITS, MASK, TAB, EXACT, U>(L, table, xa, s, q, k, mask, acc), ...);
}

// The MLP's elementwise tail on one output element, as the page's model
// code orders it (page "mlx-bun 0.0.4" (npm, page 62), section
// src/model/minicpm5.ts, MLP forward): every operation there yields a bf16
// array, so the two projections, sigmoid(gate), gate * sigmoid(gate) and
// that times up are each rounded to bf16. `gate` and `up` are the float32
// sums of the two projections.
__device__ __forceinline__ uint16_t gate_up_bits(float gate_sum, float up_sum) {
  const float gate = (float)(__bf16)gate_sum, up = (float)(__bf16)up_sum;
  const float sig = (float)(__bf16)(1.0f / (1.0f + expf(-gate)));
  const float silu = (float)(__bf16)(gate * sig);
  return __builtin_bit_cast(uint16_t, (__bf16)(silu * up));
}

// Lane l holds rows 4 (l / 16) .. 4 (l / 16) + 3 of output column
// col0 + l % 16; the row pointers come from the LDS copy of the row table. One matrix: v is the
// tile's sum. Two (gate and up): v and v2 are the two projections' sums and
// the output is the elementwise tail.
template <bool TWO>
__device__ __forceinline__ void store_tile(const uint64_t *rows, f32x4 v, f32x4 v2, int m, int ncols, int col0) {
  // The lane's column and rows are formed here, from the lane id, at the
  // store: the empty asm keeps the compiler from hoisting them out of the
  // main loop, where keeping them live would spill.
  int lane_id = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  asm volatile("" : "+v"(lane_id));
  const int col = col0 + (lane_id & 15), gr = (lane_id >> 4) * 4;
  if (col >= ncols) return;
  const uint64_t *my_rows = rows + gr;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (gr + e < m) {
      uint16_t bits;
      if constexpr (TWO) bits = gate_up_bits(v[e], v2[e]);
      else bits = __builtin_bit_cast(uint16_t, (__bf16)v[e]);
      // A global (not flat) store: a flat store might address LDS, so the
      // compiler would make every later LDS read wait for its completion.
      reinterpret_cast<__attribute__((address_space(1))) uint16_t *>(my_rows[e])[col] = bits;
    }
}

// Partials of tiles shared with other workgroups go through the workspace:
// slot [tile][panel][contributor] holds NH 16x16 fp32 partials (one per
// matrix), lane-major, 1 KB each.
template <int NH>
__device__ __forceinline__ float *partial_slot(const Plan &pl, float *ws, int tile, int panel, int idx, int lane) {
  return ws + ((((int64_t)tile * pl.panels + panel) * pl.maxc + idx) * NH) * 256 + 4 * lane;
}

// Stores a lane's four partial sums without making the wave wait for them:
// written as inline assembly, the store is not tracked by the compiler's
// memory-counter waits, so the next code-word loads are not held up behind
// its acknowledgement. A later wait for a load still covers that load (loads
// complete in order among themselves); the explicit s_waitcnt vmcnt(0) after
// the main loop covers the store. sc1: written through to the level that is
// coherent across the per-XCD L2s (agent scope). One 16-byte store per lane
// keeps every write a whole cache line per wave. The compiler does not look
// inside the asm for hazards on its inputs, so the leading s_nops give the
// wait states a vector memory instruction needs after an MFMA wrote its data
// (11 for an 8-pass MFMA) or a VALU wrote an SGPR it reads (5, such as a
// v_readlane that reloads a spilled base address); the trailing s_nop covers
// the store-data hazard of stores wider than 8 bytes.
#define TRELLIS_ASM_VMEM_PAD "s_nop 7\n\ts_nop 4\n\t"
__device__ __forceinline__ void stage_partial(float *slot, f32x4 v) {
  asm volatile(
      TRELLIS_ASM_VMEM_PAD
      "global_store_dwordx4 %0, %1, off sc1\n\t"
      "s_nop 1"
      :
      : "v"(slot), "v"(v)
      : "memory");
}

// The same for a pair of partials (two matrices) at a wave-uniform base:
// lane offsets `off` and off + 1 KB. The address stays a scalar base plus a
// 32-bit lane offset, so nothing 64-bit per lane has to be kept live.
__device__ __forceinline__ void stage_pair(float *base, uint32_t off, f32x4 v, f32x4 v2) {
  asm volatile(
      TRELLIS_ASM_VMEM_PAD
      "global_store_dwordx4 %0, %1, %3 sc1\n\t"
      "global_store_dwordx4 %0, %2, %3 offset:1024 sc1\n\t"
      "s_nop 1"
      :
      : "v"(off), "v"(v), "v"(v2), "s"(base)
      : "memory");
}

// Sums of a tile's staged partials (one per matrix), panel-major then
// contributor order. The loads (16 bytes per lane, sc1: from the coherent
// level) are issued in batches of twenty 1 KB partials before any of them
// is used, so a batch costs one round trip rather than twenty. With several
// K panels every tile is shared by four or five pieces per panel, and
// twenty covers four panels in one batch (measured 0.6 us faster per launch
// than sixteen at M = 15, K = 17408; 24 spills registers in the two-matrix
// kernels). Loads past the tile's last partial take an offset outside the
// buffer, which the hardware answers with zeros without a memory access, so
// a tile with a few partials does not send a batch of useless requests. The
// batch size is a multiple of NH, so load i of a batch belongs to matrix
// i % NH.
template <int NH>
__device__ __forceinline__ void sum_partials(const Plan &pl, float *ws, int tile, int contrib, int lane,
                                             f32x4 (&sum)[NH]) {
  constexpr int kBatch = 20;
  static_assert(kBatch % NH == 0, "a batch holds whole slots");
  constexpr int kSc1 = 16;  // cache-policy bits of the loads
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      partial_slot<NH>(pl, ws, tile, 0, 0, 0), (short)0, pl.panels * pl.maxc * NH * 1024, kRawBufferWord3);
  const int total = contrib * pl.panels * NH;  // 1 KB partials
#pragma unroll
  for (int h = 0; h < NH; ++h) sum[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  int pp = 0, cc = 0;  // slot of the next load
  for (int b0 = 0; b0 < total; b0 += kBatch) {
    f32x4 v[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const uint32_t off = b0 + i < total
                               ? ((uint32_t)(pp * pl.maxc + cc) * NH + (uint32_t)(i % NH)) * 1024 + (uint32_t)lane * 16
                               : 0x80000000u;  // outside the buffer: zeros, no memory access
      v[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kSc1));
      if (i % NH == NH - 1 && b0 + i + 1 < total && ++cc == contrib) {
        cc = 0;
        ++pp;
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (b0 + i < total)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[i % NH][e] += v[i][e];
  }
}

// TWO: the fused gate and up projections. A unit is then one block of a tile
// of both matrices, decoded in two steps (gate, then up) against the same x
// into two accumulators, so whichever wave completes a tile holds both sums
// and writes the elementwise tail directly.
template <int BITS, int MASK, int TAB, bool TWO>
__global__ __launch_bounds__(kWgThreads) void prefill_kernel(const uint32_t *__restrict__ codes,
                                                             const uint16_t *__restrict__ scales,
                                                             const uint32_t *__restrict__ codes2,
                                                             const uint16_t *__restrict__ scales2,
                                                             float *__restrict__ ws, uint32_t *__restrict__ counters,
                                                             float *__restrict__ kept, Plan pl, RowPtrs rp) {
  // The table is static LDS (address known at compile time, so table reads
  // carry their base in the instruction offset); x follows it dynamically.
  // After the main loop the x region is reused for the waves' partial tiles.
  constexpr int NH = TWO ? 2 : 1;  // accumulators (matrices) per unit
  constexpr int kSlotBytes = kCombineBytes * NH;
  __shared__ __attribute__((aligned(16))) uint32_t s_table[table_bytes(TAB) / 4];
  __shared__ uint64_t s_rows[kMaxRows];  // output row pointers
  extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
  unsigned char *const table = reinterpret_cast<unsigned char *>(s_table);
  unsigned char *const xl = lds;
  constexpr int wpb = 8 * BITS;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int j = lane & 15, g = lane >> 4;
  // The lane id again, for the code after the prologue: formed where it is
  // used (the empty asm keeps it there), so no register holds it through
  // the main loop.
  auto lane_id = []() {
    int l = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(l));
    return l;
  };
  // Row 0's pointer and this wave's output row pointer (one per wave) are
  // read with the plan: the empty asm keeps the reads at the top, not further
  // down where each would wait on its own.
  static_assert(kMaxRows == kWaves, "one output row pointer per wave");
  const uint16_t *const x_row0 = rp.x[0];
  const uint64_t out_row = reinterpret_cast<uint64_t>(rp.out[wave]);
  asm volatile("" ::"s"(x_row0), "s"(out_row));
  const int group = (int)div_by<6>(blockIdx.x, pl);
  const int panel = (int)blockIdx.x - group * pl.panels;
  const int panel_k = pl.kp * 256;
  const int64_t kbase = (int64_t)panel * panel_k;
  // x[:, panel] is requested first: it needs only the panel, and every
  // workgroup stages it before its first unit.
  const int vecs = panel_k / 8;
  const int xtotal = pl.m * vecs;  // <= kStageRegs * kWgThreads (the x panel fits in LDS)
  // Staged x vector idx (16 B) is row i = idx / vecs, column idx - i * vecs;
  // rows are one vector longer in LDS, so it lands at byte 16 (idx + i).
  // A wave skips the rounds that start past the panel; lanes past it take
  // the panel's last vector (a second load of it and an identical store).
  auto xrow = [&](int idx) { return (int)(__umul24((uint32_t)idx >> 5, pl.xmul) >> pl.xshift); };
  const int xlast = xtotal - 1;
  uint4 xv[kStageRegs];
  {
#pragma unroll
    for (int r = 0; r < kStageRegs; ++r) xv[r] = uint4{0u, 0u, 0u, 0u};  // defined on every path: keeps xv in registers
    const unsigned char *const xb = reinterpret_cast<const unsigned char *>(x_row0 + kbase);
    if (pl.x_contiguous) {
      // Rows K elements apart: vector idx is 16 (idx + i (panels - 1) vecs)
      // bytes past row 0's part of the panel.
      const uint32_t pstep = (uint32_t)((pl.panels - 1) * vecs);
#pragma unroll
      for (int r = 0; r < kStageRegs; ++r) {
        if (r * kWgThreads + wave * kWave < xtotal) {
          const int idx = min(r * kWgThreads + tid, xlast);
          xv[r] = *reinterpret_cast<const uint4 *>(xb + ((uint32_t)idx + __umul24((uint32_t)xrow(idx), pstep)) * 16u);
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < kStageRegs; ++r) {
        if (r * kWgThreads + wave * kWave >= xtotal) continue;
        // A wave's 64 vectors start at a multiple of 64 and a row holds a
        // multiple of 32 of them, so they lie in rows i0 and i0 + 1 (uniform).
        const int i0 = min(xrow(r * kWgThreads + wave * kWave), kMaxRows - 2);
        const uint16_t *const x0 = rp.x[i0], *const x1 = rp.x[i0 + 1];
        const int idx = min(r * kWgThreads + tid, xlast);
        const int i = xrow(idx), c = idx - (int)__umul24((uint32_t)i, (uint32_t)vecs);
        xv[r] = *reinterpret_cast<const uint4 *>((i == i0 ? x0 : x1) + kbase + 8 * c);
      }
    }
  }

  // This workgroup's units [cu_u0, cu_u1) and this wave's piece of them.
  const CuSplit q = cu_split(group, pl);
  const int cu_u0 = q.u0, cu_u1 = q.u0 + q.len;
  const int nseg = q.s;
  const bool active = wave < q.s;
  const int seg = (wave & 1) ? q.s - 1 - (wave >> 1) : (wave >> 1);  // position of the piece
  const int u0 = active ? piece_start(q, seg) : 0;
  const int u1 = active ? piece_start(q, seg + 1) : 0;
  const int piece = group * kWaves + seg;
  // A tile is "cross" when some of its units (of any panel) belong to another
  // workgroup; its partials are combined through the workspace.
  auto cross = [&](int t) { return pl.panels > 1 || t * pl.kp < cu_u0 || (t + 1) * pl.kp > cu_u1; };

  // Per-lane byte offsets of the code words inside a unit's buffer (see
  // load_words) and of the row scale inside its tile's scale buffer.
  const uint32_t row_bytes = (uint32_t)(pl.k >> 8) * wpb * 4;
  const uint32_t lane_off = (uint32_t)j * row_bytes + (uint32_t)g * (8 * BITS);
  const uint32_t lane_off_next = (uint32_t)j * row_bytes + (uint32_t)((2 * BITS * (g + 1)) % wpb) * 4;
  const uint32_t lane_off_scale = (uint32_t)j * 2;
  // Buffers of unit (t, bb) and of tile t's scales, of the first matrix or
  // (second) of the up matrix: rows past N are outside them, so their words
  // and scales read as zero (zero weights, never stored).
  auto unit_buffer = [&](int t, int bb, bool second) {
    const int rows = pl.n - t * 16 < 16 ? pl.n - t * 16 : 16;
    const uint32_t blk_off = (uint32_t)(panel * pl.kp + bb) * (wpb * 4);
    const unsigned char *base = reinterpret_cast<const unsigned char *>(second ? codes2 : codes) +
                                (int64_t)t * 16 * row_bytes + blk_off;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char *>(base), (short)0,
                                             (int)((uint32_t)rows * row_bytes - blk_off), kRawBufferWord3);
  };
  auto scale_buffer = [&](int t, bool second) {
    const int rows = pl.n - t * 16 < 16 ? pl.n - t * 16 : 16;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>((second ? scales2 : scales) + (int64_t)t * 16),
                                             (short)0, rows * 2, kRawBufferWord3);
  };
  // Raw scale bits are converted only when the tile starts, so the load is
  // not waited for early.
  auto scale_of = [&](uint32_t bits) { return bf16_bits_to_f32((uint16_t)bits); };

  // Code words (and the row scale) of each unit live in one of two register
  // slots: the unit being decoded and the next one in flight. The loop below
  // is unrolled by two so the slots alternate without copying registers that
  // still have loads pending. With two matrices slot 0 always holds a gate
  // block and slot 1 the same block of up. A decode-ahead prologue
  // (below) requests two units and leaves the second for the loop in slot 0.
  constexpr bool kAhead = MASK == 0x33 && TAB != kPairTable && (BITS == 4 || BITS == 2);
  struct Slot {
    LaneWords<BITS> w;
    // raw bf16 scale bits (16 bits with the decode-ahead below: the second
    // unit's scale crosses a barrier there, and widened to 32 bits it was
    // waited for before the barrier)
    std::conditional_t<kAhead, uint16_t, uint32_t> scb;
  };
  Slot S0, S1;
  int tile = (int)div_by<7>((uint32_t)u0, pl);
  int b = u0 - tile * pl.kp;
  int pt = tile, pb = b, pu = u0;  // next unit to request
  auto advance = [&](int &t, int &bb) {
    if (++bb == pl.kp) {
      bb = 0;
      ++t;
    }
  };
  // Every loop iteration requests the same number of units (straight-line
  // code keeps the compiler's memory-counter waits exact); the step of the
  // range's last unit requests nothing, so requests never leave the range.
  auto request = [&](Slot &S, auto second) {
    constexpr bool kUp = decltype(second)::value;
    load_words<BITS>(unit_buffer(pt, pb, kUp), lane_off, lane_off_next, S.w);
    S.scb = __builtin_amdgcn_raw_buffer_load_b16(scale_buffer(pt, kUp), lane_off_scale, 0, 0);
    if constexpr (!TWO || kUp) {
      if (++pu < u1) advance(pt, pb);
    }
  };
  // Prologue. x[:, panel] (M rows) is requested first, then the first unit's code words (memory-counter waits are in
  // issue order, so x can be stored to LDS without waiting for the codes);
  // the decode table is built while both are in flight.
  // With the two-phase decodes (k = 4 and k = 2 on a value or code table) a
  // barrier follows the table, and each wave decodes the first phase of its
  // first unit (gate block) before the barrier that waits for x: waves whose
  // x arrived early decode while the rest of the workgroup's x is still on
  // its way. The second unit (with two matrices: the up block of the first)
  // is requested after that decode, so that it does not compete with x and
  // the first unit's words.
  constexpr uint32_t kMaskAddr = TAB == kPairTable ? 0xFFFCu : TAB == kCodeTable ? 0x1FFEu : 0x3FFCu;
  bool ahead = false;  // the first unit's first phase is decoded (its row scales are in range)
  bf16x8 aw[4];        // its weights
  {
    // counters of the barrier-free combine start at zero
    if (wave == 0 && pl.slots_off > 0 && lane < kWaves)
      reinterpret_cast<uint32_t *>(xl + pl.slots_off + kSlotBytes)[lane] = 0u;
    request(S0, std::false_type{});
    // (every thread builds the same number of entries: no loop control)
    static_assert(2048 % kWgThreads == 0, "table entries divide among the threads");
    if constexpr (TAB == kPairTable) {
#pragma unroll
      for (int r = 0; r < 16384 / kWgThreads; ++r) s_table[r * kWgThreads + tid] = pair_entry((uint32_t)(r * kWgThreads + tid));
    } else if constexpr (TAB == kCodeTable) {
#pragma unroll
      for (int r = 0; r < 2048 / kWgThreads; ++r)
        s_table[r * kWgThreads + tid] = code_entry_pair((uint32_t)(r * kWgThreads + tid));
    } else {
#pragma unroll
      for (int r = 0; r < 4096 / kWgThreads; ++r)
        s_table[r * kWgThreads + tid] =
            __builtin_bit_cast(uint32_t, trellis_value(code_of((uint32_t)(r * kWgThreads + tid))));
    }
    // Output row pointers to LDS, one per wave (read at the top).
    if (lane == 0) s_rows[wave] = out_row;
    if constexpr (kAhead) {
      lds_barrier();  // the table is built
    }
#pragma unroll
    for (int r = 0; r < kStageRegs; ++r) {
      if (r * kWgThreads + wave * kWave >= xtotal) continue;
      const int idx = min(r * kWgThreads + tid, xlast);
      *reinterpret_cast<uint4 *>(xl + 16 * (idx + xrow(idx))) = xv[r];
    }
    if constexpr (kAhead) {
      if (u1 - u0 >= 2) {
        const float s = scale_of(S0.scb);
        float q, kq;
        alu_row_constants(s, q, kq);
        if (__all(alu_scale_ok(s))) {
          ahead = true;
          if constexpr (BITS == 4) unit4_phase1_weights<TAB>(S0.w, table, s, q, kq, kMaskAddr, aw);
          else unit2_phase1_weights<TAB>(S0.w, table, s, q, kq, kMaskAddr, aw);
        }
      }
      // the range's second unit (its first again when it holds one unit);
      // with two matrices the up block of the first unit
      request(S1, std::bool_constant<TWO>{});
    }
  }

  if constexpr (kAhead) lds_barrier();
  else __syncthreads();

  // A-operand rows j >= M read row M - 1: they only feed output rows >= M,
  // which are never stored.
  const unsigned char *xa = xl + (j < pl.m ? j : pl.m - 1) * pl.x_stride + (192 - 64 * g) * 2;

  // Tiles of this wave's range: a cross tile's partial is staged in the
  // workspace as soon as its units here are done (its counter is bumped after
  // the loop); a tile whose units (of this panel) all lie in the range is
  // stored; otherwise the first and last tile of the range may be shared with
  // neighbouring pieces of this workgroup and are kept as partials for the
  // combine below.
  const int tf = tile;
  int tl = tile;  // the range's last tile
  // Whether the range holds a tile shared with another workgroup (for one
  // K panel only its first or last tile can be).
  const bool holds_cross =
      active && (cross(tf) || cross((int)div_by<7>((uint32_t)(u1 > 0 ? u1 - 1 : 0), pl)));
  // Partials kept for the barrier combine: of the range's first tile (when
  // it ends inside the loop) and of its last tile. With two matrices the
  // first tile's pair waits in this wave's slot of `kept` (global memory)
  // instead of registers, which the loop cannot spare.
  f32x4 part_f = {0.f, 0.f, 0.f, 0.f}, part_l = {0.f, 0.f, 0.f, 0.f};
  f32x4 part_f2 = {0.f, 0.f, 0.f, 0.f}, part_l2 = {0.f, 0.f, 0.f, 0.f};
  float *const kept_base = kept + ((int64_t)blockIdx.x * kWaves + wave) * 512;  // wave-uniform
  auto stage = [&](int t, f32x4 v, f32x4 v2) {
    float *slot = partial_slot<NH>(pl, ws, t, panel, piece - piece_of(t * pl.kp, pl), lane_id());
    stage_partial(slot, v);
    if constexpr (TWO) stage_partial(slot + 256, v2);
  };
  // Barrier-free combine (dedicated slots): the piece's partial of tile T
  // goes to its slot (0: T is where the piece starts, 1: T is where it
  // ends), and an LDS counter keyed by the position of the piece holding
  // T's first unit counts the contributions. The piece that arrives last
  // adds the partials in position order and stores bf16. Its slot write
  // completes before its counter update, and the last arriver reads only
  // after its own update returned, so it sees every partial.
  auto contribute = [&](int T, f32x4 v, f32x4 v2, int which) {
    const int lane = lane_id();
    f32x4 *slots = reinterpret_cast<f32x4 *>(xl + pl.slots_off);  // [piece][first, last][matrix][lane]
    uint32_t *cnt = reinterpret_cast<uint32_t *>(xl + pl.slots_off + kSlotBytes);
    slots[((seg * 2 + which) * NH) * kWave + lane] = v;
    if constexpr (TWO) slots[((seg * 2 + which) * NH + 1) * kWave + lane] = v2;
    // (T lies in this workgroup's units: its pieces are found in this split)
    const int lead = piece_in(q, group, T * pl.kp - cu_u0, pl);
    const int contrib = piece_in(q, group, T * pl.kp + pl.kp - 1 - cu_u0, pl) - lead + 1;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(&cnt[lead], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    old = __builtin_amdgcn_readfirstlane(old);
    asm volatile("" ::: "memory");
    if ((int)old + 1 != contrib) return;
    const int t0u = T * pl.kp;
    f32x4 sum[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) sum[h] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sidx = lead; sidx < lead + contrib; ++sidx) {
      const int base = (sidx * 2 + (piece_start(q, sidx) >= t0u ? 0 : 1)) * NH;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const f32x4 w = slots[(base + h) * kWave + lane];
#pragma unroll
        for (int e = 0; e < 4; ++e) sum[h][e] += w[e];
      }
    }
    store_tile<TWO>(s_rows, sum[0], sum[NH - 1], pl.m, pl.n, T * 16);
  };
  // A tile finished inside the loop is never the range's last tile.
  // The range's first tile, when it is shared with other workgroups and
  // finished inside the loop, has its counter bumped one step after its
  // partial was staged (the wave then waits for nothing but that step's code
  // words); only the result is looked at after the loop. Counting it at the
  // end instead would often make this wave, finishing its loop after the
  // tile's other contributors, the last to arrive at two tiles, adding a
  // round trip at the end of the launch.
  bool bump_tf = false, tf_bumped = false;
  uint32_t tf_old = 0;  // lane 0: the counter before this wave's bump
  auto tile_done = [&](int t, f32x4 v, f32x4 v2) {
    if (cross(t)) {
      stage(t, v, v2);
      // (several K panels only, where every tile is shared; two matrices:
      // no VGPR to spare for the result)
      if constexpr (!TWO) bump_tf = t == tf && pl.panels > 1;
    } else if (t == tf && u0 > t * pl.kp) {
      if (pl.slots_off > 0) contribute(t, v, v2, 0);
      else if constexpr (TWO) stage_pair(kept_base, (uint32_t)lane_id() * 16, v, v2);
      else part_f = v;
    } else store_tile<TWO>(s_rows, v, v2, pl.m, pl.n, t * 16);
  };
  if (active) {
    int cur = tile;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float s = scale_of(S0.scb), q, kq;
    alu_row_constants(s, q, kq);
    bool out_of_range = !__all(alu_scale_ok(s));
    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};  // second matrix (up)
    // table byte-address mask (SDWA operand)
    const uint32_t mask_addr = TAB == kPairTable ? 0xFFFCu : TAB == kCodeTable ? 0x1FFEu : 0x3FFCu;
    int u = u0;
    // Decode unit u from slot C while unit u + 1 is requested into slot N;
    // the range's last unit requests nothing (`last`), so no load is left in
    // flight after the loop. With two matrices a unit takes two steps: the
    // gate block (slot 0, which requests the up block of the same unit) and
    // the up block (slot 1, which requests the next unit's gate block).
    auto step = [&](Slot &C, Slot &N, auto last, auto second) {
      constexpr bool kUp = decltype(second)::value;
      f32x4 &A = kUp ? acc2 : acc;
      if constexpr (!kUp) {
        if (bump_tf) {
          // The staged partial is complete before the counter moves.
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          if (lane_id() == 0) tf_old = __hip_atomic_fetch_add(&counters[(size_t)tf << pl.cshift], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          bump_tf = false;
          tf_bumped = true;
        }
        if (tile != cur) {
          tile_done(cur, acc, acc2);
          cur = tile;
          acc = f32x4{0.f, 0.f, 0.f, 0.f};
          acc2 = f32x4{0.f, 0.f, 0.f, 0.f};
          s = scale_of(C.scb);
          alu_row_constants(s, q, kq);
          out_of_range = !__all(alu_scale_ok(s));
        }
      }
      // The up block's row constants come from its scale at every step
      // (about 8 VALU ops; keeping a second set live spills registers).
      float ss = s, qq = q, kk = kq;
      bool oor = out_of_range;
      if constexpr (kUp) {
        ss = scale_of(C.scb);
        alu_row_constants(ss, qq, kk);
        oor = !__all(alu_scale_ok(ss));
      }
      if constexpr (!decltype(last)::value) request(N, std::bool_constant<TWO && !kUp>{});
      const unsigned char *xb = xa + b * 512;
      // Rows whose scale is outside the exact range of code * q: the value
      // table (with the code or pair table, the pages' chain on the ALU) for
      // every group.
      if (oor)
        unit<BITS, 0xFF, kValueTable, TAB != kValueTable>(C.w, table, xb, ss, qq, kk, mask_addr, A,
                                                          std::make_integer_sequence<int, 8>{});
      else if constexpr (BITS == 4 && MASK == 0x33 && TAB != kPairTable)
        unit4_phased<TAB>(C.w, table, xb, ss, qq, kk, mask_addr, A);
      else if constexpr (BITS == 2 && MASK == 0x33 && TAB != kPairTable)
        unit2_phased<TAB>(C.w, table, xb, ss, qq, kk, mask_addr, A);
      else
        unit<BITS, MASK, TAB, false>(C.w, table, xb, ss, qq, kk, mask_addr, A, std::make_integer_sequence<int, 8>{});
      if constexpr (TWO && !kUp) return;  // the unit's up block follows
      advance(tile, b);
      ++u;
      // A SIMD issues from its highest-priority ready wave, oldest first
      // among equals; ranking waves by the units they have left lets the
      // younger waves catch up instead of running alone at the end.
      // Pieces that hold tiles shared with other workgroups rank one level
      // higher, so their partials are published before the others finish.
      const int rem = u1 - u + (holds_cross && pl.panels == 1 ? 1 : 0);
      if (rem >= 3) __builtin_amdgcn_s_setprio(3);
      else if (rem == 2) __builtin_amdgcn_s_setprio(2);
      else __builtin_amdgcn_s_setprio(1);
    };
    using UpInSlot1 = std::bool_constant<TWO>;
    if constexpr (kAhead) {
      if (u1 - u0 >= 2) {
        // The range's first unit (gate block), its successor (up block)
        // already requested into S1; it finishes no tile. Its first phase is
        // decoded unless its row scales are out of range.
        const unsigned char *xb = xa + b * 512;
        if (ahead) {
          const bf16x8 x2 = xop(xb, 2), x6 = xop(xb, 6), x0 = xop(xb, 0), x1 = xop(xb, 1);
          mfma(x2, aw[0], acc);
          mfma(x6, aw[1], acc);
          mfma(x0, aw[2], acc);
          mfma(x1, aw[3], acc);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (BITS == 4) unit4_phase2<TAB>(S0.w, table, xb, s, q, kq, mask_addr, acc);
          else unit2_phase2<TAB>(S0.w, table, xb, s, q, kq, mask_addr, acc);
        } else {
          unit<BITS, 0xFF, kValueTable, TAB != kValueTable>(S0.w, table, xb, s, q, kq, mask_addr, acc,
                                                            std::make_integer_sequence<int, 8>{});
        }
        if constexpr (TWO) {
          // the unit's up block (requesting the next unit's gate block into
          // slot 0, where the loop starts)
          step(S1, S0, std::false_type{}, UpInSlot1{});
        } else {
          advance(tile, b);
          ++u;
          const int rem = u1 - u + (holds_cross && pl.panels == 1 ? 1 : 0);  // as at the end of a step
          if (rem >= 3) __builtin_amdgcn_s_setprio(3);
          else if (rem == 2) __builtin_amdgcn_s_setprio(2);
          else __builtin_amdgcn_s_setprio(1);
          S0 = S1;  // the loop starts from slot 0 (one copy of the words, after their load)
        }
      }
    }
    for (;;) {
      if constexpr (!TWO) {
        if (u + 1 == u1) {
          step(S0, S1, std::true_type{}, std::false_type{});
          break;
        }
      }
      step(S0, S1, std::false_type{}, std::false_type{});
      if (u + 1 == u1) {
        step(S1, S0, std::true_type{}, UpInSlot1{});
        break;
      }
      step(S1, S0, std::false_type{}, UpInSlot1{});
    }
    tl = cur;
    if (cross(cur)) stage(cur, acc, acc2);
    else if (u0 <= cur * pl.kp && u1 == (cur + 1) * pl.kp)
      store_tile<TWO>(s_rows, acc, acc2, pl.m, pl.n, cur * 16);
    else if (pl.slots_off > 0) contribute(cur, acc, acc2, cur == tf ? 0 : 1);
    else if (cur == tf) {
      part_f = acc;
      part_f2 = acc2;
    } else {
      part_l = acc;
      part_l2 = acc2;
    }
  }

  const int lane_post = lane_id();
  // ---- Publish the cross tiles of the range: once the staged partials are
  // complete, bump each tile's counter (one lane per tile); the contributor
  // that arrives last adds all partials in a fixed order (panel, then piece),
  // so the result does not depend on arrival order, stores bf16 and resets
  // the counter. Its loads are issued only after its counter update
  // returned, and every other contributor's stores completed before its own
  // update, so no cache-wide fence is needed.
  if (holds_cross) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    for (int t0 = tf; t0 <= tl; t0 += kWave) {
      const int t = t0 + lane_post;
      const bool mine = t <= tl && cross(t);
      int contrib = 0;
      uint32_t old = 0;
      if (mine) {
        contrib = piece_of((t + 1) * pl.kp - 1, pl) - piece_of(t * pl.kp, pl) + 1;
        if (t == tf && tf_bumped) old = tf_old;  // counted inside the loop
        else old = __hip_atomic_fetch_add(&counters[(size_t)t << pl.cshift], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      uint64_t last = __ballot(mine && old == (uint32_t)(contrib * pl.panels - 1));
      while (last) {
        const int i = __builtin_ctzll(last);
        last &= last - 1;
        const int T = t0 + i;
        const int c = __shfl(contrib, i);
        f32x4 sum[NH];
        sum_partials<NH>(pl, ws, T, c, lane_post, sum);
        store_tile<TWO>(s_rows, sum[0], sum[NH - 1], pl.m, pl.n, T * 16);
        if (lane_post == 0) __hip_atomic_store(&counters[(size_t)T << pl.cshift], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }

  // Shared tiles were combined without barriers (slots of their own), or
  // every tile is shared with the other K panels' workgroups (workspace).
  if (pl.slots_off > 0 || pl.panels > 1) return;

  // Two matrices: fetch the first tile's pair back from `kept` (its stores
  // were issued in the loop and have completed by the wait).
  if constexpr (TWO) {
    if (active && tl != tf && u0 > tf * pl.kp && !cross(tf)) {
      constexpr int kSc1 = 16;  // cache-policy bits of the loads
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(kept_base, (short)0, 2048, kRawBufferWord3);
      part_f = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)lane_post * 16, 0, kSc1));
      part_f2 = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 1024 + (uint32_t)lane_post * 16, 0, kSc1));
    }
  }

  // ---- Combine the CU's own shared tiles through LDS. Segment s of the CU
  // holds a partial of its first tile when its range does not cover that
  // whole tile, and a partial of its last tile (when different) when its
  // range ends inside it; cross tiles went through the workspace.
  __syncthreads();  // all waves are done reading x; its LDS holds the partials now
  f32x4 *slots = reinterpret_cast<f32x4 *>(xl);  // [segment][first, last][matrix][lane]
  if (active) {
    slots[(seg * 2 + 0) * NH * kWave + lane_post] = part_f;
    slots[(seg * 2 + 1) * NH * kWave + lane_post] = part_l;
    if constexpr (TWO) {
      slots[((seg * 2 + 0) * NH + 1) * kWave + lane_post] = part_f2;
      slots[((seg * 2 + 1) * NH + 1) * kWave + lane_post] = part_l2;
    }
  }
  __syncthreads();
  if (!active) return;
  // The segment leads each non-cross tile of its range that is not complete
  // in it and that no earlier segment of the CU holds, and adds the CU's
  // partials of it in segment order.
  for (int which = 0; which < 2; ++which) {
    int T;
    if (which == 0) {
      T = tf;
      if (u0 == T * pl.kp && u1 >= (T + 1) * pl.kp) continue;  // complete here
      if (u0 > T * pl.kp) continue;                             // an earlier segment holds T
    } else {
      T = tl;
      if (T == tf || u1 == (T + 1) * pl.kp) continue;  // same as the first, or complete
    }
    if (cross(T)) continue;
    const int t0u = T * pl.kp, t1u = t0u + pl.kp;
    f32x4 sum[NH];
#pragma unroll
    for (int h = 0; h < NH; ++h) sum[h] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int sidx = seg; sidx < nseg; ++sidx) {
      const int a = piece_start(q, sidx), e = piece_start(q, sidx + 1);
      int which_slot;
      if (a >= t0u) which_slot = 0;       // the segment starts inside T
      else if (e > t0u) which_slot = 1;   // the leader, whose range ends inside T
      else break;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const f32x4 v = slots[((sidx * 2 + which_slot) * NH + h) * kWave + lane_post];
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) sum[h][e2] += v[e2];
      }
      if (e >= t1u) break;  // T ends in this segment
    }
    store_tile<TWO>(s_rows, sum[0], sum[NH - 1], pl.m, pl.n, T * 16);
  }
}

// Device memory of trellis_prefill_noalloc (callers that cannot allocate): a
// fixed region of per-tile counters (one per tile of the largest accepted N),
// then the float32 partial tiles. One copy per device, held until the process
// ends; host code reaches it only through the address hipGetSymbolAddress
// returns for the current device.
constexpr size_t kScratchBytes = (size_t)TRELLIS_NOALLOC_SCRATCH_BYTES;
constexpr size_t kScratchCounterBytes = (size_t)(TRELLIS_MAX_N / 16) * 4;
static_assert(kScratchCounterBytes % 256 == 0 && kScratchCounterBytes < kScratchBytes, "scratch layout");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

__global__ __launch_bounds__(256) void zero_u32_kernel(uint32_t *__restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// Which MFMA groups (bit u of the mask) decode through the LDS table; the rest
// use ALU arithmetic. Mix<2, true>: k = 2 with the pair table. The k = 4 and
// k = 2 masks are those of the phased decodes (unit4_phased, unit2_phased).
template <int BITS, bool PAIR = false> struct Mix;
template <> struct Mix<2> { static constexpr int kMask = 0b00110011; };
template <> struct Mix<2, true> { static constexpr int kMask = 0b11111111; };
template <> struct Mix<3> { static constexpr int kMask = 0b01010101; };
template <> struct Mix<4> { static constexpr int kMask = 0b00110011; };

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
bool geometry_ok(const trellis_geom &g) {
  if (g.t != TRELLIS_T || g.l != TRELLIS_L) return false;
  if (g.bits != 2 && g.bits != 3 && g.bits != 4) return false;
  if (g.k < TRELLIS_T || g.k > TRELLIS_MAX_K || g.k % TRELLIS_T != 0) return false;
  if (g.n < 4 || g.n > TRELLIS_MAX_N || g.n % 4 != 0) return false;
  return true;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// The launch macro reports configuration errors through the thread's last
// error; it is cleared before each launch so a stale error from an unrelated
// earlier call is not reported as ours.
void clear_last_error() { (void)hipGetLastError(); }
trellis_status launch_status() { return hipGetLastError() == hipSuccess ? TRELLIS_OK : TRELLIS_E_HIP; }

Plan make_plan(int m, int n, int k, int cus, int table, bool two) {
  Plan pl{};
  pl.m = m;
  pl.n = n;
  pl.k = k;
  pl.tiles = (n + 15) / 16;
  const int kb = k / 256;
  int panels = kb;
  for (int p = 1; p <= kb; ++p) {
    if (kb % p) continue;
    const int stride = (kb / p) * 512 + 16;
    if (table + kRowTableBytes + m * stride <= kMaxLds) {
      panels = p;
      break;
    }
  }
  pl.panels = panels;
  pl.kp = kb / panels;
  pl.x_stride = pl.kp * 512 + 16;
  // Staging divides a vector index idx by the vectors per row (kp * 32):
  // n = idx >> 5 < 2^9, and with l = ceil(log2 kp), m = ceil(2^(9 + l) / kp)
  // (< 2^10) gives n / kp = (n * m) >> (9 + l) exactly (round-up multiplier,
  // Granlund and Montgomery 1994), one 24-bit multiply on the VALU.
  {
    uint32_t l = 0;
    while ((1u << l) < (uint32_t)pl.kp) ++l;
    pl.xshift = 9 + l;
    pl.xmul = (uint32_t)(((1ull << (9 + l)) + (uint32_t)pl.kp - 1) / (uint32_t)pl.kp);
  }
  int groups = cus / panels;
  if (groups < 1) groups = 1;
  pl.units = pl.tiles * pl.kp;  // <= 2^18 tiles * 2^10 blocks
  // Every workgroup gets at least kWaves units unless there is only one.
  while (groups > 1 && groups * kWaves > pl.units) --groups;
  pl.groups = groups;
  pl.cq = pl.units / groups;
  pl.cr = pl.units % groups;
  {
    // Multipliers of div_by: l = ceil(log2 d), m = floor(2^32 (2^l - d) / d) + 1.
    auto base_of = [](uint32_t len) -> uint32_t { return len >= kWaves ? len / kWaves : len > 0 ? 1 : 0; };
    const uint32_t bl = base_of((uint32_t)pl.cq + 1), bs = base_of((uint32_t)pl.cq);
    const uint32_t divisors[8] = {(uint32_t)pl.cq + 1, (uint32_t)pl.cq, bl + 1, bl, bs + 1, bs,
                                  (uint32_t)pl.panels, (uint32_t)pl.kp};
    pl.dl = 0;
    pl.dl2 = 0;
    for (int i = 0; i < 8; ++i) {
      const uint32_t d = divisors[i];
      uint32_t l = 0;
      while ((1ull << l) < d) ++l;
      pl.dm[i] = d <= 1 ? 0u : (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
      (i < 6 ? pl.dl : pl.dl2) |= (d <= 1 ? 0u : l) << (5 * (i % 6));
    }
  }
  // Pieces sharing one tile (per panel): at most (kp - 1) / (shortest piece) + 2.
  const int s_min = pl.cq < kWaves ? pl.cq : kWaves;
  pl.maxc = (pl.kp - 1) / (pl.cq / s_min) + 2;
  // Dynamic LDS: the x panel, later reused for the pieces' partial tiles
  // (two 16x16 fp32 tiles per wave).
  int need = m * pl.x_stride;
  // Partial-tile slots of their own (after x) when they fit: the waves then
  // combine shared tiles without barriers. Otherwise they reuse x's space
  // (one matrix), or every shared tile goes through the workspace (two).
  const int slot_bytes = kCombineBytes * (two ? 2 : 1);
  pl.slots_off = 0;
  if (table + kRowTableBytes + need + slot_bytes + kCombineCounters <= kMaxLds) {
    pl.slots_off = need;
    need += slot_bytes + kCombineCounters;
  }
  if (need < slot_bytes) need = slot_bytes;
  const int fixed = table + kRowTableBytes;  // static LDS: decode table and row table
  pl.lds_bytes = need + fixed > kMinLds ? need : kMinLds - fixed;
  return pl;
}

// Prefill kernels: k = 2, 3, 4 with the value or the code table, and k = 2
// with the pair table, each for one matrix or for gate and up. Variant =
// 2 * (k - 2) + table kind, pair = 6; plus kTables for two matrices.
enum Variant { kVariantPair = 6, kTables = 7, kVariants = 2 * kTables };
constexpr int variant_of(int bits, int tab, bool two) {
  return (tab == kPairTable ? kVariantPair : 2 * (bits - 2) + tab) + (two ? kTables : 0);
}
constexpr int variant_table(int v) { return v % kTables == kVariantPair ? kPairTable : v % kTables % 2; }

struct DeviceState {
  int cus = 0;
  bool lds_attr_set[kVariants] = {};
  // trellis_prefill_noalloc: this device's address of `scratch` (0 until the
  // first such call on the device) and whether its counters were cleared.
  unsigned char *scratch = nullptr;
};
constexpr int kMaxDevices = 64;

struct Workspace {
  float *ws = nullptr;
  size_t ws_floats = 0;
  uint32_t *counters = nullptr;
  size_t ncounters = 0;
};

std::mutex g_mu;
DeviceState g_dev[kMaxDevices];  // fixed: looking a device up allocates nothing
// Workspaces are keyed by device and stream; the per-thread default stream is
// one handle for many streams (one per host thread), so its key also holds
// the calling thread.
struct WsKey {
  int dev;
  hipStream_t stream;
  std::thread::id thread;
  bool operator<(const WsKey &o) const {
    if (dev != o.dev) return dev < o.dev;
    if (stream != o.stream) return stream < o.stream;
    return thread < o.thread;
  }
};
std::map<WsKey, Workspace> g_ws;

typedef void (*PrefillFn)(const uint32_t *, const uint16_t *, const uint32_t *, const uint16_t *, float *, uint32_t *,
                          float *, Plan, RowPtrs);
template <bool TWO>
PrefillFn prefill_fn_of(int v) {
  switch (v) {
    case 0: return &prefill_kernel<2, Mix<2>::kMask, kValueTable, TWO>;
    case 1: return &prefill_kernel<2, Mix<2>::kMask, kCodeTable, TWO>;
    case 2: return &prefill_kernel<3, Mix<3>::kMask, kValueTable, TWO>;
    case 3: return &prefill_kernel<3, Mix<3>::kMask, kCodeTable, TWO>;
    case 4: return &prefill_kernel<4, Mix<4>::kMask, kValueTable, TWO>;
    case 5: return &prefill_kernel<4, Mix<4>::kMask, kCodeTable, TWO>;
    default: return &prefill_kernel<2, Mix<2, true>::kMask, kPairTable, TWO>;
  }
}
PrefillFn prefill_fn(int v) { return v >= kTables ? prefill_fn_of<true>(v - kTables) : prefill_fn_of<false>(v); }

trellis_status device_state(DeviceState *&st, int v) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TRELLIS_E_HIP;
  DeviceState &d = g_dev[dev];
  if (d.cus == 0) {
    if (hipDeviceGetAttribute(&d.cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || d.cus <= 0)
      return TRELLIS_E_HIP;
  }
  if (!d.lds_attr_set[v]) {
    if (hipFuncSetAttribute(reinterpret_cast<const void *>(prefill_fn(v)), hipFuncAttributeMaxDynamicSharedMemorySize,
                            kMaxLds - table_bytes(variant_table(v)) - kRowTableBytes) != hipSuccess)
      return TRELLIS_E_HIP;
    d.lds_attr_set[v] = true;
  }
  st = &d;
  return TRELLIS_OK;
}

// Per (device, stream) workspace: partial tiles and self-resetting counters.
// Grown on demand and kept until process exit. A grown-out buffer is not
// freed: launches still queued on the stream, and HIP graphs captured from
// earlier calls, hold its address.
trellis_status workspace(hipStream_t stream, size_t ws_floats, size_t ncounters, Workspace *&out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TRELLIS_E_HIP;
  const std::thread::id tid = stream == hipStreamPerThread ? std::this_thread::get_id() : std::thread::id();
  Workspace &w = g_ws[WsKey{dev, stream, tid}];
  if (w.ws_floats < ws_floats) {
    float *p = nullptr;
    if (hipMalloc(&p, ws_floats * sizeof(float)) != hipSuccess) return TRELLIS_E_HIP;
    w.ws = p;
    w.ws_floats = ws_floats;
  }
  if (w.ncounters < ncounters) {
    uint32_t *c = nullptr;
    if (hipMalloc(&c, ncounters * sizeof(uint32_t)) != hipSuccess) return TRELLIS_E_HIP;
    // Zeroed by a kernel on the stream, ordered before the first use (a
    // memset node would be unsafe if a caller captured the stream).
    const dim3 grid((unsigned)((ncounters + 255) / 256));
    hipLaunchKernelGGL(zero_u32_kernel, grid, dim3(256), 0, stream, c, (int64_t)ncounters);
    if (hipGetLastError() != hipSuccess) return TRELLIS_E_HIP;
    w.counters = c;
    w.ncounters = ncounters;
  }
  out = &w;
  return TRELLIS_OK;
}

}  // namespace
}  // namespace trellis

using namespace trellis;

extern "C" {

int trellis_supported(trellis_geom g, int32_t m) {
  return geometry_ok(g) && m >= TRELLIS_MIN_M && m <= TRELLIS_MAX_M;
}

const char *trellis_status_string(trellis_status s) {
  switch (s) {
    case TRELLIS_OK: return "ok";
    case TRELLIS_E_GEOMETRY: return "unsupported geometry (need t=256, l=12, bits 2/3/4, K%256==0, N%4==0)";
    case TRELLIS_E_M: return "unsupported batch: m must be in [5, 15] (prefill) or [1, 4] (matvec)";
    case TRELLIS_E_NULL: return "null pointer argument";
    case TRELLIS_E_ALIGN: return "misaligned pointer argument";
    case TRELLIS_E_HIP: return "HIP runtime error";
    case TRELLIS_E_SCRATCH: return "the call needs more workspace than the no-allocation entry point's fixed scratch holds";
  }
  return "unknown status";
}

trellis_status trellis_decode(const uint32_t *codes, const uint16_t *scales_bf16, trellis_geom g,
                              uint16_t *w_bf16, void *hip_stream) {
  if (!geometry_ok(g)) return TRELLIS_E_GEOMETRY;
  if (!codes || !scales_bf16 || !w_bf16) return TRELLIS_E_NULL;
  if (!aligned(codes, 16) || !aligned(w_bf16, 16) || !aligned(scales_bf16, 2)) return TRELLIS_E_ALIGN;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  const int64_t threads = (int64_t)g.n * (g.k / 8);
  const dim3 grid((unsigned)((threads + 255) / 256)), block(256);
  clear_last_error();
  switch (g.bits) {
    case 2: hipLaunchKernelGGL(decode_kernel<2>, grid, block, 0, stream, codes, scales_bf16, g.n, g.k, w_bf16); break;
    case 3: hipLaunchKernelGGL(decode_kernel<3>, grid, block, 0, stream, codes, scales_bf16, g.n, g.k, w_bf16); break;
    default: hipLaunchKernelGGL(decode_kernel<4>, grid, block, 0, stream, codes, scales_bf16, g.n, g.k, w_bf16); break;
  }
  return launch_status();
}

}  // extern "C"

namespace trellis {
namespace {

// Decode-table override for tests and tuning (trellis_test_force_table):
// -1 lets the library choose; value/code/pair force that table (pair applies
// to k = 2 only). One relaxed atomic load per call, no environment lookup.
std::atomic<int> g_force_table{-1};

int table_override(int bits) {
  const int t = g_force_table.load(std::memory_order_relaxed);
  if (t == kPairTable && bits != 2) return -1;
  return t;
}

// One launch of the layer on m <= 15 rows (any m >= 1 with a valid
// geometry; the entry points restrict m to their regimes): x row i at
// x_rows[i], output row i at out_rows[i]. With a second matrix (codes2,
// scales2, the up projection) the output is the elementwise tail of the
// two projections, from the same launch.
// noalloc: the workspace is this device's `scratch` array instead of the
// stream's allocated workspace; a call whose workspace would not fit returns
// TRELLIS_E_SCRATCH before any GPU work.
trellis_status launch_rows(const uint16_t *const *x_rows, uint16_t *const *out_rows, int32_t m,
                           const uint32_t *codes, const uint16_t *scales_bf16, const uint32_t *codes2,
                           const uint16_t *scales2, trellis_geom g, hipStream_t stream, bool noalloc = false) {
  const bool two = codes2 != nullptr;
  int cus = 0;
  {
    DeviceState *st0 = nullptr;
    const trellis_status rc0 = device_state(st0, variant_of(g.bits, kValueTable, two));
    if (rc0 != TRELLIS_OK) return rc0;
    cus = st0->cus;
  }
  // The table that splits x into the fewest K panels; among equals the pair
  // table (k = 2), then the value table. The test hook (trellis_test_force_table)
  // overrides the choice.
  int tab = kValueTable;
  Plan pl = make_plan(m, g.n, g.k, cus, table_bytes(kValueTable), two);
  const int forced = table_override(g.bits);
  if (forced >= 0) {
    tab = forced;
    pl = make_plan(m, g.n, g.k, cus, table_bytes(tab), two);
  } else {
    const Plan pc = make_plan(m, g.n, g.k, cus, table_bytes(kCodeTable), two);
    if (pc.panels < pl.panels) {
      pl = pc;
      tab = kCodeTable;
    }
    if (g.bits == 2) {
      const Plan pp = make_plan(m, g.n, g.k, cus, table_bytes(kPairTable), two);
      if (pp.panels <= pl.panels) {
        pl = pp;
        tab = kPairTable;
      }
    }
  }
  const int v = variant_of(g.bits, tab, two);
  DeviceState *st = nullptr;
  trellis_status rc = device_state(st, v);
  if (rc != TRELLIS_OK) return rc;
  // Partial slots, then (two matrices) one 2 KB slot per wave for the pair
  // kept through the loop.
  const size_t slot_floats = (size_t)pl.tiles * pl.panels * pl.maxc * 256 * (two ? 2 : 1);
  const size_t kept_floats = two ? (size_t)pl.groups * pl.panels * kWaves * 512 : 0;
  float *ws = nullptr;
  uint32_t *counters = nullptr;
  if (noalloc) {
    // Counters (zero between calls: the kernel resets each one it uses, and
    // the first call on the device cleared them all), then the partial slots.
    if (two || (slot_floats + kept_floats) * 4 > kScratchBytes - kScratchCounterBytes) return TRELLIS_E_SCRATCH;
    counters = reinterpret_cast<uint32_t *>(st->scratch);
    ws = reinterpret_cast<float *>(st->scratch + kScratchCounterBytes);
    pl.cshift = 0;
  } else {
    Workspace *w = nullptr;
    pl.cshift = 4;
    rc = workspace(stream, slot_floats + kept_floats, (size_t)pl.tiles << pl.cshift, w);
    if (rc != TRELLIS_OK) return rc;
    ws = w->ws;
    counters = w->counters;
  }
  RowPtrs rp{};
  pl.x_contiguous = 1;
  for (int i = 0; i < m; ++i) {
    rp.x[i] = x_rows[i];
    if (x_rows[i] != x_rows[0] + (size_t)i * g.k) pl.x_contiguous = 0;
  }
  for (int i = 0; i < m; ++i) rp.out[i] = out_rows[i];
  // Unused slots repeat row 0 (never dereferenced).
  for (int i = m; i < kMaxRows; ++i) {
    rp.x[i] = rp.x[0];
    rp.out[i] = rp.out[0];
  }
  const dim3 grid((unsigned)(pl.groups * pl.panels)), block(kWgThreads);
  clear_last_error();
  hipLaunchKernelGGL(prefill_fn(v), grid, block, pl.lds_bytes, stream, codes, scales_bf16, codes2, scales2, ws,
                     counters, ws + slot_floats, pl, rp);
  return launch_status();
}

// Plain calls: x [m, K] and out [m, N], rows consecutive.
trellis_status launch_linear(const uint16_t *x_bf16, int32_t m, const uint32_t *codes,
                             const uint16_t *scales_bf16, const uint32_t *codes2, const uint16_t *scales2,
                             trellis_geom g, uint16_t *out_bf16, void *hip_stream) {
  const bool two = codes2 != nullptr || scales2 != nullptr;
  if (!x_bf16 || !codes || !scales_bf16 || !out_bf16 || (two && (!codes2 || !scales2))) return TRELLIS_E_NULL;
  if (!aligned(x_bf16, 16) || !aligned(codes, 16) || !aligned(out_bf16, 16) || !aligned(scales_bf16, 2))
    return TRELLIS_E_ALIGN;
  if (two && (!aligned(codes2, 16) || !aligned(scales2, 2))) return TRELLIS_E_ALIGN;
  const uint16_t *xr[kMaxRows];
  uint16_t *orow[kMaxRows];
  for (int i = 0; i < m; ++i) {
    xr[i] = x_bf16 + (size_t)i * g.k;
    orow[i] = out_bf16 + (size_t)i * g.n;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  return launch_rows(xr, orow, m, codes, scales_bf16, codes2, scales2, g,
                     reinterpret_cast<hipStream_t>(hip_stream));
}

}  // namespace
}  // namespace trellis

extern "C" {

trellis_status trellis_prefill(const uint16_t *x_bf16, int32_t m, const uint32_t *codes,
                               const uint16_t *scales_bf16, trellis_geom g, uint16_t *out_bf16,
                               void *hip_stream) {
  if (!geometry_ok(g)) return TRELLIS_E_GEOMETRY;
  if (m < TRELLIS_MIN_M || m > TRELLIS_MAX_M) return TRELLIS_E_M;
  return launch_linear(x_bf16, m, codes, scales_bf16, nullptr, nullptr, g, out_bf16, hip_stream);
}

trellis_status trellis_matvec(const uint16_t *x_bf16, int32_t m, const uint32_t *codes,
                              const uint16_t *scales_bf16, trellis_geom g, uint16_t *out_bf16,
                              void *hip_stream) {
  if (!geometry_ok(g)) return TRELLIS_E_GEOMETRY;
  if (m < 1 || m > TRELLIS_MATVEC_MAX_M) return TRELLIS_E_M;
  return launch_linear(x_bf16, m, codes, scales_bf16, nullptr, nullptr, g, out_bf16, hip_stream);
}

trellis_status trellis_prefill_packed(const uint16_t *const *x_groups, const int32_t *rows, int32_t groups,
                                      const uint32_t *codes, const uint16_t *scales_bf16, trellis_geom g,
                                      uint16_t *const *out_groups, void *hip_stream) {
  if (!geometry_ok(g)) return TRELLIS_E_GEOMETRY;
  if (!x_groups || !rows || !out_groups || !codes || !scales_bf16) return TRELLIS_E_NULL;
  if (groups < 1 || groups > TRELLIS_MAX_GROUPS) return TRELLIS_E_M;
  int64_t total = 0;
  for (int32_t i = 0; i < groups; ++i) {
    if (rows[i] < 0 || rows[i] > TRELLIS_MAX_GROUP_ROWS) return TRELLIS_E_M;
    total += rows[i];
    if (rows[i] == 0) continue;
    if (!x_groups[i] || !out_groups[i]) return TRELLIS_E_NULL;
    if (!aligned(x_groups[i], 16) || !aligned(out_groups[i], 16)) return TRELLIS_E_ALIGN;
  }
  if (total < 1) return TRELLIS_E_M;
  if (!aligned(codes, 16) || !aligned(scales_bf16, 2)) return TRELLIS_E_ALIGN;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  std::lock_guard<std::mutex> lock(g_mu);
  // Packed rows in group order, in launches of at most TRELLIS_MAX_M rows.
  const uint16_t *xr[kMaxRows];
  uint16_t *orow[kMaxRows];
  int n = 0;
  for (int32_t i = 0; i < groups; ++i) {
    for (int32_t r = 0; r < rows[i]; ++r) {
      xr[n] = x_groups[i] + (size_t)r * g.k;
      orow[n] = out_groups[i] + (size_t)r * g.n;
      if (++n == TRELLIS_MAX_M) {
        const trellis_status rc = launch_rows(xr, orow, n, codes, scales_bf16, nullptr, nullptr, g, stream);
        if (rc != TRELLIS_OK) return rc;
        n = 0;
      }
    }
  }
  if (n > 0) return launch_rows(xr, orow, n, codes, scales_bf16, nullptr, nullptr, g, stream);
  return TRELLIS_OK;
}

trellis_status trellis_prefill_noalloc(const uint16_t *x_bf16, int32_t m, const uint32_t *codes,
                                       const uint16_t *scales_bf16, trellis_geom g, uint16_t *out_bf16,
                                       void *hip_stream) {
  if (!geometry_ok(g)) return TRELLIS_E_GEOMETRY;
  if (m < TRELLIS_MIN_M || m > TRELLIS_MAX_M) return TRELLIS_E_M;
  if (!x_bf16 || !codes || !scales_bf16 || !out_bf16) return TRELLIS_E_NULL;
  if (!aligned(x_bf16, 16) || !aligned(codes, 16) || !aligned(out_bf16, 16) || !aligned(scales_bf16, 2))
    return TRELLIS_E_ALIGN;
  hipStream_t stream = reinterpret_cast<hipStream_t>(hip_stream);
  std::lock_guard<std::mutex> lock(g_mu);
  // Set-up, once per device with that device current: the device's own
  // address of `scratch` (the array's name is only a host-side stand-in),
  // and the counter region cleared by a kernel on the caller's stream, so it
  // is ordered before this call's launch (and, calls on one device being
  // serialised by the caller, before every later call).
  DeviceState *st = nullptr;
  trellis_status rc = device_state(st, variant_of(g.bits, kValueTable, false));
  if (rc != TRELLIS_OK) return rc;
  if (!st->scratch) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TRELLIS_E_HIP;
    const int64_t n = (int64_t)(kScratchCounterBytes / 4);
    clear_last_error();
    hipLaunchKernelGGL(zero_u32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                       reinterpret_cast<uint32_t *>(p), n);
    if (hipGetLastError() != hipSuccess) return TRELLIS_E_HIP;
    st->scratch = static_cast<unsigned char *>(p);
  }
  const uint16_t *xr[kMaxRows];
  uint16_t *orow[kMaxRows];
  for (int i = 0; i < m; ++i) {
    xr[i] = x_bf16 + (size_t)i * g.k;
    orow[i] = out_bf16 + (size_t)i * g.n;
  }
  return launch_rows(xr, orow, m, codes, scales_bf16, nullptr, nullptr, g, stream, true);
}

int trellis_test_force_table(int kind) {
  if (kind < -1 || kind > 2) return -2;
  return g_force_table.exchange(kind);
}

trellis_status trellis_gate_up(const uint16_t *x_bf16, int32_t m, const uint32_t *codes_gate,
                               const uint16_t *scales_gate, const uint32_t *codes_up, const uint16_t *scales_up,
                               trellis_geom g, uint16_t *h_bf16, void *hip_stream) {
  if (!geometry_ok(g)) return TRELLIS_E_GEOMETRY;
  if (m < 1 || m > TRELLIS_MAX_M) return TRELLIS_E_M;
  if (!codes_up || !scales_up) return TRELLIS_E_NULL;
  return launch_linear(x_bf16, m, codes_gate, scales_gate, codes_up, scales_up, g, h_bf16, hip_stream);
}

}  // extern "C"
