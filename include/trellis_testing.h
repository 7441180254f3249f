/*
 * trellis_testing.h -- test and tuning hooks of libtrellis.so. Not part of
 * the layer's interface: production callers never need them.
 */
#ifndef TRELLIS_TESTING_H
#define TRELLIS_TESTING_H

#ifdef __cplusplus
extern "C" {
#endif

/* Decode table used by the prefill kernels of later calls, process-wide:
 *   -1  the library's own choice (the default),
 *    0  window -> float32 value table,
 *    1  window -> float16 code table,
 *    2  14-bit pair of windows -> two float16 codes (k = 2 only; other k keep
 *       the library's choice).
 * Every table gives the same weights; the hook lets tests run each table on
 * every k. Returns the previous setting, or -2 (and changes nothing) for a
 * value outside [-1, 2]. Thread-safe; a call already enqueued is not
 * affected. */
int trellis_test_force_table(int kind);

/* Contraction of later calls, process-wide: 0 the bf16 MFMA kernels (the
 * default), 1 a VALU variant (v_dot2c_f32_bf16 dot products per lane, x read
 * from LDS per row) where one exists: k = 4, value table, one matrix, m = 5
 * or m = 1; other calls keep MFMA. The variant exists to measure the two
 * against each other and assumes row scales within [2^-110, 2^110] in
 * magnitude. Returns the previous setting, or -2 for a value outside [0, 1]. */
int trellis_test_force_contraction(int kind);

#ifdef __cplusplus
}
#endif

#endif /* TRELLIS_TESTING_H */
