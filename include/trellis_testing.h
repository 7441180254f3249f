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

#ifdef __cplusplus
}
#endif

#endif /* TRELLIS_TESTING_H */
