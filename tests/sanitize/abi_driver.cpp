// Calls every entry point of the C ABI with arguments its host-side
// validation must reject, plus in-domain calls (which, with no GPU present,
// must fail cleanly with TRELLIS_E_HIP), for an AddressSanitizer /
// UndefinedBehaviorSanitizer build of the library's host code
// (tests/test_sanitizers.py). Prints one line per call; exits 0 if every
// status is the expected one.
#include <stdint.h>
#include <stdio.h>

#include "trellis.h"
#include "trellis_testing.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
  printf("%-40s %d (%s)\n", what, got, trellis_status_string((trellis_status)got));
  if (got != want) {
    printf("  expected %d\n", want);
    ++failures;
  }
}

int main() {
  alignas(16) static uint16_t buf[4096];
  const uint16_t *x = buf;
  const uint32_t *codes = reinterpret_cast<const uint32_t *>(buf);
  const uint16_t *scales = buf;
  uint16_t *out = buf + 1024;
  trellis_geom good{256, 512, 256, 12, 4};
  trellis_geom bad_k{256, 500, 256, 12, 4};
  trellis_geom bad_bits{256, 512, 256, 12, 5};
  trellis_geom bad_n{255, 512, 256, 12, 4};
  expect("supported good", trellis_supported(good, 5), 1);
  expect("supported m=4", trellis_supported(good, 4), 0);
  expect("supported bad k", trellis_supported(bad_k, 5), 0);
  expect("prefill bad geometry", trellis_prefill(x, 5, codes, scales, bad_k, out, nullptr), TRELLIS_E_GEOMETRY);
  expect("prefill bad bits", trellis_prefill(x, 5, codes, scales, bad_bits, out, nullptr), TRELLIS_E_GEOMETRY);
  expect("prefill bad n", trellis_prefill(x, 5, codes, scales, bad_n, out, nullptr), TRELLIS_E_GEOMETRY);
  expect("prefill m=16", trellis_prefill(x, 16, codes, scales, good, out, nullptr), TRELLIS_E_M);
  expect("prefill null x", trellis_prefill(nullptr, 5, codes, scales, good, out, nullptr), TRELLIS_E_NULL);
  expect("prefill misaligned out", trellis_prefill(x, 5, codes, scales, good, out + 1, nullptr), TRELLIS_E_ALIGN);
  expect("matvec m=5", trellis_matvec(x, 5, codes, scales, good, out, nullptr), TRELLIS_E_M);
  expect("matvec m=0", trellis_matvec(x, 0, codes, scales, good, out, nullptr), TRELLIS_E_M);
  expect("decode null w", trellis_decode(codes, scales, good, nullptr, nullptr), TRELLIS_E_NULL);
  expect("decode bad geometry", trellis_decode(codes, scales, bad_k, out, nullptr), TRELLIS_E_GEOMETRY);
  expect("gate_up null up", trellis_gate_up(x, 5, codes, scales, nullptr, scales, good, out, nullptr), TRELLIS_E_NULL);
  expect("gate_up m=16", trellis_gate_up(x, 16, codes, scales, codes, scales, good, out, nullptr), TRELLIS_E_M);
  const uint16_t *xg[3] = {x, nullptr, x};
  uint16_t *og[3] = {out, nullptr, out};
  int32_t rows[3] = {3, 0, 4};
  int32_t bad_rows[3] = {3, -1, 4};
  expect("packed groups=0", trellis_prefill_packed(xg, rows, 0, codes, scales, good, og, nullptr), TRELLIS_E_M);
  expect("packed negative rows", trellis_prefill_packed(xg, bad_rows, 3, codes, scales, good, og, nullptr), TRELLIS_E_M);
  expect("packed null rows", trellis_prefill_packed(xg, nullptr, 3, codes, scales, good, og, nullptr), TRELLIS_E_NULL);
  expect("table hook bad", trellis_test_force_table(9), -2);
  expect("table hook set", trellis_test_force_table(1), -1);
  expect("table hook reset", trellis_test_force_table(-1), 1);
  // In-domain calls: with no GPU the library must report a HIP error, not crash.
  expect("prefill no gpu", trellis_prefill(x, 5, codes, scales, good, out, nullptr), TRELLIS_E_HIP);
  expect("packed no gpu", trellis_prefill_packed(xg, rows, 3, codes, scales, good, og, nullptr), TRELLIS_E_HIP);
  printf("abi driver %s\n", failures ? "FAILED" : "ok");
  return failures ? 1 : 0;
}
