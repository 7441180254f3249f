/*
 * trellis.h -- C ABI of the packed Trellis-quantized linear layer for
 * narrow-batch prefill on AMD Instinct MI355X (gfx950).
 *
 * The layer computes out[M, N] = x[M, K] . W^T in bf16, where W[N, K] is never
 * stored: every weight is decoded on the fly from a packed code stream.
 * Method: web page "mlx-bun 0.2.0 -> 0.4.0" (npm diff, page 57), section
 * src/model/trellis-wide-prefill.ts -- the Metal kernel body (decode and
 * narrow-M dot) and its host wrapper (shape and layout checks, eligibility
 * predicate). The materialising decode corresponds to the "expand" mode named
 * on the page "mlx-bun 0.4.0 -> 0.5.0" (npm diff, page 26), section
 * src/model/trellis-linear.ts.
 *
 * Data formats (all buffers are caller-owned DEVICE memory):
 *   bf16 values are passed as their 16-bit patterns (uint16_t).
 *   codes   uint32 [N, K*bits/32], row-major. Row n holds K/256 blocks of
 *           256*bits/32 words (16, 24 or 32 words for bits = 2, 3, 4); block
 *           b of row n starts at word n*(K*bits/32) + b*(256*bits/32).
 *           Within a block the bits form one cyclic stream of 256*bits bits,
 *           read LSB-first inside each word. Weight t of the block
 *           (0 <= t < 256, column kk = 256*b + t) takes the 12 stream bits
 *           starting at bit (255 - t)*bits, wrapping to the block's first
 *           word past its end.
 *   decode  window -> z = window*34038481 + 76625530 (mod 2^32);
 *           code = (sum of the 4 bytes of z) - 510;
 *           value = float32 code/147.800537109375 by the page's reciprocal
 *           refinement; weight = bf16_RNE(float32(value * scale[n])).
 *   scales  bf16 [N], one per output row.
 *   x       bf16 [M, K], row-major, rows contiguous.
 *   out     bf16 [M, N], row-major; out[m, n] = bf16_RNE(sum_kk W[n,kk]*x[m,kk])
 *           accumulated in float32 (summation order is unspecified).
 *
 * Accepted domain (anything else is rejected before any GPU work):
 *   T == 256, L == 12, bits in {2, 3, 4};
 *   K % 256 == 0, 256 <= K <= TRELLIS_MAX_K;
 *   N % 4 == 0, 4 <= N <= TRELLIS_MAX_N;
 *   5 <= M <= 15 for trellis_prefill (the narrow-batch regime of the page's
 *   eligibility predicate), 1 <= M <= 4 for trellis_matvec, 1 <= M <= 15
 *   for trellis_gate_up, any number of packed rows for
 *   trellis_prefill_packed (see there);
 *   x, codes, out and w 16-byte aligned; scales 2-byte aligned; no pointer
 *   NULL. The page's fixed K = 5120 is generalised to any multiple of 256.
 *
 * Execution: each call enqueues its work on `stream` (a hipStream_t; NULL is
 * the default stream) and returns without waiting. The stream and every
 * buffer must belong to the current device (hipGetDevice): the library sizes
 * its launch and keeps its state for that device. trellis_decode keeps no
 * state. The other calls sum tiles that are split across workgroups
 * through a workspace (float32 partial tiles and per-tile counters that the
 * kernel leaves at zero for the next call) owned by the library, one per
 * (device, stream) -- and, for the per-thread default stream
 * hipStreamPerThread, one per calling host thread as well. It is allocated
 * with hipMalloc on the first call that needs it, grown when a later call
 * needs more (the outgrown buffer is not freed: queued launches and captured
 * graphs may hold its address) and kept until the process exits.
 * Consequences:
 *   - calls on one stream are ordered by the stream and share its workspace
 *     safely; calls on different streams use different workspaces;
 *   - a call that allocates cannot be captured into a HIP graph: make one
 *     call of the same shape on the stream before capturing it;
 *   - a captured launch keeps the capture stream's workspace. Replay the
 *     graph on the capture stream, or on a stream ordered with every other
 *     use of the capture stream's workspace: a replay that overlaps an
 *     eager call (or another replay) on the capture stream races on the
 *     same counters and partial tiles and can give wrong results.
 * Host-side state is guarded by a mutex, so calls may come from several
 * threads. Errors are returned, never thrown; a validation error leaves every
 * output untouched.
 *
 * Performance: every wave of the prefill kernels reads its launch arguments
 * first thing. Run with the HIP runtime's HIP_FORCE_DEV_KERNARG=1 (set
 * before the runtime loads) so they sit in device memory; with the default
 * placement in host memory each launch takes about 1 us longer (up to 3 us
 * for trellis_gate_up and trellis_prefill_packed).
 *
 * Decode table: the library picks, per call, the LDS table that lets the
 * most of x stay in one K panel (a window -> value table, a window ->
 * float16 code table, or for k = 2 a table of code pairs); every table gives
 * the same weights. trellis_testing.h has a hook that forces one, for tests.
 */
#ifndef TRELLIS_H
#define TRELLIS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TRELLIS_T 256
#define TRELLIS_L 12
#define TRELLIS_MIN_M 5
#define TRELLIS_MAX_M 15
#define TRELLIS_MATVEC_MAX_M 4
#define TRELLIS_MAX_K (1 << 18)
#define TRELLIS_MAX_N (1 << 22)
#define TRELLIS_MAX_GROUPS 4096
#define TRELLIS_MAX_GROUP_ROWS (1 << 20)
/* Device memory of trellis_prefill_noalloc, per GPU: 1 MiB of tile counters
 * plus 31 MiB of float32 partial tiles. */
#define TRELLIS_NOALLOC_SCRATCH_BYTES (32u << 20)

/* Geometry of one packed linear layer: n output rows (out features), k input
 * columns (in features), block length t (must be 256), window length l (must
 * be 12), bits per code (2, 3 or 4). */
typedef struct trellis_geom {
    int32_t n;
    int32_t k;
    int32_t t;
    int32_t l;
    int32_t bits;
} trellis_geom;

typedef enum trellis_status {
    TRELLIS_OK = 0,
    TRELLIS_E_GEOMETRY = -1, /* t, l, bits, n or k outside the accepted domain */
    TRELLIS_E_M = -2,        /* m outside [5, 15] (prefill) or [1, 4] (matvec); bad packed group or row counts */
    TRELLIS_E_NULL = -3,     /* a required pointer is NULL */
    TRELLIS_E_ALIGN = -4,    /* a pointer is not aligned as documented */
    TRELLIS_E_HIP = -5,      /* the HIP runtime reported a launch error */
    TRELLIS_E_SCRATCH = -6   /* trellis_prefill_noalloc: the call's workspace exceeds the fixed scratch */
} trellis_status;

/* 1 if (g, m) is inside the accepted domain of trellis_prefill, else 0.
 * Pure: no GPU access, no side effects. Mirrors the page's eligibility
 * predicate (page 57, wideTrellisPrefillEligible) with K and N generalised. */
int trellis_supported(trellis_geom g, int32_t m);

/* Materialise W[N, K] as bf16 (w_bf16 is [N, K] row-major) from codes
 * [N, K*bits/32] and scales [N]. The result is bit-exact: it has exactly one
 * correct value per weight. Page 57, kernel body (decode steps); page 26,
 * trellis-linear.ts (expand mode). */
trellis_status trellis_decode(const uint32_t *codes, const uint16_t *scales_bf16,
                              trellis_geom g, uint16_t *w_bf16, void *hip_stream);

/* out[M, N] = x[M, K] . W^T with W decoded on the fly (page 57, kernel body
 * and host wrapper). x is [m, K] bf16, out is [m, N] bf16, both row-major.
 * Every output lies within 1 bf16 ulp of itself plus 1e-5 * sum|w*x| of the
 * float64 sum of the same bf16 products. */
trellis_status trellis_prefill(const uint16_t *x_bf16, int32_t m,
                               const uint32_t *codes, const uint16_t *scales_bf16,
                               trellis_geom g, uint16_t *out_bf16, void *hip_stream);

/* The small-batch regime below the wide kernel's M = 5: 1 <= m <= 4 rows
 * (decode tokens), same formats, same decode and the same tolerance as
 * trellis_prefill; m outside [1, 4] returns TRELLIS_E_M. The pages' model
 * code tells groups of at most TRELLIS_MATVEC_MAX_M rows (the matvec regime)
 * from larger prefill groups (page "mlx-bun 0.4.0 -> 0.5.0" (npm diff,
 * page 26), section src/model/qwen3_5.ts, mixed and layer-by-layer forward
 * passes) and start the wide kernel at M = 5 (page 57,
 * nativeTrellisWidePrefill); the limit's value is not printed, and 4 is the
 * reading that leaves no gap. Each weight is used at most 4 times, so the
 * call costs what the decode costs. */
trellis_status trellis_matvec(const uint16_t *x_bf16, int32_t m,
                              const uint32_t *codes, const uint16_t *scales_bf16,
                              trellis_geom g, uint16_t *out_bf16, void *hip_stream);

/* Token packing: the rows of several independent inputs go through the
 * layer together, so one decode of W serves all of them (page "mlx-bun
 * 0.4.0 -> 0.5.0" (npm diff, page 26), section src/model/token-groups.ts:
 * the tokenwise operation runs on the concatenation of the groups' rows and
 * the result is cut back into each group's shape; section
 * src/model/qwen3_5.ts, mixed forward pass, applies it to the MLP).
 *   x_groups[i]   bf16 [rows[i], K], row-major, 16-byte aligned
 *   out_groups[i] bf16 [rows[i], N], row-major, 16-byte aligned
 * for 0 <= i < groups (1 <= groups <= TRELLIS_MAX_GROUPS; 0 <= rows[i] <=
 * TRELLIS_MAX_GROUP_ROWS; a group with no rows may pass NULL pointers; at
 * least one row in total). The packed rows, in group order, are processed
 * in launches of at most TRELLIS_MAX_M rows (the wide kernel's limit; the
 * page's concatenation has no limit of its own), and no concatenated copy
 * of x or out is made: the kernel reads x rows and writes output rows
 * through per-row pointers. Each output row meets trellis_prefill's
 * tolerance; the summation order, and so the last bit, may differ from an
 * unpacked call. Same formats, codes and scales as trellis_prefill.
 * Validation errors (TRELLIS_E_M for bad group or row counts) are found
 * before any launch; a launch error stops the call with earlier launches
 * already enqueued. */
trellis_status trellis_prefill_packed(const uint16_t *const *x_groups, const int32_t *rows, int32_t groups,
                                      const uint32_t *codes, const uint16_t *scales_bf16, trellis_geom g,
                                      uint16_t *const *out_groups, void *hip_stream);

/* The MLP's gate and up projections of one x, fused:
 *   h[M, N] = bf16(bf16(gate * bf16(sigmoid(gate))) * up),
 *   gate = bf16(x . Wg^T), up = bf16(x . Wu^T),
 * following the page's model code, where each step yields a bf16 array
 * (page "mlx-bun 0.0.4" (npm, page 62), section src/model/minicpm5.ts, MLP
 * forward); sigmoid is evaluated in float32. Wg and Wu share the geometry g
 * (same N, K and bits) and the formats above; 1 <= m <= 15. One launch
 * decodes both code streams against one staging of x, each block of a gate
 * tile next to the same block of the up tile, so the wave that completes a
 * tile holds both float32 sums and writes h; the projections never reach
 * memory. */
trellis_status trellis_gate_up(const uint16_t *x_bf16, int32_t m,
                               const uint32_t *codes_gate, const uint16_t *scales_gate,
                               const uint32_t *codes_up, const uint16_t *scales_up,
                               trellis_geom g, uint16_t *h_bf16, void *hip_stream);

/* trellis_prefill for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * same arguments, formats, tolerance and kernels, but the workspace is a
 * fixed array of TRELLIS_NOALLOC_SCRATCH_BYTES in the library's device image
 * (one per GPU, held until the process ends) instead of memory the library
 * allocates. The call itself allocates nothing: no hipMalloc, no hipFree, no
 * allocating library routine. Its first call on a GPU looks up that GPU's
 * copy of the array and clears its counter region with a kernel on `stream`.
 * Limit: the partial tiles must fit in 31 MiB -- about
 * ceil(N/16) * (K panels) * (contributors per tile) KiB; every shape with
 * N <= 65536 at K = 5120 (and the K = 17408, N = 5120 down projection) fits.
 * Larger calls return TRELLIS_E_SCRATCH before any GPU work. All calls on
 * one GPU share its array, whatever their stream: calls that overlap in time
 * on one GPU race on it and can give wrong results, so the caller must order
 * them (one stream, or events). */
trellis_status trellis_prefill_noalloc(const uint16_t *x_bf16, int32_t m,
                                       const uint32_t *codes, const uint16_t *scales_bf16,
                                       trellis_geom g, uint16_t *out_bf16, void *hip_stream);

/* Static, NUL-terminated description of a status code. */
const char *trellis_status_string(trellis_status s);

#ifdef __cplusplus
}
#endif

#endif /* TRELLIS_H */
