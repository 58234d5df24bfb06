/*
 * echo.h -- C ABI of libecho: the per-rank compute path of Echo's
 * error-compensated 4-bit all-reduce on one AMD Instinct MI355X (gfx950).
 *
 * Method: "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication for
 * LLM Training and Inference" (arXiv 2610.14277v1).  The all-reduce carries
 * 4-bit integer codes, accumulates them in a wider floating-point format and
 * passes no value through the quantizer more than two times per call,
 * whatever the rank count ("Echo: Error-Compensated 4-Bit Tensor-Parallel
 * Communication", Abstract).  Before each all-reduce the input is shifted by
 * a correction formed from a fast-decaying and a slow-decaying average of
 * earlier injected error; afterwards both averages absorb the error the call
 * injected ("Tensor-parallel traffic drops to 4 bits", Interpretation).
 *
 * One rank's view.  P ranks each hold an n-element bf16 tensor.  Chunk j is
 * the element range [j*n/P, (j+1)*n/P); rank j owns chunk j.  A call is:
 *   entry   -- x' = f32(x) - (W_FAST*m_fast + W_SLOW*m_slow); 4-bit group
 *              quantize x'; chunk j of the message goes to rank j;
 *   reduce  -- rank p dequantizes the P stage-1 messages of chunk p, sums
 *              them in binary32 in rank order 0..P-1 and requantizes the sum;
 *   exit    -- every rank dequantizes the P stage-2 chunks to bf16;
 *   update  -- r = d1 - x' (+ e2 = f32(y) - S on the own chunk) refreshes
 *              m_fast <- B_FAST*m_fast + A_FAST*r and
 *              m_slow <- B_SLOW*m_slow + A_SLOW*r.
 * There is no transport in this library: the P-1 incoming stage-1 shards and
 * the P-1 gathered stage-2 chunks are device buffers the caller provides.
 *
 * Formats (all device memory, little-endian):
 *   bf16 tensor   uint16_t[n], bfloat16 bit patterns.
 *   int4 codes    uint8_t[n/2]; byte k holds element 2k in bits 0..3 and
 *                 element 2k+1 in bits 4..7, two's complement; the encoder
 *                 emits codes in [-7, 7] only (a 0x8 field decodes as -8).
 *   int8 codes    uint8_t[n]: one two's-complement byte per element, codes in
 *                 [-127, 127] (0x80 decodes as -128); used when a call is
 *                 promoted to 8 bits.  The pages promote the first half of the
 *                 layers to 8 bits in serving ("Tensor-parallel traffic drops
 *                 to 4 bits", Perspective).  The width is st->bits for calls
 *                 that take a state (set it before each call; the averages do
 *                 not depend on it) and the `bits` argument otherwise; every
 *                 "codes" array below then has n/2 (4-bit) or n (8-bit)
 *                 bytes, and QMAX is 7 or 127.
 *   scales        float[n/128]; group g covers elements [128g, 128g+128);
 *                 element value = code * scale.  Scale 0 means all codes 0.
 *   averages      float[n] each (m_fast, m_slow), caller-owned.
 *
 * Conventions for every call:
 *   - Returns ECHO_SUCCESS (0) or a negative ECHO_ERR_* code; nothing is
 *     launched when an argument check fails.  No exception crosses the ABI.
 *   - Asynchronous: work is enqueued on `stream` (a hipStream_t; NULL is the
 *     null stream).  Calls that touch the same buffers must be ordered by
 *     the caller (same stream, or events).
 *   - The library allocates no device memory and keeps no global mutable
 *     state; every buffer is owned by the caller and must stay valid until
 *     the enqueued work completes.
 *   - Alignment: bf16 tensors, codes, averages and e2 arrays must be 16-byte
 *     aligned; scale arrays 4-byte aligned (ECHO_ERR_ALIGNMENT).
 *   - Shapes: 0 <= n <= ECHO_MAX_ELEMENTS and n % (P*128) == 0
 *     (ECHO_ERR_SHAPE); 1 <= P <= ECHO_MAX_RANKS and 0 <= rank < P
 *     (ECHO_ERR_RANKS).  A tensor whose length is not a whole number of
 *     groups per chunk is padded by the caller (a zero tail quantizes to
 *     zero codes and leaves its averages at zero).
 *   - Empty calls: n == 0 (chunk_n == 0 for the stateless calls) is a
 *     no-op.  The scalar arguments (P, rank, bits) are still checked, the
 *     pointer arguments are not looked at (NULL is fine), nothing is
 *     enqueued and ECHO_SUCCESS is returned.
 *   - Aliasing: outputs may not overlap each other or any input
 *     (ECHO_ERR_ALIAS), except that y may equal x exactly (in place) where
 *     a call takes both; with the phased calls below, run the exit pass
 *     after the entry pass when y == x.
 *   - Inputs must be finite; results for inf/NaN inputs, or for sums that
 *     overflow binary32, are unspecified.
 *   - Results are deterministic and bit-identical between the fused and the
 *     unfused sequences.
 */
#ifndef ECHO_H
#define ECHO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- named parameters (readings of what the pages leave open) ------------ */
#define ECHO_GROUP 128          /* elements per scale */
#define ECHO_QMAX 7             /* symmetric int4 range [-7, 7] */
#define ECHO_QMAX8 127          /* 8-bit codes (a promoted call): [-127, 127] */
#define ECHO_W_FAST 0.5f        /* correction = W_FAST*m_fast + W_SLOW*m_slow */
#define ECHO_W_SLOW 0.5f
#define ECHO_BETA_FAST 0.5f     /* m_fast <- BETA_FAST*m_fast + ALPHA_FAST*r */
#define ECHO_ALPHA_FAST 0.5f
#define ECHO_BETA_SLOW 0.875f   /* m_slow <- BETA_SLOW*m_slow + ALPHA_SLOW*r */
#define ECHO_ALPHA_SLOW 0.125f
#define ECHO_MAX_RANKS 16
#define ECHO_MAX_ELEMENTS (INT64_C(1) << 37)
#define ECHO_ABI_VERSION 3

/* ---- status codes --------------------------------------------------------- */
#define ECHO_SUCCESS 0
#define ECHO_ERR_INVALID_ARGUMENT -1 /* a required pointer is NULL */
#define ECHO_ERR_SHAPE -2            /* n or chunk_n out of range / not a multiple */
#define ECHO_ERR_ALIGNMENT -3        /* a pointer misses its alignment */
#define ECHO_ERR_RANKS -4            /* P or rank out of range */
#define ECHO_ERR_HIP -5              /* the HIP runtime rejected one of the call's kernel
                                        launches (that launch's own status; an error an
                                        earlier HIP call left behind is neither reported
                                        nor cleared) */
#define ECHO_ERR_ALIAS -6            /* outputs overlap each other or an input */
#define ECHO_ERR_FORMAT -7           /* code width other than 4 or 8 bits */

typedef void* echo_stream_t; /* a hipStream_t */

/* The compensator of one call sequence (one direction of one model: the
 * averages are carried from call to call in execution order).  The struct is
 * plain data owned by the caller; the library reads it and writes only the
 * two buffers it points to. */
typedef struct echo_state {
  float* m_fast; /* device float[n], 16-byte aligned */
  float* m_slow; /* device float[n], 16-byte aligned */
  int64_t n;     /* elements of this rank's tensor */
  int32_t nranks;
  int32_t rank;
  int32_t bits;     /* code width of this call's messages: 4 (default) or 8 */
  int32_t reserved; /* 0 */
} echo_state;

typedef struct echo_config {
  int32_t abi_version, group, qmax, qmax8, max_ranks;
  float w_fast, w_slow, beta_fast, alpha_fast, beta_slow, alpha_slow;
  int64_t max_elements;
} echo_config;

/* Set up the compensator of a call sequence ("Tensor-parallel traffic drops
 * to 4 bits", Interpretation: the correction comes from a fast and a slow
 * moving average of the errors earlier calls injected; the pages give no
 * starting value, and this library starts both at zero).  Fills *st (bits = 4)
 * and enqueues zero-fills of m_fast[n] and m_slow[n] on `stream`; the buffers
 * stay caller-owned.  Validates shape, ranks, alignment and that the two
 * buffers do not overlap; nothing is enqueued when a check fails. */
int echo_state_init(echo_state* st, float* m_fast, float* m_slow, int64_t n, int32_t nranks,
                    int32_t rank, echo_stream_t stream);

/* Entry pass over all n elements ("Tensor-parallel traffic drops to 4 bits",
 * Interpretation: the correction is added to the input before each
 * all-reduce, fused into the entry pass):
 * x' = f32(x) - (W_FAST*m_fast + W_SLOW*m_slow); per 128-group amax = max|x'|,
 * s = amax/7 (IEEE division), code = clamp(rint(x'/s), -7, 7); s == 0 gives
 * codes 0.  Writes codes[n/2] and scales[n/128]; reads the averages, does not
 * write them. */
int echo_encode(const echo_state* st, const uint16_t* x, uint8_t* codes, float* scales,
                echo_stream_t stream);

/* Reduce stage for one chunk of chunk_n elements ("Echo: Error-Compensated
 * 4-Bit Tensor-Parallel Communication", Abstract: the 4-bit codes are summed
 * in a wide format and requantized once more, the last quantization a value
 * sees): shard_codes /
 * shard_scales are host arrays of nranks device pointers (shard q = rank q's
 * stage-1 message of this chunk: codes[chunk_n/2], scales[chunk_n/128]).
 * S = d_0 + d_1 + ... + d_{P-1} in binary32, in that order (d = code*scale);
 * requantize S like the entry pass -> out_codes[chunk_n/2], out_scales
 * [chunk_n/128].  Optional outputs (NULL to skip): out_y[chunk_n] =
 * bf16(code2*s2) rounded to nearest even, out_e2[chunk_n] = f32(y) - S.
 * chunk_n % 128 == 0; chunk_n == 0 is a no-op. */
int echo_reduce_shard(int32_t nranks, int64_t chunk_n, int32_t bits,
                      const uint8_t* const* shard_codes, const float* const* shard_scales,
                      uint8_t* out_codes, float* out_scales, uint16_t* out_y, float* out_e2,
                      echo_stream_t stream);

/* Exit pass over n elements ("Echo: Error-Compensated 4-Bit Tensor-Parallel
 * Communication", Abstract: the all-reduce moves 4-bit codes; the receiver
 * turns them back into the 16-bit tensor): y[n] = bf16(code*scale), rounded
 * to nearest even, from codes[n/2] (n bytes at 8 bits) and scales[n/128].
 * Reads the codes and scales, writes only y; y may not overlap them
 * (ECHO_ERR_ALIAS).  n % 128 == 0; n == 0 is a no-op. */
int echo_decode(int64_t n, int32_t bits, const uint8_t* codes, const float* scales, uint16_t* y,
                echo_stream_t stream);

/* Update ("Tensor-parallel traffic drops to 4 bits", Interpretation: the
 * averages are refreshed from the output residual): with the pre-call
 * averages, recompute x' as the entry
 * pass does, d1 = code1*scale1, r = d1 - x' plus e2_own[i - rank*n/P] on the
 * own chunk; then m_fast <- B_FAST*m_fast + A_FAST*r, m_slow <- B_SLOW*m_slow +
 * A_SLOW*r in place.  codes1/scales1 are this rank's entry-pass output for
 * all n elements; e2_own is float[n/P]. */
int echo_update(const echo_state* st, const uint16_t* x, const uint8_t* codes1,
                const float* scales1, const float* e2_own, echo_stream_t stream);

/* ---- the fused call, and its three phases --------------------------------- */
/* One all-reduce call of rank `st->rank` with the correction fused into the
 * entry pass and the averages refreshed from the call's own residual
 * ("Tensor-parallel traffic drops to 4 bits", Interpretation), over the two-
 * quantization structure of "Echo: Error-Compensated 4-Bit Tensor-Parallel
 * Communication", Abstract (each value is quantized once on entry and once
 * after the wide sum, whatever P is).
 * The phases split the fused call where a multi-GPU transport would sit:
 * entry -> (all-to-all of stage-1 chunks) -> reduce -> (all-gather of
 * stage-2 chunks) -> exit.  echo_call runs all three on one stream and is
 * bit-identical to echo_encode + echo_reduce_shard + echo_decode +
 * echo_update. */

/* Entry phase over every chunk except the own one ("Tensor-parallel traffic
 * drops to 4 bits", Interpretation: the correction is applied inside the
 * entry pass; "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication",
 * Abstract: the first of a value's two quantizations): correction, stage-1
 * quantization into send_codes[n/2] / send_scales[n/128] (the own chunk's
 * bytes are left untouched), and the averages' update with r = d1 - x' on
 * those elements. */
int echo_call_entry(const echo_state* st, const uint16_t* x, uint8_t* send_codes,
                    float* send_scales, echo_stream_t stream);

/* The entry phase restricted to chunks [chunk_begin, chunk_end), the own
 * chunk still skipped ("Tensor-parallel traffic drops to 4 bits",
 * Interpretation, as echo_call_entry; the split by chunk is this library's,
 * so that sending can overlap encoding): for each such chunk j exactly what
 * echo_call_entry does to chunk j (its part of send_codes / send_scales and
 * of the averages), nothing else.  Ranges that cover [0, P) once, in any order and
 * on any streams the caller orders before the reduce phase, together equal
 * one echo_call_entry; a transport can send chunk j to rank j while later
 * chunks are still being encoded.  Buffers are the full-size ones of
 * echo_call_entry.  0 <= chunk_begin <= chunk_end <= P, else ECHO_ERR_RANKS;
 * an empty range (or the own chunk alone) enqueues nothing. */
int echo_call_entry_range(const echo_state* st, const uint16_t* x, int32_t chunk_begin,
                          int32_t chunk_end, uint8_t* send_codes, float* send_scales,
                          echo_stream_t stream);

/* Reduce phase over the own chunk ("Echo: Error-Compensated 4-Bit Tensor-
 * Parallel Communication", Abstract: the codes are summed in a wide format
 * and requantized, a value's second and last quantization; "Tensor-parallel
 * traffic drops to 4 bits", Interpretation: forming the sum exposes the error
 * the call injected, which refreshes the averages): correction and stage-1
 * quantization of the own elements (kept in registers, never stored), the
 * rank-order sum with
 * the P-1 incoming shards recv_codes[q] / recv_scales[q] (host arrays of
 * nranks device pointers; slot `rank` is ignored and may be NULL; each shard
 * covers chunk `rank`: codes[n/P/2], scales[n/P/128]), requantization into
 * own_codes2[n/P/2] / own_scales2[n/P/128], y on the own chunk (y points at
 * the full n-element output), and the averages' update with r = e1 + e2. */
int echo_call_reduce(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
                     const float* const* recv_scales, uint8_t* own_codes2, float* own_scales2,
                     uint16_t* y, echo_stream_t stream);

/* Exit phase over every chunk except the own one ("Echo: Error-Compensated
 * 4-Bit Tensor-Parallel Communication", Abstract: the gathered 4-bit result
 * is decoded to the 16-bit output): y on chunk j from the
 * gathered stage-2 chunk gath_codes[j] / gath_scales[j] (host arrays of
 * nranks device pointers; slot `rank` ignored; each codes[n/P/2],
 * scales[n/P/128]). */
int echo_call_exit(const echo_state* st, const uint8_t* const* gath_codes,
                   const float* const* gath_scales, uint16_t* y, echo_stream_t stream);

/* All three phases, in order, on one stream (the fused call of
 * "Tensor-parallel traffic drops to 4 bits", Interpretation, with the
 * averages' update inside the entry and reduce kernels). */
int echo_call(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
              const float* const* recv_scales, const uint8_t* const* gath_codes,
              const float* const* gath_scales, uint8_t* send_codes, float* send_scales,
              uint8_t* own_codes2, float* own_scales2, uint16_t* y, echo_stream_t stream);

/* The uncompensated 4-bit all-reduce compute path: the same three phases with
 * x' = f32(x) and no averages (the pages' uncompensated 4-bit control,
 * "Tensor-parallel traffic drops to 4 bits", Interpretation).  Arguments as
 * echo_call, with the rank geometry given directly.  Also the control of the
 * deep-chain experiment, and the critical path the compensation is measured
 * against. */
int echo_call_plain(int32_t nranks, int32_t rank, int64_t n, int32_t bits, const uint16_t* x,
                    const uint8_t* const* recv_codes, const float* const* recv_scales,
                    const uint8_t* const* gath_codes, const float* const* gath_scales,
                    uint8_t* send_codes, float* send_scales, uint8_t* own_codes2,
                    float* own_scales2, uint16_t* y, echo_stream_t stream);

/* Deferred update.  In the pages' schedule the averages' update overlaps the
 * following matrix multiplication, off the critical path ("Tensor-parallel traffic drops to 4
 * bits", Interpretation).  With this API that schedule is: echo_encode (the
 * whole tensor, averages read-only; chunk p of its output is the own stage-1
 * message) -> transport -> echo_reduce_shard (slot p = that own message, out_e2
 * kept) -> transport -> echo_call_exit on the critical stream; then echo_update
 * (codes1 = the echo_encode output, e2_own) on a side stream, which must finish
 * before the next call's entry pass reads the averages.  Bit-identical to
 * echo_call. */

/* The same schedule with the next call's correction kept as one array, so
 * that the critical-path entry pass reads one binary32 value per element
 * instead of both averages ("Tensor-parallel traffic drops to 4 bits",
 * Interpretation: the correction is fused into the entry pass and the update
 * runs off the critical path):
 *   echo_correction once (after echo_state_init, or whenever the averages
 *   were changed by any other call) -> per call: echo_encode_corr ->
 *   transport -> echo_reduce_shard -> transport -> echo_call_exit on the
 *   critical stream; echo_update_corr on a side stream, which must finish
 *   before the next echo_encode_corr.
 * Bit-identical to echo_call: corr holds exactly the binary32 values
 * (W_FAST*m_fast) + (W_SLOW*m_slow) the fused entry pass forms. */

/* corr[n] = (W_FAST*m_fast) + (W_SLOW*m_slow) from the current averages
 * ("Tensor-parallel traffic drops to 4 bits", Interpretation: the correction
 * built from the two averages).  corr: device float[n], 16-byte aligned,
 * caller-owned, may not overlap the averages. */
int echo_correction(const echo_state* st, float* corr, echo_stream_t stream);

/* Entry pass over all n elements from the correction array ("Tensor-parallel
 * traffic drops to 4 bits", Interpretation): x' = f32(x) - corr, then the
 * stage-1 quantization of echo_encode into codes / scales.  Reads x and
 * corr only (the averages are not touched); equals echo_encode when corr
 * came from the same averages. */
int echo_encode_corr(const echo_state* st, const uint16_t* x, const float* corr, uint8_t* codes,
                     float* scales, echo_stream_t stream);

/* echo_update ("Tensor-parallel traffic drops to 4 bits", Interpretation:
 * the averages absorb the residual off the critical path), then the next
 * call's correction from the refreshed averages into corr[n].  Arguments as
 * echo_update; corr may not overlap any of them. */
int echo_update_corr(const echo_state* st, const uint16_t* x, const uint8_t* codes1,
                     const float* scales1, const float* e2_own, float* corr,
                     echo_stream_t stream);

/* ---- reduce-scatter only (sequence parallelism) ------------------------------
 * The pages propose the reduce-scatter of sequence parallelism as a further
 * use ("Tensor-parallel traffic drops to 4 bits", Perspective).  Reading:
 * the entry pass is the all-reduce's; rank p sums the P stage-1 shards of its
 * chunk in binary32, rank order, and outputs the sum as bf16 (round to nearest
 * even) -- there is no second quantization, each value is quantized once; the
 * residual on the own chunk is e = f32(y) - S in place of e2. */

/* Rank-order sum of P stage-1 shards output as bf16: out_y[chunk_n] =
 * bf16(S); out_e2 (nullable) = f32(out_y) - S.  Unfused. */
int echo_reduce_shard_sum(int32_t nranks, int64_t chunk_n, int32_t bits,
                          const uint8_t* const* shard_codes, const float* const* shard_scales,
                          uint16_t* out_y, float* out_e2, echo_stream_t stream);

/* Reduce phase of the reduce-scatter ("Tensor-parallel traffic drops to 4
 * bits", Perspective, for the variant; Interpretation, for the correction and
 * the refresh of the averages): the own chunk's correction and stage-1
 * quantization in registers, the rank-order sum with the P-1 incoming shards
 * (as echo_call_reduce), y_own[n/P] = bf16(S), and the averages' update on
 * the own chunk with r = e1 + (f32(y_own) - S).  y_own may not overlap x. */
int echo_rs_reduce(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
                   const float* const* recv_scales, uint16_t* y_own, echo_stream_t stream);

/* The fused reduce-scatter ("Tensor-parallel traffic drops to 4 bits",
 * Perspective): echo_call_entry then echo_rs_reduce on one stream.
 * Bit-identical to echo_encode + echo_reduce_shard_sum (own slot = own
 * stage-1 chunk, out_e2 kept) + echo_update. */
int echo_rs_call(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
                 const float* const* recv_scales, uint8_t* send_codes, float* send_scales,
                 uint16_t* y_own, echo_stream_t stream);

/* ---- measurement ------------------------------------------------------------
 * A plain streaming copy with the launch shape and cache hints of the path's
 * kernels (one 16-byte vector per lane, a grid covering the range,
 * non-temporal loads and stores): the practical HBM ceiling the kernels are
 * measured against.  Not part of the method.  bytes % 16 == 0 and both
 * pointers 16-byte aligned (ECHO_ERR_SHAPE / ECHO_ERR_ALIGNMENT); the ranges
 * may not overlap (ECHO_ERR_ALIAS); bytes == 0 is a no-op. */
int echo_stream_copy(const void* src, void* dst, int64_t bytes, echo_stream_t stream);

/* ---- misc ------------------------------------------------------------------ */
int echo_get_config(echo_config* out);      /* the named parameters above */
const char* echo_status_string(int status); /* static string, never NULL */
int echo_version(void);                     /* ECHO_ABI_VERSION */

#ifdef __cplusplus
}
#endif
#endif
