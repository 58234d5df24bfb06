/*
 * echo_oracle.h -- plain CPU oracle for the Echo rank pipeline.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path includes, links
 * or calls this code; only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark do.  It shares no source with the HIP library:
 * every constant below is restated here from the readings of the pages,
 * and a test checks that the library reports the same values.
 *
 * Source: "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication for
 * LLM Training and Inference" (arXiv 2610.14277v1): its Abstract, and the
 * summary page "Tensor-parallel traffic drops to 4 bits", section
 * Interpretation.
 *
 * Arithmetic: IEEE binary32, round-to-nearest-even, one rounding per
 * operation, no contraction (built with -ffp-contract=off), denormals kept.
 */
#ifndef ECHO_ORACLE_H
#define ECHO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Readings of what the pages leave open (each is a choice, not a quote). */
#define ORC_GROUP 128        /* elements sharing one scale */
#define ORC_QMAX 7           /* symmetric int4 codes in [-7, 7] */
#define ORC_W_FAST 0.5f      /* weight of the fast average in the correction */
#define ORC_W_SLOW 0.5f      /* weight of the slow average in the correction */
#define ORC_BETA_FAST 0.5f   /* fast average: m <- 0.5 m + 0.5 r */
#define ORC_ALPHA_FAST 0.5f
#define ORC_BETA_SLOW 0.875f /* slow average: m <- 0.875 m + 0.125 r */
#define ORC_ALPHA_SLOW 0.125f
#define ORC_MAX_RANKS 16
#define ORC_QMAX8 127        /* 8-bit promotion of a call: codes in [-127, 127] */

/* Number of values the quantizer has processed on the calling thread, per
 * stage (1 = entry, 2 = reduce).  Used by the pin on the number of
 * quantizations per value (single-thread calls). */
void orc_counters_reset(void);
long long orc_counter(int stage);

/* bf16 <-> f32.  The narrowing conversion rounds to nearest, ties to even. */
uint16_t orc_f32_to_bf16(float f);
float orc_bf16_to_f32(uint16_t h);

/* Quantize one group of `len` values (step "group quantize"):
 * amax = max |v|, s = amax / QMAX, q = clamp(rint(v / s), -QMAX, QMAX);
 * s == 0 (all-zero group, or amax / QMAX underflowing) gives codes 0. */
void orc_quantize_group(const float* v, int len, int8_t* q, float* scale, int stage);
/* The same with an explicit code range (7 for 4-bit, 127 for 8-bit codes). */
void orc_quantize_group_q(const float* v, int len, int qmax, int8_t* q, float* scale,
                          int stage);

/* Nibble packing: byte k holds element 2k in its low nibble and element
 * 2k+1 in its high nibble, both two's complement.  n must be even. */
void orc_pack(const int8_t* q, int64_t n, uint8_t* codes);
void orc_unpack(const uint8_t* codes, int64_t n, int8_t* q);

/* Code width `bits` (4 or 8) of every message below: 4 -> packed nibbles as
 * above, codes in [-7, 7]; 8 -> one two's-complement byte per element, codes
 * in [-127, 127] (the pages promote the first half of the layers to 8 bits in
 * serving, "Tensor-parallel traffic drops to 4 bits", Perspective). */
void orc_pack_codes(const int8_t* q, int64_t n, uint8_t* codes, int bits);
void orc_unpack_codes(const uint8_t* codes, int64_t n, int8_t* q, int bits);

/* Fold r into both averages: m_f <- B_F m_f + A_F r, m_s <- B_S m_s + A_S r. */
void orc_ema_refresh(int64_t n, float* m_fast, float* m_slow, const float* r);

/* Entry pass over n elements (n % 128 == 0): x' = f32(x) - (W_F m_f + W_S m_s)
 * (or x' = f32(x) when comp == 0), then group-quantize x'.  The state is
 * read, not written.  xp_out (nullable) receives x'. */
void orc_encode(int64_t n, const uint16_t* x, const float* m_fast, const float* m_slow,
                uint8_t* codes, float* scales, float* xp_out, int comp, int bits);

/* Reduce one chunk of chunk_n elements from P shards: S = d_0 + ... + d_{P-1}
 * in rank order, requantize S, y = bf16(code2 * s2), e2 = f32(y) - S.
 * y and e2 are nullable. */
void orc_reduce_chunk(int nranks, int64_t chunk_n, const uint8_t* const* shard_codes,
                      const float* const* shard_scales, uint8_t* codes2, float* scales2,
                      uint16_t* y, float* e2, int bits);

/* Exit pass: y = bf16(code * scale). */
void orc_decode(int64_t n, const uint8_t* codes, const float* scales, uint16_t* y, int bits);

/* Update: recompute x' from the pre-call state, d1 from codes1/scales1,
 * r = d1 - x' (+ e2_own on the chunk [rank*n/P, (rank+1)*n/P)), refresh both
 * averages in place.  r_out (nullable) receives r. */
void orc_update(int64_t n, int nranks, int rank, const uint16_t* x, float* m_fast,
                float* m_slow, const uint8_t* codes1, const float* scales1,
                const float* e2_own, float* r_out, int bits);

/* orc_update over the element range [i0, i1) only, with the own chunk given
 * as [own0, own1) (absolute indices into every array; e2_own is indexed
 * from own0).  orc_update is this over [0, n). */
void orc_update_span(int64_t i0, int64_t i1, int64_t own0, int64_t own1, const uint16_t* x,
                     float* m_fast, float* m_slow, const uint8_t* codes1, const float* scales1,
                     const float* e2_own, float* r_out, int bits);

/* One call in rank mode (rank p of P): incoming shards recv_*[q] (q != p,
 * each covering chunk p) and gathered outputs gath_*[j] (j != p, each
 * covering chunk j) are inputs.  Writes send_* for every chunk except p,
 * own_codes2/own_scales2 for chunk p, y for all n, and updates the state
 * when comp != 0.  Returns 0, or -1 on bad arguments / allocation failure. */
int orc_call(int nranks, int rank, int64_t n, const uint16_t* x, float* m_fast,
             float* m_slow, const uint8_t* const* recv_codes, const float* const* recv_scales,
             const uint8_t* const* gath_codes, const float* const* gath_scales,
             uint8_t* send_codes, float* send_scales, uint8_t* own_codes2, float* own_scales2,
             uint16_t* y, int comp, int bits);

/* One call with all P ranks simulated: xs[p], m_fast[p], m_slow[p] per rank.
 * Writes the all-gathered codes2/scales2 and the output y (identical on
 * every rank).  Optional per-rank outputs (nullable arrays of P pointers, or
 * NULL): codes1[p]/scales1[p] (stage-1 message), xp[p] (x'), r[p] (the
 * residual folded into the averages).  Returns 0, or -1. */
int orc_simulate(int nranks, int64_t n, const uint16_t* const* xs, float* const* m_fast,
                 float* const* m_slow, uint8_t* codes2, float* scales2, uint16_t* y,
                 uint8_t* const* codes1, float* const* scales1, float* const* xp,
                 float* const* r, int comp, int bits);

/* ---- the correction kept as one array -----------------------------------------
 * The pages run the averages' update beside the next matrix multiplication,
 * off the critical path ("Tensor-parallel traffic drops to 4 bits",
 * Interpretation).  With the next call's correction kept as one array, the
 * critical-path entry pass reads it instead of both averages. */

/* corr[i] = (W_F m_fast[i]) + (W_S m_slow[i]), the correction the entry pass
 * subtracts. */
void orc_correction(int64_t n, const float* m_fast, const float* m_slow, float* corr);

/* Entry pass from a correction array: x' = f32(x) - corr, then group-quantize
 * x' (stage 1).  Equals orc_encode with the averages corr was formed from. */
void orc_encode_corr(int64_t n, const uint16_t* x, const float* corr, uint8_t* codes,
                     float* scales, int bits);

/* orc_update, then corr = the correction of the refreshed averages. */
void orc_update_corr(int64_t n, int nranks, int rank, const uint16_t* x, float* m_fast,
                     float* m_slow, const uint8_t* codes1, const float* scales1,
                     const float* e2_own, float* corr, int bits);

/* ---- reduce-scatter only (the sequence-parallel variant) -------------------
 * The pages name the reduce-scatter of sequence parallelism as a next target
 * ("Tensor-parallel traffic drops to 4 bits", Perspective).  Reading: the
 * entry pass is unchanged; the owner of chunk j sums the P stage-1 shards in
 * rank order and outputs the sum as bf16 directly (no second quantization:
 * each value is quantized once); the rounding of that output, e = f32(y) - S,
 * plays the part of e2 in the residual. */

/* S = d_0 + ... + d_{P-1}; y = bf16(S); e = f32(y) - S (e nullable). */
void orc_reduce_chunk_sum(int nranks, int64_t chunk_n, const uint8_t* const* shard_codes,
                          const float* const* shard_scales, uint16_t* y, float* e, int bits);

/* Rank mode: writes send_* for every chunk except `rank`, y_own[n/P] (the
 * reduced own chunk) and updates the state when comp != 0.  Returns 0 or -1. */
int orc_rs_call(int nranks, int rank, int64_t n, const uint16_t* x, float* m_fast,
                float* m_slow, const uint8_t* const* recv_codes, const float* const* recv_scales,
                uint8_t* send_codes, float* send_scales, uint16_t* y_own, int comp, int bits);

/* All P ranks: y[n] holds chunk j as reduced by rank j.  Optional per-rank
 * xp[p] and r[p] (nullable).  Returns 0 or -1. */
int orc_rs_simulate(int nranks, int64_t n, const uint16_t* const* xs, float* const* m_fast,
                    float* const* m_slow, uint16_t* y, float* const* xp, float* const* r,
                    int comp, int bits);

/* ---- threaded driver (echo_oracle_mt.c) --------------------------------------
 * orc_call with its steps split over `threads` host threads by disjoint
 * ranges of whole groups.  Each thread runs the step functions above on its
 * range, so every output is bit-identical to orc_call's for any thread count
 * (a thread count below 1 is taken as 1).  The quantizer counters are not
 * kept.  Returns 0, or -1 on bad arguments / allocation failure. */
int orc_call_mt(int threads, int nranks, int rank, int64_t n, const uint16_t* x, float* m_fast,
                float* m_slow, const uint8_t* const* recv_codes, const float* const* recv_scales,
                const uint8_t* const* gath_codes, const float* const* gath_scales,
                uint8_t* send_codes, float* send_scales, uint8_t* own_codes2,
                float* own_scales2, uint16_t* y, int comp, int bits);

/* orc_rs_call split the same way (bit-identical for any thread count). */
int orc_rs_call_mt(int threads, int nranks, int rank, int64_t n, const uint16_t* x,
                   float* m_fast, float* m_slow, const uint8_t* const* recv_codes,
                   const float* const* recv_scales, uint8_t* send_codes, float* send_scales,
                   uint16_t* y_own, int comp, int bits);

#ifdef __cplusplus
}
#endif
#endif
