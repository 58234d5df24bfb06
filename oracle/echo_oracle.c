/*
 * echo_oracle.c -- plain, slow, obviously-correct CPU oracle of the Echo
 * rank pipeline.
 *
 * TEST INFRASTRUCTURE ONLY: used by the tests, the smoke check and the
 * CPU-baseline leg of the benchmark, never by the product path.  It shares
 * no code with the HIP library.
 *
 * What the method computes, per the pages (arXiv 2610.14277v1).  Pages:
 * "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication" (EC),
 * "Tensor-parallel traffic drops to 4 bits" (TP), "How Echo lets big AI
 * models train faster" (HE).
 *   - the payload crosses the interconnect as 4-bit integer codes and is
 *     accumulated in a wider floating-point format (TP, Interpretation; EC,
 *     Abstract);
 *   - no value is quantized more than two times in a call, whatever the
 *     rank count (EC, Abstract; HE, "How Echo keeps errors from snowballing");
 *   - before each all-reduce the input is shifted by a correction formed
 *     from a fast- and a slow-decaying average of past injected error, and
 *     the averages then absorb the error that call injected (TP,
 *     Interpretation);
 *   - forming the sum exposes the injected error, and folding it into later
 *     calls lets earlier errors cancel out (EC, Abstract).
 * Every detail the pages leave open (group size, scale type, code range,
 * rounding, nibble order, decays, how the averages combine, the residual's
 * exact definition) follows the stated readings: see echo_oracle.h.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math (no -march flags), so each
 * float operation below is one IEEE binary32 operation rounded to nearest even.
 */
#include "echo_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* Per thread, so the threaded driver's workers never race on it; the
 * counting pins call the single-thread functions from one thread. */
static _Thread_local long long g_stage_values[3];

void orc_counters_reset(void) { memset(g_stage_values, 0, sizeof(g_stage_values)); }

long long orc_counter(int stage) {
  if (stage < 0 || stage > 2) return -1;
  return g_stage_values[stage];
}

/* ---- bf16 --------------------------------------------------------------- */

/* Round a binary32 value to the nearest bfloat16 (8 significant bits), ties
 * to the candidate whose last kept bit is 0.  The kept part is the top 16
 * bits (truncation toward zero in magnitude); the dropped 16 bits decide. */
uint16_t orc_f32_to_bf16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  if ((u & 0x7F800000u) == 0x7F800000u) {
    if (u & 0x007FFFFFu) return (uint16_t)((u >> 16) | 0x0040u); /* NaN stays NaN */
    return (uint16_t)(u >> 16);                                   /* +-inf */
  }
  uint32_t kept = u >> 16;
  uint32_t dropped = u & 0xFFFFu;
  int round_up;
  if (dropped > 0x8000u) {
    round_up = 1;
  } else if (dropped < 0x8000u) {
    round_up = 0;
  } else {
    round_up = (int)(kept & 1u); /* exact tie: go to the even neighbour */
  }
  /* Adding one to the kept magnitude bits gives the next representable
   * value away from zero (a carry into the exponent is that value too). */
  return (uint16_t)(kept + (uint32_t)round_up);
}

float orc_bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* ---- group quantizer ------------------------------------------------------ */

void orc_quantize_group_q(const float* v, int len, int qmax, int8_t* q, float* scale,
                          int stage) {
  float amax = 0.0f;
  for (int i = 0; i < len; ++i) {
    float a = fabsf(v[i]);
    if (a > amax) amax = a;
  }
  float s = amax / (float)qmax;
  if (s == 0.0f) {
    for (int i = 0; i < len; ++i) q[i] = 0;
  } else {
    for (int i = 0; i < len; ++i) {
      float t = rintf(v[i] / s);
      if (t > (float)qmax) t = (float)qmax;
      if (t < -(float)qmax) t = -(float)qmax;
      q[i] = (int8_t)t;
    }
  }
  *scale = s;
  if (stage >= 0 && stage <= 2) g_stage_values[stage] += len;
}

void orc_quantize_group(const float* v, int len, int8_t* q, float* scale, int stage) {
  orc_quantize_group_q(v, len, ORC_QMAX, q, scale, stage);
}

/* ---- nibbles ---------------------------------------------------------------- */

void orc_pack(const int8_t* q, int64_t n, uint8_t* codes) {
  for (int64_t k = 0; k < n / 2; ++k) {
    unsigned lo = (unsigned)q[2 * k] & 0xFu;
    unsigned hi = (unsigned)q[2 * k + 1] & 0xFu;
    codes[k] = (uint8_t)(lo | (hi << 4));
  }
}

static int8_t nibble_value(unsigned nib) {
  /* two's complement of a 4-bit field: 0..7 -> 0..7, 8..15 -> -8..-1 */
  return (int8_t)(nib < 8u ? (int)nib : (int)nib - 16);
}

void orc_unpack(const uint8_t* codes, int64_t n, int8_t* q) {
  for (int64_t k = 0; k < n / 2; ++k) {
    q[2 * k] = nibble_value(codes[k] & 0xFu);
    q[2 * k + 1] = nibble_value(codes[k] >> 4);
  }
}

/* ---- code widths ------------------------------------------------------------
 * bits == 4: packed nibbles, codes in [-7, 7]; bits == 8: one two's-complement
 * byte per element, codes in [-127, 127] (the 8-bit promotion of a call). */

static int qmax_of(int bits) { return bits == 8 ? ORC_QMAX8 : ORC_QMAX; }

static int64_t code_bytes(int64_t n, int bits) { return bits == 8 ? n : n / 2; }

static int code_at(const uint8_t* codes, int64_t i, int bits) {
  if (bits == 8) return (int)(int8_t)codes[i];
  unsigned byte = codes[i / 2];
  unsigned nib = (i % 2 == 0) ? (byte & 0xFu) : (byte >> 4);
  return nibble_value(nib);
}

void orc_pack_codes(const int8_t* q, int64_t n, uint8_t* codes, int bits) {
  if (bits == 8) {
    for (int64_t i = 0; i < n; ++i) codes[i] = (uint8_t)q[i];
  } else {
    orc_pack(q, n, codes);
  }
}

void orc_unpack_codes(const uint8_t* codes, int64_t n, int8_t* q, int bits) {
  for (int64_t i = 0; i < n; ++i) q[i] = (int8_t)code_at(codes, i, bits);
}

static float dequant(const uint8_t* codes, const float* scales, int64_t i, int bits) {
  return (float)code_at(codes, i, bits) * scales[i / ORC_GROUP];
}

/* ---- compensator ------------------------------------------------------------ */

/* the correction of one element: the weighted sum of its two averages */
static float correction_of(float mf, float ms) { return (ORC_W_FAST * mf) + (ORC_W_SLOW * ms); }

static float corrected_input(uint16_t x, float mf, float ms, int comp) {
  float xf = orc_bf16_to_f32(x);
  if (!comp) return xf;
  float corr = correction_of(mf, ms);
  return xf - corr;
}

void orc_ema_refresh(int64_t n, float* m_fast, float* m_slow, const float* r) {
  for (int64_t i = 0; i < n; ++i) {
    m_fast[i] = (ORC_BETA_FAST * m_fast[i]) + (ORC_ALPHA_FAST * r[i]);
    m_slow[i] = (ORC_BETA_SLOW * m_slow[i]) + (ORC_ALPHA_SLOW * r[i]);
  }
}

/* ---- pipeline steps ----------------------------------------------------------- */

void orc_encode(int64_t n, const uint16_t* x, const float* m_fast, const float* m_slow,
                uint8_t* codes, float* scales, float* xp_out, int comp, int bits) {
  float v[ORC_GROUP];
  int8_t q[ORC_GROUP];
  for (int64_t g = 0; g < n / ORC_GROUP; ++g) {
    int64_t base = g * ORC_GROUP;
    for (int i = 0; i < ORC_GROUP; ++i) {
      int64_t e = base + i;
      v[i] = corrected_input(x[e], comp ? m_fast[e] : 0.0f, comp ? m_slow[e] : 0.0f, comp);
      if (xp_out) xp_out[e] = v[i];
    }
    orc_quantize_group_q(v, ORC_GROUP, qmax_of(bits), q, &scales[g], 1);
    orc_pack_codes(q, ORC_GROUP, codes + code_bytes(base, bits), bits);
  }
}

void orc_reduce_chunk(int nranks, int64_t chunk_n, const uint8_t* const* shard_codes,
                      const float* const* shard_scales, uint8_t* codes2, float* scales2,
                      uint16_t* y, float* e2, int bits) {
  float S[ORC_GROUP];
  int8_t q[ORC_GROUP];
  for (int64_t g = 0; g < chunk_n / ORC_GROUP; ++g) {
    int64_t base = g * ORC_GROUP;
    for (int i = 0; i < ORC_GROUP; ++i) {
      int64_t e = base + i;
      float acc = dequant(shard_codes[0], shard_scales[0], e, bits);
      for (int r = 1; r < nranks; ++r) acc = acc + dequant(shard_codes[r], shard_scales[r], e, bits);
      S[i] = acc;
    }
    orc_quantize_group_q(S, ORC_GROUP, qmax_of(bits), q, &scales2[g], 2);
    orc_pack_codes(q, ORC_GROUP, codes2 + code_bytes(base, bits), bits);
    for (int i = 0; i < ORC_GROUP; ++i) {
      uint16_t yi = orc_f32_to_bf16((float)q[i] * scales2[g]);
      if (y) y[base + i] = yi;
      if (e2) e2[base + i] = orc_bf16_to_f32(yi) - S[i];
    }
  }
}

void orc_decode(int64_t n, const uint8_t* codes, const float* scales, uint16_t* y, int bits) {
  for (int64_t i = 0; i < n; ++i) y[i] = orc_f32_to_bf16(dequant(codes, scales, i, bits));
}

void orc_update(int64_t n, int nranks, int rank, const uint16_t* x, float* m_fast,
                float* m_slow, const uint8_t* codes1, const float* scales1,
                const float* e2_own, float* r_out, int bits) {
  int64_t chunk = n / nranks;
  int64_t own0 = (int64_t)rank * chunk, own1 = own0 + chunk;
  orc_update_span(0, n, own0, own1, x, m_fast, m_slow, codes1, scales1, e2_own, r_out, bits);
}

void orc_update_span(int64_t i0, int64_t i1, int64_t own0, int64_t own1, const uint16_t* x,
                     float* m_fast, float* m_slow, const uint8_t* codes1, const float* scales1,
                     const float* e2_own, float* r_out, int bits) {
  for (int64_t i = i0; i < i1; ++i) {
    float xp = corrected_input(x[i], m_fast[i], m_slow[i], 1);
    float e1 = dequant(codes1, scales1, i, bits) - xp;
    float r = e1;
    if (i >= own0 && i < own1) r = e1 + e2_own[i - own0];
    if (r_out) r_out[i] = r;
    m_fast[i] = (ORC_BETA_FAST * m_fast[i]) + (ORC_ALPHA_FAST * r);
    m_slow[i] = (ORC_BETA_SLOW * m_slow[i]) + (ORC_ALPHA_SLOW * r);
  }
}

static int bits_ok(int bits) { return bits == 4 || bits == 8; }

static int shape_ok(int nranks, int64_t n) {
  if (nranks < 1 || nranks > ORC_MAX_RANKS) return 0;
  if (n <= 0 || n % ((int64_t)nranks * ORC_GROUP) != 0) return 0;
  return 1;
}

int orc_call(int nranks, int rank, int64_t n, const uint16_t* x, float* m_fast,
             float* m_slow, const uint8_t* const* recv_codes, const float* const* recv_scales,
             const uint8_t* const* gath_codes, const float* const* gath_scales,
             uint8_t* send_codes, float* send_scales, uint8_t* own_codes2, float* own_scales2,
             uint16_t* y, int comp, int bits) {
  if (!shape_ok(nranks, n) || rank < 0 || rank >= nranks || !bits_ok(bits)) return -1;
  int64_t C = n / nranks;
  const int64_t cb = code_bytes(C, bits); /* code bytes of one chunk */
  uint8_t* codes1 = malloc((size_t)code_bytes(n, bits));
  float* scales1 = malloc((size_t)(n / ORC_GROUP) * sizeof(float));
  float* e2 = malloc((size_t)C * sizeof(float));
  if (!codes1 || !scales1 || !e2) {
    free(codes1); free(scales1); free(e2);
    return -1;
  }
  /* entry pass over the whole tensor with the pre-call state */
  orc_encode(n, x, m_fast, m_slow, codes1, scales1, NULL, comp, bits);
  /* the stage-1 message of every chunk but our own is what we send */
  for (int j = 0; j < nranks; ++j) {
    if (j == rank) continue;
    memcpy(send_codes + j * cb, codes1 + j * cb, (size_t)cb);
    memcpy(send_scales + j * C / ORC_GROUP, scales1 + j * C / ORC_GROUP,
           (size_t)(C / ORC_GROUP) * sizeof(float));
  }
  /* reduce our chunk: slot `rank` is our own stage-1 message */
  const uint8_t* sc[ORC_MAX_RANKS];
  const float* ss[ORC_MAX_RANKS];
  for (int q = 0; q < nranks; ++q) {
    sc[q] = (q == rank) ? codes1 + rank * cb : recv_codes[q];
    ss[q] = (q == rank) ? scales1 + rank * C / ORC_GROUP : recv_scales[q];
  }
  orc_reduce_chunk(nranks, C, sc, ss, own_codes2, own_scales2, y + rank * C, e2, bits);
  /* exit pass over the gathered chunks */
  for (int j = 0; j < nranks; ++j) {
    if (j == rank) continue;
    orc_decode(C, gath_codes[j], gath_scales[j], y + j * C, bits);
  }
  if (comp) orc_update(n, nranks, rank, x, m_fast, m_slow, codes1, scales1, e2, NULL, bits);
  free(codes1); free(scales1); free(e2);
  return 0;
}

int orc_simulate(int nranks, int64_t n, const uint16_t* const* xs, float* const* m_fast,
                 float* const* m_slow, uint8_t* codes2, float* scales2, uint16_t* y,
                 uint8_t* const* codes1_out, float* const* scales1_out, float* const* xp_out,
                 float* const* r_out, int comp, int bits) {
  if (!shape_ok(nranks, n) || !bits_ok(bits)) return -1;
  int64_t C = n / nranks;
  const int64_t cb = code_bytes(C, bits);
  uint8_t* codes1[ORC_MAX_RANKS] = {0};
  float* scales1[ORC_MAX_RANKS] = {0};
  float* e2 = malloc((size_t)n * sizeof(float));
  int ok = e2 != NULL;
  for (int p = 0; p < nranks && ok; ++p) {
    codes1[p] = malloc((size_t)code_bytes(n, bits));
    scales1[p] = malloc((size_t)(n / ORC_GROUP) * sizeof(float));
    ok = codes1[p] && scales1[p];
  }
  if (ok) {
    /* every rank's entry pass */
    for (int p = 0; p < nranks; ++p)
      orc_encode(n, xs[p], comp ? m_fast[p] : NULL, comp ? m_slow[p] : NULL, codes1[p],
                 scales1[p], xp_out ? xp_out[p] : NULL, comp, bits);
    /* rank j reduces chunk j from everyone's stage-1 message of that chunk */
    for (int j = 0; j < nranks; ++j) {
      const uint8_t* sc[ORC_MAX_RANKS];
      const float* ss[ORC_MAX_RANKS];
      for (int q = 0; q < nranks; ++q) {
        sc[q] = codes1[q] + j * cb;
        ss[q] = scales1[q] + j * C / ORC_GROUP;
      }
      orc_reduce_chunk(nranks, C, sc, ss, codes2 + j * cb, scales2 + j * C / ORC_GROUP,
                       NULL, e2 + j * C, bits);
    }
    /* every rank decodes the same gathered message */
    orc_decode(n, codes2, scales2, y, bits);
    if (comp)
      for (int p = 0; p < nranks; ++p)
        orc_update(n, nranks, p, xs[p], m_fast[p], m_slow[p], codes1[p], scales1[p],
                   e2 + p * C, r_out ? r_out[p] : NULL, bits);
    for (int p = 0; p < nranks; ++p) {
      if (codes1_out && codes1_out[p]) memcpy(codes1_out[p], codes1[p], (size_t)code_bytes(n, bits));
      if (scales1_out && scales1_out[p])
        memcpy(scales1_out[p], scales1[p], (size_t)(n / ORC_GROUP) * sizeof(float));
    }
  }
  for (int p = 0; p < nranks; ++p) {
    free(codes1[p]);
    free(scales1[p]);
  }
  free(e2);
  return ok ? 0 : -1;
}

/* ---- the correction kept as one array --------------------------------------------
 * In the pages' schedule the averages' update runs beside the next matrix
 * multiplication, off the critical path ("Tensor-parallel traffic drops to 4
 * bits", Interpretation).  Keeping the next call's correction as one array,
 * written by that update, lets the critical-path entry pass read one value
 * per element instead of both averages; the values are the same binary32
 * numbers the entry pass would form from the averages. */

void orc_correction(int64_t n, const float* m_fast, const float* m_slow, float* corr) {
  for (int64_t i = 0; i < n; ++i) corr[i] = correction_of(m_fast[i], m_slow[i]);
}

void orc_encode_corr(int64_t n, const uint16_t* x, const float* corr, uint8_t* codes,
                     float* scales, int bits) {
  float v[ORC_GROUP];
  int8_t q[ORC_GROUP];
  for (int64_t g = 0; g < n / ORC_GROUP; ++g) {
    int64_t base = g * ORC_GROUP;
    for (int i = 0; i < ORC_GROUP; ++i) v[i] = orc_bf16_to_f32(x[base + i]) - corr[base + i];
    orc_quantize_group_q(v, ORC_GROUP, qmax_of(bits), q, &scales[g], 1);
    orc_pack_codes(q, ORC_GROUP, codes + code_bytes(base, bits), bits);
  }
}

void orc_update_corr(int64_t n, int nranks, int rank, const uint16_t* x, float* m_fast,
                     float* m_slow, const uint8_t* codes1, const float* scales1,
                     const float* e2_own, float* corr, int bits) {
  orc_update(n, nranks, rank, x, m_fast, m_slow, codes1, scales1, e2_own, NULL, bits);
  orc_correction(n, m_fast, m_slow, corr);
}

/* ---- reduce-scatter only ------------------------------------------------------ */

void orc_reduce_chunk_sum(int nranks, int64_t chunk_n, const uint8_t* const* shard_codes,
                          const float* const* shard_scales, uint16_t* y, float* e, int bits) {
  for (int64_t i = 0; i < chunk_n; ++i) {
    float acc = dequant(shard_codes[0], shard_scales[0], i, bits);
    for (int r = 1; r < nranks; ++r) acc = acc + dequant(shard_codes[r], shard_scales[r], i, bits);
    uint16_t yi = orc_f32_to_bf16(acc);
    y[i] = yi;
    if (e) e[i] = orc_bf16_to_f32(yi) - acc;
  }
}

int orc_rs_call(int nranks, int rank, int64_t n, const uint16_t* x, float* m_fast,
                float* m_slow, const uint8_t* const* recv_codes, const float* const* recv_scales,
                uint8_t* send_codes, float* send_scales, uint16_t* y_own, int comp, int bits) {
  if (!shape_ok(nranks, n) || rank < 0 || rank >= nranks || !bits_ok(bits)) return -1;
  int64_t C = n / nranks;
  const int64_t cb = code_bytes(C, bits);
  uint8_t* codes1 = malloc((size_t)code_bytes(n, bits));
  float* scales1 = malloc((size_t)(n / ORC_GROUP) * sizeof(float));
  float* e = malloc((size_t)C * sizeof(float));
  if (!codes1 || !scales1 || !e) {
    free(codes1); free(scales1); free(e);
    return -1;
  }
  orc_encode(n, x, m_fast, m_slow, codes1, scales1, NULL, comp, bits);
  for (int j = 0; j < nranks; ++j) {
    if (j == rank) continue;
    memcpy(send_codes + j * cb, codes1 + j * cb, (size_t)cb);
    memcpy(send_scales + j * C / ORC_GROUP, scales1 + j * C / ORC_GROUP,
           (size_t)(C / ORC_GROUP) * sizeof(float));
  }
  const uint8_t* sc[ORC_MAX_RANKS];
  const float* ss[ORC_MAX_RANKS];
  for (int q = 0; q < nranks; ++q) {
    sc[q] = (q == rank) ? codes1 + rank * cb : recv_codes[q];
    ss[q] = (q == rank) ? scales1 + rank * C / ORC_GROUP : recv_scales[q];
  }
  orc_reduce_chunk_sum(nranks, C, sc, ss, y_own, e, bits);
  if (comp) orc_update(n, nranks, rank, x, m_fast, m_slow, codes1, scales1, e, NULL, bits);
  free(codes1); free(scales1); free(e);
  return 0;
}

int orc_rs_simulate(int nranks, int64_t n, const uint16_t* const* xs, float* const* m_fast,
                    float* const* m_slow, uint16_t* y, float* const* xp_out,
                    float* const* r_out, int comp, int bits) {
  if (!shape_ok(nranks, n) || !bits_ok(bits)) return -1;
  int64_t C = n / nranks;
  const int64_t cb = code_bytes(C, bits);
  uint8_t* codes1[ORC_MAX_RANKS] = {0};
  float* scales1[ORC_MAX_RANKS] = {0};
  float* e = malloc((size_t)n * sizeof(float));
  int ok = e != NULL;
  for (int p = 0; p < nranks && ok; ++p) {
    codes1[p] = malloc((size_t)code_bytes(n, bits));
    scales1[p] = malloc((size_t)(n / ORC_GROUP) * sizeof(float));
    ok = codes1[p] && scales1[p];
  }
  if (ok) {
    for (int p = 0; p < nranks; ++p)
      orc_encode(n, xs[p], comp ? m_fast[p] : NULL, comp ? m_slow[p] : NULL, codes1[p],
                 scales1[p], xp_out ? xp_out[p] : NULL, comp, bits);
    for (int j = 0; j < nranks; ++j) {
      const uint8_t* sc[ORC_MAX_RANKS];
      const float* ss[ORC_MAX_RANKS];
      for (int q = 0; q < nranks; ++q) {
        sc[q] = codes1[q] + j * cb;
        ss[q] = scales1[q] + j * C / ORC_GROUP;
      }
      orc_reduce_chunk_sum(nranks, C, sc, ss, y + j * C, e + j * C, bits);
    }
    if (comp)
      for (int p = 0; p < nranks; ++p)
        orc_update(n, nranks, p, xs[p], m_fast[p], m_slow[p], codes1[p], scales1[p],
                   e + p * C, r_out ? r_out[p] : NULL, bits);
  }
  for (int p = 0; p < nranks; ++p) {
    free(codes1[p]);
    free(scales1[p]);
  }
  free(e);
  return ok ? 0 : -1;
}
