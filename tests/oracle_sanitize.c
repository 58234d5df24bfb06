/* Driver for the oracle under AddressSanitizer / UndefinedBehaviorSanitizer
 * (built by tests/test_oracle_sanitize.py with gcc, host code only).
 * Runs every oracle entry point on small seeded inputs for both code widths,
 * P = 1..16, compensation on and off, and checks that rank mode reproduces
 * the full simulation.  Exit status 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "echo_oracle.h"

static uint64_t rng_state = 0x243F6A8885A308D3ull;
static uint64_t next_u64(void) { /* SplitMix64 */
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static float uniform_pm(float a) { return a * ((float)(next_u64() >> 40) / (float)(1u << 24) * 2.0f - 1.0f); }

static int check(int P, int chunks, int bits, int comp) {
  const int64_t n = (int64_t)P * ORC_GROUP * chunks, C = n / P;
  const int64_t cb = bits == 8 ? n : n / 2, ccb = bits == 8 ? C : C / 2;
  uint16_t* xs[ORC_MAX_RANKS];
  float *mf[ORC_MAX_RANKS], *ms[ORC_MAX_RANKS], *mf0[ORC_MAX_RANKS], *ms0[ORC_MAX_RANKS];
  uint8_t* c1[ORC_MAX_RANKS];
  float* s1[ORC_MAX_RANKS];
  for (int p = 0; p < P; ++p) {
    xs[p] = malloc(n * sizeof(uint16_t));
    mf[p] = malloc(n * sizeof(float));
    ms[p] = malloc(n * sizeof(float));
    mf0[p] = malloc(n * sizeof(float));
    ms0[p] = malloc(n * sizeof(float));
    c1[p] = malloc(cb);
    s1[p] = malloc(n / ORC_GROUP * sizeof(float));
    for (int64_t i = 0; i < n; ++i) {
      xs[p][i] = orc_f32_to_bf16(uniform_pm(3.0f));
      mf[p][i] = mf0[p][i] = uniform_pm(0.1f);
      ms[p][i] = ms0[p][i] = uniform_pm(0.1f);
    }
  }
  uint8_t* codes2 = malloc(cb);
  float* scales2 = malloc(n / ORC_GROUP * sizeof(float));
  uint16_t* y = malloc(n * sizeof(uint16_t));
  int bad = orc_simulate(P, n, (const uint16_t* const*)xs, mf, ms, codes2, scales2, y, c1, s1, NULL,
                         NULL, comp, bits);
  /* rank mode for every rank against the simulation */
  uint8_t* send_c = malloc(cb);
  float* send_s = malloc(n / ORC_GROUP * sizeof(float));
  uint8_t* own_c = malloc(ccb);
  float* own_s = malloc(C / ORC_GROUP * sizeof(float));
  uint16_t* y1 = malloc(n * sizeof(uint16_t));
  uint16_t* y_own = malloc(C * sizeof(uint16_t));
  for (int p = 0; p < P && !bad; ++p) {
    const uint8_t* rc[ORC_MAX_RANKS];
    const float* rs[ORC_MAX_RANKS];
    const uint8_t* gc[ORC_MAX_RANKS];
    const float* gs[ORC_MAX_RANKS];
    for (int q = 0; q < P; ++q) {
      rc[q] = c1[q] + p * ccb;
      rs[q] = s1[q] + p * C / ORC_GROUP;
      gc[q] = codes2 + q * ccb;
      gs[q] = scales2 + q * C / ORC_GROUP;
    }
    float* f = malloc(n * sizeof(float));
    float* s = malloc(n * sizeof(float));
    memcpy(f, mf0[p], n * sizeof(float));
    memcpy(s, ms0[p], n * sizeof(float));
    bad |= orc_call(P, p, n, xs[p], f, s, rc, rs, gc, gs, send_c, send_s, own_c, own_s, y1, comp, bits);
    bad |= memcmp(y1, y, n * sizeof(uint16_t)) != 0;
    if (comp) bad |= memcmp(f, mf[p], n * sizeof(float)) != 0 || memcmp(s, ms[p], n * sizeof(float)) != 0;
    /* the threaded driver, with more threads than some steps have groups */
    for (int T = 2; T <= 5; T += 3) {
      memcpy(f, mf0[p], n * sizeof(float));
      memcpy(s, ms0[p], n * sizeof(float));
      memset(y1, 0, n * sizeof(uint16_t));
      bad |= orc_call_mt(T, P, p, n, xs[p], f, s, rc, rs, gc, gs, send_c, send_s, own_c, own_s, y1,
                         comp, bits);
      bad |= memcmp(y1, y, n * sizeof(uint16_t)) != 0;
      if (comp)
        bad |= memcmp(f, mf[p], n * sizeof(float)) != 0 || memcmp(s, ms[p], n * sizeof(float)) != 0;
    }
    memcpy(f, mf0[p], n * sizeof(float));
    memcpy(s, ms0[p], n * sizeof(float));
    bad |= orc_rs_call(P, p, n, xs[p], f, s, rc, rs, send_c, send_s, y_own, comp, bits);
    {
      float* f2 = malloc(n * sizeof(float));
      float* s2 = malloc(n * sizeof(float));
      uint16_t* y2 = malloc(C * sizeof(uint16_t));
      memcpy(f2, mf0[p], n * sizeof(float));
      memcpy(s2, ms0[p], n * sizeof(float));
      bad |= orc_rs_call_mt(3, P, p, n, xs[p], f2, s2, rc, rs, send_c, send_s, y2, comp, bits);
      bad |= memcmp(y2, y_own, C * sizeof(uint16_t)) != 0;
      bad |= memcmp(f2, f, n * sizeof(float)) != 0 || memcmp(s2, s, n * sizeof(float)) != 0;
      free(f2); free(s2); free(y2);
    }
    free(f);
    free(s);
  }
  uint16_t* yrs = malloc(n * sizeof(uint16_t));
  bad |= orc_rs_simulate(P, n, (const uint16_t* const*)xs, mf0, ms0, yrs, NULL, NULL, comp, bits);
  /* an invalid width and shape are rejected */
  bad |= orc_call(P, 0, n, xs[0], mf[0], ms[0], NULL, NULL, NULL, NULL, send_c, send_s, own_c, own_s,
                  y1, comp, 5) != -1;
  bad |= orc_simulate(P, n + 1, (const uint16_t* const*)xs, mf, ms, codes2, scales2, y, NULL, NULL, NULL,
                      NULL, comp, bits) != -1;
  for (int p = 0; p < P; ++p) {
    free(xs[p]); free(mf[p]); free(ms[p]); free(mf0[p]); free(ms0[p]); free(c1[p]); free(s1[p]);
  }
  free(codes2); free(scales2); free(y); free(send_c); free(send_s); free(own_c); free(own_s);
  free(y1); free(y_own); free(yrs);
  if (bad) fprintf(stderr, "mismatch: P=%d chunks=%d bits=%d comp=%d\n", P, chunks, bits, comp);
  return bad;
}

int main(void) {
  int bad = 0;
  for (int P = 1; P <= ORC_MAX_RANKS; P += (P < 4 ? 1 : 5))
    for (int bits = 4; bits <= 8; bits += 4)
      for (int comp = 0; comp <= 1; ++comp) bad |= check(P, 1 + P % 3, bits, comp);
  /* the quantizer on special groups */
  float v[ORC_GROUP];
  int8_t q[ORC_GROUP];
  float s;
  memset(v, 0, sizeof v);
  orc_quantize_group_q(v, ORC_GROUP, 127, q, &s, 0);
  bad |= s != 0.0f;
  v[5] = 1e-45f;
  orc_quantize_group_q(v, ORC_GROUP, 7, q, &s, 0);
  bad |= s != 0.0f || q[5] != 0;
  printf(bad ? "FAILED\n" : "ok\n");
  return bad;
}
