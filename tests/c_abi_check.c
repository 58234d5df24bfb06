/* A plain C11 consumer of libecho (include/echo.h): no Python, no torch.
 *
 *   c_abi_check cpu   library facts, argument rejections and empty calls;
 *                     makes no HIP call, so it runs without a GPU
 *   c_abi_check gpu   rank 1 of P = 4 on hipMalloc'd buffers: three fused
 *                     calls with the averages carried, the same three calls
 *                     through the phased entry points on a second state, and
 *                     through the pipelined form (entry one chunk at a time in
 *                     reverse order, reduce, exit one gathered chunk at a time
 *                     with echo_decode) on a third, and through the deferred-
 *                     update schedule with the correction array
 *                     (echo_correction, echo_encode_corr, echo_reduce_shard,
 *                     echo_call_exit, echo_update_corr) on a fourth, each
 *                     checked bit for bit against the CPU oracle
 *
 * Prints "ok" and exits 0 on success.  Test infrastructure: it links the
 * oracle (liborc.so) beside the library only to compare them. */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "echo.h"
#include "echo_oracle.h"

#define FAIL(...)                                   \
  do {                                              \
    fprintf(stderr, "c_abi_check: " __VA_ARGS__);   \
    fprintf(stderr, "\n");                          \
    exit(1);                                        \
  } while (0)

#define EXPECT(cond, ...) \
  do {                    \
    if (!(cond)) FAIL(__VA_ARGS__); \
  } while (0)

#define HIP(call)                                                              \
  do {                                                                         \
    hipError_t e_ = (call);                                                    \
    if (e_ != hipSuccess) FAIL("%s: %s", #call, hipGetErrorString(e_));       \
  } while (0)

/* SplitMix64: the inputs' random source */
static uint64_t rng_state;
static uint64_t next_u64(void) {
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
static float uniform01(void) { return (float)(next_u64() >> 40) / (float)(1u << 24); }

/* finite bf16 bit patterns with magnitudes between 2^-7 and 2^4, either sign */
static uint16_t random_bf16(void) {
  const uint64_t r = next_u64();
  const uint16_t sign = (uint16_t)((r & 1u) << 15);
  const uint16_t expo = (uint16_t)(120u + (r >> 1) % 12u);
  const uint16_t mant = (uint16_t)((r >> 8) & 0x7Fu);
  return (uint16_t)(sign | (uint16_t)(expo << 7) | mant);
}

/* a 4-bit message: bytes with no -8 field, scales in [0.05, 0.55) */
static void random_message(uint8_t* codes, float* scales, int64_t chunk) {
  for (int64_t i = 0; i < chunk / 2; ++i) {
    uint8_t b;
    do b = (uint8_t)next_u64(); while ((b & 0xFu) == 8u || (b >> 4) == 8u);
    codes[i] = b;
  }
  for (int64_t g = 0; g < chunk / ECHO_GROUP; ++g) scales[g] = 0.05f + 0.5f * uniform01();
}

static void check_cpu(void) {
  echo_config cfg;
  EXPECT(echo_get_config(&cfg) == ECHO_SUCCESS, "echo_get_config");
  EXPECT(echo_version() == ECHO_ABI_VERSION && cfg.abi_version == ECHO_ABI_VERSION, "version");
  EXPECT(cfg.group == ECHO_GROUP && cfg.qmax == ECHO_QMAX && cfg.qmax8 == ECHO_QMAX8 &&
             cfg.max_ranks == ECHO_MAX_RANKS && cfg.max_elements == ECHO_MAX_ELEMENTS,
         "config integers");
  EXPECT(cfg.w_fast == ECHO_W_FAST && cfg.w_slow == ECHO_W_SLOW && cfg.beta_fast == ECHO_BETA_FAST &&
             cfg.alpha_fast == ECHO_ALPHA_FAST && cfg.beta_slow == ECHO_BETA_SLOW &&
             cfg.alpha_slow == ECHO_ALPHA_SLOW,
         "config weights");
  EXPECT(cfg.group == ORC_GROUP && cfg.qmax == ORC_QMAX && cfg.qmax8 == ORC_QMAX8, "oracle constants");
  for (int s = 0; s >= -7; --s) EXPECT(echo_status_string(s) != NULL, "status string %d", s);

  /* rejections (fake, aligned addresses: nothing is dereferenced or launched) */
  float* const fa = (float*)(uintptr_t)(1ull << 32);
  float* const fb = (float*)(uintptr_t)(2ull << 32);
  echo_state st;
  EXPECT(echo_state_init(NULL, fa, fb, 1024, 2, 0, NULL) == ECHO_ERR_INVALID_ARGUMENT, "null state");
  EXPECT(echo_state_init(&st, fa, fb, 1000, 2, 0, NULL) == ECHO_ERR_SHAPE, "shape");
  EXPECT(echo_state_init(&st, fa, fb, 1024, 17, 0, NULL) == ECHO_ERR_RANKS, "ranks");
  EXPECT(echo_state_init(&st, fa + 1, fb, 1024, 2, 0, NULL) == ECHO_ERR_ALIGNMENT, "alignment");
  EXPECT(echo_state_init(&st, fa, fa + 256, 1024, 2, 0, NULL) == ECHO_ERR_ALIAS, "alias");
  EXPECT(echo_decode(128, 5, (const uint8_t*)fa, fb, (uint16_t*)(uintptr_t)(3ull << 32), NULL) ==
             ECHO_ERR_FORMAT,
         "format");

  /* empty calls: success, pointers not looked at */
  EXPECT(echo_state_init(&st, NULL, NULL, 0, 4, 1, NULL) == ECHO_SUCCESS, "empty init");
  const uint8_t* nc[ECHO_MAX_RANKS] = {0};
  const float* ns[ECHO_MAX_RANKS] = {0};
  EXPECT(echo_call(&st, NULL, nc, ns, nc, ns, NULL, NULL, NULL, NULL, NULL, NULL) == ECHO_SUCCESS,
         "empty call");
  EXPECT(echo_decode(0, 4, NULL, NULL, NULL, NULL) == ECHO_SUCCESS, "empty decode");
  st.bits = 3;
  EXPECT(echo_call(&st, NULL, nc, ns, nc, ns, NULL, NULL, NULL, NULL, NULL, NULL) == ECHO_ERR_FORMAT,
         "empty call keeps its scalar checks");
}

static void* dev_copy(const void* host, size_t bytes) {
  void* d = NULL;
  HIP(hipMalloc(&d, bytes));
  HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
  return d;
}

static void expect_equal(const void* dev, const void* want, size_t bytes, const char* what, int call) {
  unsigned char* got = (unsigned char*)malloc(bytes);
  if (!got) FAIL("out of host memory");
  HIP(hipMemcpy(got, dev, bytes, hipMemcpyDeviceToHost));
  for (size_t i = 0; i < bytes; ++i)
    if (got[i] != ((const unsigned char*)want)[i]) FAIL("call %d: %s differs at byte %zu", call, what, i);
  free(got);
}

static void check_gpu(void) {
  enum { P = 4, RANK = 1, K = 5 };
  const int64_t n = (int64_t)P * ECHO_GROUP * K, C = n / P;
  const size_t cb = (size_t)C / 2, cs = (size_t)(C / ECHO_GROUP) * sizeof(float);

  /* host inputs: three calls' x, and one set of incoming and gathered messages */
  uint16_t* x[3];
  for (int c = 0; c < 3; ++c) {
    x[c] = (uint16_t*)malloc((size_t)n * 2);
    if (!x[c]) FAIL("out of host memory");
    for (int64_t i = 0; i < n; ++i) x[c][i] = random_bf16();
  }
  uint8_t* hc[2][P];
  float* hs[2][P];
  const uint8_t* dc[2][P];
  const float* ds[2][P];
  for (int m = 0; m < 2; ++m)
    for (int q = 0; q < P; ++q) {
      hc[m][q] = NULL;
      hs[m][q] = NULL;
      dc[m][q] = NULL;
      ds[m][q] = NULL;
      if (q == RANK) continue;
      hc[m][q] = (uint8_t*)malloc(cb);
      hs[m][q] = (float*)malloc(cs);
      if (!hc[m][q] || !hs[m][q]) FAIL("out of host memory");
      random_message(hc[m][q], hs[m][q], C);
      dc[m][q] = (const uint8_t*)dev_copy(hc[m][q], cb);
      ds[m][q] = (const float*)dev_copy(hs[m][q], cs);
    }

  /* oracle state and outputs */
  float* omf = (float*)calloc((size_t)n, sizeof(float));
  float* oms = (float*)calloc((size_t)n, sizeof(float));
  uint8_t* o_send_c = (uint8_t*)malloc((size_t)n / 2);
  float* o_send_s = (float*)malloc((size_t)(n / ECHO_GROUP) * sizeof(float));
  uint8_t* o_own_c = (uint8_t*)malloc(cb);
  float* o_own_s = (float*)malloc(cs);
  uint16_t* o_y = (uint16_t*)malloc((size_t)n * 2);
  if (!omf || !oms || !o_send_c || !o_send_s || !o_own_c || !o_own_s || !o_y) FAIL("out of host memory");

  /* device state (four: fused, phased, pipelined, deferred update with the
   * correction array) and outputs */
  float *mf[4], *ms[4];
  echo_state st[4];
  uint16_t *dx, *dy;
  uint8_t *send_c, *own_c;
  float *send_s, *own_s, *corr, *e2;
  for (int v = 0; v < 4; ++v) {
    HIP(hipMalloc((void**)&mf[v], (size_t)n * sizeof(float)));
    HIP(hipMalloc((void**)&ms[v], (size_t)n * sizeof(float)));
    EXPECT(echo_state_init(&st[v], mf[v], ms[v], n, P, RANK, NULL) == ECHO_SUCCESS, "state init");
  }
  HIP(hipMalloc((void**)&dx, (size_t)n * 2));
  HIP(hipMalloc((void**)&dy, (size_t)n * 2));
  HIP(hipMalloc((void**)&send_c, (size_t)n / 2));
  HIP(hipMalloc((void**)&send_s, (size_t)(n / ECHO_GROUP) * sizeof(float)));
  HIP(hipMalloc((void**)&own_c, cb));
  HIP(hipMalloc((void**)&own_s, cs));
  HIP(hipMalloc((void**)&corr, (size_t)n * sizeof(float)));
  HIP(hipMalloc((void**)&e2, (size_t)C * sizeof(float)));
  hipStream_t s;
  HIP(hipStreamCreate(&s));
  EXPECT(echo_correction(&st[3], corr, (echo_stream_t)s) == ECHO_SUCCESS, "correction");

  for (int v = 0; v < 4; ++v) {
    memset(omf, 0, (size_t)n * sizeof(float));
    memset(oms, 0, (size_t)n * sizeof(float));
    for (int c = 0; c < 3; ++c) {
      HIP(hipMemcpy(dx, x[c], (size_t)n * 2, hipMemcpyHostToDevice));
      if (v == 0) {
        EXPECT(echo_call(&st[0], dx, dc[0], ds[0], dc[1], ds[1], send_c, send_s, own_c, own_s, dy,
                         (echo_stream_t)s) == ECHO_SUCCESS,
               "echo_call");
      } else if (v == 1) {
        EXPECT(echo_call_entry(&st[1], dx, send_c, send_s, (echo_stream_t)s) == ECHO_SUCCESS, "entry");
        EXPECT(echo_call_reduce(&st[1], dx, dc[0], ds[0], own_c, own_s, dy, (echo_stream_t)s) ==
                   ECHO_SUCCESS,
               "reduce");
        EXPECT(echo_call_exit(&st[1], dc[1], ds[1], dy, (echo_stream_t)s) == ECHO_SUCCESS, "exit");
      } else if (v == 3) {
        const uint8_t* sh_c[P];
        const float* sh_s[P];
        for (int q = 0; q < P; ++q) {
          sh_c[q] = q == RANK ? send_c + RANK * cb : dc[0][q];
          sh_s[q] = q == RANK ? send_s + RANK * (C / ECHO_GROUP) : ds[0][q];
        }
        EXPECT(echo_encode_corr(&st[3], dx, corr, send_c, send_s, (echo_stream_t)s) == ECHO_SUCCESS,
               "encode from the correction");
        EXPECT(echo_reduce_shard(P, C, 4, sh_c, sh_s, own_c, own_s, dy + RANK * C, e2, (echo_stream_t)s) ==
                   ECHO_SUCCESS,
               "reduce shard");
        EXPECT(echo_call_exit(&st[3], dc[1], ds[1], dy, (echo_stream_t)s) == ECHO_SUCCESS, "exit");
        EXPECT(echo_update_corr(&st[3], dx, send_c, send_s, e2, corr, (echo_stream_t)s) == ECHO_SUCCESS,
               "update and correction");
      } else {
        for (int j = P - 1; j >= 0; --j)
          EXPECT(echo_call_entry_range(&st[2], dx, j, j + 1, send_c, send_s, (echo_stream_t)s) ==
                     ECHO_SUCCESS,
                 "entry range");
        EXPECT(echo_call_reduce(&st[2], dx, dc[0], ds[0], own_c, own_s, dy, (echo_stream_t)s) ==
                   ECHO_SUCCESS,
               "reduce");
        for (int j = 0; j < P; ++j) {
          if (j == RANK) continue;
          EXPECT(echo_decode(C, 4, dc[1][j], ds[1][j], dy + j * C, (echo_stream_t)s) == ECHO_SUCCESS,
                 "decode");
        }
      }
      HIP(hipStreamSynchronize(s));
      EXPECT(orc_call(P, RANK, n, x[c], omf, oms, (const uint8_t* const*)hc[0], (const float* const*)hs[0],
                      (const uint8_t* const*)hc[1], (const float* const*)hs[1], o_send_c, o_send_s,
                      o_own_c, o_own_s, o_y, 1, 4) == 0,
             "orc_call");
      expect_equal(dy, o_y, (size_t)n * 2,
                   v == 0 ? "y" : v == 1 ? "phased y" : v == 2 ? "pipelined y" : "deferred y", c);
      expect_equal(own_c, o_own_c, cb, "own codes2", c);
      expect_equal(own_s, o_own_s, cs, "own scales2", c);
      expect_equal(mf[v], omf, (size_t)n * sizeof(float), "m_fast", c);
      expect_equal(ms[v], oms, (size_t)n * sizeof(float), "m_slow", c);
      for (int j = 0; j < P; ++j) {
        if (j == RANK) continue;
        expect_equal(send_c + j * cb, o_send_c + j * cb, cb, "send codes", c);
        expect_equal((const char*)send_s + j * cs, (const char*)o_send_s + j * cs, cs, "send scales", c);
      }
    }
  }

  HIP(hipStreamDestroy(s));
  HIP(hipFree(corr));
  HIP(hipFree(e2));
  for (int v = 0; v < 4; ++v) {
    HIP(hipFree(mf[v]));
    HIP(hipFree(ms[v]));
  }
  HIP(hipFree(dx));
  HIP(hipFree(dy));
  HIP(hipFree(send_c));
  HIP(hipFree(send_s));
  HIP(hipFree(own_c));
  HIP(hipFree(own_s));
  for (int m = 0; m < 2; ++m)
    for (int q = 0; q < P; ++q) {
      if (q == RANK) continue;
      HIP(hipFree((void*)dc[m][q]));
      HIP(hipFree((void*)ds[m][q]));
      free(hc[m][q]);
      free(hs[m][q]);
    }
  for (int c = 0; c < 3; ++c) free(x[c]);
  free(omf);
  free(oms);
  free(o_send_c);
  free(o_send_s);
  free(o_own_c);
  free(o_own_s);
  free(o_y);
}

int main(int argc, char** argv) {
  if (argc != 2 || (strcmp(argv[1], "cpu") != 0 && strcmp(argv[1], "gpu") != 0))
    FAIL("usage: c_abi_check cpu|gpu");
  rng_state = 20261203u;
  check_cpu();
  if (strcmp(argv[1], "gpu") == 0) check_gpu();
  printf("ok\n");
  return 0;
}
