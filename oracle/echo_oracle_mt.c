/*
 * echo_oracle_mt.c -- threaded driver of the CPU oracle's rank-mode call.
 *
 * TEST INFRASTRUCTURE ONLY: used by the full-size parity tests and the
 * CPU-baseline leg of the benchmark, never by the product path.
 *
 * It adds no arithmetic.  The steps of a call act on each 128-element group
 * on its own (the entry pass, the rank-order sum of the own chunk, the exit
 * pass and the averages' update), so the driver cuts each step's range into
 * disjoint runs of whole groups, one per host thread, and every thread calls
 * the single-thread step function (orc_encode, orc_reduce_chunk, orc_decode,
 * orc_update_span) on its run.  Each element therefore goes through exactly
 * the operations orc_call applies to it, and the outputs are bit-identical
 * for any thread count.  Steps run one after the other, as in orc_call:
 * entry, then reduce and exit, then update.
 */
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

#include "echo_oracle.h"

#define MT_MAX_THREADS 256

static int64_t code_bytes_of(int64_t n, int bits) { return bits == 8 ? n : n / 2; }

/* Everything a step of one call reads or writes. */
typedef struct {
  int nranks, rank, comp, bits;
  int64_t n, C;
  const uint16_t* x;
  float* m_fast;
  float* m_slow;
  const uint8_t* const* recv_codes;
  const float* const* recv_scales;
  const uint8_t* const* gath_codes;
  const float* const* gath_scales;
  uint8_t* codes1; /* stage-1 message of all n elements */
  float* scales1;
  float* e2;       /* own chunk */
  uint8_t* own_codes2;
  float* own_scales2;
  uint16_t* y;     /* all n elements (all-reduce) or the own chunk (reduce-scatter) */
} call_job;

typedef void (*step_fn)(const call_job* j, int64_t g0, int64_t g1);

/* entry pass over groups [g0, g1) of the tensor */
static void step_encode(const call_job* j, int64_t g0, int64_t g1) {
  const int64_t e0 = g0 * ORC_GROUP;
  orc_encode((g1 - g0) * ORC_GROUP, j->x + e0, j->comp ? j->m_fast + e0 : NULL,
             j->comp ? j->m_slow + e0 : NULL, j->codes1 + code_bytes_of(e0, j->bits),
             j->scales1 + g0, NULL, j->comp, j->bits);
}

/* reduce of groups [g0, g1) of the own chunk; slot `rank` is the own
 * stage-1 message */
static void step_reduce(const call_job* j, int64_t g0, int64_t g1) {
  const int64_t e0 = g0 * ORC_GROUP;
  const int64_t cb0 = code_bytes_of(e0, j->bits);
  const int64_t own = (int64_t)j->rank * j->C;
  const uint8_t* sc[ORC_MAX_RANKS];
  const float* ss[ORC_MAX_RANKS];
  for (int q = 0; q < j->nranks; ++q) {
    if (q == j->rank) {
      sc[q] = j->codes1 + code_bytes_of(own, j->bits) + cb0;
      ss[q] = j->scales1 + own / ORC_GROUP + g0;
    } else {
      sc[q] = j->recv_codes[q] + cb0;
      ss[q] = j->recv_scales[q] + g0;
    }
  }
  orc_reduce_chunk(j->nranks, (g1 - g0) * ORC_GROUP, sc, ss, j->own_codes2 + cb0,
                   j->own_scales2 + g0, j->y + own + e0, j->e2 + e0, j->bits);
}

/* reduce-scatter: rank-order sum of groups [g0, g1) of the own chunk,
 * output as bf16 into the chunk-local y */
static void step_reduce_sum(const call_job* j, int64_t g0, int64_t g1) {
  const int64_t e0 = g0 * ORC_GROUP;
  const int64_t cb0 = code_bytes_of(e0, j->bits);
  const int64_t own = (int64_t)j->rank * j->C;
  const uint8_t* sc[ORC_MAX_RANKS];
  const float* ss[ORC_MAX_RANKS];
  for (int q = 0; q < j->nranks; ++q) {
    if (q == j->rank) {
      sc[q] = j->codes1 + code_bytes_of(own, j->bits) + cb0;
      ss[q] = j->scales1 + own / ORC_GROUP + g0;
    } else {
      sc[q] = j->recv_codes[q] + cb0;
      ss[q] = j->recv_scales[q] + g0;
    }
  }
  orc_reduce_chunk_sum(j->nranks, (g1 - g0) * ORC_GROUP, sc, ss, j->y + e0, j->e2 + e0, j->bits);
}

/* exit pass over groups [g0, g1) of the gathered chunks, counted over the
 * chunks other than the own one laid end to end */
static void step_decode(const call_job* j, int64_t g0, int64_t g1) {
  const int64_t cg = j->C / ORC_GROUP;
  int64_t v = 0; /* first virtual group of the chunk below */
  for (int c = 0; c < j->nranks; ++c) {
    if (c == j->rank) continue;
    const int64_t a = g0 > v ? g0 : v, b = g1 < v + cg ? g1 : v + cg;
    if (a < b) {
      const int64_t l0 = (a - v) * ORC_GROUP; /* element offset inside chunk c */
      orc_decode((b - a) * ORC_GROUP, j->gath_codes[c] + code_bytes_of(l0, j->bits),
                 j->gath_scales[c] + (a - v), j->y + (int64_t)c * j->C + l0, j->bits);
    }
    v += cg;
  }
}

/* averages' update over groups [g0, g1) of the tensor */
static void step_update(const call_job* j, int64_t g0, int64_t g1) {
  const int64_t own0 = (int64_t)j->rank * j->C;
  orc_update_span(g0 * ORC_GROUP, g1 * ORC_GROUP, own0, own0 + j->C, j->x, j->m_fast, j->m_slow,
                  j->codes1, j->scales1, j->e2, NULL, j->bits);
}

typedef struct {
  const call_job* job;
  step_fn fn;
  int64_t g0, g1;
} span_task;

static void* run_span(void* arg) {
  const span_task* t = (const span_task*)arg;
  if (t->g0 < t->g1) t->fn(t->job, t->g0, t->g1);
  return NULL;
}

/* fn over groups [0, groups), cut into `threads` contiguous runs.  Run 0 is
 * done on the calling thread; a run whose thread cannot be started is done
 * there too. */
static void parallel_groups(int threads, int64_t groups, step_fn fn, const call_job* job) {
  span_task task[MT_MAX_THREADS];
  pthread_t tid[MT_MAX_THREADS];
  int started[MT_MAX_THREADS];
  for (int t = 0; t < threads; ++t) {
    task[t].job = job;
    task[t].fn = fn;
    task[t].g0 = groups * t / threads;
    task[t].g1 = groups * (t + 1) / threads;
    started[t] = 0;
  }
  for (int t = 1; t < threads; ++t)
    started[t] = pthread_create(&tid[t], NULL, run_span, &task[t]) == 0;
  run_span(&task[0]);
  for (int t = 1; t < threads; ++t) {
    if (started[t])
      pthread_join(tid[t], NULL);
    else
      run_span(&task[t]);
  }
}

/* the shared set-up of both threaded calls: checks, the job, its buffers */
static int job_init(call_job* j, int nranks, int rank, int64_t n, const uint16_t* x,
                    float* m_fast, float* m_slow, const uint8_t* const* recv_codes,
                    const float* const* recv_scales, uint16_t* y, int comp, int bits) {
  if (nranks < 1 || nranks > ORC_MAX_RANKS || rank < 0 || rank >= nranks) return -1;
  if (n <= 0 || n % ((int64_t)nranks * ORC_GROUP) != 0 || (bits != 4 && bits != 8)) return -1;
  memset(j, 0, sizeof *j);
  j->nranks = nranks;
  j->rank = rank;
  j->comp = comp;
  j->bits = bits;
  j->n = n;
  j->C = n / nranks;
  j->x = x;
  j->m_fast = m_fast;
  j->m_slow = m_slow;
  j->recv_codes = recv_codes;
  j->recv_scales = recv_scales;
  j->y = y;
  j->codes1 = malloc((size_t)code_bytes_of(n, bits));
  j->scales1 = malloc((size_t)(n / ORC_GROUP) * sizeof(float));
  j->e2 = malloc((size_t)j->C * sizeof(float));
  if (!j->codes1 || !j->scales1 || !j->e2) {
    free(j->codes1); free(j->scales1); free(j->e2);
    return -1;
  }
  return 0;
}

static void job_free(call_job* j) {
  free(j->codes1); free(j->scales1); free(j->e2);
}

static int clamp_threads(int threads) {
  if (threads < 1) return 1;
  return threads > MT_MAX_THREADS ? MT_MAX_THREADS : threads;
}

/* the entry pass, and the stage-1 message of every chunk but the own one */
static void entry_and_send(int threads, const call_job* j, uint8_t* send_codes, float* send_scales) {
  const int64_t cg = j->C / ORC_GROUP, cb = code_bytes_of(j->C, j->bits);
  parallel_groups(threads, j->n / ORC_GROUP, step_encode, j);
  for (int c = 0; c < j->nranks; ++c) {
    if (c == j->rank) continue;
    memcpy(send_codes + c * cb, j->codes1 + c * cb, (size_t)cb);
    memcpy(send_scales + c * cg, j->scales1 + c * cg, (size_t)cg * sizeof(float));
  }
}

int orc_call_mt(int threads, int nranks, int rank, int64_t n, const uint16_t* x, float* m_fast,
                float* m_slow, const uint8_t* const* recv_codes, const float* const* recv_scales,
                const uint8_t* const* gath_codes, const float* const* gath_scales,
                uint8_t* send_codes, float* send_scales, uint8_t* own_codes2,
                float* own_scales2, uint16_t* y, int comp, int bits) {
  call_job j;
  if (job_init(&j, nranks, rank, n, x, m_fast, m_slow, recv_codes, recv_scales, y, comp, bits))
    return -1;
  threads = clamp_threads(threads);
  j.gath_codes = gath_codes;
  j.gath_scales = gath_scales;
  j.own_codes2 = own_codes2;
  j.own_scales2 = own_scales2;
  const int64_t cg = j.C / ORC_GROUP;
  entry_and_send(threads, &j, send_codes, send_scales);
  parallel_groups(threads, cg, step_reduce, &j);
  parallel_groups(threads, (int64_t)(nranks - 1) * cg, step_decode, &j);
  if (comp) parallel_groups(threads, n / ORC_GROUP, step_update, &j);
  job_free(&j);
  return 0;
}

int orc_rs_call_mt(int threads, int nranks, int rank, int64_t n, const uint16_t* x,
                   float* m_fast, float* m_slow, const uint8_t* const* recv_codes,
                   const float* const* recv_scales, uint8_t* send_codes, float* send_scales,
                   uint16_t* y_own, int comp, int bits) {
  call_job j;
  if (job_init(&j, nranks, rank, n, x, m_fast, m_slow, recv_codes, recv_scales, y_own, comp, bits))
    return -1;
  threads = clamp_threads(threads);
  entry_and_send(threads, &j, send_codes, send_scales);
  parallel_groups(threads, j.C / ORC_GROUP, step_reduce_sum, &j);
  if (comp) parallel_groups(threads, n / ORC_GROUP, step_update, &j);
  job_free(&j);
  return 0;
}
