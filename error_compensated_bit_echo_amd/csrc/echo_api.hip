// echo_api.hip -- host side of libecho: argument checks and kernel launches
// behind the C ABI declared in include/echo.h.
//
// Every entry point validates all of its arguments before enqueueing any
// work, so a rejected call leaves the stream untouched.  The library keeps
// no global mutable state and allocates nothing: buffers, streams and their
// ordering belong to the caller.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include "echo.h"
#include "echo_device.h"

using namespace echo;

namespace {

// Launch shape.  Each wavefront takes one step of work (stage-1 and reduce:
// one slice of two groups; exit: two quads of groups) and the grid covers
// the whole range, so no wave loops: on MI355X a full grid of short-lived
// workgroups streams HBM faster than a persistent grid-stride loop (measured
// on the 1 GB message: 6.15 vs 4.37 TB/s for the entry pass).  The kernels
// keep their grid-stride loop, so a grid capped at HIP's launch limit
// (launch_shape.h) stays correct.
#ifndef ECHO_U_STAGE1
#define ECHO_U_STAGE1 1
#endif
#ifndef ECHO_U_REDUCE
#define ECHO_U_REDUCE 1
#endif
#ifndef ECHO_U_EXIT
#define ECHO_U_EXIT 2
#endif
#ifndef ECHO_U_PLAIN
#define ECHO_U_PLAIN 2
#endif
#ifndef ECHO_U_REDUCE_PLAIN
#define ECHO_U_REDUCE_PLAIN 1
#endif
constexpr int kU1 = ECHO_U_STAGE1;  // stage-1 slices (2 groups each) per wave step
constexpr int kUR = ECHO_U_REDUCE;  // reduce slices per wave step
constexpr int kUD = ECHO_U_EXIT;    // exit: quads of groups per wave step

// Launch `kernel` with its one by-value argument struct.  The status is the
// launch's own (hipLaunchKernel's return value), so an error an earlier,
// unrelated HIP call left in the thread's last-error slot is neither
// reported as this call's nor cleared.
template <typename A>
int launch(void (*kernel)(A), dim3 grid, hipStream_t s, A arg) {
  void* argv[] = {&arg};
  const hipError_t e =
      hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, dim3(kBlock), argv, 0, s);
  return e == hipSuccess ? ECHO_SUCCESS : ECHO_ERR_HIP;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

bool bits_ok(int32_t bits) { return bits == 4 || bits == 8; }

// bytes of the codes of n elements: packed nibbles, or one byte per code
int64_t code_bytes(int64_t n, int32_t bits) { return bits == 8 ? n : n / 2; }

// A check that passed with nothing to do: zero elements.  The entry point
// then returns ECHO_SUCCESS without looking at its pointers or launching.
constexpr int kEmpty = 1;

// the status an entry point returns for a check result that is not SUCCESS
int finished(int rc) { return rc < 0 ? rc : ECHO_SUCCESS; }

int check_elements(int64_t n, int64_t multiple) {
  if (n < 0 || n > ECHO_MAX_ELEMENTS || n % multiple != 0) return ECHO_ERR_SHAPE;
  return n == 0 ? kEmpty : ECHO_SUCCESS;
}

int check_ranks_shape(int64_t n, int32_t P) {
  if (P < 1 || P > ECHO_MAX_RANKS) return ECHO_ERR_RANKS;
  return check_elements(n, (int64_t)P * ECHO_GROUP);
}

int check_state(const echo_state* st) {
  if (!st) return ECHO_ERR_INVALID_ARGUMENT;
  const int shape = check_ranks_shape(st->n, st->nranks);
  if (shape < 0) return shape;
  if (st->rank < 0 || st->rank >= st->nranks) return ECHO_ERR_RANKS;
  if (!bits_ok(st->bits)) return ECHO_ERR_FORMAT;
  if (shape == kEmpty) return kEmpty;
  if (!st->m_fast || !st->m_slow) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(st->m_fast, 16) || !aligned(st->m_slow, 16)) return ECHO_ERR_ALIGNMENT;
  return ECHO_SUCCESS;
}

// Byte ranges written (outputs, including read-modify-write state) and read
// (inputs).  Outputs must be pairwise disjoint and disjoint from every
// input, except one explicitly allowed identical pair (y == x in place).
class Aliases {
 public:
  void out(const void* p, int64_t bytes) { add(outs_, no_, p, bytes); }
  void in(const void* p, int64_t bytes) { add(ins_, ni_, p, bytes); }
  void allow_identical(const void* a, const void* b) { allow_a_ = a; allow_b_ = b; }
  bool ok() const {
    for (int i = 0; i < no_; ++i) {
      for (int j = i + 1; j < no_; ++j)
        if (overlap(outs_[i], outs_[j])) return false;
      for (int j = 0; j < ni_; ++j)
        if (overlap(outs_[i], ins_[j]) && !allowed(outs_[i], ins_[j])) return false;
    }
    return true;
  }

 private:
  struct Span { uintptr_t lo, hi; };
  static constexpr int kCap = 4 * ECHO_MAX_RANKS + 16;
  static void add(Span* s, int& k, const void* p, int64_t bytes) {
    if (!p || bytes <= 0 || k >= kCap) return;
    s[k].lo = (uintptr_t)p;
    s[k].hi = (uintptr_t)p + (uintptr_t)bytes;
    ++k;
  }
  static bool overlap(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }
  bool allowed(const Span& o, const Span& i) const {
    if (!allow_a_) return false;
    const uintptr_t a = (uintptr_t)allow_a_, b = (uintptr_t)allow_b_;
    return o.lo == i.lo && o.hi == i.hi && ((o.lo == a && i.lo == b) || (o.lo == b && i.lo == a));
  }
  Span outs_[kCap], ins_[kCap];
  int no_ = 0, ni_ = 0;
  const void* allow_a_ = nullptr;
  const void* allow_b_ = nullptr;
};

#ifndef ECHO_UPDATE_MAX_BLOCKS
#define ECHO_UPDATE_MAX_BLOCKS kMaxBlocks
#endif

// slices per wave step for each stage-1 mode: the uncompensated entry pass
// moves only 2.5 bytes per element, so its waves take more work each
constexpr int u_stage1(int mode) { return mode == kEntryPlain ? ECHO_U_PLAIN : kU1; }

template <int MODE>
int launch_stage1(const Stage1Args& a, int bits, hipStream_t s) {
  constexpr int U = u_stage1(MODE);
  const uint64_t nslices = ((uint64_t)a.groups_work + 1) / 2;
  if (nslices == 0) return ECHO_SUCCESS;
  const uint32_t blocks =
      blocks_for((nslices + U - 1) / U, is_update(MODE) ? (uint32_t)ECHO_UPDATE_MAX_BLOCKS : kMaxBlocks);
  if (bits == 8) return launch(k_stage1<MODE, 8, U>, dim3(blocks), s, a);
  return launch(k_stage1<MODE, 4, U>, dim3(blocks), s, a);
}

constexpr int u_reduce(int mode) {
  return (mode == kOwnFused || mode == kOwnRS) ? kUR : ECHO_U_REDUCE_PLAIN;
}

template <int MODE, int P>
int launch_reduce_p(const ReduceArgs& a, int bits, uint32_t blocks, hipStream_t s) {
  if (bits == 8) return launch(k_reduce<MODE, 8, P, u_reduce(MODE)>, dim3(blocks), s, a);
  return launch(k_reduce<MODE, 4, P, u_reduce(MODE)>, dim3(blocks), s, a);
}

template <int MODE>
int launch_reduce(int P, const ReduceArgs& a, int bits, hipStream_t s) {
  constexpr int U = u_reduce(MODE);
  const uint64_t nslices = ((uint64_t)a.groups + 1) / 2;
  if (nslices == 0) return ECHO_SUCCESS;
  const uint32_t blocks = blocks_for((nslices + U - 1) / U);
  switch (P) {
#define ECHO_REDUCE_CASE(p) \
  case p: return launch_reduce_p<MODE, p>(a, bits, blocks, s);
    ECHO_REDUCE_CASE(1) ECHO_REDUCE_CASE(2) ECHO_REDUCE_CASE(3) ECHO_REDUCE_CASE(4)
    ECHO_REDUCE_CASE(5) ECHO_REDUCE_CASE(6) ECHO_REDUCE_CASE(7) ECHO_REDUCE_CASE(8)
    ECHO_REDUCE_CASE(9) ECHO_REDUCE_CASE(10) ECHO_REDUCE_CASE(11) ECHO_REDUCE_CASE(12)
    ECHO_REDUCE_CASE(13) ECHO_REDUCE_CASE(14) ECHO_REDUCE_CASE(15) ECHO_REDUCE_CASE(16)
#undef ECHO_REDUCE_CASE
    default: return ECHO_ERR_RANKS;
  }
}

int launch_decode(const DecodeArgs& a, uint32_t nseg, int bits, hipStream_t s) {
  const uint64_t nquads = ((uint64_t)a.groups + 3) / 4;
  if (nquads == 0 || nseg == 0) return ECHO_SUCCESS;
  const uint32_t blocks = blocks_for((nquads + kUD - 1) / kUD, kMaxBlocks / nseg);
  if (bits == 8) return launch(k_decode<8, kUD>, dim3(blocks, nseg), s, a);
  return launch(k_decode<4, kUD>, dim3(blocks, nseg), s, a);
}

// ---- per-phase argument checks and launches (shared by the fused call) ----

struct Geometry {
  int64_t n, chunk;
  uint32_t groups, chunk_groups, own_g0, own_g1;
};

Geometry geometry(const echo_state* st) {
  Geometry g;
  g.n = st->n;
  g.chunk = st->n / st->nranks;
  g.groups = (uint32_t)(st->n / ECHO_GROUP);
  g.chunk_groups = (uint32_t)(g.chunk / ECHO_GROUP);
  g.own_g0 = (uint32_t)st->rank * g.chunk_groups;
  g.own_g1 = g.own_g0 + g.chunk_groups;
  return g;
}

int check_remote_arrays(const echo_state* st, const uint8_t* const* codes,
                        const float* const* scales) {
  if (!codes || !scales) return ECHO_ERR_INVALID_ARGUMENT;
  for (int q = 0; q < st->nranks; ++q) {
    if (q == st->rank) continue;
    if (!codes[q] || !scales[q]) return ECHO_ERR_INVALID_ARGUMENT;
    if (!aligned(codes[q], 16) || !aligned(scales[q], 4)) return ECHO_ERR_ALIGNMENT;
  }
  return ECHO_SUCCESS;
}

void add_remote_inputs(Aliases& al, const echo_state* st, const uint8_t* const* codes,
                       const float* const* scales, int64_t chunk) {
  for (int q = 0; q < st->nranks; ++q) {
    if (q == st->rank) continue;
    al.in(codes[q], code_bytes(chunk, st->bits));
    al.in(scales[q], chunk / ECHO_GROUP * 4);
  }
}

// Entry pass over chunks [j0, j1) except the own chunk.  The kernel walks
// "virtual" groups that leave the own chunk out: chunk j starts at virtual
// group j*cg before the own chunk and (j-1)*cg after it.
int run_entry_range(const echo_state* st, const uint16_t* x, int32_t j0, int32_t j1,
                    uint8_t* send_codes, float* send_scales, hipStream_t s) {
  const Geometry g = geometry(st);
  const int32_t r = st->rank;
  const uint32_t chunks = (uint32_t)(j1 - j0) - ((j0 <= r && r < j1) ? 1u : 0u);
  Stage1Args a = {};
  a.x = x;
  a.mf = st->m_fast;
  a.ms = st->m_slow;
  a.codes = send_codes;
  a.scales = send_scales;
  a.e2 = nullptr;
  a.groups_work = chunks * g.chunk_groups;
  a.v_base = (uint32_t)(j0 <= r ? j0 : j0 - 1) * g.chunk_groups;
  a.own_g0 = g.own_g0;
  a.own_g1 = g.own_g1;
  return launch_stage1<kEntryFused>(a, st->bits, s);
}

int run_entry(const echo_state* st, const uint16_t* x, uint8_t* send_codes, float* send_scales,
              hipStream_t s) {
  return run_entry_range(st, x, 0, st->nranks, send_codes, send_scales, s);
}

int run_reduce_own(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
                   const float* const* recv_scales, uint8_t* own_codes2, float* own_scales2,
                   uint16_t* y, hipStream_t s) {
  const Geometry g = geometry(st);
  const int64_t e0 = (int64_t)st->rank * g.chunk;
  ReduceArgs a;
  memset(&a, 0, sizeof a);
  for (int q = 0; q < st->nranks; ++q) {
    a.codes[q] = q == st->rank ? nullptr : recv_codes[q];
    a.scales[q] = q == st->rank ? nullptr : recv_scales[q];
  }
  a.out_codes = own_codes2;
  a.out_scales = own_scales2;
  a.y = y + e0;
  a.e2 = nullptr;
  a.x = x + e0;
  a.mf = st->m_fast + e0;
  a.ms = st->m_slow + e0;
  a.groups = g.chunk_groups;
  a.rank = st->rank;
  return launch_reduce<kOwnFused>(st->nranks, a, st->bits, s);
}

int run_exit(const echo_state* st, const uint8_t* const* gath_codes,
             const float* const* gath_scales, uint16_t* y, hipStream_t s) {
  const Geometry g = geometry(st);
  DecodeArgs a;
  memset(&a, 0, sizeof a);
  uint32_t k = 0;
  for (int j = 0; j < st->nranks; ++j) {
    if (j == st->rank) continue;
    a.seg[k].codes = gath_codes[j];
    a.seg[k].scales = gath_scales[j];
    a.seg[k].y = y + (int64_t)j * g.chunk;
    ++k;
  }
  a.groups = g.chunk_groups;
  return launch_decode(a, k, st->bits, s);
}

// ---- the uncompensated call: x' = f32(x), no averages ----------------------

int run_entry_plain(const echo_state* geo, const uint16_t* x, uint8_t* send_codes,
                    float* send_scales, hipStream_t s) {
  const Geometry g = geometry(geo);
  Stage1Args a = {};
  a.x = x;
  a.codes = send_codes;
  a.scales = send_scales;
  a.groups_work = g.groups - g.chunk_groups;
  a.own_g0 = g.own_g0;
  a.own_g1 = g.own_g1;
  return launch_stage1<kEntryPlain>(a, geo->bits, s);
}

int run_reduce_plain(const echo_state* geo, const uint16_t* x, const uint8_t* const* recv_codes,
                     const float* const* recv_scales, uint8_t* own_codes2, float* own_scales2,
                     uint16_t* y, hipStream_t s) {
  const Geometry g = geometry(geo);
  const int64_t e0 = (int64_t)geo->rank * g.chunk;
  ReduceArgs a;
  memset(&a, 0, sizeof a);
  for (int q = 0; q < geo->nranks; ++q) {
    a.codes[q] = q == geo->rank ? nullptr : recv_codes[q];
    a.scales[q] = q == geo->rank ? nullptr : recv_scales[q];
  }
  a.out_codes = own_codes2;
  a.out_scales = own_scales2;
  a.y = y + e0;
  a.x = x + e0;
  a.groups = g.chunk_groups;
  a.rank = geo->rank;
  return launch_reduce<kOwnPlain>(geo->nranks, a, geo->bits, s);
}

// ---- reduce-scatter only -----------------------------------------------------

int run_rs_reduce(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
                  const float* const* recv_scales, uint16_t* y_own, hipStream_t s) {
  const Geometry g = geometry(st);
  const int64_t e0 = (int64_t)st->rank * g.chunk;
  ReduceArgs a;
  memset(&a, 0, sizeof a);
  for (int q = 0; q < st->nranks; ++q) {
    a.codes[q] = q == st->rank ? nullptr : recv_codes[q];
    a.scales[q] = q == st->rank ? nullptr : recv_scales[q];
  }
  a.y = y_own;
  a.x = x + e0;
  a.mf = st->m_fast + e0;
  a.ms = st->m_slow + e0;
  a.groups = g.chunk_groups;
  a.rank = st->rank;
  return launch_reduce<kOwnRS>(st->nranks, a, st->bits, s);
}

int check_rs_reduce(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
                    const float* const* recv_scales, uint16_t* y_own, Aliases& al) {
  if (!x || !y_own) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(y_own, 16)) return ECHO_ERR_ALIGNMENT;
  int rc = check_remote_arrays(st, recv_codes, recv_scales);
  if (rc) return rc;
  const Geometry g = geometry(st);
  al.out(y_own, g.chunk * 2);
  al.in(x, g.n * 2);
  add_remote_inputs(al, st, recv_codes, recv_scales, g.chunk);
  return ECHO_SUCCESS;
}

}  // namespace

extern "C" {

int echo_state_init(echo_state* st, float* m_fast, float* m_slow, int64_t n, int32_t nranks,
                    int32_t rank, echo_stream_t stream) {
  if (!st) return ECHO_ERR_INVALID_ARGUMENT;
  const int shape = check_ranks_shape(n, nranks);
  if (shape < 0) return shape;
  if (rank < 0 || rank >= nranks) return ECHO_ERR_RANKS;
  if (shape != kEmpty) {
    if (!m_fast || !m_slow) return ECHO_ERR_INVALID_ARGUMENT;
    if (!aligned(m_fast, 16) || !aligned(m_slow, 16)) return ECHO_ERR_ALIGNMENT;
  }
  Aliases al;
  al.out(m_fast, n * 4);
  al.out(m_slow, n * 4);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  st->m_fast = m_fast;
  st->m_slow = m_slow;
  st->n = n;
  st->nranks = nranks;
  st->rank = rank;
  st->bits = 4;
  st->reserved = 0;
  if (shape == kEmpty) return ECHO_SUCCESS;
  Zero2Args z;
  z.a = reinterpret_cast<float4*>(m_fast);
  z.b = reinterpret_cast<float4*>(m_slow);
  z.n4 = n / 4;
  return launch(k_zero2, dim3(blocks_for_items((uint64_t)z.n4)), (hipStream_t)stream, z);
}

int echo_encode(const echo_state* st, const uint16_t* x, uint8_t* codes, float* scales,
                echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  if (!x || !codes || !scales) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return ECHO_ERR_ALIGNMENT;
  const int64_t n = st->n;
  Aliases al;
  al.out(codes, code_bytes(n, st->bits));
  al.out(scales, n / ECHO_GROUP * 4);
  al.in(x, n * 2);
  al.in(st->m_fast, n * 4);
  al.in(st->m_slow, n * 4);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  Stage1Args a = {};
  a.x = x;
  a.mf = st->m_fast;
  a.ms = st->m_slow;
  a.codes = codes;
  a.scales = scales;
  a.e2 = nullptr;
  a.groups_work = (uint32_t)(n / ECHO_GROUP);
  a.v_base = 0;
  a.own_g0 = a.own_g1 = 0;
  return launch_stage1<kEncode>(a, st->bits, (hipStream_t)stream);
}

int echo_reduce_shard(int32_t nranks, int64_t chunk_n, int32_t bits,
                      const uint8_t* const* shard_codes, const float* const* shard_scales,
                      uint8_t* out_codes, float* out_scales, uint16_t* out_y, float* out_e2,
                      echo_stream_t stream) {
  if (nranks < 1 || nranks > ECHO_MAX_RANKS) return ECHO_ERR_RANKS;
  if (!bits_ok(bits)) return ECHO_ERR_FORMAT;
  const int shape = check_elements(chunk_n, ECHO_GROUP);
  if (shape) return finished(shape);
  if (!shard_codes || !shard_scales || !out_codes || !out_scales) return ECHO_ERR_INVALID_ARGUMENT;
  for (int q = 0; q < nranks; ++q) {
    if (!shard_codes[q] || !shard_scales[q]) return ECHO_ERR_INVALID_ARGUMENT;
    if (!aligned(shard_codes[q], 16) || !aligned(shard_scales[q], 4)) return ECHO_ERR_ALIGNMENT;
  }
  if (!aligned(out_codes, 16) || !aligned(out_scales, 4) || !aligned(out_y, 16) ||
      !aligned(out_e2, 16))
    return ECHO_ERR_ALIGNMENT;
  Aliases al;
  al.out(out_codes, code_bytes(chunk_n, bits));
  al.out(out_scales, chunk_n / ECHO_GROUP * 4);
  al.out(out_y, chunk_n * 2);
  al.out(out_e2, chunk_n * 4);
  for (int q = 0; q < nranks; ++q) {
    al.in(shard_codes[q], code_bytes(chunk_n, bits));
    al.in(shard_scales[q], chunk_n / ECHO_GROUP * 4);
  }
  if (!al.ok()) return ECHO_ERR_ALIAS;
  ReduceArgs a;
  memset(&a, 0, sizeof a);
  for (int q = 0; q < nranks; ++q) {
    a.codes[q] = shard_codes[q];
    a.scales[q] = shard_scales[q];
  }
  a.out_codes = out_codes;
  a.out_scales = out_scales;
  a.y = out_y;
  a.e2 = out_e2;
  a.groups = (uint32_t)(chunk_n / ECHO_GROUP);
  a.rank = -1;
  return launch_reduce<kShard>(nranks, a, bits, (hipStream_t)stream);
}

int echo_decode(int64_t n, int32_t bits, const uint8_t* codes, const float* scales, uint16_t* y,
                echo_stream_t stream) {
  const int shape = check_elements(n, ECHO_GROUP);
  if (shape < 0) return shape;
  if (!bits_ok(bits)) return ECHO_ERR_FORMAT;
  if (shape == kEmpty) return ECHO_SUCCESS;
  if (!codes || !scales || !y) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(codes, 16) || !aligned(scales, 4) || !aligned(y, 16)) return ECHO_ERR_ALIGNMENT;
  Aliases al;
  al.out(y, n * 2);
  al.in(codes, code_bytes(n, bits));
  al.in(scales, n / ECHO_GROUP * 4);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  DecodeArgs a;
  memset(&a, 0, sizeof a);
  a.seg[0].codes = codes;
  a.seg[0].scales = scales;
  a.seg[0].y = y;
  a.groups = (uint32_t)(n / ECHO_GROUP);
  return launch_decode(a, 1, bits, (hipStream_t)stream);
}

int echo_update(const echo_state* st, const uint16_t* x, const uint8_t* codes1,
                const float* scales1, const float* e2_own, echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  if (!x || !codes1 || !scales1 || !e2_own) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(codes1, 16) || !aligned(scales1, 4) || !aligned(e2_own, 16))
    return ECHO_ERR_ALIGNMENT;
  const Geometry g = geometry(st);
  Aliases al;
  al.out(st->m_fast, g.n * 4);
  al.out(st->m_slow, g.n * 4);
  al.in(x, g.n * 2);
  al.in(codes1, code_bytes(g.n, st->bits));
  al.in(scales1, g.n / ECHO_GROUP * 4);
  al.in(e2_own, g.chunk * 4);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  Stage1Args a = {};
  a.x = x;
  a.mf = st->m_fast;
  a.ms = st->m_slow;
  a.codes = const_cast<uint8_t*>(codes1);
  a.scales = const_cast<float*>(scales1);
  a.e2 = e2_own;
  a.groups_work = g.groups;
  a.v_base = 0;
  a.own_g0 = g.own_g0;
  a.own_g1 = g.own_g1;
  return launch_stage1<kUpdate>(a, st->bits, (hipStream_t)stream);
}

int echo_correction(const echo_state* st, float* corr, echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  if (!corr) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(corr, 16)) return ECHO_ERR_ALIGNMENT;
  Aliases al;
  al.out(corr, st->n * 4);
  al.in(st->m_fast, st->n * 4);
  al.in(st->m_slow, st->n * 4);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  CorrArgs c;
  c.mf = reinterpret_cast<const float4*>(st->m_fast);
  c.ms = reinterpret_cast<const float4*>(st->m_slow);
  c.corr = reinterpret_cast<float4*>(corr);
  c.n4 = st->n / 4;
  return launch(k_correction, dim3(blocks_for_items((uint64_t)c.n4)), (hipStream_t)stream, c);
}

int echo_encode_corr(const echo_state* st, const uint16_t* x, const float* corr, uint8_t* codes,
                     float* scales, echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  if (!x || !corr || !codes || !scales) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(corr, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return ECHO_ERR_ALIGNMENT;
  const int64_t n = st->n;
  Aliases al;
  al.out(codes, code_bytes(n, st->bits));
  al.out(scales, n / ECHO_GROUP * 4);
  al.in(x, n * 2);
  al.in(corr, n * 4);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  Stage1Args a = {};
  a.x = x;
  a.corr = const_cast<float*>(corr);
  a.codes = codes;
  a.scales = scales;
  a.groups_work = (uint32_t)(n / ECHO_GROUP);
  return launch_stage1<kEncodeCorr>(a, st->bits, (hipStream_t)stream);
}

int echo_update_corr(const echo_state* st, const uint16_t* x, const uint8_t* codes1,
                     const float* scales1, const float* e2_own, float* corr, echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  if (!x || !codes1 || !scales1 || !e2_own || !corr) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(codes1, 16) || !aligned(scales1, 4) || !aligned(e2_own, 16) ||
      !aligned(corr, 16))
    return ECHO_ERR_ALIGNMENT;
  const Geometry g = geometry(st);
  Aliases al;
  al.out(st->m_fast, g.n * 4);
  al.out(st->m_slow, g.n * 4);
  al.out(corr, g.n * 4);
  al.in(x, g.n * 2);
  al.in(codes1, code_bytes(g.n, st->bits));
  al.in(scales1, g.n / ECHO_GROUP * 4);
  al.in(e2_own, g.chunk * 4);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  Stage1Args a = {};
  a.x = x;
  a.mf = st->m_fast;
  a.ms = st->m_slow;
  a.corr = corr;
  a.codes = const_cast<uint8_t*>(codes1);
  a.scales = const_cast<float*>(scales1);
  a.e2 = e2_own;
  a.groups_work = g.groups;
  a.own_g0 = g.own_g0;
  a.own_g1 = g.own_g1;
  return launch_stage1<kUpdateCorr>(a, st->bits, (hipStream_t)stream);
}

int echo_call_entry(const echo_state* st, const uint16_t* x, uint8_t* send_codes,
                    float* send_scales, echo_stream_t stream) {
  return echo_call_entry_range(st, x, 0, st ? st->nranks : 0, send_codes, send_scales, stream);
}

int echo_call_entry_range(const echo_state* st, const uint16_t* x, int32_t chunk_begin,
                          int32_t chunk_end, uint8_t* send_codes, float* send_scales,
                          echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  if (chunk_begin < 0 || chunk_end > st->nranks || chunk_begin > chunk_end) return ECHO_ERR_RANKS;
  if (!x || !send_codes || !send_scales) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(send_codes, 16) || !aligned(send_scales, 4))
    return ECHO_ERR_ALIGNMENT;
  const int64_t n = st->n;
  Aliases al;
  al.out(send_codes, code_bytes(n, st->bits));
  al.out(send_scales, n / ECHO_GROUP * 4);
  al.out(st->m_fast, n * 4);
  al.out(st->m_slow, n * 4);
  al.in(x, n * 2);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  return run_entry_range(st, x, chunk_begin, chunk_end, send_codes, send_scales,
                         (hipStream_t)stream);
}

int echo_call_reduce(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
                     const float* const* recv_scales, uint8_t* own_codes2, float* own_scales2,
                     uint16_t* y, echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  if (!x || !own_codes2 || !own_scales2 || !y) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(own_codes2, 16) || !aligned(own_scales2, 4) || !aligned(y, 16))
    return ECHO_ERR_ALIGNMENT;
  rc = check_remote_arrays(st, recv_codes, recv_scales);
  if (rc) return rc;
  const Geometry g = geometry(st);
  Aliases al;
  al.out(own_codes2, code_bytes(g.chunk, st->bits));
  al.out(own_scales2, g.chunk / ECHO_GROUP * 4);
  al.out(y, g.n * 2);
  al.out(st->m_fast, g.n * 4);
  al.out(st->m_slow, g.n * 4);
  al.in(x, g.n * 2);
  add_remote_inputs(al, st, recv_codes, recv_scales, g.chunk);
  al.allow_identical(y, x);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  return run_reduce_own(st, x, recv_codes, recv_scales, own_codes2, own_scales2, y,
                        (hipStream_t)stream);
}

int echo_call_exit(const echo_state* st, const uint8_t* const* gath_codes,
                   const float* const* gath_scales, uint16_t* y, echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  if (!y) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(y, 16)) return ECHO_ERR_ALIGNMENT;
  rc = check_remote_arrays(st, gath_codes, gath_scales);
  if (rc) return rc;
  const Geometry g = geometry(st);
  Aliases al;
  al.out(y, g.n * 2);
  al.out(st->m_fast, g.n * 4);  // not written here, but must stay disjoint from y
  al.out(st->m_slow, g.n * 4);
  add_remote_inputs(al, st, gath_codes, gath_scales, g.chunk);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  return run_exit(st, gath_codes, gath_scales, y, (hipStream_t)stream);
}

int echo_call(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
              const float* const* recv_scales, const uint8_t* const* gath_codes,
              const float* const* gath_scales, uint8_t* send_codes, float* send_scales,
              uint8_t* own_codes2, float* own_scales2, uint16_t* y, echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  if (!x || !send_codes || !send_scales || !own_codes2 || !own_scales2 || !y)
    return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(send_codes, 16) || !aligned(send_scales, 4) ||
      !aligned(own_codes2, 16) || !aligned(own_scales2, 4) || !aligned(y, 16))
    return ECHO_ERR_ALIGNMENT;
  rc = check_remote_arrays(st, recv_codes, recv_scales);
  if (rc) return rc;
  rc = check_remote_arrays(st, gath_codes, gath_scales);
  if (rc) return rc;
  const Geometry g = geometry(st);
  Aliases al;
  al.out(send_codes, code_bytes(g.n, st->bits));
  al.out(send_scales, g.n / ECHO_GROUP * 4);
  al.out(own_codes2, code_bytes(g.chunk, st->bits));
  al.out(own_scales2, g.chunk / ECHO_GROUP * 4);
  al.out(y, g.n * 2);
  al.out(st->m_fast, g.n * 4);
  al.out(st->m_slow, g.n * 4);
  al.in(x, g.n * 2);
  add_remote_inputs(al, st, recv_codes, recv_scales, g.chunk);
  add_remote_inputs(al, st, gath_codes, gath_scales, g.chunk);
  al.allow_identical(y, x);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  rc = run_entry(st, x, send_codes, send_scales, s);
  if (rc) return rc;
  rc = run_reduce_own(st, x, recv_codes, recv_scales, own_codes2, own_scales2, y, s);
  if (rc) return rc;
  return run_exit(st, gath_codes, gath_scales, y, s);
}

int echo_call_plain(int32_t nranks, int32_t rank, int64_t n, int32_t bits, const uint16_t* x,
                    const uint8_t* const* recv_codes, const float* const* recv_scales,
                    const uint8_t* const* gath_codes, const float* const* gath_scales,
                    uint8_t* send_codes, float* send_scales, uint8_t* own_codes2,
                    float* own_scales2, uint16_t* y, echo_stream_t stream) {
  int rc = check_ranks_shape(n, nranks);
  if (rc < 0) return rc;
  if (rank < 0 || rank >= nranks) return ECHO_ERR_RANKS;
  if (!bits_ok(bits)) return ECHO_ERR_FORMAT;
  if (rc == kEmpty) return ECHO_SUCCESS;
  if (!x || !send_codes || !send_scales || !own_codes2 || !own_scales2 || !y)
    return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(x, 16) || !aligned(send_codes, 16) || !aligned(send_scales, 4) ||
      !aligned(own_codes2, 16) || !aligned(own_scales2, 4) || !aligned(y, 16))
    return ECHO_ERR_ALIGNMENT;
  // geometry only: the uncompensated call has no averages
  echo_state geo;
  geo.m_fast = nullptr;
  geo.m_slow = nullptr;
  geo.n = n;
  geo.nranks = nranks;
  geo.rank = rank;
  geo.bits = bits;
  geo.reserved = 0;
  rc = check_remote_arrays(&geo, recv_codes, recv_scales);
  if (rc) return rc;
  rc = check_remote_arrays(&geo, gath_codes, gath_scales);
  if (rc) return rc;
  const Geometry g = geometry(&geo);
  Aliases al;
  al.out(send_codes, code_bytes(g.n, bits));
  al.out(send_scales, g.n / ECHO_GROUP * 4);
  al.out(own_codes2, code_bytes(g.chunk, bits));
  al.out(own_scales2, g.chunk / ECHO_GROUP * 4);
  al.out(y, g.n * 2);
  al.in(x, g.n * 2);
  add_remote_inputs(al, &geo, recv_codes, recv_scales, g.chunk);
  add_remote_inputs(al, &geo, gath_codes, gath_scales, g.chunk);
  al.allow_identical(y, x);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  rc = run_entry_plain(&geo, x, send_codes, send_scales, s);
  if (rc) return rc;
  rc = run_reduce_plain(&geo, x, recv_codes, recv_scales, own_codes2, own_scales2, y, s);
  if (rc) return rc;
  return run_exit(&geo, gath_codes, gath_scales, y, s);
}

int echo_reduce_shard_sum(int32_t nranks, int64_t chunk_n, int32_t bits,
                          const uint8_t* const* shard_codes, const float* const* shard_scales,
                          uint16_t* out_y, float* out_e2, echo_stream_t stream) {
  if (nranks < 1 || nranks > ECHO_MAX_RANKS) return ECHO_ERR_RANKS;
  if (!bits_ok(bits)) return ECHO_ERR_FORMAT;
  const int shape = check_elements(chunk_n, ECHO_GROUP);
  if (shape) return finished(shape);
  if (!shard_codes || !shard_scales || !out_y) return ECHO_ERR_INVALID_ARGUMENT;
  for (int q = 0; q < nranks; ++q) {
    if (!shard_codes[q] || !shard_scales[q]) return ECHO_ERR_INVALID_ARGUMENT;
    if (!aligned(shard_codes[q], 16) || !aligned(shard_scales[q], 4)) return ECHO_ERR_ALIGNMENT;
  }
  if (!aligned(out_y, 16) || !aligned(out_e2, 16)) return ECHO_ERR_ALIGNMENT;
  Aliases al;
  al.out(out_y, chunk_n * 2);
  al.out(out_e2, chunk_n * 4);
  for (int q = 0; q < nranks; ++q) {
    al.in(shard_codes[q], code_bytes(chunk_n, bits));
    al.in(shard_scales[q], chunk_n / ECHO_GROUP * 4);
  }
  if (!al.ok()) return ECHO_ERR_ALIAS;
  ReduceArgs a;
  memset(&a, 0, sizeof a);
  for (int q = 0; q < nranks; ++q) {
    a.codes[q] = shard_codes[q];
    a.scales[q] = shard_scales[q];
  }
  a.y = out_y;
  a.e2 = out_e2;
  a.groups = (uint32_t)(chunk_n / ECHO_GROUP);
  a.rank = -1;
  return launch_reduce<kShardSum>(nranks, a, bits, (hipStream_t)stream);
}

int echo_rs_reduce(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
                   const float* const* recv_scales, uint16_t* y_own, echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  Aliases al;
  rc = check_rs_reduce(st, x, recv_codes, recv_scales, y_own, al);
  if (rc) return rc;
  al.out(st->m_fast, st->n * 4);
  al.out(st->m_slow, st->n * 4);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  return run_rs_reduce(st, x, recv_codes, recv_scales, y_own, (hipStream_t)stream);
}

int echo_rs_call(const echo_state* st, const uint16_t* x, const uint8_t* const* recv_codes,
                 const float* const* recv_scales, uint8_t* send_codes, float* send_scales,
                 uint16_t* y_own, echo_stream_t stream) {
  int rc = check_state(st);
  if (rc) return finished(rc);
  if (!send_codes || !send_scales) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(send_codes, 16) || !aligned(send_scales, 4)) return ECHO_ERR_ALIGNMENT;
  Aliases al;
  rc = check_rs_reduce(st, x, recv_codes, recv_scales, y_own, al);
  if (rc) return rc;
  const int64_t n = st->n;
  al.out(send_codes, code_bytes(n, st->bits));
  al.out(send_scales, n / ECHO_GROUP * 4);
  al.out(st->m_fast, n * 4);
  al.out(st->m_slow, n * 4);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  hipStream_t s = (hipStream_t)stream;
  rc = run_entry(st, x, send_codes, send_scales, s);
  if (rc) return rc;
  return run_rs_reduce(st, x, recv_codes, recv_scales, y_own, s);
}

int echo_get_config(echo_config* out) {
  if (!out) return ECHO_ERR_INVALID_ARGUMENT;
  out->abi_version = ECHO_ABI_VERSION;
  out->group = ECHO_GROUP;
  out->qmax = ECHO_QMAX;
  out->qmax8 = ECHO_QMAX8;
  out->max_ranks = ECHO_MAX_RANKS;
  out->w_fast = ECHO_W_FAST;
  out->w_slow = ECHO_W_SLOW;
  out->beta_fast = ECHO_BETA_FAST;
  out->alpha_fast = ECHO_ALPHA_FAST;
  out->beta_slow = ECHO_BETA_SLOW;
  out->alpha_slow = ECHO_ALPHA_SLOW;
  out->max_elements = ECHO_MAX_ELEMENTS;
  return ECHO_SUCCESS;
}

const char* echo_status_string(int status) {
  switch (status) {
    case ECHO_SUCCESS: return "success";
    case ECHO_ERR_INVALID_ARGUMENT: return "invalid argument (NULL pointer)";
    case ECHO_ERR_SHAPE: return "bad shape (n must be >= 0, a multiple of P*128, within the limit)";
    case ECHO_ERR_ALIGNMENT: return "misaligned pointer (16 bytes for tensors/codes, 4 for scales)";
    case ECHO_ERR_RANKS: return "bad rank count or rank index";
    case ECHO_ERR_HIP: return "HIP runtime error";
    case ECHO_ERR_ALIAS: return "outputs overlap each other or an input";
    case ECHO_ERR_FORMAT: return "code width must be 4 or 8 bits";
    default: return "unknown status";
  }
}

int echo_version(void) { return ECHO_ABI_VERSION; }

int echo_stream_copy(const void* src, void* dst, int64_t bytes, echo_stream_t stream) {
  if (bytes < 0 || bytes % 16 != 0) return ECHO_ERR_SHAPE;
  if (bytes == 0) return ECHO_SUCCESS;
  if (!src || !dst) return ECHO_ERR_INVALID_ARGUMENT;
  if (!aligned(src, 16) || !aligned(dst, 16)) return ECHO_ERR_ALIGNMENT;
  Aliases al;
  al.out(dst, bytes);
  al.in(src, bytes);
  if (!al.ok()) return ECHO_ERR_ALIAS;
  CopyArgs c;
  c.src = reinterpret_cast<const u32x4*>(src);
  c.dst = reinterpret_cast<u32x4*>(dst);
  c.n16 = bytes / 16;
  return launch(k_copy16, dim3(blocks_for_items((uint64_t)c.n16)), (hipStream_t)stream, c);
}

}  // extern "C"
