// echo_device.h -- gfx950 device code of libecho: the Echo rank pipeline
// (arXiv 2610.14277v1; "Tensor-parallel traffic drops to 4 bits", Interpretation, for
// the compensator; "Echo: Error-Compensated 4-Bit Tensor-Parallel Communication", Abstract, for the 4-bit
// transport whose codes are summed in binary32).
//
// Work layout.  Every kernel walks 128-element quantization groups.  The
// stage-1 / reduce kernels give each 64-lane wavefront a "slice" of two
// consecutive groups per step: lane l holds 4 consecutive elements, lanes
// 0-31 form the first group and lanes 32-63 the second, so every global
// access of a wave is one contiguous run (x: 512 B, each average: 1 KiB,
// codes: 128 B) and a group's absmax is a 32-lane reduction done with DPP
// row operations plus one ds_swizzle (no LDS traffic, no barrier).  The exit
// kernel gives each lane 8 elements (a group is 16 lanes) and needs no
// reduction.
//
// Arithmetic.  Built with -ffp-contract=off: each float operation below is
// one IEEE binary32 operation rounded to nearest even, denormals kept;
// x'/s is the correctly rounded division; rint is v_rndne_f32; the bf16
// narrowing is the hardware round-to-nearest-even convert.  The operation
// order is the method's: corr = (W_F*m_f) + (W_S*m_s); x' = f32(x) - corr;
// S = d_0 + d_1 + ... in rank order; m <- (B*m) + (A*r).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "echo.h"
#include "launch_shape.h"

namespace echo {

constexpr int kGroup = ECHO_GROUP;
// code widths: 4 -> packed nibbles, codes in [-7, 7]; 8 -> one two's-
// complement byte per element, codes in [-127, 127] (the 8-bit promotion)
template <int BITS>
__host__ __device__ constexpr float qmax_of() { return BITS == 8 ? (float)ECHO_QMAX8 : (float)ECHO_QMAX; }
constexpr int kMaxRanks = ECHO_MAX_RANKS;

// Cache policy of the streaming accesses: every byte of the averages, the
// input and the messages is touched once per call, so loads and stores of
// the big streams may carry the non-temporal hint.
#ifndef ECHO_NT_LOAD
#define ECHO_NT_LOAD 1
#endif
#ifndef ECHO_NT_STORE
#define ECHO_NT_STORE 1
#endif

// Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8), and each XCD has its own L2.  Renumbering them so that each XCD
// takes one contiguous run of tiles keeps lines shared by neighbouring tiles
// (the per-group scales: 8 bytes per wavefront) inside one L2.
#ifndef ECHO_XCD_REMAP
#define ECHO_XCD_REMAP 1
#endif
constexpr uint32_t kXcds = 8;

__device__ __forceinline__ uint32_t tile_index() {
  const uint32_t b = blockIdx.x;
  if (!ECHO_XCD_REMAP) return b;
  const uint32_t nb = gridDim.x;
  const uint32_t xcd = b % kXcds, k = b / kXcds;
  const uint32_t per = nb / kXcds, extra = nb % kXcds;
  return xcd * per + (xcd < extra ? xcd : extra) + k;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ __forceinline__ T ld_stream(const T* p) {
  if (ECHO_NT_LOAD) return __builtin_nontemporal_load(p);
  return *p;
}

template <typename T>
__device__ __forceinline__ void st_stream(T* p, T v) {
  if (ECHO_NT_STORE) __builtin_nontemporal_store(v, p);
  else *p = v;
}

// ---------------------------------------------------------------------------
// lane-level helpers

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// max over the 32 lanes of each half-wave (all 64 lanes must be active).
// Bit patterns of non-negative floats order like the floats themselves.
__device__ __forceinline__ uint32_t halfwave_max(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]: lane ^ 1
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]: lane ^ 2
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror: quad 0 <-> quad 1
  v = max(v, dpp_u32<0x140>(v));  // row_mirror: half-row 0 <-> half-row 1
  // bitmask swizzle (and 0x1F, or 0, xor 0x10): row 0 <-> row 1 in each 32
  v = max(v, (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F));
  return v;
}

__device__ __forceinline__ uint32_t abs_bits(float v) { return __float_as_uint(v) & 0x7FFFFFFFu; }

// bf16 bits -> binary32 (exact)
__device__ __forceinline__ void unpack_bf16x4(uint2 w, float (&f)[4]) {
  f[0] = __uint_as_float(w.x << 16);
  f[1] = __uint_as_float(w.x & 0xFFFF0000u);
  f[2] = __uint_as_float(w.y << 16);
  f[3] = __uint_as_float(w.y & 0xFFFF0000u);
}

// two binary32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  typedef __bf16 h2 __attribute__((ext_vector_type(2)));
  f2 v = {a, b};
  h2 h = __builtin_convertvector(v, h2);
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// the correction (W_F*m_f) + (W_S*m_s), and x' = f32(x) - correction
__device__ __forceinline__ float correction(float mf, float ms) {
  return (ECHO_W_FAST * mf) + (ECHO_W_SLOW * ms);
}

__device__ __forceinline__ float corrected(float xf, float mf, float ms) {
  float corr = correction(mf, ms);
  return xf - corr;
}

// The group scale from the group's absmax: s = amax / 7 (IEEE division).
template <int BITS>
__device__ __forceinline__ float scale_of(uint32_t amax_bits) {
  return __uint_as_float(amax_bits) / qmax_of<BITS>();
}

// Divisor used for the codes: s itself, or 1 when s == 0.  s == 0 means
// amax <= 3 * 2^-149 (all-zero group, or amax/7 underflowing), where every
// |v| / 1 < 0.5 rounds to code 0 -- the same codes as the zero-group rule.
__device__ __forceinline__ float code_divisor(float s) { return s == 0.0f ? 1.0f : s; }

// code = clamp(rint(v / s), -7, 7), v / s the correctly rounded division.
// (A reciprocal-multiply with an exact fallback near half-integers gives the
// same codes but measured no faster on MI355X: these kernels are not bound
// by the division.)
template <int BITS>
__device__ __forceinline__ int quant_code(float v, float sdiv) {
  float t = __builtin_rintf(v / sdiv);
  t = fminf(fmaxf(t, -qmax_of<BITS>()), qmax_of<BITS>());
  return (int)t;
}

// 4 codes -> 16 bits, element k in bits 4k..4k+3 (two's complement nibbles)
__device__ __forceinline__ uint32_t pack_nib4(const int (&q)[4]) {
  return ((uint32_t)q[0] & 0xFu) | (((uint32_t)q[1] & 0xFu) << 4) |
         (((uint32_t)q[2] & 0xFu) << 8) | (((uint32_t)q[3] & 0xFu) << 12);
}

// nibble k of a packed word -> signed code (sign-extend the 4-bit field)
__device__ __forceinline__ int nib(uint32_t w, int k) {
  return (int)(w << (28 - 4 * k)) >> 28;
}

// code k of a packed word of BITS-wide codes (sign-extended)
template <int BITS>
__device__ __forceinline__ int code_at(uint32_t w, int k) {
  if (BITS == 8) return (int)(w << (24 - 8 * k)) >> 24;
  return nib(w, k);
}

// 4 codes -> one word (16 bits of nibbles, or 32 bits of bytes)
template <int BITS>
__device__ __forceinline__ uint32_t pack_codes4(const int (&q)[4]) {
  if (BITS == 8)
    return ((uint32_t)q[0] & 0xFFu) | (((uint32_t)q[1] & 0xFFu) << 8) |
           (((uint32_t)q[2] & 0xFFu) << 16) | (((uint32_t)q[3] & 0xFFu) << 24);
  return pack_nib4(q);
}

// byte offset of element e's code, and the 4 codes a lane holds
template <int BITS>
__device__ __forceinline__ int64_t code_byte(int64_t e) { return BITS == 8 ? e : e / 2; }

template <int BITS>
__device__ __forceinline__ uint32_t load_codes4(const uint8_t* codes, int64_t e) {
  if (BITS == 8) return *reinterpret_cast<const uint32_t*>(codes + e);
  return *reinterpret_cast<const uint16_t*>(codes + e / 2);
}

template <int BITS>
__device__ __forceinline__ void store_codes4(uint8_t* codes, int64_t e, uint32_t w) {
  if (BITS == 8) st_stream(reinterpret_cast<uint32_t*>(codes + e), w);
  else st_stream(reinterpret_cast<uint16_t*>(codes + e / 2), (uint16_t)w);
}

// m <- (B*m) + (A*r) for both averages
__device__ __forceinline__ void refresh(float& mf, float& ms, float r) {
  mf = (ECHO_BETA_FAST * mf) + (ECHO_ALPHA_FAST * r);
  ms = (ECHO_BETA_SLOW * ms) + (ECHO_ALPHA_SLOW * r);
}

// ---------------------------------------------------------------------------
// stage-1 kernel: entry pass / plain encode / plain update / uncompensated entry

// kEncodeCorr / kUpdateCorr: the deferred-update schedule with the next
// call's correction kept as one array (the entry pass reads it instead of
// both averages; the update writes it after refreshing them)
enum Stage1Mode {
  kEncode = 0, kEntryFused = 1, kUpdate = 2, kEntryPlain = 3, kEncodeCorr = 4, kUpdateCorr = 5
};

// what each stage-1 mode does
constexpr bool skips_own(int m) { return m == kEntryFused || m == kEntryPlain; }
constexpr bool reads_state(int m) { return m != kEntryPlain && m != kEncodeCorr; }
constexpr bool reads_corr(int m) { return m == kEncodeCorr; }
constexpr bool is_update(int m) { return m == kUpdate || m == kUpdateCorr; }
constexpr bool writes_state(int m) { return m == kEntryFused || is_update(m); }
constexpr bool writes_corr(int m) { return m == kUpdateCorr; }

struct Stage1Args {
  const uint16_t* x;      // [n]
  float* mf;              // [n]
  float* ms;              // [n]
  float* corr;            // kEncodeCorr: in [n]; kUpdateCorr: out [n]
  uint8_t* codes;         // encoding modes: out [n/2]; update modes: in
  float* scales;          // encoding modes: out [n/128]; update modes: in
  const float* e2;        // kUpdate: [own chunk], indexed from own_g0*128
  uint32_t groups_work;   // virtual groups to process
  uint32_t v_base;        // first virtual group (the own chunk is not counted
                          // when the mode skips it)
  uint32_t own_g0;        // own chunk, in groups
  uint32_t own_g1;
};

template <int MODE, int BITS, int U>
__global__ __launch_bounds__(kBlock) void k_stage1(Stage1Args a) {
  const int lane = threadIdx.x & 63;
  const uint32_t half = (uint32_t)lane >> 5;
  const uint32_t sub = (uint32_t)lane & 31u;
  const uint32_t wave = tile_index() * (kBlock / 64) + (threadIdx.x >> 6);
  const uint32_t nwaves = gridDim.x * (kBlock / 64);
  const uint32_t nslices = (a.groups_work + 1u) >> 1;
  const uint32_t own_len = a.own_g1 - a.own_g0;

  for (uint32_t s0 = wave * U; s0 < nslices; s0 += nwaves * U) {
    float xf[U][4], mf[U][4], ms[U][4];
    uint32_t g[U];
    bool ok[U];
    uint32_t cw[U];
    float sc[U];
    float e2v[U][4];
    bool own[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      uint32_t v = 2u * (s0 + u) + half;
      ok[u] = (s0 + u < nslices) && (v < a.groups_work);
      uint32_t gg = a.v_base + v;
      if (skips_own(MODE)) gg = gg < a.own_g0 ? gg : gg + own_len;
      g[u] = ok[u] ? gg : 0u;
      const int64_t e = (int64_t)g[u] * kGroup + sub * 4;
      uint2 xw = make_uint2(0u, 0u);
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f), s = make_float4(0.f, 0.f, 0.f, 0.f);
      cw[u] = 0u;
      sc[u] = 0.f;
      e2v[u][0] = e2v[u][1] = e2v[u][2] = e2v[u][3] = 0.f;
      own[u] = ok[u] && g[u] >= a.own_g0 && g[u] < a.own_g1;
      if (ok[u]) {
        const u32x2 xv = ld_stream(reinterpret_cast<const u32x2*>(a.x + e));
        xw = make_uint2(xv.x, xv.y);
        if (reads_state(MODE)) {
          const f32x4 fv = ld_stream(reinterpret_cast<const f32x4*>(a.mf + e));
          const f32x4 sv = ld_stream(reinterpret_cast<const f32x4*>(a.ms + e));
          f = make_float4(fv.x, fv.y, fv.z, fv.w);
          s = make_float4(sv.x, sv.y, sv.z, sv.w);
        }
        if (reads_corr(MODE)) {  // the correction, held where m_f would be
          const f32x4 cv = ld_stream(reinterpret_cast<const f32x4*>(a.corr + e));
          f = make_float4(cv.x, cv.y, cv.z, cv.w);
        }
        if (is_update(MODE)) {
          cw[u] = load_codes4<BITS>(a.codes, e);
          sc[u] = a.scales[g[u]];
          if (own[u]) {
            float4 t = *reinterpret_cast<const float4*>(a.e2 + (e - (int64_t)a.own_g0 * kGroup));
            e2v[u][0] = t.x; e2v[u][1] = t.y; e2v[u][2] = t.z; e2v[u][3] = t.w;
          }
        }
      }
      unpack_bf16x4(xw, xf[u]);
      mf[u][0] = f.x; mf[u][1] = f.y; mf[u][2] = f.z; mf[u][3] = f.w;
      ms[u][0] = s.x; ms[u][1] = s.y; ms[u][2] = s.z; ms[u][3] = s.w;
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      float xp[4];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        xp[k] = reads_state(MODE)  ? corrected(xf[u][k], mf[u][k], ms[u][k])
                : reads_corr(MODE) ? xf[u][k] - mf[u][k]
                                   : xf[u][k];

      float d1[4];
      if (is_update(MODE)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) d1[k] = (float)code_at<BITS>(cw[u], k) * sc[u];
      } else {
        uint32_t m = max(max(abs_bits(xp[0]), abs_bits(xp[1])), max(abs_bits(xp[2]), abs_bits(xp[3])));
        m = halfwave_max(m);
        const float s = scale_of<BITS>(m);
        const float sd = code_divisor(s);
        int q[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) q[k] = quant_code<BITS>(xp[k], sd);
        const int64_t e = (int64_t)g[u] * kGroup + sub * 4;
        if (ok[u]) {
          store_codes4<BITS>(a.codes, e, pack_codes4<BITS>(q));
          if (sub == 0) a.scales[g[u]] = s;
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) d1[k] = (float)q[k] * s;
      }

      if (writes_state(MODE)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          float r = d1[k] - xp[k];
          if (is_update(MODE) && own[u]) r = r + e2v[u][k];  // e2 only on the own chunk
          refresh(mf[u][k], ms[u][k], r);
        }
        if (ok[u]) {
          const int64_t e = (int64_t)g[u] * kGroup + sub * 4;
          st_stream(reinterpret_cast<f32x4*>(a.mf + e), f32x4{mf[u][0], mf[u][1], mf[u][2], mf[u][3]});
          st_stream(reinterpret_cast<f32x4*>(a.ms + e), f32x4{ms[u][0], ms[u][1], ms[u][2], ms[u][3]});
          if (writes_corr(MODE))  // the next call's correction, from the refreshed averages
            st_stream(reinterpret_cast<f32x4*>(a.corr + e),
                      f32x4{correction(mf[u][0], ms[u][0]), correction(mf[u][1], ms[u][1]),
                            correction(mf[u][2], ms[u][2]), correction(mf[u][3], ms[u][3])});
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// reduce kernel: rank-order sum of P stage-1 shards of one chunk, requantize

// kShard / kOwnFused / kOwnPlain: all-reduce (the sum is requantized);
// kShardSum / kOwnRS: reduce-scatter only (the sum is the bf16 output).
enum ReduceMode { kShard = 0, kOwnFused = 1, kOwnPlain = 2, kShardSum = 3, kOwnRS = 4 };

// the own slot is quantized in registers from x (with or without the averages)
constexpr bool own_in_registers(int m) { return m == kOwnFused || m == kOwnPlain || m == kOwnRS; }
constexpr bool own_reads_state(int m) { return m == kOwnFused || m == kOwnRS; }
constexpr bool requantizes(int m) { return m == kShard || m == kOwnFused || m == kOwnPlain; }
constexpr bool stores_e2(int m) { return m == kShard || m == kShardSum; }

struct ReduceArgs {
  const uint8_t* codes[kMaxRanks];   // shard q codes, chunk-local
  const float* scales[kMaxRanks];    // shard q scales, chunk-local
  uint8_t* out_codes;                // [chunk/2] (requantizing modes)
  float* out_scales;                 // [chunk/128] (requantizing modes)
  uint16_t* y;                       // [chunk] (nullable in kShard / kShardSum)
  float* e2;                         // [chunk] (kShard / kShardSum, nullable)
  const uint16_t* x;                 // own modes: own chunk of x
  float* mf;                         // kOwnFused / kOwnRS: own chunk of the averages
  float* ms;
  uint32_t groups;                   // groups in the chunk
  int32_t rank;                      // own modes: the slot computed in registers
};

template <int MODE, int BITS, int P, int U>
__global__ __launch_bounds__(kBlock) void k_reduce(ReduceArgs a) {
  const int lane = threadIdx.x & 63;
  const uint32_t half = (uint32_t)lane >> 5;
  const uint32_t sub = (uint32_t)lane & 31u;
  const uint32_t wave = tile_index() * (kBlock / 64) + (threadIdx.x >> 6);
  const uint32_t nwaves = gridDim.x * (kBlock / 64);
  const uint32_t nslices = (a.groups + 1u) >> 1;

  for (uint32_t s0 = wave * U; s0 < nslices; s0 += nwaves * U) {
    // The arguments are read through a kernarg-segment pointer made opaque
    // inside each step, so their loads stay in the step instead of being
    // hoisted out of the loop and held in scalar registers across it: with
    // 2P shard pointers live beside the rest, P >= 14 spilled scalar
    // registers into vector lanes (P = 16: 21 spilled, occupancy 5).  A wave
    // runs one step at full grid, so each argument is still loaded once.
    uint64_t kp = (uint64_t)__builtin_amdgcn_kernarg_segment_ptr();
    asm volatile("" : "+s"(kp));
    const __attribute__((address_space(4))) ReduceArgs* ar =
        (const __attribute__((address_space(4))) ReduceArgs*)kp;
    // The own slot's index, opaque to the optimizer inside each step: left
    // loop-invariant, its P comparisons are hoisted out of the loop and held
    // as P live lane masks, which for large P spill the scalar registers.
    int32_t own = ar->rank;
    asm volatile("" : "+s"(own));
    // issue every load of the U slices first
    bool ok[U];
    uint32_t g[U];
    uint32_t cw[U][P];
    float sc[U][P];
    float xf[U][4], mf[U][4], ms[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t v = 2u * (s0 + u) + half;
      ok[u] = (s0 + u < nslices) && (v < a.groups);
      g[u] = ok[u] ? v : 0u;
      const int64_t e = (int64_t)g[u] * kGroup + sub * 4;
      // A lane past the end reads group 0 (always present) and stores
      // nothing, so the loads need no per-lane guard.  Only the own-slot test
      // remains, and it is uniform: with a lane-varying guard per shard the
      // compiler keeps one exec mask per shard, which for P > 9 no longer
      // fits the scalar registers and spills into vector lanes.
#pragma unroll
      for (int q = 0; q < P; ++q) {
        cw[u][q] = 0u;
        sc[u][q] = 0.f;
        if (!(own_in_registers(MODE) && q == own)) {
          cw[u][q] = load_codes4<BITS>(ar->codes[q], e);
          sc[u][q] = ar->scales[q][g[u]];
        }
      }
      uint2 xw = make_uint2(0u, 0u);
      float4 f = make_float4(0.f, 0.f, 0.f, 0.f), s = make_float4(0.f, 0.f, 0.f, 0.f);
      if (own_in_registers(MODE)) {
        const u32x2 xv = ld_stream(reinterpret_cast<const u32x2*>(ar->x + e));
        xw = make_uint2(xv.x, xv.y);
        if (own_reads_state(MODE)) {
          const f32x4 fv = ld_stream(reinterpret_cast<const f32x4*>(ar->mf + e));
          const f32x4 sv = ld_stream(reinterpret_cast<const f32x4*>(ar->ms + e));
          f = make_float4(fv.x, fv.y, fv.z, fv.w);
          s = make_float4(sv.x, sv.y, sv.z, sv.w);
        }
      }
      unpack_bf16x4(xw, xf[u]);
      mf[u][0] = f.x; mf[u][1] = f.y; mf[u][2] = f.z; mf[u][3] = f.w;
      ms[u][0] = s.x; ms[u][1] = s.y; ms[u][2] = s.z; ms[u][3] = s.w;
    }

#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t e = (int64_t)g[u] * kGroup + sub * 4;
      // own stage-1 quantization, in registers (same helpers as the entry pass)
      float xp[4] = {0.f, 0.f, 0.f, 0.f}, d_own[4] = {0.f, 0.f, 0.f, 0.f};
      if (own_in_registers(MODE)) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          xp[k] = own_reads_state(MODE) ? corrected(xf[u][k], mf[u][k], ms[u][k]) : xf[u][k];
        uint32_t m = max(max(abs_bits(xp[0]), abs_bits(xp[1])), max(abs_bits(xp[2]), abs_bits(xp[3])));
        m = halfwave_max(m);
        const float s1 = scale_of<BITS>(m);
        const float sd = code_divisor(s1);
        int q1[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          q1[k] = quant_code<BITS>(xp[k], sd);
          d_own[k] = (float)q1[k] * s1;
        }
        // the own slot holds the codes and scale it would have received, so
        // the sum below decodes every slot alike (code * scale is d_own)
        int32_t slot = own;
        asm volatile("" : "+s"(slot));
        const uint32_t own_word = pack_codes4<BITS>(q1);
#pragma unroll
        for (int q = 0; q < P; ++q) {
          if (q == slot) {
            cw[u][q] = own_word;
            sc[u][q] = s1;
          }
        }
      }

      // S = d_0 + d_1 + ... + d_{P-1}, in rank order
      float S[4];
#pragma unroll
      for (int q = 0; q < P; ++q) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float d = (float)code_at<BITS>(cw[u][q], k) * sc[u][q];
          S[k] = (q == 0) ? d : S[k] + d;
        }
      }

      // all-reduce: requantize the sum (stage 2), y = bf16(code2 * s2);
      // reduce-scatter: the sum itself is the output, y = bf16(S)
      int q2[4] = {0, 0, 0, 0};
      float s2 = 0.f;
      uint32_t y01, y23;
      if (requantizes(MODE)) {
        uint32_t m2 = max(max(abs_bits(S[0]), abs_bits(S[1])), max(abs_bits(S[2]), abs_bits(S[3])));
        m2 = halfwave_max(m2);
        s2 = scale_of<BITS>(m2);
        const float sd2 = code_divisor(s2);
#pragma unroll
        for (int k = 0; k < 4; ++k) q2[k] = quant_code<BITS>(S[k], sd2);
        y01 = pack_bf16x2((float)q2[0] * s2, (float)q2[1] * s2);
        y23 = pack_bf16x2((float)q2[2] * s2, (float)q2[3] * s2);
      } else {
        y01 = pack_bf16x2(S[0], S[1]);
        y23 = pack_bf16x2(S[2], S[3]);
      }
      float e2[4];
      e2[0] = bf16_lo(y01) - S[0];
      e2[1] = bf16_hi(y01) - S[1];
      e2[2] = bf16_lo(y23) - S[2];
      e2[3] = bf16_hi(y23) - S[3];

      if (ok[u]) {
        if (requantizes(MODE)) {
          store_codes4<BITS>(ar->out_codes, e, pack_codes4<BITS>(q2));
          if (sub == 0) ar->out_scales[g[u]] = s2;
        }
        if (ar->y) st_stream(reinterpret_cast<u32x2*>(ar->y + e), u32x2{y01, y23});
        if (stores_e2(MODE) && ar->e2)
          *reinterpret_cast<float4*>(ar->e2 + e) = make_float4(e2[0], e2[1], e2[2], e2[3]);
      }
      if (own_reads_state(MODE)) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const float e1 = d_own[k] - xp[k];
          refresh(mf[u][k], ms[u][k], e1 + e2[k]);
        }
        if (ok[u]) {
          st_stream(reinterpret_cast<f32x4*>(ar->mf + e), f32x4{mf[u][0], mf[u][1], mf[u][2], mf[u][3]});
          st_stream(reinterpret_cast<f32x4*>(ar->ms + e), f32x4{ms[u][0], ms[u][1], ms[u][2], ms[u][3]});
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// exit kernel: y = bf16(code * scale); blockIdx.y selects a segment

struct DecodeSeg {
  const uint8_t* codes;  // [groups*128*BITS/8]
  const float* scales;   // [groups]
  uint16_t* y;           // [groups*128]
};

struct DecodeArgs {
  DecodeSeg seg[kMaxRanks];
  uint32_t groups;  // groups per segment
};

template <int BITS, int U>
__global__ __launch_bounds__(kBlock) void k_decode(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const uint32_t row = (uint32_t)lane >> 4;  // group within the wave's quad of groups
  const uint32_t sub = (uint32_t)lane & 15u; // 8 elements each
  const uint32_t wave = blockIdx.x * (kBlock / 64) + (threadIdx.x >> 6);  // measured: the exit
  // pass streams faster without the XCD renumbering
  const uint32_t nwaves = gridDim.x * (kBlock / 64);
  const uint32_t nquads = (a.groups + 3u) >> 2;
  const DecodeSeg sg = a.seg[blockIdx.y];

  for (uint32_t t0 = wave * U; t0 < nquads; t0 += nwaves * U) {
    uint32_t cw[U][2];  // 8 codes: one word of nibbles, or two words of bytes
    float sc[U];
    bool ok[U];
    uint32_t g[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t v = 4u * (t0 + u) + row;
      ok[u] = (t0 + u < nquads) && (v < a.groups);
      g[u] = ok[u] ? v : 0u;
      cw[u][0] = cw[u][1] = 0u;
      sc[u] = 0.f;
      if (ok[u]) {
        const int64_t e = (int64_t)g[u] * kGroup + sub * 8;
        if (BITS == 8) {
          const u32x2 w = *reinterpret_cast<const u32x2*>(sg.codes + e);
          cw[u][0] = w.x;
          cw[u][1] = w.y;
        } else {
          cw[u][0] = *reinterpret_cast<const uint32_t*>(sg.codes + e / 2);
        }
        sc[u] = sg.scales[g[u]];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      int c[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        c[k] = BITS == 8 ? code_at<8>(cw[u][k / 4], k % 4) : nib(cw[u][0], k);
      uint4 o;
      o.x = pack_bf16x2((float)c[0] * sc[u], (float)c[1] * sc[u]);
      o.y = pack_bf16x2((float)c[2] * sc[u], (float)c[3] * sc[u]);
      o.z = pack_bf16x2((float)c[4] * sc[u], (float)c[5] * sc[u]);
      o.w = pack_bf16x2((float)c[6] * sc[u], (float)c[7] * sc[u]);
      if (ok[u])
        st_stream(reinterpret_cast<u32x4*>(sg.y + (int64_t)g[u] * kGroup + sub * 8), u32x4{o.x, o.y, o.z, o.w});
    }
  }
}

// ---------------------------------------------------------------------------
// zero fill (the averages start at zero); a kernel rather than a memset so
// the call can sit inside a captured graph

struct Zero2Args {
  float4* a;
  float4* b;
  int64_t n4;  // float4s in each
};

__global__ __launch_bounds__(kBlock) void k_zero2(Zero2Args z) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < z.n4; i += stride) {
    z.a[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    z.b[i] = make_float4(0.f, 0.f, 0.f, 0.f);
  }
}

// corr = (W_F*m_f) + (W_S*m_s) from the current averages (set-up of the
// deferred-update schedule's correction array)
struct CorrArgs {
  const float4* mf;
  const float4* ms;
  float4* corr;
  int64_t n4;  // float4s
};

__global__ __launch_bounds__(kBlock) void k_correction(CorrArgs c) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < c.n4; i += stride) {
    const float4 f = c.mf[i], s = c.ms[i];
    c.corr[i] = make_float4(correction(f.x, s.x), correction(f.y, s.y), correction(f.z, s.z),
                            correction(f.w, s.w));
  }
}

// a plain streaming copy, 16 bytes per lane (the practical bandwidth ceiling)
struct CopyArgs {
  const u32x4* src;
  u32x4* dst;
  int64_t n16;  // 16-byte vectors
};

__global__ __launch_bounds__(kBlock) void k_copy16(CopyArgs c) {
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < c.n16; i += stride)
    st_stream(c.dst + i, ld_stream(c.src + i));
}

}  // namespace echo
