// Device-side helpers shared by the CSA / HCA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace csa {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (inputs are finite; NaN stays NaN).
// fp32 -> bf16, round to nearest even (gfx950 converts in hardware:
// v_cvt_pk_bf16_f32)
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, v);
}

// Entries visible to a query at position q_pos for pooling factor m >= 1:
// entry j is visible iff m*(j+1) <= q_pos+1, capped by the valid rows.
// q_pos + 1 is at most 2^31, so an unsigned 32-bit quotient is exact (a
// 64-bit division would put a long dependent sequence in front of every
// kernel's first loads); no branch either, so that a kernel's scalar loads
// stay in one block and go out together.  q_pos < 0: max(q_pos, -1) + 1 = 0.
__device__ __forceinline__ int visible_count(int q_pos, int m, int n_entries, int n_max) {
  const unsigned v = (static_cast<unsigned>(max(q_pos, -1)) + 1u) / static_cast<unsigned>(m);
  const int cap = max(min(n_entries, n_max), 0);
  return v < static_cast<unsigned>(cap) ? static_cast<int>(v) : cap;
}

// Selection bound shared by the score and top-k kernels: every chunk of
// kBoundChunk keys reports its c-th largest score, c being the smallest value
// with floor(V / kBoundChunk) * c >= k for a row with V visible entries.  Any
// value reached by ceil(k / c) of the reports is then at most the row's k-th
// largest score (the minimum of the full chunks' reports always is).  Where
// that c is 1 but k is more than half the full chunks, c = 2 instead (also
// valid): the ceil(k / 2)-th largest of the chunks' second largest scores sits
// far closer to the k-th largest than the minimum of (almost) every chunk's
// largest, so far fewer entries survive the bound.
// Returns 0 (no bound) when c would exceed kMaxBoundC.
constexpr int kBoundChunk = 256;
constexpr int kMaxBoundC = 16;
__device__ __forceinline__ int bound_c_row(int V, int k) {
  const int full = V / kBoundChunk;
  if (full == 0 || k <= 0) return 0;
  int c = (k + full - 1) / full;
  if (c == 1 && 2 * k > full) c = 2;
  return c <= kMaxBoundC ? c : 0;
}

// Score storage: fp32, or bf16 for the 16-bit score path (round to nearest,
// ties to even; +-inf stay infinite, scores are never NaN).  Rounding is
// monotone, so the c-th largest of the rounded scores is the rounded c-th
// largest and a chunk report rounds like the scores it summarises.
__device__ __forceinline__ uint16_t bf16_rne_bits(float x) {
  const uint32_t u = __float_as_uint(x);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}
__device__ __forceinline__ float bf16_round(float x) {
  return __uint_as_float(static_cast<uint32_t>(bf16_rne_bits(x)) << 16);
}
__device__ __forceinline__ void put_score(float* p, float v) { *p = v; }
__device__ __forceinline__ void put_score(uint16_t* p, float v) { *p = bf16_rne_bits(v); }
__device__ __forceinline__ float get_score(const float* p) { return *p; }
__device__ __forceinline__ float get_score(const uint16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}
template <typename S>
__device__ __forceinline__ float2 stored_report(float2 r) {
  return sizeof(S) == 2 ? make_float2(bf16_round(r.x), bf16_round(r.y)) : r;
}

// max(x, 0) as one integer max on the bit pattern: negative values (sign bit
// set, so negative as integers) and -0.0 become +0.0, the rest pass through.
// A float max would first canonicalise x, costing a second instruction.
__device__ __forceinline__ float relu_f32(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// MX FP4 (OCP Microscaling) shared exponent of a 32-element block from its
// largest magnitude: floor(log2(amax)) - 2 (2 = the largest E2M1 exponent),
// clamped to [-127, 127], -127 for an all-zero block.  floor(log2) from the
// bit pattern, subnormals included.
__device__ __forceinline__ int mx_block_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  const uint32_t u = __float_as_uint(amax);
  const int ef = static_cast<int>(u >> 23);
  const int fl = ef != 0 ? ef - 127 : (31 - __builtin_clz(u & 0x7fffffu)) - 149;
  return max(-127, min(127, fl - 2));
}

// Two values to E2M1 codes in byte `sel` of w, x / 2^e rounded to the nearest
// E2M1 value (ties to even, saturating at 6, x's sign): gfx950's scaled FP4
// conversion with scale 2^e.  2^-127 is no normal float, so e = -127 (values
// below 2^-125) is handled as (x 2^126) / 2^-1, which is exact.
template <int SEL>
__device__ __forceinline__ uint32_t mx_cvt_pair(uint32_t w, float a, float b, int e) {
  if (e > -127)
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(
        w, a, b, __uint_as_float(static_cast<uint32_t>(e + 127) << 23), SEL);
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, a * 0x1p126f, b * 0x1p126f, 0.5f, SEL);
}

// ---- wave64 reductions and scans -------------------------------------------
// The device library's DPP implementations (row shifts and broadcasts, no LDS
// round trips).  Each uses a fixed combination order, so results are
// deterministic.  All 64 lanes must be active.
extern "C" __device__ float __ockl_wfred_max_f32(float);
extern "C" __device__ float __ockl_wfred_min_f32(float);
extern "C" __device__ float __ockl_wfred_add_f32(float);
extern "C" __device__ uint32_t __ockl_wfred_add_u32(uint32_t);
extern "C" __device__ uint32_t __ockl_wfscan_add_u32(uint32_t, bool);

__device__ __forceinline__ float wave_max(float v) { return __ockl_wfred_max_f32(v); }
__device__ __forceinline__ float wave_min(float v) { return __ockl_wfred_min_f32(v); }
__device__ __forceinline__ float wave_sum(float v) { return __ockl_wfred_add_f32(v); }
extern "C" __device__ int32_t __ockl_wfred_max_i32(int32_t);
__device__ __forceinline__ int wave_max_int(int v) { return __ockl_wfred_max_i32(v); }
extern "C" __device__ uint32_t __ockl_wfred_min_u32(uint32_t);
extern "C" __device__ uint32_t __ockl_wfred_max_u32(uint32_t);
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) { return __ockl_wfred_min_u32(v); }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) { return __ockl_wfred_max_u32(v); }
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) { return __ockl_wfred_add_u32(v); }
__device__ __forceinline__ int wave_sum_int(int v) {
  return static_cast<int>(__ockl_wfred_add_u32(static_cast<uint32_t>(v)));
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ uint32_t wave_incl_scan_u32(uint32_t v) {
  return __ockl_wfscan_add_u32(v, true);
}

// 16-byte vector load / store helpers
__device__ __forceinline__ uint4 ld16(const void* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ void st16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }
__device__ __forceinline__ bf16x8_t ld_bf16x8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8_t*>(p);
}
// 16-byte load marked non-temporal: streamed data that is read once
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4_t ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
}

}  // namespace csa
