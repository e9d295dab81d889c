// MX FP4 encoding of indexer vectors: E2M1 codes with one E8M0 scale byte
// per 32 elements, the input format of the block-scaled indexer path
// ("DeepSeek V4 技术解读", §5: the indexer QK path runs in FP4; with
// power-of-two block scales the FP4 -> FP8 widening the pages describe is
// exact).  The encoding is the OCP Microscaling one:
//   e = floor(log2(amax)) - 2 (2 = the largest E2M1 exponent), clamped to
//   [-127, 127], -127 for an all-zero block; scale byte e + 127;
//   code = nearest E2M1 magnitude of |x| / 2^e, a tie to the code with an
//   even mantissa bit, saturating at 6; the sign bit is x's own.
// One thread per 32-element block: it reads the block's 64 or 128 bytes with
// 16-byte loads, writes its 16 bytes of codes (element 2i in the low nibble
// of byte i) and its scale byte.  HBM-streaming; no cross-lane work.
#include "device_common.h"
#include "internal.h"

namespace csa {
namespace {

constexpr int kQuantThreads = 256;

template <typename T>
__device__ __forceinline__ void load_block(const T* p, float (&v)[32]);
template <>
__device__ __forceinline__ void load_block<float>(const float* p, float (&v)[32]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint4 u = ld16(p + 4 * i);
    v[4 * i] = __uint_as_float(u.x);
    v[4 * i + 1] = __uint_as_float(u.y);
    v[4 * i + 2] = __uint_as_float(u.z);
    v[4 * i + 3] = __uint_as_float(u.w);
  }
}
template <>
__device__ __forceinline__ void load_block<uint16_t>(const uint16_t* p, float (&v)[32]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = ld16(p + 8 * i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      v[8 * i + 2 * h] = __uint_as_float(w[h] << 16);
      v[8 * i + 2 * h + 1] = __uint_as_float(w[h] & 0xffff0000u);
    }
  }
}

// floor(log2(a)) for a finite a > 0, from the bit pattern (subnormals too)
__device__ __forceinline__ int floor_log2(float a) {
  const uint32_t u = __float_as_uint(a);
  const int ef = static_cast<int>(u >> 23);
  if (ef != 0) return ef - 127;
  return (31 - __builtin_clz(u & 0x7fffffu)) - 149;
}

// E2M1 magnitude index of y >= 0: '>' where a tie belongs to the lower code
// (even mantissa bit), '>=' where it belongs to the upper one
__device__ __forceinline__ uint32_t e2m1_mag(float y) {
  return static_cast<uint32_t>(y > 0.25f) + static_cast<uint32_t>(y >= 0.75f) +
         static_cast<uint32_t>(y > 1.25f) + static_cast<uint32_t>(y >= 1.75f) +
         static_cast<uint32_t>(y > 2.5f) + static_cast<uint32_t>(y >= 3.5f) +
         static_cast<uint32_t>(y > 5.0f);
}

template <typename T>
__global__ __launch_bounds__(kQuantThreads) void quantize_mx4_kernel(
    const T* __restrict__ x, int64_t x_rs, int rows, int nblk, uint8_t* __restrict__ codes,
    int64_t c_rs, uint8_t* __restrict__ scales, int64_t s_rs) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kQuantThreads + threadIdx.x;
  if (gid >= static_cast<int64_t>(rows) * nblk) return;
  const int64_t r = gid / nblk;
  const int blk = static_cast<int>(gid - r * nblk);
  float v[32];
  load_block<T>(x + r * x_rs + 32 * blk, v);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  int e = amax > 0.f ? floor_log2(amax) - 2 : -127;
  e = max(-127, min(127, e));
  // 2^-e as a normal float: e <= 125 for any finite amax, so 127 - e >= 2
  const float inv = __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
  uint32_t word[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t wv = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float xi = v[8 * q + i];
      const uint32_t code = e2m1_mag(fabsf(xi) * inv) | ((__float_as_uint(xi) >> 31) << 3);
      wv |= code << (4 * i);
    }
    word[q] = wv;
  }
  st16(codes + r * c_rs + 16 * blk, make_uint4(word[0], word[1], word[2], word[3]));
  scales[r * s_rs + blk] = static_cast<uint8_t>(e + 127);
}

}  // namespace

hipError_t launch_quantize_mx4(const void* x, int64_t x_rs, csa_dtype_t dt, int rows, int D,
                               uint8_t* codes, int64_t c_rs, uint8_t* scales, int64_t s_rs,
                               hipStream_t s) {
  const int nblk = D / 32;
  const int64_t total = static_cast<int64_t>(rows) * nblk;
  const dim3 grid(static_cast<unsigned>((total + kQuantThreads - 1) / kQuantThreads));
  if (dt == CSA_F32)
    hipLaunchKernelGGL(quantize_mx4_kernel<float>, grid, dim3(kQuantThreads), 0, s,
                       static_cast<const float*>(x), x_rs, rows, nblk, codes, c_rs, scales, s_rs);
  else
    hipLaunchKernelGGL(quantize_mx4_kernel<uint16_t>, grid, dim3(kQuantThreads), 0, s,
                       static_cast<const uint16_t*>(x), x_rs, rows, nblk, codes, c_rs, scales,
                       s_rs);
  return hipGetLastError();
}

}  // namespace csa
