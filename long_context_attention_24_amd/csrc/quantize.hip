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
// of byte i) and its scale byte.  The rounding is gfx950's scaled FP4
// conversion (v_cvt_scalef32_pk_fp4_{f32,bf16}), which takes x / scale to
// the nearest E2M1 value with ties to even, saturates at 6 and keeps x's
// sign; given scale 2^e it is the rule above, which the parity tests check
// bit for bit.  2^-127 is not a normal float, so a block with e = -127 is
// first multiplied by 2^126 (exact: its values are below 2^-125) and
// converted with scale 2^-1.
#include "device_common.h"
#include "internal.h"

namespace csa {
namespace {

constexpr int kQuantThreads = 256;

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

using csa::mx_block_exponent;

// Packs element pairs (2i, 2i+1), i = 4d..4d+3, into code word d; pair i
// comes from cvt(i, sel) with sel = i % 4 naming the byte it fills.
#define CSA_PACK4(d, CVT)                                              \
  {                                                                    \
    uint32_t w_ = 0;                                                   \
    w_ = CVT(w_, 4 * (d) + 0, 0);                                      \
    w_ = CVT(w_, 4 * (d) + 1, 1);                                      \
    w_ = CVT(w_, 4 * (d) + 2, 2);                                      \
    w_ = CVT(w_, 4 * (d) + 3, 3);                                      \
    word[d] = w_;                                                      \
  }

// 32 fp32 values as 8 uint4 loads u[0..7]: element j is component j % 4 of u[j / 4]
__device__ __forceinline__ float f32_elem(const uint4 (&u)[8], int j) {
  const uint4 q = u[j / 4];
  const uint32_t c = (j % 4 == 0) ? q.x : (j % 4 == 1) ? q.y : (j % 4 == 2) ? q.z : q.w;
  return __uint_as_float(c);
}
// 32 bf16 values as 4 uint4 loads: element pair i is 32-bit word i % 4 of u[i / 4]
__device__ __forceinline__ uint32_t bf16_pair(const uint4 (&u)[4], int i) {
  const uint4 q = u[i / 4];
  return (i % 4 == 0) ? q.x : (i % 4 == 1) ? q.y : (i % 4 == 2) ? q.z : q.w;
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ void encode_block(const float* __restrict__ p, int& e, uint32_t (&word)[4]) {
  uint4 u[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) u[i] = ld16(p + 4 * i);
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(f32_elem(u, j)));
  e = mx_block_exponent(amax);
  if (e > -127) {
    const float sc = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
#define CSA_CVT(w, i, sel) \
  __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f32_elem(u, 2 * (i)), f32_elem(u, 2 * (i) + 1), sc, sel)
#pragma unroll
    for (int d = 0; d < 4; ++d) CSA_PACK4(d, CSA_CVT)
#undef CSA_CVT
  } else {
#define CSA_CVT(w, i, sel)                                                           \
  __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, f32_elem(u, 2 * (i)) * 0x1p126f,       \
                                           f32_elem(u, 2 * (i) + 1) * 0x1p126f, 0.5f, sel)
#pragma unroll
    for (int d = 0; d < 4; ++d) CSA_PACK4(d, CSA_CVT)
#undef CSA_CVT
  }
}

__device__ __forceinline__ void encode_block(const uint16_t* __restrict__ p, int& e,
                                             uint32_t (&word)[4]) {
  uint4 u[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) u[i] = ld16(p + 8 * i);
  // |bf16| orders as its low 15 bits
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t w = bf16_pair(u, i);
    m = max(m, max(w & 0x7fffu, (w >> 16) & 0x7fffu));
  }
  e = mx_block_exponent(__uint_as_float(m << 16));
  if (e > -127) {
    const float sc = __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
#define CSA_CVT(w, i, sel) \
  __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(w, __builtin_bit_cast(bf16x2_t, bf16_pair(u, i)), sc, sel)
#pragma unroll
    for (int d = 0; d < 4; ++d) CSA_PACK4(d, CSA_CVT)
#undef CSA_CVT
  } else {
#define CSA_CVT(w, i, sel)                                                                  \
  __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, bf16_lo(bf16_pair(u, i)) * 0x1p126f,          \
                                           bf16_hi(bf16_pair(u, i)) * 0x1p126f, 0.5f, sel)
#pragma unroll
    for (int d = 0; d < 4; ++d) CSA_PACK4(d, CSA_CVT)
#undef CSA_CVT
  }
}
#undef CSA_PACK4

template <typename T>
__global__ __launch_bounds__(kQuantThreads) void quantize_mx4_kernel(
    const T* __restrict__ x, int64_t x_rs, int rows, int nblk, uint8_t* __restrict__ codes,
    int64_t c_rs, uint8_t* __restrict__ scales, int64_t s_rs) {
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * kQuantThreads + threadIdx.x;
  if (gid >= static_cast<int64_t>(rows) * nblk) return;
  const int64_t r = gid / nblk;
  const int blk = static_cast<int>(gid - r * nblk);
  int e;
  uint32_t word[4];
  encode_block(x + r * x_rs + 32 * blk, e, word);
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
