// Token-dimension compression: every m consecutive raw tokens become one
// compressed entry by softmax-weighted aggregation ("DeepSeek V4 技术解读",
// §2.1 KV cache compression; §2.2 uses m' = 128).
//
// HBM-streaming design: one workgroup per compressed entry (b, j).  Thread
// (p, ch) owns one 16-byte channel chunk ch and the tokens i = p (mod P) of
// the block, so each wave reads whole 16-byte lanes of consecutive memory.
// Per-thread partial sums are combined in LDS in a fixed order: the result
// does not depend on the batch or the grid (batch invariant, no atomics).
#include "device_common.h"
#include "internal.h"

namespace csa {
namespace {

constexpr int kCompressThreads = 256;
constexpr int kMaxPool = 4096;

template <typename T>
struct Chunk;   // 16-byte chunk <-> fp32 lanes
template <>
struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static void unpack(uint4 v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};
template <>
struct Chunk<uint16_t> {
  static constexpr int N = 8;
  __device__ static void unpack(uint4 v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
  __device__ static uint4 pack(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]),
                      pack_bf16x2(f[6], f[7]));
  }
};

// Pools one block of m rows (xb, token stride x_st; logits zb) into orow.
// With CH0 < CH the channels of chunks CH0 .. CH-1 are not stored in orow
// but MX FP4 encoded from their fp32 pooled values: codes to crow (element
// 2i in the low nibble of byte i), one E8M0 byte per 32 channels to srow.
// Must be reached by the whole workgroup (it synchronises).
template <typename T>
__device__ __forceinline__ void pool_block(const T* __restrict__ xb, int64_t x_st,
                                           const float* __restrict__ zb, T* __restrict__ orow,
                                           int m, int CH, int P, int CH0 = 1 << 30,
                                           uint8_t* __restrict__ crow = nullptr,
                                           uint8_t* __restrict__ srow = nullptr) {
  constexpr int E = Chunk<T>::N;
  __shared__ float e_s[kMaxPool];
  __shared__ float red[kCompressThreads / 64];
  __shared__ float part[kCompressThreads * E];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;

  // softmax weights of the block's logits (unnormalised; divided at the end)
  float mx = kNegInf;
  for (int i = tid; i < m; i += blockDim.x) mx = fmaxf(mx, zb[i]);
  mx = wave_max(mx);
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  mx = red[0];
  for (int w = 1; w < nwaves; ++w) mx = fmaxf(mx, red[w]);
  __syncthreads();
  float sum = 0.f;
  for (int i = tid; i < m; i += blockDim.x) {
    const float e = expf(zb[i] - mx);
    e_s[i] = e;
    sum += e;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[wave] = sum;
  __syncthreads();
  float total = 0.f;
  for (int w = 0; w < nwaves; ++w) total += red[w];

  // weighted sum of the block's rows, one 16-byte channel chunk per thread
  const int ch = tid % CH, p = tid / CH;
  if (p < P) {
    float acc[E];
#pragma unroll
    for (int c = 0; c < E; ++c) acc[c] = 0.f;
    const T* xc = xb + ch * E;
#pragma unroll 4
    for (int i = p; i < m; i += P) {
      float f[E];
      Chunk<T>::unpack(ld16(xc + static_cast<int64_t>(i) * x_st), f);
      const float e = e_s[i];
#pragma unroll
      for (int c = 0; c < E; ++c) acc[c] = fmaf(e, f[c], acc[c]);
    }
#pragma unroll
    for (int c = 0; c < E; ++c) part[(p * CH + ch) * E + c] = acc[c];
  }
  __syncthreads();
  float r[E];
#pragma unroll
  for (int c = 0; c < E; ++c) r[c] = 0.f;
  if (tid < CH) {
#pragma unroll
    for (int c = 0; c < E; ++c) r[c] = part[tid * E + c];
    for (int q = 1; q < P; ++q) {
#pragma unroll
      for (int c = 0; c < E; ++c) r[c] += part[(q * CH + tid) * E + c];
    }
#pragma unroll
    for (int c = 0; c < E; ++c) r[c] = r[c] / total;
    if (tid < CH0) st16(orow + tid * E, Chunk<T>::pack(r));
  }
  if (CH0 < CH) {
    // MX FP4 blocks of 32 channels = G consecutive chunk threads (aligned
    // groups of lanes): the block maximum by lane exchanges, then each
    // thread encodes its E channels
    constexpr int G = 32 / E;
    float am = 0.f;
#pragma unroll
    for (int c = 0; c < E; ++c) am = fmaxf(am, fabsf(r[c]));
#pragma unroll
    for (int o = 1; o < G; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    if (tid >= CH0 && tid < CH) {
      const int e = mx_block_exponent(am);
      const int q = tid - CH0;
      uint32_t w = 0;
      w = mx_cvt_pair<0>(w, r[0], r[1], e);
      w = mx_cvt_pair<1>(w, r[2], r[3], e);
      if constexpr (E == 8) {
        w = mx_cvt_pair<2>(w, r[4], r[5], e);
        w = mx_cvt_pair<3>(w, r[6], r[7], e);
        *reinterpret_cast<uint32_t*>(crow + 4 * q) = w;
      } else {
        *reinterpret_cast<uint16_t*>(crow + 2 * q) = static_cast<uint16_t>(w);
      }
      if (q % G == 0) srow[q / G] = static_cast<uint8_t>(e + 127);
    }
  }
}

// Small blocks (m <= kSmallPool): one thread per (entry, 16-byte channel
// chunk), the entries of the whole batch laid end to end, so a 256-thread
// workgroup covers several entries with coalesced loads (the threads of one
// entry read each token row contiguously).  Each thread forms the block's
// softmax weights itself from the m logits and sums its chunk over the m
// tokens in token order: no LDS and no barrier, which a workgroup per entry
// of a few kilobytes cannot amortise.  With CH0 < CH the chunks from CH0 on
// are MX FP4 encoded as in pool_block (the 32-channel blocks are aligned
// groups of consecutive threads; lanes past the end repeat the last chunk so
// that every lane takes part in the exchanges).
constexpr int kSmallPool = 16;

template <typename T>
__global__ __launch_bounds__(256) void compress_small_kernel(
    const T* __restrict__ x, int64_t x_sb, int64_t x_st, const float* __restrict__ z,
    int64_t z_sb, T* __restrict__ out, int64_t o_sb, int64_t o_sj, uint8_t* __restrict__ codes,
    int64_t c_sb, int64_t c_sj, uint8_t* __restrict__ scales, int64_t s_sb, int64_t s_sj, int m,
    int CH, int CH0, int nblk, int64_t total) {
  constexpr int E = Chunk<T>::N;
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const bool own = gid < total;
  const int64_t g = own ? gid : total - 1;
  const int ch = static_cast<int>(g % CH);
  const int64_t ent = g / CH;
  const int j = static_cast<int>(ent % nblk), b = static_cast<int>(ent / nblk);
  const float* zb = z + b * z_sb + static_cast<int64_t>(j) * m;
  const T* xb = x + b * x_sb + static_cast<int64_t>(j) * m * x_st + ch * E;
  uint4 raw[kSmallPool];
#pragma unroll
  for (int i = 0; i < kSmallPool; ++i)
    if (i < m) raw[i] = ld16(xb + static_cast<int64_t>(i) * x_st);
  float mx = kNegInf;
  for (int i = 0; i < m; ++i) mx = fmaxf(mx, zb[i]);
  float acc[E], tw = 0.f;
#pragma unroll
  for (int c = 0; c < E; ++c) acc[c] = 0.f;
#pragma unroll
  for (int i = 0; i < kSmallPool; ++i) {
    if (i < m) {
      const float wgt = expf(zb[i] - mx);
      tw += wgt;
      float f[E];
      Chunk<T>::unpack(raw[i], f);
#pragma unroll
      for (int c = 0; c < E; ++c) acc[c] = fmaf(wgt, f[c], acc[c]);
    }
  }
  float r[E];
#pragma unroll
  for (int c = 0; c < E; ++c) r[c] = acc[c] / tw;
  if (own && ch < CH0) st16(out + b * o_sb + static_cast<int64_t>(j) * o_sj + ch * E, Chunk<T>::pack(r));
  if (CH0 < CH) {
    constexpr int G = 32 / E;
    float am = 0.f;
#pragma unroll
    for (int c = 0; c < E; ++c) am = fmaxf(am, fabsf(r[c]));
#pragma unroll
    for (int o = 1; o < G; o <<= 1) am = fmaxf(am, __shfl_xor(am, o, 64));
    if (own && ch >= CH0) {
      const int e = mx_block_exponent(am);
      const int q = ch - CH0;
      uint8_t* crow = codes + b * c_sb + static_cast<int64_t>(j) * c_sj;
      uint32_t w = 0;
      w = mx_cvt_pair<0>(w, r[0], r[1], e);
      w = mx_cvt_pair<1>(w, r[2], r[3], e);
      if constexpr (E == 8) {
        w = mx_cvt_pair<2>(w, r[4], r[5], e);
        w = mx_cvt_pair<3>(w, r[6], r[7], e);
        *reinterpret_cast<uint32_t*>(crow + 4 * q) = w;
      } else {
        *reinterpret_cast<uint16_t*>(crow + 2 * q) = static_cast<uint16_t>(w);
      }
      if (q % G == 0)
        scales[b * s_sb + static_cast<int64_t>(j) * s_sj + q / G] = static_cast<uint8_t>(e + 127);
    }
  }
}

template <typename T>
hipError_t launch_small(const void* x, int64_t x_sb, int64_t x_st, const float* z, int64_t z_sb,
                        void* out, int64_t o_sb, int64_t o_sj, uint8_t* codes, int64_t c_sb,
                        int64_t c_sj, uint8_t* scales, int64_t s_sb, int64_t s_sj, int B, int nblk,
                        int CH, int CH0, int m, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(B) * nblk * CH;
  hipLaunchKernelGGL(compress_small_kernel<T>, dim3(static_cast<unsigned>((total + 255) / 256)),
                     dim3(256), 0, s, static_cast<const T*>(x), x_sb, x_st, z, z_sb,
                     static_cast<T*>(out), o_sb, o_sj, codes, c_sb, c_sj, scales, s_sb, s_sj, m,
                     CH, CH0, nblk, total);
  return hipGetLastError();
}

// One workgroup per compressed entry (j, b) of the batch.
template <typename T>
__global__ __launch_bounds__(kCompressThreads) void compress_kernel(
    const T* __restrict__ x, int64_t x_sb, int64_t x_st, const float* __restrict__ z,
    int64_t z_sb, T* __restrict__ out, int64_t o_sb, int64_t o_sj, int m, int CH, int P) {
  const int j = blockIdx.x, b = blockIdx.y;
  pool_block<T>(x + b * x_sb + static_cast<int64_t>(j) * m * x_st, x_st,
                z + b * z_sb + static_cast<int64_t>(j) * m, out + b * o_sb + static_cast<int64_t>(j) * o_sj,
                m, CH, P);
}

// The same with the channels from CH0 chunks on MX FP4 encoded.
template <typename T>
__global__ __launch_bounds__(kCompressThreads) void compress_mx4_kernel(
    const T* __restrict__ x, int64_t x_sb, int64_t x_st, const float* __restrict__ z,
    int64_t z_sb, T* __restrict__ out, int64_t o_sb, int64_t o_sj, uint8_t* __restrict__ codes,
    int64_t c_sb, int64_t c_sj, uint8_t* __restrict__ scales, int64_t s_sb, int64_t s_sj, int m,
    int CH, int P, int CH0) {
  const int j = blockIdx.x, b = blockIdx.y;
  pool_block<T>(x + b * x_sb + static_cast<int64_t>(j) * m * x_st, x_st,
                z + b * z_sb + static_cast<int64_t>(j) * m,
                out + b * o_sb + static_cast<int64_t>(j) * o_sj, m, CH, P, CH0,
                codes + b * c_sb + static_cast<int64_t>(j) * c_sj,
                scales + b * s_sb + static_cast<int64_t>(j) * s_sj);
}

// Append: one workgroup per sequence.  Token t = t_new[b] was just added; if
// it completes a block (m divides t + 1), entry j = (t + 1) / m - 1 pools
// tokens m j .. m j + m - 1, read from rows (m j + i) mod x_rows of x and z
// (x_rows a multiple of m: a ring of the latest tokens, or the whole
// sequence), and the sequence's entry count becomes j + 1.  Entries at or
// past N_max are not written.
template <typename T>
__global__ __launch_bounds__(kCompressThreads) void compress_append_kernel(
    const T* __restrict__ x, int64_t x_sb, int64_t x_st, int x_rows, const float* __restrict__ z,
    int64_t z_sb, const int32_t* __restrict__ t_new, T* __restrict__ cache, int64_t c_sb,
    int64_t c_sj, int32_t* __restrict__ n_entries, int N_max, int m, int CH, int P) {
  const int b = blockIdx.x;
  const int t = t_new[b];
  if (t < 0 || (t + 1) % m != 0) return;          // uniform over the workgroup
  const int j = (t + 1) / m - 1;
  if (j >= N_max) return;
  const int64_t r0 = static_cast<int64_t>(m) * j % x_rows;
  pool_block<T>(x + b * x_sb + r0 * x_st, x_st, z + b * z_sb + r0, cache + b * c_sb + j * c_sj, m,
                CH, P);
  if (threadIdx.x == 0) n_entries[b] = j + 1;
}

template <typename T>
hipError_t launch_typed(const void* x, int64_t x_sb, int64_t x_st, const float* z, int64_t z_sb,
                        void* out, int64_t o_sb, int64_t o_sj, int B, int n, int C, int m,
                        hipStream_t s) {
  constexpr int E = Chunk<T>::N;
  const int CH = C / E;
  int P = kCompressThreads / CH;
  if (P > m) P = m;
  int threads = ((P * CH + 63) / 64) * 64;
  const int nblk = n / m;
  if (nblk == 0) return hipSuccess;
  if (m <= kSmallPool)
    return launch_small<T>(x, x_sb, x_st, z, z_sb, out, o_sb, o_sj, nullptr, 0, 0, nullptr, 0, 0,
                           B, nblk, CH, CH, m, s);
  hipLaunchKernelGGL(compress_kernel<T>, dim3(nblk, B), dim3(threads), 0, s,
                     static_cast<const T*>(x), x_sb, x_st, z, z_sb, static_cast<T*>(out), o_sb,
                     o_sj, m, CH, P);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_append_typed(const void* x, int64_t x_sb, int64_t x_st, int x_rows,
                               const float* z, int64_t z_sb, const int32_t* t_new, void* cache,
                               int64_t c_sb, int64_t c_sj, int32_t* n_entries, int B, int C,
                               int m, int N_max, hipStream_t s) {
  constexpr int E = Chunk<T>::N;
  const int CH = C / E;
  int P = kCompressThreads / CH;
  if (P > m) P = m;
  const int threads = ((P * CH + 63) / 64) * 64;
  hipLaunchKernelGGL(compress_append_kernel<T>, dim3(B), dim3(threads), 0, s,
                     static_cast<const T*>(x), x_sb, x_st, x_rows, z, z_sb, t_new,
                     static_cast<T*>(cache), c_sb, c_sj, n_entries, N_max, m, CH, P);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_mx4_typed(const void* x, int64_t x_sb, int64_t x_st, const float* z, int64_t z_sb,
                            void* out, int64_t o_sb, int64_t o_sj, uint8_t* codes, int64_t c_sb,
                            int64_t c_sj, uint8_t* scales, int64_t s_sb, int64_t s_sj, int B,
                            int n, int C, int D_mx, int m, hipStream_t s) {
  constexpr int E = Chunk<T>::N;
  const int CH = C / E;
  int P = kCompressThreads / CH;
  if (P > m) P = m;
  const int threads = ((P * CH + 63) / 64) * 64;
  const int nblk = n / m;
  if (nblk == 0) return hipSuccess;
  if (m <= kSmallPool)
    return launch_small<T>(x, x_sb, x_st, z, z_sb, out, o_sb, o_sj, codes, c_sb, c_sj, scales,
                           s_sb, s_sj, B, nblk, CH, (C - D_mx) / E, m, s);
  hipLaunchKernelGGL(compress_mx4_kernel<T>, dim3(nblk, B), dim3(threads), 0, s,
                     static_cast<const T*>(x), x_sb, x_st, z, z_sb, static_cast<T*>(out), o_sb,
                     o_sj, codes, c_sb, c_sj, scales, s_sb, s_sj, m, CH, P, (C - D_mx) / E);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_compress_mx4(const void* x, int64_t x_sb, int64_t x_st, const float* z,
                               int64_t z_sb, void* out, int64_t o_sb, int64_t o_sj,
                               uint8_t* codes, int64_t c_sb, int64_t c_sj, uint8_t* scales,
                               int64_t s_sb, int64_t s_sj, csa_dtype_t dt, int B, int n, int C,
                               int D_mx, int m, hipStream_t s) {
  if (dt == CSA_F32)
    return launch_mx4_typed<float>(x, x_sb, x_st, z, z_sb, out, o_sb, o_sj, codes, c_sb, c_sj,
                                   scales, s_sb, s_sj, B, n, C, D_mx, m, s);
  return launch_mx4_typed<uint16_t>(x, x_sb, x_st, z, z_sb, out, o_sb, o_sj, codes, c_sb, c_sj,
                                    scales, s_sb, s_sj, B, n, C, D_mx, m, s);
}

hipError_t launch_compress_append(const void* x, int64_t x_sb, int64_t x_st, int x_rows,
                                  const float* z, int64_t z_sb, const int32_t* t_new, void* cache,
                                  int64_t c_sb, int64_t c_sj, int32_t* n_entries, csa_dtype_t dt,
                                  int B, int C, int m, int N_max, hipStream_t s) {
  if (dt == CSA_F32)
    return launch_append_typed<float>(x, x_sb, x_st, x_rows, z, z_sb, t_new, cache, c_sb, c_sj,
                                      n_entries, B, C, m, N_max, s);
  return launch_append_typed<uint16_t>(x, x_sb, x_st, x_rows, z, z_sb, t_new, cache, c_sb, c_sj,
                                       n_entries, B, C, m, N_max, s);
}

hipError_t launch_compress(const void* x, int64_t x_sb, int64_t x_st, const float* z, int64_t z_sb,
                           void* out, int64_t o_sb, int64_t o_sj, csa_dtype_t dt, int B, int n,
                           int C, int m, hipStream_t s) {
  if (dt == CSA_F32)
    return launch_typed<float>(x, x_sb, x_st, z, z_sb, out, o_sb, o_sj, B, n, C, m, s);
  return launch_typed<uint16_t>(x, x_sb, x_st, z, z_sb, out, o_sb, o_sj, B, n, C, m, s);
}

}  // namespace csa
