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
// Must be reached by the whole workgroup (it synchronises).
template <typename T>
__device__ __forceinline__ void pool_block(const T* __restrict__ xb, int64_t x_st,
                                           const float* __restrict__ zb, T* __restrict__ orow,
                                           int m, int CH, int P) {
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
  if (tid < CH) {
    float r[E];
#pragma unroll
    for (int c = 0; c < E; ++c) r[c] = part[tid * E + c];
    for (int q = 1; q < P; ++q) {
#pragma unroll
      for (int c = 0; c < E; ++c) r[c] += part[(q * CH + tid) * E + c];
    }
#pragma unroll
    for (int c = 0; c < E; ++c) r[c] = r[c] / total;
    st16(orow + tid * E, Chunk<T>::pack(r));
  }
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

}  // namespace

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
