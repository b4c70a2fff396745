// kernels_misc.hip -- the two elementwise kernels of the unfused three-kernel
// path (measurement baseline), a plain streaming read (the measured HBM read
// ceiling) and a zero-fill kernel.
//
// The unfused path is the one the opacity-barrier section of "Совместная
// работа Helion и TorchInductor: слияние операторов" describes and its
// output-code listing shows: the GEMM result is materialised, then re-read by
// a separate bias + GELU kernel whose output is materialised again, then
// re-read to scale and add the residual.  It exists to measure the HBM bytes
// the fused epilogue saves; it is not used by lin_gemm_run.
#include <mutex>
#include <set>
#include <utility>

#include "launch.hpp"

namespace lg {
namespace {

// U = act(T + bias): 8 consecutive elements of one row per thread.
template <bool F16>
__global__ __launch_bounds__(256) void bias_act_kernel(const uint16_t* __restrict__ T,
                                                       const uint16_t* __restrict__ bias,
                                                       uint16_t* __restrict__ U, int64_t M,
                                                       int64_t N, int act) {
  const int64_t nq = (N + 7) / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t m = idx / nq;
  const int64_t n = (idx - m * nq) * 8;
  if (m >= M) return;
  const uint16_t* t = T + m * N;
  uint16_t* u = U + m * N;
  if (n + 8 <= N && (N % 8) == 0) {
    float y[8], b[8];
    load_h<8, F16>(t + n, y);
    if (bias) {
      load_h<8, F16>(bias + n, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] += b[i];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = act_apply(act, y[i]);
    store_h<8, F16>(u + n, y);
  } else {
    for (int64_t j = n; j < N && j < n + 8; ++j) {
      float y = h_to_f32<F16>(t[j]);
      if (bias) y += h_to_f32<F16>(bias[j]);
      u[j] = f32_to_h<F16>(act_apply(act, y));
    }
  }
}

// C = alpha * U + residual.
template <bool F16>
__global__ __launch_bounds__(256) void scale_residual_kernel(const uint16_t* __restrict__ U,
                                                             const uint16_t* __restrict__ R,
                                                             uint16_t* __restrict__ C, int64_t M,
                                                             int64_t N, float alpha) {
  const int64_t nq = (N + 7) / 8;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t m = idx / nq;
  const int64_t n = (idx - m * nq) * 8;
  if (m >= M) return;
  const uint16_t* u = U + m * N;
  uint16_t* c = C + m * N;
  if (n + 8 <= N && (N % 8) == 0) {
    float y[8], r[8];
    load_h<8, F16>(u + n, y);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] *= alpha;
    if (R) {
      load_h<8, F16>(R + m * N + n, r);
#pragma unroll
      for (int i = 0; i < 8; ++i) y[i] += r[i];
    }
    store_h<8, F16>(c + n, y);
  } else {
    for (int64_t j = n; j < N && j < n + 8; ++j) {
      float y = h_to_f32<F16>(u[j]) * alpha;
      if (R) y += h_to_f32<F16>(R[m * N + j]);
      c[j] = f32_to_h<F16>(y);
    }
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(i32x4* __restrict__ p, int64_t n16,
                                                        int* __restrict__ tail, int64_t ntail) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = i32x4{0, 0, 0, 0};
  if (i < ntail) tail[i] = 0;
}

inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

// A plain streaming read (measurement only): the HBM read rate the weight
// stream of a decode call is compared with.  Thread t of the grid reads the
// 16-byte chunks t, t + T, t + 2T, ... (T threads in all; consecutive
// threads read consecutive chunks), U of them issued before any is used,
// and folds them with XOR.  The result is stored only when it equals one
// fixed value, so the loads cannot be dropped and nothing is written in
// practice.
template <int U>
__global__ __launch_bounds__(256) void stream_read_kernel(const i32x4* __restrict__ src,
                                                          int64_t n16, int* __restrict__ sink) {
  const int64_t T = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  i32x4 x = {0, 0, 0, 0};
  for (; i + (U - 1) * T < n16; i += U * T) {
    i32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = src[i + u * T];
#pragma unroll
    for (int u = 0; u < U; ++u) x ^= v[u];
  }
  for (; i < n16; i += T) x ^= src[i];
  const int r = x[0] ^ x[1] ^ x[2] ^ x[3];
  if (r == 0x2545F491) sink[threadIdx.x] = r;
}

}  // namespace

hipError_t launch_bias_act(const void* T, const void* bias, void* U, int64_t M, int64_t N,
                           int act, bool f16, hipStream_t s) {
  const int64_t threads = M * ((N + 7) / 8);
  if (threads == 0) return hipSuccess;
  if (f16)
    hipLaunchKernelGGL(bias_act_kernel<true>, dim3(blocks_for(threads)), dim3(256), 0, s,
                       (const uint16_t*)T, (const uint16_t*)bias, (uint16_t*)U, M, N, act);
  else
    hipLaunchKernelGGL(bias_act_kernel<false>, dim3(blocks_for(threads)), dim3(256), 0, s,
                       (const uint16_t*)T, (const uint16_t*)bias, (uint16_t*)U, M, N, act);
  return hipGetLastError();
}

hipError_t launch_scale_residual(const void* U, const void* residual, void* C, int64_t M,
                                 int64_t N, float alpha, bool f16, hipStream_t s) {
  const int64_t threads = M * ((N + 7) / 8);
  if (threads == 0) return hipSuccess;
  if (f16)
    hipLaunchKernelGGL(scale_residual_kernel<true>, dim3(blocks_for(threads)), dim3(256), 0, s,
                       (const uint16_t*)U, (const uint16_t*)residual, (uint16_t*)C, M, N, alpha);
  else
    hipLaunchKernelGGL(scale_residual_kernel<false>, dim3(blocks_for(threads)), dim3(256), 0, s,
                       (const uint16_t*)U, (const uint16_t*)residual, (uint16_t*)C, M, N, alpha);
  return hipGetLastError();
}

// Zero `bytes` bytes (a multiple of 4) at p (16-byte aligned), without
// hipMemsetAsync so the call is safe inside captured graphs.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  const int64_t ntail = (int64_t)((bytes % 16) / 4);
  int* tail = (int*)((char*)p + n16 * 16);
  const int64_t threads = n16 > ntail ? n16 : ntail;
  if (threads == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks_for(threads)), dim3(256), 0, s, (i32x4*)p,
                     n16, tail, ntail);
  return hipGetLastError();
}

hipError_t opt_in_lds(const void* fn, size_t bytes) {
  static std::mutex mu;
  static std::set<std::pair<const void*, int>> done;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  std::lock_guard<std::mutex> lock(mu);
  if (done.count({fn, dev})) return hipSuccess;
  err = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (err == hipSuccess) done.insert({fn, dev});
  return err;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, int grid, int unroll, int* sink,
                              hipStream_t s) {
  const int64_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  const dim3 g((unsigned)grid), b(256);
  const i32x4* p = (const i32x4*)src;
  switch (unroll) {
    case 4: hipLaunchKernelGGL(stream_read_kernel<4>, g, b, 0, s, p, n16, sink); break;
    case 8: hipLaunchKernelGGL(stream_read_kernel<8>, g, b, 0, s, p, n16, sink); break;
    case 16: hipLaunchKernelGGL(stream_read_kernel<16>, g, b, 0, s, p, n16, sink); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lg
