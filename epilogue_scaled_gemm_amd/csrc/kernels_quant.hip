// kernels_quant.hip -- dynamic activation quantization: X[M][K] (bf16 or
// fp16) -> codes Q[M][K] (e4m3 or int8) and fp32 scales, one scale per token
// (row) or per 1x128 block of a row.  It produces the A operand and the
// activation scales of the quantised layer modes at run time.
//
// What the pages fix: "helion-vllm-linear-backend" (section "Одно ядро
// вместо трёх вариантов") gives FP8_Dynamic a per-token activation scale,
// W8A8_INT8 the same scaling in int8 and Block_FP8 1x128 activation blocks;
// the prologue/epilogue section of "Совместная работа Helion и
// TorchInductor" lists quantization among the input-side transforms.  The
// rest is the plain reading: for each group, s = max|x| / QMAX in binary32
// (QMAX = 448 for e4m3, 127 for int8; s = 1 for an all-zero group), and each
// code rounds x / s (a correctly rounded binary32 division) to nearest, ties
// to even, saturating at +-QMAX.
//
// gfx950 design: HBM-bound (2 bytes read, 1 written per value).  A token row
// is one workgroup of 256 threads; each thread keeps up to four 16-byte
// chunks (rows of up to 8192 values) in registers between the maximum pass
// and the rounding pass, so the row is read from memory once; the maximum is
// reduced across the wave with lane shuffles and across the four waves
// through LDS.  A 1x128 block is 16 lanes x 8 values: its maximum needs only
// a 16-lane shuffle reduction, no LDS and no barrier.  e4m3 codes come from
// the hardware conversion (round to nearest even) after an explicit clamp to
// +-448; int8 codes from v_rndne and a clamp.  The quotients x / s use one
// reciprocal per group and an FMA correction per value (div_rn), which gives
// the correctly rounded quotient without a division per value.
#include "launch.hpp"

namespace lg {
namespace {

constexpr int DQ_THREADS = 256;
constexpr int DQ_CACHE = 4;  // 16-byte chunks per thread kept in registers

// One token row per workgroup.
template <bool F16, bool INT8>
__global__ __launch_bounds__(DQ_THREADS) void dq_token_kernel(const uint16_t* __restrict__ X,
                                                              int64_t K, uint8_t* __restrict__ Q,
                                                              float* __restrict__ scales) {
  const int64_t row = blockIdx.x;
  const uint16_t* x = X + row * K;
  uint8_t* q = Q + row * K;
  const int nch = (int)(K / 8);  // 16-byte chunks of the row
  const int tid = threadIdx.x;

  // Maximum pass.  Chunks past the row re-read its last chunk (in bounds;
  // a repeat does not change the maximum) and are never stored.
  i32x4 cache[DQ_CACHE];
#pragma unroll
  for (int j = 0; j < DQ_CACHE; ++j) {
    const int c = min(tid + j * DQ_THREADS, nch - 1);
    cache[j] = *(const i32x4*)(x + (int64_t)c * 8);
  }
  float am = 0.f;
#pragma unroll
  for (int j = 0; j < DQ_CACHE; ++j) {
    float v[8];
    unpack8<F16>(cache[j], v);
    am = fmaxf(am, amax8(v));
  }
  for (int c = tid + DQ_CACHE * DQ_THREADS; c < nch; c += DQ_THREADS) {
    float v[8];
    unpack8<F16>(*(const i32x4*)(x + (int64_t)c * 8), v);
    am = fmaxf(am, amax8(v));
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off));
  __shared__ float wmax[DQ_THREADS / 64];
  if ((tid & 63) == 0) wmax[tid >> 6] = am;
  __syncthreads();
  am = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  const float s = group_scale(am, INT8 ? 127.f : 448.f);
  if (tid == 0) scales[row] = s;
  const DivBy d = make_div(s, am);

  // Rounding pass.
#pragma unroll
  for (int j = 0; j < DQ_CACHE; ++j) {
    const int c = tid + j * DQ_THREADS;
    if (c < nch) {
      float v[8];
      unpack8<F16>(cache[j], v);
      *(i32x2*)(q + (int64_t)c * 8) = quant8<INT8>(v, d);
    }
  }
  for (int c = tid + DQ_CACHE * DQ_THREADS; c < nch; c += DQ_THREADS) {
    float v[8];
    unpack8<F16>(*(const i32x4*)(x + (int64_t)c * 8), v);
    *(i32x2*)(q + (int64_t)c * 8) = quant8<INT8>(v, d);
  }
}

// 1x128 blocks (e4m3): block b is X[b*128 .. b*128+128) (blocks tile each row
// in order), 16 lanes of 8 values each; its scale goes to scales[b], which
// is scales[m][kb] of the [M][K/128] layout.
template <bool F16>
__global__ __launch_bounds__(DQ_THREADS) void dq_block_kernel(const uint16_t* __restrict__ X,
                                                              int64_t nblk,
                                                              uint8_t* __restrict__ Q,
                                                              float* __restrict__ scales) {
  const int64_t t = (int64_t)blockIdx.x * DQ_THREADS + threadIdx.x;
  const int64_t b = t >> 4;
  const int sub = threadIdx.x & 15;
  // Lanes past the last block re-read it (all 16 lanes of a group take part
  // in the shuffles) and store nothing.
  const int64_t bc = b < nblk ? b : nblk - 1;
  float v[8];
  unpack8<F16>(*(const i32x4*)(X + bc * 128 + sub * 8), v);
  float am = amax8(v);
#pragma unroll
  for (int off = 8; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 16));
  const float s = group_scale(am, 448.f);
  if (b < nblk) {
    *(i32x2*)(Q + bc * 128 + sub * 8) = quant8<false>(v, make_div(s, am));
    if (sub == 0) scales[b] = s;
  }
}

}  // namespace

hipError_t launch_dynamic_quant(int kind, bool f16, const void* X, int64_t M, int64_t K, void* Q,
                                float* scales, hipStream_t s) {
  const uint16_t* x = (const uint16_t*)X;
  uint8_t* q = (uint8_t*)Q;
  if (kind == DQ_FP8_BLOCK) {
    const int64_t nblk = M * (K / 128);
    const dim3 grid((unsigned)((nblk * 16 + DQ_THREADS - 1) / DQ_THREADS));
    if (f16) hipLaunchKernelGGL((dq_block_kernel<true>), grid, dim3(DQ_THREADS), 0, s, x, nblk, q, scales);
    else hipLaunchKernelGGL((dq_block_kernel<false>), grid, dim3(DQ_THREADS), 0, s, x, nblk, q, scales);
    return hipGetLastError();
  }
  const dim3 grid((unsigned)M);
  const bool i8 = kind == DQ_INT8_TOKEN;
  if (f16 && i8) hipLaunchKernelGGL((dq_token_kernel<true, true>), grid, dim3(DQ_THREADS), 0, s, x, K, q, scales);
  else if (f16) hipLaunchKernelGGL((dq_token_kernel<true, false>), grid, dim3(DQ_THREADS), 0, s, x, K, q, scales);
  else if (i8) hipLaunchKernelGGL((dq_token_kernel<false, true>), grid, dim3(DQ_THREADS), 0, s, x, K, q, scales);
  else hipLaunchKernelGGL((dq_token_kernel<false, false>), grid, dim3(DQ_THREADS), 0, s, x, K, q, scales);
  return hipGetLastError();
}

}  // namespace lg
