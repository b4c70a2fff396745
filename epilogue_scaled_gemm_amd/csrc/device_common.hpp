// device_common.hpp -- types and register-resident epilogue pieces shared by
// the gfx950 kernels of the scaled linear layer.
//
// The epilogue follows the epilogue-fusion section of "Совместная работа
// Helion и TorchInductor: слияние операторов": the accumulator tile is still
// in registers when the K loop ends, so scaling, bias, activation, the
// residual add and the narrowing to a 16-bit float are applied there and the
// result is stored once.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lg {

// ------------------------------------------------------------ vector types
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;

// Element kinds of the operands.
enum QKind : int { QK_BF16 = 0, QK_FP16 = 1, QK_FP8 = 2, QK_I8 = 3, QK_FP8_BLOCK = 4,
                   QK_MXFP4 = 5 };
// Activation codes (1 = ReLU and 2 = GELU-tanh keep the listing's numbering).
enum ActCode : int { ACT_NONE = 0, ACT_RELU = 1, ACT_GELU_TANH = 2, ACT_SILU = 3 };

template <int QK> struct QTraits;
template <> struct QTraits<QK_BF16> { typedef float Acc; static constexpr bool out_f16 = false; };
template <> struct QTraits<QK_FP16> { typedef float Acc; static constexpr bool out_f16 = true; };
template <> struct QTraits<QK_FP8> { typedef float Acc; static constexpr bool out_f16 = false; };
template <> struct QTraits<QK_I8> { typedef int Acc; static constexpr bool out_f16 = false; };
template <> struct QTraits<QK_FP8_BLOCK> { typedef float Acc; static constexpr bool out_f16 = false; };
template <> struct QTraits<QK_MXFP4> { typedef float Acc; static constexpr bool out_f16 = false; };

// ----------------------------------------------------------- MFMA wrappers
// A 16 x 16 output tile per wave.  Every K step covers 128 bytes of each
// operand row, supplied as 32 bytes per lane: lane l owns MFMA row (weight
// side) / column (activation side) l % 16, and lane group g = l / 16 owns
// bytes [32 g, 32 g + 32) of the step, consumed as two 16-byte halves.
// prep() turns a 16-byte half into MFMA operand registers and mma() adds the
// product of a weight and an activation operand into the accumulator.  Both
// operands use the same byte-to-k assignment, so which k the hardware gives
// each byte does not change the dot product.
//
// e4m3 operands are widened to bf16 (exact: 4 significant bits) and
// multiplied with the bf16 MFMA.  gfx950's fp8 MFMAs sum small groups of
// adjacent products in a window of about 14 bits below the group's largest
// product (a 448*448 + 1*1 pair returns 200704), which moves near-zero
// outputs of long dot products by ~1e-5 of the output scale; the bf16 MFMA
// keeps fp32-like precision, so the widened path is the exact one.
template <int QK> struct Mfma;

template <> struct Mfma<QK_BF16> {
  typedef f32x4 C;
  typedef i32x4 Frag;
  static __device__ inline Frag prep(const i32x4& raw) { return raw; }
  static __device__ inline C mma(const Frag& w, const Frag& x, C c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, w),
                                                   __builtin_bit_cast(bf16x8, x), c, 0, 0, 0);
  }
};
template <> struct Mfma<QK_FP16> {
  typedef f32x4 C;
  typedef i32x4 Frag;
  static __device__ inline Frag prep(const i32x4& raw) { return raw; }
  static __device__ inline C mma(const Frag& w, const Frag& x, C c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, w),
                                                  __builtin_bit_cast(f16x8, x), c, 0, 0, 0);
  }
};
template <> struct Mfma<QK_I8> {
  typedef i32x4 C;
  typedef i32x4 Frag;
  static __device__ inline Frag prep(const i32x4& raw) { return raw; }
  static __device__ inline C mma(const Frag& w, const Frag& x, C c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(w, x, c, 0, 0, 0);
  }
};
template <> struct Mfma<QK_FP8> {
  typedef f32x4 C;
  typedef i32x8 Frag;  // 16 bf16 values
  static __device__ inline Frag prep(const i32x4& raw) {
    Frag f;
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
      bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)raw[d], 1.0f, false);
      bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)raw[d], 1.0f, true);
      f[2 * d] = __builtin_bit_cast(int, lo);
      f[2 * d + 1] = __builtin_bit_cast(int, hi);
    }
    return f;
  }
  static __device__ inline C mma(const Frag& w, const Frag& x, C c) {
    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, i32x4{w[0], w[1], w[2], w[3]}),
        __builtin_bit_cast(bf16x8, i32x4{x[0], x[1], x[2], x[3]}), c, 0, 0, 0);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8, i32x4{w[4], w[5], w[6], w[7]}),
        __builtin_bit_cast(bf16x8, i32x4{x[4], x[5], x[6], x[7]}), c, 0, 0, 0);
  }
};
template <> struct Mfma<QK_FP8_BLOCK> : Mfma<QK_FP8> {};
// MXFP4 weights meet bf16 activations in the bf16 MFMA; the decode kernel
// widens each 4-bit weight with its block scale itself (mx_widen8).
template <> struct Mfma<QK_MXFP4> : Mfma<QK_BF16> {};

// Eight E2M1 weights (one dword, low nibble first) times their E8M0 block
// scale, as eight bf16 values (an MFMA operand).  The product of an E2M1
// value (at most two significant bits) and a power of two is exact in bf16.
__device__ inline i32x4 mx_widen8(uint32_t w, float scale) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  i32x4 out;
  out[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 0));
  out[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 1));
  out[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 2));
  out[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, 3));
  return out;
}
// E8M0 code -> 2^(e - 127) as fp32 (codes 1..254; 0 and 255 are outside the
// supported domain).
__device__ inline float e8m0_to_f32(uint32_t e) { return __uint_as_float(e << 23); }

__device__ inline i32x4 lo16(const i32x8& v) { return i32x4{v[0], v[1], v[2], v[3]}; }
__device__ inline i32x4 hi16(const i32x8& v) { return i32x4{v[4], v[5], v[6], v[7]}; }

// ---------------------------------------------------------- conversions
__device__ inline float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ inline float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}
template <bool F16> __device__ inline float h_to_f32(uint32_t b) {
  return F16 ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
}
// fp32 -> 16-bit float, round to nearest even (the hardware conversions).
template <bool F16> __device__ inline uint16_t f32_to_h(float f) {
  if (F16) return __builtin_bit_cast(uint16_t, (_Float16)f);
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// ------------------------------------------- dynamic quantization helpers
// A quantization group (a token row, or a 1x128 block of one) divides every
// value by its scale s = max|x| / QMAX and rounds the binary32 quotient to a
// code.  The quotient must be the correctly rounded x / s.  Rather than a full
// division per value, the group's reciprocal y = RN(1/s) is formed once and
// each quotient takes Markstein's correction (P. Markstein, "Computation of
// elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 34(1), 1990): q = RN(x y), r = x - s q (exact in one FMA), and
// RN(q + r y) = RN(x / s) as long as nothing underflows.  Groups whose
// maximum is below 2^-60 are first scaled by 2^64 (exact; the quotient is
// unchanged), so the residual cannot underflow wherever the quotient is at
// least 2^-12; below that (values that round to a zero code in both formats)
// only the sign is guaranteed, and copysign keeps it.  An exhaustive check
// over every bf16 / fp16 value within a group's maximum, for every third bf16
// maximum and both QMAX, found no difference from the true division.
struct DivBy {
  float s;  // scale, times k
  float y;  // RN(1 / s)
  float k;  // 2^64 or 1
};
__device__ inline DivBy make_div(float s, float amax) {
  DivBy d;
  d.k = amax < 0x1p-60f ? 0x1p64f : 1.f;
  d.s = s * d.k;
  d.y = 1.f / d.s;  // correctly rounded division (the HIP default)
  return d;
}
__device__ inline float div_rn(float x, const DivBy& d) {
  const float xk = x * d.k;
  const float q = __fmul_rn(xk, d.y);
  const float r = __fmaf_rn(-d.s, q, xk);
  return __builtin_copysignf(__fmaf_rn(r, d.y, q), x);
}
// Group scale from its maximum: max / QMAX in binary32, 1 for an all-zero
// group.
__device__ inline float group_scale(float amax, float qmax) {
  return amax > 0.f ? amax / qmax : 1.f;
}

// Codes of 8 values of one group, packed into 8 bytes: e4m3 by the hardware
// conversion (round to nearest even) after an explicit clamp to +-448, int8
// by round-to-nearest-even and a clamp to +-127.
template <bool INT8>
__device__ inline i32x2 quant8(const float* x, const DivBy& d) {
  i32x2 out;
  if constexpr (INT8) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float r = __builtin_rintf(div_rn(x[4 * w + i], d));
        r = fminf(fmaxf(r, -127.f), 127.f);
        word |= ((uint32_t)(int)r & 0xFFu) << (8 * i);
      }
      out[w] = (int)word;
    }
  } else {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = fminf(fmaxf(div_rn(x[4 * w + i], d), -448.f), 448.f);
      int word = __builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false);
      word = __builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], word, true);
      out[w] = word;
    }
  }
  return out;
}

// Eight 16-bit floats of one 16-byte chunk.
template <bool F16>
__device__ inline void unpack8(i32x4 w, float* x) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = h_to_f32<F16>((uint32_t)w[j] & 0xFFFFu);
    x[2 * j + 1] = h_to_f32<F16>((uint32_t)w[j] >> 16);
  }
}

__device__ inline float amax8(const float* x) {
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(x[i]));
  return m;
}

// ----------------------------------------------------------- activations
__device__ inline float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ inline float act_apply(int act, float y) {
  if (act == ACT_RELU) return y > 0.f ? y : 0.f;
  if (act == ACT_GELU_TANH) {
    // 0.5*y*(1 + tanh(u)) == y * sigmoid(2u), u = sqrt(2/pi)*(y + 0.044715*y^3)
    float u = 0.7978845608f * (y + 0.044715f * y * y * y);
    return y * fast_rcp(1.f + __expf(-2.f * u));
  }
  if (act == ACT_SILU) return y * fast_rcp(1.f + __expf(-y));
  return y;
}

// ------------------------------------------------------------ epilogue
// Everything the fused epilogue needs.  scale_mode: 0 = none, 1 = row x col
// (sa[m] * sb[n]), 2 = already applied inside the K loop (block scales).
struct Epi {
  const float* sa;
  const float* sb;
  const uint16_t* bias;      // [N] or null
  const uint16_t* residual;  // [M][N] or null
  void* C;                   // [M][N]
  float alpha;
  int act;
  int raw;                   // store the raw accumulator (test hook)
  int scale_mode;
  int64_t M, N;
};

// The epilogue operands of expert x's rows [r0, r0 + rows) in a grouped
// (mixture-of-experts) layer: the expert's weight scales ([E][N] per
// channel, [E][N/128][KB/128] blocks, or [E][N][KB/16] E8M0 bytes) and bias
// ([E][N]); the rows' activation scales ([M] or [M][KB/128]), residual and
// output ([M][N]).
template <int QK>
__device__ inline Epi grouped_epi(const Epi& e, int64_t x, int64_t r0, int64_t rows, int64_t KB) {
  Epi ec = e;
  const int64_t N = e.N;
  if constexpr (QK == QK_MXFP4) ec.sb = (const float*)((const uint8_t*)e.sb + x * N * (KB / 16));
  else if constexpr (QK == QK_FP8_BLOCK) ec.sb = e.sb + x * (N / 128) * (KB / 128);
  else if (e.sb) ec.sb = e.sb + x * N;
  if (e.bias) ec.bias = e.bias + x * N;
  if (e.sa) ec.sa = e.sa + r0 * (QK == QK_FP8_BLOCK ? KB / 128 : 1);
  if (e.residual) ec.residual = e.residual + r0 * N;
  ec.C = (uint8_t*)e.C + r0 * N * (e.raw ? 4 : 2);
  ec.M = rows;
  return ec;
}

// Load / store G consecutive 16-bit floats (G = 4: 8 bytes, G = 8: 16 bytes).
template <int G, bool F16> __device__ inline void load_h(const uint16_t* p, float* out) {
  if (G == 8) {
    i32x4 b = *(const i32x4*)p;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      out[2 * j] = h_to_f32<F16>((uint32_t)b[j] & 0xFFFFu);
      out[2 * j + 1] = h_to_f32<F16>((uint32_t)b[j] >> 16);
    }
  } else {
    i32x2 b = *(const i32x2*)p;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      out[2 * j] = h_to_f32<F16>((uint32_t)b[j] & 0xFFFFu);
      out[2 * j + 1] = h_to_f32<F16>((uint32_t)b[j] >> 16);
    }
  }
}
template <int G, bool F16> __device__ inline void store_h(uint16_t* p, const float* y) {
  if (G == 8) {
    i32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o[j] = (int)((uint32_t)f32_to_h<F16>(y[2 * j]) | ((uint32_t)f32_to_h<F16>(y[2 * j + 1]) << 16));
    *(i32x4*)p = o;
  } else {
    i32x2 o;
#pragma unroll
    for (int j = 0; j < 2; ++j)
      o[j] = (int)((uint32_t)f32_to_h<F16>(y[2 * j]) | ((uint32_t)f32_to_h<F16>(y[2 * j + 1]) << 16));
    *(i32x2*)p = o;
  }
}

// Epilogue for a run of V consecutive outputs C[m][n0 .. n0+V) of one row,
// from accumulator values v[0..V) (V a multiple of 4).  Vector accesses of
// G = 8 or 4 elements when the run is inside the row and aligned; scalar
// accesses at the right edge or when rows are not aligned.
template <int V, bool F16, typename AccT>
__device__ inline void epilogue_run(const Epi& e, int64_t m, int64_t n0, const AccT* v) {
  static_assert(V % 4 == 0, "run length");
  constexpr int G = (V % 8 == 0) ? 8 : 4;
  if (m >= e.M) return;
  if (e.raw) {
    AccT* crow = (AccT*)e.C + m * e.N;
    for (int i = 0; i < V; ++i)
      if (n0 + i < e.N) crow[n0 + i] = v[i];
    return;
  }
  const bool full = (n0 + V <= e.N) && (e.N % G == 0) && (n0 % G == 0);
  float y[V];
#pragma unroll
  for (int i = 0; i < V; ++i) y[i] = (float)v[i];
  if (e.scale_mode == 1) {
    const float sam = e.sa[m];
    if (full) {
#pragma unroll
      for (int i = 0; i < V; i += 4) {
        f32x4 s = *(const f32x4*)(e.sb + n0 + i);
#pragma unroll
        for (int j = 0; j < 4; ++j) y[i + j] *= sam * s[j];
      }
    } else {
      for (int i = 0; i < V; ++i)
        if (n0 + i < e.N) y[i] *= sam * e.sb[n0 + i];
    }
  }
  if (e.bias) {
    if (full) {
#pragma unroll
      for (int i = 0; i < V; i += G) {
        float b[G];
        load_h<G, F16>(e.bias + n0 + i, b);
#pragma unroll
        for (int j = 0; j < G; ++j) y[i + j] += b[j];
      }
    } else {
      for (int i = 0; i < V; ++i)
        if (n0 + i < e.N) y[i] += h_to_f32<F16>(e.bias[n0 + i]);
    }
  }
#pragma unroll
  for (int i = 0; i < V; ++i) y[i] = act_apply(e.act, y[i]) * e.alpha;
  if (e.residual) {
    const uint16_t* rrow = e.residual + m * e.N;
    if (full) {
#pragma unroll
      for (int i = 0; i < V; i += G) {
        float r[G];
        load_h<G, F16>(rrow + n0 + i, r);
#pragma unroll
        for (int j = 0; j < G; ++j) y[i + j] += r[j];
      }
    } else {
      for (int i = 0; i < V; ++i)
        if (n0 + i < e.N) y[i] += h_to_f32<F16>(rrow[n0 + i]);
    }
  }
  uint16_t* crow = (uint16_t*)e.C + m * e.N;
  if (full) {
#pragma unroll
    for (int i = 0; i < V; i += G) store_h<G, F16>(crow + n0 + i, y + i);
  } else {
    for (int i = 0; i < V; ++i)
      if (n0 + i < e.N) crow[n0 + i] = f32_to_h<F16>(y[i]);
  }
}

// Epilogue for one output element (used by the generic reduction paths).
template <bool F16, typename AccT>
__device__ inline void epilogue_one(const Epi& e, int64_t m, int64_t n, AccT v) {
  if (m >= e.M || n >= e.N) return;
  if (e.raw) { ((AccT*)e.C)[m * e.N + n] = v; return; }
  float y = (float)v;
  if (e.scale_mode == 1) y *= e.sa[m] * e.sb[n];
  if (e.bias) y += h_to_f32<F16>(e.bias[n]);
  y = act_apply(e.act, y) * e.alpha;
  if (e.residual) y += h_to_f32<F16>(e.residual[m * e.N + n]);
  ((uint16_t*)e.C)[m * e.N + n] = f32_to_h<F16>(y);
}

// The epilogue operands of a 4-column run C[m][n0 .. n0+4), loaded ahead of
// time (at kernel start) so the loads' latency overlaps the K loop instead of
// following it.  Bias and residual stay as raw 16-bit pairs (low half first)
// until the epilogue widens them: widening at load time would make the wave
// wait for the loads right there.
struct EpiPre4 {
  float sam;
  float sb[4];
  uint32_t bias[2], res[2];
};
// Value i of a raw pair array (bias or residual).
template <bool F16> __device__ inline float pre_h(const uint32_t* w, int i) {
  return h_to_f32<F16>((w[i >> 1] >> (16 * (i & 1))) & 0xFFFFu);
}

template <bool F16>
__device__ inline void epilogue_prefetch4(const Epi& e, int64_t m, int64_t n0, EpiPre4& p) {
  const int64_t mm = m < e.M ? m : e.M - 1;
  const bool full = (n0 + 4 <= e.N) && (e.N % 4 == 0) && (n0 % 4 == 0);
  p.sam = 1.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) p.sb[i] = 1.f;
  p.bias[0] = p.bias[1] = p.res[0] = p.res[1] = 0u;  // +0
  if (e.raw) return;
  if (e.scale_mode == 1) {
    if (e.sa) p.sam = e.sa[mm];  // (no sa: the kernel derives it from its activations)
    if (full) {
      const f32x4 s = *(const f32x4*)(e.sb + n0);
#pragma unroll
      for (int i = 0; i < 4; ++i) p.sb[i] = s[i];
    } else {
      for (int i = 0; i < 4; ++i) if (n0 + i < e.N) p.sb[i] = e.sb[n0 + i];
    }
  }
  auto raw4 = [&](const uint16_t* row, uint32_t* w) {
    if (full) {
      const i32x2 b = *(const i32x2*)(row + n0);
      w[0] = (uint32_t)b[0];
      w[1] = (uint32_t)b[1];
    } else {
      for (int i = 0; i < 4; ++i)
        if (n0 + i < e.N) w[i >> 1] |= (uint32_t)row[n0 + i] << (16 * (i & 1));
    }
  };
  if (e.bias) raw4(e.bias, p.bias);
  if (e.residual) raw4(e.residual + mm * e.N, p.res);
}

// Epilogue of a 4-column run from prefetched operands (same arithmetic and
// order as epilogue_run).
template <bool F16, typename AccT>
__device__ inline void epilogue_run4_pre(const Epi& e, int64_t m, int64_t n0, const AccT* v,
                                         const EpiPre4& p) {
  if (m >= e.M) return;
  if (e.raw) {
    AccT* crow = (AccT*)e.C + m * e.N;
    for (int i = 0; i < 4; ++i)
      if (n0 + i < e.N) crow[n0 + i] = v[i];
    return;
  }
  float y[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    y[i] = (float)v[i];
    if (e.scale_mode == 1) y[i] *= p.sam * p.sb[i];
    y[i] += pre_h<F16>(p.bias, i);
    y[i] = act_apply(e.act, y[i]) * e.alpha + pre_h<F16>(p.res, i);
  }
  uint16_t* crow = (uint16_t*)e.C + m * e.N;
  if ((n0 + 4 <= e.N) && (e.N % 4 == 0) && (n0 % 4 == 0)) {
    store_h<4, F16>(crow + n0, y);
  } else {
    for (int i = 0; i < 4; ++i)
      if (n0 + i < e.N) crow[n0 + i] = f32_to_h<F16>(y[i]);
  }
}

}  // namespace lg
