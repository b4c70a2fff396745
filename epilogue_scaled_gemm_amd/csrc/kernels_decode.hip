// kernels_decode.hip -- small-M (decode) family: M <= 32 tokens against a
// large weight, which is streamed from HBM exactly once.
//
// The variants are the two of "helion-vllm-linear-backend" (section "Зачем
// трогать линейные слои"): split-K -- K divided among several workgroups /
// waves to add parallelism when M and N cannot fill the GPU -- and swap-AB
// -- computing (B A^T)^T so that the wide weight dimension takes the tiled
// side; plus the scale formats of its section "Одно ядро вместо трёх
// вариантов".  The variant per shape comes from a table (its sections "Одно
// ядро вместо трёх вариантов" and "Гибридный диспатч").
//
// gfx950 design:
//  * A workgroup owns 16*rows weight rows and a slice of K; its W waves split
//    that slice into contiguous runs of 128-byte steps (in-workgroup
//    split-K), so each weight byte is loaded by exactly one lane, straight
//    from HBM into registers with buffer loads over the workgroup's rows (no
//    LDS staging: there is no reuse to stage for).  Every lane loads 32 contiguous bytes per step; 4 lanes cover a
//    128-byte line; each activation slice feeds all 16*rows weight rows.
//  * A wave issues the loads of up to U steps at once (U * 2 KiB of weight),
//    then consumes them; with the wave counts used, every weight byte of the
//    call is requested at kernel start.
//  * swap = 1 puts the weight on the MFMA row side (tokens are columns): each
//    lane ends with 4 consecutive output columns of one token (8-byte
//    stores).  swap = 0 puts tokens on the row side (the direct A*B^T form).
//  * With swap and W = 8 or 12, one more wave loads the epilogue operands (scales, bias,
//    residual) into LDS while the others stream the weight, so no wave that
//    loads weights waits on them, and the epilogue reads them from LDS.
//  * Tokens past M re-read token M-1 and their outputs are dropped; tokens
//    use one or two 16-column MFMA tiles (M <= 16 or M <= 32).
//  * Partial sums of the W waves are reduced in LDS in a fixed order.  With
//    split > 1 workgroups per row group the cross-workgroup reduction is one
//    of: lastwg (each writes its partial to workspace [split][M][N]; the last
//    to arrive on a per-group counter sums them in slice order, runs the
//    epilogue and resets the counter), atomic (atomic adds into a zeroed
//    [M][N] accumulator; the last arrival runs the epilogue and re-zeroes
//    it; exact for int32, order-dependent rounding for fp32) or twopass
//    (partials, then splitk_reduce sums them in slice order).  The nonlinear
//    epilogue always runs on the complete sum.
#include <algorithm>
#include <mutex>
#include <type_traits>
#include <unordered_map>

#include "launch.hpp"

namespace lg {
namespace {

constexpr int STEPB = 128;  // bytes of K per step

template <typename T> __device__ inline T ld_agent(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T> __device__ inline void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16-byte load that is always issued (the address is valid whatever `ok`
// says) and then zeroed when `ok` is false: straight-line code, so the
// compiler knows how many loads are outstanding and can wait for one batch
// while the next is in flight.
__device__ inline i32x4 ld16(const uint8_t* p, bool ok) {
  const i32x4 v = *(const i32x4*)p;
  return ok ? v : i32x4{0, 0, 0, 0};
}

__device__ inline i32x8 cat(i32x4 a, i32x4 b) {
  return i32x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Whether a variant has the operand wave: with swap and 8 or 12 K waves.  A
// workgroup holds at most 16 waves; with 4 K waves the extra wave's share of
// the CU's wave slots cost more than it saved, and those variants prefetch
// the operands in the owning waves instead.
constexpr bool op_wave(bool swap, int w) { return swap && w >= 8 && w < 16; }

// Activation modes (the kernel's last template argument AM):
//  AM_GLOBAL  every lane loads its activation fragments from global memory.
//  AM_STAGE   per step, a wave copies the M tokens' activation bytes it needs
//             into its own slice of LDS with direct-to-LDS buffer loads (one
//             16-byte chunk per lane, only the lanes that hold distinct data
//             in range; one load covers 1 KiB), and the lanes read their
//             fragments from there.  The lanes of a token tile share tokens
//             (16 lanes per token at M = 1), so this replaces up to 16
//             redundant global loads per distinct chunk by LDS broadcasts.
//             Swap orientation.
//  AM_QUANT   the quantization prologue below.
//  AM_WIDEN   e4m3 activations, swap, one token tile: each wave widens the
//             activations of its whole K range once, all M tokens at a
//             time, to bf16 in its own slice of LDS (the activation loads
//             are issued before the first weight batch, so they return
//             first), and the lanes read ready-made bf16 fragments from
//             there.  With fewer than 16 tokens the 16 lanes of a token tile
//             hold copies of the same tokens, so per-lane widening repeats
//             the same conversions up to 16 times; here each activation
//             byte is widened once per wave.  Chunks outside the wave's
//             range or past K are stored as zeros.
//  AM_QWIDEN  AM_WIDEN on bf16 activations X[M][K] with per-token dynamic
//             e4m3 quantization fused in (the prologue fusion of the pages'
//             input-side transforms): each wave loads the bf16 values of its
//             K range, takes every token's partial maximum, the workgroup
//             combines them through LDS (one barrier; the waves together
//             cover all of K, split 1), and each wave then forms the scale,
//             the codes (those of lin_gemm_quantize, bit for bit) and their
//             exact bf16 widening in its slice.  The epilogue takes the
//             per-token scale from LDS.
//
// AM_QUANT: A holds bf16 activations X[M][K] instead of codes, and the kernel
// quantizes them itself in a prologue (swap, one token tile, split 1): the
// whole workgroup reads its tokens' rows once, takes each group's maximum
// (per token, or per 1x128 block), and writes the codes to LDS
// (dynamic shared memory: M rows of KB + 16 bytes, then the scales), while
// the first weight batch is already in flight.  The K loop then reads its
// activation fragments from LDS, and the epilogue takes the per-token scale
// from there.  Codes and scales are those of lin_gemm_quantize.
enum : int { AM_GLOBAL = 0, AM_QUANT = 1, AM_STAGE = 2, AM_WIDEN = 3, AM_WIDEN2 = 4,
             AM_WIDEN4 = 5, AM_WIDEN8 = 6, AM_QWIDEN = 7, AM_QWIDEN2 = 8, AM_QWIDEN4 = 9,
             AM_QWIDEN8 = 10 };
// AM_WIDEN .. AM_WIDEN8: the widened mode with one, two, four or eight
// 16-byte activation chunks per lane (the launch picks the smallest that
// holds the wave's M x slice: a load whose lanes are all out of range still
// costs a pass through the memory pipeline; the loads stay straight-line, so
// each chunk is widened as soon as it lands).  AM_QWIDEN .. AM_QWIDEN8: the
// same with bf16 activations quantized per token in the prologue (below).
constexpr bool am_widen(int am) { return am >= AM_WIDEN; }
constexpr bool am_qwiden(int am) { return am >= AM_QWIDEN; }

// s_waitcnt immediate for "vmcnt <= n" (expcnt and lgkmcnt not waited).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int wd_rounds(int am) { return am >= AM_WIDEN ? 1 << ((am - AM_WIDEN) % 4) : 1; }
typedef __attribute__((address_space(3))) void lds_void;
constexpr int DQ_CHUNKS = 4;  // 16-byte activation chunks per thread kept in registers
constexpr int WD_ROUNDS = 8;  // widened mode: 16-byte activation chunks per lane, at most

// AM_WIDEN layout: per wave, per token, WST steps (a power of two) of 256
// bytes of bf16 (the 128 K values of a step).  A pair of steps is one
// 512-byte window; 16-byte piece p of step t of token tok sits at window
// position ((t & 1) * 16 + p) ^ wd_swz(tok).  A fragment read takes the same
// piece of the same step for 16 tokens and two lane groups (pieces 4 apart):
// the swizzle keeps bit 2 and spreads the tokens over the other four bits,
// so the 32 addresses of a half-wave fall in distinct 16-byte bank groups.
__device__ inline int wd_swz(int tok) { return (tok & 3) | ((tok & 12) << 1); }
// Steps per wave a slice of `per` steps reserves: the smallest power of two
// that holds them and at least two steps and one batch (U is a power of two).
__host__ __device__ inline int wd_steps(int per, int U) {
  int n = U > 2 ? U : 2;
  while (n < per) n *= 2;
  return n;
}

// The quantization prologue, run by every thread of the workgroup.  X[M][K]
// is contiguous, so chunk c (8 values) of the M x K region sits at X + 8c, in
// row c / (K/8).  Per-token groups take their maximum through LDS atomics
// (one barrier); 1x128 blocks are 16 consecutive chunks, i.e. 16 consecutive
// lanes, and take theirs by a 16-lane shuffle.  Scales go to sal, codes to
// xq (row stride LS).  Ends with a barrier, after which xq and sal are
// complete.
template <int QK>
__device__ inline void quant_prologue(const uint16_t* __restrict__ X, int64_t M, int64_t K,
                                      float* sal, uint8_t* xq, int64_t LS) {
  constexpr bool BLOCK = QK == QK_FP8_BLOCK;
  constexpr bool INT8 = QK == QK_I8;
  constexpr float QMAX = INT8 ? 127.f : 448.f;
  const int tid = threadIdx.x;
  const int nthr = blockDim.x;
  const uint32_t cpr = (uint32_t)(K / 8);
  const uint32_t nchunk = (uint32_t)M * cpr;
  i32x4 xc[DQ_CHUNKS];
#pragma unroll
  for (int j = 0; j < DQ_CHUNKS; ++j) {
    // chunks past the region re-read its last chunk and are never stored
    const uint32_t c = min((uint32_t)(tid + j * nthr), nchunk - 1);
    if ((uint32_t)(j * nthr) < nchunk) xc[j] = *(const i32x4*)(X + (size_t)c * 8);
    else xc[j] = i32x4{0, 0, 0, 0};
  }
  auto store = [&](uint32_t c, const float* v, const DivBy& d) {
    const uint32_t m = c / cpr;
    *(i32x2*)(xq + m * LS + (int64_t)(c - m * cpr) * 8) = quant8<INT8>(v, d);
  };
  if constexpr (BLOCK) {
    const uint32_t kblk = (uint32_t)(K / 128);
    auto one = [&](uint32_t c, i32x4 w) {
      float v[8];
      unpack8<false>(w, v);
      float am = amax8(v);
#pragma unroll
      for (int off = 8; off > 0; off >>= 1) am = fmaxf(am, __shfl_xor(am, off, 16));
      if (c < nchunk) {
        const float sc = group_scale(am, QMAX);
        store(c, v, make_div(sc, am));
        const uint32_t m = c / cpr, k8 = c - m * cpr;
        if ((k8 & 15) == 0) sal[m * kblk + k8 / 16] = sc;
      }
    };
#pragma unroll
    for (int j = 0; j < DQ_CHUNKS; ++j) one((uint32_t)(tid + j * nthr), xc[j]);
    for (uint32_t cb = (uint32_t)(DQ_CHUNKS * nthr); cb < nchunk; cb += (uint32_t)nthr) {
      const uint32_t c = cb + (uint32_t)tid;
      one(c, *(const i32x4*)(X + (size_t)min(c, nchunk - 1) * 8));
    }
  } else {
    uint32_t* amax_u = (uint32_t*)(sal + M);
    if (tid < M) amax_u[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < DQ_CHUNKS; ++j) {
      const uint32_t c = (uint32_t)(tid + j * nthr);
      if (c < nchunk) {
        float v[8];
        unpack8<false>(xc[j], v);
        atomicMax(&amax_u[c / cpr], __float_as_uint(amax8(v)));
      }
    }
    for (uint32_t c = (uint32_t)(tid + DQ_CHUNKS * nthr); c < nchunk; c += (uint32_t)nthr) {
      float v[8];
      unpack8<false>(*(const i32x4*)(X + (size_t)c * 8), v);
      atomicMax(&amax_u[c / cpr], __float_as_uint(amax8(v)));
    }
    __syncthreads();
    auto one = [&](uint32_t c, i32x4 w) {
      const float am = __uint_as_float(amax_u[c / cpr]);
      float v[8];
      unpack8<false>(w, v);
      store(c, v, make_div(group_scale(am, QMAX), am));
    };
#pragma unroll
    for (int j = 0; j < DQ_CHUNKS; ++j) {
      const uint32_t c = (uint32_t)(tid + j * nthr);
      if (c < nchunk) one(c, xc[j]);
    }
    for (uint32_t c = (uint32_t)(tid + DQ_CHUNKS * nthr); c < nchunk; c += (uint32_t)nthr)
      one(c, *(const i32x4*)(X + (size_t)c * 8));
    if (tid < M) sal[tid] = group_scale(__uint_as_float(amax_u[tid]), QMAX);
  }
  __syncthreads();
}

// The body of the decode kernel: workgroup blockIdx.x owns weight rows
// [blockIdx.x * rpw, + rpw) and K slice sidx of `split`.
template <int QK, int NTT, bool SWAP, int W, int U, int RT, int AM>
__device__ __forceinline__ void decode_body(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, int64_t M, int64_t N,
    int64_t KB, int rpw, int split, int sidx, int steps_per_split, int reduce, Epi e,
    void* __restrict__ ws, int* __restrict__ counters) {
  using MF = Mfma<QK>;
  using C = typename MF::C;
  using AccT = typename QTraits<QK>::Acc;
  constexpr bool F16 = QTraits<QK>::out_f16;
  constexpr bool BLOCK = (QK == QK_FP8_BLOCK);
  // MXFP4 weights: 4-bit codes (KB = K/2 bytes per weight row) with an E8M0
  // scale per 32 K values, against bf16 activations (XR = 4 activation bytes
  // per weight byte).  A step is 128 weight bytes = 256 K values; a lane's
  // 32 bytes are two 32-value scale blocks.  Swap only; K % 256 == 0.
  constexpr bool MX = (QK == QK_MXFP4);
  constexpr int XR = MX ? 4 : 1;
  constexpr bool DQ = AM == AM_QUANT;
  constexpr bool XS = AM == AM_STAGE;
  constexpr bool WD = am_widen(AM);
  constexpr bool QW = am_qwiden(AM);
  constexpr int WDR = wd_rounds(AM);
  static_assert(!QW || QK == QK_FP8, "the fused quantization is per-token e4m3");
  static_assert(!WD || (SWAP && NTT == 1 && (QK == QK_FP8 || QK == QK_FP8_BLOCK)),
                "widened activations: e4m3, swap, one token tile");
  static_assert(!MX || (SWAP && !DQ), "MXFP4 weights use the swap orientation");
  static_assert(!XS || SWAP, "staged activations are for the swap orientation");
  constexpr int NS = SWAP ? 1 : 4;    // block scales per token tile per lane
  constexpr int NTILE = RT * NTT;     // 16x16 output tiles per workgroup
  // Partial sums of the W waves for the in-workgroup reduction.  With staged
  // or widened activations each wave writes its own into its LDS slice (done
  // with it by then; slices are sized to hold them), so the static array is
  // not needed.
  constexpr bool RA = XS || am_widen(AM);
  __shared__ __align__(16) AccT red[RA ? 1 : W][NTILE * 64 * 4];
  // A lane's four partial sums of a tile sit together (one 16-byte LDS
  // access each way): element r of tile q, lane l at (q * 64 + l) * 4 + r.
  typedef AccT AccT4 __attribute__((ext_vector_type(4)));
  // Epilogue operands per tile and lane: sa, sb[4], then bias and residual
  // as two raw 16-bit pairs each, staged by the operand wave.
  constexpr bool OPW = op_wave(SWAP, W);
  constexpr int NOP = 9;
  __shared__ float opnd[OPW ? NTILE : 1][NOP][64];
  __shared__ int arrival;
  // AM_QWIDEN: per-wave partial maxima and the scales of up to 16 tokens.
  __shared__ float qw_max[QW ? W : 1][QW ? 16 : 1];
  __shared__ float qw_scale[QW ? 16 : 1];
  extern __shared__ __align__(16) uint8_t dq_lds[];
  static_assert(!DQ || (SWAP && NTT == 1), "the quantization prologue is for swap, one token tile");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Wave W (one past the K waves), if present, is the operand wave: it loads
  // no weights, only the epilogue operands of the workgroup's tiles, which
  // it stages in LDS while the K waves stream the weight.
  const bool opw = OPW && wave == W;
  const int g = lane >> 4, l16 = lane & 15;
  // This workgroup's weight rows are [n0, n0 + rpw) (rpw <= 16 * RT, a
  // multiple of 4); rows of its MFMA tiles past that are masked.
  const int64_t n0 = (int64_t)blockIdx.x * rpw;
  const int64_t nend = min(n0 + rpw, N);
  const int total_steps = (int)((KB + STEPB - 1) / STEPB);
  const int beg = sidx * steps_per_split;
  const int end = min(beg + steps_per_split, total_steps);
  const int span = end - beg;
  // Wave w takes a contiguous run of steps [first, first + my) of the slice.
  const int per = (span + W - 1) / W;
  const int first = beg + wave * per;
  const int my = max(0, min(per, end - first));  // steps of this wave

  // Weight loads are buffer loads over this workgroup's rows [n0, nend)
  // (at most 64 rows of at most 8 MiB): a lane's 16-byte chunk sits at
  // wlb[rt] + st * STEPB (+16); rows past nend are out of range, and chunks
  // past the end of a row and steps past the wave's range are given an
  // out-of-range offset, so all of them read zeros without a memory access.
  const __amdgpu_buffer_rsrc_t wrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(B + n0 * KB), (short)0, (int)((nend - n0) * KB), 0x00020000);
  int wlb[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) wlb[rt] = (rt * 16 + l16) * (int)KB + g * 32;
  auto wload = [&](int rt, int st, bool live) {
    const int o0 = st * STEPB + g * 32;
    const int b = wlb[rt] + st * STEPB;
    const int off0 = live && o0 < KB ? b : 0x7FFFFFF0;
    const int off1 = live && o0 + 16 < KB ? b + 16 : 0x7FFFFFF0;
    return cat(__builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off0, 0, 0)),
               __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(wrs, off1, 0, 0)));
  };
  const uint8_t* xp[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt)
    xp[tt] = A + min((int64_t)(tt * 16 + l16), M - 1) * KB * XR + g * 32 * XR;
  // MXFP4: E8M0 scale bytes [N][KB/16]; a lane's two blocks of a step are
  // bytes st*8 + 2g and st*8 + 2g + 1 of its row.
  const uint8_t* msp[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int64_t row = n0 + rt * 16 + l16;
    msp[rt] = MX ? (const uint8_t*)e.sb + (row < nend ? row : n0) * (KB / 16) + 2 * g : nullptr;
  }
  // With DQ: the codes in LDS (row stride KB + 16) and the scales after them
  // (sal[M] per token, or sal[M][KB / 128] per block).
  const int64_t LS = KB + 16;
  float* sal = (float*)(dq_lds + M * LS);
  const uint8_t* xl[NTT];
#pragma unroll
  for (int tt = 0; tt < NTT; ++tt) xl[tt] = dq_lds + min((int64_t)(tt * 16 + l16), M - 1) * LS + g * 32;
  // With AM_STAGE: this wave's LDS slice holds, per batch step u, the M
  // tokens' activation bytes of the step (XSB bytes each, token-major), in
  // XSL bytes: whole KiB, since every direct-to-LDS load writes 64 x 16
  // bytes (lanes out of range write zeros).
  constexpr int XSB = STEPB * XR;
  const int xs_chunks = (int)M * (XSB / 16);  // 16-byte chunks per step
  // With 8 pieces of 16 bytes per token and step, piece p of token t sits at
  // position p ^ xsw(t): the 16 lanes that read one piece of 16 tokens (and
  // the 32 lanes of two lane groups) then hit distinct bank groups instead
  // of the same few (token rows are 128 bytes apart).
  constexpr bool XSW = XSB == 128;
  constexpr bool XS_FIRST = U == 1 || W >= 8;  // activation loads first (below)
  auto xsw = [](int t) { return XSW ? (t & 7) ^ (((t >> 3) & 1) * 7) : 0; };
  const int XSL = (xs_chunks + 63) / 64 * 1024;
  // A wave's slice: U steps, and at least its NTILE KiB of partial sums.
  const int XSS = max(U * XSL, NTILE * 1024);
  uint8_t* xsl = dq_lds + (int64_t)wave * XSS;
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, XS ? (int)(M * KB * XR) : 0, 0x00020000);
  bool xok[U][2];
  // With AM_WIDEN: this wave's slice, WST steps of 256 bytes per token.
  const int WST = wd_steps((steps_per_split + W - 1) / W, U);
  const int wd_sh = 31 - __builtin_clz(WST * 8);  // chunks per token = 1 << wd_sh
  const int64_t WSS = max((int64_t)M * WST * 256, (int64_t)NTILE * 1024);  // slice stride
  uint8_t* wdl = dq_lds + (int64_t)wave * WSS;

  // Block scales: sb[n0/128][kb] is uniform over the workgroup; sa[tok][kb]
  // per lane (one token per tile with swap, four without).
  const int64_t KBLK = KB / 128;
  const float* sa_p[NTT][NS];
  const float* sb_p = nullptr;
  if constexpr (BLOCK) {
    sb_p = e.sb + (n0 / 128) * KBLK;
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
      for (int r = 0; r < NS; ++r) {
        const int64_t tok = SWAP ? (tt * 16 + l16) : (tt * 16 + g * 4 + r);
        sa_p[tt][r] = DQ ? nullptr : e.sa + min(tok, M - 1) * KBLK;
      }
  }

  struct XMX { i32x4 v[8]; };  // 64 bf16 activations per lane per step (MXFP4)
  using XB = typename std::conditional<MX, XMX, i32x8>::type;
  i32x8 wb[U][RT];
  XB xb[U][NTT];
  float sc[U][NTT][NS];
  uint32_t msc[U][RT];
  // Issue a whole batch of U steps' loads (straight-line, always in bounds),
  // then consume it.  A wave's steps usually fit one batch, so every load of
  // the kernel is in flight at once and each MFMA waits only for its own
  // step.  Each activation slice feeds RT weight tiles.
  // part: 0 = weights and activations, 1 = weights only, 2 = activations
  // (and block scales) only.
  // Weight (and MXFP4 scale) loads of step u.
  auto load_weights = [&](int t0, int u) {
    const int t = t0 + u;
    const bool live = t < my;
    const int st = min(first + (live ? t : 0), total_steps - 1);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) wb[u][rt] = wload(rt, st, live);
    if constexpr (MX) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) msc[u][rt] = *(const uint16_t*)(msp[rt] + (int64_t)st * 8);
    }
  };
  // Direct-to-LDS activation loads of step u: one per 64 chunks, chunk q
  // (token q / (XSB/16), piece q % (XSB/16)) landing at byte 16 q of the
  // step's slice; lanes past the last chunk get an out-of-range offset (no
  // access).  XSB / 16 divides 64, so chunk 64 i + lane is token
  // i * 64 / (XSB/16) + lane / (XSB/16), piece lane % (XSB/16), and the
  // piece's swizzled position depends on i only through its parity: the lane
  // part of the offset is computed once, for even and for odd i.
  constexpr int CPT = XSB / 16, TPI = 64 / CPT;
  static_assert(64 % CPT == 0 && (!XSW || TPI == 8), "staged chunk layout");
  int xlb[2];
#pragma unroll
  for (int p = 0; p < 2; ++p)
    xlb[p] = (lane / CPT) * (int)(KB * XR) + (((lane % CPT) ^ xsw(lane / CPT + p * TPI)) << 4);
  auto stage_step = [&](int t0, int u) {
    const int t = t0 + u;
    const bool live = t < my;
    const int st = min(first + (live ? t : 0), total_steps - 1);
    const int64_t o0 = (int64_t)st * STEPB + g * 32;
    xok[u][0] = live && (o0 < KB);
    xok[u][1] = live && (o0 + 16 < KB);
    for (int i = 0; i * 64 < xs_chunks; ++i) {
      const int voff = i * 64 + lane < xs_chunks
                           ? xlb[i & 1] + i * TPI * (int)(KB * XR) + st * XSB
                           : 0x7FFFFFF0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xrs, (lds_void*)(xsl + (int64_t)u * XSL + i * 1024), 16, voff, 0, 0, 0);
    }
  };
  auto load_batch = [&](int t0, int part = 0) {
    if constexpr (XS) {
      // A batch issues its steps' activation loads before their weights:
      // loads complete in issue order, so the staged fragments are read
      // while the weights are still in flight.  With 4 waves a batch spans
      // more of K, and its first weights would wait behind all of its
      // activation loads (1-2% slower for int8 at 4-16 tokens): those
      // batches keep step order and wait for everything.
      if constexpr (XS_FIRST) {
#pragma unroll
        for (int u = 0; u < U; ++u) stage_step(t0, u);
#pragma unroll
        for (int u = 0; u < U; ++u) load_weights(t0, u);
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
          load_weights(t0, u);
          stage_step(t0, u);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u;
      const bool live = t < my;
      // Per-lane activation loads: steps past this wave's range re-read a
      // step inside the row (its first, clamped to the last step of K) and
      // are zeroed; chunks past the end of the row re-read the row's last 16
      // bytes and are zeroed.
      const int st = min(first + (live ? t : 0), total_steps - 1);
      const int64_t off = (int64_t)st * STEPB;
      const int64_t o0 = off + g * 32, o1 = o0 + 16;
      const bool ok0 = live && (o0 < KB);
      const bool ok1 = live && (o1 < KB);
      const int64_t c0 = (o0 < KB ? o0 : KB - 16) - g * 32;
      const int64_t c1 = (o1 < KB ? o1 : KB - 16) - g * 32;
      if (part != 2 && !XS) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) wb[u][rt] = wload(rt, st, live);
      }
      if constexpr (MX && !XS) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) msc[u][rt] = *(const uint16_t*)(msp[rt] + (int64_t)st * 8);
      }
      if (part == 1) continue;
      if constexpr (WD || XS) {
        // activations come from LDS (the widened slice, or staged above)
      } else if constexpr (MX) {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
          for (int j = 0; j < 8; ++j)
            xb[u][tt].v[j] = ld16(xp[tt] + 4 * c0 + 16 * j, j < 4 ? ok0 : ok1);
      } else if constexpr (DQ) {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
          xb[u][tt] = cat(ld16(xl[tt] + c0, ok0), ld16(xl[tt] + c1, ok1));
      } else {
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
          xb[u][tt] = cat(ld16(xp[tt] + c0, ok0), ld16(xp[tt] + c1, ok1));
      }
      if constexpr (BLOCK && DQ) {
        const float sbv = live ? sb_p[st] : 0.f;
        const int64_t tok = min((int64_t)l16, M - 1);
        sc[u][0][0] = live ? sal[tok * KBLK + st] * sbv : 0.f;
      } else if constexpr (BLOCK) {
        const float sbv = live ? sb_p[st] : 0.f;
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt)
#pragma unroll
          for (int r = 0; r < NS; ++r) sc[u][tt][r] = live ? sa_p[tt][r][st] * sbv : 0.f;
      }
    }
  };

  C acc[RT][NTT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) acc[rt][tt] = C{0, 0, 0, 0};

  // With AM_STAGE: step u's fragments from the wave's LDS slice, once its
  // direct-to-LDS loads have landed.
  auto read_staged = [&](int u) {
#pragma unroll
    for (int tt = 0; tt < NTT; ++tt) {
      const int64_t tok = min((int64_t)(tt * 16 + l16), M - 1);
      if constexpr (MX) {
        const uint8_t* xr = xsl + (int64_t)u * XSL + tok * XSB + g * 32 * XR;
#pragma unroll
        for (int j = 0; j < 8; ++j)
          xb[u][tt].v[j] = ld16(xr + 16 * j, j < 4 ? xok[u][0] : xok[u][1]);
      } else {
        const uint8_t* xt = xsl + (int64_t)u * XSL + tok * XSB;
        const int sw = xsw((int)tok);
        xb[u][tt] = cat(ld16(xt + (((2 * g) ^ sw) << 4), xok[u][0]),
                        ld16(xt + (((2 * g + 1) ^ sw) << 4), xok[u][1]));
      }
    }
  };
  // A staged batch: its fragments once its direct-to-LDS loads have landed;
  // issued first, they leave at most the batch's weight loads (two per row
  // tile and step, plus the MXFP4 scale load) in flight behind them, else
  // the batch waits for all of its loads.
  auto stage_batch = [&]() {
    if constexpr (XS) {
      static_assert(!XS_FIRST || U * (MX ? 3 : 2) * RT <= 63, "vmcnt range");
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(XS_FIRST ? U * (MX ? 3 : 2) * RT : 0));
#pragma unroll
      for (int u = 0; u < U; ++u) read_staged(u);
    }
  };

  // With AM_WIDEN: the bf16 fragment of piece pair (2c, 2c+1) of lane group
  // g, step t of the wave's slice, token tok.
  auto wide_frag = [&](int t, int c, int64_t tok) {
    const uint8_t* base = wdl + tok * WST * 256 + (t & ~1) * 256;
    const int sw = wd_swz((int)tok), p0 = (t & 1) * 16 + 4 * g + 2 * c;
    const i32x4 a = *(const i32x4*)(base + ((p0 ^ sw) << 4));
    const i32x4 b = *(const i32x4*)(base + (((p0 + 1) ^ sw) << 4));
    return cat(a, b);
  };

  auto compute_batch = [&](int t0) {
    (void)t0;
    stage_batch();
    if constexpr (MX) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float s0 = e8m0_to_f32(msc[u][rt] & 0xFFu), s1 = e8m0_to_f32(msc[u][rt] >> 8);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const i32x4 w = mx_widen8((uint32_t)wb[u][rt][j], j < 4 ? s0 : s1);
#pragma unroll
            for (int tt = 0; tt < NTT; ++tt) acc[rt][tt] = MF::mma(w, xb[u][tt].v[j], acc[rt][tt]);
          }
        }
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        typename MF::Frag x0[NTT], x1[NTT];
#pragma unroll
        for (int tt = 0; tt < NTT; ++tt) {
          if constexpr (WD) {
            const int64_t tok = min((int64_t)(tt * 16 + l16), M - 1);
            x0[tt] = wide_frag(t0 + u, 0, tok);
            x1[tt] = wide_frag(t0 + u, 1, tok);
          } else {
            x0[tt] = MF::prep(lo16(xb[u][tt]));
            x1[tt] = MF::prep(hi16(xb[u][tt]));
          }
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const typename MF::Frag w0 = MF::prep(lo16(wb[u][rt])), w1 = MF::prep(hi16(wb[u][rt]));
#pragma unroll
          for (int tt = 0; tt < NTT; ++tt) {
            if constexpr (BLOCK) {
              // One step is one 128-wide K block: scale its exact partial sum.
              C p = SWAP ? MF::mma(w0, x0[tt], C{0, 0, 0, 0}) : MF::mma(x0[tt], w0, C{0, 0, 0, 0});
              p = SWAP ? MF::mma(w1, x1[tt], p) : MF::mma(x1[tt], w1, p);
#pragma unroll
              for (int r = 0; r < 4; ++r) acc[rt][tt][r] += sc[u][tt][SWAP ? 0 : r] * p[r];
            } else {
              C a = acc[rt][tt];
              a = SWAP ? MF::mma(w0, x0[tt], a) : MF::mma(x0[tt], w0, a);
              acc[rt][tt] = SWAP ? MF::mma(w1, x1[tt], a) : MF::mma(x1[tt], w1, a);
            }
          }
        }
      }
    }
  };

  // The first batch is issued before anything else, so the weight stream
  // starts at once (a wave with no steps issues out-of-range weight loads,
  // which read zeros and add nothing).
  // Without the operand wave, each swap wave prefetches the operands of the
  // tiles it will finish (q = wave, wave + W, ...) right behind its first
  // batch.
  const bool fin_here = split == 1 || reduce != R_TWOPASS;
  constexpr int QPW = (NTILE + W - 1) / W;  // tiles per wave, at most
  EpiPre4 pre[SWAP && !OPW ? QPW : 1];
  if constexpr (DQ) {
    if (!opw) load_batch(0, 1);
    quant_prologue<QK>((const uint16_t*)A, M, KB, sal, dq_lds, LS);
  }
  // AM_WIDEN: issue this wave's activation loads (chunk q = lane + 64 r:
  // token q / (8 WST), 16-byte chunk q % (8 WST) of the slice), then the
  // first weight batch, then widen and store (the activation loads were
  // issued first, so only they are waited for).  Buffer loads: a lane
  // without a chunk in range gets an offset past the buffer, which reads
  // zeros and touches no memory (every wave of the grid reads the same few
  // activation lines; dummy loads would pile up on one of them).
  i32x4 wdv[WD ? WDR : 1];
  const int wd_chunks = WD ? (int)M * WST * 8 : 0;
  if constexpr (WD && !QW) {
    if (!opw) {
      const __amdgpu_buffer_rsrc_t ars =
          __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)(M * KB), 0x00020000);
#pragma unroll
      for (int r = 0; r < WDR; ++r) {
        const int q = lane + 64 * r;
        const int tok = q >> wd_sh, j = q & ((1 << wd_sh) - 1);
        const int64_t kb = (int64_t)(first) * STEPB + (int64_t)j * 16;
        const bool ok = q < wd_chunks && j < my * 8 && kb < KB;
        const int off = ok ? (int)(tok * KB + kb) : 0x7FFFFFF0;
        wdv[r] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(ars, off, 0, 0));
      }
    }
  }
  // AM_QWIDEN: bf16 chunks of 8 values, q = lane + 64 r: token q >> qsh,
  // chunk q & (2^qsh - 1) of the slice (2^qsh = 16 WST chunks per token).
  const int qsh = 31 - __builtin_clz(WST * 16);
  const int q_chunks = QW ? (int)M * (1 << qsh) : 0;
  if constexpr (QW) {
    if (!opw) {
      const __amdgpu_buffer_rsrc_t xrs2 =
          __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)(M * KB * 2), 0x00020000);
#pragma unroll
      for (int r = 0; r < WDR; ++r) {
        const int q = lane + 64 * r;
        const int tok = q >> qsh, j = q & ((1 << qsh) - 1);
        const int64_t kv = (int64_t)first * STEPB + (int64_t)j * 8;
        const bool ok = q < q_chunks && j < my * 16 && kv < KB;
        const int off = ok ? (int)((tok * KB + kv) * 2) : 0x7FFFFFF0;
        wdv[r] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(xrs2, off, 0, 0));
      }
    }
  }
  if (!opw) {
    load_batch(0, DQ ? 2 : 0);
    if constexpr (QW) {
      // Partial maxima: the lanes of one token within a round are a group of
      // min(64, 2^qsh) consecutive lanes; its maximum goes to
      // qw_max[wave][token] (rounds of one token combine in order).
      if (lane < 16) qw_max[wave][lane] = 0.f;
      const int gl = qsh >= 6 ? 64 : (1 << qsh);
#pragma unroll
      for (int r = 0; r < WDR; ++r) {
        float v[8];
        unpack8<false>(wdv[r], v);
        float am = amax8(v);
        for (int o = 1; o < gl; o <<= 1) am = fmaxf(am, __shfl_xor(am, o));
        const int q = lane + 64 * r;
        const int tok = q >> qsh;
        if ((lane & (gl - 1)) == 0 && q < q_chunks) qw_max[wave][tok] = fmaxf(qw_max[wave][tok], am);
      }
    }
  }
  if constexpr (QW) {
    __syncthreads();  // every wave's partial maxima are in (the operand wave too)
    if (!opw) {
#pragma unroll
      for (int r = 0; r < WDR; ++r) {
        const int q = lane + 64 * r;
        if (q < q_chunks) {
          const int tok = q >> qsh, j = q & ((1 << qsh) - 1);
          float amax = qw_max[0][tok];
#pragma unroll
          for (int w = 1; w < W; ++w) amax = fmaxf(amax, qw_max[w][tok]);
          const float sc = group_scale(amax, 448.f);
          if (wave == 0 && j == 0) qw_scale[tok] = sc;
          float v[8];
          unpack8<false>(wdv[r], v);
          const i32x2 c8 = quant8<false>(v, make_div(sc, amax));
          typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
          i32x4 wide;
          wide[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)c8[0], 1.0f, false));
          wide[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)c8[0], 1.0f, true));
          wide[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)c8[1], 1.0f, false));
          wide[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)c8[1], 1.0f, true));
          // chunk j holds values 8 j .. 8 j + 7 of the slice: piece j & 15 of step j >> 4
          const int t = j >> 4, pc = j & 15;
          uint8_t* base = wdl + (int64_t)tok * WST * 256 + (t & ~1) * 256;
          *(i32x4*)(base + ((((t & 1) * 16 + pc) ^ wd_swz(tok)) << 4)) = wide;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the wave reads what its lanes wrote
      __builtin_amdgcn_wave_barrier();
    }
  }
  if (!opw) {
    if constexpr (WD && !QW) {
#pragma unroll
      for (int r = 0; r < WDR; ++r) {
        const int q = lane + 64 * r;
        if (q < wd_chunks) {
          const int tok = q >> wd_sh, j = q & ((1 << wd_sh) - 1);
          const int t = j >> 3, p = (j & 7) * 2;
          uint8_t* base = wdl + (int64_t)tok * WST * 256 + (t & ~1) * 256;
          const int sw = wd_swz(tok), p0 = (t & 1) * 16 + p;
          const i32x8 f = MF::prep(wdv[r]);
          *(i32x4*)(base + ((p0 ^ sw) << 4)) = lo16(f);
          *(i32x4*)(base + (((p0 + 1) ^ sw) << 4)) = hi16(f);
        }
      }
      // the wave reads what its other lanes wrote
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      __builtin_amdgcn_wave_barrier();
    }
    if constexpr (SWAP && !OPW) {
      if (fin_here) {
#pragma unroll
        for (int i = 0; i < QPW; ++i) {
          const int q = wave + i * W;
          const int64_t nr = n0 + (q / NTT) * 16 + g * 4;
          if (q < NTILE && nr < nend) epilogue_prefetch4<F16>(e, (q % NTT) * 16 + l16, nr, pre[i]);
        }
      }
    }
    compute_batch(0);
    for (int t0 = U; t0 < my; t0 += U) {
      load_batch(t0);
      compute_batch(t0);
    }
  } else if (fin_here) {
    // The operand wave: the loads' latency overlaps the weight stream of the
    // K waves, and the waves that own the tiles read the operands from LDS
    // at the end.  (The two-pass reduction with split > 1 runs its epilogue
    // in splitk_reduce instead.)
#pragma unroll
    for (int q = 0; q < NTILE; ++q) {
      const int64_t nr = n0 + (q / NTT) * 16 + g * 4;
      if (nr < nend) {
        EpiPre4 p;
        epilogue_prefetch4<F16>(e, (q % NTT) * 16 + l16, nr, p);
        opnd[q][0][lane] = p.sam;
#pragma unroll
        for (int i = 0; i < 4; ++i) opnd[q][1 + i][lane] = p.sb[i];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          opnd[q][5 + i][lane] = __uint_as_float(p.bias[i]);
          opnd[q][7 + i][lane] = __uint_as_float(p.res[i]);
        }
      }
    }
  }

  // In-workgroup reduction, in wave order; wave w then owns tiles
  // q = w, w + W, ... (q = rt * NTT + tt) for the rest of the kernel.
  if (!opw) {
    AccT* mine = RA ? (AccT*)(XS ? xsl : wdl) : &red[wave][0];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int tt = 0; tt < NTT; ++tt) {
        const C& a = acc[rt][tt];
        *(AccT4*)(mine + ((rt * NTT + tt) * 64 + lane) * 4) =
            AccT4{(AccT)a[0], (AccT)a[1], (AccT)a[2], (AccT)a[3]};
      }
  }
  __syncthreads();

  // Output coordinates of value r of tile q.
  auto coord = [&](int q, int r, int64_t& m, int64_t& n) {
    const int rt = q / NTT, tt = q % NTT;
    if (SWAP) { m = tt * 16 + l16; n = n0 + rt * 16 + g * 4 + r; }
    else { m = tt * 16 + g * 4 + r; n = n0 + rt * 16 + l16; }
  };
  auto finish = [&](int q, const AccT* v) {
    if (SWAP) {
      int64_t m, n;
      coord(q, 0, m, n);
      if (n < nend) epilogue_run<4, F16>(e, m, n, v);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        int64_t m, n;
        coord(q, r, m, n);
        if (n < nend) epilogue_one<F16>(e, m, n, v[r]);
      }
    }
  };
  // Swap-orientation epilogue of tile q (the i-th tile of this wave) from the
  // operands staged in LDS, or prefetched by this wave.
  auto finish_swap = [&](int q, int i, const AccT* v) {
    const int64_t nr = n0 + (q / NTT) * 16 + g * 4;
    if (nr >= nend) return;
    const int64_t m = (q % NTT) * 16 + l16;
    EpiPre4 p;
    if constexpr (!OPW) {
      p = pre[SWAP && !OPW ? i : 0];
    } else {
      p.sam = opnd[q][0][lane];
#pragma unroll
      for (int j = 0; j < 4; ++j) p.sb[j] = opnd[q][1 + j][lane];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        p.bias[j] = __float_as_uint(opnd[q][5 + j][lane]);
        p.res[j] = __float_as_uint(opnd[q][7 + j][lane]);
      }
    }
    if constexpr (DQ && !BLOCK) p.sam = sal[min(m, M - 1)];
    if constexpr (QW) p.sam = qw_scale[min(m, M - 1)];
    epilogue_run4_pre<F16>(e, m, nr, v, p);
  };
  auto reduce_tile = [&](int q, AccT* v) {
    auto part = [&](int w) {
      return *(const AccT4*)((RA ? (const AccT*)(dq_lds + (int64_t)w * (XS ? (int64_t)XSS : WSS))
                                 : &red[w][0]) +
                             (q * 64 + lane) * 4);
    };
    AccT4 s = part(0);
#pragma unroll
    for (int w = 1; w < W; ++w) s += part(w);
#pragma unroll
    for (int r = 0; r < 4; ++r) v[r] = s[r];
  };

  if (split == 1) {
    if (opw) return;
#pragma unroll
    for (int i = 0; i < QPW; ++i) {
      const int q = wave + i * W;
      if (q >= NTILE) break;
      AccT v[4];
      reduce_tile(q, v);
      if (SWAP) finish_swap(q, i, v);
      else finish(q, v);
    }
    return;
  }

  AccT* wsa = (AccT*)ws;
  for (int q = opw ? NTILE : wave; q < NTILE; q += W) {
    AccT v[4];
    reduce_tile(q, v);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int64_t m, n;
      coord(q, r, m, n);
      if (m < M && n < nend) {
        if (reduce == R_ATOMIC)
          __hip_atomic_fetch_add(wsa + m * N + n, v[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          st_agent(wsa + ((int64_t)sidx * M + m) * N + n, v[r]);
      }
    }
  }
  if (reduce == R_TWOPASS) return;

  // Arrival: the last of the split workgroups of this row group finishes.
  // Every partial is written, and later read, with agent-scope atomic
  // stores / loads, which are coherent across the XCDs' L2s by themselves;
  // what must hold is that a workgroup's partials are complete before its
  // counter increment is.  Each wave therefore waits for its own stores to
  // be acknowledged (s_waitcnt 0) before the barrier, and thread 0 then
  // increments the counter.  A generic agent-scope release / acquire would
  // also write back and invalidate the whole L2 in every workgroup, which
  // costs more than the reduction saves.
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __syncthreads();
  if (threadIdx.x == 0)
    arrival = __hip_atomic_fetch_add(counters + blockIdx.x, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (arrival != split - 1 || opw) return;
#pragma unroll
  for (int i = 0; i < QPW; ++i) {
    const int q = wave + i * W;
    if (q >= NTILE) break;
    AccT v[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int64_t m, n;
      coord(q, r, m, n);
      AccT s = 0;
      if (m < M && n < nend) {
        if (reduce == R_ATOMIC) {
          s = ld_agent(wsa + m * N + n);
          st_agent(wsa + m * N + n, (AccT)0);
        } else {
          for (int qq = 0; qq < split; ++qq) s += ld_agent(wsa + ((int64_t)qq * M + m) * N + n);
        }
      }
      v[r] = s;
    }
    if (SWAP) finish_swap(q, i, v);
    else finish(q, v);
  }
  if (threadIdx.x == 0) st_agent(counters + blockIdx.x, 0);
}

template <int QK, int NTT, bool SWAP, int W, int U, int RT, int AM>
__global__ __launch_bounds__((W + (op_wave(SWAP, W) ? 1 : 0)) * 64) void decode_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, int64_t M, int64_t N,
    int64_t KB, int rpw, int split, int steps_per_split, int reduce, Epi e,
    void* __restrict__ ws, int* __restrict__ counters) {
  decode_body<QK, NTT, SWAP, W, U, RT, AM>(A, B, M, N, KB, rpw, split, (int)blockIdx.y,
                                           steps_per_split, reduce, e, ws, counters);
}

// The k-th expert (in expert order) whose segment [offsets[x], offsets[x+1])
// is non-empty, with the segment clamped into [0, M] (an end below its
// start is empty); x = -1 if there are at most k.  Each wave computes it
// alone (no LDS, no barrier): 64 experts per ballot, the offsets of four
// ballots loaded at once.
__device__ inline void kth_segment(const int* __restrict__ offsets, int E, int M, int k, int& x,
                                   int& lo, int& hi) {
  const int lane = threadIdx.x & 63;
  x = -1; lo = 0; hi = 0;
  for (int base = 0; base < E; base += 256) {
    int l[4], h[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = base + 64 * j + lane;
      const bool in = i < E;
      const int a = in ? offsets[i] : 0, b = in ? offsets[i + 1] : 0;
      l[j] = min(max(a, 0), M);
      h[j] = min(max(b, l[j]), M);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ne = h[j] > l[j];
      const uint64_t bits = __ballot(ne);
      const int cnt = __popcll(bits);
      if (k < cnt) {
        const int below = (int)__builtin_amdgcn_mbcnt_hi(
            (uint32_t)(bits >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bits, 0u));
        const int src = __ffsll((unsigned long long)__ballot(ne && below == k)) - 1;
        x = __builtin_amdgcn_readfirstlane(base + 64 * j + src);
        lo = __builtin_amdgcn_readfirstlane(__shfl(l[j], src));
        hi = __builtin_amdgcn_readfirstlane(__shfl(h[j], src));
        return;
      }
      k -= cnt;
    }
  }
}

// Grouped form (a mixture-of-experts layer, tokens sorted by expert):
// expert x owns rows [offsets[x], offsets[x+1]) of A, the residual and C,
// and its own weight B[x] (N rows of KB bytes) with its weight scales and
// bias.  Workgroup row y = blockIdx.y serves the y-th expert that has rows,
// so min(E, M) rows of workgroups cover every case and experts without rows
// cost nothing.  The expert's rows go through the decode body in chunks of
// 16 NTT tokens (swap orientation, no split-K: the experts already give the
// grid its width), chunk c on workgroup z = c mod gridDim.z, so any segment
// length is covered whatever the grid's depth.  Offsets are clamped into
// [0, M] and an end below its start is an empty segment: a malformed offset
// array gives wrong rows, never an access outside A, C or the residual.
template <int QK, int NTT, int W, int U, int RT, int AM>
__global__ __launch_bounds__((W + (op_wave(true, W) ? 1 : 0)) * 64) void grouped_decode_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
    const int* __restrict__ offsets, int E, int64_t M, int64_t N, int64_t KB, int rpw,
    int steps, Epi e) {
  constexpr int64_t XR = QK == QK_MXFP4 ? 4 : 1;
  constexpr int64_t MT = 16 * NTT;
  int xi, loi, hii;
  kth_segment(offsets, E, (int)M, (int)blockIdx.y, xi, loi, hii);
  if (xi < 0) return;
  const int64_t x = xi, lo = loi, hi = hii;
  const int64_t first = lo + (int64_t)blockIdx.z * MT;
  if (first >= hi) return;
  const uint8_t* Bx = B + x * N * KB;
  for (int64_t r0 = first; r0 < hi; r0 += (int64_t)gridDim.z * MT) {
    if (r0 != first) __syncthreads();  // the previous chunk is done with the LDS
    const int64_t rows = min(MT, hi - r0);
    decode_body<QK, NTT, true, W, U, RT, AM>(A + r0 * KB * XR, Bx, rows, N, KB, rpw, 1, 0,
                                             steps, R_NONE, grouped_epi<QK>(e, x, r0, rows, KB),
                                             nullptr, nullptr);
  }
}

// Second pass of the two-pass reduction: sum the split partials of 4
// consecutive columns in slice order, then the epilogue.
template <int QK>
__global__ __launch_bounds__(256) void splitk_reduce(const void* __restrict__ ws, int split,
                                                     Epi e) {
  using AccT = typename QTraits<QK>::Acc;
  const AccT* wsa = (const AccT*)ws;
  const int64_t nq = (e.N + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t m = idx / nq;
  const int64_t n = (idx - m * nq) * 4;
  if (m >= e.M) return;
  AccT v[4] = {0, 0, 0, 0};
  const int64_t slice = e.M * e.N;
  const AccT* col = wsa + m * e.N + n;
  if (n + 4 <= e.N && e.N % 4 == 0) {
    // 16-byte loads, four slices in flight at a time; the sums still run in
    // slice order.
    typedef AccT AccT4 __attribute__((ext_vector_type(4)));
    AccT4 s = {0, 0, 0, 0};
    int q = 0;
    for (; q + 4 <= split; q += 4) {
      AccT4 p[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) p[k] = *(const AccT4*)(col + (q + k) * slice);
#pragma unroll
      for (int k = 0; k < 4; ++k) s += p[k];
    }
    for (; q < split; ++q) s += *(const AccT4*)(col + q * slice);
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = s[i];
  } else {
    for (int q = 0; q < split; ++q)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < e.N) v[i] += col[q * slice + i];
  }
  epilogue_run<4, QTraits<QK>::out_f16>(e, m, n, v);
}

// Dynamic LDS of the quantization prologue: M code rows of KB + 16 bytes,
// then the scales (per token: M, plus M maxima; per block: M x KB/128).
inline size_t dq_lds_bytes(int qk, const Call& c) {
  const size_t rows = (size_t)c.M * (size_t)(c.KB + 16);
  const size_t sc = qk == QK_FP8_BLOCK ? 4 * (size_t)c.M * (size_t)(c.KB / 128) : 8 * (size_t)c.M;
  return (rows + sc + 15) & ~(size_t)15;
}

// Dynamic LDS of the staged-activation mode: W waves x U steps x the M
// tokens' activation bytes of one step, rounded up to whole KiB (the
// direct-to-LDS loads write 1 KiB each), each wave's slice at least the
// 1 KiB per 16x16 output tile that its partial sums take at the end.
inline size_t xs_lds_bytes(int qk, int W, int U, int RT, const Call& c) {
  const size_t chunks = (size_t)c.M * STEPB * (qk == QK_MXFP4 ? 4 : 1) / 16;
  const size_t ntile = (size_t)RT * (c.M <= 16 ? 1 : 2);
  return (size_t)W * std::max((size_t)U * ((chunks + 63) / 64 * 1024), ntile * 1024);
}

// Dynamic LDS of the widened-activation mode: W waves x M tokens x the
// steps a wave's slice reserves x 256 bytes; and whether one lane's share of
// the widening (M x steps x 8 chunks over 64 lanes) fits WD_ROUNDS chunks.
inline int wd_slice_steps(int W, int U, const Call& c, int split) {
  const int total_steps = (int)((c.KB + STEPB - 1) / STEPB);
  const int sps = (total_steps + split - 1) / split;
  return wd_steps((sps + W - 1) / W, U);
}
inline size_t wd_lds_bytes(int W, int U, const Call& c, int split, int RT = 2) {
  // each slice also holds the wave's partial sums (1 KiB per 16x16 tile)
  return (size_t)W * std::max((size_t)c.M * (size_t)wd_slice_steps(W, U, c, split) * 256,
                              (size_t)RT * 1024);
}
inline bool wd_fits_rounds(int W, int U, const Call& c, int split) {
  return c.M * wd_slice_steps(W, U, c, split) * 8 <= 64 * WD_ROUNDS;
}

template <int QK, int NTT, bool SWAP, int W, int U, int RT, int AM = AM_GLOBAL>
hipError_t launch_d(const Variant& v, const Call& c, int split, hipStream_t s) {
  constexpr bool DQ = AM == AM_QUANT;
  const int groups = (int)((c.N + v.rows - 1) / v.rows);
  const int total_steps = (int)((c.KB + STEPB - 1) / STEPB);
  const int sps = (total_steps + split - 1) / split;
  const size_t dyn = DQ ? dq_lds_bytes(QK, c)
                        : (AM == AM_STAGE ? xs_lds_bytes(QK, W, U, RT, c)
                                          : (am_widen(AM) ? wd_lds_bytes(W, U, c, split, RT) : 0));
  hipLaunchKernelGGL((decode_kernel<QK, NTT, SWAP, W, U, RT, AM>), dim3(groups, split),
                     dim3((W + (op_wave(SWAP, W) ? 1 : 0)) * 64),
                     dyn, s, (const uint8_t*)c.A, (const uint8_t*)c.B, c.M, c.N, c.KB, v.rows, split,
                     sps, v.reduce, c.epi, c.ws, c.counters);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || split == 1 || v.reduce != R_TWOPASS) return err;
  const int64_t threads = c.M * ((c.N + 3) / 4);
  hipLaunchKernelGGL((splitk_reduce<QK>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                     s, (const void*)c.ws, split, c.epi);
  return hipGetLastError();
}

// Compiled (waves, unroll, 16-row tiles) triples with swap-AB, and the one
// direct-orientation variant.  A variant's rows-per-workgroup value picks the
// tile count: up to 16 rows -> 1 tile, 32 -> 2, 64 -> 4.
#define LG_DECODE_SWAP(X, QK, NTT) \
  X(QK, NTT, true, 8, 1, 1) X(QK, NTT, true, 8, 2, 1) X(QK, NTT, true, 4, 4, 1) \
  X(QK, NTT, true, 16, 1, 1) X(QK, NTT, true, 8, 1, 2) X(QK, NTT, true, 4, 2, 2) \
  X(QK, NTT, true, 8, 2, 2) X(QK, NTT, true, 4, 1, 4) X(QK, NTT, true, 8, 1, 4) \
  X(QK, NTT, true, 8, 4, 1) X(QK, NTT, true, 8, 4, 2) X(QK, NTT, true, 12, 1, 1) \
  X(QK, NTT, true, 16, 1, 2) X(QK, NTT, true, 16, 2, 2) X(QK, NTT, false, 8, 2, 1)

// Tiles per workgroup for a rows-per-workgroup value: 1, 2 or 4.
inline int tiles_for(int rows) { return rows <= 16 ? 1 : (rows <= 32 ? 2 : 4); }

#define LG_DECODE_TRY(qk, ntt, sw, w, u, rt)                                             \
  if (v.swap == (sw ? 1 : 0) && v.waves == w && v.unroll == u && tiles_for(v.rows) == rt) \
    return launch_d<qk, ntt, sw, w, u, rt>(v, c, split, s);

template <int QK, int NTT>
hipError_t launch_dq(const Variant& v, const Call& c, int split, hipStream_t s) {
  LG_DECODE_SWAP(LG_DECODE_TRY, QK, NTT)
  return hipErrorInvalidValue;
}

template <int QK>
hipError_t launch_q(const Variant& v, const Call& c, int split, hipStream_t s) {
  return c.M <= 16 ? launch_dq<QK, 1>(v, c, split, s) : launch_dq<QK, 2>(v, c, split, s);
}

// Variants with the quantization prologue (bf16 activations; swap, one token
// tile, split 1).
#define LG_DECODE_DQ(X, QK)                                                            \
  X(QK, 8, 1, 1) X(QK, 8, 2, 1) X(QK, 8, 4, 1) X(QK, 8, 4, 2) X(QK, 12, 1, 1) \
  X(QK, 4, 4, 1)

// Whether a kernel's static LDS plus `dyn` bytes of dynamic LDS fit the
// current device's per-workgroup limit.  The kernel's static size and each
// device's limit are queried once and cached (the calls sit on the launch
// path).
bool lds_fits(const void* fn, size_t dyn) {
  static std::mutex mu;
  static std::unordered_map<const void*, size_t> static_lds;
  static int dev_max[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  std::lock_guard<std::mutex> lock(mu);
  auto it = static_lds.find(fn);
  if (it == static_lds.end()) {
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, fn) != hipSuccess) return false;
    it = static_lds.emplace(fn, attr.sharedSizeBytes).first;
  }
  if (dev_max[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
      return false;
    dev_max[dev] = v;
  }
  return it->second + dyn <= (size_t)dev_max[dev];
}

// Whether the prologue variant exists and its LDS (static + dynamic) fits
// the device's per-workgroup limit; if so, *fn is the kernel.
template <int QK>
bool dq_kernel(const Variant& v, const Call& c, const void** fn) {
  *fn = nullptr;
#define LG_DQ_FN(qk, w, u, rt)                                                      \
  if (v.waves == w && v.unroll == u && tiles_for(v.rows) == rt)                     \
    *fn = reinterpret_cast<const void*>(&decode_kernel<qk, 1, true, w, u, rt, AM_QUANT>);
  LG_DECODE_DQ(LG_DQ_FN, QK)
#undef LG_DQ_FN
  return *fn && lds_fits(*fn, dq_lds_bytes(QK, c));
}

template <int QK>
hipError_t launch_dq_prologue(const Variant& v, const Call& c, hipStream_t s) {
#define LG_DQ_TRY(qk, w, u, rt)                                                     \
  if (v.waves == w && v.unroll == u && tiles_for(v.rows) == rt)                     \
    return launch_d<qk, 1, true, w, u, rt, AM_QUANT>(v, c, 1, s);
  LG_DECODE_DQ(LG_DQ_TRY, QK)
#undef LG_DQ_TRY
  return hipErrorInvalidValue;
}

}  // namespace

int decode_auto_split(const Call& c, const Variant& v) {
  const int64_t groups = (c.N + v.rows - 1) / v.rows;
  const int64_t steps = (c.KB + STEPB - 1) / STEPB;
  int split = 1;
  while (groups * split < 768 && (int64_t)split * 2 * v.waves <= steps && split < 16) split *= 2;
  return split;
}

size_t decode_ws_bytes(const Variant& v, const Call& c, int split) {
  if (split <= 1) return 0;
  if (v.reduce == R_ATOMIC) return (size_t)c.M * c.N * 4;
  return (size_t)split * c.M * c.N * 4;
}

hipError_t launch_splitk_reduce(int qk, const void* ws, int split, const Epi& e, hipStream_t s) {
  const int64_t threads = e.M * ((e.N + 3) / 4);
  const dim3 grid((unsigned)((threads + 255) / 256));
  switch (qk) {
    case QK_BF16: hipLaunchKernelGGL((splitk_reduce<QK_BF16>), grid, dim3(256), 0, s, ws, split, e); break;
    case QK_FP16: hipLaunchKernelGGL((splitk_reduce<QK_FP16>), grid, dim3(256), 0, s, ws, split, e); break;
    case QK_FP8: hipLaunchKernelGGL((splitk_reduce<QK_FP8>), grid, dim3(256), 0, s, ws, split, e); break;
    case QK_I8: hipLaunchKernelGGL((splitk_reduce<QK_I8>), grid, dim3(256), 0, s, ws, split, e); break;
    case QK_FP8_BLOCK:
      hipLaunchKernelGGL((splitk_reduce<QK_FP8_BLOCK>), grid, dim3(256), 0, s, ws, split, e);
      break;
    case QK_MXFP4:
      hipLaunchKernelGGL((splitk_reduce<QK_MXFP4>), grid, dim3(256), 0, s, ws, split, e);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// MXFP4-weight variants (swap, up to two steps per batch: each step holds 64
// bf16 activations per lane and token tile in registers).
#define LG_DECODE_MX(X)                                                                \
  X(8, 1, 1) X(8, 2, 1) X(16, 1, 1) X(12, 1, 1) X(8, 1, 2) X(4, 2, 2) X(8, 2, 2) X(4, 1, 4) \
  X(8, 1, 4)

bool decode_mx_supported(const Variant& v) {
  if (v.kind != V_DECODE || v.swap != 1) return false;
#define LG_MX_HAS(w, u, rt) if (v.waves == w && v.unroll == u && tiles_for(v.rows) == rt) return true;
  LG_DECODE_MX(LG_MX_HAS)
#undef LG_MX_HAS
  return false;
}

template <int NTT>
hipError_t launch_mx(const Variant& v, const Call& c, int split, hipStream_t s) {
#define LG_MX_TRY(w, u, rt)                                                          \
  if (v.swap == 1 && v.waves == w && v.unroll == u && tiles_for(v.rows) == rt)      \
    return launch_d<QK_MXFP4, NTT, true, w, u, rt>(v, c, split, s);
  LG_DECODE_MX(LG_MX_TRY)
#undef LG_MX_TRY
  return hipErrorInvalidValue;
}

// Variants with staged activations (AM_STAGE; swap; one or two token
// tiles): e4m3, int8, block e4m3, MXFP4, bf16 and fp16 weights.
#define LG_DECODE_XS(X)                                                                \
  X(QK_FP8, 1, 8, 1, 1) X(QK_FP8, 1, 8, 2, 1) X(QK_FP8, 1, 8, 4, 1) X(QK_FP8, 1, 8, 4, 2) \
  X(QK_FP8, 1, 12, 1, 1) X(QK_MXFP4, 1, 8, 1, 1) X(QK_MXFP4, 1, 8, 2, 1)                 \
  X(QK_MXFP4, 1, 8, 1, 2) X(QK_MXFP4, 1, 12, 1, 1) X(QK_I8, 1, 4, 4, 1) X(QK_I8, 1, 8, 2, 1) \
  X(QK_I8, 1, 8, 4, 2) X(QK_FP8_BLOCK, 1, 12, 1, 1) X(QK_FP8_BLOCK, 1, 8, 1, 1)          \
  X(QK_FP8_BLOCK, 1, 16, 1, 1) X(QK_FP8, 2, 8, 1, 2) X(QK_FP8, 2, 8, 4, 2)              \
  X(QK_I8, 2, 4, 2, 2) X(QK_MXFP4, 2, 4, 2, 2) X(QK_MXFP4, 2, 8, 1, 2)                 \
  X(QK_FP8_BLOCK, 2, 8, 2, 2) X(QK_BF16, 1, 8, 1, 2) X(QK_BF16, 1, 8, 1, 1)             \
  X(QK_BF16, 1, 8, 2, 1) X(QK_BF16, 2, 8, 1, 2) X(QK_FP16, 1, 8, 1, 2)                   \
  X(QK_FP16, 1, 8, 1, 1) X(QK_FP16, 1, 8, 2, 1) X(QK_FP16, 2, 8, 1, 2)                   \
  X(QK_I8, 1, 4, 2, 2) X(QK_I8, 1, 8, 1, 2) X(QK_FP8_BLOCK, 2, 8, 1, 2)                  \
  X(QK_FP8_BLOCK, 2, 12, 1, 1) X(QK_FP8_BLOCK, 2, 16, 1, 1) X(QK_FP8_BLOCK, 2, 4, 2, 2)   \
  X(QK_FP8, 2, 16, 1, 2) X(QK_FP8, 1, 16, 1, 2) X(QK_BF16, 2, 16, 1, 2) X(QK_I8, 2, 16, 1, 2) \
  X(QK_FP8_BLOCK, 2, 16, 1, 2) X(QK_FP16, 2, 16, 1, 2) X(QK_FP8, 2, 16, 2, 2)             \
  X(QK_BF16, 2, 16, 2, 2) X(QK_FP16, 2, 16, 2, 2) X(QK_FP8_BLOCK, 2, 16, 2, 1)          \
  X(QK_FP8_BLOCK, 2, 12, 2, 1) X(QK_FP8_BLOCK, 2, 8, 1, 4)

// Whether the plain build of this decode shape exists (for every weight
// format).
bool decode_plain_supported(int swap, int waves, int unroll, int rows) {
  if (rows < 4 || rows > 64 || rows % 4 != 0) return false;
#define LG_DECODE_HAS(qk, ntt, sw, w, u, rt) \
  if (swap == (sw ? 1 : 0) && waves == w && unroll == u && tiles_for(rows) == rt) return true;
  LG_DECODE_SWAP(LG_DECODE_HAS, 0, 1)
#undef LG_DECODE_HAS
  return false;
}

// Whether some build of this decode shape exists: the plain one, or a staged
// one for some formats and token tiles only (forcing the latter where it does
// not apply fails at the call).
bool decode_supported(int swap, int waves, int unroll, int rows) {
  if (decode_plain_supported(swap, waves, unroll, rows)) return true;
  if (rows < 4 || rows > 64 || rows % 4 != 0) return false;
#define LG_DECODE_XS_HAS(q_, nt, w, u, rt) \
  if (swap == 1 && waves == w && unroll == u && tiles_for(rows) == rt) return true;
  LG_DECODE_XS(LG_DECODE_XS_HAS)
#undef LG_DECODE_XS_HAS
  return false;
}

bool decode_xs_supported(const Variant& v, const Call& c) {
  if (v.kind != V_DECODE || v.swap != 1 || c.M < 1 || c.M > 32) return false;
  const int ntt = c.M <= 16 ? 1 : 2;
  const void* fn = nullptr;
  int w_ = 0, u_ = 0;
#define LG_XS_FN(q_, nt, w, u, rt)                                                  \
  if (c.qk == q_ && ntt == nt && v.waves == w && v.unroll == u && tiles_for(v.rows) == rt) { \
    fn = reinterpret_cast<const void*>(&decode_kernel<q_, nt, true, w, u, rt, AM_STAGE>); \
    w_ = w; u_ = u; rt_ = rt;                                                       \
  }
  int rt_ = 1;
  LG_DECODE_XS(LG_XS_FN)
#undef LG_XS_FN
  return fn && lds_fits(fn, xs_lds_bytes(c.qk, w_, u_, rt_, c));
}

hipError_t launch_decode_xs(const Variant& v, const Call& c, int split, hipStream_t s) {
  const int ntt = c.M <= 16 ? 1 : 2;
#define LG_XS_TRY(q_, nt, w, u, rt)                                                 \
  if (c.qk == q_ && ntt == nt && v.waves == w && v.unroll == u && tiles_for(v.rows) == rt) \
    return launch_d<q_, nt, true, w, u, rt, AM_STAGE>(v, c, split, s);
  LG_DECODE_XS(LG_XS_TRY)
#undef LG_XS_TRY
  return hipErrorInvalidValue;
}

// Variants with widened activations (AM_WIDEN; swap; one token tile; e4m3
// activations): (quant, waves, unroll, 16-row tiles).
#define LG_DECODE_WD(X)                                                                \
  X(QK_FP8, 8, 1, 1) X(QK_FP8, 8, 2, 1) X(QK_FP8, 8, 4, 1) X(QK_FP8, 12, 1, 1)          \
  X(QK_FP8, 16, 1, 1) X(QK_FP8, 8, 1, 2) X(QK_FP8, 4, 4, 1) X(QK_FP8, 16, 1, 2)         \
  X(QK_FP8, 16, 2, 2) X(QK_FP8_BLOCK, 12, 1, 1)                                         \
  X(QK_FP8_BLOCK, 8, 1, 1) X(QK_FP8_BLOCK, 16, 1, 1) X(QK_FP8_BLOCK, 8, 2, 1)

bool decode_wd_supported(const Variant& v, const Call& c, int split) {
  if (v.kind != V_DECODE || v.swap != 1 || c.M < 1 || c.M > 16 || split < 1) return false;
  if (c.M * c.KB > 0x7FFFFFF0LL) return false;  // buffer offsets of the activation loads
  const void* fn = nullptr;
  int w_ = 0, u_ = 0;
#define LG_WD_FN(q_, w, u, rt)                                                      \
  if (c.qk == q_ && v.waves == w && v.unroll == u && tiles_for(v.rows) == rt) {     \
    fn = reinterpret_cast<const void*>(&decode_kernel<q_, 1, true, w, u, rt, AM_WIDEN8>); \
    w_ = w; u_ = u;                                                                 \
  }
  LG_DECODE_WD(LG_WD_FN)
#undef LG_WD_FN
  // (the four forms share their static LDS; the dynamic size is the same)
  return fn && wd_fits_rounds(w_, u_, c, split) && lds_fits(fn, wd_lds_bytes(w_, u_, c, split));
}

hipError_t launch_decode_wd(const Variant& v, const Call& c, int split, hipStream_t s) {
  const int rounds = (int)((c.M * wd_slice_steps(v.waves, v.unroll, c, split) * 8 + 63) / 64);
#define LG_WD_TRY(q_, w, u, rt)                                                     \
  if (c.qk == q_ && v.waves == w && v.unroll == u && tiles_for(v.rows) == rt) {     \
    if (rounds <= 1) return launch_d<q_, 1, true, w, u, rt, AM_WIDEN>(v, c, split, s);  \
    if (rounds <= 2) return launch_d<q_, 1, true, w, u, rt, AM_WIDEN2>(v, c, split, s); \
    if (rounds <= 4) return launch_d<q_, 1, true, w, u, rt, AM_WIDEN4>(v, c, split, s); \
    return launch_d<q_, 1, true, w, u, rt, AM_WIDEN8>(v, c, split, s);              \
  }
  LG_DECODE_WD(LG_WD_TRY)
#undef LG_WD_TRY
  return hipErrorInvalidValue;
}

// Fused quantization with widened activations (AM_QWIDEN; e4m3 per token,
// bf16 X, swap, one token tile, split 1): the same shapes as the widened
// mode, each with one, two, four or eight 8-value chunks per lane.
#define LG_DECODE_QW(X)                                                                \
  X(8, 1, 1) X(8, 2, 1) X(8, 4, 1) X(12, 1, 1) X(16, 1, 1) X(8, 1, 2) X(4, 4, 1)

inline int qw_rounds(const Variant& v, const Call& c) {
  return (int)((c.M * wd_slice_steps(v.waves, v.unroll, c, 1) * 16 + 63) / 64);
}

bool decode_qw_supported(const Variant& v, const Call& c) {
  if (v.kind != V_DECODE || v.swap != 1 || v.xs != 2 || c.qk != QK_FP8 || c.M < 1 || c.M > 16)
    return false;
  if (c.M * c.KB * 2 > 0x7FFFFFF0LL || qw_rounds(v, c) > WD_ROUNDS) return false;
  const void* fn = nullptr;
  int w_ = 0, u_ = 0;
#define LG_QW_FN(w, u, rt)                                                          \
  if (v.waves == w && v.unroll == u && tiles_for(v.rows) == rt) {                   \
    fn = reinterpret_cast<const void*>(&decode_kernel<QK_FP8, 1, true, w, u, rt, AM_QWIDEN8>); \
    w_ = w; u_ = u;                                                                 \
  }
  LG_DECODE_QW(LG_QW_FN)
#undef LG_QW_FN
  return fn && lds_fits(fn, wd_lds_bytes(w_, u_, c, 1));
}

hipError_t launch_decode_qw(const Variant& v, const Call& c, hipStream_t s) {
  const int rounds = qw_rounds(v, c);
#define LG_QW_TRY(w, u, rt)                                                         \
  if (v.waves == w && v.unroll == u && tiles_for(v.rows) == rt) {                   \
    if (rounds <= 1) return launch_d<QK_FP8, 1, true, w, u, rt, AM_QWIDEN>(v, c, 1, s);  \
    if (rounds <= 2) return launch_d<QK_FP8, 1, true, w, u, rt, AM_QWIDEN2>(v, c, 1, s); \
    if (rounds <= 4) return launch_d<QK_FP8, 1, true, w, u, rt, AM_QWIDEN4>(v, c, 1, s); \
    return launch_d<QK_FP8, 1, true, w, u, rt, AM_QWIDEN8>(v, c, 1, s);              \
  }
  LG_DECODE_QW(LG_QW_TRY)
#undef LG_QW_TRY
  return hipErrorInvalidValue;
}

bool decode_dq_supported(const Variant& v, const Call& c, int split) {
  if (v.kind != V_DECODE || v.swap != 1 || split != 1 || c.M < 1 || c.M > 16) return false;
  if (decode_qw_supported(v, c)) return true;
  const void* fn;
  switch (c.qk) {
    case QK_FP8: return dq_kernel<QK_FP8>(v, c, &fn);
    case QK_I8: return dq_kernel<QK_I8>(v, c, &fn);
    case QK_FP8_BLOCK: return dq_kernel<QK_FP8_BLOCK>(v, c, &fn);
  }
  return false;
}

hipError_t launch_decode_dq(const Variant& v, const Call& c, hipStream_t s) {
  if (decode_qw_supported(v, c)) return launch_decode_qw(v, c, s);
  switch (c.qk) {
    case QK_FP8: return launch_dq_prologue<QK_FP8>(v, c, s);
    case QK_I8: return launch_dq_prologue<QK_I8>(v, c, s);
    case QK_FP8_BLOCK: return launch_dq_prologue<QK_FP8_BLOCK>(v, c, s);
  }
  return hipErrorInvalidValue;
}

// Grouped (mixture-of-experts) variants, by quant mode and token tiles (one:
// chunks of up to 16 tokens, two: up to 32), with activations loaded by each
// lane (AM_GLOBAL) or staged through LDS (AM_STAGE; 8-bit and 4-bit
// weights).  The first entry of a (mode, tiles, staging) triple is its
// default: four waves, two steps per batch, 32 weight rows per workgroup --
// an expert's weight is short in K, and fewer waves each streaming longer
// runs beat the dense decode's eight (measured on a 128-expert top-8 layer,
// N = 1536, K = 2048).  The rest are alternatives for forced variants and
// the sweep.
#define LG_GROUPED_MODE(X, Q)                                                            \
  X(Q, 1, 4, 2, 2, AM_GLOBAL) X(Q, 2, 4, 2, 2, AM_GLOBAL)                                \
  X(Q, 1, 8, 2, 1, AM_GLOBAL) X(Q, 2, 8, 1, 2, AM_GLOBAL)
#define LG_GROUPED_STAGE(X, Q) X(Q, 1, 4, 2, 2, AM_STAGE) X(Q, 2, 4, 2, 2, AM_STAGE)
#define LG_GROUPED(X)                                                                    \
  LG_GROUPED_MODE(X, QK_BF16) LG_GROUPED_MODE(X, QK_FP16) LG_GROUPED_MODE(X, QK_FP8)       \
  LG_GROUPED_MODE(X, QK_I8) LG_GROUPED_MODE(X, QK_FP8_BLOCK) LG_GROUPED_MODE(X, QK_MXFP4)  \
  LG_GROUPED_STAGE(X, QK_FP8) LG_GROUPED_STAGE(X, QK_I8) LG_GROUPED_STAGE(X, QK_FP8_BLOCK)  \
  LG_GROUPED_STAGE(X, QK_MXFP4)                                                          \
  X(QK_FP8, 1, 8, 2, 1, AM_STAGE) X(QK_FP8, 2, 8, 1, 2, AM_STAGE)                        \
  X(QK_I8, 1, 8, 2, 1, AM_STAGE) X(QK_FP8_BLOCK, 1, 8, 1, 1, AM_STAGE)                   \
  X(QK_MXFP4, 1, 8, 2, 1, AM_STAGE)                                                      \
  X(QK_FP8, 1, 4, 4, 1, AM_GLOBAL) X(QK_FP8, 1, 4, 1, 4, AM_GLOBAL)                      \
  X(QK_FP8, 2, 4, 1, 4, AM_GLOBAL) X(QK_FP8, 1, 8, 2, 2, AM_GLOBAL)                      \
  X(QK_FP8, 2, 8, 2, 2, AM_GLOBAL) X(QK_FP8, 1, 8, 1, 4, AM_GLOBAL)

namespace {
// The grouped variant for (qk, ntt, staged), its kernel and its LDS need.
struct GroupedPick {
  const void* fn = nullptr;
  int w = 0, u = 0, rt = 0;
};
// w == 0: the default of (qk, ntt, xs); else the entry with waves w,
// unroll u and rt 16-row tiles, if compiled.
GroupedPick grouped_pick(int qk, int ntt, bool xs, int w, int u, int rt) {
  GroupedPick p;
#define LG_G_FN(q_, nt, w_, u_, rt_, am)                                             \
  if (!p.fn && qk == q_ && ntt == nt && xs == (am == AM_STAGE) &&                   \
      (w == 0 || (w == w_ && u == u_ && rt == rt_))) {                              \
    p.fn = reinterpret_cast<const void*>(&grouped_decode_kernel<q_, nt, w_, u_, rt_, am>); \
    p.w = w_; p.u = u_; p.rt = rt_;                                                 \
  }
  LG_GROUPED(LG_G_FN)
#undef LG_G_FN
  return p;
}
}  // namespace

bool grouped_supported(const Variant& v, int qk, int ntt, int64_t KB) {
  const int w = v.waves, rt = w ? tiles_for(v.rows) : 0;
  if (w && (v.rows < 4 || v.rows > 64 || v.rows % 4 != 0)) return false;
  if (w && qk == QK_FP8_BLOCK && 128 % v.rows != 0) return false;
  const GroupedPick p = grouped_pick(qk, ntt, v.xs != 0, w, v.unroll, rt);
  if (!p.fn) return false;
  if (!v.xs) return true;
  Call c{};
  c.qk = qk; c.M = 16 * ntt; c.KB = KB;
  return lds_fits(p.fn, xs_lds_bytes(qk, p.w, p.u, p.rt, c));
}

hipError_t launch_grouped(const Variant& v, const Call& c, const int* offsets, int64_t E,
                          int ntt, int chunks, hipStream_t s) {
  const bool xs = v.xs != 0;
  const int w = v.waves, rt = w ? tiles_for(v.rows) : 0;
  const GroupedPick p = grouped_pick(c.qk, ntt, xs, w, v.unroll, rt);
  if (!p.fn || E < 1 || E > 65535 || chunks < 1 || chunks > 65535) return hipErrorInvalidValue;
  const int rows = w ? v.rows : 16 * p.rt;
  const int64_t groups = (c.N + rows - 1) / rows;
  const int steps = (int)((c.KB + STEPB - 1) / STEPB);
  Call cm = c;
  cm.M = 16 * ntt;  // staging holds one chunk
  const size_t dyn = xs ? xs_lds_bytes(c.qk, p.w, p.u, p.rt, cm) : 0;
  const dim3 grid((unsigned)groups, (unsigned)std::min<int64_t>(E, c.M), (unsigned)chunks);
#define LG_G_TRY(q_, nt, w_, u_, rt_, am)                                               \
  if (p.fn == reinterpret_cast<const void*>(&grouped_decode_kernel<q_, nt, w_, u_, rt_, am>)) { \
    hipLaunchKernelGGL((grouped_decode_kernel<q_, nt, w_, u_, rt_, am>), grid,         \
                       dim3((w_ + (op_wave(true, w_) ? 1 : 0)) * 64), dyn, s,           \
                       (const uint8_t*)c.A, (const uint8_t*)c.B, offsets, (int)E, c.M, c.N, \
                       c.KB, rows, steps, c.epi);                                       \
    return hipGetLastError();                                                         \
  }
  LG_GROUPED(LG_G_TRY)
#undef LG_G_TRY
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const Variant& v, const Call& c, int split, hipStream_t s) {
  switch (c.qk) {
    case QK_BF16: return launch_q<QK_BF16>(v, c, split, s);
    case QK_FP16: return launch_q<QK_FP16>(v, c, split, s);
    case QK_FP8: return launch_q<QK_FP8>(v, c, split, s);
    case QK_I8: return launch_q<QK_I8>(v, c, split, s);
    case QK_FP8_BLOCK: return launch_q<QK_FP8_BLOCK>(v, c, split, s);
    case QK_MXFP4: return c.M <= 16 ? launch_mx<1>(v, c, split, s) : launch_mx<2>(v, c, split, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace lg
