// launch.hpp -- host-side view of the kernel families: the variant record the
// shape-keyed table produces, the call record built by the C ABI, and the
// launchers each kernel source file provides.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.hpp"

namespace lg {

enum VariantKind : int { V_TILE = 0, V_DECODE = 1, V_PP = 2 };
// Cross-workgroup split-K reductions of the decode family.
enum Reduce : int { R_NONE = 0, R_LASTWG = 1, R_ATOMIC = 2, R_TWOPASS = 3 };

struct Variant {
  int kind = V_TILE;
  // tile family: workgroup tile BM (tokens) x BN (weight rows), WM x WN waves
  // (the ping-pong family has a fixed tile per quant mode and uses only
  // group_m and split; split = 0 picks the split-K factor from the shape)
  int bm = 128, bn = 128, wm = 2, wn = 2, group_m = 4;
  // tile family: sk > 0 = stream-K over sk x (CU count) persistent
  // workgroups (split is then unused), 0 = one workgroup per tile / split
  int sk = 0;
  // decode family (M <= 32): swap-AB orientation, split-K factor across
  // workgroups (0 = choose from the shape), reduction, waves per workgroup
  // (the in-workgroup K split), steps of 128 bytes loaded per batch, and
  // weight rows per workgroup (4..64, a multiple of 4; each activation load
  // feeds all of them)
  int swap = 1, split = 0, reduce = R_TWOPASS, waves = 8, unroll = 2, rows = 16;
  // lin_gemm_run_dynamic with a decode variant: 1 = quantize the activations
  // in the kernel's prologue where that variant supports it, 0 = in a
  // separate kernel first (the default: the prologue pays only for one token)
  int dq = 0;
  // decode family: 1 = stage the activations through LDS where the variant
  // is compiled for it (small M), 2 = e4m3 activations widened once per
  // wave into LDS (up to 16 tokens, where compiled; the grouped layer takes
  // it as 1), 0 = every lane loads its own
  int xs = 0;
};

struct Call {
  const void* A;
  const void* B;
  int64_t M, N, K;
  int64_t KB;       // bytes per operand row
  int qk;           // QKind
  Epi epi;
  void* ws;         // split-K workspace (decode family)
  int* counters;    // arrival counters, one per workgroup row group
};

// Tile family (kernels_tile.hip).  split > 1: K split across workgroups
// into c.ws ([split][M][N] fp32 / int32, tile_ws_bytes), then the two-pass
// reduction with the epilogue.
bool tile_supported(int qk, int bm, int bn, int wm, int wn);
// Whether the tile shape is compiled in stream-K form (v.sk > 0).
bool tile_sk_supported(int qk, int bm, int bn, int wm, int wn);
int tile_auto_split(const Variant& v, const Call& c);
// Workspace of a tile call: split-K slices [split][M][N], or the stream-K
// slices [slices][M][N] (v.sk > 0), of fp32 / int32 partials.
size_t tile_ws_bytes(const Variant& v, const Call& c, int split);
hipError_t launch_tile(const Variant& v, const Call& c, int split, hipStream_t s);

// Grouped tile form (a mixture-of-experts layer with prefill-sized
// segments): the tile kernel over every BM-row tile of every expert's
// segment (offsets as in launch_grouped), tile shapes from a short list.
bool grouped_tile_supported(int bm, int bn, int wm, int wn);
hipError_t launch_grouped_tile(const Variant& v, const Call& c, const int* offsets, int64_t E,
                               hipStream_t s);

// Ping-pong family (kernels_pp.hip): bf16 / fp16 / int8 256x256 tiles and
// block FP8 256x128 tiles with optional split-K over the scale blocks.
bool pp_supported(int qk);
int pp_auto_split(const Call& c);
size_t pp_ws_bytes(const Call& c, int split);
hipError_t launch_pp(const Variant& v, const Call& c, int split, hipStream_t s);

// Decode family (kernels_decode.hip).
bool decode_supported(int swap, int waves, int unroll, int rows);
bool decode_plain_supported(int swap, int waves, int unroll, int rows);
int decode_auto_split(const Call& c, const Variant& v);
size_t decode_ws_bytes(const Variant& v, const Call& c, int split);
hipError_t launch_decode(const Variant& v, const Call& c, int split, hipStream_t s);
// Decode with the quantization prologue: c.A holds bf16 activations X[M][K],
// c.KB = K, c.epi.sa is unused (per-token scales come from the prologue).
// Supported for swap, split 1, M <= 16, e4m3 / int8 / block e4m3, the
// variants the library compiles with it, and LDS within the device limit.
// With v.xs == 2 and per-token e4m3, where it fits, the prologue also widens
// the codes once per wave into LDS (the widened-activation form).
bool decode_dq_supported(const Variant& v, const Call& c, int split);
// Whether the decode variant is compiled for MXFP4 weights (swap, waves /
// unroll / tiles from a short list).
bool decode_mx_supported(const Variant& v);
// Decode with activations staged through LDS (AM_STAGE): e4m3, int8, block
// e4m3, MXFP4, bf16 and fp16 weights, swap, M <= 32, the variants compiled with
// it, LDS within the device limit.
bool decode_xs_supported(const Variant& v, const Call& c);
hipError_t launch_decode_xs(const Variant& v, const Call& c, int split, hipStream_t s);
// Whether the widened-activation form (v.xs == 2) runs this call.
bool decode_wd_supported(const Variant& v, const Call& c, int split);
hipError_t launch_decode_wd(const Variant& v, const Call& c, int split, hipStream_t s);
hipError_t launch_decode_dq(const Variant& v, const Call& c, hipStream_t s);
// Grouped decode (a mixture-of-experts layer): E experts, expert x owning
// rows [offsets[x], offsets[x+1]) of the [M] rows of c.A / C / residual, the
// weight c.B + x N KB and its scales and bias (per-expert strides of N
// rows); token chunks of 16 ntt rows (ntt 1 or 2), `chunks` workgroups deep
// per expert and weight-row group.  Variant: waves == 0 takes the default
// of (quant, ntt, xs); otherwise waves / unroll / rows pick a compiled
// grouped variant.  v.xs: activations staged through LDS.  Check
// grouped_supported first.
bool grouped_supported(const Variant& v, int qk, int ntt, int64_t KB);
hipError_t launch_grouped(const Variant& v, const Call& c, const int* offsets, int64_t E,
                          int ntt, int chunks, hipStream_t s);
// Second pass of a two-pass split-K reduction: sums the fp32 / int32 slices
// [split][M][N] in slice order and applies the epilogue.
hipError_t launch_splitk_reduce(int qk, const void* ws, int split, const Epi& e, hipStream_t s);

// Unfused three-kernel path and utilities (kernels_misc.hip).
hipError_t launch_bias_act(const void* T, const void* bias, void* U, int64_t M, int64_t N,
                           int act, bool f16, hipStream_t s);
hipError_t launch_scale_residual(const void* U, const void* residual, void* C, int64_t M,
                                 int64_t N, float alpha, bool f16, hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
// Raise kernel fn's dynamic-LDS limit to `bytes` on the current device, once
// per (kernel, device): the attribute is held per device, so a process
// that launches on several GPUs sets it on each (kernels_misc.hip).
hipError_t opt_in_lds(const void* fn, size_t bytes);
// Measurement only: read `bytes` (a multiple of 16) at src with `grid`
// workgroups of 256 threads, `unroll` (4, 8 or 16) 16-byte loads in flight
// per thread; sink (256 ints) is written only in the practically impossible
// case that the XOR of the data equals a fixed value.
hipError_t launch_stream_read(const void* src, int64_t bytes, int grid, int unroll, int* sink,
                              hipStream_t s);
// Dynamic activation quantization (kernels_quant.hip): X[M][K] 16-bit floats
// -> Q[M][K] codes and fp32 scales, per token ([M]) or per 1x128 block
// ([M][K/128]).  K % 16 == 0 (K % 128 == 0 for blocks), M >= 1.
enum DQKind : int { DQ_FP8_TOKEN = 0, DQ_INT8_TOKEN = 1, DQ_FP8_BLOCK = 2 };
hipError_t launch_dynamic_quant(int kind, bool f16, const void* X, int64_t M, int64_t K, void* Q,
                                float* scales, hipStream_t s);

}  // namespace lg
