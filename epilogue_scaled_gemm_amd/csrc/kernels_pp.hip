// kernels_pp.hip -- "ping-pong" MFMA tile GEMMs for the large, compute-bound
// shapes (prefill), with the fused epilogue.
//
// Same computation as kernels_tile.hip: the layer of the extensible-epilogue
// listing in "Совместная работа Helion и TorchInductor: слияние операторов"
// (tiles of C, an fp32 / int32 accumulator over K, bias / activation /
// narrowing applied to the accumulator before one store), with the scale
// formats of "helion-vllm-linear-backend" (section "Одно ядро вместо трёх
// вариантов"); for Block_FP8 the exact partial sum of every 128-wide K block
// is promoted with sa[m, kb] * sb[n / 128, kb] into the fp32 accumulator.
//
// gfx950 schedule (measured on MI355X against the one-group tile kernel):
//  * 8 waves, two per SIMD, in two groups of four (waves w and w + 4 share a
//    SIMD).  The groups alternate between a memory phase (LDS fragment reads,
//    issuing the global -> LDS loads of a later stage, VALU side work) and a
//    compute phase (MFMAs only, from registers); a workgroup barrier
//    separates consecutive phases and group 1 starts one phase late, so on
//    every SIMD one wave feeds the matrix core while the other fetches.
//  * Global -> LDS by buffer loads that write LDS directly, NBUF stages deep;
//    each group issues half of a stage's loads and waits for them (vmcnt) just
//    before the barrier that precedes the stage's first reader, so loads have
//    several phases of latency budget.
//  * Weight rows sit in LDS in fragment order (MFMA row l of tile j is weight
//    row l * FN + j), so each lane ends with 4 * FN consecutive output columns
//    of one token: the epilogue loads and stores 16-byte vectors.
//  * 16-byte chunks within an LDS row are XOR-swizzled by a function of the
//    row's low four bits; fragment reads start at 16-row boundaries, so one
//    lane address serves every fragment of a wave.
//
// Shapes: bf16 / fp16 / int8 use a 256 x 256 tile (wave tile 128 x 64,
// stages of 64 bytes of K per row, one memory + one compute phase per stage).
// Block FP8 uses a 256 x 128 tile (wave tile 64 x 64) with one 128-byte scale
// block per stage and two phase pairs per stage; e4m3 is widened exactly to
// bf16 in the compute phase, the previous block's promotion runs in the
// memory phase, and K may be split across workgroups (fp32 partials, then the
// two-pass reduction applies the epilogue).
#include "launch.hpp"

namespace lg {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt immediate for "vmcnt <= n" (expcnt and lgkmcnt not waited).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Chunk swizzles; both depend on the row's low four bits only.
// 64-byte rows (4 chunks): distinct for any 16 consecutive rows under both a
// 128-byte and a 256-byte LDS access width.
__device__ inline int swz4(int r) { return ((r >> 2) ^ (r >> 1)) & 3; }
// 128-byte rows (8 chunks), read as chunk 4 h + g by lane group g (h the
// half stage): rows r and r + 8 use complementary patterns, so the 32 lanes
// of two lane groups (16 rows x 2 chunks) fall on 32 distinct 16-byte bank
// groups of a 512-byte window as well as 16 lanes on 16 of a 256-byte one.
// (r & 7) ^ (r >> 3 & 1) measured 4 bank-conflict cycles per fragment read
// (SQ_LDS_BANK_CONFLICT = 4 x SQ_INSTS_LDS on the 2048-token block FP8 call).
__device__ inline int swz8(int r) { return (r & 7) ^ (((r >> 3) & 1) * 7); }

__device__ inline void tile_coords(int tiles_m, int tiles_n, int group_m, int BM, int BN, int64_t* m0,
                                   int64_t* n0) {
  // XCD-contiguous remap (ids are dealt round-robin over the 8 XCDs), then a
  // grouped raster so each XCD's tiles share operand panels in its L2.
  const int nblk = tiles_m * tiles_n;
  int L = blockIdx.x;
  if ((nblk & 7) == 0) L = (L & 7) * (nblk >> 3) + (L >> 3);
  const int gsz = group_m * tiles_n;
  const int grp = L / gsz;
  const int first_m = grp * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int within = L - grp * gsz;
  *m0 = (int64_t)(first_m + within % gm) * BM;
  *n0 = (int64_t)(within / gm) * BN;
}

// ------------------------------------------------ bf16 / fp16 / int8, 256x256
template <int QK>
__global__ __launch_bounds__(512, 1) void pp_kernel(const uint8_t* __restrict__ A,
                                                    const uint8_t* __restrict__ B, int64_t M,
                                                    int64_t N, int64_t KB, int tiles_m,
                                                    int tiles_n, int group_m, Epi e) {
  using MF = Mfma<QK>;
  using C = typename MF::C;
  using AccT = typename QTraits<QK>::Acc;
  constexpr int BM = 256, BN = 256, TM = 128, TN = 64, FM = 8, FN = 4;
  constexpr int RB = 64;                  // bytes of K per row per stage
  constexpr int NBUF = 3;
  constexpr int STAGE = (BM + BN) * RB;   // 32 KiB
  constexpr int LPW = 4;                  // loads (16 rows x 64 bytes) per wave per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp_w = wave >> 2;
  const int wave_m = wave & 1, wave_n = wave >> 1;
  const int g = lane >> 4, l16 = lane & 15;
  int64_t m0, n0;
  tile_coords(tiles_m, tiles_n, group_m, BM, BN, &m0, &n0);

  // Loads: waves 0..3 bring the 16 activation row groups of a stage, waves
  // 4..7 the 16 weight row groups; rows past M / N and chunks past K read 0.
  const bool ldA = grp_w == 0;
  const int a_rows = (int)min((int64_t)BM, M - m0), b_rows = (int)min((int64_t)BN, N - n0);
  const __amdgpu_buffer_rsrc_t rs = ldA
      ? __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * KB), (short)0, (int)(a_rows * KB), 0x00020000)
      : __builtin_amdgcn_make_buffer_rsrc((void*)(B + n0 * KB), (short)0, (int)(b_rows * KB), 0x00020000);
  const int lw = wave & 3;
  int off0[LPW], chk[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    const int R = (lw * LPW + q) * 16 + (lane >> 2);          // LDS row within the operand
    chk[q] = ((lane & 3) ^ swz4(R)) << 4;
    const int row = ldA ? R : (R / TN) * TN + (R % 16) * FN + (R % TN) / 16;
    off0[q] = row * (int)KB + chk[q];
  }
  const int ldsdst = (ldA ? 0 : BM * RB) + lw * LPW * 1024;
  auto dload = [&](int kt, int KT) {
    uint8_t* base = lds + (kt % NBUF) * STAGE + ldsdst;
    const int koff = kt * RB;
    const int kill = kt < KT ? 0 : 0x7FFFFFF0;   // stages past the end: no data
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int off = ((koff + chk[q] < KB) ? off0[q] + koff : 0x7FFFFFF0) | kill;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + q * 1024), 16, off, 0, 0, 0);
    }
  };

  const int ch = (g ^ swz4(l16)) << 4;
  const int a_lane = (wave_m * TM + l16) * RB + ch;
  const int b_lane = BM * RB + (wave_n * TN + l16) * RB + ch;
  typename MF::Frag fa[FM], fb[FN];
  C acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = C{0, 0, 0, 0};

  const int KT = (int)((KB + RB - 1) / RB);
#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t) dload(t, KT);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (grp_w == 1) __builtin_amdgcn_s_barrier();   // group 1 runs one phase behind
  for (int kt = 0; kt < KT; ++kt) {
    const uint8_t* base = lds + (kt % NBUF) * STAGE;
    // ---- memory phase
#pragma unroll
    for (int j = 0; j < FN; ++j) fb[j] = MF::prep(*(const i32x4*)(base + b_lane + j * 16 * RB));
#pragma unroll
    for (int i = 0; i < FM; ++i) fa[i] = MF::prep(*(const i32x4*)(base + a_lane + i * 16 * RB));
    dload(kt + NBUF - 1, KT);
#pragma unroll
    for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(fb[j]));
#pragma unroll
    for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(fa[i]));
    // group 1: its loads of stage kt + 1 have landed (group 0 reads it next)
    if (grp_w == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NBUF - 2) * LPW));
    __builtin_amdgcn_s_barrier();
    // ---- compute phase
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[i][j] = MF::mma(fb[j], fa[i], acc[i][j]);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(acc[i][j]));
    // group 0: its loads of stage kt + 1 have landed
    if (grp_w == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm((NBUF - 2) * LPW));
    __builtin_amdgcn_s_barrier();
  }
  if (grp_w == 0) __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_s_waitcnt(0);

  // Fused epilogue straight from the accumulator registers.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wave_m * TM + i * 16 + l16;
    const int64_t nb = n0 + wave_n * TN + g * 4 * FN;
    AccT v[4 * FN];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < FN; ++j) v[r * FN + j] = (AccT)acc[i][j][r];
    epilogue_run<4 * FN, QTraits<QK>::out_f16>(e, m, nb, v);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// ------------------------------------------------------- block FP8, 256x128
__global__ __launch_bounds__(512, 1) void bpp_kernel(const uint8_t* __restrict__ A,
                                                     const uint8_t* __restrict__ B, int64_t M,
                                                     int64_t N, int64_t KB, int tiles_m,
                                                     int tiles_n, int group_m, int blocks_per_split,
                                                     Epi e, float* __restrict__ ws) {
  using MF = Mfma<QK_FP8_BLOCK>;
  using Frag = typename MF::Frag;
  constexpr int BM = 256, BN = 128, TM = 64, TN = 64, FM = 4, FN = 4;
  constexpr int RB = 128;                 // one 128-wide scale block per stage
  constexpr int NBUF = 3;
  // A stage: the activation and weight tiles of one scale block, then the
  // block's activation scales of the tile's 256 rows (1 KiB) and its weight
  // scale (in a 1 KiB slot), all brought by direct-to-LDS loads.
  constexpr int SA_OFF = (BM + BN) * RB, SB_OFF = SA_OFF + 1024;
  constexpr int STAGE = SB_OFF + 1024;    // 50 KiB
  constexpr int LA = BM / 8 / 4, LB = BN / 8 / 4;  // loads (8 rows x 128 bytes) per wave per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp_w = wave >> 2;
  const int wave_m = wave & 3, wave_n = wave >> 2;
  const int g = lane >> 4, l16 = lane & 15;
  const int KBLK = (int)(KB / 128);
  int64_t m0, n0;
  tile_coords(tiles_m, tiles_n, group_m, BM, BN, &m0, &n0);
  // This workgroup's scale blocks (split-K slice blockIdx.y).
  const int kb0 = blockIdx.y * blocks_per_split;
  const int KT = max(0, min(KBLK, kb0 + blocks_per_split) - kb0);

  // Loads: group 0 brings the 32 activation row groups of a stage (8 per
  // wave), group 1 the 16 weight row groups (4 per wave).
  const bool ldA = grp_w == 0;
  const int a_rows = (int)min((int64_t)BM, M - m0), b_rows = (int)min((int64_t)BN, N - n0);
  const __amdgpu_buffer_rsrc_t rs = ldA
      ? __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * KB), (short)0, (int)(a_rows * KB), 0x00020000)
      : __builtin_amdgcn_make_buffer_rsrc((void*)(B + n0 * KB), (short)0, (int)(b_rows * KB), 0x00020000);
  const int lw = wave & 3;
  const int nld = ldA ? LA : LB;
  int off0[LA];
#pragma unroll
  for (int q = 0; q < LA; ++q) {
    const int R = (lw * nld + q) * 8 + (lane >> 3);
    const int chk = ((lane & 7) ^ swz8(R)) << 4;
    const int row = ldA ? R : (R / TN) * TN + (R % 16) * FN + (R % TN) / 16;
    off0[q] = row * (int)KB + chk;
  }
  const int ldsdst = ldA ? lw * LA * 1024 : BM * RB + lw * LB * 1024;
  // Scales: group 0's wave lw brings sa[m0 + 64 lw + lane][kb] (rows past M
  // read 0 through the bounds and their outputs are never stored); group
  // 1's wave 4 brings sb[n0 / 128][kb] in its lane 0 (the other lanes' and
  // waves' offsets lie past the buffer: no access).
  const __amdgpu_buffer_rsrc_t rss = ldA
      ? __builtin_amdgcn_make_buffer_rsrc((void*)(e.sa + m0 * KBLK), (short)0, a_rows * KBLK * 4, 0x00020000)
      : __builtin_amdgcn_make_buffer_rsrc((void*)(e.sb + (n0 / 128) * KBLK), (short)0, KBLK * 4, 0x00020000);
  const int soff0 = ldA ? (lw * 64 + lane) * KBLK * 4 : ((lw == 0 && lane == 0) ? 0 : 0x7FFFFFF0);
  const int sdst = ldA ? SA_OFF + lw * 256 : SB_OFF + lw * 256;
  auto dload = [&](int kt) {
    uint8_t* sbase = lds + (kt % NBUF) * STAGE;
    uint8_t* base = sbase + ldsdst;
    const int koff = (kb0 + kt) * RB;
    const int kill = kt < KT ? 0 : 0x7FFFFFF0;
    if (ldA) {
#pragma unroll
      for (int q = 0; q < LA; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + q * 1024), 16, (off0[q] + koff) | kill, 0, 0, 0);
    } else {
#pragma unroll
      for (int q = 0; q < LB; ++q)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void*)(base + q * 1024), 16, (off0[q] + koff) | kill, 0, 0, 0);
    }
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rss, (lds_void*)(sbase + sdst), 4,
                                             (soff0 + (kb0 + kt) * 4) | kill, 0, 0, 0);
  };
  // The scales of block kt are read from its stage (sa per token, i.e. per
  // lane; sb uniform: the tile's 128 weight rows are one 128-row block).
  float sc_prev[FM];

  const int sw = swz8(l16);
  const int a_lane = (wave_m * TM + l16) * RB;
  const int b_lane = BM * RB + (wave_n * TN + l16) * RB;
  f32x4 acc[FM][FN], p[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    sc_prev[i] = 0.f;
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = p[i][j] = f32x4{0, 0, 0, 0};
  }

#pragma unroll
  for (int t = 0; t < NBUF - 1; ++t) dload(t);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (grp_w == 1) __builtin_amdgcn_s_barrier();
  for (int kt = 0; kt < KT; ++kt) {
    const uint8_t* base = lds + (kt % NBUF) * STAGE;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // ---- memory phase: raw fragments of this half block; at h == 0 the
      // loads of a later stage and the previous block's promotion
      const int ch = ((4 * h + g) ^ sw) << 4;
      i32x4 rw[FN], ra[FM];
#pragma unroll
      for (int j = 0; j < FN; ++j) rw[j] = *(const i32x4*)(base + b_lane + j * 16 * RB + ch);
#pragma unroll
      for (int i = 0; i < FM; ++i) ra[i] = *(const i32x4*)(base + a_lane + i * 16 * RB + ch);
      if (h == 0) {
        dload(kt + NBUF - 1);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] += sc_prev[i] * p[i][j];
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(acc[i][j]));
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(rw[j]));
#pragma unroll
      for (int i = 0; i < FM; ++i) asm volatile("" : "+v"(ra[i]));
      // group 1: the loads of stage kt + 1 have landed (the LB + 1 of stage
      // kt + 2 may still be in flight)
      if (h == 1 && grp_w == 1) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LB + 1));
      __builtin_amdgcn_s_barrier();
      // ---- compute phase: widen just in time, MFMA into the block partial
      Frag xa[FM];
#pragma unroll
      for (int i = 0; i < FM; ++i) xa[i] = MF::prep(ra[i]);
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const Frag w = MF::prep(rw[j]);
#pragma unroll
        for (int i = 0; i < FM; ++i) p[i][j] = MF::mma(w, xa[i], h == 0 ? f32x4{0, 0, 0, 0} : p[i][j]);
      }
      if (h == 1) {
        // group 0: the loads of stage kt + 1 have landed
        if (grp_w == 0) __builtin_amdgcn_s_waitcnt(vmcnt_imm(LA + 1));
        const float sbv = *(const float*)(base + SB_OFF);
#pragma unroll
        for (int i = 0; i < FM; ++i)
          sc_prev[i] = *(const float*)(base + SA_OFF + (wave_m * TM + i * 16 + l16) * 4) * sbv;
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) asm volatile("" : "+v"(p[i][j]));
      __builtin_amdgcn_s_barrier();
    }
  }
  if (grp_w == 0) __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] += sc_prev[i] * p[i][j];

#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + wave_m * TM + i * 16 + l16;
    const int64_t nb = n0 + wave_n * TN + g * 4 * FN;
    float v[4 * FN];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < FN; ++j) v[r * FN + j] = acc[i][j][r];
    if (gridDim.y == 1) {
      epilogue_run<4 * FN, false>(e, m, nb, v);
    } else if (m < M) {
      // split-K slice: fp32 partial into the workspace [split][M][N]
      float* row = ws + ((int64_t)blockIdx.y * M + m) * N + nb;
      if (nb + 4 * FN <= N) {
#pragma unroll
        for (int q = 0; q < 4 * FN; q += 4) *(f32x4*)(row + q) = f32x4{v[q], v[q + 1], v[q + 2], v[q + 3]};
      } else {
        for (int q = 0; q < 4 * FN; ++q)
          if (nb + q < N) row[q] = v[q];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int QK>
hipError_t launch_pp_q(const Variant& v, const Call& c, hipStream_t s) {
  constexpr size_t lds = 3 * (256 + 256) * 64;
  hipError_t err = opt_in_lds((const void*)pp_kernel<QK>, lds);
  if (err != hipSuccess) return err;
  const int tiles_m = (int)((c.M + 255) / 256), tiles_n = (int)((c.N + 255) / 256);
  const int group_m = v.group_m > 0 ? v.group_m : 4;
  hipLaunchKernelGGL(pp_kernel<QK>, dim3(tiles_m * tiles_n), dim3(512), lds, s, (const uint8_t*)c.A,
                     (const uint8_t*)c.B, c.M, c.N, c.KB, tiles_m, tiles_n, group_m, c.epi);
  return hipGetLastError();
}

}  // namespace

bool pp_supported(int qk) {
  return qk == QK_BF16 || qk == QK_FP16 || qk == QK_I8 || qk == QK_FP8_BLOCK;
}

namespace {
int pp_split_blocks(const Call& c, int split) {
  const int kblk = (int)(c.KB / 128);
  return (kblk + split - 1) / split;
}
}  // namespace

// Split-K only for block FP8: double the slices while the grid is under one
// workgroup per CU and every slice keeps at least 8 scale blocks.
int pp_auto_split(const Call& c) {
  if (c.qk != QK_FP8_BLOCK) return 1;
  const int64_t tiles = ((c.M + 255) / 256) * ((c.N + 127) / 128);
  const int64_t kblk = c.KB / 128;
  int split = 1;
  while (tiles * split < 256 && kblk / (split * 2) >= 8 && split < 16) split *= 2;
  return split;
}

size_t pp_ws_bytes(const Call& c, int split) {
  return split > 1 ? (size_t)split * c.M * c.N * 4 : 0;
}

hipError_t launch_pp(const Variant& v, const Call& c, int split, hipStream_t s) {
  switch (c.qk) {
    case QK_BF16: return launch_pp_q<QK_BF16>(v, c, s);
    case QK_FP16: return launch_pp_q<QK_FP16>(v, c, s);
    case QK_I8: return launch_pp_q<QK_I8>(v, c, s);
    case QK_FP8_BLOCK: {
      constexpr size_t lds = 3 * ((256 + 128) * 128 + 2048);
      hipError_t err = opt_in_lds((const void*)bpp_kernel, lds);
      if (err != hipSuccess) return err;
      const int tiles_m = (int)((c.M + 255) / 256), tiles_n = (int)((c.N + 127) / 128);
      const int group_m = v.group_m > 0 ? v.group_m : 4;
      const int bps = pp_split_blocks(c, split);
      hipLaunchKernelGGL(bpp_kernel, dim3(tiles_m * tiles_n, split), dim3(512), lds, s,
                         (const uint8_t*)c.A, (const uint8_t*)c.B, c.M, c.N, c.KB, tiles_m, tiles_n,
                         group_m, bps, c.epi, (float*)c.ws);
      err = hipGetLastError();
      if (err != hipSuccess || split == 1) return err;
      return launch_splitk_reduce(c.qk, c.ws, split, c.epi, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace lg
