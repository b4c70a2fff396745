// kernels_tile.hip -- LDS-staged MFMA tile GEMM with the fused epilogue, for
// any M (prefill and medium batches) in every quant mode.
//
// What it computes is the layer of the extensible-epilogue listing in
// "Совместная работа Helion и TorchInductor: слияние операторов" (a 2-D grid
// of output tiles, an fp32 accumulator over a K loop of masked tile loads,
// then bias / activation / narrowing on the accumulator and one masked
// store), extended with the scale formats of "helion-vllm-linear-backend"
// (section "Одно ядро вместо трёх вариантов"): per-token x per-channel scales
// applied in the epilogue, and 1x128 / 128x128 block scales applied once per
// 128-wide K block inside the loop.
//
// gfx950 design (not the listing's):
//  * Weight rows go on the MFMA row side and tokens on the column side, and
//    MFMA row i of the wave's j-th tile holds weight row i * FN + j.  Each
//    lane therefore ends the K loop owning 4*FN consecutive output columns of
//    one row, so bias / scale / residual loads and the store are 16-byte
//    vectors.
//  * K advances in 128-byte stages: buffer loads straight into LDS (no
//    staging registers; 8 lanes per 128-byte row), double buffered, with
//    16-byte chunks XOR swizzled and weight rows stored in fragment order so
//    the MFMA fragment reads are free of bank conflicts -> registers -> MFMA (16x16x32 bf16/fp16, 16x16x64 int8;
//    e4m3 is widened exactly to bf16 in registers and uses the 16x16x32 bf16
//    MFMA).
//  * Workgroup ids are remapped so that each XCD (ids are dealt round-robin
//    over the 8 XCDs) gets a contiguous, grouped block of tiles, which keeps
//    the operand panels it shares in its own L2.
//  * Rows past M / N and 16-byte chunks past the end of K read as zero
//    (buffer bounds); rows past M / N are masked on store.
//  * Split-K (few output tiles, medium M): workgroup row y of the grid
//    takes K stages [y * kt_per, (y + 1) * kt_per) and stores its raw fp32 /
//    int32 tile into slice y of a [split][M][N] workspace; the decode
//    family's two-pass reduction then sums the slices in order and applies
//    the epilogue.
//  * MXFP4 weights (4-bit E2M1 codes with an E8M0 scale per 32 K values)
//    against bf16 activations: a stage is 64 K values, 128 bytes of an
//    activation row and 32 bytes of a weight row.  Weight rows sit in LDS at
//    32 bytes each, their two 16-byte halves swapped on every other group of
//    8 rows, so the 8-byte fragment reads of 16 rows hit distinct banks.
//    Each lane widens its 8 weights of a k-step times their block scale to
//    bf16 in registers (exact) and the bf16 MFMA takes them; the scales are
//    read from memory one stage ahead.
#include <algorithm>

#include "launch.hpp"

namespace lg {
namespace {

constexpr int ROWB = 128;  // bytes of K per stage row

// RB: bytes of a weight row per stage (128, or 32 for 4-bit weights).
template <int BM, int BN, int WM, int WN, int RB = ROWB>
struct TileShape {
  static constexpr int NT = WM * WN * 64;
  static constexpr int TM = BM / WM, TN = BN / WN;
  static constexpr int FM = TM / 16, FN = TN / 16;
  static constexpr int STAGE = BM * ROWB + BN * RB;
  static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile");
};

// 16-byte chunk swizzle of LDS row R: chunk c of row R is stored at position
// c ^ swz(R).  Distinct for any 16 consecutive rows, so the 16 lanes that
// read one chunk of 16 consecutive rows in a pass hit 16 different
// 16-byte bank groups (64 banks x 4 bytes = two 128-byte rows).
__device__ inline int swz(int r) { return (r ^ (r >> 3)) & 7; }

// The body of the tile kernel: the workgroup computes the BM x BN output tile
// at (m0, n0) over K stages [kt0, kt1) (kt1 = -1: to the end of K); with
// `part` it stores the raw accumulator tile there ([M][N]) instead of
// running the epilogue.
template <int QK, int BM, int BN, int WM, int WN>
__device__ __forceinline__ void tile_body(const uint8_t* __restrict__ A,
                                          const uint8_t* __restrict__ B, int64_t M, int64_t N,
                                          int64_t KB, int64_t m0, int64_t n0, Epi e,
                                          int kt0 = 0, int kt1 = -1,
                                          typename QTraits<QK>::Acc* __restrict__ part = nullptr) {
  // MXFP4: KB is the weight row's bytes (K / 2); activation rows have
  // XR = 4 times as many bytes (bf16).
  constexpr bool MX = (QK == QK_MXFP4);
  constexpr int XR = MX ? 4 : 1;
  constexpr int RB = MX ? 32 : ROWB;  // weight bytes per row per stage
  using S = TileShape<BM, BN, WM, WN, RB>;
  using MF = Mfma<QK>;
  using C = typename MF::C;
  using AccT = typename QTraits<QK>::Acc;
  constexpr int FM = S::FM, FN = S::FN, TM = S::TM, TN = S::TN;
  constexpr bool BLOCK = (QK == QK_FP8_BLOCK);
  static_assert(!BLOCK || (128 % TN == 0), "a wave's columns must sit in one 128-row scale block");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wave_m = wave % WM, wave_n = wave / WM;
  const int g = lane >> 4, l16 = lane & 15;

  // Global -> LDS: buffer loads that write straight into LDS (no staging
  // registers).  One instruction moves 8 rows x 128 bytes: lane i lands at
  // LDS row i / 8, 16-byte position i % 8, and fetches the global chunk
  // that the swizzle puts there.  The buffer resources cover only this
  // tile's valid rows, and chunks past the end of K get an out-of-range
  // offset, so both read as zero.
  constexpr int NW = WM * WN;
  // Rows per direct-load instruction: 8 of 128 bytes, or 32 weight rows of
  // 32 bytes (two lanes per row).
  constexpr int BG = MX ? 32 : 8;
  constexpr int A_OCT = BM / 8 / NW, B_OCT = BN / BG / NW;  // instructions per wave per stage
  static_assert(BM % (8 * NW) == 0 && BN % (BG * NW) == 0, "direct-load split");
  const int64_t KA = KB * XR;  // bytes of an activation row
  const int a_rows = (int)min((int64_t)BM, M - m0), b_rows = (int)min((int64_t)BN, N - n0);
  const __amdgpu_buffer_rsrc_t rsrc_a =
      __builtin_amdgcn_make_buffer_rsrc((void*)(A + m0 * KA), (short)0, (int)(a_rows * KA), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_b =
      __builtin_amdgcn_make_buffer_rsrc((void*)(B + n0 * KB), (short)0, (int)(b_rows * KB), 0x00020000);
  // Weight rows sit in LDS in the order the fragments read them: within a
  // wave's TN-row section, LDS row j*16 + l holds weight row l*FN + j.
  int a_off[A_OCT], b_off[B_OCT], a_chk[A_OCT], b_chk[B_OCT];
#pragma unroll
  for (int i = 0; i < A_OCT; ++i) {
    const int r = (wave * A_OCT + i) * 8 + (lane >> 3);
    a_chk[i] = ((lane & 7) ^ swz(r)) << 4;
    a_off[i] = r * (int)KA + a_chk[i];
  }
#pragma unroll
  for (int i = 0; i < B_OCT; ++i) {
    // LDS row in the tile; with 4-bit weights, lane i fills half i % 2 of
    // row i / 2 with the half that the swap puts there.
    const int R = (wave * B_OCT + i) * BG + (MX ? (lane >> 1) : (lane >> 3));
    const int sec = R / TN, Rs = R % TN;
    const int r = sec * TN + (Rs % 16) * FN + Rs / 16;    // weight row in the tile
    b_chk[i] = MX ? (((lane & 1) ^ ((R >> 3) & 1)) << 4) : (((lane & 7) ^ swz(R)) << 4);
    b_off[i] = r * (int)KB + b_chk[i];
  }
  typedef __attribute__((address_space(3))) void lds_void;
  auto dload = [&](int kt, int buf) {
    uint8_t* base = lds + buf * S::STAGE;
    const int koff = kt * ROWB, kboff = kt * RB;
#pragma unroll
    for (int i = 0; i < A_OCT; ++i) {
      const int off = (koff + a_chk[i] < KA) ? a_off[i] + koff : 0x7FFFFFF0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_a, (lds_void*)(base + (wave * A_OCT + i) * 1024),
                                               16, off, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_OCT; ++i) {
      const int off = (kboff + b_chk[i] < KB) ? b_off[i] + kboff : 0x7FFFFFF0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc_b,
                                               (lds_void*)(base + BM * ROWB + (wave * B_OCT + i) * 1024),
                                               16, off, 0, 0, 0);
    }
  };

  // Fragment rows (within the stage) of this lane.
  // MFMA row l16 of weight tile j is weight row l16 * FN + j, i.e. LDS row
  // j * 16 + l16 of the wave's section.
  int fa_row[FM], fw_row[FN];
#pragma unroll
  for (int i = 0; i < FM; ++i) fa_row[i] = wave_m * TM + i * 16 + l16;
#pragma unroll
  for (int j = 0; j < FN; ++j) fw_row[j] = wave_n * TN + j * 16 + l16;
  auto a_frag16 = [&](const uint8_t* base, int i, int ch) {
    const int r = fa_row[i];
    return *(const i32x4*)(base + r * ROWB + ((ch ^ swz(r)) << 4));
  };
  auto w_frag16 = [&](const uint8_t* base, int j, int ch) {
    const int r = fw_row[j];
    return *(const i32x4*)(base + BM * ROWB + r * ROWB + ((ch ^ swz(r)) << 4));
  };
  // 4-bit weights: this lane's 8 bytes of the stage (16 K values, k-steps 0
  // and 1 of its lane group: bytes 8 g .. 8 g + 8 of the 32-byte row).
  auto w_frag_mx = [&](const uint8_t* base, int j) {
    const int r = fw_row[j];
    return *(const i32x2*)(base + BM * ROWB + r * RB + ((((g >> 1) ^ ((r >> 3) & 1))) << 4) +
                           (g & 1) * 8);
  };
  // E8M0 scales [N][KB / 16] of this lane's weight rows; a stage spans two
  // 32-value blocks and lane group g's values sit in block g / 2.  Rows past
  // N read the last row (their outputs are never stored).
  const uint8_t* msp[MX ? FN : 1];
  if constexpr (MX) {
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int64_t n = min(n0 + wave_n * TN + l16 * FN + j, N - 1);
      msp[j] = (const uint8_t*)e.sb + n * (KB / 16) + (g >> 1);
    }
  }
  uint32_t msc_cur[MX ? FN : 1], msc_nxt[MX ? FN : 1];
  auto mload = [&](int kt, uint32_t* o) {
    if constexpr (MX) {
#pragma unroll
      for (int j = 0; j < FN; ++j) o[j] = msp[j][kt * 2];
    }
  };

  // Block scales: sb is uniform over a wave's columns, sa varies per lane.
  const int64_t KBLK = KB / 128;
  const float* sa_ptr[FM];
  const float* sb_ptr = nullptr;
  if constexpr (BLOCK) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      sa_ptr[i] = e.sa + min(m0 + fa_row[i], M - 1) * KBLK;
    // Columns past N (a partial last tile) clamp to the last scale block;
    // their outputs are never stored.
    const int64_t nb = min((n0 + wave_n * TN) / 128, (N + 127) / 128 - 1);
    sb_ptr = e.sb + nb * KBLK;
  }

  // Block scales of the stage being computed (cur) and of the next one,
  // fetched together with that stage's tiles.
  float sa_cur[FM], sa_nxt[FM], sb_cur = 0.f, sb_nxt = 0.f;
  auto sload = [&](int kt, float* sa_o, float& sb_o) {
    if constexpr (BLOCK) {
#pragma unroll
      for (int i = 0; i < FM; ++i) sa_o[i] = sa_ptr[i][kt];
      sb_o = sb_ptr[kt];
    }
  };
#pragma unroll
  for (int i = 0; i < FM; ++i) sa_cur[i] = sa_nxt[i] = 0.f;

  C acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = C{0, 0, 0, 0};

  const int KT = kt1 < 0 ? (int)((KB + RB - 1) / RB) : kt1;
  dload(kt0, 0);
  sload(kt0, sa_cur, sb_cur);
  mload(kt0, msc_cur);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = kt0; kt < KT; ++kt) {
    const uint8_t* base = lds + ((kt - kt0) & 1) * S::STAGE;
    if (kt + 1 < KT) {
      dload(kt + 1, (kt + 1 - kt0) & 1);
      sload(kt + 1, sa_nxt, sb_nxt);
      mload(kt + 1, msc_nxt);
    }
    if constexpr (MX) {
      i32x2 wr[FN];
      float wsc[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        wr[j] = w_frag_mx(base, j);
        wsc[j] = e8m0_to_f32(msc_cur[j]);
      }
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        typename MF::Frag wf[FN], af[FM];
#pragma unroll
        for (int j = 0; j < FN; ++j) wf[j] = mx_widen8((uint32_t)wr[j][s], wsc[j]);
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = MF::prep(a_frag16(base, i, 2 * g + s));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = MF::mma(wf[j], af[i], acc[i][j]);
      }
    } else if constexpr (!BLOCK) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        typename MF::Frag wf[FN], af[FM];
#pragma unroll
        for (int j = 0; j < FN; ++j) wf[j] = MF::prep(w_frag16(base, j, 2 * g + s));
#pragma unroll
        for (int i = 0; i < FM; ++i) af[i] = MF::prep(a_frag16(base, i, 2 * g + s));
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
          for (int j = 0; j < FN; ++j) acc[i][j] = MF::mma(wf[j], af[i], acc[i][j]);
      }
    } else {
      // One K stage is one 128-wide scale block: its exact partial sum p is
      // promoted with sa[m, kb] * sb[n / 128, kb] into the fp32 accumulator.
      typename MF::Frag wf0[FN], wf1[FN];
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        wf0[j] = MF::prep(w_frag16(base, j, 2 * g));
        wf1[j] = MF::prep(w_frag16(base, j, 2 * g + 1));
      }
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const typename MF::Frag a0 = MF::prep(a_frag16(base, i, 2 * g));
        const typename MF::Frag a1 = MF::prep(a_frag16(base, i, 2 * g + 1));
        const float sc = sa_cur[i] * sb_cur;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          C p = MF::mma(wf0[j], a0, C{0, 0, 0, 0});
          p = MF::mma(wf1[j], a1, p);
          acc[i][j] += sc * p;
        }
      }
    }
    // This wave's loads of the next stage have landed in LDS; the barrier
    // then covers every wave's loads and every wave's reads of this stage.
    __builtin_amdgcn_s_waitcnt(0);
    if constexpr (BLOCK) {
#pragma unroll
      for (int i = 0; i < FM; ++i) sa_cur[i] = sa_nxt[i];
      sb_cur = sb_nxt;
    }
    if constexpr (MX) {
#pragma unroll
      for (int j = 0; j < FN; ++j) msc_cur[j] = msc_nxt[j];
    }
    __syncthreads();
  }

  // Split-K slice: the raw tile, 4 FN consecutive columns per lane and row.
  if (part) {
#pragma unroll
    for (int i = 0; i < FM; ++i) {
      const int64_t m = m0 + fa_row[i];
      const int64_t nb = n0 + wave_n * TN + g * 4 * FN;
      if (m >= M) continue;
      AccT* row = part + m * N + nb;
      if (nb + 4 * FN <= N && N % 4 == 0) {
#pragma unroll
        for (int q = 0; q < FN; ++q) {
          typedef __attribute__((ext_vector_type(4))) AccT acc4;
          acc4 w;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int c = 4 * q + t;  // column nb + c holds acc[i][c % FN][c / FN]
            w[t] = (AccT)acc[i][c % FN][c / FN];
          }
          *(acc4*)(row + 4 * q) = w;
        }
      } else {
#pragma unroll
        for (int c = 0; c < 4 * FN; ++c)
          if (nb + c < N) row[c] = (AccT)acc[i][c % FN][c / FN];
      }
    }
    return;
  }

  // Fused epilogue straight from the accumulator registers.
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const int64_t m = m0 + fa_row[i];
    const int64_t nb = n0 + wave_n * TN + g * 4 * FN;
    AccT v[4 * FN];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int j = 0; j < FN; ++j) v[r * FN + j] = (AccT)acc[i][j][r];
    epilogue_run<4 * FN, QTraits<QK>::out_f16>(e, m, nb, v);
    // One accumulator row group at a time: keeps the scheduler from hoisting
    // every row's residual loads (which would not fit beside the
    // accumulators).
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int QK, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void tile_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, int64_t M, int64_t N,
    int64_t KB, int tiles_m, int tiles_n, int group_m, Epi e, int split, int kt_per,
    void* __restrict__ ws) {
  // Tile coordinates: XCD-contiguous remap, then a grouped raster.
  const int nblk = tiles_m * tiles_n;
  int L = blockIdx.x;
  if ((nblk & 7) == 0) L = (L & 7) * (nblk >> 3) + (L >> 3);
  const int gsz = group_m * tiles_n;
  const int grp = L / gsz;
  const int first_m = grp * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int within = L - grp * gsz;
  const int64_t m0 = (int64_t)(first_m + within % gm) * BM;
  const int64_t n0 = (int64_t)(within / gm) * BN;
  using AccT = typename QTraits<QK>::Acc;
  int kt0 = 0, kt1 = -1;
  AccT* part = nullptr;
  if (split > 1) {
    constexpr int RB = QK == QK_MXFP4 ? 32 : ROWB;
    const int KT = (int)((KB + RB - 1) / RB);
    kt0 = (int)blockIdx.y * kt_per;
    kt1 = min(kt0 + kt_per, KT);
    part = (AccT*)ws + (int64_t)blockIdx.y * M * N;
    if (kt0 >= kt1) {
      // An empty slice (K shorter than split x kt_per): its partials are zero.
      for (int64_t t = threadIdx.x; t < (int64_t)BM * BN; t += blockDim.x) {
        const int64_t m = m0 + t / BN, n = n0 + t % BN;
        if (m < M && n < N) part[m * N + n] = 0;
      }
      return;
    }
  }
  tile_body<QK, BM, BN, WM, WN>(A, B, M, N, KB, m0, n0, e, kt0, kt1, part);
}

// ---------------------------------------------------------------- stream-K
//
// For shapes whose tile count leaves CUs idle (or gives an uneven last wave
// of tiles), the stream-K form of the split-K idea in
// "helion-vllm-linear-backend" (sections "Зачем трогать линейные слои" and
// "Одно ядро вместо трёх вариантов"): the tiles' K stages form one sequence
// of T x KT units, and P persistent workgroups take equal contiguous runs of
// it, so every CU has the same amount of MFMA work whatever T is.  Tiles
// [0, T_dp) go whole to one workgroup each first (data-parallel part); the
// remaining tiles' units are divided among the other P workgroups.  A tile
// that one workgroup covers entirely gets the fused epilogue at once; a
// tile split between workgroups gets each piece's raw accumulator written
// to slice (workgroup - first workgroup of the tile) of a [slices][M][N]
// workspace, and the fix-up kernel sums the slices in order and runs the
// epilogue (deterministic, no waiting between workgroups).

// First unit of stream-K workgroup j of P over `total` units.
__device__ __host__ inline int64_t sk_begin(int64_t j, int64_t total, int64_t P) {
  return j * total / P;
}

// The stream-K workgroup whose run holds unit u.
__device__ inline int64_t sk_owner(int64_t u, int64_t total, int64_t P) {
  int64_t j = u * P / total;
  while (j + 1 < P && sk_begin(j + 1, total, P) <= u) ++j;
  while (j > 0 && sk_begin(j, total, P) > u) --j;
  return j;
}

__device__ inline void sk_tile_coords(int t, int tiles_m, int tiles_n, int group_m, int BM, int BN,
                                      int64_t* m0, int64_t* n0) {
  const int gsz = group_m * tiles_n;
  const int grp = t / gsz;
  const int first_m = grp * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int within = t - grp * gsz;
  *m0 = (int64_t)(first_m + within % gm) * BM;
  *n0 = (int64_t)(within / gm) * BN;
}

template <int QK, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void tile_sk_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B, int64_t M, int64_t N,
    int64_t KB, int tiles_m, int tiles_n, int group_m, Epi e, int KT, int t_dp, int P,
    void* __restrict__ ws) {
  using AccT = typename QTraits<QK>::Acc;
  const int T = tiles_m * tiles_n;
  // Units: tile t's K stages are t KT .. t KT + KT - 1.  Workgroup g < t_dp
  // takes data-parallel tile g whole; workgroup t_dp + j takes run j of the
  // stream-K units [t_dp KT, T KT).  One tile_body call site (it is large).
  const int64_t j = (int64_t)blockIdx.x - t_dp;
  const int64_t sk0 = (int64_t)t_dp * KT, total = (int64_t)(T - t_dp) * KT;
  int64_t u0, u1;
  if (j < 0) {
    u0 = (int64_t)blockIdx.x * KT;
    u1 = u0 + KT;
  } else {
    u0 = sk0 + sk_begin(j, total, P);
    u1 = sk0 + sk_begin(j + 1, total, P);
  }
  for (int64_t u = u0; u < u1;) {
    const int t = (int)(u / KT);
    const int64_t tb = (int64_t)t * KT;
    const int k0 = (int)(u - tb), k1 = (int)(min(u1, tb + KT) - tb);
    int64_t m0, n0;
    sk_tile_coords(t, tiles_m, tiles_n, group_m, BM, BN, &m0, &n0);
    AccT* part = nullptr;
    if (k0 != 0 || k1 != KT) part = (AccT*)ws + (j - sk_owner(tb - sk0, total, P)) * M * N;
    if (u != u0) __syncthreads();  // the previous tile is done with the LDS
    tile_body<QK, BM, BN, WM, WN>(A, B, M, N, KB, m0, n0, e, k0, k1, part);
    u = tb + k1;
  }
}

// Fix-up: workgroup t sums the slices of stream-K tile t (if it was split)
// in slice order, four consecutive columns per thread, then the epilogue.
template <int QK, int BM, int BN>
__global__ __launch_bounds__(256) void tile_sk_fixup(const void* __restrict__ ws, int tiles_m,
                                                     int tiles_n, int group_m, int KT, int t_dp,
                                                     int P, Epi e) {
  using AccT = typename QTraits<QK>::Acc;
  const int T = tiles_m * tiles_n;
  const int t = blockIdx.x;
  const int64_t total = (int64_t)(T - t_dp) * KT;
  const int64_t tb = (int64_t)t * KT;
  const int64_t g0 = sk_owner(tb, total, P), g1 = sk_owner(tb + KT - 1, total, P);
  if (g0 == g1) return;  // one workgroup ran the whole tile and its epilogue
  int64_t m0, n0;
  sk_tile_coords(t_dp + t, tiles_m, tiles_n, group_m, BM, BN, &m0, &n0);
  const AccT* w = (const AccT*)ws;
  for (int q = threadIdx.x; q < BM * (BN / 4); q += 256) {
    const int64_t m = m0 + q / (BN / 4), n = n0 + (q % (BN / 4)) * 4;
    if (m >= e.M || n >= e.N) continue;
    AccT v[4] = {0, 0, 0, 0};
    for (int64_t sg = 0; sg <= g1 - g0; ++sg) {
      const AccT* row = w + (sg * e.M + m) * e.N;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (n + i < e.N) v[i] += row[n + i];
    }
    epilogue_run<4, QTraits<QK>::out_f16>(e, m, n, v);
  }
}

// The t-th BM-row tile of a token-sorted grouped layer, in expert order:
// expert x's segment [lo, hi) (offsets clamped into [0, M], an end below
// its start empty) holds tiles ceil((hi - lo) / BM); x = -1 when there are
// at most t tiles.  Each wave computes it alone: 64 experts at a time, a
// prefix sum of their tile counts across the lanes, a ballot for the lane
// whose range holds t.
__device__ inline void kth_tile(const int* __restrict__ offsets, int E, int M, int bm, int t,
                                int& x, int& lo, int& hi, int& r0) {
  const int lane = threadIdx.x & 63;
  x = -1; lo = 0; hi = 0; r0 = 0;
  int run = 0;  // tiles of the experts before this group of 64
  for (int base = 0; base < E; base += 64) {
    const int i = base + lane;
    int l = 0, h = 0;
    if (i < E) {
      l = min(max(offsets[i], 0), M);
      h = min(max(offsets[i + 1], l), M);
    }
    const int c = (h - l + bm - 1) / bm;
    int incl = c;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int total = __shfl(incl, 63);
    if (t < run + total) {
      const bool here = run + incl - c <= t && t < run + incl;
      const int src = __ffsll((unsigned long long)__ballot(here)) - 1;
      x = __builtin_amdgcn_readfirstlane(base + src);
      lo = __builtin_amdgcn_readfirstlane(__shfl(l, src));
      hi = __builtin_amdgcn_readfirstlane(__shfl(h, src));
      const int before = __builtin_amdgcn_readfirstlane(__shfl(incl - c, src));
      r0 = lo + (t - run - before) * bm;
      return;
    }
    run += total;
  }
}

// Grouped (mixture-of-experts) form for segments of prefill size: workgroup
// (blockIdx.x, blockIdx.y) computes n-tile blockIdx.x of the blockIdx.y-th
// BM-row tile in expert order, against that expert's weight B[x] (N rows of
// KB bytes), scales and bias.  The grid's y extent is a bound on the tile
// count (ceil(M / BM) + min(E, M)); workgroups past the last tile return.
template <int QK, int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64) void grouped_tile_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ B,
    const int* __restrict__ offsets, int E, int64_t M, int64_t N, int64_t KB, Epi e) {
  constexpr int64_t XR = QK == QK_MXFP4 ? 4 : 1;
  int x, lo, hi, r0;
  kth_tile(offsets, E, (int)M, BM, (int)blockIdx.y, x, lo, hi, r0);
  if (x < 0) return;
  const int64_t rows = min((int64_t)BM, (int64_t)(hi - r0));
  tile_body<QK, BM, BN, WM, WN>(A + (int64_t)r0 * KB * XR, B + x * N * KB, rows, N, KB, 0,
                                (int64_t)blockIdx.x * BN, grouped_epi<QK>(e, x, r0, rows, KB));
}

// Stream-K launch geometry: P = sk x (CUs of the device) workgroups for the
// stream-K part; the first T_dp tiles go whole to their own workgroups when
// the tile count exceeds P (all but the last P..2P tiles), the rest split.
struct SkPlan {
  int tiles_m = 0, tiles_n = 0, KT = 0, t_dp = 0, P = 0, slices = 0;
};

int device_cus() {
  static int cus[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
      v = 256;
    cus[dev] = v;
  }
  return cus[dev];
}

SkPlan sk_plan(const Variant& v, const Call& c) {
  SkPlan p;
  const int rb = c.qk == QK_MXFP4 ? 32 : ROWB;
  p.tiles_m = (int)((c.M + v.bm - 1) / v.bm);
  p.tiles_n = (int)((c.N + v.bn - 1) / v.bn);
  p.KT = (int)((c.KB + rb - 1) / rb);
  const int T = p.tiles_m * p.tiles_n;
  const int P0 = std::max(1, v.sk * device_cus());
  p.t_dp = T > 2 * P0 ? (T / P0 - 1) * P0 : 0;
  const int64_t total = (int64_t)(T - p.t_dp) * p.KT;
  // No workgroup without units: then every run holds at least upw >= 1
  // units, a tile meets at most ceil(KT / upw) + 1 runs (and at most KT),
  // and that bounds the slice index a piece is written to.
  p.P = (int)std::min<int64_t>(P0, total);
  const int64_t upw = total / p.P;
  p.slices = (int)std::min<int64_t>(p.KT, (p.KT + upw - 1) / upw + 1);
  return p;
}

template <int QK, int BM, int BN, int WM, int WN>
hipError_t launch_t_sk(const Variant& v, const Call& c, hipStream_t s) {
  using S = TileShape<BM, BN, WM, WN, QK == QK_MXFP4 ? 32 : ROWB>;
  const size_t lds = 2 * (size_t)S::STAGE;
  {
    hipError_t err = opt_in_lds((const void*)tile_sk_kernel<QK, BM, BN, WM, WN>, lds);
    if (err != hipSuccess) return err;
  }
  const SkPlan p = sk_plan(v, c);
  const int group_m = v.group_m > 0 ? v.group_m : 4;
  const int T = p.tiles_m * p.tiles_n;
  const int grid = p.t_dp + p.P;
  hipLaunchKernelGGL((tile_sk_kernel<QK, BM, BN, WM, WN>), dim3(grid), dim3(S::NT), lds, s,
                     (const uint8_t*)c.A, (const uint8_t*)c.B, c.M, c.N, c.KB, p.tiles_m,
                     p.tiles_n, group_m, c.epi, p.KT, p.t_dp, p.P, c.ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL((tile_sk_fixup<QK, BM, BN>), dim3(T - p.t_dp), dim3(256), 0, s,
                     (const void*)c.ws, p.tiles_m, p.tiles_n, group_m, p.KT, p.t_dp, p.P, c.epi);
  return hipGetLastError();
}

template <int QK, int BM, int BN, int WM, int WN>
hipError_t launch_t(const Variant& v, const Call& c, int split, hipStream_t s) {
  using S = TileShape<BM, BN, WM, WN, QK == QK_MXFP4 ? 32 : ROWB>;
  const int tiles_m = (int)((c.M + BM - 1) / BM);
  const int tiles_n = (int)((c.N + BN - 1) / BN);
  const size_t lds = 2 * (size_t)S::STAGE;
  {
    hipError_t err = opt_in_lds((const void*)tile_kernel<QK, BM, BN, WM, WN>, lds);
    if (err != hipSuccess) return err;
  }
  const int group_m = v.group_m > 0 ? v.group_m : 4;
  const int KT = (int)((c.KB + (QK == QK_MXFP4 ? 32 : ROWB) - 1) / (QK == QK_MXFP4 ? 32 : ROWB));
  const int kt_per = (KT + split - 1) / split;
  hipLaunchKernelGGL((tile_kernel<QK, BM, BN, WM, WN>), dim3(tiles_m * tiles_n, split),
                     dim3(S::NT), lds, s, (const uint8_t*)c.A, (const uint8_t*)c.B, c.M, c.N,
                     c.KB, tiles_m, tiles_n, group_m, c.epi, split, kt_per, c.ws);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess || split == 1) return err;
  return launch_splitk_reduce(QK, c.ws, split, c.epi, s);
}

// The compiled tile shapes: (BM, BN, WM, WN).
#define LG_TILE_SHAPES(X) \
  X(256, 256, 2, 2)       \
  X(128, 256, 2, 2)       \
  X(256, 128, 2, 2)       \
  X(128, 128, 2, 2)       \
  X(64, 128, 1, 4)        \
  X(64, 64, 2, 2)         \
  X(256, 256, 2, 4)       \
  X(256, 128, 2, 4)       \
  X(128, 128, 2, 4)

// 4-bit weights load 32 weight rows per instruction: BN must be a multiple
// of 32 times the wave count.
constexpr bool mx_shape_ok(int bn, int wm, int wn) { return bn % (32 * wm * wn) == 0; }

// The tile shapes compiled in stream-K form.
#define LG_SK_SHAPES(X) \
  X(128, 128, 2, 2)     \
  X(64, 128, 1, 4)      \
  X(128, 128, 2, 4)     \
  X(256, 128, 2, 4)     \
  X(256, 256, 2, 4)

template <int QK>
hipError_t launch_q(const Variant& v, const Call& c, int split, hipStream_t s) {
  if (v.sk > 0) {
#define LG_SK_TRY(b_m, b_n, w_m, w_n)                                         \
    if constexpr (QK != QK_MXFP4 || mx_shape_ok(b_n, w_m, w_n)) {              \
      if (v.bm == b_m && v.bn == b_n && v.wm == w_m && v.wn == w_n)           \
        return launch_t_sk<QK, b_m, b_n, w_m, w_n>(v, c, s);                  \
    }
    LG_SK_SHAPES(LG_SK_TRY)
#undef LG_SK_TRY
    return hipErrorInvalidValue;
  }
#define LG_TRY(b_m, b_n, w_m, w_n)                                          \
  if constexpr (QK != QK_MXFP4 || mx_shape_ok(b_n, w_m, w_n)) {              \
    if (v.bm == b_m && v.bn == b_n && v.wm == w_m && v.wn == w_n)           \
      return launch_t<QK, b_m, b_n, w_m, w_n>(v, c, split, s);              \
  }
  LG_TILE_SHAPES(LG_TRY)
#undef LG_TRY
  return hipErrorInvalidValue;
}

// Grouped tile shapes: one per segment-size class.
#define LG_GROUPED_TILES(X) X(64, 128, 1, 4) X(128, 128, 2, 2) X(256, 256, 2, 4)

template <int QK, int BM, int BN, int WM, int WN>
hipError_t launch_gt(const Call& c, const int* offsets, int64_t E, hipStream_t s) {
  using S = TileShape<BM, BN, WM, WN, QK == QK_MXFP4 ? 32 : ROWB>;
  const size_t lds = 2 * (size_t)S::STAGE;
  {
    hipError_t err = opt_in_lds((const void*)grouped_tile_kernel<QK, BM, BN, WM, WN>, lds);
    if (err != hipSuccess) return err;
  }
  const int64_t tiles_n = (c.N + BN - 1) / BN;
  const int64_t slots = (c.M + BM - 1) / BM + std::min<int64_t>(E, c.M);
  if (slots > 65535 || tiles_n > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL((grouped_tile_kernel<QK, BM, BN, WM, WN>), dim3((unsigned)tiles_n, (unsigned)slots),
                     dim3(S::NT), lds, s, (const uint8_t*)c.A, (const uint8_t*)c.B, offsets, (int)E,
                     c.M, c.N, c.KB, c.epi);
  return hipGetLastError();
}

template <int QK>
hipError_t launch_gq(const Variant& v, const Call& c, const int* offsets, int64_t E,
                     hipStream_t s) {
#define LG_GTRY(b_m, b_n, w_m, w_n)                                         \
  if (v.bm == b_m && v.bn == b_n && v.wm == w_m && v.wn == w_n)             \
    return launch_gt<QK, b_m, b_n, w_m, w_n>(c, offsets, E, s);
  LG_GROUPED_TILES(LG_GTRY)
#undef LG_GTRY
  return hipErrorInvalidValue;
}

}  // namespace

bool grouped_tile_supported(int bm, int bn, int wm, int wn) {
#define LG_GHAS(b_m, b_n, w_m, w_n) if (bm == b_m && bn == b_n && wm == w_m && wn == w_n) return true;
  LG_GROUPED_TILES(LG_GHAS)
#undef LG_GHAS
  return false;
}

hipError_t launch_grouped_tile(const Variant& v, const Call& c, const int* offsets, int64_t E,
                               hipStream_t s) {
  switch (c.qk) {
    case QK_BF16: return launch_gq<QK_BF16>(v, c, offsets, E, s);
    case QK_FP16: return launch_gq<QK_FP16>(v, c, offsets, E, s);
    case QK_FP8: return launch_gq<QK_FP8>(v, c, offsets, E, s);
    case QK_I8: return launch_gq<QK_I8>(v, c, offsets, E, s);
    case QK_FP8_BLOCK: return launch_gq<QK_FP8_BLOCK>(v, c, offsets, E, s);
    case QK_MXFP4: return launch_gq<QK_MXFP4>(v, c, offsets, E, s);
  }
  return hipErrorInvalidValue;
}

bool tile_supported(int qk, int bm, int bn, int wm, int wn) {
#define LG_HAS(b_m, b_n, w_m, w_n) \
  if (bm == b_m && bn == b_n && wm == w_m && wn == w_n) return qk != QK_MXFP4 || mx_shape_ok(bn, wm, wn);
  LG_TILE_SHAPES(LG_HAS)
#undef LG_HAS
  return false;
}

bool tile_sk_supported(int qk, int bm, int bn, int wm, int wn) {
#define LG_HAS(b_m, b_n, w_m, w_n) \
  if (bm == b_m && bn == b_n && wm == w_m && wn == w_n) return qk != QK_MXFP4 || mx_shape_ok(bn, wm, wn);
  LG_SK_SHAPES(LG_HAS)
#undef LG_HAS
  return false;
}

// Split K while the grid has fewer than 512 workgroups, every slice keeps at
// least 8 K stages, and the partials' round trip (split x M x N x 8 bytes)
// stays within the weight's bytes (N x KB).  Measured on MI355X (fp8, bf16,
// block e4m3, MXFP4; N 4096-6144, K 4096-12288): M = 64-128 runs 1.5-3x
// faster split 2-8 ways; at M = 512 with 8-bit weights splitting loses.
int tile_auto_split(const Variant& v, const Call& c) {
  const int64_t tiles = ((c.M + v.bm - 1) / v.bm) * ((c.N + v.bn - 1) / v.bn);
  const int rb = c.qk == QK_MXFP4 ? 32 : ROWB;
  const int64_t KT = (c.KB + rb - 1) / rb;
  int split = 1;
  while (split < 8 && tiles * split < 512 && KT >= 8 * (int64_t)split * 2 &&
         (int64_t)split * 2 * c.M * 8 <= c.KB)
    split *= 2;
  return split;
}

size_t tile_ws_bytes(const Variant& v, const Call& c, int split) {
  if (v.sk > 0) return (size_t)sk_plan(v, c).slices * (size_t)c.M * (size_t)c.N * 4;
  return split <= 1 ? 0 : (size_t)split * (size_t)c.M * (size_t)c.N * 4;
}

hipError_t launch_tile(const Variant& v, const Call& c, int split, hipStream_t s) {
  if (split < 1 || split > 16 || ((split > 1 || v.sk > 0) && !c.ws)) return hipErrorInvalidValue;
  if (v.sk > 0 && (v.sk > 8 || (int64_t)((c.M + v.bm - 1) / v.bm) * ((c.N + v.bn - 1) / v.bn) > 0x7FFFFFFF / 2))
    return hipErrorInvalidValue;
  switch (c.qk) {
    case QK_BF16: return launch_q<QK_BF16>(v, c, split, s);
    case QK_FP16: return launch_q<QK_FP16>(v, c, split, s);
    case QK_FP8: return launch_q<QK_FP8>(v, c, split, s);
    case QK_I8: return launch_q<QK_I8>(v, c, split, s);
    case QK_FP8_BLOCK: return launch_q<QK_FP8_BLOCK>(v, c, split, s);
    case QK_MXFP4: return launch_q<QK_MXFP4>(v, c, split, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace lg
