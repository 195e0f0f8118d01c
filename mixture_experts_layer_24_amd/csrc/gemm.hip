// gemm.hip -- grouped expert GEMMs (and the PR-MoE dense MLP) on gfx950.
//
// Method: survey notes sec. 1.1.2.1 (each expert is a two-layer FFN that
// replaces the transformer FFN); "DeepSpeed-MoE ... notes" sec. 4.4 and its
// closing outline ("sparse GEMM -> dense GEMM": after the layout transform
// each expert runs a dense GEMM on its packed rows); survey notes sec.
// 1.2.3.1 (weight-only quantisation: low-precision weights are dequantised
// for the arithmetic) with the symmetric form of sec. 1.2.2 (w = s * q).
//
// C[g][m][n] = epi( sum_k A[g][m][k] * B[g][n][k] ),  m < rows[g]
// A: activations [G][M_cap][K] (x_disp, H or x), K contiguous.
// B: weights [G][N][K] ([out, in], K contiguous), bf16 or int8 + fp16 scale
//    per 128 K-elements of a row.  epi = GELU (first layer) or identity.
//
// Register-staged kernel (int8 weights, and shapes the DMA kernel does not
// tile): a BM x BN block tile, 64-wide K steps double-buffered through LDS
// (rows padded to 144 B so the 16-byte MFMA operand reads are free of bank
// conflicts), register prefetch of the next K step while the MFMAs run.  Each wave owns a WTM x WTN sub-tile of 32x32x16 (or
// 16x16x32) bf16 MFMAs accumulating in fp32.  int8 weights are converted to
// bf16 (s * q rounded once) on their way into LDS, so the MFMA loop is the
// same as for bf16 weights.  Rows past rows[g] are neither read (their loads
// are clamped to the last valid row) nor written; blocks whose first row is
// past rows[g] exit at once, so only kept rows cost MFMA time, and only
// experts with at least one kept row stream their weights.
// Blocks are mapped to tiles XCD by XCD: with a multiple of 8 groups, XCD x
// takes experts x, x+8, ... and runs each expert's tiles back to back so
// they share its L2 for their A rows; otherwise each XCD takes a contiguous
// range of tiles.  The int8 kernel can instead follow a per-call schedule
// that deals the experts to the XCDs by their row counts
// (tile_sched_kernel), which evens out skewed loads.  The DMA kernels below
// read bf16 weights either row-major or packed in blocks of 128 rows x 64 K
// (MOE_W_BF16_PACKED), where a K step of a block is 16 KB of contiguous
// memory.
#include "common.h"
#include "dma.h"
#include "kernels.h"

#include <type_traits>

namespace moe {

template <int BM, int BN, int WM, int WN, int MF, bool BINT8, int GELU>
__global__ __launch_bounds__(64 * WM * WN) void gemm_bf16_kernel(GemmArgs a) {
  constexpr int NT = 64 * WM * WN;
  constexpr int BK = 64;
  constexpr int LDK = BK + 8;  // 144-byte LDS rows
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / MF, TN = WTN / MF;
  constexpr int KSTEP = (MF == 32) ? 16 : 32;
  constexpr int ACC = (MF == 32) ? 16 : 4;
  constexpr int A_CH = BM * 8;                    // 16-byte chunks per A stage
  constexpr int A_PT = (A_CH + NT - 1) / NT;
  constexpr int B_CPR = BINT8 ? 4 : 8;            // 16-byte chunks per B row
  constexpr int B_CH = BN * B_CPR;
  constexpr int B_PT = (B_CH + NT - 1) / NT;
  constexpr int STAGE = (BM + BN) * LDK;          // bf16 elements per LDS stage
  static_assert(TM >= 1 && TN >= 1 && WTM % MF == 0 && WTN % MF == 0, "bad tile");
  typedef typename std::conditional<MF == 32, f32x16, f32x4>::type acc_t;

  __shared__ __attribute__((aligned(16))) bf16 smem[2 * STAGE];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int tiles_n = a.N / BN;
  const int tiles_m = (int)((a.M_cap + BM - 1) / BM);
  const int total = a.G * tiles_m * tiles_n;
  const int tile = (a.G % 8 == 0) ? xcd_remap_grouped(blockIdx.x, a.G, tiles_m * tiles_n)
                                  : xcd_remap(blockIdx.x, total);
  const int g = tile / (tiles_m * tiles_n);
  const int rem = tile - g * tiles_m * tiles_n;
  int tm, tn;
  grouped_tile(rem, tiles_m, tiles_n, tm, tn);
  int64_t rows = a.M_cap;
  if (a.rows) {
    const int64_t r = a.rows[g];
    rows = r < rows ? r : rows;
  }
  const int64_t m0 = (int64_t)tm * BM;
  if (m0 >= rows) return;
  const int n0 = tn * BN;
  const int K = a.K, N = a.N;

  const bf16 *Ag = (const bf16 *)a.A + (int64_t)g * a.M_cap * K;
  const bf16 *Bg = (const bf16 *)a.B + (int64_t)g * N * K;
  const int8_t *Bq = (const int8_t *)a.B + (int64_t)g * N * K;
  const _Float16 *Sg = (const _Float16 *)a.Bscale + (int64_t)g * N * (K / 128);
  bf16 *Cg = (bf16 *)a.C + (int64_t)g * a.M_cap * N;
  bf16 *Zg = GELU == 2 ? (bf16 *)a.Zpre + (int64_t)g * a.M_cap * N : nullptr;

  u32x4 ra[A_PT], rb[B_PT];
  float rs[BINT8 ? B_PT : 1];
  auto load_tiles = [&](u32x4 (&ra)[A_PT], u32x4 (&rb)[B_PT], float (&rs)[BINT8 ? B_PT : 1],
                        int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < A_PT; p++) {
      const int c = tid + p * NT;
      if (A_CH % NT == 0 || c < A_CH) {
        int64_t m = m0 + (c >> 3);
        if (m >= rows) m = rows - 1;
        ra[p] = *(const u32x4 *)(Ag + m * K + k0 + (c & 7) * 8);
      }
    }
#pragma unroll
    for (int p = 0; p < B_PT; p++) {
      const int c = tid + p * NT;
      if (B_CH % NT == 0 || c < B_CH) {
        const int64_t n = n0 + c / B_CPR;
        if constexpr (BINT8) {
          const int kk = k0 + (c % B_CPR) * 16;
          rb[p] = *(const u32x4 *)(Bq + n * K + kk);
          rs[p] = (float)Sg[n * (K / 128) + kk / 128];
        } else {
          rb[p] = *(const u32x4 *)(Bg + n * K + k0 + (c % B_CPR) * 8);
        }
      }
    }
  };
  auto store_tiles = [&](const u32x4 (&ra)[A_PT], const u32x4 (&rb)[B_PT],
                         const float (&rs)[BINT8 ? B_PT : 1], int st) __attribute__((always_inline)) {
    bf16 *sa = smem + st * STAGE;
    bf16 *sb = sa + BM * LDK;
#pragma unroll
    for (int p = 0; p < A_PT; p++) {
      const int c = tid + p * NT;
      if (A_CH % NT == 0 || c < A_CH) *(u32x4 *)(sa + (c >> 3) * LDK + (c & 7) * 8) = ra[p];
    }
#pragma unroll
    for (int p = 0; p < B_PT; p++) {
      const int c = tid + p * NT;
      if (B_CH % NT == 0 || c < B_CH) {
        if constexpr (BINT8) {
          // 16 int8 codes -> 16 bf16 values s*q (one rounding)
          const int8_t *q = (const int8_t *)&rb[p];
          bf16x8 lo, hi;
#pragma unroll
          for (int i = 0; i < 8; i++) {
            lo[i] = (bf16)(rs[p] * (float)q[i]);
            hi[i] = (bf16)(rs[p] * (float)q[8 + i]);
          }
          bf16 *dst = sb + (c / B_CPR) * LDK + (c % B_CPR) * 16;
          *(bf16x8 *)dst = lo;
          *(bf16x8 *)(dst + 8) = hi;
        } else {
          *(u32x4 *)(sb + (c / B_CPR) * LDK + (c % B_CPR) * 8) = rb[p];
        }
      }
    }
  };

  acc_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < ACC; r++) acc[i][j][r] = 0.f;

  const int wm = wave / WN, wn = wave % WN;
  const int ksteps = K / BK;
  // MFMAs on one LDS stage
  auto compute = [&](int st) __attribute__((always_inline)) {
    const bf16 *sa = smem + st * STAGE + (wm * WTM) * LDK;
    const bf16 *sb = smem + st * STAGE + BM * LDK + (wn * WTN) * LDK;
#pragma unroll
    for (int s = 0; s < BK / KSTEP; s++) {
      int row, ch;
      if constexpr (MF == 32) {
        row = lane & 31;
        ch = 2 * s + (lane >> 5);
      } else {
        row = lane & 15;
        ch = 4 * s + (lane >> 4);
      }
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; i++) af[i] = *(const bf16x8 *)(sa + (i * MF + row) * LDK + ch * 8);
#pragma unroll
      for (int j = 0; j < TN; j++) bfr[j] = *(const bf16x8 *)(sb + (j * MF + row) * LDK + ch * 8);
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++) {
          if constexpr (MF == 32)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
          else
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
    }
  };
  // one K step in flight: load kt+1 while computing kt
  load_tiles(ra, rb, rs, 0);
  store_tiles(ra, rb, rs, 0);
  __syncthreads();
  for (int kt = 0; kt < ksteps; kt++) {
    const int st = kt & 1;
    if (kt + 1 < ksteps) load_tiles(ra, rb, rs, (kt + 1) * BK);
    compute(st);
    if (kt + 1 < ksteps) store_tiles(ra, rb, rs, st ^ 1);
    __syncthreads();
  }

  // epilogue: D[m][n] of a 32x32 MFMA sits in lane n (+32 for rows 4..7 of
  // each group of 8) -- row 8*(r/4) + 4*(lane/32) + r%4, column lane%32; of a
  // 16x16 MFMA: row 4*(lane/16) + r, column lane%16.
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < ACC; r++) {
        int mr, nc;
        if constexpr (MF == 32) {
          mr = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
          nc = lane & 31;
        } else {
          mr = 4 * (lane >> 4) + r;
          nc = lane & 15;
        }
        const int64_t m = m0 + wm * WTM + i * MF + mr;
        const int n = n0 + wn * WTN + j * MF + nc;
        float v = acc[i][j][r];
        if (GELU == 2 && m < rows) Zg[m * N + n] = (bf16)v;
        if (GELU) v = gelu_f(v);
        if (m < rows) Cg[m * N + n] = (bf16)v;
      }
}

// ---------------------------------------------------------------------------
// GELU epilogue that also keeps the pre-activation (Zpre): per row band (the
// waves with wm == band) and sub-band of RB rows, the fp32 sums go through
// LDS once, and every thread turns 8 consecutive sums into both outputs (the
// sum and its GELU, each rounded once to bf16) with coalesced 16-byte
// stores.  One pass over the accumulators, so nothing beyond them is live
// while they are written.  LDSB: bytes of LDS the sub-band may use.
template <int TM, int TN, int WM, int WTM, int WTN, int BN, int LDSB, int NT>
__device__ __forceinline__ void store_keep_pre(const f32x16 (&acc)[TM][TN], char *smem, int wm,
                                               int wn, int lane, int tid, int64_t m0, int n0,
                                               int64_t rows, int N, bf16 *Zg, bf16 *Cg) {
  constexpr int ROWF = BN * 4 + 16;  // bytes per LDS row (fp32, padded)
  constexpr int RB = WTM * ROWF <= LDSB ? WTM : (WTM / 2 * ROWF <= LDSB ? WTM / 2 : WTM / 4);
  static_assert(RB >= 32 && RB % 32 == 0 && RB * ROWF <= LDSB && WTM % RB == 0, "sub-band");
  constexpr int FPB = RB / 32;  // row fragments per sub-band
  constexpr int OCPR = BN / 8;  // 8-wide chunks per row
  for (int band = 0; band < WM; band++) {
#pragma unroll
    for (int h = 0; h < WTM / RB; h++) {
      __syncthreads();  // stage buffers (or the previous sub-band) no longer read
      if (wm == band) {
#pragma unroll
        for (int i = 0; i < TM; i++) {
          if (i / FPB != h) continue;
#pragma unroll
          for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
              const int R = (i - h * FPB) * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              const int Cc = wn * WTN + j * 32 + (lane & 31);
              *(float *)(smem + R * ROWF + Cc * 4) = acc[i][j][r];
            }
        }
      }
      __syncthreads();
      const int64_t r0 = m0 + band * WTM + h * RB;
      const int64_t mrows = rows - r0 < RB ? rows - r0 : RB;
      for (int idx = tid; idx < RB * OCPR; idx += NT) {
        const int R = idx / OCPR, ch = idx - R * OCPR;
        if (R < mrows) {
          const f32x4 *src = (const f32x4 *)(smem + R * ROWF + ch * 32);
          const f32x4 lo = src[0], hi = src[1];
          bf16x8 z, c;
#pragma unroll
          for (int q = 0; q < 4; q++) {
            z[q] = (bf16)lo[q];
            z[4 + q] = (bf16)hi[q];
            c[q] = (bf16)gelu_f(lo[q]);
            c[4 + q] = (bf16)gelu_f(hi[q]);
          }
          // non-temporal: the second layer reads H once, the backward reads
          // both much later (train step 9.36 -> 9.21-9.26 ms at the 1.3B shape)
          __builtin_nontemporal_store(z, (bf16x8 *)(Zg + (r0 + R) * N + n0 + ch * 8));
          __builtin_nontemporal_store(c, (bf16x8 *)(Cg + (r0 + R) * N + n0 + ch * 8));
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// DMA-pipelined bf16 GEMM.  Both operands travel global -> LDS with gfx950's
// global_load_lds_dwordx4 (each lane's 16 bytes land at M0 + 16 * lane), so no
// registers stage the tiles and NS - 1 K steps can be in flight per block.
// LDS tiles hold BK-wide K steps as rows of BK/8 16-byte chunks (BK = 64:
// 128-byte rows, or 32: 64-byte rows, which halves a stage so large tiles
// can keep more steps in flight).  Chunk c of row R sits in slot c ^ f(R):
//   BK = 64: f(R) = (R & 7) ^ ((R >> 3) & 1)
//   BK = 32: f(R) = (R >> 2) & 3
// which keeps the 16-byte MFMA operand reads (32 consecutive rows, one
// logical chunk) free of bank conflicts on gfx950's LDS (checked with the
// SQ_LDS_BANK_CONFLICT counter).  The DMA lane -> (row, slot) placement is
// fixed (16 bytes per lane, consecutive), so each lane fetches the global
// chunk that belongs in its slot.
// The DMA loads are issued from inline assembly (they have no register
// results); their completion is awaited with explicit vmcnt waits before the
// barrier that publishes a stage, because the compiler would otherwise wait
// for every outstanding load before each LDS read.
// NTB: load the weight operand non-temporally (read once)
// PB: B in blocks of 128 rows x 64 K (MOE_W_BF16_PACKED): a tile's K step
// reads 16 KB of contiguous memory per 128 weight rows instead of 128 bytes
// from each row, which the DRAM streams at a higher rate.
template <int BM, int BN, int WM, int WN, int BK, int NS, bool NTB, int GELU, bool PB = false>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_kernel(GemmArgs a) {
  static_assert(BK == 64 || BK == 32, "K step");
  static_assert(!PB || (BK == 64 && BN % 128 == 0), "packed weights: 64-wide K steps, 128-row blocks");
  constexpr int W = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int ROWB = BK * 2;                    // bytes per tile row
  constexpr int CPR = ROWB / 16;                  // 16-byte chunks per row
  constexpr int RPC = 1024 / ROWB;                // rows per 1 KB DMA chunk
  constexpr int STAGE = (BM + BN) * ROWB;         // bytes per stage
  constexpr int A_PW = BM / RPC / W;             // activation chunks per wave per stage
  constexpr int B_PW = BN / RPC / W;             // weight chunks per wave per stage
  constexpr int CPW = A_PW + B_PW;
  static_assert(A_PW * W * RPC == BM && B_PW * W * RPC == BN && TM >= 1 && TN >= 1, "tile");
  static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS budget");
  static_assert((NS - 2) * CPW < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform (SGPR)
  const int tiles_n = a.N / BN;
  const int tiles_m = (int)((a.M_cap + BM - 1) / BM);
  const int total = a.G * tiles_m * tiles_n;
  // spread: each group's tiles go round-robin over the XCDs (groups with few
  // rows share little in L2, and a group per XCD would leave the XCDs of the
  // groups without rows idle); else a group's tiles stay on one XCD
  const int tile = a.spread ? (int)blockIdx.x
                   : (a.G % 8 == 0) ? xcd_remap_grouped(blockIdx.x, a.G, tiles_m * tiles_n)
                                    : xcd_remap(blockIdx.x, total);
  const int g = tile / (tiles_m * tiles_n);
  const int rem = tile - g * tiles_m * tiles_n;
  // row groups: 8 for the expert GEMMs (their weight slabs are streamed
  // once, shared by an expert's row tiles); 2 for the dense MLP, whose 32
  // concurrent tiles per XCD then cover 2 row x 16 column tiles and read
  // each activation panel fewer times -- beside the expert weight stream,
  // which evicts the dense operands from the caches, the overlapped 1.3B
  // layer runs 2.527 -> 2.484 ms (row groups of 1, 4 and 16: 2.51, 2.51,
  // 2.53 ms; the serial layer is unchanged)
  int tm, tn;
  if constexpr (NTB)
    grouped_tile<8>(rem, tiles_m, tiles_n, tm, tn);
  else
    grouped_tile<2>(rem, tiles_m, tiles_n, tm, tn);
  int64_t rows = a.M_cap;
  if (a.rows) {
    const int64_t r = a.rows[g];
    rows = r < rows ? r : rows;
  }
  const int64_t m0 = (int64_t)tm * BM;
  if (m0 >= rows) return;
  const int n0 = tn * BN;
  const int K = a.K, N = a.N;
  // per-tile operand bases: every per-lane offset below is < 2^32 bytes
  // (with a row table, A's base is its first row)
  const char *Abase =
      (const char *)a.A + (a.asrc ? 0 : ((int64_t)g * a.M_cap + m0) * K * 2);
  const char *Bbase = (const char *)a.B + ((int64_t)g * N + n0) * (int64_t)K * 2;
  bf16 *Cg = (bf16 *)a.C + (int64_t)g * a.M_cap * N;
  bf16 *Zg = GELU == 2 ? (bf16 *)a.Zpre + (int64_t)g * a.M_cap * N : nullptr;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;

  // Every wave moves A_PW chunks of the activation tile and B_PW chunks of
  // the weight tile per stage (chunk = 1 KB = RPC tile rows), so the issue
  // sequence is the same straight-line code in every wave.
  // this lane's source offset for each of its chunks (K step 0)
  uint32_t voffa[A_PW], voffb[B_PW];
  const int lr = lane / CPR, slot = lane % CPR;
#pragma unroll
  for (int i = 0; i < A_PW; i++) {
    const int R = RPC * (wave * A_PW + i) + lr;
    int64_t m = R;
    if (m0 + m >= rows) m = rows - 1 - m0;  // clamp to the last valid row
    if (a.asrc) m = a.asrc[(int64_t)g * a.M_cap + m0 + m];
    voffa[i] = (uint32_t)(m * K * 2 + ((slot ^ swz_slot<BK>(R)) << 4));
  }
#pragma unroll
  for (int i = 0; i < B_PW; i++) {
    const int R = RPC * (wave * B_PW + i) + lr;
    if constexpr (PB)  // block R / 128 of the tile, row R % 128 of it (n0 is a block start)
      voffb[i] = (uint32_t)((int64_t)(R / 128) * 128 * K * 2 + (R % 128) * ROWB +
                            ((slot ^ swz_slot<BK>(R)) << 4));
    else
      voffb[i] = (uint32_t)((int64_t)R * K * 2 + ((slot ^ swz_slot<BK>(R)) << 4));
  }
  const uint32_t dsta = lds0 + wave * A_PW * 1024;
  const uint32_t dstb = lds0 + BM * ROWB + wave * B_PW * 1024;
  auto issue = [&](int st, int kt) __attribute__((always_inline)) {
    const char *ga = Abase + (int64_t)kt * ROWB;
    const char *gb = Bbase + (int64_t)kt * (PB ? 128 * ROWB : ROWB);
#pragma unroll
    for (int i = 0; i < A_PW; i++)
      dma16<false>(ga, voffa[i], __builtin_amdgcn_readfirstlane(dsta + st * STAGE + i * 1024));
#pragma unroll
    for (int i = 0; i < B_PW; i++)
      dma16<NTB>(gb, voffb[i], __builtin_amdgcn_readfirstlane(dstb + st * STAGE + i * 1024));
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  const int wm = wave / WN, wn = wave % WN;
  const int ksteps = K / BK;
#pragma unroll
  for (int p = 0; p < NS - 1; p++)
    if (p < ksteps) issue(p, p);
  for (int kt = 0; kt < ksteps; kt++) {
    // this wave's chunks of step kt have landed once at most the later
    // steps' chunks are outstanding; the barrier publishes every wave's
    if (kt + NS - 2 < ksteps)
      wait_vmcnt<(NS - 2) * CPW>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    if (kt + NS - 1 < ksteps) issue((kt + NS - 1) % NS, kt + NS - 1);
    const char *sa = smem + (kt % NS) * STAGE;
    const char *sb = sa + BM * ROWB;
#pragma unroll
    for (int s = 0; s < BK / 16; s++) {
      const int c = 2 * s + (lane >> 5);
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; i++) {
        const int R = wm * WTM + i * 32 + (lane & 31);
        af[i] = *(const bf16x8 *)(sa + R * ROWB + ((c ^ swz_slot<BK>(R)) << 4));
      }
#pragma unroll
      for (int j = 0; j < TN; j++) {
        const int R = wn * WTN + j * 32 + (lane & 31);
        bfr[j] = *(const bf16x8 *)(sb + R * ROWB + ((c ^ swz_slot<BK>(R)) << 4));
      }
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue: the tile goes through LDS (bf16, rows padded by 16 bytes) so
  // the output is written with coalesced 16-byte stores, one row band of
  // WTM rows (the waves with the same wm) at a time.  The hidden rows of the
  // first layer (GELU) are stored non-temporally: the second layer reads
  // each once, and as ordinary stores their dirty lines (256 MB at the 1.3B
  // shape) were written back from the caches in the middle of the next
  // weight stream -- 350M-shape layer 0.447 -> 0.418 ms, serial 1.3B layer
  // 2.82 -> 2.72 ms (expert GEMMs 0.866 / 0.755 -> 0.81 / 0.69 ms).
  // 32x32 MFMA layout: register r of lane l holds row
  // 8*(r/4) + 4*(l/32) + r%4, column l%32.
  constexpr int CROW = BN * 2 + 16;  // bytes per LDS row of the C band
  static_assert(WTM * CROW <= NS * STAGE, "C band fits the stage buffers");
  constexpr int OCPR = BN / 8;       // 16-byte chunks per output row
  // (the GELU, if any, applied per element as it is written to LDS); with the
  // pre-activation output (GELU == 2) the fp32 sums go through LDS instead
  if constexpr (GELU == 2) {
    store_keep_pre<TM, TN, WM, WTM, WTN, BN, NS * STAGE, 64 * W>(acc, smem, wm, wn, lane, tid, m0,
                                                                  n0, rows, N, Zg, Cg);
  } else {
    for (int band = 0; band < WM; band++) {
      __syncthreads();  // stage buffers (or the previous band) no longer read
      if (wm == band) {
#pragma unroll
        for (int i = 0; i < TM; i++)
#pragma unroll
          for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
              const int R = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              const int Cc = wn * WTN + j * 32 + (lane & 31);
              float v = acc[i][j][r];
              if (GELU) v = gelu_f(v);
              *(bf16 *)(smem + R * CROW + Cc * 2) = (bf16)v;
            }
      }
      __syncthreads();
      const int64_t r0 = m0 + band * WTM;
      const int64_t mrows = rows - r0 < WTM ? rows - r0 : WTM;
      for (int idx = tid; idx < WTM * OCPR; idx += 64 * W) {
        const int R = idx / OCPR, ch = idx - R * OCPR;
        if (R < mrows) {
          const u32x4 cv = *(const u32x4 *)(smem + R * CROW + ch * 16);
          u32x4 *dst = (u32x4 *)(Cg + (r0 + R) * N + n0 + ch * 8);
          if constexpr (GELU == 1)
            __builtin_nontemporal_store(cv, dst);  // hidden rows (see above)
          else
            *dst = cv;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// DMA-pipelined GEMM with int8 weights (symmetric codes q, one fp16 scale s
// per 128 consecutive K elements of a weight row; weight = s * q).
// The activations (bf16, 128-byte tile rows) and the int8 codes (64-byte
// tile rows: one 64-wide K step) both travel global -> LDS by DMA into NS
// stage buffers, as in gemm_dma_kernel; the scales of the tile's BN weight
// rows arrive by DMA in blocks of 8 groups (1024 K elements, 16 bytes per
// row), double-buffered.  Each wave turns its own B fragments into bf16 in
// registers, one sub-step ahead of the MFMAs that use them (the schedule of
// a K step is described at the loop): bf16(s * q) with s * q rounded once
// to fp32 (computed as fma(q + 128, s, -128 s), which is exact up to that
// one rounding), so the arithmetic is that of a bf16 GEMM on the
// dequantised weights and half the weight bytes cross LDS.
// Code tile rows: chunk c (16 codes) of row R sits in slot c ^ ((R >> 2) & 3),
// which spreads 16 consecutive rows over all 64 banks.  (One 16-byte read per
// lane with permlane32 swaps of the halves, which avoids the two-way bank
// conflict of the 8-byte reads, measured 1-3% slower.)  Requires
// K % 1024 == 0 and N % BN == 0.
// Waves whose row band lies past the group's valid rows skip their LDS reads,
// dequantisation and MFMAs (they still move their share of the DMA).
__device__ __forceinline__ int swz_q(int R) { return (R >> 2) & 3; }

// queue entry flag of the int8 schedule: the group runs light tiles
constexpr int kLightGroup = 0x10000;

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two codes (bytes b and b + 1 of w, already offset by 128) -> a packed bf16 pair
__device__ __forceinline__ uint32_t dequant2(uint32_t w, int b, float sc, float nsc) {
  const f32x2 v = {fmaf((float)((w >> (8 * b)) & 0xffu), sc, nsc),
                   fmaf((float)((w >> (8 * b + 8)) & 0xffu), sc, nsc)};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ bf16x8 dequant8(uint32_t lo, uint32_t hi, float sc, float nsc) {
  lo ^= 0x80808080u;  // q + 128 in each byte
  hi ^= 0x80808080u;
  const u32x4 r = {dequant2(lo, 0, sc, nsc), dequant2(lo, 2, sc, nsc), dequant2(hi, 0, sc, nsc),
                   dequant2(hi, 2, sc, nsc)};
  return __builtin_bit_cast(bf16x8, r);
}

// LDS bytes of an int8 tile: NS stages of activations and codes, and two
// scale blocks
template <int BM, int BN, int NS>
constexpr int i8_lds_bytes() {
  return NS * (BM * 128 + BN * 64) + 2 * BN * 16;
}

template <int BM, int BN, int WM, int WN, int NS, int GELU>
__device__ __forceinline__ void i8_tile(const GemmArgs &a, int g, int tm, int tn, char *smem) {
  constexpr int BK = 64;
  constexpr int W = WM * WN;
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  constexpr int AROWB = BK * 2;                 // bytes per activation tile row
  constexpr int BROWB = BK;                     // bytes per code tile row
  constexpr int A_CH = BM * AROWB / 1024;       // 1 KB DMA chunks per stage
  constexpr int B_CH = BN * BROWB / 1024;
  constexpr int A_PW = A_CH / W, B_PW = B_CH / W;  // chunks per wave per stage
  constexpr int CPW = A_PW + B_PW;
  constexpr int ASTAGE = BM * AROWB;
  constexpr int STAGE = ASTAGE + BN * BROWB;
  constexpr int SCB = BN * 16;                  // one scale block (8 groups)
  constexpr int SC_CH = SCB / 1024;
  constexpr int SC_PW = (SC_CH + W - 1) / W;  // scale chunks per wave
  static_assert(A_PW * W == A_CH && B_PW * W == B_CH && TM >= 1 && TN >= 1 &&
                    (SC_CH <= W || SC_PW * W == SC_CH), "tile");
  static_assert(NS >= 2 && NS * STAGE + 2 * SCB <= 160 * 1024, "LDS budget");
  static_assert((NS - 2) * CPW < 64, "vmcnt range");
  static_assert(i8_lds_bytes<BM, BN, NS>() == NS * STAGE + 2 * SCB, "LDS size");

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  int64_t rows = a.M_cap;
  if (a.rows) {
    const int64_t r = a.rows[g];
    rows = r < rows ? r : rows;
  }
  const int64_t m0 = (int64_t)tm * BM;
  if (m0 >= rows) return;
  const int n0 = tn * BN;
  const int K = a.K, N = a.N, KG = K / 128;
  const char *Abase =
      (const char *)a.A + (a.asrc ? 0 : ((int64_t)g * a.M_cap + m0) * K * 2);
  const char *Bbase = (const char *)a.B + ((int64_t)g * N + n0) * (int64_t)K;
  const char *Sbase = (const char *)a.Bscale + ((int64_t)g * N + n0) * (int64_t)KG * 2;
  bf16 *Cg = (bf16 *)a.C + (int64_t)g * a.M_cap * N;
  bf16 *Zg = GELU == 2 ? (bf16 *)a.Zpre + (int64_t)g * a.M_cap * N : nullptr;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
  const uint32_t lds_sc = lds0 + NS * STAGE;

  // every wave moves A_PW activation chunks and B_PW code chunks per stage
  uint32_t voffa[A_PW], voffb[B_PW];
#pragma unroll
  for (int i = 0; i < A_PW; i++) {
    const int R = 8 * (wave * A_PW + i) + lane / 8, slot = lane % 8;
    int64_t m = R;
    if (m0 + m >= rows) m = rows - 1 - m0;  // clamp to the last valid row
    if (a.asrc) m = a.asrc[(int64_t)g * a.M_cap + m0 + m];
    voffa[i] = (uint32_t)(m * K * 2 + ((slot ^ swz_slot<64>(R)) << 4));
  }
#pragma unroll
  for (int i = 0; i < B_PW; i++) {
    const int R = 16 * (wave * B_PW + i) + lane / 4, slot = lane % 4;
    voffb[i] = (uint32_t)((int64_t)R * K + ((slot ^ swz_q(R)) << 4));
  }
  uint32_t soff[SC_PW];  // scale chunks wave + W * i (64 weight rows each)
#pragma unroll
  for (int i = 0; i < SC_PW; i++) soff[i] = (uint32_t)((64 * (wave + W * i) + lane) * KG * 2);
  const uint32_t dsta = lds0 + wave * A_PW * 1024;
  const uint32_t dstb = lds0 + ASTAGE + wave * B_PW * 1024;
  auto issue = [&](int st, int kt) __attribute__((always_inline)) {
    const char *ga = Abase + (int64_t)kt * AROWB;
    const char *gb = Bbase + (int64_t)kt * BROWB;
#pragma unroll
    for (int i = 0; i < A_PW; i++)
      dma16<false>(ga, voffa[i], __builtin_amdgcn_readfirstlane(dsta + st * STAGE + i * 1024));
#pragma unroll
    for (int i = 0; i < B_PW; i++)
      dma16<false>(gb, voffb[i], __builtin_amdgcn_readfirstlane(dstb + st * STAGE + i * 1024));
  };
  auto issue_scales = [&](int blk) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < SC_PW; i++)
      if (wave + W * i < SC_CH)
        dma16<false>(Sbase + blk * 16, soff[i],
                     __builtin_amdgcn_readfirstlane(lds_sc + (blk & 1) * SCB + (wave + W * i) * 1024));
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  const int wm = wave / WN, wn = wave % WN;
  const int ksteps = K / BK;  // at least 16 (K % 1024 == 0)
  // waves of a row band past the group's valid rows skip LDS reads and MFMAs
  const bool act = WM == 1 || live_frags<TM>(rows - m0 - wm * WTM) > 0;

  // Schedule of one K step (four 16-wide sub-steps s = 0..3): the MFMAs of
  // sub-step s run from registers while the operands of s + 1 are read from
  // LDS and its codes dequantised (one packed pair per MFMA, interleaved), so
  // the wave's VALU and LDS work overlaps its MFMAs.  The workgroup barrier
  // sits between sub-steps 2 and 3: by then every wave has read all of this
  // stage, so the DMA of stage kt + NS can go into its buffer, and sub-step 3
  // already reads the next stage -- no exposed prologue per K step.
  constexpr int SS = BK / 16;
  static_assert(SS == 4, "four sub-steps per K step");
  bf16x8 af[2][TM], bfr[2][TN];
  uint32_t qv[2][TN][2];  // codes of sub-step c in qv[c & 1], read two sub-steps ahead
  float sc[TN], nsc[TN];
  auto rd_a = [&](const char *sa, int st, bf16x8 *dst) __attribute__((always_inline)) {
    const int c = 2 * st + (lane >> 5);
#pragma unroll
    for (int i = 0; i < TM; i++) {
      const int R = wm * WTM + i * 32 + (lane & 31);
      dst[i] = *(const bf16x8 *)(sa + R * AROWB + ((c ^ swz_slot<64>(R)) << 4));
    }
  };
  auto rd_q = [&](const char *sb, int st, uint32_t (*q)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const int R = wn * WTN + j * 32 + (lane & 31);
      const uint32_t *qp =
          (const uint32_t *)(sb + R * BROWB + ((st ^ swz_q(R)) << 4) + 8 * (lane >> 5));
      q[j][0] = qp[0];
      q[j][1] = qp[1];
    }
  };
  auto rd_sc = [&](int kt) __attribute__((always_inline)) {
    const char *ss = smem + NS * STAGE + ((kt >> 4) & 1) * SCB + ((kt >> 1) & 7) * 2;
#pragma unroll
    for (int j = 0; j < TN; j++) {
      const int R = wn * WTN + j * 32 + (lane & 31);
      sc[j] = (float)*(const _Float16 *)(ss + R * 16);
      nsc[j] = -128.f * sc[j];
    }
  };
  // the MFMAs of one sub-step, with the codes q dequantised into bn
  auto mma = [&](const bf16x8 *af_, const bf16x8 *bf_, const uint32_t (*q)[2], bf16x8 *bn)
      __attribute__((always_inline)) {
    constexpr int NM = TM * TN, NP = 4 * TN;  // MFMAs, packed pairs to dequantise
    uint32_t x[TN][2];
    u32x4 o[TN];
#pragma unroll
    for (int j = 0; j < TN; j++) {
      x[j][0] = q[j][0] ^ 0x80808080u;  // q + 128 in each byte
      x[j][1] = q[j][1] ^ 0x80808080u;
    }
#pragma unroll
    for (int t = 0; t < NM; t++) {
      acc[t / TN][t % TN] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(af_[t / TN], bf_[t % TN], acc[t / TN][t % TN], 0, 0, 0);
#pragma unroll
      for (int p = t * NP / NM; p < (t + 1) * NP / NM; p++) {
        const int j = p / 4, w = p % 4;
        o[j][w] = dequant2(x[j][w >> 1], (w & 1) * 2, sc[j], nsc[j]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < TN; j++) bn[j] = __builtin_bit_cast(bf16x8, o[j]);
  };

  issue_scales(0);
#pragma unroll
  for (int p = 0; p < NS; p++) issue(p, p);
  wait_vmcnt<(NS - 1) * CPW>();
  __syncthreads();
  if (act) {
    rd_sc(0);
    rd_a(smem, 0, af[0]);
    rd_q(smem + ASTAGE, 0, qv[0]);
    rd_q(smem + ASTAGE, 1, qv[1]);
#pragma unroll
    for (int j = 0; j < TN; j++) bfr[0][j] = dequant8(qv[0][j][0], qv[0][j][1], sc[j], nsc[j]);
  }
  for (int kt = 0; kt < ksteps; kt++) {
    const char *sa = smem + (kt % NS) * STAGE;
    if (act) {
      // sub-steps 0..2: read A of s + 1 and the codes of s + 2 (this stage)
      rd_a(sa, 1, af[1]);
      rd_q(sa + ASTAGE, 2, qv[0]);
      mma(af[0], bfr[0], qv[1], bfr[1]);
      rd_a(sa, 2, af[0]);
      rd_q(sa + ASTAGE, 3, qv[1]);
      mma(af[1], bfr[1], qv[0], bfr[0]);
      rd_a(sa, 3, af[1]);
      mma(af[0], bfr[0], qv[1], bfr[1]);
    }
    // every LDS read of stage kt has returned (its buffer is refilled below)
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), other counters open
    if (kt + NS - 1 < ksteps)
      wait_vmcnt<(NS - 2) * CPW>();  // stage kt + 1 has landed
    else
      wait_vmcnt<0>();
    __syncthreads();
    // the next scale block's buffer was last read in the previous block
    if ((kt & 15) == 0 && kt + 16 < ksteps) issue_scales((kt >> 4) + 1);
    if (kt + NS < ksteps) issue(kt % NS, kt + NS);
    if (act) {
      // sub-step 3, reading sub-steps 0 and 1 of stage kt + 1 (after the last
      // K step: a stale but in-bounds buffer whose values are never used)
      const char *na = smem + ((kt + 1) % NS) * STAGE;
      rd_sc(kt + 1);
      rd_a(na, 0, af[0]);
      rd_q(na + ASTAGE, 0, qv[0]);
      rd_q(na + ASTAGE, 1, qv[1]);
      mma(af[1], bfr[1], qv[0], bfr[0]);
    }
  }
  __builtin_amdgcn_s_waitcnt(0xC07F);  // the last (unused) reads, before the epilogue's writes

  // epilogue as in gemm_dma_kernel
  constexpr int CROW = BN * 2 + 16;
  static_assert(WTM * CROW <= NS * STAGE, "C band fits the stage buffers");
  constexpr int OCPR = BN / 8;
  if constexpr (GELU == 2) {  // with the pre-activation: fp32 sums through LDS
    store_keep_pre<TM, TN, WM, WTM, WTN, BN, NS * STAGE, 64 * W>(acc, smem, wm, wn, lane, tid, m0,
                                                                  n0, rows, N, Zg, Cg);
  } else {
    for (int band = 0; band < WM; band++) {
      __syncthreads();
      if (WM == 1 || wm == band) {
#pragma unroll
        for (int i = 0; i < TM; i++) {
#pragma unroll
          for (int j = 0; j < TN; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
              const int R = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
              const int Cc = wn * WTN + j * 32 + (lane & 31);
              float v = acc[i][j][r];
              if (GELU) v = gelu_f(v);
              *(bf16 *)(smem + R * CROW + Cc * 2) = (bf16)v;
            }
          // one fragment at a time: keeps the accumulators' copies out of
          // the VGPRs the K loop needs (no spills with 256-row wave tiles)
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __syncthreads();
      const int64_t r0 = m0 + band * WTM;
      const int64_t mrows = rows - r0 < WTM ? rows - r0 : WTM;
      for (int idx = tid; idx < WTM * OCPR; idx += 64 * W) {
        const int R = idx / OCPR, ch = idx - R * OCPR;
        if (R < mrows) {
          const u32x4 cv = *(const u32x4 *)(smem + R * CROW + ch * 16);
          u32x4 *dst = (u32x4 *)(Cg + (r0 + R) * N + n0 + ch * 8);
          if constexpr (GELU == 1)
            __builtin_nontemporal_store(cv, dst);  // hidden rows, as in gemm_dma_kernel
          else
            *dst = cv;
        }
      }
    }
  }
}

// One tile per workgroup, tiles laid over the XCDs as in gemm_dma_kernel.
template <int BM, int BN, int WM, int WN, int NS, int GELU>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_i8_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(1024))) char smem[i8_lds_bytes<BM, BN, NS>()];
  const int tiles_n = a.N / BN;
  const int tiles_m = (int)((a.M_cap + BM - 1) / BM);
  const int total = a.G * tiles_m * tiles_n;
  const int tile = (a.G % 8 == 0) ? xcd_remap_grouped(blockIdx.x, a.G, tiles_m * tiles_n)
                                  : xcd_remap(blockIdx.x, total);
  const int g = tile / (tiles_m * tiles_n);
  const int rem = tile - g * tiles_m * tiles_n;
  int tm, tn;
  grouped_tile(rem, tiles_m, tiles_n, tm, tn);
  i8_tile<BM, BN, WM, WN, NS, GELU>(a, g, tm, tn, smem);
}

// Groups placed on the XCDs by a schedule (tile_sched_kernel): the
// workgroups of XCD x (blockIdx % 8 == x) walk that XCD's queue -- its
// groups in schedule order, each group's tiles column by column -- so every
// group still runs on one XCD (operands shared in its L2) while skewed row
// counts are spread evenly over the XCDs.  A group with at most 64 rows (a
// "light" group, marked in the queue) runs BMl x BNl tiles (64 x 512): its
// work is streaming its weights, and the 256 x 256 tile would move 256
// activation rows and only 16 KB of codes per K step; the others run
// BM x BN tiles.  Queue lengths are in units of half the BN-column tiles
// of a row tile: a group of v row tiles counts 2 v, a light group 1 (the
// schedule uses light groups only when N is a multiple of 2 BN = BNl).
template <int BM, int BN, int WM, int WN, int NS, int BMl, int BNl, int WMl, int WNl, int NSl,
          int GELU>
__global__ __launch_bounds__(64 * WM * WN) void gemm_dma_i8_sched_kernel(GemmArgs a) {
  static_assert(WM * WN == WMl * WNl && BNl == 2 * BN, "tile shapes");
  constexpr int LDS = i8_lds_bytes<BM, BN, NS>() > i8_lds_bytes<BMl, BNl, NSl>()
                          ? i8_lds_bytes<BM, BN, NS>()
                          : i8_lds_bytes<BMl, BNl, NSl>();
  __shared__ __attribute__((aligned(1024))) char smem[LDS];
  const int x = blockIdx.x & 7, nbx = gridDim.x >> 3;
  const int tiles_n = a.N / BN;
  const int32_t *xs = a.xsched;
  const int nx = xs[x];
  const int32_t *lst = xs + 8 + x * a.G;
  const int32_t *pre = xs + 8 + 8 * a.G + x * (a.G + 1);
  const int64_t ntiles = (int64_t)pre[nx] * tiles_n / 2;
  for (int64_t i = blockIdx.x >> 3; i < ntiles; i += nbx) {
    // the last queue entry whose tiles start at or before i
    int lo = 0, hi = nx - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)pre[mid] * tiles_n / 2 <= i) lo = mid; else hi = mid - 1;
    }
    const int ent = lst[lo], g = ent & 0xffff;
    const int j = (int)(i - (int64_t)pre[lo] * tiles_n / 2);
    if (ent & kLightGroup) {
      i8_tile<BMl, BNl, WMl, WNl, NSl, GELU>(a, g, 0, j, smem);
    } else {
      const int v = (pre[lo + 1] - pre[lo]) / 2;
      const int tn = j / v, tm = j - tn * v;
      i8_tile<BM, BN, WM, WN, NS, GELU>(a, g, tm, tn, smem);
    }
    __syncthreads();  // the next tile's DMA reuses the LDS of this epilogue
  }
}

// Schedule of the int8 tiles over the 8 XCDs.  A group with at most 64 rows
// runs light tiles when `light` (both GEMMs' N multiples of 512) and costs
// LIGHT_COST; another group's cost is the sum over its 256-row tiles of 8
// for a tile with more than 128 rows (both row bands of waves busy) and 5
// for one with at most 128 (one band does the tile's MFMAs and
// dequantisation, the other only its share of the DMA) -- costs per 256
// output columns, after the tile times measured on the skewed int8 workload
// relative to a full tile: 0.71 (layer 1) and 0.58 (layer 2) for a one-band
// tile, 0.42 per 256 columns for a light 64 x 512 tile.  Groups are taken largest first and each
// goes to the XCD with the least cost so far; each XCD's queue then
// interleaves its light groups (weight streaming) evenly among its other
// groups (mostly MFMA work) by queue length.  Output (int32): [0, 8) queue
// entries per XCD; [8 + x * G, ...) XCD x's entries (group, | kLightGroup for
// a light group); [8 + 8 * G + x * (G + 1), ...) prefix sums of their
// lengths (a group of v row tiles counts 2 v, a light group 1).  One
// workgroup of 256 threads, G <= 256.
__global__ __launch_bounds__(256) void tile_sched_kernel(const int32_t *rows, int G, int64_t M_cap,
                                                         int light, int32_t *xs) {
  constexpr int BM = 256, LIGHT_ROWS = 64, LIGHT_COST = 3, COST_TWO_BANDS = 8, COST_ONE_BAND = 5;
  __shared__ int cost[256], unit[256], order[256], scost[256], sunit[256];
  __shared__ int hl[8][256], ll[8][256], hu[8][256];
  const int tid = threadIdx.x;
  if (tid < G) {
    const int64_t r = rows[tid] < M_cap ? rows[tid] : M_cap;
    int c = 0, u = 0;
    if (light && r > 0 && r <= LIGHT_ROWS) {
      c = LIGHT_COST;
      u = -1;  // light: one unit, flagged by the sign
    } else if (r > 0) {
      const int v = (int)((r + BM - 1) / BM);
      for (int t = 0; t < v; t++) {
        const int64_t rt = r - (int64_t)t * BM < BM ? r - (int64_t)t * BM : BM;
        c += rt > BM / 2 ? COST_TWO_BANDS : COST_ONE_BAND;
      }
      u = 2 * v;
    }
    unit[tid] = u;
    cost[tid] = c;
  }
  __syncthreads();
  if (tid < G) {  // rank by cost, ties to the lower group
    int rk = 0;
    for (int h = 0; h < G; h++) rk += cost[h] > cost[tid] || (cost[h] == cost[tid] && h < tid);
    order[rk] = tid;
    scost[rk] = cost[tid];
    sunit[rk] = unit[tid];
  }
  __syncthreads();
  // the deal: one thread, the XCD loads in registers; each group goes to the
  // XCD with the least cost so far (ties: lower XCD)
  __shared__ int xof[256];
  if (tid == 0) {
    int ld[8];
#pragma unroll
    for (int x = 0; x < 8; x++) ld[x] = 0;
    for (int i = 0; i < G; i++) {
      if (sunit[i] == 0) {  // the rest are empty too (cost 0 ranks last)
        xof[i] = -1;
        continue;
      }
      int bx = 0, bl = ld[0];
#pragma unroll
      for (int x = 1; x < 8; x++)
        if (ld[x] < bl) {
          bl = ld[x];
          bx = x;
        }
      xof[i] = bx;
#pragma unroll
      for (int x = 0; x < 8; x++)
        if (x == bx) ld[x] += scost[i];
    }
  }
  __syncthreads();
  if (tid < 8) {
    // thread x collects XCD x's heavy and light lists in deal order
    const int x = tid;
    int nh = 0, nl = 0, uh = 0;
    for (int i = 0; i < G; i++) {
      if (xof[i] != x) continue;
      const int u = sunit[i];
      if (u < 0) {
        ll[x][nl++] = order[i];
      } else {
        hl[x][nh] = order[i];
        hu[x][nh++] = u;
        uh += u;
      }
    }
    {
      // merge: a light group comes next while the share of light groups
      // placed is below the share of heavy length placed
      int32_t *lst = xs + 8 + x * G, *pre = xs + 8 + 8 * G + x * (G + 1);
      int ih = 0, il = 0, ch = 0, cnt = 0, len = 0;
      while (ih < nh || il < nl) {
        const bool take_l = il < nl && (ih == nh || (int64_t)il * uh < (int64_t)ch * nl);
        pre[cnt] = len;
        if (take_l) {
          lst[cnt++] = ll[x][il++] | kLightGroup;
          len += 1;
        } else {
          lst[cnt++] = hl[x][ih];
          len += hu[x][ih];
          ch += hu[x][ih++];
        }
      }
      xs[x] = cnt;
      pre[cnt] = len;
    }
  }
}

// Row-major [G][N][K] bf16 weights -> MOE_W_BF16_PACKED order: per group,
// blocks of 128 rows, each as K/64 consecutive 128 x 64 pieces.  Thread o
// writes 16-byte unit o of the packed tensor (writes coalesced; eight
// consecutive units read one 128-byte row piece).
__global__ __launch_bounds__(256) void pack_weights_kernel(const u32x4 *src, u32x4 *dst, int64_t N,
                                                           int64_t K, int64_t total) {
  const int64_t per = N * K / 8, kb_n = K / 64;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t g = o / per;
    int64_t r = o - g * per;
    const int64_t c = r & 7;  // unit within the row's 64-wide piece
    r >>= 3;
    const int64_t row = r & 127;  // row within the 128-row block
    r >>= 7;
    const int64_t kb = r % kb_n, nb = r / kb_n;
    dst[o] = src[g * per + ((nb * 128 + row) * K + kb * 64) / 8 + c];
  }
}

// fp32 activations and weights: a plain 64x64 tile, 4x4 outputs per thread,
// any shape (bounds-checked); the correctness path for fp32 layers.
template <int GELU>
__global__ __launch_bounds__(256) void gemm_f32_kernel(GemmArgs a) {
  constexpr int T = 64, BKF = 16;
  __shared__ float As[BKF][T + 1], Bs[BKF][T + 1];
  const int tiles_n = (a.N + T - 1) / T;
  const int tiles_m = (int)((a.M_cap + T - 1) / T);
  const int tile = blockIdx.x;
  const int g = tile / (tiles_m * tiles_n);
  const int rem = tile - g * tiles_m * tiles_n;
  int tm, tn;
  grouped_tile(rem, tiles_m, tiles_n, tm, tn);
  int64_t rows = a.M_cap;
  if (a.rows) {
    const int64_t r = a.rows[g];
    rows = r < rows ? r : rows;
  }
  const int64_t m0 = (int64_t)tm * T;
  if (m0 >= rows) return;
  const int n0 = tn * T, K = a.K, N = a.N;
  const float *Ag = (const float *)a.A + (int64_t)g * a.M_cap * K;
  const float *Bg = (const float *)a.B + (int64_t)g * N * K;
  float *Cg = (float *)a.C + (int64_t)g * a.M_cap * N;
  float *Zg = GELU == 2 ? (float *)a.Zpre + (int64_t)g * a.M_cap * N : nullptr;
  const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += BKF) {
    for (int i = threadIdx.x; i < BKF * T; i += 256) {
      const int r = i / BKF, kk = i % BKF;
      const int64_t m = m0 + r;
      const int n = n0 + r, k = k0 + kk;
      As[kk][r] = (m < rows && k < K) ? Ag[m * K + k] : 0.f;
      Bs[kk][r] = (n < N && k < K) ? Bg[(int64_t)n * K + k] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BKF; kk++)
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < 4; j++) acc[i][j] = fmaf(As[kk][ty * 4 + i], Bs[kk][tx * 4 + j], acc[i][j]);
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const int64_t m = m0 + ty * 4 + i;
      const int n = n0 + tx * 4 + j;
      if (m < rows && n < N) {
        Cg[m * N + n] = GELU ? gelu_f(acc[i][j]) : acc[i][j];
        if (GELU == 2) Zg[m * N + n] = acc[i][j];
      }
    }
}

}  // namespace moe

namespace moe_host {
using namespace moe;

// epilogue variant: 0 none, 1 GELU, 2 GELU and the pre-activation kept in Zpre
static int epi_of(const GemmArgs &a, int gelu) { return gelu ? (a.Zpre ? 2 : 1) : 0; }

template <int BM, int BN, int WM, int WN, int MF, bool I8>
static hipError_t launch_cfg_t(const GemmArgs &a, int epi, dim3 grid, dim3 block, const char *name,
                               hipStream_t s) {
  if (epi == 2)
    MOE_LAUNCH(name, (gemm_bf16_kernel<BM, BN, WM, WN, MF, I8, 2>), grid, block, 0, s, a);
  else if (epi == 1)
    MOE_LAUNCH(name, (gemm_bf16_kernel<BM, BN, WM, WN, MF, I8, 1>), grid, block, 0, s, a);
  else
    MOE_LAUNCH(name, (gemm_bf16_kernel<BM, BN, WM, WN, MF, I8, 0>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int MF>
static hipError_t launch_cfg(const GemmArgs &a, int b_int8, int gelu, hipStream_t s,
                             const char *role, const char *tile) {
  const int tiles = a.G * (int)((a.M_cap + BM - 1) / BM) * (a.N / BN);
  if (tiles <= 0) return hipGetLastError();
  const dim3 grid(tiles), block(64 * WM * WN);
  const char *name = intern_name(role, tile);
  if (b_int8) return launch_cfg_t<BM, BN, WM, WN, MF, true>(a, epi_of(a, gelu), grid, block, name, s);
  return launch_cfg_t<BM, BN, WM, WN, MF, false>(a, epi_of(a, gelu), grid, block, name, s);
}

template <int BM, int BN, int WM, int WN, int BK, int NS, bool NT, bool PB = false>
static hipError_t launch_dma_t(const GemmArgs &a, int epi, dim3 grid, dim3 block, const char *name,
                               hipStream_t s) {
  if (epi == 2)
    MOE_LAUNCH(name, (gemm_dma_kernel<BM, BN, WM, WN, BK, NS, NT, 2, PB>), grid, block, 0, s, a);
  else if (epi == 1)
    MOE_LAUNCH(name, (gemm_dma_kernel<BM, BN, WM, WN, BK, NS, NT, 1, PB>), grid, block, 0, s, a);
  else
    MOE_LAUNCH(name, (gemm_dma_kernel<BM, BN, WM, WN, BK, NS, NT, 0, PB>), grid, block, 0, s, a);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int BK, int NS>
static hipError_t launch_dma(const GemmArgs &a, int nt_b, int gelu, hipStream_t s,
                             const char *role, const char *tile) {
  const int tiles = a.G * (int)((a.M_cap + BM - 1) / BM) * (a.N / BN);
  if (tiles <= 0) return hipGetLastError();
  const dim3 grid(tiles), block(64 * WM * WN);
  if constexpr (BK == 64) {
    if (a.b_packed)  // packed expert weights: streamed once, non-temporal
      return launch_dma_t<BM, BN, WM, WN, BK, NS, true, true>(
          a, epi_of(a, gelu), grid, block, intern_name(role, tile), s);
  } else {
    if (a.b_packed) return hipErrorInvalidValue;  // the packed layout is in 64-wide K steps
  }
  const char *name = intern_name(role, tile);
  if (nt_b)
    return launch_dma_t<BM, BN, WM, WN, BK, NS, true>(a, epi_of(a, gelu), grid, block, name, s);
  return launch_dma_t<BM, BN, WM, WN, BK, NS, false>(a, epi_of(a, gelu), grid, block, name, s);
}

template <int BM, int BN, int WM, int WN, int NS>
static hipError_t launch_dma_i8(const GemmArgs &a, int gelu, hipStream_t s, const char *role,
                                const char *tile) {
  const int tiles = a.G * (int)((a.M_cap + BM - 1) / BM) * (a.N / BN);
  if (tiles <= 0) return hipGetLastError();
  const dim3 grid(tiles), block(64 * WM * WN);
  const int epi = epi_of(a, gelu);
  if constexpr (BM == 256 && BN == 256 && WM * WN == 8) {  // the schedule counts 256-row tiles
    if (a.xsched) {  // light groups: 64 x 512 tiles of 8 waves (64 x 64 each), 3 stages
      const dim3 sgrid((tiles + 7) / 8 * 8);
      const char *name = intern_name(role, "dma256x256_i8_sched");
      if (epi == 2)
        MOE_LAUNCH(name, (gemm_dma_i8_sched_kernel<BM, BN, WM, WN, NS, 64, 512, 1, 8, 3, 2>),
                   sgrid, block, 0, s, a);
      else if (epi == 1)
        MOE_LAUNCH(name, (gemm_dma_i8_sched_kernel<BM, BN, WM, WN, NS, 64, 512, 1, 8, 3, 1>),
                   sgrid, block, 0, s, a);
      else
        MOE_LAUNCH(name, (gemm_dma_i8_sched_kernel<BM, BN, WM, WN, NS, 64, 512, 1, 8, 3, 0>),
                   sgrid, block, 0, s, a);
      return hipGetLastError();
    }
  }
  const char *name = intern_name(role, tile);
  if (epi == 2)
    MOE_LAUNCH(name, (gemm_dma_i8_kernel<BM, BN, WM, WN, NS, 2>), grid, block, 0, s, a);
  else if (epi == 1)
    MOE_LAUNCH(name, (gemm_dma_i8_kernel<BM, BN, WM, WN, NS, 1>), grid, block, 0, s, a);
  else
    MOE_LAUNCH(name, (gemm_dma_i8_kernel<BM, BN, WM, WN, NS, 0>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_pack_weights(const void *w, void *wp, int64_t G, int64_t N, int64_t K,
                               hipStream_t s) {
  const int64_t total = G * N * K / 8;  // 16-byte units
  if (total <= 0) return hipGetLastError();
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  MOE_LAUNCH(intern_name("pack_weights", "b128x64"), pack_weights_kernel, dim3((unsigned)blocks),
             dim3(256), 0, s, (const u32x4 *)w, (u32x4 *)wp, N, K, total);
  return hipGetLastError();
}

hipError_t launch_tile_sched(const int32_t *rows, int G, int64_t M_cap, int light, int32_t *xs,
                             hipStream_t s) {
  if (G < 1 || G > 256) return hipErrorInvalidValue;
  MOE_LAUNCH(intern_name("expert_tile_sched", "lpt"), tile_sched_kernel, dim3(1), dim3(256), 0, s,
             rows, G, M_cap, light, xs);
  return hipGetLastError();
}

// Whether launch_gemm takes a DMA kernel for these shapes (the kernels that
// can read A's rows through a table, GemmArgs::asrc); a_rows: rows of A
// behind the table.  Follows the tile choice below.
bool gemm_reads_row_table(const GemmArgs &a, int act_bf16, int b_int8, int64_t a_rows) {
  if (!act_bf16 || a_rows * a.K * 2 > (int64_t)UINT32_MAX) return false;
  if (b_int8) return a.K % 1024 == 0 && a.N % 256 == 0;
  return a.N % 128 == 0;
}

// Tile choice (measured on MI355X at the workload shapes) by rows per group
// (the capacity, or T for the dense MLP), N, and whether the weights are
// streamed once (expert GEMMs: non-temporal weight loads).
hipError_t launch_gemm(const GemmArgs &a, int act_bf16, int b_int8, int gelu, const char *role,
                       hipStream_t s) {
  if (a.G <= 0 || a.M_cap <= 0 || a.N <= 0) return hipGetLastError();
  // a row table needs a DMA kernel (the caller also checks the row count)
  if (a.asrc && !gemm_reads_row_table(a, act_bf16, b_int8, 0)) return hipErrorInvalidValue;
  if (!act_bf16) {
    const int tiles = a.G * (int)((a.M_cap + 63) / 64) * ((a.N + 63) / 64);
    const char *name = intern_name(role, "f32");
    const int epi = epi_of(a, gelu);
    if (epi == 2)
      MOE_LAUNCH(name, gemm_f32_kernel<2>, dim3(tiles), dim3(256), 0, s, a);
    else if (epi == 1)
      MOE_LAUNCH(name, gemm_f32_kernel<1>, dim3(tiles), dim3(256), 0, s, a);
    else
      MOE_LAUNCH(name, gemm_f32_kernel<0>, dim3(tiles), dim3(256), 0, s, a);
    return hipGetLastError();
  }
  const int nt = a.rows != nullptr;  // grouped expert GEMM: weights read once
  if (b_int8) {  // int8 groups: N and K are multiples of 128 (validated)
    if (a.K % 1024 == 0 && a.N % 256 == 0) {
      if (a.M_cap > 128) return launch_dma_i8<256, 256, 2, 4, 3>(a, gelu, s, role, "dma256x256_i8");
      return launch_dma_i8<128, 256, 2, 4, 4>(a, gelu, s, role, "dma128x256_i8");
    }
    if (a.M_cap <= 32) return launch_cfg<32, 128, 1, 4, 32>(a, 1, gelu, s, role, "bm32_bn128_i8");
    if (a.M_cap <= 64) return launch_cfg<64, 128, 1, 4, 32>(a, 1, gelu, s, role, "bm64_bn128_i8");
    if (a.M_cap <= 128 || a.N % 256)
      return launch_cfg<128, 128, 2, 2, 32>(a, 1, gelu, s, role, "bm128_bn128_i8");
    return launch_cfg<256, 256, 2, 4, 32>(a, 1, gelu, s, role, "bm256_bn256_i8");
  }
  if (a.N % 128 == 0) {
    if (a.M_cap <= 32) {  // a few rows per group (decode): tiles spread over the XCDs
      GemmArgs b = a;
      b.spread = a.rows != nullptr;
      return launch_dma<32, 128, 1, 4, 64, 4>(b, nt, gelu, s, role, "dma32x128");
    }
    if (a.M_cap <= 64) {  // 64x256: two workgroups per CU, 64 KB of weights in flight
      // (three stages, one workgroup per CU, for a long K: 0.197 -> 0.189 ms for
      // the 350M shape's expert layer 2; a short K sweep loses on the longer fill)
      if (a.N % 256 == 0 && a.K >= 4096)
        return launch_dma<64, 256, 1, 4, 64, 3>(a, nt, gelu, s, role, "dma64x256");
      if (a.N % 256 == 0) return launch_dma<64, 256, 1, 4, 64, 2>(a, nt, gelu, s, role, "dma64x256");
      return launch_dma<64, 128, 1, 4, 64, 2>(a, nt, gelu, s, role, "dma64x128");
    }
    if (a.M_cap <= 128) {
      // 128x512, one K step in flight: the same 64 KB of weights in flight
      // as 128x256 with two, and 0.75 instead of 1 KB of LDS operand reads
      // per MFMA
      if (a.N % 512 == 0)
        return launch_dma<128, 512, 2, 4, 64, 2>(a, nt, gelu, s, role, "dma128x512");
      if (a.N % 256 == 0) return launch_dma<128, 256, 2, 4, 64, 3>(a, nt, gelu, s, role, "dma128x256");
    }
    if (a.M_cap > 128 && a.N % 256 == 0)
      return launch_dma<256, 256, 2, 4, 64, 2>(a, nt, gelu, s, role, "dma256x256");
    return launch_dma<128, 128, 2, 2, 64, 2>(a, nt, gelu, s, role, "dma128x128");
  }
  // any N that is a multiple of 64
  return launch_cfg<16, 64, 1, 4, 16>(a, 0, gelu, s, role, "bm16_bn64");
}

}  // namespace moe_host
