// backward.hip -- backward of the MoE layer on gfx950.
//
// Gradients of <dy, y> + g_aux * aux + g_z * z with respect to x and every
// weight, by the chain rule through the forward stages (the method's layer:
// "DeepSpeed MoE and Model Compression", section DeepSpeed-MoE; capacity
// overflow: "DeepSpeed-MoE vs Switch Transformer", where a dropped token skips
// the expert and so gets no expert gradient; gates renormalised over the
// top-k: survey notes sec. 1.1.1.1; Switch load-balance loss: survey notes
// sec. 1.1.4.1; router z-loss: "DeepSpeed-MoE vs Switch Transformer", section
// Router Z-loss).  Per kept assignment (t, j) of expert e at slot s:
//   dg[t,j] = <dy[t], y_disp[e,s]>,   dY[e,s] = g[t,j] dy[t]
// expert FFN (a = W1 x, h = GELU(a), out = W2 h), all as grouped GEMMs:
//   dZ = (dY W2) * GELU'(Z),  dX = dZ W1,  dW2 = dY^T H,  dW1 = dZ^T X
// router: dp from dg (through the renormalisation) and from the aux loss
// (f_e is piecewise constant), softmax Jacobian, plus the z-loss term
// (2/T) lse p; then dx += dlogits W_r, dW_r = dlogits^T x, db = sum dlogits.
// The PR-MoE dense MLP is the same FFN backward with d(out) = dy.
#include "common.h"
#include "dma.h"
#include "kernels.h"

namespace moe {

__device__ __forceinline__ float gelu_grad_f(float z) {
  // Phi(z) + z phi(z)
  const float cdf = 0.5f * (1.0f + erf_as(z * 0.70710678118654752440f));
  return cdf + z * 0.39894228040143267794f * __expf(-0.5f * z * z);
}

// ---------------------------------------------------------------------------
// General grouped GEMM for the backward products:
//   C(g, m, n) = epi( sum_k A(g, m, k) B(g, n, k) ),  m < rows of group g
// A(g, m, k) = A[g a_g + m a_m + k a_k] with either a_k == 1 (K contiguous)
// or a_m == 1 (K-major, the layout the forward's weights and activations have
// for the products that contract over their other index); the same for B.
// Tiles: 128 x BN x 32, four waves of 64 x BN/2, 32x32x16 bf16 MFMA, fp32
// accumulators.  Operands go through registers into LDS as [row][k] (rows of
// 40 elements: 80-byte stride, conflict-free 16-byte operand reads); a
// K-major operand is loaded 8 rows wide at one k and written transposed.
// Reduction steps past the group's valid K read as zero; rows past the
// group's valid M are clamped on load and not stored.

template <int BN, bool AKM, bool BKM, bool DGELU>
__global__ __launch_bounds__(256) void gemm_gen_kernel(GenArgs a) {
  constexpr int BM = 128, BK = 32, LDK = BK + 8;
  constexpr int WTN = BN / 2, TM = 2, TN = WTN / 32;
  __shared__ __attribute__((aligned(16))) bf16 As[2][BM * LDK];
  __shared__ __attribute__((aligned(16))) bf16 Bs[2][BN * LDK];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 2, wn = wave % 2;
  const int tiles_m = (int)((a.M + BM - 1) / BM), tiles_n = a.N / BN;
  // a group's tiles on one XCD (its operand panels shared in that L2), in
  // grouped order, as in the forward GEMMs
  const int per = tiles_m * tiles_n, total = a.G * per;
  const int tile = (a.G % 8 == 0) ? xcd_remap_grouped(blockIdx.x, a.G, per)
                                  : xcd_remap(blockIdx.x, total);
  const int g = tile / per;
  const int rem = tile - g * per;
  int tm, tn;
  grouped_tile(rem, tiles_m, tiles_n, tm, tn);
  int64_t mvalid = a.M;
  if (a.mrows) mvalid = a.mrows[g] < mvalid ? a.mrows[g] : mvalid;
  const int64_t m0 = (int64_t)tm * BM;
  if (m0 >= mvalid) return;
  const int n0 = tn * BN;
  int64_t kvalid = a.K;
  if (a.krows) kvalid = a.krows[g] < kvalid ? a.krows[g] : kvalid;
  const int ksteps = (int)((kvalid + BK - 1) / BK);
  const bf16 *Ag = a.A + (int64_t)g * a.a_g;
  const bf16 *Bg = a.B + (int64_t)g * a.b_g;

  // per thread: two 16-byte chunks of each operand per K step
  u32x4 ra[2], rb[2];
  const u32x4 zero = {0u, 0u, 0u, 0u};
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 2; p++) {
      const int c = tid + 256 * p;
      if constexpr (!AKM) {  // 128 rows x 4 chunks along k
        const int r = c >> 2, kc = (c & 3) * 8;
        int64_t m = m0 + r;
        if (m >= mvalid) m = mvalid - 1;
        ra[p] = (k0 + kc < kvalid) ? *(const u32x4 *)(Ag + m * a.a_m + (k0 + kc)) : zero;
      } else {  // 32 k rows x 16 chunks along m
        const int k = c >> 4, rc = (c & 15) * 8;
        const int64_t kk = k0 + k;
        const bool ok = kk < kvalid && kk < a.a_kmax && m0 + rc < a.M;
        ra[p] = ok ? *(const u32x4 *)(Ag + kk * a.a_k + m0 + rc) : zero;
      }
      if constexpr (!BKM) {
        const int r = c >> 2, kc = (c & 3) * 8;
        if (r < BN)
          rb[p] = (k0 + kc < kvalid) ? *(const u32x4 *)(Bg + (int64_t)(n0 + r) * a.b_n + (k0 + kc))
                                     : zero;
      } else {
        const int k = c >> 4, rc = (c & 15) * 8;
        const int64_t kk = k0 + k;
        if (rc < BN) {
          const bool ok = kk < kvalid && kk < a.b_kmax;
          rb[p] = ok ? *(const u32x4 *)(Bg + kk * a.b_k + n0 + rc) : zero;
        }
      }
    }
  };
  auto store = [&](int st) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < 2; p++) {
      const int c = tid + 256 * p;
      if constexpr (!AKM) {
        const int r = c >> 2, kc = (c & 3) * 8;
        *(u32x4 *)(&As[st][r * LDK + kc]) = ra[p];
      } else {
        const int k = c >> 4, rc = (c & 15) * 8;
        const bf16 *v = (const bf16 *)&ra[p];
#pragma unroll
        for (int i = 0; i < 8; i++) As[st][(rc + i) * LDK + k] = v[i];
      }
      if constexpr (!BKM) {
        const int r = c >> 2, kc = (c & 3) * 8;
        if (r < BN) *(u32x4 *)(&Bs[st][r * LDK + kc]) = rb[p];
      } else {
        const int k = c >> 4, rc = (c & 15) * 8;
        if (rc < BN) {
          const bf16 *v = (const bf16 *)&rb[p];
#pragma unroll
          for (int i = 0; i < 8; i++) Bs[st][(rc + i) * LDK + k] = v[i];
        }
      }
    }
  };

  f32x16 acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

  if (ksteps > 0) {
    load(0);
    store(0);
  }
  __syncthreads();
  for (int kt = 0; kt < ksteps; kt++) {
    const int st = kt & 1;
    if (kt + 1 < ksteps) load((kt + 1) * BK);
#pragma unroll
    for (int s = 0; s < BK / 16; s++) {
      const int col = 16 * s + 8 * (lane >> 5);
      bf16x8 af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; i++)
        af[i] = *(const bf16x8 *)(&As[st][(wm * 64 + i * 32 + (lane & 31)) * LDK + col]);
#pragma unroll
      for (int j = 0; j < TN; j++)
        bfr[j] = *(const bf16x8 *)(&Bs[st][(wn * WTN + j * 32 + (lane & 31)) * LDK + col]);
#pragma unroll
      for (int i = 0; i < TM; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < ksteps) store(st ^ 1);
    __syncthreads();
  }

  // 32x32 MFMA layout: register r of lane l holds row 8(r/4) + 4(l/32) + r%4,
  // column l%32
  bf16 *Cg = a.C + (int64_t)g * a.c_g;
  const bf16 *Zg = DGELU ? a.Z + (int64_t)g * a.c_g : nullptr;
#pragma unroll
  for (int i = 0; i < TM; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int64_t m = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int n = n0 + wn * WTN + j * 32 + (lane & 31);
        if (m < mvalid) {
          float v = acc[i][j][r];
          if (DGELU) v *= gelu_grad_f((float)Zg[m * a.c_m + n]);
          Cg[m * a.c_m + n] = (bf16)v;
        }
      }
}

// ---------------------------------------------------------------------------
// The same products on the LDS-DMA pipeline, for the large shapes (M and N
// multiples of 128, K a multiple of 32; reduction rows past the group's
// valid K are zeroed in LDS before use).  Tiles 128 x 128 x 32, four waves of
// 64 x 64, NS stages in flight.  A K-contiguous operand is staged as in the
// forward GEMM ([row][k], 64-byte rows, slot c ^ ((R >> 2) & 3)).  A K-major
// operand is staged as it lies in memory, [k][row] with 256-byte rows, chunk
// c of row k in slot c ^ 4 (k & 3), and its MFMA fragments are read with
// gfx950's transposing LDS read ds_read_b64_tr_b16: within each 16-lane group
// lane i receives element i % 4 of the 4-element pieces addressed by lanes
// i/4, 4 + i/4, 8 + i/4, 12 + i/4 (measured on MI355X), so lane r of a group
// addressing row k0 + r/4, elements e0 + 4 (r % 4) hands lane i the values of
// element e0 + i at k0 .. k0 + 3 -- the 32x32x16 operand layout.  The swizzle
// spreads a half-wave's 32 eight-byte reads over all 64 banks.
typedef __bf16 bf16x4v __attribute__((__vector_size__(4 * sizeof(__bf16))));

__device__ __forceinline__ int swz_km(int k) { return 4 * (k & 3); }

// 8 consecutive k (kbase + 8 (lane / 32) ...) of row row0 + lane % 32 from a
// K-major tile of 128-element rows at LDS byte address `tile`
__device__ __forceinline__ bf16x8 frag_kmajor(uint32_t tile, int row0, int kbase, int lane) {
  const int g = lane >> 4, r = lane & 15;
  const int e = row0 + 16 * (g & 1) + 4 * (r & 3);
  bf16x8 out;
#pragma unroll
  for (int p = 0; p < 2; p++) {
    const int k = kbase + 8 * (g >> 1) + 4 * p + (r >> 2);
    const uint32_t off = tile + k * 256 + ((((e >> 3) ^ swz_km(k)) << 4) | ((e & 7) << 1));
    const bf16x4v v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) bf16x4v *)(uintptr_t)off);
#pragma unroll
    for (int j = 0; j < 4; j++) out[4 * p + j] = v[j];
  }
  return out;
}

// BM = 128 (waves 2 x 2 of 64 x BN/2) or 64 (waves 1 x 4 of 64 x BN/4; the A
// operand K-contiguous), for groups of at most 64 rows (a capacity of 64).
template <bool AKM, bool BKM, bool DGELU, int NS, int BK = 32, int BM = 128, bool NTB = false,
          int BN = 128>
__global__ __launch_bounds__(256) void gemm_dmag_kernel(GenArgs a) {
  static_assert(BK == 32 || BK == 64, "K step");
  static_assert(BM == 128 || (BM == 64 && !AKM), "tile rows");
  // BN = 256 (K-major B only): the B tile is two 128-column sub-tiles, each
  // laid out as a 128-column tile, so a K row of B is 512 contiguous bytes
  static_assert(BN == 128 || (BN == 256 && BKM), "tile columns");
  constexpr int NSUB = BN / 128;
  constexpr int TILEA = BM * BK * 2, TILE = BN * BK * 2;  // bytes per operand tile
  constexpr int STAGE = TILEA + TILE;
  constexpr int CHA = TILEA / 1024 / 4, CH = TILE / 1024 / 4;  // 1-KB DMA chunks per wave
  constexpr int WM = BM / 64, WN = 4 / WM, WTN = BN / WN, TN = WTN / 32;
  constexpr int ROWB = BK * 2, CPR = ROWB / 16, RPC = 1024 / ROWB;  // K-contiguous rows
  static_assert(NS >= 2 && NS * STAGE <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[NS * STAGE];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / WN, wn = wave % WN;
  const int tiles_m = (int)((a.M + BM - 1) / BM), tiles_n = a.N / BN;
  // a group's tiles on one XCD (its operand panels shared in that L2), in
  // grouped order, as in the forward GEMMs
  const int per = tiles_m * tiles_n, total = a.G * per;
  const int tile = (a.G % 8 == 0) ? xcd_remap_grouped(blockIdx.x, a.G, per)
                                  : xcd_remap(blockIdx.x, total);
  const int g = tile / per;
  const int rem = tile - g * per;
  int tm, tn;
  grouped_tile(rem, tiles_m, tiles_n, tm, tn);
  int64_t mvalid = a.M;
  if (a.mrows) mvalid = a.mrows[g] < mvalid ? a.mrows[g] : mvalid;
  const int64_t m0 = (int64_t)tm * BM;
  if (m0 >= mvalid) return;
  const int n0 = tn * BN;
  int64_t kvalid = a.K;
  if (a.krows) kvalid = a.krows[g] < kvalid ? a.krows[g] : kvalid;
  const int ksteps = (int)((kvalid + BK - 1) / BK);
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;

  // per-tile operand bases (bytes) and this lane's offsets for its chunks:
  // every wave moves CHA chunks (1 KB each) of A and CH of B per stage
  const char *abase, *bbase;
  int64_t astep, bstep;  // bytes per K step
  uint32_t voa[CHA], vob[CH];
#pragma unroll
  for (int i = 0; i < CHA; i++) {
    const int q = CHA * wave + i;
    if constexpr (!AKM) {  // rows of ROWB bytes: RPC rows per chunk
      const int R = RPC * q + lane / CPR, slot = lane % CPR;
      int64_t m = m0 + R;
      if (m >= mvalid) m = mvalid - 1;
      voa[i] = (uint32_t)((m - m0) * a.a_m * 2 + ((slot ^ swz_slot<BK>(R)) << 4));
    } else {  // k rows of 256 bytes: 4 rows per chunk
      const int k = 4 * q + lane / 16, slot = lane % 16;
      voa[i] = (uint32_t)(k * a.a_k * 2 + ((slot ^ swz_km(k)) << 4));
    }
  }
#pragma unroll
  for (int i = 0; i < CH; i++) {
    const int q = CH * wave + i;
    if constexpr (!BKM) {
      const int R = RPC * q + lane / CPR, slot = lane % CPR;
      vob[i] = (uint32_t)(R * a.b_n * 2 + ((slot ^ swz_slot<BK>(R)) << 4));
    } else {  // sub-tile q / (BK / 4), its k rows 4 (q % (BK / 4)) ..
      const int h = q / (BK / 4), k = 4 * (q % (BK / 4)) + lane / 16, slot = lane % 16;
      vob[i] = (uint32_t)(k * a.b_k * 2 + h * 256 + ((slot ^ swz_km(k)) << 4));
    }
  }
  if constexpr (!AKM) {
    abase = (const char *)(a.A + (int64_t)g * a.a_g + m0 * a.a_m);
    astep = BK * 2;
  } else {
    abase = (const char *)(a.A + (int64_t)g * a.a_g + m0);
    astep = (int64_t)BK * a.a_k * 2;
  }
  if constexpr (!BKM) {
    bbase = (const char *)(a.B + (int64_t)g * a.b_g + (int64_t)n0 * a.b_n);
    bstep = BK * 2;
  } else {
    bbase = (const char *)(a.B + (int64_t)g * a.b_g + n0);
    bstep = (int64_t)BK * a.b_k * 2;
  }
  auto issue = [&](int st, int kt) __attribute__((always_inline)) {
    const char *ga = abase + (int64_t)kt * astep, *gb = bbase + (int64_t)kt * bstep;
#pragma unroll
    for (int i = 0; i < CHA; i++)
      dma16<false>(ga, voa[i],
                   __builtin_amdgcn_readfirstlane(lds0 + st * STAGE + (CHA * wave + i) * 1024));
#pragma unroll
    for (int i = 0; i < CH; i++)
      dma16<NTB>(gb, vob[i], __builtin_amdgcn_readfirstlane(lds0 + st * STAGE + TILEA +
                                                            (CH * wave + i) * 1024));
  };

  f32x16 acc[2][TN];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < TN; j++)
#pragma unroll
      for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

#pragma unroll
  for (int p = 0; p < NS - 1; p++)
    if (p < ksteps) issue(p, p);
  for (int kt = 0; kt < ksteps; kt++) {
    if (kt + NS - 2 < ksteps)
      wait_vmcnt<(NS - 2) * (CHA + CH)>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    const int st = kt % NS;
    const int kleft = (int)(kvalid - (int64_t)kt * BK);
    if (kleft < BK) {  // ragged last step: zero the k rows past the valid ones
      // (only K-major operands reach here: the host keeps K-contiguous K whole)
      for (int idx = tid; idx < (BK - kleft) * 16; idx += 256) {
        const int k = kleft + idx / 16, c = idx % 16;
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (AKM) *(u32x4 *)(smem + st * STAGE + k * 256 + c * 16) = z;
        if (BKM)
#pragma unroll
          for (int h = 0; h < NSUB; h++)
            *(u32x4 *)(smem + st * STAGE + TILEA + h * BK * 256 + k * 256 + c * 16) = z;
      }
      __syncthreads();
    }
    if (kt + NS - 1 < ksteps) issue((kt + NS - 1) % NS, kt + NS - 1);
    const uint32_t ta = lds0 + st * STAGE, tb = ta + TILEA;
#pragma unroll
    for (int s = 0; s < BK / 16; s++) {
      bf16x8 af[2], bfr[TN];
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int row0 = wm * 64 + i * 32;
        if constexpr (AKM) {
          af[i] = frag_kmajor(ta, row0, 16 * s, lane);
        } else {
          const int R = row0 + (lane & 31), c = 2 * s + (lane >> 5);
          af[i] = *(const bf16x8 *)(smem + st * STAGE + R * ROWB + ((c ^ swz_slot<BK>(R)) << 4));
        }
      }
#pragma unroll
      for (int j = 0; j < TN; j++) {
        const int row0 = wn * WTN + j * 32;
        if constexpr (BKM) {
          bfr[j] = frag_kmajor(tb + (row0 / 128) * BK * 256, row0 % 128, 16 * s, lane);
        } else {
          const int R = row0 + (lane & 31), c = 2 * s + (lane >> 5);
          bfr[j] = *(const bf16x8 *)(smem + st * STAGE + TILEA + R * ROWB +
                                     ((c ^ swz_slot<BK>(R)) << 4));
        }
      }
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // epilogue through LDS, one 64-row band (the two waves with wm == band) at
  // a time, in fp32 (rows of 132 floats): coalesced 16-byte stores, and the
  // GELU' factor applied before the single rounding to bf16
  bf16 *Cg = a.C + (int64_t)g * a.c_g;
  const bf16 *Zg = DGELU ? a.Z + (int64_t)g * a.c_g : nullptr;
  constexpr int CROW = BN + 4, CPRW = BN / 8;  // floats per LDS row, 8-wide chunks per row
  static_assert(64 * CROW * 4 <= NS * STAGE, "band fits the stages");
  float *cs = (float *)smem;
  for (int band = 0; band < WM; band++) {
    __syncthreads();  // stages (or the previous band) no longer read
    if (wm == band) {
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < TN; j++)
#pragma unroll
          for (int r = 0; r < 16; r++) {
            const int R = i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            const int Cc = wn * WTN + j * 32 + (lane & 31);
            cs[R * CROW + Cc] = acc[i][j][r];
          }
    }
    __syncthreads();
    const int64_t r0 = m0 + band * 64;
    for (int idx = tid; idx < 64 * CPRW; idx += 256) {
      const int R = idx / CPRW, ch = idx % CPRW;
      const int64_t m = r0 + R;
      if (m >= mvalid) continue;
      const float *src = cs + R * CROW + ch * 8;
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; q++) v[q] = src[q];
      if (DGELU) {
        const bf16x8 z = *(const bf16x8 *)(Zg + m * a.c_m + n0 + ch * 8);
#pragma unroll
        for (int q = 0; q < 8; q++) v[q] *= gelu_grad_f((float)z[q]);
      }
      bf16x8 o;
#pragma unroll
      for (int q = 0; q < 8; q++) o[q] = (bf16)v[q];
      *(bf16x8 *)(Cg + m * a.c_m + n0 + ch * 8) = o;
    }
  }
}

// ---------------------------------------------------------------------------
// Weight gradients of the experts, whose reduction runs over the expert's
// kept rows only (K <= KR <= 128):  C(g, m, n) = sum_{k < kvalid} A(g, m, k)
// B(g, n, k), both operands K-major.  A workgroup owns a 128-row panel of C
// and one of nsplit equal ranges of its 128-column tiles: it loads the
// panel's A slab (KR rows of 128 elements, as stored) once, keeps its MFMA
// fragments in registers, and streams the B slabs of its tiles through two
// LDS stages by DMA, one tile ahead.  The MFMA runs with the operands' roles
// exchanged (B slab rows as the first operand), so each lane ends with four
// consecutive columns of one row of C; every wave stages its 64 x 64 block
// in a private LDS patch and stores it as whole 128-byte row segments.  The
// stores drain while the next tile computes: the one barrier per tile orders
// LDS only, and the wait for a B slab lets this wave's eight stores of the
// previous tile stay in flight (a wave's vector memory operations complete
// in issue order).  Panels start their sweeps at different tiles (panel tm
// at tile tm of its range), so the workgroups running at once read
// different B slabs and write different column ranges instead of all
// hitting the same few L2 channels.  Reduction rows past kvalid: B rows are
// loaded from row kvalid - 1 (finite values) and the matching A rows are
// zeroed in LDS, so they add exactly zero.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int swz_patch(int m) { return (m >> 1) & 7; }

template <int KR>
__global__ __launch_bounds__(256) void gemm_dwk_kernel(GenArgs a) {
  constexpr int BM = 128, BN = 128;
  constexpr int SLAB = KR * 256;  // bytes of a K-major slab of 128 columns
  constexpr int CH = KR / 16;     // 1-KB DMA chunks per wave per slab
  constexpr int PATCH = 64 * 128;
  constexpr int STORES = PATCH / (kWave * 16);  // 16-byte stores per lane per tile
  constexpr int KS = KR / 16;                   // MFMA reduction steps
  static_assert(3 * SLAB + 4 * PATCH <= 160 * 1024, "LDS budget");
  __shared__ __attribute__((aligned(1024))) char smem[3 * SLAB + 4 * PATCH];
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / 2, wn = wave % 2;
  const int tiles_m = (int)(a.M / BM), S = a.nsplit;
  const int tiles_n = a.N / BN / S;  // tiles of this workgroup's range
  const int per_group = tiles_m * S;
  const int blk = (a.G % 8 == 0) ? xcd_remap_grouped(blockIdx.x, a.G, per_group)
                                 : xcd_remap(blockIdx.x, a.G * per_group);
  const int g = blk / per_group, rr = blk - g * per_group;
  const int tm = rr / S, t0 = (rr - tm * S) * tiles_n;  // panel, first tile of the range
  const int64_t m0 = (int64_t)tm * BM;
  int kvalid = (int)a.K;
  if (a.krows && a.krows[g] < kvalid) kvalid = a.krows[g];
  bf16 *Cg = a.C + (int64_t)g * a.c_g + m0 * a.c_m + (int64_t)t0 * BN;
  if (kvalid <= 0) {  // no kept rows: the gradient is zero
    const u32x4 z = {0u, 0u, 0u, 0u};
    const int per_row = tiles_n * BN / 8;
    for (int r = 0; r < BM; r++)
      for (int c = tid; c < per_row; c += 256) *(u32x4 *)(Cg + (int64_t)r * a.c_m + 8 * c) = z;
    return;
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
  const uint32_t lds_a = lds0, lds_b = lds0 + SLAB;
  char *patch = smem + 3 * SLAB + wave * PATCH;

  // chunk q = CH * wave + i holds k rows 4q .. 4q + 3; lane: row 4q + lane / 16,
  // slot lane % 16, which holds the row's 16-byte chunk slot ^ swz_km(k)
  uint32_t voa[CH], vob[CH];
#pragma unroll
  for (int i = 0; i < CH; i++) {
    const int k = 4 * (CH * wave + i) + lane / 16, slot = lane % 16;
    const int kk = k < kvalid ? k : kvalid - 1;
    const uint32_t c16 = (uint32_t)((slot ^ swz_km(k)) << 4);
    voa[i] = (uint32_t)(kk * a.a_k * 2) + c16;
    vob[i] = (uint32_t)(kk * a.b_k * 2) + c16;
  }
  const char *abase = (const char *)(a.A + (int64_t)g * a.a_g + m0);
  const char *bbase = (const char *)(a.B + (int64_t)g * a.b_g + (int64_t)t0 * BN);
  // the i-th tile of the sweep (staggered start) and its B slab into stage i & 1
  auto tile_of = [&](int i) { return (i + tm) % tiles_n; };
  auto issue_b = [&](int i) __attribute__((always_inline)) {
    const char *gb = bbase + (int64_t)tile_of(i) * BN * 2;
    const uint32_t st = lds_b + (i & 1) * SLAB;
#pragma unroll
    for (int c = 0; c < CH; c++)
      dma16<false>(gb, vob[c], __builtin_amdgcn_readfirstlane(st + (CH * wave + c) * 1024));
  };
#pragma unroll
  for (int i = 0; i < CH; i++)
    dma16<false>(abase, voa[i], __builtin_amdgcn_readfirstlane(lds_a + (CH * wave + i) * 1024));
  issue_b(0);
  wait_vmcnt<0>();
  lds_barrier();  // every wave's part has landed
  // A rows kvalid .. KR - 1 (loaded from row kvalid - 1) become zero
  for (int idx = tid; idx < (KR - kvalid) * 16; idx += 256) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    *(u32x4 *)(smem + (kvalid + idx / 16) * 256 + (idx % 16) * 16) = z;
  }
  lds_barrier();
  bf16x8 af[KS][2];
#pragma unroll
  for (int s = 0; s < KS; s++)
#pragma unroll
    for (int i = 0; i < 2; i++) af[s][i] = frag_kmajor(lds_a, wm * 64 + i * 32, 16 * s, lane);

  for (int it = 0; it < tiles_n; it++) {
    if (it > 0) {
      wait_vmcnt<STORES>();  // newer than slab it's DMA: this wave's stores of tile it - 1
      lds_barrier();         // every wave's part of slab it; stage (it + 1) & 1 free
    }
    if (it + 1 < tiles_n) issue_b(it + 1);
    const uint32_t tb = lds_b + (it & 1) * SLAB;
    f32x16 acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;
#pragma unroll
    for (int s = 0; s < KS; s++) {
      bf16x8 bfr[2];
#pragma unroll
      for (int j = 0; j < 2; j++) bfr[j] = frag_kmajor(tb, wn * 64 + j * 32, 16 * s, lane);
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < 2; j++)  // D[n][m]: rows from the B slab
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af[s][i], acc[i][j], 0, 0, 0);
    }
    // lane: row m = 32 i + lane % 32 of the wave's block, columns
    // 32 j + 8 q + 4 (lane / 32) + 0..3 from registers 4 q .. 4 q + 3
#pragma unroll
    for (int i = 0; i < 2; i++)
#pragma unroll
      for (int j = 0; j < 2; j++)
#pragma unroll
        for (int q = 0; q < 4; q++) {
          const int m = 32 * i + (lane & 31), c = 4 * j + q;
          bf16x4v v;
#pragma unroll
          for (int e = 0; e < 4; e++) v[e] = (bf16)acc[i][j][4 * q + e];
          *(bf16x4v *)(patch + m * 128 + ((c ^ swz_patch(m)) << 4) + 8 * (lane >> 5)) = v;
        }
    asm volatile("" ::: "memory");  // the wave's LDS operations run in order
    bf16 *Ct = Cg + (int64_t)(wm * 64) * a.c_m + tile_of(it) * BN + wn * 64;
#pragma unroll
    for (int p = 0; p < STORES; p++) {
      const int R = 8 * p + lane / 8, c = lane % 8;
      const u32x4 v = *(const u32x4 *)(patch + R * 128 + ((c ^ swz_patch(R)) << 4));
      __builtin_nontemporal_store(v, (u32x4 *)(Ct + (int64_t)R * a.c_m + 8 * c));
    }
    asm volatile("" ::: "memory");  // the stores stay ahead of the next wait
  }
}

// H = GELU(Z), elementwise (bf16)
__global__ __launch_bounds__(256) void gelu_map_kernel(const bf16 *z, bf16 *h, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    h[i] = (bf16)gelu_f((float)z[i]);
}

// one wave per assignment: dg = <dy[t], y_disp[e,s]>, dY[e,s] = g dy[t]
__global__ __launch_bounds__(256) void bwd_gate_kernel(const bf16 *dy, const bf16 *y_disp,
                                                       const int32_t *ids, const int32_t *slots,
                                                       const float *gates, int64_t n_assign,
                                                       int k, int d, int64_t C, int E, float *dg,
                                                       bf16 *dY) {
  const int lane = lane_id();
  const int64_t a = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (a >= n_assign) return;
  const int s = __builtin_amdgcn_readfirstlane(slots[a]);
  const int e = __builtin_amdgcn_readfirstlane(ids[a]);
  if (s < 0 || s >= C || e < 0 || e >= E) {
    if (lane == 0) dg[a] = 0.f;
    return;
  }
  const float g = gates[a];
  const bf16 *dyt = dy + (a / k) * (int64_t)d;
  const bf16 *yr = y_disp + ((int64_t)e * C + s) * d;
  bf16 *dr = dY + ((int64_t)e * C + s) * d;
  float acc = 0.f;
  for (int o = lane * 8; o < d; o += kWave * 8) {
    const bf16x8 u = *(const bf16x8 *)(dyt + o), v = *(const bf16x8 *)(yr + o);
    bf16x8 w;
#pragma unroll
    for (int i = 0; i < 8; i++) {
      acc += (float)u[i] * (float)v[i];
      w[i] = (bf16)(g * (float)u[i]);
    }
    *(bf16x8 *)(dr + o) = w;
  }
  acc = wave_sum(acc);
  if (lane == 0) dg[a] = acc;
}

__global__ __launch_bounds__(256) void first_choice_kernel(const int32_t *ids, int64_t T, int k,
                                                           int E, int32_t *cnt) {
  for (int64_t t = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; t < T;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int e = ids[t * k];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
}

__global__ __launch_bounds__(256) void fill_i32_kernel(int32_t *p, int n, int v) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

// one wave per token: dlogits from the gate gradients, the aux loss and the
// z-loss; fp32 [T, E] and bf16 [T, Ep] (zero past E) copies
__global__ __launch_bounds__(256) void bwd_router_kernel(
    const float *logits, const int32_t *ids, const float *gates, const float *dg,
    const int32_t *fcnt, int64_t T, int E, int Ep, int k, int normalize, float alpha,
    float g_aux, float g_z, float *dlog, bf16 *dlog16) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  float l[4], p[4], dp[4];
  float m = neg_inf();
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = lane + kWave * i;
    l[i] = e < E ? logits[t * E + e] : neg_inf();
    m = fmaxf(m, l[i]);
  }
  m = wave_max(m);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = lane + kWave * i;
    p[i] = e < E ? __expf(l[i] - m) : 0.f;
    s += p[i];
  }
  s = wave_sum(s);
  const float lse = m + logf(s);
  const float aux_scale = g_aux * alpha * (float)E / (float)T / (float)T;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = lane + kWave * i;
    p[i] = p[i] / s;
    dp[i] = e < E ? aux_scale * (float)fcnt[e] : 0.f;
  }
  // gate gradients (the same values in every lane)
  float S = 0.f, sdg = 0.f;
  for (int j = 0; j < k; j++) {
    const int ej = ids[t * k + j];
    // p[ej] lives in lane ej % 64, register ej / 64
    float pv = p[0];
    if ((ej >> 6) == 1) pv = p[1];
    if ((ej >> 6) == 2) pv = p[2];
    if ((ej >> 6) == 3) pv = p[3];
    S += __shfl(pv, ej & 63, kWave);
    sdg += dg[t * k + j] * gates[t * k + j];
  }
  const bool renorm = k >= 2 && normalize;
  for (int j = 0; j < k; j++) {
    const int ej = ids[t * k + j];
    const float v = renorm ? (dg[t * k + j] - sdg) / S : dg[t * k + j];
#pragma unroll
    for (int i = 0; i < 4; i++)
      if (lane + kWave * i == ej) dp[i] += v;
  }
  float pdp = 0.f;
#pragma unroll
  for (int i = 0; i < 4; i++) pdp += p[i] * dp[i];
  pdp = wave_sum(pdp);
  const float zc = g_z * 2.0f / (float)T * lse;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int e = lane + kWave * i;
    const float v = p[i] * (dp[i] - pdp) + zc * p[i];
    if (e < E) dlog[t * E + e] = v;
    if (e < Ep) dlog16[t * Ep + e] = (bf16)(e < E ? v : 0.f);
  }
}

// db[e] = sum over tokens of dlog[t, e], fixed order (chunks, then a tree)
__global__ __launch_bounds__(256) void colsum_kernel(const float *dlog, int64_t T, int E,
                                                     float *db) {
  __shared__ double red[256];
  const int e = blockIdx.x, tid = threadIdx.x;
  const int64_t chunk = (T + 255) / 256;
  const int64_t t0 = tid * chunk, t1 = t0 + chunk < T ? t0 + chunk : T;
  double v = 0.0;
  for (int64_t t = t0; t < t1; t++) v += (double)dlog[t * E + e];
  red[tid] = v;
  __syncthreads();
  for (int st = 128; st >= 1; st >>= 1) {
    if (tid < st) red[tid] += red[tid + st];
    __syncthreads();
  }
  if (tid == 0) db[e] = (float)red[0];
}

// one wave per token: dx = [dy] + [dx_dense] + dx_router + sum over kept j of
// dX[e_j, s_j], accumulated in fp32 in that order
__global__ __launch_bounds__(256) void bwd_dx_kernel(const bf16 *dy, const bf16 *dxd,
                                                     const bf16 *dxr, const bf16 *dX,
                                                     const int32_t *ids, const int32_t *slots,
                                                     int64_t T, int k, int d, int64_t C, int E,
                                                     bf16 *dx) {
  const int lane = lane_id();
  const int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave;
  if (t >= T) return;
  for (int o = lane * 8; o < d; o += kWave * 8) {
    float acc[8];
    const bf16x8 r = *(const bf16x8 *)(dxr + t * d + o);
#pragma unroll
    for (int i = 0; i < 8; i++) acc[i] = (float)r[i];
    if (dy) {
      const bf16x8 u = *(const bf16x8 *)(dy + t * d + o);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] += (float)u[i];
    }
    if (dxd) {
      const bf16x8 u = *(const bf16x8 *)(dxd + t * d + o);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] += (float)u[i];
    }
    for (int j = 0; j < k; j++) {
      const int s = slots[t * k + j], e = ids[t * k + j];
      if (s < 0 || s >= C || e < 0 || e >= E) continue;
      const bf16x8 u = *(const bf16x8 *)(dX + ((int64_t)e * C + s) * d + o);
#pragma unroll
      for (int i = 0; i < 8; i++) acc[i] += (float)u[i];
    }
    bf16x8 w;
#pragma unroll
    for (int i = 0; i < 8; i++) w[i] = (bf16)acc[i];
    *(bf16x8 *)(dx + t * d + o) = w;
  }
}

}  // namespace moe

namespace moe_host {
using namespace moe;

template <int BN, bool AKM, bool BKM, bool DG>
static hipError_t launch_gen_t(const GenArgs &a, const char *role, hipStream_t s) {
  const int tiles = a.G * (int)((a.M + 127) / 128) * (a.N / BN);
  if (tiles <= 0) return hipGetLastError();
  const char *name = intern_name(role, BN == 128 ? "gen128" : "gen64");
  MOE_LAUNCH(name, (gemm_gen_kernel<BN, AKM, BKM, DG>), dim3(tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

// A K-contiguous, B K-major and N a multiple of 256 (the expert and dense dZ
// and dX, the router's dx): 256-column tiles, K steps of 32, 3 stages (4 for
// 64-row tiles), two workgroups per CU -- each K row of the weight operand
// is read as 512 contiguous bytes and the activation panel is read half as
// often (measured: expert dZ 1.12 -> 0.87 ms, dense dZ / dX 0.71 / 0.62 ->
// 0.62 / 0.52 ms at the 1.3B shape; the 350M shape's 64-row dZ / dX 0.25 /
// 0.23 -> 0.22 / 0.19 ms).  Both operands K-major (the dense dW): the same
// 256-column tiles while they number at least one per CU (dense dW1 / dW2
// 0.59 / 0.58 -> 0.49 / 0.48 ms; the router's dW, 8 such tiles, stays on
// 128 columns: 0.19 vs 0.30 ms).  Otherwise 128-column tiles: K steps of 64 (3
// stages, one workgroup per CU) for a single 128-row panel with a long
// reduction (the router's dW over the tokens: streaming-bound, measured
// 14-16% faster than 32), else K steps of 32 (4 stages, two workgroups per
// CU, which the many-tile dense products need).
// NT: the B operand is streamed once (expert weights): non-temporal loads
template <bool AKM, bool BKM, bool DG, bool NT>
static hipError_t launch_dmag_t(const GenArgs &a, const char *role, hipStream_t s) {
  if constexpr (AKM && BKM) {  // 256-column tiles when they still fill the chip
    const int64_t tiles = (int64_t)a.G * (a.M / 128) * (a.N / 256);
    if (a.N % 256 == 0 && tiles >= 256) {
      MOE_LAUNCH(intern_name(role, "dma128x256"),
                 (gemm_dmag_kernel<AKM, BKM, DG, 3, 32, 128, NT, 256>), dim3((unsigned)tiles),
                 dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  if constexpr (!AKM && BKM) {  // 256-column tiles where N allows
    if (a.N % 256 == 0) {
      if (a.M <= 64) {
        const int tiles = a.G * (a.N / 256);
        if (tiles <= 0) return hipGetLastError();
        MOE_LAUNCH(intern_name(role, "dma64x256"),
                   (gemm_dmag_kernel<AKM, BKM, DG, 4, 32, 64, NT, 256>), dim3(tiles), dim3(256), 0,
                   s, a);
        return hipGetLastError();
      }
      const int tiles = a.G * (int)(a.M / 128) * (a.N / 256);
      if (tiles <= 0) return hipGetLastError();
      MOE_LAUNCH(intern_name(role, "dma128x256"),
                 (gemm_dmag_kernel<AKM, BKM, DG, 3, 32, 128, NT, 256>), dim3(tiles), dim3(256), 0,
                 s, a);
      return hipGetLastError();
    }
  }
  if constexpr (!AKM) {  // groups of at most 64 rows: 64-row tiles
    if (a.M <= 64) {
      const int tiles = a.G * (a.N / 128);
      if (tiles <= 0) return hipGetLastError();
      MOE_LAUNCH(intern_name(role, "dma64x128"), (gemm_dmag_kernel<AKM, BKM, DG, 4, 32, 64, NT>),
                 dim3(tiles), dim3(256), 0, s, a);
      return hipGetLastError();
    }
  }
  const int tiles = a.G * (int)(a.M / 128) * (a.N / 128);
  if (tiles <= 0) return hipGetLastError();
  if (a.M <= 128 && a.K >= 4096 && a.K % 64 == 0)
    MOE_LAUNCH(intern_name(role, "dma128x128k64"), (gemm_dmag_kernel<AKM, BKM, DG, 3, 64, 128, NT>),
               dim3(tiles), dim3(256), 0, s, a);
  else
    MOE_LAUNCH(intern_name(role, "dma128x128"), (gemm_dmag_kernel<AKM, BKM, DG, 4, 32, 128, NT>),
               dim3(tiles), dim3(256), 0, s, a);
  return hipGetLastError();
}

// N splits: about eight tiles per workgroup and at most ~128 workgroups per
// group (measured on MI355X: fewer, longer sweeps lose the group's operands
// from L2; shorter ones pay the A slab again per few tiles)
template <int KR>
static hipError_t launch_dwk_t(const GenArgs &a0, const char *role, hipStream_t s) {
  GenArgs a = a0;
  const int tiles_m = (int)(a.M / 128), tiles_n = a.N / 128;
  a.nsplit = 1;
  while (tiles_n % (2 * a.nsplit) == 0 && tiles_n / (2 * a.nsplit) >= 8 &&
         tiles_m * 2 * a.nsplit <= 128)
    a.nsplit *= 2;
  const int64_t blocks = (int64_t)a.G * tiles_m * a.nsplit;
  if (blocks <= 0 || a.N <= 0) return hipGetLastError();
  MOE_LAUNCH(intern_name(role, KR == 128 ? "dwk128" : (KR == 64 ? "dwk64" : "dwk32")),
             gemm_dwk_kernel<KR>, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

// the short-reduction weight-gradient kernel: both operands K-major with
// 16-byte aligned rows, M and N multiples of 128, K <= 128 rows in memory,
// 16-byte aligned output rows
static bool dwk_ok(const GenArgs &a, bool akm, bool bkm, bool dgelu) {
  if (!akm || !bkm || dgelu || a.K <= 0 || a.K > 128) return false;
  if (a.M % 128 || a.N % 128 || a.a_kmax < a.K || a.b_kmax < a.K) return false;
  if (a.a_k % 8 || a.b_k % 8 || a.c_m % 8 || a.a_g % 8 || a.b_g % 8 || a.c_g % 8) return false;
  if (a.a_k * 2 * 128 >= (int64_t(1) << 31) || a.b_k * 2 * 128 >= (int64_t(1) << 31)) return false;
  return a.G * (a.M / 128) * (a.N / 128) < (int64_t(1) << 31);
}

// the DMA kernel needs 128-multiples for M and N, K a multiple of 32, a
// whole K for K-contiguous operands, K-major extents that cover the rounded-up
// K, 16-byte aligned rows, and per-lane offsets below 2^32
// (M a multiple of 128, or at most 64 with a K-contiguous A: one 64-row tile)
static bool dmag_ok(const GenArgs &a, bool akm, bool bkm) {
  const bool m64 = !akm && a.M > 0 && a.M <= 64;
  if ((a.M % 128 && !m64) || a.N % 128 || a.K % 32 || a.K <= 0) return false;
  if ((!akm || !bkm) && a.krows) return false;
  if (akm && (a.a_kmax < a.K || a.a_k % 8)) return false;
  if (bkm && (a.b_kmax < a.K || a.b_k % 8)) return false;
  if (!akm && (a.a_m % 8 || a.a_m * 2 * 128 >= (int64_t(1) << 31))) return false;
  if (!bkm && (a.b_n % 8 || a.b_n * 2 * 128 >= (int64_t(1) << 31))) return false;
  if (akm && a.a_k * 2 * 64 >= (int64_t(1) << 31)) return false;  // k < 64 rows per step
  if (bkm && a.b_k * 2 * 64 >= (int64_t(1) << 31)) return false;
  return true;
}

// a_kmajor / b_kmajor: which operand layouts; dgelu: epilogue
hipError_t launch_gemm_gen(const GenArgs &a, bool a_kmajor, bool b_kmajor, bool dgelu,
                           const char *role, hipStream_t s) {
  if (dwk_ok(a, a_kmajor, b_kmajor, dgelu)) {
    if (a.K <= 32) return launch_dwk_t<32>(a, role, s);
    if (a.K <= 64) return launch_dwk_t<64>(a, role, s);
    return launch_dwk_t<128>(a, role, s);
  }
  if (dmag_ok(a, a_kmajor, b_kmajor)) {
    if (!a_kmajor && b_kmajor && dgelu)
      return a.b_stream ? launch_dmag_t<false, true, true, true>(a, role, s)
                        : launch_dmag_t<false, true, true, false>(a, role, s);
    if (!a_kmajor && b_kmajor)
      return a.b_stream ? launch_dmag_t<false, true, false, true>(a, role, s)
                        : launch_dmag_t<false, true, false, false>(a, role, s);
    if (a_kmajor && b_kmajor) return launch_dmag_t<true, true, false, false>(a, role, s);
  }
  const bool n128 = a.N % 128 == 0;
#define MOE_GEN(BN_)                                                                     \
  do {                                                                                   \
    if (!a_kmajor && b_kmajor && dgelu) return launch_gen_t<BN_, false, true, true>(a, role, s); \
    if (!a_kmajor && b_kmajor) return launch_gen_t<BN_, false, true, false>(a, role, s); \
    if (a_kmajor && b_kmajor) return launch_gen_t<BN_, true, true, false>(a, role, s);   \
  } while (0)
  if (n128)
    MOE_GEN(128);
  else
    MOE_GEN(64);
#undef MOE_GEN
  return hipErrorInvalidValue;
}

hipError_t launch_gelu_map(const bf16 *z, bf16 *h, int64_t n, hipStream_t s) {
  if (n <= 0) return hipGetLastError();
  int64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  MOE_LAUNCH("gelu_map", gelu_map_kernel, dim3((unsigned)blocks), dim3(256), 0, s, z, h, n);
  return hipGetLastError();
}

hipError_t launch_bwd_gate(const bf16 *dy, const bf16 *y_disp, const int32_t *ids,
                           const int32_t *slots, const float *gates, int64_t T, int k, int d,
                           int64_t C, int E, float *dg, bf16 *dY, hipStream_t s) {
  const int64_t n = T * k;
  if (n <= 0) return hipGetLastError();
  MOE_LAUNCH("bwd_gate", bwd_gate_kernel, dim3((unsigned)((n + 3) / 4)), dim3(256), 0, s, dy,
             y_disp, ids, slots, gates, n, k, d, C, E, dg, dY);
  return hipGetLastError();
}

hipError_t launch_bwd_router(const float *logits, const int32_t *ids, const float *gates,
                             const float *dg, int32_t *fcnt, int64_t T, int E, int Ep, int k,
                             int normalize, float alpha, float g_aux, float g_z, float *dlog,
                             bf16 *dlog16, float *db, hipStream_t s) {
  MOE_LAUNCH("fill_i32", fill_i32_kernel, dim3((E + 255) / 256), dim3(256), 0, s, fcnt, E, 0);
  if (T > 0) {
    int64_t blocks = (T + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    MOE_LAUNCH("first_choice", first_choice_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ids,
               T, k, E, fcnt);
    MOE_LAUNCH("bwd_router", bwd_router_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s,
               logits, ids, gates, dg, fcnt, T, E, Ep, k, normalize, alpha, g_aux, g_z, dlog,
               dlog16);
  }
  if (db) MOE_LAUNCH("colsum", colsum_kernel, dim3(E), dim3(256), 0, s, dlog, T, E, db);
  return hipGetLastError();
}

hipError_t launch_fill_i32(int32_t *p, int n, int v, hipStream_t s) {
  if (n > 0) MOE_LAUNCH("fill_i32", fill_i32_kernel, dim3((n + 255) / 256), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_bwd_dx(const bf16 *dy, const bf16 *dxd, const bf16 *dxr, const bf16 *dX,
                         const int32_t *ids, const int32_t *slots, int64_t T, int k, int d,
                         int64_t C, int E, bf16 *dx, hipStream_t s) {
  if (T <= 0) return hipGetLastError();
  MOE_LAUNCH("bwd_dx", bwd_dx_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, s, dy, dxd,
             dxr, dX, ids, slots, T, k, d, C, E, dx);
  return hipGetLastError();
}

}  // namespace moe_host
