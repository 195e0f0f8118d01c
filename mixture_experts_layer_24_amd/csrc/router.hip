// router.hip -- fused router: logits = x W_r^T (+ b), softmax, top-k gate,
// per-block load-balance statistics and per-block assignment histogram
// (both stored expert-major, [E][blocks], for the per-expert scan).
//
// Method: "DeepSpeed MoE and Model Compression", section "DeepSpeed-MoE"
// (p(x) = softmax(W_r x), TopK over p); "DeepSpeed-MoE vs Switch
// Transformer", section "router computation" (logits = x W_r, softmax);
// survey notes sec. 1.1.1.1 (renormalise after TopK) and sec. 1.1.4.1
// (f_i, Q_i of the Switch load-balance loss); "DeepSpeed-MoE ... notes" sec.
// 4.4 (top-k fused with the counting that feeds the cumsum mapping table).
//
// One block = 64 tokens x all experts (E <= 256, padded to a multiple of 32).
// bf16: the 64 x Ep logit tile is a bf16 MFMA contraction (32x32x16, fp32
// accumulate; the bf16 products are exact in fp32) over d in 64-wide K steps
// whose operand tiles move global -> LDS by DMA three steps ahead
// (router_dma_kernel); the register-staged router_bf16_kernel serves the
// raw products of two weight matrices (noisy TopK).  fp32: plain fp32 FMA
// dot products.  The epilogue is shared: the tile goes to LDS, each wave
// takes 16 rows; a row's E logits sit 1-4 per lane (one slot per 64
// experts); wave reductions (DPP within 16-lane rows, then the four row
// totals) give the row max and the softmax sum, and each top-k round takes
// the largest remaining logit and the lowest expert holding it by a ballot.
#include "common.h"
#include "dma.h"
#include "kernels.h"

namespace moe {

constexpr int RBM = 64;  // tokens per block


// L: LDS logits tile [RBM][ldl] fp32 (bias not yet added).  SL = expert
// slots per lane (E <= 64 SL): lane l holds experts l, l + 64, ...  NWV
// waves, RBM / NWV token rows each; per-wave partials summed in wave order.
template <int MAXK, int SL, int NWV = 4>
__device__ void router_epilogue(const RouterArgs &a, const float *L, int ldl,
                                float (*qpart)[256], int *fcnt, int *hcnt, int blk) {
  static_assert(RBM % NWV == 0, "rows per wave");
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int E = a.E, k = a.k;
  __shared__ float zw[NWV];
  float q[SL];
  float zacc = 0.f;
  float bias[SL];
#pragma unroll
  for (int i = 0; i < SL; i++) {
    q[i] = 0.f;
    const int e = lane + kWave * i;
    bias[i] = (a.bias && e < E) ? a.bias[e] : 0.f;
  }
  for (int rr = 0; rr < RBM / NWV; rr++) {
    // 4 waves: 16 consecutive rows each; more waves: rows dealt round-robin,
    // so a partly filled block (decode) still keeps every wave busy
    const int r = NWV == 4 ? wave * (RBM / 4) + rr : rr * NWV + wave;
    const int64_t t = (int64_t)blk * RBM + r;
    if (t >= a.T) break;
    float v[SL];
    bool live[SL];
#pragma unroll
    for (int i = 0; i < SL; i++) {
      const int e = lane + kWave * i;
      live[i] = e < E;
      v[i] = live[i] ? L[r * ldl + e] + bias[i] : neg_inf();
      if (a.logits && live[i]) a.logits[t * E + e] = v[i];
    }
    float m = v[0];
#pragma unroll
    for (int i = 1; i < SL; i++) m = fmaxf(m, v[i]);
    m = wave_max(m);
    float p[SL], s = 0.f;
#pragma unroll
    for (int i = 0; i < SL; i++) {
      p[i] = live[i] ? expf(v[i] - m) : 0.f;
      s += p[i];
    }
    s = wave_sum(s);
    if (a.zpart) {  // z-loss term: (log sum_e exp v_e)^2 = (m + log s)^2
      const float lz = m + logf(s);
      zacc += lz * lz;
    }
#pragma unroll
    for (int i = 0; i < SL; i++) {
      p[i] = p[i] / s;
      q[i] += p[i];
    }
    // top-k: round j takes the largest logit not yet taken (the softmax max m
    // in round 0) and the lowest expert holding it, from one ballot per slot
    // (slot i holds experts 64 i .. 64 i + 63, so the first hit is the lowest)
    bool taken[SL];
#pragma unroll
    for (int i = 0; i < SL; i++) taken[i] = false;
    int sel[MAXK];
    float selp[MAXK];
#pragma unroll
    for (int j = 0; j < MAXK; j++) {
      sel[j] = 0;
      selp[j] = 0.f;
      if (j < k) {
        float mj = m;
        if (j > 0) {
          float c = neg_inf();
#pragma unroll
          for (int i = 0; i < SL; i++)
            if (live[i] && !taken[i]) c = fmaxf(c, v[i]);
          mj = wave_max(c);
        }
        int be = -1;
#pragma unroll
        for (int i = 0; i < SL; i++) {
          const unsigned long long b = __ballot(live[i] && !taken[i] && v[i] == mj);
          if (be < 0 && b) be = kWave * i + __builtin_ctzll(b);
        }
        if (be < 0) {  // only NaN logits left: the lowest expert not taken
#pragma unroll
          for (int i = 0; i < SL; i++) {
            const unsigned long long b = __ballot(live[i] && !taken[i]);
            if (be < 0 && b) be = kWave * i + __builtin_ctzll(b);
          }
        }
        const int owner_i = be / kWave;
        float pi = p[0];
#pragma unroll
        for (int i = 1; i < SL; i++)
          if (owner_i == i) pi = p[i];
        selp[j] = lane_f(pi, be % kWave);  // be is wave-uniform
        sel[j] = be;
#pragma unroll
        for (int i = 0; i < SL; i++)
          if (lane + kWave * i == be) taken[i] = true;
      }
    }
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < MAXK; j++)
      if (j < k) den += selp[j];
    const bool renorm = (k >= 2) && a.normalize;
    // lane j writes choice j
    int my_e = 0;
    float my_p = 0.f;
#pragma unroll
    for (int j = 0; j < MAXK; j++)
      if (lane == j) {
        my_e = sel[j];
        my_p = selp[j];
      }
    if (lane < k) {
      a.ids[t * k + lane] = my_e;
      a.gates[t * k + lane] = renorm ? my_p / den : my_p;
      atomicAdd(&hcnt[my_e], 1);
      if (lane == 0) atomicAdd(&fcnt[my_e], 1);
    }
  }
#pragma unroll
  for (int i = 0; i < SL; i++) {
    const int e = lane + kWave * i;
    if (e < E) qpart[wave][e] = q[i];
  }
  if (lane == 0) zw[wave] = zacc;
  __syncthreads();
  if (a.zpart && threadIdx.x == 0) {
    float z = zw[0];
#pragma unroll
    for (int w = 1; w < NWV; w++) z += zw[w];
    a.zpart[blk] = z;
  }
  const int e = threadIdx.x;
  if (e < E) {
    const int64_t o = (int64_t)e * gridDim.x + blk;  // expert-major [E][nblk]
    float q = qpart[0][e];
#pragma unroll
    for (int w = 1; w < NWV; w++) q += qpart[w][e];
    a.qsum[o] = q;
    a.fcount[o] = fcnt[e];
    if (a.hist) a.hist[o] = hcnt[e];
  }
}

// NTW = 32-wide expert tiles per wave (Ep <= 64 * NTW).  BK = K step (64,
// or 128 when d allows it and the two stages fit LDS, i.e. Ep <= 128).
// SCORES: only the raw fp32 product tile is written, to a.logits with row
// stride E (the router variants' first step); rows e >= a.nw1 of the product
// come from a.w2 (row e - a.nw1), so two weight matrices act as one.
template <int NTW, int BK, bool SCORES = false>
__global__ __launch_bounds__(256) void router_bf16_kernel(RouterArgs a) {
  constexpr int EPMAX = 64 * NTW;
  static_assert(BK == 64 || (BK == 128 && NTW <= 2), "router tile does not fit LDS");
  constexpr int LDA = BK + 8;                   // bf16 elements per LDS row
  constexpr int CPR = BK / 8;                   // 16-byte chunks per row
  constexpr int RPP = 256 / CPR;                // rows per load pass
  constexpr int XP = RBM / RPP;                 // x passes
  constexpr int WP = EPMAX / RPP;               // W passes (at most)
  constexpr int STAGE = (RBM + EPMAX) * LDA;    // bf16 elements per stage
  constexpr int TILE_BYTES = 2 * STAGE * 2;
  constexpr int LOGIT_BYTES = RBM * (EPMAX + 4) * 4;
  constexpr int SMEM = TILE_BYTES > LOGIT_BYTES ? TILE_BYTES : LOGIT_BYTES;
  __shared__ __attribute__((aligned(16))) char smem[SMEM];
  __shared__ float qpart[4][256];
  __shared__ int fcnt[256], hcnt[256];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int blk = blockIdx.x;
  const int E = a.E, Ep = (E + 31) & ~31, d = a.d;
  fcnt[tid] = 0;
  hcnt[tid] = 0;
  bf16 *As = (bf16 *)smem;
  const bf16 *X = (const bf16 *)a.x;
  const bf16 *W = (const bf16 *)a.w;

  // global -> register prefetch of the next K step
  const int crow = tid / CPR, cchk = tid % CPR;
  u32x4 ra[XP], rw[WP];
  auto load_tiles = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int p = 0; p < XP; p++) {
      int64_t t = (int64_t)blk * RBM + p * RPP + crow;
      if (t >= a.T) t = a.T - 1;
      ra[p] = *(const u32x4 *)(X + t * d + k0 + cchk * 8);
    }
#pragma unroll
    for (int p = 0; p < WP; p++) {
      int e = p * RPP + crow;
      if (p * RPP < Ep) {
        if (e >= E) e = E - 1;
        if constexpr (SCORES) {
          const bf16 *Wr = e < a.nw1 ? W + (int64_t)e * d : (const bf16 *)a.w2 + (int64_t)(e - a.nw1) * d;
          rw[p] = *(const u32x4 *)(Wr + k0 + cchk * 8);
        } else {
          rw[p] = *(const u32x4 *)(W + (int64_t)e * d + k0 + cchk * 8);
        }
      }
    }
  };
  auto store_tiles = [&](int st) __attribute__((always_inline)) {
    bf16 *sa = As + st * STAGE;
    bf16 *sw = sa + RBM * LDA;
#pragma unroll
    for (int p = 0; p < XP; p++) *(u32x4 *)(sa + (p * RPP + crow) * LDA + cchk * 8) = ra[p];
#pragma unroll
    for (int p = 0; p < WP; p++)
      if (p * RPP < Ep) *(u32x4 *)(sw + (p * RPP + crow) * LDA + cchk * 8) = rw[p];
  };

  f32x16 acc[NTW];
#pragma unroll
  for (int i = 0; i < NTW; i++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[i][r] = 0.f;

  const int mt = wave & 1;  // 32-row half of the token tile
  const int ksteps = d / BK;
  load_tiles(0);
  store_tiles(0);
  __syncthreads();
  for (int kt = 0; kt < ksteps; kt++) {
    const int st = kt & 1;
    if (kt + 1 < ksteps) load_tiles((kt + 1) * BK);
    const bf16 *sa = As + st * STAGE;
    const bf16 *sw = sa + RBM * LDA;
    // branch-free as in router_dma_kernel: tiles past Ep are never stored
#pragma unroll
    for (int s = 0; s < BK / 16; s++) {
      const int ch = 2 * s + (lane >> 5);
      bf16x8 av = *(const bf16x8 *)(sa + (mt * 32 + (lane & 31)) * LDA + ch * 8);
#pragma unroll
      for (int i = 0; i < NTW; i++) {
        const int nt = (wave >> 1) + 2 * i;
        bf16x8 bv = *(const bf16x8 *)(sw + (nt * 32 + (lane & 31)) * LDA + ch * 8);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[i], 0, 0, 0);
      }
    }
    if (kt + 1 < ksteps) store_tiles(st ^ 1);
    __syncthreads();
  }
  // accumulators -> LDS logits tile
  float *L = (float *)smem;
  const int ldl = EPMAX + 4;
#pragma unroll
  for (int i = 0; i < NTW; i++) {
    const int nt = (wave >> 1) + 2 * i;
    if (nt * 32 < Ep) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        L[m * ldl + nt * 32 + (lane & 31)] = acc[i][r];
      }
    }
  }
  __syncthreads();
  if constexpr (SCORES) {
    for (int idx = tid; idx < RBM * E; idx += 256) {
      const int r = idx / E, e = idx - (idx / E) * E;
      const int64_t t = (int64_t)blk * RBM + r;
      if (t < a.T) a.logits[t * E + e] = L[r * ldl + e];
    }
    return;
  }
  if (a.k <= 2)
    router_epilogue<2, NTW>(a, L, ldl, qpart, fcnt, hcnt, blk);
  else
    router_epilogue<8, NTW>(a, L, ldl, qpart, fcnt, hcnt, blk);
}

// The same contraction with the operand tiles moved global -> LDS by DMA in
// 64-wide K steps, NS - 1 steps ahead (the router's blocks each read the
// whole weight matrix, so the stream of K steps must keep several steps in
// flight; the register-staged kernel above keeps one).  Tile rows are 128
// bytes with the 16-byte chunks XOR-swizzled as in the GEMMs.  The K order
// of the MFMAs is that of router_bf16_kernel: identical logits.  One weight
// matrix (SCORES with two matrices uses router_bf16_kernel).
template <int NTW, int NS, bool SCORES = false, int NWR = 4>
__global__ __launch_bounds__(64 * NWR) void router_dma_kernel(RouterArgs a) {
  static_assert(NWR == 4 || NWR == 8, "waves");
  constexpr int EPMAX = 64 * NTW;
  constexpr int NT = 2 * NTW;                       // 32-wide expert tiles
  constexpr int TPW = (NT + NWR / 2 - 1) / (NWR / 2);  // expert tiles per wave
  constexpr int ROWB = 128;                         // bytes per tile row (64 bf16)
  constexpr int STAGE = (RBM + EPMAX) * ROWB;
  constexpr int A_PW = RBM * ROWB / 1024 / NWR;     // 1 KB chunks per wave per stage
  constexpr int W_PW = EPMAX * ROWB / 1024 / NWR;
  constexpr int CPW = A_PW + W_PW;
  static_assert(A_PW * NWR * 1024 == RBM * ROWB && W_PW * NWR * 1024 == EPMAX * ROWB, "chunks");
  constexpr int LOGIT_BYTES = RBM * (EPMAX + 4) * 4;
  constexpr int SMEM = NS * STAGE > LOGIT_BYTES ? NS * STAGE : LOGIT_BYTES;
  static_assert(NS >= 2 && (NS - 2) * CPW < 64, "vmcnt range");
  __shared__ __attribute__((aligned(1024))) char smem[SMEM];
  __shared__ float qpart[NWR][256];
  __shared__ int fcnt[256], hcnt[256];

  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int blk = blockIdx.x;
  const int E = a.E, Ep = (E + 31) & ~31, d = a.d;
  if (tid < 256) {
    fcnt[tid] = 0;
    hcnt[tid] = 0;
  }
  const int64_t t0 = (int64_t)blk * RBM;
  const char *Xb = (const char *)a.x + t0 * d * 2;
  const char *Wb = (const char *)a.w;
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) char *)smem;
  // chunk = 8 rows of 128 bytes; lane -> row lane / 8, slot lane % 8
  const int lr = lane / 8, slot = lane % 8;
  uint32_t voffa[A_PW], voffw[W_PW];
#pragma unroll
  for (int i = 0; i < A_PW; i++) {
    const int R = 8 * (wave * A_PW + i) + lr;
    int64_t r = R;
    if (t0 + r >= a.T) r = a.T - 1 - t0;  // clamp to the last token
    voffa[i] = (uint32_t)(r * d * 2 + ((slot ^ swz_slot<64>(R)) << 4));
  }
#pragma unroll
  for (int i = 0; i < W_PW; i++) {
    const int R = 8 * (wave * W_PW + i) + lr;
    const int e = R < E ? R : E - 1;      // clamp to the last expert
    voffw[i] = (uint32_t)((int64_t)e * d * 2 + ((slot ^ swz_slot<64>(R)) << 4));
  }
  const uint32_t dsta = lds0 + wave * A_PW * 1024;
  const uint32_t dstw = lds0 + RBM * ROWB + wave * W_PW * 1024;
  auto issue = [&](int st, int kt) __attribute__((always_inline)) {
    const char *ga = Xb + (int64_t)kt * ROWB;
    const char *gw = Wb + (int64_t)kt * ROWB;
#pragma unroll
    for (int i = 0; i < A_PW; i++)
      dma16<false>(ga, voffa[i], __builtin_amdgcn_readfirstlane(dsta + st * STAGE + i * 1024));
#pragma unroll
    for (int i = 0; i < W_PW; i++)
      dma16<false>(gw, voffw[i], __builtin_amdgcn_readfirstlane(dstw + st * STAGE + i * 1024));
  };

  f32x16 acc[TPW];
#pragma unroll
  for (int i = 0; i < TPW; i++)
#pragma unroll
    for (int r = 0; r < 16; r++) acc[i][r] = 0.f;
  // expert tile i of this wave (clamped to the last tile: a wave with fewer
  // tiles than TPW multiplies a copy and never stores it)
  auto tile_of = [&](int i) __attribute__((always_inline)) {
    const int nt = (wave >> 1) + (NWR / 2) * i;
    return nt < NT ? nt : NT - 1;
  };

  const int mt = wave & 1;  // 32-row half of the token tile
  // K range of this block: all of d, or (split K, gridDim.y > 1) its share
  const int kall = d / 64, ns = gridDim.y;
  const int kbeg = (int)((int64_t)blockIdx.y * kall / ns);
  const int ksteps = (int)((int64_t)(blockIdx.y + 1) * kall / ns) - kbeg;
  auto kidx = [&](int kt) __attribute__((always_inline)) { return kbeg + kt; };
#pragma unroll
  for (int p = 0; p < NS - 1; p++)
    if (p < ksteps) issue(p, kidx(p));
  for (int kt = 0; kt < ksteps; kt++) {
    if (kt + NS - 2 < ksteps)
      wait_vmcnt<(NS - 2) * CPW>();
    else
      wait_vmcnt<0>();
    __syncthreads();  // every wave's chunks of step kt; stage (kt - 1) % NS free
    if (kt + NS - 1 < ksteps) issue((kt + NS - 1) % NS, kidx(kt + NS - 1));
    const char *sa = smem + (kt % NS) * STAGE;
    const char *sw = sa + RBM * ROWB;
    // every wave runs all NTW expert tiles (tiles past Ep multiply the
    // clamped weight rows and are never stored), so the loop has no branch
    // and the accumulators stay in place across the MFMAs
#pragma unroll
    for (int s = 0; s < 4; s++) {
      const int c = 2 * s + (lane >> 5);
      const int Ra = mt * 32 + (lane & 31);
      const bf16x8 av = *(const bf16x8 *)(sa + Ra * ROWB + ((c ^ swz_slot<64>(Ra)) << 4));
#pragma unroll
      for (int i = 0; i < TPW; i++) {
        const int Rw = tile_of(i) * 32 + (lane & 31);
        const bf16x8 bv = *(const bf16x8 *)(sw + Rw * ROWB + ((c ^ swz_slot<64>(Rw)) << 4));
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[i], 0, 0, 0);
      }
    }
  }
  __syncthreads();  // the stages are read; the logits tile reuses them
  float *L = (float *)smem;
  const int ldl = EPMAX + 4;
#pragma unroll
  for (int i = 0; i < TPW; i++) {
    const int nt = (wave >> 1) + (NWR / 2) * i;
    if (nt < NT && nt * 32 < Ep) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int m = mt * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        L[m * ldl + nt * 32 + (lane & 31)] = acc[i][r];
      }
    }
  }
  __syncthreads();
  if constexpr (SCORES) {
    // split K: partial products of K range blockIdx.y in slab blockIdx.y of
    // a.part ([splits][blocks * 64][Ep], every row and column written; the
    // columns past E hold products of the clamped weight row)
    if (ns > 1) {
      float *P = a.part + ((int64_t)blockIdx.y * gridDim.x * RBM + t0) * Ep;
      for (int idx = tid; idx < RBM * Ep / 4; idx += 64 * NWR) {
        const int r = idx / (Ep / 4), e = 4 * (idx - r * (Ep / 4));
        *(f32x4 *)(P + (int64_t)r * Ep + e) = *(const f32x4 *)(L + r * ldl + e);
      }
      return;
    }
    for (int idx = tid; idx < RBM * E; idx += 64 * NWR) {
      const int r = idx / E, e = idx - (idx / E) * E;
      const int64_t t = t0 + r;
      if (t < a.T) a.logits[t * E + e] = L[r * ldl + e];
    }
    return;
  }
  if (a.k <= 2)
    router_epilogue<2, NTW, NWR>(a, L, ldl, qpart, fcnt, hcnt, blk);
  else
    router_epilogue<8, NTW, NWR>(a, L, ldl, qpart, fcnt, hcnt, blk);
}

// Split-K router, second step (one block of 16 waves per 64-token block):
// the partial products of the splits summed in split order (fixed) into an
// LDS logits tile, 4 columns per thread with the loads of every split in
// flight together (nsplit <= kMaxSplit), then the softmax / top-k epilogue
// of the fused router on it, 4 token rows per wave.
constexpr int kMaxSplit = 16;
template <int MAXK, int SL>
__global__ __launch_bounds__(1024) void router_split_epi_kernel(RouterArgs a, int nsplit) {
  constexpr int NWV = 16, LDL = 64 * SL + 4;
  __shared__ __attribute__((aligned(16))) float L[RBM * LDL];
  __shared__ float qpart[NWV][256];
  __shared__ int fcnt[256], hcnt[256];
  const int tid = threadIdx.x, blk = blockIdx.x;
  const int Ep = (a.E + 31) & ~31;
  if (tid < 256) {
    fcnt[tid] = 0;
    hcnt[tid] = 0;
  }
  const int64_t slab = (int64_t)gridDim.x * RBM * Ep;
  const float *P = a.part + (int64_t)blk * RBM * Ep;
  const int64_t left = a.T - (int64_t)blk * RBM;  // rows past T are never read
  const int nrow = left < RBM ? (int)left : RBM;
  for (int idx = tid; idx < nrow * Ep / 4; idx += 64 * NWV) {
    const int r = idx / (Ep / 4), e = 4 * (idx - r * (Ep / 4));
    f32x4 v[kMaxSplit];
#pragma unroll
    for (int sp = 0; sp < kMaxSplit; sp++)
      if (sp < nsplit) v[sp] = *(const f32x4 *)(P + sp * slab + (int64_t)r * Ep + e);
    f32x4 acc = v[0];
#pragma unroll
    for (int sp = 1; sp < kMaxSplit; sp++)
      if (sp < nsplit) acc += v[sp];
    *(f32x4 *)(L + r * LDL + e) = acc;
  }
  __syncthreads();
  router_epilogue<MAXK, SL, NWV>(a, L, LDL, qpart, fcnt, hcnt, blk);
}

// fp32 activations: plain fp32 dot products (small shapes; correctness path)
template <bool SCORES = false>
__global__ __launch_bounds__(256) void router_f32_kernel(RouterArgs a) {
  __shared__ float L[RBM * 260];
  __shared__ float qpart[4][256];
  __shared__ int fcnt[256], hcnt[256];
  const int tid = threadIdx.x, blk = blockIdx.x;
  const int E = a.E, d = a.d, ldl = 260;
  fcnt[tid] = 0;
  hcnt[tid] = 0;
  const float *X = (const float *)a.x, *W = (const float *)a.w;
  for (int idx = tid; idx < RBM * E; idx += 256) {
    const int r = idx / E, e = idx % E;
    const int64_t t = (int64_t)blk * RBM + r;
    float s = 0.f;
    const float *Wr = W + (int64_t)e * d;
    if (SCORES && e >= a.nw1) Wr = (const float *)a.w2 + (int64_t)(e - a.nw1) * d;
    if (t < a.T)
      for (int i = 0; i < d; i++) s = fmaf(X[t * d + i], Wr[i], s);
    L[r * ldl + e] = s;
  }
  __syncthreads();
  if constexpr (SCORES) {
    for (int idx = tid; idx < RBM * E; idx += 256) {
      const int r = idx / E, e = idx - (idx / E) * E;
      const int64_t t = (int64_t)blk * RBM + r;
      if (t < a.T) a.logits[t * E + e] = L[r * ldl + e];
    }
    return;
  }
  if (a.k <= 2)
    router_epilogue<2, 4>(a, L, ldl, qpart, fcnt, hcnt, blk);
  else
    router_epilogue<8, 4>(a, L, ldl, qpart, fcnt, hcnt, blk);
}

// Switch load-balance loss, final step (moe_route): see aux_sum_wave.
__global__ __launch_bounds__(64) void aux_sum_kernel(const double *term, int E, float alpha,
                                                     float *aux) {
  aux_sum_wave(term, E, alpha, aux);
}

// Router z-loss, final step: the mean over tokens of the per-block sums,
// added in fp64 in a fixed order (contiguous chunks, then a tree).
__global__ __launch_bounds__(256) void zloss_sum_kernel(const float *zpart, int nblk, int64_t T,
                                                        float *z) {
  __shared__ double red[256];
  const int tid = threadIdx.x;
  const int chunk = (nblk + 255) / 256;
  const int b0 = tid * chunk, b1 = min(b0 + chunk, nblk);
  double v = 0.0;
  for (int b = b0; b < b1; b++) v += (double)zpart[b];
  red[tid] = v;
  __syncthreads();
  for (int st = 128; st >= 1; st >>= 1) {
    if (tid < st) red[tid] += red[tid + st];
    __syncthreads();
  }
  if (tid == 0) z[0] = T > 0 ? (float)(red[0] / (double)T) : 0.f;
}

}  // namespace moe

namespace moe_host {
using namespace moe;

int router_blocks(int64_t T) { return (int)((T + RBM - 1) / RBM); }

// K splits of the bf16 router: a batch of few 64-token blocks (decode) would
// leave most CUs idle and one block's K sweep on the critical path, so its K
// range is split over up to 16 blocks per token block, at least 4 K steps
// each; 1 = no split.
int router_splits(int64_t T, int d, int act_bf16) {
  const int nblk = router_blocks(T), ksteps = d / 64;
  if (!act_bf16 || nblk <= 0 || nblk > 16) return 1;
  int s = ksteps / 4;
  if (s > kMaxSplit) s = kMaxSplit;
  if (s * nblk > 64) s = 64 / nblk;
  return s < 2 ? 1 : s;
}

hipError_t launch_zloss_sum(const float *zpart, int nblk, int64_t T, float *z, hipStream_t s) {
  MOE_LAUNCH("zloss_sum", zloss_sum_kernel, dim3(1), dim3(256), 0, s, zpart, nblk, T, z);
  return hipGetLastError();
}

hipError_t launch_router(const RouterArgs &a, int act_bf16, hipStream_t s) {
  const int nblk = router_blocks(a.T);
  const int nsplit = a.part ? router_splits(a.T, a.d, act_bf16) : 1;
  if (nblk > 0 && nsplit > 1) {  // split K: partial products, their sums, the epilogue
    const int ntw = ((a.E + 31) / 32 + 1) / 2, Ep = (a.E + 31) & ~31;
    const dim3 g(nblk, nsplit), b(256);
    switch (ntw) {
      case 1: MOE_LAUNCH("router_split_e64", (router_dma_kernel<1, 4, true>), g, b, 0, s, a); break;
      case 2: MOE_LAUNCH("router_split_e128", (router_dma_kernel<2, 4, true>), g, b, 0, s, a); break;
      case 3: MOE_LAUNCH("router_split_e192", (router_dma_kernel<3, 4, true>), g, b, 0, s, a); break;
      default: MOE_LAUNCH("router_split_e256", (router_dma_kernel<4, 3, true>), g, b, 0, s, a); break;
    }
    (void)Ep;
    const dim3 ge(nblk), be(1024);
#define MOE_SPLIT_EPI(SL)                                                                  \
  if (a.k <= 2)                                                                            \
    MOE_LAUNCH("router_split_epi", (router_split_epi_kernel<2, SL>), ge, be, 0, s, a, nsplit); \
  else                                                                                     \
    MOE_LAUNCH("router_split_epi", (router_split_epi_kernel<8, SL>), ge, be, 0, s, a, nsplit);
    switch (ntw) {
      case 1: MOE_SPLIT_EPI(1) break;
      case 2: MOE_SPLIT_EPI(2) break;
      case 3: MOE_SPLIT_EPI(3) break;
      default: MOE_SPLIT_EPI(4) break;
    }
#undef MOE_SPLIT_EPI
    return hipGetLastError();
  }
  if (nblk > 0) {
    if (act_bf16) {  // the bf16 path guarantees d % 64 == 0
      const int ntw = ((a.E + 31) / 32 + 1) / 2;
      const dim3 g(nblk), b(512);
      switch (ntw) {
        case 1:  // E <= 64: four waves (half of eight would only repeat tiles)
          MOE_LAUNCH("router_bf16_e64", (router_dma_kernel<1, 4>), g, dim3(256), 0, s, a);
          break;
        case 2: MOE_LAUNCH("router_bf16_e128", (router_dma_kernel<2, 4, false, 8>), g, b, 0, s, a); break;
        case 3: MOE_LAUNCH("router_bf16_e192", (router_dma_kernel<3, 4, false, 8>), g, b, 0, s, a); break;
        default: MOE_LAUNCH("router_bf16_e256", (router_dma_kernel<4, 3, false, 8>), g, b, 0, s, a); break;
      }
    } else {
      MOE_LAUNCH("router_f32", router_f32_kernel<false>, dim3(nblk), dim3(256), 0, s, a);
    }
  }
  return hipGetLastError();
}

// raw fp32 products [T, a.E] of x with the a.E weight rows (a.w, then a.w2
// from row a.nw1) into a.logits: the first step of the router variants
hipError_t launch_router_scores(const RouterArgs &a, int act_bf16, hipStream_t s) {
  const int nblk = router_blocks(a.T);
  if (nblk <= 0) return hipGetLastError();
  const dim3 g(nblk), b(256);
  if (!act_bf16) {
    MOE_LAUNCH("router_scores_f32", router_f32_kernel<true>, g, b, 0, s, a);
    return hipGetLastError();
  }
  const int ntw = ((a.E + 31) / 32 + 1) / 2;
  if (!a.w2 || a.nw1 >= a.E) {  // one weight matrix: the DMA pipeline
    switch (ntw) {
      case 1: MOE_LAUNCH("router_scores_n64", (router_dma_kernel<1, 4, true>), g, b, 0, s, a); break;
      case 2: MOE_LAUNCH("router_scores_n128", (router_dma_kernel<2, 4, true>), g, b, 0, s, a); break;
      case 3: MOE_LAUNCH("router_scores_n192", (router_dma_kernel<3, 4, true>), g, b, 0, s, a); break;
      default: MOE_LAUNCH("router_scores_n256", (router_dma_kernel<4, 3, true>), g, b, 0, s, a); break;
    }
    return hipGetLastError();
  }
  const bool k128 = a.d % 128 == 0;
  switch (ntw) {
    case 1:
      if (k128) MOE_LAUNCH("router_scores_n64", (router_bf16_kernel<1, 128, true>), g, b, 0, s, a);
      else MOE_LAUNCH("router_scores_n64", (router_bf16_kernel<1, 64, true>), g, b, 0, s, a);
      break;
    case 2:
      if (k128) MOE_LAUNCH("router_scores_n128", (router_bf16_kernel<2, 128, true>), g, b, 0, s, a);
      else MOE_LAUNCH("router_scores_n128", (router_bf16_kernel<2, 64, true>), g, b, 0, s, a);
      break;
    case 3: MOE_LAUNCH("router_scores_n192", (router_bf16_kernel<3, 64, true>), g, b, 0, s, a); break;
    default: MOE_LAUNCH("router_scores_n256", (router_bf16_kernel<4, 64, true>), g, b, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_aux_sum(const double *term, int E, float alpha, float *aux, hipStream_t s) {
  MOE_LAUNCH("aux_sum", aux_sum_kernel, dim3(1), dim3(64), 0, s, term, E, alpha, aux);
  return hipGetLastError();
}

}  // namespace moe_host
