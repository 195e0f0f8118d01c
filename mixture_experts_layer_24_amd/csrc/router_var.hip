// router_var.hip -- router variants of the MoE survey notes:
//   TopP selection (sec. 1.1.4.2: experts in descending score, accumulated
//     until the sum exceeds P),
//   the cosine router (sec. 1.1.1.2: a learnable projection of the token
//     against each expert's embedding, cosine similarity over a temperature),
//   noisy TopK gating (sec. 1.1.1.1: a linear gate plus a noise term that
//     encourages exploration; TopK before the softmax),
//   and the Importance / Load losses (sec. 1.1.4.1: w * CoV^2 of the
//     per-expert sum of gates, and of the per-expert probability of a nonzero
//     gate under a new draw of the noise).
// The products x W^T come from the router GEMM in raw-score mode (router.hip);
// the kernels here form the variant's logits, select, and write the same
// outputs and per-block statistics as the fused router ([E][blocks]
// expert-major), so dispatch, the Switch aux loss and the z-loss are shared.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int VBT = 64;  // tokens per block, as the fused router
constexpr int VW = 16;   // waves per block of the variant epilogue (4 tokens each)

__device__ __forceinline__ float softplus_f(float z) {
  return z > 0.f ? z + log1pf(expf(-z)) : log1pf(expf(z));
}

// standard normal distribution function
__device__ __forceinline__ float phi_cdf(float z) { return 0.5f * erfcf(-z * 0.70710678118654752f); }

// One wave per token row (VBT / VW rows per wave), a lane holding experts
// lane + 64 i.  Logits: TopK / TopP: products + bias; cosine: the cosine
// logits + bias; noisy: clean = products[e] + bias, sigma = softplus(
// products[E + e]), logit = clean + noise * sigma.  Selection by repeated
// wave arg-max (larger logit, then lower index); TopP stops once the
// accumulated probability exceeds P; unused slots get id -1, gate 0.
// Gates: noisy: softmax over the kept logits (= p renormalised over the k);
// TopP: renormalised over the taken ones when `normalize`; TopK / cosine:
// renormalised for k >= 2 when `normalize`.  Load probability: noisy:
// Phi((clean_e - thr_e) / sigma_e), thr_e = the k-th largest logit among the
// other experts (the (k+1)-th overall when e is kept, the k-th otherwise);
// otherwise 1 for a taken expert, 0 else.  No float atomics: every per-expert
// sum is owned by one lane and summed over the waves in a fixed order.
// SL expert slots per lane (E <= 64 SL); VAR: RV_TOPK (also the cosine
// router, whose logits come precomputed), RV_TOP_P or RV_NOISY.  Rows are
// dealt round-robin over the waves, so a partly filled block keeps every
// wave busy.
template <int MAXK, int SL, int VAR>
__global__ __launch_bounds__(64 * VW) void route_logits_kernel(RouteVarArgs a) {
  __shared__ float qpart[VW][256], ipart[VW][256], lpart[VW][256];
  __shared__ int fcnt[256], hcnt[256];
  __shared__ float zw[VW];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave, blk = blockIdx.x;
  const int E = a.E, k = a.k;
  constexpr bool noisy = VAR == RV_NOISY, topp = VAR == RV_TOP_P;
  const int ns = noisy ? 2 * E : E;  // row stride of the scores
  if (tid < 256) {
    fcnt[tid] = 0;
    hcnt[tid] = 0;
  }
  __syncthreads();
  float q[SL], imp[SL], ld[SL];
  float zacc = 0.f, bias[SL];
#pragma unroll
  for (int i = 0; i < SL; i++) {
    const int e = lane + kWave * i;
    q[i] = imp[i] = ld[i] = 0.f;
    bias[i] = (a.bias && e < E) ? a.bias[e] : 0.f;
  }
  const bool renorm = noisy ? true : (topp ? a.normalize != 0 : (k >= 2 && a.normalize));
  // the wave's rows of scores (and noise) are loaded before the first row is
  // worked on, so their latencies overlap
  constexpr int RPW = VBT / VW;
  float src0[RPW][SL], src1[RPW][SL], nz[RPW][SL];
#pragma unroll
  for (int rr = 0; rr < RPW; rr++) {
    const int64_t t = (int64_t)blk * VBT + rr * VW + wave;
#pragma unroll
    for (int i = 0; i < SL; i++) {
      const int e = lane + kWave * i;
      src0[rr][i] = src1[rr][i] = nz[rr][i] = 0.f;
      if (t < a.T && e < E) {
        src0[rr][i] = a.src[t * ns + e];
        if (noisy) {
          src1[rr][i] = a.src[t * ns + E + e];
          nz[rr][i] = a.noise[t * E + e];
        }
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < RPW; rr++) {
    const int r = rr * VW + wave;
    const int64_t t = (int64_t)blk * VBT + r;
    if (t >= a.T) break;
    float v[SL], clean[SL], sig[SL];
    bool live[SL];
#pragma unroll
    for (int i = 0; i < SL; i++) {
      const int e = lane + kWave * i;
      live[i] = e < E;
      clean[i] = 0.f;
      sig[i] = 0.f;
      v[i] = neg_inf();
      if (live[i]) {
        clean[i] = src0[rr][i] + bias[i];
        v[i] = clean[i];
        if (noisy) {
          sig[i] = softplus_f(src1[rr][i]);
          v[i] = clean[i] + nz[rr][i] * sig[i];
        }
        if (a.logits) a.logits[t * E + e] = v[i];
      }
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
    if (a.zpart) {
      const float lz = m + logf(s);
      zacc += lz * lz;
    }
#pragma unroll
    for (int i = 0; i < SL; i++) {
      p[i] = p[i] / s;
      q[i] += p[i];
    }
    bool taken[SL];
#pragma unroll
    for (int i = 0; i < SL; i++) taken[i] = false;
    int sel[MAXK];
    float selp[MAXK], thr_out = neg_inf();
    int n = 0;
    float cum = 0.f;
    bool stop = false;
    // MAXK choices, then (noisy) one more round for the (k+1)-th largest logit
    float thr_in = neg_inf();
#pragma unroll
    for (int j = 0; j <= MAXK; j++) {
      if (j < MAXK) {
        sel[j] = -1;
        selp[j] = 0.f;
      }
      const bool pick = j < MAXK && j < k && !stop;
      const bool extra = noisy && j == k && k < E;
      if (pick || extra) {
        float bv = neg_inf();
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < SL; i++) {
          const int e = lane + kWave * i;
          if (live[i] && !taken[i] && (be == 0x7fffffff || v[i] > bv)) {
            bv = v[i];
            be = e;
          }
        }
        wave_argmax(bv, be);
        if (extra) {
          thr_in = bv;
        } else {
          const int oi = be / kWave;
          float pi = p[0];
#pragma unroll
          for (int i = 1; i < SL; i++)
            if (oi == i) pi = p[i];
          pi = lane_f(pi, be % kWave);  // be is wave-uniform
          sel[j] = be;
          selp[j] = pi;
          thr_out = bv;  // the k-th largest once the loop ends (noisy: n == k)
          n = j + 1;
          cum += pi;
#pragma unroll
          for (int i = 0; i < SL; i++)
            if (lane + kWave * i == be) taken[i] = true;
          if (topp && cum > a.top_p) stop = true;
        }
      }
    }
    float den = 0.f;
#pragma unroll
    for (int j = 0; j < MAXK; j++)
      if (j < n) den += selp[j];
    int my_e = -1;
    float my_g = 0.f;
#pragma unroll
    for (int j = 0; j < MAXK; j++) {
      if (j < n) {
        const float gj = renorm ? selp[j] / den : selp[j];
        if (lane == j) {
          my_e = sel[j];
          my_g = gj;
        }
        // importance: the owner lane of expert sel[j] adds its gate
        const int e = sel[j];
        if ((e & (kWave - 1)) == lane) {
          const int oi = e / kWave;
#pragma unroll
          for (int i = 0; i < SL; i++)
            if (i == oi) imp[i] += gj;
        }
      }
    }
    if (lane < k) {
      a.ids[t * k + lane] = my_e;
      a.gates[t * k + lane] = my_g;
      if (my_e >= 0) {
        atomicAdd(&hcnt[my_e], 1);
        if (lane == 0) atomicAdd(&fcnt[my_e], 1);
      }
    }
    if (a.loadp) {
#pragma unroll
      for (int i = 0; i < SL; i++) {
        if (!live[i]) continue;
        float P;
        if (noisy) {
          const float thr = taken[i] ? thr_in : thr_out;
          const float zz = clean[i] - thr;
          P = sig[i] > 0.f ? phi_cdf(zz / sig[i]) : (zz > 0.f ? 1.f : 0.f);
        } else {
          P = taken[i] ? 1.f : 0.f;
        }
        ld[i] += P;
      }
    }
  }
#pragma unroll
  for (int i = 0; i < SL; i++) {
    const int e = lane + kWave * i;
    if (e < E) {
      qpart[wave][e] = q[i];
      ipart[wave][e] = imp[i];
      lpart[wave][e] = ld[i];
    }
  }
  if (lane == 0) zw[wave] = zacc;
  __syncthreads();
  if (a.zpart && tid == 0) {
    float z = 0.f;
    for (int w = 0; w < VW; w++) z += zw[w];
    a.zpart[blk] = z;
  }
  const int e = tid;
  if (e < E) {  // the waves' partials summed in wave order
    const int64_t o = (int64_t)e * gridDim.x + blk;
    float sq = 0.f, si = 0.f, sl = 0.f;
    for (int w = 0; w < VW; w++) {
      sq += qpart[w][e];
      si += ipart[w][e];
      sl += lpart[w][e];
    }
    a.qsum[o] = sq;
    a.fcount[o] = fcnt[e];
    if (a.hist) a.hist[o] = hcnt[e];
    if (a.imp) a.imp[o] = si;
    if (a.loadp) a.loadp[o] = sl;
  }
}

// embn[e] = emb[e] / |emb[e]| in fp32 (a zero row stays zero); one wave per expert
__global__ __launch_bounds__(256) void emb_normalize_kernel(const void *emb, int act_bf16, int E,
                                                            int de, float *embn) {
  const int w = blockIdx.x * 4 + threadIdx.x / kWave, lane = lane_id();
  if (w >= E) return;
  auto val = [&](int j) {
    const int64_t i = (int64_t)w * de + j;
    return act_bf16 ? (float)((const bf16 *)emb)[i] : ((const float *)emb)[i];
  };
  float s = 0.f;
  for (int j = lane; j < de; j += kWave) {
    const float v = val(j);
    s = fmaf(v, v, s);
  }
  s = wave_sum(s);
  const float inv = s > 0.f ? 1.f / sqrtf(s) : 0.f;
  for (int j = lane; j < de; j += kWave) embn[(int64_t)w * de + j] = val(j) * inv;
}

// cosl[t][e] = <embn[e], u[t]> / (tau |u[t]|), 0 when |u[t]| = 0; u = the
// projected tokens [T, de] fp32.  A block takes 64 tokens x all experts in
// fp32 on the vector ALUs: features in chunks of 32 through LDS, stored
// feature-major so that a thread's 4 tokens and 8 experts are 16-byte reads;
// thread (tid / 16, tid % 16) owns tokens 4 (tid / 16) .. + 3 and experts
// 8 (tid % 16) .. + 7 of each 128-expert half.
__global__ __launch_bounds__(256) void cosine_logits_kernel(const float *u, const float *embn,
                                                            int64_t T, int E, int de,
                                                            float inv_tau, float *cosl) {
  constexpr int JC = 32, UP = VBT + 4, EP = 256 + 4;
  __shared__ __attribute__((aligned(16))) float us[JC][UP];
  __shared__ __attribute__((aligned(16))) float es[JC][EP];
  __shared__ float nrm[VBT];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int64_t t0 = (int64_t)blockIdx.x * VBT;
  for (int rr = 0; rr < VBT / 4; rr++) {  // token norms
    const int r = wave * (VBT / 4) + rr;
    float s = 0.f;
    if (t0 + r < T)
      for (int j = lane; j < de; j += kWave) {
        const float v = u[(t0 + r) * de + j];
        s = fmaf(v, v, s);
      }
    s = wave_sum(s);
    if (lane == 0) nrm[r] = sqrtf(s);
  }
  const int tr = (tid / 16) * 4, tc = (tid % 16) * 8;
  const int halves = E > 128 ? 2 : 1;
  float acc[2][4][8];
#pragma unroll
  for (int h = 0; h < 2; h++)
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int c = 0; c < 8; c++) acc[h][i][c] = 0.f;
  for (int j0 = 0; j0 < de; j0 += JC) {
    const int jn = de - j0 < JC ? de - j0 : JC;
    __syncthreads();
    for (int idx = tid; idx < VBT * JC; idx += 256) {
      const int r = idx / JC, jj = idx % JC;
      us[jj][r] = (t0 + r < T && jj < jn) ? u[(t0 + r) * de + j0 + jj] : 0.f;
    }
    for (int idx = tid; idx < 256 * JC; idx += 256) {
      const int e = idx / JC, jj = idx % JC;
      es[jj][e] = (e < E && jj < jn) ? embn[(int64_t)e * de + j0 + jj] : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < jn; jj++) {
      const f32x4 a = *(const f32x4 *)&us[jj][tr];
#pragma unroll
      for (int h = 0; h < 2; h++) {
        if (h < halves) {
          const f32x4 b0 = *(const f32x4 *)&es[jj][h * 128 + tc];
          const f32x4 b1 = *(const f32x4 *)&es[jj][h * 128 + tc + 4];
#pragma unroll
          for (int i = 0; i < 4; i++)
#pragma unroll
            for (int c = 0; c < 4; c++) {
              acc[h][i][c] = fmaf(a[i], b0[c], acc[h][i][c]);
              acc[h][i][c + 4] = fmaf(a[i], b1[c], acc[h][i][c + 4]);
            }
        }
      }
    }
  }
#pragma unroll
  for (int h = 0; h < 2; h++)
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
      for (int c = 0; c < 8; c++) {
        const int r = tr + i, e = h * 128 + tc + c;
        if (h < halves && e < E && t0 + r < T)
          cosl[(t0 + r) * E + e] = nrm[r] > 0.f ? acc[h][i][c] * inv_tau / nrm[r] : 0.f;
      }
}

// Importance and Load losses: the per-expert sums of the block partials in
// fp64 in a fixed order (a wave per expert: lane-strided sums, then a
// butterfly), then w * variance / mean^2 (population variance; 0 when the
// mean is 0), one per loss.
__global__ __launch_bounds__(1024) void cov_loss_kernel(const float *imp, const float *loadp,
                                                        int nblk, int E, float w_imp,
                                                        float w_load, float *out_imp,
                                                        float *out_load) {
  __shared__ double vi[256], vl[256];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  for (int e = wave; e < E; e += 16) {
    double si = 0.0, sl = 0.0;
    for (int b = lane; b < nblk; b += kWave) {
      si += (double)imp[(int64_t)e * nblk + b];
      sl += (double)loadp[(int64_t)e * nblk + b];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      si += __shfl_xor(si, m, kWave);
      sl += __shfl_xor(sl, m, kWave);
    }
    if (lane == 0) {
      vi[e] = si;
      vl[e] = sl;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    auto cov2 = [&](const double *v) {
      double mean = 0.0;
      for (int i = 0; i < E; i++) mean += v[i];
      mean /= (double)E;
      if (mean == 0.0) return 0.0;
      double var = 0.0;
      for (int i = 0; i < E; i++) var += (v[i] - mean) * (v[i] - mean);
      var /= (double)E;
      return var / (mean * mean);
    };
    if (out_imp) out_imp[0] = (float)((double)w_imp * cov2(vi));
    if (out_load) out_load[0] = (float)((double)w_load * cov2(vl));
  }
}

}  // namespace moe

namespace moe_host {
using namespace moe;

template <int MAXK, int SL>
static void launch_route_logits_sl(const RouteVarArgs &a, int nblk, hipStream_t s) {
  const dim3 g(nblk), b(64 * VW);
  if (a.variant == RV_NOISY)
    MOE_LAUNCH("route_logits", (route_logits_kernel<MAXK, SL, RV_NOISY>), g, b, 0, s, a);
  else if (a.variant == RV_TOP_P)
    MOE_LAUNCH("route_logits", (route_logits_kernel<MAXK, SL, RV_TOP_P>), g, b, 0, s, a);
  else
    MOE_LAUNCH("route_logits", (route_logits_kernel<MAXK, SL, RV_TOPK>), g, b, 0, s, a);
}

template <int MAXK>
static void launch_route_logits_k(const RouteVarArgs &a, int nblk, hipStream_t s) {
  const int sl = (a.E + kWave - 1) / kWave;
  if (sl <= 1) launch_route_logits_sl<MAXK, 1>(a, nblk, s);
  else if (sl == 2) launch_route_logits_sl<MAXK, 2>(a, nblk, s);
  else if (sl == 3) launch_route_logits_sl<MAXK, 3>(a, nblk, s);
  else launch_route_logits_sl<MAXK, 4>(a, nblk, s);
}

hipError_t launch_route_logits(const RouteVarArgs &a, hipStream_t s) {
  const int nblk = router_blocks(a.T);
  if (nblk <= 0) return hipGetLastError();
  if (a.k <= 2)
    launch_route_logits_k<2>(a, nblk, s);
  else
    launch_route_logits_k<8>(a, nblk, s);
  return hipGetLastError();
}

hipError_t launch_emb_normalize(const void *emb, int act_bf16, int E, int de, float *embn,
                                hipStream_t s) {
  MOE_LAUNCH("emb_normalize", emb_normalize_kernel, dim3((E + 3) / 4), dim3(256), 0, s, emb,
             act_bf16, E, de, embn);
  return hipGetLastError();
}

hipError_t launch_cosine_logits(const float *u, const float *embn, int64_t T, int E, int de,
                                float inv_tau, float *cosl, hipStream_t s) {
  const int nblk = router_blocks(T);
  if (nblk <= 0) return hipGetLastError();
  MOE_LAUNCH("cosine_logits", cosine_logits_kernel, dim3(nblk), dim3(256), 0, s, u, embn, T, E,
             de, inv_tau, cosl);
  return hipGetLastError();
}

hipError_t launch_cov_loss(const float *imp, const float *loadp, int nblk, int E, float w_imp,
                           float w_load, float *out_imp, float *out_load, hipStream_t s) {
  MOE_LAUNCH("cov_loss", cov_loss_kernel, dim3(1), dim3(1024), 0, s, imp, loadp, nblk, E, w_imp,
             w_load, out_imp, out_load);
  return hipGetLastError();
}

}  // namespace moe_host
