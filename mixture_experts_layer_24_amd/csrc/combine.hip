// combine.hip -- gate-weighted combine with the residual add.
//
// Method: "DeepSpeed MoE and Model Compression", pipeline step
// combine(returned, gates) and the equation's sum over the chosen experts of
// p_e(x) E_e(x); "DeepSpeed-MoE vs Switch Transformer", sections "expert
// capacity overflow" (a dropped token contributes nothing from that expert
// and goes on through the residual) and "PR-MoE" residual example (fixed
// MLP output plus gate times the expert's output).
//
//   y[t] = (base[t] + base2[t]) + sum over j < k with slots[t,j] >= 0 of
//          gates[t,j] * y_disp[ids[t,j], slots[t,j]]
// fp32 accumulation in rank order j, one rounding to the output type.
// Token-major: one wave per token reads its k expert rows (a gather), so the
// sum order is fixed and no atomics are needed.  HBM-bound: 16-byte vectors.
// An assignment whose slot is outside [0, C) or whose expert is outside
// [0, E) contributes nothing.
#include "common.h"
#include "kernels.h"

namespace moe {

// V elements of src into dst: one 16-byte load when they are 16 bytes
template <typename T, int V>
__device__ __forceinline__ void load_v(T (&dst)[V], const T *src) {
  if constexpr (sizeof(T) * V == 16) {
    *(u32x4 *)dst = *(const u32x4 *)src;
  } else {
#pragma unroll
    for (int v = 0; v < V; v++) dst[v] = src[v];
  }
}

template <typename T, int V, int MAXK>  // V elements per lane per step, k <= MAXK
__global__ __launch_bounds__(256) void combine_kernel(const T *y_disp, const int32_t *ids,
                                                      const int32_t *slots, const float *gates,
                                                      const T *base, const T *base2, T *y,
                                                      int64_t n_tok, int d, int k, int64_t C,
                                                      int E) {
  const int lane = lane_id();
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave; t < n_tok; t += nw) {
    // lane j < k loads the token's assignment j (one round trip for all k)
    int sl = -1, el = -1;
    float gl = 0.f;
    if (lane < k) {
      sl = slots[t * k + lane];
      el = ids[t * k + lane];
      gl = gates[t * k + lane];
    }
    const T *row[MAXK];
    float g[MAXK];
#pragma unroll
    for (int j = 0; j < MAXK; j++) {
      row[j] = nullptr;
      g[j] = 0.f;
      if (j < k) {
        const int s = __builtin_amdgcn_readlane(sl, j);
        const int e = __builtin_amdgcn_readlane(el, j);
        if (s >= 0 && s < C && e >= 0 && e < E) {
          row[j] = y_disp + ((int64_t)e * C + s) * d;
          g[j] = lane_f(gl, j);
        }
      }
    }
    // the operands of CU column chunks -- the k expert rows and the residual
    // terms, 16-byte vectors when V elements are 16 bytes -- are all loaded
    // before the first of those chunks is written, so they are in flight
    // together (each output element is still read before it is written, so
    // an in-place base is fine)
    constexpr int CU = 4;
    for (int c0 = lane * V; c0 < d; c0 += CU * kWave * V) {
      T in[CU][MAXK][V], b1[CU][V], b2[CU][V];
#pragma unroll
      for (int u = 0; u < CU; u++) {
        const int c = c0 + u * kWave * V;
        if (c < d) {
#pragma unroll
          for (int j = 0; j < MAXK; j++)
            if (row[j] != nullptr) load_v<T, V>(in[u][j], row[j] + c);
          if (base) load_v<T, V>(b1[u], base + t * d + c);
          if (base2) load_v<T, V>(b2[u], base2 + t * d + c);
        }
      }
#pragma unroll
      for (int u = 0; u < CU; u++) {
        const int c = c0 + u * kWave * V;
        if (c >= d) continue;
        float acc[V];
#pragma unroll
        for (int v = 0; v < V; v++) acc[v] = 0.f;
#pragma unroll
        for (int j = 0; j < MAXK; j++)
          if (row[j] != nullptr) {
#pragma unroll
            for (int v = 0; v < V; v++)
              acc[v] = fmaf(g[j], ActTraits<T>::to_f(in[u][j][v]), acc[v]);
          }
        T out[V];
#pragma unroll
        for (int v = 0; v < V; v++) {
          float b = 0.f;
          if (base) b = ActTraits<T>::to_f(b1[u][v]);
          if (base2) b += ActTraits<T>::to_f(b2[u][v]);
          out[v] = ActTraits<T>::from_f(b + acc[v]);
        }
        if constexpr (sizeof(T) * V == 16) {
          *(u32x4 *)(y + t * d + c) = *(const u32x4 *)out;
        } else {
#pragma unroll
          for (int v = 0; v < V; v++) y[t * d + c + v] = out[v];
        }
      }
    }
  }
}

}  // namespace moe

namespace moe_host {
using namespace moe;

template <int MAXK>
static hipError_t launch_combine_k(const void *y_disp, const int32_t *ids, const int32_t *slots,
                                   const float *gates, const void *base, const void *base2,
                                   void *y, int64_t T, int d, int k, int64_t C, int E,
                                   int act_bf16, hipStream_t s) {
  int64_t blocks = (T + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  const dim3 g((unsigned)blocks), b(256);
  if (act_bf16) {
    if (d % 8 == 0)
      MOE_LAUNCH("combine_bf16", (combine_kernel<bf16, 8, MAXK>), g, b, 0, s,
                 (const bf16 *)y_disp, ids, slots, gates, (const bf16 *)base, (const bf16 *)base2,
                 (bf16 *)y, T, d, k, C, E);
    else
      MOE_LAUNCH("combine_bf16_v1", (combine_kernel<bf16, 1, MAXK>), g, b, 0, s,
                 (const bf16 *)y_disp, ids, slots, gates, (const bf16 *)base, (const bf16 *)base2,
                 (bf16 *)y, T, d, k, C, E);
  } else {
    if (d % 4 == 0)
      MOE_LAUNCH("combine_f32", (combine_kernel<float, 4, MAXK>), g, b, 0, s,
                 (const float *)y_disp, ids, slots, gates, (const float *)base,
                 (const float *)base2, (float *)y, T, d, k, C, E);
    else
      MOE_LAUNCH("combine_f32_v1", (combine_kernel<float, 1, MAXK>), g, b, 0, s,
                 (const float *)y_disp, ids, slots, gates, (const float *)base,
                 (const float *)base2, (float *)y, T, d, k, C, E);
  }
  return hipGetLastError();
}

hipError_t launch_combine(const void *y_disp, const int32_t *ids, const int32_t *slots,
                          const float *gates, const void *base, const void *base2, void *y,
                          int64_t T, int d, int k, int64_t C, int E, int act_bf16,
                          hipStream_t s) {
  if (T <= 0) return hipGetLastError();
  if (k <= 2)
    return launch_combine_k<2>(y_disp, ids, slots, gates, base, base2, y, T, d, k, C, E,
                               act_bf16, s);
  return launch_combine_k<8>(y_disp, ids, slots, gates, base, base2, y, T, d, k, C, E, act_bf16,
                             s);
}

}  // namespace moe_host
