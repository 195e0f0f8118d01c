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

template <typename T, int V>  // V elements per lane per step
__global__ __launch_bounds__(256) void combine_kernel(const T *y_disp, const int32_t *ids,
                                                      const int32_t *slots, const float *gates,
                                                      const T *base, const T *base2, T *y,
                                                      int64_t n_tok, int d, int k, int64_t C,
                                                      int E) {
  constexpr int MAXK = 8;
  const int lane = lane_id();
  const int64_t nw = (int64_t)gridDim.x * 4;
  for (int64_t t = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave; t < n_tok; t += nw) {
    const T *row[MAXK];
    float g[MAXK];
#pragma unroll
    for (int j = 0; j < MAXK; j++) {
      row[j] = nullptr;
      g[j] = 0.f;
      if (j < k) {
        const int s = __builtin_amdgcn_readfirstlane(slots[t * k + j]);
        const int e = __builtin_amdgcn_readfirstlane(ids[t * k + j]);
        if (s >= 0 && s < C && e >= 0 && e < E) {
          row[j] = y_disp + ((int64_t)e * C + s) * d;
          g[j] = gates[t * k + j];
        }
      }
    }
    for (int c = lane * V; c < d; c += kWave * V) {
      float acc[V];
#pragma unroll
      for (int v = 0; v < V; v++) acc[v] = 0.f;
#pragma unroll
      for (int j = 0; j < MAXK; j++) {
        if (row[j] != nullptr) {
          T in[V];
          if constexpr (sizeof(T) * V == 16) {
            *(u32x4 *)in = *(const u32x4 *)(row[j] + c);
          } else {
#pragma unroll
            for (int v = 0; v < V; v++) in[v] = row[j][c + v];
          }
#pragma unroll
          for (int v = 0; v < V; v++) acc[v] = fmaf(g[j], ActTraits<T>::to_f(in[v]), acc[v]);
        }
      }
      T out[V];
#pragma unroll
      for (int v = 0; v < V; v++) {
        float b = 0.f;
        if (base) b = ActTraits<T>::to_f(base[t * d + c + v]);
        if (base2) b += ActTraits<T>::to_f(base2[t * d + c + v]);
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

}  // namespace moe

namespace moe_host {
using namespace moe;

hipError_t launch_combine(const void *y_disp, const int32_t *ids, const int32_t *slots,
                          const float *gates, const void *base, const void *base2, void *y,
                          int64_t T, int d, int k, int64_t C, int E, int act_bf16,
                          hipStream_t s) {
  if (T <= 0) return hipGetLastError();
  int64_t blocks = (T + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  if (act_bf16) {
    if (d % 8 == 0)
      MOE_LAUNCH("combine_bf16", (combine_kernel<bf16, 8>), dim3((unsigned)blocks), dim3(256), 0, s,
                 (const bf16 *)y_disp, ids, slots, gates, (const bf16 *)base, (const bf16 *)base2,
                 (bf16 *)y, T, d, k, C, E);
    else
      MOE_LAUNCH("combine_bf16_v1", (combine_kernel<bf16, 1>), dim3((unsigned)blocks), dim3(256), 0,
                 s, (const bf16 *)y_disp, ids, slots, gates, (const bf16 *)base,
                 (const bf16 *)base2, (bf16 *)y, T, d, k, C, E);
  } else {
    if (d % 4 == 0)
      MOE_LAUNCH("combine_f32", (combine_kernel<float, 4>), dim3((unsigned)blocks), dim3(256), 0, s,
                 (const float *)y_disp, ids, slots, gates, (const float *)base,
                 (const float *)base2, (float *)y, T, d, k, C, E);
    else
      MOE_LAUNCH("combine_f32_v1", (combine_kernel<float, 1>), dim3((unsigned)blocks), dim3(256), 0,
                 s, (const float *)y_disp, ids, slots, gates, (const float *)base,
                 (const float *)base2, (float *)y, T, d, k, C, E);
  }
  return hipGetLastError();
}

}  // namespace moe_host
