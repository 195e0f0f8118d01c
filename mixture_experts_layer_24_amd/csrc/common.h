// common.h -- shared device types and helpers of the gfx950 MoE-layer library.
// Internal to the library (not part of the C ABI in include/moe.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

namespace moe {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
// 16-byte staging register (a native vector: HIP's uint4 struct copies are
// lowered through private memory)
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ------------------------------------------------------------- wave helpers
__device__ __forceinline__ int lane_id() { return __lane_id(); }
__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

// Cross-lane reductions on VALU data movement instead of the LDS crossbar
// (ds_bpermute): DPP within each 16-lane row -- quad permutes [1,0,3,2] and
// [2,3,0,1], then the half-row mirror (lane i <-> 7 - i) and the row mirror
// (i <-> 15 - i), each pairing two groups that already hold their own
// totals -- then the four row totals read from lanes 0, 16, 32, 48 and
// combined in a fixed order.  Every lane returns the same value; the caller
// must run the whole wave (no divergent lanes).
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float lane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<0xB1>(v));   // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_f<0x4E>(v));   // quad_perm [2,3,0,1]
  v = fmaxf(v, dpp_f<0x141>(v));  // row_half_mirror
  v = fmaxf(v, dpp_f<0x140>(v));  // row_mirror
  return fmaxf(fmaxf(lane_f(v, 0), lane_f(v, 16)), fmaxf(lane_f(v, 32), lane_f(v, 48)));
}

__device__ __forceinline__ float wave_sum(float v) {
  // each step adds a lane and its partner, so a row's lanes agree bit for
  // bit; the rows are summed as (r0 + r1) + (r2 + r3)
  v += dpp_f<0xB1>(v);
  v += dpp_f<0x4E>(v);
  v += dpp_f<0x141>(v);
  v += dpp_f<0x140>(v);
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}

// (value, index) arg-max over the wave: larger value wins, equal values go
// to the smaller index (a total order, so the reduction order does not
// matter).  Every lane returns the winner.
__device__ __forceinline__ void argmax_step(float &v, int &idx, float ov, int oi) {
  if (ov > v || (ov == v && oi < idx)) {
    v = ov;
    idx = oi;
  }
}
template <int CTRL>
__device__ __forceinline__ void argmax_dpp(float &v, int &idx) {
  const float ov = dpp_f<CTRL>(v);
  const int oi = dpp_i<CTRL>(idx);
  argmax_step(v, idx, ov, oi);
}
__device__ __forceinline__ void wave_argmax(float &v, int &idx) {
  argmax_dpp<0xB1>(v, idx);
  argmax_dpp<0x4E>(v, idx);
  argmax_dpp<0x141>(v, idx);
  argmax_dpp<0x140>(v, idx);
  float bv = lane_f(v, 0);
  int bi = __builtin_amdgcn_readlane(idx, 0);
#pragma unroll
  for (int r = 16; r < 64; r += 16) argmax_step(bv, bi, lane_f(v, r), __builtin_amdgcn_readlane(idx, r));
  v = bv;
  idx = bi;
}

// ------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(bf16 b) { return (float)b; }
__device__ __forceinline__ bf16 f2bf(float f) { return (bf16)f; }  // RNE

// erf(x) by Abramowitz & Stegun, Handbook of Mathematical Functions, formula
// 7.1.26: erf(x) = 1 - (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-x^2),
// t = 1 / (1 + p x) for x >= 0 (odd extension), |error| <= 1.5e-7 -- far
// below the bf16 rounding of the values it feeds (the backward's GELU
// derivative, Phi(z) + z phi(z)).
__device__ __forceinline__ float erf_as(float x) {
  const float ax = fabsf(x);
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, ax, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  poly *= t;
  // exp(-x^2) = 2^(-x^2 * log2 e)
  const float e = __builtin_amdgcn_exp2f(-ax * ax * 1.4426950408889634f);
  return copysignf(fmaf(-poly, e, 1.0f), x);
}

// GELU with the exact (erf) form, z * Phi(z), written as
//   max(z, 0) - |z| Q(|z|),  Q(x) = Phi(-x) = 2^g(u),  u = min(x, 6) / 3 - 1,
// g a degree-9 polynomial fitted to log2 Q on [0, 6] (gelu_fit.py, which
// prints these coefficients): one exp2 and no reciprocal per element, |error|
// <= 3.1e-7 in fp32 (the erf_as form above needs a reciprocal and an exp2 and
// is as accurate; the GEMM epilogues' GELU took ~10% of the first layers'
// time with it).  Past |z| = 6, Q stays at Q(6) ~ 1e-9.
__device__ __forceinline__ float gelu_f(float z) {
  const float u = fmaf(fminf(fabsf(z), 6.0f), 1.0f / 3.0f, -1.0f);
  float g = 9.821072454e-04f;
  g = fmaf(g, u, -4.859279215e-05f);
  g = fmaf(g, u, -6.342675537e-03f);
  g = fmaf(g, u, 1.686366647e-02f);
  g = fmaf(g, u, -3.910345584e-02f);
  g = fmaf(g, u, 9.169072658e-02f);
  g = fmaf(g, u, -2.044294178e-01f);
  g = fmaf(g, u, -6.033986092e+00f);
  g = fmaf(g, u, -1.420952320e+01f);
  g = fmaf(g, u, -9.532935143e+00f);
  return fmaf(-fabsf(z), __builtin_amdgcn_exp2f(g), fmaxf(z, 0.0f));
}

template <typename T>
struct ActTraits;
template <>
struct ActTraits<float> {
  static __device__ __forceinline__ float to_f(float v) { return v; }
  static __device__ __forceinline__ float from_f(float v) { return v; }
};
template <>
struct ActTraits<bf16> {
  static __device__ __forceinline__ float to_f(bf16 v) { return (float)v; }
  static __device__ __forceinline__ bf16 from_f(float v) { return (bf16)v; }
};

// Blocks are spread over the 8 XCDs round-robin by hardware: block b runs on
// XCD b % 8.  Remap so each XCD receives a contiguous range of logical tiles
// (neighbouring tiles then share that XCD's L2).  Bijective on [0, n).
__device__ __forceinline__ int xcd_remap(int b, int n) {
  constexpr int X = 8;
  const int per = n / X, rem = n % X;
  const int x = b % X, i = b / X;
  return x * per + (x < rem ? x : rem) + i;
}

// Grouped variant for G groups of `per_group` tiles with G % 8 == 0: XCD x
// takes groups x, x+8, x+16, ... and runs each group's tiles back to back, so
// one expert's tiles share an L2 while skewed per-expert work is dealt evenly
// over the XCDs.  Returns the logical tile g * per_group + r.  Bijective.
__device__ __forceinline__ int xcd_remap_grouped(int b, int G, int per_group) {
  constexpr int X = 8;
  const int x = b % X, i = b / X;
  const int lg = i / per_group, r = i - lg * per_group;
  return (lg * X + x) * per_group + r;
}

// Tile r of a group with tiles_m x tiles_n tiles, in grouped order: GM
// row-tiles are swept column by column (r -> (tm, tn)), so the tiles that
// run at the same time share both operand slabs in L2 instead of each reading
// its own weight slab.  Bijective on [0, tiles_m * tiles_n).
template <int GM = 8>
__device__ __forceinline__ void grouped_tile(int r, int tiles_m, int tiles_n, int &tm, int &tn) {
  const int q = r / (GM * tiles_n);
  const int tm0 = q * GM;
  const int gm = tiles_m - tm0 < GM ? tiles_m - tm0 : GM;
  const int local = r - tm0 * tiles_n;
  tm = tm0 + local % gm;
  tn = local / gm;
}

// Switch load-balance loss, final step: aux = alpha * E * sum_e term[e],
// summed by one wave in a fixed order (every lane ends with the same sum).
__device__ __forceinline__ void aux_sum_wave(const double *term, int E, float alpha,
                                             float *aux) {
  const int lane = lane_id();
  double v = 0.0;
  for (int e = lane; e < E; e += kWave) v += term[e];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  if (lane == 0) aux[0] = (float)((double)alpha * (double)E * v);
}

}  // namespace moe

// ------------------------------------------------------------- host side
namespace moe_host {
// Launch bookkeeping: records per-kernel HIP events when profiling is on.
void prof_begin(hipStream_t s, const char *name);
void prof_end(hipStream_t s);

template <typename... KArgs, typename... Args>
inline void launch(const char *name, void (*kernel)(KArgs...), dim3 grid, dim3 block, size_t lds,
                   hipStream_t s, Args... args) {
  prof_begin(s, name);
  hipLaunchKernelGGL(kernel, grid, block, lds, s, static_cast<KArgs>(args)...);
  prof_end(s);
}
}  // namespace moe_host

#define MOE_LAUNCH(name, kernel, grid, block, lds, stream, ...) \
  moe_host::launch((name), kernel, (grid), (block), (lds), (stream), __VA_ARGS__)
