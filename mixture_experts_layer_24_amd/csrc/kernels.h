// kernels.h -- internal launcher declarations (host side) of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct RouterArgs {
  const void *x;      // [T, d] act
  const void *w;      // [E, d] act
  const float *bias;  // [E] or null
  int32_t *ids;       // [T, k]
  float *gates;       // [T, k]
  float *logits;      // [T, E] or null
  float *qsum;        // [E, nblk] per-block sum of router probabilities
  int32_t *fcount;    // [E, nblk] per-block count of first choices
  int32_t *hist;      // [E, nblk] per-block count of all k assignments (or null)
  float *zpart;       // [nblk] per-block sum of squared log-sum-exp (or null)
  int64_t T;
  int d, E, k, normalize;
  const void *w2;     // raw-score mode: weight rows nw1.. come from here
  int nw1;
  float *part;        // split-K partial products [splits][blocks * 64][Ep] (workspace)
};

// router variants (router_var.hip); the values are the C ABI's MOE_ROUTER_*
enum { RV_TOPK = 0, RV_TOP_P = 1, RV_COSINE = 2, RV_NOISY = 3 };

struct RouteVarArgs {
  const float *src;    // [T, E] products (TopK, TopP) or cosine logits; noisy: [T, 2E]
                       // (the gate's products, then the noise scale's)
  const float *noise;  // [T, E] standard-normal draws (noisy)
  const float *bias;   // [E] or null
  int32_t *ids;        // [T, k], -1 = unused slot
  float *gates;        // [T, k]
  float *logits;       // [T, E] or null
  float *qsum;         // [E, nblk] as RouterArgs
  int32_t *fcount, *hist;
  float *zpart;        // [nblk] or null
  float *imp, *loadp;  // [E, nblk] importance / load partials, or null
  int64_t T;
  int E, k, normalize, variant;
  float top_p;
};

// Grouped "NT" GEMM: for each group g < G and row m < rows[g] (or M_cap):
//   C[g][m][n] = epi( sum_k A[g][m][k] * B[g][n][k] )
// (with the GELU epilogue and Zpre set, Zpre[g][m][n] = the sum itself)
struct GemmArgs {
  const void *A;        // act, [G][M_cap][K] (row stride K)
  const void *B;        // act or int8, [G][N][K]
  const void *Bscale;   // fp16 [G][N][K/128] (int8 only)
  void *C;              // act, [G][M_cap][N]
  const int32_t *rows;  // [G] valid rows per group (device) or null = M_cap
  int64_t M_cap;
  int N, K, G;
  void *Zpre;  // GELU epilogue only: also store the pre-activation here (as C), or null
  // int8 groups with more than 128 rows: the XCD schedule written by
  // launch_tile_sched for these rows (16 G + 16 int32), or null
  const int32_t *xsched;
  // B in blocks of 128 rows x 64 K (MOE_W_BF16_PACKED) instead of row-major
  int b_packed;
  // tiles in launch order, dealt round-robin over the XCDs (set by the
  // launcher for groups of one row tile), instead of a group per XCD
  int spread;
  // rows of A through a table: row m of group g is row asrc[g * M_cap + m]
  // of A ([rows][K], e.g. the token rows; rows * K * 2 < 2^32), or null = A
  // is [G][M_cap][K]; only the DMA kernels take it (gemm_reads_row_table)
  const int32_t *asrc;
};

// general grouped GEMM of the backward (backward.hip)
struct GenArgs {
  const bf16 *A;
  int64_t a_g, a_m, a_k, a_kmax;  // a_kmax: k rows that exist in memory (K-major)
  const bf16 *B;
  int64_t b_g, b_n, b_k, b_kmax;
  bf16 *C;
  int64_t c_g, c_m;
  const bf16 *Z;         // DGELU epilogue: C = acc * GELU'(Z), Z laid out as C
  const int32_t *mrows;  // [G] valid rows (clamped to M) or null
  int64_t M;
  const int32_t *krows;  // [G] valid reduction length (clamped to K) or null
  int64_t K;
  int N, G;
  int nsplit;  // short-reduction weight-gradient kernel: N sweeps per row panel (set by the launcher)
  int b_stream;  // B is read once (expert weights): non-temporal loads
};

}  // namespace moe

namespace moe_host {

int router_blocks(int64_t T);
// K splits launch_router uses for this batch (1 = none); the partial
// products need splits * router_blocks(T) * 64 * Ep floats of workspace
// (Ep = E rounded up to a multiple of 32)
int router_splits(int64_t T, int d, int act_bf16);
hipError_t launch_router(const moe::RouterArgs &a, int act_bf16, hipStream_t s);
hipError_t launch_aux_sum(const double *term, int E, float alpha, float *aux, hipStream_t s);
hipError_t launch_router_scores(const moe::RouterArgs &a, int act_bf16, hipStream_t s);
hipError_t launch_route_logits(const moe::RouteVarArgs &a, hipStream_t s);
hipError_t launch_emb_normalize(const void *emb, int act_bf16, int E, int de, float *embn,
                                hipStream_t s);
hipError_t launch_cosine_logits(const float *u, const float *embn, int64_t T, int E, int de,
                                float inv_tau, float *cosl, hipStream_t s);
hipError_t launch_cov_loss(const float *imp, const float *loadp, int nblk, int E, float w_imp,
                           float w_load, float *out_imp, float *out_load, hipStream_t s);
hipError_t launch_gemm_gen(const moe::GenArgs &a, bool a_kmajor, bool b_kmajor, bool dgelu,
                           const char *role, hipStream_t s);
hipError_t launch_gelu_map(const moe::bf16 *z, moe::bf16 *h, int64_t n, hipStream_t s);
hipError_t launch_bwd_gate(const moe::bf16 *dy, const moe::bf16 *y_disp, const int32_t *ids,
                           const int32_t *slots, const float *gates, int64_t T, int k, int d,
                           int64_t C, int E, float *dg, moe::bf16 *dY, hipStream_t s);
hipError_t launch_bwd_router(const float *logits, const int32_t *ids, const float *gates,
                             const float *dg, int32_t *fcnt, int64_t T, int E, int Ep, int k,
                             int normalize, float alpha, float g_aux, float g_z, float *dlog,
                             moe::bf16 *dlog16, float *db, hipStream_t s);
hipError_t launch_bwd_dx(const moe::bf16 *dy, const moe::bf16 *dxd, const moe::bf16 *dxr,
                         const moe::bf16 *dX, const int32_t *ids, const int32_t *slots, int64_t T,
                         int k, int d, int64_t C, int E, moe::bf16 *dx, hipStream_t s);
hipError_t launch_fill_i32(int32_t *p, int n, int v, hipStream_t s);
hipError_t launch_zloss_sum(const float *zpart, int nblk, int64_t T, float *z, hipStream_t s);

// dispatch (token blocks of the same size as the router's)
hipError_t launch_dispatch_count(const int32_t *ids, int64_t T, int E, int k, int32_t *hist,
                                 hipStream_t s);
// per-expert scan of the block histograms (hist may be null: aux only) and
// the aux-loss term per expert (qsum null: no aux)
hipError_t launch_scan_aux(const int32_t *hist, const float *qsum, const int32_t *fcount,
                           int nblk, int E, int64_t T, int64_t C, int32_t *offs, int32_t *load,
                           int32_t *kept, double *term, hipStream_t s);
// slots in token order; block 0 also finishes the aux loss when aux != null
// seg == null: token-order capacity.  seg != null: gate priority (gates and
// load required; seg is workspace of T*k int32).  src != null (token order
// only): src[e * C + slot] = token of every kept assignment, the row table
// through which the first expert GEMM reads x instead of a gathered x_disp.
hipError_t launch_dispatch_place(const int32_t *ids, const int32_t *offs, int64_t T, int E, int k,
                                 int64_t C, int32_t *slots, uint8_t *drop, const double *aux_term,
                                 float aux_alpha, float *aux, hipStream_t s,
                                 const float *gates = nullptr, const int32_t *load = nullptr,
                                 int32_t *seg = nullptr, int32_t *src = nullptr);
hipError_t launch_gather(const void *x, const int32_t *ids, const int32_t *slots, int64_t T, int k,
                         int64_t C, int64_t row_bytes, void *x_disp, hipStream_t s);

// expert / dense GEMMs; gelu selects the GELU epilogue; role names the launch
// in the per-kernel timing ("expert_ffn1", "expert_ffn2", "dense_mlp1", ...)
hipError_t launch_gemm(const moe::GemmArgs &a, int act_bf16, int b_int8, int gelu,
                       const char *role, hipStream_t s);
// whether launch_gemm can read A's rows through a.asrc for these shapes, with
// a_rows rows behind the table
bool gemm_reads_row_table(const moe::GemmArgs &a, int act_bf16, int b_int8, int64_t a_rows);
// [G][N][K] row-major bf16 -> blocks of 128 rows x 64 K (N % 128 == 0, K % 64 == 0)
hipError_t launch_pack_weights(const void *w, void *wp, int64_t G, int64_t N, int64_t K,
                               hipStream_t s);
// XCD schedule of G groups' int8 tiles from their row counts (G <= 256);
// light: groups of at most 64 rows run 64 x 512 tiles (both GEMMs' N must be
// multiples of 512)
hipError_t launch_tile_sched(const int32_t *rows, int G, int64_t M_cap, int light, int32_t *xs,
                             hipStream_t s);

// a stable C string for a profiling name built at run time
const char *intern_name(const char *a, const char *b);

hipError_t launch_combine(const void *y_disp, const int32_t *ids, const int32_t *slots,
                          const float *gates, const void *base, const void *base2, void *y,
                          int64_t T, int d, int k, int64_t C, int E, int act_bf16,
                          hipStream_t s);

}  // namespace moe_host
