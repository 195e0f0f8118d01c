// dispatch.hip -- capacity-limited, token-order dispatch and the layout
// transform into the expert-major buffer [E, C, d].
//
// Method: "DeepSpeed MoE and Model Compression", pipeline step
// pack_by_expert(hidden, expert_ids, capacity); "DeepSpeed-MoE vs Switch
// Transformer", section "expert capacity overflow" (per-expert cap; an
// overflowing token skips the expert); "DeepSpeed-MoE ... notes" sec. 4.4
// (a cumulative sum over tokens gives each assignment its place in a dense
// token-to-expert mapping table, and rows are then moved with that table
// instead of one-hot masks, so the cost does not grow with E).
//
// The slot of assignment (t, j) in expert e is the number of assignments to e
// that come before it in token order; it is kept iff slot < C.  Computed
// deterministically without order-dependent atomics:
//   count : per 64-token block, an integer histogram over experts
//   scan  : one block per expert: exclusive prefix over the token blocks ->
//           block offsets, load[e] = total, kept[e] = min(load[e], C) (the
//           per-block counts are stored expert-major so this read is contiguous)
//   place : one wave per block walks its 64*k assignments in order in chunks
//           of 64; within a chunk, lanes with equal expert ids are grouped
//           with one ballot per bit of the id (eight for E <= 256, however
//           many experts the chunk holds), ranked by lane order (popcount of
//           the lower lanes), and the running per-expert count lives in
//           registers spread over the lanes (expert e in lane e % 64,
//           register e / 64)
//   gather: one wave per assignment copies the token's row to its slot with
//           16-byte vector loads/stores (each row is contiguous on both sides,
//           so the copy is fully coalesced without staging)
// Expert ids outside [0, E) are treated as dropped and not counted.
#include "common.h"
#include "kernels.h"

namespace moe {

constexpr int DBT = 64;  // tokens per dispatch block (the router's block size)

__global__ __launch_bounds__(256) void dispatch_count_kernel(const int32_t *ids, int64_t T, int E,
                                                             int k, int32_t *hist) {
  __shared__ int cnt[256];
  const int tid = threadIdx.x, blk = blockIdx.x;
  cnt[tid] = 0;
  __syncthreads();
  const int64_t a0 = (int64_t)blk * DBT * k;
  int64_t a1 = a0 + (int64_t)DBT * k;
  if (a1 > T * k) a1 = T * k;
  for (int64_t a = a0 + tid; a < a1; a += 256) {
    const int e = ids[a];
    if (e >= 0 && e < E) atomicAdd(&cnt[e], 1);
  }
  __syncthreads();
  if (tid < E) hist[(int64_t)tid * gridDim.x + blk] = cnt[tid];
}

// One block per expert e: exclusive prefix of hist[e][*] over the token
// blocks (each thread scans a contiguous chunk, chunk totals are scanned
// across the block), load[e], kept[e]; with router partials also the
// expert's aux-loss term f_e * Q_e, summed in a fixed order in fp64.
__global__ __launch_bounds__(256) void scan_aux_kernel(const int32_t *hist, const float *qsum,
                                                       const int32_t *fcount, int nblk, int E,
                                                       int64_t T, int64_t C, int32_t *offs,
                                                       int32_t *load, int32_t *kept,
                                                       double *term) {
  __shared__ int wsum[4];
  __shared__ double red[2][256];
  const int e = blockIdx.x, tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int chunk = (nblk + 255) / 256;
  const int b0 = tid * chunk;
  const int b1 = min(b0 + chunk, nblk);
  const int64_t base = (int64_t)e * nblk;
  if (hist) {
    int tot = 0;
    for (int b = b0; b < b1; b++) tot += hist[base + b];
    // inclusive scan of chunk totals within the wave, then across waves
    int inc = tot;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const int v = __shfl_up(inc, o, kWave);
      if (lane >= o) inc += v;
    }
    if (lane == kWave - 1) wsum[wave] = inc;
    __syncthreads();
    int run = inc - tot;
    for (int w = 0; w < wave; w++) run += wsum[w];
    for (int b = b0; b < b1; b++) {
      const int h = hist[base + b];
      offs[base + b] = run;
      run += h;
    }
    if (tid == 255) {
      load[e] = run;
      kept[e] = (int64_t)run < C ? run : (int32_t)C;
    }
  }
  if (qsum) {
    double q = 0.0, f = 0.0;
    for (int b = b0; b < b1; b++) {
      q += (double)qsum[base + b];
      f += (double)fcount[base + b];
    }
    red[0][tid] = q;
    red[1][tid] = f;
    __syncthreads();
    for (int st = 128; st >= 1; st >>= 1) {
      if (tid < st) {
        red[0][tid] += red[0][tid + st];
        red[1][tid] += red[1][tid + st];
      }
      __syncthreads();
    }
    if (tid == 0) term[e] = T > 0 ? (red[1][0] / (double)T) * (red[0][0] / (double)T) : 0.0;
  }
}

// Token-order position of every assignment within its expert (the n-th
// assignment of expert e in token order has position n), from the per-block
// offsets; a wave ranks 64 assignments at a time with ballots.
// Token order (seg == null): slot = position if < C, else dropped; with src,
// src[e * C + slot] = the token of each kept assignment.
// Gate priority (seg != null): no capacity here; the position goes to
// slots[] and the assignment index to seg[ebase[e] + position], where ebase
// is the exclusive prefix of load[] over experts, for rank_gate_kernel.
__global__ __launch_bounds__(64) void dispatch_place_kernel(const int32_t *ids, const int32_t *offs,
                                                            int64_t T, int E, int k, int64_t C,
                                                            int32_t *slots, uint8_t *drop,
                                                            const double *aux_term,
                                                            float aux_alpha, float *aux,
                                                            const int32_t *load, int32_t *seg,
                                                            int32_t *src) {
  const int lane = lane_id(), blk = blockIdx.x, nblk = gridDim.x;
  // this block's offsets and its first 64 assignments are loaded before
  // anything else, so their latencies overlap the aux sum and the scan below
  int run0 = 0, run1 = 0, run2 = 0, run3 = 0;
  if (lane < E) run0 = offs[(int64_t)lane * nblk + blk];
  if (lane + 64 < E) run1 = offs[(int64_t)(lane + 64) * nblk + blk];
  if (lane + 128 < E) run2 = offs[(int64_t)(lane + 128) * nblk + blk];
  if (lane + 192 < E) run3 = offs[(int64_t)(lane + 192) * nblk + blk];
  const int64_t a0 = (int64_t)blk * DBT * k;
  int64_t a1 = a0 + (int64_t)DBT * k;
  if (a1 > T * k) a1 = T * k;
  int e_next = (a0 + lane < a1) ? ids[a0 + lane] : -1;
  // the layer's aux loss is finished here, by block 0, when asked
  if (aux && blk == 0) aux_sum_wave(aux_term, E, aux_alpha, aux);
  // segment base of expert lane + 64 i (gate priority)
  int eb0 = 0, eb1 = 0, eb2 = 0, eb3 = 0;
  if (seg) {
    int carry = 0;
#pragma unroll
    for (int i = 0; i < 4; i++) {
      const int e = lane + 64 * i;
      const int v = e < E ? load[e] : 0;
      int inc = v;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int u = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += u;
      }
      const int b = carry + inc - v;
      if (i == 0) eb0 = b;
      else if (i == 1) eb1 = b;
      else if (i == 2) eb2 = b;
      else eb3 = b;
      carry += __shfl(inc, kWave - 1, kWave);
    }
  }
  // run0..run3: running slot of expert e = lane + 64 i, from this block's offset
  const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int64_t base = a0; base < a1; base += 64) {
    const int64_t a = base + lane;
    int e = e_next;
    if (base + 64 < a1) e_next = (a + 64 < a1) ? ids[a + 64] : -1;  // next chunk's ids
    const bool valid = e >= 0 && e < E;
    if (!valid) e = 0;
    // one ballot per bit of the expert id (E <= 256): the lanes holding
    // expert x in this chunk are the valid lanes that agree with x on all
    // eight bits, so every lane finds its group without a loop over experts
    const uint64_t vm = __ballot(valid);
    uint64_t bal[8];
#pragma unroll
    for (int b = 0; b < 8; b++) bal[b] = __ballot(valid && ((e >> b) & 1));
    uint64_t same = vm, mine = vm;  // lanes of this lane's expert e; of expert lane (+ 64 i)
#pragma unroll
    for (int b = 0; b < 8; b++) same &= ((e >> b) & 1) ? bal[b] : ~bal[b];
#pragma unroll
    for (int b = 0; b < 6; b++) mine &= ((lane >> b) & 1) ? bal[b] : ~bal[b];
    const uint64_t hi0 = ~bal[6] & ~bal[7], hi1 = bal[6] & ~bal[7];  // bits 6, 7 of 64 i
    const uint64_t hi2 = ~bal[6] & bal[7], hi3 = bal[6] & bal[7];
    // start of e's run: register e / 64 of lane e % 64 (before this chunk)
    const int rl = e & 63, ri = e >> 6;
    int start = __shfl(run0, rl, kWave);
    int ebase = 0;
    if (seg) ebase = __shfl(eb0, rl, kWave);
    if (E > 64) {
      const int s1 = __shfl(run1, rl, kWave);
      if (ri == 1) start = s1;
      if (seg) {
        const int b1 = __shfl(eb1, rl, kWave);
        if (ri == 1) ebase = b1;
      }
    }
    if (E > 128) {
      const int s2 = __shfl(run2, rl, kWave), s3 = __shfl(run3, rl, kWave);
      if (ri == 2) start = s2;
      if (ri == 3) start = s3;
      if (seg) {
        const int b2 = __shfl(eb2, rl, kWave), b3 = __shfl(eb3, rl, kWave);
        if (ri == 2) ebase = b2;
        if (ri == 3) ebase = b3;
      }
    }
    const int slot = start + __popcll(same & lower);
    run0 += __popcll(mine & hi0);
    if (E > 64) run1 += __popcll(mine & hi1);
    if (E > 128) {
      run2 += __popcll(mine & hi2);
      run3 += __popcll(mine & hi3);
    }
    if (a < a1) {
      // an id that is not an expert (an unused TopP slot) is no assignment
      if (seg) {
        slots[a] = valid ? slot : -1;
        if (valid) seg[ebase + slot] = (int32_t)a;
        else if (drop) drop[a] = 0;
      } else {
        const bool keep = valid && (int64_t)slot < C;
        slots[a] = keep ? slot : -1;
        if (drop) drop[a] = (valid && !keep) ? 1 : 0;
        if (src && keep) src[(int64_t)e * C + slot] = (int32_t)(a / k);
      }
    }
  }
}

// Gate-priority capacity.  Within expert e, assignment p (token-order
// position) has rank = #{q in e : gate_q > gate_p, or gate_q == gate_p and
// q < p}; it is kept, with slot = rank, iff rank < C.  Two steps:
//  select_gate_kernel (one block per expert with load > C): radix-selects
//    the C-th largest gate, keeps the assignments with a larger gate and the
//    first ones in token order with an equal gate, drops the rest, and
//    compacts the kept ones (still in token order) to the front of the
//    expert's segment;
//  rank_gate_kernel: ranks each kept assignment among the expert's
//    min(load, C) kept ones (256 per block, the list through LDS).
// Exact and deterministic; about load + min(load, C)^2 comparisons per
// expert.  Gates compare as floats (-0 equals +0); they must be finite.

// monotone unsigned key of a float (-0 mapped to +0)
__device__ __forceinline__ uint32_t gate_key(float g) {
  uint32_t b = __float_as_uint(g);
  if (b == 0x80000000u) b = 0;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// exclusive count of `f` over the block's threads in order, and the total
__device__ __forceinline__ int block_excl_count(bool f, int *wsum, int &total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const uint64_t m = __ballot(f);
  const int in = __popcll(m & ((1ull << lane) - 1ull));
  if (lane == 0) wsum[wave] = __popcll(m);
  __syncthreads();
  int off = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < 4; w++) {
    if (w < wave) off += wsum[w];
    total += wsum[w];
  }
  __syncthreads();
  return off + in;
}

// exclusive prefix over experts of load[] (and of min(load, C) tiles) into
// LDS; 256 threads, E <= 256
__device__ __forceinline__ void expert_prefix(const int32_t *load, int E, int64_t C, int *ebase,
                                              int *tbase, int (*wtot)[4]) {
  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int L = tid < E ? load[tid] : 0;
  const int K = (int64_t)L < C ? L : (int)C;
  const int nt = (K + 255) / 256;
  int incl = L, inct = nt;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int u = __shfl_up(incl, o, kWave), w = __shfl_up(inct, o, kWave);
    if (lane >= o) {
      incl += u;
      inct += w;
    }
  }
  if (lane == kWave - 1) {
    wtot[0][wave] = incl;
    wtot[1][wave] = inct;
  }
  __syncthreads();
  int bl = 0, bt = 0;
  for (int w = 0; w < wave; w++) {
    bl += wtot[0][w];
    bt += wtot[1][w];
  }
  ebase[tid] = bl + incl - L;
  tbase[tid] = bt + inct - nt;
  if (tid == 255) {
    ebase[256] = bl + incl;
    tbase[256] = bt + inct;
  }
  __syncthreads();
}

__global__ __launch_bounds__(256) void select_gate_kernel(int32_t *seg, const float *gates,
                                                          const int32_t *load, int E, int64_t C,
                                                          int32_t *slots, uint8_t *drop) {
  __shared__ int ebase[257], tbase[257];
  __shared__ int wtot[2][4], wsum[4];
  __shared__ int hist[256];
  __shared__ int sel_bucket, sel_rem;
  const int tid = threadIdx.x, e = blockIdx.x;
  expert_prefix(load, E, C, ebase, tbase, wtot);
  const int L = load[e];
  if ((int64_t)L <= C) return;  // every assignment kept; the segment is the list
  int32_t *sg = seg + ebase[e];
  // radix select, 8 bits at a time from the top: the key of the C-th largest
  uint32_t prefix = 0, pmask = 0;
  int rem = (int)C;  // rank sought among the candidates (1 = largest)
  for (int shift = 24; shift >= 0; shift -= 8) {
    hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < L; i += 256) {
      const uint32_t k = gate_key(gates[sg[i]]);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, b = 255;
      for (; b > 0; b--) {
        if (cum + hist[b] >= rem) break;
        cum += hist[b];
      }
      sel_bucket = b;
      sel_rem = rem - cum;
    }
    __syncthreads();
    prefix |= (uint32_t)sel_bucket << shift;
    pmask |= 0xFFu << shift;
    rem = sel_rem;
  }
  // keep key > prefix, and the first `rem` (token order) with key == prefix;
  // compact the kept to the front of the segment, in place (each chunk is
  // read before any of it is overwritten; writes never pass the read point)
  int carry_eq = 0, carry_k = 0;
  for (int c0 = 0; c0 < L; c0 += 256) {
    const int i = c0 + tid;
    const bool valid = i < L;
    const int32_t a = valid ? sg[i] : 0;
    const uint32_t k = valid ? gate_key(gates[a]) : 0u;
    const bool gt = valid && k > prefix, eq = valid && k == prefix;
    int n_eq, n_keep;
    const int eq_before = carry_eq + block_excl_count(eq, wsum, n_eq);
    const bool keep = gt || (eq && eq_before < rem);
    const int kidx = carry_k + block_excl_count(keep, wsum, n_keep);
    if (valid) {
      if (keep) {
        sg[kidx] = a;
      } else {
        slots[a] = -1;
        if (drop) drop[a] = 1;
      }
    }
    carry_eq += n_eq;
    carry_k += n_keep;
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void rank_gate_kernel(const int32_t *seg, const float *gates,
                                                        const int32_t *load, int E, int64_t C,
                                                        int32_t *slots, uint8_t *drop) {
  __shared__ int ebase[257], tbase[257];
  __shared__ int wtot[2][4];
  __shared__ float cg[256];
  const int tid = threadIdx.x;
  expert_prefix(load, E, C, ebase, tbase, wtot);
  const int b = blockIdx.x;
  if (b >= tbase[256]) return;
  // expert of this block: the last e with tbase[e] <= b (experts without
  // kept assignments have no tiles, so that e has some)
  int lo = 0, hi = E - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tbase[mid] <= b) lo = mid;
    else hi = mid - 1;
  }
  const int e = lo;
  const int K = (int64_t)load[e] < C ? load[e] : (int)C;
  const int p = (b - tbase[e]) * 256 + tid;
  const int32_t *sg = seg + ebase[e];
  const float g = p < K ? gates[sg[p]] : 0.f;
  int rank = 0;
  for (int c0 = 0; c0 < K; c0 += 256) {
    __syncthreads();
    const int q = c0 + tid;
    cg[tid] = q < K ? gates[sg[q]] : 0.f;
    __syncthreads();
    const int n = K - c0 < 256 ? K - c0 : 256;
    for (int j = 0; j < n; j++) {
      const float h = cg[j];
      rank += (h > g || (h == g && c0 + j < p)) ? 1 : 0;
    }
  }
  if (p < K) {
    const int32_t a = sg[p];
    slots[a] = rank;
    if (drop) drop[a] = 0;
  }
}

// one wave per assignment; VT = the vector type moved per lane.  A row is
// copied in passes of up to GV vectors per lane, every load of a pass issued
// before its first store (x and x_disp never overlap).
template <typename VT>
__global__ __launch_bounds__(256) void gather_kernel(const char *__restrict__ x,
                                                     const int32_t *__restrict__ ids,
                                                     const int32_t *__restrict__ slots,
                                                     int64_t n_assign, int k, int64_t C,
                                                     int64_t row_bytes, char *__restrict__ x_disp) {
  constexpr int GV = 8;
  const int lane = lane_id();
  const int64_t nw = (int64_t)gridDim.x * 4;
  const int64_t nvec = row_bytes / (int64_t)sizeof(VT);
  for (int64_t a = (int64_t)blockIdx.x * 4 + threadIdx.x / kWave; a < n_assign; a += nw) {
    const int slot = __builtin_amdgcn_readfirstlane(slots[a]);
    if (slot < 0) continue;
    const int e = __builtin_amdgcn_readfirstlane(ids[a]);
    const VT *src = (const VT *)(x + (a / k) * row_bytes);
    VT *dst = (VT *)(x_disp + ((int64_t)e * C + slot) * row_bytes);
    for (int64_t c0 = lane; c0 < nvec; c0 += GV * kWave) {
      VT v[GV];
#pragma unroll
      for (int i = 0; i < GV; i++)
        if (c0 + i * kWave < nvec) v[i] = src[c0 + i * kWave];
#pragma unroll
      for (int i = 0; i < GV; i++)
        if (c0 + i * kWave < nvec) dst[c0 + i * kWave] = v[i];
    }
  }
}

}  // namespace moe

namespace moe_host {
using namespace moe;

hipError_t launch_dispatch_count(const int32_t *ids, int64_t T, int E, int k, int32_t *hist,
                                 hipStream_t s) {
  const int nblk = (int)((T + DBT - 1) / DBT);
  if (nblk > 0)
    MOE_LAUNCH("dispatch_count", dispatch_count_kernel, dim3(nblk), dim3(256), 0, s, ids, T, E, k,
               hist);
  return hipGetLastError();
}

hipError_t launch_scan_aux(const int32_t *hist, const float *qsum, const int32_t *fcount,
                           int nblk, int E, int64_t T, int64_t C, int32_t *offs, int32_t *load,
                           int32_t *kept, double *term, hipStream_t s) {
  MOE_LAUNCH("scan_aux", scan_aux_kernel, dim3(E), dim3(256), 0, s, hist, qsum, fcount, nblk, E,
             T, C, offs, load, kept, term);
  return hipGetLastError();
}

hipError_t launch_dispatch_place(const int32_t *ids, const int32_t *offs, int64_t T, int E, int k,
                                 int64_t C, int32_t *slots, uint8_t *drop, const double *aux_term,
                                 float aux_alpha, float *aux, hipStream_t s, const float *gates,
                                 const int32_t *load, int32_t *seg, int32_t *src) {
  const int nblk = (int)((T + DBT - 1) / DBT);
  if (nblk > 0)
    MOE_LAUNCH("dispatch_place", dispatch_place_kernel, dim3(nblk), dim3(64), 0, s, ids, offs, T,
               E, k, C, slots, drop, aux_term, aux_alpha, aux, load, seg, seg ? nullptr : src);
  else if (aux)
    return launch_aux_sum(aux_term, E, aux_alpha, aux, s);
  if (seg && T > 0) {
    MOE_LAUNCH("select_gate", select_gate_kernel, dim3(E), dim3(256), 0, s, seg, gates, load, E, C,
               slots, drop);
    // tiles of 256 kept positions, at most T*k/256 + E of them
    const int64_t tiles = (T * k + 255) / 256 + E;
    MOE_LAUNCH("rank_gate", rank_gate_kernel, dim3((unsigned)tiles), dim3(256), 0, s, seg, gates,
               load, E, C, slots, drop);
  }
  return hipGetLastError();
}

hipError_t launch_gather(const void *x, const int32_t *ids, const int32_t *slots, int64_t T, int k,
                         int64_t C, int64_t row_bytes, void *x_disp, hipStream_t s) {
  const int64_t n = T * k;
  if (n <= 0) return hipGetLastError();
  int64_t blocks = (n + 3) / 4;
  if (blocks > 16384) blocks = 16384;
  if (row_bytes % 16 == 0)
    MOE_LAUNCH("gather_x16", gather_kernel<u32x4>, dim3((unsigned)blocks), dim3(256), 0, s,
               (const char *)x, ids, slots, n, k, C, row_bytes, (char *)x_disp);
  else
    MOE_LAUNCH("gather_x4", gather_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, s,
               (const char *)x, ids, slots, n, k, C, row_bytes, (char *)x_disp);
  return hipGetLastError();
}

}  // namespace moe_host
