// api.hip -- the C ABI declared in include/moe.h: argument validation (all of
// it before anything is enqueued), capacity, workspace layout, the launch
// sequence of each entry point, and the optional per-kernel event timing.
#include <math.h>
#include <string.h>

#include <mutex>
#include <set>
#include <string>
#include <vector>

#include "../../include/moe.h"
#include "common.h"
#include "kernels.h"

using namespace moe;

namespace {

constexpr int64_t kMaxTokens = int64_t(1) << 30;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

size_t act_size(const moe_config *c) { return c->act_dtype == MOE_F32 ? 4 : 2; }

int check_config(const moe_config *c) {
  if (!c) return MOE_ERR_INVALID_ARG;
  if (c->T < 0 || c->d < 1 || c->E < 1 || c->k < 1 || c->k > c->E || c->d_ff < 1)
    return MOE_ERR_INVALID_ARG;
  if (c->act_dtype != MOE_F32 && c->act_dtype != MOE_BF16) return MOE_ERR_INVALID_ARG;
  if (c->expert_wfmt != MOE_W_PLAIN && c->expert_wfmt != MOE_W_INT8_G128 &&
      c->expert_wfmt != MOE_W_BF16_PACKED)
    return MOE_ERR_INVALID_ARG;
  if ((c->normalize_topk | c->pr_moe | c->add_skip | c->read_x_rows) & ~1) return MOE_ERR_INVALID_ARG;
  if (c->capacity < 0) return MOE_ERR_INVALID_ARG;
  if (c->capacity == 0 && !(c->capacity_factor > 0.0 && isfinite(c->capacity_factor)))
    return MOE_ERR_INVALID_ARG;
  if (c->pr_moe && c->d_ff_dense < 1) return MOE_ERR_INVALID_ARG;
  if (!isfinite(c->aux_alpha)) return MOE_ERR_INVALID_ARG;
  if (c->drop_policy != MOE_DROP_TOKEN_ORDER && c->drop_policy != MOE_DROP_GATE_PRIORITY)
    return MOE_ERR_INVALID_ARG;
  if (c->router < MOE_ROUTER_TOPK || c->router > MOE_ROUTER_NOISY_TOPK) return MOE_ERR_INVALID_ARG;
  if (!isfinite(c->w_importance) || !isfinite(c->w_load)) return MOE_ERR_INVALID_ARG;
  if (c->router == MOE_ROUTER_TOP_P && !(c->top_p > 0.f && isfinite(c->top_p)))
    return MOE_ERR_INVALID_ARG;
  if (c->router == MOE_ROUTER_COSINE &&
      (!(c->cos_tau > 0.f && isfinite(c->cos_tau)) || c->cos_dim < 1 || c->cos_dim > 256))
    return MOE_ERR_INVALID_ARG;
  if (c->router == MOE_ROUTER_NOISY_TOPK && c->E > 128) return MOE_ERR_UNSUPPORTED;
  if (c->E > 256 || c->k > 8 || c->T > kMaxTokens) return MOE_ERR_UNSUPPORTED;
  if (c->T * c->k >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;  // int32 slots/positions
  if (c->d > (1 << 20) || c->d_ff > (1 << 20) || c->d_ff_dense > (1 << 20))
    return MOE_ERR_UNSUPPORTED;
  if (c->act_dtype == MOE_BF16) {
    if (c->d % 64 || c->d_ff % 64 || (c->pr_moe && c->d_ff_dense % 64))
      return MOE_ERR_UNSUPPORTED;
  }
  if (c->expert_wfmt == MOE_W_INT8_G128 || c->expert_wfmt == MOE_W_BF16_PACKED) {
    if (c->act_dtype != MOE_BF16 || c->d % 128 || c->d_ff % 128) return MOE_ERR_UNSUPPORTED;
  }
  return MOE_OK;
}

int64_t capacity_of(const moe_config *c) {
  int64_t C;
  if (c->capacity > 0)
    C = c->capacity;
  else
    C = (int64_t)ceil((double)c->k * (double)c->T * c->capacity_factor / (double)c->E);
  if (C > c->T) C = c->T;
  if (C < 0) C = 0;
  return C;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// a pointer that must be given when `n` elements are to be read or written
bool need(const void *p, int64_t n, size_t align) {
  if (n <= 0) return true;
  return p != nullptr && aligned(p, align);
}
bool opt(const void *p, size_t align) { return p == nullptr || aligned(p, align); }

// ---- workspace layout
struct Layout {
  size_t qsum, fcount, hist, offs, term, zpart, seg, x_disp, y_disp, hidden, hidden_dense, dense,
      xsched, rpart, src, total;  // src: 0 = not in this layout
  // router variants
  size_t scores, cosl, embn, imp, loadp;
  // backward
  size_t dg, fcnt, ecount, dlog, dlog16, dY, Z, H, dZ, dX, dxr, Zd, Hd, dZd, dxd;
};

// layout() selector of the allocation-free layer forward (not a C ABI entry)
constexpr int kEntryLayerScratch = 100;

int64_t padded_experts(const moe_config *c) { return (c->E + 7) / 8 * 8; }

// int8 expert GEMMs on 256-row tiles with enough experts to balance: their
// tiles follow a per-call XCD schedule (16 E + 16 int32 of workspace)
bool sched_experts(const moe_config *c) {
  return c->expert_wfmt == MOE_W_INT8_G128 && c->act_dtype == MOE_BF16 && capacity_of(c) > 128 &&
         c->E >= 32 && c->E <= 256;
}
size_t sched_bytes(const moe_config *c) { return (size_t)(16 * c->E + 16) * 4; }

static_assert(MOE_ROUTER_TOPK == moe::RV_TOPK && MOE_ROUTER_TOP_P == moe::RV_TOP_P &&
                  MOE_ROUTER_COSINE == moe::RV_COSINE && MOE_ROUTER_NOISY_TOPK == moe::RV_NOISY,
              "router ids");

// the router runs as raw products + a variant epilogue (router_var.hip)
// instead of the fused softmax-TopK router
bool variant_router(const moe_config *c) {
  return c->router != MOE_ROUTER_TOPK || c->w_importance != 0.f || c->w_load != 0.f;
}

// columns of the raw product: E, 2E (gate and noise scale) or the projection
int64_t score_cols(const moe_config *c) {
  if (c->router == MOE_ROUTER_NOISY_TOPK) return 2 * c->E;
  if (c->router == MOE_ROUTER_COSINE) return c->cos_dim;
  return c->E;
}

Layout layout(const moe_config *c, int entry) {
  Layout L{};
  const int64_t nblk = moe_host::router_blocks(c->T);
  const size_t blkE = align256((size_t)nblk * (size_t)c->E * 4);
  const size_t termE = (size_t)c->E * sizeof(double);
  const int64_t C = capacity_of(c);
  const size_t as = act_size(c);
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o += align256(bytes);
    return at;
  };
  const bool gp = c->drop_policy == MOE_DROP_GATE_PRIORITY;
  const size_t segB = (size_t)c->T * (size_t)c->k * 4;
  // split-K partial products of the fused router (few token blocks)
  const int rsplit = variant_router(c) ? 1 : moe_host::router_splits(c->T, (int)c->d,
                                                                     c->act_dtype == MOE_BF16);
  const size_t rpartB = rsplit > 1 ? (size_t)rsplit * nblk * 64 * ((c->E + 31) / 32 * 32) * 4 : 0;
  auto take_variant = [&]() {
    if (!variant_router(c)) return;
    L.scores = take((size_t)c->T * score_cols(c) * 4);
    if (c->router == MOE_ROUTER_COSINE) {
      L.cosl = take((size_t)c->T * c->E * 4);
      L.embn = take((size_t)c->E * c->cos_dim * 4);
    }
    L.imp = take(blkE);
    L.loadp = take(blkE);
  };
  switch (entry) {
    case MOE_ENTRY_ROUTE:
      L.qsum = take(blkE);
      L.fcount = take(blkE);
      L.term = take(termE);
      L.zpart = take((size_t)nblk * 4);
      if (rpartB) L.rpart = take(rpartB);
      take_variant();
      break;
    case MOE_ENTRY_DISPATCH:
      L.hist = take(blkE);
      L.offs = take(blkE);
      if (gp) L.seg = take(segB);
      break;
    case MOE_ENTRY_EXPERT_FFN:
      L.hidden = take((size_t)c->E * C * c->d_ff * as);
      if (sched_experts(c)) L.xsched = take(sched_bytes(c));
      break;
    case MOE_ENTRY_COMBINE:
      break;
    case MOE_ENTRY_LAYER:
    case kEntryLayerScratch: {
      // kEntryLayerScratch: the allocation-free layer, whose caller gives
      // x_disp, y_disp, the hidden rows and (PR-MoE) D(x) and its hidden
      const bool big = entry == MOE_ENTRY_LAYER;
      L.qsum = take(blkE);
      L.fcount = take(blkE);
      L.hist = take(blkE);
      L.offs = take(blkE);
      L.term = take(termE);
      L.zpart = take((size_t)nblk * 4);
      if (rpartB) L.rpart = take(rpartB);
      take_variant();
      if (gp) L.seg = take(segB);
      if (big) {
        L.src = take((size_t)c->E * C * 4);
        L.x_disp = take((size_t)c->E * C * c->d * as);
        L.y_disp = take((size_t)c->E * C * c->d * as);
        L.hidden = take((size_t)c->E * C * c->d_ff * as);
        if (c->pr_moe) {
          L.hidden_dense = take((size_t)c->T * c->d_ff_dense * as);
          L.dense = take((size_t)c->T * c->d * as);
        }
      }
      if (sched_experts(c)) L.xsched = take(sched_bytes(c));
      break;
    }
    case MOE_ENTRY_BACKWARD: {
      const size_t TB = (size_t)c->T, ECd = (size_t)c->E * C * c->d * as;
      const size_t ECF = (size_t)c->E * C * c->d_ff * as;
      L.dg = take(TB * c->k * 4);
      L.fcnt = take((size_t)c->E * 4);
      L.ecount = take(4);
      L.dlog = take(TB * c->E * 4);
      L.dlog16 = take(TB * padded_experts(c) * as);
      L.dY = take(ECd);
      L.Z = take(ECF);
      L.H = take(ECF);
      L.dZ = take(ECF);
      L.dX = take(ECd);
      L.dxr = take(TB * c->d * as);
      if (c->pr_moe) {
        L.Zd = take(TB * c->d_ff_dense * as);
        L.Hd = take(TB * c->d_ff_dense * as);
        L.dZd = take(TB * c->d_ff_dense * as);
        L.dxd = take(TB * c->d * as);
      }
      break;
    }
    default:
      break;
  }
  L.total = o;
  return L;
}

int check_ws(const moe_config *c, int entry, void *ws, size_t ws_bytes) {
  const size_t need_b = layout(c, entry).total;
  if (need_b == 0) return MOE_OK;
  if (!ws || ws_bytes < need_b || !aligned(ws, 16)) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

char *at(void *ws, size_t off) { return (char *)ws + off; }

// ---- launch sequences (arguments already validated)
hipError_t do_router(const moe_config *c, const void *x, const void *wr, const float *br,
                     int32_t *ids, float *gates, float *logits, float *qsum, int32_t *fcount,
                     int32_t *hist, float *zpart, float *z_loss, float *rpart, hipStream_t s) {
  RouterArgs a{};
  a.part = rpart;
  a.x = x;
  a.w = wr;
  a.bias = br;
  a.ids = ids;
  a.gates = gates;
  a.logits = logits;
  a.qsum = qsum;
  a.fcount = fcount;
  a.hist = hist;
  a.T = c->T;
  a.d = (int)c->d;
  a.E = (int)c->E;
  a.k = (int)c->k;
  a.normalize = c->normalize_topk;
  a.zpart = z_loss ? zpart : nullptr;
  hipError_t e = moe_host::launch_router(a, c->act_dtype == MOE_BF16, s);
  if (e == hipSuccess && z_loss)
    e = moe_host::launch_zloss_sum(zpart, moe_host::router_blocks(c->T), c->T, z_loss, s);
  return e;
}

// any router: the fused softmax-TopK router, or raw products -> (cosine
// logits) -> the variant epilogue; imp_loss / load_loss optional
hipError_t do_router_v(const moe_config *c, const Layout &L, void *ws, const void *x,
                       const moe_weights *w, int32_t *ids, float *gates, float *logits,
                       float *qsum, int32_t *fcount, int32_t *hist, float *zpart, float *z_loss,
                       float *imp_loss, float *load_loss, hipStream_t s) {
  if (!variant_router(c))
    return do_router(c, x, w->w_router, w->b_router, ids, gates, logits, qsum, fcount, hist,
                     zpart, z_loss, L.rpart ? (float *)at(ws, L.rpart) : nullptr, s);
  const int bf = c->act_dtype == MOE_BF16, E = (int)c->E;
  const int nblk = moe_host::router_blocks(c->T);
  float *scores = (float *)at(ws, L.scores);
  RouterArgs ra{};
  ra.x = x;
  ra.T = c->T;
  ra.d = (int)c->d;
  ra.k = (int)c->k;
  ra.logits = scores;
  ra.E = (int)score_cols(c);
  ra.nw1 = ra.E;
  if (c->router == MOE_ROUTER_COSINE) {
    ra.w = w->w_proj;
  } else {
    ra.w = w->w_router;
    if (c->router == MOE_ROUTER_NOISY_TOPK) {
      ra.w2 = w->w_noise;
      ra.nw1 = E;
    }
  }
  hipError_t e = moe_host::launch_router_scores(ra, bf, s);
  const float *src = scores;
  if (e == hipSuccess && c->router == MOE_ROUTER_COSINE) {
    float *embn = (float *)at(ws, L.embn), *cosl = (float *)at(ws, L.cosl);
    e = moe_host::launch_emb_normalize(w->expert_emb, bf, E, c->cos_dim, embn, s);
    if (e == hipSuccess)
      e = moe_host::launch_cosine_logits(scores, embn, c->T, E, c->cos_dim, 1.f / c->cos_tau,
                                         cosl, s);
    src = cosl;
  }
  RouteVarArgs va{};
  va.src = src;
  va.noise = w->noise;
  va.bias = w->b_router;
  va.ids = ids;
  va.gates = gates;
  va.logits = logits;
  va.qsum = qsum;
  va.fcount = fcount;
  va.hist = hist;
  va.zpart = z_loss ? zpart : nullptr;
  va.imp = (float *)at(ws, L.imp);
  va.loadp = (float *)at(ws, L.loadp);
  va.T = c->T;
  va.E = E;
  va.k = (int)c->k;
  va.normalize = c->normalize_topk;
  va.variant = c->router;
  va.top_p = c->top_p;
  if (e == hipSuccess) e = moe_host::launch_route_logits(va, s);
  if (e == hipSuccess && z_loss) e = moe_host::launch_zloss_sum(zpart, nblk, c->T, z_loss, s);
  if (e == hipSuccess && (imp_loss || load_loss))  // T = 0: no blocks, both losses 0
    e = moe_host::launch_cov_loss(va.imp, va.loadp, nblk, E, c->w_importance, c->w_load,
                                  imp_loss, load_loss, s);
  return e;
}

// the router's weights and inputs for cfg->router
bool router_weights_ok(const moe_config *c, const moe_weights *w) {
  if (!opt(w->b_router, 4)) return false;
  if (c->router == MOE_ROUTER_COSINE)
    return need(w->w_proj, 1, 16) && need(w->expert_emb, 1, 16);
  if (!need(w->w_router, 1, 16)) return false;
  if (c->router == MOE_ROUTER_NOISY_TOPK)
    return need(w->w_noise, 1, 16) && need(w->noise, c->T * c->E, 4);
  return true;
}

// loss outputs need their weights
bool loss_outputs_ok(const moe_config *c, const moe_outputs *o) {
  if (!opt(o->importance_loss, 4) || !opt(o->load_loss, 4)) return false;
  if (o->importance_loss && c->w_importance == 0.f) return false;
  if (o->load_loss && c->w_load == 0.f) return false;
  return true;
}

// place slots (token order, or gate priority through the segment array
// `seg`, which needs gates and load) and gather the kept rows; hist/offs are
// the per-block counts and offsets ([E][blocks]); aux_term non-null -> the
// place kernel also finishes the aux loss.  src non-null (token order): the
// slot -> token table is written instead of the gathered rows.
hipError_t do_place_gather(const moe_config *c, const void *x, const int32_t *ids,
                           const float *gates, const int32_t *offs, const int32_t *load,
                           int32_t *seg, int32_t *slots, uint8_t *drop, const double *aux_term,
                           float *aux, void *x_disp, hipStream_t s, int32_t *src = nullptr) {
  const int64_t C = capacity_of(c);
  const bool gp = c->drop_policy == MOE_DROP_GATE_PRIORITY;
  if (gp && src) return hipErrorInvalidValue;
  hipError_t e = moe_host::launch_dispatch_place(ids, offs, c->T, (int)c->E, (int)c->k, C, slots,
                                                 drop, aux_term, c->aux_alpha, aux, s,
                                                 gp ? gates : nullptr, gp ? load : nullptr,
                                                 gp ? seg : nullptr, src);
  if (e != hipSuccess || src) return e;
  return moe_host::launch_gather(x, ids, slots, c->T, (int)c->k, C,
                                 c->d * (int64_t)act_size(c), x_disp, s);
}

// hidden: GELU(W1 x) of the kept rows; zpre: W1 x itself, or null (not kept);
// xsched: workspace for the XCD schedule of the int8 tiles (sched_experts),
// or null; asrc: the slot -> token table, with x_disp then the token rows x
hipError_t do_expert_ffn(const moe_config *c, const void *x_disp, const int32_t *kept,
                         const void *w1, const void *s1, const void *w2, const void *s2,
                         void *y_disp, void *hidden, hipStream_t s, void *zpre = nullptr,
                         int32_t *xsched = nullptr, const int32_t *asrc = nullptr) {
  const int64_t C = capacity_of(c);
  if (C == 0) return hipSuccess;
  const int bf = c->act_dtype == MOE_BF16, q8 = c->expert_wfmt == MOE_W_INT8_G128;
  hipError_t e = hipSuccess;
  if (xsched && sched_experts(c)) {
    e = moe_host::launch_tile_sched(kept, (int)c->E, C, c->d % 512 == 0 && c->d_ff % 512 == 0,
                                    xsched, s);
    if (e != hipSuccess) return e;
  } else {
    xsched = nullptr;
  }
  const int pk = c->expert_wfmt == MOE_W_BF16_PACKED;
  GemmArgs g1{x_disp, w1, s1, hidden, kept, C, (int)c->d_ff, (int)c->d, (int)c->E, zpre, xsched,
              pk};
  g1.asrc = asrc;
  e = moe_host::launch_gemm(g1, bf, q8, 1, "expert_ffn1", s);
  if (e != hipSuccess) return e;
  GemmArgs g2{hidden, w2, s2, y_disp, kept, C, (int)c->d, (int)c->d_ff, (int)c->E, nullptr, xsched,
              pk};
  return moe_host::launch_gemm(g2, bf, q8, 0, "expert_ffn2", s);
}

hipError_t do_dense(const moe_config *c, const void *x, const void *wm1, const void *wm2,
                    void *out, void *hidden, hipStream_t s, void *zpre = nullptr) {
  if (c->T == 0) return hipSuccess;
  const int bf = c->act_dtype == MOE_BF16;
  GemmArgs g1{x, wm1, nullptr, hidden, nullptr, c->T, (int)c->d_ff_dense, (int)c->d, 1, zpre};
  hipError_t e = moe_host::launch_gemm(g1, bf, 0, 1, "dense_mlp1", s);
  if (e != hipSuccess) return e;
  GemmArgs g2{hidden, wm2, nullptr, out, nullptr, c->T, (int)c->d, (int)c->d_ff_dense, 1};
  return moe_host::launch_gemm(g2, bf, 0, 0, "dense_mlp2", s);
}

// ---- profiling records
struct ProfRec {
  const char *name;
  hipEvent_t a, b;
};
bool g_prof = false;
bool g_open = false;       // a record was begun for the launch in flight
std::string g_only;        // profile only launches of this name ("" = all)
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;

hipEvent_t pool_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

}  // namespace

namespace moe_host {
const char *intern_name(const char *a, const char *b) {
  static std::mutex mu;
  static std::set<std::string> names;  // host-side, grows with distinct names only
  std::lock_guard<std::mutex> lock(mu);
  return names.insert(std::string(a) + ":" + b).first->c_str();
}

void prof_begin(hipStream_t s, const char *name) {
  g_open = false;
  if (!g_prof || (!g_only.empty() && g_only != name)) return;
  ProfRec r{name, pool_event(), pool_event()};
  if (r.a) (void)hipEventRecord(r.a, s);
  g_recs.push_back(r);
  g_open = true;
}
void prof_end(hipStream_t s) {
  if (!g_open || g_recs.empty()) return;
  g_open = false;
  if (g_recs.back().b) (void)hipEventRecord(g_recs.back().b, s);
}
}  // namespace moe_host

// ---- scratch of the allocation-free layer forward
// Per-device scratch of moe_layer_forward_noalloc: a file-scope device array
// of MOE_NOALLOC_SCRATCH_BYTES (each GPU the library runs on holds its own
// copy until the process ends).  Host code never passes `scratch` itself to a
// kernel (on the host it only names the symbol); it uses the device address
// that hipGetSymbolAddress returns, taken once per device on that device's
// first call and kept in g_scratch_ptr.  Nothing in it needs to start at
// zero: every kernel writes the scratch it reads earlier in the same call.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_address(void **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace

extern "C" {

int64_t moe_capacity(const moe_config *cfg) {
  const int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  return capacity_of(cfg);
}

size_t moe_workspace_bytes(const moe_config *cfg, int entry) {
  if (check_config(cfg) != MOE_OK) return 0;
  if (entry < MOE_ENTRY_ROUTE || entry > MOE_ENTRY_BACKWARD) return 0;
  return layout(cfg, entry).total;
}

int moe_route(const moe_config *cfg, const void *x, const void *w_router, const float *b_router,
              int32_t *expert_ids, float *gates, float *logits, float *aux_loss, float *z_loss,
              void *ws, size_t ws_bytes, void *stream) {
  int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  if (cfg->router != MOE_ROUTER_TOPK) return MOE_ERR_UNSUPPORTED;
  const int64_t T = cfg->T, Tk = T * cfg->k;
  if (!need(x, T, 16) || !need(w_router, 1, 16) || !opt(b_router, 4) ||
      !need(expert_ids, Tk, 4) || !need(gates, Tk, 4) || !opt(logits, 4) ||
      !need(aux_loss, 1, 4) || !opt(z_loss, 4))
    return MOE_ERR_INVALID_ARG;
  rc = check_ws(cfg, MOE_ENTRY_ROUTE, ws, ws_bytes);
  if (rc != MOE_OK) return rc;
  const Layout L = layout(cfg, MOE_ENTRY_ROUTE);
  hipStream_t s = (hipStream_t)stream;
  float *qsum = (float *)at(ws, L.qsum);
  int32_t *fcount = (int32_t *)at(ws, L.fcount);
  double *term = (double *)at(ws, L.term);
  hipError_t e = do_router(cfg, x, w_router, b_router, expert_ids, gates, logits, qsum, fcount,
                           nullptr, (float *)at(ws, L.zpart), z_loss,
                           L.rpart ? (float *)at(ws, L.rpart) : nullptr, s);
  if (e == hipSuccess)
    e = moe_host::launch_scan_aux(nullptr, qsum, fcount, moe_host::router_blocks(T),
                                  (int)cfg->E, T, 0, nullptr, nullptr, nullptr, term, s);
  if (e == hipSuccess) e = moe_host::launch_aux_sum(term, (int)cfg->E, cfg->aux_alpha, aux_loss, s);
  return hip_status(e);
}

int moe_route_ex(const moe_config *cfg, const void *x, const moe_weights *w, moe_outputs *out,
                 void *ws, size_t ws_bytes, void *stream) {
  int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  if (!w || !out) return MOE_ERR_INVALID_ARG;
  const int64_t T = cfg->T, Tk = T * cfg->k;
  if (!need(x, T, 16) || !router_weights_ok(cfg, w) || !need(out->expert_ids, Tk, 4) ||
      !need(out->gates, Tk, 4) || !opt(out->logits, 4) || !need(out->aux_loss, 1, 4) ||
      !opt(out->z_loss, 4) || !loss_outputs_ok(cfg, out))
    return MOE_ERR_INVALID_ARG;
  rc = check_ws(cfg, MOE_ENTRY_ROUTE, ws, ws_bytes);
  if (rc != MOE_OK) return rc;
  const Layout L = layout(cfg, MOE_ENTRY_ROUTE);
  hipStream_t s = (hipStream_t)stream;
  float *qsum = (float *)at(ws, L.qsum);
  int32_t *fcount = (int32_t *)at(ws, L.fcount);
  double *term = (double *)at(ws, L.term);
  hipError_t e = do_router_v(cfg, L, ws, x, w, out->expert_ids, out->gates, out->logits, qsum,
                             fcount, nullptr, (float *)at(ws, L.zpart), out->z_loss,
                             out->importance_loss, out->load_loss, s);
  if (e == hipSuccess)
    e = moe_host::launch_scan_aux(nullptr, qsum, fcount, moe_host::router_blocks(T),
                                  (int)cfg->E, T, 0, nullptr, nullptr, nullptr, term, s);
  if (e == hipSuccess)
    e = moe_host::launch_aux_sum(term, (int)cfg->E, cfg->aux_alpha, out->aux_loss, s);
  return hip_status(e);
}

int moe_dispatch(const moe_config *cfg, const void *x, const int32_t *expert_ids,
                 const float *gates, int32_t *slots, uint8_t *drop_mask, int32_t *load,
                 int32_t *kept, void *x_disp, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  const int64_t T = cfg->T, Tk = T * cfg->k, C = capacity_of(cfg);
  const bool gp = cfg->drop_policy == MOE_DROP_GATE_PRIORITY;
  if (!need(x, T, 16) || !need(expert_ids, Tk, 4) || !need(slots, Tk, 4) || !opt(drop_mask, 1) ||
      !need(load, 1, 4) || !need(kept, 1, 4) || !need(x_disp, cfg->E * C, 16) ||
      (gp ? !need(gates, Tk, 4) : !opt(gates, 4)))
    return MOE_ERR_INVALID_ARG;
  rc = check_ws(cfg, MOE_ENTRY_DISPATCH, ws, ws_bytes);
  if (rc != MOE_OK) return rc;
  const Layout L = layout(cfg, MOE_ENTRY_DISPATCH);
  hipStream_t s = (hipStream_t)stream;
  int32_t *hist = (int32_t *)at(ws, L.hist), *offs = (int32_t *)at(ws, L.offs);
  hipError_t e = moe_host::launch_dispatch_count(expert_ids, T, (int)cfg->E, (int)cfg->k, hist, s);
  if (e == hipSuccess)
    e = moe_host::launch_scan_aux(hist, nullptr, nullptr, moe_host::router_blocks(T), (int)cfg->E,
                                  T, C, offs, load, kept, nullptr, s);
  if (e == hipSuccess)
    e = do_place_gather(cfg, x, expert_ids, gates, offs, load,
                        gp ? (int32_t *)at(ws, L.seg) : nullptr, slots, drop_mask, nullptr,
                        nullptr, x_disp, s);
  return hip_status(e);
}

int moe_expert_ffn(const moe_config *cfg, const void *x_disp, const int32_t *kept, const void *w1,
                   const void *w1_scale, const void *w2, const void *w2_scale, void *y_disp,
                   void *ws, size_t ws_bytes, void *stream) {
  int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  const int64_t rowsE = cfg->E * capacity_of(cfg);
  const bool q8 = cfg->expert_wfmt == MOE_W_INT8_G128;
  if (!need(x_disp, rowsE, 16) || !need(kept, 1, 4) || !need(w1, 1, 16) || !need(w2, 1, 16) ||
      !need(y_disp, rowsE, 16))
    return MOE_ERR_INVALID_ARG;
  if (q8 ? (!need(w1_scale, 1, 2) || !need(w2_scale, 1, 2)) : (w1_scale || w2_scale))
    return MOE_ERR_INVALID_ARG;
  rc = check_ws(cfg, MOE_ENTRY_EXPERT_FFN, ws, ws_bytes);
  if (rc != MOE_OK) return rc;
  const Layout L = layout(cfg, MOE_ENTRY_EXPERT_FFN);
  int32_t *xs = sched_experts(cfg) ? (int32_t *)at(ws, L.xsched) : nullptr;
  return hip_status(do_expert_ffn(cfg, x_disp, kept, w1, w1_scale, w2, w2_scale, y_disp,
                                  at(ws, L.hidden), (hipStream_t)stream, nullptr, xs));
}

int moe_dense_mlp(const moe_config *cfg, const void *x, const void *wm1, const void *wm2,
                  void *dense_out, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  if (!cfg->pr_moe) return MOE_ERR_INVALID_ARG;
  const int64_t T = cfg->T;
  if (!need(x, T, 16) || !need(wm1, 1, 16) || !need(wm2, 1, 16) || !need(dense_out, T, 16))
    return MOE_ERR_INVALID_ARG;
  const size_t hid = (size_t)T * cfg->d_ff_dense * act_size(cfg);
  if (hid > 0 && (!ws || ws_bytes < hid || !aligned(ws, 16))) return MOE_ERR_WORKSPACE;
  return hip_status(do_dense(cfg, x, wm1, wm2, dense_out, ws, (hipStream_t)stream));
}

int moe_combine(const moe_config *cfg, const void *y_disp, const int32_t *expert_ids,
                const int32_t *slots, const float *gates, const void *base, const void *base2,
                void *y, void *stream) {
  int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  const int64_t T = cfg->T, Tk = T * cfg->k;
  if (!need(expert_ids, Tk, 4) || !need(slots, Tk, 4) || !need(gates, Tk, 4) ||
      !opt(base, 16) || !opt(base2, 16) || !need(y, T, 16) ||
      !need(y_disp, cfg->E * capacity_of(cfg) > 0 ? Tk : 0, 16))
    return MOE_ERR_INVALID_ARG;
  return hip_status(moe_host::launch_combine(y_disp, expert_ids, slots, gates, base, base2, y, T,
                                             (int)cfg->d, (int)cfg->k, capacity_of(cfg),
                                             (int)cfg->E, cfg->act_dtype == MOE_BF16,
                                             (hipStream_t)stream));
}

// PR-MoE: the dense MLP depends only on x, the expert path only on x and the
// router, so the layer forks the dense MLP (MFMA-bound) onto a second stream
// beside the expert path (weight-streaming) and joins it before the combine.
// One non-blocking side stream (default priority) and one fork/join event
// pair per device, created on first use and kept for the life of the process;
// the mutex keeps the record/wait pairs of concurrent callers from
// interleaving (their dense MLPs queue on the one side stream).
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
static std::mutex g_side_mu;
static std::vector<SideStream> g_side;

static hipError_t side_stream(SideStream **out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if ((int)g_side.size() <= dev) g_side.resize(dev + 1);
  SideStream &r = g_side[dev];
  if (!r.s) {
    e = hipStreamCreateWithFlags(&r.s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&r.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&r.join, hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  *out = &r;
  return hipSuccess;
}

// argument checks of the layer forward (both entry points)
static int check_layer_args(const moe_config *cfg, const void *x, const moe_weights *w,
                     const moe_outputs *out) {
  if (!w || !out) return MOE_ERR_INVALID_ARG;
  const int64_t T = cfg->T, Tk = T * cfg->k;
  const bool q8 = cfg->expert_wfmt == MOE_W_INT8_G128;
  if (!need(x, T, 16) || !router_weights_ok(cfg, w) || !need(w->w1, 1, 16) ||
      !need(w->w2, 1, 16))
    return MOE_ERR_INVALID_ARG;
  if (q8 ? (!need(w->w1_scale, 1, 2) || !need(w->w2_scale, 1, 2))
         : (w->w1_scale || w->w2_scale))
    return MOE_ERR_INVALID_ARG;
  if (cfg->pr_moe && (!need(w->wm1, 1, 16) || !need(w->wm2, 1, 16))) return MOE_ERR_INVALID_ARG;
  if (!need(out->y, T, 16) || !need(out->expert_ids, Tk, 4) || !need(out->gates, Tk, 4) ||
      !need(out->slots, Tk, 4) || !need(out->load, 1, 4) || !need(out->kept, 1, 4) ||
      !need(out->aux_loss, 1, 4) || !opt(out->drop_mask, 1) || !opt(out->logits, 4) ||
      !opt(out->x_disp, 16) || !opt(out->y_disp, 16) || !opt(out->dense_out, 16) ||
      !opt(out->z_loss, 4) || !opt(out->h_disp, 16) || !opt(out->z_disp, 16) ||
      !opt(out->h_dense, 16) || !opt(out->z_dense, 16) || !loss_outputs_ok(cfg, out))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

// the layer's launch sequence; `L` places the scratch in `ws` (the buffers
// the caller gives in `out` are not taken from it); side_ok: PR-MoE may run
// the dense MLP on the side stream (cfg->overlap_dense)
static hipError_t layer_forward_launch(const moe_config *cfg, const void *x, const moe_weights *w,
                                moe_outputs *out, void *ws, const Layout &L, hipStream_t s,
                                bool side_ok) {
  const int64_t T = cfg->T;
  float *qsum = (float *)at(ws, L.qsum);
  int32_t *fcount = (int32_t *)at(ws, L.fcount), *hist = (int32_t *)at(ws, L.hist);
  int32_t *offs = (int32_t *)at(ws, L.offs);
  void *x_disp = out->x_disp ? out->x_disp : at(ws, L.x_disp);
  void *y_disp = out->y_disp ? out->y_disp : at(ws, L.y_disp);
  void *hidden = out->h_disp ? out->h_disp : at(ws, L.hidden);
  void *dense = nullptr, *hidden_dense = nullptr;
  if (cfg->pr_moe) {
    dense = out->dense_out ? out->dense_out : at(ws, L.dense);
    hidden_dense = out->h_dense ? out->h_dense : at(ws, L.hidden_dense);
  }
  void *zd = cfg->pr_moe ? out->z_dense : nullptr;

  hipError_t e = hipSuccess;
  // fork: the dense MLP on the side stream
  std::unique_lock<std::mutex> side_lock;
  SideStream *side = nullptr;
  if (cfg->pr_moe && cfg->overlap_dense && side_ok && T > 0) {
    side_lock = std::unique_lock<std::mutex>(g_side_mu);
    e = side_stream(&side);
    if (e == hipSuccess) e = hipEventRecord(side->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e == hipSuccess)
      e = do_dense(cfg, x, w->wm1, w->wm2, dense, hidden_dense, side->s, zd);
    if (e == hipSuccess) e = hipEventRecord(side->join, side->s);
  } else if (cfg->pr_moe) {
    e = do_dense(cfg, x, w->wm1, w->wm2, dense, hidden_dense, s, zd);
  }
  // read_x_rows and x_disp not asked for: the first expert GEMM reads the
  // token rows of x through the slot -> token table that placement writes,
  // and no gathered copy is made (token-order dispatch, shapes on the DMA
  // tiles); otherwise the gather builds x_disp
  int32_t *asrc = nullptr;
  if (cfg->read_x_rows && !out->x_disp && L.src && cfg->drop_policy != MOE_DROP_GATE_PRIORITY &&
      capacity_of(cfg) > 0) {
    GemmArgs g1{x, nullptr, nullptr, nullptr, nullptr, capacity_of(cfg), (int)cfg->d_ff,
                (int)cfg->d, (int)cfg->E};
    if (moe_host::gemm_reads_row_table(g1, cfg->act_dtype == MOE_BF16,
                                       cfg->expert_wfmt == MOE_W_INT8_G128, T))
      asrc = (int32_t *)at(ws, L.src);
  }
  double *term = (double *)at(ws, L.term);
  if (e == hipSuccess)
    e = do_router_v(cfg, L, ws, x, w, out->expert_ids, out->gates, out->logits, qsum, fcount,
                    hist, (float *)at(ws, L.zpart), out->z_loss, out->importance_loss,
                    out->load_loss, s);
  if (e == hipSuccess)
    e = moe_host::launch_scan_aux(hist, qsum, fcount, moe_host::router_blocks(T), (int)cfg->E, T,
                                  capacity_of(cfg), offs, out->load, out->kept, term, s);
  if (e == hipSuccess)
    e = do_place_gather(cfg, x, out->expert_ids, out->gates, offs, out->load,
                        cfg->drop_policy == MOE_DROP_GATE_PRIORITY ? (int32_t *)at(ws, L.seg)
                                                                   : nullptr,
                        out->slots, out->drop_mask, term, out->aux_loss, x_disp, s, asrc);
  if (e == hipSuccess)
    e = do_expert_ffn(cfg, asrc ? x : x_disp, out->kept, w->w1, w->w1_scale, w->w2, w->w2_scale,
                      y_disp, hidden, s, out->z_disp,
                      sched_experts(cfg) ? (int32_t *)at(ws, L.xsched) : nullptr, asrc);
  // join: the combine reads D(x)
  if (e == hipSuccess && side) e = hipStreamWaitEvent(s, side->join, 0);
  if (e == hipSuccess)
    e = moe_host::launch_combine(y_disp, out->expert_ids, out->slots, out->gates,
                                 cfg->add_skip ? x : nullptr, dense, out->y, T, (int)cfg->d,
                                 (int)cfg->k, capacity_of(cfg), (int)cfg->E,
                                 cfg->act_dtype == MOE_BF16, s);
  return e;
}

int moe_layer_forward(const moe_config *cfg, const void *x, const moe_weights *w,
                      moe_outputs *out, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  rc = check_layer_args(cfg, x, w, out);
  if (rc != MOE_OK) return rc;
  rc = check_ws(cfg, MOE_ENTRY_LAYER, ws, ws_bytes);
  if (rc != MOE_OK) return rc;
  return hip_status(layer_forward_launch(cfg, x, w, out, ws, layout(cfg, MOE_ENTRY_LAYER),
                                         (hipStream_t)stream, true));
}

size_t moe_layer_forward_noalloc_scratch_bytes(const moe_config *cfg) {
  if (check_config(cfg) != MOE_OK) return 0;
  return layout(cfg, kEntryLayerScratch).total;
}

int moe_layer_forward_noalloc(const moe_config *cfg, const void *x, const moe_weights *w,
                              moe_outputs *out, void *stream) {
  int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  rc = check_layer_args(cfg, x, w, out);
  if (rc != MOE_OK) return rc;
  const int64_t C = capacity_of(cfg);
  const bool rows = cfg->E * C > 0;
  if (!need(out->x_disp, rows, 16) || !need(out->y_disp, rows, 16) ||
      !need(out->h_disp, rows, 16))
    return MOE_ERR_INVALID_ARG;
  if (cfg->pr_moe && (!need(out->dense_out, cfg->T, 16) || !need(out->h_dense, cfg->T, 16)))
    return MOE_ERR_INVALID_ARG;
  const Layout L = layout(cfg, kEntryLayerScratch);
  if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_SCRATCH;
  void *ws = nullptr;
  hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(layer_forward_launch(cfg, x, w, out, ws, L, (hipStream_t)stream, false));
}

int moe_layer_backward(const moe_config *cfg, const void *x, const moe_weights *w,
                       const moe_outputs *fwd, const void *dy, float g_aux, float g_z,
                       moe_grads *gr, void *ws, size_t ws_bytes, void *stream) {
  int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  if (!w || !fwd || !gr) return MOE_ERR_INVALID_ARG;
  if (cfg->act_dtype != MOE_BF16 || cfg->expert_wfmt != MOE_W_PLAIN ||
      cfg->router != MOE_ROUTER_TOPK)
    return MOE_ERR_UNSUPPORTED;
  const int64_t T = cfg->T, Tk = T * cfg->k, E = cfg->E, C = capacity_of(cfg);
  const int64_t d = cfg->d, F = cfg->d_ff, Fd = cfg->d_ff_dense;
  const bool pr = cfg->pr_moe != 0;
  if (!need(x, T, 16) || !need(w->w_router, 1, 16) || !need(w->w1, 1, 16) ||
      !need(w->w2, 1, 16) || (pr && (!need(w->wm1, 1, 16) || !need(w->wm2, 1, 16))))
    return MOE_ERR_INVALID_ARG;
  if (!need(fwd->expert_ids, Tk, 4) || !need(fwd->gates, Tk, 4) || !need(fwd->slots, Tk, 4) ||
      !need(fwd->logits, T, 4) || !need(fwd->x_disp, E * C, 16) || !need(fwd->y_disp, E * C, 16) ||
      !need(dy, T, 16) || !opt(fwd->z_disp, 16) || !opt(fwd->h_disp, 16) ||
      !opt(fwd->z_dense, 16) || !opt(fwd->h_dense, 16))
    return MOE_ERR_INVALID_ARG;
  if (!need(gr->dx, T, 16) || !need(gr->dw_router, 1, 16) || !opt(gr->db_router, 4) ||
      !need(gr->dw1, 1, 16) || !need(gr->dw2, 1, 16) ||
      (pr && (!need(gr->dwm1, 1, 16) || !need(gr->dwm2, 1, 16))))
    return MOE_ERR_INVALID_ARG;
  rc = check_ws(cfg, MOE_ENTRY_BACKWARD, ws, ws_bytes);
  if (rc != MOE_OK) return rc;
  const Layout L = layout(cfg, MOE_ENTRY_BACKWARD);
  hipStream_t s = (hipStream_t)stream;
  using moe::bf16;
  using moe::GenArgs;
  const int Ep = (int)padded_experts(cfg);
  float *dg = (float *)at(ws, L.dg), *dlog = (float *)at(ws, L.dlog);
  int32_t *fcnt = (int32_t *)at(ws, L.fcnt), *ecount = (int32_t *)at(ws, L.ecount);
  bf16 *dlog16 = (bf16 *)at(ws, L.dlog16), *dY = (bf16 *)at(ws, L.dY), *Z = (bf16 *)at(ws, L.Z);
  bf16 *H = (bf16 *)at(ws, L.H), *dZ = (bf16 *)at(ws, L.dZ), *dX = (bf16 *)at(ws, L.dX);
  bf16 *dxr = (bf16 *)at(ws, L.dxr);
  const bf16 *xb = (const bf16 *)x, *dyb = (const bf16 *)dy;
  const int32_t *ids = fwd->expert_ids, *slots = fwd->slots, *kept = fwd->kept;
  const bf16 *xd = (const bf16 *)fwd->x_disp;

  hipError_t e = moe_host::launch_bwd_gate(dyb, (const bf16 *)fwd->y_disp, ids, slots, fwd->gates,
                                           T, (int)cfg->k, (int)d, C, (int)E, dg, dY, s);
  if (e == hipSuccess)
    e = moe_host::launch_bwd_router(fwd->logits, ids, fwd->gates, dg, fcnt, T, (int)E, Ep,
                                    (int)cfg->k, cfg->normalize_topk, cfg->aux_alpha, g_aux, g_z,
                                    dlog, dlog16, gr->db_router, s);
  if (e == hipSuccess) e = moe_host::launch_fill_i32(ecount, 1, (int)E, s);
  // router: dx_r = dlogits W_r, dW_r = dlogits^T x
  if (e == hipSuccess) {
    GenArgs a{};
    a.A = dlog16; a.a_m = Ep; a.a_k = 1;
    a.B = (const bf16 *)w->w_router; a.b_n = 1; a.b_k = d; a.b_kmax = E;
    a.C = dxr; a.c_m = d; a.M = T; a.K = Ep; a.N = (int)d; a.G = 1;
    e = moe_host::launch_gemm_gen(a, false, true, false, "bwd_router_dx", s);
  }
  if (e == hipSuccess) {
    GenArgs a{};
    a.A = dlog16; a.a_m = 1; a.a_k = Ep; a.a_kmax = T;
    a.B = xb; a.b_n = 1; a.b_k = d; a.b_kmax = T;
    a.C = (bf16 *)gr->dw_router; a.c_m = d; a.mrows = ecount; a.M = Ep; a.K = T;
    a.N = (int)d; a.G = 1;
    e = moe_host::launch_gemm_gen(a, true, true, false, "bwd_router_dw", s);
  }
  // experts: the forward's saved W1 x and GELU(W1 x), else recomputed
  if (fwd->z_disp && fwd->h_disp) {
    Z = (bf16 *)fwd->z_disp;
    H = (bf16 *)fwd->h_disp;
  } else {
    if (e == hipSuccess && C > 0) {
      GemmArgs z{xd, w->w1, nullptr, Z, kept, C, (int)F, (int)d, (int)E};
      e = moe_host::launch_gemm(z, 1, 0, 0, "bwd_expert_z", s);
    }
    if (e == hipSuccess) e = moe_host::launch_gelu_map(Z, H, E * C * F, s);
  }
  if (e == hipSuccess && C > 0) {  // dZ = (dY W2) * GELU'(Z)
    GenArgs a{};
    a.A = dY; a.a_g = C * d; a.a_m = d; a.a_k = 1;
    a.B = (const bf16 *)w->w2; a.b_g = d * F; a.b_n = 1; a.b_k = F; a.b_kmax = d;
    a.C = dZ; a.c_g = C * F; a.c_m = F; a.Z = Z; a.mrows = kept; a.M = C; a.K = d;
    a.N = (int)F; a.G = (int)E; a.b_stream = 1;
    e = moe_host::launch_gemm_gen(a, false, true, true, "bwd_expert_dz", s);
  }
  if (e == hipSuccess && C > 0) {  // dX = dZ W1
    GenArgs a{};
    a.A = dZ; a.a_g = C * F; a.a_m = F; a.a_k = 1;
    a.B = (const bf16 *)w->w1; a.b_g = F * d; a.b_n = 1; a.b_k = d; a.b_kmax = F;
    a.C = dX; a.c_g = C * d; a.c_m = d; a.mrows = kept; a.M = C; a.K = F; a.N = (int)d;
    a.G = (int)E; a.b_stream = 1;
    e = moe_host::launch_gemm_gen(a, false, true, false, "bwd_expert_dx", s);
  }
  if (e == hipSuccess) {  // dW2 = dY^T H  (K = kept rows of the expert)
    GenArgs a{};
    a.A = dY; a.a_g = C * d; a.a_m = 1; a.a_k = d; a.a_kmax = C;
    a.B = H; a.b_g = C * F; a.b_n = 1; a.b_k = F; a.b_kmax = C;
    a.C = (bf16 *)gr->dw2; a.c_g = d * F; a.c_m = F; a.M = d; a.krows = kept; a.K = C;
    a.N = (int)F; a.G = (int)E;
    e = moe_host::launch_gemm_gen(a, true, true, false, "bwd_expert_dw2", s);
  }
  if (e == hipSuccess) {  // dW1 = dZ^T X
    GenArgs a{};
    a.A = dZ; a.a_g = C * F; a.a_m = 1; a.a_k = F; a.a_kmax = C;
    a.B = xd; a.b_g = C * d; a.b_n = 1; a.b_k = d; a.b_kmax = C;
    a.C = (bf16 *)gr->dw1; a.c_g = F * d; a.c_m = d; a.M = F; a.krows = kept; a.K = C;
    a.N = (int)d; a.G = (int)E;
    e = moe_host::launch_gemm_gen(a, true, true, false, "bwd_expert_dw1", s);
  }
  // PR-MoE dense MLP
  bf16 *dxd = nullptr;
  if (pr && e == hipSuccess) {
    bf16 *Zd = (bf16 *)at(ws, L.Zd), *Hd = (bf16 *)at(ws, L.Hd), *dZd = (bf16 *)at(ws, L.dZd);
    dxd = (bf16 *)at(ws, L.dxd);
    if (fwd->z_dense && fwd->h_dense) {
      Zd = (bf16 *)fwd->z_dense;
      Hd = (bf16 *)fwd->h_dense;
    } else {
      if (T > 0) {
        GemmArgs z{x, w->wm1, nullptr, Zd, nullptr, T, (int)Fd, (int)d, 1};
        e = moe_host::launch_gemm(z, 1, 0, 0, "bwd_dense_z", s);
      }
      if (e == hipSuccess) e = moe_host::launch_gelu_map(Zd, Hd, T * Fd, s);
    }
    if (e == hipSuccess && T > 0) {
      GenArgs a{};
      a.A = dyb; a.a_m = d; a.a_k = 1;
      a.B = (const bf16 *)w->wm2; a.b_n = 1; a.b_k = Fd; a.b_kmax = d;
      a.C = dZd; a.c_m = Fd; a.Z = Zd; a.M = T; a.K = d; a.N = (int)Fd; a.G = 1;
      e = moe_host::launch_gemm_gen(a, false, true, true, "bwd_dense_dz", s);
    }
    if (e == hipSuccess && T > 0) {
      GenArgs a{};
      a.A = dZd; a.a_m = Fd; a.a_k = 1;
      a.B = (const bf16 *)w->wm1; a.b_n = 1; a.b_k = d; a.b_kmax = Fd;
      a.C = dxd; a.c_m = d; a.M = T; a.K = Fd; a.N = (int)d; a.G = 1;
      e = moe_host::launch_gemm_gen(a, false, true, false, "bwd_dense_dx", s);
    }
    if (e == hipSuccess) {
      GenArgs a{};
      a.A = dyb; a.a_m = 1; a.a_k = d; a.a_kmax = T;
      a.B = Hd; a.b_n = 1; a.b_k = Fd; a.b_kmax = T;
      a.C = (bf16 *)gr->dwm2; a.c_m = Fd; a.M = d; a.K = T; a.N = (int)Fd; a.G = 1;
      e = moe_host::launch_gemm_gen(a, true, true, false, "bwd_dense_dw2", s);
    }
    if (e == hipSuccess) {
      GenArgs a{};
      a.A = dZd; a.a_m = 1; a.a_k = Fd; a.a_kmax = T;
      a.B = xb; a.b_n = 1; a.b_k = d; a.b_kmax = T;
      a.C = (bf16 *)gr->dwm1; a.c_m = d; a.M = Fd; a.K = T; a.N = (int)d; a.G = 1;
      e = moe_host::launch_gemm_gen(a, true, true, false, "bwd_dense_dw1", s);
    }
  }
  if (e == hipSuccess)
    e = moe_host::launch_bwd_dx(cfg->add_skip ? dyb : nullptr, dxd, dxr, dX, ids, slots, T,
                                (int)cfg->k, (int)d, C, (int)E, (bf16 *)gr->dx, s);
  return hip_status(e);
}

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_SCRATCH:
      return "configuration needs more scratch than the allocation-free entry point holds";
    default: return "unknown status";
  }
}

int moe_pack_expert_weights(const moe_config *cfg, int which, const void *w, void *w_packed,
                            void *stream) {
  const int rc = check_config(cfg);
  if (rc != MOE_OK) return rc;
  if (which != 1 && which != 2) return MOE_ERR_INVALID_ARG;
  if (cfg->act_dtype != MOE_BF16 || cfg->d % 128 || cfg->d_ff % 128) return MOE_ERR_UNSUPPORTED;
  const int64_t N = which == 1 ? cfg->d_ff : cfg->d, K = which == 1 ? cfg->d : cfg->d_ff;
  const uint64_t bytes = (uint64_t)cfg->E * N * K * 2;
  if (!need(w, 1, 16) || !need(w_packed, 1, 16)) return MOE_ERR_INVALID_ARG;
  const uintptr_t a = (uintptr_t)w, b = (uintptr_t)w_packed;
  if (a < b + bytes && b < a + bytes) return MOE_ERR_INVALID_ARG;  // overlapping buffers
  return hip_status(moe_host::launch_pack_weights(w, w_packed, cfg->E, N, K, (hipStream_t)stream));
}

int moe_profile_enable(int on) {
  g_prof = on != 0;
  return MOE_OK;
}

int moe_profile_filter(const char *name) {
  g_only = name ? name : "";
  return MOE_OK;
}

int moe_profile_reset(void) {
  for (auto &r : g_recs) {
    if (r.b) (void)hipEventSynchronize(r.b);
    if (r.a) g_pool.push_back(r.a);
    if (r.b) g_pool.push_back(r.b);
  }
  g_recs.clear();
  return MOE_OK;
}

int moe_profile_read(char *names, int64_t *launches, double *total_ms, int cap) {
  std::vector<const char *> keys;
  std::vector<int64_t> cnt;
  std::vector<double> ms;
  for (auto &r : g_recs) {
    float t = 0.f;
    if (r.a && r.b && hipEventSynchronize(r.b) == hipSuccess &&
        hipEventElapsedTime(&t, r.a, r.b) == hipSuccess) {
      size_t i = 0;
      while (i < keys.size() && strcmp(keys[i], r.name) != 0) i++;
      if (i == keys.size()) {
        keys.push_back(r.name);
        cnt.push_back(0);
        ms.push_back(0.0);
      }
      cnt[i]++;
      ms[i] += t;
    }
  }
  moe_profile_reset();
  for (size_t i = 0; i < keys.size() && (int)i < cap; i++) {
    if (names) {
      strncpy(names + 64 * i, keys[i], 63);
      names[64 * i + 63] = 0;
    }
    if (launches) launches[i] = cnt[i];
    if (total_ms) total_ms[i] = ms[i];
  }
  return (int)keys.size();
}

}  // extern "C"
