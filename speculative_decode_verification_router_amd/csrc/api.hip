// C ABI of the MoE verify-step library: argument validation, workspace
// carving and the launch sequence on the caller's stream.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "moe_verify.h"
#include "mv_internal.h"
#include "lm_core.h"

#define MV_API extern "C" __attribute__((visibility("default")))

// Workspace of moe_verify_step_noalloc: one array per GPU, loaded with the
// library's code object and held until the process ends.  In host code the
// name stands for a host-side symbol, not a device address: the address of
// each device's copy comes from hipGetSymbolAddress (scratch_on_device).
constexpr size_t kScratchBytes = static_cast<size_t>(16) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

thread_local std::string g_err;
// Polls a fused-launch wait makes before it gives up (mv_set_spin_limit).
std::atomic<int> g_spin_limit{mv::kSpinLimitDefault};

int fail(int code, const char *msg) {
  g_err = msg;
  return code;
}

constexpr int kMaxTokens = 65535;
// Up to this many rows the routing kernel takes one token per block.
constexpr int kOneTokenRouteT = 256;
constexpr int kMaxK = 15;

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Expert-kernel family for a batch of T rows: 16-row tiles streaming the
// weights (up to kMidMinT rows), 64-row tiles (up to kLargeMinT rows, or
// fp32), and the LDS-tiled GEMMs of 256-row tiles (bf16 above kLargeMinT).
enum Path { kSmallTiles, kMidTiles, kGemmTiles };
Path path_for(const mv_config &c, int T) {
  if (T <= mv::kMidMinT) return kSmallTiles;
  if (c.dtype == MV_BF16 && T > mv::kLargeMinT && c.d_model % 256 == 0 && c.d_ff % 128 == 0 &&
      c.n_shared <= 2)
    return kGemmTiles;
  return kMidTiles;
}
int tile_rows(const mv_config &c, int T) {
  switch (path_for(c, T)) {
    case kSmallTiles: return mv::kTileM;
    case kMidTiles: return mv::kMidRows;
    default: return mv::gemm_tile_rows();
  }
}

// Upper bound of the number of expert tiles of tm rows for T tokens.
int max_tiles(const mv_config &c, int T, int tm) {
  const int pairs = T * c.top_k;
  const int busy = pairs < c.n_routed ? pairs : c.n_routed;
  return (pairs + (tm - 1) * busy) / tm + c.n_shared * ((T + tm - 1) / tm);
}
int max_tiles(const mv_config &c, int T) { return max_tiles(c, T, tile_rows(c, T)); }

struct Layout {
  size_t status, hbuf, hbuf2, hbuf3, x, ids, gates, seg, tiles, tinfo, rows, a, slots, argkey, done, bcnt, logits, tdone,
      ol_ctr, ol_args, total;
};

// Words of one set of fused-launch counters: one per tile and one per copy of
// the routing counter, each on its own 256-byte line.
size_t done_set_words(const mv_config &c, int T) {
  return (static_cast<size_t>(max_tiles(c, T, mv::kTileM)) + mv::kRouteCopies) * mv::kDoneStride;
}

Layout layout(const mv_config &c, int T) {
  const size_t es = c.dtype == MV_BF16 ? 2 : 4;
  const size_t nslot = static_cast<size_t>(c.top_k + c.n_shared);
  const size_t ne = static_cast<size_t>(c.n_routed + c.n_shared + 1);
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  // the call's status word, at offset 0 whatever T is (mv_step_status)
  L.status = take(4);
  L.hbuf = take(static_cast<size_t>(T) * c.d_model * es);
  // the combines of a verify step alternate between hidden-state buffers
  L.hbuf2 = take(static_cast<size_t>(T) * c.d_model * es);
  L.hbuf3 = take(static_cast<size_t>(T) * c.d_model * es);
  L.x = take(static_cast<size_t>(T) * c.d_model * es);
  L.ids = take(static_cast<size_t>(T) * c.top_k * 4);
  L.gates = take(static_cast<size_t>(T) * c.top_k * 4);
  L.seg = take(ne * 4);
  L.tiles = take(ne * 4);
  // sized for the smallest tiles so that the workspace grows with T
  L.tinfo = take(static_cast<size_t>(max_tiles(c, T, mv::kTileM)) * 16);
  L.rows = take(static_cast<size_t>(T) * nslot * 4);
  L.a = take(static_cast<size_t>(T) * nslot * c.d_ff * es);
  L.slots = take(static_cast<size_t>(T) * nslot * c.d_model * 4);
  L.argkey = take(static_cast<size_t>(T) * 8);
  L.done = take(4);
  L.bcnt = take(static_cast<size_t>(mv::route_large_blocks(T)) * 64 * 4);
  // router logits of the batches routed to logits, one buffer per layer parity
  L.logits = take(2 * static_cast<size_t>(T) * 64 * 4);
  // two sets of fused-launch counters (tiles, then the routing copies)
  L.tdone = take(2 * done_set_words(c, T) * 4);
  // the one-launch step (batches routed to logits): its counters and arguments
  const bool one = T <= mv::kLogitsMaxT && c.n_layers <= mv::kOneLaunchMaxLayers;
  L.ol_ctr = take(one ? mv::one_launch_counter_words(c.n_layers, max_tiles(c, T, mv::kTileM)) * 4 : 0);
  L.ol_args = take(one ? sizeof(mv::OneLaunchDev) : 0);
  L.total = off;
  return L;
}

int check_config(const mv_config *c) {
  if (!c) return fail(MV_ERR_NULL, "config is NULL");
  if (c->dtype != MV_F32 && c->dtype != MV_BF16) return fail(MV_ERR_UNSUPPORTED, "dtype must be MV_F32 or MV_BF16");
  if (c->d_model <= 0 || c->d_model % 64 || c->d_model > 4096)
    return fail(MV_ERR_UNSUPPORTED, "d_model must be a positive multiple of 64, at most 4096");
  if (c->d_ff <= 0 || c->d_ff % 64 || c->d_ff > 8192)
    return fail(MV_ERR_UNSUPPORTED, "d_ff must be a positive multiple of 64, at most 8192");
  if (c->n_routed < 1 || c->n_routed > 64) return fail(MV_ERR_UNSUPPORTED, "n_routed must be in [1, 64]");
  if (c->top_k < 1 || c->top_k > 8 || c->top_k > c->n_routed)
    return fail(MV_ERR_UNSUPPORTED, "top_k must be in [1, min(8, n_routed)]");
  if (c->n_shared < 0 || c->n_shared > 4) return fail(MV_ERR_UNSUPPORTED, "n_shared must be in [0, 4]");
  if (c->n_layers < 1) return fail(MV_ERR_UNSUPPORTED, "n_layers must be >= 1");
  if (c->vocab < 1) return fail(MV_ERR_UNSUPPORTED, "vocab must be >= 1");
  if (!(c->rms_eps > 0.f)) return fail(MV_ERR_UNSUPPORTED, "rms_eps must be > 0");
  return MV_OK;
}

int check_layer_weights(const mv_config *c, const mv_weights *w) {
  if (!w) return fail(MV_ERR_NULL, "weights is NULL");
  if (!w->ffn_norm || !w->router_w || !w->w_gate_up || !w->w_down)
    return fail(MV_ERR_NULL, "a layer weight pointer is NULL");
  if (c->n_shared > 0 && (!w->ws_gate_up || !w->ws_down))
    return fail(MV_ERR_NULL, "shared-expert weights are NULL with n_shared > 0");
  return MV_OK;
}

int check_ws(const mv_config *c, int T, const void *ws, size_t ws_bytes) {
  if (!ws) return fail(MV_ERR_NULL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(MV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < layout(*c, T).total) return fail(MV_ERR_WORKSPACE, "workspace smaller than mv_workspace_bytes(cfg, T)");
  return MV_OK;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return MV_OK;
  g_err = std::string("HIP launch failed: ") + hipGetErrorString(e);
  return MV_ERR_HIP;
}

struct LayerPtrs {
  const void *norm, *router, *gu, *down, *sgu, *sdown;
  const float *bias;
};

LayerPtrs layer_ptrs(const mv_config &c, const mv_weights &w, int layer) {
  const size_t es = c.dtype == MV_BF16 ? 2 : 4;
  const size_t d = c.d_model, F = c.d_ff, E = c.n_routed, S = c.n_shared;
  auto at = [&](const void *base, size_t elems) {
    return base ? static_cast<const void *>(static_cast<const char *>(base) + layer * elems * es) : nullptr;
  };
  LayerPtrs p;
  p.norm = at(w.ffn_norm, d);
  p.router = at(w.router_w, E * d);
  p.gu = at(w.w_gate_up, E * 2 * F * d);
  p.down = at(w.w_down, E * d * F);
  p.sgu = at(w.ws_gate_up, S * 2 * F * d);
  p.sdown = at(w.ws_down, S * d * F);
  p.bias = w.router_b ? w.router_b + static_cast<size_t>(layer) * E : nullptr;
  return p;
}

struct Step {
  const mv_config &c;
  const mv_weights &w;
  int T;
  char *ws;
  Layout L;
  hipStream_t s;

  int *seg() const { return reinterpret_cast<int *>(ws + L.seg); }
  int *tiles() const { return reinterpret_cast<int *>(ws + L.tiles); }
  int *rows() const { return reinterpret_cast<int *>(ws + L.rows); }
  int4 *tinfo() const { return reinterpret_cast<int4 *>(ws + L.tinfo); }
  float *slots() const { return reinterpret_cast<float *>(ws + L.slots); }
  float *gates() const { return reinterpret_cast<float *>(ws + L.gates); }
  unsigned long long *argkey() const { return reinterpret_cast<unsigned long long *>(ws + L.argkey); }
  unsigned *done() const { return reinterpret_cast<unsigned *>(ws + L.done); }

  mv::RouteArgs route_args(int layer, int mode, int *ids, float *gates_out) const {
    mv::RouteArgs a{};
    a.T = T;
    a.d = c.d_model;
    a.E = c.n_routed;
    a.S = c.n_shared;
    a.k = c.top_k;
    a.nslot = c.top_k + c.n_shared;
    a.mode = mode;
    a.tile_m = tile_rows(c, T);
    a.eps = c.rms_eps;
    a.x_out = ws + L.x;
    a.seg = seg();
    a.tile_start = tiles();
    a.rows = rows();
    a.tile_info = tinfo();
    a.ids = ids;
    a.gates = gates_out;
    if (mode == mv::kFinal) {
      a.gamma = w.final_norm;
      a.argkey = argkey();
      a.done = done();
    } else if (mode == mv::kRoute) {
      const LayerPtrs lp = layer_ptrs(c, w, layer);
      a.gamma = lp.norm;
      a.router_w = lp.router;
      a.router_b = lp.bias;
    }
    return a;
  }

  bool small() const { return T <= mv::kSmallT; }
  // Router logits spread over expert groups, top-k in the gate/up kernel.
  bool logits_route() const { return T <= mv::kLogitsMaxT; }
  // logits buffer of the layers of parity `par` (the fused launch of a
  // layer fills the next one's with kLogitUnset before that layer routes)
  float *logits(int par = 0) const {
    return reinterpret_cast<float *>(ws + L.logits) + static_cast<size_t>(par & 1) * T * 64;
  }
  // fused-launch counter set s (0 or 1): tile counters, then the routing copies
  unsigned *done_set(int s) const {
    return reinterpret_cast<unsigned *>(ws + L.tdone) + static_cast<size_t>(s) * done_set_words(c, T);
  }
  int done_count() const { return max_tiles(c, T, mv::kTileM) + mv::kRouteCopies; }
  unsigned *status() const { return reinterpret_cast<unsigned *>(ws + L.status); }
  // LDS-tiled GEMMs; the combine is in the shared experts' down projection
  bool gemm() const { return path_for(c, T) == kGemmTiles; }

  // One routing launch (+ the grouping kernel on the large-batch path).
  // With `slots`, h_dst = h_src + the previous layer's expert outputs first.
  // `logits`: routing stops at the logits (mode kRoute only; the ffn of the
  // same layer then takes the top-k).
  // `first`: the call's first launch, which clears its status word.
  int route(int layer, int mode, const void *h_src, void *h_dst, const float *slots_in,
            float *y_moe, int *ids, float *gates_out, bool logits = false, bool first = false) const {
    mv::RouteArgs a = route_args(layer, mode, ids, gates_out);
    if (first) a.status = status();
    if (logits && mode == mv::kRoute) {  // also clears counter set 0 for the first fused launch
      a.mode = mv::kLogits;
      a.logits = this->logits();
      a.tile_done = done_set(0);
      a.n_tile_done = done_count();
    }
    if (mode == mv::kRoute && gemm()) {  // h_src is already combined on this path
      return hip_status(mv::launch_route_large(a, h_src, reinterpret_cast<int *>(ws + L.bcnt), s));
    }
    mv::CombineArgs cb{};
    cb.h_src = h_src;
    cb.h_dst = h_dst;
    cb.slots = slots_in;
    cb.y_moe = y_moe;
    const int ntok = T <= kOneTokenRouteT ? 1 : mv::kTileM;
    int rc = hip_status(mv::launch_route(c.dtype, a, cb, ntok, s));
    if (rc || mode != mv::kRoute || small()) return rc;
    return hip_status(mv::launch_permute(a, s));
  }

  // gate/up then down for `layer`, leaving the weighted expert outputs in
  // slots; on the GEMM path also the combine h_dst = h_src + y (y_moe: y).
  // `logits`: the routing of this layer stops at the logits (done by the
  // routing kernel before, or with ra / ca inside this launch); the fused
  // expert launch takes the top-k and writes ids and gates.  It uses counter
  // set layer % 2 and clears the other one for the next layer.
  int ffn(int layer, int *ids, float *gates, const void *h_src = nullptr, void *h_dst = nullptr,
          float *y_moe = nullptr, bool logits = false, const mv::RouteArgs *ra = nullptr,
          const mv::CombineArgs *ca = nullptr) const {
    const LayerPtrs lp = layer_ptrs(c, w, layer);
    mv::ExpertArgs e = expert_args(layer, ids, gates, logits);
    const int mt = max_tiles(c, T);
    if (logits) {
      e.logits = this->logits(layer);
      e.logits_next = this->logits(layer + 1);
      return hip_status(mv::launch_ffn_small(c.dtype, e, ra, ca, mt, s));
    }
    const Path path = path_for(c, T);
    int rc = hip_status(path == kGemmTiles  ? mv::launch_gemm_gate_up(e, mt, s)
                        : path == kMidTiles ? mv::launch_gate_up_mid(c.dtype, e, mt, s)
                                            : mv::launch_gate_up(c.dtype, e, mt, s));
    if (rc) return rc;
    e.w_routed = lp.down;
    e.w_shared = lp.sdown;
    if (path == kGemmTiles) {
      if ((rc = hip_status(mv::launch_gemm_down(e, mt, s)))) return rc;
      mv::CombineArgs cb{h_src, h_dst, slots(), y_moe};
      return hip_status(mv::launch_gemm_down_shared(e, cb, s));
    }
    return hip_status(path == kMidTiles ? mv::launch_down_mid(c.dtype, e, mt, s)
                                        : mv::launch_down(c.dtype, e, mt, s));
  }

  // Expert-launch arguments of `layer` (gate/up weights; with `logits`, the
  // fused launch's: down weights, top-k outputs, counter set layer % 2).
  mv::ExpertArgs expert_args(int layer, int *ids, float *gates, bool logits) const {
    const LayerPtrs lp = layer_ptrs(c, w, layer);
    mv::ExpertArgs e{};
    e.T = T;
    e.d = c.d_model;
    e.F = c.d_ff;
    e.E = c.n_routed;
    e.S = c.n_shared;
    e.k = c.top_k;
    e.nslot = c.top_k + c.n_shared;
    e.x = ws + L.x;
    e.a = ws + L.a;
    e.a_out = ws + L.a;
    e.seg = seg();
    e.tile_start = tiles();
    e.rows = rows();
    e.tile_info = tinfo();
    e.ids = ids;
    e.group_in_block = small() ? 1 : 0;
    e.gates = gates;
    e.slots = slots();
    e.w_routed = lp.gu;
    e.w_shared = lp.sgu;
    if (logits) {  // gate/up and down in one launch
      e.logits = this->logits();
      e.ids_out = ids;
      e.gates_out = gates;
      const int set = layer % 2;
      e.tile_done = done_set(set);
      e.route_done = done_set(set) + static_cast<size_t>(max_tiles(c, T, mv::kTileM)) * mv::kDoneStride;
      e.done_next = done_set(1 - set);
      e.n_done = done_count();
      e.err = status();
      e.spin_limit = g_spin_limit.load(std::memory_order_relaxed);
      e.w_routed_down = lp.down;
      e.w_shared_down = lp.sdown;
    }
    return e;
  }
};

}  // namespace

MV_API size_t mv_workspace_bytes(const mv_config *cfg, int32_t max_tokens) {
  if (check_config(cfg) != MV_OK) return 0;
  if (max_tokens < 0 || max_tokens > kMaxTokens) {
    g_err = "max_tokens must be in [0, 65535]";
    return 0;
  }
  return layout(*cfg, max_tokens).total;
}

MV_API int moe_layer_forward(const mv_config *cfg, const mv_weights *w, int32_t layer, int32_t T,
                             const void *h_in, void *h_out, int32_t *topk_ids, float *topk_w,
                             float *y_moe, void *ws, size_t ws_bytes, void *stream) {
  g_err.clear();
  int rc = check_config(cfg);
  if (rc) return rc;
  if (layer < 0 || layer >= cfg->n_layers) return fail(MV_ERR_SHAPE, "layer index out of range");
  if (T < 0 || T > kMaxTokens) return fail(MV_ERR_SHAPE, "T must be in [0, 65535]");
  if ((rc = check_layer_weights(cfg, w))) return rc;
  if (T == 0) return MV_OK;
  if (!h_in || !h_out) return fail(MV_ERR_NULL, "h_in and h_out are required");
  if ((rc = check_ws(cfg, T, ws, ws_bytes))) return rc;

  Step st{*cfg, *w, T, static_cast<char *>(ws), layout(*cfg, T), static_cast<hipStream_t>(stream)};
  int *ids = topk_ids ? topk_ids : reinterpret_cast<int *>(st.ws + st.L.ids);
  float *gates = topk_w ? topk_w : st.gates();
  if ((rc = st.route(layer, mv::kRoute, h_in, nullptr, nullptr, nullptr, ids, gates, false, true))) return rc;
  if (st.gemm()) return st.ffn(layer, ids, gates, h_in, h_out, y_moe);
  if ((rc = st.ffn(layer, ids, gates))) return rc;
  return st.route(layer, mv::kCombine, h_in, h_out, st.slots(), y_moe, nullptr, nullptr);
}

namespace {

// Arguments of a verify step other than the workspace; B > 0 means there is
// work (the workspace is checked next).
int check_verify(const mv_config *cfg, const mv_weights *w, int32_t B, int32_t K, const void *h_in,
                 const int32_t *drafts, const int32_t *argmax, const int32_t *n_accepted, const int32_t *committed,
                 const int32_t *n_committed) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (B < 0 || K < 0) return fail(MV_ERR_SHAPE, "B and K must be >= 0");
  if (K > kMaxK) return fail(MV_ERR_SHAPE, "K must be at most 15");
  const long long Tl = static_cast<long long>(B) * (K + 1);
  if (Tl > kMaxTokens) return fail(MV_ERR_SHAPE, "B*(K+1) must be at most 65535");
  if ((rc = check_layer_weights(cfg, w))) return rc;
  if (!w->final_norm || !w->lm_head) return fail(MV_ERR_NULL, "final_norm and lm_head are required");
  if (B == 0) return MV_OK;
  if (!h_in || !argmax || !n_accepted || !committed || !n_committed)
    return fail(MV_ERR_NULL, "h_in, argmax, n_accepted, committed and n_committed are required");
  if (K > 0 && !drafts) return fail(MV_ERR_NULL, "drafts is required when K > 0");
  return MV_OK;
}

// The verify step's launch sequence, arguments and workspace already checked.
int verify_launches(const mv_config *cfg, const mv_weights *w, int32_t B, int32_t K, const void *h_in,
                    const int32_t *drafts, void *h_out, int32_t *argmax, int32_t *n_accepted, int32_t *committed,
                    int32_t *n_committed, int32_t *dbg_topk_ids, void *ws, void *stream) {
  int rc = MV_OK;
  const int T = B * (K + 1);
  Step st{*cfg, *w, T, static_cast<char *>(ws), layout(*cfg, T), static_cast<hipStream_t>(stream)};
  void *hbuf = h_out ? h_out : static_cast<void *>(st.ws + st.L.hbuf);
  const int L = cfg->n_layers, k = cfg->top_k;
  float *gates = st.gates();
  const bool gemm = st.gemm();
  const void *cur = h_in;  // hidden state entering the next combine (small and medium paths)
  for (int layer = 0; layer < L; ++layer) {
    int *ids = dbg_topk_ids ? dbg_topk_ids + static_cast<size_t>(layer) * T * k
                            : reinterpret_cast<int *>(st.ws + st.L.ids);
    const void *src = layer == 0 ? h_in : hbuf;
    if (gemm) {  // the layer's own combine writes hbuf
      if ((rc = st.route(layer, mv::kRoute, src, nullptr, nullptr, nullptr, ids, gates, false, layer == 0)) ||
          (rc = st.ffn(layer, ids, gates, src, hbuf)))
        return rc;
      continue;
    }
    // layer 0 routes h_in; later layers first add the previous layer's
    // experts.  Logits routing runs several blocks per token that all read the
    // row one of them writes, so each combine writes a buffer other than the
    // one it reads (the final one, one block per token, may stay in place).
    // Up to kLogitsMaxT rows, layers after the first route inside their
    // fused expert launch.
    const bool lg = st.logits_route();
    if (layer == 0) {
      rc = st.route(0, mv::kRoute, h_in, nullptr, nullptr, nullptr, ids, gates, lg, true);
      if (rc || (rc = st.ffn(0, ids, gates, nullptr, nullptr, nullptr, lg))) return rc;
      continue;
    }
    void *dst = (L - layer) % 2 == 0 ? hbuf : static_cast<void *>(st.ws + st.L.hbuf2);
    if (dst == cur) dst = st.ws + st.L.hbuf3;
    if (lg) {
      mv::RouteArgs ra = st.route_args(layer, mv::kRoute, ids, gates);
      ra.mode = mv::kLogits;
      ra.logits = st.logits(layer);
      const mv::CombineArgs cb{cur, dst, st.slots(), nullptr};
      rc = st.ffn(layer, ids, gates, nullptr, nullptr, nullptr, true, &ra, &cb);
    } else if (!(rc = st.route(layer, mv::kRoute, cur, dst, st.slots(), nullptr, ids, gates))) {
      rc = st.ffn(layer, ids, gates);
    }
    if (rc) return rc;
    cur = dst;
  }
  if (gemm)
    rc = st.route(L - 1, mv::kFinal, hbuf, nullptr, nullptr, nullptr, nullptr, nullptr);
  else
    rc = st.route(L - 1, mv::kFinal, cur, hbuf, st.slots(), nullptr, nullptr, nullptr);
  if (rc) return rc;

  // LM head; its last block to finish applies the accept rule
  const mv::AcceptArgs aa{B, K, st.argkey(), nullptr, argmax, drafts, n_accepted, committed, n_committed};
  const mv::LmArgs la{T, cfg->d_model, cfg->vocab, st.ws + st.L.x, w->lm_head, st.argkey(), st.done(), aa};
  return hip_status(mv::launch_lm_argmax(cfg->dtype, la, st.s));
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the
// first use on that device, with that device current).
int scratch_on_device(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return fail(MV_ERR_UNSUPPORTED, "device index beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_err = std::string("hipGetSymbolAddress of the static scratch failed: ") + hipGetErrorString(e);
      return MV_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MV_OK;
}

}  // namespace

// The verify step of a batch routed to logits as one launch: the setup kernel
// writes every virtual block's arguments and clears the counters, then
// k_one_launch runs the layers' fused launches, the final norm and the LM
// head with the accept rule as the blocks of one launch.  Buffers
// and arithmetic are those of verify_launches, so the results are
// bit-identical to moe_verify_step's.
int one_launch_step(const mv_config *cfg, const mv_weights *w, int32_t B, int32_t K, const void *h_in,
                    const int32_t *drafts, void *h_out, int32_t *argmax, int32_t *n_accepted, int32_t *committed,
                    int32_t *n_committed, int32_t *dbg_topk_ids, void *ws, void *stream) {
  const int T = B * (K + 1), L = cfg->n_layers, k = cfg->top_k;
  if (T > mv::kLogitsMaxT || L > mv::kOneLaunchMaxLayers)
    return fail(MV_ERR_UNSUPPORTED, "the one-launch verify step takes at most 8 rows (B*(K+1)) and 16 layers");
  Step st{*cfg, *w, T, static_cast<char *>(ws), layout(*cfg, T), static_cast<hipStream_t>(stream)};
  void *hbuf = h_out ? h_out : static_cast<void *>(st.ws + st.L.hbuf);
  float *gates = st.gates();
  const int mt = max_tiles(*cfg, T);
  mv::OneLaunchArgs a{};
  a.e = st.expert_args(0, nullptr, gates, true);
  a.e.n_done = 0;  // the setup kernel clears every counter
  a.e.done_next = nullptr;
  a.r = st.route_args(0, mv::kRoute, nullptr, gates);
  a.r.mode = mv::kLogits;
  a.r.logits = st.logits();
  a.f = st.route_args(L - 1, mv::kFinal, nullptr, nullptr);
  a.slots = st.slots();
  a.ctr = reinterpret_cast<unsigned *>(st.ws + st.L.ol_ctr);
  a.L = L;
  a.max_tiles = mt;
  a.n_route = T * ((cfg->n_routed + mv::kRouteGroup - 1) / mv::kRouteGroup);
  a.n_lm = (cfg->vocab + mv::kLmRowsPerBlock - 1) / mv::kLmRowsPerBlock;
  a.set_lines = mt + mv::kRouteCopies + 1;
  unsigned *lm_done = a.ctr + (static_cast<size_t>(L) * a.set_lines + 1) * mv::kDoneStride;
  const mv::AcceptArgs aa{B, K, st.argkey(), nullptr, argmax, drafts, n_accepted, committed, n_committed};
  a.lm = mv::LmArgs{T, cfg->d_model, cfg->vocab, st.ws + st.L.x, w->lm_head, st.argkey(), lm_done, aa};
  const void *cur = h_in;  // the same hidden-state buffers as verify_launches
  for (int layer = 0; layer < L; ++layer) {
    const LayerPtrs lp = layer_ptrs(*cfg, *w, layer);
    mv::StepLayer &sl = a.layer[layer];
    sl = mv::StepLayer{lp.gu, lp.down, lp.sgu, lp.sdown, lp.norm, lp.router, lp.bias,
                       dbg_topk_ids ? dbg_topk_ids + static_cast<size_t>(layer) * T * k
                                    : reinterpret_cast<int *>(st.ws + st.L.ids),
                       h_in, nullptr};
    if (layer == 0) continue;
    void *dst = (L - layer) % 2 == 0 ? hbuf : static_cast<void *>(st.ws + st.L.hbuf2);
    if (dst == cur) dst = st.ws + st.L.hbuf3;
    sl.h_src = cur;
    sl.h_dst = dst;
    cur = dst;
  }
  a.h_last = cur;
  a.h_final = hbuf;
  const size_t smem = mv::one_launch_smem(cfg->dtype, T, cfg->d_model, cfg->d_ff);
  return hip_status(mv::launch_one_launch(cfg->dtype, a, reinterpret_cast<mv::OneLaunchDev *>(st.ws + st.L.ol_args),
                                          st.status(), smem, st.s));
}

MV_API int moe_verify_step(const mv_config *cfg, const mv_weights *w, int32_t B, int32_t K,
                           const void *h_in, const int32_t *drafts, void *h_out, int32_t *argmax,
                           int32_t *n_accepted, int32_t *committed, int32_t *n_committed,
                           int32_t *dbg_topk_ids, void *ws, size_t ws_bytes, void *stream) {
  g_err.clear();
  int rc = check_verify(cfg, w, B, K, h_in, drafts, argmax, n_accepted, committed, n_committed);
  if (rc || B == 0) return rc;
  if ((rc = check_ws(cfg, B * (K + 1), ws, ws_bytes))) return rc;
  return verify_launches(cfg, w, B, K, h_in, drafts, h_out, argmax, n_accepted, committed, n_committed,
                         dbg_topk_ids, ws, stream);
}

MV_API int moe_verify_step_one_launch(const mv_config *cfg, const mv_weights *w, int32_t B, int32_t K,
                                      const void *h_in, const int32_t *drafts, void *h_out, int32_t *argmax,
                                      int32_t *n_accepted, int32_t *committed, int32_t *n_committed,
                                      int32_t *dbg_topk_ids, void *ws, size_t ws_bytes, void *stream) {
  g_err.clear();
  int rc = check_verify(cfg, w, B, K, h_in, drafts, argmax, n_accepted, committed, n_committed);
  if (rc || B == 0) return rc;
  if ((rc = check_ws(cfg, B * (K + 1), ws, ws_bytes))) return rc;
  return one_launch_step(cfg, w, B, K, h_in, drafts, h_out, argmax, n_accepted, committed, n_committed, dbg_topk_ids,
                         ws, stream);
}

MV_API int moe_verify_step_noalloc(const mv_config *cfg, const mv_weights *w, int32_t B, int32_t K,
                                   const void *h_in, const int32_t *drafts, void *h_out, int32_t *argmax,
                                   int32_t *n_accepted, int32_t *committed, int32_t *n_committed,
                                   int32_t *dbg_topk_ids, void *stream) {
  g_err.clear();
  int rc = check_verify(cfg, w, B, K, h_in, drafts, argmax, n_accepted, committed, n_committed);
  if (rc || B == 0) return rc;
  if (layout(*cfg, B * (K + 1)).total > kScratchBytes)
    return fail(MV_ERR_WORKSPACE, "this step needs more than the 16 MiB static scratch of moe_verify_step_noalloc "
                                  "(mv_workspace_bytes(cfg, B*(K+1)) > 16 MiB); use moe_verify_step");
  void *ws = nullptr;
  if ((rc = scratch_on_device(&ws))) return rc;
  return verify_launches(cfg, w, B, K, h_in, drafts, h_out, argmax, n_accepted, committed, n_committed,
                         dbg_topk_ids, ws, stream);
}

MV_API int spec_accept(int32_t B, int32_t K, const int32_t *argmax, const int32_t *drafts,
                       int32_t *n_accepted, int32_t *committed, int32_t *n_committed, void *stream) {
  g_err.clear();
  if (B < 0 || K < 0) return fail(MV_ERR_SHAPE, "B and K must be >= 0");
  if (K > kMaxK) return fail(MV_ERR_SHAPE, "K must be at most 15");
  if (B == 0) return MV_OK;
  if (!argmax || !n_accepted || !committed || !n_committed)
    return fail(MV_ERR_NULL, "argmax, n_accepted, committed and n_committed are required");
  if (K > 0 && !drafts) return fail(MV_ERR_NULL, "drafts is required when K > 0");
  mv::AcceptArgs aa{B, K, nullptr, argmax, nullptr, drafts, n_accepted, committed, n_committed};
  return hip_status(mv::launch_accept(aa, static_cast<hipStream_t>(stream)));
}

// ------------------------------------------------------- FastMTP draft block

namespace {

struct MtpLayout {
  size_t acc, acc2, gu, a, hcur, xo, argkey, u, x, total;
};

MtpLayout mtp_layout(const mv_config &c, int Fm, int B) {
  const size_t es = c.dtype == MV_BF16 ? 2 : 4, d = static_cast<size_t>(c.d_model), b = static_cast<size_t>(B);
  MtpLayout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t at = off;
    off += align256(bytes);
    return at;
  };
  L.acc = take(mv::kMtpSplit * b * d * 4);   // K-split partials of z
  L.acc2 = take(mv::kMtpSplit * b * d * 4);  // and of y
  // and of the FFN's gate and up (up to kMtpFusedMaxB sequences; above, the
  // FFN's SwiGLU products a)
  const bool fused = b <= static_cast<size_t>(mv::kMtpFusedMaxB);
  L.gu = take(fused ? mv::kMtpSplit * b * 2 * static_cast<size_t>(Fm) * 4 : 0);
  L.a = take(fused ? 0 : b * static_cast<size_t>(Fm) * es);
  L.hcur = take(b * d * es);
  L.xo = take(b * d * es);
  L.argkey = take(2 * b * 8);
  L.u = take(b > static_cast<size_t>(mv::kMtpFusedMaxB) ? b * 2 * d * es : 0);
  L.x = take(b > static_cast<size_t>(mv::kMtpFusedMaxB) ? b * d * es : 0);
  L.total = off;
  return L;
}

// The projection and the dense FFN stage 16 rows of width 2d and Fm (and the
// rows' chunk sums) in LDS.
int check_mtp(const mv_config *c, int Fm) {
  if (Fm <= 0 || Fm % 64) return fail(MV_ERR_UNSUPPORTED, "the draft block's d_ff must be a positive multiple of 64");
  const int es = c->dtype == MV_BF16 ? 2 : 4;
  const size_t lds = 152 * 1024;  // dynamic LDS, leaving room for the kernels' static arrays
  if (mv::mtp_proj_lds(c->d_model, es) > lds)
    return fail(MV_ERR_UNSUPPORTED, "2*d_model is too wide for the draft block's projection tile");
  if (mv::mtp_ffn_lds(c->d_model, Fm, es) > lds)
    return fail(MV_ERR_UNSUPPORTED, "the draft block's d_ff is too wide for its FFN tile");
  return MV_OK;
}

// One-expert arguments of the dense layers: rows [0, B) in tiles of 16.
mv::ExpertArgs dense_args(const mv_config &c, int B, int K_in, const void *a_in, const void *w, float *out) {
  mv::ExpertArgs e{};
  e.T = B;
  e.d = c.d_model;
  e.F = K_in;
  e.E = 1;
  e.S = 0;
  e.k = 0;
  e.nslot = 1;
  e.x = a_in;
  e.a = a_in;
  e.w_routed = w;
  e.slots = out;
  return e;
}

}  // namespace

MV_API size_t mtp_workspace_bytes(const mv_config *cfg, int32_t d_ff_mtp, int32_t max_rows) {
  if (check_config(cfg) != MV_OK || check_mtp(cfg, d_ff_mtp) != MV_OK) return 0;
  if (max_rows < 0 || max_rows > kMaxTokens) {
    g_err = "max_rows must be in [0, 65535]";
    return 0;
  }
  return mtp_layout(*cfg, d_ff_mtp, max_rows).total;
}

MV_API int mtp_draft(const mv_config *cfg, const mv_weights *w, const mtp_weights *m, int32_t B, int32_t K,
                     const void *h_in, const int32_t *tokens, int32_t *drafts, void *h_out, void *ws,
                     size_t ws_bytes, void *stream) {
  g_err.clear();
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!w || !m) return fail(MV_ERR_NULL, "weights are NULL");
  if (B < 0 || K < 0) return fail(MV_ERR_SHAPE, "B and K must be >= 0");
  if (K > kMaxK) return fail(MV_ERR_SHAPE, "K must be at most 15");
  if (B > kMaxTokens) return fail(MV_ERR_SHAPE, "B must be at most 65535");
  if ((rc = check_mtp(cfg, m->d_ff))) return rc;
  if (B == 0 || K == 0) return MV_OK;
  if (!w->lm_head || !m->embed || !m->norm_h || !m->norm_e || !m->w_proj || !m->norm_ffn || !m->w_gate_up ||
      !m->w_down || !m->norm_out)
    return fail(MV_ERR_NULL, "a draft-block or LM-head weight pointer is NULL");
  if (!h_in || !tokens || !drafts) return fail(MV_ERR_NULL, "h_in, tokens and drafts are required");
  if (!ws) return fail(MV_ERR_NULL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(MV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  const MtpLayout L = mtp_layout(*cfg, m->d_ff, B);
  if (ws_bytes < L.total) return fail(MV_ERR_WORKSPACE, "workspace smaller than mtp_workspace_bytes(cfg, d_ff, B)");

  char *base = static_cast<char *>(ws);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const int dt = cfg->dtype, d = cfg->d_model;
  mv::MtpArgs a{};
  a.B = B;
  a.K = K;
  a.d = d;
  a.V = cfg->vocab;
  a.eps = cfg->rms_eps;
  a.tokens = tokens;
  a.argkey = reinterpret_cast<unsigned long long *>(base + L.argkey);
  a.drafts = drafts;
  a.h_in = h_in;
  a.h_cur = base + L.hcur;
  a.h_out = h_out;
  a.embed = m->embed;
  a.norm_h = m->norm_h;
  a.norm_e = m->norm_e;
  a.norm_ffn = m->norm_ffn;
  a.norm_out = m->norm_out;
  a.acc = reinterpret_cast<float *>(base + L.acc);
  a.acc2 = reinterpret_cast<float *>(base + L.acc2);
  a.gu = reinterpret_cast<float *>(base + L.gu);
  a.xo = base + L.xo;
  a.u = base + L.u;
  a.x = base + L.x;

  const mv::ExpertArgs proj = dense_args(*cfg, B, 2 * d, nullptr, m->w_proj, a.acc);
  mv::ExpertArgs gate_up = dense_args(*cfg, B, m->d_ff, nullptr, m->w_gate_up, nullptr);
  gate_up.a_out = base + L.a;  // above kMtpFusedMaxB sequences
  const mv::ExpertArgs down = dense_args(*cfg, B, m->d_ff, base + L.a, m->w_down, a.acc2);
  for (int step = 0; step < K; ++step) {
    // this position's LM head folds into key buffer step % 2
    const mv::LmArgs la{B, d, cfg->vocab, a.xo, w->lm_head, a.argkey + static_cast<size_t>(step & 1) * B, nullptr,
                        mv::AcceptArgs{}};
    if ((rc = hip_status(mv::launch_mtp_position(dt, proj, gate_up, down, a, step, s))) ||
        (rc = hip_status(mv::launch_mtp_lm(dt, la, a, step, s))))
      return rc;
  }
  return hip_status(mv::launch_mtp_last(a, s));
}

// ------------------------------------------------------------- draft length

MV_API int mv_choose_k(int32_t k_max, float q, const float *cost, int32_t *k_best, float *rate) {
  g_err.clear();
  if (!cost || !k_best) return fail(MV_ERR_NULL, "cost and k_best are required");
  if (k_max < 0 || k_max > kMaxK) return fail(MV_ERR_SHAPE, "k_max must be in [0, 15]");
  if (!(q >= 0.f && q <= 1.f)) return fail(MV_ERR_SHAPE, "q must be in [0, 1]");
  for (int k = 0; k <= k_max; ++k)
    if (!(cost[k] > 0.f)) return fail(MV_ERR_SHAPE, "every cost must be > 0");
  // E(K) = sum_{i <= K} q^i, accumulated in double
  double e = 0.0, qi = 1.0, best_rate = -1.0;
  int best = 0;
  for (int k = 0; k <= k_max; ++k) {
    e += qi;
    qi *= static_cast<double>(q);
    const double r = e / static_cast<double>(cost[k]);
    if (r > best_rate) {
      best_rate = r;
      best = k;
    }
  }
  *k_best = best;
  if (rate) *rate = static_cast<float>(best_rate);
  return MV_OK;
}

MV_API double mv_step_bytes(const mv_config *cfg, int32_t B, int32_t K, int32_t d_ff_mtp) {
  g_err.clear();
  if (check_config(cfg) != MV_OK) return -1.0;
  if (B < 0 || K < 0 || K > kMaxK || d_ff_mtp < 0) {
    g_err = "B, K and d_ff_mtp must be >= 0 and K <= 15";
    return -1.0;
  }
  const double es = cfg->dtype == MV_BF16 ? 2.0 : 4.0, d = cfg->d_model, F = cfg->d_ff, E = cfg->n_routed;
  const double V = cfg->vocab, L = cfg->n_layers, T = static_cast<double>(B) * (K + 1);
  const double miss = std::pow(1.0 - static_cast<double>(cfg->top_k) / E, T);
  const double distinct = E * (1.0 - miss);
  double bytes = L * (distinct + cfg->n_shared) * 3.0 * F * d * es;  // routed and shared experts
  bytes += L * (E * d + d) * es + V * d * es + d * es;               // router, norms, LM head
  bytes += 2.0 * T * d * es;                                         // rows in and out
  bytes += K * ((2.0 * d * d + 3.0 * d_ff_mtp * d + V * d + 4.0 * d) * es + B * 3.0 * d * es);  // draft block
  return bytes;
}

MV_API int mv_step_status(const void *ws, int32_t *status, void *stream) {
  g_err.clear();
  if (!status) return fail(MV_ERR_NULL, "status is required");
  if (!ws) {  // the current device's static scratch (moe_verify_step_noalloc)
    void *p = nullptr;
    const int rc = scratch_on_device(&p);
    if (rc) return rc;
    ws = p;
  }
  if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(MV_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  // the status word sits at offset 0 of every layout
  const unsigned *word = static_cast<const unsigned *>(ws);
  return hip_status(mv::launch_copy_status(word, status, static_cast<hipStream_t>(stream)));
}

MV_API int32_t mv_set_spin_limit(int32_t polls) {
  return g_spin_limit.exchange(polls < 0 ? mv::kSpinLimitDefault : polls);
}

MV_API const char *mv_last_error(void) { return g_err.c_str(); }
