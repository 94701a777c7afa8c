// Host-side plan: validates the packed layout and builds the tile geometry.
//
// Geometry mapper ("Ref2VA VSA : noeud d'attention sparse pour le Ref2VA H3",
// "Le correctif d'attention a deux niveaux", item 1; "ComfyUI-Ref2VA-VSA",
// "The Solution"): every conditioning segment (text, reference image,
// reference audio) is cut into tiles of 64 consecutive tokens that hold no
// other segment; the video span is cut into 4x4x4 tiles ("ComfyUI-Ref2VA-VSA",
// "Technical Architecture").  The plan is a few scalars and at most 16
// segments, so kernels take it by value; the library never allocates device
// memory.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "vsa_internal.h"

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

struct Seg {
  int64_t start, length;
  int32_t kind;
};

}  // namespace

extern "C" int vsa_plan_geometry(const vsa_segment* segs, int n_segs, int batch, int video_T,
                                 int video_H, int video_W, int heads, int head_dim,
                                 float keep_percent, const vsa_options* opts, vsa_plan** out) {
  if (out == nullptr) return VSA_ERR_INVALID_ARGUMENT;
  *out = nullptr;
  if (segs == nullptr || n_segs <= 0 || batch <= 0 || heads <= 0 || video_T <= 0 ||
      video_H <= 0 || video_W <= 0 || head_dim <= 0)
    return VSA_ERR_INVALID_ARGUMENT;
  if (head_dim != VSA_HEAD_DIM) return VSA_ERR_UNSUPPORTED;
  if (video_T % 4 || video_H % 4 || video_W % 4) return VSA_ERR_UNSUPPORTED;

  vsa_options o{VSA_SINK_EXACT_KV, VSA_SELECT_TOPK, VSA_COARSE_MEAN, 0.0f};
  if (opts != nullptr) o = *opts;
  if (o.sink != VSA_SINK_OFF && o.sink != VSA_SINK_EXACT_KV && o.sink != VSA_SINK_EXACT_KV_AND_ROWS)
    return VSA_ERR_UNSUPPORTED;
  if (o.select != VSA_SELECT_TOPK && o.select != VSA_SELECT_TAU && o.select != VSA_SELECT_DENSE)
    return VSA_ERR_UNSUPPORTED;
  const bool dense_all = o.select == VSA_SELECT_DENSE;
  if (o.coarse != VSA_COARSE_MEAN && o.coarse != VSA_COARSE_MEAN_LOGMASS &&
      o.coarse != VSA_COARSE_WEIGHTED_LOGMASS)
    return VSA_ERR_UNSUPPORTED;
  if (o.select == VSA_SELECT_TOPK && !(keep_percent > 0.0f && keep_percent <= 100.0f))
    return VSA_ERR_UNSUPPORTED;
  if (o.select == VSA_SELECT_TAU && !std::isfinite(o.tau)) return VSA_ERR_UNSUPPORTED;
  if (o.extra_tokens < 0) return VSA_ERR_INVALID_ARGUMENT;
  if (o.extra_tokens > VSA_MAX_EXTRA) return VSA_ERR_UNSUPPORTED;
  if (dense_all && o.extra_tokens > 0) return VSA_ERR_UNSUPPORTED;  // no sparse row to take them
  if (o.reblock != 0 && o.reblock != 1) return VSA_ERR_UNSUPPORTED;
  if (o.reblock && (dense_all || o.extra_tokens > 0)) return VSA_ERR_UNSUPPORTED;

  // spans: sort by start, must partition [0, N)
  std::vector<Seg> s;
  s.reserve(n_segs);
  for (int i = 0; i < n_segs; ++i) {
    if (segs[i].start < 0 || segs[i].length <= 0) return VSA_ERR_INVALID_ARGUMENT;
    if (segs[i].kind < VSA_SEG_TEXT || segs[i].kind > VSA_SEG_VIDEO)
      return VSA_ERR_INVALID_ARGUMENT;
    s.push_back({segs[i].start, segs[i].length, segs[i].kind});
  }
  std::sort(s.begin(), s.end(), [](const Seg& a, const Seg& b) { return a.start < b.start; });
  int64_t pos = 0;
  int n_video = 0, n_prefix = 0;
  for (const Seg& x : s) {
    if (x.start != pos) return VSA_ERR_INVALID_ARGUMENT;  // gap or overlap
    pos += x.length;
    if (x.kind == VSA_SEG_VIDEO) ++n_video; else ++n_prefix;
  }
  const int64_t N = pos;
  if (n_video != 1) return VSA_ERR_UNSUPPORTED;
  if (n_prefix > VSA_MAX_PREFIX_SEGS) return VSA_ERR_UNSUPPORTED;
  // 32-bit token and element indexing inside the kernels; the fine kernel's buffer loads
  // address one batch item's K or V with 32-bit byte offsets and keep 2^31 free for an
  // always-out-of-range offset
  if (N * (int64_t)heads * VSA_HEAD_DIM >= ((int64_t)1 << 30)) return VSA_ERR_UNSUPPORTED;

  vsa_plan* p = new (std::nothrow) vsa_plan();
  if (p == nullptr) return VSA_ERR_NO_MEMORY;
  VsaGeom& g = p->g;
  std::memset(&g, 0, sizeof(g));
  int tile = 0;
  for (const Seg& x : s) {
    if (x.kind == VSA_SEG_VIDEO) {
      if (x.length != (int64_t)video_T * video_H * video_W) {
        delete p;
        return VSA_ERR_INVALID_ARGUMENT;
      }
      g.vstart = (int32_t)x.start;
      continue;
    }
    g.pre_start[g.n_pre_segs] = (int32_t)x.start;
    g.pre_len[g.n_pre_segs] = (int32_t)x.length;
    g.pre_tile0[g.n_pre_segs] = tile;
    tile += (int)((x.length + VSA_TILE_TOKENS - 1) / VSA_TILE_TOKENS);
    ++g.n_pre_segs;
  }
  g.pre_tile0[g.n_pre_segs] = tile;
  for (int i = g.n_pre_segs + 1; i <= VSA_MAX_PREFIX_SEGS; ++i) g.pre_tile0[i] = tile;
  g.T = video_T;
  g.H = video_H;
  g.W = video_W;
  g.tw_n = video_W / 4;
  g.th_n = video_H / 4;
  g.P = tile;
  g.Vt = (video_T / 4) * (video_H / 4) * (video_W / 4);
  if (g.Vt > VSA_MAX_VIDEO_TILES) {
    delete p;
    return VSA_ERR_UNSUPPORTED;
  }
  g.Tq = g.P + g.Vt;
  if (g.Tq > 65535) {  // tiles index the second grid dimension of the pooling launches
    delete p;
    return VSA_ERR_UNSUPPORTED;
  }
  // candidates: the video tiles, or with sink off every tile ("BSAI FastH3 Native VSA
  // (recipe)", "The inputs that matter": off protects no conditioning tile)
  g.npin = (o.sink == VSA_SINK_OFF || dense_all) ? 0 : g.P;
  g.kc0 = g.npin;
  g.Kc = dense_all ? 0 : g.Tq - g.kc0;  // the dense mode scores no candidate
  if (g.Kc > VSA_MAX_VIDEO_TILES) {
    delete p;
    return VSA_ERR_UNSUPPORTED;
  }
  g.N = (int32_t)N;
  g.heads = heads;
  g.batch = batch;
  g.n_dense = dense_all ? g.Tq : (o.sink == VSA_SINK_EXACT_KV_AND_ROWS) ? g.P : 0;
  g.Qs = g.Tq - g.n_dense;
  // k = ceil(keep * Kc / 100), clamped to [1, Kc]
  if (dense_all) {
    g.k = 0;
    g.cap = 0;
  } else if (o.select == VSA_SELECT_TOPK) {
    int k = (int)std::ceil((double)keep_percent * g.Kc / 100.0 - 1e-9);
    g.k = std::max(1, std::min(g.Kc, k));
    g.cap = g.npin + g.k;
  } else {
    g.k = 0;
    g.cap = g.npin + g.Kc;
  }
  if (g.cap > VSA_MAX_LIST) {
    delete p;
    return VSA_ERR_UNSUPPORTED;
  }
  g.extra = o.extra_tokens;
  // the fine kernel addresses a (b, h) plane of the extra-token staging with 32-bit offsets
  if (g.extra > 0 && (int64_t)g.Qs * VSA_MAX_EXTRA * heads * VSA_HEAD_DIM * 2 >= ((int64_t)1 << 31)) {
    delete p;
    return VSA_ERR_UNSUPPORTED;
  }
  // the extra-token threshold kernel holds a row's per-tile keys in registers: 8192 tiles at most
  if (g.extra > 0 && g.Tq > 64 * 128) {
    delete p;
    return VSA_ERR_UNSUPPORTED;
  }
  // Extra-token select: the (64-row block, tile) steps split evenly over xg workgroups (at
  // least 64 steps each); xms is the most workgroups whose ranges meet one row block.
  g.xg = 0;
  g.xms = 0;
  g.xs1 = 0;
  if (g.extra > 0 && g.Qs > 0) {
    const int64_t nrb = (g.Qs + 63) / 64;
    const int64_t NRB = nrb * heads * batch;
    const int64_t TS = NRB * g.Tq;
    const int64_t G = std::max<int64_t>(1, std::min<int64_t>(VSA_EXTRA_WGS, TS / 64));
    auto wg_of = [&](int64_t x) { return ((x + 1) * G + TS - 1) / TS - 1; };
    int64_t ms = 1;
    for (int64_t r = 0; r < NRB; ++r) ms = std::max(ms, wg_of((r + 1) * g.Tq - 1) - wg_of(r * g.Tq) + 1);
    g.xg = (int32_t)G;
    g.xms = (int32_t)ms;
    // pass 1: 128-row blocks; about four rounds of three workgroups per CU (3,072 items),
    // chunks of about 32 tiles or more
    const int64_t NRB1 = (g.Qs + 127) / 128 * heads * batch;
    g.xs1 = (int32_t)std::max<int64_t>(1, std::min<int64_t>((g.Tq + 31) / 32, (6 * VSA_EXTRA_WGS + NRB1 - 1) / NRB1));
  }
  g.sink = o.sink;
  g.select = o.select;
  g.coarse = o.coarse;
  g.tau = o.tau;
  g.reblock = o.reblock;
  g.rb_nsplit = o.reblock ? std::min(32, g.Vt) : 0;
  g.scale = (float)(1.0 / std::sqrt((double)VSA_HEAD_DIM));
  // The coarse kernel runs 64 rows per workgroup; with few row blocks per head the
  // candidate tiles are cut into slices of whole 64-tile chunks (each slice a workgroup,
  // merged by a small kernel) so that the grid spreads evenly over the CUs.
  {
    const int row_blocks = (g.Qs + VSA_COARSE_ROWS - 1) / VSA_COARSE_ROWS;
    const int nchunks = std::max(1, (g.Kc + 63) / 64);
    const int target = nchunks >= 4 ? 3 : 1;
    g.cchunks = (nchunks + target - 1) / target;
    g.csplit = (nchunks + g.cchunks - 1) / g.cchunks;
    g.coarse_blocks = row_blocks * g.csplit;
  }

  // workspace layout
  const size_t BH = (size_t)batch * heads;
  const size_t A = 256;
  VsaLayout& L = p->ws;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = align_up(off + std::max<size_t>(bytes, 1), A);
    return at;
  };
  // the dense mode pools nothing: only its (empty) sparse-row sections remain
  L.qbar = take(dense_all ? 0 : BH * g.Tq * VSA_HEAD_DIM * 4);
  L.kbar = take(BH * g.Kc * VSA_HEAD_DIM * 4);
  L.vbar = take(BH * g.Kc * VSA_HEAD_DIM * 4);
  L.bias = take(BH * g.Kc * 4);
  L.anchor = take(dense_all ? 0 : BH * VSA_HEAD_DIM * 4);
  L.scores = take(BH * (size_t)g.Qs * g.Kc * 4);
  L.ocoarse = take(BH * (size_t)g.Qs * VSA_HEAD_DIM * 4);
  L.thr = take(dense_all ? 0 : BH * 4);
  L.lists = take(BH * (size_t)g.Qs * g.cap * 4);
  L.counts = take(BH * (size_t)g.Qs * 4);
  L.statp = take(BH * (size_t)g.coarse_blocks * 2 * 8);
  const size_t xrows = g.extra > 0 ? (size_t)batch * g.Qs * VSA_MAX_EXTRA : 0;
  L.xtok = take(g.extra > 0 ? BH * (size_t)g.Qs * VSA_MAX_EXTRA * 4 : 0);
  L.xcnt = take(g.extra > 0 ? BH * (size_t)g.Qs * 4 : 0);
  L.vx = take(xrows / VSA_MAX_EXTRA * VSA_XSTAGE * heads * VSA_HEAD_DIM * 2);
  {
    const size_t xrb = g.extra > 0 ? BH * (size_t)((g.Qs + 63) / 64) * g.xms * 64 : 0;  // segment rows
    L.xpart = take(xrb * VSA_MAX_EXTRA * 8);
    L.xpcnt = take(xrb * 4);
    const size_t xr = g.extra > 0 ? BH * (size_t)g.Qs : 0;  // sparse rows
    // per (tile, row): [bh][tile][row], rows padded to a multiple of 32
    const size_t xrp = g.extra > 0 ? BH * (size_t)((g.Qs + 31) & ~31) : 0;
    L.xtm1 = take(xrp * g.Tq * 4);
    L.xtm4 = take(xrp * g.Tq * 4);
    L.xthr = take(xr * 4);
    L.xmask = take(xr * ((g.Tq + 31) / 32) * 4);
    L.xccnt = take(xr * 4);
    L.xcand = take(xr * VSA_EXTRA_CAND * 8);
    L.xqsplit = take(xr * 3 * VSA_HEAD_DIM * 2);
    L.xknorm = take(g.extra > 0 ? BH * (size_t)g.Tq * 4 : 0);
  }
  L.cpart = take(g.csplit > 1 ? BH * (size_t)g.Qs * g.csplit * (VSA_HEAD_DIM + 4) * 4 : 0);
  {
    const bool rb = g.reblock != 0;
    const size_t Nv = (size_t)VSA_TILE_TOKENS * g.Vt;
    const size_t DD = (size_t)VSA_HEAD_DIM * VSA_HEAD_DIM;
    const int levels = rb ? vsa_reblock_levels(g.Vt) : 0;
    size_t maxparts = 1;
    for (int lv = 0; lv < levels; ++lv)
      maxparts = std::max(maxparts, ((size_t)1 << lv) * (size_t)vsa_reblock_chunks(g.Vt, lv));
    const size_t maxnodes = levels > 0 ? ((size_t)1 << (levels - 1)) : 1;
    const size_t tb = (size_t)batch * N * heads * VSA_HEAD_DIM * 2;
    L.rb_mpart = take(rb ? BH * g.rb_nsplit * DD * 4 : 0);
    L.rb_m = take(rb ? BH * DD * 4 : 0);
    L.rb_mhl = take(rb ? BH * 2 * DD * 2 : 0);
    L.rb_a0 = take(rb ? BH * VSA_HEAD_DIM * 4 : 0);
    L.rb_norms = take(rb ? BH * Nv * 4 : 0);
    L.rb_list_a = take(rb ? BH * Nv * 4 : 0);
    L.rb_list_b = take(rb ? BH * Nv * 4 : 0);
    L.rb_tiles = (levels % 2 == 0) ? L.rb_list_a : L.rb_list_b;
    L.rb_pbuf = take(rb ? BH * Nv * 4 : 0);
    L.rb_part = take(rb ? BH * maxparts * 2 * VSA_HEAD_DIM * 4 : 0);
    L.rb_state = take(rb ? BH * maxnodes * VSA_RB_STATE * 4 : 0);
    L.rb_q = take(rb ? tb : 0);
    L.rb_k = take(rb ? tb : 0);
    L.rb_v = take(rb ? tb : 0);
    L.rb_g = take(rb ? tb : 0);
    L.rb_o = take(rb ? tb : 0);
  }
  L.total = off;

  p->opts = o;
  p->keep = keep_percent;
  p->n_tokens = N;
  *out = p;
  return VSA_OK;
}

extern "C" int vsa_plan_workspace_bytes(const vsa_plan* plan, size_t* bytes) {
  if (plan == nullptr || bytes == nullptr) return VSA_ERR_INVALID_ARGUMENT;
  *bytes = plan->ws.total;
  return VSA_OK;
}

extern "C" int vsa_plan_describe(const vsa_plan* plan, vsa_plan_desc* out) {
  if (plan == nullptr || out == nullptr) return VSA_ERR_INVALID_ARGUMENT;
  const VsaGeom& g = plan->g;
  out->batch = g.batch;
  out->heads = g.heads;
  out->head_dim = VSA_HEAD_DIM;
  out->n_tokens = plan->n_tokens;
  out->n_prefix_tiles = g.P;
  out->n_video_tiles = g.Vt;
  out->n_tiles = g.Tq;
  out->k = g.k;
  out->n_dense_rows = g.n_dense;
  out->n_sparse_rows = g.Qs;
  out->list_capacity = g.cap;
  out->options = plan->opts;
  out->keep_percent = plan->keep;
  out->first_candidate = g.kc0;
  out->n_candidates = g.Kc;
  return VSA_OK;
}

extern "C" int vsa_debug_views(const vsa_plan* plan, vsa_debug* out) {
  if (plan == nullptr || out == nullptr) return VSA_ERR_INVALID_ARGUMENT;
  const VsaLayout& L = plan->ws;
  out->qbar = L.qbar;
  out->kbar = L.kbar;
  out->vbar = L.vbar;
  out->bias = L.bias;
  out->anchor = L.anchor;
  out->scores = L.scores;
  out->ocoarse = L.ocoarse;
  out->thr = L.thr;
  out->lists = L.lists;
  out->counts = L.counts;
  out->xtok = L.xtok;
  out->xcnt = L.xcnt;
  out->tiles = L.rb_tiles;
  out->total_bytes = L.total;
  return VSA_OK;
}

extern "C" int vsa_plan_destroy(vsa_plan* plan) {
  delete plan;
  return VSA_OK;
}

extern "C" const char* vsa_status_string(int status) {
  switch (status) {
    case VSA_OK: return "VSA_OK";
    case VSA_ERR_INVALID_ARGUMENT: return "VSA_ERR_INVALID_ARGUMENT";
    case VSA_ERR_UNSUPPORTED: return "VSA_ERR_UNSUPPORTED";
    case VSA_ERR_WORKSPACE: return "VSA_ERR_WORKSPACE";
    case VSA_ERR_HIP: return "VSA_ERR_HIP";
    case VSA_ERR_NO_MEMORY: return "VSA_ERR_NO_MEMORY";
    default: return "VSA_ERR_UNKNOWN";
  }
}
