// vsa_forward: argument checks and the launch sequence on the caller's stream;
// stats read-back and the per-kernel event timer.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "vsa_internal.h"
#include "vsa_kernels.h"

namespace {

bool log_enabled() {
  static const int on = [] {
    const char* e = std::getenv("VSA_LOG");
    return (e != nullptr && e[0] == '1') ? 1 : 0;
  }();
  return on != 0;
}

// Text of the last HIP failure seen by this thread (step and HIP error name).
thread_local char g_last_error[160] = "";

int hip_fail(const char* step, hipError_t e) {
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s (%s)", step, hipGetErrorName(e),
                hipGetErrorString(e));
  return VSA_ERR_HIP;
}

// 1 = gfx950, -1 = other, 0 = not yet checked (per device ordinal)
int g_arch_ok[64];

int check_device() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= 64) return VSA_ERR_UNSUPPORTED;
  if (g_arch_ok[dev] == 0) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) return hip_fail("hipGetDeviceProperties", e);
    g_arch_ok[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
  }
  return g_arch_ok[dev] == 1 ? VSA_OK : VSA_ERR_UNSUPPORTED;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (a == nullptr || b == nullptr) return false;
  const char* pa = static_cast<const char*>(a);
  const char* pb = static_cast<const char*>(b);
  return pa < pb + nb && pb < pa + na;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace

extern "C" const char* vsa_last_error(void) { return g_last_error; }

struct vsa_timer {
  struct Rec {
    int stage;
    hipEvent_t a, b;
  };
  std::vector<Rec> recs;          // recorded since the last read
  std::vector<hipEvent_t> pool;   // free events
  std::vector<std::string> names;
  std::vector<double> total_ms;
  std::vector<int> launches;

  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
  }
  int stage_id(const char* name) {
    for (size_t i = 0; i < names.size(); ++i)
      if (names[i] == name) return (int)i;
    names.emplace_back(name);
    total_ms.push_back(0.0);
    launches.push_back(0);
    return (int)names.size() - 1;
  }
};

namespace {

// Runs `launch` between two events when a timer is given.
template <class F>
int timed(vsa_timer* tm, const char* name, hipStream_t st, F&& launch) {
  if (tm == nullptr) {
    launch();
    return VSA_OK;
  }
  vsa_timer::Rec r{tm->stage_id(name), tm->get(), tm->get()};
  if (r.a == nullptr || r.b == nullptr) return VSA_ERR_HIP;
  if (hipEventRecord(r.a, st) != hipSuccess) return VSA_ERR_HIP;
  launch();
  if (hipEventRecord(r.b, st) != hipSuccess) return VSA_ERR_HIP;
  tm->recs.push_back(r);
  return VSA_OK;
}

}  // namespace

int vsa_launch_forward(const vsa_plan* plan, const void* q, const void* k, const void* v,
                       const void* g, void* o, void* workspace, void* stream, vsa_timer* tm) {
  const VsaGeom& G = plan->g;
  const VsaLayout& L = plan->ws;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  float* qbar = reinterpret_cast<float*>(ws + L.qbar);
  float* kbar = reinterpret_cast<float*>(ws + L.kbar);
  float* vbar = reinterpret_cast<float*>(ws + L.vbar);
  float* bias = reinterpret_cast<float*>(ws + L.bias);
  float* anchor = reinterpret_cast<float*>(ws + L.anchor);
  float* scores = reinterpret_cast<float*>(ws + L.scores);
  float* ocoarse = reinterpret_cast<float*>(ws + L.ocoarse);
  float* thr = reinterpret_cast<float*>(ws + L.thr);
  int* lists = reinterpret_cast<int*>(ws + L.lists);
  int* counts = reinterpret_cast<int*>(ws + L.counts);
  double* statp = reinterpret_cast<double*>(ws + L.statp);
  float* cpart = reinterpret_cast<float*>(ws + L.cpart);
  int* xtok = reinterpret_cast<int*>(ws + L.xtok);
  int* xcnt = reinterpret_cast<int*>(ws + L.xcnt);
  void* vx = ws + L.vx;
  VsaExtraBuffers xb;
  xb.tm1 = reinterpret_cast<float*>(ws + L.xtm1);
  xb.tm4 = reinterpret_cast<float*>(ws + L.xtm4);
  xb.thr = reinterpret_cast<float*>(ws + L.xthr);
  xb.mask = reinterpret_cast<unsigned*>(ws + L.xmask);
  xb.ccnt = reinterpret_cast<int*>(ws + L.xccnt);
  xb.cand = reinterpret_cast<unsigned long long*>(ws + L.xcand);
  xb.qsplit = ws + L.xqsplit;
  xb.knorm = reinterpret_cast<const float*>(ws + L.xknorm);
  xb.part = reinterpret_cast<unsigned long long*>(ws + L.xpart);
  xb.pcnt = reinterpret_cast<int*>(ws + L.xpcnt);
  xb.xtok = xtok;
  xb.xcnt = xcnt;
  xb.vx = vx;
  void* o_user = o;

  (void)hipGetLastError();  // clear a stale error so the checks below see only ours
  int rc = VSA_OK;
#define VSA_STEP(name, call)                                   \
  do {                                                         \
    rc = timed(tm, name, st, [&] { call; });                   \
    if (rc != VSA_OK) return rc;                               \
    const hipError_t e_ = hipGetLastError();                   \
    if (e_ != hipSuccess) return hip_fail(name, e_);           \
  } while (0)

  // Spark-Reblock: the mapper's leaves become the video tiles of each (b, h) by permuting the
  // inputs' video rows; the rest of the forward runs on the permuted tensors and the output
  // rows are scattered back at the end
  const int* rb_tiles = nullptr;
  if (G.reblock) {
    VSA_STEP("reblock", rb_tiles = vsa_launch_reblock(
                            G, q, k, reinterpret_cast<float*>(ws + L.rb_mpart), reinterpret_cast<float*>(ws + L.rb_m),
                            reinterpret_cast<unsigned short*>(ws + L.rb_mhl), reinterpret_cast<float*>(ws + L.rb_a0),
                            reinterpret_cast<float*>(ws + L.rb_norms),
                            reinterpret_cast<int*>(ws + L.rb_list_a), reinterpret_cast<int*>(ws + L.rb_list_b),
                            reinterpret_cast<float*>(ws + L.rb_pbuf), reinterpret_cast<float*>(ws + L.rb_part),
                            reinterpret_cast<float*>(ws + L.rb_state), st));
    void* gp = g != nullptr ? static_cast<void*>(ws + L.rb_g) : nullptr;
    VSA_STEP("permute", vsa_launch_rb_permute(G, rb_tiles, q, k, v, g, ws + L.rb_q, ws + L.rb_k, ws + L.rb_v, gp, st));
    q = ws + L.rb_q;
    k = ws + L.rb_k;
    v = ws + L.rb_v;
    g = gp;
    o = ws + L.rb_o;
  }
  // with no sparse row (the dense mode) nothing is pooled, scored or selected
  if (G.Qs > 0) {
    VSA_STEP("pool", vsa_launch_pool(G, q, k, v, qbar, kbar, vbar, bias,
                                    G.extra > 0 ? reinterpret_cast<float*>(ws + L.xknorm) : nullptr, st));
    if (G.coarse == VSA_COARSE_MEAN_LOGMASS || G.coarse == VSA_COARSE_WEIGHTED_LOGMASS) {
      VSA_STEP("anchor", vsa_launch_anchor(G, qbar, anchor, st));
      VSA_STEP("logmass", vsa_launch_logmass(G, k, v, kbar, vbar, anchor, bias, st));
    }
    VSA_STEP("coarse", vsa_launch_coarse(G, qbar, kbar, vbar, bias, scores, ocoarse, statp, cpart, st));
    if (G.select == VSA_SELECT_TAU) VSA_STEP("tau", vsa_launch_tau(G, statp, thr, st));
    VSA_STEP("select", vsa_launch_select(G, scores, thr, lists, counts, st));
    if (G.extra > 0) VSA_STEP("extra", vsa_launch_extra(G, k, v, qbar, lists, counts, xb, st));
  }
  VSA_STEP("fine", vsa_launch_fine(G, q, k, v, g, ocoarse, lists, counts, o, xtok, vx, xcnt, st));
  if (G.reblock) VSA_STEP("unpermute", vsa_launch_rb_unpermute(G, rb_tiles, o, o_user, st));
#undef VSA_STEP
  return VSA_OK;
}

namespace {

int forward_common(const vsa_plan* plan, const void* q, const void* k, const void* v, const void* g,
                   void* o, void* workspace, size_t workspace_bytes, void* stream, vsa_timer* tm) {
  if (plan == nullptr || q == nullptr || k == nullptr || v == nullptr || o == nullptr)
    return VSA_ERR_INVALID_ARGUMENT;
  if (workspace == nullptr || workspace_bytes < plan->ws.total) return VSA_ERR_WORKSPACE;
  const void* bufs[5] = {q, k, v, g, o};
  for (const void* p : bufs)
    if (p != nullptr && !aligned(p, 16)) return VSA_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 256)) return VSA_ERR_INVALID_ARGUMENT;
  const size_t tbytes = (size_t)plan->g.batch * plan->n_tokens * plan->g.heads * VSA_HEAD_DIM * 2;
  for (int i = 0; i < 4; ++i)
    if (overlaps(o, tbytes, bufs[i], tbytes)) return VSA_ERR_INVALID_ARGUMENT;
  if (overlaps(o, tbytes, workspace, plan->ws.total)) return VSA_ERR_INVALID_ARGUMENT;
  for (int i = 0; i < 4; ++i)
    if (overlaps(workspace, plan->ws.total, bufs[i], tbytes)) return VSA_ERR_INVALID_ARGUMENT;
  const int dev = check_device();
  if (dev != VSA_OK) return dev;
  const int rc = vsa_launch_forward(plan, q, k, v, g, o, workspace, stream, tm);
  if (log_enabled()) {
    const VsaGeom& G = plan->g;
    std::fprintf(stderr,
                 "[vsa] forward B=%d N=%d heads=%d P=%d Vt=%d k=%d sink=%d select=%d coarse=%d "
                 "tau=%g gate=%d status=%d %s\n",
                 G.batch, G.N, G.heads, G.P, G.Vt, G.k, G.sink, G.select, G.coarse, (double)G.tau,
                 g != nullptr, rc, rc == VSA_ERR_HIP ? g_last_error : "");
  }
  return rc;
}

}  // namespace

extern "C" int vsa_forward(const vsa_plan* plan, const void* q, const void* k, const void* v,
                           const void* g, void* o, void* workspace, size_t workspace_bytes,
                           void* stream) {
  return forward_common(plan, q, k, v, g, o, workspace, workspace_bytes, stream, nullptr);
}

// ---- the no-allocation forward ---------------------------------------------------
// The workspace of vsa_forward_noalloc: one static device array per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in, not a device address:
// the host only ever uses the per-device address that hipGetSymbolAddress returns.
static __device__ __align__(256) unsigned char scratch[VSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch` on each device, once looked up

// Address of the scratch array on the current device, looked up on the first call there
// (with that device current).  No allocation.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail("hipGetDevice", e);
  if (dev < 0 || dev >= kMaxDevices) return VSA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail("hipGetSymbolAddress(scratch)", e);
    if (ptr == nullptr) return hip_fail("hipGetSymbolAddress(scratch)", hipErrorInvalidSymbol);
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return VSA_OK;
}

}  // namespace

extern "C" int vsa_forward_noalloc(const vsa_plan* plan, const void* q, const void* k, const void* v,
                                   const void* g, void* o, void* stream) {
  if (plan == nullptr || q == nullptr || k == nullptr || v == nullptr || o == nullptr)
    return VSA_ERR_INVALID_ARGUMENT;
  if (plan->ws.total > VSA_NOALLOC_SCRATCH_BYTES) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "vsa_forward_noalloc: the plan needs %zu workspace bytes; the static scratch holds %zu",
                  plan->ws.total, (size_t)VSA_NOALLOC_SCRATCH_BYTES);
    return VSA_ERR_WORKSPACE;
  }
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != VSA_OK) return rc;
  return forward_common(plan, q, k, v, g, o, ws, VSA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

extern "C" int vsa_forward_timed(const vsa_plan* plan, const void* q, const void* k, const void* v,
                                 const void* g, void* o, void* workspace, size_t workspace_bytes,
                                 void* stream, vsa_timer* timer) {
  if (timer == nullptr) return VSA_ERR_INVALID_ARGUMENT;
  return forward_common(plan, q, k, v, g, o, workspace, workspace_bytes, stream, timer);
}

extern "C" int vsa_read_stats(const vsa_plan* plan, const void* workspace, void* stream,
                              vsa_stats* out) {
  if (plan == nullptr || workspace == nullptr || out == nullptr) return VSA_ERR_INVALID_ARGUMENT;
  const VsaGeom& G = plan->g;
  const size_t n = (size_t)G.batch * G.heads * G.Qs;
  std::vector<int> cnt(n), xc(G.extra > 0 ? n : 0);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (n > 0) {
    const char* ws = static_cast<const char*>(workspace);
    if (hipMemcpyAsync(cnt.data(), ws + plan->ws.counts, n * sizeof(int), hipMemcpyDeviceToHost,
                       st) != hipSuccess)
      return VSA_ERR_HIP;
    if (G.extra > 0 && hipMemcpyAsync(xc.data(), ws + plan->ws.xcnt, n * sizeof(int), hipMemcpyDeviceToHost,
                                      st) != hipSuccess)
      return VSA_ERR_HIP;
  }
  if (hipStreamSynchronize(st) != hipSuccess) return VSA_ERR_HIP;
  const int64_t BH = (int64_t)G.batch * G.heads;
  int64_t pairs = BH * G.n_dense * (int64_t)G.Tq, kept = 0, extra = 0;
  for (size_t i = 0; i < n; ++i) {
    pairs += cnt[i];
    kept += cnt[i] - G.npin;
  }
  for (size_t i = 0; i < xc.size(); ++i) {
    pairs += xc[i] > 0 ? 1 : 0;  // the extra tokens' tile
    extra += xc[i];
  }
  out->executed_pairs = pairs;
  out->dense_pairs = BH * (int64_t)G.Tq * G.Tq;
  out->sparse_rows = BH * G.Qs;
  out->dense_rows = BH * G.n_dense;
  out->kept_video_tiles = kept;
  out->k = G.k;
  out->reserved = 0;
  out->extra_tokens = extra;
  return VSA_OK;
}

extern "C" int vsa_timer_create(vsa_timer** out) {
  if (out == nullptr) return VSA_ERR_INVALID_ARGUMENT;
  *out = new (std::nothrow) vsa_timer();
  return *out == nullptr ? VSA_ERR_NO_MEMORY : VSA_OK;
}

extern "C" int vsa_timer_destroy(vsa_timer* t) {
  if (t == nullptr) return VSA_OK;
  for (auto& r : t->recs) {
    (void)hipEventDestroy(r.a);
    (void)hipEventDestroy(r.b);
  }
  for (auto e : t->pool) (void)hipEventDestroy(e);
  delete t;
  return VSA_OK;
}

namespace {
int drain(vsa_timer* t) {
  for (auto& r : t->recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return VSA_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return VSA_ERR_HIP;
    t->total_ms[r.stage] += ms;
    t->launches[r.stage] += 1;
    t->pool.push_back(r.a);
    t->pool.push_back(r.b);
  }
  t->recs.clear();
  return VSA_OK;
}
}  // namespace

extern "C" int vsa_timer_reset(vsa_timer* t) {
  if (t == nullptr) return VSA_ERR_INVALID_ARGUMENT;
  const int rc = drain(t);
  for (auto& x : t->total_ms) x = 0.0;
  for (auto& x : t->launches) x = 0;
  return rc;
}

extern "C" int vsa_timer_read(vsa_timer* t, vsa_kernel_time* out, int max, int* n) {
  if (t == nullptr || n == nullptr || (out == nullptr && max > 0)) return VSA_ERR_INVALID_ARGUMENT;
  const int rc = drain(t);
  if (rc != VSA_OK) return rc;
  const int m = (int)t->names.size();
  for (int i = 0; i < m && i < max; ++i) {
    std::memset(out[i].name, 0, sizeof(out[i].name));
    std::strncpy(out[i].name, t->names[i].c_str(), sizeof(out[i].name) - 1);
    out[i].launches = t->launches[i];
    out[i].total_ms = t->total_ms[i];
  }
  *n = m;
  return VSA_OK;
}
