// Wave-level selector: per sparse query tile, the list of key tiles the fine
// branch runs.
//
// "BSAI FastH3 Native VSA (recipe)", "The mechanism, briefly": blocks are
// scored and exact attention runs only on the top share.  "ComfyUI Agrega
// Nodo Central de Atencion Dispersa...", "un nodo, tres backends": top-k keeps
// a fixed share of key blocks; Sol-Attn keeps blocks above a per-head
// threshold in standard deviations.  "Ref2VA VSA : noeud d'attention sparse
// pour le Ref2VA H3", items 1-2: the conditioning tiles are never pruned; top-k
// applies to video key tiles only.  "BSAI FastH3 Native VSA (recipe)", "The
// inputs that matter": with sink_conditioning off nothing is protected, and
// every tile is a candidate.
//
// One wave per row.  The Kc candidate logits of the row (tiles kc0 .. kc0 +
// Kc - 1) sit in registers as order-preserving 32-bit keys (lane l, slot e
// holds candidate 64 e + l, so slot-major order is index order).  TOPK: an
// MSB-first bitwise search finds the k-th largest key T in 32 ballot rounds;
// every key > T is kept, and the keys equal to T are kept lowest index first
// until k are kept.  TAU: keep S > thr.  Kept tiles are compacted in
// ascending order with ballot + mbcnt after the npin protected prefix tile ids
// (P, or none with sink off).  Integer output, no atomics: deterministic.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

// Order-preserving map float -> uint32 (larger float, larger key); -0 == +0.
__device__ __forceinline__ unsigned int order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const unsigned int u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((unsigned int)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((unsigned int)mask, 0u));
}

template <int NPL>
__global__ __launch_bounds__(256) void vsa_select_kernel(VsaGeom g, const float* __restrict__ scores,
                                                         const float* __restrict__ thr,
                                                         int* __restrict__ lists,
                                                         int* __restrict__ counts) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + wave;
  if (s >= g.Qs) return;
  const size_t bh = (size_t)blockIdx.z * g.heads + blockIdx.y;
  const float* S = scores + (bh * g.Qs + s) * g.Kc;
  int* L = lists + (bh * g.Qs + s) * g.cap;

  unsigned int key[NPL];  // padding slots hold 0, below every real key
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const int j = e * 64 + lane;
    key[e] = j < g.Kc ? order_key(S[j]) : 0u;
  }
  for (int t = lane; t < g.npin; t += 64) L[t] = t;

  unsigned int T;
  int need_eq;  // keys equal to T still to keep (TOPK); unused for TAU
  if (g.select == VSA_SELECT_TOPK) {
    unsigned int prefix = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned int cand = prefix | (1u << bit);
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < NPL; ++e) cnt += __popcll(__ballot(key[e] >= cand));
      if (cnt >= g.k) prefix = cand;
    }
    T = prefix;
    int gt = 0;
#pragma unroll
    for (int e = 0; e < NPL; ++e) gt += __popcll(__ballot(key[e] > T));
    need_eq = g.k - gt;
  } else {
    T = order_key(thr[bh]);
    need_eq = 0;
  }

  int base = 0, eq_seen = 0;
#pragma unroll
  for (int e = 0; e < NPL; ++e) {
    const bool gt = key[e] > T;
    const unsigned long long beq = __ballot(key[e] == T && key[e] != 0u);
    const bool eq_take = ((beq >> lane) & 1ull) && (eq_seen + lanes_below(beq) < need_eq);
    eq_seen += __popcll(beq);
    const bool take = gt || eq_take;
    const unsigned long long bt = __ballot(take);
    if (take) L[g.npin + base + lanes_below(bt)] = g.kc0 + e * 64 + lane;
    base += __popcll(bt);
  }
  if (lane == 0) counts[bh * g.Qs + s] = g.npin + base;
}

template <int NPL>
void launch_npl(const VsaGeom& g, const float* scores, const float* thr, int* lists, int* counts,
                hipStream_t st) {
  dim3 grid((g.Qs + 3) / 4, g.heads, g.batch);
  hipLaunchKernelGGL(vsa_select_kernel<NPL>, grid, dim3(256), 0, st, g, scores, thr, lists, counts);
}

}  // namespace

void vsa_launch_select(const VsaGeom& g, const float* scores, const float* thr, int* lists,
                       int* counts, hipStream_t st) {
  if (g.Qs == 0) return;
  // slots per lane; exact up to 16, so no all-padding slot joins the 32 ballot rounds
  const int npl = (g.Kc + 63) / 64;
  switch (npl) {
    case 1: launch_npl<1>(g, scores, thr, lists, counts, st); break;
    case 2: launch_npl<2>(g, scores, thr, lists, counts, st); break;
    case 3: launch_npl<3>(g, scores, thr, lists, counts, st); break;
    case 4: launch_npl<4>(g, scores, thr, lists, counts, st); break;
    case 5: launch_npl<5>(g, scores, thr, lists, counts, st); break;
    case 6: launch_npl<6>(g, scores, thr, lists, counts, st); break;
    case 7: launch_npl<7>(g, scores, thr, lists, counts, st); break;
    case 8: launch_npl<8>(g, scores, thr, lists, counts, st); break;
    case 9: launch_npl<9>(g, scores, thr, lists, counts, st); break;
    case 10: launch_npl<10>(g, scores, thr, lists, counts, st); break;
    case 11: launch_npl<11>(g, scores, thr, lists, counts, st); break;
    case 12: launch_npl<12>(g, scores, thr, lists, counts, st); break;
    case 13: launch_npl<13>(g, scores, thr, lists, counts, st); break;
    case 14: launch_npl<14>(g, scores, thr, lists, counts, st); break;
    case 15: launch_npl<15>(g, scores, thr, lists, counts, st); break;
    case 16: launch_npl<16>(g, scores, thr, lists, counts, st); break;
    default:
      if (npl <= 32) launch_npl<32>(g, scores, thr, lists, counts, st);
      else launch_npl<64>(g, scores, thr, lists, counts, st);
  }
}
