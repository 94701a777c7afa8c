// Geometry gather + mean pooling, and the log-mass anchor and bias.
//
// Pooling: the compressed branch summarises each tile by the mean of its
// tokens ("Spark-H3: atencion dispersa por bloques acelera MiniMax-H3 en
// ComfyUI", "Que cambia Spark-Attn"; "ComfyUI Agrega Nodo Central de Atencion
// Dispersa...", VSA item: cubic tiling plus a coarse compression branch).
// Log-mass bias: same Spark page, Spark-Reweight item: mean pooling stands
// exp(E[x]) in for E[exp(x)]; a bias per tile, scored with the mean video
// query as the anchor, restores the missing mass.  The same item's weighted
// summaries replace the means by the anchor's attention over each tile.
// K and V summaries and biases cover the candidate key tiles [kc0, kc0 + Kc):
// the video tiles, or every tile when sink_conditioning is off ("BSAI FastH3
// Native VSA (recipe)", "The inputs that matter"); a partial prefix tile is
// summarised over its valid tokens.
//
// With extra tokens the step also writes every tile's largest key L2 norm, from the
// key rows it holds (loading K for a prefix tile that is no key candidate): the
// extra-token screen's error bound scales with it.
//
// HBM-bound: each (tile, head) slice of Q, K, V is read once; one wave per
// (tile, head), 16 lanes per token (16 x 16 B = one 256-byte head row), four
// tokens per load instruction; a candidate tile's 48 loads (Q, K, V) are all in flight at once.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

// This wave's 64 tile rows of one head: lane group grp = lane/16 owns rows 4p + grp, lane
// chunk c = lane%16 owns dims 8c..8c+7.  tile_load only issues the loads, so a wave can
// have the Q, K and V rows of a tile in flight at once; tile_sum reduces them over the
// four groups (every lane holds its chunk's sums).  VIDEO: t is a video tile, whose 64
// rows are all valid, so the loads need no padding test.
template <bool VIDEO>
__device__ __forceinline__ void tile_load(const VsaGeom& g, const u32x4* __restrict__ X, int b, int h,
                                          int t, int grp, int c, u32x4 buf[16]) {
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    if (VIDEO) {
      buf[p] = X[row_offset(g, b, video_token(g, t, 4 * p + grp), h) / 8 + c];
    } else {
      const int tok = tile_token(g, t, 4 * p + grp);
      if (tok >= 0)
        buf[p] = X[row_offset(g, b, tok, h) / 8 + c];
      else
        buf[p] = u32x4{0u, 0u, 0u, 0u};
    }
  }
}
__device__ __forceinline__ void tile_sum(const u32x4 buf[16], float acc[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc[2 * w] += bf16lo(buf[p][w]);
      acc[2 * w + 1] += bf16hi(buf[p][w]);
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = group_sum(acc[i]);
}

// The largest L2 norm among the tile's 64 rows in buf (laid out as tile_load leaves them;
// padding rows are zero), in every lane.  Each lane first sums the squares of its 8 dims of
// its 16 rows; the 16 lanes of a row then add their sums in four exchange steps, each lane
// keeping half of the rows it still holds (after the steps lane c holds row 4c + grp whole),
// and a max over the wave ends it.  Used to bound the extra-token screen's error.
__device__ __forceinline__ float tile_max_norm(const u32x4 buf[16], int lane) {
  float s16[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float lo = bf16lo(buf[p][w]), hi = bf16hi(buf[p][w]);
      a = fmaf(lo, lo, a);
      a = fmaf(hi, hi, a);
    }
    s16[p] = a;
  }
  const bool b3 = lane & 8, b2 = lane & 4, b1 = lane & 2, b0 = lane & 1;
  float s8[8], s4[4], s2[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) s8[i] = (b3 ? s16[i + 8] : s16[i]) + __shfl_xor(b3 ? s16[i] : s16[i + 8], 8);
#pragma unroll
  for (int i = 0; i < 4; ++i) s4[i] = (b2 ? s8[i + 4] : s8[i]) + __shfl_xor(b2 ? s8[i] : s8[i + 4], 4);
#pragma unroll
  for (int i = 0; i < 2; ++i) s2[i] = (b1 ? s4[i + 2] : s4[i]) + __shfl_xor(b1 ? s4[i] : s4[i + 2], 2);
  const float m = (b0 ? s2[1] : s2[0]) + __shfl_xor(b0 ? s2[0] : s2[1], 1);
  return sqrtf(wave_max(m));
}

__device__ __forceinline__ void store8(float* dst, const float v[8], float mul) {
  f32x4* d4 = reinterpret_cast<f32x4*>(dst);
  d4[0] = f32x4{v[0] * mul, v[1] * mul, v[2] * mul, v[3] * mul};
  d4[1] = f32x4{v[4] * mul, v[5] * mul, v[6] * mul, v[7] * mul};
}

// Q-bar of tile t, and K-bar / V-bar when KV (t is a candidate key tile); with KN also the
// tile's largest key norm (every tile).
template <bool VIDEO, bool KV, bool KN>
__device__ __forceinline__ void pool_tile(const VsaGeom& g, const u32x4* __restrict__ q,
                                          const u32x4* __restrict__ k, const u32x4* __restrict__ v,
                                          float* __restrict__ qbar, float* __restrict__ kbar,
                                          float* __restrict__ vbar, float* __restrict__ bias,
                                          float* __restrict__ knorm, int b, int h, int t, int lane) {
  const int grp = lane >> 4, c = lane & 15;
  const size_t bh = (size_t)b * g.heads + h;
  const float inv = VIDEO ? 1.0f / VSA_TILE_TOKENS : 1.0f / (float)tile_valid(g, t);
  float acc[8];
  u32x4 bq[16];
  tile_load<VIDEO>(g, q, b, h, t, grp, c, bq);
  if (!KV) {
    tile_sum(bq, acc);
    if (grp == 0) store8(qbar + (bh * g.Tq + t) * VSA_HEAD_DIM + 8 * c, acc, inv);
    if (KN) {
      u32x4 bk[16];
      tile_load<VIDEO>(g, k, b, h, t, grp, c, bk);
      const float n = tile_max_norm(bk, lane);
      if (lane == 0) knorm[bh * g.Tq + t] = n;
    }
    return;
  }
  // candidate key tile: all 48 loads in flight before the first sum
  u32x4 bk[16], bv[16];
  tile_load<VIDEO>(g, k, b, h, t, grp, c, bk);
  tile_load<VIDEO>(g, v, b, h, t, grp, c, bv);
  const int j = t - g.kc0;
  tile_sum(bq, acc);
  if (grp == 0) store8(qbar + (bh * g.Tq + t) * VSA_HEAD_DIM + 8 * c, acc, inv);
  if (KN) {
    const float n = tile_max_norm(bk, lane);
    if (lane == 0) knorm[bh * g.Tq + t] = n;
  }
  tile_sum(bk, acc);
  if (grp == 0) store8(kbar + (bh * g.Kc + j) * VSA_HEAD_DIM + 8 * c, acc, inv);
  tile_sum(bv, acc);
  if (grp == 0) store8(vbar + (bh * g.Kc + j) * VSA_HEAD_DIM + 8 * c, acc, inv);
  if (g.coarse == VSA_COARSE_MEAN && lane == 0) bias[bh * g.Kc + j] = 0.0f;
}

template <bool KN>
__global__ __launch_bounds__(256) void vsa_pool_kernel(VsaGeom g, const u32x4* __restrict__ q,
                                                       const u32x4* __restrict__ k,
                                                       const u32x4* __restrict__ v,
                                                       float* __restrict__ qbar,
                                                       float* __restrict__ kbar,
                                                       float* __restrict__ vbar,
                                                       float* __restrict__ bias,
                                                       float* __restrict__ knorm) {
  // head groups fastest: consecutive workgroups read neighbouring 1 KB pieces of the same
  // token rows, which keeps HBM page locality
  const int t = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + wave;
  const int b = blockIdx.z;
  if (h >= g.heads) return;
  if (t >= g.P)  // video tiles are always candidates
    pool_tile<true, true, KN>(g, q, k, v, qbar, kbar, vbar, bias, knorm, b, h, t, lane);
  else if (t >= g.kc0)  // prefix candidate (sink off)
    pool_tile<false, true, KN>(g, q, k, v, qbar, kbar, vbar, bias, knorm, b, h, t, lane);
  else
    pool_tile<false, false, KN>(g, q, k, v, qbar, kbar, vbar, bias, knorm, b, h, t, lane);
}

// q_a = mean of the video tiles' qbar (every video tile holds 64 tokens, so
// this is the mean of all video queries).  Fixed-order reduction.
__global__ __launch_bounds__(1024) void vsa_anchor_kernel(VsaGeom g, const float* __restrict__ qbar,
                                                          float* __restrict__ anchor) {
  __shared__ float part[8][VSA_HEAD_DIM];
  const int d = threadIdx.x & 127, slice = threadIdx.x >> 7;
  const size_t bh = (size_t)blockIdx.y * g.heads + blockIdx.x;
  const float* base = qbar + (bh * g.Tq + g.P) * VSA_HEAD_DIM + d;
  float s = 0.f;
  for (int j = slice; j < g.Vt; j += 8) s += base[(size_t)j * VSA_HEAD_DIM];
  part[slice][d] = s;
  __syncthreads();
  if (slice == 0) {
    float tot = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) tot += part[i][d];
    anchor[bh * VSA_HEAD_DIM + d] = tot / (float)g.Vt;
  }
}

// b_j = log(mean_t exp(s q_a . (k_t - kbar_j))), max-shifted, means and sums over the
// tile's valid tokens.  One wave per (candidate tile, head).  WEIGHTED (Spark-Reweight's weighted summaries, read as the
// anchor's attention over the tile): with the centred logits l'_t = s q_a . (k_t - kbar_j)
// and w_t = softmax_t(l'_t), the kernel also writes
//   ktil_j = kbar_j + sum_t w_t (k_t - kbar_j),  vtil_j = sum_t w_t v_t
// over kbar_j and vbar_j, and the bias b_j = log(mean_t exp(l'_t)) - sum_t w_t l'_t, which is
// log(mean_t exp(s q_a . k_t)) - s q_a . ktil_j.
// PARTIAL: the launch covers prefix candidate tiles (sink off), which may hold padding
// rows; a video tile always holds 64 tokens, so its launch skips the masking.
template <bool WEIGHTED, bool PARTIAL>
__global__ __launch_bounds__(256) void vsa_logmass_kernel(VsaGeom g, int t_first, const u32x4* __restrict__ k,
                                                          const u32x4* __restrict__ v,
                                                          float* __restrict__ kbar,
                                                          float* __restrict__ vbar,
                                                          const float* __restrict__ anchor,
                                                          float* __restrict__ bias) {
  const int t = t_first + blockIdx.y;
  const int j = t - g.kc0;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + wave;
  const int b = blockIdx.z;
  if (h >= g.heads) return;
  const int grp = lane >> 4, c = lane & 15;
  const size_t bh = (size_t)b * g.heads + h;
  float qa[8], kb[8];
  const f32x4* a4 = reinterpret_cast<const f32x4*>(anchor + bh * VSA_HEAD_DIM + 8 * c);
  const f32x4* k4 = reinterpret_cast<const f32x4*>(kbar + (bh * g.Kc + j) * VSA_HEAD_DIM + 8 * c);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    qa[i] = a4[0][i];
    qa[4 + i] = a4[1][i];
    kb[i] = k4[0][i];
    kb[4 + i] = k4[1][i];
  }
  // rows 4 p + grp of the tile, dims 8 c .. 8 c + 7.  A padding row of a partial prefix
  // tile reloads row 0 (always valid) and takes no part: ok bit p clear, weight 0.
  u32x4 buf[16], vbuf[16];
  unsigned ok = 0xffffu;
  const int tok0 = PARTIAL ? tile_token(g, t, 0) : 0;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    int tok = PARTIAL ? tile_token(g, t, 4 * p + grp) : video_token(g, t, 4 * p + grp);
    if (PARTIAL) {
      if (tok < 0) {
        ok &= ~(1u << p);
        tok = tok0;
      }
    }
    const long long ro = row_offset(g, b, tok, h) / 8 + c;
    buf[p] = k[ro];
    if (WEIGHTED) vbuf[p] = v[ro];
  }
  float ell[16];
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      s += qa[2 * w] * (bf16lo(buf[p][w]) - kb[2 * w]);
      s += qa[2 * w + 1] * (bf16hi(buf[p][w]) - kb[2 * w + 1]);
    }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) s += __shfl_xor(s, m);
    ell[p] = s * g.scale;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int p = 0; p < 16; ++p)
    if (!PARTIAL || (ok & (1u << p))) mx = fmaxf(mx, ell[p]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  float e[16], se = 0.f;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    e[p] = (!PARTIAL || (ok & (1u << p))) ? expf(ell[p] - mx) : 0.f;  // row 0 is always valid
    se += e[p];
  }
  se += __shfl_xor(se, 16);
  se += __shfl_xor(se, 32);
  const float nvalid = PARTIAL ? (float)tile_valid(g, t) : (float)VSA_TILE_TOKENS;
  const float lme = mx + logf(se / nvalid);  // log mean exp of the l'_t
  if (!WEIGHTED) {
    if (lane == 0) bias[bh * g.Kc + j] = lme;
    return;
  }
  // weighted sums over this lane's rows, then over the four row groups
  float ew = 0.f, ak[8], av[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) ak[i] = av[i] = 0.f;
#pragma unroll
  for (int p = 0; p < 16; ++p) {
    ew += e[p] * ell[p];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      ak[2 * w] += e[p] * (bf16lo(buf[p][w]) - kb[2 * w]);
      ak[2 * w + 1] += e[p] * (bf16hi(buf[p][w]) - kb[2 * w + 1]);
      av[2 * w] += e[p] * bf16lo(vbuf[p][w]);
      av[2 * w + 1] += e[p] * bf16hi(vbuf[p][w]);
    }
  }
  ew += __shfl_xor(ew, 16);
  ew += __shfl_xor(ew, 32);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ak[i] += __shfl_xor(ak[i], 16);
    ak[i] += __shfl_xor(ak[i], 32);
    av[i] += __shfl_xor(av[i], 16);
    av[i] += __shfl_xor(av[i], 32);
  }
  const float inv = 1.0f / se;
  if (grp == 0) {
    float kt[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) kt[i] = kb[i] + ak[i] * inv;
    store8(kbar + (bh * g.Kc + j) * VSA_HEAD_DIM + 8 * c, kt, 1.0f);
    store8(vbar + (bh * g.Kc + j) * VSA_HEAD_DIM + 8 * c, av, inv);
  }
  if (lane == 0) bias[bh * g.Kc + j] = lme - ew * inv;
}

}  // namespace

void vsa_launch_pool(const VsaGeom& g, const void* q, const void* k, const void* v, float* qbar,
                     float* kbar, float* vbar, float* bias, float* knorm, hipStream_t st) {
  dim3 grid((g.heads + 3) / 4, g.Tq, g.batch);
  if (knorm != nullptr)
    hipLaunchKernelGGL(vsa_pool_kernel<true>, grid, dim3(256), 0, st, g, (const u32x4*)q, (const u32x4*)k,
                       (const u32x4*)v, qbar, kbar, vbar, bias, knorm);
  else
    hipLaunchKernelGGL(vsa_pool_kernel<false>, grid, dim3(256), 0, st, g, (const u32x4*)q, (const u32x4*)k,
                       (const u32x4*)v, qbar, kbar, vbar, bias, knorm);
}

void vsa_launch_anchor(const VsaGeom& g, const float* qbar, float* anchor, hipStream_t st) {
  hipLaunchKernelGGL(vsa_anchor_kernel, dim3(g.heads, g.batch), dim3(1024), 0, st, g, qbar, anchor);
}

namespace {
template <bool WEIGHTED>
void launch_logmass(const VsaGeom& g, const void* k, const void* v, float* kbar, float* vbar,
                    const float* anchor, float* bias, hipStream_t st) {
  const dim3 block(256);
  // prefix candidates (sink off only), then the video tiles
  if (g.kc0 < g.P) {
    dim3 grid((g.heads + 3) / 4, g.P - g.kc0, g.batch);
    hipLaunchKernelGGL((vsa_logmass_kernel<WEIGHTED, true>), grid, block, 0, st, g, g.kc0, (const u32x4*)k,
                       (const u32x4*)v, kbar, vbar, anchor, bias);
  }
  dim3 grid((g.heads + 3) / 4, g.Vt, g.batch);
  hipLaunchKernelGGL((vsa_logmass_kernel<WEIGHTED, false>), grid, block, 0, st, g, g.P, (const u32x4*)k,
                     (const u32x4*)v, kbar, vbar, anchor, bias);
}
}  // namespace

void vsa_launch_logmass(const VsaGeom& g, const void* k, const void* v, float* kbar, float* vbar,
                        const float* anchor, float* bias, hipStream_t st) {
  if (g.coarse == VSA_COARSE_WEIGHTED_LOGMASS)
    launch_logmass<true>(g, k, v, kbar, vbar, anchor, bias, st);
  else
    launch_logmass<false>(g, k, v, kbar, vbar, anchor, bias, st);
}
