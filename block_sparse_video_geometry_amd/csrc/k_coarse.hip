// Coarse branch: pooled logits, row softmax, O_coarse, and the tau statistics.
//
// "ComfyUI Agrega Nodo Central de Atencion Dispersa...", section "un nodo,
// tres backends": VSA scores cubic tiles through a coarse compression branch;
// Sol-Attn thresholds each head at a number of standard deviations of its
// score distribution.  "Spark-H3...", "Que cambia Spark-Attn": the compressed
// branch attends over mean-pooled summaries.
//
// S_ij = s qbar_i . kbar_j + b_j for every sparse query tile i and every
// video key tile j; P = softmax_j(S); O_c,i = sum_j P_ij vbar_j.  All fp32
// (the ranking must hold the oracle's order wherever its logit gap > 1e-4;
// bf16 inputs to this dot product would not).  Small next to the fine
// branch: ~4.6 GFLOP fp32 at 32 heads x 564 tiles.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

constexpr int ROWS = VSA_COARSE_ROWS;  // 32 sparse rows per workgroup
constexpr int CHUNK = 64;              // video tiles per LDS chunk
constexpr int LDSW = VSA_HEAD_DIM + 4; // padded row (floats)

__global__ __launch_bounds__(256) void vsa_scores_kernel(VsaGeom g, const float* __restrict__ qbar,
                                                         const float* __restrict__ kbar,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ scores,
                                                         double* __restrict__ statp) {
  __shared__ float qs[ROWS][LDSW];
  __shared__ float ks[CHUNK][LDSW];
  __shared__ double red[4][2];
  const int tid = threadIdx.x;
  const int blk = blockIdx.x;
  const size_t bh = (size_t)blockIdx.z * g.heads + blockIdx.y;
  const int s0 = blk * ROWS;
  for (int i = tid; i < ROWS * 32; i += 256) {
    const int r = i >> 5, c4 = i & 31;
    f32x4 x = {0.f, 0.f, 0.f, 0.f};
    if (s0 + r < g.Qs)
      x = reinterpret_cast<const f32x4*>(qbar + (bh * g.Tq + g.n_dense + s0 + r) * VSA_HEAD_DIM)[c4];
    *reinterpret_cast<f32x4*>(&qs[r][4 * c4]) = x;
  }
  const int ty = tid >> 4, tx = tid & 15;
  const float* bias_bh = bias + bh * g.Vt;
  double ssum = 0.0, ssq = 0.0;
  for (int j0 = 0; j0 < g.Vt; j0 += CHUNK) {
    __syncthreads();
    for (int i = tid; i < CHUNK * 32; i += 256) {
      const int r = i >> 5, c4 = i & 31;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (j0 + r < g.Vt)
        x = reinterpret_cast<const f32x4*>(kbar + (bh * g.Vt + j0 + r) * VSA_HEAD_DIM)[c4];
      *reinterpret_cast<f32x4*>(&ks[r][4 * c4]) = x;
    }
    __syncthreads();
    float acc[2][4];
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int m = 0; m < 4; ++m) acc[r][m] = 0.f;
#pragma unroll 4
    for (int d = 0; d < VSA_HEAD_DIM; d += 4) {
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(&qs[2 * ty][d]);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(&qs[2 * ty + 1][d]);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const f32x4 bv = *reinterpret_cast<const f32x4*>(&ks[tx + 16 * m][d]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[0][m] = fmaf(a0[e], bv[e], acc[0][m]);
          acc[1][m] = fmaf(a1[e], bv[e], acc[1][m]);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int s = s0 + 2 * ty + r;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int j = j0 + tx + 16 * m;
        if (s < g.Qs && j < g.Vt) {
          const float S = acc[r][m] * g.scale + bias_bh[j];
          scores[(bh * g.Qs + s) * g.Vt + j] = S;
          ssum += (double)S;
          ssq += (double)S * (double)S;
        }
      }
    }
  }
  if (g.select != VSA_SELECT_TAU) return;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    ssum += __shfl_xor(ssum, m);
    ssq += __shfl_xor(ssq, m);
  }
  if ((tid & 63) == 0) {
    red[tid >> 6][0] = ssum;
    red[tid >> 6][1] = ssq;
  }
  __syncthreads();
  if (tid == 0) {
    double a = 0.0, q = 0.0;
    for (int w = 0; w < 4; ++w) {
      a += red[w][0];
      q += red[w][1];
    }
    statp[(bh * g.coarse_blocks + blk) * 2 + 0] = a;
    statp[(bh * g.coarse_blocks + blk) * 2 + 1] = q;
  }
}

constexpr int OROWS = 16;  // sparse rows per workgroup of the output kernel
constexpr int OCH = 32;    // video tiles per chunk

__global__ __launch_bounds__(256) void vsa_coarse_out_kernel(VsaGeom g, const float* __restrict__ scores,
                                                             const float* __restrict__ vbar,
                                                             float* __restrict__ ocoarse) {
  __shared__ float rowm[OROWS], rowinv[OROWS];
  __shared__ float vs[OCH][VSA_HEAD_DIM];
  __shared__ float ps[OROWS][OCH + 1];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const size_t bh = (size_t)blockIdx.z * g.heads + blockIdx.y;
  const int s0 = blockIdx.x * OROWS;
  for (int rr = 0; rr < OROWS / 4; ++rr) {
    const int r = wave * (OROWS / 4) + rr;
    const int s = s0 + r;
    float mx = -INFINITY, se = 0.f;
    if (s < g.Qs) {
      const float* S = scores + (bh * g.Qs + s) * g.Vt;
      for (int j = lane; j < g.Vt; j += 64) mx = fmaxf(mx, S[j]);
      mx = wave_max(mx);
      for (int j = lane; j < g.Vt; j += 64) se += expf(S[j] - mx);
      se = wave_sum(se);
    }
    if (lane == 0) {
      rowm[r] = mx;
      rowinv[r] = s < g.Qs ? 1.0f / se : 0.f;
    }
  }
  const int r = tid >> 4, c0 = (tid & 15) * 8;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j0 = 0; j0 < g.Vt; j0 += OCH) {
    __syncthreads();
    for (int i = tid; i < OCH * 32; i += 256) {
      const int jr = i >> 5, c4 = i & 31;
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
      if (j0 + jr < g.Vt)
        x = reinterpret_cast<const f32x4*>(vbar + (bh * g.Vt + j0 + jr) * VSA_HEAD_DIM)[c4];
      *reinterpret_cast<f32x4*>(&vs[jr][4 * c4]) = x;
    }
    for (int i = tid; i < OROWS * OCH; i += 256) {
      const int pr = i / OCH, pj = i % OCH;
      const int s = s0 + pr, j = j0 + pj;
      float p = 0.f;
      if (s < g.Qs && j < g.Vt) p = expf(scores[(bh * g.Qs + s) * g.Vt + j] - rowm[pr]) * rowinv[pr];
      ps[pr][pj] = p;
    }
    __syncthreads();
#pragma unroll 8
    for (int jj = 0; jj < OCH; ++jj) {
      const float p = ps[r][jj];
      const f32x4 v0 = *reinterpret_cast<const f32x4*>(&vs[jj][c0]);
      const f32x4 v1 = *reinterpret_cast<const f32x4*>(&vs[jj][c0 + 4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] = fmaf(p, v0[e], acc[e]);
        acc[4 + e] = fmaf(p, v1[e], acc[4 + e]);
      }
    }
  }
  const int s = s0 + r;
  if (s < g.Qs) {
    f32x4* dst = reinterpret_cast<f32x4*>(ocoarse + (bh * g.Qs + s) * VSA_HEAD_DIM + c0);
    dst[0] = f32x4{acc[0], acc[1], acc[2], acc[3]};
    dst[1] = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

// thr = mu + tau * sigma (population) over all Qs * Vt logits of a (batch, head).
__global__ void vsa_tau_kernel(VsaGeom g, const double* __restrict__ statp, float* __restrict__ thr) {
  const size_t bh = (size_t)blockIdx.y * g.heads + blockIdx.x;
  if (threadIdx.x != 0) return;
  double a = 0.0, q = 0.0;
  for (int i = 0; i < g.coarse_blocks; ++i) {
    a += statp[(bh * g.coarse_blocks + i) * 2 + 0];
    q += statp[(bh * g.coarse_blocks + i) * 2 + 1];
  }
  const double n = (double)g.Qs * (double)g.Vt;
  const double mu = a / n;
  double var = q / n - mu * mu;
  if (var < 0.0) var = 0.0;
  thr[bh] = (float)(mu + (double)g.tau * sqrt(var));
}

}  // namespace

void vsa_launch_scores(const VsaGeom& g, const float* qbar, const float* kbar, const float* bias,
                       float* scores, double* statp, hipStream_t st) {
  if (g.Qs == 0) return;
  dim3 grid(g.coarse_blocks, g.heads, g.batch);
  hipLaunchKernelGGL(vsa_scores_kernel, grid, dim3(256), 0, st, g, qbar, kbar, bias, scores, statp);
}

void vsa_launch_coarse_out(const VsaGeom& g, const float* scores, const float* vbar, float* ocoarse,
                           hipStream_t st) {
  if (g.Qs == 0) return;
  dim3 grid((g.Qs + OROWS - 1) / OROWS, g.heads, g.batch);
  hipLaunchKernelGGL(vsa_coarse_out_kernel, grid, dim3(256), 0, st, g, scores, vbar, ocoarse);
}

void vsa_launch_tau(const VsaGeom& g, const double* statp, float* thr, hipStream_t st) {
  if (g.Qs == 0) return;
  hipLaunchKernelGGL(vsa_tau_kernel, dim3(g.heads, g.batch), dim3(64), 0, st, g, statp, thr);
}
