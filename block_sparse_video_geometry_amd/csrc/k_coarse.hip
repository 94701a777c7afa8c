// Coarse branch: pooled logits, row softmax, O_coarse, and the tau statistics.
//
// "ComfyUI Agrega Nodo Central de Atencion Dispersa...", section "un nodo,
// tres backends": VSA scores cubic tiles through a coarse compression branch;
// Sol-Attn thresholds each head at a number of standard deviations of its
// score distribution.  "Spark-H3...", "Que cambia Spark-Attn": the compressed
// branch attends over mean-pooled summaries.
//
// S_ij = s qbar_i . kbar_j + b_j for every sparse query tile i and every
// candidate key tile j (the video tiles; every tile when sink_conditioning is
// off, "BSAI FastH3 Native VSA (recipe)", "The inputs that matter");
// P = softmax_j(S); O_c,i = sum_j P_ij vbar_j.  All fp32
// (the ranking must hold the oracle's order wherever its logit gap > 1e-4;
// bf16 inputs to this dot product would not), on the fp32 MFMAs: two dense
// contractions per head, ~4.6 GFLOP at 32 heads x 564 tiles, fused in one
// kernel so the logits are written once and never read back here.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

constexpr int CROWS = VSA_COARSE_ROWS;  // 64 sparse rows per workgroup, 16 per wave
constexpr int CCH = 64;                 // candidate tiles per LDS chunk
constexpr int LW = VSA_HEAD_DIM + 4;    // padded LDS row (floats)
constexpr float LOG2E_F = 1.4426950408889634f;

// One workgroup per (64 sparse rows, slice of the candidate tiles, head, batch); wave w owns
// rows 16 w .. 16 w + 15.  With four or more 64-tile chunks the candidates are cut into
// slices of whole chunks (so 288 row blocks at 32 heads do not leave two workgroups on a few
// CUs and one on the rest); each slice writes its running max, sum and unnormalised O, and
// vsa_coarse_merge_kernel combines them.  Per chunk of 64 candidate tiles (K-bar, V-bar and the bias staged in LDS, the next chunk's
// loads in flight meanwhile):
//   S^T = K-bar Q-bar^T on fp32 MFMAs (v_mfma_f32_16x16x4_f32).  MFMA step t of a
//     16-tile block contracts dims k(t, g) = 16 (t >> 2) + 4 g + (t & 3) for lane group g,
//     so both operands are 16-byte reads (Q-bar stays in registers).  Lane (g, r) ends
//     with S[row r][tiles 16 cb + 4 g .. +3] of block cb.
//   S = scale S + b goes out to the scores (and the tau sums), then an online softmax in
//     fp32 (exp2 of log2-scaled logits, the running max and sum per row).
//   O^T += V-bar^T P^T on fp32 MFMAs: P^T is exactly the S^T layout, and the output dims
//     are ordered d(db, r) = 64 (db >> 2) + 4 r + (db & 3) so V-bar is read 16 bytes at a
//     time.  A lane's O values all belong to its own row, so the rescale and the final
//     1 / l stay in the lane.
__global__ __launch_bounds__(256) void vsa_coarse_kernel(VsaGeom g, const float* __restrict__ qbar,
                                                         const float* __restrict__ kbar,
                                                         const float* __restrict__ vbar,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ scores,
                                                         float* __restrict__ ocoarse,
                                                         double* __restrict__ statp,
                                                         float* __restrict__ cpart) {
  __shared__ __attribute__((aligned(16))) float ks[CCH][LW];
  __shared__ __attribute__((aligned(16))) float vs[CCH][LW];
  __shared__ float bs[CCH];
  __shared__ double red[4][2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lg = lane >> 4, lr = lane & 15;
  // XCD-aware: each XCD takes a contiguous range of (batch x head, block) items, head-major,
  // so a head's K-bar and V-bar are read through few L2s
  const int G = gridDim.x, L = blockIdx.x, xcd = L & 7;
  const int w = xcd * (G >> 3) + min(xcd, G & 7) + (L >> 3);
  const int blk = w % g.coarse_blocks;
  const size_t bh = (size_t)(w / g.coarse_blocks);
  const int rb = blk / g.csplit, slice = blk % g.csplit;
  const int c_begin = slice * g.cchunks * CCH;                  // this slice's candidate tiles:
  const int c_end = min(g.Kc, c_begin + g.cchunks * CCH);       // [c_begin, c_end)
  const int row = rb * CROWS + 16 * wave + lr;  // the sparse row of this lane's values
  const bool live = row < g.Qs;

  // Q-bar operand: qf[m] = Q-bar[row][16 m + 4 lg .. +3] (zeros past the last row)
  f32x4 qf[8];
  {
    const f32x4* qp = reinterpret_cast<const f32x4*>(qbar + (bh * g.Tq + g.n_dense + (live ? row : 0)) * VSA_HEAD_DIM);
#pragma unroll
    for (int m = 0; m < 8; ++m) qf[m] = live ? qp[4 * m + lg] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float* kb = kbar + bh * g.Kc * VSA_HEAD_DIM;
  const float* vb = vbar + bh * g.Kc * VSA_HEAD_DIM;
  const float* bb = bias + bh * g.Kc;

  // chunk staging: thread tid moves rows (tid >> 5) + 8 r, 16-byte column tid & 31
  f32x4 kr[8], vr[8];
  float br = 0.f;
  auto fetch = [&](int j0) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int j = j0 + (tid >> 5) + 8 * r;
      kr[r] = vr[r] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (j < c_end) {
        kr[r] = reinterpret_cast<const f32x4*>(kb + (size_t)j * VSA_HEAD_DIM)[tid & 31];
        vr[r] = reinterpret_cast<const f32x4*>(vb + (size_t)j * VSA_HEAD_DIM)[tid & 31];
      }
    }
    br = (tid < CCH && j0 + tid < c_end) ? bb[j0 + tid] : 0.f;
  };
  auto stash = [&]() {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      *reinterpret_cast<f32x4*>(&ks[(tid >> 5) + 8 * r][4 * (tid & 31)]) = kr[r];
      *reinterpret_cast<f32x4*>(&vs[(tid >> 5) + 8 * r][4 * (tid & 31)]) = vr[r];
    }
    if (tid < CCH) bs[tid] = br;
  };

  float mrow = -INFINITY, lrow = 0.f;  // running max (log2 units) and this lane's share of the sum
  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  double ssum = 0.0, ssq = 0.0;
  const bool tau_sums = g.select == VSA_SELECT_TAU;  // the fp64 sums only feed the tau threshold
  const bool vec_out = (g.Kc & 3) == 0;  // 16-byte score stores stay aligned

  fetch(c_begin);
  for (int j0 = c_begin; j0 < c_end; j0 += CCH) {
    __syncthreads();  // the previous chunk's LDS reads are done
    stash();
    __syncthreads();
    if (j0 + CCH < c_end) fetch(j0 + CCH);

    f32x4 st[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const f32x4 kv = *reinterpret_cast<const f32x4*>(&ks[16 * cb + lr][16 * m + 4 * lg]);
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[e], qf[m][e], acc, 0, 0, 0);
      }
      st[cb] = acc;
    }

    // logits out (and the tau sums), then the chunk's softmax step
    float cm = -INFINITY;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int jl = 16 * cb + 4 * lg;
      f32x4 sv;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sv[i] = st[cb][i] * g.scale + bs[jl + i];
        const bool valid = j0 + jl + i < c_end;
        if (tau_sums && live && valid) {
          ssum += (double)sv[i];
          ssq += (double)sv[i] * (double)sv[i];
        }
        st[cb][i] = valid ? sv[i] * LOG2E_F : -INFINITY;
        cm = fmaxf(cm, st[cb][i]);
      }
      if (live) {
        float* dst = scores + (bh * g.Qs + row) * g.Kc + j0 + jl;
        if (vec_out && j0 + jl + 3 < c_end) {
          *reinterpret_cast<f32x4*>(dst) = sv;
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (j0 + jl + i < c_end) dst[i] = sv[i];
        }
      }
    }
    const float mn = fmaxf(mrow, group_max(cm));
    const float alpha = __builtin_amdgcn_exp2f(mrow - mn);  // 0 on the first chunk
    mrow = mn;
    lrow *= alpha;
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        st[cb][i] = __builtin_amdgcn_exp2f(st[cb][i] - mn);
        lrow += st[cb][i];
      }

    // O^T += V-bar^T P^T: step (cb, t) covers tiles 16 cb + 4 lg + t
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const f32x4 vv = *reinterpret_cast<const f32x4*>(&vs[16 * cb + 4 * lg + t][64 * hh + 4 * lr]);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            oacc[4 * hh + q] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv[q], st[cb][t], oacc[4 * hh + q], 0, 0, 0);
        }
  }

  // O_c = O / l: oacc[4 hh + q][i] = O[row][64 hh + 16 lg + 4 i + q]; with several slices
  // the slice's max, sum and unnormalised O go to the merge instead
  const float lt = group_sum(lrow);
  if (live && g.csplit > 1) {
    float* prow = cpart + ((bh * g.Qs + row) * g.csplit + slice) * (VSA_HEAD_DIM + 4);
    if (lg == 0) *reinterpret_cast<f32x4*>(prow) = f32x4{mrow, lt, 0.f, 0.f};
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(prow + 4 + 64 * hh + 16 * lg + 4 * i) =
            f32x4{oacc[4 * hh][i], oacc[4 * hh + 1][i], oacc[4 * hh + 2][i], oacc[4 * hh + 3][i]};
  }
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (live && g.csplit == 1) {
    float* orow = ocoarse + (bh * g.Qs + row) * VSA_HEAD_DIM;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4*>(orow + 64 * hh + 16 * lg + 4 * i) =
            f32x4{oacc[4 * hh][i], oacc[4 * hh + 1][i], oacc[4 * hh + 2][i], oacc[4 * hh + 3][i]} * inv;
  }

  if (g.select != VSA_SELECT_TAU) return;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    ssum += __shfl_xor(ssum, m);
    ssq += __shfl_xor(ssq, m);
  }
  if (lane == 0) {
    red[wave][0] = ssum;
    red[wave][1] = ssq;
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

// O_c of a row from its slices: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, M the
// largest slice max (log2 units).  One workgroup per (row, head, batch), one thread per dim.
__global__ __launch_bounds__(VSA_HEAD_DIM) void vsa_coarse_merge_kernel(VsaGeom g, const float* __restrict__ cpart,
                                                                       float* __restrict__ ocoarse) {
  const size_t ro = ((size_t)blockIdx.z * g.heads + blockIdx.y) * g.Qs + blockIdx.x;
  const float* base = cpart + ro * g.csplit * (VSA_HEAD_DIM + 4);
  const int d = threadIdx.x;
  float mx = -INFINITY;
  for (int s = 0; s < g.csplit; ++s) mx = fmaxf(mx, base[s * (VSA_HEAD_DIM + 4)]);
  float num = 0.f, den = 0.f;
  for (int s = 0; s < g.csplit; ++s) {
    const float* ps = base + s * (VSA_HEAD_DIM + 4);
    const float w = ps[0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ps[0] - mx);
    num += w * ps[4 + d];
    den += w * ps[1];
  }
  ocoarse[ro * VSA_HEAD_DIM + d] = den > 0.f ? num / den : 0.f;
}

// thr = mu + tau * sigma (population) over all Qs * Kc logits of a (batch, head).
__global__ void vsa_tau_kernel(VsaGeom g, const double* __restrict__ statp, float* __restrict__ thr) {
  const size_t bh = (size_t)blockIdx.y * g.heads + blockIdx.x;
  if (threadIdx.x != 0) return;
  double a = 0.0, q = 0.0;
  for (int i = 0; i < g.coarse_blocks; ++i) {
    a += statp[(bh * g.coarse_blocks + i) * 2 + 0];
    q += statp[(bh * g.coarse_blocks + i) * 2 + 1];
  }
  const double n = (double)g.Qs * (double)g.Kc;
  const double mu = a / n;
  double var = q / n - mu * mu;
  if (var < 0.0) var = 0.0;
  thr[bh] = (float)(mu + (double)g.tau * sqrt(var));
}

}  // namespace

void vsa_launch_coarse(const VsaGeom& g, const float* qbar, const float* kbar, const float* vbar,
                       const float* bias, float* scores, float* ocoarse, double* statp, float* cpart,
                       hipStream_t st) {
  if (g.Qs == 0) return;
  dim3 grid(g.coarse_blocks * g.heads * g.batch);
  hipLaunchKernelGGL(vsa_coarse_kernel, grid, dim3(256), 0, st, g, qbar, kbar, vbar, bias, scores, ocoarse,
                     statp, cpart);
  if (g.csplit > 1)
    hipLaunchKernelGGL(vsa_coarse_merge_kernel, dim3(g.Qs, g.heads, g.batch), dim3(VSA_HEAD_DIM), 0, st, g,
                       cpart, ocoarse);
}

void vsa_launch_tau(const VsaGeom& g, const double* statp, float* thr, hipStream_t st) {
  if (g.Qs == 0) return;
  hipLaunchKernelGGL(vsa_tau_kernel, dim3(g.heads, g.batch), dim3(64), 0, st, g, statp, thr);
}
