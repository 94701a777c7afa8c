// Fine branch: block-sparse flash attention over each query tile's list, with
// the gated combine and the scatter back to packed order fused in.
//
// "ComfyUI Agrega Nodo Central de Atencion Dispersa...", first paragraph:
// each query block is routed to a chosen subset of key blocks.  "Spark-H3...",
// "Que cambia Spark-Attn": the exact branch computes the top-ranked key/value
// blocks in full.  "BSAI FastH3 Native VSA (recipe)", "The inputs that
// matter": exact_kv_and_rows runs conditioning query rows dense.  "Ref2VA VSA
// : noeud d'attention sparse pour le Ref2VA H3", item 3, and "ComfyUI-Ref2VA-
// VSA", "Technical Architecture": the learned gate (to_gate_compress) scales
// the compressed branch, O = O_fine + G * O_coarse.
//
// Work item: one (batch, head, query tile) per 256-thread workgroup; wave w
// owns query rows 16w..16w+15.  Per key tile on the list, all 256 threads
// stage K [64 keys x 128] and V^T [128 x 64 keys] in LDS (16 KB each, XOR
// swizzled so every ds_read_b128 / ds_write_b64 is bank-conflict free), then
// each wave runs
//   S^T (64 x 16) = K (64 x 128) . Q^T (128 x 16)   16 x mfma_f32_16x16x32_bf16
//   online softmax in fp32 (exp2, running max / sum)
//   O^T (128 x 16) += V^T (128 x 64) . P^T (64 x 16)  16 x mfma_f32_16x16x32_bf16
// Computing S^T (keys as MFMA rows) leaves every lane holding one query row:
// row statistics need only two cross-lane steps, the O rescale is a per-lane
// scalar, and P^T feeds the PV product straight from registers because the
// key order inside each 32-key step is permuted so that a lane's eight
// probabilities are eight consecutive keys (kperm below).
//
// Rows are ordered head-major, dense rows first, and mapped XCD-aware: the
// hardware deals workgroup i to XCD i % 8, so XCD x receives a contiguous
// range of heads and its L2 sees one head's K/V at a time.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;

// key held by row r of 16-row MFMA block kb in the S^T product
__device__ __forceinline__ int kperm(int kb, int r) {
  return 32 * (kb >> 1) + 8 * (r >> 2) + 4 * (kb & 1) + (r & 3);
}
// K tile: 16-byte chunk c of key row `key` lives at chunk c ^ kswz(key)
__device__ __forceinline__ int kswz(int key) { return (key & 3) | (((key >> 3) & 3) << 2); }
// V^T tile: 16-byte key chunk c of row d lives at chunk c ^ vswz(d)
__device__ __forceinline__ int vswz(int d) { return ((d >> 1) ^ (d >> 4)) & 7; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (unsigned int)__builtin_bit_cast(unsigned short, a) |
         ((unsigned int)__builtin_bit_cast(unsigned short, b) << 16);
}

__global__ __launch_bounds__(256) void vsa_fine_kernel(
    VsaGeom g, const u32x4* __restrict__ q, const u32x4* __restrict__ k,
    const u32x4* __restrict__ v, const unsigned short* __restrict__ gate,
    const float* __restrict__ ocoarse, const int* __restrict__ lists,
    const int* __restrict__ counts, unsigned short* __restrict__ o, int per_xcd) {
  __shared__ u32x4 klds[64 * 16];  // [key][chunk ^ kswz(key)]
  __shared__ u32x4 vlds[128 * 8];  // V^T: [d][keychunk ^ vswz(d)], 8 keys per chunk

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int item = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (item >= g.batch * g.heads * g.Tq) return;
  const int bh = item / g.Tq;
  const int qt = item - bh * g.Tq;
  const int b = bh / g.heads, h = bh - b * g.heads;
  const bool dense = qt < g.n_dense;
  const int srow = qt - g.n_dense;
  int nlist;
  const int* lst = nullptr;
  if (dense) {
    nlist = g.Tq;
  } else {
    nlist = counts[(size_t)bh * g.Qs + srow];
    lst = lists + ((size_t)bh * g.Qs + srow) * g.cap;
  }

  // Q^T operand: lane holds query row 16*wave + ql, dims 32 ks + 8 grp .. +7
  const int grp = lane >> 4, ql = lane & 15;
  const int qtok = tile_token(g, qt, wave * 16 + ql);
  bf16x8 qv[4];
  if (qtok >= 0) {
    const u32x4* qp = q + row_offset(g, b, qtok, h) / 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qv[ks] = as_bf16x8(qp[4 * ks + grp]);
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qv[ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
  }

  // loader: thread stages key rows 4 lq .. 4 lq + 3, 16-byte chunk lc (dims 8 lc .. 8 lc + 7)
  const int lq = tid >> 4, lc = tid & 15;
  u32x4 kr[4], vr[4];
  auto load_tile = [&](int t) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = tile_token(g, t, 4 * lq + i);
      if (tok >= 0) {
        const long long off = row_offset(g, b, tok, h) / 8 + lc;
        kr[i] = k[off];
        vr[i] = v[off];
      } else {
        kr[i] = u32x4{0u, 0u, 0u, 0u};
        vr[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  f32x4 oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) oacc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;
  const float sl2 = g.scale * LOG2E;

  int t_next = 0;
  if (nlist > 0) {
    t_next = dense ? 0 : lst[0];
    load_tile(t_next);
  }
  u32x2* vlds2 = reinterpret_cast<u32x2*>(vlds);
  for (int it = 0; it < nlist; ++it) {
    const int t = t_next;
    __syncthreads();  // the previous tile is no longer read
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = 4 * lq + i;
      klds[key * 16 + (lc ^ kswz(key))] = kr[i];
    }
    // transpose 4 keys x 8 dims -> 8 dims x 4 keys (bf16 pairs via byte permutes)
    u32x2 vt[8];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      vt[2 * w] = u32x2{__builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x05040100u),
                        __builtin_amdgcn_perm(vr[3][w], vr[2][w], 0x05040100u)};
      vt[2 * w + 1] = u32x2{__builtin_amdgcn_perm(vr[1][w], vr[0][w], 0x07060302u),
                            __builtin_amdgcn_perm(vr[3][w], vr[2][w], 0x07060302u)};
    }
    // odd lc lanes write their rows in the order s ^ 1 so each write spreads over all banks
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      const int dd = s ^ (lc & 1);
      const int d = 8 * lc + dd;
      const u32x2 val = (lc & 1) ? vt[s ^ 1] : vt[s];
      vlds2[d * 16 + (((lq >> 1) ^ vswz(d)) << 1) + (lq & 1)] = val;
    }
    __syncthreads();
    if (it + 1 < nlist) {
      t_next = dense ? it + 1 : lst[it + 1];
      load_tile(t_next);  // in flight during the math below
    }
    const int nvalid = tile_valid(g, t);

    // S^T = K Q^T
    f32x4 sacc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      sacc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int key = kperm(kb, ql);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a = as_bf16x8(klds[key * 16 + ((4 * ks + grp) ^ kswz(key))]);
        sacc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qv[ks], sacc[kb], 0, 0, 0);
      }
    }
    // online softmax; lane holds keys 32(kb>>1) + 8 grp + 4(kb&1) + i of query ql
    float z[4][4];
    float mloc = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = 32 * (kb >> 1) + 8 * grp + 4 * (kb & 1) + i;
        z[kb][i] = key < nvalid ? sacc[kb][i] * sl2 : -INFINITY;
        mloc = fmaxf(mloc, z[kb][i]);
      }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float mnew = fmaxf(mrun, mloc);
    const float alpha = __builtin_amdgcn_exp2f(mrun - mnew);
    mrun = mnew;
    float ls = 0.f;
    float p[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[kb][i] = __builtin_amdgcn_exp2f(z[kb][i] - mnew);
        ls += p[kb][i];
      }
    lrun = lrun * alpha + ls;
#pragma unroll
    for (int db = 0; db < 8; ++db) oacc[db] *= alpha;
    bf16x8 pb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 w;
      w[0] = pack_bf16x2(p[2 * c][0], p[2 * c][1]);
      w[1] = pack_bf16x2(p[2 * c][2], p[2 * c][3]);
      w[2] = pack_bf16x2(p[2 * c + 1][0], p[2 * c + 1][1]);
      w[3] = pack_bf16x2(p[2 * c + 1][2], p[2 * c + 1][3]);
      pb[c] = as_bf16x8(w);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = 16 * db + ql;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 a = as_bf16x8(vlds[d * 8 + ((4 * c + grp) ^ vswz(d))]);
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[c], oacc[db], 0, 0, 0);
      }
    }
  }

  // epilogue: normalise, add G * O_coarse on sparse rows, bf16 RNE, packed order
  float ltot = lrun + __shfl_xor(lrun, 16);
  ltot += __shfl_xor(ltot, 32);
  if (qtok < 0) return;
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;  // an empty list gives O_fine = 0
  const long long orow = row_offset(g, b, qtok, h);
  const bool combine = !dense && gate != nullptr;
  const float* ocp = combine ? ocoarse + ((size_t)bh * g.Qs + srow) * VSA_HEAD_DIM : nullptr;
#pragma unroll
  for (int db = 0; db < 8; ++db) {
    const int d0 = 16 * db + 4 * grp;
    float r[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = oacc[db][i] * inv;
    if (combine) {
      const u32x2 gv = *reinterpret_cast<const u32x2*>(gate + orow + d0);
      const f32x4 oc = *reinterpret_cast<const f32x4*>(ocp + d0);
      r[0] += bf16lo(gv[0]) * oc[0];
      r[1] += bf16hi(gv[0]) * oc[1];
      r[2] += bf16lo(gv[1]) * oc[2];
      r[3] += bf16hi(gv[1]) * oc[3];
    }
    *reinterpret_cast<u32x2*>(o + orow + d0) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
  }
}

}  // namespace

void vsa_launch_fine(const VsaGeom& g, const void* q, const void* k, const void* v, const void* gate,
                     const float* ocoarse, const int* lists, const int* counts, void* o,
                     hipStream_t st) {
  const int total = g.batch * g.heads * g.Tq;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL(vsa_fine_kernel, dim3(8 * per_xcd), dim3(256), 0, st, g, (const u32x4*)q,
                     (const u32x4*)k, (const u32x4*)v, (const unsigned short*)gate, ocoarse, lists,
                     counts, (unsigned short*)o, per_xcd);
}
