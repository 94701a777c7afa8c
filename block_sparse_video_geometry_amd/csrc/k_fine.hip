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
// Work item: one (batch, head, query tile) per 256-thread workgroup.  The four
// waves split the row's key-tile list (wave w takes entries w, w+4, ...) and
// each runs all 64 queries against its tiles, so every K/V byte is read from
// LDS once.  Per wave and tile:
//   K, V tiles  -> LDS by direct global->LDS DMA (global_load_lds_dwordx4),
//                  16 KB each, XOR-swizzled 16-byte chunks; the next tile's K
//                  is fetched while this tile's softmax and PV run, its V while
//                  the next QK runs.  Waits are per wave (vmcnt), no barriers.
//   S^T (64 keys x 64 queries) = K . Q^T     64 x mfma_f32_16x16x32_bf16
//   online softmax in fp32 with exp2; the running max moves only when a row's
//   max grows by more than 2^8, so the O rescale is skipped on most tiles
//   O^T (128 x 64) += V^T . P^T               64 x mfma_f32_16x16x32_bf16,
//                  V^T operands read with ds_read_b64_tr_b16
// S^T puts keys on MFMA rows: each lane holds one query per 16-query block,
// and the key order inside every 32-key step is permuted (kperm) so a lane's
// eight probabilities are eight consecutive keys -- exactly the P^T operand
// of the PV product, with no register shuffles.  At the end the four waves'
// (max, sum, O) partials are merged through LDS and each wave writes 16 query
// rows (gate combine, bf16 round-to-nearest-even, packed order).
//
// Rows are ordered head-major, dense rows first, and mapped XCD-aware: the
// hardware deals workgroup i to XCD i % 8, so XCD x receives a contiguous
// range of heads and its L2 sees one head's K/V at a time.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;
constexpr float RESCALE_TH = 8.0f;   // lazy rescale threshold (log2 units)
constexpr int NW = 4;                // waves per workgroup
constexpr int TILE_BYTES = 16384;    // one 64 x 128 bf16 tile
constexpr int LIST_LDS = VSA_MAX_LIST;  // a sparse row's list is staged whole in LDS

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) char lds_char;

// Direct global -> LDS copy of 16 bytes per lane: lane i of the wave writes LDS bytes
// [lds + 16 i, lds + 16 i + 16) with the 16 bytes at base + voff.  Issued from asm so the
// compiler neither inserts its own (whole-queue) waits for the LDS write nor moves LDS
// reads across it; completion is tracked with vmcnt by the waits below.  No register
// results, so nothing is left pending in a VGPR.
__device__ __forceinline__ void dma16(const char* base, unsigned voff, unsigned lds) {
  unsigned saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(base), "s"(lds)
      : "memory");
}
// Wait until at most N vector-memory operations of this wave are outstanding; also a
// compiler memory barrier, so LDS reads stay after it.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
// Wait for this wave's LDS reads; a compiler memory barrier before the next DMA.
__device__ __forceinline__ void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" : : : "memory"); }

// key held by row r of 16-row MFMA block kb in the S^T product
__device__ __forceinline__ int kperm(int kb, int r) {
  return 32 * (kb >> 1) + 8 * (r >> 2) + 4 * (kb & 1) + (r & 3);
}
// K tile: 16-byte chunk c of key row `row` lives at chunk c ^ kswz(row)
__device__ __forceinline__ int kswz(int row) { return (row & 3) | (((row >> 3) & 3) << 2); }
// V tile: 16-byte chunk c of key row `row` lives at chunk c ^ vswz(row)
__device__ __forceinline__ int vswz(int row) { return (2 * (row & 3) + 8 * ((row >> 3) & 1)) & 15; }

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// LDS byte address of an LDS pointer (wave-uniform here)
__device__ __forceinline__ unsigned lds_u32(lds_char* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(size_t)p);
}

__device__ __forceinline__ unsigned int pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;
  return (unsigned int)__builtin_bit_cast(unsigned short, a) |
         ((unsigned int)__builtin_bit_cast(unsigned short, b) << 16);
}

// Uniform description of where a key tile's 64 rows live.
struct TileSrc {
  long long base;   // byte offset of the tile's first token row (head h)
  int video;        // 4x4x4 video tile (else prefix run of consecutive tokens)
  int nvalid;       // valid rows
};

__device__ __forceinline__ TileSrc tile_src(const VsaGeom& g, int b, int h, int t) {
  TileSrc s;
  int tok0;
  if (t >= g.P) {
    const int j = t - g.P;
    const int tw = j % g.tw_n;
    const int rest = j / g.tw_n;
    const int th = rest % g.th_n;
    const int tt = rest / g.th_n;
    tok0 = g.vstart + (4 * tt * g.H + 4 * th) * g.W + 4 * tw;
    s.video = 1;
    s.nvalid = VSA_TILE_TOKENS;
  } else {
    const int sg = prefix_seg(g, t);
    const int off = (t - g.pre_tile0[sg]) * VSA_TILE_TOKENS;
    tok0 = g.pre_start[sg] + off;
    const int rem = g.pre_len[sg] - off;
    s.video = 0;
    s.nvalid = rem < VSA_TILE_TOKENS ? rem : VSA_TILE_TOKENS;
  }
  s.base = row_offset(g, b, tok0, h) * 2;
  return s;
}

__global__ __launch_bounds__(256) void vsa_fine_kernel(
    VsaGeom g, const char* __restrict__ kptr, const char* __restrict__ vptr,
    const u32x4* __restrict__ q, const unsigned short* __restrict__ gate,
    const float* __restrict__ ocoarse, const int* __restrict__ lists,
    const int* __restrict__ counts, unsigned short* __restrict__ o, int per_xcd) {
  // per wave: K tile then V tile; separate arrays so LDS reads of one are never
  // taken as aliasing DMA writes in flight to the other
  __shared__ __attribute__((aligned(16))) char klds_all[NW * TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char vlds_all[NW * TILE_BYTES];
  __shared__ float mbuf[NW][64];
  __shared__ float lbuf[NW][64];
  __shared__ int lst_lds[LIST_LDS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
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
    nlist = min(counts[(size_t)bh * g.Qs + srow], g.cap);  // cap <= LIST_LDS (plan)
    lst = lists + ((size_t)bh * g.Qs + srow) * g.cap;
  }

  // stage the list in LDS: the loop then reads tile ids without touching the memory counters
  if (!dense)
    for (int i = tid; i < nlist; i += 256) lst_lds[i] = lst[i];  // nlist <= cap <= LIST_LDS (plan)
  __syncthreads();
  auto tile_at = [&](int i) -> int { return dense ? i : lst_lds[i]; };

  const int grp = lane >> 4, ql = lane & 15;
  // Q^T operands: lane holds queries 16 qb + ql, dims 32 ks + 8 grp .. +7
  bf16x8 qv[4][4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int tok = tile_token(g, qt, 16 * qb + ql);
    if (tok >= 0) {
      const u32x4* qp = q + row_offset(g, b, tok, h) / 8;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qv[qb][ks] = as_bf16x8(qp[4 * ks + grp]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qv[qb][ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }

  // Q must be in registers before the first DMA: a wait the compiler sees, so it does not
  // re-wait (whole queue) for these loads inside the loop
  __builtin_amdgcn_s_waitcnt(0);

  // per-lane DMA offsets.  Rows 4n + gi of instruction n (gi = lane / 16),
  // 16-byte position lane % 16 holds chunk (lane % 16) ^ swizzle(row).
  const int rowbytes = g.heads * VSA_HEAD_DIM * 2;
  const int gi = lane >> 4, pos = lane & 15;
  unsigned koff[4], voff[2];
#pragma unroll
  for (int m = 0; m < 4; ++m) koff[m] = gi * rowbytes + ((pos ^ (gi | (m << 2))) << 4);
#pragma unroll
  for (int m = 0; m < 2; ++m) voff[m] = gi * rowbytes + ((pos ^ ((2 * gi + 8 * m) & 15)) << 4);
  const long long plane = (long long)g.H * g.W * rowbytes;  // token stride dt -> bytes
  const long long line = (long long)g.W * rowbytes;         // token stride dh -> bytes

  lds_char* kbuf = (lds_char*)(klds_all + wave * TILE_BYTES);
  lds_char* vbuf = (lds_char*)(vlds_all + wave * TILE_BYTES);

  auto issue = [&](const char* __restrict__ X, const TileSrc& s, lds_char* dst, bool is_k) {
    if (s.nvalid == VSA_TILE_TOKENS) {
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        // rows 4n..4n+3: video (dt, dh) = (n >> 2, n & 3); prefix tokens 4n..4n+3
        const long long sb = s.video ? s.base + (n >> 2) * plane + (n & 3) * line
                                     : s.base + (long long)(4 * n) * rowbytes;
        const unsigned off = is_k ? koff[(n >> 1) & 3] : voff[(n >> 1) & 1];
        dma16(X + sb, off, lds_u32(dst) + 1024 * n);  // uniform SGPR base + 32-bit lane offset
      }
    } else {
      // partial prefix tile: padding rows re-read the last valid row (masked later)
      const char* base = X + s.base;
#pragma unroll
      for (int n = 0; n < 16; ++n) {
        const int row = min(4 * n + gi, s.nvalid - 1);
        const unsigned off = (is_k ? koff[(n >> 1) & 3] : voff[(n >> 1) & 1]) +
                             (unsigned)((row - gi) * rowbytes);
        dma16(base, off, lds_u32(dst) + 1024 * n);
      }
    }
  };

  f32x4 oacc[8][4];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun[4], lsum[4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    mrun[qb] = -INFINITY;
    lsum[qb] = 0.f;
  }
  const float sl2 = g.scale * LOG2E;

  const int my_n = nlist > wave ? (nlist - wave + NW - 1) / NW : 0;
  int t_cur = 0;
  TileSrc src{};
  if (my_n > 0) {
    t_cur = tile_at(wave);
    src = tile_src(g, b, h, t_cur);
    issue(kptr, src, kbuf, true);
    issue(vptr, src, vbuf, false);
  }
  for (int j = 0; j < my_n; ++j) {
    const bool has_next = j + 1 < my_n;
    int t_next = 0;
    if (has_next) t_next = tile_at(wave + NW * (j + 1));
    const int nvalid = src.nvalid;

    // ---- S^T = K Q^T (K(t) landed; V(t) may still be in flight)
    wait_vm<16>();
    f32x4 sacc[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) sacc[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = kperm(kb, ql);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 a =
            as_bf16x8(((lds_u32x4*)kbuf)[key * 16 + ((4 * ks + grp) ^ kswz(key))]);
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qv[qb][ks], sacc[kb][qb], 0, 0, 0);
      }
    }
    // K buffer is free once its reads returned: fetch the next tile's K
    wait_lgkm0();
    TileSrc nsrc{};
    if (has_next) {
      nsrc = tile_src(g, b, h, t_next);
      issue(kptr, nsrc, kbuf, true);
    }

    // ---- online softmax; lane holds keys 32(kb>>1) + 8 grp + 4(kb&1) + i of queries 16 qb + ql
    if (nvalid < VSA_TILE_TOKENS) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 32 * (kb >> 1) + 8 * grp + 4 * (kb & 1) + i;
          if (key >= nvalid)
#pragma unroll
            for (int qb = 0; qb < 4; ++qb) sacc[kb][qb][i] = -INFINITY;
        }
    }
    float mloc[4];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      float m = sacc[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, sacc[kb][qb][i]);
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      mloc[qb] = m * sl2;
      grow |= mloc[qb] > mrun[qb] + RESCALE_TH;
    }
    if (__ballot(grow)) {  // wave-uniform: move the running max, rescale O and l
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const float mn = fmaxf(mrun[qb], mloc[qb]);
        const float alpha = __builtin_amdgcn_exp2f(mrun[qb] - mn);
        mrun[qb] = mn;
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 8; ++db) oacc[db][qb] *= alpha;
      }
    }
    bf16x8 pb[4][2];
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      float p[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[kb][i] = __builtin_amdgcn_exp2f(fmaf(sacc[kb][qb][i], sl2, -mrun[qb]));
          lsum[qb] += p[kb][i];
        }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u32x4 w;
        w[0] = pack_bf16x2(p[2 * c][0], p[2 * c][1]);
        w[1] = pack_bf16x2(p[2 * c][2], p[2 * c][3]);
        w[2] = pack_bf16x2(p[2 * c + 1][0], p[2 * c + 1][1]);
        w[3] = pack_bf16x2(p[2 * c + 1][2], p[2 * c + 1][3]);
        pb[qb][c] = as_bf16x8(w);
      }
    }

    // ---- O^T += V^T P^T (V(t) landed; K(t_next) may be in flight)
    if (has_next)
      wait_vm<16>();
    else
      wait_vm<0>();
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        // lanes of group grp read rows 32c + 8 grp + (ql >> 2) (+4), dims 16 db + 4 (ql & 3)
        const int row0 = 32 * c + 8 * grp + (ql >> 2);
        const int chunk = 2 * db + ((ql & 3) >> 1);
        const int half = (ql & 1) * 8;
        const int a0 = row0 * 256 + ((chunk ^ vswz(row0)) << 4) + half;
        const int a1 = (row0 + 4) * 256 + ((chunk ^ vswz(row0 + 4)) << 4) + half;
        const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbuf + a0));
        const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vbuf + a1));
        const u32x2 w0 = __builtin_bit_cast(u32x2, r0);
        const u32x2 w1 = __builtin_bit_cast(u32x2, r1);
        const bf16x8 a = as_bf16x8(u32x4{w0[0], w0[1], w1[0], w1[1]});
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[qb][c], oacc[db][qb], 0, 0, 0);
      }
    }
    wait_lgkm0();
    if (has_next) issue(vptr, nsrc, vbuf, false);
    src = nsrc;
    t_cur = t_next;
  }
  (void)t_cur;

  // ---- merge the four waves' partials
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    lsum[qb] += __shfl_xor(lsum[qb], 16);
    lsum[qb] += __shfl_xor(lsum[qb], 32);
  }
  __syncthreads();  // every wave is done with its K/V buffers
  if (grp == 0) {
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) mbuf[wave][16 * qb + ql] = mrun[qb];
  }
  __syncthreads();
  // partial O of this wave: queries 0..31 in its K tile area, 32..63 in its V tile area,
  // each [32 q][32 chunks of 4 fp32]
  auto part = [&](int w, int qq) -> lds_u32x4* {
    return (lds_u32x4*)((qq < 32 ? klds_all : vlds_all) + w * TILE_BYTES) + (qq & 31) * 32;
  };
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int qq = 16 * qb + ql;
    float mt = mbuf[0][qq];
#pragma unroll
    for (int w = 1; w < NW; ++w) mt = fmaxf(mt, mbuf[w][qq]);
    const float sc = mrun[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun[qb] - mt);
    if (grp == 0) lbuf[wave][qq] = lsum[qb] * sc;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const f32x4 v = oacc[db][qb] * sc;
      part(wave, qq)[(4 * db + grp) ^ (qq & 31)] = __builtin_bit_cast(u32x4, v);
    }
  }
  __syncthreads();

  // ---- epilogue: wave w writes queries 16 w + lane/4, dims 32 (lane%4) .. +31
  const int qq = 16 * wave + (lane >> 2);
  const int qr = lane & 3;
  const int qtok = tile_token(g, qt, qq);
  if (qtok < 0) return;
  float ltot = 0.f;
#pragma unroll
  for (int w = 0; w < NW; ++w) ltot += lbuf[w][qq];
  const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;  // an empty list gives O_fine = 0
  float r[32];
#pragma unroll
  for (int cc = 0; cc < 8; ++cc) {
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w)
      s += __builtin_bit_cast(f32x4, part(w, qq)[(8 * qr + cc) ^ (qq & 31)]);
#pragma unroll
    for (int e = 0; e < 4; ++e) r[4 * cc + e] = s[e] * inv;
  }
  const long long orow = row_offset(g, b, qtok, h) + 32 * qr;
  if (!dense && gate != nullptr) {
    const u32x4* gp = reinterpret_cast<const u32x4*>(gate + orow);
    const f32x4* cp = reinterpret_cast<const f32x4*>(ocoarse + ((size_t)bh * g.Qs + srow) * VSA_HEAD_DIM + 32 * qr);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const u32x4 gv = gp[c4];
      const f32x4 o0 = cp[2 * c4], o1 = cp[2 * c4 + 1];
      r[8 * c4 + 0] += bf16lo(gv[0]) * o0[0];
      r[8 * c4 + 1] += bf16hi(gv[0]) * o0[1];
      r[8 * c4 + 2] += bf16lo(gv[1]) * o0[2];
      r[8 * c4 + 3] += bf16hi(gv[1]) * o0[3];
      r[8 * c4 + 4] += bf16lo(gv[2]) * o1[0];
      r[8 * c4 + 5] += bf16hi(gv[2]) * o1[1];
      r[8 * c4 + 6] += bf16lo(gv[3]) * o1[2];
      r[8 * c4 + 7] += bf16hi(gv[3]) * o1[3];
    }
  }
  u32x4* op = reinterpret_cast<u32x4*>(o + orow);
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4)
    op[c4] = u32x4{pack_bf16x2(r[8 * c4], r[8 * c4 + 1]), pack_bf16x2(r[8 * c4 + 2], r[8 * c4 + 3]),
                   pack_bf16x2(r[8 * c4 + 4], r[8 * c4 + 5]), pack_bf16x2(r[8 * c4 + 6], r[8 * c4 + 7])};
}

}  // namespace

void vsa_launch_fine(const VsaGeom& g, const void* q, const void* k, const void* v, const void* gate,
                     const float* ocoarse, const int* lists, const int* counts, void* o,
                     hipStream_t st) {
  const int total = g.batch * g.heads * g.Tq;
  const int per_xcd = (total + 7) / 8;
  hipLaunchKernelGGL(vsa_fine_kernel, dim3(8 * per_xcd), dim3(256), 0, st, g, (const char*)k,
                     (const char*)v, (const u32x4*)q, (const unsigned short*)gate, ocoarse, lists,
                     counts, (unsigned short*)o, per_xcd);
}
