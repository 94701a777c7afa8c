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
//   max grows by more than 2^16, so the O rescale is skipped on almost every tile
//   O^T (128 x 64) += V^T . P^T               64 x mfma_f32_16x16x32_bf16,
//                  V^T operands read with ds_read_b64_tr_b16
// S^T puts keys on MFMA rows: each lane holds one query per 16-query block,
// and the key order inside every 32-key step is permuted (kperm) so a lane's
// eight probabilities are eight consecutive keys -- exactly the P^T operand
// of the PV product, with no register shuffles.  At the end the four waves'
// (max, sum, O) partials are merged through LDS and each wave writes 16 query
// rows (gate combine, bf16 round-to-nearest-even, packed order).
//
// Per-tile scalar work is kept small: every LDS read address is a per-lane
// base fixed for the whole kernel plus an immediate offset, and the source
// location of the wave's tiles is computed 64 tiles at a time (one per lane)
// and read back with readlane.
//
// Rows are ordered head-major, dense rows first, and mapped XCD-aware: the
// hardware deals workgroup i to XCD i % 8, so XCD x receives a contiguous
// range of heads and its L2 sees one head's K/V at a time.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;
// Lazy rescale threshold (log2 units): P = exp2(S sl2 - m) is taken against a running max
// that may lag the true one by up to 2^16.  P, O and l stay far inside the fp32 / bf16
// exponent range, and with logits of std 3 a rescale is then practically never needed
// (at 2^8 about one tile in twelve paid for one).
constexpr float RESCALE_TH = 16.0f;
constexpr int NW = 4;                // waves per workgroup
constexpr int TILE_BYTES = 16384;    // one 64 x 128 bf16 tile
constexpr int LIST_LDS = VSA_MAX_LIST;  // a sparse row's list is staged whole in LDS

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) char lds_char;

// Direct buffer -> LDS copy of 16 bytes per lane: lane i of the wave writes LDS bytes
// [lds + 16 i, lds + 16 i + 16) with the 16 bytes at buffer offset soff + voff (zero when
// out of the resource's range).  Issued from asm so the compiler neither inserts its own
// (whole-queue) waits for the LDS write nor moves LDS reads across it; completion is
// tracked with vmcnt by the waits below.  No register results, so nothing is left pending
// in a VGPR.  M0 is used by nothing else in this kernel, so it is set here and not restored.
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned soff, unsigned lds) {
  asm volatile(
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, %2 offen lds"
      :
      : "v"(voff), "s"(rs), "s"(soff), "s"(lds)
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

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ unsigned lds_u32(lds_char* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(size_t)p);
}

// Value of an accumulator register moved to a VGPR by an explicit, non-speculated move.
__device__ __forceinline__ float acc_read(float x) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
  return r;
}

__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Tile layout in LDS.
//  K: key row r at r*256; its 16-byte chunk c at position c ^ kswz(r),
//     kswz(r) = (r & 3) | ((r >> 3) & 3) << 2.
//  V: key row r at r*256; chunk c at position c ^ vswz(r),
//     vswz(r) = (2 (r & 3) + 8 ((r >> 3) & 1)) & 15.
// QK reads K rows kperm(kb, ql) = 32(kb>>1) + 8(ql>>2) + 4(kb&1) + (ql&3), for which
// kswz = ql: the lane address is base_k[ks] + 256 * (32(kb>>1) + 4(kb&1)).
// PV reads V rows 32c + 8 grp + (ql>>2) + 4h, for which vswz = 2(ql>>2) + 8(grp&1):
// the lane address is base_v[db] + 256 * (32c + 4h).
// The DMA lane offsets below follow the same two swizzles.

__global__ __launch_bounds__(256) void vsa_fine_kernel(
    VsaGeom g, const char* __restrict__ kptr, const char* __restrict__ vptr,
    const u32x4* __restrict__ q, const unsigned short* __restrict__ gate,
    const float* __restrict__ ocoarse, const int* __restrict__ lists,
    const int* __restrict__ counts, unsigned short* __restrict__ o, int per_xcd) {
  // per wave: a K tile and a V tile; separate arrays so LDS reads of one are never
  // taken as aliasing DMA writes in flight to the other
  __shared__ __attribute__((aligned(16))) char klds_all[NW * TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char vlds_all[NW * TILE_BYTES];
  __shared__ float mbuf[NW][64];
  __shared__ float lbuf[NW][64];
  __shared__ __attribute__((aligned(16))) float sbuf[NW][64];
  __shared__ int lst_lds[LIST_LDS];
  __shared__ int seg_lds[3][VSA_MAX_PREFIX_SEGS + 1];  // prefix segment table (start, len, tile0)

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
  if (dense) {
    nlist = g.Tq;
  } else {
    nlist = min(counts[(size_t)bh * g.Qs + srow], g.cap);  // cap <= LIST_LDS (plan)
    const int* lst = lists + ((size_t)bh * g.Qs + srow) * g.cap;
    for (int i = tid; i < nlist; i += 256) lst_lds[i] = lst[i];
  }
  if (tid <= VSA_MAX_PREFIX_SEGS) {
    seg_lds[0][tid] = tid < VSA_MAX_PREFIX_SEGS ? g.pre_start[tid] : 0;
    seg_lds[1][tid] = tid < VSA_MAX_PREFIX_SEGS ? g.pre_len[tid] : 0;
    seg_lds[2][tid] = g.pre_tile0[tid];
  }
  __syncthreads();

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

  // DMA lane offsets: instruction n covers key rows 4n .. 4n+3; lane = 16 gi + pos writes
  // row 4n + gi, position pos, i.e. chunk pos ^ swizzle(4n + gi).  The swizzles depend on
  // n only through (n >> 1) & 3 (K) and (n >> 1) & 1 (V).
  const unsigned rowbytes = (unsigned)g.heads * VSA_HEAD_DIM * 2;
  const int gi = lane >> 4, pos = lane & 15;
  unsigned koff[4], voff[2];
#pragma unroll
  for (int m = 0; m < 4; ++m) koff[m] = gi * rowbytes + ((pos ^ (gi | (m << 2))) << 4);
#pragma unroll
  for (int m = 0; m < 2; ++m) voff[m] = gi * rowbytes + ((pos ^ ((2 * gi + 8 * m) & 15)) << 4);
  const unsigned plane = (unsigned)g.H * g.W * rowbytes;  // token stride dt -> bytes
  const unsigned line = (unsigned)g.W * rowbytes;         // token stride dh -> bytes
  const long long bh_off = ((long long)b * g.N * g.heads + h) * (VSA_HEAD_DIM * 2);
  // One buffer resource per tensor over this (b, h) plane.  Offsets past its last byte read
  // zero: the padding rows of a partial prefix tile at the end of the sequence, and the
  // loads for the tile after a wave's last one (offset >= 2^31, never in range).
  const int nrec = (int)((unsigned)(g.N - 1) * rowbytes + VSA_HEAD_DIM * 2);
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)(kptr + bh_off), 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)(vptr + bh_off), 0, nrec, 0x00020000);
  constexpr unsigned NO_TILE = 0x80000000u;

  lds_char* kbuf = (lds_char*)(klds_all + wave * TILE_BYTES);
  lds_char* vbuf = (lds_char*)(vlds_all + wave * TILE_BYTES);
  const unsigned kbuf_u = lds_u32(kbuf), vbuf_u = lds_u32(vbuf);

  // LDS read bases (see the layout note above)
  unsigned kbase[4], vbase[8];
  {
    const unsigned lrow = (unsigned)(8 * (ql >> 2) + (ql & 3)) * 256;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kbase[ks] = kbuf_u + lrow + (((4 * ks + grp) ^ ql) << 4);
    const unsigned vrow = (unsigned)(8 * grp + (ql >> 2)) * 256 + 8 * (ql & 1);
    const int vm = (ql >> 2) + 4 * (grp & 1);
#pragma unroll
    for (int db = 0; db < 8; ++db)
      vbase[db] = vbuf_u + vrow + ((2 * (db ^ vm) + ((ql & 3) >> 1)) << 4);
  }

  // Tile descriptors, 64 at a time: lane l describes this wave's tile 64 batch + l.
  // off = byte offset of the tile's first token row in the (b, h) plane;
  // flags = video | nvalid << 1.
  const int my_n = nlist > wave ? (nlist - wave + NW - 1) / NW : 0;
  unsigned d_off = 0, d_flags = 0;
  auto describe = [&](int batch) {
    const int j = batch * 64 + lane;
    int t = 0;
    if (j < my_n) t = dense ? wave + NW * j : lst_lds[wave + NW * j];
    int tok0, video, nvalid;
    if (t >= g.P) {
      const int jv = t - g.P;
      const int tw = jv % g.tw_n;
      const int rest = jv / g.tw_n;
      const int th = rest % g.th_n;
      const int tt = rest / g.th_n;
      tok0 = g.vstart + (4 * tt * g.H + 4 * th) * g.W + 4 * tw;
      video = 1;
      nvalid = VSA_TILE_TOKENS;
    } else {
      // per-lane segment lookup from LDS (indexing the argument struct per lane would
      // become vector loads, whose waits would drain the DMA queue)
      int sg = 0;
      for (int i = 1; i < g.n_pre_segs; ++i)
        if (t >= seg_lds[2][i]) sg = i;
      const int off = (t - seg_lds[2][sg]) * VSA_TILE_TOKENS;
      tok0 = seg_lds[0][sg] + off;
      const int rem = seg_lds[1][sg] - off;
      video = 0;
      nvalid = rem < VSA_TILE_TOKENS ? rem : VSA_TILE_TOKENS;
    }
    d_off = (unsigned)tok0 * rowbytes;
    d_flags = (unsigned)video | ((unsigned)nvalid << 1);
  };
  // Row group n (key rows 4n .. 4n+3) of a tile starts at off + (n >> 2) * stp + (n & 3) * stl:
  // a video tile steps dt and dh, a prefix tile 16 and 4 tokens.
  auto steps = [&](unsigned flags, unsigned& stp, unsigned& stl) {
    stp = (flags & 1) ? plane : 16 * rowbytes;
    stl = (flags & 1) ? line : 4 * rowbytes;
  };
  auto kdma = [&](int n, unsigned off, unsigned stp, unsigned stl) {
    bdma16(krs, koff[(n >> 1) & 3], off + (n >> 2) * stp + (n & 3) * stl, kbuf_u + 1024 * n);
  };
  auto vdma = [&](int n, unsigned off, unsigned stp, unsigned stl) {
    bdma16(vrs, voff[(n >> 1) & 1], off + (n >> 2) * stp + (n & 3) * stl, vbuf_u + 1024 * n);
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

  // Per tile t: V(t) is fetched while QK(t) runs (one row group per four MFMAs), K(t+1)
  // while the softmax of t runs.  At the top of an iteration only K(t) is outstanding.
  unsigned c_off = 0, c_flags = 0;  // current tile
  if (my_n > 0) {
    describe(0);
    c_off = __builtin_amdgcn_readlane(d_off, 0);
    c_flags = __builtin_amdgcn_readlane(d_flags, 0);
    unsigned stp, stl;
    steps(c_flags, stp, stl);
#pragma unroll
    for (int n = 0; n < 16; ++n) kdma(n, c_off, stp, stl);
  }
  for (int j = 0; j < my_n; ++j) {
    unsigned n_off = NO_TILE, n_flags = 0;
    if (j + 1 < my_n) {
      if (((j + 1) & 63) == 0) describe((j + 1) >> 6);
      n_off = __builtin_amdgcn_readlane(d_off, (j + 1) & 63);
      n_flags = __builtin_amdgcn_readlane(d_flags, (j + 1) & 63);
    }
    const int nvalid = (int)(c_flags >> 1);
    unsigned c_stp, c_stl, n_stp, n_stl;
    steps(c_flags, c_stp, c_stl);
    steps(n_flags, n_stp, n_stl);

    // ---- S^T = K Q^T (K(t) landed), with the V(t) loads spread over the MFMAs
    wait_vm<0>();
    f32x4 sacc[4][4];
    {
      // operands of key block kb+1 are read while the 16 MFMAs of block kb issue
      bf16x8 ka[2][4];
      auto kread = [&](int kb, bf16x8* dst) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          dst[ks] = as_bf16x8(*(const lds_u32x4*)(size_t)(kbase[ks] + 256 * (32 * (kb >> 1) + 4 * (kb & 1))));
      };
      kread(0, ka[0]);
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if (kb < 3) kread(kb + 1, ka[(kb + 1) & 1]);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
          for (int qb = 0; qb < 4; ++qb)
            sacc[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                ka[kb & 1][ks], qv[qb][ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : sacc[kb][qb], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
          vdma(4 * kb + ks, c_off, c_stp, c_stl);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
    // K buffer is free once its reads returned
    wait_lgkm0();
#pragma unroll
    for (int n = 0; n < 4; ++n) kdma(n, n_off, n_stp, n_stl);
    __builtin_amdgcn_sched_barrier(0);

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
      mloc[qb] = group_max(m) * sl2;
      grow |= mloc[qb] > mrun[qb] + RESCALE_TH;
    }
    if (j == 0) {
      // first tile: O and l are still zero, only the running max is set
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) mrun[qb] = mloc[qb];
    } else if (__ballot(grow)) {  // wave-uniform, rare: move the running max, rescale O and l
      float alpha[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const float mn = fmaxf(mrun[qb], mloc[qb]);
        alpha[qb] = __builtin_amdgcn_exp2f(mrun[qb] - mn);
        mrun[qb] = mn;
        lsum[qb] *= alpha[qb];
      }
      // O <- diag(alpha) O with exact fp32 MFMAs (one product and zero additions per
      // element), so O is never touched by VALU inside the loop and stays in the
      // accumulator registers.  For accumulator element i the B operand (4 x 16) is
      // O[4 g + i][d] at lane (g, d), and A_i (16 x 4) has alpha[r] at [r][g] where
      // r == 4 g + i: lane (grp, ql) holds A_i[ql][grp].
      float asel[4][4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
#pragma unroll
        for (int i = 0; i < 4; ++i) asel[qb][i] = ql == 4 * grp + i ? alpha[qb] : 0.f;
      // The B operands are read out of the accumulator file by explicit moves inside this
      // branch (the compiler would otherwise copy all 128 accumulators on every iteration);
      // the NOPs cover the MFMA-result-to-VALU-read latency for those moves.
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          float ob[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) ob[i] = acc_read(oacc[db][qb][i]);
          f32x4 acc = __builtin_amdgcn_mfma_f32_16x16x4f32(asel[qb][0], ob[0], f32x4{0.f, 0.f, 0.f, 0.f},
                                                           0, 0, 0);
#pragma unroll
          for (int i = 1; i < 4; ++i) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(asel[qb][i], ob[i], acc, 0, 0, 0);
          oacc[db][qb] = acc;
        }
    }
    // P = exp2(S sl2 - m) as bf16 PV operands, with the rest of K(t+1) in between
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
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int n = 0; n < 3; ++n) kdma(4 + 3 * qb + n, n_off, n_stp, n_stl);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- O += P V (V(t) landed; the 16 loads of K(t+1) may be in flight)
    wait_vm<16>();
    {
      // V operands of dim block db+1 (both 32-key steps) are read while the 8 MFMAs of
      // block db issue
      bf16x8 va[2][2];
      auto vread = [&](int db, bf16x8* dst) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const unsigned a0 = vbase[db] + 256 * (32 * c);
          const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)a0);
          const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)(a0 + 1024));
          const u32x2 w0 = __builtin_bit_cast(u32x2, r0);
          const u32x2 w1 = __builtin_bit_cast(u32x2, r1);
          dst[c] = as_bf16x8(u32x4{w0[0], w0[1], w1[0], w1[1]});
        }
      };
      vread(0, va[0]);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        if (db < 7) vread(db + 1, va[(db + 1) & 1]);
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int qb = 0; qb < 4; ++qb)
            oacc[db][qb] =
                __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb[qb][c], va[db & 1][c], oacc[db][qb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        if (db < 7) __builtin_amdgcn_sched_group_barrier(0x100, 4, 1);
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 1);
      }
    }
    // V buffer is free once its reads returned
    wait_lgkm0();
    c_off = n_off;
    c_flags = n_flags;
  }
  // the loads issued for the tile after the last one (out of range, writing zeros) must
  // land before the K buffer is reused below
  wait_vm<0>();

  // ---- merge the four waves' partials.  Softmax statistics are per lane for queries
  // 16 qb + ql; O is held as oacc[db][qb][i] = O[16 qb + 4 grp + i][16 db + ql].
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    lsum[qb] = group_sum(lsum[qb]);
  }
  __syncthreads();  // every wave is done with its K/V buffers
  if (grp == 0) {
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) mbuf[wave][16 * qb + ql] = mrun[qb];
  }
  __syncthreads();
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int qq = 16 * qb + ql;
    float mt = mbuf[0][qq];
#pragma unroll
    for (int w = 1; w < NW; ++w) mt = fmaxf(mt, mbuf[w][qq]);
    const float sc = mrun[qb] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrun[qb] - mt);
    if (grp == 0) {
      lbuf[wave][qq] = lsum[qb] * sc;
      sbuf[wave][qq] = sc;
    }
  }
  __syncthreads();
  // partial O^T of wave w: dims 0..63 in its K tile area, 64..127 in its V tile area, each
  // dim a 256-byte row of 64 fp32 queries; the 16-byte chunk of queries 4c..4c+3 sits at
  // chunk c ^ (dim & 15)
  auto part = [&](int w, int d) -> lds_u32x4* {
    return (lds_u32x4*)((d < 64 ? klds_all : vlds_all) + w * TILE_BYTES) + (d & 63) * 16;
  };
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const f32x4 sc4 = *(const f32x4*)&sbuf[wave][16 * qb + 4 * grp];
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const f32x4 v = oacc[db][qb] * sc4;
      part(wave, 16 * db + ql)[(4 * qb + grp) ^ ql] = __builtin_bit_cast(u32x4, v);
    }
  }
  __syncthreads();

  // ---- epilogue: wave w writes queries 16 w + 4 (lane / 16) .. +3, dims 8 (lane % 16) .. +7
  const int qg = lane >> 4, dg = lane & 15;
  const int q0 = 16 * wave + 4 * qg;
  float r[4][8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int d = 8 * dg + e;
    f32x4 s = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < NW; ++w) s += __builtin_bit_cast(f32x4, part(w, d)[(q0 >> 2) ^ (d & 15)]);
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i][e] = s[i];
  }
  f32x4 oc0 = f32x4{0.f, 0.f, 0.f, 0.f}, oc1 = oc0;
  const bool gated = !dense && gate != nullptr;
  if (gated) {
    const f32x4* cp = reinterpret_cast<const f32x4*>(ocoarse + ((size_t)bh * g.Qs + srow) * VSA_HEAD_DIM + 8 * dg);
    oc0 = cp[0];
    oc1 = cp[1];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int qq = q0 + i;
    const int qtok = tile_token(g, qt, qq);
    if (qtok < 0) continue;
    float ltot = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) ltot += lbuf[w][qq];
    const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;  // an empty list gives O_fine = 0
    float y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = r[i][e] * inv;
    const long long orow = row_offset(g, b, qtok, h) + 8 * dg;
    if (gated) {
      const u32x4 gv = *reinterpret_cast<const u32x4*>(gate + orow);
      y[0] += bf16lo(gv[0]) * oc0[0];
      y[1] += bf16hi(gv[0]) * oc0[1];
      y[2] += bf16lo(gv[1]) * oc0[2];
      y[3] += bf16hi(gv[1]) * oc0[3];
      y[4] += bf16lo(gv[2]) * oc1[0];
      y[5] += bf16hi(gv[2]) * oc1[1];
      y[6] += bf16lo(gv[3]) * oc1[2];
      y[7] += bf16hi(gv[3]) * oc1[3];
    }
    *reinterpret_cast<u32x4*>(o + orow) = u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]),
                                                pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
  }
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
