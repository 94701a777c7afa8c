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
// Work item: one (batch, head, query tile) per 64-thread workgroup: one wave
// runs all 64 queries against the row's whole key-tile list, so every K/V byte
// is read from LDS once and no partials are merged.  About 33 KB of LDS, so
// four workgroups (one per SIMD) share a CU.  Per tile:
//   K, V tiles  -> LDS by direct buffer->LDS DMA (buffer_load_dwordx4 ... lds),
//                  16 KB each, XOR-swizzled 16-byte chunks, refilled by 32-row
//                  halves as soon as a half has been read.  Waits are vmcnt
//                  counts, no barriers.
//   S^T (64 keys x 64 queries) = K . Q^T     64 x mfma_f32_16x16x32_bf16
//   online softmax in fp32 with exp2, software-pipelined: the softmax of tile j
//   runs on the VALU between the QK MFMAs of tile j+1.  The running max is
//   moved only when a tile's probabilities against it grow past 2^16, so the O
//   rescale is skipped on almost every tile.
//   O (64 x 128) += P . V                     64 x mfma_f32_16x16x32_bf16,
//                  V operands read with ds_read_b64_tr_b16
// S^T puts keys on MFMA rows: each lane holds one query per 16-query block,
// and the key order inside every 32-key step is permuted (kperm) so a lane's
// eight probabilities are eight consecutive keys -- exactly the P operand of
// the PV product, with no register shuffles.  At the end O^T goes through LDS
// and the wave writes the 64 query rows (gate combine, bf16 round-to-nearest-
// even, packed order).
//
// Per-tile scalar work is kept small: every K read address is a per-lane base
// fixed for the whole kernel plus an immediate offset (a V read address adds
// one XOR and shift to a fixed base), and the source
// location of the wave's tiles is computed 64 tiles at a time (one per lane)
// and read back with readlane.
//
// Rows are mapped XCD-aware: the hardware deals workgroup i to XCD i % 8, so XCD x
// receives a contiguous head-major range of rows and its L2 sees few heads' K/V at a time;
// within the range its dense rows run first, so that none of these long rows starts late.
//
// The dense call (every row dense, every row the same list of all tiles) runs the same
// pipeline four query tiles at a time: a workgroup of four waves, one per SIMD, of one
// (batch, head), moving through the tiles in step.  Each wave copies a quarter of every K
// and V half-tile into the buffers the four share, waits for its own copies and meets the
// others at a barrier before the half is read, and before it is refilled once all four
// have read it.  Per wave the arithmetic, and its order, is unchanged.
//
// Extra tokens ("ComfyUI Agrega Nodo Central de Atencion Dispersa...", schedule
// paragraph): a sparse row's extra key tokens, staged by the extra-token kernels
// as 64 consecutive rows (padding zero) with the token stride of K and V, run as
// the row's first tile.  Only the loads of that first tile (K and V rows 0-31 in
// the prologue, V rows 32-63 in the first iteration) use the staging buffers'
// resources; the rest of the pipeline is unchanged.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

constexpr float LOG2E = 1.4426950408889634f;
// Lazy rescale: P = exp2(S sl2 - m) is taken against a running max m that may lag the
// true one.  m is moved (O and l rescaled) only when, for some row, one lane's sum of the
// tile's probabilities passes 2^16: that sum bounds each of them, so P, O and l stay far
// inside the fp32 / bf16 range, and an overflow to inf is caught by the same test.  With
// logits of std 3 a rescale is then practically never needed.
constexpr float RESCALE_SUM = 65536.0f;
constexpr int TILE_BYTES = 16384;    // one 64 x 128 bf16 tile

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) char lds_char;

// Direct buffer -> LDS copy of 16 bytes per lane: lane i of the wave writes LDS bytes
// [M0 + IMM + 16 i, +16) with the 16 bytes at buffer offset soff + voff + IMM (zero when out
// of the resource's range): the immediate offset moves both addresses.  Four consecutive
// copies into consecutive 1 KB rows of a buffer therefore share one M0 value (the first of
// the four sets it, SET_M0) and differ by IMM = 0, 1024, 2048, 3072, the caller taking IMM
// off soff.  Issued from asm so the compiler neither inserts its own (whole-queue) waits
// for the LDS write nor moves LDS reads across it; completion is tracked with vmcnt by the
// waits below.  No register results, so nothing is left pending in a VGPR.  M0 is used by
// nothing else in this kernel, so it is set here and not restored.
template <int IMM, bool SET_M0>
__device__ __forceinline__ void bdma16(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned soff, unsigned lds) {
  if (SET_M0)
    asm volatile(
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %0, %1, %2 offen offset:%4 lds"
        :
        : "v"(voff), "s"(rs), "s"(soff), "s"(lds), "n"(IMM)
        : "memory");
  else
    asm volatile("buffer_load_dwordx4 %0, %1, %2 offen offset:%3 lds"
                 :
                 : "v"(voff), "s"(rs), "s"(soff), "n"(IMM)
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

// A wave-uniform pointer, held in SGPRs (the buffer resources feed scalar asm operands)
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const unsigned long long x = (unsigned long long)p;
  const unsigned lo = __builtin_amdgcn_readfirstlane((unsigned)x);
  const unsigned hi = __builtin_amdgcn_readfirstlane((unsigned)(x >> 32));
  return (const void*)(((unsigned long long)hi << 32) | lo);
}

constexpr bf16x2 ONES_BF16X2 = {(__bf16)1.0f, (__bf16)1.0f};

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

// XT: the plan has extra tokens (a sparse row may then run its extra tokens' tile first).
// SH: every row is dense (the dense call): a workgroup of four waves, one per SIMD, runs four
// query tiles of one (batch, head) in step over the same key tiles, each wave copying a
// quarter of every K and V tile into LDS buffers the four share.
template <bool XT, bool SH>
__global__ __launch_bounds__(SH ? 256 : 64) void vsa_fine_kernel(
    VsaGeom g, const char* __restrict__ kptr, const char* __restrict__ vptr,
    const u32x4* __restrict__ q, const unsigned short* __restrict__ gate,
    const float* __restrict__ ocoarse, const int* __restrict__ lists,
    const int* __restrict__ counts, unsigned short* __restrict__ o, int per_xcd,
    const int* __restrict__ xtok, const char* __restrict__ vxptr, const int* __restrict__ xcnt) {
  // a K tile and a V tile; separate arrays so LDS reads of one are never taken as aliasing
  // DMA writes in flight to the other.  About 33 KB in all, so four workgroups share a CU.
  __shared__ __attribute__((aligned(16))) char klds[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char vlds[TILE_BYTES];
  __shared__ float lbuf[SH ? 256 : 64];
  __shared__ int seg_lds[3][VSA_MAX_PREFIX_SEGS + 1];  // prefix segment table (start, len, tile0)
  extern __shared__ int lst_lds[];                     // a sparse row's list (cap entries)
  // (SH: no lists; the dynamic area holds the O^T staging of waves 1-3 instead, wave 0
  // staging in the K and V buffers)

  const int lane = SH ? (int)(threadIdx.x & 63) : (int)threadIdx.x;
  const int wv = SH ? __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) : 0;
  // XCD x takes the head-major item range [a, e); within it, its dense rows (the long ones)
  // first, then its sparse rows, each in head-major order.  D(p) and S(p): dense and sparse
  // items before head-major position p.
  int bh, qt;
  if (SH) {
    // XCD x takes the head-major range of groups of four query tiles [a, a + per_xcd)
    const int ng = (g.Tq + 3) >> 2;
    const int total = g.batch * g.heads * ng;
    const int a = (int)(blockIdx.x & 7) * per_xcd, k = (int)(blockIdx.x >> 3);
    if (a + k >= min(a + per_xcd, total)) return;  // the whole workgroup
    bh = (a + k) / ng;
    qt = 4 * (a + k - bh * ng) + wv;  // past the last tile: a wave that only keeps step
  } else {
    const int total = g.batch * g.heads * g.Tq;
    const int a = (int)(blockIdx.x & 7) * per_xcd, k = (int)(blockIdx.x >> 3);
    const int e = min(a + per_xcd, total);
    if (a + k >= e) return;
    const int nd = g.n_dense, ns = g.Tq - g.n_dense;
    auto D = [&](int p) { return (p / g.Tq) * nd + min(p % g.Tq, nd); };
    const int da = D(a), ndr = D(e) - da;
    if (k < ndr) {
      const int jd = da + k;
      bh = jd / nd;
      qt = jd - bh * nd;
    } else {
      const int js = (a / g.Tq) * ns + max(a % g.Tq - nd, 0) + (k - ndr);
      bh = js / ns;
      qt = nd + (js - bh * ns);
    }
  }
  const int b = bh / g.heads, h = bh - b * g.heads;
  const bool qvalid = !SH || qt < g.Tq;
  const bool dense = SH || qt < g.n_dense;
  const int srow = qt - g.n_dense;
  const int grp = lane >> 4, ql = lane & 15;
  // Q^T operands: lane holds queries 16 qb + ql, dims 32 ks + 8 grp .. +7.  Issued first,
  // so they land while the list is staged.
  bf16x8 qv[4][4];
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int tok = qvalid ? tile_token(g, qt, 16 * qb + ql) : -1;
    if (tok >= 0) {
      const u32x4* qp = q + row_offset(g, b, tok, h) / 8;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qv[qb][ks] = as_bf16x8(qp[4 * ks + grp]);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) qv[qb][ks] = as_bf16x8(u32x4{0u, 0u, 0u, 0u});
    }
  }

  const unsigned rowbytes = (unsigned)g.heads * VSA_HEAD_DIM * 2;
  const long long bh_off = ((long long)b * g.N * g.heads + h) * (VSA_HEAD_DIM * 2);
  // One buffer resource per tensor over this (b, h) plane.  Offsets past its last byte read
  // zero: the padding rows of a partial prefix tile at the end of the sequence, and the
  // loads for the tile after a wave's last one (offset >= 2^31, never in range).
  const int nrec = (int)((unsigned)(g.N - 1) * rowbytes + VSA_HEAD_DIM * 2);
  constexpr unsigned NO_TILE = 0x80000000u;

  int nlist;
  if (dense) {
    nlist = g.Tq;
  } else {
    // the list is staged to its capacity (entries past the count are never read), so its
    // loads need not wait for the count's
    const int cnt = counts[(size_t)bh * g.Qs + srow];
    const int* lst = lists + ((size_t)bh * g.Qs + srow) * g.cap;
    for (int i = lane; i < g.cap; i += 64) lst_lds[i] = lst[i];
    nlist = min(cnt, g.cap);
  }
  if (wv == 0 && lane <= VSA_MAX_PREFIX_SEGS) {
    seg_lds[0][lane] = lane < VSA_MAX_PREFIX_SEGS ? g.pre_start[lane] : 0;
    seg_lds[1][lane] = lane < VSA_MAX_PREFIX_SEGS ? g.pre_len[lane] : 0;
    seg_lds[2][lane] = g.pre_tile0[lane];
  }
  __syncthreads();

  // DMA lane offsets: instruction n covers key rows 4n .. 4n+3; lane = 16 gi + pos writes
  // row 4n + gi, position pos, i.e. chunk pos ^ swizzle(4n + gi).  The swizzles depend on
  // n only through (n >> 1) & 3 (K) and (n >> 1) & 1 (V).
  const int gi = lane >> 4, pos = lane & 15;
  unsigned koff[4], voff[2];
#pragma unroll
  for (int m = 0; m < 4; ++m) koff[m] = gi * rowbytes + ((pos ^ (gi | (m << 2))) << 4);
#pragma unroll
  for (int m = 0; m < 2; ++m) voff[m] = gi * rowbytes + ((pos ^ ((2 * gi + 8 * m) & 15)) << 4);
  // a sparse row's staged extra tokens (nx of them, none when the option is off) run first
  int nx = 0;
  if (XT && !dense) nx = __builtin_amdgcn_readfirstlane(xcnt[(size_t)bh * g.Qs + srow]);
  const int hx = nx > 0 ? 1 : 0;
  const unsigned plane = (unsigned)g.H * g.W * rowbytes;  // token stride dt -> bytes
  const unsigned line = (unsigned)g.W * rowbytes;         // token stride dh -> bytes
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(kptr + bh_off), 0, nrec, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)uniform_ptr(vptr + bh_off), 0, nrec, 0x00020000);
  // The extra tokens' tile (a row with extra tokens runs it first): its K rows and V rows
  // 0-31 are loaded in the prologue straight from K and V by token id; its V rows 32-63,
  // which the loop loads during the tile's first phase like any tile's, come from the
  // staging buffer [batch, Qs, 32, heads, 128].  Their resource starts 32 rows before the
  // row's staging block, so that row r of the tile sits at the tile offset + r row bytes.
  const long long bhx_off =
      ((long long)b * g.Qs * VSA_XSTAGE * g.heads + h) * (VSA_HEAD_DIM * 2) - (long long)VSA_XSTAGE * rowbytes;
  const int nrec_x = (int)((unsigned)(g.Qs * VSA_XSTAGE + VSA_XSTAGE - 1) * rowbytes + VSA_HEAD_DIM * 2);
  const __amdgpu_buffer_rsrc_t vrs0 = __builtin_amdgcn_make_buffer_rsrc(
      (void*)uniform_ptr(hx ? vxptr + bhx_off : vptr + bh_off), 0, hx ? nrec_x : nrec, 0x00020000);

  lds_char* kbuf = (lds_char*)klds;
  lds_char* vbuf = (lds_char*)vlds;
  const unsigned kbuf_u = lds_u32(kbuf), vbuf_u = lds_u32(vbuf);

  // LDS read bases (see the layout note above)
  unsigned kbase[4];
  {
    const unsigned lrow = (unsigned)(8 * (ql >> 2) + (ql & 3)) * 256;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kbase[ks] = kbuf_u + lrow + (((4 * ks + grp) ^ ql) << 4);
  }
  // V read address of dim block db: vbase0 + 32 (db ^ vm), computed per use (an XOR and
  // an add) to keep eight address registers free
  const unsigned vbase0 = vbuf_u + (unsigned)(8 * grp + (ql >> 2)) * 256 + 8 * (ql & 1) + (((ql & 3) >> 1) << 4);
  const unsigned vm = (unsigned)((ql >> 2) + 4 * (grp & 1));

  // Tile descriptors, 64 at a time: lane l describes tile 64 batch + l of the list.
  // off = byte offset of the tile's first token row in the (b, h) plane;
  // flags = video | nvalid << 1.
  const int my_n = nlist + hx;
  unsigned d_off = 0, d_flags = 0;
  auto describe = [&](int batch) {
    const int j = batch * 64 + lane;
    int t = 0;
    if (j < my_n && j >= hx) t = dense ? j : lst_lds[j - hx];
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
    if (j < hx) {  // the extra tokens' tile: nx valid rows; V rows 32-63 from the staging
      d_off = (unsigned)srow * VSA_XSTAGE * rowbytes;
      d_flags = (unsigned)nx << 1;
    }
  };
  // Row group n (key rows 4n .. 4n+3) of a tile starts at off + (n >> 2) * stp + (n & 3) * stl:
  // a video tile steps dt and dh, a prefix tile 16 and 4 tokens.
  auto steps = [&](unsigned flags, unsigned& stp, unsigned& stl) {
    stp = (flags & 1) ? plane : 16 * rowbytes;
    stl = (flags & 1) ? line : 4 * rowbytes;
  };
  // Copy n writes LDS rows 4n .. 4n + 3 (1 KB at buffer + 1024 n): M0 = buffer + 4096 (n >> 2)
  // is set by copy 4 (n >> 2) and the immediate 1024 (n & 3) reaches the row, so soff takes
  // that immediate off again.  (stl >= 4 row bytes >= 1 KB, so soff stays non-negative, and
  // an out-of-range tile offset stays out of range.)
  // (n is a constant once the loops around the calls are unrolled, so the switch folds away.)
  auto dma = [&](__amdgpu_buffer_rsrc_t rs, unsigned vo, int n, unsigned off, unsigned stp, unsigned stl,
                 unsigned buf) {
    const unsigned so = off + (unsigned)(n >> 2) * stp + (unsigned)(n & 3) * (stl - 1024u);
    const unsigned lds = buf + 4096u * (unsigned)(n >> 2);
    switch (n & 3) {
      case 0: bdma16<0, true>(rs, vo, so, lds); break;
      case 1: bdma16<1024, false>(rs, vo, so, lds); break;
      case 2: bdma16<2048, false>(rs, vo, so, lds); break;
      default: bdma16<3072, false>(rs, vo, so, lds); break;
    }
  };
  auto kdma_r = [&](__amdgpu_buffer_rsrc_t rs, int n, unsigned off, unsigned stp, unsigned stl) {
    dma(rs, koff[(n >> 1) & 3], n, off, stp, stl, kbuf_u);
  };
  auto vdma_r = [&](__amdgpu_buffer_rsrc_t rs, int n, unsigned off, unsigned stp, unsigned stl) {
    dma(rs, voff[(n >> 1) & 1], n, off, stp, stl, vbuf_u);
  };
  auto kdma = [&](int n, unsigned off, unsigned stp, unsigned stl) { kdma_r(krs, n, off, stp, stl); };
  auto vdma = [&](int n, unsigned off, unsigned stp, unsigned stl) { vdma_r(vrs, n, off, stp, stl); };
  // SH: this wave's quarter of a 32-row half (hf = 0: rows 0-31, 1: rows 32-63) of a shared
  // tile: copies n = 8 hf + 2 wv and n + 1, one M0 write for the pair.  M0 takes the LDS
  // address of copy n itself, so the pair's immediates are 0 and 1024 (copy n + 1's source
  // offset takes the 1024 off again).  Their lane offsets are those of koff / voff for this n.
  const unsigned kofw = gi * rowbytes + ((pos ^ (gi | ((wv & 3) << 2))) << 4);
  const unsigned vofw = gi * rowbytes + ((pos ^ ((2 * gi + 8 * (wv & 1)) & 15)) << 4);
  auto dma_q = [&](__amdgpu_buffer_rsrc_t rs, unsigned vo, int hf, unsigned off, unsigned stp, unsigned stl,
                   unsigned buf) {
    const unsigned n = 8u * (unsigned)hf + 2u * (unsigned)wv, r = n & 3u;
    const unsigned so = off + (n >> 2) * stp + r * stl;
    const unsigned lds = __builtin_amdgcn_readfirstlane(buf + 4096u * (n >> 2) + 1024u * r);
    bdma16<0, true>(rs, vo, so, lds);
    bdma16<1024, false>(rs, vo, so + stl - 1024u, lds);
  };
  auto kdma_q = [&](int hf, unsigned off, unsigned stp, unsigned stl) { dma_q(krs, kofw, hf, off, stp, stl, kbuf_u); };
  auto vdma_q = [&](int hf, unsigned off, unsigned stp, unsigned stl) { dma_q(vrs, vofw, hf, off, stp, stl, vbuf_u); };
  // SH: the four waves meet (no memory wait of its own: each wave waits for its own copies
  // and LDS reads just before)
  auto meet = [&]() {
    if (SH) __builtin_amdgcn_s_barrier();
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
  const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};

  // K operand of MFMA step s = (key block s >> 2, dims 32 (s & 3) ..): rows kperm, see the
  // layout note
  auto kread = [&](int s) -> bf16x8 {
    const int kb = s >> 2;
    return as_bf16x8(*(const lds_u32x4*)(size_t)(kbase[s & 3] + 256 * (32 * (kb >> 1) + 4 * (kb & 1))));
  };
  // V operand of PV step u = (32-key step c = u >> 3, dim block db = u & 7)
  auto vread = [&](int u) -> bf16x8 {
    const unsigned c = (unsigned)u >> 3, db = (unsigned)u & 7;
    const unsigned a0 = vbase0 + ((db ^ vm) << 5) + 256 * (32 * c);
    const s16x4 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)a0);
    const s16x4 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(size_t)(a0 + 1024));
    const u32x2 w0 = __builtin_bit_cast(u32x2, r0);
    const u32x2 w1 = __builtin_bit_cast(u32x2, r1);
    return as_bf16x8(u32x4{w0[0], w0[1], w1[0], w1[1]});
  };
  // Keys past the end of a partial tile never win.  Lane holds keys
  // 32 (kb >> 1) + 8 grp + 4 (kb & 1) + i of queries 16 qb + ql.
  auto mask = [&](f32x4 (&s)[4][4], int nvalid) {
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool dead = 32 * (kb >> 1) + 8 * grp + 4 * (kb & 1) + i >= nvalid;
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) s[kb][qb][i] = dead ? -INFINITY : s[kb][qb][i];
      }
  };

  // Tile pipeline.  Iteration j starts with S(j) in registers and runs two phases:
  //   R1: S(j+1) = K(j+1) Q^T on the MFMAs (key rows 0-31, then 32-63), with the softmax
  //       of S(j) on the VALU in between;
  //   R2: O += P(j) V(j) on the MFMAs (key rows 0-31 of V, then 32-63), with the moves of
  //       S(j+1) out of the accumulator registers in between.
  // So the exp work of one tile runs under the MFMAs of the next.  The K and V buffers are
  // refilled by 32-row halves as soon as a half has been read, one load per four MFMAs:
  //   R1 first half:  V(j) rows 32-63      R1 second half: K(j+2) rows 0-31
  //   R2 first half:  K(j+2) rows 32-63    R2 second half: V(j+1) rows 0-31
  // Every half lands at least half a phase after it was issued; each wait leaves the 15 or
  // 16 loads issued after the awaited half in flight.  P(j) is taken against the running
  // max as it stands; in the rare case its row sums pass RESCALE_SUM the max is moved to
  // the tile's (O and l rescaled) and P(j) is taken again.
  unsigned c_off = NO_TILE, c_flags = 0, n_off = NO_TILE, n_flags = 0;
  f32x4 scur[4][4];
  // the extra tokens' tile: byte offset of the token row of this lane's row 4 n + gi in copy
  // n (out of range past the nx tokens, so that row reads zero)
  unsigned xo[16];
  if (hx) {
    const int* xt = xtok + ((size_t)bh * g.Qs + srow) * VSA_MAX_EXTRA;
#pragma unroll
    for (int n = 0; n < 16; ++n) {
      const int r = 4 * n + gi;
      xo[n] = r < nx ? (unsigned)xt[r] * rowbytes : NO_TILE;
    }
  }
  // copy n of the extra tokens' K or V rows 0-31: the token rows' 16-byte chunks, swizzled as
  // the lane offsets koff / voff place them (their gi row term replaced by the token's row)
  auto xdma = [&](__amdgpu_buffer_rsrc_t rs, unsigned vo, int n, unsigned buf) {
    bdma16<0, true>(rs, xo[n] + (vo - (unsigned)gi * rowbytes), 0u, buf + 1024u * (unsigned)n);
  };
  if (my_n > 0) {
    describe(0);
    c_off = __builtin_amdgcn_readlane(d_off, 0);
    c_flags = __builtin_amdgcn_readlane(d_flags, 0);
    if (my_n > 1) {
      n_off = __builtin_amdgcn_readlane(d_off, 1);
      n_flags = __builtin_amdgcn_readlane(d_flags, 1);
    }
    unsigned stp, stl;
    steps(c_flags, stp, stl);
    if (SH) {
      kdma_q(0, c_off, stp, stl);
      kdma_q(1, c_off, stp, stl);
    } else if (hx) {
      // the extra tokens' K rows into the V buffer and K(1) into the K buffer, as below
#pragma unroll
      for (int n = 0; n < 16; ++n) xdma(krs, koff[(n >> 1) & 3], n, vbuf_u);
      unsigned n_stp, n_stl;
      steps(n_flags, n_stp, n_stl);
#pragma unroll
      for (int n = 0; n < 16; ++n) kdma(n, n_off, n_stp, n_stl);
    } else {
      // K(0) into the (still idle) V buffer and K(1) into the K buffer, both in flight
      // together: the first tile's product then reads the V buffer, and the loop finds K(1)
      // in place without a second round trip
#pragma unroll
      for (int n = 0; n < 16; ++n) dma(krs, koff[(n >> 1) & 3], n, c_off, stp, stl, vbuf_u);
      unsigned n_stp, n_stl;
      steps(n_flags, n_stp, n_stl);
#pragma unroll
      for (int n = 0; n < 16; ++n) kdma(n, n_off, n_stp, n_stl);
    }
  }
  // K(0) sits in the V buffer (same layout) except in the dense call: its reads are offset by this
  const unsigned k0_shift = !SH ? vbuf_u - kbuf_u : 0u;
  // Q, the epilogue's copies and K(0) (outside the dense call K(1) too) landed.  A wait the compiler
  // sees, on every path to the loop, so it does not wait (whole queue) for the Q loads again.
  __builtin_amdgcn_s_waitcnt(0);
  meet();  // SH: every wave's quarter of K(0) landed
  if (my_n > 0) {
    unsigned stp, stl;
    steps(c_flags, stp, stl);
    {
      auto kread0 = [&](int s) -> bf16x8 {
        const int kb = s >> 2;
        return as_bf16x8(*(const lds_u32x4*)(size_t)(kbase[s & 3] + k0_shift + 256 * (32 * (kb >> 1) + 4 * (kb & 1))));
      };
      f32x4 s0[4][4];
      bf16x8 ka[2];
      ka[0] = kread0(0);
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        if (s < 15) ka[(s + 1) & 1] = kread0(s + 1);
        const int kb = s >> 2, ks = s & 3;
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          s0[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s & 1], qv[qb][ks],
                                                               ks == 0 ? zero4 : s0[kb][qb], 0, 0, 0);
      }
      // S(0) to VGPRs by the same explicit moves as every later tile, so S stays in one
      // register file across the loop.  The scheduling barrier keeps every MFMA above the
      // NOPs, which cover the MFMA-result-to-VALU-read latency the compiler does not see
      // through the asm moves.
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i) scur[kb][qb][i] = acc_read(s0[kb][qb][i]);
    }
    // The buffer K(0) was read from is free once its reads returned: K(1) (zeros past the
    // end of the list; outside the dense call already in place), then V(0) rows 0-31, as
    // iteration 0 expects them in flight
    wait_lgkm0();
    meet();  // SH: every wave has read K(0)
    unsigned n_stp, n_stl;
    steps(n_flags, n_stp, n_stl);
    if (SH) {
      kdma_q(0, n_off, n_stp, n_stl);
      kdma_q(1, n_off, n_stp, n_stl);
      vdma_q(0, c_off, stp, stl);
    }
    if (SH) {
    } else if (hx) {
#pragma unroll
      for (int n = 0; n < 8; ++n) xdma(vrs, voff[(n >> 1) & 1], n, vbuf_u);
    } else {
#pragma unroll
      for (int n = 0; n < 8; ++n) vdma_r(vrs0, n, c_off, stp, stl);
    }
    if ((int)(c_flags >> 1) < VSA_TILE_TOKENS) mask(scur, (int)(c_flags >> 1));
    // the first tile sets the running max
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      float m = scur[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) m = fmaxf(m, scur[kb][qb][i]);
      mrun[qb] = group_max(m) * sl2;
    }
  }

  __amdgpu_buffer_rsrc_t vrs_c = vrs0;  // V(j)'s resource: the first tile's, then the plain one
  for (int j = 0; j < my_n; ++j) {
    unsigned nn_off = NO_TILE, nn_flags = 0;
    if (j + 2 < my_n) {
      if (((j + 2) & 63) == 0) describe((j + 2) >> 6);
      nn_off = __builtin_amdgcn_readlane(d_off, (j + 2) & 63);
      nn_flags = __builtin_amdgcn_readlane(d_flags, (j + 2) & 63);
    }
    unsigned c_stp, c_stl, n_stp, n_stl, nn_stp, nn_stl;
    steps(c_flags, c_stp, c_stl);
    steps(n_flags, n_stp, n_stl);
    steps(nn_flags, nn_stp, nn_stl);

    // softmax of S(j), chunk s = (key block s >> 2, query block s & 3): P against the
    // running max and the lane's share of the tile's row sums; P packed to bf16 PV
    // operands once both key blocks of a 32-key step are done
    bf16x8 pb[4][2];
    float lt[4];
    unsigned pe[4][2];  // bf16 pairs of the even key block, until its odd partner is done
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) lt[qb] = 0.f;
    // The row sums add the bf16-rounded probabilities, two per dot2 against (1, 1): the
    // normaliser is then the sum of exactly the weights the PV product applies.
    auto soft = [&](int s) {
      const int kb = s >> 2, qb = s & 3;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(fmaf(scur[kb][qb][i], sl2, -mrun[qb]));
      const unsigned w0 = pack_bf16x2(p[0], p[1]), w1 = pack_bf16x2(p[2], p[3]);
      lt[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w0), ONES_BF16X2, lt[qb], false);
      lt[qb] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w1), ONES_BF16X2, lt[qb], false);
      if (kb & 1) {
        pb[qb][kb >> 1] = as_bf16x8(u32x4{pe[qb][0], pe[qb][1], w0, w1});
      } else {
        pe[qb][0] = w0;
        pe[qb][1] = w1;
      }
    };

    // ---- R1.  On the last tile the K buffer holds the zeros loaded for the tile past the
    // end; that product is not used, and costs nothing next to the softmax beside it.
    // K(j+1) rows 0-31 landed (in flight after them: K(j+1) rows 32-63, V(j) rows 0-31).
    if (SH) {
      wait_vm<4>();  // own K(j+1) rows 0-31 (after them: K(j+1) rows 32-63, V(j) rows 0-31)
      meet();
    } else {
      wait_vm<16>();
    }
    f32x4 snext[4][4];
    {
      bf16x8 ka[2];
      ka[0] = kread(0);
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        // K(j+1) rows 32-63 landed before their first read (in flight after them: V(j)
        // rows 0-31 and the 7 loads of V(j) rows 32-63 issued so far)
        if (s == 7) {
          if (SH) {
            // own K(j+1) rows 32-63 (after them: V(j) rows 0-31, V(j) rows 32-63), and this
            // wave's reads of rows 0-31 done before any wave refills them
            wait_lgkm0();
            wait_vm<4>();
            meet();
          } else {
            wait_vm<15>();
          }
        }
        if (s < 15) ka[(s + 1) & 1] = kread(s + 1);
        const int kb = s >> 2, ks = s & 3;
#pragma unroll
        for (int qb = 0; qb < 4; ++qb)
          snext[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s & 1], qv[qb][ks],
                                                                  ks == 0 ? zero4 : snext[kb][qb], 0, 0, 0);
        soft(s);
        if (s < 15) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x402, 4, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (SH) {
          if (s == 0) vdma_q(1, c_off, c_stp, c_stl);    // V(j) rows 32-63
          if (s == 8) kdma_q(0, nn_off, nn_stp, nn_stl);  // K(j+2) rows 0-31
        } else if (s < 8) {
          vdma_r(vrs_c, 8 + s, c_off, c_stp, c_stl);  // V(j) rows 32-63
        } else {
          kdma(s - 8, nn_off, nn_stp, nn_stl);  // K(j+2) rows 0-31 (read by steps 0-7)
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }

    // P(j) and its row sums are produced above, under the MFMAs, even though the rare
    // path below takes them again: an empty asm that reads and rewrites them keeps the
    // compiler from sinking that work past the check.
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) {
      asm volatile("" : "+v"(pb[qb][0]), "+v"(pb[qb][1]), "+v"(lt[qb]));
    }

    // ---- the rescale check (wave-uniform; rarely taken): a lane's share of a row sum
    // passing RESCALE_SUM (or not finite) moves the running max to the tile's max
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) grow |= !(lt[qb] <= RESCALE_SUM);
    if (__ballot(grow)) {
      float alpha[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        float m = scur[0][qb][0];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) m = fmaxf(m, scur[kb][qb][i]);
        const float mn = fmaxf(mrun[qb], group_max(m) * sl2);
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
      // Per (db, qb) block one asm sequence: O's four accumulator values are moved to four
      // distinct VGPRs, then the four MFMAs, with explicit waits (the compiler sees none of
      // these instructions): after the moves before the MFMAs read them, between the
      // dependent MFMAs, and at the end so that no later write reaches a register an MFMA
      // may still be reading.  The whole rescale is rare, so the waits cost nothing.
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          f32x4 acc;
          float t0, t1, t2, t3;
          asm volatile(
              "v_accvgpr_read_b32 %[t0], %[o0]\n\t"
              "v_accvgpr_read_b32 %[t1], %[o1]\n\t"
              "v_accvgpr_read_b32 %[t2], %[o2]\n\t"
              "v_accvgpr_read_b32 %[t3], %[o3]\n\t"
              "s_nop 4\n\t"
              "v_mfma_f32_16x16x4_f32 %[d], %[a0], %[t0], 0\n\t"
              "s_nop 3\n\t"
              "v_mfma_f32_16x16x4_f32 %[d], %[a1], %[t1], %[d]\n\t"
              "s_nop 3\n\t"
              "v_mfma_f32_16x16x4_f32 %[d], %[a2], %[t2], %[d]\n\t"
              "s_nop 3\n\t"
              "v_mfma_f32_16x16x4_f32 %[d], %[a3], %[t3], %[d]\n\t"
              "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
              : [d] "=&a"(acc), [t0] "=&v"(t0), [t1] "=&v"(t1), [t2] "=&v"(t2), [t3] "=&v"(t3)
              : [o0] "a"(oacc[db][qb][0]), [o1] "a"(oacc[db][qb][1]), [o2] "a"(oacc[db][qb][2]),
                [o3] "a"(oacc[db][qb][3]), [a0] "v"(asel[qb][0]), [a1] "v"(asel[qb][1]),
                [a2] "v"(asel[qb][2]), [a3] "v"(asel[qb][3]));
          oacc[db][qb] = acc;
        }
      // the last MFMA results are complete before anything reads them
      asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      // P(j) again, against the moved max
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) lt[qb] = 0.f;
#pragma unroll
      for (int s = 0; s < 16; ++s) soft(s);
    }
#pragma unroll
    for (int qb = 0; qb < 4; ++qb) lsum[qb] += lt[qb];

    // ---- R2.  K(j+1) reads returned (the K buffer may be refilled); V(j) rows 0-31 landed
    // (in flight after them: V(j) rows 32-63, K(j+2) rows 0-31).
    wait_lgkm0();
    if (SH) {
      wait_vm<4>();  // own V(j) rows 0-31 (after them: V(j) rows 32-63, K(j+2) rows 0-31)
      meet();
    } else {
      wait_vm<16>();
    }
    // S(j+1) is read out of the accumulator registers below: cover the MFMA-result latency
    // (the barrier keeps the QK MFMAs above the NOPs)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    {
      // step u = (32-key step u >> 3, dim block u & 7); its V operand is read during step u-1
      bf16x8 va[2];
      va[0] = vread(0);
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        // V(j) rows 32-63 landed before their first read (in flight after them: K(j+2)
        // rows 0-31 and the 7 loads of K(j+2) rows 32-63 issued so far)
        if (u == 7) {
          if (SH) {
            // own V(j) rows 32-63 (after them: K(j+2) rows 0-31, K(j+2) rows 32-63), and this
            // wave's reads of rows 0-31 done before any wave refills them
            wait_lgkm0();
            wait_vm<4>();
            meet();
          } else {
            wait_vm<15>();
          }
        }
        if (u < 15) va[(u + 1) & 1] = vread(u + 1);
        const int c = u >> 3, db = u & 7;
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          oacc[db][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pb[qb][c], va[u & 1], oacc[db][qb], 0, 0, 0);
          // four of the 64 values of S(j+1) per step: key block u >> 2, query block u & 3
          scur[u >> 2][u & 3][qb] = acc_read(snext[u >> 2][u & 3][qb]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (SH) {
          if (u == 0) kdma_q(1, nn_off, nn_stp, nn_stl);  // K(j+2) rows 32-63
          if (u == 8) vdma_q(0, n_off, n_stp, n_stl);     // V(j+1) rows 0-31
        } else if (u < 8) {
          kdma(8 + u, nn_off, nn_stp, nn_stl);  // K(j+2) rows 32-63 (read by R1 steps 8-15)
        } else {
          vdma(u - 8, n_off, n_stp, n_stl);  // V(j+1) rows 0-31 (read by steps 0-7)
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // V buffer is free once its reads returned
    wait_lgkm0();
    c_off = n_off;
    c_flags = n_flags;
    n_off = nn_off;
    n_flags = nn_flags;
    vrs_c = vrs;
    if (j + 1 < my_n && (int)(c_flags >> 1) < VSA_TILE_TOKENS) mask(scur, (int)(c_flags >> 1));
  }
  // the loads issued past the end of the list (out of range, writing zeros) must land
  // before the K buffer is reused below
  wait_vm<0>();
  if (SH) {
    wait_lgkm0();
    meet();  // every wave is done with the shared K and V buffers
  }
  // ---- O and l to LDS.  Softmax statistics are per lane for queries 16 qb + ql; O is
  // held as oacc[db][qb][i] = O[16 qb + 4 grp + i][16 db + ql].  O^T goes to the K/V
  // buffers: dims 0..63 in the K area, 64..127 in the V area, each dim a 256-byte row of
  // 64 fp32 queries; the 16-byte chunk of queries 4c..4c+3 sits at chunk c ^ (dim & 15).
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    lsum[qb] = group_sum(lsum[qb]);
    if (grp == 0) lbuf[64 * wv + 16 * qb + ql] = lsum[qb];
  }
  auto part = [&](int d) -> lds_u32x4* {
    if (SH && wv > 0)
      return (lds_u32x4*)((char*)lst_lds + (2 * (wv - 1) + (d < 64 ? 0 : 1)) * TILE_BYTES) + (d & 63) * 16;
    return (lds_u32x4*)(d < 64 ? klds : vlds) + (d & 63) * 16;
  };
#pragma unroll
  for (int qb = 0; qb < 4; ++qb)
#pragma unroll
    for (int db = 0; db < 8; ++db) part(16 * db + ql)[(4 * qb + grp) ^ ql] = __builtin_bit_cast(u32x4, oacc[db][qb]);
  __syncthreads();

  // ---- epilogue, four passes: pass w writes queries 16 w + 4 (lane / 16) .. +3, dims
  // 8 (lane % 16) .. +7.  The gate and coarse-output loads are issued first.
  const int qg = lane >> 4, dg = lane & 15;
  const bool gated = !dense && gate != nullptr;
  f32x4 oc0 = f32x4{0.f, 0.f, 0.f, 0.f}, oc1 = oc0;
  u32x4 gv[4][4];
  int qtok[4][4];
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qtok[w][i] = qvalid ? tile_token(g, qt, 16 * w + 4 * qg + i) : -1;
      gv[w][i] = u32x4{0u, 0u, 0u, 0u};
      if (gated && qtok[w][i] >= 0)
        gv[w][i] = *reinterpret_cast<const u32x4*>(gate + row_offset(g, b, qtok[w][i], h) + 8 * dg);
    }
  if (gated) {
    const f32x4* cp = reinterpret_cast<const f32x4*>(ocoarse + ((size_t)bh * g.Qs + srow) * VSA_HEAD_DIM + 8 * dg);
    oc0 = cp[0];
    oc1 = cp[1];
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int q0 = 16 * w + 4 * qg;
    float r[4][8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = 8 * dg + e;
      const f32x4 sv = __builtin_bit_cast(f32x4, part(d)[(q0 >> 2) ^ (d & 15)]);
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i][e] = sv[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (qtok[w][i] < 0) continue;
      const float ltot = lbuf[64 * wv + q0 + i];
      const float inv = ltot > 0.f ? 1.0f / ltot : 0.f;  // an empty list gives O_fine = 0
      float y[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) y[e] = r[i][e] * inv;
      if (gated) {
        const u32x4 gw = gv[w][i];
        y[0] += bf16lo(gw[0]) * oc0[0];
        y[1] += bf16hi(gw[0]) * oc0[1];
        y[2] += bf16lo(gw[1]) * oc0[2];
        y[3] += bf16hi(gw[1]) * oc0[3];
        y[4] += bf16lo(gw[2]) * oc1[0];
        y[5] += bf16hi(gw[2]) * oc1[1];
        y[6] += bf16lo(gw[3]) * oc1[2];
        y[7] += bf16hi(gw[3]) * oc1[3];
      }
      *reinterpret_cast<u32x4*>(o + row_offset(g, b, qtok[w][i], h) + 8 * dg) =
          u32x4{pack_bf16x2(y[0], y[1]), pack_bf16x2(y[2], y[3]), pack_bf16x2(y[4], y[5]), pack_bf16x2(y[6], y[7])};
    }
  }
}

}  // namespace

void vsa_launch_fine(const VsaGeom& g, const void* q, const void* k, const void* v, const void* gate,
                     const float* ocoarse, const int* lists, const int* counts, void* o,
                     const int* xtok, const void* vx, const int* xcnt, hipStream_t st) {
  if (g.n_dense == g.Tq) {
    // every row dense (the dense call): four query tiles of a (batch, head) per workgroup
    const int groups = g.batch * g.heads * ((g.Tq + 3) / 4);
    const int per_xcd = (groups + 7) / 8;
    hipLaunchKernelGGL((vsa_fine_kernel<false, true>), dim3(8 * per_xcd), dim3(256), (size_t)6 * TILE_BYTES, st, g,
                       (const char*)k,
                       (const char*)v, (const u32x4*)q, (const unsigned short*)gate, ocoarse, lists, counts,
                       (unsigned short*)o, per_xcd, xtok, (const char*)vx, xcnt);
    return;
  }
  const int total = g.batch * g.heads * g.Tq;
  const int per_xcd = (total + 7) / 8;
  auto kern = g.extra > 0 ? vsa_fine_kernel<true, false> : vsa_fine_kernel<false, false>;
  hipLaunchKernelGGL(kern, dim3(8 * per_xcd), dim3(64), (size_t)g.cap * sizeof(int), st, g, (const char*)k,
                     (const char*)v, (const u32x4*)q, (const unsigned short*)gate, ocoarse, lists,
                     counts, (unsigned short*)o, per_xcd, xtok, (const char*)vx, xcnt);
}
