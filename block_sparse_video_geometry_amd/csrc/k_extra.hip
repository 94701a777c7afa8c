// Extra tokens: per sparse query tile, the best-scoring single key tokens outside
// the tiles of its list.
//
// "ComfyUI Agrega Nodo Central de Atencion Dispersa y Compilador Comfy", the
// schedule paragraph: extra_tokens adds the top-scoring tokens beyond the
// selected blocks, to stay closer to dense.  The score of key token t for
// sparse query tile i is the coarse branch's pooled query against the raw key,
// z = s qbar_i . k_t (no tile bias); over the valid tokens of the tiles not in
// i's list the E largest are kept, equal scores to the lower packed token index.
//
// vsa_extra_select_kernel: one workgroup per (64 sparse rows, head, batch), wave
// w owns rows 16 w .. 16 w + 15.  Every key tile of the head streams through LDS
// in tile-id order (the next two tiles' loads in flight in registers meanwhile):
//   Z^T (64 keys x 16 rows) = K qbar^T on the bf16 MFMAs, with qbar split exactly
//     into three bf16 terms hi + mid + lo, so the products are exact and only the
//     fp32 accumulation rounds: the ranking then holds the fp32 order (a plain
//     bf16 qbar would move logits by ~2^-9 of their size).
//   A tile in the row's list is skipped with a per-row cursor into the (ascending)
//     list; padding rows of a partial prefix tile are skipped by their index.
//   Streaming top-E: a key enters the row's LDS candidate buffer only if it beats
//     the row's threshold, the E-th best (score, token) seen so far.  When a tile's
//     entrants would overflow a buffer the wave first cuts it back to its E best
//     with a bitwise ballot search over the 64-bit keys (score order, then ~token),
//     which also raises the threshold, and tests the tile's keys again.  The keys
//     are unique, so every cut keeps exactly E.  With E = 64 a row is cut about
//     (64 + 64 ln(tiles / 2)) / 64 times.
//   Scoring: a key passes if its float score is >= the threshold's; only a score equal
//     to it needs the full (score, token) key, and keys are built only for the few
//     that enter.
// At the end each row is cut to at most E, ranked by token and written ascending.
// The kernel issues ~0.4k VALU instructions per tile per wave against 48 MFMAs, at
// about one wave per SIMD, so it is bound by issue and latency rather than by the MFMAs.
//
// vsa_extra_gather_kernel: copies each row's extra K and V rows into staging
// buffers laid out [batch, Qs, 64, heads, 128] (padding rows zero), i.e. with
// the token stride of K and V themselves, so the fine kernel reads a row's
// extra tokens as one more 64-row tile of consecutive rows.
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

constexpr int XROWS = 64;   // sparse rows per workgroup, 16 per wave
constexpr int XCAP = 128;   // candidate buffer entries per row (a tile adds at most 64)

__device__ __forceinline__ unsigned order_key(float f) {
  if (f == 0.0f) f = 0.0f;
  const unsigned u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lanes_below(unsigned long long mask) {
  return __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

// The value x of the four lanes (lane & 15) + 16 r, r = 0..3, in every one of them: out[r] from
// 16-lane row r.  permlane16_swap(x, x) gives {x of row r & ~1, x of row r | 1}; a permlane32_swap
// of each half of that gives rows 0 and 2, or 1 and 3.
__device__ __forceinline__ void row_values4(int x, int out[4]) {
  const auto a = __builtin_amdgcn_permlane16_swap((unsigned)x, (unsigned)x, false, false);
  const auto e = __builtin_amdgcn_permlane32_swap(a[0], a[0], false, false);
  const auto o = __builtin_amdgcn_permlane32_swap(a[1], a[1], false, false);
  out[0] = (int)e[0];
  out[1] = (int)o[0];
  out[2] = (int)e[1];
  out[3] = (int)o[1];
}

// The bits of a where m is set and of b elsewhere: one v_bfi_b32, written as asm so that a
// tree of these is not folded back into an indexed read of a register array (which the
// compiler would place in scratch memory).
__device__ __forceinline__ unsigned bit_pick(unsigned m, unsigned a, unsigned b) {
  unsigned r;
  asm("v_bfi_b32 %0, %1, %2, %3" : "=v"(r) : "v"(m), "v"(a), "v"(b));
  return r;
}

// x = hi + mid + lo exactly (each term the bf16 round-to-nearest of what is left).
__device__ __forceinline__ void split3(float x, __bf16& hi, __bf16& mid, __bf16& lo) {
  hi = (__bf16)x;
  const float r1 = x - (float)hi;
  mid = (__bf16)r1;
  const float r2 = r1 - (float)mid;
  lo = (__bf16)r2;
}

// Walks the tiles in id order without divisions: tile t's first packed token, its valid
// token count and whether it is a video tile (rows then step dt, dh, dw through the grid;
// a prefix tile's rows are consecutive tokens).  All fields are wave-uniform.
struct TileWalk {
  int t, tok0, nv, video;
  int seg, tin;    // prefix: segment, tile within it
  int tw, th, tt;  // video: tile coordinates
};
__device__ __forceinline__ void walk_set(const VsaGeom& g, TileWalk& w) {
  if (w.t < g.P) {
    const int off = VSA_TILE_TOKENS * w.tin;
    w.tok0 = g.pre_start[w.seg] + off;
    w.nv = min(VSA_TILE_TOKENS, g.pre_len[w.seg] - off);
    w.video = 0;
  } else {
    w.tok0 = g.vstart + (4 * w.tt * g.H + 4 * w.th) * g.W + 4 * w.tw;
    w.nv = VSA_TILE_TOKENS;
    w.video = 1;
  }
}
__device__ __forceinline__ void walk_init(const VsaGeom& g, TileWalk& w) {
  w.t = w.seg = w.tin = w.tw = w.th = w.tt = 0;
  walk_set(g, w);
}
__device__ __forceinline__ void walk_next(const VsaGeom& g, TileWalk& w) {
  if (w.t < g.P) {  // leaving a prefix tile
    if (w.t + 1 < g.pre_tile0[w.seg + 1]) {
      ++w.tin;
    } else {
      ++w.seg;
      w.tin = 0;
    }
  } else if (++w.tw == g.tw_n) {
    w.tw = 0;
    if (++w.th == g.th_n) {
      w.th = 0;
      ++w.tt;
    }
  }
  ++w.t;
  walk_set(g, w);
}

// A buffer entry holds the float score's bits over ~token.  Its 64-bit order key is larger
// for the better candidate (score order, then the lower token); an empty slot's key is 0.
__device__ __forceinline__ unsigned long long entry(float z, int tok) {
  return ((unsigned long long)__float_as_uint(z) << 32) | (unsigned)(~tok);
}
__device__ __forceinline__ unsigned long long entry_key(unsigned long long e) {
  return ((unsigned long long)order_key(__uint_as_float((unsigned)(e >> 32))) << 32) | (unsigned)e;
}

__global__ __launch_bounds__(256) void vsa_extra_select_kernel(VsaGeom g, const u32x4* __restrict__ k,
                                                               const float* __restrict__ qbar,
                                                               const int* __restrict__ lists,
                                                               const int* __restrict__ counts,
                                                               int* __restrict__ xtok,
                                                               int* __restrict__ xcnt) {
  // K tile: key row r at 256 r, 16-byte chunk c at position c ^ (r & 15)
  __shared__ __attribute__((aligned(16))) char ktile[64 * 256];
  __shared__ unsigned long long cbuf[XROWS][XCAP];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, ql = lane & 15;
  const int b = blockIdx.z, h = blockIdx.y;
  const size_t bh = (size_t)b * g.heads + h;
  const int rl = 16 * wave + ql;           // this lane's row in the workgroup
  const int r = blockIdx.x * XROWS + rl;   // its sparse row
  const bool live = r < g.Qs;
  const int E = g.extra;

  // B operands: qbar of row r, dims 32 ks + 8 grp .. +7, as hi / mid / lo bf16 terms
  bf16x8 qs[3][4];
  {
    const f32x4* qp = reinterpret_cast<const f32x4*>(qbar + (bh * g.Tq + g.n_dense + (live ? r : 0)) * VSA_HEAD_DIM);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x4 a = live ? qp[8 * ks + 2 * grp] : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x4 c = live ? qp[8 * ks + 2 * grp + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
      const float x[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hi, mid, lo;
        split3(x[e], hi, mid, lo);
        qs[0][ks][e] = hi;
        qs[1][ks][e] = mid;
        qs[2][ks][e] = lo;
      }
    }
  }

  // list cursor: entry cur of this row's (ascending) list is the next listed tile; it is
  // loaded every tile, one tile ahead of its use, so every step issues the same loads
  const int* lst = lists + (bh * g.Qs + (live ? r : 0)) * g.cap;
  const int cnt_l = live ? counts[bh * g.Qs + r] : 0;
  int cur = 0;
  int nl = lst[0];

  int nrow = 0;                  // entries in this row's buffer (same in its four lanes)
  unsigned long long th = 0ull;  // a key must beat this to enter (0: nothing seen yet)
  float thz = -INFINITY;         // the score of th: a key scoring below it cannot enter

  // Cut row rc (workgroup row) from n entries to its best `keep`; returns the keep-th key.
  auto cut = [&](int rc, int n, int keep) -> unsigned long long {
    const bool v0 = lane < n, v1 = lane + 64 < n;
    const unsigned long long r0 = v0 ? cbuf[rc][lane] : 0ull;
    const unsigned long long r1 = v1 ? cbuf[rc][lane + 64] : 0ull;
    const unsigned long long k0 = v0 ? entry_key(r0) : 0ull;
    const unsigned long long k1 = v1 ? entry_key(r1) : 0ull;
    // the keep-th largest score word (an empty slot's 0 is below every real one) ...
    const unsigned h0 = (unsigned)(k0 >> 32), h1 = (unsigned)(k1 >> 32);
    unsigned ph = 0u;
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned cand = ph | (1u << bit);
      const int c = __popcll(__ballot(h0 >= cand)) + __popcll(__ballot(h1 >= cand));
      if (c >= keep) ph = cand;
    }
    // ... then, only if several entries share it at the boundary, the token word
    const int need = keep - (__popcll(__ballot(h0 > ph)) + __popcll(__ballot(h1 > ph)));
    const bool e0 = v0 && h0 == ph, e1 = v1 && h1 == ph;
    unsigned pl = 0u;
    if (__popcll(__ballot(e0)) + __popcll(__ballot(e1)) > need) {
      const unsigned l0 = (unsigned)k0, l1 = (unsigned)k1;
      for (int bit = 31; bit >= 0; --bit) {
        const unsigned cand = pl | (1u << bit);
        const int c = __popcll(__ballot(e0 && l0 >= cand)) + __popcll(__ballot(e1 && l1 >= cand));
        if (c >= need) pl = cand;
      }
    }
    const unsigned long long pre = ((unsigned long long)ph << 32) | pl;
    const bool s0 = v0 && k0 >= pre, s1 = v1 && k1 >= pre;
    const unsigned long long b0 = __ballot(s0), b1 = __ballot(s1);
    // every lane has its two entries in registers before any write below
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    if (s0) cbuf[rc][lanes_below(b0)] = r0;
    if (s1) cbuf[rc][__popcll(b0) + lanes_below(b1)] = r1;
    return pre;
  };

  // staging of a key tile: thread tid moves rows r = (tid >> 4) + 16 m, chunk tid & 15;
  // in a video tile row r is (dt, dh, dw) = (m, (tid >> 6) & 3, (tid >> 4) & 3)
  const int hw = g.H * g.W;
  const int fdhw = ((tid >> 6) & 3) * g.W + ((tid >> 4) & 3);
  const u32x4* kbh = k + (((size_t)b * g.N) * g.heads + h) * (VSA_HEAD_DIM / 8) + (tid & 15);
  const int tokstride = g.heads * (VSA_HEAD_DIM / 8);  // u32x4 per token
  // two tiles in flight: slot t & 1 holds tile t, loaded two steps back.  A padding row
  // loads row 0 (always valid) and is zeroed when stashed (bit m of the slot's mask), so
  // every load is unconditional and nothing reads a slot before its stash.
  u32x4 kr[2][4];
  unsigned kv[2];
  auto fetch = [&](const TileWalk& w, u32x4 (&dst)[4], unsigned& vmask) {
    vmask = 0u;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int r = (tid >> 4) + 16 * m;
      const bool valid = w.video || r < w.nv;
      const int tok = w.tok0 + (w.video ? m * hw + fdhw : (valid ? r : 0));
      dst[m] = kbh[(size_t)tok * tokstride];
      vmask |= (unsigned)valid << m;
    }
  };
  auto stash = [&](const u32x4 (&src)[4], unsigned vmask) {
    if (vmask == 0xfu) {  // all four rows valid (every video tile)
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = (tid >> 4) + 16 * m;
        *reinterpret_cast<u32x4*>(ktile + 256 * row + 16 * ((tid & 15) ^ (row & 15))) = src[m];
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = (tid >> 4) + 16 * m;
        *reinterpret_cast<u32x4*>(ktile + 256 * row + 16 * ((tid & 15) ^ (row & 15))) =
            ((vmask >> m) & 1u) ? src[m] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  TileWalk wc, wf;  // the tile being scored and the last one fetched
  walk_init(g, wc);
  wf = wc;
  fetch(wf, kr[0], kv[0]);
  if (g.Tq > 1) walk_next(g, wf);
  fetch(wf, kr[1], kv[1]);
  // one tile: stage it, refill its slot two tiles ahead, score it, admit its keys
  auto step = [&](int t, u32x4 (&slot)[4], unsigned& vmask) {
    __syncthreads();  // every wave is done with the previous tile
    stash(slot, vmask);
    __syncthreads();
    // refill two tiles ahead (past the end the last tile again: every step issues the
    // same loads, so the wait before a stash leaves the other slot's loads in flight)
    if (t + 2 < g.Tq) walk_next(g, wf);
    fetch(wf, slot, vmask);
    __builtin_amdgcn_sched_barrier(0);  // the refill is issued before the wait for nl below
    // the list entry loaded last step, then the next one (used next step, after that
    // step's refill has been issued)
    const bool excl = cur < cnt_l && nl == t;
    cur += excl ? 1 : 0;
    nl = lst[min(cur, g.cap - 1)];

    // all 16 A operands first, then the 48 MFMAs with the four key blocks' accumulator
    // chains interleaved, so no MFMA waits on the one just before it
    bf16x8 a[4][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        a[kb][ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(ktile + 256 * (16 * kb + ql) + 16 * ((4 * ks + grp) ^ ql)));
    f32x4 acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int p = 2; p >= 0; --p) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kb][ks], qs[p][ks], acc[kb], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);  // keep the four chains interleaved
      }

    // lane holds keys 16 kb + 4 grp + i of the tile for its row
    const bool video = wc.video;
    const int tok0 = wc.tok0;
    const int nv = wc.nv;
    // admission on the float score: a key beats th iff z > thz, or z == thz and its
    // (score, token) order key is above th (thz is th's score; -inf before the first cut).
    // z >= thz is tested first; only a score equal to thz (rare) needs the exact key.
    float z[16];
    unsigned ge = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      z[e] = acc[e >> 2][e & 3] * g.scale;
      ge |= (unsigned)(z[e] >= thz) << e;
    }
    if (!video) {  // a prefix tile may end early: key 16 kb + 4 grp + i is valid iff below nv
      unsigned vm = 0u;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int nk = min(max(nv - 16 * kb - 4 * grp, 0), 4);
        vm |= ((1u << nk) - 1u) << (4 * kb);
      }
      ge &= vm;
    }
    if (!live || excl) ge = 0u;
    if (__ballot(ge != 0u) == 0ull) {  // nothing of this tile can enter any row
      walk_next(g, wc);
      return;
    }
    const int tokl = tok0 + (video ? grp * g.W : 4 * grp);  // key e: tokl + (video ? kb hw + i : 16 kb + i)
    auto tok_of = [&](int e) { return tokl + (e >> 2) * (video ? hw : 16) + (e & 3); };
    auto admit = [&]() {
      unsigned f = 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool beat = z[e] > thz || (z[e] == thz && entry_key(entry(z[e], tok_of(e))) > th);
        f |= (unsigned)(((ge >> e) & 1u) && beat) << e;
      }
      return f;
    };
    // a score equal to the row's threshold score anywhere in the lane (a superset of the
    // candidate ties; admit() applies ge)
    bool tie = false;
#pragma unroll
    for (int e = 0; e < 16; ++e) tie |= z[e] == thz;
    // counts over the four lanes of the row (lanes ql + 16 grp)
    unsigned flag = ge;
    if (__ballot(tie) != 0ull) flag = admit();  // a score tie with the threshold (rare)
    int c = __popc(flag);
    int cr[4];
    row_values4(c, cr);
    int c0 = cr[0], c1 = cr[1], c2 = cr[2], c3 = cr[3];
    // a row whose buffer would overflow is cut back to its E best first (raising its
    // threshold), and its keys are tested again; after a cut E + 64 <= XCAP entries fit
    unsigned long long full = __ballot(nrow + c0 + c1 + c2 + c3 > XCAP) & 0xffffull;
    if (full) {
      while (full) {
        const int rc = __builtin_ctzll(full);
        full &= full - 1;
        const int n = __shfl(nrow, rc);
        const unsigned long long T = cut(16 * wave + rc, n, E);
        if (ql == rc) {
          nrow = E;
          th = T;
          const unsigned sk = (unsigned)(T >> 32);  // back from the order key to the float
          thz = __uint_as_float((sk & 0x80000000u) ? (sk & 0x7fffffffu) : ~sk);
        }
      }
      // the keys again against the raised thresholds: the same float test, the exact key
      // only on a tie
      unsigned ge2 = 0u;
      bool tie2 = false;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        ge2 |= (unsigned)(z[e] >= thz) << e;
        tie2 |= z[e] == thz;
      }
      ge &= ge2;
      flag = ge;
      if (__ballot(tie2) != 0ull) flag = admit();
      c = __popc(flag);
      row_values4(c, cr);
      c0 = cr[0];
      c1 = cr[1];
      c2 = cr[2];
      c3 = cr[3];
    }
    int at = nrow + (grp > 0 ? c0 : 0) + (grp > 1 ? c1 : 0) + (grp > 2 ? c2 : 0);
    // the admitted keys, lowest e first: one pass per key of the lane that admits the most
    // (few once the buffer is warm); key e's score picked by a select tree on e's bits
    for (unsigned f = flag; __ballot(f != 0u) != 0ull;) {
      if (f != 0u) {
        const int e = __builtin_ctz(f);
        f &= f - 1u;
        const unsigned m0 = 0u - (e & 1), m1 = 0u - ((e >> 1) & 1), m2 = 0u - ((e >> 2) & 1),
                       m3 = 0u - ((e >> 3) & 1);
        unsigned l1[8], l2[4], l3[2];
#pragma unroll
        for (int j = 0; j < 8; ++j) l1[j] = bit_pick(m0, __float_as_uint(z[2 * j + 1]), __float_as_uint(z[2 * j]));
#pragma unroll
        for (int j = 0; j < 4; ++j) l2[j] = bit_pick(m1, l1[2 * j + 1], l1[2 * j]);
#pragma unroll
        for (int j = 0; j < 2; ++j) l3[j] = bit_pick(m2, l2[2 * j + 1], l2[2 * j]);
        cbuf[rl][at++] = entry(__uint_as_float(bit_pick(m3, l3[1], l3[0])), tok_of(e));
      }
    }
    nrow += c0 + c1 + c2 + c3;
    walk_next(g, wc);
  };
  for (int t = 0; t < g.Tq; t += 2) {
    step(t, kr[0], kv[0]);
    if (t + 1 < g.Tq) step(t + 1, kr[1], kv[1]);
  }

  // final cut to at most E, then rank by token and write ascending
  __builtin_amdgcn_s_waitcnt(0xc07f);
  for (int rc = 0; rc < 16; ++rc) {
    const int row = blockIdx.x * XROWS + 16 * wave + rc;
    if (row >= g.Qs) break;
    int n = __shfl(nrow, rc);
    if (n > E) {
      cut(16 * wave + rc, n, E);
      n = E;
      __builtin_amdgcn_s_waitcnt(0xc07f);
    }
    const int mytok = lane < n ? ~(int)(unsigned)cbuf[16 * wave + rc][lane] : 0;
    int rank = 0;
    for (int e = 0; e < n; ++e) rank += (~(int)(unsigned)cbuf[16 * wave + rc][e] < mytok) ? 1 : 0;
    const size_t ro = bh * g.Qs + row;
    if (lane < n) xtok[ro * VSA_MAX_EXTRA + rank] = mytok;
    if (lane == 0) xcnt[ro] = n;
  }
}

// One workgroup per (sparse row, head, batch): thread tid copies 64 bytes of extra row
// tid >> 2 (zeros past the row's count) of K and of V.
__global__ __launch_bounds__(256) void vsa_extra_gather_kernel(VsaGeom g, const u32x4* __restrict__ k,
                                                               const u32x4* __restrict__ v,
                                                               const int* __restrict__ xtok,
                                                               const int* __restrict__ xcnt,
                                                               u32x4* __restrict__ kx,
                                                               u32x4* __restrict__ vx) {
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t ro = ((size_t)b * g.heads + h) * g.Qs + s;
  const int e = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int n = xcnt[ro];
  // destination row (b, s, e) of the [batch, Qs, 64, heads, 128] staging, head h
  const size_t dst = ((((size_t)b * g.Qs + s) * VSA_MAX_EXTRA + e) * g.heads + h) * 16 + 4 * part;
  u32x4 ka[4], va[4];
  if (e < n) {
    // (a token id outside the sequence cannot come from the select kernel; clamped all the
    // same, so that a read never leaves the (b, h) plane)
    const int tok = min(max(xtok[ro * VSA_MAX_EXTRA + e], 0), g.N - 1);
    const long long src = row_offset(g, b, tok, h) / 8 + 4 * part;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ka[i] = k[src + i];
      va[i] = v[src + i];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) ka[i] = va[i] = u32x4{0u, 0u, 0u, 0u};
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    kx[dst + i] = ka[i];
    vx[dst + i] = va[i];
  }
}

}  // namespace

void vsa_launch_extra(const VsaGeom& g, const void* k, const void* v, const float* qbar, const int* lists,
                      const int* counts, int* xtok, int* xcnt, void* kx, void* vx, hipStream_t st) {
  if (g.Qs == 0 || g.extra == 0) return;
  dim3 grid((g.Qs + XROWS - 1) / XROWS, g.heads, g.batch);
  hipLaunchKernelGGL(vsa_extra_select_kernel, grid, dim3(256), 0, st, g, (const u32x4*)k, qbar, lists, counts,
                     xtok, xcnt);
  hipLaunchKernelGGL(vsa_extra_gather_kernel, dim3(g.Qs, g.heads, g.batch), dim3(256), 0, st, g,
                     (const u32x4*)k, (const u32x4*)v, xtok, xcnt, (u32x4*)kx, (u32x4*)vx);
}
