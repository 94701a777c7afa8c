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
// The exact score: z^T (64 keys x 16 rows) = K qbar^T on the bf16 MFMAs, with qbar split
// exactly into three bf16 terms hi + mid + lo, so the products are exact and only the fp32
// accumulation rounds (a plain bf16 qbar would move logits by ~2^-9 of their size).  Keys are
// ranked by these raw dot products; the positive scale s does not change the order.  A tile in
// the row's list, and the padding rows of a partial prefix tile, take no part.  The select
// runs in two passes over the keys:
// vsa_extra_tmax_kernel (pass 1, a screen): every (sparse row, tile) pair once, scored with hi
//   alone (a third of the MFMAs), keeping only M1, the row's best screening score in the tile,
//   and M4, the least of the four lane maxima (four keys of the tile score at least that).
//   One workgroup per (head, tile chunk, 128-row block), key tiles staged by buffer-to-LDS
//   loads two tiles ahead; M1 / M4 stored [bh][tile][row], one coalesced store per wave and tile.
// vsa_extra_thr_kernel: eps bounds the screen's error against the exact score per (row, tile)
//   (from |qbar - hi| and the tile's largest key norm, written by the pool step).  Per row
//   T = max(E-th largest M1 - eps, ceil(E/4)-th largest M4 - eps), read from the top 16 bits
//   of the order keys: a lower bound of the row's E-th best exact score (E tiles hold a key
//   >= the one, ceil(E/4) tiles four keys >= the other).  The row's E best keys then all lie
//   in its candidate tiles, those with M1 + eps >= T, which are recorded as bits.
// vsa_extra_score_kernel (pass 2): per (two tiles, head), the rows with a tile among their
//   candidates, 16 to an MFMA group, scored exactly; every key scoring >= its row's T is
//   appended to the row's candidate list (an atomic count gives the slot).  About E + a few
//   keys per row on the pages' workloads; the list keeps VSA_EXTRA_CAND.
// vsa_extra_select_kernel (fallback): a row whose list overflowed (heavy exact ties, say) is
//   selected by streaming every key tile with a running threshold (described at the kernel);
//   segments with no such row are skipped, so the kernel costs ~8 us when none overflowed.
// vsa_extra_gather_kernel: the exact best E of the row's candidates (or of the fallback's
//   partial lists) by (score, then lower token), ranked by token.
// Measured on the 36,096-token, 32-head workload at E = 64: pass 1 0.25 ms, threshold 0.06,
// pass 2 0.24, fallback 0.01 (1.69 ms as one streaming pass, 0.82 with an exact pass 1).
// About 75 candidate tiles per row pass the screen (65 with exact maxima).
//
// vsa_extra_gather_kernel also copies the V rows of each row's extra tokens 32..63 into a
// staging buffer [batch, Qs, 32, heads, 128] (padding rows zero), with the token stride of V
// itself: the fine kernel runs the extra tokens as its first tile, reading their K rows and
// V rows 0-31 by token id in its prologue, and these 32 V rows in its main loop like any
// tile's, by base-plus-stride addressing.
#include <type_traits>

#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

constexpr int XROWS = 64;   // streaming fallback: sparse rows per workgroup, 16 per wave
constexpr int XCAP = 128;   // candidate buffer entries per row (a tile adds at most 64)
constexpr int XSLACK = 16;  // a cut inside the stream may keep up to E + XSLACK entries

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
  // every field is wave-uniform: said so, the segment tables are read with scalar loads
  // rather than vector loads (whose waits would also wait for the tile loads)
  w.t = __builtin_amdgcn_readfirstlane(w.t);
  w.seg = __builtin_amdgcn_readfirstlane(w.seg);
  w.tin = __builtin_amdgcn_readfirstlane(w.tin);
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

// Positions a walk at tile t (prefix: its segment and index in it; video: its coordinates).
__device__ __forceinline__ void walk_seek(const VsaGeom& g, TileWalk& w, int t) {
  w.t = t;
  w.seg = w.tin = w.tw = w.th = w.tt = 0;
  if (t < g.P) {
    while (t >= g.pre_tile0[w.seg + 1]) ++w.seg;
    w.tin = t - g.pre_tile0[w.seg];
  } else {
    const int v = t - g.P;
    w.tw = v % g.tw_n;
    w.th = (v / g.tw_n) % g.th_n;
    w.tt = v / g.tw_n / g.th_n;
  }
  walk_set(g, w);
}

// The workgroup whose step range holds step x: the largest w with floor(w TS / G) <= x.
__device__ __forceinline__ int xwg_of(long long x, long long TS, int G) {
  return (int)(((x + 1) * G + TS - 1) / TS) - 1;
}

// A buffer entry holds the float score's bits over ~token.  Its 64-bit order key is larger
// for the better candidate (score order, then the lower token); an empty slot's key is 0.
__device__ __forceinline__ unsigned long long entry(float z, int tok) {
  return ((unsigned long long)__float_as_uint(z) << 32) | (unsigned)(~tok);
}
__device__ __forceinline__ unsigned long long entry_key(unsigned long long e) {
  return ((unsigned long long)order_key(__uint_as_float((unsigned)(e >> 32))) << 32) | (unsigned)e;
}

// Streaming selection (the fallback for rows whose candidate list overflowed).  One
// workgroup per range of (64-row block, tile) steps, wave w owning rows 16 w .. 16 w + 15;
// every key tile of the segment streams through LDS (two tiles in flight in registers).
// A key enters the row's LDS candidate buffer if its score is at least the row's
// threshold, a lower bound of the E-th best score seen so far (equal scores enter too: only
// the cuts order ties, by token).  When a tile's entrants would overflow a buffer the wave
// first cuts it back with a bitwise ballot search over the 64-bit keys (score order, then
// ~token) that stops as soon as a candidate keeps between E and E + 16 entries (exactly E if
// it has to go down to the token word), raising the threshold, and tests the tile's keys
// again.  Each segment leaves every row's best E in the partial lists.
__global__ __launch_bounds__(256) void vsa_extra_select_kernel(VsaGeom g, const u32x4* __restrict__ k,
                                                               const float* __restrict__ qbar,
                                                               const int* __restrict__ lists,
                                                               const int* __restrict__ counts,
                                                               const int* __restrict__ ccnt,
                                                               unsigned long long* __restrict__ xpart,
                                                               int* __restrict__ xpcnt) {
  // K tile: key row r at 256 r, 16-byte chunk c at position c ^ (r & 15)
  __shared__ __attribute__((aligned(16))) char ktile[64 * 256];
  __shared__ unsigned long long cbuf[XROWS][XCAP];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, ql = lane & 15;
  // The work is the sequence of (row block, tile) steps, row blocks in (batch, head, block)
  // order and tiles in id order; workgroup w takes steps [w TS / G, (w + 1) TS / G), so every
  // workgroup has the same share and G = 2 per CU run at once.  Its range falls into
  // segments, one per row block it touches; a segment streams its tiles like a whole row
  // block would and leaves each row's best E of them in the partial lists, which the gather
  // kernel merges.  Logical ids are dealt so that XCD x (ids L = x mod 8) takes a run of
  // consecutive ranges: the row blocks of one (batch, head), which stream the same keys,
  // share an XCD and its L2.
  const int nrb = (g.Qs + XROWS - 1) / XROWS;
  const long long TS = (long long)nrb * g.heads * g.batch * g.Tq;
  const int G = gridDim.x, L = blockIdx.x, xcd = L & 7;
  const int w = xcd * (G >> 3) + min(xcd, G & 7) + (L >> 3);
  const long long lo = (long long)w * TS / G, hi = (long long)(w + 1) * TS / G;
  const int rl = 16 * wave + ql;  // this lane's row in the workgroup
  const int E = g.extra;

  // the segment's row block and this lane's row (set per segment)
  int rb = 0, h = 0, b = 0;
  size_t bh = 0;
  int r = 0;
  bool live = false, wlive = false;
  int t1 = 0;  // the segment's tiles end here
  // B operands: qbar of row r, dims 32 ks + 8 grp .. +7, as hi / mid / lo bf16 terms
  bf16x8 qs[3][4];
  // list cursor: entry cur of this row's (ascending) list is the next listed tile; it is
  // loaded every tile, one tile ahead of its use, so every step issues the same loads
  const int* lst = lists;
  int cnt_l = 0, cur = 0, nl = 0;
  int nrow = 0;            // entries in this row's buffer (same in its four lanes)
  float thz = -INFINITY;   // the row's threshold: a lower bound of its E-th best raw score

  // Cuts workgroup row rc (n > E entries) to its entries at or above the threshold key
  // `pre` returned, keeping `kept` of them, E <= kept <= lim: the score word is found by a
  // bitwise ballot search from the top, which stops at the first candidate that keeps
  // between E and lim entries.  Run to its end the search gives the E-th best score word;
  // if ties at that score still keep more than lim, the token word is searched as well and
  // exactly E are kept.  n and lim are wave-uniform; every valid key is above 0.
  struct Cut {
    unsigned long long pre;
    int kept;
  };
  auto cut = [&](int rc, int n, int lim) -> Cut {
    n = __builtin_amdgcn_readfirstlane(n);
    lim = __builtin_amdgcn_readfirstlane(lim);
    const bool v0 = lane < n, v1 = lane + 64 < n;
    const unsigned long long r0 = v0 ? cbuf[rc][lane] : 0ull;
    const unsigned long long r1 = v1 ? cbuf[rc][lane + 64] : 0ull;
    const unsigned long long k0 = v0 ? entry_key(r0) : 0ull;
    const unsigned long long k1 = v1 ? entry_key(r1) : 0ull;
    const unsigned h0 = (unsigned)(k0 >> 32), h1 = (unsigned)(k1 >> 32);
    unsigned ph = 0u;
    int kept = n;
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned cand = ph | (1u << bit);
      const int c = __popcll(__ballot(h0 >= cand)) + __popcll(__ballot(h1 >= cand));
      if (c >= E) {
        ph = cand;
        kept = c;
        if (c <= lim) break;
      }
    }
    unsigned pl = 0u;
    if (kept > lim) {
      // ties at the E-th best score word: the token word decides, and exactly E stay
      const int need = E - (__popcll(__ballot(h0 > ph)) + __popcll(__ballot(h1 > ph)));
      const bool e0 = v0 && h0 == ph, e1 = v1 && h1 == ph;
      const unsigned l0 = (unsigned)k0, l1 = (unsigned)k1;
      for (int bit = 31; bit >= 0; --bit) {
        const unsigned cand = pl | (1u << bit);
        const int c = __popcll(__ballot(e0 && l0 >= cand)) + __popcll(__ballot(e1 && l1 >= cand));
        if (c >= need) pl = cand;
      }
      kept = E;
    }
    const unsigned long long pre = ((unsigned long long)ph << 32) | pl;
    const bool s0 = v0 && k0 >= pre, s1 = v1 && k1 >= pre;
    const unsigned long long b0 = __ballot(s0), b1 = __ballot(s1);
    // every lane has its two entries in registers before any write below
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    if (s0) cbuf[rc][lanes_below(b0)] = r0;
    if (s1) cbuf[rc][__popcll(b0) + lanes_below(b1)] = r1;
    return Cut{pre, kept};
  };

  // staging of a key tile: thread tid moves rows r = (tid >> 4) + 16 m, chunk tid & 15;
  // in a video tile row r is (dt, dh, dw) = (m, (tid >> 6) & 3, (tid >> 4) & 3)
  const int hw = g.H * g.W;
  const int fdhw = ((tid >> 6) & 3) * g.W + ((tid >> 4) & 3);
  const u32x4* kbh = k;  // this thread's 16-byte chunk of token 0 of the segment's (b, h)
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
  // one tile: stage it, refill its slot two tiles ahead, score it, admit its keys
  auto step = [&](int t, u32x4 (&slot)[4], unsigned& vmask) {
    __syncthreads();  // every wave is done with the previous tile
    stash(slot, vmask);
    __syncthreads();
    // The list entry loaded last step, then the next one.  Loads complete in issue order
    // as far as the waits can tell, so each list load is issued before the step's tile
    // refill: waiting for it next step then leaves that refill in flight.
    const bool excl = cur < cnt_l && nl == t;
    cur += excl ? 1 : 0;
    nl = lst[min(cur, g.cap - 1)];
    __builtin_amdgcn_sched_barrier(0);
    // refill two tiles ahead (past the end the last tile again: every step issues the
    // same loads, so the wait before a stash leaves the other slot's loads in flight)
    if (t + 2 < t1) walk_next(g, wf);
    fetch(wf, slot, vmask);
    __builtin_amdgcn_sched_barrier(0);

    if (!wlive) {  // a wave past the last sparse row only helps stage the tiles
      walk_next(g, wc);
      return;
    }
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

    // lane holds the raw dot products of keys 16 kb + 4 grp + i of the tile for its row
    // (e = 4 kb + i).  Ranking by them ranks by the scaled score, the scale being positive.
    const bool video = wc.video;
    const int tok0 = wc.tok0;
    const int nv = wc.nv;
    // A key enters if its score is >= the row's threshold score thz (-inf before the first
    // cut).  A key that only ties the threshold's score enters too: the cuts order equal
    // scores by token, so such an entrant costs buffer room, never the result.
    float z[16];
    unsigned ge = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      z[e] = acc[e >> 2][e & 3];
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
    // counts over the four lanes of the row (lanes ql + 16 grp)
    int c = __popc(ge);
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
        // room for this tile's entrants of the row after the cut
        const int lim = min(E + XSLACK, XCAP - __shfl(c0 + c1 + c2 + c3, rc));
        const Cut T = cut(16 * wave + rc, n, lim);
        if (ql == rc) {
          nrow = T.kept;
          const unsigned sk = (unsigned)(T.pre >> 32);  // back from the order key to the float
          thz = __uint_as_float((sk & 0x80000000u) ? (sk & 0x7fffffffu) : ~sk);
        }
      }
      // the keys again against the raised thresholds
      unsigned ge2 = 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e) ge2 |= (unsigned)(z[e] >= thz) << e;
      ge &= ge2;
      c = __popc(ge);
      row_values4(c, cr);
      c0 = cr[0];
      c1 = cr[1];
      c2 = cr[2];
      c3 = cr[3];
    }
    int at = nrow + (grp > 0 ? c0 : 0) + (grp > 1 ? c1 : 0) + (grp > 2 ? c2 : 0);
    // the admitted keys, lowest e first.  Where a lane takes several (early in the stream)
    // one step per key index e, skipping the e no lane takes ...
    if (__ballot(c > 3) != 0ull) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const bool in = (ge >> e) & 1u;
        if (__ballot(in) != 0ull) {
          if (in) cbuf[rl][at++] = entry(z[e], tok_of(e));
        }
      }
      nrow += c0 + c1 + c2 + c3;
      walk_next(g, wc);
      return;
    }
    // ... else one pass per key of the lane that takes the most, key e's score picked by a
    // select tree on e's bits
    for (unsigned f = ge; __ballot(f != 0u) != 0ull;) {
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
  for (long long pos = lo; pos < hi;) {
    // the segment: tiles [t0, t1) of row block rbg
    const int rbg = (int)(pos / g.Tq);
    const int t0 = (int)(pos - (long long)rbg * g.Tq);
    t1 = (int)min((long long)g.Tq, t0 + (hi - pos));
    const int seg = w - xwg_of((long long)rbg * g.Tq, TS, G);  // its index among the row block's
    pos += t1 - t0;
    rb = rbg % nrb;
    h = (rbg / nrb) % g.heads;
    b = rbg / nrb / g.heads;
    bh = (size_t)b * g.heads + h;
    r = rb * XROWS + rl;
    // only the rows whose candidate list overflowed; a segment without one is skipped
    live = r < g.Qs && ccnt[bh * g.Qs + r] > VSA_EXTRA_CAND;
    if (!__syncthreads_or(live)) continue;
    wlive = __ballot(live) != 0ull;
    {
      const f32x4* qp = reinterpret_cast<const f32x4*>(qbar + (bh * g.Tq + g.n_dense + (live ? r : 0)) * VSA_HEAD_DIM);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const f32x4 a = live ? qp[8 * ks + 2 * grp] : f32x4{0.f, 0.f, 0.f, 0.f};
        const f32x4 c = live ? qp[8 * ks + 2 * grp + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
        const float x[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          __bf16 hi3, mid3, lo3;
          split3(x[e], hi3, mid3, lo3);
          qs[0][ks][e] = hi3;
          qs[1][ks][e] = mid3;
          qs[2][ks][e] = lo3;
        }
      }
    }
    // the list cursor at the first listed tile >= t0 (binary search of the ascending list)
    lst = lists + (bh * g.Qs + (live ? r : 0)) * g.cap;
    cnt_l = live ? counts[bh * g.Qs + r] : 0;
    {
      int a = 0, c = cnt_l;
      while (a < c) {
        const int m = (a + c) >> 1;
        if (lst[m] < t0) a = m + 1;
        else c = m;
      }
      cur = a;
    }
    nl = lst[min(cur, g.cap - 1)];
    nrow = 0;
    thz = -INFINITY;
    kbh = k + (((size_t)b * g.N) * g.heads + h) * (VSA_HEAD_DIM / 8) + (tid & 15);
    walk_seek(g, wc, t0);
    wf = wc;
    fetch(wf, kr[0], kv[0]);
    if (t0 + 1 < t1) walk_next(g, wf);
    fetch(wf, kr[1], kv[1]);
    // both steps of the loop body unconditional: a conditional second step would make the
    // wait before the first stash drain the other slot's loads as well
    int t = t0;
    for (; t + 1 < t1; t += 2) {
      step(t, kr[0], kv[0]);
      step(t + 1, kr[1], kv[1]);
    }
    if (t < t1) step(t, kr[0], kv[0]);

    // each row's best E of the segment (exactly), into the partial lists
    if (wlive) {
      __builtin_amdgcn_s_waitcnt(0xc07f);
      for (int rc = 0; rc < 16; ++rc) {
        const int row = rb * XROWS + 16 * wave + rc;
        if (row >= g.Qs) break;
        int n = __shfl(nrow, rc);
        if (n > E) {
          cut(16 * wave + rc, n, E);  // lim = E: exactly the E best
          n = E;
          __builtin_amdgcn_s_waitcnt(0xc07f);
        }
        const size_t pr = ((size_t)rbg * g.xms + seg) * XROWS + 16 * wave + rc;
        if (lane < n) xpart[pr * VSA_MAX_EXTRA + lane] = cbuf[16 * wave + rc][lane];
        if (lane == 0) xpcnt[pr] = n;
      }
    }
  }
}

// Pass 1 of the two-pass select, a screen.  Per (sparse row, tile): M1, the row's best
// screening score among the tile's eligible keys, and M4, the least of the four lane maxima
// (each lane holds 16 of the 64 keys, so at least four keys score >= M4); both -inf for a
// tile in the row's list.  The screening score is the MFMA product with hi(qbar), the first
// bf16 term of the row's split, alone: one third of the MFMAs of the exact score.  Its error
// against the exact score is bounded per (row, tile) and the threshold kernel widens M1 and
// M4 by that bound.
// One workgroup of four waves per (batch x head, tile chunk, 128-row block): the tiles are
// cut into xs1 chunks, and the row blocks of one chunk get consecutive logical ids, dealt to
// one XCD so that they stream the same key tiles through its L2 together.  A wave scores 32
// rows, two MFMA row groups sharing every key operand it reads from LDS.  Key tiles come into
// a ring of three LDS buffers by buffer-to-LDS loads issued two tiles ahead (each wave four
// 1 KB loads per tile; padding rows of a partial prefix tile read out of range, so as zeros),
// one barrier per tile; 52 KB of LDS, three workgroups per CU.
constexpr int X1ROWS = 128;
constexpr int XNB = 3;
// 16 bytes per lane from buffer offset voff into LDS at lds + 16 lane (M0 holds the LDS base).
// Written as asm so that the compiler neither waits for it before unrelated LDS reads nor
// counts it: the kernels that use it wait for these loads themselves, and nothing else in
// them uses M0.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t rs, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rs), "s"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}
template <int N>
using IC = std::integral_constant<int, N>;
__global__ __launch_bounds__(256, 3) void vsa_extra_tmax_kernel(VsaGeom g, const char* __restrict__ kp,
                                                             const float* __restrict__ qbar,
                                                             const int* __restrict__ lists,
                                                             const int* __restrict__ counts,
                                                             float* __restrict__ tm1, float* __restrict__ tm4,
                                                             int* __restrict__ ccnt, u32x4* __restrict__ qsplit) {
  __shared__ __attribute__((aligned(16))) char kring[XNB][64 * 256];
  __shared__ unsigned xbits[X1ROWS][8];  // listed tiles of each row among the current 256
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, ql = lane & 15;
  const int nrb = (g.Qs + X1ROWS - 1) / X1ROWS;
  const int G = gridDim.x, L = blockIdx.x, xcd = L & 7;
  const int w = xcd * (G >> 3) + min(xcd, G & 7) + (L >> 3);
  const unsigned rowbytes = (unsigned)g.heads * VSA_HEAD_DIM * 2;
  const unsigned nrec = (unsigned)(g.N - 1) * rowbytes + VSA_HEAD_DIM * 2;
  const int rb = w % nrb;
  const int tch = (w / nrb) % g.xs1;  // the tile chunk
  const int bhl = w / nrb / g.xs1;
  const int h = bhl % g.heads, b = bhl / g.heads;
  const size_t bh = (size_t)b * g.heads + h;
  const int t0 = (int)((long long)tch * g.Tq / g.xs1);
  const int t1 = (int)((long long)(tch + 1) * g.Tq / g.xs1);
  // row group u of this wave: rows 32 wave + 16 u .. + 15 of the block, this lane's is + ql
  const int wr0 = rb * X1ROWS + 32 * wave;
  const int Qsp = (g.Qs + 31) & ~31;  // rows of the M1 / M4 arrays
  int r[2];
  bool live[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    r[u] = wr0 + 16 * u + ql;
    live[u] = r[u] < g.Qs;
  }
  // live row groups of the wave (wave-uniform): a group with a live row has its first row live
  const int nl = (wr0 < g.Qs) + (wr0 + 16 < g.Qs);
  bf16x8 qh[2][4];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const f32x4* qp = reinterpret_cast<const f32x4*>(qbar + (bh * g.Tq + g.n_dense + (live[u] ? r[u] : 0)) * VSA_HEAD_DIM);
    bf16x8 qs[3][4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const f32x4 a = live[u] ? qp[8 * ks + 2 * grp] : f32x4{0.f, 0.f, 0.f, 0.f};
      const f32x4 c = live[u] ? qp[8 * ks + 2 * grp + 1] : f32x4{0.f, 0.f, 0.f, 0.f};
      const float x[8] = {a[0], a[1], a[2], a[3], c[0], c[1], c[2], c[3]};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        __bf16 hi3, mid3, lo3;
        split3(x[e], hi3, mid3, lo3);
        qs[0][ks][e] = hi3;
        qs[1][ks][e] = mid3;
        qs[2][ks][e] = lo3;
      }
      qh[u][ks] = qs[0][ks];
    }
    // the row's three bf16 terms of qbar, in the lane order of the MFMA operands, for pass 2
    // (layout per row: (term, ks, grp) at 16 term + 4 ks + grp, 16 bytes each)
    if (tch == 0 && live[u]) {
      u32x4* qo = qsplit + (bh * g.Qs + r[u]) * 48 + grp;
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qo[16 * pp + 4 * ks] = __builtin_bit_cast(u32x4, qs[pp][ks]);
    }
  }
  // the listed tiles: lane (ql, grp < 2) keeps the list cursor of row group grp's row ql
  const bool lister = grp < 2 && live[grp & 1];
  const int lrow = r[grp & 1];
  const int* lst = lists + (bh * g.Qs + (lister ? lrow : 0)) * g.cap;
  const int cnt_l = lister ? counts[bh * g.Qs + lrow] : 0;
  int cur;
  {
    int a = 0, c = cnt_l;
    while (a < c) {
      const int m = (a + c) >> 1;
      if (lst[m] < t0) a = m + 1;
      else c = m;
    }
    cur = a;
  }
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kp + ((size_t)b * g.N * g.heads + h) * (VSA_HEAD_DIM * 2)), 0, (int)nrec, 0x00020000);
  // this lane's share of a tile's loads: wave w moves rows 4 w + 16 m + (lane >> 4), m = 0..3,
  // i.e. (dt, dh, dw) = (m, w, lane >> 4) of a video tile; its 16 bytes land at position
  // lane & 15 of the row, which holds chunk (lane & 15) ^ (row & 15)
  const unsigned chunk = (unsigned)((lane & 15) ^ ((4 * wave + (lane >> 4)) & 15)) * 16u;
  const unsigned vrow = (unsigned)(wave * g.W + (lane >> 4));  // (dh, dw) offset in tokens
  const unsigned plane = (unsigned)(g.H * g.W);
  auto issue = [&](const TileWalk& tw, auto bic) {
    constexpr int BI = decltype(bic)::value;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int row = 4 * wave + 16 * m + (lane >> 4);
      unsigned off;
      if (tw.video) off = (unsigned)(tw.tok0 + m * (int)plane + (int)vrow) * rowbytes + chunk;
      else off = row < tw.nv ? (unsigned)(tw.tok0 + row) * rowbytes + chunk : nrec;
      lds_dma16(rs, off, (unsigned)(size_t)(kring[BI] + 1024 * (wave + 4 * m)));
    }
  };
  // Every step issues the loads of one tile (past the chunk's end, its last tile again), so
  // the loads issued after tile t's are always the next tile's four plus the stores since.
  TileWalk wc, wf;
  walk_seek(g, wc, t0);
  wf = wc;
  issue(wf, IC<0>{});
  if (t0 + 1 < t1) walk_next(g, wf);
  issue(wf, IC<1>{});
  // one tile from ring buffer BI (a constant, so that the compiler can tell the buffer read
  // from the ones being loaded and adds no wait for the loads in flight)
  auto step = [&](int t, auto bic) {
    constexpr int BI = decltype(bic)::value;
    const int i = t - t0;
    if ((i & 255) == 0) {
      // the row's listed tiles among the next 256, as bits (by its lister lane; the wave's
      // other lanes read them after this wave's LDS writes)
      if (grp < 2) {
        unsigned* xm = xbits[32 * wave + 16 * grp + ql];
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) xm[jj] = 0u;
        while (cur < cnt_l) {
          const int x = lst[cur];
          if (x >= t + 256) break;
          atomicOr(&xm[(x - t) >> 5], 1u << ((x - t) & 31));
          ++cur;
        }
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    }
    // Wait for this wave's loads of tile t: issued after them are the next tile's four and,
    // in a live wave, the one M1 / M4 store of each tile since (one tile at i = 1, two
    // later).  A plain barrier would make the compiler wait for every load in flight first;
    // the bare barrier between two compiler fences does not.
    if (i == 0 || nl == 0) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
    else if (i == 1) asm volatile("s_waitcnt vmcnt(5)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(6)" ::: "memory");
    __builtin_amdgcn_s_barrier();  // tile t is in LDS; every wave is done with tile t - 1
    asm volatile("" ::: "memory");
    if (t + 2 < t1) walk_next(g, wf);
    issue(wf, IC<(BI + 2) % XNB>{});  // into the buffer tile t - 1 held
    if (nl > 0) {
      const char* kt = kring[BI];
      f32x4 acc[2][4];
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc[u][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        bf16x8 a[4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          a[kb] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + 256 * (16 * kb + ql) + 16 * ((4 * ks + grp) ^ ql)));
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            acc[u][kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kb], qh[u][ks], acc[u][kb], 0, 0, 0);
      }
      float v1[2], v4[2];  // M1 and M4 of this lane's row in each row group
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        float z[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) z[e] = acc[u][e >> 2][e & 3];
        if (!wc.video) {  // padding keys of a partial prefix tile take no part
          const int nv = wc.nv;
#pragma unroll
          for (int e = 0; e < 16; ++e)
            if (16 * (e >> 2) + 4 * grp + (e & 3) >= nv) z[e] = -INFINITY;
        }
        float mx = z[0];
#pragma unroll
        for (int e = 1; e < 16; ++e) mx = fmaxf(mx, z[e]);
        const bool excl = (xbits[32 * wave + 16 * u + ql][(i & 255) >> 5] >> (i & 31)) & 1u;
        if (!live[u] || excl) mx = -INFINITY;
        int rv[4];
        row_values4(__float_as_int(mx), rv);
        const float a0 = __int_as_float(rv[0]), a1 = __int_as_float(rv[1]);
        const float a2 = __int_as_float(rv[2]), a3 = __int_as_float(rv[3]);
        v1[u] = fmaxf(fmaxf(a0, a1), fmaxf(a2, a3));
        v4[u] = fminf(fminf(a0, a1), fminf(a2, a3));
        if (t == 0 && grp == 0 && live[u]) ccnt[bh * g.Qs + r[u]] = 0;  // the row's candidate count
      }
      // One store for the wave's 32 rows: lane group grp writes M1 (grp even) or M4 (odd) of
      // row group grp / 2, 16 consecutive floats of the tile's row of [bh][tile][padded row]
      // (rows past Qs land in the padding).
      const int uu = grp >> 1;
      const float val = (grp & 1) ? (uu ? v4[1] : v4[0]) : (uu ? v1[1] : v1[0]);
      float* dst = (grp & 1) ? tm4 : tm1;
      dst[(bh * g.Tq + t) * (size_t)Qsp + wr0 + 16 * uu + ql] = val;
    }
    walk_next(g, wc);
  };
  int t = t0;
  for (; t + 2 < t1; t += 3) {
    step(t, IC<0>{});
    step(t + 1, IC<1>{});
    step(t + 2, IC<2>{});
  }
  if (t < t1) step(t, IC<0>{});
  if (t + 1 < t1) step(t + 1, IC<1>{});
  // the loads issued past the chunk's end land before the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// The screen's error per (row, tile).  Pass 1 scores a key k with hi, the first bf16 term of
// the row's qbar; pass 2 and the fallback with all three terms, whose sum is qbar exactly.
// The products of bf16 values are exact in fp32, so the two scores differ by r . k, with
// r = qbar - hi, plus the fp32 rounding of the sums: recursive summation of n terms errs by at
// most about n 2^-24 of their absolute sum, here 3 x 128 and 128 terms (and the MFMA
// accumulator adds), under 2^-14 |qbar| |k| together.  With |r . k| <= |r| |k|
// (Cauchy-Schwarz) and |k| at most the tile's largest key norm:
//   |exact - screen| <= eps = (|r| (1 + 2^-10) + |qbar| 2^-13) knorm(tile) + 1e-35,
// the factor and the doubled 2^-13 covering the rounding of eps itself and of the sums below,
// the constant any flushed denormal products.
// Threshold kernel: with lo1 = M1 - eps and lo4 = M4 - eps (each tile then holds a key, or
// four keys, whose exact score is >= these), T = max(E-th largest lo1, ceil(E/4)-th largest
// lo4) bounds the row's E-th best exact score from below, and a tile can hold a key scoring
// >= T only if M1 + eps >= T: those are the candidates.
// One workgroup of R waves per R consecutive rows, a wave per row.  The workgroup stages
// each chunk of 64 tiles of its rows' M1 and M4 ([bh][tile][padded row]: R consecutive floats
// per tile) through LDS, so that the loads are coalesced; each wave then holds its row's keys,
// one tile per lane and chunk, in registers (R shrinks as the tile count grows).
template <int NC, int R>
__global__ __launch_bounds__(64 * R) void vsa_extra_thr_kernel(VsaGeom g, const float* __restrict__ qbar,
                                                               const float* __restrict__ knorm,
                                                               const float* __restrict__ tm1,
                                                               const float* __restrict__ tm4,
                                                               float* __restrict__ xthr,
                                                               unsigned* __restrict__ xmask) {
  __shared__ float sm[2][64][R + 1];  // one chunk: [M1 / M4][tile][row], padded against bank conflicts
  // row blocks in order within an XCD: the blocks that share a 128-byte line of M1 / M4 are
  // read through one L2
  const int G = gridDim.x, L = blockIdx.x, xcd = L & 7;
  const int w = xcd * (G >> 3) + min(xcd, G & 7) + (L >> 3);
  const int nrb = (g.Qs + R - 1) / R;
  const int s0 = (w % nrb) * R;
  const size_t bh = w / nrb;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int s = s0 + wave;  // this wave's row
  const bool live = s < g.Qs;
  const int Tq = g.Tq, E = g.extra, E4 = (g.extra + 3) / 4;
  const int nc = (Tq + 63) / 64;
  const size_t Qsp = (g.Qs + 31) & ~31;
  const float* m1b = tm1 + bh * Tq * Qsp + s0;  // tile t, row s0 + i at [t Qsp + i]
  const float* m4b = tm4 + bh * Tq * Qsp + s0;
  const float* kn = knorm + bh * (size_t)Tq;
  // the row's error scale: eps(tile) = es knorm(tile) + 1e-35
  float es = 0.f;
  if (live) {
    const float* qr = qbar + (bh * g.Tq + g.n_dense + s) * VSA_HEAD_DIM;
    const float x0 = qr[lane], x1 = qr[lane + 64];
    const float r0 = x0 - (float)(__bf16)x0, r1 = x1 - (float)(__bf16)x1;  // as split3 rounds
    const float rn = sqrtf(wave_sum(r0 * r0 + r1 * r1)), qn = sqrtf(wave_sum(x0 * x0 + x1 * x1));
    es = rn * 1.0009765625f + qn * 0x1p-13f;
  }
  // keys of lo1 = M1 - eps, lo4 = M4 - eps and hi1 = M1 + eps; 0: absent (every present key
  // is above 0)
  unsigned k1[NC], k4[NC], kh[NC];
  const int tl = tid / R, rr = tid % R;  // this thread's element of a chunk
  // every chunk's loads in flight at once (from clamped addresses, so that no lane branches)
  const bool rin = s0 + rr < g.Qs;
  const int rc = rin ? rr : 0;
  float la[NC], lc[NC], lk[NC];
#pragma unroll
  for (int j = 0; j < NC; ++j)
    if (j < nc) {
      const size_t o = (size_t)min(64 * j + tl, Tq - 1) * Qsp + rc;
      la[j] = m1b[o];
      lc[j] = m4b[o];
      lk[j] = kn[min(64 * j + lane, Tq - 1)];
    }
#pragma unroll
  for (int j = 0; j < NC; ++j) {
    k1[j] = k4[j] = kh[j] = 0u;
    if (j < nc) {
      const bool in = rin && 64 * j + tl < Tq;
      __syncthreads();  // the last chunk has been read
      sm[0][tl][rr] = in ? la[j] : -INFINITY;
      sm[1][tl][rr] = in ? lc[j] : -INFINITY;
      __syncthreads();
      const int tt = 64 * j + lane;
      const float m1 = sm[0][lane][wave], m4 = sm[1][lane][wave];
      const float e = tt < Tq ? fmaf(es, lk[j], 1e-35f) : 0.f;
      if (m1 != -INFINITY) {
        k1[j] = order_key(m1 - e);
        kh[j] = order_key(m1 + e);
      }
      if (m4 != -INFINITY) k4[j] = order_key(m4 - e);
    }
  }
  if (!live) return;
  auto counts = [&](unsigned c1, unsigned c4, int& n1, int& n4) {
    n1 = 0;
    n4 = 0;
#pragma unroll
    for (int j = 0; j < NC; ++j)
      if (j < nc) {
        n1 += __popcll(__ballot(k1[j] >= c1));
        n4 += __popcll(__ballot(k4[j] >= c4));
      }
  };
  int h1, h4;
  counts(1u, 1u, h1, h4);
  // The top 16 bits of the keys only: the threshold then sits at most one step of the 16-bit
  // prefix (2^-7 of its value) below the exact order statistic, still a lower bound.
  unsigned p1 = 0u, p4 = 0u;
  for (int bit = 31; bit >= 16; --bit) {
    int n1, n4;
    counts(p1 | (1u << bit), p4 | (1u << bit), n1, n4);
    if (n1 >= E) p1 |= 1u << bit;
    if (n4 >= E4) p4 |= 1u << bit;
  }
  const unsigned kt = max(h1 >= E ? p1 : 0u, h4 >= E4 ? p4 : 0u);
  float T = -INFINITY;
  if (kt != 0u) T = __uint_as_float((kt & 0x80000000u) ? (kt & 0x7fffffffu) : ~kt);
  if (lane == 0) xthr[bh * g.Qs + s] = T;
  const int nw = (Tq + 31) / 32;
#pragma unroll
  for (int j = 0; j < NC; ++j)
    if (j < nc) {
      const unsigned long long m = __ballot(kh[j] != 0u && kh[j] >= kt);
      if (lane == 0) {
        xmask[(bh * nw + 2 * j) * g.Qs + s] = (unsigned)m;
        if (2 * j + 1 < nw) xmask[(bh * nw + 2 * j + 1) * g.Qs + s] = (unsigned)(m >> 32);
      }
    }
}

// Pass 2: one workgroup of four waves per (TPW consecutive tiles, batch x head).  The tiles'
// keys come into LDS by buffer-to-LDS loads (padding rows of a partial prefix tile read out of
// range, so as zeros) while the rows that have each tile among their candidates are gathered
// from the masks (in any order, through LDS counts); the waves then take the (tile, 16-row
// group) items in turn and score them against the tile's keys on the MFMAs with the rows'
// exact three-term split, and a key scoring >= its row's T is appended to the row's candidate
// list (its slot from an atomic count; past VSA_EXTRA_CAND the count keeps growing but nothing
// is written).
template <int TPW>
__global__ __launch_bounds__(256, 4) void vsa_extra_score_kernel(VsaGeom g, const char* __restrict__ kp,
                                                              const float* __restrict__ xthr,
                                                              const unsigned* __restrict__ xmask,
                                                              int* __restrict__ ccnt,
                                                              unsigned long long* __restrict__ xcand,
                                                              const u32x4* __restrict__ qsplit) {
  __shared__ __attribute__((aligned(16))) char ktile[TPW][64 * 256];
  __shared__ int nrows_s[TPW];
  extern __shared__ int rowlist[];  // TPW x Qs entries
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, ql = lane & 15;
  // XCD-aware: each XCD takes a contiguous range of (head, tile pair) items, head-major, so
  // a head's split qbar rows are read through few L2s
  const int ntp = (g.Tq + TPW - 1) / TPW;
  const int G = gridDim.x, L = blockIdx.x, xcd = L & 7;
  const int w = xcd * (G >> 3) + min(xcd, G & 7) + (L >> 3);
  const size_t bh = w / ntp;
  const int b = (int)(bh / g.heads), h = (int)(bh % g.heads);
  const int tb = (w % ntp) * TPW;       // the first tile
  const int nt = min(TPW, g.Tq - tb);   // tiles of this workgroup
  const int nw = (g.Tq + 31) / 32;
  const unsigned rowbytes = (unsigned)g.heads * VSA_HEAD_DIM * 2;
  const unsigned nrec = (unsigned)(g.N - 1) * rowbytes + VSA_HEAD_DIM * 2;
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(kp + ((size_t)b * g.N * g.heads + h) * (VSA_HEAD_DIM * 2)), 0, (int)nrec, 0x00020000);
  // the keys, as in pass 1: wave w moves rows 4 w + 16 m + (lane >> 4) of each tile
  const unsigned chunk = (unsigned)((lane & 15) ^ ((4 * wave + (lane >> 4)) & 15)) * 16u;
  const unsigned vrow = (unsigned)(wave * g.W + (lane >> 4));
  const unsigned plane = (unsigned)(g.H * g.W);
  TileWalk tw[TPW];
  walk_seek(g, tw[0], tb);
#pragma unroll
  for (int i = 1; i < TPW; ++i) {
    tw[i] = tw[i - 1];
    if (i < nt) walk_next(g, tw[i]);
  }
#pragma unroll
  for (int i = 0; i < TPW; ++i)
    if (i < nt) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int row = 4 * wave + 16 * m + (lane >> 4);
        unsigned off;
        if (tw[i].video) off = (unsigned)(tw[i].tok0 + m * (int)plane + (int)vrow) * rowbytes + chunk;
        else off = row < tw[i].nv ? (unsigned)(tw[i].tok0 + row) * rowbytes + chunk : nrec;
        lds_dma16(rs, off, (unsigned)(size_t)(ktile[i] + 1024 * (wave + 4 * m)));
      }
    }
  if (tid < TPW) nrows_s[tid] = 0;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < TPW; ++i)
    if (i < nt) {
      const int t = tb + i;
      const unsigned* mk = xmask + (bh * nw + (t >> 5)) * g.Qs;
      for (int base = 64 * wave; base < g.Qs; base += 256) {
        const int s = base + lane;
        const bool in = s < g.Qs && ((mk[s] >> (t & 31)) & 1u);
        const unsigned long long m = __ballot(in);
        int at = 0;
        if (m != 0ull && lane == 0) at = atomicAdd(&nrows_s[i], __popcll(m));
        at = __shfl(at, 0);
        if (in) rowlist[i * g.Qs + at + lanes_below(m)] = s;
      }
    }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's key loads
  __syncthreads();
  int n[TPW], ng = 0;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    n[i] = nrows_s[i];
    ng += (n[i] + 15) / 16;
  }
  for (int gi = wave; gi < ng; gi += 4) {
    // the item's tile i and row group gg (per-tile values picked by selects, not by index)
    int i = 0, gg = gi, cnt = n[0], tok0 = tw[0].tok0, nv = tw[0].nv, video = tw[0].video;
#pragma unroll
    for (int ii = 1; ii < TPW; ++ii)
      if (i == ii - 1 && gg >= (cnt + 15) / 16) {
        gg -= (cnt + 15) / 16;
        i = ii;
        cnt = n[ii];
        tok0 = tw[ii].tok0;
        nv = tw[ii].nv;
        video = tw[ii].video;
      }
    const int idx = 16 * gg + ql;
    const bool live = idx < cnt;
    const int s = rowlist[i * g.Qs + (live ? idx : 0)];
    bf16x8 qs[3][4];
    {
      const u32x4* qi = qsplit + (bh * g.Qs + s) * 48 + grp;
#pragma unroll
      for (int pp = 0; pp < 3; ++pp)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) qs[pp][ks] = as_bf16x8(qi[16 * pp + 4 * ks]);
    }
    const float T = live ? xthr[bh * g.Qs + s] : INFINITY;
    const char* kt = ktile[0] + i * (64 * 256);
    f32x4 acc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) acc[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bf16x8 a[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        a[kb] = as_bf16x8(*reinterpret_cast<const u32x4*>(kt + 256 * (16 * kb + ql) + 16 * ((4 * ks + grp) ^ ql)));
#pragma unroll
      for (int p = 2; p >= 0; --p)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kb], qs[p][ks], acc[kb], 0, 0, 0);
    }
    float z[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) z[e] = acc[e >> 2][e & 3];
    if (!video) {  // padding keys get a NaN, which never passes
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (16 * (e >> 2) + 4 * grp + (e & 3) >= nv) z[e] = __builtin_nanf("");
    }
    // key e of this lane: row 16 (e >> 2) + 4 grp + (e & 3) of the tile, whose token is
    // tokl + (e >> 2) kstep + (e & 3)
    const int tokl = tok0 + (video ? grp * g.W : 4 * grp);
    const int kstep = video ? g.H * g.W : 16;
    unsigned ge = 0u;
#pragma unroll
    for (int e = 0; e < 16; ++e) ge |= (unsigned)(z[e] >= T) << e;
    const int c = __popc(ge);
    int slot = 0;
    if (c > 0) slot = atomicAdd(&ccnt[bh * g.Qs + s], c);
    unsigned long long* dst = xcand + (bh * g.Qs + s) * (size_t)VSA_EXTRA_CAND;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const bool in = (ge >> e) & 1u;
      if (__ballot(in) != 0ull) {
        if (in) {
          if (slot < VSA_EXTRA_CAND) dst[slot] = entry(z[e], tokl + (e >> 2) * kstep + (e & 3));
          ++slot;
        }
      }
    }
  }
}

// The keep-th largest of n unique 64-bit order keys in LDS (keep <= n): the high words by a
// bitwise ballot search, then, only where several keys share the boundary's high word, the
// low words among those.  One wave.
__device__ unsigned long long kth_key(const unsigned long long* keys, int n, int keep, int lane) {
  auto count = [&](unsigned ph, unsigned pl, int mode) {  // 0: hi >= ph; 1: hi > ph; 2: hi == ph (and lo >= pl)
    int c = 0;
    for (int j = 0; j < n; j += 64) {
      const unsigned long long x = j + lane < n ? keys[j + lane] : 0ull;
      const unsigned xh = (unsigned)(x >> 32), xl = (unsigned)x;
      const bool in = j + lane < n &&
                      (mode == 0 ? xh >= ph : mode == 1 ? xh > ph : (xh == ph && xl >= pl));
      c += __popcll(__ballot(in));
    }
    return c;
  };
  unsigned ph = 0u;
  for (int bit = 31; bit >= 0; --bit) {
    const unsigned cand = ph | (1u << bit);
    if (count(cand, 0u, 0) >= keep) ph = cand;
  }
  const int need = keep - count(ph, 0u, 1);
  unsigned pl = 0u;
  if (count(ph, 0u, 2) > need) {
    for (int bit = 31; bit >= 0; --bit) {
      const unsigned cand = pl | (1u << bit);
      if (count(ph, cand, 2) >= need) pl = cand;
    }
  }
  return ((unsigned long long)ph << 32) | pl;
}

// One workgroup per (sparse row, head, batch).  Wave 0 picks the row's extra tokens: the best
// E of its candidate list by the 64-bit order key (keys are unique: the tokens differ), or,
// for a row whose list overflowed, of the union of the fallback's segment lists.  It ranks them
// by token and writes the row's extra tokens and count.  Then thread tid copies 64 bytes of
// extra row tid >> 2 (zeros past the count) of K and of V.
__global__ __launch_bounds__(128) void vsa_extra_gather_kernel(VsaGeom g, const u32x4* __restrict__ v,
                                                               const int* __restrict__ ccnt,
                                                               const unsigned long long* __restrict__ xcand,
                                                               const unsigned long long* __restrict__ xpart,
                                                               const int* __restrict__ xpcnt,
                                                               int* __restrict__ xtok,
                                                               int* __restrict__ xcnt,
                                                               u32x4* __restrict__ vx) {
  __shared__ unsigned long long ckey[VSA_EXTRA_CAND];
  __shared__ unsigned long long mbuf[VSA_MAX_EXTRA];
  __shared__ int mtok[VSA_MAX_EXTRA];
  __shared__ int stok[VSA_MAX_EXTRA];
  __shared__ int mcnt;
  const int s = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const size_t ro = ((size_t)b * g.heads + h) * g.Qs + s;
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int E = g.extra;
    const int cc = ccnt[ro];
    int n;
    unsigned long long e0;  // the lane's kept entry (its low word is ~token)
    if (cc <= VSA_EXTRA_CAND) {
      const unsigned long long* cand = xcand + ro * VSA_EXTRA_CAND;
      for (int j = lane; j < cc; j += 64) ckey[j] = entry_key(cand[j]);
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): one wave, its writes are in LDS
      n = min(E, cc);
      const unsigned long long pre = n > 0 ? kth_key(ckey, cc, n, lane) : ~0ull;
      int at = 0;
      for (int j = 0; j < cc; j += 64) {
        const unsigned long long x = j + lane < cc ? ckey[j + lane] : 0ull;
        const bool sel = j + lane < cc && x >= pre;
        const unsigned long long m = __ballot(sel);
        if (sel) mbuf[at + lanes_below(m)] = x;
        at += __popcll(m);
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      e0 = lane < n ? mbuf[lane] : 0ull;
    } else {
      // the fallback's segment lists: the top E of their union, pairwise
      const int nrb = (g.Qs + XROWS - 1) / XROWS;
      const long long TS = (long long)nrb * g.heads * g.batch * g.Tq;
      const int G = g.xg;
      const int rbg = (b * g.heads + h) * nrb + s / XROWS, rw = s % XROWS;
      const int w0 = xwg_of((long long)rbg * g.Tq, TS, G);
      const int w1 = xwg_of((long long)(rbg + 1) * g.Tq - 1, TS, G);
      size_t pr = (size_t)rbg * g.xms * XROWS + rw;
      n = xpcnt[pr];
      e0 = lane < n ? xpart[pr * VSA_MAX_EXTRA + lane] : 0ull;
      for (int sg = 1; sg <= w1 - w0; ++sg) {
        pr = ((size_t)rbg * g.xms + sg) * XROWS + rw;
        const int n1 = xpcnt[pr];
        const unsigned long long e1 = lane < n1 ? xpart[pr * VSA_MAX_EXTRA + lane] : 0ull;
        ckey[lane] = lane < n ? entry_key(e0) : 0ull;
        ckey[64 + lane] = lane < n1 ? entry_key(e1) : 0ull;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        // both lists padded to 64 with empty keys (0, below every real key)
        const int keep = min(E, n + n1);
        const unsigned long long pre = keep > 0 ? kth_key(ckey, 128, keep, lane) : ~0ull;
        const unsigned long long k0 = ckey[lane], k1 = ckey[64 + lane];
        const bool s0 = lane < n && k0 >= pre, s1 = lane < n1 && k1 >= pre;
        const unsigned long long b0 = __ballot(s0), b1 = __ballot(s1);
        if (s0) mbuf[lanes_below(b0)] = e0;
        if (s1) mbuf[__popcll(b0) + lanes_below(b1)] = e1;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        n = keep;
        e0 = lane < n ? mbuf[lane] : 0ull;
        __builtin_amdgcn_s_waitcnt(0xc07f);  // every lane has read before the next writes
      }
    }
  // rank by token and write ascending
    const int mytok = lane < n ? ~(int)(unsigned)e0 : 0;
    mtok[lane] = mytok;
    __builtin_amdgcn_s_waitcnt(0xc07f);
    int rank = 0;
    for (int e = 0; e < n; ++e) rank += mtok[e] < mytok ? 1 : 0;
    if (lane < n) {
      xtok[ro * VSA_MAX_EXTRA + rank] = mytok;
      stok[rank] = mytok;
    }
    if (lane == 0) {
      xcnt[ro] = n;
      mcnt = n;
    }
  }
  __syncthreads();
  // the V rows of tokens 32..63 (the fine kernel reads the rest straight from K and V):
  // row 32 + e of the tile to row e of the [batch, Qs, 32, heads, 128] staging, head h
  const int e = threadIdx.x >> 2, part = threadIdx.x & 3;
  const int n = mcnt;
  const size_t dst = ((((size_t)b * g.Qs + s) * VSA_XSTAGE + e) * g.heads + h) * 16 + 4 * part;
  u32x4 va[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) va[i] = u32x4{0u, 0u, 0u, 0u};
  if (VSA_MAX_EXTRA - VSA_XSTAGE + e < n) {
    // (a token id outside the sequence cannot come from the select kernel; clamped all the
    // same, so that a read never leaves the (b, h) plane)
    const int tok = min(max(stok[VSA_MAX_EXTRA - VSA_XSTAGE + e], 0), g.N - 1);
    const long long src = row_offset(g, b, tok, h) / 8 + 4 * part;
#pragma unroll
    for (int i = 0; i < 4; ++i) va[i] = v[src + i];
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) vx[dst + i] = va[i];
}

}  // namespace

void vsa_launch_extra(const VsaGeom& g, const void* k, const void* v, const float* qbar, const int* lists,
                      const int* counts, const VsaExtraBuffers& x, hipStream_t st) {
  if (g.Qs == 0 || g.extra == 0) return;
  const int BH = g.heads * g.batch;
  hipLaunchKernelGGL(vsa_extra_tmax_kernel, dim3((g.Qs + X1ROWS - 1) / X1ROWS * BH * g.xs1), dim3(256), 0, st, g,
                     (const char*)k, qbar, lists, counts, x.tm1, x.tm4, x.ccnt, (u32x4*)x.qsplit);
  {
    const int nc = (g.Tq + 63) / 64;
    auto thr = nc <= 16 ? vsa_extra_thr_kernel<16, 4> : nc <= 32 ? vsa_extra_thr_kernel<32, 8>
             : nc <= 64 ? vsa_extra_thr_kernel<64, 4> : vsa_extra_thr_kernel<128, 2>;
    const int R = nc <= 16 ? 4 : nc <= 32 ? 8 : nc <= 64 ? 4 : 2;
    hipLaunchKernelGGL(thr, dim3((g.Qs + R - 1) / R * BH), dim3(64 * R), 0, st, g, qbar, x.knorm,
                       (const float*)x.tm1, (const float*)x.tm4, x.thr, x.mask);
  }
  {
    constexpr int TPW = 2;
    hipLaunchKernelGGL(vsa_extra_score_kernel<TPW>, dim3((g.Tq + TPW - 1) / TPW * BH), dim3(256),
                       4 * TPW * g.Qs, st, g, (const char*)k, (const float*)x.thr, (const unsigned*)x.mask,
                       x.ccnt, x.cand, (const u32x4*)x.qsplit);
  }
  hipLaunchKernelGGL(vsa_extra_select_kernel, dim3(g.xg), dim3(256), 0, st, g, (const u32x4*)k, qbar, lists, counts,
                     (const int*)x.ccnt, x.part, x.pcnt);
  hipLaunchKernelGGL(vsa_extra_gather_kernel, dim3(g.Qs, g.heads, g.batch), dim3(128), 0, st, g,
                     (const u32x4*)v, (const int*)x.ccnt, (const unsigned long long*)x.cand,
                     (const unsigned long long*)x.part, (const int*)x.pcnt, x.xtok, x.xcnt, (u32x4*)x.vx);
}
