// Internal definitions shared by the host plan and the gfx950 kernels.
#pragma once

#include <cstddef>
#include <cstdint>

#include "vsa.h"

#define VSA_MAX_PREFIX_SEGS 16
#define VSA_MAX_VIDEO_TILES 4096  // also the most candidate key tiles (selector: 64 per lane)
#define VSA_MAX_LIST 2048        // key tiles in one sparse row's list (staged in LDS by the fine kernel)
#define VSA_HEAD_DIM 128
#define VSA_TILE_TOKENS 64
#define VSA_COARSE_ROWS 64   // sparse rows per workgroup of the coarse kernel
#define VSA_MAX_EXTRA 64     // extra tokens per sparse row (one tile)
#define VSA_XSTAGE 32        // of their V rows, those past the first 32 are staged

// Geometry and options of one plan, passed to every kernel by value.  Tile ids:
// prefix tiles [0, P) in packed order, video tiles [P, P + Vt) raster (tt, th, tw).
struct VsaGeom {
  int32_t n_pre_segs;
  int32_t pre_start[VSA_MAX_PREFIX_SEGS];  // packed start token of each prefix segment
  int32_t pre_len[VSA_MAX_PREFIX_SEGS];
  int32_t pre_tile0[VSA_MAX_PREFIX_SEGS + 1];  // first tile id of each prefix segment; [n] = P
  int32_t vstart;                          // packed start of the video span
  int32_t T, H, W;                         // video latent grid
  int32_t tw_n, th_n;                      // W/4, H/4
  int32_t P, Vt, Tq;
  int32_t npin;                            // tiles listed in every sparse row: P, or 0 with sink off
  int32_t kc0, Kc;                         // candidate key tiles [kc0, kc0 + Kc): the video tiles,
                                           // or every tile with sink off
  int32_t N, heads, batch;
  int32_t n_dense;                         // dense query tiles per (batch, head): 0 or P
  int32_t Qs;                              // sparse query tiles per (batch, head): Tq - n_dense
  int32_t cap;                             // list capacity per sparse row
  int32_t k;                               // TOPK keep count
  int32_t extra;                           // extra tokens per sparse row (0: off)
  int32_t sink, select, coarse;
  float tau;
  float scale;                             // softmax scale 1/sqrt(128)
  int32_t coarse_blocks;                   // workgroups per (batch, head) of the score kernel:
                                           // row blocks x csplit
  int32_t csplit;                          // candidate-tile slices per row block (1: no merge)
  int32_t cchunks;                         // 64-tile chunks per slice
  int32_t reblock;                         // 1: Spark-Reblock video tiles per (batch, head)
  int32_t rb_nsplit;                       // tile ranges per (batch, head) of the key-moment sums
  int32_t xg;                              // extra-token select workgroups (equal step ranges)
  int32_t xms;                             // most segments (workgroups) a 64-row block spans
  int32_t xs1;                             // extra-token pass 1: tile chunks per row block
};

// The extra-token select runs this many workgroups at most: two per CU of the 256-CU part,
// each holding 80 KB of LDS.
constexpr int VSA_EXTRA_WGS = 512;
// Candidate entries kept per sparse row by the two-pass extra-token select; a row with more
// takes the streaming fallback.
constexpr int VSA_EXTRA_CAND = 1024;

struct VsaLayout {        // byte offsets into the workspace
  size_t qbar, kbar, vbar, bias, anchor, scores, ocoarse, thr, lists, counts, statp;
  size_t xtok, xcnt, vx;      // extra tokens: ids, counts, staged V rows 32-63 of their tile
  size_t xpart, xpcnt;        // extra tokens: per-segment best E of each row, and counts
  size_t xtm1, xtm4, xthr, xmask, xccnt, xcand;  // two-pass select: maxima, thresholds, candidates
  size_t xqsplit;                                // two-pass select: qbar as three bf16 terms
  size_t xknorm;                                 // two-pass select: largest key norm per tile
  size_t cpart;               // coarse partials per (row, slice): max, sum, 2 pad, O[128]
  // Spark-Reblock: key-moment partials and M (fp32, bf16 hi/lo), video-token norms, token
  // lists (ping-pong; `tiles` is the final one), projections, pass partials, node states,
  // and the permuted Q, K, V, G and the permuted output
  size_t rb_mpart, rb_m, rb_mhl, rb_a0, rb_norms, rb_list_a, rb_list_b, rb_tiles, rb_pbuf, rb_part, rb_state;
  size_t rb_q, rb_k, rb_v, rb_g, rb_o;
  size_t total;
};

struct vsa_plan {
  VsaGeom g;
  VsaLayout ws;
  vsa_options opts;
  float keep;
  int64_t n_tokens;
};

// Spark-Reblock tree shape (defined in k_reblock.hip): levels = ceil(log2 Vt); pass
// workgroups per node at a level.
int vsa_reblock_levels(int Vt);
int vsa_reblock_chunks(int Vt, int level);
constexpr int VSA_RB_STATE = 260;  // floats of a node state: mu[128], a[128], mu.a, pad

// kernel launch sequence (defined in vsa_forward.hip)
struct vsa_timer;
int vsa_launch_forward(const vsa_plan* plan, const void* q, const void* k, const void* v,
                       const void* g, void* o, void* workspace, void* stream, vsa_timer* timer);
