// Host launchers of the gfx950 kernels (one translation unit per step).
#pragma once

#include <hip/hip_runtime.h>

#include "vsa_internal.h"

// Geometry gather + mean pooling: qbar for every tile, kbar/vbar for video
// tiles; writes bias = 0 when the coarse mode has no log-mass bias.  With knorm
// (extra tokens), also every tile's largest key L2 norm, [batch x head][tile].
void vsa_launch_pool(const VsaGeom& g, const void* q, const void* k, const void* v, float* qbar,
                     float* kbar, float* vbar, float* bias, float* knorm, hipStream_t st);

// Mean video query per (batch, head) (log-mass anchor).
void vsa_launch_anchor(const VsaGeom& g, const float* qbar, float* anchor, hipStream_t st);

// Log-mass bias per video key tile; in the weighted mode also the weighted key / value
// summaries, written over kbar and vbar.
void vsa_launch_logmass(const VsaGeom& g, const void* k, const void* v, float* kbar, float* vbar,
                        const float* anchor, float* bias, hipStream_t st);

// Coarse branch: S = scale qbar kbar^T + b for the sparse rows against the video tiles
// (written to scores, with the per-block tau sums), the row softmax, and
// O_coarse = softmax(S) vbar, in one fused fp32-MFMA kernel.
void vsa_launch_coarse(const VsaGeom& g, const float* qbar, const float* kbar, const float* vbar,
                       const float* bias, float* scores, float* ocoarse, double* statp, float* cpart,
                       hipStream_t st);

// tau threshold mean + tau * std per (batch, head) from the partials.
void vsa_launch_tau(const VsaGeom& g, const double* statp, float* thr, hipStream_t st);

// Per sparse row list of key tiles: prefix tiles, then selected video tiles.
void vsa_launch_select(const VsaGeom& g, const float* scores, const float* thr, int* lists,
                       int* counts, hipStream_t st);

// Extra tokens per sparse row (best pooled-query scores outside the listed tiles): ids
// ascending and counts, and their K / V rows staged [batch, Qs, 64, heads, 128].
struct VsaExtraBuffers {
  float *tm1, *tm4, *thr;      // per (row, tile) maxima; per row threshold
  unsigned* mask;              // candidate tiles, [bh][tile / 32][row]
  int* ccnt;                   // candidate counts
  unsigned long long* cand;    // candidate entries, VSA_EXTRA_CAND per row
  void* qsplit;                // per row: qbar as three bf16 terms in MFMA operand order
  const float* knorm;          // per tile: largest key L2 norm (written by the pool step)
  unsigned long long* part;    // fallback: per-segment best E of each row
  int* pcnt;
  int *xtok, *xcnt;            // the extra tokens and their count per row
  void* vx;                    // staged V rows 32-63 of the extra tokens' tile
};
void vsa_launch_extra(const VsaGeom& g, const void* k, const void* v, const float* qbar, const int* lists,
                      const int* counts, const VsaExtraBuffers& x, hipStream_t st);

// Spark-Reblock mapper: M, norms and the tree levels; returns the final token list
// ([batch, heads, Vt, 64] packed token ids, leaf j = video tile j).
const int* vsa_launch_reblock(const VsaGeom& g, const void* q, const void* k, float* mpart, float* M,
                              unsigned short* mhl, float* a0, float* norms, int* list_a, int* list_b, float* pbuf,
                              float* part, float* state, hipStream_t st);
// Q, K, V, G with each head's video rows permuted onto the reblocked tiles, and back for O.
void vsa_launch_rb_permute(const VsaGeom& g, const int* tiles, const void* q, const void* k, const void* v,
                           const void* gate, void* q2, void* k2, void* v2, void* g2, hipStream_t st);
void vsa_launch_rb_unpermute(const VsaGeom& g, const int* tiles, const void* o2, void* o, hipStream_t st);

// Block-sparse fine attention + gated combine, output in packed order; a sparse row's
// extra tokens (xtok, xcnt, and their staged V rows 32-63 in vx; unused when the option is
// off) run as its first tile.
void vsa_launch_fine(const VsaGeom& g, const void* q, const void* k, const void* v, const void* gate,
                     const float* ocoarse, const int* lists, const int* counts, void* o,
                     const int* xtok, const void* vx, const int* xcnt, hipStream_t st);
