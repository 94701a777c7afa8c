// Device-side helpers for the gfx950 kernels: vector types, bf16 unpacking and
// the tile -> packed-token map of the geometry mapper.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>

#include "vsa_internal.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// bf16 pair packed in a 32-bit word -> the two floats (exact).
__device__ __forceinline__ float bf16lo(unsigned int x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float bf16hi(unsigned int x) { return __uint_as_float(x & 0xffff0000u); }

// Segment of prefix tile t (t < P).  Uniform loop over at most 16 segments.
__device__ __forceinline__ int prefix_seg(const VsaGeom& g, int t) {
  int s = 0;
#pragma unroll
  for (int i = 1; i < VSA_MAX_PREFIX_SEGS; ++i)
    if (i < g.n_pre_segs && t >= g.pre_tile0[i]) s = i;
  return s;
}

// Number of valid tokens of tile t (64 except the last tile of a prefix segment).
__device__ __forceinline__ int tile_valid(const VsaGeom& g, int t) {
  if (t >= g.P) return VSA_TILE_TOKENS;
  const int s = prefix_seg(g, t);
  const int rem = g.pre_len[s] - (t - g.pre_tile0[s]) * VSA_TILE_TOKENS;
  return rem < VSA_TILE_TOKENS ? rem : VSA_TILE_TOKENS;
}

// Packed token of row r (0..63) of tile t, or -1 for a padding row.
// Prefix tile: 64 consecutive tokens of its segment.  Video tile j = t - P:
// (tt, th, tw) raster over the (T/4, H/4, W/4) grid, row r = (dt, dh, dw)
// raster, token vstart + ((4tt+dt) H + 4th+dh) W + 4tw+dw.
__device__ __forceinline__ int video_token(const VsaGeom& g, int t, int r) {
  const int j = t - g.P;
  const int tw = j % g.tw_n;
  const int rest = j / g.tw_n;
  const int th = rest % g.th_n;
  const int tt = rest / g.th_n;
  const int dt = r >> 4, dh = (r >> 2) & 3, dw = r & 3;
  return g.vstart + ((4 * tt + dt) * g.H + 4 * th + dh) * g.W + 4 * tw + dw;
}
__device__ __forceinline__ int tile_token(const VsaGeom& g, int t, int r) {
  if (t < g.P) {
    const int s = prefix_seg(g, t);
    const int off = (t - g.pre_tile0[s]) * VSA_TILE_TOKENS + r;
    return off < g.pre_len[s] ? g.pre_start[s] + off : -1;
  }
  return video_token(g, t, r);
}

// Element offset of (batch b, token tok, head h, dim 0) in a [B, N, heads, 128] tensor.
__device__ __forceinline__ long long row_offset(const VsaGeom& g, int b, int tok, int h) {
  return (((long long)b * g.N + tok) * g.heads + h) * VSA_HEAD_DIM;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x = fmaxf(x, __shfl_xor(x, m));
  return x;
}

// Reductions over the four lanes l, l + 16, l + 32, l + 48 (rows of the wave) with the
// row-swap VALU permutes, which do not go through the LDS queue.
__device__ __forceinline__ float group_max(float m) {
  const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  const u32x2 a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const u32x2 b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

