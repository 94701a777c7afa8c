// Spark-Reblock geometry mapper: an adaptive partition of each (batch, head)'s video tokens
// into 64-token tiles, in place of the fixed 4x4x4 cubes.
//
// "Spark-H3: atencion dispersa por bloques acelera MiniMax-H3 en ComfyUI", "Que cambia
// Spark-Attn", Spark-Reblock item: two queries are similar when their attention-score
// patterns over the keys are, measured by a cosine distance in the metric of the opposite
// side's second moment; a hierarchical splitter divides groups until each leaf holds one
// block, in O(N log N).  Its "Flujos de trabajo" fix reblock_layout=q_reuse_k: the key
// tiles reuse the query partition.  Reading (the page gives no split rule):
//   M = mean over the video keys of k k^T; psi = q / sqrt(q^T M q) (the M-cosine of two
//   queries is the cosine of their score patterns K q, K q').  A group of m tiles (64 m
//   tokens, m >= 2) is split along its principal axis in the metric M: three power steps
//   z <- C M z from z = 1 (C the group's centred psi covariance, z at M-norm 1 before each
//   step), projections p = psi^T M z / |z|_M; the 64 floor(m/2) tokens lowest by
//   (p, token id) form the left child (tiles [t0, t0 + floor(m/2))), the rest the right.
//   The tree's shape depends on Vt only: at level L the node n covers the tiles reached by
//   the bits of n from the root; ceil(log2 Vt) levels leave every node with one tile.
//   Each node's tokens stay in ascending token order (stable partitions), so leaf j holds
//   its 64 tokens ascending.
//
// Kernels (all per (batch, head), launched by vsa_launch_reblock):
//   moment      k k^T over ranges of video tiles with bf16 MFMAs (products exact, fp32 sums)
//   reduce      the ranges summed in a fixed order; M, its bf16 hi/lo split, and the first
//               direction a0 = M 1 / |1|_M (the same for every node: z starts at 1)
//   norm        |q|_M per video token with bf16 MFMAs against the hi/lo split of M (staged
//               in LDS, 512 tokens per workgroup); the level-0 token list (tokens ascending)
//   per level:  pass(first) finish  2 x [pass(power) finish]  pass(projection)  split
//     pass      chunks of up to 512 tokens of one node.  first: the sums of psi and of
//               (psi.a0) psi (then C a0 = those / n - mu (mu.a0), since the centred psi sum
//               to zero); power: the sums of (psi.a - mu.a)(psi - mu); projection: psi.a
//     finish    per node: the chunk sums added in chunk order, then z, a = M z / |z|_M
//               and mu.a
//     split     per node: the k-th smallest projection by an MSB radix search over
//               order-preserving keys, then a stable partition (ties to the lower token)
//   permute     Q, K, V, G with each head's video rows reordered so that fixed tile j of
//               the video grid holds leaf j (row r = the leaf's r-th token): the rest of the
//               forward then runs unchanged on the reblocked tiles
//   unpermute   the output rows scattered back to their tokens
#include "vsa_device.h"
#include "vsa_kernels.h"

namespace {

constexpr int RB_STEPS = 3;       // power steps per split
constexpr int RB_STATE = VSA_RB_STATE;  // per node: mu[128], a[128], mu.a, 3 pad

__device__ __forceinline__ unsigned short bf16_rne(float x) {
  const unsigned u = __float_as_uint(x);
  return (unsigned short)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Tile range [t0, t0 + m) of node `node` at `level` (m = 0: no node there).
__device__ __forceinline__ void node_range(int Vt, int level, int node, int& t0, int& m) {
  t0 = 0;
  m = Vt;
  for (int bit = level - 1; bit >= 0; --bit) {
    const int ml = m >> 1;
    if ((node >> bit) & 1) {
      t0 += ml;
      m -= ml;
    } else {
      m = ml;
    }
  }
}

// Order-preserving unsigned key of a float (no NaN reaches here).
__device__ __forceinline__ unsigned fkey(float x) {
  const unsigned u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ void unpack8(const u32x4 w, float (&x)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16lo(w[i]);
    x[2 * i + 1] = bf16hi(w[i]);
  }
}

// Sum over the 16 lanes of a 16-lane row (lanes 16 r .. 16 r + 15), result in every lane.
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
  for (int m = 8; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// ---------------------------------------------------------------- second moment of K
// Workgroup (s, bh): video tiles [Vt s / nsplit, Vt (s + 1) / nsplit).  Per 32 tokens K is
// staged transposed in LDS (dim-major); the 128 x 128 sum is 8 x 8 blocks of 16 x 16, wave w
// owning block rows 2w, 2w + 1.  MFMA 16x16x32: A[m][t] = K[t][16 br + m] and
// B[t][n] = K[t][16 bc + n] are both "8 consecutive tokens of one dim" per lane.
__global__ __launch_bounds__(256) void vsa_rb_moment_kernel(VsaGeom g, const unsigned short* __restrict__ k,
                                                            float* __restrict__ mpart, int nsplit) {
  __shared__ __attribute__((aligned(16))) unsigned short kt[128][40];  // 32 tokens + pad per dim
  const int bh = blockIdx.x, s = blockIdx.y;  // (batch, head) fastest, as in the pass kernel
  const int b = bh / g.heads, h = bh - b * g.heads;
  const int j0 = (int)((long long)g.Vt * s / nsplit), j1 = (int)((long long)g.Vt * (s + 1) / nsplit);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, ql = lane & 15;
  const size_t ts = (size_t)g.heads * VSA_HEAD_DIM;
  const unsigned short* kb = k + ((size_t)b * g.N * g.heads + h) * VSA_HEAD_DIM;
  f32x4 acc[2][8];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[r][c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int tk = tid >> 3, d0 = 16 * (tid & 7);
  u32x4 n0 = u32x4{0u, 0u, 0u, 0u}, n1 = n0;
  if (j1 > j0) {
    const unsigned short* row = kb + (size_t)(g.vstart + 64 * j0 + tk) * ts + d0;
    n0 = *reinterpret_cast<const u32x4*>(row);
    n1 = *reinterpret_cast<const u32x4*>(row + 8);
  }
  for (int t = 64 * j0; t < 64 * j1; t += 32) {
    const u32x4 w0 = n0, w1 = n1;
    if (t + 32 < 64 * j1) {  // the next chunk's rows, in flight during this chunk's MFMAs
      const unsigned short* row = kb + (size_t)(g.vstart + t + 32 + tk) * ts + d0;
      n0 = *reinterpret_cast<const u32x4*>(row);
      n1 = *reinterpret_cast<const u32x4*>(row + 8);
    }
    __syncthreads();  // the previous chunk's operand reads are done
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      kt[d0 + 2 * e][tk] = (unsigned short)(w0[e] & 0xffffu);
      kt[d0 + 2 * e + 1][tk] = (unsigned short)(w0[e] >> 16);
      kt[d0 + 8 + 2 * e][tk] = (unsigned short)(w1[e] & 0xffffu);
      kt[d0 + 8 + 2 * e + 1][tk] = (unsigned short)(w1[e] >> 16);
    }
    __syncthreads();
    bf16x8 A[2], B[8];
#pragma unroll
    for (int r = 0; r < 2; ++r) A[r] = *reinterpret_cast<const bf16x8*>(&kt[16 * (2 * wave + r) + ql][8 * grp]);
#pragma unroll
    for (int c = 0; c < 8; ++c) B[c] = *reinterpret_cast<const bf16x8*>(&kt[16 * c + ql][8 * grp]);
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[r][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[r], B[c], acc[r][c], 0, 0, 0);
  }
  // accumulator layout: lane (grp, ql) holds C[4 grp + i][ql] of each 16 x 16 block
  float* out = mpart + ((size_t)bh * nsplit + s) * (VSA_HEAD_DIM * VSA_HEAD_DIM);
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        out[(16 * (2 * wave + r) + 4 * grp + i) * VSA_HEAD_DIM + 16 * c + ql] = acc[r][c][i];
}

// M = (sum of the ranges, in range order) / Nv, and its split M = hi + lo into two bf16
// matrices (hi = M rounded to bf16, lo = the remainder rounded).  Workgroup (x, bh): rows
// 8 x .. 8 x + 7 of M; the workgroup of row block 0 also leaves nothing else to do.
__global__ __launch_bounds__(256) void vsa_rb_moment_reduce_kernel(VsaGeom g, const float* __restrict__ mpart,
                                                                   int nsplit, float* __restrict__ M,
                                                                   unsigned short* __restrict__ mhl) {
  const int bh = blockIdx.y;
  constexpr int DD = VSA_HEAD_DIM * VSA_HEAD_DIM;
  const float inv = 1.0f / (float)(VSA_TILE_TOKENS * g.Vt);
  for (int r = 0; r < 4; ++r) {
    const int e = blockIdx.x * 1024 + r * 256 + threadIdx.x;
    float s = 0.f;
    for (int i = 0; i < nsplit; ++i) s += mpart[((size_t)bh * nsplit + i) * DD + e];
    s *= inv;
    M[(size_t)bh * DD + e] = s;
    const unsigned short hi = bf16_rne(s);
    mhl[((size_t)bh * 2) * DD + e] = hi;
    mhl[((size_t)bh * 2 + 1) * DD + e] = bf16_rne(s - __uint_as_float((unsigned)hi << 16));
  }
}

// a0 = M 1 / sqrt(1^T M 1) per (b, h) (0 if that is 0): the first power step's direction.
__global__ __launch_bounds__(VSA_HEAD_DIM) void vsa_rb_a0_kernel(const float* __restrict__ M, float* __restrict__ a0) {
  __shared__ float red[2];
  const int bh = blockIdx.x, d = threadIdx.x;
  const float* Mr = M + (size_t)bh * VSA_HEAD_DIM * VSA_HEAD_DIM + (size_t)d * VSA_HEAD_DIM;
  float av = 0.f;
  for (int e = 0; e < VSA_HEAD_DIM; ++e) av += Mr[e];
  const float za = wave_sum(av);
  if ((d & 63) == 0) red[d >> 6] = za;
  __syncthreads();
  const float zat = red[0] + red[1];
  a0[(size_t)bh * VSA_HEAD_DIM + d] = zat > 0.f ? av / sqrtf(zat) : 0.f;
}

// |q|_M = sqrt(q^T M q) of each video token, and the level-0 token list (video tokens
// ascending).  Workgroup (x, bh): video offsets 512 x .. 512 x + 511, 16 per wave step.
// M's hi and lo parts are staged in LDS once per workgroup.  U = Q M with MFMA 16x16x32
// (A = 16 tokens x 32 dims, contiguous in global memory; B = rows of M by symmetry), then
// q . u per token from the Q rows kept in LDS.
constexpr int RB_NORM_TOKENS = 512;

__global__ __launch_bounds__(256) void vsa_rb_norm_kernel(VsaGeom g, const unsigned short* __restrict__ q,
                                                          const unsigned short* __restrict__ mhl,
                                                          float* __restrict__ norms, int* __restrict__ list0) {
  __shared__ __attribute__((aligned(16))) unsigned short ms[2][VSA_HEAD_DIM][VSA_HEAD_DIM + 8];
  __shared__ __attribute__((aligned(16))) unsigned short qs[4][16][VSA_HEAD_DIM + 8];
  const int bh = blockIdx.x;  // (batch, head) fastest, as in the pass kernel
  const int b = bh / g.heads, h = bh - b * g.heads;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, grp = lane >> 4, ql = lane & 15;
  const int Nv = VSA_TILE_TOKENS * g.Vt;
  const unsigned short* Mh = mhl + (size_t)bh * 2 * VSA_HEAD_DIM * VSA_HEAD_DIM;
  for (int i = tid; i < 2 * VSA_HEAD_DIM * 16; i += 256) {  // 16-byte pieces of M hi, lo
    const int part = i >> 11, row = (i >> 4) & 127, c = i & 15;
    *reinterpret_cast<u32x4*>(&ms[part][row][8 * c]) =
        *reinterpret_cast<const u32x4*>(Mh + (size_t)part * VSA_HEAD_DIM * VSA_HEAD_DIM + row * VSA_HEAD_DIM + 8 * c);
  }
  const int base = RB_NORM_TOKENS * blockIdx.y;
  for (int i = tid; i < RB_NORM_TOKENS; i += 256)
    if (base + i < Nv) list0[(size_t)bh * Nv + base + i] = g.vstart + base + i;
  __syncthreads();
  const size_t ts = (size_t)g.heads * VSA_HEAD_DIM;
  const unsigned short* qh = q + ((size_t)b * g.N * g.heads + h) * VSA_HEAD_DIM;
  u32x4 nq[4];
  {
    const int off0 = base + 16 * wave;
    if (off0 < Nv) {
      const unsigned short* qrow = qh + (size_t)(g.vstart + off0 + ql) * ts;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) nq[ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * grp);
    }
  }
  for (int step = 0; step < RB_NORM_TOKENS / 64; ++step) {
    const int off0 = base + 64 * step + 16 * wave;  // the wave's 16 tokens (wave-uniform)
    if (off0 >= Nv) break;
    bf16x8 A[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      A[ks] = __builtin_bit_cast(bf16x8, nq[ks]);
      *reinterpret_cast<u32x4*>(&qs[wave][ql][32 * ks + 8 * grp]) = nq[ks];
    }
    if (step + 1 < RB_NORM_TOKENS / 64 && off0 + 64 < Nv) {  // the next step's rows, in flight
      const unsigned short* qrow = qh + (size_t)(g.vstart + off0 + 64 + ql) * ts;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) nq[ks] = *reinterpret_cast<const u32x4*>(qrow + 32 * ks + 8 * grp);
    }
    f32x4 acc[8];
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int part = 0; part < 2; ++part) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(&ms[part][16 * nb + ql][32 * ks + 8 * grp]);
          acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A[ks], __builtin_bit_cast(bf16x8, w), acc[nb], 0, 0, 0);
        }
    }
    // the wave's own Q rows in qs: written above and read below by this wave (LDS keeps a
    // wave's accesses in order; the barrier keeps the compiler from moving them)
    __builtin_amdgcn_wave_barrier();
    // lane (grp, ql) holds U[token 4 grp + i][dim 16 nb + ql]
    float part[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      part[i] = 0.f;
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        part[i] += __uint_as_float((unsigned)qs[wave][4 * grp + i][16 * nb + ql] << 16) * acc[nb][i];
      part[i] = row16_sum(part[i]);
    }
    if (ql == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) norms[(size_t)bh * Nv + off0 + 4 * grp + i] = sqrtf(fmaxf(part[i], 0.f));
    }
    __builtin_amdgcn_wave_barrier();  // qs is rewritten by the next step
  }
}

// ---------------------------------------------------------------- per-level passes
// MODE 0 (first power step): sums of psi and of (psi.a0) psi; 1 (later power steps): sums of
// (psi.a - mu.a)(psi - mu); 2: projections psi.a to pbuf.  Workgroup (x, bh): node x / cpn,
// positions [chunk c, chunk (c + 1)) of it (c = x % cpn; chunk = the level's largest node
// split evenly into cpn whole tiles, at most RB_CH tokens).  16 lanes per token (8 dims each),
// 16 tokens per step, eight steps' loads in flight.
constexpr int RB_CH = 512;
constexpr int RB_PART = 2 * VSA_HEAD_DIM;  // floats per chunk partial
constexpr int RB_FNB = 8;                   // most nodes per finish workgroup

template <int MODE>
__global__ __launch_bounds__(256) void vsa_rb_pass_kernel(VsaGeom g, const unsigned short* __restrict__ q,
                                                          const float* __restrict__ norms,
                                                          const int* __restrict__ list,
                                                          const float* __restrict__ state,
                                                          const float* __restrict__ a0,
                                                          float* __restrict__ part, float* __restrict__ pbuf,
                                                          int level, int cpn, int chunk) {
  __shared__ float red[16][RB_PART];
  // (batch, head) runs fastest in the grid, so the workgroups in flight read the rows of one
  // token range for every head (neighbouring 256-byte pieces of the same token rows) rather
  // than one head's rows, 8 KB apart
  const int bh = blockIdx.x, item = blockIdx.y;
  const int b = bh / g.heads, h = bh - b * g.heads;
  const int node = item / cpn, c = item - node * cpn;
  int t0, m;
  node_range(g.Vt, level, node, t0, m);
  const int Nv = VSA_TILE_TOKENS * g.Vt;
  const int n = VSA_TILE_TOKENS * m;
  const int lo = c * chunk, hi = min(n, lo + chunk);
  const int tid = threadIdx.x, l16 = tid & 15, slot = tid >> 4;
  float* pp = part + ((size_t)bh * gridDim.y + item) * RB_PART;
  if (m < 2) return;  // no split there: the finish kernel reads no partial of such a node
  if (lo >= hi) {       // an empty chunk of a node that splits: its partial sums are zero
    if (MODE != 2)
      for (int i = tid; i < RB_PART; i += 256) pp[i] = 0.f;
    return;
  }
  const float* st = state + ((size_t)bh * (1 << level) + node) * RB_STATE;
  float a[8], mu[8], mua = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = MODE == 0 ? a0[(size_t)bh * VSA_HEAD_DIM + 8 * l16 + e] : st[VSA_HEAD_DIM + 8 * l16 + e];
    mu[e] = MODE == 1 ? st[8 * l16 + e] : 0.f;
  }
  if (MODE == 1) mua = st[2 * VSA_HEAD_DIM];
  const size_t ts = (size_t)g.heads * VSA_HEAD_DIM;
  const unsigned short* qb = q + ((size_t)b * g.N * g.heads + h) * VSA_HEAD_DIM + 8 * l16;
  const int* lst = list + (size_t)bh * Nv + VSA_TILE_TOKENS * t0;
  const float* nrm = norms + (size_t)bh * Nv - g.vstart;
  float acc[8], acc2[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = acc2[e] = 0.f;
  constexpr int U = 8;
  for (int i0 = lo + slot; i0 < hi; i0 += 16 * U) {
    int tok[U];
    u32x4 w[U];
    float nv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int i = i0 + 16 * u;
      // list entries are video tokens; the clamp only keeps every address inside the tensors
      tok[u] = i < hi ? min(max(lst[i], g.vstart), g.vstart + Nv - 1) : -1;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tok[u] >= 0) {
        w[u] = *reinterpret_cast<const u32x4*>(qb + (size_t)tok[u] * ts);
        nv[u] = nrm[tok[u]];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (tok[u] < 0) continue;
      float x[8];
      unpack8(w[u], x);
      const float inv = nv[u] > 0.f ? 1.0f / nv[u] : 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= inv;
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d = fmaf(x[e], a[e], d);
      d = row16_sum(d);
      if (MODE == 0) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          acc[e] += x[e];
          acc2[e] = fmaf(d, x[e], acc2[e]);
        }
      } else if (MODE == 1) {
        const float cc = d - mua;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = fmaf(cc, x[e] - mu[e], acc[e]);
      } else if (l16 == 0) {
        pbuf[(size_t)bh * Nv + VSA_TILE_TOKENS * t0 + i0 + 16 * u] = d;
      }
    }
  }
  if (MODE == 2) return;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    red[slot][8 * l16 + e] = acc[e];
    red[slot][VSA_HEAD_DIM + 8 * l16 + e] = acc2[e];
  }
  __syncthreads();
  {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) s += red[i][tid];
    pp[tid] = s;
  }
}

// Per node (128 threads, one per dim; NB nodes of one (batch, head) per workgroup, so that
// each thread's row of M is read once for all of them).  The chunk sums added in chunk
// order and divided by n; after the first pass mu = sum psi / n and z = C a0 = sum (psi.a0)
// psi / n - mu (mu.a0); after a later pass z = sum / n.  Then a = M z / |z|_M (0 if
// |z|_M = 0) and mu . a go to the node state.  A node's arithmetic, and its order, does not
// depend on the other nodes of its workgroup.
template <int NB>
__global__ __launch_bounds__(VSA_HEAD_DIM) void vsa_rb_finish_kernel(VsaGeom g, const float* __restrict__ M,
                                                                     const float* __restrict__ a0,
                                                                     const float* __restrict__ part,
                                                                     float* __restrict__ state, int level,
                                                                     int cpn, int first) {
  __shared__ float zs[NB][VSA_HEAD_DIM];
  __shared__ float red[NB][3][2];
  const int bh = blockIdx.y;
  const int d = threadIdx.x, wave = d >> 6;
  const int nodes = 1 << level;
  const int n0 = blockIdx.x * NB;
  const float a0d = first ? a0[(size_t)bh * VSA_HEAD_DIM + d] : 0.f;
  float mu[NB], z[NB], v2s[NB], inv_n[NB];
  bool live[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int node = n0 + i;
    int t0 = 0, m = 0;
    if (node < nodes) node_range(g.Vt, level, node, t0, m);
    live[i] = m >= 2;
    mu[i] = z[i] = v2s[i] = 0.f;
    inv_n[i] = live[i] ? 1.0f / (float)(VSA_TILE_TOKENS * m) : 0.f;
    if (!live[i]) continue;
    const float* pp = part + ((size_t)bh * nodes * cpn + (size_t)node * cpn) * RB_PART;
    float v = 0.f, v2 = 0.f;
    for (int c = 0; c < cpn; ++c) {
      v += pp[(size_t)c * RB_PART + d];
      if (first) v2 += pp[(size_t)c * RB_PART + VSA_HEAD_DIM + d];
    }
    if (first) {
      mu[i] = v * inv_n[i];
      v2s[i] = v2;
    } else {
      mu[i] = state[((size_t)bh * nodes + node) * RB_STATE + d];
      z[i] = v * inv_n[i];
    }
  }
  if (first) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const float ma0 = wave_sum(mu[i] * a0d);
      if ((d & 63) == 0) red[i][0][wave] = ma0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if (!live[i]) continue;
      z[i] = v2s[i] * inv_n[i] - mu[i] * (red[i][0][0] + red[i][0][1]);
      state[((size_t)bh * nodes + n0 + i) * RB_STATE + d] = mu[i];
    }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) zs[i][d] = z[i];
  __syncthreads();
  float av[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) av[i] = 0.f;
  const float* Mr = M + (size_t)bh * VSA_HEAD_DIM * VSA_HEAD_DIM + (size_t)d * VSA_HEAD_DIM;
#pragma unroll 4
  for (int e = 0; e < VSA_HEAD_DIM; e += 4) {
    const f32x4 mr = *reinterpret_cast<const f32x4*>(Mr + e);
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      av[i] = fmaf(mr[0], zs[i][e], av[i]);
      av[i] = fmaf(mr[1], zs[i][e + 1], av[i]);
      av[i] = fmaf(mr[2], zs[i][e + 2], av[i]);
      av[i] = fmaf(mr[3], zs[i][e + 3], av[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const float za = wave_sum(z[i] * av[i]);
    if ((d & 63) == 0) red[i][1][wave] = za;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const float zat = red[i][1][0] + red[i][1][1];
    const float sc = zat > 0.f ? 1.0f / sqrtf(zat) : 0.f;
    av[i] *= sc;
    const float ma = wave_sum(mu[i] * av[i]);
    if ((d & 63) == 0) red[i][2][wave] = ma;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    if (!live[i]) continue;
    float* st = state + ((size_t)bh * nodes + n0 + i) * RB_STATE;
    st[VSA_HEAD_DIM + d] = av[i];
    if (d == 0) st[2 * VSA_HEAD_DIM] = red[i][2][0] + red[i][2][1];
  }
}

// Per node: the split.  k = 64 floor(m/2); the k-th smallest key T by a four-round 8-bit MSB
// radix search, need = the number of keys equal to T among the k smallest; then a stable
// partition in position order (positions are ascending tokens): left = keys below T and the
// first `need` keys equal to T.
template <int BS>
__global__ __launch_bounds__(BS) void vsa_rb_split_kernel(VsaGeom g, const float* __restrict__ pbuf,
                                                            const int* __restrict__ src, int* __restrict__ dst,
                                                            int level) {
  __shared__ unsigned hist[256];
  __shared__ unsigned s_sel[2];
  __shared__ unsigned wsum[2][BS / 64];
  const int bh = blockIdx.y, node = blockIdx.x;
  int t0, m;
  node_range(g.Vt, level, node, t0, m);
  if (m == 0) return;
  const int Nv = VSA_TILE_TOKENS * g.Vt;
  const size_t base = (size_t)bh * Nv + VSA_TILE_TOKENS * t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (m == 1) {
    if (tid < VSA_TILE_TOKENS) dst[base + tid] = src[base + tid];
    return;
  }
  const int n = VSA_TILE_TOKENS * m;
  const unsigned k = (unsigned)(VSA_TILE_TOKENS * (m >> 1));
  const float* pb = pbuf + base;
  unsigned prefix = 0u, mask = 0u, kk = k;
  for (int round = 0; round < 4; ++round) {
    const int shift = 24 - 8 * round;
    for (int i = tid; i < 256; i += BS) hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += BS) {
      const unsigned key = fkey(pb[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns bins 4 l .. 4 l + 3; inclusive scan over lanes, then the first bin whose
      // running count reaches kk
      unsigned hv[4], run = 0u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        hv[i] = hist[4 * lane + i];
        run += hv[i];
      }
      unsigned incl = run;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned y = __shfl_up(incl, o);
        if (lane >= o) incl += y;
      }
      const unsigned excl = incl - run;
      const unsigned long long hit = __ballot(incl >= kk);
      const int owner = __ffsll((long long)hit) - 1;
      if (lane == owner) {
        unsigned cum = excl;
        int bin = 4 * lane;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (cum + hv[i] >= kk) {
            bin = 4 * lane + i;
            break;
          }
          cum += hv[i];
        }
        s_sel[0] = prefix | ((unsigned)bin << shift);
        s_sel[1] = kk - cum;
      }
    }
    __syncthreads();
    prefix = s_sel[0];
    kk = s_sel[1];
    mask |= 0xFFu << shift;
    __syncthreads();
  }
  const unsigned T = prefix;
  const unsigned need = kk;  // keys equal to T that go left (the first ones in position order)
  // stable partition, BS positions per step
  unsigned eq_before = 0u, left_before = 0u;
  for (int i0 = 0; i0 < n; i0 += BS) {
    const int i = i0 + tid;
    const bool valid = i < n;
    const unsigned key = valid ? fkey(pb[i]) : 0xFFFFFFFFu;
    const bool eq = valid && key == T;
    const unsigned long long eb = __ballot(eq);
    const unsigned eq_in_wave = __builtin_amdgcn_mbcnt_hi((unsigned)(eb >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)eb, 0u));
    if (lane == 0) wsum[0][wave] = (unsigned)__popcll(eb);
    __syncthreads();
    unsigned eq_rank = eq_before + eq_in_wave;
    unsigned eq_tot = 0u;
    for (int w2 = 0; w2 < BS / 64; ++w2) {
      const unsigned cnt = wsum[0][w2];
      if (w2 < wave) eq_rank += cnt;
      eq_tot += cnt;
    }
    const bool left = valid && (key < T || (eq && eq_rank < need));
    const unsigned long long lb = __ballot(left);
    const unsigned l_in_wave = __builtin_amdgcn_mbcnt_hi((unsigned)(lb >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)lb, 0u));
    if (lane == 0) wsum[1][wave] = (unsigned)__popcll(lb);
    __syncthreads();
    unsigned lrank = left_before + l_in_wave;
    unsigned l_tot = 0u;
    for (int w2 = 0; w2 < BS / 64; ++w2) {
      const unsigned cnt = wsum[1][w2];
      if (w2 < wave) lrank += cnt;
      l_tot += cnt;
    }
    if (valid) {
      const unsigned di = left ? lrank : k + ((unsigned)i - lrank);
      if (di < (unsigned)n) dst[base + di] = src[base + i];  // always true for a correct count
    }
    eq_before += eq_tot;
    left_before += l_tot;
    __syncthreads();  // wsum is rewritten by the next step
  }
}

// ---------------------------------------------------------------- permutation of the inputs
// Source token of packed position p for head bh: p itself outside the video span; inside it,
// row r of fixed tile j (p's cube and its raster place in it) maps to leaf j's r-th token.
__device__ __forceinline__ int rb_source(const VsaGeom& g, const int* __restrict__ tiles, int bh, int p) {
  const int o = p - g.vstart;
  if (o < 0 || o >= VSA_TILE_TOKENS * g.Vt) return p;
  const int hw = g.H * g.W;
  const int t = o / hw, rem = o - t * hw;
  const int hh = rem / g.W, ww = rem - hh * g.W;
  const int j = ((t >> 2) * g.th_n + (hh >> 2)) * g.tw_n + (ww >> 2);
  const int r = ((t & 3) * 4 + (hh & 3)) * 4 + (ww & 3);
  const int t2 = tiles[(size_t)bh * VSA_TILE_TOKENS * g.Vt + VSA_TILE_TOKENS * j + r];
  return min(max(t2, 0), g.N - 1);  // entries are tokens; the clamp only bounds the address
}

// Q', K', V' (and G' when given) at packed position p = the inputs at rb_source(p); 16 bytes
// per thread, 16 threads per (batch, token, head) row.
__global__ __launch_bounds__(256) void vsa_rb_permute_kernel(VsaGeom g, const int* __restrict__ tiles,
                                                             const u32x4* __restrict__ q, const u32x4* __restrict__ k,
                                                             const u32x4* __restrict__ v, const u32x4* __restrict__ gate,
                                                             u32x4* __restrict__ q2, u32x4* __restrict__ k2,
                                                             u32x4* __restrict__ v2, u32x4* __restrict__ g2) {
  const long long total = (long long)g.batch * g.N * g.heads * 16;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
    const int c = (int)(idx & 15);
    const long long row = idx >> 4;
    const int h = (int)(row % g.heads);
    const long long bp = row / g.heads;
    const int p = (int)(bp % g.N), b = (int)(bp / g.N);
    const int src = rb_source(g, tiles, b * g.heads + h, p);
    const long long so = (((long long)b * g.N + src) * g.heads + h) * 16 + c;
    q2[idx] = q[so];
    k2[idx] = k[so];
    v2[idx] = v[so];
    if (gate != nullptr) g2[idx] = gate[so];
  }
}

// O at rb_source(p) = O' at packed position p.
__global__ __launch_bounds__(256) void vsa_rb_unpermute_kernel(VsaGeom g, const int* __restrict__ tiles,
                                                               const u32x4* __restrict__ o2, u32x4* __restrict__ o) {
  const long long total = (long long)g.batch * g.N * g.heads * 16;
  for (long long idx = (long long)blockIdx.x * 256 + threadIdx.x; idx < total; idx += (long long)gridDim.x * 256) {
    const int c = (int)(idx & 15);
    const long long row = idx >> 4;
    const int h = (int)(row % g.heads);
    const long long bp = row / g.heads;
    const int p = (int)(bp % g.N), b = (int)(bp / g.N);
    const int dst = rb_source(g, tiles, b * g.heads + h, p);
    o[(((long long)b * g.N + dst) * g.heads + h) * 16 + c] = o2[idx];
  }
}

}  // namespace

int vsa_reblock_levels(int Vt) {
  int d = 0;
  while ((1 << d) < Vt) ++d;
  return d;
}

// Tokens per pass workgroup at a level: the largest node's tiles split evenly over the
// level's cpn chunks (at most RB_CH tokens each), so that no chunk is a small remainder.
int vsa_reblock_chunk_tokens(int Vt, int level) {
  const int maxm = (Vt + (1 << level) - 1) >> level;
  const int cpn = vsa_reblock_chunks(Vt, level);
  return VSA_TILE_TOKENS * ((maxm + cpn - 1) / cpn);
}

int vsa_reblock_chunks(int Vt, int level) {
  const int maxm = (Vt + (1 << level) - 1) >> level;
  return std::max(1, (VSA_TILE_TOKENS * maxm + RB_CH - 1) / RB_CH);
}

const int* vsa_launch_reblock(const VsaGeom& g, const void* q, const void* k, float* mpart, float* M,
                              unsigned short* mhl, float* a0, float* norms, int* list_a, int* list_b, float* pbuf,
                              float* part, float* state, hipStream_t st) {
  const int BH = g.batch * g.heads;
  const int nsplit = g.rb_nsplit;
  const int Nv = VSA_TILE_TOKENS * g.Vt;
  const unsigned short* qs = (const unsigned short*)q;
  hipLaunchKernelGGL(vsa_rb_moment_kernel, dim3(BH, nsplit), dim3(256), 0, st, g, (const unsigned short*)k, mpart,
                     nsplit);
  hipLaunchKernelGGL(vsa_rb_moment_reduce_kernel, dim3(VSA_HEAD_DIM * VSA_HEAD_DIM / 1024, BH), dim3(256), 0, st, g,
                     mpart, nsplit, M, mhl);
  hipLaunchKernelGGL(vsa_rb_a0_kernel, dim3(BH), dim3(VSA_HEAD_DIM), 0, st, (const float*)M, a0);
  hipLaunchKernelGGL(vsa_rb_norm_kernel, dim3(BH, (Nv + RB_NORM_TOKENS - 1) / RB_NORM_TOKENS), dim3(256), 0, st, g,
                     qs, mhl, norms, list_a);
  int* src = list_a;
  int* dst = list_b;
  const int levels = vsa_reblock_levels(g.Vt);
  for (int L = 0; L < levels; ++L) {
    const int cpn = vsa_reblock_chunks(g.Vt, L);
    const int chunk = vsa_reblock_chunk_tokens(g.Vt, L);
    const dim3 pgrid(BH, (1 << L) * cpn), ngrid(1 << L, BH), fgrid(((1 << L) + RB_FNB - 1) / RB_FNB, BH);
    // finish: min(RB_FNB, nodes) nodes per workgroup
    auto finish = [&](int first) {
      if (L == 0)
        hipLaunchKernelGGL(vsa_rb_finish_kernel<1>, fgrid, dim3(VSA_HEAD_DIM), 0, st, g, M, a0, part, state, L, cpn,
                           first);
      else if (L == 1)
        hipLaunchKernelGGL(vsa_rb_finish_kernel<2>, fgrid, dim3(VSA_HEAD_DIM), 0, st, g, M, a0, part, state, L, cpn,
                           first);
      else if (L == 2)
        hipLaunchKernelGGL(vsa_rb_finish_kernel<4>, fgrid, dim3(VSA_HEAD_DIM), 0, st, g, M, a0, part, state, L, cpn,
                           first);
      else
        hipLaunchKernelGGL(vsa_rb_finish_kernel<RB_FNB>, fgrid, dim3(VSA_HEAD_DIM), 0, st, g, M, a0, part, state, L,
                           cpn, first);
    };
    // power step 1 (z from 1: the direction a0 is the head's), steps 2 .. RB_STEPS
    hipLaunchKernelGGL(vsa_rb_pass_kernel<0>, pgrid, dim3(256), 0, st, g, qs, norms, src, state, a0, part, pbuf, L,
                       cpn, chunk);
    finish(1);
    for (int s = 1; s < RB_STEPS; ++s) {
      hipLaunchKernelGGL(vsa_rb_pass_kernel<1>, pgrid, dim3(256), 0, st, g, qs, norms, src, state, a0, part, pbuf, L,
                         cpn, chunk);
      finish(0);
    }
    hipLaunchKernelGGL(vsa_rb_pass_kernel<2>, pgrid, dim3(256), 0, st, g, qs, norms, src, state, a0, part, pbuf, L,
                       cpn, chunk);
    // the split's workgroup size: the level's largest node, rounded up to 256, 512 or 1024
    // tokens (the result does not depend on it)
    const int nmax = VSA_TILE_TOKENS * ((g.Vt + (1 << L) - 1) >> L);
    if (nmax <= 256)
      hipLaunchKernelGGL(vsa_rb_split_kernel<256>, ngrid, dim3(256), 0, st, g, pbuf, src, dst, L);
    else if (nmax <= 512)
      hipLaunchKernelGGL(vsa_rb_split_kernel<512>, ngrid, dim3(512), 0, st, g, pbuf, src, dst, L);
    else
      hipLaunchKernelGGL(vsa_rb_split_kernel<1024>, ngrid, dim3(1024), 0, st, g, pbuf, src, dst, L);
    int* t = src;
    src = dst;
    dst = t;
  }
  return src;  // the final token list: leaf j at positions 64 j .. 64 j + 63 of each (b, h)
}

void vsa_launch_rb_permute(const VsaGeom& g, const int* tiles, const void* q, const void* k, const void* v,
                           const void* gate, void* q2, void* k2, void* v2, void* g2, hipStream_t st) {
  const long long total = (long long)g.batch * g.N * g.heads * 16;
  const int blocks = (int)std::min<long long>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(vsa_rb_permute_kernel, dim3(blocks), dim3(256), 0, st, g, tiles, (const u32x4*)q, (const u32x4*)k,
                     (const u32x4*)v, (const u32x4*)gate, (u32x4*)q2, (u32x4*)k2, (u32x4*)v2, (u32x4*)g2);
}

void vsa_launch_rb_unpermute(const VsaGeom& g, const int* tiles, const void* o2, void* o, hipStream_t st) {
  const long long total = (long long)g.batch * g.N * g.heads * 16;
  const int blocks = (int)std::min<long long>((total + 255) / 256, 65536);
  hipLaunchKernelGGL(vsa_rb_unpermute_kernel, dim3(blocks), dim3(256), 0, st, g, tiles, (const u32x4*)o2, (u32x4*)o);
}
