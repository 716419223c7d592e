// Fused causal attention on the matrix cores, forward and backward.
//
// [AE] "Attention 用组合": attention is softmax(scale(Q K^T, alpha)
// [+ causal]) V.  The composed form materialises the [S, S] probabilities of
// every (sequence, head); this one keeps a 32 x 32 tile of them in
// registers at a time (online softmax: a running row maximum m and sum l,
// the output rescaled by exp(m_old - m_new) when m grows) and saves only
// the row log-sum-exp L = m + log l, from which the backward rebuilds each
// probability tile as exp(alpha S - L).
//
// Layout: q, k, v and out are [B*S, H*Dh] (row b*S + s, head h in columns
// h*Dh ..); L is [B*S, H] f32.  Two kernel families:
//   - f32 storage, and bf16 rows that are not 16-byte aligned: one block of
//     four waves per 32 query rows (forward, dQ) or 32 key rows (dK, dV) of
//     one (sequence, head), the waves splitting the loop over the other
//     operand's tiles; products are v_mfma_f32_32x32x2f32 in f32 (bf16 widened on
//     load): for a contraction of length n, MFMA j takes index h*(n/2) + j
//     from lane half h for both operands (a fixed permutation of the
//     summation order).  A probability tile leaves the MFMA in the
//     accumulator layout (row by register, column by lane).  The forward
//     forms its scores transposed (one query per lane column), so the
//     softmax needs no cross-lane reduction beyond one exchange and P^T is
//     the B operand of O^T += V^T P^T as it stands; the backward passes
//     take a tile through a per-wave 32 x 33 LDS tile to make it the A
//     operand of the next product.
//   - aligned bf16 storage: blocks of four waves on the bf16 matrix cores
//     (v_mfma_f32_32x32x16_bf16, f32 accumulation), with the f32
//     probabilities split into two bf16 parts so every product keeps f32
//     accuracy (see the section below).
//
// The backward is two launches with no atomics: D = rowsum(dO * O) per
// (row, head) and dQ per query tile over its key tiles; dK and dV per key
// tile over its query tiles.  Results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "common.h"
#include "internal.h"

namespace xt {
namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16_t;   // one 32 x 32 MFMA accumulator

constexpr float LOG2E = 1.4426950408889634f;

template <typename T>
__device__ __forceinline__ float ldv(const T* p);
template <> __device__ __forceinline__ float ldv<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldv<bf16_t>(const bf16_t* p) { return bf2f(*p); }

template <typename T>
__device__ __forceinline__ void stv(T* p, float v);
template <> __device__ __forceinline__ void stv<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void stv<bf16_t>(bf16_t* p, float v) { *p = (bf16_t)f2bf(v); }

__device__ __forceinline__ float ex(float z) { return exp2f(z * LOG2E); }

struct Geo {
  int64_t S, H, ld, ldl;   // sequence length, heads, row stride of q/k/v/out (elements), of L
};

// Row `r` (token index within the sequence) of head h of sequence b.
template <typename T>
__device__ __forceinline__ const T* rowp(const T* x, const Geo& g, int64_t b, int64_t h, int64_t r, int DH) {
  return x + (b * g.S + r) * g.ld + h * DH;
}

// Accumulator layout of a 32 x 32 MFMA tile: register i of lane l holds
// row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32.
__device__ __forceinline__ int crow(int i, int l) { return 8 * (i / 4) + 4 * (l / 32) + (i % 4); }

// Operand fragment of a contraction over the head dimension: lane l, MFMA
// j: x[row0 + l % 32][h * DH/2 + j] (0 past the sequence end).
template <typename T, int DH>
__device__ __forceinline__ void frag_dh(const T* x, const Geo& g, int64_t b, int64_t hd, int64_t row0, int l,
                                        float (&f)[DH / 2]) {
  const int64_t r = row0 + l % 32;
  const int k0 = (l / 32) * (DH / 2);
  if (r < g.S) {
    const T* p = rowp(x, g, b, hd, r, DH) + k0;
#pragma unroll
    for (int j = 0; j < DH / 2; ++j) f[j] = ldv<T>(p + j);
  } else {
#pragma unroll
    for (int j = 0; j < DH / 2; ++j) f[j] = 0.f;
  }
}

// Operand fragment of a contraction over 32 tile rows (keys or queries):
// lane l, MFMA j: x[row0 + h * 16 + j][col0 + l % 32] (0 past the end).
template <typename T, int DH>
__device__ __forceinline__ void frag_rows(const T* x, const Geo& g, int64_t b, int64_t hd, int64_t row0, int col0,
                                          int l, float (&f)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int64_t r = row0 + (l / 32) * 16 + j;
    f[j] = r < g.S ? ldv<T>(rowp(x, g, b, hd, r, DH) + col0 + l % 32) : 0.f;
  }
}

// S = X Y^T over the head dimension (X, Y fragments from frag_dh).
template <int DH>
__device__ __forceinline__ f32x16_t dot_tile(const float (&x)[DH / 2], const float (&y)[DH / 2]) {
  f32x16_t c;
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = 0.f;
#pragma unroll
  for (int j = 0; j < DH / 2; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(x[j], y[j], c, 0, 0, 0);
  return c;
}

// An accumulator tile as the A operand of a contraction over its columns:
// through a 32 x 33 LDS tile private to the wave.
__device__ __forceinline__ void c_to_a(const f32x16_t& c, float* t, int l, float (&a)[16]) {
#pragma unroll
  for (int i = 0; i < 16; ++i) t[crow(i, l) * 33 + l % 32] = c[i];
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 16; ++j) a[j] = t[(l % 32) * 33 + (l / 32) * 16 + j];
  __builtin_amdgcn_wave_barrier();
}

// acc[t] += A (32 x 32, rows = tile rows, k = 32 columns) times the 32 x DH
// matrix whose fragment rows are row0 + h*16 + j of x.
template <typename T, int DH>
__device__ __forceinline__ void mul_rows(const float (&a)[16], const T* x, const Geo& g, int64_t b, int64_t hd,
                                         int64_t row0, int l, f32x16_t (&acc)[DH / 32]) {
#pragma unroll
  for (int t = 0; t < DH / 32; ++t) {
    float f[16];
    frag_rows<T, DH>(x, g, b, hd, row0, t * 32, l, f);
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], f[j], acc[t], 0, 0, 0);
  }
}

// Operand fragment of a contraction over 32 rows of x (keys or queries) taken
// in an accumulator's row order: lane l, MFMA j: x[row0 + arow(j, l)][col0 +
// l % 32] (0 past the sequence end), arow(j, l) = 8 (j / 4) + 4 (l / 32) +
// j % 4.  Register j of an accumulator tile whose rows are those 32 rows is
// then the other operand of MFMA j as it is: the tile needs no transpose.
template <typename T, int DH>
__device__ __forceinline__ void frag_acc_rows(const T* x, const Geo& g, int64_t b, int64_t hd, int64_t row0,
                                              int col0, int l, float (&f)[16]) {
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int64_t r = row0 + crow(j, l);
    const float u = ldv<T>(rowp(x, g, b, hd, r < g.S ? r : g.S - 1, DH) + col0 + l % 32);
    f[j] = r < g.S ? u : 0.f;
  }
}

// acc[t] (rows: head dimension t*32 .., columns: the tile's 32 columns) +=
// X^T C, the contraction over the 32 rows of the accumulator tile C, with
// X^T's fragments from frag_acc_rows.
template <int DH>
__device__ __forceinline__ void mul_acc(const float (&x)[DH / 32][16], const f32x16_t& c, f32x16_t (&acc)[DH / 32]) {
#pragma unroll
  for (int t = 0; t < DH / 32; ++t)
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(x[t][j], c[j], acc[t], 0, 0, 0);
}

// Store an accumulator tile whose rows are the head dimension and whose
// column l % 32 is token `row` (when inside the sequence): register 4a + c
// holds dimension 8a + 4 (l / 32) + c, four consecutive values.
template <typename T, int DH>
__device__ __forceinline__ void store_dh(T* dst, const Geo& g, int64_t b, int64_t hd, int64_t row, int l,
                                         const f32x16_t (&acc)[DH / 32], float scale, int accumulate) {
  if (row >= g.S) return;
  T* p = dst + (b * g.S + row) * g.ld + hd * DH + 4 * (l / 32);
#pragma unroll
  for (int t = 0; t < DH / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      T* q = p + t * 32 + 8 * (i / 4) + (i % 4);
      float v = scale * acc[t][i];
      if (accumulate) v = acc_add(ldv<T>(q), v);
      stv<T>(q, v);
    }
}

// Blocks of KW waves share one 32-row tile: wave w takes the loop's tiles
// w, w + KW, ... (the key tiles of a query tile, or the query tiles of a
// key tile) with its own online state or partial sums, and wave 0 merges
// the waves' states in wave order (fixed: bitwise reproducible) and writes
// the result.  KW > 1 shortens the serial loop of each block KW-fold where
// the (sequence, head, tile) grid alone is too small to fill the chip.
constexpr int AKW = 4;

// Forward, scores transposed: S^T = K Q^T puts this lane's query (column
// l % 32) against the tile's keys in its 16 registers and the other lane
// half, so the row maximum and sum are in-lane plus one exchange with lane
// l ^ 32, and the probability tile P^T is directly the B operand of
// O^T += V^T P^T.
template <typename T, int DH, int KW>
__global__ __launch_bounds__(WAVE * KW) void attn_fwd_k(const T* __restrict__ q, const T* __restrict__ k,
                                                        const T* __restrict__ v, T* __restrict__ out,
                                                        float* __restrict__ lse, Geo g, float alpha, int causal) {
  __shared__ float mrg[KW > 1 ? KW - 1 : 1][2 + 16 * (DH / 32)][WAVE];   // m, s, O^T per register and lane
  const int l = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
  const int64_t q0 = (int64_t)blockIdx.x * 32, hd = blockIdx.y, b = blockIdx.z, qme = q0 + l % 32;
  float qf[DH / 2];
  frag_dh<T, DH>(q, g, b, hd, q0, l, qf);
  float m = -INFINITY, s = 0.f;
  f32x16_t o[DH / 32];
#pragma unroll
  for (int t = 0; t < DH / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  const int64_t kend = causal ? (q0 + 32 < g.S ? q0 + 32 : g.S) : g.S;
  // every tile a wave takes keeps at least one key of each query (causal:
  // k0 <= q0 <= the query), so m is finite after a wave's first tile
  for (int64_t k0 = (int64_t)w * 32; k0 < kend; k0 += 32 * KW) {
    // V^T fragments are loaded with K's, or (head size 128, where they
    // would not fit the registers) one 32-wide slice at a time before its
    // products
    constexpr bool EARLY = DH <= 64;
    float kf[DH / 2], vt[DH / 32][16];
    frag_dh<T, DH>(k, g, b, hd, k0, l, kf);
    if constexpr (EARLY) {
#pragma unroll
      for (int t = 0; t < DH / 32; ++t) frag_acc_rows<T, DH>(v, g, b, hd, k0, t * 32, l, vt[t]);
    }
    const f32x16_t z = dot_tile<DH>(kf, qf);
    float zs[16], mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t key = k0 + crow(i, l);
      const bool keep = key < g.S && (!causal || key <= qme);
      zs[i] = keep ? alpha * z[i] : -INFINITY;
      mx = fmaxf(mx, zs[i]);
    }
    const float mn = fmaxf(m, xor32_reduce(mx, OpMax{}));
    const float sc = ex(m - mn);                     // 0 on the first tile (m = -inf)
    f32x16_t p;
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      p[i] = zs[i] == -INFINITY ? 0.f : ex(zs[i] - mn);
      ps += p[i];
    }
    s = s * sc + xor32_reduce(ps, OpAdd{});
    m = mn;
#pragma unroll
    for (int t = 0; t < DH / 32; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) o[t][i] *= sc;
    if constexpr (EARLY) {
      mul_acc<DH>(vt, p, o);
    } else {
#pragma unroll
      for (int t = 0; t < DH / 32; ++t) {
        __builtin_amdgcn_sched_barrier(0);
        frag_acc_rows<T, DH>(v, g, b, hd, k0, t * 32, l, vt[0]);
#pragma unroll
        for (int j = 0; j < 16; ++j) o[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(vt[0][j], p[j], o[t], 0, 0, 0);
      }
    }
  }
  if constexpr (KW > 1) {
    if (w > 0) {
      mrg[w - 1][0][l] = m;
      mrg[w - 1][1][l] = s;
#pragma unroll
      for (int t = 0; t < DH / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mrg[w - 1][2 + 16 * t + i][l] = o[t][i];
    }
    __syncthreads();
    if (w > 0) return;
    // a wave with no tile holds m = -inf, s = 0, o = 0 and adds nothing
    for (int u = 1; u < KW; ++u) {
      const float mu = mrg[u - 1][0][l];
      const float mn = fmaxf(m, mu);
      const float ca = m == -INFINITY ? 0.f : ex(m - mn), cb = mu == -INFINITY ? 0.f : ex(mu - mn);
      s = s * ca + mrg[u - 1][1][l] * cb;
#pragma unroll
      for (int t = 0; t < DH / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) o[t][i] = o[t][i] * ca + mrg[u - 1][2 + 16 * t + i][l] * cb;
      m = mn;
    }
  }
  store_dh<T, DH>(out, g, b, hd, qme, l, o, 1.f / s, 0);
  if (qme < g.S && l < 32) lse[(b * g.S + qme) * g.ldl + hd] = m + logf(s);
}

// dQ of 32 query rows: over key tiles, P = exp(alpha S - L), dP = dO V^T,
// dS = P (dP - D), dQ += alpha dS K.  D = rowsum(dO * O) of the block's
// rows is formed here (each lane half sums its half of the head dimension,
// the halves are then added) and stored for the dK / dV pass; with
// dq == nullptr only D is produced.
template <typename T, int DH, int KW>
__global__ __launch_bounds__(WAVE * KW) void attn_bwd_dq_k(const T* __restrict__ q, const T* __restrict__ k,
                                                           const T* __restrict__ v, const T* __restrict__ dout,
                                                           const T* __restrict__ out, const float* __restrict__ lse,
                                                           float* __restrict__ dd, T* __restrict__ dq, int acc_dq,
                                                           Geo g, float alpha, int causal) {
  __shared__ float tiles[KW][32 * 33];
  __shared__ float mrg[KW > 1 ? KW - 1 : 1][DH / 32][16][WAVE];
  const int l = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
  float* tile = tiles[w];
  const int64_t q0 = (int64_t)blockIdx.x * 32, hd = blockIdx.y, b = blockIdx.z;
  float qf[DH / 2], df[DH / 2];
  frag_dh<T, DH>(q, g, b, hd, q0, l, qf);
  frag_dh<T, DH>(dout, g, b, hd, q0, l, df);
  float Dme;                                       // D of row q0 + l % 32 (0 past the end)
  {
    float of[DH / 2], part = 0.f;
    frag_dh<T, DH>(out, g, b, hd, q0, l, of);
#pragma unroll
    for (int j = 0; j < DH / 2; ++j) part += df[j] * of[j];
    Dme = xor32_reduce(part, OpAdd{});
  }
  if (w == 0 && l < 32 && q0 + l < g.S) dd[(b * g.S + q0 + l) * g.H + hd] = Dme;
  if (dq == nullptr) return;
  float Lr[16], Dr[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t qr = q0 + crow(i, l);
    Lr[i] = qr < g.S ? lse[(b * g.S + qr) * g.ldl + hd] : 0.f;
    Dr[i] = __shfl(Dme, crow(i, l));
  }
  f32x16_t acc[DH / 32];
#pragma unroll
  for (int t = 0; t < DH / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  const int64_t kend = causal ? (q0 + 32 < g.S ? q0 + 32 : g.S) : g.S;
  for (int64_t k0 = (int64_t)w * 32; k0 < kend; k0 += 32 * KW) {
    float kf[DH / 2], vf[DH / 2];
    frag_dh<T, DH>(k, g, b, hd, k0, l, kf);
    frag_dh<T, DH>(v, g, b, hd, k0, l, vf);
    const f32x16_t z = dot_tile<DH>(qf, kf);
    const f32x16_t dp = dot_tile<DH>(df, vf);
    const int64_t key = k0 + l % 32;
    f32x16_t ds;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t qr = q0 + crow(i, l);
      const bool keep = key < g.S && qr < g.S && (!causal || key <= qr);
      const float p = keep ? ex(alpha * z[i] - Lr[i]) : 0.f;
      ds[i] = p * (dp[i] - Dr[i]);
    }
    float da[16];
    c_to_a(ds, tile, l, da);
    mul_rows<T, DH>(da, k, g, b, hd, k0, l, acc);
  }
  if constexpr (KW > 1) {
    if (w > 0) {
#pragma unroll
      for (int t = 0; t < DH / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) mrg[w - 1][t][i][l] = acc[t][i];
    }
    __syncthreads();
    if (w > 0) return;
    for (int u = 1; u < KW; ++u)
#pragma unroll
      for (int t = 0; t < DH / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[t][i] += mrg[u - 1][t][i][l];
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t qr = q0 + crow(i, l);
    if (qr >= g.S) continue;
    T* row = dq + (b * g.S + qr) * g.ld + hd * DH;
#pragma unroll
    for (int t = 0; t < DH / 32; ++t) {
      float val = alpha * acc[t][i];
      if (acc_dq) val = acc_add(ldv<T>(row + t * 32 + l % 32), val);
      stv<T>(row + t * 32 + l % 32, val);
    }
  }
}

// dK, dV of 32 key rows: over query tiles, with rows = keys:
// P^T = exp(alpha K Q^T - L), dV += P^T dO, dP^T = V dO^T,
// dS^T = P^T (dP^T - D), dK += alpha dS^T Q.
template <typename T, int DH, int KW>
__global__ __launch_bounds__(WAVE * KW) void attn_bwd_dkv_k(const T* __restrict__ q, const T* __restrict__ k,
                                                            const T* __restrict__ v, const T* __restrict__ dout,
                                                            const float* __restrict__ lse, const float* __restrict__ dd,
                                                            T* __restrict__ dk, int acc_dk, T* __restrict__ dv,
                                                            int acc_dv, Geo g, float alpha, int causal) {
  __shared__ float tiles[KW][32 * 33];
  __shared__ float mrg[KW > 1 ? KW - 1 : 1][2 * (DH / 32)][16][WAVE];
  const int l = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
  float* tile = tiles[w];
  const int64_t k0 = (int64_t)blockIdx.x * 32, hd = blockIdx.y, b = blockIdx.z;
  float kf[DH / 2], vf[DH / 2];
  frag_dh<T, DH>(k, g, b, hd, k0, l, kf);
  frag_dh<T, DH>(v, g, b, hd, k0, l, vf);
  f32x16_t ak[DH / 32], av[DH / 32];
#pragma unroll
  for (int t = 0; t < DH / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) { ak[t][i] = 0.f; av[t][i] = 0.f; }
  for (int64_t q0 = (causal ? k0 : 0) + (int64_t)w * 32; q0 < g.S; q0 += 32 * KW) {
    float qf[DH / 2], df[DH / 2];
    frag_dh<T, DH>(q, g, b, hd, q0, l, qf);
    frag_dh<T, DH>(dout, g, b, hd, q0, l, df);
    const int64_t qr = q0 + l % 32;                 // this lane's query (column)
    const float Lq = qr < g.S ? lse[(b * g.S + qr) * g.ldl + hd] : 0.f;
    const float Dq = qr < g.S ? dd[(b * g.S + qr) * g.H + hd] : 0.f;
    const f32x16_t zt = dot_tile<DH>(kf, qf);       // [key][query]
    const f32x16_t dpt = dot_tile<DH>(vf, df);
    f32x16_t pt, dst;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t key = k0 + crow(i, l);
      const bool keep = key < g.S && qr < g.S && (!causal || key <= qr);
      pt[i] = keep ? ex(alpha * zt[i] - Lq) : 0.f;
      dst[i] = pt[i] * (dpt[i] - Dq);
    }
    float pa[16], sa[16];
    c_to_a(pt, tile, l, pa);
    mul_rows<T, DH>(pa, dout, g, b, hd, q0, l, av);
    c_to_a(dst, tile, l, sa);
    mul_rows<T, DH>(sa, q, g, b, hd, q0, l, ak);
  }
  if constexpr (KW > 1) {
    if (w > 0) {
#pragma unroll
      for (int t = 0; t < DH / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          mrg[w - 1][t][i][l] = ak[t][i];
          mrg[w - 1][DH / 32 + t][i][l] = av[t][i];
        }
    }
    __syncthreads();
    if (w > 0) return;
    for (int u = 1; u < KW; ++u)
#pragma unroll
      for (int t = 0; t < DH / 32; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          ak[t][i] += mrg[u - 1][t][i][l];
          av[t][i] += mrg[u - 1][DH / 32 + t][i][l];
        }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t key = k0 + crow(i, l);
    if (key >= g.S) continue;
    T* rk = dk + (b * g.S + key) * g.ld + hd * DH;
    T* rv = dv + (b * g.S + key) * g.ld + hd * DH;
#pragma unroll
    for (int t = 0; t < DH / 32; ++t) {
      const int c = t * 32 + l % 32;
      if (dk) {
        float val = alpha * ak[t][i];
        if (acc_dk) val = acc_add(ldv<T>(rk + c), val);
        stv<T>(rk + c, val);
      }
      if (dv) {
        float val = av[t][i];
        if (acc_dv) val = acc_add(ldv<T>(rv + c), val);
        stv<T>(rv + c, val);
      }
    }
  }
}

// ===========================================================================
// bf16 storage: bf16 MFMAs (v_mfma_f32_32x32x16_bf16, f32 accumulation).
//
// Blocks of 4 waves share K / V (or Q / dO) tiles that are staged through a
// double-buffered LDS ring: each thread loads its 16-byte chunks of tile j+1
// into registers while tile j is multiplied, and writes them to the other
// buffer before the block's one barrier per tile.  Each wave owns 32 rows.
//
// Score tiles are computed transposed where the softmax runs over the
// accumulator rows: S^T = K Q^T puts one query per lane (column), its keys
// in the lane's 16 registers and the other lane half, so a row maximum is 15
// in-lane max plus one exchange with lane l ^ 32.  An accumulator tile
// converted to bf16 is directly the B (or A) operand of the next product when
// its contraction index is taken in the accumulator's own row order
// (8 (e / 4) + 4 (l / 32) + e % 4 for element e of lane l); the other operand
// is read in that order by the transposing LDS read ds_read_b64_tr_b16.
//
// Precision: S and dP are exact products of the stored bf16 operands with
// f32 sums.  The probabilities P and dS = P (dP - D) are f32 values; they
// enter the second products (P V, P^T dO, dS K, dS^T Q) as two bf16 parts,
// hi + lo (split8), two MFMAs per product, so those products are as
// accurate as f32 arithmetic would make them, not rounded to bf16.  Maxima,
// exponentials, row sums and all accumulation are f32; only the outputs
// are rounded, once, to bf16 storage.
// ===========================================================================
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

namespace fa {
constexpr int NT = 256;            // 4 waves
// Row strides (elements) of LDS tiles.  RS: tiles read along rows with
// 16-byte reads (an odd multiple of 16 bytes: 16 consecutive rows hit 16
// distinct bank groups).  TS: tiles only read transposed (rows v = 0..3 of
// a read land on distinct 64-byte bank windows).
template <int DH> constexpr int RS = DH + 8;
template <int DH> constexpr int TS = DH == 32 ? 32 : DH == 64 ? 96 : 160;
}  // namespace fa

__device__ __forceinline__ bf16x8_t lds8(const bf16_t* p) { return *reinterpret_cast<const bf16x8_t*>(p); }

// Operand from a row-major LDS tile whose rows run along the contraction:
// lane l gets tile[r0 + 8 (e / 4) + 4 (l / 32) + e % 4][col0 + l % 32] as
// element e.  ds_read_b64_tr_b16: within each group of 16 lanes, lane j
// receives element j % 4 of the 8-byte pieces that lanes 4 v + j / 4
// address, v = 0..3.
template <int STRIDE>
__device__ __forceinline__ bf16x8_t tr_frag(const bf16_t* tile, int r0, int col0, int l) {
  const int g = l / 16, j = l % 16;
  const int col = col0 + 16 * (g & 1) + 4 * (j & 3);
  s16x4_t v[2];
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    const int row = r0 + 8 * r + 4 * (g >> 1) + j / 4;
    v[r] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + row * STRIDE + col));
  }
  const short __attribute__((ext_vector_type(8))) w8 = {v[0][0], v[0][1], v[0][2], v[0][3],
                                                        v[1][0], v[1][1], v[1][2], v[1][3]};
  return __builtin_bit_cast(bf16x8_t, w8);
}

// Registers 8 m .. 8 m + 7 of an accumulator as a pair of bf16 operands
// whose sum carries the f32 values to about 2^-17: hi = bf16(x) (nearest),
// lo = bf16(x - hi).  x - hi is exact in f32 (the rounding error of a
// nearest rounding to 8 significant bits), so hi + lo differs from x by at
// most 2^-9 |x - hi| <= 2^-18 |x|; a product taken as A hi + A lo is then
// f32-accurate, not bf16-accurate, in this operand.
struct Split8 {
  bf16x8_t hi, lo;
};
// x - hi is formed as a two-term bf16 dot product of the packed hi pair
// with (-1, 0) or (0, -1), accumulated onto x: one instruction per element,
// exact like the subtraction (both products are exact and the sum is an f32
// value).  With sum given, the hi and lo parts are added to it pairwise by
// the same dot product with (1, 1): the row sum of exactly the operand
// values that enter the product.
// The three packed constants are passed in scalar registers: the compiler
// would encode the pair (-1, 0) as the inline constant -1.0, which the
// instruction does not read as that bf16 pair.
__device__ __forceinline__ Split8 split8(const f32x16_t& c, int m, float* sum = nullptr) {
  uint32_t kl = 0x0000BF80u, kh = 0xBF800000u, k1 = 0x3F803F80u;
  asm("" : "+s"(kl), "+s"(kh), "+s"(k1));
  const bf16x2_t neg_lo = __builtin_bit_cast(bf16x2_t, kl), neg_hi = __builtin_bit_cast(bf16x2_t, kh);
  const bf16x2_t ones = __builtin_bit_cast(bf16x2_t, k1);
  uint32_t h[4], r[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float a = c[8 * m + 2 * q], b = c[8 * m + 2 * q + 1];
    const uint32_t u = f2bf2(a, b);
    h[q] = u;
    const bf16x2_t hp = __builtin_bit_cast(bf16x2_t, u);
    r[q] = f2bf2(__builtin_amdgcn_fdot2_f32_bf16(hp, neg_lo, a, false),
                 __builtin_amdgcn_fdot2_f32_bf16(hp, neg_hi, b, false));
    if (sum) {
      *sum = __builtin_amdgcn_fdot2_f32_bf16(hp, ones, *sum, false);
      *sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, r[q]), ones, *sum, false);
    }
  }
  const u32x4_t uh = {h[0], h[1], h[2], h[3]}, ur = {r[0], r[1], r[2], r[3]};
  return Split8{__builtin_bit_cast(bf16x8_t, uh), __builtin_bit_cast(bf16x8_t, ur)};
}

__device__ __forceinline__ f32x16_t mfma16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void zero(f32x16_t& c) {
#pragma unroll
  for (int i = 0; i < 16; ++i) c[i] = 0.f;
}

// Row within an accumulator tile of register i of lane half h.
__device__ __forceinline__ int arow(int i, int h) { return 8 * (i / 4) + 4 * h + (i % 4); }

// This lane's 16-byte pieces of row `row` (clamped into the sequence) of a
// [B*S, H*Dh] tensor as the fragments of a contraction over the head
// dimension: piece kk holds columns 16 kk + 8 h .. +7.
template <int DH>
__device__ __forceinline__ void row_frags(const bf16_t* x, const Geo& g, int64_t b, int64_t hd, int64_t row, int h,
                                          bool valid, bf16x8_t (&f)[DH / 16]) {
  const bf16_t* p = x + (b * g.S + row) * g.ld + hd * DH + 8 * h;
#pragma unroll
  for (int kk = 0; kk < DH / 16; ++kk) {
    if (valid) {
      f[kk] = *reinterpret_cast<const bf16x8_t*>(p + 16 * kk);
    } else {
      const u32x4_t z = {0u, 0u, 0u, 0u};
      f[kk] = __builtin_bit_cast(bf16x8_t, z);
    }
  }
}

// Staging of an R-row tile of two tensors (rows clamped to the sequence):
// thread t moves 16-byte chunks t, t + 256, ...  Addresses are a
// tile-uniform base (row r0) plus 32-bit lane offsets (R ld < 2^31 elements,
// which fa_aligned guarantees), fixed for every tile that lies inside the
// sequence; only a tile that reaches past its end clamps rows per lane.
template <int DH, int R>
struct Stage2 {
  static constexpr int CPR = DH / 8, NC = R * CPR, N = (NC + fa::NT - 1) / fa::NT;   // chunks per row, tile, thread
  u32x4_t a[N], b[N];
  __device__ __forceinline__ void load(const bf16_t* xa, const bf16_t* xb, const Geo& g, int64_t base, int64_t r0,
                                       int tid) {
    const bf16_t* pa = xa + base + r0 * g.ld;
    const bf16_t* pb = xb + base + r0 * g.ld;
    const int ld = (int)g.ld;
    if (r0 + R <= g.S) {
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int c = tid + fa::NT * i, row = c / CPR, col = c % CPR;
        if (NC % fa::NT == 0 || c < NC) {
          const uint32_t off = (uint32_t)(row * ld + col * 8);
          a[i] = *reinterpret_cast<const u32x4_t*>(pa + off);
          b[i] = *reinterpret_cast<const u32x4_t*>(pb + off);
        }
      }
    } else {
      const int last = (int)(g.S - 1 - r0);   // < R - 1 here
#pragma unroll
      for (int i = 0; i < N; ++i) {
        const int c = tid + fa::NT * i, row = c / CPR, col = c % CPR;
        if (NC % fa::NT == 0 || c < NC) {
          const uint32_t off = (uint32_t)((row < last ? row : last) * ld + col * 8);
          a[i] = *reinterpret_cast<const u32x4_t*>(pa + off);
          b[i] = *reinterpret_cast<const u32x4_t*>(pb + off);
        }
      }
    }
  }
  template <int SA, int SB>
  __device__ __forceinline__ void store(bf16_t* ta, bf16_t* tb, int tid) const {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const int c = tid + fa::NT * i, row = c / CPR, col = c % CPR;
      if (NC % fa::NT == 0 || c < NC) {
        *reinterpret_cast<u32x4_t*>(ta + row * SA + col * 8) = a[i];
        *reinterpret_cast<u32x4_t*>(tb + row * SB + col * 8) = b[i];
      }
    }
  }
};

// Block -> (row block, sequence * heads + head).  Consecutive blocks take
// different heads, so a head keeps to one XCD when the head count is a
// multiple of 8.  Under a causal mask the work of a row block grows (query
// blocks) or shrinks (key blocks) along the sequence; blocks are dealt
// zig-zag: the heavier half first, heaviest first, then the lighter half,
// lightest first, so a compute unit that takes block i and later block
// i + half the grid gets about the same total work as any other.
__device__ __forceinline__ void fa_block(int nrb, int heavy_end, int& rb, int64_t& hb) {
  const int HB = gridDim.x / nrb, r = blockIdx.x / HB, half = (nrb + 1) / 2;
  hb = blockIdx.x % HB;
  const int heavy = r < half ? r : nrb - 1 - (r - half);   // rank from the heaviest
  rb = heavy_end > 0 ? nrb - 1 - heavy : heavy_end < 0 ? heavy : r;
}

// Forward: 128 queries per block (32 per wave), K / V tiles of 64 keys.
template <int DH>
__global__ __launch_bounds__(fa::NT, 2) void fa_fwd_k(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                      const bf16_t* __restrict__ v, bf16_t* __restrict__ out,
                                                      float* __restrict__ lse, Geo g, float alpha, int causal,
                                                      int nqb, int pair) {
  constexpr int BK = 64, KS = fa::RS<DH>, VS = fa::TS<DH>, KT = BK * KS, ST = KT + BK * VS;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * ST];
  const int tid = threadIdx.x, w = tid / WAVE, l = tid % WAVE, h = l / 32, c = l % 32;
  int64_t hb;
  // one query block of (sequence, head) hb
  auto run = [&](int qb) {
  const int64_t b = hb / g.H, hd = hb % g.H, base = b * g.S * g.ld + hd * DH;
  const int64_t q0 = (int64_t)qb * 128, qw = q0 + 32 * w, qme = qw + c;
  bf16x8_t qf[DH / 16];
  row_frags<DH>(q, g, b, hd, qme, h, qme < g.S, qf);
  const int64_t kend = causal ? (q0 + 128 < g.S ? q0 + 128 : g.S) : g.S;
  const int nt = (int)((kend + BK - 1) / BK);
  Stage2<DH, BK> st;
  st.load(k, v, g, base, 0, tid);
  st.template store<KS, VS>(lds, lds + KT, tid);
  __syncthreads();
  const float sl = alpha * LOG2E;
  const int klim = causal && qme < g.S ? (int)qme : (int)g.S - 1;   // last key this lane's query sees
  float m = -INFINITY, ls = 0.f;        // running maximum (log2 units), this lane half's sum
  f32x16_t o[DH / 32];                  // O^T: rows = head dimension, column = this lane's query
#pragma unroll
  for (int bb = 0; bb < DH / 32; ++bb) zero(o[bb]);
  // Tiles 0 .. nact-1 hold keys this wave's queries see; the rest (causal)
  // only pass through the staging ring.  Two loops, so the accumulators
  // never merge with a skipped tile.
  const int nact = causal ? (int)((qw + 31) / BK + 1 < nt ? (qw + 31) / BK + 1 : nt) : nt;
  auto stage_next = [&](int j) {
    if (j + 1 < nt) st.template store<KS, VS>(lds + ((j + 1) & 1) * ST, lds + ((j + 1) & 1) * ST + KT, tid);
    __syncthreads();
  };
  int j = 0;
  for (; j < nact; ++j) {
    const int64_t k0 = (int64_t)j * BK;
    if (j + 1 < nt) st.load(k, v, g, base, k0 + BK, tid);
    const bf16_t* Kt = lds + (j & 1) * ST;
    const bf16_t* Vt = Kt + KT;
    {
      // the two 32-key halves' products alternate: consecutive MFMAs are
      // independent
      f32x16_t s[2];
      zero(s[0]);
      zero(s[1]);
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        const bf16x8_t k0f = lds8(Kt + c * KS + 16 * kk + 8 * h), k1f = lds8(Kt + (32 + c) * KS + 16 * kk + 8 * h);
        s[0] = mfma16(k0f, qf[kk], s[0]);
        s[1] = mfma16(k1f, qf[kk], s[1]);
      }
      // Row maximum of the raw scores (alpha > 0, so the order is that of
      // alpha S); masked keys become -inf.
      const bool edge = k0 + BK > g.S || (causal && k0 + BK - 1 > qw);
      float mx = -INFINITY;
      if (edge) {                       // keys past klim are masked
        // arow(i, h) = arow(i, 0) + 4 h: compare immediates with a shifted limit
        const int kl = klim - (int)k0 - 4 * h;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            s[t][i] = 32 * t + arow(i, 0) <= kl ? s[t][i] : -INFINITY;
            mx = fmaxf(mx, s[t][i]);
          }
      } else {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[t][i]);
      }
      mx = xor32_reduce(mx, OpMax{}) * sl;
      // The reference point m only moves when some row's maximum exceeds it
      // by more than 8 (log2 units): exponentials stay below 2^8, and the
      // final division by the row sum cancels the choice of m exactly.
      if (__any(mx > m + 8.f)) {
        const float mn = fmaxf(m, mx);
        const float sc = __builtin_amdgcn_exp2f(m - mn);   // 0 on the first tile (m = -inf)
        ls *= sc;
#pragma unroll
        for (int bb = 0; bb < DH / 32; ++bb)
#pragma unroll
          for (int i = 0; i < 16; ++i) o[bb][i] *= sc;
        m = mn;
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) s[t][i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[t][i], sl, -m));
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int mm = 0; mm < 2; ++mm) {
          const Split8 pf = split8(s[t], mm, &ls);
          bf16x8_t vf[DH / 32];
#pragma unroll
          for (int bb = 0; bb < DH / 32; ++bb) vf[bb] = tr_frag<VS>(Vt, 32 * t + 16 * mm, 32 * bb, l);
#pragma unroll
          for (int bb = 0; bb < DH / 32; ++bb) o[bb] = mfma16(vf[bb], pf.lo, o[bb]);
#pragma unroll
          for (int bb = 0; bb < DH / 32; ++bb) o[bb] = mfma16(vf[bb], pf.hi, o[bb]);
        }
    }
    stage_next(j);
  }
  for (; j < nt; ++j) {
    if (j + 1 < nt) st.load(k, v, g, base, (int64_t)(j + 1) * BK, tid);
    stage_next(j);
  }
  const float tot = xor32_reduce(ls, OpAdd{});
  if (qme < g.S) {
    const float inv = 1.f / tot;
    bf16_t* orow = out + (b * g.S + qme) * g.ld + hd * DH;
#pragma unroll
    for (int bb = 0; bb < DH / 32; ++bb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * bb + 8 * i4 + 4 * h;
        const uint2 u = make_uint2(f2bf2(o[bb][4 * i4] * inv, o[bb][4 * i4 + 1] * inv),
                                   f2bf2(o[bb][4 * i4 + 2] * inv, o[bb][4 * i4 + 3] * inv));
        *reinterpret_cast<uint2*>(orow + d) = u;
      }
    if (h == 0) lse[(b * g.S + qme) * g.ldl + hd] = (m + __log2f(tot)) * 0.6931471805599453f;
  }
  };
  if (pair) {
    // causal pairs: the heaviest query block of the pair, then the lightest,
    // so every block carries about the same work
    const int np = (nqb + 1) / 2, HB = gridDim.x / np, r = blockIdx.x / HB;
    hb = blockIdx.x % HB;
    run(nqb - 1 - r);
    if (r != nqb - 1 - r) {
      __syncthreads();
      run(r);
    }
  } else {
    int qb;
    fa_block(nqb, causal ? 1 : 0, qb, hb);
    run(qb);
  }
}

// Backward, dQ and D: 128 queries per block (32 per wave), K / V tiles of 32
// keys.  D = rowsum(dO * O) is formed here for the wave's queries and stored
// for the dK / dV kernel.  With dq == nullptr only D is produced.
template <int DH>
__global__ __launch_bounds__(fa::NT, 2) void fa_dq_k(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                     const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                                                     const bf16_t* __restrict__ out, const float* __restrict__ lse,
                                                     float* __restrict__ dd, bf16_t* __restrict__ dq, int acc_dq,
                                                     Geo g, float alpha, int causal, int nqb, int pair) {
  constexpr int BK = 32, KS = fa::RS<DH>, KT = BK * KS, ST = 2 * KT;
  __shared__ __attribute__((aligned(16))) bf16_t lds[2 * ST];
  const int tid = threadIdx.x, w = tid / WAVE, l = tid % WAVE, h = l / 32, c = l % 32;
  int64_t hb;
  // one query block of (sequence, head) hb
  auto run = [&](int qb) {
  const int64_t b = hb / g.H, hd = hb % g.H, base = b * g.S * g.ld + hd * DH;
  const int64_t q0 = (int64_t)qb * 128, qw = q0 + 32 * w, qme = qw + c;
  const bool qok = qme < g.S;
  bf16x8_t qf[DH / 16], df[DH / 16];
  row_frags<DH>(dout, g, b, hd, qme, h, qok, df);
  float Dq;
  {
    bf16x8_t of[DH / 16];
    row_frags<DH>(out, g, b, hd, qme, h, qok, of);
    float acc = 0.f;
#pragma unroll
    for (int kk = 0; kk < DH / 16; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc += (float)df[kk][e] * (float)of[kk][e];
    Dq = xor32_reduce(acc, OpAdd{});
    if (qok && h == 0) dd[(b * g.S + qme) * g.H + hd] = Dq;
  }
  if (!dq) return;
  row_frags<DH>(q, g, b, hd, qme, h, qok, qf);
  const float sl = alpha * LOG2E;
  const float L2 = qok ? lse[(b * g.S + qme) * g.ldl + hd] * LOG2E : 0.f;
  // last key this lane's query sees (-1: a row past the sequence sees none)
  const int klim = !qok ? -1 : causal ? (int)qme : (int)g.S - 1;
  const int64_t kend = causal ? (q0 + 128 < g.S ? q0 + 128 : g.S) : g.S;
  const int nt = (int)((kend + BK - 1) / BK);
  Stage2<DH, BK> st;
  st.load(k, v, g, base, 0, tid);
  st.template store<KS, KS>(lds, lds + KT, tid);
  __syncthreads();
  f32x16_t acc[DH / 32];                // dQ^T: rows = head dimension, column = this lane's query
#pragma unroll
  for (int bb = 0; bb < DH / 32; ++bb) zero(acc[bb]);
  const int nact = causal ? (int)((qw + 31) / BK + 1 < nt ? (qw + 31) / BK + 1 : nt) : nt;
  auto stage_next = [&](int j) {
    if (j + 1 < nt) st.template store<KS, KS>(lds + ((j + 1) & 1) * ST, lds + ((j + 1) & 1) * ST + KT, tid);
    __syncthreads();
  };
  int j = 0;
  for (; j < nact; ++j) {
    const int64_t k0 = (int64_t)j * BK;
    if (j + 1 < nt) st.load(k, v, g, base, k0 + BK, tid);
    const bf16_t* Kt = lds + (j & 1) * ST;
    const bf16_t* Vt = Kt + KT;
    {
      f32x16_t s, dp;
      zero(s);
      zero(dp);
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        s = mfma16(lds8(Kt + c * KS + 16 * kk + 8 * h), qf[kk], s);
        dp = mfma16(lds8(Vt + c * KS + 16 * kk + 8 * h), df[kk], dp);
      }
      const bool edge = k0 + BK > g.S || (causal && k0 + BK - 1 > qw);
      if (edge) {
        const int kl = klim - (int)k0 - 4 * h;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = arow(i, 0) <= kl ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sl, -L2)) : 0.f;
          s[i] = p * (dp[i] - Dq);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sl, -L2)) * (dp[i] - Dq);
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const Split8 sf = split8(s, mm);
        bf16x8_t kf[DH / 32];
#pragma unroll
        for (int bb = 0; bb < DH / 32; ++bb) kf[bb] = tr_frag<KS>(Kt, 16 * mm, 32 * bb, l);
#pragma unroll
        for (int bb = 0; bb < DH / 32; ++bb) acc[bb] = mfma16(kf[bb], sf.lo, acc[bb]);
#pragma unroll
        for (int bb = 0; bb < DH / 32; ++bb) acc[bb] = mfma16(kf[bb], sf.hi, acc[bb]);
      }
    }
    stage_next(j);
  }
  for (; j < nt; ++j) {
    if (j + 1 < nt) st.load(k, v, g, base, (int64_t)(j + 1) * BK, tid);
    stage_next(j);
  }
  if (qok) {
    bf16_t* row = dq + (b * g.S + qme) * g.ld + hd * DH;
#pragma unroll
    for (int bb = 0; bb < DH / 32; ++bb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d = 32 * bb + 8 * i4 + 4 * h;
        float r[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = alpha * acc[bb][4 * i4 + e];
        if (acc_dq) {
          const uint2 old = *reinterpret_cast<const uint2*>(row + d);
          r[0] = acc_add(bf2f(old.x & 0xffffu), r[0]);
          r[1] = acc_add(bf2f(old.x >> 16), r[1]);
          r[2] = acc_add(bf2f(old.y & 0xffffu), r[2]);
          r[3] = acc_add(bf2f(old.y >> 16), r[3]);
        }
        *reinterpret_cast<uint2*>(row + d) = make_uint2(f2bf2(r[0], r[1]), f2bf2(r[2], r[3]));
      }
  }
  };
  if (pair) {                        // (heaviest, lightest) pairs, as in the forward
    const int np = (nqb + 1) / 2, HB = gridDim.x / np, r = blockIdx.x / HB;
    hb = blockIdx.x % HB;
    run(nqb - 1 - r);
    if (r != nqb - 1 - r) {
      __syncthreads();
      run(r);
    }
  } else {
    int qb;
    fa_block(nqb, causal ? 1 : 0, qb, hb);
    run(qb);
  }
}

// Backward, dK and dV: 128 keys per block, in two groups of four waves
// (32 keys per wave); Q / dO tiles of 32 queries, with their L and D.
// Group gq takes the query tiles gq, gq + 2, ... of the block's range, so
// each SIMD holds two waves working on the block's K and V (one from each
// group), and group 1's dK, dV are added to group 0's through LDS at the
// end (fixed order: bitwise reproducible).  Scores are not transposed here:
// S = Q K^T has the wave's key per lane (column) and the queries in
// registers, which is the A-operand order of P^T and dS^T for dV += P^T dO,
// dK += dS^T Q.  The block's K and V rows stay in LDS for the whole kernel
// (registers go to the two 32 x Dh accumulators).
template <int DH>
__global__ __launch_bounds__(2 * fa::NT, 1) void fa_dkv_k(const bf16_t* __restrict__ q, const bf16_t* __restrict__ k,
                                                          const bf16_t* __restrict__ v, const bf16_t* __restrict__ dout,
                                                          const float* __restrict__ lse, const float* __restrict__ dd,
                                                          bf16_t* __restrict__ dk, int acc_dk, bf16_t* __restrict__ dv,
                                                          int acc_dv, Geo g, float alpha, int causal, int nkb, int pair) {
  constexpr int BQ = 32, QS = fa::RS<DH>, QT = BQ * QS, ST = 2 * QT + 4 * BQ;   // + L2 and D: 2 BQ f32
  constexpr int KV = 128 * QS;                        // the block's K (then V) rows
  constexpr int NACC = 2 * (DH / 32) * 16;            // accumulator registers per lane (dK, dV)
  static_assert((size_t)4 * WAVE * NACC * sizeof(float) <= (4 * ST + 2 * KV) * sizeof(bf16_t),
                "group 1's accumulators fit the block's LDS");
  __shared__ __attribute__((aligned(16))) bf16_t lds[4 * ST + 2 * KV];   // [group][stage] tiles, then K, V
  const int tid = threadIdx.x, gq = tid / fa::NT, gt = tid % fa::NT;
  const int w = gt / WAVE, l = tid % WAVE, h = l / 32, c = l % 32;
  int64_t hb;
  // one key block of (sequence, head) hb
  auto run = [&](int kb) {
  const int64_t b = hb / g.H, hd = hb % g.H, base = b * g.S * g.ld + hd * DH;
  const int64_t k0 = (int64_t)kb * 128, kw = k0 + 32 * w, kme = kw + c;
  const bool kok = kme < g.S;
  bf16_t* const Kb = lds + 4 * ST;                    // rows k0 .. k0 + 127 (clamped)
  bf16_t* const Vb = Kb + KV;
  if (gq == 0) {
    Stage2<DH, 128> kv;
    kv.load(k, v, g, base, k0, gt);
    kv.template store<QS, QS>(Kb, Vb, gt);
  }
  const bf16_t* const Kw = Kb + 32 * w * QS + c * QS + 8 * h;   // this lane's key row, piece kk at + 16 kk
  const bf16_t* const Vw = Vb + 32 * w * QS + c * QS + 8 * h;
  const float sl = alpha * LOG2E;
  const int64_t qbeg = causal ? k0 / BQ : 0;          // first query tile
  const int nt = (int)((g.S + BQ - 1) / BQ - qbeg);
  bf16_t* const G = lds + gq * 2 * ST;                // this group's two stages
  Stage2<DH, BQ> st;
  float lq = 0.f;                                     // this thread's L2 or D entry of the staged tile
  auto load_ld = [&](int64_t r0) {
    if (gt < 2 * BQ) {
      const int64_t r = r0 + gt % BQ < g.S ? r0 + gt % BQ : g.S - 1;
      lq = gt < BQ ? lse[(b * g.S + r) * g.ldl + hd] * LOG2E : dd[(b * g.S + r) * g.H + hd];
    }
  };
  auto store_ld = [&](bf16_t* t) {
    if (gt < 2 * BQ) reinterpret_cast<float*>(t + 2 * QT)[gt] = lq;
  };
  if (gq < nt) {
    st.load(q, dout, g, base, (qbeg + gq) * BQ, gt);
    load_ld((qbeg + gq) * BQ);
    st.template store<QS, QS>(G, G + QT, gt);
    store_ld(G);
  }
  __syncthreads();
  f32x16_t ak[DH / 32], av[DH / 32];   // rows = the wave's keys, column = head dimension
#pragma unroll
  for (int bb = 0; bb < DH / 32; ++bb) { zero(ak[bb]); zero(av[bb]); }
  // Query tiles before jfirst lie wholly before this wave's keys (causal):
  // they only pass through the staging ring.
  int jfirst = 0;
  if (causal) {
    const int64_t f = (kw - BQ + 1 + BQ - 1) / BQ - qbeg;   // first tile with q0 + BQ - 1 >= kw
    jfirst = f < 0 ? 0 : f > nt ? nt : (int)f;
  }
  // both groups run the same rounds (the barriers are the block's)
  const int rounds = (nt + 1) / 2;
  for (int jj = 0; jj < rounds; ++jj) {
    const int j = 2 * jj + gq;
    const int64_t q0 = (qbeg + j) * BQ;
    if (j + 2 < nt) { st.load(q, dout, g, base, q0 + 2 * BQ, gt); load_ld(q0 + 2 * BQ); }
    if (j < nt && j >= jfirst) {
    const bf16_t* Qt = G + (jj & 1) * ST;
    const bf16_t* Dt = Qt + QT;
    const float* LD = reinterpret_cast<const float*>(Qt + 2 * QT);   // [0, BQ): L2, [BQ, 2 BQ): D
    {
      f32x16_t s, dp;
      zero(s);
      zero(dp);
#pragma unroll
      for (int kk = 0; kk < DH / 16; ++kk) {
        s = mfma16(lds8(Qt + c * QS + 16 * kk + 8 * h), lds8(Kw + 16 * kk), s);
        dp = mfma16(lds8(Dt + c * QS + 16 * kk + 8 * h), lds8(Vw + 16 * kk), dp);
      }
      const bool edge = q0 + BQ > g.S || (causal && q0 < kw + 31) || kw + 31 >= g.S;
      float Lv[16], Dv[16];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const float4 L4 = *reinterpret_cast<const float4*>(LD + 8 * i4 + 4 * h);
        const float4 D4 = *reinterpret_cast<const float4*>(LD + BQ + 8 * i4 + 4 * h);
        Lv[4 * i4] = L4.x; Lv[4 * i4 + 1] = L4.y; Lv[4 * i4 + 2] = L4.z; Lv[4 * i4 + 3] = L4.w;
        Dv[4 * i4] = D4.x; Dv[4 * i4 + 1] = D4.y; Dv[4 * i4 + 2] = D4.z; Dv[4 * i4 + 3] = D4.w;
      }
      if (edge) {
        // visible rows of the tile: qlo .. qhi (none for a key past the sequence)
        const int qlo = (causal ? (int)(kme - q0) : 0) - 4 * h;
        const int qhi = (kok ? (int)(g.S - 1 - q0) : -1) - 4 * h;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = arow(i, 0);
          const float p = r >= qlo && r <= qhi ? __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sl, -Lv[i])) : 0.f;
          s[i] = p;
          dp[i] = p * (dp[i] - Dv[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], sl, -Lv[i]));
          s[i] = p;
          dp[i] = p * (dp[i] - Dv[i]);
        }
      }
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const Split8 pf = split8(s, mm), sf = split8(dp, mm);
#pragma unroll
        for (int bb = 0; bb < DH / 32; ++bb) {
          const bf16x8_t df = tr_frag<QS>(Dt, 16 * mm, 32 * bb, l), qf = tr_frag<QS>(Qt, 16 * mm, 32 * bb, l);
          av[bb] = mfma16(pf.lo, df, av[bb]);
          ak[bb] = mfma16(sf.lo, qf, ak[bb]);
          av[bb] = mfma16(pf.hi, df, av[bb]);
          ak[bb] = mfma16(sf.hi, qf, ak[bb]);
        }
      }
    }
    }
    if (j + 2 < nt) {
      bf16_t* nx = G + ((jj + 1) & 1) * ST;
      st.template store<QS, QS>(nx, nx + QT, gt);
      store_ld(nx);
    }
    __syncthreads();
  }
  // group 1's sums through LDS (every wave is past its last LDS read)
  float* red = reinterpret_cast<float*>(lds) + (size_t)w * NACC * WAVE;
  if (gq == 1) {
#pragma unroll
    for (int bb = 0; bb < DH / 32; ++bb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        red[(bb * 16 + i) * WAVE + l] = ak[bb][i];
        red[((DH / 32 + bb) * 16 + i) * WAVE + l] = av[bb][i];
      }
  }
  __syncthreads();
  if (gq == 0) {
#pragma unroll
    for (int bb = 0; bb < DH / 32; ++bb)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        ak[bb][i] = acc_add(ak[bb][i], red[(bb * 16 + i) * WAVE + l]);
        av[bb][i] = acc_add(av[bb][i], red[((DH / 32 + bb) * 16 + i) * WAVE + l]);
      }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t key = kw + arow(i, h);
      if (key >= g.S) continue;
      const int64_t off = (b * g.S + key) * g.ld + hd * DH + c;
#pragma unroll
      for (int bb = 0; bb < DH / 32; ++bb) {
        if (dk) {
          float val = alpha * ak[bb][i];
          if (acc_dk) val = acc_add(bf2f(dk[off + 32 * bb]), val);
          dk[off + 32 * bb] = (bf16_t)f2bf(val);
        }
        if (dv) {
          float val = av[bb][i];
          if (acc_dv) val = acc_add(bf2f(dv[off + 32 * bb]), val);
          dv[off + 32 * bb] = (bf16_t)f2bf(val);
        }
      }
    }
  }
  };
  if (pair) {
    // causal pairs: the heaviest key block of the pair (the first keys see
    // every query), then the lightest, so every block carries the same work
    const int np = (nkb + 1) / 2, HB = gridDim.x / np, r = blockIdx.x / HB;
    hb = blockIdx.x % HB;
    run(r);
    if (r != nkb - 1 - r) {
      __syncthreads();
      run(nkb - 1 - r);
    }
  } else {
    int kb;
    fa_block(nkb, causal ? -1 : 0, kb, hb);
    run(kb);
  }
}

// Compute units of the current device (0 if unknown).
int device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  return cus;
}

// Causal query blocks go in (heaviest, lightest) pairs when the paired grid
// still holds two blocks per CU (measured, forward: 1 x 8192 tokens, 16
// heads: 359 -> 315 us); with fewer pairs, one block per CU runs slower than
// the unpaired grid (2 x 2048 tokens: 63 -> 73 us).
int fa_pair(const AttnArgs& a, int nqb) {
  const int64_t pairs = (int64_t)((nqb + 1) / 2) * a.H * a.B;
  const int cus = device_cus();
  return a.causal && nqb > 1 && cus > 0 && pairs >= 2 * (int64_t)cus ? 1 : 0;
}

template <int DH>
hipError_t fa_fwd(const AttnArgs& a, hipStream_t s) {
  const Geo g{a.S, a.H, a.ld, a.ldl};
  const int nqb = (int)((a.S + 127) / 128);
  const int pair = fa_pair(a, nqb);
  const int nb = pair ? (nqb + 1) / 2 : nqb;
  fa_fwd_k<DH><<<(unsigned)(nb * a.H * a.B), fa::NT, 0, s>>>((const bf16_t*)a.q, (const bf16_t*)a.k,
                                                              (const bf16_t*)a.v, (bf16_t*)a.out, a.lse, g, a.alpha,
                                                              a.causal, nqb, pair);
  return hipGetLastError();
}

template <int DH>
hipError_t fa_bwd(const AttnArgs& a, hipStream_t s) {
  const Geo g{a.S, a.H, a.ld, a.ldl};
  const int nb = (int)((a.S + 127) / 128);
  const unsigned grid = (unsigned)(nb * a.H * a.B);
  const int pair = fa_pair(a, nb);
  const unsigned gq = pair ? (unsigned)((nb + 1) / 2 * a.H * a.B) : grid;
  fa_dq_k<DH><<<gq, fa::NT, 0, s>>>((const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v,
                                    (const bf16_t*)a.dout, (const bf16_t*)a.out, a.lse, a.dd, (bf16_t*)a.dq,
                                    a.acc_dq, g, a.alpha, a.causal, nb, pair);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || (!a.dk && !a.dv)) return e;
  // dK / dV run one block per CU: key blocks pair up once the pairs alone
  // fill every CU
  const int cus = device_cus();
  const int64_t npair = (int64_t)((nb + 1) / 2) * a.H * a.B;
  const int kpair = a.causal && nb > 1 && cus > 0 && npair >= (int64_t)cus ? 1 : 0;
  const unsigned gk = kpair ? (unsigned)npair : grid;
  fa_dkv_k<DH><<<gk, 2 * fa::NT, 0, s>>>((const bf16_t*)a.q, (const bf16_t*)a.k, (const bf16_t*)a.v,
                                     (const bf16_t*)a.dout, a.lse, a.dd, (bf16_t*)a.dk, a.acc_dk, (bf16_t*)a.dv,
                                     a.acc_dv, g, a.alpha, a.causal, nb, kpair);
  return hipGetLastError();
}

// The bf16 kernels move 16-byte pieces: every tensor 16-byte aligned with a
// row stride that keeps rows aligned; and they take alpha > 0.
bool fa_aligned(const AttnArgs& a) {
  if (a.ld % 8 || !(a.alpha > 0.f)) return false;   // the forward orders scores by the raw products
  if (a.ld >= (int64_t)1 << 23) return false;        // tile offsets are 32-bit (128 rows of ld elements)
  const void* p[] = {a.q, a.k, a.v, a.out, a.dout, a.dq, a.dk, a.dv};
  for (const void* x : p)
    if (x && ((uintptr_t)x & 15u)) return false;
  return true;
}

template <typename T, int DH>
hipError_t fwd_dh(const AttnArgs& a, hipStream_t s) {
  const Geo g{a.S, a.H, a.ld, a.ldl};
  const dim3 grid((unsigned)((a.S + 31) / 32), (unsigned)a.H, (unsigned)a.B);
  attn_fwd_k<T, DH, AKW><<<grid, WAVE * AKW, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, g,
                                          a.alpha, a.causal);
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t bwd_dh(const AttnArgs& a, hipStream_t s) {
  const Geo g{a.S, a.H, a.ld, a.ldl};
  const dim3 grid((unsigned)((a.S + 31) / 32), (unsigned)a.H, (unsigned)a.B);
  // D for every row, and dQ when asked for
  attn_bwd_dq_k<T, DH, AKW><<<grid, WAVE * AKW, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout,
                                                         (const T*)a.out, a.lse, a.dd, (T*)a.dq, a.acc_dq, g, a.alpha,
                                                         a.causal);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.dk || a.dv) {
    attn_bwd_dkv_k<T, DH, AKW><<<grid, WAVE * AKW, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout,
                                                a.lse, a.dd, (T*)a.dk, a.acc_dk, (T*)a.dv, a.acc_dv, g, a.alpha,
                                                a.causal);
    e = hipGetLastError();
  }
  return e;
}

template <typename T>
hipError_t fwd_t(const AttnArgs& a, hipStream_t s) {
  switch (a.Dh) {
    case 32: return fwd_dh<T, 32>(a, s);
    case 64: return fwd_dh<T, 64>(a, s);
    default: return fwd_dh<T, 128>(a, s);
  }
}

template <typename T>
hipError_t bwd_t(const AttnArgs& a, hipStream_t s) {
  switch (a.Dh) {
    case 32: return bwd_dh<T, 32>(a, s);
    case 64: return bwd_dh<T, 64>(a, s);
    default: return bwd_dh<T, 128>(a, s);
  }
}

}  // namespace

hipError_t launch_attention_fwd(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.S == 0 || a.H == 0) return hipSuccess;
  if (a.bf16 && fa_aligned(a)) {
    switch (a.Dh) {
      case 32: return fa_fwd<32>(a, s);
      case 64: return fa_fwd<64>(a, s);
      default: return fa_fwd<128>(a, s);
    }
  }
  return a.bf16 ? fwd_t<bf16_t>(a, s) : fwd_t<float>(a, s);
}

hipError_t launch_attention_bwd(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.S == 0 || a.H == 0) return hipSuccess;
  if (a.bf16 && fa_aligned(a)) {
    switch (a.Dh) {
      case 32: return fa_bwd<32>(a, s);
      case 64: return fa_bwd<64>(a, s);
      default: return fa_bwd<128>(a, s);
    }
  }
  return a.bf16 ? bwd_t<bf16_t>(a, s) : bwd_t<float>(a, s);
}

}  // namespace xt
