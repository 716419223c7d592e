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
// h*Dh ..); L is [B*S, H] f32.  One wave per 32 query rows (forward, dQ) or
// 32 key rows (dK, dV) of one (sequence, head).  Products are
// v_mfma_f32_32x32x2f32 in f32 (bf16 storage is widened on load): for a
// contraction of length n, MFMA j takes index h*(n/2) + j from lane half h
// for both operands (a fixed permutation of the summation order).  A
// probability tile leaves the MFMA in the accumulator layout (row by
// register, column by lane); it goes through a per-wave 32 x 33 LDS tile to
// become the A operand of the next product.
//
// The backward is three launches with no atomics: D = rowsum(dO * O) per
// (row, head); dQ per query tile over its key tiles; dK and dV per key tile
// over its query tiles.  Results are bitwise reproducible.
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

// Max / sum over the 32 lanes of a lane half (one accumulator row).
__device__ __forceinline__ float half_max(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float half_sum(float v) {
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <typename T, int DH>
__global__ __launch_bounds__(WAVE) void attn_fwd_k(const T* __restrict__ q, const T* __restrict__ k,
                                                   const T* __restrict__ v, T* __restrict__ out,
                                                   float* __restrict__ lse, Geo g, float alpha, int causal) {
  __shared__ float tile[32 * 33];
  const int l = threadIdx.x;
  const int64_t q0 = (int64_t)blockIdx.x * 32, hd = blockIdx.y, b = blockIdx.z;
  float qf[DH / 2];
  frag_dh<T, DH>(q, g, b, hd, q0, l, qf);
  float m[16], s[16];
  f32x16_t o[DH / 32];
#pragma unroll
  for (int i = 0; i < 16; ++i) { m[i] = -INFINITY; s[i] = 0.f; }
#pragma unroll
  for (int t = 0; t < DH / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) o[t][i] = 0.f;
  const int64_t kend = causal ? (q0 + 32 < g.S ? q0 + 32 : g.S) : g.S;
  for (int64_t k0 = 0; k0 < kend; k0 += 32) {
    float kf[DH / 2];
    frag_dh<T, DH>(k, g, b, hd, k0, l, kf);
    f32x16_t z = dot_tile<DH>(qf, kf);
    const int64_t key = k0 + l % 32;
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t qr = q0 + crow(i, l);
      const bool keep = key < g.S && (!causal || key <= qr);
      const float zi = keep ? alpha * z[i] : -INFINITY;
      const float mn = fmaxf(m[i], half_max(zi));
      const float sc = ex(m[i] - mn);                     // 0 on the first tile (m = -inf)
      p[i] = keep ? ex(zi - mn) : 0.f;
      s[i] = s[i] * sc + half_sum(p[i]);
      m[i] = mn;
#pragma unroll
      for (int t = 0; t < DH / 32; ++t) o[t][i] *= sc;
    }
    f32x16_t pc;
#pragma unroll
    for (int i = 0; i < 16; ++i) pc[i] = p[i];
    float pa[16];
    c_to_a(pc, tile, l, pa);
    mul_rows<T, DH>(pa, v, g, b, hd, k0, l, o);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t qr = q0 + crow(i, l);
    if (qr >= g.S) continue;
    const float inv = 1.f / s[i];
    T* orow = out + (b * g.S + qr) * g.ld + hd * DH;
#pragma unroll
    for (int t = 0; t < DH / 32; ++t) stv<T>(orow + t * 32 + l % 32, o[t][i] * inv);
    if (l % 32 == 0) lse[(b * g.S + qr) * g.ldl + hd] = m[i] + logf(s[i]);
  }
}

// D[row, h] = sum over the head dimension of dO * O (f32).
template <typename T, int DH>
__global__ __launch_bounds__(256) void attn_bwd_d_k(const T* __restrict__ dout, const T* __restrict__ out,
                                                    float* __restrict__ dd, Geo g, int64_t rows) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;     // (row, head)
  if (idx >= rows * g.H) return;
  const int64_t r = idx / g.H, hd = idx % g.H;
  const T* a = dout + r * g.ld + hd * DH;
  const T* o = out + r * g.ld + hd * DH;
  float acc = 0.f;
  for (int j = 0; j < DH; ++j) acc += ldv<T>(a + j) * ldv<T>(o + j);
  dd[idx] = acc;
}

// dQ of 32 query rows: over key tiles, P = exp(alpha S - L), dP = dO V^T,
// dS = P (dP - D), dQ += alpha dS K.
template <typename T, int DH>
__global__ __launch_bounds__(WAVE) void attn_bwd_dq_k(const T* __restrict__ q, const T* __restrict__ k,
                                                      const T* __restrict__ v, const T* __restrict__ dout,
                                                      const float* __restrict__ lse, const float* __restrict__ dd,
                                                      T* __restrict__ dq, int acc_dq, Geo g, float alpha,
                                                      int causal) {
  __shared__ float tile[32 * 33];
  const int l = threadIdx.x;
  const int64_t q0 = (int64_t)blockIdx.x * 32, hd = blockIdx.y, b = blockIdx.z;
  float qf[DH / 2], df[DH / 2];
  frag_dh<T, DH>(q, g, b, hd, q0, l, qf);
  frag_dh<T, DH>(dout, g, b, hd, q0, l, df);
  float Lr[16], Dr[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t qr = q0 + crow(i, l);
    Lr[i] = qr < g.S ? lse[(b * g.S + qr) * g.ldl + hd] : 0.f;
    Dr[i] = qr < g.S ? dd[(b * g.S + qr) * g.H + hd] : 0.f;
  }
  f32x16_t acc[DH / 32];
#pragma unroll
  for (int t = 0; t < DH / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  const int64_t kend = causal ? (q0 + 32 < g.S ? q0 + 32 : g.S) : g.S;
  for (int64_t k0 = 0; k0 < kend; k0 += 32) {
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
template <typename T, int DH>
__global__ __launch_bounds__(WAVE) void attn_bwd_dkv_k(const T* __restrict__ q, const T* __restrict__ k,
                                                       const T* __restrict__ v, const T* __restrict__ dout,
                                                       const float* __restrict__ lse, const float* __restrict__ dd,
                                                       T* __restrict__ dk, int acc_dk, T* __restrict__ dv,
                                                       int acc_dv, Geo g, float alpha, int causal) {
  __shared__ float tile[32 * 33];
  const int l = threadIdx.x;
  const int64_t k0 = (int64_t)blockIdx.x * 32, hd = blockIdx.y, b = blockIdx.z;
  float kf[DH / 2], vf[DH / 2];
  frag_dh<T, DH>(k, g, b, hd, k0, l, kf);
  frag_dh<T, DH>(v, g, b, hd, k0, l, vf);
  f32x16_t ak[DH / 32], av[DH / 32];
#pragma unroll
  for (int t = 0; t < DH / 32; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) { ak[t][i] = 0.f; av[t][i] = 0.f; }
  for (int64_t q0 = causal ? k0 : 0; q0 < g.S; q0 += 32) {
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

template <typename T, int DH>
hipError_t fwd_dh(const AttnArgs& a, hipStream_t s) {
  const Geo g{a.S, a.H, a.ld, a.ldl};
  const dim3 grid((unsigned)((a.S + 31) / 32), (unsigned)a.H, (unsigned)a.B);
  attn_fwd_k<T, DH><<<grid, WAVE, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (T*)a.out, a.lse, g,
                                          a.alpha, a.causal);
  return hipGetLastError();
}

template <typename T, int DH>
hipError_t bwd_dh(const AttnArgs& a, hipStream_t s) {
  const Geo g{a.S, a.H, a.ld, a.ldl};
  const int64_t rows = a.B * a.S;
  attn_bwd_d_k<T, DH><<<(unsigned)((rows * a.H + 255) / 256), 256, 0, s>>>((const T*)a.dout, (const T*)a.out,
                                                                          a.dd, g, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((a.S + 31) / 32), (unsigned)a.H, (unsigned)a.B);
  if (a.dq) {
    attn_bwd_dq_k<T, DH><<<grid, WAVE, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout,
                                               a.lse, a.dd, (T*)a.dq, a.acc_dq, g, a.alpha, a.causal);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (a.dk || a.dv) {
    attn_bwd_dkv_k<T, DH><<<grid, WAVE, 0, s>>>((const T*)a.q, (const T*)a.k, (const T*)a.v, (const T*)a.dout,
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
  return a.bf16 ? fwd_t<bf16_t>(a, s) : fwd_t<float>(a, s);
}

hipError_t launch_attention_bwd(const AttnArgs& a, hipStream_t s) {
  if (a.B == 0 || a.S == 0 || a.H == 0) return hipSuccess;
  return a.bf16 ? bwd_t<bf16_t>(a, s) : bwd_t<float>(a, s);
}

}  // namespace xt
