// Row-wise reductions on the rows the register-resident kernels of
// rowwise.hip do not take: rows longer than a row group's registers hold
// (f32 softmax rows past 16384 columns, layer_norm backward rows whose
// parameter partials would not fit the block's LDS fold), and rows that are
// not a whole number of 16-byte packs or do not start on a 16-byte boundary
// (a 50257-wide vocabulary row).
//
// [AE] "RMSNorm" paragraph and the op-backward rows "softmax" / "Softmax
// 反向推导"; [BP] k_layernorm_fwd / k_layernorm_bwd, "Sparade tensorer",
// "En baklängeskärnas uppgift" -- the same mathematics as the register
// kernels, with the same saved statistics and outputs.
//
// One 1024-thread block per row (blocks loop over rows).  The kernels that
// fit 64 registers without spilling and write no partial rows (f32 softmax
// forward, softmax backward, f32 rms_norm dx) are held to 64, so two blocks
// (two rows' loads in flight) share a CU.  Each row is split
// at 16-byte boundaries into a scalar head (elements before the first
// boundary), a body of 16-byte packs and a scalar tail; every tensor the op
// touches is split the same way when their rows start at the same offset
// modulo 16 bytes (else the whole row goes element by element).  A row is
// traversed twice (three times for the layer_norm forward, whose variance is
// taken about the mean): a reduction pass with ordinary loads, so the row's
// lines stay in the L2 and the Infinity Cache, then the pass that writes,
// whose re-read is served from there -- HBM sees the algorithmic bytes once.
// Block reductions are DPP wave reductions plus a fixed-order LDS combine:
// deterministic.
//
// Parameter gradients (rms_norm dgamma, layer_norm dgamma | dbeta): when
// every row has the same split (row starts 16-byte aligned), thread t owns
// the same columns in every row -- packs t, t + 1024, ... and tail element
// t -- and keeps their partial sums in registers over the block's rows; at
// the end it writes them to the block's partial row (no LDS).  The fixed-
// order column fold of rowwise.hip then sums the partial rows.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace xt {
namespace {

constexpr int ST = 1024, SW = ST / WAVE;    // threads and waves per block
constexpr int SU = 8;                       // packs per thread in flight (forward)
constexpr int SUB = 2;                      // (backward, three tensors)
constexpr float LOG2E = 1.4426950408889634f;

struct Split {
  int64_t head, packs;   // elements before the first 16-byte boundary; whole packs after them
};

template <typename T>
__device__ __forceinline__ Split split_of(const void* p, int64_t C) {
  constexpr int V = io<T>::VEC;
  const uintptr_t a = (uintptr_t)p;
  int64_t h = (int64_t)(((16 - (a & 15)) & 15) / sizeof(T));
  if (h > C) h = C;
  return {h, (C - h) / V};
}

__device__ __forceinline__ bool same16(const void* a, const void* b) {
  return !b || ((((uintptr_t)a) ^ ((uintptr_t)b)) & 15) == 0;
}

template <typename T> __device__ __forceinline__ const T* crow(const void* p, int64_t r, int64_t ld) {
  return reinterpret_cast<const T*>(p) + r * ld;
}
template <typename T> __device__ __forceinline__ T* wrow(void* p, int64_t r, int64_t ld) {
  return reinterpret_cast<T*>(p) + r * ld;
}

template <bool NT>
__device__ __forceinline__ uint4 ld16(const void* p) {
  if constexpr (NT) return ld_nt(p);
  else return *reinterpret_cast<const uint4*>(p);
}

// One pass over a row of NTS tensors: fs(c) for every head / tail element,
// fp(c0, q) for every body pack (q[t] the raw pack of tensor t at column
// c0), U packs' loads in flight per thread.  NT: nontemporal loads (the
// last pass over the row).
template <typename T, int NTS, int U, bool NT, class FS, class FP>
__device__ __forceinline__ void row_pass(const T* const (&src)[NTS], const Split& sp, int64_t C, FS fs, FP fp) {
  constexpr int V = io<T>::VEC;
  const int tid = threadIdx.x;
  for (int64_t c = tid; c < sp.head; c += ST) fs(c);
  for (int64_t p0 = tid; p0 < sp.packs; p0 += (int64_t)ST * U) {
    uint4 q[U][NTS];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = p0 + (int64_t)u * ST;
      if (p < sp.packs)
#pragma unroll
        for (int t = 0; t < NTS; ++t) q[u][t] = ld16<NT>(src[t] + sp.head + p * V);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t p = p0 + (int64_t)u * ST;
      if (p < sp.packs) fp(sp.head + p * V, q[u]);
    }
  }
  for (int64_t c = sp.head + sp.packs * V + tid; c < C; c += ST) fs(c);
}

// Block-wide (max, sum) merge: wave_merge, then the waves in order.  `ms`
// holds two sets of SW states; consecutive calls alternate between them.
template <int NW = SW>
__device__ __forceinline__ MS block_merge(MS st, float (*ms)[2][NW], int& ph) {
  st = wave_merge(st);
  const int w = threadIdx.x / WAVE;
  if ((threadIdx.x % WAVE) == 0) { ms[ph][0][w] = st.m; ms[ph][1][w] = st.s; }
  lds_barrier();
  MS tot{ms[ph][0][0], ms[ph][1][0]};
#pragma unroll
  for (int i = 1; i < NW; ++i) tot = ms_merge(tot, MS{ms[ph][0][i], ms[ph][1][i]});
  ph ^= 1;
  return tot;
}

template <typename T>
__device__ __forceinline__ void store_acc1(T* p, float v, bool acc) {
  io<T>::st(p, acc ? acc_add(io<T>::ld(p), v) : v);
}

// V consecutive f32 of a parameter vector from column c0 (c0 + V <= C).  A
// row's packs start at c0 = head + p*V, so their 4-float phase
// (g + c0) mod 16 bytes is the same for the whole row: the covering span is
// read with aligned 16-byte loads and the V values taken out with a
// row-uniform select; a span that would reach past C goes element by element.
template <int V>
__device__ __forceinline__ void load_par(const float* __restrict__ g, int64_t c0, int64_t C, float* out) {
  const int mis = (int)((((uintptr_t)(g + c0)) >> 2) & 3);
  if (mis == 0) {
#pragma unroll
    for (int k = 0; k < V; k += 4) {
      const float4 q = *reinterpret_cast<const float4*>(g + c0 + k);
      out[k] = q.x; out[k + 1] = q.y; out[k + 2] = q.z; out[k + 3] = q.w;
    }
    return;
  }
  constexpr int NQ = V / 4 + 1;
  if (c0 - mis + 4 * NQ > C) {
#pragma unroll
    for (int k = 0; k < V; ++k) out[k] = g[c0 + k];
    return;
  }
  const float* base = g + c0 - mis;
  float w[4 * NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const float4 q = *reinterpret_cast<const float4*>(base + 4 * i);
    w[4 * i] = q.x; w[4 * i + 1] = q.y; w[4 * i + 2] = q.z; w[4 * i + 3] = q.w;
  }
  if (mis == 1) {
#pragma unroll
    for (int k = 0; k < V; ++k) out[k] = w[k + 1];
  } else if (mis == 2) {
#pragma unroll
    for (int k = 0; k < V; ++k) out[k] = w[k + 2];
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) out[k] = w[k + 3];
  }
}

// ================================================================ softmax
template <typename T>
__global__ __launch_bounds__(ST, sizeof(T) == 4 ? 8 : 1) void sm_fwd_stream(const void* __restrict__ x, int64_t ldx, void* __restrict__ y,
                                                    int64_t ldy, int64_t R, int64_t C, float alpha, int causal,
                                                    int seq_len) {
  constexpr int V = io<T>::VEC;
  __shared__ float ms[2][2][SW];
  int ph = 0;
  const float sl = alpha * LOG2E;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* xr = crow<T>(x, r, ldx);
    T* yr = wrow<T>(y, r, ldy);
    const int64_t lim = causal ? min(C, (int64_t)(r % seq_len) + 1) : C;
    const Split sp = same16(xr, yr) ? split_of<T>(xr, C) : Split{C, 0};
    float m = -__builtin_inff(), s = 0.f;     // base-2 online state of this thread
    const T* src[1] = {xr};
    row_pass<T, 1, SU, false>(src, sp, C,
        [&](int64_t c) {
          if (c < lim) {
            const float t = io<T>::ld(xr + c) * sl;
            if (t > m) { s = s * __builtin_amdgcn_exp2f(m - t) + 1.f; m = t; }
            else s += __builtin_amdgcn_exp2f(t - m);
          }
        },
        [&](int64_t c0, const uint4 (&q)[1]) {
          float v[V];
          io<T>::unpack(q[0], v);
          float pm = -__builtin_inff();
#pragma unroll
          for (int k = 0; k < V; ++k) {
            v[k] = c0 + k < lim ? v[k] * sl : -__builtin_inff();
            pm = fmaxf(pm, v[k]);
          }
          if (pm == -__builtin_inff()) return;      // the whole pack is past the causal limit
          if (pm > m) { s *= __builtin_amdgcn_exp2f(m - pm); m = pm; }
          float a = 0.f;
#pragma unroll
          for (int k = 0; k < V; ++k) a += __builtin_amdgcn_exp2f(v[k] - m);
          s += a;
        });
    const MS tot = block_merge(MS{m, s}, ms, ph);
    const float inv = 1.f / tot.s, mm = tot.m;
    row_pass<T, 1, SU, true>(src, sp, C,
        [&](int64_t c) { io<T>::st(yr + c, c < lim ? __builtin_amdgcn_exp2f(io<T>::ld(xr + c) * sl - mm) * inv : 0.f); },
        [&](int64_t c0, const uint4 (&q)[1]) {
          float v[V];
          io<T>::unpack(q[0], v);
#pragma unroll
          for (int k = 0; k < V; ++k) v[k] = c0 + k < lim ? __builtin_amdgcn_exp2f(v[k] * sl - mm) * inv : 0.f;
          st_nt(yr + c0, io<T>::pack(v));
        });
  }
}

template <typename T>
__global__ __launch_bounds__(ST, 8) void sm_bwd_stream(const void* __restrict__ d, int64_t ldd, const void* __restrict__ y,
                                                    int64_t ldy, void* __restrict__ dx, int64_t lddx, int acc,
                                                    int64_t R, int64_t C, float alpha) {
  constexpr int V = io<T>::VEC;
  __shared__ float lds[4 * SW];
  int ph = 0;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* dr = crow<T>(d, r, ldd);
    const T* yr = crow<T>(y, r, ldy);
    T* xr = wrow<T>(dx, r, lddx);
    const Split sp = same16(dr, yr) && same16(dr, xr) ? split_of<T>(dr, C) : Split{C, 0};
    const T* src[2] = {dr, yr};
    float dot = 0.f;
    row_pass<T, 2, SUB, false>(src, sp, C, [&](int64_t c) { dot += io<T>::ld(dr + c) * io<T>::ld(yr + c); },
        [&](int64_t, const uint4 (&q)[2]) {
          float a[V], b[V];
          io<T>::unpack(q[0], a);
          io<T>::unpack(q[1], b);
#pragma unroll
          for (int k = 0; k < V; ++k) dot += a[k] * b[k];
        });
    dot = group_sum<SW>(dot, lds, ph);
    row_pass<T, 2, SUB, true>(src, sp, C,
        [&](int64_t c) { store_acc1<T>(xr + c, alpha * io<T>::ld(yr + c) * (io<T>::ld(dr + c) - dot), acc != 0); },
        [&](int64_t c0, const uint4 (&q)[2]) {
          float a[V], b[V], o[V];
          io<T>::unpack(q[0], a);
          io<T>::unpack(q[1], b);
#pragma unroll
          for (int k = 0; k < V; ++k) o[k] = alpha * b[k] * (a[k] - dot);
          if (acc) {
            float old[V];
            io<T>::unpack(ld_nt(xr + c0), old);
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = acc_add(old[k], o[k]);
          }
          st_nt(xr + c0, io<T>::pack(o));
        });
  }
}

// =============================================================== rms_norm
template <typename T>
__global__ __launch_bounds__(ST) void rms_fwd_stream(const void* __restrict__ x, int64_t ldx,
                                                     const float* __restrict__ gamma, void* __restrict__ y,
                                                     int64_t ldy, float* __restrict__ ir, int64_t ldir, int64_t R,
                                                     int64_t C, float eps, float invC) {
  constexpr int V = io<T>::VEC;
  __shared__ float lds[4 * SW];
  int ph = 0;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* xr = crow<T>(x, r, ldx);
    T* yr = wrow<T>(y, r, ldy);
    const Split sp = same16(xr, yr) ? split_of<T>(xr, C) : Split{C, 0};
    const T* src[1] = {xr};
    float ss = 0.f;
    row_pass<T, 1, SU, false>(src, sp, C, [&](int64_t c) { const float v = io<T>::ld(xr + c); ss += v * v; },
        [&](int64_t, const uint4 (&q)[1]) {
          float v[V];
          io<T>::unpack(q[0], v);
#pragma unroll
          for (int k = 0; k < V; ++k) ss += v[k] * v[k];
        });
    ss = group_sum<SW>(ss, lds, ph);
    const float irv = rsqrtf(ss * invC + eps);
    if (threadIdx.x == 0) ir[r * ldir] = irv;
    row_pass<T, 1, SU, true>(src, sp, C, [&](int64_t c) { io<T>::st(yr + c, io<T>::ld(xr + c) * irv * gamma[c]); },
        [&](int64_t c0, const uint4 (&q)[1]) {
          float v[V], g[V];
          io<T>::unpack(q[0], v);
          load_par<V>(gamma, c0, C, g);
#pragma unroll
          for (int k = 0; k < V; ++k) v[k] = v[k] * irv * g[k];
          st_nt(yr + c0, io<T>::pack(v));
        });
  }
}

// Columns owned by this thread when every row has the same split with no
// head: packs tid + k*ST (k < PK) and tail element tid.  Partial sums of
// NP per-column terms are kept for them over the block's rows.
template <int NP, int PK, int V>
struct OwnedPartials {
  float pk[NP][PK][V];
  float tl[NP];
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int q = 0; q < NP; ++q) {
      tl[q] = 0.f;
#pragma unroll
      for (int k = 0; k < PK; ++k)
#pragma unroll
        for (int e = 0; e < V; ++e) pk[q][k][e] = 0.f;
    }
  }
  // writes this thread's columns of the block's partial row (NP vectors of C)
  __device__ __forceinline__ void write(float* part, int64_t packs, int64_t C) const {
    float* out = part + (int64_t)blockIdx.x * NP * C;
    const int tid = threadIdx.x;
#pragma unroll
    for (int q = 0; q < NP; ++q) {
#pragma unroll
      for (int k = 0; k < PK; ++k) {
        const int64_t p = tid + (int64_t)k * ST;
        if (p < packs)
#pragma unroll
          for (int e = 0; e < V; ++e) out[q * C + p * V + e] = pk[q][k][e];
      }
      const int64_t c = packs * V + tid;
      if (c < C) out[q * C + c] = tl[q];
    }
  }
};

// rms_norm backward, fixed split (PK > 0: owned partials of dgamma) or any
// split (PK == 0: dx only; the partials come from a separate column pass).
template <typename T, int PK>
__global__ __launch_bounds__(ST, PK == 0 && sizeof(T) == 4 ? 8 : 1) void rms_bwd_stream(const void* __restrict__ d, int64_t ldd, const void* __restrict__ x,
                                                     int64_t ldx, const float* __restrict__ gamma,
                                                     const float* __restrict__ ir, int64_t ldir, void* __restrict__ dx,
                                                     int64_t lddx, int acc, float* __restrict__ part, int64_t R,
                                                     int64_t C, float invC) {
  constexpr int V = io<T>::VEC;
  __shared__ float lds[4 * SW];
  int ph = 0;
  OwnedPartials<1, PK ? PK : 1, V> pp;
  pp.zero();
  const int tid = threadIdx.x;
  int64_t packs_fixed = 0;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* dr = crow<T>(d, r, ldd);
    const T* xr = crow<T>(x, r, ldx);
    T* or_ = dx ? wrow<T>(dx, r, lddx) : nullptr;
    const Split sp = same16(dr, xr) && same16(dr, or_) ? split_of<T>(dr, C) : Split{C, 0};
    const float irv = ir[r * ldir];
    const T* src[2] = {dr, xr};
    float dot = 0.f;
    row_pass<T, 2, SUB, false>(src, sp, C, [&](int64_t c) { dot += io<T>::ld(dr + c) * gamma[c] * io<T>::ld(xr + c); },
        [&](int64_t c0, const uint4 (&q)[2]) {
          float a[V], b[V], g[V];
          io<T>::unpack(q[0], a);
          io<T>::unpack(q[1], b);
          load_par<V>(gamma, c0, C, g);
#pragma unroll
          for (int k = 0; k < V; ++k) dot += a[k] * g[k] * b[k];
        });
    dot = group_sum<SW>(dot, lds, ph);
    const float c1 = irv * irv * irv * invC * dot;
    if constexpr (PK > 0) {
      // fixed split (head 0): pack tid + k*ST of every row is this thread's
      packs_fixed = sp.packs;
#pragma unroll
      for (int k0 = 0; k0 < PK; k0 += SUB) {
        uint4 q[SUB][2];
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
          const int64_t p = tid + (int64_t)(k0 + u) * ST;
          if (p < sp.packs) { q[u][0] = ld_nt(dr + p * V); q[u][1] = ld_nt(xr + p * V); }
        }
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
          const int64_t p = tid + (int64_t)(k0 + u) * ST;
          if (p >= sp.packs) continue;
          float a[V], b[V], g[V], o[V];
          io<T>::unpack(q[u][0], a);
          io<T>::unpack(q[u][1], b);
          load_par<V>(gamma, p * V, C, g);
#pragma unroll
          for (int k = 0; k < V; ++k) {
            o[k] = irv * (a[k] * g[k]) - b[k] * c1;
            pp.pk[0][k0 + u][k] += a[k] * b[k] * irv;
          }
          if (or_) {
            if (acc) {
              float old[V];
              io<T>::unpack(ld_nt(or_ + p * V), old);
#pragma unroll
              for (int k = 0; k < V; ++k) o[k] = acc_add(old[k], o[k]);
            }
            st_nt(or_ + p * V, io<T>::pack(o));
          }
        }
      }
      const int64_t c = sp.packs * V + tid;
      if (c < C) {
        const float a = io<T>::ld(dr + c), b = io<T>::ld(xr + c);
        pp.tl[0] += a * b * irv;
        if (or_) store_acc1<T>(or_ + c, irv * (a * gamma[c]) - b * c1, acc != 0);
      }
    } else if (or_) {
      row_pass<T, 2, SUB, true>(src, sp, C,
          [&](int64_t c) { store_acc1<T>(or_ + c, irv * (io<T>::ld(dr + c) * gamma[c]) - io<T>::ld(xr + c) * c1, acc != 0); },
          [&](int64_t c0, const uint4 (&q)[2]) {
            float a[V], b[V], g[V], o[V];
            io<T>::unpack(q[0], a);
            io<T>::unpack(q[1], b);
            load_par<V>(gamma, c0, C, g);
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = irv * (a[k] * g[k]) - b[k] * c1;
            if (acc) {
              float old[V];
              io<T>::unpack(ld_nt(or_ + c0), old);
#pragma unroll
              for (int k = 0; k < V; ++k) o[k] = acc_add(old[k], o[k]);
            }
            st_nt(or_ + c0, io<T>::pack(o));
          });
    }
  }
  if constexpr (PK > 0)
    if (part) pp.write(part, packs_fixed, C);
}

// ============================================================= layer_norm
template <typename T>
__global__ __launch_bounds__(ST) void ln_fwd_stream(const void* __restrict__ x, int64_t ldx,
                                                    const float* __restrict__ gamma, const float* __restrict__ beta,
                                                    void* __restrict__ y, int64_t ldy, float* __restrict__ mean,
                                                    int64_t ldm, float* __restrict__ rstd, int64_t ldr, int64_t R,
                                                    int64_t C, float eps, float invC) {
  constexpr int V = io<T>::VEC;
  __shared__ float lds[4 * SW];
  int ph = 0;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* xr = crow<T>(x, r, ldx);
    T* yr = wrow<T>(y, r, ldy);
    const Split sp = same16(xr, yr) ? split_of<T>(xr, C) : Split{C, 0};
    const T* src[1] = {xr};
    float s = 0.f;
    row_pass<T, 1, SU, false>(src, sp, C, [&](int64_t c) { s += io<T>::ld(xr + c); },
        [&](int64_t, const uint4 (&q)[1]) {
          float v[V];
          io<T>::unpack(q[0], v);
#pragma unroll
          for (int k = 0; k < V; ++k) s += v[k];
        });
    const float mu = group_sum<SW>(s, lds, ph) * invC;
    float qv = 0.f;        // sum of squared deviations about the mean (a second pass)
    row_pass<T, 1, SU, false>(src, sp, C, [&](int64_t c) { const float t = io<T>::ld(xr + c) - mu; qv += t * t; },
        [&](int64_t, const uint4 (&q)[1]) {
          float v[V];
          io<T>::unpack(q[0], v);
#pragma unroll
          for (int k = 0; k < V; ++k) { const float t = v[k] - mu; qv += t * t; }
        });
    const float rs = rsqrtf(group_sum<SW>(qv, lds, ph) * invC + eps);
    if (threadIdx.x == 0) { mean[r * ldm] = mu; rstd[r * ldr] = rs; }
    row_pass<T, 1, SU, true>(src, sp, C,
        [&](int64_t c) { io<T>::st(yr + c, (io<T>::ld(xr + c) - mu) * rs * gamma[c] + beta[c]); },
        [&](int64_t c0, const uint4 (&q)[1]) {
          float v[V], g[V], b[V];
          io<T>::unpack(q[0], v);
          load_par<V>(gamma, c0, C, g);
          load_par<V>(beta, c0, C, b);
#pragma unroll
          for (int k = 0; k < V; ++k) v[k] = (v[k] - mu) * rs * g[k] + b[k];
          st_nt(yr + c0, io<T>::pack(v));
        });
  }
}

template <typename T, int PK>
__global__ __launch_bounds__(ST) void ln_bwd_stream(const void* __restrict__ d, int64_t ldd, const void* __restrict__ x,
                                                    int64_t ldx, const float* __restrict__ gamma,
                                                    const float* __restrict__ mean, int64_t ldm,
                                                    const float* __restrict__ rstd, int64_t ldr,
                                                    void* __restrict__ dx, int64_t lddx, int acc,
                                                    float* __restrict__ part, int64_t R, int64_t C, float invC) {
  constexpr int V = io<T>::VEC;
  __shared__ float lds[4 * SW];
  int ph = 0;
  OwnedPartials<2, PK ? PK : 1, V> pp;
  pp.zero();
  const int tid = threadIdx.x;
  int64_t packs_fixed = 0;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* dr = crow<T>(d, r, ldd);
    const T* xr = crow<T>(x, r, ldx);
    T* or_ = dx ? wrow<T>(dx, r, lddx) : nullptr;
    const Split sp = same16(dr, xr) && same16(dr, or_) ? split_of<T>(dr, C) : Split{C, 0};
    const float mu = mean[r * ldm], rs = rstd[r * ldr];
    const T* src[2] = {dr, xr};
    float s1 = 0.f, s2 = 0.f;
    row_pass<T, 2, SUB, false>(src, sp, C,
        [&](int64_t c) {
          const float gv = io<T>::ld(dr + c) * gamma[c];
          s1 += gv;
          s2 += gv * ((io<T>::ld(xr + c) - mu) * rs);
        },
        [&](int64_t c0, const uint4 (&q)[2]) {
          float a[V], b[V], g[V];
          io<T>::unpack(q[0], a);
          io<T>::unpack(q[1], b);
          load_par<V>(gamma, c0, C, g);
#pragma unroll
          for (int k = 0; k < V; ++k) {
            const float gv = a[k] * g[k];
            s1 += gv;
            s2 += gv * ((b[k] - mu) * rs);
          }
        });
    group_sum2<SW>(s1, s2, lds, ph);
    const float a1 = s1 * invC, b1 = s2 * invC;
    auto dxv = [&](float dv, float gv, float xv) { return rs * (dv * gv - a1 - ((xv - mu) * rs) * b1); };
    if constexpr (PK > 0) {
      packs_fixed = sp.packs;
#pragma unroll
      for (int k0 = 0; k0 < PK; k0 += SUB) {
        uint4 q[SUB][2];
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
          const int64_t p = tid + (int64_t)(k0 + u) * ST;
          if (p < sp.packs) { q[u][0] = ld_nt(dr + p * V); q[u][1] = ld_nt(xr + p * V); }
        }
#pragma unroll
        for (int u = 0; u < SUB; ++u) {
          const int64_t p = tid + (int64_t)(k0 + u) * ST;
          if (p >= sp.packs) continue;
          float a[V], b[V], g[V], o[V];
          io<T>::unpack(q[u][0], a);
          io<T>::unpack(q[u][1], b);
          load_par<V>(gamma, p * V, C, g);
#pragma unroll
          for (int k = 0; k < V; ++k) {
            o[k] = dxv(a[k], g[k], b[k]);
            pp.pk[0][k0 + u][k] += a[k] * ((b[k] - mu) * rs);
            pp.pk[1][k0 + u][k] += a[k];
          }
          if (or_) {
            if (acc) {
              float old[V];
              io<T>::unpack(ld_nt(or_ + p * V), old);
#pragma unroll
              for (int k = 0; k < V; ++k) o[k] = acc_add(old[k], o[k]);
            }
            st_nt(or_ + p * V, io<T>::pack(o));
          }
        }
      }
      const int64_t c = sp.packs * V + tid;
      if (c < C) {
        const float a = io<T>::ld(dr + c), b = io<T>::ld(xr + c);
        pp.tl[0] += a * ((b - mu) * rs);
        pp.tl[1] += a;
        if (or_) store_acc1<T>(or_ + c, dxv(a, gamma[c], b), acc != 0);
      }
    } else if (or_) {
      row_pass<T, 2, SUB, true>(src, sp, C,
          [&](int64_t c) { store_acc1<T>(or_ + c, dxv(io<T>::ld(dr + c), gamma[c], io<T>::ld(xr + c)), acc != 0); },
          [&](int64_t c0, const uint4 (&q)[2]) {
            float a[V], b[V], g[V], o[V];
            io<T>::unpack(q[0], a);
            io<T>::unpack(q[1], b);
            load_par<V>(gamma, c0, C, g);
#pragma unroll
            for (int k = 0; k < V; ++k) o[k] = dxv(a[k], g[k], b[k]);
            if (acc) {
              float old[V];
              io<T>::unpack(ld_nt(or_ + c0), old);
#pragma unroll
              for (int k = 0; k < V; ++k) o[k] = acc_add(old[k], o[k]);
            }
            st_nt(or_ + c0, io<T>::pack(o));
          });
    }
  }
  if constexpr (PK > 0)
    if (part) pp.write(part, packs_fixed, C);
}

// ======================================================= register rows
// Rows of at most NPR packs per thread are loaded once into registers: thread
// t holds packs t + k*ST (k < NPR) of each tensor, and at most one head and
// one tail element (both are shorter than a pack).  Both passes then run on
// the registers: HBM sees each byte once, no second read.  The tensors'
// rows must start at the same offset modulo 16 bytes (checked on the host).

template <typename T, int NTS, int NPR, int BT = ST>
struct RegRow {
  static constexpr int V = io<T>::VEC;
  uint4 q[NPR][NTS];
  float h[NTS], t[NTS];     // this thread's head element (column tid) and tail element
  int64_t tc;                // column of the tail element
  bool hv, tv;
  __device__ __forceinline__ void load(const T* const (&src)[NTS], const Split& sp, int64_t C) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      const int64_t p = tid + (int64_t)k * BT;
#pragma unroll
      for (int i = 0; i < NTS; ++i) q[k][i] = p < sp.packs ? ld_nt(src[i] + sp.head + p * V) : make_uint4(0, 0, 0, 0);
    }
    hv = tid < sp.head;
    tc = sp.head + sp.packs * V + tid;
    tv = tc < C;
#pragma unroll
    for (int i = 0; i < NTS; ++i) {
      h[i] = hv ? io<T>::ld(src[i] + tid) : 0.f;
      t[i] = tv ? io<T>::ld(src[i] + tc) : 0.f;
    }
  }
  // An empty asm that claims to rewrite the raw packs: values unpacked
  // from them before it cannot be kept past it, so only the raw packs stay
  // live across a block reduction (half the registers of bf16 values as
  // f32) and each pass unpacks again where it uses them.
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int k = 0; k < NPR; ++k)
#pragma unroll
      for (int i = 0; i < NTS; ++i) asm volatile("" : "+v"(q[k][i].x), "+v"(q[k][i].y), "+v"(q[k][i].z), "+v"(q[k][i].w));
  }
  // The packs from an LDS copy ([tensor][k][thread], 16 bytes each), the
  // head and tail elements from global memory.
  __device__ __forceinline__ void load_lds(const unsigned* bufw, const T* const (&src)[NTS], const Split& sp,
                                           int64_t C) {
    const uint4* buf = reinterpret_cast<const uint4*>(bufw);
    const int tid = threadIdx.x;
    // every slot is read (a pack past the row is read but never used), so
    // the reads are all in flight at once
#pragma unroll
    for (int k = 0; k < NPR; ++k)
#pragma unroll
      for (int i = 0; i < NTS; ++i) q[k][i] = buf[(i * NPR + k) * BT + tid];
    hv = tid < sp.head;
    tc = sp.head + sp.packs * V + tid;
    tv = tc < C;
#pragma unroll
    for (int i = 0; i < NTS; ++i) {
      h[i] = hv ? io<T>::ld(src[i] + tid) : 0.f;
      t[i] = tv ? io<T>::ld(src[i] + tc) : 0.f;
    }
  }
  // load_lds for f32 rows with no head (16-byte aligned starts) whose tail
  // elements are in the copy too (after the packs), with the LDS reads
  // written out and waited for in one asm statement: the compiler then sees
  // no read of the copy that a pending global-to-LDS transfer may write, so
  // it adds no wait for every outstanding vector memory operation in front
  // of them, and the row needs no global load; the caller has already
  // waited for the transfers that wrote the copy.  (Reads and wait share
  // one statement so no output is used before its data has arrived.)
  // Slot J = i*NPR + k (tensor i, pack k) is 16 bytes at J*BT*16 + 16*tid.
  __device__ __forceinline__ void load_lds_direct(const unsigned* bufw, const Split& sp, int64_t C) {
    static_assert(BT == 1024 && NTS == 2 && (NPR == 2 || NPR == 4) && sizeof(T) == 4, "prefetched f32 rows");
    typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
    const unsigned base = (unsigned)(uintptr_t)bufw;
    const unsigned a0 = base + threadIdx.x * 16;
    const unsigned at = base + NTS * NPR * BT * 16 + (threadIdx.x & 3) * 4;   // tail words 4 i + tid (tid < 4)
    u32x4 v[2 * NPR];
    unsigned tw0, tw1;
    if constexpr (NPR == 2) {
      asm volatile(
          "ds_read_b128 %0, %6 offset:0\n\t"
          "ds_read_b128 %1, %6 offset:16384\n\t"
          "ds_read_b128 %2, %6 offset:32768\n\t"
          "ds_read_b128 %3, %6 offset:49152\n\t"
          "ds_read_b32 %4, %7 offset:0\n\t"
          "ds_read_b32 %5, %7 offset:16\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(tw0), "=&v"(tw1)
          : "v"(a0), "v"(at)
          : "memory");
    } else {
      asm volatile(
          "ds_read_b128 %0, %10 offset:0\n\t"
          "ds_read_b128 %1, %10 offset:16384\n\t"
          "ds_read_b128 %2, %10 offset:32768\n\t"
          "ds_read_b128 %3, %10 offset:49152\n\t"
          "ds_read_b128 %4, %11 offset:0\n\t"
          "ds_read_b128 %5, %11 offset:16384\n\t"
          "ds_read_b128 %6, %11 offset:32768\n\t"
          "ds_read_b128 %7, %11 offset:49152\n\t"
          "ds_read_b32 %8, %12 offset:0\n\t"
          "ds_read_b32 %9, %12 offset:16\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]),
            "=&v"(v[7]), "=&v"(tw0), "=&v"(tw1)
          : "v"(a0), "v"(a0 + 65536u), "v"(at)
          : "memory");
    }
#pragma unroll
    for (int j = 0; j < 2 * NPR; ++j) q[j % NPR][j / NPR] = make_uint4(v[j].x, v[j].y, v[j].z, v[j].w);
    // rows of at most 2^31 elements: 32-bit offsets from the row starts
    const int tci = (int)(sp.packs * V) + threadIdx.x;
    hv = false;
    tc = tci;
    tv = tci < C;
    h[0] = h[1] = 0.f;
    t[0] = tv ? __uint_as_float(tw0) : 0.f;
    t[1] = tv ? __uint_as_float(tw1) : 0.f;
  }
  __device__ __forceinline__ bool has(const Split& sp, int k) const { return threadIdx.x + (int64_t)k * BT < sp.packs; }
  __device__ __forceinline__ int64_t col(const Split& sp, int k) const {
    return sp.head + (threadIdx.x + (int64_t)k * BT) * V;
  }
};

template <typename T>
__device__ __forceinline__ void store_pack_acc_full(T* p, float* o, bool acc) {
  constexpr int V = io<T>::VEC;
  if (acc) {
    float old[V];
    io<T>::unpack(ld_nt(p), old);
#pragma unroll
    for (int k = 0; k < V; ++k) o[k] = acc_add(old[k], o[k]);
  }
  st_nt(p, io<T>::pack(o));
}

// softmax backward on register rows: d and y of a row read once (thread t:
// packs t + 1024 k, at most one head and one tail element each), the dot
// product and dx from the registers.  Addresses are a row-uniform base per
// pack slot plus one 32-bit lane offset (rows of at most 65536 elements).
// Up to 4 packs per thread the kernel is held to 64 registers, so two rows
// share a CU.
template <typename T, int NPR>
__global__ __launch_bounds__(ST, NPR <= 4 ? 8 : 1) void sm_bwd_reg(const void* __restrict__ d, int64_t ldd,
                                                                  const void* __restrict__ y, int64_t ldy,
                                                                  void* __restrict__ dx, int64_t lddx, int acc,
                                                                  int64_t R, int64_t C, float alpha) {
  constexpr int V = io<T>::VEC;
  __shared__ float lds[4 * SW];
  int ph = 0;
  const int tid = threadIdx.x, lo = tid * V, Ci = (int)C;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* dr = crow<T>(d, r, ldd);
    const T* yr = crow<T>(y, r, ldy);
    T* xr = wrow<T>(dx, r, lddx);
    const Split sp = split_of<T>(dr, C);
    const int head = (int)sp.head, packs = (int)sp.packs;
    const T* db = dr + head;
    const T* yb = yr + head;
    uint4 qd[NPR], qy[NPR];
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      const bool ok = tid + k * ST < packs;
      qd[k] = ok ? ld_nt(db + k * ST * V + lo) : make_uint4(0, 0, 0, 0);
      qy[k] = ok ? ld_nt(yb + k * ST * V + lo) : make_uint4(0, 0, 0, 0);
    }
    const bool hv = tid < head;
    const int tc = head + packs * V + tid;
    const bool tv = tc < Ci;
    const float hd = hv ? io<T>::ld(dr + tid) : 0.f, hy = hv ? io<T>::ld(yr + tid) : 0.f;
    const float td = tv ? io<T>::ld(dr + tc) : 0.f, ty = tv ? io<T>::ld(yr + tc) : 0.f;
    float dot = hd * hy + td * ty;
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      float a[V], b[V];
      io<T>::unpack(qd[k], a);
      io<T>::unpack(qy[k], b);
#pragma unroll
      for (int e = 0; e < V; ++e) dot += a[e] * b[e];
    }
    dot = group_sum<SW>(dot, lds, ph);
    // only the raw packs stay live across the reduction (as RegRow::pin)
#pragma unroll
    for (int k = 0; k < NPR; ++k) asm volatile("" : "+v"(qd[k].x), "+v"(qd[k].y), "+v"(qd[k].z), "+v"(qd[k].w),
                                                    "+v"(qy[k].x), "+v"(qy[k].y), "+v"(qy[k].z), "+v"(qy[k].w));
    T* xb = xr + head;
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      if (tid + k * ST >= packs) continue;
      float a[V], b[V], o[V];
      io<T>::unpack(qd[k], a);
      io<T>::unpack(qy[k], b);
#pragma unroll
      for (int e = 0; e < V; ++e) o[e] = alpha * b[e] * (a[e] - dot);
      store_pack_acc_full<T>(xb + k * ST * V + lo, o, acc != 0);
    }
    if (hv) store_acc1<T>(xr + tid, alpha * hy * (hd - dot), acc != 0);
    if (tv) store_acc1<T>(xr + tc, alpha * ty * (td - dot), acc != 0);
  }
}

// Forwards on register rows of at most 8 packs per thread (f32 rows up to
// 32768 columns, bf16 up to 65536): the row is read from HBM once and both
// passes (statistics, then the output) run on the registers.  At most 32
// registers of packs, so the softmax (and the narrower norms) are held to
// 64 registers and two blocks share a CU: one block's loads are in flight
// while the other reduces and writes.  Addresses are a row-uniform base per pack slot plus
// one 32-bit lane offset (the rows are at most 65536 wide).
template <typename T, int NPR>
struct FwdRow {
  static constexpr int V = io<T>::VEC;
  uint4 q[NPR];
  float h, t;         // head element (column tid) and tail element (column tc)
  int tc;
  bool hv, tv;
  __device__ __forceinline__ void load(const T* xr, const Split& sp, int C) {
    const int tid = threadIdx.x, lo = tid * V;
    const T* xb = xr + sp.head;
#pragma unroll
    for (int k = 0; k < NPR; ++k) q[k] = has(sp, k) ? ld_nt(xb + k * ST * V + lo) : make_uint4(0, 0, 0, 0);
    hv = tid < sp.head;
    tc = (int)(sp.head + sp.packs * V) + tid;
    tv = tc < C;
    h = hv ? io<T>::ld(xr + tid) : 0.f;
    t = tv ? io<T>::ld(xr + tc) : 0.f;
  }
  __device__ __forceinline__ bool has(const Split& sp, int k) const { return (int)threadIdx.x + k * ST < (int)sp.packs; }
  // the same empty-asm barrier as RegRow::pin
  __device__ __forceinline__ void pin() {
#pragma unroll
    for (int k = 0; k < NPR; ++k) asm volatile("" : "+v"(q[k].x), "+v"(q[k].y), "+v"(q[k].z), "+v"(q[k].w));
  }
};

template <typename T, int NPR, bool CAUSAL>
__global__ __launch_bounds__(ST, 8) void sm_fwd_reg(const void* __restrict__ x, int64_t ldx, void* __restrict__ y,
                                                    int64_t ldy, int64_t R, int64_t C, float alpha, int causal,
                                                    int seq_len) {
  constexpr int V = io<T>::VEC;
  __shared__ float ms[2][2][SW];
  int ph = 0;
  const float sl = alpha * LOG2E;
  const int tid = threadIdx.x, lo = tid * V, Ci = (int)C;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* xr = crow<T>(x, r, ldx);
    T* yr = wrow<T>(y, r, ldy);
    const int lim = CAUSAL ? min(Ci, (int)(r % seq_len) + 1) : Ci;
    const Split sp = split_of<T>(xr, C);
    FwdRow<T, NPR> rr;
    rr.load(xr, sp, Ci);
    // base-2 scaled scores; columns at or past the causal limit are -inf.
    // Pack slot k holds columns head + k*ST*V + lo + e: its limit relative
    // to the lane offset is row-uniform.
    auto lim_k = [&](int k) { return lim - (int)sp.head - k * ST * V; };
    auto sc = [&](float v, int c, int l) { return !CAUSAL || c < l ? v * sl : -__builtin_inff(); };
    // this thread's online (max, sum) state, one pack at a time
    float m = fmaxf(rr.hv ? sc(rr.h, tid, lim) : -__builtin_inff(), rr.tv ? sc(rr.t, rr.tc, lim) : -__builtin_inff());
    float s = (rr.hv && (!CAUSAL || tid < lim) ? __builtin_amdgcn_exp2f(rr.h * sl - m) : 0.f) +
              (rr.tv && (!CAUSAL || rr.tc < lim) ? __builtin_amdgcn_exp2f(rr.t * sl - m) : 0.f);
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      if (!rr.has(sp, k)) continue;
      float v[V];
      io<T>::unpack(rr.q[k], v);
      const int l = lim_k(k);
      float pm = -__builtin_inff();
#pragma unroll
      for (int e = 0; e < V; ++e) {
        v[e] = sc(v[e], lo + e, l);
        pm = fmaxf(pm, v[e]);
      }
      if (CAUSAL && pm == -__builtin_inff()) continue;    // the whole pack is past the causal limit
      if (pm > m) { s *= __builtin_amdgcn_exp2f(m - pm); m = pm; }
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < V; ++e) a += __builtin_amdgcn_exp2f(v[e] - m);
      s += a;
    }
    rr.pin();
    const MS tot = block_merge(MS{m, s}, ms, ph);
    const float inv = 1.f / tot.s, mm = tot.m;
    auto out = [&](float v, int c, int l) { return !CAUSAL || c < l ? __builtin_amdgcn_exp2f(fmaf(v, sl, -mm)) * inv : 0.f; };
    T* yb = yr + sp.head;
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      if (!rr.has(sp, k)) continue;
      float v[V];
      io<T>::unpack(rr.q[k], v);
      const int l = lim_k(k);
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] = out(v[e], lo + e, l);
      st_nt(yb + k * ST * V + lo, io<T>::pack(v));
    }
    if (rr.hv) io<T>::st(yr + tid, out(rr.h, tid, lim));
    if (rr.tv) io<T>::st(yr + rr.tc, out(rr.t, rr.tc, lim));
  }
}

// The norm forwards on register rows fit 64 registers without spilling
// (two blocks per CU) up to these packs per thread (es: element bytes);
// wider rows take the streaming kernels, which measured faster there than
// a register row at one block per CU (bf16 layer_norm, 50257 columns:
// 0.70 vs 0.76 ms).
__host__ __device__ constexpr bool norm_fwd_fits(int es, int npr, bool ln) {
  return ln ? (es == 4 ? npr <= 2 : npr <= 1) : npr <= 4;
}

// rms_norm (LN = false; st0 = inv_rms) or layer_norm (st0 = mean, st1 =
// rstd; the variance about the mean, a second pass over the registers).
template <typename T, int NPR, bool LN>
__global__ __launch_bounds__(ST, 8) void norm_fwd_reg(const void* __restrict__ x, int64_t ldx,
                                                      const float* __restrict__ gamma, const float* __restrict__ beta,
                                                      void* __restrict__ y, int64_t ldy, float* __restrict__ st0,
                                                      int64_t ld0, float* __restrict__ st1, int64_t ld1, int64_t R,
                                                      int64_t C, float eps, float invC) {
  constexpr int V = io<T>::VEC;
  __shared__ float lds[4 * SW];
  int ph = 0;
  const int tid = threadIdx.x, lo = tid * V, Ci = (int)C;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* xr = crow<T>(x, r, ldx);
    T* yr = wrow<T>(y, r, ldy);
    const Split sp = split_of<T>(xr, C);
    FwdRow<T, NPR> rr;
    rr.load(xr, sp, Ci);
    // layer_norm: the mean first (empty slots hold 0 and add nothing)
    float mu = 0.f;
    if constexpr (LN) {
      float a = rr.h + rr.t;
#pragma unroll
      for (int k = 0; k < NPR; ++k) {
        float v[V];
        io<T>::unpack(rr.q[k], v);
#pragma unroll
        for (int e = 0; e < V; ++e) a += v[e];
      }
      rr.pin();
      mu = group_sum<SW>(a, lds, ph) * invC;
    }
    // sum of squares (rms_norm) or of squared deviations about the mean
    auto dev = [&](float v) { return LN ? v - mu : v; };
    float q2 = (rr.hv ? dev(rr.h) * dev(rr.h) : 0.f) + (rr.tv ? dev(rr.t) * dev(rr.t) : 0.f);
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      if (!rr.has(sp, k)) continue;
      float v[V];
      io<T>::unpack(rr.q[k], v);
#pragma unroll
      for (int e = 0; e < V; ++e) q2 += dev(v[e]) * dev(v[e]);
    }
    rr.pin();
    const float rs = rsqrtf(group_sum<SW>(q2, lds, ph) * invC + eps);
    if (tid == 0) {
      if constexpr (LN) { st0[r * ld0] = mu; st1[r * ld1] = rs; }
      else st0[r * ld0] = rs;
    }
    T* yb = yr + sp.head;
    const float* gb = gamma + sp.head;
    const float* bb = LN ? beta + sp.head : nullptr;
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      if (!rr.has(sp, k)) continue;
      float v[V], g[V], b[V];
      io<T>::unpack(rr.q[k], v);
      load_par<V>(gb + k * ST * V, lo, (int64_t)(Ci - (int)sp.head - k * ST * V), g);
      if constexpr (LN) load_par<V>(bb + k * ST * V, lo, (int64_t)(Ci - (int)sp.head - k * ST * V), b);
#pragma unroll
      for (int e = 0; e < V; ++e) v[e] = LN ? dev(v[e]) * rs * g[e] + b[e] : v[e] * rs * g[e];
      st_nt(yb + k * ST * V + lo, io<T>::pack(v));
    }
    if (rr.hv) io<T>::st(yr + tid, LN ? dev(rr.h) * rs * gamma[tid] + beta[tid] : rr.h * rs * gamma[tid]);
    if (rr.tv) io<T>::st(yr + rr.tc, LN ? dev(rr.t) * rs * gamma[rr.tc] + beta[rr.tc] : rr.t * rs * gamma[rr.tc]);
  }
}

// f32 row r's packs of d and x into the LDS copy [tensor][k][thread] (16-byte
// packs, NPR <= 4 per thread) by global_load_lds: 16 bytes per lane, no
// registers held.  The row's tail elements (C - 4*packs < 4 of each tensor)
// follow the packs: d's at word 8*npr*ST, x's 4 words on.
__device__ __forceinline__ void reg_row_dma_f32(const float* dr, const float* xr, int64_t packs, int npr, int64_t C,
                                                unsigned* __restrict__ buf) {
  const int tid = threadIdx.x, w = __builtin_amdgcn_readfirstlane(tid / WAVE);
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // uniform base of the k-th run of ST packs, plus one lane offset shared by all k
    const float* dk = dr + k * ST * 4;
    const float* xk = xr + k * ST * 4;
    if (k < npr && tid + k * ST < packs) {
      __builtin_amdgcn_global_load_lds(dk + tid * 4, buf + 4 * (k * ST + w * WAVE), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(xk + tid * 4, buf + 4 * ((npr + k) * ST + w * WAVE), 16, 0, 0);
    }
  }
  // 4 bytes per lane: lane l of wave 0 writes word l of the tail region
  if (tid < C - packs * 4) {
    __builtin_amdgcn_global_load_lds(dr + packs * 4 + tid, buf + 8 * npr * ST, 4, 0, 0);
    __builtin_amdgcn_global_load_lds(xr + packs * 4 + tid, buf + 8 * npr * ST + 4, 4, 0, 0);
  }
}

// rms_norm / layer_norm backward on register rows (LN = false: rms_norm).
// OWN: every row starts 16-byte aligned (no head), so thread t's columns
// are the same in every row and it keeps their parameter-gradient partial
// sums; otherwise dx only (the partials come from the column pass).
//
// f32 rows with owned partials (every row 16-byte aligned, so the split is
// the same for every row) are prefetched (PF): a block copies row r (packs
// and tail elements) from its LDS copy into registers and at once sends its
// next row into the LDS copy (2 NPR 16-byte packs per thread: at most
// 128 KB), so that transfer runs under row r's first pass.  The row then
// needs no global load: gamma is the same for every row of a thread and is
// loaded once.  vmcnt counts the vector memory operations in issue order,
// so the wait at the top of a row leaves the previous row's stores (issued
// after the transfer, counted in nvm) in flight.
template <typename T, int NPR, bool LN, bool OWN>
__global__ __launch_bounds__(ST) void norm_bwd_reg(const void* __restrict__ d, int64_t ldd, const void* __restrict__ x,
                                                   int64_t ldx, const float* __restrict__ gamma,
                                                   const float* __restrict__ st0, int64_t ld0,
                                                   const float* __restrict__ st1, int64_t ld1, void* __restrict__ dx,
                                                   int64_t lddx, int acc, float* __restrict__ part, int64_t R,
                                                   int64_t C, float invC) {
  constexpr int V = io<T>::VEC, NP = LN ? 2 : 1;
  constexpr bool PF = OWN && sizeof(T) == 4;
  __shared__ float lds[4 * SW];
  __shared__ __align__(16) unsigned buf[PF ? 2 * NPR * ST * 4 + 8 : ST * 4];   // [tensor][k][thread] packs, tails
  int ph = 0;
  OwnedPartials<NP, OWN ? NPR : 1, V> pp;
  pp.zero();
  int64_t packs_fixed = 0;
  const int tid = threadIdx.x;
  // PF: this thread's gamma packs (columns (tid + k*ST)*V of every row)
  float gk[PF ? NPR : 1][V];
  int nvm = 0;                          // PF: vector memory operations since the last transfer
  float gtf = 0.f;                      // PF: gamma at this thread's tail column
  if constexpr (PF) {
    const int64_t tcf = C / V * V + tid;
    if (tcf < C) gtf = gamma[tcf];
    const bool ga = (((uintptr_t)gamma) & 15) == 0;
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      const int c0 = (tid + k * ST) * V;   // < 2^31: OWN rows are at most 16384 wide
      if (c0 + V > C) continue;
      if (ga) {
        const float4 g4 = *reinterpret_cast<const float4*>(gamma + c0);
        gk[k][0] = g4.x; gk[k][1] = g4.y; gk[k][2] = g4.z; gk[k][3] = g4.w;
      } else {
        load_par<V>(gamma, c0, C, gk[k]);
      }
    }
    if (blockIdx.x < R)
      reg_row_dma_f32(crow<float>(d, blockIdx.x, ldd), crow<float>(x, blockIdx.x, ldx),
                      split_of<T>(crow<T>(d, blockIdx.x, ldd), C).packs, NPR, C, buf);
  }
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* dr = crow<T>(d, r, ldd);
    const T* xr = crow<T>(x, r, ldx);
    T* orr = dx ? wrow<T>(dx, r, lddx) : nullptr;
    const Split sp = split_of<T>(dr, C);
    packs_fixed = sp.packs;
    const T* src[2] = {dr, xr};
    RegRow<T, 2, NPR> rr;
    if constexpr (PF) {
      wait_vmcnt_at_most(nvm);          // this thread's transfers of row r have landed
      lds_barrier();                    // ... and every other thread's
      rr.load_lds_direct(buf, sp, C);
    } else {
      rr.load(src, sp, C);
    }
    // rms_norm: st0 = inv_rms; layer_norm: st0 = mean, st1 = rstd
    const float s0 = st0[r * ld0], s1v = LN ? st1[r * ld1] : 0.f;
    auto xhat = [&](float xv) { return LN ? (xv - s0) * s1v : xv; };
    const float gh = !PF && rr.hv ? gamma[tid] : 0.f, gt = PF ? gtf : rr.tv ? gamma[rr.tc] : 0.f;
    if constexpr (PF) {
      lds_barrier();                    // every thread's reads of buf complete before anyone refills it
      const int64_t rn = r + gridDim.x;
      if (rn < R) reg_row_dma_f32(crow<float>(d, rn, ldd), crow<float>(x, rn, ldx), sp.packs, NPR, C, buf);
      nvm = 0;
    }
    float a1 = rr.h[0] * gh + rr.t[0] * gt;                                   // layer_norm: sum d*gamma
    float a2 = rr.h[0] * gh * xhat(rr.h[1]) + rr.t[0] * gt * xhat(rr.t[1]);   // sum d*gamma*xhat (rms: *x)
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      if (!rr.has(sp, k)) continue;
      float a[V], b[V], g[V];
      io<T>::unpack(rr.q[k][0], a);
      io<T>::unpack(rr.q[k][1], b);
      if constexpr (PF) {
#pragma unroll
        for (int e = 0; e < V; ++e) g[e] = gk[k][e];
      } else {
        load_par<V>(gamma, rr.col(sp, k), C, g);
      }
#pragma unroll
      for (int e = 0; e < V; ++e) {
        const float gv = a[e] * g[e];
        a1 += gv;
        a2 += gv * xhat(b[e]);
        if constexpr (PF) {
          pp.pk[0][k][e] += LN ? a[e] * xhat(b[e]) : a[e] * b[e] * s0;
          if constexpr (LN) pp.pk[NP - 1][k][e] += a[e];
          a[e] = gv;
        }
      }
      if constexpr (PF) rr.q[k][0] = io<T>::pack(a);       // d * gamma from here on
    }
    // the next row's transfer is waited for before the reduction: letting it
    // run on under the reduction and this row's stores measured slower
    // (16384-wide f32 rows: 625 -> 615 us)
    if constexpr (PF) wait_vmcnt_at_most(0);
    float c1, mg, mgx;
    if constexpr (LN) {
      group_sum2<SW>(a1, a2, lds, ph);
      mg = a1 * invC;
      mgx = a2 * invC;
      c1 = 0.f;
    } else {
      a2 = group_sum<SW>(a2, lds, ph);
      c1 = s0 * s0 * s0 * invC * a2;
      mg = mgx = 0.f;
    }
    rr.pin();
    // dx from d * gamma (dg) and x
    auto dxg = [&](float dg, float xv) { return LN ? s1v * (dg - mg - xhat(xv) * mgx) : s0 * dg - xv * c1; };
#pragma unroll
    for (int k = 0; k < NPR; ++k) {
      if (!rr.has(sp, k)) continue;
      float a[V], b[V], o[V];
      io<T>::unpack(rr.q[k][0], a);
      io<T>::unpack(rr.q[k][1], b);
      // PF rows are at most 16384 wide: a 32-bit offset from the row start
      const int64_t c0 = PF ? (int64_t)(int)rr.col(sp, k) : rr.col(sp, k);
      if constexpr (PF) {
#pragma unroll
        for (int e = 0; e < V; ++e) o[e] = dxg(a[e], b[e]);
      } else {
        float g[V];
        load_par<V>(gamma, c0, C, g);
#pragma unroll
        for (int e = 0; e < V; ++e) {
          o[e] = dxg(a[e] * g[e], b[e]);
          if constexpr (OWN) {
            pp.pk[0][k][e] += LN ? a[e] * xhat(b[e]) : a[e] * b[e] * s0;
            if constexpr (LN) pp.pk[NP - 1][k][e] += a[e];
          }
        }
      }
      if (orr) {
        store_pack_acc_full<T>(orr + c0, o, acc != 0);
        nvm += acc ? 2 : 1;
      }
    }
    if (!PF && rr.hv && orr) {
      store_acc1<T>(orr + tid, dxg(rr.h[0] * gh, rr.h[1]), acc != 0);
      nvm += acc ? 2 : 1;
    }
    if (rr.tv) {
      if (orr) {
        store_acc1<T>(orr + rr.tc, dxg(rr.t[0] * gt, rr.t[1]), acc != 0);
        nvm += acc ? 2 : 1;
      }
      if constexpr (OWN) {
        pp.tl[0] += LN ? rr.t[0] * xhat(rr.t[1]) : rr.t[0] * rr.t[1] * s0;
        if constexpr (LN) pp.tl[NP - 1] += rr.t[0];
      }
    }
  }
  if constexpr (OWN)
    if (part) pp.write(part, packs_fixed, C);
}

bool al16(const xt_tensor* t) {
  if (!t) return true;
  const int es = t->dtype == XT_F32 ? 4 : 2;
  return (((uintptr_t)t->data) & 15) == 0 && ((t->ld * es) & 15) == 0;
}

// Every row of a and of b starts at the same offset modulo 16 bytes.
bool same_phase(const xt_tensor& a, const xt_tensor* b) {
  if (!b) return true;
  const int es = a.dtype == XT_F32 ? 4 : 2;
  return ((((uintptr_t)a.data) - ((uintptr_t)b->data)) & 15) == 0 && (((a.ld - b->ld) * es) & 15) == 0;
}

// Packs per thread a register row needs (the head takes at most V - 1 more
// elements, which never add a pack): 1, 2, 4, 8 or 16; 0 past `cap`.
int reg_npr(int dtype, int64_t C, int cap, int bt = ST) {
  const int V = dtype == XT_F32 ? 4 : 8;
  const int64_t per = (C / V + bt - 1) / bt;
  int n = 1;
  while (n < per) n *= 2;
  return n <= cap ? n : 0;
}

// Packs per thread when every row starts 16-byte aligned and has at most
// 4 (f32) / 2 (bf16) packs per thread, i.e. up to 16384 columns; 0
// otherwise (no owned partials).  More packs per thread spill registers.
int owned_pk(int dtype, int64_t C, bool fixed) {
  const int V = dtype == XT_F32 ? 4 : 8;
  if (!fixed) return 0;
  const int64_t per = (C / V + ST - 1) / ST;
  const int cap = dtype == XT_F32 ? 4 : 2;
  if (per > cap) return 0;
  return per <= 2 ? 2 : 4;
}

#define XT_NPR_CASES(NPRV, MAXN, ...)                                               \
  do {                                                                             \
    if (NPRV == 1) { constexpr int NPR = 1; __VA_ARGS__; }                         \
    else if (NPRV == 2) { constexpr int NPR = 2; __VA_ARGS__; }                    \
    else if (NPRV == 4) { constexpr int NPR = 4; __VA_ARGS__; }                    \
    else if (NPRV == 8 && MAXN >= 8) { constexpr int NPR = (MAXN >= 8 ? 8 : 1); __VA_ARGS__; } \
    else if (MAXN >= 16) { constexpr int NPR = (MAXN >= 16 ? 16 : 1); __VA_ARGS__; } \
  } while (0)

}  // namespace

int stream_bwd_grid(int64_t R) { return (int)std::max<int64_t>(1, std::min<int64_t>(R, STREAM_BWD_GRID)); }

bool stream_owns_partials(int dtype, int64_t C, const xt_tensor& d, const xt_tensor& x, const xt_tensor* dx) {
  return owned_pk(dtype, C, al16(&d) && al16(&x) && al16(dx)) > 0;
}

hipError_t launch_sm_fwd_stream(const xt_tensor& x, const xt_tensor& y, float alpha, int causal, int seq_len,
                                int grid, hipStream_t s) {
  const int npr = same_phase(x, &y) ? reg_npr(x.dtype, x.cols, 8) : 0;
  if (npr) {
    if (x.dtype == XT_F32)
      XT_NPR_CASES(npr, 8, {
        auto kf = causal ? sm_fwd_reg<float, NPR, true> : sm_fwd_reg<float, NPR, false>;
        kf<<<grid, ST, 0, s>>>(x.data, x.ld, y.data, y.ld, x.rows, x.cols, alpha, causal, seq_len);
      });
    else
      XT_NPR_CASES(npr, 8, {
        auto kf = causal ? sm_fwd_reg<bf16_t, NPR, true> : sm_fwd_reg<bf16_t, NPR, false>;
        kf<<<grid, ST, 0, s>>>(x.data, x.ld, y.data, y.ld, x.rows, x.cols, alpha, causal, seq_len);
      });
    return hipGetLastError();
  }
  if (x.dtype == XT_F32)
    sm_fwd_stream<float><<<grid, ST, 0, s>>>(x.data, x.ld, y.data, y.ld, x.rows, x.cols, alpha, causal, seq_len);
  else
    sm_fwd_stream<bf16_t><<<grid, ST, 0, s>>>(x.data, x.ld, y.data, y.ld, x.rows, x.cols, alpha, causal, seq_len);
  return hipGetLastError();
}

hipError_t launch_sm_bwd_stream(const xt_tensor& d, const xt_tensor& y, const xt_tensor& dx, bool acc, float alpha,
                                int grid, hipStream_t s) {
  const int npr = same_phase(d, &y) && same_phase(d, &dx) ? reg_npr(d.dtype, d.cols, 8) : 0;
  if (npr) {
    if (d.dtype == XT_F32)
      XT_NPR_CASES(npr, 8, sm_bwd_reg<float, NPR><<<grid, ST, 0, s>>>(d.data, d.ld, y.data, y.ld, dx.data, dx.ld, acc,
                                                                      d.rows, d.cols, alpha));
    else
      XT_NPR_CASES(npr, 8, sm_bwd_reg<bf16_t, NPR><<<grid, ST, 0, s>>>(d.data, d.ld, y.data, y.ld, dx.data, dx.ld, acc,
                                                                       d.rows, d.cols, alpha));
    return hipGetLastError();
  }
  if (d.dtype == XT_F32)
    sm_bwd_stream<float><<<grid, ST, 0, s>>>(d.data, d.ld, y.data, y.ld, dx.data, dx.ld, acc, d.rows, d.cols, alpha);
  else
    sm_bwd_stream<bf16_t><<<grid, ST, 0, s>>>(d.data, d.ld, y.data, y.ld, dx.data, dx.ld, acc, d.rows, d.cols, alpha);
  return hipGetLastError();
}

hipError_t launch_rms_fwd_stream(const xt_tensor& x, const float* gamma, const xt_tensor& y, const xt_tensor& ir,
                                 float eps, int grid, hipStream_t s) {
  const float invC = 1.0f / (float)x.cols;
  const int npr = same_phase(x, &y) ? reg_npr(x.dtype, x.cols, 8) : 0;
  if (npr && norm_fwd_fits(x.dtype == XT_F32 ? 4 : 2, npr, false)) {
    if (x.dtype == XT_F32)
      XT_NPR_CASES(npr, 4, norm_fwd_reg<float, NPR, false><<<grid, ST, 0, s>>>(x.data, x.ld, gamma, nullptr, y.data, y.ld,
          (float*)ir.data, ir.ld, nullptr, 0, x.rows, x.cols, eps, invC));
    else
      XT_NPR_CASES(npr, 4, norm_fwd_reg<bf16_t, NPR, false><<<grid, ST, 0, s>>>(x.data, x.ld, gamma, nullptr, y.data, y.ld,
          (float*)ir.data, ir.ld, nullptr, 0, x.rows, x.cols, eps, invC));
    return hipGetLastError();
  }
  if (x.dtype == XT_F32)
    rms_fwd_stream<float><<<grid, ST, 0, s>>>(x.data, x.ld, gamma, y.data, y.ld, (float*)ir.data, ir.ld, x.rows,
                                              x.cols, eps, invC);
  else
    rms_fwd_stream<bf16_t><<<grid, ST, 0, s>>>(x.data, x.ld, gamma, y.data, y.ld, (float*)ir.data, ir.ld, x.rows,
                                               x.cols, eps, invC);
  return hipGetLastError();
}

hipError_t launch_ln_fwd_stream(const xt_tensor& x, const float* gamma, const float* beta, const xt_tensor& y,
                                const xt_tensor& mean, const xt_tensor& rstd, float eps, int grid, hipStream_t s) {
  const float invC = 1.0f / (float)x.cols;
  const int npr = same_phase(x, &y) ? reg_npr(x.dtype, x.cols, 8) : 0;
  if (npr && norm_fwd_fits(x.dtype == XT_F32 ? 4 : 2, npr, true)) {
    if (x.dtype == XT_F32)
      XT_NPR_CASES(npr, 4, norm_fwd_reg<float, NPR, true><<<grid, ST, 0, s>>>(x.data, x.ld, gamma, beta, y.data, y.ld,
          (float*)mean.data, mean.ld, (float*)rstd.data, rstd.ld, x.rows, x.cols, eps, invC));
    else
      XT_NPR_CASES(npr, 4, norm_fwd_reg<bf16_t, NPR, true><<<grid, ST, 0, s>>>(x.data, x.ld, gamma, beta, y.data, y.ld,
          (float*)mean.data, mean.ld, (float*)rstd.data, rstd.ld, x.rows, x.cols, eps, invC));
    return hipGetLastError();
  }
  if (x.dtype == XT_F32)
    ln_fwd_stream<float><<<grid, ST, 0, s>>>(x.data, x.ld, gamma, beta, y.data, y.ld, (float*)mean.data, mean.ld,
                                             (float*)rstd.data, rstd.ld, x.rows, x.cols, eps, invC);
  else
    ln_fwd_stream<bf16_t><<<grid, ST, 0, s>>>(x.data, x.ld, gamma, beta, y.data, y.ld, (float*)mean.data, mean.ld,
                                              (float*)rstd.data, rstd.ld, x.rows, x.cols, eps, invC);
  return hipGetLastError();
}

// part: the block partial rows of dgamma when the split is fixed (owned
// partials); otherwise the caller computes them with a column pass.
#define XT_STREAM_PK(DT, PKV, ...)                                                   \
  do {                                                                              \
    if (DT == XT_F32) {                                                             \
      using T = float;                                                              \
      if (PKV == 0) { constexpr int PK = 0; __VA_ARGS__; }                          \
      else if (PKV == 2) { constexpr int PK = 2; __VA_ARGS__; }                     \
      else { constexpr int PK = 4; __VA_ARGS__; }                                   \
    } else {                                                                        \
      using T = bf16_t;                                                             \
      if (PKV == 0) { constexpr int PK = 0; __VA_ARGS__; }                          \
      else { constexpr int PK = 2; __VA_ARGS__; }                                   \
    }                                                                               \
  } while (0)

namespace {
// Launches the register-row backward when the rows fit (up to 8 packs per
// thread; with owned partials, the owned_pk sizes); returns false to leave
// the row to the two-pass kernels.  part != nullptr only with owned
// partials (pk > 0).
template <bool LN>
bool norm_bwd_reg_launch(const xt_tensor& d, const xt_tensor& x, const float* gamma, const float* st0, int64_t ld0,
                         const float* st1, int64_t ld1, const xt_tensor* dx, bool acc, float* part, int pk, int grid,
                         hipStream_t s) {
  const int64_t R = d.rows, C = d.cols;
  if (!same_phase(d, &x) || !same_phase(d, dx)) return false;
  const float invC = 1.0f / (float)C;
  void* dxp = dx ? dx->data : nullptr;
  const int64_t lddx = dx ? dx->ld : 0;
  if (part) {
    // owned partials: NPR = pk packs per thread
    if (d.dtype == XT_F32) {
      if (pk == 2) norm_bwd_reg<float, 2, LN, true><<<grid, ST, 0, s>>>(d.data, d.ld, x.data, x.ld, gamma, st0, ld0, st1, ld1, dxp, lddx, acc, part, R, C, invC);
      else norm_bwd_reg<float, 4, LN, true><<<grid, ST, 0, s>>>(d.data, d.ld, x.data, x.ld, gamma, st0, ld0, st1, ld1, dxp, lddx, acc, part, R, C, invC);
    } else {
      norm_bwd_reg<bf16_t, 2, LN, true><<<grid, ST, 0, s>>>(d.data, d.ld, x.data, x.ld, gamma, st0, ld0, st1, ld1, dxp, lddx, acc, part, R, C, invC);
    }
    return true;
  }
  if (!dx) return true;                 // no dx and no owned partials: nothing for this kernel
  const int npr = reg_npr(d.dtype, C, 8);
  if (!npr) return false;
  if (d.dtype == XT_F32)
    XT_NPR_CASES(npr, 8, norm_bwd_reg<float, NPR, LN, false><<<grid, ST, 0, s>>>(d.data, d.ld, x.data, x.ld, gamma, st0, ld0, st1, ld1, dxp, lddx, acc, nullptr, R, C, invC));
  else
    XT_NPR_CASES(npr, 8, norm_bwd_reg<bf16_t, NPR, LN, false><<<grid, ST, 0, s>>>(d.data, d.ld, x.data, x.ld, gamma, st0, ld0, st1, ld1, dxp, lddx, acc, nullptr, R, C, invC));
  return true;
}
}  // namespace

hipError_t launch_rms_bwd_stream(const xt_tensor& d, const xt_tensor& x, const float* gamma, const xt_tensor& ir,
                                 const xt_tensor* dx, bool acc_dx, float* part, int grid, hipStream_t s) {
  const int64_t R = d.rows, C = d.cols;
  const float invC = 1.0f / (float)C;
  const int pk = part ? owned_pk(d.dtype, C, al16(&d) && al16(&x) && al16(dx)) : 0;
  if (norm_bwd_reg_launch<false>(d, x, gamma, (const float*)ir.data, ir.ld, nullptr, 0, dx, acc_dx, pk ? part : nullptr,
                                 pk, grid, s))
    return hipGetLastError();
  XT_STREAM_PK(d.dtype, pk,
      rms_bwd_stream<T, PK><<<grid, ST, 0, s>>>(d.data, d.ld, x.data, x.ld, gamma, (const float*)ir.data, ir.ld,
                                                dx ? dx->data : nullptr, dx ? dx->ld : 0, acc_dx, pk ? part : nullptr,
                                                R, C, invC));
  return hipGetLastError();
}

hipError_t launch_ln_bwd_stream(const xt_tensor& d, const xt_tensor& x, const float* gamma, const xt_tensor& mean,
                                const xt_tensor& rstd, const xt_tensor* dx, bool acc_dx, float* part, int grid,
                                hipStream_t s) {
  const int64_t R = d.rows, C = d.cols;
  const float invC = 1.0f / (float)C;
  const int pk = part ? owned_pk(d.dtype, C, al16(&d) && al16(&x) && al16(dx)) : 0;
  if (norm_bwd_reg_launch<true>(d, x, gamma, (const float*)mean.data, mean.ld, (const float*)rstd.data, rstd.ld, dx,
                                acc_dx, pk ? part : nullptr, pk, grid, s))
    return hipGetLastError();
  XT_STREAM_PK(d.dtype, pk,
      ln_bwd_stream<T, PK><<<grid, ST, 0, s>>>(d.data, d.ld, x.data, x.ld, gamma, (const float*)mean.data, mean.ld,
                                               (const float*)rstd.data, rstd.ld, dx ? dx->data : nullptr,
                                               dx ? dx->ld : 0, acc_dx, pk ? part : nullptr, R, C, invC));
  return hipGetLastError();
}

}  // namespace xt
