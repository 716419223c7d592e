// Elementwise forward/backward kernels, in-place gradient accumulation and
// counter-based dropout.
//
// [AE] op-backward table rows add, mul, scale, add_bias, silu, swiglu;
// [BP] k_mlp (GELU) and k_residual_add pairs; [AE] "梯度累加" for the
// accumulate; [DO] "RNG：counter-based" and "dropout 节点的 backward".
//
// All of these are pure HBM streams.  Tensors are walked as rows of 16-byte
// packs (contiguous tensors are first flattened to one long row by the
// host), each thread handling up to 4 packs; the grid is sized to a few
// waves per SIMD.  Rows whose starts are not 16-byte aligned use an
// element-wise path.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace xt {
namespace {

constexpr int EW_BLOCK = 256;
constexpr int EW_UNROLL = 1;   // one pack per thread over a full grid (see common.h)

// ---- loading N elements of type T as f32 (aligned, in bounds) --------------
template <typename T, int N>
__device__ __forceinline__ void load_n(const T* p, float* f) {
  constexpr int BYTES = N * (int)sizeof(T);
  if constexpr (BYTES == 16) {
    io<T>::unpack(*reinterpret_cast<const uint4*>(p), f);
  } else if constexpr (BYTES == 32) {
    io<T>::unpack(reinterpret_cast<const uint4*>(p)[0], f);
    io<T>::unpack(reinterpret_cast<const uint4*>(p)[1], f + io<T>::VEC);
  } else {   // 8 bytes: 4 bf16
    static_assert(BYTES == 8, "pack size");
    const uint2 q = *reinterpret_cast<const uint2*>(p);
    f[0] = __uint_as_float(q.x << 16); f[1] = __uint_as_float(q.x & 0xffff0000u);
    f[2] = __uint_as_float(q.y << 16); f[3] = __uint_as_float(q.y & 0xffff0000u);
  }
}

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }
__device__ __forceinline__ float silu_(float x) { return x * sigmoidf_(x); }
__device__ __forceinline__ float dsilu_(float x) {
  const float s = sigmoidf_(x);
  return s + x * s * (1.0f - s);
}
// Complementary error function from the Chebyshev-fitted formula of
// Numerical Recipes (Press, Teukolsky, Vetterling & Flannery, 2nd ed.,
// section 6.2): for z >= 0, erfc(z) = t exp(-z^2 + P(t)) with t = 1/(1+z/2)
// and P a fixed degree-9 polynomial, fractional error below 1.2e-7 over the
// whole line (so the lower tail of Phi keeps its relative accuracy);
// erfc(-z) = 2 - erfc(z).  Branch-free: one reciprocal, one exp, nine FMAs,
// where the library erfcf takes range-dependent paths that diverge within a
// wave on normally distributed inputs.
__device__ __forceinline__ float erfc_nr(float z) {
  const float a = fabsf(z);
  const float t = __builtin_amdgcn_rcpf(1.0f + 0.5f * a);
  float p = 0.17087277f;
  p = fmaf(p, t, -0.82215223f);
  p = fmaf(p, t, 1.48851587f);
  p = fmaf(p, t, -1.13520398f);
  p = fmaf(p, t, 0.27886807f);
  p = fmaf(p, t, -0.18628806f);
  p = fmaf(p, t, 0.09678418f);
  p = fmaf(p, t, 0.37409196f);
  p = fmaf(p, t, 1.00002368f);
  p = fmaf(p, t, -1.26551223f);
  // hardware exp2 of the scaled argument: the rounding of the argument adds
  // at most |a^2 - P| * 2^-24 * log2(e) relative error, below 2e-6 wherever
  // Phi is above 1e-9 (beyond, the GELU terms are far below 1e-6 absolute)
  const float r = t * __expf(fmaf(-a, a, p));
  return z >= 0.f ? r : 2.0f - r;
}
// Phi(x) = erfc(-x / sqrt 2) / 2
__device__ __forceinline__ float gelu_(float x) { return x * 0.5f * erfc_nr(-x * 0.70710678118654752f); }
__device__ __forceinline__ float dgelu_(float x) {
  const float cdf = 0.5f * erfc_nr(-x * 0.70710678118654752f);
  const float pdf = __expf(-0.5f * x * x) * 0.39894228040143268f;
  return cdf + x * pdf;
}

// tanh form of GELU (Hendrycks & Gimpel, "Gaussian Error Linear Units"):
// g(x) = x (1 + tanh u) / 2, u = sqrt(2/pi) (x + 0.044715 x^3);
// g'(x) = (1 + tanh u) / 2 + x (1 - tanh^2 u) u'(x) / 2.
// With a = e^{-2|u|} in (0, 1] and s = 1 / (1 + a): 1 + tanh u = 2s for
// u >= 0 and 2as for u < 0, and 1 - tanh^2 u = 4as^2. Neither form
// subtracts nearly equal numbers or overflows, so both keep full relative
// precision far into the tails.
__device__ __forceinline__ void tanh_parts_(float x, float& onep, float& sech2, float& du) {
  const float k = 0.79788456080286536f;  // sqrt(2/pi)
  const float x2 = x * x;
  const float u = k * x * (1.0f + 0.044715f * x2);
  const float a = __expf(-2.0f * fabsf(u));
  const float s = 1.0f / (1.0f + a);
  onep = 2.0f * s * (u < 0.0f ? a : 1.0f);
  sech2 = 4.0f * a * s * s;
  du = k * (1.0f + 3.0f * 0.044715f * x2);
}
__device__ __forceinline__ float gelu_tanh_(float x) {
  float onep, sech2, du;
  tanh_parts_(x, onep, sech2, du);
  return 0.5f * x * onep;
}
__device__ __forceinline__ float dgelu_tanh_(float x) {
  float onep, sech2, du;
  tanh_parts_(x, onep, sech2, du);
  return 0.5f * onep + 0.5f * x * sech2 * du;
}

// One element: reads up to 3 inputs, produces up to 2 outputs.
template <int OP>
__device__ __forceinline__ void ew_apply(const float* in, float* out, float alpha, float colv) {
  if constexpr (OP == EW_ADD) out[0] = in[0] + in[1];
  else if constexpr (OP == EW_MUL) out[0] = in[0] * in[1];
  else if constexpr (OP == EW_SCALE) { out[0] = alpha * in[0]; out[1] = out[0]; }
  else if constexpr (OP == EW_ADD_BIAS) out[0] = in[0] + colv;
  else if constexpr (OP == EW_SILU) out[0] = silu_(in[0]);
  else if constexpr (OP == EW_GELU) out[0] = gelu_(in[0]);
  else if constexpr (OP == EW_SWIGLU) out[0] = silu_(in[0]) * in[1];
  else if constexpr (OP == EW_MUL_BWD) { out[0] = in[0] * in[2]; out[1] = in[0] * in[1]; }
  else if constexpr (OP == EW_SILU_BWD) out[0] = in[0] * dsilu_(in[1]);
  else if constexpr (OP == EW_GELU_BWD) out[0] = in[0] * dgelu_(in[1]);
  else if constexpr (OP == EW_GELU_TANH) out[0] = gelu_tanh_(in[0]);
  else if constexpr (OP == EW_GELU_TANH_BWD) out[0] = in[0] * dgelu_tanh_(in[1]);
  else if constexpr (OP == EW_SWIGLU_BWD) {
    const float g = in[1], u = in[2], d = in[0];
    out[0] = (d * u) * dsilu_(g);
    out[1] = d * silu_(g);
  } else if constexpr (OP == EW_ACCUMULATE) out[0] = in[0];
}

template <int OP> constexpr int n_in() {
  return (OP == EW_MUL_BWD || OP == EW_SWIGLU_BWD) ? 3
         : (OP == EW_ADD || OP == EW_MUL || OP == EW_SWIGLU || OP == EW_SILU_BWD || OP == EW_GELU_BWD ||
            OP == EW_GELU_TANH_BWD) ? 2 : 1;
}
template <int OP> constexpr int n_out() {
  return (OP == EW_MUL_BWD || OP == EW_SWIGLU_BWD || OP == EW_SCALE) ? 2 : 1;
}

struct EwK {
  const void* in[3]; int64_t ldi[3];
  void* out[2]; int64_t ldo[2];
  uint32_t acc;
  float alpha;
  const float* colvec;
  int64_t R, C;
  int64_t ccol;          // columns of the logical tensor (for the bias column)
};

// T: activation/output dtype; TS: dtype of in[0] (only differs for the
// accumulate, whose source may be f32 or bf16).
// Raw storage of N elements of type TS (one or two 16-byte packs, or 8 bytes).
template <typename TS, int N>
struct RawN {
  static constexpr int WORDS = (N * (int)sizeof(TS) + 15) / 16;
  uint4 w[WORDS];
  __device__ __forceinline__ void load(const TS* row, int64_t c0, int64_t C) {
    if (c0 + N <= C) {
      if constexpr (N * sizeof(TS) == 8) {
        const uint2 q = *reinterpret_cast<const uint2*>(row + c0);
        w[0] = make_uint4(q.x, q.y, 0, 0);
      } else {
#pragma unroll
        for (int i = 0; i < WORDS; ++i) w[i] = ld_nt(reinterpret_cast<const uint4*>(row + c0) + i);
      }
    } else {
      TS tmp[WORDS * 16 / sizeof(TS)];
#pragma unroll
      for (int k = 0; k < N; ++k) tmp[k] = (c0 + k < C) ? row[c0 + k] : (TS)0;
#pragma unroll
      for (int i = 0; i < WORDS; ++i) w[i] = reinterpret_cast<const uint4*>(tmp)[i];
    }
  }
  __device__ __forceinline__ void unpack(float* f) const {
    if constexpr (N * sizeof(TS) == 8) {
      f[0] = __uint_as_float(w[0].x << 16); f[1] = __uint_as_float(w[0].x & 0xffff0000u);
      f[2] = __uint_as_float(w[0].y << 16); f[3] = __uint_as_float(w[0].y & 0xffff0000u);
    } else {
#pragma unroll
      for (int i = 0; i < WORDS; ++i) io<TS>::unpack(w[i], f + i * io<TS>::VEC);
    }
  }
};

// ACC: bit o set = out[o] is accumulated into (compile-time, so the old
// values occupy registers only when needed).  The EW_UNROLL packs of a
// thread are all loaded (raw) before any is computed or stored.
template <typename T, typename TS, int OP, int ACC>
__global__ __launch_bounds__(EW_BLOCK) void ew_vec_k(EwK a) {
  constexpr int V = io<T>::VEC, NI = n_in<OP>(), NO = n_out<OP>();
  const int64_t ppr = (a.C + V - 1) / V;
  for (int64_t r = blockIdx.y; r < a.R; r += gridDim.y) {
    for (int64_t pb = (int64_t)blockIdx.x * EW_BLOCK * EW_UNROLL; pb < ppr; pb += (int64_t)gridDim.x * EW_BLOCK * EW_UNROLL) {
      RawN<TS, V> in0[EW_UNROLL];
      RawN<T, V> inr[EW_UNROLL][NI > 1 ? NI - 1 : 1];
      RawN<T, V> old[EW_UNROLL][(ACC != 0) ? NO : 1];
#pragma unroll
      for (int u = 0; u < EW_UNROLL; ++u) {
        const int64_t p = pb + u * EW_BLOCK + threadIdx.x;
        if (p >= ppr) continue;
        const int64_t c0 = p * V;
        in0[u].load(reinterpret_cast<const TS*>(a.in[0]) + r * a.ldi[0], c0, a.C);
#pragma unroll
        for (int i = 1; i < NI; ++i) inr[u][i - 1].load(reinterpret_cast<const T*>(a.in[i]) + r * a.ldi[i], c0, a.C);
        if constexpr (ACC != 0) {
#pragma unroll
          for (int o = 0; o < NO; ++o)
            if (((ACC >> o) & 1) && a.out[o]) old[u][o].load(reinterpret_cast<const T*>(a.out[o]) + r * a.ldo[o], c0, a.C);
        }
      }
#pragma unroll
      for (int u = 0; u < EW_UNROLL; ++u) {
        const int64_t p = pb + u * EW_BLOCK + threadIdx.x;
        if (p >= ppr) break;
        const int64_t c0 = p * V;
        float vin[3][V], vout[2][V];
        in0[u].unpack(vin[0]);
#pragma unroll
        for (int i = 1; i < NI; ++i) inr[u][i - 1].unpack(vin[i]);
        float colv[V];
#pragma unroll
        for (int k = 0; k < V; ++k) colv[k] = 0.f;
        if constexpr (OP == EW_ADD_BIAS) {
#pragma unroll
          for (int k = 0; k < V; ++k) {
            const int64_t c = c0 + k;
            if (c < a.C) colv[k] = a.colvec[(r * a.C + c) % a.ccol];
          }
        }
#pragma unroll
        for (int k = 0; k < V; ++k) {
          float i3[3] = {vin[0][k], NI > 1 ? vin[1][k] : 0.f, NI > 2 ? vin[2][k] : 0.f};
          float o2[2];
          ew_apply<OP>(i3, o2, a.alpha, colv[k]);
          vout[0][k] = o2[0];
          vout[1][k] = o2[1];
        }
#pragma unroll
        for (int o = 0; o < NO; ++o) {
          if (!a.out[o]) continue;
          if constexpr (ACC != 0) {
            if ((ACC >> o) & 1) {
              float ov[V];
              old[u][o].unpack(ov);
#pragma unroll
              for (int k = 0; k < V; ++k) vout[o][k] = acc_add(ov[k], vout[o][k]);
            }
          }
          T* row = reinterpret_cast<T*>(a.out[o]) + r * a.ldo[o];
          store_pack<T>(row, c0, a.C, vout[o]);
        }
      }
    }
  }
}

// Element-wise path for rows that are not 16-byte aligned.
template <typename T, typename TS, int OP>
__global__ __launch_bounds__(EW_BLOCK) void ew_scalar_k(EwK a) {
  constexpr int NI = n_in<OP>(), NO = n_out<OP>();
  for (int64_t r = blockIdx.y; r < a.R; r += gridDim.y) {
    for (int64_t c = (int64_t)blockIdx.x * EW_BLOCK + threadIdx.x; c < a.C; c += (int64_t)gridDim.x * EW_BLOCK) {
      float i3[3] = {0.f, 0.f, 0.f}, o2[2];
      i3[0] = io<TS>::ld(reinterpret_cast<const TS*>(a.in[0]) + r * a.ldi[0] + c);
#pragma unroll
      for (int i = 1; i < NI; ++i) i3[i] = io<T>::ld(reinterpret_cast<const T*>(a.in[i]) + r * a.ldi[i] + c);
      const float colv = (OP == EW_ADD_BIAS) ? a.colvec[(r * a.C + c) % a.ccol] : 0.f;
      ew_apply<OP>(i3, o2, a.alpha, colv);
#pragma unroll
      for (int o = 0; o < NO; ++o) {
        if (!a.out[o]) continue;
        T* q = reinterpret_cast<T*>(a.out[o]) + r * a.ldo[o] + c;
        const bool acc = (OP == EW_ACCUMULATE) || ((a.acc >> o) & 1u);
        io<T>::st(q, acc ? acc_add(io<T>::ld(q), o2[o]) : o2[o]);
      }
    }
  }
}

// ------------------------------------------------------------------ dropout
constexpr uint64_t GOLDEN = 0x9E3779B97F4A7C15ull;

// SplitMix64 output for state `key` (Steele, Lea & Flood 2014 with the
// Mix13 finalizer), only the top 24 bits: the last xor-shift by 31 cannot
// reach bits 40..63, so it is skipped.
__device__ __forceinline__ uint32_t splitmix_top24(uint64_t key) {
  uint64_t z = key + GOLDEN;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return (uint32_t)(z >> 40);
}

__device__ __forceinline__ void unpack_mask(const uint8_t* mr, int64_t c0, int64_t C, int V, bool vec,
                                            uint8_t* m) {
  if (vec && V == 8 && c0 + 8 <= C) {
    const uint2 q = *reinterpret_cast<const uint2*>(mr);
#pragma unroll
    for (int k = 0; k < 4; ++k) { m[k] = (q.x >> (8 * k)) & 0xff; m[k + 4] = (q.y >> (8 * k)) & 0xff; }
  } else if (vec && V == 4 && c0 + 4 <= C) {
    const uint32_t q = *reinterpret_cast<const uint32_t*>(mr);
#pragma unroll
    for (int k = 0; k < 4; ++k) m[k] = (q >> (8 * k)) & 0xff;
  } else {
    for (int k = 0; k < V; ++k) m[k] = c0 + k < C ? mr[k] : 0;
  }
}

__device__ __forceinline__ void store_mask(uint8_t* mr, int64_t c0, int64_t C, int V, bool vec,
                                           const uint8_t* m) {
  if (vec && V == 8 && c0 + 8 <= C) {
    uint2 q;
    q.x = m[0] | (m[1] << 8) | (m[2] << 16) | ((uint32_t)m[3] << 24);
    q.y = m[4] | (m[5] << 8) | (m[6] << 16) | ((uint32_t)m[7] << 24);
    *reinterpret_cast<uint2*>(mr) = q;
  } else if (vec && V == 4 && c0 + 4 <= C) {
    *reinterpret_cast<uint32_t*>(mr) = m[0] | (m[1] << 8) | (m[2] << 16) | ((uint32_t)m[3] << 24);
  } else {
    for (int k = 0; k < V; ++k) if (c0 + k < C) mr[k] = m[k];
  }
}

// MODE 0: forward (y, optional mask); MODE 1: mask only; MODE 2: backward
// (dx = mask ? d*scale : 0).  Each thread handles DU packs per iteration,
// issuing every load before any store.
constexpr int DU = EW_UNROLL;
template <typename T, int MODE, bool VEC, bool ACC>
__global__ __launch_bounds__(EW_BLOCK) void dropout_k(
    const void* __restrict__ x, int64_t ldx, void* __restrict__ y, int64_t ldy,
    uint8_t* __restrict__ mask, int64_t ldm, int64_t R, int64_t C, int64_t Clog,
    int64_t r0log, uint32_t thr, float scale, uint64_t seed) {
  constexpr int V = VEC ? io<T>::VEC : 1;
  const int64_t ppr = (C + V - 1) / V;
  for (int64_t r = blockIdx.y; r < R; r += gridDim.y) {
    for (int64_t pb = (int64_t)blockIdx.x * EW_BLOCK * DU; pb < ppr; pb += (int64_t)gridDim.x * EW_BLOCK * DU) {
      uint4 xq[DU], oq[ACC ? DU : 1];
      uint8_t m[DU][V];
      // every load first
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        const int64_t p = pb + u * EW_BLOCK + threadIdx.x;
        if (p >= ppr) continue;
        const int64_t c0 = p * V;
        if (MODE != 1) {
          const T* xr = reinterpret_cast<const T*>(x) + r * ldx;
          if constexpr (VEC) xq[u] = load_raw<T>(xr, c0, C);
          else xq[u].x = __float_as_uint(io<T>::ld(xr + c0));
        }
        if (MODE == 2) {
          unpack_mask(mask + r * ldm + c0, c0, C, V, VEC, m[u]);
          if constexpr (ACC) {
            const T* yr = reinterpret_cast<const T*>(y) + r * ldy;
            if constexpr (VEC) oq[u] = load_raw<T>(yr, c0, C);
            else oq[u].x = __float_as_uint(io<T>::ld(yr + c0));
          }
        }
      }
#pragma unroll
      for (int u = 0; u < DU; ++u) {
        const int64_t p = pb + u * EW_BLOCK + threadIdx.x;
        if (p >= ppr) break;
        const int64_t c0 = p * V;
        if (MODE != 2) {
          // counter of element (r, c): logical row-major index r*Clog + c
          const int64_t i0 = ((r0log + r) * Clog) + c0;
          uint64_t kg = (uint64_t)i0 * GOLDEN;
#pragma unroll
          for (int k = 0; k < V; ++k) {
            m[u][k] = splitmix_top24(seed ^ kg) >= thr ? 1 : 0;
            kg += GOLDEN;
          }
        }
        if (MODE != 1) {
          float v[V];
          if constexpr (VEC) io<T>::unpack(xq[u], v);
          else v[0] = __uint_as_float(xq[u].x);
#pragma unroll
          for (int k = 0; k < V; ++k) v[k] = m[u][k] ? v[k] * scale : 0.f;
          if constexpr (ACC) {
            float o[V];
            if constexpr (VEC) io<T>::unpack(oq[u], o);
            else o[0] = __uint_as_float(oq[u].x);
#pragma unroll
            for (int k = 0; k < V; ++k) v[k] = acc_add(o[k], v[k]);
          }
          T* yr = reinterpret_cast<T*>(y) + r * ldy;
          if constexpr (VEC) store_pack<T>(yr, c0, C, v);
          else io<T>::st(yr + c0, v[0]);
        }
        if (MODE != 2 && mask) store_mask(mask + r * ldm + c0, c0, C, V, VEC, m[u]);
      }
    }
  }
}

// Dense fast path: x, y and the mask are contiguous, 16-byte aligned and
// the element count is a whole number of packs.  One pack per thread over a
// full grid (no loop, no partial packs), 32-bit lane arithmetic for the
// hash: per element two 64-bit products by constants, the second reduced to
// the high word it needs.  The counter of element i is i itself.
template <typename T, int MODE, bool ACC>
__global__ __launch_bounds__(EW_BLOCK) void dropout_flat_k(
    const void* __restrict__ x, void* __restrict__ y, uint8_t* __restrict__ mask, int64_t npacks,
    uint32_t thr, float scale, uint64_t seed) {
  constexpr int V = io<T>::VEC;
  constexpr uint32_t M1L = 0x1CE4E5B9u, M1H = 0xBF58476Du, M2L = 0x133111EBu, M2H = 0x94D049BBu;
  const int64_t p = (int64_t)blockIdx.x * EW_BLOCK + threadIdx.x;
  if (p >= npacks) return;
  const int64_t i0 = p * V;
  uint4 xq{}, oq{};
  uint8_t m[V];
  if (MODE != 1) xq = ld_nt(reinterpret_cast<const T*>(x) + i0);
  if (MODE == 2) {
    unpack_mask(mask + i0, 0, V, V, true, m);
    if constexpr (ACC) oq = ld_nt(reinterpret_cast<const T*>(y) + i0);
  } else {
    uint64_t kg = (uint64_t)i0 * GOLDEN;
#pragma unroll
    for (int k = 0; k < V; ++k) {
      uint64_t z = (seed ^ kg) + GOLDEN;
      z ^= z >> 30;
      const uint32_t zl = (uint32_t)z, zh = (uint32_t)(z >> 32);
      const uint64_t pl = (uint64_t)zl * M1L;
      const uint32_t h1 = (uint32_t)(pl >> 32) + zl * M1H + zh * M1L;
      uint64_t z1 = ((uint64_t)h1 << 32) | (uint32_t)pl;
      z1 ^= z1 >> 27;
      const uint32_t al = (uint32_t)z1, ah = (uint32_t)(z1 >> 32);
      const uint32_t top = __umulhi(al, M2L) + al * M2H + ah * M2L;   // bits 32..63 of z1 * M2
      m[k] = (top >> 8) >= thr ? 1 : 0;
      kg += GOLDEN;
    }
    if (mask) store_mask(mask + i0, 0, V, V, true, m);
  }
  if (MODE != 1) {
    float v[V];
    io<T>::unpack(xq, v);
#pragma unroll
    for (int k = 0; k < V; ++k) v[k] = m[k] ? v[k] * scale : 0.f;
    if constexpr (ACC) {
      float o[V];
      io<T>::unpack(oq, o);
#pragma unroll
      for (int k = 0; k < V; ++k) v[k] = acc_add(o[k], v[k]);
    }
    st_nt(reinterpret_cast<T*>(y) + i0, io<T>::pack(v));
  }
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int es(int dt) { return dt == XT_F32 ? 4 : (dt == XT_BF16 ? 2 : (dt == XT_I32 ? 4 : 1)); }

bool contiguous(const xt_tensor* t) { return !t || t->ld == t->cols || t->rows <= 1; }
bool aligned(const xt_tensor* t) {
  return !t || ((((uintptr_t)t->data) & 15) == 0 && ((t->ld * es(t->dtype)) & 15) == 0);
}

dim3 ew_grid(int64_t R, int64_t C, int V, bool vec) {
  // one thread per pack (vec) or per element, every pack covered in one pass
  const int64_t ppr = vec ? cdiv(C, V) : C;
  const int64_t per_block = vec ? (int64_t)EW_BLOCK * EW_UNROLL : EW_BLOCK;
  const int64_t gx = std::min<int64_t>(cdiv(ppr, per_block), 0x7fffffff);
  const int64_t gy = std::min<int64_t>(std::max<int64_t>(R, 1), 65535);
  return dim3((unsigned)std::max<int64_t>(gx, 1), (unsigned)gy);
}

template <typename T, typename TS, int OP>
hipError_t ew_go(const EwArgs& e, hipStream_t s) {
  const xt_tensor* ref = e.out[0] ? e.out[0] : e.out[1];
  EwK a{};
  a.R = ref->rows; a.C = ref->cols; a.ccol = ref->cols;
  a.acc = e.acc; a.alpha = e.alpha; a.colvec = e.colvec;
  constexpr int NI = n_in<OP>(), NO = n_out<OP>();
  bool flat = true, al = true;
  for (int i = 0; i < NI; ++i) { flat = flat && contiguous(e.in[i]); al = al && aligned(e.in[i]); }
  for (int o = 0; o < NO; ++o) { flat = flat && contiguous(e.out[o]); al = al && aligned(e.out[o]); }
  for (int i = 0; i < NI; ++i) { a.in[i] = e.in[i]->data; a.ldi[i] = e.in[i]->ld; }
  for (int o = 0; o < NO; ++o) { a.out[o] = e.out[o] ? e.out[o]->data : nullptr; a.ldo[o] = e.out[o] ? e.out[o]->ld : 0; }
  if (a.R == 0 || a.C == 0) return hipSuccess;
  if (flat && a.R > 1) {      // one long row; ADD_BIAS recovers the column as index % ccol
    a.C = a.R * a.C;
    a.R = 1;
    for (int i = 0; i < NI; ++i) a.ldi[i] = a.C;
    for (int o = 0; o < NO; ++o) a.ldo[o] = a.C;
    al = true;
    for (int i = 0; i < NI; ++i) al = al && ((((uintptr_t)a.in[i]) & 15) == 0);
    for (int o = 0; o < NO; ++o) al = al && (!a.out[o] || (((uintptr_t)a.out[o]) & 15) == 0);
  }
  constexpr int V = io<T>::VEC;
  if (al) {
    const dim3 grid = ew_grid(a.R, a.C, V, true);
    const unsigned accb = (OP == EW_ACCUMULATE) ? 1u : (a.acc & ((1u << NO) - 1u));
    if (accb == 0) ew_vec_k<T, TS, OP, 0><<<grid, EW_BLOCK, 0, s>>>(a);
    else if (accb == 1) ew_vec_k<T, TS, OP, 1><<<grid, EW_BLOCK, 0, s>>>(a);
    else if (accb == 2) ew_vec_k<T, TS, OP, (NO > 1 ? 2 : 1)><<<grid, EW_BLOCK, 0, s>>>(a);
    else ew_vec_k<T, TS, OP, (NO > 1 ? 3 : 1)><<<grid, EW_BLOCK, 0, s>>>(a);
  } else {
    ew_scalar_k<T, TS, OP><<<ew_grid(a.R, a.C, 1, false), EW_BLOCK, 0, s>>>(a);
  }
  return hipGetLastError();
}

template <int OP>
hipError_t ew_dt(const EwArgs& e, hipStream_t s) {
  const xt_tensor* ref = e.out[0] ? e.out[0] : e.out[1];
  if (ref->dtype == XT_F32) return ew_go<float, float, OP>(e, s);
  return ew_go<bf16_t, bf16_t, OP>(e, s);
}

}  // namespace

hipError_t launch_ew(EwOp op, const EwArgs& e, hipStream_t s) {
  switch (op) {
    case EW_ADD: return ew_dt<EW_ADD>(e, s);
    case EW_MUL: return ew_dt<EW_MUL>(e, s);
    case EW_SCALE: return ew_dt<EW_SCALE>(e, s);
    case EW_ADD_BIAS: return ew_dt<EW_ADD_BIAS>(e, s);
    case EW_SILU: return ew_dt<EW_SILU>(e, s);
    case EW_GELU: return ew_dt<EW_GELU>(e, s);
    case EW_SWIGLU: return ew_dt<EW_SWIGLU>(e, s);
    case EW_MUL_BWD: return ew_dt<EW_MUL_BWD>(e, s);
    case EW_SILU_BWD: return ew_dt<EW_SILU_BWD>(e, s);
    case EW_GELU_BWD: return ew_dt<EW_GELU_BWD>(e, s);
    case EW_GELU_TANH: return ew_dt<EW_GELU_TANH>(e, s);
    case EW_GELU_TANH_BWD: return ew_dt<EW_GELU_TANH_BWD>(e, s);
    case EW_SWIGLU_BWD: return ew_dt<EW_SWIGLU_BWD>(e, s);
    case EW_ACCUMULATE: {
      const int dd = e.out[0]->dtype, sd = e.in[0]->dtype;
      if (dd == XT_F32 && sd == XT_F32) return ew_go<float, float, EW_ACCUMULATE>(e, s);
      if (dd == XT_F32 && sd == XT_BF16) return ew_go<float, bf16_t, EW_ACCUMULATE>(e, s);
      if (dd == XT_BF16 && sd == XT_F32) return ew_go<bf16_t, float, EW_ACCUMULATE>(e, s);
      return ew_go<bf16_t, bf16_t, EW_ACCUMULATE>(e, s);
    }
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int MODE>
static hipError_t dropout_go(const xt_tensor* x, const xt_tensor* y, const xt_tensor* mask, bool acc,
                             uint32_t thr, float scale, uint64_t seed, hipStream_t s) {
  const xt_tensor& ref = mask && MODE != 0 ? *mask : *y;
  int64_t R = ref.rows, C = ref.cols;
  if (R == 0 || C == 0) return hipSuccess;
  const int64_t Clog = C;                 // counter index = r*Clog + c of the logical tensor
  int64_t ldx = x ? x->ld : 0, ldy = y ? y->ld : 0, ldm = mask ? mask->ld : 0;
  constexpr int V = io<T>::VEC;
  bool flat = contiguous(x) && contiguous(y) && contiguous(mask);
  int64_t Cw = C, Rw = R, Clw = Clog;
  if (flat && R > 1) { Cw = R * C; Rw = 1; Clw = Cw; ldx = ldy = ldm = Cw; }
  bool vec = (!x || (((uintptr_t)x->data & 15) == 0 && ((ldx * es(x->dtype)) & 15) == 0)) &&
             (!y || (((uintptr_t)y->data & 15) == 0 && ((ldy * es(y->dtype)) & 15) == 0)) &&
             (!mask || (((uintptr_t)mask->data & (V - 1)) == 0 && (ldm % V) == 0));
  const dim3 grid = ew_grid(Rw, Cw, vec ? V : 1, true);     // DU == EW_UNROLL packs per thread
  const void* xp = x ? x->data : nullptr;
  void* yp = y ? y->data : nullptr;
  uint8_t* mp = mask ? (uint8_t*)mask->data : nullptr;
  if (vec && Rw == 1 && Cw % V == 0) {
    const int64_t np = Cw / V;
    const unsigned g = (unsigned)cdiv(np, EW_BLOCK);
    if (acc) dropout_flat_k<T, MODE, true><<<g, EW_BLOCK, 0, s>>>(xp, yp, mp, np, thr, scale, seed);
    else dropout_flat_k<T, MODE, false><<<g, EW_BLOCK, 0, s>>>(xp, yp, mp, np, thr, scale, seed);
    return hipGetLastError();
  }
#define XT_DROP(VEC_, ACC_) \
  dropout_k<T, MODE, VEC_, ACC_><<<grid, EW_BLOCK, 0, s>>>(xp, ldx, yp, ldy, mp, ldm, Rw, Cw, Clw, 0, thr, scale, seed)
  if (vec) { if (acc) XT_DROP(true, true); else XT_DROP(true, false); }
  else { if (acc) XT_DROP(false, true); else XT_DROP(false, false); }
#undef XT_DROP
  return hipGetLastError();
}

hipError_t launch_dropout_fwd(const xt_tensor& x, const xt_tensor& y, const xt_tensor* mask,
                              uint32_t thr, float scale, uint64_t seed, hipStream_t s) {
  if (x.dtype == XT_F32) return dropout_go<float, 0>(&x, &y, mask, false, thr, scale, seed, s);
  return dropout_go<bf16_t, 0>(&x, &y, mask, false, thr, scale, seed, s);
}

hipError_t launch_dropout_bwd(const xt_tensor& d, const xt_tensor& mask, const xt_tensor& dx,
                              bool acc, float scale, hipStream_t s) {
  if (d.dtype == XT_F32) return dropout_go<float, 2>(&d, &dx, &mask, acc, 0, scale, 0, s);
  return dropout_go<bf16_t, 2>(&d, &dx, &mask, acc, 0, scale, 0, s);
}

hipError_t launch_dropout_mask_only(const xt_tensor& mask, uint32_t thr, uint64_t seed, hipStream_t s) {
  return dropout_go<bf16_t, 1>(nullptr, nullptr, &mask, false, thr, 1.f, seed, s);
}

}  // namespace xt
