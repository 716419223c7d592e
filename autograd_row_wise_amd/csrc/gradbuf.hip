// Gradient buffers after the backward: the global L2 norm of a list of
// gradient tensors and its clipping coefficient, in-place scaling and
// zeroing.
//
// [BP] kernel-pair table "Varje Forward-op Får En Backward-tvilling": the
// helper kernels k_grad_norm_partial, k_grad_norm_final and k_grad_scale
// for gradient clipping; [BP] "Ackumulation över mikrobatcher":
// scale_grads(1/n) after the microbatches, zero_grads() before the next
// step.  Clipping rule (the pages name the kernels only): Pascanu, Mikolov &
// Bengio, "On the difficulty of training recurrent neural networks" (2013),
// section 3.2 -- when the norm exceeds the threshold, every gradient is
// multiplied by threshold / norm.
//
// All three walk the same work decomposition.  A tensor is a set of rows
// (a contiguous tensor is one row of rows*cols elements); each row is cut
// into units of UNIT elements and one 256-thread block takes one unit.  A
// launch covers up to MAXT tensors, described by value in the kernel
// arguments (no device-side table, nothing to allocate or copy); longer
// lists take several launches.
//
// The norm is two passes: per-unit partial sums of squares (each square is
// exact in f64, summed in f64 in a fixed order) into caller workspace, then
// one block sums the partials in a fixed order, takes the square root and
// writes the norm and the coefficient.  Results are bitwise reproducible.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "common.h"
#include "internal.h"

namespace xt {
namespace {

constexpr int MAXT = 64;
constexpr int GB = 256;                 // threads per block
constexpr int64_t UNIT = 8192;          // elements per block

struct GbTable {                        // 2.8 KB of kernel arguments
  char* p[MAXT];
  int64_t cols[MAXT];                   // elements per row
  int64_t ldb[MAXT];                    // row stride in bytes
  int64_t upr[MAXT];                    // units per row
  int64_t u0[MAXT + 1];                 // first unit of each tensor
  int32_t flags[MAXT];                  // bit 0: bf16, bit 1: 16-byte packs usable
  int32_t n;
};

struct Unit {
  char* row;                            // first byte of the unit's row
  int64_t c0, c1;                       // element range in the row
  bool bf16, vec;
};

__device__ __forceinline__ Unit unit_of(const GbTable& L, int64_t U) {
  int lo = 0, hi = L.n - 1;             // the last t with u0[t] <= U
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (L.u0[mid] <= U) lo = mid;
    else hi = mid - 1;
  }
  const int t = lo;
  const int64_t k = U - L.u0[t], r = k / L.upr[t], ch = k % L.upr[t];
  Unit u;
  u.row = L.p[t] + r * L.ldb[t];
  u.c0 = ch * UNIT;
  u.c1 = u.c0 + UNIT < L.cols[t] ? u.c0 + UNIT : L.cols[t];
  u.bf16 = (L.flags[t] & 1) != 0;
  u.vec = (L.flags[t] & 2) != 0;
  return u;
}

__device__ __forceinline__ float ld_el(const Unit& u, int64_t c) {
  return u.bf16 ? bf2f(reinterpret_cast<const uint16_t*>(u.row)[c]) : reinterpret_cast<const float*>(u.row)[c];
}

__device__ __forceinline__ void st_el(const Unit& u, int64_t c, float v) {
  if (u.bf16) reinterpret_cast<uint16_t*>(u.row)[c] = (uint16_t)f2bf(v);
  else reinterpret_cast<float*>(u.row)[c] = v;
}

// A double from lane `CTRL` (DPP control) away: its two halves moved alike.
template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ double dpp_d(double v) {
  const int2 h = __builtin_bit_cast(int2, v);
  const int lo = __builtin_amdgcn_update_dpp(0, h.x, CTRL, ROW_MASK, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(0, h.y, CTRL, ROW_MASK, 0xf, false);
  return __builtin_bit_cast(double, make_int2(lo, hi));
}

// Wave sum of doubles in the order of wave_reduce (common.h): rows by DPP
// steps, rows 1, 3 add rows 0, 2, rows 2, 3 add lane 31, lane 63 read.
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dpp_d<dpp::XOR1>(v);
  v += dpp_d<dpp::XOR2>(v);
  v += dpp_d<dpp::HALF_MIRROR>(v);
  v += dpp_d<dpp::MIRROR>(v);
  const int lane = __lane_id();
  const double a = v + dpp_d<dpp::BCAST15, 0xa>(v);
  v = (lane & 16) ? a : v;
  const double b = v + dpp_d<dpp::BCAST31, 0xc>(v);
  v = (lane & 32) ? b : v;
  const int2 h = __builtin_bit_cast(int2, v);
  return __builtin_bit_cast(double, make_int2(__builtin_amdgcn_readlane(h.x, 63), __builtin_amdgcn_readlane(h.y, 63)));
}

// Block sum of one double per thread in a fixed order: the DPP wave sum,
// then the four wave sums in wave order.
__device__ __forceinline__ double block_sum(double v) {
  __shared__ double ws[GB / WAVE];
  v = wave_sum_d(v);
  if (threadIdx.x % WAVE == 0) ws[threadIdx.x / WAVE] = v;
  __syncthreads();
  double s = 0.0;
  if (threadIdx.x == 0)
    for (int w = 0; w < GB / WAVE; ++w) s += ws[w];
  return s;
}

// Pass 1: part[U] = sum of squares of unit U (f64).
__global__ __launch_bounds__(GB) void gn_partial_k(GbTable L, double* __restrict__ part) {
  const Unit u = unit_of(L, blockIdx.x);
  const int tid = threadIdx.x;
  double acc = 0.0;
  int64_t done = u.c0;
  if (u.vec) {
    const int V = u.bf16 ? 8 : 4;
    const int64_t np = (u.c1 - u.c0) / V;
    const u32x4_t* P = reinterpret_cast<const u32x4_t*>(u.row + u.c0 * (u.bf16 ? 2 : 4));
    constexpr int MAXP = (int)(UNIT / 4 / GB);           // packs per thread, f32
    u32x4_t q[MAXP];
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      const int64_t i = tid + (int64_t)k * GB;
      q[k] = i < np ? __builtin_nontemporal_load(P + i) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (u.bf16) {
          const float lo = __uint_as_float(q[k][e] << 16), hi = __uint_as_float(q[k][e] & 0xffff0000u);
          acc += (double)lo * (double)lo;
          acc += (double)hi * (double)hi;
        } else {
          const float f = __uint_as_float(q[k][e]);
          acc += (double)f * (double)f;
        }
      }
    }
    done = u.c0 + np * V;
  }
  for (int64_t c = done + tid; c < u.c1; c += GB) {
    const double f = (double)ld_el(u, c);
    acc += f * f;
  }
  const double s = block_sum(acc);
  if (tid == 0) part[blockIdx.x] = s;
}

// Pass 2: out[0] = sqrt(sum of part), out[1] = clipping coefficient.  One
// block of FB threads; thread t sums part[t + FB j] for j = 0, 1, ... into
// four accumulators by j mod 4 (independent loads in flight), combined in a
// fixed order, then a fixed tree over the block.
constexpr int FB = 1024;
__global__ __launch_bounds__(FB) void gn_final_k(const double* __restrict__ part, int64_t n, float max_norm,
                                                  float* __restrict__ out) {
  __shared__ double s[FB];
  double a[4] = {0.0, 0.0, 0.0, 0.0};
  int64_t i = threadIdx.x;
  for (; i + 3 * FB < n; i += 4 * FB) {
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] += part[i + j * FB];
  }
  for (int j = 0; i < n; i += FB, ++j) a[j] += part[i];
  s[threadIdx.x] = (a[0] + a[1]) + (a[2] + a[3]);
  __syncthreads();
  for (int o = FB / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) s[threadIdx.x] += s[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double norm = sqrt(s[0]);
    out[0] = (float)norm;
    out[1] = (max_norm > 0.f && norm > (double)max_norm) ? (float)((double)max_norm / norm) : 1.f;
  }
}

// g = g * factor (factor = alpha, times *scale when given), one f32 product
// per element rounded once into g's dtype; ZERO: g = 0.
template <bool ZERO>
__global__ __launch_bounds__(GB) void gs_k(GbTable L, float alpha, const float* __restrict__ scale) {
  const Unit u = unit_of(L, blockIdx.x);
  const int tid = threadIdx.x;
  const float f = ZERO ? 0.f : (scale ? alpha * scale[0] : alpha);
  int64_t done = u.c0;
  if (u.vec) {
    const int V = u.bf16 ? 8 : 4;
    const int64_t np = (u.c1 - u.c0) / V;
    u32x4_t* P = reinterpret_cast<u32x4_t*>(u.row + u.c0 * (u.bf16 ? 2 : 4));
    constexpr int MAXP = (int)(UNIT / 4 / GB);           // packs per thread, f32
    u32x4_t q[MAXP];
    if constexpr (!ZERO) {
#pragma unroll
      for (int k = 0; k < MAXP; ++k) {
        const int64_t i = tid + (int64_t)k * GB;
        q[k] = i < np ? __builtin_nontemporal_load(P + i) : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int k = 0; k < MAXP; ++k) {
      const int64_t i = tid + (int64_t)k * GB;
      if (i >= np) break;
      u32x4_t o = {0u, 0u, 0u, 0u};
      if constexpr (!ZERO) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (u.bf16) {
            const float lo = __uint_as_float(q[k][e] << 16) * f, hi = __uint_as_float(q[k][e] & 0xffff0000u) * f;
            o[e] = f2bf2(lo, hi);
          } else {
            o[e] = __float_as_uint(__uint_as_float(q[k][e]) * f);
          }
        }
      }
      __builtin_nontemporal_store(o, P + i);
    }
    done = u.c0 + np * V;
  }
  for (int64_t c = done + tid; c < u.c1; c += GB) st_el(u, c, ZERO ? 0.f : ld_el(u, c) * f);
}

// Fills `L` from grads[i0 ..] (at most MAXT non-empty tensors); returns the
// index after the last one taken and sets `units`.
int fill_table(const xt_tensor* g, int n, int i0, GbTable& L, int64_t& units) {
  L.n = 0;
  units = 0;
  int i = i0;
  for (; i < n && L.n < MAXT; ++i) {
    const xt_tensor& t = g[i];
    if (t.rows <= 0 || t.cols <= 0) continue;
    const int64_t esz = t.dtype == XT_BF16 ? 2 : 4;
    const bool flat = t.rows == 1 || t.ld == t.cols;
    const int64_t rows = flat ? 1 : t.rows, cols = flat ? t.rows * t.cols : t.cols;
    const int k = L.n++;
    L.p[k] = (char*)t.data;
    L.cols[k] = cols;
    L.ldb[k] = flat ? 0 : t.ld * esz;
    L.upr[k] = (cols + UNIT - 1) / UNIT;
    L.u0[k] = units;
    const bool vec = (((uintptr_t)t.data) % 16 == 0) && (L.ldb[k] % 16 == 0);
    L.flags[k] = (t.dtype == XT_BF16 ? 1 : 0) | (vec ? 2 : 0);
    units += rows * L.upr[k];
  }
  L.u0[L.n] = units;
  return i;
}

}  // namespace

int64_t grad_norm_units(const xt_tensor* g, int n) {
  int64_t total = 0;
  GbTable L;
  for (int i = 0; i < n;) {
    int64_t u = 0;
    i = fill_table(g, n, i, L, u);
    total += u;
  }
  return total;
}

hipError_t launch_grad_norm(const xt_tensor* g, int n, float max_norm, float* out, double* part, hipStream_t s) {
  int64_t off = 0;
  GbTable L;
  for (int i = 0; i < n;) {
    int64_t u = 0;
    i = fill_table(g, n, i, L, u);
    if (u > 0) {
      gn_partial_k<<<(unsigned)u, GB, 0, s>>>(L, part + off);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    off += u;
  }
  gn_final_k<<<1, FB, 0, s>>>(part, off, max_norm, out);
  return hipGetLastError();
}

hipError_t launch_grads_scale(const xt_tensor* g, int n, bool zero, float alpha, const float* scale,
                              hipStream_t s) {
  GbTable L;
  for (int i = 0; i < n;) {
    int64_t u = 0;
    i = fill_table(g, n, i, L, u);
    if (u == 0) continue;
    if (zero) gs_k<true><<<(unsigned)u, GB, 0, s>>>(L, 0.f, nullptr);
    else gs_k<false><<<(unsigned)u, GB, 0, s>>>(L, alpha, scale);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace xt
