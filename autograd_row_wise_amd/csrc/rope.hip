// Rotate-half rotary position embedding, forward and backward.
//
// [AE] op-backward table row "rope" and "RoPE 反向推导": each pair
// (x_i, x_{i+h}) of a head is rotated by R(theta); R is orthogonal, so the
// backward applies R(-theta) to the upstream gradient; position 0 is the
// identity.  theta(pos, i) = pos * base^(-2i/head_dim), i < head_dim/2,
// pos = row mod seq_len.
//
// The angles of a row are the same for all of its heads, so a block computes
// them once per row, in f64 (pos*theta reaches ~4e3 rad, where f32 would
// lose ~1e-4 rad), rounds cos/sin to f32 into LDS, and then streams the
// row's heads as 16-byte packs: each thread reads the pack of x_i and the
// pack of x_{i+h} and writes both rotated packs.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace xt {
namespace {

constexpr int RB = 256;

template <typename T, bool VEC>
__global__ __launch_bounds__(RB) void rope_k(const void* __restrict__ x, int64_t ldx,
                                             void* __restrict__ y, int64_t ldy, int acc,
                                             int64_t R, int64_t C, int head_dim, double base,
                                             int seq_len, float sign) {
  constexpr int V = VEC ? io<T>::VEC : 1;
  extern __shared__ float cs[];           // [2][half] f32 cos, sin
  const int half = head_dim / 2;
  const int64_t heads = C / head_dim;
  const int64_t per_head = half / V;
  const int64_t items = heads * per_head;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const double pos = (double)(r % seq_len);
    __syncthreads();
    for (int i = threadIdx.x; i < half; i += RB) {
      const double th = pos * pow(base, -2.0 * (double)i / (double)head_dim);
      double sn, cn;
      sincos(th, &sn, &cn);
      cs[i] = (float)cn;
      cs[half + i] = sign * (float)sn;
    }
    __syncthreads();
    const T* xr = reinterpret_cast<const T*>(x) + r * ldx;
    T* yr = reinterpret_cast<T*>(y) + r * ldy;
    // two work items per thread, both loaded before either is stored
    for (int64_t w0 = threadIdx.x; w0 < items; w0 += 2 * RB) {
      float a[2][V], b[2][V], oa[2][V], ob[2][V];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t w = w0 + u * RB;
        if (w >= items) continue;
        const int64_t h = w / per_head, vi = w % per_head;
        const int64_t ca = h * head_dim + vi * V, cb = ca + half;
        if constexpr (VEC) {
          io<T>::unpack(ld_nt(xr + ca), a[u]);
          io<T>::unpack(ld_nt(xr + cb), b[u]);
          if (acc) {
            io<T>::unpack(ld_nt(yr + ca), oa[u]);
            io<T>::unpack(ld_nt(yr + cb), ob[u]);
          }
        } else {
          a[u][0] = io<T>::ld(xr + ca);
          b[u][0] = io<T>::ld(xr + cb);
          if (acc) { oa[u][0] = io<T>::ld(yr + ca); ob[u][0] = io<T>::ld(yr + cb); }
        }
      }
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int64_t w = w0 + u * RB;
        if (w >= items) break;
        const int64_t h = w / per_head, vi = w % per_head;
        const int64_t ca = h * head_dim + vi * V, cb = ca + half;
        float ya[V], yb[V];
#pragma unroll
        for (int k = 0; k < V; ++k) {
          const int i = (int)(vi * V + k);
          const float c = cs[i], sn = cs[half + i];
          ya[k] = a[u][k] * c - b[u][k] * sn;
          yb[k] = a[u][k] * sn + b[u][k] * c;
          if (acc) { ya[k] = acc_add(oa[u][k], ya[k]); yb[k] = acc_add(ob[u][k], yb[k]); }
        }
        if constexpr (VEC) {
          st_nt(yr + ca, io<T>::pack(ya));
          st_nt(yr + cb, io<T>::pack(yb));
        } else {
          io<T>::st(yr + ca, ya[0]);
          io<T>::st(yr + cb, yb[0]);
        }
      }
    }
  }
}

int es_(int dt) { return dt == XT_F32 ? 4 : 2; }

}  // namespace

hipError_t launch_rope(const xt_tensor& x, const xt_tensor& y, bool acc, int head_dim,
                       float base, int seq_len, bool inverse, hipStream_t s) {
  const int64_t R = x.rows, C = x.cols;
  if (R == 0 || C == 0) return hipSuccess;
  const int half = head_dim / 2;
  const int V = x.dtype == XT_F32 ? 4 : 8;
  const bool vec = (half % V) == 0 && (((uintptr_t)x.data) & 15) == 0 && (((uintptr_t)y.data) & 15) == 0 &&
                   ((x.ld * es_(x.dtype)) & 15) == 0 && ((y.ld * es_(y.dtype)) & 15) == 0;
  const unsigned grid = (unsigned)std::min<int64_t>(R, 8192);
  const size_t shm = (size_t)2 * half * sizeof(float);
  const float sign = inverse ? -1.f : 1.f;
  if (x.dtype == XT_F32) {
    if (vec) rope_k<float, true><<<grid, RB, shm, s>>>(x.data, x.ld, y.data, y.ld, acc, R, C, head_dim, base, seq_len, sign);
    else rope_k<float, false><<<grid, RB, shm, s>>>(x.data, x.ld, y.data, y.ld, acc, R, C, head_dim, base, seq_len, sign);
  } else {
    if (vec) rope_k<bf16_t, true><<<grid, RB, shm, s>>>(x.data, x.ld, y.data, y.ld, acc, R, C, head_dim, base, seq_len, sign);
    else rope_k<bf16_t, false><<<grid, RB, shm, s>>>(x.data, x.ld, y.data, y.ld, acc, R, C, head_dim, base, seq_len, sign);
  }
  return hipGetLastError();
}

}  // namespace xt
