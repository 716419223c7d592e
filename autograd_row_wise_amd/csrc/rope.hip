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
#include <cmath>

#include "common.h"
#include "internal.h"

namespace xt {
namespace {

constexpr int RB = 256;

// cos and sin of th (0 <= th < 2^30) rounded once to f32.  The argument is
// reduced by pi/2 in f64 with a two-part constant (Cody and Waite, "Software
// Manual for the Elementary Functions", 1980): k = nearest integer to
// th * 2/pi; pi/2 = P1 + P2 with P1 holding 33 significant bits, so k * P1
// is exact for k < 2^20 and r = (th - k P1) - k P2 lies in [-pi/4, pi/4]
// within ~1e-16 k.  sin r and cos r are Taylor polynomials in f64 through
// r^13 and r^16 (truncation below 3e-14 on |r| <= pi/4), and the quadrant
// k mod 4 picks and signs them.  The f64 result is within ~1e-13 of the
// exact value before its one rounding to f32; about 25 f64 operations
// instead of a general library sincos.
__device__ __forceinline__ void sincos_f32(double th, float& c, float& s) {
  const double INV_PIO2 = 0.63661977236758138;        // 2/pi
  const double P1 = 1.5707963267341256;               // pi/2, first 33 bits
  const double P2 = 6.077100506506192e-11;            // pi/2 - P1
  const double k = __builtin_rint(th * INV_PIO2);
  const double r = __builtin_fma(-k, P2, __builtin_fma(-k, P1, th));
  const double r2 = r * r;
  double sp = 1.0 / 6227020800.0;                      // 1/13!
  sp = __builtin_fma(sp, r2, -1.0 / 39916800.0);       // 1/11!
  sp = __builtin_fma(sp, r2, 1.0 / 362880.0);          // 1/9!
  sp = __builtin_fma(sp, r2, -1.0 / 5040.0);
  sp = __builtin_fma(sp, r2, 1.0 / 120.0);
  sp = __builtin_fma(sp, r2, -1.0 / 6.0);
  const double sn = __builtin_fma(sp * r2, r, r);
  double cp = 1.0 / 20922789888000.0;                  // 1/16!
  cp = __builtin_fma(cp, r2, -1.0 / 87178291200.0);    // 1/14!
  cp = __builtin_fma(cp, r2, 1.0 / 479001600.0);       // 1/12!
  cp = __builtin_fma(cp, r2, -1.0 / 3628800.0);
  cp = __builtin_fma(cp, r2, 1.0 / 40320.0);
  cp = __builtin_fma(cp, r2, -1.0 / 720.0);
  cp = __builtin_fma(cp, r2, 1.0 / 24.0);
  cp = __builtin_fma(cp, r2, -0.5);
  const double cn = __builtin_fma(cp, r2, 1.0);
  const int q = (int)((long long)k & 3);
  const double cq = q == 0 ? cn : q == 1 ? -sn : q == 2 ? -cn : sn;
  const double sq = q == 0 ? sn : q == 1 ? cn : q == 2 ? -sn : -cn;
  c = (float)cq;
  s = (float)sq;
}

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
      float cn, sn;
      sincos_f32(th, cn, sn);
      cs[i] = cn;
      cs[half + i] = sign * sn;
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

// Pipelined form for 16-byte packs and rows of at most 2 * RB pack pairs.
// The block works on tiles of `rpi` rows (several short rows per tile, so
// every thread has work); thread slot s = tid + j*RB, j < 2, owns pack pair
// s % items of tile row s / items.  The frequencies base^(-2i/D) are
// computed once per block (f64, LDS); per tile, the angles pos * freq are
// formed in f64 and their cos/sin rounded to f32 into one of two LDS
// buffers, while the block's next tile's packs (if it has more than one
// tile) are already being fetched: one barrier per tile.  With one tile
// per block, the frequencies come from the host-computed table in the
// kernel arguments (wider heads compute them with pow).
// The frequencies base^(-2i/head_dim) of heads up to 128 wide, computed once
// on the host (f64) and passed in the kernel arguments.
constexpr int FREQ_MAX = 64;
struct FreqTable {
  double f[FREQ_MAX];
};

template <typename T>
__global__ __launch_bounds__(RB) void rope_pipe_k(const void* __restrict__ x, int64_t ldx,
                                                  void* __restrict__ y, int64_t ldy, int acc,
                                                  int64_t R, int head_dim, double base, int seq_len,
                                                  float sign, int items, int rpi, FreqTable ft) {
  constexpr int V = io<T>::VEC, NIT = 2;
  extern __shared__ double rsh[];                 // freq[half] (f64), then cs[2][rpi][2*half] (f32)
  const int half = head_dim / 2, per_head = half / V;
  double* freq = rsh;
  float* cs = reinterpret_cast<float*>(rsh + half);
  const int tid = threadIdx.x;
  for (int i = tid; i < half; i += RB) freq[i] = half <= FREQ_MAX ? ft.f[i] : pow(base, -2.0 * (double)i / (double)head_dim);

  int srow[NIT], scol[NIT], sv[NIT];
  bool sok[NIT];
#pragma unroll
  for (int j = 0; j < NIT; ++j) {
    const int sl = tid + j * RB;
    sok[j] = sl < rpi * items;
    const int it = sok[j] ? sl % items : 0;
    srow[j] = sok[j] ? sl / items : 0;
    sv[j] = it % per_head;
    scol[j] = (it / per_head) * head_dim + sv[j] * V;
  }
  const int64_t tiles = (R + rpi - 1) / rpi;
  const T* X = reinterpret_cast<const T*>(x);
  T* Y = reinterpret_cast<T*>(y);
  uint4 ca[NIT], cb[NIT], na[NIT], nb[NIT];
  auto fetch = [&](int64_t tile, uint4 (&pa)[NIT], uint4 (&pb)[NIT]) {
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int64_t r = tile * rpi + srow[j];
      if (sok[j] && r < R) {
        const T* xr = X + r * ldx + scol[j];
        pa[j] = ld_nt(xr);
        pb[j] = ld_nt(xr + half);
      }
    }
  };
  int64_t t = blockIdx.x;
  if (t < tiles) fetch(t, ca, cb);
  __syncthreads();                                // freq ready
  for (int k = 0; t < tiles; t += gridDim.x, ++k) {
    float* cb_ = cs + (k & 1) * (rpi * 2 * half);
    for (int idx = tid; idx < rpi * half; idx += RB) {
      const int rr = idx / half, i = idx % half;
      const int64_t r = t * rpi + rr;
      const double th = (double)(r % seq_len) * freq[i];
      float cn, sn;
      sincos_f32(th, cn, sn);
      cb_[rr * 2 * half + i] = cn;
      cb_[rr * 2 * half + half + i] = sign * sn;
    }
    const int64_t tn = t + gridDim.x;
    if (tn < tiles) fetch(tn, na, nb);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NIT; ++j) {
      const int64_t r = t * rpi + srow[j];
      if (!sok[j] || r >= R) continue;
      float a[V], b[V], ya[V], yb[V];
      io<T>::unpack(ca[j], a);
      io<T>::unpack(cb[j], b);
      const float* crow = cb_ + srow[j] * 2 * half + sv[j] * V;
      T* yr = Y + r * ldy + scol[j];
#pragma unroll
      for (int q = 0; q < V; ++q) {
        const float c = crow[q], sn = crow[half + q];
        ya[q] = a[q] * c - b[q] * sn;
        yb[q] = a[q] * sn + b[q] * c;
      }
      if (acc) {
        float oa[V], ob[V];
        io<T>::unpack(ld_nt(yr), oa);
        io<T>::unpack(ld_nt(yr + half), ob);
#pragma unroll
        for (int q = 0; q < V; ++q) { ya[q] = acc_add(oa[q], ya[q]); yb[q] = acc_add(ob[q], yb[q]); }
      }
      st_nt(yr, io<T>::pack(ya));
      st_nt(yr + half, io<T>::pack(yb));
    }
#pragma unroll
    for (int j = 0; j < NIT; ++j) { ca[j] = na[j]; cb[j] = nb[j]; }
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
  const float sign = inverse ? -1.f : 1.f;
  const int64_t items = (C / head_dim) * (half / V);
  if (vec && items <= 2 * RB) {
    // rows per tile: enough pack pairs for every thread, angle buffers <= 32 KB
    const int64_t rpi_lds = (32768 - 8 * (int64_t)half) / (16 * (int64_t)half);
    const int rpi = (int)std::max<int64_t>(1, std::min<int64_t>((2 * RB) / items, rpi_lds));
    const int64_t tiles = (R + rpi - 1) / rpi;
    // one tile per block over the full grid: measured 3-15% faster on 1 GiB
    // tensors than 2048 resident blocks looping over tiles
    const unsigned g = (unsigned)std::min<int64_t>(tiles, INT32_MAX);
    const size_t sh = (size_t)half * sizeof(double) + (size_t)2 * rpi * 2 * half * sizeof(float);
    FreqTable ft{};
    if (half <= FREQ_MAX)
      for (int i = 0; i < half; ++i) ft.f[i] = std::pow((double)base, -2.0 * (double)i / (double)head_dim);
    if (x.dtype == XT_F32)
      rope_pipe_k<float><<<g, RB, sh, s>>>(x.data, x.ld, y.data, y.ld, acc, R, head_dim, base, seq_len, sign,
                                           (int)items, rpi, ft);
    else
      rope_pipe_k<bf16_t><<<g, RB, sh, s>>>(x.data, x.ld, y.data, y.ld, acc, R, head_dim, base, seq_len, sign,
                                            (int)items, rpi, ft);
    return hipGetLastError();
  }
  const unsigned grid = (unsigned)std::min<int64_t>(R, 8192);
  const size_t shm = (size_t)2 * half * sizeof(float);
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
