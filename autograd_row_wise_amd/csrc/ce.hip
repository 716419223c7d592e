// Mean cross-entropy over int32 targets, forward and backward.
//
// [AE] op-backward table row "cross_entropy" and "Cross-entropy 反向推导":
// L = mean_r -log softmax(x_r)[t_r];  dx = (softmax(x) - onehot(t)) * g / R,
// with the upstream scalar g and 1/R folded into the kernel.
//
// Rows are long (4096 .. 128256 columns: up to 250 KB), so one 256-thread
// block streams each row once with an online max/sum (no row staging): the
// forward reads the logits once and writes lse[r] and loss_row[r]; the mean
// is a separate one-block pass over loss_row in a fixed order (f64
// accumulation).  The backward saves nothing but lse: it rebuilds
// p = exp(x - lse) and writes dx in the same pass.  Row starts need not be
// 16-byte aligned (50257 f32 columns): each row is split into a scalar head
// up to the first 16-byte boundary, aligned 16-byte packs, and a scalar tail.
#include <algorithm>

#include "common.h"
#include "internal.h"

namespace xt {
namespace {

constexpr int CE_BLOCK = 256;
constexpr int CE_WAVES = CE_BLOCK / WAVE;

__device__ __forceinline__ float exp2_(float t) { return __builtin_amdgcn_exp2f(t); }
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Elements [first, first+count) of the row, split at 16-byte boundaries.
template <typename T>
__device__ __forceinline__ void split_row(const T* row, int64_t n, int64_t& head, int64_t& body_packs) {
  constexpr int V = io<T>::VEC;
  const uintptr_t a = (uintptr_t)row;
  int64_t h = (int64_t)(((16 - (a & 15)) & 15) / sizeof(T));
  if (h > n) h = n;
  head = h;
  body_packs = (n - h) / V;
}

template <typename T>
__global__ __launch_bounds__(CE_BLOCK) void ce_fwd_k(
    const void* __restrict__ logits, int64_t ld, const int32_t* __restrict__ tgt, int64_t ldt,
    float* __restrict__ lse, int64_t ldl, float* __restrict__ loss, int64_t ldo, int64_t R,
    int64_t V_) {
  constexpr int V = io<T>::VEC;
  __shared__ float sm[CE_WAVES], ss[CE_WAVES];
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* row = reinterpret_cast<const T*>(logits) + r * ld;
    int64_t head, bp;
    split_row<T>(row, V_, head, bp);
    const T* body = row + head;
    float m = -__builtin_inff(), s = 0.f;     // base-2 state of this thread
    auto push = [&](float x) {
      const float t = x * LOG2E;
      if (t > m) { s = s * exp2_(m - t) + 1.f; m = t; }
      else s += exp2_(t - m);
    };
    for (int64_t c = threadIdx.x; c < head; c += CE_BLOCK) push(io<T>::ld(row + c));
    // aligned body: four packs per thread in flight per iteration
    const uint4* bq = reinterpret_cast<const uint4*>(body);
    int p = threadIdx.x;
    const int bpi = (int)bp;
    for (; p + 3 * CE_BLOCK < bpi; p += 4 * CE_BLOCK) {
      float a[4][V];
#pragma unroll
      for (int u = 0; u < 4; ++u) io<T>::unpack(ld_nt(bq + p + u * CE_BLOCK), a[u]);
      float pm = a[0][0];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < V; ++k) pm = fmaxf(pm, a[u][k]);
      const float t = pm * LOG2E;
      if (t > m) { s *= exp2_(m - t); m = t; }
      float acc = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int k = 0; k < V; ++k) acc += exp2_(fmaf(a[u][k], LOG2E, -m));
      s += acc;
    }
    for (; p < bpi; p += CE_BLOCK) {
      float a[V];
      io<T>::unpack(ld_nt(bq + p), a);
      float pm = a[0];
#pragma unroll
      for (int k = 1; k < V; ++k) pm = fmaxf(pm, a[k]);
      const float t = pm * LOG2E;
      if (t > m) { s *= exp2_(m - t); m = t; }
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < V; ++k) acc += exp2_(fmaf(a[k], LOG2E, -m));
      s += acc;
    }
    for (int64_t c = head + bp * V + threadIdx.x; c < V_; c += CE_BLOCK) push(io<T>::ld(row + c));
    // (m, s) merged over the wave on the DPP paths, then the waves in order
    const MS st = wave_merge(MS{m, s});
    const int w = threadIdx.x / WAVE;
    __syncthreads();
    if ((threadIdx.x % WAVE) == 0) { sm[w] = st.m; ss[w] = st.s; }
    __syncthreads();
    if (threadIdx.x == 0) {
      MS tot{sm[0], ss[0]};
      for (int i = 1; i < CE_WAVES; ++i) tot = ms_merge(tot, MS{sm[i], ss[i]});
      const float l = (tot.m + log2f(tot.s)) * LN2;          // natural-log lse
      const int32_t t = tgt[r * ldt];
      const float xt = (t >= 0 && t < V_) ? io<T>::ld(row + t) : __builtin_nanf("");
      lse[r * ldl] = l;
      loss[r * ldo] = l - xt;
    }
  }
}

// L = (1/R) sum_r loss[r], fixed order: thread i sums rows i, i+1024, ...
// in f64, then a fixed tree over the 1024 partial sums.
__global__ __launch_bounds__(1024) void ce_mean_k(const float* __restrict__ loss, int64_t ldo,
                                                  int64_t R, float* __restrict__ L) {
  __shared__ double part[1024];
  double a = 0.0;
  for (int64_t r = threadIdx.x; r < R; r += 1024) a += (double)loss[r * ldo];
  part[threadIdx.x] = a;
  __syncthreads();
  for (int w = 512; w > 0; w >>= 1) {
    if (threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) L[0] = R > 0 ? (float)(part[0] / (double)R) : __builtin_nanf("");
}

// Backward: a 2-D grid, block (x, y) writes the x-th run of CE_BLOCK
// 16-byte packs of row y (one pack per thread, the pattern that streams
// fastest), block 0 also the scalar head and the last block the tail.
template <typename T>
__global__ __launch_bounds__(CE_BLOCK) void ce_bwd_k(
    const float* __restrict__ dL, const void* __restrict__ logits, int64_t ld,
    const int32_t* __restrict__ tgt, int64_t ldt, const float* __restrict__ lse, int64_t ldl,
    void* __restrict__ dx, int64_t lddx, int acc, int64_t R, int64_t V_) {
  constexpr int V = io<T>::VEC;
  const float scale = dL[0] / (float)R;
  const int n = (int)V_;
  for (int64_t r = blockIdx.y; r < R; r += gridDim.y) {
    const T* row = reinterpret_cast<const T*>(logits) + r * ld;
    T* orow = reinterpret_cast<T*>(dx) + r * lddx;
    const int32_t t = tgt[r * ldt];
    const bool ok = t >= 0 && t < n;
    // p = exp(x - lse) = 2^(x*log2e - lse*log2e); a bad target poisons the row
    const float nl = ok ? lse[r * ldl] * LOG2E : __builtin_nanf("");
    auto put = [&](int c) {
      const float p = exp2_(fmaf(io<T>::ld(row + c), LOG2E, -nl));
      const float v = (c == t ? p - 1.f : p) * scale;
      io<T>::st(orow + c, acc ? acc_add(io<T>::ld(orow + c), v) : v);
    };
    int64_t head64, bp64;
    split_row<T>(row, V_, head64, bp64);
    const int head = (int)head64, bp = (int)bp64;
    const int x = blockIdx.x, nx = gridDim.x;
    if (((((uintptr_t)row) ^ ((uintptr_t)orow)) & 15) != 0) {      // misaligned pair: scalar
      for (int c = x * CE_BLOCK + threadIdx.x; c < n; c += nx * CE_BLOCK) put(c);
      continue;
    }
    if (x == 0)
      for (int c = threadIdx.x; c < head; c += CE_BLOCK) put(c);
    if (x == nx - 1)
      for (int c = head + bp * V + threadIdx.x; c < n; c += CE_BLOCK) put(c);
    const uint4* body = reinterpret_cast<const uint4*>(row + head);
    uint4* obody = reinterpret_cast<uint4*>(orow + head);
    for (int p = x * CE_BLOCK + threadIdx.x; p < bp; p += nx * CE_BLOCK) {
      float a[V];
      io<T>::unpack(ld_nt(body + p), a);
      float b[V];
      if (acc) io<T>::unpack(ld_nt(obody + p), b);
#pragma unroll
      for (int k = 0; k < V; ++k) a[k] = exp2_(fmaf(a[k], LOG2E, -nl)) * scale;
      const int c0 = head + p * V;
      if ((unsigned)(t - c0) < (unsigned)V) {     // this pack holds the target column
#pragma unroll
        for (int k = 0; k < V; ++k)
          if (c0 + k == t) a[k] = (exp2_(fmaf(io<T>::ld(row + t), LOG2E, -nl)) - 1.f) * scale;
      }
      if (acc) {
#pragma unroll
        for (int k = 0; k < V; ++k) a[k] = acc_add(b[k], a[k]);
      }
      st_nt(obody + p, io<T>::pack(a));
    }
  }
}

int ce_grid(int64_t R) { return (int)std::max<int64_t>(1, std::min<int64_t>(R, 65536)); }

}  // namespace

hipError_t launch_ce_fwd(const xt_tensor& x, const int32_t* targets, int64_t ld_t, float* L,
                         float* lse, int64_t ld_lse, float* loss_row, int64_t ld_loss,
                         hipStream_t s) {
  const int64_t R = x.rows, V_ = x.cols;
  if (R > 0) {
    if (x.dtype == XT_F32)
      ce_fwd_k<float><<<ce_grid(R), CE_BLOCK, 0, s>>>(x.data, x.ld, targets, ld_t, lse, ld_lse, loss_row, ld_loss, R, V_);
    else
      ce_fwd_k<bf16_t><<<ce_grid(R), CE_BLOCK, 0, s>>>(x.data, x.ld, targets, ld_t, lse, ld_lse, loss_row, ld_loss, R, V_);
  }
  ce_mean_k<<<1, 1024, 0, s>>>(loss_row, ld_loss, R, L);
  return hipGetLastError();
}

hipError_t launch_ce_bwd(const float* dL, const xt_tensor& x, const int32_t* targets,
                         int64_t ld_t, const float* lse, int64_t ld_lse,
                         const xt_tensor& dx, bool acc, hipStream_t s) {
  const int64_t R = x.rows, V_ = x.cols;
  if (R == 0) return hipSuccess;
  // x blocks per row: enough CE_BLOCK-pack runs to cover the aligned body
  const int V = x.dtype == XT_F32 ? 4 : 8;
  const int64_t nx = std::max<int64_t>(1, (V_ / V + CE_BLOCK - 1) / CE_BLOCK);
  const dim3 grid((unsigned)nx, (unsigned)std::min<int64_t>(R, 65535));
  if (x.dtype == XT_F32)
    ce_bwd_k<float><<<grid, CE_BLOCK, 0, s>>>(dL, x.data, x.ld, targets, ld_t, lse, ld_lse, dx.data, dx.ld, acc, R, V_);
  else
    ce_bwd_k<bf16_t><<<grid, CE_BLOCK, 0, s>>>(dL, x.data, x.ld, targets, ld_t, lse, ld_lse, dx.data, dx.ld, acc, R, V_);
  return hipGetLastError();
}

}  // namespace xt
