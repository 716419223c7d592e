// Row-wise reductions: rms_norm, layer_norm and softmax, forward and backward,
// plus the fixed-order column reductions that finish parameter gradients.
//
// [AE] "RMSNorm" paragraph, op-backward table rows "softmax" and the
// "Softmax 反向推导"; [BP] k_layernorm_fwd/k_layernorm_bwd, "Sparade
// tensorer" (mean and variance saved by the forward) and "En baklängeskärnas
// uppgift" (one launch yields grad_input and the parameter gradient).
//
// Fast path: a row is held in registers by a group of RW waves (RW = 1, 4 or
// 16), each thread keeping NV 16-byte packs, so x (and d) are read from HBM
// exactly once per op.  Reductions are wave butterflies then a fixed-order
// LDS combine: results do not depend on scheduling.  Backward kernels run at
// most 512 blocks of 512 threads (one or two per CU) whose rows interleave
// (block b, group g takes rows b NG + g + k gridDim NG: the rows in flight
// form one contiguous window, measured 5-15% faster than a contiguous run of
// rows per block); each thread accumulates the parameter-gradient terms of
// its own columns over the block's rows, the groups of a block are folded in
// LDS in group order, and one partial row per block goes to the workspace.
// A separate pass sums the partial rows in block order.
//
// Generic path (rows that do not fit in registers or are not 16-byte
// aligned): one 256-thread block per row, several passes over global memory.
#include <algorithm>
#include <map>
#include <mutex>
#include <tuple>

#include "common.h"
#include "internal.h"

namespace xt {

namespace {

constexpr int BWD_BLOCK = 512;       // 8 waves: up to 256 VGPRs per thread, no spills
constexpr int BWD_GRID_MAX = 512;     // two backward blocks per CU
// Forward and softmax grids are not capped by what the chip holds at once:
// measured on MI355X, many short-lived blocks that the dispatcher hands to
// whichever CU is free stream 8-15% faster than resident blocks looping over
// many rows each (no tail of late blocks).  rms/layer-norm forward blocks
// still take NORM_FWD_STEPS row steps per group, which amortises the gamma
// (and beta) loads; softmax rows of 8 waves or more keep a 4096-block grid
// (8192 for the backward), measured faster for 32K-wide rows.
constexpr int NORM_FWD_STEPS = 4;
constexpr int LONG_ROW_GRID = 4096;
constexpr int GEN_BLOCK = 256;

__device__ __forceinline__ float fast_exp(float t) {
  return __builtin_amdgcn_exp2f(t * 1.4426950408889634f);
}

template <typename T> __device__ __forceinline__ const T* row_ptr(const void* p, int64_t r, int64_t ld) {
  return reinterpret_cast<const T*>(p) + r * ld;
}
template <typename T> __device__ __forceinline__ T* row_ptr_w(void* p, int64_t r, int64_t ld) {
  return reinterpret_cast<T*>(p) + r * ld;
}

// Whole 16-byte pack store with optional accumulation (row width is a
// multiple of the pack width on the register-resident path).
template <typename T>
__device__ __forceinline__ void store_full(T* p, float* f, bool acc) {
  if (acc) {
    float o[io<T>::VEC];
    io<T>::unpack(ld_nt(p), o);
#pragma unroll
    for (int k = 0; k < io<T>::VEC; ++k) f[k] = acc_add(o[k], f[k]);
  }
  st_nt(p, io<T>::pack(f));
}

// The fast kernels walk their rows with the next row's packs already in
// flight: they are loaded (raw, 16 bytes each) before the current row's
// reductions and stores (the rms_norm backward: right after them), so HBM
// latency overlaps the barrier phase.

// An empty asm that claims to rewrite the raw packs: values unpacked from
// them before it cannot be reused after it, so bf16 rows stay live as raw
// packs (half the registers of their f32 values) across a reduction and
// are unpacked again where they are used.
template <typename T, int NV, int G>
__device__ __forceinline__ void keep_raw(RowPacks<T, NV, G>& p) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int j = 0; j < NV; ++j)
      asm volatile("" : "+v"(p.q[j].x), "+v"(p.q[j].y), "+v"(p.q[j].z), "+v"(p.q[j].w));
  }
}

// ===================================================================== RMS
template <typename T, int RW, int NV, int BLOCK>
__global__ __launch_bounds__(BLOCK) void rms_fwd_fast(
    const void* __restrict__ x, int64_t ldx, const float* __restrict__ gamma,
    void* __restrict__ y, int64_t ldy, float* __restrict__ ir, int64_t ldir,
    int64_t R, int64_t C, float eps, float invC) {
  constexpr int V = io<T>::VEC, G = WAVE * RW, NG = BLOCK / G;
  __shared__ float lds[4 * BLOCK / WAVE];
  int ph = 0;
  const int g = threadIdx.x / G, gl = threadIdx.x % G;
  const int Ci = (int)C;
  const int64_t stride = (int64_t)gridDim.x * NG;
  float gam[NV][V];
#pragma unroll
  for (int j = 0; j < NV; ++j) load_f32s<V, int>(gamma, pack_col<NV, V>(j, gl), Ci, gam[j]);
  RowPacks<T, NV, G> b0, b1;
  int64_t base = (int64_t)blockIdx.x * NG;
  b0.load(row_ptr<T>(x, base + g < R ? base + g : 0, ldx), gl, Ci, base + g < R);
  if (base + stride < R) b1.load(row_ptr<T>(x, base + stride + g < R ? base + stride + g : 0, ldx), gl, Ci, base + stride + g < R);
  auto step = [&](RowPacks<T, NV, G>& cur, int64_t bs) {
    const int64_t r = bs + g, rn = bs + 2 * stride + g;
    const bool active = r < R;
    float v[NV][V];
    cur.unpack(v);
    if (bs + 2 * stride < R) cur.load(row_ptr<T>(x, rn < R ? rn : 0, ldx), gl, Ci, rn < R);
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int k = 0; k < V; ++k) ss += v[j][k] * v[j][k];
    ss = group_sum<RW>(ss, lds, ph);
    const float irv = rsqrtf(ss * invC + eps);
    if (active) {
      T* yr = row_ptr_w<T>(y, r, ldy);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int c0 = pack_col<NV, V>(j, gl);
        if (c0 < Ci) {
          float o[V];
#pragma unroll
          for (int k = 0; k < V; ++k) o[k] = v[j][k] * irv * gam[j][k];
          st_nt(yr + c0, io<T>::pack(o));
        }
      }
      if (gl == 0) ir[r * ldir] = irv;
    }
  };
  for (; base < R; base += 2 * stride) {
    step(b0, base);
    if (base + stride < R) step(b1, base + stride);
  }
}

// Folds the per-group parameter partials of a block (NG groups, fixed group
// order) into LDS and writes one partial row (NP vectors of C) per block.
template <int NV, int V, int G, int NG, int NP, int BLOCK>
__device__ __forceinline__ void fold_partials(float (&pp)[NP][NV][V], float* red, float* part,
                                              int64_t C) {
  const int g = threadIdx.x / G, gl = threadIdx.x % G;
  const int Ci = (int)C;
  for (int gi = 0; gi < NG; ++gi) {
    if (g == gi) {
#pragma unroll
      for (int q = 0; q < NP; ++q)
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
          for (int k = 0; k < V; ++k) {
            const int c = pack_col<NV, V>(j, gl) + k;
            if (c < C) red[q * C + c] = (gi == 0) ? pp[q][j][k] : red[q * C + c] + pp[q][j][k];
          }
    }
    __syncthreads();
  }
  float* out = part + (int64_t)blockIdx.x * NP * C;
  for (int64_t c = threadIdx.x; c < NP * C; c += BLOCK) out[c] = red[c];
}

template <typename T, int RW, int NV>
__global__ __launch_bounds__(BWD_BLOCK, sizeof(T) == 2 && NV <= 2 ? 4 : 1) void rms_bwd_fast(
    const void* __restrict__ d, int64_t ldd, const void* __restrict__ x, int64_t ldx,
    const float* __restrict__ gamma, const float* __restrict__ ir, int64_t ldir,
    void* __restrict__ dx, int64_t lddx, int acc_dx, float* __restrict__ part,
    int64_t R, int64_t C, float invC) {
  constexpr int V = io<T>::VEC, G = WAVE * RW, NG = BWD_BLOCK / G;
  extern __shared__ float red[];               // C floats
  __shared__ float lds[4 * BWD_BLOCK / WAVE];
  int ph = 0;
  const int g = threadIdx.x / G, gl = threadIdx.x % G;
  const int Ci = (int)C;
  float gam[NV][V], pp[1][NV][V];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    load_f32s<V, int>(gamma, pack_col<NV, V>(j, gl), Ci, gam[j]);
#pragma unroll
    for (int k = 0; k < V; ++k) pp[0][j][k] = 0.f;
  }
  // rows interleaved over the blocks: step k of group g is row
  // blockIdx.x NG + g + k gridDim.x NG, so the rows in flight across the
  // chip at any time form one contiguous window of the tensor
  const int64_t stride = (int64_t)gridDim.x * NG, first = (int64_t)blockIdx.x * NG, end = R;
  // two register sets of raw packs: while row base is reduced and written,
  // row base+NG is in flight; a set is refilled (row base+2NG) once its row
  // is written.  Only raw packs stay live (unpacked pack by pack where
  // used): the bf16 shapes then fit the 128 VGPRs of four waves per SIMD
  // (two blocks per CU) without spills, measured 10% faster on long
  // tensors than the unpacked ring at two waves per SIMD.
  RowPacks<T, NV, G> d0, x0, d1, x1;
  {
    const int64_t r = first + g, r1 = first + stride + g;
    d0.load(row_ptr<T>(d, r < end ? r : 0, ldd), gl, Ci, r < end);
    x0.load(row_ptr<T>(x, r < end ? r : 0, ldx), gl, Ci, r < end);
    if (first + stride < end) {
      d1.load(row_ptr<T>(d, r1 < end ? r1 : 0, ldd), gl, Ci, r1 < end);
      x1.load(row_ptr<T>(x, r1 < end ? r1 : 0, ldx), gl, Ci, r1 < end);
    }
  }
  auto step = [&](RowPacks<T, NV, G>& cd, RowPacks<T, NV, G>& cx, int64_t base) {
    const int64_t r = base + g, rn = base + 2 * stride + g;
    const bool active = r < end;
    const float irv = active ? ir[r * ldir] : 0.f;
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float dv[V], xv[V];
      io<T>::unpack(cd.q[j], dv);
      io<T>::unpack(cx.q[j], xv);
#pragma unroll
      for (int k = 0; k < V; ++k) dot += dv[k] * gam[j][k] * xv[k];
    }
    dot = group_sum<RW>(dot, lds, ph);
    keep_raw(cd);
    keep_raw(cx);
    if (active) {
      const float c1 = irv * irv * irv * invC * dot;
      T* dxr = dx ? row_ptr_w<T>(dx, r, lddx) : nullptr;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int c0 = pack_col<NV, V>(j, gl);
        if (c0 < Ci) {
          float dv[V], xv[V], o[V];
          io<T>::unpack(cd.q[j], dv);
          io<T>::unpack(cx.q[j], xv);
#pragma unroll
          for (int k = 0; k < V; ++k) {
            o[k] = irv * (dv[k] * gam[j][k]) - xv[k] * c1;
            pp[0][j][k] += dv[k] * xv[k] * irv;
          }
          if (dxr) store_full<T>(dxr + c0, o, acc_dx != 0);
        }
      }
    }
    if (base + 2 * stride < end) {
      cd.load(row_ptr<T>(d, rn < end ? rn : 0, ldd), gl, Ci, rn < end);
      cx.load(row_ptr<T>(x, rn < end ? rn : 0, ldx), gl, Ci, rn < end);
    }
  };
  for (int64_t base = first; base < end; base += 2 * stride) {
    step(d0, x0, base);
    if (base + stride < end) step(d1, x1, base + stride);
  }
  if (part) fold_partials<NV, V, G, NG, 1, BWD_BLOCK>(pp, red, part, C);
}

// ================================================================ LayerNorm
template <typename T, int RW, int NV, int BLOCK>
__global__ __launch_bounds__(BLOCK) void ln_fwd_fast(
    const void* __restrict__ x, int64_t ldx, const float* __restrict__ gamma,
    const float* __restrict__ beta, void* __restrict__ y, int64_t ldy,
    float* __restrict__ mean, int64_t ldm, float* __restrict__ rstd, int64_t ldr,
    int64_t R, int64_t C, float eps, float invC) {
  constexpr int V = io<T>::VEC, G = WAVE * RW, NG = BLOCK / G;
  __shared__ float lds[4 * BLOCK / WAVE];
  int ph = 0;
  const int g = threadIdx.x / G, gl = threadIdx.x % G;
  const int Ci = (int)C;
  const int64_t stride = (int64_t)gridDim.x * NG;
  float gam[NV][V], bet[NV][V];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    load_f32s<V, int>(gamma, pack_col<NV, V>(j, gl), Ci, gam[j]);
    load_f32s<V, int>(beta, pack_col<NV, V>(j, gl), Ci, bet[j]);
  }
  RowPacks<T, NV, G> b0, b1;
  int64_t base = (int64_t)blockIdx.x * NG;
  b0.load(row_ptr<T>(x, base + g < R ? base + g : 0, ldx), gl, Ci, base + g < R);
  if (base + stride < R) b1.load(row_ptr<T>(x, base + stride + g < R ? base + stride + g : 0, ldx), gl, Ci, base + stride + g < R);
  auto step = [&](RowPacks<T, NV, G>& cur, int64_t bs) {
    const int64_t r = bs + g, rn = bs + 2 * stride + g;
    const bool active = r < R;
    float v[NV][V];
    cur.unpack(v);
    if (bs + 2 * stride < R) cur.load(row_ptr<T>(x, rn < R ? rn : 0, ldx), gl, Ci, rn < R);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int k = 0; k < V; ++k) s += v[j][k];
    const float mu = group_sum<RW>(s, lds, ph) * invC;
    float q = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const float t = v[j][k] - mu;
        if (pack_col<NV, V>(j, gl) + k < Ci) q += t * t;
      }
    const float var = group_sum<RW>(q, lds, ph) * invC;
    const float rs = rsqrtf(var + eps);
    if (active) {
      T* yr = row_ptr_w<T>(y, r, ldy);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int c0 = pack_col<NV, V>(j, gl);
        if (c0 < Ci) {
          float o[V];
#pragma unroll
          for (int k = 0; k < V; ++k) o[k] = (v[j][k] - mu) * rs * gam[j][k] + bet[j][k];
          st_nt(yr + c0, io<T>::pack(o));
        }
      }
      if (gl == 0) { mean[r * ldm] = mu; rstd[r * ldr] = rs; }
    }
  };
  for (; base < R; base += 2 * stride) {
    step(b0, base);
    if (base + stride < R) step(b1, base + stride);
  }
}

template <typename T, int RW, int NV>
__global__ __launch_bounds__(BWD_BLOCK, sizeof(T) == 2 && RW == 1 && NV <= 2 ? 4 : 1) void ln_bwd_fast(
    const void* __restrict__ d, int64_t ldd, const void* __restrict__ x, int64_t ldx,
    const float* __restrict__ gamma, const float* __restrict__ mean, int64_t ldm,
    const float* __restrict__ rstd, int64_t ldr, void* __restrict__ dx, int64_t lddx,
    int acc_dx, float* __restrict__ part, int64_t R, int64_t C, float invC) {
  constexpr int V = io<T>::VEC, G = WAVE * RW, NG = BWD_BLOCK / G;
  // bf16 rows held by one wave keep gamma in LDS (read where used) rather
  // than in registers, so the raw-pack form below fits four waves per SIMD
  // (measured at d = 768: 634 -> 573 us over 1 GiB).  Rows of several waves
  // keep the unpacked ring with gamma in registers (two waves per SIMD),
  // measured faster for them (d = 3072: 602 vs 660 us; 4096: 527 vs 584 us).
  constexpr bool GLDS = sizeof(T) == 2 && RW == 1;
  constexpr int NVG = GLDS ? 1 : NV;
  extern __shared__ float red[];               // 2C floats (partials fold); bf16: gamma in the first C
  __shared__ float lds[4 * BWD_BLOCK / WAVE];
  int ph = 0;
  const int g = threadIdx.x / G, gl = threadIdx.x % G;
  const int Ci = (int)C;
  float gam[NVG][V], pp[2][NV][V];
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    if constexpr (!GLDS) load_f32s<V, int>(gamma, pack_col<NV, V>(j, gl), Ci, gam[j]);
#pragma unroll
    for (int k = 0; k < V; ++k) { pp[0][j][k] = 0.f; pp[1][j][k] = 0.f; }
  }
  if constexpr (GLDS) {
    for (int c = threadIdx.x; c < Ci; c += BWD_BLOCK) red[c] = gamma[c];
    __syncthreads();
  }
  // gamma of elements k of pack j of this lane (bf16: from LDS)
  auto gam_of = [&](int j, float (&gv)[V]) {
    if constexpr (GLDS) {
      const float4* p = reinterpret_cast<const float4*>(red + pack_col<NV, V>(j, gl));
#pragma unroll
      for (int k = 0; k < V; k += 4) {
        const float4 q = p[k / 4];
        gv[k] = q.x; gv[k + 1] = q.y; gv[k + 2] = q.z; gv[k + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int k = 0; k < V; ++k) gv[k] = gam[j < NVG ? j : 0][k];
    }
  };
  // rows interleaved over the blocks: step k of group g is row
  // blockIdx.x NG + g + k gridDim.x NG, so the rows in flight across the
  // chip at any time form one contiguous window of the tensor
  const int64_t stride = (int64_t)gridDim.x * NG, first = (int64_t)blockIdx.x * NG, end = R;
  RowPacks<T, NV, G> d0, x0, d1, x1;
  {
    const int64_t r = first + g, r1 = first + stride + g;
    d0.load(row_ptr<T>(d, r < end ? r : 0, ldd), gl, Ci, r < end);
    x0.load(row_ptr<T>(x, r < end ? r : 0, ldx), gl, Ci, r < end);
    if (first + stride < end) {
      d1.load(row_ptr<T>(d, r1 < end ? r1 : 0, ldd), gl, Ci, r1 < end);
      x1.load(row_ptr<T>(x, r1 < end ? r1 : 0, ldx), gl, Ci, r1 < end);
    }
  }
  auto step = [&](RowPacks<T, NV, G>& cd, RowPacks<T, NV, G>& cx, int64_t base) {
    const int64_t r = base + g, rn = base + 2 * stride + g;
    const bool active = r < end;
    const float mu = active ? mean[r * ldm] : 0.f;
    const float rs = active ? rstd[r * ldr] : 0.f;
    float dv[NV][V], xh[NV][V];
    cd.unpack(dv);
    cx.unpack(xh);
    if (base + 2 * stride < end) {
      cd.load(row_ptr<T>(d, rn < end ? rn : 0, ldd), gl, Ci, rn < end);
      cx.load(row_ptr<T>(x, rn < end ? rn : 0, ldx), gl, Ci, rn < end);
    }
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c0 = pack_col<NV, V>(j, gl);
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const bool ok = c0 + k < Ci;
        xh[j][k] = ok ? (xh[j][k] - mu) * rs : 0.f;
        const float gv = dv[j][k] * gam[j < NVG ? j : 0][k];
        s1 += gv;
        s2 += gv * xh[j][k];
      }
    }
    group_sum2<RW>(s1, s2, lds, ph);
    if (active) {
      const float a = s1 * invC, b = s2 * invC;
      T* dxr = dx ? row_ptr_w<T>(dx, r, lddx) : nullptr;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int c0 = pack_col<NV, V>(j, gl);
        if (c0 < Ci) {
          float o[V];
#pragma unroll
          for (int k = 0; k < V; ++k) {
            o[k] = rs * (dv[j][k] * gam[j < NVG ? j : 0][k] - a - xh[j][k] * b);
            pp[0][j][k] += dv[j][k] * xh[j][k];
            pp[1][j][k] += dv[j][k];
          }
          if (dxr) store_full<T>(dxr + c0, o, acc_dx != 0);
        }
      }
    }
  };
  // bf16: only raw packs stay live across the reduction (unpacked where
  // used, as in the rms_norm backward), and a ring set is refilled once its
  // row is written; the unpacked f32 ring needs 171-176 VGPRs at two packs
  // per lane (two waves per SIMD), the raw one fits four.
  auto step_raw = [&](RowPacks<T, NV, G>& cd, RowPacks<T, NV, G>& cx, int64_t base) {
    const int64_t r = base + g, rn = base + 2 * stride + g;
    const bool active = r < end;
    const float mu = active ? mean[r * ldm] : 0.f;
    const float rs = active ? rstd[r * ldr] : 0.f;
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      float dv[V], xv[V], gm[V];
      io<T>::unpack(cd.q[j], dv);
      io<T>::unpack(cx.q[j], xv);
      gam_of(j, gm);
#pragma unroll
      for (int k = 0; k < V; ++k) {
        const float gv = dv[k] * gm[k];      // 0 past the row: those packs load as 0
        s1 += gv;
        s2 += gv * ((xv[k] - mu) * rs);
      }
    }
    group_sum2<RW>(s1, s2, lds, ph);
    keep_raw(cd);
    keep_raw(cx);
    if (active) {
      const float a = s1 * invC, b = s2 * invC;
      T* dxr = dx ? row_ptr_w<T>(dx, r, lddx) : nullptr;
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int c0 = pack_col<NV, V>(j, gl);
        if (c0 < Ci) {
          float dv[V], xv[V], gm[V], o[V];
          io<T>::unpack(cd.q[j], dv);
          io<T>::unpack(cx.q[j], xv);
          gam_of(j, gm);
#pragma unroll
          for (int k = 0; k < V; ++k) {
            const float xh = (xv[k] - mu) * rs;
            o[k] = rs * (dv[k] * gm[k] - a - xh * b);
            pp[0][j][k] += dv[k] * xh;
            pp[1][j][k] += dv[k];
          }
          if (dxr) store_full<T>(dxr + c0, o, acc_dx != 0);
        }
      }
    }
    if (base + 2 * stride < end) {
      cd.load(row_ptr<T>(d, rn < end ? rn : 0, ldd), gl, Ci, rn < end);
      cx.load(row_ptr<T>(x, rn < end ? rn : 0, ldx), gl, Ci, rn < end);
    }
  };
  for (int64_t base = first; base < end; base += 2 * stride) {
    if constexpr (GLDS) {
      step_raw(d0, x0, base);
      if (base + stride < end) step_raw(d1, x1, base + stride);
    } else {
      step(d0, x0, base);
      if (base + stride < end) step(d1, x1, base + stride);
    }
  }
  if constexpr (GLDS) __syncthreads();         // every group is done with gamma before the fold reuses red
  if (part) fold_partials<NV, V, G, NG, 2, BWD_BLOCK>(pp, red, part, C);
}

// ================================================================== softmax
// The causal limit is applied per pack (one subtraction per pack, the
// element offsets are immediates), so no per-element column indices stay
// live.
template <typename T, int RW, int NV, int BLOCK, bool CAUSAL>
__global__ __launch_bounds__(BLOCK) void sm_fwd_fast(
    const void* __restrict__ x, int64_t ldx, void* __restrict__ y, int64_t ldy,
    int64_t R, int64_t C, float alpha, int seq_len) {
  constexpr int V = io<T>::VEC, G = WAVE * RW, NG = BLOCK / G;
  __shared__ float lds[4 * BLOCK / WAVE];
  int ph = 0;
  const int g = threadIdx.x / G, gl = threadIdx.x % G;
  const int Ci = (int)C;
  const float NEG_INF = -__builtin_inff();
  const int64_t stride = (int64_t)gridDim.x * NG;
  // Two register sets of raw packs in a ring: the packs of row r+2 strides
  // are fetched into the set of row r as soon as row r is unpacked (after
  // the max barrier), so each row has about one and a half row times of
  // lead; the current row is held once, in f32.
  RowPacks<T, NV, G> b0, b1;
  int64_t base = (int64_t)blockIdx.x * NG;
  b0.load(row_ptr<T>(x, base + g < R ? base + g : 0, ldx), gl, Ci, base + g < R);
  if (base + stride < R) b1.load(row_ptr<T>(x, base + stride + g < R ? base + stride + g : 0, ldx), gl, Ci, base + stride + g < R);
  auto step = [&](RowPacks<T, NV, G>& cur, int64_t bs) {
    const int64_t r = bs + g, rn = bs + 2 * stride + g;
    const bool active = r < R;
    const int lim = !active ? 0 : (CAUSAL ? (int)min(C, (int64_t)(r % seq_len) + 1) : Ci);
    float v[NV][V];
    cur.unpack(v);
    float m = NEG_INF;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int left = lim - pack_col<NV, V>(j, gl);
#pragma unroll
      for (int k = 0; k < V; ++k) {
        v[j][k] = k < left ? alpha * v[j][k] : NEG_INF;
        m = fmaxf(m, v[j][k]);
      }
    }
    m = group_max<RW>(m, lds, ph);
    if (bs + 2 * stride < R) cur.load(row_ptr<T>(x, rn < R ? rn : 0, ldx), gl, Ci, rn < R);
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int k = 0; k < V; ++k) {
        v[j][k] = fast_exp(v[j][k] - m);
        s += v[j][k];
      }
    s = group_sum<RW>(s, lds, ph);
    const float inv = 1.0f / s;
    if (active) {
      T* yr = row_ptr_w<T>(y, r, ldy);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int c0 = pack_col<NV, V>(j, gl);
        if (c0 < Ci) {
          float o[V];
#pragma unroll
          for (int k = 0; k < V; ++k) o[k] = v[j][k] * inv;
          st_nt(yr + c0, io<T>::pack(o));
        }
      }
    }
  };
  for (; base < R; base += 2 * stride) {
    step(b0, base);
    if (base + stride < R) step(b1, base + stride);
  }
}

template <typename T, int RW, int NV, int BLOCK>
__global__ __launch_bounds__(BLOCK) void sm_bwd_fast(
    const void* __restrict__ d, int64_t ldd, const void* __restrict__ y, int64_t ldy,
    void* __restrict__ dx, int64_t lddx, int acc, int64_t R, int64_t C, float alpha) {
  constexpr int V = io<T>::VEC, G = WAVE * RW, NG = BLOCK / G;
  __shared__ float lds[4 * BLOCK / WAVE];
  int ph = 0;
  const int g = threadIdx.x / G, gl = threadIdx.x % G;
  const int Ci = (int)C;
  const int64_t stride = (int64_t)gridDim.x * NG;
  RowPacks<T, NV, G> cd, cy, nd, ny;
  int64_t base = (int64_t)blockIdx.x * NG;
  {
    const int64_t r = base + g;
    cd.load(row_ptr<T>(d, r < R ? r : 0, ldd), gl, Ci, r < R);
    cy.load(row_ptr<T>(y, r < R ? r : 0, ldy), gl, Ci, r < R);
  }
  for (; base < R; base += stride) {
    const int64_t r = base + g, rn = base + stride + g;
    const bool active = r < R;
    if (base + stride < R) {
      nd.load(row_ptr<T>(d, rn < R ? rn : 0, ldd), gl, Ci, rn < R);
      ny.load(row_ptr<T>(y, rn < R ? rn : 0, ldy), gl, Ci, rn < R);
    }
    float dv[NV][V], yv[NV][V];
    cd.unpack(dv);
    cy.unpack(yv);
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < NV; ++j)
#pragma unroll
      for (int k = 0; k < V; ++k) dot += dv[j][k] * yv[j][k];
    dot = group_sum<RW>(dot, lds, ph);
    if (active) {
      T* dxr = row_ptr_w<T>(dx, r, lddx);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int c0 = pack_col<NV, V>(j, gl);
        if (c0 < Ci) {
          float o[V];
#pragma unroll
          for (int k = 0; k < V; ++k) o[k] = alpha * yv[j][k] * (dv[j][k] - dot);
          store_full<T>(dxr + c0, o, acc != 0);
        }
      }
    }
    cd = nd;
    cy = ny;
  }
}

// =============================================================== generic path
// Rows the register-resident kernels do not take go to the streaming
// kernels of rowstream.hip.  What remains here: the parameter-gradient
// partials of rows whose starts are not 16-byte aligned (the streaming
// backward then keeps no per-thread column partials), by columns.
template <typename T> __device__ __forceinline__ float gl1(const void* p, int64_t r, int64_t ld, int64_t c) {
  return io<T>::ld(reinterpret_cast<const T*>(p) + r * ld + c);
}

// Parameter-gradient partials of rows whose starts are not 16-byte aligned:
// block (bx, by) sums rows [by*rpb, (by+1)*rpb) of columns bx*256 + t, one
// column per thread, eight rows' loads in flight, added in row order; one
// partial row (NP vectors of C) per block row by.  kind 0: d*x*ir (rms_norm
// dgamma); kind 1: d*xhat and d (layer_norm dgamma, dbeta).
template <typename T, int KIND>
__global__ __launch_bounds__(GEN_BLOCK) void norm_partials_gen(
    const void* d, int64_t ldd, const void* x, int64_t ldx, const float* st0, int64_t ld0,
    const float* st1, int64_t ld1, float* part, int64_t R, int64_t C, int64_t rpb) {
  constexpr int NP = KIND == 0 ? 1 : 2, U = 8;
  const int64_t start = (int64_t)blockIdx.y * rpb, end = min(R, start + rpb);
  const int64_t c = (int64_t)blockIdx.x * GEN_BLOCK + threadIdx.x;
  if (c >= C) return;
  float a = 0.f, b = 0.f;
  int64_t r = start;
  for (; r + U <= end; r += U) {
    float dv[U], xv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) { dv[u] = gl1<T>(d, r + u, ldd, c); xv[u] = gl1<T>(x, r + u, ldx, c); }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (KIND == 0) a += dv[u] * xv[u] * st0[(r + u) * ld0];
      else { a += dv[u] * (xv[u] - st0[(r + u) * ld0]) * st1[(r + u) * ld1]; b += dv[u]; }
    }
  }
  for (; r < end; ++r) {
    const float dv = gl1<T>(d, r, ldd, c), xv = gl1<T>(x, r, ldx, c);
    if (KIND == 0) a += dv * xv * st0[r * ld0];
    else { a += dv * (xv - st0[r * ld0]) * st1[r * ld1]; b += dv; }
  }
  float* out = part + (int64_t)blockIdx.y * NP * C;
  out[c] = a;
  if (KIND == 1) out[C + c] = b;
}

// ============================================================ column sums
// Second pass: column c of the partial rows, summed over b = 0..P-1 in a
// fixed order, goes to out0[c] for c < n0 and to out1[c - n0] otherwise
// (the two parameter gradients of layer_norm in one launch), each stored or
// added (acc0 / acc1).  A 512-thread block takes 32 columns (one 128-byte
// segment of each partial row): thread t sums column t % 32 over the
// partial rows b = p, p + 16, ... of its phase p = t / 32 (FOLD_U rows'
// loads in flight, added in b order), then the 16 phase sums are added in
// phase order.  Against 64 columns per block this spreads the pass over
// twice the blocks (a 4096-wide gradient: 128); 16 columns per block
// (64-byte segments) measured twice the fetched bytes and was slower.
constexpr int FOLD_T = 512, FOLD_W = 32, FOLD_PH = FOLD_T / FOLD_W, FOLD_U = 32;

__global__ __launch_bounds__(FOLD_T) void fold_columns(const float* __restrict__ part, int64_t P,
                                                      int64_t stride, int64_t C, float* __restrict__ out0,
                                                      int acc0, int64_t n0, float* __restrict__ out1,
                                                      int acc1) {
  __shared__ float lds[FOLD_PH][FOLD_W];
  const int ph = threadIdx.x / FOLD_W, cl = threadIdx.x % FOLD_W;
  const int64_t c = (int64_t)blockIdx.x * FOLD_W + cl;
  float s = 0.f;
  if (c < C) {
    for (int64_t b0 = ph; b0 < P; b0 += FOLD_PH * FOLD_U) {
      float v[FOLD_U];
#pragma unroll
      for (int u = 0; u < FOLD_U; ++u) {
        const int64_t b = b0 + FOLD_PH * u;
        v[u] = b < P ? part[b * stride + c] : 0.f;
      }
#pragma unroll
      for (int u = 0; u < FOLD_U; ++u)
        if (b0 + FOLD_PH * u < P) s += v[u];
    }
  }
  lds[ph][cl] = s;
  __syncthreads();
  if (ph == 0 && c < C) {
    float t = lds[0][cl];
#pragma unroll
    for (int i = 1; i < FOLD_PH; ++i) t += lds[i][cl];
    float* o = c < n0 ? out0 + c : out1 + (c - n0);
    *o = (c < n0 ? acc0 : acc1) ? acc_add(*o, t) : t;
  }
}

// First pass of a plain column sum (add_bias backward): a 1024-thread block
// holds TPC threads per row (one 16-byte pack each) and 1024/TPC row phases;
// block (bx, by) covers packs [bx*TPC, ...) of rows by*nph + phase + k*gy*nph.  The row
// phases are folded in LDS in phase order; one partial row per block row.
template <typename T>
__global__ __launch_bounds__(1024) void colsum_partials(
    const void* __restrict__ d, int64_t ldd, int64_t R, int64_t C, int tpc,
    float* __restrict__ part) {
  constexpr int V = io<T>::VEC;
  extern __shared__ float red[];                 // tpc * V floats
  const int ph = threadIdx.x / tpc, t = threadIdx.x % tpc, nph = 1024 / tpc;
  const int64_t c0 = ((int64_t)blockIdx.x * tpc + t) * V;
  // rows interleaved over the block rows (contiguous window in flight)
  const int64_t end = R, rstep = (int64_t)gridDim.y * nph;
  float a[V];
#pragma unroll
  for (int k = 0; k < V; ++k) a[k] = 0.f;
  if (c0 < C) {
    int64_t r = (int64_t)blockIdx.y * nph + ph;
    // eight rows' packs per group, added in row order; the next group's
    // loads are issued before the current group is added, so a thread
    // always has a group in flight
    constexpr int U = 8;
    auto load8 = [&](uint4 (&q)[U], int64_t r0) {
#pragma unroll
      for (int u = 0; u < U; ++u) q[u] = load_raw<T>(row_ptr<T>(d, r0 + u * rstep, ldd), c0, C);
    };
    auto add8 = [&](const uint4 (&q)[U]) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float v[V];
        io<T>::unpack(q[u], v);
#pragma unroll
        for (int k = 0; k < V; ++k) a[k] += v[k];
      }
    };
    if (r + (U - 1) * rstep < end) {
      uint4 qa[U], qb[U];
      load8(qa, r);
      for (;;) {
        const int64_t r2 = r + U * rstep;
        const bool m2 = r2 + (U - 1) * rstep < end;
        if (m2) load8(qb, r2);
        add8(qa);
        r = r2;
        if (!m2) break;
        const int64_t r3 = r + U * rstep;
        const bool m3 = r3 + (U - 1) * rstep < end;
        if (m3) load8(qa, r3);
        add8(qb);
        r = r3;
        if (!m3) break;
      }
    }
    for (; r < end; r += rstep) {
      float v0[V];
      load_pack<T>(row_ptr<T>(d, r, ldd), c0, C, v0, 0.f);
#pragma unroll
      for (int k = 0; k < V; ++k) a[k] += v0[k];
    }
  }
  for (int p = 0; p < nph; ++p) {
    if (ph == p)
#pragma unroll
      for (int k = 0; k < V; ++k) red[t * V + k] = (p == 0) ? a[k] : red[t * V + k] + a[k];
    __syncthreads();
  }
  float* out = part + (int64_t)blockIdx.y * C;
  for (int i = threadIdx.x; i < tpc * V; i += 1024) {
    const int64_t c = (int64_t)blockIdx.x * tpc * V + i;
    if (c < C) out[c] = red[i];
  }
}

// Generic first pass for rows that are not 16-byte aligned: block y sums
// its row chunk for every column (threads stride over columns).
template <typename T>
__global__ __launch_bounds__(GEN_BLOCK) void colsum_partials_gen(
    const void* __restrict__ d, int64_t ldd, int64_t R, int64_t C, int64_t rpb,
    float* __restrict__ part) {
  const int64_t start = (int64_t)blockIdx.y * rpb, end = min(R, start + rpb);
  for (int64_t c = threadIdx.x; c < C; c += GEN_BLOCK) {
    float a = 0.f;
    for (int64_t r = start; r < end; ++r) a += gl1<T>(d, r, ldd, c);
    part[(int64_t)blockIdx.y * C + c] = a;
  }
}

__global__ void fill_f32_k(float* p, int64_t n, float v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

// ============================================================== dispatching
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool is_bwd(RowKind k) { return k == RK_RMS_BWD || k == RK_LN_BWD; }

// Register-resident shapes each kind may use: waves per row, block size and
// the largest packs-per-thread for f32 / bf16.  The limits keep every
// selectable instantiation free of register spills (checked in the gfx950
// ISA): 1024-thread blocks cap a thread at 128 VGPRs, 512-thread blocks at
// 256, and the kernels hold the current and the prefetched row.
struct RowShape { int rw, block, nv_f32, nv_bf16; };

int row_shapes(RowKind k, const RowShape** out) {
  static const RowShape fwd[] = {{1, 256, 8, 4}, {4, 256, 8, 4}, {8, 512, 8, 8}};
  static const RowShape lnf[] = {{1, 256, 8, 4}, {4, 256, 8, 4}, {8, 512, 8, 4}};
  static const RowShape smb[] = {{1, 256, 8, 4}, {4, 256, 8, 4}, {16, 1024, 4, 4}};
  // bf16 rms_norm rows of up to 4 packs per lane stay on one wave (d = 2048
  // over 1 GiB: 622 -> 610 us); layer_norm keeps them on 4 waves (562 vs
  // 638 us), its backward holding more per lane
  static const RowShape rmsb[] = {{1, BWD_BLOCK, 4, 4}, {4, BWD_BLOCK, 4, 2}, {8, BWD_BLOCK, 4, 2}};
  static const RowShape bwd[] = {{1, BWD_BLOCK, 4, 2}, {4, BWD_BLOCK, 4, 2}, {8, BWD_BLOCK, 4, 2}};
  if (k == RK_SM_BWD) *out = smb;
  else if (k == RK_RMS_BWD) *out = rmsb;
  else if (is_bwd(k)) *out = bwd;
  else if (k == RK_LN_FWD) *out = lnf;
  else *out = fwd;
  return 3;
}

}  // namespace

RowPlan plan_rows(RowKind kind, int dtype, int64_t R, int64_t C, bool aligned) {
  RowPlan p{};
  const int V = dtype == XT_F32 ? 4 : 8;
  const int64_t packs = cdiv(C, V);
  p.fast = false;
  if (aligned && C > 0 && C % V == 0) {
    const RowShape* sh;
    const int n = row_shapes(kind, &sh);
    for (int i = 0; i < n && !p.fast; ++i) {
      const int64_t need = cdiv(packs, (int64_t)WAVE * sh[i].rw);
      int nv = 1;
      while (nv < need) nv *= 2;
      const int nvmax = dtype == XT_F32 ? sh[i].nv_f32 : sh[i].nv_bf16;
      if (nv > nvmax) continue;
      // A backward group whose share of the rows is under 8 never fills its
      // prefetch ring; with rows that wide (4 packs per lane) a wider group
      // (fewer registers, more groups per CU) is used instead when one fits
      // (GPT-2-small-shaped layer_norm backward: 29 -> 25 us).
      if (is_bwd(kind) && nv >= 4 && i + 1 < n) {
        const int64_t groups = sh[i].block / (WAVE * sh[i].rw);
        const int64_t grid = std::min<int64_t>(cdiv(R, groups), BWD_GRID_MAX);
        if (R < 8 * grid * groups) continue;
      }
      p.fast = true; p.rw = sh[i].rw; p.nv = nv; p.block = sh[i].block;
    }
    // backward folds parameter partials in LDS: keep them within 64 KiB
    const int np = kind == RK_LN_BWD ? 2 : 1;
    if (is_bwd(kind) && (int64_t)np * C * 4 > 65536) p.fast = false;
    // f32 rms_norm rows past 8192 columns: the register-row forward of
    // rowstream.hip (one row per 1024-thread block, two blocks per CU) is
    // faster than a multi-wave row group here (16384 columns, 1 GiB:
    // 410 -> 381 us); the layer_norm forward does not fit its registers
    // (426 vs 394 us) and keeps this kernel
    if (kind == RK_RMS_FWD && dtype == XT_F32 && C > 8192) p.fast = false;
  }
  if (p.fast) {
    p.groups = p.block / (WAVE * p.rw);
    int64_t g;
    if (is_bwd(kind)) g = std::min<int64_t>(cdiv(R, p.groups), BWD_GRID_MAX);
    else if (kind == RK_RMS_FWD || kind == RK_LN_FWD) g = cdiv(R, (int64_t)p.groups * NORM_FWD_STEPS);
    else g = p.rw <= 4 ? cdiv(R, p.groups)
                       : std::min<int64_t>(cdiv(R, p.groups), kind == RK_SM_BWD ? 2 * LONG_ROW_GRID : LONG_ROW_GRID);
    p.grid = (int)std::max<int64_t>(1, std::min<int64_t>(g, INT32_MAX));
  } else {
    // streaming kernels: one row per 1024-thread block step; a backward's
    // blocks each write one partial row of the parameter gradients
    p.rw = 16; p.nv = 0; p.block = 1024; p.groups = 1;
    p.grid = is_bwd(kind) ? stream_bwd_grid(R) : (int)std::max<int64_t>(1, std::min<int64_t>(R, LONG_ROW_GRID));
  }
  return p;
}

// Grid of a streaming backward that writes no parameter-gradient partial
// rows: one 1024-thread block per row step, up to LONG_ROW_GRID blocks.
static int dx_grid(int64_t R) { return (int)std::max<int64_t>(1, std::min<int64_t>(R, LONG_ROW_GRID)); }

size_t row_bwd_workspace(RowKind kind, int dtype, int64_t R, int64_t C, bool aligned) {
  if (R <= 0 || C <= 0) return 0;
  const RowPlan p = plan_rows(kind, dtype, R, C, aligned);
  const int np = kind == RK_LN_BWD ? 2 : 1;
  return (size_t)p.grid * np * C * sizeof(float);
}

// Blocks of kernel f (block threads, shm bytes of dynamic LDS) that the
// current device holds at once: occupancy per CU times the CU count, cached
// per (device, kernel, shape).  Row kernels loop over rows, so a grid of
// this size keeps every block resident (no second round of blocks) and
// lets each block run its prefetch pipeline over many rows.
static int resident_blocks(const void* f, int block, size_t shm) {
  static std::mutex mu;
  static std::map<std::tuple<int, const void*, int, size_t>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1 << 30;
  const auto key = std::make_tuple(dev, f, block, shm);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, f, block, shm) != hipSuccess || cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();
    return 1 << 30;                               // unknown: keep the planned grid
  }
  return cache[key] = per_cu * cus;
}

static int fit_grid(const void* f, int block, size_t shm, int want) {
  return std::max(1, std::min(want, resident_blocks(f, block, shm)));
}

// Dispatch over the (RW, NV, BLOCK) shapes plan_rows can return.
#define XT_ROW_CASE(RW_, NV_, B_, ...) \
  else if (p.rw == RW_ && p.nv == NV_ && p.block == B_) { constexpr int RW = RW_, NV = NV_, BLOCK = B_; (void)BLOCK; __VA_ARGS__; }
#define XT_ROW_SWITCH_FWD(...) \
  do { \
    if (false) {} \
    XT_ROW_CASE(1, 1, 256, __VA_ARGS__) XT_ROW_CASE(1, 2, 256, __VA_ARGS__) XT_ROW_CASE(1, 4, 256, __VA_ARGS__) XT_ROW_CASE(1, 8, 256, __VA_ARGS__) XT_ROW_CASE(4, 1, 256, __VA_ARGS__) XT_ROW_CASE(4, 2, 256, __VA_ARGS__) XT_ROW_CASE(4, 4, 256, __VA_ARGS__) XT_ROW_CASE(4, 8, 256, __VA_ARGS__) XT_ROW_CASE(8, 1, 512, __VA_ARGS__) XT_ROW_CASE(8, 2, 512, __VA_ARGS__) XT_ROW_CASE(8, 4, 512, __VA_ARGS__) XT_ROW_CASE(8, 8, 512, __VA_ARGS__) \
    else return hipErrorInvalidValue; \
  } while (0)
#define XT_ROW_SWITCH_SMB(...) \
  do { \
    if (false) {} \
    XT_ROW_CASE(1, 1, 256, __VA_ARGS__) XT_ROW_CASE(1, 2, 256, __VA_ARGS__) XT_ROW_CASE(1, 4, 256, __VA_ARGS__) XT_ROW_CASE(1, 8, 256, __VA_ARGS__) XT_ROW_CASE(4, 1, 256, __VA_ARGS__) XT_ROW_CASE(4, 2, 256, __VA_ARGS__) XT_ROW_CASE(4, 4, 256, __VA_ARGS__) XT_ROW_CASE(4, 8, 256, __VA_ARGS__) XT_ROW_CASE(16, 1, 1024, __VA_ARGS__) XT_ROW_CASE(16, 2, 1024, __VA_ARGS__) XT_ROW_CASE(16, 4, 1024, __VA_ARGS__) XT_ROW_CASE(16, 8, 1024, __VA_ARGS__) \
    else return hipErrorInvalidValue; \
  } while (0)
#define XT_ROW_SWITCH_BWD(...) \
  do { \
    if (false) {} \
    XT_ROW_CASE(1, 1, BWD_BLOCK, __VA_ARGS__) XT_ROW_CASE(1, 2, BWD_BLOCK, __VA_ARGS__) XT_ROW_CASE(1, 4, BWD_BLOCK, __VA_ARGS__) XT_ROW_CASE(4, 1, BWD_BLOCK, __VA_ARGS__) XT_ROW_CASE(4, 2, BWD_BLOCK, __VA_ARGS__) XT_ROW_CASE(4, 4, BWD_BLOCK, __VA_ARGS__) XT_ROW_CASE(8, 1, BWD_BLOCK, __VA_ARGS__) XT_ROW_CASE(8, 2, BWD_BLOCK, __VA_ARGS__) XT_ROW_CASE(8, 4, BWD_BLOCK, __VA_ARGS__) \
    else return hipErrorInvalidValue; \
  } while (0)


static bool aligned16(const xt_tensor& t) {
  const int es = t.dtype == XT_F32 ? 4 : 2;
  return (((uintptr_t)t.data) & 15) == 0 && ((t.ld * es) & 15) == 0;
}

template <typename T>
static hipError_t rms_fwd_t(const xt_tensor& x, const float* gamma, const xt_tensor& y,
                            const xt_tensor& ir, float eps, hipStream_t s) {
  const int64_t R = x.rows, C = x.cols;
  const float invC = 1.0f / (float)C;
  const RowPlan p = plan_rows(RK_RMS_FWD, x.dtype, R, C, aligned16(x) && aligned16(y));
  if (p.fast) {
    XT_ROW_SWITCH_FWD(
        auto kf = rms_fwd_fast<T, RW, NV, BLOCK>;
        kf<<<p.grid, BLOCK, 0, s>>>(x.data, x.ld, gamma, y.data, y.ld, (float*)ir.data, ir.ld, R, C, eps, invC));
    return hipGetLastError();
  }
  return launch_rms_fwd_stream(x, gamma, y, ir, eps, p.grid, s);
}

hipError_t launch_rms_fwd(const xt_tensor& x, const float* gamma, const xt_tensor& y,
                          const xt_tensor& inv_rms, float eps, hipStream_t s) {
  if (x.rows == 0) return hipSuccess;
  return x.dtype == XT_F32 ? rms_fwd_t<float>(x, gamma, y, inv_rms, eps, s)
                           : rms_fwd_t<bf16_t>(x, gamma, y, inv_rms, eps, s);
}

// Largest block count whose partial rows (np vectors of C floats) fit ws_bytes.
static RowPlan clamp_to_workspace(RowPlan p, int np, int64_t C, size_t ws_bytes, bool want) {
  if (!want) return p;
  const int64_t fit = (int64_t)(ws_bytes / ((size_t)np * C * sizeof(float)));
  if (fit < p.grid) p.grid = (int)fit;
  return p;
}

template <typename T>
static hipError_t rms_bwd_t(const xt_tensor& d, const xt_tensor& x, const float* gamma,
                            const xt_tensor& ir, const xt_tensor* dx, bool acc_dx, float* dgamma,
                            bool acc_dg, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t R = d.rows, C = d.cols;
  const float invC = 1.0f / (float)C;
  const bool al = aligned16(d) && aligned16(x) && (!dx || aligned16(*dx));
  RowPlan p = clamp_to_workspace(plan_rows(RK_RMS_BWD, d.dtype, R, C, al), 1, C, ws_bytes, dgamma != nullptr);
  if (p.grid < 1) return hipErrorInvalidValue;
  float* part = dgamma ? (float*)ws : nullptr;
  if (p.fast) {
    const size_t shm = dgamma ? (size_t)C * sizeof(float) : 0;
    XT_ROW_SWITCH_BWD(
      auto kf = rms_bwd_fast<T, RW, NV>;
      p.grid = fit_grid((const void*)kf, BWD_BLOCK, shm, p.grid);
      kf<<<p.grid, BWD_BLOCK, shm, s>>>(d.data, d.ld, x.data, x.ld, gamma, (const float*)ir.data, ir.ld,
                                        dx ? dx->data : nullptr, dx ? dx->ld : 0, acc_dx, part, R, C, invC));
  } else {
    // streaming rows: dgamma partials in registers when every row starts
    // 16-byte aligned, else by a column pass
    const bool own = dgamma && stream_owns_partials(d.dtype, C, d, x, dx);
    hipError_t e = hipSuccess;
    // without owned partials the dx kernel writes no partial rows: it takes
    // as many blocks as the rows allow, several resident per CU
    if (dx || own) e = launch_rms_bwd_stream(d, x, gamma, ir, dx, acc_dx, own ? part : nullptr, own ? p.grid : dx_grid(R), s);
    if (e != hipSuccess) return e;
    if (dgamma && !own)
      norm_partials_gen<T, 0><<<dim3((unsigned)cdiv(C, GEN_BLOCK), p.grid), GEN_BLOCK, 0, s>>>(
          d.data, d.ld, x.data, x.ld, (const float*)ir.data, ir.ld, nullptr, 0, part, R, C, cdiv(R, p.grid));
  }
  if (dgamma) fold_columns<<<(unsigned)cdiv(C, FOLD_W), FOLD_T, 0, s>>>(part, p.grid, C, C, dgamma, acc_dg, C, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_rms_bwd(const xt_tensor& d, const xt_tensor& x, const float* gamma,
                          const xt_tensor& inv_rms, const xt_tensor* dx, bool acc_dx,
                          float* dgamma, bool acc_dgamma, void* ws, size_t ws_bytes, hipStream_t s) {
  if (d.rows == 0) {                 // dgamma is a sum over no rows: zero
    if (dgamma && !acc_dgamma) return launch_fill_f32(dgamma, d.cols, 0.f, s);
    return hipSuccess;
  }
  return d.dtype == XT_F32 ? rms_bwd_t<float>(d, x, gamma, inv_rms, dx, acc_dx, dgamma, acc_dgamma, ws, ws_bytes, s)
                           : rms_bwd_t<bf16_t>(d, x, gamma, inv_rms, dx, acc_dx, dgamma, acc_dgamma, ws, ws_bytes, s);
}

template <typename T>
static hipError_t ln_fwd_t(const xt_tensor& x, const float* gamma, const float* beta,
                           const xt_tensor& y, const xt_tensor& mean, const xt_tensor& rstd,
                           float eps, hipStream_t s) {
  const int64_t R = x.rows, C = x.cols;
  const float invC = 1.0f / (float)C;
  const RowPlan p = plan_rows(RK_LN_FWD, x.dtype, R, C, aligned16(x) && aligned16(y));
  if (p.fast) {
    XT_ROW_SWITCH_FWD(
        auto kf = ln_fwd_fast<T, RW, NV, BLOCK>;
        kf<<<p.grid, BLOCK, 0, s>>>(x.data, x.ld, gamma, beta, y.data, y.ld, (float*)mean.data, mean.ld, (float*)rstd.data, rstd.ld, R, C, eps, invC));
    return hipGetLastError();
  }
  return launch_ln_fwd_stream(x, gamma, beta, y, mean, rstd, eps, p.grid, s);
}

hipError_t launch_ln_fwd(const xt_tensor& x, const float* gamma, const float* beta,
                         const xt_tensor& y, const xt_tensor& mean, const xt_tensor& rstd,
                         float eps, hipStream_t s) {
  if (x.rows == 0) return hipSuccess;
  return x.dtype == XT_F32 ? ln_fwd_t<float>(x, gamma, beta, y, mean, rstd, eps, s)
                           : ln_fwd_t<bf16_t>(x, gamma, beta, y, mean, rstd, eps, s);
}

template <typename T>
static hipError_t ln_bwd_t(const xt_tensor& d, const xt_tensor& x, const float* gamma,
                           const xt_tensor& mean, const xt_tensor& rstd, const xt_tensor* dx,
                           bool acc_dx, float* dgamma, bool acc_dg, float* dbeta, bool acc_db,
                           void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t R = d.rows, C = d.cols;
  const float invC = 1.0f / (float)C;
  const bool al = aligned16(d) && aligned16(x) && (!dx || aligned16(*dx));
  const bool want_p = dgamma || dbeta;
  RowPlan p = clamp_to_workspace(plan_rows(RK_LN_BWD, d.dtype, R, C, al), 2, C, ws_bytes, want_p);
  if (p.grid < 1) return hipErrorInvalidValue;
  float* part = want_p ? (float*)ws : nullptr;
  if (p.fast) {
    // partial-row fold: 2C floats; one-wave bf16 rows also stage gamma (C floats) there
    const size_t shm = (want_p ? (size_t)2 * C : sizeof(T) == 2 && p.rw == 1 ? (size_t)C : 0) * sizeof(float);
    XT_ROW_SWITCH_BWD(
      auto kf = ln_bwd_fast<T, RW, NV>;
      p.grid = fit_grid((const void*)kf, BWD_BLOCK, shm, p.grid);
      kf<<<p.grid, BWD_BLOCK, shm, s>>>(d.data, d.ld, x.data, x.ld, gamma, (const float*)mean.data, mean.ld,
                                        (const float*)rstd.data, rstd.ld, dx ? dx->data : nullptr, dx ? dx->ld : 0,
                                        acc_dx, part, R, C, invC));
  } else {
    const bool own = want_p && stream_owns_partials(d.dtype, C, d, x, dx);
    hipError_t e = hipSuccess;
    if (dx || own) e = launch_ln_bwd_stream(d, x, gamma, mean, rstd, dx, acc_dx, own ? part : nullptr, own ? p.grid : dx_grid(R), s);
    if (e != hipSuccess) return e;
    if (want_p && !own)
      norm_partials_gen<T, 1><<<dim3((unsigned)cdiv(C, GEN_BLOCK), p.grid), GEN_BLOCK, 0, s>>>(
          d.data, d.ld, x.data, x.ld, (const float*)mean.data, mean.ld, (const float*)rstd.data, rstd.ld, part, R, C,
          cdiv(R, p.grid));
  }
  if (dgamma && dbeta)        // partial rows are [dgamma | dbeta]: one fold over 2C columns
    fold_columns<<<(unsigned)cdiv(2 * C, FOLD_W), FOLD_T, 0, s>>>(part, p.grid, 2 * C, 2 * C, dgamma, acc_dg, C, dbeta, acc_db);
  else if (dgamma)
    fold_columns<<<(unsigned)cdiv(C, FOLD_W), FOLD_T, 0, s>>>(part, p.grid, 2 * C, C, dgamma, acc_dg, C, nullptr, 0);
  else if (dbeta)
    fold_columns<<<(unsigned)cdiv(C, FOLD_W), FOLD_T, 0, s>>>(part + C, p.grid, 2 * C, C, dbeta, acc_db, C, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_ln_bwd(const xt_tensor& d, const xt_tensor& x, const float* gamma,
                         const xt_tensor& mean, const xt_tensor& rstd,
                         const xt_tensor* dx, bool acc_dx, float* dgamma, bool acc_dgamma,
                         float* dbeta, bool acc_dbeta, void* ws, size_t ws_bytes, hipStream_t s) {
  if (d.rows == 0) {                 // dgamma, dbeta are sums over no rows: zero
    hipError_t e = hipSuccess;
    if (dgamma && !acc_dgamma) e = launch_fill_f32(dgamma, d.cols, 0.f, s);
    if (e == hipSuccess && dbeta && !acc_dbeta) e = launch_fill_f32(dbeta, d.cols, 0.f, s);
    return e;
  }
  return d.dtype == XT_F32
             ? ln_bwd_t<float>(d, x, gamma, mean, rstd, dx, acc_dx, dgamma, acc_dgamma, dbeta, acc_dbeta, ws, ws_bytes, s)
             : ln_bwd_t<bf16_t>(d, x, gamma, mean, rstd, dx, acc_dx, dgamma, acc_dgamma, dbeta, acc_dbeta, ws, ws_bytes, s);
}

template <typename T>
static hipError_t sm_fwd_t(const xt_tensor& x, const xt_tensor& y, float alpha, int causal,
                           int seq_len, hipStream_t s) {
  const int64_t R = x.rows, C = x.cols;
  const RowPlan p = plan_rows(RK_SM_FWD, x.dtype, R, C, aligned16(x) && aligned16(y));
  if (p.fast) {
    XT_ROW_SWITCH_FWD(
        auto kf = causal ? sm_fwd_fast<T, RW, NV, BLOCK, true> : sm_fwd_fast<T, RW, NV, BLOCK, false>;
        kf<<<p.grid, BLOCK, 0, s>>>(x.data, x.ld, y.data, y.ld, R, C, alpha, seq_len));
    return hipGetLastError();
  }
  return launch_sm_fwd_stream(x, y, alpha, causal, seq_len, p.grid, s);
}

hipError_t launch_softmax_fwd(const xt_tensor& x, const xt_tensor& y, float alpha,
                              int causal, int seq_len, hipStream_t s) {
  if (x.rows == 0) return hipSuccess;
  return x.dtype == XT_F32 ? sm_fwd_t<float>(x, y, alpha, causal, seq_len, s)
                           : sm_fwd_t<bf16_t>(x, y, alpha, causal, seq_len, s);
}

template <typename T>
static hipError_t sm_bwd_t(const xt_tensor& d, const xt_tensor& y, const xt_tensor& dx, bool acc,
                           float alpha, hipStream_t s) {
  const int64_t R = d.rows, C = d.cols;
  const RowPlan p = plan_rows(RK_SM_BWD, d.dtype, R, C, aligned16(d) && aligned16(y) && aligned16(dx));
  if (p.fast) {
    XT_ROW_SWITCH_SMB(
        sm_bwd_fast<T, RW, NV, BLOCK><<<p.grid, BLOCK, 0, s>>>(d.data, d.ld, y.data, y.ld, dx.data, dx.ld, acc, R, C, alpha));
    return hipGetLastError();
  }
  return launch_sm_bwd_stream(d, y, dx, acc, alpha, dx_grid(R), s);   // no partial rows: as for the forward
}

hipError_t launch_softmax_bwd(const xt_tensor& d, const xt_tensor& y, const xt_tensor& dx,
                              bool acc, float alpha, hipStream_t s) {
  if (d.rows == 0) return hipSuccess;
  return d.dtype == XT_F32 ? sm_bwd_t<float>(d, y, dx, acc, alpha, s)
                           : sm_bwd_t<bf16_t>(d, y, dx, acc, alpha, s);
}

// Column-sum geometry shared by the workspace query and the launch.
struct ColsumPlan { int tpc; unsigned gx, gy; int64_t rpb; };

static ColsumPlan colsum_plan(int dtype, int64_t R, int64_t C) {
  const int V = dtype == XT_F32 ? 4 : 8;
  const int64_t packs = cdiv(C, V);
  int tpc = 64;
  while (tpc < packs && tpc < 1024) tpc *= 2;
  ColsumPlan p;
  p.tpc = tpc;
  p.gx = (unsigned)cdiv(packs, tpc);
  const int64_t gy_max = std::max<int64_t>(1, 256 / (int64_t)p.gx);
  p.gy = (unsigned)std::max<int64_t>(1, std::min<int64_t>(gy_max, cdiv(R, 1024 / tpc)));
  p.rpb = cdiv(R, p.gy);
  return p;
}

size_t colsum_workspace(int dtype, int64_t R, int64_t C) {
  if (R <= 0 || C <= 0) return 0;
  return (size_t)colsum_plan(dtype, R, C).gy * C * sizeof(float);
}

hipError_t launch_colsum(const xt_tensor& d, float* out, bool acc, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t R = d.rows, C = d.cols;
  if (C == 0) return hipSuccess;
  if (R == 0) {
    if (!acc) fill_f32_k<<<(unsigned)cdiv(C, 256), 256, 0, s>>>(out, C, 0.f);
    return hipGetLastError();
  }
  ColsumPlan p = colsum_plan(d.dtype, R, C);
  // never write more partial rows than the workspace holds
  const int64_t fit = (int64_t)(ws_bytes / ((size_t)C * sizeof(float)));
  if (fit < 1) return hipErrorInvalidValue;
  if ((int64_t)p.gy > fit) { p.gy = (unsigned)fit; p.rpb = cdiv(R, p.gy); }
  float* part = (float*)ws;
  const bool al = aligned16(d);
  const int V = d.dtype == XT_F32 ? 4 : 8;
  if (al) {
    const size_t shm = (size_t)p.tpc * V * sizeof(float);
    if (d.dtype == XT_F32)
      colsum_partials<float><<<dim3(p.gx, p.gy), 1024, shm, s>>>(d.data, d.ld, R, C, p.tpc, part);
    else
      colsum_partials<bf16_t><<<dim3(p.gx, p.gy), 1024, shm, s>>>(d.data, d.ld, R, C, p.tpc, part);
  } else {
    if (d.dtype == XT_F32)
      colsum_partials_gen<float><<<dim3(1, p.gy), GEN_BLOCK, 0, s>>>(d.data, d.ld, R, C, p.rpb, part);
    else
      colsum_partials_gen<bf16_t><<<dim3(1, p.gy), GEN_BLOCK, 0, s>>>(d.data, d.ld, R, C, p.rpb, part);
  }
  fold_columns<<<(unsigned)cdiv(C, FOLD_W), FOLD_T, 0, s>>>(part, p.gy, C, C, out, acc, C, nullptr, 0);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n == 0) return hipSuccess;
  fill_f32_k<<<(unsigned)std::min<int64_t>(cdiv(n, 256), 4096), 256, 0, s>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace xt
