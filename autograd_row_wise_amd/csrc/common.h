// Device helpers shared by the HIP kernels of libxt (gfx950, wave64).
//
// Storage types: f32 and bf16 (carried as uint16_t bit patterns, the upper
// half of an IEEE binary32).  All arithmetic is f32.  Global traffic moves
// in 16-byte packs (4 f32 or 8 bf16) so every wave issues 1 KiB per
// global_load_dwordx4 / global_store_dwordx4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xt {

typedef uint16_t bf16_t;

constexpr int WAVE = 64;

// ---------------------------------------------------------------- bf16 <-> f32
__device__ __forceinline__ float bf2f(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two f32 -> packed bf16 pair (low = a), round-to-nearest-even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  f32x2_t v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ uint32_t f2bf(float f) { return f2bf2(f, 0.f) & 0xffffu; }

// Accumulating add that the compiler may not fuse with a preceding multiply:
// a gradient contribution is rounded to f32 first, then added (one rounding
// per push, in push order).
__device__ __forceinline__ float acc_add(float a, float b) {
#pragma clang fp contract(off)
  return a + b;
}

// ------------------------------------------------------- streaming 16-byte I/O
// Tensors here are streamed once per kernel, so global traffic uses the
// nontemporal cache policy (measured on MI355X: plain copy ~5.3 TB/s with
// grid-stride loops, 6.3 TB/s with one pack per thread over a full grid and
// nontemporal stores; reads 6.4 -> 7.0 TB/s with nontemporal loads).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 ld_nt(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void st_nt(void* p, const uint4& q) {
  const u32x4_t v = {q.x, q.y, q.z, q.w};
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4_t*>(p));
}

// ---------------------------------------------------------------- type traits
template <typename T> struct io;

template <> struct io<float> {
  static constexpr int VEC = 4;               // elements per 16-byte pack
  __device__ static __forceinline__ float ld(const float* p) { return *p; }
  __device__ static __forceinline__ void st(float* p, float v) { *p = v; }
  __device__ static __forceinline__ void unpack(const uint4& q, float* f) {
    f[0] = __uint_as_float(q.x); f[1] = __uint_as_float(q.y);
    f[2] = __uint_as_float(q.z); f[3] = __uint_as_float(q.w);
  }
  __device__ static __forceinline__ uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]),
                      __float_as_uint(f[2]), __float_as_uint(f[3]));
  }
};

template <> struct io<bf16_t> {
  static constexpr int VEC = 8;
  __device__ static __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  __device__ static __forceinline__ void st(bf16_t* p, float v) { *p = (bf16_t)f2bf(v); }
  __device__ static __forceinline__ void unpack(const uint4& q, float* f) {
    f[0] = __uint_as_float(q.x << 16); f[1] = __uint_as_float(q.x & 0xffff0000u);
    f[2] = __uint_as_float(q.y << 16); f[3] = __uint_as_float(q.y & 0xffff0000u);
    f[4] = __uint_as_float(q.z << 16); f[5] = __uint_as_float(q.z & 0xffff0000u);
    f[6] = __uint_as_float(q.w << 16); f[7] = __uint_as_float(q.w & 0xffff0000u);
  }
  __device__ static __forceinline__ uint4 pack(const float* f) {
    return make_uint4(f2bf2(f[0], f[1]), f2bf2(f[2], f[3]), f2bf2(f[4], f[5]), f2bf2(f[6], f[7]));
  }
};

// Load VEC elements starting at column c0 of a row (valid columns < n):
// a full in-bounds pack is one 16-byte load; a partial pack is read
// element by element with the missing lanes set to `fill`.
template <typename T, typename I = int64_t>
__device__ __forceinline__ void load_pack(const T* row, I c0, I n, float* f, float fill) {
  constexpr int V = io<T>::VEC;
  if (c0 + V <= n) {
    io<T>::unpack(ld_nt(row + c0), f);
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k) f[k] = (c0 + k < n) ? io<T>::ld(row + c0 + k) : fill;
  }
}

template <typename T, typename I = int64_t>
__device__ __forceinline__ void store_pack(T* row, I c0, I n, const float* f) {
  constexpr int V = io<T>::VEC;
  if (c0 + V <= n) {
    st_nt(row + c0, io<T>::pack(f));
  } else {
#pragma unroll
    for (int k = 0; k < V; ++k)
      if (c0 + k < n) io<T>::st(row + c0 + k, f[k]);
  }
}

// Raw 16-byte pack at column c0 (valid columns < n); a partial pack is read
// element by element with zero fill.  Callers mask columns >= n themselves
// where zero is not neutral.
template <typename T, typename I = int64_t>
__device__ __forceinline__ uint4 load_raw(const T* row, I c0, I n) {
  constexpr int V = io<T>::VEC;
  if (c0 + V <= n) return ld_nt(row + c0);
  T tmp[V];
#pragma unroll
  for (int k = 0; k < V; ++k) tmp[k] = (c0 + k < n) ? row[c0 + k] : (T)0;
  return *reinterpret_cast<const uint4*>(tmp);
}

// A row slice held as raw packs: pack j of group lane gl covers columns
// [(j*G + gl)*VEC, +VEC).
template <typename T, int NV, int G>
struct RowPacks;

// Column of element 0 of pack j held by lane gl of a G-lane row group.  The
// group's waves split the row into contiguous runs (wave w owns packs
// [w*NV*64, (w+1)*NV*64)), and within a wave pack j of lane l is pack
// j*64 + l of the run: one load instruction covers 64 consecutive packs
// (1 KB) and a lane's NV packs lie at compile-time offsets (1 KB apart)
// from one base address.
template <int NV, int VEC>
__device__ __forceinline__ int pack_col(int j, int gl) {
  return (((gl / WAVE) * NV + j) * WAVE + (gl % WAVE)) * VEC;
}

template <typename T, int NV, int G>
struct RowPacks {
  uint4 q[NV];
  // Whole packs only: the row width is a multiple of VEC on this path.
  __device__ __forceinline__ void load(const T* row, int gl, int C, bool active) {
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int c0 = pack_col<NV, io<T>::VEC>(j, gl);
      q[j] = (active && c0 < C) ? ld_nt(row + c0) : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void unpack(float (&f)[NV][io<T>::VEC]) const {
#pragma unroll
    for (int j = 0; j < NV; ++j) io<T>::unpack(q[j], f[j]);
  }
};

// Store with optional in-place accumulation (dst += v, one rounding).
template <typename T, typename I = int64_t>
__device__ __forceinline__ void store_pack_acc(T* row, I c0, I n, float* f, bool acc) {
  if (acc) {
    float o[io<T>::VEC];
    load_pack<T, I>(row, c0, n, o, 0.f);
#pragma unroll
    for (int k = 0; k < io<T>::VEC; ++k) f[k] = acc_add(o[k], f[k]);
  }
  store_pack<T, I>(row, c0, n, f);
}

// --------------------------------------------------------------- reductions
// Butterfly over the 64 lanes: every lane ends with the same bits (each level
// adds the same two operands in both lanes), so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}

// Sum over a group of RW consecutive waves of the block (one row per group).
// Every thread of the block must call it (it contains barriers when RW > 1).
// `lds` holds one float per wave of the block.
template <int RW>
__device__ __forceinline__ float group_sum(float v, float* lds) {
  v = wave_sum(v);
  if constexpr (RW == 1) {
    return v;
  } else {
    const int w = threadIdx.x / WAVE;
    const int g0 = (w / RW) * RW;
    __syncthreads();
    if ((threadIdx.x % WAVE) == 0) lds[w] = v;
    __syncthreads();
    float s = lds[g0];
#pragma unroll
    for (int i = 1; i < RW; ++i) s += lds[g0 + i];
    return s;
  }
}

template <int RW>
__device__ __forceinline__ float group_max(float v, float* lds) {
  v = wave_max(v);
  if constexpr (RW == 1) {
    return v;
  } else {
    const int w = threadIdx.x / WAVE;
    const int g0 = (w / RW) * RW;
    __syncthreads();
    if ((threadIdx.x % WAVE) == 0) lds[w] = v;
    __syncthreads();
    float s = lds[g0];
#pragma unroll
    for (int i = 1; i < RW; ++i) s = fmaxf(s, lds[g0 + i]);
    return s;
  }
}

// Two sums over the group with one pair of barriers.  `lds` holds two
// floats per wave of the block.
template <int RW>
__device__ __forceinline__ void group_sum2(float& a, float& b, float* lds) {
  a = wave_sum(a);
  b = wave_sum(b);
  if constexpr (RW > 1) {
    const int w = threadIdx.x / WAVE;
    const int g0 = (w / RW) * RW;
    __syncthreads();
    if ((threadIdx.x % WAVE) == 0) { lds[2 * w] = a; lds[2 * w + 1] = b; }
    __syncthreads();
    a = lds[2 * g0];
    b = lds[2 * g0 + 1];
#pragma unroll
    for (int i = 1; i < RW; ++i) { a += lds[2 * (g0 + i)]; b += lds[2 * (g0 + i) + 1]; }
  }
}

// Load n (multiple of 4, <= 8) f32 values starting at column c0 of a f32
// vector of length `len` (gamma/beta/bias); missing entries read as 0.
template <int N, typename I = int64_t>
__device__ __forceinline__ void load_f32s(const float* p, I c0, I len, float* f) {
  if (c0 + N <= len && (((uintptr_t)(p + c0)) & 15) == 0) {
#pragma unroll
    for (int k = 0; k < N; k += 4) {
      float4 q = *reinterpret_cast<const float4*>(p + c0 + k);
      f[k] = q.x; f[k + 1] = q.y; f[k + 2] = q.z; f[k + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int k = 0; k < N; ++k) f[k] = (c0 + k < len) ? p[c0 + k] : 0.f;
  }
}

}  // namespace xt
