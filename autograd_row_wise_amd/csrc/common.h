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
// Wave reductions run on the VALU's cross-lane operand paths, not through
// LDS: DPP (data-parallel primitives) hands an instruction the operand of
// another lane of the same 16-lane row (quad_perm, row_half_mirror,
// row_mirror) or the last lane of a row to the next rows (row_bcast15,
// row_bcast31); one readlane then makes the wave's result uniform.
namespace dpp {
constexpr int XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int HALF_MIRROR = 0x141;  // lane i of each 8 <- lane 7 - i
constexpr int MIRROR = 0x140;       // lane i of each 16 <- lane 15 - i
constexpr int BCAST15 = 0x142;      // lane 15 of row r -> row r + 1
constexpr int BCAST31 = 0x143;      // lane 31 -> rows 2 and 3
}  // namespace dpp

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK, 0xf,
                                                               false));
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// op over each 16-lane row: after the four steps every lane of a row holds
// the row's result, with the same bits in every lane (each step combines
// the same two values in both lanes of a pair, and op is commutative).
template <class Op>
__device__ __forceinline__ float row16_reduce(float v, Op op) {
  v = op(v, dpp_f<dpp::XOR1>(v));
  v = op(v, dpp_f<dpp::XOR2>(v));
  v = op(v, dpp_f<dpp::HALF_MIRROR>(v));
  v = op(v, dpp_f<dpp::MIRROR>(v));
  return v;
}

// op over the 64 lanes, result uniform (one readlane): rows, then rows 1
// and 3 take rows 0 and 2, then rows 2 and 3 take lane 31; lane 63 ends
// with op((r2 op r3), (r0 op r1)).  A fixed order: deterministic.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
  v = row16_reduce(v, op);
  const int lane = __lane_id();
  const float a = op(v, dpp_f<dpp::BCAST15, 0xa>(v));
  v = (lane & 16) ? a : v;
  const float b = op(v, dpp_f<dpp::BCAST31, 0xc>(v));
  v = (lane & 32) ? b : v;
  return readlane_f(v, 63);
}

// op over each 32-lane half of the wave; every lane gets its half's result.
template <class Op>
__device__ __forceinline__ float half_reduce(float v, Op op) {
  v = row16_reduce(v, op);
  const float a = op(v, dpp_f<dpp::BCAST15, 0xa>(v));   // lanes 31 and 63: their half's result
  const float lo = readlane_f(a, 31), hi = readlane_f(a, 63);
  return __lane_id() < 32 ? lo : hi;
}

struct OpAdd {
  __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};
struct OpMax {
  __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};

__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, OpAdd{}); }
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, OpMax{}); }

// The value of lane l ^ 32 (v_permlane32_swap: the two halves of two
// registers trade places).  The compiler's builtin for this instruction
// loses its second result, so it is written out; the s_nop gives the swap
// the two wait states it needs after a VALU write of its operands.
__device__ __forceinline__ void swap_halves(float& lo_out, float& hi_out, float v) {
  uint32_t a = __float_as_uint(v), b = a;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo_out = __uint_as_float(a);     // every lane: v of lane (l mod 32)
  hi_out = __uint_as_float(b);     // every lane: v of lane (l mod 32) + 32
}

// op(v of lane l mod 32, v of lane l mod 32 + 32): the same two operands,
// in the same order, in lanes l and l ^ 32.
template <class Op>
__device__ __forceinline__ float xor32_reduce(float v, Op op) {
  float lo, hi;
  swap_halves(lo, hi, v);
  return op(lo, hi);
}

// Online (max, sum of exp) state, in base-2 units: value = s * 2^(m) with
// m = max * log2(e).
struct MS { float m, s; };

__device__ __forceinline__ MS ms_merge(MS a, MS b) {
  const float m = fmaxf(a.m, b.m);
  if (m == -__builtin_inff()) return {m, 0.f};
  return {m, a.s * __builtin_amdgcn_exp2f(a.m - m) + b.s * __builtin_amdgcn_exp2f(b.m - m)};
}

template <int CTRL, int ROW_MASK = 0xf>
__device__ __forceinline__ MS dpp_ms(MS a) {
  return {dpp_f<CTRL, ROW_MASK>(a.m), dpp_f<CTRL, ROW_MASK>(a.s)};
}

// ms_merge over the 64 lanes in the order of wave_reduce (above): the 16
// lanes of a row by DPP steps, then rows 1, 3 take rows 0, 2 and rows 2, 3
// take lane 31; the wave's state is read from lane 63.  ms_merge combines
// its two arguments symmetrically, so both lanes of a pair hold the same
// bits after each step.
__device__ __forceinline__ MS wave_merge(MS st) {
  st = ms_merge(st, dpp_ms<dpp::XOR1>(st));
  st = ms_merge(st, dpp_ms<dpp::XOR2>(st));
  st = ms_merge(st, dpp_ms<dpp::HALF_MIRROR>(st));
  st = ms_merge(st, dpp_ms<dpp::MIRROR>(st));
  const int lane = __lane_id();
  const MS a = ms_merge(st, dpp_ms<dpp::BCAST15, 0xa>(st));
  if (lane & 16) st = a;
  const MS b = ms_merge(st, dpp_ms<dpp::BCAST31, 0xc>(st));
  if (lane & 32) st = b;
  return {readlane_f(st.m, 63), readlane_f(st.s, 63)};
}

// Reductions over a group of RW consecutive waves of the block (one row per
// group).  Every thread of the block must make the same sequence of calls
// (they contain barriers when RW > 1).  `lds` holds 4 floats per wave of
// the block: two slot sets of up to two values per wave.  Successive calls
// alternate between the sets (`ph`, a per-thread counter starting at 0), so
// a set is written again only after the next call's barrier, by which time
// every wave has read it: one barrier per reduction.  The waves' results are
// combined in wave order, so the result is deterministic.
// Block barrier for LDS traffic: this wave's LDS accesses complete, then
// s_barrier.  Unlike __syncthreads() it does not wait for the wave's global
// memory operations in flight (loads, stores, transfers into LDS issued by
// global_load_lds), so a reduction does not stall on a prefetch or on the
// previous row's stores.  The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt and expcnt not waited for
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Waits until at most n of the wave's vector memory operations are
// outstanding (n clamped to 15).  vmcnt retires them in issue order, so
// every operation issued before the last n has completed.  n may differ
// between lanes: the wave then waits for the smallest, which is stronger.
__device__ __forceinline__ void wait_vmcnt_at_most(int n) {
  asm volatile("" ::: "memory");
  // s_waitcnt immediate: vmcnt in bits 3:0, expcnt 6:4 and lgkmcnt 11:8 at
  // their maxima (not waited for)
#define XT_VMW(N) case N: __builtin_amdgcn_s_waitcnt(0x0F70 | N); break;
  switch (n < 15 ? (n < 0 ? 0 : n) : 15) {
    XT_VMW(0) XT_VMW(1) XT_VMW(2) XT_VMW(3) XT_VMW(4) XT_VMW(5) XT_VMW(6) XT_VMW(7)
    XT_VMW(8) XT_VMW(9) XT_VMW(10) XT_VMW(11) XT_VMW(12) XT_VMW(13) XT_VMW(14)
    default: __builtin_amdgcn_s_waitcnt(0x0F70 | 15); break;
  }
#undef XT_VMW
  asm volatile("" ::: "memory");
}

template <int RW>
__device__ __forceinline__ float* group_slot(float* lds, int& ph) {
  float* slot = lds + ph * 2 * (int)(blockDim.x / WAVE);
  ph ^= 1;
  return slot;
}

template <int RW>
__device__ __forceinline__ float group_sum(float v, float* lds, int& ph) {
  v = wave_sum(v);
  if constexpr (RW == 1) {
    return v;
  } else {
    const int w = threadIdx.x / WAVE;
    const int g0 = (w / RW) * RW;
    float* slot = group_slot<RW>(lds, ph);
    if ((threadIdx.x % WAVE) == 0) slot[w] = v;
    lds_barrier();
    float s = slot[g0];
#pragma unroll
    for (int i = 1; i < RW; ++i) s += slot[g0 + i];
    return s;
  }
}

template <int RW>
__device__ __forceinline__ float group_max(float v, float* lds, int& ph) {
  v = wave_max(v);
  if constexpr (RW == 1) {
    return v;
  } else {
    const int w = threadIdx.x / WAVE;
    const int g0 = (w / RW) * RW;
    float* slot = group_slot<RW>(lds, ph);
    if ((threadIdx.x % WAVE) == 0) slot[w] = v;
    lds_barrier();
    float s = slot[g0];
#pragma unroll
    for (int i = 1; i < RW; ++i) s = fmaxf(s, slot[g0 + i]);
    return s;
  }
}

// Two sums over the group with one barrier.
template <int RW>
__device__ __forceinline__ void group_sum2(float& a, float& b, float* lds, int& ph) {
  a = wave_sum(a);
  b = wave_sum(b);
  if constexpr (RW > 1) {
    const int w = threadIdx.x / WAVE;
    const int g0 = (w / RW) * RW;
    float* slot = group_slot<RW>(lds, ph);
    if ((threadIdx.x % WAVE) == 0) { slot[2 * w] = a; slot[2 * w + 1] = b; }
    lds_barrier();
    a = slot[2 * g0];
    b = slot[2 * g0 + 1];
#pragma unroll
    for (int i = 1; i < RW; ++i) { a += slot[2 * (g0 + i)]; b += slot[2 * (g0 + i) + 1]; }
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
