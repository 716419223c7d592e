// Token embedding: y[r, :] = E[ids[r], :] and its backward
// dE[v, :] (+)= sum over r with ids[r] = v of d[r, :].
//
// [BP] kernel-pair table "Varje Forward-op Får En Backward-tvilling"
// (k_embed_fwd / k_embed_bwd, the token-embedding lookup) and the forward of
// "Framåtgåendet" (x = embed(token_ids); the tied output projection
// LN(x) @ embed^T is a MATMUL with trans_b on the same table, so its
// gradient reaches dE as a second, accumulated contribution).
//
// An id outside [0, V) gives a NaN output row and contributes nothing.
//
// The backward is deterministic without atomics on floats.  The (id, row)
// keys are sorted (bitonic sorts of 2048 keys in LDS, then merge rounds
// that place each key by its rank in the other run; keys are unique, so the
// order is fixed).  Runs of equal ids are cut into segments of SEG
// consecutive rows, one block per segment summing it in row order; a run of
// one segment is added to dE[v] at once, a longer run's segment sums are
// added in order by one block (so a frequent token does not serialise the
// pass) and the total is added to dE[v]: one rounding per dE row.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <utility>

#include "common.h"
#include "internal.h"

namespace xt {
namespace {

constexpr int SORT_T = 1024;                   // threads of a local-sort block
constexpr int L = 2048;                        // keys per local sort (16 KB of LDS)
constexpr int SUM_T = 256;
constexpr int SEG = 32;                        // rows per segment sum

template <typename T>
__device__ __forceinline__ float ldf(const T* p);
template <> __device__ __forceinline__ float ldf<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float ldf<bf16_t>(const bf16_t* p) { return bf2f(*p); }

template <typename T>
__device__ __forceinline__ void stf(T* p, float v);
template <> __device__ __forceinline__ void stf<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void stf<bf16_t>(bf16_t* p, float v) { *p = (bf16_t)f2bf(v); }

// y[r, :] = E[ids[r], :]; one block per row, 16-byte packs when rows allow.
template <typename T>
__global__ __launch_bounds__(SUM_T) void embed_fwd_k(const T* __restrict__ E, int64_t lde, int64_t V,
                                                     const int32_t* __restrict__ ids, int64_t ldi,
                                                     T* __restrict__ y, int64_t ldy, int64_t D, int vec) {
  const int64_t r = blockIdx.x;
  const int32_t v = ids[r * ldi];
  T* yr = y + r * ldy;
  if (v < 0 || v >= V) {
    for (int64_t c = threadIdx.x; c < D; c += SUM_T) stf<T>(yr + c, __builtin_nanf(""));
    return;
  }
  const T* er = E + (int64_t)v * lde;
  if (vec) {
    constexpr int P = 16 / sizeof(T);
    const int64_t np = D / P;
    for (int64_t i = threadIdx.x; i < np; i += SUM_T)
      reinterpret_cast<u32x4_t*>(yr)[i] = reinterpret_cast<const u32x4_t*>(er)[i];
    for (int64_t c = np * P + threadIdx.x; c < D; c += SUM_T) yr[c] = er[c];
  } else {
    for (int64_t c = threadIdx.x; c < D; c += SUM_T) yr[c] = er[c];
  }
}

// Key of row r: id << 32 | r, with an id outside [0, V) mapped to
// 0xffffffff (sorted last, skipped by the sums).  Keys are unique, so any
// correct sort gives the same order.
__device__ __forceinline__ uint64_t row_key(const int32_t* ids, int64_t ldi, int64_t r, int64_t V) {
  const int32_t v = ids[r * ldi];
  const uint32_t id = (v >= 0 && v < V) ? (uint32_t)v : 0xffffffffu;
  return ((uint64_t)id << 32) | (uint64_t)(uint32_t)r;
}

// Sorts the keys of rows [L b, L b + L), padded with ~0, by a bitonic
// network.  Thread t holds elements t and t + 1024 in registers; the
// partner of element e at stride j is e ^ j: a lane of the same wave for
// j < 64 (__shfl_xor), the thread's other element for j = 1024, and an LDS
// exchange (the only stages with barriers) for 64 <= j < 1024.
__device__ __forceinline__ uint64_t shfl_xor64(uint64_t v, int m) {
  const uint32_t lo = __shfl_xor((uint32_t)v, m), hi = __shfl_xor((uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// Element e's value after the compare-exchange with its partner at stride
// j inside bitonic sequences of length `size`: the smaller of the pair goes
// to the lower index in ascending sequences, the larger in descending ones.
__device__ __forceinline__ uint64_t bitonic_keep(uint64_t mine, uint64_t other, int e, int j, int size) {
  const bool up = (e & size) == 0, lo = (e & j) == 0;
  const uint64_t mn = mine < other ? mine : other, mx = mine < other ? other : mine;
  return lo == up ? mn : mx;
}

// Zero fill of the table gradient by blocks [nsort, gridDim.x) of the sort
// launch, so the 50257 x 768 f32 fill (154 MB, the largest step of the
// backward) streams while the few sort blocks run.  z: first byte of dE,
// nrows rows of rowb bytes, ldz bytes apart.
__device__ __forceinline__ void zero_rows(char* __restrict__ z, int64_t ldz, int64_t rowb, int64_t nrows, int f,
                                          int nf) {
  const int t = threadIdx.x;
  const bool al = ((uintptr_t)z % 16 == 0) && (ldz % 16 == 0) && (rowb % 16 == 0);
  if (al && ldz == rowb) {                            // one contiguous range of 16-byte packs
    const int64_t np = nrows * rowb / 16;
    const u32x4_t zero = {0u, 0u, 0u, 0u};
    u32x4_t* P = reinterpret_cast<u32x4_t*>(z);
    for (int64_t i = (int64_t)f * SORT_T + t; i < np; i += (int64_t)nf * SORT_T) __builtin_nontemporal_store(zero, P + i);
  } else {                                            // row by row, 2-byte stores (both element types)
    for (int64_t r = f; r < nrows; r += nf) {
      uint16_t* row = reinterpret_cast<uint16_t*>(z + r * ldz);
      for (int64_t c = t; c < rowb / 2; c += SORT_T) row[c] = 0;
    }
  }
}

__global__ __launch_bounds__(SORT_T) void embed_sort_k(const int32_t* __restrict__ ids, int64_t ldi, int64_t R,
                                                        int64_t V, uint64_t* __restrict__ keys, char* __restrict__ z,
                                                        int64_t ldz, int64_t rowb, int nsort) {
  static_assert(L == 2 * SORT_T, "two keys per thread");
  if ((int)blockIdx.x >= nsort) {
    zero_rows(z, ldz, rowb, V, (int)blockIdx.x - nsort, (int)gridDim.x - nsort);
    return;
  }
  __shared__ uint64_t k[L];
  const int64_t r0 = (int64_t)blockIdx.x * L;
  const int n = (int)(R - r0 < L ? R - r0 : L);
  const int t = threadIdx.x, e0 = t, e1 = t + SORT_T;
  uint64_t x0 = e0 < n ? row_key(ids, ldi, r0 + e0, V) : ~0ull;
  uint64_t x1 = e1 < n ? row_key(ids, ldi, r0 + e1, V) : ~0ull;
  for (int size = 2; size <= L; size <<= 1) {
    for (int j = size >> 1; j > 0; j >>= 1) {
      uint64_t p0, p1;
      if (j == SORT_T) {
        p0 = x1;
        p1 = x0;
      } else if (j < WAVE) {
        p0 = shfl_xor64(x0, j);
        p1 = shfl_xor64(x1, j);
      } else {
        __syncthreads();                     // earlier reads of k are done
        k[e0] = x0;
        k[e1] = x1;
        __syncthreads();
        p0 = k[e0 ^ j];
        p1 = k[e1 ^ j];
      }
      x0 = bitonic_keep(x0, p0, e0, j, size);
      x1 = bitonic_keep(x1, p1, e1, j, size);
    }
  }
  if (e0 < n) keys[r0 + e0] = x0;
  if (e1 < n) keys[r0 + e1] = x1;
}

// First index in [lo, hi) whose key is >= key.
__device__ __forceinline__ int64_t lower_key(const uint64_t* a, int64_t lo, int64_t hi, uint64_t key) {
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (a[mid] < key) lo = mid + 1;
    else hi = mid;
  }
  return lo;
}

// One merge round: sorted runs of width w pair up into runs of 2w.  Each
// key's place is its index in its own run plus its rank in the other run
// (keys are unique).
__global__ __launch_bounds__(SUM_T) void embed_merge_k(const uint64_t* __restrict__ src, uint64_t* __restrict__ dst,
                                                       int64_t n, int64_t w) {
  const int64_t i = (int64_t)blockIdx.x * SUM_T + threadIdx.x;
  if (i >= n) return;
  const uint64_t key = src[i];
  const int64_t base = i / (2 * w) * (2 * w), off = i - base;
  if (off < w) {
    const int64_t b0 = base + w < n ? base + w : n, b1 = base + 2 * w < n ? base + 2 * w : n;
    dst[base + off + (lower_key(src, b0, b1, key) - b0)] = key;
  } else {
    dst[base + (off - w) + (lower_key(src, base, base + w, key) - base)] = key;
  }
}

__device__ __forceinline__ uint32_t key_id(const uint64_t* keys, int64_t i) { return (uint32_t)(keys[i] >> 32); }

// run[i] = (first, end) positions of the run of equal ids holding sorted
// position i; (-1, -1) for out-of-range ids.  One thread per position.
__global__ __launch_bounds__(SUM_T) void embed_runs_k(const uint64_t* __restrict__ keys, int64_t n,
                                                      int2* __restrict__ run) {
  const int64_t i = (int64_t)blockIdx.x * SUM_T + threadIdx.x;
  if (i >= n) return;
  const uint32_t id = key_id(keys, i);
  if (id == 0xffffffffu) {
    run[i] = make_int2(-1, -1);
    return;
  }
  const uint64_t k0 = (uint64_t)id << 32, k1 = (uint64_t)(id + 1) << 32;
  run[i] = make_int2((int)lower_key(keys, 0, i + 1, k0), (int)lower_key(keys, i, n, k1));
}

// Partial-sum slot of a segment starting at sorted position i: two per
// SEG-window of positions (a window holds at most one segment start that
// opens a run and one that continues a run longer than SEG).
__device__ __forceinline__ int64_t part_slot(int i, bool run_start) { return 2 * (int64_t)(i / SEG) + (run_start ? 1 : 0); }

// Sum of d over the rows at sorted positions [p0, p1), in position (= row)
// order, columns c0 + tid + j*SUM_T; eight rows' loads in flight.
template <typename T, int CPT>
__device__ __forceinline__ void run_sum(const uint64_t* keys, int p0, int p1, const T* d, int64_t ldd, int64_t D,
                                        int64_t c0, float (&acc)[CPT]) {
#pragma unroll
  for (int j = 0; j < CPT; ++j) acc[j] = 0.f;
  int q = p0;
  for (; q + 8 <= p1; q += 8) {
    float v[8][CPT];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const T* dr = d + (int64_t)(uint32_t)keys[q + u] * ldd;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        const int64_t c = c0 + threadIdx.x + (int64_t)j * SUM_T;
        v[u][j] = c < D ? ldf<T>(dr + c) : 0.f;
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int j = 0; j < CPT; ++j) acc[j] += v[u][j];
  }
  for (; q < p1; ++q) {
    const T* dr = d + (int64_t)(uint32_t)keys[q] * ldd;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = c0 + threadIdx.x + (int64_t)j * SUM_T;
      if (c < D) acc[j] += ldf<T>(dr + c);
    }
  }
}

// One block per sorted position.  Runs of equal ids are cut
// into segments of SEG rows; the block at a segment start sums it (row
// order).  A run of at most SEG rows is added to dE[id] right away (one
// rounding); a longer run's segment sums go to `part` for the combine pass.
template <typename T>
__global__ __launch_bounds__(SUM_T) void embed_segsum_k(const uint64_t* __restrict__ keys, const int2* __restrict__ run,
                                                        const T* __restrict__ d, int64_t ldd,
                                                        T* __restrict__ dE, int64_t lde, int64_t D,
                                                        float* __restrict__ part) {
  constexpr int CPT = 4;
  const int i = blockIdx.x;
  const int2 rr = run[i];
  const int lo = rr.x, hi = rr.y;
  if (lo < 0 || (i - lo) % SEG != 0) return;
  const uint32_t id = key_id(keys, i);
  const int p1 = i + SEG < hi ? i + SEG : hi;
  const bool single = hi - lo <= SEG;
  T* out = dE + (int64_t)id * lde;
  float* ps = part + part_slot(i, i == lo) * D;
  for (int64_t c0 = 0; c0 < D; c0 += SUM_T * CPT) {
    float acc[CPT];
    run_sum<T, CPT>(keys, i, p1, d, ldd, D, c0, acc);
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = c0 + threadIdx.x + (int64_t)j * SUM_T;
      if (c >= D) continue;
      if (single) stf<T>(out + c, acc_add(ldf<T>(out + c), acc[j]));
      else ps[c] = acc[j];
    }
  }
}

// Runs longer than SEG: the block at the run start adds the segment sums
// in order and then adds the total to dE[id] (one rounding).
template <typename T>
__global__ __launch_bounds__(SUM_T) void embed_combine_k(const uint64_t* __restrict__ keys, const int2* __restrict__ run,
                                                         T* __restrict__ dE, int64_t lde, int64_t D,
                                                         const float* __restrict__ part) {
  const int i = blockIdx.x;
  const int2 rr = run[i];
  if (rr.x != i || rr.y - i <= SEG) return;
  const int hi = rr.y;
  const uint32_t id = key_id(keys, i);
  T* out = dE + (int64_t)id * lde;
  for (int64_t c = threadIdx.x; c < D; c += SUM_T) {
    // eight segment sums' loads in flight, added in segment order
    float acc = 0.f;
    int j = i;
    for (; j + 8 * SEG <= hi; j += 8 * SEG) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = part[part_slot(j + u * SEG, j + u * SEG == i) * D + c];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += v[u];
    }
    for (; j < hi; j += SEG) acc += part[part_slot(j, j == i) * D + c];
    stf<T>(out + c, acc_add(ldf<T>(out + c), acc));
  }
}

template <typename T>
hipError_t fwd_t(const xt_tensor& E, const int32_t* ids, int64_t ldi, const xt_tensor& y, hipStream_t s) {
  const int64_t R = y.rows, D = y.cols;
  if (R == 0 || D == 0) return hipSuccess;
  const int vec = (((uintptr_t)E.data | (uintptr_t)y.data) % 16 == 0) && (E.ld * (int64_t)sizeof(T)) % 16 == 0 &&
                  (y.ld * (int64_t)sizeof(T)) % 16 == 0;
  embed_fwd_k<T><<<(unsigned)R, SUM_T, 0, s>>>((const T*)E.data, E.ld, E.rows, ids, ldi, (T*)y.data, y.ld, D, vec);
  return hipGetLastError();
}

// Workspace layout: two key buffers (merge ping-pong), the run table, the
// segment sums.
struct EmbedWs {
  uint64_t* k0;
  uint64_t* k1;
  int2* run;
  float* part;
};

size_t al256(size_t b) { return (b + 255) / 256 * 256; }

EmbedWs carve(void* ws, int64_t R) {
  char* p = (char*)ws;
  EmbedWs w;
  w.k0 = (uint64_t*)p; p += al256((size_t)R * 8);
  w.k1 = (uint64_t*)p; p += al256((size_t)R * 8);
  w.run = (int2*)p; p += al256((size_t)R * 8);
  w.part = (float*)p;
  return w;
}

template <typename T>
hipError_t bwd_t(const xt_tensor& d, const int32_t* ids, int64_t ldi, const xt_tensor& dE, bool acc, void* ws,
                 hipStream_t s) {
  const int64_t R = d.rows, D = d.cols, V = dE.rows;
  if (R == 0 || D == 0) {               // no rows: dE is zero unless accumulating
    if (acc || D == 0) return hipSuccess;
    return launch_grads_scale(&dE, 1, true, 0.f, nullptr, s);
  }
  EmbedWs w = carve(ws, R);
  const int nsort = (int)((R + L - 1) / L);
  const int64_t rowb = D * (int64_t)sizeof(T), tb = V * rowb;
  // fill blocks: about 64 KB of zeros each, at most 2048
  const int nfill = acc || tb == 0 ? 0 : (int)std::min<int64_t>(2048, std::max<int64_t>(1, tb / 65536));
  embed_sort_k<<<(unsigned)(nsort + nfill), SORT_T, 0, s>>>(ids, ldi, R, V, w.k0, (char*)dE.data,
                                                            dE.ld * (int64_t)sizeof(T), rowb, nsort);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  uint64_t *src = w.k0, *dst = w.k1;
  const unsigned g = (unsigned)((R + SUM_T - 1) / SUM_T);
  for (int64_t width = L; width < R; width *= 2) {
    embed_merge_k<<<g, SUM_T, 0, s>>>(src, dst, R, width);
    std::swap(src, dst);
  }
  embed_runs_k<<<g, SUM_T, 0, s>>>(src, R, w.run);
  embed_segsum_k<T><<<(unsigned)R, SUM_T, 0, s>>>(src, w.run, (const T*)d.data, d.ld, (T*)dE.data, dE.ld, D, w.part);
  embed_combine_k<T><<<(unsigned)R, SUM_T, 0, s>>>(src, w.run, (T*)dE.data, dE.ld, D, w.part);
  return hipGetLastError();
}

}  // namespace

// Two key buffers, the run table (8 bytes per row each) and the segment
// sums: two D-float slots per SEG rows.
size_t embed_bwd_workspace(int64_t R, int64_t D) {
  if (R <= 0 || D <= 0) return 0;
  return 3 * al256((size_t)R * 8) + (size_t)(2 * ((R + SEG - 1) / SEG)) * (size_t)D * sizeof(float);
}

hipError_t launch_embed_fwd(const xt_tensor& E, const int32_t* ids, int64_t ldi, const xt_tensor& y, hipStream_t s) {
  return E.dtype == XT_BF16 ? fwd_t<bf16_t>(E, ids, ldi, y, s) : fwd_t<float>(E, ids, ldi, y, s);
}

hipError_t launch_embed_bwd(const xt_tensor& d, const int32_t* ids, int64_t ldi, const xt_tensor& dE, bool acc,
                            void* ws, hipStream_t s) {
  return d.dtype == XT_BF16 ? bwd_t<bf16_t>(d, ids, ldi, dE, acc, ws, s) : bwd_t<float>(d, ids, ldi, dE, acc, ws, s);
}

}  // namespace xt
