// Matmul forward and backward on the matrix cores (MFMA) of gfx950.
//
// [AE] op-backward table row "matmul": C = A@B, dA = d@B^T, dB = A^T@d.
// All three are one kernel, C (+)= alpha * op(A) op(B), with op() the
// identity or the transpose of the stored operand; batches (attention
// heads) run along gridDim.z with two-level element strides.
//
// Tiling: a 256-thread block (4 waves, 2 x 2) computes a 128 x 128 tile of C;
// each wave owns 64 x 64 = 2 x 2 MFMA 32x32 accumulators.  K advances in
// tiles of BK staged in LDS as [row][k] for both operands (k contiguous), so
// every MFMA operand is one or two 16-byte LDS reads per lane.  The next K
// tile is fetched into registers while the current one is multiplied (LDS
// double buffer, one barrier per K tile).
//   bf16: v_mfma_f32_32x32x16_bf16, BK = 32 (two MFMA steps of 16).
//   f32 : v_mfma_f32_32x32x2_f32, BK = 16; lane l supplies k = 8*(l/32)+j to
//         the j-th of eight MFMAs (a permutation of the summation order).
// Accumulation is f32; the epilogue scales by alpha, optionally adds the
// existing C, and rounds once to C's dtype.
#include <algorithm>
#include <cstdint>

#include "common.h"
#include "internal.h"

namespace xt {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int BM = 128, BN = 128, NT = 256;

template <typename TA> struct gcfg;
template <> struct gcfg<bf16_t> { static constexpr int BK = 32, PAD = 8; };
template <> struct gcfg<float> { static constexpr int BK = 16, PAD = 4; };

// Registers holding one thread's share of a BM x BK (or BN x BK) tile.
// Non-transposed storage ([rows][K], k contiguous): each thread moves
// 16-byte chunks along k.  Transposed storage ([K][rows]): chunks along rows,
// scattered into the [row][k] LDS layout.
template <typename TA, bool KCONTIG, int ROWS = BM>
struct TileLoader {
  static constexpr int BK = gcfg<TA>::BK;
  static constexpr int V = 16 / sizeof(TA);                    // elements per chunk
  static constexpr int CHUNKS = ROWS * BK / V;                 // chunks per tile
  static constexpr int PER_T = CHUNKS / NT;                    // chunks per thread
  uint4 r[PER_T];

  // g: operand base (batch applied); rows_total: M or N; K; ld: storage ld
  __device__ __forceinline__ void load(const TA* g, int64_t ld, int64_t row0, int64_t rows_total,
                                       int64_t k0, int64_t K, bool full) {
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = i * NT + threadIdx.x;
      int row, kk;
      if (KCONTIG) { row = c / (BK / V); kk = (c % (BK / V)) * V; }
      else { kk = c / (ROWS / V); row = (c % (ROWS / V)) * V; }
      const int64_t gr = row0 + row, gk = k0 + kk;
      if (full) {
        const TA* p = KCONTIG ? g + gr * ld + gk : g + gk * ld + gr;
        r[i] = *reinterpret_cast<const uint4*>(p);
      } else {
        TA tmp[V];
#pragma unroll
        for (int j = 0; j < V; ++j) {
          const int64_t rr = KCONTIG ? gr : gr + j, kq = KCONTIG ? gk + j : gk;
          tmp[j] = (rr < rows_total && kq < K) ? g[KCONTIG ? rr * ld + kq : kq * ld + rr] : (TA)0;
        }
        r[i] = *reinterpret_cast<const uint4*>(tmp);
      }
    }
  }

  __device__ __forceinline__ void store(TA* lds) const {
    constexpr int LDK = BK + gcfg<TA>::PAD;
#pragma unroll
    for (int i = 0; i < PER_T; ++i) {
      const int c = i * NT + threadIdx.x;
      if (KCONTIG) {
        const int row = c / (BK / V), kk = (c % (BK / V)) * V;
        *reinterpret_cast<uint4*>(lds + row * LDK + kk) = r[i];
      } else {
        const int kk = c / (ROWS / V), row = (c % (ROWS / V)) * V;
        const TA* v = reinterpret_cast<const TA*>(&r[i]);
#pragma unroll
        for (int j = 0; j < V; ++j) lds[(row + j) * LDK + kk] = v[j];
      }
    }
  }
};

template <typename TA, int TT = 2>
__device__ __forceinline__ void mfma_tile(const TA* As, const TA* Bs, int wm, int wn,
                                          f32x16_t (&acc)[TT][TT]) {
  constexpr int BK = gcfg<TA>::BK, LDK = BK + gcfg<TA>::PAD;
  const int l = threadIdx.x % WAVE;
  const int lr = l % 32, lk = (l / 32) * 8;
  if constexpr (sizeof(TA) == 2) {
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8_t a[TT], b[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        a[t] = *reinterpret_cast<const bf16x8_t*>(As + (wm + t * 32 + lr) * LDK + ks + lk);
        b[t] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn + t * 32 + lr) * LDK + ks + lk);
      }
#pragma unroll
      for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < TT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  } else {
    float a[TT][8], b[TT][8];
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float4* pa = reinterpret_cast<const float4*>(As + (wm + t * 32 + lr) * LDK + lk);
      const float4* pb = reinterpret_cast<const float4*>(Bs + (wn + t * 32 + lr) * LDK + lk);
      const float4 a0 = pa[0], a1 = pa[1], b0 = pb[0], b1 = pb[1];
      a[t][0] = a0.x; a[t][1] = a0.y; a[t][2] = a0.z; a[t][3] = a0.w;
      a[t][4] = a1.x; a[t][5] = a1.y; a[t][6] = a1.z; a[t][7] = a1.w;
      b[t][0] = b0.x; b[t][1] = b0.y; b[t][2] = b0.z; b[t][3] = b0.w;
      b[t][4] = b1.x; b[t][5] = b1.y; b[t][6] = b1.z; b[t][7] = b1.w;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
#pragma unroll
      for (int i = 0; i < TT; ++i)
#pragma unroll
        for (int j = 0; j < TT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][k], b[j][k], acc[i][j], 0, 0, 0);
  }
}

// TB x TB tiles of C (TB = 128, or 64 for products with few 128-tiles: four
// times the blocks, each wave one 32 x 32 accumulator).
template <typename TA, typename TC, bool TRANS_A, bool TRANS_B, int TB = BM>
__global__ __launch_bounds__(NT) void gemm_k(
    const TA* __restrict__ A, int64_t lda, int64_t sa0, int64_t sa1,
    const TA* __restrict__ B, int64_t ldb, int64_t sb0, int64_t sb1,
    TC* __restrict__ C, int64_t ldc, int64_t sc0, int64_t sc1,
    int64_t M, int64_t N, int64_t K, int64_t nb1, float alpha, int acc_c,
    int64_t kchunk, int64_t nbatch, int64_t scs) {
  constexpr int BK = gcfg<TA>::BK, LDK = BK + gcfg<TA>::PAD, TT = TB / 64;
  __shared__ __align__(16) TA As[2][TB * LDK];
  __shared__ __align__(16) TA Bs[2][TB * LDK];

  // gridDim.z = splits x batches; split s sums k in [s*kchunk, (s+1)*kchunk)
  const int64_t z = blockIdx.z, split = z / nbatch, bz = z % nbatch, b0 = bz / nb1, b1 = bz % nb1;
  const int64_t kb = split * kchunk;
  A += b0 * sa0 + b1 * sa1 + (TRANS_A ? kb * lda : kb);
  B += b0 * sb0 + b1 * sb1 + (TRANS_B ? kb : kb * ldb);
  C += b0 * sc0 + b1 * sc1 + split * scs;
  K = K - kb < kchunk ? K - kb : kchunk;
  const int64_t m0 = (int64_t)blockIdx.y * TB, n0 = (int64_t)blockIdx.x * TB;
  const int w = threadIdx.x / WAVE;
  const int wm = (w / 2) * (TB / 2), wn = (w % 2) * (TB / 2);

  // A as [M][K] is k-contiguous unless transposed; B as [K][N] is k-contiguous
  // only when transposed ([N][K] storage).
  TileLoader<TA, !TRANS_A, TB> la;
  TileLoader<TA, TRANS_B, TB> lb;
  const bool fullMN = (m0 + TB <= M) && (n0 + TB <= N);
  const bool alA = (((uintptr_t)A) & 15) == 0 && ((lda * (int64_t)sizeof(TA)) & 15) == 0;
  const bool alB = (((uintptr_t)B) & 15) == 0 && ((ldb * (int64_t)sizeof(TA)) & 15) == 0;

  f32x16_t acc[TT][TT];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int64_t nk = (K + BK - 1) / BK;
  if (nk > 0) {
    bool full = fullMN && BK <= K && alA && alB;
    la.load(A, lda, m0, M, 0, K, full);
    lb.load(B, ldb, n0, N, 0, K, full);
    la.store(As[0]);
    lb.store(Bs[0]);
    __syncthreads();
    for (int64_t kt = 0; kt < nk; ++kt) {
      const int cur = kt & 1;
      const bool more = kt + 1 < nk;
      if (more) {
        const int64_t k0 = (kt + 1) * BK;
        full = fullMN && (k0 + BK <= K) && alA && alB;
        la.load(A, lda, m0, M, k0, K, full);
        lb.load(B, ldb, n0, N, k0, K, full);
      }
      mfma_tile<TA, TT>(As[cur], Bs[cur], wm, wn, acc);
      if (more) {
        la.store(As[cur ^ 1]);
        lb.store(Bs[cur ^ 1]);
      }
      __syncthreads();
    }
  }

  // epilogue: 32x32 accumulator layout -- lane l, register q holds
  // row 8*(q/4) + 4*(l/32) + q%4, column l%32 of the tile
  const int l = threadIdx.x % WAVE;
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < TT; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm + i * 32 + 8 * (q / 4) + 4 * (l / 32) + (q % 4);
        const int64_t col = n0 + wn + j * 32 + (l % 32);
        if (row < M && col < N) {
          TC* p = C + row * ldc + col;
          float v = alpha * acc[i][j][q];
          if (acc_c) v = acc_add(io<TC>::ld(p), v);
          io<TC>::st(p, v);
        }
      }
}

// ==========================================================================
// Large-tile kernel for aligned f32 problems (every tile full, K a multiple
// of BK, 16-byte aligned operands): 128 x 128 block tile, BK = 32, 4 waves
// of 64 x 64, 2 x 2 accumulators of v_mfma_f32_32x32x2_f32.
//
// Both operands sit in LDS as [row][k] (k contiguous) rows of 128 bytes =
// eight 16-byte chunks, XOR-swizzled (swz below) so that the lanes of an
// MFMA fragment read (32 consecutive rows, one chunk) spread over all banks
// without padding.  Operands stored transposed in HBM ([K][rows]) are read
// as 4 x 4 blocks with 16-byte loads and transposed in registers before the
// 16-byte LDS stores.  The next K tile is fetched into registers while the
// current one is multiplied.  Tiles are ordered so that each of the 8 XCDs
// (blocks are dealt to XCDs round-robin) owns whole rows of tiles and reuses
// their A panels in its own L2.
//
// big<bf16_t> holds the alignment rule of the bf16 large-tile kernel further
// below (256 x 256 tiles; K, and every split-K slice, a multiple of 64).
// ==========================================================================
template <typename TA> struct big;
template <> struct big<bf16_t> { static constexpr int BM = 256, BN = 256, BK = 64, TM = 4, TN = 4; };
template <> struct big<float> { static constexpr int BM = 128, BN = 128, BK = 32, TM = 2, TN = 2; };

// 16-byte chunk c of LDS row r (rows of 128 bytes) is stored at chunk
// c ^ ((r >> 1) & 7): gfx950's LDS serves a 128-bit access sixteen lanes
// (256 bytes, all 64 banks) at a time, and the sixteen rows an MFMA
// fragment read touches at once then land in sixteen different 16-byte bank
// groups (two rows share a 256-byte bank row; the XOR term differs between
// rows of equal parity).
__device__ __forceinline__ int swz(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }

// One thread's share of a BM x BK operand tile, staged in registers.
template <typename TA, int ROWS, bool KCONTIG>
struct BigLoader {
  static constexpr int BK = big<TA>::BK;
  static constexpr int V = 16 / sizeof(TA);                 // elements per chunk
  static constexpr int PER_T = ROWS * 8 / NT;               // 16-byte chunks per thread
  uint4 r[PER_T];

  __device__ __forceinline__ void load(const TA* g, int64_t ld, int64_t row0, int64_t k0) {
    if constexpr (KCONTIG) {
      // chunk i of thread t: row t/8 + i*(NT/8), k chunk t%8 (coalesced rows)
#pragma unroll
      for (int i = 0; i < PER_T; ++i) {
        const int row = threadIdx.x / 8 + i * (NT / 8), c = threadIdx.x % 8;
        r[i] = ld_nt_ro(g + (row0 + row) * ld + k0 + c * V);
      }
    } else {
      // one V x V block: k rows kb*V.., rows mb*V..  (PER_T == V); kb
      // varies fastest so that LDS store phases hit distinct chunk columns
      constexpr int KB = BK / V;
      const int kb = threadIdx.x % KB, mb = threadIdx.x / KB;
#pragma unroll
      for (int i = 0; i < V; ++i) r[i] = ld_nt_ro(g + (k0 + kb * V + i) * ld + row0 + mb * V);
    }
  }

  __device__ __forceinline__ void store(TA* lds) const {
    uint4* L = reinterpret_cast<uint4*>(lds);
    if constexpr (KCONTIG) {
#pragma unroll
      for (int i = 0; i < PER_T; ++i) {
        const int row = threadIdx.x / 8 + i * (NT / 8), c = threadIdx.x % 8;
        L[swz(row, c)] = r[i];
      }
    } else {
      constexpr int KB = BK / V;
      const int kb = threadIdx.x % KB, mb = threadIdx.x / KB;
      static_assert(V == 4, "register transpose is written for 4 x 4 f32 blocks");
      uint4 t[V];
      // 4 x 4 f32: r[k] = (m0..m3) of k row; t[m] = (k0..k3)
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
      for (int m = 0; m < 4; ++m) t[m] = make_uint4(w0[m], w1[m], w2[m], w3[m]);
#pragma unroll
      for (int j = 0; j < V; ++j) L[swz(mb * V + j, kb)] = t[j];
    }
  }

  // plain (cached) 16-byte load: operand panels are re-read by other blocks
  __device__ static __forceinline__ uint4 ld_nt_ro(const TA* p) { return *reinterpret_cast<const uint4*>(p); }
};

template <typename TA, typename TC, bool TRANS_A, bool TRANS_B>
__global__ __launch_bounds__(NT) void gemm_big_k(
    const TA* __restrict__ A, int64_t lda, int64_t sa0, int64_t sa1,
    const TA* __restrict__ B, int64_t ldb, int64_t sb0, int64_t sb1,
    TC* __restrict__ C, int64_t ldc, int64_t sc0, int64_t sc1,
    int64_t M, int64_t N, int64_t K, int64_t nb1, float alpha, int acc_c,
    int64_t kchunk, int64_t nbatch, int64_t scs) {
  constexpr int BM_ = big<TA>::BM, BN_ = big<TA>::BN, BK_ = big<TA>::BK, TM = big<TA>::TM, TN = big<TA>::TN;
  __shared__ __align__(16) TA As[BM_ * BK_];
  __shared__ __align__(16) TA Bs[BN_ * BK_];

  // gridDim.z = splits x batches; split s sums k in [s*kchunk, (s+1)*kchunk)
  const int64_t z = blockIdx.z, split = z / nbatch, bz = z % nbatch, b0 = bz / nb1, b1 = bz % nb1;
  const int64_t kb = split * kchunk;
  A += b0 * sa0 + b1 * sa1 + (TRANS_A ? kb * lda : kb);
  B += b0 * sb0 + b1 * sb1 + (TRANS_B ? kb : kb * ldb);
  C += b0 * sc0 + b1 * sc1 + split * scs;
  K = K - kb < kchunk ? K - kb : kchunk;
  // XCD-aware tile order: block g runs on XCD g % 8; give each XCD a
  // contiguous run of tiles (whole tile rows when they divide evenly)
  const int tiles_n = (int)(N / BN_);
  const int tiles = (int)(M / BM_) * tiles_n;
  const int g = blockIdx.x;
  const int t = (tiles % 8 == 0) ? (g % 8) * (tiles / 8) + g / 8 : g;
  const int64_t m0 = (int64_t)(t / tiles_n) * BM_, n0 = (int64_t)(t % tiles_n) * BN_;

  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  const int wm = (w / 2) * (BM_ / 2), wn = (w % 2) * (BN_ / 2);
  BigLoader<TA, BM_, !TRANS_A> la;
  BigLoader<TA, BN_, TRANS_B> lb;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int nk = (int)(K / BK_);
  la.load(A, lda, m0, 0);
  lb.load(B, ldb, n0, 0);
  const uint4* LA = reinterpret_cast<const uint4*>(As);
  const uint4* LB = reinterpret_cast<const uint4*>(Bs);
  for (int kt = 0; kt < nk; ++kt) {
    la.store(As);
    lb.store(Bs);
    __syncthreads();
    if (kt + 1 < nk) {                      // next tile in flight during the MFMAs
      la.load(A, lda, m0, (int64_t)(kt + 1) * BK_);
      lb.load(B, ldb, n0, (int64_t)(kt + 1) * BK_);
    }
    const int lr = l % 32, lh = l / 32;
    if constexpr (sizeof(TA) == 2) {
#pragma unroll
      for (int s = 0; s < BK_ / 16; ++s) {
        bf16x8_t a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm + i * 32 + lr;
          a[i] = __builtin_bit_cast(bf16x8_t, LA[swz(row, 2 * s + lh)]);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row = wn + j * 32 + lr;
          b[j] = __builtin_bit_cast(bf16x8_t, LB[swz(row, 2 * s + lh)]);
        }
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int s = 0; s < BK_ / 16; ++s) {
        // lane l supplies k = 16*s + 8*(l/32) + j to the j-th MFMA
        float a[TM][8], b[TN][8];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const int row = wm + i * 32 + lr;
          const uint4 q0 = LA[swz(row, 4 * s + 2 * lh)], q1 = LA[swz(row, 4 * s + 2 * lh + 1)];
          a[i][0] = __uint_as_float(q0.x); a[i][1] = __uint_as_float(q0.y);
          a[i][2] = __uint_as_float(q0.z); a[i][3] = __uint_as_float(q0.w);
          a[i][4] = __uint_as_float(q1.x); a[i][5] = __uint_as_float(q1.y);
          a[i][6] = __uint_as_float(q1.z); a[i][7] = __uint_as_float(q1.w);
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int row = wn + j * 32 + lr;
          const uint4 q0 = LB[swz(row, 4 * s + 2 * lh)], q1 = LB[swz(row, 4 * s + 2 * lh + 1)];
          b[j][0] = __uint_as_float(q0.x); b[j][1] = __uint_as_float(q0.y);
          b[j][2] = __uint_as_float(q0.z); b[j][3] = __uint_as_float(q0.w);
          b[j][4] = __uint_as_float(q1.x); b[j][5] = __uint_as_float(q1.y);
          b[j][6] = __uint_as_float(q1.z); b[j][7] = __uint_as_float(q1.w);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k)
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < TN; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][k], b[j][k], acc[i][j], 0, 0, 0);
      }
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm + i * 32 + 8 * (q / 4) + 4 * (l / 32) + (q % 4);
        const int64_t col = n0 + wn + j * 32 + (l % 32);
        TC* p = C + row * ldc + col;
        float v = alpha * acc[i][j][q];
        if (acc_c) v = acc_add(io<TC>::ld(p), v);
        io<TC>::st(p, v);
      }
}

// ==========================================================================
// bf16 large-tile kernel.  A 512-thread block (8 waves, 2 per SIMD) computes
// a 256 x 256 tile of C; the waves form 2 (m) x 4 (n), each owning 128 x 64
// of C = 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16, so one wave's LDS
// reads and waits overlap the other's MFMAs on the same SIMD.
//
// Operands reach LDS without staging registers: each lane issues
// global_load_lds_dwordx4, which writes its 16 bytes straight into LDS at
// the wave's destination + 16 * lane.  An operand stored k-contiguous lands
// as [row][k]; one stored transposed lands as [k][row] and is turned into
// MFMA fragments by the transposing LDS read (ds_read_b64_tr_b16), so all
// four layouts (d B^T, A^T d, ...) share the kernel and no transpose copy
// exists.  K tiles are 64 deep in two 64 KB stages (schedule below).
//
// Measured alternatives that ran slower on this product (8192 x 4096 x
// 4096): 32-deep tiles in four stages (each k-contiguous 128-byte line then
// reaches L2 as two 64-byte requests); two 4-wave groups alternating load
// and MFMA phases with a barrier per phase; 4 waves of 128 x 128 (one wave
// per SIMD, with 32- or 64-deep tiles), whose LDS reads per MFMA are fewer
// but whose stalls no second wave covers.
//
// Tile order: blocks are dealt to the 8 XCDs round-robin; XCD x takes the
// contiguous tile range x * tiles / 8 .., walked in groups of four tile rows
// (tile_of), so the 32 tiles an XCD runs at once form a 4 x 8 patch whose A
// and B panels its L2 shares.
// ==========================================================================
namespace b8 {
constexpr int BM = 256, BN = 256, NT = 512;
}  // namespace b8

// Tile tt (in an XCD's range) -> (m0, n0): groups of GM tile rows, column by
// column within a group.
__device__ __forceinline__ void tile_of(int tt, int tiles_m, int tiles_n, int64_t& m0, int64_t& n0, int bm, int bn) {
  const int GM = 4, span = GM * tiles_n, first = (tt / span) * GM;
  const int gm = tiles_m - first < GM ? tiles_m - first : GM, r = tt % span;
  m0 = (int64_t)(first + r % gm) * bm; n0 = (int64_t)(r / gm) * bn;
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// MFMA operand of fragment rows f0 .. f0+31, k 16 s .. 16 s + 15 (lane l:
// row f0 + l % 32, k 16 s + 8 (l / 32) .. +7) from a [k][row] tile: two
// transposing reads (ds_read_b64_tr_b16: within each group of 16 lanes, lane
// j receives element j % 4 of the 8-byte rows that lanes 4 v + j / 4
// address, v = 0..3).
__device__ __forceinline__ bf16x8_t tr_frag(const bf16_t* __restrict__ tile, int f0, int s, int l) {
  const int g = l / 16, q = l % 16;                  // source role of this lane within its group
  const int row = f0 + 16 * (g & 1) + 4 * (q & 3);   // 4 consecutive rows from here
  const int c = row / 8, half = (row / 4) & 1;
  s16x4_t v[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int kr = 16 * s + 8 * (g >> 1) + 4 * h + q / 4;
    const bf16_t* p = tile + kr * 256 + ((c ^ (4 * (kr & 3))) * 8) + half * 4;
    v[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)p);
  }
  const short __attribute__((ext_vector_type(8))) w8 = {v[0][0], v[0][1], v[0][2], v[0][3],
                                                        v[1][0], v[1][1], v[1][2], v[1][3]};
  return __builtin_bit_cast(bf16x8_t, w8);
}

struct b8d_frags { bf16x8_t a[4], b[2]; };

__device__ __forceinline__ void b8d_mfma(const b8d_frags& f, f32x16_t (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Issue order for one substep: its 8 MFMAs with the NR LDS reads of the
// next substep's fragments spread between them.
template <int NR>
__device__ __forceinline__ void b8d_sched_half() {
  if constexpr (NR == 6) {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  } else if constexpr (NR == 8) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  } else if constexpr (NR == 10) {
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
  }
}

// K tiles are 64 deep in two 64 KB stages.  A k-contiguous operand row is
// then 128 bytes per tile: each transfer reads whole cache lines (with
// 32-deep tiles every line is fetched as two 64-byte halves, one tile apart,
// which doubles the requests to L2), and there is one barrier per 64 k.
//
// Step kt multiplies the four 16-deep substeps of tile kt (stage kt % 2),
// each while the next substep's fragments are read.  After the third
// substep's MFMAs are issued, a wave waits until its transfers of tile kt+1
// have landed and its reads of stage kt % 2 are complete, then the block
// barrier; after it, every wave requests its share of tile kt+2 into stage
// kt % 2 and reads substep 0 of tile kt+1 during substep 3's MFMAs.  A
// transfer thus has one whole step (the 32 MFMAs of each wave) to land.
namespace k64 {
constexpr int BK = 64, TILE = 256 * BK;              // elements of one operand tile
}  // namespace k64

// k-contiguous tiles: [row][64 k] (128-byte rows, 16-byte chunk c of row r
// at c ^ ((r >> 1) & 7): the 16 rows one ds_read_b128 phase touches fall in
// 16 different bank groups).  Others: [k][row] (512-byte k-rows, chunk c of
// k-row kr at c ^ 4 (kr & 3), read by tr_frag).  32 transfers of 1 KB per
// tile, NB per wave: transfer b covers rows 8 b .. 8 b + 7 (or k-rows 2 b,
// 2 b + 1).
template <bool KCONTIG, int NB = 4>
__device__ __forceinline__ void k64_dma_tile(const bf16_t* g, int64_t ld, int64_t row0, int64_t k0,
                                             bf16_t* __restrict__ lds_tile, int w, int l) {
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int blk = w * NB + j;
    const bf16_t* src;
    if constexpr (KCONTIG) {
      const int row = blk * 8 + l / 8;
      const int c = (l % 8) ^ ((row >> 1) & 7);
      src = g + (row0 + row) * ld + k0 + c * 8;
    } else {
      const int kr = blk * 2 + l / 32;
      const int c = (l % 32) ^ (4 * (kr & 3));
      src = g + (k0 + kr) * ld + row0 + c * 8;
    }
    __builtin_amdgcn_global_load_lds(src, lds_tile + blk * 64 * 8, 16, 0, 0);
  }
}

template <bool KCONTIG>
__device__ __forceinline__ bf16x8_t k64_frag(const bf16_t* __restrict__ tile, int f0, int s, int l) {
  if constexpr (KCONTIG) {
    const u32x4_t* L = reinterpret_cast<const u32x4_t*>(tile);
    const int row = f0 + l % 32, c = 2 * s + l / 32;
    return __builtin_bit_cast(bf16x8_t, L[row * 8 + (c ^ ((row >> 1) & 7))]);
  } else {
    return tr_frag(tile, f0, s, l);
  }
}

template <bool KA, bool KB>
__device__ __forceinline__ void k64_read(const bf16_t* __restrict__ st, int s, b8d_frags& f, int wm, int wn, int l) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = k64_frag<KA>(st, wm + i * 32, s, l);
#pragma unroll
  for (int j = 0; j < 2; ++j) f.b[j] = k64_frag<KB>(st + k64::TILE, wn + j * 32, s, l);
}

// Substeps 0..2 of a step: MFMAs of `cur` substep s while substep s+1 is
// read (restrict: the reads do not wait for the transfers in flight).
template <bool KA, bool KB>
__device__ __forceinline__ void k64_sub(const bf16_t* __restrict__ st, int s, const b8d_frags& fc, b8d_frags& fn,
                                        f32x16_t (&acc)[4][2], int wm, int wn, int l) {
  k64_read<KA, KB>(st, s + 1, fn, wm, wn, l);
  b8d_mfma(fc, acc);
  b8d_sched_half<(KA ? 4 : 8) + (KB ? 2 : 4)>();
}

// After the barrier: request tile kn into `dst` (the stage just released),
// then substep 3's MFMAs while substep 0 of the next tile is read from `nxt`.
template <bool KA, bool KB>
__device__ __forceinline__ void k64_last(const bf16_t* __restrict__ nxt, bf16_t* __restrict__ dst,
                                         const bf16_t* A, int64_t lda, int64_t m0, const bf16_t* B, int64_t ldb,
                                         int64_t n0, int64_t k0, const b8d_frags& fc, b8d_frags& fn,
                                         f32x16_t (&acc)[4][2], int w, int l, int wm, int wn, bool more) {
  if (more) {
    k64_dma_tile<KA>(A, lda, m0, k0, dst, w, l);
    k64_dma_tile<KB>(B, ldb, n0, k0, dst + k64::TILE, w, l);
  }
  k64_read<KA, KB>(nxt, 0, fn, wm, wn, l);
  b8d_mfma(fc, acc);
  b8d_sched_half<(KA ? 4 : 8) + (KB ? 2 : 4)>();
}

__device__ __forceinline__ void k64_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <typename TC, bool KA, bool KB>
__global__ __launch_bounds__(b8::NT) void gemm_k64_k(
    const bf16_t* __restrict__ A, int64_t lda, int64_t sa0, int64_t sa1,
    const bf16_t* __restrict__ B, int64_t ldb, int64_t sb0, int64_t sb1,
    TC* __restrict__ C, int64_t ldc, int64_t sc0, int64_t sc1,
    int64_t M, int64_t N, int64_t K, int64_t nb1, float alpha, int acc_c,
    int64_t kchunk, int64_t nbatch, int64_t scs) {
  constexpr int BM8 = b8::BM, BN8 = b8::BN, BK = k64::BK, TILE = k64::TILE;
  __shared__ __align__(16) bf16_t lds[2][2 * TILE];        // [stage][A tile, B tile]

  const int64_t z = blockIdx.z, split = z / nbatch, bz = z % nbatch, b0 = bz / nb1, b1 = bz % nb1;
  const int64_t kb0 = split * kchunk;
  A += b0 * sa0 + b1 * sa1 + (KA ? kb0 : kb0 * lda);
  B += b0 * sb0 + b1 * sb1 + (KB ? kb0 : kb0 * ldb);
  C += b0 * sc0 + b1 * sc1 + split * scs;
  K = K - kb0 < kchunk ? K - kb0 : kchunk;

  const int tiles_n = (int)(N / BN8);
  const int tiles = (int)(M / BM8) * tiles_n;
  const int g = blockIdx.x;
  const int tt = (tiles % 8 == 0) ? (g % 8) * (tiles / 8) + g / 8 : g;
  int64_t m0, n0;
  tile_of(tt, (int)(M / BM8), tiles_n, m0, n0, BM8, BN8);

  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / WAVE), l = threadIdx.x % WAVE;
  const int wm = (w / 4) * 128, wn = (w % 4) * 64;
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int nk = (int)(K / BK);
  // prologue: tile 0 landed and substep 0 read; tile 1 requested
  k64_dma_tile<KA>(A, lda, m0, 0, lds[0], w, l);
  k64_dma_tile<KB>(B, ldb, n0, 0, lds[0] + TILE, w, l);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (nk > 1) {
    k64_dma_tile<KA>(A, lda, m0, BK, lds[1], w, l);
    k64_dma_tile<KB>(B, ldb, n0, BK, lds[1] + TILE, w, l);
  }
  b8d_frags f0, f1;
  k64_read<KA, KB>(lds[0], 0, f0, wm, wn, l);
  for (int kt = 0; kt < nk; ++kt) {
    const bf16_t* cur = lds[kt & 1];
    k64_sub<KA, KB>(cur, 0, f0, f1, acc, wm, wn, l);
    k64_sub<KA, KB>(cur, 1, f1, f0, acc, wm, wn, l);
    k64_sub<KA, KB>(cur, 2, f0, f1, acc, wm, wn, l);
    // this wave's transfers of tile kt+1 landed, its reads of stage kt done
    __builtin_amdgcn_s_waitcnt(0x0070);                      // vmcnt(0) expcnt(7) lgkmcnt(0)
    k64_barrier();
    // the last step reads stage kt+1 % 2 too: never written past the end,
    // its substep-0 fragments are simply not used
    k64_last<KA, KB>(lds[(kt + 1) & 1], lds[kt & 1], A, lda, m0, B, ldb, n0, (int64_t)(kt + 2) * BK, f1, f0,
                     acc, w, l, wm, wn, kt + 2 < nk);
  }
  __builtin_amdgcn_s_waitcnt(0);

#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int64_t row = m0 + wm + i * 32 + 8 * (q / 4) + 4 * (l / 32) + (q % 4);
        const int64_t col = n0 + wn + j * 32 + (l % 32);
        TC* p = C + row * ldc + col;
        float v = alpha * acc[i][j][q];
        if (acc_c) v = acc_add(io<TC>::ld(p), v);
        io<TC>::st(p, v);
      }
}

// ==========================================================================
// Small f32 products (at most 256 tiles of 64 x 64 of C): one block per
// tile of TB x TB (TB = 64: 16 waves; TB = 32: 4 waves), in four groups.
// Group q sums k over its quarter of K (whole 16-deep K tiles) into its own
// 32 x 32 accumulators (2 x 2 waves, or one wave), through its own
// double-buffered LDS tiles, with the next PD K tiles of its quarter already
// requested into registers; the four partial tiles are then added in group
// order (fixed: bitwise reproducible) and written once.
//
// The four groups share one CU's matrix cores, so a block's time is bounded
// by its MFMA work (64 x 64 x 256 in f32: about 4 us); products with few
// tiles therefore take the 32 x 32 tiles, a quarter of that work per block
// on four times the CUs.  Operand tiles move as 16-byte chunks whose loads
// are the same in every step (no branch around them, out-of-range chunks
// read a block of zeros): the compiler then waits for exactly the tile a
// step stores, not for every load in flight.
// ==========================================================================
namespace sk {
constexpr int G = 4, BK = 16, LDK = BK + 4, PD = 4;
// Per tile edge TB (64 or 32): threads of a group (2 x 2 waves of 32 x 32
// accumulators, or one wave), of the block, and 16-byte chunks each thread
// moves per operand tile (TB x 16 floats).
template <int TB> struct cfg {
  static constexpr int GT = TB == 64 ? 256 : 64, NTB = G * GT, CH = TB * BK / 4 / GT;
};
}

// Never written: the source of out-of-range chunks.
__device__ __align__(16) float sk_zeros[4] = {0.f, 0.f, 0.f, 0.f};

// Chunk j of thread t in a TB x 16 operand tile: k-contiguous storage
// ([rows][K]) moves row c / 4, k (c % 4) * 4; transposed storage ([K][rows])
// moves k row c / (TB / 4), rows (c % (TB / 4)) * 4, with c = t + j * GT.
template <int TB, bool KCONTIG>
__device__ __forceinline__ void sk_pos(int c, int& row, int& kk) {
  row = KCONTIG ? c / 4 : (c % (TB / 4)) * 4;
  kk = KCONTIG ? (c % 4) * 4 : c / (TB / 4);
}

// Every lane loads, a chunk out of range from a 16-byte block of zeros, so
// each step issues the same loads and nothing is left to do on their data
// (the host guarantees no chunk straddles the end of its range).
template <int TB, bool KCONTIG>
__device__ __forceinline__ uint4 sk_load(const float* g, int64_t ld, int64_t row0, int64_t rows_total, int64_t k0,
                                         int64_t kend, int c) {
  int row, kk;
  sk_pos<TB, KCONTIG>(c, row, kk);
  const int64_t gr = row0 + row, gk = k0 + kk;
  const bool ok = gr < rows_total && gk < kend;
  typedef __attribute__((address_space(1))) const float gf;
  typedef __attribute__((address_space(1))) const u32x4_t gu4;
  gf* z = (gf*)sk_zeros;
  asm("" : "+s"(z));
  gf* p = ok ? (gf*)(KCONTIG ? g + gr * ld + gk : g + gk * ld + gr) : z;
  const u32x4_t v = *(gu4*)p;
  return make_uint4(v[0], v[1], v[2], v[3]);
}

template <int TB, bool KCONTIG>
__device__ __forceinline__ void sk_store(float* lds, uint4 r, int c) {
  int row, kk;
  sk_pos<TB, KCONTIG>(c, row, kk);
  if constexpr (KCONTIG) {
    *reinterpret_cast<uint4*>(lds + row * sk::LDK + kk) = r;
  } else {
    lds[(row + 0) * sk::LDK + kk] = __uint_as_float(r.x);
    lds[(row + 1) * sk::LDK + kk] = __uint_as_float(r.y);
    lds[(row + 2) * sk::LDK + kk] = __uint_as_float(r.z);
    lds[(row + 3) * sk::LDK + kk] = __uint_as_float(r.w);
  }
}

template <typename TC, bool TRANS_A, bool TRANS_B, int TB>
__global__ __launch_bounds__(sk::cfg<TB>::NTB) void gemm_sk_k(
    const float* __restrict__ A, int64_t lda, int64_t sa0, int64_t sa1,
    const float* __restrict__ B, int64_t ldb, int64_t sb0, int64_t sb1,
    TC* __restrict__ C, int64_t ldc, int64_t sc0, int64_t sc1,
    int64_t M, int64_t N, int64_t K, int64_t nb1, float alpha, int acc_c,
    int64_t kchunk, int64_t nbatch, int64_t scs) {
  constexpr int BK = sk::BK, LDK = sk::LDK, PD = sk::PD, GT = sk::cfg<TB>::GT, CH = sk::cfg<TB>::CH;
  constexpr int WG = GT / WAVE;                                // waves per group
  __shared__ __align__(16) float lds[sk::G][2][2][TB * LDK];   // [group][stage][A, B]

  const int64_t z = blockIdx.z, split = z / nbatch, bz = z % nbatch, b0 = bz / nb1, b1 = bz % nb1;
  const int64_t kb = split * kchunk;
  A += b0 * sa0 + b1 * sa1 + (TRANS_A ? kb * lda : kb);
  B += b0 * sb0 + b1 * sb1 + (TRANS_B ? kb : kb * ldb);
  C += b0 * sc0 + b1 * sc1 + split * scs;
  K = K - kb < kchunk ? K - kb : kchunk;
  const int64_t m0 = (int64_t)blockIdx.y * TB, n0 = (int64_t)blockIdx.x * TB;
  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  const int q = w / WG, t = threadIdx.x % GT, wg = w % WG;     // group, thread and wave within the group
  const int wm = TB == 64 ? (wg / 2) * 32 : 0, wn = TB == 64 ? (wg % 2) * 32 : 0;
  // this group's k range: whole 16-deep tiles, quarters as equal as they come
  const int64_t ntk = (K + BK - 1) / BK, per = (ntk + sk::G - 1) / sk::G;
  const int64_t kt0 = q * per, kt1 = kt0 + per < ntk ? kt0 + per : ntk;
  const int nkt = kt1 > kt0 ? (int)(kt1 - kt0) : 0;
  auto fetch = [&](int i, uint4 (&ra)[CH], uint4 (&rb)[CH]) {
    const int64_t k0 = (kt0 + i) * BK;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      ra[j] = sk_load<TB, !TRANS_A>(A, lda, m0, M, k0, K, t + j * GT);
      rb[j] = sk_load<TB, TRANS_B>(B, ldb, n0, N, k0, K, t + j * GT);
    }
  };

  f32x16_t acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  uint4 ra[PD][CH], rb[PD][CH];
#pragma unroll
  for (int u = 0; u < PD; ++u) fetch(u, ra[u], rb[u]);
  // Every group runs the same number of rounds (the barriers are the
  // block's); a group past its own tiles only passes the barriers.
  const int rounds = (int)per;
  const int lr = l % 32, lk = (l / 32) * 8;
  for (int i0 = 0; i0 < rounds; i0 += PD) {
#pragma unroll
    for (int u = 0; u < PD; ++u) {
      const int i = i0 + u;
      if (i >= rounds) break;
      float* As = lds[q][i & 1][0];
      float* Bs = lds[q][i & 1][1];
      if (i < nkt) {
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          sk_store<TB, !TRANS_A>(As, ra[u][j], t + j * GT);
          sk_store<TB, TRANS_B>(Bs, rb[u][j], t + j * GT);
        }
      }
      // a group of one wave (32 x 32 tiles) reads only what it wrote: its
      // stores complete before its reads, no block barrier
      if constexpr (WG == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      else __syncthreads();
      fetch(i + PD, ra[u], rb[u]);
      if (i < nkt) {
        const float4* pa = reinterpret_cast<const float4*>(As + (wm + lr) * LDK + lk);
        const float4* pb = reinterpret_cast<const float4*>(Bs + (wn + lr) * LDK + lk);
        const float4 a0 = pa[0], a1 = pa[1], b0v = pb[0], b1v = pb[1];
        const float a[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
        const float b[8] = {b0v.x, b0v.y, b0v.z, b0v.w, b1v.x, b1v.y, b1v.z, b1v.w};
#pragma unroll
        for (int k = 0; k < 8; ++k) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[k], b[k], acc, 0, 0, 0);
      }
    }
  }
  // partial tiles of groups 1..3 through LDS, added by group 0 in group order
  __syncthreads();
  float* red = &lds[0][0][0][0];                               // [group - 1][wave in group][16][64]
  if (q > 0) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(((q - 1) * WG + wg) * 16 + i) * WAVE + l] = acc[i];
  }
  __syncthreads();
  if (q == 0) {
#pragma unroll
    for (int g = 1; g < sk::G; ++g)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] = acc_add(acc[i], red[(((g - 1) * WG + wg) * 16 + i) * WAVE + l]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t row = m0 + wm + 8 * (i / 4) + 4 * (l / 32) + (i % 4);
      const int64_t col = n0 + wn + (l % 32);
      if (row < M && col < N) {
        TC* p = C + row * ldc + col;
        float v = alpha * acc[i];
        if (acc_c) v = acc_add(io<TC>::ld(p), v);
        io<TC>::st(p, v);
      }
    }
  }
}

// f32 products with at most 256 tiles of 64 x 64 (one per CU) run those
// tiles: a product of a few hundred rows (the tiny block's projections and
// attention scores) then spreads over four times the CUs of its 128 x 128
// tiles instead of being split along K and summed in a second pass.  Larger
// outputs keep the 128 x 128 kernels (with split-K for long K).
template <typename TA>
bool small_tiles(const xt_tensor& A, bool ta, const xt_tensor& B, bool tb, const xt_tensor& C) {
  (void)A; (void)ta; (void)B; (void)tb;
  if constexpr (sizeof(TA) == 2) return false;
  const int64_t t64 = ((C.rows + 63) / 64) * ((C.cols + 63) / 64) * C.nb[0] * C.nb[1];
  return t64 > 0 && t64 <= 256;
}

template <typename TA>
bool big_ok(const xt_tensor& A, bool ta, const xt_tensor& B, bool tb, const xt_tensor& C) {
  const int64_t M = C.rows, N = C.cols, K = ta ? A.rows : A.cols;
  const int64_t e = 16 / sizeof(TA);
  auto al = [&](const xt_tensor& t) {
    return (((uintptr_t)t.data) & 15) == 0 && t.ld % e == 0 && t.sb[0] % e == 0 && t.sb[1] % e == 0;
  };
  return M % big<TA>::BM == 0 && N % big<TA>::BN == 0 && K % big<TA>::BK == 0 && K > 0 && al(A) && al(B);
}

// ---------------------------------------------------------------- split-K
// A product with few output tiles and a long K leaves most CUs idle (weight
// gradients: a small [K_in, N_out] output summed over thousands of rows).
// Then K is cut into S slices of whole K tiles; every (tile, slice) pair is
// one block writing an f32 partial product into the workspace
// [S][batch][M][N], and a second kernel sums the S partials in slice order
// (fixed order: bitwise reproducible), scales by alpha, optionally adds C,
// and rounds once into C.  S is chosen so that tiles x S is about what the
// chip holds at once, with at least 4 K tiles per slice and at most 16
// slices, and never more slices than the workspace can hold.
struct SplitPlan { int64_t S, kchunk; };

// Kernel choice for a small f32 product (sk_kind, below).
enum { SK_NONE = 0, SK_32 = 1, SK_64 = 2, SK_GEN = 3 };

// Blocks resident on the 256 CUs at once (a SIMD holds 512 registers per
// lane; each block puts one wave on each SIMD): the f32 large-tile kernel
// uses 152 (3 per CU), the bf16 one 512 (1 per CU), the 128 x 128 kernel
// 172 (2 per CU).
SplitPlan split_plan(bool bf16, bool bigk, int sk, int64_t M, int64_t N, int64_t K, int64_t nbatch,
                     size_t ws_bytes) {
  const bool small = sk != SK_NONE;
  const int64_t tb = sk == SK_32 ? 32 : small ? 64 : BM;
  const int64_t bm = bigk ? (bf16 ? 256 : 128) : tb, bn = bigk ? (bf16 ? 256 : 128) : tb;
  const int64_t bk = bigk ? (bf16 ? big<bf16_t>::BK : big<float>::BK) : (bf16 ? gcfg<bf16_t>::BK : gcfg<float>::BK);
  // blocks the split aims at: what the chip holds at once (the generic
  // kernel on 64 x 64 tiles: 20 KB of LDS, four per CU); for the K-split
  // small kernels one block per CU, since a block already keeps its CU's
  // matrix cores busy (two 32 x 32 blocks per CU and a second summing pass
  // measured slower: tiny block 471 vs 479 us)
  const int64_t resident = bigk ? (bf16 ? 256 : 768) : sk == SK_32 ? 256 : sk == SK_64 ? 256 : sk == SK_GEN ? 1024 : 512;
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn) * nbatch;
  const int64_t nk = (K + bk - 1) / bk;
  const int64_t per = nbatch * M * N * (int64_t)sizeof(float);
  if (tiles <= 0 || nk <= 0 || per <= 0) return {1, K};
  int64_t S = resident / tiles;
  // a slice must be long enough to pay for the summing pass: at least 4 K
  // tiles (bf16), 512 of K for the f32 128-tiles and 256 for the 64-tiles
  // (measured: 1024 x 4096 x 256 f32 split in two 40 us, unsplit 12 us)
  S = std::min<int64_t>(S, small ? K / 256 : (bigk && !bf16) ? K / 512 : nk / 4);
  S = std::min<int64_t>(S, 16);
  S = std::min<int64_t>(S, (int64_t)(ws_bytes / (size_t)per));
  if (S < 2) return {1, K};
  const int64_t kchunk = (nk + S - 1) / S * bk;
  S = (K + kchunk - 1) / kchunk;
  if (S < 2) return {1, K};
  return {S, kchunk};
}

template <typename TC, int VW>
__global__ __launch_bounds__(256) void splitk_sum_k(const float* __restrict__ P, int S, int64_t scs,
                                                   TC* __restrict__ C, int64_t ldc, int64_t sc0, int64_t sc1,
                                                   int64_t M, int64_t N, int64_t nb1, int64_t items,
                                                   float alpha, int acc_c) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= items) return;
  const int64_t e = i * VW;                      // flat index in [batch][M][N]
  const int64_t n = e % N, mb = e / N, m = mb % M, bz = mb / M;
  float v[VW];
  if constexpr (VW == 4) {
    const float4 q = *reinterpret_cast<const float4*>(P + e);
    v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    for (int k = 1; k < S; ++k) {
      const float4 r = *reinterpret_cast<const float4*>(P + k * scs + e);
      v[0] += r.x; v[1] += r.y; v[2] += r.z; v[3] += r.w;
    }
  } else {
    v[0] = P[e];
    for (int k = 1; k < S; ++k) v[0] += P[k * scs + e];
  }
  TC* c = C + (bz / nb1) * sc0 + (bz % nb1) * sc1 + m * ldc + n;
#pragma unroll
  for (int j = 0; j < VW; ++j) {
    float o = alpha * v[j];
    if (acc_c) o = acc_add(io<TC>::ld(c + j), o);
    io<TC>::st(c + j, o);
  }
}

template <typename TC>
hipError_t splitk_sum(const float* P, int64_t S, int64_t scs, const xt_tensor& C, int64_t nbatch,
                      float alpha, bool acc, hipStream_t s) {
  const int64_t M = C.rows, N = C.cols, total = nbatch * M * N;
  TC* c = (TC*)C.data;
  if (N % 4 == 0) {
    const int64_t items = total / 4;
    splitk_sum_k<TC, 4><<<(unsigned)((items + 255) / 256), 256, 0, s>>>(
        P, (int)S, scs, c, C.ld, C.sb[0], C.sb[1], M, N, C.nb[1], items, alpha, acc ? 1 : 0);
  } else {
    splitk_sum_k<TC, 1><<<(unsigned)((total + 255) / 256), 256, 0, s>>>(
        P, (int)S, scs, c, C.ld, C.sb[0], C.sb[1], M, N, C.nb[1], total, alpha, acc ? 1 : 0);
  }
  return hipGetLastError();
}

// One launch of either kernel family: C (+)= alpha op(A) op(B) over k slices
// of kchunk (kchunk = K: no split), writing through C's own strides, or
// (split) into partial slices `scs` elements apart.
// Operands the small-product kernel moves as 16-byte chunks: aligned, and no
// chunk (4 consecutive k of a k-contiguous operand, 4 consecutive rows of a
// transposed one) straddles the end of its range.
bool sk_vec_ok(const xt_tensor& A, bool ta, const xt_tensor& B, bool tb, int64_t M, int64_t N, int64_t K) {
  auto al = [](const xt_tensor& t) {
    return (((uintptr_t)t.data) & 15) == 0 && t.ld % 4 == 0 && t.sb[0] % 4 == 0 && t.sb[1] % 4 == 0;
  };
  return al(A) && al(B) && (ta ? M % 4 == 0 : K % 4 == 0) && (tb ? K % 4 == 0 : N % 4 == 0);
}

// Kernel for a small f32 product: none (not small), the 16-byte-chunk
// kernel on 32 x 32 or 64 x 64 tiles, or the generic kernel on 64 x 64 tiles
// for operands it cannot move in chunks.  Products of at most 192 tiles of
// 64 x 64 take the 32 x 32 tiles: four times the CUs, each with a quarter of
// the MFMA work (1024 x 256 x 256: 11.1 -> 6.5 us; 1024 x 688 x 256: 11.7 ->
// 11.5 us); at 256 tiles the larger tiles are faster (1024 x 1024 x 256:
// 12.0 vs 15.6 us).
int sk_kind(bool small, const xt_tensor& A, bool ta, const xt_tensor& B, bool tb, const xt_tensor& C, int64_t K) {
  if (!small) return SK_NONE;
  if (!sk_vec_ok(A, ta, B, tb, C.rows, C.cols, K)) return SK_GEN;
  const int64_t t64 = ((C.rows + 63) / 64) * ((C.cols + 63) / 64) * C.nb[0] * C.nb[1];
  return t64 <= 192 ? SK_32 : SK_64;
}

template <typename TA, typename TC>
hipError_t gemm_run(bool bigk, int sk, const xt_tensor& A, bool ta, const xt_tensor& B, bool tb,
                    TC* c, int64_t ldc, int64_t sc0, int64_t sc1, int64_t M, int64_t N, int64_t K,
                    int64_t nb0, int64_t nb1, float alpha, bool acc, int64_t S, int64_t kchunk, int64_t scs,
                    hipStream_t s) {
  const TA* a = (const TA*)A.data;
  const TA* b = (const TA*)B.data;
  const int64_t nbatch = nb0 * nb1;
  if constexpr (sizeof(TA) == 2) {
   if (bigk) {
    dim3 grid((unsigned)((M / b8::BM) * (N / b8::BN)), 1, (unsigned)(S * nbatch));
    const bf16_t* a8 = (const bf16_t*)A.data;
    const bf16_t* b8p = (const bf16_t*)B.data;
#define XT_B8D(KA_, KB_)                                                                                   \
    gemm_k64_k<TC, KA_, KB_><<<grid, b8::NT, 0, s>>>(a8, A.ld, A.sb[0], A.sb[1], b8p, B.ld, B.sb[0], B.sb[1], c, \
                                                       ldc, sc0, sc1, M, N, K, nb1, alpha, acc ? 1 : 0, kchunk,  \
                                                       nbatch, scs)
    if (!ta && tb) XT_B8D(true, true);
    else if (ta && !tb) XT_B8D(false, false);
    else if (!ta && !tb) XT_B8D(true, false);
    else XT_B8D(false, true);
#undef XT_B8D
    return hipGetLastError();
   }
  } else if (bigk) {
    dim3 grid((unsigned)((M / big<TA>::BM) * (N / big<TA>::BN)), 1, (unsigned)(S * nbatch));
#define XT_BIG(TA_, TB_)                                                                           \
    gemm_big_k<TA, TC, TA_, TB_><<<grid, NT, 0, s>>>(a, A.ld, A.sb[0], A.sb[1], b, B.ld, B.sb[0], \
                                                     B.sb[1], c, ldc, sc0, sc1, M, N, K, nb1,     \
                                                     alpha, acc ? 1 : 0, kchunk, nbatch, scs)
    if (!ta && !tb) XT_BIG(false, false);
    else if (!ta && tb) XT_BIG(false, true);
    else if (ta && !tb) XT_BIG(true, false);
    else XT_BIG(true, true);
#undef XT_BIG
    return hipGetLastError();
  }
  {
    const int tbs = sk == SK_32 ? 32 : sk != SK_NONE ? 64 : BM;
    dim3 grid((unsigned)((N + tbs - 1) / tbs), (unsigned)((M + tbs - 1) / tbs), (unsigned)(S * nbatch));
    // small f32 products on the 16-wave K-split tiles (the tiny block's
    // fwd+bwd: 645 -> 607 us; keeping the 4-wave tiles for K < 128 or more
    // than 128 tiles measured 623 us)
#define XT_SK(TA_, TB_, T)                                                                              \
      gemm_sk_k<TC, TA_, TB_, T><<<grid, sk::cfg<T>::NTB, 0, s>>>((const float*)a, A.ld, A.sb[0], A.sb[1], \
                                                                  (const float*)b, B.ld, B.sb[0], B.sb[1], \
                                                                  c, ldc, sc0, sc1, M, N, K, nb1, alpha,   \
                                                                  acc ? 1 : 0, kchunk, nbatch, scs)
#define XT_GEMM_LAUNCH(TA_, TB_)                                                                        \
    if (sk == SK_32)                                                                                    \
      XT_SK(TA_, TB_, 32);                                                                              \
    else if (sk == SK_64)                                                                               \
      XT_SK(TA_, TB_, 64);                                                                              \
    else if (sk == SK_GEN)                                                                              \
      gemm_k<TA, TC, TA_, TB_, 64><<<grid, NT, 0, s>>>(a, A.ld, A.sb[0], A.sb[1], b, B.ld, B.sb[0],    \
                                                       B.sb[1], c, ldc, sc0, sc1, M, N, K, nb1, alpha, \
                                                       acc ? 1 : 0, kchunk, nbatch, scs);              \
    else                                                                                                \
      gemm_k<TA, TC, TA_, TB_><<<grid, NT, 0, s>>>(a, A.ld, A.sb[0], A.sb[1], b, B.ld, B.sb[0],        \
                                                   B.sb[1], c, ldc, sc0, sc1, M, N, K, nb1,            \
                                                   alpha, acc ? 1 : 0, kchunk, nbatch, scs)
    if (!ta && !tb) XT_GEMM_LAUNCH(false, false);
    else if (!ta && tb) XT_GEMM_LAUNCH(false, true);
    else if (ta && !tb) XT_GEMM_LAUNCH(true, false);
    else XT_GEMM_LAUNCH(true, true);
#undef XT_GEMM_LAUNCH
#undef XT_SK
  }
  return hipGetLastError();
}

template <typename TA, typename TC>
hipError_t gemm_go(const xt_tensor& A, bool ta, const xt_tensor& B, bool tb, const xt_tensor& C,
                   float alpha, bool acc, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t M = C.rows, N = C.cols, K = ta ? A.rows : A.cols;
  const int64_t nb0 = C.nb[0], nb1 = C.nb[1], nbatch = nb0 * nb1;
  if (M == 0 || N == 0 || nbatch == 0) return hipSuccess;
  const bool small = small_tiles<TA>(A, ta, B, tb, C);
  const bool bigk = !small && big_ok<TA>(A, ta, B, tb, C);
  const int sk = sk_kind(small, A, ta, B, tb, C, K);
  const SplitPlan sp = split_plan(sizeof(TA) == 2, bigk, sk, M, N, K, nbatch, ws ? ws_bytes : 0);
  if (sp.S == 1)
    return gemm_run<TA, TC>(bigk, sk, A, ta, B, tb, (TC*)C.data, C.ld, C.sb[0], C.sb[1], M, N, K, nb0, nb1,
                            alpha, acc, 1, K, 0, s);
  float* P = (float*)ws;
  const int64_t scs = nbatch * M * N;
  hipError_t e = gemm_run<TA, float>(bigk, sk, A, ta, B, tb, P, N, nb1 * M * N, M * N, M, N, K, nb0, nb1,
                                     1.f, false, sp.S, sp.kchunk, scs, s);
  if (e != hipSuccess) return e;
  return splitk_sum<TC>(P, sp.S, scs, C, nbatch, alpha, acc, s);
}

}  // namespace

hipError_t launch_gemm(const xt_tensor& A, bool ta, const xt_tensor& B, bool tb, const xt_tensor& C,
                       float alpha, bool acc, void* ws, size_t ws_bytes, hipStream_t s) {
  if (A.dtype == XT_BF16) {
    return C.dtype == XT_BF16 ? gemm_go<bf16_t, bf16_t>(A, ta, B, tb, C, alpha, acc, ws, ws_bytes, s)
                              : gemm_go<bf16_t, float>(A, ta, B, tb, C, alpha, acc, ws, ws_bytes, s);
  }
  return C.dtype == XT_BF16 ? gemm_go<float, bf16_t>(A, ta, B, tb, C, alpha, acc, ws, ws_bytes, s)
                            : gemm_go<float, float>(A, ta, B, tb, C, alpha, acc, ws, ws_bytes, s);
}

size_t gemm_workspace(const xt_tensor& A, bool ta, const xt_tensor& B, bool tb, int64_t M, int64_t N,
                      int64_t nbatch) {
  const int64_t K = ta ? A.rows : A.cols;
  if (M <= 0 || N <= 0 || K <= 0 || nbatch <= 0) return 0;
  xt_tensor C{};
  C.rows = M;
  C.cols = N;
  C.nb[0] = nbatch;
  C.nb[1] = 1;
  const bool bf = A.dtype == XT_BF16;
  // Which kernel runs depends on the operands' alignment; when the views
  // carry no pointers yet, size for the larger of the two plans.
  bool cand[2] = {false, false};
  if (A.data && B.data) cand[bf ? big_ok<bf16_t>(A, ta, B, tb, C) : big_ok<float>(A, ta, B, tb, C)] = true;
  else {
    cand[0] = true;
    xt_tensor a = A, b = B;
    a.data = b.data = nullptr;
    cand[1] = bf ? big_ok<bf16_t>(a, ta, b, tb, C) : big_ok<float>(a, ta, b, tb, C);
  }
  const bool small = bf ? small_tiles<bf16_t>(A, ta, B, tb, C) : small_tiles<float>(A, ta, B, tb, C);
  if (small) cand[0] = cand[1] = false;
  size_t best = 0;
  for (int k = 0; k < 5; ++k) {
    if (k < 2 ? !cand[k] : !small) continue;
    const SplitPlan sp = split_plan(bf, k == 1, k < 2 ? SK_NONE : k - 1, M, N, K, nbatch, SIZE_MAX);
    if (sp.S > 1) best = std::max(best, (size_t)sp.S * (size_t)(nbatch * M * N) * sizeof(float));
  }
  return best;
}

}  // namespace xt
