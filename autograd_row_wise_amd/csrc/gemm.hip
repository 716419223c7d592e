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
template <typename TA, bool KCONTIG>
struct TileLoader {
  static constexpr int BK = gcfg<TA>::BK;
  static constexpr int V = 16 / sizeof(TA);                    // elements per chunk
  static constexpr int CHUNKS = BM * BK / V;                   // chunks per tile
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
      else { kk = c / (BM / V); row = (c % (BM / V)) * V; }
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
        const int kk = c / (BM / V), row = (c % (BM / V)) * V;
        const TA* v = reinterpret_cast<const TA*>(&r[i]);
#pragma unroll
        for (int j = 0; j < V; ++j) lds[(row + j) * LDK + kk] = v[j];
      }
    }
  }
};

template <typename TA>
__device__ __forceinline__ void mfma_tile(const TA* As, const TA* Bs, int wm, int wn,
                                          f32x16_t (&acc)[2][2]) {
  constexpr int BK = gcfg<TA>::BK, LDK = BK + gcfg<TA>::PAD;
  const int l = threadIdx.x % WAVE;
  const int lr = l % 32, lk = (l / 32) * 8;
  if constexpr (sizeof(TA) == 2) {
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
      bf16x8_t a[2], b[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        a[t] = *reinterpret_cast<const bf16x8_t*>(As + (wm + t * 32 + lr) * LDK + ks + lk);
        b[t] = *reinterpret_cast<const bf16x8_t*>(Bs + (wn + t * 32 + lr) * LDK + ks + lk);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
    }
  } else {
    float a[2][8], b[2][8];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
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
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i][k], b[j][k], acc[i][j], 0, 0, 0);
  }
}

template <typename TA, typename TC, bool TRANS_A, bool TRANS_B>
__global__ __launch_bounds__(NT) void gemm_k(
    const TA* __restrict__ A, int64_t lda, int64_t sa0, int64_t sa1,
    const TA* __restrict__ B, int64_t ldb, int64_t sb0, int64_t sb1,
    TC* __restrict__ C, int64_t ldc, int64_t sc0, int64_t sc1,
    int64_t M, int64_t N, int64_t K, int64_t nb1, float alpha, int acc_c,
    int64_t kchunk, int64_t nbatch, int64_t scs) {
  constexpr int BK = gcfg<TA>::BK, LDK = BK + gcfg<TA>::PAD;
  __shared__ __align__(16) TA As[2][BM * LDK];
  __shared__ __align__(16) TA Bs[2][BN * LDK];

  // gridDim.z = splits x batches; split s sums k in [s*kchunk, (s+1)*kchunk)
  const int64_t z = blockIdx.z, split = z / nbatch, bz = z % nbatch, b0 = bz / nb1, b1 = bz % nb1;
  const int64_t kb = split * kchunk;
  A += b0 * sa0 + b1 * sa1 + (TRANS_A ? kb * lda : kb);
  B += b0 * sb0 + b1 * sb1 + (TRANS_B ? kb : kb * ldb);
  C += b0 * sc0 + b1 * sc1 + split * scs;
  K = K - kb < kchunk ? K - kb : kchunk;
  const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
  const int w = threadIdx.x / WAVE;
  const int wm = (w / 2) * 64, wn = (w % 2) * 64;

  // A as [M][K] is k-contiguous unless transposed; B as [K][N] is k-contiguous
  // only when transposed ([N][K] storage).
  TileLoader<TA, !TRANS_A> la;
  TileLoader<TA, TRANS_B> lb;
  const bool fullMN = (m0 + BM <= M) && (n0 + BN <= N);
  const bool alA = (((uintptr_t)A) & 15) == 0 && ((lda * (int64_t)sizeof(TA)) & 15) == 0;
  const bool alB = (((uintptr_t)B) & 15) == 0 && ((ldb * (int64_t)sizeof(TA)) & 15) == 0;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
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
      mfma_tile<TA>(As[cur], Bs[cur], wm, wn, acc);
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
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
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
// Large-tile kernel for aligned problems (every tile full, K a multiple of
// BK, 16-byte aligned operands).
//
//   bf16: 256 x 256 block tile, BK = 64, 4 waves (2 x 2) of 128 x 128, each
//         wave 4 x 4 accumulators of v_mfma_f32_32x32x16_bf16.
//   f32 : 128 x 128 block tile, BK = 32, 4 waves of 64 x 64, 2 x 2
//         accumulators of v_mfma_f32_32x32x2_f32.
//
// Both operands sit in LDS as [row][k] (k contiguous) rows of 128 bytes =
// eight 16-byte chunks, XOR-swizzled (swz below) so that the lanes of an
// MFMA fragment read (32 consecutive rows, one chunk) spread over all banks
// without padding.  Operands stored transposed in
// HBM ([K][rows]) are read as 8 x 8 (bf16) or 4 x 4 (f32) blocks with
// 16-byte loads and transposed in registers (v_perm_b32 for bf16) before
// the 16-byte LDS stores.  The next K tile is fetched into registers while
// the current one is multiplied.  Tiles are ordered so that each of the 8
// XCDs (blocks are dealt to XCDs round-robin) owns whole rows of tiles and
// reuses their A panels in its own L2.
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

// 8 x 8 bf16 transpose: in[k] holds m = 0..7 of row k; out[m] holds k = 0..7.
__device__ __forceinline__ void transpose8x8_bf16(const uint4 (&in)[8], uint4 (&out)[8]) {
  const uint32_t* w[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) w[k] = reinterpret_cast<const uint32_t*>(&in[k]);
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint32_t sel = (m & 1) ? 0x07060302u : 0x05040100u;
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) o[j] = __builtin_amdgcn_perm(w[2 * j + 1][m >> 1], w[2 * j][m >> 1], sel);
    out[m] = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

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
      uint4 t[V];
      if constexpr (V == 8) {
        transpose8x8_bf16(reinterpret_cast<const uint4(&)[8]>(r), reinterpret_cast<uint4(&)[8]>(t));
      } else {
        // 4 x 4 f32: r[k] = (m0..m3) of k row; t[m] = (k0..k3)
        const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
        const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
        const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
        const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
        for (int m = 0; m < 4; ++m) t[m] = make_uint4(w0[m], w1[m], w2[m], w3[m]);
      }
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
// bf16 large-tile kernel with eight waves.  A 512-thread block computes a
// 256 x 256 tile of C with BK = 64.  The waves form 2 (m) x 4 (n), each
// owning 128 x 64 of C = 4 x 2 accumulators of v_mfma_f32_32x32x16_bf16
// (128 AGPRs), so two waves share each SIMD and one wave's LDS reads and
// waits overlap the other's MFMAs.  LDS holds two K tiles (2 x 64 KB): the
// next tile is written while the current one is multiplied, with one
// barrier per K tile.  Waves 0-3 fetch the A tile and waves 4-7 the B tile,
// eight 16-byte chunks per thread, issued two K tiles ahead of their use
// (two register sets).  LDS layout and swizzle as in the kernel above.
// ==========================================================================
namespace b8 {
constexpr int BM = 256, BN = 256, BK = 64, NT = 512;
constexpr int TILE = BM * BK;                   // elements of one operand tile
}  // namespace b8

template <bool KCONTIG>
__device__ __forceinline__ void b8_load(u32x4_t (&r)[8], const bf16_t* g, int64_t ld, int64_t row0, int64_t k0,
                                        int t) {
  if constexpr (KCONTIG) {
    // rows t/8 + 32 i, k chunk t % 8: eight lanes cover one 128-byte row run
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = t / 8 + i * 32, c = t % 8;
      r[i] = *reinterpret_cast<const u32x4_t*>(g + (row0 + row) * ld + k0 + c * 8);
    }
  } else {
    // one 8 (k) x 8 (rows) block per thread: k rows 8 kb.., rows 8 mb..;
    // kb = t % 8 so that the eight lanes of an LDS store phase write eight
    // different swizzled chunk columns (no bank conflicts); each load still
    // reads 128 contiguous bytes per group of eight lanes
    const int kb = t % 8, mb = t / 8;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[i] = *reinterpret_cast<const u32x4_t*>(g + (k0 + kb * 8 + i) * ld + row0 + mb * 8);
  }
}

template <bool KCONTIG>
__device__ __forceinline__ void b8_store(const u32x4_t (&r)[8], u32x4_t* L, int t) {
  if constexpr (KCONTIG) {
#pragma unroll
    for (int i = 0; i < 8; ++i) L[swz(t / 8 + i * 32, t % 8)] = r[i];
  } else {
    // Transposed in registers: row m of the block is, per pair of k rows,
    // the m-th bf16 of each (v_perm_b32 picks the low or high halves).
    // Lanes with odd mb emit their rows in the order j ^ 1 (only the perm
    // selector changes), so the two groups of eight lanes in a sixteen-lane
    // LDS phase write rows of opposite parity: opposite halves of the
    // 256-byte bank row, no conflicts.
    const int kb = t % 8, mb = t / 8, flip = mb & 1;
    const uint32_t lo = 0x05040100u, hi = 0x07060302u;
    const uint32_t sel_even = flip ? hi : lo, sel_odd = flip ? lo : hi;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t sel = (j & 1) ? sel_odd : sel_even;
      u32x4_t o;
#pragma unroll
      for (int w = 0; w < 4; ++w) o[w] = __builtin_amdgcn_perm(r[2 * w + 1][j >> 1], r[2 * w][j >> 1], sel);
      L[swz(mb * 8 + (j ^ flip), kb)] = o;
    }
  }
}

template <bool TRANS_A, bool TRANS_B>
__device__ __forceinline__ void b8_fetch(u32x4_t (&r)[8], bool fetchA, const bf16_t* A, int64_t lda, int64_t m0,
                                         const bf16_t* B, int64_t ldb, int64_t n0, int64_t k0, int t) {
  if constexpr (!TRANS_A == TRANS_B) {            // both tiles in one layout: one code path
    b8_load<TRANS_B>(r, fetchA ? A : B, fetchA ? lda : ldb, fetchA ? m0 : n0, k0, t);
  } else {
    if (fetchA) b8_load<!TRANS_A>(r, A, lda, m0, k0, t);
    else b8_load<TRANS_B>(r, B, ldb, n0, k0, t);
  }
}

template <bool TRANS_A, bool TRANS_B>
__device__ __forceinline__ void b8_put(const u32x4_t (&r)[8], bool fetchA, u32x4_t* L, int t) {
  if constexpr (!TRANS_A == TRANS_B) {
    b8_store<TRANS_B>(r, fetchA ? L : L + b8::TILE / 8, t);
  } else {
    if (fetchA) b8_store<!TRANS_A>(r, L, t);
    else b8_store<TRANS_B>(r, L + b8::TILE / 8, t);
  }
}

// One K tile of a wave's 128 x 64 block: four k steps of 16, each 4 A and
// 2 B fragments (one 16-byte LDS read per lane each) and 8 MFMAs.
__device__ __forceinline__ void b8_mma(const u32x4_t* LA, f32x16_t (&acc)[4][2], int wm, int wn, int lr, int lh) {
  const u32x4_t* LB = LA + b8::TILE / 8;
#pragma unroll
  for (int s = 0; s < b8::BK / 16; ++s) {
    bf16x8_t a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(bf16x8_t, LA[swz(wm + i * 32 + lr, 2 * s + lh)]);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = __builtin_bit_cast(bf16x8_t, LB[swz(wn + j * 32 + lr, 2 * s + lh)]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

template <typename TC, bool TRANS_A, bool TRANS_B>
__global__ __launch_bounds__(b8::NT) void gemm_b8_k(
    const bf16_t* __restrict__ A, int64_t lda, int64_t sa0, int64_t sa1,
    const bf16_t* __restrict__ B, int64_t ldb, int64_t sb0, int64_t sb1,
    TC* __restrict__ C, int64_t ldc, int64_t sc0, int64_t sc1,
    int64_t M, int64_t N, int64_t K, int64_t nb1, float alpha, int acc_c,
    int64_t kchunk, int64_t nbatch, int64_t scs) {
  constexpr int BM8 = b8::BM, BN8 = b8::BN, BK = b8::BK, TILE = b8::TILE;
  __shared__ __align__(16) bf16_t lds[2][2 * TILE];      // [stage][A tile, B tile]

  const int64_t z = blockIdx.z, split = z / nbatch, bz = z % nbatch, b0 = bz / nb1, b1 = bz % nb1;
  const int64_t kb0 = split * kchunk;
  A += b0 * sa0 + b1 * sa1 + (TRANS_A ? kb0 * lda : kb0);
  B += b0 * sb0 + b1 * sb1 + (TRANS_B ? kb0 : kb0 * ldb);
  C += b0 * sc0 + b1 * sc1 + split * scs;
  K = K - kb0 < kchunk ? K - kb0 : kchunk;

  const int tiles_n = (int)(N / BN8);
  const int tiles = (int)(M / BM8) * tiles_n;
  const int g = blockIdx.x;
  const int tt = (tiles % 8 == 0) ? (g % 8) * (tiles / 8) + g / 8 : g;
  const int64_t m0 = (int64_t)(tt / tiles_n) * BM8, n0 = (int64_t)(tt % tiles_n) * BN8;

  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  const bool fetchA = w < 4;                     // wave-uniform role
  const int t = threadIdx.x % 256;
  const int wm = (w / 4) * 128, wn = (w % 4) * 64;

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int nk = (int)(K / BK);
  const int lr = l % 32, lh = l / 32;
  u32x4_t r0[8];
  b8_fetch<TRANS_A, TRANS_B>(r0, fetchA, A, lda, m0, B, ldb, n0, 0, t);
  b8_put<TRANS_A, TRANS_B>(r0, fetchA, reinterpret_cast<u32x4_t*>(lds[0]), t);
  if (nk > 1) b8_fetch<TRANS_A, TRANS_B>(r0, fetchA, A, lda, m0, B, ldb, n0, BK, t);
  __syncthreads();
  // K tile kt: multiply stage kt&1 while tile kt+1 is in flight; then write
  // it into the other stage and fetch tile kt+2.
  for (int kt = 0; kt < nk; ++kt) {
    b8_mma(reinterpret_cast<const u32x4_t*>(lds[kt & 1]), acc, wm, wn, lr, lh);
    if (kt + 1 < nk) {
      b8_put<TRANS_A, TRANS_B>(r0, fetchA, reinterpret_cast<u32x4_t*>(lds[(kt + 1) & 1]), t);
      if (kt + 2 < nk) b8_fetch<TRANS_A, TRANS_B>(r0, fetchA, A, lda, m0, B, ldb, n0, (int64_t)(kt + 2) * BK, t);
    }
    __syncthreads();
  }

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

// --------------------------------------------------------------------------
// bf16 NT products (both operands stored k-contiguous: dA = d B^T, and every
// product whose second operand is read transposed) skip the register
// staging: each lane issues global_load_lds_dwordx4, which writes its 16
// bytes straight into LDS at the wave's destination + 16 * lane.  K tiles
// are 32 deep (LDS rows of 64 bytes, four 16-byte chunks, chunk c of row r
// at c ^ ((r >> 2) & 3): sixteen consecutive rows read at one chunk hit
// sixteen distinct 16-byte bank groups), held in a ring of four LDS stages
// (4 x 32 KB): tile kt+3 is requested while tile kt is multiplied, and each
// wave waits only until its transfers of tile kt+1 have landed (the two
// newer tiles stay in flight) before the barrier that publishes them.
// --------------------------------------------------------------------------
namespace b8d {
constexpr int BK = 32, STAGES = 4;
constexpr int TILE = 256 * BK;                       // elements of one operand tile
}  // namespace b8d

__device__ __forceinline__ int swz4(int row, int chunk) { return row * 4 + (chunk ^ ((row >> 2) & 3)); }

// Four DMA instructions per wave per tile: operand rows row0.., k0.., both
// 256 x 32; instruction j of wave w fills slots 64 blk .. 64 blk + 63.
__device__ __forceinline__ void b8d_dma_tile(const bf16_t* g, int64_t ld, int64_t row0, int64_t k0,
                                             bf16_t* __restrict__ lds_tile, int w, int l) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int blk = w * 2 + j;                       // 64 slots = rows 16 blk .. 16 blk + 15
    const int row = blk * 16 + l / 4;
    const int c = (l % 4) ^ ((row >> 2) & 3);
    __builtin_amdgcn_global_load_lds(g + (row0 + row) * ld + k0 + c * 8, lds_tile + blk * 64 * 8, 16, 0, 0);
  }
}

__device__ __forceinline__ void b8d_mma(const u32x4_t* LA, f32x16_t (&acc)[4][2], int wm, int wn, int lr, int lh) {
  const u32x4_t* LB = LA + b8d::TILE / 8;
#pragma unroll
  for (int s = 0; s < b8d::BK / 16; ++s) {
    bf16x8_t a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = __builtin_bit_cast(bf16x8_t, LA[swz4(wm + i * 32 + lr, 2 * s + lh)]);
#pragma unroll
    for (int j = 0; j < 2; ++j) b[j] = __builtin_bit_cast(bf16x8_t, LB[swz4(wn + j * 32 + lr, 2 * s + lh)]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
  }
}

// One K tile: request tile kt+3 into `nxt`, multiply out of `cur`; restrict
// pointers let the compiler see that the reads of `cur` do not depend on the
// transfers into `nxt`.
__device__ __forceinline__ void b8d_step(const bf16_t* __restrict__ cur, bf16_t* __restrict__ nxt, bool more,
                                         const bf16_t* A, int64_t lda, int64_t m0, const bf16_t* B, int64_t ldb,
                                         int64_t n0, int64_t k0, f32x16_t (&acc)[4][2], int w, int l, int wm,
                                         int wn, int lr, int lh) {
  if (more) {
    b8d_dma_tile(A, lda, m0, k0, nxt, w, l);
    b8d_dma_tile(B, ldb, n0, k0, nxt + b8d::TILE, w, l);
  }
  b8d_mma(reinterpret_cast<const u32x4_t*>(cur), acc, wm, wn, lr, lh);
}

template <typename TC>
__global__ __launch_bounds__(b8::NT) void gemm_b8dma_k(
    const bf16_t* __restrict__ A, int64_t lda, int64_t sa0, int64_t sa1,
    const bf16_t* __restrict__ B, int64_t ldb, int64_t sb0, int64_t sb1,
    TC* __restrict__ C, int64_t ldc, int64_t sc0, int64_t sc1,
    int64_t M, int64_t N, int64_t K, int64_t nb1, float alpha, int acc_c,
    int64_t kchunk, int64_t nbatch, int64_t scs) {
  constexpr int BM8 = b8::BM, BN8 = b8::BN, BK = b8d::BK, TILE = b8d::TILE, NS = b8d::STAGES;
  __shared__ __align__(16) bf16_t lds[NS][2 * TILE];       // [stage][A tile, B tile]

  const int64_t z = blockIdx.z, split = z / nbatch, bz = z % nbatch, b0 = bz / nb1, b1 = bz % nb1;
  const int64_t kb0 = split * kchunk;
  A += b0 * sa0 + b1 * sa1 + kb0;                            // A [M][K], B [N][K]
  B += b0 * sb0 + b1 * sb1 + kb0;
  C += b0 * sc0 + b1 * sc1 + split * scs;
  K = K - kb0 < kchunk ? K - kb0 : kchunk;

  const int tiles_n = (int)(N / BN8);
  const int tiles = (int)(M / BM8) * tiles_n;
  const int g = blockIdx.x;
  const int tt = (tiles % 8 == 0) ? (g % 8) * (tiles / 8) + g / 8 : g;
  const int64_t m0 = (int64_t)(tt / tiles_n) * BM8, n0 = (int64_t)(tt % tiles_n) * BN8;

  const int w = threadIdx.x / WAVE, l = threadIdx.x % WAVE;
  const int wm = (w / 4) * 128, wn = (w % 4) * 64;
  const int lr = l % 32, lh = l / 32;
  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;

  const int nk = (int)(K / BK);
  // prologue: tiles 0, 1, 2 requested; tile 0 landed and published
#pragma unroll
  for (int p = 0; p < NS - 1; ++p)
    if (p < nk) {
      b8d_dma_tile(A, lda, m0, (int64_t)p * BK, lds[p], w, l);
      b8d_dma_tile(B, ldb, n0, (int64_t)p * BK, lds[p] + TILE, w, l);
    }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    b8d_step(lds[kt % NS], lds[(kt + NS - 1) % NS], kt + NS - 1 < nk, A, lda, m0, B, ldb, n0,
             (int64_t)(kt + NS - 1) * BK, acc, w, l, wm, wn, lr, lh);
    // Tile kt+1 must have landed: its 4 transfers are older than the (up
    // to) 8 of tiles kt+2 and kt+3, so vmcnt <= 8 suffices; lgkmcnt 0 makes
    // this wave's reads of stage kt complete before anyone may overwrite it
    // (the next step requests tile kt+4 into that stage).  Then a bare
    // s_barrier publishes tile kt+1: a full __syncthreads() fence would
    // wait for every transfer in flight.  The empty asm statements keep the
    // compiler from moving LDS accesses across the barrier.
    __builtin_amdgcn_s_waitcnt(0x078);              // vmcnt(8) expcnt(7) lgkmcnt(0)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }

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

// Blocks resident on the 256 CUs at once (a SIMD holds 512 registers per
// lane; each block puts one wave on each SIMD): the f32 large-tile kernel
// uses 152 (3 per CU), the bf16 one 512 (1 per CU), the 128 x 128 kernel
// 172 (2 per CU).
SplitPlan split_plan(bool bf16, bool bigk, int64_t M, int64_t N, int64_t K, int64_t nbatch, size_t ws_bytes) {
  const int64_t bm = bigk ? (bf16 ? 256 : 128) : BM, bn = bigk ? (bf16 ? 256 : 128) : BN;
  const int64_t bk = bigk ? (bf16 ? big<bf16_t>::BK : big<float>::BK) : (bf16 ? gcfg<bf16_t>::BK : gcfg<float>::BK);
  const int64_t resident = bigk ? (bf16 ? 256 : 768) : 512;
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + bn - 1) / bn) * nbatch;
  const int64_t nk = (K + bk - 1) / bk;
  const int64_t per = nbatch * M * N * (int64_t)sizeof(float);
  if (tiles <= 0 || nk <= 0 || per <= 0) return {1, K};
  int64_t S = resident / tiles;
  S = std::min<int64_t>(S, nk / 4);
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
template <typename TA, typename TC>
hipError_t gemm_run(bool bigk, const xt_tensor& A, bool ta, const xt_tensor& B, bool tb,
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
    if (!ta && tb) {
      gemm_b8dma_k<TC><<<grid, b8::NT, 0, s>>>(a8, A.ld, A.sb[0], A.sb[1], b8p, B.ld, B.sb[0], B.sb[1], c, ldc, sc0,
                                               sc1, M, N, K, nb1, alpha, acc ? 1 : 0, kchunk, nbatch, scs);
      return hipGetLastError();
    }
#define XT_B8(TA_, TB_)                                                                                   gemm_b8_k<TC, TA_, TB_><<<grid, b8::NT, 0, s>>>(a8, A.ld, A.sb[0], A.sb[1], b8p, B.ld, B.sb[0],                                                      B.sb[1], c, ldc, sc0, sc1, M, N, K, nb1, alpha,                                                      acc ? 1 : 0, kchunk, nbatch, scs)
    if (!ta && !tb) XT_B8(false, false);
    else if (!ta && tb) XT_B8(false, true);
    else if (ta && !tb) XT_B8(true, false);
    else XT_B8(true, true);
#undef XT_B8
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
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM), (unsigned)(S * nbatch));
#define XT_GEMM_LAUNCH(TA_, TB_)                                                              \
    gemm_k<TA, TC, TA_, TB_><<<grid, NT, 0, s>>>(a, A.ld, A.sb[0], A.sb[1], b, B.ld, B.sb[0], \
                                                 B.sb[1], c, ldc, sc0, sc1, M, N, K, nb1,     \
                                                 alpha, acc ? 1 : 0, kchunk, nbatch, scs)
    if (!ta && !tb) XT_GEMM_LAUNCH(false, false);
    else if (!ta && tb) XT_GEMM_LAUNCH(false, true);
    else if (ta && !tb) XT_GEMM_LAUNCH(true, false);
    else XT_GEMM_LAUNCH(true, true);
#undef XT_GEMM_LAUNCH
  }
  return hipGetLastError();
}

template <typename TA, typename TC>
hipError_t gemm_go(const xt_tensor& A, bool ta, const xt_tensor& B, bool tb, const xt_tensor& C,
                   float alpha, bool acc, void* ws, size_t ws_bytes, hipStream_t s) {
  const int64_t M = C.rows, N = C.cols, K = ta ? A.rows : A.cols;
  const int64_t nb0 = C.nb[0], nb1 = C.nb[1], nbatch = nb0 * nb1;
  if (M == 0 || N == 0 || nbatch == 0) return hipSuccess;
  const bool bigk = big_ok<TA>(A, ta, B, tb, C);
  const SplitPlan sp = split_plan(sizeof(TA) == 2, bigk, M, N, K, nbatch, ws ? ws_bytes : 0);
  if (sp.S == 1)
    return gemm_run<TA, TC>(bigk, A, ta, B, tb, (TC*)C.data, C.ld, C.sb[0], C.sb[1], M, N, K, nb0, nb1,
                            alpha, acc, 1, K, 0, s);
  float* P = (float*)ws;
  const int64_t scs = nbatch * M * N;
  hipError_t e = gemm_run<TA, float>(bigk, A, ta, B, tb, P, N, nb1 * M * N, M * N, M, N, K, nb0, nb1,
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
  size_t best = 0;
  for (int k = 0; k < 2; ++k) {
    if (!cand[k]) continue;
    const SplitPlan sp = split_plan(bf, k == 1, M, N, K, nbatch, SIZE_MAX);
    if (sp.S > 1) best = std::max(best, (size_t)sp.S * (size_t)(nbatch * M * N) * sizeof(float));
  }
  return best;
}

}  // namespace xt
