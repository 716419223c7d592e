// Internal launch interface between the C ABI (abi.cpp) and the kernels.
// Every launcher enqueues on `stream`, returns hipSuccess or the launch
// error, and assumes the ABI layer has already validated shapes, dtypes,
// alignment and workspace size.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/xt.h"

namespace xt {

// Sets the thread-local text xt_last_error() returns (printf format) and
// returns `s`.
xt_status set_error(xt_status s, const char* fmt, ...);

// --- row-wise reductions (rowwise.hip) ---------------------------------
// Plan of a row-resident launch: RW waves share one row, each thread keeps
// NV 16-byte packs of it in registers; rows longer than the register
// capacity, or rows that are not 16-byte aligned, use the generic path.
struct RowPlan {
  bool fast;        // register-resident vector path
  int rw, nv;       // waves per row, packs per thread
  int block;        // threads per block
  int grid;         // blocks
  int groups;       // rows in flight per block (block / (64*rw))
};

enum RowKind { RK_RMS_FWD, RK_RMS_BWD, RK_LN_FWD, RK_LN_BWD, RK_SM_FWD, RK_SM_BWD };

RowPlan plan_rows(RowKind kind, int dtype, int64_t R, int64_t C, bool aligned);
// Workspace (bytes) of the parameter-gradient partials of a row backward.
size_t row_bwd_workspace(RowKind kind, int dtype, int64_t R, int64_t C, bool aligned);

hipError_t launch_rms_fwd(const xt_tensor& x, const float* gamma, const xt_tensor& y,
                          const xt_tensor& inv_rms, float eps, hipStream_t s);
// Backward launchers never write past ws_bytes: the block count is clamped so
// the per-block partial rows fit the workspace they are given.
hipError_t launch_rms_bwd(const xt_tensor& d, const xt_tensor& x, const float* gamma,
                          const xt_tensor& inv_rms, const xt_tensor* dx, bool acc_dx,
                          float* dgamma, bool acc_dgamma, void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_ln_fwd(const xt_tensor& x, const float* gamma, const float* beta,
                         const xt_tensor& y, const xt_tensor& mean, const xt_tensor& rstd,
                         float eps, hipStream_t s);
hipError_t launch_ln_bwd(const xt_tensor& d, const xt_tensor& x, const float* gamma,
                         const xt_tensor& mean, const xt_tensor& rstd,
                         const xt_tensor* dx, bool acc_dx, float* dgamma, bool acc_dgamma,
                         float* dbeta, bool acc_dbeta, void* ws, size_t ws_bytes, hipStream_t s);
hipError_t launch_softmax_fwd(const xt_tensor& x, const xt_tensor& y, float alpha,
                              int causal, int seq_len, hipStream_t s);
hipError_t launch_softmax_bwd(const xt_tensor& d, const xt_tensor& y, const xt_tensor& dx,
                              bool acc, float alpha, hipStream_t s);

// Streaming row kernels (rowstream.hip) for rows the register-resident
// kernels do not take: one 1024-thread block per row step, `grid` blocks.
// The backward launchers write `part` (one partial row of the parameter
// gradients per block) only where every row starts 16-byte aligned and
// stream_owns_partials holds; `part` = nullptr skips them.
constexpr int STREAM_BWD_GRID = 256;
int stream_bwd_grid(int64_t R);
bool stream_owns_partials(int dtype, int64_t C, const xt_tensor& d, const xt_tensor& x, const xt_tensor* dx);
hipError_t launch_sm_fwd_stream(const xt_tensor& x, const xt_tensor& y, float alpha, int causal, int seq_len,
                                int grid, hipStream_t s);
hipError_t launch_sm_bwd_stream(const xt_tensor& d, const xt_tensor& y, const xt_tensor& dx, bool acc, float alpha,
                                int grid, hipStream_t s);
hipError_t launch_rms_fwd_stream(const xt_tensor& x, const float* gamma, const xt_tensor& y, const xt_tensor& ir,
                                 float eps, int grid, hipStream_t s);
hipError_t launch_ln_fwd_stream(const xt_tensor& x, const float* gamma, const float* beta, const xt_tensor& y,
                                const xt_tensor& mean, const xt_tensor& rstd, float eps, int grid, hipStream_t s);
hipError_t launch_rms_bwd_stream(const xt_tensor& d, const xt_tensor& x, const float* gamma, const xt_tensor& ir,
                                 const xt_tensor* dx, bool acc_dx, float* part, int grid, hipStream_t s);
hipError_t launch_ln_bwd_stream(const xt_tensor& d, const xt_tensor& x, const float* gamma, const xt_tensor& mean,
                                const xt_tensor& rstd, const xt_tensor* dx, bool acc_dx, float* part, int grid,
                                hipStream_t s);

// Column sums: out[c] (+)= sum_r d[r, c]  (add_bias backward).
size_t colsum_workspace(int dtype, int64_t R, int64_t C);
hipError_t launch_colsum(const xt_tensor& d, float* out, bool acc, void* ws, size_t ws_bytes, hipStream_t s);

// --- cross entropy (ce.hip) --------------------------------------------
hipError_t launch_ce_fwd(const xt_tensor& logits, const int32_t* targets, int64_t ld_t,
                         float* L, float* lse, int64_t ld_lse, float* loss_row,
                         int64_t ld_loss, hipStream_t s);
hipError_t launch_ce_bwd(const float* dL, const xt_tensor& logits, const int32_t* targets,
                         int64_t ld_t, const float* lse, int64_t ld_lse,
                         const xt_tensor& dlogits, bool acc, hipStream_t s);

// --- elementwise (elementwise.hip) ---------------------------------------
enum EwOp {
  EW_ADD, EW_MUL, EW_SCALE, EW_ADD_BIAS, EW_SILU, EW_GELU, EW_SWIGLU,
  EW_COPY_SCALED,              // out0 (+)= alpha * in0
  EW_MUL_BWD,                  // out0 (+)= d*b, out1 (+)= d*a
  EW_SILU_BWD, EW_GELU_BWD, EW_SWIGLU_BWD,
  EW_GELU_TANH, EW_GELU_TANH_BWD,
  EW_ACCUMULATE                // out0 += in0 (dtypes may differ)
};
struct EwArgs {
  const xt_tensor* in[3];
  const xt_tensor* out[2];     // NULL = not wanted
  uint32_t acc;                // bit k: out[k] +=
  float alpha;
  const float* colvec;         // ADD_BIAS: bias[C]
};
hipError_t launch_ew(EwOp op, const EwArgs& a, hipStream_t s);

// --- dropout (elementwise.hip) -------------------------------------------
// keep iff (splitmix64(seed ^ i*gamma) >> 40) >= thr, thr = ceil(p * 2^24).
hipError_t launch_dropout_fwd(const xt_tensor& x, const xt_tensor& y, const xt_tensor* mask,
                              uint32_t thr, float scale, uint64_t seed, hipStream_t s);
hipError_t launch_dropout_mask_only(const xt_tensor& mask, uint32_t thr, uint64_t seed,
                                    hipStream_t s);
hipError_t launch_dropout_bwd(const xt_tensor& d, const xt_tensor& mask, const xt_tensor& dx,
                              bool acc, float scale, hipStream_t s);

// --- rope (rope.hip) ------------------------------------------------------
hipError_t launch_rope(const xt_tensor& x, const xt_tensor& y, bool acc, int head_dim,
                       float base, int seq_len, bool inverse, hipStream_t s);

// --- matmul (gemm.hip) ----------------------------------------------------
// C (+)= alpha * op(A) op(B), batched over nb[0] x nb[1].  With workspace,
// products with few output tiles and a long K are split along K (f32
// partials + a fixed-order sum); with less workspace they split less.
hipError_t launch_gemm(const xt_tensor& A, bool ta, const xt_tensor& B, bool tb, const xt_tensor& C,
                       float alpha, bool acc, void* ws, size_t ws_bytes, hipStream_t s);
// Workspace that launch_gemm would use for C = op(A) op(B) of M x N, nbatch batches.
size_t gemm_workspace(const xt_tensor& A, bool ta, const xt_tensor& B, bool tb, int64_t M, int64_t N,
                      int64_t nbatch);

// --- misc -------------------------------------------------------------------
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);

// embed.hip: token-embedding gather and its deterministic scatter-add
// backward (per-chunk LDS sort of (id, row) keys into `ws`, then per-run sums).
size_t embed_bwd_workspace(int64_t R, int64_t D);
hipError_t launch_embed_fwd(const xt_tensor& E, const int32_t* ids, int64_t ldi, const xt_tensor& y, hipStream_t s);
hipError_t launch_embed_bwd(const xt_tensor& d, const int32_t* ids, int64_t ldi, const xt_tensor& dE, bool acc,
                            void* ws, hipStream_t s);

// attention.hip: fused (flash-style) attention over [B*S, H*Dh] q, k, v.
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;          // forward output; read by the backward (D = rowsum(dO * O))
  float* lse;         // [B*S, H] log-sum-exp, row stride ldl
  const void* dout;   // backward
  float* dd;          // backward workspace: [B*S, H] f32
  void* dq;
  void* dk;
  void* dv;
  int acc_dq, acc_dk, acc_dv;
  int64_t B, S, H, Dh, ld, ldl;
  float alpha;
  int causal;
  bool bf16;
};
hipError_t launch_attention_fwd(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_bwd(const AttnArgs& a, hipStream_t s);

// gradbuf.hip: global gradient norm (two passes through `part`, f64 per
// work unit) and in-place scaling / zeroing of a list of gradient tensors.
int64_t grad_norm_units(const xt_tensor* g, int n);
hipError_t launch_grad_norm(const xt_tensor* g, int n, float max_norm, float* out, double* part, hipStream_t s);
hipError_t launch_grads_scale(const xt_tensor* g, int n, bool zero, float alpha, const float* scale,
                              hipStream_t s);

}  // namespace xt
