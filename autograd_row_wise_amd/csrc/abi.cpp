// The C ABI of libxt: argument validation on the host, then dispatch to the
// kernel launchers.  Nothing here allocates device memory or synchronises.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/xt.h"
#include "internal.h"

using namespace xt;

namespace {

thread_local std::string g_err;

xt_status fail(xt_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

xt_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return XT_OK;
  return fail(XT_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool is_act(int dt) { return dt == XT_F32 || dt == XT_BF16; }

// Structural validity of one view.
xt_status check_view(const xt_tensor* t, const char* name) {
  if (!t) return fail(XT_ERR_INVALID_ARG, "%s: null tensor", name);
  if (t->dtype < XT_F32 || t->dtype > XT_U8) return fail(XT_ERR_DTYPE, "%s: unknown dtype %d", name, t->dtype);
  if (t->reserved != 0) return fail(XT_ERR_INVALID_ARG, "%s: reserved field must be 0", name);
  if (t->rows < 0 || t->cols < 0) return fail(XT_ERR_SHAPE, "%s: negative shape", name);
  if (t->rows > 0 && t->ld < t->cols) return fail(XT_ERR_SHAPE, "%s: ld (%lld) < cols (%lld)", name, (long long)t->ld, (long long)t->cols);
  if (t->nb[0] < 1 || t->nb[1] < 1) return fail(XT_ERR_SHAPE, "%s: batch extents must be >= 1", name);
  if (t->sb[0] < 0 || t->sb[1] < 0) return fail(XT_ERR_SHAPE, "%s: negative batch stride", name);
  if (t->rows > 0 && t->cols > 0) {
    // one past the last element, in elements: every index the kernels form
    // stays below it, so it must not wrap (bound: 2^56 elements)
    int64_t end = 0, b0 = 0, b1 = 0;
    if (__builtin_mul_overflow(t->rows - 1, t->ld, &end) || __builtin_add_overflow(end, t->cols, &end) ||
        __builtin_mul_overflow(t->nb[0] - 1, t->sb[0], &b0) || __builtin_add_overflow(end, b0, &end) ||
        __builtin_mul_overflow(t->nb[1] - 1, t->sb[1], &b1) || __builtin_add_overflow(end, b1, &end) ||
        end > (INT64_C(1) << 56))
      return fail(XT_ERR_SHAPE, "%s: extent of the view overflows", name);
    if (!t->data) return fail(XT_ERR_INVALID_ARG, "%s: null data", name);
  }
  return XT_OK;
}

bool unbatched(const xt_tensor& t) { return t.nb[0] == 1 && t.nb[1] == 1; }
bool same_shape(const xt_tensor& a, const xt_tensor& b) { return a.rows == b.rows && a.cols == b.cols; }

#define XT_TRY(expr) do { xt_status s_ = (expr); if (s_ != XT_OK) return s_; } while (0)

// A [1, C] or [C, 1] f32 parameter vector, contiguous.
xt_status check_param_vec(const xt_tensor* t, int64_t C, const char* name) {
  XT_TRY(check_view(t, name));
  if (t->dtype != XT_F32) return fail(XT_ERR_DTYPE, "%s must be f32", name);
  const bool row = t->rows == 1 && t->cols == C;
  const bool col = t->cols == 1 && t->rows == C && t->ld == 1;
  if (!(row || col) && C > 0) return fail(XT_ERR_SHAPE, "%s must hold %lld contiguous values", name, (long long)C);
  return XT_OK;
}

// A per-row statistic: [R, 1] of dtype dt.
xt_status check_row_vec(const xt_tensor* t, int64_t R, int dt, const char* name) {
  XT_TRY(check_view(t, name));
  if (t->dtype != dt) return fail(XT_ERR_DTYPE, "%s has the wrong dtype", name);
  if (t->rows != R || t->cols != 1) return fail(XT_ERR_SHAPE, "%s must be [%lld, 1]", name, (long long)R);
  return XT_OK;
}

xt_status check_act(const xt_tensor* t, const char* name) {
  XT_TRY(check_view(t, name));
  if (!is_act(t->dtype)) return fail(XT_ERR_DTYPE, "%s must be f32 or bf16", name);
  if (!unbatched(*t)) return fail(XT_ERR_SHAPE, "%s: batch extents are only read by MATMUL", name);
  return XT_OK;
}

xt_status check_like(const xt_tensor* t, const xt_tensor& ref, const char* name) {
  XT_TRY(check_act(t, name));
  if (!same_shape(*t, ref)) return fail(XT_ERR_SHAPE, "%s: shape [%lld, %lld] differs from [%lld, %lld]", name,
                                        (long long)t->rows, (long long)t->cols, (long long)ref.rows, (long long)ref.cols);
  if (t->dtype != ref.dtype) return fail(XT_ERR_DTYPE, "%s: dtype differs from the input's", name);
  return XT_OK;
}

bool wanted(const xt_tensor* din, int n_din, int k) { return k < n_din && din[k].data != nullptr; }

// Fill unbatched fields for a [R,1] view reading.
int64_t ld_of(const xt_tensor& t) { return t.cols == 1 ? t.ld : 1; }

// dropout threshold on the 24-bit grid: keep iff u24 >= ceil(p * 2^24)
uint32_t dropout_thr(float p) { return (uint32_t)std::ceil((double)p * 16777216.0); }
float dropout_scale(float p) {
  volatile float one = 1.0f;
  return one / (one - p);
}

xt_status check_dropout_p(float p) {
  if (!(p >= 0.f && p < 1.f)) return fail(XT_ERR_INVALID_ARG, "dropout p must be in [0, 1) (got %g)", (double)p);
  return XT_OK;
}

// matmul shape check: returns M, N, K.
xt_status check_matmul(const xt_params* prm, const xt_tensor* A, const xt_tensor* B,
                       const xt_tensor* C, int64_t* M, int64_t* N, int64_t* K) {
  XT_TRY(check_view(A, "A"));
  XT_TRY(check_view(B, "B"));
  if (!is_act(A->dtype) || A->dtype != B->dtype) return fail(XT_ERR_DTYPE, "matmul operands must both be f32 or both bf16");
  const bool ta = prm->trans_a != 0, tb = prm->trans_b != 0;
  *M = ta ? A->cols : A->rows;
  *K = ta ? A->rows : A->cols;
  const int64_t Kb = tb ? B->cols : B->rows;
  *N = tb ? B->rows : B->cols;
  if (Kb != *K) return fail(XT_ERR_SHAPE, "matmul inner dimensions differ (%lld vs %lld)", (long long)*K, (long long)Kb);
  if (C) {
    XT_TRY(check_view(C, "C"));
    if (!is_act(C->dtype)) return fail(XT_ERR_DTYPE, "matmul output must be f32 or bf16");
    if (C->rows != *M || C->cols != *N) return fail(XT_ERR_SHAPE, "matmul output must be [%lld, %lld]", (long long)*M, (long long)*N);
    for (int i = 0; i < 2; ++i) {
      if (A->nb[i] != C->nb[i] && !(A->nb[i] == 1 && A->sb[i] == 0))
        return fail(XT_ERR_SHAPE, "A batch extents differ from the output's");
      if (B->nb[i] != C->nb[i] && !(B->nb[i] == 1 && B->sb[i] == 0))
        return fail(XT_ERR_SHAPE, "B batch extents differ from the output's");
    }
  }
  return XT_OK;
}

// Partial-gradient workspace of a row backward: the larger of the
// register-resident and the generic plan (alignment is not known when the
// caller asks), exactly what the launch will use.
size_t row_ws_bound(RowKind kind, int dtype, int64_t R, int64_t C) {
  if (R <= 0 || C <= 0) return 0;
  return std::max(row_bwd_workspace(kind, dtype, R, C, true), row_bwd_workspace(kind, dtype, R, C, false));
}

// Split-K workspace of the matmul forward (C = op(A) op(B)) or of the two
// backward products (dA, dB run one after the other and share it).  The
// upstream gradient is not among the inputs: a pointer-less stand-in of its
// shape makes the plan assume the larger of the two kernels' needs.
size_t matmul_ws(const xt_params* prm, const xt_tensor* in, int n_in, int is_bwd) {
  if (!prm || n_in < 2) return 0;
  const xt_tensor &A = in[0], &B = in[1];
  const bool ta = prm->trans_a != 0, tb = prm->trans_b != 0;
  const int64_t M = ta ? A.cols : A.rows, K = ta ? A.rows : A.cols, N = tb ? B.rows : B.cols;
  const int64_t nb0 = std::max(A.nb[0], B.nb[0]), nb1 = std::max(A.nb[1], B.nb[1]), nb = nb0 * nb1;
  if (!is_bwd) return gemm_workspace(A, ta, B, tb, M, N, nb);
  xt_tensor D{};
  D.dtype = A.dtype;
  D.rows = M;
  D.cols = N;
  D.ld = N;
  D.nb[0] = nb0;
  D.nb[1] = nb1;
  D.sb[0] = nb1 * M * N;
  D.sb[1] = M * N;
  const size_t wa = !ta ? gemm_workspace(D, false, B, !tb, M, K, nb) : gemm_workspace(B, tb, D, true, K, M, nb);
  const size_t wb = !tb ? gemm_workspace(A, !ta, D, false, K, N, nb) : gemm_workspace(D, true, A, ta, N, K, nb);
  return std::max(wa, wb);
}

}  // namespace

namespace xt {
xt_status set_error(xt_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}
}  // namespace xt

extern "C" {

const char* xt_status_str(xt_status s) {
  switch (s) {
    case XT_OK: return "ok";
    case XT_ERR_INVALID_ARG: return "invalid argument";
    case XT_ERR_SHAPE: return "shape mismatch";
    case XT_ERR_DTYPE: return "unsupported dtype";
    case XT_ERR_UNSUPPORTED: return "unsupported";
    case XT_ERR_WORKSPACE: return "workspace too small";
    case XT_ERR_HIP: return "HIP error";
    case XT_ERR_ALLOC: return "allocation failed";
  }
  return "unknown status";
}

const char* xt_last_error(void) { return g_err.c_str(); }

int xt_abi_version(void) { return 1; }

// Fused attention: q, k, v (and every [R, H*Dh] tensor passed with them)
// share shape, dtype and row stride; fills the geometry of `a`.
xt_status check_attention(const xt_params* prm, const xt_tensor* in, AttnArgs& a) {
  XT_TRY(check_act(&in[0], "q"));
  XT_TRY(check_like(&in[1], in[0], "k"));
  XT_TRY(check_like(&in[2], in[0], "v"));
  if (in[1].ld != in[0].ld || in[2].ld != in[0].ld) return fail(XT_ERR_SHAPE, "attention: q, k, v must share a row stride");
  const int Dh = prm->head_dim;
  if (Dh != 32 && Dh != 64 && Dh != 128) return fail(XT_ERR_UNSUPPORTED, "attention head_dim must be 32, 64 or 128");
  if (in[0].cols % Dh) return fail(XT_ERR_SHAPE, "attention: cols must be a multiple of head_dim");
  if (prm->seq_len <= 0) return fail(XT_ERR_INVALID_ARG, "attention needs seq_len > 0");
  if (in[0].rows % prm->seq_len) return fail(XT_ERR_SHAPE, "attention: rows must be a multiple of seq_len");
  if (prm->causal != 0 && prm->causal != 1) return fail(XT_ERR_INVALID_ARG, "attention causal must be 0 or 1");
  a = AttnArgs{};
  a.q = in[0].data; a.k = in[1].data; a.v = in[2].data;
  a.S = prm->seq_len; a.B = in[0].rows / prm->seq_len; a.H = in[0].cols / Dh; a.Dh = Dh; a.ld = in[0].ld;
  if (a.B > 65535 || a.H > 65535) return fail(XT_ERR_UNSUPPORTED, "attention: at most 65535 sequences and heads");
  a.alpha = prm->alpha;
  a.causal = prm->causal;
  a.bf16 = in[0].dtype == XT_BF16;
  return XT_OK;
}

xt_status check_lse(const xt_tensor* t, const AttnArgs& a) {
  XT_TRY(check_view(t, "lse"));
  if (t->dtype != XT_F32 || t->rows != a.B * a.S || t->cols != a.H) return fail(XT_ERR_SHAPE, "lse must be [R, H] f32");
  return XT_OK;
}

size_t xt_workspace_bytes(xt_op op, int is_bwd, const xt_params* prm, const xt_tensor* in, int n_in) {
  if (!in || n_in < 1) return 0;
  if (op == XT_OP_MATMUL) return matmul_ws(prm, in, n_in, is_bwd);
  if (!is_bwd) return 0;
  const int64_t R = in[0].rows, C = in[0].cols;
  switch (op) {
    case XT_OP_RMS_NORM: return row_ws_bound(RK_RMS_BWD, in[0].dtype, R, C);
    case XT_OP_LAYER_NORM: return row_ws_bound(RK_LN_BWD, in[0].dtype, R, C);
    case XT_OP_ADD_BIAS: return colsum_workspace(in[0].dtype, R, C);
    case XT_OP_EMBED: return n_in >= 2 ? embed_bwd_workspace(in[1].rows, in[0].cols) : 0;
    case XT_OP_ATTENTION:
      return prm && prm->head_dim > 0 && R > 0 ? (size_t)R * (size_t)(C / prm->head_dim) * sizeof(float) : 0;
    default: return 0;
  }
}

xt_status xt_op_fwd(xt_op op, const xt_params* prm, const xt_tensor* in, int n_in,
                    const xt_tensor* out, int n_out, void* ws, size_t ws_bytes, void* stream) {
  if (!prm) return fail(XT_ERR_INVALID_ARG, "null params");
  if (!in || !out) return fail(XT_ERR_INVALID_ARG, "null tensor list");
  hipStream_t s = (hipStream_t)stream;
  auto need = [&](int ni, int no) -> xt_status {
    if (n_in != ni) return fail(XT_ERR_INVALID_ARG, "op %d expects %d inputs (got %d)", (int)op, ni, n_in);
    if (n_out != no) return fail(XT_ERR_INVALID_ARG, "op %d expects %d outputs (got %d)", (int)op, no, n_out);
    return XT_OK;
  };
  switch (op) {
    case XT_OP_MATMUL: {
      XT_TRY(need(2, 1));
      int64_t M, N, K;
      XT_TRY(check_matmul(prm, &in[0], &in[1], &out[0], &M, &N, &K));
      return hip_status(launch_gemm(in[0], prm->trans_a != 0, in[1], prm->trans_b != 0, out[0], prm->alpha, false,
                                    ws, ws_bytes, s), "matmul");
    }
    case XT_OP_ADD:
    case XT_OP_MUL: {
      XT_TRY(need(2, 1));
      XT_TRY(check_act(&in[0], "a"));
      XT_TRY(check_like(&in[1], in[0], "b"));
      XT_TRY(check_like(&out[0], in[0], "y"));
      EwArgs e{{&in[0], &in[1], nullptr}, {&out[0], nullptr}, 0u, 1.f, nullptr};
      return hip_status(launch_ew(op == XT_OP_ADD ? EW_ADD : EW_MUL, e, s), "add/mul");
    }
    case XT_OP_SCALE: {
      XT_TRY(need(1, 1));
      XT_TRY(check_act(&in[0], "x"));
      XT_TRY(check_like(&out[0], in[0], "y"));
      EwArgs e{{&in[0], nullptr, nullptr}, {&out[0], nullptr}, 0u, prm->alpha, nullptr};
      return hip_status(launch_ew(EW_SCALE, e, s), "scale");
    }
    case XT_OP_ADD_BIAS: {
      XT_TRY(need(2, 1));
      XT_TRY(check_act(&in[0], "x"));
      XT_TRY(check_param_vec(&in[1], in[0].cols, "bias"));
      XT_TRY(check_like(&out[0], in[0], "y"));
      EwArgs e{{&in[0], nullptr, nullptr}, {&out[0], nullptr}, 0u, 1.f, (const float*)in[1].data};
      return hip_status(launch_ew(EW_ADD_BIAS, e, s), "add_bias");
    }
    case XT_OP_SILU:
    case XT_OP_GELU: {
      XT_TRY(need(1, 1));
      XT_TRY(check_act(&in[0], "x"));
      XT_TRY(check_like(&out[0], in[0], "y"));
      if (op == XT_OP_GELU && prm->gelu_tanh != 0 && prm->gelu_tanh != 1)
        return fail(XT_ERR_INVALID_ARG, "gelu_tanh must be 0 (erf form) or 1 (tanh form)");
      EwArgs e{{&in[0], nullptr, nullptr}, {&out[0], nullptr}, 0u, 1.f, nullptr};
      const EwOp k = op == XT_OP_SILU ? EW_SILU : (prm->gelu_tanh ? EW_GELU_TANH : EW_GELU);
      return hip_status(launch_ew(k, e, s), "silu/gelu");
    }
    case XT_OP_SWIGLU: {
      XT_TRY(need(2, 1));
      XT_TRY(check_act(&in[0], "g"));
      XT_TRY(check_like(&in[1], in[0], "u"));
      XT_TRY(check_like(&out[0], in[0], "y"));
      EwArgs e{{&in[0], &in[1], nullptr}, {&out[0], nullptr}, 0u, 1.f, nullptr};
      return hip_status(launch_ew(EW_SWIGLU, e, s), "swiglu");
    }
    case XT_OP_RMS_NORM: {
      XT_TRY(need(2, 2));
      XT_TRY(check_act(&in[0], "x"));
      XT_TRY(check_param_vec(&in[1], in[0].cols, "gamma"));
      XT_TRY(check_like(&out[0], in[0], "y"));
      XT_TRY(check_row_vec(&out[1], in[0].rows, XT_F32, "inv_rms"));
      if (!(prm->eps >= 0.f)) return fail(XT_ERR_INVALID_ARG, "eps must be >= 0");
      if (in[0].cols == 0 && in[0].rows > 0) return fail(XT_ERR_SHAPE, "rms_norm needs cols >= 1");
      xt_tensor ir = out[1]; ir.ld = ld_of(out[1]);
      return hip_status(launch_rms_fwd(in[0], (const float*)in[1].data, out[0], ir, prm->eps, s), "rms_norm");
    }
    case XT_OP_LAYER_NORM: {
      XT_TRY(need(3, 3));
      XT_TRY(check_act(&in[0], "x"));
      XT_TRY(check_param_vec(&in[1], in[0].cols, "gamma"));
      XT_TRY(check_param_vec(&in[2], in[0].cols, "beta"));
      XT_TRY(check_like(&out[0], in[0], "y"));
      XT_TRY(check_row_vec(&out[1], in[0].rows, XT_F32, "mean"));
      XT_TRY(check_row_vec(&out[2], in[0].rows, XT_F32, "rstd"));
      if (!(prm->eps >= 0.f)) return fail(XT_ERR_INVALID_ARG, "eps must be >= 0");
      if (in[0].cols == 0 && in[0].rows > 0) return fail(XT_ERR_SHAPE, "layer_norm needs cols >= 1");
      xt_tensor mu = out[1], rs = out[2];
      mu.ld = ld_of(out[1]); rs.ld = ld_of(out[2]);
      return hip_status(launch_ln_fwd(in[0], (const float*)in[1].data, (const float*)in[2].data, out[0], mu, rs, prm->eps, s), "layer_norm");
    }
    case XT_OP_SOFTMAX: {
      XT_TRY(need(1, 1));
      XT_TRY(check_act(&in[0], "x"));
      XT_TRY(check_like(&out[0], in[0], "y"));
      if (prm->causal && prm->seq_len <= 0) return fail(XT_ERR_INVALID_ARG, "causal softmax needs seq_len > 0");
      if (in[0].cols == 0 && in[0].rows > 0) return fail(XT_ERR_SHAPE, "softmax needs cols >= 1");
      return hip_status(launch_softmax_fwd(in[0], out[0], prm->alpha, prm->causal, prm->seq_len, s), "softmax");
    }
    case XT_OP_CROSS_ENTROPY: {
      XT_TRY(need(2, 3));
      XT_TRY(check_act(&in[0], "logits"));
      XT_TRY(check_row_vec(&in[1], in[0].rows, XT_I32, "targets"));
      XT_TRY(check_view(&out[0], "L"));
      if (out[0].dtype != XT_F32 || out[0].rows * out[0].cols != 1) return fail(XT_ERR_SHAPE, "L must be one f32");
      XT_TRY(check_row_vec(&out[1], in[0].rows, XT_F32, "lse"));
      XT_TRY(check_row_vec(&out[2], in[0].rows, XT_F32, "loss_row"));
      if (in[0].cols == 0) return fail(XT_ERR_SHAPE, "cross_entropy needs cols >= 1");
      return hip_status(launch_ce_fwd(in[0], (const int32_t*)in[1].data, ld_of(in[1]), (float*)out[0].data,
                                      (float*)out[1].data, ld_of(out[1]), (float*)out[2].data, ld_of(out[2]), s),
                        "cross_entropy");
    }
    case XT_OP_ROPE: {
      XT_TRY(need(1, 1));
      XT_TRY(check_act(&in[0], "x"));
      XT_TRY(check_like(&out[0], in[0], "y"));
      if (prm->head_dim <= 0 || (prm->head_dim & 1)) return fail(XT_ERR_INVALID_ARG, "rope head_dim must be even and > 0");
      if (in[0].cols % prm->head_dim) return fail(XT_ERR_SHAPE, "rope: cols must be a multiple of head_dim");
      if (prm->seq_len <= 0) return fail(XT_ERR_INVALID_ARG, "rope needs seq_len > 0");
      if (!(prm->rope_base > 0.f)) return fail(XT_ERR_INVALID_ARG, "rope_base must be > 0");
      if (in[0].rows * in[0].cols > 0 && in[0].data == out[0].data)
        return fail(XT_ERR_INVALID_ARG, "rope cannot run in place");
      return hip_status(launch_rope(in[0], out[0], false, prm->head_dim, prm->rope_base, prm->seq_len, false, s), "rope");
    }
    case XT_OP_DROPOUT: {
      if (n_in != 1 || (n_out != 1 && n_out != 2)) return fail(XT_ERR_INVALID_ARG, "dropout expects 1 input and 1 or 2 outputs");
      XT_TRY(check_act(&in[0], "x"));
      XT_TRY(check_like(&out[0], in[0], "y"));
      XT_TRY(check_dropout_p(prm->p));
      const xt_tensor* mask = nullptr;
      if (n_out == 2 && out[1].data) {
        XT_TRY(check_view(&out[1], "mask"));
        if (out[1].dtype != XT_U8 || !same_shape(out[1], in[0])) return fail(XT_ERR_SHAPE, "mask must be u8 of x's shape");
        mask = &out[1];
      }
      return hip_status(launch_dropout_fwd(in[0], out[0], mask, dropout_thr(prm->p), dropout_scale(prm->p), prm->seed, s), "dropout");
    }
    case XT_OP_ATTENTION: {
      XT_TRY(need(3, 2));
      AttnArgs a;
      XT_TRY(check_attention(prm, in, a));
      XT_TRY(check_like(&out[0], in[0], "out"));
      if (out[0].ld != in[0].ld) return fail(XT_ERR_SHAPE, "attention: out must share q's row stride");
      XT_TRY(check_lse(&out[1], a));
      a.out = out[0].data;
      a.lse = (float*)out[1].data;
      a.ldl = out[1].ld;
      return hip_status(launch_attention_fwd(a, s), "attention");
    }
    case XT_OP_EMBED: {
      XT_TRY(need(2, 1));
      XT_TRY(check_act(&in[0], "E"));
      XT_TRY(check_view(&in[1], "ids"));
      if (in[1].dtype != XT_I32 || in[1].cols != 1) return fail(XT_ERR_SHAPE, "ids must be [R, 1] int32");
      if (in[1].rows > 0x7fffffff) return fail(XT_ERR_UNSUPPORTED, "embed: at most 2^31-1 rows");
      XT_TRY(check_act(&out[0], "y"));
      if (out[0].dtype != in[0].dtype || out[0].rows != in[1].rows || out[0].cols != in[0].cols)
        return fail(XT_ERR_SHAPE, "embed output must be [R, D] in E's dtype");
      return hip_status(launch_embed_fwd(in[0], (const int32_t*)in[1].data, in[1].ld, out[0], s), "embed");
    }
    default:
      return fail(XT_ERR_INVALID_ARG, "unknown op %d", (int)op);
  }
}

xt_status xt_op_bwd(xt_op op, const xt_params* prm, const xt_tensor* dout,
                    const xt_tensor* in, int n_in, const xt_tensor* saved, int n_saved,
                    const xt_tensor* din, int n_din, uint32_t accumulate,
                    void* ws, size_t ws_bytes, void* stream) {
  if (!prm) return fail(XT_ERR_INVALID_ARG, "null params");
  if (!dout || !in || (!din && n_din)) return fail(XT_ERR_INVALID_ARG, "null tensor list");
  hipStream_t s = (hipStream_t)stream;
  auto acc = [&](int k) { return ((accumulate >> k) & 1u) != 0; };
  auto need = [&](int ni, int ns, int nd) -> xt_status {
    if (n_in != ni) return fail(XT_ERR_INVALID_ARG, "op %d backward expects %d inputs (got %d)", (int)op, ni, n_in);
    if (n_saved != ns || (ns && !saved)) return fail(XT_ERR_INVALID_ARG, "op %d backward expects %d saved tensors (got %d)", (int)op, ns, n_saved);
    if (n_din != nd) return fail(XT_ERR_INVALID_ARG, "op %d backward expects %d gradient slots (got %d)", (int)op, nd, n_din);
    return XT_OK;
  };
  const size_t ws_need = xt_workspace_bytes(op, 1, prm, in, n_in);
  switch (op) {
    case XT_OP_MATMUL: {
      XT_TRY(need(2, 0, 2));
      int64_t M, N, K;
      XT_TRY(check_matmul(prm, &in[0], &in[1], dout, &M, &N, &K));
      const bool ta = prm->trans_a != 0, tb = prm->trans_b != 0;
      const xt_tensor &A = in[0], &B = in[1], &D = *dout;
      if (wanted(din, n_din, 0)) {
        XT_TRY(check_view(&din[0], "dA"));
        if (!is_act(din[0].dtype) || !same_shape(din[0], A)) return fail(XT_ERR_SHAPE, "dA must have A's shape");
        xt_tensor dA = din[0];
        for (int i = 0; i < 2; ++i) if (dA.nb[i] != D.nb[i]) return fail(XT_ERR_SHAPE, "dA batch extents must match the output's");
        hipError_t e;
        // stored dA: !ta -> d op(B)^T ; ta -> op(B) d^T
        if (!ta) e = launch_gemm(D, false, B, !tb, dA, prm->alpha, acc(0), ws, ws_bytes, s);
        else e = launch_gemm(B, tb, D, true, dA, prm->alpha, acc(0), ws, ws_bytes, s);
        XT_TRY(hip_status(e, "matmul dA"));
      }
      if (wanted(din, n_din, 1)) {
        XT_TRY(check_view(&din[1], "dB"));
        if (!is_act(din[1].dtype) || !same_shape(din[1], B)) return fail(XT_ERR_SHAPE, "dB must have B's shape");
        xt_tensor dB = din[1];
        for (int i = 0; i < 2; ++i) if (dB.nb[i] != D.nb[i]) return fail(XT_ERR_SHAPE, "dB batch extents must match the output's");
        hipError_t e;
        // stored dB: !tb -> op(A)^T d ; tb -> d^T op(A)
        if (!tb) e = launch_gemm(A, !ta, D, false, dB, prm->alpha, acc(1), ws, ws_bytes, s);
        else e = launch_gemm(D, true, A, ta, dB, prm->alpha, acc(1), ws, ws_bytes, s);
        XT_TRY(hip_status(e, "matmul dB"));
      }
      return XT_OK;
    }
    case XT_OP_ADD:
    case XT_OP_SCALE: {
      const int ni = op == XT_OP_ADD ? 2 : 1;
      XT_TRY(need(ni, 0, ni));
      XT_TRY(check_act(dout, "dout"));
      const xt_tensor* o[2] = {nullptr, nullptr};
      for (int k = 0; k < ni; ++k)
        if (wanted(din, n_din, k)) { XT_TRY(check_like(&din[k], *dout, "din")); o[k] = &din[k]; }
      if (!o[0] && !o[1]) return XT_OK;
      if (!o[0]) { o[0] = o[1]; o[1] = nullptr; accumulate = acc(1) ? 1u : 0u; }
      EwArgs e{{dout, nullptr, nullptr}, {o[0], o[1]}, accumulate, op == XT_OP_ADD ? 1.f : prm->alpha, nullptr};
      return hip_status(launch_ew(EW_SCALE, e, s), "add/scale backward");
    }
    case XT_OP_MUL: {
      XT_TRY(need(2, 0, 2));
      XT_TRY(check_act(dout, "dout"));
      XT_TRY(check_like(&in[0], *dout, "a"));
      XT_TRY(check_like(&in[1], *dout, "b"));
      const xt_tensor* o[2] = {nullptr, nullptr};
      for (int k = 0; k < 2; ++k)
        if (wanted(din, n_din, k)) { XT_TRY(check_like(&din[k], *dout, "din")); o[k] = &din[k]; }
      if (!o[0] && !o[1]) return XT_OK;
      EwArgs e{{dout, &in[0], &in[1]}, {o[0], o[1]}, accumulate, 1.f, nullptr};
      if (!o[0]) { e.out[0] = nullptr; }
      return hip_status(launch_ew(EW_MUL_BWD, e, s), "mul backward");
    }
    case XT_OP_ADD_BIAS: {
      XT_TRY(need(2, 0, 2));
      XT_TRY(check_act(dout, "dout"));
      XT_TRY(check_like(&in[0], *dout, "x"));
      XT_TRY(check_param_vec(&in[1], dout->cols, "bias"));
      if (wanted(din, n_din, 0)) {
        XT_TRY(check_like(&din[0], *dout, "dx"));
        EwArgs e{{dout, nullptr, nullptr}, {&din[0], nullptr}, acc(0) ? 1u : 0u, 1.f, nullptr};
        XT_TRY(hip_status(launch_ew(EW_SCALE, e, s), "add_bias dx"));
      }
      if (wanted(din, n_din, 1)) {
        XT_TRY(check_param_vec(&din[1], dout->cols, "dbias"));
        if (ws_bytes < ws_need || (ws_need && !ws)) return fail(XT_ERR_WORKSPACE, "add_bias backward needs %zu workspace bytes", ws_need);
        XT_TRY(hip_status(launch_colsum(*dout, (float*)din[1].data, acc(1), ws, ws_bytes, s), "add_bias dbias"));
      }
      return XT_OK;
    }
    case XT_OP_SILU:
    case XT_OP_GELU: {
      XT_TRY(need(1, 0, 1));
      XT_TRY(check_act(dout, "dout"));
      XT_TRY(check_like(&in[0], *dout, "x"));
      if (!wanted(din, n_din, 0)) return XT_OK;
      XT_TRY(check_like(&din[0], *dout, "dx"));
      if (op == XT_OP_GELU && prm->gelu_tanh != 0 && prm->gelu_tanh != 1)
        return fail(XT_ERR_INVALID_ARG, "gelu_tanh must be 0 (erf form) or 1 (tanh form)");
      EwArgs e{{dout, &in[0], nullptr}, {&din[0], nullptr}, acc(0) ? 1u : 0u, 1.f, nullptr};
      const EwOp k = op == XT_OP_SILU ? EW_SILU_BWD : (prm->gelu_tanh ? EW_GELU_TANH_BWD : EW_GELU_BWD);
      return hip_status(launch_ew(k, e, s), "silu/gelu backward");
    }
    case XT_OP_SWIGLU: {
      XT_TRY(need(2, 0, 2));
      XT_TRY(check_act(dout, "dout"));
      XT_TRY(check_like(&in[0], *dout, "g"));
      XT_TRY(check_like(&in[1], *dout, "u"));
      const xt_tensor* o[2] = {nullptr, nullptr};
      for (int k = 0; k < 2; ++k)
        if (wanted(din, n_din, k)) { XT_TRY(check_like(&din[k], *dout, "din")); o[k] = &din[k]; }
      if (!o[0] && !o[1]) return XT_OK;
      EwArgs e{{dout, &in[0], &in[1]}, {o[0], o[1]}, accumulate, 1.f, nullptr};
      return hip_status(launch_ew(EW_SWIGLU_BWD, e, s), "swiglu backward");
    }
    case XT_OP_RMS_NORM: {
      XT_TRY(need(2, 1, 2));
      XT_TRY(check_act(dout, "dout"));
      XT_TRY(check_like(&in[0], *dout, "x"));
      XT_TRY(check_param_vec(&in[1], dout->cols, "gamma"));
      XT_TRY(check_row_vec(&saved[0], dout->rows, XT_F32, "inv_rms"));
      const xt_tensor* dx = nullptr;
      float* dg = nullptr;
      if (wanted(din, n_din, 0)) { XT_TRY(check_like(&din[0], *dout, "dx")); dx = &din[0]; }
      if (wanted(din, n_din, 1)) { XT_TRY(check_param_vec(&din[1], dout->cols, "dgamma")); dg = (float*)din[1].data; }
      if (!dx && !dg) return XT_OK;
      if (dg && (ws_bytes < ws_need || (ws_need && !ws))) return fail(XT_ERR_WORKSPACE, "rms_norm backward needs %zu workspace bytes", ws_need);
      xt_tensor ir = saved[0]; ir.ld = ld_of(saved[0]);
      return hip_status(launch_rms_bwd(*dout, in[0], (const float*)in[1].data, ir, dx, acc(0), dg, acc(1), ws, ws_bytes, s),
                        "rms_norm backward");
    }
    case XT_OP_LAYER_NORM: {
      XT_TRY(need(3, 2, 3));
      XT_TRY(check_act(dout, "dout"));
      XT_TRY(check_like(&in[0], *dout, "x"));
      XT_TRY(check_param_vec(&in[1], dout->cols, "gamma"));
      XT_TRY(check_param_vec(&in[2], dout->cols, "beta"));
      XT_TRY(check_row_vec(&saved[0], dout->rows, XT_F32, "mean"));
      XT_TRY(check_row_vec(&saved[1], dout->rows, XT_F32, "rstd"));
      const xt_tensor* dx = nullptr;
      float *dg = nullptr, *db = nullptr;
      if (wanted(din, n_din, 0)) { XT_TRY(check_like(&din[0], *dout, "dx")); dx = &din[0]; }
      if (wanted(din, n_din, 1)) { XT_TRY(check_param_vec(&din[1], dout->cols, "dgamma")); dg = (float*)din[1].data; }
      if (wanted(din, n_din, 2)) { XT_TRY(check_param_vec(&din[2], dout->cols, "dbeta")); db = (float*)din[2].data; }
      if (!dx && !dg && !db) return XT_OK;
      if ((dg || db) && (ws_bytes < ws_need || (ws_need && !ws))) return fail(XT_ERR_WORKSPACE, "layer_norm backward needs %zu workspace bytes", ws_need);
      xt_tensor mu = saved[0], rs = saved[1];
      mu.ld = ld_of(saved[0]); rs.ld = ld_of(saved[1]);
      return hip_status(launch_ln_bwd(*dout, in[0], (const float*)in[1].data, mu, rs, dx, acc(0), dg, acc(1), db, acc(2), ws,
                                      ws_bytes, s),
                        "layer_norm backward");
    }
    case XT_OP_SOFTMAX: {
      XT_TRY(need(1, 1, 1));
      XT_TRY(check_act(dout, "dout"));
      XT_TRY(check_like(&saved[0], *dout, "y"));
      if (!wanted(din, n_din, 0)) return XT_OK;
      XT_TRY(check_like(&din[0], *dout, "dx"));
      return hip_status(launch_softmax_bwd(*dout, saved[0], din[0], acc(0), prm->alpha, s), "softmax backward");
    }
    case XT_OP_CROSS_ENTROPY: {
      XT_TRY(need(2, 1, n_din < 1 ? 1 : n_din));
      if (n_din < 1 || n_din > 2) return fail(XT_ERR_INVALID_ARG, "cross_entropy backward takes 1 or 2 gradient slots");
      if (n_din == 2 && din[1].data) return fail(XT_ERR_INVALID_ARG, "targets have no gradient");
      XT_TRY(check_view(dout, "dL"));
      if (dout->dtype != XT_F32 || dout->rows * dout->cols != 1) return fail(XT_ERR_SHAPE, "dL must be one f32");
      XT_TRY(check_act(&in[0], "logits"));
      XT_TRY(check_row_vec(&in[1], in[0].rows, XT_I32, "targets"));
      XT_TRY(check_row_vec(&saved[0], in[0].rows, XT_F32, "lse"));
      if (!wanted(din, n_din, 0)) return XT_OK;
      XT_TRY(check_like(&din[0], in[0], "dlogits"));
      return hip_status(launch_ce_bwd((const float*)dout->data, in[0], (const int32_t*)in[1].data, ld_of(in[1]),
                                      (const float*)saved[0].data, ld_of(saved[0]), din[0], acc(0), s),
                        "cross_entropy backward");
    }
    case XT_OP_ROPE: {
      XT_TRY(need(1, 0, 1));
      XT_TRY(check_act(dout, "dout"));
      if (prm->head_dim <= 0 || (prm->head_dim & 1)) return fail(XT_ERR_INVALID_ARG, "rope head_dim must be even and > 0");
      if (dout->cols % prm->head_dim) return fail(XT_ERR_SHAPE, "rope: cols must be a multiple of head_dim");
      if (prm->seq_len <= 0) return fail(XT_ERR_INVALID_ARG, "rope needs seq_len > 0");
      if (!(prm->rope_base > 0.f)) return fail(XT_ERR_INVALID_ARG, "rope_base must be > 0");
      if (!wanted(din, n_din, 0)) return XT_OK;
      XT_TRY(check_like(&din[0], *dout, "dx"));
      if (din[0].data == dout->data) return fail(XT_ERR_INVALID_ARG, "rope backward cannot run in place");
      return hip_status(launch_rope(*dout, din[0], acc(0), prm->head_dim, prm->rope_base, prm->seq_len, true, s), "rope backward");
    }
    case XT_OP_DROPOUT: {
      XT_TRY(need(1, 1, 1));
      XT_TRY(check_act(dout, "dout"));
      XT_TRY(check_dropout_p(prm->p));
      XT_TRY(check_view(&saved[0], "mask"));
      if (saved[0].dtype != XT_U8 || !same_shape(saved[0], *dout)) return fail(XT_ERR_SHAPE, "mask must be u8 of dout's shape");
      if (!wanted(din, n_din, 0)) return XT_OK;
      XT_TRY(check_like(&din[0], *dout, "dx"));
      return hip_status(launch_dropout_bwd(*dout, saved[0], din[0], acc(0), dropout_scale(prm->p), s), "dropout backward");
    }
    case XT_OP_ATTENTION: {
      XT_TRY(need(3, 2, 3));
      AttnArgs a;
      XT_TRY(check_attention(prm, in, a));
      XT_TRY(check_like(dout, in[0], "dout"));
      XT_TRY(check_like(&saved[0], in[0], "out"));
      if (dout->ld != in[0].ld || saved[0].ld != in[0].ld) return fail(XT_ERR_SHAPE, "attention: dout and out must share q's row stride");
      XT_TRY(check_lse(&saved[1], a));
      for (int i = 0; i < 3; ++i) {
        if (!wanted(din, n_din, i)) continue;
        XT_TRY(check_like(&din[i], in[0], i == 0 ? "dq" : i == 1 ? "dk" : "dv"));
        if (din[i].ld != in[0].ld) return fail(XT_ERR_SHAPE, "attention: gradients must share q's row stride");
      }
      if (!wanted(din, n_din, 0) && !wanted(din, n_din, 1) && !wanted(din, n_din, 2)) return XT_OK;
      if (ws_need && (!ws || ws_bytes < ws_need)) return fail(XT_ERR_WORKSPACE, "attention backward needs %zu bytes of workspace", ws_need);
      a.out = saved[0].data;
      a.lse = (float*)saved[1].data;
      a.ldl = saved[1].ld;
      a.dout = dout->data;
      a.dd = (float*)ws;
      a.dq = wanted(din, n_din, 0) ? din[0].data : nullptr;
      a.dk = wanted(din, n_din, 1) ? din[1].data : nullptr;
      a.dv = wanted(din, n_din, 2) ? din[2].data : nullptr;
      a.acc_dq = acc(0); a.acc_dk = acc(1); a.acc_dv = acc(2);
      return hip_status(launch_attention_bwd(a, s), "attention backward");
    }
    case XT_OP_EMBED: {
      if (n_in != 2 || n_saved != 0 || n_din < 1 || n_din > 2)
        return fail(XT_ERR_INVALID_ARG, "embed backward takes E, ids, no saved tensors and 1 or 2 gradient slots");
      if (n_din == 2 && din[1].data) return fail(XT_ERR_INVALID_ARG, "ids have no gradient");
      XT_TRY(check_act(&in[0], "E"));
      XT_TRY(check_view(&in[1], "ids"));
      if (in[1].dtype != XT_I32 || in[1].cols != 1) return fail(XT_ERR_SHAPE, "ids must be [R, 1] int32");
      if (in[1].rows > 0x7fffffff) return fail(XT_ERR_UNSUPPORTED, "embed: at most 2^31-1 rows");
      XT_TRY(check_act(dout, "dout"));
      if (dout->rows != in[1].rows || dout->cols != in[0].cols || dout->dtype != in[0].dtype)
        return fail(XT_ERR_SHAPE, "embed dout must be [R, D] in E's dtype");
      if (!wanted(din, n_din, 0)) return XT_OK;
      XT_TRY(check_like(&din[0], in[0], "dE"));
      if (ws_need && (!ws || ws_bytes < ws_need)) return fail(XT_ERR_WORKSPACE, "embed backward needs %zu bytes of workspace", ws_need);
      return hip_status(launch_embed_bwd(*dout, (const int32_t*)in[1].data, in[1].ld, din[0], acc(0), ws, s),
                        "embed backward");
    }
    default:
      return fail(XT_ERR_INVALID_ARG, "unknown op %d", (int)op);
  }
}

xt_status xt_grad_accumulate(const xt_tensor* dst, const xt_tensor* src, void* stream) {
  XT_TRY(check_act(dst, "dst"));
  XT_TRY(check_act(src, "src"));
  if (!same_shape(*dst, *src)) return fail(XT_ERR_SHAPE, "accumulate: shapes differ");
  EwArgs e{{src, nullptr, nullptr}, {dst, nullptr}, 1u, 1.f, nullptr};
  return hip_status(launch_ew(EW_ACCUMULATE, e, (hipStream_t)stream), "grad_accumulate");
}

xt_status xt_dropout_mask(const xt_tensor* mask, float p, uint64_t seed, void* stream) {
  XT_TRY(check_view(mask, "mask"));
  if (mask->dtype != XT_U8) return fail(XT_ERR_DTYPE, "mask must be u8");
  if (!unbatched(*mask)) return fail(XT_ERR_SHAPE, "mask must be unbatched");
  XT_TRY(check_dropout_p(p));
  return hip_status(launch_dropout_mask_only(*mask, dropout_thr(p), seed, (hipStream_t)stream), "dropout_mask");
}

// ---- gradient buffers after the backward ----
static xt_status check_grad_list(const xt_tensor* g, int32_t n) {
  if (n < 0) return fail(XT_ERR_INVALID_ARG, "negative tensor count");
  if (n > 0 && !g) return fail(XT_ERR_INVALID_ARG, "null tensor list");
  for (int32_t i = 0; i < n; ++i) {
    char name[32];
    snprintf(name, sizeof name, "grads[%d]", (int)i);
    XT_TRY(check_act(&g[i], name));
  }
  return XT_OK;
}

size_t xt_grad_norm_workspace(const xt_tensor* grads, int32_t n) {
  if (check_grad_list(grads, n) != XT_OK) return 0;
  return (size_t)grad_norm_units(grads, n) * sizeof(double);
}

xt_status xt_grad_norm(const xt_tensor* grads, int32_t n, float max_norm, float* out, void* ws, size_t ws_bytes,
                       void* stream) {
  XT_TRY(check_grad_list(grads, n));
  if (!out) return fail(XT_ERR_INVALID_ARG, "grad_norm: null output");
  if (!(max_norm >= 0.f)) return fail(XT_ERR_INVALID_ARG, "grad_norm: max_norm must be >= 0 (0 = no clipping)");
  const int64_t units = grad_norm_units(grads, n);
  if (units > 0x7fffffff) return fail(XT_ERR_UNSUPPORTED, "grad_norm: too many work units");
  const size_t need = (size_t)units * sizeof(double);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(XT_ERR_WORKSPACE, "grad_norm needs %zu bytes of workspace", need);
  if (((uintptr_t)ws) % 8 != 0) return fail(XT_ERR_INVALID_ARG, "grad_norm: workspace must be 8-byte aligned");
  return hip_status(launch_grad_norm(grads, n, max_norm, out, (double*)ws, (hipStream_t)stream), "grad_norm");
}

xt_status xt_grads_scale(const xt_tensor* grads, int32_t n, float alpha, const float* scale, void* stream) {
  XT_TRY(check_grad_list(grads, n));
  return hip_status(launch_grads_scale(grads, n, false, alpha, scale, (hipStream_t)stream), "grads_scale");
}

xt_status xt_grads_zero(const xt_tensor* grads, int32_t n, void* stream) {
  XT_TRY(check_grad_list(grads, n));
  return hip_status(launch_grads_scale(grads, n, true, 0.f, nullptr, (hipStream_t)stream), "grads_zero");
}

}  // extern "C"
