/*
 * xt.h -- C ABI of libxt.so: forward kernels, hand-derived backward kernels
 * and a reverse-mode tape for the row-wise ops of a small transformer, on
 * AMD Instinct MI355X (gfx950).
 *
 * Pages cited:
 *   [AE] xtrain design document "Phase: Autograd Engine + Op Backward"
 *        (docs/03-autograd-engine.md) -- sections "Module Layout",
 *        "Tape 设计", "梯度累加（扇出求和）", the op-backward table
 *        "各算子 backward 数学", the RMSNorm / RoPE / Softmax / Cross-entropy
 *        derivations, "Attention 用组合".
 *   [BP] "Träna en språkmodell: Backprop i anpassad CUDA" -- the kernel-pair
 *        table "Varje Forward-op Får En Backward-tvilling",
 *        "En baklängeskärnas uppgift", "Sparade tensorer",
 *        "Ackumulation över mikrobatcher".
 *   [DO] xtrain design document "Phase T18: Dropout (device RNG + mask)"
 *        (docs/17-dropout.md) -- "Module Layout" (dropout_mask_apply /
 *        dropout_apply_mask), "RNG：counter-based", "dropout 节点的 backward".
 *
 * Conventions for every entry point
 *   - All calls are made from the host.  Kernels are enqueued on `stream`
 *     (a hipStream_t; NULL = the null stream) and the call returns without
 *     synchronising.  Device buffers must stay alive until the stream has
 *     passed the kernels.
 *   - Every pointer inside an xt_tensor is a DEVICE pointer owned by the
 *     caller.  The op entry points allocate nothing and keep no pointer
 *     after they return.  Workspace is caller-provided (xt_workspace_bytes).
 *   - Argument, shape, dtype and workspace problems are detected on the
 *     host before anything is launched: the call returns a nonzero
 *     xt_status and launches nothing.  xt_last_error() then holds a
 *     thread-local text naming the problem.  A failed launch returns
 *     XT_ERR_HIP.  No C++ exception crosses this ABI.
 *   - Data-dependent problems are not detected on the host: a
 *     cross-entropy target outside [0, cols) gives that row a NaN loss and
 *     a NaN gradient row (so the mean loss is NaN).
 *   - Rows = 0 is a valid no-op.  Every function is re-entrant.
 */
#ifndef XT_H
#define XT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  XT_OK = 0,
  XT_ERR_INVALID_ARG = 1,   /* null pointer, bad parameter value, bad count */
  XT_ERR_SHAPE = 2,         /* shapes do not agree, ld < cols, ...          */
  XT_ERR_DTYPE = 3,         /* dtype combination not supported              */
  XT_ERR_UNSUPPORTED = 4,   /* valid request this build does not implement  */
  XT_ERR_WORKSPACE = 5,     /* workspace missing or too small               */
  XT_ERR_HIP = 6,           /* a HIP runtime call or launch failed          */
  XT_ERR_ALLOC = 7          /* the tape's allocator callback returned NULL  */
} xt_status;

typedef enum { XT_F32 = 0, XT_BF16 = 1, XT_I32 = 2, XT_U8 = 3 } xt_dtype;

/*
 * A caller-owned device view, row-major: element (r, c) of batch (i, j)
 * lives at data + i*sb[0] + j*sb[1] + r*ld + c  (all in elements).
 * Unbatched views use nb = {1, 1}, sb = {0, 0}; only MATMUL reads nb/sb.
 * Batch strides are >= 0 (0 broadcasts); a non-empty view's extent,
 * (nb[0]-1)*sb[0] + (nb[1]-1)*sb[1] + (rows-1)*ld + cols, must stay within
 * 2^56 elements, else XT_ERR_SHAPE.
 * bf16 is the upper half of an IEEE binary32 (round-to-nearest-even).
 */
typedef struct {
  void*   data;
  int32_t dtype;        /* xt_dtype */
  int32_t reserved;     /* must be 0 */
  int64_t rows, cols;
  int64_t ld;           /* >= cols */
  int64_t nb[2];        /* batch extents */
  int64_t sb[2];        /* batch strides */
} xt_tensor;

typedef enum {
  XT_OP_MATMUL = 0,        /* C = alpha * op(A) op(B)                      */
  XT_OP_ADD = 1,           /* y = a + b                                    */
  XT_OP_MUL = 2,           /* y = a * b (elementwise)                      */
  XT_OP_SCALE = 3,         /* y = alpha * x                                */
  XT_OP_ADD_BIAS = 4,      /* y[r,c] = x[r,c] + bias[c]                    */
  XT_OP_RMS_NORM = 5,      /* y = x * inv_rms * gamma                      */
  XT_OP_LAYER_NORM = 6,    /* y = (x - mean) * rstd * gamma + beta         */
  XT_OP_SOFTMAX = 7,       /* y = softmax(alpha * x) per row (+ causal)    */
  XT_OP_CROSS_ENTROPY = 8, /* L = mean_r(lse_r - x[r, t_r])                */
  XT_OP_SILU = 9,          /* y = x * sigmoid(x)                           */
  XT_OP_SWIGLU = 10,       /* y = silu(g) * u                              */
  XT_OP_GELU = 11,         /* y = x * Phi(x) (erf form; tanh form if set)  */
  XT_OP_ROPE = 12,         /* rotate-half rotary embedding                 */
  XT_OP_DROPOUT = 13,      /* counter-based inverted dropout               */
  XT_OP_EMBED = 14,        /* y[r,:] = E[ids[r],:] (token embedding)       */
  XT_OP_ATTENTION = 15,    /* softmax(alpha Q K^T [+ causal]) V, fused     */
  XT_OP_COUNT = 16
} xt_op;

typedef struct {
  float    eps;        /* RMS_NORM, LAYER_NORM: added to the mean square /
                          variance inside the square root (e.g. 1e-5)        */
  float    alpha;      /* SCALE factor; SOFTMAX pre-scale; MATMUL scale      */
  int32_t  causal;     /* SOFTMAX: 1 = column c > (row mod seq_len) excluded  */
  int32_t  seq_len;    /* SOFTMAX causal and ROPE: position = row mod seq_len */
  int32_t  head_dim;   /* ROPE: even head width; cols must be a multiple     */
  float    rope_base;  /* ROPE: theta(pos, i) = pos * base^(-2i/head_dim)    */
  float    p;          /* DROPOUT: drop probability, 0 <= p < 1              */
  int32_t  gelu_tanh;  /* GELU: 0 = exact x*Phi(x); 1 = tanh form
                          0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3)))     */
  uint64_t seed;       /* DROPOUT: 64-bit counter-RNG seed                   */
  int32_t  trans_a;    /* MATMUL: read A transposed                          */
  int32_t  trans_b;    /* MATMUL: read B transposed                          */
} xt_params;

/*
 * Per-op tensor lists (in = inputs, out = out[0] result + saved tensors,
 * din = one gradient per input; a din with data == NULL is not computed).
 *
 *  op            in                 out (fwd)                    din (bwd)
 *  MATMUL        A, B               C                            dA, dB
 *  ADD           a, b               y                            da, db
 *  MUL           a, b               y                            da, db
 *  SCALE         x                  y                            dx
 *  ADD_BIAS      x, bias[1,C] f32   y                            dx, dbias
 *  RMS_NORM      x, gamma[1,C] f32  y, inv_rms[R,1] f32          dx, dgamma
 *  LAYER_NORM    x, gamma, beta     y, mean[R,1], rstd[R,1] f32  dx, dgamma, dbeta
 *  SOFTMAX       x                  y (y is also what bwd saves) dx
 *  CROSS_ENTROPY logits, targets    L[1,1], lse[R,1], loss_row[R,1] (all f32)
 *                [R,1] i32                                       dlogits (+ a
 *                                                                NULL slot for targets)
 *  SILU, GELU    x                  y                            dx
 *  SWIGLU        g, u               y                            dg, du
 *  ROPE          x                  y                            dx
 *  DROPOUT       x                  y, mask[R,C] u8 (1 = keep)   dx
 *  EMBED         E[V,D], ids[R,1]   y[R,D] (E's dtype)           dE (+ a NULL
 *                i32                                             slot for ids)
 *  ATTENTION     q, k, v [R, H*Dh]  out [R, H*Dh], lse [R, H] f32  dq, dk, dv
 *
 * EMBED: [BP] kernel pairs (k_embed_fwd / k_embed_bwd) and the forward of
 * "Framåtgåendet" (x = embed(token_ids)); the tied output projection
 * LN(x) @ E^T is a MATMUL with trans_b on the same table.  An id outside
 * [0, V) gives a NaN output row and contributes nothing to dE.  dE[v] is
 * the sum of d over the rows with id v (f32: sums of 32 consecutive rows
 * of the id, in row order, added in order; one rounding into dE); it needs
 * workspace (24 bytes per row and 8 D bytes per 32 rows) and is bitwise
 * reproducible.
 *
 * ATTENTION: [AE] "Attention 用组合" computed without materialising the
 * probabilities.  R = B*S rows (row b*S + s = token s of sequence b), head h
 * in columns h*Dh ..; head_dim = Dh in {32, 64, 128}, seq_len = S (R a
 * multiple of S), alpha = the score scale (1/sqrt(Dh) usually), causal =
 * key t visible to query s iff t <= s.  q, k, v, out, dout and the
 * gradients share one row stride.  lse[r, h] is the log-sum-exp of the
 * scaled, masked scores of that query; the backward rebuilds the
 * probabilities from it and needs R*H*4 bytes of workspace.  Arithmetic is
 * f32-accurate for both storage types: f32 storage (and bf16 rows not
 * 16-byte aligned) runs f32 matrix-core products (MFMA 32x32x2 f32); aligned
 * bf16 storage runs bf16 matrix-core products with f32 accumulation, where
 * the operands are the stored bf16 values, except the f32 probabilities P
 * and dS = P (dP - D), which enter as the sum of two bf16 parts (hi = P
 * rounded, lo = the remainder rounded), so no product sees P or dS rounded
 * to bf16.  Only the outputs are rounded to the storage type.  Bitwise
 * reproducible.
 *
 * Backward "saved" lists: MATMUL none (reads in); RMS_NORM {inv_rms};
 * LAYER_NORM {mean, rstd}; SOFTMAX {y}; CROSS_ENTROPY {lse}; DROPOUT {mask};
 * ATTENTION {out, lse};
 * every other op none.  `dout` is the gradient of out[0] (for
 * CROSS_ENTROPY: a device f32[1,1] holding dL).
 *
 * dtypes: activations, their gradients and matmul operands are f32 or bf16
 * (all of one op's activation tensors share one dtype, except MATMUL's
 * outputs/gradients which may each be f32 or bf16); arithmetic is f32.
 * gamma/beta/bias and their gradients, and all row statistics, are f32.
 */

/* Bytes of workspace xt_op_fwd (is_bwd = 0) or xt_op_bwd (is_bwd = 1) needs
 * for these inputs; 0 if none.  Ops that need workspace: the backward of
 * RMS_NORM, LAYER_NORM and ADD_BIAS (per-block partial parameter
 * gradients, summed by a fixed-order second pass) and of EMBED (sorted
 * (id, row) keys); the MATMUL forward and backward when split-K pays. */
size_t xt_workspace_bytes(xt_op op, int is_bwd, const xt_params* prm,
                          const xt_tensor* in, int n_in);

/* Forward of `op`: reads in[0..n_in), writes out[0..n_out).
 *   [AE] op-backward table (forward column) for matmul, add, mul, add_bias,
 *   scale, rms_norm, silu, swiglu, rope, softmax, cross_entropy; [BP] kernel
 *   pairs for layer_norm, the GELU MLP and the residual add; [DO] for
 *   dropout (the mask is written to out[1]).
 * CROSS_ENTROPY writes L = (1/R) sum_r loss_row[r] by a fixed-order second
 * pass, so results are bitwise reproducible. */
xt_status xt_op_fwd(xt_op op, const xt_params* prm,
                    const xt_tensor* in, int n_in,
                    const xt_tensor* out, int n_out,
                    void* ws, size_t ws_bytes, void* stream);

/* Backward of `op`: given dout, the forward inputs and the saved tensors,
 * writes each wanted din[k].  Bit k of `accumulate` selects din[k] += grad
 * (one rounding into din's dtype) instead of din[k] = grad -- [BP]
 * "Ackumulation över mikrobatcher" (backward kernels add into the gradient
 * buffers) and [AE] "梯度累加" (fan-out sums).  Parameter gradients of
 * RMS_NORM / LAYER_NORM / ADD_BIAS come out of the same launch as dx as
 * per-block partials ([BP] "En baklängeskärnas uppgift"), then a
 * fixed-order second pass sums them: results are bitwise reproducible.
 * Two din entries must not alias each other or any input. */
xt_status xt_op_bwd(xt_op op, const xt_params* prm, const xt_tensor* dout,
                    const xt_tensor* in, int n_in,
                    const xt_tensor* saved, int n_saved,
                    const xt_tensor* din, int n_din, uint32_t accumulate,
                    void* ws, size_t ws_bytes, void* stream);

/* Size of the static device array xt_op_bwd_noalloc takes its workspace
 * from: 32 MiB, held on every GPU the library runs on until the process
 * ends. */
#define XT_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * xt_op_bwd with the same arguments and results, its workspace taken from a
 * static device array of XT_NOALLOC_SCRATCH_BYTES inside the library
 * instead of from the caller.  Calls no hipMalloc / hipFree.
 *   - Inputs, outputs and gradients are caller-owned device buffers, as for
 *     xt_op_bwd.
 *   - A backward whose workspace (xt_workspace_bytes) exceeds the array is
 *     rejected with XT_ERR_WORKSPACE before anything is launched; MATMUL
 *     instead splits its contraction less so as to fit.
 *   - The first call on a device resolves that device's copy of the array
 *     (hipGetSymbolAddress, with the device current); the array is then
 *     kept until the process ends.
 *   - Every call on one GPU uses that GPU's one array: calls whose kernels
 *     overlap on a GPU (other streams, other host threads) race.  Nothing in
 *     the array needs to start at zero, and its contents after a call are
 *     unspecified. */
xt_status xt_op_bwd_noalloc(xt_op op, const xt_params* prm, const xt_tensor* dout,
                            const xt_tensor* in, int n_in,
                            const xt_tensor* saved, int n_saved,
                            const xt_tensor* din, int n_din, uint32_t accumulate,
                            void* stream);

/* dst += src elementwise, in place (f32 arithmetic, one rounding into dst's
 * dtype).  dst and src have the same shape; dtypes may differ.
 * [AE] "梯度累加（扇出求和）": the accumulate of push_grad. */
xt_status xt_grad_accumulate(const xt_tensor* dst, const xt_tensor* src, void* stream);

/* Writes the u8 dropout mask (1 = keep) of a tensor of mask's shape:
 * element (r, c) uses counter i = r*cols + c; keep iff
 * (splitmix64(seed ^ i*0x9E3779B97F4A7C15) >> 40) * 2^-24 >= p (f32).
 * [DO] "RNG：counter-based".  0 <= p < 1, mask dtype XT_U8. */
xt_status xt_dropout_mask(const xt_tensor* mask, float p, uint64_t seed, void* stream);

/* ------------------------------------------------------------------------
 * Gradient buffers after the backward.  [BP] kernel-pair table: the helper
 * kernels k_grad_norm_partial, k_grad_norm_final and k_grad_scale for
 * gradient clipping; [BP] "Ackumulation över mikrobatcher": scale_grads(1/n)
 * averages the summed microbatch gradients, zero_grads() clears them.
 * `grads` is a host array of n caller views (f32 or bf16, unbatched, any
 * ld >= cols; empty tensors are skipped); the data are device memory.
 * ---------------------------------------------------------------------- */

/* Bytes of device workspace xt_grad_norm needs for this list: 8 per work
 * unit of 8192 elements of a row (a contiguous tensor is one row).  0 for
 * an invalid list. */
size_t xt_grad_norm_workspace(const xt_tensor* grads, int32_t n);

/* Global L2 norm over every element of every tensor, and the clipping
 * coefficient of Pascanu, Mikolov & Bengio (2013, section 3.2):
 *   out[0] = sqrt(sum g^2)  (squares exact in f64, summed in f64 in a fixed
 *            order by a partial pass and a final pass, rounded once to f32);
 *   out[1] = max_norm / norm if max_norm > 0 and norm > max_norm, else 1.
 * out: device, two f32.  max_norm >= 0 (0 = no clipping).  ws: device,
 * 8-byte aligned, xt_grad_norm_workspace bytes.  Bitwise reproducible for a
 * given list.  An empty list gives norm 0. */
xt_status xt_grad_norm(const xt_tensor* grads, int32_t n, float max_norm, float* out,
                       void* ws, size_t ws_bytes, void* stream);

/* In place: g = g * f with f = alpha, or f = alpha * scale[0] (f32) when
 * `scale` (a device f32, e.g. out + 1 of xt_grad_norm) is not NULL; each
 * element is the f32 product rounded once into g's dtype.  Reading the
 * factor on the device keeps clipping free of host synchronisation. */
xt_status xt_grads_scale(const xt_tensor* grads, int32_t n, float alpha, const float* scale, void* stream);

/* In place: g = 0 (a fill kernel, so it may be captured in a HIP graph). */
xt_status xt_grads_zero(const xt_tensor* grads, int32_t n, void* stream);

const char* xt_status_str(xt_status s);
const char* xt_last_error(void);    /* thread-local detail of the last failure */
int         xt_abi_version(void);   /* 1 */

/* ------------------------------------------------------------------------
 * Tape: define-by-run reverse mode over the ops above.
 * [AE] "Tape 设计": each op records a node (parents + what its backward
 * needs); backward() builds a post-order DFS topological order from the
 * loss (deduplicated by node), seeds the one-element loss with 1 and visits
 * the order in reverse; [AE] "梯度累加": every contribution that reaches a
 * node is summed, also when one op uses the same node twice (mul(x, x)
 * pushes twice; the node is visited once).
 *
 * Memory: the tape takes device memory only from the caller's callbacks
 * (alloc(ctx, bytes, stream) returns a device pointer or NULL; free(ctx,
 * ptr, stream) releases it in stream order), in slabs of 64 MiB or more
 * that it sub-allocates (256-byte aligned) for node values, saved tensors,
 * gradients and backward workspace; everything is released by
 * xt_tape_destroy.  Leaf values are caller views; they must outlive the tape.
 * Gradients of leaves accumulate across backward() calls until
 * xt_tape_zero_grad ([BP] "Ackumulation över mikrobatcher").
 * Functions returning xt_var return a negative value -(xt_status) on error.
 * A tape is not thread-safe.
 * ---------------------------------------------------------------------- */
typedef struct xt_tape xt_tape;
typedef int64_t xt_var;
typedef void* (*xt_alloc_fn)(void* ctx, size_t bytes, void* stream);
typedef void  (*xt_free_fn)(void* ctx, void* ptr, void* stream);

xt_tape*  xt_tape_create(xt_alloc_fn alloc, xt_free_fn free_fn, void* ctx, void* stream);
void      xt_tape_destroy(xt_tape* t);
/* A leaf over a caller view (not copied).  requires_grad = 0 for inputs that
 * get no gradient (e.g. cross-entropy targets). */
xt_var    xt_tape_leaf(xt_tape* t, const xt_tensor* value, int requires_grad);
/* Record one op on the parents (in the op's input order); the result is a
 * fresh dense tensor of the op's output shape (MATMUL with batch extents:
 * [nb0, nb1, M, N] contiguous). */
xt_var    xt_tape_apply(xt_tape* t, xt_op op, const xt_params* prm,
                        const xt_var* parents, int n_parents);
/* As xt_tape_apply, but the output is laid out by `layout` (data ignored;
 * rows, cols, ld, nb, sb, dtype used) in a fresh buffer spanning it -- e.g.
 * a batched attention product written straight into a [B*S, H*Dh] matrix. */
xt_var    xt_tape_apply_layout(xt_tape* t, xt_op op, const xt_params* prm,
                               const xt_var* parents, int n_parents,
                               const xt_tensor* layout);
/* A node that re-reads `parent`'s buffer through another layout that covers
 * the same elements exactly once (e.g. [B*S, H*Dh] as B x H heads of
 * [S, Dh]).  Its gradient is the parent's gradient seen through the layout.
 * layout->data is an element offset into the parent buffer (cast to a
 * pointer, usually 0). */
xt_var    xt_tape_view(xt_tape* t, xt_var parent, const xt_tensor* layout);
xt_status xt_tape_value(xt_tape* t, xt_var v, xt_tensor* out_view);
/* Extra forward outputs of a node (RMS_NORM inv_rms, CROSS_ENTROPY lse and
 * loss_row, DROPOUT mask, ...): index k of the op's out list, k >= 1. */
xt_status xt_tape_saved(xt_tape* t, xt_var v, int k, xt_tensor* out_view);
/* Reverse pass from a one-element loss (seeded with 1). */
xt_status xt_tape_backward(xt_tape* t, xt_var loss);
/* Reverse pass from any node, seeded with the caller's upstream gradient
 * `dout` (out's shape and dtype; unbatched): the vector-Jacobian product
 * of [AE] "验证方法" (L = sum(W * out) gives dOut = W). */
xt_status xt_tape_backward_seeded(xt_tape* t, xt_var out, const xt_tensor* dout);
/* View of v's gradient; data == NULL if no gradient reached v. */
xt_status xt_tape_grad(xt_tape* t, xt_var v, xt_tensor* out_view);
xt_status xt_tape_zero_grad(xt_tape* t);
/* Activation recompute.  [DO] "RNG：counter-based": activation recompute is
 * why the dropout mask is a pure function of (seed, element index) -- a
 * checkpoint segment re-runs its forward during backward and must draw the
 * same masks.  Ops recorded between _begin and _end form a segment: their
 * values and saved tensors live in a recompute arena that the next segment
 * (or recompute) reuses, so the tape holds one segment's activations at a
 * time.  _end(out) copies the segment's output `out` (an op node recorded
 * inside it, not a view) out of the arena; later ops may use `out` (and
 * nodes from before the segment) but no other node of the segment
 * (XT_ERR_INVALID_ARG).  xt_tape_value / xt_tape_saved of a segment's other
 * nodes fail once its arena has been reused; after a backward they read the
 * recomputed values until the next segment or recompute.  The reverse walk
 * re-runs a segment's ops when it reaches `out`, then runs their backward
 * calls: the gradients are bitwise those of the same graph recorded without
 * segments.  Segments do not nest; backward with a segment open is
 * XT_ERR_INVALID_ARG. */
xt_status xt_tape_checkpoint_begin(xt_tape* t);
xt_status xt_tape_checkpoint_end(xt_tape* t, xt_var out);
int64_t   xt_tape_num_nodes(const xt_tape* t);

#ifdef __cplusplus
}
#endif
#endif /* XT_H */
