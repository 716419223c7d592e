// Reverse-mode tape over the libxt ops.
//
// [AE] "Tape 设计": each recorded op is a node holding its value, its parents
// and what its backward needs (here: the op, its parameters and the saved
// forward outputs); backward() builds a post-order depth-first topological
// order from the loss (each node once), seeds the loss gradient with 1 and
// walks the order in reverse, pushing each node's gradient to its parents.
// [AE] "梯度累加（扇出求和）": a push into a parent that already holds a
// gradient adds to it -- here the `accumulate` bit of xt_op_bwd, so the sum
// is fused into the producing kernel instead of a separate add.  When an op
// uses one node twice (mul(x, x)) the backward is issued once per use, each
// writing only that use's gradient, so the two pushes are summed in order
// and never race.
//
// All device memory (values, saved tensors, gradients, workspace) comes from
// the caller's allocator callbacks; all work is enqueued on one stream and
// nothing here synchronises.
//
// Activation recompute ([DO] "RNG：counter-based": a checkpoint segment
// re-runs its forward during backward, which is why the dropout mask is a
// pure function of (seed, element index)): the ops recorded between
// xt_tape_checkpoint_begin and xt_tape_checkpoint_end form a segment whose
// values and saved tensors live in a recompute arena that the next segment
// reuses; only the segment's output is copied out and stays readable.  The
// reverse walk reaches a segment through its output (no other node of a
// segment may be used outside it), re-runs the segment's ops into the arena
// and then runs their backward calls, newest first.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/xt.h"
#include "internal.h"

namespace {

int elem_size(int dt) {
  switch (dt) {
    case XT_F32: return 4;
    case XT_BF16: return 2;
    case XT_I32: return 4;
    default: return 1;
  }
}

// Number of elements a layout reaches from its base (largest offset + 1).
int64_t span_elems(const xt_tensor& t) {
  if (t.rows == 0 || t.cols == 0) return 0;
  return (t.nb[0] - 1) * t.sb[0] + (t.nb[1] - 1) * t.sb[1] + (t.rows - 1) * t.ld + t.cols;
}

xt_tensor dense(void* p, int dt, int64_t rows, int64_t cols) {
  xt_tensor t{};
  t.data = p; t.dtype = dt; t.rows = rows; t.cols = cols; t.ld = cols;
  t.nb[0] = t.nb[1] = 1;
  return t;
}

struct Node {
  xt_op op = XT_OP_COUNT;        // XT_OP_COUNT: leaf or view
  bool leaf = false, view = false;
  bool needs_grad = false;
  xt_params prm{};
  std::vector<xt_var> parents;
  xt_tensor value{};
  std::vector<xt_tensor> extra;  // forward outputs after the first (saved tensors)
  xt_tensor grad{};              // same layout as value; data == NULL until allocated
  bool grad_live = false;        // a gradient has been written (this pass / since zero_grad)
  int64_t root = -1;             // views: the node owning the buffers
  int64_t offset = 0;            // views: element offset from the parent's value
  int seg = -1;                  // checkpoint segment whose arena holds the buffers
  bool seg_out = false;          // the segment's output (value copied out of the arena)
  uint64_t epoch = 0;            // arena epoch the buffers were written in
};

struct Segment {
  xt_var first = 0, last = -1, out = -1;
};

}  // namespace

// Device memory of a tape comes from the caller's allocator in slabs of at
// least SLAB bytes; values, saved tensors, gradients and workspace are
// carved from them with 256-byte alignment and live until the tape is
// destroyed.  One allocator callback serves many tensors, which keeps the
// per-op host cost of recording and of backward low.
struct xt_tape {
  static constexpr size_t SLAB = size_t(64) << 20;
  static constexpr size_t ALIGN = 256;
  xt_alloc_fn alloc;
  xt_free_fn release;
  void* ctx;
  hipStream_t stream;
  std::vector<Node> nodes;
  std::vector<void*> owned;      // every slab the tape allocated
  char* cur = nullptr;           // bump region of the newest slab
  size_t left = 0;
  void* ws = nullptr;            // op workspace, reused by every call (stream order)
  size_t ws_cap = 0;
  std::string err;
  // recompute arena: chunks reused from the start by every segment (forward
  // or recompute); `epoch` counts the rewinds
  std::vector<std::pair<char*, size_t>> arena;
  size_t a_chunk = 0, a_off = 0;
  uint64_t epoch = 1;
  int open_seg = -1;
  std::vector<Segment> segs;

  void rewind() {
    a_chunk = 0;
    a_off = 0;
    ++epoch;
  }

  void* aget(size_t bytes) {
    bytes = (bytes + ALIGN - 1) / ALIGN * ALIGN;
    if (bytes == 0) bytes = ALIGN;
    while (a_chunk < arena.size() && arena[a_chunk].second - a_off < bytes) {
      ++a_chunk;
      a_off = 0;
    }
    if (a_chunk == arena.size()) {
      const size_t n = bytes > SLAB ? bytes : SLAB;
      void* p = alloc(ctx, n, (void*)stream);
      if (!p) return nullptr;
      owned.push_back(p);
      arena.push_back({static_cast<char*>(p), n});
      a_off = 0;
    }
    char* p = arena[a_chunk].first + a_off;
    a_off += bytes;
    return p;
  }

  // Workspace of one op call.  Calls run in stream order on the tape's
  // stream, so one buffer serves them all; it only grows.
  void* scratch(size_t bytes) {
    if (bytes <= ws_cap) return ws;
    bytes = (bytes + ALIGN - 1) / ALIGN * ALIGN;
    void* p = alloc(ctx, bytes, (void*)stream);
    if (!p) return nullptr;
    owned.push_back(p);
    ws = p;
    ws_cap = bytes;
    return ws;
  }

  void* get(size_t bytes) {
    bytes = (bytes + ALIGN - 1) / ALIGN * ALIGN;
    if (bytes == 0) bytes = ALIGN;
    if (bytes > left) {
      const size_t n = bytes > SLAB ? bytes : SLAB;
      void* p = alloc(ctx, n, (void*)stream);
      if (!p) return nullptr;
      owned.push_back(p);
      cur = static_cast<char*>(p);
      left = n;
    }
    void* p = cur;
    cur += bytes;
    left -= bytes;
    return p;
  }
};

namespace {

xt_var bad(xt_status s) { return -(xt_var)s; }

bool valid_var(const xt_tape* t, xt_var v) { return t && v >= 0 && v < (xt_var)t->nodes.size(); }

// A node later ops may read: outside every segment, a segment's output, or
// a node of the segment being recorded.
bool usable(const xt_tape* t, xt_var v) {
  const Node& n = t->nodes[v];
  return n.seg < 0 || n.seg_out || n.seg == t->open_seg;
}

// Whether v's buffers hold its current values (a closed segment's arena
// buffers are only valid between its recompute and the next rewind).
bool current(const xt_tape* t, xt_var v) {
  const Node& n = t->nodes[v];
  return n.seg < 0 || n.epoch == t->epoch;
}

// Owner of the gradient storage of node v (itself unless it is a view).
int64_t grad_owner(const xt_tape* t, xt_var v) {
  const Node& n = t->nodes[v];
  return n.view ? n.root : v;
}

// Make sure v's gradient view exists; views map into their root's buffer.
xt_status ensure_grad(xt_tape* t, xt_var v) {
  Node& n = t->nodes[v];
  if (n.grad.data) return XT_OK;
  if (n.view) {
    Node& p = t->nodes[n.parents[0]];
    xt_status s = ensure_grad(t, n.parents[0]);
    if (s != XT_OK) return s;
    n.grad = n.value;
    n.grad.data = (char*)p.grad.data + n.offset * elem_size(n.value.dtype);
    return XT_OK;
  }
  const int64_t span = span_elems(n.value);
  void* buf = t->get((size_t)span * elem_size(n.value.dtype));
  if (!buf && span > 0) return XT_ERR_ALLOC;
  n.grad = n.value;
  n.grad.data = buf;
  return XT_OK;
}

bool grad_live(const xt_tape* t, xt_var v) { return t->nodes[grad_owner(t, v)].grad_live; }
void set_grad_live(xt_tape* t, xt_var v) { t->nodes[grad_owner(t, v)].grad_live = true; }

// Output shapes of an op applied to parent values.
xt_status out_shapes(xt_op op, const xt_params& prm, const std::vector<const xt_tensor*>& in,
                     std::vector<xt_tensor>& outs) {
  const xt_tensor& x = *in[0];
  outs.clear();
  switch (op) {
    case XT_OP_MATMUL: {
      const xt_tensor& b = *in[1];
      const int64_t M = prm.trans_a ? x.cols : x.rows;
      const int64_t N = prm.trans_b ? b.rows : b.cols;
      xt_tensor c = dense(nullptr, x.dtype, M, N);
      c.nb[0] = std::max(x.nb[0], b.nb[0]);
      c.nb[1] = std::max(x.nb[1], b.nb[1]);
      c.sb[1] = M * N;
      c.sb[0] = c.nb[1] * M * N;
      outs.push_back(c);
      return XT_OK;
    }
    case XT_OP_EMBED:
      outs.push_back(dense(nullptr, x.dtype, in[1]->rows, x.cols));
      return XT_OK;
    case XT_OP_ATTENTION:
      if (prm.head_dim <= 0) return XT_ERR_INVALID_ARG;
      outs.push_back(dense(nullptr, x.dtype, x.rows, x.cols));
      outs.push_back(dense(nullptr, XT_F32, x.rows, x.cols / prm.head_dim));
      return XT_OK;
    case XT_OP_CROSS_ENTROPY:
      outs.push_back(dense(nullptr, XT_F32, 1, 1));
      outs.push_back(dense(nullptr, XT_F32, x.rows, 1));
      outs.push_back(dense(nullptr, XT_F32, x.rows, 1));
      return XT_OK;
    default:
      break;
  }
  outs.push_back(dense(nullptr, x.dtype, x.rows, x.cols));
  if (op == XT_OP_RMS_NORM) outs.push_back(dense(nullptr, XT_F32, x.rows, 1));
  if (op == XT_OP_LAYER_NORM) {
    outs.push_back(dense(nullptr, XT_F32, x.rows, 1));
    outs.push_back(dense(nullptr, XT_F32, x.rows, 1));
  }
  if (op == XT_OP_DROPOUT) outs.push_back(dense(nullptr, XT_U8, x.rows, x.cols));
  return XT_OK;
}

// Saved tensors the backward of `op` reads (after the inputs).
std::vector<xt_tensor> saved_of(const Node& n) {
  switch (n.op) {
    case XT_OP_RMS_NORM: return {n.extra[0]};
    case XT_OP_LAYER_NORM: return {n.extra[0], n.extra[1]};
    case XT_OP_SOFTMAX: return {n.value};
    case XT_OP_CROSS_ENTROPY: return {n.extra[0]};
    case XT_OP_DROPOUT: return {n.extra[0]};
    case XT_OP_ATTENTION: return {n.value, n.extra[0]};
    default: return {};
  }
}

xt_var apply_impl(xt_tape* t, xt_op op, const xt_params* prm, const xt_var* parents, int n,
                  const xt_tensor* layout) {
  if (!t || !prm || (n > 0 && !parents)) return bad(XT_ERR_INVALID_ARG);
  if (op < 0 || op >= XT_OP_COUNT || n < 1 || n > 3) return bad(XT_ERR_INVALID_ARG);
  for (int i = 0; i < n; ++i)
    if (!valid_var(t, parents[i]) || !usable(t, parents[i])) return bad(XT_ERR_INVALID_ARG);
  // [DO] "dropout 节点": p == 0 is the identity and records no node
  if (op == XT_OP_DROPOUT && prm->p == 0.f) return parents[0];

  std::vector<const xt_tensor*> in;
  std::vector<xt_tensor> in_vals;
  for (int i = 0; i < n; ++i) in_vals.push_back(t->nodes[parents[i]].value);
  for (auto& v : in_vals) in.push_back(&v);
  std::vector<xt_tensor> outs;
  xt_status s = out_shapes(op, *prm, in, outs);
  if (s != XT_OK) return bad(s);
  if (layout) {
    xt_tensor l = *layout;
    if (l.rows != outs[0].rows || l.cols != outs[0].cols || l.nb[0] != outs[0].nb[0] || l.nb[1] != outs[0].nb[1])
      return bad(XT_ERR_SHAPE);
    l.data = nullptr;
    outs[0] = l;
  }
  const bool in_seg = t->open_seg >= 0;
  for (auto& o : outs) {
    const size_t bytes = (size_t)span_elems(o) * elem_size(o.dtype);
    o.data = in_seg ? t->aget(bytes) : t->get(bytes);
    if (!o.data) return bad(XT_ERR_ALLOC);
  }
  const size_t wsb = xt_workspace_bytes(op, 0, prm, in_vals.data(), n);
  void* ws = nullptr;
  if (wsb && !(ws = t->scratch(wsb))) return bad(XT_ERR_ALLOC);
  s = xt_op_fwd(op, prm, in_vals.data(), n, outs.data(), (int)outs.size(), ws, wsb, (void*)t->stream);
  if (s != XT_OK) return bad(s);
  Node nd;
  nd.op = op;
  nd.prm = *prm;
  nd.parents.assign(parents, parents + n);
  nd.value = outs[0];
  nd.extra.assign(outs.begin() + 1, outs.end());
  for (int i = 0; i < n; ++i) nd.needs_grad = nd.needs_grad || t->nodes[parents[i]].needs_grad;
  nd.seg = t->open_seg;
  nd.epoch = t->epoch;
  t->nodes.push_back(nd);
  return (xt_var)t->nodes.size() - 1;
}

// Re-runs segment `sg`'s ops into the (rewound) arena, in recording order:
// the same ops on the same inputs, so the values, saved tensors and dropout
// masks are the ones the first forward computed.  The output's value stays
// in its copy outside the arena; its saved tensors are rewritten.
xt_status recompute(xt_tape* t, int sg) {
  const Segment& S = t->segs[sg];
  t->rewind();
  for (xt_var u = S.first; u <= S.last; ++u) {
    Node& n = t->nodes[u];
    if (n.seg != sg) continue;
    if (n.view) {
      const Node& r = t->nodes[n.root];
      n.value.data = (char*)r.value.data + n.offset * elem_size(n.value.dtype);
      n.epoch = t->epoch;
      continue;
    }
    const int np = (int)n.parents.size();
    std::vector<xt_tensor> in_vals(np);
    for (int i = 0; i < np; ++i) in_vals[i] = t->nodes[n.parents[i]].value;
    std::vector<xt_tensor> outs;
    outs.push_back(n.value);
    for (const auto& e : n.extra) outs.push_back(e);
    for (auto& o : outs) {
      o.data = t->aget((size_t)span_elems(o) * elem_size(o.dtype));
      if (!o.data) return XT_ERR_ALLOC;
    }
    const size_t wsb = xt_workspace_bytes(n.op, 0, &n.prm, in_vals.data(), np);
    void* ws = nullptr;
    if (wsb && !(ws = t->scratch(wsb))) return XT_ERR_ALLOC;
    const xt_status s = xt_op_fwd(n.op, &n.prm, in_vals.data(), np, outs.data(), (int)outs.size(), ws, wsb,
                                  (void*)t->stream);
    if (s != XT_OK) return s;
    if (!n.seg_out) n.value = outs[0];
    for (size_t i = 0; i < n.extra.size(); ++i) n.extra[i] = outs[i + 1];
    n.epoch = t->epoch;
  }
  return XT_OK;
}

}  // namespace

extern "C" {

xt_tape* xt_tape_create(xt_alloc_fn alloc, xt_free_fn free_fn, void* ctx, void* stream) {
  if (!alloc || !free_fn) return nullptr;
  xt_tape* t = new (std::nothrow) xt_tape;
  if (!t) return nullptr;
  t->alloc = alloc;
  t->release = free_fn;
  t->ctx = ctx;
  t->stream = (hipStream_t)stream;
  return t;
}

void xt_tape_destroy(xt_tape* t) {
  if (!t) return;
  for (void* p : t->owned) t->release(t->ctx, p, (void*)t->stream);
  delete t;
}

int64_t xt_tape_num_nodes(const xt_tape* t) { return t ? (int64_t)t->nodes.size() : 0; }

xt_var xt_tape_leaf(xt_tape* t, const xt_tensor* value, int requires_grad) {
  if (!t || !value) return bad(XT_ERR_INVALID_ARG);
  if (value->rows < 0 || value->cols < 0 || value->nb[0] < 1 || value->nb[1] < 1) return bad(XT_ERR_SHAPE);
  if (value->rows * value->cols > 0 && !value->data) return bad(XT_ERR_INVALID_ARG);
  Node nd;
  nd.leaf = true;
  nd.value = *value;
  nd.needs_grad = requires_grad != 0;
  t->nodes.push_back(nd);
  return (xt_var)t->nodes.size() - 1;
}

xt_var xt_tape_apply(xt_tape* t, xt_op op, const xt_params* prm, const xt_var* parents, int n) {
  return apply_impl(t, op, prm, parents, n, nullptr);
}

xt_var xt_tape_apply_layout(xt_tape* t, xt_op op, const xt_params* prm, const xt_var* parents,
                            int n, const xt_tensor* layout) {
  if (!layout) return bad(XT_ERR_INVALID_ARG);
  return apply_impl(t, op, prm, parents, n, layout);
}

xt_var xt_tape_view(xt_tape* t, xt_var parent, const xt_tensor* layout) {
  if (!valid_var(t, parent) || !layout || !usable(t, parent)) return bad(XT_ERR_INVALID_ARG);
  const Node& p = t->nodes[parent];
  const int64_t off = (int64_t)(intptr_t)layout->data;
  xt_tensor v = *layout;
  v.dtype = p.value.dtype;
  if (v.rows * v.cols * v.nb[0] * v.nb[1] != p.value.rows * p.value.cols * p.value.nb[0] * p.value.nb[1])
    return bad(XT_ERR_SHAPE);                       // must cover the parent's elements
  if (off < 0 || off + span_elems(v) > span_elems(p.value)) return bad(XT_ERR_SHAPE);
  v.data = (char*)p.value.data + off * elem_size(p.value.dtype);
  Node nd;
  nd.view = true;
  nd.parents = {parent};
  nd.value = v;
  nd.root = p.view ? p.root : parent;
  nd.offset = off;
  nd.needs_grad = p.needs_grad;
  nd.seg = (p.seg >= 0 && !p.seg_out) ? p.seg : -1;   // shares its root's buffer
  nd.epoch = t->epoch;
  t->nodes.push_back(nd);
  return (xt_var)t->nodes.size() - 1;
}

xt_status xt_tape_value(xt_tape* t, xt_var v, xt_tensor* out) {
  if (!valid_var(t, v) || !out) return XT_ERR_INVALID_ARG;
  if (!t->nodes[v].seg_out && !current(t, v)) return XT_ERR_INVALID_ARG;   // in a rewound arena
  *out = t->nodes[v].value;
  return XT_OK;
}

xt_status xt_tape_saved(xt_tape* t, xt_var v, int k, xt_tensor* out) {
  if (!valid_var(t, v) || !out || k < 1) return XT_ERR_INVALID_ARG;
  const Node& n = t->nodes[v];
  if (k - 1 >= (int)n.extra.size() || !current(t, v)) return XT_ERR_INVALID_ARG;
  *out = n.extra[k - 1];
  return XT_OK;
}

xt_status xt_tape_grad(xt_tape* t, xt_var v, xt_tensor* out) {
  if (!valid_var(t, v) || !out) return XT_ERR_INVALID_ARG;
  *out = t->nodes[v].value;
  out->data = grad_live(t, v) ? t->nodes[v].grad.data : nullptr;
  return XT_OK;
}

xt_status xt_tape_zero_grad(xt_tape* t) {
  if (!t) return XT_ERR_INVALID_ARG;
  for (auto& n : t->nodes) n.grad_live = false;
  return XT_OK;
}

xt_status xt_tape_checkpoint_begin(xt_tape* t) {
  if (!t || t->open_seg >= 0) return XT_ERR_INVALID_ARG;
  Segment sg;
  sg.first = (xt_var)t->nodes.size();
  t->segs.push_back(sg);
  t->open_seg = (int)t->segs.size() - 1;
  t->rewind();
  return XT_OK;
}

xt_status xt_tape_checkpoint_end(xt_tape* t, xt_var out) {
  if (!t || t->open_seg < 0 || !valid_var(t, out)) return XT_ERR_INVALID_ARG;
  Node& o = t->nodes[out];
  if (o.seg != t->open_seg || o.view || o.leaf) return XT_ERR_INVALID_ARG;
  const size_t bytes = (size_t)span_elems(o.value) * elem_size(o.value.dtype);
  void* dst = t->get(bytes);
  if (!dst) return XT_ERR_ALLOC;
  if (bytes && hipMemcpyAsync(dst, o.value.data, bytes, hipMemcpyDeviceToDevice, t->stream) != hipSuccess)
    return XT_ERR_HIP;
  o.value.data = dst;
  o.seg_out = true;
  Segment& sg = t->segs[t->open_seg];
  sg.last = (xt_var)t->nodes.size() - 1;
  sg.out = out;
  // views of the output recorded inside the segment now read the copy
  for (xt_var u = sg.first; u <= sg.last; ++u) {
    Node& n = t->nodes[u];
    if (n.view && n.root == out) {
      n.value.data = (char*)dst + n.offset * elem_size(n.value.dtype);
      n.seg = -1;
    }
  }
  t->open_seg = -1;
  t->rewind();
  return XT_OK;
}

}  // extern "C"

namespace {
// Shared reverse walk: `seed` writes the gradient of `out` once its buffer exists.
template <typename Seed>
xt_status reverse_pass(xt_tape* t, xt_var out, Seed seed) {
  // post-order DFS (iterative), each node once
  std::vector<xt_var> order;
  std::vector<char> state(t->nodes.size(), 0);     // 0 new, 1 open, 2 done
  std::vector<std::pair<xt_var, size_t>> stack{{out, 0}};
  state[out] = 1;
  while (!stack.empty()) {
    auto& top = stack.back();
    const Node& n = t->nodes[top.first];
    if (top.second < n.parents.size()) {
      const xt_var p = n.parents[top.second++];
      if (state[p] == 0) { state[p] = 1; stack.push_back({p, 0}); }
    } else {
      state[top.first] = 2;
      order.push_back(top.first);
      stack.pop_back();
    }
  }
  // intermediate gradients belong to this pass; leaf gradients keep
  // accumulating until xt_tape_zero_grad
  for (xt_var v : order)
    if (!t->nodes[v].leaf) t->nodes[v].grad_live = false;
  xt_status s = ensure_grad(t, out);
  if (s != XT_OK) return s;
  s = seed(t->nodes[out].grad, grad_live(t, out));
  if (s != XT_OK) return s;
  set_grad_live(t, out);
  auto visit = [&](xt_var v) -> xt_status {
    Node& n = t->nodes[v];
    if (n.leaf || n.view || !n.needs_grad || !grad_live(t, v)) return XT_OK;
    const int np = (int)n.parents.size();
    std::vector<xt_tensor> in_vals(np);
    for (int i = 0; i < np; ++i) in_vals[i] = t->nodes[n.parents[i]].value;
    std::vector<xt_tensor> saved = saved_of(n);
    s = XT_OK;
    const size_t wsb = xt_workspace_bytes(n.op, 1, &n.prm, in_vals.data(), np);
    void* ws = nullptr;
    if (wsb) {
      ws = t->scratch(wsb);
      if (!ws) return XT_ERR_ALLOC;
    }
    // Backward calls: each call serves a set of parent positions whose nodes
    // are pairwise distinct (so no two gradient slots alias); positions are
    // taken in ascending order, so repeated uses of one node push in order.
    std::vector<char> served(np, 0);
    auto wants = [&](int j) {
      return t->nodes[n.parents[j]].needs_grad && !((n.op == XT_OP_CROSS_ENTROPY || n.op == XT_OP_EMBED) && j == 1);
    };
    for (int k = 0; k < np && s == XT_OK; ++k) {
      if (served[k] || !wants(k)) continue;
      std::vector<xt_tensor> din(np);
      for (int i = 0; i < np; ++i) { din[i] = in_vals[i]; din[i].data = nullptr; }
      std::vector<xt_var> used;
      uint32_t accbits = 0;
      for (int j = k; j < np; ++j) {
        if (served[j] || !wants(j)) continue;
        const xt_var q = n.parents[j];
        if (std::find(used.begin(), used.end(), q) != used.end()) continue;
        s = ensure_grad(t, q);
        if (s != XT_OK) break;
        din[j] = t->nodes[q].grad;
        if (grad_live(t, q)) accbits |= 1u << j;
        used.push_back(q);
        served[j] = 1;
      }
      if (s != XT_OK) break;
      s = xt_op_bwd(n.op, &n.prm, &n.grad, in_vals.data(), np, saved.data(), (int)saved.size(),
                    din.data(), np, accbits, ws, wsb, (void*)t->stream);
      if (s != XT_OK) break;
      for (xt_var q : used) set_grad_live(t, q);
    }
    return s;
  };
  // A segment is reached through its output, after every consumer of the
  // output; its other nodes feed only each other and the output, so the
  // whole segment is recomputed and its backward calls run right there,
  // newest node first (recording order is a topological order).
  std::vector<char> seg_done(t->segs.size(), 0);
  for (auto it = order.rbegin(); it != order.rend(); ++it) {
    const xt_var v = *it;
    const int sg = t->nodes[v].seg;
    if (sg < 0) {
      s = visit(v);
      if (s != XT_OK) return s;
      continue;
    }
    if (seg_done[sg]) continue;
    if (v != t->segs[sg].out) return XT_ERR_INVALID_ARG;
    seg_done[sg] = 1;
    bool need = false;
    for (xt_var u = t->segs[sg].first; u <= t->segs[sg].last; ++u)
      need = need || (state[u] == 2 && t->nodes[u].seg == sg && grad_live(t, u) && t->nodes[u].needs_grad);
    if (!need) continue;
    s = recompute(t, sg);
    if (s != XT_OK) return s;
    for (xt_var u = t->segs[sg].last; u >= t->segs[sg].first; --u) {
      if (state[u] != 2 || t->nodes[u].seg != sg) continue;
      s = visit(u);
      if (s != XT_OK) return s;
    }
  }
  return XT_OK;
}
}  // namespace

extern "C" {

xt_status xt_tape_backward(xt_tape* t, xt_var loss) {
  if (!valid_var(t, loss) || t->open_seg >= 0) return XT_ERR_INVALID_ARG;
  const Node& L = t->nodes[loss];
  if (L.value.rows * L.value.cols * L.value.nb[0] * L.value.nb[1] != 1 || L.value.dtype != XT_F32)
    return XT_ERR_SHAPE;
  return reverse_pass(t, loss, [&](const xt_tensor& g, bool live) -> xt_status {
    (void)live;
    return xt::launch_fill_f32((float*)g.data, 1, 1.0f, t->stream) == hipSuccess ? XT_OK : XT_ERR_HIP;
  });
}

xt_status xt_tape_backward_seeded(xt_tape* t, xt_var out, const xt_tensor* dout) {
  if (!valid_var(t, out) || !dout || t->open_seg >= 0) return XT_ERR_INVALID_ARG;
  const Node& n = t->nodes[out];
  if (dout->rows != n.value.rows || dout->cols != n.value.cols || dout->nb[0] != 1 ||
      dout->nb[1] != 1 || n.value.nb[0] != 1 || n.value.nb[1] != 1)
    return XT_ERR_SHAPE;                 // unbatched outputs only
  if (dout->dtype != n.value.dtype || !dout->data) return XT_ERR_DTYPE;
  return reverse_pass(t, out, [&](const xt_tensor& g, bool live) -> xt_status {
    // grad(out) (+)= dout: a leaf keeps accumulating across passes
    xt::EwArgs e{{dout, nullptr, nullptr}, {&g, nullptr}, live && t->nodes[out].leaf ? 1u : 0u, 1.f, nullptr};
    return xt::launch_ew(xt::EW_SCALE, e, t->stream) == hipSuccess ? XT_OK : XT_ERR_HIP;
  });
}

}  // extern "C"
