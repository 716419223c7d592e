"""Python binding of libxt (the C ABI declared in include/xt.h).

Argument marshalling only: every step of every op runs in libxt's HIP
kernels.  PyTorch supplies device memory and the current stream.  The module
refuses to import without a built libxt.so -- there is no fallback path.

The C entry points keep their names (xt_op_fwd, xt_op_bwd,
xt_grad_accumulate, xt_dropout_mask, xt_workspace_bytes, xt_tape_*); a
nonzero status raises XtError carrying xt_last_error().
"""
from __future__ import annotations

import ctypes as C
import os

__all__ = [
    "XtError", "Tensor", "Params", "OP", "DT", "lib", "view", "params",
    "xt_op_fwd", "xt_op_bwd", "xt_op_bwd_noalloc", "xt_grad_accumulate", "xt_dropout_mask", "xt_workspace_bytes",
    "xt_status_str", "xt_last_error", "xt_abi_version", "Tape", "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libxt.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built: run `python autograd_row_wise_amd/build.py` "
        "(or __graft_entry__.build()); there is no non-HIP fallback")

# torch loads the HIP runtime its device memory and streams come from; libxt
# must bind to that same runtime, so torch is loaded first.  (Loaded the other
# way round, the process holds two HIP runtimes and libxt's launches find no
# device.)
import torch  # noqa: E402,F401

lib = C.CDLL(LIB_PATH)


class DT:
    F32, BF16, I32, U8 = 0, 1, 2, 3


class OP:
    MATMUL, ADD, MUL, SCALE, ADD_BIAS, RMS_NORM, LAYER_NORM, SOFTMAX, CROSS_ENTROPY, \
        SILU, SWIGLU, GELU, ROPE, DROPOUT, EMBED, ATTENTION = range(16)


class Tensor(C.Structure):
    _fields_ = [("data", C.c_void_p), ("dtype", C.c_int32), ("reserved", C.c_int32),
                ("rows", C.c_int64), ("cols", C.c_int64), ("ld", C.c_int64),
                ("nb", C.c_int64 * 2), ("sb", C.c_int64 * 2)]


class Params(C.Structure):
    _fields_ = [("eps", C.c_float), ("alpha", C.c_float), ("causal", C.c_int32),
                ("seq_len", C.c_int32), ("head_dim", C.c_int32), ("rope_base", C.c_float),
                ("p", C.c_float), ("gelu_tanh", C.c_int32), ("seed", C.c_uint64),
                ("trans_a", C.c_int32), ("trans_b", C.c_int32)]


class XtError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {xt_status_str(status)} ({status}): {xt_last_error()}")


_ALLOC = C.CFUNCTYPE(C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p)
_FREE = C.CFUNCTYPE(None, C.c_void_p, C.c_void_p, C.c_void_p)
_TP = C.POINTER(Tensor)

lib.xt_status_str.restype = C.c_char_p
lib.xt_status_str.argtypes = [C.c_int]
lib.xt_last_error.restype = C.c_char_p
lib.xt_abi_version.restype = C.c_int
lib.xt_workspace_bytes.restype = C.c_size_t
lib.xt_workspace_bytes.argtypes = [C.c_int, C.c_int, C.POINTER(Params), _TP, C.c_int]
lib.xt_op_fwd.restype = C.c_int
lib.xt_op_fwd.argtypes = [C.c_int, C.POINTER(Params), _TP, C.c_int, _TP, C.c_int,
                          C.c_void_p, C.c_size_t, C.c_void_p]
lib.xt_op_bwd.restype = C.c_int
lib.xt_op_bwd.argtypes = [C.c_int, C.POINTER(Params), _TP, _TP, C.c_int, _TP, C.c_int,
                          _TP, C.c_int, C.c_uint32, C.c_void_p, C.c_size_t, C.c_void_p]
lib.xt_op_bwd_noalloc.restype = C.c_int
lib.xt_op_bwd_noalloc.argtypes = [C.c_int, C.POINTER(Params), _TP, _TP, C.c_int, _TP, C.c_int,
                                  _TP, C.c_int, C.c_uint32, C.c_void_p]
lib.xt_grad_accumulate.restype = C.c_int
lib.xt_grad_accumulate.argtypes = [_TP, _TP, C.c_void_p]
lib.xt_dropout_mask.restype = C.c_int
lib.xt_dropout_mask.argtypes = [_TP, C.c_float, C.c_uint64, C.c_void_p]
lib.xt_grad_norm_workspace.restype = C.c_size_t
lib.xt_grad_norm_workspace.argtypes = [_TP, C.c_int32]
lib.xt_grad_norm.restype = C.c_int
lib.xt_grad_norm.argtypes = [_TP, C.c_int32, C.c_float, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
lib.xt_grads_scale.restype = C.c_int
lib.xt_grads_scale.argtypes = [_TP, C.c_int32, C.c_float, C.c_void_p, C.c_void_p]
lib.xt_grads_zero.restype = C.c_int
lib.xt_grads_zero.argtypes = [_TP, C.c_int32, C.c_void_p]
lib.xt_tape_create.restype = C.c_void_p
lib.xt_tape_create.argtypes = [_ALLOC, _FREE, C.c_void_p, C.c_void_p]
lib.xt_tape_destroy.argtypes = [C.c_void_p]
lib.xt_tape_leaf.restype = C.c_int64
lib.xt_tape_leaf.argtypes = [C.c_void_p, _TP, C.c_int]
lib.xt_tape_apply.restype = C.c_int64
lib.xt_tape_apply.argtypes = [C.c_void_p, C.c_int, C.POINTER(Params), C.POINTER(C.c_int64), C.c_int]
lib.xt_tape_apply_layout.restype = C.c_int64
lib.xt_tape_apply_layout.argtypes = [C.c_void_p, C.c_int, C.POINTER(Params), C.POINTER(C.c_int64),
                                     C.c_int, _TP]
lib.xt_tape_view.restype = C.c_int64
lib.xt_tape_view.argtypes = [C.c_void_p, C.c_int64, _TP]
for _n in ("xt_tape_value", "xt_tape_grad"):
    getattr(lib, _n).restype = C.c_int
    getattr(lib, _n).argtypes = [C.c_void_p, C.c_int64, _TP]
lib.xt_tape_saved.restype = C.c_int
lib.xt_tape_saved.argtypes = [C.c_void_p, C.c_int64, C.c_int, _TP]
lib.xt_tape_backward.restype = C.c_int
lib.xt_tape_backward.argtypes = [C.c_void_p, C.c_int64]
lib.xt_tape_backward_seeded.restype = C.c_int
lib.xt_tape_backward_seeded.argtypes = [C.c_void_p, C.c_int64, _TP]
lib.xt_tape_zero_grad.restype = C.c_int
lib.xt_tape_zero_grad.argtypes = [C.c_void_p]
lib.xt_tape_checkpoint_begin.restype = C.c_int
lib.xt_tape_checkpoint_begin.argtypes = [C.c_void_p]
lib.xt_tape_checkpoint_end.restype = C.c_int
lib.xt_tape_checkpoint_end.argtypes = [C.c_void_p, C.c_int64]
lib.xt_tape_num_nodes.restype = C.c_int64
lib.xt_tape_num_nodes.argtypes = [C.c_void_p]


def xt_status_str(s: int) -> str:
    return lib.xt_status_str(s).decode()


def xt_last_error() -> str:
    return lib.xt_last_error().decode()


def xt_abi_version() -> int:
    return lib.xt_abi_version()


def _check(s: int, where: str) -> None:
    if s != 0:
        raise XtError(s, where)


# ----------------------------------------------------------------- marshalling
def _torch_dt(t) -> int:
    import torch
    m = {torch.float32: DT.F32, torch.bfloat16: DT.BF16, torch.int32: DT.I32, torch.uint8: DT.U8}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def view(t, rows=None, cols=None, ld=None, nb=(1, 1), sb=(0, 0), offset=0) -> Tensor:
    """xt_tensor over a torch tensor's storage (no copy).  A 2-D tensor maps to
    [rows, cols] with ld = its row stride; 1-D maps to [1, n]; pass explicit
    rows/cols/ld/nb/sb for batched or strided layouts (strides in elements)."""
    v = Tensor()
    if t is None:
        v.data = None
        return v
    v.data = C.c_void_p(t.data_ptr() + offset * t.element_size())
    v.dtype = _torch_dt(t)
    if rows is None:
        if t.dim() == 2:
            rows, cols = t.shape
            if t.numel() == 0:          # an empty tensor's strides carry no layout
                ld = cols if ld is None else ld
            else:
                ld = t.stride(0) if ld is None else ld
                if t.stride(1) != 1:
                    raise ValueError("columns must be contiguous")
        elif t.dim() == 1:
            rows, cols = 1, t.shape[0]
            ld = cols if ld is None else ld
        elif t.dim() == 0:
            rows, cols, ld = 1, 1, 1
        else:
            raise ValueError("pass rows/cols/ld for tensors of rank > 2")
    v.rows, v.cols = int(rows), int(cols)
    v.ld = int(cols if ld is None else ld)
    v.nb[0], v.nb[1] = int(nb[0]), int(nb[1])
    v.sb[0], v.sb[1] = int(sb[0]), int(sb[1])
    return v


def empty_view(t) -> Tensor:
    """A gradient slot that is not wanted (data = NULL) with t's shape."""
    v = view(t)
    v.data = None
    return v


def params(eps=1e-5, alpha=1.0, causal=0, seq_len=0, head_dim=0, rope_base=10000.0, p=0.0,
           seed=0, trans_a=0, trans_b=0, gelu_tanh=0) -> Params:
    return Params(eps, alpha, int(causal), int(seq_len), int(head_dim), rope_base, p, int(gelu_tanh),
                  int(seed) & 0xFFFFFFFFFFFFFFFF, int(trans_a), int(trans_b))


def _arr(views):
    n = len(views)
    a = (Tensor * max(n, 1))()
    for i, v in enumerate(views):
        a[i] = v
    return a, n


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def xt_workspace_bytes(op: int, is_bwd: int, prm: Params, ins) -> int:
    a, n = _arr(ins)
    return lib.xt_workspace_bytes(op, is_bwd, C.byref(prm), a, n)


def xt_op_fwd(op: int, prm: Params, ins, outs, ws=None, ws_bytes=0, stream=None) -> None:
    a, n = _arr(ins)
    b, m = _arr(outs)
    _check(lib.xt_op_fwd(op, C.byref(prm), a, n, b, m, ws, ws_bytes, _stream(stream)), "xt_op_fwd")


def xt_op_bwd(op: int, prm: Params, dout: Tensor, ins, saved, din, accumulate=0, ws=None,
              ws_bytes=0, stream=None) -> None:
    a, n = _arr(ins)
    s, ns = _arr(saved)
    d, nd = _arr(din)
    _check(lib.xt_op_bwd(op, C.byref(prm), C.byref(dout), a, n, s, ns, d, nd, accumulate, ws,
                         ws_bytes, _stream(stream)), "xt_op_bwd")


def xt_op_bwd_noalloc(op: int, prm: Params, dout: Tensor, ins, saved, din, accumulate=0, stream=None) -> None:
    a, n = _arr(ins)
    s, ns = _arr(saved)
    d, nd = _arr(din)
    _check(lib.xt_op_bwd_noalloc(op, C.byref(prm), C.byref(dout), a, n, s, ns, d, nd, accumulate,
                                 _stream(stream)), "xt_op_bwd_noalloc")


def xt_grad_accumulate(dst: Tensor, src: Tensor, stream=None) -> None:
    _check(lib.xt_grad_accumulate(C.byref(dst), C.byref(src), _stream(stream)), "xt_grad_accumulate")


def xt_dropout_mask(mask: Tensor, p: float, seed: int, stream=None) -> None:
    _check(lib.xt_dropout_mask(C.byref(mask), p, int(seed) & 0xFFFFFFFFFFFFFFFF, _stream(stream)),
           "xt_dropout_mask")


def xt_grad_norm_workspace(grads) -> int:
    a, n = _arr(grads)
    return lib.xt_grad_norm_workspace(a, n)


def xt_grad_norm(grads, max_norm: float, out, ws=None, ws_bytes=0, stream=None) -> None:
    """out: device pointer (int or c_void_p) of two f32: the norm and the clipping coefficient."""
    a, n = _arr(grads)
    _check(lib.xt_grad_norm(a, n, max_norm, out, ws, ws_bytes, _stream(stream)), "xt_grad_norm")


def xt_grads_scale(grads, alpha: float = 1.0, scale=None, stream=None) -> None:
    a, n = _arr(grads)
    _check(lib.xt_grads_scale(a, n, alpha, scale, _stream(stream)), "xt_grads_scale")


def xt_grads_zero(grads, stream=None) -> None:
    a, n = _arr(grads)
    _check(lib.xt_grads_zero(a, n, _stream(stream)), "xt_grads_zero")


def workspace(op: int, is_bwd: int, prm: Params, ins):
    """Allocate (torch) the workspace an op call needs; returns (tensor|None, ptr, bytes)."""
    nbytes = xt_workspace_bytes(op, is_bwd, prm, ins)
    if nbytes == 0:
        return None, None, 0
    import torch
    w = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    return w, C.c_void_p(w.data_ptr()), nbytes


# ------------------------------------------------------------------------ tape
class Tape:
    """xt_tape_* with torch's caching allocator supplying device memory."""

    def __init__(self, stream=None):
        import torch
        self._torch = torch
        self._dev = torch.cuda.current_device()

        def _alloc(ctx, nbytes, strm):
            try:
                return torch.cuda.caching_allocator_alloc(int(nbytes), self._dev, strm)
            except Exception:
                return None

        def _free(ctx, ptr, strm):
            torch.cuda.caching_allocator_delete(ptr)

        self._cb = (_ALLOC(_alloc), _FREE(_free))
        s = _stream(stream)
        self.stream = s
        self.h = lib.xt_tape_create(self._cb[0], self._cb[1], None, s)
        if not self.h:
            raise XtError(7, "xt_tape_create")

    def close(self):
        if self.h:
            lib.xt_tape_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _var(v: int, where: str) -> int:
        if v < 0:
            raise XtError(-v, where)
        return v

    def leaf(self, v: Tensor, requires_grad: bool = True) -> int:
        return self._var(lib.xt_tape_leaf(self.h, C.byref(v), int(requires_grad)), "xt_tape_leaf")

    def apply(self, op: int, prm: Params, *parents, layout: Tensor | None = None) -> int:
        arr = (C.c_int64 * len(parents))(*parents)
        if layout is None:
            r = lib.xt_tape_apply(self.h, op, C.byref(prm), arr, len(parents))
        else:
            r = lib.xt_tape_apply_layout(self.h, op, C.byref(prm), arr, len(parents), C.byref(layout))
        return self._var(r, "xt_tape_apply")

    def checkpoint_begin(self) -> None:
        _check(lib.xt_tape_checkpoint_begin(self.h), "xt_tape_checkpoint_begin")

    def checkpoint_end(self, out: int) -> int:
        _check(lib.xt_tape_checkpoint_end(self.h, out), "xt_tape_checkpoint_end")
        return out

    def view(self, parent: int, layout: Tensor) -> int:
        return self._var(lib.xt_tape_view(self.h, parent, C.byref(layout)), "xt_tape_view")

    def value(self, v: int) -> Tensor:
        out = Tensor()
        _check(lib.xt_tape_value(self.h, v, C.byref(out)), "xt_tape_value")
        return out

    def saved(self, v: int, k: int) -> Tensor:
        out = Tensor()
        _check(lib.xt_tape_saved(self.h, v, k, C.byref(out)), "xt_tape_saved")
        return out

    def grad(self, v: int) -> Tensor:
        out = Tensor()
        _check(lib.xt_tape_grad(self.h, v, C.byref(out)), "xt_tape_grad")
        return out

    def backward(self, loss: int) -> None:
        _check(lib.xt_tape_backward(self.h, loss), "xt_tape_backward")

    def backward_seeded(self, out: int, dout: Tensor) -> None:
        _check(lib.xt_tape_backward_seeded(self.h, out, C.byref(dout)), "xt_tape_backward_seeded")

    def zero_grad(self) -> None:
        _check(lib.xt_tape_zero_grad(self.h), "xt_tape_zero_grad")

    def num_nodes(self) -> int:
        return lib.xt_tape_num_nodes(self.h)


def to_torch(v: Tensor, like=None):
    """Copy the dense [rows, cols] (or batched [nb0, nb1, rows, cols]) content of
    a view into a new torch tensor (uses torch's as_strided on the storage)."""
    import torch
    if not v.data:
        return None
    tdt = {DT.F32: torch.float32, DT.BF16: torch.bfloat16, DT.I32: torch.int32, DT.U8: torch.uint8}[v.dtype]
    es = torch.tensor([], dtype=tdt).element_size()
    span = 0
    if v.rows and v.cols:
        span = (v.nb[0] - 1) * v.sb[0] + (v.nb[1] - 1) * v.sb[1] + (v.rows - 1) * v.ld + v.cols
    # wrap raw memory through a UntypedStorage view
    from torch.cuda import caching_allocator_alloc  # noqa: F401  (ensures CUDA init)
    buf = _raw_cuda_tensor(v.data, span * es)
    base = buf.view(tdt)
    out = base.as_strided((v.nb[0], v.nb[1], v.rows, v.cols), (v.sb[0], v.sb[1], v.ld, 1)).clone()
    if v.nb[0] == 1 and v.nb[1] == 1:
        out = out[0, 0]
    return out


def _raw_cuda_tensor(ptr: int, nbytes: int):
    """A uint8 torch view of nbytes of device memory at ptr (not owned)."""
    import torch

    class _CAI:
        pass

    cai = _CAI()
    cai.__cuda_array_interface__ = {"shape": (int(nbytes),), "typestr": "|u1",
                                    "data": (int(ptr), False), "version": 2, "strides": None}
    return torch.as_tensor(cai, device="cuda")
