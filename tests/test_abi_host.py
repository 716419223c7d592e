"""Host-side checks of the C ABI that need no GPU: the library loads, it
exports every function include/xt.h declares, and argument validation
rejects bad calls with the documented status before launching anything."""
import ctypes as C
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "xt.h")
LIB = os.path.join(ROOT, "autograd_row_wise_amd", "libxt.so")

needs_lib = pytest.mark.skipif(not os.path.exists(LIB), reason="libxt.so not built")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = set(re.findall(r"\b(xt_[a-z_0-9]+)\s*\(", text))
    # typedef'd callback types are not functions
    return sorted(n for n in names if not n.endswith("_fn"))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("xt_op_fwd", "xt_op_bwd", "xt_grad_accumulate", "xt_dropout_mask", "xt_workspace_bytes"):
        assert must in names


@needs_lib
def test_library_exports_every_declared_function():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(xt_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    lib = C.CDLL(LIB)
    for n in declared_functions():
        assert getattr(lib, n) is not None


@needs_lib
def test_validation_rejects_without_launch():
    import autograd_row_wise_amd as xt
    import numpy as np

    buf = np.zeros(64, dtype=np.float32)   # host memory: never touched, validation fails first
    def host_view(rows, cols, dtype=xt.DT.F32, ld=None):
        v = xt.Tensor()
        v.data = C.c_void_p(buf.ctypes.data)
        v.dtype = dtype
        v.rows, v.cols, v.ld = rows, cols, cols if ld is None else ld
        v.nb[0] = v.nb[1] = 1
        return v
    x = host_view(2, 4)
    # dropout p outside [0, 1)
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.DROPOUT, xt.params(p=1.0), [x], [host_view(2, 4)], stream=C.c_void_p(0))
    assert e.value.status == 1 and "p must be in [0, 1)" in str(e.value)
    # ld < cols
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.SILU, xt.params(), [host_view(2, 4, ld=3)], [host_view(2, 4)], stream=C.c_void_p(0))
    assert e.value.status == 2
    # a view whose extent wraps 64-bit element offsets, and a negative batch stride
    for big in (host_view(1 << 40, 1 << 40), host_view(2, 4, ld=(1 << 62))):
        with pytest.raises(xt.XtError) as e:
            xt.xt_op_fwd(xt.OP.SILU, xt.params(), [big], [host_view(2, 4)], stream=C.c_void_p(0))
        assert e.value.status == 2 and "extent" in str(e.value)
    neg = host_view(2, 4)
    neg.sb[0] = -8
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.SILU, xt.params(), [neg], [host_view(2, 4)], stream=C.c_void_p(0))
    assert e.value.status == 2 and "negative batch stride" in str(e.value)
    # shape mismatch
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.ADD, xt.params(), [x, host_view(2, 3)], [host_view(2, 4)], stream=C.c_void_p(0))
    assert e.value.status == 2
    # odd rope head_dim
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.ROPE, xt.params(head_dim=3, seq_len=4), [host_view(2, 6)], [host_view(2, 6)],
                     stream=C.c_void_p(0))
    assert e.value.status == 1
    # int32 activations are not supported
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.SILU, xt.params(), [host_view(2, 4, xt.DT.I32)], [host_view(2, 4)], stream=C.c_void_p(0))
    assert e.value.status == 3
    # GELU form flag outside {0, 1}
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.GELU, xt.params(gelu_tanh=2), [x], [host_view(2, 4)], stream=C.c_void_p(0))
    assert e.value.status == 1 and "gelu_tanh" in str(e.value)
    # wrong tensor counts
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.RMS_NORM, xt.params(), [x], [host_view(2, 4)], stream=C.c_void_p(0))
    assert e.value.status == 1
    # matmul inner dimensions
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_fwd(xt.OP.MATMUL, xt.params(), [host_view(2, 4), host_view(3, 2)], [host_view(2, 2)],
                     stream=C.c_void_p(0))
    assert e.value.status == 2
    # rms_norm backward without its workspace
    with pytest.raises(xt.XtError) as e:
        xt.xt_op_bwd(xt.OP.RMS_NORM, xt.params(), host_view(2, 4), [x, host_view(1, 4)],
                     [host_view(2, 1)], [host_view(2, 4), host_view(1, 4)], 0, None, 0, stream=C.c_void_p(0))
    assert e.value.status == 5
    assert xt.xt_status_str(5) == "workspace too small"
    assert xt.xt_abi_version() == 1


@needs_lib
def test_grad_buffer_validation_without_launch():
    import autograd_row_wise_amd as xt
    import numpy as np

    buf = np.zeros(64, dtype=np.float32)
    def host_view(rows, cols, dtype=xt.DT.F32, nb=1):
        v = xt.Tensor()
        v.data = C.c_void_p(buf.ctypes.data)
        v.dtype = dtype
        v.rows, v.cols, v.ld = rows, cols, cols
        v.nb[0], v.nb[1] = nb, 1
        return v
    g = [host_view(2, 4), host_view(1, 3, xt.DT.BF16)]
    # two units of 8192 elements at most -> 8 bytes each
    assert xt.xt_grad_norm_workspace(g) == 2 * 8
    assert xt.xt_grad_norm_workspace([host_view(3, 8192 * 2 + 1)]) == 7 * 8   # contiguous: one row of 49155
    with pytest.raises(xt.XtError) as e:            # no workspace
        xt.xt_grad_norm(g, 1.0, buf.ctypes.data, None, 0, stream=C.c_void_p(0))
    assert e.value.status == 5
    with pytest.raises(xt.XtError) as e:            # negative threshold
        xt.xt_grad_norm(g, -1.0, buf.ctypes.data, buf.ctypes.data, 256, stream=C.c_void_p(0))
    assert e.value.status == 1
    with pytest.raises(xt.XtError) as e:            # null output
        xt.xt_grad_norm(g, 1.0, None, buf.ctypes.data, 256, stream=C.c_void_p(0))
    assert e.value.status == 1
    with pytest.raises(xt.XtError) as e:            # u8 is not a gradient dtype
        xt.xt_grads_scale([host_view(2, 4, xt.DT.U8)], 0.5, stream=C.c_void_p(0))
    assert e.value.status == 3
    with pytest.raises(xt.XtError) as e:            # batched views are rejected
        xt.xt_grads_zero([host_view(2, 4, nb=2)], stream=C.c_void_p(0))
    assert e.value.status == 2
    assert xt.xt_grad_norm_workspace([host_view(2, 4, xt.DT.U8)]) == 0


@needs_lib
def test_workspace_query_is_host_only():
    import autograd_row_wise_amd as xt
    def shape(rows, cols, dtype=xt.DT.F32):
        v = xt.Tensor()
        v.dtype, v.rows, v.cols, v.ld = dtype, rows, cols, cols
        v.nb[0] = v.nb[1] = 1
        return v
    assert xt.xt_workspace_bytes(xt.OP.SILU, 1, xt.params(), [shape(8, 64)]) == 0
    assert xt.xt_workspace_bytes(xt.OP.RMS_NORM, 0, xt.params(), [shape(8, 64)]) == 0
    assert xt.xt_workspace_bytes(xt.OP.RMS_NORM, 1, xt.params(), [shape(8, 64)]) == 8 * 64 * 4
    # partial-gradient workspaces are whole partial rows (np vectors of C
    # floats), at most one per block and never more blocks than rows
    for op, np_, R, C, dt in [(xt.OP.LAYER_NORM, 2, 8192, 768, xt.DT.F32), (xt.OP.RMS_NORM, 1, 16384, 4096, xt.DT.BF16),
                              (xt.OP.RMS_NORM, 1, 1024, 256, xt.DT.F32), (xt.OP.LAYER_NORM, 2, 5, 3001, xt.DT.BF16)]:
        w = xt.xt_workspace_bytes(op, 1, xt.params(), [shape(R, C, dt)])
        row = np_ * C * 4
        assert w > 0 and w % row == 0 and w // row <= min(R, 512), (op, R, C, w)
    w = xt.xt_workspace_bytes(xt.OP.ADD_BIAS, 1, xt.params(), [shape(65536, 4096, xt.DT.BF16)])
    assert w > 0 and w % (4096 * 4) == 0


@needs_lib
def test_matmul_split_workspace_query():
    """Weight-gradient shapes (few output tiles, long K) ask for split-K
    workspace: whole f32 slices of the output, between 2 and 16 of them;
    shapes with many tiles ask for none."""
    import autograd_row_wise_amd as xt
    def shape(rows, cols, dtype=xt.DT.F32):
        v = xt.Tensor()
        v.dtype, v.rows, v.cols, v.ld = dtype, rows, cols, cols
        v.nb[0] = v.nb[1] = 1
        return v
    prm = xt.params()
    # x[8192, 768] @ W[768, 3072]: dW = x^T d is 768 x 3072 summed over 8192 rows
    w = xt.xt_workspace_bytes(xt.OP.MATMUL, 1, prm, [shape(8192, 768), shape(768, 3072)])
    slice_ = 768 * 3072 * 4
    assert w % slice_ == 0 or w % (8192 * 768 * 4) == 0
    assert 2 * min(slice_, 8192 * 768 * 4) <= w <= 16 * 8192 * 768 * 4
    # 8192 x 4096 x 4096 bf16 has 256 or more 256 x 256 tiles everywhere: no split
    assert xt.xt_workspace_bytes(xt.OP.MATMUL, 1, prm, [shape(8192, 4096, xt.DT.BF16), shape(4096, 4096, xt.DT.BF16)]) == 0
    assert xt.xt_workspace_bytes(xt.OP.MATMUL, 0, prm, [shape(8192, 4096, xt.DT.BF16), shape(4096, 4096, xt.DT.BF16)]) == 0
