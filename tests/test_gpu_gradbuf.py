"""GPU parity of the gradient-buffer helpers (global norm and clipping
coefficient, in-place scaling, zeroing) through the C ABI against the
oracle: f32 and bf16 lists, ragged sizes, strided views (whose gap columns
must stay untouched), more tensors than one launch takes, empty tensors and
lists, and the full gradient set of a 12-layer GPT-2-small-sized model."""
import numpy as np
import pytest

from oracle import ops
from oracle.numerics import round_bf16
import synth

pytestmark = pytest.mark.gpu

if True:  # GPU-only imports are deferred so CPU collection never loads libxt
    try:
        import torch
        import autograd_row_wise_amd as xt
        from xt_testutil import dev, host
    except Exception:  # pragma: no cover - CPU host without the library
        pass

# (rows, cols, ld or None, dtype)
SHAPES = [(1, 1, None, "f32"), (7, 13, None, "f32"), (300, 1001, None, "f32"), (4096, 1027, None, "bf16"),
          (33, 500, 512, "f32"), (17, 999, 1008, "bf16"), (1, 8193, None, "bf16"), (2, 16385, None, "f32"),
          (0, 5, None, "f32"), (64, 64, 72, "f32")]
SENTINEL = 12345.0


def make(shapes, seed):
    """Device tensors (possibly narrow views of wider rows whose gap columns
    hold a sentinel) and the f64 values of each view."""
    views, vals, bases = [], [], []
    for k, (R, C, ld, dt) in enumerate(shapes):
        a = synth.host_normal((R, C), seed, 100 + k, 0.0, 1.0 + k % 3, "f32")
        bits = synth.host_bf16_bits(a) if dt == "bf16" else a
        v = synth.bf16_bits_to_f32(bits).astype(np.float64) if dt == "bf16" else a.astype(np.float64)
        if ld is None:
            t = dev(bits, dt)
            views.append(t)
            bases.append(None)
        else:
            full = np.full((R, ld), SENTINEL, dtype=np.float32)
            fb = synth.host_bf16_bits(full) if dt == "bf16" else full
            fb[:, :C] = bits
            base = dev(fb, dt)
            views.append(base[:, :C])
            bases.append((base, C))
        vals.append(v)
    return views, vals, bases


def xviews(ts):
    return [xt.view(t) for t in ts]


def run_norm(ts, max_norm):
    vs = xviews(ts)
    nbytes = xt.xt_grad_norm_workspace(vs)
    ws = torch.empty(max(nbytes, 8), dtype=torch.uint8, device="cuda")
    out = torch.full((2,), float("nan"), dtype=torch.float32, device="cuda")
    xt.xt_grad_norm(vs, max_norm, out.data_ptr(), ws.data_ptr(), nbytes)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def gaps_untouched(bases):
    for b in bases:
        if b is None:
            continue
        base, C = b
        gap = host(base)[:, C:]
        want = float(round_bf16(np.array([SENTINEL]))[0]) if base.dtype == torch.bfloat16 else SENTINEL
        assert np.all(gap == want)


@pytest.mark.parametrize("max_norm", [0.0, 1.0, 1e9])
def test_grad_norm_and_coefficient(max_norm):
    ts, vals, bases = make(SHAPES, 1)
    out = run_norm(ts, max_norm)
    ref = ops.grad_norm(vals)
    assert abs(out[0] - ref) <= 2e-7 * ref
    coef = ops.clip_coefficient(ref, max_norm)
    assert abs(out[1] - coef) <= 2e-7 * coef
    # bitwise reproducible
    again = run_norm(ts, max_norm)
    assert np.array_equal(out, again)
    gaps_untouched(bases)


def test_grad_norm_many_tensors_and_empty():
    shapes = [(1 + (k * 7) % 23, 1 + (k * 131) % 3000, None, "f32" if k % 3 else "bf16") for k in range(70)]
    ts, vals, _ = make(shapes, 2)
    out = run_norm(ts, 0.0)
    ref = ops.grad_norm(vals)
    assert abs(out[0] - ref) <= 2e-7 * ref and out[1] == 1.0
    assert np.array_equal(run_norm([], 1.0), [0.0, 1.0])
    e, _, _ = make([(0, 9, None, "f32"), (3, 0, None, "bf16")], 3)
    assert np.array_equal(run_norm(e, 1.0), [0.0, 1.0])


@pytest.mark.parametrize("factor", [0.3, 0.125, 1.0 / 3.0])
def test_grads_scale_device_factor_bit_exact(factor):
    ts, vals, bases = make(SHAPES, 4)
    s = torch.tensor([factor], dtype=torch.float32, device="cuda")
    xt.xt_grads_scale(xviews(ts), 1.0, s.data_ptr())
    torch.cuda.synchronize()
    for t, v, (R, C, ld, dt) in zip(ts, vals, SHAPES):
        assert np.array_equal(host(t), ops.scale_grad(v, np.float32(factor), dt)), (R, C, ld, dt)
    gaps_untouched(bases)


def test_grads_scale_alpha_and_zero():
    ts, vals, bases = make(SHAPES, 5)
    alpha = np.float32(1.0 / 4.0 * 0.9)
    xt.xt_grads_scale(xviews(ts), float(alpha))
    torch.cuda.synchronize()
    for t, v, (R, C, ld, dt) in zip(ts, vals, SHAPES):
        assert np.array_equal(host(t), ops.scale_grad(v, alpha, dt))
    xt.xt_grads_zero(xviews(ts))
    torch.cuda.synchronize()
    for t in ts:
        assert np.all(host(t) == 0.0)
    gaps_untouched(bases)


def test_clip_pipeline_on_device():
    """norm -> coefficient -> scale by the device coefficient: afterwards the
    global norm is the threshold, and each element is the oracle's scaling
    of the stored value (f32 factors may differ from the oracle's by the
    last bit of the norm, hence one f32 rounding step of tolerance)."""
    ts, vals, _ = make(SHAPES[:8], 6)
    ref = ops.grad_norm(vals)
    max_norm = ref / 7.0
    out_t = torch.empty(2, dtype=torch.float32, device="cuda")
    vs = xviews(ts)
    nbytes = xt.xt_grad_norm_workspace(vs)
    ws = torch.empty(max(nbytes, 8), dtype=torch.uint8, device="cuda")
    xt.xt_grad_norm(vs, max_norm, out_t.data_ptr(), ws.data_ptr(), nbytes)
    xt.xt_grads_scale(vs, 1.0, out_t.data_ptr() + 4)
    torch.cuda.synchronize()
    coef = ops.clip_coefficient(ref, max_norm)
    for t, v, (R, C, ld, dt) in zip(ts, vals, SHAPES[:8]):
        want = ops.scale_grad(v, coef, dt)
        tol = (2.0 ** -7 if dt == "bf16" else 2.0 ** -22) * np.abs(want)
        assert np.all(np.abs(host(t) - want) <= tol)
    after = run_norm(ts, 0.0)[0]
    assert abs(after - max_norm) <= 1e-3 * max_norm


def test_full_model_gradient_set():
    """Every gradient buffer of a 12-layer model of GPT-2-small width
    (d = 768, MLP 3072, vocabulary 50257, 1024 positions; about 124M f32),
    drawn on the device; the oracle reads the same inputs back."""
    shapes = []
    for _ in range(12):
        shapes += [(768, 768)] * 4 + [(768, 3072), (3072, 768)] + [(1, 768)] * 4
    shapes += [(50257, 768), (1024, 768), (1, 768), (1, 768)]
    ts = [synth.device_normal(s, 7, 200 + k, 0.0, 1e-3 * (1 + k % 5)) for k, s in enumerate(shapes)]
    out = run_norm(ts, 1.0)
    ref = ops.grad_norm([host(t) for t in ts])
    assert abs(out[0] - ref) <= 2e-7 * ref
    assert abs(out[1] - ops.clip_coefficient(ref, 1.0)) <= 2e-7
