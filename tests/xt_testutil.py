"""Helpers shared by the GPU parity tests: moving seeded inputs to the device,
calling the C ABI through the binding, and the comparison rules.

Comparison rules (written out so a reader can check them against the tests):
  f32 : |gpu - ref| <= 1e-6 + 1e-5 * |ref| per element.  For outputs that are
        signed sums of n >= 64 terms (matmul entries, column sums), |ref| is
        replaced by max(|ref|, A/sqrt(n)) with A = sum of |terms| (computed by
        the oracle side): near a zero crossing of a long sum the literal bar is
        below f32 resolution.
  bf16: |gpu - ref| <= 2e-2 * |ref| + 1e-2 * rms(ref) per element (a pure
        relative bound is undefined at 0, hence the floor).
  f32 through a composed graph (gradients that pass through tens of ops on
        the tape, where no per-element term magnitude is at hand):
        |gpu - ref| <= 1e-6 + 1e-5 * (|ref| + rms(ref)) per element, the f32
        rule with the bf16 rule's kind of floor; the share of elements that
        also meet the literal 1e-6 + 1e-5 * |ref| is printed beside it.
  masks, int32 indexing: bit-exact.
"""
from __future__ import annotations

import numpy as np
import torch

import autograd_row_wise_amd as xt
from synth import bf16_bits_to_f32


def dev(a: np.ndarray, dtype: str = "f32") -> torch.Tensor:
    """Host array (f32 values, or bf16 bit patterns as uint16) -> device tensor."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 numpy (bf16 widened exactly)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        bits = t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
        return bf16_bits_to_f32(bits).astype(np.float64)
    if t.dtype in (torch.uint8, torch.int32, torch.int64):
        return t.cpu().numpy()
    return t.float().cpu().numpy().astype(np.float64)


def empty(shape, dtype: str) -> torch.Tensor:
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "u8": torch.uint8, "i32": torch.int32}[dtype]
    return torch.empty(shape, dtype=tdt, device="cuda")


def fwd(op, prm, ins, outs):
    xt.xt_op_fwd(op, prm, [xt.view(t) for t in ins], [xt.view(t) for t in outs])


def bwd(op, prm, dout, ins, saved, din, acc=0):
    """din: list of torch tensors or None (not wanted)."""
    iv = [xt.view(t) for t in ins]
    dv = []
    for k, t in enumerate(din):
        if t is None:
            v = xt.view(ins[k]) if k < len(ins) else xt.Tensor()
            v.data = None
            dv.append(v)
        else:
            dv.append(xt.view(t))
    w, wp, wb = xt.workspace(op, 1, prm, iv)
    xt.xt_op_bwd(op, prm, xt.view(dout), iv, [xt.view(t) for t in saved], dv, acc, wp, wb)
    torch.cuda.synchronize()
    del w


def close_f32(gpu, ref, scale=None, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    mag = np.abs(ref) if scale is None else np.maximum(np.abs(ref), scale)
    bad = np.abs(gpu - ref) > 1e-6 + 1e-5 * mag
    if scale is not None:
        print(f"[f32 sum] {what}: literal 1e-5/1e-6 bar met by {100 * literal_rate(gpu, ref):.3f}% of {ref.size}")
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} f32 elements off; first at {tuple(i)}: "
                             f"gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r}")


def close_bf16(gpu, ref, what=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    bad = np.abs(gpu - ref) > 2e-2 * np.abs(ref) + 1e-2 * rms
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} bf16 elements off; first at {tuple(i)}: "
                             f"gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r}")


def literal_rate(gpu, ref) -> float:
    """Share of elements within the literal f32 bar 1e-6 + 1e-5 * |ref|."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if ref.size == 0:
        return 1.0
    return float(np.mean(np.abs(gpu - ref) <= 1e-6 + 1e-5 * np.abs(ref)))


def close_chain_f32(gpu, ref, what=""):
    """Per-element f32 bar for outputs of a composed graph (see the module
    docstring); prints the literal-bar pass rate beside it."""
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (what, gpu.shape, ref.shape)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(gpu - ref)
    bad = err > 1e-6 + 1e-5 * (np.abs(ref) + rms)
    print(f"[f32 chain] {what}: literal 1e-5/1e-6 bar met by {100 * literal_rate(gpu, ref):.3f}% of {ref.size}; "
          f"max |err|/rms {float(err.max() / rms) if ref.size and rms > 0 else 0.0:.2e}")
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} f32 elements off; first at {tuple(i)}: "
                             f"gpu={gpu[tuple(i)]!r} ref={ref[tuple(i)]!r} rms={rms!r}")


def close(gpu, ref, dtype: str, scale=None, what=""):
    if dtype == "f32":
        close_f32(gpu, ref, scale, what)
    else:
        close_bf16(gpu, ref, what)


def sum_scale(terms_abs_sum: np.ndarray, n: int) -> np.ndarray:
    """max(|ref|, A/sqrt(n)) helper: the A/sqrt(n) part."""
    return np.asarray(terms_abs_sum, dtype=np.float64) / np.sqrt(max(n, 1))
