"""Shared helpers of the GPU parity tests: device copies, guarded output
buffers, and the acceptance bound.

Acceptance (elementwise), with S = sum_k |x_k * w_k| from the oracle:
    |y - y_ref| <= g * B * S + 8 * 2^-24 * (|y_ref| + |v| + |bias| + |y_old|)
B = 2^-8 on the MFMA path (X rounded to bf16), 1e-5 on the all-f32 paths;
g is the largest slope of the activation (an error before it is stretched by
at most that factor): 1.13 for GELU, 1.1 for SiLU, 1 for ReLU, tanh or none;
v is the pre-activation value. With a factor alpha on the activated value
(wq_linear), the first term and v, bias scale by |alpha|. The last term
covers the f32 roundings of the epilogue itself (bias add, the activation's
evaluation, the alpha product, the residual add), which S does not scale.
"""
from __future__ import annotations

import numpy as np

import oracle

CANARY = 12345.0
B_MFMA = 2.0 ** -8
B_F32 = 1e-5
GELU_SLOPE = 1.13
SLOPES = {2: GELU_SLOPE, 8: 1.1, 16: 1.0, 32: 1.0}  # max |act'| of GELU, SiLU, ReLU, tanh
ULP_SLACK = 8 * 2.0 ** -24


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def guarded_out(rows: int, cols: int, y_old=None, guard: int = 64):
    """A NaN-filled [rows x cols] output (or y_old) followed by `guard` canaries."""
    import torch
    buf = torch.full((rows * cols + guard,), float("nan"), dtype=torch.float32, device="cuda")
    buf[rows * cols:] = CANARY
    if y_old is not None:
        buf[: rows * cols] = dev(np.asarray(y_old, np.float32).reshape(-1))
    return buf, buf[: rows * cols].view(rows, cols)


def read_guarded(buf, rows: int, cols: int) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert (host[rows * cols:] == CANARY).all(), "write past the end of the output"
    return host[: rows * cols].reshape(rows, cols)


def tolerance(S, y_ref, bound, flags=0, v=None, bias=None, y_old=None, alpha=1.0):
    g = max([SLOPES[a] for a in SLOPES if flags & a], default=1.0)
    a = abs(float(alpha))
    mag = np.abs(y_ref)
    if v is not None:
        mag = mag + a * np.abs(v)
    if bias is not None and flags & oracle.FLAG_BIAS:
        mag = mag + a * np.abs(np.asarray(bias, np.float64))[None, :]
    if y_old is not None and flags & oracle.FLAG_RESIDUAL:
        mag = mag + np.abs(np.asarray(y_old, np.float64))
    return a * g * bound * S + ULP_SLACK * mag


def assert_within(got, y_ref, tol, what=""):
    got = np.asarray(got, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs at {np.argwhere(~np.isfinite(got))[:5]}"
    err = np.abs(got - y_ref)
    bad = err > tol
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise AssertionError(
            f"{what}: {bad.sum()} of {bad.size} outside the bound; first at {i}: got {got[i]!r}, "
            f"want {y_ref[i]!r}, err {err[i]:.3e} > tol {tol[i]:.3e}; worst err/tol "
            f"{(err / np.maximum(tol, 1e-300)).max():.3f}")
    return float((err / np.maximum(tol, 1e-300)).max())


ACT_FLAGS = 2 | 8 | 16 | 32


def oracle_with_tol(x, w, wtype, m, k, bias, flags, y_old, bound, rows=None, alpha=1.0):
    """(y_ref, tol) from the oracle for one layer call."""
    y_ref, S = oracle.linear(x, w, wtype, m, k, bias, flags, y_old, rows=rows, alpha=alpha)
    v = None
    if flags & ACT_FLAGS:
        v, _ = oracle.linear(x, w, wtype, m, k, bias, flags & oracle.FLAG_BIAS, rows=rows)
    b = None if bias is None else (np.asarray(bias)[rows] if rows is not None else bias)
    yo = None
    if y_old is not None:
        yo = np.asarray(y_old, np.float64).reshape(-1, m)
        yo = yo[:, rows] if rows is not None else yo
    return y_ref, tolerance(S, y_ref, bound, flags, v, b, yo, alpha)


def literal_ratio(got, y_ref, S, bound) -> float:
    """max |y - y_ref| / (bound * S) over the outputs with S > 0: the error against the bound as
    the workload states it (B * S alone, with no slope or f32 epilogue slack added)."""
    got = np.asarray(got, np.float64)
    S = np.asarray(S, np.float64)
    pos = S > 0
    if not pos.any():
        return 0.0
    return float((np.abs(got - y_ref)[pos] / (bound * S[pos])).max())


def guarded_at_offset(rows: int, cols: int, offset: int, y_old=None, guard: int = 64):
    """An output that starts `offset` floats into its buffer: canaries before and after it, NaN
    (or y_old) inside. Returns (buffer, the [rows x cols] view)."""
    import torch
    total = offset + rows * cols + guard
    buf = torch.full((total,), CANARY, dtype=torch.float32, device="cuda")
    inner = buf[offset: offset + rows * cols]
    inner.fill_(float("nan"))
    if y_old is not None:
        inner.copy_(dev(np.asarray(y_old, np.float32).reshape(-1)))
    return buf, inner.view(rows, cols)


def read_at_offset(buf, rows: int, cols: int, offset: int) -> np.ndarray:
    import torch
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    assert (host[:offset] == CANARY).all(), "write before the start of the output"
    assert (host[offset + rows * cols:] == CANARY).all(), "write past the end of the output"
    return host[offset: offset + rows * cols].reshape(rows, cols)
