"""Shared helpers of the GPU parity tests (host-side marshalling only)."""
from __future__ import annotations

import numpy as np

import oracle
from fp8_blockwise_quantized_token_amd import synth

_DEV = None


def dev():
    global _DEV
    if _DEV is None:
        import torch
        assert torch.cuda.is_available(), "GPU tests need an MI355X"
        _DEV = torch.device("cuda:0")
    return _DEV


def say(*parts) -> None:
    """Name the case before a GPU step, flushed, so a failing run says where it was."""
    print("[gpu]", *parts, flush=True)


def to_dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def to_dev_bf16(bits: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(torch.bfloat16)


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return (t.view(torch.int16).cpu().numpy().view(np.uint16).astype(np.uint32) << 16).view(np.float32)
    return t.cpu().numpy()


def tolerance(y_ref: np.ndarray) -> np.ndarray:
    """|y - y_ref| <= 1e-2 |y_ref| + 1e-3 max|y_ref| (max over the compared output)."""
    return 1e-2 * np.abs(y_ref) + 1e-3 * np.abs(y_ref).max()


def assert_close(y: np.ndarray, y_ref: np.ndarray, what: str = "") -> None:
    y = y.astype(np.float64)
    err = np.abs(y - y_ref)
    tol = tolerance(y_ref)
    bad = err > tol
    if bad.any():
        i = np.unravel_index(np.argmax(err - tol), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} outside tolerance; worst at {i}: "
                             f"y={y[i]} ref={y_ref[i]} tol={tol[i]}")


_WCACHE: dict = {}


def oracle_weight(N: int, K: int, ue8m0: bool):
    """Oracle-quantized synthetic weight (codes, scales), cached per shape."""
    key = (N, K, ue8m0)
    if key not in _WCACHE:
        if len(_WCACHE) > 4:
            _WCACHE.clear()
        w = synth.weights_f32(N, K)
        _WCACHE[key] = oracle.weight_block_quant(w, ue8m0=ue8m0)
    return _WCACHE[key]


def sample_rows(M: int, n: int = 12, key: int = 0, band: int = 256) -> np.ndarray:
    """First, last, one seeded row in every band of `band` rows (so every
    256-row tile row of the GEMM is checked) and a seeded spread of n - 2
    more rows."""
    if M <= n:
        return np.arange(M)
    rng = synth.generator(500, M, key)
    mid = rng.choice(np.arange(1, M - 1), size=n - 2, replace=False)
    starts = np.arange(0, M, band)
    per_band = starts + (rng.random(starts.size) * np.minimum(band, M - starts)).astype(np.int64)
    return np.unique(np.concatenate([[0, M - 1], mid, per_band]))
