"""CPU oracle for the FP8 blockwise-quantized linear layer.

TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this package.  The GPU library never loads it
and shares no code with it.

Thin ctypes marshalling over ``oracle.c`` (plain C, fp32 steps in IEEE single
precision, the GEMM reference in fp64).  Every function documents which
passage of the pages it follows; see ``oracle.c`` for the definitions.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against the OCP e4m3fn definition, closed forms, invariants, brute force and
independent library routines (torch's float8 conversion, numpy fp32 division,
numpy matmul).  Nothing is "parity unpinned" except the interface conventions
(eps default, scale layouts), which the pages leave open.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

GROUP = 128
E4M3_MAX = 448.0
DEFAULT_EPS = np.float32(1e-10)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        from . import build as _build
        _build.build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    I64 = ctypes.c_int64
    lib.orc_e4m3_decode.restype = ctypes.c_double
    lib.orc_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.orc_e4m3_encode.restype = ctypes.c_uint8
    lib.orc_e4m3_encode.argtypes = [ctypes.c_float]
    lib.orc_e4m3_encode_array_mt.restype = ctypes.c_int
    lib.orc_e4m3_encode_array_mt.argtypes = [P, P, I64, ctypes.c_int]
    lib.orc_pow2_ceil.restype = ctypes.c_float
    lib.orc_pow2_ceil.argtypes = [ctypes.c_float]
    lib.orc_scale_from_amax.restype = ctypes.c_float
    lib.orc_scale_from_amax.argtypes = [ctypes.c_float, ctypes.c_float, ctypes.c_int]
    lib.orc_group_quant_mt.restype = ctypes.c_int
    lib.orc_group_quant_mt.argtypes = [P, I64, I64, I64, P, I64, P, I64,
                                       ctypes.c_float, ctypes.c_int, ctypes.c_int]
    lib.orc_weight_block_quant.restype = None
    lib.orc_weight_block_quant.argtypes = [P, I64, I64, P, P, ctypes.c_float, ctypes.c_int]
    lib.orc_weight_block_quant_mt.restype = ctypes.c_int
    lib.orc_weight_block_quant_mt.argtypes = [P, I64, I64, P, P, ctypes.c_float, ctypes.c_int, ctypes.c_int]
    lib.orc_block_gemm.restype = ctypes.c_int
    lib.orc_block_gemm.argtypes = [P, P, P, P, I64, I64, I64, P, I64, P, ctypes.c_int]
    lib.orc_token_quant_mt.restype = ctypes.c_int
    lib.orc_token_quant_mt.argtypes = [P, I64, I64, I64, P, I64, P, ctypes.c_float, ctypes.c_int, ctypes.c_int]
    lib.orc_channel_quant.restype = None
    lib.orc_channel_quant.argtypes = [P, I64, I64, P, P, ctypes.c_float, ctypes.c_int]
    lib.orc_rms_norm_per_block_quant.restype = None
    lib.orc_rms_norm_per_block_quant.argtypes = [P, P, I64, I64, ctypes.c_float, P, P, ctypes.c_float, ctypes.c_int]
    lib.orc_silu_and_mul_per_block_quant.restype = None
    lib.orc_silu_and_mul_per_block_quant.argtypes = [P, I64, I64, P, P, ctypes.c_float, ctypes.c_int]
    lib.orc_group_quant_f32.restype = None
    lib.orc_group_quant_f32.argtypes = [P, I64, I64, P, P, ctypes.c_float, ctypes.c_int]
    lib.orc_rms_norm_inv_rms.restype = None
    lib.orc_rms_norm_inv_rms.argtypes = [P, I64, I64, ctypes.c_float, P]
    lib.orc_rms_norm_apply.restype = None
    lib.orc_rms_norm_apply.argtypes = [P, P, I64, I64, P, P, P, ctypes.c_float, ctypes.c_int]
    lib.orc_silu_and_mul_values.restype = None
    lib.orc_silu_and_mul_values.argtypes = [P, I64, I64, P]
    lib.orc_scaled_mm.restype = ctypes.c_int
    lib.orc_scaled_mm.argtypes = [P, P, P, P, I64, I64, I64, P, I64, P, ctypes.c_int]
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def default_threads() -> int:
    return max(1, min(64, os.cpu_count() or 1))


def e4m3_decode(codes) -> np.ndarray:
    """Value of each e4m3fn code (OCP definition), as float64."""
    lib = _load()
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib.orc_e4m3_decode(c) for c in range(256)], dtype=np.float64)
    return table[codes]


def e4m3_encode(t, nthreads: int | None = None) -> np.ndarray:
    """Round-to-nearest-even e4m3fn code of each fp32 value with |t| <= 448.

    The clamp to +-448 is not applied here (it belongs to the quantizer)."""
    lib = _load()
    t = np.ascontiguousarray(np.asarray(t, dtype=np.float32))
    q = np.empty(t.shape, dtype=np.uint8)
    lib.orc_e4m3_encode_array_mt(_ptr(t), _ptr(q), t.size, nthreads or default_threads())
    return q


def pow2_ceil(s: float) -> np.float32:
    return np.float32(_load().orc_pow2_ceil(float(s)))


def scale_from_amax(amax: float, eps=DEFAULT_EPS, ue8m0: bool = False) -> np.float32:
    return np.float32(_load().orc_scale_from_amax(float(np.float32(amax)), float(np.float32(eps)), int(ue8m0)))


def group_quant(x_bf16_bits: np.ndarray, eps=DEFAULT_EPS, ue8m0: bool = False,
                nthreads: int | None = None):
    """per_token_group_fp8_quant of bf16 X [M, K] (given as uint16 bit patterns).

    Returns (q uint8 [M, K], s float32 [M, K/128])."""
    lib = _load()
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, K = x.shape
    assert K % GROUP == 0
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // GROUP), dtype=np.float32)
    lib.orc_group_quant_mt(_ptr(x), M, K, K, _ptr(q), K, _ptr(s), K // GROUP,
                           float(np.float32(eps)), int(ue8m0), nthreads or default_threads())
    return q, s


def weight_block_quant(w: np.ndarray, eps=DEFAULT_EPS, ue8m0: bool = False,
                       nthreads: int | None = None):
    """128x128 block quantization of fp32 W [N, K].

    Returns (q uint8 [N, K], s float32 [N/128, K/128])."""
    lib = _load()
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert N % GROUP == 0 and K % GROUP == 0
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((N // GROUP, K // GROUP), dtype=np.float32)
    lib.orc_weight_block_quant_mt(_ptr(w), N, K, _ptr(q), _ptr(s), float(np.float32(eps)),
                                  int(ue8m0), nthreads or default_threads())
    return q, s


def block_gemm(qa, sa, qw, sw, rows=None, nthreads: int | None = None) -> np.ndarray:
    """fp64 Y = dequant(A) @ dequant(W)^T, optionally on a subset of rows.

    Returns float64 [len(rows) or M, N]."""
    lib = _load()
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2 and K % GROUP == 0 and N % GROUP == 0
    assert sa.shape == (M, K // GROUP) and sw.shape == (N // GROUP, K // GROUP)
    if rows is None:
        nrows = M
        rows_arr = None
        rows_ptr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows_arr.size == 0 or (rows_arr.min() >= 0 and rows_arr.max() < M)
        nrows = rows_arr.size
        rows_ptr = _ptr(rows_arr)
    y = np.empty((nrows, N), dtype=np.float64)
    if nrows:
        lib.orc_block_gemm(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K,
                           rows_ptr, nrows, _ptr(y), nthreads or default_threads())
    return y


def token_quant(x_bf16_bits: np.ndarray, eps=DEFAULT_EPS, ue8m0: bool = False,
                nthreads: int | None = None):
    """dynamic_per_token_scaled_fp8_quant (FP8_Dynamic activations) of bf16
    X [M, K]: one scale per row.  Returns (q uint8 [M, K], s float32 [M])."""
    lib = _load()
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, K = x.shape
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M,), dtype=np.float32)
    lib.orc_token_quant_mt(_ptr(x), M, K, K, _ptr(q), K, _ptr(s), float(np.float32(eps)),
                           int(ue8m0), nthreads or default_threads())
    return q, s


def channel_quant(w: np.ndarray, eps=DEFAULT_EPS, ue8m0: bool = False):
    """Per-channel (per row of W [N, K]) quantization of fp32 weights (FP8_Dynamic
    weights).  Returns (q uint8 [N, K], s float32 [N])."""
    lib = _load()
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((N,), dtype=np.float32)
    lib.orc_channel_quant(_ptr(w), N, K, _ptr(q), _ptr(s), float(np.float32(eps)), int(ue8m0))
    return q, s


def scaled_mm(qa, sa, qw, sw, rows=None, nthreads: int | None = None) -> np.ndarray:
    """fp64 scaled_mm with per-token sa [M] and per-channel sw [N]:
    Y = (dec(A) * sa[:, None]) @ (dec(W) * sw[:, None])^T.  Float64 [rows, N]."""
    lib = _load()
    qa = np.ascontiguousarray(qa, dtype=np.uint8)
    sa = np.ascontiguousarray(sa, dtype=np.float32)
    qw = np.ascontiguousarray(qw, dtype=np.uint8)
    sw = np.ascontiguousarray(sw, dtype=np.float32)
    M, K = qa.shape
    N, K2 = qw.shape
    assert K == K2 and sa.shape == (M,) and sw.shape == (N,)
    if rows is None:
        nrows, rows_ptr = M, None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        assert rows_arr.size == 0 or (rows_arr.min() >= 0 and rows_arr.max() < M)
        nrows, rows_ptr = rows_arr.size, _ptr(rows_arr)
    y = np.empty((nrows, N), dtype=np.float64)
    if nrows:
        lib.orc_scaled_mm(_ptr(qa), _ptr(sa), _ptr(qw), _ptr(sw), M, N, K, rows_ptr, nrows,
                          _ptr(y), nthreads or default_threads())
    return y


def rms_norm_per_block_quant(x_bf16_bits: np.ndarray, w: np.ndarray, eps_norm=1e-6,
                             eps=DEFAULT_EPS, ue8m0: bool = False):
    """rms_norm_per_block_quant: RMSNorm of bf16 X [M, H] with fp32 weight [H],
    then the 1x128 group quantizer.  Returns (q uint8 [M, H], s float32 [M, H/128])."""
    lib = _load()
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    M, H = x.shape
    assert H % GROUP == 0 and w.shape == (H,)
    q = np.empty((M, H), dtype=np.uint8)
    s = np.empty((M, H // GROUP), dtype=np.float32)
    lib.orc_rms_norm_per_block_quant(_ptr(x), _ptr(w), M, H, float(np.float32(eps_norm)), _ptr(q), _ptr(s),
                                 float(np.float32(eps)), int(ue8m0))
    return q, s


def silu_and_mul_per_block_quant(x_bf16_bits: np.ndarray, eps=DEFAULT_EPS, ue8m0: bool = False):
    """silu_and_mul_per_block_quant of bf16 X [M, 2I] = [gate | up]: SiLU(gate) * up,
    then the 1x128 group quantizer.  Returns (q uint8 [M, I], s float32 [M, I/128])."""
    lib = _load()
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, I2 = x.shape
    I = I2 // 2
    assert I2 % 2 == 0 and I % GROUP == 0
    q = np.empty((M, I), dtype=np.uint8)
    s = np.empty((M, I // GROUP), dtype=np.float32)
    lib.orc_silu_and_mul_per_block_quant(_ptr(x), M, I, _ptr(q), _ptr(s), float(np.float32(eps)), int(ue8m0))
    return q, s


def group_quant_f32(y: np.ndarray, eps=DEFAULT_EPS, ue8m0: bool = False):
    """The group rule on float32 values Y [M, K] already computed (the last step
    of both fused producers).  Returns (q uint8 [M, K], s float32 [M, K/128])."""
    lib = _load()
    y = np.ascontiguousarray(y, dtype=np.float32)
    M, K = y.shape
    assert K % GROUP == 0
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // GROUP), dtype=np.float32)
    lib.orc_group_quant_f32(_ptr(y), M, K, _ptr(q), _ptr(s), float(np.float32(eps)), int(ue8m0))
    return q, s


def rms_norm_inv_rms(x_bf16_bits: np.ndarray, eps_norm=1e-6) -> np.ndarray:
    """RMSNorm's 1/rms of every row of X [M, H] in float64, before the oracle
    rounds it to float32."""
    lib = _load()
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, H = x.shape
    r = np.empty((M,), dtype=np.float64)
    lib.orc_rms_norm_inv_rms(_ptr(x), M, H, float(np.float32(eps_norm)), _ptr(r))
    return r


def rms_norm_apply(x_bf16_bits: np.ndarray, w: np.ndarray, r: np.ndarray, eps=DEFAULT_EPS,
                   ue8m0: bool = False):
    """rms_norm_per_block_quant with the float32 1/rms of every row given."""
    lib = _load()
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w, dtype=np.float32)
    r = np.ascontiguousarray(r, dtype=np.float32)
    M, H = x.shape
    assert H % GROUP == 0 and w.shape == (H,) and r.shape == (M,)
    q = np.empty((M, H), dtype=np.uint8)
    s = np.empty((M, H // GROUP), dtype=np.float32)
    lib.orc_rms_norm_apply(_ptr(x), _ptr(w), M, H, _ptr(r), _ptr(q), _ptr(s), float(np.float32(eps)),
                           int(ue8m0))
    return q, s


def silu_and_mul_values(x_bf16_bits: np.ndarray) -> np.ndarray:
    """silu(gate) * up of X [M, 2I] in float64, before the oracle rounds it to
    float32.  Returns float64 [M, I]."""
    lib = _load()
    x = np.ascontiguousarray(x_bf16_bits, dtype=np.uint16)
    M, I2 = x.shape
    I = I2 // 2
    y = np.empty((M, I), dtype=np.float64)
    lib.orc_silu_and_mul_values(_ptr(x), M, I, _ptr(y))
    return y


def lib_path() -> str:
    return _LIB_PATH
