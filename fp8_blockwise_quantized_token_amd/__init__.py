"""MI355X (gfx950) FP8 blockwise-quantized linear layer.

Python binding of ``libfp8blk.so`` (C ABI in ``include/fp8blk.h``).  This
module only marshals arguments: every step of the computation runs in the
library's HIP kernels.  PyTorch provides device memory and streams.  If the
library has not been built, every call raises ``RuntimeError``; there is no
fallback implementation.

Entry points (same names as the C ABI):
  fp8_group_quant        per-token 1x128 group quantization (bf16 -> e4m3fn + fp32 scales)
  fp8_weight_block_quant 128x128 weight block quantization (fp32 -> e4m3fn + fp32 scales)
  fp8_e4m3_encode        the saturating round-to-nearest-even encoder alone
  fp8_block_gemm_select  per-shape dispatch (host only)
  fp8_block_gemm_workspace_size
  fp8_block_gemm         blockwise-scaled FP8 GEMM, bf16 out
  fp8_linear_workspace_size
  fp8_linear             the whole layer (quantize x, then the GEMM; fused for Swap-AB)
  fp8_linear_noalloc     fp8_linear with the library's per-GPU scratch array as workspace
  fp8_token_quant        per-token quantization (FP8_Dynamic activations)
  fp8_weight_channel_quant  per-channel weight quantization (FP8_Dynamic weights)
  fp8_scaled_mm          GEMM with per-token / per-channel scales
  fp8_rms_norm_per_block_quant      RMSNorm fused with the 1x128 group quantizer
  fp8_silu_and_mul_per_block_quant  SiLU(gate) * up fused with the 1x128 group quantizer
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libfp8blk.so")

ABI_VERSION = 6  # FP8BLK_ABI_VERSION of the header this binding follows
GROUP = 128
FLAG_UE8M0 = 1
FLAG_WEIGHT_POW2 = 8  # the weight scales are powers of two (fp8_linear, fp8_block_gemm_select)
STANDARD = 0
SWAPAB = 1
DEFAULT_EPS = 1e-10
MIN_EPS = 2.0 ** -80  # smallest eps the library accepts (FP8BLK_MIN_EPS)

_STATUS = {0: "ok", -1: "null pointer", -2: "unsupported shape", -3: "misaligned",
           -4: "leading dimension too small", -5: "workspace too small",
           -6: "unsupported configuration", -7: "HIP launch failure"}


class GemmConfig(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("split_k", ctypes.c_int32),
                ("kwaves", ctypes.c_int32), ("stages", ctypes.c_int32),
                ("scale_mode", ctypes.c_int32), ("split_tail", ctypes.c_int32)]

    def as_dict(self) -> dict:
        return {"variant": "swapab" if self.variant == SWAPAB else "standard",
                "tile_m": self.tile_m, "tile_n": self.tile_n,
                "split_k": self.split_k, "kwaves": self.kwaves, "stages": self.stages,
                "scale_mode": self.scale_mode, "split_tail": self.split_tail}

    def __repr__(self) -> str:
        return f"GemmConfig({self.as_dict()})"


SCALES_FP32 = 0
SCALES_POW2 = 1
SCALES_SA_MN_MAJOR = 2  # bit: fp8_block_gemm's activation scales are [K/128, >= M]


def make_config(variant: int, tile_m: int, tile_n: int, split_k: int = 1, kwaves: int = 1,
                stages: int = 0, scale_mode: int = SCALES_FP32, split_tail: int = 0) -> GemmConfig:
    c = GemmConfig()
    c.variant, c.tile_m, c.tile_n, c.split_k, c.kwaves, c.stages = variant, tile_m, tile_n, split_k, kwaves, stages
    c.scale_mode, c.split_tail = scale_mode, split_tail
    return c


class Fp8BlkError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed: status {status} ({_STATUS.get(status, 'unknown')})")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (ctypes handle with argument types set)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -c 'import __graft_entry__ as g; g.build()'`")
    L = ctypes.CDLL(LIB_PATH)
    P, I64, I32, U32, F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
    L.fp8_abi_version.restype = ctypes.c_int
    L.fp8_abi_version.argtypes = []
    L.fp8_status_string.restype = ctypes.c_char_p
    L.fp8_status_string.argtypes = [ctypes.c_int]
    L.fp8_group_quant.restype = ctypes.c_int
    L.fp8_group_quant.argtypes = [P, I64, I64, I64, P, I64, P, I64, I32, F, U32, P]
    L.fp8_weight_block_quant.restype = ctypes.c_int
    L.fp8_weight_block_quant.argtypes = [P, I64, I64, I64, P, I64, P, I64, F, U32, P]
    L.fp8_e4m3_encode.restype = ctypes.c_int
    L.fp8_e4m3_encode.argtypes = [P, P, I64, P]
    L.fp8_block_gemm_select.restype = ctypes.c_int
    L.fp8_block_gemm_select.argtypes = [I64, I64, I64, U32, ctypes.POINTER(GemmConfig)]
    L.fp8_block_gemm_workspace_size.restype = I64
    L.fp8_block_gemm_workspace_size.argtypes = [I64, I64, I64, ctypes.POINTER(GemmConfig)]
    L.fp8_block_gemm.restype = ctypes.c_int
    L.fp8_block_gemm.argtypes = [P, P, I64, I64, P, P, I64, I64, P, I64, I64, I64, I64,
                                 ctypes.POINTER(GemmConfig), P, I64, P]
    L.fp8_token_quant.restype = ctypes.c_int
    L.fp8_token_quant.argtypes = [P, I64, I64, I64, P, I64, P, F, U32, P]
    L.fp8_weight_channel_quant.restype = ctypes.c_int
    L.fp8_weight_channel_quant.argtypes = [P, I64, I64, I64, P, I64, P, F, U32, P]
    L.fp8_scaled_mm.restype = ctypes.c_int
    L.fp8_scaled_mm.argtypes = [P, P, I64, P, P, I64, P, I64, I64, I64, I64,
                                ctypes.POINTER(GemmConfig), P, I64, P]
    L.fp8_linear_workspace_size.restype = I64
    L.fp8_linear_workspace_size.argtypes = [I64, I64, I64, ctypes.POINTER(GemmConfig)]
    L.fp8_linear.restype = ctypes.c_int
    L.fp8_linear.argtypes = [P, I64, P, P, I64, I64, P, I64, I64, I64, I64, F, U32,
                             ctypes.POINTER(GemmConfig), P, I64, P]
    L.fp8_linear_noalloc.restype = ctypes.c_int
    L.fp8_linear_noalloc.argtypes = [P, I64, P, P, I64, I64, P, I64, I64, I64, I64, F, U32,
                                     ctypes.POINTER(GemmConfig), P]
    L.fp8_rms_norm_per_block_quant.restype = ctypes.c_int
    L.fp8_rms_norm_per_block_quant.argtypes = [P, I64, I64, I64, P, F, P, I64, P, I64, F, U32, P]
    L.fp8_silu_and_mul_per_block_quant.restype = ctypes.c_int
    L.fp8_silu_and_mul_per_block_quant.argtypes = [P, I64, I64, I64, P, I64, P, I64, F, U32, P]
    if L.fp8_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{LIB_PATH} has ABI version {L.fp8_abi_version()}, the binding expects "
                           f"{ABI_VERSION}: rebuild it")
    _lib = L
    return L


def _stream(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _ld(t, what: str) -> int:
    """Row pitch in elements.  A single-row tensor may carry any stride for
    its row dimension (0 included); its pitch is then its row length."""
    if t.dim() != 2 or (t.stride(1) != 1 and t.shape[1] > 1):
        raise ValueError(f"{what}: expected a 2-D tensor with unit column stride")
    if t.shape[0] <= 1:
        return max(t.stride(0), t.shape[1])
    return t.stride(0)


def _check(st: int, what: str) -> None:
    if st != 0:
        raise Fp8BlkError(st, what)


def fp8_abi_version() -> int:
    return lib().fp8_abi_version()


def fp8_status_string(status: int) -> str:
    return lib().fp8_status_string(status).decode()


FLAG_SCALE_E8M0 = 2
FLAG_SCALE_MN_MAJOR = 4


def fp8_group_quant(x, q, s, eps: float = DEFAULT_EPS, ue8m0: bool = False, stream=None,
                    scale_e8m0: bool = False, scale_mn_major: bool = False) -> None:
    """x: bf16 [M, K] (cuda), q: 1-byte [M, K], s: float32 [M, K/128] (MN-major:
    [K/128, >= M]; E8M0: 1-byte elements); outputs overwritten."""
    M, K = x.shape
    srows = K // GROUP if scale_mn_major else M
    if q.shape != (M, K) or s.shape[0] != srows or x.element_size() != 2 or q.element_size() != 1:
        raise ValueError("fp8_group_quant: shape/dtype mismatch")
    if s.element_size() != (1 if scale_e8m0 else 4):
        raise ValueError("fp8_group_quant: scale dtype mismatch")
    flags = (FLAG_UE8M0 if ue8m0 else 0) | (FLAG_SCALE_E8M0 if scale_e8m0 else 0) | \
        (FLAG_SCALE_MN_MAJOR if scale_mn_major else 0)
    st = lib().fp8_group_quant(x.data_ptr(), M, K, _ld(x, "x"), q.data_ptr(), _ld(q, "q"),
                               s.data_ptr(), _ld(s, "s"), GROUP, eps, flags, _stream(stream))
    _check(st, "fp8_group_quant")


def _scale_flags(ue8m0: bool, scale_e8m0: bool, scale_mn_major: bool) -> int:
    return (FLAG_UE8M0 if ue8m0 else 0) | (FLAG_SCALE_E8M0 if scale_e8m0 else 0) | \
        (FLAG_SCALE_MN_MAJOR if scale_mn_major else 0)


def _check_group_out(what: str, M: int, K: int, q, s, scale_e8m0: bool, scale_mn_major: bool) -> None:
    srows = K // GROUP if scale_mn_major else M
    if q.shape != (M, K) or q.element_size() != 1 or s.dim() != 2 or s.shape[0] != srows:
        raise ValueError(f"{what}: output shape/dtype mismatch")
    if s.element_size() != (1 if scale_e8m0 else 4):
        raise ValueError(f"{what}: scale dtype mismatch")


def fp8_rms_norm_per_block_quant(x, weight, q, s, eps_norm: float = 1e-6, eps: float = DEFAULT_EPS,
                                 ue8m0: bool = False, stream=None, scale_e8m0: bool = False,
                                 scale_mn_major: bool = False) -> None:
    """x: bf16 [M, H], weight: float32 [H] (contiguous), q: 1-byte [M, H],
    s: float32 [M, H/128] (MN-major / E8M0 as fp8_group_quant)."""
    M, H = x.shape
    if x.element_size() != 2 or weight.element_size() != 4 or tuple(weight.shape) != (H,) \
            or not weight.is_contiguous():
        raise ValueError("fp8_rms_norm_per_block_quant: x/weight shape or dtype mismatch")
    _check_group_out("fp8_rms_norm_per_block_quant", M, H, q, s, scale_e8m0, scale_mn_major)
    st = lib().fp8_rms_norm_per_block_quant(x.data_ptr(), M, H, _ld(x, "x"), weight.data_ptr(), eps_norm,
                                            q.data_ptr(), _ld(q, "q"), s.data_ptr(), _ld(s, "s"), eps,
                                            _scale_flags(ue8m0, scale_e8m0, scale_mn_major), _stream(stream))
    _check(st, "fp8_rms_norm_per_block_quant")


def fp8_silu_and_mul_per_block_quant(x, q, s, eps: float = DEFAULT_EPS, ue8m0: bool = False, stream=None,
                                     scale_e8m0: bool = False, scale_mn_major: bool = False) -> None:
    """x: bf16 [M, 2I] = [gate | up], q: 1-byte [M, I], s: float32 [M, I/128]."""
    M, I2 = x.shape
    if x.element_size() != 2 or I2 % 2 != 0:
        raise ValueError("fp8_silu_and_mul_per_block_quant: x shape or dtype mismatch")
    I = I2 // 2
    _check_group_out("fp8_silu_and_mul_per_block_quant", M, I, q, s, scale_e8m0, scale_mn_major)
    st = lib().fp8_silu_and_mul_per_block_quant(x.data_ptr(), M, I, _ld(x, "x"), q.data_ptr(), _ld(q, "q"),
                                                s.data_ptr(), _ld(s, "s"), eps,
                                                _scale_flags(ue8m0, scale_e8m0, scale_mn_major),
                                                _stream(stream))
    _check(st, "fp8_silu_and_mul_per_block_quant")


def fp8_weight_block_quant(w, q, s, eps: float = DEFAULT_EPS, ue8m0: bool = False, stream=None) -> None:
    """w: float32 [N, K], q: 1-byte [N, K], s: float32 [N/128, K/128]."""
    N, K = w.shape
    if q.shape != (N, K) or w.element_size() != 4 or q.element_size() != 1:
        raise ValueError("fp8_weight_block_quant: shape/dtype mismatch")
    st = lib().fp8_weight_block_quant(w.data_ptr(), N, K, _ld(w, "w"), q.data_ptr(), _ld(q, "q"),
                                      s.data_ptr(), _ld(s, "s"), eps,
                                      FLAG_UE8M0 if ue8m0 else 0, _stream(stream))
    _check(st, "fp8_weight_block_quant")


def fp8_e4m3_encode(t, q, stream=None) -> None:
    """t: contiguous float32 (any shape), q: contiguous 1-byte, same number of elements."""
    if not (t.is_contiguous() and q.is_contiguous()) or t.numel() != q.numel():
        raise ValueError("fp8_e4m3_encode: need contiguous tensors of equal size")
    _check(lib().fp8_e4m3_encode(t.data_ptr(), q.data_ptr(), t.numel(), _stream(stream)),
           "fp8_e4m3_encode")


def fp8_block_gemm_select(M: int, N: int, K: int, flags: int = 0) -> GemmConfig:
    c = GemmConfig()
    _check(lib().fp8_block_gemm_select(M, N, K, flags, ctypes.byref(c)), "fp8_block_gemm_select")
    return c


def fp8_block_gemm_workspace_size(M: int, N: int, K: int, cfg: GemmConfig | None = None) -> int:
    n = lib().fp8_block_gemm_workspace_size(M, N, K, ctypes.byref(cfg) if cfg is not None else None)
    if n < 0:
        raise Fp8BlkError(int(n), "fp8_block_gemm_workspace_size")
    return int(n)


def fp8_block_gemm(a, sa, w, sw, y, cfg: GemmConfig | None = None, workspace=None,
                   stream=None) -> None:
    """y[M, N] (bf16) = blockwise-scaled a[M, K] (e4m3fn) x w[N, K]^T."""
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K or y.shape != (M, N):
        raise ValueError("fp8_block_gemm: shape mismatch")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fp8_block_gemm(a.data_ptr(), sa.data_ptr(), _ld(a, "a"), _ld(sa, "sa"),
                              w.data_ptr(), sw.data_ptr(), _ld(w, "w"), _ld(sw, "sw"),
                              y.data_ptr(), _ld(y, "y"), M, N, K,
                              ctypes.byref(cfg) if cfg is not None else None,
                              ws_ptr, ws_bytes, _stream(stream))
    _check(st, "fp8_block_gemm")


def fp8_linear_workspace_size(M: int, N: int, K: int, cfg: GemmConfig | None = None) -> int:
    n = lib().fp8_linear_workspace_size(M, N, K, ctypes.byref(cfg) if cfg is not None else None)
    if n < 0:
        raise Fp8BlkError(int(n), "fp8_linear_workspace_size")
    return int(n)


def fp8_linear(x, w, sw, y, eps: float = DEFAULT_EPS, ue8m0: bool = False,
               cfg: GemmConfig | None = None, workspace=None, stream=None,
               weight_pow2: bool = False) -> None:
    """y[M, N] (bf16) = blockwise GEMM of group-quantized x[M, K] (bf16) and w[N, K]^T.

    ue8m0: power-of-two activation scales; weight_pow2: the caller's weight
    scales sw are powers of two (both are needed for the power-of-two GEMM mode)."""
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or y.shape != (M, N) or x.element_size() != 2:
        raise ValueError("fp8_linear: shape/dtype mismatch")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fp8_linear(x.data_ptr(), _ld(x, "x"), w.data_ptr(), sw.data_ptr(), _ld(w, "w"),
                          _ld(sw, "sw"), y.data_ptr(), _ld(y, "y"), M, N, K, eps,
                          (FLAG_UE8M0 if ue8m0 else 0) | (FLAG_WEIGHT_POW2 if weight_pow2 else 0),
                          ctypes.byref(cfg) if cfg is not None else None,
                          ws_ptr, ws_bytes, _stream(stream))
    _check(st, "fp8_linear")


NOALLOC_SCRATCH_BYTES = 64 << 20  # FP8BLK_NOALLOC_SCRATCH_BYTES


def fp8_linear_noalloc(x, w, sw, y, eps: float = DEFAULT_EPS, ue8m0: bool = False,
                       cfg: GemmConfig | None = None, stream=None, weight_pow2: bool = False) -> None:
    """fp8_linear without a workspace: the library's own per-GPU scratch array
    (NOALLOC_SCRATCH_BYTES) stands in for it; calls on one GPU must not overlap."""
    M, K = x.shape
    N = w.shape[0]
    if w.shape[1] != K or y.shape != (M, N) or x.element_size() != 2:
        raise ValueError("fp8_linear_noalloc: shape/dtype mismatch")
    st = lib().fp8_linear_noalloc(x.data_ptr(), _ld(x, "x"), w.data_ptr(), sw.data_ptr(), _ld(w, "w"),
                                  _ld(sw, "sw"), y.data_ptr(), _ld(y, "y"), M, N, K, eps,
                                  (FLAG_UE8M0 if ue8m0 else 0) | (FLAG_WEIGHT_POW2 if weight_pow2 else 0),
                                  ctypes.byref(cfg) if cfg is not None else None, _stream(stream))
    _check(st, "fp8_linear_noalloc")


def fp8_token_quant(x, q, s, eps: float = DEFAULT_EPS, ue8m0: bool = False, stream=None) -> None:
    """dynamic_per_token_scaled_fp8_quant: x bf16 [M, K] -> q 1-byte [M, K], s float32 [M]."""
    M, K = x.shape
    if q.shape != (M, K) or s.numel() != M or x.element_size() != 2 or q.element_size() != 1:
        raise ValueError("fp8_token_quant: shape/dtype mismatch")
    st = lib().fp8_token_quant(x.data_ptr(), M, K, _ld(x, "x"), q.data_ptr(), _ld(q, "q"),
                               s.data_ptr(), eps, FLAG_UE8M0 if ue8m0 else 0, _stream(stream))
    _check(st, "fp8_token_quant")


def fp8_weight_channel_quant(w, q, s, eps: float = DEFAULT_EPS, ue8m0: bool = False, stream=None) -> None:
    """Per-channel quantization of float32 W [N, K] -> q [N, K], s float32 [N]."""
    N, K = w.shape
    if q.shape != (N, K) or s.numel() != N or w.element_size() != 4 or q.element_size() != 1:
        raise ValueError("fp8_weight_channel_quant: shape/dtype mismatch")
    st = lib().fp8_weight_channel_quant(w.data_ptr(), N, K, _ld(w, "w"), q.data_ptr(), _ld(q, "q"),
                                        s.data_ptr(), eps, FLAG_UE8M0 if ue8m0 else 0, _stream(stream))
    _check(st, "fp8_weight_channel_quant")


def fp8_scaled_mm(a, sa, w, sw, y, cfg: GemmConfig | None = None, workspace=None, stream=None) -> None:
    """y[M, N] (bf16) = (a @ w^T) * sa[:, None] * sw[None, :] (per-token / per-channel scales)."""
    M, K = a.shape
    N = w.shape[0]
    if w.shape[1] != K or y.shape != (M, N) or sa.numel() != M or sw.numel() != N:
        raise ValueError("fp8_scaled_mm: shape mismatch")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().fp8_scaled_mm(a.data_ptr(), sa.data_ptr(), _ld(a, "a"), w.data_ptr(), sw.data_ptr(),
                             _ld(w, "w"), y.data_ptr(), _ld(y, "y"), M, N, K,
                             ctypes.byref(cfg) if cfg is not None else None,
                             ws_ptr, ws_bytes, _stream(stream))
    _check(st, "fp8_scaled_mm")


# -- conveniences that allocate their outputs with torch (plumbing only) ----

def quantize_activations(x, eps: float = DEFAULT_EPS, ue8m0: bool = False, stream=None):
    import torch
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, K // GROUP), dtype=torch.float32, device=x.device)
    fp8_group_quant(x, q, s, eps, ue8m0, stream)
    return q, s


def quantize_weight(w, eps: float = DEFAULT_EPS, ue8m0: bool = False, stream=None):
    import torch
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((N // GROUP, K // GROUP), dtype=torch.float32, device=w.device)
    fp8_weight_block_quant(w, q, s, eps, ue8m0, stream)
    return q, s


def workspace_for(M: int, N: int, K: int, cfg: GemmConfig | None, device):
    import torch
    n = fp8_block_gemm_workspace_size(M, N, K, cfg)
    return torch.empty((max(n, 16),), dtype=torch.uint8, device=device) if n else None


def block_gemm(a, sa, w, sw, cfg: GemmConfig | None = None, stream=None):
    import torch
    M, K = a.shape
    N = w.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    ws = workspace_for(M, N, K, cfg, a.device)
    fp8_block_gemm(a, sa, w, sw, y, cfg, ws, stream)
    return y


def linear_workspace(M: int, N: int, K: int, cfg: GemmConfig | None, device):
    import torch
    n = fp8_linear_workspace_size(M, N, K, cfg)
    return torch.empty((max(n, 16),), dtype=torch.uint8, device=device) if n else None


def linear(x, qw, sw, eps: float = DEFAULT_EPS, ue8m0: bool = False, cfg: GemmConfig | None = None,
           stream=None, weight_pow2: bool = False):
    """The whole FP8 linear layer (fp8_linear): quantize x per 1x128 group, then the blockwise GEMM."""
    import torch
    M, K = x.shape
    N = qw.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    ws = linear_workspace(M, N, K, cfg, x.device)
    fp8_linear(x, qw, sw, y, eps, ue8m0, cfg, ws, stream, weight_pow2)
    return y


def quantize_tokens(x, eps: float = DEFAULT_EPS, ue8m0: bool = False, stream=None):
    import torch
    M, K = x.shape
    q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    s = torch.empty((M,), dtype=torch.float32, device=x.device)
    fp8_token_quant(x, q, s, eps, ue8m0, stream)
    return q, s


def quantize_weight_channels(w, eps: float = DEFAULT_EPS, ue8m0: bool = False, stream=None):
    import torch
    N, K = w.shape
    q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
    s = torch.empty((N,), dtype=torch.float32, device=w.device)
    fp8_weight_channel_quant(w, q, s, eps, ue8m0, stream)
    return q, s


def scaled_mm(a, sa, w, sw, cfg: GemmConfig | None = None, stream=None):
    import torch
    M, K = a.shape
    N = w.shape[0]
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    ws = workspace_for(M, N, K, cfg, a.device)
    fp8_scaled_mm(a, sa, w, sw, y, cfg, ws, stream)
    return y


def dynamic_linear(x, qw, sw, eps: float = DEFAULT_EPS, cfg: GemmConfig | None = None, stream=None):
    """The FP8_Dynamic linear layer: per-token quantization of x, then scaled_mm."""
    qa, sa = quantize_tokens(x, eps, False, stream)
    return scaled_mm(qa, sa, qw, sw, cfg, stream)


def rms_norm_quant(x, weight, eps_norm: float = 1e-6, eps: float = DEFAULT_EPS, ue8m0: bool = False,
                   stream=None):
    """rms_norm_per_block_quant into new tensors: (q uint8 [M, H], s float32 [M, H/128])."""
    import torch
    M, H = x.shape
    q = torch.empty((M, H), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, H // GROUP), dtype=torch.float32, device=x.device)
    fp8_rms_norm_per_block_quant(x, weight, q, s, eps_norm, eps, ue8m0, stream)
    return q, s


def silu_and_mul_quant(x, eps: float = DEFAULT_EPS, ue8m0: bool = False, stream=None):
    """silu_and_mul_per_block_quant into new tensors: (q uint8 [M, I], s float32 [M, I/128])."""
    import torch
    M, I2 = x.shape
    q = torch.empty((M, I2 // 2), dtype=torch.uint8, device=x.device)
    s = torch.empty((M, I2 // 2 // GROUP), dtype=torch.float32, device=x.device)
    fp8_silu_and_mul_per_block_quant(x, q, s, eps, ue8m0, stream)
    return q, s
