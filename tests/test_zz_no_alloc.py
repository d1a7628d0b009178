"""fp8_linear_noalloc -- fp8_linear with the library's per-GPU scratch array
as its workspace -- against fp8_linear with a caller-provided workspace,
through the C ABI.  The two run the same kernels on the same data, so the
outputs must be identical bit for bit (stronger than the GEMM tolerance).
Every case makes two calls in a row, the second with fewer tokens and other
data, so that the second call cannot lean on what the first left in the
shared array.  Covered: the fused Swap-AB path with and without split-K
partials, and Standard configurations that stage the quantized activations
(and split-K partials) in the array."""
import numpy as np
import pytest

import fp8_blockwise_quantized_token_amd as fb
from fp8_blockwise_quantized_token_amd import synth

from gpu_common import dev, host, oracle_weight, say, to_dev, to_dev_bf16

pytestmark = pytest.mark.gpu


def _x(M, K, key):
    return synth.activations_bf16(synth.Case("decode_8b", f"na{key}", M, 128, K, "normal_outlier", False, 900 + key))


CASES = [
    # (first M, second M, N, K, configuration or None for the dispatched one)
    (64, 8, 24576, 4096, None),
    (32, 1, 4096, 4096, None),
    (256, 100, 5120, 25600, None),
    (48, 17, 2048, 2048, fb.make_config(fb.SWAPAB, 64, 16, 2, 8)),
    (24, 5, 6144, 4096, fb.make_config(fb.SWAPAB, 32, 32, 4, 4)),
    (200, 130, 4096, 4096, fb.make_config(fb.STANDARD, 128, 128, 3)),
    (700, 300, 2048, 6144, fb.make_config(fb.STANDARD, 256, 128, 1, stages=3)),
]


@pytest.mark.parametrize("M1,M2,N,K,cfg", CASES)
def test_noalloc_equals_fp8_linear_twice_in_a_row(M1, M2, N, K, cfg):
    import torch
    assert M2 < M1
    qw, sw = oracle_weight(N, K, False)
    qwd, swd = to_dev(qw), to_dev(sw)
    # the M = 0 call only looks the scratch array up on this device
    x0 = torch.empty((0, K), dtype=torch.bfloat16, device=dev())
    fb.fp8_linear_noalloc(x0, qwd, swd, torch.empty((0, N), dtype=torch.bfloat16, device=dev()), cfg=cfg)
    outs = []
    for i, M in enumerate((M1, M2)):
        need = fb.fp8_linear_workspace_size(M, N, K, cfg)
        assert need <= fb.NOALLOC_SCRATCH_BYTES, (M, N, K, need)
        x = to_dev_bf16(_x(M, K, 10 * i + M % 7))
        say("noalloc", M, N, K, cfg.as_dict() if cfg is not None else "dispatched", "workspace", need)
        y_ref = fb.linear(x, qwd, swd, cfg=cfg)
        y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev())
        fb.fp8_linear_noalloc(x, qwd, swd, y, cfg=cfg)
        torch.cuda.synchronize()
        outs.append((host(y), host(y_ref)))
    for (y, y_ref), M in zip(outs, (M1, M2)):
        assert np.array_equal(y.view(np.uint32), y_ref.view(np.uint32)), f"M={M}: differs from fp8_linear"


def test_noalloc_refuses_calls_beyond_the_array():
    import torch
    M, N, K = 16384, 4096, 12288
    need = fb.fp8_linear_workspace_size(M, N, K, None)
    assert need > fb.NOALLOC_SCRATCH_BYTES
    x = torch.empty((M, K), dtype=torch.bfloat16, device=dev())
    w = torch.empty((N, K), dtype=torch.uint8, device=dev())
    sw = torch.empty((N // 128, K // 128), dtype=torch.float32, device=dev())
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    with pytest.raises(fb.Fp8BlkError) as e:
        fb.fp8_linear_noalloc(x, w, sw, y)
    assert e.value.status == -5
