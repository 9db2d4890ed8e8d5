"""GPU check of nvfp4_quantize_noalloc, the variant of nvfp4_quantize that
allocates nothing (its amax pass uses the library's own static workspace):
its outputs must equal nvfp4_quantize's bit for bit, for two calls in a row
(the second on a smaller input, after the first left its partial maxima in
the shared workspace), in every mode the entry point serves."""

import numpy as np
import pytest

import workloads as wl
from tests._helpers import announce, host, require_gpu, to_device

pytestmark = pytest.mark.gpu

CASES = [
    # (block, rounding, outputs, dtype)
    (0, 0, 1, "bf16"),
    (0, 0, 3, "bf16"),
    (0, 1, 2, "bf16"),
    (0, 1, 1, "fp32"),
    (1, 0, 3, "bf16"),
]


def _outputs(torch, rows, cols, block, outputs):
    e = lambda *s: torch.full(s, 0xAB, dtype=torch.uint8, device="cuda")
    two_d = block == 1
    q_row = e(rows, cols // 2) if outputs & 1 else None
    s_row = (e(rows // 16, cols // 16) if two_d else e(rows, cols // 16)) if outputs & 1 else None
    q_col = e(cols, rows // 2) if outputs & 2 else None
    s_col = (e(cols // 16, rows // 16) if two_d else e(cols, rows // 16)) if outputs & 2 else None
    ts = torch.zeros(4, dtype=torch.float32, device="cuda")
    return [q_row, s_row, q_col, s_col, ts]


@pytest.mark.parametrize("block,rounding,outputs,dtype", CASES)
def test_noalloc_equals_quantize_twice(block, rounding, outputs, dtype):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    for shape, seed in (((1040, 2064), 1), ((272, 400), 2)):
        announce(f"noalloc {shape} block={block} r={rounding} out={outputs} {dtype}")
        x_np = (wl.activation(shape[0], shape[1], seed=seed) if dtype == "bf16"
                else wl.normal(shape, seed, dtype="fp32"))
        x = to_device(x_np, dtype)
        ref = _outputs(torch, *shape, block, outputs)
        got = _outputs(torch, *shape, block, outputs)
        ws = nv.amax_workspace("cuda")
        nv.nvfp4_quantize(x, block, rounding, 9, 4, outputs, None, ws, *ref)
        nv.nvfp4_quantize_noalloc(x, block, rounding, 9, 4, outputs, None, *got)
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            if b is not None:
                assert np.array_equal(host(a), host(b))


def test_noalloc_with_amax_given():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    announce("noalloc amax_in")
    x = to_device(wl.laplace((528, 272), seed=4), "bf16")
    amax = torch.tensor([0.5, 0, 0, 0], dtype=torch.float32, device="cuda")
    ref = _outputs(torch, 528, 272, 0, 3)
    got = _outputs(torch, 528, 272, 0, 3)
    nv.nvfp4_quantize(x, 0, 0, 0, 0, 3, amax, None, *ref)
    nv.nvfp4_quantize_noalloc(x, 0, 0, 0, 0, 3, amax, *got)
    torch.cuda.synchronize()
    for a, b in zip(got, ref):
        assert np.array_equal(host(a), host(b))
