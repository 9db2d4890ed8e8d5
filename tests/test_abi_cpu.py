"""CPU-only checks of the C-ABI library: it loads, exports every entry point
that include/nvfp4.h declares, derives the Hadamard sign vector on the host
exactly as the oracle does, and rejects bad arguments before any HIP call
(so none of these calls touches a GPU)."""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def L():
    from bit_block_scaled_bf16_amd import _lib

    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libnvfp4.so is not built (run __graft_entry__.build())")
    return _lib.lib()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|uint32_t|const char\*)\s+((?:nvfp4|mxfp4|fp8)_\w+)\(",
                                 text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("nvfp4_quantize", "nvfp4_dequantize", "nvfp4_rht_quantize", "nvfp4_gemm"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    from bit_block_scaled_bf16_amd import _lib

    names = declared_functions()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(_lib.EXPORTED)


def test_sign_mask_matches_oracle(L):
    for seed in (0, 1, 7, 12345, 2 ** 40 + 3, 2 ** 64 - 1):
        mask = int(L.nvfp4_rht_sign_mask(seed))
        d = o.rht_signs(seed)
        want = sum(1 << i for i in range(16) if d[i] < 0)
        assert mask == want, seed


def test_status_strings(L):
    for code in range(6):
        assert L.nvfp4_status_string(code)
    assert L.nvfp4_status_string(99) == b"unknown status"


# A fake, 16-byte aligned "device" address: every call below must be rejected
# by the host-side checks before anything dereferences it.
FAKE = 0x10000
MIS = 0x10008  # 8-byte aligned only


def q(L, **kw):
    a = dict(x=FAKE, x_dtype=1, rows=32, cols=32, ldx=32, block=0, rounding=0, seed=0, offset=0,
             outputs=3, amax_in=None, amax_ws=FAKE, q_row=FAKE, s_row=FAKE, q_col=FAKE,
             s_col=FAKE, tensor_scale=FAKE, dev_status=None, stream=None)
    a.update(kw)
    return L.nvfp4_quantize(*a.values())


def test_quantize_argument_errors(L):
    assert q(L, x_dtype=7) == 3
    assert q(L, block=2) == 3
    assert q(L, rounding=2) == 3
    assert q(L, outputs=0) == 3 and q(L, outputs=4) == 3
    assert q(L, block=1, rounding=1) == 3          # SR on 16x16 weight blocks
    assert q(L, cols=24, ldx=24) == 2               # cols % 16
    assert q(L, rows=24) == 2                       # column copy needs rows % 16
    assert q(L, rows=-1) == 2
    assert q(L, ldx=16) == 2                        # ldx < cols
    assert q(L, block=1, rows=24, outputs=1) == 2   # 2D needs rows % 16
    assert q(L, x=None) == 1
    assert q(L, tensor_scale=None) == 1
    assert q(L, amax_in=None, amax_ws=None) == 1
    assert q(L, q_col=None) == 1
    assert q(L, outputs=1, s_row=None) == 1
    assert q(L, x=MIS) == 4
    assert q(L, ldx=36) == 4                        # bf16 rows of 72 bytes
    assert q(L, q_row=MIS) == 4
    assert q(L, x_dtype=0, ldx=34) == 4             # fp32 rows of 136 bytes


def test_quantize_noalloc_argument_errors(L):
    """The no-allocation variant checks its arguments like nvfp4_quantize,
    before any HIP call (it has no amax_ws; amax_in may be NULL)."""
    def n(**kw):
        a = dict(x=FAKE, x_dtype=1, rows=32, cols=32, ldx=32, block=0, rounding=0, seed=0,
                 offset=0, outputs=3, amax_in=FAKE, q_row=FAKE, s_row=FAKE, q_col=FAKE,
                 s_col=FAKE, tensor_scale=FAKE, dev_status=None, stream=None)
        a.update(kw)
        return L.nvfp4_quantize_noalloc(*a.values())

    assert n(x_dtype=7) == 3
    assert n(block=2) == 3
    assert n(block=1, rounding=1) == 3
    assert n(outputs=0) == 3
    assert n(cols=24, ldx=24) == 2
    assert n(rows=24) == 2
    assert n(ldx=16) == 2
    assert n(x=None) == 1
    assert n(tensor_scale=None) == 1
    assert n(amax_in=None, tensor_scale=None) == 1
    assert n(q_col=None) == 1
    assert n(x=MIS) == 4
    assert n(amax_in=MIS) == 4
    assert n(q_row=MIS) == 4


def test_stream_reference_argument_errors(L):
    assert L.nvfp4_stream_read(FAKE, 24, FAKE, None) == 2      # bytes % 16
    assert L.nvfp4_stream_read(FAKE, -16, FAKE, None) == 2
    assert L.nvfp4_stream_read(None, 64, FAKE, None) == 1
    assert L.nvfp4_stream_read(FAKE, 64, None, None) == 1
    assert L.nvfp4_stream_read(MIS, 64, FAKE, None) == 4
    assert L.nvfp4_stream_read(FAKE, 0, None, None) == 0        # nothing to read
    assert L.nvfp4_stream_copy(FAKE, FAKE + 4096, 40, None) == 2
    assert L.nvfp4_stream_copy(FAKE, None, 64, None) == 1
    assert L.nvfp4_stream_copy(FAKE, MIS + 4096, 64, None) == 4
    assert L.nvfp4_stream_copy(FAKE, FAKE + 32, 64, None) == 2  # overlapping
    assert L.nvfp4_stream_copy(FAKE, FAKE, 0, None) == 0


def test_rht_quantize_argument_errors(L):
    def r(**kw):
        a = dict(x=FAKE, x_dtype=1, tokens=32, cols=32, ldx=32, rht_seed=7, rounding=1, seed=7,
                 offset=0, amax_in=None, amax_ws=FAKE, q_t=FAKE, s_t=FAKE, tensor_scale=FAKE,
                 dev_status=None, stream=None)
        a.update(kw)
        return L.nvfp4_rht_quantize(*a.values())

    assert r(tokens=24) == 2
    assert r(cols=40, ldx=40) == 2
    assert r(rounding=5) == 3
    assert r(q_t=None) == 1
    assert r(amax_ws=None) == 1
    assert r(s_t=MIS) == 4


def test_quantize_row_rht_argument_errors(L):
    def f(**kw):
        a = dict(x=FAKE, x_dtype=1, tokens=32, cols=32, ldx=32, rht_seed=7, rounding_t=0, seed=0,
                 offset=0, amax_in=None, amax_ws=FAKE, q_row=FAKE, s_row=FAKE, ts_row=FAKE,
                 q_t=FAKE, s_t=FAKE, ts_t=FAKE, dev_status=None, stream=None)
        a.update(kw)
        return L.nvfp4_quantize_row_rht(*a.values())

    assert f(x_dtype=3) == 3
    assert f(rounding_t=2) == 3
    assert f(tokens=24) == 2                        # the Hadamard copy needs tokens % 16
    assert f(cols=40, ldx=40) == 2
    assert f(ldx=16) == 2
    assert f(x=None) == 1
    assert f(ts_row=None) == 1 and f(ts_t=None) == 1
    assert f(amax_ws=None) == 1
    assert f(q_row=None) == 1 and f(s_row=None) == 1
    assert f(q_t=None) == 1 and f(s_t=None) == 1
    assert f(x=MIS) == 4
    assert f(ts_t=MIS) == 4 and f(ts_row=MIS) == 4
    assert f(amax_in=MIS) == 4
    assert f(q_row=MIS) == 4 and f(s_t=MIS) == 4
    # an empty tensor needs no output arrays (only the two tensor scales are
    # written), so the missing arrays are accepted; nothing is launched here
    # because the check of the scale pointers comes first and fails
    assert f(tokens=0, q_row=None, s_row=None, q_t=None, s_t=None, ts_t=None) == 1


def test_dequantize_and_gemm_argument_errors(L):
    d = lambda **kw: L.nvfp4_dequantize(*dict(dict(q=FAKE, s=FAKE, ts=FAKE, rows=32, cols=32,
                                                   block=0, out=0, y=FAKE, ldy=32, st=None),
                                              **kw).values())
    assert d(cols=20, ldy=20) == 2
    assert d(ldy=16) == 2
    assert d(block=1, rows=8) == 2
    assert d(block=9) == 3
    assert d(out=3) == 3
    assert d(y=None) == 1
    assert d(q=MIS) == 4
    g = lambda **kw: L.nvfp4_gemm(*dict(dict(qa=FAKE, sa=FAKE, ta=FAKE, ab=0, qb=FAKE, sb=FAKE,
                                             tb=FAKE, bb=0, M=32, N=32, K=32, c=FAKE, cd=1,
                                             ldc=32, st=None), **kw).values())
    assert g(K=40) == 2
    assert g(ldc=16) == 2
    assert g(ab=1, M=40) == 2
    assert g(bb=1, N=24) == 2
    # 16x16-blocked operands need their row count to be a multiple of 16
    assert g(bb=1, M=300, N=520, K=80) == 2
    assert g(bb=1, M=33, N=47, K=208) == 2
    assert g(ab=1, M=33, N=48, K=208) == 2
    assert g(ab=3) == 3
    assert g(cd=2) == 3
    assert g(c=None) == 1
    assert g(qa=None) == 1
    assert g(c=FAKE + 1) == 4        # bf16 output needs 2-byte alignment only
    assert g(cd=0, c=FAKE + 2) == 4  # float32 output needs 4-byte alignment
    assert g(qa=MIS) == 4
    # empty products enqueue nothing and succeed
    assert g(M=0) == 0 and g(N=0) == 0


def test_mxfp4_argument_errors(L):
    q = lambda **kw: L.mxfp4_quantize(*dict(dict(x=FAKE, xd=1, rows=32, cols=64, ldx=64, q=FAKE,
                                                 s=FAKE, st=None), **kw).values())
    assert q(cols=48, ldx=48) == 2   # 32-element blocks
    assert q(ldx=32) == 2
    assert q(xd=5) == 3
    assert q(q=None) == 1
    assert q(s=MIS) == 4
    assert q(rows=0) == 0
    d = lambda **kw: L.mxfp4_dequantize(*dict(dict(q=FAKE, s=FAKE, rows=32, cols=64, od=0, y=FAKE,
                                                   ldy=64, st=None), **kw).values())
    assert d(cols=80, ldy=80) == 2
    assert d(od=7) == 3
    assert d(y=None) == 1
    g = lambda **kw: L.mxfp4_gemm(*dict(dict(qa=FAKE, sa=FAKE, qb=FAKE, sb=FAKE, M=32, N=32, K=128,
                                             c=FAKE, cd=1, ldc=32, st=None), **kw).values())
    assert g(K=96) == 2              # K steps of 128
    assert g(ldc=16) == 2
    assert g(cd=4) == 3
    assert g(qb=None) == 1
    assert g(qa=MIS) == 4
    assert g(N=0) == 0


def test_fp8_argument_errors(L):
    q = lambda **kw: L.fp8_quantize(*dict(dict(x=FAKE, xd=1, rows=32, cols=64, ldx=64, outputs=3,
                                               amax_in=None, ws=FAKE, q_row=FAKE, q_col=FAKE,
                                               ts=FAKE, st=None, stream=None), **kw).values())
    assert q(outputs=0) == 3 and q(outputs=4) == 3
    assert q(xd=4) == 3
    assert q(cols=40, ldx=40) == 2      # cols % 16
    assert q(rows=24) == 2              # the column copy needs rows % 16
    assert q(ldx=32) == 2
    assert q(ts=None) == 1
    assert q(ws=None) == 1
    assert q(q_col=None) == 1
    assert q(outputs=1, q_row=None) == 1
    assert q(q_row=MIS) == 4
    assert q(x=MIS) == 4
    d = lambda **kw: L.fp8_dequantize(*dict(dict(q=FAKE, ts=FAKE, rows=32, cols=64, od=0, y=FAKE,
                                                 ldy=64, st=None), **kw).values())
    assert d(cols=24, ldy=24) == 2
    assert d(od=3) == 3
    assert d(ts=None) == 1
    assert d(y=MIS) == 4
    g = lambda **kw: L.fp8_gemm(*dict(dict(qa=FAKE, ta=FAKE, qb=FAKE, tb=FAKE, M=32, N=32, K=64,
                                           c=FAKE, cd=1, ldc=32, st=None), **kw).values())
    assert g(K=96) == 2              # K steps of 64
    assert g(ldc=16) == 2
    assert g(cd=5) == 3
    assert g(tb=None) == 1
    assert g(qb=MIS) == 4
    assert g(c=FAKE + 1, cd=0) == 4
    assert g(M=0) == 0


def test_hook_argument_errors(L):
    assert L.nvfp4_philox_fill(1, 0, 0, -1, FAKE, None) == 2
    assert L.nvfp4_philox_fill(1, 0, 0, 4, None, None) == 1
    assert L.nvfp4_philox_fill(1, 0, 0, 0, None, None) == 0
    assert L.nvfp4_rht_transform(FAKE, 1, 24, 32, 32, 7, FAKE, None) == 2
    assert L.nvfp4_rht_transform(FAKE, 1, 32, 32, 32, 7, None, None) == 1


def test_amax_workspace_size_matches_header():
    """The binding's workspace size is the header's, and it refuses smaller
    buffers (the library cannot check a plain pointer)."""
    import re

    import torch

    from bit_block_scaled_bf16_amd import _lib

    text = open(os.path.join(ROOT, "include", "nvfp4.h")).read()
    m = re.search(r"#define NVFP4_AMAX_WS_BYTES (\d+)", text)
    assert m is not None and int(m.group(1)) == _lib.AMAX_WS_BYTES
    with pytest.raises(ValueError):
        _lib._ws(torch.zeros(4, dtype=torch.float32))
    assert _lib._ws(torch.zeros(_lib.AMAX_WS_BYTES // 4, dtype=torch.float32)) is not None


def test_nvfp4_linear_refuses_cpu_tensors_and_opts_out_to_bf16():
    """The NVFP4 layer has no CPU path (it raises); the bf16 opt-out is a
    plain matmul and runs anywhere."""
    import torch

    from bit_block_scaled_bf16_amd.linear import NVFP4Linear

    x = torch.randn(32, 64).to(torch.bfloat16)
    layer = NVFP4Linear(64, 16)
    with pytest.raises(RuntimeError):
        layer(x)
    off = NVFP4Linear(64, 16, nvfp4=False)
    assert torch.equal(off(x), x @ off.weight.t())


def test_header_sr_examples_match_the_oracle():
    """The worked stochastic-rounding examples in include/nvfp4.h state the
    rule the library implements; the oracle must give the same codes."""
    text = open(HEADER).read()
    lines = re.findall(r"SR example: (.*)", text)
    assert len(lines) >= 3
    checked = 0
    for line in lines:
        y = float(re.match(r"y = ([-+0-9.e]+)", line).group(1))
        for u16, code in re.findall(r"u16 = (\d+) -> code (0x[0-9A-Fa-f])", line):
            got = o.e2m1_encode_sr(np.array([y], np.float32), np.array([int(u16)]))[0]
            assert int(got) == int(code, 16), (y, u16, code, int(got))
            checked += 1
    assert checked >= 7
