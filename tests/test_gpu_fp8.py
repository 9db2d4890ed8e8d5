"""GPU parity of the FP8 (E4M3, one scale per tensor) baseline path with the
oracle: the quantizer's row and column copies, the decode scale and the
amax bit for bit; the dequantizer bit for bit; the GEMM on the FP8 MFMA
within relative Frobenius error <= 1e-2 (the NVFP4 GEMM's bar) and a
per-element bound.

The per-element bound has one term more than the NVFP4 GEMM's. The FP8 MFMA
does not reduce its K = 64 slice like a float32 sum of exact products: with
all-positive operands its result is within one float32 rounding of the exact
sum, but under cancellation its error is up to about 2^-13 of the slice's
largest product (seen on N(0,1) data with outlier channels), the signature
of products aligned to the largest one in a window of about 14 bits. The
bound therefore adds (K / 64) 2^-12 max|a| max|b| (row maxima) to the output
rounding and the float32 accumulation bound of the slices."""

import numpy as np
import pytest

import oracle as o
import workloads as wl
from tests._helpers import announce, host, require_gpu, to_device
from tests.test_gpu_gemm import check


def check_fp8(c_gpu, ra, rb, s, bf16=True):
    """ra [M, K], rb [N, K]: decoded E4M3 operands; s = S8_a * S8_b."""
    k = ra.shape[1]
    ref = (ra @ rb.T) * s
    absref = (np.abs(ra) @ np.abs(rb).T) * s
    c = c_gpu.astype(np.float64)
    fro = np.linalg.norm(c - ref) / max(np.linalg.norm(ref), 1e-30)
    assert fro <= 1e-2, fro
    rel = 2.0 ** -8 if bf16 else 2.0 ** -22
    slice_term = (k / 64) * 2.0 ** -12 * np.outer(np.max(np.abs(ra), axis=1),
                                                 np.max(np.abs(rb), axis=1)) * s
    bound = rel * np.abs(ref) + k * 2.0 ** -23 * absref + slice_term + 1e-30
    assert np.all(np.abs(c - ref) <= bound), float(np.max(np.abs(c - ref) / bound))
    return ref

pytestmark = pytest.mark.gpu


def run_f8(x_np, dtype, outputs=3, amax=None, pad_cols=0):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    rows, cols = x_np.shape
    if pad_cols:
        big = np.zeros((rows, cols + pad_cols), np.float32)
        big[:, :cols] = x_np
        xd = to_device(big, dtype)[:, :cols]
    else:
        xd = to_device(x_np, dtype)
    q_row = torch.empty((rows, cols), dtype=torch.uint8, device="cuda") if outputs & 1 else None
    q_col = torch.empty((cols, rows), dtype=torch.uint8, device="cuda") if outputs & 2 else None
    ts = torch.zeros(4, dtype=torch.float32, device="cuda")
    ws = nv.amax_workspace("cuda")
    st = torch.zeros(4, dtype=torch.int32, device="cuda")
    amax_t = None if amax is None else torch.tensor([amax, 0, 0, 0], dtype=torch.float32, device="cuda")
    nv.fp8_quantize(xd, outputs, amax_t, ws, q_row, q_col, ts, st)
    return q_row, q_col, ts, ws, st


def check_f8(x_np, dtype, outputs=3, amax=None, pad_cols=0):
    x_np = np.asarray(x_np, np.float32)
    q_row, q_col, ts, ws, st = run_f8(x_np, dtype, outputs, amax, pad_cols)
    rq, rqt, rs = o.fp8_quantize(x_np, amax=amax)
    assert host(ts)[0].view(np.uint32) == np.float32(rs).view(np.uint32)
    if amax is None:
        want_amax = np.float32(np.max(np.abs(x_np))) if x_np.size else np.float32(0)
        assert host(ws)[0].view(np.uint32) == want_amax.view(np.uint32)
    if outputs & 1:
        assert np.array_equal(host(q_row), rq)
    if outputs & 2:
        assert np.array_equal(host(q_col), rqt)
    assert host(st)[0] == 0
    return q_row, q_col, ts, rq, rs


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("rows,cols,outputs", [(1, 16, 1), (8, 64, 1), (37, 1024, 1), (16, 16, 3),
                                               (64, 256, 3), (304, 5120, 3), (1040, 272, 3),
                                               (80, 48, 2)])
def test_fp8_quantize_parity(dtype, rows, cols, outputs):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    announce(f"fp8 quantize {rows}x{cols} {dtype} outputs={outputs}")
    x = wl.normal((rows, cols), seed=rows + 3 * cols, outlier_channels=min(4, cols // 16),
                  dtype=dtype)
    q_row, _, ts, rq, rs = check_f8(x, dtype, outputs)
    if q_row is not None:
        want = o.fp8_dequantize(rq, rs)
        assert np.array_equal(host(nv.f8_dequantize(q_row, ts)), want)
        wb = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
        assert np.array_equal(host(nv.f8_dequantize(q_row, ts, torch.bfloat16).float()), wb)


def test_fp8_every_tie_and_grid_point():
    """amax = 448 makes S8 = 1 and y = x: every float32 within 6 ulps of every
    E4M3 value and midpoint, both signs, signed zeros and subnormal-range
    values, through the kernel's own rounding."""
    require_gpu()
    vals = o.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    pts = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2])
    near = []
    for m in pts:
        b = int(np.float32(m).view(np.uint32))
        near.append((np.arange(-6, 7, dtype=np.int64) + b).astype(np.uint32).view(np.float32))
    y = np.concatenate(near)
    y = y[np.isfinite(y) & (np.abs(y) <= 448.0)]
    y = np.concatenate([y, -y, np.array([448.0, -0.0, 0.0, 1e-30, -1e-30], np.float32)])
    cols = 1024
    n = -(-y.size // cols) * cols
    x = np.zeros(n, np.float32)
    x[:y.size] = y
    x = x.reshape(-1, cols)
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 16, cols), np.float32)])
    announce(f"fp8 tie sweep {x.shape}")
    check_f8(x, "fp32", 3)


def test_fp8_strided_input_caller_amax_and_saturation():
    require_gpu()
    x = wl.normal((96, 320), seed=4, dtype="bf16")
    announce("fp8 strided / amax_in")
    check_f8(x, "bf16", 3, pad_cols=64)
    a = np.float32(np.max(np.abs(x)))
    check_f8(x, "bf16", 3, amax=a)
    check_f8(x, "bf16", 3, amax=np.float32(a / 5))  # most of the tail saturates at 448
    z = np.zeros((32, 64), np.float32)
    q_row, _, ts, _, _ = check_f8(z, "fp32", 3)  # amax 0: S8 = 1, all bytes 0
    assert host(ts)[0] == 1.0 and not host(q_row).any()


def test_fp8_empty_and_non_finite():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    ts = torch.zeros(4, dtype=torch.float32, device="cuda")
    ws = nv.amax_workspace("cuda")
    nv.fp8_quantize(x, 1, None, ws, None, None, ts)
    assert host(ts)[0] == 1.0
    y = np.ones((32, 32), np.float32)
    y[3, 5] = np.inf
    _, _, ts, _, st = run_f8(y, "fp32", 1)
    assert host(st)[0] == 1


@pytest.mark.parametrize("m,n,k", [(32, 32, 64), (256, 256, 64), (300, 520, 128), (33, 47, 192),
                                   (512, 768, 1024), (2500, 2608, 512), (272, 256, 5120),
                                   (3072, 6144, 128), (4096, 5120, 128)])
def test_fp8_gemm_parity(m, n, k):
    """(3072, 6144, 128): 12 x 24 tiles, nine 4 x 8 tile blocks: eight handed
    to the XCDs together, one after them in plain order. (4096, 5120, 128):
    16 x 20 tiles, ten 8 x 4 blocks."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    announce(f"fp8 gemm {m}x{n}x{k}")
    a = wl.normal((m, k), seed=m + k, outlier_channels=4 if k >= 256 else 0)
    b = wl.normal((n, k), seed=n + k + 1)
    qa, _, ta = nv.f8_quantize(to_device(a, "bf16"))
    qb, _, tb = nv.f8_quantize(to_device(b, "bf16"))
    sa, sb = float(host(ta)[0]), float(host(tb)[0])
    ra = o.e4m3_decode(host(qa))
    rb = o.e4m3_decode(host(qb))
    check_fp8(host(nv.f8_gemm(qa, ta, qb, tb).float()), ra, rb, sa * sb)
    c32 = host(nv.f8_gemm(qa, ta, qb, tb, out_dtype=torch.float32))
    ref = check_fp8(c32, ra, rb, sa * sb, bf16=False)
    # the oracle's own product is that reference rounded once to float32
    want = o.fp8_gemm(host(qa), sa, host(qb), sb)
    assert np.array_equal(want, ref.astype(np.float32))


def test_fp8_gemm_positive_operands_round_once():
    """All-positive operands (no cancellation): the GEMM is within the
    float32 accumulation bound of the exact product, with no slice term."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    rng = np.random.default_rng(1)
    a = rng.uniform(0.5, 1.0, (256, 1024)).astype(np.float32)
    b = rng.uniform(0.5, 1.0, (320, 1024)).astype(np.float32)
    qa, _, ta = nv.f8_quantize(to_device(a, "bf16"))
    qb, _, tb = nv.f8_quantize(to_device(b, "bf16"))
    ra, rb = o.e4m3_decode(host(qa)), o.e4m3_decode(host(qb))
    s = float(host(ta)[0]) * float(host(tb)[0])
    c32 = host(nv.f8_gemm(qa, ta, qb, tb, out_dtype=torch.float32))
    check(c32, (ra @ rb.T) * s, (np.abs(ra) @ np.abs(rb).T) * s, 1024, bf16=False)


def test_fp8_gemm_k_zero_writes_zeros():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    c = torch.full((40, 72), 7.0, dtype=torch.float32, device="cuda")
    t = torch.ones(4, dtype=torch.float32, device="cuda")
    nv.fp8_gemm(None, t, None, t, 40, 72, 0, c)
    assert not host(c).any()


def test_fp8_full_fprop_sampled():
    """FP8 operands of the linear layer's fprop (X 16384 x 5120, W 20480 x
    5120) and X's column copy: sampled rows against the oracle."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x_np, w_np, _ = wl.linear_layer()
    announce("fp8 full fprop 16384x20480x5120")
    xd = to_device(x_np, "bf16")
    qa, qat, ta = nv.f8_quantize(xd, nv.OUT_ROW | nv.OUT_COL)
    qb, _, tb = nv.f8_quantize(to_device(w_np, "bf16"))
    c = nv.f8_gemm(qa, ta, qb, tb)
    torch.cuda.synchronize()
    ax, aw = np.float32(np.max(np.abs(x_np))), np.float32(np.max(np.abs(w_np)))
    rows = np.sort(np.random.default_rng(8).choice(x_np.shape[0], 16, replace=False))
    wrows = np.sort(np.random.default_rng(10).choice(w_np.shape[0], 64, replace=False))
    rq, _, rs = o.fp8_quantize(x_np[rows], amax=ax)
    rqw, _, rsw = o.fp8_quantize(w_np[wrows], amax=aw)
    assert host(ta)[0] == rs and host(tb)[0] == rsw
    idx = torch.as_tensor(rows, device="cuda")
    widx = torch.as_tensor(wrows, device="cuda")
    assert np.array_equal(host(qa[idx]), rq)
    assert np.array_equal(host(qb[widx]), rqw)
    cols = np.sort(np.random.default_rng(9).choice(x_np.shape[1], 16, replace=False))
    rqc, _, _ = o.fp8_quantize(x_np[:, cols], amax=ax)
    assert np.array_equal(host(qat[torch.as_tensor(cols, device="cuda")]), rqc.T)
    got = host(c[idx][:, widx].float())
    check_fp8(got, o.e4m3_decode(rq), o.e4m3_decode(rqw), float(rs) * float(rsw))


def test_fp8_error_below_nvfp4():
    """The baseline's quantization error on the linear layer's activation:
    FP8's 3 mantissa bits give a smaller error than NVFP4's 1."""
    require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x_np = wl.normal((2048, 5120), seed=5, outlier_channels=16, channel_gain=20.0)
    x = to_device(x_np, "bf16")
    q, _, ts = nv.f8_quantize(x)
    err_f8 = np.mean((host(nv.f8_dequantize(q, ts)) - x_np) ** 2)
    row, _, _ = nv.quantize(x, outputs=nv.OUT_ROW)
    err_nv = np.mean((host(nv.dequantize(row)) - x_np) ** 2)
    announce(f"mse fp8 {err_f8:.4e} nvfp4 {err_nv:.4e}")
    assert err_f8 < err_nv
