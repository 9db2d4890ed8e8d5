"""GPU parity of nvfp4_quantize (1x16 / 16x1 / 16x16, RN and SR) with the
CPU oracle: scale bytes, codes, tensor scale and amax bit for bit.

Sizes are small enough for the oracle to finish in seconds while spanning
several 256 x 128 workgroup tiles and ragged tile tails; the full-size
workloads are checked on sampled rows and columns.
"""

import numpy as np
import pytest

import oracle as o
from oracle.philox import STREAM_ROW
import workloads as wl
from tests._helpers import announce, host, require_gpu, to_device

pytestmark = pytest.mark.gpu


def run_quantize(x_np, dtype, block=0, rounding=0, seed=0, offset=0, outputs=3, amax=None):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x = to_device(x_np, dtype)
    amax_t = None
    if amax is not None:
        amax_t = torch.tensor([amax, 0, 0, 0], dtype=torch.float32, device="cuda")
    row, col, ws = nv.quantize(x, block=block, rounding=rounding, seed=seed, offset=offset,
                               outputs=outputs, amax=amax_t)
    torch.cuda.synchronize()
    return row, col, ws


def check_against_oracle(x_np, dtype, rounding="rn", seed=0, offset=0, outputs=("row", "col"),
                         amax=None):
    mask = (1 if "row" in outputs else 0) | (2 if "col" in outputs else 0)
    row, col, ws = run_quantize(x_np, dtype, 0, 0 if rounding == "rn" else 1, seed, offset, mask,
                                amax)
    ref = o.quantize(x_np, rounding=rounding, seed=seed, offset=offset, outputs=outputs, amax=amax)
    some = row if row is not None else col
    s_gpu = host(some.tensor_scale)[0]
    first = next(iter(ref.values()))
    assert s_gpu.view(np.uint32) == np.float32(first.tensor_scale).view(np.uint32)
    if ws is not None:
        assert host(ws)[0].view(np.uint32) == np.float32(first.amax).view(np.uint32)
    if row is not None:
        assert np.array_equal(host(row.scales), ref["row"].scales)
        assert np.array_equal(host(row.codes), ref["row"].codes)
    if col is not None:
        assert np.array_equal(host(col.scales), ref["col"].scales)
        assert np.array_equal(host(col.codes), ref["col"].codes)


def test_fp32_outlier_matrix_rn_round_trip():
    """fp32 256x1024, N(0,1), 0.1% outliers x50, 1x16 RN + dequant."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x = wl.fp32_outlier_matrix()
    announce("fp32 256x1024 RN")
    check_against_oracle(x, "fp32", outputs=("row",))
    row, _, _ = run_quantize(x, "fp32", outputs=1)
    ref = o.quantize(x, outputs=("row",))["row"]
    deq = host(nv.dequantize(row))
    want = o.dequantize(ref.codes, ref.scales, ref.tensor_scale)
    assert np.array_equal(deq.view(np.uint32), want.view(np.uint32))
    deq16 = host(nv.dequantize(row, torch.bfloat16).float())
    want16 = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
    assert np.array_equal(deq16, want16)


# Dequantization on its own, from arbitrary stored bytes: every code pair and
# every non-NaN scale byte (0x00 zero, 0x01-0x07 E4M3 subnormals) appear.
# A wave covers 512 bf16 or 256 float32 values of a row; the shapes leave
# partial pieces at row ends (400, 1040, 528 columns), row counts that are
# not multiples of the workgroup's 4 rows (5, 33), and padded output rows.
@pytest.mark.parametrize("rows,cols,block2d,pad", [(1, 16, False, 0), (5, 400, False, 8),
                                                    (33, 1040, False, 0), (64, 528, True, 16),
                                                    (48, 4096, True, 0), (256, 5120, False, 24)])
@pytest.mark.parametrize("out", ["fp32", "bf16"])
def test_dequantize_parity(rows, cols, block2d, pad, out):
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    announce(f"dequantize {rows}x{cols} 2d={block2d} pad={pad} {out}")
    rng = np.random.default_rng(rows * 7 + cols)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    sshape = (rows // 16, cols // 16) if block2d else (rows, cols // 16)
    scales = rng.integers(0, 0x7F, size=sshape, dtype=np.uint8)  # 0x00 .. 0x7E
    scales.flat[: min(8, scales.size)] = np.arange(min(8, scales.size), dtype=np.uint8)
    ts = np.float32(0.37)
    want = o.dequantize(codes, scales, ts, block="2d" if block2d else "1d")
    dt = torch.float32 if out == "fp32" else torch.bfloat16
    elem_pad = pad if out == "fp32" else 2 * pad  # keeps the row pitch a multiple of 16 bytes
    full = torch.full((rows, cols + elem_pad), 7.0, dtype=dt, device="cuda")
    y = full[:, :cols]
    nv.nvfp4_dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                        torch.tensor([ts], device="cuda"), rows, cols,
                        nv.BLOCK_2D if block2d else nv.BLOCK_1D, y)
    got = host(full.float())
    if out == "fp32":
        assert np.array_equal(got[:, :cols].view(np.uint32), want.view(np.uint32))
    else:
        want16 = torch.from_numpy(want).to(torch.bfloat16).float().numpy()
        assert np.array_equal(got[:, :cols], want16)
    assert np.all(got[:, cols:] == 7.0)  # the padding is untouched


# (2320, 400): 10 tile rows, i.e. a full band of 8 and a band of 2 whose
# last tile is ragged (tiles go to the XCDs in bands walked column by column)
@pytest.mark.parametrize("shape", [(16, 16), (48, 160), (272, 400), (528, 272), (2320, 400)])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_dual_rn_ragged_tiles(shape, dtype):
    announce(f"dual RN {shape} {dtype}")
    x = wl.normal(shape, seed=shape[0] + shape[1], outlier_channels=min(4, shape[1] // 16),
                  dtype=dtype)
    check_against_oracle(x, dtype)


@pytest.mark.parametrize("outputs", [("row",), ("col",)])
def test_single_orientation(outputs):
    x = wl.activation(272, 400, seed=11)
    announce(f"single {outputs}")
    check_against_oracle(x, "bf16", outputs=outputs)


def test_row_only_needs_no_row_multiple_of_16():
    x = wl.normal((37, 64), seed=3)
    announce("row-only 37x64")
    check_against_oracle(x, "bf16", outputs=("row",))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_sr_bit_exact(dtype):
    x = wl.laplace((272, 400), seed=5, dtype=dtype)
    announce(f"SR {dtype}")
    check_against_oracle(x, dtype, rounding="sr", seed=7, offset=3)
    check_against_oracle(x, dtype, rounding="sr", seed=(1 << 40) + 9, offset=0xFFFFFFFF)


def _sr_boundary_matrix(rows, cols, seed, offset, stream):
    """A float32 matrix whose SR decisions sit on their boundaries.

    The tensor amax is 2688 (S = 1) and every 16-block holds a 6.0, so
    s_f = 1 and y = x exactly. The other elements are built from the random
    word u that the oracle's Philox gives their index, with
    k = 2^16 - u:
      kind 0: y = (256 k - 1) 2^-25 < 0.5, so frac 2^16 = k - 2^-8 and the
              element rounds down; rounding y * 2^23 to nearest instead of
              toward zero would round it up;
      kind 1: y = k 2^-17, frac 2^16 = k exactly: rounds up;
      kind 2: y = 1 + k 2^-17 - 2^-23 in [1, 2): rounds down;
      kind 3: y = 1 + k 2^-17: rounds up;
      kind 4: y in (6, 6.375]: saturates at 6;
      kind 5: y = 2^-140 (a float32 subnormal): rounds to 0;
    each with a random sign. Returns (x, expected magnitude codes, mask of
    the constructed elements)."""
    rng = np.random.default_rng(11)
    e = np.arange(rows * cols, dtype=np.int64).reshape(rows, cols)
    u = o.sr_random_u16(seed, offset, stream, e).astype(np.int64)
    k = 65536 - u
    kind = rng.integers(0, 6, (rows, cols))
    mag = np.select(
        [kind == 0, kind == 1, kind == 2, kind == 3, kind == 4],
        [(256.0 * k - 1.0) * 2.0 ** -25, k * 2.0 ** -17, 1.0 + k * 2.0 ** -17 - 2.0 ** -23,
         1.0 + k * 2.0 ** -17, rng.uniform(6.0001, 6.375, (rows, cols))],
        2.0 ** -140)
    want = np.select(
        [kind == 0, kind == 1, kind == 2, kind == 3, kind == 4],
        [np.zeros_like(k), np.where(k == 65536, 1, 1), np.where(k * 2 >= 65536, 2, 2),
         np.where(1.0 + k * 2.0 ** -17 >= 1.5, 4, 3), np.full_like(k, 7)], 0)
    # kind 2 stays on its lower grid point: 1.0, or 1.5 when y >= 1.5
    want = np.where((kind == 2) & (mag >= 1.5), 3, want)
    # kind 3: the grid point above y (1.5 below 1.5, 2.0 from 1.5 on)
    want = np.where(kind == 3, np.where(mag >= 1.5, 4, 3), want)
    x = (mag * np.where(rng.integers(0, 2, (rows, cols)) == 1, -1.0, 1.0)).astype(np.float32)
    x[:, ::16] = 6.0
    x[0, 0] = 2688.0
    built = np.ones((rows, cols), bool)
    built[:, ::16] = False
    built[0, :16] = False  # the block holding the tensor amax has another scale
    return x, want, built


def test_sr_decisions_on_their_boundaries():
    """Row-blocked SR at the exact decision boundaries (see the matrix
    builder): the kernel's codes equal the oracle's, and both equal the
    codes the rule prescribes."""
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    rows, cols, seed, offset = 64, 512, 7, 5
    x, want, built = _sr_boundary_matrix(rows, cols, seed, offset, STREAM_ROW)
    announce("SR boundary values")
    ref = o.quantize(x, rounding="sr", seed=seed, offset=offset, outputs=("row",))["row"]
    ref_codes = o.unpack_codes(ref.codes)
    assert np.all(ref.scales[1:] == 0x38) and np.all(ref.scales[0, 1:] == 0x38)
    assert np.array_equal((ref_codes & 7)[built], want[built].astype(np.uint8))
    row, _, _ = nv.quantize(to_device(x, "fp32"), rounding=nv.ROUND_SR, seed=seed, offset=offset,
                            outputs=nv.OUT_ROW)
    assert np.array_equal(host(row.scales), ref.scales)
    assert np.array_equal(o.unpack_codes(host(row.codes)), ref_codes)


def test_caller_supplied_amax():
    x = wl.activation(256, 256, seed=12)
    announce("amax_in")
    a = float(np.max(np.abs(x)))
    check_against_oracle(x, "bf16", amax=a)
    # a smaller amax saturates blocks; still bit-exact with the same definition
    check_against_oracle(x, "bf16", amax=a / 3)


@pytest.mark.parametrize("shape", [(16, 16), (272, 400), (512, 384), (2320, 384)])
def test_2d_weight_blocks(shape):
    announce(f"2D {shape}")
    x = wl.weight(*shape, seed=4)
    row, col, _ = run_quantize(x, "bf16", block=1, outputs=3)
    ref = o.quantize_2d(x)
    assert np.array_equal(host(row.scales), ref["row"].scales)
    assert np.array_equal(host(col.scales), ref["col"].scales)
    assert np.array_equal(host(row.codes), ref["row"].codes)
    assert np.array_equal(host(col.codes), ref["col"].codes)
    # W and W^T decode to transposes of each other, bit for bit
    import bit_block_scaled_bf16_amd as nv

    d = host(nv.dequantize(row))
    dt = host(nv.dequantize(col))
    assert np.array_equal(d.T, dt)


def test_golden_blocks_on_gpu():
    import json, os

    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_blocks.json")))
    case = g["row_case"]
    x = np.concatenate([np.array(b["values"], dtype=np.float32) for b in case["blocks"]])[None, :]
    announce("golden")
    for dtype in ("fp32",):
        row, _, _ = run_quantize(x, dtype, outputs=1)
        assert [int(v) for v in host(row.scales)[0]] == [int(b["scale"], 16) for b in case["blocks"]]
        codes = o.unpack_codes(host(row.codes))[0]
        assert codes.tolist() == sum((b["codes"] for b in case["blocks"]), [])


def test_rn_sweep_of_ties_through_the_kernel():
    """Every float32 within 600 ulps of each E2M1 tie and grid point, fed
    through the full kernel with S = 1 and block multiplier 1 (each 16-block
    holds a 6.0 and the tensor holds 2688), so y == x."""
    ties = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    pts = np.asarray(ties, dtype=np.float32).view(np.int32)
    k = np.arange(-600, 601, dtype=np.int32)
    vals = (pts[:, None] + k[None, :]).reshape(-1).view(np.float32)
    vals = vals[np.abs(vals) <= 6.0]
    vals = np.concatenate([vals, -vals, np.float32([0.0, -0.0, 1e-40, -1e-40])])
    nblk = -(-len(vals) // 15)
    body = np.zeros(nblk * 15, np.float32)
    body[: len(vals)] = vals
    blocks = np.concatenate([np.full((nblk, 1), 6.0, np.float32), body.reshape(nblk, 15)], axis=1)
    flat = blocks.reshape(-1)
    cols = 256
    rows = -(-(len(flat) + 16) // cols)
    rows += (-rows) % 16
    x = np.zeros(rows * cols, np.float32)
    x[:16] = np.float32(2688.0)
    x[16:16 + len(flat)] = flat
    x = x.reshape(rows, cols)
    announce(f"tie sweep {x.shape}")
    check_against_oracle(x, "fp32", outputs=("row",))


@pytest.mark.parametrize("k", [-75, -60, -53, -50, -20, 0, 40, 100])
def test_block_scale_division_across_tensor_scales(k):
    """The same tensor scaled by 2^k (exactly) through every quantizer mode:
    the kernels divide block maxima by 6 S with a reciprocal and one
    correction step where 6 S >= 2^-60 (|x| up to about 2^-52 and above),
    and with an IEEE division below; both must give the oracle's bytes."""
    x = (wl.activation(528, 400, seed=31) * np.float32(2.0 ** k)).astype(np.float32)
    assert np.all(np.isfinite(x))
    announce(f"division 2^{k}")
    check_against_oracle(x, "fp32")
    check_against_oracle(x, "fp32", rounding="sr", seed=3, offset=1, outputs=("row",))
    for dtype in ("fp32", "bf16"):
        xb = x if dtype == "fp32" else wl.to_bf16_values(x)
        row, col, _ = run_quantize(xb, dtype, block=1, outputs=3)
        ref = o.quantize_2d(xb)
        assert np.array_equal(host(row.scales), ref["row"].scales)
        assert np.array_equal(host(row.codes), ref["row"].codes)
        assert np.array_equal(host(col.codes), ref["col"].codes)


def test_zero_tiny_and_empty_tensors():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    for v in (0.0, -0.0, 1e-31):
        x = np.full((32, 64), v, np.float32)
        announce(f"constant {v}")
        check_against_oracle(x, "fp32")
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    row, col, ws = nv.quantize(x, outputs=1)
    assert host(row.tensor_scale)[0] == 1.0 and host(ws)[0] == 0.0


def test_non_finite_amax_sets_status():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    x = np.zeros((32, 32), np.float32)
    x[5, 7] = np.inf
    status = torch.zeros(4, dtype=torch.int32, device="cuda")
    nv.quantize(to_device(x, "fp32"), dev_status=status)
    assert host(status)[0] == 1
    status.zero_()
    nv.quantize(to_device(np.ones((32, 32), np.float32), "fp32"), dev_status=status)
    assert host(status)[0] == 0


def test_deterministic_repeat():
    x = wl.laplace((512, 256), seed=9)
    announce("determinism")
    r1, c1, _ = run_quantize(x, "bf16", rounding=1, seed=7)
    r2, c2, _ = run_quantize(x, "bf16", rounding=1, seed=7)
    assert np.array_equal(host(r1.codes), host(r2.codes))
    assert np.array_equal(host(c1.codes), host(c2.codes))


def test_leading_dimension():
    torch = require_gpu()
    import bit_block_scaled_bf16_amd as nv

    big = wl.normal((64, 200), seed=21)
    x = to_device(big, "bf16")[:, :160]  # ldx = 200 (400 bytes, 16-aligned)
    announce("ldx")
    row, col, _ = nv.quantize(x)
    ref = o.quantize(np.ascontiguousarray(big[:, :160]))
    assert np.array_equal(host(row.codes), ref["row"].codes)
    assert np.array_equal(host(col.codes), ref["col"].codes)


# ---------------------------------------------------------------------------
# Full-size workloads, checked on sampled rows / columns.
# ---------------------------------------------------------------------------


def _sampled_rows_check(x, row, col, s, rows_idx, cols_idx):
    """Row copy on sampled rows, column copy on sampled columns, given S."""
    for r in rows_idx:
        codes, sb = o.quantize_rows(x[r:r + 1], s)
        assert np.array_equal(host(row.codes[r:r + 1]), o.pack_codes(codes)), r
        assert np.array_equal(host(row.scales[r:r + 1]), sb), r
    xt = x[:, cols_idx].T.copy()
    codes, sb = o.quantize_rows(xt, s)
    assert np.array_equal(host(col.codes[cols_idx]), o.pack_codes(codes))
    assert np.array_equal(host(col.scales[cols_idx]), sb)


def test_full_activation_dual_rn():
    """bf16 8192x5120, N(0,1) + 16 outlier channels x20, row and column
    copies in one pass; sampled rows and columns checked bit for bit."""
    x = wl.activation()
    announce("full activation 8192x5120")
    row, col, ws = run_quantize(x, "bf16", outputs=3)
    a = np.float32(np.max(np.abs(x)))
    s = o.tensor_scale(a)
    assert host(ws)[0] == a
    assert host(row.tensor_scale)[0] == s
    rng = np.random.default_rng(0)
    _sampled_rows_check(x, row, col, s, rng.choice(x.shape[0], 24, replace=False),
                        np.sort(rng.choice(x.shape[1], 48, replace=False)))


def test_full_weight_2d():
    """bf16 20480x5120 weight, N(0, 0.02^2), 16x16 blocks, both orientations;
    sampled 16-row bands checked bit for bit, W^T identity on a band."""
    x = wl.weight()
    announce("full weight 20480x5120")
    row, col, _ = run_quantize(x, "bf16", block=1, outputs=3)
    a = np.float32(np.max(np.abs(x)))
    rng = np.random.default_rng(1)
    grid_row = host(row.scales)
    grid_col = host(col.scales)
    assert np.array_equal(grid_row.T, grid_col)
    for band in rng.choice(x.shape[0] // 16, 6, replace=False):
        sl = slice(16 * band, 16 * band + 16)
        ref = o.quantize_2d(x[sl], amax=a)
        assert np.array_equal(host(row.codes[sl]), ref["row"].codes)
        assert np.array_equal(grid_row[band:band + 1], ref["row"].scales)
        colcodes = host(col.codes[:, 8 * band: 8 * band + 8])
        assert np.array_equal(colcodes, ref["col"].codes)
