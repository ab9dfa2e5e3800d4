"""GPU path vs CPU oracle, element by element, through the C ABI (small and ragged shapes).

Codes and scales must be bit-exact; dequantized values bit-exact; GEMM outputs within
|gpu - exact| <= 2^-20 * sum_k |a_k b_k| (fp32 out) or the bf16 rounding bracket of that bound.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from tests.parity import assert_bytes_equal, check_gemm, host

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def mx():
    import mxfp4_block_scaled_hadamard32_amd as m
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    m.lib()
    return m


def special_input(rows, cols, dtype, seed):
    """t(3) data with outlier columns, an all-zero block, signed zeros, fp32-subnormal-range
    values, large magnitudes and exact ties at the grid midpoints."""
    x = wl.student_t3((rows, cols), seed=seed)
    wl.outlier_columns(x, max(1, cols // 64), 100.0, seed=seed)
    x[0, :32] = 0.0
    if rows > 2:
        x[1, :32] = -0.0
        x[2, :32] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0] * 4) * 2.0 ** -3
        x[2, 5] = 6.0
    if rows > 3 and cols >= 64:
        x[3, 32:64] = torch.linspace(-1, 1, 32) * 1e-39  # fp32 subnormals
    if rows > 4 and cols >= 96:
        x[4, 64:96] = torch.linspace(-3, 3, 32) * 1e30
    x = x.to(dtype)
    return x


def hostx(x):
    return wl.host_input(x)


QUANT_CASES = [
    # rows, cols, axis, dtype
    (64, 96, 1, torch.bfloat16),
    (96, 256, 1, torch.float32),
    (40, 544, 1, torch.bfloat16),   # rows not a multiple of 32, ragged chunk tail
    (72, 160, 1, torch.float32),    # 360 blocks: the last wave of 64 lanes is partial (fp32 pieces)
    (8, 64, 1, torch.bfloat16),     # 16 blocks: one partial wave
    (64, 96, 0, torch.bfloat16),
    (96, 136, 0, torch.float32),    # cols not a multiple of 128 (ragged lane groups)
    (160, 392, 0, torch.bfloat16),
    (544, 264, 0, torch.bfloat16),  # three 256-row tiles, the last partial; ragged columns
]
OPTS = [
    # scale_rule, round, hadamard, sign_mask
    (0, 0, 0, 0),
    (1, 0, 0, 0),
    (1, 1, 0, 0),
    (1, 1, 1, 0x9E3779B9),
    (0, 0, 1, 0),
    (1, 0, 1, 0xFFFFFFFF),
]


@pytest.mark.parametrize("rows,cols,axis,dtype", QUANT_CASES)
@pytest.mark.parametrize("rule,rnd,had,mask", OPTS)
def test_quantize_1d_bit_exact(mx, orc, rows, cols, axis, dtype, rule, rnd, had, mask):
    x = special_input(rows, cols, dtype, seed=rows * 7 + cols)
    seed = 1234 + rows
    c, s = mx.mx_quantize(x.to(DEV), axis=axis, scale_rule=rule, round=rnd, hadamard=had,
                          sign_mask=mask, seed=seed)
    torch.cuda.synchronize()
    rc, rs = orc.quantize(hostx(x), axis=axis, scale_rule=rule, round_mode=rnd, hadamard=had,
                          sign_mask=mask, seed=seed)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(c, rc, "codes")


@pytest.mark.parametrize("rule,rnd,had,mask", [(1, 1, 1, 0x9E3779B9), (0, 0, 0, 0), (1, 0, 1, 0)])
def test_quantize_rows_many_waves_ragged_last(mx, orc, rule, rnd, had, mask):
    """Contiguous bf16 rows over more waves than the GPU holds at once (8192 x 64 blocks), the
    last wave holding 4 blocks."""
    x = special_input(4100, 4128, torch.bfloat16, seed=41)
    assert (4100 * 4128 // 32) % 64 == 4 and 4100 * 4128 // 32 > 8192 * 64
    c, s = mx.mx_quantize(x.to(DEV), axis=1, scale_rule=rule, round=rnd, hadamard=had,
                          sign_mask=mask, seed=1234)
    rc, rs = orc.quantize(hostx(x), axis=1, scale_rule=rule, round_mode=rnd, hadamard=had,
                          sign_mask=mask, seed=1234, nthreads=8)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(c, rc, "codes")


@pytest.mark.parametrize("axis", [1, 0])
def test_quantize_strided_rows(mx, orc, axis):
    """ld > cols: a column slice of a wider tensor."""
    big = special_input(64, 320, torch.bfloat16, seed=5).to(DEV)
    x = big[:, 64:256]
    c, s = mx.mx_quantize(x, axis=axis, scale_rule=1, round=1, hadamard=1, sign_mask=0x12345678,
                          seed=77)
    rc, rs = orc.quantize(hostx(x.contiguous()), axis=axis, scale_rule=1, round_mode=1, hadamard=1,
                          sign_mask=0x12345678, seed=77)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(c, rc, "codes")


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_strided_rows_hadamard_sr(mx, orc, dtype):
    """ld > cols with row counts that leave partial waves: blocks loaded per lane."""
    big = special_input(72, 416, dtype, seed=6).to(DEV)
    x = big[:, 32:352]
    c, s = mx.mx_quantize(x, axis=1, scale_rule=1, round=1, hadamard=1, sign_mask=0xA5A50F0F,
                          seed=78)
    rc, rs = orc.quantize(hostx(x.contiguous()), axis=1, scale_rule=1, round_mode=1, hadamard=1,
                          sign_mask=0xA5A50F0F, seed=78)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(c, rc, "codes")


@pytest.mark.parametrize("rnd", [1, 0])
@pytest.mark.parametrize("had,rule", [(1, 1), (0, 1), (1, 0)])
def test_quantize_columns_strided_ragged(mx, orc, had, rule, rnd):
    """Down the columns of a bf16 slice (ld > cols): 200 columns leave a last column tile of 8
    (64-column tiles with SR, 128-column tiles with two waves per row block for nearest-even,
    whose second half then has no columns), and 288 rows a last 256-row tile of one row block."""
    big = special_input(288, 360, torch.bfloat16, seed=9).to(DEV)
    x = big[:, 40:240]
    opts = dict(scale_rule=rule, hadamard=had, sign_mask=0x9E3779B9 if had else 0, seed=4321)
    c, s = mx.mx_quantize(x, axis=0, round=rnd, **opts)
    rc, rs = orc.quantize(hostx(x.contiguous()), axis=0, round_mode=rnd, **opts)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(c, rc, "codes")


def fold_boundary_blocks(nblk, had, seed):
    """nblk 32-element blocks (one per row of the result) whose scale exponents straddle the
    bounds of the SR kernels' folded scaling (e in [-104, 16]), with bf16 subnormal elements.
    Without the transform: [M, t1 .. t31], M = 2^k or 1.5 2^k, t_j in {0, +-2^-133, +-2^-132,
    +-3 2^-133}. With it (no random signs): [A, A, s2 .. s31], whose odd outputs are exactly the
    transform of the small part (multiples of 2^-133, some of them +-2^-133) and even outputs
    2A. Half of the blocks sit at e = 14 .. 19, the rest from e = -110 to 21."""
    g = torch.Generator().manual_seed(seed)
    k = torch.randint(-108, 24, (nblk,), generator=g)
    near = torch.rand(nblk, generator=g) < 0.5
    k = torch.where(near, torch.randint(16, 22, (nblk,), generator=g), k)
    m = torch.where(torch.rand(nblk, generator=g) < 0.5, 1.0, 1.5) * torch.pow(2.0, k.double())
    tiny = torch.tensor([0.0, 2.0 ** -133, -2.0 ** -133, 2.0 ** -132, -2.0 ** -132,
                         3 * 2.0 ** -133, -3 * 2.0 ** -133], dtype=torch.float64)
    small = tiny[torch.randint(0, len(tiny), (nblk, 32), generator=g)]
    if had:
        small[:, :2] = 0.0
        small[:, 0] = m
        small[:, 1] = m
    else:
        small[:, 0] = m
    return small.to(torch.float32).to(torch.bfloat16)


@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("had", [0, 1])
@pytest.mark.parametrize("rule", [0, 1])
def test_sr_scale_fold_boundaries(mx, orc, axis, had, rule):
    """The SR kernels fold the block scale into the rounding for bf16 input unless the scale
    exponent is above 16 or below -104; there, elements as small as 2^-133 scale to 2^-150 and
    below, which round to zero first. 2^18 blocks (8M elements): a wrong bound would show on
    the ~1 in 65536 elements whose random field is zero."""
    blocks = fold_boundary_blocks(1 << 18, had, seed=11 + 2 * had + rule)
    x = blocks.reshape(512, 512 * 32)  # row c: blocks 512c .. 512c + 511
    if axis == 0:
        x = x.t().contiguous()  # the same blocks down the columns
    opts = dict(scale_rule=rule, hadamard=had, sign_mask=0, seed=97)
    c, s = mx.mx_quantize(x.to(DEV), axis=axis, round=1, **opts)
    rc, rs = orc.quantize(hostx(x), axis=axis, round_mode=1, nthreads=8, **opts)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(c, rc, "codes")


@pytest.mark.parametrize("axis", [1, 0])
@pytest.mark.parametrize("rnd", [0, 1])
def test_hadamard_overflow_block(mx, orc, axis, rnd):
    """Finite inputs near the fp32 limit whose transform overflows: sums reach infinity, and
    infinity minus infinity gives NaN in some outputs while others stay finite. The block
    maximum must see the NaN and infinity outputs exactly as the oracle does."""
    x = wl.student_t3((64, 96), seed=10)
    big = 3.0e38
    x[5, 0:8] = torch.tensor([big, big, big, big, big, big, -big, -big])
    x[9, 32:40] = torch.tensor([big, big, -big, -big, big, -big, big, -big])
    x[13, 64:96] = big
    if axis == 0:
        x = x.t().contiguous()
    c, s = mx.mx_quantize(x.to(DEV), axis=axis, scale_rule=1, round=rnd, hadamard=1,
                          sign_mask=0x0F0F3C3C, seed=91)
    rc, rs = orc.quantize(hostx(x), axis=axis, scale_rule=1, round_mode=rnd, hadamard=1,
                          sign_mask=0x0F0F3C3C, seed=91)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(c, rc, "codes")


def test_non_finite_block(mx, orc):
    x = wl.student_t3((32, 64), seed=9)
    x[3, 40] = float("inf")
    x[7, 2] = float("nan")
    for axis in (1, 0):
        c, s = mx.mx_quantize(x.to(DEV), axis=axis, scale_rule=1)
        rc, rs = orc.quantize(hostx(x), axis=axis, scale_rule=1)
        assert_bytes_equal(s, rs, "scales")
        assert_bytes_equal(c, rc, "codes")
        assert (host(s) == 0xFF).sum() == (2 if axis == 1 else 2)


@pytest.mark.parametrize("rows,cols,dtype", [(64, 64, torch.bfloat16), (96, 160, torch.float32),
                                             (256, 384, torch.bfloat16),
                                             (288, 544, torch.bfloat16)])  # partial 256x256 tiles
@pytest.mark.parametrize("rule,rnd", [(1, 0), (1, 1), (0, 0)])
def test_quantize_2d_bit_exact(mx, orc, rows, cols, dtype, rule, rnd):
    x = special_input(rows, cols, dtype, seed=rows + cols)
    c, s, ct, st = mx.mx_quantize_2d(x.to(DEV), scale_rule=rule, round=rnd, seed=4321)
    rc, rs, rct, rst = orc.quantize_2d(hostx(x), scale_rule=rule, round_mode=rnd, seed=4321)
    assert_bytes_equal(s, rs, "scales")
    assert_bytes_equal(st, rst, "scales_t")
    assert_bytes_equal(c, rc, "codes")
    assert_bytes_equal(ct, rct, "codes_t")
    # without the transposed copy
    c2, s2, _, _ = mx.mx_quantize_2d(x.to(DEV), scale_rule=rule, round=rnd, seed=4321,
                                     transposed=False)
    assert_bytes_equal(c2, rc, "codes (no transpose)")


def test_2d_transposition_invariance_on_gpu(mx):
    w = wl.student_t3((128, 96), seed=3).to(torch.bfloat16).to(DEV)
    c, s, ct, st = mx.mx_quantize_2d(w, scale_rule=1)
    c2, s2, ct2, st2 = mx.mx_quantize_2d(w.t().contiguous(), scale_rule=1)
    assert torch.equal(s, s2.t()) and torch.equal(ct, c2) and torch.equal(c, ct2)


@pytest.mark.parametrize("block_rows,inv_had", [(1, 0), (1, 1), (32, 0)])
def test_dequantize_bit_exact(mx, orc, block_rows, inv_had):
    rng = np.random.default_rng(block_rows + inv_had)
    rows, cols = 64, 96
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 256, (rows // block_rows, cols // 32), dtype=np.uint8)
    scales[0, 0] = 0xFF
    scales[-1, -1] = 0
    scales[min(1, scales.shape[0] - 1), 1] = 254
    mask = 0xA5A5F00F
    out = mx.mx_dequantize(torch.from_numpy(codes).to(DEV), torch.from_numpy(scales).to(DEV), rows,
                           cols, block_rows, inv_had, mask)
    ref = orc.dequantize(codes, scales, rows, cols, block_rows, inv_had, mask)
    got = host(out)
    # NaN blocks (scale byte 0xFF) must be NaN at the same places; a NaN's sign and payload
    # after arithmetic is not specified by IEEE 754, everything else is bit-exact.
    nan_g, nan_r = np.isnan(got), np.isnan(ref)
    assert np.array_equal(nan_g, nan_r)
    bad = np.argwhere(got.view(np.uint32)[~nan_r] != ref.view(np.uint32)[~nan_r])
    assert len(bad) == 0, (len(bad), got[~nan_r][bad[:4, 0]], ref[~nan_r][bad[:4, 0]])


def quantize_pair(mx, a, b, rule=0, rnd=0, had=0, mask=0, seed=0, axis=1):
    qa = mx.mx_quantize(a, axis=axis, scale_rule=rule, round=rnd, hadamard=had, sign_mask=mask,
                        seed=seed)
    qb = mx.mx_quantize(b, axis=axis, scale_rule=rule, round=rnd, hadamard=had, sign_mask=mask,
                        seed=seed + 1)
    return qa, qb


GEMM_CASES = [
    # M, N, K
    (32, 32, 32),
    (64, 96, 128),
    (256, 256, 256),
    (288, 320, 416),     # ragged against the 256x256 tile and the 128 k-step
    (512, 256, 1024),
    (96, 544, 2080),
    (128, 256, 640),     # 5 k-steps: one unrolled round + 1 remainder step
    (256, 288, 896),     # 7 k-steps: remainder of 3
    (64, 64, 4096),      # 32 k-steps
    (544, 800, 768),     # several tiles in both directions, partial edge tiles
    (256, 256, 2560),    # 256-wide k stages: 10 steps, last scale group partial
    (288, 96, 1536),     # 6 steps, partial M tile
    # K a multiple of 1024 (the two-waves-per-SIMD kernel): one scale group per 4 steps
    (32, 32, 1024),      # one partial tile, 4 steps
    (288, 320, 1024),    # partial tiles in both directions
    (1056, 96, 2048),    # 5 tile rows, one partial
    (544, 800, 3072),    # 3 x 4 tiles, 12 steps
]


@pytest.mark.parametrize("M,N,K", GEMM_CASES)
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("which", ["fprop", "dgrad", "wgrad"])
def test_gemm_within_bound(mx, orc, M, N, K, out_dtype, which):
    a = wl.student_t3((M, K), seed=M + K).to(DEV)
    b = wl.normal((N, K), 0.02, seed=N + K).to(DEV)
    (aq, as_), (bq, bs) = quantize_pair(mx, a, b, rule=1)
    fn = getattr(mx, "mx_gemm_" + which)
    out = fn(aq, as_, 1, bq, bs, 1, alpha_exp=0, out_dtype=out_dtype)
    torch.cuda.synchronize()
    C, Cabs = orc.gemm(host(aq), host(as_), 1, host(bq), host(bs), 1, M, N, K, 0)
    check_gemm(out, C, Cabs)


@pytest.mark.parametrize("K", [384, 2048, 3072])
@pytest.mark.parametrize("ga,gb", [(32, 1), (1, 32), (32, 32)])
def test_gemm_2d_scales(mx, orc, ga, gb, K):
    M, N = 288, 256
    a = wl.student_t3((M, K), seed=1).to(DEV)
    b = wl.student_t3((N, K), seed=2).to(DEV)
    aq, as_ = (mx.mx_quantize_2d(a, scale_rule=1)[:2] if ga == 32 else mx.mx_quantize(a, scale_rule=1))
    bq, bs = (mx.mx_quantize_2d(b, scale_rule=1)[:2] if gb == 32 else mx.mx_quantize(b, scale_rule=1))
    out = mx.mx_gemm_fprop(aq, as_, ga, bq, bs, gb, out_dtype=torch.float32)
    C, Cabs = orc.gemm(host(aq), host(as_), ga, host(bq), host(bs), gb, M, N, K, 0)
    check_gemm(out, C, Cabs)


def test_gemm_hadamard_alpha(mx, orc):
    """Both operands rotated along K with the same signs: alpha = -5 undoes H.H = 32 I, so the
    product approximates the unrotated one."""
    M, N, K = 128, 96, 512
    a = wl.student_t3((M, K), seed=11).to(DEV)
    b = wl.student_t3((N, K), seed=12).to(DEV)
    mask = wl.sign_mask()
    (aq, as_), (bq, bs) = quantize_pair(mx, a, b, rule=1, had=1, mask=mask)
    out = mx.mx_gemm_fprop(aq, as_, 1, bq, bs, 1, alpha_exp=-5, out_dtype=torch.float32)
    C, Cabs = orc.gemm(host(aq), host(as_), 1, host(bq), host(bs), 1, M, N, K, -5)
    check_gemm(out, C, Cabs)
    exact = (a.double() @ b.double().t()).cpu().numpy()
    rel = np.linalg.norm(host(out) - exact) / np.linalg.norm(exact)
    assert rel < 0.2


@pytest.mark.parametrize("M,N,K,out_dtype", [(8096, 4064, 2048, torch.bfloat16),
                                               (4352, 4352, 4096, torch.bfloat16),
                                               (4384, 8224, 1024, torch.bfloat16),
                                               (4384, 4128, 3072, torch.float32),
                                               (4608, 4352, 1024, torch.float32)])
def test_gemm_chained_tiles(mx, orc, M, N, K, out_dtype):
    """More 256x256 tiles than compute units, so every workgroup of the resident grid walks
    several tiles (each loading the next one's first steps while it finishes), with Hadamard +
    SR operands, bf16 or fp32 output and whole 4-step scale groups (one, two, three or four per
    tile). Ragged M and N put partial tiles among them, and the columns of the output rows past
    N must stay untouched."""
    a = wl.student_t3((M, K), seed=31).to(DEV)
    b = wl.normal((N, K), 0.02, seed=32).to(DEV)
    (aq, as_), (bq, bs) = quantize_pair(mx, a, b, rule=1, rnd=1, had=1, mask=wl.sign_mask())
    big = torch.full((M, N + 32), 7.0, dtype=out_dtype, device=DEV)
    out = mx.mx_gemm_fprop(aq, as_, 1, bq, bs, 1, out=big[:, :N], out_dtype=out_dtype)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, M, 11), np.arange(M - 40, M)]))
    cols = np.arange(N)
    C, Cabs = orc.gemm(host(aq), host(as_), 1, host(bq), host(bs), 1, M, N, K, 0,
                       rows=rows, cols=cols)
    check_gemm(out, C, Cabs, rows=rows, cols=cols)
    assert torch.all(big[:, N:] == 7.0)


def test_gemm_output_leading_dimension(mx, orc):
    M, N, K = 64, 96, 128
    a = wl.student_t3((M, K), seed=21).to(DEV)
    b = wl.student_t3((N, K), seed=22).to(DEV)
    (aq, as_), (bq, bs) = quantize_pair(mx, a, b)
    big = torch.full((M, 136), 7.0, device=DEV)
    out = mx.mx_gemm_fprop(aq, as_, 1, bq, bs, 1, out=big[:, :N], out_dtype=torch.float32)
    C, Cabs = orc.gemm(host(aq), host(as_), 1, host(bq), host(bs), 1, M, N, K, 0)
    check_gemm(out, C, Cabs)
    assert torch.all(big[:, N:] == 7.0)


def test_empty_inputs_are_noops(mx):
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    c, s = mx.mx_quantize(x)
    assert c.numel() == 0 and s.numel() == 0
    aq = torch.empty((0, 32), dtype=torch.uint8, device=DEV)
    out = mx.mx_gemm_fprop(aq, torch.empty((0, 2), dtype=torch.uint8, device=DEV), 1,
                           torch.zeros((32, 32), dtype=torch.uint8, device=DEV),
                           torch.zeros((32, 2), dtype=torch.uint8, device=DEV), 1)
    assert out.shape == (0, 32)
    # K == 0: an empty reduction, every output is zero
    z = torch.empty((32, 0), dtype=torch.uint8, device=DEV)
    out = mx.mx_gemm_fprop(z, z, 1, z, z, 1, out=torch.full((32, 32), 7.0, device=DEV))
    assert torch.count_nonzero(out).item() == 0


def test_bad_shape_raises(mx):
    x = torch.zeros((32, 48), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mx.MxError):
        mx.mx_quantize(x)
