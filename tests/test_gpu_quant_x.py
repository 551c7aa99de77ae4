"""GPU parity of the packed 2:4 FP8 GEMM with the activation quantisation
fused in (sg_fp8_sparse24_gemm_packed_quant_x).  It must return, bit for bit,
what sg_fp8_quant_groupwise(x, 1, 128) followed by
sg_fp8_sparse24_gemm_groupwise_packed returns (the fused kernel quantises each
1 x 128 block with the same arithmetic and sums the same terms in the same
order), and stay within the oracle's tolerance of the oracle's
quantise-then-GEMM.  Covered: the decode shapes of the torchao PR's workload
(M = 16 and 37, (N, K) = (14336, 4096) and (4096, 14336)) in both output
forms, ragged small shapes spanning every sub-tile count, fp32 and bf16
activations, strided X rows, zero blocks and non-finite blocks."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_layers_amd as sg
import workloads
from gpu_helpers import DEV, assert_within_tolerance, down, say, up, up_scales

pytestmark = pytest.mark.gpu


def weight(seed, n, k):
    w = workloads.decode(seed=seed, m=1, n=n, k=k)["w"]
    wv32, meta = oracle.prune_compress24(w)
    wq, sw = oracle.fp8_quant_groupwise(wv32, 128, 64)
    return wq, meta, sw


def bits(t):
    t = t.detach()
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()


def fused_and_separate(x_dev, wp, n, sw_dev, out, form):
    y_f = sg.fp8_sparse24_gemm_packed_quant_x(x_dev, wp, n, sw_dev, 128, out_dtype=out, form=form)
    xq, sx = sg.fp8_quant_groupwise(x_dev, 1, 128)
    y_s = sg.fp8_sparse24_gemm_groupwise_packed(xq, sx, wp, n, sw_dev, 1, 128, out_dtype=out, form=form)
    torch.cuda.synchronize()
    return y_f, y_s


def assert_same_bits(y_f, y_s, what):
    a, b = bits(y_f), bits(y_s)
    if not np.array_equal(a, b):
        bad = np.argwhere(a != b)
        raise AssertionError(f"{what}: {len(bad)} outputs differ from quantise-then-GEMM, first at {bad[0].tolist()}")


def x_as(x32, xdt):
    """(device tensor, the fp32 values the oracle sees)."""
    if xdt == "bf16":
        b = workloads.to_bf16_bits(x32)
        return up(b), (b.astype(np.uint32) << 16).view(np.float32)
    return up(x32), x32


@pytest.mark.parametrize("m,n,k", workloads.DECODE_SHAPES)
@pytest.mark.parametrize("form", ["y", "yt"])
def test_decode_shapes_match_quantise_then_gemm(m, n, k, form):
    say(f"quant_x decode M={m} N={n} K={k} form={form}")
    x32 = workloads.decode(seed=4, m=m, n=n, k=k)["x"]
    wq, meta, sw = weight(40 + m, n, k)
    wp = up(oracle.pack24_gfx950(wq, meta))
    xd, xo = x_as(x32, "f32")
    y_f, y_s = fused_and_separate(xd, wp, n, up_scales(sw), torch.bfloat16, form)
    assert_same_bits(y_f, y_s, f"M={m} N={n} K={k} {form}")
    xq, sx = oracle.fp8_quant_groupwise(xo, 1, 128)
    ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq, sx, 1, wq, meta, sw, 128, bound=True)
    got = down(y_f)
    got = got.T if form == "yt" else got
    assert_within_tolerance(got.astype(np.float64), ref, bound, f"fused M={m} N={n} K={k} {form}")


SMALL = [(1, 256, 128), (5, 130, 384), (16, 512, 1024), (17, 300, 256), (32, 1000, 512), (33, 256, 640),
         (48, 384, 128), (49, 512, 384), (64, 1024, 256), (64, 15000, 256),
         # more row blocks than CUs: one workgroup per CU, 2, 3 or 4 row blocks each
         (16, 5120, 256), (20, 11008, 256), (37, 12288, 128), (60, 13000, 256)]


@pytest.mark.parametrize("m,n,k", SMALL)
@pytest.mark.parametrize("xdt", ["f32", "bf16"])
def test_ragged_shapes_both_activation_dtypes(m, n, k, xdt):
    say(f"quant_x M={m} N={n} K={k} x={xdt}")
    x32 = workloads.decode(seed=m + n, m=m, n=n, k=k)["x"]
    wq, meta, sw = weight(m * 3 + k, n, k)
    wp = up(oracle.pack24_gfx950(wq, meta))
    xd, xo = x_as(x32, xdt)
    for out, form in ((torch.float32, "y"), (torch.bfloat16, "yt")):
        y_f, y_s = fused_and_separate(xd, wp, n, up_scales(sw), out, form)
        assert_same_bits(y_f, y_s, f"M={m} N={n} K={k} {xdt} {out} {form}")
    xq, sx = oracle.fp8_quant_groupwise(xo, 1, 128)
    ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq, sx, 1, wq, meta, sw, 128, bound=True)
    assert_within_tolerance(down(y_f).T.astype(np.float64), ref, bound, f"fused M={m} N={n} K={k}")


def test_strided_rows_zero_and_nonfinite_blocks():
    m, n, k = 21, 512, 512
    rng = np.random.default_rng(9)
    x32 = rng.standard_normal((m, k)).astype(np.float32)
    x32[3, 128:256] = 0.0                  # an all-zero block: scale 1, codes 0
    x32[4, :128] *= np.float32(1e-30)      # tiny values: a tiny scale
    x32[5, 300] = np.nan                   # a NaN block: NaN outputs in row 5
    x32[6, 10] = np.inf                    # an infinite block
    buf = torch.zeros((m, k + 64), dtype=torch.float32, device=DEV)
    buf[:, :k] = up(x32)
    wq, meta, sw = weight(7, n, k)
    wp = up(oracle.pack24_gfx950(wq, meta))
    y_f, y_s = fused_and_separate(buf[:, :k], wp, n, up_scales(sw), torch.float32, "y")
    a, b = y_f.cpu().numpy(), y_s.cpu().numpy()
    assert np.array_equal(np.isnan(a), np.isnan(b)) and np.isnan(a[5]).all() and np.isnan(a[6]).all()
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok].view(np.uint32), b[ok].view(np.uint32))
    assert np.isfinite(a[[0, 1, 2, 3, 4]]).all()


def identity_weight(k):
    """A 2:4 weight whose GEMM is the identity: W = I (N = K) as e4m3 codes 1.0
    with W scales 1, so y[m, k] = sx[m, k / 128] * e4m3(x_code[m, k]) for one
    product each -- the dequantise-by-identity check of the torchao PR
    (jcaip's review), used here to read the fused kernel's codes one by one."""
    keep_vals, meta = oracle.prune_compress24(np.eye(k, dtype=np.float32))
    codes = oracle.e4m3_encode(keep_vals)
    return codes, meta, np.ones((k // 128, k // 128), np.float32)


def near_midpoint_rows(rng, m, k):
    """Rows whose quotients v / s fall on and next to the rounding boundaries of
    e4m3 (the midpoints between neighbouring codes), for scales with awkward
    mantissas across a wide exponent range: any quotient that is off by an ulp
    shows up as a different code."""
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2.0
    x = np.zeros((m, k), np.float32)
    for r in range(m):
        for kb in range(k // 128):
            s_mant = rng.choice([1.0, 1.5, 2.0 - 2.0 ** -23, 1.0 + 2.0 ** -23, rng.uniform(1, 2)])
            e = int(rng.integers(-110, 80))     # below 2^-90 the scale takes plain divides
            amax = np.float32(448.0 * s_mant * 2.0 ** e)
            s = np.float32(amax / np.float32(448.0))
            blk = np.empty(128, np.float32)
            blk[0] = amax
            mid = rng.choice(mids, 127) * rng.choice([-1.0, 1.0], 127)
            base = (mid * np.float64(s)).astype(np.float32)
            step = rng.integers(-2, 3, 127)
            for i in range(127):
                v = base[i]
                for _ in range(abs(int(step[i]))):
                    v = np.nextafter(v, np.float32(np.inf) if step[i] > 0 else np.float32(-np.inf))
                blk[1 + i] = v
            x[r, kb * 128:(kb + 1) * 128] = blk
    return x


@pytest.mark.parametrize("m", [16, 37, 64])
def test_identity_weight_shows_every_code_near_rounding_boundaries(m):
    k = 256
    rng = np.random.default_rng(m)
    x = near_midpoint_rows(rng, m, k)
    codes, meta, sw = identity_weight(k)
    wp = up(oracle.pack24_gfx950(codes, meta))
    y_f, y_s = fused_and_separate(up(x), wp, k, up_scales(sw), torch.float32, "y")
    assert_same_bits(y_f, y_s, f"identity M={m}")
    xq, sx = oracle.fp8_quant_groupwise(x, 1, 128)
    want = (oracle.e4m3_decode(xq) * np.repeat(sx.astype(np.float64), 128, axis=1)).astype(np.float32)
    want = want + np.float32(0.0)       # the sum over the waves starts at +0: -0 comes out as +0
    assert np.array_equal(y_f.cpu().numpy().view(np.uint32), want.view(np.uint32))
