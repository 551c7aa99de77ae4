"""GPU parity of the quantisers and of 2:4 pruning + packing against the
oracle: codes, scales, kept values and metadata must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_layers_amd as sg
import workloads
from gpu_helpers import DEV, say, up

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("gr,gc,rows,cols,dist", [
    (1, 128, 1, 128, "normal"), (1, 128, 37, 256, "outliers"), (1, 128, 2048, 4096, "outliers"),
    (128, 128, 4096, 4096, "weight"), (128, 128, 130, 384, "weight"), (128, 64, 4096, 2048, "weight"),
    (128, 64, 37, 64, "normal"), (1, 64, 300, 192, "normal"),
])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fp8_quant_matches_oracle(gr, gc, rows, cols, dist, dtype):
    say(f"fp8_quant gr={gr} gc={gc} {rows}x{cols} {dist} {dtype}")
    if dist == "outliers":
        x = workloads.dense_outliers(seed=100 + rows, m=rows, n=8, k=cols)["x"]
    else:
        x = workloads.sparse_large(seed=200 + rows, m=rows, n=rows, k=cols)["w" if dist == "weight" else "x"]
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x)
        x_or = (bits.astype(np.uint32) << 16).view(np.float32)
        xt = up(bits)
    else:
        x_or, xt = x, up(x)
    q, s = sg.fp8_quant_groupwise(xt, gr=gr, gc=gc)
    oq, os_ = oracle.fp8_quant_groupwise(x_or, gr, gc)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), oq)


def _extreme_rows(rows, cols, seed):
    """Row groups at the ends of the fp32 range: subnormal magnitudes (the scale
    itself subnormal), magnitudes near the fp32 maximum, exact powers of two,
    zeros, and blocks of mixed extremes."""
    rng = np.random.default_rng(seed)
    u = rng.uniform(-1.0, 1.0, size=(rows, cols))
    kind = np.arange(rows) % 5
    x = np.where(kind[:, None] == 0, u * 1e-40, 0.0)
    x = np.where(kind[:, None] == 1, u * 3.0e38, x)
    x = np.where(kind[:, None] == 2, np.sign(u) * np.exp2(rng.integers(-149, 127, size=(rows, cols))), x)
    mixed = np.where(rng.integers(0, 2, size=(rows, cols)) == 1, u * 1e-38, u * 1e30)
    x = np.where(kind[:, None] == 4, mixed, x)
    return x.astype(np.float32)


@pytest.mark.parametrize("gr,gc,rows", [(1, 128, 10), (1, 64, 10), (128, 64, 256), (1, 512, 10), (10, 512, 10)])
def test_fp8_and_int8_quant_at_the_ends_of_the_fp32_range(gr, gc, rows):
    x = _extreme_rows(rows, 512, seed=300 + gr + gc)
    say(f"extreme quant gr={gr} gc={gc} rows={rows}")
    for fn, ofn in ((sg.fp8_quant_groupwise, oracle.fp8_quant_groupwise),
                    (sg.int8_quant_groupwise, oracle.int8_quant_groupwise)):
        q, s = fn(up(x), gr=gr, gc=gc)
        oq, os_ = ofn(x, gr, gc)
        torch.cuda.synchronize()
        assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32)), fn.__name__
        assert np.array_equal(q.cpu().numpy(), oq), fn.__name__


@pytest.mark.parametrize("gc", [128, 64])
def test_int4_quant_at_the_ends_of_the_fp32_range(gc):
    x = _extreme_rows(10, 512, seed=310 + gc)
    q, s = sg.int4_quant_groupwise(up(x), gc=gc)
    oq, os_ = oracle.int4_quant_groupwise(x, gc)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), oq)


def test_fp8_encoder_on_every_midpoint_and_neighbour():
    """Blocks whose amax is 448 have scale 1, so the codes are the encoder's
    output for the raw values: every e4m3 midpoint, its fp32 neighbours, every
    finite e4m3 value, signed zeros, subnormals and a million random values."""
    pos = oracle.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mid = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    vals = np.concatenate([mid, np.nextafter(mid, np.float32(1e9)), np.nextafter(mid, np.float32(0)),
                           pos.astype(np.float32), np.array([0.0, 2.0 ** -10, 2.0 ** -12, 1e-30, 2.0 ** -6], np.float32)])
    vals = np.concatenate([vals, -vals])
    rng = np.random.default_rng(7)
    rnd = (np.exp2(rng.uniform(-14, np.log2(448.0), 1_000_000)) *
           np.where(rng.random(1_000_000) < 0.5, -1, 1)).astype(np.float32)
    vals = np.concatenate([vals, rnd])
    n = -(-len(vals) // 127) * 127
    v = np.zeros(n, np.float32)
    v[:len(vals)] = vals
    x = np.concatenate([np.full((n // 127, 1), 448.0, np.float32), v.reshape(-1, 127)], axis=1)
    say(f"encoder sweep: {x.shape}")
    q, s = sg.fp8_quant_groupwise(up(x), gr=1, gc=128)
    torch.cuda.synchronize()
    assert np.all(s.cpu().numpy() == 1.0)
    assert np.array_equal(q.cpu().numpy(), oracle.e4m3_encode(x))


def test_fp8_quant_saturates_a_quotient_just_above_448():
    """For some block maxima a, fl32(a / fl32(a / 448)) is 448.00003, just above
    the largest e4m3 value: the code must saturate to 0x7E (448), as the oracle's
    encoder does, not become NaN."""
    rng = np.random.default_rng(11)
    a = (rng.uniform(1, 2, 200_000) * np.exp2(rng.integers(-20, 20, 200_000))).astype(np.float32)
    over = a[(a / (a / np.float32(448)).astype(np.float32)).astype(np.float32) > np.float32(448)][:256]
    assert len(over) == 256
    x = np.zeros((256, 128), np.float32)
    x[:, 0] = over
    x[:, 1] = -over
    x[:, 2:] = over[:, None] * rng.uniform(-1, 1, (256, 126)).astype(np.float32)
    q, s = sg.fp8_quant_groupwise(up(x), gr=1, gc=128)
    torch.cuda.synchronize()
    rq, rs = oracle.fp8_quant_groupwise(x, 1, 128)
    qc = q.cpu().numpy()
    assert np.all(qc[:, 0] == 0x7E) and np.all(qc[:, 1] == 0xFE)
    assert np.array_equal(qc, rq) and np.array_equal(s.cpu().numpy(), rs)


def test_fp8_quant_all_zero_and_scale_layouts():
    x = np.zeros((5, 384), np.float32)
    x[2, 130:140] = -3.5
    x[4, 0] = -0.0
    xt = up(x)
    q, s = sg.fp8_quant_groupwise(xt, gr=1, gc=128)
    oq, os_ = oracle.fp8_quant_groupwise(x, 1, 128)
    assert np.array_equal(q.cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)
    # row-major scales through explicit strides
    s_rm = torch.empty((5, 3), dtype=torch.float32, device=DEV)
    sg.fp8_quant_groupwise(xt, gr=1, gc=128, s=s_rm)
    assert np.array_equal(s_rm.cpu().numpy(), os_)


def test_fp8_quant_strided_rows():
    x = workloads.sparse_large(seed=9, m=40, n=8, k=512)["x"]
    big = torch.zeros((40, 640), dtype=torch.float32, device=DEV)
    big[:, :512] = up(x)
    q = torch.zeros((40, 528), dtype=torch.uint8, device=DEV)
    qv, s = sg.fp8_quant_groupwise(big[:, :512], gr=1, gc=128, q=q[:, :512])
    oq, os_ = oracle.fp8_quant_groupwise(x, 1, 128)
    assert np.array_equal(q[:, :512].cpu().numpy(), oq) and np.array_equal(s.cpu().numpy(), os_)
    assert not q[:, 512:].any()


@pytest.mark.parametrize("rows,cols,dtype", [(9, 384, "f32"), (2048, 4096, "f32"), (4096, 4096, "bf16"),
                                             (1, 128, "bf16")])
def test_int4_quant_matches_oracle(rows, cols, dtype):
    say(f"int4_quant {rows}x{cols} {dtype}")
    x = workloads.mixed_add(seed=300 + rows, m=rows, n=4, k1=cols, k2=32)["x1"]
    if dtype == "bf16":
        bits = workloads.to_bf16_bits(x)
        x_or, xt = (bits.astype(np.uint32) << 16).view(np.float32), up(bits)
    else:
        x_or, xt = x, up(x)
    q, s = sg.int4_quant_groupwise(xt)
    oq, os_ = oracle.int4_quant_groupwise(x_or, 128)
    torch.cuda.synchronize()
    assert np.array_equal(s.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    assert np.array_equal(q.cpu().numpy(), oq)


def test_int4_quant_ties_round_to_even():
    x = np.zeros((1, 128), np.float32)
    x[0, :8] = [7.0, 0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 3.5]
    q, s = sg.int4_quant_groupwise(up(x))
    oq, _ = oracle.int4_quant_groupwise(x, 128)
    assert np.array_equal(q.cpu().numpy(), oq)
    assert oracle.int4_decode(oq)[0, :8].tolist() == [7, 0, 2, 2, 0, -2, -2, 4]


@pytest.mark.parametrize("rows,k,dtype", [(128, 256, "f32"), (4096, 4096, "f32"), (333, 520, "f32"),
                                          (4096, 4096, "bf16"), (1, 8, "bf16")])
def test_prune_compress_matches_oracle(rows, k, dtype):
    say(f"prune {rows}x{k} {dtype}")
    w = workloads.sparse_large(seed=400 + rows, m=4, n=rows, k=k)["w"]
    wo = workloads.to_bf16_bits(w) if dtype == "bf16" else w
    v, m = sg.sparse24_prune_compress(up(wo))
    ov, om = oracle.prune_compress24(wo)
    torch.cuda.synchronize()
    got = v.cpu()
    got = got.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else got.numpy().view(np.uint32)
    want = ov.view(np.uint16) if dtype == "bf16" else ov.view(np.uint32)
    assert np.array_equal(m.cpu().numpy(), om)
    assert np.array_equal(got, want)


def test_prune_ties_signed_zeros_and_all_zero_rows():
    """Every group of the 8-letter alphabet {+-0, +-1, +-2, +-3}^4 (4096
    groups), plus an all-zero row: exact agreement with the oracle's ranking."""
    import itertools
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, 2.0, -2.0, 3.0, -3.0], np.float32)
    groups = alphabet[np.array(list(itertools.product(range(8), repeat=4)))].reshape(512, 32)
    w = np.concatenate([groups, np.zeros((1, 32), np.float32)])
    v, m = sg.sparse24_prune_compress(up(w))
    ov, om = oracle.prune_compress24(w)
    assert np.array_equal(m.cpu().numpy(), om)
    assert np.array_equal(v.cpu().numpy().view(np.uint32), ov.view(np.uint32))


@pytest.mark.parametrize("n,k", [(256, 128), (300, 384), (4096, 4096), (14336, 4096), (1, 128), (37, 14336)])
def test_pack_gfx950_matches_oracle(n, k):
    say(f"pack {n}x{k}")
    rng = np.random.default_rng(n + k)
    vals = workloads.random_e4m3_codes(rng, (n, k // 2))
    meta = rng.integers(0, 256, size=(n, k // 8)).astype(np.uint8)
    packed = sg.sparse24_pack_gfx950(up(vals), up(meta))
    want = oracle.pack24_gfx950(vals, meta)
    torch.cuda.synchronize()
    assert packed.numel() == want.size == sg.sparse24_packed_bytes(n, k)
    assert np.array_equal(packed.cpu().numpy(), want)


def test_pack_strided_inputs():
    rng = np.random.default_rng(5)
    vals = workloads.random_e4m3_codes(rng, (40, 256))
    meta = rng.integers(0, 256, size=(40, 64)).astype(np.uint8)
    vb = torch.zeros((40, 320), dtype=torch.uint8, device=DEV)
    vb[:, :256] = up(vals)
    mb = torch.zeros((40, 80), dtype=torch.uint8, device=DEV)
    mb[:, :64] = up(meta)
    packed = sg.sparse24_pack_gfx950(vb[:, :256], mb[:, :64])
    assert np.array_equal(packed.cpu().numpy(), oracle.pack24_gfx950(vals, meta))


def _nan_aware_equal(got: np.ndarray, want: np.ndarray) -> bool:
    """Equal bit patterns, except that any NaN matches any NaN."""
    gn, wn = np.isnan(got), np.isnan(want)
    return np.array_equal(gn, wn) and np.array_equal(got[~gn].view(np.uint32), want[~wn].view(np.uint32))


def _nonfinite_x(rows, cols, seed):
    """Normal values with NaN and +-inf planted in some 1 x 64 blocks (and so in
    the 128-wide and 128-row blocks around them)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    for r, c, v in [(0, 3, np.nan), (1, 70, -np.inf), (2, 130, np.inf), (2, 131, np.nan), (5, 200, -np.nan),
                    (rows - 1, cols - 1, np.inf)]:
        x[r % rows, c % cols] = v
    return x


@pytest.mark.parametrize("gr,gc", [(1, 128), (1, 64), (128, 128), (128, 64)])
@pytest.mark.parametrize("mode", ["fp8", "int8"])
def test_quant_nan_and_inf_blocks(gr, gc, mode):
    """A block holding a NaN gets a NaN scale, one holding an infinity an
    infinite scale; codes are the encoder applied to v / s (e4m3: 0x7F for NaN;
    int8: 0)."""
    x = _nonfinite_x(260, 384, 7)
    say(f"{mode} quant non-finite gr={gr} gc={gc}")
    if mode == "fp8":
        q, s = sg.fp8_quant_groupwise(up(x), gr=gr, gc=gc)
        oq, os_ = oracle.fp8_quant_groupwise(x, gr, gc)
    else:
        q, s = sg.int8_quant_groupwise(up(x), gr=gr, gc=gc)
        oq, os_ = oracle.int8_quant_groupwise(x, gr, gc)
    torch.cuda.synchronize()
    assert np.isnan(os_).any() and np.isinf(os_).any()
    assert _nan_aware_equal(s.cpu().numpy(), os_)
    assert np.array_equal(q.cpu().numpy(), oq)


@pytest.mark.parametrize("whole", ["rows", "tensor"])
def test_quant_nan_and_inf_scales_constant_along_k(whole):
    x = _nonfinite_x(6, 256, 8)
    if whole == "tensor":      # one scale: an infinity alone (no NaN) gives s = inf
        x = np.where(np.isnan(x), np.float32(1.0), x)
    gr = 1 if whole == "rows" else 6
    q, s = sg.fp8_quant_groupwise(up(x), gr=gr, gc=256)
    oq, os_ = oracle.fp8_quant_groupwise(x, gr, 256)
    torch.cuda.synchronize()
    assert _nan_aware_equal(s.cpu().numpy(), os_)
    assert np.array_equal(q.cpu().numpy(), oq)


def test_int4_quant_nan_and_inf_blocks():
    x = _nonfinite_x(9, 384, 9)
    q, s = sg.int4_quant_groupwise(up(x))
    oq, os_ = oracle.int4_quant_groupwise(x, 128)
    torch.cuda.synchronize()
    assert _nan_aware_equal(s.cpu().numpy(), os_)
    assert np.array_equal(q.cpu().numpy(), oq)


def _bf16_bits(f32):
    """Upper halves of fp32 values that bf16 represents exactly."""
    return (np.ascontiguousarray(f32, np.float32).view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prune_nan_and_inf_every_group(dtype):
    """Every group over {+-0, +-1, +-inf, +-NaN}^4 (4096 groups), plus NaNs with
    other payloads: NaN outranks infinity, NaNs tie, bits copied unchanged."""
    import itertools
    alphabet = np.array([0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, -np.nan], np.float32)
    groups = alphabet[np.array(list(itertools.product(range(8), repeat=4)))].reshape(512, 32)
    odd = np.array([0x7F800001, 0xFFFFFFFF, 0x7FC00001, 0x00000001] * 8, np.uint32).view(np.float32)
    w = np.concatenate([groups, odd[None, :]])
    if dtype == "bf16":
        w = _bf16_bits(w)
        w[-1, ::4] = 0x7F81          # a bf16 NaN with the smallest payload
    v, m = sg.sparse24_prune_compress(up(w))
    ov, om = oracle.prune_compress24(w)
    torch.cuda.synchronize()
    assert np.array_equal(m.cpu().numpy(), om)
    got = v.cpu().view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else v.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, ov.view(np.uint16) if dtype == "bf16" else ov.view(np.uint32))


@pytest.mark.parametrize("rows,k", [(128, 256), (333, 528), (4096, 4096), (1, 16), (14336, 4096)])
def test_prune_e4m3_codes_match_oracle(rows, k):
    """Already-quantised weights: e4m3 codes ranked by the magnitude they
    encode (NaN codes 0x7F / 0xFF above 448, -0 equal to +0)."""
    say(f"prune e4m3 {rows}x{k}")
    rng = np.random.default_rng(rows + k)
    c = rng.integers(0, 256, size=(rows, k)).astype(np.uint8)
    special = rng.random((rows, k)) < 0.2
    c[special] = rng.choice(np.array([0x00, 0x80, 0x7F, 0xFF, 0x7E, 0xFE, 0x01, 0x81], np.uint8),
                            size=int(special.sum()))
    v, m = sg.sparse24_prune_compress(up(c))
    ov, om = oracle.prune_compress24(c)
    torch.cuda.synchronize()
    assert v.dtype == torch.uint8
    assert np.array_equal(m.cpu().numpy(), om)
    assert np.array_equal(v.cpu().numpy(), ov)


def test_prune_e4m3_then_pack_feeds_the_sparse_gemm():
    """Quantise W to e4m3 codes, prune the codes, pack them: the sparse GEMM on
    that weight matches the oracle's GEMM on the oracle's pruned codes."""
    d = workloads.sparse_large(seed=17, m=96, n=256, k=512)
    xq, sx = oracle.fp8_quant_groupwise(d["x"], 1, 128)
    wq, sw = oracle.fp8_quant_groupwise(d["w"], 128, 128)
    v, m = sg.sparse24_prune_compress(up(wq))
    ov, om = oracle.prune_compress24(wq)
    torch.cuda.synchronize()
    assert np.array_equal(v.cpu().numpy(), ov) and np.array_equal(m.cpu().numpy(), om)
    from gpu_helpers import up_scales, down, assert_within_tolerance
    y = down(sg.fp8_sparse24_gemm_groupwise(up(xq), up_scales(sx), v, m, up_scales(sw), 1, 128,
                                            out_dtype=torch.float32))
    ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq, sx, 1, ov, om, sw, 128, bound=True)
    assert_within_tolerance(y.astype(np.float64), ref, bound, "GEMM on pruned e4m3 codes")
