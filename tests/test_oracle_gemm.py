"""Pins of the oracle's GEMMs: exact rational brute force, the identity-matrix
dequantisation, a per-element-dequantisation route, integer matmuls, the
sparse = dense(decompressed) identity and the swap identity."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_e4m3_values(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.float().numpy()


def _fraction_gemm(xq, sx, gm, wq, sw, gn):
    """Exact rational y = sum_kb sx*sw*sum_k x*w, element by element."""
    xv, wv = _torch_e4m3_values(xq), _torch_e4m3_values(wq)
    m, k = xq.shape
    n = wq.shape[0]
    out = [[Fraction(0)] * n for _ in range(m)]
    for i in range(m):
        for j in range(n):
            acc = Fraction(0)
            for kb in range(k // 128):
                p = sum((Fraction(float(xv[i, q])) * Fraction(float(wv[j, q]))
                         for q in range(kb * 128, kb * 128 + 128)), Fraction(0))
                acc += Fraction(float(sx[i // gm, kb])) * Fraction(float(sw[j // gn, kb])) * p
            out[i][j] = acc
    return out


@pytest.mark.parametrize("m,n,k,gm,gn", [(3, 4, 128, 1, 1), (4, 2, 256, 1, 128),
                                         (2, 3, 256, 128, 128), (1, 1, 384, 128, 1)])
def test_exact_rational_brute_force(m, n, k, gm, gn):
    rng = np.random.default_rng(m * 100 + n * 10 + k)
    xq = workloads.random_e4m3_codes(rng, (m, k))
    wq = workloads.random_e4m3_codes(rng, (n, k))
    sx = workloads.random_scales(rng, (-(-m // gm), k // 128))
    sw = workloads.random_scales(rng, (-(-n // gn), k // 128))
    y = oracle.fp8_gemm_groupwise(xq, sx, gm, wq, sw, gn)
    ref = _fraction_gemm(xq, sx, gm, wq, sw, gn)
    for i in range(m):
        for j in range(n):
            # y is the fp64 sum of 128-term exact partials times exact scale
            # products: within a few fp64 ulps of the exact value.
            assert abs(Fraction(y[i, j]) - ref[i][j]) <= abs(ref[i][j]) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 200)


def test_identity_dequantises_weight():
    """Multiplying by an identity matrix returns the dequantised weight
    (torchao PR #3258, jcaip: dequantise a sparse tensor via the identity)."""
    rng = np.random.default_rng(31)
    k, n = 256, 300
    wq = workloads.random_e4m3_codes(rng, (n, k))
    sw = workloads.random_scales(rng, (-(-n // 128), k // 128))
    eye = np.zeros((k, k), dtype=np.uint8)
    eye[np.arange(k), np.arange(k)] = 0x38                 # 1.0
    sx = np.ones((k, k // 128), dtype=np.float32)
    y = oracle.fp8_gemm_groupwise(eye, sx, 1, wq, sw, 128)
    want = (oracle.e4m3_decode(wq) * np.repeat(np.repeat(sw, 128, 0)[:n], 128, 1).astype(np.float64)).T
    assert np.array_equal(y, want)


@pytest.mark.parametrize("gm,gn", [(1, 1), (1, 128), (128, 128), (128, 1)])
def test_matches_per_element_dequantised_matmul(gm, gn):
    rng = np.random.default_rng(32 + gm + gn)
    m, n, k = 130, 260, 384
    xq = workloads.random_e4m3_codes(rng, (m, k))
    wq = workloads.random_e4m3_codes(rng, (n, k))
    sx = workloads.random_scales(rng, (-(-m // gm), k // 128))
    sw = workloads.random_scales(rng, (-(-n // gn), k // 128))
    y, t = oracle.fp8_gemm_groupwise(xq, sx, gm, wq, sw, gn, bound=True)
    sxe = np.repeat(np.repeat(sx, gm, 0)[:m], 128, 1).astype(np.float64)
    swe = np.repeat(np.repeat(sw, gn, 0)[:n], 128, 1).astype(np.float64)
    xdq = _torch_e4m3_values(xq).astype(np.float64) * sxe
    wdq = _torch_e4m3_values(wq).astype(np.float64) * swe
    y2 = xdq @ wdq.T
    t2 = np.abs(xdq) @ np.abs(wdq).T
    assert np.all(np.abs(y - y2) <= 1e-12 * t)
    assert np.allclose(t, t2, rtol=1e-12, atol=0)


def test_integer_codes_unit_scales_match_int64_matmul():
    rng = np.random.default_rng(33)
    ints = np.arange(-8, 9)
    # e4m3 represents every integer in [-8, 8] exactly
    codes_of = {int(v): int(oracle.e4m3_encode(np.array([v], np.float32))[0]) for v in ints}
    xi = rng.integers(-8, 9, size=(33, 256))
    wi = rng.integers(-8, 9, size=(17, 256))
    xq = np.vectorize(codes_of.get)(xi).astype(np.uint8)
    wq = np.vectorize(codes_of.get)(wi).astype(np.uint8)
    y = oracle.fp8_gemm_groupwise(xq, np.ones((33, 2), np.float32), 1, wq, np.ones((1, 2), np.float32), 128)
    assert np.array_equal(y, (xi @ wi.T).astype(np.float64))


def test_swap_gives_bit_exact_transpose():
    """C^T = B^T A^T (CUTLASS issue #2029, klevzoff's swap+transpose answer)."""
    rng = np.random.default_rng(34)
    xq = workloads.random_e4m3_codes(rng, (37, 256))
    wq = workloads.random_e4m3_codes(rng, (150, 256))
    sx = workloads.random_scales(rng, (37, 2))
    sw = workloads.random_scales(rng, (2, 2))
    y = oracle.fp8_gemm_groupwise(xq, sx, 1, wq, sw, 128)
    yt = oracle.fp8_gemm_groupwise(wq, sw, 128, xq, sx, 1)
    assert np.array_equal(yt, y.T)


def test_sparse_equals_dense_on_decompressed_weight():
    d = workloads.tiny_sparse()
    wv32, meta = oracle.prune_compress24(d["w"])
    wv, sw = oracle.fp8_quant_groupwise(wv32, 128, 64)
    xq, sx = oracle.fp8_quant_groupwise(d["x"], 1, 128)
    ys = oracle.fp8_sparse24_gemm_groupwise(xq, sx, 1, wv, meta, sw, 128)
    yd = oracle.fp8_gemm_groupwise(xq, sx, 1, oracle.decompress24(wv, meta), sw, 128)
    assert np.array_equal(ys, yd)


def test_compress_then_quantise_equals_quantise_pruned_dense():
    """Scales of 128x64 blocks of compressed values equal the 128x128 block
    scales of the pruned dense weight (pruning keeps each group's maximum),
    and the codes are the gathered dense codes."""
    w = workloads.sparse_large(seed=35, m=4, n=200, k=512)["w"]
    keep, pruned = oracle.prune24(w)
    vals, meta = oracle.compress24(pruned, keep)
    cq, cs = oracle.fp8_quant_groupwise(vals, 128, 64)
    dq, ds = oracle.fp8_quant_groupwise(pruned, 128, 128)
    assert np.array_equal(cs, ds)
    gq, gmeta = oracle.compress24(dq, keep)
    assert np.array_equal(gq, cq) and np.array_equal(gmeta, meta)


def test_hand_worked_gemm():
    """One output: K = 256, x = 1.0 everywhere, w = 0.5 in block 0 and -2.0 in
    block 1, sx = (2, 3), sw = (0.25, 4):
    y = 2*0.25*(128*0.5) + 3*4*(128*-2) = 32 - 3072 = -3040; T = 32 + 3072."""
    xq = np.full((1, 256), 0x38, np.uint8)
    wq = np.concatenate([np.full((1, 128), 0x30, np.uint8), np.full((1, 128), 0xC0, np.uint8)], 1)
    assert oracle.e4m3_decode(wq[0, [0, 200]]).tolist() == [0.5, -2.0]
    y, t = oracle.fp8_gemm_groupwise(xq, np.array([[2.0, 3.0]], np.float32), 1,
                                     wq, np.array([[0.25, 4.0]], np.float32), 128, bound=True)
    assert y[0, 0] == -3040.0 and t[0, 0] == 3104.0


def test_tolerance_rule():
    ref = np.array([100.0, 0.0, -5.0])
    t = np.array([1000.0, 1000.0, 10.0])
    ok = oracle.within_tolerance(np.array([101.9, 0.99, -5.0 - 0.06]), ref, t)
    bad = oracle.within_tolerance(np.array([102.1, 1.01, -5.0 - 0.061]), ref, t)
    assert ok.all() and not bad.any()


# --- fused int4 + bf16 add -------------------------------------------------

def test_mixed_int_part_matches_int64_matmul_and_bf16_part_is_exact_small():
    rng = np.random.default_rng(36)
    m, n, k1, k2 = 5, 7, 256, 32
    qx = rng.integers(-8, 8, size=(m, k1))
    qw = rng.integers(-8, 8, size=(n, k1))
    pack = lambda q: ((q[:, 0::2] & 15) | ((q[:, 1::2] & 15) << 4)).astype(np.uint8)
    sx1 = workloads.random_scales(rng, (m, 2))
    sw1 = workloads.random_scales(rng, (n, 2))
    x2 = workloads.to_bf16_bits(rng.standard_normal((m, k2)).astype(np.float32))
    w2 = workloads.to_bf16_bits(rng.standard_normal((n, k2)).astype(np.float32))
    y = oracle.mixed_gemm_add(pack(qx), sx1, pack(qw), sw1, x2, w2)
    x2f = torch.from_numpy(x2.view(np.int16)).view(torch.bfloat16).float().numpy()
    w2f = torch.from_numpy(w2.view(np.int16)).view(torch.bfloat16).float().numpy()
    for i in range(m):
        for j in range(n):
            exact, mag = Fraction(0), Fraction(0)
            for kb in range(2):
                xs, ws = qx[i, kb * 128:(kb + 1) * 128], qw[j, kb * 128:(kb + 1) * 128]
                s = Fraction(float(sx1[i, kb])) * Fraction(float(sw1[j, kb]))
                exact += s * int(xs @ ws)
                mag += s * int(np.abs(xs) @ np.abs(ws))
            for q in range(k2):
                p = Fraction(float(x2f[i, q])) * Fraction(float(w2f[j, q]))
                exact += p
                mag += abs(p)
            # the int part is exact; rounding comes only from fp64 sums of
            # terms bounded by mag
            assert abs(Fraction(y[i, j]) - exact) <= mag * Fraction(1, 2 ** 46)


def test_page_shapes_and_modes():
    vals, modes = {}, []
    for line in open(os.path.join(GOLDEN, "page_shapes.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        parts = line.split()
        if parts[0] == "mode":
            modes.append((int(parts[1]), int(parts[2])))
        else:
            vals[parts[0]] = int(parts[1])
    d = workloads.mixed_add(m=8, n=8, k1=128, k2=8)   # shapes only checked on defaults below
    import inspect
    sig = inspect.signature(workloads.mixed_add).parameters
    assert (sig["m"].default, sig["k1"].default, sig["k2"].default, sig["n"].default) == \
        (vals["L"], vals["D1"], vals["D2"], vals["D"])
    assert d["x2"].dtype == np.uint16
    rng = np.random.default_rng(37)
    xq = workloads.random_e4m3_codes(rng, (130, 128))
    wq = workloads.random_e4m3_codes(rng, (129, 128))
    for gm, gn in modes:
        sx = workloads.random_scales(rng, (-(-130 // gm), 1))
        sw = workloads.random_scales(rng, (-(-129 // gn), 1))
        assert oracle.fp8_gemm_groupwise(xq, sx, gm, wq, sw, gn).shape == (130, 129)
    assert sorted(modes) == [(1, 1), (1, 128), (128, 1), (128, 128)]
