"""GPU parity of scales constant along K (rowwise / tensorwise, applied once
after the K loop in the large-M kernels) and of the batched ("L" mode) GEMMs,
against the oracle: ragged shapes, both output forms, fp32 and bf16 outputs,
dense / canonical 2:4 / packed 2:4 weights, FP8 and int8 codes, the decode
sizes (which keep the per-block kernels), and the full 2048 x 4096 x 4096
size on sampled outputs."""
import numpy as np
import pytest
import torch

import oracle
import sparse_gemm_layers_amd as sg
import workloads
from gpu_helpers import DEV, assert_within_tolerance, down, say, up

pytestmark = pytest.mark.gpu


def rowwise_operands(m, n, k, seed, tensor=False, int8=False, sparse=True):
    """Codes with one scale per row over the whole row (the oracle's quantiser
    with one block per row), or one per tensor (one block for the tensor)."""
    d = workloads.sparse_large(seed=seed, m=m, n=n, k=k)
    quant = oracle.int8_quant_groupwise if int8 else oracle.fp8_quant_groupwise
    xq, sx = quant(d["x"], m if tensor else 1, k)
    if sparse:
        wv32, meta = oracle.prune_compress24(d["w"])
        wq, sw = quant(wv32, n if tensor else 1, k // 2)
    else:
        wq, sw = quant(d["w"], n if tensor else 1, k)
        meta = None
    return xq, sx[:, 0].copy(), wq, meta, sw[:, 0].copy()


def run_rowwise(kind, xq, sx, wq, meta, sw, n, k, out_dtype, form, int8=False):
    m = xq.shape[0]
    sxt = sg.k_constant_scales(up(sx), m, k)
    swt = sg.k_constant_scales(up(sw), n, k)
    if kind == "dense":
        return sg.fp8_gemm_groupwise(up(xq), sxt, up(wq), swt, 1, 1, out_dtype=out_dtype, form=form)
    if kind == "sparse":
        f = sg.int8_sparse24_gemm_groupwise if int8 else sg.fp8_sparse24_gemm_groupwise
        return f(up(xq), sxt, up(wq), up(meta), swt, 1, 1, out_dtype=out_dtype, form=form)
    wp = sg.sparse24_pack_gfx950(up(wq), up(meta))
    f = sg.int8_sparse24_gemm_groupwise_packed if int8 else sg.fp8_sparse24_gemm_groupwise_packed
    return f(up(xq), sxt, wp, n, swt, 1, 1, out_dtype=out_dtype, form=form)


def check_rowwise(kind, m, n, k, seed, tensor=False, int8=False, out_dtype=torch.bfloat16, forms=("y", "yt")):
    say(f"rowwise {kind} M={m} N={n} K={k} tensor={tensor} int8={int8} {out_dtype} seed={seed}")
    xq, sx, wq, meta, sw = rowwise_operands(m, n, k, seed, tensor, int8, sparse=kind != "dense")
    if kind == "dense":
        ref, bound = oracle.fp8_gemm_rowwise(xq, sx, wq, sw, bound=True)
    elif int8:
        ref, bound = oracle.int8_sparse24_gemm_rowwise(xq, sx, wq, meta, sw, bound=True)
    else:
        ref, bound = oracle.fp8_sparse24_gemm_rowwise(xq, sx, wq, meta, sw, bound=True)
    outs = {}
    for form in forms:
        got = down(run_rowwise(kind, xq, sx, wq, meta, sw, n, k, out_dtype, form, int8))
        got = got.T if form == "yt" else got
        assert got.shape == (m, n)
        assert_within_tolerance(got.astype(np.float64), ref, bound, f"form={form}")
        outs[form] = got
    if len(outs) == 2:
        assert np.array_equal(outs["y"], outs["yt"])


# M > 64 takes the accumulate-then-scale kernels; partial M and N tiles, K
# blocks of either parity (the last double stage half full), and M <= 64
# (the per-block decode kernels reading repeated scales).
SHAPES = [(65, 256, 128), (128, 256, 256), (200, 300, 384), (129, 513, 640), (300, 1000, 896),
          (16, 256, 256), (37, 300, 384)]


@pytest.mark.parametrize("kind", ["packed", "sparse", "dense"])
@pytest.mark.parametrize("m,n,k", SHAPES)
def test_rowwise_ragged(kind, m, n, k):
    check_rowwise(kind, m, n, k, seed=m + n + k)


@pytest.mark.parametrize("kind", ["packed", "dense"])
@pytest.mark.parametrize("m", [16, 200])
def test_tensorwise(kind, m):
    check_rowwise(kind, m, 384, 512, seed=31 + m, tensor=True)


@pytest.mark.parametrize("kind", ["packed", "sparse"])
@pytest.mark.parametrize("m,n,k", [(65, 256, 128), (200, 300, 384), (300, 700, 1024), (37, 512, 256)])
def test_int8_rowwise_exact_sums(kind, m, n, k):
    check_rowwise(kind, m, n, k, seed=7 * m + n, int8=True)


@pytest.mark.parametrize("kind", ["packed", "dense"])
def test_rowwise_fp32_output(kind):
    check_rowwise(kind, 150, 260, 384, seed=41, out_dtype=torch.float32)


def test_rowwise_128_row_blocks_constant_along_k():
    """gran 128 with K-block stride 0: one scale per 128 rows for all of K."""
    m, n, k = 200, 384, 512
    say(f"rowwise gran 128 M={m} N={n} K={k}")
    d = workloads.sparse_large(seed=43, m=m, n=n, k=k)
    xq, sx = oracle.fp8_quant_groupwise(d["x"], 128, k)
    wv32, meta = oracle.prune_compress24(d["w"])
    wq, sw = oracle.fp8_quant_groupwise(wv32, 128, k // 2)
    kb = k // 128
    sxe, swe = np.repeat(sx, kb, axis=1), np.repeat(sw, kb, axis=1)
    ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq, sxe, 128, wq, meta, swe, 128, bound=True)
    sxt = up(sx[:, 0].copy())[:, None].expand(sx.shape[0], kb)
    swt = up(sw[:, 0].copy())[:, None].expand(sw.shape[0], kb)
    wp = sg.sparse24_pack_gfx950(up(wq), up(meta))
    got = down(sg.fp8_sparse24_gemm_groupwise_packed(up(xq), sxt, wp, n, swt, 128, 128))
    assert_within_tolerance(got, ref, bound, "gran 128")


def test_rowwise_full_size_sampled():
    """2048 x 4096 x 4096 packed 2:4, rowwise scales, in the launch the benchmark
    times; 4096 sampled outputs against the oracle, computed one by one."""
    m, n, k = 2048, 4096, 4096
    say(f"rowwise full size M={m} N={n} K={k}")
    xq, sx, wq, meta, sw = rowwise_operands(m, n, k, seed=44)
    got = down(run_rowwise("packed", xq, sx, wq, meta, sw, n, k, torch.bfloat16, "y"))
    rng = np.random.default_rng(45)
    rows = np.concatenate([[0, m - 1], rng.integers(0, m, 62)])
    cols = np.concatenate([[0, n - 1], rng.integers(0, n, 62)])
    wd = oracle.decompress24(wq[cols], meta[cols])
    ref, bound = oracle.fp8_gemm_rowwise(xq[rows], sx[rows], wd, sw[cols], bound=True)
    assert_within_tolerance(got[np.ix_(rows, cols)], ref, bound, "full size sample")


# --------------------------------------------------------------- batched

def batched_operands(L, m, n, k, seed, gm=1, gn=128):
    xs, sxs, wqs, metas, sws = [], [], [], [], []
    for z in range(L):
        d = workloads.sparse_large(seed=seed + z, m=m, n=n, k=k)
        xq, sx = oracle.fp8_quant_groupwise(d["x"], gm, 128)
        wv32, meta = oracle.prune_compress24(d["w"])
        wq, sw = oracle.fp8_quant_groupwise(wv32, gn, 64)
        xs.append(xq); sxs.append(sx); wqs.append(wq); metas.append(meta); sws.append(sw)
    return [np.stack(a) for a in (xs, sxs, wqs, metas, sws)]


def up_scales3(s):
    """[L, rows, KB] oracle scales -> device [L, rows, KB] view, each problem M-major."""
    return torch.from_numpy(np.ascontiguousarray(np.swapaxes(s, 1, 2))).to(DEV).transpose(1, 2)


@pytest.mark.parametrize("kind", ["packed", "sparse", "dense"])
@pytest.mark.parametrize("L,m,n,k,form", [(3, 200, 300, 384, "y"), (2, 16, 512, 256, "y"), (4, 129, 256, 256, "yt"),
                                          (1, 70, 260, 128, "y")])
def test_batched(kind, L, m, n, k, form):
    say(f"batched {kind} L={L} M={m} N={n} K={k} form={form}")
    xq, sx, wq, meta, sw = batched_operands(L, m, n, k, seed=50 + L + m)
    if kind == "dense":
        wd = np.stack([oracle.decompress24(wq[z], meta[z]) for z in range(L)])
        y = sg.fp8_gemm_groupwise_batched(up(xq), up_scales3(sx), up(wd), up_scales3(sw), 1, 128, form=form)
    elif kind == "sparse":
        y = sg.fp8_sparse24_gemm_groupwise_batched(up(xq), up_scales3(sx), up(wq), up(meta), up_scales3(sw), 1, 128,
                                                   form=form)
    else:
        wp = torch.stack([sg.sparse24_pack_gfx950(up(wq[z]), up(meta[z])) for z in range(L)])
        y = sg.fp8_sparse24_gemm_groupwise_packed_batched(up(xq), up_scales3(sx), wp, n, up_scales3(sw), 1, 128,
                                                          form=form)
    got = down(y)
    for z in range(L):
        ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq[z], sx[z], 1, wq[z], meta[z], sw[z], 128, bound=True)
        gz = got[z].T if form == "yt" else got[z]
        assert_within_tolerance(gz, ref, bound, f"problem {z}")


@pytest.mark.parametrize("m", [16, 200])
def test_batched_shared_weight_and_rowwise(m):
    """One packed weight for every problem (batch stride 0), rowwise scales."""
    L, n, k = 3, 384, 512
    say(f"batched shared weight rowwise L={L} M={m} N={n} K={k}")
    d = [workloads.sparse_large(seed=60 + z, m=m, n=n, k=k) for z in range(L)]
    wv32, meta = oracle.prune_compress24(d[0]["w"])
    wq, sw = oracle.fp8_quant_groupwise(wv32, 1, k // 2)
    xs = [oracle.fp8_quant_groupwise(dz["x"], 1, k) for dz in d]
    xq = np.stack([a for a, _ in xs])
    sx = np.stack([s[:, 0] for _, s in xs])                        # [L, M]
    sxt = up(sx)[:, :, None].expand(L, m, k // 128)
    swt = sg.k_constant_scales(up(sw[:, 0].copy()), n, k)
    wp = sg.sparse24_pack_gfx950(up(wq), up(meta))
    got = down(sg.fp8_sparse24_gemm_groupwise_packed_batched(up(xq), sxt, wp, n, swt, 1, 1))
    for z in range(L):
        ref, bound = oracle.fp8_sparse24_gemm_rowwise(xq[z], sx[z], wq, meta, sw[:, 0], bound=True)
        assert_within_tolerance(got[z], ref, bound, f"problem {z}")


def test_batched_output_leaves_other_memory_alone():
    """Problem z writes only its own slice of a padded output."""
    L, m, n, k = 3, 100, 260, 256
    say(f"batched padded output L={L} M={m} N={n} K={k}")
    xq, sx, wq, meta, sw = batched_operands(L, m, n, k, seed=70)
    ybuf = torch.full((L, m + 3, n + 8), 5.0, dtype=torch.bfloat16, device=DEV)
    wp = torch.stack([sg.sparse24_pack_gfx950(up(wq[z]), up(meta[z])) for z in range(L)])
    sg.fp8_sparse24_gemm_groupwise_packed_batched(up(xq), up_scales3(sx), wp, n, up_scales3(sw), 1, 128,
                                                  y=ybuf[:, :m, :n])
    yb = down(ybuf)
    assert np.all(yb[:, m:, :] == 5.0) and np.all(yb[:, :, n:] == 5.0)
    for z in range(L):
        ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq[z], sx[z], 1, wq[z], meta[z], sw[z], 128, bound=True)
        assert_within_tolerance(yb[z, :m, :n], ref, bound, f"problem {z}")


# --------------------------------------------------------------- bias

@pytest.mark.parametrize("kind", ["packed", "sparse", "dense"])
@pytest.mark.parametrize("L,m,n,k,form,out", [(2, 200, 300, 384, "y", torch.bfloat16),
                                              (1, 16, 520, 256, "yt", torch.bfloat16),
                                              (2, 129, 256, 128, "yt", torch.float32),
                                              (3, 37, 260, 384, "y", torch.float32)])
def test_bias(kind, L, m, n, k, form, out):
    say(f"bias {kind} L={L} M={m} N={n} K={k} form={form} {out}")
    xq, sx, wq, meta, sw = batched_operands(L, m, n, k, seed=80 + m + n)
    bias = (np.random.default_rng(81 + n).standard_normal((L, n)) * 0.5).astype(np.float32)
    bt = up(bias)
    if kind == "dense":
        wd = np.stack([oracle.decompress24(wq[z], meta[z]) for z in range(L)])
        y = sg.fp8_gemm_groupwise_batched(up(xq), up_scales3(sx), up(wd), up_scales3(sw), 1, 128, out_dtype=out,
                                          form=form, bias=bt)
    elif kind == "sparse":
        y = sg.fp8_sparse24_gemm_groupwise_batched(up(xq), up_scales3(sx), up(wq), up(meta), up_scales3(sw), 1, 128,
                                                   out_dtype=out, form=form, bias=bt)
    else:
        wp = torch.stack([sg.sparse24_pack_gfx950(up(wq[z]), up(meta[z])) for z in range(L)])
        y = sg.fp8_sparse24_gemm_groupwise_packed_batched(up(xq), up_scales3(sx), wp, n, up_scales3(sw), 1, 128,
                                                          out_dtype=out, form=form, bias=bt)
    got = down(y)
    for z in range(L):
        ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq[z], sx[z], 1, wq[z], meta[z], sw[z], 128, bound=True)
        ref, bound = oracle.add_bias(ref, bound, bias[z])
        gz = got[z].T if form == "yt" else got[z]
        assert_within_tolerance(gz.astype(np.float64), ref, bound, f"problem {z}")


@pytest.mark.parametrize("kind", ["packed", "dense"])
@pytest.mark.parametrize("m", [16, 300])
def test_rowwise_with_shared_bias(kind, m):
    """Scales constant along K (accumulate-then-scale for M > 64) plus one bias
    shared by the batch."""
    L, n, k = 2, 392, 512
    say(f"rowwise + shared bias {kind} L={L} M={m} N={n} K={k}")
    ops = [rowwise_operands(m, n, k, seed=90 + z, sparse=kind != "dense") for z in range(L)]
    bias = (np.random.default_rng(91).standard_normal(n) * 2).astype(np.float32)
    xq = np.stack([o[0] for o in ops])
    sxt = up(np.stack([o[1] for o in ops]))[:, :, None].expand(L, m, k // 128)
    swt = up(np.stack([o[4] for o in ops]))[:, :, None].expand(L, n, k // 128)
    if kind == "dense":
        y = sg.fp8_gemm_groupwise_batched(up(xq), sxt, up(np.stack([o[2] for o in ops])), swt, 1, 1, bias=up(bias))
    else:
        wp = torch.stack([sg.sparse24_pack_gfx950(up(o[2]), up(o[3])) for o in ops])
        y = sg.fp8_sparse24_gemm_groupwise_packed_batched(up(xq), sxt, wp, n, swt, 1, 1, bias=up(bias))
    got = down(y)
    for z, (xqz, sxz, wqz, metaz, swz) in enumerate(ops):
        if kind == "dense":
            ref, bound = oracle.fp8_gemm_rowwise(xqz, sxz, wqz, swz, bound=True)
        else:
            ref, bound = oracle.fp8_sparse24_gemm_rowwise(xqz, sxz, wqz, metaz, swz, bound=True)
        ref, bound = oracle.add_bias(ref, bound, bias)
        assert_within_tolerance(got[z], ref, bound, f"problem {z}")


# --------------------------------------------------------------- rowwise / tensorwise quantiser

@pytest.mark.parametrize("int8", [False, True])
@pytest.mark.parametrize("bf16", [False, True])
@pytest.mark.parametrize("whole,rows,cols", [("rows", 37, 4096), ("rows", 2, 14336), ("rows", 300, 384),
                                             ("rows", 1, 16), ("tensor", 300, 128), ("tensor", 64, 512),
                                             ("tensor", 1, 256), ("tensor", 129, 4096)])
def test_whole_row_and_tensor_quant_bit_exact(whole, rows, cols, bf16, int8):
    say(f"quant whole={whole} {rows}x{cols} bf16={bf16} int8={int8}")
    x = workloads.sparse_large(seed=rows + cols, m=rows, n=8, k=cols)["x"]
    if rows > 3:
        x[3] = 0.0                                               # an all-zero row
    xt = up(x)
    if bf16:
        xt = xt.to(torch.bfloat16)
        x = xt.float().cpu().numpy()
    gr = 1 if whole == "rows" else rows
    f = sg.int8_quant_groupwise if int8 else sg.fp8_quant_groupwise
    q, s = f(xt, gr=gr, gc=cols)
    rq, rs = (oracle.int8_quant_groupwise if int8 else oracle.fp8_quant_groupwise)(x, gr, cols)
    assert np.array_equal(down(q), rq)
    assert np.array_equal(down(s), rs)


def test_all_zero_tensor_gets_unit_scale():
    say("quant tensor all zero")
    q, s = sg.fp8_quant_groupwise(torch.zeros((40, 256), device=DEV), gr=40, gc=256)
    assert np.array_equal(down(s), np.ones((1, 1), np.float32)) and not down(q).any()


@pytest.mark.parametrize("m", [16, 300])
def test_rowwise_end_to_end_on_the_gpu(m):
    """GPU rowwise quantisation of X and of the pruned W, then the packed 2:4
    GEMM with those scales constant along K, against the oracle's chain."""
    n, k = 512, 1024
    say(f"rowwise end to end M={m} N={n} K={k}")
    d = workloads.sparse_large(seed=95 + m, m=m, n=n, k=k)
    wv32, meta = sg.sparse24_prune_compress(up(d["w"]))
    wq, sw = sg.fp8_quant_groupwise(wv32, gr=1, gc=k // 2)
    xq, sx = sg.fp8_quant_groupwise(up(d["x"]), gr=1, gc=k)
    wp = sg.sparse24_pack_gfx950(wq, meta)
    y = down(sg.fp8_sparse24_gemm_groupwise_packed(xq, sg.k_constant_scales(sx[:, 0], m, k), wp, n,
                                                   sg.k_constant_scales(sw[:, 0], n, k), 1, 1))
    oxq, osx = oracle.fp8_quant_groupwise(d["x"], 1, k)
    ov32, ometa = oracle.prune_compress24(d["w"])
    owq, osw = oracle.fp8_quant_groupwise(ov32, 1, k // 2)
    assert np.array_equal(down(xq), oxq) and np.array_equal(down(sx), osx)
    assert np.array_equal(down(wq), owq) and np.array_equal(down(sw), osw)
    ref, bound = oracle.fp8_sparse24_gemm_rowwise(oxq, osx[:, 0], owq, ometa, osw[:, 0], bound=True)
    assert_within_tolerance(y, ref, bound, "end to end")


def test_batched_full_size_sampled():
    """The benchmark's batched launch: 8 problems of 256 x 4096 x 4096, each
    with its own packed 2:4 weight; sampled outputs of every problem against
    the oracle, computed one by one."""
    L, m, n, k = 8, 256, 4096, 4096
    say(f"batched full size L={L} M={m} N={n} K={k}")
    xq, sx, wq, meta, sw = batched_operands(L, m, n, k, seed=100)
    wp = torch.stack([sg.sparse24_pack_gfx950(up(wq[z]), up(meta[z])) for z in range(L)])
    got = down(sg.fp8_sparse24_gemm_groupwise_packed_batched(up(xq), up_scales3(sx), wp, n, up_scales3(sw), 1, 128))
    rng = np.random.default_rng(101)
    for z in range(L):
        rows = np.concatenate([[0, m - 1], rng.integers(0, m, 14)])
        cols = np.concatenate([[0, n - 1], rng.integers(0, n, 30)])
        ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq[z][rows], sx[z][rows], 1, wq[z][cols], meta[z][cols],
                                                         sw[z][cols // 128], 1, bound=True)
        assert_within_tolerance(got[z][np.ix_(rows, cols)], ref, bound, f"problem {z}")


@pytest.mark.parametrize("whole", ["rows", "tensor"])
def test_whole_row_and_tensor_quant_full_size(whole):
    """The benchmark's 2048 x 4096 activation, bit-exact."""
    m, k = 2048, 4096
    say(f"quant full size whole={whole}")
    x = workloads.sparse_large(seed=3, m=m, n=8, k=k)["x"]
    gr = 1 if whole == "rows" else m
    q, s = sg.fp8_quant_groupwise(up(x), gr=gr, gc=k)
    rq, rs = oracle.fp8_quant_groupwise(x, gr, k)
    assert np.array_equal(down(q), rq) and np.array_equal(down(s), rs)


# --------------------------------------------------------------- grouped (ragged M)

def grouped_operands(sizes, n, k, seed, gn=128):
    """X rows of all groups one after another (1 x 128 scales), one pruned,
    quantised, packed weight per group."""
    m = sum(sizes)
    d = workloads.sparse_large(seed=seed, m=max(m, 1), n=8, k=k)
    xq, sx = oracle.fp8_quant_groupwise(d["x"][:m], 1, 128)
    ws = []
    for g in range(len(sizes)):
        w = workloads.sparse_large(seed=seed + 1 + g, m=1, n=n, k=k)["w"]
        wv32, meta = oracle.prune_compress24(w)
        wq, sw = oracle.fp8_quant_groupwise(wv32, gn, 64)
        ws.append((wq, meta, sw))
    return xq, sx, ws


@pytest.mark.parametrize("sizes,form,out,gn", [([300, 0, 1, 128, 129, 64], "y", torch.bfloat16, 128),
                                               ([5, 7, 300], "yt", torch.bfloat16, 128),
                                               ([200, 72], "yt", torch.float32, 1),
                                               ([16], "y", torch.float32, 128),
                                               # every group <= 48 rows: the decode-sized grouped kernel
                                               ([1, 0, 17, 48, 33], "yt", torch.bfloat16, 128),
                                               ([16, 16, 3, 9], "y", torch.float32, 128),
                                               ([20, 32], "y", torch.bfloat16, 128),
                                               ([7, 40], "yt", torch.float32, 128),
                                               ([64, 0, 49, 3], "y", torch.bfloat16, 128)])
def test_grouped(sizes, form, out, gn):
    n, k = 384, 512
    say(f"grouped sizes={sizes} N={n} K={k} form={form} {out} gn={gn}")
    xq, sx, ws = grouped_operands(sizes, n, k, seed=110 + len(sizes), gn=gn)
    wp = torch.stack([sg.sparse24_pack_gfx950(up(wq), up(meta)) for wq, meta, _ in ws])
    sw = torch.stack([up_m_major(s) for _, _, s in ws])
    bias = (np.random.default_rng(111).standard_normal((len(sizes), n))).astype(np.float32)
    got = down(sg.fp8_sparse24_gemm_groupwise_packed_grouped(up(xq), up_m_major(sx), sizes, wp, n, sw, gn,
                                                             out_dtype=out, form=form, bias=up(bias)))
    got = got.T if form == "yt" else got
    assert got.shape == (sum(sizes), n)
    r = 0
    for g, mg in enumerate(sizes):
        if mg:
            wq, meta, swg = ws[g]
            ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq[r:r + mg], sx[r:r + mg], 1, wq, meta, swg, gn,
                                                             bound=True)
            ref, bound = oracle.add_bias(ref, bound, bias[g])
            assert_within_tolerance(got[r:r + mg].astype(np.float64), ref, bound, f"group {g}")
        r += mg


@pytest.mark.parametrize("sizes,form", [([5, 16, 1, 12, 0, 16, 7, 2], "y"), ([3, 9], "yt"),
                                        ([64, 33, 0, 20, 64, 1, 40, 9], "yt")])
def test_grouped_decode_wide(sizes, form):
    """MoE decode: many small groups over a wide weight (four row blocks per
    workgroup for the 8-group and the 64-row cases, one for the 2-group case)."""
    n, k = 4096, 1024
    say(f"grouped decode sizes={sizes} N={n} K={k} form={form}")
    xq, sx, ws = grouped_operands(sizes, n, k, seed=130 + len(sizes))
    wp = torch.stack([sg.sparse24_pack_gfx950(up(wq), up(meta)) for wq, meta, _ in ws])
    sw = torch.stack([up_m_major(s) for _, _, s in ws])
    got = down(sg.fp8_sparse24_gemm_groupwise_packed_grouped(up(xq), up_m_major(sx), sizes, wp, n, sw, 128,
                                                             out_dtype=torch.bfloat16, form=form))
    got = got.T if form == "yt" else got
    r = 0
    for g, mg in enumerate(sizes):
        if mg:
            wq, meta, swg = ws[g]
            ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq[r:r + mg], sx[r:r + mg], 1, wq, meta, swg, 128,
                                                             bound=True)
            assert_within_tolerance(got[r:r + mg].astype(np.float64), ref, bound, f"group {g}")
        r += mg


# Ragged groups whose large tiles would need a second round over the CUs:
# each group's last <= 64 rows take the grouped decode kernel instead, with
# as many 16-row sub-tiles as the tail needs (1 row: one; 20 / 32 rows: two;
# 44 / 40 rows: three; 64 rows: four).
@pytest.mark.parametrize("sizes,form,out", [([300] * 6 + [40], "y", torch.bfloat16),
                                            ([320] * 7 + [64], "yt", torch.float32),
                                            ([0, 300, 1, 300, 300, 300, 300, 300, 44], "y", torch.bfloat16),
                                            ([276] * 6 + [20, 160], "yt", torch.bfloat16)])
def test_grouped_tails_on_the_decode_kernel(sizes, form, out):
    n, k = 4096, 256
    say(f"grouped tails sizes={sizes} N={n} K={k} form={form} {out}")
    xq, sx, ws = grouped_operands(sizes, n, k, seed=140 + len(sizes))
    wp = torch.stack([sg.sparse24_pack_gfx950(up(wq), up(meta)) for wq, meta, _ in ws])
    sw = torch.stack([up_m_major(s) for _, _, s in ws])
    bias = (np.random.default_rng(141).standard_normal((len(sizes), n))).astype(np.float32)
    got = down(sg.fp8_sparse24_gemm_groupwise_packed_grouped(up(xq), up_m_major(sx), sizes, wp, n, sw, 128,
                                                             out_dtype=out, form=form, bias=up(bias)))
    got = got.T if form == "yt" else got
    r = 0
    for g, mg in enumerate(sizes):
        if mg:
            wq, meta, swg = ws[g]
            ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq[r:r + mg], sx[r:r + mg], 1, wq, meta, swg, 128,
                                                             bound=True)
            ref, bound = oracle.add_bias(ref, bound, bias[g])
            assert_within_tolerance(got[r:r + mg].astype(np.float64), ref, bound, f"group {g}")
        r += mg


def test_grouped_maximum_group_count():
    """64 groups (the most one call takes), ragged sizes with empty groups."""
    sizes = [int(v) for v in np.random.default_rng(150).integers(0, 300, size=64)]
    sizes[5] = sizes[40] = 0
    n, k = 768, 128   # 303 large tiles (two rounds over 256 CUs), 201 with the tails split off
    say(f"grouped G=64 M={sum(sizes)} N={n} K={k}")
    xq, sx, ws = grouped_operands(sizes, n, k, seed=151)
    wp = torch.stack([sg.sparse24_pack_gfx950(up(wq), up(meta)) for wq, meta, _ in ws])
    sw = torch.stack([up_m_major(s) for _, _, s in ws])
    got = down(sg.fp8_sparse24_gemm_groupwise_packed_grouped(up(xq), up_m_major(sx), sizes, wp, n, sw, 128))
    r = 0
    for g, mg in enumerate(sizes):
        if mg:
            wq, meta, swg = ws[g]
            ref, bound = oracle.fp8_sparse24_gemm_groupwise(xq[r:r + mg], sx[r:r + mg], 1, wq, meta, swg, 128,
                                                             bound=True)
            assert_within_tolerance(got[r:r + mg].astype(np.float64), ref, bound, f"group {g}")
        r += mg


def test_grouped_rowwise_scales():
    sizes, n, k = [130, 3, 257], 512, 640
    say(f"grouped rowwise sizes={sizes} N={n} K={k}")
    m = sum(sizes)
    d = workloads.sparse_large(seed=120, m=m, n=8, k=k)
    xq, sx = oracle.fp8_quant_groupwise(d["x"], 1, k)
    ops = []
    for g in range(len(sizes)):
        w = workloads.sparse_large(seed=121 + g, m=1, n=n, k=k)["w"]
        wv32, meta = oracle.prune_compress24(w)
        wq, sw = oracle.fp8_quant_groupwise(wv32, 1, k // 2)
        ops.append((wq, meta, sw[:, 0].copy()))
    wp = torch.stack([sg.sparse24_pack_gfx950(up(wq), up(meta)) for wq, meta, _ in ops])
    swt = up(np.stack([s for _, _, s in ops]))[:, :, None].expand(len(sizes), n, k // 128)
    sxt = sg.k_constant_scales(up(sx[:, 0].copy()), m, k)
    got = down(sg.fp8_sparse24_gemm_groupwise_packed_grouped(up(xq), sxt, sizes, wp, n, swt, 1))
    r = 0
    for g, mg in enumerate(sizes):
        wq, meta, swg = ops[g]
        ref, bound = oracle.fp8_sparse24_gemm_rowwise(xq[r:r + mg], sx[r:r + mg, 0], wq, meta, swg, bound=True)
        assert_within_tolerance(got[r:r + mg], ref, bound, f"group {g}")
        r += mg


def up_m_major(s):
    """[rows, KB] scales -> device view stored M-major."""
    return torch.from_numpy(np.ascontiguousarray(s.T)).to(DEV).t()
