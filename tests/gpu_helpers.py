"""Helpers shared by the GPU parity tests: uploads, oracle-side input
preparation and the GEMM comparison against the oracle's tolerance."""
import sys

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")


def say(*args):
    print(*args, flush=True)
    sys.stdout.flush()


def up(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def up_scales(s: np.ndarray, m_major: bool = True) -> torch.Tensor:
    """Oracle scales [row_blocks, k_blocks] -> device view of the same shape,
    stored M-major (column-contiguous) or row-major."""
    if m_major:
        return torch.from_numpy(np.ascontiguousarray(s.T)).to(DEV).t()
    return torch.from_numpy(np.ascontiguousarray(s)).to(DEV)


def down(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def oracle_operands(x, w, gm, gn, sparse):
    """Quantise (and for sparse, prune + compress) with the oracle."""
    xq, sx = oracle.fp8_quant_groupwise(x, gm, 128)
    if sparse:
        wv32, meta = oracle.prune_compress24(w)
        wq, sw = oracle.fp8_quant_groupwise(wv32, gn, 64)
        return xq, sx, wq, meta, sw
    wq, sw = oracle.fp8_quant_groupwise(w, gn, 128)
    return xq, sx, wq, None, sw


def assert_within_tolerance(got: np.ndarray, ref: np.ndarray, bound: np.ndarray, what: str):
    ok = oracle.within_tolerance(got, ref, bound)
    if not ok.all():
        bad = np.argwhere(~ok)
        i, j = bad[0]
        raise AssertionError(f"{what}: {len(bad)} of {ok.size} outputs outside tolerance; first at "
                             f"({i},{j}) got {got[i, j]!r} ref {ref[i, j]!r} T {bound[i, j]!r}")
    err = np.abs(got - ref) / (1e-2 * np.abs(ref) + 1e-3 * bound + 1e-300)
    say(f"  {what}: max |err| / allowed = {err.max():.3g}")
