"""pk_topk through the sdm_select seam on crafted half scores, against the
oracle's selection of the very same scores: indices bit-exact, weights within
one ulp.  The scores are built to hit every exact path of the kernel: heavy
ties inside a half (more than 64 scores at the per-half bound), float sums that
tie although their half scores differ (then slot order decides at the W-th
sum), signed zeros, wide magnitudes, and the plain random case."""
import numpy as np
import pytest

import oracle
import sdm_inputs as gi
from parity import check_selection_exact

pytestmark = pytest.mark.gpu

SHAPES = [(480, 32, 64), (128, 16, 64), (64, 8, 16), (100, 10, 37), (1024, 64, 64), (480, 64, 64),
          (200, 5, 25), (33, 1, 1), (640, 32, 64)]
ROWS = 192


def scores_for(kind, S, rng):
    shape = (ROWS, 2, S)
    if kind == "normal":
        return rng.standard_normal(shape).astype(np.float32)
    if kind == "all_equal":
        return np.full(shape, 0.5, np.float32)
    if kind == "few_levels":
        return rng.integers(0, 6, shape).astype(np.float32)
    if kind == "quantised":
        return (np.round(rng.standard_normal(shape) * 300) / 300).astype(np.float32)
    if kind == "sum_ties":
        # half 0 in [1, 1 + 64 ulp), half 1 in [3, 3 + 64 ulp): distinct half scores whose
        # float sums (spacing 2^-21 in [4, 8)) coincide often
        s = np.empty(shape, np.float32)
        s[:, 0] = (1.0 + rng.integers(0, 64, (ROWS, S)) * 2.0 ** -23).astype(np.float32)
        s[:, 1] = (3.0 + rng.integers(0, 64, (ROWS, S)) * 2.0 ** -22).astype(np.float32)
        return s
    if kind == "signed_zeros":
        s = np.where(rng.random(shape) < 0.5, np.float32(-0.0), np.float32(0.0)).astype(np.float32)
        s[:, :, ::7] = rng.standard_normal(s[:, :, ::7].shape).astype(np.float32) * 1e-3
        return s
    if kind == "wide":
        s = rng.standard_normal(shape).astype(np.float32)
        big = rng.random(shape) < 0.05
        s[big] *= np.float32(1e18)
        return s
    raise ValueError(kind)


KINDS = ["normal", "all_equal", "few_levels", "quantised", "sum_ties", "signed_zeros", "wide"]


@pytest.mark.parametrize("S,k,W", SHAPES)
def test_selection_of_crafted_scores_is_exact(S, k, W):
    import torch
    from sparse_memory_linear_pk_amd import SDM
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    orc = oracle.get()
    cfg = gi.config(0).replace(B=1, H=1, T=ROWS, d=8, S=S, dk=32, k=k, W=W)
    rng = np.random.default_rng(S * 1000 + k * 10 + W)
    with SDM.from_config(cfg) as layer:
        for kind in KINDS:
            sc = scores_for(kind, S, rng)
            print(f"[select {S},{k},{W}] {kind}", flush=True)
            dev = torch.from_numpy(sc).cuda()
            idx = torch.empty((ROWS, W), dtype=torch.int32, device="cuda")
            wt = torch.empty((ROWS, W), dtype=torch.float32, device="cuda")
            layer.select(dev, idx, wt)
            torch.cuda.synchronize()
            ui, uw, _ = orc.address_from_scores(cfg, sc)
            check_selection_exact(idx.cpu().numpy(), wt.cpu().numpy(), ui, uw)
