"""pk_topk through the sdm_select seam on crafted half scores, against the
oracle's selection of the very same scores: indices bit-exact, weights within
one ulp.  The scores are built to hit every exact path of the kernel: heavy
ties inside a half (more than 64 scores at the per-half bound), float sums that
tie although their half scores differ (then slot order decides at the W-th
sum), signed zeros, wide magnitudes, and the plain random case.  Then the
forward's addressing (sdm_address, which makes the scores that can reach a top
k exact) from crafted queries and sub-keys against the oracle's addressing."""
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


# ---------------------------------------------------------------------------
# the forward's addressing (sdm_address) from crafted queries and sub-keys
# ---------------------------------------------------------------------------

def _crafted_tables(S, dh, rng, kind):
    """Sub-key tables [1, 2, S, dh] and the rows of the queries they are built for."""
    K = (rng.standard_normal((1, 2, S, dh)) * 0.25).astype(np.float32)
    if kind == "cancellation":
        # row 0: 1 + 2^-25 - 1 (exactly 2^-25; a float32 sum in index order loses it), row 1: 2^-26,
        # both above every other row for a query of ones; the other half the same, shifted by 2
        for half in range(2):
            K[0, half] = -1.0
            K[0, half, 2 * half, :3] = [1.0, 2.0 ** -25, -1.0]
            K[0, half, 2 * half, 3:] = 0.0
            K[0, half, 2 * half + 1] = 0.0
            K[0, half, 2 * half + 1, 0] = 2.0 ** -26
    elif kind == "equal_rows":
        # every sub-key of half 0 the same: more than 64 candidates tie, every score is made exact
        K[0, 0] = K[0, 0, :1]
    elif kind == "duplicate_rows":
        K[0, 1, 1::2] = K[0, 1, ::2][: S // 2]
    elif kind == "near_binary16_limit":
        # sum |q| max |K| just under the forward's binary16 limit: scores near 1000, where a binary16
        # step is 0.5, far wider than the float32 error the threshold otherwise allows for
        K *= 60.0
    elif kind == "beyond_binary16":
        # scores past binary16's range: every score of the half is made exact
        K *= 300.0
    elif kind == "shifted_mean":
        # a common offset far above the spread: the fused scoring's threshold must follow the mean row
        K += 3.0
    elif kind == "low_rank":
        # sub-keys along two directions only: scores far from the isotropic spread the threshold
        # assumes, so many halves take the whole-half rescoring
        K = (rng.standard_normal((1, 2, S, 2)) @ rng.standard_normal((2, dh)) * 0.25
             + rng.standard_normal((1, 2, S, dh)) * 1e-3).astype(np.float32)
    return K


@pytest.mark.parametrize("in_bf16", [False, True])
@pytest.mark.parametrize("kind,S,k,W", [("cancellation", 8, 1, 1), ("cancellation", 8, 2, 3), ("equal_rows", 100, 6, 20),
                                         ("duplicate_rows", 48, 8, 30), ("random", 480, 32, 64),
                                         ("near_binary16_limit", 480, 32, 64), ("beyond_binary16", 480, 32, 64),
                                         ("equal_rows", 480, 32, 64), ("duplicate_rows", 480, 32, 64),
                                         ("shifted_mean", 480, 32, 64), ("low_rank", 480, 32, 64),
                                         ("random_dh128", 640, 32, 64), ("low_rank_dh128", 480, 16, 40)])
def test_forward_addressing_equals_the_oracle(kind, S, k, W, in_bf16):
    """sdm_address (the forward's addressing) against the oracle's addressing of the same queries:
    the same slots, weights within one float32 unit, also where float32 sums order scores wrongly
    (cancellation), where more than 64 scores of a half tie (every score made exact), and, for bf16
    inputs (whose forward stores binary16 scores), with scores near binary16's range limit, where
    its rounding step is wide, and beyond it.  With bf16 inputs, S a multiple of 32 and dh 64 or
    128 the forward's scoring is fused with the candidate search: tables with equal or duplicated
    rows, a large common offset or two directions only steer its threshold wrong on purpose, and
    every row must still select exactly."""
    import torch
    from parity import to_dev, to_host
    from sdm_inputs import bf16_bits_from_f32, f32_from_bf16_bits
    from sparse_memory_linear_pk_amd import SDM
    orc = oracle.get()
    dh = 16 if kind == "cancellation" else 128 if kind.endswith("_dh128") else 64
    kind = kind.removesuffix("_dh128")
    T = 40
    cfg = gi.config(0).replace(B=1, H=1, T=T, d=8, S=S, dk=2 * dh, k=k, W=W, in_bf16=in_bf16)
    rng = np.random.default_rng(7)
    K = _crafted_tables(S, dh, rng, kind)
    q = rng.standard_normal((1, T, 1, 2 * dh)).astype(np.float32)
    if kind == "cancellation":
        q[:, ::2] = 1.0
        q[:, 1::4] = 2.0
    if kind in ("near_binary16_limit", "beyond_binary16"):
        q *= 8.0 if kind == "near_binary16_limit" else 100.0
    if in_bf16:
        K = bf16_bits_from_f32(K).reshape(K.shape)
        q = bf16_bits_from_f32(q).reshape(q.shape)
    with SDM.from_config(cfg) as layer:
        idx = torch.empty((T, W), dtype=torch.int32, device="cuda")
        wt = torch.empty((T, W), dtype=torch.float32, device="cuda")
        layer.address(to_dev(q), to_dev(K), idx, wt)
        sc = torch.empty((T, 2, S), dtype=torch.float32, device="cuda")
        layer.score(to_dev(q), to_dev(K), sc)
        torch.cuda.synchronize()
    gi_, gw = to_host(idx), to_host(wt)
    ri, rw, _ = orc.address(cfg, q, K)
    fi, _, _ = orc.address_from_scores(cfg, to_host(sc))
    print(f"[exact {kind} bf16={in_bf16}] rows where the float32 scores alone would select differently: "
          f"{int((fi != ri).any(axis=1).sum())} of {T}", flush=True)
    bad = np.nonzero((gi_ != ri).any(axis=1))[0]
    assert bad.size == 0, f"{bad.size} rows differ from the oracle, first {bad[:4]}"
    u = np.abs(gw.view(np.int32).astype(np.int64) - rw.view(np.int32).astype(np.int64))
    assert u.max() <= 1
