"""sdm_project (input projections on MFMA) and sdm_broadcast_memory through the C ABI.

Each bf16 output agrees with the oracle's (the exact sum rounded once) within one bf16 unit of the
oracle's value plus twice the float32 accumulation bound of a D-term dot product,
1.01 * D * 2^-24 * sum_k |x_k w_k|: the GPU rounds its float32 sum, which lies within that bound of
the exact one, so the two roundings can differ by at most that much.  The gates agree within a
quarter of the bound (the sigmoid's slope is at most 1/4) plus 1e-6.
"""
import sys

import numpy as np
import pytest

import oracle
import sdm_inputs as gi
from parity import to_dev, to_host
from sdm_inputs import f32_from_bf16_bits

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _cfg(**kw):
    base = dict(name="proj", B=2, H=2, T=50, d=32, S=16, dk=32, k=4, W=8, in_bf16=True, state_bf16=False)
    base.update(kw)
    return gi.Config(**base)


CASES = {
    "ragged_two_heads": (_cfg(), 72),
    "one_head": (_cfg(B=1, H=1, T=200, d=96, dk=64), 256),
    "1.4B_columns_T256": (gi.config(2, B=1, T=256), 2048),
    "three_heads_tail": (_cfg(B=3, H=3, T=37, d=40, dk=32), 136),
}


def _bf(a):
    return f32_from_bf16_bits(a).reshape(a.shape).astype(np.float64)


@pytest.mark.parametrize("name", list(CASES))
def test_projection_matches_the_oracle(name):
    import torch
    from sparse_memory_linear_pk_amd import SDM
    cfg, D = CASES[name]
    say(f"[project {name}] D={D} {cfg}")
    p = gi.make_projection_inputs(cfg, D)
    dev = {k: to_dev(v) for k, v in p.items()}
    B, T, H, dk, d = cfg.B, cfg.T, cfg.H, cfg.dk, cfg.d
    bf = dict(dtype=torch.bfloat16, device="cuda")
    out = {"wq": torch.empty((B, T, H, dk), **bf), "rq": torch.empty((B, T, H, dk), **bf),
           "v": torch.empty((B, T, H, d), **bf), "alpha": torch.empty((B, T, H), dtype=torch.float32, device="cuda"),
           "beta": torch.empty((B, T, H), dtype=torch.float32, device="cuda")}
    with SDM.from_config(cfg) as layer:
        layer.project(D, dev["x"], dev["w"], dev["gate_bias"], out["wq"], out["rq"], out["v"], out["alpha"],
                      out["beta"])
        torch.cuda.synchronize()
    got = {k: to_host(v) for k, v in out.items()}
    ref = dict(zip(("wq", "rq", "v", "alpha", "beta"), oracle.get_proj().project(B, T, H, D, dk, d, p["x"], p["w"],
                                                                                  p["gate_bias"])))
    # |x| |w|^T per (row, output column), the accumulation bound's sum
    ax = np.abs(_bf(p["x"])).reshape(B * T, D)
    aw = np.abs(_bf(p["w"]))
    bound = 1.01 * D * 2.0 ** -24 * (ax @ aw.T)            # [rows, H*C]
    C = 2 * dk + d + 2
    bound = bound.reshape(B, T, H, C)
    parts = {"wq": (0, dk), "rq": (dk, 2 * dk), "v": (2 * dk, 2 * dk + d)}
    for k, (lo, hi) in parts.items():
        g, r = _bf(got[k]), _bf(ref[k])
        ulp = np.maximum(np.abs(r), 2.0 ** -126) * 2.0 ** -7
        excess = np.abs(g - r) - (ulp + 2 * bound[..., lo:hi])
        say(f"[project {name}] {k}: max |diff| {np.max(np.abs(g - r)):.3g}, differing {np.mean(g != r):.4f}")
        assert np.all(excess <= 0), f"{k}: {np.sum(excess > 0)} outputs outside the bound"
    for gi_, k in ((0, "alpha"), (1, "beta")):
        lim = 0.25 * bound[..., 2 * dk + d + gi_] + 1e-6
        diff = np.abs(got[k].astype(np.float64) - ref[k].astype(np.float64))
        say(f"[project {name}] {k}: max |diff| {diff.max():.3g}")
        assert np.all(diff <= lim), k


def test_broadcast_memory_copies_bit_for_bit():
    import torch
    from sparse_memory_linear_pk_amd import SDM
    cfg = _cfg(B=3, H=2, S=8, d=64)
    m0 = torch.randn((cfg.H, cfg.N, cfg.d), device="cuda")
    mem = torch.full((cfg.B, cfg.H, cfg.N, cfg.d), float("nan"), device="cuda")
    with SDM.from_config(cfg) as layer:
        layer.broadcast_memory(m0, mem)
        torch.cuda.synchronize()
    ref = oracle.get_proj().broadcast_memory(cfg.B, m0.cpu().numpy())
    assert np.array_equal(mem.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_projection_feeds_the_forward():
    """The projection's outputs are the forward's inputs: one call chain runs end to end and
    matches the forward run on the same (oracle-projected) tensors bit for bit."""
    import torch
    from sparse_memory_linear_pk_amd import SDM
    cfg = gi.config(1, B=1, T=64, in_bf16=True)
    D = 128
    p = gi.make_projection_inputs(cfg, D)
    x = gi.make_inputs(cfg)
    dev = {k: to_dev(v) for k, v in p.items()}
    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    wq = torch.empty((cfg.B, cfg.T, cfg.H, cfg.dk), **bf)
    rq = torch.empty_like(wq)
    v = torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), **bf)
    al = torch.empty((cfg.B, cfg.T, cfg.H), **f32)
    be = torch.empty_like(al)
    sub = to_dev(x["subkeys"])
    with SDM.from_config(cfg) as layer:
        layer.project(D, dev["x"], dev["w"], dev["gate_bias"], wq, rq, v, al, be)
        m0 = to_dev(x["mem0"][0])
        mem = torch.empty((cfg.B, cfg.H, cfg.N, cfg.d), **f32)
        layer.broadcast_memory(m0, mem)
        out = torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), **f32)
        layer.forward(wq, rq, v, al, be, sub, mem, out)
        mem2 = to_dev(np.ascontiguousarray(x["mem0"][:1]))
        out2 = torch.empty_like(out)
        layer.forward(wq.clone(), rq.clone(), v.clone(), al.clone(), be.clone(), sub, mem2, out2)
        torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, out2) and torch.equal(mem, mem2)
