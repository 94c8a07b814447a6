"""sdm_overlap, the write/read bucket-overlap diagnostic, through the C ABI.

Staged as for the forward: the GPU's slots against the oracle's (a difference excused only at a
near-tie), then the diagnostic oracle driven by the GPU's slots and weights.  The bucket masses are
the same double sums in the same order, so they match bit for bit; an overlap value is a sum of at
most W exact products whose order differs, so it matches within one float32 unit.  On the planted
needle (the read query of token T - 17 is the write query of token 61) the query reads exactly the
slots the needle wrote, and the overlap peaks there.
"""
import sys

import numpy as np
import pytest

import oracle
import sdm_inputs as gi
from parity import compare_index_sets, to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _addressing(cfg, x):
    import torch
    from sparse_memory_linear_pk_amd import SDM
    R = cfg.B * cfg.T * cfg.H
    out = {}
    with SDM.from_config(cfg) as layer:
        for s_, q in (("w", "wq"), ("r", "rq")):
            idx = torch.empty((R, cfg.W), dtype=torch.int32, device="cuda")
            wt = torch.empty((R, cfg.W), dtype=torch.float32, device="cuda")
            layer.address(to_dev(x[q]), to_dev(x["subkeys"]), idx, wt)
            out[s_] = (idx, wt)
        torch.cuda.synchronize()
    return out


def _run(cfg, addr, K, queries):
    import torch
    from sparse_memory_linear_pk_amd import SDM
    f32 = dict(dtype=torch.float32, device="cuda")
    wc = torch.full((cfg.B, cfg.H, cfg.T, K), float("nan"), **f32)
    rd = torch.full_like(wc, float("nan"))
    q = torch.tensor(queries, dtype=torch.int32, device="cuda")
    ov = torch.full((cfg.B, cfg.H, len(queries), cfg.T), float("nan"), **f32)
    with SDM.from_config(cfg) as layer:
        layer.overlap(addr["w"][0], addr["w"][1], addr["r"][0], addr["r"][1], K, wc, rd, q, ov)
        torch.cuda.synchronize()
    return to_host(wc), to_host(rd), to_host(ov)


CASES = {
    "planted_needle_1.4B_addressing": (gi.config(3, T=256), 480, [239, 100, 0, 255]),
    "two_heads_small_buckets": (gi.config(1, B=2, T=96, H=2), 7, [95, 50, -3, 96]),
}


@pytest.mark.parametrize("name", list(CASES))
def test_overlap_matches_the_oracle(name):
    cfg, K, queries = CASES[name]
    say(f"[overlap {name}] K={K} queries={queries} {cfg}")
    orc = oracle.get()
    x = gi.make_inputs(cfg, with_mem0=False)
    addr = _addressing(cfg, x)
    host = {s_: (to_host(i), to_host(w)) for s_, (i, w) in addr.items()}
    for s_, q in (("w", x["wq"]), ("r", x["rq"])):
        ri, rw, rs = orc.address(cfg, q, x["subkeys"])
        differ, exc = compare_index_sets(orc, cfg, host[s_][0], ri, rs, orc.scores(cfg, q, x["subkeys"]))
        say(f"[overlap {name}] {s_}: rows differing {differ} (excused {exc})")
    wc, rd, ov = _run(cfg, addr, K, queries)
    # a query outside [0, T) gives a zero row; the oracle takes only valid ones
    valid = [i for i, q in enumerate(queries) if 0 <= q < cfg.T]
    rwc, rrd, rov = oracle.get_proj().overlap(cfg.B, cfg.T, cfg.H, cfg.W, cfg.N, K, host["w"][0], host["w"][1],
                                              host["r"][0], host["r"][1], [queries[i] for i in valid])
    assert np.array_equal(wc.view(np.uint32), rwc.view(np.uint32))
    assert np.array_equal(rd.view(np.uint32), rrd.view(np.uint32))
    got = ov[:, :, valid]
    assert np.all(np.abs(got - rov) <= 2.0 ** -23 * np.abs(rov) + 1e-30)
    for i, q in enumerate(queries):
        if not 0 <= q < cfg.T:
            assert np.all(ov[:, :, i] == 0)
    if name.startswith("planted"):
        curve = ov[0, 0, 0]
        w61 = host["w"][1][61].astype(np.float64)
        say(f"[overlap {name}] query 239: peak at token {int(np.argmax(curve))}, value {curve.max():.4f}, "
            f"sum of squared needle weights {np.sum(w61 * w61):.4f}")
        assert int(np.argmax(curve)) == 61 and curve[61] == np.float32(np.sum(w61 * w61))
