"""sdm_step, the decode step, through the C ABI: T consecutive steps leave
exactly (bit for bit) the memory and outputs of one T-token sdm_forward, and
agree with the oracle."""
import sys

import numpy as np
import pytest

import oracle
import sdm_inputs as gi
from parity import check_scan, compare_index_sets, plain_err, rel_max_err, to_dev, to_host

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _edge(**kw):
    base = dict(name="edge", B=1, H=1, T=9, d=32, S=16, dk=32, k=4, W=8, in_bf16=False, state_bf16=False,
                alpha_shift=2.0, m0_std=0.5, subkey_std=0.25)
    base.update(kw)
    return gi.Config(**base)


CASES = {
    "f32": _edge(T=24, B=2, H=2, d=32, S=32, k=6, W=16),
    "1.4B_shape_T12": gi.config(2, T=12, B=2),
    "bf16_state_8B_shape_T8": gi.config(4, T=8, B=2),
    "bf16_state_small": _edge(T=20, B=2, H=3, d=64, S=24, k=5, W=20, in_bf16=True, state_bf16=True),
    "k_eq_W_64": _edge(T=10, S=64, k=64, W=64, d=64),
}


def run_steps_and_forward(cfg, x):
    import torch
    from sparse_memory_linear_pk_amd import SDM
    dev = {k: to_dev(v) for k, v in x.items()}
    with SDM.from_config(cfg) as layer:
        mem_f = dev["mem0"].clone()
        out_f = torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), dtype=torch.float32, device="cuda")
        layer.forward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem_f, out_f)
        mem_s = dev["mem0"].clone()
        out_s = torch.empty_like(out_f)
        o = torch.empty((cfg.B, cfg.H, cfg.d), dtype=torch.float32, device="cuda")
        for t in range(cfg.T):
            tok = {k: dev[k][:, t].contiguous() for k in ("wq", "rq", "v", "alpha", "beta")}
            layer.step(tok["wq"], tok["rq"], tok["v"], tok["alpha"], tok["beta"], dev["subkeys"], mem_s, o)
            out_s[:, t] = o
        torch.cuda.synchronize()
    return to_host(out_f), to_host(mem_f), to_host(out_s), to_host(mem_s)


@pytest.mark.parametrize("name", list(CASES))
def test_steps_equal_forward_bitwise(name):
    cfg = CASES[name]
    x = gi.make_inputs(cfg)
    say(f"[step {name}] {cfg}")
    out_f, mem_f, out_s, mem_s = run_steps_and_forward(cfg, x)
    assert np.array_equal(out_s.view(np.uint32), out_f.view(np.uint32))
    assert np.array_equal(mem_s, mem_f)


def test_steps_with_repeated_slots_equal_forward_bitwise():
    """Every token writes and reads the same few slots: each step rewrites what
    the previous step wrote and reads what it writes itself."""
    cfg = _edge(T=30, B=2, H=2, d=64, S=16, k=4, W=16)
    x = gi.make_inputs(cfg)
    x["wq"][:] = x["wq"][:, :2][:, np.arange(cfg.T) % 2]
    x["rq"][:, ::2] = x["wq"][:, ::2]
    out_f, mem_f, out_s, mem_s = run_steps_and_forward(cfg, x)
    assert np.array_equal(out_s.view(np.uint32), out_f.view(np.uint32))
    assert np.array_equal(mem_s, mem_f)


@pytest.mark.parametrize("name", ["f32", "bf16_state_small", "1.4B_shape_T12"])
def test_steps_match_the_oracle(name):
    """Staged, as for the forward: the slots the GPU selects against the
    oracle's (a difference is excused only at a near-tie), then the steps'
    outputs and memory against the oracle's scan driven by those slots."""
    import torch
    from sparse_memory_linear_pk_amd import SDM
    cfg = CASES[name]
    orc = oracle.get()
    x = gi.make_inputs(cfg)
    _, _, out_s, mem_s = run_steps_and_forward(cfg, x)
    R = cfg.B * cfg.T * cfg.H
    addr = {}
    with SDM.from_config(cfg) as layer:
        for s_, q in (("w", x["wq"]), ("r", x["rq"])):
            idx = torch.empty((R, cfg.W), dtype=torch.int32, device="cuda")
            wt = torch.empty((R, cfg.W), dtype=torch.float32, device="cuda")
            layer.address(to_dev(q), to_dev(x["subkeys"]), idx, wt)
            torch.cuda.synchronize()
            addr[s_] = (to_host(idx), to_host(wt))
            ri, rw, rs = orc.address(cfg, q, x["subkeys"])
            differ, exc = compare_index_sets(orc, cfg, addr[s_][0], ri, rs, orc.scores(cfg, q, x["subkeys"]))
            say(f"[step oracle {name}] {s_}: rows differing {differ} (excused {exc})")
    mem = x["mem0"].copy()
    out = orc.scan(cfg, addr["w"][0], addr["w"][1], addr["r"][0], addr["r"][1], x["v"], x["alpha"], x["beta"], mem)
    check_scan(cfg, 4, f"step oracle {name}", {"out": (plain_err(out_s, out), rel_max_err(out_s, out)),
                                                "mem": (plain_err(mem_s, mem), rel_max_err(mem_s, mem))}, say)


def test_step_rejects_an_unsupported_width():
    import torch
    from sparse_memory_linear_pk_amd import SDM, SDMError
    cfg = _edge(d=24)  # 96-byte float32 rows: no 128-byte segments
    with SDM.from_config(cfg) as layer:
        z = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
        with pytest.raises(SDMError):
            layer.step(z(1, 1, 32), z(1, 1, 32), z(1, 1, 24), z(1, 1), z(1, 1), z(1, 2, 16, 16),
                       z(1, 1, 256, 24), z(1, 1, 24))


def test_steps_on_a_one_token_handle_equal_forward_bitwise():
    """A handle made with T = 1 (the natural one for decode), float32 queries
    (the two-launch path, whose addressing passes 2*B*H*W slot ids and weights
    through the workspace) and B*H*W a multiple of 64: the step's ids and weights
    must not share memory, however few rows the forward's buffers hold."""
    import torch
    from sparse_memory_linear_pk_amd import SDM
    cfg = _edge(T=6, B=2, H=2, d=64, S=64, k=8, W=64)
    x = gi.make_inputs(cfg)
    dev = {k: to_dev(v) for k, v in x.items()}
    with SDM.from_config(cfg) as layer:
        mem_f = dev["mem0"].clone()
        out_f = torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), dtype=torch.float32, device="cuda")
        layer.forward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem_f, out_f)
        torch.cuda.synchronize()
    with SDM.from_config(cfg, T=1) as layer:
        mem_s = dev["mem0"].clone()
        o = torch.empty((cfg.B, cfg.H, cfg.d), dtype=torch.float32, device="cuda")
        for t in range(cfg.T):
            tok = {k: dev[k][:, t].contiguous() for k in ("wq", "rq", "v", "alpha", "beta")}
            layer.step(tok["wq"], tok["rq"], tok["v"], tok["alpha"], tok["beta"], dev["subkeys"], mem_s, o)
            torch.cuda.synchronize()
            assert torch.equal(o, out_f[:, t]), f"token {t}: step output differs from the forward"
    assert torch.equal(mem_s, mem_f)
