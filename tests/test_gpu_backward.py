"""sdm_forward_train and sdm_backward through the C ABI.

The training forward leaves exactly (bit for bit) the memory and outputs of
sdm_forward, and its log holds the oracle's memory values before each write.
The backward restores the memory bit for bit and its gradients agree with the
gradient oracle's, staged as for the forward: the slots the GPU selects
against the oracle's (a difference is excused only at a near-tie), then the
gradient oracle driven by the GPU's slots and weights.  Every gradient tensor
is within TOL of the oracle's as max |got - ref| / RMS(ref) (each tensor's
own RMS): the GPU works in float32 throughout, and each gradient is
a sum of at most a few hundred float32 terms per stage (d-long dot products
over one 128-byte column then over the columns, W-long softmax sums, 2BT-long
sub-key sums), whose rounding stays below 2^-24 times the term count.
"""
import sys

import numpy as np
import pytest

import oracle
import sdm_inputs as gi
from parity import compare_index_sets, plain_err, rel_max_err, to_dev, to_host

pytestmark = pytest.mark.gpu

TOL = 1e-4


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _cfg(**kw):
    base = dict(name="bwd", B=2, H=2, T=40, d=64, S=16, dk=32, k=4, W=8, in_bf16=False, state_bf16=False,
                alpha_shift=2.0, m0_std=0.5, subkey_std=0.25)
    base.update(kw)
    return gi.Config(**base)


CASES = {
    "f32": _cfg(),
    "bf16_inputs": _cfg(B=2, H=1, T=72, d=128, S=32, dk=64, k=8, W=16, in_bf16=True),
    "1.4B_addressing_d256": gi.config(2, B=2, T=48, d=256),
    "ragged_tiles": _cfg(B=1, H=3, T=33, d=96, S=40, dk=96, k=7, W=24),
    "one_slot": _cfg(B=2, H=1, T=17, d=32, S=8, dk=32, k=1, W=1),
    "k_eq_W_64": _cfg(B=1, H=1, T=20, d=32, S=64, dk=32, k=64, W=64),
    # long enough to scan in chunks (640 tokens, then the rest): the log of every chunk
    "chunked_T2600": _cfg(B=2, H=1, T=2600, d=32, S=16, dk=32, k=4, W=8),
    # bf16 state (the 8B-shaped workload's): bf16 memory and log, float32 gradient
    "bf16_state": _cfg(B=2, H=2, T=48, d=64, S=16, dk=32, k=4, W=8, in_bf16=True, state_bf16=True),
    "bf16_state_8B_addressing_d128": gi.config(4, B=1, T=40, d=128),
}


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _run_gpu(cfg, x, g, reps=1):
    import torch
    from sparse_memory_linear_pk_amd import SDM
    dev = {k: to_dev(v) for k, v in x.items()}
    R = cfg.B * cfg.T * cfg.H
    f32 = dict(dtype=torch.float32, device="cuda")
    res = {}
    with SDM.from_config(cfg) as layer:
        mem_f = dev["mem0"].clone()
        out_f = torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), **f32)
        layer.forward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem_f, out_f)
        mem = dev["mem0"].clone()
        out = torch.empty_like(out_f)
        log = torch.empty((cfg.B, cfg.H, cfg.T, cfg.W, cfg.d),
                          dtype=torch.bfloat16 if cfg.state_bf16 else torch.float32, device="cuda")
        layer.forward_train(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem, out, log)
        torch.cuda.synchronize()
        res.update(out_f=to_host(out_f), mem_f=to_host(mem_f), out=to_host(out), mem_T=to_host(mem), log=to_host(log))
        for s_, q in (("w", "wq"), ("r", "rq")):
            idx = torch.empty((R, cfg.W), dtype=torch.int32, device="cuda")
            wt = torch.empty((R, cfg.W), **f32)
            layer.address(dev[q], dev["subkeys"], idx, wt)
            torch.cuda.synchronize()
            res["idx_" + s_], res["wt_" + s_] = to_host(idx), to_host(wt)
        gd = {k: to_dev(v) for k, v in g.items()}
        runs = []
        for _ in range(reps):
            m = mem.clone()
            dm = gd["dmem"].clone()
            outs = {"dwq": torch.empty((cfg.B, cfg.T, cfg.H, cfg.dk), **f32),
                    "drq": torch.empty((cfg.B, cfg.T, cfg.H, cfg.dk), **f32),
                    "dv": torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), **f32),
                    "dalpha": torch.empty((cfg.B, cfg.T, cfg.H), **f32),
                    "dbeta": torch.empty((cfg.B, cfg.T, cfg.H), **f32),
                    "dsub": torch.empty((cfg.H, 2, cfg.S, cfg.dk // 2), **f32)}
            layer.backward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], m, log,
                           gd["dout"], dm, outs["dwq"], outs["drq"], outs["dv"], outs["dalpha"], outs["dbeta"],
                           outs["dsub"])
            torch.cuda.synchronize()
            runs.append({**{k: to_host(v) for k, v in outs.items()}, "dmem0": to_host(dm), "mem0": to_host(m)})
        res["runs"] = runs
    return res


def _sigma_of(orc, cfg, q, subkeys, idx):
    """The oracle's float sums s1[a] + s2[b] for given slots n = a*S + b."""
    sc = orc.scores(cfg, q, subkeys)
    R = idx.shape[0]
    a, b = idx // cfg.S, idx % cfg.S
    rr = np.arange(R)[:, None]
    return (sc[rr, 0, a] + sc[rr, 1, b]).astype(np.float32)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_the_gradient_oracle(name):
    cfg = CASES[name]
    say(f"[bwd {name}] {cfg}")
    orc, go = oracle.get(), oracle.get_grad()
    x = gi.make_inputs(cfg)
    g = gi.make_upstream_grads(cfg)
    res = _run_gpu(cfg, x, g)
    run = res["runs"][0]

    # the training forward is the forward
    assert np.array_equal(_bits(res["out"]), _bits(res["out_f"]))
    assert np.array_equal(_bits(res["mem_T"]), _bits(res["mem_f"]))
    # the reverse walk restores the initial memory exactly
    assert np.array_equal(_bits(run["mem0"]), _bits(x["mem0"]))

    for s_, q in (("w", x["wq"]), ("r", x["rq"])):
        ri, rw, rs = orc.address(cfg, q, x["subkeys"])
        differ, exc = compare_index_sets(orc, cfg, res["idx_" + s_], ri, rs, orc.scores(cfg, q, x["subkeys"]))
        say(f"[bwd {name}] {s_}: rows differing {differ} (excused {exc})")

    ref = go.scan_grad(cfg, res["idx_w"], res["wt_w"], res["idx_r"], res["wt_r"], x["v"], x["alpha"], x["beta"],
                       x["mem0"], g["dout"], g["dmem"].astype(np.float64))
    dq_w, dsub_w = go.address_grad(cfg, x["wq"], x["subkeys"], res["idx_w"],
                                   _sigma_of(orc, cfg, x["wq"], x["subkeys"], res["idx_w"]), ref["dwt_w"])
    dq_r, dsub_r = go.address_grad(cfg, x["rq"], x["subkeys"], res["idx_r"],
                                   _sigma_of(orc, cfg, x["rq"], x["subkeys"], res["idx_r"]), ref["dwt_r"])
    pairs = {
        "dv": (run["dv"], ref["dv"]), "dalpha": (run["dalpha"], ref["dalpha"]),
        "dbeta": (run["dbeta"], ref["dbeta"]), "dmem0": (run["dmem0"], ref["dmem0"]),
        "dwq": (run["dwq"].reshape(-1, cfg.dk), dq_w), "drq": (run["drq"].reshape(-1, cfg.dk), dq_r),
        "dsubkeys": (run["dsub"], dsub_w + dsub_r),
    }
    errs = {k: rel_max_err(a.astype(np.float32), b.astype(np.float64)) for k, (a, b) in pairs.items()
            if np.any(b != 0)}
    plain = {k: plain_err(a.astype(np.float32), b.astype(np.float64)) for k, (a, b) in pairs.items()
             if np.any(b != 0)}
    say(f"[bwd {name}] per element: " + ", ".join(f"{k} {v:.3g}" for k, v in errs.items())
        + "; max/RMS: " + ", ".join(f"{k} {v:.3g}" for k, v in plain.items()))
    for k, (a, b) in pairs.items():
        if not np.any(b != 0):  # one selected slot: no gradient reaches the queries or sub-keys
            assert not np.any(a != 0), k
    bad = {k: v for k, v in plain.items() if v > TOL}
    assert not bad, f"gradients outside {TOL} (max |got - ref| / RMS(ref)): {bad}"

    # the log: the oracle's memory value of every write slot before its write, replayed on the GPU's slots
    one = cfg.replace(B=1, H=1, T=1)
    ref_log = np.empty_like(res["log"])
    for b in range(cfg.B):
        for h in range(cfg.H):
            mem = np.ascontiguousarray(x["mem0"][b, h][None, None]).copy()
            for t in range(cfg.T):
                r = (b * cfg.T + t) * cfg.H + h
                ref_log[b, h, t] = mem[0, 0, res["idx_w"][r]]
                orc.scan(one, res["idx_w"][r:r + 1], res["wt_w"][r:r + 1], res["idx_r"][r:r + 1],
                         res["wt_r"][r:r + 1], x["v"][b, t, h][None, None, None], x["alpha"][b, t, h].reshape(1, 1, 1),
                         x["beta"][b, t, h].reshape(1, 1, 1), mem, threads=1)
    el = plain_err(res["log"], ref_log)
    say(f"[bwd {name}] log max/RMS {el:.3g}")
    assert el <= TOL


def test_backward_is_deterministic_and_repeatable():
    """Two backward calls from the same state give the same bits (every sum has a fixed order)."""
    cfg = CASES["bf16_inputs"]
    x = gi.make_inputs(cfg)
    g = gi.make_upstream_grads(cfg)
    runs = _run_gpu(cfg, x, g, reps=2)["runs"]
    for k in runs[0]:
        assert np.array_equal(_bits(runs[0][k]), _bits(runs[1][k])), k


def test_backward_with_heavy_slot_reuse():
    """Every token writes the same slots and reads them back: the read gradient of a token
    flows into its own write, and each token's state gradient into the next one back."""
    cfg = _cfg(B=1, H=2, T=30, d=64, S=16, k=4, W=16)
    orc, go = oracle.get(), oracle.get_grad()
    x = gi.make_inputs(cfg)
    x["wq"][:] = x["wq"][:, :1]
    x["rq"][:] = x["wq"]
    g = gi.make_upstream_grads(cfg)
    res = _run_gpu(cfg, x, g)
    run = res["runs"][0]
    ref = go.scan_grad(cfg, res["idx_w"], res["wt_w"], res["idx_r"], res["wt_r"], x["v"], x["alpha"], x["beta"],
                       x["mem0"], g["dout"], g["dmem"].astype(np.float64))
    for k in ("dv", "dalpha", "dbeta", "dmem0"):
        e = plain_err(run[k], ref[k])
        say(f"[bwd reuse] {k} max/RMS {e:.3g}")
        assert e <= TOL, k
    assert np.array_equal(_bits(run["mem0"]), _bits(x["mem0"]))


def test_backward_rejects_a_bf16_state_of_partial_columns():
    """A bf16 state needs whole 128-byte columns of 64 elements: d = 96 is refused on the host."""
    import torch
    from sparse_memory_linear_pk_amd import SDM, SDMError
    cfg = _cfg(state_bf16=True, d=96)
    with SDM.from_config(cfg) as layer:
        t = lambda *s: torch.zeros(s, dtype=torch.float32, device="cuda")
        b = lambda *s: torch.zeros(s, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(SDMError, match="multiple of 64"):
            layer.forward_train(t(cfg.B, cfg.T, cfg.H, cfg.dk), t(cfg.B, cfg.T, cfg.H, cfg.dk),
                                t(cfg.B, cfg.T, cfg.H, cfg.d), t(cfg.B, cfg.T, cfg.H), t(cfg.B, cfg.T, cfg.H),
                                t(cfg.H, 2, cfg.S, cfg.dk // 2), b(cfg.B, cfg.H, cfg.N, cfg.d),
                                t(cfg.B, cfg.T, cfg.H, cfg.d), b(cfg.B, cfg.H, cfg.T, cfg.W, cfg.d))


@pytest.mark.timeout(600)
def test_backward_with_a_gradient_past_4_gib():
    """The 8B shape (N = 640^2, d = 3840, bf16 state, rows padded to 3904): the float32 memory gradient
    is 6.4 GB per memory, past what a 32-bit buffer offset reaches, so the reverse scan addresses it with
    64-bit pointers.  The memory gradient, the restored memory and dv are per-element given the slots and
    weights, so the gradient oracle checks them on column slices (d = 64: the first and the last 64
    columns, every one of the 409,600 slots), driven by the GPU's slots."""
    import torch
    from sparse_memory_linear_pk_amd import SDM
    cfg = gi.config(4, B=1, T=16)
    ms = SDM.stride_hint(cfg.d, True)
    assert cfg.S ** 2 * ms * 4 >= 2 ** 32
    go = oracle.get_grad()
    x = gi.make_inputs(cfg)
    g = gi.make_upstream_grads(cfg)
    say(f"[bwd wide] {cfg} mem_stride {ms}")
    dev = {k: to_dev(v) for k, v in x.items()}
    f32 = dict(dtype=torch.float32, device="cuda")
    R = cfg.B * cfg.T * cfg.H
    with SDM.from_config(cfg, mem_stride=ms) as layer:
        mem = layer.empty_state(cfg.B, cfg.H)
        mem.copy_(dev["mem0"])
        dmem = layer.empty_state(cfg.B, cfg.H, dtype=torch.float32)
        dmem.copy_(to_dev(g["dmem"]))
        out = torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), **f32)
        log = torch.empty((cfg.B, cfg.H, cfg.T, cfg.W, cfg.d), dtype=torch.bfloat16, device="cuda")
        layer.forward_train(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem, out, log)
        idx = {}
        for s_, q in (("w", "wq"), ("r", "rq")):
            i_ = torch.empty((R, cfg.W), dtype=torch.int32, device="cuda")
            w_ = torch.empty((R, cfg.W), **f32)
            layer.address(dev[q], dev["subkeys"], i_, w_)
            idx[s_] = (to_host(i_), to_host(w_))
        outs = {"dwq": torch.empty((cfg.B, cfg.T, cfg.H, cfg.dk), **f32),
                "drq": torch.empty((cfg.B, cfg.T, cfg.H, cfg.dk), **f32),
                "dv": torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), **f32),
                "dalpha": torch.empty((cfg.B, cfg.T, cfg.H), **f32),
                "dbeta": torch.empty((cfg.B, cfg.T, cfg.H), **f32),
                "dsub": torch.empty((cfg.H, 2, cfg.S, cfg.dk // 2), **f32)}
        layer.backward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem, log,
                       to_dev(g["dout"]), dmem, outs["dwq"], outs["drq"], outs["dv"], outs["dalpha"], outs["dbeta"],
                       outs["dsub"])
        torch.cuda.synchronize()
        # the reverse walk restores the initial memory exactly
        assert torch.equal(mem.view(torch.int16), dev["mem0"].view(torch.int16))
        hi = int((idx["w"][0] >= 2 ** 32 // (ms * 4)).sum())
        say(f"[bwd wide] write slots past the first 4 GiB of the gradient: {hi} of {idx['w'][0].size}")
        assert hi > 0
        for c0 in (0, cfg.d - 64):
            sl = slice(c0, c0 + 64)
            cs = cfg.replace(d=64)
            ref = go.scan_grad(cs, idx["w"][0], idx["w"][1], idx["r"][0], idx["r"][1],
                               np.ascontiguousarray(x["v"][..., sl]), x["alpha"], x["beta"],
                               np.ascontiguousarray(x["mem0"][..., sl]), np.ascontiguousarray(g["dout"][..., sl]),
                               np.ascontiguousarray(g["dmem"][..., sl]).astype(np.float64))
            e_g = plain_err(to_host(dmem[..., sl]), ref["dmem0"])
            e_v = plain_err(to_host(outs["dv"][..., sl]), ref["dv"])
            say(f"[bwd wide] columns {c0}..{c0 + 63}: max/RMS dmem0 {e_g:.3g}, dv {e_v:.3g}")
            assert e_g <= TOL and e_v <= TOL
