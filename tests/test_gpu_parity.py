"""The HIP path (through the C ABI) against the oracle, stage by stage.

Small and reduced-length cases compare every row and every element; the full
workload sizes compare sampled rows (addressing) and sampled slot elements
(the scan is independent per element, so the oracle runs all T tokens over
every slot for just those elements).
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import sdm_inputs as gi
from parity import (as_f32, check_scores, check_selection_exact, compare_index_sets, rel_max_err, rms_max_err,
                    scan_tol, score_error_bound, to_dev, to_host)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(scope="module")
def orc():
    return oracle.get()


@pytest.fixture(scope="module")
def T():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return torch


def run_gpu(T, cfg, x, stages=True):
    """All stage outputs of the HIP path on inputs x (numpy)."""
    from sparse_memory_linear_pk_amd import SDM
    R = cfg.B * cfg.T * cfg.H
    dev = {k: to_dev(v) for k, v in x.items()}
    res = {}
    with SDM.from_config(cfg) as layer:
        if stages:
            for name, q in (("w", dev["wq"]), ("r", dev["rq"])):
                sc = T.empty((R, 2, cfg.S), dtype=T.float32, device="cuda")
                idx = T.empty((R, cfg.W), dtype=T.int32, device="cuda")
                wt = T.empty((R, cfg.W), dtype=T.float32, device="cuda")
                layer.score(q, dev["subkeys"], sc)
                layer.select(sc, idx, wt)
                idx2 = T.empty_like(idx)
                wt2 = T.empty_like(wt)
                layer.address(q, dev["subkeys"], idx2, wt2)
                res[f"scores_{name}"], res[f"idx_{name}"], res[f"wt_{name}"] = sc, idx, wt
                res[f"idx2_{name}"], res[f"wt2_{name}"] = idx2, wt2
        mem = dev["mem0"].clone()
        out = T.empty((cfg.B, cfg.T, cfg.H, cfg.d), dtype=T.float32, device="cuda")
        layer.forward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem, out)
        res["mem"], res["out"] = mem, out
        if stages:
            mem2 = dev["mem0"].clone()
            out2 = T.empty_like(out)
            layer.scan_with(res["idx_w"], res["wt_w"], res["idx_r"], res["wt_r"], dev["v"], dev["alpha"],
                            dev["beta"], mem2, out2)
            res["mem2"], res["out2"] = mem2, out2
        T.cuda.synchronize()
    return {k: to_host(v) for k, v in res.items()}


def full_parity(orc, cfg, x, g, label):
    """Stages 1-5 on every row and element."""
    R = cfg.B * cfg.T * cfg.H
    rows = np.arange(R)
    # the forward and the stage seams run the same kernels
    for s in "wr":
        assert np.array_equal(g[f"idx_{s}"], g[f"idx2_{s}"]) and np.array_equal(g[f"wt_{s}"], g[f"wt2_{s}"])
    assert np.array_equal(g["out"], g["out2"]) and np.array_equal(g["mem"], g["mem2"])
    excused_rows = 0
    ref_addr = {}
    for s, q in (("w", x["wq"]), ("r", x["rq"])):
        ref_scores = orc.scores(cfg, q, x["subkeys"])
        err = check_scores(cfg, g[f"scores_{s}"], ref_scores, score_error_bound(cfg, q, x["subkeys"], rows))
        ui, uw, _ = orc.address_from_scores(cfg, g[f"scores_{s}"])
        ulp = check_selection_exact(g[f"idx_{s}"], g[f"wt_{s}"], ui, uw)
        ri, rw, rs = orc.address(cfg, q, x["subkeys"])
        ref_addr[s] = (ri, rw)
        differ, exc = compare_index_sets(orc, cfg, g[f"idx_{s}"], ri, rs, ref_scores)
        excused_rows += exc
        say(f"[{label}] {s}: score err {err:.3g}, weight ulp {ulp}, rows differing {differ} (excused {exc})")
    mem = x["mem0"].copy()
    out = orc.scan(cfg, g["idx_w"], g["wt_w"], g["idx_r"], g["wt_r"], x["v"], x["alpha"], x["beta"], mem)
    eo, em = rel_max_err(g["out"], out), rel_max_err(g["mem"], mem)
    say(f"[{label}] scan: out {eo:.3g}, mem {em:.3g} (tol {scan_tol(cfg)}); plain max/RMS: "
        f"out {rms_max_err(g['out'], out):.3g}, mem {rms_max_err(g['mem'], mem):.3g}")
    assert eo <= scan_tol(cfg) and em <= scan_tol(cfg)
    if excused_rows == 0:
        mem = x["mem0"].copy()
        out = orc.scan(cfg, ref_addr["w"][0], ref_addr["w"][1], ref_addr["r"][0], ref_addr["r"][1], x["v"],
                       x["alpha"], x["beta"], mem)
        eo, em = rel_max_err(g["out"], out), rel_max_err(g["mem"], mem)
        say(f"[{label}] end-to-end: out {eo:.3g}, mem {em:.3g}")
        assert eo <= scan_tol(cfg) and em <= scan_tol(cfg)


REDUCED = {
    "tiny": (0, dict()),
    "small_T256": (1, dict(T=256)),
    "1.4B_T48_B2": (2, dict(T=48, B=2)),
    "long_T160": (3, dict(T=160)),
    "8B_T40_B2": (4, dict(T=40, B=2)),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_workloads_reduced(orc, T, name):
    i, ov = REDUCED[name]
    cfg = gi.config(i, **ov)
    say(f"[{name}] {cfg}")
    x = gi.make_inputs(cfg)
    g = run_gpu(T, cfg, x)
    full_parity(orc, cfg, x, g, name)


def _edge(**kw):
    base = dict(name="edge", B=1, H=1, T=9, d=32, S=16, dk=32, k=4, W=8, in_bf16=False, state_bf16=False,
                alpha_shift=2.0, m0_std=0.5, subkey_std=0.25)
    base.update(kw)
    return gi.Config(**base)


EDGES = {
    "T1": _edge(T=1),
    "T7_ragged_epoch": _edge(T=7),
    "T13_bf16": _edge(T=13, in_bf16=True, state_bf16=True, d=64),
    "W1_k1": _edge(k=1, W=1, T=20),
    "k_eq_W": _edge(k=8, W=8, T=20),
    "S40_ragged_tile": _edge(S=40, k=6, W=30, T=35, H=3),
    "rows_ragged_B3": _edge(B=3, T=11, H=2),
    "d8_bf16_lps1": _edge(d=8, in_bf16=True, state_bf16=True, T=17),
    "d24_f32_lps2": _edge(d=24, T=17),
    "dh48": _edge(dk=96, T=10),
    "dh256_bf16": _edge(dk=512, T=6, in_bf16=True),
    "W64_k64": _edge(S=64, k=64, W=64, T=10, d=16),
    "mixed_state_f32_in_bf16": _edge(in_bf16=True, state_bf16=False, T=12),
    "mixed_state_bf16_in_f32": _edge(in_bf16=False, state_bf16=True, d=32, T=12),
    # 32-byte segments, 4 per memory, 24 workgroups: renumbered into 8 runs of 3, so the runs cross from
    # one memory to the next (T13_bf16, 4 workgroups, keeps the plain numbering)
    "bf16_segments_runs_cross_memories": _edge(B=3, H=2, d=64, T=19, in_bf16=True, state_bf16=True),
}


@pytest.mark.parametrize("name", list(EDGES))
def test_edge_shapes(orc, T, name):
    cfg = EDGES[name]
    say(f"[edge {name}] {cfg}")
    x = gi.make_inputs(cfg)
    g = run_gpu(T, cfg, x)
    full_parity(orc, cfg, x, g, name)


def test_heavy_forwarding(orc, T):
    """Every token writes (and reads) the same slots: each slot value is carried
    through the LDS ring from token to token, and only the last write of each
    epoch reaches memory."""
    cfg = _edge(T=37, W=16, k=4, H=2, d=64)
    x = gi.make_inputs(cfg)
    x["wq"][:] = x["wq"][:, :1]
    x["rq"][:, ::3] = x["wq"][:, ::3]            # reads of the slots the same token wrote
    x["rq"][:, 1::3] = x["wq"][:, 0:1]
    g = run_gpu(T, cfg, x)
    full_parity(orc, cfg, x, g, "heavy_forwarding")


def test_random_reuse(orc, T):
    """Queries drawn from a handful of repeating patterns: overlaps at every distance."""
    cfg = _edge(T=97, W=8, k=3, H=1, d=32, S=12, B=2)
    x = gi.make_inputs(cfg)
    rng = np.random.default_rng(3)
    pats = rng.standard_normal((4, cfg.dk)).astype(np.float32)
    x["wq"][:] = pats[rng.integers(0, 4, (cfg.B, cfg.T, cfg.H))]
    x["rq"][:] = pats[rng.integers(0, 4, (cfg.B, cfg.T, cfg.H))]
    g = run_gpu(T, cfg, x)
    full_parity(orc, cfg, x, g, "random_reuse")


def test_identity_gates_leave_memory_bitwise(orc, T):
    cfg = gi.config(2, T=32, B=1)
    x = gi.make_inputs(cfg)
    x["alpha"][:] = 1.0
    x["beta"][:] = 0.0
    g = run_gpu(T, cfg, x, stages=False)
    assert np.array_equal(g["mem"], x["mem0"])


def test_chunked_calls_are_bitwise_equal(T):
    from sparse_memory_linear_pk_amd import SDM
    cfg = gi.config(1, T=64, B=2, H=2)
    x = gi.make_inputs(cfg)
    g = run_gpu(T, cfg, x, stages=False)
    mem = to_dev(x["mem0"])
    outs = []
    for sl in (slice(0, 23), slice(23, 64)):
        c = cfg.replace(T=sl.stop - sl.start)
        xs = {k: to_dev(np.ascontiguousarray(v[:, sl])) for k, v in x.items() if k in ("wq", "rq", "v", "alpha", "beta")}
        out = T.empty((c.B, c.T, c.H, c.d), dtype=T.float32, device="cuda")
        with SDM.from_config(c) as layer:
            layer.forward(xs["wq"], xs["rq"], xs["v"], xs["alpha"], xs["beta"], to_dev(x["subkeys"]), mem, out)
        outs.append(to_host(out))
    assert np.array_equal(np.concatenate(outs, axis=1), g["out"])
    assert np.array_equal(to_host(mem), g["mem"])


# Forwards longer than 2048 tokens scan in several launches (512, 2048, ...
# tokens) while the next chunk's addressing runs on a second stream.
CHUNKED = {
    "f32_state_f32_in": _edge(T=2600, B=2, H=2, d=32, S=32, k=6, W=16),
    "f32_state_bf16_in": _edge(T=2700, B=1, H=3, d=64, S=48, k=8, W=24, in_bf16=True),
    "bf16_state": _edge(T=2600, B=2, H=1, d=64, S=32, k=6, W=16, in_bf16=True, state_bf16=True),
}


@pytest.mark.parametrize("name", list(CHUNKED))
def test_chunked_forward_parity(orc, T, name):
    """Every row and element of a forward that the library splits into chunks,
    with queries that repeat across the chunk boundaries (slots written just
    before a boundary are read and rewritten just after it)."""
    cfg = CHUNKED[name]
    x = gi.make_inputs(cfg)
    rng = np.random.default_rng(11)
    pats = x["wq"][:, :6].copy()
    for t0 in (500, 512, 2555, 2560):
        if t0 + 24 <= cfg.T:
            x["wq"][:, t0:t0 + 24] = pats[:, rng.integers(0, 6, 24)]
            x["rq"][:, t0:t0 + 24] = pats[:, rng.integers(0, 6, 24)]
    say(f"[chunked {name}] {cfg}")
    g = run_gpu(T, cfg, x)
    full_parity(orc, cfg, x, g, f"chunked {name}")


def test_chunked_forward_is_bitwise_one_launch_per_call(T):
    """The library's chunking changes no bit: one forward of 2600 tokens equals
    two forwards of 1300 (each scanned in a single launch)."""
    from sparse_memory_linear_pk_amd import SDM
    cfg = CHUNKED["f32_state_bf16_in"].replace(T=2600)
    x = gi.make_inputs(cfg)
    g = run_gpu(T, cfg, x, stages=False)
    mem = to_dev(x["mem0"])
    outs = []
    for sl in (slice(0, 1300), slice(1300, 2600)):
        c = cfg.replace(T=sl.stop - sl.start)
        xs = {k: to_dev(np.ascontiguousarray(v[:, sl])) for k, v in x.items() if k in ("wq", "rq", "v", "alpha", "beta")}
        out = T.empty((c.B, c.T, c.H, c.d), dtype=T.float32, device="cuda")
        with SDM.from_config(c) as layer:
            layer.forward(xs["wq"], xs["rq"], xs["v"], xs["alpha"], xs["beta"], to_dev(x["subkeys"]), mem, out)
        outs.append(to_host(out))
    assert np.array_equal(np.concatenate(outs, axis=1), g["out"])
    assert np.array_equal(to_host(mem), g["mem"])


def test_permuted_elements_are_bitwise_permuted(T):
    cfg = gi.config(1, T=40, B=1, H=2)
    x = gi.make_inputs(cfg)
    g = run_gpu(T, cfg, x, stages=False)
    p = np.random.default_rng(9).permutation(cfg.d)
    xp = dict(x)
    xp["v"] = np.ascontiguousarray(x["v"][..., p])
    xp["mem0"] = np.ascontiguousarray(x["mem0"][..., p])
    gp = run_gpu(T, cfg, xp, stages=False)
    assert np.array_equal(gp["out"], g["out"][..., p]) and np.array_equal(gp["mem"], g["mem"][..., p])


# ---------------------------------------------------------------------------
# full workload sizes, sampled
# ---------------------------------------------------------------------------

def sampled_parity(orc, T, cfg, label, n_rows=512, n_elem=16, extra_rows=()):
    from sparse_memory_linear_pk_amd import SDM
    rng = np.random.default_rng(1234)
    say(f"[{label}] generating inputs {cfg}")
    x = gi.make_inputs(cfg)
    R = cfg.B * cfg.T * cfg.H
    rows = np.unique(np.concatenate([rng.choice(R, size=min(n_rows, R), replace=False), np.asarray(extra_rows, int)]))
    DC = 64
    chunks = rng.choice(cfg.d // DC, size=min(4, cfg.d // DC), replace=False)
    elems = np.unique(np.concatenate([c * DC + rng.choice(DC, size=n_elem // 4, replace=False) for c in chunks]))
    say(f"[{label}] upload + GPU run")
    dev = {k: to_dev(v) for k, v in x.items() if k != "mem0"}
    mem = to_dev(x["mem0"])
    out = T.empty((cfg.B, cfg.T, cfg.H, cfg.d), dtype=T.float32, device="cuda")
    rows_t = T.from_numpy(rows).cuda()
    g = {}
    with SDM.from_config(cfg) as layer:
        for s in "wr":
            sc = T.empty((R, 2, cfg.S), dtype=T.float32, device="cuda")
            idx = T.empty((R, cfg.W), dtype=T.int32, device="cuda")
            wt = T.empty((R, cfg.W), dtype=T.float32, device="cuda")
            layer.score(dev[s + "q"], dev["subkeys"], sc)
            layer.select(sc, idx, wt)
            g[f"scores_{s}"] = to_host(sc.index_select(0, rows_t))
            g[f"idx_{s}"], g[f"wt_{s}"] = to_host(idx), to_host(wt)
            del sc
        layer.forward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem, out)
        T.cuda.synchronize()
    el_t = T.from_numpy(elems).cuda()
    g_out = to_host(out.index_select(3, el_t))
    g_mem = to_host(mem.index_select(3, el_t))
    del mem, out, dev
    T.cuda.empty_cache()
    say(f"[{label}] oracle addressing on {rows.size} rows")
    for s in "wr":
        q = x[s + "q"]
        ref_scores = orc.scores(cfg, q, x["subkeys"], rows=rows)
        err = check_scores(cfg, g[f"scores_{s}"], ref_scores, score_error_bound(cfg, q, x["subkeys"], rows))
        ui, uw, _ = orc.address_from_scores(cfg, g[f"scores_{s}"])
        check_selection_exact(g[f"idx_{s}"][rows], g[f"wt_{s}"][rows], ui, uw)
        ri, rw, rs = orc.address(cfg, q, x["subkeys"], rows=rows)
        differ, exc = compare_index_sets(orc, cfg, g[f"idx_{s}"][rows], ri, rs, ref_scores, rows=rows)
        say(f"[{label}] {s}: score err {err:.3g}, rows differing {differ} (excused {exc}) of {rows.size}")
    say(f"[{label}] oracle scan over {elems.size} elements x all slots x {cfg.T} tokens")
    c = cfg.replace(d=elems.size)
    mem0 = np.ascontiguousarray(x["mem0"][..., elems])
    v = np.ascontiguousarray(x["v"][..., elems])
    ref_out = orc.scan(c, g["idx_w"], g["wt_w"], g["idx_r"], g["wt_r"], v, x["alpha"], x["beta"], mem0)
    eo, em = rel_max_err(g_out, ref_out), rel_max_err(g_mem, mem0)
    say(f"[{label}] scan: out {eo:.3g}, mem {em:.3g} (tol {scan_tol(cfg)}); plain max/RMS: "
        f"out {rms_max_err(g_out, ref_out):.3g}, mem {rms_max_err(g_mem, mem0):.3g}")
    assert eo <= scan_tol(cfg) and em <= scan_tol(cfg)
    return g


@pytest.mark.timeout(900)
def test_full_small(orc, T):
    sampled_parity(orc, T, gi.config(1), "small")


@pytest.mark.timeout(900)
def test_full_1p4b(orc, T):
    sampled_parity(orc, T, gi.config(2), "1.4B")


@pytest.mark.timeout(900)
def test_full_long_planted(orc, T):
    cfg = gi.config(3)
    g = sampled_parity(orc, T, cfg, "long", extra_rows=(61, cfg.T - 17))
    # the recurring query selects bit-identical slots and weights on the GPU
    assert np.array_equal(g["idx_r"][cfg.T - 17], g["idx_w"][61])
    assert np.array_equal(g["wt_r"][cfg.T - 17], g["wt_w"][61])


@pytest.mark.timeout(900)
def test_full_8b(orc, T):
    sampled_parity(orc, T, gi.config(4), "8B")
