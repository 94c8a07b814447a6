"""The HIP path (through the C ABI) against the oracle, stage by stage.

Every case compares every row (addressing) and every element (outputs and
final memory): the reduced-length and edge cases in one piece, the full
workload sizes sequence by sequence (memories are independent), with the
figure of the whole tensor accumulated over the sequences.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
import sdm_inputs as gi
from parity import (PlainAccum, check_scan, check_scores, check_selection_exact, compare_index_sets, plain_err,
                    rel_max_err, score_error_bound, to_dev, to_host)

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
            # both sets in the forward's own launches equal the one-set seam bit for bit
            pair = [T.empty_like(res["idx2_w"]), T.empty_like(res["wt2_w"]), T.empty_like(res["idx2_r"]),
                    T.empty_like(res["wt2_r"])]
            layer.address_pair(dev["wq"], dev["rq"], dev["subkeys"], *pair)
            for a, b in zip(pair, ("idx2_w", "wt2_w", "idx2_r", "wt2_r")):
                assert T.equal(a.view(T.int32), res[b].view(T.int32)), f"sdm_address_pair differs from sdm_address: {b}"
        mem = dev["mem0"].clone()
        out = T.empty((cfg.B, cfg.T, cfg.H, cfg.d), dtype=T.float32, device="cuda")
        layer.forward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem, out)
        res["mem"], res["out"] = mem, out
        if stages:
            mem2 = dev["mem0"].clone()
            out2 = T.empty_like(out)
            layer.scan_with(res["idx2_w"], res["wt2_w"], res["idx2_r"], res["wt2_r"], dev["v"], dev["alpha"],
                            dev["beta"], mem2, out2)
            res["mem2"], res["out2"] = mem2, out2
        T.cuda.synchronize()
    return {k: to_host(v) for k, v in res.items()}


def check_exact_addressing(got_idx, got_wt, ref_idx, ref_wt, label, say_):
    """The forward's addressing against the oracle's, from the same queries: the same slots in the
    same order, weights within one float32 unit (the softmax's exp is a library routine on each side)."""
    bad = np.nonzero((got_idx != ref_idx).any(axis=1))[0]
    assert bad.size == 0, f"[{label}] {bad.size} rows address other slots than the oracle, first {bad[:5]}"
    u = np.abs(got_wt.view(np.int32).astype(np.int64) - ref_wt.view(np.int32).astype(np.int64))
    assert u.max() <= 1, f"[{label}] weights differ by {u.max()} units"
    return int(u.max())


def full_parity(orc, cfg, x, g, label):
    """Stages 1-5 on every row and element."""
    R = cfg.B * cfg.T * cfg.H
    rows = np.arange(R)
    # the scan seam on the forward's addressing is the forward
    assert np.array_equal(g["out"], g["out2"]) and np.array_equal(g["mem"], g["mem2"])
    for s, q in (("w", x["wq"]), ("r", x["rq"])):
        ref_scores = orc.scores(cfg, q, x["subkeys"])
        err = check_scores(cfg, g[f"scores_{s}"], ref_scores, score_error_bound(cfg, q, x["subkeys"], rows))
        ui, uw, _ = orc.address_from_scores(cfg, g[f"scores_{s}"])
        ulp = check_selection_exact(g[f"idx_{s}"], g[f"wt_{s}"], ui, uw)
        ri, rw, rs = orc.address(cfg, q, x["subkeys"])
        # the float32 scores alone choose as the oracle except across near-ties
        differ, exc = compare_index_sets(orc, cfg, g[f"idx_{s}"], ri, rs, ref_scores)
        # the forward's addressing makes the scores that matter exact: the oracle's slots and weights
        ulp3 = check_exact_addressing(g[f"idx2_{s}"], g[f"wt2_{s}"], ri, rw, label, say)
        say(f"[{label}] {s}: score err {err:.3g}, selection from the same scores exact (weight ulp {ulp}); "
            f"float32 scores alone would choose differently on {differ} rows (near-ties: {exc}); "
            f"forward addressing equals the oracle's (weight ulp {ulp3})")
    mem = x["mem0"].copy()
    out = orc.scan(cfg, g["idx2_w"], g["wt2_w"], g["idx2_r"], g["wt2_r"], x["v"], x["alpha"], x["beta"], mem)
    check_scan(cfg, 4, label, {"out": (plain_err(g["out"], out), rel_max_err(g["out"], out)),
                               "mem": (plain_err(g["mem"], mem), rel_max_err(g["mem"], mem))}, say)
    mem = x["mem0"].copy()
    out = orc.forward(cfg, x["wq"], x["rq"], x["v"], x["alpha"], x["beta"], x["subkeys"], mem)[0]
    check_scan(cfg, 5, label, {"out": (plain_err(g["out"], out), rel_max_err(g["out"], out)),
                               "mem": (plain_err(g["mem"], mem), rel_max_err(g["mem"], mem))}, say)


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


# Forwards longer than 2048 tokens scan in several launches (640 tokens first,
# then each chunk 3/2 of the one before up to 3072, a remainder below 1536
# joining the chunk before it: 640 and 1960 at 2600 tokens, 640, 960 and 1700
# at 3300; where the two would exceed 3072 tokens they split in about half
# instead: 640, 960, 1408, 2112, 1984 and 2088 at 9192) while the next chunk's
# addressing runs on a second stream.
CHUNKED = {
    "f32_state_f32_in": _edge(T=2600, B=2, H=2, d=32, S=32, k=6, W=16),
    "f32_state_bf16_in": _edge(T=3300, B=1, H=3, d=64, S=48, k=8, W=24, in_bf16=True),
    "bf16_state": _edge(T=2600, B=2, H=1, d=64, S=32, k=6, W=16, in_bf16=True, state_bf16=True),
    "split_tail": _edge(T=9192, B=1, H=1, d=32, S=16, k=4, W=8),
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
    for t0 in (620, 640, 1580, 1600, 7090, 7104):
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
# full workload sizes: every row and every element
# ---------------------------------------------------------------------------

def full_gpu_run(T, cfg, label, padded=False) -> dict:
    """The GPU half of a full-size parity case.  The GPU runs the whole call (B
    sequences, the library's chunked forward) as bench.py does, and the scoring
    and selection seams and the forward's own addressing of both query sets.
    padded: the same forward also on slot rows padded to sdm_mem_stride_hint
    (bench.py's layout), which must equal the dense one bit for bit."""
    from sparse_memory_linear_pk_amd import SDM
    R = cfg.B * cfg.T * cfg.H
    say(f"[{label}] inputs {cfg}")
    x = gi.make_inputs(cfg, with_mem0=False)
    dev = {k: to_dev(v) for k, v in x.items()}
    sdt = T.bfloat16 if cfg.state_bf16 else T.float32
    mem = T.empty((cfg.B, cfg.H, cfg.N, cfg.d), dtype=sdt, device="cuda")
    for b in range(cfg.B):
        mem[b].copy_(to_dev(gi.make_mem0_seqs(cfg, b, b + 1))[0])
    mem0 = mem.clone()  # the initial memory, read back sequence by sequence for the oracle
    out = T.empty((cfg.B, cfg.T, cfg.H, cfg.d), dtype=T.float32, device="cuda")
    say(f"[{label}] GPU: scores and selection of both query sets, then the forward")
    g = {}
    with SDM.from_config(cfg) as layer:
        for s_ in "wr":
            sc = T.empty((R, 2, cfg.S), dtype=T.float32, device="cuda")
            idx = T.empty((R, cfg.W), dtype=T.int32, device="cuda")
            wt = T.empty((R, cfg.W), dtype=T.float32, device="cuda")
            layer.score(dev[s_ + "q"], dev["subkeys"], sc)
            layer.select(sc, idx, wt)
            g[f"scores_{s_}"], g[f"idx_{s_}"], g[f"wt_{s_}"] = to_host(sc), to_host(idx), to_host(wt)
            layer.address(dev[s_ + "q"], dev["subkeys"], idx, wt)
            g[f"idx2_{s_}"], g[f"wt2_{s_}"] = to_host(idx), to_host(wt)
            del sc
        pair = [T.empty((R, cfg.W), dtype=dt, device="cuda") for dt in (T.int32, T.float32, T.int32, T.float32)]
        layer.address_pair(dev["wq"], dev["rq"], dev["subkeys"], *pair)
        for a, b in zip(pair, ("idx2_w", "wt2_w", "idx2_r", "wt2_r")):
            assert np.array_equal(to_host(a).view(np.int32), g[b].view(np.int32)), f"sdm_address_pair: {b}"
        del pair
        layer.forward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem, out)
        T.cuda.synchronize()
    if padded:
        ms = SDM.stride_hint(cfg.d, cfg.state_bf16)
        assert ms > cfg.d, "the stride hint pads these rows"
        with SDM.from_config(cfg, mem_stride=ms) as lp:
            mp = lp.empty_state(cfg.B, cfg.H)
            mp.copy_(mem0)
            op = T.empty_like(out)
            say(f"[{label}] GPU: the same forward on slot rows {ms} elements apart")
            lp.forward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mp, op)
            T.cuda.synchronize()
            ity = T.int16 if cfg.state_bf16 else T.int32
            same_out = bool(T.equal(op.view(T.int32), out.view(T.int32)))
            same_mem = all(bool(T.equal(mp[b].contiguous().view(ity), mem[b].view(ity))) for b in range(cfg.B))
        del mp, op
        say(f"[{label}] padded rows against dense rows: out bitwise {same_out}, memory bitwise {same_mem}")
        assert same_out and same_mem
    g_out = to_host(out)
    del out, dev
    T.cuda.empty_cache()
    acc = {k: PlainAccum() for k in ("out4", "mem4", "out5", "mem5")}
    return {"x": x, "g": g, "g_out": g_out, "mem": mem, "mem0": mem0, "acc": acc, "seqs_done": set()}


def full_addressing(orc, cfg, st, label, sets="wr"):
    """Stages 1-3 on every row of the query sets named in `sets`."""
    x, g = st["x"], st["g"]
    R = cfg.B * cfg.T * cfg.H
    for s_ in sets:
        q = x[s_ + "q"]
        say(f"[{label}] {s_}: oracle scores of {R} rows")
        ref_scores = orc.scores(cfg, q, x["subkeys"])
        err = 0.0
        for r0 in range(0, R, 16384):
            rows = np.arange(r0, min(R, r0 + 16384))
            err = max(err, check_scores(cfg, g[f"scores_{s_}"][rows], ref_scores[rows],
                                        score_error_bound(cfg, q, x["subkeys"], rows)))
        ui, uw, _ = orc.address_from_scores(cfg, g[f"scores_{s_}"])
        ulp = check_selection_exact(g[f"idx_{s_}"], g[f"wt_{s_}"], ui, uw)
        del ui, uw
        ri, rw, rs = orc.address_from_scores(cfg, ref_scores)
        differ, exc = compare_index_sets(orc, cfg, g[f"idx_{s_}"], ri, rs, ref_scores)
        ulp3 = check_exact_addressing(g[f"idx2_{s_}"], g[f"wt2_{s_}"], ri, rw, label, say)
        say(f"[{label}] {s_}: score err {err:.3g}, selection from the same scores exact (weight ulp {ulp}); "
            f"float32 scores alone would choose differently on {differ} of {R} rows (near-ties: {exc}); "
            f"forward addressing equals the oracle's on every row (weight ulp {ulp3})")
        del ref_scores, g[f"scores_{s_}"], ri, rw, rs


def full_scan(orc, cfg, st, label, seqs):
    """Stages 4 and 5 on the sequences `seqs` (memories are independent); the
    oracle addresses from the queries for stage 5.  The whole tensors' figures
    accumulate in st["acc"]; each sequence's own figures are asserted here."""
    x, g, g_out, mem, mem0, acc = st["x"], st["g"], st["g_out"], st["mem"], st["mem0"], st["acc"]
    c1 = cfg.replace(B=1)
    per = cfg.T * cfg.H
    for b in seqs:
        rows = slice(b * per, (b + 1) * per)
        xb = {k: np.ascontiguousarray(x[k][b:b + 1]) for k in ("wq", "rq", "v", "alpha", "beta")}
        m0 = to_host(mem0[b:b + 1])
        gm = to_host(mem[b:b + 1])
        one = {k: PlainAccum() for k in acc}
        m = m0.copy()
        o4 = orc.scan(c1, g["idx2_w"][rows], g["wt2_w"][rows], g["idx2_r"][rows], g["wt2_r"][rows], xb["v"],
                      xb["alpha"], xb["beta"], m)
        for a in (acc, one):
            a["out4"].add(g_out[b:b + 1], o4)
            a["mem4"].add(gm, m)
        m = m0
        o5 = orc.forward(c1, xb["wq"], xb["rq"], xb["v"], xb["alpha"], xb["beta"], x["subkeys"], m)[0]
        for a in (acc, one):
            a["out5"].add(g_out[b:b + 1], o5)
            a["mem5"].add(gm, m)
        say(f"[{label}] sequence {b}: stage 4 out max/RMS {one['out4'].value():.3g}, memory "
            f"{one['mem4'].value():.3g}; stage 5 out {one['out5'].value():.3g}, memory {one['mem5'].value():.3g}")
        for stage in (4, 5):
            check_scan(cfg, stage, f"{label} sequence {b}",
                       {"out": (one[f"out{stage}"].value(), one[f"out{stage}"].rel),
                        "mem": (one[f"mem{stage}"].value(), one[f"mem{stage}"].rel)}, say)
        st["seqs_done"].add(b)
        del m0, m, gm


def full_scan_check(cfg, st, label):
    """The whole tensors' figures of stages 4 and 5, once every sequence is in."""
    assert st["seqs_done"] == set(range(cfg.B)), "every sequence's scan compared"
    acc = st["acc"]
    for stage in (4, 5):
        check_scan(cfg, stage, label, {"out": (acc[f"out{stage}"].value(), acc[f"out{stage}"].rel),
                                       "mem": (acc[f"mem{stage}"].value(), acc[f"mem{stage}"].rel)}, say)


def full_size_parity(orc, T, cfg, label, padded=False):
    """Stages 1-5 at a full workload size: the GPU run, then the oracle checks
    every row's addressing and scans sequence by sequence, accumulating the
    whole tensors' figures."""
    st = full_gpu_run(T, cfg, label, padded)
    full_addressing(orc, cfg, st, label)
    full_scan(orc, cfg, st, label, range(cfg.B))
    full_scan_check(cfg, st, label)
    g = st["g"]
    del st
    T.cuda.empty_cache()
    return g


@pytest.mark.timeout(900)
def test_full_small(orc, T):
    full_size_parity(orc, T, gi.config(1), "small")


@pytest.mark.timeout(900)
def test_full_1p4b_dense_and_padded_rows(orc, T):
    full_size_parity(orc, T, gi.config(2), "1.4B", padded=True)


@pytest.mark.timeout(900)
def test_full_long_planted(orc, T):
    cfg = gi.config(3)
    g = full_size_parity(orc, T, cfg, "long")
    # the recurring query selects bit-identical slots and weights on the GPU
    assert np.array_equal(g["idx2_r"][cfg.T - 17], g["idx2_w"][61])
    assert np.array_equal(g["wt2_r"][cfg.T - 17], g["wt2_w"][61])


# The 8B-shaped workload in parts (its memories are 3.1 GB each): the GPU run
# once for the module, then each query set's addressing and each sequence's scan
# as a test of its own.
@pytest.fixture(scope="module")
def full8b(T):
    st = full_gpu_run(T, gi.config(4), "8B")
    yield st
    st.clear()
    T.cuda.empty_cache()


@pytest.mark.timeout(600)
def test_full_8b_gpu_run(full8b):
    assert np.isfinite(full8b["g_out"]).all()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("s_", ["w", "r"])
def test_full_8b_addressing(orc, full8b, s_):
    full_addressing(orc, gi.config(4), full8b, "8B", s_)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("b", range(gi.config(4).B))
def test_full_8b_scan(orc, full8b, b):
    full_scan(orc, gi.config(4), full8b, "8B", [b])


def test_full_8b_whole_tensors(full8b):
    full_scan_check(gi.config(4), full8b, "8B")
