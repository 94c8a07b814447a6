"""Pins that tie the projection oracle (oracle/sdm_oracle_proj.c) to something
other than itself: a hand-worked example, identity and one-hot weights that
must return the embedding's own entries, head and output-block placement,
sigmoid values known in closed form, and the nearest-even rounding of sums
that land exactly halfway between two bf16 values.  Each pin takes a
projection-oracle handle and raises AssertionError on disagreement; the same
pins run against planted mistakes (test_oracle_proj_mutants.py).

What is computed: SDM blog post, section "How does SDM work?" and its "Write &
Read" subsection (the embedding projected to the write keys and, separately,
to the read query); the value and the gates as in the gated delta rule the
layer extends.  Readings as stated in sdm_oracle_proj.h.
"""
from __future__ import annotations

import math

import numpy as np

from sdm_inputs import bf16_bits_from_f32, f32_from_bf16_bits


def _b(a):
    return bf16_bits_from_f32(np.asarray(a, np.float32))


def _f(bits):
    return f32_from_bf16_bits(np.asarray(bits)).reshape(np.asarray(bits).shape)


def pin_worked_example(p):
    """D = 2, one head, dk = d = 1: x = (1, 2);
    wq row (1, 0.5) -> 2;  rq row (0.25, -1) -> -1.75;  v row (3, 0) -> 3;
    alpha logit row (0, 0), bias 0 -> sigmoid(0) = 0.5;  beta row (1, 1), bias -3 -> sigmoid(0) = 0.5."""
    x = _b([[[1.0, 2.0]]])
    w = _b([[1.0, 0.5], [0.25, -1.0], [3.0, 0.0], [0.0, 0.0], [1.0, 1.0]])
    bias = np.array([[0.0, -3.0]], np.float32)
    wq, rq, v, al, be = p.project(1, 1, 1, 2, 1, 1, x, w, bias)
    assert _f(wq)[0, 0, 0, 0] == 2.0 and _f(rq)[0, 0, 0, 0] == -1.75 and _f(v)[0, 0, 0, 0] == 3.0
    assert al[0, 0, 0] == 0.5 and be[0, 0, 0] == 0.5


def pin_identity_and_one_hot(p):
    """Identity weights return the embedding; negated identity its negation; one-hot rows pick
    single entries, for two heads whose blocks select different entries."""
    rng = np.random.default_rng(3)
    B, T, H, D, dk, d = 2, 3, 2, 8, 8, 4
    x = _b(rng.standard_normal((B, T, D)))
    C = 2 * dk + d + 2
    w = np.zeros((H * C, D), np.float32)
    for h in range(H):
        w[h * C: h * C + dk] = np.eye(D) * (1 if h == 0 else 2)      # wq: x (head 0), 2x (head 1)
        w[h * C + dk: h * C + 2 * dk] = -np.eye(D)                     # rq: -x
        for j in range(d):                                              # v: entries 7-j (head 0), j (head 1)
            w[h * C + 2 * dk + j, (D - 1 - j) if h == 0 else j] = 1.0
    wq, rq, v, al, be = p.project(B, T, H, D, dk, d, x, _b(w), np.zeros((H, 2), np.float32))
    xf = _f(x)
    assert np.array_equal(_f(wq)[:, :, 0], xf) and np.array_equal(_f(wq)[:, :, 1], 2 * xf)
    assert np.array_equal(_f(rq)[:, :, 0], -xf) and np.array_equal(_f(rq)[:, :, 1], -xf)
    assert np.array_equal(_f(v)[:, :, 0], xf[:, :, ::-1][:, :, :d]) and np.array_equal(_f(v)[:, :, 1], xf[:, :, :d])
    assert np.all(al == 0.5) and np.all(be == 0.5)


def pin_gate_closed_forms(p):
    """Zero beta weights: sigmoid(ln 3) = 3/4, sigmoid(-ln 3) = 1/4; an alpha logit of x_0 * 1 with
    x_0 = 2 and bias -2 gives 1/2, with bias ln 3 - 2 gives 3/4."""
    B, T, H, D, dk, d = 1, 2, 1, 4, 1, 1
    x = _b([[[2.0, 0.0, 0.0, 0.0], [2.0, 1.0, 0.0, 0.0]]])
    C = 2 * dk + d + 2
    w = np.zeros((C, D), np.float32)
    w[2 * dk + d, 0] = 1.0
    bias = np.array([[-2.0, math.log(3.0)]], np.float32)
    _, _, _, al, be = p.project(B, T, H, D, dk, d, x, _b(w), bias)
    assert np.all(al == 0.5)
    assert np.allclose(be, 0.75, rtol=0, atol=1e-7)
    bias = np.array([[math.log(3.0) - 2.0, -math.log(3.0)]], np.float32)
    _, _, _, al, be = p.project(B, T, H, D, dk, d, x, _b(w), bias)
    assert np.allclose(be, 0.25, rtol=0, atol=1e-7)
    assert np.allclose(al, 0.75, rtol=0, atol=1e-7)


def pin_rounding_of_ties(p):
    """Sums exactly halfway between two bf16 values round to the even one:
    1 + 2^-8 -> 1;  1 + 3*2^-8 -> 1 + 2^-6;  -(1 + 2^-8) -> -1."""
    B, T, H, D, dk, d = 1, 3, 1, 2, 1, 1
    x = _b([[[1.0, 2.0 ** -8], [1.0, 3 * 2.0 ** -8], [-1.0, -(2.0 ** -8)]]])
    C = 2 * dk + d + 2
    w = np.zeros((C, D), np.float32)
    w[0] = [1.0, 1.0]
    wq, _, _, _, _ = p.project(B, T, H, D, dk, d, x, _b(w), np.zeros((1, 2), np.float32))
    assert list(_f(wq)[0, :, 0, 0]) == [1.0, 1.0 + 2.0 ** -6, -1.0]


def pin_broadcast(p):
    m0 = np.arange(2 * 5 * 3, dtype=np.float32).reshape(2, 5, 3)
    mem = p.broadcast_memory(4, m0)
    assert mem.shape == (4, 2, 5, 3) and all(np.array_equal(mem[b], m0) for b in range(4))


PINS = [pin_worked_example, pin_identity_and_one_hot, pin_gate_closed_forms, pin_rounding_of_ties, pin_broadcast]


# --- the write/read bucket-overlap diagnostic (sdm_oracle_diag.c) -----------------------------

def pin_overlap_worked_example(p):
    """T = 3 tokens, W = 2, N = 8 slots, K = 4 buckets (bucket = n // 2).
    writes: t0 {1: .5, 6: .5}, t1 {2: .25, 3: .75}, t2 {6: 1, 0: 0};  reads: t0 {6: 1, 5: 0},
    t1 {1: .5, 2: .5}, t2 {6: .5, 3: .5}.
    cumulative write mass per bucket: t0 (.5, 0, 0, .5), t1 (.5, 1, 0, .5), t2 (.5, 1, 0, 1.5);
    read mass (slot 5 of t0 carries weight 0): t0 (0, 0, 0, 1), t1 (.5, .5, 0, 0), t2 (0, .5, 0, .5).  Overlap for query 2: a=0 shares slot 6: .5*.5 = .25; a=1 shares slot 3:
    .75*.5 = .375; a=2 shares slot 6: 1*.5 = .5.  Query 0: a=0 shares slot 6: .5*1 = .5; later tokens 0."""
    idx_w = np.array([[1, 6], [2, 3], [6, 0]], np.int32)
    wt_w = np.array([[.5, .5], [.25, .75], [1.0, 0.0]], np.float32)
    idx_r = np.array([[6, 5], [1, 2], [6, 3]], np.int32)
    wt_r = np.array([[1.0, 0.0], [.5, .5], [.5, .5]], np.float32)
    wc, rd, ov = p.overlap(1, 3, 1, 2, 8, 4, idx_w, wt_w, idx_r, wt_r, [2, 0])
    assert np.array_equal(wc[0, 0], np.array([[.5, 0, 0, .5], [.5, 1, 0, .5], [.5, 1, 0, 1.5]], np.float32))
    assert np.array_equal(rd[0, 0], np.array([[0, 0, 0, 1], [.5, .5, 0, 0], [0, .5, 0, .5]], np.float32))
    assert np.array_equal(ov[0, 0], np.array([[.25, .375, .5], [.5, 0, 0]], np.float32))


def pin_overlap_planted_needle(p):
    """A read query equal to an earlier write query selects the same slots with the same weights (the
    forward oracle's addressing), so their overlap is the sum of the squared weights; the total write
    mass after t tokens is t + 1 and every token's read mass is 1 (softmax weights), up to rounding."""
    import oracle as _o
    from sdm_inputs import Config
    cfg = Config(name="needle", B=1, H=2, T=40, d=8, S=16, dk=16, k=4, W=8, in_bf16=False, state_bf16=False)
    rng = np.random.default_rng(7)
    wq = rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dk)).astype(np.float32)
    rq = rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dk)).astype(np.float32)
    rq[:, 33] = wq[:, 5]
    sub = (rng.standard_normal((cfg.H, 2, cfg.S, cfg.dk // 2)) * 0.5).astype(np.float32)
    f = _o.get()
    iw, ww, _ = f.address(cfg, wq, sub)
    ir, wr, _ = f.address(cfg, rq, sub)
    wc, rd, ov = p.overlap(cfg.B, cfg.T, cfg.H, cfg.W, cfg.N, cfg.S, iw, ww, ir, wr, [33])
    for h in range(cfg.H):
        w5 = ww[(0 * cfg.T + 5) * cfg.H + h].astype(np.float64)
        assert ov[0, h, 0, 5] == np.float32(np.sum(w5 * w5))
        assert np.all(ov[0, h, 0, 34:] == 0)
        assert np.allclose(wc[0, h].sum(axis=1), np.arange(1, cfg.T + 1), rtol=0, atol=1e-5)
        assert np.allclose(rd[0, h].sum(axis=1), 1.0, rtol=0, atol=1e-6)


PINS += [pin_overlap_worked_example, pin_overlap_planted_needle]
