"""Pins that tie the oracle to something other than itself.

Each pin takes an oracle handle and raises AssertionError when the oracle
disagrees with an independent statement of what SDM computes: a hand-worked
example, closed forms, brute force over every slot, the dense Gated DeltaNet
recurrence the method reduces to, and invariances of the recurrence.  None of
them calls the GPU library.  The same pins are re-run against deliberately
broken builds of the oracle (test_oracle_mutants.py) to show that each planted
mistake is caught by at least one of them.

Sources of the statements (SDM blog post, lcabannes.github.io/sdm-blogpost):
  - section "How does SDM work?" and its "Write & Read" subsection: a d x N
    memory of slot vectors; select slots with product keys, decay the
    write-selected slots and apply the delta rule, then read a weighted sum of
    (possibly different) read-selected slots;
  - caption of the figure "The SDM mechanism, end to end": two sub-key score
    sets, outer sum, top-k (W = 64), decay then delta-v, softmax-weighted read;
  - section "Background": SDM extends Gated DeltaNet by swapping its dense
    state for the slot memory; W = 64 of about 230K slots at 1.4B.
Readings where the pages are silent (slot n = a*S + b, lower index wins ties,
softmax weights also for the write, no temperature, decay only on written
slots, read after the write) are the ones the oracle states.
"""
from __future__ import annotations

import math

import numpy as np

from sdm_inputs import Config, f32_from_bf16_bits

F32 = np.float32


def _cfg(**kw) -> Config:
    base = dict(name="pin", B=1, H=1, T=8, d=4, S=4, dk=4, k=2, W=2, in_bf16=False, state_bf16=False)
    base.update(kw)
    return Config(**base)


def _rand_inputs(cfg: Config, seed: int, m0_std=0.5, alpha=None, beta=None):
    rng = np.random.default_rng(seed)
    wq = rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dk)).astype(F32)
    rq = rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dk)).astype(F32)
    v = rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.d)).astype(F32)
    a = (1 / (1 + np.exp(-(rng.standard_normal((cfg.B, cfg.T, cfg.H)) + 2)))).astype(F32)
    b = (1 / (1 + np.exp(-rng.standard_normal((cfg.B, cfg.T, cfg.H))))).astype(F32)
    if alpha is not None:
        a[...] = alpha
    if beta is not None:
        b[...] = beta
    sk = (rng.standard_normal((cfg.H, 2, cfg.S, cfg.dh)) * 0.5).astype(F32)
    m0 = (rng.standard_normal((cfg.B, cfg.H, cfg.N, cfg.d)) * m0_std).astype(F32)
    return dict(wq=wq, rq=rq, v=v, alpha=a, beta=b, subkeys=sk, mem0=m0)


def _forward(o, cfg, x):
    mem = x["mem0"].copy()
    out, aw, ar = o.forward(cfg, x["wq"], x["rq"], x["v"], x["alpha"], x["beta"], x["subkeys"], mem, threads=1)
    return out, mem, aw, ar


# --------------------------------------------------------------------------
# independent statements of the addressing
# --------------------------------------------------------------------------

def np_scores(cfg, q, subkeys):
    """[R, 2, S] half scores: float64 dot products, one rounding to float32."""
    R = cfg.B * cfg.T * cfg.H
    q = q.reshape(R, cfg.dk).astype(np.float64)
    out = np.empty((R, 2, cfg.S), F32)
    for r in range(R):
        h = r % cfg.H
        for half in range(2):
            tab = subkeys[h, half].astype(np.float64)
            out[r, half] = (tab @ q[r, half * cfg.dh:(half + 1) * cfg.dh]).astype(F32)
    return out


def _order(values, ids):
    """Permutation sorting by value descending, then id ascending."""
    return np.lexsort((ids, -values))


def brute_select_all_slots(s1, s2, W):
    """Top-W over every one of the S*S slot sums (no product-key pruning)."""
    S = s1.size
    sig = (s1[:, None] + s2[None, :]).astype(F32).ravel()
    n = (np.arange(S)[:, None] * S + np.arange(S)[None, :]).ravel()
    o = _order(sig, n)[:W]
    return n[o].astype(np.int32), sig[o]


def brute_select_candidates(s1, s2, k, W):
    """Per-half top-k, then top-W over all k*k candidate pairs, by enumeration."""
    S = s1.size
    A = _order(s1, np.arange(S))[:k]
    B = _order(s2, np.arange(S))[:k]
    sig = np.array([F32(s1[a]) + F32(s2[b]) for a in A for b in B], dtype=F32)
    n = np.array([a * S + b for a in A for b in B], dtype=np.int64)
    o = _order(sig, n)[:W]
    return n[o].astype(np.int32), sig[o]


def softmax_f32(sig):
    z = np.exp(sig.astype(np.float64) - sig.astype(np.float64).max())
    return (z / z.sum()).astype(F32)


# --------------------------------------------------------------------------
# pins
# --------------------------------------------------------------------------

def pin_bf16_bits(o):
    """Nearest-even rounding to bfloat16, straight from double, on hand-computed bit patterns."""
    cases = [
        (1.0, 0x3F80), (-2.5, 0xC020), (3.140625, 0x4049),
        (1 + 2 ** -8, 0x3F80),                 # tie -> even (down)
        (1 + 3 * 2 ** -8, 0x3F82),             # tie -> even (up)
        (1 + 2 ** -8 + 2 ** -30, 0x3F81),      # just above a tie: one rounding from double
        (1 + 2 ** -8 - 2 ** -30, 0x3F80),
        ((2 - 2 ** -8) * 2.0 ** 127, 0x7F80),  # tie above the largest finite value -> inf
        ((2 - 2 ** -7) * 2.0 ** 127, 0x7F7F),  # largest finite
        (2.0 ** -133, 0x0001),                 # smallest subnormal
        (2.0 ** -134, 0x0000),                 # tie between 0 and the smallest subnormal -> even
        (1.5 * 2.0 ** -133, 0x0002),           # tie -> even
        (2.0 ** -126, 0x0080),                 # smallest normal
        (0.0, 0x0000), (-0.0, 0x8000), (math.inf, 0x7F80), (-math.inf, 0xFF80),
    ]
    for x, bits in cases:
        got = o.bf16_round(x)
        assert got == bits, f"bf16({x!r}) = {got:#06x}, expected {bits:#06x}"
    assert (o.bf16_round(math.nan) & 0x7FC0) == 0x7FC0


def pin_worked_example(o):
    """Two tokens on a 2x2 product-key memory, worked by hand.

    Sub-key tables (dk/2 = 1): K0 = [1, 0.5], K1 = [-1, 0.25]; slots n = a*2 + b.
    Token 0 write query (1, 2): s1 = (1, .5), s2 = (-2, .5); sums (a,b):
      (0,1)=1.5 n=1, (1,1)=1.0 n=3, (0,0)=-1 n=0, (1,0)=-1.5 n=2 -> slots (1, 3),
      weights (1, e^-.5)/(1 + e^-.5).
    Token 1 write query (0, 4): s1 = (0, 0) tied, s2 = (-4, 1): slots (1, 3) with the
      sums tied at 1.0 -> the lower slot comes first; weights (1/2, 1/2).
    Token 0 read query (2, 0): s2 = (0, 0) tied -> slots (0, 1) tied at 2 -> (1/2, 1/2).
    Token 1 read query (1, 2): as token 0's write -> slots (1, 3).
    Memory slot n starts at (2n+1, 2n+2); alpha = (.5, 1), beta = (.5, .25),
    v = ((10, 20), (-4, 8)).
    """
    cfg = _cfg(T=2, d=2, S=2, dk=2, k=2, W=2)
    wq = np.array([[1, 2], [0, 4]], F32).reshape(1, 2, 1, 2)
    rq = np.array([[2, 0], [1, 2]], F32).reshape(1, 2, 1, 2)
    sk = np.array([[[1.0], [0.5]], [[-1.0], [0.25]]], F32).reshape(1, 2, 2, 1)
    v = np.array([[10, 20], [-4, 8]], F32).reshape(1, 2, 1, 2)
    alpha = np.array([0.5, 1.0], F32).reshape(1, 2, 1)
    beta = np.array([0.5, 0.25], F32).reshape(1, 2, 1)
    m0 = np.array([[1, 2], [3, 4], [5, 6], [7, 8]], F32).reshape(1, 1, 4, 2)
    x = dict(wq=wq, rq=rq, v=v, alpha=alpha, beta=beta, subkeys=sk, mem0=m0)
    out, mem, (iw, ww, sw), (ir, wr, sr) = _forward(o, cfg, x)

    e = math.exp(-0.5)
    w0, w1 = 1 / (1 + e), e / (1 + e)
    assert iw.tolist() == [[1, 3], [1, 3]], iw
    assert ir.tolist() == [[0, 1], [1, 3]], ir
    assert sw.tolist() == [[1.5, 1.0], [1.0, 1.0]], sw
    assert sr.tolist() == [[2.0, 2.0], [1.5, 1.0]], sr
    np.testing.assert_allclose(ww, [[w0, w1], [0.5, 0.5]], rtol=2 ** -23)
    np.testing.assert_allclose(wr, [[0.5, 0.5], [w0, w1]], rtol=2 ** -23)
    W0, W1 = float(F32(w0)), float(F32(w1))  # the weights are float32 values

    # token 0: decay slots 1 and 3 by 0.5, predict, delta-rule write, read slots 0 and 1
    x1, x3 = np.array([1.5, 2.0]), np.array([3.5, 4.0])
    vhat = W0 * x1 + W1 * x3
    delta = 0.5 * (np.array([10.0, 20.0]) - vhat)
    m1, m3 = (x1 + W0 * delta).astype(F32), (x3 + W1 * delta).astype(F32)
    out0 = 0.5 * np.array([1.0, 2.0]) + 0.5 * m1.astype(np.float64)
    # token 1: no decay, equal weights, beta 0.25; read slots 1 and 3
    vhat = 0.5 * m1.astype(np.float64) + 0.5 * m3.astype(np.float64)
    delta = 0.25 * (np.array([-4.0, 8.0]) - vhat)
    m1b = (m1.astype(np.float64) + 0.5 * delta).astype(F32)
    m3b = (m3.astype(np.float64) + 0.5 * delta).astype(F32)
    out1 = W0 * m1b.astype(np.float64) + W1 * m3b.astype(np.float64)

    np.testing.assert_allclose(out[0, :, 0], np.stack([out0, out1]), rtol=3e-7, atol=0)
    exp_mem = np.array([[1, 2], m1b, [5, 6], m3b], dtype=np.float64)
    np.testing.assert_allclose(mem[0, 0], exp_mem, rtol=3e-7, atol=0)


def pin_scores(o):
    """Half scores against float64 matrix products: bit-equal on dyadic inputs
    (every sum exact), within one float32 rounding on Gaussian inputs."""
    rng = np.random.default_rng(11)
    cfg = _cfg(B=2, T=5, H=3, S=7, dk=10, k=3, W=4)
    q = (rng.integers(-16, 17, (cfg.B, cfg.T, cfg.H, cfg.dk)) / 8).astype(F32)
    sk = (rng.integers(-16, 17, (cfg.H, 2, cfg.S, cfg.dh)) / 4).astype(F32)
    got = o.scores(cfg, q, sk, threads=1)
    assert np.array_equal(got, np_scores(cfg, q, sk))
    q = rng.standard_normal(q.shape).astype(F32)
    sk = rng.standard_normal(sk.shape).astype(F32)
    got = o.scores(cfg, q, sk, threads=1)
    ref = np_scores(cfg, q, sk)
    np.testing.assert_allclose(got, ref, rtol=2 ** -23, atol=1e-30)
    # bf16 inputs are widened exactly
    qb = (q.view(np.uint32) >> 16).astype(np.uint16)
    skb = (sk.view(np.uint32) >> 16).astype(np.uint16)
    got = o.scores(cfg.replace(in_bf16=True), qb, skb, threads=1)
    ref = np_scores(cfg, f32_from_bf16_bits(qb).reshape(q.shape), f32_from_bf16_bits(skb).reshape(sk.shape))
    np.testing.assert_allclose(got, ref, rtol=2 ** -23, atol=1e-30)


def pin_select_equals_exhaustive_when_k_ge_W(o):
    """With k >= W, product-key top-W equals top-W over all S*S slots: a pair
    left out of a per-half top-k is beaten by >= k >= W pairs of its column or row."""
    rng = np.random.default_rng(5)
    for S, k, W in ((8, 8, 8), (16, 16, 16), (16, 12, 12), (5, 5, 3), (9, 4, 1), (12, 6, 6)):
        for _ in range(40):
            s1 = rng.standard_normal(S).astype(F32)
            s2 = rng.standard_normal(S).astype(F32)
            if rng.random() < 0.3:  # coarse values -> many exact ties
                s1, s2 = np.round(s1 * 2) / 2, np.round(s2 * 2) / 2
                s1, s2 = s1.astype(F32), s2.astype(F32)
            got_n, got_s = o.select(s1, s2, k, W)
            ref_n, ref_s = brute_select_all_slots(s1, s2, W)
            assert np.array_equal(got_n, ref_n), (S, k, W, got_n, ref_n)
            assert np.array_equal(got_s, ref_s)


def pin_select_candidates_k_lt_W(o):
    """With k < W the result is top-W of the k*k candidate pairs (enumerated)."""
    rng = np.random.default_rng(6)
    for S, k, W in ((16, 4, 16), (16, 5, 9), (30, 6, 20), (64, 8, 16)):
        for _ in range(30):
            s1 = rng.standard_normal(S).astype(F32)
            s2 = rng.standard_normal(S).astype(F32)
            got_n, got_s = o.select(s1, s2, k, W)
            ref_n, ref_s = brute_select_candidates(s1, s2, k, W)
            assert np.array_equal(got_n, ref_n), (S, k, W)
            assert np.array_equal(got_s, ref_s)


def pin_ties_lower_index_wins(o):
    """Duplicated sub-key rows give exactly tied scores; the lower index goes first."""
    rng = np.random.default_rng(7)
    cfg = _cfg(T=3, S=6, dk=8, k=3, W=5)
    sk = (rng.standard_normal((1, 2, 6, 4)) * 0.1).astype(F32)
    sk[0, 0, 1] = sk[0, 0, 4] = [1, 1, 1, 1]      # table 0: sub-keys 1 and 4 identical
    sk[0, 1, 0] = sk[0, 1, 5] = [1, -1, 1, -1]    # table 1: sub-keys 0 and 5 identical
    q = np.zeros((1, 3, 1, 8), F32)
    q[0, :, 0, :4] = [1, 1, 1, 1]
    q[0, :, 0, 4:] = [1, -1, 1, -1]
    sc = o.scores(cfg, q, sk, threads=1)
    assert sc[0, 0, 1] == sc[0, 0, 4] and sc[0, 1, 0] == sc[0, 1, 5]
    assert o.topk(sc[0, 0], 2).tolist() == [1, 4]
    assert o.topk(sc[0, 1], 2).tolist() == [0, 5]
    idx, _, sig = o.address(cfg, q, sk, threads=1)
    # the four tied best pairs (1,0) (1,5) (4,0) (4,5) in slot order
    assert idx[0, :4].tolist() == [1 * 6 + 0, 1 * 6 + 5, 4 * 6 + 0, 4 * 6 + 5], idx[0]
    assert len(set(sig[0, :4].tolist())) == 1


def pin_softmax(o):
    """Weights are positive, ordered like the sums, sum to one; two-way closed form."""
    rng = np.random.default_rng(8)
    for W in (1, 2, 7, 64):
        sig = np.sort(rng.standard_normal(W).astype(F32) * 4)[::-1].copy()
        w = o.softmax(sig)
        assert (w > 0).all() and np.all(np.diff(w) <= 0)
        assert abs(float(w.astype(np.float64).sum()) - 1.0) <= W * 2 ** -24
    for d in (0.0, 0.5, 3.0, 20.0):
        w = o.softmax(np.array([d, 0.0], F32))
        assert w[0] == F32(1 / (1 + math.exp(-d))) and w[1] == F32(math.exp(-d) / (1 + math.exp(-d)))
    assert np.all(o.softmax(np.full(8, 1.25, F32)) == F32(0.125))
    # invariance to a common shift of the sums (dyadic values: the shift is exact)
    s = (np.round(rng.standard_normal(16) * 64) / 64).astype(F32)
    assert np.array_equal(o.softmax(s), o.softmax(s + F32(8)))


def pin_one_hot_write(o):
    """W = 1: the slot becomes alpha*(1-beta)*M + beta*v; with alpha = beta = 1 it
    becomes v exactly, and a read with the same query returns v exactly."""
    cfg = _cfg(B=1, H=2, T=16, d=5, S=6, dk=6, k=1, W=1)
    x = _rand_inputs(cfg, 21)
    mem0 = x["mem0"].copy()
    out, mem, (iw, ww, _), _ = _forward(o, cfg, x)
    assert np.all(ww == 1.0)
    # replay the closed form slot by slot
    ref = mem0.astype(np.float64)
    for t in range(cfg.T):
        for h in range(cfg.H):
            r = t * cfg.H + h
            n = iw[r, 0]
            a, b = float(x["alpha"][0, t, h]), float(x["beta"][0, t, h])
            ref[0, h, n] = (a * (1 - b) * ref[0, h, n] + b * x["v"][0, t, h].astype(np.float64))
            ref[0, h, n] = ref[0, h, n].astype(F32)
    np.testing.assert_allclose(mem, ref, rtol=2 ** -22, atol=1e-30)
    # alpha = beta = 1 and read query = write query -> out == v bit for bit
    x2 = _rand_inputs(cfg, 22, alpha=1.0, beta=1.0)
    x2["rq"] = x2["wq"].copy()
    out, mem, (iw, _, _), _ = _forward(o, cfg, x2)
    assert np.array_equal(out, x2["v"])
    for t in range(cfg.T):
        for h in range(cfg.H):
            last = max(tt for tt in range(cfg.T) if iw[tt * cfg.H + h, 0] == iw[t * cfg.H + h, 0])
            assert np.array_equal(mem[0, h, iw[t * cfg.H + h, 0]], x2["v"][0, last, h])


def _dense_run(cfg, x, sel_w, w_w, sel_r, w_r, state_round):
    """Matrix form of the recurrence on M (d x N) per memory, float64 math:
         M <- M D_t  with D_t = I - (1 - alpha_t) diag(selected_t)
         M <- M + beta_t (v_t - M k_t) k_t^T
         o_t = M q_t
    where k_t, q_t are the length-N weight vectors (zero off the selection).
    With every slot selected this is Gated DeltaNet's recurrence."""
    B, T, H, N = cfg.B, cfg.T, cfg.H, cfg.N
    out = np.zeros((B, T, H, cfg.d), F32)
    M = x["mem0"].astype(np.float64).transpose(0, 1, 3, 2).copy()  # [B, H, d, N]
    for b in range(B):
        for h in range(H):
            Mb = M[b, h]
            for t in range(T):
                r = (b * T + t) * H + h
                kv = np.zeros(N)
                kv[sel_w[r]] = w_w[r]
                qv = np.zeros(N)
                qv[sel_r[r]] = w_r[r]
                dmask = np.ones(N)
                dmask[sel_w[r]] = x["alpha"][b, t, h]
                Mb = Mb * dmask[None, :]
                pred = Mb @ kv
                Mb = Mb + x["beta"][b, t, h] * np.outer(x["v"][b, t, h].astype(np.float64) - pred, kv)
                Mb[:, sel_w[r]] = state_round(Mb[:, sel_w[r]])
                out[b, t, h] = (Mb @ qv).astype(F32)
            M[b, h] = Mb
    return out, M.transpose(0, 1, 3, 2)


def _round_f32(a):
    return a.astype(F32).astype(np.float64)


def pin_dense_gdn_all_slots(o):
    """W = N (k = S, every slot selected): the sparse scan is the dense gated
    delta rule with the softmax over all N slot scores as its key and query."""
    cfg = _cfg(B=2, H=2, T=12, d=3, S=4, dk=4, k=4, W=16)
    x = _rand_inputs(cfg, 31)
    out, mem, aw, ar = _forward(o, cfg, x)
    sw = np_scores(cfg, x["wq"], x["subkeys"])
    sr = np_scores(cfg, x["rq"], x["subkeys"])
    R = cfg.B * cfg.T * cfg.H
    all_n = np.arange(cfg.N)
    sig = lambda s: (s[:, 0, :, None] + s[:, 1, None, :]).astype(F32).reshape(R, cfg.N)
    kw = np.stack([softmax_f32(z) for z in sig(sw)])
    kr = np.stack([softmax_f32(z) for z in sig(sr)])
    ref_out, ref_mem = _dense_run(cfg, x, [all_n] * R, list(kw), [all_n] * R, list(kr), _round_f32)
    scale_o = np.sqrt(np.mean(ref_out.astype(np.float64) ** 2))
    scale_m = np.sqrt(np.mean(ref_mem ** 2))
    assert np.max(np.abs(out - ref_out)) <= 1e-6 * scale_o
    assert np.max(np.abs(mem - ref_mem)) <= 1e-6 * scale_m


def pin_dense_masked(o):
    """General W: the scan equals the masked dense form (decay only the selected
    columns), with the selection done by candidate enumeration."""
    for state_bf16, tol in ((False, 1e-6), (True, 2 ** -5)):
        cfg = _cfg(B=1, H=2, T=24, d=6, S=6, dk=6, k=3, W=5, state_bf16=state_bf16)
        x = _rand_inputs(cfg, 41)
        if state_bf16:
            x["mem0"] = (x["mem0"].view(np.uint32) >> 16).astype(np.uint16)
        out, mem, aw, ar = _forward(o, cfg, x)
        sw = np_scores(cfg, x["wq"], x["subkeys"])
        sr = np_scores(cfg, x["rq"], x["subkeys"])
        R = cfg.B * cfg.T * cfg.H
        sel_w, w_w, sel_r, w_r = [], [], [], []
        for r in range(R):
            n, s = brute_select_candidates(sw[r, 0], sw[r, 1], cfg.k, cfg.W)
            sel_w.append(n)
            w_w.append(softmax_f32(s))
            n, s = brute_select_candidates(sr[r, 0], sr[r, 1], cfg.k, cfg.W)
            sel_r.append(n)
            w_r.append(softmax_f32(s))
        xx = dict(x)
        if state_bf16:
            xx["mem0"] = f32_from_bf16_bits(x["mem0"]).reshape(x["mem0"].shape)
            rnd = lambda a: f32_from_bf16_bits(
                ((a.astype(F32).view(np.uint32) + 0x7FFF + ((a.astype(F32).view(np.uint32) >> 16) & 1)) >> 16)
                .astype(np.uint16)).reshape(a.shape).astype(np.float64)
            got_mem = f32_from_bf16_bits(mem).reshape(mem.shape)
        else:
            rnd = _round_f32
            got_mem = mem
        ref_out, ref_mem = _dense_run(cfg, xx, sel_w, w_w, sel_r, w_r, rnd)
        scale_o = np.sqrt(np.mean(ref_out.astype(np.float64) ** 2))
        scale_m = np.sqrt(np.mean(ref_mem ** 2))
        assert np.max(np.abs(out - ref_out)) <= tol * scale_o, (state_bf16, np.max(np.abs(out - ref_out)))
        assert np.max(np.abs(got_mem - ref_mem)) <= tol * scale_m


def pin_identity_gates(o):
    """alpha = 1, beta = 0: the memory is unchanged bit for bit and the output is
    a plain weighted gather of the initial slots."""
    cfg = _cfg(B=2, H=2, T=10, d=7, S=8, dk=6, k=3, W=6)
    x = _rand_inputs(cfg, 51, alpha=1.0, beta=0.0)
    out, mem, aw, (ir, wr, _) = _forward(o, cfg, x)
    assert np.array_equal(mem, x["mem0"])
    R = cfg.B * cfg.T * cfg.H
    ref = np.empty_like(out)
    for r in range(R):
        b, t, h = r // (cfg.T * cfg.H), (r // cfg.H) % cfg.T, r % cfg.H
        ref[b, t, h] = (wr[r].astype(np.float64) @ x["mem0"][b, h, ir[r]].astype(np.float64)).astype(F32)
    np.testing.assert_allclose(out, ref, rtol=2 ** -22, atol=1e-30)


def pin_chunking(o):
    """Running T1 tokens and then T2 tokens from the resulting memory equals one
    run over T1 + T2 tokens, bit for bit."""
    cfg = _cfg(B=2, H=1, T=20, d=4, S=5, dk=4, k=3, W=4)
    x = _rand_inputs(cfg, 61)
    out, mem, _, _ = _forward(o, cfg, x)
    T1 = 7
    parts, m = [], x["mem0"].copy()
    for sl in (slice(0, T1), slice(T1, cfg.T)):
        c = cfg.replace(T=sl.stop - sl.start)
        xs = {k_: (v_[:, sl].copy() if k_ in ("wq", "rq", "v", "alpha", "beta") else v_) for k_, v_ in x.items()}
        xs["mem0"] = m
        o_, m, _, _ = _forward(o, c, xs)
        parts.append(o_)
    assert np.array_equal(np.concatenate(parts, axis=1), out)
    assert np.array_equal(m, mem)


def pin_permute_d(o):
    """Permuting the slot elements of (v, M0) permutes (out, M_T) bit for bit."""
    cfg = _cfg(B=1, H=2, T=9, d=6, S=5, dk=4, k=2, W=3)
    x = _rand_inputs(cfg, 71)
    out, mem, _, _ = _forward(o, cfg, x)
    p = np.random.default_rng(72).permutation(cfg.d)
    xp = dict(x)
    xp["v"] = x["v"][..., p].copy()
    xp["mem0"] = x["mem0"][..., p].copy()
    out_p, mem_p, _, _ = _forward(o, cfg, xp)
    assert np.array_equal(out_p, out[..., p]) and np.array_equal(mem_p, mem[..., p])


def pin_power_of_two_scaling(o):
    """Scaling (v, M0) by 2^p scales (out, M_T) by 2^p bit for bit (float32 state)."""
    cfg = _cfg(B=1, H=1, T=11, d=5, S=5, dk=4, k=3, W=4)
    x = _rand_inputs(cfg, 81)
    out, mem, _, _ = _forward(o, cfg, x)
    for p in (-3, 5):
        xs = dict(x)
        xs["v"] = (x["v"] * F32(2.0 ** p)).astype(F32)
        xs["mem0"] = (x["mem0"] * F32(2.0 ** p)).astype(F32)
        out_s, mem_s, _, _ = _forward(o, cfg, xs)
        assert np.array_equal(out_s, (out * F32(2.0 ** p)).astype(F32))
        assert np.array_equal(mem_s, (mem * F32(2.0 ** p)).astype(F32))


def pin_planted_query(o):
    """A read query equal to an earlier write query selects the same slots with
    the same weights (the long-context workload plants token 61 -> T-17)."""
    from sdm_inputs import config, make_inputs
    cfg = config(3, T=128, d=8, S=32, m0_std=0.02)
    x = make_inputs(cfg, with_mem0=False)
    rows_w, rows_r = [61], [cfg.T - 17]
    iw, ww, sw = o.address(cfg, x["wq"], x["subkeys"], rows=rows_w, threads=1)
    ir, wr, sr = o.address(cfg, x["rq"], x["subkeys"], rows=rows_r, threads=1)
    assert np.array_equal(iw, ir) and np.array_equal(ww, wr) and np.array_equal(sw, sr)


def pin_address_from_scores(o):
    """Selection from given scores, row by row: against candidate enumeration and
    a float64 softmax written here (indices exact, weights within one float32
    unit), on rows with ties planted, and bit for bit against the oracle's own
    addressing from queries when handed the oracle's scores of those queries.
    The staged GPU checks lean on this routine; it must address every row."""
    cfg = _cfg(B=3, H=2, T=7, d=4, S=13, dk=8, k=4, W=10)
    R = cfg.B * cfg.T * cfg.H
    rng = np.random.default_rng(91)
    sc = rng.standard_normal((R, 2, cfg.S)).astype(F32)
    sc[3, 0, 5] = sc[3, 0, 9]                        # a tie inside one half
    sc[7, 1] = np.round(sc[7, 1] * 2) / 2            # quantised half: many ties
    sc[11] = 0.25                                    # every score equal
    sc[12, 0, 2], sc[12, 1, 0] = 1.5, 1.0            # two pairs with the same sum
    sc[12, 0, 3], sc[12, 1, 4] = 1.0, 1.5
    idx, wt, sig = o.address_from_scores(cfg, sc, threads=3)
    for r in range(R):
        n, s = brute_select_candidates(sc[r, 0], sc[r, 1], cfg.k, cfg.W)
        assert np.array_equal(idx[r], n), f"row {r}: slots {idx[r]} != {n}"
        assert np.array_equal(sig[r], s), f"row {r}: sums differ"
        u = np.abs(wt[r].view(np.int32).astype(np.int64) - softmax_f32(s).view(np.int32).astype(np.int64))
        assert u.max() <= 1, f"row {r}: weights differ by {u.max()} units"
    x = _rand_inputs(cfg, 92)
    for q in (x["wq"], x["rq"]):
        ai, aw, asg = o.address(cfg, q, x["subkeys"], threads=1)
        fi, fw, fsg = o.address_from_scores(cfg, o.scores(cfg, q, x["subkeys"], threads=1), threads=1)
        assert np.array_equal(ai, fi) and np.array_equal(aw.view(np.uint32), fw.view(np.uint32))
        assert np.array_equal(asg.view(np.uint32), fsg.view(np.uint32))


def pin_threads_bitwise(o):
    """The driver's split of the work over threads changes no bit: row spans of
    the scores and addressing, and the scan's slot-element slices (the element
    offset inside the C scan), against one thread over everything; the scores
    also against float64 dot products written here."""
    cfg = _cfg(B=2, H=2, T=23, d=37, S=9, dk=6, k=3, W=7)
    x = _rand_inputs(cfg, 93)
    R = cfg.B * cfg.T * cfg.H
    s1 = o.scores(cfg, x["wq"], x["subkeys"], threads=1)
    s16 = o.scores(cfg, x["wq"], x["subkeys"], threads=16)
    assert np.array_equal(s1.view(np.uint32), s16.view(np.uint32))
    assert np.array_equal(s16, np_scores(cfg, x["wq"], x["subkeys"]))
    a1 = o.address(cfg, x["wq"], x["subkeys"], threads=1)
    a16 = o.address(cfg, x["wq"], x["subkeys"], threads=16)
    f16 = o.address_from_scores(cfg, s16, threads=16)
    sub = o.address(cfg, x["wq"], x["subkeys"], rows=np.arange(R)[::-1], threads=16)
    for u, w in zip(a1, a16):
        assert np.array_equal(u.view(np.uint32), w.view(np.uint32))
    for u, w in zip(a1, f16):
        assert np.array_equal(u.view(np.uint32), w.view(np.uint32))
    for u, w in zip(a1, sub):
        assert np.array_equal(u[::-1].view(np.uint32), w.view(np.uint32))
    ar = o.address(cfg, x["rq"], x["subkeys"], threads=1)
    runs = []
    for threads, e_split in ((1, 1), (16, None), (16, 5), (4, cfg.d)):
        mem = x["mem0"].copy()
        out = o.scan(cfg, a1[0], a1[1], ar[0], ar[1], x["v"], x["alpha"], x["beta"], mem, threads=threads,
                     e_split=e_split)
        runs.append((out, mem))
    for out, mem in runs[1:]:
        assert np.array_equal(out.view(np.uint32), runs[0][0].view(np.uint32))
        assert np.array_equal(mem.view(np.uint32), runs[0][1].view(np.uint32))


PINS = [
    pin_bf16_bits,
    pin_worked_example,
    pin_scores,
    pin_select_equals_exhaustive_when_k_ge_W,
    pin_select_candidates_k_lt_W,
    pin_ties_lower_index_wins,
    pin_softmax,
    pin_one_hot_write,
    pin_dense_gdn_all_slots,
    pin_dense_masked,
    pin_identity_gates,
    pin_chunking,
    pin_permute_d,
    pin_power_of_two_scaling,
    pin_planted_query,
    pin_address_from_scores,
    pin_threads_bitwise,
]
