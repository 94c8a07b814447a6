"""Pins that tie the gradient oracle (oracle/sdm_oracle_grad.c) to something
other than itself.

A gradient is pinned by what defines it: the derivative of the forward.  Each
finite-difference pin perturbs one input of the forward oracle's own scan (a
float64-storage build of it, so that the loss is smooth) or of the double
weight function, and compares Richardson-extrapolated central differences with
the gradient the backward oracle returns.  The closed-form pins take the cases
where the recurrence collapses: with decay 1 and step size 0 the memory never
changes, so every gradient has a short explicit form; with one selected slot
the softmax weight is always 1 and the queries get no gradient.  Each pin
takes a gradient-oracle handle and raises AssertionError on disagreement; the
same pins run against planted mistakes (test_oracle_grad_mutants.py).

What is differentiated: SDM blog post, section "How does SDM work?", its
"Write & Read" subsection and the caption of the figure "The SDM mechanism,
end to end" (decay, delta-rule write, read after the write; softmax weights of
product-key selected slots).  Readings: the selection is held fixed and the
state rounding is the identity for the gradient.
"""
from __future__ import annotations

import numpy as np

from sdm_inputs import Config

Q = 2.0 ** -12  # inputs on this grid, so that x +- 2^-8 and x +- 2^-9 are exact in float32
H1, H2 = 2.0 ** -8, 2.0 ** -9


def _cfg(**kw) -> Config:
    base = dict(name="gpin", B=2, H=2, T=9, d=6, S=3, dk=4, k=2, W=4, in_bf16=False, state_bf16=2)
    base.update(kw)
    return Config(**base)


def _grid(x):
    return (np.round(np.asarray(x, np.float64) / Q) * Q).astype(np.float32)


def scan_inputs(cfg: Config, seed: int, alpha=None, beta=None):
    """Random scan inputs; slots distinct within a token, repeated across tokens, and the
    write and read sets of some tokens overlapping (one token has them equal)."""
    rng = np.random.default_rng(seed)
    R, W, N = cfg.B * cfg.T * cfg.H, cfg.W, cfg.N
    idx_w = np.stack([rng.permutation(N)[:W] for _ in range(R)]).astype(np.int32)
    idx_r = np.stack([rng.permutation(N)[:W] for _ in range(R)]).astype(np.int32)
    idx_r[R // 2] = idx_w[R // 2][::-1]
    x = {
        "idx_w": idx_w, "idx_r": idx_r,
        "wt_w": _grid(rng.uniform(0.05, 0.5, (R, W))), "wt_r": _grid(rng.uniform(0.05, 0.5, (R, W))),
        "v": _grid(rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.d))),
        "alpha": _grid(rng.uniform(0.5, 1.0, (cfg.B, cfg.T, cfg.H)) if alpha is None
                       else np.full((cfg.B, cfg.T, cfg.H), alpha)),
        "beta": _grid(rng.uniform(0.1, 0.9, (cfg.B, cfg.T, cfg.H)) if beta is None
                      else np.full((cfg.B, cfg.T, cfg.H), beta)),
        "mem0": rng.standard_normal((cfg.B, cfg.H, N, cfg.d)),
        "dout": _grid(rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.d))),
        "dmem": rng.standard_normal((cfg.B, cfg.H, N, cfg.d)),
    }
    return x


def _loss(g, cfg, x):
    """L = sum_t <dout_t, out_t> + <dmem, M_T>, with out_t formed in double from the float64
    memory after each token's write (one-token calls of the forward oracle's scan)."""
    one = cfg.replace(B=1, H=1, T=1)
    L = 0.0
    for b in range(cfg.B):
        for h in range(cfg.H):
            mem = np.array(x["mem0"][b, h][None, None], np.float64, copy=True, order="C")
            for t in range(cfg.T):
                r = (b * cfg.T + t) * cfg.H + h
                g.scan_forward(one, x["idx_w"][r:r + 1], x["wt_w"][r:r + 1], x["idx_r"][r:r + 1],
                               x["wt_r"][r:r + 1], x["v"][b, t, h][None, None, None],
                               x["alpha"][b, t, h].reshape(1, 1, 1), x["beta"][b, t, h].reshape(1, 1, 1), mem)
                out = (x["wt_r"][r].astype(np.float64)[:, None] * mem[0, 0, x["idx_r"][r]]).sum(0)
                L += float(np.dot(x["dout"][b, t, h].astype(np.float64), out))
            L += float(np.sum(x["dmem"][b, h] * mem[0, 0]))
    return L


def _richardson(f, x0, h1=H1, h2=H2):
    d1 = (f(x0 + h1) - f(x0 - h1)) / (2 * h1)
    d2 = (f(x0 + h2) - f(x0 - h2)) / (2 * h2)
    return (4 * d2 - d1) / 3


def _scan_grad(g, cfg, x):
    return g.scan_grad(cfg, x["idx_w"], x["wt_w"], x["idx_r"], x["wt_r"], x["v"], x["alpha"], x["beta"],
                       x["mem0"], x["dout"], x["dmem"])


def _check_fd(g, cfg, x, name, grad, picks, tol):
    for pos in picks:
        def f(val, pos=pos):
            y = dict(x)
            y[name] = x[name].copy()
            y[name][pos] = val
            return _loss(g, cfg, y)

        fd = _richardson(f, float(x[name][pos]))
        got = float(grad[pos])
        assert abs(fd - got) <= tol * (1.0 + abs(fd)), f"d/d{name}{pos}: finite differences {fd!r}, gradient {got!r}"


def pin_scan_grad_finite_differences(g):
    cfg = _cfg()
    x = scan_inputs(cfg, 11)
    gr = _scan_grad(g, cfg, x)
    rng = np.random.default_rng(5)
    R = cfg.B * cfg.T * cfg.H

    def picks(shape, n):
        return [tuple(int(rng.integers(0, s)) for s in shape) for _ in range(n)]

    _check_fd(g, cfg, x, "v", gr["dv"], picks(x["v"].shape, 6), 1e-8)
    _check_fd(g, cfg, x, "alpha", gr["dalpha"], picks(x["alpha"].shape, 6), 1e-7)
    _check_fd(g, cfg, x, "beta", gr["dbeta"], picks(x["beta"].shape, 6), 1e-7)
    _check_fd(g, cfg, x, "wt_w", gr["dwt_w"], picks((R, cfg.W), 6), 1e-7)
    _check_fd(g, cfg, x, "wt_r", gr["dwt_r"], picks((R, cfg.W), 6), 1e-7)
    # the memory before the forward: touched slots (written, read) and one never touched
    _check_fd(g, cfg, x, "mem0", gr["dmem0"], picks(x["mem0"].shape, 8), 1e-8)


def pin_scan_grad_read_write_overlap(g):
    """Every token reads exactly the slots it writes (reversed order): the read gradient must
    flow into the write of the same token."""
    cfg = _cfg(B=1, H=1, T=6)
    x = scan_inputs(cfg, 23)
    x["idx_r"] = np.ascontiguousarray(x["idx_w"][:, ::-1])
    gr = _scan_grad(g, cfg, x)
    rng = np.random.default_rng(9)
    _check_fd(g, cfg, x, "v", gr["dv"], [tuple(int(rng.integers(0, s)) for s in x["v"].shape) for _ in range(4)],
              1e-8)
    _check_fd(g, cfg, x, "mem0", gr["dmem0"],
              [(0, 0, int(x["idx_w"][0, i]), 1) for i in range(cfg.W)], 1e-8)


def pin_scan_grad_frozen_memory(g):
    """Decay 1 and step size 0: the write stores x_i = M[n_i] unchanged, so M stays M0 and
      dr_j(t)  = <dout_t, M0[m_j]>,   dM0 = dM_T + sum_t sum_j r_j dout_t e_{m_j},
      dw = 0,  dv = 0,  dalpha(t) = sum_i <G_t[n_i], M0[n_i]>,
      dbeta(t) = <sum_i w_i G_t[n_i], v_t - sum_i w_i M0[n_i]>,
    with G_t = dM_T + (read terms of tokens t..T-1), written out here per memory."""
    cfg = _cfg(state_bf16=0)
    x = scan_inputs(cfg, 31, alpha=1.0, beta=0.0)
    x["mem0"] = _grid(x["mem0"])  # exactly representable in the float32 state
    gr = _scan_grad(g, cfg, x)
    W = cfg.W
    for b in range(cfg.B):
        for h in range(cfg.H):
            M0 = x["mem0"][b, h].astype(np.float64)
            G = x["dmem"][b, h].copy()
            for t in reversed(range(cfg.T)):
                r = (b * cfg.T + t) * cfg.H + h
                n, m = x["idx_w"][r], x["idx_r"][r]
                w, rw = x["wt_w"][r].astype(np.float64), x["wt_r"][r].astype(np.float64)
                go = x["dout"][b, t, h].astype(np.float64)
                np.testing.assert_allclose(gr["dwt_r"][r], M0[m] @ go, rtol=1e-12, atol=1e-12)
                for j in range(W):
                    G[m[j]] += rw[j] * go
                assert np.all(gr["dwt_w"][r] == 0.0) and np.all(gr["dv"][b, t, h] == 0.0)
                np.testing.assert_allclose(gr["dalpha"][b, t, h], np.sum(G[n] * M0[n]), rtol=1e-12, atol=1e-12)
                v = x["v"][b, t, h].astype(np.float64)
                np.testing.assert_allclose(gr["dbeta"][b, t, h], np.dot(w @ G[n], v - w @ M0[n]), rtol=1e-12,
                                           atol=1e-12)
            np.testing.assert_allclose(gr["dmem0"][b, h], G, rtol=1e-12, atol=1e-12)


def _address_case(seed, **kw):
    cfg = _cfg(**{**dict(B=1, H=2, T=5, S=8, dk=8, k=4, W=6, state_bf16=0), **kw})
    rng = np.random.default_rng(seed)
    q = _grid(rng.standard_normal((cfg.B, cfg.T, cfg.H, cfg.dk)))
    sub = _grid(rng.standard_normal((cfg.H, 2, cfg.S, cfg.dk // 2)) * 0.5)
    return cfg, q, sub, rng


def pin_weights_f64_match_forward(g, o):
    """The double weight function gives the forward oracle's weights for its own selection."""
    cfg, q, sub, _ = _address_case(41)
    idx, wt, _ = o.address(cfg, q, sub)
    for r in range(cfg.B * cfg.T * cfg.H):
        w = g.weights_f64(cfg, q.reshape(-1, cfg.dk)[r], sub, r % cfg.H, idx[r])
        np.testing.assert_allclose(w, wt[r], rtol=0, atol=2e-7)


def pin_address_grad_finite_differences(g, o):
    cfg, q, sub, rng = _address_case(43)
    idx, wt, sigma = o.address(cfg, q, sub)
    R = cfg.B * cfg.T * cfg.H
    dwt = rng.standard_normal((R, cfg.W))
    dq, dsub = g.address_grad(cfg, q, sub, idx, sigma, dwt)
    qf = q.reshape(R, cfg.dk).astype(np.float64)
    sf = sub.astype(np.float64)

    def loss(qq, ss):
        return sum(float(np.dot(dwt[r], g.weights_f64(cfg, qq[r], ss, r % cfg.H, idx[r]))) for r in range(R))

    for r, j in [(0, 0), (3, 5), (7, 7), (9, 2)]:
        def fq(val, r=r, j=j):
            qq = qf.copy()
            qq[r, j] = val
            return loss(qq, sf)

        fd = _richardson(fq, qf[r, j], 1e-3, 5e-4)
        assert abs(fd - dq[r, j]) <= 1e-6 * (1 + abs(fd)), f"dq[{r},{j}]: {fd!r} vs {dq[r, j]!r}"
    # sub-keys that some row selected, in both halves and both heads, and one no row selected
    used = set()
    for r in range(R):
        for n in idx[r]:
            used.add((r % cfg.H, 0, int(n) // cfg.S))
            used.add((r % cfg.H, 1, int(n) % cfg.S))
    picks = sorted(used)[::3][:6]
    unused = [(h, half, s) for h in range(cfg.H) for half in range(2) for s in range(cfg.S)
              if (h, half, s) not in used][:1]
    for (h, half, s) in picks + unused:
        for j in (0, cfg.dk // 2 - 1):
            def fs(val, h=h, half=half, s=s, j=j):
                ss = sf.copy()
                ss[h, half, s, j] = val
                return loss(qf, ss)

            fd = _richardson(fs, sf[h, half, s, j], 1e-3, 5e-4)
            got = dsub[h, half, s, j]
            assert abs(fd - got) <= 1e-6 * (1 + abs(fd)), f"dsub[{h},{half},{s},{j}]: {fd!r} vs {got!r}"


def pin_address_grad_one_slot(g, o):
    """One selected slot: its softmax weight is 1 whatever the query, so no gradient."""
    cfg, q, sub, rng = _address_case(47, k=1, W=1)
    idx, wt, sigma = o.address(cfg, q, sub)
    dq, dsub = g.address_grad(cfg, q, sub, idx, sigma, rng.standard_normal((cfg.B * cfg.T * cfg.H, 1)))
    assert np.all(dq == 0.0) and np.all(dsub == 0.0)


def pin_address_grad_uniform_upstream(g, o):
    """The same upstream value on every weight: the weights sum to 1, so the gradient is 0
    (up to rounding of the mean)."""
    cfg, q, sub, _ = _address_case(53)
    idx, wt, sigma = o.address(cfg, q, sub)
    dq, dsub = g.address_grad(cfg, q, sub, idx, sigma, np.full((cfg.B * cfg.T * cfg.H, cfg.W), 0.75))
    assert np.max(np.abs(dq)) < 1e-13 and np.max(np.abs(dsub)) < 1e-13


SCAN_PINS = [pin_scan_grad_finite_differences, pin_scan_grad_read_write_overlap, pin_scan_grad_frozen_memory]
ADDRESS_PINS = [pin_weights_f64_match_forward, pin_address_grad_finite_differences, pin_address_grad_one_slot,
                pin_address_grad_uniform_upstream]
