"""Staged comparison of the HIP path against the oracle.

Addressing never reads the memory, so parity splits into exact stages:
  1. scores: GPU half scores against the oracle's (double accumulation, one
     rounding), within the float32 accumulation error bound of a dh-term dot;
  2. selection: the GPU selection of the GPU's own scores against the oracle's
     selection of those same scores: indices bit-exact, weights within 1 ulp;
  3. the forward's addressing (sdm_address: the float32 scores locate the
     candidates, the scores that can reach a top k are recomputed exactly)
     against the oracle's addressing of the same queries: the same slots and
     weights within one float32 unit, on every row.  The selection from the
     float32 scores alone is also compared with the oracle's as sets: a slot in
     the symmetric difference is allowed only where the oracle's scores leave
     the choice open (a gap < 1e-5 at the per-half k-th or the W-th boundary);
  4. scan: the oracle's scan driven by the forward's indices and weights
     against the GPU's out and final memory: max |got - ref| / RMS(ref) <= tol,
     each tensor with its own RMS, tol = 1e-4 (float32 state) or 2e-2 (bf16);
  5. end-to-end: the GPU forward against the oracle's forward (its own
     addressing), the same figure.  Stage 3 makes the addressing the same, so
     stages 4 and 5 differ only in rounding of the scan arithmetic; without it,
     float32 scores against double ones change the weights in their last bits
     and a bf16 state's roundings drift apart over a long sequence (the oracle
     against itself with float32-rounded scores: 0.029 of the RMS per element on
     the 8B-shaped layer's outputs at T = 16,384).
"""
from __future__ import annotations

import numpy as np

from sdm_inputs import f32_from_bf16_bits

F32 = np.float32
GAP = 1e-5          # score gap under which a selection boundary is a tie
TOL_F32_STATE = 1e-4
TOL_BF16_STATE = 2e-2


def torch():
    import torch as _t
    return _t


def to_dev(a: np.ndarray):
    t = torch()
    if a.dtype == np.uint16:
        return t.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(t.bfloat16)
    return t.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(x) -> np.ndarray:
    t = torch()
    if x.dtype == t.bfloat16:
        return x.contiguous().cpu().view(t.int16).numpy().view(np.uint16)
    return x.contiguous().cpu().numpy()


def as_f32(a: np.ndarray) -> np.ndarray:
    return f32_from_bf16_bits(a).reshape(a.shape) if a.dtype == np.uint16 else a.astype(F32)


# ---------------------------------------------------------------------------
# stage 1
# ---------------------------------------------------------------------------

def score_error_bound(cfg, q: np.ndarray, subkeys: np.ndarray, rows) -> np.ndarray:
    """Per-score bound on float32 accumulation error of dh products:
    1.01 * dh * 2^-24 * sum |q_c k_c|  plus one rounding of the result."""
    qf = np.abs(as_f32(q).reshape(-1, cfg.dk).astype(np.float64))
    kf = np.abs(as_f32(subkeys).astype(np.float64))
    rows = np.asarray(rows, np.int64)
    out = np.empty((rows.size, 2, cfg.S))
    heads = rows % cfg.H
    for h in range(cfg.H):
        sel = np.nonzero(heads == h)[0]
        for half in range(2):
            out[sel, half] = qf[rows[sel], half * cfg.dh:(half + 1) * cfg.dh] @ kf[h, half].T
    return 1.01 * cfg.dh * 2.0 ** -24 * out


def check_scores(cfg, got, ref, bound):
    err = np.abs(got.astype(np.float64) - ref.astype(np.float64))
    lim = bound + np.abs(ref) * 2.0 ** -24 + 1e-30
    bad = err > lim
    assert not bad.any(), f"{bad.sum()} scores outside the accumulation bound; worst {err.max():.3g}"
    return float(err.max())


# ---------------------------------------------------------------------------
# stage 2
# ---------------------------------------------------------------------------

def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    ia = a.astype(F32).view(np.int32).astype(np.int64)
    ib = b.astype(F32).view(np.int32).astype(np.int64)
    return np.abs(ia - ib)


def check_selection_exact(gpu_idx, gpu_wt, ref_idx, ref_wt):
    mism = np.nonzero((gpu_idx != ref_idx).any(axis=1))[0]
    assert mism.size == 0, f"{mism.size} rows select differently from the same scores, first row {mism[:5]}"
    u = ulp_diff(gpu_wt, ref_wt)
    assert u.max() <= 1, f"weights differ by {u.max()} ulp"
    return int(u.max())


# ---------------------------------------------------------------------------
# stage 3
# ---------------------------------------------------------------------------

def _desc_order(vals):
    return np.lexsort((np.arange(vals.size), -vals))


def compare_index_sets(o, cfg, gpu_idx, ref_idx, ref_sig, ref_scores, rows=None):
    """Returns (rows differing, rows excused).  Raises on an unexcused difference."""
    S, k, W = cfg.S, cfg.k, cfg.W
    R = gpu_idx.shape[0]
    rows = np.arange(R) if rows is None else np.asarray(rows)
    differ = excused = 0
    same = np.all(np.sort(gpu_idx, axis=1) == np.sort(ref_idx, axis=1), axis=1)
    for j in np.nonzero(~same)[0]:
        g = set(gpu_idx[j].tolist())
        r = set(ref_idx[j].tolist())
        if g == r:
            continue
        differ += 1
        s1, s2 = ref_scores[j, 0], ref_scores[j, 1]
        o1, o2 = _desc_order(s1), _desc_order(s2)
        band1 = _band(s1[o1], k)
        band2 = _band(s2[o2], k)
        if W < k * k:
            n_next, sig_next = o.select(s1, s2, k, W + 1)
            sig_w, sig_w1 = float(sig_next[W - 1]), float(sig_next[W])
        else:
            sig_w, sig_w1 = float(ref_sig[j, W - 1]), -np.inf
        for n in g ^ r:
            a, b = divmod(n, S)
            sig = float(F32(s1[a]) + F32(s2[b]))
            ok = (band1 is not None and band1[0] <= s1[a] <= band1[1]) or \
                 (band2 is not None and band2[0] <= s2[b] <= band2[1]) or \
                 (sig_w - sig_w1 <= GAP and sig_w1 - GAP <= sig <= sig_w + GAP)
            if not ok:
                raise AssertionError(
                    f"row {rows[j]}: slot {n} (sum {sig:.7g}) differs and no boundary is within {GAP}: "
                    f"W-th {sig_w:.7g}, (W+1)-th {sig_w1:.7g}")
        excused += 1
    return differ, excused


def _band(sorted_vals, k):
    """Score band around the k-th / (k+1)-th boundary, or None when the gap is wide."""
    if k >= sorted_vals.size:
        return None
    hi, lo = float(sorted_vals[k - 1]), float(sorted_vals[k])
    if hi - lo > GAP:
        return None
    return lo - GAP, hi + GAP


# ---------------------------------------------------------------------------
# stage 4
# ---------------------------------------------------------------------------

def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max_e |got - ref| / max(|ref_e|, RMS(ref)): each element's error relative
    to its own magnitude, with the tensor's RMS as the floor (printed beside the
    plain figure)."""
    got = as_f32(got).astype(np.float64)
    ref = as_f32(ref).astype(np.float64)
    rms = max(np.sqrt(np.mean(ref ** 2)), 1e-30)
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), rms)))


def rms_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    """The plain figure: max |got - ref| / RMS(ref)."""
    got = as_f32(got).astype(np.float64)
    ref = as_f32(ref).astype(np.float64)
    return float(np.max(np.abs(got - ref)) / max(np.sqrt(np.mean(ref ** 2)), 1e-30))


plain_err = rms_max_err


class PlainAccum:
    """max |got - ref| / RMS(ref) over a tensor compared in parts (sequence by
    sequence): the largest difference and the sum of squares of ref are
    accumulated, so the figure is that of the whole tensor."""

    def __init__(self):
        self.maxabs, self.sumsq, self.n = 0.0, 0.0, 0
        self.rel = 0.0  # per-element figure of the parts (RMS floor per part)

    def add(self, got: np.ndarray, ref: np.ndarray, block: int = 1 << 24):
        """Adds one part, in flat blocks of `block` elements (a full-size memory is billions of them)."""
        g, r = got.reshape(-1), ref.reshape(-1)
        n = r.size
        rms_part = np.sqrt(sum(float(np.sum(as_f32(r[i:i + block]).astype(np.float64) ** 2))
                               for i in range(0, n, block)) / max(n, 1))
        rms_part = max(rms_part, 1e-30)
        for i in range(0, n, block):
            gb = as_f32(g[i:i + block]).astype(np.float64)
            rb = as_f32(r[i:i + block]).astype(np.float64)
            diff = np.abs(gb - rb)
            self.maxabs = max(self.maxabs, float(diff.max()))
            self.sumsq += float(np.sum(rb * rb))
            self.rel = max(self.rel, float(np.max(diff / np.maximum(np.abs(rb), rms_part))))
        self.n += n

    def value(self) -> float:
        return self.maxabs / max(np.sqrt(self.sumsq / max(self.n, 1)), 1e-30)


def scan_tol(cfg) -> float:
    return TOL_BF16_STATE if cfg.state_bf16 else TOL_F32_STATE


def check_scan(cfg, stage: int, label: str, errs: dict, say=print):
    """errs: tensor name -> (plain figure, per-element figure).  Asserts the plain
    figure max |got - ref| / RMS(ref) and prints both."""
    tol = scan_tol(cfg)
    say(f"[{label}] stage {stage}: " + ", ".join(f"{k} max/RMS {p:.3g} (per element {e:.3g})"
                                                for k, (p, e) in errs.items()) + f"; tol {tol}")
    for k, (p, e) in errs.items():
        assert p <= tol, f"[{label}] stage {stage}: {k} {p:.3g} > {tol}"
