"""The fused scoring's threshold on the workloads' inputs (host arithmetic, no GPU).

pk_score_cand marks the sub-keys whose float32 score reaches
tau = <q, mu> + z sigma |q| (mu the table's mean row, sigma its root mean square
deviation, z the normal quantile leaving (k + 64) / 2 of S above it), and the
selection rescores the whole half when fewer than k or more than 64 pass.  The
result never depends on tau; its cost does.  This checks that on the 1.4B-shaped
and 8B-shaped workloads (iid and Gaussian-mixture queries) the whole-half path
stays rare.
"""
import numpy as np
import pytest
from scipy.stats import norm

import sdm_inputs as gi


def _fallback_rate(cfg):
    x = gi.make_inputs(cfg, with_mem0=False)
    K = gi.f32_from_bf16_bits(x["subkeys"]).reshape(cfg.H, 2, cfg.S, cfg.dh).astype(np.float64)
    z = norm.isf(((cfg.k + 64) // 2) / cfg.S)
    bad = n = 0
    for name in ("wq", "rq"):
        q = gi.f32_from_bf16_bits(x[name]).reshape(-1, 2, cfg.dh).astype(np.float64)
        for hf in range(2):
            tab = K[0, hf]
            mu = tab.mean(0)
            sig = np.sqrt(((tab - mu) ** 2).mean())
            s = q[:, hf] @ tab.T
            tau = q[:, hf] @ mu + z * sig * np.sqrt((q[:, hf] ** 2).sum(1))
            c = (s >= tau[:, None]).sum(1)
            bad += int(((c < cfg.k) | (c > 64)).sum())
            n += c.size
    return bad / n


@pytest.mark.parametrize("ci,T", [(2, 1024), (4, 512)])
def test_whole_half_rescoring_is_rare(ci, T):
    cfg = gi.config(ci).replace(B=1, T=T)
    rate = _fallback_rate(cfg)
    print(f"[{cfg.name}] halves rescored whole: {rate:.4%}")
    assert rate < 0.01
