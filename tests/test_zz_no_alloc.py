"""sdm_step_static, the decode step that allocates nothing, through the C ABI.

It must equal sdm_step (on a handle) bit for bit.  Two calls in a row, the
second with a smaller input, show that the per-device scratch it keeps its slot
ids and weights in carries nothing from one call to the next; both the
two-launch path (float32 queries: the scratch is used) and the one-launch path
(bf16 queries of the workload widths: LDS only) are covered.
"""
import ctypes as C
import sys

import numpy as np
import pytest

import sdm_inputs as gi
from parity import to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _edge(**kw):
    base = dict(name="noalloc", B=4, H=2, T=3, d=64, S=32, dk=32, k=6, W=16, in_bf16=False, state_bf16=False,
                alpha_shift=2.0, m0_std=0.5, subkey_std=0.25)
    base.update(kw)
    return gi.Config(**base)


def _cconfig(cfg):
    from sparse_memory_linear_pk_amd._lib import SDM_BF16, SDM_F32, Config
    return Config(cfg.B, cfg.H, 1, cfg.d, cfg.S, cfg.dk, cfg.k, cfg.W, SDM_BF16 if cfg.in_bf16 else SDM_F32,
                  SDM_BF16 if cfg.state_bf16 else SDM_F32, 0)


def _steps_both_ways(cfg, seed):
    """cfg.T tokens through sdm_step on a handle and through sdm_step_static; returns
    (outputs, memories) of both."""
    import torch
    from sparse_memory_linear_pk_amd import SDM
    from sparse_memory_linear_pk_amd._lib import check, lib
    x = gi.make_inputs(cfg, seed=seed)
    dev = {k: to_dev(v) for k, v in x.items()}
    L = lib()
    stream = torch.cuda.current_stream()
    ccfg = _cconfig(cfg)
    mem_h, mem_s = dev["mem0"].clone(), dev["mem0"].clone()
    outs_h, outs_s = [], []
    with SDM.from_config(cfg, T=1, stream=stream) as layer:
        for t in range(cfg.T):
            tok = {k: dev[k][:, t].contiguous() for k in ("wq", "rq", "v", "alpha", "beta")}
            o_h = torch.empty((cfg.B, cfg.H, cfg.d), dtype=torch.float32, device="cuda")
            o_s = torch.full_like(o_h, float("nan"))
            layer.step(tok["wq"], tok["rq"], tok["v"], tok["alpha"], tok["beta"], dev["subkeys"], mem_h, o_h)
            args = [tok["wq"], tok["rq"], tok["v"], tok["alpha"], tok["beta"], dev["subkeys"], mem_s, o_s]
            check(L.sdm_step_static(C.byref(ccfg), C.c_void_p(stream.cuda_stream),
                                    *[C.c_void_p(a.data_ptr()) for a in args]), "sdm_step_static")
            outs_h.append(o_h)
            outs_s.append(o_s)
        torch.cuda.synchronize()
    return outs_h, outs_s, mem_h, mem_s


@pytest.mark.parametrize("path,first,second", [
    # float32 queries: two launches, slot ids and weights through the scratch; the second
    # call is smaller (fewer memories, narrower selection)
    ("two_launch", _edge(B=4, H=2, W=16), _edge(B=2, H=1, W=8, k=4, S=24)),
    # bf16 queries with 128-wide halves and S > 256 (the workload widths): one launch
    ("one_launch", _edge(B=2, H=1, d=64, S=260, dk=256, k=8, W=32, in_bf16=True, state_bf16=True),
     _edge(B=1, H=1, d=64, S=260, dk=256, k=8, W=16, in_bf16=True, state_bf16=True)),
])
def test_step_static_equals_step(path, first, second):
    import torch
    for i, cfg in enumerate((first, second)):
        say(f"[no-alloc {path}] call {i}: {cfg}")
        oh, os_, mh, ms = _steps_both_ways(cfg, seed=10 + i)
        for t, (a, b) in enumerate(zip(oh, os_)):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{path} call {i} token {t}: outputs differ"
        ity = torch.int16 if cfg.state_bf16 else torch.int32
        assert torch.equal(mh.view(ity), ms.view(ity)), f"{path} call {i}: memories differ"


def test_step_static_rejects_a_selection_past_its_scratch():
    from sparse_memory_linear_pk_amd._lib import SDM_ERR_UNSUPPORTED, lib
    import torch
    cfg = _edge(B=1025, H=1, W=64, k=8)
    z = torch.zeros(16, dtype=torch.float32, device="cuda")
    L = lib()
    rc = L.sdm_step_static(C.byref(_cconfig(cfg)), None, *([C.c_void_p(z.data_ptr())] * 8))
    assert rc == SDM_ERR_UNSUPPORTED and b"scratch" in L.sdm_last_error()
