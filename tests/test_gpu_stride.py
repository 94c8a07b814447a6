"""Padded slot rows (sdm_config.mem_stride) through the C ABI.

With rows mem_stride elements apart, every entry point that touches a state
tensor (sdm_forward, sdm_step, sdm_forward_train, sdm_backward,
sdm_broadcast_memory) must give bit for bit the results of the dense layout:
only the addresses change, not one operation.  The padding itself (elements d
and up of each row) is never read or written: it is filled with a byte
pattern first and must hold it afterwards.  The small cases also compare the
padded forward with the oracle (the scan driven by the GPU's own slots, as in
test_gpu_parity.py); the dense path is compared with the oracle at full size
there.
"""
import sys

import pytest

import oracle
import sdm_inputs as gi
from parity import check_scan, plain_err, rel_max_err, to_dev, to_host

pytestmark = pytest.mark.gpu

FILL = 0x5A  # byte pattern of the padding


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def _edge(**kw):
    base = dict(name="stride", B=2, H=2, T=40, d=256, S=16, dk=32, k=4, W=8, in_bf16=False, state_bf16=False,
                alpha_shift=2.0, m0_std=0.5, subkey_std=0.25)
    base.update(kw)
    return gi.Config(**base)


# (config, padded row stride in elements, runs the oracle)
CASES = {
    "f32_staged": (_edge(), 288, True),                                    # 1024-byte rows -> 1152
    # a bf16 state over few 128-byte columns scans in narrower segments: under 64 columns in 32-byte
    # ones, 64 to 127 in 64-byte ones
    "bf16_state_8_columns": (_edge(d=128, in_bf16=True, state_bf16=True), 192, True),
    "bf16_state_64_columns": (_edge(B=1, H=1, T=24, d=4096, in_bf16=True, state_bf16=True), 4160, True),
    "bf16_state_120_columns": (_edge(B=2, H=1, T=24, d=3840, in_bf16=True, state_bf16=True), 3904, True),
    "f32_register_ring": (_edge(d=40, T=24), 44, True),                     # 160-byte rows: not staged
    "1.4B_shape": (gi.config(2, T=24, B=1), 2080, False),                  # 8192-byte rows -> 8320
    "8B_shape_bf16": (gi.config(4, T=16, B=1), 3904, False),               # 7680 -> 7808
    # long enough for the library's chunked forward (several scan launches, addressing on a second stream)
    "f32_chunked_T2600": (_edge(T=2600, B=2, H=1, d=64, S=32, k=6, W=16), 96, True),  # 256-byte rows -> 384
}


def _padded(T, src, ms):
    """A [.., N, ms] tensor of the FILL pattern with src copied into its [..., :d] view; returns the view."""
    full = T.empty((*src.shape[:-1], ms), dtype=src.dtype, device="cuda")
    full.view(T.uint8).fill_(FILL)
    view = full[..., :src.shape[-1]]
    view.copy_(src)
    return view


def _padding_intact(T, view, ms):
    d = view.shape[-1]
    if ms == d:
        return True
    full = T.as_strided(view, (*view.shape[:-1], ms), (*view.stride()[:-1], 1))
    pad = full[..., d:].contiguous().view(T.uint8)
    return bool((pad == FILL).all().item())


def _bits(T, t):
    """A bitwise view of a float32 or bf16 tensor (comparable with torch.equal)."""
    return t.view(T.int32) if t.dtype == T.float32 else t.view(T.int16)


def _steps(cfg):
    """sdm_step and the training pair need whole 128-byte columns."""
    return cfg.d * (2 if cfg.state_bf16 else 4) % 128 == 0


def _trains(cfg, ms):
    """... and the training pair a float32 gradient under 4 GiB per memory."""
    return _steps(cfg) and cfg.S ** 2 * max(ms, cfg.d) * 4 < 2 ** 32


def _digest(T, t):
    """Two sums over a tensor's bit patterns: a later write into it changes them."""
    b = _bits(T, t).to(T.int64) if t.dtype in (T.float32, T.bfloat16) else t.to(T.int64)
    return int(b.sum().item()), float((b.to(T.float64) ** 2).sum().item())


def _run(T, cfg, x, g, ms, m0):
    """Every state entry point with rows ms apart (ms = d: dense).  Returns device tensors (dense views).
    Each result is fingerprinted when it is produced and checked again at the end, so that a later
    call writing outside its own tensors is caught."""
    from sparse_memory_linear_pk_amd import SDM
    dev = {k: to_dev(v) for k, v in x.items()}
    f32 = dict(dtype=T.float32, device="cuda")
    res, intact = {}, []
    with SDM.from_config(cfg, mem_stride=0 if ms == cfg.d else ms) as layer:
        mem = _padded(T, dev["mem0"], ms)
        out = T.empty((cfg.B, cfg.T, cfg.H, cfg.d), **f32)
        layer.forward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem, out)
        res["mem"], res["out"] = mem, out
        fp = {k: _digest(T, res[k]) for k in ("mem", "out")}
        intact.append(_padding_intact(T, mem, ms))
        if _steps(cfg):
            mem_s = _padded(T, dev["mem0"], ms)
            out_s = T.empty_like(out)
            o = T.empty((cfg.B, cfg.H, cfg.d), **f32)
            for t in range(cfg.T):
                tok = {k: dev[k][:, t].contiguous() for k in ("wq", "rq", "v", "alpha", "beta")}
                layer.step(tok["wq"], tok["rq"], tok["v"], tok["alpha"], tok["beta"], dev["subkeys"], mem_s, o)
                out_s[:, t] = o
            res["mem_step"], res["out_step"] = mem_s, out_s
            fp.update({k: _digest(T, res[k]) for k in ("mem_step", "out_step")})
            intact.append(_padding_intact(T, mem_s, ms))
            # T steps equal the T-token forward bit for bit; where not, name the first token that differs
            same = (_bits(T, out_s) == _bits(T, out)).reshape(cfg.B, cfg.T, cfg.H, cfg.d).all(dim=-1)
            bad = [(b, h, int((~same[b, :, h]).nonzero()[0])) for b in range(cfg.B) for h in range(cfg.H)
                   if not bool(same[b, :, h].all())]
            say(f"[stride ms={ms}] steps against the forward: first differing token per (b, h): {bad or 'none'}")
            assert not bad, f"ms={ms}: the decode steps differ from the forward at (b, h, t) {bad}"
        if g:
            mem_t = _padded(T, dev["mem0"], ms)
            out_t = T.empty_like(out)
            log = T.empty((cfg.B, cfg.H, cfg.T, cfg.W, cfg.d), dtype=mem.dtype, device="cuda")
            layer.forward_train(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem_t,
                                out_t, log)
            res["mem_train"], res["out_train"], res["log"] = mem_t.clone(), out_t, log
            fp.update({k: _digest(T, res[k]) for k in ("mem_train", "out_train", "log")})
            gd = {k: to_dev(v) for k, v in g.items()}
            dm = _padded(T, gd["dmem"], ms)
            outs = {"dwq": T.empty((cfg.B, cfg.T, cfg.H, cfg.dk), **f32),
                    "drq": T.empty((cfg.B, cfg.T, cfg.H, cfg.dk), **f32),
                    "dv": T.empty((cfg.B, cfg.T, cfg.H, cfg.d), **f32),
                    "dalpha": T.empty((cfg.B, cfg.T, cfg.H), **f32),
                    "dbeta": T.empty((cfg.B, cfg.T, cfg.H), **f32),
                    "dsub": T.empty((cfg.H, 2, cfg.S, cfg.dk // 2), **f32)}
            layer.backward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem_t, log,
                           gd["dout"], dm, outs["dwq"], outs["drq"], outs["dv"], outs["dalpha"], outs["dbeta"],
                           outs["dsub"])
            res.update(outs)
            res["mem_restored"], res["dmem0"] = mem_t, dm
            fp.update({k: _digest(T, res[k]) for k in list(outs) + ["mem_restored", "dmem0"]})
            intact += [_padding_intact(T, mem_t, ms), _padding_intact(T, dm, ms)]
        src = _padded(T, m0, ms)
        dst = _padded(T, T.zeros((cfg.B, *m0.shape), dtype=m0.dtype, device="cuda"), ms)
        layer.broadcast_memory(src, dst)
        res["broadcast"] = dst
        fp["broadcast"] = _digest(T, dst)
        intact.append(_padding_intact(T, dst, ms))
        if ms != cfg.d:
            R = cfg.B * cfg.T * cfg.H
            for s_, q in (("w", "wq"), ("r", "rq")):
                idx = T.empty((R, cfg.W), dtype=T.int32, device="cuda")
                wt = T.empty((R, cfg.W), **f32)
                layer.address(dev[q], dev["subkeys"], idx, wt)
                res["idx_" + s_], res["wt_" + s_] = idx, wt
        T.cuda.synchronize()
        changed = [k for k in res if k in fp and _digest(T, res[k]) != fp[k]]
        say(f"[stride ms={ms}] results changed after they were produced: {changed or 'none'}")
        assert not changed, f"ms={ms}: later calls wrote into {changed}"
    return res, intact


@pytest.mark.parametrize("name", list(CASES))
def test_padded_rows_equal_dense_rows_bitwise(name):
    import torch as T
    cfg, ms, with_oracle = CASES[name]
    say(f"[stride {name}] ms={ms} {cfg}")
    x = gi.make_inputs(cfg)
    g = gi.make_upstream_grads(cfg) if _trains(cfg, ms) else {}
    m0 = to_dev(x["mem0"][0])  # a learned initial memory stand-in [H, N, d]
    dense, ok_dense = _run(T, cfg, x, g, cfg.d, m0)
    padded, ok = _run(T, cfg, x, g, ms, m0)
    assert all(ok), f"padding written: {ok}"
    for k in dense:
        assert T.equal(_bits(T, padded[k]), _bits(T, dense[k])), f"{k} differs between padded and dense rows"
    if "out_step" in padded:  # and the decode steps are the forward's, as with dense rows
        assert T.equal(_bits(T, padded["out_step"]), _bits(T, padded["out"]))
        assert T.equal(_bits(T, padded["mem_step"]), _bits(T, padded["mem"]))
    assert T.equal(_bits(T, padded["broadcast"][-1]), _bits(T, m0))
    say(f"[stride {name}] {len(dense)} tensors bitwise equal, padding intact")
    if with_oracle:
        orc = oracle.get()
        h = {k: to_host(padded[k]) for k in ("idx_w", "wt_w", "idx_r", "wt_r", "out", "mem")}
        mem = x["mem0"].copy()
        out = orc.scan(cfg, h["idx_w"], h["wt_w"], h["idx_r"], h["wt_r"], x["v"], x["alpha"], x["beta"], mem)
        check_scan(cfg, 4, f"stride {name}", {"out": (plain_err(h["out"], out), rel_max_err(h["out"], out)),
                                               "mem": (plain_err(h["mem"], mem), rel_max_err(h["mem"], mem))}, say)


def test_dense_view_of_a_padded_tensor_is_required():
    """A contiguous [B, H, N, d] memory is refused by a layer configured for padded rows, and a padded view by
    a dense one: the binding checks the strides before calling the library."""
    import torch as T
    from sparse_memory_linear_pk_amd import SDM
    cfg = _edge(T=4)
    x = gi.make_inputs(cfg)
    dev = {k: to_dev(v) for k, v in x.items()}
    out = T.empty((cfg.B, cfg.T, cfg.H, cfg.d), dtype=T.float32, device="cuda")
    args = (dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"])
    with SDM.from_config(cfg, mem_stride=288) as layer:
        with pytest.raises(ValueError, match="view of a contiguous"):
            layer.forward(*args, dev["mem0"].clone(), out)
        mem = layer.empty_state(cfg.B, cfg.H)
        assert mem.shape == (cfg.B, cfg.H, cfg.S ** 2, cfg.d) and mem.stride()[-2] == 288
    with SDM.from_config(cfg) as layer:
        with pytest.raises(ValueError, match="contiguous"):
            layer.forward(*args, _padded(T, dev["mem0"], 288), out)
