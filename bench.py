"""Benchmark of the SDM layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one sdm_forward over the whole batch of the 1.4B-shaped layer
(B=4 sequences, T=8192 tokens, H=1, slot width d=2048, N=480^2 slots, query
width 256, k=32, W=64; bf16 queries, values and sub-keys; float32 state and
arithmetic).  The memory carries over from step to step, as consecutive chunks
of a long sequence would.  Inputs are seeded synthetic data already resident in
HBM when the timed region starts.  Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0           # MI355X HBM3E, published
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
F32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 matrix, published
METRIC = "SDM layer tokens/sec (1 GPU) + achieved HBM GB/s vs roofline, 1.4B shape"
WORKLOAD = 2  # the 1.4B-shaped single layer
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "sdm_scan_1p4b_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def scan_bytes_per_step(cfg) -> int:
    """Algorithmic state bytes of one forward: per token and memory, W slots
    read for the write, W read for the read and W written."""
    s = 2 if cfg.state_bf16 else 4
    return cfg.B * cfg.T * cfg.H * 3 * cfg.W * cfg.d * s


def score_flops_per_step(cfg) -> int:
    """Sub-key scoring of one forward: 2 query sets x 2 halves x S sub-keys x dh
    multiply-adds of 2 FLOP, per row."""
    return cfg.B * cfg.T * cfg.H * 2 * 2 * cfg.S * cfg.dh * 2


def scoring_output(cfg) -> str:
    """What the forward's scoring kernel writes for this shape: with bf16 inputs, S a multiple of 32
    (at least 128, at most 1120), 64- or 128-wide halves and k <= 48 the scoring is fused with the
    exact selection's candidate search and writes one bitmask record per row and half (the rule of
    pk_cand_path in pk_score.hip); other bf16 shapes store binary16 scores, float32 inputs float32."""
    target = (cfg.k + 64) // 2
    rw = (cfg.S // 32 + 1 + 3) & ~3
    if (cfg.in_bf16 and cfg.S % 32 == 0 and cfg.S >= 128 and rw <= 36 and cfg.dh in (64, 128) and cfg.k <= 48
            and 2 * target <= cfg.S):
        return f"candidate bitmasks ({rw * 4} bytes per row and half; no scores leave the CUs)"
    return "binary16" if cfg.in_bf16 else "float32"


def cpu_baseline(cfg, x, budget_s: float):
    """The oracle, untouched, on a bounded sample of the same workload: whole
    sequences (all T tokens, full slot width, all N slots), as many of the B as
    fit the time budget, at least the first."""
    import numpy as np

    import oracle
    o = oracle.get()
    threads = oracle.default_threads()

    def run(nb, tn, nthreads):
        c = cfg.replace(B=nb, T=tn)
        sl = {k: np.ascontiguousarray(x[k][:nb, :tn]) for k in ("wq", "rq", "v", "alpha", "beta")}
        mem = np.ascontiguousarray(x["mem0"][:nb])
        t0 = time.perf_counter()
        o.forward(c, sl["wq"], sl["rq"], sl["v"], sl["alpha"], sl["beta"], x["subkeys"], mem, threads=nthreads)
        return time.perf_counter() - t0

    per_tok = run(1, 256, threads) / 256
    nb = int(max(1, min(cfg.B, budget_s // max(per_tok * cfg.T, 1e-9))))
    tn = cfg.T if nb > 1 or per_tok * cfg.T <= budget_s else int(max(256, budget_s / per_tok))
    dt = run(nb, tn, threads)
    # one thread, on the first tokens of sequence 0 (about a third of the budget)
    per_tok1 = run(1, 128, 1) / 128
    tn1 = int(min(cfg.T, max(128, (budget_s / 3) / per_tok1)))
    dt1 = run(1, tn1, 1)
    visible = len(os.sched_getaffinity(0))
    return {"value": nb * tn / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "host_cpus_visible": visible,
            "threads_note": f"{threads} threads: the oracle driver uses min(16, visible CPUs), 16 being the host "
                            f"CPU share of one GPU on this machine ({visible} visible)",
            "sample": f"sequences 0..{nb - 1} of {cfg.B}, tokens 0..{tn - 1} of {cfg.T}, full d and N "
                      f"({nb * tn} of {cfg.B * cfg.T} tokens); {dt:.1f} s wall with {threads} threads "
                      f"(addressing rows and slot elements split over threads)",
            "single_thread": {"value": tn1 / dt1, "unit": "tokens/s", "cores": 1,
                              "sample": f"sequence 0, tokens 0..{tn1 - 1}, full d and N; {dt1:.1f} s wall"}}


def load_traffic(kernel_signature: str, mem_stride: int):
    """HBM bytes the scan moves per forward, from the committed rocprofv3 counter
    summary, if it was taken on the kernel as it is now and on the same memory
    layout."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_signature") != kernel_signature or t.get("mem_stride") != mem_stride:
        return None
    return t.get("bytes_per_forward")


def state_rows(args, cfg) -> int:
    """Elements from one slot row to the next in the state tensors: the library's
    stride hint (rows padded to an odd number of 128-byte units, which spreads the
    scan's row segments over the memory channels) unless --dense-rows."""
    from sparse_memory_linear_pk_amd import SDM
    return cfg.d if args.dense_rows else SDM.stride_hint(cfg.d, cfg.state_bf16)


def with_rows(t, ms: int):
    """The [..., :d] view of a copy of t whose rows are ms elements apart (t itself
    when ms is its row length)."""
    import torch
    d = t.shape[-1]
    if ms == d:
        return t
    full = torch.empty((*t.shape[:-1], ms), dtype=t.dtype, device=t.device)
    full[..., :d].copy_(t)
    return full[..., :d]


def copy_bandwidth() -> dict:
    """Bytes read plus bytes written per second by plain device copies of 2 GiB between the halves of a
    4 GiB scratch tensor: the runtime's copy (torch copy_) and an elementwise kernel (torch mul by 1 into
    the other half); the faster is the measured stand-in for the HBM peak."""
    import torch
    flat = torch.empty(1 << 30, dtype=torch.float32, device="cuda")
    a, b = flat[:1 << 29], flat[1 << 29:]
    a.fill_(1.0)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn in (("runtime copy", lambda: b.copy_(a)), ("elementwise kernel", lambda: torch.mul(a, 1.0, out=b))):
        fn()
        e0.record()
        for _ in range(5):
            fn()
        e1.record()
        torch.cuda.synchronize()
        res[name] = 5 * 2 * (2 << 30) / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del flat
    best = max(res, key=res.get)
    return {"achieved": res[best], "kernel": best, "all": res}


def rows_note(cfg, ms: int) -> dict:
    s = 2 if cfg.state_bf16 else 4
    return {"stride_elements": ms, "row_bytes": cfg.d * s, "stride_bytes": ms * s,
            "layout": "dense" if ms == cfg.d else "padded (sdm_mem_stride_hint)"}


def kernel_signature() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ("sdm_scan.hip", "sdm_scan_staged.hip", "scan_device.h", "sdm_internal.h"):
        h.update(open(os.path.join(ROOT, "sparse_memory_linear_pk_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def decode_bench(args, cfg):
    """One token per sequence per call over a persistent memory: sdm_step, timed
    over consecutive tokens of the same synthetic sequences, and sdm_forward of
    one token for comparison."""
    import numpy as np
    import torch

    import sdm_inputs as gi
    from sparse_memory_linear_pk_amd import SDM

    steps = max(args.steps, 64)
    c = cfg.replace(T=steps + args.warmup)
    log(f"generating inputs for {c}")
    x = gi.make_inputs(c)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    d = {k: dev(v) for k, v in x.items()}
    ms = state_rows(args, c)
    d["mem0"] = with_rows(d["mem0"], ms)
    tok = [{k: d[k][:, t].contiguous() for k in ("wq", "rq", "v", "alpha", "beta")} for t in range(c.T)]
    out = torch.empty((c.B, c.H, c.d), dtype=torch.float32, device="cuda")
    layer = SDM.from_config(c, mem_stride=ms)
    for t in range(args.warmup):
        layer.step(tok[t]["wq"], tok[t]["rq"], tok[t]["v"], tok[t]["alpha"], tok[t]["beta"], d["subkeys"], d["mem0"], out)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.warmup, c.T):
        layer.step(tok[t]["wq"], tok[t]["rq"], tok[t]["v"], tok[t]["alpha"], tok[t]["beta"], d["subkeys"], d["mem0"], out)
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    # the device time of each step: the same tokens again with HIP events around the launches
    layer.set_timing(True)
    for t in range(args.warmup, c.T):
        layer.step(tok[t]["wq"], tok[t]["rq"], tok[t]["v"], tok[t]["alpha"], tok[t]["beta"], d["subkeys"], d["mem0"], out)
    tm = layer.timing()
    layer.close()
    # the same tokens through a one-token forward
    one = SDM.from_config(c.replace(T=1), mem_stride=ms)
    o1 = torch.empty((c.B, 1, c.H, c.d), dtype=torch.float32, device="cuda")
    x1 = [{k: v.unsqueeze(1) for k, v in tk.items()} for tk in tok]
    for t in range(args.warmup):
        one.forward(x1[t]["wq"], x1[t]["rq"], x1[t]["v"], x1[t]["alpha"], x1[t]["beta"], d["subkeys"], d["mem0"], o1)
    torch.cuda.synchronize()
    f0 = time.perf_counter()
    for t in range(args.warmup, c.T):
        one.forward(x1[t]["wq"], x1[t]["rq"], x1[t]["v"], x1[t]["alpha"], x1[t]["beta"], d["subkeys"], d["mem0"], o1)
    torch.cuda.synchronize()
    fsec = time.perf_counter() - f0
    one.close()
    s_bytes = 2 if c.state_bf16 else 4
    step_bytes = c.B * c.H * 3 * c.W * c.d * s_bytes
    dev_ms = tm["ms_step"] / max(1, tm["n_step"])
    res = {
        "metric": "SDM decode step tokens/sec (1 GPU), sdm_step",
        "value": c.B * steps / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3 / steps,
        "higher_is_better": True,
        "dtype": "f32",
        "data": "synthetic (seeded), consecutive tokens of the workload's sequences",
        "config": {"workload": f"sdm-{c.name} decode: B={c.B} H={c.H} d={c.d} N={c.S}^2 dk={c.dk} k={c.k} W={c.W}, "
                               f"one token per sequence per step", "state_rows": rows_note(c, ms)},
        "step_device_us": dev_ms * 1e3,
        "step_state_bytes": step_bytes,
        "step_device_GBps": step_bytes / (dev_ms * 1e-3) / 1e9,
        "forward_T1_ms_per_step": fsec * 1e3 / steps,
    }
    print(json.dumps(res))


def train_bench(args, cfg):
    """One training step of the layer: sdm_forward_train (the forward, logging every write
    slot's old value), then sdm_backward (the reverse walk, the softmax derivative, query and
    sub-key gradients), with the gradient buffer of the initial memory zeroed first.  The
    backward restores the memory, so every step starts from the same one."""
    import numpy as np
    import torch

    import sdm_inputs as gi
    from sparse_memory_linear_pk_amd import SDM, pattern_probe_mix

    log(f"generating inputs for {cfg}")
    x = gi.make_inputs(cfg)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    d = {k: dev(v) for k, v in x.items()}
    ms = state_rows(args, cfg)
    d["mem0"] = with_rows(d["mem0"], ms)
    f32 = dict(dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda").manual_seed(7)
    dout = torch.randn((cfg.B, cfg.T, cfg.H, cfg.d), generator=gen, **f32)
    out = torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), **f32)
    log_buf = torch.empty((cfg.B, cfg.H, cfg.T, cfg.W, cfg.d),
                          dtype=torch.bfloat16 if cfg.state_bf16 else torch.float32, device="cuda")
    dmem = torch.empty((cfg.B, cfg.H, cfg.N, ms), **f32)[..., :cfg.d]
    g = {"dwq": torch.empty((cfg.B, cfg.T, cfg.H, cfg.dk), **f32), "drq": torch.empty((cfg.B, cfg.T, cfg.H, cfg.dk), **f32),
         "dv": torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), **f32), "dalpha": torch.empty((cfg.B, cfg.T, cfg.H), **f32),
         "dbeta": torch.empty((cfg.B, cfg.T, cfg.H), **f32), "dsub": torch.empty((cfg.H, 2, cfg.S, cfg.dh), **f32)}
    layer = SDM.from_config(cfg, mem_stride=ms)
    mem_check = d["mem0"][0, 0, :4096].clone()

    def step():
        dmem.zero_()
        layer.forward_train(d["wq"], d["rq"], d["v"], d["alpha"], d["beta"], d["subkeys"], d["mem0"], out, log_buf)
        layer.backward(d["wq"], d["rq"], d["v"], d["alpha"], d["beta"], d["subkeys"], d["mem0"], log_buf, dout, dmem,
                       g["dwq"], g["drq"], g["dv"], g["dalpha"], g["dbeta"], g["dsub"])

    steps = max(1, min(args.steps, 10))
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
        log(f"train step {i + 1}/{steps}")
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    # per-kernel device times: the same steps again with HIP events around every launch
    layer.set_timing(True)
    for i in range(steps):
        step()
    tm = layer.timing()
    layer.close()
    if not torch.equal(d["mem0"][0, 0, :4096], mem_check):
        raise RuntimeError("the backward did not restore the memory")
    for k, v in g.items():
        if not torch.isfinite(v).all():
            raise RuntimeError(f"non-finite {k}")
    # the ceiling of the reverse scan's access pattern (float32 state: every segment 128 bytes):
    # 4 reads and 3 writes of random 128-byte segments per slot position and token, same geometry,
    # no arithmetic (scrambles the memory).  A bf16 state mixes 128-byte memory segments with
    # 256-byte gradient segments, which the probe does not model.
    del log_buf
    probe_ms = None
    if not cfg.state_bf16:
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        pattern_probe_mix(d["mem0"], cfg.B * cfg.H, cfg.N, cfg.d * 4, cfg.T, cfg.W, 4, 3, seed=11, row_stride=ms * 4)
        s0.record()
        for r in range(2):
            pattern_probe_mix(d["mem0"], cfg.B * cfg.H, cfg.N, cfg.d * 4, cfg.T, cfg.W, 4, 3, seed=12 + r,
                              row_stride=ms * 4)
        s1.record()
        torch.cuda.synchronize()
        probe_ms = s0.elapsed_time(s1) / 2
    tokens = cfg.B * cfg.T
    s_ = 2 if cfg.state_bf16 else 4
    wd = cfg.W * cfg.d
    # reverse scan per token: reads M and G of the read slots, G and the log of the write slots;
    # writes G of both and the restored M (state s_ bytes, gradient 4 bytes per element)
    bwd_bytes = tokens * cfg.H * wd * (s_ + 4 + 4 + s_ + 4 + 4 + s_)
    fwd_bytes = tokens * cfg.H * wd * s_ * 4  # 2W rows read, W written, W logged
    bwd_ms = tm["ms_bwd_scan"] / max(1, tm["n_bwd_scan"])
    fwd_ms = tm["ms_train"] / steps  # the forward's scan launches (one per chunk)
    res = {
        "metric": "SDM layer training step tokens/sec (1 GPU): sdm_forward_train + sdm_backward",
        "value": tokens * steps / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16 state, f32 gradients" if cfg.state_bf16 else "f32",
        "data": "synthetic (seeded inputs as for the forward; upstream gradient of out ~N(0,1), none of the final memory)",
        "config": {"workload": f"sdm-{cfg.name} layer training step: B={cfg.B} H={cfg.H} T={cfg.T} d={cfg.d} "
                               f"N={cfg.S}^2 dk={cfg.dk} k={cfg.k} W={cfg.W}", "global_batch": cfg.B,
                   "seq_len": cfg.T, "parallelism": "single GPU", "state_rows": rows_note(cfg, ms)},
        "roofline": {"bound": "hbm", "kernel": "grad_scan", "achieved": bwd_bytes / (bwd_ms * 1e-3) / 1e9,
                     "peak": 8000.0, "unit": "GB/s", "frac": bwd_bytes / (bwd_ms * 1e-3) / 1e9 / 8000.0,
                     "traffic": None, "bytes_per_launch": bwd_bytes, "ms_per_launch": bwd_ms,
                     "pattern_ceiling": None if probe_ms is None else {
                         "achieved": bwd_bytes / (probe_ms * 1e-3) / 1e9, "unit": "GB/s",
                         "ms_per_launch": probe_ms, "frac": probe_ms / bwd_ms,
                         "what": "sdm_pattern_probe_mix 4:3: the reverse scan's random 128-byte "
                                 "segment reads and writes with no arithmetic; frac = scan / this"}},
        "kernels_ms_per_step": {"train_scan": fwd_ms, "train_scan_GBps": fwd_bytes / (fwd_ms * 1e-3) / 1e9,
                                "pk_score": tm["ms_score"] / steps, "pk_topk": tm["ms_select"] / steps,
                                "grad_scan": bwd_ms, "grad_rows": tm["ms_bwd_rows"] / steps,
                                "grad_subkeys": tm["ms_bwd_sub"] / steps},
    }
    print(json.dumps(res))


def project_bench(args, cfg):
    """The input projections (sdm_project) of the workload's B*T tokens from a D = d wide embedding:
    one MFMA product [B*T, D] x [D, H*(2dk+d+2)] with the bf16 / sigmoid epilogue."""
    import numpy as np
    import torch

    import sdm_inputs as gi
    from sparse_memory_linear_pk_amd import SDM

    D = cfg.d
    log(f"generating projection inputs for {cfg}, D={D}")
    p = gi.make_projection_inputs(cfg, D)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    d = {k: dev(v) for k, v in p.items()}
    bf = dict(dtype=torch.bfloat16, device="cuda")
    f32 = dict(dtype=torch.float32, device="cuda")
    wq = torch.empty((cfg.B, cfg.T, cfg.H, cfg.dk), **bf)
    rq = torch.empty_like(wq)
    v = torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), **bf)
    al = torch.empty((cfg.B, cfg.T, cfg.H), **f32)
    be = torch.empty_like(al)
    layer = SDM.from_config(cfg)
    for _ in range(max(1, args.warmup)):
        layer.project(D, d["x"], d["w"], d["gate_bias"], wq, rq, v, al, be)
    torch.cuda.synchronize()
    reps = max(args.steps, 10)
    t0 = time.perf_counter()
    for _ in range(reps):
        layer.project(D, d["x"], d["w"], d["gate_bias"], wq, rq, v, al, be)
    torch.cuda.synchronize()
    sec = time.perf_counter() - t0
    # the kernel's device time: the same calls again with HIP events around each launch
    layer.set_timing(True)
    for _ in range(reps):
        layer.project(D, d["x"], d["w"], d["gate_bias"], wq, rq, v, al, be)
    tm = layer.timing()
    layer.close()
    ms = tm["ms_project"] / tm["n_project"]
    C = 2 * cfg.dk + cfg.d + 2
    flops = 2.0 * cfg.B * cfg.T * D * cfg.H * C
    res = {
        "metric": "SDM input projections tokens/sec (1 GPU), sdm_project",
        "value": cfg.B * cfg.T * reps / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3 / reps,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded embedding ~N(0,1), weights ~N(0,1/sqrt(D)))",
        "config": {"workload": f"sdm-{cfg.name} projections: {cfg.B * cfg.T} tokens, D={D} -> H={cfg.H} x "
                               f"(2*{cfg.dk} + {cfg.d} + 2) outputs"},
        "roofline": {"bound": "mfma", "kernel": "project_kernel", "achieved": flops / (ms * 1e-3) / 1e12,
                     "peak": 2500.0, "unit": "TFLOP/s", "frac": flops / (ms * 1e-3) / 1e12 / 2500.0,
                     "traffic": None, "flops_per_launch": flops, "ms_per_launch": ms},
    }
    print(json.dumps(res))


def overlap_bench(args, cfg):
    """The bucket-overlap diagnostic (sdm_overlap) on the long-context needle workload: the call's
    addressing, then the bucket masses (K = S buckets) and the overlap of every token's writes with the
    read of the query token T - 17."""
    import numpy as np
    import torch

    import sdm_inputs as gi
    from sparse_memory_linear_pk_amd import SDM

    if cfg.query != "planted":
        cfg = gi.config(3)
    log(f"generating inputs for {cfg}")
    x = gi.make_inputs(cfg, with_mem0=False)

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    R = cfg.B * cfg.T * cfg.H
    K = cfg.S
    f32 = dict(dtype=torch.float32, device="cuda")
    layer = SDM.from_config(cfg)
    addr = {}
    for s_, q in (("w", "wq"), ("r", "rq")):
        idx = torch.empty((R, cfg.W), dtype=torch.int32, device="cuda")
        wt = torch.empty((R, cfg.W), **f32)
        layer.address(dev(x[q]), dev(x["subkeys"]), idx, wt)
        addr[s_] = (idx, wt)
    wc = torch.empty((cfg.B, cfg.H, cfg.T, K), **f32)
    rd = torch.empty_like(wc)
    qs = torch.tensor([cfg.T - 17], dtype=torch.int32, device="cuda")
    ov = torch.empty((cfg.B, cfg.H, 1, cfg.T), **f32)
    args_ = (addr["w"][0], addr["w"][1], addr["r"][0], addr["r"][1], K, wc, rd, qs, ov)
    layer.overlap(*args_)
    torch.cuda.synchronize()
    reps = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        layer.overlap(*args_)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    curve = ov[0, 0, 0].cpu().numpy()
    layer.close()
    res = {
        "metric": "SDM write/read bucket-overlap diagnostic tokens/sec (1 GPU), sdm_overlap",
        "value": cfg.B * cfg.T / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": reps,
        "warmup": 1,
        "ms_per_step": ms,
        "higher_is_better": True,
        "dtype": "f64 sums",
        "data": "synthetic long-context needle: read query of token T-17 = write query of token 61",
        "config": {"workload": f"sdm-{cfg.name} diagnostic: B={cfg.B} T={cfg.T} N={cfg.S}^2 W={cfg.W}, "
                               f"{K} buckets, query token {cfg.T - 17}"},
        "needle": {"query": cfg.T - 17, "peak_token": int(np.argmax(curve)), "peak": float(curve.max())},
    }
    print(json.dumps(res))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--workload", type=int, default=WORKLOAD,
                    help="workload index (default 2, the 1.4B shape the metric is quoted on; 3 long-context, "
                         "4 8B-shaped: bf16 state)")
    ap.add_argument("--decode", action="store_true",
                    help="time the decode step (sdm_step, one token per sequence per call) instead of the forward")
    ap.add_argument("--overlap", action="store_true",
                    help="time the write/read bucket-overlap diagnostic on the long-context needle workload")
    ap.add_argument("--project", action="store_true",
                    help="time the input projections (sdm_project) instead of the forward")
    ap.add_argument("--train", action="store_true",
                    help="time a training step (sdm_forward_train + sdm_backward) instead of the forward")
    ap.add_argument("--dense-rows", action="store_true",
                    help="keep the memory's slot rows dense (d elements apart) instead of the library's padded "
                         "stride hint")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 4 GiB device copy (for scaling HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sdm_inputs as gi
    from sparse_memory_linear_pk_amd import SDM, pattern_probe_mix

    torch.cuda.set_device(0)
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.float32, device="cuda").fill_(1.0)
        b = torch.empty_like(a)
        for _ in range(5):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each_way": a.numel() * 4, "launches": 5}))
        return

    cfg = gi.config(args.workload)
    if args.decode:
        return decode_bench(args, cfg)
    if args.train:
        return train_bench(args, cfg)
    if args.project:
        return project_bench(args, cfg)
    if args.overlap:
        return overlap_bench(args, cfg)
    log(f"generating inputs for {cfg}")
    t0 = time.perf_counter()
    x = gi.make_inputs(cfg)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s; uploading")

    def dev(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(a).cuda()

    d = {k: dev(v) for k, v in x.items()}
    ms = state_rows(args, cfg)
    dense_mem = d["mem0"]
    d["mem0"] = with_rows(dense_mem, ms)
    if ms == cfg.d:
        dense_mem = None
    else:
        # the benchmarked layout against dense rows, bit for bit, on one forward from the same memory
        # (the full-size parity tests compare both with the oracle)
        log("checking the padded layout against dense rows on one forward")
        mem_p, mem_d = with_rows(dense_mem, ms), dense_mem.clone()
        out_p, out_d = (torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), dtype=torch.float32, device="cuda")
                        for _ in range(2))
        with SDM.from_config(cfg, mem_stride=ms) as pl, SDM.from_config(cfg) as dl:
            pl.forward(d["wq"], d["rq"], d["v"], d["alpha"], d["beta"], d["subkeys"], mem_p, out_p)
            dl.forward(d["wq"], d["rq"], d["v"], d["alpha"], d["beta"], d["subkeys"], mem_d, out_d)
            torch.cuda.synchronize()
        ity = torch.int16 if cfg.state_bf16 else torch.int32
        padded_equals_dense = bool(torch.equal(out_p.view(torch.int32), out_d.view(torch.int32))) and all(
            bool(torch.equal(mem_p[b].contiguous().view(ity), mem_d[b].view(ity))) for b in range(cfg.B))
        del mem_p, mem_d, out_p, out_d
        if not padded_equals_dense:
            raise RuntimeError("the padded layout's forward differs from the dense one")
    out = torch.empty((cfg.B, cfg.T, cfg.H, cfg.d), dtype=torch.float32, device="cuda")
    layer = SDM.from_config(cfg, mem_stride=ms)

    def step():
        layer.forward(d["wq"], d["rq"], d["v"], d["alpha"], d["beta"], d["subkeys"], d["mem0"], out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the headline: K forwards with nothing recorded between the library's launches
    t0 = time.perf_counter()
    for i in range(args.steps):
        step()
        if (i + 1) % 10 == 0:
            log(f"step {i + 1}/{args.steps}")
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    if not torch.isfinite(out).all():
        raise RuntimeError("non-finite output")
    # the same K forwards again with HIP events around every launch, on the stream it runs on: the
    # device time of each kernel (the scan's per launch gives the roofline); the events themselves
    # add about 10 us between dependent launches, so this region is not the headline
    layer.set_timing(True)
    torch.cuda.synchronize()
    te0 = time.perf_counter()
    for i in range(args.steps):
        step()
    torch.cuda.synchronize()
    te1 = time.perf_counter()
    tm = layer.timing()
    layer.set_timing(False)

    # The same forwards on dense slot rows (d elements apart), for comparison with the
    # padded layout the headline uses.
    dense = None
    if dense_mem is not None:
        with SDM.from_config(cfg) as dl:
            dn = min(args.steps, 10)
            dl.forward(d["wq"], d["rq"], d["v"], d["alpha"], d["beta"], d["subkeys"], dense_mem, out)
            torch.cuda.synchronize()
            t2 = time.perf_counter()
            for _ in range(dn):
                dl.forward(d["wq"], d["rq"], d["v"], d["alpha"], d["beta"], d["subkeys"], dense_mem, out)
            torch.cuda.synchronize()
            dsec = time.perf_counter() - t2
        dense = {"value": cfg.B * cfg.T * dn / dsec, "unit": "tokens/s", "ms_per_step": dsec * 1e3 / dn, "steps": dn,
                 "what": "the same forward with the memory's slot rows dense (d elements apart)"}
        del dense_mem

    # Sub-key scoring and selection on their own (in the forward they share the
    # GPU with the scan): both query sets through sdm_address_pair, the
    # forward's own launches (one scoring and one selection launch for both
    # sets) over every row, each timed with HIP events.
    rows = cfg.B * cfg.T * cfg.H
    a_out = [torch.empty((rows, cfg.W), dtype=dt, device="cuda")
             for dt in (torch.int32, torch.float32, torch.int32, torch.float32)]
    layer.set_timing(True)
    reps = 5
    for _ in range(reps):
        layer.address_pair(d["wq"], d["rq"], d["subkeys"], *a_out)
    torch.cuda.synchronize()
    tm_alone = layer.timing()
    score_alone_ms = tm_alone["ms_score"] / reps
    select_alone_ms = tm_alone["ms_select"] / reps
    del a_out

    # The ceiling of the scan's access pattern: the same random 128-byte segment
    # reads and writes with no arithmetic (scrambles the memory, which is no
    # longer needed).
    s_bytes = 2 if cfg.state_bf16 else 4
    pat = []
    for i in range(4):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        pattern_probe_mix(d["mem0"], cfg.B * cfg.H, cfg.N, cfg.d * s_bytes, cfg.T, cfg.W, 2, 1, seed=i,
                          row_stride=ms * s_bytes)
        e1.record()
        torch.cuda.synchronize()
        if i:
            pat.append(e0.elapsed_time(e1))
    pattern_ms = sum(pat) / len(pat)
    layer.close()
    copy = copy_bandwidth()

    sec = t1 - t0
    tokens = cfg.B * cfg.T * args.steps
    # device time per forward of each kernel (a forward scans in chunks: several
    # scan launches, with the next chunk's addressing and plan overlapping)
    per_step = {k: tm[f"ms_{k}"] / args.steps for k in ("score", "select", "plan", "scan")}
    timed_ms_per_step = (te1 - te0) * 1e3 / args.steps
    scan_launches = tm["n_scan"] / args.steps
    scan_ms = per_step["scan"]
    nbytes = scan_bytes_per_step(cfg)
    achieved = nbytes / (scan_ms * 1e-3) / 1e9
    sig = kernel_signature()
    traffic = load_traffic(sig, ms) if args.workload == WORKLOAD else None
    score_tflops = score_flops_per_step(cfg) / (score_alone_ms * 1e-3) / 1e12
    peak_mfma = BF16_MFMA_PEAK_TFLOPS if cfg.in_bf16 else F32_MFMA_PEAK_TFLOPS

    res = {
        "metric": METRIC if args.workload == WORKLOAD else METRIC.replace("1.4B shape", f"{cfg.name} shape"),
        "value": tokens / sec,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": sec * 1e3 / args.steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": f"synthetic (seeded; queries, values and sub-keys {'bf16' if cfg.in_bf16 else 'float32'}, "
                f"state {'bf16' if cfg.state_bf16 else 'float32'} ~N(0,{cfg.m0_std}))",
        "config": {"workload": f"sdm-{cfg.name} layer: B={cfg.B} H={cfg.H} T={cfg.T} d={cfg.d} N={cfg.S}^2 "
                               f"dk={cfg.dk} k={cfg.k} W={cfg.W}, {'bf16' if cfg.in_bf16 else 'float32'} inputs, "
                               f"{'bf16' if cfg.state_bf16 else 'float32'} state",
                   "global_batch": cfg.B, "seq_len": cfg.T, "parallelism": "single GPU",
                   "state_rows": rows_note(cfg, ms)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if traffic is None else traffic / scan_launches,
                     "kernel": "sdm_scan", "launches_per_step": scan_launches,
                     "timing": "HIP events around each scan launch on the caller's stream, over a second run "
                               "of the same steps right after the headline run",
                     "bytes_per_launch": nbytes / scan_launches, "ms_per_launch": scan_ms / scan_launches,
                     "pattern_ceiling": {"achieved": nbytes / (pattern_ms * 1e-3) / 1e9, "unit": "GB/s",
                                         "ms_per_launch": pattern_ms,
                                         "frac": (nbytes / (scan_ms * 1e-3)) / (nbytes / (pattern_ms * 1e-3)),
                                         "what": "sdm_pattern_probe_mix 2:1: the scan's random 128-byte segment "
                                                 "reads and writes with no arithmetic, on rows as far apart as "
                                                 "the memory's; frac = scan / this"},
                     "copy_peak": {"achieved": copy["achieved"], "unit": "GB/s", "frac": achieved / copy["achieved"],
                                   "kernel": copy["kernel"], "all": copy["all"],
                                   "what": "the faster of two plain 2 GiB device copies (bytes read + written "
                                           "per second), the measured stand-in for the HBM peak; "
                                           "frac = scan / this"}},
        "kernels_ms_per_step": {"pk_score": per_step["score"], "pk_topk": per_step["select"],
                                "sdm_plan": per_step["plan"], "sdm_scan": scan_ms,
                                "ms_per_step_with_events": timed_ms_per_step,
                                "note": "device time of each kernel in the forward, from HIP events around every "
                                        "launch over a second run of the same steps (the headline run records "
                                        "none); after the first chunk, pk_score, pk_topk and sdm_plan run on a "
                                        "second stream under the scan"},
        "pk_score": {"tflops": score_tflops, "peak_tflops": peak_mfma, "frac": score_tflops / peak_mfma,
                     "ms_per_step_alone": score_alone_ms,
                     "stored_scores": scoring_output(cfg),
                     "note": "both query sets scored alone by the forward's kernel, in one launch as the forward "
                             "runs it (sdm_address_pair over every row, HIP events around pk_score only); in the "
                             "forward the scoring of the next chunk shares the GPU with the scan, so "
                             "kernels_ms_per_step shows it longer"},
        "pk_topk": {"ms_per_step_alone": select_alone_ms,
                    "note": "both query sets' exact selection alone, in one launch (sdm_address_pair, HIP events "
                            "around pk_topk)"},
        "kernel_signature": sig,
    }
    if dense is not None:
        dense["bitwise_equal_to_padded"] = padded_equals_dense
        res["dense_rows"] = dense
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        res["cpu_baseline"] = cpu_baseline(cfg, x, args.cpu_seconds)
    print(json.dumps(res))


if __name__ == "__main__":
    main()
