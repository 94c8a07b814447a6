"""Counter-seeded generators for the five SDM workloads (see package docstring)."""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# Elements per independently seeded chunk.  Chunk c of tensor id t under seed s
# is drawn from PCG64(SeedSequence(s, spawn_key=(t, c))), so a tensor's values
# do not depend on how many threads generate it.
CHUNK = 1 << 22

# tensor ids
_WQ, _RQ, _V, _ALPHA, _BETA, _SUBKEYS, _MEM0, _CENTROIDS, _PICK_W, _PICK_R, _NOISE_W, _NOISE_R = range(1, 13)
_DOUT, _DMEM = 13, 14
_EMB, _PROJ_W, _GATE_B = 15, 16, 17


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    T: int
    d: int
    S: int            # sub-keys per half; N = S*S slots
    dk: int           # addressing dim, two halves of dk/2
    k: int            # per-half candidates
    W: int            # slots selected per token, for write and for read
    in_bf16: bool     # wq, rq, v, subkeys stored as bf16
    state_bf16: bool  # memory stored as bf16
    alpha_shift: float = 3.0   # alpha = sigmoid(N(0,1) + alpha_shift)
    m0_std: float = 0.02       # initial memory ~ N(0, m0_std); 0 -> zeros
    subkey_std: float = 0.25
    query: str = "iid"         # "iid" | "planted" | "zipf"
    zipf_centroids: int = 512
    zipf_s: float = 1.1
    zipf_noise: float = 0.1

    @property
    def N(self) -> int:
        return self.S * self.S

    @property
    def dh(self) -> int:
        return self.dk // 2

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


CONFIGS = {
    0: Config("tiny", B=1, H=1, T=256, d=32, S=64, dk=32, k=8, W=16, in_bf16=False,
              state_bf16=False, alpha_shift=3.0, m0_std=0.0),
    1: Config("small", B=4, H=4, T=4096, d=128, S=128, dk=128, k=16, W=64, in_bf16=False,
              state_bf16=False, alpha_shift=3.0, m0_std=0.02),
    2: Config("1.4B", B=4, H=1, T=8192, d=2048, S=480, dk=256, k=32, W=64, in_bf16=True,
              state_bf16=False, alpha_shift=4.0, m0_std=0.02),
    3: Config("long", B=1, H=1, T=131072, d=2048, S=480, dk=256, k=32, W=64, in_bf16=True,
              state_bf16=True, alpha_shift=4.0, m0_std=0.02, query="planted"),
    4: Config("8B", B=8, H=1, T=16384, d=3840, S=640, dk=256, k=32, W=64, in_bf16=True,
              state_bf16=True, alpha_shift=4.0, m0_std=0.02, query="zipf"),
}


def config(i: int, **overrides) -> Config:
    c = CONFIGS[i]
    return c.replace(**overrides) if overrides else c


def _threads(threads):
    if threads:
        return threads
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _gen(seed: int, tid: int, c: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tid, c))))


def _chunked(n: int, fn, threads=None):
    nchunks = (n + CHUNK - 1) // CHUNK
    if nchunks <= 1:
        for c in range(nchunks):
            fn(c, 0, n)
        return
    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(lambda c: fn(c, c * CHUNK, min(n, (c + 1) * CHUNK)), range(nchunks)))


def normal_f32(shape, seed: int, tid: int, std: float = 1.0, threads=None) -> np.ndarray:
    """N(0, std) in float32, chunk-seeded."""
    n = int(np.prod(shape))
    out = np.empty(n, np.float32)

    def fill(c, lo, hi):
        _gen(seed, tid, c).standard_normal(out=out[lo:hi], dtype=np.float32)
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    _chunked(n, fill, threads)
    return out.reshape(shape)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even), returned as uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    nan = (u & 0x7FFFFFFF) > 0x7F800000
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)).astype(np.uint16)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return r


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _store_in(x: np.ndarray, bf16: bool) -> np.ndarray:
    return bf16_bits_from_f32(x) if bf16 else np.ascontiguousarray(x, np.float32)


def _sigmoid_f32(z: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-z.astype(np.float64)))).astype(np.float32)


def _queries(cfg: Config, seed: int, threads=None):
    shape = (cfg.B, cfg.T, cfg.H, cfg.dk)
    if cfg.query in ("iid", "planted"):
        wq = normal_f32(shape, seed, _WQ, 1.0, threads)
        rq = normal_f32(shape, seed, _RQ, 1.0, threads)
        if cfg.query == "planted":
            # the write query of token 61 comes back as the read query of token T-17
            assert cfg.T > 61 + 17, "planted pattern needs T > 78"
            rq[:, cfg.T - 17] = wq[:, 61]
        return wq, rq
    if cfg.query == "zipf":
        C = normal_f32((cfg.zipf_centroids, cfg.dk), seed, _CENTROIDS, 1.0, threads)
        ranks = np.arange(1, cfg.zipf_centroids + 1, dtype=np.float64)
        p = ranks ** (-cfg.zipf_s)
        cdf = np.cumsum(p / p.sum())
        cdf[-1] = 1.0
        out = []
        for pick_id, noise_id in ((_PICK_W, _NOISE_W), (_PICK_R, _NOISE_R)):
            u = _gen(seed, pick_id, 0).random(cfg.B * cfg.T * cfg.H)
            choice = np.minimum(np.searchsorted(cdf, u, side="right"), cfg.zipf_centroids - 1)
            q = normal_f32(shape, seed, noise_id, cfg.zipf_noise, threads)
            q += C[choice].reshape(shape)
            out.append(q)
        return out[0], out[1]
    raise ValueError(f"unknown query recipe {cfg.query!r}")


def make_mem0(cfg: Config, seed: int = 0, threads=None) -> np.ndarray:
    """Initial memory [B, H, N, d] in the state storage format."""
    shape = (cfg.B, cfg.H, cfg.N, cfg.d)
    if cfg.m0_std == 0.0:
        return np.zeros(shape, np.uint16 if cfg.state_bf16 else np.float32)
    if not cfg.state_bf16:
        return normal_f32(shape, seed, _MEM0, cfg.m0_std, threads)
    n = int(np.prod(shape))
    out = np.empty(n, np.uint16)
    tmp_std = np.float32(cfg.m0_std)

    def fill(c, lo, hi):
        x = np.empty(hi - lo, np.float32)
        _gen(seed, _MEM0, c).standard_normal(out=x, dtype=np.float32)
        x *= tmp_std
        out[lo:hi] = bf16_bits_from_f32(x)

    _chunked(n, fill, threads)
    return out.reshape(shape)


def make_mem0_seqs(cfg: Config, b0: int, b1: int, seed: int = 0, threads=None) -> np.ndarray:
    """Sequences b0 .. b1-1 of make_mem0(cfg, seed), [b1-b0, H, N, d], bit for bit, without
    drawing the others (the seeded chunks that cover them are drawn, each from its start)."""
    shape = (b1 - b0, cfg.H, cfg.N, cfg.d)
    per_seq = cfg.H * cfg.N * cfg.d
    dtype = np.uint16 if cfg.state_bf16 else np.float32
    if cfg.m0_std == 0.0:
        return np.zeros(shape, dtype)
    lo, hi = b0 * per_seq, b1 * per_seq
    out = np.empty(hi - lo, dtype)
    c0, c1 = lo // CHUNK, (hi - 1) // CHUNK
    std = np.float32(cfg.m0_std)

    def fill(c):
        a, b = max(lo, c * CHUNK), min(hi, (c + 1) * CHUNK)
        x = np.empty(b - c * CHUNK, np.float32)
        _gen(seed, _MEM0, c).standard_normal(out=x, dtype=np.float32)
        x = x[a - c * CHUNK:]
        x *= std
        out[a - lo:b - lo] = bf16_bits_from_f32(x) if cfg.state_bf16 else x

    with ThreadPoolExecutor(_threads(threads)) as ex:
        list(ex.map(fill, range(c0, c1 + 1)))
    return out.reshape(shape)


def make_inputs(cfg: Config, seed: int = 0, threads=None, with_mem0: bool = True) -> dict:
    """All layer inputs for one configuration, as numpy arrays (see package docstring)."""
    wq, rq = _queries(cfg, seed, threads)
    v = normal_f32((cfg.B, cfg.T, cfg.H, cfg.d), seed, _V, 1.0, threads)
    za = normal_f32((cfg.B, cfg.T, cfg.H), seed, _ALPHA, 1.0, threads)
    zb = normal_f32((cfg.B, cfg.T, cfg.H), seed, _BETA, 1.0, threads)
    alpha = _sigmoid_f32(za.astype(np.float64) + cfg.alpha_shift)
    beta = _sigmoid_f32(zb)
    subkeys = normal_f32((cfg.H, 2, cfg.S, cfg.dh), seed, _SUBKEYS, cfg.subkey_std, threads)
    out = {
        "wq": _store_in(wq, cfg.in_bf16),
        "rq": _store_in(rq, cfg.in_bf16),
        "v": _store_in(v, cfg.in_bf16),
        "alpha": alpha,
        "beta": beta,
        "subkeys": _store_in(subkeys, cfg.in_bf16),
    }
    if with_mem0:
        out["mem0"] = make_mem0(cfg, seed, threads)
    return out


def make_upstream_grads(cfg: Config, seed: int = 0, dmem_std: float = 0.1, threads=None) -> dict:
    """Seeded upstream gradients for a backward pass: dout [B, T, H, d] ~ N(0, 1) and
    dmem [B, H, N, d] ~ N(0, dmem_std) (the gradient reaching the final memory), float32."""
    return {"dout": normal_f32((cfg.B, cfg.T, cfg.H, cfg.d), seed, _DOUT, 1.0, threads),
            "dmem": normal_f32((cfg.B, cfg.H, cfg.N, cfg.d), seed, _DMEM, dmem_std, threads)}


def make_projection_inputs(cfg: Config, D: int, seed: int = 0, threads=None) -> dict:
    """Seeded inputs of the input projections: embedding x [B, T, D] ~ N(0, 1), weights
    w [H*(2dk+d+2), D] ~ N(0, 1/sqrt(D)) (both bf16 bits), gate biases [H, 2] float32: alpha's
    N(4, 1), beta's N(0, 1) (the workloads' gate distributions when the projection adds N(0, 1))."""
    C = 2 * cfg.dk + cfg.d + 2
    x = normal_f32((cfg.B, cfg.T, D), seed, _EMB, 1.0, threads)
    w = normal_f32((cfg.H * C, D), seed, _PROJ_W, 1.0 / float(np.sqrt(D)), threads)
    gb = normal_f32((cfg.H, 2), seed, _GATE_B, 1.0, threads)
    gb[:, 0] += np.float32(4.0)
    return {"x": bf16_bits_from_f32(x), "w": bf16_bits_from_f32(w), "gate_bias": gb}
