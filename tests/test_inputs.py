"""The seeded input generator: determinism, shapes, recipes, and the pages' shape constants."""
import json
import os

import numpy as np

import sdm_inputs as gi

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_constants.json")


def test_configs_match_the_pages_constants():
    g = json.load(open(GOLDEN))
    c2, c3, c4 = gi.config(2), gi.config(3), gi.config(4)
    assert c2.N == g["slots_1p4b"]["value"] == 480 * 480
    for c in (c2, c3, c4):
        assert c.W == g["active_slots_per_token"]["value"]
    assert c4.d == g["slot_width_8b"]["value"] and c4.state_bf16
    # the planted recurring query keeps the needle geometry: 239 = 256 - 17
    assert g["query_token"]["value"] == g["needle_task_tokens"]["value"] - 17
    assert g["needle_token"]["value"] == 61


def test_deterministic_and_thread_independent():
    cfg = gi.config(1, T=64)
    a = gi.make_inputs(cfg, seed=0, threads=1)
    b = gi.make_inputs(cfg, seed=0, threads=7)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    c = gi.make_inputs(cfg, seed=1, threads=2)
    assert not np.array_equal(a["wq"], c["wq"])
    # a tensor spanning several chunks is also thread independent
    x1 = gi.normal_f32((3, gi.gen.CHUNK + 17), 0, 99, 0.5, threads=1)
    x2 = gi.normal_f32((3, gi.gen.CHUNK + 17), 0, 99, 0.5, threads=5)
    assert np.array_equal(x1, x2)


def test_shapes_and_dtypes():
    for i, T in ((0, 256), (1, 32), (2, 16), (3, 128), (4, 16)):
        cfg = gi.config(i, T=T)
        x = gi.make_inputs(cfg, with_mem0=False)
        inb = np.uint16 if cfg.in_bf16 else np.float32
        assert x["wq"].shape == (cfg.B, T, cfg.H, cfg.dk) and x["wq"].dtype == inb
        assert x["rq"].shape == x["wq"].shape
        assert x["v"].shape == (cfg.B, T, cfg.H, cfg.d) and x["v"].dtype == inb
        assert x["alpha"].shape == (cfg.B, T, cfg.H) and x["alpha"].dtype == np.float32
        assert x["subkeys"].shape == (cfg.H, 2, cfg.S, cfg.dh) and x["subkeys"].dtype == inb
        assert np.all((x["alpha"] > 0) & (x["alpha"] < 1)) and np.all((x["beta"] > 0) & (x["beta"] < 1))


def test_distributions():
    cfg = gi.config(1, T=512)
    x = gi.make_inputs(cfg)
    assert abs(x["wq"].std() - 1) < 0.02 and abs(x["v"].mean()) < 0.02
    assert abs(x["subkeys"].std() - 0.25) < 0.01
    assert abs(x["mem0"].std() - 0.02) < 0.001
    za = np.log(x["alpha"] / (1 - x["alpha"])) - cfg.alpha_shift
    assert abs(za.mean()) < 0.05 and abs(za.std() - 1) < 0.05
    assert np.all(gi.make_mem0(gi.config(0)) == 0)


def test_planted_and_zipf_recipes():
    c3 = gi.config(3, T=300)
    x = gi.make_inputs(c3, with_mem0=False)
    assert np.array_equal(x["rq"][:, c3.T - 17], x["wq"][:, 61])
    assert not np.array_equal(x["rq"][:, c3.T - 18], x["wq"][:, 61])
    c4 = gi.config(4, T=2048, B=2)
    x = gi.make_inputs(c4, with_mem0=False)
    q = gi.f32_from_bf16_bits(x["wq"]).reshape(-1, c4.dk)[:600].astype(np.float64)
    msd = ((q[:, None, :] - q[None, :, :]) ** 2).mean(-1)
    iu = np.triu_indices(q.shape[0], 1)
    same = msd[iu] < 0.1  # same centroid: 2 * 0.1^2 per element; different: about 2
    # pairs sharing a centroid: sum_r p_r^2 for Zipf(1.1) over 512 ranks, about 0.065
    assert 0.03 < same.mean() < 0.12, same.mean()
    assert np.all((msd[iu] < 0.1) | (msd[iu] > 0.5))


def test_bf16_conversion():
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, -2.5, np.inf, 0.0], np.float32)
    assert gi.bf16_bits_from_f32(x).tolist() == [0x3F80, 0x3F80, 0x3F82, 0xC020, 0x7F80, 0x0000]
    assert gi.f32_from_bf16_bits(np.array([0x3F80, 0xC020], np.uint16)).tolist() == [1.0, -2.5]


def test_initial_memory_by_sequence_equals_the_whole():
    """make_mem0_seqs draws the same bits as make_mem0 for any sequence range,
    also where a sequence starts or ends inside a seeded chunk."""
    for cfg in (gi.config(1, T=8, B=5, H=3, S=100, d=72),                      # float32, ragged chunks
                gi.config(4, T=8, B=3, S=90, d=3840 // 8),                     # bf16
                gi.config(0, T=8, B=3)):                                       # zero memory
        whole = gi.make_mem0(cfg)
        for b0, b1 in ((0, 1), (1, 3), (2, cfg.B), (0, cfg.B)):
            part = gi.make_mem0_seqs(cfg, b0, b1, threads=3)
            assert part.dtype == whole.dtype and np.array_equal(part, whole[b0:b1]), (cfg.name, b0, b1)
