"""The measurement entry point sdm_pattern_probe on the GPU: it runs, moves the
memory it is given and leaves memory past it alone."""
import pytest

pytestmark = pytest.mark.gpu


def test_pattern_probe_runs_and_stays_in_bounds():
    import torch
    from sparse_memory_linear_pk_amd import pattern_probe
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    memories, rows, row_bytes, T, W = 2, 1000, 512, 64, 64
    n = memories * rows * row_bytes // 4
    buf = torch.randn(n + 4096, device="cuda")
    guard = buf[n:].clone()
    before = buf[:n].clone()
    pattern_probe(buf, memories, rows, row_bytes, T, W, seed=3)
    torch.cuda.synchronize()
    assert torch.equal(buf[n:], guard)
    assert not torch.equal(buf[:n], before)


def test_pattern_probe_with_the_backward_mix_stays_in_bounds():
    """4 reads : 3 writes per slot position and token (the reverse scan's traffic)."""
    import torch
    from sparse_memory_linear_pk_amd import pattern_probe_mix
    memories, rows, row_bytes, T, W = 3, 777, 384, 50, 40
    n = memories * rows * row_bytes // 4
    buf = torch.randn(n + 4096, device="cuda")
    guard = buf[n:].clone()
    before = buf[:n].clone()
    pattern_probe_mix(buf, memories, rows, row_bytes, T, W, 4, 3, seed=5)
    torch.cuda.synchronize()
    assert torch.equal(buf[n:], guard)
    assert not torch.equal(buf[:n], before)
