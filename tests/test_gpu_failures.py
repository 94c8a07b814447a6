"""Failure handling on the device, forced from the host (no kernel runs on bad
data): sdm_create asked for a workspace larger than the device's memory
returns SDM_ERR_OOM with a message, leaves no handle, and the library works
normally afterwards (no error left behind in the HIP runtime)."""
import ctypes as C
import sys

import numpy as np
import pytest

import sdm_inputs as gi
from parity import to_dev

pytestmark = pytest.mark.gpu


def test_workspace_larger_than_the_device_is_out_of_memory():
    import torch
    from sparse_memory_linear_pk_amd import SDM
    from sparse_memory_linear_pk_amd._lib import SDM_ERR_OOM, SDM_F32, Config, lib
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    total = torch.cuda.get_device_properties(0).total_memory
    L = lib()
    # 2^25 rows of 1024-wide half scores, W = 64: about 10 KB of workspace per row
    cfg = Config(4096, 1, 8192, 32, 1024, 32, 8, 64, SDM_F32, SDM_F32, 0)
    need = C.c_size_t()
    assert L.sdm_workspace_bytes(C.byref(cfg), C.byref(need)) == 0
    print(f"workspace {need.value / 1e9:.0f} GB against {total / 1e9:.0f} GB of device memory", file=sys.stderr)
    if need.value < 1.1 * total:
        pytest.skip("this device holds the workspace")
    h = C.c_void_p(1)
    st = L.sdm_create(C.byref(cfg), None, C.byref(h))
    assert st == SDM_ERR_OOM, (st, L.sdm_last_error())
    assert h.value is None
    assert b"workspace" in L.sdm_last_error()
    # nothing sticks: a small forward right after runs and matches a second, independent one
    c = gi.config(0, T=16)
    x = gi.make_inputs(c)
    dev = {k: to_dev(v) for k, v in x.items()}
    outs = []
    for _ in range(2):
        mem = dev["mem0"].clone()
        out = torch.empty((c.B, c.T, c.H, c.d), dtype=torch.float32, device="cuda")
        with SDM.from_config(c) as layer:
            layer.forward(dev["wq"], dev["rq"], dev["v"], dev["alpha"], dev["beta"], dev["subkeys"], mem, out)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.isfinite(outs[0]).all() and np.array_equal(outs[0], outs[1])
