"""The C ABI without a GPU: the library loads, exports what include/sdm.h declares,
and rejects bad arguments on the host before touching a device."""
import ctypes as C

import pytest

from sparse_memory_linear_pk_amd import _lib
from sparse_memory_linear_pk_amd._lib import Config, Timing, SDM_OK, SDM_ERR_INVALID_ARG, SDM_ERR_UNSUPPORTED

EXPECTED = ["sdm_create", "sdm_forward", "sdm_destroy", "sdm_status_str", "sdm_last_error", "sdm_workspace_bytes",
            "sdm_score", "sdm_select", "sdm_address", "sdm_address_pair", "sdm_scan_with", "sdm_set_timing", "sdm_get_timing",
            "sdm_pattern_probe", "sdm_step", "sdm_forward_train", "sdm_backward_workspace_bytes", "sdm_backward",
            "sdm_pattern_probe_mix", "sdm_project", "sdm_broadcast_memory", "sdm_overlap", "sdm_mem_stride_hint",
            "sdm_step_static"]


def _cfg(**kw):
    base = dict(B=4, H=1, T=8192, d=2048, n_sub=480, dk=256, k=32, W=64, in_dtype=1, state_dtype=0)
    base.update(kw)
    return Config(**base)


def test_header_declares_the_entry_points():
    assert sorted(_lib.declared_symbols()) == sorted(EXPECTED)


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in _lib.declared_symbols():
        assert hasattr(L, name), name


def test_status_strings():
    L = _lib.lib()
    assert L.sdm_status_str(SDM_OK) == b"ok"
    assert L.sdm_status_str(SDM_ERR_INVALID_ARG) == b"invalid argument"
    assert L.sdm_status_str(99) == b"unknown status"


def test_workspace_bytes_for_the_1p4b_shape():
    L = _lib.lib()
    n = C.c_size_t()
    assert L.sdm_workspace_bytes(C.byref(_cfg()), C.byref(n)) == SDM_OK
    rows = 4 * 8192
    # bf16 inputs: the forward's half scores are binary16; slot ids and weights of both query sets
    assert n.value >= rows * 2 * 480 * 2 + 2 * 2 * rows * 64 * 4
    f32 = C.c_size_t()
    assert L.sdm_workspace_bytes(C.byref(_cfg(in_dtype=0)), C.byref(f32)) == SDM_OK
    assert f32.value - n.value >= rows * 2 * 480 * 2 - 4096  # float32 scores for float32 inputs


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), SDM_ERR_INVALID_ARG),
    (dict(dk=255), SDM_ERR_INVALID_ARG),
    (dict(k=481), SDM_ERR_INVALID_ARG),
    (dict(k=4, W=17), SDM_ERR_INVALID_ARG),
    (dict(in_dtype=7), SDM_ERR_INVALID_ARG),
    (dict(dk=2 * 40), SDM_ERR_UNSUPPORTED),
    (dict(k=65, W=64), SDM_ERR_UNSUPPORTED),
    (dict(W=65, k=33), SDM_ERR_UNSUPPORTED),
    (dict(n_sub=1025), SDM_ERR_UNSUPPORTED),
    (dict(d=2044), SDM_ERR_UNSUPPORTED),
    (dict(n_sub=640, d=3840, state_dtype=0), SDM_ERR_UNSUPPORTED),  # 6.3 GB per memory in float32
    (dict(mem_stride=2047), SDM_ERR_INVALID_ARG),                   # rows closer than d
    (dict(mem_stride=2050), SDM_ERR_INVALID_ARG),                   # rows not 16 bytes apart
    (dict(mem_stride=4700), SDM_ERR_UNSUPPORTED),                   # 4.3 GB per memory with the padding
    (dict(state_dtype=1, n_sub=640, d=3840, mem_stride=6000), SDM_ERR_UNSUPPORTED),  # 4.9 GB of bf16
    # rows of 8200 float32 values (the register-ring scan) over 64 heads: one sequence's v of a
    # 2048-token chunk is 4.3 GB, past a 32-bit buffer offset
    (dict(H=64, T=2048, d=8200, n_sub=64, dk=32, k=4, W=8), SDM_ERR_UNSUPPORTED),
])
def test_bad_configs_are_rejected_on_the_host(kw, status):
    L = _lib.lib()
    n = C.c_size_t()
    assert L.sdm_workspace_bytes(C.byref(_cfg(**kw)), C.byref(n)) == status
    assert L.sdm_last_error() != b""
    h = C.c_void_p()
    assert L.sdm_create(C.byref(_cfg(**kw)), None, C.byref(h)) == status
    assert h.value is None


def test_null_arguments():
    L = _lib.lib()
    assert L.sdm_workspace_bytes(None, None) == SDM_ERR_INVALID_ARG
    assert L.sdm_create(C.byref(_cfg()), None, None) == SDM_ERR_INVALID_ARG
    for f, n in (("sdm_forward", 8), ("sdm_score", 3), ("sdm_select", 3), ("sdm_address", 4),
                 ("sdm_address_pair", 7), ("sdm_scan_with", 9), ("sdm_step", 8), ("sdm_forward_train", 9),
                 ("sdm_backward", 16), ("sdm_broadcast_memory", 2)):
        assert getattr(L, f)(None, *([None] * n)) == SDM_ERR_INVALID_ARG, f
    assert L.sdm_project(None, 64, *([None] * 8)) == SDM_ERR_INVALID_ARG
    assert L.sdm_overlap(None, None, None, None, None, 4, None, None, 0, None, None) == SDM_ERR_INVALID_ARG
    assert L.sdm_destroy(None) == SDM_ERR_INVALID_ARG
    assert L.sdm_set_timing(None, 1) == SDM_ERR_INVALID_ARG
    assert L.sdm_get_timing(None, C.byref(Timing())) == SDM_ERR_INVALID_ARG
    assert b"handle" in L.sdm_last_error()


def test_forged_handle_is_rejected():
    L = _lib.lib()
    junk = (C.c_uint32 * 64)()
    assert L.sdm_forward(C.cast(junk, C.c_void_p), *([None] * 8)) == SDM_ERR_INVALID_ARG
    assert L.sdm_destroy(C.cast(junk, C.c_void_p)) == SDM_ERR_INVALID_ARG


@pytest.mark.parametrize("mem,memories,rows,row_bytes,T,W", [
    (None, 4, 230400, 8192, 8192, 64),       # no memory
    (16, 4, 230400, 8192, 8192, 65),         # W past 64
    (8, 4, 230400, 8192, 8192, 64),          # misaligned
    (16, 4, 230400, 8000, 8192, 64),         # row not a multiple of 128 bytes
    (16, 4, 640 * 640, 3840 * 4, 16, 64),    # one memory of 6.3 GB
    (16, 0, 230400, 8192, 16, 64),           # no memories
])
def test_pattern_probe_rejects_bad_arguments_on_the_host(mem, memories, rows, row_bytes, T, W):
    L = _lib.lib()
    assert L.sdm_pattern_probe(mem, memories, rows, row_bytes, T, W, 0, None) == SDM_ERR_INVALID_ARG
    assert L.sdm_last_error().startswith(b"sdm_pattern_probe")


@pytest.mark.parametrize("row_stride", [8191, 8200, 8192 * 3])  # closer than a row, not 16-byte, 5.7 GB
def test_pattern_probe_rejects_bad_row_strides(row_stride):
    L = _lib.lib()
    assert L.sdm_pattern_probe_mix(16, 4, 230400, 8192, row_stride, 16, 64, 2, 1, 0, None) == SDM_ERR_INVALID_ARG
    assert b"row_stride" in L.sdm_last_error()


@pytest.mark.parametrize("kw,want", [
    (dict(), 2080),                                  # 8192-byte rows -> 8320
    (dict(state_dtype=1), 2112),                     # 4096 -> 4224
    (dict(state_dtype=1, n_sub=640, d=3840), 3904),  # 7680 -> 7808
    (dict(d=2080), 2080),                            # already an odd number of 128-byte units
    (dict(d=128), 128),                              # under 1 KB: dense
    (dict(d=2040), 2040),                            # not whole 128-byte units: dense
])
def test_mem_stride_hint(kw, want):
    L = _lib.lib()
    assert L.sdm_mem_stride_hint(C.byref(_cfg(**kw))) == want
    assert L.sdm_mem_stride_hint(None) == 0


def test_backward_workspace_for_the_1p4b_shape():
    """Column partials (2W+2 floats per row and 128-byte column), dense dsigma rows of both query
    sets, and the split sub-key sums."""
    L = _lib.lib()
    n = C.c_size_t()
    assert L.sdm_backward_workspace_bytes(C.byref(_cfg()), C.byref(n)) == SDM_OK
    rows = 4 * 8192
    assert n.value >= rows * 64 * 130 * 4 + 2 * rows * 2 * 480 * 4


@pytest.mark.parametrize("kw", [dict(state_dtype=1, n_sub=240, d=2016), dict(d=2040)])
def test_backward_rejects_what_it_does_not_build(kw):
    """Slot rows that are not whole 128-byte columns (64 bf16 or 32 float32 elements)."""
    L = _lib.lib()
    n = C.c_size_t()
    assert L.sdm_backward_workspace_bytes(C.byref(_cfg(**kw)), C.byref(n)) == SDM_ERR_UNSUPPORTED
    assert b"sdm_backward" in L.sdm_last_error()


@pytest.mark.parametrize("kw", [dict(state_dtype=1, n_sub=640, d=3840, T=2048, B=8),
                                dict(state_dtype=1, n_sub=640, d=3840, T=2048, B=8, mem_stride=3904)])
def test_backward_takes_a_gradient_past_4_gib(kw):
    """The 8B shape: its float32 memory gradient is 6.3 GB per memory (640^2 rows of 3840 values), which
    the reverse scan addresses with 64-bit pointers."""
    L = _lib.lib()
    n = C.c_size_t()
    assert L.sdm_backward_workspace_bytes(C.byref(_cfg(**kw)), C.byref(n)) == SDM_OK


@pytest.mark.parametrize("reads,writes", [(3, 1), (4, 4), (2, 2), (0, 0)])
def test_pattern_probe_mix_rejects_unbuilt_mixes(reads, writes):
    L = _lib.lib()
    assert L.sdm_pattern_probe_mix(16, 4, 230400, 8192, 0, 16, 64, reads, writes, 0, None) == SDM_ERR_INVALID_ARG
    assert b"reads:writes" in L.sdm_last_error()


def test_step_static_rejects_on_the_host():
    """The allocation-free decode step checks its arguments before it touches a device: a missing
    config or pointer, an unsupported row width, and more slot entries than its scratch holds."""
    L = _lib.lib()
    fake = [16] * 8  # aligned, never dereferenced: every case fails before any device call
    assert L.sdm_step_static(None, None, *fake) == SDM_ERR_INVALID_ARG
    small = dict(B=2, H=1, T=1, d=64, n_sub=32, dk=32, k=6, W=16, in_dtype=0, state_dtype=0)
    assert L.sdm_step_static(C.byref(_cfg(**small)), None, *([None] * 8)) == SDM_ERR_INVALID_ARG
    assert L.sdm_step_static(C.byref(_cfg(**dict(small, d=24))), None, *fake) == SDM_ERR_UNSUPPORTED
    # B*H*W = 1025 * 64 > 65536
    assert L.sdm_step_static(C.byref(_cfg(**dict(small, B=1025, W=64, k=8))), None, *fake) == SDM_ERR_UNSUPPORTED
    assert b"scratch" in L.sdm_last_error()
