"""The C ABI library loads and exports what include/fastar.h declares (CPU only).

Only host-side paths are called here: argument validation that returns before
any HIP call, and the workspace-size computation.
"""

import ctypes
import os
import re

import pytest

import kv_cache_attention_tempcache_amd as fa
from kv_cache_attention_tempcache_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fastar.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fastar_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_four_core_calls():
    names = _declared()
    for core in ("fastar_cache_create", "fastar_hash", "fastar_match_merge", "fastar_attend"):
        assert core in names


def test_library_exports_every_declared_symbol():
    lib = fa.library()
    missing = [n for n in _declared() if not hasattr(lib, n)]
    assert not missing, missing
    # the binding declares a signature for each of them
    assert set(_declared()) == set(binding._SIGS)


def _cfg(**kw):
    base = dict(num_heads=2, head_dim=128, budget_slots=512, num_tables=4, num_bits=32,
                cos_threshold=0.95, dtype=binding.BF16)
    base.update(kw)
    return binding.Config(**base)


@pytest.mark.parametrize("bad", [
    dict(num_heads=0), dict(head_dim=96), dict(budget_slots=0), dict(budget_slots=40000),
    dict(num_tables=0), dict(num_tables=9), dict(num_bits=33), dict(num_bits=-1),
    dict(cos_threshold=float("nan")), dict(dtype=7),
])
def test_invalid_config_is_rejected_on_host(bad):
    lib = fa.library()
    n = ctypes.c_size_t(0)
    c = _cfg(**bad)
    st = lib.fastar_cache_workspace_bytes(ctypes.byref(c), ctypes.byref(n))
    assert st == 1  # FASTAR_ERR_INVALID_ARGUMENT
    assert lib.fastar_last_error().decode()


def test_workspace_bytes_covers_the_state():
    lib = fa.library()
    n = ctypes.c_size_t(0)
    c = _cfg(num_heads=12, budget_slots=8192)
    assert lib.fastar_cache_workspace_bytes(ctypes.byref(c), ctypes.byref(n)) == 0
    H, B, d = 12, 8192, 128
    # fp32 masters + bf16 mirrors of K and V at least
    assert n.value >= H * B * d * (4 + 4 + 2 + 2)
    assert n.value % 256 == 0
    assert lib.fastar_last_error().decode() == ""


def test_host_validation_before_any_launch():
    lib = fa.library()
    # d must be 64 or 128
    assert lib.fastar_hash(None, 1, 1, 1, 96, 96, 96, None, 1, 8, None, None) == 1
    # L out of range
    assert lib.fastar_hash(None, 1, 1, 1, 128, 128, 128, None, 9, 8, None, None) == 1
    # null cache handle
    assert lib.fastar_match_merge(None, None, None, 0, 0, None, 1, 1, None, None, None) == 1
    assert lib.fastar_attend(None, None, 0, 0, 1, 0.0, None, 0, 0, None, None) == 1
    # AnnCA limits
    assert lib.fastar_annca_select(None, 5000, 1, None, 10, 1, 1, None, None, None) == 1
    assert lib.fastar_attend_subset(None, 0, 0, None, None, 0, 0, None, None, 1, 1, 1, 1, 100,
                                    1, 0.0, None, 0, 0, None) == 1
    # zero-sized hash is a no-op that succeeds without touching the device
    assert lib.fastar_hash(None, 1, 0, 5, 128, 128, 128, None, 4, 32, None, None) == 0


def test_static_annca_refuses_sizes_beyond_its_array_on_host():
    lib = fa.library()
    # H * F = 4097 segments: beyond the static array, refused before any HIP call
    st = lib.fastar_annca_attend_static(None, 0, 0, None, None, None, 0, 0, None, 1, 4097, 8, 1,
                                        128, 4, 1, 0.0, None, 0, 0, None)
    assert st == 3  # FASTAR_ERR_CAPACITY
    assert "4096" in lib.fastar_last_error().decode()
    # H * F * Np beyond 2^20 selected ids
    st = lib.fastar_annca_attend_static(None, 0, 0, None, None, None, 0, 0, None, 1, 64, 16384, 2,
                                        128, 4, 1, 0.0, None, 0, 0, None)
    assert st == 3


def test_two_launch_annca_refuses_bad_arguments_on_host():
    """fastar_annca_attend checks sizes, pointers and alignment before any HIP
    call; a frame with no queries is a no-op that succeeds."""
    lib = fa.library()
    fake = ctypes.c_void_p(4096)  # never dereferenced: every call below is refused

    def call(q=fake, L=4, b=16, qc=fake, pc=fake, k=fake, v=fake, Nf=64, F=2, Np=512, H=2, d=128,
             scale=0.0, o=fake, stride=128):
        return lib.fastar_annca_attend(q, stride, stride, fake, L, b, qc, pc, k, v, stride, stride,
                                       Nf, F, Np, H, d, scale, o, stride, stride, None)

    assert call(d=64) == 1                       # d = 128 only
    assert call(L=5) == 1                        # 1..4 tables
    assert call(L=0) == 1
    assert call(b=17) == 1                       # codes of at most 16 bits
    assert call(Np=4097) == 1                    # the gather list must fit beside the ring
    assert call(Np=0) == 1
    assert call(H=0) == 1
    assert call(Nf=4097) == 1                    # FASTAR_MAX_ANNCA_QUERIES_PER_FRAME
    assert call(scale=-1.0) == 1
    assert call(scale=float("nan")) == 1
    assert call(qc=None) == 1                    # the query codes buffer is required
    assert call(o=None) == 1
    assert call(q=ctypes.c_void_p(4096 + 8)) == 1  # 16-byte alignment
    assert call(stride=100) == 1                 # strides in whole 16-byte units
    assert "stride" in lib.fastar_last_error().decode()
    assert call(Nf=0) == 0                       # nothing to do
