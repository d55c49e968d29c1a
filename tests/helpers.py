"""Helpers shared by the GPU parity tests: conversions between the oracle's
state arrays and the library's export format, and tolerant code comparison."""

from __future__ import annotations

import numpy as np
import torch

from oracle import TempCacheOracle, simhash


def to_device(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.cuda()


def mirror_to_f32(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Library mirror export (uint16 bf16 bits or float32) as float32 values."""
    if dtype == "bf16":
        return (arr.astype(np.uint32) << 16).view(np.float32)
    return arr.astype(np.float32)


def oracle_codes_for_device(codes_per_head) -> torch.Tensor:
    """[H] x [T][L] uint32 oracle codes -> int32 device tensor [H][L][T]."""
    c = np.stack([np.asarray(x, dtype=np.uint32).T for x in codes_per_head])
    return torch.from_numpy(np.ascontiguousarray(c).view(np.int32)).cuda()


def oracle_state_for_import(orc: TempCacheOracle, dtype: str) -> dict:
    st = orc.state()
    if dtype == "bf16":
        km = (st["k_hat"].view(np.uint32) >> 16).astype(np.uint16)
        vm = (st["v_hat"].view(np.uint32) >> 16).astype(np.uint16)
    else:
        km, vm = st["k_hat"], st["v_hat"]
    return {
        "k_master": st["K_m"], "v_master": st["V_m"], "k_mirror": km, "v_mirror": vm,
        "count": st["count"].astype(np.int32), "last": st["last"].astype(np.int32),
        "codes": np.ascontiguousarray(st["codes"].transpose(0, 2, 1)),
        "n_live": st["n_live"].astype(np.int32),
        "evicted_tokens": st["evicted_tokens"].astype(np.int64), "frame": st["frame"],
    }


def ambiguous_bit_mask(x: np.ndarray, planes: np.ndarray, tol: float = 1e-4) -> np.ndarray:
    """[n][L] uint32 mask of bits whose float64 projection satisfies |proj| < tol."""
    _, proj = simhash(x, planes)
    amb = np.abs(proj) < tol
    n, L, b = proj.shape
    mask = np.zeros((n, L), dtype=np.uint64)
    for j in range(b):
        mask |= amb[:, :, j].astype(np.uint64) << np.uint64(j)
    return mask.astype(np.uint32)


def code_ambiguity_mask(x: np.ndarray, planes: np.ndarray, subspaces: int) -> np.ndarray:
    """[n][L] uint32 mask of code bits a lower precision may set differently:
    SimHash bits with |proj| < 1e-4, or for product quantization every bit of
    a code whose slice has two centroids at nearly the same distance."""
    if subspaces:
        from oracle.pq import ambiguous_codes
        return np.where(ambiguous_codes(x, planes), np.uint32(0xFFFFFFFF), np.uint32(0))
    return ambiguous_bit_mask(x, planes)


def compare_codes(gpu: np.ndarray, ref: np.ndarray, amb: np.ndarray):
    """Return (#differing bits outside the ambiguity mask, #differing ambiguous bits)."""
    diff = (gpu.astype(np.uint32) ^ ref.astype(np.uint32))
    bad = diff & ~amb
    ok = diff & amb
    popcount = np.vectorize(lambda v: bin(int(v)).count("1"))
    nb = int(popcount(bad).sum()) if bad.any() else 0
    na = int(popcount(ok).sum()) if ok.any() else 0
    return nb, na


def compare_state(gpu: dict, orc: TempCacheOracle, dtype: str, heads=None, codes_amb=None):
    """Assert the exported device state equals the oracle's (bit-exact)."""
    st = orc.state()
    hs = list(range(len(orc.heads))) if heads is None else heads
    for j, h in enumerate(hs):
        n = int(st["n_live"][j])
        assert int(gpu["n_live"][h]) == n, (h, int(gpu["n_live"][h]), n)
        assert int(gpu["evicted_tokens"][h]) == int(st["evicted_tokens"][j])
        np.testing.assert_array_equal(gpu["count"][h, :n], st["count"][j, :n])
        np.testing.assert_array_equal(gpu["last"][h, :n], st["last"][j, :n])
        np.testing.assert_array_equal(gpu["k_master"][h, :n].view(np.uint32),
                                      st["K_m"][j, :n].view(np.uint32))
        np.testing.assert_array_equal(gpu["v_master"][h, :n].view(np.uint32),
                                      st["V_m"][j, :n].view(np.uint32))
        np.testing.assert_array_equal(mirror_to_f32(gpu["k_mirror"][h, :n], dtype).view(np.uint32),
                                      st["k_hat"][j, :n].view(np.uint32))
        np.testing.assert_array_equal(mirror_to_f32(gpu["v_mirror"][h, :n], dtype).view(np.uint32),
                                      st["v_hat"][j, :n].view(np.uint32))
    assert int(gpu["frame"]) == int(st["frame"])
