"""The allocation-free AnnCA entry point against the pair it replaces.

fastar_annca_attend_static keeps the per-frame selection in the library's
static device array; its output must equal fastar_annca_select followed by
fastar_attend_subset on the same inputs, call after call (the array keeps the
previous call's selection, so a second, smaller call must not see it).
"""

import numpy as np
import pytest
import torch

import kv_cache_attention_tempcache_amd as fa
from synth import ClusterPrompt
from tests.helpers import to_device

pytestmark = pytest.mark.gpu


def _inputs(heads, frames, qpf, dtype, seed_bits=16):
    cp = ClusterPrompt(heads=heads, queries_per_frame=qpf, frames=frames, bits=seed_bits,
                       dtype=dtype)
    q = to_device(cp.Q, dtype)
    kp, vp = to_device(cp.Kp, dtype), to_device(cp.Vp, dtype)
    pl = torch.from_numpy(np.ascontiguousarray(cp.planes())).to(q.dtype).cuda().contiguous()
    qc = fa.hash_codes(q, pl, cp.tables, cp.bits)
    pc = fa.hash_codes(kp, pl, cp.tables, cp.bits)
    return q, kp, vp, qc, pc


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_static_annca_equals_select_then_subset_attention(dtype):
    # the second call is smaller in every dimension that sizes the selection
    for heads, frames, qpf in ((12, 3, 1560), (2, 2, 300)):
        print(f"static AnnCA: {dtype} heads={heads} frames={frames} queries/frame={qpf}", flush=True)
        q, kp, vp, qc, pc = _inputs(heads, frames, qpf, dtype)
        sel, cnt = fa.annca_select(qc, pc, frames)
        ref = fa.attend_subset(q, kp, vp, frames, sel, cnt)
        got = fa.annca_attend_static(q, qc, kp, vp, pc, frames)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)
        kept = cnt.cpu().numpy()
        assert (kept > 0).all() and (kept < kp.shape[1]).all()


def test_static_annca_refuses_sizes_beyond_its_array():
    q, kp, vp, qc, pc = _inputs(2, 1, 64, "bf16")
    H, Np = 2, kp.shape[1]
    # 4096 segments: H*F over the limit with one query per frame
    F = 2049
    qbig = torch.zeros((H, F, q.shape[2]), dtype=q.dtype, device="cuda")
    qcb = torch.zeros((H, qc.shape[1], F), dtype=torch.int32, device="cuda")
    with pytest.raises(fa.FastarError):
        fa.annca_attend_static(qbig, qcb, kp, vp, pc, F)
