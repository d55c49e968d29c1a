"""Pins of the CPU oracle against facts fixed outside its own code.

Every check here compares the oracle with something it cannot agree with by
construction: a hand-derived worked example, a closed form (Lemma 5.1, the
SimHash collision law), an independent library routine (torch's attention and
bfloat16 conversion), or a brute-force search written differently from the
oracle's bucketed one.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import HeadCache, TempCacheOracle, bf16_round, simhash
from oracle import annca as oannca
from synth import WORKLOADS, ClusterPrompt, DriftStream


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _cache_from(g, threshold=None):
    return HeadCache(g["head_dim"], g["budget"], g["tables"], g["bits"],
                     g["threshold"] if threshold is None else threshold,
                     g.get("dtype", "f32"), np.array(g["planes"], dtype=np.float64))


def _sdpa(q, k, v, scale=None, mask=None):
    """torch's CPU attention in float64: an independent softmax-attention routine."""
    qt = torch.from_numpy(np.asarray(q, np.float64))[None]
    kt = torch.from_numpy(np.asarray(k, np.float64))[None]
    vt = torch.from_numpy(np.asarray(v, np.float64))[None]
    m = None if mask is None else torch.from_numpy(mask)[None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, scale=scale)
    return out[0].numpy()


# ---------------------------------------------------------------- bfloat16 RNE

def test_bf16_round_hand_values():
    cases = {
        0x3F800000: 0x3F800000,   # 1.0
        0x3F808000: 0x3F800000,   # tie, kept pattern even -> down
        0x3F818000: 0x3F820000,   # tie, kept pattern odd -> up
        0x3F808001: 0x3F810000,   # above the tie -> up
        0x3F807FFF: 0x3F800000,   # below the tie -> down
        0x7F7FFFFF: 0x7F800000,   # largest finite rounds to +inf
        0x80000000: 0x80000000,   # -0.0 stays
    }
    src = np.array(list(cases), dtype=np.uint32).view(np.float32)
    out = bf16_round(src).view(np.uint32)
    assert [int(v) for v in out] == list(cases.values())


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        (rng.standard_normal(1000) * 1e30).astype(np.float32),
                        (rng.standard_normal(1000) * 1e-38).astype(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(bf16_round(x).view(np.uint32), ref.view(np.uint32))


# ---------------------------------------------------------------- SimHash

def test_simhash_basis_golden(golden_dir):
    g = _load(golden_dir, "simhash_basis.json")
    codes, _ = simhash(np.array(g["inputs"]), np.array(g["planes"], dtype=np.float64))
    assert codes.tolist() == g["expected_codes"]


@pytest.mark.parametrize("bits", [8, 16, 32])
@pytest.mark.parametrize("theta", [0.05, 0.3, 1.0, 2.0])
def test_simhash_collision_law(bits, theta):
    """Per table, P[codes equal] = (1 - theta/pi)^bits for random hyperplanes."""
    d, L = 24, 40000
    rng = np.random.default_rng(int(1000 * theta) + bits)
    x = rng.standard_normal(d)
    x /= np.linalg.norm(x)
    u = rng.standard_normal(d)
    u -= (u @ x) * x
    u /= np.linalg.norm(u)
    y = math.cos(theta) * x + math.sin(theta) * u
    planes = rng.standard_normal((L, bits, d))
    codes, _ = simhash(np.stack([x, y]), planes)
    rate = float(np.mean(codes[0] == codes[1]))
    p = (1.0 - theta / math.pi) ** bits
    sigma = math.sqrt(max(p * (1 - p), 1e-12) / L)
    assert abs(rate - p) <= 4 * sigma + 1e-9, (rate, p, sigma)


# ---------------------------------------------------------------- worked examples

def test_lemma_two_slots_golden(golden_dir):
    g = _load(golden_dir, "lemma_two_slots.json")
    hc = _cache_from(g)
    for fr in g["frames"]:
        hc.process_frame(np.array(fr["keys"]), np.array(fr["values"]))
    assert hc.count[:hc.n_live].tolist() == g["expected_count"]
    np.testing.assert_allclose(hc.V_m[:hc.n_live], g["expected_value_slots"], rtol=0, atol=0)
    O, lse = hc.attend(np.array(g["queries"]))
    np.testing.assert_allclose(O, g["expected_output"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, g["expected_lse"], rtol=0, atol=1e-12)


def test_running_mean_golden(golden_dir):
    g = _load(golden_dir, "running_mean.json")
    hc = _cache_from(g)
    for fr in g["frames"]:
        hc.process_frame(np.array(fr["keys"]), np.array(fr["values"]))
    e = g["expected"]
    assert hc.n_live == e["n_live"] and hc.evicted_tokens == e["evicted_tokens"]
    assert hc.K_m[0].tolist() == e["K_m"] and hc.V_m[0].tolist() == e["V_m"]
    assert int(hc.count[0]) == e["count"] and int(hc.last[0]) == e["last"]


def test_threshold_and_ties_golden(golden_dir):
    g = _load(golden_dir, "threshold_and_ties.json")
    hc = _cache_from(g)
    res = [hc.process_frame(np.array(fr["keys"]), np.array(fr["values"])) for fr in g["frames"]]
    e = g["expected"]
    assert res[1].best_slot.tolist() == e["best_slot_frame1"]
    assert res[1].merged.tolist() == e["merged_frame1"]
    assert hc.count[:hc.n_live].tolist() == e["count"] and hc.n_live == e["n_live"]
    assert hc.K_m[0].tolist() == e["K_m_slot0"] and hc.V_m[0].tolist() == e["V_m_slot0"]


def test_lru_eviction_golden(golden_dir):
    g = _load(golden_dir, "lru_eviction.json")
    hc = _cache_from(g)
    res = [hc.process_frame(np.array(fr["keys"]), np.array(fr["values"])) for fr in g["frames"]]
    e = g["expected"]
    assert res[2].slot.tolist() == e["slot_frame2"]
    assert res[2].merged.tolist() == e["merged_frame2"]
    assert res[2].evicted == e["evicted_frame2"]
    assert hc.count[:3].tolist() == e["count"] and hc.last[:3].tolist() == e["last"]
    assert hc.evicted_tokens == e["evicted_tokens"] and hc.n_live == e["n_live"]


def test_rehash_from_mirror_golden(golden_dir):
    """A merge moves the bf16 mirror across a hyperplane: the slot's codes and the
    next frame's candidates follow the mirror, not the master or the old codes."""
    g = _load(golden_dir, "rehash_mirror.json")
    hc = _cache_from(g)
    e = g["expected"]
    res = []
    for f, fr in enumerate(g["frames"]):
        res.append(hc.process_frame(np.array(fr["keys"]), np.array(fr["values"])))
        assert hc.codes[:hc.n_live].tolist() == e["codes_after_frame"][f], f
    assert res[1].merged.tolist() == e["merged_frame1"]
    assert hc.K_m[0].tolist() == e["K_m_slot0"]
    assert hc.k_hat[0].tolist() == e["k_hat_slot0"]
    assert hc.V_m[0].tolist() == e["V_m_slot0"]
    assert res[2].best_slot.tolist() == e["best_slot_frame2"]
    assert res[2].n_candidates.tolist() == e["n_candidates_frame2"]
    assert res[2].merged.tolist() == e["merged_frame2"]
    np.testing.assert_allclose(res[2].best_cos, e["best_cos_frame2"], rtol=0, atol=1e-15)
    assert res[2].slot.tolist() == e["slot_frame2"]
    assert hc.count[:hc.n_live].tolist() == e["count"] and hc.n_live == e["n_live"]


def test_zero_key_golden(golden_dir):
    """A zero-norm key has cosine 0: inserted at threshold 0.95, merged at 0."""
    g = _load(golden_dir, "zero_key.json")
    for case in g["cases"]:
        hc = _cache_from(g, threshold=case["threshold"])
        for f, fr in enumerate(g["frames"][:case["frames"]]):
            r = hc.process_frame(np.array(fr["keys"]), np.array(fr["values"]))
            assert r.best_slot.tolist() == case["best_slot"][f]
            want = [np.nan if c is None else c for c in case["best_cos"][f]]
            np.testing.assert_array_equal(r.best_cos, np.array(want))
            assert r.n_candidates.tolist() == case["n_candidates"][f]
            assert r.merged.tolist() == case["merged"][f]
            assert r.slot.tolist() == case["slot"][f]
        assert hc.count[:hc.n_live].tolist() == case["count"] and hc.n_live == case["n_live"]
        if "K_m_slot0" in case:
            assert hc.K_m[0].tolist() == case["K_m_slot0"]
            assert hc.V_m[0].tolist() == case["V_m_slot0"]
            assert hc.codes[0].tolist() == case["codes_slot0"]


def _codes_by_loops(key, planes):
    """SimHash code of one key with explicit loops over tables, bits and features."""
    L, b, d = planes.shape
    code, margin = [], math.inf
    for t in range(L):
        word = 0
        for j in range(b):
            acc = 0.0
            for k in range(d):
                acc += float(planes[t, j, k]) * float(key[k])
            margin = min(margin, abs(acc))
            if acc > 0.0:
                word |= 1 << j
        code.append(word)
    return code, margin


def test_slot_codes_are_the_mirror_keys_codes_every_frame():
    """After every frame, each live slot's stored codes equal SimHash of its bf16
    mirror key, recomputed here by plain loops (merged slots were re-hashed, the
    inserted ones carry their token's codes, which is the same thing since a new
    slot's mirror is the token's key)."""
    w = WORKLOADS["dit1.3b"].with_(heads=1, tokens_per_frame=96, budget=400, head_dim=64,
                                  tables=2, bits=16)
    st = DriftStream(w)
    planes = np.asarray(st.planes(), dtype=np.float64).reshape(w.tables, w.bits, w.head_dim)
    hc = TempCacheOracle.for_workload(w, st.planes()).heads[0]
    checked_merged = 0
    for f in range(6):
        K, V, _, _ = st.next_frame()
        res = hc.process_frame(K[0], V[0])
        merged_slots = set(res.best_slot[res.merged].tolist())
        for s in range(hc.n_live):
            code, margin = _codes_by_loops(hc.k_hat[s], planes)
            if margin < 1e-9:            # loop and matmul round differently at ~0
                continue
            assert hc.codes[s].tolist() == code, (f, s)
            checked_merged += s in merged_slots
    # the master and the mirror of merged slots differ; the check above must
    # have seen many merged slots, and the masters must hash differently often
    # enough that a re-hash from the master would be caught
    assert checked_merged > 200
    S = hc.n_live
    differs = (simhash(hc.K_m[:S], planes)[0] != simhash(hc.k_hat[:S], planes)[0]).any(axis=1)
    assert differs.sum() >= 1


# ---------------------------------------------------------------- Lemma 5.1

def _run_stream(w, frames, heads=None):
    st = DriftStream(w)
    orc = TempCacheOracle.for_workload(w, st.planes(), heads=heads)
    raw_k, raw_v, last_q = [], [], None
    for _ in range(frames):
        K, V, Q, _ = st.next_frame()
        if heads is not None:
            K, V, Q = K[:heads], V[:heads], Q[:heads]
        orc.process_frame(K, V)
        raw_k.append(K)
        raw_v.append(V)
        last_q = Q
    return orc, np.concatenate(raw_k, axis=1), np.concatenate(raw_v, axis=1), last_q


def test_lemma51_tiny_variant():
    """Exact copies merged with mean values + ln(count) = dense attention (1e-5)."""
    w = WORKLOADS["tiny_lemma"]
    orc, Kr, Vr, Q = _run_stream(w, 5)
    hc = orc.heads[0]
    assert hc.count[:hc.n_live].max() >= 4          # merges really happened
    assert hc.n_live < Kr.shape[1]
    O, _ = hc.attend(Q[0])
    dense = _sdpa(Q[0], Kr[0], Vr[0], scale=1 / math.sqrt(w.head_dim))
    assert np.abs(O - dense).max() < 1e-5


def test_lemma51_two_heads_d128_variant():
    w = WORKLOADS["dit1.3b"].with_(heads=2, tokens_per_frame=256, dtype="f32", p_exact=0.6,
                                  p_pert=0.0, budget=2048, seed=1101)
    orc, Kr, Vr, Q = _run_stream(w, 6)
    for h in range(2):
        hc = orc.heads[h]
        assert hc.count[:hc.n_live].max() >= 5
        O, _ = hc.attend(Q[h])
        dense = _sdpa(Q[h], Kr[h], Vr[h], scale=1 / math.sqrt(128))
        assert np.abs(O - dense).max() < 1e-5


def test_lemma_fails_without_log_count_bias():
    """Sanity of the pin itself: dropping the bias moves the output well past 1e-5."""
    w = WORKLOADS["tiny_lemma"]
    orc, Kr, Vr, Q = _run_stream(w, 5)
    hc = orc.heads[0]
    S = hc.n_live
    nobias = _sdpa(Q[0], hc.k_hat[:S], hc.v_hat[:S], scale=1 / math.sqrt(w.head_dim))
    dense = _sdpa(Q[0], Kr[0], Vr[0], scale=1 / math.sqrt(w.head_dim))
    assert np.abs(nobias - dense).max() > 1e-3


# ---------------------------------------------------------------- attention special cases

def test_no_merge_is_plain_attention():
    """Threshold above 1: nothing merges, every count is 1, attend = plain softmax."""
    w = WORKLOADS["tiny"].with_(threshold=1.5)
    orc, Kr, Vr, Q = _run_stream(w, 3)
    hc = orc.heads[0]
    assert hc.n_live == Kr.shape[1] and (hc.count[:hc.n_live] == 1).all()
    O, _ = hc.attend(Q[0])
    ref = _sdpa(Q[0], Kr[0], Vr[0], scale=1 / math.sqrt(w.head_dim))
    np.testing.assert_allclose(O, ref, rtol=0, atol=1e-12)


def test_softmax_rows_sum_to_one():
    w = WORKLOADS["tiny"]
    orc, Kr, Vr, Q = _run_stream(w, 5)
    hc = orc.heads[0]
    O, lse, P = hc.attend(Q[0], return_probs=True)
    np.testing.assert_allclose(P.sum(axis=1), 1.0, atol=1e-12)
    hc.v_hat[:hc.n_live] = 1.0
    O1, _ = hc.attend(Q[0])
    np.testing.assert_allclose(O1, 1.0, atol=1e-12)
    # lse is the log of the shifted partition function
    S = hc.n_live
    z = Q[0].astype(np.float64) @ hc.k_hat[:S].astype(np.float64).T / 8.0 + np.log(hc.count[:S])
    np.testing.assert_allclose(lse, np.log(np.exp(z).sum(axis=1)), rtol=1e-12)


# ---------------------------------------------------------------- matching

def _snapshot(hc):
    S = hc.n_live
    return hc.k_hat[:S].astype(np.float64).copy(), hc.codes[:S].copy()


def _bruteforce_best(x, keys, allowed):
    """argmax of cosine over allowed rows, computed on normalised matrices."""
    idx = np.flatnonzero(allowed)
    if idx.size == 0:
        return -1, None
    kn = keys[idx] / np.maximum(np.linalg.norm(keys[idx], axis=1, keepdims=True), 1e-300)
    c = kn @ (x / np.linalg.norm(x))
    top = c.max()
    # lowest id among (numerically) equal maxima
    return int(idx[np.flatnonzero(c >= top - 1e-12)[0]]), top


def test_zero_bits_is_bruteforce_top1():
    """b = 0: every live slot shares the single bucket, so match = global top-1."""
    w = WORKLOADS["tiny"].with_(bits=0)
    st = DriftStream(w)
    hc = TempCacheOracle.for_workload(w, st.planes()).heads[0]
    checked = 0
    for _ in range(4):
        K, V, _, _ = st.next_frame()
        keys, _ = _snapshot(hc)
        allowed = np.ones(keys.shape[0], dtype=bool)
        res = hc.process_frame(K[0], V[0])
        for i in range(K.shape[1]):
            b, _ = _bruteforce_best(K[0, i].astype(np.float64), keys, allowed)
            assert res.best_slot[i] == b
            checked += keys.shape[0] > 0
    assert checked > 0


def test_bucketed_match_is_restricted_bruteforce():
    """Match = brute-force top-1 over slots sharing a code in any table."""
    w = WORKLOADS["tiny"].with_(tables=3, bits=6)
    st = DriftStream(w)
    hc = TempCacheOracle.for_workload(w, st.planes()).heads[0]
    found_global = 0
    for _ in range(5):
        K, V, _, cat = st.next_frame()
        keys, codes = _snapshot(hc)
        res = hc.process_frame(K[0], V[0])
        for i in range(K.shape[1]):
            allowed = (codes == res.codes[i][None, :]).any(axis=1)
            assert res.n_candidates[i] == allowed.sum()
            b, _ = _bruteforce_best(K[0, i].astype(np.float64), keys, allowed)
            assert res.best_slot[i] == b
            if keys.shape[0]:
                g, _ = _bruteforce_best(K[0, i].astype(np.float64), keys,
                                        np.ones(keys.shape[0], dtype=bool))
                if allowed[g]:
                    assert res.best_slot[i] == g
                    found_global += 1
    assert found_global > 100


def test_exact_copies_merge():
    w = WORKLOADS["tiny"]
    st = DriftStream(w)
    hc = TempCacheOracle.for_workload(w, st.planes()).heads[0]
    for f in range(5):
        K, V, _, cat = st.next_frame()
        res = hc.process_frame(K[0], V[0])
        if f:
            # an exact copy always finds the slot its source went to (same key
            # bits, so the same codes) and is similar enough to merge
            assert res.merged[cat == 0].all()
            assert (res.best_cos[cat == 0] >= w.threshold).all()


# ---------------------------------------------------------------- merge / evict invariants

def test_conservation_and_contiguity_under_eviction():
    w = WORKLOADS["tiny"].with_(budget=100)
    st = DriftStream(w)
    hc = TempCacheOracle.for_workload(w, st.planes()).heads[0]
    total_evicted = 0
    for f in range(12):
        K, V, _, _ = st.next_frame()
        before_last = hc.last.copy()
        res = hc.process_frame(K[0], V[0])
        assert hc.count[:hc.n_live].sum() + hc.evicted_tokens == hc.tokens_seen
        assert hc.n_live <= hc.B
        assert (hc.count[:hc.n_live] >= 1).all()
        if res.evicted:
            total_evicted += len(res.evicted)
            merged_slots = set(res.best_slot[res.merged].tolist())
            assert not merged_slots & set(res.evicted)
            # evicted = the smallest (last, id) among slots not merged this frame
            elig = sorted((int(before_last[s]), s) for s in range(hc.B) if s not in merged_slots)
            assert sorted(res.evicted) == sorted(s for _, s in elig[:len(res.evicted)])
    assert total_evicted > 0 and hc.n_live == hc.B


def test_member_means_match_masters():
    """fp64 mean over each slot's members equals the fp32 running mean (1e-5 rel)."""
    w = WORKLOADS["tiny"].with_(budget=120)
    st = DriftStream(w)
    hc = TempCacheOracle.for_workload(w, st.planes()).heads[0]
    frames_k, frames_v = [], []
    for _ in range(8):
        K, V, _, _ = st.next_frame()
        frames_k.append(K[0])
        frames_v.append(V[0])
        hc.process_frame(K[0], V[0])
    multi = 0
    for s in range(hc.n_live):
        mem = hc.members[s]
        assert len(mem) == hc.count[s]
        mk = np.mean([frames_k[f][i].astype(np.float64) for f, i in mem], axis=0)
        mv = np.mean([frames_v[f][i].astype(np.float64) for f, i in mem], axis=0)
        scale_k = max(1.0, np.abs(mk).max())
        scale_v = max(1.0, np.abs(mv).max())
        assert np.abs(hc.K_m[s] - mk).max() <= 1e-5 * scale_k
        assert np.abs(hc.V_m[s] - mv).max() <= 1e-5 * scale_v
        multi += len(mem) > 1
    assert multi > 20


def test_bf16_mirror_is_rounded_master():
    w = WORKLOADS["dit1.3b"].with_(heads=1, tokens_per_frame=128, budget=512)
    orc, _, _, _ = _run_stream(w, 4)
    hc = orc.heads[0]
    S = hc.n_live
    ref = torch.from_numpy(hc.K_m[:S]).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(hc.k_hat[:S], ref)


# ---------------------------------------------------------------- AnnCA

def test_annca_selection_bruteforce_pairs():
    rng = np.random.default_rng(3)
    cq = rng.integers(0, 6, size=(40, 3)).astype(np.uint32)
    cp = rng.integers(0, 6, size=(30, 3)).astype(np.uint32)
    sel = oannca.select(cq, cp)
    ref = [j for j in range(30) if any(cp[j, t] == cq[i, t] for i in range(40) for t in range(3))]
    assert sel.tolist() == ref


def test_annca_zero_bits_selects_all_and_equals_dense():
    cp = ClusterPrompt(heads=1, queries_per_frame=64, frames=1, bits=0)
    r = oannca.annca_frame(cp.Q[0], cp.Kp[0], cp.Vp[0], cp.planes())
    assert r["sel"].size == cp.prompt_tokens
    np.testing.assert_array_equal(r["o_sparse"], r["o_dense"])
    ref = _sdpa(cp.Q[0], cp.Kp[0], cp.Vp[0], scale=1 / math.sqrt(128))
    np.testing.assert_allclose(r["o_dense"], ref, atol=1e-12)


def test_annca_sparse_is_masked_dense_and_bounded():
    cp = ClusterPrompt(heads=1, queries_per_frame=200, frames=1)
    r = oannca.annca_frame(cp.Q[0], cp.Kp[0], cp.Vp[0], cp.planes())
    keep = np.zeros(cp.prompt_tokens, dtype=bool)
    keep[r["sel"]] = True
    assert 0 < keep.sum() < cp.prompt_tokens
    mask = np.where(keep, 0.0, -np.inf)[None, :].repeat(200, axis=0)
    ref = _sdpa(cp.Q[0], cp.Kp[0], cp.Vp[0], scale=1 / math.sqrt(128), mask=mask)
    np.testing.assert_allclose(r["o_sparse"], ref, atol=1e-12)
    vmax = np.abs(cp.Vp[0]).max()
    err = np.abs(r["o_sparse"] - r["o_dense"]).max(axis=1)
    assert (err <= 2 * r["delta"] * vmax + 1e-12).all()


# ---------------------------------------------------------------- AnnSA

from oracle import annsa as oannsa  # noqa: E402


def _annsa_case(seed, n_q=60, S=90, d=64, L=3, alphabet=7):
    """Random slot state and codes over a small alphabet (many shared buckets)."""
    rng = np.random.default_rng(seed)
    Q = rng.standard_normal((n_q, d))
    k = rng.standard_normal((S, d))
    v = rng.standard_normal((S, d))
    count = rng.integers(1, 9, size=S)
    cq = rng.integers(0, alphabet, size=(n_q, L)).astype(np.uint32)
    ck = rng.integers(0, alphabet, size=(S, L)).astype(np.uint32)
    return Q, k, v, count, cq, ck


def test_annsa_mask_bruteforce_pairs():
    _, _, _, _, cq, ck = _annsa_case(5)
    mask = oannsa.shared_mask(cq, ck)
    for i in range(cq.shape[0]):
        for s in range(ck.shape[0]):
            assert mask[i, s] == any(cq[i, t] == ck[s, t] for t in range(cq.shape[1]))


def test_annsa_is_masked_sdpa_with_log_count_bias():
    """Equals torch's attention with an additive mask: ln(count) where a bucket
    is shared, -inf elsewhere (queries with no shared bucket give zeros)."""
    Q, k, v, count, cq, ck = _annsa_case(6)
    O, lse, n_shared = oannsa.annsa_attend(Q, k, v, count, cq, ck)
    pairs = np.array([[any(cq[i, t] == ck[s, t] for t in range(cq.shape[1]))
                       for s in range(ck.shape[0])] for i in range(cq.shape[0])])
    assert (n_shared == pairs.sum(axis=1)).all() and 0 < pairs.mean() < 1
    bias = np.where(pairs, np.log(count.astype(np.float64))[None, :], -np.inf)
    rows = pairs.any(axis=1)
    ref = _sdpa(Q[rows], k, v, scale=1 / math.sqrt(Q.shape[1]), mask=bias[rows])
    np.testing.assert_allclose(O[rows], ref, atol=1e-12)
    assert (O[~rows] == 0).all() and np.isneginf(lse[~rows]).all()


def test_annsa_all_shared_is_cache_attention():
    """One common bucket: AnnSA reduces to the dense step over the cache."""
    w = WORKLOADS["tiny"]
    orc, _, _, Q = _run_stream(w, 4)
    hc = orc.heads[0]
    S = hc.n_live
    cq = np.zeros((Q.shape[1], 2), np.uint32)
    ck = np.zeros((S, 2), np.uint32)
    O, lse, _ = oannsa.annsa_attend(Q[0], hc.k_hat[:S], hc.v_hat[:S], hc.count[:S], cq, ck)
    O_ref, lse_ref = hc.attend(Q[0])
    np.testing.assert_allclose(O, O_ref, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_annsa_union_of_tables_closed_form():
    """Slots sharing a bucket in different tables are both attended; with equal
    keys the output is their count-weighted value mean, the rest is ignored."""
    d = 32
    rng = np.random.default_rng(8)
    key = rng.standard_normal(d)
    k = np.stack([key, key, rng.standard_normal(d)])
    v = np.stack([np.full(d, 1.0), np.full(d, 4.0), np.full(d, 1e6)])
    count = np.array([3, 1, 5])
    cq = np.array([[7, 9]], np.uint32)
    ck = np.array([[7, 0], [1, 9], [2, 3]], np.uint32)   # table 0, table 1, none
    O, _, n_shared = oannsa.annsa_attend(key[None], k, v, count, cq, ck)
    assert n_shared[0] == 2
    np.testing.assert_allclose(O[0], (3 * 1.0 + 1 * 4.0) / 4, rtol=0, atol=1e-12)


def test_annsa_single_shared_slot_returns_its_value():
    Q, k, v, count, _, _ = _annsa_case(9, n_q=5, S=20)
    cq = np.arange(5, dtype=np.uint32)[:, None] + 100
    ck = np.full((20, 1), 7, np.uint32)
    ck[[3, 11, 4, 0, 19], 0] = cq[:, 0]          # query i shares only with one slot
    O, lse, n_shared = oannsa.annsa_attend(Q, k, v, count, cq, ck)
    assert (n_shared == 1).all()
    np.testing.assert_array_equal(O, v[[3, 11, 4, 0, 19]])


def test_annsa_slot_order_invariance():
    Q, k, v, count, cq, ck = _annsa_case(10)
    O, lse, _ = oannsa.annsa_attend(Q, k, v, count, cq, ck)
    perm = np.random.default_rng(11).permutation(k.shape[0])
    O2, lse2, _ = oannsa.annsa_attend(Q, k[perm], v[perm], count[perm], cq, ck[perm])
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(lse2, lse, atol=1e-12)


# ---------------------------------------------------------------- product quantization

from oracle import pq as opq  # noqa: E402


def test_pq_small_golden(golden_dir):
    g = _load(golden_dir, "pq_small.json")
    codes, _ = opq.pq_codes(np.array(g["inputs"]), np.array(g["codebooks"], dtype=np.float64))
    assert codes.tolist() == g["expected_codes"]


def test_pq_ambiguous_golden(golden_dir):
    g = _load(golden_dir, "pq_ambiguous.json")
    C = np.array(g["codebooks"], dtype=np.float64)
    rows = np.array(g["rows"], dtype=np.float64)
    codes, _ = opq.pq_codes(rows, C)
    assert codes.tolist() == g["expected_codes"]
    assert opq.ambiguous_codes(rows, C).tolist() == g["expected_ambiguous"]


def test_pq_codes_match_scipy_vq():
    """Each slice's index is scipy's nearest-centroid assignment."""
    from scipy.cluster.vq import vq
    rng = np.random.default_rng(21)
    L, M, K, w = 3, 4, 16, 8
    C = rng.standard_normal((L, M, K, w))
    x = rng.standard_normal((200, M * w))
    codes, _ = opq.pq_codes(x, C)
    for t in range(L):
        ref = np.zeros(200, dtype=np.uint64)
        for m in range(M):
            idx, _ = vq(x[:, m * w:(m + 1) * w], C[t, m])
            ref |= idx.astype(np.uint64) << np.uint64(m * 4)
        np.testing.assert_array_equal(codes[:, t], ref.astype(np.uint32))


def test_pq_centroids_map_to_their_index_and_permute():
    rng = np.random.default_rng(22)
    L, M, K, w = 2, 2, 8, 4
    C = rng.standard_normal((L, M, K, w))
    # a row made of centroid (a, b) of table 0's slices codes as a + 8b there
    rows = np.array([np.concatenate([C[0, 0, a], C[0, 1, b]]) for a in range(K) for b in range(K)])
    codes, _ = opq.pq_codes(rows, C)
    np.testing.assert_array_equal(codes[:, 0], [a + K * b for a in range(K) for b in range(K)])
    perm = rng.permutation(K)
    Cp = C.copy()
    Cp[:, 0] = C[:, 0][:, perm]          # permute slice 0's centroids of every table
    x = rng.standard_normal((100, M * w))
    c1, _ = opq.pq_codes(x, C)
    c2, _ = opq.pq_codes(x, Cp)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(c2 & (K - 1), inv[c1 & (K - 1)])
    np.testing.assert_array_equal(c2 >> 3, c1 >> 3)


def test_pq_ties_go_to_the_lower_index():
    C = np.zeros((1, 1, 4, 3))
    C[0, 0, 1] = C[0, 0, 3] = [1.0, 2.0, 3.0]     # duplicate centroids
    C[0, 0, 0] = C[0, 0, 2] = [9.0, 9.0, 9.0]
    codes, gap = opq.pq_codes(np.array([[1.0, 2.0, 3.5]]), C)
    assert codes[0, 0] == 1 and gap[0, 0, 0] == 0.0


def test_lemma51_with_pq_codes():
    """Exact copies share every PQ code, so they merge, and the merged step
    equals dense attention over the raw tokens (Lemma 5.1) as with SimHash."""
    w = WORKLOADS["tiny_lemma"].with_(subspaces=2, bits=8)
    orc, Kr, Vr, Q = _run_stream(w, 5)
    hc = orc.heads[0]
    assert hc.M == 2 and hc.count[:hc.n_live].max() >= 4 and hc.n_live < Kr.shape[1]
    O, _ = hc.attend(Q[0])
    dense = _sdpa(Q[0], Kr[0], Vr[0], scale=1 / math.sqrt(w.head_dim))
    assert np.abs(O - dense).max() < 1e-5


def test_bucketed_match_with_pq_is_restricted_bruteforce():
    w = WORKLOADS["tiny_pq"].with_(tables=2)
    st = DriftStream(w)
    hc = TempCacheOracle.for_workload(w, st.planes()).heads[0]
    checked = 0
    for _ in range(5):
        K, V, _, _ = st.next_frame()
        keys, codes = _snapshot(hc)
        res = hc.process_frame(K[0], V[0])
        np.testing.assert_array_equal(res.codes, opq.pq_codes(K[0], hc.planes)[0])
        for i in range(K.shape[1]):
            allowed = (codes == res.codes[i][None, :]).any(axis=1)
            assert res.n_candidates[i] == allowed.sum()
            b, _ = _bruteforce_best(K[0, i].astype(np.float64), keys, allowed)
            assert res.best_slot[i] == b
            checked += int(allowed.any())
    assert checked > 50


# ---------------------------------------------------------------- denoising loop

from oracle import denoise as odenoise  # noqa: E402


def test_denoise_two_steps_golden(golden_dir):
    g = _load(golden_dir, "denoise_two_steps.json")
    orc = TempCacheOracle(1, g["head_dim"], g["budget"], g["tables"], g["bits"], g["threshold"],
                          "f32", np.array(g["planes"], dtype=np.float64))
    for fr in g["prefill"]:
        orc.process_frame(np.array([fr["keys"]]), np.array([fr["values"]]))
    steps = g["steps"]
    Qs = [np.array([s["q"]]) for s in steps]
    Ks = [np.array([s["k"]]) for s in steps]
    Vs = [np.array([s["v"]]) for s in steps]
    outs, lses, res = odenoise.denoise_chunk(orc, Qs, Ks, Vs, frames=1, scale=g["scale"])
    for s in range(len(steps)):
        np.testing.assert_allclose(outs[s][0], g["expected_output"][s], atol=1e-12)
        np.testing.assert_allclose(lses[s][0], g["expected_lse"][s], atol=1e-12)
    hc = orc.heads[0]
    assert hc.n_live == len(g["expected_after_merge"]["count"])
    np.testing.assert_array_equal(hc.count[:hc.n_live], g["expected_after_merge"]["count"])
    np.testing.assert_allclose(hc.v_hat[:hc.n_live], g["expected_after_merge"]["value"], atol=1e-12)
    assert bool(res[0][0].merged[0])


def _history_with_duplicates(rng, d, n_distinct, T):
    """Raw tokens whose keys repeat exactly (1 to 4 times each), the merged
    slots Lemma 5.1 gives for them, and T fresh chunk tokens."""
    keys = rng.standard_normal((n_distinct, d))
    reps = rng.integers(1, 5, size=n_distinct)
    raw_k = np.repeat(keys, reps, axis=0)
    raw_v = rng.standard_normal((raw_k.shape[0], d))
    owner = np.repeat(np.arange(n_distinct), reps)
    v_hat = np.stack([raw_v[owner == i].mean(axis=0) for i in range(n_distinct)])
    return raw_k, raw_v, keys, v_hat, reps, rng.standard_normal((T, d)), rng.standard_normal((T, d))


def test_attend_with_chunk_lemma51_against_dense_raw_history():
    """Merged slots plus raw chunk tokens equal torch's dense attention over the
    uncompressed history followed by the chunk."""
    rng = np.random.default_rng(21)
    d = 32
    raw_k, raw_v, k_hat, v_hat, count, Kn, Vn = _history_with_duplicates(rng, d, 40, 25)
    Q = rng.standard_normal((17, d))
    O, lse = odenoise.attend_with_chunk(Q, k_hat, v_hat, count, Kn, Vn)
    ref = _sdpa(Q, np.concatenate([raw_k, Kn]), np.concatenate([raw_v, Vn]))
    np.testing.assert_allclose(O, ref, atol=1e-12)
    z = Q @ np.concatenate([raw_k, Kn]).T / math.sqrt(d)
    np.testing.assert_allclose(lse, np.log(np.exp(z).sum(axis=1)), atol=1e-10)


def test_attend_with_chunk_without_chunk_is_cache_attention():
    w = WORKLOADS["tiny"]
    orc, _, _, Q = _run_stream(w, 4)
    hc = orc.heads[0]
    S = hc.n_live
    d = Q.shape[2]
    O, lse = odenoise.attend_with_chunk(Q[0], hc.k_hat[:S], hc.v_hat[:S], hc.count[:S],
                                        np.zeros((0, d)), np.zeros((0, d)))
    O_ref, lse_ref = hc.attend(Q[0])
    np.testing.assert_allclose(O, O_ref, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_attend_with_chunk_on_empty_cache_is_sdpa():
    rng = np.random.default_rng(22)
    d = 16
    Q, Kn, Vn = (rng.standard_normal((n, d)) for n in (9, 30, 30))
    O, _ = odenoise.attend_with_chunk(Q, np.zeros((0, d)), np.zeros((0, d)), np.zeros(0), Kn, Vn)
    np.testing.assert_allclose(O, _sdpa(Q, Kn, Vn), atol=1e-12)
    O0, lse0 = odenoise.attend_with_chunk(Q, np.zeros((0, d)), np.zeros((0, d)), np.zeros(0),
                                          np.zeros((0, d)), np.zeros((0, d)))
    assert (O0 == 0).all() and np.isneginf(lse0).all()


def test_chunk_token_equal_to_a_slot_counts_as_one_more_member():
    """A chunk token with slot s's key and value weighs like count[s] + 1."""
    rng = np.random.default_rng(23)
    d, S = 24, 12
    k = rng.standard_normal((S, d))
    v = rng.standard_normal((S, d))
    count = rng.integers(1, 6, size=S)
    Q = rng.standard_normal((7, d))
    s = 5
    O, lse = odenoise.attend_with_chunk(Q, k, v, count, k[s:s + 1], v[s:s + 1])
    c2 = count.copy()
    c2[s] += 1
    O_ref, lse_ref = odenoise.attend_with_chunk(Q, k, v, c2, np.zeros((0, d)), np.zeros((0, d)))
    np.testing.assert_allclose(O, O_ref, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_attend_with_chunk_is_order_invariant():
    rng = np.random.default_rng(24)
    d = 16
    _, _, k_hat, v_hat, count, Kn, Vn = _history_with_duplicates(rng, d, 20, 33)
    Q = rng.standard_normal((5, d))
    O, _ = odenoise.attend_with_chunk(Q, k_hat, v_hat, count, Kn, Vn)
    ps, pc = rng.permutation(len(count)), rng.permutation(Kn.shape[0])
    O2, _ = odenoise.attend_with_chunk(Q, k_hat[ps], v_hat[ps], count[ps], Kn[pc], Vn[pc])
    np.testing.assert_allclose(O, O2, atol=1e-12)


def test_denoise_chunk_merges_only_the_final_step():
    """The cache after the loop equals a cache that saw only the final step's
    frames; every step attends with the cache as it was before the chunk."""
    w = WORKLOADS["tiny"]
    st = DriftStream(w)
    planes = st.planes()
    a = TempCacheOracle.for_workload(w, planes)
    b = TempCacheOracle.for_workload(w, planes)
    for _ in range(3):
        K, V, _, _ = st.next_frame()
        a.process_frame(K, V)
        b.process_frame(K, V)
    frames = [st.next_frame() for _ in range(2)]
    Kc = np.concatenate([f[0] for f in frames], axis=1)
    Vc = np.concatenate([f[1] for f in frames], axis=1)
    Qc = np.concatenate([f[2] for f in frames], axis=1)
    rng = np.random.default_rng(25)
    noisy = [Kc + s * rng.standard_normal(Kc.shape) for s in (0.5, 0.25)]
    Ks, Vs, Qs = noisy + [Kc], [Vc + 0.3, Vc - 0.1, Vc], [Qc, Qc, Qc]
    before = [(hc.k_hat[:hc.n_live].copy(), hc.v_hat[:hc.n_live].copy(),
               hc.count[:hc.n_live].copy()) for hc in a.heads]
    outs, _, _ = odenoise.denoise_chunk(a, Qs, Ks, Vs, frames=2)
    for f in range(2):
        T = w.tokens_per_frame
        b.process_frame(Kc[:, f * T:(f + 1) * T], Vc[:, f * T:(f + 1) * T])
    for ha, hb in zip(a.heads, b.heads):
        assert ha.n_live == hb.n_live
        np.testing.assert_array_equal(ha.count[:ha.n_live], hb.count[:hb.n_live])
        np.testing.assert_array_equal(ha.k_hat[:ha.n_live], hb.k_hat[:hb.n_live])
    for s in range(3):
        for h, (k, v, c) in enumerate(before):
            O, _ = odenoise.attend_with_chunk(Qs[s][h], k, v, c, Ks[s][h], Vs[s][h])
            np.testing.assert_array_equal(outs[s][h], O)


# ---------------------------------------------------------------- K projection + hash

from oracle import project as oproject  # noqa: E402


def test_round_bf16_exact_hand_values():
    e = 2.0 ** -8
    cases = {
        1.0 + e: 1.0,                       # halfway between 1 and 1 + 2^-7: to even
        1.0 + 3 * e: 1.0 + 4 * e,           # halfway between 1 + 2^-7 and 1 + 2^-6: to even
        1.0 + e + 2.0 ** -30: 1.0 + 2 * e,  # just above halfway
        -(1.0 + e): -1.0,
        3.0: 3.0, 0.0: 0.0,
        255.5: 256.0,                       # 8 significant bits: 255 | 256, halfway to even
        2.0 ** -100 * (1 + 2 * e): 2.0 ** -100 * (1 + 2 * e),
    }
    for v, want in cases.items():
        assert oproject.round_bf16_exact(v) == want, v


def test_round_bf16_exact_matches_torch_on_binary32_values():
    rng = np.random.default_rng(31)
    x = (rng.standard_normal(20000) * np.exp(rng.uniform(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oproject.round_bf16_exact(x.astype(np.float64)), ref)


def test_project_keys_identity_weight_is_the_input():
    rng = np.random.default_rng(32)
    H, d, N = 3, 16, 40
    X = bf16_round(rng.standard_normal((N, H * d)).astype(np.float32))
    planes = bf16_round(rng.standard_normal((2, 8, d)).astype(np.float32)).reshape(2, 8, d)
    K, codes, _ = oproject.project_keys(X, np.eye(H * d), H, planes)
    for h in range(H):
        np.testing.assert_array_equal(K[h], X[:, h * d:(h + 1) * d])
        np.testing.assert_array_equal(codes[h], simhash(X[:, h * d:(h + 1) * d], planes)[0])


def test_project_keys_small_integers_by_loops():
    """Integer inputs small enough for every product and sum to be exact in
    bfloat16: keys and sign bits by plain Python loops."""
    rng = np.random.default_rng(33)
    H, d, Din, N, L, b = 2, 4, 6, 5, 2, 3
    X = rng.integers(-3, 4, size=(N, Din)).astype(np.float64)
    W = rng.integers(-2, 3, size=(H * d, Din)).astype(np.float64)
    P = rng.integers(-2, 3, size=(L, b, d)).astype(np.float64)
    K, codes, _ = oproject.project_keys(X, W, H, P)
    for h in range(H):
        for n in range(N):
            k = [sum(X[n][i] * W[h * d + f][i] for i in range(Din)) for f in range(d)]
            assert list(K[h, n]) == k
            for t in range(L):
                code = 0
                for j in range(b):
                    if sum(P[t][j][f] * k[f] for f in range(d)) > 0:
                        code |= 1 << j
                assert codes[h, n, t] == code


# ---------------------------------------------------------------- rotation-corrected M-degree

from oracle import rope as orope  # noqa: E402


def test_rope_t_closed_forms():
    # one pair, frequency 1: (1, 0) turned by `frame` radians
    for t in (0.0, 0.5, 2.0, -1.25):
        np.testing.assert_allclose(orope.rope_t([1.0, 0.0], t, 2), [math.cos(t), math.sin(t)],
                                   atol=1e-15)
    rng = np.random.default_rng(41)
    x = rng.standard_normal((6, 16))
    y = orope.rope_t(x, 7, 10)
    np.testing.assert_allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-13)
    np.testing.assert_array_equal(y[:, 10:], x[:, 10:])            # untouched features
    np.testing.assert_allclose(orope.rope_t(orope.rope_t(x, 3, 10), 4, 10), y, atol=1e-12)
    # only the frame difference matters: <R(a) q, R(b) k> = <q, R(b - a) k>
    q, k = rng.standard_normal(16), rng.standard_normal(16)
    lhs = orope.rope_t(q, 5, 10) @ orope.rope_t(k, 11, 10)
    np.testing.assert_allclose(lhs, q @ orope.rope_t(k, 6, 10), atol=1e-12)


def _static_cache(rng, d, d_t, frames=4, static=6, fresh=5):
    """Frames whose first `static` tokens repeat exactly (key and value), plus
    fresh tokens; returns the oracle cache and the raw (rotated) history."""
    hc = HeadCache(d, 64, 1, 4, 0.98, "f32", rng.standard_normal((1, 4, d)))
    sk = rng.standard_normal((static, d)).astype(np.float32)
    sv = rng.standard_normal((static, d)).astype(np.float32)
    raw_k, raw_v = [], []
    for f in range(frames):
        K = np.concatenate([sk, rng.standard_normal((fresh, d)).astype(np.float32)])
        V = np.concatenate([sv, rng.standard_normal((fresh, d)).astype(np.float32)])
        hc.process_frame(K, V)
        raw_k.append(orope.rope_t(K, f, d_t))
        raw_v.append(V)
    return hc, np.concatenate(raw_k), np.concatenate(raw_v)


def test_mdegree_with_every_member_is_dense_attention_over_rotated_tokens():
    """Static tokens (identical key and value in every frame) merge; with m at
    least their count the approximation is exact: dense attention (torch) over
    the raw tokens, each rotated to its own frame."""
    rng = np.random.default_rng(42)
    d, d_t = 32, 16
    hc, rk, rv = _static_cache(rng, d, d_t)
    n = hc.n_live
    assert hc.count[:n].max() == 4 and n < rk.shape[0]
    Q = orope.rope_t(rng.standard_normal((9, d)), 4, d_t)
    fr = orope.recent_frames(hc, 4)
    O, lse = orope.mdegree_attend(Q, hc.k_hat[:n], hc.v_hat[:n], hc.count[:n], fr, 4, d_t)
    np.testing.assert_allclose(O, _sdpa(Q, rk, rv), atol=1e-12)
    z = Q @ rk.T / math.sqrt(d)
    np.testing.assert_allclose(lse, np.log(np.exp(z).sum(axis=1)), atol=1e-12)
    # with m = 1 it is not exact (the static slots' rotations differ by frame)
    O1, _ = orope.mdegree_attend(Q, hc.k_hat[:n], hc.v_hat[:n], hc.count[:n], fr, 1, d_t)
    assert np.abs(O1 - O).max() > 1e-3


def test_mdegree_without_rotation_is_the_cache_step():
    rng = np.random.default_rng(43)
    hc, _, _ = _static_cache(rng, 32, 16)
    n = hc.n_live
    Q = rng.standard_normal((7, 32))
    O_ref, lse_ref = hc.attend(Q)
    for m in (1, 2, 3, 4):
        O, lse = orope.mdegree_attend(Q, hc.k_hat[:n], hc.v_hat[:n], hc.count[:n],
                                      orope.recent_frames(hc, m), m, 0)
        np.testing.assert_allclose(O, O_ref, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, atol=1e-12)


def test_mdegree_one_is_log_count_attention_at_the_last_rotation():
    rng = np.random.default_rng(44)
    d, d_t = 32, 16
    hc, _, _ = _static_cache(rng, d, d_t)
    n = hc.n_live
    Q = rng.standard_normal((7, d))
    last = np.array([hc.members[s][-1][0] for s in range(n)])
    rk = np.stack([orope.rope_t(hc.k_hat[s], last[s], d_t) for s in range(n)])
    bias = np.broadcast_to(np.log(hc.count[:n].astype(np.float64)), (7, n)).copy()
    O, _ = orope.mdegree_attend(Q, hc.k_hat[:n], hc.v_hat[:n], hc.count[:n],
                                orope.recent_frames(hc, 1), 1, d_t)
    np.testing.assert_allclose(O, _sdpa(Q, rk, hc.v_hat[:n], mask=bias), atol=1e-12)


def test_mdegree_depends_on_frame_differences_only():
    rng = np.random.default_rng(45)
    d, d_t = 32, 16
    hc, _, _ = _static_cache(rng, d, d_t)
    n = hc.n_live
    Qh = rng.standard_normal((5, d))
    fr = orope.recent_frames(hc, 3)
    O, _ = orope.mdegree_attend(orope.rope_t(Qh, 4, d_t), hc.k_hat[:n], hc.v_hat[:n],
                                hc.count[:n], fr, 3, d_t)
    shifted = [[f + 9 for f in fs] for fs in fr]
    O2, _ = orope.mdegree_attend(orope.rope_t(Qh, 13, d_t), hc.k_hat[:n], hc.v_hat[:n],
                                 hc.count[:n], shifted, 3, d_t)
    np.testing.assert_allclose(O, O2, atol=1e-12)


def test_recent_frames_most_recent_first():
    rng = np.random.default_rng(46)
    hc, _, _ = _static_cache(rng, 16, 8, frames=5, static=2, fresh=1)
    fr = orope.recent_frames(hc, 3)
    assert fr[0] == [4, 3, 2] and fr[1] == [4, 3, 2]       # static slots: a member per frame
    assert hc.count[0] == 5
