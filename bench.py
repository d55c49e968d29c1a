"""Benchmark of the TempCache compressed-KV attention step on one MI355X.

A step is one pass of the whole hot path over one chunk of new frames:
SimHash of the chunk's keys, then per frame match -> merge/evict/insert ->
re-hash -> bucket-index rebuild, then attention of the chunk's queries over the
merged cache with the ln(count) bias.

Default workload: one attention layer shaped like a 14B video DiT (40 heads,
d=128, 3600 tokens/frame, chunks of 3 frames = 10800 queries, bf16, SimHash
4 tables x 32 bits, threshold 0.95, 16384 slots/head), cache pre-filled with 21
frames of the drift model (50% exact, 35% perturbed, 15% fresh).  Every timed
step processes the chunk of frames 21-23 on its own copy of the pre-filled
cache, so all steps do identical work; the copies are made before the timed
region and every input is resident in HBM.  The line's `detail` also carries
the 1.3B-layer step, the tiny fp32 step, the 240-frame rollout's per-chunk
latency and memory, and the chunk's hash bits against the CPU oracle.

Prints one JSON line (rank 0).  Other workloads (`--workload`): dit1.3b,
dit1.3b_pq, rollout, annca, annsa, denoise, project, rope, tiny.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def _parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="dit14b",
                   choices=["dit1.3b", "dit1.3b_pq", "dit14b", "rollout", "annca", "annsa",
                            "denoise", "project", "rope", "tiny"])
    p.add_argument("--annsa-bits", type=int, default=16, help="bits per table of the AnnSA buckets")
    p.add_argument("--denoise-steps", type=int, default=4, help="denoising steps per chunk")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--headline-only", action="store_true",
                   help="dit14b: skip the 1.3B-layer step, tiny step and rollout in the detail")
    p.add_argument("--cpu-heads", type=int, default=0,
                   help="heads the CPU oracle times (0 = all for dit1.3b, 2 for dit14b, 1 with PQ codes)")
    p.add_argument("--frames", type=int, default=240, help="rollout length")
    p.add_argument("--measure-traffic", action="store_true",
                   help="run rocprofv3 FETCH_SIZE / WRITE_SIZE passes and record them in profiles/")
    p.add_argument("--out-dir", default=os.path.join(ROOT, "profiles"),
                   help="where --measure-traffic writes its summary")
    p.add_argument("--traffic-child", action="store_true", help=argparse.SUPPRESS)
    p.add_argument("--fenced-events", action="store_true",
                   help="time with torch's default events (system-scope fence at every record)")
    return p.parse_args()


class _HipEvents:
    """Timing events recorded on a HIP stream without a system-scope fence.

    torch's events are created with the default flags, under which every
    record on ROCm also releases to system scope (an L2 write-back across all
    XCDs) and so costs the stream a few microseconds between kernels.  The
    timed step only needs device-side timestamps, so these events are created
    with hipEventDisableSystemFence through the HIP runtime torch has loaded.
    """

    _FLAG_NO_SYSTEM_FENCE = 0x20000000

    def __init__(self, n, stream_handle):
        import ctypes
        self._ct = ctypes
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._stream = ctypes.c_void_p(stream_handle)
        self.ev = []
        for _ in range(n):
            e = ctypes.c_void_p()
            self._check(self._hip.hipEventCreateWithFlags(ctypes.byref(e),
                                                          ctypes.c_uint(self._FLAG_NO_SYSTEM_FENCE)),
                        "hipEventCreateWithFlags")
            self.ev.append(e)

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self, i):
        self._check(self._hip.hipEventRecord(self.ev[i], self._stream), "hipEventRecord")

    def elapsed_ms(self, i, j):
        ms = self._ct.c_float()
        self._check(self._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev[i], self.ev[j]),
                    "hipEventElapsedTime")
        return float(ms.value)

    def close(self):
        for e in self.ev:
            self._hip.hipEventDestroy(e)
        self.ev = []


class _TorchEvents:
    """The same interface over torch.cuda.Event (default flags)."""

    def __init__(self, n, stream):
        import torch
        self._stream = stream
        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]

    def record(self, i):
        self.ev[i].record(self._stream)

    def elapsed_ms(self, i, j):
        return self.ev[i].elapsed_time(self.ev[j])

    def close(self):
        pass


def _events(args, n, stream):
    if args.fenced_events:
        return _TorchEvents(n, stream)
    return _HipEvents(n, stream.cuda_stream)


def _workload_desc(w):
    return {
        "workload": f"{w.name}: {w.heads} heads x d={w.head_dim}, {w.tokens_per_frame} tokens/frame, "
                    f"chunk {w.frames_per_chunk} frames, {w.prefill_frames}-frame prefill, drift "
                    f"{int(w.p_exact*100)}/{int(w.p_pert*100)}/{int(round((1-w.p_exact-w.p_pert)*100))}",
        "heads": w.heads, "head_dim": w.head_dim, "tokens_per_frame": w.tokens_per_frame,
        "frames_per_chunk": w.frames_per_chunk, "queries_per_step": w.chunk_tokens,
        "prefill_frames": w.prefill_frames, "budget_slots": w.budget, "tables": w.tables,
        "bits": w.bits, "threshold": w.threshold, "dtype": w.dtype,
        "codes": (f"product quantization: {w.tables} tables x {w.subspaces} slices x "
                  f"{1 << (w.bits // w.subspaces)} centroids" if w.subspaces
                  else f"SimHash: {w.tables} tables x {w.bits} bits"),
    }


def _cpu_info():
    name = platform.processor() or ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return name


def _oracle_leg(fn, units, unit, what, scale=1.0):
    """Time one call of an oracle function on the host: `units` of the bench
    line's metric per second (a one-head sample counts as 1/H of a query
    token's work, noted through `scale`), for a bench line's cpu_baseline."""
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report what numpy would use
        blas_threads = os.cpu_count() or 1
    t0 = time.perf_counter()
    fn()
    dt = time.perf_counter() - t0
    return {"value": units / dt, "unit": unit, "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{what}; {dt:.2f} s measured{'' if scale == 1.0 else f', counted as {scale:.4g} of the work per query token (one of all heads)'}; "
                      f"float64 numpy on {blas_threads} BLAS threads; host '{_cpu_info()}'"}


def _random_slots(rng, S, d):
    """Slot state of the GPU workload's shape (timing does not depend on values)."""
    return (rng.standard_normal((S, d)), rng.standard_normal((S, d)),
            rng.integers(1, 12, size=S))


def cpu_baseline(w, frames, planes, heads, gpu_codes=None):
    """Time the CPU oracle (as it stands) on one chunk step of `heads` heads.

    With `gpu_codes` ([heads][L][chunk tokens], the library's SimHash codes of
    the chunk's keys), also count the hash bits where they differ from the
    oracle's, split by whether the oracle's float64 projection is below 1e-4
    in magnitude (ambiguous) or not.  Returns (baseline, bit counts or None).
    """
    from oracle import TempCacheOracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas_threads = 1
    hs = list(range(heads))
    orc = TempCacheOracle.for_workload(w, planes, heads=len(hs))
    for f in range(w.prefill_frames):
        K, V, _ = frames[f]
        orc.process_frame(K[hs], V[hs])
        print(f"cpu baseline: prefill frame {f} done", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    Qs, results = [], []
    for f in range(w.prefill_frames, w.prefill_frames + w.frames_per_chunk):
        K, V, Q = frames[f]
        results.append(orc.process_frame(K[hs], V[hs]))
        Qs.append(Q[hs])
    orc.attend(np.concatenate(Qs, axis=1))
    dt = time.perf_counter() - t0
    full = dt * w.heads / len(hs)
    base = {
        "value": w.chunk_tokens / full,
        "unit": "query tokens/s",
        "cores": int(blas_threads),
        "kind": "oracle",
        "sample": (f"one chunk step (frames {w.prefill_frames}-{w.prefill_frames + w.frames_per_chunk - 1}"
                   f" after a {w.prefill_frames}-frame prefill) for {len(hs)} of {w.heads} heads, "
                   f"{dt:.2f} s measured, scaled by {w.heads}/{len(hs)}; hash/match/merge are "
                   f"single-threaded Python loops, attention is float64 numpy matmul on "
                   f"{blas_threads} BLAS threads; host '{_cpu_info()}', "
                   f"{len(os.sched_getaffinity(0))} cores visible"),
    }
    if gpu_codes is None:
        return base, None
    T = w.tokens_per_frame
    total = differ = differ_amb = amb = 0
    for fi, res in enumerate(results):
        for h in hs:
            fr = res[h]
            got = gpu_codes[h][:, fi * T:(fi + 1) * T].T.astype(np.uint64)   # [T][L]
            want = fr.codes.astype(np.uint64)
            ambig = np.abs(fr.proj) < 1e-4                                   # [T][L][b]
            for j in range(w.bits):
                bit = np.uint64(1) << np.uint64(j)
                dif = ((got & bit) != (want & bit))
                a = ambig[:, :, j]
                total += dif.size
                differ += int(dif.sum())
                differ_amb += int((dif & a).sum())
                amb += int(a.sum())
    return base, {"heads_checked": len(hs), "tokens_per_head": w.chunk_tokens,
                  "bits_compared": total, "ambiguous_bits": amb,
                  "differing_bits": differ, "differing_ambiguous": differ_amb,
                  "differing_not_ambiguous": differ - differ_amb,
                  "rule": "bits may differ only where the oracle's float64 |projection| < 1e-4"}


ATTEND_SRC = os.path.join(ROOT, "kv_cache_attention_tempcache_amd", "csrc", "attend.hip")
CALIB_BYTES = 1 << 30   # plain device copy used to scale the HBM counters


def _attend_src_hash() -> str:
    """Hash of the attention source's code: // comments and blank lines are
    left out, so a comment edit keeps a traffic record valid."""
    import hashlib
    with open(ATTEND_SRC, encoding="utf-8") as f:
        code = [ln.split("//", 1)[0].rstrip() for ln in f]
    return hashlib.sha256("\n".join(ln for ln in code if ln).encode()).hexdigest()[:16]


def _traffic_path(workload: str, out_dir: str | None = None) -> str:
    return os.path.join(out_dir or os.path.join(ROOT, "profiles"),
                        f"attend_traffic_{workload}.txt")


def _load_traffic(workload: str):
    """Measured HBM bytes per attend launch, if taken on the current kernel."""
    path = _traffic_path(workload)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        for line in f:
            if line.startswith("RESULT "):
                rec = json.loads(line[len("RESULT "):])
                if rec.get("attend_src_sha256_16") == _attend_src_hash():
                    return rec
    return None


def _build_step_caches(fa, torch, w, nrep):
    """The prefilled cache, its copies, and the chunk inputs of the timed step."""
    from synth import DriftStream
    st = DriftStream(w)
    planes = st.planes()
    n_frames = w.prefill_frames + w.frames_per_chunk
    frames = []
    for _ in range(n_frames):
        K, V, Q, _ = st.next_frame()
        frames.append((K, V, Q))
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()  # noqa: E731
    T, F = w.tokens_per_frame, w.frames_per_chunk
    cfg = fa.CacheConfig(w.heads, w.head_dim, w.budget, w.tables, w.bits, w.threshold, w.dtype,
                         w.subspaces)
    base = fa.Cache(cfg, planes)
    for c0 in range(0, w.prefill_frames, F):
        n = min(F, w.prefill_frames - c0)
        kd = dev(np.concatenate([frames[f][0] for f in range(c0, c0 + n)], axis=1))
        vd = dev(np.concatenate([frames[f][1] for f in range(c0, c0 + n)], axis=1))
        base.match_merge(kd, vd, T, n)
    chunk = [dev(np.concatenate([frames[f][i] for f in range(w.prefill_frames, n_frames)], axis=1))
             for i in range(3)]
    torch.cuda.synchronize()
    caches = []
    for _ in range(nrep):
        c = fa.Cache(cfg, planes)
        c.workspace.copy_(base.workspace)
        caches.append(c)
    torch.cuda.synchronize()
    return base, caches, chunk, frames, planes


def traffic_child(args, fa, torch):
    """Workload profiled by the counter passes: one plain copy, then steps."""
    from synth import WORKLOADS
    w = WORKLOADS[args.workload]
    src = torch.empty(CALIB_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    _, caches, (ck, cv, cq), _, _ = _build_step_caches(fa, torch, w, 3)
    out = torch.empty_like(cq)
    for c in caches:
        c.match_merge(ck, cv, w.tokens_per_frame, w.frames_per_chunk)
        c.attend(cq, out=out)
    torch.cuda.synchronize()
    print("traffic child done", flush=True)


def measure_traffic(args):
    """Two rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) of traffic_child."""
    import csv
    import subprocess
    import tempfile
    out = {}
    cmds = []
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        d = tempfile.mkdtemp(prefix="fastar_pmc_", dir=os.environ.get("TMPDIR", "/tmp"))
        cmd = ["rocprofv3", "--pmc", counter, "--output-format", "csv", "-d", d, "-o", "pmc", "--",
               sys.executable, os.path.abspath(__file__), "--traffic-child", "--workload",
               args.workload]
        cmds.append(" ".join(cmd[:6] + ["<dir>", "-o", "pmc", "--", "python3", "<repo>/bench.py"]
                             + cmd[12:]))
        subprocess.run(["timeout", "-s", "KILL", "300"] + cmd, check=True, cwd=d)
        rows = []
        for root, _, files in os.walk(d):
            for fn in files:
                if fn.endswith("counter_collection.csv"):
                    with open(os.path.join(root, fn)) as f:
                        rows.extend(csv.DictReader(f))
        copies = [float(r["Counter_Value"]) for r in rows
                  if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == counter]
        att = [float(r["Counter_Value"]) for r in rows
               if "attend_cache_kernel" in r["Kernel_Name"] and r["Counter_Name"] == counter]
        if not copies or not att:
            raise RuntimeError(f"{counter}: no copy or attend dispatches in the counter output")
        kib_copy = max(copies)
        out[counter] = {"copy_kib": kib_copy, "attend_kib_mean": float(np.mean(att)),
                        "attend_dispatches": len(att),
                        "scale": (CALIB_BYTES / 1024.0) / kib_copy}
        # every kernel of the step (merge path included), mean per dispatch
        per = {}
        for r in rows:
            name = r["Kernel_Name"]
            if "fastar::" not in name or r["Counter_Name"] != counter:
                continue
            short = (name.replace("(anonymous namespace)::", "").replace("void ", "")
                     .split("(")[0].split("<")[0].split("::")[-1])
            per.setdefault(short, []).append(float(r["Counter_Value"]))
        out[counter]["kernels_kib_mean"] = {k: float(np.mean(v)) for k, v in per.items()}
        out[counter]["kernels_dispatches"] = {k: len(v) for k, v in per.items()}
    fetch = out["FETCH_SIZE"]["attend_kib_mean"] * 1024 * out["FETCH_SIZE"]["scale"]
    write = out["WRITE_SIZE"]["attend_kib_mean"] * 1024 * out["WRITE_SIZE"]["scale"]
    kernels = {}
    for counter, key in (("FETCH_SIZE", "fetch_bytes"), ("WRITE_SIZE", "write_bytes")):
        for k, kib in out[counter]["kernels_kib_mean"].items():
            kernels.setdefault(k, {})[key] = kib * 1024 * out[counter]["scale"]
            kernels[k]["dispatches"] = out[counter]["kernels_dispatches"][k]
    rec = {"workload": args.workload, "attend_fetch_bytes": fetch, "attend_write_bytes": write,
           "attend_bytes": fetch + write, "counters": out, "kernels": kernels,
           "attend_src_sha256_16": _attend_src_hash()}
    write_traffic(rec, cmds, _traffic_path(args.workload, args.out_dir))
    print(json.dumps(rec), flush=True)


def write_traffic(rec, cmds, path):
    """Summary of the two counter passes, with the RESULT line bench.py reads."""
    out = rec["counters"]
    fetch, write = rec["attend_fetch_bytes"], rec["attend_write_bytes"]
    with open(path, "w") as f:
        f.write(f"# HBM traffic of attend_cache_kernel, workload {rec['workload']}\n")
        f.write("# commands (run from a scratch directory, one counter per pass):\n")
        for c in cmds:
            f.write(f"#   timeout -s KILL 300 {c}\n")
        f.write(f"# produced by: python bench.py --measure-traffic --workload {rec['workload']}\n")
        f.write(f"# scale = {CALIB_BYTES} B plain device copy / its counter reading\n")
        for k, v in out.items():
            f.write(f"# {k}: copy {v['copy_kib']:.0f} KiB, attend mean {v['attend_kib_mean']:.0f} KiB"
                    f" over {v['attend_dispatches']} dispatches, scale {v['scale']:.4f}\n")
        f.write(f"# attend HBM bytes per launch: fetch {fetch:.4g}, write {write:.4g}\n")
        if rec.get("kernels"):
            f.write("# every kernel, mean HBM bytes per dispatch (prefill chunks included):\n")
            for k, v in sorted(rec["kernels"].items()):
                f.write(f"#   {k:24s} fetch {v.get('fetch_bytes', 0):.4g}  write "
                        f"{v.get('write_bytes', 0):.4g}  dispatches {v['dispatches']}\n")
        f.write("RESULT " + json.dumps(rec) + "\n")


def main():
    args = _parse()
    if args.measure_traffic:
        return measure_traffic(args)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the TempCache step "
              "shards by head with no exchange inside the step, and this library runs it on "
              "a single GPU.", file=sys.stderr)
        sys.exit(2)

    import torch

    import kv_cache_attention_tempcache_amd as fa
    from synth import WORKLOADS, DriftStream

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.init()
    fa.library()

    if args.traffic_child:
        return traffic_child(args, fa, torch)
    if args.workload == "rollout":
        return rollout(args, fa, torch)
    if args.workload == "annca":
        return annca(args, fa, torch)
    if args.workload == "annsa":
        return annsa(args, fa, torch)
    if args.workload == "denoise":
        return denoise(args, fa, torch)
    if args.workload == "project":
        return project(args, fa, torch)
    if args.workload == "rope":
        return rope(args, fa, torch)
    if args.workload == "tiny":
        return tiny(args, fa, torch)

    return step_line(args, fa, torch, WORKLOADS[args.workload])


def _measure_step(args, fa, torch, w, steps, warmup):
    """Time `steps` chunk steps of workload `w` (each on its own copy of the
    prefilled cache) after `warmup` untimed ones; returns the measurements."""
    T, F = w.tokens_per_frame, w.frames_per_chunk
    nrep = warmup + steps
    base, caches, (ck, cv, cq), frames, planes = _build_step_caches(fa, torch, w, nrep)
    pre = base.stats()
    out = torch.empty_like(cq)
    torch.cuda.synchronize()

    # HIP events on the launch stream bracket every attention launch; the merge
    # path of step i runs between the end of step i-1 and the start of its
    # attention, so no extra event sits between the steps
    stream = torch.cuda.current_stream()
    ev = _events(args, 2 * nrep, stream)   # 2i: before attention of step i, 2i+1: after

    def step(i):
        c = caches[i]
        c.match_merge(ck, cv, T, F)
        ev.record(2 * i)
        c.attend(cq, out=out)
        ev.record(2 * i + 1)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(warmup, nrep):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    timed = range(warmup, nrep)
    attend_ms = [ev.elapsed_ms(2 * i, 2 * i + 1) for i in timed]
    # (from the second timed step: the first follows the host-side sync)
    merge_ms = [ev.elapsed_ms(2 * i - 1, 2 * i) for i in range(warmup + 1, nrep)]
    ev.close()
    post = caches[-1].stats()
    # every copy did identical work
    assert all(c.stats()["live_slots"] == post["live_slots"] for c in caches[:2])
    ex = caches[-1].export_state()
    n_live = ex["n_live"].astype(np.int64)
    ms_per_step = elapsed * 1e3 / steps
    # attention: algorithmic flops = 4 * Nq * S_h * d summed over heads (QK^T and PV)
    attend_flops = float(4 * w.chunk_tokens * n_live.sum() * w.head_dim)
    attend_avg_s = float(np.mean(attend_ms)) / 1e3
    merged = int(post["merged_tokens"] - pre["merged_tokens"])
    inserted = int(post["inserted_tokens"] - pre["inserted_tokens"])
    r = {
        "qps": w.chunk_tokens * steps / elapsed,
        "ms_per_step": ms_per_step,
        "attend_ms": attend_ms,
        "merge_ms": merge_ms,
        "attend_flops": attend_flops,
        "attend_tflops": attend_flops / attend_avg_s / 1e12,
        # algorithmic HBM bytes of one attend launch: Q and O once, every live
        # slot's K and V rows and its log2-count once per head
        "attend_bytes": float(w.heads * w.chunk_tokens * w.head_dim * 2 * 2 +
                              n_live.sum() * (w.head_dim * 2 * 2 + 4)),
        "n_live": n_live,
        "pre": pre,
        "post": post,
        "merged": merged,
        "inserted": inserted,
        "workspace_mb": caches[0].workspace.numel() / 2**20,
        "frames": frames,
        "planes": planes,
        "chunk_keys": ck,
    }
    del base, caches, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return r


def _step_summary(w, r):
    """The figures of one measured step workload, for the bench line's detail."""
    return {
        "workload": _workload_desc(w)["workload"],
        "query_tokens_per_s": r["qps"],
        "ms_per_step": r["ms_per_step"],
        "attend_ms_mean": float(np.mean(r["attend_ms"])),
        "attend_frac_of_bf16_peak": r["attend_tflops"] / PEAK_BF16_TFLOPS,
        "merge_path_ms_mean": float(np.mean(r["merge_ms"])) if r["merge_ms"] else None,
        "n_live_at_attend": int(r["n_live"].sum()),
        "merged_tokens_per_step": r["merged"],
        "inserted_tokens_per_step": r["inserted"],
        "evicted_slots_per_step": int(r["post"]["evicted_slots"] - r["pre"]["evicted_slots"]),
        "step_roofline_frac": _step_roofline(w, r["merged"], r["inserted"], int(r["n_live"].sum()),
                                             r["ms_per_step"])["frac"],
        "workspace_mb_per_cache": r["workspace_mb"],
    }


def _tiny_step(args, fa, torch, reps=50):
    """Latency of the tiny fp32 step: 4 frames merged one at a time, then the
    fifth frame merged and its 64 queries attending (median over reps, each on
    a copy of the cache after the first four frames)."""
    from synth import WORKLOADS, DriftStream
    w = WORKLOADS["tiny"]
    st = DriftStream(w)
    planes = st.planes()
    cfg = fa.CacheConfig(w.heads, w.head_dim, w.budget, w.tables, w.bits, w.threshold, w.dtype)
    base = fa.Cache(cfg, planes)
    dev = lambda x: torch.from_numpy(x).cuda()  # noqa: E731
    for _ in range(4):
        K, V, _, _ = st.next_frame()
        base.match_merge(dev(K), dev(V), w.tokens_per_frame, 1)
    K, V, Q, _ = st.next_frame()
    k, v, q = dev(K), dev(V), dev(Q)
    caches = []
    for _ in range(reps):
        c = fa.Cache(cfg, planes)
        c.workspace.copy_(base.workspace)
        caches.append(c)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    ev = _events(args, 2 * reps, stream)
    torch.cuda.synchronize()
    for i, c in enumerate(caches):
        ev.record(2 * i)
        c.match_merge(k, v, w.tokens_per_frame, 1)
        c.attend(q, out=out)
        ev.record(2 * i + 1)
    torch.cuda.synchronize()
    us = [1e3 * ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)]
    ev.close()
    res = {"workload": "tiny: 1 head x d=64, 64 tokens/frame, fp32, SimHash 1 x 16 bits, "
                       "threshold 0.98, 256 slots; frame 4 merged, then its 64 queries attend",
           "us_median": float(np.median(us)), "us_p95": float(np.percentile(us, 95)),
           "live_slots": int(caches[0].stats()["live_slots"]), "reps": reps,
           "note": "eager calls: the interval includes the host's enqueue of every launch"}
    res["graph_replay"] = _tiny_graph(args, fa, torch, cfg, planes, base, k, v, q, out,
                                      w.tokens_per_frame, caches[0].stats(), reps)
    return res


def _tiny_graph(args, fa, torch, cfg, planes, base, k, v, q, out_eager, T, stats_eager, reps):
    """The same tiny step captured once as a HIP graph (restore the saved
    workspace, merge the frame, attend) and replayed: the GPU-side latency
    without the host's per-launch enqueue.  Every replay's output and slot
    statistics are compared with the eager run's."""
    try:
        c = fa.Cache(cfg, planes)
        src = base.workspace.clone()
        out = torch.empty_like(out_eager)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                c.workspace.copy_(src)
                c.match_merge(k, v, T, 1)
                c.attend(q, out=out)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            c.workspace.copy_(src)
            c.match_merge(k, v, T, 1)
            c.attend(q, out=out)
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        ev = _events(args, 2 * reps, stream)
        same = True
        for i in range(reps):
            out.zero_()
            ev.record(2 * i)
            g.replay()
            ev.record(2 * i + 1)
            torch.cuda.synchronize()
            same = same and bool(torch.equal(out, out_eager)) and c.stats() == stats_eager
        us = [1e3 * ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(reps)]
        ev.close()
        return {"us_median": float(np.median(us)), "us_p95": float(np.percentile(us, 95)),
                "replays": reps, "replays_equal_eager": same,
                "note": "one graph: workspace restore (device copy of the saved state), merge, attend"}
    except Exception as e:  # reported, not fatal: the eager figure above stands
        return {"error": f"{type(e).__name__}: {e}"}


def _rollout_series(fa, torch, frames_total=240):
    """The 240-frame rollout (1.3B layer shape, 2 %/frame of positions turning
    from static to moving, 8192 slots/head, from an empty cache): per-chunk
    latency of merge + attention against frame index, and memory."""
    from synth import WORKLOADS, DriftStream
    w = WORKLOADS["rollout"].with_(total_frames=frames_total)
    st = DriftStream(w)
    planes = st.planes()
    T, F = w.tokens_per_frame, w.frames_per_chunk
    cfg = fa.CacheConfig(w.heads, w.head_dim, w.budget, w.tables, w.bits, w.threshold, w.dtype)
    cache = fa.Cache(cfg, planes)
    stream = torch.cuda.current_stream()
    n_chunks = w.total_frames // F
    ms, live, evicted = [], [], []
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    out = None
    for i in range(n_chunks):
        ks, vs, qs = [], [], []
        for _ in range(F):
            K, V, Q, _ = st.next_frame()
            ks.append(K)
            vs.append(V)
            qs.append(Q)
        k, v, q = (torch.from_numpy(np.concatenate(x, 1)).to(torch.bfloat16).cuda()
                   for x in (ks, vs, qs))
        if out is None:
            out = torch.empty_like(q)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        cache.match_merge(k, v, T, F)
        cache.attend(q, out=out)
        e1.record(stream)
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1))
        s = cache.stats()
        live.append(int(s["live_slots"]))
        evicted.append(int(s["evicted_slots"]))
    ms = np.array(ms)
    half = len(ms) // 2
    slope = float(np.polyfit(np.arange(half, len(ms)) * F, ms[half:], 1)[0])
    return {"workload": f"rollout: {w.total_frames} frames of the 1.3B layer shape, chunks of {F}, "
                        f"2 %/frame static->moving, {w.budget} slots/head, from empty",
            "chunk_ms": [round(float(x), 4) for x in ms],
            "live_slots": live, "evicted_slots_cumulative": evicted,
            "ms_mean_first_half": float(ms[:half].mean()),
            "ms_mean_second_half": float(ms[half:].mean()),
            "ms_slope_per_frame_second_half": slope,
            "workspace_mb": cache.workspace.numel() / 2**20,
            "max_memory_allocated_mb": torch.cuda.max_memory_allocated() / 2**20}


def step_line(args, fa, torch, w):
    """The bench line of a step workload (the 14B layer by default)."""
    r = _measure_step(args, fa, torch, w, args.steps, args.warmup)
    n_live = r["n_live"]
    res = {
        "metric": "query tokens/s per compressed-KV attention step",
        "value": r["qps"],
        "unit": "query tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": r["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded drift-model frames; no dataset or trained weights)",
        "config": _workload_desc(w),
        "roofline": {
            "bound": "mfma",
            "kernel": "attend_cache_kernel",
            "achieved": r["attend_tflops"],
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": r["attend_tflops"] / PEAK_BF16_TFLOPS,
            "traffic": None,
            "algorithmic_bytes": r["attend_bytes"],
        },
        "detail": {
            "attend_ms_mean": float(np.mean(r["attend_ms"])),
            "attend_ms_p95": float(np.percentile(r["attend_ms"], 95)),
            "merge_path_ms_mean": float(np.mean(r["merge_ms"])) if r["merge_ms"] else None,
            "step_ms_median_events": (float(np.median(np.array(r["attend_ms"][1:]) +
                                                      np.array(r["merge_ms"])))
                                      if r["merge_ms"] else None),
            "n_live_after_prefill": int(r["pre"]["live_slots"]),
            "n_live_at_attend": int(n_live.sum()),
            "n_live_per_head_mean": float(n_live.mean()),
            "merged_tokens_per_step": r["merged"],
            "inserted_tokens_per_step": r["inserted"],
            "evicted_slots_per_step": int(r["post"]["evicted_slots"] - r["pre"]["evicted_slots"]),
            "attend_gflop_per_step": r["attend_flops"] / 1e9,
            "step_roofline": _step_roofline(w, r["merged"], r["inserted"], int(n_live.sum()),
                                            r["ms_per_step"]),
            "workspace_mb_per_cache": r["workspace_mb"],
            "timing_events": ("torch default (system fence)" if args.fenced_events
                              else "hipEventDisableSystemFence"),
        },
        "context": "pages report end-to-end only: FAST-AR 5-10x vs dense FlashAttention-3 with "
                   "constant memory; LIPAR 1.45x (NVIDIA A6000); not comparable to this step",
    }
    tr = _load_traffic(args.workload)
    if tr is not None:
        res["roofline"]["traffic"] = tr["attend_bytes"]
    if args.workload == "dit14b" and not args.headline_only:
        from synth import WORKLOADS
        w13 = WORKLOADS["dit1.3b"]
        r13 = _measure_step(args, fa, torch, w13, args.steps, args.warmup)
        res["detail"]["dit1.3b_step"] = _step_summary(w13, r13)
        del r13
        print("bench: 1.3B-layer step done", file=sys.stderr, flush=True)
        res["detail"]["tiny_f32_step"] = _tiny_step(args, fa, torch)
        res["detail"]["rollout_240"] = _rollout_series(fa, torch)
        print("bench: rollout done", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline:
        heads = args.cpu_heads or (1 if w.subspaces else w.heads if w.heads <= 12 else 2)
        gpu_codes = None
        if not w.subspaces:
            # the codes the library's hash kernel gives the chunk's keys, for
            # the heads the oracle runs (the same kernel hashes inside
            # match_merge when no codes are passed)
            ck = r["chunk_keys"][:heads].contiguous()
            pl = torch.from_numpy(np.asarray(r["planes"])).to(torch.bfloat16).cuda().contiguous()
            gpu_codes = fa.hash_codes(ck, pl, w.tables, w.bits).cpu().numpy().view(np.uint32)
        base, bits = cpu_baseline(w, r["frames"], r["planes"], heads, gpu_codes)
        res["cpu_baseline"] = base
        if bits is not None:
            res["detail"]["hash_bits_vs_oracle"] = bits
    print(json.dumps(res), flush=True)


def _step_roofline(w, merged, inserted, live_slots, step_ms):
    """Time one step needs at the roofline: for every kernel the larger of its
    algorithmic flops over the bf16 MFMA peak and its algorithmic bytes over
    the HBM peak, summed over the step's launches; and that over the measured
    step time.  Bytes per unit (storage bf16, fp32 masters): hash 2d + 4L per
    new key; match 4d + 4L + 8 per token (its key, codes, one candidate row,
    the decision); plan 16 per token; apply 24d + 16 + 4L per merged token
    and 16d + 16 + 4L per inserted one (inputs, masters read and written,
    mirrors, counters, codes); index 12 per live slot and table plus the
    bucket offsets; attend Q and O once, every live slot's K, V and shift once.
    The index and attend terms use the live count at attend time (an upper
    bound for the earlier frames)."""
    d, L, H, F, T = w.head_dim, w.tables, w.heads, w.frames_per_chunk, w.tokens_per_frame
    nb = 6
    while (1 << nb) * 4 < w.budget:
        nb += 1
    hbm = PEAK_HBM_GBS * 1e9
    mfma = PEAK_BF16_TFLOPS * 1e12
    nbytes = {
        "hash": H * F * T * (2 * d + 4 * L),
        "match": H * F * T * (4 * d + 4 * L + 8),
        "plan": H * F * T * 16,
        "apply": merged * (24 * d + 16 + 4 * L) + inserted * (16 * d + 16 + 4 * L),
        "index": F * (live_slots * L * 12 + H * L * ((1 << nb) + 1) * 4),
        "attend": H * F * T * d * 2 * 2 + live_slots * (d * 2 * 2 + 4),
    }
    flops = {"hash": 2 * d * L * w.bits * H * F * T, "attend": 4 * F * T * live_slots * d}
    us = {k: max(b / hbm, flops.get(k, 0) / mfma) * 1e6 for k, b in nbytes.items()}
    total = sum(us.values())
    return {"bound_us": {k: round(v, 2) for k, v in us.items()}, "bound_us_total": total,
            "measured_us": step_ms * 1e3, "frac": total / (step_ms * 1e3),
            "algorithmic_bytes": nbytes}


def annca(args, fa, torch):
    """AnnCA cross-attention step: hash queries, select prompt tokens per frame,
    attend over the kept ones, in two launches (fastar_annca_attend: hash, then
    attention with the selection in its prologue) and in three (hash, select,
    subset attention); timed against dense cross-attention (all prompt tokens)
    through the same attention kernel."""
    from synth import ClusterPrompt
    cp = ClusterPrompt()
    H, d, F = cp.heads, cp.head_dim, cp.frames
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).cuda()  # noqa: E731
    q, kp, vp = dev(cp.Q), dev(cp.Kp), dev(cp.Vp)
    planes = dev(cp.planes())
    p_codes = fa.hash_codes(kp, planes, cp.tables, cp.bits)  # the fixed prompt, hashed once
    q_codes = torch.empty((H, cp.tables, q.shape[1]), dtype=torch.int32, device="cuda")
    sel_idx = torch.empty((H, F, kp.shape[1]), dtype=torch.int32, device="cuda")
    sel_cnt = torch.empty((H, F), dtype=torch.int32, device="cuda")
    o_sparse, o_dense = torch.empty_like(q), torch.empty_like(q)

    def sparse():
        fa.hash_codes(q, planes, cp.tables, cp.bits, out=q_codes)
        fa.annca_select(q_codes, p_codes, F, sel_idx, sel_cnt)
        fa.attend_subset(q, kp, vp, F, sel_idx, sel_cnt, out=o_sparse)

    def dense():
        fa.attend_subset(q, kp, vp, F, out=o_dense)

    o_fused = torch.empty_like(q)

    def fused():
        fa.annca_attend(q, planes, cp.tables, cp.bits, p_codes, kp, vp, F, out=o_fused,
                        q_codes=q_codes)

    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in (("sparse", sparse), ("dense", dense), ("fused", fused)):
        for _ in range(args.warmup):
            fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.steps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record(stream)
            fn()
            e1.record(stream)
        torch.cuda.synchronize()
        ms = np.array([e0.elapsed_time(e1) for e0, e1 in ev])
        res[name] = {"ms_median": float(np.median(ms)), "ms_p95": float(np.percentile(ms, 95)),
                     "query_tokens_per_s": q.shape[1] / (float(np.median(ms)) / 1e3)}
    # the one-launch step computes exactly what the three launches do
    assert torch.equal(o_fused, o_sparse)
    # accuracy of the sparse step against dense attention, and the dense
    # probability mass of the dropped prompt tokens (float32 reference)
    kept = sel_cnt.float().mean().item() / kp.shape[1]
    err = (o_sparse.float() - o_dense.float()).abs().max().item()
    qf = q.float().view(H, F, -1, d)
    logits = torch.matmul(qf, kp.float().transpose(1, 2).contiguous().unsqueeze(1)) / d ** 0.5
    prob = torch.softmax(logits, dim=-1)                      # [H][F][q][Np]
    keep = torch.zeros((H, F, kp.shape[1]), device="cuda")
    for hh in range(H):
        for ff in range(F):
            n = int(sel_cnt[hh, ff])
            keep[hh, ff, sel_idx[hh, ff, :n].long()] = 1.0
    dropped = (prob * (1.0 - keep.unsqueeze(2))).sum(-1)     # [H][F][q]
    line = {
        "metric": "query tokens/s per AnnCA cross-attention step",
        "value": res["fused"]["query_tokens_per_s"], "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["fused"]["ms_median"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded clustered prompt; no dataset or trained weights)",
        "config": {"workload": f"annca: {H} heads x d={d}, {F} frames x {cp.queries_per_frame} "
                               f"queries, {kp.shape[1]}-token prompt ({cp.clusters} clusters), "
                               f"{cp.tables} x {cp.bits}-bit codes"},
        "detail": {"fused": res["fused"], "three_launches": res["sparse"], "dense": res["dense"],
                   "speedup_vs_dense": res["dense"]["ms_median"] / res["fused"]["ms_median"],
                   "three_launches_vs_dense": res["dense"]["ms_median"] / res["sparse"]["ms_median"],
                   "kept_fraction": kept, "max_abs_sparse_vs_dense": err,
                   "dropped_dense_mass_max": dropped.max().item(),
                   "dropped_dense_mass_mean": dropped.mean().item()},
    }
    print(json.dumps(line), flush=True)


def annsa(args, fa, torch):
    """AnnSA at the 1.3B layer: after the timed chunk is merged, its 4680
    queries attend only to the slots that share a bucket with them (4 tables
    x --annsa-bits bits, hyperplanes of their own); the step is hashing the
    queries, hashing and indexing the slot keys and the bucket-restricted
    attention, timed against the dense step's attention over all live slots."""
    from synth import WORKLOADS, make_planes
    w = WORKLOADS["dit1.3b"]
    base, _, (ck, cv, cq), _, _ = _build_step_caches(fa, torch, w, 0)
    base.match_merge(ck, cv, w.tokens_per_frame, w.frames_per_chunk)
    H, d, Nq = w.heads, w.head_dim, cq.shape[1]
    L, b = 4, args.annsa_bits
    pl = torch.from_numpy(make_planes(np.random.default_rng(2024), L, b, d, "bf16")).to(
        torch.bfloat16).cuda().contiguous()
    q_codes = torch.empty((H, L, Nq), dtype=torch.int32, device="cuda")
    k_codes = torch.empty((H, L, w.budget), dtype=torch.int32, device="cuda")
    o_sparse, o_dense = torch.empty_like(cq), torch.empty_like(cq)
    fa.hash_codes(cq, pl, L, b, out=q_codes)
    base.hash_slots(pl, L, b, out=k_codes)

    def step():
        fa.hash_codes(cq, pl, L, b, out=q_codes)
        base.hash_slots(pl, L, b)
        base.annsa_attend(cq, q_codes, out=o_sparse)

    def kernel_only():
        base.annsa_attend(cq, q_codes, out=o_sparse)

    def dense():
        base.attend(cq, out=o_dense)

    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in (("step", step), ("annsa_attend", kernel_only), ("dense", dense)):
        for _ in range(args.warmup):
            fn()
        ev = _events(args, 2 * args.steps, stream)
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev.record(2 * i)
            fn()
            ev.record(2 * i + 1)
        torch.cuda.synchronize()
        ms = np.array([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)])
        ev.close()
        res[name] = {"ms_median": float(np.median(ms)), "ms_p95": float(np.percentile(ms, 95))}
    # how sparse the mask is: shared slots per query, queries with none, and
    # the dense probability mass the shared slots carry (heads 0 and 1)
    n_live = base.export_state()["n_live"]
    shared_mean, none_frac, kept_mass = [], [], []
    for h in range(H):
        S = int(n_live[h])
        qc, kc = q_codes[h], k_codes[h, :, :S]
        m = (qc[:, :, None] == kc[:, None, :]).any(0)                  # [Nq][S]
        shared_mean.append(m.sum(1).float().mean().item())
        none_frac.append((m.sum(1) == 0).float().mean().item())
        if h < 2:
            st = base.export_state()
            kf = torch.from_numpy((st["k_mirror"][h, :S].astype(np.uint32) << 16).view(np.float32)).cuda()
            lc = torch.from_numpy(np.log(st["count"][h, :S].astype(np.float64))).float().cuda()
            logits = cq[h].float() @ kf.T.contiguous() / d ** 0.5 + lc
            kept_mass.append((torch.softmax(logits, -1) * m).sum(1).mean().item())
    dense_flops = float(4 * Nq * n_live.astype(np.int64).sum() * d)
    line = {
        "metric": "query tokens/s per AnnSA attention step",
        "value": Nq / (res["step"]["ms_median"] / 1e3), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["step"]["ms_median"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded drift-model frames; no dataset or trained weights)",
        "config": {"workload": f"annsa: {H} heads x d={d}, {Nq} queries over the merged "
                               f"1.3B-layer cache, {L} x {b}-bit buckets"},
        "detail": {"step": res["step"], "annsa_attend": res["annsa_attend"], "dense_attend": res["dense"],
                   "attend_speedup_vs_dense": res["dense"]["ms_median"] / res["annsa_attend"]["ms_median"],
                   "step_speedup_vs_dense": res["dense"]["ms_median"] / res["step"]["ms_median"],
                   "shared_slots_per_query": float(np.mean(shared_mean)),
                   "shared_fraction": float(np.mean(shared_mean) / n_live.mean()),
                   "queries_without_shared_slot": float(np.mean(none_frac)),
                   "dense_mass_kept_mean_heads01": float(np.mean(kept_mass)),
                   "dense_equivalent_tflops": dense_flops / (res["annsa_attend"]["ms_median"] / 1e3) / 1e12},
    }
    if not args.no_cpu_baseline:
        from oracle import annsa as oannsa
        rng = np.random.default_rng(10)
        S = int(n_live.mean())
        kh, vh, cnt = _random_slots(rng, S, d)
        cqs = rng.integers(0, 1 << b, size=(Nq, L)).astype(np.uint32)
        cks = rng.integers(0, 1 << b, size=(S, L)).astype(np.uint32)
        q = rng.standard_normal((Nq, d))
        line["cpu_baseline"] = _oracle_leg(
            lambda: oannsa.annsa_attend(q, kh, vh, cnt, cqs, cks), Nq / H, "query tokens/s",
            f"AnnSA of the {Nq} queries of one head over {S} slots, {L} x {b}-bit codes", scale=1.0 / H)
    print(json.dumps(line), flush=True)


def denoise(args, fa, torch):
    """A chunk through its denoising loop at the 1.3B layer: each of
    --denoise-steps steps attends the chunk's 4680 queries over the compressed
    past (the cache before the chunk) plus the chunk's 4680 current tokens
    (count 1), whose noise falls linearly to zero at the last step; then the
    clean chunk is hashed and merged.  One step of this workload is the whole
    chunk: S attention launches and one merge path."""
    from synth import WORKLOADS, denoising_steps
    w = WORKLOADS["dit1.3b"]
    S = args.denoise_steps
    T, F = w.tokens_per_frame, w.frames_per_chunk
    nrep = args.warmup + args.steps
    base, caches, (ck, cv, cq), frames, _ = _build_step_caches(fa, torch, w, nrep)
    chunk = [np.concatenate([frames[f][i] for f in range(w.prefill_frames, len(frames))], axis=1)
             for i in range(3)]
    rng = np.random.default_rng(2025)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()  # noqa: E731
    Ks, Vs, Qs = ([dev(x) for x in denoising_steps(rng, chunk[i], S, 0.5, "bf16")] for i in range(3))
    out = torch.empty_like(cq)
    n_live = base.export_state()["n_live"].astype(np.int64)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    per = S + 2   # before attention 0, after each attention, after the merge
    ev = _events(args, per * nrep, stream)

    def step(i):
        c = caches[i]
        ev.record(per * i)
        for s in range(S):
            c.attend_with_chunk(Qs[s], Ks[s], Vs[s], out=out)
            ev.record(per * i + s + 1)
        c.match_merge(ck, cv, T, F)
        ev.record(per * i + S + 1)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.warmup, nrep):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    timed = range(args.warmup, nrep)
    att = np.array([[ev.elapsed_ms(per * i + s, per * i + s + 1) for s in range(S)] for i in timed])
    merge = np.array([ev.elapsed_ms(per * i + S, per * i + S + 1) for i in timed])
    ev.close()
    Nq = cq.shape[1]
    flops = float(4 * Nq * (n_live.sum() + w.heads * Nq) * w.head_dim)   # QK^T and PV
    att_s = float(np.mean(att)) / 1e3
    tflops = flops / att_s / 1e12
    ms_chunk = elapsed * 1e3 / args.steps
    line = {
        "metric": "query tokens/s per denoising-step attention (compressed past + chunk)",
        "value": S * Nq * args.steps / elapsed, "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_chunk,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded drift-model frames, Gaussian noise on the chunk's tokens; "
                "no dataset or trained weights)",
        "config": {"workload": f"denoise: {w.heads} heads x d={w.head_dim}, {S} denoising steps "
                               f"of {Nq} queries over ~{int(n_live.mean())} slots per head plus "
                               f"{Nq} chunk tokens, then the merge of the clean chunk "
                               f"({F} frames x {T} tokens)"},
        "roofline": {"bound": "mfma", "kernel": "attend_cache_kernel (slots + chunk tiles)",
                     "achieved": tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": tflops / PEAK_BF16_TFLOPS, "traffic": None},
        "detail": {"attend_ms_mean": float(np.mean(att)), "attend_ms_p95": float(np.percentile(att, 95)),
                   "merge_path_ms_mean": float(np.mean(merge)),
                   "chunk_ms": ms_chunk, "generated_tokens_per_s": Nq * args.steps / elapsed,
                   "slots_per_head_mean": float(n_live.mean()), "chunk_tokens": Nq,
                   "attend_gflop_per_step": flops / 1e9},
    }
    if not args.no_cpu_baseline:
        from oracle import denoise as odenoise
        rng = np.random.default_rng(7)
        H, d, n_slots = w.heads, w.head_dim, int(n_live.mean())
        kh, vh, cnt = _random_slots(rng, n_slots, d)
        q = rng.standard_normal((Nq, d))
        kn, vn = rng.standard_normal((Nq, d)), rng.standard_normal((Nq, d))
        line["cpu_baseline"] = _oracle_leg(
            lambda: odenoise.attend_with_chunk(q, kh, vh, cnt, kn, vn), Nq / H,
            "query tokens/s", f"one denoising step of the {Nq} queries of one head over {n_slots} "
            f"slots plus {Nq} chunk tokens, shapes of the GPU workload", scale=1.0 / H)
    print(json.dumps(line), flush=True)


def project(args, fa, torch):
    """The chunk's key projection with the SimHash codes in its epilogue, at
    the 1.3B layer: 4680 tokens of width 1536 through a 1536 x 1536 key weight
    (12 heads x 128), codes of 4 tables x 32 bits; against torch's bf16
    matmul followed by the library's hash kernel on its output."""
    from synth import WORKLOADS, DriftStream
    w = WORKLOADS["dit1.3b"]
    H, d, N, Din = w.heads, w.head_dim, w.chunk_tokens, 1536
    st = DriftStream(w)
    planes = st.planes()
    cfg = fa.CacheConfig(H, d, w.budget, w.tables, w.bits, w.threshold, w.dtype)
    cache = fa.Cache(cfg, planes)
    g = torch.Generator(device="cuda").manual_seed(2026)
    x = torch.randn((N, Din), generator=g, device="cuda").to(torch.bfloat16)
    wt = (torch.randn((H * d, Din), generator=g, device="cuda") / Din ** 0.5).to(torch.bfloat16)
    pl = torch.from_numpy(planes).to(torch.bfloat16).cuda().contiguous()
    k = torch.empty((H, N, d), dtype=torch.bfloat16, device="cuda")
    codes = torch.empty((H, w.tables, N), dtype=torch.int32, device="cuda")
    kk = torch.empty((N, H * d), dtype=torch.bfloat16, device="cuda")
    codes2 = torch.empty_like(codes)

    def fused():
        cache.project_keys(x, wt, k_out=k, codes_out=codes)

    def matmul():
        torch.matmul(x, wt.t(), out=kk)

    def hash_only():
        fa.hash_codes(kk.view(N, H, d).transpose(0, 1), pl, w.tables, w.bits, out=codes2)

    def unfused():
        matmul()
        hash_only()

    stream = torch.cuda.current_stream()
    res = {}
    for name, fn in (("fused", fused), ("unfused", unfused), ("matmul", matmul), ("hash", hash_only)):
        for _ in range(args.warmup):
            fn()
        ev = _events(args, 2 * args.steps, stream)
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev.record(2 * i)
            fn()
            ev.record(2 * i + 1)
        torch.cuda.synchronize()
        ms = np.array([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)])
        ev.close()
        res[name] = {"ms_median": float(np.median(ms)), "ms_p95": float(np.percentile(ms, 95))}
    same_k = bool(torch.equal(k, kk.view(N, H, d).transpose(0, 1)))
    flops = 2.0 * N * Din * H * d
    tf = flops / (res["fused"]["ms_median"] / 1e3) / 1e12
    line = {
        "metric": "tokens/s through the key projection with SimHash codes",
        "value": N / (res["fused"]["ms_median"] / 1e3), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": res["fused"]["ms_median"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (Gaussian tokens and weights; no trained weights)",
        "config": {"workload": f"project: {N} tokens x {Din} -> {H} heads x {d}, "
                               f"{w.tables} x {w.bits}-bit SimHash codes"},
        "roofline": {"bound": "mfma", "kernel": "project_hash_kernel", "achieved": tf,
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_BF16_TFLOPS,
                     "traffic": None},
        "detail": {"fused": res["fused"], "unfused_matmul_then_hash": res["unfused"],
                   "torch_matmul": res["matmul"], "hash_kernel": res["hash"],
                   "speedup_vs_unfused": res["unfused"]["ms_median"] / res["fused"]["ms_median"],
                   "keys_bit_identical_to_torch_matmul": same_k,
                   "gemm_gflop": flops / 1e9},
    }
    if not args.no_cpu_baseline:
        from oracle import project as oproject
        rng = np.random.default_rng(9)
        xs = rng.standard_normal((N, Din))
        ws = rng.standard_normal((H * d, Din)) / Din ** 0.5
        line["cpu_baseline"] = _oracle_leg(
            lambda: oproject.project_keys(xs, ws, H, planes), N, "tokens/s",
            f"projection and codes of the chunk's {N} tokens for all {H} heads")
    print(json.dumps(line), flush=True)


def _rope_rotate(torch, x, frames, d_t, base=10000.0):
    """x [..., n, d] (float32) turned to per-row frames [n] on the first d_t features."""
    p = torch.arange(d_t // 2, device=x.device, dtype=torch.float64)
    ang = frames.to(torch.float64)[:, None] * base ** (-2.0 * p / d_t)[None, :]
    c, s = torch.cos(ang).float(), torch.sin(ang).float()
    out = x.clone()
    a, b = x[..., 0:d_t:2], x[..., 1:d_t:2]
    out[..., 0:d_t:2] = a * c - b * s
    out[..., 1:d_t:2] = a * s + b * c
    return out


def rope(args, fa, torch):
    """The M-degree attention at the 1.3B layer after the timed chunk is merged
    (keys cached without their temporal rotation, the first 32 of 128 features
    rotated by frame): the chunk's 4680 queries, rotated at their own frames,
    attend with m = 1, 2, 4 most recent member rotations per slot; timed
    against the plain step, and compared on heads 0 and 1 with dense attention
    over the uncompressed history, each raw token rotated to its own frame."""
    from synth import WORKLOADS
    w = WORKLOADS["dit1.3b"]
    d_t, H, d = 32, w.heads, w.head_dim
    T, F = w.tokens_per_frame, w.frames_per_chunk
    base, _, (ck, cv, cq), frames, planes = _build_step_caches(fa, torch, w, 0)
    cfg = fa.CacheConfig(w.heads, w.head_dim, w.budget, w.tables, w.bits, w.threshold, w.dtype,
                         0, 4)
    cache = fa.Cache(cfg, planes)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()  # noqa: E731
    for c0 in range(0, len(frames), F):
        n = min(F, len(frames) - c0)
        cache.match_merge(dev(np.concatenate([frames[f][0] for f in range(c0, c0 + n)], axis=1)),
                          dev(np.concatenate([frames[f][1] for f in range(c0, c0 + n)], axis=1)), T, n)
    qf = torch.arange(w.prefill_frames, len(frames), device="cuda").repeat_interleave(T)
    q = _rope_rotate(torch, cq.float(), qf, d_t).to(torch.bfloat16)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()
    res = {}
    fns = {"plain": lambda: cache.attend(q, out=out)}
    for m in (1, 2, 4):
        fns[f"m{m}"] = (lambda m=m: cache.attend_rope(q, m, d_t, out=out))
    outs = {}
    for name, fn in fns.items():
        for _ in range(args.warmup):
            fn()
        ev = _events(args, 2 * args.steps, stream)
        torch.cuda.synchronize()
        for i in range(args.steps):
            ev.record(2 * i)
            fn()
            ev.record(2 * i + 1)
        torch.cuda.synchronize()
        ms = np.array([ev.elapsed_ms(2 * i, 2 * i + 1) for i in range(args.steps)])
        ev.close()
        res[name] = {"ms_median": float(np.median(ms)), "ms_p95": float(np.percentile(ms, 95))}
        outs[name] = out[:2].float().clone()
    # dense reference on heads 0 and 1: every raw token rotated to its frame
    kf = torch.arange(len(frames), device="cuda").repeat_interleave(T)
    acc = {}
    for h in range(2):
        K = torch.from_numpy(np.concatenate([fr[0][h] for fr in frames])).cuda().float()
        V = torch.from_numpy(np.concatenate([fr[1][h] for fr in frames])).cuda().float()
        Kr = _rope_rotate(torch, K, kf, d_t)
        z = q[h].float() @ Kr.T.contiguous() / d ** 0.5
        ref = torch.softmax(z, -1) @ V
        for name, o in outs.items():
            e = (o[h] - ref).abs()
            acc.setdefault(name, []).append((e.max().item(), e.mean().item()))
    n_live = cache.export_state()["n_live"].astype(np.int64)
    flops = {m: float(4 * cq.shape[1] * n_live.sum() * d * m) for m in (1, 2, 4)}
    best = res["m4"]["ms_median"]
    line = {
        "metric": "query tokens/s per M-degree attention step (m = 4)",
        "value": cq.shape[1] / (best / 1e3), "unit": "query tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": best,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded drift-model frames, temporal rotation on 32 of 128 features)",
        "config": {"workload": f"rope: {H} heads x d={d}, {cq.shape[1]} queries over "
                               f"~{int(n_live.mean())} slots per head, m = 1, 2, 4 member rotations"},
        "roofline": {"bound": "mfma", "kernel": "attend_cache_kernel (regions), m = 4",
                     "achieved": flops[4] / (best / 1e3) / 1e12, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops[4] / (best / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
                     "traffic": None},
        "detail": {"times": res,
                   "max_abs_err_vs_dense_rotated_heads01": {k: max(a for a, _ in v) for k, v in acc.items()},
                   "mean_abs_err_vs_dense_rotated_heads01": {k: float(np.mean([b for _, b in v]))
                                                             for k, v in acc.items()},
                   "slots_per_head_mean": float(n_live.mean())},
    }
    if not args.no_cpu_baseline:
        from oracle import rope as orope
        rng = np.random.default_rng(8)
        S = int(n_live.mean())
        kh, vh, cnt = _random_slots(rng, S, d)
        fr = [list(range(24, 24 - 4, -1))] * S
        q = rng.standard_normal((cq.shape[1] // 10, d))
        line["cpu_baseline"] = _oracle_leg(
            lambda: orope.mdegree_attend(q, kh, vh, cnt, fr, 4, d_t), (cq.shape[1] // 10) / H,
            "query tokens/s", f"M-degree attention (m = 4) of {cq.shape[1] // 10} queries (every "
            f"10th) of one head over {S} slots, shapes of the GPU workload", scale=1.0 / H)
    print(json.dumps(line), flush=True)


def tiny(args, fa, torch):
    """The tiny fp32 step alone (one frame merged, then its 64 queries attend),
    eager and as one replayed HIP graph; latency-bound, so no roofline."""
    r = _tiny_step(args, fa, torch, reps=max(args.steps, 20))
    line = {
        "metric": "query tokens/s per tiny fp32 step (merge of one frame, then its queries attend)",
        "value": 64 / (r["us_median"] / 1e6), "unit": "query tokens/s", "n_gpus": 1,
        "steps": r["reps"], "warmup": 0, "ms_per_step": r["us_median"] / 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded drift-model frames)",
        "config": {"workload": r["workload"]},
        "detail": r,
    }
    print(json.dumps(line), flush=True)


def rollout(args, fa, torch):
    """Stream `--frames` frames chunk by chunk through one cache (from empty)."""
    from synth import WORKLOADS, DriftStream

    w = WORKLOADS["rollout"].with_(total_frames=args.frames)
    st = DriftStream(w)
    planes = st.planes()
    T, F = w.tokens_per_frame, w.frames_per_chunk
    cfg = fa.CacheConfig(w.heads, w.head_dim, w.budget, w.tables, w.bits, w.threshold, w.dtype,
                         w.subspaces)
    cache = fa.Cache(cfg, planes)
    dev = lambda x: torch.from_numpy(x).to(torch.bfloat16).cuda()  # noqa: E731
    chunks = []
    for c0 in range(0, w.total_frames, F):
        ks, vs, qs = [], [], []
        for _ in range(F):
            K, V, Q, _ = st.next_frame()
            ks.append(K)
            vs.append(V)
            qs.append(Q)
        chunks.append((dev(np.concatenate(ks, 1)), dev(np.concatenate(vs, 1)),
                       dev(np.concatenate(qs, 1))))
    out = torch.empty_like(chunks[0][2])
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in chunks]
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    rows = []
    for i, (k, v, q) in enumerate(chunks):
        evs[i][0].record(stream)
        cache.match_merge(k, v, T, F)
        cache.attend(q, out=out)
        evs[i][1].record(stream)
        torch.cuda.synchronize()
        s = cache.stats()
        rows.append({"chunk": i, "frames": [i * F, i * F + F - 1],
                     "ms": evs[i][0].elapsed_time(evs[i][1]), "live_slots": s["live_slots"],
                     "evicted_slots": s["evicted_slots"], "merged_tokens": s["merged_tokens"],
                     "inserted_tokens": s["inserted_tokens"],
                     "max_memory_allocated_mb": torch.cuda.max_memory_allocated() / 2**20})
    ms = np.array([r["ms"] for r in rows])
    half = len(ms) // 2
    slope = float(np.polyfit(np.arange(half, len(ms)) * F, ms[half:], 1)[0])
    print(json.dumps({"workload": "rollout", "frames": w.total_frames, "chunks": rows,
                      "ms_mean_second_half": float(ms[half:].mean()),
                      "ms_slope_per_frame_second_half": slope,
                      "workspace_mb": cache.workspace.numel() / 2**20}), flush=True)


if __name__ == "__main__":
    main()
