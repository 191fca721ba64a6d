"""Benchmark of one decode step over a PQ-coded KV cache on one MI355X.

A step is the whole hot path for one layer and one new token, in one launch
(pq_attn_decode_step):
  1. the new token's K and V vectors (B*Hkv each) are encoded by nearest
     codeword straight into the code cache, at position lens[b]-1;
  2. lookup-table build, code streaming, chunk softmax, V histograms and
     codebook contraction -> per-chunk (m, l, o);
  3. the last workgroup of each (request, KV head) merges the chunks -> out.
The same step through three launches (pq_encode_many, pq_attn_partials,
pq_attn_reduce) is timed too and reported under "detail".
The headline workload is the GQA decode shape (B=8, Hq=64, Hkv=8, L=8192,
M=8, K=256).  Inputs live in HBM before timing starts; N seeded replicas of
every input are rotated so that the working set (>= 512 MiB) is twice the
256 MB Infinity Cache and each step reads its codes from HBM.

Further legs in the same line: "workloads" (the step on every workload:
tiny, page-sizing, gqa, long-splitk, ragged), "long_context" (chunk 2048 and
the library's chunk), "paged", "fp8" (the plain decode with FP8 codebooks
next to fp16 ones), "encode", "kmeans" and "stream_reference" (a read-only
streaming kernel and device copies of the step's size and of 512 MiB: what
one launch reaches on the same box), and "cpu_baselines" (the oracle on
every workload).

Prints one JSON line.  `value` = KV tokens scanned per second over the timed
steps (sum of lens per step / step time).  `roofline` is the step kernel's
algorithmic bytes per launch over its average duration in the timed region
(the step is one launch, so that is the time per step between HIP events
around K back-to-back steps).  `cpu_baseline` is the CPU oracle on the same
workload (repeated for 10+ s), on the host cores.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
WORKLOAD_IDS = {"tiny": 1, "page-sizing": 2, "gqa": 3, "long-splitk": 4, "ragged": 5}


def algorithmic_bytes(w, lens, step=True):
    """What the method must move for one decode step: the valid K and V codes,
    both codebooks once per KV head, q (fp16) and out (fp32); with the new
    token appended, also its K and V vectors (fp16) in and their codes out."""
    codes = int(np.sum(lens)) * w.n_kv_heads * 2 * w.n_sub
    cbs = w.n_kv_heads * 2 * w.n_sub * w.n_codes * w.sub_dim * 2
    q = w.batch * w.n_q_heads * w.head_dim * 2
    out = w.batch * w.n_q_heads * w.head_dim * 4
    new = w.batch * w.n_kv_heads * 2 * (w.head_dim * 2 + w.n_sub) if step else 0
    return codes + cbs + q + out + new


class HipEvents:
    """Raw hipEvent_t handles from the process's HIP runtime (the one torch
    loaded), for pq_attn_partials_timed, which has the runtime stamp them at
    the score kernel's own start and end."""

    def __init__(self):
        import ctypes
        path = next(l.split()[-1] for l in open("/proc/self/maps") if "libamdhip64" in l)
        self.hip = ctypes.CDLL(path)
        self.ct = ctypes
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = self.ct.c_void_p()
            if self.hip.hipEventCreate(self.ct.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            out.append(h.value)
        return out

    def elapsed_ms(self, a, b):
        f = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_partials_gqa_traffic.json")
KERNEL_SOURCE = os.path.join(ROOT, "decode_attention_product_amd", "csrc", "decode_kernel.hpp")


def kernel_source_hash():
    import hashlib
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()


def stored_traffic():
    """HBM bytes per score-kernel launch from the committed counter runs, or
    None when the kernel source changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


def _repeat(fn, min_seconds, max_seconds):
    """Run fn until min_seconds have passed (or the next run would pass
    max_seconds); returns (runs, seconds)."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        fn()
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el + el / reps > max_seconds:
            return reps, el


def _blas_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return 1


def _one_thread():
    try:
        from threadpoolctl import threadpool_limits
        return threadpool_limits(1)
    except Exception:
        import contextlib
        return contextlib.nullcontext()


def cpu_baseline(wid, min_seconds=10.0, max_seconds=30.0, single_thread=False):
    """The oracle's whole decode step on workload wid (every KV head), repeated
    for min_seconds.  Its NumPy elementwise work is single-threaded; its
    matrix-vector products run on the BLAS threads (`cores`), or on one with
    single_thread."""
    import oracle
    from synth import gen
    inp = gen.workload_inputs(wid, with_encode=False)
    args = [inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")]
    tokens = int(inp["lens"].sum())
    import contextlib
    with (_one_thread() if single_thread else contextlib.nullcontext()):
        cores = 1 if single_thread else _blas_threads()
        reps, el = _repeat(lambda: oracle.decode_attention(*args), min_seconds, max_seconds)
    return {"value": tokens * reps / el, "unit": "KV tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{gen.WORKLOADS[wid].name} workload, whole decode step, repeated {reps}x "
                      f"({el:.1f} s); elementwise NumPy on one thread, BLAS on {cores}"}


def cpu_baselines(seconds=3.0):
    """The oracle beside every workload, on bounded samples of a few seconds
    each: the whole decode step of the tiny, page-sizing and ragged workloads
    (the first two also on one thread), one KV head of the long-context one
    (scaled to KV tokens: a token is one cached step of all 8 KV heads), and
    the ragged prefill's encode on a 500-token sample of K vectors."""
    import oracle
    from synth import gen
    res = {}
    for wid in (1, 2):
        name = gen.WORKLOADS[wid].name
        res[name] = cpu_baseline(wid, seconds, 4 * seconds)
        res[name + " (1 thread)"] = cpu_baseline(wid, seconds, 4 * seconds, single_thread=True)
    w = gen.WORKLOADS[4]
    inp = gen.workload_inputs(4, with_encode=False)
    G = w.group
    args = (inp["q"][:, :G], inp["k_codes"][:, :1], inp["v_codes"][:, :1], inp["k_cb"][:1],
            inp["v_cb"][:1], inp["lens"])
    reps, el = _repeat(lambda: oracle.decode_attention(*args), seconds, 4 * seconds)
    head_tokens = int(inp["lens"].sum())
    res[w.name] = {"value": head_tokens * reps / el / w.n_kv_heads, "unit": "KV tokens/s",
                   "cores": _blas_threads(), "kind": "oracle",
                   "sample": f"KV head 0 and its {G} query heads over {head_tokens} tokens, "
                             f"repeated {reps}x ({el:.1f} s); scaled by 1/{w.n_kv_heads} KV heads"}
    res["ragged"] = cpu_baseline(5, seconds, 4 * seconds)
    w = gen.WORKLOADS[5]
    rng = gen.rng_for(5)
    cb = gen.codebooks(rng, w.n_kv_heads, w.n_sub, w.n_codes, w.sub_dim)
    x, _ = gen.noisy_codewords(rng, cb, 500, w.encode_sigma)
    reps, el = _repeat(lambda: oracle.encode(x, cb), seconds, 4 * seconds)
    n = x.shape[0] * x.shape[1]
    res["ragged prefill encode"] = {
        "value": n * reps / el, "unit": "vectors/s", "cores": _blas_threads(), "kind": "oracle",
        "sample": f"{n} K vectors (500 tokens x {w.n_kv_heads} heads) of the ragged prefill, "
                  f"repeated {reps}x ({el:.1f} s)"}
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="gqa", choices=sorted(WORKLOAD_IDS))
    ap.add_argument("--replicas", type=int, default=0, help="0: enough for 512 MiB")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--chunk", type=int, default=0)
    ap.add_argument("--no-encode", action="store_true", help="skip the prefill-encode leg")
    ap.add_argument("--encode-reps", type=int, default=5)
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache leg")
    ap.add_argument("--paged-steps", type=int, default=500)
    ap.add_argument("--no-kmeans", action="store_true", help="skip the codebook-learning leg")
    ap.add_argument("--no-long", action="store_true", help="skip the long-context step leg")
    ap.add_argument("--no-stream", action="store_true", help="skip the streaming references")
    ap.add_argument("--no-workloads", action="store_true", help="skip the per-workload step legs")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-codebook leg")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="also run 3 device copies of this many MiB (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this library has no "
              "multi-GPU path; see the sharding notes in DESIGN.md.", file=sys.stderr)
        sys.exit(2)

    import torch
    import decode_attention_product_amd as pq
    from synth import gen

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    pq.load_library()
    wid = WORKLOAD_IDS[args.workload]
    w = gen.WORKLOADS[wid]
    if w.prefill_encode:
        print("the ragged workload's decode step is benchmarked without its prefill", file=sys.stderr)
    dev = torch.device("cuda:0")
    B, Hq, Hkv, L, M, D = w.batch, w.n_q_heads, w.n_kv_heads, w.max_len, w.n_sub, w.head_dim

    base = gen.workload_inputs(wid, with_encode=False)
    per_rep = sum(base[k].nbytes for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb"))
    R = args.replicas or max(2, math.ceil((512 << 20) / per_rep))
    reps = []
    for r in range(R):
        inp = base if r == 0 else gen.workload_inputs(wid, replica=r, with_encode=False)
        rng = np.random.default_rng([7000 + wid, r])
        xk, _, xv, _ = gen.step_tokens(rng, inp["k_cb"], inp["v_cb"], B)
        t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
             for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")}
        t["xk"] = torch.from_numpy(xk).to(dev)
        t["xv"] = torch.from_numpy(xv).to(dev)
        lens = inp["lens"].astype(np.int64)
        slots = np.arange(B, dtype=np.int64) * Hkv * L + np.maximum(lens - 1, 0)
        t["slots"] = torch.from_numpy(slots).to(dev)
        reps.append(t)
    lens_np = base["lens"]
    tokens_per_step = int(lens_np.sum())

    desc = pq.attn_desc(reps[0]["q"], reps[0]["k_codes"], reps[0]["k_cb"], chunk=args.chunk)
    C = pq.pq_attn_num_chunks(desc)
    enc_desc = pq.cache_encode_desc(B, B, Hkv, L, n_sub=M)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    pm = torch.empty((B, Hq, C), dtype=torch.float32, device=dev)
    pl = torch.empty((B, Hq, C), dtype=torch.float32, device=dev)
    po = torch.empty((B, Hq, C, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    ws = pq.step_workspace(desc, dev)       # zero-filled once; every step leaves it so

    def step(t, ev=None):
        pq.pq_attn_decode_step(t["q"], t["xk"], t["xv"], t["k_codes"], t["v_codes"], t["k_cb"],
                               t["v_cb"], t["lens"], out, desc=desc, workspace=ws, stream=stream,
                               events=ev)

    def step_three_launches(t):
        pq.pq_encode_many([t["xk"], t["xv"]], [t["k_cb"], t["v_cb"]], [t["k_codes"], t["v_codes"]],
                          slots=t["slots"], desc=enc_desc, stream=stream)
        pq.pq_attn_partials(t["q"], t["k_codes"], t["v_codes"], t["k_cb"], t["v_cb"], t["lens"],
                            desc=desc, part_m=pm, part_l=pl, part_o=po, stream=stream)
        pq.pq_attn_reduce(pm, pl, po, out, stream=stream)

    for i in range(args.warmup):
        step(reps[i % R])
        step_three_launches(reps[i % R])
    torch.cuda.synchronize()

    K = args.steps
    # (a) the timed region: K whole steps; the runtime stamps a pair of events
    # at each step kernel's own start and end
    hip = HipEvents()
    raw = hip.create(2 * K)
    evs = [(raw[2 * i], raw[2 * i + 1]) for i in range(K)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record(stream)
    t0 = time.perf_counter()
    for i in range(K):
        step(reps[i % R], evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = start.elapsed_time(end) / K
    kern_ms = [hip.elapsed_ms(a, b) for a, b in evs]
    hip.destroy(raw)
    score_ms = float(np.mean(kern_ms))

    # (b) the same steps without the per-kernel events (the throughput figure)
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step(reps[i % R])
    end.record(stream)
    torch.cuda.synchronize()
    step_ms_plain = start.elapsed_time(end) / K

    # (c) the same step as three launches, for comparison
    torch.cuda.synchronize()
    start.record(stream)
    for i in range(K):
        step_three_launches(reps[i % R])
    end.record(stream)
    torch.cuda.synchronize()
    step_ms_three = start.elapsed_time(end) / K

    value = tokens_per_step / (step_ms_plain * 1e-3)
    alg = algorithmic_bytes(w, lens_np)
    # the step is one launch: its average duration in the timed region is the
    # time per step between the events around K back-to-back steps
    achieved = alg / (step_ms_plain * 1e-3) / 1e9

    result = {
        "metric": "PQ-KV decode attn: KV tokens scanned/s + % of HBM peak GB/s; encode vectors/s",
        "value": value,
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": step_ms_plain,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 in / fp32 compute",
        "data": "synthetic (seeded generators; codebooks and q fp16 N(0,1), codes uniform uint8)",
        "config": {"workload": f"{w.name}: B={B} Hq={Hq} Hkv={Hkv} L={L} D={D} M={M} K={w.n_codes}",
                   "chunk": int(desc.chunk) or "library", "n_chunks": C, "replicas": R,
                   "step": "one launch: encode new K and V into the cache, attend, merge chunks"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": stored_traffic(),
                     "kernel": "decode_partials_kernel (decode-step variant)", "algorithmic_bytes": alg,
                     "avg_launch_us": step_ms_plain * 1e3,
                     "avg_launch_us_kernel_events": score_ms * 1e3},
        "detail": {"step_us_with_kernel_events": step_ms * 1e3, "step_us": step_ms_plain * 1e3,
                   "step_kernel_us_p50": float(np.median(kern_ms)) * 1e3,
                   "step_us_three_launches": step_ms_three * 1e3,
                   "wall_s": wall, "tokens_per_step": tokens_per_step},
    }
    if args.copy_probe_mib:
        # a plain device copy of known size, to calibrate FETCH_SIZE/WRITE_SIZE
        n = args.copy_probe_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        result["copy_probe_bytes"] = n
    if not args.no_workloads:
        result["workloads"] = {}
        for wi in (1, 2, 3):
            if wi == wid:
                result["workloads"][w.name] = {
                    "value": value, "unit": "KV tokens/s", "step_us": step_ms_plain * 1e3,
                    "roofline": {"bound": "hbm", "achieved": achieved, "frac": achieved / HBM_PEAK_GBS,
                                 "algorithmic_bytes": alg}}
            else:
                ww = gen.WORKLOADS[wi]
                result["workloads"][ww.name] = step_leg(pq, torch, dev, wi, args.paged_steps,
                                                        args.warmup, chunk=ww.chunk)
    if not args.no_long and wid != 4:
        result["long_context"] = long_context_leg(pq, torch, dev, args.paged_steps, args.warmup)
        if "workloads" in result:
            lc = result["long_context"]
            result["workloads"]["long-splitk"] = {
                k: lc[k] for k in ("workload", "chunk", "n_chunks", "value", "unit", "step_us", "roofline")}
    if not args.no_paged:
        result["paged"] = paged_leg(pq, torch, dev, args.paged_steps, args.warmup,
                                    step_ms_plain * 1e3 if wid == 3 else None)
    if not args.no_fp8:
        result["fp8"] = fp8_leg(pq, torch, dev, args.paged_steps, args.warmup)
    if not args.no_encode:
        result["encode"] = encode_leg(pq, torch, dev, args.encode_reps)
    if not args.no_kmeans:
        result["kmeans"] = kmeans_leg(pq, torch, dev)
    if not args.no_stream:
        result["stream_reference"] = stream_leg(torch, dev)
    if "paged" in result and "workloads" in result:
        rg = result["paged"]["ragged"]
        result["workloads"]["ragged"] = {
            "value": rg["dense_value"], "unit": "KV tokens/s", "step_us": rg["dense_step_us"],
            "roofline": rg["dense_roofline"], "paged_step_us": rg["step_us"],
            "note": "dense padded cache; the paged step is in paged.ragged"}
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wid)
        result["cpu_baselines"] = cpu_baselines()
    print(json.dumps(result), flush=True)


def to_pages(torch, dense, lens, P, perm):
    """Device gather of a dense code cache [B, Hkv, L, M] into a pool
    [Hkv, n_pages * P, M] of P-token pages: the used pages of every request,
    in the physical order `perm` (logical page i -> physical page perm[i]).
    Returns (pool, block_table int32 [B, L // P], n_pages); table entries
    past a request's pages hold -1."""
    B, Hkv, L, M = dense.shape
    need = [-(-int(x) // P) for x in lens]
    n_pages = sum(need)
    table = np.full((B, L // P), -1, dtype=np.int32)
    src = np.empty(n_pages * P, dtype=np.int64)
    i = 0
    for b in range(B):
        for j in range(need[b]):
            page = int(perm[i])
            table[b, j] = page
            src[page * P:(page + 1) * P] = b * L + j * P + np.arange(P)
            i += 1
    flat = dense.permute(1, 0, 2, 3).reshape(Hkv, B * L, M)
    pool = flat[:, torch.from_numpy(src).to(dense.device)].contiguous()
    return pool, torch.from_numpy(table).to(dense.device), n_pages


def paged_leg(pq, torch, dev, steps, warmup, dense_gqa_us):
    """Decode steps over paged code caches (256-token pages in a seeded
    shuffled order), timed like the headline step: kernel-stamped events for
    the kernel, plain back-to-back steps for the step time.
      gqa     the headline workload on pages (paging overhead vs. dense)
      ragged  64 requests of 512 or 4096 tokens, Lmax 4096, one query head
              per KV head: the paged and the dense (padded) step on the same
              cache (encode kernel + request-batched score kernel), the plain
              decode of both, and the capacity each layout needs."""
    from synth import gen
    P = 256
    stream = torch.cuda.current_stream()
    res = {"page_tokens": P}
    for name, wid in (("gqa", 3), ("ragged", 5)):
        w = gen.WORKLOADS[wid]
        B, Hq, Hkv, L, M, D = w.batch, w.n_q_heads, w.n_kv_heads, w.max_len, w.n_sub, w.head_dim
        base = gen.workload_inputs(wid, with_encode=False)
        lens_np = base["lens"]
        alg = algorithmic_bytes(w, lens_np) + B * (L // P) * 4          # + the block table
        R = max(2, math.ceil((512 << 20) / alg))
        reps = []
        for r in range(R):
            inp = base if r == 0 else gen.workload_inputs(wid, replica=r, with_encode=False)
            rng = np.random.default_rng([7100 + wid, r])
            xk, _, xv, _ = gen.step_tokens(rng, inp["k_cb"], inp["v_cb"], B)
            t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
                 for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")}
            t["xk"], t["xv"] = torch.from_numpy(xk).to(dev), torch.from_numpy(xv).to(dev)
            n_used = sum(-(-int(x) // P) for x in inp["lens"])
            perm = rng.permutation(n_used)
            t["k_pool"], t["table"], n_pages = to_pages(torch, t["k_codes"], inp["lens"], P, perm)
            t["v_pool"], _, _ = to_pages(torch, t["v_codes"], inp["lens"], P, perm)
            if name == "gqa":       # only the pools are read in this leg
                del t["k_codes"], t["v_codes"]
            reps.append(t)
        desc, _ = pq.paged_desc(reps[0]["q"], reps[0]["k_pool"], reps[0]["k_cb"], reps[0]["table"], P)
        ws = pq.step_workspace(desc, dev)
        ws_dense = pq.step_workspace(desc, dev)
        out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)

        def paged(t, ev=None):
            pq.pq_attn_decode_step_paged(t["q"], t["xk"], t["xv"], t["k_pool"], t["v_pool"], t["k_cb"],
                                         t["v_cb"], t["table"], t["lens"], out, page_tokens=P,
                                         workspace=ws, stream=stream, events=ev)

        def dense(t):
            pq.pq_attn_decode_step(t["q"], t["xk"], t["xv"], t["k_codes"], t["v_codes"], t["k_cb"],
                                   t["v_cb"], t["lens"], out, desc=desc, workspace=ws_dense,
                                   stream=stream)

        def timed(fn):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            a.record(stream)
            for i in range(steps):
                fn(reps[i % R])
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) * 1e3 / steps

        for i in range(warmup):
            paged(reps[i % R])
            if name == "ragged":
                dense(reps[i % R])
        hip = HipEvents()
        raw = hip.create(2 * steps)
        torch.cuda.synchronize()
        for i in range(steps):
            paged(reps[i % R], (raw[2 * i], raw[2 * i + 1]))
        torch.cuda.synchronize()
        kern_us = float(np.mean([hip.elapsed_ms(raw[2 * i], raw[2 * i + 1]) for i in range(steps)])) * 1e3
        hip.destroy(raw)
        step_us = timed(paged)
        tokens = int(lens_np.sum())
        achieved = alg / (step_us * 1e-6) / 1e9
        kernel = ("decode_paged_kernel (decode-step variant), one launch" if name == "gqa" else
                  "encode_kernel (new tokens) + decode_mha_kernel (paged), two launches")
        leg = {"workload": f"{w.name}: B={B} Hq={Hq} Hkv={Hkv} Lmax={L} M={M}, {tokens} tokens",
               "value": tokens / (step_us * 1e-6), "unit": "KV tokens/s", "step_us": step_us,
               "events_us": kern_us, "replicas": R,
               "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes": alg,
                            "kernel": kernel},
               "pool_slots_per_head": n_pages * P, "padded_slots_per_head": B * L}
        if name == "gqa" and dense_gqa_us is not None:
            leg["dense_step_us"] = dense_gqa_us
        if name == "ragged":
            leg["dense_step_us"] = timed(dense)
            alg_dense = algorithmic_bytes(w, lens_np)
            ach = alg_dense / (leg["dense_step_us"] * 1e-6) / 1e9
            leg["dense_value"] = tokens / (leg["dense_step_us"] * 1e-6)
            leg["dense_roofline"] = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                                     "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                                     "algorithmic_bytes": alg_dense,
                                     "kernel": "encode_kernel (new tokens) + decode_mha_kernel, "
                                               "two launches"}
            # the plain decode over the same caches (no new token): with one
            # query head per KV head and 2048 pairs it runs the
            # request-batched score kernel
            ws_plain = torch.empty(max(pq.pq_attn_workspace_bytes(desc), 16), dtype=torch.uint8,
                                   device=dev)

            def paged_plain(t):
                pq.pq_attn_decode_paged(t["q"], t["k_pool"], t["v_pool"], t["k_cb"], t["v_cb"],
                                        t["table"], t["lens"], out, page_tokens=P,
                                        workspace=ws_plain, stream=stream)

            def dense_plain(t):
                pq.pq_attn_decode(t["q"], t["k_codes"], t["v_codes"], t["k_cb"], t["v_cb"], t["lens"],
                                  out, desc=desc, workspace=ws_plain, stream=stream)

            for i in range(warmup):
                paged_plain(reps[i % R])
                dense_plain(reps[i % R])
            leg["decode_us"] = timed(paged_plain)
            leg["dense_decode_us"] = timed(dense_plain)
            leg["decode_value"] = tokens / (leg["decode_us"] * 1e-6)
        res[name] = leg
    return res


def long_context_leg(pq, torch, dev, steps, warmup):
    """The decode step on the long-context split-K workload (B=1, Hq=64,
    Hkv=8, L=131072, M=4), timed like the headline step: with the workload's
    chunks of 2048 tokens (64 chunk records per KV head merged in the same
    launch), and with the chunk length the library picks (4096: one
    workgroup per CU)."""
    from synth import gen
    wid = 4
    w = gen.WORKLOADS[wid]
    B, Hq, Hkv, L, M, D = w.batch, w.n_q_heads, w.n_kv_heads, w.max_len, w.n_sub, w.head_dim
    stream = torch.cuda.current_stream()
    base = gen.workload_inputs(wid, with_encode=False)
    lens_np = base["lens"]
    alg = algorithmic_bytes(w, lens_np)
    R = max(2, math.ceil((512 << 20) / alg))
    reps = []
    for r in range(R):
        inp = base if r == 0 else gen.workload_inputs(wid, replica=r, with_encode=False)
        rng = np.random.default_rng([7200 + wid, r])
        xk, _, xv, _ = gen.step_tokens(rng, inp["k_cb"], inp["v_cb"], B)
        t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
             for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")}
        t["xk"], t["xv"] = torch.from_numpy(xk).to(dev), torch.from_numpy(xv).to(dev)
        reps.append(t)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    tokens = int(lens_np.sum())

    def run(chunk):
        desc = pq.attn_desc(reps[0]["q"], reps[0]["k_codes"], reps[0]["k_cb"], chunk=chunk)
        ws = pq.step_workspace(desc, dev)

        def step(t, ev=None):
            pq.pq_attn_decode_step(t["q"], t["xk"], t["xv"], t["k_codes"], t["v_codes"], t["k_cb"],
                                   t["v_cb"], t["lens"], out, desc=desc, workspace=ws, stream=stream,
                                   events=ev)

        for i in range(warmup):
            step(reps[i % R])
        hip = HipEvents()
        raw = hip.create(2 * steps)
        torch.cuda.synchronize()
        for i in range(steps):
            step(reps[i % R], (raw[2 * i], raw[2 * i + 1]))
        torch.cuda.synchronize()
        kern_us = float(np.mean([hip.elapsed_ms(raw[2 * i], raw[2 * i + 1]) for i in range(steps)])) * 1e3
        hip.destroy(raw)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(steps):
            step(reps[i % R])
        b.record(stream)
        torch.cuda.synchronize()
        step_us = a.elapsed_time(b) * 1e3 / steps
        achieved = alg / (step_us * 1e-6) / 1e9
        return {"chunk": chunk,
                "n_chunks": pq.pq_attn_num_chunks(desc),
                "value": tokens / (step_us * 1e-6), "unit": "KV tokens/s", "step_us": step_us,
                "events_us": kern_us,
                "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes": alg,
                             "kernel": "decode_partials_kernel (decode-step variant)"}}

    leg = {"workload": f"{w.name}: B={B} Hq={Hq} Hkv={Hkv} L={L} M={M}", "replicas": R}
    leg.update(run(w.chunk))
    lib = run(0)
    lib["chunk"] = "library"
    leg["library_chunk"] = lib
    return leg


def step_replicas(torch, dev, wid, seed, budget=512 << 20, max_reps=None):
    """Seeded replicas of workload wid's inputs on the device plus each one's
    new-token K and V, enough that they fill `budget` bytes."""
    from synth import gen
    w = gen.WORKLOADS[wid]
    base = gen.workload_inputs(wid, with_encode=False)
    alg = algorithmic_bytes(w, base["lens"])
    R = max(2, math.ceil(budget / alg))
    if max_reps:
        R = min(R, max_reps)
    reps = []
    for r in range(R):
        inp = base if r == 0 else gen.workload_inputs(wid, replica=r, with_encode=False)
        rng = np.random.default_rng([seed + wid, r])
        xk, _, xv, _ = gen.step_tokens(rng, inp["k_cb"], inp["v_cb"], w.batch)
        t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
             for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")}
        t["xk"], t["xv"] = torch.from_numpy(xk).to(dev), torch.from_numpy(xv).to(dev)
        reps.append(t)
    return w, base["lens"], reps


def step_leg(pq, torch, dev, wid, steps, warmup, chunk=0):
    """The one-launch decode step on workload wid, timed as the headline step:
    HIP events around `steps` back-to-back steps over rotated replicas."""
    w, lens_np, reps = step_replicas(torch, dev, wid, 7400)
    R = len(reps)
    stream = torch.cuda.current_stream()
    B, Hq, D = w.batch, w.n_q_heads, w.head_dim
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    desc = pq.attn_desc(reps[0]["q"], reps[0]["k_codes"], reps[0]["k_cb"], chunk=chunk)
    ws = pq.step_workspace(desc, dev)

    def step(t):
        pq.pq_attn_decode_step(t["q"], t["xk"], t["xv"], t["k_codes"], t["v_codes"], t["k_cb"],
                               t["v_cb"], t["lens"], out, desc=desc, workspace=ws, stream=stream)

    for i in range(warmup):
        step(reps[i % R])
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for i in range(steps):
        step(reps[i % R])
    b.record(stream)
    torch.cuda.synchronize()
    step_us = a.elapsed_time(b) * 1e3 / steps
    tokens = int(lens_np.sum())
    alg = algorithmic_bytes(w, lens_np)
    ach = alg / (step_us * 1e-6) / 1e9
    return {"workload": f"{w.name}: B={B} Hq={Hq} Hkv={w.n_kv_heads} L={w.max_len} M={w.n_sub}",
            "chunk": int(desc.chunk) or "library", "n_chunks": pq.pq_attn_num_chunks(desc),
            "replicas": R, "value": tokens / (step_us * 1e-6), "unit": "KV tokens/s",
            "step_us": step_us,
            "roofline": {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": ach / HBM_PEAK_GBS, "algorithmic_bytes": alg,
                         "kernel": "decode_partials_kernel (decode-step variant), one launch"}}


def fp8_leg(pq, torch, dev, steps, warmup):
    """The plain decode (score kernel + merge kernel) of the GQA workload with
    FP8 E4M3 codebooks (pq_attn_decode_fp8cb) next to the same decode with
    fp16 ones (pq_attn_decode): codebook bytes halve, the codes do not."""
    from synth import gen
    w, lens_np, reps = step_replicas(torch, dev, 3, 7500)
    R = len(reps)
    rng = np.random.default_rng(7501)
    for t in reps:
        t["k_cb8"] = torch.from_numpy(gen.codebooks_fp8(rng, w.n_kv_heads, w.n_sub, 256, w.sub_dim)).to(dev)
        t["v_cb8"] = torch.from_numpy(gen.codebooks_fp8(rng, w.n_kv_heads, w.n_sub, 256, w.sub_dim)).to(dev)
    stream = torch.cuda.current_stream()
    out = torch.empty((w.batch, w.n_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    desc = pq.attn_desc(reps[0]["q"], reps[0]["k_codes"], reps[0]["k_cb"])
    ws = torch.empty(max(16, pq.pq_attn_workspace_bytes(desc)), dtype=torch.uint8, device=dev)

    def f16(t):
        pq.pq_attn_decode(t["q"], t["k_codes"], t["v_codes"], t["k_cb"], t["v_cb"], t["lens"], out,
                          desc=desc, workspace=ws, stream=stream)

    def f8(t):
        pq.pq_attn_decode_fp8cb(t["q"], t["k_codes"], t["v_codes"], t["k_cb8"], t["v_cb8"], t["lens"],
                                out, desc=desc, workspace=ws, stream=stream)

    res = {"workload": f"{w.name}: B={w.batch} Hq={w.n_q_heads} Hkv={w.n_kv_heads} L={w.max_len} "
                       f"M={w.n_sub}, plain decode (score + merge launches)", "replicas": R}
    tokens = int(lens_np.sum())
    cb16 = w.n_kv_heads * 2 * w.n_sub * w.n_codes * w.sub_dim * 2
    for name, fn, alg in (("fp16", f16, algorithmic_bytes(w, lens_np, step=False)),
                          ("fp8", f8, algorithmic_bytes(w, lens_np, step=False) - cb16 // 2)):
        for i in range(warmup):
            fn(reps[i % R])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(steps):
            fn(reps[i % R])
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / steps
        ach = alg / (us * 1e-6) / 1e9
        res[name] = {"decode_us": us, "value": tokens / (us * 1e-6), "unit": "KV tokens/s",
                     "algorithmic_bytes": alg, "hbm_gbs": ach, "frac": ach / HBM_PEAK_GBS}
    return res


def _bench_lib():
    import ctypes
    path = os.path.join(ROOT, "decode_attention_product_amd", "libpqbench.so")
    lib = ctypes.CDLL(path)
    lib.pqbench_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.pqbench_stream_read.restype = ctypes.c_int
    return lib


def stream_read_leg(torch, dev, reps=200):
    """Read-only streaming kernel (libpqbench.so, 16-byte loads, one checksum
    word per workgroup out): the step's algorithmic bytes on the step kernel's grid (256
    workgroups of 1024 threads) and on 2048 workgroups of 256, and 512 MiB,
    rotated over 1 GiB of buffers so every launch reads HBM, not the
    Infinity Cache.  Timed with HIP events around back-to-back launches."""
    lib = _bench_lib()
    stream = torch.cuda.current_stream()
    chk = torch.zeros(8192, dtype=torch.int32, device=dev)
    res = {}
    for name, nbytes, grid, block in (("10MB_256x1024", 9864192, 256, 1024),
                                      ("10MB_2048x256", 9864192, 2048, 256),
                                      ("512MiB_2048x256", 512 << 20, 2048, 256),
                                      ("512MiB_8192x256", 512 << 20, 8192, 256)):
        nbuf = max(2, math.ceil((1 << 30) / nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3) for _ in range(nbuf)]
        n = reps if nbytes < (64 << 20) else 20

        def run(i):
            st = lib.pqbench_stream_read(bufs[i % nbuf].data_ptr(), nbytes, chk.data_ptr(), grid, block,
                                         stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"pqbench_stream_read: hip error {st}")

        for i in range(10):
            run(i)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            run(i)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / n
        gbs = nbytes / (us * 1e-6) / 1e9
        res[name] = {"bytes": nbytes, "grid": [grid, block], "us_per_read": us, "gbs_read": gbs,
                     "frac": gbs / HBM_PEAK_GBS}
        del bufs
    return res


def stream_leg(torch, dev, reps=200):
    """Reference HBM rates on the same box: the read-only streaming kernel
    (stream_read_leg), and device-to-device copies (one read and one write per
    byte) of the step kernel's size (~10 MB, one launch each) and of 512 MiB,
    rotated over enough buffers that the copies miss the Infinity Cache.
    What one launch of this size can reach, next to the step kernel's
    roofline fraction."""
    stream = torch.cuda.current_stream()
    res = {"read_only": stream_read_leg(torch, dev, reps)}
    for name, nbytes in (("10MB", 9864192), ("512MiB", 512 << 20)):
        nbuf = max(2, math.ceil((1 << 30) / nbytes))
        bufs = [torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1) for _ in range(nbuf)]
        n = reps if nbytes < (64 << 20) else 20
        for i in range(10):
            bufs[(i + 1) % nbuf].copy_(bufs[i % nbuf])
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            bufs[(2 * i + 1) % nbuf].copy_(bufs[(2 * i) % nbuf])
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / n
        gbs = 2 * nbytes / (us * 1e-6) / 1e9
        res[name] = {"bytes": nbytes, "us_per_copy": us, "gbs_read_plus_write": gbs,
                     "frac": gbs / HBM_PEAK_GBS}
        del bufs
    return res


def kmeans_leg(pq, torch, dev, n_iter=10, reps=20):
    """Codebook learning: pq_kmeans_many (n_iter Lloyd iterations, then the
    final assignment) of the K and the V codebooks of 32 heads (M=4, K=256)
    together on a sample of N vectors per head -- the pages' 32-vector sample
    and a 4096-token prefill -- from a perturbed start (one launch each; the
    timed region also restores the two start codebooks, two small copies).
    Timed with events around `reps` learns.  HBM bytes per iteration: the sample
    read by the assignment and by the update, its codes written and read."""
    from synth import gen
    stream = torch.cuda.current_stream()
    res = {"n_iter": n_iter, "heads": 32, "n_sub": 4}
    for name, N in (("sample32", 32), ("prefill4096", 4096)):
        rng = np.random.default_rng(7300 + N)
        cases = [gen.kmeans_case(rng, N, 32, 4, sigma=0.1, init_sigma=0.3, n_used=min(N, 256))
                 for _ in range(2)]
        xs = [torch.from_numpy(c["x"]).to(dev) for c in cases]
        starts = [torch.from_numpy(c["cb_init"]).to(dev) for c in cases]
        cbs = [t.clone() for t in starts]
        codes = [torch.empty((N, 32, 4), dtype=torch.uint8, device=dev) for _ in cases]

        def learn():
            for cb, st in zip(cbs, starts):
                cb.copy_(st)
            pq.pq_kmeans_many(xs, cbs, n_iter, codes, stream=stream)

        learn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            learn()
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3 / reps
        per_iter = 2 * (2 * N * 32 * 128 * 2 + 2 * N * 32 * 4)     # K and V
        res[name] = {"vectors_per_head": N, "us_per_learn_k_and_v": us,
                     "vector_iterations_per_s": 2 * N * 32 * n_iter / (us * 1e-6),
                     "hbm_gbs": per_iter * n_iter / (us * 1e-6) / 1e9}
    return res


def encode_leg(pq, torch, dev, reps):
    """Prefill encode of the ragged workload: every prefill token's K and V
    (6,455,296 vectors of D=128) by nearest codeword straight into the code
    cache (K and V in one launch), timed with HIP events around `reps` calls."""
    from synth import gen
    w = gen.WORKLOADS[5]
    inp = gen.workload_inputs(5)
    B, H, L, M = w.batch, w.n_kv_heads, w.max_len, w.n_sub
    N = int(inp["lens"].sum())
    t = {k: torch.from_numpy(np.ascontiguousarray(inp[k])).to(dev)
         for k in ("x_k", "x_v", "k_cb", "v_cb", "k_codes", "v_codes", "slots")}
    desc = pq.cache_encode_desc(N, B, H, L, n_sub=M)
    stream = torch.cuda.current_stream()

    def call():
        pq.pq_encode_many([t["x_k"], t["x_v"]], [t["k_cb"], t["v_cb"]], [t["k_codes"], t["v_codes"]],
                          slots=t["slots"], desc=desc, stream=stream)

    call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    us_pair = a.elapsed_time(b) * 1e3 / reps
    n_vec = 2 * N * H
    bytes_pair = 2 * (N * H * w.head_dim * 2 + N * H * M + H * M * w.n_codes * w.sub_dim * 2)
    flops_pair = n_vec * 2 * w.n_codes * w.head_dim
    return {"value": n_vec / (us_pair * 1e-6), "unit": "vectors/s",
            "workload": f"ragged prefill: {N} tokens x {H} heads x (K, V) = {n_vec} vectors",
            "us_per_kv_pair": us_pair,
            "hbm_gbs": bytes_pair / (us_pair * 1e-6) / 1e9,
            "hbm_frac": bytes_pair / (us_pair * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "mfma_tflops": flops_pair / (us_pair * 1e-6) / 1e12,
            "mfma_frac_fp16": flops_pair / (us_pair * 1e-6) / 1e12 / 2500.0}


if __name__ == "__main__":
    main()
