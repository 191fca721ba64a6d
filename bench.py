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
The workload is the GQA decode shape (B=8, Hq=64, Hkv=8, L=8192, M=8,
K=256).  Inputs live in HBM before timing starts; N seeded replicas of every
input are rotated so that the working set (>= 512 MiB) is twice the 256 MB
Infinity Cache and each step reads its codes from HBM.

Further legs in the same line: "long_context" (the same one-launch step on
the long-context split-K workload, B=1, Hq=64, Hkv=8, L=131072, M=4, 64
chunks of 2048 tokens per KV head), "paged", "encode", "kmeans" and
"stream_reference" (device copies of the step's size and of 512 MiB: what
one launch reaches on the same box).

Prints one JSON line.  `value` = KV tokens scanned per second over the timed
steps (sum of lens per step / step time).  `roofline` is the step kernel's
algorithmic bytes per launch over its average duration, timed with HIP
events the runtime stamps at the kernel's own start and end.  `cpu_baseline` is the
CPU oracle on the same workload (repeated for 10+ s), on the host cores.
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


def cpu_baseline(wid, min_seconds=10.0, max_seconds=30.0):
    import oracle
    from synth import gen
    inp = gen.workload_inputs(wid, with_encode=False)
    args = [inp[k] for k in ("q", "k_codes", "v_codes", "k_cb", "v_cb", "lens")]
    tokens = int(inp["lens"].sum())
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode_attention(*args)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or el + el / reps > max_seconds:
            break
    return {"value": tokens * reps / el, "unit": "KV tokens/s", "cores": _oracle_threads(),
            "kind": "oracle",
            "sample": f"{gen.WORKLOADS[wid].name} workload, whole decode step, repeated {reps}x "
                      f"({el:.1f} s)"}


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        return int(max(n)) if n else 1
    except Exception:
        return 1


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
    ap.add_argument("--no-stream", action="store_true", help="skip the device-copy reference")
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
    achieved = alg / (score_ms * 1e-3) / 1e9

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
                     "avg_launch_us": score_ms * 1e3},
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
    if not args.no_long and wid != 4:
        result["long_context"] = long_context_leg(pq, torch, dev, args.paged_steps, args.warmup)
    if not args.no_paged:
        result["paged"] = paged_leg(pq, torch, dev, args.paged_steps, args.warmup,
                                    step_ms_plain * 1e3 if wid == 3 else None)
    if not args.no_encode:
        result["encode"] = encode_leg(pq, torch, dev, args.encode_reps)
    if not args.no_kmeans:
        result["kmeans"] = kmeans_leg(pq, torch, dev)
    if not args.no_stream:
        result["stream_reference"] = stream_leg(torch, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(wid)
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
        achieved = alg / (kern_us * 1e-6) / 1e9
        leg = {"workload": f"{w.name}: B={B} Hq={Hq} Hkv={Hkv} Lmax={L} M={M}, {tokens} tokens",
               "value": tokens / (step_us * 1e-6), "unit": "KV tokens/s", "step_us": step_us,
               "kernel_us": kern_us, "replicas": R,
               "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                            "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes": alg,
                            "kernel": "decode_paged_kernel (decode-step variant)"},
               "pool_slots_per_head": n_pages * P, "padded_slots_per_head": B * L}
        if name == "gqa" and dense_gqa_us is not None:
            leg["dense_step_us"] = dense_gqa_us
        if name == "ragged":
            leg["dense_step_us"] = timed(dense)
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
        achieved = alg / (kern_us * 1e-6) / 1e9
        return {"chunk": chunk,
                "n_chunks": pq.pq_attn_num_chunks(desc),
                "value": tokens / (step_us * 1e-6), "unit": "KV tokens/s", "step_us": step_us,
                "kernel_us": kern_us,
                "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": achieved / HBM_PEAK_GBS, "algorithmic_bytes": alg,
                             "kernel": "decode_partials_kernel (decode-step variant)"}}

    leg = {"workload": f"{w.name}: B={B} Hq={Hq} Hkv={Hkv} L={L} M={M}", "replicas": R}
    leg.update(run(w.chunk))
    lib = run(0)
    lib["chunk"] = "library"
    leg["library_chunk"] = lib
    return leg


def stream_leg(torch, dev, reps=200):
    """Reference HBM rates on the same box: device-to-device copies (one
    read and one write per byte) of the step kernel's size (~10 MB, one
    launch each) and of 512 MiB, rotated over enough buffers that the copies
    miss the Infinity Cache.  What one launch of this size can reach, next to
    the step kernel's roofline fraction."""
    stream = torch.cuda.current_stream()
    res = {}
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
