"""Benchmark of the MXFP4 attention hot path on one MI355X.

A step is one pass of the forward hot path over one batch: MXFP4 quantization of Q, K (along d)
and V (along the sequence, block-major) followed by the fused FP4 attention forward, on the
video-DiT-shaped workload B=1, H=24, N=32768, d=128, non-causal.  Inputs (bf16) are resident in
HBM before the timed region.  The metric counts 4*B*H*N^2*d flops per step.

Printed: one JSON line with the step throughput, a roofline object for the dominant kernel (the
fused forward, timed alone with HIP events on the stream it runs on), the backward of the QAT
workload (B=1, H=16, N=8192, d=128) measured the same way, the forward with the exp-free EFQ
probability codes, the forward over NVFP4-style operands (E4M3 scale per 16 elements, fp16
operands on the fp16 matrix core) on the same inputs, the forward on the causal LLM and
GQA-prefill workloads, the cache forward on a decode batch and a chunked-prefill step, and the CPU
oracle timed on a bounded sample of the same workload.  The secondary workloads are timed once the
GPU runs at its steady clock (settle_and_time); the step itself takes exactly --warmup untimed
steps, then --steps timed ones.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "FP4 attn fwd TFLOPS (4·B·H·N²·d) at N=32K,d=128; % of MXFP4 MFMA peak"
PEAK_FP4_TFLOPS = 10100.0      # MI355X dense MXFP4 matrix peak (published 10.1 PFLOP/s)
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 / fp16 matrix peak (published 2.5 PFLOP/s)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E (published 8 TB/s)
QUANT_BYTES_PER_ELEM = 2.0 + 0.5 + 1.0 / 32.0

# Measured HBM traffic of one forward launch at the bench shape: rocprofv3 --pmc FETCH_SIZE and
# --pmc WRITE_SIZE, each scaled by the factor the same counter shows on a plain 1 GiB device copy
# (FETCH_SIZE 2.000, WRITE_SIZE 1.000).  Valid only for the kernel source and build flags it was
# measured with.  (The source changed since, in the split cache forward only; the plain forward's
# gfx950 assembly compiled from fwd.hip is identical to the one measured.)
FWD_TRAFFIC = {"source_sha1": "c495500128b625d38ced583e5d25a8878ca46eeb", "bytes": 1.0566e9}


def fwd_source_sha1():
    import hashlib
    h = hashlib.sha1()
    for f in ("bit_attention_amd/csrc/fwd.hip", "bit_attention_amd/csrc/fwd_kernel.h", "bit_attention_amd/csrc/common.h",
              "bit_attention_amd/build.py"):
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gen_inputs(w, tensors):
    """Seeded synthetic inputs of the workload, generated per head in parallel processes."""
    import numpy as np
    from concurrent.futures import ProcessPoolExecutor
    from bit_attention_amd import workloads as W
    out = {}
    with ProcessPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        for t in tensors:
            H = W.heads_of(w, t)
            jobs = [(b, h) for b in range(w.B) for h in range(H)]
            heads = list(ex.map(_gen_one, [(w.name, t, b, h) for b, h in jobs]))
            arr = np.empty((w.B, H, w.N, w.d), dtype=np.float32)
            for (b, h), x in zip(jobs, heads):
                arr[b, h] = x
            out[t] = arr
    return out


def _gen_one(a):
    from bit_attention_amd import workloads as W
    name, t, b, h = a
    return W.gen_head(W.WORKLOADS[name], t, b, h)


def _gen_cache_one(a):
    from bit_attention_amd import workloads as W
    name, t, b, h = a
    return W.gen_cache_head(W.CACHE_WORKLOADS[name], t, b, h)


def gen_cache_inputs(w, torch):
    """Seeded inputs of a cache workload as bf16 device tensors: q [B,Hq,Nq,d], k, v [B,Hkv,Nk,d]."""
    import numpy as np
    from concurrent.futures import ProcessPoolExecutor
    out = {}
    with ProcessPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        for t in ("q", "k", "v"):
            H, n = (w.Hq, w.Nq) if t == "q" else (w.Hkv, w.Nk)
            jobs = [(b, h) for b in range(w.B) for h in range(H)]
            dev = torch.empty((w.B, H, n, w.d), dtype=torch.bfloat16, device="cuda")
            for (b, h), x in zip(jobs, ex.map(_gen_cache_one, [(w.name, t, b, h) for b, h in jobs])):
                dev[b, h] = torch.from_numpy(x).to(torch.bfloat16)
            out[t] = dev
    return out


def time_region(fn, reps, stream):
    import torch
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        fn()
    e1.record(stream)
    e1.synchronize()
    return e0.elapsed_time(e1) / reps


_QUICK = False


def settle_and_time(fn, min_reps, stream, warm_s=0.3, timed_s=0.15, max_reps=5000):
    """Time fn on the GPU once it runs at its steady clock: the secondary workloads follow seconds
    of host-side input generation with the GPU idle, and a cold GPU runs a ~1 ms kernel 10-15%
    slower for its first few hundred milliseconds.  fn runs untimed for warm_s seconds, then is
    timed over at least min_reps calls and at least timed_s seconds (HIP events, as time_region).
    Returns (ms per call, calls timed)."""
    import torch
    if _QUICK:                                    # profiler runs: exactly min_reps calls, no settling
        return time_region(fn, min_reps, stream), min_reps
    t0 = time.perf_counter()
    n = 0
    while True:
        fn()
        n += 1
        if n % 4 == 0 or n == 1:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= warm_s:
                break
    est_ms = (time.perf_counter() - t0) * 1e3 / n
    reps = int(min(max(min_reps, math.ceil(timed_s * 1e3 / max(est_ms, 1e-3))), max_reps))
    return time_region(fn, reps, stream), reps


_ONE_THREAD_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def _cpu_worker_init():
    # one BLAS thread per worker process: the pool itself spreads the work over the cores (the
    # environment set at spawn covers the BLAS loaded by numpy; the limit covers any loaded later)
    import numpy  # noqa: F401
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)
    except Exception:  # pragma: no cover
        pass


def _cpu_task(a):
    """Oracle forward of some query rows of one head (fresh process: numpy only, no GPU state)."""
    import numpy as np
    import oracle
    from bit_attention_amd import workloads as W
    name, b, h, rows = a
    w = W.WORKLOADS[name]
    g = h // (w.Hq // w.Hkv)
    q = W.gen_head(w, "q", b, h)[None, None]
    k = W.gen_head(w, "k", b, g)[None, None]
    v = W.gen_head(w, "v", b, g)[None, None]
    t0 = time.perf_counter()
    oracle.attn_fwd(q, k, v, causal=w.causal, rows=None if rows is None else np.asarray(rows))
    return time.perf_counter() - t0


def cpu_share():
    """Cores this process may use: the affinity mask, capped by a cgroup CPU quota and by
    OMP_NUM_THREADS when they are set (a shared host's per-job share).  Returns (cores, note)."""
    aff = len(os.sched_getaffinity(0))
    cores, why = aff, ["affinity %d" % aff]
    try:
        q, per = open("/sys/fs/cgroup/cpu.max").read().split()[:2]
        if q != "max":
            quota = max(1, int(int(q) / int(per)))
            why.append("cgroup quota %d" % quota)
            cores = min(cores, quota)
    except Exception:
        pass
    omp = os.environ.get("OMP_NUM_THREADS", "")
    if omp.isdigit() and int(omp) > 0:
        why.append("OMP_NUM_THREADS %s" % omp)
        cores = min(cores, int(omp))
    return cores, ", ".join(why)


def cpu_baseline(w, seconds_target=15.0, chunk=1024,
                 full_workloads=("tiny_b1h2n256d64", "llm_causal_b2h16n4096d128")):
    """The oracle, untouched, on a bounded sample of the same workload, spread over the host cores
    this process may use (one process per core, one BLAS thread each).  Before it, the small
    workloads in ``full_workloads`` are run in full over the same pool (a few seconds).

    Each task is one call of the oracle forward: one head, ``chunk`` sampled query rows against all
    keys.  The heads cycle over the tasks; every core keeps one task in flight until about
    ``seconds_target`` seconds have passed, then the tasks in flight finish.  The full-problem time
    is extrapolated from the measured rate and labelled as such: the full problem is not run."""
    import multiprocessing as mp
    from bit_attention_amd import workloads as W
    cores, share = cpu_share()
    H = w.B * w.Hq
    count = [0]

    def next_task():
        i = count[0]
        count[0] += 1
        hh = i % H
        rows = W.sample_rows(w.N, chunk, seed=W.BASE_SEED + i).tolist()
        return (w.name, hh // w.Hq, hh % w.Hq, rows)

    ctx = mp.get_context("spawn")     # fresh interpreters: nothing of this GPU process is inherited
    saved = {k: os.environ.get(k) for k in _ONE_THREAD_ENV}
    os.environ.update({k: "1" for k in _ONE_THREAD_ENV})
    try:
        pool = ctx.Pool(cores, initializer=_cpu_worker_init)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    with pool:
        # the two small workloads in full first (every row of every head; one task per head)
        full = {}
        for name in full_workloads:
            fw = W.WORKLOADS[name]
            tasks = [(name, b, h, None) for b in range(fw.B) for h in range(fw.Hq)]
            t0 = time.perf_counter()
            for r in [pool.apply_async(_cpu_task, (t,)) for t in tasks]:
                r.get()
            fwall = time.perf_counter() - t0
            pairs = fw.B * fw.Hq * (fw.N * (fw.N + 1) // 2 if fw.causal else fw.N * fw.N)
            full[name] = {"wall_s": fwall, "rows": fw.B * fw.Hq * fw.N, "heads": len(tasks),
                          "tflops": 4.0 * pairs * fw.d / fwall / 1e12,
                          "note": "full problem run (not sampled); visible pairs for causal"}
        t0 = time.perf_counter()
        inflight = [pool.apply_async(_cpu_task, (next_task(),)) for _ in range(cores)]
        done = 0
        while inflight:
            inflight[0].wait()
            still = []
            for r in inflight:
                if r.ready():
                    r.get()
                    done += 1
                    if time.perf_counter() - t0 < seconds_target:
                        still.append(pool.apply_async(_cpu_task, (next_task(),)))
                else:
                    still.append(r)
            inflight = still
        wall = time.perf_counter() - t0
    rows = done * chunk
    flops = 4.0 * rows * w.N * w.d
    total_rows = w.B * w.Hq * w.N
    return {"value": flops / wall / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
            "sample": ("float64 NumPy oracle forward, %d processes (one per core, 1 BLAS thread each; %s); %d "
                       "calls of %d sampled query rows of one head (heads in turn) against all %d keys; %d rows "
                       "in %.1f s wall (worker start-up included); metric flops 4*rows*N*d"
                       % (cores, share, done, chunk, w.N, rows, wall)),
            "rows_per_s": rows / wall, "seconds": wall, "full_runs": full,
            "extrapolated_full_s": total_rows / (rows / wall),
            "extrapolated_note": ("EXTRAPOLATED, not run: %d query rows of the full problem at the sampled %.1f rows/s"
                                  % (total_rows, rows / wall))}


# ---- accuracy context: cosine similarity against exact fp64 softmax attention ----
# Plain float64 softmax attention on the unquantized bf16 inputs (textbook formula, no tiling, no
# quantization); the GPU outputs are compared with it on sampled heads and rows.  Context only:
# the parity gate is the fake-quant oracle in the tests.
def _exact_rows(q, k, v, rows, causal):
    import numpy as np
    q = q.astype(np.float64)[rows]
    s = (q @ k.astype(np.float64).T) / np.sqrt(q.shape[-1])
    if causal:
        s = np.where(np.arange(k.shape[0])[None, :] <= np.asarray(rows)[:, None], s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    return (p / p.sum(axis=1, keepdims=True)) @ v.astype(np.float64)


def _cosine(a, b):
    import numpy as np
    a = np.asarray(a, dtype=np.float64).ravel()
    b = np.asarray(b, dtype=np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def fwd_cosine(w, x, o_dev, heads=None, nrows=256):
    """Cosine of the GPU forward output with exact fp64 attention over sampled rows of some heads.
    x: the workload's host inputs (bf16-valued float32 [B, H, N, d]); o_dev: the GPU O."""
    from bit_attention_amd import workloads as W
    heads = heads if heads is not None else sorted({(0, 0), (w.B - 1, w.Hq - 1)})
    rows = W.sample_rows(w.N, nrows)
    got, ref = [], []
    for b, h in heads:
        g = h // (w.Hq // w.Hkv)
        ref.append(_exact_rows(x["q"][b, h], x["k"][b, g], x["v"][b, g], rows, w.causal))
        got.append(o_dev[b, h, rows].float().cpu().numpy())
    return {"cos_O": _cosine(got, ref), "heads": [list(h) for h in heads], "rows_per_head": int(rows.size)}


def bwd_cosine(w, x, dq, dk, dv, b=0, h=0):
    """Cosine of the GPU gradients (one head, all rows and keys) with the exact fp64 gradients of
    softmax attention at the unquantized inputs (D from the exact output)."""
    import numpy as np
    q, k, v, do = (x[t][b, h].astype(np.float64) for t in ("q", "k", "v", "do"))
    sc = 1.0 / np.sqrt(q.shape[-1])
    s = (q @ k.T) * sc
    p = np.exp(s - s.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    o = p @ v
    dp = do @ v.T
    ds = p * (dp - np.sum(do * o, axis=1, keepdims=True))
    del s, dp
    ref = {"dQ": (ds @ k) * sc, "dK": (ds.T @ q) * sc, "dV": p.T @ do}
    got = {"dQ": dq[b, h], "dK": dk[b, h], "dV": dv[b, h]}
    return {"cos_" + n: _cosine(got[n].float().cpu().numpy(), ref[n]) for n in ref}


def bench_backward(args, torch, ops, W):
    w = W.WORKLOADS["qat_bwd_b1h16n8192d128"]
    x = gen_inputs(w, ["q", "k", "v", "do"])
    dev = {t: torch.from_numpy(a).to(torch.bfloat16).cuda() for t, a in x.items()}
    qc, qs = ops.attn_fp4_quantize(dev["q"], 0)
    kc, ks = ops.attn_fp4_quantize(dev["k"], 0)
    vc, vs = ops.attn_fp4_quantize(dev["v"], 1)
    o, m, l = ops.attn_fp4_fwd(qc, qs, kc, ks, vc, vs)
    try:
        res = ops.attn_fp4_bwd_recompute(qc, qs, kc, ks, vc, vs, o, dev["do"], m, l)
    except ops.AttnFp4Error as e:
        return {"workload": w.name, "status": str(e)}
    dq, dk, dv = res
    torch.cuda.synchronize()
    acc = fwd_cosine(w, x, o)
    acc.update(bwd_cosine(w, x, dq, dk, dv))
    del x
    ws = torch.empty(ops.attn_fp4_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.N, w.d), dtype=torch.uint8,
                     device="cuda")
    stream = torch.cuda.current_stream()
    fn = lambda: ops.attn_fp4_bwd_recompute(qc, qs, kc, ks, vc, vs, o, dev["do"], m, l, dq=dq, dk=dk, dv=dv,
                                            workspace=ws)
    ms, reps = settle_and_time(fn, max(3, args.steps), stream)
    pairs = w.B * w.Hq * w.N * w.N
    fp4 = 2.0 * w.d * pairs
    bf16 = 8.0 * w.d * pairs
    t_roof = fp4 / (PEAK_FP4_TFLOPS * 1e9) + bf16 / (PEAK_BF16_TFLOPS * 1e9)
    return {"workload": w.name, "ms": ms, "accuracy": acc, "fp4_flops": fp4, "bf16_flops": bf16,
            "tflops_total": (fp4 + bf16) / ms / 1e9, "roofline_ms": t_roof, "frac": t_roof / ms}


def bench_forward_configs(args, torch, ops, W):
    """The forward alone on the other forward workloads (causal LLM shape, GQA prefill), seeded
    inputs, HIP events on its stream; flops count the visible (query, key) pairs, 4 d each."""
    out = {}
    for name in ("tiny_b1h2n256d64", "llm_causal_b2h16n4096d128", "gqa_causal_b1hq32hkv8n16384d128"):
        w = W.WORKLOADS[name]
        x = gen_inputs(w, ["q", "k", "v"])
        dev = {t: torch.from_numpy(a).to(torch.bfloat16).cuda() for t, a in x.items()}
        qq = ops.attn_fp4_quantize(dev["q"], 0)
        kq = ops.attn_fp4_quantize(dev["k"], 0)
        vq = ops.attn_fp4_quantize(dev["v"], 1)
        del dev
        o, m, l = ops.attn_fp4_fwd(*qq, *kq, *vq, causal=w.causal)
        torch.cuda.synchronize()
        acc = fwd_cosine(w, x, o)
        del x
        fn = lambda: ops.attn_fp4_fwd(*qq, *kq, *vq, causal=w.causal, o=o, m=m, l=l)
        ms, reps = settle_and_time(fn, max(5, args.steps), torch.cuda.current_stream())
        pairs = w.B * w.Hq * (w.N * (w.N + 1) // 2 if w.causal else w.N * w.N)
        tf = 4.0 * w.d * pairs / ms / 1e9
        out[name] = {"ms": ms, "calls_timed": reps, "visible_pairs": pairs, "tflops": tf,
                     "frac_mfma": tf / PEAK_FP4_TFLOPS, "accuracy": acc}
    return out


def bench_nvfp4(args, torch, ops, w, dev, reps=None):
    """The NVFP4-style path on the same inputs: quantize Q, K (along d) and V (along the sequence) to
    16-element blocks with E4M3 block scales and fp32 tensor scales, then the forward (its three
    exact fp16 dequantization launches and the fp16 matrix-core attention kernel), each timed with
    HIP events on its stream."""
    stream = torch.cuda.current_stream()
    B, H, N, d = w.B, w.Hq, w.N, w.d
    quant = [ops.attn_fp4_nv_quantize(dev[t], 1 if t == "v" else 0) for t in ("q", "k", "v")]
    (qc, qs, qt), (kc, ks, kt), (vc, vs, vt) = quant
    ws = torch.empty(ops.attn_fp4_nv_fwd_workspace_bytes(B, H, H, N, d), dtype=torch.uint8, device="cuda")
    o, m, l = ops.attn_fp4_nv_fwd(qc, qs, qt, kc, ks, kt, vc, vs, vt, causal=w.causal, workspace=ws)
    fwd = lambda: ops.attn_fp4_nv_fwd(qc, qs, qt, kc, ks, kt, vc, vs, vt, causal=w.causal, o=o, m=m, l=l,
                                      workspace=ws)
    if reps:
        for _ in range(reps):
            fwd()
        torch.cuda.synchronize()
        return {"ran": reps}

    def quantize():
        for t, (c, sc, ts) in zip(("q", "k", "v"), quant):
            ops.attn_fp4_nv_quantize(dev[t], 1 if t == "v" else 0, c, sc, ts)

    quantize()
    ms, _ = settle_and_time(fwd, max(3, args.steps), stream)
    qms, _ = settle_and_time(quantize, max(3, args.steps), stream, warm_s=0.05)
    flops = 4.0 * B * H * N * N * d
    tf = flops / ms / 1e9
    return {"ms_fwd": ms, "ms_quantize_qkv": qms, "tflops": tf, "frac_f16_mfma": tf / PEAK_BF16_TFLOPS,
            "format": "E2M1, E4M3 scale per 16, fp32 tensor scale (a reading of NVFP4); fp16 matrix core",
            "timed": "attn_fp4_nv_fwd entry point: three fp16 dequantization launches + the attention kernel"}


def bench_kvcache(args, torch, ops, W, only=None):
    """The cache forward (attn_fp4_fwd_kvcache) on the decode and chunked-prefill workloads: the
    forward alone (K^/V^ already quantized in the cache), HIP events on its stream."""
    import numpy as np
    out = {}
    for name, w in W.CACHE_WORKLOADS.items():
        if only is not None and name not in only:
            continue
        x = gen_cache_inputs(w, torch)
        qq = ops.attn_fp4_quantize(x["q"], 0)
        kq = ops.attn_fp4_quantize(x["k"], 0)
        vq = ops.attn_fp4_quantize(x["v"], 1)
        del x
        lens = W.cache_lengths(w)
        sl = torch.from_numpy(lens).cuda()
        o = torch.empty((w.B, w.Hq, w.Nq, w.d), dtype=torch.bfloat16, device="cuda")
        m = torch.empty((w.B, w.Hq, w.Nq), dtype=torch.float32, device="cuda")
        l = torch.empty_like(m)
        need = ops.attn_fp4_fwd_kvcache_workspace_bytes(w.B, w.Hq, w.Hkv, w.Nq, w.Nk, w.d)
        ws = torch.empty(need, dtype=torch.uint8, device="cuda") if need > 0 else None
        fn = lambda: ops.attn_fp4_fwd_kvcache(*qq, *kq, *vq, seqlens_k=sl, causal=w.causal, o=o, m=m, l=l,
                                              workspace=ws)
        ms, reps = settle_and_time(fn, max(10, args.steps), torch.cuda.current_stream())
        lens64 = lens.astype(np.int64)
        pairs = 0
        for L in lens64:
            pos = L - w.Nq + np.arange(w.Nq)
            vis = np.minimum(pos + 1, L) if w.causal else np.full(w.Nq, L)
            pairs += int(np.maximum(vis, 0).sum()) * w.Hq
        # algorithmic bytes: the valid part of the cache (K^ and V^ codes and scales) once, Q^ once,
        # O (bf16) and m, l written once
        cache_b = int(lens64.sum()) * w.Hkv * 2 * (w.d // 2 + w.d // 32)
        io_b = w.B * w.Hq * w.Nq * (w.d // 2 + w.d // 32 + 2 * w.d + 8)
        out[name] = {"ms": ms, "calls_timed": reps, "split": need > 0, "visible_pairs": pairs,
                     "tflops": 4.0 * w.d * pairs / ms / 1e9,
                     "frac_mfma": 4.0 * w.d * pairs / ms / 1e9 / PEAK_FP4_TFLOPS,
                     "bytes": cache_b + io_b, "gbps": (cache_b + io_b) / ms / 1e6,
                     "frac_hbm": (cache_b + io_b) / ms / 1e6 / PEAK_HBM_GBS,
                     "cache_lengths": "seeded U[%d, %d]" % (w.len_lo, w.Nk)}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-baseline-only", action="store_true", help="only time the CPU oracle (no GPU)")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--fwd-only-reps", type=int, default=0,
                    help="if > 0: only run the forward kernel this many times (for profilers)")
    ap.add_argument("--bwd-only-reps", type=int, default=0,
                    help="if > 0: only run the QAT-workload backward this many times (for profilers)")
    ap.add_argument("--kv-only-reps", type=int, default=0,
                    help="if > 0: only run the decode cache forward this many times (for profilers)")
    ap.add_argument("--causal-only-reps", type=int, default=0,
                    help="if > 0: only run the causal LLM and causal GQA forwards this many times each "
                         "(for profilers)")
    ap.add_argument("--nv-only-reps", type=int, default=0,
                    help="if > 0: only run the NVFP4-style forward this many times (for profilers)")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="if > 0: only run a plain device copy of this many bytes 3 times "
                         "(calibrates the HBM byte counters of a profiler)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(the single-GPU kernel is what scales; see the sharding notes). Use --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.cpu_baseline_only:
        from bit_attention_amd import workloads as W
        print(json.dumps(cpu_baseline(W.WORKLOADS["dit_b1h24n32768d128"])), flush=True)
        return

    import torch
    from bit_attention_amd import ops
    from bit_attention_amd import workloads as W

    if args.copy_bytes > 0:
        src = torch.empty(args.copy_bytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d bytes 3 times" % (src.numel() * 4))
        return

    global _QUICK
    _QUICK = args.bwd_only_reps > 0 or args.kv_only_reps > 0 or args.nv_only_reps > 0 or args.causal_only_reps > 0

    if args.bwd_only_reps > 0:
        args.steps = args.bwd_only_reps
        log("backward", bench_backward(args, torch, ops, W))
        return

    if args.causal_only_reps > 0:
        for name in ("llm_causal_b2h16n4096d128", "gqa_causal_b1hq32hkv8n16384d128"):
            w = W.WORKLOADS[name]
            x = gen_inputs(w, ["q", "k", "v"])
            dev = {t: torch.from_numpy(a).to(torch.bfloat16).cuda() for t, a in x.items()}
            qq = ops.attn_fp4_quantize(dev["q"], 0)
            kq = ops.attn_fp4_quantize(dev["k"], 0)
            vq = ops.attn_fp4_quantize(dev["v"], 1)
            o, m, l = ops.attn_fp4_fwd(*qq, *kq, *vq, causal=w.causal)
            for _ in range(args.causal_only_reps):
                ops.attn_fp4_fwd(*qq, *kq, *vq, causal=w.causal, o=o, m=m, l=l)
            torch.cuda.synchronize()
            log("%s: %d forwards" % (name, args.causal_only_reps))
        return

    if args.kv_only_reps > 0:
        args.steps = args.kv_only_reps
        log("kvcache", bench_kvcache(args, torch, ops, W, only=["decode_b8hq32hkv8nk32768d128"]))
        return

    w = W.WORKLOADS["dit_b1h24n32768d128"]
    log("generating inputs for", w.name)
    t0 = time.perf_counter()
    x = gen_inputs(w, ["q", "k", "v"])
    log("  %.1f s" % (time.perf_counter() - t0))
    dev = {t: torch.from_numpy(a).to(torch.bfloat16).cuda() for t, a in x.items()}
    B, H, N, d = w.B, w.Hq, w.N, w.d
    qc = torch.empty((B, H, N, d // 2), dtype=torch.uint8, device="cuda")
    qs = torch.empty((B, H, N, d // 32), dtype=torch.uint8, device="cuda")
    kc, ks = torch.empty_like(qc), torch.empty_like(qs)
    vc = torch.empty((B, H, N // 32, d, 16), dtype=torch.uint8, device="cuda")
    vs = torch.empty((B, H, N // 32, d), dtype=torch.uint8, device="cuda")
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device="cuda")
    m = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    l = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()

    def quantize():
        ops.attn_fp4_quantize(dev["q"], 0, qc, qs)
        ops.attn_fp4_quantize(dev["k"], 0, kc, ks)
        ops.attn_fp4_quantize(dev["v"], 1, vc, vs)

    def fwd():
        ops.attn_fp4_fwd(qc, qs, kc, ks, vc, vs, causal=w.causal, o=o, m=m, l=l)

    def step():
        quantize()
        fwd()

    if args.nv_only_reps > 0:
        log("nvfp4", bench_nvfp4(args, torch, ops, w, dev, reps=args.nv_only_reps))
        return

    if args.fwd_only_reps > 0:
        quantize()
        for _ in range(args.fwd_only_reps):
            fwd()
        torch.cuda.synchronize()
        log("ran the forward %d times" % args.fwd_only_reps)
        return

    # accuracy of this workload's output first (host-side work), so that nothing but the warmup
    # steps sits between the GPU going idle and the timed region
    step()
    torch.cuda.synchronize()
    acc_main = fwd_cosine(w, x, o)
    del x
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log("warmup done")
    # timed region: exactly K steps, synchronised on both sides
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ms_step = time_region(step, args.steps, stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log("step %.3f ms (events), %.3f ms (wall)" % (ms_step, wall_ms))
    # dominant kernel alone (same launch configuration), HIP events on its stream
    fwd_ms = time_region(fwd, args.steps, stream)
    quant_ms = time_region(quantize, args.steps, stream)
    efq_ms = time_region(lambda: ops.attn_fp4_fwd(qc, qs, kc, ks, vc, vs, causal=w.causal, o=o, m=m, l=l,
                                                  p_rule=ops.P_EFQ), args.steps, stream)
    fwd()                                         # O back to the exp-then-quantize forward's
    flops = 4.0 * B * H * N * N * d
    fwd_tflops = flops / fwd_ms / 1e9
    log("fwd kernel %.3f ms = %.1f TFLOPS; quantize q,k,v %.3f ms" % (fwd_ms, fwd_tflops, quant_ms))

    result = {
        "metric": METRIC,
        "value": flops / ms_step / 1e9,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "H": H, "N": N, "d": d, "causal": w.causal,
                   "step": "quantize Q,K,V (bf16->MXFP4) + fused FP4 attention forward",
                   "flops_per_step": flops},
        "roofline": {"bound": "mfma", "achieved": fwd_tflops, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                     "frac": fwd_tflops / PEAK_FP4_TFLOPS,
                     "traffic": FWD_TRAFFIC["bytes"] if fwd_source_sha1() == FWD_TRAFFIC["source_sha1"] else None,
                     "kernel": "attn_fp4 forward (fwd_kernel<128,...,false>)", "kernel_ms": fwd_ms,
                     "flops_per_launch": flops},
        "quantize": {"ms": quant_ms, "elements": 3 * B * H * N * d,
                     "gbps": QUANT_BYTES_PER_ELEM * 3 * B * H * N * d / quant_ms / 1e6,
                     "frac_hbm": QUANT_BYTES_PER_ELEM * 3 * B * H * N * d / quant_ms / 1e6 / PEAK_HBM_GBS},
    }
    result["efq"] = {"ms": efq_ms, "tflops": flops / efq_ms / 1e9, "frac": flops / efq_ms / 1e9 / PEAK_FP4_TFLOPS,
                     "p_rule": "exp-free EFQ codes (a reading of the pages; not the headline definition)"}
    result["nvfp4"] = bench_nvfp4(args, torch, ops, w, dev)
    log("nvfp4", result["nvfp4"])
    del dev
    if not args.no_backward:
        result["backward"] = bench_backward(args, torch, ops, W)
        log("backward", result["backward"])
    result["forward_configs"] = bench_forward_configs(args, torch, ops, W)
    log("forward_configs", result["forward_configs"])
    result["kvcache"] = bench_kvcache(args, torch, ops, W)
    log("kvcache", result["kvcache"])
    # accuracy context: cosine of the GPU outputs with exact fp64 softmax attention
    accuracy = {w.name: acc_main}
    for name, r in result["forward_configs"].items():
        accuracy[name] = r["accuracy"]
    if "backward" in result and "accuracy" in result["backward"]:
        accuracy[result["backward"]["workload"]] = result["backward"]["accuracy"]
    result["accuracy"] = {"reference": "exact float64 softmax attention (and its gradients) on the unquantized "
                                       "bf16 inputs; sampled rows of the first and last heads (gradients: one "
                                       "whole head)", "cosine": accuracy}
    log("accuracy", result["accuracy"])
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a bounded sample")
        cb = cpu_baseline(w)
        result["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample", "rows_per_s",
                                                     "extrapolated_full_s", "extrapolated_note", "full_runs")}
        log("cpu_baseline", result["cpu_baseline"])
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
