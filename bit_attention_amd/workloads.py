"""Seeded synthetic inputs for the attention workloads (no attention arithmetic here).

This module only draws random numbers and rounds them to bfloat16; it holds
none of the method's arithmetic, so both the HIP path's tests/bench and the
CPU oracle can consume its output.  Every head of every tensor comes from its
own stream, ``PCG64(SeedSequence([seed, workload_id, tensor_id, b, h]))``, so
any single head can be regenerated alone (the oracle does this for sampled
parity at full size).

The shapes and value distributions stand in for the LLM and video-DiT
workloads on which the pages evaluate 4-bit attention (Qwen3 and WAN2.2 in
the EFQ-Softmax abstract; diffusion and language models in the Attn-QAT
abstract).  None of those models or evaluation suites is used.
"""

import math
from dataclasses import dataclass, field

import numpy as np

BASE_SEED = 20261203

TENSOR_ID = {"q": 0, "k": 1, "v": 2, "do": 3, "outlier": 9}


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    N: int
    d: int
    causal: bool
    kind: str                      # distribution recipe, see _draw_head
    backward: bool = False
    note: str = field(default="", compare=False)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_b1h2n256d64", 0, 1, 2, 2, 256, 64, False, "normal",
                 note="Q,K,V i.i.d. N(0,1)"),
        Workload("llm_causal_b2h16n4096d128", 1, 2, 16, 16, 4096, 128, True, "llm_outlier",
                 note="Q,K N(0,1) with 2 of 128 channels (same in Q and K) x20; V Student-t(3)"),
        Workload("dit_b1h24n32768d128", 2, 1, 24, 24, 32768, 128, False, "dit_heavy",
                 note="Student-t(4)/sqrt(2) times a per-token log-normal(0,0.5) magnitude"),
        Workload("gqa_causal_b1hq32hkv8n16384d128", 3, 1, 32, 8, 16384, 128, True, "gqa_outlier",
                 note="N(0,1); 1 of 128 K channels x30 per KV head"),
        Workload("qat_bwd_b1h16n8192d128", 4, 1, 16, 16, 8192, 128, False, "normal_bwd", backward=True,
                 note="Q,K,V,dO N(0,1); dO x1e-2"),
    ]
}


def round_to_bf16(x):
    """Round float64/float32 values to bfloat16 (via float32, then round-to-nearest-even).

    Returns float32 arrays whose low 16 bits are zero.
    """
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).reshape(f.shape)


def _rng(seed, wid, tensor, b, h):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, TENSOR_ID[tensor], b, h])))


def _outlier_channels(w, seed, b, h, count):
    return _rng(seed, w.wid, "outlier", b, h).choice(w.d, size=count, replace=False)


def _draw_head(w, tensor, b, h, seed):
    N, d = w.N, w.d
    r = _rng(seed, w.wid, tensor, b, h)
    if w.kind in ("normal", "normal_bwd"):
        x = r.standard_normal((N, d))
        if tensor == "do":
            x *= 1e-2
    elif w.kind == "llm_outlier":
        if tensor == "v":
            x = r.standard_t(3.0, size=(N, d))
        else:
            x = r.standard_normal((N, d))
            x[:, _outlier_channels(w, seed, b, h, math.ceil(0.01 * d))] *= 20.0
    elif w.kind == "dit_heavy":
        x = r.standard_t(4.0, size=(N, d)) / math.sqrt(2.0)
        x *= np.exp(0.5 * r.standard_normal(N))[:, None]
    elif w.kind == "gqa_outlier":
        x = r.standard_normal((N, d))
        if tensor == "k":
            x[:, _outlier_channels(w, seed, b, h, math.ceil(0.005 * d))] *= 30.0
    else:
        raise ValueError(w.kind)
    return round_to_bf16(x)


def heads_of(w, tensor):
    return w.Hq if tensor in ("q", "do") else w.Hkv


def gen_head(w, tensor, b, h, seed=BASE_SEED):
    """One head [N, d] of ``tensor`` ('q', 'k', 'v' or 'do') as bf16-valued float32."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    if not (0 <= b < w.B and 0 <= h < heads_of(w, tensor)):
        raise IndexError("head (%d, %d) out of range for %s" % (b, h, tensor))
    return _draw_head(w, tensor, b, h, seed)


def gen_tensor(w, tensor, seed=BASE_SEED):
    """Whole tensor [B, H, N, d] as bf16-valued float32."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    H = heads_of(w, tensor)
    out = np.empty((w.B, H, w.N, w.d), dtype=np.float32)
    for b in range(w.B):
        for h in range(H):
            out[b, h] = _draw_head(w, tensor, b, h, seed)
    return out


def sample_rows(N, count=512, seed=BASE_SEED, edge=64):
    """Sorted query rows for sampled parity: the first and last ``edge`` rows plus seeded random ones."""
    edge = min(edge, N // 2)
    if count >= N:
        return np.arange(N)
    fixed = np.concatenate([np.arange(edge), np.arange(N - edge, N)])
    pool = np.setdiff1d(np.arange(N), fixed)
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, N, 77])))
    extra = r.choice(pool, size=max(0, count - fixed.shape[0]), replace=False)
    return np.sort(np.concatenate([fixed, extra]))


# ---- cache forward workloads: Nq new rows against a key/value cache of capacity Nk -------------
@dataclass(frozen=True)
class CacheWorkload:
    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    causal: bool
    kind: str                      # distribution recipe, as for Workload
    len_lo: int                    # valid cache lengths are drawn uniformly in [len_lo, Nk]
    note: str = field(default="", compare=False)


CACHE_WORKLOADS = {
    w.name: w
    for w in [
        CacheWorkload("decode_b8hq32hkv8nk32768d128", 5, 8, 32, 8, 1, 32768, 128, True, "llm_outlier", 8192,
                      note="one new token per sequence; cache lengths U[8192, 32768]; LLM value mix"),
        CacheWorkload("prefill_chunk_b1hq32hkv8nq2048nk32768d128", 6, 1, 32, 8, 2048, 32768, 128, True,
                      "gqa_outlier", 32768,
                      note="the last 2048-token chunk of a 32768-token prompt, causal"),
    ]
}


def gen_cache_head(w, tensor, b, h, seed=BASE_SEED):
    """One head of a cache workload: 'q' [Nq, d], or 'k' / 'v' [Nk, d] (the whole capacity)."""
    if isinstance(w, str):
        w = CACHE_WORKLOADS[w]
    nh = w.Hq if tensor == "q" else w.Hkv
    if not (0 <= b < w.B and 0 <= h < nh):
        raise IndexError("head (%d, %d) out of range for %s" % (b, h, tensor))
    n = w.Nq if tensor == "q" else w.Nk
    shape = Workload(w.name, w.wid, w.B, w.Hq, w.Hkv, n, w.d, w.causal, w.kind)
    return _draw_head(shape, tensor, b, h, seed)


def gen_cache_tensor(w, tensor, seed=BASE_SEED):
    """Whole tensor of a cache workload: q [B, Hq, Nq, d] or k / v [B, Hkv, Nk, d]."""
    if isinstance(w, str):
        w = CACHE_WORKLOADS[w]
    nh, n = (w.Hq, w.Nq) if tensor == "q" else (w.Hkv, w.Nk)
    out = np.empty((w.B, nh, n, w.d), dtype=np.float32)
    for b in range(w.B):
        for h in range(nh):
            out[b, h] = gen_cache_head(w, tensor, b, h, seed)
    return out


def cache_lengths(w, seed=BASE_SEED):
    """Valid cache lengths [B] (int32), seeded, uniform in [len_lo, Nk]."""
    if isinstance(w, str):
        w = CACHE_WORKLOADS[w]
    r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, w.wid, 101])))
    return r.integers(w.len_lo, w.Nk, size=w.B, endpoint=True).astype(np.int32)
