"""Fake-quantized FlashAttention forward and Attn-QAT backward, float64 CPU oracle.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The method is an approximation (4-bit fake-quantized attention), so this is
the algorithm taken step by step, not a closed-form definition.

Forward (EFQ-Softmax abstract, "exp-then-quantize" path; HiFA4 abstract for
both GEMMs in 4 bits; Attn-QAT abstract for the FP4 forward).  Per query row
i, with Q^, K^ MXFP4 along the head dim and V^ MXFP4 along the sequence:

  m = -inf, l = 0, acc = 0
  for key tiles t = 0, 1, ... of BC = 64 keys, in ascending order
  (causal: only tiles whose first key is <= i; keys j > i masked):
      s_j   = (q^_i . k^_j) * scale
      m_new = max(m, max_j s_j)
      p_j   = exp(s_j - m_new)                       (0 for masked keys)
      P~    = MXFP4(p) over the tile's two 32-key blocks
      alpha = exp(m - m_new)                         (0 while m = -inf)
      l     = alpha * l + sum_j P~_j                 (same P~ as the numerator)
      acc   = alpha * acc + sum_j P~_j v^_j
      m     = m_new
  o_i = acc / l

Readings of what the pages leave open (all listed in the design notes):
the key-tile width BC = 64 and ascending visiting order are part of the
definition of P quantization; the denominator uses the quantized P~; scores
are scaled before the max and exp is the natural exponential; causal masking
is top-left aligned (key j visible iff j <= i); query head h uses KV head
h // (Hq // Hkv).

Cache forward (`attn_fwd_kvcache`: FP4 attention for LLM inference, where the
new rows of a sequence attend to keys and values quantized once and kept):
the same tile loop for Nq new rows placed at the last Nq positions of each
sequence (bottom-right causal alignment), over a cache of per-sequence length
L_b, with V^ quantized over the cache's whole capacity in 32-token blocks
from position 0.  A row that sees no key gives O = 0, m = -inf, l = 0.

Backward (Attn-QAT abstract: scores recomputed with the same FP4 QK^T as
the forward; the D term taken from the FP4 forward's own output).  With the
forward's final m, l per row and straight-through gradients for the four
quantizers:

  D_i   = sum_c dO_ic O_ic
  s^_ij = (q^_i . k^_j) * scale ;  p_ij = exp(s^_ij - m_i) ;  P_ij = p_ij / l_i
  A_ij  = MXFP4(p_i.)_j / l_i   (per 32-key block along j)
  dV_j  = sum_i A_ij dO_i
  dP_ij = dO_i . v^_j ;  dS_ij = P_ij (dP_ij - D_i)
  dQ_i  = scale * sum_j dS_ij k^_j ;  dK_j = scale * sum_i dS_ij q^_i

Parity pins (tests/test_oracle_attention.py): quantizers off -> textbook
softmax attention for several tile widths, causal and GQA; single tile with
quantizers on -> the direct formula; Q = 0 -> mean of V^ (causal: prefix
mean); identical V^ rows -> that row; V -> 2^k V scales O exactly;
quantizers off -> float64 autograd of textbook attention and central finite
differences; Q = 0 with quantizers on -> autograd at (Q^, K^, V^);
quantizers on with all keys in one tile (so that the forward's running max
is the final row max) -> float64 autograd of the fake-quant forward with
straight-through Q^, K^, V^, P~ and a constant row max, causal, GQA, d = 64
and 128 (this fixes which of P, P~ and MXFP4(P) feeds dV and dS);
D = rowsum(P o dP) with quantizers off.  Cache forward
(tests/test_oracle_kvcache.py): quantizers off -> textbook attention over
the visible keys; quantizers on -> rows of the full forward at those
positions; Q = 0 -> mean of V^ over the visible keys (ragged lengths); empty
rows; cache contents past the length have no effect.  NVFP4-style forward
(fmt="nv", tests/test_oracle_nv.py): quantizers off -> textbook attention;
Q = 0 and identical keys -> mean of V^ (causal: prefix mean), l = count;
V -> 2^k V scales O exactly; sampled rows match the full result.
"""

import numpy as np

from .efq import efq_fake_quant
from .mx import fake_quant_mx
from .nv import fake_quant_nv, nv_p_fake_quant, nv_tensor_scale

BC = 64  # key-tile width; part of the definition of P quantization


def _identity(x, axis=-1):
    return np.asarray(x, dtype=np.float64)


def _check_shapes(q, k, v):
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    B, Hq, N, d = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
        raise ValueError("k and v must be [B, Hkv, N, d] matching q")
    if Hq % k.shape[1]:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, k.shape[1], N, d


def softmax_attention(q, k, v, causal=False, scale=None):
    """Textbook softmax(Q K^T * scale) V in float64 (no quantization, no tiling)."""
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, Hq, Hkv, N, d = _check_shapes(q, k, v)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    group = Hq // Hkv
    out = np.empty_like(q)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            s = (q[b, h] @ k[b, g].T) * scale
            if causal:
                s = np.where(np.tril(np.ones((N, N), dtype=bool)), s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            out[b, h] = (e / e.sum(axis=1, keepdims=True)) @ v[b, g]
    return out


def _fwd_rows(q_hat, k_hat, v_hat, limit, scale, bc, fq, p_rule, quant):
    """The tile loop for R query rows of one head: row r sees keys 0 .. limit[r] (none if < 0).

    q_hat [R, d], k_hat, v_hat [Nk, d] (already quantized, Nk a multiple of bc).  A tile is
    visited by the rows that see at least its first key; keys past a row's limit are masked.
    A row that sees no key gets O = 0, m = -inf, l = 0.  Returns (O [R, d], m [R], l [R]).
    """
    R, d = q_hat.shape
    m = np.full(R, -np.inf)
    l = np.zeros(R)
    acc = np.zeros((R, d))
    last = int(limit.max()) if R else -1
    for t in range(last // bc + 1 if last >= 0 else 0):
        keys = np.arange(t * bc, (t + 1) * bc)
        act = limit >= t * bc
        if not act.any():
            continue
        s = (q_hat[act] @ k_hat[keys].T) * scale
        s = np.where(keys[None, :] <= limit[act][:, None], s, -np.inf)
        m_old = m[act]
        m_new = np.maximum(m_old, s.max(axis=1))
        if p_rule == "efq" and quant:
            p_tilde = efq_fake_quant((s - m_new[:, None]) / np.log(2.0), axis=-1)
        else:
            p = np.exp(s - m_new[:, None])
            p_tilde = fq(p, axis=-1)
        alpha = np.where(np.isneginf(m_old), 0.0, np.exp(m_old - m_new))
        l[act] = alpha * l[act] + p_tilde.sum(axis=1)
        acc[act] = alpha[:, None] * acc[act] + p_tilde @ v_hat[keys]
        m[act] = m_new
    O = np.where(l[:, None] > 0, acc / np.where(l > 0, l, 1.0)[:, None], 0.0)
    return O, m, l


def attn_fwd(q, k, v, causal=False, scale=None, bc=BC, quant=True, rows=None, p_rule="exp", fmt="mx",
             nv_tensor_scales=None):
    """Tile-by-tile fake-quantized attention forward.

    q: [B, Hq, N, d]; k, v: [B, Hkv, N, d] (values read exactly as float64).
    rows: optional 1-D array of query rows to compute (rows are independent).
    quant=False replaces all four quantizers by the identity.
    p_rule: "exp" -- P~ = MXFP4(exp(s - m)) (exp-then-quantize, the definition); "efq" -- P~ from
    the EFQ-Softmax codes of the shifted scores (oracle/efq.py, a reading of the pages).
    fmt: "mx" -- MXFP4 operands; "nv" -- the NVFP4-style reading of oracle/nv.py (16-element
    blocks, E4M3 block scales, one fp32 scale per tensor of Q, K and V; P~ per 16 keys), with
    the exp rule only.  nv_tensor_scales: (G_Q, G_K, G_V) of the whole tensors when q, k, v are
    slices of them (default: the scales of q, k, v themselves).
    Returns (O [B, Hq, R, d], m [B, Hq, R], l [B, Hq, R]), float64.
    """
    if p_rule not in ("exp", "efq"):
        raise ValueError("p_rule must be 'exp' or 'efq'")
    if fmt not in ("mx", "nv") or (fmt == "nv" and p_rule != "exp"):
        raise ValueError("fmt must be 'mx', or 'nv' with p_rule 'exp'")
    q, k, v = (np.asarray(t, dtype=np.float64) for t in (q, k, v))
    B, Hq, Hkv, N, d = _check_shapes(q, k, v)
    if N % bc:
        raise ValueError("N must be a multiple of the tile width")
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    fq = fake_quant_mx if quant else _identity
    fq_q = fq_k = fq_v = fq_p = fq
    if fmt == "nv" and quant:
        # one tensor scale per operand, taken over the whole tensor (also when sampling rows)
        gq, gk, gv = (nv_tensor_scales if nv_tensor_scales is not None
                      else [nv_tensor_scale(t)[0] for t in (q, k, v)])
        fq_q = lambda x, axis: fake_quant_nv(x, axis, gq)   # noqa: E731
        fq_k = lambda x, axis: fake_quant_nv(x, axis, gk)   # noqa: E731
        fq_v = lambda x, axis: fake_quant_nv(x, axis, gv)   # noqa: E731
        fq_p = nv_p_fake_quant
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    group = Hq // Hkv
    O = np.empty((B, Hq, R, d))
    M = np.empty((B, Hq, R))
    L = np.empty((B, Hq, R))
    # causal: row i sees keys 0 .. i (top-left alignment); otherwise all N keys
    limit = rows.copy() if causal else np.full(R, N - 1, dtype=np.int64)
    for b in range(B):
        for g in range(Hkv):
            k_hat = fq_k(k[b, g], axis=-1)        # along the head dim
            v_hat = fq_v(v[b, g], axis=0)         # along the sequence
            for h in range(g * group, (g + 1) * group):
                q_hat = fq_q(q[b, h][rows], axis=-1)
                O[b, h], M[b, h], L[b, h] = _fwd_rows(q_hat, k_hat, v_hat, limit, scale, bc, fq_p, p_rule,
                                                      quant)
    return O, M, L


def attn_fwd_kvcache(q, k_cache, v_cache, seqlens=None, causal=False, scale=None, bc=BC,
                     quant=True, rows=None, p_rule="exp"):
    """Forward of Nq new query rows against a cache of keys and values (chunked prefill, decode).

    q: [B, Hq, Nq, d], the queries of the last Nq positions of each sequence;
    k_cache, v_cache: [B, Hkv, Nk, d], Nk a multiple of bc (the cache capacity);
    seqlens: [B] valid cache lengths L_b in [0, Nk] (default Nk); the new rows' keys and values
    are already in the cache, so query i sits at position L_b - Nq + i.
    K^ is quantized per row along d and V^ along the sequence over the whole capacity, in
    32-token blocks from position 0, exactly as the cache itself would be quantized.
    Visible keys: j < L_b, and with causal also j <= L_b - Nq + i (bottom-right alignment).  A row
    that sees no key (causal, L_b - Nq + i < 0, or L_b = 0) gives O = 0, m = -inf, l = 0.
    With Nq = Nk = L_b this is `attn_fwd`.  Returns (O [B, Hq, R, d], m, l [B, Hq, R]).
    """
    if p_rule not in ("exp", "efq"):
        raise ValueError("p_rule must be 'exp' or 'efq'")
    q, k_cache, v_cache = (np.asarray(t, dtype=np.float64) for t in (q, k_cache, v_cache))
    B, Hq, Nq, d = q.shape
    Hkv, Nk = k_cache.shape[1], k_cache.shape[2]
    if k_cache.shape != v_cache.shape or k_cache.shape[0] != B or k_cache.shape[3] != d or Hq % Hkv:
        raise ValueError("k_cache and v_cache must be [B, Hkv, Nk, d] matching q")
    if Nk % bc:
        raise ValueError("the cache capacity must be a multiple of the tile width")
    seqlens = np.full(B, Nk, dtype=np.int64) if seqlens is None else np.asarray(seqlens, dtype=np.int64)
    if seqlens.shape != (B,) or (seqlens < 0).any() or (seqlens > Nk).any():
        raise ValueError("seqlens must be [B] with values in [0, Nk]")
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    fq = fake_quant_mx if quant else _identity
    rows = np.arange(Nq) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rows.shape[0]
    group = Hq // Hkv
    O = np.empty((B, Hq, R, d))
    M = np.empty((B, Hq, R))
    L = np.empty((B, Hq, R))
    for b in range(B):
        Lb = int(seqlens[b])
        limit = (Lb - Nq + rows) if causal else np.full(R, Lb - 1, dtype=np.int64)
        limit = np.minimum(limit, Lb - 1)
        for g in range(Hkv):
            k_hat = fq(k_cache[b, g], axis=-1)
            v_hat = fq(v_cache[b, g], axis=0)
            for h in range(g * group, (g + 1) * group):
                q_hat = fq(q[b, h][rows], axis=-1)
                O[b, h], M[b, h], L[b, h] = _fwd_rows(q_hat, k_hat, v_hat, limit, scale, bc, fq, p_rule, quant)
    return O, M, L


def attn_row_max(q, k, causal=False, scale=None, quant=True, chunk=1024):
    """Final row max m_i = max over visible keys j of (q^_i . k^_j) * scale (float64).

    This is the running max the forward ends with, written as its plain definition; the
    backward's P~ is quantized against it.  Returns [B, Hq, N].
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, Hq, N, d = q.shape
    Hkv = k.shape[1]
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    fq = fake_quant_mx if quant else _identity
    group = Hq // Hkv
    out = np.empty((B, Hq, N))
    for b in range(B):
        for g in range(Hkv):
            k_hat = fq(k[b, g], axis=-1)
            for h in range(g * group, (g + 1) * group):
                q_hat = fq(q[b, h], axis=-1)
                for r0 in range(0, N, chunk):
                    rr = np.arange(r0, min(N, r0 + chunk))
                    s = (q_hat[rr] @ k_hat.T) * scale
                    if causal:
                        s = np.where(np.arange(N)[None, :] <= rr[:, None], s, -np.inf)
                    out[b, h, rr] = s.max(axis=1)
    return out


def attn_bwd(q, k, v, o, do, m, l, causal=False, scale=None, quant=True,
             rows=None, key_blocks=None, chunk=1024):
    """Attn-QAT backward with FP4 recomputation of the scores.

    q, do, o: [B, Hq, N, d]; k, v: [B, Hkv, N, d]; m, l: [B, Hq, N] (the
    forward's final row max and row sum, natural-log units).
    rows: query rows for which dQ is returned (default all).
    key_blocks: indices of 32-key blocks for which dK, dV are returned
    (default all); dK, dV are summed over the query heads sharing a KV head.
    Returns (dQ [B, Hq, R, d], dK [B, Hkv, J, d], dV [B, Hkv, J, d]) with J
    the selected keys in ascending order.
    """
    q, k, v, o, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, o, do))
    m = np.asarray(m, dtype=np.float64)
    l = np.asarray(l, dtype=np.float64)
    B, Hq, Hkv, N, d = _check_shapes(q, k, v)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    fq = fake_quant_mx if quant else _identity
    rows = np.arange(N) if rows is None else np.asarray(rows, dtype=np.int64)
    if key_blocks is None:
        keys = np.arange(N)
    else:
        kb = np.sort(np.asarray(key_blocks, dtype=np.int64))
        keys = (kb[:, None] * 32 + np.arange(32)[None, :]).reshape(-1)
    group = Hq // Hkv
    dQ = np.zeros((B, Hq, rows.shape[0], d))
    dK = np.zeros((B, Hkv, keys.shape[0], d))
    dV = np.zeros((B, Hkv, keys.shape[0], d))

    def probs(q_rows, k_cols, rr, kk, m_h, l_h):
        s = (q_rows @ k_cols.T) * scale
        p = np.exp(s - m_h[rr][:, None])
        if causal:
            p = np.where(kk[None, :] <= rr[:, None], p, 0.0)
        return p, p / l_h[rr][:, None]

    for b in range(B):
        for g in range(Hkv):
            k_hat = fq(k[b, g], axis=-1)
            v_hat = fq(v[b, g], axis=0)
            for h in range(g * group, (g + 1) * group):
                q_hat = fq(q[b, h], axis=-1)
                m_h, l_h = m[b, h], l[b, h]
                D = np.sum(do[b, h] * o[b, h], axis=1)
                # dQ on the requested rows: every key contributes
                p, P = probs(q_hat[rows], k_hat, rows, np.arange(N), m_h, l_h)
                dP = do[b, h][rows] @ v_hat.T
                dS = P * (dP - D[rows][:, None])
                dQ[b, h] = scale * (dS @ k_hat)
                # dK, dV on the requested keys: every row contributes
                for r0 in range(0, N, chunk):
                    rr = np.arange(r0, min(N, r0 + chunk))
                    p, P = probs(q_hat[rr], k_hat[keys], rr, keys, m_h, l_h)
                    A = fq(p, axis=-1) / l_h[rr][:, None]
                    dV[b, g] += A.T @ do[b, h][rr]
                    dP = do[b, h][rr] @ v_hat[keys].T
                    dS = P * (dP - D[rr][:, None])
                    dK[b, g] += scale * (dS.T @ q_hat[rr])
    return dQ, dK, dV
