"""Single-query (decode) softmax attention over dequantized K/V, in float64
(test infrastructure only).

What the pages fix
------------------
* Attention runs over the K/V values that dequantization gives back,
  x_hat = (Q(x) - zero_point) * scale, computed on the fly inside the
  attention (tbr8.org §5, point 2; yunthe.com "quantization principle").
* K/V of a layer are [heads, seq_len, head_dim] per sequence (yunthe.com,
  "quantization principle").

Readings
--------
* The attention itself is the standard scaled dot-product attention of one
  query token against every stored token of its sequence (the stored tokens
  include the current one): score_t = sm_scale * <q, K_hat_t>,
  p = softmax(score), out = sum_t p_t * V_hat_t.  The pages do not print it;
  ``sm_scale`` is an argument and the workloads use 1 / sqrt(head_dim).
* Grouped-query attention: query head h reads KV head h // (Hq / Hkv).
* An empty context (ctx = 0) gives a zero output.

Several query tokens per sequence (chunked prefill over a cached prefix,
yunthe.com "prefix caching": with the prefix's blocks cached, only the new
tokens are computed; several candidates or draft tokens of one sequence):
* Reading: the n query tokens of a sequence are its last n stored tokens,
  at positions ctx - n .. ctx - 1, and each attends causally to the stored
  tokens up to and including its own position (the usual causal mask of a
  decoder's self-attention; the pages do not print it).
"""

import numpy as np


def decode_attention(q, khat, vhat, sm_scale: float):
    """q: [Hq, D] (any float dtype); khat, vhat: float64 [Hkv, ctx, D].
    Returns float64 [Hq, D]."""
    q = np.asarray(q, np.float64)
    hq, d = q.shape
    hkv, ctx, _ = khat.shape
    if hq % hkv:
        raise ValueError("num_q_heads must be a multiple of num_kv_heads")
    group = hq // hkv
    out = np.zeros((hq, d), np.float64)
    if ctx == 0:
        return out
    for h in range(hq):
        g = h // group
        scores = float(sm_scale) * (khat[g] @ q[h])          # [ctx]
        m = np.max(scores)
        p = np.exp(scores - m)
        out[h] = (p @ vhat[g]) / np.sum(p)
    return out


def paged_decode(pool, tables, ctx_lens, q, sm_scale: float):
    """Decode attention for a batch read through block tables.

    pool: ``paged.PoolArrays``; tables: list of per-sequence block-id lists;
    ctx_lens: tokens per sequence; q: [S, Hq, D].  Returns float64 [S, Hq, D].
    """
    from .paged import gather_dequant
    q = np.asarray(q)
    out = np.zeros(q.shape, np.float64)
    for s, (table, ctx) in enumerate(zip(tables, ctx_lens)):
        khat, vhat = gather_dequant(pool, table, int(ctx))
        out[s] = decode_attention(q[s], khat, vhat, sm_scale)
    return out


def multi_query_attention(q, khat, vhat, sm_scale: float):
    """q: [n, Hq, D], the last n of ctx stored tokens; khat, vhat: float64
    [Hkv, ctx, D].  Query token i (position ctx - n + i) attends to tokens
    0 .. ctx - n + i.  Returns float64 [n, Hq, D]."""
    q = np.asarray(q, np.float64)
    n = q.shape[0]
    ctx = khat.shape[1]
    if n > ctx:
        raise ValueError("more query tokens than stored tokens")
    out = np.zeros(q.shape, np.float64)
    for i in range(n):
        pos = ctx - n + i
        out[i] = decode_attention(q[i], khat[:, :pos + 1], vhat[:, :pos + 1], sm_scale)
    return out


def paged_multi_query(pool, tables, ctx_lens, q_rows, cu_seqlens, sm_scale: float):
    """multi_query_attention for a batch read through block tables: q_rows
    [T, Hq, D] with sequence s's queries at rows cu_seqlens[s] ..
    cu_seqlens[s+1] - 1.  Returns float64 [T, Hq, D]."""
    from .paged import gather_dequant
    q_rows = np.asarray(q_rows)
    out = np.zeros(q_rows.shape, np.float64)
    for s, (table, ctx) in enumerate(zip(tables, ctx_lens)):
        a, b = int(cu_seqlens[s]), int(cu_seqlens[s + 1])
        if b > a:
            khat, vhat = gather_dequant(pool, table, int(ctx))
            out[a:b] = multi_query_attention(q_rows[a:b], khat, vhat, sm_scale)
    return out
