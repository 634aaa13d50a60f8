"""Seeded synthetic inputs for the decode and store workloads.

Random numbers and shapes only: no quantization, allocation or attention
arithmetic lives here.  The same draws feed the HIP path and the CPU oracle.

Workloads (shapes stand in for the pages' examples: the Llama-2-7B batch-32,
length-4096 case of deepinsea.top "pain points"; the LLaMA-70B grouped-query
serving of yunthe.com "monitoring and evaluation"; mean lengths 500-2000 from
deepinsea.top "best practice"; shared prompt prefixes from yunthe.com "prefix
caching"):

* ``tiny``           1 layer, 2 heads, D 64, bs 16, a 64-block pool in seeded
                     random order, 4 sequences of {1, 17, 50, 100} tokens,
                     K/V/Q ~ N(0,1) fp16, INT8 K and V.
* ``llama7b``        32 heads (MHA), D 128, bs 16, 32 sequences of 4096
                     tokens; K and V ~ N(0,1) times a per-(KV head, dim)
                     factor ~ LogNormal(0, 0.5) drawn separately for K and V
                     (outlier channels); Q ~ N(0,1); INT8 K and V; a pool of
                     exactly the needed 8192 blocks in random order.
* ``gqa70b``         64 query heads over 8 KV heads, D 128, bs 32, 128
                     sequences of U{500..2000} tokens; INT8 K, INT4 V; inputs
                     N(0,1) with an independent 1 % of entries (K, V and Q)
                     multiplied by 8.
* ``prefill_store``  64 prompts x 2048 tokens, 32 KV heads, D 128, N(0,1),
                     stored as bs-16 INT8 blocks into a 16384-block pool in
                     random order.
* ``shared_prefix``  32 sequences of 32768 tokens whose first 4096 are one
                     shared prefix, bs 32, 32 heads x D 128, INT8 K / INT4 V,
                     N(0,1), 512-token split-K partitions.
* ``llama7b_fp8``, ``gqa70b_fp8``  the same shapes and draws with FP8 E4M3 K
                     and V (the cache dtype yunthe.com "vLLM deployment"
                     names); ``llama7b_i8a`` with INT8 asymmetric V.
* ``prefill_chunk``  chunked prefill over a cached prefix (yunthe.com "prefix
                     caching": only the new tokens are computed): 32
                     sequences of 4096 stored tokens whose last 512 are the
                     queries, llama7b's heads, channel factors and codecs;
                     queries N(0,1).
* ``prefill_chunk_gqa``  the same over gqa70b's heads and codecs (64 query
                     heads on 8 KV heads, bs 32, INT8 K / INT4 V), 16
                     sequences of 4096 tokens, 512 queries each.
"""

from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    v_codec: str                   # "i8", "i4", "i8a" or "fp8" (K: see k_codec)
    ctx_kind: str                  # "fixed", "list", "uniform"
    ctx: tuple = ()                # fixed: (n,), list: lengths, uniform: (lo, hi)
    channel_sigma: float = 0.0     # LogNormal sigma of per-(head, dim) factors
    outlier_frac: float = 0.0
    outlier_mult: float = 1.0
    prefix: int = 0                # shared prefix tokens
    pool_blocks: int = 0           # 0: exactly the blocks needed
    partition: int = 0             # split-K partition tokens (0: library default)
    seed: int = 0
    q_len: int = 0                 # query tokens per sequence (multi-query workloads)
    store_only: bool = False       # measured as quantize-and-store (no attention)
    k_codec: str = ""              # "" : FP8 with FP8 V, else INT8; or "i4" (INT4 K, V "i4" or "i8")
    extra: dict = field(default_factory=dict, compare=False, hash=False)


WORKLOADS = {
    "tiny": Workload("tiny", 4, 2, 2, 64, 16, "i8", "list", (1, 17, 50, 100),
                     pool_blocks=64, seed=1),
    "llama7b": Workload("llama7b", 32, 32, 32, 128, 16, "i8", "fixed", (4096,),
                        channel_sigma=0.5, seed=2),
    "gqa70b": Workload("gqa70b", 128, 64, 8, 128, 32, "i4", "uniform", (500, 2000),
                       outlier_frac=0.01, outlier_mult=8.0, seed=3),
    "prefill_store": Workload("prefill_store", 64, 32, 32, 128, 16, "i8", "fixed", (2048,),
                              pool_blocks=16384, seed=4, store_only=True),
    "shared_prefix": Workload("shared_prefix", 32, 32, 32, 128, 32, "i4", "fixed", (32768,),
                              prefix=4096, partition=512, seed=5),
    "llama7b_fp8": Workload("llama7b_fp8", 32, 32, 32, 128, 16, "fp8", "fixed", (4096,),
                            channel_sigma=0.5, seed=2),
    "llama7b_i8a": Workload("llama7b_i8a", 32, 32, 32, 128, 16, "i8a", "fixed", (4096,),
                            channel_sigma=0.5, seed=2),
    "gqa70b_fp8": Workload("gqa70b_fp8", 128, 64, 8, 128, 32, "fp8", "uniform", (500, 2000),
                           outlier_frac=0.01, outlier_mult=8.0, seed=3),
    "prefill_chunk": Workload("prefill_chunk", 32, 32, 32, 128, 16, "i8", "fixed", (4096,),
                              channel_sigma=0.5, q_len=512, seed=6),
    "prefill_chunk_gqa": Workload("prefill_chunk_gqa", 16, 64, 8, 128, 32, "i4", "fixed", (4096,),
                                  q_len=512, seed=7),
    # INT4 K (tbr8.org §3: blocks in INT8 or even INT4): the llama7b and
    # gqa70b shapes with INT4 K and INT4 or INT8 V, the same draws
    "llama7b_k4v4": Workload("llama7b_k4v4", 32, 32, 32, 128, 16, "i4", "fixed", (4096,),
                             channel_sigma=0.5, seed=2, k_codec="i4"),
    "llama7b_k4v8": Workload("llama7b_k4v8", 32, 32, 32, 128, 16, "i8", "fixed", (4096,),
                             channel_sigma=0.5, seed=2, k_codec="i4"),
    "gqa70b_k4": Workload("gqa70b_k4", 128, 64, 8, 128, 32, "i4", "uniform", (500, 2000),
                          outlier_frac=0.01, outlier_mult=8.0, seed=3, k_codec="i4"),
}


def k_codec_of(w: Workload) -> str:
    """The workload's K codec: its own when set, else FP8 with FP8 V and
    INT8 symmetric otherwise."""
    if w.k_codec:
        return w.k_codec
    return "fp8" if w.v_codec == "fp8" else "i8"


def context_lengths(w: Workload) -> np.ndarray:
    if w.ctx_kind == "fixed":
        return np.full(w.num_seqs, w.ctx[0], np.int64)
    if w.ctx_kind == "list":
        return np.array(w.ctx, np.int64)
    rng = np.random.default_rng([w.seed, 1])
    return rng.integers(w.ctx[0], w.ctx[1] + 1, w.num_seqs).astype(np.int64)


def free_order(w: Workload, num_blocks: int) -> np.ndarray:
    """Seeded random permutation of the pool's block ids."""
    return np.random.default_rng([w.seed, 2]).permutation(num_blocks).astype(np.int32)


def channel_factors(w: Workload):
    """Per-(KV head, dim) factors for K and for V (ones when sigma = 0)."""
    shape = (w.num_kv_heads, w.head_dim)
    if w.channel_sigma <= 0:
        return np.ones(shape, np.float32), np.ones(shape, np.float32)
    rng = np.random.default_rng([w.seed, 3])
    ck = rng.lognormal(0.0, w.channel_sigma, shape).astype(np.float32)
    cv = rng.lognormal(0.0, w.channel_sigma, shape).astype(np.float32)
    return ck, cv


def _gen(device, *key):
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence(list(key)).generate_state(1, np.uint64)[0] >> 1))
    return g


def _draw(w: Workload, shape, device, key, factor=None):
    g = _gen(device, w.seed, *key)
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if w.outlier_frac > 0:
        mask = torch.rand(shape, generator=g, device=device) < w.outlier_frac
        x = torch.where(mask, x * w.outlier_mult, x)
    if factor is not None:
        x = x * torch.as_tensor(factor, device=device)
    return x.to(torch.float16)


def kv_tokens(w: Workload, key, n_tokens: int, device="cpu"):
    """fp16 K and V rows [n_tokens, Hkv, D] for one stream of tokens; ``key``
    names the stream (a sequence index, or "prefix")."""
    ck, cv = channel_factors(w)
    tag = 1_000_000 if key == "prefix" else int(key)
    shape = (n_tokens, w.num_kv_heads, w.head_dim)
    k = _draw(w, shape, device, (10, tag), ck if w.channel_sigma > 0 else None)
    v = _draw(w, shape, device, (11, tag), cv if w.channel_sigma > 0 else None)
    return k, v


def queries(w: Workload, device="cpu", step: int = 0):
    """fp16 queries [S, Hq, D] for decode step ``step``."""
    return _draw(w, (w.num_seqs, w.num_q_heads, w.head_dim), device, (12, step))


def multi_queries(w: Workload, device="cpu"):
    """fp16 query rows [S * q_len, Hq, D] of a multi-query workload, sequence
    s's at rows s * q_len .. (s + 1) * q_len - 1."""
    return _draw(w, (w.num_seqs * w.q_len, w.num_q_heads, w.head_dim), device, (13,))
