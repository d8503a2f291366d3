"""Seeded synthetic inputs for the 4-bit paged KV cache.

These generators feed both the HIP library and the CPU oracle with the same
tensors; they hold none of the method's arithmetic (no quantization, no
attention), only random draws and page-table bookkeeping.

Workload shapes follow the pages' Qwen3.8-27B geometry ("SGLang's 4-bit KV
cache: the 56% is exact, the 1.78x is untested", per-token table in "The 56%
survives its own scale, and names the block size": 16 full-attention layers,
4 KV heads, head dim 256) and the INT4 lane ("KV cache in 4 bits: 8.8 instead
of 4.7 full sessions on the same four RTX 5090s": 220,000-token sessions,
1,600-token pages).  The 24 query heads (GQA group 6) are a stated workload
choice; the pages give no query-head count.

Every host-side draw uses ``numpy.random.default_rng(SeedSequence([workload,
layer, stream]))`` with the stream ids below; GPU-side draws (benchmark sizes)
use torch's generator seeded from the same triple.
"""
from __future__ import annotations

import numpy as np

STREAM_K, STREAM_V, STREAM_Q, STREAM_KSCALE, STREAM_VSCALE, STREAM_PERM, STREAM_OUTLIER = range(7)


def rng(workload: int, layer: int, stream: int) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([workload, layer, stream]))


def seed_int(workload: int, layer: int, stream: int) -> int:
    """A 63-bit seed for torch generators, derived from the same triple."""
    return int(np.random.SeedSequence([workload, layer, stream]).generate_state(1, np.uint64)[0] >> np.uint64(1))


def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bfloat16 (round-to-nearest-even, via torch's cast)
    and return them widened back to fp32, so both sides see identical bf16
    inputs."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def kv_outlier_channels(workload: int, layer: int, n_tok: int, num_kv_heads: int, head_dim: int,
                        n_outliers: int = 4, factor: float = 8.0):
    """K, V fp32 ~ N(0,1) [n_tok][Hkv][D]; for each tensor, n_outliers channels
    (drawn independently for K and V) are multiplied by `factor` for every
    token and head."""
    out = []
    for stream, ostream in ((STREAM_K, STREAM_OUTLIER), (STREAM_V, STREAM_OUTLIER + 16)):
        x = rng(workload, layer, stream).standard_normal((n_tok, num_kv_heads, head_dim)).astype(np.float32)
        ch = rng(workload, layer, ostream).choice(head_dim, size=n_outliers, replace=False)
        x[:, :, ch] *= np.float32(factor)
        out.append(x)
    return out[0], out[1]


def kv_lognormal_channels(workload: int, layer: int, n_tok: int, num_kv_heads: int, head_dim: int,
                          sigma: float = 1.0):
    """K, V = exp(N(0, sigma^2)) per (head, channel) times N(0,1) per element,
    rounded to bf16 values (returned as fp32)."""
    out = []
    for stream, sstream in ((STREAM_K, STREAM_KSCALE), (STREAM_V, STREAM_VSCALE)):
        scale = np.exp(sigma * rng(workload, layer, sstream).standard_normal((num_kv_heads, head_dim)))
        x = rng(workload, layer, stream).standard_normal((n_tok, num_kv_heads, head_dim)) * scale[None]
        out.append(to_bf16_values(x.astype(np.float32)))
    return out[0], out[1]


def kv_student_t(workload: int, layer: int, n_tok: int, num_kv_heads: int, head_dim: int, nu: float = 4.0):
    """K, V = t_nu / sqrt(nu / (nu - 2)) (unit-variance heavy tails), bf16 values."""
    out = []
    norm = np.sqrt(nu / (nu - 2.0))
    for stream in (STREAM_K, STREAM_V):
        x = rng(workload, layer, stream).standard_t(nu, (n_tok, num_kv_heads, head_dim)) / norm
        out.append(to_bf16_values(x.astype(np.float32)))
    return out[0], out[1]


def query(workload: int, layer: int, batch: int, num_q_heads: int, head_dim: int) -> np.ndarray:
    """q ~ N(0,1) rounded to bf16 values, [B][Hq][D]."""
    x = rng(workload, layer, STREAM_Q).standard_normal((batch, num_q_heads, head_dim)).astype(np.float32)
    return to_bf16_values(x)


def page_tables(workload: int, batch: int, pages_per_seq: int, num_pages: int | None = None,
                shuffled: bool = False) -> np.ndarray:
    """Block table [B][pages_per_seq] int32.  Identity: sequence b owns pages
    b*pages_per_seq ... in order.  Shuffled: a seeded permutation of the
    physical pool dealt to the sequences in order."""
    n = num_pages if num_pages is not None else batch * pages_per_seq
    assert n >= batch * pages_per_seq
    ids = np.arange(n, dtype=np.int64)
    if shuffled:
        ids = rng(workload, 0, STREAM_PERM).permutation(n)
    return np.ascontiguousarray(ids[: batch * pages_per_seq].reshape(batch, pages_per_seq).astype(np.int32))


def slots_for(block_table: np.ndarray, page_size: int, b: int, t0: int, t1: int) -> np.ndarray:
    """Cache slots (page * page_size + offset) of tokens [t0, t1) of sequence b."""
    t = np.arange(t0, t1, dtype=np.int64)
    return (block_table[b, t // page_size].astype(np.int64) * page_size + t % page_size).astype(np.int32)
