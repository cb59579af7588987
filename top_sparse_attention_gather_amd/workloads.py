"""Seeded synthetic workloads for the sparse-attention backward.

This module only *creates inputs*: shapes, seeded normal tensors rounded to
bf16, and the top-k index lists (with -1 padding) that stand in for the
output of an upstream top-k selector.  It holds none of the attention
arithmetic, so both the fp64 oracle (tests) and the HIP path (tests, bench)
can draw from it without sharing any of the method.

Workload shapes follow the five cases that the sparse-attention backward is
exercised on: a tiny token-sparse GQA case, an NSA-style block-sparse GQA
case, the shared-KV MLA token-sparse case (the headline), a compressed
sparse MLA case with a sliding window, attention sinks and variable-length
sequences, and a long-context MLA case at one GPU's share.  The selection
rules (which keys a query may pick) are those of the pages:
  * aclnnSparseFlashAttentionGrad, "Formula": keys/values are gathered by
    topkIndices, each index naming a piece of block_size rows;
  * SparseFlashMlaGrad README, "Computation formula", Stage 1: with
    cmp_ratio = 4 the selected KV is the original KV (here a sliding window)
    concatenated with rows of cmp_kv gathered by the indices.

Conventions (shared with the C ABI):
  * token-major tensors: q [T, Hq, d_qk], d_o [T, Hq, d_v], lse [T, Hq];
    kv tensors [T_kv, Hkv, d]; indices [T, Hkv, K] int32.
  * BSND is [B, S, N, D] row-major, i.e. T = B*S with the same memory.
  * TND uses cu_seqlens (int32 [B+1], cu[0] = 0).
  * index values are sequence-local row numbers; any negative value is an
    unused slot; valid slots are written first in ascending order with -1 at
    the tail (kernels must nevertheless accept -1 anywhere).
"""
from __future__ import annotations

import dataclasses
import math
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

SEL_TOKEN = 0
SEL_BLOCK = 1
SEL_WINDOW_CMP = 2

LAYOUT_BSND = 0
LAYOUT_TND = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """Static description of one synthetic problem (sizes + sampling policy)."""

    name: str
    select: int                      # SEL_TOKEN / SEL_BLOCK / SEL_WINDOW_CMP
    layout: int                      # LAYOUT_BSND / LAYOUT_TND
    seqlens: tuple                   # per-sequence query lengths (and kv lengths unless kv_seqlens)
    n_q_heads: int
    n_kv_heads: int
    d_qk: int
    d_v: int
    kv_shared: bool                  # MLA: V is the first d_v columns of KV
    topk: int                        # index slots per (token, kv head)
    block_size: int = 1
    win_left: int = 0                # window (SEL_WINDOW_CMP): keys [t-win_left, t+win_right]
    win_right: int = 0
    cmp_ratio: int = 1
    has_sinks: bool = False
    scale: float = 0.0               # 0 -> 1/sqrt(d_qk)
    index_policy: str = "uniform_causal"
    kv_std: float = 1.0
    cmp_noise_std: float = 0.1
    seed: int = 0
    kv_seqlens: tuple = ()           # per-sequence kv lengths when they differ from the query's
    dtype: str = "bf16"              # format of the 16-bit tensors: "bf16" or "fp16"
    mask_causal: int = 1             # 1: key <= query position (top-left); 2: aligned at the ends (bottom-right)
    local_window: int = 4096         # "local_half": the window the first half of the indices comes from

    # -- derived sizes -------------------------------------------------
    @property
    def batch(self) -> int:
        return len(self.seqlens)

    @property
    def total_q(self) -> int:
        return int(sum(self.seqlens))

    @property
    def kv_lens(self) -> tuple:
        return tuple(self.kv_seqlens) if self.kv_seqlens else tuple(self.seqlens)

    @property
    def total_kv(self) -> int:
        return int(sum(self.kv_lens))

    @property
    def cmp_seqlens(self) -> tuple:
        if self.select != SEL_WINDOW_CMP:
            return tuple(0 for _ in self.seqlens)
        return tuple(s // self.cmp_ratio for s in self.kv_lens)

    def q_offset(self, b: int) -> int:
        """Key position of query 0 of sequence b: 0 (top-left), or kv length
        minus query length when the masks align the sequences' ends."""
        return self.kv_lens[b] - self.seqlens[b] if self.mask_causal == 2 else 0

    @property
    def total_cmp(self) -> int:
        return int(sum(self.cmp_seqlens))

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale != 0.0 else 1.0 / math.sqrt(self.d_qk)

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def cu_seqlens_kv(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.kv_lens)]).astype(np.int32)

    def cu_seqlens_cmp(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.cmp_seqlens)]).astype(np.int32)


def _bsnd(name, B, S, Hq, Hkv, dqk, dv, shared, topk, **kw) -> Workload:
    return Workload(name=name, layout=LAYOUT_BSND, seqlens=tuple([S] * B), n_q_heads=Hq,
                    n_kv_heads=Hkv, d_qk=dqk, d_v=dv, kv_shared=shared, topk=topk, **kw)


# The five workloads (sizes and sampling rules as stated with each).
WORKLOADS: Dict[str, Workload] = {
    # Tiny token-sparse GQA: B=1, S=128, 2 query heads on 1 KV head, d=64,
    # top-16 tokens per query drawn without replacement from [0, t], always
    # including t; all of [0, t] when t < 15.
    "tiny_token_gqa": _bsnd("tiny_token_gqa", 1, 128, 2, 1, 64, 64, False, 16,
                            select=SEL_TOKEN, index_policy="self_plus_uniform", seed=1001),
    # NSA-style block-sparse GQA: B=2, S=4096, 16 query heads per KV head,
    # d=128, 16 blocks of 64 rows per query, own block always included and
    # causally masked inside.
    "nsa_block_gqa": _bsnd("nsa_block_gqa", 2, 4096, 16, 1, 128, 128, False, 16,
                           select=SEL_BLOCK, block_size=64, index_policy="own_block_plus_uniform",
                           seed=1002),
    # MLA shared-KV token-sparse: B=1, S=8192, 64 heads, latent KV 576 (V =
    # first 512), top-2048 uniform over the causal range, KV scaled by 0.5.
    "mla_token_8k": _bsnd("mla_token_8k", 1, 8192, 64, 1, 576, 512, True, 2048,
                          select=SEL_TOKEN, index_policy="uniform_causal", kv_std=0.5, seed=1003),
    # Compressed sparse MLA with sinks, varlen: lengths {1024, 3000, 6000,
    # 16000}, window of the last 128 tokens + top-512 rows of cmp_kv
    # (cmp_ratio 4), per-head fp32 sink logits.
    "mla_cmp_sinks_varlen": Workload(
        name="mla_cmp_sinks_varlen", select=SEL_WINDOW_CMP, layout=LAYOUT_TND,
        seqlens=(1024, 3000, 6000, 16000), n_q_heads=64, n_kv_heads=1, d_qk=576, d_v=512,
        kv_shared=True, topk=512, win_left=127, win_right=0, cmp_ratio=4, has_sinks=True,
        index_policy="cmp_uniform_visible", seed=1004),
    # Long-context MLA at one GPU's share: S=32768, 128 heads, top-2048 with
    # half the indices from a 4096-token local window, half over the prefix.
    "mla_token_32k_local": _bsnd("mla_token_32k_local", 1, 32768, 128, 1, 576, 512, True, 2048,
                                 select=SEL_TOKEN, index_policy="local_half", seed=1005),
}

WORKLOAD_ORDER = ["tiny_token_gqa", "nsa_block_gqa", "mla_token_8k", "mla_cmp_sinks_varlen",
                  "mla_token_32k_local"]

# Sparse lightning-indexer gradient with the KL loss (the indexer that picks
# the top-k rows: aclnnSparseLightningIndexerGradKLLoss).  n_q_heads is the
# indexer's query heads per token, d_qk = d_v its head dim; the indexer key
# is one row per token (n_kv_heads = 1).  The index lists use the same
# policies as above; the target distribution is a random point of the
# simplex over each token's used slots.
INDEXER_WORKLOADS: Dict[str, Workload] = {
    # 8K tokens, 64 indexer heads of dim 128, top-2048 uniform over the
    # causal range (the index lists of the MLA 8K workload's shape).
    "indexer_8k": _bsnd("indexer_8k", 1, 8192, 64, 1, 128, 128, True, 2048,
                        select=SEL_TOKEN, index_policy="uniform_causal", seed=1006),
}


def small_workload(base: str, **overrides) -> Workload:
    """A copy of a named workload with some fields overridden (tests)."""
    return dataclasses.replace(WORKLOADS[base], **overrides)


# ----------------------------------------------------------------------------
# seeded generation
# ----------------------------------------------------------------------------

_STREAMS = ["q", "kv", "v", "do", "idx", "sinks", "cmp_noise", "iq", "ik", "iw", "ip"]
_CHUNK_ELEMS = 1 << 22


def _streams(seed: int) -> Dict[str, np.random.SeedSequence]:
    children = np.random.SeedSequence(seed).spawn(len(_STREAMS))
    return dict(zip(_STREAMS, children))


def _normal_f32(ss: np.random.SeedSequence, shape: Sequence[int], std: float = 1.0,
                threads: int = 8) -> np.ndarray:
    """N(0, std^2) fp32 array, generated in fixed-size chunks from spawned
    child streams so the values do not depend on the thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, (n + _CHUNK_ELEMS - 1) // _CHUNK_ELEMS)
    kids = ss.spawn(nchunks)

    def fill(i):
        lo = i * _CHUNK_ELEMS
        hi = min(n, lo + _CHUNK_ELEMS)
        g = np.random.Generator(np.random.PCG64(kids[i]))
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        if std != 1.0:
            out[lo:hi] *= np.float32(std)

    if nchunks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(max_workers=threads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _to_bf16(a: np.ndarray, dtype: str = "bf16") -> torch.Tensor:
    """Round-to-nearest-even fp32 -> bf16 (or fp16 with dtype="fp16"),
    torch's conversion."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.to(torch.float16 if dtype == "fp16" else torch.bfloat16)


def _rows_self_plus_uniform(rng, t: int, k: int) -> np.ndarray:
    if t + 1 <= k - 1:
        return np.arange(t + 1)
    pick = rng.choice(t, size=k - 1, replace=False)
    return np.sort(np.concatenate([pick, [t]]))


def _rows_uniform(rng, n: int, k: int) -> np.ndarray:
    """k distinct values from [0, n) (all of them when n <= k), ascending."""
    if n <= k:
        return np.arange(n)
    return np.sort(rng.choice(n, size=k, replace=False))


def _rows_local_half(rng, t: int, k: int, window: int) -> np.ndarray:
    if t + 1 <= k:
        return np.arange(t + 1)
    half = k // 2
    lo = max(0, t - window + 1)
    local = lo + rng.choice(t + 1 - lo, size=half, replace=False)
    mask = np.ones(t + 1, dtype=bool)
    mask[local] = False
    cand = np.flatnonzero(mask)
    rest = cand[rng.choice(cand.size, size=k - half, replace=False)]
    return np.sort(np.concatenate([local, rest]))


def make_indices(wl: Workload, rng: Optional[np.random.Generator] = None) -> np.ndarray:
    """int32 [T, Hkv, K] index lists for the workload's policy (-1 tail)."""
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(_streams(wl.seed)["idx"]))
    T, Hkv, K = wl.total_q, wl.n_kv_heads, wl.topk
    out = np.full((T, Hkv, K), -1, dtype=np.int32)
    tok = 0
    for b, L in enumerate(wl.seqlens):
        Lkv = wl.kv_lens[b]
        for tq in range(L):
            # the last key the query may see (its own position in key
            # coordinates, inside the kv sequence); none when negative
            t = min(tq + wl.q_offset(b), Lkv - 1)
            if t < 0:
                continue
            for g in range(Hkv):
                if wl.index_policy == "self_plus_uniform":
                    rows = _rows_self_plus_uniform(rng, t, K)
                elif wl.index_policy == "uniform_causal":
                    rows = _rows_uniform(rng, t + 1, K)
                elif wl.index_policy == "local_half":
                    rows = _rows_local_half(rng, t, K, wl.local_window)
                elif wl.index_policy == "own_block_plus_uniform":
                    own = t // wl.block_size
                    rows = np.sort(np.concatenate([_rows_uniform(rng, own, K - 1), [own]]))
                elif wl.index_policy == "cmp_uniform_visible":
                    # cmp row j summarises tokens [r*j, r*j + r - 1]; it may be
                    # picked once all of them are in the past of t.
                    visible = (t + 1) // wl.cmp_ratio
                    rows = _rows_uniform(rng, visible, K)
                elif wl.index_policy == "full":
                    # every causal row / block / cmp row (coverage tests)
                    if wl.select == SEL_BLOCK:
                        n = t // wl.block_size + 1
                    elif wl.select == SEL_WINDOW_CMP:
                        n = (t + 1) // wl.cmp_ratio
                    else:
                        n = t + 1
                    rows = np.arange(min(n, K))
                elif wl.index_policy == "self_only":
                    rows = np.array([t])
                else:
                    raise ValueError(f"unknown index policy {wl.index_policy!r}")
                out[tok + tq, g, :rows.size] = rows
        tok += L
    return out


def make_index_inputs(wl: Workload) -> Dict[str, object]:
    """Only the index lists and sequence offsets of `wl` (no tensors)."""
    return {"workload": wl, "idx": torch.from_numpy(make_indices(wl)),
            "cu_seqlens": torch.from_numpy(wl.cu_seqlens()), "cu_seqlens_cmp": torch.from_numpy(wl.cu_seqlens_cmp())}


def make_inputs(wl: Workload, with_indices: bool = True, threads: int = 8) -> Dict[str, object]:
    """Seeded bf16 inputs for `wl` on the CPU (torch tensors), plus metadata.

    Keys: q, d_o, and either (k, v) or kv; cmp_kv (window+cmp); sinks;
    idx (int32 [T, Hkv, K]); cu_seqlens, cu_seqlens_cmp (int32).
    O and lse are *not* produced here: they are the forward's outputs.
    """
    st = _streams(wl.seed)
    T, Hq, Hkv = wl.total_q, wl.n_q_heads, wl.n_kv_heads
    out: Dict[str, object] = {"workload": wl}
    out["q"] = _to_bf16(_normal_f32(st["q"], (T, Hq, wl.d_qk), threads=threads), wl.dtype)
    if wl.kv_shared:
        kv32 = _normal_f32(st["kv"], (wl.total_kv, Hkv, wl.d_qk), std=wl.kv_std, threads=threads)
        out["kv"] = _to_bf16(kv32, wl.dtype)
    else:
        out["k"] = _to_bf16(_normal_f32(st["kv"], (wl.total_kv, Hkv, wl.d_qk), std=wl.kv_std,
                                        threads=threads), wl.dtype)
        out["v"] = _to_bf16(_normal_f32(st["v"], (wl.total_kv, Hkv, wl.d_v), std=wl.kv_std,
                                        threads=threads), wl.dtype)
    out["d_o"] = _to_bf16(_normal_f32(st["do"], (T, Hq, wl.d_v), threads=threads), wl.dtype)
    if wl.select == SEL_WINDOW_CMP:
        # cmp_kv row j of a sequence = mean of its ori rows [r*j, r*j + r), taken
        # in fp32 over the bf16 values, plus N(0, noise_std^2) noise, rounded to bf16.
        ori = (out["kv"] if wl.kv_shared else out["k"]).to(torch.float32).numpy()
        noise = _normal_f32(st["cmp_noise"], (wl.total_cmp, Hkv, wl.d_qk), std=wl.cmp_noise_std,
                            threads=threads)
        cmp = np.empty_like(noise)
        cu, cuc = wl.cu_seqlens_kv(), wl.cu_seqlens_cmp()
        r = wl.cmp_ratio
        for b in range(wl.batch):
            n = int(cuc[b + 1] - cuc[b])
            seg = ori[cu[b]:cu[b] + n * r].reshape(n, r, Hkv, wl.d_qk)
            cmp[cuc[b]:cuc[b + 1]] = seg.mean(axis=1, dtype=np.float32)
        cmp += noise
        out["cmp_kv"] = _to_bf16(cmp, wl.dtype)
    if wl.has_sinks:
        g = np.random.Generator(np.random.PCG64(st["sinks"]))
        out["sinks"] = torch.from_numpy(g.standard_normal(Hq, dtype=np.float32))
    out["cu_seqlens"] = torch.from_numpy(wl.cu_seqlens())
    out["cu_seqlens_kv"] = torch.from_numpy(wl.cu_seqlens_kv())
    out["cu_seqlens_cmp"] = torch.from_numpy(wl.cu_seqlens_cmp())
    if with_indices:
        out["idx"] = torch.from_numpy(make_indices(wl))
    return out


def make_indexer_inputs(wl: Workload, with_indices: bool = True, threads: int = 8) -> Dict[str, object]:
    """Seeded inputs of an indexer-gradient problem (CPU torch tensors).

    Keys: q_idx [T, Hq, d] bf16 and k_idx [T_kv, d] bf16 (N(0, 1)),
    weights [T, Hq] fp32 (N(0, 1 / (Hq d)), so the scores spread over a
    few units), idx [T, 1, K] int32, target [T, 1, K] fp32 (per token a
    Dirichlet(1) draw over the used slots, i.e. normalised Exp(1) weights,
    0 on unused slots), cu_seqlens.
    """
    st = _streams(wl.seed)
    T, Hq, d = wl.total_q, wl.n_q_heads, wl.d_qk
    out: Dict[str, object] = {"workload": wl}
    out["q_idx"] = _to_bf16(_normal_f32(st["iq"], (T, Hq, d), threads=threads))
    out["k_idx"] = _to_bf16(_normal_f32(st["ik"], (wl.total_kv, d), threads=threads))
    out["weights"] = torch.from_numpy(_normal_f32(st["iw"], (T, Hq), std=1.0 / math.sqrt(Hq * d),
                                                  threads=threads))
    out["cu_seqlens"] = torch.from_numpy(wl.cu_seqlens())
    out["cu_seqlens_kv"] = torch.from_numpy(wl.cu_seqlens_kv())
    out["cu_seqlens_cmp"] = torch.from_numpy(wl.cu_seqlens_cmp())
    if with_indices:
        idx = make_indices(wl)
        g = np.random.Generator(np.random.PCG64(st["ip"]))
        u = g.standard_exponential(idx.shape, dtype=np.float32)
        u[idx < 0] = 0.0
        tot = u.sum(axis=-1, keepdims=True)
        out["idx"] = torch.from_numpy(idx)
        out["target"] = torch.from_numpy(np.where(tot > 0, u / np.where(tot > 0, tot, 1), 0).astype(np.float32))
    return out


def expected_pair_count(wl: Workload) -> int:
    """Closed-form count of valid (token, kv-head, key-row) pairs for the
    five standard policies (cross-checked against the generated indices)."""
    total = 0
    for L in wl.seqlens:
        t = np.arange(L, dtype=np.int64)
        if wl.select == SEL_TOKEN:
            if wl.index_policy == "self_plus_uniform":
                per = np.minimum(t + 1, wl.topk)
            else:
                per = np.minimum(t + 1, wl.topk)
        elif wl.select == SEL_BLOCK:
            own = t // wl.block_size
            per = wl.block_size * np.minimum(own, wl.topk - 1) + (t % wl.block_size) + 1
        else:
            per = np.minimum(t + 1, wl.win_left + 1) + np.minimum((t + 1) // wl.cmp_ratio, wl.topk)
        total += int(per.sum())
    return total * wl.n_kv_heads
