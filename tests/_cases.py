"""Tiny problem builders shared by the CPU pin tests and the GPU parity tests."""
import dataclasses

import numpy as np
import torch

from top_sparse_attention_gather_amd import workloads as W


def tiny(mode: str, **kw) -> W.Workload:
    """Small workloads of every selection mode (oracle pins)."""
    if mode == "token_gqa":
        base = dict(name="t_token_gqa", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(12, 12),
                    n_q_heads=4, n_kv_heads=2, d_qk=8, d_v=6, kv_shared=False, topk=5,
                    index_policy="uniform_causal", seed=11)
    elif mode == "block_gqa":
        base = dict(name="t_block_gqa", select=W.SEL_BLOCK, layout=W.LAYOUT_BSND, seqlens=(16, 16),
                    n_q_heads=4, n_kv_heads=2, d_qk=8, d_v=8, kv_shared=False, topk=3, block_size=4,
                    index_policy="own_block_plus_uniform", seed=12)
    elif mode == "mla":
        base = dict(name="t_mla", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(12,),
                    n_q_heads=3, n_kv_heads=1, d_qk=10, d_v=6, kv_shared=True, topk=5,
                    index_policy="uniform_causal", kv_std=0.5, seed=13)
    elif mode == "wcmp_sinks":
        base = dict(name="t_wcmp", select=W.SEL_WINDOW_CMP, layout=W.LAYOUT_TND, seqlens=(9, 14),
                    n_q_heads=2, n_kv_heads=1, d_qk=10, d_v=6, kv_shared=True, topk=2, win_left=3,
                    win_right=0, cmp_ratio=4, has_sinks=True, index_policy="cmp_uniform_visible",
                    seed=14)
    elif mode == "token_sinks":
        base = dict(name="t_token_sinks", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(10,),
                    n_q_heads=2, n_kv_heads=1, d_qk=8, d_v=8, kv_shared=False, topk=4,
                    has_sinks=True, index_policy="uniform_causal", seed=15)
    else:
        raise ValueError(mode)
    base.update(kw)
    return W.Workload(**base)


ALL_TINY = ["token_gqa", "block_gqa", "mla", "wcmp_sinks", "token_sinks"]


def to_f64_inputs(inp):
    """Copy of a generator dict with every float tensor widened to fp64 (FD)."""
    out = {}
    for k, v in inp.items():
        if isinstance(v, torch.Tensor) and v.is_floating_point():
            out[k] = v.to(torch.float64).clone()
        else:
            out[k] = v
    return out


def check_close(name, got, ref, atol_frac=1e-2, atol_abs=1e-3, frob=5e-3):
    """Per-tensor bar: max|err| <= atol_frac*max|ref| + atol_abs and relative
    Frobenius error <= frob.  Returns (max_err, bound, rel_frob)."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    err = np.abs(got - ref)
    max_err = float(err.max()) if err.size else 0.0
    bound = atol_frac * (float(np.abs(ref).max()) if ref.size else 0.0) + atol_abs
    nref = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(got - ref)) / nref if nref > 0 else float(np.linalg.norm(got - ref))
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    assert max_err <= bound, f"{name}: max|err| {max_err:.3e} > {bound:.3e}"
    assert rel <= frob, f"{name}: rel Frobenius {rel:.3e} > {frob:.1e}"
    return max_err, bound, rel
