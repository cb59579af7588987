"""The right-hand sides of the full-size global-sum checks
(tests/test_gpu_global_sums.py) against the oracle's own backward on small
shapes: the oracle's dK/dV (or dKV plus dCmpKV) rows, summed, must equal
them up to fp64 rounding.  This pins the helper on the CPU (sinks, window +
cmp, block selection, GQA and 128 heads per kv head)."""
import numpy as np
import pytest
import torch

from oracle import sparse_attn_oracle as O
from top_sparse_attention_gather_amd import workloads as W
from tests.test_gpu_global_sums import _identity_sums


def _wl(**kw):
    base = dict(name="sums_case", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(64,), n_q_heads=2,
                n_kv_heads=1, d_qk=64, d_v=64, kv_shared=False, topk=16, index_policy="uniform_causal", seed=71)
    base.update(kw)
    return W.Workload(**base)


CASES = {
    "token_gqa_g2": _wl(seqlens=(90, 70), n_q_heads=4, n_kv_heads=2, topk=24),
    "block": _wl(select=W.SEL_BLOCK, seqlens=(256,), n_q_heads=4, d_qk=32, d_v=32, topk=3, block_size=16,
                 index_policy="own_block_plus_uniform"),
    "mla_wcmp_sinks": _wl(select=W.SEL_WINDOW_CMP, layout=W.LAYOUT_TND, seqlens=(40, 71), n_q_heads=3,
                          d_qk=48, d_v=32, kv_shared=True, topk=6, win_left=7, win_right=0, cmp_ratio=4,
                          has_sinks=True, index_policy="uniform_causal"),
}


@pytest.mark.parametrize("name", list(CASES))
def test_identity_sums_match_the_oracle_row_sums(name):
    wl = CASES[name]
    inp = W.make_inputs(wl)
    pb = O.Problem(inp)
    out, lse = O.sparse_fwd(pb)
    o = torch.from_numpy(np.asarray(out)).reshape(wl.total_q, wl.n_q_heads, wl.d_v)
    L = torch.from_numpy(np.asarray(lse)).reshape(wl.total_q, wl.n_q_heads)
    ref = O.sparse_bwd(pb, o, L)
    dev = {"q": inp["q"], "d_o": inp["d_o"]}
    if wl.has_sinks:
        dev["sinks"] = inp["sinks"]
    rv, rk = _identity_sums(wl, dev, o, L, chunk=29)
    if wl.kv_shared:
        s = torch.from_numpy(ref["dkv"]).double().sum(0)
        if ref.get("dcmp_kv") is not None:
            s = s + torch.from_numpy(ref["dcmp_kv"]).double().sum(0)
        rhs = rk.clone()
        rhs[:, :wl.d_v] += rv
        pairs = [(s, rhs)]
    else:
        pairs = [(torch.from_numpy(ref["dk"]).double().sum(0), rk),
                 (torch.from_numpy(ref["dv"]).double().sum(0), rv)]
    for s, rhs in pairs:
        assert s.shape == rhs.shape
        np.testing.assert_allclose(s.numpy(), rhs.numpy(), rtol=1e-9, atol=1e-9 * max(1.0, float(rhs.abs().max())))
