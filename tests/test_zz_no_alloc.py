"""The allocation-free backward (sparse_attn_bwd_noalloc) against the
workspace entry point (sparse_attn_bwd): two calls in a row on the fixed
per-GPU workspace, the second with a smaller problem, each compared with
the workspace call on the same inputs (bitwise in deterministic mode, to
the parity bar in atomic mode), and the size limit."""
import ctypes

import numpy as np
import pytest
import torch

from top_sparse_attention_gather_amd import binding as B
from top_sparse_attention_gather_amd import workloads as W
from tests import gpu_util as U
from tests._cases import check_close

SCRATCH = 128 << 20

CALLS = [
    # window + cmp with sinks, varlen, 64 heads: the MLA kernel with D fused
    W.Workload(name="na_wcmp_sinks", select=W.SEL_WINDOW_CMP, layout=W.LAYOUT_TND, seqlens=(64, 203, 37),
               n_q_heads=64, n_kv_heads=1, d_qk=576, d_v=512, kv_shared=True, topk=20, win_left=47, win_right=0,
               cmp_ratio=4, has_sinks=True, index_policy="cmp_uniform_visible", seed=91),
    # smaller: token GQA, 2 kv heads
    W.Workload(name="na_token_gqa", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(96,), n_q_heads=4,
               n_kv_heads=2, d_qk=64, d_v=64, kv_shared=False, topk=24, index_policy="uniform_causal", seed=92),
]


def test_noalloc_rejects_problems_past_the_scratch():
    """Host-side check, no GPU: a problem whose workspace exceeds the fixed
    128 MiB returns SA_ERR_WORKSPACE_TOO_SMALL before any launch."""
    wl = W.WORKLOADS["mla_token_8k"]
    d = B.make_desc(wl, B.DKV_DETERMINISTIC)
    assert B.sparse_attn_bwd_workspace_size(d) > SCRATCH
    a = B.SaBwdArgs()
    assert B.load().sparse_attn_bwd_noalloc(ctypes.byref(d), ctypes.byref(a), None) == 4
    for wl in CALLS:
        for mode in (B.DKV_ATOMIC, B.DKV_DETERMINISTIC):
            assert B.sparse_attn_bwd_workspace_size(B.make_desc(wl, mode)) <= SCRATCH


@pytest.mark.gpu
@pytest.mark.parametrize("mode", ["det", "atomic"])
def test_noalloc_matches_workspace_entry_point(mode):
    dkv_mode = B.DKV_DETERMINISTIC if mode == "det" else B.DKV_ATOMIC
    cases = []
    for wl in CALLS:
        U.say(f"[noalloc] {wl.name} mode {mode}: inputs, forward, workspace call")
        dev = B.device_tensors(W.make_inputs(wl))
        desc = B.make_desc(wl, dkv_mode)
        dev["o"], dev["lse"] = B.sparse_attn_fwd(desc, dev)
        cases.append((wl, desc, dev, B.sparse_attn_bwd(desc, dev)))
    # the two allocation-free calls back to back: the second (smaller) one
    # runs on the scratch contents the first left
    outs = []
    for wl, desc, dev, _ in cases:
        U.say(f"[noalloc] {wl.name} mode {mode}: allocation-free call")
        outs.append(B.sparse_attn_bwd_noalloc(desc, dev))
    torch.cuda.synchronize()
    for (wl, _, _, ref), got in zip(cases, outs):
        assert set(got) == set(ref)
        for k in ref:
            g, r = got[k].float().cpu().numpy(), ref[k].float().cpu().numpy()
            if dkv_mode == B.DKV_DETERMINISTIC:
                assert np.array_equal(g.view(np.uint32), r.view(np.uint32)), (wl.name, k)
            else:
                check_close(f"{wl.name}:{k}", g, r)
