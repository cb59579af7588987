"""GPU parity of the shared-KV 576/512 kernels off their home shape: head
counts per kv head that are not a multiple of 64 (SparseFlashMlaGrad
README, constraints: 1 to 128 query heads), rows of more than one
2048-position compaction pass, and fp16 inputs (the README's parameter
table: BFLOAT16 or FLOAT16) at full size; and the edge cases of the index
lists (padding in any slot, duplicates, out-of-range indices, empty rows
with sinks) on these kernels."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import sparse_attn_oracle as O
from top_sparse_attention_gather_amd import binding as B
from top_sparse_attention_gather_amd import workloads as W
from tests import gpu_util as U
from tests._cases import check_close
from tests.test_gpu_parity import _sampled_full_size_case

pytestmark = pytest.mark.gpu

MODES = {"atomic": B.DKV_ATOMIC, "det": B.DKV_DETERMINISTIC, "xcd": B.DKV_ATOMIC_XCD}


def _mla(heads, **kw):
    base = dict(name=f"mla_{heads}h_masked", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(160,),
                n_q_heads=heads, n_kv_heads=1, d_qk=576, d_v=512, kv_shared=True, topk=96, kv_std=0.5,
                seed=100 + heads)
    base.update(kw)
    return W.Workload(**base)


_ORACLE = {}


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("heads", [1, 16, 48, 96])
def test_bwd_mla_masked_heads(heads, mode):
    """1, 16 and 48 heads: one 64-head group with 63, 48 and 16 heads
    masked; 96 heads: a full group and one with 32 masked.  Every output row,
    with the softmax L1-norm outputs."""
    wl = _mla(heads)
    if heads not in _ORACLE:
        _ORACLE.clear()
        _ORACLE[heads] = U.oracle_case(wl, l1=True)
    U.say(f"[mla heads={heads}] {mode}")
    res, _, _ = U.run_full_case(wl, dkv_mode=MODES[mode], l1=True, oracle=_ORACLE[heads])
    assert "ori_softmax_l1" in res


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("heads", [1, 8, 20, 48, 96])
def test_fwd_mla_masked_heads(heads, dtype):
    wl = _mla(heads, dtype=dtype)
    inp = W.make_inputs(wl)
    U.say(f"[fwd mla heads={heads} {dtype}]")
    out_ref, lse_ref = O.sparse_fwd(O.Problem(inp))
    o, lse = B.sparse_attn_fwd(B.make_desc(wl), B.device_tensors(inp))
    torch.cuda.synchronize()
    check_close(f"fwd {heads}h {dtype}:o", o.float().cpu().numpy(), out_ref)
    np.testing.assert_allclose(lse.cpu().numpy(), lse_ref, rtol=0, atol=2e-5 * max(1.0, np.abs(lse_ref).max()))


# up to 4200 positions per row: the late tokens take three compaction passes
# (2048 + 2048 + 104)
MLA_3PASS = W.Workload(name="mla_rows_3_passes", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(4400,),
                       n_q_heads=64, n_kv_heads=1, d_qk=576, d_v=512, kv_shared=True, topk=4200, kv_std=0.5,
                       seed=111)


@pytest.mark.parametrize("mode", list(MODES))
def test_bwd_mla_rows_of_three_passes(mode):
    _sampled_full_size_case(MLA_3PASS, n_tail=8, n_early=3, dkv_mode=MODES[mode])
    assert int((W.make_index_inputs(MLA_3PASS)["idx"].numpy()[-1] >= 0).sum()) > 4096


@pytest.mark.parametrize("mode", ["det", "atomic"])
def test_bwd_mla_fp16_full_size_sampled(mode):
    """The MLA 8K workload in fp16 (the same draws rounded to fp16), every
    dKV row and sampled dq rows, on the 64-head kernel."""
    wl = dataclasses.replace(W.WORKLOADS["mla_token_8k"], dtype="fp16", name="mla_token_8k_fp16")
    _sampled_full_size_case(wl, dkv_mode=MODES[mode])


def test_fwd_mla_rows_of_three_passes_fp16():
    wl = dataclasses.replace(MLA_3PASS, dtype="fp16", name="mla_rows_3_passes_fp16")
    inp = W.make_inputs(wl)
    U.say("[fwd 3 passes fp16]")
    o, lse = B.sparse_attn_fwd(B.make_desc(wl), B.device_tensors(inp))
    torch.cuda.synchronize()
    toks = [0, 2047, 2048, 4095, 4096, 4300, 4399]
    out_ref, lse_ref = O.sparse_fwd(O.Problem(inp), toks)
    sel = torch.tensor(toks, device=o.device)
    check_close("fwd 3 passes fp16:o", o[sel].float().cpu().numpy(), out_ref)
    np.testing.assert_allclose(lse[sel].cpu().numpy(), lse_ref, rtol=0, atol=2e-5 * max(1.0, np.abs(lse_ref).max()))


def _mla_edge_inputs(dtype="bf16"):
    """20 heads with sinks (one 64-head group, 44 masked): -1 shuffled into
    any slot, a duplicated index, an out-of-range index, and rows with no
    valid key (lse = the sink alone)."""
    wl = dataclasses.replace(_mla(20, dtype=dtype), name=f"mla_edge_{dtype}", has_sinks=True, seed=141)
    inp = W.make_inputs(wl)
    idx = inp["idx"].numpy().copy()
    rng = np.random.default_rng(11)
    for t in range(idx.shape[0]):
        rng.shuffle(idx[t, 0])
    idx[150, 0, 0] = idx[150, 0, 1] = 7          # duplicate
    idx[151, 0, 2] = 5000                          # out of range -> unused
    idx[60] = -1                                   # no valid key
    idx[61, 0, :] = -1
    inp["idx"] = torch.from_numpy(idx)
    return wl, inp


_EDGE = {}


@pytest.mark.parametrize("mode", list(MODES))
def test_bwd_mla_edge_padding_duplicates_empty_rows(mode):
    """The MLA backward on shuffled padding, a duplicate, an out-of-range
    index and empty rows with sinks: every output row against the oracle;
    an empty row's dq is 0 and its dsinks term still counts (SparseFlashMlaGrad
    README, Stage 3: dSinks over every row)."""
    if not _EDGE:
        wl, inp = _mla_edge_inputs()
        _EDGE["case"] = (wl, U.oracle_case(wl, inp, l1=True))
    wl, orc = _EDGE["case"]
    U.say(f"[mla edge] {mode}")
    res, got, ref = U.run_full_case(wl, dkv_mode=MODES[mode], l1=True, oracle=orc)
    assert "dsinks" in res
    assert np.all(got["dq"].reshape(ref["dq"].shape)[60] == 0)
    l1 = got["ori_softmax_l1"].reshape(ref["ori_l1"].shape)
    assert np.all(l1[60] == 0) and np.all(l1[61] == 0)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fwd_mla_edge_padding_duplicates_empty_rows(dtype):
    """The MLA forward on the same edge cases: an empty row's O is 0 and its
    lse is the sink logit (aclnnNsaSelectedAttentionInfer, "Formula", with the
    sink in the softmax denominator)."""
    wl, inp = _mla_edge_inputs(dtype)
    U.say(f"[fwd mla edge {dtype}]")
    out_ref, lse_ref = O.sparse_fwd(O.Problem(inp))
    o, lse = B.sparse_attn_fwd(B.make_desc(wl), B.device_tensors(inp))
    torch.cuda.synchronize()
    o = o.float().cpu().numpy()
    lse = lse.cpu().numpy()
    check_close(f"fwd edge {dtype}:o", o, out_ref)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=2e-5 * max(1.0, np.abs(lse_ref).max()))
    assert np.all(o[60] == 0) and np.all(o[61] == 0)
    np.testing.assert_allclose(lse[60], inp["sinks"].numpy(), rtol=1e-6)
