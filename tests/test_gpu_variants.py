"""GPU parity of the descriptor variants: explicit per-row top-k lengths,
window-only attention (no cmp table, no index slots), and window + dense cmp
concatenation at another compression ratio (every visible cmp row, r = 8).
Same bar as the other parity tests."""
import dataclasses

import numpy as np
import pytest
import torch

from oracle import sparse_attn_oracle as O
from top_sparse_attention_gather_amd import binding as B
from top_sparse_attention_gather_amd import workloads as W
from tests import gpu_util as U
from tests._cases import check_close
from tests.test_gpu_parity import MODES, SMALL

pytestmark = pytest.mark.gpu


def _lens(wl, seed):
    rng = np.random.default_rng(seed)
    return rng.integers(-1, wl.topk + 2, size=(wl.total_q, wl.n_kv_heads)).astype(np.int32)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", ["token_gqa_d64_g2", "block_gqa_d128", "mla_64h", "mla_wcmp_sinks_varlen"])
def test_per_row_topk_lengths(name, mode):
    """Random per-row lengths (some < 0, some > topk): backward against the
    oracle with the same lengths, L1-norm outputs included; in deterministic
    mode bitwise equal to the call with -1 written past each length."""
    wl = SMALL[name]
    inp = W.make_inputs(wl)
    inp["topk_len"] = _lens(wl, 3)
    res, got, ref = U.run_full_case(wl, inputs=inp, dkv_mode=MODES[mode], l1=True)
    if mode == "det":
        masked = dict(inp)
        idx = inp["idx"].numpy().copy()
        for t in range(idx.shape[0]):
            for g in range(idx.shape[1]):
                idx[t, g, max(0, int(inp["topk_len"][t, g])):] = -1
        masked["idx"] = torch.from_numpy(idx)
        del masked["topk_len"]
        pb, Ob, Lb = U.oracle_fwd_rounded(inp)
        U.say(f"  {name}: masked-index call")
        got_m = U.gpu_bwd(wl, masked, Ob, Lb, MODES[mode], l1=True)
        for k in got:
            assert np.array_equal(got[k].view(np.uint32), got_m[k].view(np.uint32)), k


@pytest.mark.parametrize("name", ["mla_64h", "mla_wcmp_sinks_varlen"])
def test_fwd_per_row_topk_lengths(name):
    wl = SMALL[name]
    inp = W.make_inputs(wl)
    inp["topk_len"] = _lens(wl, 4)
    U.say(f"[fwd lens] {name}")
    out_ref, lse_ref = O.sparse_fwd(O.Problem(inp))
    o, lse = B.sparse_attn_fwd(B.make_desc(wl), B.device_tensors(inp))
    torch.cuda.synchronize()
    check_close(f"{name}:o", o.float().cpu().numpy(), out_ref)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse.cpu().numpy()), fin)
    np.testing.assert_allclose(lse.cpu().numpy()[fin], lse_ref[fin], rtol=0, atol=2e-5 * max(1.0, np.abs(lse_ref[fin]).max()))


@pytest.mark.parametrize("mode", list(MODES))
def test_window_only(mode):
    """Sliding window without cmp rows or index slots (topk = 0): no cmp
    table, cmp offsets or index tensor is passed."""
    wl = W.Workload(name="swa_only", select=W.SEL_WINDOW_CMP, layout=W.LAYOUT_TND, seqlens=(64, 203, 37),
                    n_q_heads=64, n_kv_heads=1, d_qk=576, d_v=512, kv_shared=True, topk=0, win_left=47,
                    win_right=0, cmp_ratio=4, has_sinks=True, index_policy="cmp_uniform_visible", seed=81)
    U.say(f"[swa] {mode}")
    inp = W.make_inputs(wl)
    pb, Ob, Lb = U.oracle_fwd_rounded(inp)
    ref = O.sparse_bwd(pb, Ob, Lb)
    ref.update({k + "_l1": v for k, v in O.softmax_l1_norm(pb, Lb).items()})
    dev = B.device_tensors(inp)
    for k in ("cmp_kv", "cu_seqlens_cmp", "topk_indices"):
        dev.pop(k, None)
    dev["o"], dev["lse"] = Ob.cuda(), Lb.cuda()
    desc = B.make_desc(wl, MODES[mode], total_cmp=0, softmax_l1=1)
    out = B.sparse_attn_bwd(desc, dev)
    torch.cuda.synchronize()
    got = {k: v.float().cpu().numpy() for k, v in out.items()}
    assert "d_cmp_kv" not in got and "cmp_softmax_l1" not in got
    ref.pop("dcmp_kv", None)
    ref.pop("cmp_l1", None)
    U.compare_all(got, ref, tag="swa_only")


@pytest.mark.parametrize("mode", list(MODES))
def test_window_dense_cmp_ratio8(mode):
    """Window + every visible cmp row (dense concatenation) at cmp_ratio 8."""
    wl = W.Workload(name="cfa_r8", select=W.SEL_WINDOW_CMP, layout=W.LAYOUT_TND, seqlens=(64, 203, 37),
                    n_q_heads=64, n_kv_heads=1, d_qk=576, d_v=512, kv_shared=True, topk=26, win_left=31,
                    win_right=0, cmp_ratio=8, has_sinks=True, index_policy="full", seed=82)
    U.run_full_case(wl, dkv_mode=MODES[mode], l1=True)


ALIGNED = {
    # MLA token selection, one sequence of 96 queries over 160 kv rows
    "mla_q96_kv160": W.Workload(name="mla_q96_kv160", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(96,),
                                kv_seqlens=(160,), n_q_heads=64, n_kv_heads=1, d_qk=576, d_v=512, kv_shared=True,
                                topk=64, kv_std=0.5, mask_causal=2, seed=83),
    # block selection (d 128, blocks of 32), varlen with longer and equal kv sequences
    "block_varlen": W.Workload(name="block_varlen", select=W.SEL_BLOCK, layout=W.LAYOUT_TND, seqlens=(128, 200),
                               kv_seqlens=(256, 200), n_q_heads=16, n_kv_heads=1, d_qk=128, d_v=128,
                               kv_shared=False, topk=5, block_size=32, index_policy="own_block_plus_uniform",
                               mask_causal=2, seed=84),
    # window + cmp with sinks, varlen, kv longer than the queries
    "wcmp_varlen": W.Workload(name="wcmp_varlen", select=W.SEL_WINDOW_CMP, layout=W.LAYOUT_TND, seqlens=(64, 120),
                              kv_seqlens=(100, 150), n_q_heads=64, n_kv_heads=1, d_qk=576, d_v=512, kv_shared=True,
                              topk=12, win_left=31, win_right=0, cmp_ratio=4, has_sinks=True,
                              index_policy="cmp_uniform_visible", mask_causal=2, seed=85),
}


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", list(ALIGNED))
def test_s1_ne_s2_ends_aligned(name, mode):
    """Query and kv sequences of different lengths with the ends-aligned
    causal mask (L1-norm outputs included)."""
    U.run_full_case(ALIGNED[name], dkv_mode=MODES[mode], l1=True)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", list(ALIGNED))
def test_seqused_padding(name, mode):
    """seqused: padding query rows get dq = 0, padding kv / cmp rows are
    never selected (gradient 0), against the oracle with the same counts."""
    wl = ALIGNED[name]
    if wl.layout == W.LAYOUT_BSND:
        wl = dataclasses.replace(wl, layout=W.LAYOUT_TND)
    inp = W.make_inputs(wl)
    rng = np.random.default_rng(6)
    inp["seqused_q"] = np.array([int(rng.integers(L // 2, L + 1)) for L in wl.seqlens], np.int32)
    inp["seqused_kv"] = np.array([int(rng.integers(L // 2, L + 1)) for L in wl.kv_lens], np.int32)
    if wl.select == W.SEL_WINDOW_CMP:
        inp["seqused_cmp"] = np.array([int(rng.integers(c // 2, c + 1)) for c in wl.cmp_seqlens], np.int32)
    res, got, ref = U.run_full_case(wl, inputs=inp, dkv_mode=MODES[mode], l1=True)
    cq = wl.cu_seqlens()
    pad = np.concatenate([np.arange(cq[b] + inp["seqused_q"][b], cq[b + 1]) for b in range(wl.batch)])
    assert np.all(got["dq"].reshape(ref["dq"].shape)[pad] == 0)


def test_fwd_s1_ne_s2_ends_aligned_seqused():
    wl = ALIGNED["wcmp_varlen"]
    inp = W.make_inputs(wl)
    inp["seqused_q"] = np.array([50, 120], np.int32)
    inp["seqused_kv"] = np.array([90, 141], np.int32)
    U.say("[fwd aligned]")
    out_ref, lse_ref = O.sparse_fwd(O.Problem(inp))
    o, lse = B.sparse_attn_fwd(B.make_desc(wl), B.device_tensors(inp))
    torch.cuda.synchronize()
    check_close("wcmp_varlen:o", o.float().cpu().numpy(), out_ref)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse.cpu().numpy()), fin)
    np.testing.assert_allclose(lse.cpu().numpy()[fin], lse_ref[fin], rtol=0, atol=2e-5 * max(1.0, np.abs(lse_ref[fin]).max()))


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", ["token_gqa_d128_g20", "block_gqa_d128", "mla_64h", "mla_wcmp_sinks_varlen"])
def test_fp16_inputs(name, mode):
    """fp16 q, k/v/kv, cmp_kv, O, dO and gradients (fp16 MFMA, fp32
    accumulation) against the oracle on the same fp16 values."""
    wl = dataclasses.replace(SMALL[name], dtype="fp16")
    res, got, ref = U.run_full_case(wl, dkv_mode=MODES[mode], l1=True)


@pytest.mark.parametrize("name", ["block_gqa_d128", "mla_wcmp_sinks_varlen"])
def test_fwd_fp16(name):
    wl = dataclasses.replace(SMALL[name], dtype="fp16")
    inp = W.make_inputs(wl)
    U.say(f"[fwd fp16] {name}")
    out_ref, lse_ref = O.sparse_fwd(O.Problem(inp))
    o, lse = B.sparse_attn_fwd(B.make_desc(wl), B.device_tensors(inp))
    torch.cuda.synchronize()
    assert o.dtype == torch.float16
    check_close(f"{name}:o", o.float().cpu().numpy(), out_ref)
    np.testing.assert_allclose(lse.cpu().numpy(), lse_ref, rtol=0, atol=2e-5 * max(1.0, np.abs(lse_ref).max()))
