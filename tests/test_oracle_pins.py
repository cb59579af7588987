"""Pins of the fp64 oracle against things other than itself (CPU only).

* finite differences of sum(dO * O) through the oracle's forward, for every
  selection mode, pin the backward's dQ, dK/dV/dKV, dCmpKV and dSinks;
* full-coverage top-k equals dense causal attention: forward O and the
  gradients against torch's CPU fp64 scaled_dot_product_attention + autograd,
  and lse against torch.logsumexp of the dense masked score matrix;
* closed forms (top-1 self-only), invariants (the softmax row sums to one
  with the sink; global sums of dK and dV);
* selection decode and the CSR transpose against brute-force loops.
"""
import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import sparse_attn_oracle as O
from top_sparse_attention_gather_amd import workloads as W
from tests._cases import ALL_TINY, tiny, to_f64_inputs


def _loss(inp, dO):
    pb = O.Problem(inp)
    out, _ = O.sparse_fwd(pb)
    return float((out * dO).sum())


def _fd_check(inp, name, grad, dO, n_probe=40, h=1e-5, seed=0):
    """Central differences on a random subset of elements of inp[name]."""
    rng = np.random.default_rng(seed)
    base = inp[name]
    flat = base.view(-1)
    idxs = rng.choice(flat.numel(), size=min(n_probe, flat.numel()), replace=False)
    g = np.asarray(grad).reshape(-1)
    scale = max(1e-3, float(np.abs(g).max()))
    for i in idxs:
        old = float(flat[i])
        flat[i] = old + h
        lp = _loss(inp, dO)
        flat[i] = old - h
        lm = _loss(inp, dO)
        flat[i] = old
        fd = (lp - lm) / (2 * h)
        assert abs(fd - g[i]) <= 1e-6 * scale + 1e-8, (name, int(i), fd, g[i])


@pytest.mark.parametrize("mode", ALL_TINY)
def test_backward_matches_finite_differences(mode):
    wl = tiny(mode)
    inp = to_f64_inputs(W.make_inputs(wl))
    pb = O.Problem(inp)
    out, lse = O.sparse_fwd(pb)
    dO = inp["d_o"].numpy()
    grads = O.sparse_bwd(pb, torch.from_numpy(out), torch.from_numpy(lse))
    # the loss is sum(dO * O) with dO held fixed
    _fd_check(inp, "q", grads["dq"], dO)
    if wl.kv_shared:
        _fd_check(inp, "kv", grads["dkv"], dO)
    else:
        _fd_check(inp, "k", grads["dk"], dO)
        _fd_check(inp, "v", grads["dv"], dO)
    if "cmp_kv" in inp:
        assert np.abs(grads["dcmp_kv"]).max() > 0
        _fd_check(inp, "cmp_kv", grads["dcmp_kv"], dO)
    if wl.has_sinks:
        _fd_check(inp, "sinks", grads["dsinks"], dO, n_probe=wl.n_q_heads)


def _dense_reference(inp, wl):
    """Dense causal attention through torch (fp64, autograd) for full coverage."""
    q = inp["q"].to(torch.float64).clone()
    if wl.kv_shared:
        kv = inp["kv"].to(torch.float64).clone().requires_grad_(True)
        k, v = kv, kv[..., :wl.d_v]
    else:
        k = inp["k"].to(torch.float64).clone().requires_grad_(True)
        v = inp["v"].to(torch.float64).clone().requires_grad_(True)
    q = q.requires_grad_(True)
    outs = []
    G = wl.group
    cu = wl.cu_seqlens()
    for b in range(wl.batch):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        qb = q[sl].transpose(0, 1)                                  # [Hq, S, d]
        kb = k[sl].transpose(0, 1).repeat_interleave(G, dim=0)      # [Hq, S, d]
        vb = v[sl].transpose(0, 1).repeat_interleave(G, dim=0)
        ob = F.scaled_dot_product_attention(qb, kb, vb, is_causal=True, scale=wl.softmax_scale)
        outs.append(ob.transpose(0, 1))
    out = torch.cat(outs, 0)
    (out * inp["d_o"].to(torch.float64)).sum().backward()
    grads = {"dq": q.grad}
    if wl.kv_shared:
        grads["dkv"] = kv.grad
    else:
        grads["dk"], grads["dv"] = k.grad, v.grad
    # lse of the dense masked scores via torch.logsumexp
    lses = []
    with torch.no_grad():
        for b in range(wl.batch):
            sl = slice(int(cu[b]), int(cu[b + 1]))
            qb = q[sl].transpose(0, 1)
            kb = k[sl].transpose(0, 1).repeat_interleave(G, dim=0)
            s = wl.softmax_scale * qb @ kb.transpose(1, 2)
            S = s.shape[-1]
            s = s.masked_fill(torch.triu(torch.ones(S, S, dtype=torch.bool), 1), float("-inf"))
            lses.append(torch.logsumexp(s, dim=-1).transpose(0, 1))
    return out.detach(), torch.cat(lses, 0), grads


@pytest.mark.parametrize("mode", ["token_gqa", "block_gqa", "mla"])
def test_full_coverage_equals_dense_causal(mode):
    wl = tiny(mode, index_policy="full")
    if wl.select == W.SEL_BLOCK:
        wl = tiny(mode, index_policy="full", topk=(max(wl.seqlens) + wl.block_size - 1) // wl.block_size)
    else:
        wl = tiny(mode, index_policy="full", topk=max(wl.seqlens))
    inp = to_f64_inputs(W.make_inputs(wl))
    pb = O.Problem(inp)
    out, lse = O.sparse_fwd(pb)
    ref_out, ref_lse, ref_g = _dense_reference(inp, wl)
    np.testing.assert_allclose(out, ref_out.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse.numpy(), rtol=1e-12, atol=1e-12)
    g = O.sparse_bwd(pb, torch.from_numpy(out), torch.from_numpy(lse))
    for k, v in ref_g.items():
        np.testing.assert_allclose(g[k], v.numpy(), rtol=1e-10, atol=1e-12, err_msg=k)


@pytest.mark.parametrize("mode", ["token_gqa", "mla"])
def test_self_only_closed_form(mode):
    """top-1 self-only: O = v_t, lse = scale <q, k_t>, dQ = dK = 0,
    dV_t = sum over the group's heads of dO[t, h]."""
    wl = tiny(mode, index_policy="self_only", topk=3)
    inp = W.make_inputs(wl)
    pb = O.Problem(inp)
    out, lse = O.sparse_fwd(pb)
    k = (inp["kv"] if wl.kv_shared else inp["k"]).to(torch.float64).numpy()
    v = k[..., :wl.d_v] if wl.kv_shared else inp["v"].to(torch.float64).numpy()
    q = inp["q"].to(torch.float64).numpy()
    G = wl.group
    for t in range(wl.total_q):
        for h in range(wl.n_q_heads):
            g = h // G
            np.testing.assert_array_equal(out[t, h], v[t, g])
            assert abs(lse[t, h] - wl.softmax_scale * q[t, h] @ k[t, g]) < 1e-12
    # O = v_t is exact in bf16; lse is kept in fp64 so that P = 1 exactly
    Ob, _ = O.round_fwd_outputs(out, lse)
    grads = O.sparse_bwd(pb, Ob, torch.from_numpy(lse))
    assert np.abs(grads["dq"]).max() < 1e-12
    dO = inp["d_o"].to(torch.float64).numpy()
    dv_ref = dO.reshape(wl.total_q, wl.n_kv_heads, G, wl.d_v).sum(axis=2)
    if wl.kv_shared:
        np.testing.assert_allclose(grads["dkv"][..., :wl.d_v], dv_ref, atol=1e-12)
        assert np.abs(grads["dkv"][..., wl.d_v:]).max() < 1e-12
    else:
        assert np.abs(grads["dk"]).max() < 1e-12
        np.testing.assert_allclose(grads["dv"], dv_ref, atol=1e-12)


@pytest.mark.parametrize("mode", ["token_gqa", "token_sinks", "wcmp_sinks"])
def test_softmax_rows_sum_to_one(mode):
    """With every value row = 1, O = sum_j P_j = 1 - P_sink."""
    wl = tiny(mode)
    inp = to_f64_inputs(W.make_inputs(wl))
    if wl.kv_shared:
        # d_v columns of shared KV set to 1; the logits use the whole row
        inp["kv"][..., :wl.d_v] = 1.0
        if "cmp_kv" in inp:
            inp["cmp_kv"][..., :wl.d_v] = 1.0
    else:
        inp["v"][:] = 1.0
    pb = O.Problem(inp)
    out, lse = O.sparse_fwd(pb)
    if wl.has_sinks:
        p_sink = np.exp(inp["sinks"].numpy()[None, :] - lse)
    else:
        p_sink = np.zeros_like(lse)
    np.testing.assert_allclose(out, np.broadcast_to((1 - p_sink)[..., None], out.shape), atol=1e-13)


@pytest.mark.parametrize("mode", ["token_gqa", "block_gqa", "mla", "token_sinks", "wcmp_sinks"])
def test_global_gradient_sums(mode):
    """sum_j dK_j = scale * sum_{t,h} P_sink D q (zero without sinks) and
    sum_j dV_j = sum_{t,h} (1 - P_sink) dO, from the exact (fp64) forward."""
    wl = tiny(mode)
    inp = to_f64_inputs(W.make_inputs(wl))
    pb = O.Problem(inp)
    out, lse = O.sparse_fwd(pb)
    g = O.sparse_bwd(pb, torch.from_numpy(out), torch.from_numpy(lse))
    dO = inp["d_o"].numpy()
    q = inp["q"].numpy()
    D = (dO * out).sum(-1)
    p_sink = np.exp(inp["sinks"].numpy()[None, :] - lse) if wl.has_sinks else np.zeros_like(lse)
    G = wl.group
    for gi in range(wl.n_kv_heads):
        hs = slice(gi * G, (gi + 1) * G)
        dk_sum = wl.softmax_scale * ((p_sink[:, hs] * D[:, hs])[..., None] * q[:, hs]).sum((0, 1))
        dv_sum = ((1 - p_sink[:, hs])[..., None] * dO[:, hs]).sum((0, 1))
        if wl.kv_shared:
            tot = g["dkv"][:, gi].sum(0) + (g["dcmp_kv"][:, gi].sum(0) if "dcmp_kv" in g else 0)
            np.testing.assert_allclose(tot[wl.d_v:], dk_sum[wl.d_v:], atol=1e-12)
            np.testing.assert_allclose(tot[:wl.d_v], dk_sum[:wl.d_v] + dv_sum, atol=1e-12)
        else:
            np.testing.assert_allclose(g["dk"][:, gi].sum(0), dk_sum, atol=1e-12)
            np.testing.assert_allclose(g["dv"][:, gi].sum(0), dv_sum, atol=1e-12)


def _brute_selection(wl, idx, t, g, lens=None):
    """Rows selected by (t, g) from the rules, by plain loops (multiset);
    with `lens`, only slots below lens[t, g] count."""
    if lens is not None:
        idx = idx.copy()
        idx[t, g, max(0, int(lens[t, g])):] = -1
    cu = wl.cu_seqlens()
    b = int(np.searchsorted(cu, t, side="right") - 1)
    tl = t - int(cu[b])
    L = int(cu[b + 1] - cu[b])
    sel = []
    if wl.select == W.SEL_TOKEN:
        for s in range(idx.shape[2]):
            j = int(idx[t, g, s])
            if 0 <= j < L and j <= tl:
                sel.append((0, int(cu[b]) + j))
    elif wl.select == W.SEL_BLOCK:
        for s in range(idx.shape[2]):
            i = int(idx[t, g, s])
            if i < 0:
                continue
            for j in range(i * wl.block_size, (i + 1) * wl.block_size):
                if j < L and j <= tl:
                    sel.append((0, int(cu[b]) + j))
    else:
        for j in range(L):
            if tl - wl.win_left <= j <= tl + wl.win_right and j <= tl:
                sel.append((0, int(cu[b]) + j))
        cuc = wl.cu_seqlens_cmp()
        for s in range(idx.shape[2]):
            j = int(idx[t, g, s])
            if 0 <= j < int(cuc[b + 1] - cuc[b]) and wl.cmp_ratio * j + wl.cmp_ratio - 1 <= tl:
                sel.append((1, int(cuc[b]) + j))
    return sorted(sel)


@pytest.mark.parametrize("mode", ALL_TINY)
@pytest.mark.parametrize("shuffle", [False, True])
def test_selection_and_csr_brute_force(mode, shuffle):
    wl = tiny(mode)
    inp = W.make_inputs(wl)
    idx = inp["idx"].numpy().copy()
    rng = np.random.default_rng(5)
    if shuffle:
        # -1 slots anywhere, a duplicate, and an out-of-range index
        for t in range(idx.shape[0]):
            rng.shuffle(idx[t, 0])
        idx[-1, 0, 0] = idx[-1, 0, 1] = max(0, int(idx[-1, 0].max()))
        idx[-2, 0, -1] = 10_000
        inp["idx"] = torch.from_numpy(idx)
    pb = O.Problem(inp)
    for t in range(wl.total_q):
        for g in range(wl.n_kv_heads):
            srcs, rows = pb.selection(t, g)
            got = sorted(zip(srcs.tolist(), rows.tolist()))
            assert got == _brute_selection(wl, idx, t, g), (t, g)
    # CSR against a dict of lists filled by loops over (t, g, slot) in order
    row_ptr, entries = O.csr_transpose(pb)
    lists = {}
    cu = wl.cu_seqlens()
    for t, g, s in itertools.product(range(wl.total_q), range(wl.n_kv_heads), range(idx.shape[2])):
        j = int(idx[t, g, s])
        b = int(np.searchsorted(cu, t, side="right") - 1)
        tl, L = t - int(cu[b]), int(cu[b + 1] - cu[b])
        if j < 0:
            continue
        if wl.select == W.SEL_TOKEN:
            if j >= L or j > tl:
                continue
            key = (int(cu[b]) + j) * wl.n_kv_heads + g
        elif wl.select == W.SEL_BLOCK:
            bs = wl.block_size
            if j * bs >= L or j * bs > tl:
                continue
            nb_before = sum((int(cu[c + 1] - cu[c]) + bs - 1) // bs for c in range(b))
            key = (nb_before + j) * wl.n_kv_heads + g
        else:
            cuc = wl.cu_seqlens_cmp()
            r = wl.cmp_ratio
            if j >= int(cuc[b + 1] - cuc[b]) or r * j + r - 1 > tl:
                continue
            key = (int(cuc[b]) + j) * wl.n_kv_heads + g
        lists.setdefault(key, []).append((t * wl.n_kv_heads + g) * idx.shape[2] + s)
    assert row_ptr[0] == 0 and row_ptr[-1] == entries.size
    for key in range(row_ptr.size - 1):
        assert entries[row_ptr[key]:row_ptr[key + 1]].tolist() == lists.get(key, []), key


def test_duplicates_are_a_multiset():
    """A duplicated slot counts twice: equal to the same key listed once with
    its value row doubled in weight (checked via FD consistency instead)."""
    wl = tiny("token_gqa")
    inp = to_f64_inputs(W.make_inputs(wl))
    idx = inp["idx"].numpy().copy()
    t = wl.total_q - 1
    idx[t, 0, -1] = idx[t, 0, 0]
    inp["idx"] = torch.from_numpy(idx)
    pb = O.Problem(inp)
    assert pb.selection(t, 0)[1].tolist().count(pb.selection(t, 0)[1][0]) == 2
    out, lse = O.sparse_fwd(pb)
    g = O.sparse_bwd(pb, torch.from_numpy(out), torch.from_numpy(lse))
    _fd_check(inp, "k", g["dk"], inp["d_o"].numpy(), n_probe=30)
    _fd_check(inp, "q", g["dq"], inp["d_o"].numpy(), n_probe=30)


def test_empty_row_has_no_gradient():
    """A row with no valid key and no sink: lse = -inf, O = 0, zero grads."""
    wl = tiny("token_gqa")
    inp = W.make_inputs(wl)
    idx = inp["idx"].numpy().copy()
    idx[3] = -1
    inp["idx"] = torch.from_numpy(idx)
    pb = O.Problem(inp)
    out, lse = O.sparse_fwd(pb)
    assert np.all(np.isneginf(lse[3])) and np.all(out[3] == 0)
    Ob, Lb = O.round_fwd_outputs(out, lse)
    g = O.sparse_bwd(pb, Ob, Lb)
    assert np.all(g["dq"][3] == 0)
    assert all(np.isfinite(v).all() for v in g.values())


def test_empty_row_with_a_sink_is_the_sink_alone():
    """A row with no valid key but a sink: the softmax runs over the sink
    logit alone, so lse = sink exactly, O = 0, and the row has no dQ."""
    wl = tiny("token_sinks")
    inp = W.make_inputs(wl)
    idx = inp["idx"].numpy().copy()
    idx[3] = -1
    inp["idx"] = torch.from_numpy(idx)
    pb = O.Problem(inp)
    out, lse = O.sparse_fwd(pb)
    sinks = inp["sinks"].to(torch.float64).numpy()
    heads = slice(0, wl.n_q_heads)
    np.testing.assert_array_equal(lse[3][heads], sinks)
    assert np.all(out[3] == 0)
    Ob, Lb = O.round_fwd_outputs(out, lse)
    g = O.sparse_bwd(pb, Ob, Lb)
    assert np.all(g["dq"][3] == 0)
    assert all(np.isfinite(v).all() for v in g.values())


@pytest.mark.parametrize("mode", ["token_gqa", "block_gqa", "wcmp_sinks"])
def test_per_row_topk_lengths(mode):
    """Per-row top-k lengths: slots at or past a row's length are unused.
    Pinned by plain loops, and by the equivalence with writing -1 into those
    slots (selection, CSR, forward and backward all identical)."""
    wl = tiny(mode)
    inp = to_f64_inputs(W.make_inputs(wl))
    idx = inp["idx"].numpy()
    rng = np.random.default_rng(9)
    lens = rng.integers(-1, idx.shape[2] + 2, size=idx.shape[:2])      # includes < 0 and > K
    with_len = dict(inp, topk_len=lens)
    masked = dict(inp)
    midx = idx.copy()
    for t in range(idx.shape[0]):
        for g in range(idx.shape[1]):
            midx[t, g, max(0, int(lens[t, g])):] = -1
    masked["idx"] = torch.from_numpy(midx)
    pa, pm = O.Problem(with_len), O.Problem(masked)
    for t in range(wl.total_q):
        for g in range(wl.n_kv_heads):
            sa, ra, qa = pa.selection_positions(t, g)
            sm_, rm, qm = pm.selection_positions(t, g)
            assert np.array_equal(sa, sm_) and np.array_equal(ra, rm) and np.array_equal(qa, qm)
            got = sorted(zip(sa.tolist(), ra.tolist()))
            assert got == _brute_selection(wl, idx, t, g, lens), (t, g)
    for x, y in zip(O.csr_transpose(pa), O.csr_transpose(pm)):
        assert np.array_equal(x, y)
    oa, la = O.sparse_fwd(pa)
    om, lm = O.sparse_fwd(pm)
    assert np.array_equal(oa, om) and np.array_equal(la, lm)
    ga = O.sparse_bwd(pa, torch.from_numpy(oa), torch.from_numpy(la))
    gm = O.sparse_bwd(pm, torch.from_numpy(om), torch.from_numpy(lm))
    for k in ga:
        assert np.array_equal(ga[k], gm[k]), k
