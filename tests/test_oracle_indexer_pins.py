"""Pins of the oracle's sparse lightning-indexer gradient with the KL loss
(CPU only).

* central finite differences of the oracle's loss pin dq~, dK~ and dW;
* full coverage (every causal row selected, slots shuffled with unused slots
  between them) equals the dense formulation written with torch ops and
  differentiated by torch autograd: loss and all three gradients;
* W = 0 gives the closed form loss_t = sum_j p_j log(p_j n_t) (uniform
  softmax over the n_t selected rows) and dq~ = dK~ = 0;
* a target equal to the indexer's own softmax (scores from a plain loop,
  softmax from scipy) gives zero loss and zero gradients;
* a token with no used slot contributes nothing.

Each helper takes the oracle module, so the mutation tests can run the same
pins on a copy of the oracle with a planted mistake.
"""
import dataclasses

import numpy as np
import pytest
import scipy.special
import torch

from oracle import sparse_attn_oracle as O
from top_sparse_attention_gather_amd import workloads as W


def tiny_indexer(**kw):
    base = dict(name="t_indexer", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(14, 14), n_q_heads=4,
                n_kv_heads=1, d_qk=8, d_v=8, kv_shared=True, topk=6, index_policy="uniform_causal", seed=31)
    base.update(kw)
    return W.Workload(**base)


def _inputs(wl, f64=True):
    """Indexer inputs; with f64, widened to fp64 and the target renormalised
    in fp64 (the printed gradient dI = softmax(I) - p is the loss's gradient
    when p sums to one)."""
    inp = W.make_indexer_inputs(wl)
    if f64:
        for k in ("q_idx", "k_idx", "weights", "target"):
            inp[k] = inp[k].to(torch.float64).clone()
        tot = inp["target"].sum(-1, keepdim=True)
        inp["target"] = torch.where(tot > 0, inp["target"] / torch.where(tot > 0, tot, 1), 0)
    return inp


def pin_finite_differences(mod, n_probe=30, h=1e-6):
    wl = tiny_indexer()
    inp = _inputs(wl)
    g = mod.indexer_grad_kl(inp)
    rng = np.random.default_rng(0)
    for name, key in (("q_idx", "dq"), ("k_idx", "dk"), ("weights", "dweights")):
        flat = inp[name].view(-1)
        grad = np.asarray(g[key]).reshape(-1)
        sc = max(1e-3, float(np.abs(grad).max()))
        for i in rng.choice(flat.numel(), size=min(n_probe, flat.numel()), replace=False):
            old = float(flat[i])
            flat[i] = old + h
            lp = mod.indexer_grad_kl(inp)["loss"]
            flat[i] = old - h
            lm = mod.indexer_grad_kl(inp)["loss"]
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[i]) <= 1e-6 * sc + 1e-8, (name, int(i), fd, grad[i])


def pin_dense_autograd(mod, shuffle=True):
    """Every causal row selected: the dense masked formulation in torch."""
    wl = tiny_indexer(index_policy="full", topk=16)
    inp = _inputs(wl)
    idx = inp["idx"].numpy().copy()
    tgt = inp["target"].numpy().copy()
    if shuffle:
        rng = np.random.default_rng(7)
        for t in range(idx.shape[0]):
            perm = rng.permutation(idx.shape[2])
            idx[t, 0] = idx[t, 0, perm]
            tgt[t, 0] = tgt[t, 0, perm]
        inp["idx"] = torch.from_numpy(idx)
        inp["target"] = torch.from_numpy(tgt)
    got = mod.indexer_grad_kl(inp)
    cu = wl.cu_seqlens()
    q = inp["q_idx"].clone().requires_grad_(True)
    k = inp["k_idx"].clone().requires_grad_(True)
    w = inp["weights"].clone().requires_grad_(True)
    loss = torch.zeros((), dtype=torch.float64)
    per_tok = []
    for b in range(wl.batch):
        sl = slice(int(cu[b]), int(cu[b + 1]))
        L = int(cu[b + 1] - cu[b])
        s = torch.einsum("thd,jd->thj", q[sl], k[sl])                 # [L, H, L]
        I = torch.einsum("th,thj->tj", w[sl], torch.relu(s))           # [L, L]
        I = I.masked_fill(torch.triu(torch.ones(L, L, dtype=torch.bool), 1), float("-inf"))
        logs = torch.log_softmax(I, dim=-1)
        # target by key: slot s of token t names key idx[t, 0, s]
        p = torch.zeros(L, L, dtype=torch.float64)
        for t in range(L):
            for sl_ in range(wl.topk):
                j = int(idx[int(cu[b]) + t, 0, sl_])
                if j >= 0:
                    p[t, j] = float(tgt[int(cu[b]) + t, 0, sl_])
        term = torch.xlogy(p, p) - torch.where(p > 0, p * logs, torch.zeros_like(p))
        lt = term.sum(-1)
        per_tok.append(lt.detach())
        loss = loss + lt.sum()
    loss.backward()
    assert abs(got["loss"] - float(loss.detach())) <= 1e-10 * max(1.0, abs(float(loss.detach())))
    np.testing.assert_allclose(got["loss_per_token"], torch.cat(per_tok).numpy(), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(got["dq"], q.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(got["dk"], k.grad.numpy(), rtol=1e-9, atol=1e-12)
    np.testing.assert_allclose(got["dweights"], w.grad.numpy(), rtol=1e-9, atol=1e-12)


def _brute_rows(wl, idx, t):
    cu = wl.cu_seqlens()
    b = int(np.searchsorted(cu, t, side="right") - 1)
    tl = t - int(cu[b])
    L = int(cu[b + 1] - cu[b])
    return [(s, int(cu[b]) + int(idx[t, 0, s])) for s in range(idx.shape[2])
            if 0 <= int(idx[t, 0, s]) < L and int(idx[t, 0, s]) <= tl]


def pin_zero_weights(mod):
    wl = tiny_indexer()
    inp = _inputs(wl)
    inp["weights"][:] = 0.0
    got = mod.indexer_grad_kl(inp)
    idx = inp["idx"].numpy()
    tgt = inp["target"].numpy()
    for t in range(wl.total_q):
        rows = _brute_rows(wl, idx, t)
        p = np.array([tgt[t, 0, s] for s, _ in rows])
        p = p[p > 0]
        exp = float((p * np.log(p * len(rows))).sum()) if rows else 0.0
        assert abs(got["loss_per_token"][t] - exp) <= 1e-12, t
    assert np.all(got["dq"] == 0) and np.all(got["dk"] == 0)


def pin_self_consistent_target(mod):
    """p = softmax of the indexer's own scores: zero loss, zero gradients."""
    wl = tiny_indexer()
    inp = _inputs(wl)
    idx = inp["idx"].numpy()
    q, k, w = inp["q_idx"].numpy(), inp["k_idx"].numpy(), inp["weights"].numpy()
    tgt = np.zeros_like(inp["target"].numpy())
    for t in range(wl.total_q):
        rows = _brute_rows(wl, idx, t)
        if not rows:
            continue
        scores = []
        for _, j in rows:
            scores.append(sum(w[t, h] * max(0.0, float(q[t, h] @ k[j])) for h in range(wl.n_q_heads)))
        for (s, _), v in zip(rows, scipy.special.softmax(np.array(scores))):
            tgt[t, 0, s] = v
    inp["target"] = torch.from_numpy(tgt)
    got = mod.indexer_grad_kl(inp)
    assert abs(got["loss"]) < 1e-12
    for key in ("dq", "dk", "dweights"):
        assert np.abs(got[key]).max() < 1e-12, key


def pin_empty_token(mod):
    wl = tiny_indexer()
    inp = _inputs(wl)
    idx = inp["idx"].numpy().copy()
    idx[5] = -1
    inp["idx"] = torch.from_numpy(idx)
    got = mod.indexer_grad_kl(inp)
    assert got["loss_per_token"][5] == 0 and np.all(got["dq"][5] == 0) and np.all(got["dweights"][5] == 0)


def test_indexer_finite_differences():
    pin_finite_differences(O)


@pytest.mark.parametrize("shuffle", [False, True])
def test_indexer_full_coverage_equals_dense_autograd(shuffle):
    pin_dense_autograd(O, shuffle)


def test_indexer_zero_weights_closed_form():
    pin_zero_weights(O)


def test_indexer_self_consistent_target_is_stationary():
    pin_self_consistent_target(O)


def test_indexer_empty_token():
    pin_empty_token(O)
