"""GPU parity where the dK/dV (dKV) reduction is long: every output row of
shared-KV 576/512 cases whose key rows are named by thousands of (token,
slot) entries, against the fp64 oracle, in every dK/dV mode (the per-XCD
atomic form included).

SparseFlashMlaGrad README, "Computation formula", Stage 3: dKV of a row
collects scale dS^T Q + P^T dO from every query that gathered it
(aclnnSparseFlashAttentionGrad, "Formula", Phase 3: dK[u], dV[u]).  The
deterministic MLA path rounds each (token, key) contribution to bf16
before the fp32 key-major sum, so these cases check that the error does
not grow with the length of a key's list: besides the whole tensor, the
bar is applied to the rows with the longest lists, and the relative
Frobenius error of each band of list lengths is printed.
"""
import numpy as np
import pytest

from top_sparse_attention_gather_amd import binding as B
from top_sparse_attention_gather_amd import workloads as W
from tests import gpu_util as U
from tests._cases import check_close

pytestmark = pytest.mark.gpu

CASES = {
    # every token selects its whole causal prefix (top-2048 over 2048
    # tokens): key j is named by 2048 - j entries, key 0 by 2048
    "mla_dense_prefix_2k": W.Workload(
        name="mla_dense_prefix_2k", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(2048,), n_q_heads=64,
        n_kv_heads=1, d_qk=576, d_v=512, kv_shared=True, topk=2048, kv_std=0.5, seed=83),
    # the long-context pattern at a smaller size: 128 heads, half of the 384
    # indices from a 512-token local window, half over the prefix
    "mla_128h_local_1536": W.Workload(
        name="mla_128h_local_1536", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(1536,), n_q_heads=128,
        n_kv_heads=1, d_qk=576, d_v=512, kv_shared=True, topk=384, kv_std=1.0, seed=84,
        index_policy="local_half", local_window=512),
}

MODES = {"atomic": B.DKV_ATOMIC, "det": B.DKV_DETERMINISTIC, "xcd": B.DKV_ATOMIC_XCD}

_ORACLE = {}


def _oracle(name):
    if name not in _ORACLE:
        _ORACLE.clear()
        U.say(f"[reuse] {name}: oracle forward + backward")
        _ORACLE[name] = U.oracle_case(CASES[name])
    return _ORACLE[name]


def _list_lengths(inputs, n_rows):
    """Entries naming each kv row (the length of its CSR list)."""
    idx = inputs["idx"].numpy().reshape(-1)
    return np.bincount(idx[idx >= 0], minlength=n_rows)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("name", list(CASES))
def test_bwd_every_row_long_key_lists(name, mode):
    wl = CASES[name]
    inputs, Ob, Lb, ref = _oracle(name)
    U.say(f"[reuse] {name}: GPU backward, mode {mode}")
    got = U.gpu_bwd(wl, inputs, Ob, Lb, MODES[mode])
    res = U.compare_all(got, ref, tag=f"{name}/{mode}")
    assert set(res) == {"dq", "dkv"}
    g = got["dkv"].reshape(ref["dkv"].shape)[:, 0].astype(np.float64)
    r = ref["dkv"][:, 0]
    n = _list_lengths(inputs, r.shape[0])
    order = np.argsort(-n, kind="stable")
    # the 64 rows with the longest lists must meet the bar on their own
    top = order[:64]
    check_close(f"{name}/{mode}:dkv longest lists", g[top], r[top])
    # error by band of list length (printed for the record)
    edges = [1, 64, 256, 1024, 1536, 4096]
    for lo, hi in zip(edges[:-1], edges[1:]):
        sel = (n >= lo) & (n < hi)
        if not sel.any():
            continue
        rel = float(np.linalg.norm(g[sel] - r[sel]) / np.linalg.norm(r[sel]))
        U.say(f"  {name}/{mode} dkv rows with {lo}-{hi - 1} entries: {int(sel.sum())} rows, "
              f"rel_frob {rel:.3e}, longest {int(n[sel].max())}")
    assert int(n.max()) >= (2048 if name == "mla_dense_prefix_2k" else 500)
