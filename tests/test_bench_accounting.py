"""Host-side checks of bench.py's accounting (no GPU): the FLOPs per selected
pair follow from the products each pass forms, the pair counts from the
index lists, and a multi-GPU request is refused."""
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from top_sparse_attention_gather_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _products_bwd(d_qk, d_v):
    # per (query head, selected row): S = q.k (d_qk), dP = dO.v (d_v),
    # dQ += dS k (d_qk), dK += dS q (d_qk), dV += P dO (d_v); 2 FLOPs each
    return 2 * (d_qk + d_v + d_qk + d_qk + d_v)


def _products_fwd(d_qk, d_v):
    # S = q.k (d_qk) and O += P v (d_v)
    return 2 * (d_qk + d_v)


@pytest.mark.parametrize("name", ["mla_token_8k", "nsa_block_gqa", "mla_cmp_sinks_varlen", "tiny_token_gqa"])
def test_flops_per_pair_from_the_products(name):
    wl = W.WORKLOADS[name]
    assert bench.flops_per_pair(wl) == wl.group * _products_bwd(wl.d_qk, wl.d_v)
    assert bench.fwd_flops_per_pair(wl) == wl.group * _products_fwd(wl.d_qk, wl.d_v)


def test_mla_8k_selected_kv_flops():
    # 64 heads, 576/512: 2 * 64 * (3 * 576 + 2 * 512) = 352 256 FLOPs per pair
    wl = W.WORKLOADS["mla_token_8k"]
    assert bench.flops_per_pair(wl) == 352256
    assert bench.fwd_flops_per_pair(wl) == 139264


def test_token_pairs_are_the_non_negative_slots():
    wl = W.small_workload("mla_token_8k", seqlens=(300,), topk=64)
    idx = W.make_indices(wl)
    assert bench.valid_pairs(wl, idx) == int((idx >= 0).sum())
    # causal uniform selection: token t has min(t + 1, topk) rows
    T = wl.total_q
    expect = sum(min(t + 1, wl.topk) for t in range(T)) * wl.n_kv_heads
    assert bench.valid_pairs(wl, idx) == expect


def test_multi_gpu_request_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_stored_traffic_is_keyed_to_its_kernel_source(monkeypatch):
    """roofline.traffic is a stored counter reading: it is reported only
    while the kernel source it was taken on is unchanged (SHA-256), and is
    null otherwise."""
    import hashlib
    for key, t in bench.MEASURED_TRAFFIC.items():
        path = os.path.join(ROOT, t["kernel_source"])
        assert os.path.exists(path), key
        with open(path, "rb") as f:
            current = hashlib.sha256(f.read()).hexdigest()
        got = bench.measured_traffic(*key)
        assert got == (t["fetch_bytes"] + t["write_bytes"] if current == t["sha256"] else None), key
    key = next(iter(bench.MEASURED_TRAFFIC))
    stale = dict(bench.MEASURED_TRAFFIC[key], sha256="0" * 64)
    monkeypatch.setitem(bench.MEASURED_TRAFFIC, key, stale)
    assert bench.measured_traffic(*key) is None
    f = bench.traffic_fields(*key)
    assert f["traffic"] is None and "not valid" in f["traffic_source"]
