"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/sparse_attn.h, the ctypes structures match the C
layout, and phase-1 validation returns the documented status codes."""
import ctypes
import os
import re
import subprocess

import pytest

from top_sparse_attention_gather_amd import binding as B
from top_sparse_attention_gather_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sparse_attn.h")


def _declared():
    src = open(HEADER).read()
    return sorted(set(re.findall(r"^\S[^\n(]*?\b(sparse_attn_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_binding_names():
    assert _declared() == sorted(B.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = B.load()
    out = subprocess.run(["nm", "-D", "--defined-only", B.library_path()], capture_output=True, text=True).stdout
    syms = set(re.findall(r"\bT (\w+)", out))
    for name in _declared():
        assert name in syms, name
        assert hasattr(lib, name)


def test_struct_layout_matches_c(tmp_path):
    """Compile a C probe of the header with gcc and compare sizes/offsets."""
    fields = {"sa_desc_t": B.SaDesc, "sa_bwd_args_t": B.SaBwdArgs, "sa_fwd_args_t": B.SaFwdArgs,
              "sa_indexer_desc_t": B.SaIndexerDesc, "sa_indexer_args_t": B.SaIndexerArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "sparse_attn.h"', 'int main(void){']
    for cname, cls in fields.items():
        lines.append(f'printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines.append("return 0;}")
    c = tmp_path / "probe.c"
    c.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.dirname(HEADER), str(c), "-o", str(exe)], check=True)
    got = {}
    for ln in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        a, b, v = ln.split()
        got[(a, b)] = int(v)
    for cname, cls in fields.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert got[(cname, f)] == getattr(cls, f).offset, (cname, f)


def _ws(desc):
    n = ctypes.c_size_t(0)
    return B.load().sparse_attn_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)), n.value


def test_phase1_validation_codes():
    wl = W.WORKLOADS["mla_token_8k"]
    st, n = _ws(B.make_desc(wl))
    assert st == 0 and n > 0
    # fp32 D + fp32 dKV accumulator
    assert n >= 8192 * 64 * 4 + 8192 * 576 * 4
    assert _ws(B.make_desc(wl, n_q_heads=63))[0] == 0          # any head count with one kv head
    cases = {
        "bad layout": (dict(layout=5), 7),
        "bad select": (dict(select=9), 7),
        "bad mode": (dict(dkv_mode=3), 7),
        "nan scale": (dict(scale=float("nan")), 7),
        "heads not divisible": (dict(n_kv_heads=3), 2),
        "d_v > d_qk shared": (dict(d_v=640), 2),
        "unbuilt head dim": (dict(d_qk=96, d_v=96), 3),
        "no batch": (dict(batch=0), 2),
        "topk 0": (dict(topk=0), 2),
        "bad softmax_l1 flag": (dict(softmax_l1=2), 7),
        "bad dtype": (dict(dtype=2), 7),
        "bad mask mode": (dict(mask_causal=3), 7),
    }
    for name, (over, code) in cases.items():
        if name == "heads not divisible":
            d = B.make_desc(wl, n_q_heads=64, n_kv_heads=3)
        else:
            d = B.make_desc(wl, **over)
        assert _ws(d)[0] == code, name
    assert B.load().sparse_attn_bwd_workspace_size(None, None) == 1
    st = B.load().sparse_attn_bwd_workspace_size(ctypes.byref(B.make_desc(wl)), None)
    assert st == 1


def test_softmax_l1_workspace():
    """The L1-norm sums take one fp32 plane per head group of the P kernel:
    T * Hkv * positions * 4 bytes more for the 64-head MLA kernel (which
    serves every dK/dV mode of this shape)."""
    wl = W.WORKLOADS["mla_token_8k"]
    for mode in (B.DKV_ATOMIC, B.DKV_DETERMINISTIC):
        st0, n0 = _ws(B.make_desc(wl, mode))
        st1, n1 = _ws(B.make_desc(wl, mode, softmax_l1=1))
        assert st0 == st1 == 0
        planes = 1                                          # 64 heads: one head group of the MLA kernel
        assert n1 - n0 == planes * wl.total_q * wl.n_kv_heads * wl.topk * 4


def test_atomic_modes_workspace():
    """MLA shape: atomic mode holds one fp32 dKV accumulator (plus the D
    plane), the per-XCD form eight; the per-XCD form is only built for the
    shared-KV MLA kernel."""
    wl = W.WORKLOADS["mla_token_8k"]
    acc = wl.total_kv * wl.d_qk * 4
    st1, n1 = _ws(B.make_desc(wl, B.DKV_ATOMIC))
    st8, n8 = _ws(B.make_desc(wl, B.DKV_ATOMIC_XCD))
    assert st1 == st8 == 0
    assert n8 - n1 == 7 * acc
    assert _ws(B.make_desc(W.WORKLOADS["nsa_block_gqa"], B.DKV_ATOMIC_XCD))[0] == 3
    assert _ws(B.make_desc(wl, 3))[0] == 7


def test_window_cmp_requires_shared_kv():
    wl = W.WORKLOADS["mla_cmp_sinks_varlen"]
    assert _ws(B.make_desc(wl))[0] == 0
    assert _ws(B.make_desc(wl, kv_shared=0))[0] == 3


def test_empty_query_returns_ok_without_launch():
    """T == 0: SA_OK and nothing enqueued (safe without a GPU)."""
    wl = W.small_workload("tiny_token_gqa", seqlens=(0,))
    d = B.make_desc(wl)
    a = B.SaBwdArgs()
    assert B.load().sparse_attn_bwd(ctypes.byref(d), ctypes.byref(a), None, 0, None) == 0
    f = B.SaFwdArgs()
    assert B.load().sparse_attn_fwd(ctypes.byref(d), ctypes.byref(f), None) == 0


def test_status_strings():
    for code in range(8):
        s = B.sparse_attn_status_string(code)
        assert s.startswith(B.STATUS_NAMES[code])


def test_indexer_phase1_validation_codes():
    wl = W.INDEXER_WORKLOADS["indexer_8k"]
    n = ctypes.c_size_t(0)
    lib = B.load()

    def ws(d):
        return lib.sparse_attn_indexer_grad_kl_workspace_size(ctypes.byref(d), ctypes.byref(n))

    assert ws(B.make_indexer_desc(wl)) == 0
    # partial dK~ rows (bf16) + fp32 accumulator at least
    assert n.value >= 8192 * 2048 * 128 * 2 + 8192 * 128 * 4
    assert ws(B.make_indexer_desc(wl, layout=4)) == 7
    assert ws(B.make_indexer_desc(wl, mask_causal=2)) == 7
    assert ws(B.make_indexer_desc(wl, d=64)) == 3
    assert ws(B.make_indexer_desc(wl, n_heads=65)) == 3
    assert ws(B.make_indexer_desc(wl, topk=4096)) == 3
    assert ws(B.make_indexer_desc(wl, topk=0)) == 2
    assert ws(B.make_indexer_desc(wl, batch=0)) == 2
    assert lib.sparse_attn_indexer_grad_kl_workspace_size(None, ctypes.byref(n)) == 1
    # empty query: SA_OK, nothing launched
    e = B.make_indexer_desc(W.small_workload("tiny_token_gqa", seqlens=(0,)), n_heads=4, d=128, topk=16)
    a = B.SaIndexerArgs()
    assert lib.sparse_attn_indexer_grad_kl(ctypes.byref(e), ctypes.byref(a), None, 0, None) == 0


def test_deterministic_workspace_holds_one_chunk_of_partial_rows():
    """Deterministic MLA: the workspace holds the bf16 partial rows of one
    token chunk (one 1152-byte row per (head group, token, position)) plus
    the fp32 dKV accumulator; tokens are chunked so that the partial rows
    stay under 24 GiB (the 32K-token, 128-head shape needs 154 GB of them in
    all).  Atomic mode needs only the accumulators."""
    cap = 24 << 30
    for name, groups in (("mla_token_8k", 1), ("mla_token_32k_local", 2)):
        wl = W.WORKLOADS[name]
        T = wl.total_q
        per_token = groups * wl.n_kv_heads * wl.topk * wl.d_qk * 2
        tc = min(T, max(1, cap // per_token))
        acc = T * wl.n_kv_heads * wl.d_qk * 4
        st, n = _ws(B.make_desc(wl, B.DKV_DETERMINISTIC))
        assert st == 0
        assert tc * per_token + acc <= n <= tc * per_token + acc + (2 << 30), (name, n)
        if name == "mla_token_32k_local":
            assert tc < T and tc * per_token <= cap      # chunked
        st, na = _ws(B.make_desc(wl, B.DKV_ATOMIC))
        assert st == 0
        assert acc <= na < acc + (256 << 20), (name, na)


def test_int32_slot_and_key_counts_are_checked():
    """Slot ids and CSR keys are int32 on the device.  A key space (kv rows
    times kv heads, plus the sentinel) past 2^31 - 1 is rejected; a
    backward whose slots pass 2^31 in all still gets a workspace (tokens are
    chunked so every chunk's slot ids fit); the standalone CSR transpose,
    which writes the slot ids of every token, rejects it."""
    wl = W.WORKLOADS["mla_token_8k"]
    lib = B.load()
    # 2^29 kv rows x 4 kv heads = 2^31 keys
    big_keys = B.make_desc(wl, n_q_heads=4, n_kv_heads=4, seqlen_kv=1 << 29, seqlen_q=1 << 10)
    assert _ws(big_keys)[0] == 2
    # 2^20 tokens x 2048 slots = 2^31 slots: chunked backward is fine
    many_slots = B.make_desc(wl, seqlen_q=1 << 20, seqlen_kv=1 << 20)
    for mode in (B.DKV_ATOMIC, B.DKV_DETERMINISTIC):
        st, n = _ws(B.make_desc(wl, mode, seqlen_q=1 << 20, seqlen_kv=1 << 20))
        assert st == 0 and n > 0
    nk, nws = ctypes.c_int64(0), ctypes.c_size_t(0)
    assert lib.sparse_attn_csr_size(ctypes.byref(many_slots), None, ctypes.byref(nk), ctypes.byref(nws)) == 2
    ok = B.make_desc(wl)
    assert lib.sparse_attn_csr_size(ctypes.byref(ok), None, ctypes.byref(nk), ctypes.byref(nws)) == 0
    assert nk.value == 8192
    # the slots of one (token, kv head set) must fit one chunk
    assert _ws(B.make_desc(wl, n_q_heads=1024, n_kv_heads=1024, topk=1 << 21, seqlen_kv=1 << 10,
                           seqlen_q=1 << 10, d_qk=128, d_v=128, kv_shared=0))[0] == 2
