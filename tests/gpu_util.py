"""Helpers of the GPU parity tests: run the HIP path through the C ABI and
the fp64 oracle on the same seeded inputs, and compare."""
import sys

import numpy as np
import torch

from oracle import sparse_attn_oracle as O
from top_sparse_attention_gather_amd import binding as B
from top_sparse_attention_gather_amd import workloads as W
from tests._cases import check_close


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def oracle_fwd_rounded(inputs, tokens=None):
    pb = O.Problem(inputs)
    out, lse = O.sparse_fwd(pb, tokens)
    dt = torch.float16 if getattr(inputs["workload"], "dtype", "bf16") == "fp16" else torch.bfloat16
    Ob, Lb = O.round_fwd_outputs(out, lse, dt)
    return pb, Ob, Lb


def gpu_bwd(wl, inputs, O_bf16, lse_f32, dkv_mode=B.DKV_ATOMIC, l1=False):
    dev = device_inputs(wl, inputs)
    dev["o"] = O_bf16.to("cuda").contiguous()
    dev["lse"] = lse_f32.to("cuda").contiguous()
    desc = B.make_desc(wl, dkv_mode, softmax_l1=int(l1))
    out = B.sparse_attn_bwd(desc, dev)
    torch.cuda.synchronize()
    return {k: v.float().cpu().numpy() for k, v in out.items()}


def device_inputs(wl, inputs):
    return B.device_tensors(inputs)


def compare_all(got, ref, rows=None, tag=""):
    """Compare every output; `rows` optionally restricts dq / dkv rows."""
    keymap = {"dq": "dq", "dk": "dk", "dv": "dv", "dkv": "dkv", "d_cmp_kv": "dcmp_kv", "dsinks": "dsinks",
              "ori_softmax_l1": "ori_l1", "cmp_softmax_l1": "cmp_l1"}
    res = {}
    for k, rk in keymap.items():
        if k not in got:
            continue
        g = got[k].reshape(ref[rk].shape)
        r = ref[rk]
        if rows is not None and k in rows:
            g, r = g[rows[k]], r[rows[k]]
        res[k] = check_close(f"{tag}:{k}", g, r)
        say(f"  {tag} {k}: max_err {res[k][0]:.3e} (bound {res[k][1]:.3e}) rel_frob {res[k][2]:.3e}")
    return res


def oracle_case(wl, inputs=None, l1=False):
    """Inputs, rounded forward outputs and the oracle's backward (plus, with
    l1, its softmax L1-norm outputs as ori_l1 / cmp_l1)."""
    if inputs is None:
        inputs = W.make_inputs(wl)
    pb, Ob, Lb = oracle_fwd_rounded(inputs)
    ref = O.sparse_bwd(pb, Ob, Lb)
    if l1:
        ref.update({k + "_l1": v for k, v in O.softmax_l1_norm(pb, Lb).items()})
    return inputs, Ob, Lb, ref


def run_full_case(wl, inputs=None, dkv_mode=B.DKV_ATOMIC, l1=False, oracle=None):
    """Oracle forward -> rounded O/lse -> GPU backward and oracle backward.
    `oracle`: a precomputed oracle_case(wl, inputs, l1) result."""
    say(f"[case] {wl.name}: seqlens={wl.seqlens[:4]} Hq={wl.n_q_heads} Hkv={wl.n_kv_heads} "
        f"d={wl.d_qk}/{wl.d_v} topk={wl.topk} select={wl.select} mode={dkv_mode} l1={int(l1)}")
    inputs, Ob, Lb, ref = oracle if oracle is not None else oracle_case(wl, inputs, l1)
    got = gpu_bwd(wl, inputs, Ob, Lb, dkv_mode, l1)
    return compare_all(got, ref, tag=wl.name), got, ref
