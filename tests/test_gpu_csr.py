"""CSR transpose of the index lists on the GPU: bit-exact against the
oracle's counting sort (row_ptr and entries), including shuffled -1
padding, duplicates and out-of-range indices, and at full workload sizes."""
import numpy as np
import pytest
import torch

from oracle import sparse_attn_oracle as O
from top_sparse_attention_gather_amd import binding as B
from top_sparse_attention_gather_amd import workloads as W
from tests import gpu_util as U
from tests.test_gpu_parity import SMALL

pytestmark = pytest.mark.gpu


def _gpu_csr(wl, inputs):
    desc = B.make_desc(wl)
    dev = B.device_tensors(inputs)
    cu_kv = dev.get("cu_seqlens_cmp") if wl.select == W.SEL_WINDOW_CMP else dev.get("cu_seqlens_kv")
    if wl.select == W.SEL_WINDOW_CMP and cu_kv is None:
        cu_kv = inputs["cu_seqlens_cmp"].cuda()
    rp, ent = B.sparse_attn_csr_transpose(desc, dev["topk_indices"], dev.get("cu_seqlens_q"), cu_kv,
                                          host_cu_seqlens_kv=inputs["cu_seqlens"].tolist())
    torch.cuda.synchronize()
    return rp.cpu().numpy().astype(np.int64), ent.cpu().numpy().astype(np.int64)


def _check(wl, inputs):
    U.say(f"[csr] {wl.name}")
    rp, ent = _gpu_csr(wl, inputs)
    rp0, ent0 = O.csr_transpose(O.Problem(inputs))
    # the GPU numbers every block of a TND sequence like the oracle; extra
    # bound keys (if any) are empty and sit at the end
    assert rp.size >= rp0.size
    np.testing.assert_array_equal(rp[:rp0.size], rp0)
    assert np.all(rp[rp0.size - 1:] == rp0[-1])
    np.testing.assert_array_equal(ent, ent0)


@pytest.mark.parametrize("name", ["tiny_token_gqa", "token_gqa_d64_g2", "block_gqa_d128", "mla_64h",
                                  "mla_wcmp_sinks_varlen"])
def test_csr_bit_exact_small(name):
    wl = SMALL[name]
    _check(wl, W.make_inputs(wl))


def test_csr_shuffled_duplicates_out_of_range():
    wl = SMALL["token_gqa_d64_g2"]
    inp = W.make_inputs(wl)
    idx = inp["idx"].numpy().copy()
    rng = np.random.default_rng(11)
    for t in range(idx.shape[0]):
        for g in range(idx.shape[1]):
            rng.shuffle(idx[t, g])
    idx[150, 0, :3] = 17          # triplicate
    idx[151, 1, 4] = 10 ** 6      # out of range
    idx[152] = -7                 # any negative is unused
    inp["idx"] = torch.from_numpy(idx)
    _check(wl, inp)


@pytest.mark.parametrize("name", ["nsa_block_gqa", "mla_token_8k", "mla_cmp_sinks_varlen"])
def test_csr_bit_exact_full_size(name):
    wl = W.WORKLOADS[name]
    _check(wl, W.make_index_inputs(wl))


def test_csr_three_radix_passes():
    """70 000 kv rows, so more than 2^16 keys: the sort takes three 8-bit
    passes, the middle one reading and writing (key, slot) pairs."""
    wl = W.Workload(name="csr_70k_keys", select=W.SEL_TOKEN, layout=W.LAYOUT_BSND, seqlens=(70000,), n_q_heads=2,
                    n_kv_heads=1, d_qk=64, d_v=64, kv_shared=False, topk=4, seed=17)
    _check(wl, W.make_index_inputs(wl))
