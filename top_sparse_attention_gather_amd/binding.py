"""Thin Python binding of the C ABI in include/sparse_attn.h.

Argument marshalling only: every step of the computation runs in the HIP
library.  torch provides device memory and the current stream.  If the
shared library is not built the functions raise; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

import torch

from . import workloads as W

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "libsparse_attn.so")

SA_OK = 0
STATUS_NAMES = {0: "SA_OK", 1: "SA_ERR_NULL_PTR", 2: "SA_ERR_BAD_SHAPE", 3: "SA_ERR_UNSUPPORTED",
                4: "SA_ERR_WORKSPACE_TOO_SMALL", 5: "SA_ERR_MISALIGNED", 6: "SA_ERR_HIP",
                7: "SA_ERR_BAD_ARG"}
DKV_ATOMIC = 0
DKV_DETERMINISTIC = 1
DKV_ATOMIC_XCD = 2     # shared-KV MLA kernel only: fp32 atomics into one accumulator copy per XCD
DTYPE_BF16 = 0
DTYPE_FP16 = 1

EXPORTED = ["sparse_attn_bwd_workspace_size", "sparse_attn_bwd", "sparse_attn_bwd_timed", "sparse_attn_fwd",
            "sparse_attn_csr_size",
            "sparse_attn_csr_transpose", "sparse_attn_indexer_grad_kl_workspace_size", "sparse_attn_indexer_grad_kl",
            "sparse_attn_indexer_grad_kl_timed", "sparse_attn_status_string", "sparse_attn_version",
            "sparse_attn_bwd_noalloc"]


class SaDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "layout", "batch", "seqlen_q", "seqlen_kv", "total_q", "total_kv", "total_cmp", "n_q_heads",
        "n_kv_heads", "d_qk", "d_v", "kv_shared", "select", "topk", "block_size", "mask_causal",
        "win_left", "win_right", "cmp_ratio", "has_sinks", "dkv_mode")] + [("scale", ctypes.c_float),
                                                                           ("softmax_l1", ctypes.c_int32),
                                                                           ("dtype", ctypes.c_int32)]


_P = ctypes.c_void_p


class SaBwdArgs(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "q", "k", "v", "kv", "cmp_kv", "o", "d_o", "lse", "sinks", "topk_indices", "cu_seqlens_q",
        "cu_seqlens_kv", "cu_seqlens_cmp", "dq", "dk", "dv", "dkv", "d_cmp_kv", "dsinks", "ori_softmax_l1",
        "cmp_softmax_l1", "topk_lengths", "seqused_q", "seqused_kv", "seqused_cmp")]


class SaFwdArgs(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "q", "k", "v", "kv", "cmp_kv", "sinks", "topk_indices", "cu_seqlens_q", "cu_seqlens_kv",
        "cu_seqlens_cmp", "o", "lse", "topk_lengths", "seqused_q", "seqused_kv", "seqused_cmp")]


class SaIndexerDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "layout", "batch", "seqlen_q", "seqlen_kv", "total_q", "total_kv", "n_heads", "d", "topk", "mask_causal")]


class SaIndexerArgs(ctypes.Structure):
    _fields_ = [(n, _P) for n in (
        "q", "k", "weights", "topk_indices", "target", "cu_seqlens_q", "cu_seqlens_kv", "dq", "dk", "dweights",
        "loss", "loss_per_token")]


class SparseAttnError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} returned {STATUS_NAMES.get(status, status)}")
        self.status = status


_lib = None


def library_path() -> str:
    return _LIB_PATH


def load() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"{_LIB_PATH} is not built; run `python -m top_sparse_attention_gather_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    pd = ctypes.POINTER(SaDesc)
    lib.sparse_attn_bwd_workspace_size.argtypes = [pd, ctypes.POINTER(ctypes.c_size_t)]
    lib.sparse_attn_bwd.argtypes = [pd, ctypes.POINTER(SaBwdArgs), _P, ctypes.c_size_t, _P]
    lib.sparse_attn_bwd_timed.argtypes = [pd, ctypes.POINTER(SaBwdArgs), _P, ctypes.c_size_t, _P, _P, _P]
    lib.sparse_attn_fwd.argtypes = [pd, ctypes.POINTER(SaFwdArgs), _P]
    lib.sparse_attn_bwd_noalloc.argtypes = [pd, ctypes.POINTER(SaBwdArgs), _P]
    lib.sparse_attn_csr_size.argtypes = [pd, _P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_size_t)]
    lib.sparse_attn_csr_transpose.argtypes = [pd, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    pi = ctypes.POINTER(SaIndexerDesc)
    lib.sparse_attn_indexer_grad_kl_workspace_size.argtypes = [pi, ctypes.POINTER(ctypes.c_size_t)]
    lib.sparse_attn_indexer_grad_kl.argtypes = [pi, ctypes.POINTER(SaIndexerArgs), _P, ctypes.c_size_t, _P]
    lib.sparse_attn_indexer_grad_kl_timed.argtypes = [pi, ctypes.POINTER(SaIndexerArgs), _P, ctypes.c_size_t, _P,
                                                      _P, _P]
    lib.sparse_attn_status_string.argtypes = [ctypes.c_int]
    lib.sparse_attn_status_string.restype = ctypes.c_char_p
    lib.sparse_attn_version.restype = ctypes.c_int32
    for fn in ("sparse_attn_bwd_workspace_size", "sparse_attn_bwd", "sparse_attn_bwd_timed", "sparse_attn_bwd_noalloc",
               "sparse_attn_fwd",
               "sparse_attn_csr_size", "sparse_attn_csr_transpose", "sparse_attn_indexer_grad_kl_workspace_size",
               "sparse_attn_indexer_grad_kl", "sparse_attn_indexer_grad_kl_timed"):
        getattr(lib, fn).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(fn: str, st: int) -> None:
    if st != SA_OK:
        raise SparseAttnError(fn, st)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    assert t.is_contiguous(), "tensors must be contiguous"
    return t.data_ptr()


def make_desc(wl: W.Workload, dkv_mode: int = DKV_ATOMIC, **over) -> SaDesc:
    """Descriptor of a workload (BSND when all sequences have one length)."""
    d = SaDesc()
    if wl.layout == W.LAYOUT_BSND:
        d.layout, d.batch = W.LAYOUT_BSND, wl.batch
        d.seqlen_q, d.seqlen_kv = wl.seqlens[0], wl.kv_lens[0]
    else:
        d.layout, d.batch = W.LAYOUT_TND, wl.batch
        d.total_q, d.total_kv = wl.total_q, wl.total_kv
    d.total_cmp = wl.total_cmp
    d.n_q_heads, d.n_kv_heads, d.d_qk, d.d_v = wl.n_q_heads, wl.n_kv_heads, wl.d_qk, wl.d_v
    d.kv_shared = int(wl.kv_shared)
    d.select, d.topk = wl.select, wl.topk
    d.block_size = wl.block_size if wl.select == W.SEL_BLOCK else 1
    d.mask_causal = wl.mask_causal
    d.win_left, d.win_right, d.cmp_ratio = wl.win_left, wl.win_right, wl.cmp_ratio
    d.has_sinks = int(wl.has_sinks)
    d.dkv_mode = dkv_mode
    d.scale = wl.softmax_scale
    d.dtype = DTYPE_FP16 if wl.dtype == "fp16" else DTYPE_BF16
    for k, v in over.items():
        setattr(d, k, v)
    return d


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def sparse_attn_bwd_workspace_size(desc: SaDesc) -> int:
    n = ctypes.c_size_t(0)
    _check("sparse_attn_bwd_workspace_size", load().sparse_attn_bwd_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def alloc_bwd_outputs(desc: SaDesc, tensors: Dict[str, torch.Tensor]) -> Dict[str, torch.Tensor]:
    """Output tensors of the right shapes on the inputs' device."""
    q = tensors["q"]
    dev = q.device
    out = {"dq": torch.empty_like(q)}
    if desc.kv_shared:
        out["dkv"] = torch.empty_like(tensors["kv"])
    else:
        out["dk"] = torch.empty_like(tensors["k"])
        out["dv"] = torch.empty_like(tensors["v"])
    if desc.select == W.SEL_WINDOW_CMP and desc.total_cmp > 0:
        out["d_cmp_kv"] = torch.empty_like(tensors["cmp_kv"])
    if desc.has_sinks:
        out["dsinks"] = torch.empty(desc.n_q_heads, dtype=torch.float32, device=dev)
    if desc.softmax_l1:
        T = q.numel() // (desc.n_q_heads * desc.d_qk)
        if desc.select == W.SEL_TOKEN:
            n_ori = desc.topk
        elif desc.select == W.SEL_BLOCK:
            n_ori = desc.topk * desc.block_size
        else:
            n_ori = desc.win_left + 1 + desc.win_right
        out["ori_softmax_l1"] = torch.empty((T, desc.n_kv_heads, n_ori), dtype=torch.float32, device=dev)
        if desc.select == W.SEL_WINDOW_CMP and desc.topk > 0:
            out["cmp_softmax_l1"] = torch.empty((T, desc.n_kv_heads, desc.topk), dtype=torch.float32, device=dev)
    return out


def sparse_attn_bwd(desc: SaDesc, tensors: Dict[str, torch.Tensor], outputs: Optional[Dict[str, torch.Tensor]] = None,
                    workspace: Optional[torch.Tensor] = None, stream=None, events=None) -> Dict[str, torch.Tensor]:
    """Enqueue the backward on `stream` (default: torch's current stream).

    `tensors` holds device tensors named as in sa_bwd_args_t (q, k, v, kv,
    cmp_kv, o, d_o, lse, sinks, topk_indices, cu_seqlens_q, cu_seqlens_kv,
    cu_seqlens_cmp).  Outputs and workspace are allocated when not given.
    """
    lib = load()
    if outputs is None:
        outputs = alloc_bwd_outputs(desc, tensors)
    need = sparse_attn_bwd_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=tensors["q"].device)
    a = SaBwdArgs()
    for name in ("q", "k", "v", "kv", "cmp_kv", "o", "d_o", "lse", "sinks", "topk_indices", "cu_seqlens_q",
                 "cu_seqlens_kv", "cu_seqlens_cmp", "topk_lengths", "seqused_q", "seqused_kv", "seqused_cmp"):
        setattr(a, name, _ptr(tensors.get(name)))
    for name in ("dq", "dk", "dv", "dkv", "d_cmp_kv", "dsinks", "ori_softmax_l1", "cmp_softmax_l1"):
        setattr(a, name, _ptr(outputs.get(name)))
    if events is None:
        _check("sparse_attn_bwd", lib.sparse_attn_bwd(ctypes.byref(desc), ctypes.byref(a), _ptr(workspace),
                                                      workspace.numel(), _stream(stream)))
    else:
        _check("sparse_attn_bwd_timed",
               lib.sparse_attn_bwd_timed(ctypes.byref(desc), ctypes.byref(a), _ptr(workspace), workspace.numel(),
                                         _stream(stream), events[0], events[1]))
    return outputs


def sparse_attn_bwd_noalloc(desc: SaDesc, tensors: Dict[str, torch.Tensor],
                            outputs: Optional[Dict[str, torch.Tensor]] = None, stream=None) -> Dict[str, torch.Tensor]:
    """The backward on the library's fixed per-GPU workspace (no workspace
    argument, no allocation inside the call).  Outputs are allocated here
    when not given; pass them in to allocate nothing at all."""
    lib = load()
    if outputs is None:
        outputs = alloc_bwd_outputs(desc, tensors)
    a = SaBwdArgs()
    for name in ("q", "k", "v", "kv", "cmp_kv", "o", "d_o", "lse", "sinks", "topk_indices", "cu_seqlens_q",
                 "cu_seqlens_kv", "cu_seqlens_cmp", "topk_lengths", "seqused_q", "seqused_kv", "seqused_cmp"):
        setattr(a, name, _ptr(tensors.get(name)))
    for name in ("dq", "dk", "dv", "dkv", "d_cmp_kv", "dsinks", "ori_softmax_l1", "cmp_softmax_l1"):
        setattr(a, name, _ptr(outputs.get(name)))
    _check("sparse_attn_bwd_noalloc", lib.sparse_attn_bwd_noalloc(ctypes.byref(desc), ctypes.byref(a), _stream(stream)))
    return outputs


class HipEvents:
    """Raw hipEvent_t pairs from the HIP runtime (for timing one kernel on
    the stream it is launched on)."""

    def __init__(self, n: int):
        self.rt = ctypes.CDLL("libamdhip64.so")
        self.rt.hipEventCreate.argtypes = [ctypes.POINTER(_P)]
        self.rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), _P, _P]
        self.rt.hipEventSynchronize.argtypes = [_P]
        self.rt.hipEventDestroy.argtypes = [_P]
        self.pairs = []
        for _ in range(n):
            a, b = _P(), _P()
            assert self.rt.hipEventCreate(ctypes.byref(a)) == 0 and self.rt.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a.value, b.value))

    def elapsed_ms(self, i: int) -> float:
        a, b = self.pairs[i]
        assert self.rt.hipEventSynchronize(b) == 0
        ms = ctypes.c_float(0.0)
        assert self.rt.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)

    def close(self):
        for a, b in self.pairs:
            self.rt.hipEventDestroy(a)
            self.rt.hipEventDestroy(b)
        self.pairs = []


def sparse_attn_fwd(desc: SaDesc, tensors: Dict[str, torch.Tensor], o: Optional[torch.Tensor] = None,
                    lse: Optional[torch.Tensor] = None, stream=None):
    """Enqueue the selected-attention forward; returns (o bf16, lse fp32)."""
    lib = load()
    q = tensors["q"]
    T = q.numel() // (desc.n_q_heads * desc.d_qk)
    if o is None:
        o = torch.empty((T, desc.n_q_heads, desc.d_v), dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((T, desc.n_q_heads), dtype=torch.float32, device=q.device)
    a = SaFwdArgs()
    for name in ("q", "k", "v", "kv", "cmp_kv", "sinks", "topk_indices", "cu_seqlens_q", "cu_seqlens_kv",
                 "cu_seqlens_cmp", "topk_lengths", "seqused_q", "seqused_kv", "seqused_cmp"):
        setattr(a, name, _ptr(tensors.get(name)))
    a.o, a.lse = _ptr(o), _ptr(lse)
    _check("sparse_attn_fwd", lib.sparse_attn_fwd(ctypes.byref(desc), ctypes.byref(a), _stream(stream)))
    return o, lse


def sparse_attn_status_string(status: int) -> str:
    return load().sparse_attn_status_string(status).decode()


def sparse_attn_version() -> int:
    return int(load().sparse_attn_version())


def device_tensors(inputs: Dict[str, object], device="cuda") -> Dict[str, torch.Tensor]:
    """Move a generator dict to the device under the C ABI's argument names."""
    wl = inputs["workload"]
    out = {}
    for k in ("q", "k", "v", "kv", "cmp_kv", "d_o", "sinks", "o", "lse"):
        if k in inputs:
            out[k] = inputs[k].to(device).contiguous()
    out["topk_indices"] = inputs["idx"].to(device).contiguous()
    if inputs.get("topk_len") is not None:
        out["topk_lengths"] = torch.as_tensor(inputs["topk_len"], dtype=torch.int32).to(device).contiguous()
    if wl.layout == W.LAYOUT_TND:
        out["cu_seqlens_q"] = inputs["cu_seqlens"].to(device)
        out["cu_seqlens_kv"] = inputs.get("cu_seqlens_kv", inputs["cu_seqlens"]).to(device)
    if wl.select == W.SEL_WINDOW_CMP:
        out["cu_seqlens_cmp"] = inputs["cu_seqlens_cmp"].to(device)
    for k in ("seqused_q", "seqused_kv", "seqused_cmp"):
        if inputs.get(k) is not None:
            out[k] = torch.as_tensor(inputs[k], dtype=torch.int32).to(device).contiguous()
    return out


def sparse_attn_csr_size(desc: SaDesc, host_cu_seqlens_kv=None):
    """(n_keys, workspace bytes) of the CSR transpose."""
    nk = ctypes.c_int64(0)
    nb = ctypes.c_size_t(0)
    cu = None
    if host_cu_seqlens_kv is not None:
        arr = (ctypes.c_int32 * len(host_cu_seqlens_kv))(*[int(x) for x in host_cu_seqlens_kv])
        cu = ctypes.cast(arr, _P)
    _check("sparse_attn_csr_size", load().sparse_attn_csr_size(ctypes.byref(desc), cu, ctypes.byref(nk),
                                                               ctypes.byref(nb)))
    return nk.value, nb.value


def sparse_attn_csr_transpose(desc: SaDesc, topk_indices: torch.Tensor, cu_seqlens_q=None, cu_seqlens_kv=None,
                              host_cu_seqlens_kv=None, stream=None):
    """CSR transpose of the index lists on the GPU: (row_ptr [n_keys+1],
    entries [n_valid]) as int32 device tensors."""
    lib = load()
    n_keys, nbytes = sparse_attn_csr_size(desc, host_cu_seqlens_kv)
    dev = topk_indices.device
    row_ptr = torch.empty(n_keys + 1, dtype=torch.int32, device=dev)
    entries = torch.empty(max(1, topk_indices.numel()), dtype=torch.int32, device=dev)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=dev)
    _check("sparse_attn_csr_transpose",
           lib.sparse_attn_csr_transpose(ctypes.byref(desc), _ptr(topk_indices), _ptr(cu_seqlens_q),
                                         _ptr(cu_seqlens_kv), _ptr(row_ptr), _ptr(entries), _ptr(ws), ws.numel(),
                                         _stream(stream)))
    n_valid = int(row_ptr[-1].item())
    return row_ptr, entries[:n_valid]


# ---- sparse lightning-indexer gradient with the KL loss --------------------

def make_indexer_desc(wl: W.Workload, **over) -> SaIndexerDesc:
    """Descriptor of an indexer workload (n_q_heads indexer heads, d_qk head dim)."""
    d = SaIndexerDesc()
    if wl.layout == W.LAYOUT_BSND:
        d.layout, d.batch = W.LAYOUT_BSND, wl.batch
        d.seqlen_q = d.seqlen_kv = wl.seqlens[0]
    else:
        d.layout, d.batch = W.LAYOUT_TND, wl.batch
        d.total_q = d.total_kv = wl.total_q
    d.n_heads, d.d, d.topk, d.mask_causal = wl.n_q_heads, wl.d_qk, wl.topk, 1
    for k, v in over.items():
        setattr(d, k, v)
    return d


def indexer_device_tensors(inputs: Dict[str, object], device="cuda") -> Dict[str, torch.Tensor]:
    """Move an indexer generator dict to the device under the C ABI's names."""
    wl = inputs["workload"]
    out = {"q": inputs["q_idx"].to(device).contiguous(), "k": inputs["k_idx"].to(device).contiguous(),
           "weights": inputs["weights"].to(device).contiguous(),
           "topk_indices": inputs["idx"].to(device).contiguous(),
           "target": inputs["target"].to(device).contiguous()}
    if wl.layout == W.LAYOUT_TND:
        out["cu_seqlens_q"] = inputs["cu_seqlens"].to(device)
        out["cu_seqlens_kv"] = inputs.get("cu_seqlens_kv", inputs["cu_seqlens"]).to(device)
    return out


def sparse_attn_indexer_grad_kl_workspace_size(desc: SaIndexerDesc) -> int:
    n = ctypes.c_size_t(0)
    _check("sparse_attn_indexer_grad_kl_workspace_size",
           load().sparse_attn_indexer_grad_kl_workspace_size(ctypes.byref(desc), ctypes.byref(n)))
    return n.value


def sparse_attn_indexer_grad_kl(desc: SaIndexerDesc, tensors: Dict[str, torch.Tensor],
                                outputs: Optional[Dict[str, torch.Tensor]] = None,
                                workspace: Optional[torch.Tensor] = None, stream=None,
                                events=None) -> Dict[str, torch.Tensor]:
    """Enqueue the indexer gradient; returns dq, dk (bf16), dweights,
    loss_per_token and loss (fp32)."""
    lib = load()
    q, k = tensors["q"], tensors["k"]
    dev = q.device
    if outputs is None:
        T = q.shape[0]
        outputs = {"dq": torch.empty_like(q), "dk": torch.empty_like(k),
                   "dweights": torch.empty((T, desc.n_heads), dtype=torch.float32, device=dev),
                   "loss": torch.empty(1, dtype=torch.float32, device=dev),
                   "loss_per_token": torch.empty(T, dtype=torch.float32, device=dev)}
    need = sparse_attn_indexer_grad_kl_workspace_size(desc)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    a = SaIndexerArgs()
    for name in ("q", "k", "weights", "topk_indices", "target", "cu_seqlens_q", "cu_seqlens_kv"):
        setattr(a, name, _ptr(tensors.get(name)))
    for name in ("dq", "dk", "dweights", "loss", "loss_per_token"):
        setattr(a, name, _ptr(outputs.get(name)))
    if events is None:
        _check("sparse_attn_indexer_grad_kl",
               lib.sparse_attn_indexer_grad_kl(ctypes.byref(desc), ctypes.byref(a), _ptr(workspace),
                                               workspace.numel(), _stream(stream)))
    else:
        _check("sparse_attn_indexer_grad_kl_timed",
               lib.sparse_attn_indexer_grad_kl_timed(ctypes.byref(desc), ctypes.byref(a), _ptr(workspace),
                                                     workspace.numel(), _stream(stream), events[0], events[1]))
    return outputs
