"""Plain fp64 CPU oracle for attention over top-k-gathered key/value rows.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this module: only the tests, the package's smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP library
(no kernels, headers, helpers or tables); the only common code is the
seeded input generator, which holds none of the method's arithmetic.

What it computes, and where the pages define it:

* Selection (aclnnSparseFlashAttentionGrad, "Formula": selectedKey /
  selectedValue = Gather(key/value, topkIndices[i]), each index naming a
  piece of block_size rows; SparseFlashMlaGrad README, "Computation
  formula", Stage 1: with cmp_ratio = 4 the selected KV is the original KV
  concatenated with Gather(cmp_kv, topkIndices[i])).
* Forward (aclnnNsaSelectedAttentionInfer, "Formula": softmax of the scaled
  query/selected-key products times the selected values; SparseFlashMlaGrad
  README, parameter table: lse is the forward's log-sum-exp output).
* Backward (aclnnSparseFlashAttentionGrad, "Formula", Phases 1-3;
  SparseFlashMlaGrad README, "Computation formula", Stages 2-3):
      P  = exp(scale * Q K_sel^T - lse)           (no renormalisation)
      dP = dO V_sel^T
      D  = rowsum(dO * O)                         (the softmax-grad term)
      dS = P * (dP - D)                           (element-wise)
      dQ = scale * dS K_sel
      dK[u] += scale * dS^T Q,   dV[u] += P^T dO  (scatter into gathered rows)
      MLA (shared KV): dKV = scale * dS^T Q + P^T dO  (P^T dO in the first d_v cols)
      dSinks[h] = sum over rows of -P_sink * D,  P_sink = exp(sink_h - lse)
* Softmax L1-norm side outputs (SparseFlashMlaGrad README, parameter
  table; aclnnSparseLightningIndexerGradKLLoss, "Formula": the target
  distribution p): P summed over the group's heads, L1-normalised over the
  ori entries and, separately, over the cmp entries.
* Sparse lightning-indexer gradient with the KL loss
  (aclnnSparseLightningIndexerGradKLLoss, "Formula"; the dense page's
  "Formulas" 1-4): index score I = W ReLU(q~ K~^T) over the selected rows,
  loss = KL(p || softmax(I)), dI = softmax(I) - p, and dW, dq~, dK~ by the
  chain rule.
* CSR transpose of the index lists (no passage on the pages: it is the
  bookkeeping for a deterministic key-major reduction): for every key, the
  flat ids p = (t * Hkv + g) * K + slot of the valid entries naming it, in
  increasing p.

Readings taken where the pages are silent or garbled (each also listed in the
design notes):
  R1  the softmax-grad term is D = rowsum(dO * O) from the O passed in;
  R2  "@" between P and (dP - D) is an element-wise product;
  R3  the scale is the descriptor's scale value (1/sqrt(d_qk) by default);
  R4  lse is the natural-log LSE over the selected, masked logits (plus the
      sink logit when sinks are present); SimpleSoftmax(x, lse) = exp(x - lse);
  R5  sinks are one fp32 logit per query head, in the denominator only;
  R6  masks: causal means key position <= query position (per sequence;
      with the ends-aligned mode, query i of n_q sits at key position
      i + n_kv - n_q, and padding rows past seqused take no part);
      window keys are [t - win_left, t + win_right] within [0, t]; cmp row j
      (covering ori tokens [r*j, r*j + r - 1]) is visible iff r*j + r - 1 <= t;
      a masked key is simply absent;
  R7  index i names rows [i * block_size, (i + 1) * block_size);
  R8  any negative index is an unused slot; an index >= the sequence's row
      count is also unused; with per-row top-k lengths, slots at or past the
      row's length are unused (lengths clamped to [0, K]);
  R9  duplicate indices form a multiset: each slot is its own softmax term
      and its own scatter;
  R10 a row with no valid key and no sink has lse = -inf, O = 0 and no
      gradient contribution;
  R11 cu_seqlens are cumulative ([B+1], cu[0] = 0);
  R12 index values and window positions are sequence-local;
  R15 GQA: query head h uses kv head h // G; indices are per (token, kv head);
  R18 the softmax L1-norm outputs sum the backward's P (given lse, sinks in
      the denominator) over the G heads of a kv head and normalise the ori
      and the cmp entries separately; they are laid out by virtual position
      (slot, block row, window offset) with 0 where nothing is selected;
  R19 the indexer's S~ is the raw product q~ K~^T (no scale); its softmax and
      loss run over the selected rows; the target p is given per slot and
      only used slots count; dI = softmax(I) - p as printed;
  R23 the cmp residual (the remainder of the ori length by cmp_ratio) follows
      from R6's blocks and the lengths, so no residual input exists.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

SEL_TOKEN = 0
SEL_BLOCK = 1
SEL_WINDOW_CMP = 2


def _f64(t: torch.Tensor) -> np.ndarray:
    """fp64 copy of a CPU tensor (exact for bf16, fp16 and fp32 values).

    The 16-bit formats are widened in numpy from their bit patterns (a bf16
    value is the top half of the fp32 with the same bits), which keeps
    torch's intra-op thread pool out of the per-token loops: next to the
    BLAS threads it made these small copies ~100x slower."""
    if t.dtype in (torch.bfloat16, torch.float16):
        return _widen16(t.view(torch.int16).numpy(), t.dtype)
    return t.numpy().astype(np.float64)


def _widen16(bits: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """fp64 values of 16-bit bf16 / fp16 bit patterns (an int16 array)."""
    u = bits.view(np.uint16)
    if dtype == torch.float16:
        return u.view(np.float16).astype(np.float64)
    return (u.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _take_f64(t: torch.Tensor, rows: np.ndarray, g) -> np.ndarray:
    """fp64 copy of t[rows, g] (rows: a numpy index array; g: an index or a
    slice)."""
    if t.dtype in (torch.bfloat16, torch.float16):
        return _widen16(t.view(torch.int16).numpy()[rows, g], t.dtype)
    return t.numpy()[rows, g].astype(np.float64)


class Problem:
    """Inputs of one problem, viewed by the oracle.

    Built from the generator's dict (torch CPU tensors) and the workload's
    static description; bf16 tensors stay bf16 and are widened to fp64 row
    by row (every bf16 value is exact in fp64).
    """

    def __init__(self, inputs: Dict[str, object]):
        wl = inputs["workload"]
        self.wl = wl
        self.select = wl.select
        self.G = wl.n_q_heads // wl.n_kv_heads
        self.Hq, self.Hkv = wl.n_q_heads, wl.n_kv_heads
        self.d_qk, self.d_v = wl.d_qk, wl.d_v
        self.kv_shared = wl.kv_shared
        self.scale = wl.softmax_scale
        self.block_size = wl.block_size
        self.win_left, self.win_right = wl.win_left, wl.win_right
        self.cmp_ratio = wl.cmp_ratio
        # 1: key position <= query position, positions counted from each
        # sequence's start; 2: the query and kv sequences aligned at their
        # ends (query i of n_q sits at key position i + n_kv - n_q)
        self.mask = int(getattr(wl, "mask_causal", 1))
        self.causal = self.mask != 0
        self.q = inputs.get("q")
        self.d_o = inputs.get("d_o")
        if wl.kv_shared:
            self.k = inputs.get("kv")
            self.v = None
        else:
            self.k = inputs.get("k")
            self.v = inputs.get("v")
        self.cmp_kv = inputs.get("cmp_kv")
        self.sinks = inputs.get("sinks")
        self.idx = inputs["idx"].numpy()
        # optional selectable slots per (token, kv head): slots at or past
        # the length are unused (SparseFlashMlaGrad README, parameter table:
        # the per-row top-k lengths)
        tl = inputs.get("topk_len")
        self.topk_len = None if tl is None else np.clip(np.asarray(tl, np.int64), 0, self.idx.shape[2])
        self.cu = inputs["cu_seqlens"].numpy().astype(np.int64)
        self.cu_kv = np.asarray(inputs.get("cu_seqlens_kv", inputs["cu_seqlens"]), np.int64)
        self.cu_cmp = inputs["cu_seqlens_cmp"].numpy().astype(np.int64)
        # optional per-sequence counts of the query / kv / cmp rows that take
        # part (SparseFlashMlaGrad README, parameter table: seqused*): rows
        # past them are padding
        self.used = {k: (None if inputs.get(k) is None else np.asarray(inputs[k], np.int64))
                     for k in ("seqused_q", "seqused_kv", "seqused_cmp")}
        self.T = int(self.cu[-1])
        self.K = self.idx.shape[2]
        # sequence id of every token
        self.seq_of = np.repeat(np.arange(len(self.cu) - 1), np.diff(self.cu))

    # -- selection --------------------------------------------------------
    def selection(self, t: int, g: int) -> Tuple[np.ndarray, np.ndarray]:
        """Ordered multiset of (source, global row) selected by token t for kv
        head g.  source 0 = the primary K/V (ori) rows, 1 = cmp_kv rows.
        Slot order is kept; unused and masked slots are dropped."""
        srcs, rows, _ = self.selection_positions(t, g)
        return srcs, rows

    def selection_positions(self, t: int, g: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        """selection(t, g) plus the virtual position of every entry: the
        index slot (token), slot * block_size + row in block (block), or the
        window offset followed by window length + slot (window+cmp).  These
        are the columns of the softmax L1-norm outputs."""
        b, tl, n_kv, base, n_cmp_used = self.query_pos(t)
        K = self.idx.shape[2]
        if tl is None:                            # a padding query row
            e = np.zeros(0, dtype=np.int64)
            return e, e, e
        n_sel = K if self.topk_len is None else int(self.topk_len[t, g])
        usable = np.arange(K) < n_sel             # slots inside the row's length
        if self.select == SEL_TOKEN:
            j = self.idx[t, g].astype(np.int64)
            keep = (j >= 0) & (j < n_kv)
            if self.causal:
                keep &= j <= tl
            keep &= usable
            rows = base + j[keep]
            return np.zeros(rows.size, dtype=np.int64), rows, np.flatnonzero(keep)
        if self.select == SEL_BLOCK:
            bs = self.block_size
            blk = self.idx[t, g].astype(np.int64)
            slots = np.flatnonzero((blk >= 0) & usable)
            blk = blk[slots]
            j = (blk[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)   # block-major
            keep = j < n_kv
            if self.causal:
                keep &= j <= tl
            rows = base + j[keep]
            pos = (slots[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)[keep]
            return np.zeros(rows.size, dtype=np.int64), rows, pos
        # window over the ori rows, then the gathered cmp rows
        w = np.arange(tl - self.win_left, tl + self.win_right + 1, dtype=np.int64)
        keep = (w >= 0) & (w < n_kv)
        if self.causal:
            keep &= w <= tl
        ori = base + w[keep]
        r = self.cmp_ratio
        n_cmp = n_cmp_used
        j = self.idx[t, g].astype(np.int64)
        keepc = (j >= 0) & (j < n_cmp)
        if self.causal:
            keepc &= r * j + r - 1 <= tl
        keepc &= usable
        cmp = int(self.cu_cmp[b]) + j[keepc]
        srcs = np.concatenate([np.zeros(ori.size, np.int64), np.ones(cmp.size, np.int64)])
        pos = np.concatenate([np.flatnonzero(keep), w.size + np.flatnonzero(keepc)])
        return srcs, np.concatenate([ori, cmp]), pos

    def query_pos(self, t: int):
        """(sequence b, key position of query t or None for a padding row,
        kv rows taking part, first kv row, cmp rows taking part)."""
        b = int(self.seq_of[t])
        i = t - int(self.cu[b])                   # index within the query sequence
        n_q = int(self.cu[b + 1] - self.cu[b])
        n_kv = int(self.cu_kv[b + 1] - self.cu_kv[b])
        n_cmp = int(self.cu_cmp[b + 1] - self.cu_cmp[b])
        if self.used["seqused_q"] is not None:
            n_q = min(n_q, int(self.used["seqused_q"][b]))
        if self.used["seqused_kv"] is not None:
            n_kv = min(n_kv, int(self.used["seqused_kv"][b]))
        if self.used["seqused_cmp"] is not None:
            n_cmp = min(n_cmp, int(self.used["seqused_cmp"][b]))
        if i >= n_q:
            return b, None, n_kv, int(self.cu_kv[b]), n_cmp
        pos = i + (n_kv - n_q if self.mask == 2 else 0)
        return b, pos, n_kv, int(self.cu_kv[b]), n_cmp

    def gather(self, srcs: np.ndarray, rows: np.ndarray, g: int) -> Tuple[np.ndarray, np.ndarray]:
        """fp64 K_sel [n, d_qk] and V_sel [n, d_v] for a selection."""
        n = rows.size
        K = np.zeros((n, self.d_qk))
        m0 = srcs == 0
        if m0.any():
            K[m0] = _take_f64(self.k, rows[m0], g)
        if (~m0).any():
            K[~m0] = _take_f64(self.cmp_kv, rows[~m0], g)
        if self.kv_shared:
            V = K[:, :self.d_v]
        else:
            V = np.zeros((n, self.d_v))
            if n:
                V[:] = _take_f64(self.v, rows, g)
        return K, V


def sparse_fwd(pb: Problem, tokens: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Selected-attention forward in fp64 for the given tokens (all by default).

    Returns O [n, Hq, d_v] and lse [n, Hq] (natural log; -inf when a row has
    neither a valid key nor a sink).
    """
    toks = range(pb.T) if tokens is None else tokens
    toks = list(toks)
    O = np.zeros((len(toks), pb.Hq, pb.d_v))
    L = np.full((len(toks), pb.Hq), -np.inf)
    sinks = None if pb.sinks is None else pb.sinks.to(torch.float64).numpy()
    for n, t in enumerate(toks):
        q_t = _f64(pb.q[t])
        for g in range(pb.Hkv):
            srcs, rows = pb.selection(t, g)
            K, V = pb.gather(srcs, rows, g)
            hs = slice(g * pb.G, (g + 1) * pb.G)
            S = pb.scale * (q_t[hs] @ K.T)                       # [G, n]
            if sinks is not None:
                sk = sinks[hs]
                m = np.maximum(S.max(axis=1) if rows.size else -np.inf, sk)
                z = np.exp(S - m[:, None]).sum(axis=1) + np.exp(sk - m)
            else:
                if rows.size == 0:
                    continue
                m = S.max(axis=1)
                z = np.exp(S - m[:, None]).sum(axis=1)
            lse = m + np.log(z)
            P = np.exp(S - lse[:, None])
            O[n, hs] = P @ V
            L[n, hs] = lse
    return O, L


def round_fwd_outputs(O: np.ndarray, lse: np.ndarray,
                      dtype: torch.dtype = torch.bfloat16) -> Tuple[torch.Tensor, torch.Tensor]:
    """O -> bf16 (or `dtype`, round to nearest even), lse -> fp32: the stored
    forward outputs that the backward receives as inputs."""
    # fp64 -> fp32 -> bf16: the bf16 value is the fp32 value's nearest-even
    # rounding (the stored O is an input to both backwards, so only the fact
    # that both receive the same array matters).
    return (torch.from_numpy(O).to(torch.float32).to(dtype),
            torch.from_numpy(lse).to(torch.float32))


def sparse_bwd(pb: Problem, O: torch.Tensor, lse: torch.Tensor,
               tokens: Optional[Sequence[int]] = None,
               want_rows: bool = True) -> Dict[str, np.ndarray]:
    """Sparse attention backward in fp64.

    O ([T, Hq, d_v], any float dtype) and lse ([T, Hq]) are the stored forward
    outputs, indexed by global token.  With `tokens`, only those query tokens
    contribute (dq rows of other tokens stay 0 and dK/dV/dKV hold the partial
    sums from those tokens only).

    Returns fp64 arrays: dq [T, Hq, d_qk]; dk [T_kv, Hkv, d_qk] and
    dv [T_kv, Hkv, d_v] (separate K/V) or dkv [T_kv, 1, d_qk] (shared);
    dcmp_kv [T_cmp, Hkv, d_qk] for window+cmp; dsinks [Hq] with sinks.
    """
    toks = range(pb.T) if tokens is None else tokens
    n_kv = pb.k.shape[0]
    dq = np.zeros((pb.T, pb.Hq, pb.d_qk))
    dk = np.zeros((n_kv, pb.Hkv, pb.d_qk))
    dv = None if pb.kv_shared else np.zeros((n_kv, pb.Hkv, pb.d_v))
    dcmp = None if pb.cmp_kv is None else np.zeros((pb.cmp_kv.shape[0], pb.Hkv, pb.d_qk))
    sinks = None if pb.sinks is None else pb.sinks.to(torch.float64).numpy()
    dsinks = None if sinks is None else np.zeros(pb.Hq)
    for t in toks:
        q_t = _f64(pb.q[t])
        do_t = _f64(pb.d_o[t])
        o_t = _f64(O[t]) if isinstance(O, torch.Tensor) else np.asarray(O[t], np.float64)
        l_t = _f64(lse[t]) if isinstance(lse, torch.Tensor) else np.asarray(lse[t], np.float64)
        for g in range(pb.Hkv):
            hs = slice(g * pb.G, (g + 1) * pb.G)
            Qg, dOg, Og, Lg = q_t[hs], do_t[hs], o_t[hs], l_t[hs]
            finite = np.isfinite(Lg)
            Lsafe = np.where(finite, Lg, 0.0)
            D = (dOg * Og).sum(axis=1)                           # softmax-grad term
            if dsinks is not None:
                p_sink = np.where(finite, np.exp(sinks[hs] - Lsafe), 0.0)
                dsinks[hs] += -p_sink * D
            srcs, rows = pb.selection(t, g)
            if rows.size == 0:
                continue
            K, V = pb.gather(srcs, rows, g)
            S = pb.scale * (Qg @ K.T)
            P = np.where(finite[:, None], np.exp(S - Lsafe[:, None]), 0.0)
            dP = dOg @ V.T
            dS = P * (dP - D[:, None])
            dq[t, hs] = pb.scale * (dS @ K)
            dK_sel = pb.scale * (dS.T @ Qg)                      # [n, d_qk]
            dV_sel = P.T @ dOg                                   # [n, d_v]
            if pb.kv_shared:
                dK_sel[:, :pb.d_v] += dV_sel
            m0 = srcs == 0
            np.add.at(dk[:, g], rows[m0], dK_sel[m0])
            if dv is not None:
                np.add.at(dv[:, g], rows[m0], dV_sel[m0])
            if dcmp is not None and (~m0).any():
                np.add.at(dcmp[:, g], rows[~m0], dK_sel[~m0])
    out: Dict[str, np.ndarray] = {"dq": dq}
    if pb.kv_shared:
        out["dkv"] = dk
    else:
        out["dk"] = dk
        out["dv"] = dv
    if dcmp is not None:
        out["dcmp_kv"] = dcmp
    if dsinks is not None:
        out["dsinks"] = dsinks
    return out


def softmax_l1_norm(pb: Problem, lse: torch.Tensor,
                    tokens: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Softmax L1-norm side outputs in fp64.

    SparseFlashMlaGrad README, parameter table: two fp32 outputs holding the
    softmax of the query against the ori KV and against the cmp KV;
    aclnnSparseLightningIndexerGradKLLoss, "Formula": the indexer's target
    distribution is the main attention's probabilities summed over the heads
    and then L1-normalised along the context.  For every (t, g):

        P_h   = exp(scale * q_h K_sel^T - lse_h)   for the G heads of group g
        p     = sum over h of P_h                  (one value per selected entry)
        ori_j = p_j / sum of p over the ori entries   (source 0)
        cmp_j = p_j / sum of p over the cmp entries   (source 1, window+cmp)

    Readings: P is the backward's P (the given lse, sinks included, so a
    head's mass may be below one); each set is normalised on its own; the
    outputs are laid out by virtual position (selection_positions) --
    ori [T, Hkv, n_ori] with n_ori = topk (token), topk * block_size (block)
    or the window length (window+cmp), and cmp [T, Hkv, topk] -- and a
    position that selects nothing, or a set whose mass is zero, holds 0.
    A duplicated slot has its own position and its own value.
    """
    toks = range(pb.T) if tokens is None else tokens
    nwin = pb.win_left + 1 + pb.win_right
    if pb.select == SEL_TOKEN:
        n_ori = pb.K
    elif pb.select == SEL_BLOCK:
        n_ori = pb.K * pb.block_size
    else:
        n_ori = nwin
    ori = np.zeros((pb.T, pb.Hkv, n_ori))
    cmp = np.zeros((pb.T, pb.Hkv, pb.K)) if pb.select == SEL_WINDOW_CMP else None
    for t in toks:
        q_t = _f64(pb.q[t])
        l_t = _f64(lse[t]) if isinstance(lse, torch.Tensor) else np.asarray(lse[t], np.float64)
        for g in range(pb.Hkv):
            hs = slice(g * pb.G, (g + 1) * pb.G)
            srcs, rows, pos = pb.selection_positions(t, g)
            if rows.size == 0:
                continue
            Lg = l_t[hs]
            finite = np.isfinite(Lg)
            K, _ = pb.gather(srcs, rows, g)
            S = pb.scale * (q_t[hs] @ K.T)
            P = np.where(finite[:, None], np.exp(S - np.where(finite, Lg, 0.0)[:, None]), 0.0)
            p = P.sum(axis=0)                                     # heads summed
            for src, out, off in ((0, ori, 0), (1, cmp, nwin)):
                m = srcs == src
                if out is None or not m.any():
                    continue
                tot = p[m].sum()
                if tot > 0:
                    out[t, g, pos[m] - off] = p[m] / tot
    res = {"ori": ori}
    if cmp is not None:
        res["cmp"] = cmp
    return res


# ----------------------------------------------------------------------------
# Sparse lightning-indexer gradient with the KL loss
# ----------------------------------------------------------------------------

def indexer_grad_kl(inputs: Dict[str, object], tokens: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Gradient of the indexer's KL loss over the top-k selected rows, fp64.

    aclnnSparseLightningIndexerGradKLLoss, "Formula", and the same steps on
    aclnnDenseLightningIndexerGradKLLoss, "Formulas" 1-4, restricted to the
    selected keys.  For every token t, over the rows j it selected (token
    selection rules of `Problem.selection`, kv head 0):

        S~ = q~_t K~_sel^T                    [heads, n]   (raw product)
        I  = W_t ReLU(S~)                     [n]          (index score)
        s  = softmax(I)                       over the selected rows
        loss_t = sum_j p_j log(p_j / s_j)     (terms with p_j = 0 vanish)
        dI = s - p
        dW_t   = ReLU(S~) dI
        dS~    = W_t[h] * [S~ > 0] * dI       (chain rule through the ReLU)
        dq~_t  = dS~ K~_sel,   dK~[j] += dS~^T q~_t   (scatter into rows j)

    p (`target` [T, 1, K]) is the target distribution by slot, taken as
    given; only the used slots count.  Readings: S~ is the raw product (the
    dense page's statement; the sparse page's "softmax of QK" is taken as a
    garble), there is no scale, the softmax runs over the selected rows only,
    duplicated slots are separate terms, a token with no used slot has loss 0
    and no gradient.

    Returns dq [T, H, d], dk [T_kv, d], dweights [T, H], loss_per_token [T]
    and loss (the sum over tokens).
    """
    wl = inputs["workload"]
    view = {"workload": wl, "idx": inputs["idx"], "cu_seqlens": inputs["cu_seqlens"],
            "cu_seqlens_kv": inputs.get("cu_seqlens_kv", inputs["cu_seqlens"]),
            "cu_seqlens_cmp": inputs["cu_seqlens_cmp"], "kv": inputs["k_idx"][:, None, :]}
    pb = Problem(view)
    q = inputs["q_idx"]
    k = inputs["k_idx"]
    W = _f64(inputs["weights"])
    P = _f64(inputs["target"])[:, 0, :]
    T, H, d = q.shape
    dq = np.zeros((T, H, d))
    dk = np.zeros((k.shape[0], d))
    dW = np.zeros((T, H))
    loss_t = np.zeros(T)
    toks = range(T) if tokens is None else tokens
    for t in toks:
        _, rows, pos = pb.selection_positions(t, 0)
        if rows.size == 0:
            continue
        qt = _f64(q[t])                                   # [H, d]
        K = _take_f64(k, rows, slice(None))               # [n, d]
        S = qt @ K.T                                      # [H, n]
        R = np.maximum(S, 0.0)
        I = W[t] @ R                                      # [n]
        m = I.max()
        logs = I - m - np.log(np.exp(I - m).sum())        # log softmax over the selected rows
        s_ = np.exp(logs)
        p = P[t, pos]
        nz = p > 0
        loss_t[t] = float((p[nz] * (np.log(p[nz]) - logs[nz])).sum())
        dI = s_ - p
        dW[t] = R @ dI
        dS = (W[t][:, None] * (S > 0)) * dI[None, :]
        dq[t] = dS @ K
        np.add.at(dk, rows, dS.T @ qt)
    return {"dq": dq, "dk": dk, "dweights": dW, "loss_per_token": loss_t, "loss": float(loss_t.sum())}


# ----------------------------------------------------------------------------
# CSR transpose of the index lists
# ----------------------------------------------------------------------------

def _block_base(pb: Problem) -> np.ndarray:
    """First global block id of every sequence (ceil(len / bs) blocks each)."""
    bs = pb.block_size
    nb = (np.diff(pb.cu_kv) + bs - 1) // bs
    return np.concatenate([[0], np.cumsum(nb)])


def entry_keys(pb: Problem) -> np.ndarray:
    """Key id named by every slot, flattened as p = (t * Hkv + g) * K + slot,
    or -1 when the slot is unused.

    token mode: key = global kv row * Hkv + g; block mode: key = global block
    id * Hkv + g with blocks numbered per sequence at ceil(len / bs) each;
    window+cmp: key = global cmp row * Hkv + g (the window part has no slot).
    A slot is used when its index is >= 0, inside its sequence and not fully
    masked (token: j <= t; block: first row j * bs <= t; cmp: r*j + r - 1 <= t,
    t the query's key position), inside the row's top-k length, and the
    query row is not padding.
    """
    T, Hkv, K = pb.idx.shape
    j = pb.idx.astype(np.int64)
    out = np.full((T, Hkv, K), -1, dtype=np.int64)
    bb = _block_base(pb)
    r = pb.cmp_ratio
    for t in range(T):
        b, tl, n_kv, kv_base, n_cmp = pb.query_pos(t)
        if tl is None:
            continue
        for g in range(Hkv):
            jj = j[t, g]
            if pb.select == SEL_TOKEN:
                ok = (jj >= 0) & (jj < n_kv) & ((jj <= tl) if pb.causal else True)
                key = (kv_base + jj) * Hkv + g
            elif pb.select == SEL_BLOCK:
                bs = pb.block_size
                ok = (jj >= 0) & (jj * bs < n_kv) & ((jj * bs <= tl) if pb.causal else True)
                key = (bb[b] + jj) * Hkv + g
            else:
                ok = (jj >= 0) & (jj < n_cmp) & ((r * jj + r - 1 <= tl) if pb.causal else True)
                key = (int(pb.cu_cmp[b]) + jj) * Hkv + g
            if pb.topk_len is not None:
                ok &= np.arange(K) < pb.topk_len[t, g]
            out[t, g] = np.where(ok, key, -1)
    return out.reshape(-1)


def n_keys(pb: Problem) -> int:
    if pb.select == SEL_TOKEN:
        return int(pb.cu_kv[-1]) * pb.Hkv
    if pb.select == SEL_BLOCK:
        return int(_block_base(pb)[-1]) * pb.Hkv
    return int(pb.cu_cmp[-1]) * pb.Hkv


def csr_transpose(pb: Problem) -> Tuple[np.ndarray, np.ndarray]:
    """Counting sort of the valid entries by key: returns row_ptr [n_keys+1]
    (exclusive prefix of the per-key counts) and entries [n_valid] holding
    the flat entry ids p, ascending within a key (a stable sort by key)."""
    keys = entry_keys(pb)
    valid = np.flatnonzero(keys >= 0)                     # ascending p
    counts = np.bincount(keys[valid], minlength=n_keys(pb))
    row_ptr = np.zeros(counts.size + 1, dtype=np.int64)
    row_ptr[1:] = np.cumsum(counts)
    order = np.argsort(keys[valid], kind="stable")        # ties keep p order
    return row_ptr, valid[order]
