/*
 * sparse_attn.h -- C ABI of the MI355X (gfx950) sparse-attention library.
 *
 * The library computes the backward pass of attention over top-k-gathered
 * key/value rows, and the selected-attention forward that produces its
 * saved outputs.  All entry points take plain pointers and sizes; device
 * pointers are HIP device memory owned by the caller, and `stream` is a
 * hipStream_t passed as void* (NULL = the null stream).
 *
 * What is computed (per sequence b, query token t, query head h, kv head
 * g = h / G with G = n_q_heads / n_kv_heads):
 *
 *   Selection -- aclnnSparseFlashAttentionGrad, "Formula": the selected keys
 *     and values are Gather(key/value, topkIndices[i]) over the index slots,
 *     each index naming a piece of block_size rows; SparseFlashMlaGrad
 *     README, "Computation formula", Stage 1: with cmp_ratio = 4 the
 *     selected KV is the original KV (here: a sliding window over it)
 *     concatenated with Gather(cmp_kv, topkIndices[i]).
 *   Backward -- aclnnSparseFlashAttentionGrad, "Formula", Phases 1-3, and
 *     SparseFlashMlaGrad README, "Computation formula", Stages 2-3:
 *       P  = exp(scale * q K_sel^T - lse)      dP = dO V_sel^T
 *       D  = rowsum(dO * O)                    dS = P * (dP - D)
 *       dQ = scale * dS K_sel
 *       dK[u] += scale * dS^T q                dV[u] += P^T dO
 *       shared KV (MLA): dKV[u] += scale * dS^T q + P^T dO (P^T dO into the
 *       first d_v columns)
 *       dSinks[h] = sum over rows of -exp(sink_h - lse) * D
 *   Forward -- aclnnNsaSelectedAttentionInfer, "Formula": softmax over the
 *     selected keys of scale * q k^T (plus the sink logit in the
 *     denominator when sinks are given) times the selected values; lse is
 *     the natural-log log-sum-exp of those logits.
 *
 * Masking and index conventions (the pages' mask table is not available;
 * these are the readings the library implements):
 *   - index values are sequence-local; any negative value is an unused slot
 *     and may appear in any position; an index past the sequence's rows is
 *     also unused; duplicates count once per slot;
 *   - causal (mask_causal = 1): key position <= query position within the
 *     sequence (top-left aligned); mask_causal = 2 aligns the query and kv
 *     sequences at their ends (for seqlen_q != seqlen_kv); in block mode
 *     the rows of a selected block past the query are masked individually;
 *   - window (select = SA_SEL_WINDOW_CMP): ori keys [t - win_left,
 *     t + win_right] inside the sequence and the causal range, followed by
 *     the cmp rows named by topk_indices; cmp row j covers ori tokens
 *     [r*j, r*j + r - 1] (r = cmp_ratio) and is visible iff r*j + r - 1 <= t;
 *   - a row with no visible key and no sink contributes nothing (no NaN).
 *
 * Layouts (row-major, contiguous, innermost dimension last):
 *   BSND:  q [batch, seqlen_q, n_q_heads, d_qk], k [batch, seqlen_kv,
 *          n_kv_heads, d_qk], ...; this is the same memory as TND with
 *          T = batch * seqlen_q.
 *   TND:   q [total_q, n_q_heads, d_qk], kv [total_kv, n_kv_heads, d], with
 *          cu_seqlens_q / cu_seqlens_kv int32 [batch + 1], cu[0] = 0.
 *   lse, D: [T, n_q_heads] fp32.  topk_indices: [T, n_kv_heads, topk] int32.
 *   q, k, v, kv, cmp_kv, o, d_o and all gradients except dsinks: bf16, or
 *   fp16 with desc->dtype = SA_DTYPE_FP16.
 *   sinks, dsinks: [n_q_heads] fp32.
 *
 * Error behaviour: every entry point returns a status and never aborts.
 * Phase 1 (the *_workspace_size calls) validates the descriptor on the
 * host and touches no device state.  Phase 2 validates pointers and the
 * workspace size, then only enqueues work on `stream` and returns;
 * buffers must stay alive until the stream has drained.  A failed launch
 * is reported as SA_ERR_HIP.  Index *contents* are not validated.
 * An empty query (T == 0 or n_q_heads == 0) returns SA_OK and launches
 * nothing, leaving the outputs untouched (aclnnSparseFlashAttentionGrad,
 * "Constraints": an empty query returns directly).
 *
 * Ownership: the caller allocates every input, output and workspace
 * buffer.  The library's own state is one stream and two events per
 * device for the block-selection backward (sparse_attn_bwd) and the fixed
 * scratch array of the allocation-free entry point
 * (sparse_attn_bwd_noalloc); calls on different streams with disjoint
 * buffers may overlap.
 */
#ifndef SPARSE_ATTN_H_
#define SPARSE_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sa_status {
  SA_OK = 0,
  SA_ERR_NULL_PTR = 1,             /* a required pointer is NULL */
  SA_ERR_BAD_SHAPE = 2,            /* inconsistent or non-positive sizes */
  SA_ERR_UNSUPPORTED = 3,          /* valid request outside the built kernels */
  SA_ERR_WORKSPACE_TOO_SMALL = 4,  /* workspace_bytes below the phase-1 size */
  SA_ERR_MISALIGNED = 5,           /* a device pointer is not 16-byte aligned */
  SA_ERR_HIP = 6,                  /* a HIP launch or runtime call failed */
  SA_ERR_BAD_ARG = 7               /* invalid enum value, scale or flag */
} sa_status_t;

enum { SA_SEL_TOKEN = 0, SA_SEL_BLOCK = 1, SA_SEL_WINDOW_CMP = 2 };
enum { SA_LAYOUT_BSND = 0, SA_LAYOUT_TND = 1 };
/* dK/dV reduction: fp32 atomics in an unspecified order (the pages'
 * non-deterministic default, aclnnSparseFlashAttentionGrad, "Deterministic
 * computation"); a bitwise-repeatable key-major pass; or, for the shared-KV
 * 576/512 kernel only, fp32 atomics into one accumulator copy per XCD summed
 * afterwards in a fixed order of the copies. */
enum { SA_DKV_ATOMIC = 0, SA_DKV_DETERMINISTIC = 1, SA_DKV_ATOMIC_XCD = 2 };
enum { SA_DTYPE_BF16 = 0, SA_DTYPE_FP16 = 1 };

/* Static problem description (host memory, read during the call only).
 * Attribute names follow the SparseFlashMlaGrad parameter table
 * (scaleValue, cmpRatio, oriWinLeft/Right, layout, N1 = n_q_heads,
 * N2 = n_kv_heads). */
typedef struct sa_desc {
  int32_t layout;       /* SA_LAYOUT_BSND or SA_LAYOUT_TND */
  int32_t batch;        /* number of sequences B (>= 1) */
  int32_t seqlen_q;     /* BSND: query tokens per sequence */
  int32_t seqlen_kv;    /* BSND: kv rows per sequence */
  int32_t total_q;      /* TND: total query tokens (= cu_seqlens_q[B]) */
  int32_t total_kv;     /* TND: total kv rows (= cu_seqlens_kv[B]) */
  int32_t total_cmp;    /* SA_SEL_WINDOW_CMP: rows of cmp_kv (= cu_seqlens_cmp[B]) */
  int32_t n_q_heads;    /* N1 */
  int32_t n_kv_heads;   /* N2; must divide n_q_heads */
  int32_t d_qk;         /* head dim of q and k (shared KV: the full KV row) */
  int32_t d_v;          /* head dim of v (shared KV: leading columns of KV) */
  int32_t kv_shared;    /* 1: one KV tensor, K = KV, V = KV[..., :d_v] (MLA) */
  int32_t select;       /* SA_SEL_TOKEN / SA_SEL_BLOCK / SA_SEL_WINDOW_CMP */
  int32_t topk;         /* index slots per (token, kv head) */
  int32_t block_size;   /* rows per index in SA_SEL_BLOCK (1 = token) */
  int32_t mask_causal;  /* 0: none; 1: key position <= query position, both
                           counted from the sequence's start; 2: the same with
                           query and kv sequences aligned at their ends (query
                           i of n_q sits at key position i + n_kv - n_q; with
                           seqused, the used lengths) -- windows and cmp
                           visibility use that position too */
  int32_t win_left;     /* SA_SEL_WINDOW_CMP window: keys [t-win_left, t+win_right] */
  int32_t win_right;
  int32_t cmp_ratio;    /* SA_SEL_WINDOW_CMP: ori tokens per cmp row */
  int32_t has_sinks;    /* 1: per-head sink logits in the softmax denominator */
  int32_t dkv_mode;     /* SA_DKV_ATOMIC, SA_DKV_DETERMINISTIC or SA_DKV_ATOMIC_XCD */
  float scale;          /* softmax scale (finite, > 0) */
  int32_t softmax_l1;   /* 1: the backward also writes the softmax L1-norm
                           side outputs (sa_bwd_args_t); 0: it does not */
  int32_t dtype;        /* SA_DTYPE_BF16 or SA_DTYPE_FP16: the format of q, k,
                           v, kv, cmp_kv, o, d_o and of dq, dk, dv, dkv,
                           d_cmp_kv (SparseFlashMlaGrad README, parameter
                           table: BFLOAT16 or FLOAT16); products on the
                           matching MFMA with fp32 accumulation.  The 64-head
                           MLA kernel and the block key-major kernels are
                           built for bf16; fp16 runs the generic row kernel */
} sa_desc_t;

/* Device pointers for the backward.  Unused fields may be NULL.
 * Separate K/V: k, v in; dk, dv out.  Shared KV: kv in; dkv out.
 * SA_SEL_WINDOW_CMP: kv (ori) and cmp_kv in; dkv and d_cmp_kv out, and
 * topk_indices index cmp_kv rows.  With topk = 0 this is window-only
 * attention: cmp_kv, cu_seqlens_cmp and topk_indices may be NULL, and
 * d_cmp_kv too when total_cmp = 0.  Sinks: sinks in, dsinks out. */
typedef struct sa_bwd_args {
  const void* q;
  const void* k;
  const void* v;
  const void* kv;
  const void* cmp_kv;
  const void* o;
  const void* d_o;
  const float* lse;
  const float* sinks;
  const int32_t* topk_indices;
  const int32_t* cu_seqlens_q;    /* TND only */
  const int32_t* cu_seqlens_kv;   /* TND only */
  const int32_t* cu_seqlens_cmp;  /* SA_SEL_WINDOW_CMP only */
  void* dq;
  void* dk;
  void* dv;
  void* dkv;
  void* d_cmp_kv;
  float* dsinks;
  /* Softmax L1-norm side outputs (desc->softmax_l1 = 1), fp32, written in
   * full (SparseFlashMlaGrad README, parameter table: the softmax of the
   * query against the ori KV and against the cmp KV; the target
   * distribution of aclnnSparseLightningIndexerGradKLLoss, "Formula": the
   * main attention's probabilities summed over heads, then L1-normalised
   * along the context).  For every (t, g), with P the backward's P (given
   * lse, sinks in the denominator):
   *   p[pos] = sum over the G query heads of kv head g of P[h][pos]
   *   ori[t][g][pos] = p[pos] / (sum of p over the ori positions)
   *   cmp[t][g][j]   = p[win + j] / (sum of p over the cmp positions)
   * Columns are the virtual positions of the selection: ori is
   * [T, n_kv_heads, n_ori] with n_ori = topk (SA_SEL_TOKEN), topk *
   * block_size (SA_SEL_BLOCK, slot-major) or win = win_left + 1 +
   * win_right (SA_SEL_WINDOW_CMP, key t - win_left + pos); cmp is
   * [T, n_kv_heads, topk] (SA_SEL_WINDOW_CMP only, NULL otherwise).  A
   * position that selects no key (unused slot, masked, past the sequence)
   * and every position of a set whose sum is 0 holds 0.  Deterministic. */
  float* ori_softmax_l1;
  float* cmp_softmax_l1;
  /* Optional per-row top-k lengths [T, n_kv_heads] int32 (SparseFlashMlaGrad
   * README, parameter table: the selectable top-k length of each query row):
   * index slots at or past a row's length are unused; values are clamped
   * to [0, topk].  NULL: every slot may be used.  In SA_SEL_WINDOW_CMP they
   * limit the cmp slots; the window is not affected. */
  const int32_t* topk_lengths;
  /* Optional [batch] int32 counts of the query / kv / cmp rows of each
   * sequence that take part (SparseFlashMlaGrad README, parameter table:
   * seqused*); rows past them are padding: a padding query row selects
   * nothing (dq = 0) and a padding kv / cmp row is never selected (its
   * gradient is 0).  NULL: every row takes part. */
  const int32_t* seqused_q;
  const int32_t* seqused_kv;
  const int32_t* seqused_cmp;
} sa_bwd_args_t;

/* Device pointers for the forward (o, lse out; the rest as above). */
typedef struct sa_fwd_args {
  const void* q;
  const void* k;
  const void* v;
  const void* kv;
  const void* cmp_kv;
  const float* sinks;
  const int32_t* topk_indices;
  const int32_t* cu_seqlens_q;
  const int32_t* cu_seqlens_kv;
  const int32_t* cu_seqlens_cmp;
  void* o;
  float* lse;
  const int32_t* topk_lengths;   /* as in sa_bwd_args_t (NULL: all slots) */
  const int32_t* seqused_q;      /* as in sa_bwd_args_t (NULL: all rows) */
  const int32_t* seqused_kv;
  const int32_t* seqused_cmp;
} sa_fwd_args_t;

/* Phase 1 of the backward (aclnnSparseFlashAttentionGrad, "Function
 * prototype": the operator is called in two phases, the first of which
 * checks the parameters and computes the workspace size the second needs):
 * validates `desc` (host only, no HIP call) and returns in *bytes the
 * device workspace that sparse_attn_bwd needs for it (fp32 accumulators,
 * the softmax-grad term D, CSR buffers, and with softmax_l1 the
 * per-head-group sums behind the L1-norm outputs).
 * Errors: SA_ERR_NULL_PTR, SA_ERR_BAD_SHAPE (also when a key count times
 * the kv heads, or the slots of one token, would not fit int32),
 * SA_ERR_BAD_ARG, SA_ERR_UNSUPPORTED (e.g. a head dim the kernels are not
 * built for). */
sa_status_t sparse_attn_bwd_workspace_size(const sa_desc_t* desc, size_t* bytes);

/* Phase 2 of the backward (aclnnSparseFlashAttentionGrad, "Formula";
 * SparseFlashMlaGrad README, Stages 1-3): enqueues the whole backward on
 * `stream`.  `workspace` is device memory of at least the phase-1 size,
 * 256-byte aligned; its contents on entry are ignored.  Outputs are fully
 * overwritten (gradients are not accumulated into them).  dkv_mode =
 * SA_DKV_DETERMINISTIC gives bitwise-repeatable results; SA_DKV_ATOMIC
 * sums dK/dV contributions with fp32 atomics in an unspecified order.
 * Block selection in deterministic mode runs its key-major dK/dV chain on
 * a stream the library makes on first use on each device (default
 * priority, kept until the process ends), forked from and joined back
 * into `stream` with events, so the call still completes in `stream`'s
 * order; calls from several host threads are serialized while they
 * enqueue.  The environment variable SPARSE_ATTN_SIDE_STREAM=0 keeps every
 * launch on `stream`. */
sa_status_t sparse_attn_bwd(const sa_desc_t* desc, const sa_bwd_args_t* args,
                            void* workspace, size_t workspace_bytes, void* stream);

/* Same as sparse_attn_bwd, and additionally records the caller's events
 * (hipEvent_t passed as void*, either may be NULL) on `stream` immediately
 * before and after the dominant kernel, so a caller can time that kernel
 * alone with hipEventElapsedTime: the row kernel that gathers the selected
 * rows and runs the MFMA products (all launches of it when tokens are
 * processed in chunks), or, for block selection in deterministic mode, the
 * dQ pass over the selected blocks.  Same errors as sparse_attn_bwd; a failed event
 * record is SA_ERR_HIP. */
sa_status_t sparse_attn_bwd_timed(const sa_desc_t* desc, const sa_bwd_args_t* args, void* workspace,
                                  size_t workspace_bytes, void* stream, void* ev_main_start,
                                  void* ev_main_stop);

/* Selected-attention forward (aclnnNsaSelectedAttentionInfer, "Formula";
 * the forward whose o and lse the backward consumes): enqueues on
 * `stream`, writes o (in the inputs' 16-bit type, desc->dtype) and lse
 * (fp32; -inf for a row with no visible key and no sink).  No workspace. */
sa_status_t sparse_attn_fwd(const sa_desc_t* desc, const sa_fwd_args_t* args, void* stream);

/* Number of CSR keys for `desc`: token mode n_kv_rows * n_kv_heads, block
 * mode (sum over sequences of ceil(len_kv / block_size)) * n_kv_heads,
 * window+cmp total_cmp * n_kv_heads; and the workspace the CSR build needs.
 * Requires the sequence lengths (BSND: from desc; TND: host copies of
 * cu_seqlens_kv, may be NULL for BSND).  SA_ERR_BAD_SHAPE when the key
 * count or T * n_kv_heads * topk exceeds 2^31 - 1. */
sa_status_t sparse_attn_csr_size(const sa_desc_t* desc, const int32_t* host_cu_seqlens_kv,
                                 int64_t* n_keys, size_t* workspace_bytes);

/* CSR transpose of the index lists (the bookkeeping of the deterministic
 * key-major dK/dV reduction): for every key, the flat entry ids
 * p = (t * n_kv_heads + g) * topk + slot of the used slots naming it, in
 * increasing p.  row_ptr [n_keys + 1] gets the exclusive prefix sum of the
 * per-key counts (row_ptr[n_keys] = number of used slots); entries needs
 * room for T * n_kv_heads * topk ids.  Bit-exact and deterministic.
 * SA_ERR_BAD_SHAPE when T * n_kv_heads * topk exceeds 2^31 - 1 (the ids
 * are int32; the backward itself transposes token chunks that fit). */
sa_status_t sparse_attn_csr_transpose(const sa_desc_t* desc, const int32_t* topk_indices,
                                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                      int32_t* row_ptr, int32_t* entries, void* workspace,
                                      size_t workspace_bytes, void* stream);

/* ---- Sparse lightning-indexer gradient with the KL loss ------------------
 *
 * aclnnSparseLightningIndexerGradKLLoss, "Formula" (the same steps are
 * spelled out on aclnnDenseLightningIndexerGradKLLoss, "Formulas" 1-4):
 * the indexer scores the rows a query may attend to and is trained to match
 * the main attention's head-summed, L1-normalised probabilities p (the
 * softmax L1-norm output of sparse_attn_bwd).  For every query token t,
 * over the rows j its index list selects (token selection rules above, one
 * index list per token):
 *   S~ = q~_t K~_sel^T   (raw product, no scale)        [n_heads, n]
 *   I  = W_t ReLU(S~)                                    [n]
 *   loss_t = sum_j p_j log(p_j / softmax(I)_j)   (terms with p_j = 0 vanish)
 *   dI = softmax(I) - p       dW_t = ReLU(S~) dI
 *   dS~ = W_t[h] [S~ > 0] dI  dq~_t = dS~ K~_sel   dK~[j] += dS~^T q~_t
 * The softmax and the loss run over the selected rows only; p is read at
 * the used slots (its values elsewhere are ignored); a token with no used
 * slot has loss 0 and zero dq~ and dW.  dK~ is summed over tokens in a fixed
 * order (bitwise repeatable); loss = sum over tokens of loss_t (fixed order,
 * fp64 accumulation). */
typedef struct sa_indexer_desc {
  int32_t layout;       /* SA_LAYOUT_BSND or SA_LAYOUT_TND */
  int32_t batch;        /* number of sequences (>= 1) */
  int32_t seqlen_q;     /* BSND: query tokens per sequence */
  int32_t seqlen_kv;    /* BSND: key rows per sequence */
  int32_t total_q;      /* TND: total query tokens */
  int32_t total_kv;     /* TND: total key rows */
  int32_t n_heads;      /* indexer query heads per token (built: 1..64) */
  int32_t d;            /* indexer head dim (built: 128) */
  int32_t topk;         /* index slots per token (built: 1..2048) */
  int32_t mask_causal;  /* 1: key position <= query position */
} sa_indexer_desc_t;

/* Device pointers of the indexer gradient (row-major, contiguous). */
typedef struct sa_indexer_args {
  const void* q;                  /* q~ [T, n_heads, d] bf16 */
  const void* k;                  /* K~ [T_kv, d] bf16 */
  const float* weights;           /* W [T, n_heads] fp32 */
  const int32_t* topk_indices;    /* [T, topk] int32, sequence-local, negative = unused */
  const float* target;            /* p [T, topk] fp32 by slot */
  const int32_t* cu_seqlens_q;    /* TND only */
  const int32_t* cu_seqlens_kv;   /* TND only */
  void* dq;                       /* dq~ [T, n_heads, d] bf16 */
  void* dk;                       /* dK~ [T_kv, d] bf16 */
  float* dweights;                /* dW [T, n_heads] fp32 */
  float* loss;                    /* [1] fp32: the summed loss */
  float* loss_per_token;          /* [T] fp32, may be NULL */
} sa_indexer_args_t;

/* Phase 1: validates `desc` on the host and returns the workspace size
 * (per-token losses, CSR buffers, bf16 partial dK~ rows, fp32 dK~
 * accumulator).  SA_ERR_UNSUPPORTED outside the built sizes. */
sa_status_t sparse_attn_indexer_grad_kl_workspace_size(const sa_indexer_desc_t* desc, size_t* bytes);

/* Phase 2: enqueues the indexer gradient on `stream`; outputs are fully
 * overwritten.  Same error behaviour as sparse_attn_bwd; an empty query
 * returns SA_OK and launches nothing. */
sa_status_t sparse_attn_indexer_grad_kl(const sa_indexer_desc_t* desc, const sa_indexer_args_t* args,
                                        void* workspace, size_t workspace_bytes, void* stream);

/* Same, recording the caller's events (may be NULL) around the main kernel
 * (all its launches when tokens are processed in chunks). */
sa_status_t sparse_attn_indexer_grad_kl_timed(const sa_indexer_desc_t* desc, const sa_indexer_args_t* args,
                                              void* workspace, size_t workspace_bytes, void* stream,
                                              void* ev_main_start, void* ev_main_stop);

/* The backward without a workspace argument and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same
 * arguments, outputs and launch sequence as sparse_attn_bwd; the workspace
 * is a fixed 128 MiB device array of the library, one per GPU it runs on,
 * held from the library's load on that GPU until the process ends.
 * Returns SA_ERR_WORKSPACE_TOO_SMALL when sparse_attn_bwd_workspace_size
 * gives more than 128 MiB for `desc` (nothing is launched then).  Every
 * call on one GPU shares that GPU's array: calls that overlap on one GPU
 * (other streams, other host threads) race and give wrong results; calls
 * ordered on one stream are safe.  Each call clears what must start at
 * zero itself. */
sa_status_t sparse_attn_bwd_noalloc(const sa_desc_t* desc, const sa_bwd_args_t* args, void* stream);

/* Static string for a status code (every call returns one, as the pages'
 * operator API returns a status code: aclnnSparseFlashAttentionGrad,
 * "Returns").  Unknown codes give "unknown sa_status_t"; never NULL. */
const char* sparse_attn_status_string(sa_status_t status);

/* Library version as major * 10000 + minor * 100 + patch. */
int32_t sparse_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H_ */
