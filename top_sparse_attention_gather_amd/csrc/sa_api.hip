// C ABI of the sparse-attention library: descriptor validation (phase 1),
// workspace layout, and the launch sequence of each call on the caller's
// stream (phase 2).  The two-phase shape (size query, then execute) and the
// status-code returns follow the operator API pattern of the pages
// (aclnnSparseFlashAttentionGrad, "Function prototype" / first-phase
// parameter verification); the empty-query early return follows the same
// page's "Constraints".
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/sparse_attn.h"
#include "sa_launch.h"

namespace {

using sa::BwdBuffers;
using sa::Params;

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

long long total_q(const sa_desc_t* d) {
  return d->layout == SA_LAYOUT_BSND ? (long long)d->batch * d->seqlen_q : (long long)d->total_q;
}

long long rows_kv(const sa_desc_t* d) {
  return d->layout == SA_LAYOUT_BSND ? (long long)d->batch * d->seqlen_kv : (long long)d->total_kv;
}

long long rows_cmp(const sa_desc_t* d) { return d->select == SA_SEL_WINDOW_CMP ? (long long)d->total_cmp : 0; }

long long csr_keys_bound(const sa_desc_t* d);

// Largest int32 count: slot ids, CSR keys and their sentinel are int32 on
// the device.
constexpr long long kMaxI32 = (1LL << 31) - 1;

// Phase-1 checks shared by every entry point.
sa_status_t validate(const sa_desc_t* d) {
  if (!d) return SA_ERR_NULL_PTR;
  if (d->layout != SA_LAYOUT_BSND && d->layout != SA_LAYOUT_TND) return SA_ERR_BAD_ARG;
  if (d->select < SA_SEL_TOKEN || d->select > SA_SEL_WINDOW_CMP) return SA_ERR_BAD_ARG;
  if (d->dkv_mode != SA_DKV_ATOMIC && d->dkv_mode != SA_DKV_DETERMINISTIC && d->dkv_mode != SA_DKV_ATOMIC_XCD)
    return SA_ERR_BAD_ARG;
  if (d->kv_shared != 0 && d->kv_shared != 1) return SA_ERR_BAD_ARG;
  if (d->mask_causal < 0 || d->mask_causal > 2) return SA_ERR_BAD_ARG;
  if (d->has_sinks != 0 && d->has_sinks != 1) return SA_ERR_BAD_ARG;
  if (!std::isfinite(d->scale)) return SA_ERR_BAD_ARG;
  if (d->softmax_l1 != 0 && d->softmax_l1 != 1) return SA_ERR_BAD_ARG;
  if (d->dtype != SA_DTYPE_BF16 && d->dtype != SA_DTYPE_FP16) return SA_ERR_BAD_ARG;
  if (d->batch < 1 || d->n_q_heads < 0 || d->n_kv_heads < 1) return SA_ERR_BAD_SHAPE;
  if (d->n_q_heads % d->n_kv_heads != 0) return SA_ERR_BAD_SHAPE;
  if (d->d_qk <= 0 || d->d_v <= 0) return SA_ERR_BAD_SHAPE;
  if (d->kv_shared && d->d_v > d->d_qk) return SA_ERR_BAD_SHAPE;
  if (d->layout == SA_LAYOUT_BSND) {
    if (d->seqlen_q < 0 || d->seqlen_kv < 0) return SA_ERR_BAD_SHAPE;
  } else {
    if (d->total_q < 0 || d->total_kv < 0) return SA_ERR_BAD_SHAPE;
  }
  if (d->select == SA_SEL_BLOCK) {
    if (d->block_size < 1 || d->topk < 1) return SA_ERR_BAD_SHAPE;
  } else if (d->select == SA_SEL_TOKEN) {
    if (d->topk < 1) return SA_ERR_BAD_SHAPE;
  } else {
    if (!d->kv_shared) return SA_ERR_UNSUPPORTED;   // cmp_kv is one shared K(V) tensor
    if (d->topk < 0 || d->cmp_ratio < 1 || d->win_left < 0 || d->win_right < 0 || d->total_cmp < 0)
      return SA_ERR_BAD_SHAPE;
  }
  const long long T = total_q(d);
  if (T > 0 && d->n_q_heads > 0 && rows_kv(d) < 1) return SA_ERR_BAD_SHAPE;
  // row ids must stay below the cmp flag bit and T * n_kv_heads must fit a grid
  if (rows_kv(d) >= (1LL << 30) || rows_cmp(d) >= (1LL << 30) || T * d->n_kv_heads >= (1LL << 31))
    return SA_ERR_BAD_SHAPE;
  const long long npos = d->select == SA_SEL_BLOCK ? (long long)d->topk * d->block_size
                         : d->select == SA_SEL_TOKEN ? d->topk
                                                     : (long long)d->win_left + 1 + d->win_right + d->topk;
  if (npos >= (1LL << 30)) return SA_ERR_BAD_SHAPE;
  // CSR keys (kv row, block or cmp row, times the kv heads) and the
  // sentinel key past them must fit int32; the slots of one token fit one
  // token chunk (chunks keep fewer than 2^31 slots)
  if (csr_keys_bound(d) >= kMaxI32) return SA_ERR_BAD_SHAPE;
  if ((long long)d->n_kv_heads * d->topk > kMaxI32) return SA_ERR_BAD_SHAPE;
  return SA_OK;
}

// Tokens per chunk whose slot ids (chunk-local, int32) all fit.
long long max_chunk_tokens(long long Hkv, long long topk) { return topk > 0 ? kMaxI32 / (Hkv * topk) : kMaxI32; }

// Partial-row buffer cap of the deterministic path; larger problems are
// processed in token chunks whose partials fit under it.
constexpr size_t kPartialCap = size_t(24) << 30;

long long n_positions_host(const sa_desc_t* d) {
  if (d->select == SA_SEL_TOKEN) return d->topk;
  if (d->select == SA_SEL_BLOCK) return (long long)d->topk * d->block_size;
  return (long long)d->win_left + 1 + d->win_right + d->topk;
}

// Keys of the internal CSR (an upper bound of the block count for TND).
long long csr_keys_bound(const sa_desc_t* d) {
  if (d->select == SA_SEL_TOKEN) return rows_kv(d) * d->n_kv_heads;
  if (d->select == SA_SEL_BLOCK) {
    if (d->layout == SA_LAYOUT_BSND)
      return (long long)d->batch * ((d->seqlen_kv + d->block_size - 1) / d->block_size) * d->n_kv_heads;
    return (rows_kv(d) / d->block_size + d->batch) * d->n_kv_heads;
  }
  return rows_cmp(d) * d->n_kv_heads;
}

Params make_params(const sa_desc_t* d);

struct BwdLayout {
  size_t D, sink_term, acc_k, acc_v, acc_cmp;                   // atomic modes
  size_t rep_floats;                                            // MLA atomic: floats per accumulator replica
  int n_rep, mla;
  size_t l1;                                                    // softmax L1-norm head-chunk sums
  int n_hg_l1;
  size_t blk_base, row_ptr, entries, csr_ws, partial, dump, acc;   // deterministic mode
  size_t bpart, bchunk, bcnt, bscan;                            // block key-major chunks
  long long max_chunks;
  int Tc, n_hc, RW, fast, blk_km, n_hc_blk;
  size_t total;
};

BwdLayout bwd_layout(const sa_desc_t* d, const Params& p) {
  const size_t T = (size_t)total_q(d), Hq = (size_t)d->n_q_heads, Hkv = (size_t)d->n_kv_heads;
  BwdLayout L;
  std::memset(&L, 0, sizeof(L));
  size_t off = 0;
  L.D = off;
  off += align_up(T * Hq * sizeof(float));
  L.sink_term = off;
  if (d->has_sinks) off += align_up(T * Hq * sizeof(float));
  // head chunks of the kernel that computes P (it writes one plane of
  // softmax L1-norm sums per chunk)
  const bool det = d->dkv_mode == SA_DKV_DETERMINISTIC;
  L.mla = sa::mla_bwd_supported(p) ? 1 : 0;
  if (L.mla) L.n_hg_l1 = sa::mla_bwd_head_groups(p);
  else if (det && sa::blk_dkv_supported(p) && sa::blk_dq_supported(p)) L.n_hg_l1 = sa::blk_dkv_head_chunks(p);
  else L.n_hg_l1 = sa::bwd_rows_head_chunks(p);
  L.l1 = off;
  if (d->softmax_l1) off += align_up((size_t)L.n_hg_l1 * T * Hkv * (size_t)n_positions_host(d) * sizeof(float));
  if (d->dkv_mode != SA_DKV_DETERMINISTIC && L.mla) {
    // the MLA kernel's atomic forms: dKV rows then cmp rows in one fp32
    // array, one copy per XCD for the per-XCD form, and an fp32 dump row
    L.n_rep = d->dkv_mode == SA_DKV_ATOMIC_XCD ? sa::kXcdReplicas : 1;
    L.rep_floats = (size_t)(rows_kv(d) + rows_cmp(d)) * Hkv * d->d_qk;
    L.acc_k = off;
    L.acc_cmp = off + (size_t)rows_kv(d) * Hkv * d->d_qk * sizeof(float);
    off += align_up((size_t)L.n_rep * L.rep_floats * sizeof(float));
    L.dump = off;
    off += align_up((size_t)d->d_qk * sizeof(float));
    L.Tc = (int)T;
    L.total = off;
    return L;
  }
  if (d->dkv_mode != SA_DKV_DETERMINISTIC) {
    L.acc_k = off;
    off += align_up((size_t)rows_kv(d) * Hkv * d->d_qk * sizeof(float));
    L.acc_v = off;
    if (!d->kv_shared) off += align_up((size_t)rows_kv(d) * Hkv * d->d_v * sizeof(float));
    L.acc_cmp = off;
    if (d->select == SA_SEL_WINDOW_CMP) off += align_up((size_t)rows_cmp(d) * Hkv * d->d_qk * sizeof(float));
    L.Tc = (int)T;
    L.total = off;
    return L;
  }
  L.RW = d->kv_shared ? d->d_qk : d->d_qk + d->d_v;
  L.fast = sa::mla_bwd_supported(p) ? 1 : 0;
  L.n_hc = L.fast ? sa::mla_bwd_head_groups(p) : sa::bwd_rows_head_chunks(p);
  const size_t npos = (size_t)n_positions_host(d);
  const size_t elem = L.fast ? 2 : 4;   // bf16 partials from the MLA kernel, fp32 otherwise
  // block selection with separate K/V: dK/dV from the key-major block
  // kernel, no partial rows, one pass over all tokens
  // (one pass over every token: its slot ids must fit int32)
  L.blk_km = (!L.fast && sa::blk_dkv_supported(p) && (long long)T * (long long)Hkv * d->topk <= kMaxI32) ? 1 : 0;
  const size_t per_token = L.blk_km ? 0 : (size_t)L.n_hc * Hkv * npos * L.RW * elem;
  size_t Tc = per_token ? std::max<size_t>(1, kPartialCap / per_token) : T;
  Tc = std::min<size_t>(Tc, (size_t)max_chunk_tokens((long long)Hkv, d->topk));
  L.Tc = (int)std::min<size_t>(std::max<size_t>(T, 1), Tc);
  const long long nk = csr_keys_bound(d);
  if (L.blk_km) {
    L.n_hc_blk = sa::blk_dkv_head_chunks(p);
    L.max_chunks = sa::blk_max_chunks(nk, (long long)T * Hkv * d->topk);
  }
  L.blk_base = off;
  off += align_up((size_t)(d->batch + 1) * 4);
  L.row_ptr = off;
  off += align_up((size_t)(nk + 1) * 4);
  L.entries = off;
  off += align_up((size_t)L.Tc * Hkv * d->topk * 4);
  L.csr_ws = off;
  off += align_up(sa::csr_workspace_bytes((long long)L.Tc * Hkv * d->topk, nk, d->batch));
  L.partial = off;
  off += align_up((size_t)L.Tc * per_token);
  L.dump = off;
  off += align_up((size_t)L.RW * sizeof(float));
  L.acc = off;
  if (!L.blk_km) off += align_up((size_t)(rows_kv(d) + rows_cmp(d)) * Hkv * L.RW * sizeof(float));
  L.bpart = off;
  if (L.blk_km) {
    off += align_up((size_t)L.n_hc_blk * L.max_chunks * 64 * (size_t)(2 * d->d_qk) * sizeof(float));
    L.bchunk = off;
    off += align_up((size_t)(nk + 1) * 4);
    L.bcnt = off;
    off += align_up((size_t)(nk + 1) * 4);
    L.bscan = off;
    off += align_up((size_t)sa::scan_bsum_ints(nk + 1) * 4);
  }
  L.total = off;
  return L;
}

Params make_params(const sa_desc_t* d) {
  Params p;
  std::memset(&p, 0, sizeof(p));
  p.T = (int)total_q(d);
  p.Hq = d->n_q_heads;
  p.Hkv = d->n_kv_heads;
  p.G = d->n_q_heads / d->n_kv_heads;
  p.dqk = d->d_qk;
  p.dv = d->d_v;
  p.topk = d->topk;
  p.bs = d->select == SA_SEL_BLOCK ? d->block_size : 1;
  p.select = d->select;
  p.causal = d->mask_causal;
  p.win_left = d->win_left;
  p.win_right = d->win_right;
  p.cmp_ratio = d->cmp_ratio;
  p.has_sinks = d->has_sinks;
  p.shared = d->kv_shared;
  p.layout = d->layout;
  p.B = d->batch;
  p.Sq = d->seqlen_q;
  p.Skv = d->seqlen_kv;
  p.fp16 = d->dtype == SA_DTYPE_FP16 ? 1 : 0;
  p.scale = d->scale;
  return p;
}

bool aligned16(const void* ptr) { return ((uintptr_t)ptr & 15u) == 0; }

#define SA_TRY_HIP(expr)                     \
  do {                                       \
    if ((expr) != hipSuccess) return SA_ERR_HIP; \
  } while (0)

// Pointer checks shared by forward and backward.
sa_status_t check_inputs(const sa_desc_t* d, const void* q, const void* k, const void* v, const void* kv,
                         const void* cmp_kv, const float* sinks, const int32_t* idx, const int32_t* cu_q,
                         const int32_t* cu_kv, const int32_t* cu_cmp) {
  if (!q) return SA_ERR_NULL_PTR;
  if (d->kv_shared ? !kv : (!k || !v)) return SA_ERR_NULL_PTR;
  if (d->topk > 0 && !idx) return SA_ERR_NULL_PTR;
  if (d->layout == SA_LAYOUT_TND && (!cu_q || !cu_kv)) return SA_ERR_NULL_PTR;
  // window+cmp: the cmp table is only read through index slots
  if (d->select == SA_SEL_WINDOW_CMP && d->topk > 0 && (!cmp_kv || !cu_cmp)) return SA_ERR_NULL_PTR;
  if (d->has_sinks && !sinks) return SA_ERR_NULL_PTR;
  if (!aligned16(q) || !aligned16(d->kv_shared ? kv : k) || (!d->kv_shared && !aligned16(v)) ||
      (cmp_kv && !aligned16(cmp_kv)))
    return SA_ERR_MISALIGNED;
  return SA_OK;
}

// ---- sparse lightning-indexer gradient ---------------------------------------

long long idx_total_q(const sa_indexer_desc_t* d) {
  return d->layout == SA_LAYOUT_BSND ? (long long)d->batch * d->seqlen_q : (long long)d->total_q;
}

long long idx_rows_kv(const sa_indexer_desc_t* d) {
  return d->layout == SA_LAYOUT_BSND ? (long long)d->batch * d->seqlen_kv : (long long)d->total_kv;
}

Params make_idx_params(const sa_indexer_desc_t* d) {
  Params p;
  std::memset(&p, 0, sizeof(p));
  p.T = (int)idx_total_q(d);
  p.Hq = d->n_heads;
  p.Hkv = 1;
  p.G = d->n_heads;
  p.dqk = d->d;
  p.dv = d->d;
  p.topk = d->topk;
  p.bs = 1;
  p.select = SA_SEL_TOKEN;
  p.causal = d->mask_causal;
  p.cmp_ratio = 1;
  p.layout = d->layout;
  p.B = d->batch;
  p.Sq = d->seqlen_q;
  p.Skv = d->seqlen_kv;
  p.scale = 1.f;
  return p;
}

sa_status_t validate_idx(const sa_indexer_desc_t* d) {
  if (!d) return SA_ERR_NULL_PTR;
  if (d->layout != SA_LAYOUT_BSND && d->layout != SA_LAYOUT_TND) return SA_ERR_BAD_ARG;
  if (d->mask_causal != 0 && d->mask_causal != 1) return SA_ERR_BAD_ARG;
  if (d->batch < 1 || d->n_heads < 1 || d->d < 1 || d->topk < 1) return SA_ERR_BAD_SHAPE;
  if (d->layout == SA_LAYOUT_BSND) {
    if (d->seqlen_q < 0 || d->seqlen_kv < 0) return SA_ERR_BAD_SHAPE;
  } else {
    if (d->total_q < 0 || d->total_kv < 0) return SA_ERR_BAD_SHAPE;
  }
  const long long T = idx_total_q(d);
  if (T > 0 && idx_rows_kv(d) < 1) return SA_ERR_BAD_SHAPE;
  if (idx_rows_kv(d) >= (1LL << 30) || T >= (1LL << 31)) return SA_ERR_BAD_SHAPE;
  if (d->topk > (1 << 30)) return SA_ERR_BAD_SHAPE;
  if (!sa::idx_grad_supported(make_idx_params(d))) return SA_ERR_UNSUPPORTED;
  return SA_OK;
}

struct IdxLayout {
  size_t loss_tok, blk_base, row_ptr, entries, csr_ws, partial, dump, acc, total;
  int Tc;
};

IdxLayout idx_layout(const sa_indexer_desc_t* d) {
  IdxLayout L;
  std::memset(&L, 0, sizeof(L));
  const size_t T = (size_t)idx_total_q(d), K = (size_t)d->topk, D = (size_t)d->d;
  const long long nk = idx_rows_kv(d);
  const size_t per_token = K * D * sizeof(uint16_t);   // bf16 partial rows
  L.Tc = (int)std::min<size_t>(std::max<size_t>(T, 1), std::max<size_t>(1, kPartialCap / per_token));
  L.Tc = (int)std::min<long long>(L.Tc, max_chunk_tokens(1, (long long)K));
  size_t off = 0;
  L.loss_tok = off;
  off += align_up(T * sizeof(float));
  L.blk_base = off;
  off += align_up((size_t)(d->batch + 1) * 4);
  L.row_ptr = off;
  off += align_up((size_t)(nk + 1) * 4);
  L.entries = off;
  off += align_up((size_t)L.Tc * K * 4);
  L.csr_ws = off;
  off += align_up(sa::csr_workspace_bytes((long long)L.Tc * (long long)K, nk, d->batch));
  L.partial = off;
  off += align_up((size_t)L.Tc * per_token);
  L.dump = off;
  off += align_up(D * sizeof(uint16_t));
  L.acc = off;
  off += align_up((size_t)nk * D * sizeof(float));
  L.total = off;
  return L;
}

// ---- the two block-selection passes side by side ----------------------------
//
// With block selection in deterministic mode the dQ pass (query-major) and
// the CSR build, chunk count and key-major dK/dV pass do not depend on each
// other; both passes are latency-bound and one workgroup of each fits a CU
// together (registers and LDS).  The second chain runs on a library-owned
// stream (default priority, no CU mask) forked from and joined back into the
// caller's stream.  SPARSE_ATTN_SIDE_STREAM=0 keeps everything on the
// caller's stream.
constexpr int kMaxDev = 64;

struct SideCtx {
  int state = 0;                   // 0: not tried, 1: ready, -1: unavailable
  hipStream_t s = nullptr;
  hipEvent_t ev_fork = nullptr, ev_join = nullptr;
};

std::mutex g_side_mu;
SideCtx g_side[kMaxDev];

int stream_device(hipStream_t stream) {
  int dev = -1;
  if (!stream) return hipGetDevice(&dev) == hipSuccess ? dev : -1;
  hipDevice_t d;
  return hipStreamGetDevice(stream, &d) == hipSuccess ? (int)d : -1;
}

// The side stream of device `dev`, made on first use with that device
// current (null if it cannot be made).  Called with g_side_mu held.
SideCtx* side_ctx(int dev) {
  if (dev < 0 || dev >= kMaxDev) return nullptr;
  SideCtx& c = g_side[dev];
  if (c.state) return c.state > 0 ? &c : nullptr;
  c.state = -1;
  int cur = -1;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
  const bool ok = hipStreamCreateWithFlags(&c.s, hipStreamNonBlocking) == hipSuccess &&
                  hipEventCreateWithFlags(&c.ev_fork, hipEventDisableTiming) == hipSuccess &&
                  hipEventCreateWithFlags(&c.ev_join, hipEventDisableTiming) == hipSuccess;
  if (cur != dev) (void)hipSetDevice(cur);
  if (!ok) return nullptr;
  c.state = 1;
  return &c;
}

}  // namespace

extern "C" {

sa_status_t sparse_attn_indexer_grad_kl_workspace_size(const sa_indexer_desc_t* desc, size_t* bytes) {
  if (!bytes) return SA_ERR_NULL_PTR;
  const sa_status_t st = validate_idx(desc);
  if (st != SA_OK) return st;
  *bytes = idx_layout(desc).total;
  return SA_OK;
}

sa_status_t sparse_attn_indexer_grad_kl_timed(const sa_indexer_desc_t* desc, const sa_indexer_args_t* a,
                                              void* workspace, size_t workspace_bytes, void* stream,
                                              void* ev_main_start, void* ev_main_stop) {
  size_t need = 0;
  sa_status_t st = sparse_attn_indexer_grad_kl_workspace_size(desc, &need);
  if (st != SA_OK) return st;
  if (!a) return SA_ERR_NULL_PTR;
  if (idx_total_q(desc) == 0) return SA_OK;   // empty query: nothing to do
  if (!a->q || !a->k || !a->weights || !a->topk_indices || !a->target || !a->dq || !a->dk || !a->dweights ||
      !a->loss)
    return SA_ERR_NULL_PTR;
  if (desc->layout == SA_LAYOUT_TND && (!a->cu_seqlens_q || !a->cu_seqlens_kv)) return SA_ERR_NULL_PTR;
  if (!workspace) return SA_ERR_NULL_PTR;
  if (workspace_bytes < need) return SA_ERR_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return SA_ERR_MISALIGNED;
  if (!aligned16(a->q) || !aligned16(a->k)) return SA_ERR_MISALIGNED;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const IdxLayout L = idx_layout(desc);
  Params p = make_idx_params(desc);
  p.k = static_cast<const bf16*>(a->k);
  p.q = static_cast<const bf16*>(a->q);
  p.idx = a->topk_indices;
  p.cu_q = a->cu_seqlens_q;
  p.cu_kv = a->cu_seqlens_kv;

  sa::IdxArgs ia;
  std::memset(&ia, 0, sizeof(ia));
  ia.q = p.q;
  ia.k = p.k;
  ia.w = a->weights;
  ia.target = a->target;
  ia.dq = static_cast<bf16*>(a->dq);
  ia.dw = a->dweights;
  ia.loss_tok = a->loss_per_token ? a->loss_per_token : reinterpret_cast<float*>(ws + L.loss_tok);
  ia.part = reinterpret_cast<bf16*>(ws + L.partial);
  ia.dump = reinterpret_cast<bf16*>(ws + L.dump);
  ia.H = desc->n_heads;

  int* blk_base = reinterpret_cast<int*>(ws + L.blk_base);
  int* row_ptr = reinterpret_cast<int*>(ws + L.row_ptr);
  int* entries = reinterpret_cast<int*>(ws + L.entries);
  float* acc = reinterpret_cast<float*>(ws + L.acc);
  const long long nk = idx_rows_kv(desc);
  sa::ReduceArgs r;
  std::memset(&r, 0, sizeof(r));
  r.partial = ia.part;
  r.partial_bf16 = 1;
  r.RW = desc->d;
  r.npos = desc->topk;
  r.n_hc = 1;
  r.row_ptr = row_ptr;
  r.entries = entries;
  r.blk_base = blk_base;
  r.n_kv_out = nk;
  r.n_out_rows = nk;
  r.acc = acc;
  bool first = true;
  for (int t0 = 0; t0 < p.T; t0 += L.Tc) {
    const int t1 = std::min(p.T, t0 + L.Tc);
    SA_TRY_HIP(sa::launch_csr_transpose(p, t0, t1, nk, blk_base, row_ptr, entries, ws + L.csr_ws, s));
    ia.t0 = t0;
    ia.Tc = t1 - t0;
    if (ev_main_start && first) SA_TRY_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(ev_main_start), s));
    SA_TRY_HIP(sa::launch_idx_grad(p, ia, s));
    if (ev_main_stop && t1 == p.T) SA_TRY_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(ev_main_stop), s));
    r.t0 = t0;
    r.Tc = t1 - t0;
    r.accumulate = first ? 0 : 1;
    SA_TRY_HIP(sa::launch_reduce(p, r, s));
    first = false;
  }
  SA_TRY_HIP(sa::launch_cast(acc, a->dk, (size_t)nk * desc->d, 0, s));
  // loss = fixed-order sum of the per-token losses (the dSinks reduction
  // over one "head")
  Params pl = p;
  pl.Hq = 1;
  BwdBuffers wl;
  std::memset(&wl, 0, sizeof(wl));
  wl.sink_term = ia.loss_tok;
  wl.dsinks = a->loss;
  SA_TRY_HIP(sa::launch_dsinks(pl, wl, s));
  return SA_OK;
}

sa_status_t sparse_attn_indexer_grad_kl(const sa_indexer_desc_t* desc, const sa_indexer_args_t* args,
                                        void* workspace, size_t workspace_bytes, void* stream) {
  return sparse_attn_indexer_grad_kl_timed(desc, args, workspace, workspace_bytes, stream, nullptr, nullptr);
}

sa_status_t sparse_attn_bwd_workspace_size(const sa_desc_t* desc, size_t* bytes) {
  if (!bytes) return SA_ERR_NULL_PTR;
  sa_status_t st = validate(desc);
  if (st != SA_OK) return st;
  if (!sa::bwd_rows_supported(desc->d_qk, desc->d_v, desc->kv_shared)) return SA_ERR_UNSUPPORTED;
  const Params p = make_params(desc);
  // the per-XCD atomic form exists for the shared-KV MLA kernel only
  if (desc->dkv_mode == SA_DKV_ATOMIC_XCD && !sa::mla_bwd_supported(p)) return SA_ERR_UNSUPPORTED;
  *bytes = bwd_layout(desc, p).total;
  return SA_OK;
}

}  // extern "C"

namespace sa {

// The backward's launch sequence; allow_side = 0 keeps every launch on the
// caller's stream (no library-owned stream: the allocation-free entry point).
sa_status_t bwd_entry(const sa_desc_t* desc, const sa_bwd_args_t* a, void* workspace, size_t workspace_bytes,
                      void* stream, void* ev_main_start, void* ev_main_stop, int allow_side) {
  size_t need = 0;
  sa_status_t st = sparse_attn_bwd_workspace_size(desc, &need);
  if (st != SA_OK) return st;
  if (!a) return SA_ERR_NULL_PTR;
  if (total_q(desc) == 0 || desc->n_q_heads == 0) return SA_OK;   // empty query: nothing to do
  st = check_inputs(desc, a->q, a->k, a->v, a->kv, a->cmp_kv, a->sinks, a->topk_indices, a->cu_seqlens_q,
                    a->cu_seqlens_kv, a->cu_seqlens_cmp);
  if (st != SA_OK) return st;
  if (!a->o || !a->d_o || !a->lse || !a->dq) return SA_ERR_NULL_PTR;
  if (desc->kv_shared ? !a->dkv : (!a->dk || !a->dv)) return SA_ERR_NULL_PTR;
  if (desc->select == SA_SEL_WINDOW_CMP && rows_cmp(desc) > 0 && !a->d_cmp_kv) return SA_ERR_NULL_PTR;
  if (desc->has_sinks && !a->dsinks) return SA_ERR_NULL_PTR;
  if (desc->softmax_l1) {
    if (!a->ori_softmax_l1 || (desc->select == SA_SEL_WINDOW_CMP && desc->topk > 0 && !a->cmp_softmax_l1))
      return SA_ERR_NULL_PTR;
    if (((uintptr_t)a->ori_softmax_l1 & 3u) != 0 || ((uintptr_t)a->cmp_softmax_l1 & 3u) != 0)
      return SA_ERR_MISALIGNED;
  }
  if (!workspace) return SA_ERR_NULL_PTR;
  if (workspace_bytes < need) return SA_ERR_WORKSPACE_TOO_SMALL;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return SA_ERR_MISALIGNED;
  if (!aligned16(a->o) || !aligned16(a->d_o)) return SA_ERR_MISALIGNED;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  Params p = make_params(desc);
  const BwdLayout L = bwd_layout(desc, p);
  p.q = static_cast<const bf16*>(a->q);
  p.k = static_cast<const bf16*>(desc->kv_shared ? a->kv : a->k);
  p.v = desc->kv_shared ? nullptr : static_cast<const bf16*>(a->v);
  p.cmp = static_cast<const bf16*>(a->cmp_kv);
  p.o = static_cast<const bf16*>(a->o);
  p.dO = static_cast<const bf16*>(a->d_o);
  p.lse = a->lse;
  p.sinks = a->sinks;
  p.idx = a->topk_indices;
  p.cu_q = a->cu_seqlens_q;
  p.cu_kv = a->cu_seqlens_kv;
  p.cu_cmp = desc->topk > 0 ? a->cu_seqlens_cmp : nullptr;
  p.topk_len = a->topk_lengths;
  p.used_q = a->seqused_q;
  p.used_kv = a->seqused_kv;
  p.used_cmp = a->seqused_cmp;

  BwdBuffers w;
  std::memset(&w, 0, sizeof(w));
  w.D = reinterpret_cast<float*>(ws + L.D);
  w.sink_term = desc->has_sinks ? reinterpret_cast<float*>(ws + L.sink_term) : nullptr;
  w.dq = static_cast<bf16*>(a->dq);
  w.dsinks = a->dsinks;
  w.l1 = desc->softmax_l1 ? reinterpret_cast<float*>(ws + L.l1) : nullptr;
  w.t0 = 0;
  w.Tc = p.T;
  // softmax L1-norm outputs from the head-chunk sums the P kernel wrote
  auto l1_norm = [&]() -> hipError_t {
    if (!w.l1) return hipSuccess;
    return sa::launch_l1_norm(p, w.l1, L.n_hg_l1, a->ori_softmax_l1, a->cmp_softmax_l1, s);
  };

  const size_t Hkv = (size_t)desc->n_kv_heads;
  // The MLA kernel forms D and the dSinks terms from its own staged dO and
  // the O rows it loads beside them (their loads ride with the Q/dO staging),
  // which saves the separate pass's re-read of dO and O; every other call
  // takes them from the preprocess.
  const bool fused_d = L.mla;
  w.fuse_d = fused_d ? 1 : 0;
  if (!fused_d) {
    SA_TRY_HIP(sa::launch_preprocess(p, w, s));
    if (desc->has_sinks) SA_TRY_HIP(sa::launch_dsinks(p, w, s));
  }

  if (desc->dkv_mode != SA_DKV_DETERMINISTIC && L.mla) {
    // shared-KV MLA kernel, fp32 atomic adds (into the XCD's replica in the
    // per-XCD form), then one pass that sums the replicas in a fixed order
    // and casts
    w.acc_k = reinterpret_cast<float*>(ws + L.acc_k);
    w.acc_cmp = reinterpret_cast<float*>(ws + L.acc_cmp);
    w.out = L.n_rep > 1 ? sa::kOutAtomicXcd : sa::kOutAtomic;
    w.rep_stride = (long long)L.rep_floats;
    w.dump = ws + L.dump;
    w.npos = (int)n_positions_host(desc);
    w.RW = desc->d_qk;
    SA_TRY_HIP(sa::launch_fill_zero(w.acc_k, (size_t)L.n_rep * L.rep_floats, s));
    if (ev_main_start) SA_TRY_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(ev_main_start), s));
    SA_TRY_HIP(sa::launch_bwd_mla(p, w, s));
    if (ev_main_stop) SA_TRY_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(ev_main_stop), s));
    if (fused_d && desc->has_sinks) SA_TRY_HIP(sa::launch_dsinks(p, w, s));
    SA_TRY_HIP(l1_norm());
    const long long n_a = rows_kv(desc) * (long long)Hkv * desc->d_qk;
    SA_TRY_HIP(sa::launch_replica_sum_cast(w.acc_k, (long long)L.rep_floats, L.n_rep, (long long)L.rep_floats, n_a,
                                           a->dkv, a->d_cmp_kv, p.fp16, s));
    return SA_OK;
  }
  if (desc->dkv_mode == SA_DKV_ATOMIC) {
    w.acc_k = reinterpret_cast<float*>(ws + L.acc_k);
    w.acc_v = desc->kv_shared ? nullptr : reinterpret_cast<float*>(ws + L.acc_v);
    w.acc_cmp = desc->select == SA_SEL_WINDOW_CMP ? reinterpret_cast<float*>(ws + L.acc_cmp) : nullptr;
    const size_t nk = (size_t)rows_kv(desc) * Hkv * desc->d_qk;
    const size_t nv = desc->kv_shared ? 0 : (size_t)rows_kv(desc) * Hkv * desc->d_v;
    const size_t nc = (size_t)rows_cmp(desc) * Hkv * desc->d_qk;
    SA_TRY_HIP(sa::launch_fill_zero(w.acc_k, nk, s));
    if (nv) SA_TRY_HIP(sa::launch_fill_zero(w.acc_v, nv, s));
    if (nc) SA_TRY_HIP(sa::launch_fill_zero(w.acc_cmp, nc, s));
    if (ev_main_start) SA_TRY_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(ev_main_start), s));
    SA_TRY_HIP(sa::launch_bwd_rows(p, w, s));
    if (ev_main_stop) SA_TRY_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(ev_main_stop), s));
    SA_TRY_HIP(l1_norm());
    SA_TRY_HIP(sa::launch_cast(w.acc_k, desc->kv_shared ? a->dkv : a->dk, nk, p.fp16, s));
    if (nv) SA_TRY_HIP(sa::launch_cast(w.acc_v, a->dv, nv, p.fp16, s));
    if (nc) SA_TRY_HIP(sa::launch_cast(w.acc_cmp, a->d_cmp_kv, nc, p.fp16, s));
    return SA_OK;
  }

  // deterministic: per token chunk, CSR of the chunk's slots, partial rows,
  // key-major reduce into the fp32 accumulator; then one cast
  int* blk_base = reinterpret_cast<int*>(ws + L.blk_base);
  int* row_ptr = reinterpret_cast<int*>(ws + L.row_ptr);
  int* entries = reinterpret_cast<int*>(ws + L.entries);
  float* acc = reinterpret_cast<float*>(ws + L.acc);
  const long long nk = csr_keys_bound(desc);
  const bool has_slots = desc->topk > 0;
  if (desc->select == SA_SEL_BLOCK) SA_TRY_HIP(sa::launch_block_base(p, blk_base, s));
  if (L.blk_km) {
    // dQ from the row kernel; dK/dV key-major over the CSR of block keys.
    // The CSR, chunk count and key-major pass run on the side stream beside
    // the dQ pass where there is one (see above).
    std::unique_lock<std::mutex> side_lock(g_side_mu, std::defer_lock);
    SideCtx* side = nullptr;
    if (allow_side) {
      const char* env = std::getenv("SPARSE_ATTN_SIDE_STREAM");
      if (!env || std::atoi(env) != 0) {
        side_lock.lock();
        side = side_ctx(stream_device(s));
        if (!side) side_lock.unlock();
      }
    }
    hipStream_t ks = s;   // the key-major chain's stream
    if (side) {
      SA_TRY_HIP(hipEventRecord(side->ev_fork, s));
      SA_TRY_HIP(hipStreamWaitEvent(side->s, side->ev_fork, 0));
      ks = side->s;
    }
    sa::BlkArgs ba;
    std::memset(&ba, 0, sizeof(ba));
    ba.row_ptr = row_ptr;
    ba.entries = entries;
    ba.blk_base = blk_base;
    ba.D = w.D;
    ba.part = reinterpret_cast<float*>(ws + L.bpart);
    ba.chunk_base = reinterpret_cast<int*>(ws + L.bchunk);
    ba.max_chunks = L.max_chunks;
    ba.n_hc = L.n_hc_blk;
    ba.n_keys = nk;
    const long long nrows = rows_kv(desc) * (long long)Hkv;
    if (has_slots) SA_TRY_HIP(sa::launch_csr_transpose(p, 0, p.T, nk, blk_base, row_ptr, entries, ws + L.csr_ws, ks));
    else SA_TRY_HIP(sa::launch_fill_zero(reinterpret_cast<float*>(row_ptr), (size_t)(nk + 1), ks));
    SA_TRY_HIP(sa::launch_blk_chunks(row_ptr, nk, reinterpret_cast<int*>(ws + L.bcnt), ba.chunk_base,
                                     reinterpret_cast<int*>(ws + L.bscan), ks));
    if (has_slots) {
      SA_TRY_HIP(sa::launch_blk_dkv(p, ba, ks));
    }
    // the chunk sums and cast need only the key-major pass
    SA_TRY_HIP(sa::launch_blk_sum_cast(p, ba, nrows, static_cast<bf16*>(a->dk), static_cast<bf16*>(a->dv), ks));
    w.det = 1;
    w.dq_only = 1;
    // the timed "main" kernel of this path: the dQ pass (the larger one)
    if (ev_main_start) SA_TRY_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(ev_main_start), s));
    SA_TRY_HIP(sa::blk_dq_supported(p) ? sa::launch_blk_dq(p, w, s) : sa::launch_bwd_rows(p, w, s));
    if (ev_main_stop) SA_TRY_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(ev_main_stop), s));
    SA_TRY_HIP(l1_norm());
    if (side) {
      SA_TRY_HIP(hipEventRecord(side->ev_join, side->s));
      SA_TRY_HIP(hipStreamWaitEvent(s, side->ev_join, 0));
    }
    return SA_OK;
  }
  w.det = 1;
  w.partial = ws + L.partial;
  w.dump = ws + L.dump;
  w.npos = (int)n_positions_host(desc);
  w.RW = L.RW;
  sa::ReduceArgs r;
  std::memset(&r, 0, sizeof(r));
  r.partial = w.partial;
  r.partial_bf16 = L.fast;
  r.RW = L.RW;
  r.npos = w.npos;
  r.n_hc = L.n_hc;
  r.row_ptr = row_ptr;
  r.entries = entries;
  r.blk_base = blk_base;
  r.n_kv_out = rows_kv(desc) * (long long)Hkv;
  r.n_out_rows = r.n_kv_out + rows_cmp(desc) * (long long)Hkv;
  r.acc = acc;
  // no index slots (window only): every key list is empty
  if (!has_slots) SA_TRY_HIP(sa::launch_fill_zero(reinterpret_cast<float*>(row_ptr), (size_t)(nk + 1), s));
  bool first = true;
  for (int t0 = 0; t0 < p.T; t0 += L.Tc) {
    const int t1 = std::min(p.T, t0 + L.Tc);
    w.t0 = t0;
    w.Tc = t1 - t0;
    if (has_slots)
      SA_TRY_HIP(sa::launch_csr_transpose(p, t0, t1, nk, blk_base, row_ptr, entries, ws + L.csr_ws, s));
    if (ev_main_start && first) SA_TRY_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(ev_main_start), s));
    SA_TRY_HIP(L.fast ? sa::launch_bwd_mla(p, w, s) : sa::launch_bwd_rows(p, w, s));
    if (ev_main_stop && t1 == p.T) SA_TRY_HIP(hipEventRecord(reinterpret_cast<hipEvent_t>(ev_main_stop), s));
    r.t0 = t0;
    r.Tc = t1 - t0;
    r.accumulate = first ? 0 : 1;
    SA_TRY_HIP(sa::launch_reduce(p, r, s));
    first = false;
  }
  if (fused_d && desc->has_sinks) SA_TRY_HIP(sa::launch_dsinks(p, w, s));
  SA_TRY_HIP(l1_norm());
  bf16* out_a = static_cast<bf16*>(desc->kv_shared ? a->dkv : a->dk);
  bf16* out_b = desc->kv_shared ? nullptr : static_cast<bf16*>(a->dv);
  SA_TRY_HIP(sa::launch_split_cast(acc, r.n_kv_out, L.RW, desc->d_qk, out_a, out_b, p.fp16, s));
  if (desc->select == SA_SEL_WINDOW_CMP)
    SA_TRY_HIP(sa::launch_cast(acc + r.n_kv_out * L.RW, a->d_cmp_kv, (size_t)(r.n_out_rows - r.n_kv_out) * L.RW,
                               p.fp16, s));
  return SA_OK;
}

}  // namespace sa

extern "C" {

sa_status_t sparse_attn_bwd_timed(const sa_desc_t* desc, const sa_bwd_args_t* a, void* workspace,
                                  size_t workspace_bytes, void* stream, void* ev_main_start,
                                  void* ev_main_stop) {
  return sa::bwd_entry(desc, a, workspace, workspace_bytes, stream, ev_main_start, ev_main_stop, 1);
}

sa_status_t sparse_attn_bwd(const sa_desc_t* desc, const sa_bwd_args_t* a, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return sparse_attn_bwd_timed(desc, a, workspace, workspace_bytes, stream, nullptr, nullptr);
}

sa_status_t sparse_attn_fwd(const sa_desc_t* desc, const sa_fwd_args_t* a, void* stream) {
  sa_status_t st = validate(desc);
  if (st != SA_OK) return st;
  if (!sa::fwd_rows_supported(desc->d_qk, desc->d_v, desc->kv_shared)) return SA_ERR_UNSUPPORTED;
  if (!a) return SA_ERR_NULL_PTR;
  if (total_q(desc) == 0 || desc->n_q_heads == 0) return SA_OK;
  st = check_inputs(desc, a->q, a->k, a->v, a->kv, a->cmp_kv, a->sinks, a->topk_indices, a->cu_seqlens_q,
                    a->cu_seqlens_kv, a->cu_seqlens_cmp);
  if (st != SA_OK) return st;
  if (!a->o || !a->lse) return SA_ERR_NULL_PTR;
  Params p = make_params(desc);
  p.q = static_cast<const bf16*>(a->q);
  p.k = static_cast<const bf16*>(desc->kv_shared ? a->kv : a->k);
  p.v = desc->kv_shared ? nullptr : static_cast<const bf16*>(a->v);
  p.cmp = static_cast<const bf16*>(a->cmp_kv);
  p.sinks = a->sinks;
  p.idx = a->topk_indices;
  p.cu_q = a->cu_seqlens_q;
  p.cu_kv = a->cu_seqlens_kv;
  p.cu_cmp = desc->topk > 0 ? a->cu_seqlens_cmp : nullptr;
  p.topk_len = a->topk_lengths;
  p.used_q = a->seqused_q;
  p.used_kv = a->seqused_kv;
  p.used_cmp = a->seqused_cmp;
  SA_TRY_HIP(sa::launch_fwd_rows(p, a->o, a->lse, reinterpret_cast<hipStream_t>(stream)));
  return SA_OK;
}

sa_status_t sparse_attn_csr_size(const sa_desc_t* desc, const int32_t* host_cu_seqlens_kv, int64_t* n_keys,
                                 size_t* workspace_bytes) {
  if (!n_keys || !workspace_bytes) return SA_ERR_NULL_PTR;
  sa_status_t st = validate(desc);
  if (st != SA_OK) return st;
  long long nk;
  if (desc->select == SA_SEL_BLOCK && desc->layout == SA_LAYOUT_TND) {
    if (!host_cu_seqlens_kv) return SA_ERR_NULL_PTR;
    long long blocks = 0;
    for (int b = 0; b < desc->batch; ++b) {
      const int len = host_cu_seqlens_kv[b + 1] - host_cu_seqlens_kv[b];
      if (len < 0) return SA_ERR_BAD_SHAPE;
      blocks += (len + desc->block_size - 1) / desc->block_size;
    }
    nk = blocks * desc->n_kv_heads;
  } else {
    nk = csr_keys_bound(desc);
  }
  if (nk >= kMaxI32) return SA_ERR_BAD_SHAPE;
  *n_keys = nk;
  const long long n_slots = total_q(desc) * desc->n_kv_heads * desc->topk;
  if (n_slots > kMaxI32) return SA_ERR_BAD_SHAPE;   // entries are int32 slot ids
  *workspace_bytes = align_up((size_t)(desc->batch + 1) * 4) + sa::csr_workspace_bytes(n_slots, nk, desc->batch);
  return SA_OK;
}

sa_status_t sparse_attn_csr_transpose(const sa_desc_t* desc, const int32_t* topk_indices,
                                      const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_kv,
                                      int32_t* row_ptr, int32_t* entries, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  sa_status_t st = validate(desc);
  if (st != SA_OK) return st;
  if (desc->topk < 1) return SA_ERR_BAD_SHAPE;
  if (!topk_indices || !row_ptr || !entries || !workspace) return SA_ERR_NULL_PTR;
  if (desc->layout == SA_LAYOUT_TND && (!cu_seqlens_q || !cu_seqlens_kv)) return SA_ERR_NULL_PTR;
  if (desc->select == SA_SEL_WINDOW_CMP && !cu_seqlens_kv) return SA_ERR_NULL_PTR;
  if (((uintptr_t)workspace & (kAlign - 1)) != 0) return SA_ERR_MISALIGNED;
  // exact key count (BSND or TND token/window) comes from the descriptor;
  // TND block mode uses the bound, whose extra keys stay empty
  const long long nk = csr_keys_bound(desc);
  const long long n_slots = total_q(desc) * desc->n_kv_heads * desc->topk;
  if (n_slots > kMaxI32) return SA_ERR_BAD_SHAPE;   // entries are int32 slot ids
  const size_t need = align_up((size_t)(desc->batch + 1) * 4) + sa::csr_workspace_bytes(n_slots, nk, desc->batch);
  if (workspace_bytes < need) return SA_ERR_WORKSPACE_TOO_SMALL;
  if (total_q(desc) == 0) return SA_OK;
  Params p = make_params(desc);
  p.idx = topk_indices;
  p.cu_q = cu_seqlens_q;
  p.cu_kv = cu_seqlens_kv;
  p.cu_cmp = cu_seqlens_kv;   // window+cmp: the key table is cmp_kv
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int* blk_base = static_cast<int*>(workspace);
  void* ws = static_cast<char*>(workspace) + align_up((size_t)(desc->batch + 1) * 4);
  if (desc->select == SA_SEL_BLOCK) SA_TRY_HIP(sa::launch_block_base(p, blk_base, s));
  SA_TRY_HIP(sa::launch_csr_transpose(p, 0, p.T, nk, blk_base, row_ptr, entries, ws, s));
  return SA_OK;
}

const char* sparse_attn_status_string(sa_status_t status) {
  switch (status) {
    case SA_OK: return "SA_OK";
    case SA_ERR_NULL_PTR: return "SA_ERR_NULL_PTR: a required pointer is NULL";
    case SA_ERR_BAD_SHAPE: return "SA_ERR_BAD_SHAPE: inconsistent or non-positive sizes";
    case SA_ERR_UNSUPPORTED: return "SA_ERR_UNSUPPORTED: request outside the built kernels";
    case SA_ERR_WORKSPACE_TOO_SMALL: return "SA_ERR_WORKSPACE_TOO_SMALL: workspace below the phase-1 size";
    case SA_ERR_MISALIGNED: return "SA_ERR_MISALIGNED: pointer not 16-byte (workspace: 256-byte) aligned";
    case SA_ERR_HIP: return "SA_ERR_HIP: a HIP launch or runtime call failed";
    case SA_ERR_BAD_ARG: return "SA_ERR_BAD_ARG: invalid enum value, flag or scale";
  }
  return "unknown sa_status_t";
}

int32_t sparse_attn_version(void) { return 100; }

}  // extern "C"
