// Host-side launchers of the library's kernels (one translation unit per
// kernel family; the C ABI in sa_api.hip sequences them on one stream).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "sa_device.h"

namespace sa {

// Output forms of the shared-KV MLA kernel's phase B.
constexpr int kOutPartial = 0;     // bf16 partial rows, key-major reduce afterwards
constexpr int kOutAtomic = 1;      // fp32 atomic adds into one accumulator
constexpr int kOutAtomicXcd = 2;   // fp32 atomic adds into the XCD's accumulator replica
constexpr int kXcdReplicas = 8;

// Output/workspace pointers of one backward call.
struct BwdBuffers {
  float* D;          // [T][Hq] softmax-grad term
  float* sink_term;  // [T][Hq] per-row dSinks terms (sinks only)
  int fuse_d;        // MLA kernel: form D (and the dSinks terms) itself instead of reading D
  float* acc_k;      // fp32 dK (or shared dKV) accumulator, rows x Hkv x dqk (atomic mode)
  float* acc_v;      // fp32 dV accumulator (separate V, atomic mode)
  float* acc_cmp;    // fp32 dCmpKV accumulator (window+cmp, atomic mode)
  // MLA kernel: how phase B leaves the kernel (kOutPartial, kOutAtomic or
  // kOutAtomicXcd); with kOutAtomicXcd, replica x of acc_k / acc_cmp starts
  // x * rep_stride floats further on
  int out;
  long long rep_stride;
  bf16* dq;
  float* dsinks;
  // deterministic mode: one partial row per (head chunk, token, kv head,
  // selected position) of tokens [t0, t0 + Tc), RW columns each
  // (shared KV: dKV [dqk]; separate: dK [dqk] then dV [dv])
  void* partial;
  void* dump;        // one never-read row: target of the stores of unused tile rows
  // softmax L1-norm outputs: the row kernels write, for every (token, kv
  // head) row and used virtual position, the sum of P over the workgroup's
  // heads to l1[(head chunk * T * Hkv + row) * npos + position] (null: not
  // requested); the normalisation pass sums the head chunks
  float* l1;
  int det;
  int dq_only;       // row kernel: dQ only (dK/dV come from the key-major block kernel)
  int t0, Tc, npos, RW;
};

// Arguments of the key-major reduction of partial rows.
struct ReduceArgs {
  const void* partial;
  int partial_bf16;
  int RW, npos, n_hc, t0, Tc;
  const int* row_ptr;    // CSR over keys of the chunk's slots
  const int* entries;
  const int* blk_base;   // block mode: first block id of every sequence
  long long n_out_rows;  // kv rows * Hkv (+ cmp rows * Hkv)
  long long n_kv_out;    // kv rows * Hkv
  float* acc;            // [n_out_rows][RW]
  int accumulate;        // 0: overwrite, 1: add
};

hipError_t launch_fill_zero(float* p, size_t n, hipStream_t s);
hipError_t launch_preprocess(const Params& p, const BwdBuffers& w, hipStream_t s);
hipError_t launch_bwd_rows(const Params& p, const BwdBuffers& w, hipStream_t s);
hipError_t launch_dsinks(const Params& p, const BwdBuffers& w, hipStream_t s);
// fp32 -> bf16 (fp16 = 0) or fp16 (fp16 = 1), round to nearest even
hipError_t launch_cast(const float* src, void* dst, size_t n, int fp16, hipStream_t s);
bool bwd_rows_supported(int dqk, int dv, int shared);
int bwd_rows_head_chunks(const Params& p);

hipError_t launch_fwd_rows(const Params& p, void* o, float* lse, hipStream_t s);
bool fwd_rows_supported(int dqk, int dv, int shared);

// CSR transpose of the index lists of tokens [t0, t1): row_ptr[n_keys + 1]
// and entries (flat slot ids minus t0 * Hkv * topk, ascending per key; the
// range must hold fewer than 2^31 slots).
size_t csr_workspace_bytes(long long n_slots, long long n_keys, int batch);
hipError_t launch_block_base(const Params& p, int* blk_base, hipStream_t s);
hipError_t launch_csr_transpose(const Params& p, int t0, int t1, long long n_keys, const int* blk_base,
                                int* row_ptr, int* entries, void* ws, hipStream_t s);

hipError_t launch_reduce(const Params& p, const ReduceArgs& r, hipStream_t s);
hipError_t launch_split_cast(const float* acc, long long n_rows, int RW, int dqk, void* a, void* b, int fp16,
                             hipStream_t s);
// out[i] = sum over x = 0..n_rep-1, in that order, of acc[x * stride + i],
// cast to the 16-bit output: elements [0, n_a) to a, [n_a, n) to b
hipError_t launch_replica_sum_cast(const float* acc, long long stride, int n_rep, long long n, long long n_a, void* a,
                                   void* b, int fp16, hipStream_t s);

// Softmax L1-norm outputs from the head-chunk sums `l1` ([n_hg][T * Hkv]
// [npos]): per (token, kv head) row, the chunk sums of every used position
// are added in chunk order, then divided by the ori (resp. cmp) total.
hipError_t launch_l1_norm(const Params& p, const float* l1, int n_hg, float* ori, float* cmp, hipStream_t s);

}  // namespace sa

namespace sa {
// Key-major dK/dV of block selection (separate K/V, d_qk = d_v): every
// block key's CSR list is cut into chunks of kBlkChunk queries; one
// workgroup per (chunk, 16-head chunk) writes the fp32 dK|dV rows of its
// block into its own slot of `part` ([n_hc][max_chunks][64][2 d]); the
// chunks of a key are then summed in chunk order.
constexpr int kBlkChunk = 64;
struct BlkArgs {
  const int* row_ptr;
  const int* entries;
  const int* blk_base;
  const float* D;        // [T][Hq] softmax-grad term
  int* chunk_base;       // [n_keys + 1]: first chunk of every key (exclusive scan)
  float* part;
  long long max_chunks;  // bound on the number of chunks (grid size)
  long long n_keys;      // CSR keys (bound)
  int n_hc;              // head chunks of 16
};
bool blk_dkv_supported(const Params& p);
int blk_dkv_head_chunks(const Params& p);
long long blk_max_chunks(long long n_keys, long long n_slots);
// chunk_base from row_ptr (uses `cnt` [n_keys + 1] and `scan_ws` scratch)
hipError_t launch_blk_chunks(const int* row_ptr, long long n_keys, int* cnt, int* chunk_base, int* scan_ws,
                             hipStream_t s);
hipError_t launch_blk_dkv(const Params& p, const BlkArgs& a, hipStream_t s);
// n_rows: kv rows * Hkv
hipError_t launch_blk_sum_cast(const Params& p, const BlkArgs& a, long long n_rows, bf16* dk, bf16* dv,
                               hipStream_t s);
// exclusive scan of in[0..n) into out[0..n_out) (out past n: the total);
// `bsum` holds scan_bsum_ints(max(n, n_out)) ints
hipError_t launch_scan_excl(const int* in, long long n, int* out, long long n_out, int* bsum, hipStream_t s);
long long scan_bsum_ints(long long n);
// dQ of block selection, query-major (d = 128, up to 256 slots, block_size a
// multiple of 16 and at most 64)
bool blk_dq_supported(const Params& p);
hipError_t launch_blk_dq(const Params& p, const BwdBuffers& w, hipStream_t s);

// Sparse lightning-indexer gradient with the KL loss (d = 128, up to 64
// heads, up to 2048 slots per token, one kv row table).  Tokens [t0, t0 +
// Tc) write their dq~, dW and loss, and one bf16 partial dK~ row per
// (token, slot) to part[(t - t0) * topk + slot][128].
struct IdxArgs {
  const bf16* q;         // [T][H][128]
  const bf16* k;         // [T_kv][128]
  const float* w;        // [T][H]
  const float* target;   // [T][topk]
  bf16* dq;              // [T][H][128]
  float* dw;             // [T][H]
  float* loss_tok;       // [T]
  bf16* part;
  bf16* dump;            // >= 256 bytes, never read
  int H, t0, Tc;
};
bool idx_grad_supported(const Params& p);
hipError_t launch_idx_grad(const Params& p, const IdxArgs& a, hipStream_t s);

// Shared-KV 576/512 backward with 64 heads per workgroup (bf16 partials).
bool mla_bwd_supported(const Params& p);
int mla_bwd_head_groups(const Params& p);
hipError_t launch_bwd_mla(const Params& p, const BwdBuffers& w, hipStream_t s);
}  // namespace sa
