// Deterministic key-major reduction of the per-pair dK/dV (dKV) partial rows.
//
// The row kernels write one partial row per (head chunk, token, kv head,
// selected position) into a token-major buffer; this kernel sums, for
// every output row, the partials that name it in a fixed order -- by the
// CSR transpose of the index lists (ascending slot id; for rows narrower
// than a wave, interleaved batches of the list per sub-group, the sub-group
// sums then in sub-group order), or for window keys by ascending query
// token -- and adds the sum into an fp32 accumulator.  The order never
// depends on scheduling, so results are bitwise repeatable.  (aclnnSparseFlashAttentionGrad, "Formula": dK[u] and
// dV[u] collect the contributions of every query that gathered row u.)
#include "sa_launch.h"

namespace sa {

namespace {

// Every partial row is read exactly once, so the loads are non-temporal:
// the rows stream past the caches instead of evicting lines that are still
// in use (measured on the 8192-token shared-KV shape: 5.9 -> 6.6 TB/s).
template <typename PT>
struct Vec8;

template <>
struct Vec8<float> {
  static constexpr int kPer = 4;   // columns per thread-step
  typedef float4 T;
  __device__ static T load(const float* p) {
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v v = __builtin_nontemporal_load(reinterpret_cast<const f4v*>(p));
    return make_float4(v[0], v[1], v[2], v[3]);
  }
  __device__ static void add(const T& v, float* acc) {
    acc[0] += v.x;
    acc[1] += v.y;
    acc[2] += v.z;
    acc[3] += v.w;
  }
};

template <>
struct Vec8<bf16> {
  static constexpr int kPer = 8;
  typedef bf16x8 T;
  __device__ static T load(const bf16* p) { return __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p)); }
  __device__ static void add(const T& v, float* acc) {
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += (float)v[i];
  }
};

constexpr int kBatch = 16;  // partial rows whose loads are in flight together

// One group of TPR threads per output row; each thread owns kPer columns.
// SPLIT (token selection only, TPR a divisor of 64 below 64): one wave per
// output row, whose 64 / TPR sub-groups take the row's CSR list in
// interleaved batches (sub-group q: batches q, q + 64 / TPR, ...); their sums
// are then added in sub-group order.  Short rows (few columns) otherwise
// leave most of the GPU idle while the longest list is walked one batch
// after another, each batch waiting for its entries and then its rows.
// NSUB > 1 (rows of a wave or more, e.g. the 576-column bf16 rows of the
// shared-KV kernel): NSUB groups of TPR threads per output row take its
// list in interleaved batches (group q: batches q, q + NSUB, ...), and
// their sums are added in group order through LDS.  The longest lists
// (several thousand entries on the shared-KV workloads) otherwise set the
// kernel's time, one batch after another.
constexpr int kRedLds = 4096;   // floats of LDS for the NSUB > 1 group sums
constexpr int kRedSub = 2;      // NSUB of the wide bf16 rows
template <typename PT, bool SPLIT, int NSUB>
__global__ void reduce_kernel(Params p, ReduceArgs r) {
  static_assert(!SPLIT || NSUB == 1, "one split form at a time");
  constexpr int kPer = Vec8<PT>::kPer;
  const int tpr = r.RW / kPer;
  const int grp = SPLIT ? 64 : tpr * NSUB;               // threads per output row
  const int nsg = SPLIT ? 64 / tpr : NSUB;               // sub-groups per output row
  const int sg = SPLIT ? (int)(threadIdx.x & 63) / tpr : (int)(threadIdx.x % grp) / tpr;
  const int sub = threadIdx.x % tpr;
  const int rpb = blockDim.x / grp;                      // output rows per block
  const long long lin = (long long)blockIdx.x * rpb + threadIdx.x / grp;
  const bool valid = lin < r.n_out_rows && (int)(threadIdx.x / grp) < rpb;
  // SPLIT: lin is uniform over the wave, so whole waves leave here (NSUB >
  // 1: every thread stays for the barrier of the group sums)
  if (NSUB == 1 && !valid) return;
  // Heavy rows first: the cmp rows (each named by the cmp slots of many
  // queries) are scheduled before the window rows (at most win_left + 1 +
  // win_right partials each), so the long sums do not form the grid's tail.
  // A bijection on the output rows; each row's summation order is unchanged.
  const long long n_cmp_out = r.n_out_rows - r.n_kv_out;
  const long long orow = !valid ? 0 : lin < n_cmp_out ? r.n_kv_out + lin : lin - n_cmp_out;
  const int col = sub * kPer;
  const PT* part = static_cast<const PT*>(r.partial);
  float acc[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) acc[i] = 0.f;
  const long long rows_chunk = (long long)r.Tc * p.Hkv;          // partial rows per head chunk
  const long long row0 = (long long)r.t0 * p.Hkv;
  const int npos = r.npos;

  const long long hc_stride = rows_chunk * npos * (long long)r.RW;
  // Adds up to kBatch partial rows (element offsets off[], for every head
  // chunk) in the listed order; all loads are issued before the first add.
  auto add_batch = [&](const long long* off, const bool* ok) {
    for (int hc = 0; hc < r.n_hc; ++hc) {
      typename Vec8<PT>::T v[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) v[u] = Vec8<PT>::load(part + hc * hc_stride + off[u]);
#pragma unroll
      for (int u = 0; u < kBatch; ++u)
        if (ok[u]) Vec8<PT>::add(v[u], acc);
    }
  };
  // partial row of position `pos` of chunk-local (token, kv head) row lrow
  auto offset_of = [&](long long lrow, int pos) -> long long { return (lrow * npos + pos) * r.RW + col; };

  if (valid) {
  const bool is_cmp = orow >= r.n_kv_out;   // cmp rows follow the kv rows
  if (!is_cmp && p.select == kSelWindowCmp) {
    // window keys: query tokens t with t - win_left <= j <= t + win_right
    const long long jg = orow / p.Hkv;                 // global kv row
    const int g = (int)(orow - jg * p.Hkv);
    // sequence of this kv row
    int b = 0;
    if (p.layout == kLayoutBSND) {
      b = (int)(jg / p.Skv);
    } else {
      int lo = 0, hi = p.B;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_kv[mid] <= jg) lo = mid; else hi = mid;
      }
      b = lo;
    }
    const SeqLens L = seq_lens(p, b);
    const int jl = (int)(jg - L.kv_base);
    // query i sits at key position i + L.off; its window is [pos - win_left,
    // pos + win_right] (and <= pos when causal); kv rows past the used ones
    // are in no window
    int tl_lo = max(0, jl - p.win_right - L.off);
    int tl_hi = min(L.q_len - 1, jl + p.win_left - L.off);
    if (p.causal) tl_lo = max(tl_lo, jl - L.off);
    if (jl >= L.kv_len) tl_hi = -1;
    // only query tokens of this chunk contribute
    tl_lo = max(tl_lo, r.t0 - L.q_base);
    tl_hi = min(tl_hi, r.t0 + r.Tc - 1 - L.q_base);
    for (int tb = tl_lo + sg * kBatch; tb <= tl_hi; tb += nsg * kBatch) {
      long long off[kBatch];
      bool ok[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        ok[u] = tb + u <= tl_hi;
        const int tl = ok[u] ? tb + u : tl_lo;
        off[u] = offset_of((long long)(L.q_base + tl) * p.Hkv + g - row0, jl - (tl + L.off - p.win_left));
      }
      add_batch(off, ok);
    }
  } else {
    const long long key = is_cmp ? orow - r.n_kv_out : orow;
    const long long kcsr = key;   // CSR key id (kv row * Hkv + g, block key, or cmp row * Hkv + g)
    const int nwin = p.select == kSelWindowCmp ? p.win_left + 1 + p.win_right : 0;
    if (p.select == kSelBlock) {
      // orow is (global kv row, g); its block key comes from the sequence
      const long long jg = orow / p.Hkv;
      const int g = (int)(orow - jg * p.Hkv);
      int b = 0;
      if (p.layout == kLayoutBSND) {
        b = (int)(jg / p.Skv);
      } else {
        int lo = 0, hi = p.B;
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (p.cu_kv[mid] <= jg) lo = mid; else hi = mid;
        }
        b = lo;
      }
      const SeqLens L = seq_lens(p, b);
      const int jl = (int)(jg - L.kv_base);
      const long long bkey = (long long)(r.blk_base[b] + jl / p.bs) * p.Hkv + g;
      const int off = jl % p.bs;
      const int eb = r.row_ptr[bkey];
      const int ee = jl < L.kv_len ? r.row_ptr[bkey + 1] : eb;   // rows past the used ones: nothing
      for (int e = eb + sg * kBatch; e < ee; e += nsg * kBatch) {
        long long offs[kBatch];
        bool ok[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          ok[u] = e + u < ee;
          // chunk-local slot id -> chunk-local row and slot
          const int slot = r.entries[ok[u] ? e + u : eb];
          const int lrow = (int)((unsigned)slot / (unsigned)p.topk);
          const int s = slot - lrow * p.topk;
          if (ok[u] && p.causal) {
            const SeqPos sp = seq_pos(p, (int)((row0 + lrow) / p.Hkv));
            ok[u] = jl <= sp.tl;     // row masked inside the selected block
          }
          offs[u] = offset_of(lrow, s * p.bs + off);
        }
        add_batch(offs, ok);
      }
    } else {
      const int eb = r.row_ptr[kcsr], ee = r.row_ptr[kcsr + 1];
      if (nwin == 0) {
        // Chunk-local slot id (lrow * topk + s) -> partial row lrow * npos
        // + s, and npos = topk here: the slot id itself, no division.
        for (int e = eb + sg * kBatch; e < ee; e += nsg * kBatch) {
          long long offs[kBatch];
          bool ok[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            ok[u] = e + u < ee;
            offs[u] = (long long)r.entries[ok[u] ? e + u : eb] * r.RW + col;
          }
          add_batch(offs, ok);
        }
      } else {
        // cmp slots follow the nwin window positions of their row.  (A
        // division-free form of this offset, slot + (row + 1) nwin - row0
        // npos, measured slower here: 4.1 against 3.3 ms on the window+cmp
        // varlen shape.)
        for (int e = eb + sg * kBatch; e < ee; e += nsg * kBatch) {
          long long offs[kBatch];
          bool ok[kBatch];
#pragma unroll
          for (int u = 0; u < kBatch; ++u) {
            ok[u] = e + u < ee;
            const long long slot = r.entries[ok[u] ? e + u : eb];
            const long long lrow = slot / p.topk;
            offs[u] = offset_of(lrow, nwin + (int)(slot - lrow * p.topk));
          }
          add_batch(offs, ok);
        }
      }
    }
  }
  }   // valid
  if constexpr (SPLIT) {
    // sub-group sums in sub-group order (lane sub + q * tpr: sub-group q)
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      float t = __shfl(acc[i], sub);
      for (int q = 1; q < nsg; ++q) t += __shfl(acc[i], sub + q * tpr);
      acc[i] = t;
    }
    if (sg != 0) return;
  }
  if constexpr (NSUB > 1) {
    // group sums in group order: groups 1.. through LDS, added by group 0
    __shared__ float red[kRedLds];
    const int slot = (int)(threadIdx.x / grp) * (NSUB - 1);
    if (valid && sg > 0) {
#pragma unroll
      for (int i = 0; i < kPer; ++i) red[(slot + sg - 1) * r.RW + col + i] = acc[i];
    }
    __syncthreads();
    if (!valid || sg != 0) return;
#pragma unroll
    for (int q = 1; q < NSUB; ++q)
#pragma unroll
      for (int i = 0; i < kPer; ++i) acc[i] += red[(slot + q - 1) * r.RW + col + i];
  }
  float* dst = r.acc + orow * (long long)r.RW + col;
  if (r.accumulate) {
#pragma unroll
    for (int i = 0; i < kPer; ++i) dst[i] += acc[i];
  } else {
#pragma unroll
    for (int i = 0; i < kPer; ++i) dst[i] = acc[i];
  }
}

// fp32 accumulator rows [n][RW] -> bf16 outputs: first dqk columns to
// `a`, the next dv columns (separate K/V) to `b`.
template <typename E>
__global__ void split_cast_kernel(const float* __restrict__ acc, long long n, int RW, int dqk, E* __restrict__ a,
                                  E* __restrict__ b) {
  const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (i >= n * RW) return;
  const long long row = i / RW;
  const int c = (int)(i - row * RW);
  if (c < dqk) a[row * dqk + c] = (E)acc[i];
  else b[row * (RW - dqk) + (c - dqk)] = (E)acc[i];
}

// Fixed-order sum of the accumulator replicas of the per-XCD atomic form,
// cast to the 16-bit output (the first n_a elements to a, the rest to b).
template <typename E>
__global__ void replica_sum_cast_kernel(const float* __restrict__ acc, long long stride, int n_rep, long long n,
                                        long long n_a, E* __restrict__ a, E* __restrict__ b) {
  const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (i >= n) return;
  float v = acc[i];
  for (int x = 1; x < n_rep; ++x) v += acc[x * stride + i];
  if (i < n_a) a[i] = (E)v;
  else b[i - n_a] = (E)v;
}

}  // namespace

hipError_t launch_replica_sum_cast(const float* acc, long long stride, int n_rep, long long n, long long n_a, void* a,
                                   void* b, int fp16, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (fp16)
    hipLaunchKernelGGL(replica_sum_cast_kernel<f16>, grid, dim3(256), 0, s, acc, stride, n_rep, n, n_a,
                       static_cast<f16*>(a), static_cast<f16*>(b));
  else
    hipLaunchKernelGGL(replica_sum_cast_kernel<bf16>, grid, dim3(256), 0, s, acc, stride, n_rep, n, n_a,
                       static_cast<bf16*>(a), static_cast<bf16*>(b));
  return hipGetLastError();
}

hipError_t launch_reduce(const Params& p, const ReduceArgs& r, hipStream_t s) {
  if (r.n_out_rows == 0) return hipSuccess;
  const int kPer = r.partial_bf16 ? 8 : 4;
  const int tpr = r.RW / kPer;
  // token selection: every output row takes the CSR branch, which is the
  // one that splits its list
  const bool split = p.select == kSelToken && tpr < 64 && 64 % tpr == 0;
  // bf16 rows of more than a wave (the shared-KV kernel's 576 columns):
  // kRedSub groups per row, when their sums fit the LDS of a block
  const int nsub = !split && r.partial_bf16 && tpr >= 64 ? kRedSub : 1;
  const int grp = split ? 64 : tpr * nsub;
  const int rpw = std::max(1, 512 / grp);
  const int threads = grp * rpw;
  const unsigned blocks = (unsigned)((r.n_out_rows + rpw - 1) / rpw);
  if (nsub > 1 && rpw * (nsub - 1) * r.RW > kRedLds) return hipErrorInvalidValue;
  if (r.partial_bf16) {
    if (split) hipLaunchKernelGGL((reduce_kernel<bf16, true, 1>), dim3(blocks), dim3(threads), 0, s, p, r);
    else if (nsub > 1)
      hipLaunchKernelGGL((reduce_kernel<bf16, false, kRedSub>), dim3(blocks), dim3(threads), 0, s, p, r);
    else hipLaunchKernelGGL((reduce_kernel<bf16, false, 1>), dim3(blocks), dim3(threads), 0, s, p, r);
  } else {
    if (split) hipLaunchKernelGGL((reduce_kernel<float, true, 1>), dim3(blocks), dim3(threads), 0, s, p, r);
    else hipLaunchKernelGGL((reduce_kernel<float, false, 1>), dim3(blocks), dim3(threads), 0, s, p, r);
  }
  return hipGetLastError();
}

hipError_t launch_split_cast(const float* acc, long long n_rows, int RW, int dqk, void* a, void* b, int fp16,
                             hipStream_t s) {
  const long long n = n_rows * RW;
  if (n == 0) return hipSuccess;
  const dim3 grid((unsigned)((n + 255) / 256));
  if (fp16)
    hipLaunchKernelGGL(split_cast_kernel<f16>, grid, dim3(256), 0, s, acc, n_rows, RW, dqk, static_cast<f16*>(a),
                       static_cast<f16*>(b));
  else
    hipLaunchKernelGGL(split_cast_kernel<bf16>, grid, dim3(256), 0, s, acc, n_rows, RW, dqk, static_cast<bf16*>(a),
                       static_cast<bf16*>(b));
  return hipGetLastError();
}

}  // namespace sa
