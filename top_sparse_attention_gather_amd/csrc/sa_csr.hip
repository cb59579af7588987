// CSR transpose of the top-k index lists on the GPU: for every key, the
// flat slot ids p = (t * Hkv + g) * K + slot that name it, ascending,
// counted from the first slot of the token range transposed (for a range
// starting at token 0, the global ids).
//
// A slot's key follows the selection rules of the backward (token: the kv
// row; block: the sequence's block; window+cmp: the cmp row) and unused or
// fully masked slots get a sentinel key that sorts last.  The order is
// produced by a stable LSD radix sort (8-bit digits) of (key, p) pairs in
// p order: per pass a digit histogram per 4096-element tile, one
// exclusive scan over the digit-major table, and a stable scatter that
// ranks equal digits inside a tile with wave ballots.  Between passes a
// pair travels as one 8-byte (key, p) element, so each scattered write is
// one store; the last pass writes only p (the entries).  Per-key counts come
// from an integer histogram and the same scan, giving row_ptr.  Everything
// is integer work, so the result is bit-exact and run-to-run identical.
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kItems = 16;
constexpr int kTile = kThreads * kItems;   // elements per radix tile
constexpr int kScanChunk = 1024;           // elements per scan block (4 per thread)

// ---------------------------------------------------------------------------
// Device-wide exclusive scan of int32 (values and totals must fit int32).

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int u = __shfl_up(v, off, 64);
    if (lane >= off) v += u;
  }
  return v;
}

// Block-wide exclusive scan of one value per thread; returns the block total.
__device__ int block_excl_scan(int v, int* excl, int* sWave) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v);
  if (lane == 63) sWave[w] = inc;
  __syncthreads();
  int off = 0, total = 0;
#pragma unroll
  for (int i = 0; i < kThreads / 64; ++i) {
    if (i < w) off += sWave[i];
    total += sWave[i];
  }
  *excl = off + inc - v;
  __syncthreads();
  return total;
}

__global__ __launch_bounds__(kThreads) void scan_sums_kernel(const int* __restrict__ in, long long n,
                                                             int* __restrict__ bsum) {
  __shared__ int sWave[4];
  const long long base = (long long)blockIdx.x * kScanChunk + threadIdx.x * 4;
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (base + i < n) s += in[base + i];
  int excl;
  const int total = block_excl_scan(s, &excl, sWave);
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// Single workgroup: exclusive scan of the block sums in place.
__global__ __launch_bounds__(kThreads) void scan_bsums_kernel(int* __restrict__ bsum, int nb) {
  __shared__ int sWave[4];
  int carry = 0;
  for (int base = 0; base < nb; base += kThreads) {
    const int i = base + threadIdx.x;
    const int v = i < nb ? bsum[i] : 0;
    int excl;
    const int total = block_excl_scan(v, &excl, sWave);
    if (i < nb) bsum[i] = carry + excl;
    carry += total;
  }
}

__global__ __launch_bounds__(kThreads) void scan_apply_kernel(const int* __restrict__ in, long long n,
                                                              const int* __restrict__ bsum,
                                                              int* __restrict__ out, long long n_out) {
  __shared__ int sWave[4];
  const long long base = (long long)blockIdx.x * kScanChunk + threadIdx.x * 4;
  int v[4], s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = base + i < n ? in[base + i] : 0;
    s += v[i];
  }
  int excl;
  block_excl_scan(s, &excl, sWave);
  int run = bsum[blockIdx.x] + excl;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (base + i < n_out) out[base + i] = run;
    run += v[i];
  }
}

// ---------------------------------------------------------------------------
// Slot keys and per-key counts.

__device__ __forceinline__ int slot_key(const Params& p, const SeqPos& s, int g, int j,
                                        const int* __restrict__ blk_base, int sentinel) {
  if (!s.active) return sentinel;
  if (p.select == kSelToken) {
    if (j < 0 || j >= s.kv_len || (p.causal && j > s.tl)) return sentinel;
    return (s.kv_base + j) * p.Hkv + g;
  }
  if (p.select == kSelBlock) {
    if (j < 0 || (long long)j * p.bs >= s.kv_len || (p.causal && (long long)j * p.bs > s.tl)) return sentinel;
    return (blk_base[s.b] + j) * p.Hkv + g;
  }
  if (j < 0 || j >= s.cmp_len || (p.causal && (long long)p.cmp_ratio * j + p.cmp_ratio - 1 > s.tl))
    return sentinel;
  return (s.cmp_base + j) * p.Hkv + g;
}

// First block id of every sequence (block mode): blk_base[b] = sum over
// c < b of ceil(len_kv(c) / bs); one thread, B is small.
__global__ void block_base_kernel(Params p, int* __restrict__ blk_base) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int acc = 0;
  for (int b = 0; b < p.B; ++b) {
    blk_base[b] = acc;
    const int len = p.layout == kLayoutBSND ? p.Skv : p.cu_kv[b + 1] - p.cu_kv[b];
    acc += (len + p.bs - 1) / p.bs;
  }
  blk_base[p.B] = acc;
}

__global__ __launch_bounds__(kThreads) void slot_keys_kernel(Params p, long long slot0, long long n,
                                                             const int* __restrict__ blk_base, int sentinel,
                                                             int* __restrict__ keys, int* __restrict__ counts) {
  const long long i = blockIdx.x * (long long)kThreads + threadIdx.x;
  if (i >= n) return;
  const long long slot = slot0 + i;
  const int row = (int)(slot / p.topk);
  const int t = row / p.Hkv, g = row - t * p.Hkv;
  const SeqPos s = seq_pos(p, t);
  const int key = (int)(slot - (long long)row * p.topk) < row_len(p, row)
                      ? slot_key(p, s, g, p.idx[slot], blk_base, sentinel)
                      : sentinel;
  keys[i] = key;
  if (key != sentinel) atomicAdd(&counts[key], 1);
}

// Same keys, with the counts first gathered in an LDS histogram (few keys:
// one global atomic per used bin and workgroup instead of one per slot).
// Each workgroup takes a contiguous range of slots.
constexpr int kHistKeys = 8192;

__global__ __launch_bounds__(kThreads) void slot_keys_hist_kernel(Params p, long long slot0, long long n,
                                                                  long long per_block, int n_keys,
                                                                  const int* __restrict__ blk_base, int sentinel,
                                                                  int* __restrict__ keys, int* __restrict__ counts) {
  __shared__ int hist[kHistKeys];
  for (int i = threadIdx.x; i < n_keys; i += kThreads) hist[i] = 0;
  __syncthreads();
  const long long i0 = blockIdx.x * per_block;
  const long long i1 = std::min(n, i0 + per_block);
  // The thread's slots are i0 + tid, i0 + tid + 256, ...: its (row, slot in
  // row) pair advances by 256 slots per step, and the row's sequence data
  // is recomputed only when the row changes.  The indices of kBatch steps
  // are loaded before any is used, so their loads overlap.
  constexpr int kBatch = 8;
  long long i = i0 + threadIdx.x;
  if (i < i1) {
    int row = (int)((slot0 + i) / p.topk);
    int sl = (int)(slot0 + i - (long long)row * p.topk);
    int cur = -1, g = 0, len = 0;
    SeqPos s;
    for (; i < i1; i += kBatch * kThreads) {
      int j[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const long long iu = i + (long long)u * kThreads;
        j[u] = iu < i1 ? p.idx[slot0 + iu] : -1;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const long long iu = i + (long long)u * kThreads;
        if (iu >= i1) break;
        if (row != cur) {
          cur = row;
          const int t = row / p.Hkv;
          g = row - t * p.Hkv;
          s = seq_pos(p, t);
          len = row_len(p, row);
        }
        const int key = sl < len ? slot_key(p, s, g, j[u], blk_base, sentinel) : sentinel;
        keys[iu] = key;
        if (key != sentinel) atomicAdd(&hist[key], 1);
        sl += kThreads;
        if (sl >= p.topk) {
          const int q = sl / p.topk;
          row += q;
          sl -= q * p.topk;
        }
      }
    }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < n_keys; k += kThreads)
    if (hist[k]) atomicAdd(&counts[k], hist[k]);
}

// ---------------------------------------------------------------------------
// LSD radix sort passes.

// keys: element i's key at keys[i * kstride] (1: the key array, 2: the
// (key, p) pair array)
__global__ __launch_bounds__(kThreads) void radix_hist_kernel(const int* __restrict__ keys, int kstride, long long n,
                                                              int shift, int nb, int* __restrict__ hist) {
  __shared__ int h[256];
  h[threadIdx.x] = 0;
  __syncthreads();
  const long long base = (long long)blockIdx.x * kTile;
  for (int r = 0; r < kItems; ++r) {
    const long long i = base + r * kThreads + threadIdx.x;
    if (i < n) atomicAdd(&h[(keys[i * kstride] >> shift) & 255], 1);
  }
  __syncthreads();
  hist[(long long)threadIdx.x * nb + blockIdx.x] = h[threadIdx.x];
}

// Stable scatter: element e = base + r * 256 + tid is ranked after every
// element of an earlier round or a lower thread with the same digit.  The
// ranks are tile-local and digit-major: the tile is first ordered in LDS
// and then written out, so the elements of one digit go to consecutive
// addresses (runs of ~kTile / 256) instead of one scattered store each.
// FIRST: the input is the key array and p = val0 + e; otherwise (key, p)
// pairs.  LAST: only p is written (to vals_out); otherwise (key, p) pairs.
// offs: the exclusively scanned digit-major histogram, 256 * nb + 1 entries
// (the last one the total), so a tile's count of digit d is the difference
// of two neighbouring entries.
template <bool FIRST, bool LAST>
__global__ __launch_bounds__(kThreads) void radix_scatter_kernel(const int* __restrict__ keys_in,
                                                                 const int2* __restrict__ pairs_in,
                                                                 long long val0, long long n, int shift, int nb,
                                                                 const int* __restrict__ offs,
                                                                 int2* __restrict__ pairs_out,
                                                                 int* __restrict__ vals_out) {
  __shared__ int cnt[256];     // next tile-local position of each digit
  __shared__ int goff[256];    // global position of the digit's run minus its tile-local start
  __shared__ int wcnt[4][256];
  __shared__ int sWave[4];
  __shared__ int2 stage[kTile];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const long long tix = (long long)tid * nb + blockIdx.x;
  const int o = offs[tix];
  int loc;
  block_excl_scan(offs[tix + 1] - o, &loc, sWave);
  cnt[tid] = loc;
  goff[tid] = o - loc;
  for (int i = 0; i < 4; ++i) wcnt[i][tid] = 0;
  __syncthreads();
  const long long base = (long long)blockIdx.x * kTile;
  const unsigned long long lt = (1ull << lane) - 1ull;
  // every round's element loaded up front, so that the loads overlap
  // instead of one round trip per round
  int2 kvs[kItems];
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const long long i = base + r * kThreads + tid;
    kvs[r] = make_int2(0, 0);
    if (i < n) kvs[r] = FIRST ? make_int2(keys_in[i], (int)(val0 + i)) : pairs_in[i];
  }
#pragma unroll
  for (int r = 0; r < kItems; ++r) {
    const long long i = base + r * kThreads + tid;
    const bool ok = i < n;
    const int key = kvs[r].x, val = kvs[r].y;
    const int d = (key >> shift) & 255;
    // lanes of this wave holding the same digit
    unsigned long long peers = __ballot(ok);
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const unsigned long long m = __ballot((d >> b) & 1);
      peers &= ((d >> b) & 1) ? m : ~m;
    }
    if (ok && (peers & lt) == 0) wcnt[w][d] = __popcll(peers);
    __syncthreads();
    if (ok) {
      int rank = cnt[d] + __popcll(peers & lt);
      for (int ww = 0; ww < w; ++ww) rank += wcnt[ww][d];
      stage[rank] = make_int2(key, val);
    }
    __syncthreads();
    cnt[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    wcnt[0][tid] = wcnt[1][tid] = wcnt[2][tid] = wcnt[3][tid] = 0;
    __syncthreads();
  }
  // the tile in digit-major order: element j of digit d goes to goff[d] + j
  const int m = (int)std::min<long long>(kTile, n - base);
  for (int j = tid; j < m; j += kThreads) {
    const int2 kv = stage[j];
    const int pos = goff[(kv.x >> shift) & 255] + j;
    if (LAST) vals_out[pos] = kv.y;
    else pairs_out[pos] = kv;
  }
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

int csr_sentinel_bits(long long n_keys) {
  int bits = 1;
  while ((1LL << bits) <= n_keys) ++bits;
  return bits;
}

// 8-bit LSD passes that cover every key and the sentinel (n_keys)
int csr_passes(long long n_keys) { return (csr_sentinel_bits(n_keys) + 7) / 8; }

// Workspace: the slot keys, one (key, p) pair buffer (two from the third
// pass on), the per-key counts, the digit histograms and the scan sums.
struct CsrWs {
  int* keys;
  int2 *pairs_a, *pairs_b;
  int *counts, *hist, *bsum;
  long long nb_tiles, nb_scan;
};

CsrWs carve(void* ws, long long n, long long n_keys) {
  CsrWs c;
  char* p = static_cast<char*>(ws);
  c.nb_tiles = (n + kTile - 1) / kTile;
  const long long hist_n = 256 * c.nb_tiles + 1;   // + the total
  const long long scan_n = std::max(hist_n, n_keys + 1);
  c.nb_scan = (scan_n + kScanChunk - 1) / kScanChunk;
  c.keys = reinterpret_cast<int*>(p); p += align256(n * 4);
  c.pairs_a = reinterpret_cast<int2*>(p); p += align256(n * 8);
  c.pairs_b = nullptr;
  if (csr_passes(n_keys) > 2) {
    c.pairs_b = reinterpret_cast<int2*>(p);
    p += align256(n * 8);
  }
  c.counts = reinterpret_cast<int*>(p); p += align256((n_keys + 1) * 4);
  c.hist = reinterpret_cast<int*>(p); p += align256(hist_n * 4);
  c.bsum = reinterpret_cast<int*>(p); p += align256(c.nb_scan * 4);
  return c;
}

hipError_t scan_excl(const int* in, long long n, int* out, long long n_out, int* bsum, hipStream_t s) {
  const long long nb = (std::max(n, n_out) + kScanChunk - 1) / kScanChunk;
  hipLaunchKernelGGL(scan_sums_kernel, dim3((unsigned)nb), dim3(kThreads), 0, s, in, n, bsum);
  hipLaunchKernelGGL(scan_bsums_kernel, dim3(1), dim3(kThreads), 0, s, bsum, (int)nb);
  hipLaunchKernelGGL(scan_apply_kernel, dim3((unsigned)nb), dim3(kThreads), 0, s, in, n, bsum, out, n_out);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_scan_excl(const int* in, long long n, int* out, long long n_out, int* bsum, hipStream_t s) {
  return scan_excl(in, n, out, n_out, bsum, s);
}

long long scan_bsum_ints(long long n) { return (n + kScanChunk - 1) / kScanChunk; }

size_t csr_workspace_bytes(long long n, long long n_keys, int batch) {
  const long long nb_tiles = (n + kTile - 1) / kTile;
  const long long hist_n = 256 * nb_tiles + 1;
  const long long scan_n = std::max(hist_n, n_keys + 1);
  const long long nb_scan = (scan_n + kScanChunk - 1) / kScanChunk;
  return align256(n * 4) + align256(n * 8) * (csr_passes(n_keys) > 2 ? 2 : 1) + align256((n_keys + 1) * 4) +
         align256(hist_n * 4) + align256(nb_scan * 4) + align256((size_t)(batch + 1) * 4);
}

hipError_t launch_block_base(const Params& p, int* blk_base, hipStream_t s) {
  hipLaunchKernelGGL(block_base_kernel, dim3(1), dim3(64), 0, s, p, blk_base);
  return hipGetLastError();
}

hipError_t launch_csr_transpose(const Params& p, int t0, int t1, long long n_keys, const int* blk_base,
                                int* row_ptr, int* entries, void* ws, hipStream_t s) {
  const long long slot0 = (long long)t0 * p.Hkv * p.topk;
  const long long n = (long long)(t1 - t0) * p.Hkv * p.topk;
  CsrWs c = carve(ws, n, n_keys);
  const int sentinel = (int)n_keys;
  hipError_t e;
  if ((e = launch_fill_zero(reinterpret_cast<float*>(c.counts), (size_t)(n_keys + 1), s)) != hipSuccess) return e;
  if (n > 0 && n_keys <= kHistKeys) {
    // about 512 workgroups, each with a contiguous slot range
    const long long per = std::max<long long>(kThreads, (n + 511) / 512);
    const unsigned nb = (unsigned)((n + per - 1) / per);
    hipLaunchKernelGGL(slot_keys_hist_kernel, dim3(nb), dim3(kThreads), 0, s, p, slot0, n, per, (int)n_keys, blk_base,
                       sentinel, c.keys, c.counts);
  } else if (n > 0) {
    hipLaunchKernelGGL(slot_keys_kernel, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s, p,
                       slot0, n, blk_base, sentinel, c.keys, c.counts);
  }
  if ((e = scan_excl(c.counts, n_keys, row_ptr, n_keys + 1, c.bsum, s)) != hipSuccess) return e;
  if (n == 0) return hipGetLastError();
  const int passes = csr_passes(n_keys);
  const int nb = (int)c.nb_tiles;
  // pass 0 reads the key array; later passes read the pair buffer the
  // previous pass wrote (pairs_a, pairs_b alternating); the last pass
  // writes only the slot ids, into `entries`
  const int2* pin = nullptr;
  for (int pass = 0; pass < passes; ++pass) {
    const bool first = pass == 0, last = pass == passes - 1;
    int2* pout = (pass % 2 == 0) ? c.pairs_a : c.pairs_b;
    const int* hkeys = first ? c.keys : reinterpret_cast<const int*>(pin);
    hipLaunchKernelGGL(radix_hist_kernel, dim3(nb), dim3(kThreads), 0, s, hkeys, first ? 1 : 2, n, pass * 8, nb,
                       c.hist);
    if ((e = scan_excl(c.hist, 256LL * nb, c.hist, 256LL * nb + 1, c.bsum, s)) != hipSuccess) return e;
    // entries are chunk-local slot ids (slot - slot0), so they fit int32
    // whenever the chunk's slot count does
    if (first && last)
      hipLaunchKernelGGL((radix_scatter_kernel<true, true>), dim3(nb), dim3(kThreads), 0, s, c.keys, pin, 0LL, n,
                         pass * 8, nb, c.hist, pout, entries);
    else if (first)
      hipLaunchKernelGGL((radix_scatter_kernel<true, false>), dim3(nb), dim3(kThreads), 0, s, c.keys, pin, 0LL, n,
                         pass * 8, nb, c.hist, pout, entries);
    else if (last)
      hipLaunchKernelGGL((radix_scatter_kernel<false, true>), dim3(nb), dim3(kThreads), 0, s, c.keys, pin, 0LL, n,
                         pass * 8, nb, c.hist, pout, entries);
    else
      hipLaunchKernelGGL((radix_scatter_kernel<false, false>), dim3(nb), dim3(kThreads), 0, s, c.keys, pin, 0LL, n,
                         pass * 8, nb, c.hist, pout, entries);
    pin = pout;
  }
  return hipGetLastError();
}

}  // namespace sa
