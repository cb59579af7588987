// Device-side types and helpers shared by the gfx950 kernels of the
// sparse-attention library.  Only included by the library's .hip files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace sa {

constexpr int kSelToken = 0;
constexpr int kSelBlock = 1;
constexpr int kSelWindowCmp = 2;
constexpr int kLayoutBSND = 0;
constexpr int kLayoutTND = 1;

// A selected row is encoded as its global row index; rows of cmp_kv carry
// this flag; -1 marks an unused position.
constexpr int kCmpFlag = 1 << 30;

// Problem description handed to every kernel by value.  Element strides:
// q/dq [T][Hq][dqk], o/dO [T][Hq][dv], k [rows][Hkv][dqk], v [rows][Hkv][dv],
// cmp [cmp_rows][Hkv][dqk], lse/D [T][Hq], idx [T][Hkv][topk].
struct Params {
  int T, Hq, Hkv, G, dqk, dv, topk, bs, select, causal, win_left, win_right, cmp_ratio;
  int has_sinks, shared, layout, B, Sq, Skv;
  int fp16;            // 1: the 16-bit tensors (q, k, v, cmp, o, dO, gradients) are fp16, else bf16
  float scale;
  const bf16* q;
  const bf16* k;      // K rows, or the shared KV rows
  const bf16* v;      // separate V rows (null when shared)
  const bf16* cmp;    // cmp_kv rows (window+cmp)
  const bf16* o;
  const bf16* dO;
  const float* lse;
  const float* sinks;
  const int* idx;
  const int* cu_q;
  const int* cu_kv;
  const int* cu_cmp;
  const int* topk_len;   // [T][Hkv] selectable slots per row, or null (all topk)
  // [B] query / kv / cmp rows of each sequence that take part (the rest is
  // padding), or null (all of them)
  const int* used_q;
  const int* used_kv;
  const int* used_cmp;
};

// Rows of sequence b: first query row and the query rows taking part,
// first kv row and the kv rows taking part, and the key position of query
// 0 -- 0, or kv_len - q_len when the mask aligns the sequences' ends
// (causal = 2).
struct SeqLens {
  int q_base, q_len, kv_base, kv_len, off;
};

__device__ __forceinline__ SeqLens seq_lens(const Params& p, int b) {
  SeqLens L;
  if (p.layout == kLayoutBSND) {
    L.q_base = b * p.Sq;
    L.q_len = p.Sq;
    L.kv_base = b * p.Skv;
    L.kv_len = p.Skv;
  } else {
    L.q_base = p.cu_q[b];
    L.q_len = p.cu_q[b + 1] - p.cu_q[b];
    L.kv_base = p.cu_kv[b];
    L.kv_len = p.cu_kv[b + 1] - p.cu_kv[b];
  }
  if (p.used_q) L.q_len = min(L.q_len, max(p.used_q[b], 0));
  if (p.used_kv) L.kv_len = min(L.kv_len, max(p.used_kv[b], 0));
  L.off = p.causal == 2 ? L.kv_len - L.q_len : 0;
  return L;
}

// Where a query token sits: its sequence, its position in key coordinates
// (tl: the local index, shifted by the sequence's offset when the mask
// aligns the ends), whether it takes part (not a padding row), and the
// first row / used row count of its sequence in the kv and cmp tables.
struct SeqPos {
  int b, tl, kv_base, kv_len, cmp_base, cmp_len, active;
};

__device__ __forceinline__ SeqPos seq_pos(const Params& p, int t) {
  SeqPos s;
  if (p.layout == kLayoutBSND) {
    s.b = t / p.Sq;
  } else {
    int lo = 0, hi = p.B;           // largest b with cu_q[b] <= t
    while (hi - lo > 1) {
      int mid = (lo + hi) >> 1;
      if (p.cu_q[mid] <= t) lo = mid; else hi = mid;
    }
    s.b = lo;
  }
  const SeqLens L = seq_lens(p, s.b);
  const int i = t - L.q_base;
  s.active = i < L.q_len;
  s.tl = i + L.off;
  s.kv_base = L.kv_base;
  s.kv_len = L.kv_len;
  if (p.select == kSelWindowCmp && p.cu_cmp) {   // no cmp table without index slots
    s.cmp_base = p.cu_cmp[s.b];
    s.cmp_len = p.cu_cmp[s.b + 1] - p.cu_cmp[s.b];
    if (p.used_cmp) s.cmp_len = min(s.cmp_len, max(p.used_cmp[s.b], 0));
  } else {
    s.cmp_base = 0;
    s.cmp_len = 0;
  }
  return s;
}

// Selectable index slots of row (token, kv head) = t * Hkv + g: all topk,
// or the caller's per-row length clamped to [0, topk] (slots at or past it
// are unused).
__device__ __forceinline__ int row_len(const Params& p, int row) {
  if (!p.topk_len) return p.topk;
  return min(max(p.topk_len[row], 0), p.topk);
}

// Number of virtual positions of a (token, kv head) row before masking:
// index slots (token), slots * block_size rows (block), or the window
// followed by the cmp slots (window+cmp).
__device__ __forceinline__ int n_positions(const Params& p) {
  if (p.select == kSelToken) return p.topk;
  if (p.select == kSelBlock) return p.topk * p.bs;
  return p.win_left + 1 + p.win_right + p.topk;
}

// The index slot that virtual position `pos` reads, loaded (-1 where it
// reads none: a window position, or a slot at or past `len`).  It depends
// on nothing of the query's sequence, so the loads of a row's positions can
// be issued before anything else is known about the row.
__device__ __forceinline__ int position_index(const Params& p, const int* __restrict__ irow, int pos, int len) {
  if (p.select == kSelToken) return pos < len ? irow[pos] : -1;
  if (p.select == kSelBlock) {
    const int slot = pos / p.bs;
    return slot < len ? irow[slot] : -1;
  }
  const int q = pos - (p.win_left + 1 + p.win_right);
  return q >= 0 && q < len ? irow[q] : -1;
}

// Decode virtual position `pos` of row (t, g) from its loaded index `raw`
// (position_index): the encoded selected row, or -1 when the slot is unused
// or masked.
__device__ __forceinline__ int decode_loaded(const Params& p, const SeqPos& s, int pos, int raw) {
  if (!s.active) return -1;   // a padding query row selects nothing
  if (p.select == kSelToken) {
    const int j = raw;
    if (j < 0 || j >= s.kv_len || (p.causal && j > s.tl)) return -1;
    return s.kv_base + j;
  }
  if (p.select == kSelBlock) {
    if (raw < 0) return -1;
    const long long j = (long long)raw * p.bs + (pos - (pos / p.bs) * p.bs);
    if (j >= s.kv_len || (p.causal && j > s.tl)) return -1;
    return s.kv_base + (int)j;
  }
  const int nwin = p.win_left + 1 + p.win_right;
  if (pos < nwin) {
    const int j = s.tl - p.win_left + pos;
    if (j < 0 || j >= s.kv_len || (p.causal && j > s.tl)) return -1;
    return s.kv_base + j;
  }
  const int j = raw;
  if (j < 0 || j >= s.cmp_len) return -1;
  if (p.causal && (long long)p.cmp_ratio * j + p.cmp_ratio - 1 > s.tl) return -1;
  return (s.cmp_base + j) | kCmpFlag;
}

// Decode virtual position `pos` of row (t, g).  `irow` points at
// idx[t][g][0]; `len` is the row's selectable slot count (row_len).
__device__ __forceinline__ int decode_position(const Params& p, const SeqPos& s,
                                               const int* __restrict__ irow, int pos, int len = 0x7fffffff) {
  return decode_loaded(p, s, pos, position_index(p, irow, pos, len));
}

// Compact positions [pos0, pos0 + n) of a row into sRows, keeping position
// order; returns the number of used positions (the same in every thread).
// Block of 256 threads (4 waves); sWave holds 4 ints.  With sVpos, also
// stores each used position's index.  Ends with a barrier.
__device__ __forceinline__ int compact_positions(const Params& p, const SeqPos& s,
                                                 const int* __restrict__ irow, int pos0, int n,
                                                 int* sRows, int* sWave, int* sVpos = nullptr,
                                                 int len = 0x7fffffff) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int total = 0;
  for (int base = 0; base < n; base += 256) {
    const int pos = base + tid;
    int code = -1;
    if (pos < n) code = decode_position(p, s, irow, pos0 + pos, len);
    const unsigned long long m = __ballot(code >= 0);
    const int before = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) sWave[w] = __popcll(m);
    __syncthreads();
    int off = total;
    for (int i = 0; i < w; ++i) off += sWave[i];
    if (code >= 0) {
      sRows[off + before] = code;
      if (sVpos) sVpos[off + before] = pos0 + pos;
    }
    total += sWave[0] + sWave[1] + sWave[2] + sWave[3];
    __syncthreads();
  }
  return total;
}

// Same result as compact_positions for positions [pos0, pos0 + n), n <=
// 256 * ROUNDS, from indices the caller has already loaded -- raw[r] is
// position_index of position pos0 + 256 r + tid (-1 past n) -- so that
// their loads can be in flight with the caller's others.  One barrier for
// all rounds instead of two per round: each wave ballots its ROUNDS rounds
// and publishes the counts (sCnt holds 4 ROUNDS ints), and a used
// position's slot is the number of used positions before it in (round,
// wave, lane) order, i.e. in position order.  sVpos receives the positions
// themselves.  The barriers are LDS-only (the caller's loads may stay in
// flight); ends with one.
template <int ROUNDS>
__device__ __forceinline__ int compact_loaded(const Params& p, const SeqPos& s, const int (&raw)[ROUNDS], int n,
                                              int* sRows, int* sCnt, int* sVpos, int pos0 = 0) {
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  int code[ROUNDS];
  unsigned long long m[ROUNDS];
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int pos = r * 256 + tid;
    code[r] = pos < n ? decode_loaded(p, s, pos0 + pos, raw[r]) : -1;
    m[r] = __ballot(code[r] >= 0);
  }
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r)
    if (lane == r) sCnt[r * 4 + w] = __popcll(m[r]);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  int total = 0;
#pragma unroll
  for (int r = 0; r < ROUNDS; ++r) {
    const int c0 = sCnt[r * 4], c1 = sCnt[r * 4 + 1], c2 = sCnt[r * 4 + 2], c3 = sCnt[r * 4 + 3];
    const int off = total + (w > 0 ? c0 : 0) + (w > 1 ? c1 : 0) + (w > 2 ? c2 : 0) +
                    __popcll(m[r] & ((1ull << lane) - 1ull));
    if (code[r] >= 0) {
      sRows[off] = code[r];
      sVpos[off] = pos0 + r * 256 + tid;
    }
    total += c0 + c1 + c2 + c3;
  }
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  return total;
}

__device__ __forceinline__ f32x4 mfma16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma16x16x16(const i16x4& a, const i16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32x32x16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ short bf16_bits(bf16 x) { return __builtin_bit_cast(short, x); }

// The two 16-bit input formats: 8- and 4-element operand vectors and the
// 16x16x32 / 16x16x16 MFMA products (fp32 accumulate) on each.
template <typename E>
struct Elem;

template <>
struct Elem<bf16> {
  typedef bf16x8 V8;
  typedef bf16x4 V4;
  __device__ static f32x4 mma32(const V8& a, const V8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static f32x4 mma16(const V4& a, const V4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                      0, 0, 0);
  }
};

template <>
struct Elem<f16> {
  typedef f16x8 V8;
  typedef f16x4 V4;
  __device__ static f32x4 mma32(const V8& a, const V8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  __device__ static f32x4 mma16(const V4& a, const V4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
  }
};

// Sum over each row of 16 lanes, the result in all 16 (DPP: swap
// neighbours, swap pairs, mirror within 8, mirror within 16).  Every lane
// of a row ends with the same bits: each step adds two operands whose
// order differs between lanes only by commutation.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);    // quad_perm [1, 0, 3, 2]
  v += dpp_f32<0x4E>(v);    // quad_perm [2, 3, 0, 1]
  v += dpp_f32<0x141>(v);   // row_half_mirror
  v += dpp_f32<0x140>(v);   // row_mirror
  return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace sa
