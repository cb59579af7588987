// Selected-attention forward: O = softmax(scale q K_sel^T [, sink]) V_sel and
// lse = log-sum-exp of the same logits (aclnnNsaSelectedAttentionInfer,
// "Formula"; the lse output named in the SparseFlashMlaGrad parameter table).
//
// One workgroup of 4 waves owns one (token, kv head) row and up to 16 of its
// query heads, compacts the row's selected rows into LDS and walks them in
// tiles of 32 keys with an online softmax: S = Q K^T on MFMA (bf16 or fp16), running
// max / sum per head in LDS, O += P V on MFMA with the fp32 accumulator in
// registers.  A sink logit enters as the initial running max with sum 1.
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kNT = 32;
constexpr int kHC = 16;
constexpr int kMaxPos = 2048;

typedef __attribute__((address_space(3))) i16x4 gen_lds_i16x4;

template <int DQK, int DV, bool SHARED, typename E>
__global__ __launch_bounds__(kThreads) void fwd_rows_kernel(Params p, E* __restrict__ out_o,
                                                            float* __restrict__ out_lse) {
  constexpr int QS = DQK + 8;
  constexpr int VS = DV + 8;
  constexpr int PS = kNT + 8;
  constexpr int NVB = DV / 16;
  constexpr int NVB_W = (NVB + 3) / 4;
  // 16-byte chunks of a tile's K (V) rows per thread
  constexpr int CK = (kNT * (DQK / 8) + kThreads - 1) / kThreads;
  constexpr int CV = SHARED ? 0 : (kNT * (DV / 8) + kThreads - 1) / kThreads;
  constexpr int CVA = CV > 0 ? CV : 1;   // register array size
  static_assert(DQK % 32 == 0 && DV % 32 == 0 && DV <= DQK, "head dims");

  typedef typename Elem<E>::V8 V8;
  __shared__ __attribute__((aligned(16))) E sQ[kHC * QS];
  __shared__ __attribute__((aligned(16))) E sK[kNT * QS];
  __shared__ __attribute__((aligned(16))) E sV[SHARED ? 8 : kNT * VS];
  __shared__ float sS[kHC * kNT];
  __shared__ __attribute__((aligned(16))) E sP[kHC * PS];
  __shared__ float sM[kHC], sL[kHC], sAlpha[kHC];
  __shared__ int sRows[kMaxPos];
  __shared__ int sWave[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int row = blockIdx.x;
  const int t = row / p.Hkv, g = row - t * p.Hkv;
  const int h0 = g * p.G + blockIdx.y * kHC;
  const int Gc = min(kHC, p.G - blockIdx.y * kHC);
  const SeqPos s = seq_pos(p, t);
  const int* irow = p.idx + (size_t)row * p.topk;
  const E* Qg = reinterpret_cast<const E*>(p.q);
  const E* Kg = reinterpret_cast<const E*>(p.k);
  const E* Cg = reinterpret_cast<const E*>(p.cmp);
  const E* Vbase = reinterpret_cast<const E*>(SHARED ? p.k : p.v);

  for (int c = tid; c < kHC * (DQK / 8); c += kThreads) {
    const int h = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (h < Gc) v = *reinterpret_cast<const uint4*>(Qg + ((size_t)t * p.Hq + h0 + h) * DQK + col);
    *reinterpret_cast<uint4*>(&sQ[h * QS + col]) = v;
  }
  if (tid < kHC) {
    // running max and sum; a sink logit starts them at (sink, 1)
    const bool sk = p.has_sinks && tid < Gc;
    sM[tid] = sk ? p.sinks[h0 + tid] : -INFINITY;
    sL[tid] = sk ? 1.f : 0.f;
  }

  f32x4 accO[NVB_W];
#pragma unroll
  for (int i = 0; i < NVB_W; ++i) accO[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int npos = n_positions(p);
  for (int pos0 = 0; pos0 < npos; pos0 += kMaxPos) {
    __syncthreads();
    const int cnt =
        compact_positions(p, s, irow, pos0, min(kMaxPos, npos - pos0), sRows, sWave, nullptr, row_len(p, row));
    // the tile's K (and V) rows are loaded into registers one tile ahead,
    // while the previous tile is computed, and written to LDS at the top of
    // its own iteration (rows past cnt are zero)
    uint4 kreg[CK], vreg[CVA];
    auto load_tile = [&](int k0) {
#pragma unroll
      for (int j = 0; j < CK; ++j) {
        const int c = tid + j * kThreads;
        const int r = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
        kreg[j] = make_uint4(0, 0, 0, 0);
        if (c < kNT * (DQK / 8) && k0 + r < cnt) {
          const int code = sRows[k0 + r];
          const E* src = (code & kCmpFlag) ? Cg + ((size_t)(code & ~kCmpFlag) * p.Hkv + g) * DQK
                                           : Kg + ((size_t)code * p.Hkv + g) * DQK;
          kreg[j] = *reinterpret_cast<const uint4*>(src + col);
        }
      }
#pragma unroll
      for (int j = 0; j < CV; ++j) {
        const int c = tid + j * kThreads;
        const int r = c / (DV / 8), col = (c % (DV / 8)) * 8;
        vreg[j] = make_uint4(0, 0, 0, 0);
        if (c < kNT * (DV / 8) && k0 + r < cnt) {
          const int code = sRows[k0 + r];
          vreg[j] = *reinterpret_cast<const uint4*>(Vbase + ((size_t)code * p.Hkv + g) * DV + col);
        }
      }
    };
    if (cnt > 0) load_tile(0);
    for (int k0 = 0; k0 < cnt; k0 += kNT) {
#pragma unroll
      for (int j = 0; j < CK; ++j) {
        const int c = tid + j * kThreads;
        if (c < kNT * (DQK / 8))
          *reinterpret_cast<uint4*>(&sK[(c / (DQK / 8)) * QS + (c % (DQK / 8)) * 8]) = kreg[j];
      }
#pragma unroll
      for (int j = 0; j < CV; ++j) {
        const int c = tid + j * kThreads;
        if (c < kNT * (DV / 8)) *reinterpret_cast<uint4*>(&sV[(c / (DV / 8)) * VS + (c % (DV / 8)) * 8]) = vreg[j];
      }
      if (k0 + kNT < cnt) load_tile(k0 + kNT);
      __syncthreads();

      if (wv < 2) {
        const int kb = wv;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 2
        for (int kk = 0; kk < DQK / 32; ++kk) {
          const V8 a = *reinterpret_cast<const V8*>(&sQ[l16 * QS + kk * 32 + lq * 8]);
          const V8 b = *reinterpret_cast<const V8*>(&sK[(kb * 16 + l16) * QS + kk * 32 + lq * 8]);
          acc = Elem<E>::mma32(a, b, acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) sS[(lq * 4 + i) * kNT + kb * 16 + l16] = acc[i];
      }
      __syncthreads();

      // online softmax: 16 threads per head, 2 keys each
      {
        const int h = tid >> 4, part = tid & 15;
        const float m_old = sM[h];
        float v0 = -INFINITY, v1 = -INFINITY;
        if (k0 + part * 2 < cnt) v0 = sS[h * kNT + part * 2] * p.scale;
        if (k0 + part * 2 + 1 < cnt) v1 = sS[h * kNT + part * 2 + 1] * p.scale;
        float mx = fmaxf(v0, v1);
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 16));
        const float m_new = fmaxf(m_old, mx);
        const float base = (m_new == -INFINITY) ? 0.f : m_new;
        const float p0 = __expf(v0 - base), p1 = __expf(v1 - base);
        float sum = p0 + p1;
#pragma unroll
        for (int off = 8; off > 0; off >>= 1) sum += __shfl_xor(sum, off, 16);
        sP[h * PS + part * 2] = (E)p0;
        sP[h * PS + part * 2 + 1] = (E)p1;
        __syncthreads();   // every thread has read sM[h] before it changes
        if (part == 0) {
          const float alpha = __expf(m_old - base);
          sAlpha[h] = alpha;
          sL[h] = sL[h] * alpha + sum;
          sM[h] = m_new;
        }
      }
      __syncthreads();

      {
        const E* vt = SHARED ? sK : sV;
        constexpr int VT = SHARED ? QS : VS;
        const V8 a = *reinterpret_cast<const V8*>(&sP[l16 * PS + lq * 8]);
        f32x4 al;
#pragma unroll
        for (int r = 0; r < 4; ++r) al[r] = sAlpha[lq * 4 + r];
        // B = V^T of 16 columns, keys 8lq .. 8lq + 7 in order: two
        // transposing reads of 4 rows each (rows 8lq + l16/4 and
        // 8lq + 4 + l16/4, columns 4(l16 % 4) of the block)
        const E* vrow = vt + (lq * 8 + (l16 >> 2)) * VT + (l16 & 3) * 4;
#pragma unroll
        for (int i = 0; i < NVB_W; ++i) {
          const int cb = wv + 4 * i;
          if (cb < NVB) {
            const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((gen_lds_i16x4*)(vrow + cb * 16));
            const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((gen_lds_i16x4*)(vrow + 4 * VT + cb * 16));
            typedef short i16x8_t __attribute__((ext_vector_type(8)));
            const i16x8_t vb = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
            accO[i] = Elem<E>::mma32(a, __builtin_bit_cast(V8, vb), accO[i] * al);
          }
        }
      }
      __syncthreads();
    }
  }

#pragma unroll
  for (int i = 0; i < NVB_W; ++i) {
    const int cb = wv + 4 * i;
    if (cb < NVB) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = lq * 4 + r;
        if (h < Gc) {
          const float l = sL[h];
          const float o = l > 0.f ? accO[i][r] / l : 0.f;
          out_o[((size_t)t * p.Hq + h0 + h) * DV + cb * 16 + l16] = (E)o;
        }
      }
    }
  }
  if (tid < Gc) {
    const float l = sL[tid];
    out_lse[(size_t)t * p.Hq + h0 + tid] = l > 0.f ? sM[tid] + __logf(l) : -INFINITY;
  }
}


// Shared-KV 576/512 forward with 64 query heads per workgroup: the selected
// rows of one (token, kv head) are gathered once for all 64 heads (the
// generic kernel above gathers them once per 16-head chunk).
//
// 12 waves in three roles, three per SIMD, pipelined over the row's tiles of
// kRows rows (three tile buffers, one barrier per stage):
//  - softmax waves 0..3, wave w with heads 16w..16w+15, at stage st:
//    S^T = K Q^T for tile st (16x16x32 MFMA, K from LDS, Q resident in
//    registers), each lane holding one head's logits for 4 rows of each
//    16-row block; the online softmax (running max and sum of a head in the
//    4 lanes of its column, log2 domain, a sink logit starting them at
//    (sink, 1)); P = exp(S - m) to an LDS exchange [head][k-slot] in the
//    row order an A operand of the 16x16x32 MFMA wants, the rescale factor
//    of each head beside it;
//  - P.V waves 4..7, wave 4 + c with O columns 128c..128c+127 of all 64
//    heads, at stage st: O = O alpha + P V for tile st - 1, with P from the
//    exchange and V^T from transposing LDS reads of the wave's columns only;
//  - loader waves 8..11: the direct global->LDS loads of tile st + 1.
// Splitting O by columns makes every V^T element read once per tile instead
// of once per 16 heads, which bounded the single-role form (each of 4 waves
// reading the whole V^T for its 16 heads: 6.3-6.5 ms on the 8192-token
// top-2048 shape: 3.2 ms split).  A direct load waits at issue while the
// CU's vector-memory path works through the loads queued before it (the 37
// of a tile keep it busy ~2200 cycles), so the waves that issue them do
// nothing else: issued by the softmax waves the loads held each stage's S^T
// back (3.2 -> 2.8 ms with loader waves).
namespace mla_fwd {
constexpr int kD = 576, kDV = 512;
constexpr int kKS = kD + 8;                    // LDS row stride (elements)
constexpr int kRows = 32;                      // rows per tile (one 16x16x32 K step of P V)
constexpr int kHeads = 64;                     // query heads per workgroup
constexpr int kWaves = 12;                     // 4 softmax waves, 4 P.V waves, 4 loader waves
constexpr int kThreadsF = kWaves * 64;
constexpr int kBufs = 3;                       // tiles in LDS: P.V reads st - 1, softmax st, loads st + 1
constexpr int kCompact = 1024;                 // positions compacted at a time
constexpr int kRowChunks = kKS / 8;            // 16-byte chunks per LDS row (the last one padding)
constexpr int kTileChunks = kRows * kRowChunks;
constexpr int kPS = kRows + 8;                 // P exchange row stride (elements)
constexpr int kColsPV = kDV / 4;               // O columns per P.V wave
static_assert(kCompact % kRows == 0, "tile shape");
}  // namespace mla_fwd

typedef __attribute__((address_space(3))) i16x4 fwd_lds_i16x4;
typedef __attribute__((address_space(3))) void fwd_lds_void;

// Direct global->LDS load of 16 bytes per lane to the wave-uniform LDS
// address `lds` + 16 x lane.  Written as inline asm because the compiler
// treats the builtin as a FLAT access that may touch LDS and would then
// drain every LDS wait; the kernel waits for these loads itself (vmcnt).
__device__ __forceinline__ void fwd_load_lds16(const void* src, void* lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(fwd_lds_void*)lds);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(base) : "memory");
}
typedef short fwd_i16x8 __attribute__((ext_vector_type(8)));

// x and its value in lane ^ 16 (resp. lane ^ 32), as a pair, by swapping a
// register with itself across 16-lane rows (resp. 32-lane halves): a VALU
// exchange instead of an LDS-routed lane shuffle.  Every lane then combines
// the same two operands (in either order).
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <typename E>
__global__ __launch_bounds__(mla_fwd::kThreadsF, 1) void fwd_mla_kernel(Params p, E* __restrict__ out_o,
                                                                       float* __restrict__ out_lse) {
  using namespace mla_fwd;
  typedef typename Elem<E>::V8 V8;
  __shared__ __attribute__((aligned(16))) E sK[kBufs][kRows * kKS];
  __shared__ __attribute__((aligned(16))) E sP[2][kHeads * kPS];   // P of a tile, [head][k-slot]
  __shared__ float sAl[2][kHeads];                                  // its rescale factor per head
  __shared__ int sFl[2][4];                                         // per head block: any factor != 1
  __shared__ float sL[kHeads];                                      // final softmax sum per head
  __shared__ int sRows[kCompact];
  __shared__ int sWave[kWaves];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  const int row = blockIdx.x;
  const int t = row / p.Hkv, g = row - t * p.Hkv;
  const int hg = g * p.G + blockIdx.y * kHeads;                     // the group's first head
  // heads of this group present (the last group may hold fewer than 64: the
  // missing ones repeat a present head's Q and are not stored)
  const int gh = min(kHeads, p.G - (int)blockIdx.y * kHeads);
  const SeqPos s = seq_pos(p, t);
  const int* irow = p.idx + (size_t)row * p.topk;
  const E* Kg = reinterpret_cast<const E*>(p.k);
  const E* Cg = reinterpret_cast<const E*>(p.cmp);
  const int npos = n_positions(p);
  const int len = row_len(p, row);

  auto src_of = [&](int code) -> const E* {
    return (code & kCmpFlag) ? Cg + ((size_t)(code & ~kCmpFlag) * p.Hkv + g) * kD : Kg + ((size_t)code * p.Hkv + g) * kD;
  };
  // positions [pos0, pos0 + n) of the row compacted into sRows over all 12
  // waves, in position order (same code and barriers in every role)
  auto compact = [&](int pos0, int n) -> int {
    int total = 0;
    for (int base = 0; base < n; base += kThreadsF) {
      const int pos = base + tid;
      const int code = pos < n ? decode_position(p, s, irow, pos0 + pos, len) : -1;
      const unsigned long long m = __ballot(code >= 0);
      const int before = __popcll(m & ((1ull << lane) - 1ull));
      if (lane == 0) sWave[wv] = __popcll(m);
      __syncthreads();
      int off = total;
      for (int i = 0; i < wv; ++i) off += sWave[i];
      if (code >= 0) sRows[off + before] = code;
      for (int i = 0; i < kWaves; ++i) total += sWave[i];
      __syncthreads();
    }
    return total;
  };
  // one barrier per stage: every loader wave's loads of the stage's tile
  // have landed, the exchange of the previous stage is written, and the
  // buffer the P.V waves read at the previous stage is free
  auto stage_barrier = [&]() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); };
  // rows k0 .. k0 + kRows - 1 of the compacted list into `buf` by direct
  // loads, issuing wave iw (of 4) taking the 64-chunk blocks iw, iw + 4, ...;
  // rows past cnt repeat row cnt - 1 (finite values, masked out of S), the
  // padding chunk of each LDS row repeats its first chunk.  All source
  // addresses come first: the loads are asm statements that the compiler
  // does not move LDS reads across, so reading each row number just before
  // its load would wait out one LDS latency per load.
  constexpr int kJ = (kTileChunks / 64 + 4) / 4;
  auto issue_tile = [&](int iw, int k0, int cnt, E* buf) {
    const E* src[kJ];
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int c = (j * 4 + iw) * 64 + lane;
      const int r = c / kRowChunks, ch = c - r * kRowChunks;
      src[j] = src_of(sRows[min(k0 + r, cnt - 1)]) + (ch < kD / 8 ? ch : 0) * 8;
    }
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int c0 = (j * 4 + iw) * 64;
      if (c0 < kTileChunks && c0 + lane < kTileChunks) fwd_load_lds16(src[j], buf + c0 * 8);
    }
  };

  if (wv < 4) {
    // ---- softmax waves: heads hg + 16 wv + l16 --------------------------
    const int hl = wv * 16 + l16;                       // the lane's head in the group
    const int hq = hg + min(hl, gh - 1);                // clamped to a present head
    const float sl2 = p.scale * 1.4426950408889634f;    // scale * log2(e)
    // Q of the lane's head, columns 32kk + 8lq .. +7 (B operand of S^T)
    V8 q[kD / 32];
    {
      const E* qrow = reinterpret_cast<const E*>(p.q) + ((size_t)t * p.Hq + hq) * kD + lq * 8;
#pragma unroll
      for (int kk = 0; kk < kD / 32; ++kk) q[kk] = *reinterpret_cast<const V8*>(qrow + kk * 32);
    }
    const bool sk = p.has_sinks;
    float m_run = sk ? p.sinks[hq] * 1.4426950408889634f : -INFINITY;
    float l_run = sk ? 1.f : 0.f;
    for (int pos0 = 0; pos0 < npos; pos0 += kCompact) {
      __syncthreads();   // the previous pass's rows and tiles are no longer read
      const int cnt = compact(pos0, min(kCompact, npos - pos0));
      const int ntiles = (cnt + kRows - 1) / kRows;
      for (int st = 0; st <= ntiles; ++st) {
        stage_barrier();
        if (st == ntiles) continue;
        const int k0 = st * kRows;
        const E* kb = sK[st % kBufs];
        // S^T for rows k0 + 16b + 4lq + i (i < 4), head hl
        float sv[2][4];
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const E* arow = kb + (b * 16 + l16) * kKS + lq * 8;
#pragma unroll
          for (int kk = 0; kk < kD / 32; ++kk)
            acc = Elem<E>::mma32(*reinterpret_cast<const V8*>(arow + kk * 32), q[kk], acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) sv[b][i] = (k0 + b * 16 + lq * 4 + i < cnt) ? acc[i] * sl2 : -INFINITY;
        }
        float mx = sv[0][0];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[b][i]);
        mx = max_xor32(max_xor16(mx));
        const float m_new = fmaxf(m_run, mx);
        const float base = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - base);
        V8 pv;
        float sum = 0.f;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pr = __builtin_amdgcn_exp2f(sv[b][i] - base);
            sum += pr;
            pv[b * 4 + i] = (E)pr;
          }
        sum = add_xor32(add_xor16(sum));
        l_run = l_run * alpha + sum;
        m_run = m_new;
        // k-slot 8lq + 4b + i of head hl holds row 16b + 4lq + i: the order
        // of the transposing V reads of the P.V waves
        *reinterpret_cast<V8*>(&sP[st & 1][hl * kPS + lq * 8]) = pv;
        if (lq == 0) sAl[st & 1][hl] = alpha;
        const bool moved = __ballot(alpha != 1.f) != 0ull;
        if (lane == 0) sFl[st & 1][wv] = moved ? 1 : 0;
      }
    }
    if (lq == 0) sL[hl] = l_run;
    __syncthreads();
    if (lq == 0 && hl < gh)
      out_lse[(size_t)t * p.Hq + hg + hl] = l_run > 0.f ? m_run * 0.6931471805599453f + __logf(l_run) : -INFINITY;
  } else if (wv >= 8) {
    // ---- loader waves: the direct loads of tile st + 1 at stage st --------
    for (int pos0 = 0; pos0 < npos; pos0 += kCompact) {
      __syncthreads();
      const int cnt = compact(pos0, min(kCompact, npos - pos0));
      const int ntiles = (cnt + kRows - 1) / kRows;
      if (ntiles > 0) issue_tile(wv - 8, 0, cnt, sK[0]);
      for (int st = 0; st <= ntiles; ++st) {
        stage_barrier();
        if (st + 1 < ntiles) issue_tile(wv - 8, (st + 1) * kRows, cnt, sK[(st + 1) % kBufs]);
      }
    }
    __syncthreads();
  } else {
    // ---- P.V waves: O columns c0 .. c0 + kColsPV - 1 of all 64 heads ------
    const int c0 = (wv - 4) * kColsPV;
    f32x4 acc[4][kColsPV / 16];
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int c = 0; c < kColsPV / 16; ++c) acc[hb][c] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int pos0 = 0; pos0 < npos; pos0 += kCompact) {
      __syncthreads();
      const int cnt = compact(pos0, min(kCompact, npos - pos0));
      const int ntiles = (cnt + kRows - 1) / kRows;
      for (int st = 0; st <= ntiles; ++st) {
        stage_barrier();
        if (st == 0) continue;
        const int ts = st - 1;                  // the tile whose P the softmax waves wrote
        const E* kb = sK[ts % kBufs];
        const E* pb = sP[ts & 1];
        // O rows are heads 16hb + 4lq + i: rescale by their factors (a
        // block whose heads' maxima did not move keeps its rows: factor 1)
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) {
          if (sFl[ts & 1][hb]) {
            f32x4 al;
#pragma unroll
            for (int i = 0; i < 4; ++i) al[i] = sAl[ts & 1][hb * 16 + lq * 4 + i];
#pragma unroll
            for (int c = 0; c < kColsPV / 16; ++c) acc[hb][c] = acc[hb][c] * al;
          }
        }
        V8 pa[4];
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) pa[hb] = *reinterpret_cast<const V8*>(&pb[(hb * 16 + l16) * kPS + lq * 8]);
        // B = V^T of 16 columns: k-slot 8lq + j is row 4lq + j (j < 4) or
        // 12 + 4lq + j, from two transposing reads (rows 4lq + l16/4 and
        // 16 + 4lq + l16/4, columns 4(l16 % 4) of the block)
        const E* vrow = kb + (lq * 4 + (l16 >> 2)) * kKS + c0 + (l16 & 3) * 4;
#pragma unroll
        for (int c = 0; c < kColsPV / 16; ++c) {
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((fwd_lds_i16x4*)(vrow + c * 16));
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((fwd_lds_i16x4*)(vrow + 16 * kKS + c * 16));
          const fwd_i16x8 vb = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int hb = 0; hb < 4; ++hb) acc[hb][c] = Elem<E>::mma32(pa[hb], __builtin_bit_cast(V8, vb), acc[hb][c]);
        }
      }
    }
    __syncthreads();   // the softmax waves' final sums are in sL
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = hb * 16 + lq * 4 + i;
        if (h >= gh) continue;
        const float l = sL[h];
        const float linv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int c = 0; c < kColsPV / 16; ++c)
          out_o[((size_t)t * p.Hq + hg + h) * kDV + c0 + c * 16 + l16] = (E)(acc[hb][c][i] * linv);
      }
  }
}

template <int DQK, int DV, bool SHARED>
hipError_t launch_t(const Params& p, void* o, float* lse, hipStream_t s) {
  dim3 grid((unsigned)(p.T * p.Hkv), (unsigned)((p.G + kHC - 1) / kHC));
  if (p.fp16)
    hipLaunchKernelGGL((fwd_rows_kernel<DQK, DV, SHARED, f16>), grid, dim3(kThreads), 0, s, p, static_cast<f16*>(o), lse);
  else
    hipLaunchKernelGGL((fwd_rows_kernel<DQK, DV, SHARED, bf16>), grid, dim3(kThreads), 0, s, p, static_cast<bf16*>(o),
                       lse);
  return hipGetLastError();
}

}  // namespace

bool fwd_rows_supported(int dqk, int dv, int shared) {
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 576 && dv == 512);
}

hipError_t launch_fwd_rows(const Params& p, void* o, float* lse, hipStream_t s) {
  // 64 heads per workgroup at any number of heads per kv head (the last
  // group's missing heads masked: one head runs in about the time of 64,
  // still below the 16-head row kernel's time for 1-15 heads)
  if (p.dqk == 576 && p.dv == 512 && p.shared) {
    const dim3 grid((unsigned)(p.T * p.Hkv), (unsigned)((p.G + mla_fwd::kHeads - 1) / mla_fwd::kHeads));
    if (p.fp16)
      hipLaunchKernelGGL(fwd_mla_kernel<f16>, grid, dim3(mla_fwd::kThreadsF), 0, s, p, static_cast<f16*>(o), lse);
    else
      hipLaunchKernelGGL(fwd_mla_kernel<bf16>, grid, dim3(mla_fwd::kThreadsF), 0, s, p, static_cast<bf16*>(o), lse);
    return hipGetLastError();
  }
  if (p.dqk == 64 && p.dv == 64) return p.shared ? launch_t<64, 64, true>(p, o, lse, s) : launch_t<64, 64, false>(p, o, lse, s);
  if (p.dqk == 128 && p.dv == 128) return p.shared ? launch_t<128, 128, true>(p, o, lse, s) : launch_t<128, 128, false>(p, o, lse, s);
  if (p.dqk == 576 && p.dv == 512) return p.shared ? launch_t<576, 512, true>(p, o, lse, s) : launch_t<576, 512, false>(p, o, lse, s);
  return hipErrorInvalidValue;
}

}  // namespace sa
