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

template <int DQK, int DV, bool SHARED, typename E>
__global__ __launch_bounds__(kThreads) void fwd_rows_kernel(Params p, E* __restrict__ out_o,
                                                            float* __restrict__ out_lse) {
  constexpr int QS = DQK + 8;
  constexpr int VS = DV + 8;
  constexpr int PS = kNT + 8;
  constexpr int NVB = DV / 16;
  constexpr int NVB_W = (NVB + 3) / 4;
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
    for (int k0 = 0; k0 < cnt; k0 += kNT) {
      for (int c = tid; c < kNT * (DQK / 8); c += kThreads) {
        const int r = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (k0 + r < cnt) {
          const int code = sRows[k0 + r];
          const E* src = (code & kCmpFlag) ? Cg + ((size_t)(code & ~kCmpFlag) * p.Hkv + g) * DQK
                                           : Kg + ((size_t)code * p.Hkv + g) * DQK;
          v = *reinterpret_cast<const uint4*>(src + col);
        }
        *reinterpret_cast<uint4*>(&sK[r * QS + col]) = v;
      }
      if (!SHARED) {
        for (int c = tid; c < kNT * (DV / 8); c += kThreads) {
          const int r = c / (DV / 8), col = (c % (DV / 8)) * 8;
          uint4 v = make_uint4(0, 0, 0, 0);
          if (k0 + r < cnt) {
            const int code = sRows[k0 + r];
            v = *reinterpret_cast<const uint4*>(Vbase + ((size_t)code * p.Hkv + g) * DV + col);
          }
          *reinterpret_cast<uint4*>(&sV[r * VS + col]) = v;
        }
      }
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
#pragma unroll
        for (int i = 0; i < NVB_W; ++i) {
          const int cb = wv + 4 * i;
          if (cb < NVB) {
            V8 b;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) b[jj] = vt[(lq * 8 + jj) * VT + cb * 16 + l16];
            accO[i] = Elem<E>::mma32(a, b, accO[i] * al);
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
// Wave w owns heads 16w..16w+15.  Per tile of kRows rows it forms S^T =
// K Q^T (16x16x32 MFMA, K from LDS, Q resident in registers), so that each
// lane holds one head's logits for 4 consecutive rows of each 16-row block:
// with two blocks side by side that is an A operand of the 16x16x32 MFMA,
// so P = exp(S - m) feeds O += P V straight from registers.  V is the first
// 512 columns of the same LDS rows, read as B operands by transposing LDS
// reads.  The running max and sum of a
// head live in the 4 lanes of its column (log2 domain); a sink logit
// starts them at (sink, 1).  Tiles come by direct global->LDS loads, the
// next one issued while the current one is computed (two buffers: on the
// 8192-token top-2048 shape, loads issued two or three tiles ahead measured
// no faster).
namespace mla_fwd {
constexpr int kD = 576, kDV = 512;
constexpr int kKS = kD + 8;                    // LDS row stride (elements)
constexpr int kRows = 32;                      // rows per tile (a multiple of 32)
constexpr int kNB = kRows / 16;                // 16-row blocks per tile
constexpr int kHeads = 64;                     // query heads per workgroup
constexpr int kCompact = 1024;                 // positions compacted at a time
constexpr int kRowChunks = kKS / 8;            // 16-byte chunks per LDS row (the last one padding)
constexpr int kTileChunks = kRows * kRowChunks;
static_assert(kRows % 32 == 0 && kCompact % kRows == 0, "tile shape");
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
__global__ __launch_bounds__(kThreads) void fwd_mla_kernel(Params p, E* __restrict__ out_o,
                                                           float* __restrict__ out_lse) {
  using namespace mla_fwd;
  typedef typename Elem<E>::V8 V8;
  __shared__ __attribute__((aligned(16))) E sK[2][kRows * kKS];
  __shared__ int sRows[kCompact];
  __shared__ int sWave[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int row = blockIdx.x;
  const int t = row / p.Hkv, g = row - t * p.Hkv;
  const int h0 = g * p.G + blockIdx.y * kHeads + wv * 16;   // the wave's first head
  const SeqPos s = seq_pos(p, t);
  const int* irow = p.idx + (size_t)row * p.topk;
  const E* Kg = reinterpret_cast<const E*>(p.k);
  const E* Cg = reinterpret_cast<const E*>(p.cmp);
  const float sl2 = p.scale * 1.4426950408889634f;   // scale * log2(e)

  // Q of head h0 + l16, columns 32kk + 8lq .. +7 (B operand of S^T)
  V8 q[kD / 32];
  {
    const E* qrow = reinterpret_cast<const E*>(p.q) + ((size_t)t * p.Hq + h0 + l16) * kD + lq * 8;
#pragma unroll
    for (int kk = 0; kk < kD / 32; ++kk) q[kk] = *reinterpret_cast<const V8*>(qrow + kk * 32);
    // wait for Q here: the compiler does not count the direct loads below,
    // so a wait for Q inside the tile loop would not be one it could place
#pragma unroll
    for (int kk = 0; kk < kD / 32; ++kk) asm volatile("" ::"v"(q[kk]));
  }
  // running max (log2 units) and sum of head h0 + l16
  const bool sk = p.has_sinks;
  float m_run = sk ? p.sinks[h0 + l16] * 1.4426950408889634f : -INFINITY;
  float l_run = sk ? 1.f : 0.f;
  f32x4 acc[kDV / 16];
#pragma unroll
  for (int c = 0; c < kDV / 16; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto src_of = [&](int code) -> const E* {
    return (code & kCmpFlag) ? Cg + ((size_t)(code & ~kCmpFlag) * p.Hkv + g) * kD : Kg + ((size_t)code * p.Hkv + g) * kD;
  };
  // rows k0 .. k0 + kRows - 1 of the compacted list into `buf` by direct loads;
  // rows past cnt repeat row cnt - 1 (finite values, masked out of S), the
  // padding chunk of each LDS row repeats its first chunk
  auto issue_tile = [&](int k0, int cnt, E* buf) {
#pragma unroll
    for (int j = 0; j < (kTileChunks + kThreads - 1) / kThreads; ++j) {
      const int c0 = (j * 4 + wv) * 64;
      if (c0 < kTileChunks) {
        const int c = c0 + lane;
        if (c < kTileChunks) {
          const int r = c / kRowChunks, ch = c - r * kRowChunks;
          const E* src = src_of(sRows[min(k0 + r, cnt - 1)]) + (ch < kD / 8 ? ch : 0) * 8;
          fwd_load_lds16(src, buf + c0 * 8);
        }
      }
    }
  };
  // every wave's loads of tile it are done (the tile is complete) and tile
  // it - 1 is no longer read, so its buffer takes tile it + 1
  auto wait_tile = [&]() { asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory"); };

  const int npos = n_positions(p);
  for (int pos0 = 0; pos0 < npos; pos0 += kCompact) {
    __syncthreads();   // the previous chunk's rows and tiles are no longer read
    const int cnt =
        compact_positions(p, s, irow, pos0, min(kCompact, npos - pos0), sRows, sWave, nullptr, row_len(p, row));
    const int ntiles = (cnt + kRows - 1) / kRows;
    if (ntiles == 0) continue;
    issue_tile(0, cnt, sK[0]);
    for (int it = 0; it < ntiles; ++it) {
      const int k0 = it * kRows;
      const E* kb = sK[it & 1];
      wait_tile();
      if (it + 1 < ntiles) issue_tile(k0 + kRows, cnt, sK[(it + 1) & 1]);

      // S^T for rows k0 + 16b + 4lq + i (i < 4), head h0 + l16
      float sv[kNB][4];
#pragma unroll
      for (int b = 0; b < kNB; ++b) {
        f32x4 st = {0.f, 0.f, 0.f, 0.f};
        const E* arow = kb + (b * 16 + l16) * kKS + lq * 8;
#pragma unroll
        for (int kk = 0; kk < kD / 32; ++kk)
          st = Elem<E>::mma32(*reinterpret_cast<const V8*>(arow + kk * 32), q[kk], st);
#pragma unroll
        for (int i = 0; i < 4; ++i) sv[b][i] = (k0 + b * 16 + lq * 4 + i < cnt) ? st[i] * sl2 : -INFINITY;
      }
      // online softmax over the tile's rows (the 4 lanes of head l16)
      float mx = sv[0][0];
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sv[b][i]);
      mx = max_xor32(max_xor16(mx));
      const float m_new = fmaxf(m_run, mx);
      const float base = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - base);
      float pr[kNB][4];
      float sum = 0.f;
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pr[b][i] = __builtin_amdgcn_exp2f(sv[b][i] - base);
          sum += pr[b][i];
        }
      sum = add_xor32(add_xor16(sum));
      l_run = l_run * alpha + sum;
      m_run = m_new;
      // O rows are heads 4lq + i: their rescale factors from lanes 4lq + i
      // (skipped when no head's max moved: the factors are then exactly 1)
      if (__ballot(alpha != 1.f)) {
        f32x4 al;
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, lq * 4 + i);
#pragma unroll
        for (int c = 0; c < kDV / 16; ++c) acc[c] = acc[c] * al;
      }
      // O += P V, one 16x16x32 MFMA per 16 columns and 32 rows: k-slot
      // 8lq + j stands for row 4lq + j of the step's first 16-row block
      // (j < 4) or row 12 + 4lq + j of its second, in A (P of head l16) and
      // in B alike; B = V^T from two transposing reads (rows 16b + 4lq +
      // l16/4, columns 16c + 4(l16 % 4))
#pragma unroll
      for (int ks = 0; ks < kNB / 2; ++ks) {   // 32 rows (two 16-row blocks) per MFMA
        V8 pa;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pa[i] = (E)pr[2 * ks][i];
          pa[4 + i] = (E)pr[2 * ks + 1][i];
        }
        const E* vrow = kb + (32 * ks + lq * 4 + (l16 >> 2)) * kKS + (l16 & 3) * 4;
#pragma unroll
        for (int c = 0; c < kDV / 16; ++c) {
          const i16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((fwd_lds_i16x4*)(vrow + c * 16));
          const i16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((fwd_lds_i16x4*)(vrow + 16 * kKS + c * 16));
          const fwd_i16x8 vb = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          acc[c] = Elem<E>::mma32(pa, __builtin_bit_cast(V8, vb), acc[c]);
        }
      }
    }
  }

  // O = acc / l for heads h0 + 4lq + i; lse of head h0 + l16
  float linv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float l = __shfl(l_run, lq * 4 + i);
    linv[i] = l > 0.f ? 1.f / l : 0.f;
  }
#pragma unroll
  for (int c = 0; c < kDV / 16; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      out_o[((size_t)t * p.Hq + h0 + lq * 4 + i) * kDV + c * 16 + l16] = (E)(acc[c][i] * linv[i]);
  if (lq == 0)
    out_lse[(size_t)t * p.Hq + h0 + l16] =
        l_run > 0.f ? m_run * 0.6931471805599453f + __logf(l_run) : -INFINITY;
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
  if (p.dqk == 576 && p.dv == 512 && p.shared && p.G % mla_fwd::kHeads == 0) {
    const dim3 grid((unsigned)(p.T * p.Hkv), (unsigned)(p.G / mla_fwd::kHeads));
    if (p.fp16)
      hipLaunchKernelGGL(fwd_mla_kernel<f16>, grid, dim3(kThreads), 0, s, p, static_cast<f16*>(o), lse);
    else
      hipLaunchKernelGGL(fwd_mla_kernel<bf16>, grid, dim3(kThreads), 0, s, p, static_cast<bf16*>(o), lse);
    return hipGetLastError();
  }
  if (p.dqk == 64 && p.dv == 64) return p.shared ? launch_t<64, 64, true>(p, o, lse, s) : launch_t<64, 64, false>(p, o, lse, s);
  if (p.dqk == 128 && p.dv == 128) return p.shared ? launch_t<128, 128, true>(p, o, lse, s) : launch_t<128, 128, false>(p, o, lse, s);
  if (p.dqk == 576 && p.dv == 512) return p.shared ? launch_t<576, 512, true>(p, o, lse, s) : launch_t<576, 512, false>(p, o, lse, s);
  return hipErrorInvalidValue;
}

}  // namespace sa
