// Backward of attention over top-k-gathered KV rows: the row kernel and the
// small kernels around it (preprocess, zero fill, dSinks reduce, cast).
//
// Formulas: aclnnSparseFlashAttentionGrad, "Formula" (Phase 1: dP = dO V^T
// and dV[u] = P^T dO; Phase 2: dS = P * (dP - softmax-grad(dO, O)); Phase 3:
// dQ = dS K[u] * scale, dK[u] = dS^T Q * scale) and SparseFlashMlaGrad
// README, "Computation formula" (Stage 2: P = exp(scale Q KV^T - lse);
// Stage 3: dKV = dS^T Q scale + P^T dO, dSinks = sum of -P dP softmax(sink)).
//
// Row kernel layout: one workgroup of 4 waves owns one (token, kv head)
// row and a chunk of up to 16 of its query heads.  It compacts the row's
// selected rows into LDS, then walks them in tiles of 32 keys: gather the
// tile's K (and V) rows into LDS, S = Q K^T and dP = dO V^T on bf16 MFMA
// (16x16x32), P and dS element-wise in fp32, dQ += dS K in registers, and
// the tile's dK/dV (dKV) contributions on MFMA (16x16x16, the head sum is
// the MFMA's inner dimension) added into fp32 accumulators with atomics.
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kNT = 32;        // keys per tile
constexpr int kHC = 16;        // query heads per workgroup
constexpr int kMaxPos = 2048;  // positions compacted per pass

// ---------------------------------------------------------------------------
// D = rowsum(dO * O) per (token, head); with sinks also the row's dSinks term
// -exp(sink_h - lse) * D.  TPR threads per row, 8 elements (bf16 or fp16,
// E) per thread per step.
template <int TPR, typename E>
__global__ __launch_bounds__(kThreads) void preprocess_kernel(Params p, float* __restrict__ D,
                                                              float* __restrict__ sink_term) {
  const int rows = p.T * p.Hq;
  const int row = blockIdx.x * (kThreads / TPR) + threadIdx.x / TPR;
  const int sub = threadIdx.x % TPR;
  float acc = 0.f;
  if (row < rows) {
    const uint4* po = reinterpret_cast<const uint4*>(reinterpret_cast<const E*>(p.o) + (size_t)row * p.dv);
    const uint4* pd = reinterpret_cast<const uint4*>(reinterpret_cast<const E*>(p.dO) + (size_t)row * p.dv);
    for (int c = sub; c < p.dv / 8; c += TPR) {
      uint4 a = po[c];
      uint4 b = pd[c];
      const E* ea = reinterpret_cast<const E*>(&a);
      const E* eb = reinterpret_cast<const E*>(&b);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc += (float)ea[i] * (float)eb[i];
    }
  }
#pragma unroll
  for (int off = TPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, TPR);
  if (row < rows && sub == 0) {
    D[row] = acc;
    if (p.has_sinks) {
      const float l = p.lse[row];
      const float sk = p.sinks[row % p.Hq];
      sink_term[row] = (l > -INFINITY) ? -__expf(sk - l) * acc : 0.f;
    }
  }
}

__global__ void fill_zero_kernel(float4* __restrict__ p, size_t n4) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n4;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ void fill_zero_tail_kernel(float* __restrict__ p, size_t n) {
  size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

// dSinks[h] = sum over tokens of sink_term[t][h], in a fixed order (each
// thread a strided fp64 partial, then a fixed tree) so it is repeatable.
__global__ __launch_bounds__(kThreads) void dsinks_kernel(Params p, const float* __restrict__ sink_term,
                                                          float* __restrict__ dsinks) {
  __shared__ double part[kThreads];
  const int h = blockIdx.x;
  double acc = 0.0;
  // tokens tid, tid + 256, ... in that order; eight loads in flight at a time
  constexpr int kU = 8;
  for (int t0 = threadIdx.x; t0 < p.T; t0 += kU * kThreads) {
    float v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int t = t0 + u * kThreads;
      v[u] = t < p.T ? sink_term[(size_t)t * p.Hq + h] : 0.f;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (t0 + u * kThreads < p.T) acc += (double)v[u];
  }
  part[threadIdx.x] = acc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) dsinks[h] = (float)part[0];
}

template <typename E>
__global__ void cast_kernel(const float* __restrict__ src, E* __restrict__ dst, size_t n) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    dst[i] = (E)src[i];
}

// Softmax L1-norm outputs (SparseFlashMlaGrad README, parameter table;
// aclnnSparseLightningIndexerGradKLLoss, "Formula": the head-summed main
// attention probabilities, L1-normalised along the context).  One
// workgroup per (token, kv head) row: the head-chunk sums of every used
// position are added in chunk order (unused positions count 0 and are not
// read), each thread keeps a strided partial of the ori and of the cmp
// total, a fixed tree adds them, and a second pass writes value / total
// (0 when the total is 0).  Repeatable: no atomics, a fixed order.
__global__ __launch_bounds__(kThreads) void l1_norm_kernel(Params p, const float* __restrict__ l1, int n_hg,
                                                           float* __restrict__ ori, float* __restrict__ cmp) {
  __shared__ float red[2][kThreads];
  const int tid = threadIdx.x;
  const int row = blockIdx.x;   // (token, kv head)
  const SeqPos s = seq_pos(p, row / p.Hkv);
  const int* irow = p.idx + (size_t)row * p.topk;
  const int npos = n_positions(p);
  const int n_ori = p.select == kSelWindowCmp ? p.win_left + 1 + p.win_right : npos;
  const size_t plane = (size_t)p.T * p.Hkv * npos;
  const float* src = l1 + (size_t)row * npos;
  const int len = row_len(p, row);
  auto value = [&](int pos) {
    float v = 0.f;
    if (decode_position(p, s, irow, pos, len) >= 0)
      for (int c = 0; c < n_hg; ++c) v += src[(size_t)c * plane + pos];
    return v;
  };
  float so = 0.f, sc = 0.f;
  for (int pos = tid; pos < npos; pos += kThreads) {
    const float v = value(pos);
    if (pos < n_ori) so += v;
    else sc += v;
  }
  red[0][tid] = so;
  red[1][tid] = sc;
  __syncthreads();
  for (int w = kThreads / 2; w > 0; w >>= 1) {
    if (tid < w) {
      red[0][tid] += red[0][tid + w];
      red[1][tid] += red[1][tid + w];
    }
    __syncthreads();
  }
  const float to = red[0][0], tc = red[1][0];
  for (int pos = tid; pos < npos; pos += kThreads) {
    const float v = value(pos);
    if (pos < n_ori) ori[(size_t)row * n_ori + pos] = to > 0.f ? v / to : 0.f;
    else cmp[(size_t)row * p.topk + (pos - n_ori)] = tc > 0.f ? v / tc : 0.f;
  }
}

template <int DQK, int DV, bool SHARED, typename E>
__global__ __launch_bounds__(kThreads) void bwd_rows_kernel(Params p, BwdBuffers w) {
  typedef typename Elem<E>::V8 V8;
  typedef typename Elem<E>::V4 V4;
  constexpr int QS = DQK + 8;   // LDS row stride (elements) of Q and K tiles
  constexpr int VS = DV + 8;    // of dO and V tiles
  constexpr int PS = kNT + 8;   // of P / dS  [head][key]
  constexpr int TS = kHC + 4;   // of P^T / dS^T [key][head]
  constexpr int NQB = DQK / 16; // 16-wide column blocks of dQ / dK
  constexpr int NVB = DV / 16;
  constexpr int NQB_W = (NQB + 3) / 4;
  static_assert(DQK % 32 == 0 && DV % 32 == 0 && DV <= DQK, "head dims");

  __shared__ __attribute__((aligned(16))) E sQ[kHC * QS];
  __shared__ __attribute__((aligned(16))) E sdO[kHC * VS];
  __shared__ __attribute__((aligned(16))) E sK[kNT * QS];
  __shared__ __attribute__((aligned(16))) E sV[SHARED ? 8 : kNT * VS];
  __shared__ float sS[kHC * kNT];
  __shared__ float sdP[kHC * kNT];
  __shared__ __attribute__((aligned(16))) E sP[kHC * PS];
  __shared__ __attribute__((aligned(16))) E sdS[kHC * PS];
  __shared__ __attribute__((aligned(16))) E sPt[kNT * TS];
  __shared__ __attribute__((aligned(16))) E sdSt[kNT * TS];
  __shared__ int sRows[kMaxPos];
  __shared__ int sVpos[kMaxPos];
  __shared__ float sL[kHC], sD[kHC];
  __shared__ int sWave[4];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  const int row = w.t0 * p.Hkv + blockIdx.x;  // (token, kv head)
  const int t = row / p.Hkv, g = row - t * p.Hkv;
  const int h0 = g * p.G + blockIdx.y * kHC;  // first query head of the chunk
  const int Gc = min(kHC, p.G - blockIdx.y * kHC);
  const SeqPos s = seq_pos(p, t);
  const int* irow = p.idx + (size_t)row * p.topk;
  const E* Qg = reinterpret_cast<const E*>(p.q);
  const E* dOg = reinterpret_cast<const E*>(p.dO);
  const E* Cg = reinterpret_cast<const E*>(p.cmp);
  const E* Kbase = reinterpret_cast<const E*>(p.k);
  const E* Vbase = reinterpret_cast<const E*>(SHARED ? p.k : p.v);
  E* dQg = reinterpret_cast<E*>(w.dq);

  // Q and dO of the chunk's heads (zero rows past Gc), lse and D.
  for (int c = tid; c < kHC * (DQK / 8); c += kThreads) {
    const int h = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (h < Gc) v = *reinterpret_cast<const uint4*>(Qg + ((size_t)t * p.Hq + h0 + h) * DQK + col);
    *reinterpret_cast<uint4*>(&sQ[h * QS + col]) = v;
  }
  for (int c = tid; c < kHC * (DV / 8); c += kThreads) {
    const int h = c / (DV / 8), col = (c % (DV / 8)) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (h < Gc) v = *reinterpret_cast<const uint4*>(dOg + ((size_t)t * p.Hq + h0 + h) * DV + col);
    *reinterpret_cast<uint4*>(&sdO[h * VS + col]) = v;
  }
  if (tid < kHC) {
    const bool ok = tid < Gc;
    sL[tid] = ok ? p.lse[(size_t)t * p.Hq + h0 + tid] : INFINITY;
    sD[tid] = ok ? w.D[(size_t)t * p.Hq + h0 + tid] : 0.f;
  }

  f32x4 accQ[NQB_W];
#pragma unroll
  for (int i = 0; i < NQB_W; ++i) accQ[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int npos = n_positions(p);
  for (int pos0 = 0; pos0 < npos; pos0 += kMaxPos) {
    __syncthreads();
    const int cnt =
        compact_positions(p, s, irow, pos0, min(kMaxPos, npos - pos0), sRows, sWave, sVpos, row_len(p, row));
    for (int k0 = 0; k0 < cnt; k0 += kNT) {
      // ---- gather the tile's K (and V) rows into LDS -----------------------
      for (int c = tid; c < kNT * (DQK / 8); c += kThreads) {
        const int r = c / (DQK / 8), col = (c % (DQK / 8)) * 8;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (k0 + r < cnt) {
          const int code = sRows[k0 + r];
          const E* src = (code & kCmpFlag) ? Cg + ((size_t)(code & ~kCmpFlag) * p.Hkv + g) * DQK
                                           : Kbase + ((size_t)code * p.Hkv + g) * DQK;
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

      // ---- S = Q K^T (waves 0,1) and dP = dO V^T (waves 2,3) ---------------
      {
        const int kb = wv & 1;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (wv < 2) {
#pragma unroll 2
          for (int kk = 0; kk < DQK / 32; ++kk) {
            const V8 a = *reinterpret_cast<const V8*>(&sQ[l16 * QS + kk * 32 + lq * 8]);
            const V8 b = *reinterpret_cast<const V8*>(&sK[(kb * 16 + l16) * QS + kk * 32 + lq * 8]);
            acc = Elem<E>::mma32(a, b, acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) sS[(lq * 4 + i) * kNT + kb * 16 + l16] = acc[i];
        } else {
          const E* vt = SHARED ? sK : sV;
          constexpr int VT = SHARED ? QS : VS;
#pragma unroll 2
          for (int kk = 0; kk < DV / 32; ++kk) {
            const V8 a = *reinterpret_cast<const V8*>(&sdO[l16 * VS + kk * 32 + lq * 8]);
            const V8 b = *reinterpret_cast<const V8*>(&vt[(kb * 16 + l16) * VT + kk * 32 + lq * 8]);
            acc = Elem<E>::mma32(a, b, acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) sdP[(lq * 4 + i) * kNT + kb * 16 + l16] = acc[i];
        }
      }
      __syncthreads();

      // ---- P = exp(scale S - lse), dS = P (dP - D) --------------------------
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int e = tid * 2 + e2;
        const int h = e / kNT, j = e % kNT;
        const float l = sL[h];
        float pv = 0.f;
        if (k0 + j < cnt && l > -INFINITY) pv = __expf(sS[e] * p.scale - l);
        const float ds = pv * (sdP[e] - sD[h]);
        const E pb = (E)pv, db = (E)ds;
        sP[h * PS + j] = pb;
        sdS[h * PS + j] = db;
        if (!w.dq_only) {
          sPt[j * TS + h] = pb;
          sdSt[j * TS + h] = db;
        }
        if (w.l1) sS[e] = pv;   // fp32 P for the head sums (only this thread read sS[e])
      }
      __syncthreads();

      // ---- softmax L1-norm: sum of P over the chunk's heads per key ------
      // (heads past Gc have lse = +inf, so P = 0 there)
      if (w.l1 && tid < kNT && k0 + tid < cnt) {
        float acc = 0.f;
#pragma unroll
        for (int h = 0; h < kHC; ++h) acc += sS[h * kNT + tid];
        w.l1[((size_t)blockIdx.y * p.T * p.Hkv + row) * npos + sVpos[k0 + tid]] = acc;
      }

      // ---- dQ += dS K (column blocks split over the 4 waves) ----------------
      {
        const V8 a = *reinterpret_cast<const V8*>(&sdS[l16 * PS + lq * 8]);
#pragma unroll
        for (int i = 0; i < NQB_W; ++i) {
          const int cb = wv + 4 * i;
          if (cb < NQB) {
            V8 b;
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) b[jj] = sK[(lq * 8 + jj) * QS + cb * 16 + l16];
            accQ[i] = Elem<E>::mma32(a, b, accQ[i]);
          }
        }
      }

      // ---- dK / dV (dKV) tile contributions -> fp32 atomics -----------------
      if (!w.dq_only) {
        constexpr int NOB = SHARED ? 2 * NQB : 2 * (NQB + NVB);
        for (int ob = wv; ob < NOB; ob += 4) {
          const int kb = ob & 1;
          int cb = ob >> 1;
          const bool is_v = !SHARED && cb >= NQB;
          if (is_v) cb -= NQB;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          if (!is_v) {
            const V4 a = *reinterpret_cast<const V4*>(&sdSt[(kb * 16 + l16) * TS + lq * 4]);
            V4 b;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) b[jj] = sQ[(lq * 4 + jj) * QS + cb * 16 + l16];
            acc = Elem<E>::mma16(a, b, acc);
            acc *= p.scale;
          }
          if (is_v || (SHARED && cb < NVB)) {
            const V4 a = *reinterpret_cast<const V4*>(&sPt[(kb * 16 + l16) * TS + lq * 4]);
            V4 b;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) b[jj] = sdO[(lq * 4 + jj) * VS + cb * 16 + l16];
            acc = Elem<E>::mma16(a, b, acc);
          }
          if (w.det) {
            // one partial row per (head chunk, token row, position)
            float* part = static_cast<float*>(w.partial) +
                          (((size_t)blockIdx.y * w.Tc * p.Hkv + blockIdx.x) * w.npos) * w.RW +
                          (is_v ? DQK : 0) + cb * 16 + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = kb * 16 + lq * 4 + i;
              if (k0 + r < cnt) part[(size_t)sVpos[k0 + r] * w.RW] = acc[i];
            }
            continue;
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int r = kb * 16 + lq * 4 + i;
            if (k0 + r < cnt) {
              const int code = sRows[k0 + r];
              float* dst;
              if (is_v) {
                dst = w.acc_v + ((size_t)code * p.Hkv + g) * DV;
              } else if (code & kCmpFlag) {
                dst = w.acc_cmp + ((size_t)(code & ~kCmpFlag) * p.Hkv + g) * DQK;
              } else {
                dst = w.acc_k + ((size_t)code * p.Hkv + g) * DQK;
              }
              unsafeAtomicAdd(dst + cb * 16 + l16, acc[i]);
            }
          }
        }
      }
      __syncthreads();
    }
  }

  // ---- dQ out ------------------------------------------------------------------
#pragma unroll
  for (int i = 0; i < NQB_W; ++i) {
    const int cb = wv + 4 * i;
    if (cb < NQB) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = lq * 4 + r;
        if (h < Gc) dQg[((size_t)t * p.Hq + h0 + h) * DQK + cb * 16 + l16] = (E)(accQ[i][r] * p.scale);
      }
    }
  }
}

template <int DQK, int DV, bool SHARED>
hipError_t launch_rows_t(const Params& p, const BwdBuffers& w, hipStream_t s) {
  dim3 grid((unsigned)(w.Tc * p.Hkv), (unsigned)((p.G + kHC - 1) / kHC));
  if (p.fp16) hipLaunchKernelGGL((bwd_rows_kernel<DQK, DV, SHARED, f16>), grid, dim3(kThreads), 0, s, p, w);
  else hipLaunchKernelGGL((bwd_rows_kernel<DQK, DV, SHARED, bf16>), grid, dim3(kThreads), 0, s, p, w);
  return hipGetLastError();
}

}  // namespace

int bwd_rows_head_chunks(const Params& p) { return (p.G + kHC - 1) / kHC; }

bool bwd_rows_supported(int dqk, int dv, int shared) {
  return (dqk == 64 && dv == 64) || (dqk == 128 && dv == 128) || (dqk == 576 && dv == 512);
}

hipError_t launch_bwd_rows(const Params& p, const BwdBuffers& w, hipStream_t s) {
  if (p.dqk == 64 && p.dv == 64) return p.shared ? launch_rows_t<64, 64, true>(p, w, s) : launch_rows_t<64, 64, false>(p, w, s);
  if (p.dqk == 128 && p.dv == 128) return p.shared ? launch_rows_t<128, 128, true>(p, w, s) : launch_rows_t<128, 128, false>(p, w, s);
  if (p.dqk == 576 && p.dv == 512) return p.shared ? launch_rows_t<576, 512, true>(p, w, s) : launch_rows_t<576, 512, false>(p, w, s);
  return hipErrorInvalidValue;
}

template <typename E>
void launch_preprocess_t(const Params& p, const BwdBuffers& w, hipStream_t s) {
  const int rows = p.T * p.Hq;
  const int cpr = p.dv / 8;   // 16-byte chunks per row
  if (cpr >= 64) {
    hipLaunchKernelGGL((preprocess_kernel<64, E>), dim3((rows + 3) / 4), dim3(kThreads), 0, s, p, w.D, w.sink_term);
  } else if (cpr >= 16) {
    hipLaunchKernelGGL((preprocess_kernel<16, E>), dim3((rows + 15) / 16), dim3(kThreads), 0, s, p, w.D,
                       w.sink_term);
  } else {
    hipLaunchKernelGGL((preprocess_kernel<8, E>), dim3((rows + 31) / 32), dim3(kThreads), 0, s, p, w.D,
                       w.sink_term);
  }
}

hipError_t launch_preprocess(const Params& p, const BwdBuffers& w, hipStream_t s) {
  if (p.fp16) launch_preprocess_t<f16>(p, w, s);
  else launch_preprocess_t<bf16>(p, w, s);
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* ptr, size_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const size_t n4 = n / 4;
  if (n4) {
    const unsigned blocks = (unsigned)std::min<size_t>((n4 + 255) / 256, 8192);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, s, reinterpret_cast<float4*>(ptr), n4);
  }
  const size_t rest = n - n4 * 4;
  if (rest) hipLaunchKernelGGL(fill_zero_tail_kernel, dim3(1), dim3(64), 0, s, ptr + n4 * 4, rest);
  return hipGetLastError();
}

hipError_t launch_l1_norm(const Params& p, const float* l1, int n_hg, float* ori, float* cmp, hipStream_t s) {
  const long long rows = (long long)p.T * p.Hkv;
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(l1_norm_kernel, dim3((unsigned)rows), dim3(kThreads), 0, s, p, l1, n_hg, ori, cmp);
  return hipGetLastError();
}

hipError_t launch_dsinks(const Params& p, const BwdBuffers& w, hipStream_t s) {
  hipLaunchKernelGGL(dsinks_kernel, dim3(p.Hq), dim3(kThreads), 0, s, p, w.sink_term, w.dsinks);
  return hipGetLastError();
}

hipError_t launch_cast(const float* src, void* dst, size_t n, int fp16, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const unsigned blocks = (unsigned)std::min<size_t>((n + 255) / 256, 16384);
  if (fp16) hipLaunchKernelGGL(cast_kernel<f16>, dim3(blocks), dim3(256), 0, s, src, static_cast<f16*>(dst), n);
  else hipLaunchKernelGGL(cast_kernel<bf16>, dim3(blocks), dim3(256), 0, s, src, static_cast<bf16*>(dst), n);
  return hipGetLastError();
}

}  // namespace sa
