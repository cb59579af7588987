// Sparse lightning-indexer gradient with the KL loss.
//
// Formulas: aclnnSparseLightningIndexerGradKLLoss, "Formula", and the same
// steps on aclnnDenseLightningIndexerGradKLLoss, "Formulas" 1-4, over the
// top-k selected rows: index score I = W ReLU(q~ K~^T), loss =
// KL(p || softmax(I)), dI = softmax(I) - p, dW = dI ReLU(S~)^T and, with
// dS~ = W [S~ > 0] dI, dq~ = dS~ K~ and dK~ = dS~^T q~.
//
// One workgroup of 4 waves per query token; wave w owns indexer heads
// 16w..16w+15 (heads past H are zero).  The token's used slots are
// compacted into LDS, then two passes run over tiles of 32 selected rows,
// each tile's K~ rows loaded straight into LDS one tile ahead (XOR-swizzled
// 16-byte chunks):
//   pass 1: S~^T = K~ q~^T (16x16x32 MFMA, lane = head), W ReLU(S~) summed
//     over the wave's heads (DPP row sums) and over the waves (LDS) gives I
//     per row; then the softmax over the row's I, dI = s - p and the
//     token's loss, with fixed-order block reductions;
//   pass 2: S~ again; dW += dI ReLU(S~); dS~ = W [S~ > 0] dI in registers
//     -- the C layout of S~^T is the A operand of dq~ += dS~ K~ (16x16x16,
//     transposing reads of the K~ tile) -- and into an LDS exchange
//     [row][head]; dK~^T of the wave's 32 columns = q~^T dS~ over all 64
//     heads (16x16x32), written as one bf16 partial row per (token, slot)
//     (64 contiguous bytes of a row per 16-byte lane store)
//     for the deterministic key-major sum over the CSR transpose.
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kD = 128;          // indexer head dim
constexpr int kHeads = 64;       // indexer heads per workgroup (zero-padded)
constexpr int kNT = 32;          // selected rows per tile
constexpr int kNKB = kNT / 16;   // 16-row blocks per tile
constexpr int kLPW = kNT / 16;   // direct 1 KiB loads per wave per tile (4 rows each)
constexpr int kMaxPos = 2048;    // slots per token
constexpr int kXS = kHeads + 8;  // exchange row stride (elements)
static_assert(kNT % 16 == 0 && kNT <= 64, "tile rows: whole 16-row blocks, one wave sums them");

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

struct __attribute__((aligned(16))) IdxSmem {
  bf16 k[2][kNT * kD];    // K~ tiles (q~ of the 64 heads is staged here at the start)
  bf16 x[kNT * kXS];      // dS~ exchange [row][head]
  float ival[kMaxPos];    // I, then dI, per compacted position
  float ip[4][kNT];       // per-wave head sums of W ReLU(S~)
  float red[3][4];
  int rows[kMaxPos];
  int vpos[kMaxPos];
  int wave[4 * (kMaxPos / 256)];   // per-round wave counts of the compaction
};

// element offset of 16-byte chunk `chunk` of tile row r
__device__ __forceinline__ int koff(int r, int chunk) { return r * kD + ((chunk ^ (r & 15)) * 8); }

// Direct global->LDS load, 16 bytes per lane, to the wave-uniform LDS
// address `lds` (+ 16 x lane), as inline asm: the compiler models the
// builtin as a FLAT access that may touch LDS and, while one is
// outstanding, turns every LDS wait into a full drain.  The wait-count
// insertion does not see these loads; the kernel waits for them itself
// (vmcnt(0) before each tile's barrier and before the workgroup ends).  M0
// (the LDS base) is an input operand, so the compiler sets it.
__device__ __forceinline__ void load_lds16(const bf16* src, bf16* lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_void*)lds);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(base) : "memory");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

// (at most 168 registers, so three workgroups share a CU instead of two:
// 1.95 -> 1.91 ms on the 8192-token top-2048 shape, no spills)
__global__ __launch_bounds__(kThreads, 3) void idx_grad_kernel(Params p, IdxArgs a) {
  __shared__ IdxSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  // tokens in descending order: with causal selection the late tokens use
  // the most slots, so the short rows come last and fill the grid's tail
  const int t = a.t0 + (a.Tc - 1 - (int)blockIdx.x);
  const int H = a.H;
  const SeqPos s = seq_pos(p, t);
  const int* irow = p.idx + (size_t)t * p.topk;

  // ---- the token's slots and q~ of its 64 heads, all loads in flight
  // together; then the used slots compacted, and q~ via LDS into both
  // operand layouts ---------------------------------------------------------
  constexpr int kRounds = kMaxPos / 256;
  int raw[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int pos = r * 256 + tid;
    raw[r] = pos < p.topk ? position_index(p, irow, pos, 0x7fffffff) : -1;
  }
  constexpr int kQPer = kHeads * kD / 8 / kThreads;   // 16-byte pieces of q~ per thread
  uint4 qv[kQPer];
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int c = i * kThreads + tid;
    const int h = c / (kD / 8), col = (c % (kD / 8)) * 8;
    qv[i] = h < H ? *reinterpret_cast<const uint4*>(a.q + ((size_t)t * H + h) * kD + col) : make_uint4(0, 0, 0, 0);
  }
  const int hl = wv * 16 + l16;   // this lane's head in the S~^T layout
  const float wh = hl < H ? a.w[(size_t)t * H + hl] : 0.f;
  const int cnt = compact_loaded(p, s, raw, p.topk, sm.rows, sm.wave, sm.vpos);

  bf16* qs = &sm.k[0][0];
#pragma unroll
  for (int i = 0; i < kQPer; ++i) {
    const int c = i * kThreads + tid;
    const int h = c / (kD / 8), col = (c % (kD / 8)) * 8;
    *reinterpret_cast<uint4*>(qs + h * kD + col) = qv[i];
  }
  __syncthreads();
  bf16x8 QB[kD / 32];             // B operand: head hl, dims 32kk + 8lq .. +8
#pragma unroll
  for (int kk = 0; kk < kD / 32; ++kk) QB[kk] = *reinterpret_cast<const bf16x8*>(qs + hl * kD + kk * 32 + lq * 8);
  bf16x8 AT[2][2];                // A operand: column 32wv + 16cb + l16, heads 32ks + 8lq .. +8
#pragma unroll
  for (int cb = 0; cb < 2; ++cb)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int j = 0; j < 8; ++j) AT[cb][ks][j] = qs[(32 * ks + 8 * lq + j) * kD + 32 * wv + 16 * cb + l16];
  // consume wh here: its load must not stay outstanding into the tile loops,
  // where the wait for it would also wait for the tile loads in flight
  asm volatile("" ::"v"(wh));
  __syncthreads();

  const int ntiles = (cnt + kNT - 1) / kNT;
  // direct loads of tile `it` into buffer `buf`: kNT / 4 loads of 4 rows x
  // 256 B, wave w issues loads kLPW w .. kLPW w + kLPW - 1; lane: row
  // 4n + lane / 16, chunk slot lane % 16 <- chunk (lane % 16) ^ (row % 16).
  // Rows past the list reload the tile's first row (never used).
  auto gather = [&](int it, int buf) {
    const int k0 = it * kNT;
#pragma unroll
    for (int u = 0; u < kLPW; ++u) {
      const int n = wv * kLPW + u;
      const int r = n * 4 + (lane >> 4);
      const int row = sm.rows[(k0 + r < cnt) ? k0 + r : k0];
      const int ch = (lane & 15) ^ (r & 15);
      load_lds16(a.k + (size_t)row * kD + ch * 8, &sm.k[buf][n * 4 * kD]);
    }
  };
  // S~^T of the tile for the wave's heads: lane (head hl, rows 16kb + 4lq + i)
  auto scores = [&](const bf16* kt, f32x4 (&S)[kNKB]) {
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb) {
      S[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kD / 32; ++kk) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kt + koff(kb * 16 + l16, kk * 4 + lq));
        S[kb] = mfma16x16x32(kf, QB[kk], S[kb]);
      }
    }
  };

  // ---- pass 1: I per selected row ------------------------------------------
  if (ntiles > 0) gather(0, 0);
  for (int it = 0; it < ntiles; ++it) {
    const int buf = it & 1;
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    gather(it + 1 < ntiles ? it + 1 : 0, buf ^ 1);   // next tile, or pass 2's first
    f32x4 S[kNKB];
    scores(sm.k[buf], S);
    const int i = l16 & 3;
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb) {
      float hs[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) hs[r] = row16_sum(wh * fmaxf(S[kb][r], 0.f));
      // lanes with l16 % 4 == r store row 4lq + r (equal values, no branch)
      sm.ip[wv][kb * 16 + lq * 4 + i] = i == 0 ? hs[0] : i == 1 ? hs[1] : i == 2 ? hs[2] : hs[3];
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (tid < kNT && it * kNT + tid < cnt)   // kNT <= 64: one wave
      sm.ival[it * kNT + tid] = sm.ip[0][tid] + sm.ip[1][tid] + sm.ip[2][tid] + sm.ip[3][tid];
  }
  __syncthreads();

  // ---- softmax over the selected rows, dI = s - p, the token's loss --------
  float m = -INFINITY;
  for (int j = tid; j < cnt; j += kThreads) m = fmaxf(m, sm.ival[j]);
  m = wave_max(m);
  if (lane == 0) sm.red[0][wv] = m;
  __syncthreads();
  const float mx = fmaxf(fmaxf(sm.red[0][0], sm.red[0][1]), fmaxf(sm.red[0][2], sm.red[0][3]));
  float z = 0.f;
  for (int j = tid; j < cnt; j += kThreads) z += __expf(sm.ival[j] - mx);
  z = wave_sum(z);
  if (lane == 0) sm.red[1][wv] = z;
  __syncthreads();
  const float lse = mx + __logf(sm.red[1][0] + sm.red[1][1] + sm.red[1][2] + sm.red[1][3]);
  float lt = 0.f;
  for (int j = tid; j < cnt; j += kThreads) {
    const float ls = sm.ival[j] - lse;   // log softmax
    const float pj = a.target[(size_t)t * p.topk + sm.vpos[j]];
    if (pj > 0.f) lt += pj * (__logf(pj) - ls);
    sm.ival[j] = __expf(ls) - pj;
  }
  lt = wave_sum(lt);
  if (lane == 0) sm.red[2][wv] = lt;
  __syncthreads();
  if (tid == 0) a.loss_tok[t] = sm.red[2][0] + sm.red[2][1] + sm.red[2][2] + sm.red[2][3];

  // ---- pass 2: dW, dq~, dK~ partial rows -------------------------------------
  f32x4 dQ[kD / 16];
#pragma unroll
  for (int c = 0; c < kD / 16; ++c) dQ[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  float accW = 0.f;
  bf16* part_tok = a.part + (size_t)(t - a.t0) * p.topk * kD;
  const int tq = l16 & 3;
  auto pk2 = [](float x, float y) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, bf16x2{(bf16)x, (bf16)y});
  };
  for (int it = 0; it < ntiles; ++it) {
    const int buf = (ntiles + it) & 1;
    const int k0 = it * kNT;
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (it + 1 < ntiles) gather(it + 1, buf ^ 1);
    const bf16* kt = sm.k[buf];
    f32x4 S[kNKB];
    scores(kt, S);
    i16x4 dSa[kNKB];
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = kb * 16 + lq * 4 + r;
        const bool v = k0 + key < cnt;
        const float dI = sm.ival[v ? k0 + key : 0];
        const float dIv = v ? dI : 0.f;
        const float sv = S[kb][r];
        accW += dIv * fmaxf(sv, 0.f);
        const bf16 db = (bf16)(sv > 0.f ? wh * dIv : 0.f);
        dSa[kb][r] = bf16_bits(db);
        sm.x[key * kXS + hl] = db;
      }
    }
    // dq~ += dS~ K~: lane (heads 4lq + i of the wave, column 16c + l16)
#pragma unroll
    for (int c = 0; c < kD / 16; ++c) {
#pragma unroll
      for (int kb = 0; kb < kNKB; ++kb) {
        const int rt = kb * 16 + lq * 4 + (l16 >> 2);
        const int ch = c * 2 + (tq >> 1);
        const i16x4 kf = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(kt + rt * kD + ((ch ^ (rt & 15)) * 8) + (tq & 1) * 4));
        dQ[c] = mfma16x16x16(dSa[kb], kf, dQ[c]);
      }
    }
    // exchange written
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // dK~^T[32wv + 16cb + 4lq + i][row 16kb + l16] over all 64 heads
#pragma unroll
    for (int kb = 0; kb < kNKB; ++kb) {
      const int key = kb * 16 + l16;
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(&sm.x[key * kXS + lq * 8]);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(&sm.x[key * kXS + 32 + lq * 8]);
      const bool v = k0 + key < cnt;
      bf16* rowp = v ? part_tok + (size_t)sm.vpos[v ? k0 + key : 0] * kD : a.dump;
      f32x4 acc[2];
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) {
        acc[cb] = mfma16x16x32(AT[cb][0], b0, f32x4{0.f, 0.f, 0.f, 0.f});
        acc[cb] = mfma16x16x32(AT[cb][1], b1, acc[cb]);
      }
      // lane (key l16, lq) holds columns 16cb + 4lq .. +3 of both blocks;
      // after swapping halves with the neighbouring 16-lane row it holds 8
      // contiguous columns (lq even: block 0 from 4lq, lq odd: block 1 from
      // 4(lq - 1)), so one 16-byte store per lane writes 64 contiguous bytes
      // of each row
      const auto s0 = __builtin_amdgcn_permlane16_swap(pk2(acc[0][0], acc[0][1]), pk2(acc[1][0], acc[1][1]), false, false);
      const auto s1 = __builtin_amdgcn_permlane16_swap(pk2(acc[0][2], acc[0][3]), pk2(acc[1][2], acc[1][3]), false, false);
      const uint4 o = {s0[0], s1[0], s0[1], s1[1]};
      *reinterpret_cast<uint4*>(rowp + 32 * wv + (lq & 1) * 16 + (lq >> 1) * 8) = o;
    }
  }
  // no direct load may still be writing this workgroup's LDS when it ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- dq~ and dW out --------------------------------------------------------
#pragma unroll
  for (int c = 0; c < kD / 16; ++c) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int h = wv * 16 + lq * 4 + r;
      if (h < H) a.dq[((size_t)t * H + h) * kD + c * 16 + l16] = (bf16)dQ[c][r];
    }
  }
  accW += __shfl_xor(accW, 16, 64);
  accW += __shfl_xor(accW, 32, 64);
  if (lq == 0 && hl < H) a.dw[(size_t)t * H + hl] = accW;
}

}  // namespace

bool idx_grad_supported(const Params& p) {
  return p.dqk == kD && p.Hq >= 1 && p.Hq <= kHeads && p.Hkv == 1 && p.topk >= 1 && p.topk <= kMaxPos &&
         p.select == kSelToken;
}

hipError_t launch_idx_grad(const Params& p, const IdxArgs& a, hipStream_t s) {
  if (a.Tc <= 0) return hipSuccess;
  hipLaunchKernelGGL(idx_grad_kernel, dim3((unsigned)a.Tc), dim3(kThreads), 0, s, p, a);
  return hipGetLastError();
}

}  // namespace sa
