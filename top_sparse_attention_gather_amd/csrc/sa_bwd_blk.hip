// Key-major dK/dV for block selection (NSA-style block-sparse GQA).
//
// Formulas: aclnnSparseFlashAttentionGrad, "Formula": Phase 1 dV[u] = P^T dO,
// Phase 2 dS = P * (dP - softmax-grad(dO, O)), Phase 3 dK[u] = dS^T Q scale,
// with u the rows of the blocks a query's index list names; P is recomputed
// as exp(scale Q K^T - lse) (SparseFlashMlaGrad README, "Computation
// formula", Stage 2).
//
// A selected block holds block_size rows and is named by many queries, so
// instead of one partial row per (query, row) -- 1 KB of fp32 traffic per
// pair at d = 128 -- one workgroup takes a block and walks the queries that
// selected it (the CSR transpose of the index lists, in ascending slot
// order), recomputing P and dS for the block's rows and accumulating dK and
// dV in registers.  A key's list is cut into `n_split` slices (and the
// query heads into chunks of 16) so that enough workgroups exist; each
// writes its fp32 dK|dV rows to its own slice of the output buffer, and the
// slices are summed in a fixed order afterwards, so the result is bitwise
// repeatable.
//
// Workgroup: 4 waves; wave w owns block rows 16w..16w+15 (their K and V
// fragments stay in registers for the whole list).  Per query: its 16
// heads' Q and dO rows (and lse, D) are double-buffered through LDS;
// S = Q K^T and dP = dO V^T on 16x16x32 MFMA; P and dS in registers, taken
// straight from the MFMA result layout as the A operand of the 16x16x16
// MFMAs dV += P^T dO and dK += dS^T Q, whose B operands are transposing LDS
// reads of dO and Q.
#include <type_traits>

#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kHeads = 16;   // query heads per workgroup
constexpr int kPD = 8;       // queries fetched ahead (the query loop below is unrolled by kPD)
constexpr int kIds = 512;    // query token ids staged in LDS at a time

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

__device__ __forceinline__ i16x4 tr_read4(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

// f(integral_constant<int, U>) for U = B .. E-1, unrolled at compile time
template <int B, int E, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>());
    unroll<B + 1, E>(f);
  }
}

// LDS rows of the staged Q / dO (one per head): D columns, 16-byte chunk c
// of row r at slot (c + rot(r)) mod D/8, rot(r) = 2 (r % 8) + (r / 8) % 2.
// The 16 rows of a fragment read (one chunk) then take 16 distinct slots,
// and each 32-lane pass of the transposing reads (8 rows x 32 bytes) covers
// 8 disjoint 32-byte bank ranges.
template <int D>
__device__ __forceinline__ int qrow_off(int r, int col) {
  constexpr int CPR = D / 8;
  const int rot = 2 * (r & 7) + ((r >> 3) & 1);
  return r * D + (((col >> 3) + rot) & (CPR - 1)) * 8 + (col & 7);
}

template <int D>
__global__ __launch_bounds__(kThreads) void blk_dkv_kernel(Params p, BlkArgs a) {
  constexpr int QS = D;            // LDS row stride (rows rotated, see qrow_off)
  constexpr int NK = D / 32;       // 16x16x32 steps over d
  constexpr int NC = D / 16;       // 16-column blocks of dK / dV
  constexpr int CPR = D / 8;       // 16-byte chunks per head row
  __shared__ __attribute__((aligned(16))) bf16 sQ[2][kHeads * QS];
  __shared__ __attribute__((aligned(16))) bf16 sdO[2][kHeads * QS];
  __shared__ float sL[2][kHeads], sD[2][kHeads];
  __shared__ int sTok[kIds];   // tokens of the current part of the list

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int l16 = lane & 15, lq = lane >> 4;
  // chunk w of the list of block key `bkey` (chunk_base is ascending)
  const long long wch = blockIdx.x;
  const int hc = blockIdx.y;
  if (wch >= a.chunk_base[a.n_keys]) return;         // past the last chunk (uniform)
  long long bkey = 0;
  {
    long long lo = 0, hi = a.n_keys;                 // largest key with chunk_base[key] <= wch
    while (hi - lo > 1) {
      const long long mid = (lo + hi) >> 1;
      if (a.chunk_base[mid] <= wch) lo = mid; else hi = mid;
    }
    bkey = lo;
  }
  const int cidx = (int)(wch - a.chunk_base[bkey]);
  const int bn = (int)(bkey / p.Hkv), g = (int)(bkey - (long long)bn * p.Hkv);
  int b = 0;
  {
    int lo = 0, hi = p.B;                            // largest b with blk_base[b] <= bn
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (a.blk_base[mid] <= bn) lo = mid; else hi = mid;
    }
    b = lo;
  }
  const int jb = bn - a.blk_base[b];                 // block index within the sequence
  const SeqLens SL = seq_lens(p, b);
  const int kv_base = SL.kv_base;
  const int kv_len = SL.kv_len;                      // used rows
  const int q_base = SL.q_base - SL.off;             // token - q_base = key position
  const int h0 = g * p.G + hc * kHeads;
  const int Gc = min(kHeads, p.G - hc * kHeads);
  const int eb = a.row_ptr[bkey] + cidx * kBlkChunk;
  const int ee = min(a.row_ptr[bkey + 1], eb + kBlkChunk);

  // the wave's 16 block rows; this lane's row (B operand n index)
  const int r0 = wv * 16;
  const int jl = jb * p.bs + r0 + l16;               // sequence-local key row
  const bool krow_ok = r0 + l16 < p.bs && jl < kv_len;
  bf16x8 Kf[NK], Vf[NK];
  {
    const size_t off = ((size_t)(kv_base + (krow_ok ? jl : 0)) * p.Hkv + g) * D + lq * 8;
    const bf16x8 z = {};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const bf16x8 kv = *reinterpret_cast<const bf16x8*>(p.k + off + kk * 32);
      const bf16x8 vv = *reinterpret_cast<const bf16x8*>(p.v + off + kk * 32);
      Kf[kk] = krow_ok ? kv : z;
      Vf[kk] = krow_ok ? vv : z;
    }
  }
  f32x4 dK[NC], dV[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) dK[c] = dV[c] = f32x4{0.f, 0.f, 0.f, 0.f};

  // staging of one query's rows: token t, heads h0..h0+Gc-1 (rows past Gc
  // are zero, with lse = +inf so that their P is 0)
  // queries are fetched kPD ahead into a register ring (slot = position in
  // the list mod kPD) so the load latency spans several queries' work
  constexpr int kR = (kHeads * CPR + kThreads - 1) / kThreads;
  u32x4 qn[kPD][kR], dn[kPD][kR];
  float ln[kPD], dln[kPD];
  auto fetch = [&](int i, int u) {                    // i: position in the staged part
    const int t = sTok[i];
#pragma unroll
    for (int i = 0; i < (kHeads * CPR + kThreads - 1) / kThreads; ++i) {
      const int c = tid + i * kThreads;
      const int h = c / CPR, col = (c - h * CPR) * 8;
      // unconditional loads from a valid row (no branch, so the compiler
      // can count the ring's loads in flight); zeroed past the head chunk
      // when written to LDS
      const bool ok = c < kHeads * CPR && h < Gc;
      const size_t src = ((size_t)t * p.Hq + h0 + min(h, Gc - 1)) * D + (ok ? col : 0);
      qn[u][i] = *reinterpret_cast<const u32x4*>(p.q + src);
      dn[u][i] = *reinterpret_cast<const u32x4*>(p.dO + src);
    }
    const size_t hr = (size_t)t * p.Hq + h0 + min(tid, Gc - 1);   // always a valid head
    ln[u] = p.lse[hr];
    dln[u] = a.D[hr];
  };
  auto put = [&](int buf, int u) {
#pragma unroll
    for (int i = 0; i < (kHeads * CPR + kThreads - 1) / kThreads; ++i) {
      const int c = tid + i * kThreads;
      const int h = c / CPR, col = (c - h * CPR) * 8;
      if (c < kHeads * CPR) {
        // rows past the head chunk are zero (the select is made here, not at
        // the load, so that the load's latency is not waited for early)
        const u32x4 z = {0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(&sQ[buf][qrow_off<D>(h, col)]) = h < Gc ? qn[u][i] : z;
        *reinterpret_cast<u32x4*>(&sdO[buf][qrow_off<D>(h, col)]) = h < Gc ? dn[u][i] : z;
      }
    }
    if (tid < kHeads) {
      sL[buf][tid] = tid < Gc ? ln[u] : INFINITY;
      sD[buf][tid] = tid < Gc ? dln[u] : 0.f;
    }
  };

  const float kLog2e = 1.4426950408889634f;
  const float sl2 = p.scale * kLog2e;
  // transposing-read offsets: heads 4lq + l16/4, columns 4 (l16 % 4)
  const int trow = lq * 4 + (l16 >> 2), tcol = (l16 & 3) * 4;
  for (int c0 = eb; c0 < ee; c0 += kIds) {
    const int n = min(kIds, ee - c0);
    __syncthreads();   // the previous part's tokens are no longer read
    for (int i = tid; i < n; i += kThreads) sTok[i] = (a.entries[c0 + i] / p.topk) / p.Hkv;
    __syncthreads();
    // the part is walked in groups of kPD queries; positions past the end
    // reload the last query and contribute nothing, so the sequence of
    // loads has no branches and the compiler can count them in flight
    unroll<0, kPD>([&](auto U) { fetch(min(decltype(U)::value, n - 1), decltype(U)::value); });
    put(0, 0);
    __syncthreads();
    // one query of the list; U: its ring slot (compile time, so the ring
    // stays in registers)
    auto query = [&](int i, auto U) {
      constexpr int u = decltype(U)::value;
      const int buf = i & 1;
      // entry i's registers went to LDS at the end of the previous step
      fetch(min(i + kPD, n - 1), u);
      const int tl = sTok[min(i, n - 1)] - q_base;
      if (r0 < p.bs) {
        // S[h][key], dP[h][key]: lane holds heads 4lq + i of key l16
        f32x4 S = {0.f, 0.f, 0.f, 0.f}, dP = S;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
          const int ao = qrow_off<D>(l16, kk * 32 + lq * 8);
          const bf16x8 aq = *reinterpret_cast<const bf16x8*>(&sQ[buf][ao]);
          const bf16x8 ad = *reinterpret_cast<const bf16x8*>(&sdO[buf][ao]);
          S = mfma16x16x32(aq, Kf[kk], S);
          dP = mfma16x16x32(ad, Vf[kk], dP);
        }
        const bool key_ok = i < n && krow_ok && (!p.causal || jl <= tl);
        i16x4 Pa, dSa;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int h = lq * 4 + r;
          const float l = sL[buf][h];
          const bool v = key_ok && l > -INFINITY && l < INFINITY;
          const float pr = v ? __builtin_amdgcn_exp2f(S[r] * sl2 - l * kLog2e) : 0.f;
          const float ds = pr * (dP[r] - sD[buf][h]);
          Pa[r] = bf16_bits((bf16)pr);
          dSa[r] = bf16_bits((bf16)ds);
        }
        // dV[key][d] += P^T dO, dK[key][d] += dS^T Q (head sum inside the MFMA)
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          const int to = qrow_off<D>(trow, c * 16 + tcol);
          const i16x4 bo = tr_read4(&sdO[buf][to]);
          const i16x4 bq = tr_read4(&sQ[buf][to]);
          dV[c] = mfma16x16x16(Pa, bo, dV[c]);
          dK[c] = mfma16x16x16(dSa, bq, dK[c]);
        }
      }
      // all waves are done with the other buffer (read two queries ago)
      put(buf ^ 1, (u + 1) % kPD);
      __syncthreads();
    };
    for (int i0 = 0; i0 < n; i0 += kPD) {
      unroll<0, kPD>([&](auto U) { query(i0 + decltype(U)::value, U); });
    }
  }

  // this chunk's dK|dV rows of the block (slot [hc][wch], 64 rows): lane
  // holds rows r0 + 4lq + i, columns 16c + l16
  if (r0 < p.bs) {
    float* slot = a.part + ((size_t)hc * a.max_chunks + wch) * 64 * (2 * D);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = r0 + lq * 4 + i;
      const int jr = jb * p.bs + rr;
      if (rr < p.bs && jr < kv_len) {
        float* dst = slot + rr * (2 * D);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          dst[c * 16 + l16] = dK[c][i] * p.scale;
          dst[D + c * 16 + l16] = dV[c][i];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// dQ of block selection (the query-major half of the same backward): one
// workgroup per (token, kv head, 16-head chunk).  The row's selected blocks
// are walked one at a time; each block's K and V rows are brought into LDS
// with direct global->LDS loads (double-buffered, one block ahead), and
// wave w takes the block's rows 16w..16w+15:
//   S^T = K Q^T and dP^T = V dO^T (16x16x32 MFMA; Q / dO of the 16 heads are
//   the B operands, resident in registers; lane: head l16, keys 4lq + i, so
//   each lane needs one head's lse and D),
//   P = exp(scale S - lse), dS = P (dP - D) in registers,
//   dQ += dS K (16x16x16 MFMA: the result layout of S^T is exactly the A
//   operand, K comes from transposing LDS reads).
// The four waves' dQ partial sums are added through LDS at the end.
// LDS rows of a block are 256 B (128 columns) with the 16-byte chunk c of
// row r at position c ^ (r % 16): 16 rows of one chunk hit 16 bank quads.
constexpr int kDqMaxSlots = 256;

template <int D>
__global__ __launch_bounds__(kThreads) void blk_dq_kernel(Params p, BwdBuffers w) {
  static_assert(D == 128, "row layout assumes 16 chunks of 16 bytes");
  constexpr int NK = D / 32, NC = D / 16;
  __shared__ __attribute__((aligned(16))) bf16 sK[2][64 * D];
  __shared__ __attribute__((aligned(16))) bf16 sV[2][64 * D];
  __shared__ int sBlk[kDqMaxSlots];
  __shared__ int sSlot[kDqMaxSlots];   // index slot of every usable block (L1-norm positions)

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  const int row = w.t0 * p.Hkv + blockIdx.x;     // (token, kv head)
  const int t = row / p.Hkv, g = row - t * p.Hkv;
  const int h0 = g * p.G + blockIdx.y * kHeads;
  const int Gc = min(kHeads, p.G - blockIdx.y * kHeads);
  const SeqPos sp = seq_pos(p, t);
  const int* irow = p.idx + (size_t)row * p.topk;

  // the row's usable blocks, in slot order (a block past the sequence or
  // wholly after the query is unused; duplicates are kept); every thread
  // votes, so every thread reaches the barriers
  __shared__ int sW[4];
  bool ok = false;
  int blk = -1;
  if (sp.active && tid < row_len(p, row)) {
    blk = irow[tid];
    ok = blk >= 0 && (long long)blk * p.bs < sp.kv_len && (!p.causal || (long long)blk * p.bs <= sp.tl);
  }
  const unsigned long long m = __ballot(ok);
  if (lane == 0) sW[wv] = __popcll(m);
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wv; ++i) base += sW[i];
  if (ok) {
    sBlk[base + __popcll(m & ((1ull << lane) - 1ull))] = blk;
    sSlot[base + __popcll(m & ((1ull << lane) - 1ull))] = tid;
  }
  const int nb = sW[0] + sW[1] + sW[2] + sW[3];
  __syncthreads();

  // Q / dO of head l16 as B operands (columns 32kk + 8lq .. +8)
  const bool hv = l16 < Gc;
  const size_t hrow = (size_t)t * p.Hq + h0 + (hv ? l16 : 0);
  bf16x8 QB[NK], OB[NK];
  {
    const bf16x8 z = {};
#pragma unroll
    for (int kk = 0; kk < NK; ++kk) {
      const bf16x8 qv = *reinterpret_cast<const bf16x8*>(p.q + hrow * D + kk * 32 + lq * 8);
      const bf16x8 ov = *reinterpret_cast<const bf16x8*>(p.dO + hrow * D + kk * 32 + lq * 8);
      QB[kk] = hv ? qv : z;
      OB[kk] = hv ? ov : z;
    }
  }
  const float lse = hv ? p.lse[hrow] : INFINITY;
  const float Dh = hv ? w.D[hrow] : 0.f;
  const float kLog2e = 1.4426950408889634f;
  const float sl2 = p.scale * kLog2e, lse2 = lse * kLog2e;
  const bool live = lse > -INFINITY && lse < INFINITY;

  // direct loads of one block: 16 loads of 1 KiB (4 rows) for K and for V;
  // wave w issues loads 4w..4w+3 of each.  Lane: row 4n + lane / 16,
  // position lane % 16 <- chunk (lane % 16) ^ (row % 16).
  auto load_block = [&](int bi, int buf) {
    const long long j0 = (long long)sBlk[bi] * p.bs;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = wv * 4 + i;
      const int r = n * 4 + (lane >> 4);
      const long long jr = j0 + min(r, p.bs - 1);
      const int jl = (int)min(jr, (long long)sp.kv_len - 1);
      const int ch = (lane & 15) ^ (r & 15);
      const size_t src = ((size_t)(sp.kv_base + jl) * p.Hkv + g) * D + ch * 8;
      __builtin_amdgcn_global_load_lds((gbl_void*)(p.k + src), (lds_void*)(&sK[buf][n * 4 * D]), 16, 0, 0);
      __builtin_amdgcn_global_load_lds((gbl_void*)(p.v + src), (lds_void*)(&sV[buf][n * 4 * D]), 16, 0, 0);
    }
  };

  f32x4 dQ[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) dQ[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int r0 = wv * 16;                        // the wave's block rows
  // LDS element offsets: A-operand rows r0 + l16 (chunk 4kk + lq), and the
  // transposing reads of rows r0 + 4lq + l16/4, columns 16c + 4(l16 % 4)
  const int ra = r0 + l16;
  const int rt = r0 + lq * 4 + (l16 >> 2);
  const int tq = l16 & 3;

  if (nb > 0) load_block(0, 0);
  // Two of these workgroups share a CU and do equal work, so they would run
  // in lockstep, both waiting for their block loads at the same time;
  // starting a pseudo-random half of them ~500 cycles late lets one compute
  // while the other waits (0.360 -> 0.331 ms on the NSA block workload).
  if ((blockIdx.x * 2654435761u) >> 31) __builtin_amdgcn_s_sleep(8);
  for (int bi = 0; bi < nb; ++bi) {
    const int buf = bi & 1;
    // this block's loads are done and every wave has left the other buffer
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    if (bi + 1 < nb) load_block(bi + 1, buf ^ 1);
    if (r0 < p.bs) {
      f32x4 S = {0.f, 0.f, 0.f, 0.f}, dP = S;
#pragma unroll
      for (int kk = 0; kk < NK; ++kk) {
        const int off = ra * D + (((kk * 4 + lq) ^ (ra & 15)) * 8);
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&sK[buf][off]);
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(&sV[buf][off]);
        S = mfma16x16x32(ka, QB[kk], S);
        dP = mfma16x16x32(va, OB[kk], dP);
      }
      // lane: head l16, block rows r0 + 4lq + i
      const long long jb = (long long)sBlk[bi] * p.bs;
      i16x4 dSa;
      float prs[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = r0 + lq * 4 + i;
        const long long jl = jb + rr;
        const bool v = live && rr < p.bs && jl < sp.kv_len && (!p.causal || jl <= sp.tl);
        const float pr = v ? __builtin_amdgcn_exp2f(S[i] * sl2 - lse2) : 0.f;
        dSa[i] = bf16_bits((bf16)(pr * (dP[i] - Dh)));
        prs[i] = pr;
      }
      if (w.l1) {
        // softmax L1-norm: P summed over the chunk's 16 heads (a 16-lane
        // row); lane l16 < 4 writes block row r0 + 4lq + l16 at its virtual
        // position slot * bs + row (rows past the block's end are skipped)
        float hs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) hs[i] = row16_sum(prs[i]);
        const int i = l16 & 3;
        const float mine = i == 0 ? hs[0] : i == 1 ? hs[1] : i == 2 ? hs[2] : hs[3];
        const int rr = r0 + lq * 4 + i;
        if (l16 < 4 && rr < p.bs)
          w.l1[((size_t)blockIdx.y * p.T * p.Hkv + row) * ((size_t)p.topk * p.bs) + (size_t)sSlot[bi] * p.bs + rr] =
              mine;
      }
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int ch = c * 2 + (tq >> 1);
        const i16x4 kb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_i16x4*)(&sK[buf][rt * D + ((ch ^ (rt & 15)) * 8) + (tq & 1) * 4]));
        dQ[c] = mfma16x16x16(dSa, kb, dQ[c]);
      }
    }
  }

  // sum the waves' partial dQ (rows: heads 4lq + i, columns 16c + l16)
  __syncthreads();
  float* red = reinterpret_cast<float*>(&sK[0][0]);   // 4 x 16 x D fp32 = 32 KiB
#pragma unroll
  for (int c = 0; c < NC; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wv * kHeads + lq * 4 + i) * D + c * 16 + l16] = dQ[c][i];
  __syncthreads();
  for (int e = tid; e < kHeads * D; e += kThreads) {
    const int h = e / D, col = e - h * D;
    if (h < Gc) {
      const float v = red[h * D + col] + red[(kHeads + h) * D + col] + red[(2 * kHeads + h) * D + col] +
                      red[(3 * kHeads + h) * D + col];
      w.dq[((size_t)t * p.Hq + h0 + h) * D + col] = (bf16)(v * p.scale);
    }
  }
}

// Chunks of every block key's list: cnt[k] = ceil(len_k / kBlkChunk).
__global__ void blk_chunk_count_kernel(const int* __restrict__ row_ptr, long long n_keys, int* __restrict__ cnt) {
  const long long k = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (k < n_keys) cnt[k] = (row_ptr[k + 1] - row_ptr[k] + kBlkChunk - 1) / kBlkChunk;
}

// dK / dV of every kv row = sum over its block key's chunks (head chunk
// outer, chunk order inner), rounded to bf16; rows whose block no query
// selected get 0.
__global__ void blk_sum_cast_kernel(Params p, BlkArgs a, long long n_rows, bf16* __restrict__ dk,
                                    bf16* __restrict__ dv) {
  const int d = p.dqk;
  const long long i = blockIdx.x * (long long)blockDim.x + threadIdx.x;
  if (i >= n_rows * 2 * d) return;
  const long long rg = i / (2 * d);                  // (kv row, kv head)
  const int c = (int)(i - rg * 2 * d);
  const long long j = rg / p.Hkv;
  const int g = (int)(rg - j * p.Hkv);
  int b = 0;
  if (p.layout == kLayoutBSND) {
    b = (int)(j / p.Skv);
  } else {
    int lo = 0, hi = p.B;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.cu_kv[mid] <= j) lo = mid; else hi = mid;
    }
    b = lo;
  }
  const int jl = (int)(j - (p.layout == kLayoutBSND ? (long long)b * p.Skv : p.cu_kv[b]));
  const long long bkey = (long long)(a.blk_base[b] + jl / p.bs) * p.Hkv + g;
  const int rr = jl % p.bs;
  // rows past the sequence's used kv rows take no part (their chunk rows
  // are never written)
  const long long w0 = a.chunk_base[bkey];
  const long long w1 = jl < seq_lens(p, b).kv_len ? a.chunk_base[bkey + 1] : w0;
  float acc = 0.f;
  for (int hc = 0; hc < a.n_hc; ++hc)
    for (long long w = w0; w < w1; ++w) acc += a.part[(((size_t)hc * a.max_chunks + w) * 64 + rr) * (2 * d) + c];
  if (c < d) dk[rg * d + c] = (bf16)acc;
  else dv[rg * d + (c - d)] = (bf16)acc;
}

}  // namespace

bool blk_dkv_supported(const Params& p) {
  return !p.fp16 && p.select == kSelBlock && !p.shared && p.dqk == p.dv && (p.dqk == 64 || p.dqk == 128) && p.bs >= 1 &&
         p.bs <= 64;
}

int blk_dkv_head_chunks(const Params& p) { return (p.G + kHeads - 1) / kHeads; }

long long blk_max_chunks(long long n_keys, long long n_slots) {
  return n_keys + (n_slots + kBlkChunk - 1) / kBlkChunk;
}

hipError_t launch_blk_chunks(const int* row_ptr, long long n_keys, int* cnt, int* chunk_base, int* scan_ws,
                             hipStream_t s) {
  if (n_keys > 0)
    hipLaunchKernelGGL(blk_chunk_count_kernel, dim3((unsigned)((n_keys + 255) / 256)), dim3(256), 0, s, row_ptr,
                       n_keys, cnt);
  return launch_scan_excl(cnt, n_keys, chunk_base, n_keys + 1, scan_ws, s);
}

hipError_t launch_blk_dkv(const Params& p, const BlkArgs& a, hipStream_t s) {
  if (a.n_keys == 0 || a.max_chunks == 0) return hipSuccess;
  dim3 grid((unsigned)a.max_chunks, (unsigned)a.n_hc);
  if (p.dqk == 128)
    hipLaunchKernelGGL(blk_dkv_kernel<128>, grid, dim3(kThreads), 0, s, p, a);
  else if (p.dqk == 64)
    hipLaunchKernelGGL(blk_dkv_kernel<64>, grid, dim3(kThreads), 0, s, p, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

bool blk_dq_supported(const Params& p) {
  return blk_dkv_supported(p) && p.dqk == 128 && p.topk <= kDqMaxSlots && p.bs % 16 == 0;
}

hipError_t launch_blk_dq(const Params& p, const BwdBuffers& w, hipStream_t s) {
  dim3 grid((unsigned)(w.Tc * p.Hkv), (unsigned)((p.G + kHeads - 1) / kHeads));
  hipLaunchKernelGGL(blk_dq_kernel<128>, grid, dim3(kThreads), 0, s, p, w);
  return hipGetLastError();
}

hipError_t launch_blk_sum_cast(const Params& p, const BlkArgs& a, long long n_rows, bf16* dk, bf16* dv,
                               hipStream_t s) {
  const long long n = n_rows * 2 * p.dqk;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(blk_sum_cast_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, p, a, n_rows, dk, dv);
  return hipGetLastError();
}

}  // namespace sa
