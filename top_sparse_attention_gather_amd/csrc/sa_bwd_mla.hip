// Shared-KV (MLA) sparse-attention backward, d_qk = 576, d_v = 512, 64
// query heads of one (token, kv head) row per workgroup.
//
// Formulas: SparseFlashMlaGrad README, "Computation formula", Stage 2
// (P = SimpleSoftmax(scale Q KV^T, lse), dP = dO KV^T, dS = P (dP - D)) and
// Stage 3 (dQ = scale dS KV, dKV = scale dS^T Q + P^T dO); gathers as in
// aclnnSparseFlashAttentionGrad, "Formula".
//
// Work split (4 waves, one per SIMD, 1 workgroup per CU):
//   phase A, wave w owns heads 16w..16w+15 for every key of a 32-key tile:
//     S^T = KV Q^T and dP^T = V dO^T (16x16x32 MFMA, KV fragments read once
//     from LDS for both, Q/dO of the wave's heads resident in registers),
//     P and dS in registers, dQ^T += KV^T dS^T (KV^T read from the same LDS
//     tile with the transposing ds_read_b64_tr_b16; dS^T taken straight from
//     the MFMA result layout, no LDS round trip).
//   phase B, wave w owns dKV columns 128w..128w+127 and 512+16w..+15 for
//     every key of the tile: dKV^T = Q^T (scale dS) + dO^T P over all 64
//     heads (dS, P exchanged through LDS; Q^T/dO^T column slices resident in
//     registers), written as bf16 into an LDS staging tile.
//   The staging tile is stored (coalesced 16-byte stores of whole partial
//   rows) at the start of the next tile, and the next KV tile is gathered
//   with direct global->LDS loads while the current one computes, so
//   neither the gather nor the store latency sits on the MFMA path.
// Partial rows go to the token-major buffer consumed by the key-major
// reduce (deterministic sum in CSR order).
#include <type_traits>

#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kNT = 32;            // keys per tile
constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kHeads = 64;         // heads per workgroup
constexpr int kKS = kDQK + 8;      // LDS row stride (elements) of KV / Q / dO tiles: 1168 B
constexpr int kSS = kDQK + 8;      // staging row stride: 1168 B (16-byte rows, conflict-free 8-byte writes)
constexpr int kXS = kHeads + 8;    // exchange row stride: 144 B
constexpr int kMaxPos = 2048;
// KV tile layout in LDS: 16-byte chunks (8 columns) grouped in pairs; pair
// j holds chunks 2j (parity 0) and 2j+1 (parity 1), each as 32 row slots,
// and row r of parity q sits in slot (r + 8q) mod 32.  One direct
// global->LDS load (64 lanes x 16 B) fills one pair, with every lane on the
// same row for the whole tile; the MFMA reads (16-byte rows of one chunk,
// and the transposing 8-byte reads that span both parities) touch each
// bank once per pass.
constexpr int kTileElems = kDQK * kNT;               // 18432 (36 KiB)
constexpr int kTilePairs = kDQK / 16;                // 36 pairs = 36 wave-wide loads
constexpr int kStageElems = kHeads * kKS;            // Q / dO staging at token start (row-major)

__device__ __forceinline__ int tile_off(int row, int chunk) {
  const int par = chunk & 1;
  return (chunk >> 1) * 512 + par * 256 + ((row + 8 * par) & 31) * 8;
}

// dO^T operand blocks of phase B kept in LDS instead of registers (the
// registers go to prefetching the MFMA operands).
constexpr int kDotLds = 3;

struct __attribute__((aligned(16))) MlaSmem {
  bf16 kv[kStageElems];            // KV tiles at 0 and kTileElems; Q / dO staging at token start
  bf16 stage[kNT * kSS];           // dKV partial tile (bf16)
  bf16 xds[kNT * kXS];             // scale * dS  [key][head]
  bf16 xp[kNT * kXS];              // P           [key][head]
  bf16x8 dot[4][kDotLds][2][64];   // phase-B dO^T operand blocks 0..kDotLds-1, register layout per lane
  int rows[kMaxPos];
  int vpos[kMaxPos];
  int wave[4];
};

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) const void gbl_void;

__device__ __forceinline__ i16x4 tr_read(const bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ bf16x8 join(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ const bf16* row_ptr(const Params& p, int code, int g) {
  return (code & kCmpFlag) ? p.cmp + ((size_t)(code & ~kCmpFlag) * p.Hkv + g) * kDQK
                           : p.k + ((size_t)code * p.Hkv + g) * kDQK;
}

// Gather the tile's rows (positions k0 .. k0+31 of the compacted list) into
// `dst` with direct global->LDS loads; wave w issues loads w, w+4, ...
__device__ __forceinline__ void gather_tile(const Params& p, const MlaSmem& sm, bf16* dst, int k0, int cnt,
                                            int g, int wv, int lane) {
  const int par = lane >> 5;
  const int r = ((lane & 31) - 8 * par) & 31;          // the row this lane fills in every pair
  const int code = sm.rows[(k0 + r < cnt) ? k0 + r : k0];
  const bf16* src = row_ptr(p, code, g) + par * 8;
#pragma unroll
  for (int i = 0; i < kTilePairs / 4; ++i) {
    const int j = wv + 4 * i;
    __builtin_amdgcn_global_load_lds((gbl_void*)(src + j * 16), (lds_void*)(dst + j * 512), 16, 0, 0);
  }
}

// Store the staged partial rows of a finished tile (nvalid rows): thread
// t owns row t / 8 and chunks t % 8 + 8i, so each lane looks up one row.
__device__ __forceinline__ void store_stage(const MlaSmem& sm, bf16* part_row0, int k0, int nvalid, int tid) {
  const int r = tid >> 3, c0 = tid & 7;
  if (r >= nvalid) return;
  bf16* dst = part_row0 + (size_t)sm.vpos[k0 + r] * kDQK;
  const bf16* src = &sm.stage[r * kSS];
#pragma unroll
  for (int i = 0; i < 9; ++i)
    *reinterpret_cast<uint4*>(dst + (c0 + 8 * i) * 8) = *reinterpret_cast<const uint4*>(src + (c0 + 8 * i) * 8);
}

__global__ __launch_bounds__(kThreads, 1) void mla_bwd_kernel(Params p, BwdBuffers w) {
  __shared__ MlaSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform: keep it (and everything derived from it,
  // e.g. the LDS destinations of the direct loads) in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  const int row = w.t0 * p.Hkv + blockIdx.x;   // (token, kv head)
  const int t = row / p.Hkv, g = row - t * p.Hkv;
  const int h0 = g * p.G + blockIdx.y * kHeads;
  const SeqPos s = seq_pos(p, t);
  const int* irow = p.idx + (size_t)row * p.topk;
  bf16* part_row0 = static_cast<bf16*>(w.partial) +
                    (((size_t)blockIdx.y * w.Tc * p.Hkv + blockIdx.x) * w.npos) * kDQK;

  // ---- compacted selection (positions and their row codes) --------------
  const int cnt = compact_positions_batched<kMaxPos / 256>(p, s, irow, n_positions(p), sm.rows, sm.wave, sm.vpos);

  // ---- lse / D of the wave's heads (phase-A layout: head = 16 wv + l16) ---
  const int hA = h0 + wv * 16 + l16;
  const float lse = p.lse[(size_t)t * p.Hq + hA];
  const float Dv = w.D[(size_t)t * p.Hq + hA];
  const float kLog2e = 1.4426950408889634f;
  const float lse2 = lse * kLog2e;
  const float sl2 = p.scale * kLog2e;
  const bool row_live = lse > -INFINITY;

  // ---- Q and dO into registers, via LDS, in both operand layouts ---------
  bf16x8 QA[18], dOA[16];          // phase A: [head 16wv + l16][32kk + 8lq .. +8]
  bf16x8 QT[9][2], dOT[8][2];      // phase B: [col][heads 32ks + 8lq .. +8]
  {
    // 32 heads per buffer, in the tile layout; every lane owns one head row
    const int par = lane >> 5;
    const int hr = ((lane & 31) - 8 * par) & 31;
    // QA: head 16wv + l16 = buffer wv / 2, local row 16 (wv % 2) + l16
    const bf16* qa = sm.kv + (wv >> 1) * kTileElems;
    const int qrow = (wv & 1) * 16 + l16;
    {
      const bf16* src = p.q + ((size_t)t * p.Hq + h0 + hr) * kDQK + par * 8;
#pragma unroll
      for (int i = 0; i < 18; ++i) {
        const int j = wv + 4 * i;          // 72 loads: pair j % 36 of buffer j / 36
        const int hb = j >= 36 ? 1 : 0;
        const int pj = j - 36 * hb;
        __builtin_amdgcn_global_load_lds((gbl_void*)(src + (size_t)hb * 32 * kDQK + pj * 16),
                                         (lds_void*)(sm.kv + hb * kTileElems + pj * 512), 16, 0, 0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) QA[kk] = *reinterpret_cast<const bf16x8*>(&qa[tile_off(qrow, 4 * kk + lq)]);
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      const int col0 = c < 8 ? wv * 128 + c * 16 : 512 + wv * 16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16* b = sm.kv + ks * kTileElems;
        const int r0 = lq * 8 + (l16 >> 2);
        const int ch = (col0 >> 3) + ((l16 & 3) >> 1);
        const int sub = (l16 & 1) * 4;
        QT[c][ks] = join(tr_read(&b[tile_off(r0, ch) + sub]), tr_read(&b[tile_off(r0 + 4, ch) + sub]));
      }
    }
    __syncthreads();
    {
      const bf16* src = p.dO + ((size_t)t * p.Hq + h0 + hr) * kDV + par * 8;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int j = wv + 4 * i;          // 64 loads: pair j % 32 of buffer j / 32
        const int hb = j >= 32 ? 1 : 0;
        const int pj = j - 32 * hb;
        __builtin_amdgcn_global_load_lds((gbl_void*)(src + (size_t)hb * 32 * kDV + pj * 16),
                                         (lds_void*)(sm.kv + hb * kTileElems + pj * 512), 16, 0, 0);
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) dOA[kk] = *reinterpret_cast<const bf16x8*>(&qa[tile_off(qrow, 4 * kk + lq)]);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int col0 = wv * 128 + c * 16;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16* b = sm.kv + ks * kTileElems;
        const int r0 = lq * 8 + (l16 >> 2);
        const int ch = (col0 >> 3) + ((l16 & 3) >> 1);
        const int sub = (l16 & 1) * 4;
        const bf16x8 v = join(tr_read(&b[tile_off(r0, ch) + sub]), tr_read(&b[tile_off(r0 + 4, ch) + sub]));
        if (c < kDotLds) sm.dot[wv][c][ks][lane] = v;
        else dOT[c][ks] = v;
      }
    }
    __syncthreads();
  }

  f32x4 dQ[36];
#pragma unroll
  for (int m = 0; m < 36; ++m) dQ[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int ntiles = (cnt + kNT - 1) / kNT;
  if (ntiles > 0) gather_tile(p, sm, sm.kv, 0, cnt, g, wv, lane);

  // per-lane LDS offsets inside a tile: phase-A fragments (row l16 or
  // 16 + l16, chunk 4kk + lq) and the transposing reads of phase A4 (rows
  // 4lq + l16/4 and 16 + 4lq + l16/4, columns 16m + 4(l16 % 4))
  const int offA0 = tile_off(l16, lq);
  const int offA1 = tile_off(16 + l16, lq);
  const int trq = l16 & 3;
  const int offT0 = tile_off(lq * 4 + (l16 >> 2), trq >> 1) + (trq & 1) * 4;
  const int offT1 = tile_off(16 + lq * 4 + (l16 >> 2), trq >> 1) + (trq & 1) * 4;

  // One tile.  kvb (read) and kvn (filled by direct loads for the next
  // tile) are restrict-qualified: they never overlap, and the alias scopes
  // this gives every LDS access let the compiler skip waiting for the
  // in-flight loads before each LDS read.
  const int gpar = lane >> 5;
  const int grow = ((lane & 31) - 8 * gpar) & 31;   // the row this lane gathers in every pair
  const int srow = tid >> 3, scol = tid & 7;        // the staged row / chunks this thread stores

  // STORE: whether the previous tile's staged partial rows are stored here.
  // The next tile's direct loads and these stores are spread over the
  // phase-A MFMAs (one or two per step) instead of being issued in a burst.
  auto step = [&](const bf16* __restrict__ kvb, bf16* __restrict__ kvn, int it, auto store_tag) {
    constexpr bool STORE = decltype(store_tag)::value;
    const int k0 = it * kNT;
    const int nvalid = min(kNT, cnt - k0);
    // every wave's loads of this tile (and stores of older tiles) are done
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int kn = k0 + kNT;   // next tile (for the last tile a harmless reload into the free buffer)
    const bf16* gsrc = row_ptr(p, sm.rows[(kn + grow < cnt) ? kn + grow : k0], g) + gpar * 8;
    bf16* sdst = part_row0 + (size_t)sm.vpos[(STORE ? k0 - kNT : k0) + srow] * kDQK + scol * 8;
    const bf16* ssrc = &sm.stage[srow * kSS + scol * 8];
    auto vmem_step = [&](int kk) {
      if (kk < 9) {
        const int j = wv + 4 * kk;
        __builtin_amdgcn_global_load_lds((gbl_void*)(gsrc + j * 16), (lds_void*)(kvn + j * 512), 16, 0, 0);
      }
      if (STORE && kk >= 2 && kk < 11) {
        const int i = kk - 2;
        *reinterpret_cast<uint4*>(sdst + i * 64) = *reinterpret_cast<const uint4*>(ssrc + i * 64);
      }
    };

    // ---- phase A: S^T and dP^T for the wave's 16 heads -------------------
    f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = S0, P0 = S0, P1 = S0;
    {
      constexpr int kPF = 2;   // KV fragments in flight ahead of their MFMAs
      bf16x8 f0[kPF + 1], f1[kPF + 1];
#pragma unroll
      for (int kk = 0; kk < kPF; ++kk) {
        f0[kk] = *reinterpret_cast<const bf16x8*>(&kvb[offA0 + kk * 1024]);
        f1[kk] = *reinterpret_cast<const bf16x8*>(&kvb[offA1 + kk * 1024]);
      }
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) {
        if (kk + kPF < 18) {
          f0[(kk + kPF) % (kPF + 1)] = *reinterpret_cast<const bf16x8*>(&kvb[offA0 + (kk + kPF) * 1024]);
          f1[(kk + kPF) % (kPF + 1)] = *reinterpret_cast<const bf16x8*>(&kvb[offA1 + (kk + kPF) * 1024]);
        }
        const bf16x8 a0 = f0[kk % (kPF + 1)], a1 = f1[kk % (kPF + 1)];
        vmem_step(kk);
        S0 = mfma16x16x32(a0, QA[kk], S0);
        S1 = mfma16x16x32(a1, QA[kk], S1);
        if (kk < 16) {
          P0 = mfma16x16x32(a0, dOA[kk], P0);
          P1 = mfma16x16x32(a1, dOA[kk], P1);
        }
      }
    }
    // P = exp(scale S - lse), dS = P (dP - D); lane: keys 16b + 4lq + r, head l16
    bf16x8 Bds;
    {
      float pr[2][4], dsr[2][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int kA = lq * 4 + r;
        const bool vA = row_live && kA < nvalid;
        const bool vB = row_live && 16 + kA < nvalid;
        pr[0][r] = vA ? __builtin_amdgcn_exp2f(S0[r] * sl2 - lse2) : 0.f;
        pr[1][r] = vB ? __builtin_amdgcn_exp2f(S1[r] * sl2 - lse2) : 0.f;
        dsr[0][r] = pr[0][r] * (P0[r] - Dv);
        dsr[1][r] = pr[1][r] * (P1[r] - Dv);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = b * 16 + lq * 4 + r;
          sm.xds[key * kXS + wv * 16 + l16] = (bf16)(dsr[b][r] * p.scale);
          sm.xp[key * kXS + wv * 16 + l16] = (bf16)pr[b][r];
          Bds[b * 4 + r] = (bf16)dsr[b][r];
        }
      }
    }
    // dQ^T[d][h] += KV^T[d][keys] dS^T[keys][h]; keys of k-group lq:
    // 4lq..4lq+3 and 16+4lq..16+4lq+3, matching Bds
    {
      constexpr int kPF = 3;   // transposed KV operands in flight
      bf16x8 fa[kPF + 1];
#pragma unroll
      for (int m = 0; m < kPF; ++m) fa[m] = join(tr_read(&kvb[offT0 + m * 512]), tr_read(&kvb[offT1 + m * 512]));
#pragma unroll
      for (int m = 0; m < 36; ++m) {
        if (m + kPF < 36)
          fa[(m + kPF) % (kPF + 1)] = join(tr_read(&kvb[offT0 + (m + kPF) * 512]), tr_read(&kvb[offT1 + (m + kPF) * 512]));
        dQ[m] = mfma16x16x32(fa[m % (kPF + 1)], Bds, dQ[m]);
      }
    }
    // exchange written, staging free (its stores were issued): an LDS-only
    // barrier, so the next tile's gather stays in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    // ---- phase B: dKV^T columns of this wave over all 64 heads -----------
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int krow = kb * 16 + l16;
      const bf16x8 d0 = *reinterpret_cast<const bf16x8*>(&sm.xds[krow * kXS + lq * 8]);
      const bf16x8 d1 = *reinterpret_cast<const bf16x8*>(&sm.xds[krow * kXS + 32 + lq * 8]);
      const bf16x8 p0 = *reinterpret_cast<const bf16x8*>(&sm.xp[krow * kXS + lq * 8]);
      const bf16x8 p1 = *reinterpret_cast<const bf16x8*>(&sm.xp[krow * kXS + 32 + lq * 8]);
      // two column blocks at a time so their MFMA chains interleave
#pragma unroll
      for (int c = 0; c < 9; c += 2) {
        f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (c + u < 9) acc[u] = mfma16x16x32(QT[c + u][0], d0, acc[u]);
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (c + u < 9) acc[u] = mfma16x16x32(QT[c + u][1], d1, acc[u]);
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int cc = c + u;
          if (cc < 8) {
            const bf16x8 o0 = cc < kDotLds ? sm.dot[wv][cc < kDotLds ? cc : 0][0][lane] : dOT[cc][0];
            acc[u] = mfma16x16x32(o0, p0, acc[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int cc = c + u;
          if (cc < 8) {
            const bf16x8 o1 = cc < kDotLds ? sm.dot[wv][cc < kDotLds ? cc : 0][1][lane] : dOT[cc][1];
            acc[u] = mfma16x16x32(o1, p1, acc[u]);
          }
        }
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int cc = c + u;
          if (cc < 9) {
            const int col0 = (cc < 8 ? wv * 128 + cc * 16 : 512 + wv * 16) + lq * 4;
            typedef short i16x4v __attribute__((ext_vector_type(4)));
            i16x4v o = {bf16_bits((bf16)acc[u][0]), bf16_bits((bf16)acc[u][1]), bf16_bits((bf16)acc[u][2]),
                        bf16_bits((bf16)acc[u][3])};
            *reinterpret_cast<i16x4v*>(&sm.stage[krow * kSS + col0]) = o;
          }
        }
      }
    }
  };
  if (ntiles > 0) step(sm.kv, sm.kv + kTileElems, 0, std::integral_constant<bool, false>());
  for (int it = 1; it < ntiles; ++it) {
    bf16* b0 = sm.kv + (it & 1) * kTileElems;
    bf16* b1 = sm.kv + ((it + 1) & 1) * kTileElems;
    step(b0, b1, it, std::integral_constant<bool, true>());
  }

  // ---- last tile's partial rows, then dQ ----------------------------------
  if (ntiles > 0) {
    __syncthreads();
    store_stage(sm, part_row0, (ntiles - 1) * kNT, cnt - (ntiles - 1) * kNT, tid);
  }
  bf16* dq = w.dq + ((size_t)t * p.Hq + h0 + wv * 16 + l16) * kDQK;
#pragma unroll
  for (int m = 0; m < 36; ++m) {
    typedef short i16x4v __attribute__((ext_vector_type(4)));
    i16x4v o = {bf16_bits((bf16)(dQ[m][0] * p.scale)), bf16_bits((bf16)(dQ[m][1] * p.scale)),
                bf16_bits((bf16)(dQ[m][2] * p.scale)), bf16_bits((bf16)(dQ[m][3] * p.scale))};
    *reinterpret_cast<i16x4v*>(dq + m * 16 + lq * 4) = o;
  }
}

}  // namespace

bool mla_bwd_supported(const Params& p) {
  return p.shared && p.dqk == kDQK && p.dv == kDV && p.G % kHeads == 0 && p.select != kSelBlock &&
         (p.select == kSelToken ? p.topk : p.win_left + 1 + p.win_right + p.topk) <= kMaxPos;
}

int mla_bwd_head_groups(const Params& p) { return p.G / kHeads; }

hipError_t launch_bwd_mla(const Params& p, const BwdBuffers& w, hipStream_t s) {
  dim3 grid((unsigned)(w.Tc * p.Hkv), (unsigned)(p.G / kHeads));
  hipLaunchKernelGGL(mla_bwd_kernel, grid, dim3(kThreads), 0, s, p, w);
  return hipGetLastError();
}

}  // namespace sa
