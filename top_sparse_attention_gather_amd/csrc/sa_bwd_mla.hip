// Shared-KV (MLA) sparse-attention backward, d_qk = 576, d_v = 512, 64
// query heads of one (token, kv head) row per workgroup.
//
// Formulas: SparseFlashMlaGrad README, "Computation formula", Stage 2
// (P = SimpleSoftmax(scale Q KV^T, lse), dP = dO KV^T, dS = P (dP - D)) and
// Stage 3 (dQ = scale dS KV, dKV = scale dS^T Q + P^T dO); gathers as in
// aclnnSparseFlashAttentionGrad, "Formula".
//
// Work split (4 waves, one per SIMD, 1 workgroup per CU), per 32-key tile:
//   phase A, wave w owns heads 16w..16w+15 for every key of the tile:
//     S^T = KV Q^T and dP^T = V dO^T (16x16x32 MFMA, KV fragments read once
//     from LDS for both, Q/dO of the wave's heads resident in registers),
//     keys 0..15 then 16..31, so that P and dS of the first half are
//     computed while the MFMAs of the second half run; scale dS and P go
//     to an LDS exchange ([key][head]).
//   phase B, wave w owns dKV / dQ columns 128w..128w+127 and 512+16w..+15:
//     dKV^T = Q^T (scale dS) + dO^T P over all 64 heads (Q^T/dO^T column
//     slices resident in registers), stored as bf16 partial rows straight
//     from the MFMA results; then dQ^T += KV^T (scale dS)^T for all 64
//     heads, with KV^T of the wave's columns only (transposing
//     ds_read_b64_tr_b16 reads) -- every wave reads a quarter of the tile
//     instead of all of it.
//   Phase B of a tile runs during the next tile's phase A (its MFMA chains
//   and stores interleaved with the phase-A steps); the first tile has none
//   before it and the last tile's runs after the loop.  The next KV tile is
//   gathered with direct global->LDS loads during phase A, so the gather
//   latency is off the MFMA path.
// D = rowsum(dO o O) is formed at the workgroup's start from the staged dO
// and the O rows (with the dSinks terms) when the launch asks for it (the
// library always does), else read from the preprocess pass's output.
// Partial rows go to the
// token-major buffer consumed by the key-major reduce (deterministic sum in
// CSR order).
#include <type_traits>

#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kThreads = 256;
constexpr int kNT = 32;            // keys per tile
constexpr int kDQK = 576;
constexpr int kDV = 512;
constexpr int kHeads = 64;         // heads per workgroup
constexpr int kKS = kDQK + 8;      // sizes the KV tile / Q staging region: 64 rows of 1168 B
constexpr int kXS = kHeads + 8;    // exchange row stride: 144 B
constexpr int kMaxPos = 2048;
// KV tile layout in LDS (32 rows x 72 chunks of 16 bytes): the rows form 4
// groups of 8; group rg starts at rg * (9 KiB + 64 B) and holds 9
// segments of 1 KiB, segment s = columns 64s..64s+63 of its 8 rows (row rr
// at rr * 128 B), with chunk c at position (c & 4) | ((c & 3) ^ (rr >> 1)).
//  - One direct global->LDS load (64 lanes x 16 B) fills one segment of one
//    group: 8 whole 128-byte lines, half the address-unit work per byte of
//    loads that touch a line per lane pair.  Wave w loads group w.
//  - A 16-byte MFMA fragment read (16 rows, one chunk) hits 16 distinct
//    4-bank groups (row parity, the 64-byte group skew and the XOR split
//    them), and chunk c + 4 sits at a fixed offset from chunk c.
constexpr int kSegElems = 512;                       // one 1 KiB segment
constexpr int kGroupElems = 9 * kSegElems;           // 8 rows x 576 columns
constexpr int kGroupStride = kGroupElems + 32;       // groups 64 B apart in bank phase
constexpr int kTileElems = 4 * kGroupStride;         // 18560 (36.25 KiB)
constexpr int kStageElems = kHeads * kKS;            // LDS of the KV tiles and of the Q / dO staging
static_assert(2 * kTileElems <= kStageElems, "two tiles fit the staging region");

// dO (512 columns) is staged in the same layout with 8 segments per group.
constexpr int kDoGroupStride = 8 * kSegElems + 32;
constexpr int kDoTileElems = 4 * kDoGroupStride;     // 32 heads of dO (33 KiB)

__device__ __forceinline__ int group_base(int rg, int gstride = kGroupStride) { return rg * gstride; }

__device__ __forceinline__ int tile_off(int row, int chunk, int gstride = kGroupStride) {
  const int rr = row & 7;
  return group_base(row >> 3, gstride) + (chunk >> 3) * kSegElems + rr * 64 +
         ((chunk & 4) | ((chunk & 3) ^ (rr >> 1))) * 8;
}

// The chunk (within its segment) that lane `lane` of a wave-wide segment
// load fetches: position lane & 7 of row lane >> 3 (the XOR is its own
// inverse).
__device__ __forceinline__ int seg_chunk(int lane) {
  const int pos = lane & 7, rr = lane >> 3;
  return (pos & 4) | ((pos & 3) ^ (rr >> 1));
}

// dO^T operand blocks of phase B kept in LDS instead of registers (the
// registers go to prefetching the MFMA operands).
constexpr int kDotLds = 6;

struct __attribute__((aligned(16))) MlaSmem {
  bf16 kv[kStageElems];            // KV tiles at 0 and kTileElems; Q staging at token start
  union {
    struct {
      bf16 xds[2][kNT * kXS];          // scale * dS  [key][head], tiles alternate
      bf16 xp[2][kNT * kXS];           // P           [key][head]
      bf16x8 dot[4][kDotLds][2][64];   // phase-B dO^T operand blocks 0..kDotLds-1, register layout per lane
    };
    bf16 dost[2 * kDoTileElems];       // dO staging at token start (free until the tile loop)
  };
  int rows[kMaxPos];
  int vpos[kMaxPos];
  int wave[4 * (kMaxPos / 256)];   // per-round wave counts of the compaction
  float l1s[4][kNT];               // softmax L1-norm: P summed over each wave's 16 heads, per key
};

static_assert(2 * kDoTileElems * 2 <= 2 * (2 * kNT * kXS * 2) + 4 * kDotLds * 2 * 64 * 16,
              "the dO staging fits the exchange and dO^T-block area");

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

// The two 16-bit input formats.  Operands travel through LDS and registers
// as raw 16-bit containers (typed bf16 here); only the MFMA, the
// conversions from and to fp32 and the exchange factor depend on the
// format.  fp16 multiplies the exchanged P and scale dS (small at long
// lists: about 1/2048 and 2e-5) by 2^10, which keeps them out of fp16's
// subnormal range; the fp32 results are divided by it (exact).
template <typename E>
struct Fmt;

template <>
struct Fmt<bf16> {
  static constexpr float kX = 1.f;
  __device__ static f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) { return mfma16x16x32(a, b, c); }
  __device__ static bf16 to16(float x) { return (bf16)x; }
  __device__ static float from16(bf16 x) { return (float)x; }
};

template <>
struct Fmt<f16> {
  static constexpr float kX = 1024.f;
  __device__ static f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
  }
  __device__ static bf16 to16(float x) { return __builtin_bit_cast(bf16, (f16)x); }
  __device__ static float from16(bf16 x) { return (float)__builtin_bit_cast(f16, x); }
};

__device__ __forceinline__ const bf16* row_ptr(const Params& p, int code, int g) {
  return (code & kCmpFlag) ? p.cmp + ((size_t)(code & ~kCmpFlag) * p.Hkv + g) * kDQK
                           : p.k + ((size_t)code * p.Hkv + g) * kDQK;
}

// Direct global->LDS load, 16 bytes per lane, to the wave-uniform LDS
// address `lds` (+ 16 x lane).  Inline asm instead of the builtin: the
// compiler models the builtin as a FLAT access that may touch LDS, and while
// one is outstanding it turns every LDS wait into a full drain
// (lgkmcnt(0)), which cancels the read-ahead of the MFMA operands.  The
// wait-count insertion does not see these loads, so the kernel waits for
// them itself: vmcnt(0) before the barrier that hands a filled tile buffer
// to its readers, and before the workgroup ends.  No register receives data
// (it goes to LDS), so nothing else can depend on a load in flight.  M0
// (the LDS base) is an input operand, so the compiler sets it.
__device__ __forceinline__ void load_lds16(const bf16* src, bf16* lds) {
  const unsigned base = __builtin_amdgcn_readfirstlane((unsigned)(size_t)(lds_void*)lds);
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(base) : "memory");
}

// Gather the tile's rows (positions k0 .. k0+31 of the compacted list) into
// `dst` with direct global->LDS loads; wave w loads row group w, one
// segment per load.
__device__ __forceinline__ void gather_tile(const Params& p, const MlaSmem& sm, bf16* dst, int k0, int cnt,
                                            int g, int wv, int lane) {
  const int r = wv * 8 + (lane >> 3);                   // the row this lane fills
  const int code = sm.rows[(k0 + r < cnt) ? k0 + r : k0];
  const bf16* src = row_ptr(p, code, g) + seg_chunk(lane) * 8;
  bf16* d = dst + group_base(wv);
#pragma unroll
  for (int sg = 0; sg < 9; ++sg)
    load_lds16(src + sg * 64, d + sg * kSegElems);
}

// The XCD (accelerator complex die) the wave runs on, 0..7: it picks the
// fp32 accumulator replica of the per-XCD atomic form.  Any value is
// correct (the adds are device-scope atomics); one replica per XCD keeps
// the XCDs off each other's lines.
__device__ __forceinline__ int xcc_id() {
  int x;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
  return x & 7;
}

// L1: also write the head sums of P behind the softmax L1-norm outputs
// (SparseFlashMlaGrad README, parameter table).
// OUT: how phase B's per-(token, key) dKV rows leave the kernel -- kOutPartial:
// bf16 partial rows for the deterministic key-major reduce; kOutAtomic: fp32
// atomic adds into the accumulator; kOutAtomicXcd: the same into the
// accumulator replica of the wave's XCD (summed in a fixed order afterwards).
// E: the inputs' 16-bit format (bf16 or fp16).  The workgroup's head group
// may hold fewer than 64 heads (the last group when the heads per kv head
// are not a multiple of 64): the missing heads are masked (P = 0, so they
// add nothing; their loads repeat a present head's row and their dQ is not
// stored).  Rows longer than kMaxPos positions are compacted and processed
// in passes of kMaxPos positions.
template <typename E, bool L1, int OUT>
__global__ __launch_bounds__(kThreads, 1) void mla_bwd_kernel(Params p, BwdBuffers w) {
  using F = Fmt<E>;
  constexpr float kX = F::kX, kInvX = 1.f / F::kX;
  __shared__ MlaSmem sm;
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index is uniform: keep it (and everything derived from it,
  // e.g. the LDS destinations of the direct loads) in scalar registers
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15, lq = lane >> 4;
  const int row = w.t0 * p.Hkv + blockIdx.x;   // (token, kv head)
  const int t = row / p.Hkv, g = row - t * p.Hkv;
  const int h0 = g * p.G + blockIdx.y * kHeads;
  const int gh = min(kHeads, p.G - (int)blockIdx.y * kHeads);   // heads present in this group
  const SeqPos s = seq_pos(p, t);
  const int* irow = p.idx + (size_t)row * p.topk;
  bf16* part_row0 = static_cast<bf16*>(w.partial) +
                    (((size_t)blockIdx.y * w.Tc * p.Hkv + blockIdx.x) * w.npos) * kDQK;

  // ---- indices of the first pass of at most kMaxPos positions: loaded
  // here, compacted (positions and their row codes) once they and the Q / dO
  // staging loads below have landed -- one wait for both ----------------------
  const int npos = n_positions(p);
  const int len = row_len(p, row);
  constexpr int kRounds = kMaxPos / 256;
  int raw[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const int pos = r * 256 + tid;
    raw[r] = pos < min(npos, kMaxPos) ? position_index(p, irow, pos, len) : -1;
  }

  // ---- lse / D of the wave's heads (phase-A layout: head = 16 wv + l16);
  // with fuse_d, D follows from the staged dO and O below -------------------
  const bool head_ok = wv * 16 + l16 < gh;
  const int hA = h0 + min(wv * 16 + l16, gh - 1);
  const float lse = p.lse[(size_t)t * p.Hq + hA];
  float Dv = w.fuse_d ? 0.f : w.D[(size_t)t * p.Hq + hA];
  const float kLog2e = 1.4426950408889634f;
  const float lse2 = lse * kLog2e;
  const float sl2 = p.scale * kLog2e;
  const bool row_live = head_ok && lse > -INFINITY;

  // ---- Q and dO into registers, via LDS, in both operand layouts ---------
  // Q goes to the two KV tile buffers and dO to the exchange / dO^T-block
  // area (both free until the tile loop), with all the loads in flight
  // together (with fuse_d, so do the O rows of the wave's 16 heads, into
  // registers).  The first pass's positions are compacted behind them (the
  // index loads went out first, so their latency and the staging's overlap
  // instead of adding up); one wait, then (fuse_d) D = rowsum(dO o O)
  // (SparseFlashMlaGrad README, Stage 2) and the operand layouts are read out.
  bf16x8 QA[18], dOA[16];          // phase A: [head 16wv + l16][32kk + 8lq .. +8]
  bf16x8 QT[9][2], dOT[8][2];      // phase B: [col][heads 32ks + 8lq .. +8]
  int cnt;
  {
    // 32 heads per buffer, in the tile layout; wave w loads row group w of
    // both buffers (heads 32hb + 8w + lane / 8)
    const int hr = wv * 8 + (lane >> 3);
    const int sc = seg_chunk(lane) * 8;
    {
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int hq = h0 + min(hb * 32 + hr, gh - 1);   // a missing head repeats the last present one
        const bf16* src = p.q + ((size_t)t * p.Hq + hq) * kDQK + sc;
        const bf16* srcd = p.dO + ((size_t)t * p.Hq + hq) * kDV + sc;
#pragma unroll
        for (int sg = 0; sg < 9; ++sg)
          load_lds16(src + sg * 64, sm.kv + hb * kTileElems + group_base(wv) + sg * kSegElems);
#pragma unroll
        for (int sg = 0; sg < 8; ++sg)
          load_lds16(srcd + sg * 64, sm.dost + hb * kDoTileElems + group_base(wv, kDoGroupStride) + sg * kSegElems);
      }
    }
    uint4 orow[16];   // O of head 16wv + i, columns 8 lane .. 8 lane + 7
    if (w.fuse_d) {
#pragma unroll
      for (int i = 0; i < 16; ++i)
        orow[i] = *reinterpret_cast<const uint4*>(p.o + ((size_t)t * p.Hq + h0 + min(wv * 16 + i, gh - 1)) * kDV +
                                                  lane * 8);
    }
    cnt = compact_loaded(p, s, raw, min(npos, kMaxPos), sm.rows, sm.wave, sm.vpos);
    asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    // D of head 16wv + i: the lane's 8 products with chunk `lane` of the
    // staged dO row, summed over the 64 lanes; lane l16 keeps head l16's
    if (w.fuse_d) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int hh = wv * 16 + i;
        const bf16x8 dv = *reinterpret_cast<const bf16x8*>(
            &sm.dost[(hh >> 5) * kDoTileElems + tile_off(hh & 31, lane, kDoGroupStride)]);
        const bf16x8 ov = __builtin_bit_cast(bf16x8, orow[i]);
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) a += F::from16(ov[j]) * F::from16(dv[j]);
        a = wave_sum(a);
        Dv = l16 == i ? a : Dv;
      }
      // the dSinks term of each (token, head) row (SparseFlashMlaGrad
      // README, Stage 3), summed over the tokens after the kernel
      if (p.has_sinks && lq == 0 && head_ok)
        w.sink_term[(size_t)t * p.Hq + hA] = lse > -INFINITY ? -__expf(p.sinks[hA] - lse) * Dv : 0.f;
    }
    // QA / dOA: head 16wv + l16 = buffer wv / 2, local row 16 (wv % 2) + l16
    const int qrow = (wv & 1) * 16 + l16;
    const bf16* qa = sm.kv + (wv >> 1) * kTileElems;
    const bf16* da = sm.dost + (wv >> 1) * kDoTileElems;
#pragma unroll
    for (int kk = 0; kk < 18; ++kk) QA[kk] = *reinterpret_cast<const bf16x8*>(&qa[tile_off(qrow, 4 * kk + lq)]);
#pragma unroll
    for (int kk = 0; kk < 16; ++kk)
      dOA[kk] = *reinterpret_cast<const bf16x8*>(&da[tile_off(qrow, 4 * kk + lq, kDoGroupStride)]);
    const int r0 = lq * 8 + (l16 >> 2);
    const int sub = (l16 & 1) * 4;
#pragma unroll
    for (int c = 0; c < 9; ++c) {
      const int col0 = c < 8 ? wv * 128 + c * 16 : 512 + wv * 16;
      const int ch = (col0 >> 3) + ((l16 & 3) >> 1);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16* b = sm.kv + ks * kTileElems;
        QT[c][ks] = join(tr_read(&b[tile_off(r0, ch) + sub]), tr_read(&b[tile_off(r0 + 4, ch) + sub]));
        if (c < 8) {
          const bf16* bd = sm.dost + ks * kDoTileElems;
          dOT[c][ks] = join(tr_read(&bd[tile_off(r0, ch, kDoGroupStride) + sub]),
                            tr_read(&bd[tile_off(r0 + 4, ch, kDoGroupStride) + sub]));
        }
      }
    }
    // every wave has read the staged Q and dO before the dO^T blocks (which
    // overlay the dO staging) are written and the first KV tile is gathered
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kDotLds; ++c)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) sm.dot[wv][c][ks][lane] = dOT[c][ks];
  }

  f32x4 dQ[36];
#pragma unroll
  for (int m = 0; m < 36; ++m) dQ[m] = f32x4{0.f, 0.f, 0.f, 0.f};

  int ntiles = (cnt + kNT - 1) / kNT;
  if (ntiles > 0) gather_tile(p, sm, sm.kv, 0, cnt, g, wv, lane);

  // per-lane LDS offsets inside a tile: phase-A fragments (row l16 or
  // 16 + l16, chunk 4kk + lq) and the transposing reads of the dQ product
  // (rows 4lq + l16/4 and 16 + 4lq + l16/4, columns 4(l16 % 4) of a
  // 16-column block)
  // chunk 4kk + lq of a row sits at tile_off(row, lq) + (kk / 2) 512 +
  // (kk % 2) 32; the transposing read of column block m (chunks 2m, 2m+1)
  // at tile_off(row, 2 (m % 2) + b) + (m / 4) 512 + ((m / 2) % 2) 32
  const int offA0 = tile_off(l16, lq);
  const int offA1 = tile_off(16 + l16, lq);
  const int trq = l16 & 3;
  const int tr0 = lq * 4 + (l16 >> 2), tr1 = 16 + tr0;
  const int offT0e = tile_off(tr0, trq >> 1) + (trq & 1) * 4, offT0o = tile_off(tr0, 2 + (trq >> 1)) + (trq & 1) * 4;
  const int offT1e = tile_off(tr1, trq >> 1) + (trq & 1) * 4, offT1o = tile_off(tr1, 2 + (trq >> 1)) + (trq & 1) * 4;
  auto kvt = [&](const bf16* kvb, int m) {   // KV^T fragment of column block m
    const int o = (m >> 2) * kSegElems + ((m >> 1) & 1) * 32;
    return join(tr_read(&kvb[((m & 1) ? offT0o : offT0e) + o]), tr_read(&kvb[((m & 1) ? offT1o : offT1e) + o]));
  };
  // the same key rows of the exchange ([key][head], heads 4(l16 % 4)..+3)
  const int offX0 = (lq * 4 + (l16 >> 2)) * kXS + trq * 4;
  const int offX1 = (16 + lq * 4 + (l16 >> 2)) * kXS + trq * 4;
  bf16* dump = static_cast<bf16*>(w.dump);
  float* l1_row = L1 ? w.l1 + ((size_t)blockIdx.y * p.T * p.Hkv + row) * npos : nullptr;
  const int grow = wv * 8 + (lane >> 3);            // the row this lane gathers (row group wv)
  const int gcol = seg_chunk(lane) * 8;
  // phase-B / dQ column block c of this wave (16 columns)
  auto col_block = [&](int c) { return c < 8 ? wv * 128 + c * 16 : 512 + wv * 16; };

  // ---- phase B: dKV^T columns of this wave over all 64 heads for one key
  // half (kb) of tile `itb`, stored as partial rows.  The 9 column-block
  // MFMA chains of a half are spread over the phase-A steps of the next
  // tile, so that the partial-row stores (the HBM write stream) go out
  // evenly instead of in one burst that stalls the wave.
  struct BHalf {
    bf16x8 d0, d1, p0, p1;   // scale dS and P, B operands (key krow, heads 8lq..)
    bf16* row;               // partial row of key krow (or the dump row)
  };
  auto b_setup = [&](int itb, int kb, bool live) {
    BHalf h;
    const bf16* xd = sm.xds[itb & 1];
    const bf16* xpp = sm.xp[itb & 1];
    const int krow = kb * 16 + l16;
    h.d0 = *reinterpret_cast<const bf16x8*>(&xd[krow * kXS + lq * 8]);
    h.d1 = *reinterpret_cast<const bf16x8*>(&xd[krow * kXS + 32 + lq * 8]);
    h.p0 = *reinterpret_cast<const bf16x8*>(&xpp[krow * kXS + lq * 8]);
    h.p1 = *reinterpret_cast<const bf16x8*>(&xpp[krow * kXS + 32 + lq * 8]);
    // rows past the end of the list go to the dump row, so the stores need
    // no branch
    const int k0 = itb * kNT;
    const bool kvalid = live && krow < cnt - k0;
    // 0 <= index < kMaxPos always (k0 = -32 for the tile before the first,
    // a stale position past the list), so the load needs no branch; the
    // select picks the dump row
    const int vp = sm.vpos[max(k0 + krow, 0)];
    bf16* const rowp = part_row0 + (size_t)vp * kDQK;
    h.row = kvalid ? rowp : dump;
    return h;
  };
  // dO^T operand block ks of column block cc < 8 (the first kDotLds from LDS)
  auto dot_op = [&](int cc, int ks) -> bf16x8 {
    const int c = cc < 8 ? cc : 0;
    return c < kDotLds ? sm.dot[wv][c < kDotLds ? c : 0][ks][lane] : dOT[c][ks];
  };
  // one column-block chain: Q^T (scale dS) + dO^T P (no dO part for the
  // rope columns, cc = 8); o0 / o1 are its dO^T operands
  auto b_chain = [&](const BHalf& h, int cc, const bf16x8& o0, const bf16x8& o1) {
    f32x4 acc = F::mma(QT[cc][0], h.d0, f32x4{0.f, 0.f, 0.f, 0.f});
    acc = F::mma(QT[cc][1], h.d1, acc);
    if (cc < 8) {
      acc = F::mma(o0, h.p0, acc);
      acc = F::mma(o1, h.p1, acc);
    }
    return acc;
  };
  // Stores of the MFMA results (lane: columns 4lq..4lq+3 of a 16-column
  // block, key l16).  Blocks c and c + 1 (c even, < 8) go out together:
  // after swapping halves with the neighbouring 16-lane row, lane lq holds
  // 8 contiguous columns (lq even: block c from 4lq, lq odd: block c + 1
  // from 4(lq - 1)), so one 16-byte store per lane writes 64 contiguous
  // bytes of every row -- half as many L1 write requests as 8-byte stores.
  auto pk2 = [](float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(unsigned, bf16x2{(bf16)a, (bf16)b});
  };
  auto b_put_pair = [&](const BHalf& h, int c, f32x4 a, f32x4 b) {
    if constexpr (kX != 1.f) {
      a *= kInvX;
      b *= kInvX;
    }
    const auto s0 = __builtin_amdgcn_permlane16_swap(pk2(a[0], a[1]), pk2(b[0], b[1]), false, false);
    const auto s1 = __builtin_amdgcn_permlane16_swap(pk2(a[2], a[3]), pk2(b[2], b[3]), false, false);
    const uint4 v = {s0[0], s1[0], s0[1], s1[1]};
    *reinterpret_cast<uint4*>(h.row + col_block(c) + (lq & 1) * 16 + (lq >> 1) * 8) = v;
  };
  auto b_put_single = [&](const BHalf& h, int c, f32x4 a) {
    if constexpr (kX != 1.f) a *= kInvX;
    const uint2 v = {pk2(a[0], a[1]), pk2(a[2], a[3])};
    *reinterpret_cast<uint2*>(h.row + col_block(c) + lq * 4) = v;
  };

  // ---- atomic forms of phase B: the same products with the operands
  // swapped, dKV[key][col] = (scale dS)^T Q + P^T dO, so that lane (l16, lq)
  // holds keys 4lq..4lq+3 of column l16 of a 16-column block and one atomic
  // instruction adds 4 keys x 16 contiguous columns.
  float* const acc_k = OUT == kOutAtomicXcd ? w.acc_k + (size_t)xcc_id() * w.rep_stride : w.acc_k;
  float* const acc_c = OUT == kOutAtomicXcd ? w.acc_cmp + (size_t)xcc_id() * w.rep_stride : w.acc_cmp;
  struct AHalf {
    bf16x8 d0, d1, p0, p1;
    float* row[4];            // accumulator rows of keys 4lq + r (or the dump row)
  };
  auto a_setup = [&](int itb, int kb) {
    AHalf h;
    const bf16* xd = sm.xds[itb & 1];
    const bf16* xpp = sm.xp[itb & 1];
    const int krow = kb * 16 + l16;
    h.d0 = *reinterpret_cast<const bf16x8*>(&xd[krow * kXS + lq * 8]);
    h.d1 = *reinterpret_cast<const bf16x8*>(&xd[krow * kXS + 32 + lq * 8]);
    h.p0 = *reinterpret_cast<const bf16x8*>(&xpp[krow * kXS + lq * 8]);
    h.p1 = *reinterpret_cast<const bf16x8*>(&xpp[krow * kXS + 32 + lq * 8]);
    const int k0 = itb * kNT;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kb * 16 + lq * 4 + r;
      const bool valid = key < cnt - k0;
      const int code = valid ? sm.rows[k0 + key] : 0;   // k0 + key < kMaxPos
      float* const rp = (code & kCmpFlag) ? acc_c + ((size_t)(code & ~kCmpFlag) * p.Hkv + g) * kDQK
                                          : acc_k + ((size_t)code * p.Hkv + g) * kDQK;
      h.row[r] = valid ? rp : static_cast<float*>(w.dump);
    }
    return h;
  };
  auto a_chain = [&](const AHalf& h, int cc, const bf16x8& o0, const bf16x8& o1) {
    f32x4 acc = F::mma(h.d0, QT[cc][0], f32x4{0.f, 0.f, 0.f, 0.f});
    acc = F::mma(h.d1, QT[cc][1], acc);
    if (cc < 8) {
      acc = F::mma(h.p0, o0, acc);
      acc = F::mma(h.p1, o1, acc);
    }
    return acc;
  };
  auto a_add = [&](const AHalf& h, int c, const f32x4& a) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      __hip_atomic_fetch_add(h.row[r] + col_block(c) + l16, a[r] * kInvX, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  // One tile.  kvb (read) and kvn (filled by direct loads for the next
  // tile) are restrict-qualified: they never overlap, and the alias scopes
  // this gives every LDS access let the compiler skip waiting for the
  // in-flight loads before each LDS read.
  // PB: whether the tile before this one exists, i.e. whether its phase B
  // runs here (not for the first tile)
  auto step = [&](auto pb, const bf16* __restrict__ kvb, bf16* __restrict__ kvn, int it) {
    constexpr bool PB = decltype(pb)::value;
    const int k0 = it * kNT;
    const int nvalid = min(kNT, cnt - k0);
    // every wave's loads of this tile are done and the previous tile's
    // exchange / KV buffer reads are finished
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    bf16* xw = sm.xds[it & 1];
    bf16* pw = sm.xp[it & 1];
    const int kn = k0 + kNT;   // next tile
    const bf16* gsrc = row_ptr(p, sm.rows[(kn + grow < cnt) ? kn + grow : k0], g) + gcol;
    bf16* gdst = kvn + group_base(wv);

    // ---- phase A: S^T and dP^T for the wave's 16 heads, two key halves ---
    // P = exp(scale S - lse), dS = P (dP - D) for keys 16b + 4lq + r, head
    // l16; scale dS and P into the exchange
    auto softmax_grad = [&](int b, const f32x4& S, const f32x4& dP) {
      float prs[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = b * 16 + lq * 4 + r;
        const bool v = row_live && key < nvalid;
        const float pr = v ? __builtin_amdgcn_exp2f(S[r] * sl2 - lse2) : 0.f;
        const float ds = pr * (dP[r] - Dv);
        xw[key * kXS + wv * 16 + l16] = F::to16(ds * (p.scale * kX));
        pw[key * kXS + wv * 16 + l16] = F::to16(pr * kX);
        prs[r] = pr;
      }
      if constexpr (L1) {
        // sum over the wave's 16 heads (the lanes of a 16-lane row); the
        // lanes with l16 % 4 == r store key 4lq + r (equal values, no branch)
        float hs[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) hs[r] = row16_sum(prs[r]);
        const int r = l16 & 3;
        const float mine = r == 0 ? hs[0] : r == 1 ? hs[1] : r == 2 ? hs[2] : hs[3];
        sm.l1s[wv][b * 16 + lq * 4 + r] = mine;
      }
    };
    f32x4 Sh0, Ph0;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const int off = b ? offA1 : offA0;
      constexpr int kPF = 2;   // KV fragments in flight ahead of their MFMAs
      bf16x8 f[kPF + 1];
#pragma unroll
      for (int kk = 0; kk < kPF; ++kk)
        f[kk] = *reinterpret_cast<const bf16x8*>(&kvb[off + (kk >> 1) * kSegElems + (kk & 1) * 32]);
      f32x4 S = {0.f, 0.f, 0.f, 0.f}, dP = S;
      // phase B of the previous tile, key half b (none for the first tile)
      BHalf hb;
      AHalf ha;
      if constexpr (PB) {
        if constexpr (OUT == kOutPartial) hb = b_setup(it - 1, b, true);
        else ha = a_setup(it - 1, b);
      }
      f32x4 br[9];
      // the dO^T operands of each chain are read one chain ahead (and the
      // KV fragments kPF steps ahead): the scheduling barriers keep those
      // LDS reads in front of the MFMAs that do not need them yet
      bf16x8 od0, od1;
      if constexpr (PB) {
        od0 = dot_op(0, 0);
        od1 = dot_op(0, 1);
      }
#pragma unroll
      for (int kk = 0; kk < 18; ++kk) {
        if (PB && (kk & 1) == 0) {
          const int cc = kk >> 1;
          if constexpr (OUT == kOutPartial)
            br[cc] = b_chain(hb, cc, cc < kDotLds ? od0 : dot_op(cc, 0), cc < kDotLds ? od1 : dot_op(cc, 1));
          else
            br[cc] = a_chain(ha, cc, cc < kDotLds ? od0 : dot_op(cc, 0), cc < kDotLds ? od1 : dot_op(cc, 1));
          if (cc + 1 < kDotLds) {
            od0 = dot_op(cc + 1, 0);
            od1 = dot_op(cc + 1, 1);
          }
          if constexpr (OUT == kOutPartial) {
            if (cc >= 2 && (cc & 1) == 0) b_put_pair(hb, cc - 2, br[cc - 2], br[cc - 1]);
          } else {
            if (cc >= 2) a_add(ha, cc - 2, br[cc - 2]);
          }
        }
        if (kk + kPF < 18) {
          const int k2 = kk + kPF;
          f[k2 % (kPF + 1)] = *reinterpret_cast<const bf16x8*>(&kvb[off + (k2 >> 1) * kSegElems + (k2 & 1) * 32]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (b == 0 && (kk & 1) == 0) {
          // next tile's rows: one direct load every other step (for the
          // last tile a harmless reload into the free buffer)
          const int sg = kk >> 1;
          load_lds16(gsrc + sg * 64, gdst + sg * kSegElems);
        }
        const bf16x8 a = f[kk % (kPF + 1)];
        S = F::mma(a, QA[kk], S);
        if (kk < 16) dP = F::mma(a, dOA[kk], dP);
        if (b == 1 && kk == 2) softmax_grad(0, Sh0, Ph0);
      }
      if constexpr (PB) {
        if constexpr (OUT == kOutPartial) {
          b_put_single(hb, 8, br[8]);
        } else {
          a_add(ha, 7, br[7]);
          a_add(ha, 8, br[8]);
        }
      }
      if (b == 0) {
        Sh0 = S;
        Ph0 = dP;
      } else {
        softmax_grad(1, S, dP);
      }
    }
    // exchange written: an LDS-only barrier, so the gather stays in flight
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    if constexpr (L1) {
      // wave 0: the four waves' head sums of key `lane % 32`, to the key's
      // virtual position (lanes without a key of the tile: to the dump row)
      if (wv == 0) {
        const int key = lane & 31;
        const float v = sm.l1s[0][key] + sm.l1s[1][key] + sm.l1s[2][key] + sm.l1s[3][key];
        const bool ok = lane < nvalid;
        float* dst = ok ? l1_row + sm.vpos[k0 + key] : reinterpret_cast<float*>(dump) + lane;
        *dst = v;
      }
    }

    // ---- dQ^T[cols][h] += KV^T[cols][keys] (scale dS^T)[keys][h] ---------
    // keys of k-group lq: 4lq..4lq+3 and 16+4lq..16+4lq+3 on both operands
    {
      bf16x8 bt[4];
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
        bt[hb] = join(tr_read(&xw[offX0 + hb * 16]), tr_read(&xw[offX1 + hb * 16]));
      constexpr int kPF = 2;   // transposed KV operands in flight
      bf16x8 fa[kPF + 1];
#pragma unroll
      for (int c = 0; c < kPF; ++c) {
        fa[c] = kvt(kvb, col_block(c) >> 4);
      }
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        if (c + kPF < 9) {
          fa[(c + kPF) % (kPF + 1)] = kvt(kvb, col_block(c + kPF) >> 4);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int hb = 0; hb < 4; ++hb) dQ[c * 4 + hb] = F::mma(fa[c % (kPF + 1)], bt[hb], dQ[c * 4 + hb]);
      }
    }
  };
  for (int pos0 = 0; pos0 < npos; pos0 += kMaxPos) {
  if (pos0 > 0) {
    // the next pass of positions: the previous pass's loads into the tile
    // buffers have landed and every wave is done with its rows, positions,
    // tiles and exchange before they are rewritten
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    int rawp[kRounds];
#pragma unroll
    for (int r = 0; r < kRounds; ++r) {
      const int pos = r * 256 + tid;
      rawp[r] = pos < min(kMaxPos, npos - pos0) ? position_index(p, irow, pos0 + pos, len) : -1;
    }
    cnt = compact_loaded(p, s, rawp, min(kMaxPos, npos - pos0), sm.rows, sm.wave, sm.vpos, pos0);
    ntiles = (cnt + kNT - 1) / kNT;
    if (ntiles > 0) gather_tile(p, sm, sm.kv, 0, cnt, g, wv, lane);
  }
  if (ntiles > 0) step(std::false_type{}, sm.kv, sm.kv + kTileElems, 0);
  for (int it = 1; it < ntiles; ++it) {
    const bf16* b0 = sm.kv + (it & 1) * kTileElems;
    bf16* b1 = sm.kv + ((it + 1) & 1) * kTileElems;
    step(std::true_type{}, b0, b1, it);
  }

  // phase B of the pass's last tile
  if (ntiles > 0) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 br[9];
      if constexpr (OUT == kOutPartial) {
        const BHalf h = b_setup(ntiles - 1, kb, true);
#pragma unroll
        for (int cc = 0; cc < 9; ++cc) {
          br[cc] = b_chain(h, cc, dot_op(cc, 0), dot_op(cc, 1));
          if (cc >= 2 && (cc & 1) == 0) b_put_pair(h, cc - 2, br[cc - 2], br[cc - 1]);
        }
        b_put_single(h, 8, br[8]);
      } else {
        const AHalf h = a_setup(ntiles - 1, kb);
#pragma unroll
        for (int cc = 0; cc < 9; ++cc) {
          br[cc] = a_chain(h, cc, dot_op(cc, 0), dot_op(cc, 1));
          if (cc >= 2) a_add(h, cc - 2, br[cc - 2]);
        }
        a_add(h, 7, br[7]);
        a_add(h, 8, br[8]);
      }
    }
  }
  }   // passes of positions
  // no direct load may still be writing this workgroup's LDS when it ends
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- dQ (already scaled: the exchange holds scale dS) -------------------
  // The 64 heads' rows of the token are contiguous in dq: they go through
  // LDS (the tile buffers, free once every wave is past its last dQ
  // product) so that every store writes 16 contiguous bytes per lane and
  // whole lines per instruction, instead of 8 bytes of 16 rows apart.
  // lane: columns col_block(c) + 4lq .. +3 of head 16hb + l16
  __syncthreads();
  bf16* sq = sm.kv;   // [head][kKS]
#pragma unroll
  for (int c = 0; c < 9; ++c) {
#pragma unroll
    for (int hb = 0; hb < 4; ++hb) {
      const f32x4 v = dQ[c * 4 + hb] * kInvX;
      typedef short i16x4v __attribute__((ext_vector_type(4)));
      i16x4v o = {bf16_bits(F::to16(v[0])), bf16_bits(F::to16(v[1])), bf16_bits(F::to16(v[2])),
                  bf16_bits(F::to16(v[3]))};
      *reinterpret_cast<i16x4v*>(&sq[(hb * 16 + l16) * kKS + col_block(c) + lq * 4]) = o;
    }
  }
  __syncthreads();
  bf16* dqb = w.dq + ((size_t)t * p.Hq + h0) * kDQK;
  constexpr int kRowChunks = kDQK / 8;   // 16-byte pieces of a row
#pragma unroll
  for (int i = 0; i < kHeads * kRowChunks / kThreads; ++i) {
    const int id = i * kThreads + tid;
    const int hh = id / kRowChunks, ch = id - hh * kRowChunks;
    if (hh < gh)   // a missing head has no row
      *reinterpret_cast<uint4*>(dqb + (size_t)hh * kDQK + ch * 8) = *reinterpret_cast<const uint4*>(&sq[hh * kKS + ch * 8]);
  }
}

}  // namespace

// Heads per kv head from which the 64-head kernel (with the missing heads of
// its last group masked) serves a request: any count.  It computes all 64
// heads of a group, but gathers each row and writes each partial row once
// per group, and measured 4.3x faster than the 16-head row kernel even for
// one head (MLA 8K shape: 5.96 against 25.7 ms).
constexpr int kMinHeads = 1;

bool mla_bwd_supported(const Params& p) {
  return p.shared && p.dqk == kDQK && p.dv == kDV && p.G >= kMinHeads && p.select != kSelBlock;
}

int mla_bwd_head_groups(const Params& p) { return (p.G + kHeads - 1) / kHeads; }

template <typename E>
hipError_t launch_bwd_mla_t(const Params& p, const BwdBuffers& w, hipStream_t s) {
  dim3 grid((unsigned)(w.Tc * p.Hkv), (unsigned)mla_bwd_head_groups(p));
  const bool l1 = w.l1 != nullptr;
  switch (w.out) {
    case kOutAtomic:
      if (l1) hipLaunchKernelGGL((mla_bwd_kernel<E, true, kOutAtomic>), grid, dim3(kThreads), 0, s, p, w);
      else hipLaunchKernelGGL((mla_bwd_kernel<E, false, kOutAtomic>), grid, dim3(kThreads), 0, s, p, w);
      break;
    case kOutAtomicXcd:
      if (l1) hipLaunchKernelGGL((mla_bwd_kernel<E, true, kOutAtomicXcd>), grid, dim3(kThreads), 0, s, p, w);
      else hipLaunchKernelGGL((mla_bwd_kernel<E, false, kOutAtomicXcd>), grid, dim3(kThreads), 0, s, p, w);
      break;
    default:
      if (l1) hipLaunchKernelGGL((mla_bwd_kernel<E, true, kOutPartial>), grid, dim3(kThreads), 0, s, p, w);
      else hipLaunchKernelGGL((mla_bwd_kernel<E, false, kOutPartial>), grid, dim3(kThreads), 0, s, p, w);
  }
  return hipGetLastError();
}

hipError_t launch_bwd_mla(const Params& p, const BwdBuffers& w, hipStream_t s) {
  return p.fp16 ? launch_bwd_mla_t<f16>(p, w, s) : launch_bwd_mla_t<bf16>(p, w, s);
}

}  // namespace sa
