// Relation forward, bf16 storage, for gfx950 (CDNA4): both dense contractions
// on bf16 MFMA (v_mfma_f32_32x32x16_bf16) with fp32 accumulation, the Self /
// Exchange maps and the online scan on the VALU.
//
// What is computed (Sec. 3.1, Sec. 5.1, App. A.3 of the Relation paper): for
// every query row i, the strictly historical Exchange entries
// E_ij = SiLU(U_ij), j < i, are scanned tile by tile with running (m, l, z);
// the Self entry S_i = sigmoid(U_ii / tau_S) is taken from the diagonal of the
// diagonal tile; the row is completed as in App. A.3.5. The count correction
// -lambda ln i is a per-row constant that cancels in the allocation within
// history (Sec. 4.3), so it is applied once per row in the completion, not
// per entry.
//
// Work decomposition
//   * A workgroup of 4 waves owns a block of 128 query rows of one (b, h);
//     each wave owns 32 rows. Workgroups are dispatched longest-first (the
//     last query blocks of every head first; a grid of at most two per CU
//     pairs each long block with a short one on a CU) and the linear block id keeps all
//     query blocks of a head on the same XCD (ids differ by a multiple of the
//     head count), so K / V of a head are shared through one L2.
//   * Key / value tiles of 64 rows are staged row-major in LDS from
//     registers loaded ahead, one barrier per tile: K in a ring of three
//     (tiles t and t+1 resident while t+2 lands), V double-buffered. The V^T
//     operand of the second contraction is fetched with the gfx950
//     transposing LDS read.
//   * Every tile before the workgroup's own query block is strictly
//     historical for all its rows: those run a loop with no masking at all,
//     software-pipelined so that a wave's score MFMAs for the next 32 keys
//     are in flight while it works through the exponentials of the current
//     32 (the matrix unit and the VALU otherwise take turns).
//     Only the last two tiles (the block's diagonal) classify each 32-key
//     sub-block per wave as historical, diagonal or beyond the causal range.
//   * Per wave and 32-key sub-block: the score tile is computed transposed,
//     S^T = K Q^T (32 keys x 32 queries), so that each lane holds 16 scores of
//     ONE query (lane % 32) and the accumulator feeds the second MFMA,
//     Y^T += V^T P^T, directly as its B operand without an LDS round trip;
//     the Y^T accumulator then also holds a single query per lane, so the
//     per-row online rescaling is a per-lane scalar multiply.
//   * Scores are taken to the base-2 domain in fp32 straight off the MFMA
//     accumulator (q and k enter the MFMA exactly as stored):
//     u' = (q . k) * scale * log2(e) = U * log2(e), so
//       exp(-U) = exp2(-u'),  E * log2(e) = u' * sigmoid(U),
//       exp(E - m) = exp2(E * log2(e) - m').
//   * Stabiliser: m' only has to bound E' from above closely enough that no
//     exp2 overflows. SiLU(x) <= max(x, 0), so the running bound only moves
//     (and the accumulators are rescaled) when a tile's raw max u' exceeds it
//     by more than kLazy; otherwise exp2(E' - m') <= 2^kLazy, safe in fp32
//     and bf16.
//   * The row sum l accumulates the bf16-rounded P (v_dot2 with ones), the
//     same values the P V contraction consumes.
//   * SK (a grid of at most one wave even at 64 rows per workgroup): 64-row
//     blocks whose two 32-row groups each split every key tile between two
//     waves, merged before the row completion.
//   * SPLIT (a grid too small to fill the chip, with a caller workspace):
//     long query blocks are cut over their historical key tiles into pieces
//     of at least 16 tiles; the pieces' (acc, m, l) rows are merged by
//     split_combine_kernel (see struct Split and plan_split).
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace rel {
namespace fwdbf16 {

constexpr int NW = 4;             // waves per workgroup
constexpr int BM = 32 * NW;       // query rows per workgroup
constexpr int BN = 64;            // keys per LDS tile
constexpr float kLazy = 8.0f;     // log2-domain slack before rescaling

// Shapes for head dimension DR (a multiple of 16: 48, 64 or 80). The score
// contraction runs DR / 16 K-steps; the P V contraction produces ND blocks of
// 32 value columns, the last one zero-padded past DR (the V tile in LDS has
// ND * 32 columns, the padding zeroed once). HBM rows are DR wide.
template <int DR>
struct Dims {
  static constexpr int D = DR;
  static constexpr int NQ = DR / 16;                  // score K-steps
  static constexpr int ND = (DR + 31) / 32;           // value column blocks
  static constexpr int KS = DR + 8;                   // K tile row stride (bf16), 16 B aligned
  static constexpr int VS = ND * 32 + 8;              // V tile row stride (bf16)
  static constexpr int CPR = DR / 8;                  // 16 B chunks per row
  static constexpr int NCH = (BN * CPR + 255) / 256;  // chunks per thread per tile
  static_assert(DR % 16 == 0, "head dimension must be a multiple of 16");
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

// Per-lane running state of one query row (this lane's half of the keys).
template <int ND>
struct RowState {
  f32x16 acc[ND];     // Y^T: d in [32 db, 32 db + 32)
  float m;            // log2-domain stabiliser (upper bound of E' up to 2^kLazy)
  float mlim;         // m + kLazy
  float lsum;         // sum of bf16(P) over this lane's keys
  float uself;        // u'_ii, valid in the lane that met the diagonal
  bool has_self;
};

// Score tile of 32-key sub-block `sb` of the K tile at `ks`: S^T = K Q^T.
// Element vi of the result is key k0 + (vi>>2)*8 + hf*4 + (vi&3), query
// q0 + r (raw q . k).
template <int DR>
struct KFrag {
  bf16x8 k[Dims<DR>::NQ];
};
template <int DR>
__device__ __forceinline__ KFrag<DR> load_kfrag(const uint16_t* ks, int sb, int r, int hf) {
  constexpr int NQ = Dims<DR>::NQ, KS = Dims<DR>::KS;
  KFrag<DR> f;
#pragma unroll
  for (int c = 0; c < NQ; ++c)
    f.k[c] = as_bf16x8(*reinterpret_cast<const uint4*>(&ks[(sb * 32 + r) * KS + hf * 8 + 16 * c]));
  return f;
}
template <int DR>
__device__ __forceinline__ f32x16 score_from(const KFrag<DR>& f, const bf16x8 (&qf)[Dims<DR>::NQ]) {
  f32x16 s = {0};
#pragma unroll
  for (int c = 0; c < Dims<DR>::NQ; ++c)
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.k[c], qf[c], s, 0, 0, 0);
  return s;
}
template <int DR>
__device__ __forceinline__ f32x16 score(const uint16_t* ks, int sb,
                                        const bf16x8 (&qf)[Dims<DR>::NQ], int r, int hf) {
  constexpr int NQ = Dims<DR>::NQ, KS = Dims<DR>::KS;
  bf16x8 kr[NQ];
#pragma unroll
  for (int c = 0; c < NQ; ++c)
    kr[c] = as_bf16x8(*reinterpret_cast<const uint4*>(&ks[(sb * 32 + r) * KS + hf * 8 + 16 * c]));
  f32x16 s = {0};
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[c], qf[c], s, 0, 0, 0);
  }
  return s;
}

// First half of consuming a score tile: scaling to u' (in place); DIAG (the
// sub-block reaches this lane's query) masks keys j >= i and captures the
// Self score, with rd = the lane's query position minus the sub-block's
// first key (rd = r when the sub-block starts at the wave's first query);
// then the stabiliser moves if the tile's largest bound exceeds it by more
// than kLazy (rare), rescaling the row's accumulators.
template <bool DIAG, int ND>
__device__ __forceinline__ void stabilise(f32x16& s, float qscale, int rd, int hf,
                                          RowState<ND>& st) {
#pragma unroll
  for (int vi = 0; vi < 16; ++vi) s[vi] *= qscale;
  if (DIAG) {
    const int vself = ((rd >> 3) << 2) + (rd & 3);
    const bool mine = rd >= 0 && rd < 32 && hf == ((rd >> 2) & 1);
#pragma unroll
    for (int vi = 0; vi < 16; ++vi) {
      if (mine && vi == vself) st.uself = s[vi];
      const int kk = (vi >> 2) * 8 + hf * 4 + (vi & 3);
      if (kk >= rd) s[vi] = -INFINITY;  // not strictly historical
    }
    st.has_self = st.has_self || mine;
  }
  float mx = vmax(vmax(s[0], s[1]), s[2]);
#pragma unroll
  for (int vi = 3; vi < 15; vi += 2) mx = vmax(vmax(mx, s[vi]), s[vi + 1]);
  mx = vmax(mx, s[15]);
  mx = max_across_halves(mx);
  const bool grow = mx > st.mlim;
  if (__any(grow)) {  // rare: move the stabiliser, rescale this row
    const float mn = grow ? mx : st.m;
    const float a = fast_exp2(st.m - mn);
    st.lsum *= a;
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int vi = 0; vi < 16; ++vi) st.acc[db][vi] *= a;
    st.m = mn;
    st.mlim = mn + kLazy;
  }
}

// Second half: P = exp(E - m) in bf16, the row sum, and Y^T += V^T P^T with
// the V tile at `vs`.
template <bool DIAG, int DR>
__device__ __forceinline__ void accumulate(const uint16_t* vs, int sb, const f32x16& s, int hf,
                                           RowState<Dims<DR>::ND>& st) {
  constexpr int ND = Dims<DR>::ND, VS = Dims<DR>::VS;
  // V^T operands first: their LDS latency runs under the exponentials
  const int l16 = threadIdx.x & 15;
  const int dcol = 16 * ((threadIdx.x >> 4) & 1) + 4 * (l16 & 3);
  uint2 vt[2][ND][2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int o = (sb * 32 + c * 16 + hf * 4 + (l16 >> 2)) * VS + dcol;
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      vt[c][db][0] = lds_read_tr16(&vs[o + 32 * db]);
      vt[c][db][1] = lds_read_tr16(&vs[o + 8 * VS + 32 * db]);
    }
  }
  uint32_t pw[8];
  const bf16x2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    float p2[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const float x = s[2 * w + e];
      const float sg = fast_rcp(1.0f + fast_exp2(-x));
      float p = fast_exp2(fmaf(x, sg, -st.m));
      if (DIAG) p = (x == -INFINITY) ? 0.f : p;
      p2[e] = p;
    }
    pw[w] = pack_bf16x2(p2[0], p2[1]);
    st.lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[w]), one2, st.lsum, false);
  }
  // Y^T += V^T P^T. k-slot hf*8 + e of step c <-> key c*16 + (e>>2)*8 +
  // hf*4 + (e&3) of the sub-block, which is exactly element c*8 + e of P.
  // V^T (d rows, those keys) by transposing reads: lane (l16, group) reads
  // key row k0 + (l16>>2), columns d0 + 4*(l16&3), so lane i gets keys
  // k0..k0+3 of column d0 + i; d0 = 32*db + 16*((lane>>4)&1) makes the
  // column 32*db + (lane&31).
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const bf16x8 pb = as_bf16x8(make_uint4(pw[4 * c], pw[4 * c + 1], pw[4 * c + 2], pw[4 * c + 3]));
#pragma unroll
    for (int db = 0; db < ND; ++db) {
      const uint2 al = vt[c][db][0], ah = vt[c][db][1];
      st.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          as_bf16x8(make_uint4(al.x, al.y, ah.x, ah.y)), pb, st.acc[db], 0, 0, 0);
    }
  }
}

// Rows at an offset (OFF: prefill into a Relation Cache): the T query rows
// of every head (q, y: [BH, T, D]) sit at positions pos0 .. pos0 + T - 1 of
// their sequence, pos0 = p0s[b] (device lengths) or p0 (uniform). Keys and
// values at positions 0 .. pos0 - 1 are the cache's rows (head stride ld
// rows); those at pos0 .. pos0 + T - 1 are the new rows kn / vn ([BH, T, D]),
// which piece 0 of each query block also copies into the cache (no workgroup
// of the launch reads them there). Sequences with pos0 < 0, pos0 > bound or
// pos0 + T > ld get NaN rows and no copy.
struct Seg {
  const int* p0s;
  int p0, bound, ld, H;
  const uint16_t* kn = nullptr;
  const uint16_t* vn = nullptr;
  uint16_t* kc = nullptr;  // the caches (the same buffers as k, v), written
                           // only at rows pos0 .. pos0 + T - 1
  uint16_t* vc = nullptr;
};

// Split over keys (SPLIT): on a grid too small to fill the chip, a query
// block's strictly historical tiles are cut into pieces of spl tiles; piece s
// covers tiles [s spl, min((s + 1) spl, nfull)) and the last piece also the
// block's own tiles (the diagonal and the Self entry). A block of one piece
// completes its rows itself; the pieces of a longer block leave their rows'
// partial scan (acc, m, l and, from the last piece, u'_ii) in `part` for
// split_combine_kernel, which merges them by App. A.3.2's rule.
struct Split {
  float* part;  // [BH][nqb][nsp][BM][D + 4] fp32: acc[D], m, l, u'_ii, unused
  int spl;      // tiles per piece
  int nsp;      // pieces per block in the grid (>= the most any block needs)
};
struct SplitPlan {
  int spl, nsp;  // spl = 0: no split
  size_t bytes;  // workspace for the partial rows
};

template <bool MHR, bool OFF, int DR, bool SPLIT = false, bool SK = false>
__global__ __launch_bounds__(256, DR <= 64 ? 3 : 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ y, float* __restrict__ lse,
    float* __restrict__ gate, int T, int BH, int nqb, float qscale, float inv_tau, Lam lam,
    Mhr mh, Seg sg, Split sp = Split{}) {
  using Dm = Dims<DR>;
  constexpr int D = Dm::D, NQ = Dm::NQ, ND = Dm::ND, KS = Dm::KS, VS = Dm::VS;
  constexpr int CPR = Dm::CPR, NCH = Dm::NCH;
  __shared__ uint16_t kbuf[3][BN * KS];  // K ring: tiles t, t+1 resident, t+2 landing
  __shared__ uint16_t vbuf[2][BN * VS];  // V: tile t resident, t+1 landing
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 31;   // query within the wave's 32 rows / key row in A operands
  const int hf = lane >> 5;  // which half of the K dimension this lane feeds
  // SK (a grid that fits the GPU in one wave even at half the rows per
  // workgroup): blocks of 64 query rows; wave w owns row group w & 1 and, of
  // every key tile, the 32-key sub-block w >> 1, so a block's chain of tiles
  // takes half as long. The two waves of a row group merge their scans
  // before the row completion.
  static_assert(!SK || (!OFF && !SPLIT), "SK is a mode of the aligned, unsplit forward");
  constexpr int BMW = SK ? 64 : BM;  // query rows per workgroup
  const int rgrp = SK ? (wave & 1) : wave;
  const int khalf = SK ? (wave >> 1) : 0;

  const int L = blockIdx.x;
  const int head = L % BH;
  // Longest query blocks first. A grid of at most two workgroups per CU
  // (<= 512) runs in one wave, with workgroups L and L + 256 on one CU; the
  // older of the two issues first, so two long blocks on a CU leave the
  // younger at half speed. There the second half of the grid takes the
  // blocks shortest first, pairing every long block with a short one.
  const int qj = (L / BH) % nqb;
  const int qb = (!SPLIT && !OFF && BH * nqb <= 512 && nqb % 2 == 0 && qj >= nqb / 2)
                     ? qj - nqb / 2
                     : nqb - 1 - qj;
  const int piece = SPLIT ? L / (BH * nqb) : 0;
  const size_t base = static_cast<size_t>(head) * T * D;
  const int q0 = qb * BMW + rgrp * 32;
  const int qi = q0 + r;
  const bool wave_live = q0 < T;
  // keys / values: this head's T rows, or (OFF) the cache's rows
  // 0 .. pos0 + T - 1 with the query rows at positions pos0 + [0, T)
  size_t kvbase = base;
  int pos0 = 0, Tk = T;
  if (OFF) {
    pos0 = sg.p0s ? sg.p0s[head / sg.H] : sg.p0;
    if (pos0 < 0 || pos0 > sg.bound || pos0 + T > sg.ld) {  // out of range: NaN rows
      if (piece != 0) return;
      const int r0 = qb * BM, r1 = min(T, r0 + BM);
      for (int e = tid; e < (r1 - r0) * D; e += 256) y[base + static_cast<size_t>(r0) * D + e] = 0x7fc0;
      for (int i = r0 + tid; i < r1; i += 256) {
        if (lse) lse[static_cast<size_t>(head) * T + i] = NAN;
        if (gate) gate[static_cast<size_t>(head) * T + i] = NAN;
      }
      return;
    }
    kvbase = static_cast<size_t>(head) * sg.ld * D;
    Tk = pos0 + T;
  }
  // Multi-Head Relation: RoPE of this head's query rows, fused into the Q
  // fragment load (keys and values arrive already rotated / mixed; the
  // fragment pairing below needs D = 64)
  const bool rope = MHR && DR == 64 && mh.cos != nullptr;

  // ---- Q fragments: B operands of S^T = K Q^T. Lane holds query r,
  // d = hf*8 + 16*c + [0, 8) for c = 0..3 (rows past T read row T-1 and are
  // zeroed); c and c + 2 hold a RoPE pair (d, d + 32) when D = 64.
  bf16x8 qf[NQ];
  {
    const int qr = qi < T ? qi : T - 1;
    u32x4 raw[NQ];
#pragma unroll
    for (int c = 0; c < NQ; ++c) {
      raw[c] = *reinterpret_cast<const u32x4*>(q + base + static_cast<size_t>(qr) * D + hf * 8 + 16 * c);
      const u32x4 z = {0, 0, 0, 0};
      raw[c] = qi < T ? raw[c] : z;
    }
    if constexpr (DR == 64) if (rope) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const size_t t0 = static_cast<size_t>(qr) * (D / 2) + 16 * c + hf * 8;
        const f32x4 cs[2] = {*reinterpret_cast<const f32x4*>(mh.cos + t0),
                             *reinterpret_cast<const f32x4*>(mh.cos + t0 + 4)};
        const f32x4 sn[2] = {*reinterpret_cast<const f32x4*>(mh.sin + t0),
                             *reinterpret_cast<const f32x4*>(mh.sin + t0 + 4)};
        rope8(raw[c], raw[c + 2], cs, sn);
      }
    }
#pragma unroll
    for (int c = 0; c < NQ; ++c) qf[c] = __builtin_bit_cast(bf16x8, raw[c]);
  }

  RowState<ND> st;
#pragma unroll
  for (int db = 0; db < ND; ++db) st.acc[db] = f32x16{0};
  st.m = 0.f;
  st.mlim = kLazy;
  st.lsum = 0.f;
  st.uself = 0.f;
  st.has_self = false;

  // tiles of keys before the block's first query position are history for
  // every row of the block
  const int kend = min(Tk, pos0 + (qb + 1) * BMW);
  const int ntiles = (kend + BN - 1) / BN;
  const int nfull = (pos0 + qb * BMW) / BN;
  // this workgroup's tiles: historical [kt0, hend), then (last piece) the
  // block's own up to ntiles; tend bounds the look-ahead (nfull < ntiles, so
  // a piece that stops at hend < nfull may stage tile hend unused)
  int kt0 = 0, hend = nfull, tend = ntiles, npc = 1;
  bool last = true;
  if (SPLIT) {
    npc = nfull > 0 ? (nfull + sp.spl - 1) / sp.spl : 1;
    if (piece >= npc) return;
    kt0 = piece * sp.spl;
    last = piece == npc - 1;
    if (!last) {
      hend = kt0 + sp.spl;
      tend = hend + 1;
    }
  }

  // ---- global -> register prefetch: the tile's 16 B chunks c = tid + 256 i
  // (row c / CPR, column chunk c % CPR; i < NCH), as 32-bit offsets from the
  // head's base. Tiles that may run past the keys clamp the row and zero the
  // chunk when it is stored to LDS, so no load waits early and no pointer
  // select turns the loads into generic ones.
  const uint16_t* __restrict__ kh = k + kvbase;
  const uint16_t* __restrict__ vh = v + kvbase;
  // OFF: rows at or after pos0 come from the new rows instead of the cache
  const uint16_t* __restrict__ knh = OFF ? sg.kn + base : kh;
  const uint16_t* __restrict__ vnh = OFF ? sg.vn + base : vh;
  auto rowp = [&](const uint16_t* src, const uint16_t* srcn, uint32_t r0, int col) {
    if constexpr (OFF) {
      const uint32_t p = static_cast<uint32_t>(pos0);
      return r0 < p ? src + (r0 * D + col) : srcn + ((r0 - p) * D + col);
    } else {
      return src + (r0 * D + col);
    }
  };
  // OFF: tile kt lies wholly in the cache (a wave-uniform test), so its rows
  // need no per-row source select
  auto in_cache = [&](int kt) { return !OFF || (kt + 1) * BN <= pos0; };
  int crow[NCH], ccol[NCH];
  uint32_t toff[NCH];  // element offset of the chunk within a tile
  bool cin[NCH];  // chunk exists (BN * CPR need not be a multiple of 256)
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    const int c = tid + 256 * i;
    cin[i] = c < BN * CPR;
    crow[i] = cin[i] ? c / CPR : 0;
    ccol[i] = cin[i] ? c % CPR : 0;
    toff[i] = static_cast<uint32_t>(crow[i] * D + ccol[i] * 8);
  }
  struct Chunks {
    u32x4 a[NCH];
    bool ok[NCH];
  };
  auto fetch = [&](const uint16_t* __restrict__ src, const uint16_t* __restrict__ srcn, int kt,
                   Chunks& c) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int key = kt * BN + crow[i];
      c.ok[i] = cin[i] && key < Tk;
      const uint32_t r0 = static_cast<uint32_t>(key < Tk ? key : Tk - 1);
      c.a[i] = *reinterpret_cast<const u32x4*>(rowp(src, srcn, r0, ccol[i] * 8));
    }
  };
  // a tile wholly inside the keys: no clamp, no zero-fill
  auto fetch_full = [&](const uint16_t* __restrict__ src, const uint16_t* __restrict__ srcn,
                        int kt, Chunks& c) {
    if (in_cache(kt)) {
      // uniform tile base (scalar registers) plus a per-thread offset fixed
      // for the whole loop: no per-tile vector address arithmetic (1-2 %)
      const uint16_t* tb = src + static_cast<uint32_t>(kt * BN * D);
#pragma unroll
      for (int i = 0; i < NCH; ++i) c.a[i] = *reinterpret_cast<const u32x4*>(tb + toff[i]);
    } else {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const uint32_t r0 = static_cast<uint32_t>(kt * BN + crow[i]);
        c.a[i] = *reinterpret_cast<const u32x4*>(rowp(src, srcn, r0, ccol[i] * 8));
      }
    }
  };
  auto stash_full = [&](uint16_t* dst, const Chunks& c, int stride) {
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (cin[i]) *reinterpret_cast<u32x4*>(&dst[crow[i] * stride + ccol[i] * 8]) = c.a[i];
  };
  auto stash = [&](uint16_t* dst, const Chunks& c, int stride) {
    const u32x4 z = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NCH; ++i)
      if (cin[i]) *reinterpret_cast<u32x4*>(&dst[crow[i] * stride + ccol[i] * 8]) = c.ok[i] ? c.a[i] : z;
  };
  if (ND * 32 > DR) {  // zero the V tiles' padding columns once (never stored to again)
    for (int e = tid; e < 2 * BN * (ND * 32 - DR) / 8; e += 256) {
      const int bufi = e / (BN * (ND * 32 - DR) / 8), rem = e % (BN * (ND * 32 - DR) / 8);
      const int rowp = rem / ((ND * 32 - DR) / 8), colp = DR + 8 * (rem % ((ND * 32 - DR) / 8));
      *reinterpret_cast<u32x4*>(&vbuf[bufi][rowp * VS + colp]) = u32x4{0, 0, 0, 0};
    }
  }

  // K tile t lives in kbuf[t % 3], V tile t in vbuf[t % 2]; kp0..kp2 point
  // at K tiles t, t+1, t+2 of the current step.
  uint16_t* kp0 = kbuf[0];
  uint16_t* kp1 = kbuf[1];
  uint16_t* kp2 = kbuf[2];
  Chunks ck, cv;
  {
    Chunks cn;
    fetch(kh, knh, kt0, ck);
    fetch(vh, vnh, kt0, cv);
    if (kt0 + 1 < tend) fetch(kh, knh, kt0 + 1, cn);
    stash(kp0, ck, KS);
    stash(vbuf[0], cv, VS);
    if (kt0 + 1 < tend) stash(kp1, cn, KS);
  }
  __syncthreads();

  // ---- strictly historical tiles, software-pipelined: sub-block 1's score
  // MFMAs run under sub-block 0's exponentials, and the next tile's
  // sub-block 0 score under sub-block 1's (SK: the wave's one sub-block of
  // the next tile under this tile's). No masking.
  f32x16 sa = {0};
  if (kt0 < hend) sa = score<DR>(kp0, khalf, qf, r, hf);
  int kt = kt0;
  KFrag<DR> kn;
  if (!SK && kt0 < hend) kn = load_kfrag<DR>(kp0, 1, r, hf);
  for (; kt < hend; ++kt) {
    const bool more_k = kt + 2 < tend;  // kt + 1 < tend always holds here
    const bool kfull = (kt + 3) * BN <= Tk, vfull = (kt + 2) * BN <= Tk;
    if (more_k) {
      if (kfull) fetch_full(kh, knh, kt + 2, ck);
      else fetch(kh, knh, kt + 2, ck);
    }
    if (vfull) fetch_full(vh, vnh, kt + 1, cv);
    else fetch(vh, vnh, kt + 1, cv);
    const uint16_t* vs = vbuf[(kt - kt0) & 1];
    if constexpr (SK) {
      stabilise<false>(sa, qscale, r, hf, st);
      const f32x16 sn = score<DR>(kp1, khalf, qf, r, hf);  // tile kt + 1 <= nfull is resident
      accumulate<false, DR>(vs, khalf, sa, hf, st);
      sa = sn;
    } else {
      stabilise<false>(sa, qscale, r, hf, st);
      f32x16 sb = score_from<DR>(kn, qf);
      kn = load_kfrag<DR>(kp1, 0, r, hf);  // tile kt + 1 <= nfull is resident
      accumulate<false, DR>(vs, 0, sa, hf, st);
      stabilise<false>(sb, qscale, r, hf, st);
      sa = score_from<DR>(kn, qf);
      kn = load_kfrag<DR>(kp1, 1, r, hf);
      accumulate<false, DR>(vs, 1, sb, hf, st);
    }
    if (more_k) {
      if (kfull) stash_full(kp2, ck, KS);
      else stash(kp2, ck, KS);
    }
    if (vfull) stash_full(vbuf[(kt + 1 - kt0) & 1], cv, VS);
    else stash(vbuf[(kt + 1 - kt0) & 1], cv, VS);
    __syncthreads();
    uint16_t* kfree = kp0;
    kp0 = kp1;
    kp1 = kp2;
    kp2 = kfree;
  }
  // ---- the workgroup's own block: per-wave historical / diagonal /
  // beyond. Aligned rows (pos0 = 0) span at most two tiles, both resident;
  // rows at an offset may span three, so K keeps streaming two tiles ahead.
  for (; last && kt < ntiles; ++kt) {
    const bool more_k = kt + 2 < ntiles;
    if (more_k) fetch(kh, knh, kt + 2, ck);
    if (kt + 1 < ntiles) fetch(vh, vnh, kt + 1, cv);
    const uint16_t* vs = vbuf[(kt - kt0) & 1];
    if (wave_live) {
      const int pw = pos0 + q0;  // position of the wave's first query
#pragma unroll
      for (int sb = 0; sb < 2; ++sb) {
        if (SK && sb != khalf) continue;
        const int k0 = kt * BN + sb * 32;
        if (k0 + 31 < pw) {  // history for every row of the wave
          f32x16 s = score<DR>(kp0, sb, qf, r, hf);
          stabilise<false>(s, qscale, r, hf, st);
          accumulate<false, DR>(vs, sb, s, hf, st);
        } else if (k0 <= pw + 31) {  // reaches the wave's queries: mask + Self
          f32x16 s = score<DR>(kp0, sb, qf, r, hf);
          stabilise<true>(s, qscale, pw + r - k0, hf, st);
          accumulate<true, DR>(vs, sb, s, hf, st);
        }
      }
    }
    if (more_k) stash(kp2, ck, KS);
    if (kt + 1 < ntiles) stash(vbuf[(kt + 1 - kt0) & 1], cv, VS);
    __syncthreads();
    uint16_t* kfree = kp0;
    kp0 = kp1;
    kp1 = kp2;
    kp2 = kfree;
  }

  // OFF: piece 0 appends its query block's new rows to the cache, after its
  // scan so that the copies of the grid's first wave spread out under the
  // compute of the others (all threads of the workgroup are still here)
  if constexpr (OFF) {
    if (piece == 0) {
      const int r0 = qb * BM, r1 = min(T, r0 + BM);
      constexpr int CPR16 = D / 8;  // 16-byte chunks per row
      for (int e = tid; e < (r1 - r0) * CPR16; e += 256) {
        const int rr = r0 + e / CPR16, cc = e % CPR16;
        const size_t from = base + static_cast<size_t>(rr) * D + cc * 8;
        const size_t to = kvbase + static_cast<size_t>(pos0 + rr) * D + cc * 8;
        *reinterpret_cast<u32x4*>(sg.kc + to) = *reinterpret_cast<const u32x4*>(sg.kn + from);
        *reinterpret_cast<u32x4*>(sg.vc + to) = *reinterpret_cast<const u32x4*>(sg.vn + from);
      }
    }
  }
  if constexpr (SK) {
    // Each row group's second key half hands its (acc, m, l, u'_ii) to the
    // first through LDS (the K ring is free after the loops' last barrier);
    // the first merges them by App. A.3.2's rule and completes the rows.
    constexpr int SW = ND * 16 + 4;  // floats per lane: acc, m, l, u'_ii, has_self
    static_assert(128 * SW * sizeof(float) <= sizeof(kbuf), "merge area");
    float* xs = reinterpret_cast<float*>(&kbuf[0][0]) + (rgrp * 64 + lane) * SW;
    if (khalf == 1) {
#pragma unroll
      for (int db = 0; db < ND; ++db)
#pragma unroll
        for (int vi = 0; vi < 16; ++vi) xs[db * 16 + vi] = st.acc[db][vi];
      xs[ND * 16 + 0] = st.m;
      xs[ND * 16 + 1] = st.lsum;
      xs[ND * 16 + 2] = st.uself;
      xs[ND * 16 + 3] = st.has_self ? 1.f : 0.f;
    }
    __syncthreads();
    if (khalf == 1) return;
    const float m1 = xs[ND * 16 + 0];
    const float mx = fmaxf(st.m, m1);  // both bounds start at 0 and only grow
    const float a0 = fast_exp2(st.m - mx), a1 = fast_exp2(m1 - mx);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int vi = 0; vi < 16; ++vi)
        st.acc[db][vi] = fmaf(st.acc[db][vi], a0, xs[db * 16 + vi] * a1);
    st.lsum = fmaf(st.lsum, a0, xs[ND * 16 + 1] * a1);
    st.m = mx;
    if (xs[ND * 16 + 3] != 0.f) {  // the diagonal sat in the second half
      st.uself = xs[ND * 16 + 2];
      st.has_self = true;
    }
  }
  if (!wave_live) return;
  // ---- row completion (App. A.3.5), base-2 domain
  // cross-lane exchanges first, with every lane active, then select
  const float ltot = sum_across_halves(st.lsum);
  const float uo = other_half(st.uself);
  const float us = st.has_self ? st.uself : uo;
  if (qi >= T) return;
  if (SPLIT && npc > 1) {  // partial row for the combine
    float* pr = sp.part + ((((static_cast<size_t>(head) * nqb + qb) * sp.nsp + piece) * BM) +
                           wave * 32 + r) * (D + 4);
#pragma unroll
    for (int db = 0; db < ND; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + g4 * 8 + hf * 4;
        if (d0 < DR)
          *reinterpret_cast<f32x4*>(pr + d0) =
              f32x4{st.acc[db][g4 * 4], st.acc[db][g4 * 4 + 1], st.acc[db][g4 * 4 + 2],
                    st.acc[db][g4 * 4 + 3]};
      }
    if (hf == 0) *reinterpret_cast<f32x4*>(pr + D) = f32x4{st.m, ltot, us, 0.f};
    return;
  }
  const float S = fast_rcp(1.0f + fast_exp2(-us * inv_tau));  // sigmoid(U_ii / tau)
  const float S2 = S * kLog2e;
  float g, lz;
  if (ltot > 0.f) {
    const float A2 = st.m + fast_log2(ltot) - lam.get() * fast_log2(static_cast<float>(pos0 + qi + 1));
    g = fast_rcp(1.0f + fast_exp2(S2 - A2));
    lz = kLn2 * (fmaxf(S2, A2) + fast_log2(1.0f + fast_exp2(-fabsf(S2 - A2))));
  } else {  // row 1: empty history, A = -inf
    g = 0.f;
    lz = S;
  }
  const float gl = (ltot > 0.f) ? g * fast_rcp(ltot) : 0.f;
  const float gs = 1.0f - g;
  const size_t row = base + static_cast<size_t>(qi) * D;
  // I_i, the row's own value. Aligned rows read it from the block's own V
  // tile, still resident in LDS after the loops (tile t sits in
  // vbuf[(t - kt0) & 1] and nothing restages it); OFF reads the new row from
  // HBM, since rows at an offset may span a third tile that the ring no
  // longer holds.
  const uint16_t* vown = OFF ? sg.vn + base + static_cast<size_t>(qi) * D
                             : &vbuf[(qi / BN - kt0) & 1][(qi % BN) * VS];
#pragma unroll
  for (int db = 0; db < ND; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + g4 * 8 + hf * 4;
      if (d0 >= DR) continue;  // padding columns
      const uint2 vr = *reinterpret_cast<const uint2*>(vown + d0);
      const f32x16& acc = st.acc[db];
      const float y0 = fmaf(gs, __uint_as_float(vr.x << 16), gl * acc[g4 * 4 + 0]);
      const float y1 = fmaf(gs, __uint_as_float(vr.x & 0xffff0000u), gl * acc[g4 * 4 + 1]);
      const float y2 = fmaf(gs, __uint_as_float(vr.y << 16), gl * acc[g4 * 4 + 2]);
      const float y3 = fmaf(gs, __uint_as_float(vr.y & 0xffff0000u), gl * acc[g4 * 4 + 3]);
      *reinterpret_cast<uint2*>(y + row + d0) = make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
    }
  }
  if (hf == 0) {
    const size_t ri = static_cast<size_t>(head) * T + qi;
    if (lse) lse[ri] = lz;
    if (gate) gate[ri] = g;
  }
}

}  // namespace fwdbf16

namespace fwdbf16 {

// Merge of a split block's pieces and the row completion (App. A.3.5), one
// thread per (row, 4 value columns). The pieces' scans combine by App.
// A.3.2's rule: M = max m_s, l = sum l_s 2^(m_s - M), acc likewise; the Self
// score comes from the last piece. Rows of blocks the forward kernel
// completed itself (one piece) and rows of out-of-range sequences are left
// alone.
template <int DR>
__global__ __launch_bounds__(256) void split_combine_kernel(
    const float* __restrict__ part, const uint16_t* __restrict__ v, uint16_t* __restrict__ y,
    float* __restrict__ lse, float* __restrict__ gate, int T, int BH, int nqb, float inv_tau,
    Lam lam, Seg sg, Split sp, bool off) {
  constexpr int D = DR, CQ = DR / 4, PW = DR + 4;
  const size_t g = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t row = g / CQ;
  if (row >= static_cast<size_t>(BH) * T) return;
  const int quad = static_cast<int>(g % CQ);
  const int head = static_cast<int>(row / T), qi = static_cast<int>(row % T);
  int pos0 = 0;
  size_t kvbase = static_cast<size_t>(head) * T * D;
  if (off) {
    pos0 = sg.p0s ? sg.p0s[head / sg.H] : sg.p0;
    if (pos0 < 0 || pos0 > sg.bound || pos0 + T > sg.ld) return;
    kvbase = static_cast<size_t>(head) * sg.ld * D;
  }
  const int qb = qi / BM;
  const int nfull = (pos0 + qb * BM) / BN;
  const int npc = nfull > 0 ? (nfull + sp.spl - 1) / sp.spl : 1;
  if (npc == 1) return;
  const float* pr = part + (((static_cast<size_t>(head) * nqb + qb) * sp.nsp) * BM + qi % BM) * PW;
  const size_t ps = static_cast<size_t>(BM) * PW;  // piece stride
  float mx = -INFINITY;
  for (int s = 0; s < npc; ++s) mx = fmaxf(mx, pr[s * ps + D]);
  float l = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s = 0; s < npc; ++s) {
    const f32x4 st = *reinterpret_cast<const f32x4*>(pr + s * ps + D);
    const float a = fast_exp2(st[0] - mx);
    l = fmaf(st[1], a, l);
    const f32x4 u = *reinterpret_cast<const f32x4*>(pr + s * ps + 4 * quad);
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(u[e], a, acc[e]);
  }
  const float us = pr[(npc - 1) * ps + D + 2];
  const float S = fast_rcp(1.0f + fast_exp2(-us * inv_tau));
  const float S2 = S * kLog2e;
  float gt, lz;
  if (l > 0.f) {
    const float A2 = mx + fast_log2(l) - lam.get() * fast_log2(static_cast<float>(pos0 + qi + 1));
    gt = fast_rcp(1.0f + fast_exp2(S2 - A2));
    lz = kLn2 * (fmaxf(S2, A2) + fast_log2(1.0f + fast_exp2(-fabsf(S2 - A2))));
  } else {
    gt = 0.f;
    lz = S;
  }
  const float gl = l > 0.f ? gt * fast_rcp(l) : 0.f;
  const float gs = 1.0f - gt;
  const uint16_t* vo = off ? sg.vn + row * D : v + kvbase + static_cast<size_t>(pos0 + qi) * D;
  const uint2 vr = *reinterpret_cast<const uint2*>(vo + 4 * quad);
  const float y0 = fmaf(gs, __uint_as_float(vr.x << 16), gl * acc[0]);
  const float y1 = fmaf(gs, __uint_as_float(vr.x & 0xffff0000u), gl * acc[1]);
  const float y2 = fmaf(gs, __uint_as_float(vr.y << 16), gl * acc[2]);
  const float y3 = fmaf(gs, __uint_as_float(vr.y & 0xffff0000u), gl * acc[3]);
  *reinterpret_cast<uint2*>(y + row * D + 4 * quad) =
      make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
  if (quad == 0) {
    if (lse) lse[row] = lz;
    if (gate) gate[row] = gt;
  }
}

// Split plan for a grid of BH x nqb query blocks whose rows sit at positions
// up to pbound + [0, T). A grid that already has two workgroups per slot
// (256 CUs x the workgroups resident per CU) is not split. Otherwise pieces
// are sized for about 1.5 per slot: the blocks' total tile work (for
// per-sequence lengths half the bound's, the lengths taken as spread over
// [0, bound]) over 1.5 x the slots, and at least 16 tiles, since a short
// workgroup is dominated by its start (the query fragments and first tiles
// before its first barrier): 6-tile pieces made the 10M-layer forward
// slower, and 20-23-tile pieces were fastest on the ragged cache prefill.
SplitPlan plan_split(int BH, int T, int pbound, bool ragged, int DR) {
  SplitPlan pl{0, 1, 0};
  const int nqb = (T + BM - 1) / BM;
  const long long slots = 256LL * (DR <= 64 ? 3 : 2);
  if (static_cast<long long>(BH) * nqb >= 2 * slots) return pl;
  long long work = 0;
  int nfmax = 0;
  for (int qb = 0; qb < nqb; ++qb) {
    const int nfull = (pbound + qb * BM) / BN;
    const int kend = pbound + min(T, (qb + 1) * BM);
    work += (kend + BN - 1) / BN;
    nfmax = max(nfmax, nfull);
  }
  work *= BH;
  if (ragged) work /= 2;
  const int spl = static_cast<int>(max(16LL, (2 * work + 3 * slots - 1) / (3 * slots)));
  const int nsp = nfmax > 0 ? (nfmax + spl - 1) / spl : 1;
  if (nsp < 2) return pl;
  pl.spl = spl;
  pl.nsp = nsp;
  pl.bytes = static_cast<size_t>(BH) * nqb * nsp * BM * (DR + 4) * sizeof(float);
  return pl;
}

template <int DR>
hipError_t run_fwd(int BH, int H, int T, const uint16_t* q, const uint16_t* k,
                   const uint16_t* v, uint16_t* y, float* lse, float* gate, float scale, float tau,
                   Lam lam, hipStream_t stream, const float* rope_cos, const float* rope_sin,
                   float* ws, size_t ws_bytes) {
  const int nqb = (T + BM - 1) / BM;
  const dim3 grid(static_cast<unsigned>(nqb) * BH);
  const Mhr mh{rope_cos, rope_sin, nullptr, 0, H};
  const Seg sg{nullptr, 0, 0, T, H};
  const SplitPlan pl = ws ? plan_split(BH, T, 0, false, DR) : SplitPlan{0, 1, 0};
  if (rope_cos == nullptr && pl.spl > 0 && ws_bytes >= pl.bytes) {
    const Split sp{ws, pl.spl, pl.nsp};
    hipLaunchKernelGGL((fwd_bf16_kernel<false, false, DR, true>),
                       dim3(static_cast<unsigned>(nqb) * BH * pl.nsp), dim3(256), 0, stream, q, k,
                       v, y, lse, gate, T, BH, nqb, scale * kLog2e, 1.0f / tau, lam, mh, sg, sp);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t threads = static_cast<size_t>(BH) * T * (DR / 4);
    hipLaunchKernelGGL((split_combine_kernel<DR>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                       dim3(256), 0, stream, ws, v, y, lse, gate, T, BH, nqb, 1.0f / tau, lam, sg,
                       sp, false);
    return hipGetLastError();
  }
  // A grid whose 64-row blocks still fit the GPU in one wave (256 CUs x the
  // workgroups resident per CU) takes the SK mode: half the rows per
  // workgroup, twice the workgroups, each block's chain of tiles halved.
  // (Query RoPE is fused into the fragment load at D = 64 only; at 48 / 80
  // the Multi-Head Relation pre-pass has rotated q already.)
  const long long nqb64 = (T + 63) / 64;
  const bool qrope = rope_cos != nullptr && DR == 64;
  if (nqb64 * BH <= 256LL * (DR <= 64 ? 3 : 2)) {
    const dim3 g64(static_cast<unsigned>(nqb64 * BH));
    if (qrope)
      hipLaunchKernelGGL((fwd_bf16_kernel<true, false, DR, false, true>), g64, dim3(256), 0,
                         stream, q, k, v, y, lse, gate, T, BH, static_cast<int>(nqb64),
                         scale * kLog2e, 1.0f / tau, lam, mh, sg);
    else
      hipLaunchKernelGGL((fwd_bf16_kernel<false, false, DR, false, true>), g64, dim3(256), 0,
                         stream, q, k, v, y, lse, gate, T, BH, static_cast<int>(nqb64),
                         scale * kLog2e, 1.0f / tau, lam, mh, sg);
  } else if (!qrope)
    hipLaunchKernelGGL((fwd_bf16_kernel<false, false, DR>), grid, dim3(256), 0, stream, q, k, v,
                       y, lse, gate, T, BH, nqb, scale * kLog2e, 1.0f / tau, lam, mh, sg);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<true, false, DR>), grid, dim3(256), 0, stream, q, k, v,
                       y, lse, gate, T, BH, nqb, scale * kLog2e, 1.0f / tau, lam, mh, sg);
  return hipGetLastError();
}

// Appends the m new tokens of every (b, h) to cache slots n_b .. n_b + m - 1
// (an exact 16-bit copy); sequences out of range are left untouched.
template <int DR>
hipError_t run_prefill(int BH, int H, int m, const uint16_t* q, const uint16_t* k_new,
                       const uint16_t* v_new, uint16_t* k_cache, uint16_t* v_cache, int capacity,
                       const int* n_hist_dev, int n_hist, uint16_t* y, float* lse, float* gate,
                       float scale, float tau, float lam, hipStream_t stream, float* ws,
                       size_t ws_bytes) {
  const int nqb = (m + BM - 1) / BM;
  const Mhr mh{nullptr, nullptr, nullptr, 0, H};
  // the kernel reads the new rows from k_new / v_new and appends them itself
  const Seg sg{n_hist_dev, n_hist, n_hist, capacity, H, k_new, v_new, k_cache, v_cache};
  hipError_t e;
  const SplitPlan pl =
      ws ? plan_split(BH, m, n_hist, n_hist_dev != nullptr, DR) : SplitPlan{0, 1, 0};
  if (pl.spl > 0 && ws_bytes >= pl.bytes) {
    const Split sp{ws, pl.spl, pl.nsp};
    hipLaunchKernelGGL((fwd_bf16_kernel<false, true, DR, true>),
                       dim3(static_cast<unsigned>(nqb) * BH * pl.nsp), dim3(256), 0, stream, q,
                       k_cache, v_cache, y, lse, gate, m, BH, nqb, scale * kLog2e, 1.0f / tau, lam,
                       mh, sg, sp);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const size_t threads = static_cast<size_t>(BH) * m * (DR / 4);
    hipLaunchKernelGGL((split_combine_kernel<DR>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                       dim3(256), 0, stream, ws, v_cache, y, lse, gate, m, BH, nqb, 1.0f / tau,
                       lam, sg, sp, true);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<false, true, DR>), dim3(static_cast<unsigned>(nqb) * BH),
                     dim3(256), 0, stream, q, k_cache, v_cache, y, lse, gate, m, BH, nqb,
                     scale * kLog2e, 1.0f / tau, lam, mh, sg);
  return hipGetLastError();
}
}  // namespace fwdbf16

size_t fwd_bf16_workspace_bytes(int B, int H, int T, int D) {
  return fwdbf16::plan_split(B * H, T, 0, false, D).bytes;
}

size_t prefill_workspace_bytes(int B, int H, int D, int m, int n_hist, bool per_sequence) {
  return fwdbf16::plan_split(B * H, m, n_hist, per_sequence, D).bytes;
}

hipError_t launch_fwd_bf16(int B, int H, int T, int D, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, uint16_t* y, float* lse, float* gate, float scale,
                           float tau, Lam lam, hipStream_t stream, const float* rope_cos,
                           const float* rope_sin, float* ws, size_t ws_bytes) {
  const int BH = B * H;
  if (D == 48)
    return fwdbf16::run_fwd<48>(BH, H, T, q, k, v, y, lse, gate, scale, tau, lam, stream,
                                rope_cos, rope_sin, ws, ws_bytes);
  if (D == 80)
    return fwdbf16::run_fwd<80>(BH, H, T, q, k, v, y, lse, gate, scale, tau, lam, stream,
                                rope_cos, rope_sin, ws, ws_bytes);
  return fwdbf16::run_fwd<64>(BH, H, T, q, k, v, y, lse, gate, scale, tau, lam, stream, rope_cos,
                              rope_sin, ws, ws_bytes);
}

hipError_t launch_prefill_bf16(int B, int H, int D, int m, const uint16_t* q,
                               const uint16_t* k_new, const uint16_t* v_new, uint16_t* k_cache,
                               uint16_t* v_cache, int capacity, const int* n_hist_dev, int n_hist,
                               uint16_t* y, float* lse, float* gate, float scale, float tau,
                               float lam, hipStream_t stream, float* ws, size_t ws_bytes) {
  const int BH = B * H;
  if (D == 48)
    return fwdbf16::run_prefill<48>(BH, H, m, q, k_new, v_new, k_cache, v_cache, capacity,
                                    n_hist_dev, n_hist, y, lse, gate, scale, tau, lam, stream, ws,
                                    ws_bytes);
  if (D == 80)
    return fwdbf16::run_prefill<80>(BH, H, m, q, k_new, v_new, k_cache, v_cache, capacity,
                                    n_hist_dev, n_hist, y, lse, gate, scale, tau, lam, stream, ws,
                                    ws_bytes);
  return fwdbf16::run_prefill<64>(BH, H, m, q, k_new, v_new, k_cache, v_cache, capacity,
                                  n_hist_dev, n_hist, y, lse, gate, scale, tau, lam, stream, ws,
                                  ws_bytes);
}

}  // namespace rel
