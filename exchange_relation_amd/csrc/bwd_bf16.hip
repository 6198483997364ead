// Relation backward, bf16 storage, for gfx950: five dense contractions on
// bf16 MFMA with fp32 accumulation, everything else on the VALU, by
// recomputation (nothing T x T is stored; App. A.3.6 of the Relation paper).
//
// Per entry (1-based i >= j), G_i = dL/dY_i (App. A.1.7), with
// c_i = lambda ln i + LSE_i and Dr_i = G_i . Y_i:
//   U_ij  = scale q_i . k_j                              (MFMA, recomputed)
//   dP_ij = G_i . v_j                                    (MFMA)
//   j < i : sg = sigmoid(U), F = exp(U sg - c_i), dR = F (dP - Dr_i),
//           dU = dR (sg + E (1 - sg)),  E = U sg         (SiLU')
//   j = i : S = sigmoid(U / tau), F = exp(S - LSE_i), dR = F (dP - Dr_i),
//           dU = dR S (1 - S) / tau
//   dV = F^T G,  dK = scale dU^T Q,  dQ = scale dU K     (MFMA)
//
// Work decomposition: a workgroup of 8 waves owns 256 keys of one (b, h),
// each wave 32 keys, and loops over 64-query tiles from its first key to T
// (first key blocks, i.e. the longest loops, are dispatched first; all key
// blocks of a head share an XCD). Scores are computed as S = Q K^T with keys
// on the MFMA N axis, so each lane holds one key and 16 queries; F and dU
// then feed dV^T += G^T F and dK^T += Q^T dU directly as B operands, and dV /
// dK accumulate in registers for the whole loop. All tiles sit in LDS
// row-major; the transposed operands (G^T, Q^T, and the dQ operands) are
// fetched with the gfx950 transposing LDS read, so nothing is stored twice.
// dQ needs the sum over the workgroup's 256 keys: each wave stores its dU
// tile (keys x queries, 8-byte rows of 4 queries), and after a barrier each
// wave forms a 32-query x 16-d share of the tile's dQ with 16x16x32 MFMAs
// (its K fragments stay in registers for the whole kernel) and adds it into
// an fp32 accumulator with hardware float atomics, 16 consecutive floats per
// instruction. The wide key block halves those atomics (they resolve at
// memory across XCDs) relative to 128-key blocks. A finalize kernel scales and rounds dQ to bf16 and reduces
// the dL/dlambda partials; Dr and those partials come from the shared
// preprocess.
//
// Scores use the base-2 domain as in the forward: the fp32 accumulator of
// q . k is multiplied by scale * log2(e), u' = U log2(e), so
// exp(-U) = exp2(-u'), F = exp2(u' sg - c'_i) with c'_i = c_i log2(e).
#include <math.h>

#include <type_traits>

#include "bwd_common.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace rel {
namespace bwdbf16 {

#ifndef REL_BWD_WAVES
#define REL_BWD_WAVES 8
#endif
constexpr int D = 64;          // head width of the tiles and MFMAs (real widths <= 64 zero-padded)
constexpr int NW = REL_BWD_WAVES;  // waves per workgroup (4 or 8)
constexpr int NT = 64 * NW;        // threads per workgroup
constexpr int BK = 32 * NW;        // keys per workgroup
constexpr int QBW = 4 * 4 / NW;    // 16-query blocks of the dQ tile per wave (4 or 2)
constexpr int KST = BK / 32;       // 32-key steps of the dQ contraction
constexpr int BQ = 64;       // queries per tile
constexpr int RS = D + 8;    // row-major q / dY / K tile stride (bf16): 144 B
constexpr int US = BQ + 8;   // dU^T tile stride (bf16): 144 B

// Query tiles are triple-buffered (tile t read, t+1 resident, t+2 landing)
// and the dU^T tile double-buffered, so one barrier per tile suffices. The
// workgroup's K rows pass through ut[1] once, before the loop, on their way
// into registers.
struct __align__(16) Smem {
  uint16_t qr[3][BQ * RS];   // q tile, [query][d]
  uint16_t gr[3][BQ * RS];   // dY tile, [query][d]
  uint16_t ut[2][BK * US];   // dU^T tile, [key][query]
  float cq[3][BQ];           // c'_i = (lambda ln i + LSE_i) log2 e   (+inf past T)
  float lq[3][BQ];           // LSE_i log2 e                           (+inf past T)
  float dr[3][BQ];           // -Dr_i (the dP accumulator's seed)
};
static_assert(US == RS, "the K staging rows reuse a dU^T buffer");

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ bf16x8 cat(uint2 a, uint2 b) {
  return as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
}

// DR: the real head width (48 or 64); HBM rows are DR wide and everything
// past DR is zero in the tiles and never stored.
template <int DR>
__global__ __launch_bounds__(NT, 8 / NW) void bwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dy,
    const float* __restrict__ lse, const float* __restrict__ Dr, float* __restrict__ dq_acc,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int T, int BH, float kscale,
    float scale, float inv_tau, Lam lamp, float* __restrict__ dk32, float* __restrict__ dv32,
    const float* __restrict__ rc, const float* __restrict__ rs, float* __restrict__ part,
    int nbt) {
  __shared__ Smem sm;
  const float lam = lamp.get();
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 31;   // key row of this lane in S / dP; d row in A operands
  const int hf = lane >> 5;  // K-axis half this lane feeds
  const int l16 = lane & 15, g16 = lane >> 4;  // 16-lane group layout (16x16x32, tr16)

  const int L = blockIdx.x;
  const int head = L % BH;
  const int kb = L / BH;  // first key blocks (longest query loops) first
  static_assert(DR % 16 == 0 && DR <= D, "real head width");
  const size_t base = static_cast<size_t>(head) * T * DR;
  const size_t rbase = static_cast<size_t>(head) * T;
  const int kw0 = kb * BK + wave * 32;  // this wave's first key
  const int kj = kw0 + r;               // this lane's key

  // ---- own keys: k and v rows as B operands of S = Q K^T and dP = G V^T
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    uint4 kr4 = make_uint4(0, 0, 0, 0), vr4 = make_uint4(0, 0, 0, 0);
    if (kj < T && 16 * c + hf * 8 < DR) {
      kr4 = *reinterpret_cast<const uint4*>(k + base + static_cast<size_t>(kj) * DR + hf * 8 + 16 * c);
      vr4 = *reinterpret_cast<const uint4*>(v + base + static_cast<size_t>(kj) * DR + hf * 8 + 16 * c);
    }
    kf[c] = as_bf16x8(kr4);
    vf[c] = as_bf16x8(vr4);
  }
  // ---- the workgroup's key rows to LDS (zero past T), staged in ut[1]
  uint16_t* kr = sm.ut[1];
#pragma unroll
  for (int pass = 0; pass < BK * 8 / NT; ++pass) {
    const int c = tid + NT * pass;  // chunks of 16 B
    const int key = kb * BK + (c >> 3);
    const int kr_ = key < T ? key : T - 1;
    const int cc = (c & 7) < DR / 8 ? (c & 7) : 0;  // columns past DR: zero
    u32x4 x = *reinterpret_cast<const u32x4*>(k + base + static_cast<size_t>(kr_) * DR + cc * 8);
    const u32x4 z = {0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(&kr[(c >> 3) * RS + (c & 7) * 8]) = (key < T && (c & 7) < DR / 8) ? x : z;
  }
  __syncthreads();
  // ---- this wave's dQ B operand (K rows, d in [16 dw, 16 dw + 16)) for all
  // the workgroup's keys, kept in registers: k-slot e of step st <-> key
  // 32 st + 8 g16 + e, column d = 16 dw + l16. ut[1] is next written after
  // the loop's first barrier.
  const int dw = wave & 3;         // d block of this wave's dQ share
  const int qw = (wave >> 2) * QBW;  // first 16-query block of this wave's dQ share
  bf16x8 kq[KST];
#pragma unroll
  for (int st = 0; st < KST; ++st) {
    const int k0 = st * 32 + g16 * 8 + (l16 >> 2);
    const int d0 = dw * 16 + 4 * (l16 & 3);
    kq[st] = cat(lds_read_tr16(&kr[k0 * RS + d0]), lds_read_tr16(&kr[(k0 + 4) * RS + d0]));
  }

  f32x16 dv0 = {0}, dv1 = {0}, dk0 = {0}, dk1 = {0};  // dV^T, dK^T: key r, d rows
  float dl_acc = 0.f;  // this lane's dL/dlambda term (its Self entry, diagonal sub-tile)

  // ---- query tile prefetch: q and dY rows, 16 B chunks (2 per thread with 4
  // waves, 1 with 8; chunk c: row c >> 3, d chunk c & 7)
  // (rows past T are read clamped to T - 1 and zeroed when stored)
  constexpr int NCH = BQ * 8 / NT;
  const int c0 = tid, c1 = tid + NT;
  const u32x4 z4 = {0, 0, 0, 0};
  u32x4 pq0, pq1 = z4, pg0, pg1 = z4;
  bool ok0 = false, ok1 = false;
  float pc = 0.f, pl = 0.f, pd = 0.f;
  auto fetch = [&](int qt0) {
    const int i0 = qt0 + (c0 >> 3), i1 = qt0 + (c1 >> 3);
    ok0 = i0 < T && (c0 & 7) < DR / 8;
    ok1 = i1 < T && (c1 & 7) < DR / 8;
    const size_t o0 = base + static_cast<size_t>(i0 < T ? i0 : T - 1) * DR +
                      ((c0 & 7) < DR / 8 ? (c0 & 7) : 0) * 8;
    pq0 = *reinterpret_cast<const u32x4*>(q + o0);
    pg0 = *reinterpret_cast<const u32x4*>(dy + o0);
    if (NCH > 1) {
      const size_t o1 = base + static_cast<size_t>(i1 < T ? i1 : T - 1) * DR +
                        ((c1 & 7) < DR / 8 ? (c1 & 7) : 0) * 8;
      pq1 = *reinterpret_cast<const u32x4*>(q + o1);
      pg1 = *reinterpret_cast<const u32x4*>(dy + o1);
    }
    if (tid < BQ) {
      const int i = qt0 + tid;
      if (i < T) {
        const float ls = lse[rbase + i];
        pc = (lam * logf(static_cast<float>(i + 1)) + ls) * kLog2e;
        pl = ls * kLog2e;
        pd = -Dr[rbase + i];
      } else {
        pc = INFINITY;
        pl = INFINITY;
        pd = 0.f;
      }
    }
  };
  auto stash = [&](int b) {
    *reinterpret_cast<u32x4*>(&sm.qr[b][(c0 >> 3) * RS + (c0 & 7) * 8]) = ok0 ? pq0 : z4;
    *reinterpret_cast<u32x4*>(&sm.gr[b][(c0 >> 3) * RS + (c0 & 7) * 8]) = ok0 ? pg0 : z4;
    if (NCH > 1) {
      *reinterpret_cast<u32x4*>(&sm.qr[b][(c1 >> 3) * RS + (c1 & 7) * 8]) = ok1 ? pq1 : z4;
      *reinterpret_cast<u32x4*>(&sm.gr[b][(c1 >> 3) * RS + (c1 & 7) * 8]) = ok1 ? pg1 : z4;
    }
    if (tid < BQ) {
      sm.cq[b][tid] = pc;
      sm.lq[b][tid] = pl;
      sm.dr[b][tid] = pd;
    }
  };

  const int qstart = kb * BK;  // < T
  const int ntile = (T - qstart + BQ - 1) / BQ;
  fetch(qstart);
  stash(0);
  if (ntile > 1) {
    fetch(qstart + BQ);
    stash(1);
  }
  __syncthreads();
  int buf = 0;  // query-tile buffer of tile t (t % 3)
  for (int t = 0; t < ntile; ++t) {
    const int qt0 = qstart + t * BQ;
    const bool more = t + 2 < ntile;
    if (more) fetch(qt0 + 2 * BQ);
    const uint16_t* qr = sm.qr[buf];
    const uint16_t* gr = sm.gr[buf];
    uint16_t* ut = sm.ut[t & 1];

    // One 32-query sub-tile against this wave's 32 keys. DIAG: the sub-tile
    // starts at the wave's first key (qs0 == kw0); queries before a key are
    // masked and the Self entry (query == key) takes the App. A.1.7 form.
    // Otherwise every query follows every key and no entry needs a check.
    auto subtile = [&](const int sub, auto diag_tag) {
      constexpr bool DIAG = decltype(diag_tag)::value;
      uint16_t* urow = &ut[(wave * 32 + r) * US + sub * 32 + hf * 4];
      // per-query constants of this lane's 16 entries: element vi <-> query
      // sub*32 + (vi>>2)*8 + hf*4 + (vi&3) of the tile
      float cc[16];
      f32x16 sc = {0}, dp;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ql = sub * 32 + g4 * 8 + hf * 4;
        const float4 c4 = *reinterpret_cast<const float4*>(&sm.cq[buf][ql]);
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.dr[buf][ql]);
        cc[g4 * 4 + 0] = c4.x; cc[g4 * 4 + 1] = c4.y; cc[g4 * 4 + 2] = c4.z; cc[g4 * 4 + 3] = c4.w;
        dp[g4 * 4 + 0] = d4.x; dp[g4 * 4 + 1] = d4.y; dp[g4 * 4 + 2] = d4.z; dp[g4 * 4 + 3] = d4.w;
      }
      // ---- S = Q K^T and dP - Dr = dY V^T - Dr (32 queries x 32 keys); all
      // operand reads are issued first, and the S chain goes first so that
      // the exponentials can start while dP is still in the matrix unit
      bf16x8 qa[4], ga[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        qa[c] = as_bf16x8(*reinterpret_cast<const uint4*>(&qr[(sub * 32 + r) * RS + hf * 8 + 16 * c]));
        ga[c] = as_bf16x8(*reinterpret_cast<const uint4*>(&gr[(sub * 32 + r) * RS + hf * 8 + 16 * c]));
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[c], kf[c], sc, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < 4; ++c) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[c], vf[c], dp, 0, 0, 0);
      // sc[vi], dp[vi]: key = kw0 + r, query = qs0 + (vi>>2)*8 + hf*4 + (vi&3)

      // Self entry of this lane's key (DIAG): element vself, present in the
      // lane half that holds query r
      float fself = 0.f, uself = 0.f;
      const int vself = ((r >> 3) << 2) + (r & 3);
      const bool mine = hf == ((r >> 2) & 1);
      if (DIAG) {
        float us_ = 0.f, dps = 0.f;
#pragma unroll
        for (int vi = 0; vi < 16; ++vi) {
          us_ = (vi == vself) ? sc[vi] : us_;
          dps = (vi == vself) ? dp[vi] : dps;
        }
        const float ll = sm.lq[buf][sub * 32 + r];
        const float S = fast_rcp(1.0f + fast_exp2(-us_ * kscale * inv_tau));
        fself = fast_exp2(S * kLog2e - ll);
        uself = fself * dps * S * (1.0f - S) * inv_tau;
        // dL/dlambda = sum_i ln(i) dR_ii with dR_ii = F_ii (dP_ii - Dr_i); the
        // row is kw0 + r (this sub-tile's queries start at the wave's keys)
        if (mine) dl_acc += logf(static_cast<float>(kw0 + r + 1)) * fself * dps;
      }

      uint32_t fw[8], uw[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        float f2[2], u2[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int vi = 2 * w + e;
          const float u = sc[vi] * kscale;
          const float sg = fast_rcp(1.0f + fast_exp2(-u));
          const float us = u * sg;  // SiLU(U) log2(e)
          float F = fast_exp2(us - cc[vi]);
          // dR (sg + E (1 - sg)) with E = us ln 2: the SiLU derivative
          float dU = F * dp[vi] * fmaf(fmaf(-us, sg, us), kLn2, sg);
          if (DIAG) {
            const int qq = (vi >> 2) * 8 + hf * 4 + (vi & 3);  // query offset in the sub-tile
            const bool self = mine && vi == vself;
            F = (qq < r) ? 0.f : (self ? fself : F);
            dU = (qq < r) ? 0.f : (self ? uself : dU);
          }
          f2[e] = F;
          u2[e] = dU;
        }
        fw[w] = pack_bf16x2(f2[0], f2[1]);
        uw[w] = pack_bf16x2(u2[0], u2[1]);
      }

      // ---- dV^T += G^T F, dK^T += Q^T dU. B operands: k-slot hf*8 + e of
      // step c <-> query c*16 + (e>>2)*8 + hf*4 + (e&3) = element c*8 + e.
      // A operands (G^T, Q^T: d rows, those queries) by transposing reads:
      // lane (l16, g16) of the 16-lane group reads query row q0 + (l16>>2),
      // columns d0 + 4*(l16&3), so lane i gets queries q0..q0+3 of column
      // d0 + i; d0 = 32*db + 16*(g16&1) makes the column 32*db + (lane&31).
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const bf16x8 fb = as_bf16x8(make_uint4(fw[4 * c], fw[4 * c + 1], fw[4 * c + 2], fw[4 * c + 3]));
        const bf16x8 ub = as_bf16x8(make_uint4(uw[4 * c], uw[4 * c + 1], uw[4 * c + 2], uw[4 * c + 3]));
        const int qrow = sub * 32 + c * 16 + hf * 4 + (l16 >> 2);
        const int dcol = 16 * (g16 & 1) + 4 * (l16 & 3);
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const int o = qrow * RS + db * 32 + dcol;
          const bf16x8 ga = cat(lds_read_tr16(&gr[o]), lds_read_tr16(&gr[o + 8 * RS]));
          const bf16x8 qa = cat(lds_read_tr16(&qr[o]), lds_read_tr16(&qr[o + 8 * RS]));
          if (db == 0) {
            dv0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, fb, dv0, 0, 0, 0);
            dk0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, ub, dk0, 0, 0, 0);
          } else {
            dv1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, fb, dv1, 0, 0, 0);
            dk1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, ub, dk1, 0, 0, 0);
          }
        }
      }
      // ---- dU^T tile ([key][query]): queries g4*8 + hf*4 .. +3 are the
      // words 2*g4 and 2*g4 + 1
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<uint2*>(urow + g4 * 8) = make_uint2(uw[2 * g4], uw[2 * g4 + 1]);
    };
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int qs0 = qt0 + sub * 32;  // first query of this 32-query sub-tile
      if (qs0 + 31 < kw0 || kw0 >= T) {  // every query precedes every key: no entries
        uint16_t* urow = &ut[(wave * 32 + r) * US + sub * 32 + hf * 4];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4)
          *reinterpret_cast<uint2*>(urow + g4 * 8) = make_uint2(0, 0);
      } else if (qs0 == kw0) {
        subtile(sub, std::true_type{});
      } else {
        subtile(sub, std::false_type{});
      }
    }
    // the one barrier per tile: dU^T of tile t complete; every wave is done
    // with tile t-1's query buffer (restaged below) and dU^T buffer
    __syncthreads();

    // ---- dQ[16-query blocks qw .. qw+QBW-1][16 dw .. +15] +=
    // dU (those queries x BK keys) K (BK keys x 16) with 16x16x32 MFMAs.
    // A operand (query l16, keys 8 g16 + e of step st) by transposing reads
    // of dU^T, four 32-key steps in flight: lane (l16, g16) reads key row
    // 32 st + 8 g16 + (l16>>2) (+4), columns 16 qb + 4 (l16&3).
    {
      f32x4 aq[QBW];
#pragma unroll
      for (int b = 0; b < QBW; ++b) aq[b] = f32x4{0, 0, 0, 0};
      constexpr int SG = 4;  // steps per batch of reads
#pragma unroll
      for (int s0 = 0; s0 < KST; s0 += SG) {
        bf16x8 ua[SG][QBW];
#pragma unroll
        for (int i = 0; i < SG; ++i) {
          const int krow = (s0 + i) * 32 + g16 * 8 + (l16 >> 2);
#pragma unroll
          for (int b = 0; b < QBW; ++b) {
            const int o = krow * US + (qw + b) * 16 + 4 * (l16 & 3);
            ua[i][b] = cat(lds_read_tr16(&ut[o]), lds_read_tr16(&ut[o + 4 * US]));
          }
        }
#pragma unroll
        for (int i = 0; i < SG; ++i)
#pragma unroll
          for (int b = 0; b < QBW; ++b)
            aq[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua[i][b], kq[s0 + i], aq[b], 0, 0, 0);
      }
      // aq[b][j]: query qt0 + 16 (qw + b) + 4 g16 + j, d = 16 dw + l16
      // Tile t+2 is staged first: its wait for the prefetch loads then does
      // not also wait for these atomics, which resolve at memory. Its buffer
      // last held tile t-1, which every wave finished before the barrier.
      if (more) stash(buf == 0 ? 2 : buf - 1);
      // 32-bit offsets from the head's base; only the last tile can hold
      // queries past T
      float* __restrict__ dqh = dq_acc + base;
      const bool full = qt0 + BQ <= T;
      if (dw * 16 < DR) {
        if (full) {  // straight-line: no per-lane test
#pragma unroll
          for (int b = 0; b < QBW; ++b) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = qt0 + (qw + b) * 16 + g16 * 4 + j;
              unsafeAtomicAdd(dqh + static_cast<uint32_t>(i * DR + dw * 16 + l16), aq[b][j]);
            }
          }
        } else {
#pragma unroll
          for (int b = 0; b < QBW; ++b) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int i = qt0 + (qw + b) * 16 + g16 * 4 + j;
              if (i < T)
                unsafeAtomicAdd(dqh + static_cast<uint32_t>(i * DR + dw * 16 + l16), aq[b][j]);
            }
          }
        }
      }
    }
    buf = buf == 2 ? 0 : buf + 1;
  }

  // ---- the dL/dlambda terms of this wave's 32 rows: part[head][kw0 / 32]
  if (part) {
    float sdl = dl_acc;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) sdl += __shfl_xor(sdl, o);
    if (lane == 0 && kw0 < T) part[static_cast<size_t>(head) * nbt + kw0 / 32] = sdl;
  }

  // ---- dK = scale * dK^T^T, dV = dV^T^T (key kj, d rows of the accumulators)
  if (kj >= T) return;
  const size_t row = base + static_cast<size_t>(kj) * DR;
  if (dv32) {  // Multi-Head Relation: dV in fp32 for the Givens transpose pass
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + g4 * 8 + hf * 4;
        if (d0 >= DR) continue;
        const f32x16& va = db == 0 ? dv0 : dv1;
        *reinterpret_cast<f32x4*>(dv32 + row + d0) =
            f32x4{va[g4 * 4], va[g4 * 4 + 1], va[g4 * 4 + 2], va[g4 * 4 + 3]};
      }
    }
    if constexpr (DR == 64) if (rc) {
      // dp2 = RoPE^T(scale dK) of this key's position: the rotate-half pairs
      // (d, d + 32) sit in dk0 / dk1 of one lane. The same fp32 operations as
      // the separate transpose pass, rounded once.
      const size_t tr = static_cast<size_t>(kj) * (DR / 2);
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = g4 * 8 + hf * 4;
        const f32x4 c = *reinterpret_cast<const f32x4*>(rc + tr + d0);
        const f32x4 sn = *reinterpret_cast<const f32x4*>(rs + tr + d0);
        float lo[4], hi[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = dk0[g4 * 4 + e] * scale, b2 = dk1[g4 * 4 + e] * scale;
          lo[e] = fmaf(a, c[e], b2 * sn[e]);
          hi[e] = fmaf(-a, sn[e], b2 * c[e]);
        }
        *reinterpret_cast<uint2*>(dk + row + d0) =
            make_uint2(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]));
        *reinterpret_cast<uint2*>(dk + row + d0 + 32) =
            make_uint2(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]));
      }
      return;
    }
#pragma unroll
    for (int db = 0; db < 2; ++db) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d0 = db * 32 + g4 * 8 + hf * 4;
        if (d0 >= DR) continue;
        const f32x16& ka = db == 0 ? dk0 : dk1;
        *reinterpret_cast<f32x4*>(dk32 + row + d0) =
            f32x4{ka[g4 * 4] * scale, ka[g4 * 4 + 1] * scale, ka[g4 * 4 + 2] * scale,
                  ka[g4 * 4 + 3] * scale};
      }
    }
    return;
  }
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + g4 * 8 + hf * 4;
      if (d0 >= DR) continue;
      const f32x16& ka = db == 0 ? dk0 : dk1;
      const f32x16& va = db == 0 ? dv0 : dv1;
      *reinterpret_cast<uint2*>(dk + row + d0) =
          make_uint2(pack_bf16x2(ka[g4 * 4] * scale, ka[g4 * 4 + 1] * scale),
                     pack_bf16x2(ka[g4 * 4 + 2] * scale, ka[g4 * 4 + 3] * scale));
      *reinterpret_cast<uint2*>(dv + row + d0) =
          make_uint2(pack_bf16x2(va[g4 * 4], va[g4 * 4 + 1]), pack_bf16x2(va[g4 * 4 + 2], va[g4 * 4 + 3]));
    }
  }
}

// dq = bf16(scale * accumulator); workgroup 0 also sums the dL/dlambda
// partials of the preprocess in a fixed order (deterministic).
__global__ __launch_bounds__(256) void dq_finalize_kernel(const float4* __restrict__ acc,
                                                          uint2* __restrict__ dq, size_t n4,
                                                          float scale,
                                                          const float* __restrict__ part,
                                                          int npart, float* __restrict__ dlambda) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<size_t>(gridDim.x) * 256) {
    const float4 a = acc[i];
    dq[i] = make_uint2(pack_bf16x2(a.x * scale, a.y * scale), pack_bf16x2(a.z * scale, a.w * scale));
  }
  if (blockIdx.x == 0 && dlambda) {
    __shared__ float red[256];
    float s = 0.f;
#pragma unroll 8
    for (int i = threadIdx.x; i < npart; i += 256) s += part[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (unsigned w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) *dlambda = red[0];
  }
}

}  // namespace bwdbf16

hipError_t launch_bwd_bf16(int B, int H, int T, int D, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* y, const uint16_t* dy,
                           const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                           float* dlambda, void* ws, float scale, float tau, Lam lam,
                           hipStream_t stream, float* dk32, float* dv32, const float* rope_cos,
                           const float* rope_sin, hipEvent_t ev0, hipEvent_t ev1) {
  using namespace bwdbf16;
  const BwdWorkspace w = bwd_workspace_layout(1, B, H, T, D);
  char* wsb = static_cast<char*>(ws);
  float* dq_acc = reinterpret_cast<float*>(wsb + w.off_dq);
  const size_t n4 = static_cast<size_t>(B) * H * T * D / 4;
  const unsigned eg = static_cast<unsigned>(n4 < 4096 * 256 ? (n4 + 255) / 256 : 4096);
  hipError_t e = launch_bwd_pre(1, T, D, q, k, v, y, dy, lse, nullptr, w, wsb, scale, tau,
                                stream);
  if (e != hipSuccess) return e;
  const float* Dr = reinterpret_cast<const float*>(wsb + w.off_dr);
  float* part = reinterpret_cast<float*>(wsb + w.off_part);  // dL/dlambda terms
  const int BH = B * H;
  const int nkb = (T + BK - 1) / BK;
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  if (D == 80) {  // the wider layout of bwd80.hip
    e = launch_bwd80_kernel(B, H, T, q, k, v, dy, lse, Dr, dq_acc, dk, dv, scale, tau, lam, stream,
                            dk32, dv32);
  } else {
    if (D == 48)
      hipLaunchKernelGGL(bwd_bf16_kernel<48>, dim3(static_cast<unsigned>(nkb) * BH), dim3(NT), 0,
                         stream, q, k, v, dy, lse, Dr, dq_acc, dk, dv, T, BH, scale * kLog2e,
                         scale, 1.0f / tau, lam, dk32, dv32, nullptr, nullptr, part,
                         (T + 31) / 32);
    else
      hipLaunchKernelGGL(bwd_bf16_kernel<64>, dim3(static_cast<unsigned>(nkb) * BH), dim3(NT), 0,
                         stream, q, k, v, dy, lse, Dr, dq_acc, dk, dv, T, BH, scale * kLog2e,
                         scale, 1.0f / tau, lam, dk32, dv32, rope_cos, rope_sin, part,
                         (T + 31) / 32);
    e = hipGetLastError();
  }
  if (e != hipSuccess) return e;
  if (ev1 && (e = hipEventRecord(ev1, stream)) != hipSuccess) return e;
  // with fp32 results requested (dv32), dq stays in the accumulator and the
  // caller's transpose pass scales it and reduces the dL/dlambda partials
  if (dv32) return hipSuccess;
  hipLaunchKernelGGL(dq_finalize_kernel, dim3(eg), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(dq_acc), reinterpret_cast<uint2*>(dq), n4,
                     scale, reinterpret_cast<const float*>(wsb + w.off_part), w.npart, dlambda);
  return hipGetLastError();
}

}  // namespace rel
