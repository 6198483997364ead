// Relation backward for head width 80 (the paper's 100M model), bf16
// storage. The same recomputation and the same five contractions as
// bwd_bf16.hip (see there for the formulas, App. A.1.7 of the Relation
// paper), laid out for the wider head:
//  * four waves of 32 keys per workgroup (128 keys) and one wave per SIMD, so
//    that a wave may hold up to 512 registers: the dV^T / dK^T accumulators
//    (three 32-column blocks each, 96 wide, the last half zero) live in the
//    accumulation registers next to the five K-step fragments of its keys;
//  * q / dY / K tiles 96 columns wide in LDS, columns 80..95 zero (written
//    once), so the 32-column operand reads of the last block need no checks;
//  * the score contractions step over the real 80 columns (five 16-deep
//    steps);
//  * dQ: each wave forms one 16-query block of the tile's dQ over all five
//    16-column blocks, with K read from the resident K tile.
#include <math.h>

#include <type_traits>

#include "bwd_common.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace rel {
namespace bwd80 {

constexpr int DR = 80;        // real head width
constexpr int NQ = DR / 16;   // score K-steps
constexpr int NDB = 3;        // 32-column output blocks
constexpr int TW = NDB * 32;  // tile width (columns DR..TW-1 zero)
constexpr int NW = 4;         // waves per workgroup
constexpr int NT = 64 * NW;
constexpr int BK = 32 * NW;   // keys per workgroup
constexpr int KST = BK / 32;  // 32-key steps of the dQ contraction
constexpr int BQ = 64;        // queries per tile
constexpr int RS = TW + 8;    // q / dY / K tile row stride (bf16): 208 B
constexpr int US = BQ + 8;    // dU^T tile stride (bf16)
constexpr int CPR = DR / 8;   // 16 B chunks of real data per row
constexpr int NDQ = DR / 16;  // 16-column blocks of dQ

struct __align__(16) Smem {
  uint16_t qr[3][BQ * RS];   // q tile, [query][d]
  uint16_t gr[3][BQ * RS];   // dY tile, [query][d]
  uint16_t ut[2][BK * US];   // dU^T tile, [key][query]
  uint16_t kt[BK * RS];      // this workgroup's K rows, [key][d]
  float cq[3][BQ];           // c'_i = (lambda ln i + LSE_i) log2 e   (+inf past T)
  float lq[3][BQ];           // LSE_i log2 e                           (+inf past T)
  float dr[3][BQ];           // -Dr_i
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }
__device__ __forceinline__ bf16x8 cat(uint2 a, uint2 b) {
  return as_bf16x8(make_uint4(a.x, a.y, b.x, b.y));
}

__global__ __launch_bounds__(NT, 1) void bwd80_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dy,
    const float* __restrict__ lse, const float* __restrict__ Dr, float* __restrict__ dq_acc,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int T, int BH, float kscale,
    float scale, float inv_tau, Lam lamp, float* __restrict__ dk32, float* __restrict__ dv32) {
  const float lam = lamp.get();
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 31;   // key row of this lane in S / dP
  const int hf = lane >> 5;  // K-axis half this lane feeds
  const int l16 = lane & 15, g16 = lane >> 4;

  const int L = blockIdx.x;
  const int head = L % BH;
  const int kb = L / BH;  // first key blocks (longest query loops) first
  const size_t base = static_cast<size_t>(head) * T * DR;
  const size_t rbase = static_cast<size_t>(head) * T;
  const int kw0 = kb * BK + wave * 32;
  const int kj = kw0 + r;

  // ---- own keys: k and v rows as B operands of S = Q K^T and dP = G V^T
  bf16x8 kf[NQ], vf[NQ];
#pragma unroll
  for (int c = 0; c < NQ; ++c) {
    uint4 kr4 = make_uint4(0, 0, 0, 0), vr4 = make_uint4(0, 0, 0, 0);
    if (kj < T) {
      kr4 = *reinterpret_cast<const uint4*>(k + base + static_cast<size_t>(kj) * DR + hf * 8 + 16 * c);
      vr4 = *reinterpret_cast<const uint4*>(v + base + static_cast<size_t>(kj) * DR + hf * 8 + 16 * c);
    }
    kf[c] = as_bf16x8(kr4);
    vf[c] = as_bf16x8(vr4);
  }
  // ---- the workgroup's K rows (zero past T) and the zero columns of the
  // q / dY tiles
  {
    const u32x4 z = {0, 0, 0, 0};
    for (int c = tid; c < BK * (TW / 8); c += NT) {
      const int key = kb * BK + c / (TW / 8), ch = c % (TW / 8);
      u32x4 x = z;
      if (key < T && ch < CPR) x = *reinterpret_cast<const u32x4*>(k + base + static_cast<size_t>(key) * DR + ch * 8);
      *reinterpret_cast<u32x4*>(&sm.kt[(c / (TW / 8)) * RS + ch * 8]) = x;
    }
    for (int c = tid; c < 3 * BQ * (TW / 8 - CPR); c += NT) {
      const int b = c / (BQ * (TW / 8 - CPR)), rest = c % (BQ * (TW / 8 - CPR));
      const int row = rest / (TW / 8 - CPR), ch = CPR + rest % (TW / 8 - CPR);
      *reinterpret_cast<u32x4*>(&sm.qr[b][row * RS + ch * 8]) = z;
      *reinterpret_cast<u32x4*>(&sm.gr[b][row * RS + ch * 8]) = z;
    }
  }

  f32x16 dva[NDB], dka[NDB];  // dV^T, dK^T: key r, d rows 32 db ..
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
    dva[db] = f32x16{0};
    dka[db] = f32x16{0};
  }

  // ---- query tile prefetch: q and dY rows in 16 B chunks (BQ * CPR chunks,
  // up to three per thread); rows past T are read clamped and zeroed
  constexpr int NCH = (BQ * CPR + NT - 1) / NT;
  const u32x4 z4 = {0, 0, 0, 0};
  u32x4 pq[NCH], pg[NCH];
  bool okc[NCH];
  float pc = 0.f, pl = 0.f, pd = 0.f;
  auto fetch = [&](int qt0) {
#pragma unroll
    for (int p = 0; p < NCH; ++p) {
      const int c = tid + NT * p;
      const int cc = c < BQ * CPR ? c : 0;
      const int i = qt0 + cc / CPR;
      okc[p] = c < BQ * CPR && i < T;
      const size_t o = base + static_cast<size_t>(i < T ? i : T - 1) * DR + (cc % CPR) * 8;
      pq[p] = *reinterpret_cast<const u32x4*>(q + o);
      pg[p] = *reinterpret_cast<const u32x4*>(dy + o);
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
#pragma unroll
    for (int p = 0; p < NCH; ++p) {
      const int c = tid + NT * p;
      if (c < BQ * CPR) {
        const int o = (c / CPR) * RS + (c % CPR) * 8;
        *reinterpret_cast<u32x4*>(&sm.qr[b][o]) = okc[p] ? pq[p] : z4;
        *reinterpret_cast<u32x4*>(&sm.gr[b][o]) = okc[p] ? pg[p] : z4;
      }
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
  int buf = 0;
  for (int t = 0; t < ntile; ++t) {
    const int qt0 = qstart + t * BQ;
    const bool more = t + 2 < ntile;
    if (more) fetch(qt0 + 2 * BQ);
    const uint16_t* qr = sm.qr[buf];
    const uint16_t* gr = sm.gr[buf];
    uint16_t* ut = sm.ut[t & 1];

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
      bf16x8 qa[NQ], ga[NQ];
#pragma unroll
      for (int c = 0; c < NQ; ++c) {
        qa[c] = as_bf16x8(*reinterpret_cast<const uint4*>(&qr[(sub * 32 + r) * RS + hf * 8 + 16 * c]));
        ga[c] = as_bf16x8(*reinterpret_cast<const uint4*>(&gr[(sub * 32 + r) * RS + hf * 8 + 16 * c]));
      }
#pragma unroll
      for (int c = 0; c < NQ; ++c) sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[c], kf[c], sc, 0, 0, 0);
#pragma unroll
      for (int c = 0; c < NQ; ++c) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga[c], vf[c], dp, 0, 0, 0);
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
        for (int db = 0; db < NDB; ++db) {
          const int o = qrow * RS + db * 32 + dcol;
          const bf16x8 ga = cat(lds_read_tr16(&gr[o]), lds_read_tr16(&gr[o + 8 * RS]));
          const bf16x8 qa = cat(lds_read_tr16(&qr[o]), lds_read_tr16(&qr[o + 8 * RS]));
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ga, fb, dva[db], 0, 0, 0);
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, ub, dka[db], 0, 0, 0);
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

    // ---- dQ[16-query block `wave`][all 80 columns] += dU (those queries x
    // BK keys) K (BK keys x 80) with 16x16x32 MFMAs: A from dU^T, B from the
    // resident K tile, both by transposing reads
    {
      f32x4 aq[NDQ];
#pragma unroll
      for (int b = 0; b < NDQ; ++b) aq[b] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < KST; ++st) {
        const int krow = st * 32 + g16 * 8 + (l16 >> 2);
        const int ou = krow * US + wave * 16 + 4 * (l16 & 3);
        const bf16x8 ua = cat(lds_read_tr16(&ut[ou]), lds_read_tr16(&ut[ou + 4 * US]));
#pragma unroll
        for (int b = 0; b < NDQ; ++b) {
          const int ok_ = krow * RS + b * 16 + 4 * (l16 & 3);
          const bf16x8 kb_ = cat(lds_read_tr16(&sm.kt[ok_]), lds_read_tr16(&sm.kt[ok_ + 4 * RS]));
          aq[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ua, kb_, aq[b], 0, 0, 0);
        }
      }
      // aq[b][j]: query qt0 + 16 wave + 4 g16 + j, d = 16 b + l16
      if (more) stash(buf == 0 ? 2 : buf - 1);
      float* __restrict__ dqh = dq_acc + base;
      const bool full = qt0 + BQ <= T;
#pragma unroll
      for (int b = 0; b < NDQ; ++b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = qt0 + wave * 16 + g16 * 4 + j;
          if (full || i < T) unsafeAtomicAdd(dqh + static_cast<uint32_t>(i * DR + b * 16 + l16), aq[b][j]);
        }
      }
    }
    buf = buf == 2 ? 0 : buf + 1;
  }

  // ---- dK = scale * dK^T^T, dV = dV^T^T (key kj, d rows of the accumulators)
  if (kj >= T) return;
  const size_t row = base + static_cast<size_t>(kj) * DR;
#pragma unroll
  for (int db = 0; db < NDB; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + g4 * 8 + hf * 4;
      if (d0 >= DR) continue;  // zero padding columns
      const f32x16& ka = dka[db];
      const f32x16& va = dva[db];
      if (dk32) {  // fp32 results for a later pass (Multi-Head Relation's transposes)
        *reinterpret_cast<f32x4*>(dk32 + row + d0) =
            f32x4{ka[g4 * 4] * scale, ka[g4 * 4 + 1] * scale, ka[g4 * 4 + 2] * scale,
                  ka[g4 * 4 + 3] * scale};
        *reinterpret_cast<f32x4*>(dv32 + row + d0) =
            f32x4{va[g4 * 4], va[g4 * 4 + 1], va[g4 * 4 + 2], va[g4 * 4 + 3]};
      } else {
        *reinterpret_cast<uint2*>(dk + row + d0) =
            make_uint2(pack_bf16x2(ka[g4 * 4] * scale, ka[g4 * 4 + 1] * scale),
                       pack_bf16x2(ka[g4 * 4 + 2] * scale, ka[g4 * 4 + 3] * scale));
        *reinterpret_cast<uint2*>(dv + row + d0) =
            make_uint2(pack_bf16x2(va[g4 * 4], va[g4 * 4 + 1]), pack_bf16x2(va[g4 * 4 + 2], va[g4 * 4 + 3]));
      }
    }
  }
}

}  // namespace bwd80

hipError_t launch_bwd80_kernel(int B, int H, int T, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const uint16_t* dy, const float* lse,
                               const float* Dr, float* dq_acc, uint16_t* dk, uint16_t* dv,
                               float scale, float tau, Lam lam, hipStream_t stream, float* dk32,
                               float* dv32) {
  using namespace bwd80;
  const int BH = B * H;
  const int nkb = (T + BK - 1) / BK;
  hipLaunchKernelGGL(bwd80_kernel, dim3(static_cast<unsigned>(nkb) * BH), dim3(NT), 0, stream, q, k,
                     v, dy, lse, Dr, dq_acc, dk, dv, T, BH, scale * kLog2e, scale, 1.0f / tau, lam,
                     dk32, dv32);
  return hipGetLastError();
}

}  // namespace rel
