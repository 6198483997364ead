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
// Work decomposition: a workgroup of 4 waves owns 128 keys of one (b, h),
// each wave 32 keys, and loops over 64-query tiles from its first key to T.
// Scores are computed as S = Q K^T with keys on the MFMA N axis, so each lane
// holds one key and 16 queries; F and dU then feed dV^T += G^T F and
// dK^T += Q^T dU directly as B operands (keys fixed per lane, queries on the
// K axis), and dV / dK accumulate in registers for the whole loop. dQ needs
// the sum over the workgroup's 128 keys: each wave writes its dU tile to LDS,
// then every wave forms 16 query rows of dQ with 16x16x32 MFMAs and adds them
// into an fp32 accumulator in the workspace with hardware float atomics
// (coalesced: 16 consecutive d per instruction). A finalize kernel scales and
// rounds dQ to bf16. dL/dlambda and Dr come from the shared preprocess.
//
// Scores use the base-2 domain as in the forward: the fp32 accumulator of
// q . k is multiplied by scale * log2(e), u' = U log2(e), so
// exp(-U) = exp2(-u'), F = exp2(u' sg - c'_i) with c'_i = c_i log2(e).
#include <math.h>

#include "bwd_common.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace rel {
namespace bwdbf16 {

constexpr int D = 64;
constexpr int NW = 4;
constexpr int BK = 32 * NW;  // keys per workgroup
constexpr int BQ = 64;       // queries per tile
constexpr int RS = D + 8;    // row-major q / dY tile stride (bf16), 144 B
constexpr int TS = BQ + 4;   // transposed q / dY tile stride (bf16), 136 B
constexpr int KTS = BK + 8;  // K^T stride (bf16), 272 B
constexpr int US = BK + 8;   // dU tile stride (bf16), 272 B

struct Smem {
  uint16_t qr[BQ * RS];   // q tile, [query][d]
  uint16_t gr[BQ * RS];   // dY tile, [query][d]
  uint16_t qt[D * TS];    // q tile transposed, [d][query]
  uint16_t gt[D * TS];    // dY tile transposed, [d][query]
  uint16_t kt[D * KTS];   // this workgroup's keys, transposed, [d][key]
  uint16_t du[BQ * US];   // dU tile, [query][key]
  float cq[BQ];           // c'_i = (lambda ln i + LSE_i) log2 e   (+inf past T)
  float lq[BQ];           // LSE_i log2 e                           (+inf past T)
  float dr[BQ];           // Dr_i
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

// Writes 2 rows x 8 consecutive columns of a row-major bf16 block transposed:
// dst[(c0 + e) * stride + r0 + {0, 1}] for e in [0, 8).
__device__ __forceinline__ void store_transposed_pair(uint16_t* dst, int stride, int c0, int r0,
                                                      uint4 a, uint4 b) {
  const uint32_t x[4] = {a.x, a.y, a.z, a.w};
  const uint32_t y[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    *reinterpret_cast<uint32_t*>(&dst[(c0 + 2 * i) * stride + r0]) = (x[i] & 0xffffu) | (y[i] << 16);
    *reinterpret_cast<uint32_t*>(&dst[(c0 + 2 * i + 1) * stride + r0]) = (x[i] >> 16) | (y[i] & 0xffff0000u);
  }
}

__global__ __launch_bounds__(256, 1) void bwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ dy,
    const float* __restrict__ lse, const float* __restrict__ Dr, float* __restrict__ dq_acc,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, int T, int BH, float kscale,
    float scale, float inv_tau, float lam) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 31;
  const int hf = lane >> 5;

  const int L = blockIdx.x;
  const int head = L % BH;
  const int kb = L / BH;  // first key blocks (longest query loops) first
  const size_t base = static_cast<size_t>(head) * T * D;
  const size_t rbase = static_cast<size_t>(head) * T;
  const int kw0 = kb * BK + wave * 32;  // this wave's first key
  const int kj = kw0 + r;               // this lane's key

  // ---- own keys: k (B operand of S), v (B operand of dP)
  bf16x8 kf[4], vf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 kr = make_uint4(0, 0, 0, 0), vr = make_uint4(0, 0, 0, 0);
    if (kj < T) {
      kr = *reinterpret_cast<const uint4*>(k + base + static_cast<size_t>(kj) * D + hf * 8 + 16 * s);
      vr = *reinterpret_cast<const uint4*>(v + base + static_cast<size_t>(kj) * D + hf * 8 + 16 * s);
    }
    kf[s] = as_bf16x8(kr);
    vf[s] = as_bf16x8(vr);
  }
  // ---- K^T of the workgroup's 128 keys (raw k), for dQ = dU K
  {
    const int kp = tid >> 3, dc = tid & 7;  // 64 key pairs over 2 passes
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
      const int key0 = kb * BK + 2 * (kp + 32 * pass);
      const uint4 a = (key0 < T) ? *reinterpret_cast<const uint4*>(k + base + static_cast<size_t>(key0) * D + dc * 8) : make_uint4(0, 0, 0, 0);
      const uint4 b = (key0 + 1 < T) ? *reinterpret_cast<const uint4*>(k + base + static_cast<size_t>(key0 + 1) * D + dc * 8) : make_uint4(0, 0, 0, 0);
      store_transposed_pair(sm.kt, KTS, dc * 8, 2 * (kp + 32 * pass), a, b);
    }
  }

  f32x16 dv0 = {0}, dv1 = {0}, dk0 = {0}, dk1 = {0};  // dV^T, dK^T: key r, d rows

  // ---- query tile prefetch: q and dY rows; each thread 2 rows (pair) x 16 B
  const int pr = tid >> 3, pdc = tid & 7;  // query pair 0..31, d chunk
  uint4 pq0, pq1, pg0, pg1;
  float pc = 0.f, pl = 0.f, pd = 0.f;
  auto fetch = [&](int qt0) {
    const int i0 = qt0 + 2 * pr, i1 = i0 + 1;
    pq0 = (i0 < T) ? *reinterpret_cast<const uint4*>(q + base + static_cast<size_t>(i0) * D + pdc * 8) : make_uint4(0, 0, 0, 0);
    pq1 = (i1 < T) ? *reinterpret_cast<const uint4*>(q + base + static_cast<size_t>(i1) * D + pdc * 8) : make_uint4(0, 0, 0, 0);
    pg0 = (i0 < T) ? *reinterpret_cast<const uint4*>(dy + base + static_cast<size_t>(i0) * D + pdc * 8) : make_uint4(0, 0, 0, 0);
    pg1 = (i1 < T) ? *reinterpret_cast<const uint4*>(dy + base + static_cast<size_t>(i1) * D + pdc * 8) : make_uint4(0, 0, 0, 0);
    if (tid < BQ) {
      const int i = qt0 + tid;
      if (i < T) {
        const float ls = lse[rbase + i];
        pc = (lam * logf(static_cast<float>(i + 1)) + ls) * kLog2e;
        pl = ls * kLog2e;
        pd = Dr[rbase + i];
      } else {
        pc = INFINITY;
        pl = INFINITY;
        pd = 0.f;
      }
    }
  };
  auto stash = [&]() {
    *reinterpret_cast<uint4*>(&sm.qr[(2 * pr) * RS + pdc * 8]) = pq0;
    *reinterpret_cast<uint4*>(&sm.qr[(2 * pr + 1) * RS + pdc * 8]) = pq1;
    *reinterpret_cast<uint4*>(&sm.gr[(2 * pr) * RS + pdc * 8]) = pg0;
    *reinterpret_cast<uint4*>(&sm.gr[(2 * pr + 1) * RS + pdc * 8]) = pg1;
    store_transposed_pair(sm.qt, TS, pdc * 8, 2 * pr, pq0, pq1);
    store_transposed_pair(sm.gt, TS, pdc * 8, 2 * pr, pg0, pg1);
    if (tid < BQ) {
      sm.cq[tid] = pc;
      sm.lq[tid] = pl;
      sm.dr[tid] = pd;
    }
  };

  const int qstart = kb * BK;
  fetch(qstart);
  for (int qt0 = qstart; qt0 < T; qt0 += BQ) {
    __syncthreads();  // previous tile (incl. its dQ phase) done with LDS
    stash();
    __syncthreads();
    if (qt0 + BQ < T) fetch(qt0 + BQ);

#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      const int qs0 = qt0 + sub * 32;  // first query of this 32-query sub-tile
      uint16_t* durow = &sm.du[(sub * 32) * US + wave * 32 + r];
      if (qs0 + 31 < kw0 || kw0 >= T) {  // every query precedes every key: no entries
#pragma unroll
        for (int vi = 0; vi < 16; ++vi)
          durow[((vi >> 2) * 8 + hf * 4 + (vi & 3)) * US] = 0;
        continue;
      }
      const bool diag = (qs0 == kw0);

      // ---- S = Q K^T and dP = dY V^T (32 queries x 32 keys)
      f32x16 sc = {0}, dp = {0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 qa = *reinterpret_cast<const uint4*>(&sm.qr[(sub * 32 + r) * RS + hf * 8 + 16 * s]);
        const uint4 ga = *reinterpret_cast<const uint4*>(&sm.gr[(sub * 32 + r) * RS + hf * 8 + 16 * s]);
        sc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(qa), kf[s], sc, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(ga), vf[s], dp, 0, 0, 0);
      }
      // sc[vi], dp[vi]: key = kw0 + r, query = qs0 + (vi>>2)*8 + hf*4 + (vi&3)

      float fv[16], uv[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ql = sub * 32 + g4 * 8 + hf * 4;  // tile-local query of vi = g4*4
        const float4 c4 = *reinterpret_cast<const float4*>(&sm.cq[ql]);
        const float4 d4 = *reinterpret_cast<const float4*>(&sm.dr[ql]);
        const float4 l4 = *reinterpret_cast<const float4*>(&sm.lq[ql]);
        const float cc[4] = {c4.x, c4.y, c4.z, c4.w};
        const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
        const float ll[4] = {l4.x, l4.y, l4.z, l4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int vi = g4 * 4 + j;
          const float u = sc[vi] * kscale;
          const float t = fast_exp2(-u);
          const float sg = fast_rcp(1.0f + t);
          const float e = u * sg;
          float F = fast_exp2(e - cc[j]);
          float dR = F * (dp[vi] - dd[j]);
          const float e2 = e * kLn2;
          float dU = dR * fmaf(-e2, sg, sg + e2);
          if (diag) {
            const int qq = g4 * 8 + hf * 4 + j;  // query offset within sub-tile
            if (qq == r) {  // Self entry
              const float S = fast_rcp(1.0f + fast_exp2(-u * inv_tau));
              F = fast_exp2(S * kLog2e - ll[j]);
              dR = F * (dp[vi] - dd[j]);
              dU = dR * S * (1.0f - S) * inv_tau;
            } else if (qq < r) {  // future key: not in row i
              F = 0.f;
              dU = 0.f;
            }
          }
          fv[vi] = F;
          uv[vi] = dU;
        }
      }
      // bf16 packing (round to nearest even): word w of step c holds the
      // elements c*8 + 2w (low half) and c*8 + 2w + 1 (high half)
      uint32_t fw[8], uw[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        fw[w] = pack_bf16x2(fv[2 * w], fv[2 * w + 1]);
        uw[w] = pack_bf16x2(uv[2 * w], uv[2 * w + 1]);
      }
      const bf16x8 fb[2] = {as_bf16x8(make_uint4(fw[0], fw[1], fw[2], fw[3])),
                            as_bf16x8(make_uint4(fw[4], fw[5], fw[6], fw[7]))};
      const bf16x8 ub[2] = {as_bf16x8(make_uint4(uw[0], uw[1], uw[2], uw[3])),
                            as_bf16x8(make_uint4(uw[4], uw[5], uw[6], uw[7]))};

      // ---- dV^T += G^T F, dK^T += Q^T dU (k-slot hf*8+e of step c <->
      // query c*16 + (e>>2)*8 + hf*4 + (e&3) = element c*8+e of fb / ub)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int qo = sub * 32 + c * 16 + hf * 4;
        const uint2 g0l = *reinterpret_cast<const uint2*>(&sm.gt[r * TS + qo]);
        const uint2 g0h = *reinterpret_cast<const uint2*>(&sm.gt[r * TS + qo + 8]);
        const uint2 g1l = *reinterpret_cast<const uint2*>(&sm.gt[(32 + r) * TS + qo]);
        const uint2 g1h = *reinterpret_cast<const uint2*>(&sm.gt[(32 + r) * TS + qo + 8]);
        const uint2 q0l = *reinterpret_cast<const uint2*>(&sm.qt[r * TS + qo]);
        const uint2 q0h = *reinterpret_cast<const uint2*>(&sm.qt[r * TS + qo + 8]);
        const uint2 q1l = *reinterpret_cast<const uint2*>(&sm.qt[(32 + r) * TS + qo]);
        const uint2 q1h = *reinterpret_cast<const uint2*>(&sm.qt[(32 + r) * TS + qo + 8]);
        dv0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(make_uint4(g0l.x, g0l.y, g0h.x, g0h.y)), fb[c], dv0, 0, 0, 0);
        dv1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(make_uint4(g1l.x, g1l.y, g1h.x, g1h.y)), fb[c], dv1, 0, 0, 0);
        dk0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(make_uint4(q0l.x, q0l.y, q0h.x, q0h.y)), ub[c], dk0, 0, 0, 0);
        dk1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(make_uint4(q1l.x, q1l.y, q1h.x, q1h.y)), ub[c], dk1, 0, 0, 0);
      }
      // ---- dU tile to LDS for the dQ contraction ([query][key])
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int vi = 2 * w;  // elements vi (low half) and vi + 1 (high half)
        durow[((vi >> 2) * 8 + hf * 4 + (vi & 3)) * US] = static_cast<uint16_t>(uw[w] & 0xffffu);
        durow[((vi >> 2) * 8 + hf * 4 + (vi & 3) + 1) * US] = static_cast<uint16_t>(uw[w] >> 16);
      }
    }
    __syncthreads();

    // ---- dQ rows [qt0 + 16*wave, +16) += dU (16 x 128) K (128 x 64)
    {
      const int l16 = lane & 15, g = lane >> 4;
      f32x4 aq[4] = {{0}, {0}, {0}, {0}};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const uint4 a = *reinterpret_cast<const uint4*>(&sm.du[(wave * 16 + l16) * US + st * 32 + g * 8]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const uint4 b = *reinterpret_cast<const uint4*>(&sm.kt[(dt * 16 + l16) * KTS + st * 32 + g * 8]);
          aq[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), aq[dt], 0, 0, 0);
        }
      }
      // aq[dt][j]: d = dt*16 + l16, query = qt0 + wave*16 + g*4 + j
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = qt0 + wave * 16 + g * 4 + j;
        if (i < T) {
          float* dst = dq_acc + base + static_cast<size_t>(i) * D + l16;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) unsafeAtomicAdd(dst + dt * 16, aq[dt][j]);
        }
      }
    }
  }

  // ---- dK = scale * dK^T^T, dV = dV^T^T (key kj, d rows of the accumulators)
  if (kj >= T) return;
  const size_t row = base + static_cast<size_t>(kj) * D;
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + g4 * 8 + hf * 4;
      uint32_t ok[2], ov[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int vi = g4 * 4 + 2 * j;
        const float k0 = (db == 0 ? dk0 : dk1)[vi] * scale;
        const float k1 = (db == 0 ? dk0 : dk1)[vi + 1] * scale;
        const float v0 = (db == 0 ? dv0 : dv1)[vi];
        const float v1 = (db == 0 ? dv0 : dv1)[vi + 1];
        ok[j] = static_cast<uint32_t>(f32_to_bf16_bits(k0)) | (static_cast<uint32_t>(f32_to_bf16_bits(k1)) << 16);
        ov[j] = static_cast<uint32_t>(f32_to_bf16_bits(v0)) | (static_cast<uint32_t>(f32_to_bf16_bits(v1)) << 16);
      }
      *reinterpret_cast<uint2*>(dk + row + d0) = make_uint2(ok[0], ok[1]);
      *reinterpret_cast<uint2*>(dv + row + d0) = make_uint2(ov[0], ov[1]);
    }
  }
}

__global__ __launch_bounds__(256) void zero_f32x4_kernel(float4* __restrict__ p, size_t n4) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<size_t>(gridDim.x) * 256)
    p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(256) void dq_finalize_kernel(const float4* __restrict__ acc,
                                                          uint2* __restrict__ dq, size_t n4,
                                                          float scale) {
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n4;
       i += static_cast<size_t>(gridDim.x) * 256) {
    const float4 a = acc[i];
    const uint32_t lo = static_cast<uint32_t>(f32_to_bf16_bits(a.x * scale)) |
                        (static_cast<uint32_t>(f32_to_bf16_bits(a.y * scale)) << 16);
    const uint32_t hi = static_cast<uint32_t>(f32_to_bf16_bits(a.z * scale)) |
                        (static_cast<uint32_t>(f32_to_bf16_bits(a.w * scale)) << 16);
    dq[i] = make_uint2(lo, hi);
  }
}

}  // namespace bwdbf16

hipError_t launch_bwd_bf16(int B, int H, int T, int D, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, const uint16_t* y, const uint16_t* dy,
                           const float* lse, uint16_t* dq, uint16_t* dk, uint16_t* dv,
                           float* dlambda, void* ws, float scale, float tau, float lam,
                           hipStream_t stream) {
  using namespace bwdbf16;
  const BwdWorkspace w = bwd_workspace_layout(1, B, H, T, D);
  char* wsb = static_cast<char*>(ws);
  float* dq_acc = reinterpret_cast<float*>(wsb + w.off_dq);
  const size_t n4 = static_cast<size_t>(B) * H * T * D / 4;
  const unsigned eg = static_cast<unsigned>(n4 < 4096 * 256 ? (n4 + 255) / 256 : 4096);
  hipLaunchKernelGGL(zero_f32x4_kernel, dim3(eg), dim3(256), 0, stream,
                     reinterpret_cast<float4*>(dq_acc), n4);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_bwd_pre(1, B, H, T, D, q, k, v, y, dy, lse, dlambda, w, wsb, scale, tau, stream);
  if (e != hipSuccess) return e;
  const float* Dr = reinterpret_cast<const float*>(wsb + w.off_dr);
  const int BH = B * H;
  const int nkb = (T + BK - 1) / BK;
  hipLaunchKernelGGL(bwd_bf16_kernel, dim3(static_cast<unsigned>(nkb) * BH), dim3(256), 0,
                     stream, q, k, v, dy, lse, Dr, dq_acc, dk, dv, T, BH,
                     scale * kLog2e, scale, 1.0f / tau, lam);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq_finalize_kernel, dim3(eg), dim3(256), 0, stream,
                     reinterpret_cast<const float4*>(dq_acc), reinterpret_cast<uint2*>(dq), n4,
                     scale);
  return hipGetLastError();
}

}  // namespace rel
