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
//     last query blocks of every head first) and the linear block id keeps all
//     query blocks of a head on the same XCD (ids differ by a multiple of the
//     head count), so K / V of a head are shared through one L2.
//   * Key / value tiles of 64 rows are staged in LDS (K row-major, V
//     transposed) and prefetched into registers one tile ahead.
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
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace rel {
namespace fwdbf16 {

constexpr int D = 64;
constexpr int NW = 4;             // waves per workgroup
constexpr int BM = 32 * NW;       // query rows per workgroup
constexpr int BN = 64;            // keys per LDS tile
constexpr int KS = D + 8;         // K tile row stride (bf16): 144 B, 16 B aligned
constexpr int VS = BN + 4;        // V^T tile row stride (bf16): 136 B, 8 B aligned
constexpr float kLazy = 8.0f;     // log2-domain slack before rescaling

struct Smem {
  uint16_t ks[BN * KS];
  uint16_t vt[D * VS];
};

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

__global__ __launch_bounds__(256, 2) void fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* __restrict__ y, float* __restrict__ lse,
    float* __restrict__ gate, int T, int BH, int nqb, float qscale, float inv_tau, float lam) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int r = lane & 31;   // query within the wave's 32 rows / key row in A operands
  const int hf = lane >> 5;  // which half of the K dimension this lane feeds

  const int L = blockIdx.x;
  const int head = L % BH;
  const int qb = nqb - 1 - L / BH;  // longest query blocks first
  const size_t base = static_cast<size_t>(head) * T * D;
  const int q0 = qb * BM + wave * 32;
  const int qi = q0 + r;
  const bool wave_live = q0 < T;

  // ---- Q fragment: B operand of S^T = K Q^T. Lane holds query r,
  // d = hf*8 + 16*s + [0, 8) for s = 0..3.
  bf16x8 qf[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (qi < T) raw = *reinterpret_cast<const uint4*>(q + base + static_cast<size_t>(qi) * D + hf * 8 + 16 * s);
    qf[s] = as_bf16x8(raw);
  }

  f32x16 acc0 = {0}, acc1 = {0};  // Y^T, d in [0, 32) and [32, 64), query r
  float m = 0.f;                  // log2-domain stabiliser (upper bound of E')
  float lsum = 0.f;               // row sum of bf16(P), this lane's half
  float uself = 0.f;              // u'_ii, held by the lane that meets the diagonal
  bool has_self = false;

  const int kend = min(T, (qb + 1) * BM);
  const int ntiles = (kend + BN - 1) / BN;

  // ---- global -> register prefetch of one tile (K: 2 x 16 B; V: 2 rows x 16 B)
  const int kc0 = tid, kc1 = tid + 256;  // K chunks: key = c >> 3, dchunk = c & 7
  const int vkp = tid >> 3, vdc = tid & 7;  // V: key pair, dchunk
  uint4 pk0, pk1, pv0, pv1;
  auto fetch = [&](int kt) {
    const int key0 = kt * BN + (kc0 >> 3), key1 = kt * BN + (kc1 >> 3);
    pk0 = (key0 < T) ? *reinterpret_cast<const uint4*>(k + base + static_cast<size_t>(key0) * D + (kc0 & 7) * 8) : make_uint4(0, 0, 0, 0);
    pk1 = (key1 < T) ? *reinterpret_cast<const uint4*>(k + base + static_cast<size_t>(key1) * D + (kc1 & 7) * 8) : make_uint4(0, 0, 0, 0);
    const int vk0 = kt * BN + 2 * vkp, vk1 = vk0 + 1;
    pv0 = (vk0 < T) ? *reinterpret_cast<const uint4*>(v + base + static_cast<size_t>(vk0) * D + vdc * 8) : make_uint4(0, 0, 0, 0);
    pv1 = (vk1 < T) ? *reinterpret_cast<const uint4*>(v + base + static_cast<size_t>(vk1) * D + vdc * 8) : make_uint4(0, 0, 0, 0);
  };
  auto stash = [&]() {
    *reinterpret_cast<uint4*>(&sm.ks[(kc0 >> 3) * KS + (kc0 & 7) * 8]) = pk0;
    *reinterpret_cast<uint4*>(&sm.ks[(kc1 >> 3) * KS + (kc1 & 7) * 8]) = pk1;
    const uint32_t a[4] = {pv0.x, pv0.y, pv0.z, pv0.w};
    const uint32_t b[4] = {pv1.x, pv1.y, pv1.z, pv1.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // d = vdc*8 + 2i (low halves) and + 2i + 1 (high halves); keys 2kp, 2kp+1
      const uint32_t lo = (a[i] & 0xffffu) | (b[i] << 16);
      const uint32_t hi = (a[i] >> 16) | (b[i] & 0xffff0000u);
      *reinterpret_cast<uint32_t*>(&sm.vt[(vdc * 8 + 2 * i) * VS + 2 * vkp]) = lo;
      *reinterpret_cast<uint32_t*>(&sm.vt[(vdc * 8 + 2 * i + 1) * VS + 2 * vkp]) = hi;
    }
  };

  fetch(0);
  for (int kt = 0; kt < ntiles; ++kt) {
    __syncthreads();  // previous tile fully consumed
    stash();
    __syncthreads();
    if (kt + 1 < ntiles) fetch(kt + 1);
    if (!wave_live) continue;

#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int k0 = kt * BN + sb * 32;
      if (k0 > q0) break;  // whole sub-block beyond this wave's causal range
      const bool diag = (k0 == q0);

      // ---- S^T = K Q^T: A = K rows (key r, d = hf*8 + 16s + [0,8))
      f32x16 st = {0};
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const uint4 kr = *reinterpret_cast<const uint4*>(&sm.ks[(sb * 32 + r) * KS + hf * 8 + 16 * s]);
        st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(kr), qf[s], st, 0, 0, 0);
      }
      // st[vi]: key = k0 + (vi>>2)*8 + hf*4 + (vi&3), query = q0 + r; to u'.
#pragma unroll
      for (int vi = 0; vi < 16; ++vi) st[vi] *= qscale;

      // ---- diagonal sub-block: capture Self, mask j >= i
      if (diag) {
        const int vself = ((r >> 3) << 2) + (r & 3);
        const bool mine = hf == ((r >> 2) & 1);
#pragma unroll
        for (int vi = 0; vi < 16; ++vi) {
          const int kk = (vi >> 2) * 8 + hf * 4 + (vi & 3);
          if (mine && vi == vself) uself = st[vi];
          if (kk >= r) st[vi] = -INFINITY;  // not strictly historical
        }
        has_self = mine;
      }

      // ---- running stabiliser (lazy)
      float mx = st[0];
#pragma unroll
      for (int vi = 1; vi < 16; ++vi) mx = fmaxf(mx, st[vi]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const bool grow = mx > m + kLazy;
      if (__any(grow)) {
        const float mn = grow ? mx : m;
        const float a = fast_exp2(m - mn);
        lsum *= a;
#pragma unroll
        for (int vi = 0; vi < 16; ++vi) {
          acc0[vi] *= a;
          acc1[vi] *= a;
        }
        m = mn;
      }

      // ---- P = exp2(E' - m'), E' = u' * sigmoid(U); masked entries -> 0
      float pv[16];
#pragma unroll
      for (int vi = 0; vi < 16; ++vi) {
        const float u = st[vi];
        const float sg = fast_rcp(1.0f + fast_exp2(-u));
        float p = fast_exp2(fmaf(u, sg, -m));
        if (diag) p = (u == -INFINITY) ? 0.f : p;
        pv[vi] = p;
      }
      uint32_t pw[8];
      const bf16x2 one2 = {static_cast<__bf16>(1.0f), static_cast<__bf16>(1.0f)};
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        pw[w] = pack_bf16x2(pv[2 * w], pv[2 * w + 1]);
        lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pw[w]), one2, lsum, false);
      }
      const bf16x8 pb[2] = {as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3])),
                            as_bf16x8(make_uint4(pw[4], pw[5], pw[6], pw[7]))};

      // ---- Y^T += V^T P^T. k-slot hf*8 + e of step c <-> key
      // c*16 + (e>>2)*8 + hf*4 + (e&3), which is exactly st[c*8 + e].
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int kofs = sb * 32 + c * 16 + hf * 4;
        const uint2 a0l = *reinterpret_cast<const uint2*>(&sm.vt[r * VS + kofs]);
        const uint2 a0h = *reinterpret_cast<const uint2*>(&sm.vt[r * VS + kofs + 8]);
        const uint2 a1l = *reinterpret_cast<const uint2*>(&sm.vt[(32 + r) * VS + kofs]);
        const uint2 a1h = *reinterpret_cast<const uint2*>(&sm.vt[(32 + r) * VS + kofs + 8]);
        const bf16x8 va0 = as_bf16x8(make_uint4(a0l.x, a0l.y, a0h.x, a0h.y));
        const bf16x8 va1 = as_bf16x8(make_uint4(a1l.x, a1l.y, a1h.x, a1h.y));
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va0, pb[c], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va1, pb[c], acc1, 0, 0, 0);
      }
    }
  }

  if (!wave_live) return;
  // ---- row completion (App. A.3.5), base-2 domain
  const float ltot = lsum + __shfl_xor(lsum, 32);
  const float uo = __shfl_xor(uself, 32);
  const float us = has_self ? uself : uo;
  if (qi >= T) return;
  const float S = fast_rcp(1.0f + fast_exp2(-us * inv_tau));  // sigmoid(U_ii / tau)
  const float S2 = S * kLog2e;
  float g, lz;
  if (ltot > 0.f) {
    const float A2 = m + fast_log2(ltot) - lam * fast_log2(static_cast<float>(qi + 1));
    g = fast_rcp(1.0f + fast_exp2(S2 - A2));
    lz = kLn2 * (fmaxf(S2, A2) + fast_log2(1.0f + fast_exp2(-fabsf(S2 - A2))));
  } else {
    g = 0.f;
    lz = S;
  }
  const float gl = (ltot > 0.f) ? g * fast_rcp(ltot) : 0.f;
  const float gs = 1.0f - g;
  const size_t row = base + static_cast<size_t>(qi) * D;
#pragma unroll
  for (int db = 0; db < 2; ++db) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = db * 32 + g4 * 8 + hf * 4;
      const uint2 vr = *reinterpret_cast<const uint2*>(v + row + d0);
      const uint32_t w[2] = {vr.x, vr.y};
      uint32_t o[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float z0 = (db == 0 ? acc0 : acc1)[g4 * 4 + 2 * j];
        const float z1 = (db == 0 ? acc0 : acc1)[g4 * 4 + 2 * j + 1];
        const float y0 = fmaf(gs, __uint_as_float(w[j] << 16), gl * z0);
        const float y1 = fmaf(gs, __uint_as_float(w[j] & 0xffff0000u), gl * z1);
        o[j] = static_cast<uint32_t>(f32_to_bf16_bits(y0)) |
               (static_cast<uint32_t>(f32_to_bf16_bits(y1)) << 16);
      }
      *reinterpret_cast<uint2*>(y + row + d0) = make_uint2(o[0], o[1]);
    }
  }
  if (hf == 0) {
    const size_t ri = static_cast<size_t>(head) * T + qi;
    if (lse) lse[ri] = lz;
    if (gate) gate[ri] = g;
  }
}

}  // namespace fwdbf16

hipError_t launch_fwd_bf16(int B, int H, int T, int D, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, uint16_t* y, float* lse, float* gate, float scale,
                           float tau, float lam, hipStream_t stream) {
  (void)D;
  const int BH = B * H;
  const int nqb = (T + fwdbf16::BM - 1) / fwdbf16::BM;
  const dim3 grid(static_cast<unsigned>(nqb) * BH);
  hipLaunchKernelGGL(fwdbf16::fwd_bf16_kernel, grid, dim3(256), 0, stream, q, k, v, y, lse, gate,
                     T, BH, nqb, scale * kLog2e, 1.0f / tau, lam);
  return hipGetLastError();
}

}  // namespace rel
