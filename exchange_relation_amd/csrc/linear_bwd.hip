// Linear Relation backward, bf16 storage, D = 64.
//
// Gradients of the recurrence of Sec. 5.2 (App. A.4) with respect to p1, p2,
// I, the log retention g and the initial state. With q = S p^_1, k = S p^_2,
// B_t the cumulative log retention and dE = dY, per chunk of 128 tokens
// (C_prev: the state before it, dC: the gradient of the state after it):
//   dq_t  = sum_{j<t} dA_tj k_j e^{B_t - B_j} + e^{B_t - B_0} (C_prev dE_t)
//   dk_j  = sum_{t>j} dA_tj q_t e^{B_t - B_j} + e^{B_L - B_j} (dC I_j)
//   dI_j  = dY_j + sum_{t>j} A_tj dE_t + (k_j e^{B_L - B_j})^T dC
//   dA_tj = dE_t . I_j,   A_tj = sum_c q_t k_j e^{B_t - B_j}
//   dC_prev = e^{B_L - B_0} dC + sum_t (q_t e^{B_t - B_0}) dE_t^T
//   dg_t  = sum_{t' >= t} (q dq - k dk)_t'  (+ the final state's term),
// then the chain rule through S = sigmoid(s x1.x2 / tau), the normalisation
// and RoPE. Every e^{.} factor is split at sub-chunk boundaries into factors
// <= 1 as in the forward (linear.hip); a diagonal 16 x 16 block uses the
// ratio form unless the sub-chunk's retention span is beyond 2^60, where an
// exact per-pair path runs instead.
//
// Three passes: the forward's state pass stores the state before every chunk
// (and the final state); linear_dstate_kernel walks the chunks backwards and
// stores dC, the gradient of the state after every chunk; linear_grad_kernel
// then handles every chunk independently (one workgroup per chunk and head).
// For batches with heads for most CUs, linear_bwd_fused_kernel does passes 2
// and 3 in one: one workgroup per head runs the same per-chunk body from the
// last chunk, with dC in registers instead of memory.
// The reverse sum of dg needs no sequential pass: the sum of (q dq - k dk)
// over all tokens after chunk n equals sum_v dC[c][v] C[c][v] of the state
// after chunk n (shifting the log retention of every later token by d only
// rescales that state by e^d), so each chunk adds it to its own suffix sums.
// In the gradient kernel wave w owns the 16 rows of sub-chunk w and does, for
// them, dq against key blocks s' <= w and dk / dI against query blocks
// w' >= w: nine block pairs on every wave.
#include <cstdlib>
#include <cstring>

#include "launch.hpp"
#include "linear_common.hpp"

namespace rel {
namespace linrel {

struct SmemG {
  uint16_t iv[CH * IS];   // I rows
  uint16_t dy[CH * IS];   // dY rows
  uint16_t qq[CH * IS];   // q e^{B_t - B_start(sub)}
  uint16_t kk[CH * IS];   // k e^{B_end(sub) - B_j}
  uint16_t chi[D * IS];   // state before the chunk, [c][v], bf16 hi / lo
  uint16_t clo[D * IS];
  uint16_t dhi[D * IS];   // gradient of the state after the chunk, hi / lo
  uint16_t dlo[D * IS];
  float stage[NW][16 * KS];  // per-wave layout change (MFMA output -> rows)
  float dec[NW][D];          // e^{L_s[c]}
  float tot[NW][D];          // sum of dB over each sub-chunk
  float carry[D];            // sum of dB over every token after the chunk
  float carry2[2][D];        // fused form: halves of the next chunk's carry
};

struct SmemR {
  uint16_t dy[CH * IS];
  uint16_t qq[CH * IS];
  float dec[NW][D];
};

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// 8 consecutive fp32 -> bf16 hi / lo into two LDS rows
__device__ __forceinline__ void put_hilo(uint16_t* hi_row, uint16_t* lo_row, f32x4 a, f32x4 b) {
  float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  const u32x4 hi = pack8(x);
  float hx[8], lo[8];
  unpack8(hi, hx);
#pragma unroll
  for (int e = 0; e < 8; ++e) lo[e] = x[e] - hx[e];
  *reinterpret_cast<u32x4*>(hi_row) = hi;
  *reinterpret_cast<u32x4*>(lo_row) = pack8(lo);
}

// dC_T -> dC after every chunk, [BH][nch][D][D]; dc0: the gradient of the
// initial state (or NULL). One workgroup per head, chunks from the last.
template <bool ROPE>
__global__ __launch_bounds__(NT, 1) void linear_dstate_kernel(
    const uint16_t* __restrict__ p1, const uint16_t* __restrict__ p2,
    const float* __restrict__ g, const float* __restrict__ rc, const float* __restrict__ rs,
    const uint16_t* __restrict__ dy, const float* __restrict__ dcT, float* __restrict__ dstates,
    float* __restrict__ dc0, int T, float sl2) {
  __shared__ SmemR sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int head = blockIdx.x;
  const size_t base = static_cast<size_t>(head) * T * D;
  const size_t sbase = static_cast<size_t>(head) * D * D;
  const int nch = (T + CH - 1) / CH;
  const int rb = w >> 1, cb0 = 2 * (w & 1);
  f32x4 dcs[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dcs[i][r] = dcT ? dcT[sbase + (16 * rb + 4 * grp + r) * D + 16 * (cb0 + i) + l16] : 0.f;
  Raw raw;
  u32x4 rdy[2];
  auto prefetch = [&](int n) {
    const int t = n * CH + 16 * w + l16;
    load_raw<ROPE>(raw, p1, p2, p1, g, rc, rs, base, t, T, grp);
    const size_t row = base + static_cast<size_t>(t < T ? t : T - 1) * D + 8 * grp;
    rdy[0] = *reinterpret_cast<const u32x4*>(dy + row);
    rdy[1] = *reinterpret_cast<const u32x4*>(dy + row + 32);
  };
  prefetch(nch - 1);
  for (int n = nch - 1; n >= 0; --n) {
    // the gradient of the state after chunk n
    {
      float* st = dstates + (static_cast<size_t>(head) * nch + n) * D * D;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st[(16 * rb + 4 * grp + r) * D + 16 * (cb0 + i) + l16] = dcs[i][r];
    }
    RowLocal rl;
    row_local<ROPE>(raw, sl2, kSafeLog2Bwd, rl);
    const u32x4 z = {0, 0, 0, 0};
    const u32x4 y0 = raw.ok ? rdy[0] : z, y1 = raw.ok ? rdy[1] : z;
    float qq[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) qq[i] = rl.q[i] * fast_exp2(rl.b2[i]);
    {
      const int o = (16 * w + l16) * IS + 8 * grp;
      *reinterpret_cast<u32x4*>(&sm.dy[o]) = y0;
      *reinterpret_cast<u32x4*>(&sm.dy[o + 32]) = y1;
      *reinterpret_cast<u32x4*>(&sm.qq[o]) = __builtin_bit_cast(u32x4, pack_x8(&qq[0]));
      *reinterpret_cast<u32x4*>(&sm.qq[o + 32]) = __builtin_bit_cast(u32x4, pack_x8(&qq[8]));
      if (l16 == 15) {
        float* dr = &sm.dec[w][8 * grp];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          *reinterpret_cast<f32x4*>(dr + 32 * s) =
              f32x4{fast_exp2(rl.lw[8 * s]), fast_exp2(rl.lw[8 * s + 1]), fast_exp2(rl.lw[8 * s + 2]),
                    fast_exp2(rl.lw[8 * s + 3])};
          *reinterpret_cast<f32x4*>(dr + 32 * s + 4) =
              f32x4{fast_exp2(rl.lw[8 * s + 4]), fast_exp2(rl.lw[8 * s + 5]),
                    fast_exp2(rl.lw[8 * s + 6]), fast_exp2(rl.lw[8 * s + 7])};
        }
      }
    }
    if (n > 0) prefetch(n - 1);
    __syncthreads();  // (1) q, dY, retentions of the chunk published
    // dC_prev = e^{B_L - B_0} dC + sum_t (q_t e^{B_t - B_0}) dE_t^T
    f32x4 tot4 = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int s = 0; s < NW; ++s) {
      const f32x4 u = *reinterpret_cast<const f32x4*>(&sm.dec[s][16 * rb + 4 * grp]);
#pragma unroll
      for (int r = 0; r < 4; ++r) tot4[r] *= u[r];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) dcs[i][r] *= tot4[r];
    f32x4 pb = {1.f, 1.f, 1.f, 1.f};  // e^{B_start(s) - B_0} at rows 16 rb + 4 grp + r
#pragma unroll
    for (int s = 0; s < NW; ++s) {
      const int o = (16 * s + 4 * grp + (l16 >> 2)) * IS + 4 * (l16 & 3);
      // A operand q^T[c = 16 rb + l16][t = 16 s + 4 grp + r], B operand dE[t][v]
      const s16x4 a = __builtin_bit_cast(s16x4, lds_read_tr16(&sm.qq[o + 16 * rb]));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const f32x4 t = mfma16(
            a, __builtin_bit_cast(s16x4, lds_read_tr16(&sm.dy[o + 16 * (cb0 + i)])),
            f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int r = 0; r < 4; ++r) dcs[i][r] = fmaf(t[r], pb[r], dcs[i][r]);
      }
      const f32x4 u = *reinterpret_cast<const f32x4*>(&sm.dec[s][16 * rb + 4 * grp]);
#pragma unroll
      for (int r = 0; r < 4; ++r) pb[r] *= u[r];
    }
    __syncthreads();  // (2) tiles free for the next chunk
  }
  if (dc0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dc0[sbase + (16 * rb + 4 * grp + r) * D + 16 * (cb0 + i) + l16] = dcs[i][r];
  }
}

// One chunk's gradients for the 16 rows of this wave's sub-chunk, given the
// chunk's raw rows (raw, rdy: loaded, not yet consumed) and, already in LDS,
// the state before the chunk (chi / clo), the gradient of the state after it
// (dhi / dlo) and carry[c], the sum of dB over every token after the chunk
// (the final state's term included). Publishes the rows, retentions and the
// sub-chunk sums of dB (barriers (1) and (2)); stores dp1, dp2, dI and dg of
// the rows. The published tiles stay valid until the caller's next barrier.
template <bool ROPE>
__device__ __forceinline__ void grad_chunk(SmemG& sm, Raw& raw, u32x4 (&rdy)[2],
                                           const float* __restrict__ rc,
                                           const float* __restrict__ rs,
                                           uint16_t* __restrict__ dp1, uint16_t* __restrict__ dp2,
                                           uint16_t* __restrict__ dI, float* __restrict__ dg,
                                           size_t base, int trow, int T, float sl2, float slope,
                                           int tid) {
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  RowLocal rl;
  row_local<ROPE>(raw, sl2, kSafeLog2Bwd, rl);
  const bool ok = raw.ok;
  const bool safe = rl.safe;
  {
    const u32x4 z = {0, 0, 0, 0};
    rdy[0] = ok ? rdy[0] : z;
    rdy[1] = ok ? rdy[1] : z;
  }
  float qq[16], kk[16], dw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    qq[i] = rl.q[i] * fast_exp2(rl.b2[i]);
    kk[i] = rl.k[i] * fast_exp2(rl.lw[i] - rl.b2[i]);
    dw[i] = fast_exp2(rl.lw[i]);
  }
  const bf16x8 bdy[2] = {__builtin_bit_cast(bf16x8, rdy[0]), __builtin_bit_cast(bf16x8, rdy[1])};
  const bf16x8 biv[2] = {__builtin_bit_cast(bf16x8, raw.iv[0]), __builtin_bit_cast(bf16x8, raw.iv[1])};
  {
    const int o = (16 * w + l16) * IS + 8 * grp;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      *reinterpret_cast<u32x4*>(&sm.iv[o + 32 * s]) = raw.iv[s];
      *reinterpret_cast<u32x4*>(&sm.dy[o + 32 * s]) = rdy[s];
      *reinterpret_cast<u32x4*>(&sm.qq[o + 32 * s]) = __builtin_bit_cast(u32x4, pack_x8(&qq[8 * s]));
      *reinterpret_cast<u32x4*>(&sm.kk[o + 32 * s]) = __builtin_bit_cast(u32x4, pack_x8(&kk[8 * s]));
    }
    if (l16 == 15) {
      float* dr = &sm.dec[w][8 * grp];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        *reinterpret_cast<f32x4*>(dr + 32 * s) = f32x4{dw[8 * s], dw[8 * s + 1], dw[8 * s + 2], dw[8 * s + 3]};
        *reinterpret_cast<f32x4*>(dr + 32 * s + 4) =
            f32x4{dw[8 * s + 4], dw[8 * s + 5], dw[8 * s + 6], dw[8 * s + 7]};
      }
    }
  }
  __syncthreads();  // (1) rows, retentions and states published

    // per-lane column factors read from the sub-chunk retentions:
    // dec of sub-chunk s at the lane's MFMA-output columns 16 cb + l16
    auto dec_col = [&](int s, int cb) { return sm.dec[s][16 * cb + l16]; };

    f32x4 dqa[4], dka[4], dia[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      dqa[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      dka[b] = f32x4{0.f, 0.f, 0.f, 0.f};
      dia[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // ---- dq against key blocks s' = w .. 0: dA^T[j][t] = I_j . dE_t, then
    // dq_raw[t][c] += fac[c] sum_j dA[t][j] kk[j][c]
    float fac[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) fac[cb] = fast_rcp(dec_col(w, cb));  // diagonal: k e^{B_start - B_j}
    f32x4 dat_diag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int sp = w; sp >= 0; --sp) {
      f32x4 dat = {0.f, 0.f, 0.f, 0.f};
      const uint16_t* ir = &sm.iv[(16 * sp + l16) * IS + 8 * grp];
      dat = mfma32(ld_bf16x8(ir), bdy[0], dat);
      dat = mfma32(ld_bf16x8(ir + 32), bdy[1], dat);
      if (sp == w) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * grp + r >= l16) dat[r] = 0.f;
        dat_diag = dat;
      }
      if (sp < w || safe) {
        const s16x4 a = pack_x4(dat);
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const uint2 kv =
              lds_read_tr16(&sm.kk[(16 * sp + 4 * grp + (l16 >> 2)) * IS + 16 * cb + 4 * (l16 & 3)]);
          const f32x4 t = mfma16(a, __builtin_bit_cast(s16x4, kv), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) dqa[cb][r] = fmaf(t[r], fac[cb], dqa[cb][r]);
        }
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) fac[cb] = sp == w ? 1.f : fac[cb] * dec_col(sp, cb);
    }
    // fac = e^{B_start(w) - B_0}: the inter-chunk factor of dq
    float before[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) before[cb] = w == 0 ? 1.f : fac[cb];

    // ---- dk, dI against query blocks w' = w .. 7
    float ch16[16], fac4[4];
#pragma unroll
    for (int i = 0; i < 16; ++i) ch16[i] = fast_rcp(dw[i]);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) fac4[cb] = fast_rcp(dec_col(w, cb));
    f32x4 da_diag = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int wq = w; wq < NW; ++wq) {
      const uint16_t* qr = &sm.qq[(16 * wq + l16) * IS + 8 * grp];
      const uint16_t* yr = &sm.dy[(16 * wq + l16) * IS + 8 * grp];
      // A[t][j] (rows t of block wq, columns j of this wave)
      float kx[16];
      {
        const int o = (16 * w + l16) * IS + 8 * grp;
        float u[16];
        unpack8(*reinterpret_cast<const u32x4*>(&sm.kk[o]), *reinterpret_cast<float(*)[8]>(&u[0]));
        unpack8(*reinterpret_cast<const u32x4*>(&sm.kk[o + 32]), *reinterpret_cast<float(*)[8]>(&u[8]));
#pragma unroll
        for (int i = 0; i < 16; ++i) kx[i] = u[i] * ch16[i];
      }
      f32x4 at = {0.f, 0.f, 0.f, 0.f};
      at = mfma32(ld_bf16x8(qr), pack_x8(&kx[0]), at);
      at = mfma32(ld_bf16x8(qr + 32), pack_x8(&kx[8]), at);
      // dA[t][j] = dE_t . I_j
      f32x4 da = {0.f, 0.f, 0.f, 0.f};
      da = mfma32(ld_bf16x8(yr), biv[0], da);
      da = mfma32(ld_bf16x8(yr + 32), biv[1], da);
      if (wq == w) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (4 * grp + r <= l16) {
            at[r] = 0.f;
            da[r] = 0.f;
          }
        da_diag = da;
      }
      if (wq > w || safe) {
        const s16x4 aa = pack_x4(da);   // dA^T[j = l16][t = 4 grp + r]
        const s16x4 ab = pack_x4(at);   // A^T[j = l16][t = 4 grp + r]
#pragma unroll
        for (int cb = 0; cb < 4; ++cb) {
          const int o = (16 * wq + 4 * grp + (l16 >> 2)) * IS + 16 * cb + 4 * (l16 & 3);
          const f32x4 t = mfma16(aa, __builtin_bit_cast(s16x4, lds_read_tr16(&sm.qq[o])),
                                 f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int r = 0; r < 4; ++r) dka[cb][r] = fmaf(t[r], fac4[cb], dka[cb][r]);
          dia[cb] = mfma16(ab, __builtin_bit_cast(s16x4, lds_read_tr16(&sm.dy[o])), dia[cb]);
        }
      }
      // chain(wq + 1, w) = 1 after the diagonal, then times e^{L_wq}
      const float* dr = &sm.dec[wq][8 * grp];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(dr + 32 * s);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(dr + 32 * s + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          ch16[8 * s + e] = wq == w ? 1.f : ch16[8 * s + e] * u0[e];
          ch16[8 * s + 4 + e] = wq == w ? 1.f : ch16[8 * s + 4 + e] * u1[e];
        }
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) fac4[cb] = wq == w ? 1.f : fac4[cb] * dec_col(wq, cb);
    }
    // ch16 / fac4 = e^{B_L - B_end(w)}: the inter-chunk factors of dk and dI
    float after[4];
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) after[cb] = w == NW - 1 ? 1.f : fac4[cb];
#pragma unroll
    for (int i = 0; i < 16; ++i) ch16[i] = w == NW - 1 ? 1.f : ch16[i];

    // ---- inter-chunk terms
    {
      float kt[16];
      {
        const int o = (16 * w + l16) * IS + 8 * grp;
        float u[16];
        unpack8(*reinterpret_cast<const u32x4*>(&sm.kk[o]), *reinterpret_cast<float(*)[8]>(&u[0]));
        unpack8(*reinterpret_cast<const u32x4*>(&sm.kk[o + 32]), *reinterpret_cast<float(*)[8]>(&u[8]));
#pragma unroll
        for (int i = 0; i < 16; ++i) kt[i] = u[i] * ch16[i];  // k e^{B_L - B_j}
      }
      const bf16x8 kt0 = pack_x8(&kt[0]), kt1 = pack_x8(&kt[8]);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int ro = (16 * cb + l16) * IS + 8 * grp;
        f32x4 tq = {0.f, 0.f, 0.f, 0.f}, tk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          tq = mfma32(bdy[ks], ld_bf16x8(&sm.chi[ro + 32 * ks]), tq);  // (dE C_prev^T)[t][c]
          tq = mfma32(bdy[ks], ld_bf16x8(&sm.clo[ro + 32 * ks]), tq);
          tk = mfma32(biv[ks], ld_bf16x8(&sm.dhi[ro + 32 * ks]), tk);  // (I dC^T)[j][c]
          tk = mfma32(biv[ks], ld_bf16x8(&sm.dlo[ro + 32 * ks]), tk);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          dqa[cb][r] = fmaf(tq[r], before[cb], dqa[cb][r]);
          dka[cb][r] = fmaf(tk[r], after[cb], dka[cb][r]);
        }
        // dI_j += (k e^{B_L - B_j})_j^T dC  (K = c)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int o = (32 * ks + 8 * grp + (l16 >> 2)) * IS + 16 * cb + 4 * (l16 & 3);
          const bf16x8 dh = cat(lds_read_tr16(&sm.dhi[o]), lds_read_tr16(&sm.dhi[o + 4 * IS]));
          const bf16x8 dl = cat(lds_read_tr16(&sm.dlo[o]), lds_read_tr16(&sm.dlo[o + 4 * IS]));
          dia[cb] = mfma32(ks ? kt1 : kt0, dh, dia[cb]);
          dia[cb] = mfma32(ks ? kt1 : kt0, dl, dia[cb]);
        }
      }
    }
  float* st = sm.stage[w];
  const float* b2 = rl.b2;
  const float* lw = rl.lw;
    // ---- exact diagonal block for a sub-chunk with a near-total reset
    // (the tiles are still valid: barrier (2) is ahead). A[jj][j] for dI
    // here; its dq / dk terms are added to the rows below.
    if (!safe) {
      f32x4 aexact = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
      for (int jj = 0; jj < 16; ++jj) {
        const int src = (lane & 48) | jj;
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float qj = __shfl(rl.q[i], src), bj = __shfl(b2[i], src);
          part = fmaf(qj * rl.k[i], fast_exp2(fminf(bj - b2[i], 0.f)), part);  // A[jj][j = l16]
        }
        part = sum_groups(part);
        if ((jj >> 2) == grp) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((jj & 3) == r) aexact[r] = jj > l16 ? part : 0.f;
        }
      }
      const s16x4 ab = pack_x4(aexact);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int o = (16 * w + 4 * grp + (l16 >> 2)) * IS + 16 * cb + 4 * (l16 & 3);
        dia[cb] = mfma16(ab, __builtin_bit_cast(s16x4, lds_read_tr16(&sm.dy[o])), dia[cb]);
      }
    }
    // ---- this wave's rows: MFMA-output layout -> row layout (wave-private
    // staging; a wave's LDS accesses complete in order)
    auto to_rows = [&](const f32x4 (&acc)[4], float (&out)[16]) {
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int r = 0; r < 4; ++r) st[(4 * grp + r) * KS + 16 * cb + l16] = acc[cb][r];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const f32x4 u = *reinterpret_cast<const f32x4*>(&st[l16 * KS + 32 * s + 8 * grp + 4 * h]);
#pragma unroll
          for (int e = 0; e < 4; ++e) out[8 * s + 4 * h + e] = u[e];
        }
    };
    float dq[16], dk[16], di[16];
    to_rows(dqa, dq);
    to_rows(dka, dk);
    to_rows(dia, di);
    float dB[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dq[i] *= fast_exp2(b2[i]);
      dk[i] *= fast_exp2(lw[i] - b2[i]);
    }
    if (!safe) {
      // exact diagonal terms: dq_t += dA[t][jj] k_jj e^{B_t - B_jj} (jj < t),
      // dk_j += dA[jj][j] q_jj e^{B_jj - B_j} (jj > j); dA from the blocks above
#pragma unroll 1
      for (int jj = 0; jj < 16; ++jj) {
        const int src = (lane & 48) | jj;
        float dsel = dat_diag[0], esel = da_diag[0];
#pragma unroll
        for (int r = 1; r < 4; ++r) {
          if ((jj & 3) == r) dsel = dat_diag[r];
          if ((jj & 3) == r) esel = da_diag[r];
        }
        // the shuffles run on every lane; the masks are applied after
        const float vq = __shfl(dsel, l16 + 16 * (jj >> 2));
        const float vk = __shfl(esel, l16 + 16 * (jj >> 2));
        const float dAq = jj < l16 ? vq : 0.f;
        const float dAk = jj > l16 ? vk : 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float kj = __shfl(rl.k[i], src), qj = __shfl(rl.q[i], src);
          const float bj = __shfl(b2[i], src);
          dq[i] = fmaf(dAq * kj, fast_exp2(fminf(b2[i] - bj, 0.f)), dq[i]);
          dk[i] = fmaf(dAk * qj, fast_exp2(fminf(bj - b2[i], 0.f)), dk[i]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) dB[i] = fmaf(rl.q[i], dq[i], -rl.k[i] * dk[i]);
    // dI = dY + the contractions
    {
      const int o = (16 * w + l16) * IS + 8 * grp;
      float yv[16];
      unpack8(*reinterpret_cast<const u32x4*>(&sm.dy[o]), *reinterpret_cast<float(*)[8]>(&yv[0]));
      unpack8(*reinterpret_cast<const u32x4*>(&sm.dy[o + 32]), *reinterpret_cast<float(*)[8]>(&yv[8]));
#pragma unroll
      for (int i = 0; i < 16; ++i) di[i] += yv[i];
    }
    // chain rule through S, the normalisation and RoPE. The coordinates are
    // recovered from q = S x1 / ||x1||, k = S x2 / ||x2|| (S > 0); a zero row
    // has q = 0 and x = 0.
    const float S = rl.S;
    const float rS = fast_rcp(S);
    const float u1 = rl.inv1 > 0.f ? fast_rcp(S * rl.inv1) : 0.f;  // x1 = u1 q
    const float u2 = rl.inv2 > 0.f ? fast_rcp(S * rl.inv2) : 0.f;
    float dot1 = 0.f, dot2 = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dot1 = fmaf(rl.q[i] * rS, dq[i], dot1);  // p^_1 . dq
      dot2 = fmaf(rl.k[i] * rS, dk[i], dot2);
    }
    dot1 = sum_groups(dot1);
    dot2 = sum_groups(dot2);
    const float da = (dot1 + dot2) * S * (1.f - S) * slope;
    const float f1 = S * rl.inv1, f2 = S * rl.inv2;
    float dx1[16], dx2[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      dx1[i] = fmaf(f1, fmaf(-rl.q[i] * rS, dot1, dq[i]), da * u2 * rl.k[i]);
      dx2[i] = fmaf(f2, fmaf(-rl.k[i] * rS, dot2, dk[i]), da * u1 * rl.q[i]);
    }
    if constexpr (ROPE) {  // transpose of the rotate-half map
      const size_t tr = static_cast<size_t>(ok ? trow : T - 1) * (D / 2) + 8 * grp;
      f32x4 tcs[2], tsn[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        tcs[h] = *reinterpret_cast<const f32x4*>(rc + tr + 4 * h);
        tsn[h] = *reinterpret_cast<const f32x4*>(rs + tr + 4 * h);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = tcs[e >> 2][e & 3], s_ = tsn[e >> 2][e & 3];
        float a = dx1[e], b = dx1[8 + e];
        dx1[e] = fmaf(a, c, b * s_);
        dx1[8 + e] = fmaf(-a, s_, b * c);
        a = dx2[e];
        b = dx2[8 + e];
        dx2[e] = fmaf(a, c, b * s_);
        dx2[8 + e] = fmaf(-a, s_, b * c);
      }
    }
    float sfx[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) sfx[i] = row_suffix(dB[i]);
    if (l16 == 0) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        *reinterpret_cast<f32x4*>(&sm.tot[w][32 * s + 8 * grp]) =
            f32x4{sfx[8 * s], sfx[8 * s + 1], sfx[8 * s + 2], sfx[8 * s + 3]};
        *reinterpret_cast<f32x4*>(&sm.tot[w][32 * s + 8 * grp + 4]) =
            f32x4{sfx[8 * s + 4], sfx[8 * s + 5], sfx[8 * s + 6], sfx[8 * s + 7]};
      }
    }
    if (ok) {
      const size_t row = base + static_cast<size_t>(trow) * D + 8 * grp;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        *reinterpret_cast<u32x4*>(dp1 + row + 32 * s) = pack8(*reinterpret_cast<float(*)[8]>(&dx1[8 * s]));
        *reinterpret_cast<u32x4*>(dp2 + row + 32 * s) = pack8(*reinterpret_cast<float(*)[8]>(&dx2[8 * s]));
        *reinterpret_cast<u32x4*>(dI + row + 32 * s) = pack8(*reinterpret_cast<float(*)[8]>(&di[8 * s]));
      }
    }
  __syncthreads();  // (2) sub-chunk sums of dB published

  // dg_t = sum over t' >= t of dB: this sub-chunk's suffix, the later
  // sub-chunks of the chunk and every token after the chunk
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = 32 * (i >> 3) + 8 * grp + (i & 7);
    float later = sm.carry[c];
#pragma unroll
    for (int s = 0; s < NW; ++s) later += s > w ? sm.tot[s][c] : 0.f;
    sfx[i] += later;
  }
  if (ok) {
    float* gr = dg + base + static_cast<size_t>(trow) * D + 8 * grp;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      *reinterpret_cast<f32x4*>(gr + 32 * s) = f32x4{sfx[8 * s], sfx[8 * s + 1], sfx[8 * s + 2], sfx[8 * s + 3]};
      *reinterpret_cast<f32x4*>(gr + 32 * s + 4) =
          f32x4{sfx[8 * s + 4], sfx[8 * s + 5], sfx[8 * s + 6], sfx[8 * s + 7]};
    }
  }
}

// One workgroup per (chunk, head): blockIdx.x = head * nch + n. states:
// [BH][nch + 1][D][D] (the state before every chunk, then the final state);
// dstates: [BH][nch][D][D] (the gradient of the state after every chunk).
template <bool ROPE>
__global__ __launch_bounds__(NT, 1) void linear_grad_kernel(
    const uint16_t* __restrict__ p1, const uint16_t* __restrict__ p2,
    const uint16_t* __restrict__ iv, const float* __restrict__ g, const float* __restrict__ rc,
    const float* __restrict__ rs, const uint16_t* __restrict__ dy,
    const float* __restrict__ states, const float* __restrict__ dstates,
    uint16_t* __restrict__ dp1, uint16_t* __restrict__ dp2, uint16_t* __restrict__ dI,
    float* __restrict__ dg, int T, float sl2, float slope) {
  __shared__ SmemG sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int nch = (T + CH - 1) / CH;
  const int head = blockIdx.x / nch, n = blockIdx.x % nch;
  const size_t base = static_cast<size_t>(head) * T * D;
  const int trow = n * CH + 16 * w + l16;
  const float* cprev = states + (static_cast<size_t>(head) * (nch + 1) + n) * D * D;
  const float* cnext = cprev + D * D;  // the state after the chunk
  const float* dcn = dstates + (static_cast<size_t>(head) * nch + n) * D * D;

  Raw raw;
  load_raw<ROPE>(raw, p1, p2, iv, g, rc, rs, base, trow, T, grp);
  u32x4 rdy[2];
  {
    const size_t row = base + static_cast<size_t>(trow < T ? trow : T - 1) * D + 8 * grp;
    rdy[0] = *reinterpret_cast<const u32x4*>(dy + row);
    rdy[1] = *reinterpret_cast<const u32x4*>(dy + row + 32);
  }
  // the states (8 consecutive elements of row c = tid / 8) and the reverse
  // sum of dB over the tokens after the chunk
  {
    const int c = tid >> 3, v0 = 8 * (tid & 7);
    const int o = c * D + v0;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(cprev + o);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(cprev + o + 4);
    const f32x4 d0 = *reinterpret_cast<const f32x4*>(dcn + o);
    const f32x4 d1 = *reinterpret_cast<const f32x4*>(dcn + o + 4);
    const f32x4 n0 = *reinterpret_cast<const f32x4*>(cnext + o);
    const f32x4 n1 = *reinterpret_cast<const f32x4*>(cnext + o + 4);
    put_hilo(&sm.chi[c * IS + v0], &sm.clo[c * IS + v0], a0, a1);
    put_hilo(&sm.dhi[c * IS + v0], &sm.dlo[c * IS + v0], d0, d1);
    float f = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) f = fmaf(d0[e], n0[e], fmaf(d1[e], n1[e], f));
    f += __shfl_xor(f, 1);
    f += __shfl_xor(f, 2);
    f += __shfl_xor(f, 4);
    if ((tid & 7) == 0) sm.carry[c] = f;
  }

  grad_chunk<ROPE>(sm, raw, rdy, rc, rs, dp1, dp2, dI, dg, base, trow, T, sl2, slope, tid);
}

// The state-gradient pass and the gradient pass fused, for batches with at
// least one head per CU: one workgroup per head walks the chunks from the
// last, keeping dC (the gradient of the state after the current chunk) in
// fp32 registers (the dstate kernel's layout), so no dC is stored. The
// reverse sum of dB over the tokens after a chunk (carry) is
// sum_v dC[c][v] C[c][v] of the state after it, as in the chunk-parallel
// form: formed from the fp32 dC and the next chunk's C_prev tile in LDS
// (bf16 hi + lo). Adding up the chunks' own sums of dB instead would carry
// their bf16-operand errors over every later chunk.
template <bool ROPE>
__global__ __launch_bounds__(NT, 1) void linear_bwd_fused_kernel(
    const uint16_t* __restrict__ p1, const uint16_t* __restrict__ p2,
    const uint16_t* __restrict__ iv, const float* __restrict__ g, const float* __restrict__ rc,
    const float* __restrict__ rs, const uint16_t* __restrict__ dy,
    const float* __restrict__ states, const float* __restrict__ dcT,
    uint16_t* __restrict__ dp1, uint16_t* __restrict__ dp2, uint16_t* __restrict__ dI,
    float* __restrict__ dg, float* __restrict__ dc0, int T, float sl2, float slope) {
  __shared__ SmemG sm;
  const int tid = threadIdx.x;
  const int w = tid >> 6, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int nch = (T + CH - 1) / CH;
  const int head = blockIdx.x;
  const size_t base = static_cast<size_t>(head) * T * D;
  const size_t sbase = static_cast<size_t>(head) * D * D;
  const float* hstates = states + static_cast<size_t>(head) * (nch + 1) * D * D;
  const int rb = w >> 1, cb0 = 2 * (w & 1);
  // dC after the last chunk, rows 16 rb + 4 grp + r, columns 16 (cb0 + i) + l16
  f32x4 dcs[2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      dcs[i][r] = dcT ? dcT[sbase + (16 * rb + 4 * grp + r) * D + 16 * (cb0 + i) + l16] : 0.f;
  {  // carry = the final state's term (8 consecutive elements of row c = tid / 8)
    const int c = tid >> 3, o = c * D + 8 * (tid & 7);
    float f = 0.f;
    if (dcT) {
      const float* cf = hstates + static_cast<size_t>(nch) * D * D;
#pragma unroll
      for (int e = 0; e < 8; ++e) f = fmaf(dcT[sbase + o + e], cf[o + e], f);
    }
    f += __shfl_xor(f, 1);
    f += __shfl_xor(f, 2);
    f += __shfl_xor(f, 4);
    if ((tid & 7) == 0) sm.carry[c] = f;
  }
#pragma unroll 1
  for (int n = nch - 1; n >= 0; --n) {
    // the thread index passed through an empty asm, so that the compiler
    // forms the LDS addresses inside the loop instead of keeping them all
    // live across it (which spills)
    int tidv = tid;
    asm volatile("" : "+v"(tidv));
    const int w = tidv >> 6, lane = tidv & 63, l16 = lane & 15, grp = lane >> 4;
    const int rb = w >> 1, cb0 = 2 * (w & 1);
    const int trow = n * CH + 16 * w + l16;
    Raw raw;
    load_raw<ROPE>(raw, p1, p2, iv, g, rc, rs, base, trow, T, grp);
    u32x4 rdy[2];
    {
      const size_t row = base + static_cast<size_t>(trow < T ? trow : T - 1) * D + 8 * grp;
      rdy[0] = *reinterpret_cast<const u32x4*>(dy + row);
      rdy[1] = *reinterpret_cast<const u32x4*>(dy + row + 32);
    }
    {  // the state before the chunk as bf16 hi / lo
      const int c = tidv >> 3, v0 = 8 * (tidv & 7);
      const float* cprev = hstates + static_cast<size_t>(n) * D * D + c * D + v0;
      put_hilo(&sm.chi[c * IS + v0], &sm.clo[c * IS + v0], *reinterpret_cast<const f32x4*>(cprev),
               *reinterpret_cast<const f32x4*>(cprev + 4));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)  // dC after the chunk as bf16 hi / lo
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * rb + 4 * grp + r) * IS + 16 * (cb0 + i) + l16;
        const float x = dcs[i][r];
        const uint16_t hi = f32_to_bf16_bits(x);
        sm.dhi[o] = hi;
        sm.dlo[o] = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
      }
    grad_chunk<ROPE>(sm, raw, rdy, rc, rs, dp1, dp2, dI, dg, base, trow, T, sl2, slope, tidv);
    // dC before the chunk = e^{B_L - B_0} dC + sum_t (q_t e^{B_t - B_0}) dE_t^T,
    // from the chunk's published q e^{B_t - B_start(s)}, dY and e^{L_s}
    f32x4 tot4 = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
    for (int s = 0; s < NW; ++s) {
      const f32x4 u = *reinterpret_cast<const f32x4*>(&sm.dec[s][16 * rb + 4 * grp]);
#pragma unroll
      for (int r = 0; r < 4; ++r) tot4[r] *= u[r];
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) dcs[i][r] *= tot4[r];
    f32x4 pb = {1.f, 1.f, 1.f, 1.f};  // e^{B_start(s) - B_0} at rows 16 rb + 4 grp + r
#pragma unroll
    for (int s = 0; s < NW; ++s) {
      const int o = (16 * s + 4 * grp + (l16 >> 2)) * IS + 4 * (l16 & 3);
      const s16x4 a = __builtin_bit_cast(s16x4, lds_read_tr16(&sm.qq[o + 16 * rb]));
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const f32x4 t = mfma16(
            a, __builtin_bit_cast(s16x4, lds_read_tr16(&sm.dy[o + 16 * (cb0 + i)])),
            f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int r = 0; r < 4; ++r) dcs[i][r] = fmaf(t[r], pb[r], dcs[i][r]);
      }
      const f32x4 u = *reinterpret_cast<const f32x4*>(&sm.dec[s][16 * rb + 4 * grp]);
#pragma unroll
      for (int r = 0; r < 4; ++r) pb[r] *= u[r];
    }
    // the previous chunk's carry, sum_v dC[c][v] C[c][v] of the state between
    // the two chunks (this chunk's C_prev, still in LDS as hi / lo): this
    // wave's 32 columns of its 16 rows, summed over the 16 lanes of a row
    float part[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int o = (16 * rb + 4 * grp + r) * IS + 16 * cb0 + l16;
      part[r] = 0.f;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const float c = bf16_bits_to_f32(sm.chi[o + 16 * i]) + bf16_bits_to_f32(sm.clo[o + 16 * i]);
        part[r] = fmaf(dcs[i][r], c, part[r]);
      }
      part[r] = row_suffix(part[r]);  // lane 0 of the row: the row's sum
    }
    if (l16 == 0) {
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.carry2[w & 1][16 * rb + 4 * grp + r] = part[r];
    }
    __syncthreads();  // (3) every wave done with the chunk's tiles and carry
    if (tidv < D) sm.carry[tidv] = sm.carry2[0][tidv] + sm.carry2[1][tidv];
  }
  if (dc0) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        dc0[sbase + (16 * rb + 4 * grp + r) * D + 16 * (cb0 + i) + l16] = dcs[i][r];
  }
}

}  // namespace linrel

namespace {
// The fused backward form walks each head's chunks in sequence on one CU, so
// it needs heads for most CUs: from 3/4 of the CU count on it is faster
// (B*H = 192 on 256 CUs at T = 1024: 162 against 168 us; 128: 164 against
// 138 us); smaller batches keep the chunk-parallel gradient pass.
// RELATION_LINEAR_BWD=fused or =chunked in the environment forces one form
// (the two agree to fp32 rounding).
bool use_fused_bwd(size_t BH) {
  if (const char* f = std::getenv("RELATION_LINEAR_BWD")) {
    if (std::strcmp(f, "fused") == 0) return true;
    if (std::strcmp(f, "chunked") == 0) return false;
  }
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return false;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      return false;
    cus[dev] = n;
  }
  return 4 * BH >= 3 * static_cast<size_t>(cus[dev]);
}
}  // namespace

hipError_t launch_linear_bwd(int B, int H, int T, const uint16_t* p1, const uint16_t* p2,
                             const uint16_t* iv, const float* g, const float* rope_cos,
                             const float* rope_sin, const float* state_in, const uint16_t* dy,
                             const float* dstate_out, uint16_t* dp1, uint16_t* dp2, uint16_t* dI,
                             float* dg, float* dstate_in, const float* fwd_states, float* ws,
                             float scale, float tau, hipStream_t stream) {
  using namespace linrel;
  const int nch = (T + CH - 1) / CH;
  const size_t BH = static_cast<size_t>(B) * H;
  // [BH][nch][D][D], after the state pass's region unless the forward's
  // states are given (then the workspace holds only the state gradients)
  float* dstates = fwd_states ? ws : ws + BH * (nch + 1) * D * D;
  // pass 1: the state before every chunk and the final state ([BH][nch + 1][D][D]),
  // unless the forward stored them
  const float* states = fwd_states;
  hipError_t e = hipSuccess;
  if (!states) {
    e = launch_linear_fwd_states(B, H, T, p1, p2, iv, g, rope_cos, rope_sin, state_in, ws, scale,
                                 tau, stream);
    if (e != hipSuccess) return e;
    states = ws;
  }
  const float sl2 = scale * kLog2e / tau, slope = scale / tau;
  const dim3 gh(static_cast<unsigned>(BH)), gc(static_cast<unsigned>(BH * nch));
  if (use_fused_bwd(BH)) {
    // passes 2 and 3 in one launch: one workgroup per head, chunks from the last
    if (rope_cos)
      hipLaunchKernelGGL(linear_bwd_fused_kernel<true>, gh, dim3(NT), 0, stream, p1, p2, iv, g,
                         rope_cos, rope_sin, dy, states, dstate_out, dp1, dp2, dI, dg, dstate_in,
                         T, sl2, slope);
    else
      hipLaunchKernelGGL(linear_bwd_fused_kernel<false>, gh, dim3(NT), 0, stream, p1, p2, iv, g,
                         nullptr, nullptr, dy, states, dstate_out, dp1, dp2, dI, dg, dstate_in,
                         T, sl2, slope);
    return hipGetLastError();
  }
  // pass 2: the gradient of the state after every chunk
  if (rope_cos)
    hipLaunchKernelGGL(linear_dstate_kernel<true>, gh, dim3(NT), 0, stream, p1, p2, g, rope_cos,
                       rope_sin, dy, dstate_out, dstates, dstate_in, T, sl2);
  else
    hipLaunchKernelGGL(linear_dstate_kernel<false>, gh, dim3(NT), 0, stream, p1, p2, g, nullptr,
                       nullptr, dy, dstate_out, dstates, dstate_in, T, sl2);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // pass 3: every chunk's gradients
  if (rope_cos)
    hipLaunchKernelGGL(linear_grad_kernel<true>, gc, dim3(NT), 0, stream, p1, p2, iv, g, rope_cos,
                       rope_sin, dy, states, dstates, dp1, dp2, dI, dg, T, sl2, slope);
  else
    hipLaunchKernelGGL(linear_grad_kernel<false>, gc, dim3(NT), 0, stream, p1, p2, iv, g, nullptr,
                       nullptr, dy, states, dstates, dp1, dp2, dI, dg, T, sl2, slope);
  return hipGetLastError();
}

size_t linear_bwd_workspace_bytes(int B, int H, int T, bool with_fwd_states) {
  using namespace linrel;
  const size_t nch = (T + CH - 1) / CH;
  return static_cast<size_t>(B) * H * ((with_fwd_states ? 0 : nch + 1) + nch) * D * D *
         sizeof(float);
}

size_t linear_states_bytes(int B, int H, int T) {
  using namespace linrel;
  const size_t nch = (T + CH - 1) / CH;
  return static_cast<size_t>(B) * H * (nch + 1) * D * D * sizeof(float);
}

}  // namespace rel
