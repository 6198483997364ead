// Linear Relation forward (chunked recurrence) and its single-token step, bf16
// storage, D = 64.
//
// Source: "Ask Self, Ask Others: Relation Is All You Need", Sec. 5.2 and
// App. A.4. Per head, with S_t = sigma(s p1_t . p2_t / tau_S) and the
// normalised coordinates p^ = p / ||p|| (after RoPE when tables are given):
//   E_t = S_t (Diag(alpha_t) C_{t-1})^T p^_1t,  Y_t = I_t + E_t,
//   C_t = Diag(alpha_t) C_{t-1} + S_t p^_2t I_t^T,  alpha_t = exp(g_t).
// With q_t = S_t p^_1t, k_t = S_t p^_2t and the cumulative log-retention
// B_t = sum_{u <= t} g_u (per key channel), the unrolled form (App. A.4.5) is
//   E_t = sum_{j<t} (sum_c q_t[c] k_j[c] e^{B_t[c] - B_j[c]}) I_j + (q_t e^{B_t})^T C_0.
//
// One workgroup (8 waves) per head walks the sequence in chunks of 128
// tokens; wave w owns the 16-token sub-chunk w of every chunk. Per chunk:
//  * row-local work in the MFMA operand layout (lane (l16, g) holds row l16
//    of its sub-chunk, channels 8g..8g+7 and 32+8g..32+8g+7): RoPE, the norms,
//    S, q, k, and the prefix of g over the sub-chunk by DPP row shifts;
//  * every retention factor is taken relative to a sub-chunk boundary that
//    lies between the two tokens it connects, so each is <= 1 and products of
//    them never overflow: q e^{B_t - B_start}, k e^{B_end - B_j}, and
//    per-channel sub-chunk retentions e^{L_s} chained by multiplication;
//  * A^T blocks (keys x queries) by 16x16x32 MFMAs; in the MFMA output
//    layout they are already the A operand of the 16x16x16 MFMAs that apply
//    them to I (no LDS round trip);
//  * the diagonal 16 x 16 block uses the ratio form (k e^{B_start - B_j} may
//    exceed 1): exact while a sub-chunk's retention span stays within 2^120;
//    a sub-chunk with a larger span (a near-total reset) takes an exact
//    per-pair path instead (wave-uniform branch);
//  * the state (fp32, in registers: 2 blocks of 16 x 16 per wave) feeds the
//    next chunk through LDS as bf16 hi + lo, so the read of the state keeps
//    about 16 bits of its mantissa.
#include "launch.hpp"
#include "linear_common.hpp"

namespace rel {
namespace linrel {

struct Smem {
  uint16_t iv[2][CH * IS];  // I rows of the chunk, by chunk parity
  float kk[CH * KS];        // k_j e^{B_end(sub) - B_j}, fp32
  uint16_t kt[CH * IS];     // k_j e^{B_L - B_j}, bf16 (state update)
  uint16_t chi[D * IS];     // state before the chunk, [c][v], bf16 hi
  uint16_t clo[D * IS];     //   and lo parts
  uint16_t ys[CH * IS];     // Y staging for coalesced stores
  float dec[2][NW][D];      // e^{L_s[c]}: retention over sub-chunk s, by parity
};

// blockIdx.x = head (b * H + h). states (optional): the state before every
// chunk and then the final state, [BH][nch + 1][D][D] fp32, for the
// backward. YOUT false: the state pass alone (no Y; the backward's first
// pass).
template <bool ROPE, bool YOUT>
__global__ __launch_bounds__(NT, 1) void linear_fwd_kernel(
    const uint16_t* __restrict__ p1, const uint16_t* __restrict__ p2,
    const uint16_t* __restrict__ iv, const float* __restrict__ g, const float* __restrict__ rc,
    const float* __restrict__ rs, const float* __restrict__ c0, uint16_t* __restrict__ y,
    float* __restrict__ cT, float* __restrict__ states, int T, float sl2) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  // Wave (tid >> 6) owns sub-chunk w = (tid >> 6) ^ 4. Waves 0-3 and 4-7 pair
  // up on the four SIMDs, and timestamps show waves 0-3 getting through the
  // row-local phase about 1.5x faster than their partners; giving them the
  // sub-chunks with the most blocks below the diagonal (4-7) is 1.8 % faster
  // than the identity mapping.
  const int w = (tid >> 6) ^ 4, lane = tid & 63, l16 = lane & 15, grp = lane >> 4;
  const int head = blockIdx.x;
  const size_t base = static_cast<size_t>(head) * T * D;
  const int nch = (T + CH - 1) / CH;

  // ---- state: wave w holds rows 16 rb .. +15, column blocks cb0, cb0 + 1
  const int rb = w >> 1, cb0 = 2 * (w & 1);
  f32x4 cst[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int c = 16 * rb + 4 * grp + r, v = 16 * (cb0 + i) + l16;
      cst[i][r] = c0 ? c0[static_cast<size_t>(head) * D * D + c * D + v] : 0.f;
    }
  }
  auto put_state = [&]() {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int o = (16 * rb + 4 * grp + r) * IS + 16 * (cb0 + i) + l16;
        const float x = cst[i][r];
        const uint16_t hb = f32_to_bf16_bits(x);
        sm.chi[o] = hb;
        sm.clo[o] = f32_to_bf16_bits(x - bf16_bits_to_f32(hb));
      }
    }
  };
  put_state();

  Raw raw;
  load_raw<ROPE>(raw, p1, p2, iv, g, rc, rs, base, 16 * w + l16, T, grp);

  for (int n = 0; n < nch; ++n) {
    const int par = n & 1;
    const int t0 = n * CH;
    const int trow = t0 + 16 * w + l16;  // this lane's row
    // ---------------- row-local: coordinates, Self, q, k, prefix of g
    RowLocal rl;
    row_local<ROPE>(raw, sl2, kSafeLog2Fwd, rl);
    const float* q = rl.q;
    const float* k = rl.k;
    const float* b2 = rl.b2;
    const float* lw = rl.lw;
    const bool safe = rl.safe;
    // retention factors relative to the sub-chunk's boundaries (all <= 1)
    float qq[16], kk[16], dw[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      qq[i] = q[i] * fast_exp2(b2[i]);
      kk[i] = k[i] * fast_exp2(lw[i] - b2[i]);
      dw[i] = fast_exp2(lw[i]);
    }
    // ---------------- publish k, I, the sub-chunk retention
    {
      float* kr = &sm.kk[(16 * w + l16) * KS + 8 * grp];
      uint16_t* ir = &sm.iv[par][(16 * w + l16) * IS + 8 * grp];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        *reinterpret_cast<f32x4*>(kr + 32 * s) = f32x4{kk[8 * s], kk[8 * s + 1], kk[8 * s + 2], kk[8 * s + 3]};
        *reinterpret_cast<f32x4*>(kr + 32 * s + 4) =
            f32x4{kk[8 * s + 4], kk[8 * s + 5], kk[8 * s + 6], kk[8 * s + 7]};
        *reinterpret_cast<u32x4*>(ir + 32 * s) = raw.iv[s];
      }
      if (l16 == 15) {
        float* dr = &sm.dec[par][w][8 * grp];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          *reinterpret_cast<f32x4*>(dr + 32 * s) = f32x4{dw[8 * s], dw[8 * s + 1], dw[8 * s + 2], dw[8 * s + 3]};
          *reinterpret_cast<f32x4*>(dr + 32 * s + 4) =
              f32x4{dw[8 * s + 4], dw[8 * s + 5], dw[8 * s + 6], dw[8 * s + 7]};
        }
      }
    }
    // B operand of the A^T blocks: this wave's queries
    const bf16x8 bq0 = pack_x8(&qq[0]), bq1 = pack_x8(&qq[8]);
    // ---------------- diagonal block A^T[j][t], j < t inside the sub-chunk
    f32x4 ad = {0.f, 0.f, 0.f, 0.f};
    if (!YOUT) {
    } else if (safe) {
      float kd[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) kd[i] = kk[i] * fast_rcp(dw[i]);  // k e^{B_start - B_j}
      ad = mfma32(pack_x8(&kd[0]), bq0, ad);
      ad = mfma32(pack_x8(&kd[8]), bq1, ad);
    } else {
      // exact per pair: sum_c q_t k_j e^{B_t - B_j}
#pragma unroll 1
      for (int jj = 0; jj < 16; ++jj) {
        const int src = (lane & 48) | jj;
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const float kj = __shfl(k[i], src), bj = __shfl(b2[i], src);
          part = fmaf(q[i] * kj, fast_exp2(fminf(b2[i] - bj, 0.f)), part);
        }
        part = sum_groups(part);
        if ((jj >> 2) == grp) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if ((jj & 3) == r) ad[r] = part;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (4 * grp + r >= l16) ad[r] = 0.f;

    // ---------------- prefetch the next chunk
    if (n + 1 < nch) load_raw<ROPE>(raw, p1, p2, iv, g, rc, rs, base, trow + CH, T, grp);

    __syncthreads();  // (1) k, I, retentions of every sub-chunk published

    const uint16_t* ivb = sm.iv[par];
    if constexpr (YOUT) {
    f32x4 acc[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[b] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A I over one 16-key block: B operand I[16 sb + 4 grp + r][16 b + l16]
    auto apply = [&](f32x4 at, int sb) {
      const s16x4 a = pack_x4(at);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const uint2 v = lds_read_tr16(&ivb[(16 * sb + 4 * grp + (l16 >> 2)) * IS + 16 * b + 4 * (l16 & 3)]);
        acc[b] = mfma16(a, __builtin_bit_cast(s16x4, v), acc[b]);
      }
    };
    apply(ad, w);
    // off-diagonal blocks, nearest first: chain = e^{B_start(w) - B_end(s')}.
    // Unrolled over every possible block with a wave-uniform guard, so the
    // LDS reads of a block can be issued ahead of the previous block's MFMAs
    // (a rolled loop measured 9 % slower).
    float chain[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) chain[i] = 1.f;
#pragma unroll
    for (int sp = NW - 2; sp >= 0; --sp) {
      if (sp >= w) continue;
      const float* kr = &sm.kk[(16 * sp + l16) * KS + 8 * grp];
      float kx[16];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(kr + 32 * s);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(kr + 32 * s + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kx[8 * s + e] = u0[e] * chain[8 * s + e];
          kx[8 * s + 4 + e] = u1[e] * chain[8 * s + 4 + e];
        }
      }
      f32x4 at = {0.f, 0.f, 0.f, 0.f};
      at = mfma32(pack_x8(&kx[0]), bq0, at);
      at = mfma32(pack_x8(&kx[8]), bq1, at);
      apply(at, sp);
      const float* dr = &sm.dec[par][sp][8 * grp];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x4 u0 = *reinterpret_cast<const f32x4*>(dr + 32 * s);
        const f32x4 u1 = *reinterpret_cast<const f32x4*>(dr + 32 * s + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          chain[8 * s + e] *= u0[e];
          chain[8 * s + 4 + e] *= u1[e];
        }
      }
    }
    // inter-chunk read: (q e^{B_t})^T C_prev with e^{B_t} = chain * e^{B_t - B_start}
    {
      float qt[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) qt[i] = qq[i] * chain[i];
      const bf16x8 a0 = pack_x8(&qt[0]), a1v = pack_x8(&qt[8]);
#pragma unroll
      for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int o = (32 * ks + 8 * grp + (l16 >> 2)) * IS + 16 * b + 4 * (l16 & 3);
          const bf16x8 ch = cat(lds_read_tr16(&sm.chi[o]), lds_read_tr16(&sm.chi[o + 4 * IS]));
          const bf16x8 cl = cat(lds_read_tr16(&sm.clo[o]), lds_read_tr16(&sm.clo[o + 4 * IS]));
          acc[b] = mfma32(ks ? a1v : a0, ch, acc[b]);
          acc[b] = mfma32(ks ? a1v : a0, cl, acc[b]);
        }
      }
    }
    // Y = I + E into the staging tile (rows 16 w + 4 grp + r, column 16 b + l16)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const uint2 v = lds_read_tr16(&ivb[(16 * w + 4 * grp + (l16 >> 2)) * IS + 16 * b + 4 * (l16 & 3)]);
      const uint32_t vv[2] = {v.x, v.y};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float iv_ = bf16_bits_to_f32(static_cast<uint16_t>(vv[r >> 1] >> (16 * (r & 1))));
        sm.ys[(16 * w + 4 * grp + r) * IS + 16 * b + l16] = f32_to_bf16_bits(iv_ + acc[b][r]);
      }
    }
    }  // YOUT
    // K~ = k e^{B_L - B_j} = kk * prod_{s > w} e^{L_s}
    {
      float after[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) after[i] = 1.f;
#pragma unroll 1
      for (int s2 = w + 1; s2 < NW; ++s2) {
        const float* dr = &sm.dec[par][s2][8 * grp];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const f32x4 u0 = *reinterpret_cast<const f32x4*>(dr + 32 * s);
          const f32x4 u1 = *reinterpret_cast<const f32x4*>(dr + 32 * s + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            after[8 * s + e] *= u0[e];
            after[8 * s + 4 + e] *= u1[e];
          }
        }
      }
      float kt[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) kt[i] = kk[i] * after[i];
      uint16_t* kr = &sm.kt[(16 * w + l16) * IS + 8 * grp];
      *reinterpret_cast<u32x4*>(kr) = __builtin_bit_cast(u32x4, pack_x8(&kt[0]));
      *reinterpret_cast<u32x4*>(kr + 32) = __builtin_bit_cast(u32x4, pack_x8(&kt[8]));
    }

    __syncthreads();  // (2) K~ published; every wave is done reading C_prev

    // ---------------- state update: C = e^{B_L} C + K~^T I (rows 16 rb.., 2 column blocks)
    if (states) {
      float* st = states + (static_cast<size_t>(head) * (nch + 1) + n) * D * D;
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          st[(16 * rb + 4 * grp + r) * D + 16 * (cb0 + i) + l16] = cst[i][r];
    }
    {
      f32x4 tot = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int s = 0; s < NW; ++s) {
        const f32x4 u = *reinterpret_cast<const f32x4*>(&sm.dec[par][s][16 * rb + 4 * grp]);
#pragma unroll
        for (int r = 0; r < 4; ++r) tot[r] *= u[r];
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r) cst[i][r] *= tot[r];
#pragma unroll
      for (int ks = 0; ks < CH / 32; ++ks) {
        const int ro = (32 * ks + 8 * grp + (l16 >> 2)) * IS;
        const int oa = ro + 16 * rb + 4 * (l16 & 3);
        const bf16x8 a = cat(lds_read_tr16(&sm.kt[oa]), lds_read_tr16(&sm.kt[oa + 4 * IS]));
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int ob = ro + 16 * (cb0 + i) + 4 * (l16 & 3);
          const bf16x8 bv = cat(lds_read_tr16(&ivb[ob]), lds_read_tr16(&ivb[ob + 4 * IS]));
          cst[i] = mfma32(a, bv, cst[i]);
        }
      }
      put_state();
    }
    // ---------------- Y rows of this wave, coalesced
    if (YOUT && trow < T) {
      const uint16_t* yr = &sm.ys[(16 * w + l16) * IS + 8 * grp];
      uint16_t* yo = y + base + static_cast<size_t>(trow) * D + 8 * grp;
      *reinterpret_cast<u32x4*>(yo) = *reinterpret_cast<const u32x4*>(yr);
      *reinterpret_cast<u32x4*>(yo + 32) = *reinterpret_cast<const u32x4*>(yr + 32);
    }
  }
  if (cT) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        cT[static_cast<size_t>(head) * D * D + (16 * rb + 4 * grp + r) * D + 16 * (cb0 + i) + l16] =
            cst[i][r];
  }
  if (states) {  // the final state after the per-chunk ones
    float* st = states + (static_cast<size_t>(head) * (nch + 1) + nch) * D * D;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[(16 * rb + 4 * grp + r) * D + 16 * (cb0 + i) + l16] = cst[i][r];
  }
}

// ---------------------------------------------------------------- one step
// One token per head (the recurrent step of Sec. 5.2): 256 threads; thread
// (kg, v) owns state rows 16 kg .. +15 of column v.
__global__ __launch_bounds__(256) void linear_step_kernel(
    const uint16_t* __restrict__ p1, const uint16_t* __restrict__ p2,
    const uint16_t* __restrict__ iv, const float* __restrict__ g, const float* __restrict__ rc,
    const float* __restrict__ rs, float* __restrict__ state, uint16_t* __restrict__ y,
    float sl2) {
  __shared__ float h1[D], h2[D], al[D], part[4][D];
  const int tid = threadIdx.x, v = tid & 63, kg = tid >> 6;
  const size_t head = blockIdx.x;
  const size_t ro = head * D;
  if (kg == 0) {
    float a = bf16_bits_to_f32(p1[ro + v]), b = bf16_bits_to_f32(p2[ro + v]);
    if (rc) {  // rotate-half: lane v < 32 pairs with v + 32
      const int j = v & 31;
      const float c = rc[j], s_ = rs[j];
      const float ao = __shfl_xor(a, 32), bo = __shfl_xor(b, 32);
      a = v < 32 ? fmaf(a, c, -ao * s_) : fmaf(ao, s_, a * c);
      b = v < 32 ? fmaf(b, c, -bo * s_) : fmaf(bo, s_, b * c);
    }
    float dot = a * b, n1 = a * a, n2 = b * b;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      dot += __shfl_xor(dot, o);
      n1 += __shfl_xor(n1, o);
      n2 += __shfl_xor(n2, o);
    }
    const float S = fast_rcp(1.f + fast_exp2(-sl2 * dot));
    h1[v] = n1 > 0.f ? S * a * __builtin_amdgcn_rsqf(n1) : 0.f;  // q = S p^1
    h2[v] = n2 > 0.f ? S * b * __builtin_amdgcn_rsqf(n2) : 0.f;  // k = S p^2
    al[v] = fast_exp2(g[ro + v] * kLog2e);
  }
  __syncthreads();
  float* st = state + head * D * D;
  const float iv_ = bf16_bits_to_f32(iv[ro + v]);
  float e = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int c = 16 * kg + i;
    const float cr = al[c] * st[c * D + v];  // Diag(alpha) C_{t-1}
    e = fmaf(cr, h1[c], e);                  // read before the write
    st[c * D + v] = fmaf(h2[c], iv_, cr);
  }
  part[kg][v] = e;
  __syncthreads();
  if (kg == 0) y[ro + v] = f32_to_bf16_bits(iv_ + part[0][v] + part[1][v] + part[2][v] + part[3][v]);
}

}  // namespace linrel

hipError_t launch_linear_fwd(int B, int H, int T, const uint16_t* p1, const uint16_t* p2,
                             const uint16_t* iv, const float* g, const float* rope_cos,
                             const float* rope_sin, const float* state_in, uint16_t* y,
                             float* state_out, float* states, float scale, float tau,
                             hipStream_t stream) {
  using namespace linrel;
  const float sl2 = scale * kLog2e / tau;
  const dim3 grid(static_cast<unsigned>(B) * H);
  if (rope_cos)
    hipLaunchKernelGGL((linear_fwd_kernel<true, true>), grid, dim3(NT), 0, stream, p1, p2, iv, g,
                       rope_cos, rope_sin, state_in, y, state_out, states, T, sl2);
  else
    hipLaunchKernelGGL((linear_fwd_kernel<false, true>), grid, dim3(NT), 0, stream, p1, p2, iv, g,
                       nullptr, nullptr, state_in, y, state_out, states, T, sl2);
  return hipGetLastError();
}

hipError_t launch_linear_fwd_states(int B, int H, int T, const uint16_t* p1, const uint16_t* p2,
                                    const uint16_t* iv, const float* g, const float* rope_cos,
                                    const float* rope_sin, const float* state_in, float* states,
                                    float scale, float tau, hipStream_t stream) {
  using namespace linrel;
  const float sl2 = scale * kLog2e / tau;
  const dim3 grid(static_cast<unsigned>(B) * H);
  if (rope_cos)
    hipLaunchKernelGGL((linear_fwd_kernel<true, false>), grid, dim3(NT), 0, stream, p1, p2, iv, g,
                       rope_cos, rope_sin, state_in, nullptr, nullptr, states, T, sl2);
  else
    hipLaunchKernelGGL((linear_fwd_kernel<false, false>), grid, dim3(NT), 0, stream, p1, p2, iv,
                       g, nullptr, nullptr, state_in, nullptr, nullptr, states, T, sl2);
  return hipGetLastError();
}

int linear_chunk_rows() { return linrel::CH; }

hipError_t launch_linear_step(int B, int H, const uint16_t* p1, const uint16_t* p2,
                              const uint16_t* iv, const float* g, const float* rope_cos,
                              const float* rope_sin, float* state, uint16_t* y, float scale,
                              float tau, hipStream_t stream) {
  using namespace linrel;
  hipLaunchKernelGGL(linear_step_kernel, dim3(static_cast<unsigned>(B) * H), dim3(256), 0, stream,
                     p1, p2, iv, g, rope_cos, rope_sin, state, y, scale * kLog2e / tau);
  return hipGetLastError();
}

}  // namespace rel
