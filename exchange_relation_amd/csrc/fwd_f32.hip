// Relation forward in fp32 (storage and arithmetic), VALU only.
//
// One 64-lane wave per block of 64 query rows; each lane owns one row i and
// scans its strictly historical Exchange entries j < i with the running
// (m, l, z) of FlashRelation (Sec. 5.1; App. A.3.1-A.3.3), then completes
// the row as in App. A.3.5: A = m + ln l - lambda ln i, g = sigmoid(A - S),
// Y = (1 - g) v_i + g z / l. Row 1 has no history (App. A.1.8): g = 0,
// Y = v_1. Key / value tiles of 64 rows are staged in LDS and read by all
// lanes as broadcasts. This path serves accuracy (fp32 end to end, libm
// expf / logf), not speed.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace rel {

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(const float* __restrict__ q,
                                                     const float* __restrict__ k,
                                                     const float* __restrict__ v,
                                                     float* __restrict__ y,
                                                     float* __restrict__ lse,
                                                     float* __restrict__ gate, int T, int nblk,
                                                     float scale, float tau, Lam lam) {
  __shared__ float Ks[64][D + 1];
  __shared__ float Vs[64][D + 1];
  const int lane = threadIdx.x;
  const int blk = blockIdx.x % nblk;
  const int head = blockIdx.x / nblk;
  const size_t base = static_cast<size_t>(head) * T * D;
  const int t = blk * 64 + lane;  // 0-based row; the pages' i = t + 1

  float qi[D];
  float z[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qi[d] = (t < T) ? q[base + static_cast<size_t>(t) * D + d] * scale : 0.f;
    z[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f, S = 0.f;

  const int kend = min(T, blk * 64 + 64);
  for (int kt = 0; kt < kend; kt += 64) {
    __syncthreads();
    const int kr = kt + lane;
#pragma unroll
    for (int d = 0; d < D; ++d) {
      Ks[lane][d] = (kr < T) ? k[base + static_cast<size_t>(kr) * D + d] : 0.f;
      Vs[lane][d] = (kr < T) ? v[base + static_cast<size_t>(kr) * D + d] : 0.f;
    }
    __syncthreads();
    if (t < T) {
      const int jn = min(64, t - kt + 1);  // keys j <= t inside this tile
      for (int jj = 0; jj < jn; ++jj) {
        float u = 0.f;
#pragma unroll
        for (int d = 0; d < D; ++d) u = fmaf(qi[d], Ks[jj][d], u);
        if (kt + jj == t) {  // Self entry S_i = sigmoid(U_ii / tau_S)
          S = 1.f / (1.f + expf(-u / tau));
          continue;
        }
        const float E = u / (1.f + expf(-u));  // Exchange entry SiLU(U_ij)
        const float mn = fmaxf(m, E);
        const float a = expf(m - mn);
        const float p = expf(E - mn);
        l = l * a + p;
#pragma unroll
        for (int d = 0; d < D; ++d) z[d] = fmaf(p, Vs[jj][d], z[d] * a);
        m = mn;
      }
    }
  }
  if (t >= T) return;

  const size_t row = base + static_cast<size_t>(t) * D;
  float g, lz;
  if (l > 0.f) {
    const float A = m + logf(l) - lam.get() * logf(static_cast<float>(t + 1));
    g = 1.f / (1.f + expf(S - A));
    lz = fmaxf(S, A) + log1pf(expf(-fabsf(S - A)));
  } else {  // empty history: A = -inf
    g = 0.f;
    lz = S;
  }
  const float inv_l = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int d = 0; d < D; ++d) y[row + d] = (1.f - g) * v[row + d] + g * (z[d] * inv_l);
  if (lse) lse[static_cast<size_t>(head) * T + t] = lz;
  if (gate) gate[static_cast<size_t>(head) * T + t] = g;
}

hipError_t launch_fwd_f32(int B, int H, int T, int D, const float* q, const float* k,
                          const float* v, float* y, float* lse, float* gate, float scale,
                          float tau, Lam lam, hipStream_t stream) {
  const int nblk = (T + 63) / 64;
  const dim3 grid(static_cast<unsigned>(nblk) * B * H);
  if (D == 32) {
    hipLaunchKernelGGL(fwd_f32_kernel<32>, grid, dim3(64), 0, stream, q, k, v, y, lse, gate, T,
                       nblk, scale, tau, lam);
  } else {
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(64), 0, stream, q, k, v, y, lse, gate, T,
                       nblk, scale, tau, lam);
  }
  return hipGetLastError();
}

}  // namespace rel
