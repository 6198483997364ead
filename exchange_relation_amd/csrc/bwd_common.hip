// Backward pieces shared by the fp32 and bf16 paths.
//
// With G_i = dL/dY_i (App. A.1.7 of the Relation paper), the softmax
// Jacobian gives dL/dR_ij = F_ij (G_i . v_j - Dr_i) with the row term
// Dr_i = sum_j F_ij G_i . v_j = G_i . Y_i. Every row of dL/dR sums to zero,
// so dL/dlambda = sum_{j<i} dL/dR_ij (-ln i) = sum_i ln(i) dL/dR_ii: only the
// Self entry of each row is needed, F_ii = exp(S_i - LSE_i).
//
// bwd_pre_kernel: Dr_i (to the workspace), the per-block partial of
// sum ln(i) dL/dR_ii and (bf16 path) the zero-fill of the fp32 dq
// accumulator. bwd_dlambda_kernel: one workgroup sums the partials in a fixed
// order (deterministic) into *dlambda.
#include <math.h>

#include "bwd_common.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace rel {

// One row per 8-lane group: workgroup b covers rows 32 (b % nbt) .. +31 of
// head b / nbt (nbt = ceil(T / 32) blocks per head); each lane reads D/8
// consecutive elements of the row vectors with one vector load, so every
// wave-wide load covers whole 128-byte rows. When dq_acc is given, the group
// also zero-fills the row of the fp32 dq accumulator. With with_dl the
// workgroup also forms its rows' dL/dlambda terms ln(i) F_ii (dY_i . v_i -
// Dr_i) (from q, k, v) into part[b]; without it the backward kernel forms
// them from its diagonal tiles and only dY and Y are read here.
template <typename TE, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const TE* __restrict__ q,
                                                      const TE* __restrict__ k,
                                                      const TE* __restrict__ v,
                                                      const TE* __restrict__ y,
                                                      const TE* __restrict__ dy,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ Dr,
                                                      float* __restrict__ part,
                                                      float* __restrict__ dq_acc, int T,
                                                      int nbt, bool with_dl, float scale,
                                                      float tau) {
  constexpr int E = D / 8;
  __shared__ float red[32];
  const int sub = threadIdx.x & 7;
  const int grp = threadIdx.x >> 3;
  const int t = (blockIdx.x % nbt) * 32 + grp;  // row of the head
  const long long gr = static_cast<long long>(blockIdx.x / nbt) * T + t;
  float contrib = 0.f;
  if (t < T) {
    const size_t off = static_cast<size_t>(gr) * D + sub * E;
    float a[E], b[E];
    float dYY = 0.f, dYV = 0.f, qk = 0.f;
    load_row_piece<TE, D>(dy + off, a);
    load_row_piece<TE, D>(y + off, b);
#pragma unroll
    for (int e = 0; e < E; ++e) dYY = fmaf(a[e], b[e], dYY);
    if (with_dl) {
      load_row_piece<TE, D>(v + off, b);
#pragma unroll
      for (int e = 0; e < E; ++e) dYV = fmaf(a[e], b[e], dYV);
      load_row_piece<TE, D>(q + off, a);
      load_row_piece<TE, D>(k + off, b);
#pragma unroll
      for (int e = 0; e < E; ++e) qk = fmaf(a[e], b[e], qk);
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      dYY += __shfl_xor(dYY, o, 8);
      dYV += __shfl_xor(dYV, o, 8);
      qk += __shfl_xor(qk, o, 8);
    }
    if (dq_acc) {
      if constexpr (E % 4 == 0) {
#pragma unroll
        for (int e = 0; e < E; e += 4)
          *reinterpret_cast<float4*>(dq_acc + off + e) = make_float4(0.f, 0.f, 0.f, 0.f);
      } else {  // E = 6: the piece is only 8-byte aligned
#pragma unroll
        for (int e = 0; e < E; e += 2)
          *reinterpret_cast<float2*>(dq_acc + off + e) = make_float2(0.f, 0.f);
      }
    }
    if (sub == 0) {
      Dr[gr] = dYY;
      if (with_dl && t > 0) {  // ln(1) = 0 for row 1
        const float S = 1.f / (1.f + expf(-scale * qk / tau));
        const float Fii = expf(S - lse[gr]);
        contrib = logf(static_cast<float>(t + 1)) * Fii * (dYV - dYY);
      }
    }
  }
  if (!with_dl) return;
  if (sub == 0) red[grp] = contrib;
  __syncthreads();
  if (threadIdx.x < 32) {
    float s = red[threadIdx.x];
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, 32);
    if (threadIdx.x == 0) part[blockIdx.x] = s;
  }
}

__global__ __launch_bounds__(256) void bwd_dlambda_kernel(const float* __restrict__ part, int n,
                                                          float* __restrict__ out) {
  __shared__ float red[256];
  float s = 0.f;
#pragma unroll 8
  for (int i = threadIdx.x; i < n; i += 256) s += part[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (unsigned w = 128; w > 0; w >>= 1) {
    if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) *out = red[0];
}

BwdWorkspace bwd_workspace_layout(int dtype, int B, int H, int T, int D) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  BwdWorkspace w;
  const size_t rows = static_cast<size_t>(B) * H * T;
  w.npart = B * H * ((T + 31) / 32);  // one per 32-row block of a head
  w.off_dr = 0;
  w.off_part = al(rows * sizeof(float));
  w.off_dq = w.off_part + al(static_cast<size_t>(w.npart) * sizeof(float));
  w.total = w.off_dq + (dtype == 1 ? al(rows * D * sizeof(float)) : 0);
  return w;
}

size_t bwd_workspace_bytes(int dtype, int B, int H, int T, int D) {
  return bwd_workspace_layout(dtype, B, H, T, D).total;
}

template <typename TE, int D>
hipError_t launch_bwd_pre_t(int T, const TE* q, const TE* k, const TE* v,
                            const TE* y, const TE* dy, const float* lse, float* dlambda,
                            const BwdWorkspace& w, char* ws, float scale, float tau,
                            bool zero_dq, bool with_dl, hipStream_t stream) {
  float* Dr = reinterpret_cast<float*>(ws + w.off_dr);
  float* part = reinterpret_cast<float*>(ws + w.off_part);
  float* dq_acc = zero_dq ? reinterpret_cast<float*>(ws + w.off_dq) : nullptr;
  hipLaunchKernelGGL((bwd_pre_kernel<TE, D>), dim3(w.npart), dim3(256), 0, stream, q, k, v, y, dy,
                     lse, Dr, part, dq_acc, T, (T + 31) / 32, with_dl, scale, tau);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !dlambda) return e;
  hipLaunchKernelGGL(bwd_dlambda_kernel, dim3(1), dim3(256), 0, stream, part, w.npart, dlambda);
  return hipGetLastError();
}

hipError_t launch_bwd_pre(int dtype, int T, int D, const void* q, const void* k,
                          const void* v, const void* y, const void* dy, const float* lse,
                          float* dlambda, const BwdWorkspace& w, char* ws, float scale, float tau,
                          hipStream_t stream) {
  // the bf16 kernels at D = 48 / 64 form the dL/dlambda terms themselves
  const auto b16 = [](const void* p) { return static_cast<const uint16_t*>(p); };
  const auto f32 = [](const void* p) { return static_cast<const float*>(p); };
  if (dtype == 1 && D == 80)
    return launch_bwd_pre_t<uint16_t, 80>(T, b16(q), b16(k), b16(v), b16(y), b16(dy), lse,
                                          dlambda, w, ws, scale, tau, true, true, stream);
  if (dtype == 1 && D == 48)
    return launch_bwd_pre_t<uint16_t, 48>(T, b16(q), b16(k), b16(v), b16(y), b16(dy), lse,
                                          dlambda, w, ws, scale, tau, true, false, stream);
  if (dtype == 1)
    return launch_bwd_pre_t<uint16_t, 64>(T, b16(q), b16(k), b16(v), b16(y), b16(dy), lse,
                                          dlambda, w, ws, scale, tau, true, false, stream);
  if (D == 64)
    return launch_bwd_pre_t<float, 64>(T, f32(q), f32(k), f32(v), f32(y), f32(dy), lse,
                                       dlambda, w, ws, scale, tau, false, true, stream);
  return launch_bwd_pre_t<float, 32>(T, f32(q), f32(k), f32(v), f32(y), f32(dy), lse,
                                     dlambda, w, ws, scale, tau, false, true, stream);
}

}  // namespace rel
