// Relation backward in fp32 (storage and arithmetic), VALU only, by
// recomputation: nothing T x T is stored (App. A.3.6 of the Relation paper).
//
// Per entry (1-based rows i, j <= i), with c_i = lambda ln i + LSE_i:
//   j < i : sg = sigmoid(U_ij), F_ij = exp(U_ij sg - c_i),
//           dR_ij = F_ij (dY_i . v_j - Dr_i),
//           dU_ij = dR_ij sg (1 + U_ij (1 - sg))            (SiLU')
//   j = i : S_i = sigmoid(U_ii / tau), F_ii = exp(S_i - LSE_i),
//           dU_ii = dR_ii S_i (1 - S_i) / tau              (App. A.1.7)
//   dq_i = scale sum_j dU_ij k_j,  dk_j = scale sum_i dU_ij q_i,
//   dv_j = sum_i F_ij dY_i.
// Two kernels: one lane per query row for dq, one lane per key row for
// dk / dv; the lane's own rows sit in LDS, the scanned rows are staged in
// 64-row LDS tiles and read as broadcasts. Accuracy path, not a fast path.
#include <math.h>

#include "bwd_common.hpp"
#include "common.hpp"
#include "launch.hpp"

namespace rel {

__device__ __forceinline__ void bwd_entry(float u, float dp, bool self, float lse_i, float c_i,
                                          float dr_i, float tau, float& F, float& dU) {
  if (self) {
    const float S = 1.f / (1.f + expf(-u / tau));
    F = expf(S - lse_i);
    const float dR = F * (dp - dr_i);
    dU = dR * S * (1.f - S) / tau;
  } else {
    const float sg = 1.f / (1.f + expf(-u));
    F = expf(u * sg - c_i);
    const float dR = F * (dp - dr_i);
    dU = dR * sg * (1.f + u * (1.f - sg));
  }
}

template <int D>
__global__ __launch_bounds__(64) void bwd_f32_dq_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dy, const float* __restrict__ lse, const float* __restrict__ Dr,
    float* __restrict__ dq, int T, int nblk, float scale, float tau, Lam lamp) {
  const float lam = lamp.get();
  __shared__ float Qo[64][D + 1], Go[64][D + 1];  // own q_i, dY_i
  __shared__ float Ks[64][D + 1], Vs[64][D + 1];
  const int lane = threadIdx.x;
  const int blk = blockIdx.x % nblk;
  const int head = blockIdx.x / nblk;
  const size_t base = static_cast<size_t>(head) * T * D;
  const int t = blk * 64 + lane;
  for (int d = 0; d < D; ++d) {
    Qo[lane][d] = (t < T) ? q[base + static_cast<size_t>(t) * D + d] : 0.f;
    Go[lane][d] = (t < T) ? dy[base + static_cast<size_t>(t) * D + d] : 0.f;
  }
  const float lse_i = (t < T) ? lse[static_cast<size_t>(head) * T + t] : 0.f;
  const float dr_i = (t < T) ? Dr[static_cast<size_t>(head) * T + t] : 0.f;
  const float c_i = lam * logf(static_cast<float>(t + 1)) + lse_i;
  float acc[D];
  for (int d = 0; d < D; ++d) acc[d] = 0.f;

  const int kend = min(T, blk * 64 + 64);
  for (int kt = 0; kt < kend; kt += 64) {
    __syncthreads();
    const int kr = kt + lane;
    for (int d = 0; d < D; ++d) {
      Ks[lane][d] = (kr < T) ? k[base + static_cast<size_t>(kr) * D + d] : 0.f;
      Vs[lane][d] = (kr < T) ? v[base + static_cast<size_t>(kr) * D + d] : 0.f;
    }
    __syncthreads();
    if (t < T) {
      const int jn = min(64, t - kt + 1);
      for (int jj = 0; jj < jn; ++jj) {
        float u = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          u = fmaf(Qo[lane][d], Ks[jj][d], u);
          dp = fmaf(Go[lane][d], Vs[jj][d], dp);
        }
        float F, dU;
        bwd_entry(u * scale, dp, kt + jj == t, lse_i, c_i, dr_i, tau, F, dU);
#pragma unroll
        for (int d = 0; d < D; ++d) acc[d] = fmaf(dU, Ks[jj][d], acc[d]);
      }
    }
  }
  if (t >= T) return;
  for (int d = 0; d < D; ++d) dq[base + static_cast<size_t>(t) * D + d] = scale * acc[d];
}

template <int D>
__global__ __launch_bounds__(64) void bwd_f32_dkdv_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dy, const float* __restrict__ lse, const float* __restrict__ Dr,
    float* __restrict__ dk, float* __restrict__ dv, int T, int nblk, float scale, float tau,
    Lam lamp) {
  const float lam = lamp.get();
  __shared__ float Ko[64][D + 1], Vo[64][D + 1];  // own k_j, v_j
  __shared__ float Qs[64][D + 1], Gs[64][D + 1];  // scanned q_i, dY_i
  __shared__ float Ls[64], Rs[64], Cs[64];
  const int lane = threadIdx.x;
  const int blk = blockIdx.x % nblk;
  const int head = blockIdx.x / nblk;
  const size_t base = static_cast<size_t>(head) * T * D;
  const int j = blk * 64 + lane;
  for (int d = 0; d < D; ++d) {
    Ko[lane][d] = (j < T) ? k[base + static_cast<size_t>(j) * D + d] : 0.f;
    Vo[lane][d] = (j < T) ? v[base + static_cast<size_t>(j) * D + d] : 0.f;
  }
  float ak[D], av[D];
  for (int d = 0; d < D; ++d) ak[d] = av[d] = 0.f;

  for (int it = blk * 64; it < T; it += 64) {
    __syncthreads();
    const int ir = it + lane;
    for (int d = 0; d < D; ++d) {
      Qs[lane][d] = (ir < T) ? q[base + static_cast<size_t>(ir) * D + d] : 0.f;
      Gs[lane][d] = (ir < T) ? dy[base + static_cast<size_t>(ir) * D + d] : 0.f;
    }
    const float li = (ir < T) ? lse[static_cast<size_t>(head) * T + ir] : 0.f;
    Ls[lane] = li;
    Rs[lane] = (ir < T) ? Dr[static_cast<size_t>(head) * T + ir] : 0.f;
    Cs[lane] = lam * logf(static_cast<float>(ir + 1)) + li;
    __syncthreads();
    if (j < T) {
      const int i0 = max(0, j - it);
      const int i1 = min(64, T - it);
      for (int ii = i0; ii < i1; ++ii) {
        float u = 0.f, dp = 0.f;
        for (int d = 0; d < D; ++d) {
          u = fmaf(Qs[ii][d], Ko[lane][d], u);
          dp = fmaf(Gs[ii][d], Vo[lane][d], dp);
        }
        float F, dU;
        bwd_entry(u * scale, dp, it + ii == j, Ls[ii], Cs[ii], Rs[ii], tau, F, dU);
#pragma unroll
        for (int d = 0; d < D; ++d) {
          ak[d] = fmaf(dU, Qs[ii][d], ak[d]);
          av[d] = fmaf(F, Gs[ii][d], av[d]);
        }
      }
    }
  }
  if (j >= T) return;
  for (int d = 0; d < D; ++d) {
    dk[base + static_cast<size_t>(j) * D + d] = scale * ak[d];
    dv[base + static_cast<size_t>(j) * D + d] = av[d];
  }
}

hipError_t launch_bwd_f32(int B, int H, int T, int D, const float* q, const float* k,
                          const float* v, const float* y, const float* dy, const float* lse,
                          float* dq, float* dk, float* dv, float* dlambda, void* ws, float scale,
                          float tau, Lam lam, hipStream_t stream, hipEvent_t ev0,
                          hipEvent_t ev1) {
  const BwdWorkspace w = bwd_workspace_layout(0, B, H, T, D);
  char* wsb = static_cast<char*>(ws);
  hipError_t e = launch_bwd_pre(0, T, D, q, k, v, y, dy, lse, dlambda, w, wsb, scale, tau,
                                stream);
  if (e != hipSuccess) return e;
  const float* Dr = reinterpret_cast<const float*>(wsb + w.off_dr);
  const int nblk = (T + 63) / 64;
  const dim3 grid(static_cast<unsigned>(nblk) * B * H);
  if (ev0 && (e = hipEventRecord(ev0, stream)) != hipSuccess) return e;
  if (D == 32) {
    hipLaunchKernelGGL(bwd_f32_dq_kernel<32>, grid, dim3(64), 0, stream, q, k, v, dy, lse, Dr, dq,
                       T, nblk, scale, tau, lam);
    hipLaunchKernelGGL(bwd_f32_dkdv_kernel<32>, grid, dim3(64), 0, stream, q, k, v, dy, lse, Dr,
                       dk, dv, T, nblk, scale, tau, lam);
  } else {
    hipLaunchKernelGGL(bwd_f32_dq_kernel<64>, grid, dim3(64), 0, stream, q, k, v, dy, lse, Dr, dq,
                       T, nblk, scale, tau, lam);
    hipLaunchKernelGGL(bwd_f32_dkdv_kernel<64>, grid, dim3(64), 0, stream, q, k, v, dy, lse, Dr,
                       dk, dv, T, nblk, scale, tau, lam);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return ev1 ? hipEventRecord(ev1, stream) : hipSuccess;
}

}  // namespace rel
