// Multi-Head Relation's upstream maps around the Relation operator, as
// separate bandwidth-bound passes (Sec. 3.1-3.2; App. A.2.2-A.2.3):
//
//   prepare : q = RoPE(p1), k = RoPE(p2), v = Givens(I) into a workspace, so
//             the plain kernels run on them. Keys and values are rotated /
//             mixed once here rather than in the forward's tile loads, where
//             every query block of a head would redo them on the VALU the
//             forward is bound by; the bf16 forward only fuses the rotation
//             of its own query rows, with the same arithmetic (rope8), so
//             forward and backward see bit-identical q, k, v;
//   unrotate: dp = RoPE^T(dq) for dq and dk, in fp32, rounded once into the
//             output dtype;
//   unmix   : dI = Givens^T(dv) for both heads of every pair, and the angle
//             gradient dtheta_p = sum(dv_a v_b - dv_b v_a) (the rotation's
//             derivative maps v_a -> v_b and v_b -> -v_a), reduced per
//             workgroup and then over workgroups in a fixed order.
//
// RoPE pairs element d with d + D/2 and reads the caller's tables cos, sin
// [T, D/2] (fp32) at the row's position. Thread layout of every pass: one
// thread per (row, 4 pairs) - the chunk j of elements d = 4j..4j+3 and the
// matching chunk of d + D/2 - so D/8 threads per row, each half of a row read
// by consecutive threads as one contiguous run (8 pairs per thread, with two
// strided 16-byte pieces per half, ran the dI and dp1 passes 15-18 % slower).
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace rel {
namespace mhr {

// Pairs per thread: 4, so that the 8 threads of a 64-wide row read each half
// of it as one contiguous run (16-byte fp32 / 8-byte bf16 pieces).
constexpr int NP = 4;
template <typename TE> struct Io;
template <> struct Io<uint16_t> {  // NP bf16 per chunk
  __device__ static void load(const uint16_t* p, float (&x)[NP]) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    x[0] = __uint_as_float(w.x << 16);
    x[1] = __uint_as_float(w.x & 0xffff0000u);
    x[2] = __uint_as_float(w.y << 16);
    x[3] = __uint_as_float(w.y & 0xffff0000u);
  }
  __device__ static void store(uint16_t* p, const float (&x)[NP]) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]));
  }
};
template <> struct Io<float> {  // NP floats per chunk
  __device__ static void load(const float* p, float (&x)[NP]) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
  }
  __device__ static void store(float* p, const float (&x)[NP]) {
    *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
  }
};
__device__ __forceinline__ void loadf(const float* p, float (&x)[NP]) { Io<float>::load(p, x); }

// Thread -> (row of [B*H*T], chunk j) for a tensor of D-wide rows.
struct Slot {
  size_t row;
  int j;
  bool ok;
};
template <int D>
__device__ __forceinline__ Slot slot_of(size_t rows) {
  constexpr int CPR = D / (2 * NP);  // chunks of NP pairs per row
  const size_t g = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  return {g / CPR, static_cast<int>(g % CPR), g / CPR < rows};
}

// The same arithmetic as rope8 / the fused forward's mixing, on fp32 lanes.
__device__ __forceinline__ void rope_pairs(float (&a)[NP], float (&b)[NP], const float (&c)[NP],
                                           const float (&s)[NP]) {
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const float a2 = fmaf(a[e], c[e], -b[e] * s[e]);
    b[e] = fmaf(a[e], s[e], b[e] * c[e]);
    a[e] = a2;
  }
}
__device__ __forceinline__ void rope_pairs_t(float (&a)[NP], float (&b)[NP], const float (&c)[NP],
                                             const float (&s)[NP]) {
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const float a2 = fmaf(a[e], c[e], b[e] * s[e]);
    b[e] = fmaf(-a[e], s[e], b[e] * c[e]);
    a[e] = a2;
  }
}

// q = RoPE(p1), k = RoPE(p2), v = Givens(I); rows = B*H*T. A NULL output is
// not produced (q, k need the RoPE tables, v the angles).
template <typename TE, int D>
__global__ __launch_bounds__(256) void prepare_kernel(const TE* __restrict__ p1,
                                                      const TE* __restrict__ p2,
                                                      const TE* __restrict__ vi, TE* __restrict__ q,
                                                      TE* __restrict__ k, TE* __restrict__ v,
                                                      size_t rows, int T, Mhr mh) {
  const Slot sl = slot_of<D>(rows);
  if (!sl.ok) return;
  const int t = static_cast<int>(sl.row % T);
  const size_t o = sl.row * D + sl.j * NP;
  float a[NP], b[NP];
  if (q || k) {  // RoPE tables of the row (requested only with RoPE)
    float c[NP], s[NP];
    loadf(mh.cos + static_cast<size_t>(t) * (D / 2) + sl.j * NP, c);
    loadf(mh.sin + static_cast<size_t>(t) * (D / 2) + sl.j * NP, s);
    if (q) {
      Io<TE>::load(p1 + o, a);
      Io<TE>::load(p1 + o + D / 2, b);
      rope_pairs(a, b, c, s);
      Io<TE>::store(q + o, a);
      Io<TE>::store(q + o + D / 2, b);
    }
    if (k) {
      Io<TE>::load(p2 + o, a);
      Io<TE>::load(p2 + o + D / 2, b);
      rope_pairs(a, b, c, s);
      Io<TE>::store(k + o, a);
      Io<TE>::store(k + o + D / 2, b);
    }
  }
  if (!v) return;
  Io<TE>::load(vi + o, a);
  Io<TE>::load(vi + o + D / 2, b);
  {
    const size_t head = sl.row / T;
    const int h = static_cast<int>(head % mh.H);
    int pair, partner;
    float sgn;
    givens_role(h, mh.H, mh.pairing, pair, partner, sgn);
    const float mixc = cosf(mh.theta[pair]), mixs = sgn * sinf(mh.theta[pair]);
    const size_t po = o + (static_cast<size_t>(partner) - h) * T * D;
    float pa[NP], pb[NP];
    Io<TE>::load(vi + po, pa);
    Io<TE>::load(vi + po + D / 2, pb);
#pragma unroll
    for (int e = 0; e < NP; ++e) {
      a[e] = fmaf(mixc, a[e], mixs * pa[e]);
      b[e] = fmaf(mixc, b[e], mixs * pb[e]);
    }
  }
  Io<TE>::store(v + o, a);
  Io<TE>::store(v + o + D / 2, b);
}

// dp = RoPE^T(scale * g) for one gradient tensor (g fp32, may alias dp when
// TE = float: every thread reads its elements before writing them).
template <typename TE, int D>
__global__ __launch_bounds__(256) void unrotate_kernel(const float* g, TE* dp, size_t rows, int T,
                                                       float scale, const float* __restrict__ cs,
                                                       const float* __restrict__ sn,
                                                       const float* __restrict__ dl_part,
                                                       int dl_npart, float* __restrict__ dlambda) {
  if (blockIdx.x == 0 && dlambda) {  // dL/dlambda: fixed-order sum of the partials
    __shared__ float red[256];
    float s = 0.f;
#pragma unroll 8
    for (int i = threadIdx.x; i < dl_npart; i += 256) s += dl_part[i];
    red[threadIdx.x] = s;
    __syncthreads();
    for (unsigned w = 128; w > 0; w >>= 1) {
      if (threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
      __syncthreads();
    }
    if (threadIdx.x == 0) *dlambda = red[0];
  }
  const Slot sl = slot_of<D>(rows);
  if (!sl.ok) return;
  const int t = static_cast<int>(sl.row % T);
  const size_t o = sl.row * D + sl.j * NP;
  float a[NP], b[NP];
  loadf(g + o, a);
  loadf(g + o + D / 2, b);
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    a[e] *= scale;
    b[e] *= scale;
  }
  if (cs) {
    float c[NP], s[NP];
    loadf(cs + static_cast<size_t>(t) * (D / 2) + sl.j * NP, c);
    loadf(sn + static_cast<size_t>(t) * (D / 2) + sl.j * NP, s);
    rope_pairs_t(a, b, c, s);
  }
  Io<TE>::store(dp + o, a);
  Io<TE>::store(dp + o + D / 2, b);
}

// dI = Givens^T(dv) and the dtheta partials. One thread per (pair p, batch b,
// position t, chunk j); blockIdx.y = p * B + b, so a workgroup never mixes
// pairs and its partial belongs to pair p alone. dv (fp32) may alias dI when
// TE = float. v holds the mixed values (the forward's I').
template <typename TE, int D>
__global__ __launch_bounds__(256) void unmix_kernel(const float* dv, TE* dI,
                                                    const TE* __restrict__ v, int B, int T,
                                                    Mhr mh, float* __restrict__ part) {
  __shared__ float red[4];
  constexpr int CPR = D / (2 * NP);
  const int p = blockIdx.y / B, b = blockIdx.y % B;
  const size_t g = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  const size_t t = g / CPR;
  const int j = static_cast<int>(g % CPR);
  float acc = 0.f;
  if (t < static_cast<size_t>(T)) {
    // the pair's heads: first a (sign +), second bb
    const int ha = mh.pairing == 0 ? 2 * p : 2 * p + 1;
    const int hb = mh.pairing == 0 ? 2 * p + 1 : (2 * p + 2) % mh.H;
    const float c = cosf(mh.theta[p]), s = sinf(mh.theta[p]);
    const size_t oa = ((static_cast<size_t>(b) * mh.H + ha) * T + t) * D + j * NP;
    const size_t ob = ((static_cast<size_t>(b) * mh.H + hb) * T + t) * D + j * NP;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const size_t xa = oa + half * (D / 2), xb = ob + half * (D / 2);
      float ga[NP], gb[NP], va[NP], vb[NP];
      loadf(dv + xa, ga);
      loadf(dv + xb, gb);
      Io<TE>::load(v + xa, va);
      Io<TE>::load(v + xb, vb);
      float ia[NP], ib[NP];
#pragma unroll
      for (int e = 0; e < NP; ++e) {
        acc = fmaf(ga[e], vb[e], acc);
        acc = fmaf(-gb[e], va[e], acc);
        ia[e] = fmaf(c, ga[e], -s * gb[e]);
        ib[e] = fmaf(s, ga[e], c * gb[e]);
      }
      Io<TE>::store(dI + xa, ia);
      Io<TE>::store(dI + xb, ib);
    }
  }
  // the workgroup's partial: each wave by lane exchanges, then the 4 waves
  // in a fixed order
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0)
    part[static_cast<size_t>(blockIdx.y) * gridDim.x + blockIdx.x] = (red[0] + red[1]) + (red[2] + red[3]);
}

// dtheta[p] = sum of pair p's partials, in a fixed order (deterministic).
__global__ __launch_bounds__(256) void dtheta_kernel(const float* __restrict__ part, int nper,
                                                     float* __restrict__ dtheta) {
  __shared__ float red[256];
  const float* pp = part + static_cast<size_t>(blockIdx.x) * nper;
  float s = 0.f;
  for (int i = threadIdx.x; i < nper; i += 256) s += pp[i];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int w = 128; w > 0; w >>= 1) {
    if (static_cast<int>(threadIdx.x) < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) dtheta[blockIdx.x] = red[0];
}

template <typename TE, int D>
hipError_t run_prepare(int B, int H, int T, const void* p1, const void* p2, const void* vi,
                       void* q, void* k, void* v, const Mhr& mh, hipStream_t stream) {
  const size_t rows = static_cast<size_t>(B) * H * T;
  const size_t threads = rows * (D / (2 * NP));
  hipLaunchKernelGGL((prepare_kernel<TE, D>), dim3(static_cast<unsigned>((threads + 255) / 256)),
                     dim3(256), 0, stream, static_cast<const TE*>(p1), static_cast<const TE*>(p2),
                     static_cast<const TE*>(vi), static_cast<TE*>(q), static_cast<TE*>(k),
                     static_cast<TE*>(v), rows, T, mh);
  return hipGetLastError();
}

template <typename TE, int D>
hipError_t run_post(int B, int H, int T, const float* dq, float dq_scale, const float* dk,
                    const float* dv, const void* vmix, void* dp1, void* dp2, void* dI,
                    float* dtheta, float* part, const Mhr& mh, hipStream_t stream,
                    const float* dl_part, int dl_npart, float* dlambda) {
  const size_t rows = static_cast<size_t>(B) * H * T;
  const unsigned nb = static_cast<unsigned>((rows * (D / (2 * NP)) + 255) / 256);
  hipLaunchKernelGGL((unrotate_kernel<TE, D>), dim3(nb), dim3(256), 0, stream, dq,
                     static_cast<TE*>(dp1), rows, T, dq_scale, mh.cos, mh.sin, dl_part, dl_npart,
                     dl_part ? dlambda : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dk) {  // else the backward wrote dp2 itself
    hipLaunchKernelGGL((unrotate_kernel<TE, D>), dim3(nb), dim3(256), 0, stream, dk,
                       static_cast<TE*>(dp2), rows, T, 1.0f, mh.cos, mh.sin, nullptr, 0,
                       nullptr);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mh.theta == nullptr) {  // no mixing: dI = dv (a plain copy / rounding)
    hipLaunchKernelGGL((unrotate_kernel<TE, D>), dim3(nb), dim3(256), 0, stream, dv,
                       static_cast<TE*>(dI), rows, T, 1.0f, nullptr, nullptr, nullptr, 0,
                       nullptr);
    return hipGetLastError();
  }
  const unsigned nx = static_cast<unsigned>((static_cast<size_t>(T) * (D / (2 * NP)) + 255) / 256);
  hipLaunchKernelGGL((unmix_kernel<TE, D>), dim3(nx, static_cast<unsigned>(H / 2 * B)), dim3(256),
                     0, stream, dv, static_cast<TE*>(dI), static_cast<const TE*>(vmix), B, T, mh,
                     part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (dtheta) {
    hipLaunchKernelGGL(dtheta_kernel, dim3(static_cast<unsigned>(H / 2)), dim3(256), 0, stream,
                       part, static_cast<int>(nx) * B, dtheta);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace mhr

size_t mhr_part_floats(int B, int H, int T, int D) {
  const size_t nx = (static_cast<size_t>(T) * (D / (2 * mhr::NP)) + 255) / 256;
  return nx * static_cast<size_t>(B) * (H / 2 > 0 ? H / 2 : 1);
}

hipError_t launch_mhr_prepare(int dtype, int B, int H, int T, int D, const void* p1,
                              const void* p2, const void* vi, void* q, void* k, void* v,
                              const float* rope_cos, const float* rope_sin, const float* theta,
                              int pairing, hipStream_t stream) {
  const Mhr mh{rope_cos, rope_sin, theta, pairing, H};
  if (dtype == 1 && D == 48)
    return mhr::run_prepare<uint16_t, 48>(B, H, T, p1, p2, vi, q, k, v, mh, stream);
  if (dtype == 1 && D == 80)
    return mhr::run_prepare<uint16_t, 80>(B, H, T, p1, p2, vi, q, k, v, mh, stream);
  if (dtype == 1) return mhr::run_prepare<uint16_t, 64>(B, H, T, p1, p2, vi, q, k, v, mh, stream);
  if (D == 64) return mhr::run_prepare<float, 64>(B, H, T, p1, p2, vi, q, k, v, mh, stream);
  return mhr::run_prepare<float, 32>(B, H, T, p1, p2, vi, q, k, v, mh, stream);
}

hipError_t launch_mhr_post(int dtype, int B, int H, int T, int D, const float* dq, float dq_scale,
                           const float* dk, const float* dv, const void* vmix, void* dp1,
                           void* dp2, void* dI, float* dtheta, float* part,
                           const float* rope_cos, const float* rope_sin, const float* theta,
                           int pairing, hipStream_t stream, const float* dl_part, int dl_npart,
                           float* dlambda) {
  const Mhr mh{rope_cos, rope_sin, theta, pairing, H};
  if (dtype == 1 && D == 80)
    return mhr::run_post<uint16_t, 80>(B, H, T, dq, dq_scale, dk, dv, vmix, dp1, dp2, dI, dtheta,
                                       part, mh, stream, dl_part, dl_npart, dlambda);
  if (dtype == 1 && D == 48)
    return mhr::run_post<uint16_t, 48>(B, H, T, dq, dq_scale, dk, dv, vmix, dp1, dp2, dI, dtheta,
                                       part, mh, stream, dl_part, dl_npart, dlambda);
  if (dtype == 1)
    return mhr::run_post<uint16_t, 64>(B, H, T, dq, dq_scale, dk, dv, vmix, dp1, dp2, dI, dtheta,
                                       part, mh, stream, dl_part, dl_npart, dlambda);
  if (D == 64)
    return mhr::run_post<float, 64>(B, H, T, dq, dq_scale, dk, dv, vmix, dp1, dp2, dI, dtheta,
                                    part, mh, stream, dl_part, dl_npart, dlambda);
  return mhr::run_post<float, 32>(B, H, T, dq, dq_scale, dk, dv, vmix, dp1, dp2, dI, dtheta, part,
                                  mh, stream, dl_part, dl_npart, dlambda);
}

}  // namespace rel
