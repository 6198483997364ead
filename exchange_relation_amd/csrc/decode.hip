// Relation Cache decode: one new token per sequence over a KV-style cache.
//
// The new token sits at 1-based position i = n_hist + 1. Its Relation row
// (Sec. 3.1) has n_hist historical Exchange entries, read from cache slots
// [0, n_hist), and one Self entry from its own q and k. The history is split
// into chunks; every chunk is scanned with FlashRelation's running (m, l, z)
// (Sec. 5.1; App. A.3.1-A.3.3), the chunk partials are merged with the
// tile-merge rule of App. A.3.2, and the row is completed as in App. A.3.5.
// The new k / v are then written to slot n_hist, an exact copy.
//
// Kernel 1 (split): one workgroup per (chunk, b, h), 256 lanes = 32 groups of
// 8 lanes. A group handles one cache slot at a time, each lane D/8 of its
// elements, so a wave reads 8 consecutive 128-byte K rows (and V rows) per
// load: fully coalesced streaming. Groups interleave over the chunk and keep
// their own (m, l, z); the 32 group states are merged in LDS and one partial
// per chunk goes to the workspace. This kernel is HBM-bound by design.
// The first split workgroup of each (b, h) also appends k_new / v_new to slot
// n_hist (no split reads that slot).
// Kernel 2 (combine): one 64-lane wave per (b, h) merges the chunk partials
// (every partial load issued up front), adds Self and writes y / gate.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace rel {
namespace dec {

#ifndef REL_DECODE_CHUNK
#define REL_DECODE_CHUNK 512
#endif
#ifndef REL_DECODE_UNROLL
#define REL_DECODE_UNROLL 8
#endif
constexpr int kChunk = REL_DECODE_CHUNK;    // target slots per split workgroup
constexpr int kGroups = 32;                 // 8-lane groups per 256-lane workgroup
constexpr int kUnroll = REL_DECODE_UNROLL;  // slots per group per iteration (loads in flight)
constexpr int kBatch = 8;                   // partials loaded at once by the combine

inline int num_splits(int n) { return (n + kChunk - 1) / kChunk; }

// Partial record per (head, split): [m, l, z_0 .. z_{D-1}] in fp32, base-2
// domain (m is a log2 stabiliser; l, z are scaled by 2^-m).
template <typename TE, int D>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const TE* __restrict__ q, const TE* __restrict__ kn, const TE* __restrict__ vn,
    TE* __restrict__ kc, TE* __restrict__ vc, float* __restrict__ part, int capacity, int n,
    int nsplit, int chunk, float qscale) {
  constexpr int E = D / 8;
  __shared__ float s_m[kGroups], s_l[kGroups];
  __shared__ float s_z[kGroups][D + 1];

  const int tid = threadIdx.x;
  const int grp = tid >> 3;
  const int sub = tid & 7;
  const int split = blockIdx.x % nsplit;
  const int head = blockIdx.x / nsplit;
  const size_t cbase = static_cast<size_t>(head) * capacity * D;
  const int c0 = split * chunk;
  const int c1 = min(n, c0 + chunk);
  if (split == 0 && tid < D) {  // append: exact copy of the new token into slot n
    const size_t slot = cbase + static_cast<size_t>(n) * D + tid;
    kc[slot] = kn[static_cast<size_t>(head) * D + tid];
    vc[slot] = vn[static_cast<size_t>(head) * D + tid];
  }

  float qv[E];
  load_row_piece<TE, D>(q + static_cast<size_t>(head) * D + sub * E, qv);
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] *= qscale;

  float m = -INFINITY, l = 0.f, z[E];
#pragma unroll
  for (int e = 0; e < E; ++e) z[e] = 0.f;

  for (int s0 = c0 + grp; s0 < c1; s0 += kGroups * kUnroll) {
    float kx[kUnroll][E], vx[kUnroll][E];
    bool ok[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int slot = s0 + u * kGroups;
      ok[u] = slot < c1;
      const int sl = ok[u] ? slot : c0;  // in-range dummy for masked slots
      load_row_piece<TE, D>(kc + cbase + static_cast<size_t>(sl) * D + sub * E, kx[u]);
      load_row_piece<TE, D>(vc + cbase + static_cast<size_t>(sl) * D + sub * E, vx[u]);
    }
    float ev[kUnroll];
    float mx = m;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float acc = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) acc = fmaf(qv[e], kx[u][e], acc);
      acc += __shfl_xor(acc, 1, 8);
      acc += __shfl_xor(acc, 2, 8);
      acc += __shfl_xor(acc, 4, 8);
      // acc = u' = U * log2(e); E' = u' * sigmoid(U)
      const float sg = fast_rcp(1.0f + fast_exp2(-acc));
      ev[u] = ok[u] ? acc * sg : -INFINITY;
      mx = fmaxf(mx, ev[u]);
    }
    if (mx == -INFINITY) continue;  // nothing valid yet for this group
    const float a = fast_exp2(m - mx);  // m = -inf -> 0
    l *= a;
#pragma unroll
    for (int e = 0; e < E; ++e) z[e] *= a;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float p = fast_exp2(ev[u] - mx);  // -inf -> 0
      l += p;
#pragma unroll
      for (int e = 0; e < E; ++e) z[e] = fmaf(p, vx[u][e], z[e]);
    }
    m = mx;
  }

  // merge the 32 group states
  if (sub == 0) {
    s_m[grp] = m;
    s_l[grp] = l;
  }
#pragma unroll
  for (int e = 0; e < E; ++e) s_z[grp][sub * E + e] = z[e];
  __syncthreads();
  float* out = part + (static_cast<size_t>(head) * nsplit + split) * (D + 2);
  if (tid < D) {
    float M = -INFINITY;
    for (int g2 = 0; g2 < kGroups; ++g2) M = fmaxf(M, s_m[g2]);
    float Z = 0.f, Ls = 0.f;
    if (M != -INFINITY) {
      for (int g2 = 0; g2 < kGroups; ++g2) {
        const float w = fast_exp2(s_m[g2] - M);
        Z = fmaf(w, s_z[g2][tid], Z);
        Ls = fmaf(w, s_l[g2], Ls);
      }
    }
    out[2 + tid] = Z;
    if (tid == 0) {
      out[0] = M;
      out[1] = Ls;
    }
  }
}

template <typename TE, int D>
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const TE* __restrict__ q, const TE* __restrict__ kn, const TE* __restrict__ vn,
    TE* __restrict__ kc, TE* __restrict__ vc, const float* __restrict__ part, TE* __restrict__ y,
    float* __restrict__ gate, int capacity, int n, int nsplit, float qscale, float inv_tau,
    float lam) {
  const int tid = threadIdx.x;  // one lane per element d (lanes >= D idle)
  const int head = blockIdx.x;
  const bool act = tid < D;
  const size_t hv = static_cast<size_t>(head) * D;
  const float qd = act ? Elem<TE>::load(q + hv + tid) : 0.f;
  const float kd = act ? Elem<TE>::load(kn + hv + tid) : 0.f;
  const float vd = act ? Elem<TE>::load(vn + hv + tid) : 0.f;
  if (nsplit == 0) {  // no history: the append was not done by a split kernel
    if (act) {
      const size_t slot = (static_cast<size_t>(head) * capacity + n) * D + tid;
      kc[slot] = kn[hv + tid];
      vc[slot] = vn[hv + tid];
    }
  }

  // Self: u'_ii = scale*log2(e) * q . k_new
  float us = qd * kd;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) us += __shfl_xor(us, o);
  us *= qscale;

  // merge the chunk partials (App. A.3.2), kBatch partials per round with
  // all their loads issued before any is used
  float M = -INFINITY, Ls = 0.f, Z = 0.f;
  const float* ph = part + static_cast<size_t>(head) * nsplit * (D + 2);
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    float pm[kBatch], pl[kBatch], pz[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const bool ok = s0 + b < nsplit;
      const float* pr = ph + static_cast<size_t>(ok ? s0 + b : 0) * (D + 2);
      pm[b] = ok ? pr[0] : -INFINITY;
      pl[b] = ok ? pr[1] : 0.f;
      pz[b] = (ok && act) ? pr[2 + tid] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) Mn = fmaxf(Mn, pm[b]);
    if (Mn == -INFINITY) continue;  // nothing yet
    const float a = fast_exp2(M - Mn);  // M = -inf -> 0
    Ls *= a;
    Z *= a;
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const float w = fast_exp2(pm[b] - Mn);  // -inf -> 0
      Ls = fmaf(w, pl[b], Ls);
      Z = fmaf(w, pz[b], Z);
    }
    M = Mn;
  }
  const float S = fast_rcp(1.0f + fast_exp2(-us * inv_tau));  // sigmoid(U_ii / tau)
  float g = 0.f;
  if (Ls > 0.f) {
    const float A2 = M + fast_log2(Ls) - lam * fast_log2(static_cast<float>(n + 1));
    g = fast_rcp(1.0f + fast_exp2(S * kLog2e - A2));
  }
  const float yd = (1.0f - g) * vd + ((Ls > 0.f) ? g * Z * fast_rcp(Ls) : 0.f);
  if (act) Elem<TE>::store(y + hv + tid, yd);
  if (tid == 0 && gate) gate[head] = g;
}

template <typename TE, int D>
hipError_t run(int BH, const void* q, const void* k_new, const void* v_new, void* k_cache,
               void* v_cache, int capacity, int n, void* y, float* gate, void* ws, float scale,
               float tau, float lam, hipStream_t stream) {
  const float qscale = scale * kLog2e;
  float* part = static_cast<float*>(ws);
  int nsplit = 0;
  if (n > 0) {
    nsplit = num_splits(n);
    const int chunk = ((n + nsplit - 1) / nsplit + 31) / 32 * 32;
    nsplit = (n + chunk - 1) / chunk;
    hipLaunchKernelGGL((decode_split_kernel<TE, D>), dim3(static_cast<unsigned>(nsplit) * BH),
                       dim3(256), 0, stream, static_cast<const TE*>(q),
                       static_cast<const TE*>(k_new), static_cast<const TE*>(v_new),
                       static_cast<TE*>(k_cache), static_cast<TE*>(v_cache), part, capacity, n,
                       nsplit, chunk, qscale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_combine_kernel<TE, D>), dim3(BH), dim3(64), 0, stream,
                     static_cast<const TE*>(q), static_cast<const TE*>(k_new),
                     static_cast<const TE*>(v_new), static_cast<TE*>(k_cache),
                     static_cast<TE*>(v_cache), part, static_cast<TE*>(y), gate, capacity, n,
                     nsplit, qscale, 1.0f / tau, lam);
  return hipGetLastError();
}

}  // namespace dec

size_t decode_workspace_bytes(int dtype, int B, int H, int D, int capacity) {
  (void)dtype;
  const size_t ns = static_cast<size_t>(dec::num_splits(capacity > 0 ? capacity : 1));
  return static_cast<size_t>(B) * H * ns * (D + 2) * sizeof(float);
}

hipError_t launch_decode(int dtype, int B, int H, int D, const void* q, const void* k_new,
                         const void* v_new, void* k_cache, void* v_cache, int capacity,
                         int n_hist, void* y, float* gate, void* ws, float scale, float tau,
                         float lam, hipStream_t stream) {
  const int BH = B * H;
  if (dtype == 1)
    return dec::run<uint16_t, 64>(BH, q, k_new, v_new, k_cache, v_cache, capacity, n_hist, y,
                                  gate, ws, scale, tau, lam, stream);
  if (D == 64)
    return dec::run<float, 64>(BH, q, k_new, v_new, k_cache, v_cache, capacity, n_hist, y, gate,
                               ws, scale, tau, lam, stream);
  return dec::run<float, 32>(BH, q, k_new, v_new, k_cache, v_cache, capacity, n_hist, y, gate,
                             ws, scale, tau, lam, stream);
}

}  // namespace rel
