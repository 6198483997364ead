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
// load: fully coalesced streaming. The cache rows are read with the
// non-temporal hint: each is read once per step, and letting them through
// without displacing the caches took the 256-step decode at n = 4096 from 77
// to 66 us per step. Groups interleave over the chunk and keep
// their own (m, l, z); the 32 group states are merged in LDS and one partial
// per chunk goes to the workspace. This kernel is HBM-bound by design.
// The first split workgroup of each (b, h) also appends k_new / v_new to slot
// n_hist (no split reads that slot).
// Kernel 2 (combine): one 64-lane wave per (b, h) (lane: elements d = lane +
// 64 e) merges the chunk partials
// (every partial load issued up front), adds Self and writes y / gate.
//
// Whole-history mode (WHOLE, uniform lengths): when the batch has enough
// heads to fill the chip on its own (B * H >= kWholeHeads), every (b, h)
// gets ONE workgroup that scans its whole history, merges its 32 group
// states in LDS and completes the row itself (Self, A, g, y; App. A.3.5),
// with the append; no partials and no second launch (cache workload: 60.7
// us per step against 62.6 + 4.2 split and combine). Every workgroup streams
// at the same rate (their loads in flight are alike and HBM is the shared
// bound), so the workgroups that share a CU do not set the time. Ragged
// batches keep the split: there one workgroup per head would leave the
// longest histories to a few slow workgroups (measured 51 against 40 us per
// step at lengths uniform in [0, 4096]).
//
// Ragged batches: each sequence b has its own history length n_b (a device
// int array). The launch is sized for an upper bound of the lengths; a split
// workgroup whose chunk lies past its sequence's n_b exits at once, and the
// combine does the append. The ragged grid is split-major (chunk s of every
// head before chunk s + 1 of any), so the chunks that hold work are spread
// over the whole launch rather than bunched by sequence: 45.9 -> 34.3 us per
// step at lengths uniform in [0, 4096] (32 x 12 heads). A sequence whose n_b is out of range (negative,
// above the bound, or without a free slot) gets NaN outputs and no append.
#include <math.h>

#include <mutex>

#include "common.hpp"
#include "launch.hpp"

namespace rel {
namespace dec {

#ifndef REL_DECODE_CHUNK
#define REL_DECODE_CHUNK 256
#endif
#ifndef REL_DECODE_UNROLL
#define REL_DECODE_UNROLL 8
#endif
// target slots per split workgroup: one pass of the 32 groups x 8 slots
constexpr int kChunk = REL_DECODE_CHUNK;
constexpr int kGroups = 32;                 // 8-lane groups per 256-lane workgroup
constexpr int kUnroll = REL_DECODE_UNROLL;  // slots per group per iteration (loads in flight)
constexpr int kBatch = 8;                   // partials loaded at once by the combine
constexpr int kWholeHeads = 256;            // heads from which one workgroup per head fills the chip

__host__ __device__ inline int num_splits(int n) { return (n + kChunk - 1) / kChunk; }

// Split plan of a history of n >= 1 slots: chunks of a multiple of 32 slots,
// about kChunk each, and the number of chunks (<= num_splits(n)).
struct SplitPlan {
  int nsplit, chunk;
};
__host__ __device__ inline SplitPlan split_plan(int n) {
  const int ns = num_splits(n);
  const int chunk = ((n + ns - 1) / ns + 31) / 32 * 32;
  return {(n + chunk - 1) / chunk, chunk};
}

// Partial record per (head, split): [m, l, z_0 .. z_{D-1}] in fp32, base-2
// domain (m is a log2 stabiliser; l, z are scaled by 2^-m).
// Uniform batches pass the common length in n (and nh = NULL); ragged ones
// pass the per-sequence lengths nh[B], the heads per sequence H and the
// length bound n (the grid has nsplit = num_splits(bound) chunks per head).
template <typename TE, int D, bool RAGGED, bool WHOLE = false>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const TE* __restrict__ q, const TE* __restrict__ kn, const TE* __restrict__ vn,
    TE* __restrict__ kc, TE* __restrict__ vc, float* __restrict__ part, int capacity, int n,
    const int* __restrict__ nh, int H, int nsplit, int chunk, float qscale,
    TE* __restrict__ y = nullptr, float* __restrict__ gate = nullptr, float inv_tau = 0.f,
    float lam = 0.f) {
  constexpr int E = D / 8;
  __shared__ float s_m[kGroups], s_l[kGroups];
  __shared__ float s_z[kGroups][D + 1];

  const int tid = threadIdx.x;
  const int grp = tid >> 3;
  const int sub = tid & 7;
  // ragged: split-major grid (every head's first chunk is dispatched first)
  const int bhg = gridDim.x / nsplit;
  const int split = WHOLE ? 0 : RAGGED ? blockIdx.x / bhg : blockIdx.x % nsplit;
  const int head = WHOLE ? blockIdx.x : RAGGED ? blockIdx.x % bhg : blockIdx.x / nsplit;
  const size_t cbase = static_cast<size_t>(head) * capacity * D;
  const size_t hv = static_cast<size_t>(head) * D;
  static_assert(!(RAGGED && WHOLE), "the whole-history mode is for uniform lengths");
  if (RAGGED) {
    const int bound = n;
    n = nh[head / H];
    if (n < 1 || n > bound || n >= capacity) return;  // no history, or out of range
    const SplitPlan sp = split_plan(n);
    if (split >= sp.nsplit) return;
    chunk = sp.chunk;
  }
  if (WHOLE) chunk = n;
  const int c0 = split * chunk;
  const int c1 = min(n, c0 + chunk);
  if (!RAGGED && split == 0 && tid < D) {  // append: exact copy of the new token into slot n
    const size_t slot = cbase + static_cast<size_t>(n) * D + tid;
    kc[slot] = kn[hv + tid];
    vc[slot] = vn[hv + tid];
  }

  float qv[E];
  load_row_piece<TE, D>(q + hv + sub * E, qv);
#pragma unroll
  for (int e = 0; e < E; ++e) qv[e] *= qscale;
  float us = 0.f;  // WHOLE: u'_ii = scale*log2(e) * q . k_new, in every lane of each group
  if (WHOLE) {
    float kx[E];
    load_row_piece<TE, D>(kn + hv + sub * E, kx);
#pragma unroll
    for (int e = 0; e < E; ++e) us = fmaf(qv[e], kx[e], us);
    us += __shfl_xor(us, 1, 8);
    us += __shfl_xor(us, 2, 8);
    us += __shfl_xor(us, 4, 8);
  }

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
      load_row_piece<TE, D, true>(kc + cbase + static_cast<size_t>(sl) * D + sub * E, kx[u]);
      load_row_piece<TE, D, true>(vc + cbase + static_cast<size_t>(sl) * D + sub * E, vx[u]);
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
    if (WHOLE) {  // row completion (App. A.3.5), base-2 domain
      const float S = fast_rcp(1.0f + fast_exp2(-us * inv_tau));  // sigmoid(U_ii / tau)
      float g = 0.f;
      if (Ls > 0.f) {
        const float A2 = M + fast_log2(Ls) - lam * fast_log2(static_cast<float>(n + 1));
        g = fast_rcp(1.0f + fast_exp2(S * kLog2e - A2));
      }
      const float gl = (Ls > 0.f) ? g * fast_rcp(Ls) : 0.f;
      Elem<TE>::store(y + hv + tid, (1.0f - g) * Elem<TE>::load(vn + hv + tid) + gl * Z);
      if (tid == 0 && gate) gate[head] = g;
    } else {
      float* out = part + (static_cast<size_t>(head) * nsplit + split) * (D + 2);
      out[2 + tid] = Z;
      if (tid == 0) {
        out[0] = M;
        out[1] = Ls;
      }
    }
  }
}

// Uniform: n is the common length and nsplit the chunks per head (0 when
// n = 0). Ragged: n is the length bound, nh[B] the lengths, H the heads per
// sequence and pstride the chunks per head of the split grid.
template <typename TE, int D, bool RAGGED>
__global__ __launch_bounds__(64) void decode_combine_kernel(
    const TE* __restrict__ q, const TE* __restrict__ kn, const TE* __restrict__ vn,
    TE* __restrict__ kc, TE* __restrict__ vc, const float* __restrict__ part, TE* __restrict__ y,
    float* __restrict__ gate, int capacity, int n, const int* __restrict__ nh, int H, int nsplit,
    int pstride, float qscale, float inv_tau, float lam) {
  constexpr int EL = (D + 63) / 64;  // elements per lane: d = lane + 64 e
  const int tid = threadIdx.x;
  const int head = blockIdx.x;
  const size_t hv = static_cast<size_t>(head) * D;
  bool act[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) act[e] = tid + 64 * e < D;
  // Every load that does not depend on the sequence's length is issued
  // first: the new token's q / k / v and, for a ragged batch, every partial
  // slot of the head (the grid's pstride chunks; slots past the sequence's
  // own chunks hold stale values and are dropped by selects below).
  const int bound = n;
  if (RAGGED) n = nh[head / H];
  float qd[EL], kd[EL], vd[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    const int d = act[e] ? tid + 64 * e : 0;
    qd[e] = Elem<TE>::load(q + hv + d);
    kd[e] = Elem<TE>::load(kn + hv + d);
    vd[e] = Elem<TE>::load(vn + hv + d);
  }
  const float* ph = part + static_cast<size_t>(head) * (RAGGED ? pstride : nsplit) * (D + 2);
  float M = -INFINITY, Ls = 0.f, Z[EL];
#pragma unroll
  for (int e = 0; e < EL; ++e) Z[e] = 0.f;
  // merge the chunk partials (App. A.3.2), kBatch partials per round (2 kBatch
  // for a ragged batch) with all their loads issued before any is used
  auto merge = [&](int s0, int ns, int nvalid) {
    constexpr int KB = RAGGED ? 2 * kBatch : kBatch;
    float pm[KB], pl[KB], pz[KB][EL];
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const bool in = s0 + b < ns;
      const float* pr = ph + static_cast<size_t>(in ? s0 + b : 0) * (D + 2);
      pm[b] = pr[0];
      pl[b] = pr[1];
#pragma unroll
      for (int e = 0; e < EL; ++e) pz[b][e] = pr[2 + (act[e] ? tid + 64 * e : 0)];
    }
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const bool ok = s0 + b < nvalid;
      pm[b] = ok ? pm[b] : -INFINITY;
      pl[b] = ok ? pl[b] : 0.f;
#pragma unroll
      for (int e = 0; e < EL; ++e) pz[b][e] = (ok && act[e]) ? pz[b][e] : 0.f;
    }
    float Mn = M;
#pragma unroll
    for (int b = 0; b < KB; ++b) Mn = fmaxf(Mn, pm[b]);
    if (Mn == -INFINITY) return;  // nothing yet
    const float a = fast_exp2(M - Mn);  // M = -inf -> 0
    Ls *= a;
#pragma unroll
    for (int e = 0; e < EL; ++e) Z[e] *= a;
#pragma unroll
    for (int b = 0; b < KB; ++b) {
      const float w = fast_exp2(pm[b] - Mn);  // -inf -> 0
      Ls = fmaf(w, pl[b], Ls);
#pragma unroll
      for (int e = 0; e < EL; ++e) Z[e] = fmaf(w, pz[b][e], Z[e]);
    }
    M = Mn;
  };
  if (RAGGED) {
    const bool bad = n < 0 || n > bound || n >= capacity;
    if (bad) {  // out of range: NaN outputs, no append
#pragma unroll
      for (int e = 0; e < EL; ++e)
        if (act[e]) Elem<TE>::store(y + hv + tid + 64 * e, NAN);
      if (tid == 0 && gate) gate[head] = NAN;
      return;
    }
  }
  if (RAGGED || nsplit == 0) {  // the append was not done by a split kernel
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      if (!act[e]) continue;
      const size_t slot = (static_cast<size_t>(head) * capacity + n) * D + tid + 64 * e;
      kc[slot] = kn[hv + tid + 64 * e];
      vc[slot] = vn[hv + tid + 64 * e];
    }
  }
  // Self: u'_ii = scale*log2(e) * q . k_new
  float us = 0.f;
#pragma unroll
  for (int e = 0; e < EL; ++e) us = act[e] ? fmaf(qd[e], kd[e], us) : us;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) us += __shfl_xor(us, o);
  us *= qscale;

  if (RAGGED) {
    const int nvalid = n > 0 ? split_plan(n).nsplit : 0;
    for (int s0 = 0; s0 < pstride; s0 += 2 * kBatch) merge(s0, pstride, nvalid);
  } else {
    for (int s0 = 0; s0 < nsplit; s0 += kBatch) merge(s0, nsplit, nsplit);
  }
  const float S = fast_rcp(1.0f + fast_exp2(-us * inv_tau));  // sigmoid(U_ii / tau)
  float g = 0.f;
  if (Ls > 0.f) {
    const float A2 = M + fast_log2(Ls) - lam * fast_log2(static_cast<float>(n + 1));
    g = fast_rcp(1.0f + fast_exp2(S * kLog2e - A2));
  }
  const float gl = (Ls > 0.f) ? g * fast_rcp(Ls) : 0.f;
#pragma unroll
  for (int e = 0; e < EL; ++e)
    if (act[e]) Elem<TE>::store(y + hv + tid + 64 * e, (1.0f - g) * vd[e] + gl * Z[e]);
  if (tid == 0 && gate) gate[head] = g;
}

// nh == NULL: uniform length n. Otherwise per-sequence lengths nh[B] with
// upper bound n.
template <typename TE, int D>
hipError_t run(int BH, int H, const void* q, const void* k_new, const void* v_new, void* k_cache,
               void* v_cache, int capacity, int n, const int* nh, void* y, float* gate, void* ws,
               float scale, float tau, float lam, hipStream_t stream) {
  const float qscale = scale * kLog2e;
  float* part = static_cast<float*>(ws);
  const TE* qt = static_cast<const TE*>(q);
  const TE* knt = static_cast<const TE*>(k_new);
  const TE* vnt = static_cast<const TE*>(v_new);
  TE* kct = static_cast<TE*>(k_cache);
  TE* vct = static_cast<TE*>(v_cache);
  int nsplit = 0;
  if (nh == nullptr && BH >= kWholeHeads && n > 0) {  // one workgroup per head completes its row
    hipLaunchKernelGGL((decode_split_kernel<TE, D, false, true>), dim3(BH), dim3(256), 0, stream,
                       qt, knt, vnt, kct, vct, part, capacity, n, nullptr, H, 1, 0, qscale,
                       static_cast<TE*>(y), gate, 1.0f / tau, lam);
    return hipGetLastError();
  }
  if (nh == nullptr) {
    if (n > 0) {
      const SplitPlan sp = split_plan(n);
      nsplit = sp.nsplit;
      hipLaunchKernelGGL((decode_split_kernel<TE, D, false>),
                         dim3(static_cast<unsigned>(nsplit) * BH), dim3(256), 0, stream, qt, knt,
                         vnt, kct, vct, part, capacity, n, nullptr, H, nsplit, sp.chunk, qscale);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((decode_combine_kernel<TE, D, false>), dim3(BH), dim3(64), 0, stream, qt,
                       knt, vnt, kct, vct, part, static_cast<TE*>(y), gate, capacity, n, nullptr,
                       H, nsplit, nsplit, qscale, 1.0f / tau, lam);
    return hipGetLastError();
  }
  if (n > 0) {
    nsplit = num_splits(n);  // chunks per head of the grid: enough for any length <= n
    hipLaunchKernelGGL((decode_split_kernel<TE, D, true>), dim3(static_cast<unsigned>(nsplit) * BH),
                       dim3(256), 0, stream, qt, knt, vnt, kct, vct, part, capacity, n, nh, H,
                       nsplit, 0, qscale);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((decode_combine_kernel<TE, D, true>), dim3(BH), dim3(64), 0, stream, qt, knt,
                     vnt, kct, vct, part, static_cast<TE*>(y), gate, capacity, n, nh, H, 0, nsplit,
                     qscale, 1.0f / tau, lam);
  return hipGetLastError();
}

}  // namespace dec

// ---- allocation-free decode: the workspace lives in a static device array.
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends; the host uses the address hipGetSymbolAddress returns for
// the current device (the array's name is only a host-side stand-in). The
// decode kernels write every partial they read within the call, so nothing
// in it has to start at zero; it keeps the last call's partials.
namespace dec {
constexpr size_t kScratchBytes = 8u << 20;
constexpr int kMaxDevices = 64;
}  // namespace dec

static __device__ __align__(256) unsigned char scratch[dec::kScratchBytes];

namespace dec {
namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's scratch address, looked up at the first call on the device
// (with that device current) and kept.
hipError_t scratch_for_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (stream != nullptr) {
    hipDevice_t sdev = -1;
    if ((e = hipStreamGetDevice(stream, &sdev)) != hipSuccess) return e;
    if (sdev != dev) return hipErrorInvalidDevice;  // the stream must be the current device's
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if ((e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch))) != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}
}  // namespace
}  // namespace dec

size_t decode_scratch_bytes() { return dec::kScratchBytes; }

hipError_t launch_decode_noalloc(int dtype, int B, int H, int D, const void* q,
                                 const void* k_new, const void* v_new, void* k_cache,
                                 void* v_cache, int capacity, int n_hist, void* y, float* gate,
                                 float scale, float tau, float lam, hipStream_t stream) {
  void* ws = nullptr;
  hipError_t e = dec::scratch_for_device(stream, &ws);
  if (e != hipSuccess) return e;
  return launch_decode(dtype, B, H, D, q, k_new, v_new, k_cache, v_cache, capacity, n_hist,
                       nullptr, y, gate, ws, scale, tau, lam, stream);
}

size_t decode_uniform_need_bytes(int B, int H, int D, int n_hist) {
  const long long bh = static_cast<long long>(B) * H;
  if (n_hist <= 0 || bh >= dec::kWholeHeads) return 0;  // no partials: combine only, or WHOLE
  return static_cast<size_t>(bh) * dec::split_plan(n_hist).nsplit * (D + 2) * sizeof(float);
}

size_t decode_workspace_bytes(int dtype, int B, int H, int D, int capacity) {
  (void)dtype;
  const size_t ns = static_cast<size_t>(dec::num_splits(capacity > 0 ? capacity : 1));
  return static_cast<size_t>(B) * H * ns * (D + 2) * sizeof(float);
}

hipError_t launch_decode(int dtype, int B, int H, int D, const void* q, const void* k_new,
                         const void* v_new, void* k_cache, void* v_cache, int capacity,
                         int n_hist, const int* n_hist_dev, void* y, float* gate, void* ws,
                         float scale, float tau, float lam, hipStream_t stream) {
  const int BH = B * H;
  if (dtype == 1 && D == 48)
    return dec::run<uint16_t, 48>(BH, H, q, k_new, v_new, k_cache, v_cache, capacity, n_hist,
                                  n_hist_dev, y, gate, ws, scale, tau, lam, stream);
  if (dtype == 1 && D == 80)
    return dec::run<uint16_t, 80>(BH, H, q, k_new, v_new, k_cache, v_cache, capacity, n_hist,
                                  n_hist_dev, y, gate, ws, scale, tau, lam, stream);
  if (dtype == 1)
    return dec::run<uint16_t, 64>(BH, H, q, k_new, v_new, k_cache, v_cache, capacity, n_hist,
                                  n_hist_dev, y, gate, ws, scale, tau, lam, stream);
  if (D == 64)
    return dec::run<float, 64>(BH, H, q, k_new, v_new, k_cache, v_cache, capacity, n_hist,
                               n_hist_dev, y, gate, ws, scale, tau, lam, stream);
  return dec::run<float, 32>(BH, H, q, k_new, v_new, k_cache, v_cache, capacity, n_hist,
                             n_hist_dev, y, gate, ws, scale, tau, lam, stream);
}

}  // namespace rel
