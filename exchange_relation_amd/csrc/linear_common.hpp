// Device helpers shared by the Linear Relation kernels (linear.hip,
// linear_bwd.hip): tile constants, MFMA wrappers, DPP scans over the 16 rows
// of a sub-chunk, the chunk loader and the row-local part of the recurrence
// (Sec. 5.2: RoPE, Self, the normalised coordinates, the retention prefix).
#pragma once

#include "common.hpp"

namespace rel {
namespace linrel {

constexpr int D = 64;
constexpr int NW = 8;        // waves per workgroup
constexpr int NT = NW * 64;  // threads
constexpr int CH = NW * 16;  // tokens per chunk
constexpr int IS = 72;       // bf16 row stride of the tiles in LDS
constexpr int KS = 68;       // fp32 row stride of fp32 tiles
// A sub-chunk whose retention over its 16 tokens is above 2^kSafeLog2* on
// every channel uses the ratio form for its diagonal block. The forward's
// ratio factors stay within 2^+-120 and its largest partial sums (the masked
// entries, up to 2^120) within fp32; the gradient kernel multiplies its
// factors by dA = I . dE as well, so it keeps a wider margin.
constexpr float kSafeLog2Fwd = -120.f;
constexpr float kSafeLog2Bwd = -60.f;

typedef short s16x4 __attribute__((ext_vector_type(4)));


__device__ __forceinline__ bf16x8 cat(uint2 a, uint2 b) {
  const u32x4 w = {a.x, a.y, b.x, b.y};
  return __builtin_bit_cast(bf16x8, w);
}
__device__ __forceinline__ bf16x8 pack_x8(const float* x) {
  float t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = x[e];
  return __builtin_bit_cast(bf16x8, pack8(t));
}
__device__ __forceinline__ s16x4 pack_x4(f32x4 a) {
  const uint2 w = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
  return __builtin_bit_cast(s16x4, w);
}
__device__ __forceinline__ f32x4 mfma32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// inclusive prefix sum over the 16 lanes of a DPP row
template <int N>
__device__ __forceinline__ float row_shr(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 | N, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_prefix(float x) {
  x += row_shr<1>(x);
  x += row_shr<2>(x);
  x += row_shr<4>(x);
  x += row_shr<8>(x);
  return x;
}
// sum over the four 16-lane groups (the four channel groups of a row)
// lane 15 of each 16-lane row, broadcast over the row (DPP row_newbcast)
__device__ __forceinline__ float row_bcast15(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x15F, 0xF, 0xF, false));
}
// The exchanges between 16-lane rows use v_permlane16_swap / v_permlane32_swap
// (register moves, no LDS round trip).
__device__ __forceinline__ float sum_groups(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  return sum_across_halves(x);
}
__device__ __forceinline__ float min_groups(float x) {
  const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fminf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fminf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// One chunk's raw rows for one lane (slot s: channels 32s + 8g .. +7).
// Rows past T are loaded clamped and zeroed only where they are consumed
// (a select right after the load would make the prefetch wait for it).
struct Raw {
  u32x4 a1[2], a2[2], iv[2];
  f32x4 gg[4];
  f32x4 cs[2], sn[2];
  bool ok;
};

template <bool ROPE>
__device__ __forceinline__ void load_raw(Raw& r, const uint16_t* p1, const uint16_t* p2,
                                         const uint16_t* iv, const float* g, const float* rc,
                                         const float* rs, size_t base, int t, int T, int grp) {
  const bool ok = t < T;
  r.ok = ok;
  const size_t row = base + static_cast<size_t>(ok ? t : T - 1) * D + 8 * grp;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    r.a1[s] = *reinterpret_cast<const u32x4*>(p1 + row + 32 * s);
    r.a2[s] = *reinterpret_cast<const u32x4*>(p2 + row + 32 * s);
    r.iv[s] = *reinterpret_cast<const u32x4*>(iv + row + 32 * s);
#pragma unroll
    for (int h = 0; h < 2; ++h)
      r.gg[2 * s + h] = *reinterpret_cast<const f32x4*>(g + row + 32 * s + 4 * h);
  }
  if constexpr (ROPE) {
    const size_t tr = static_cast<size_t>(ok ? t : T - 1) * (D / 2) + 8 * grp;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      r.cs[h] = *reinterpret_cast<const f32x4*>(rc + tr + 4 * h);
      r.sn[h] = *reinterpret_cast<const f32x4*>(rs + tr + 4 * h);
    }
  }
}

// inclusive suffix sum over the 16 lanes of a DPP row (lane i: sum of lanes
// i..15)
template <int N>
__device__ __forceinline__ float row_shl(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 | N, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_suffix(float x) {
  x += row_shl<1>(x);
  x += row_shl<2>(x);
  x += row_shl<4>(x);
  x += row_shl<8>(x);
  return x;
}

// Row-local part of one sub-chunk row (lane (l16, grp): row l16, channels
// 8 grp + e and 32 + 8 grp + e in slots e and 8 + e): rotated coordinates,
// S, q = S p^_1, k = S p^_2, the inclusive prefix b2 of g (log2 units) over
// the sub-chunk and its total lw (the same on the 16 lanes of a group).
struct RowLocal {
  float x1[16], x2[16];  // rotated p1, p2
  float q[16], k[16], b2[16], lw[16];
  float S, inv1, inv2;   // 1 / ||x|| (0 for a zero row)
  bool safe;             // the diagonal block may use the ratio form
};

template <bool ROPE>
__device__ __forceinline__ void row_local(Raw& raw, float sl2, float safe_log2,
                                          RowLocal& o) {
  const u32x4 z = {0, 0, 0, 0};
  const f32x4 zf = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    raw.a1[s] = raw.ok ? raw.a1[s] : z;
    raw.a2[s] = raw.ok ? raw.a2[s] : z;
    raw.iv[s] = raw.ok ? raw.iv[s] : z;
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) raw.gg[h] = raw.ok ? raw.gg[h] : zf;
  unpack8(raw.a1[0], *reinterpret_cast<float(*)[8]>(&o.x1[0]));
  unpack8(raw.a1[1], *reinterpret_cast<float(*)[8]>(&o.x1[8]));
  unpack8(raw.a2[0], *reinterpret_cast<float(*)[8]>(&o.x2[0]));
  unpack8(raw.a2[1], *reinterpret_cast<float(*)[8]>(&o.x2[8]));
  if constexpr (ROPE) {  // rotate-half pairs (c, c + 32) sit in one lane
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float c = raw.cs[e >> 2][e & 3], s_ = raw.sn[e >> 2][e & 3];
      float x = o.x1[e], zz = o.x1[8 + e];
      o.x1[e] = fmaf(x, c, -zz * s_);
      o.x1[8 + e] = fmaf(x, s_, zz * c);
      x = o.x2[e];
      zz = o.x2[8 + e];
      o.x2[e] = fmaf(x, c, -zz * s_);
      o.x2[8 + e] = fmaf(x, s_, zz * c);
    }
  }
  float dot = 0.f, n1 = 0.f, n2 = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    dot = fmaf(o.x1[i], o.x2[i], dot);
    n1 = fmaf(o.x1[i], o.x1[i], n1);
    n2 = fmaf(o.x2[i], o.x2[i], n2);
  }
  dot = sum_groups(dot);
  n1 = sum_groups(n1);
  n2 = sum_groups(n2);
  o.S = fast_rcp(1.f + fast_exp2(-sl2 * dot));
  o.inv1 = n1 > 0.f ? __builtin_amdgcn_rsqf(n1) : 0.f;
  o.inv2 = n2 > 0.f ? __builtin_amdgcn_rsqf(n2) : 0.f;
  const float r1 = o.S * o.inv1, r2 = o.S * o.inv2;
  float lmin = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    o.q[i] = o.x1[i] * r1;
    o.k[i] = o.x2[i] * r2;
    o.b2[i] = row_prefix(raw.gg[i >> 2][i & 3] * kLog2e);
    o.lw[i] = row_bcast15(o.b2[i]);
    lmin = fminf(lmin, o.lw[i]);
  }
  // every lane holds the wave's minimum; make the branch scalar
  o.safe = __builtin_amdgcn_readfirstlane(min_groups(lmin) >= safe_log2 ? 1 : 0) != 0;
}

}  // namespace linrel
}  // namespace rel
