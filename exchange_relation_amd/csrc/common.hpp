// Shared device helpers for librelation's gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rel {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 <-> fp32. Storage is raw 16-bit patterns; bf16 -> fp32 is exact, and
// fp32 -> bf16 rounds to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  __bf16 h = static_cast<__bf16>(f);
  return __builtin_bit_cast(uint16_t, h);
}

// Two fp32 values -> one word of two bf16 (round to nearest even); `lo` in
// bits 0..15.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Hardware base-2 exponential and reciprocal (v_exp_f32, v_rcp_f32). Both
// are accurate to about 1 ulp over the ranges used here; exp2 saturates to
// +inf / 0, and rcp(+inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// IEEE-754 maximum (NaN-propagating): v_maximum3_f32 on gfx950, which needs
// none of the quieting moves that fmaxf's NaN-ignoring form costs.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Exchanges between the two 32-lane halves of a wave (v_permlane32_swap):
// the swap returns {own value in lanes < 32, other half's in lanes >= 32}
// and {other half's in lanes < 32, own in lanes >= 32}. Call them with both
// partner lanes active (never inside a lane-divergent branch).
__device__ __forceinline__ float max_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return (threadIdx.x & 32) ? __uint_as_float(r[0]) : __uint_as_float(r[1]);
}

// LDS transposing read (ds_read_b64_tr_b16, gfx950). Within each group of 16
// lanes, lane i receives element (i & 3) of the 8-byte chunks that lanes
// (i >> 2) + {0, 4, 8, 12} of its group address. So if lane j of a group
// addresses row (r0 + (j >> 2)), columns c0 + 4 * (j & 3) .. +3 of a
// row-major bf16 tile, lane i receives rows r0 .. r0 + 3 of column c0 + i:
// a 4-deep MFMA operand fragment along the row index.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
  return __builtin_bit_cast(uint2, v);
}

// Element loads/stores for the two storage types.
template <typename TE> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_bits_to_f32(*p); }
  __device__ __forceinline__ static void store(uint16_t* p, float x) { *p = f32_to_bf16_bits(x); }
};

// A vector (or scalar) load. NT: a streaming load (the non-temporal hint), for
// data read once per call, so that it does not displace what the caches hold.
template <bool NT, typename V>
__device__ __forceinline__ V vload(const V* p) {
  if constexpr (NT) return __builtin_nontemporal_load(p);
  else return *p;
}

// One lane's D/8 consecutive elements of a row, widened to fp32, with one
// vector load (bf16 D=64: 16 B; fp32 D=64: 32 B; fp32 D=32: 16 B). bf16 rows
// of 48 or 80 elements: a lane's piece (6 or 10 elements) starts only 4-byte
// aligned, so it is read as 32-bit words.
template <typename TE, int D, bool NT>
struct RowPiece;

template <bool NT>
struct RowPiece<uint16_t, 64, NT> {
  __device__ __forceinline__ static void load(const uint16_t* p, float* x) {
    const u32x4 w = vload<NT>(reinterpret_cast<const u32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __uint_as_float(w[i] << 16);
      x[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};
template <bool NT>
struct RowPiece<float, 64, NT> {
  __device__ __forceinline__ static void load(const float* p, float* x) {
    const f32x4 a = vload<NT>(reinterpret_cast<const f32x4*>(p));
    const f32x4 b = vload<NT>(reinterpret_cast<const f32x4*>(p + 4));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[i] = a[i];
      x[4 + i] = b[i];
    }
  }
};
template <bool NT>
struct RowPiece<float, 32, NT> {
  __device__ __forceinline__ static void load(const float* p, float* x) {
    const f32x4 a = vload<NT>(reinterpret_cast<const f32x4*>(p));
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = a[i];
  }
};
template <int E, bool NT>
struct Bf16Words {
  __device__ __forceinline__ static void load(const uint16_t* p, float* x) {
    const uint32_t* w = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
    for (int i = 0; i < E / 2; ++i) {
      const uint32_t a = vload<NT>(w + i);
      x[2 * i] = __uint_as_float(a << 16);
      x[2 * i + 1] = __uint_as_float(a & 0xffff0000u);
    }
  }
};
template <bool NT>
struct RowPiece<uint16_t, 48, NT> : Bf16Words<6, NT> {};
template <bool NT>
struct RowPiece<uint16_t, 80, NT> : Bf16Words<10, NT> {};

template <typename TE, int D, bool NT = false>
__device__ __forceinline__ void load_row_piece(const TE* p, float* x) {
  RowPiece<TE, D, NT>::load(p, x);
}

// 8 bf16 <-> 8 fp32
__device__ __forceinline__ void unpack8(u32x4 w, float (&x)[8]) {
  const uint32_t a[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = __uint_as_float(a[i] << 16);
    x[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ u32x4 pack8(const float (&x)[8]) {
  const u32x4 w = {pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]), pack_bf16x2(x[4], x[5]),
                   pack_bf16x2(x[6], x[7])};
  return w;
}
// RoPE of 8 pairs (lo_e, hi_e) = (x_d, x_{d+D/2}) at one position (Sec. 3.1,
// rotate-half pairing): lo' = lo cos - hi sin, hi' = lo sin + hi cos.
__device__ __forceinline__ void rope8(u32x4& lo, u32x4& hi, const f32x4 (&cs)[2],
                                      const f32x4 (&sn)[2]) {
  float a[8], b[8];
  unpack8(lo, a);
  unpack8(hi, b);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float c = cs[e >> 2][e & 3], s_ = sn[e >> 2][e & 3];
    const float a2 = fmaf(a[e], c, -b[e] * s_);
    b[e] = fmaf(a[e], s_, b[e] * c);
    a[e] = a2;
  }
  lo = pack8(a);
  hi = pack8(b);
}

// Multi-Head Relation's upstream maps (Sec. 3.1-3.2, App. A.2.2-A.2.3): rotary tables cos / sin [T, D/2] fp32 (NULL: none) and
// one Givens angle per head pair (NULL: no mixing) with the pairing pattern
// (0: heads (0,1), (2,3), ...; 1: (1,2), ..., (H-1,0)) of H heads.
struct Mhr {
  const float* cos;
  const float* sin;
  const float* theta;
  int pairing;
  int H;
};

// Givens role of head h: its pair, its partner and the sign of the partner's
// term, I'_h = cos I_h + sgn sin I_partner (first of a pair: +, second: -).
__device__ __forceinline__ void givens_role(int h, int H, int pairing, int& pair, int& partner,
                                            float& sgn) {
  if (pairing == 0) {
    pair = h >> 1;
    partner = h ^ 1;
    sgn = (h & 1) ? -1.f : 1.f;
  } else if (h & 1) {  // first of (2p+1, 2p+2)
    pair = h >> 1;
    partner = (h + 1) % H;
    sgn = 1.f;
  } else {  // second of (h-1, h); head 0 closes the ring with head H-1
    pair = (h == 0 ? H : h) / 2 - 1;
    partner = (h + H - 1) % H;
    sgn = -1.f;
  }
}

}  // namespace rel
