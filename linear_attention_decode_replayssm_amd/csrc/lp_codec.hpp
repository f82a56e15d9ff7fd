// lp_codec.hpp -- low-precision checkpoint codecs shared by the Mamba-2 and
// Gated DeltaNet kernels: bfloat16 (round to nearest even) and OCP FP8 E4M3
// with one fp32 scale per (sequence, head) tile.
//
// Encoding of a tile for E4M3: scale = amax / 448 in fp32 (1 if that is 0,
// or if the tile holds NaN or an infinity), code = E4M3(s / scale) with the
// fp32 quotient rounded once and the conversion saturating at +-448.
// Decoding: value = code * scale.
//
// Tile geometry used by the whole-tile helpers: NTH threads hold an fp32 tile
// of ROWS x COLS values, thread t owning the float4 at column group
// cl = t % LPR (LPR = COLS / 4) of rows r0 + k * RPL, r0 = t / LPR,
// k = 0..NLD-1.
#pragma once

#include "common.hpp"

namespace rssm {

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// bf16 round-to-nearest-even of an fp32 value (NaN -> quiet NaN, sign kept).
__device__ __forceinline__ uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) & 0x8000u) | 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// OCP E4M3 code pair -> fp32 via the gfx950 conversion (bytes 0,1 or 2,3).
__device__ __forceinline__ f32x2 e4m3_pair(uint32_t w, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
            : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
}

// Four fp32 values (already divided by the scale) -> four E4M3 codes.
// Values are clamped to the largest finite magnitude first, so the
// conversion never overflows: saturating, round to nearest even.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -448.f), 448.f);
  b = fminf(fmaxf(b, -448.f), 448.f);
  c = fminf(fmaxf(c, -448.f), 448.f);
  d = fminf(fmaxf(d, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
  return (uint32_t)w;
}

// As e4m3_pack4, for a tile that holds NaN or an infinity: infinities
// saturate to +-448 like any large value; a NaN gets the E4M3 NaN code with
// its sign (the clamp above would have turned it into a number).
__device__ inline uint32_t e4m3_pack4_nonfinite(float a, float b, float c, float d) {
  uint32_t w = e4m3_pack4(a, b, c, d);
  const float v[4] = {a, b, c, d};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (v[i] != v[i]) {
      const uint32_t nan = ((__float_as_uint(v[i]) >> 24) & 0x80u) | 0x7Fu;
      w = (w & ~(0xFFu << (8 * i))) | (nan << (8 * i));
    }
  }
  return w;
}

// One 16-byte lane load of EB-byte elements -> 16 / EB fp32 values (E4M3
// values unscaled).
template <int EB>
__device__ __forceinline__ void expand(u32x4 w, float (&f)[16 / EB]) {
  if constexpr (EB == 4) {
#pragma unroll
    for (int e = 0; e < 4; ++e) f[e] = __uint_as_float(w[e]);
  } else if constexpr (EB == 2) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[2 * e] = bf16_lo(w[e]);
      f[2 * e + 1] = bf16_hi(w[e]);
    }
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const f32x2 lo = e4m3_pair(w[e], false), hi = e4m3_pair(w[e], true);
      f[4 * e] = lo.x;
      f[4 * e + 1] = lo.y;
      f[4 * e + 2] = hi.x;
      f[4 * e + 3] = hi.y;
    }
  }
}

constexpr int kLpBf16 = 1, kLpE4m3 = 2;

// ---- E4M3 tile encoder -----------------------------------------------------
// The scale needs the tile's largest magnitude.  It is taken on the bit
// patterns: with the sign cleared, unsigned order is magnitude order, and an
// infinity (0x7f800000) or a NaN (above it) is larger than every finite value,
// so one integer max per element both finds amax and detects a non-finite
// tile.
//
// The codes need the fp32 quotient v / scale rounded once, as an IEEE
// division rounds it.  The division instruction sequence costs about ten
// instructions per element; the tile's scale is fixed, so the quotient is
// formed in four by one correction step of a reciprocal (Markstein's method,
// "IA-64 and Elementary Functions", 2000): write scale = m 2^-k with m in
// [1, 2), take y = RN(1/m) once per tile, and per element
//   a = v 2^k (exact),  q0 = RN(a y),  r = fma(q0, m, -a) = q0 m - a (exact),
//   q = fma(-r, y, q0) = RN(a / m) = RN(v / scale).
// The prescaling keeps the residual r a normal number, which the exactness of
// the correction needs.  Checked against the IEEE quotient on 1.2e9 operand
// pairs spanning every binade, subnormal scales and signed zeros: equal
// wherever |v / scale| >= 2^-60, and below that (where every code is +-0)
// of the same sign.  The negation sits on the FMA operands so that a zero
// keeps its sign.
struct E4m3Scale {
  float scale;  // the tile's scale: amax / 448, or 1 (zero or non-finite tile, or amax / 448 == 0)
  float m, y;   // scale 2^k in [1, 2) and RN(1 / m)
  int k;
  bool fin;     // the tile holds no NaN and no infinity
};

__device__ __forceinline__ E4m3Scale e4m3_scale_of(uint32_t amax_bits) {
  E4m3Scale s;
  s.fin = amax_bits < 0x7f800000u;
  const float q = __uint_as_float(amax_bits) / 448.f;
  s.scale = (s.fin && q > 0.f) ? q : 1.f;
  int e;
  const float mant = frexpf(s.scale, &e);   // scale = mant 2^e, mant in [0.5, 1)
  s.k = 1 - e;
  s.m = 2.f * mant;
  s.y = 1.f / s.m;
  return s;
}

__device__ __forceinline__ float e4m3_quot(float v, const E4m3Scale& s) {
#pragma clang fp contract(off)
  const float a = __builtin_amdgcn_ldexpf(v, s.k);
  const float q0 = a * s.y;
  const float r = __builtin_fmaf(q0, s.m, -a);
  return __builtin_fmaf(-r, s.y, q0);
}

// Four fp32 values -> four E4M3 codes of a tile with scale s (the non-finite
// path encodes the values unscaled, as the scale is then 1).
__device__ __forceinline__ uint32_t e4m3_encode4(f32x4 v, const E4m3Scale& s) {
  if (s.fin)
    return e4m3_pack4(e4m3_quot(v.x, s), e4m3_quot(v.y, s), e4m3_quot(v.z, s), e4m3_quot(v.w, s));
  return e4m3_pack4_nonfinite(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint32_t abs_bits_max(uint32_t m, f32x4 v) {
  const uint32_t a = __float_as_uint(v.x) & 0x7fffffffu, b = __float_as_uint(v.y) & 0x7fffffffu;
  const uint32_t c = __float_as_uint(v.z) & 0x7fffffffu, d = __float_as_uint(v.w) & 0x7fffffffu;
  return max(max(m, max(a, b)), max(c, d));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
  m = max(m, __float_as_uint(rpartner<32>(__uint_as_float(m))));
  m = max(m, __float_as_uint(rpartner<16>(__uint_as_float(m))));
  m = max(m, __float_as_uint(rpartner<8>(__uint_as_float(m))));
  m = max(m, __float_as_uint(rpartner<4>(__uint_as_float(m))));
  m = max(m, __float_as_uint(rpartner<2>(__uint_as_float(m))));
  m = max(m, __float_as_uint(rpartner<1>(__uint_as_float(m))));
  return m;
}

// Scale of the tile held in the geometry above (all NTH threads call it; it
// contains barriers).  red: NTH / 64 words of LDS.
template <int NTH, int NLD>
__device__ E4m3Scale tile_e4m3_scale(const f32x4 (&hv)[NLD], uint32_t* red) {
  uint32_t m = 0u;
#pragma unroll
  for (int k = 0; k < NLD; ++k) m = abs_bits_max(m, hv[k]);
  m = wave_max_u32(m);
  __syncthreads();   // red may still be read by a previous use
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < NTH / 64; ++w) r = max(r, red[w]);
  return e4m3_scale_of(r);
}

// Write the low-precision image of an fp32 tile held in the geometry above.
// lp: the tile's first code (bf16 bits or E4M3 bytes, row pitch COLS);
// scale_out: the tile's scale (E4M3 only; written by thread 0).  Raises
// kStatusNonfinite for an E4M3 tile holding NaN or an infinity.  Contains
// barriers (E4M3): all threads call it.
template <int LP, int NTH, int NLD, int RPL, int COLS>
__device__ void store_lp_tile(const f32x4 (&hv)[NLD], void* lp, float* scale_out,
                              uint32_t* status, int r0, int cl, float* red) {
  if constexpr (LP == kLpBf16) {
    uint16_t* base = reinterpret_cast<uint16_t*>(lp);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      u32x2 w;
      w.x = bf16_rne(hv[k].x) | (bf16_rne(hv[k].y) << 16);
      w.y = bf16_rne(hv[k].z) | (bf16_rne(hv[k].w) << 16);
      *reinterpret_cast<u32x2*>(base + (k * RPL + r0) * COLS + cl * 4) = w;
    }
  } else {
    const E4m3Scale sc = tile_e4m3_scale<NTH, NLD>(hv, reinterpret_cast<uint32_t*>(red));
    if (!sc.fin && threadIdx.x == 0) raise_status(status, kStatusNonfinite);
    uint8_t* base = reinterpret_cast<uint8_t*>(lp);
#pragma unroll
    for (int k = 0; k < NLD; ++k)
      *reinterpret_cast<uint32_t*>(base + (k * RPL + r0) * COLS + cl * 4) = e4m3_encode4(hv[k], sc);
    if (threadIdx.x == 0) *scale_out = sc.scale;
  }
}

// Read a low-precision tile into the fp32 geometry (exact value for bf16;
// code * scale rounded to fp32 for E4M3).
template <int LP, int NLD, int RPL, int COLS>
__device__ void load_lp_tile(f32x4 (&hv)[NLD], const void* lp, const float* scale_in, int r0,
                             int cl) {
  if constexpr (LP == kLpBf16) {
    const uint16_t* base = reinterpret_cast<const uint16_t*>(lp);
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const u32x2 w = *reinterpret_cast<const u32x2*>(base + (k * RPL + r0) * COLS + cl * 4);
      hv[k] = f32x4{bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y)};
    }
  } else {
    const uint8_t* base = reinterpret_cast<const uint8_t*>(lp);
    const float scale = *scale_in;
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const uint32_t w = *reinterpret_cast<const uint32_t*>(base + (k * RPL + r0) * COLS + cl * 4);
      const f32x2 lo = e4m3_pair(w, false), hi = e4m3_pair(w, true);
      hv[k] = f32x4{lo.x * scale, lo.y * scale, hi.x * scale, hi.y * scale};
    }
  }
}

}  // namespace rssm
