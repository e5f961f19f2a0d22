// Device-side helpers shared by the HIP kernels of the CSA/HCA core (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

namespace csa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));

// DT_MX4: OCP MXFP4 -- FP4 E2M1 codes packed two per byte (the even channel in
// the low nibble) with one E8M0 scale byte per 32 channels in a separate array
// DT_MIX: mixed KV rows -- the first c - rope_dim channels as e4m3 codes (one
// fp32 scale per row in a separate array), then the last rope_dim channels as
// bf16: c + rope_dim bytes per row
enum : int { DT_F32 = 0, DT_BF16 = 1, DT_FP8 = 2, DT_MX4 = 3, DT_MIX = 4 };

// ---- scalar conversions ---------------------------------------------------
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(((uint32_t)b) << 16);
}

// round-to-nearest-even fp32 -> bf16 bits (NaN kept quiet)
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7fffu + lsb;
  return (uint16_t)(u >> 16);
}

// two fp32 -> packed bf16x2 (low half = a)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}

// OCP e4m3fn encode, round to nearest even, saturating to +-448 (NaN -> 0x7f).
// Subnormal range |v| < 2^-6 has a fixed step of 2^-9.
__device__ __forceinline__ uint8_t f32_to_e4m3(float v) {
  if (v != v) return 0x7f;
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // 2^-6
    code = (uint32_t)rintf(a * 512.0f);      // 0..8 (8 is the smallest normal)
  } else {
    int ex;
    float mant = frexpf(a, &ex);             // a = mant * 2^ex, mant in [0.5, 1)
    int E = ex - 1;
    uint32_t f = (uint32_t)rintf((mant * 2.0f - 1.0f) * 8.0f);
    if (f == 8u) { f = 0u; ++E; }
    code = ((uint32_t)(E + 7) << 3) | f;
  }
  return (uint8_t)(sign | code);
}

// ---- OCP MX, FP4 E2M1 elements with an E8M0 scale per block of 32 ----------
// Shared exponent of a block: floor(log2(amax)) - 2 (E2M1's largest power of
// two is 2^2), clamped to E8M0's [-127, 127]; a zero (or fp32-subnormal)
// maximum gives -127.  The scale byte is the exponent + 127.
__device__ __forceinline__ int mx4_shared_exp(float amax) {
  const int e = (int)((__float_as_uint(amax) >> 23) & 0xff);   // amax >= 0
  return e == 0 ? -127 : min(max(e - 127 - 2, -127), 127);
}
// E2M1 code of y (a value already divided by its block scale): round to the
// nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even code (mantissa bit
// 0), saturating at 6; the sign goes to bit 3
__device__ __forceinline__ uint32_t f32_to_e2m1(float y) {
  const float a = fabsf(y);
  const uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
                     (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(y) >> 28) & 8u);
}
// value of an E2M1 code (exact)
__device__ __forceinline__ float e2m1_to_f32(uint32_t code) {
  const uint32_t e = (code >> 1) & 3u, m = code & 1u;
  const float mag = e == 0 ? 0.5f * (float)m : ldexpf(1.0f + 0.5f * (float)m, (int)e - 1);
  return (code & 8u) ? -mag : mag;
}

// order-preserving map of a float score to uint32 (-0.0 canonicalised to +0.0)
__device__ __forceinline__ uint32_t ord_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---- loads of one element of any supported storage type --------------------
template <int DT>
__device__ __forceinline__ float load_as_f32(const void* p, size_t i) {
  if constexpr (DT == DT_F32) return ((const float*)p)[i];
  else return bf16_bits_to_f32(((const uint16_t*)p)[i]);
}

template <int DT>
__device__ __forceinline__ void store_from_f32(void* p, size_t i, float v) {
  if constexpr (DT == DT_F32) ((float*)p)[i] = v;
  else ((uint16_t*)p)[i] = f32_to_bf16_bits(v);
}

// ---- RoPE angle.  theta_u = base^(-2u/rope_dim) = r^u with r = base^(-2/rope_dim):
// the host supplies r in fp64 and the relative rounding error of r (RopeRatio,
// from an 80-bit power), the device raises r to u by square-and-multiply and
// removes r's own error amplified u-fold, leaving ~2 log2(u) roundings (about
// 1e-15 relative).  The angle p * theta_u is formed and reduced modulo 2*pi in
// fp64 (Cody-Waite with a two-part constant; with FMA k * hi is exact for
// |k| < 2^29), so the angle error stays below 2e-8 rad for positions up to
// 2^24 and below 3e-6 rad up to 2^31; cos and sin of the reduced angle
// (|r| <= pi) are taken in fp32, a few 1e-8 from exact.  All of it is a few
// dozen instructions: a library pow and sincos in fp64 cost ~2k cycles of
// latency and most of a kernel's registers where this sits on a short path.
struct RopeRatio {
  double r;     // base^(-2 / rope_dim), rounded
  double rel;   // (exact - r) / r
};

// (host) the ratio for rope_dim and base, from an 80-bit power
static inline RopeRatio rope_ratio(int rope_dim, float base) {
  if (rope_dim <= 0) return RopeRatio{1.0, 0.0};
  const long double rl = powl((long double)base, -2.0L / (long double)rope_dim);
  const double r = (double)rl;
  return RopeRatio{r, (double)((rl - (long double)r) / (long double)r)};
}

__device__ __forceinline__ void rope_cos_sin(long long pos, int u, RopeRatio rr, float* c, float* s) {
  const double kTwoPiHi = 6.283185307179586;          // nearest double to 2*pi
  const double kTwoPiLo = 2.4492935982947064e-16;      // 2*pi - kTwoPiHi
  const double kInvTwoPi = 0.15915494309189535;
  double t = 1.0, p = rr.r;
  for (int e = u; e > 0; e >>= 1) {
    if (e & 1) t *= p;
    p *= p;
  }
  const double theta = fma(t, (double)u * rr.rel, t);   // r^u (1 + u rel)
  const double ang = (double)pos * theta;
  const double k = rint(ang * kInvTwoPi);
  double r = fma(-k, kTwoPiHi, ang);
  r = fma(-k, kTwoPiLo, r);
  float sn, cs;
  sincosf((float)r, &sn, &cs);
  *c = cs;
  *s = sn;
}

// 1024 ones: the weights of a missing RMSNorm gamma, so that gamma loads need
// no guard (a guarded load compiles to a branch with its own wait)
struct OnesTable {
  float v[1024];
  constexpr OnesTable() : v() {
    for (int i = 0; i < 1024; ++i) v[i] = 1.f;
  }
};
static __device__ const OnesTable k_ones{};

// ---- wave / block reductions ------------------------------------------------
// A butterfly inside each row of 16 lanes through DPP (quad permutes, half-row
// and row mirrors), then across rows with the gfx950 row swaps; every step
// combines a lane's value with its partner's symmetrically, so every lane ends
// with the same bits.  No LDS round trips.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <bool MAX>
__device__ __forceinline__ float wave_reduce_f(float v) {
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  v = op(v, dpp_f<0xB1>(v));    // quad_perm [1,0,3,2]
  v = op(v, dpp_f<0x4E>(v));    // quad_perm [2,3,0,1]
  v = op(v, dpp_f<0x141>(v));   // row_half_mirror
  v = op(v, dpp_f<0x140>(v));   // row_mirror
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = op(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// block-wide sum / max for up to 1024 threads; `red` is __shared__ float[>= blockDim / 64];
// all threads get the result (the waves' results are combined in wave order)
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6, nw = (blockDim.x + 63) >> 6;
  v = wave_reduce_f<MAX>(v);
  __syncthreads();   // an earlier reduction may still be reading red
  if (lane == 0) red[wid] = v;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < 16; ++w) {
    const float x = red[min(w, nw - 1)];   // unguarded reads: all in flight together
    r = (w < nw) ? (MAX ? fmaxf(r, x) : (r + x)) : r;
  }
  return r;
}

}  // namespace csa
