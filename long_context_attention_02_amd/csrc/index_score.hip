// a2 — lightning-indexer score for gfx950.
//
// DeepSeek-V4 method page, section 3.3:
//   I[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . K[s,:])
// with entries the query cannot see (s >= floor((i+1)/m)) set to -inf.
//
// The ReLU sits between each head's dot product and the head sum, so heads
// cannot be folded into the contraction.  The matrix-core kernels therefore
// take (head) as the M dimension of v_mfma_f32_16x16x32_bf16, keys as N and
// the key width d_I as K; the epilogue applies ReLU, weights each head row and
// reduces the 64 head rows of a key column (16 per lane in registers, then
// across the 4 lane groups with two cross-lane adds).
//
// The contraction order over d_I is permuted so that each lane reads one
// contiguous slice of a key row: lane group g owns dims [g*d_I/4,
// (g+1)*d_I/4) and K-step ks takes the ks-th 8-element chunk of it.  Queries
// use the same permutation, so the dot products are unchanged.
//
// fp8 keys (OCP e4m3fn) are widened to bf16 exactly (3 mantissa bits fit in
// 7) and the per-row scale (> 0) multiplies the head sum, which equals
// scaling the key inside the ReLU.  MXFP4 keys (OCP MX: FP4 E2M1 with an
// E8M0 scale per 32 dims) run the QK products in FP4 on both sides, with the
// block-scaled matrix instruction (index_mx4_decode).
#include <algorithm>

#include "compress_wave.h"
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
  f32x2_t v = __builtin_amdgcn_cvt_pk_f32_fp8((int)code, false);
  return v[0];
}

template <int KDT>
__device__ __forceinline__ float load_key(const void* K, size_t i) {
  if constexpr (KDT == DT_F32) return ((const float*)K)[i];
  else if constexpr (KDT == DT_BF16) return bf16_bits_to_f32(((const uint16_t*)K)[i]);
  else return e4m3_to_f32(((const uint8_t*)K)[i]);
}

// 4 fp8 codes (one dword) -> 4 bf16 in two dwords, exactly
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& lo, uint32_t& hi) {
  f32x2_t a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  f32x2_t c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  lo = __builtin_amdgcn_perm(__float_as_uint(a[1]), __float_as_uint(a[0]), 0x07060302u);
  hi = __builtin_amdgcn_perm(__float_as_uint(c[1]), __float_as_uint(c[0]), 0x07060302u);
}

// ---------------------------------------------------------------------------
// generic path: one thread per entry, fp32 arithmetic on the VALU
// ---------------------------------------------------------------------------
static constexpr int VALU_HMAX = 64;

template <int QDT, int KDT>
__global__ __launch_bounds__(256) void index_valu_kernel(
    const void* __restrict__ q, const float* __restrict__ w, const void* __restrict__ K,
    const float* __restrict__ Ks, const int* __restrict__ q_pos, int Tq, int H, int dI,
    long long N_cap, int m, float* __restrict__ out) {
  extern __shared__ float sq[];  // [H * dI] query, then [H] weights
  const int b = blockIdx.z, t = blockIdx.y;
  const size_t qrow = (size_t)b * Tq + t;
  for (int e = threadIdx.x; e < H * dI; e += blockDim.x)
    sq[e] = load_as_f32<QDT>(q, qrow * (size_t)(H * dI) + e);
  for (int e = threadIdx.x; e < H; e += blockDim.x) sq[H * dI + e] = w[qrow * H + e];
  __syncthreads();
  if constexpr (KDT == DT_MX4) {
    // the FP4 QK path: the query too is MXFP4, quantised per head and 32-dim block
    for (int p = threadIdx.x; p < H * (dI / 32); p += blockDim.x) {
      float* x = sq + (p / (dI / 32)) * dI + 32 * (p % (dI / 32));
      float a = 0.f;
      for (int e = 0; e < 32; ++e) a = fmaxf(a, fabsf(x[e]));
      const int se = mx4_shared_exp(a);
      for (int e = 0; e < 32; ++e) x[e] = ldexpf(e2m1_to_f32(f32_to_e2m1(ldexpf(x[e], -se))), se);
    }
    __syncthreads();
  }
  const long long s = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (s >= N_cap) return;
  const long long i = q_pos[qrow];
  const long long nvis = min(N_cap, (i + 1) / m);
  float res = -INFINITY;
  if (s < nvis) {
    float dot[VALU_HMAX];
#pragma unroll
    for (int h = 0; h < VALU_HMAX; ++h) dot[h] = 0.f;
    const size_t kb = ((size_t)b * (size_t)N_cap + (size_t)s) * (size_t)dI;
    for (int d = 0; d < dI; ++d) {
      float kv;
      if constexpr (KDT == DT_MX4) {
        const uint32_t byte = ((const uint8_t*)K)[(kb + d) >> 1];
        const uint32_t sc = ((const uint8_t*)Ks)[((size_t)b * (size_t)N_cap + (size_t)s) * (size_t)(dI / 32) + d / 32];
        kv = ldexpf(e2m1_to_f32((byte >> (4 * (d & 1))) & 15u), (int)sc - 127);
      } else {
        kv = load_key<KDT>(K, kb + d);
      }
#pragma unroll
      for (int h = 0; h < VALU_HMAX; ++h)
        if (h < H) dot[h] += sq[h * dI + d] * kv;
    }
    float acc = 0.f;
#pragma unroll
    for (int h = 0; h < VALU_HMAX; ++h)
      if (h < H) acc += sq[H * dI + h] * fmaxf(dot[h], 0.f);
    if constexpr (KDT == DT_FP8) acc *= Ks[(size_t)b * (size_t)N_cap + (size_t)s];
    res = acc;
  }
  out[qrow * (size_t)N_cap + (size_t)s] = res;
}

// ---------------------------------------------------------------------------
// matrix-core path, shared pieces
// ---------------------------------------------------------------------------
template <int QH, int KS>
struct IdxFrags {
  bf16x8_t A[QH][KS];   // query rows (heads) for the MFMA A operand
  float wv[QH][4];      // head weights of the 4 rows a lane holds in each M tile
};

// lane (g, j): A[mt][ks] = q[16 mt + j][g*GW + 8 ks .. + 8]
template <int QH, int KS>
__device__ __forceinline__ void load_query_frags(IdxFrags<QH, KS>& f, const uint16_t* __restrict__ qp,
                                                 const float* __restrict__ wp, int g, int j) {
  constexpr int DI = 32 * KS, GW = DI / 4;
#pragma unroll
  for (int mt = 0; mt < QH; ++mt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      f.A[mt][ks] = *(const bf16x8_t*)(qp + (size_t)(16 * mt + j) * DI + GW * g + 8 * ks);
#pragma unroll
    for (int r = 0; r < 4; ++r) f.wv[mt][r] = wp[16 * mt + 4 * g + r];
  }
}

// this lane's share (its 4 QH head rows) of sum_h w * ReLU(dot) for its key
// column; reduce_scatter4 completes four of them
template <int QH, int KS>
__device__ __forceinline__ float partial_column(const IdxFrags<QH, KS>& f, const bf16x8_t (&Bf)[KS]) {
  f32x4_t acc[QH];
#pragma unroll
  for (int mt = 0; mt < QH; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
#pragma unroll
    for (int mt = 0; mt < QH; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.A[mt][ks], Bf[ks], acc[mt], 0, 0, 0);
  float part = 0.f;
#pragma unroll
  for (int mt = 0; mt < QH; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) part += f.wv[mt][r] * __int_as_float(max(__float_as_int(acc[mt][r]), 0));   // ReLU
  return part;
}

// B fragments of one key row slice straight from global memory
template <int KS, int KDT>
__device__ __forceinline__ void load_key_frags(bf16x8_t (&Bf)[KS], const void* __restrict__ K,
                                               size_t row, int g, bool valid) {
  constexpr int DI = 32 * KS, GW = DI / 4;
  if constexpr (KDT == DT_BF16) {
    const uint16_t* kp = (const uint16_t*)K + row * DI + GW * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      Bf[ks] = valid ? *(const bf16x8_t*)(kp + 8 * ks) : bf16x8_t{};
  } else {
    const uint8_t* kp = (const uint8_t*)K + row * DI + GW * g;   // GW = 8 KS bytes
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x2_t w2 = valid ? *(const u32x2_t*)(kp + 8 * ks) : u32x2_t{0u, 0u};
      u32x4_t o;
      uint32_t lo, hi;
      fp8x4_to_bf16x4(w2[0], lo, hi);
      o[0] = lo; o[1] = hi;
      fp8x4_to_bf16x4(w2[1], lo, hi);
      o[2] = lo; o[3] = hi;
      Bf[ks] = __builtin_bit_cast(bf16x8_t, o);
    }
  }
}

// ---------------------------------------------------------------------------
// decode: few query rows, keys streamed from HBM through registers.
// The waves of one query row share its keys and walk them in subtiles of 16
// keys, with a register ring of PF subtiles in flight.  A subtile is loaded
// contiguously (each load instruction covers whole 128-byte lines: a layout
// with 16 rows per instruction, each read in part, streams markedly slower)
// and turned into the MFMA operand layout through a small wave-private LDS
// tile.  Four subtiles form a group: every lane first sums its 16 head rows
// per subtile, then a reduce-scatter across the 4 lane groups (3 cross-lane
// adds) leaves lane (g, j) with the full score of key j of subtile g.
// ---------------------------------------------------------------------------
template <int KS, int KDT>
struct RawSub {                       // one lane's bytes of one subtile
  static constexpr int WORDS = (KDT == DT_FP8 ? 8 * KS : 16 * KS) / 4;
  uint32_t w[WORDS];
};

template <int KS, int KDT>
struct SubGeom {
  static constexpr int RB = KDT == DT_FP8 ? 32 * KS : 64 * KS;   // bytes per key row
  static constexpr int SB = 16 * RB;                             // bytes per subtile
  static constexpr int LB = SB / 64;                             // bytes per lane
  static constexpr int NP = RB / 16;                             // 16-byte pieces per row
  static constexpr int RPB = RB >= 256 ? 1 : 256 / RB;           // rows per 256 LDS bytes
  // LDS slot of piece P of row R: pieces are XOR-swizzled within their row so
  // that the 16 rows one lane group reads land on distinct banks
  static __device__ __forceinline__ int slot(int R, int P) { return RB * R + 16 * (P ^ ((R / RPB) % NP)); }
};

// Contiguous load of subtile rows row0 .. row0 + 15 (rows past klast read row
// klast instead: their scores are never stored, and a slot only feeds its own
// key column).  Lane l holds bytes [64 c + 16 l, +16) of instruction c of the
// subtile (8 bytes at 8 l when a lane's share is 8 bytes).  Unconditional, so
// no select waits on the load; streamed once, so non-temporal.
template <int KS, int KDT>
__device__ __forceinline__ void load_lin(RawSub<KS, KDT>& r, const uint8_t* __restrict__ Kb, int row0,
                                         int klast, int lane) {
  // Kb: the sequence's first key row; rows are < 2^31 (the entry point checks N_cap)
  using G = SubGeom<KS, KDT>;
  if constexpr (G::LB >= 16) {
#pragma unroll
    for (int c = 0; c < G::LB / 16; ++c) {
      const int L = 64 * c + lane;
      const uint32_t row = min((uint32_t)row0 + (uint32_t)(L / G::NP), (uint32_t)klast);
      const u32x4_t v = __builtin_nontemporal_load(
          (const u32x4_t*)(Kb + (size_t)row * G::RB + 16 * (L % G::NP)));
#pragma unroll
      for (int e = 0; e < 4; ++e) r.w[4 * c + e] = v[e];
    }
  } else {
    static_assert(G::LB == 8, "8-byte lane share");
    const uint32_t row = min((uint32_t)row0 + (uint32_t)((8 * lane) / G::RB), (uint32_t)klast);
    const u32x2_t v = __builtin_nontemporal_load((const u32x2_t*)(Kb + (size_t)row * G::RB + (8 * lane) % G::RB));
    r.w[0] = v[0];
    r.w[1] = v[1];
  }
}

// Linear subtile bytes -> the decode operand layout through the wave's LDS tile:
// lane (g, j) gets row j, 16-byte pieces g + 4 c (bytes 64 c + 16 g), or the
// 8 bytes at 8 g when its share is 8 bytes.  The wave's own LDS operations run
// in order, so the read sees the write without a barrier.
template <int KS, int KDT>
__device__ __forceinline__ void lds_transpose(RawSub<KS, KDT>& out, const RawSub<KS, KDT>& in,
                                              uint8_t* tile, int lane, int g, int j) {
  using G = SubGeom<KS, KDT>;
  if constexpr (G::LB >= 16) {
#pragma unroll
    for (int c = 0; c < G::LB / 16; ++c) {
      const int L = 64 * c + lane;
      const u32x4_t v = {in.w[4 * c], in.w[4 * c + 1], in.w[4 * c + 2], in.w[4 * c + 3]};
      *(u32x4_t*)(tile + G::slot(L / G::NP, L % G::NP)) = v;
    }
#pragma unroll
    for (int c = 0; c < G::LB / 16; ++c) {
      const u32x4_t v = *(const u32x4_t*)(tile + G::slot(j, g + 4 * c));
#pragma unroll
      for (int e = 0; e < 4; ++e) out.w[4 * c + e] = v[e];
    }
  } else {
    const int byte = 8 * lane;
    *(u32x2_t*)(tile + G::slot(byte / G::RB, (byte % G::RB) / 16) + (byte & 8)) = u32x2_t{in.w[0], in.w[1]};
    const u32x2_t v = *(const u32x2_t*)(tile + G::slot(j, g / 2) + 8 * (g & 1));
    out.w[0] = v[0];
    out.w[1] = v[1];
  }
}

// first of the 8 dims lane group g holds in K-step ks of a decode subtile
template <int KS, int KDT>
__device__ __forceinline__ int dec_dim(int ks, int g) {
  if constexpr (KDT == DT_FP8) {
    if constexpr (KS == 1) return 8 * g;                 // one 8-byte piece at 8 g
    else return 64 * (ks / 2) + 16 * g + 8 * (ks % 2);   // two K-steps per 16-byte piece
  } else {
    return 32 * ks + 8 * g;                              // one K-step per 16-byte piece
  }
}

template <int QH, int KS, int KDT>
__device__ __forceinline__ void load_query_frags_dec(IdxFrags<QH, KS>& f, const uint16_t* __restrict__ qp,
                                                     const float* __restrict__ wp, int g, int j) {
  constexpr int DI = 32 * KS;
#pragma unroll
  for (int mt = 0; mt < QH; ++mt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      f.A[mt][ks] = *(const bf16x8_t*)(qp + (size_t)(16 * mt + j) * DI + dec_dim<KS, KDT>(ks, g));
#pragma unroll
    for (int r = 0; r < 4; ++r) f.wv[mt][r] = wp[16 * mt + 4 * g + r];
  }
}

// partial_column straight from the raw key bytes, converting one K-step at a
// time (fewer registers live than converting the whole subtile first)
template <int QH, int KS, int KDT>
__device__ __forceinline__ float partial_column_raw(const IdxFrags<QH, KS>& f, const RawSub<KS, KDT>& r) {
  f32x4_t acc[QH];
#pragma unroll
  for (int mt = 0; mt < QH; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    bf16x8_t b;
    if constexpr (KDT == DT_FP8) {
      const bf16x2_t x0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w[2 * ks], 1.0f, false);
      const bf16x2_t x1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w[2 * ks], 1.0f, true);
      const bf16x2_t x2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w[2 * ks + 1], 1.0f, false);
      const bf16x2_t x3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w[2 * ks + 1], 1.0f, true);
      const u32x4_t o = {__builtin_bit_cast(uint32_t, x0), __builtin_bit_cast(uint32_t, x1),
                         __builtin_bit_cast(uint32_t, x2), __builtin_bit_cast(uint32_t, x3)};
      b = __builtin_bit_cast(bf16x8_t, o);
    } else {
      const u32x4_t o = {r.w[4 * ks], r.w[4 * ks + 1], r.w[4 * ks + 2], r.w[4 * ks + 3]};
      b = __builtin_bit_cast(bf16x8_t, o);
    }
#pragma unroll
    for (int mt = 0; mt < QH; ++mt)
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.A[mt][ks], b, acc[mt], 0, 0, 0);
  }
  // ReLU as a signed-integer max on the bits: negative floats (and -0.0) are
  // negative integers, so one v_max_i32 clears them
  float part = 0.f;
#pragma unroll
  for (int mt = 0; mt < QH; ++mt)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4)
      part += f.wv[mt][r4] * __int_as_float(max(__float_as_int(acc[mt][r4]), 0));
  return part;
}

// P[u] = lane group g's share for subtile u; returns the full sum for subtile g
__device__ __forceinline__ float reduce_scatter4(const float (&P)[4], int g) {
  const bool hi = (g >> 1) & 1, lo = g & 1;
  const float s0 = hi ? P[0] : P[2], s1 = hi ? P[1] : P[3];
  const float k0 = (hi ? P[2] : P[0]) + __shfl_xor(s0, 32, 64);   // subtile 2*hi
  const float k1 = (hi ? P[3] : P[1]) + __shfl_xor(s1, 32, 64);   // subtile 2*hi + 1
  const float s = lo ? k0 : k1;
  return (lo ? k1 : k0) + __shfl_xor(s, 16, 64);                  // subtile 2*hi + lo = g
}

static constexpr int IDX_STAGE = 2048;   // keys per wave whose scores are staged in LDS
static constexpr int IDX_UNIT = 4;       // subtiles of 16 keys per interleaving unit
static constexpr int IDX_FLUSH = 32;     // staged subtiles written out together (0: all at the end)
static_assert(IDX_FLUSH % 16 == 0 && IDX_FLUSH * 16 <= IDX_STAGE, "flush windows of whole store rounds");
// a wave gets at most ceil(units / W) units, W >= units * 16 * IDX_UNIT / IDX_STAGE (launcher)
static_assert(IDX_STAGE % (16 * IDX_UNIT) == 0, "stage holds whole units");

// Decode (few query rows): the waves of one query row interleave over its keys
// in units of IDX_UNIT subtiles (wave w takes units w, w + W, w + 2W, ...), so
// at any moment the device reads a few narrow moving windows of the key array
// rather than one far-apart stream per wave.
//
// One wave's share of query row (b, t): units wid, wid + W, ... below nunits,
// over key rows 0 .. n_keys - 1 (rows of N_cap, the row stride of K and of
// the scores; n_keys <= N_cap).
template <int QH, int KS, int KDT>
__device__ __forceinline__ void index_decode_wave(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const void* __restrict__ K,
    const float* __restrict__ Ks, const int* __restrict__ q_pos, int Tq, long long N_cap, long long n_keys,
    int m, float* __restrict__ out, int flush_ok, int b, int t, long long wid, long long W,
    long long nunits) {
  constexpr int H = 16 * QH, DI = 32 * KS;
  // subtiles in flight per wave (a ring of 8 measured no faster: the loop is
  // not short of loads in flight)
  constexpr int PF = 4;
  static_assert(PF % 4 == 0, "whole groups of four slots");
  constexpr int U = IDX_UNIT;
  // the wave index through readfirstlane: the compiler then knows everything
  // derived from it is wave-uniform (scalar registers, uniform branches)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;
  const size_t qrow = (size_t)b * Tq + t;
  if (wid >= nunits) return;
  const int nls = (int)((nunits - 1 - wid) / W + 1) * U;   // subtiles of this wave
  // (at least one: stated so that the ring's first loads are not sunk into a
  // loop guard, behind the wait for the query loads)
  __builtin_assume(nls >= 1);
  const long long i = q_pos[qrow];
  const long long nvis = min(N_cap, (i + 1) / m);
  // first key of the wave's local subtile ls (32-bit: keys are < 2^31, and a
  // subtile index up to PF past the wave's last one stays far below that)
  const int wid32 = (int)wid, W32 = (int)W;
  auto key0 = [&](int ls) -> int { return 16 * ((wid32 + W32 * (ls / U)) * U + ls % U); };

  IdxFrags<QH, KS> f;
  load_query_frags_dec<QH, KS, KDT>(f, q + qrow * (size_t)(H * DI), w + qrow * H, g, j);
  const size_t kbase = (size_t)b * (size_t)N_cap;
  float* orow = out + qrow * (size_t)N_cap;
  const int klast = (int)(n_keys - 1);   // absent keys load this row (their scores are never stored)
  const uint8_t* Kb = (const uint8_t*)K + kbase * SubGeom<KS, KDT>::RB;

  // Scores are staged in LDS (slot 16 ls + j for key j of local subtile ls)
  // and written once the wave's keys are all read: stores share the memory
  // counter with the loads, and waiting for a key would also wait for every
  // store issued before it.  For fp8 keys the slots first receive the keys'
  // row scales, straight from memory (4-byte LDS DMA, one key per lane).
  __shared__ __attribute__((aligned(16))) float stage[4][IDX_STAGE];
  if constexpr (KDT == DT_FP8) {
    // a fixed count of DMAs (slots past the wave's keys read row klast), so the
    // compiler can count the loads in flight after them
    const float* sb = Ks + kbase;
#pragma unroll
    for (int c = 0; c < IDX_STAGE / 64; ++c) {
      const int e = 64 * c + lane;
      const int key = (e >> 4) < nls ? min(key0(e >> 4) + (e & 15), klast) : klast;
      __builtin_amdgcn_global_load_lds((const void*)(sb + key),
                                       (__attribute__((address_space(3))) void*)&stage[wave][64 * c], 4, 0, 0);
    }
  }

  // The key ring holds PF subtiles in flight; a slot is consumed (moved
  // through the LDS tile), then refilled with the subtile PF later.
  RawSub<KS, KDT> ring[PF];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load_lin<KS, KDT>(ring[p], Kb, p < nls ? key0(p) : klast, klast, lane);
    __builtin_amdgcn_sched_barrier(0);   // issue in slot order, as the loop refills them
  }
  // Retire the query loads here, with the ring already in flight: an (empty,
  // register-only) rewrite of every fragment makes the compiler wait for them
  // at this point, so the loop's wait counts are fixed by the ring alone
  // (otherwise every iteration would wait for all keys in flight, as the first
  // one must for these loads).  Not volatile: a volatile asm counts as a
  // memory access and would also wait for the scale DMA and the whole ring.
#pragma unroll
  for (int mt = 0; mt < QH; ++mt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm("" : "+v"(f.A[mt][ks]));
#pragma unroll
    for (int r = 0; r < 4; ++r) asm("" : "+v"(f.wv[mt][r]));
  }
  __shared__ __attribute__((aligned(16))) uint8_t tile[4][SubGeom<KS, KDT>::SB];
  int flushed = 0;   // subtiles already written out
  // two groups of four slots per pass, so every slot index is a constant
#pragma unroll 1
  for (int st0 = 0; st0 < nls; st0 += PF) {
#pragma unroll
    for (int half = 0; half < PF / 4; ++half) {
      // first subtile of this group of four.  A group past the wave's last
      // subtile still runs (its slots hold row klast, and nothing of it is
      // staged or stored): an early exit here would make the compiler merge
      // two orders of the ring's loads at the loop head and wait for most of
      // the ring at every slot.
      const int gs = st0 + 4 * half;
      float P[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int slot = 4 * half + u;
        RawSub<KS, KDT> T;
        lds_transpose<KS, KDT>(T, ring[slot], tile[wave], lane, g, j);
        const int nx = gs + u + PF;
        load_lin<KS, KDT>(ring[slot], Kb, nx < nls ? key0(nx) : klast, klast, lane);
        P[u] = partial_column_raw<QH, KS, KDT>(f, T);
        // the sum is materialised here, so the epilogue is not sunk below the
        // later subtiles (which would keep 64 accumulators live instead of 16)
        asm volatile("" : "+v"(P[u]));
        // keep the next slot's conversions out of this one (they would wait on its load)
        __builtin_amdgcn_sched_barrier(0);
      }
      // (the scale fetch is older than every key load waited for above, and the
      // memory counter retires loads in order, so the scales are in LDS by now)
      const float v = reduce_scatter4(P, g);
      const int ls = gs + g;
      if (ls < nls) {
        const int e = 16 * ls + j;
        float r = v;
        if constexpr (KDT == DT_FP8) r *= stage[wave][e];
        stage[wave][e] = key0(ls) + j < nvis ? r : -INFINITY;
      }
      // Every IDX_FLUSH subtiles, write the window out: spreading the stores
      // over the loop keeps them off the wave's tail.  flush_ok (set by the
      // launcher) says every output row is 16-byte aligned and every unit lies
      // inside the sequence, so a window of the wave's subtiles holds only keys
      // that exist.  (A test in terms other than nls and such a flag here makes
      // the compiler lose its count of the loads in flight and wait for all.)
      if constexpr (IDX_FLUSH > 0) {
        if ((gs + 4) % IDX_FLUSH == 0 && gs + 4 <= nls && flush_ok) {
          const int e0 = 16 * (gs + 4 - IDX_FLUSH) + 4 * lane;
#pragma unroll
          for (int c = 0; c < IDX_FLUSH / 16; ++c) {
            const int e = e0 + 256 * c;
            __builtin_nontemporal_store(*(const f32x4_t*)&stage[wave][e],
                                        (f32x4_t*)(orow + key0(e >> 4) + (e & 15)));
          }
          flushed = gs + 4;
        }
      }
    }
  }
  // write pass for the rest: four keys per lane, 16 lanes per subtile, LDS to memory only
  for (int e = 16 * flushed + 4 * lane; e < 16 * nls; e += 256) {
    const int key = key0(e >> 4) + (e & 15);
    if (key > klast) continue;
    const f32x4_t v = *(const f32x4_t*)&stage[wave][e];
    if (key + 3 <= klast && (((uintptr_t)(orow + key)) & 15u) == 0) {
      __builtin_nontemporal_store(v, (f32x4_t*)(orow + key));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (key + c <= klast) orow[key + c] = v[c];
    }
  }
}

template <int QH, int KS, int KDT>
__global__ __launch_bounds__(256) void index_mfma_decode(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const void* __restrict__ K,
    const float* __restrict__ Ks, const int* __restrict__ q_pos, int Tq, long long N_cap, int m,
    float* __restrict__ out, int flush_ok) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  index_decode_wave<QH, KS, KDT>(q, w, K, Ks, q_pos, Tq, N_cap, N_cap, m, out, flush_ok, blockIdx.z, blockIdx.y,
                                 4LL * blockIdx.x + wave, 4LL * gridDim.x,
                                 (N_cap + 16 * IDX_UNIT - 1) / (16 * IDX_UNIT));
}

// ---------------------------------------------------------------------------
// The front of a decode step in one launch: the step's compressions (the new
// token's window row, the newest KV entry, the newest indexer key) run as one
// extra workgroup per sequence beside the indexer, instead of as a launch of
// their own in front of it.  The indexer workgroups score every unit of 64
// keys but the last; the wave that writes the new key then scores that last
// unit with the same code, so every score equals the one the indexer alone
// computes from the same key rows.  Each job of the extra workgroup runs on
// one wave, with the wave-per-entry compressor's arithmetic.  One query row
// per sequence.
// ---------------------------------------------------------------------------
// The scores of one unit (four subtiles of 16 keys from key0, a multiple of
// 64) of decode row b (one query row per sequence), by one wave, with the
// per-key arithmetic of index_decode_wave (the same subtile products,
// reduce-scatter over the unit's four subtiles, scale and mask): used on the
// unit whose key rows the same launch writes.  The operands are loaded
// straight into their lane layout, without the LDS tile: a second LDS object
// in the launch hides from the compiler that the indexer's tile and its
// score-stage DMA do not overlap, and its loop then waits for every load in
// flight.
template <int QH, int KS, int KDT>
__device__ __forceinline__ void index_score_unit(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                                 const void* __restrict__ K, const float* __restrict__ Ks,
                                                 const int* __restrict__ q_pos, long long N_cap, int m,
                                                 float* __restrict__ out, int b, long long key0) {
  constexpr int H = 16 * QH, DI = 32 * KS;
  const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15;
  IdxFrags<QH, KS> f;
  load_query_frags_dec<QH, KS, KDT>(f, q + (size_t)b * (H * DI), w + (size_t)b * H, g, j);
  const uint8_t* Kb = (const uint8_t*)K + (size_t)b * (size_t)N_cap * SubGeom<KS, KDT>::RB;
  using G = SubGeom<KS, KDT>;
  float P[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    // lane (g, j) loads what lds_transpose hands it: row j, 16-byte pieces
    // g + 4 c (or the 8 bytes at 8 g when its share is 8 bytes)
    RawSub<KS, KDT> T;
    const uint8_t* row = Kb + (size_t)(key0 + 16 * u + j) * G::RB;
    if constexpr (G::LB >= 16) {
#pragma unroll
      for (int c = 0; c < G::LB / 16; ++c) {
        const u32x4_t v = *(const u32x4_t*)(row + 16 * (g + 4 * c));
#pragma unroll
        for (int e = 0; e < 4; ++e) T.w[4 * c + e] = v[e];
      }
    } else {
      const u32x2_t v = *(const u32x2_t*)(row + 8 * g);
      T.w[0] = v[0];
      T.w[1] = v[1];
    }
    P[u] = partial_column_raw<QH, KS, KDT>(f, T);
  }
  float v = reduce_scatter4(P, g);   // key key0 + 16 g + j
  const long long key = key0 + 16 * g + j;
  if constexpr (KDT == DT_FP8) v *= Ks[(size_t)b * (size_t)N_cap + (size_t)key];
  const long long nvis = min(N_cap, ((long long)q_pos[b] + 1) / m);
  out[(size_t)b * (size_t)N_cap + (size_t)key] = key < nvis ? v : -INFINITY;
}

static constexpr int FRONT_MAX_JOBS = 4;   // one wave each
struct FrontJobs {
  CompressJob job[FRONT_MAX_JOBS];
  int n_jobs, key_job;   // key_job: the job that writes the indexer's key rows
};

template <int QH, int KS, int KDT>
__global__ __launch_bounds__(256) void index_decode_front(
    const FrontJobs fj, const uint16_t* __restrict__ q, const float* __restrict__ w,
    const void* __restrict__ K, const float* __restrict__ Ks, const int* __restrict__ q_pos,
    long long N_cap, int m, float* __restrict__ out, int flush_ok, int gx, int B) {
  // the jobs are read where they lie, in the kernel-argument segment (fj is
  // the first argument, at offset 0): indexing the by-value record with the
  // wave index would make the compiler copy all of it to scratch memory
  (void)fj;
  const FrontJobs& F = *(const FrontJobs*)__builtin_amdgcn_kernarg_segment_ptr();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long nunits = N_cap / (16 * IDX_UNIT);   // (host: N_cap % 64 == 0)
  // a 1-D grid: gx indexer workgroups per sequence, then one front workgroup
  // per sequence at the end, so the indexer's workgroups spread over the
  // compute units as they do alone (two per unit at the 1M decode) and the
  // light front workgroups take the slots left over.  Measured slower: the
  // front workgroups first (1M decode 106 against 102 us); leaving their slots
  // out of the indexer's round when bf16 keys allow two waves per SIMD
  // (Flash-like decode 17.6 against 16.8 us: half the indexer's waves); and
  // the key wave scoring the unit's older subtiles before its compression
  // (Flash-like 19.1 against 16.8 us: at that shape the front workgroup runs
  // after an indexer workgroup ends, and the extra round trip is in its path)
  const int nidx = gx * B;
  if ((int)blockIdx.x < nidx) {
    // the indexer over every unit but the last; its rows past the scored ones
    // are never read, so no load meets the key row being written
    const int b = (int)blockIdx.x / gx, x = (int)blockIdx.x - b * gx;
    index_decode_wave<QH, KS, KDT>(q, w, K, Ks, q_pos, 1, N_cap, N_cap - 16 * IDX_UNIT, m, out, flush_ok, b, 0,
                                   4LL * x + wave, 4LL * gx, nunits - 1);
    return;
  }
  const int b = (int)blockIdx.x - nidx;
  if (wave < F.n_jobs) {
    const CompressJob& J = F.job[wave];
    for (long long e = 0; e < J.n_entries; ++e) {
      const long long s = J.s_begin + e;
      if (J.out_dtype == DT_FP8) compress_entry_wave<DT_BF16, DT_FP8, COMPW_MAXC>(J, s, b, lane);
      else if (J.out_dtype == DT_MIX) compress_entry_wave<DT_BF16, DT_MIX, COMPW_MAXC>(J, s, b, lane);
      else compress_entry_wave<DT_BF16, DT_BF16, COMPW_MAXC>(J, s, b, lane);
    }
  }
  if (wave != F.key_job) return;
  // the key rows and scales written above are complete before the unit's loads
  // (the wave's own stores, read back through the same compute unit)
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // (the key rows through the key job's own pointers, equal to K and Ks: a load
  // through K after the stores above makes the compiler wait for every load in
  // flight at the head of the indexer's loop)
  index_score_unit<QH, KS, KDT>(q, w, F.job[F.key_job].E, F.job[F.key_job].E_scale, q_pos, N_cap, m, out, b,
                                16 * IDX_UNIT * (nunits - 1));
}

// ---------------------------------------------------------------------------
// decode with MXFP4 keys: the FP4 query-key path (DeepSeek-V4 method page,
// section 3.6).  Keys are E2M1 codes, 64 bytes per 128-dim row, with four E8M0
// block scales per row in a separate array; the query is quantised to MXFP4
// by the same rule in the prologue.  One v_mfma_scale_f32_16x16x128_f8f6f4
// per 16-head tile covers all 128 dims of 16 keys: lane (g, j) holds dims
// 32 g .. 32 g + 31 (low nibble first) of head row j (A) and of key j (B) and
// the scale byte of that block, so a 16-key subtile is one contiguous kilobyte
// that every lane loads straight into its operand (16 bytes; four lanes per
// 64-byte row), with no LDS transpose.  The work split over waves, the score
// staging in LDS and the flushes are those of index_mfma_decode.
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8_t;

template <int QH>
__device__ __forceinline__ float mx4_partial(const u32x4_t (&qa)[QH], const int (&qsc)[QH],
                                             const float (&wv)[QH][4], const u32x4_t kc, int ksc) {
  const i32x8_t Bv = {(int)kc[0], (int)kc[1], (int)kc[2], (int)kc[3], 0, 0, 0, 0};
  float part = 0.f;
#pragma unroll
  for (int mt = 0; mt < QH; ++mt) {
    const i32x8_t Av = {(int)qa[mt][0], (int)qa[mt][1], (int)qa[mt][2], (int)qa[mt][3], 0, 0, 0, 0};
    // cbsz = blgp = 4: both operands FP4 E2M1; op_sel 0: the scale is byte 0
    const f32x4_t acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
        Av, Bv, f32x4_t{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, qsc[mt], 0, ksc);
#pragma unroll
    for (int r = 0; r < 4; ++r) part += wv[mt][r] * __int_as_float(max(__float_as_int(acc[r]), 0));
  }
  return part;
}

// One wave's share of query row (b, t) (as index_decode_wave): units wid,
// wid + W, ... below nunits, over key rows 0 .. n_keys - 1 of N_cap.
template <int QH>
__device__ __forceinline__ void index_mx4_wave(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ K,
    const uint8_t* __restrict__ Ks, const int* __restrict__ q_pos, int Tq, long long N_cap, long long n_keys, int m,
    float* __restrict__ out, int flush_ok, int b, int t, long long wid, long long W, long long nunits) {
  constexpr int H = 16 * QH, DI = 128, RB = DI / 2, SB = DI / 32;   // code and scale bytes per key
  constexpr int PF = 8;   // subtiles in flight per wave (two groups of four)
  constexpr int U = IDX_UNIT;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;
  const size_t qrow = (size_t)b * Tq + t;
  if (wid >= nunits) return;
  const int nls = (int)((nunits - 1 - wid) / W + 1) * U;   // subtiles of this wave (a multiple of 4)
  __builtin_assume(nls >= 1);
  const long long i = q_pos[qrow];
  const long long nvis = min(N_cap, (i + 1) / m);
  const int wid32 = (int)wid, W32 = (int)W;
  auto key0 = [&](int ls) -> int { return 16 * ((wid32 + W32 * (ls / U)) * U + ls % U); };
  const int klast = (int)(n_keys - 1);
  const uint8_t* Kb = K + (size_t)b * (size_t)N_cap * RB;
  const uint8_t* Sb = Ks + (size_t)b * (size_t)N_cap * SB;
  float* orow = out + qrow * (size_t)N_cap;

  // the query rows and head weights first (head 16 mt + j, dims 32 g ..
  // 32 g + 31), then the key ring: subtile p's codes (lane (g, j): bytes 16 g
  // of key j) and the key's scale dword (byte g is this lane's block).  The
  // memory counter retires loads in order, so waiting for the query leaves
  // the ring in flight.
  u32x4_t raw[QH][4];
  float wv[QH][4];
#pragma unroll
  for (int mt = 0; mt < QH; ++mt) {
    const uint16_t* qp = q + (qrow * H + 16 * mt + j) * (size_t)DI + 32 * g;
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[mt][c] = *(const u32x4_t*)(qp + 8 * c);
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = w[qrow * H + 16 * mt + 4 * g + r];
  }
  u32x4_t rc[PF];
  uint32_t rs[PF];
  auto load_sub = [&](int first, u32x4_t& c, uint32_t& sc) {
    const uint32_t row = min((uint32_t)first + (uint32_t)j, (uint32_t)klast);
    c = __builtin_nontemporal_load((const u32x4_t*)(Kb + (size_t)row * RB + 16 * g));
    sc = __builtin_nontemporal_load((const uint32_t*)(Sb + (size_t)row * SB));
  };
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    load_sub(p < nls ? key0(p) : klast, rc[p], rs[p]);
    __builtin_amdgcn_sched_barrier(0);
  }

  // the query quantised to MXFP4
  u32x4_t qa[QH];
  int qsc[QH];
#pragma unroll
  for (int mt = 0; mt < QH; ++mt) {
    float x[32];
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * c + 2 * e] = __uint_as_float(raw[mt][c][e] << 16);
        x[8 * c + 2 * e + 1] = __uint_as_float(raw[mt][c][e] & 0xffff0000u);
        a = fmaxf(a, fmaxf(fabsf(x[8 * c + 2 * e]), fabsf(x[8 * c + 2 * e + 1])));
      }
    const int se = mx4_shared_exp(a);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t pk = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) pk |= f32_to_e2m1(ldexpf(x[8 * d + e], -se)) << (4 * e);
      qa[mt][d] = pk;
    }
    qsc[mt] = se + 127;
  }
  // Retire the weight loads here (an empty register-only rewrite): their first
  // use inside the loop would otherwise carry a wait for them, and that wait,
  // counted in every pass, would drain the ring each time.
#pragma unroll
  for (int mt = 0; mt < QH; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) asm("" : "+v"(wv[mt][r]));

  __shared__ __attribute__((aligned(16))) float stage[4][IDX_STAGE];
  int flushed = 0;
#pragma unroll 1
  for (int st0 = 0; st0 < nls; st0 += 8) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // first subtile of this group of four.  A group past the wave's last
      // subtile still runs (its slots hold row klast, and nothing of it is
      // staged or stored): an early exit here would make the compiler merge
      // two orders of the ring's loads at the loop head and wait for most of
      // the ring at every slot.
      const int gs = st0 + 4 * half;
      float P[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int slot = 4 * half + u;
        const int sc = (int)((rs[slot] >> (8 * g)) & 0xffu);
        const int nx = gs + u + PF;
        P[u] = mx4_partial<QH>(qa, qsc, wv, rc[slot], sc);
        // the refill after the products that read the slot: loading first
        // made the compiler load into a temporary and copy it into the slot
        // at the loop's end, a copy that waits for nearly the whole ring
        load_sub(nx < nls ? key0(nx) : klast, rc[slot], rs[slot]);
        asm volatile("" : "+v"(P[u]));
        __builtin_amdgcn_sched_barrier(0);
      }
      const float v = reduce_scatter4(P, g);
      const int ls = gs + g;
      if (ls < nls) stage[wave][16 * ls + j] = key0(ls) + j < nvis ? v : -INFINITY;
      if constexpr (IDX_FLUSH > 0) {
        if ((gs + 4) % IDX_FLUSH == 0 && gs + 4 <= nls && flush_ok) {
          const int e0 = 16 * (gs + 4 - IDX_FLUSH) + 4 * lane;
#pragma unroll
          for (int c = 0; c < IDX_FLUSH / 16; ++c) {
            const int e = e0 + 256 * c;
            __builtin_nontemporal_store(*(const f32x4_t*)&stage[wave][e],
                                        (f32x4_t*)(orow + key0(e >> 4) + (e & 15)));
          }
          flushed = gs + 4;
        }
      }
    }
  }
  for (int e = 16 * flushed + 4 * lane; e < 16 * nls; e += 256) {
    const int key = key0(e >> 4) + (e & 15);
    if (key > klast) continue;
    const f32x4_t v = *(const f32x4_t*)&stage[wave][e];
    if (key + 3 <= klast && (((uintptr_t)(orow + key)) & 15u) == 0) {
      __builtin_nontemporal_store(v, (f32x4_t*)(orow + key));
    } else {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (key + c <= klast) orow[key + c] = v[c];
    }
  }
}

template <int QH>
__global__ __launch_bounds__(256) void index_mx4_decode(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const uint8_t* __restrict__ K,
    const uint8_t* __restrict__ Ks, const int* __restrict__ q_pos, int Tq, long long N_cap, int m,
    float* __restrict__ out, int flush_ok) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  index_mx4_wave<QH>(q, w, K, Ks, q_pos, Tq, N_cap, N_cap, m, out, flush_ok, blockIdx.z, blockIdx.y,
                     4LL * blockIdx.x + wave, 4LL * gridDim.x, (N_cap + 16 * IDX_UNIT - 1) / (16 * IDX_UNIT));
}

// The decode front with MXFP4 keys (as index_decode_front): the last unit's
// scores by the key wave, with index_mx4_wave's arithmetic -- the query
// quantised by the same rule, one block-scaled product per 16-head tile,
// the reduce-scatter over the unit's four subtiles, the mask.
template <int QH>
__device__ __forceinline__ void mx4_score_unit(const uint16_t* __restrict__ q, const float* __restrict__ w,
                                               const uint8_t* __restrict__ K, const uint8_t* __restrict__ Ks,
                                               const int* __restrict__ q_pos, long long N_cap, int m,
                                               float* __restrict__ out, int b, long long key0) {
  constexpr int H = 16 * QH, DI = 128, RB = DI / 2, SB = DI / 32;
  const int lane = threadIdx.x & 63, g = lane >> 4, j = lane & 15;
  u32x4_t qa[QH];
  int qsc[QH];
  float wv[QH][4];
#pragma unroll
  for (int mt = 0; mt < QH; ++mt) {
    const uint16_t* qp = q + ((size_t)b * H + 16 * mt + j) * (size_t)DI + 32 * g;
    u32x4_t raw[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) raw[c] = *(const u32x4_t*)(qp + 8 * c);
#pragma unroll
    for (int r = 0; r < 4; ++r) wv[mt][r] = w[(size_t)b * H + 16 * mt + 4 * g + r];
    float x[32];
    float a = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[8 * c + 2 * e] = __uint_as_float(raw[c][e] << 16);
        x[8 * c + 2 * e + 1] = __uint_as_float(raw[c][e] & 0xffff0000u);
        a = fmaxf(a, fmaxf(fabsf(x[8 * c + 2 * e]), fabsf(x[8 * c + 2 * e + 1])));
      }
    const int se = mx4_shared_exp(a);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      uint32_t pk = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) pk |= f32_to_e2m1(ldexpf(x[8 * d + e], -se)) << (4 * e);
      qa[mt][d] = pk;
    }
    qsc[mt] = se + 127;
  }
  const uint8_t* Kb = K + (size_t)b * (size_t)N_cap * RB;
  const uint8_t* Sb = Ks + (size_t)b * (size_t)N_cap * SB;
  float P[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const size_t row = (size_t)(key0 + 16 * u + j);
    const u32x4_t c = *(const u32x4_t*)(Kb + row * RB + 16 * g);
    const uint32_t sc = *(const uint32_t*)(Sb + row * SB);
    P[u] = mx4_partial<QH>(qa, qsc, wv, c, (int)((sc >> (8 * g)) & 0xffu));
  }
  const float v = reduce_scatter4(P, g);
  const long long key = key0 + 16 * g + j;
  const long long nvis = min(N_cap, ((long long)q_pos[b] + 1) / m);
  out[(size_t)b * (size_t)N_cap + (size_t)key] = key < nvis ? v : -INFINITY;
}

template <int QH>
__global__ __launch_bounds__(256) void index_mx4_front(
    const FrontJobs fj, const uint16_t* __restrict__ q, const float* __restrict__ w,
    const uint8_t* __restrict__ K, const uint8_t* __restrict__ Ks, const int* __restrict__ q_pos,
    long long N_cap, int m, float* __restrict__ out, int flush_ok, int gx, int B) {
  (void)fj;
  const FrontJobs& F = *(const FrontJobs*)__builtin_amdgcn_kernarg_segment_ptr();
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const long long nunits = N_cap / (16 * IDX_UNIT);   // (host: N_cap % 64 == 0)
  const int nidx = gx * B;
  if ((int)blockIdx.x < nidx) {
    const int b = (int)blockIdx.x / gx, x = (int)blockIdx.x - b * gx;
    index_mx4_wave<QH>(q, w, K, Ks, q_pos, 1, N_cap, N_cap - 16 * IDX_UNIT, m, out, flush_ok, b, 0,
                       4LL * x + wave, 4LL * gx, nunits - 1);
    return;
  }
  const int b = (int)blockIdx.x - nidx;
  if (wave < F.n_jobs) {
    const CompressJob& J = F.job[wave];
    for (long long e = 0; e < J.n_entries; ++e) {
      const long long s = J.s_begin + e;
      if (J.out_dtype == DT_MX4) compress_entry_wave<DT_BF16, DT_MX4, COMPW_MAXC>(J, s, b, lane);
      else if (J.out_dtype == DT_MIX) compress_entry_wave<DT_BF16, DT_MIX, COMPW_MAXC>(J, s, b, lane);
      else compress_entry_wave<DT_BF16, DT_BF16, COMPW_MAXC>(J, s, b, lane);
    }
  }
  if (wave != F.key_job) return;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
  // (through the key job's own pointers, equal to K and Ks; see index_decode_front)
  mx4_score_unit<QH>(q, w, (const uint8_t*)F.job[F.key_job].E, (const uint8_t*)F.job[F.key_job].E_scale, q_pos,
                     N_cap, m, out, b, 16 * IDX_UNIT * (nunits - 1));
}

// ---------------------------------------------------------------------------
// prefill: a workgroup owns 4*QPW consecutive query rows (QPW per wave, query
// fragments resident in registers) and sweeps the visible keys in tiles of
// 64 staged through LDS (double-buffered, widened to bf16), so every key tile
// read from L2 feeds 4*QPW query rows.
// ---------------------------------------------------------------------------
static constexpr int PF_TK = 64;

template <int QH, int KS, int KDT, int QPW>
__global__ __launch_bounds__(256) void index_mfma_prefill(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const void* __restrict__ K,
    const float* __restrict__ Ks, const int* __restrict__ q_pos, int Tq, long long N_cap, int m,
    float* __restrict__ out) {
  constexpr int H = 16 * QH, DI = 32 * KS, GW = DI / 4;
  constexpr int ROWB = DI * 2 + 16;                     // padded LDS row (bytes), bf16
  constexpr int ESZ = (KDT == DT_FP8) ? 1 : 2;
  constexpr int PIECES = PF_TK * DI * ESZ / 16;         // 16-byte global pieces per tile
  constexpr int PPT = (PIECES + 255) / 256;
  constexpr int PPR = DI * ESZ / 16;                    // pieces per key row
  __shared__ __attribute__((aligned(16))) uint8_t kt[2][PF_TK * ROWB];
  __shared__ float ksc[2][PF_TK];

  // the wave index through readfirstlane: a wave's query rows, their visible
  // counts and output rows are then scalar (registers are what bound occupancy here)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int b = blockIdx.y;
  const int ncap = (int)N_cap;   // < 2^31 (the entry point checks)
  const int t0 = blockIdx.x * (4 * QPW);

  // visible range of the whole workgroup
  long long kend = 0;
  for (int e = 0; e < 4 * QPW; ++e) {
    const int t = t0 + e;
    if (t < Tq) kend = max(kend, min(N_cap, ((long long)q_pos[(size_t)b * Tq + t] + 1) / m));
  }
  const long long ntiles = (kend + PF_TK - 1) / PF_TK;

  IdxFrags<QH, KS> f[QPW];
  int nvis[QPW];
  bool tok[QPW];
  float* orow[QPW];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    const int t = t0 + wave * QPW + qq;
    tok[qq] = t < Tq;
    const size_t qrow = (size_t)b * Tq + (tok[qq] ? t : t0);
    load_query_frags<QH, KS>(f[qq], q + qrow * (size_t)(H * DI), w + qrow * H, g, j);
    nvis[qq] = (int)min(N_cap, ((long long)q_pos[qrow] + 1) / m);
    orow[qq] = out + qrow * (size_t)N_cap;
  }
  const size_t kbase = (size_t)b * (size_t)N_cap;

  u32x4_t stage[PPT];
  float sstage = 1.f;
  auto gload = [&](long long tile) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int p = threadIdx.x + 256 * u;
      const int r = p / PPR, c16 = p % PPR;
      const long long key = tile * PF_TK + r;
      stage[u] = (p < PIECES && key < N_cap)
                     ? *(const u32x4_t*)((const uint8_t*)K + ((kbase + (size_t)key) * DI) * ESZ + c16 * 16)
                     : u32x4_t{0u, 0u, 0u, 0u};
    }
    if constexpr (KDT == DT_FP8) {
      const long long key = tile * PF_TK + threadIdx.x;
      sstage = (threadIdx.x < PF_TK && key < N_cap) ? Ks[kbase + (size_t)key] : 1.f;
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PPT; ++u) {
      const int p = threadIdx.x + 256 * u;
      if (p >= PIECES) continue;
      const int r = p / PPR, c16 = p % PPR;
      if constexpr (KDT == DT_BF16) {
        *(u32x4_t*)(&kt[buf][r * ROWB + c16 * 16]) = stage[u];
      } else {
        u32x4_t o0, o1;
        uint32_t lo, hi;
        fp8x4_to_bf16x4(stage[u][0], lo, hi); o0[0] = lo; o0[1] = hi;
        fp8x4_to_bf16x4(stage[u][1], lo, hi); o0[2] = lo; o0[3] = hi;
        fp8x4_to_bf16x4(stage[u][2], lo, hi); o1[0] = lo; o1[1] = hi;
        fp8x4_to_bf16x4(stage[u][3], lo, hi); o1[2] = lo; o1[3] = hi;
        *(u32x4_t*)(&kt[buf][r * ROWB + c16 * 32]) = o0;
        *(u32x4_t*)(&kt[buf][r * ROWB + c16 * 32 + 16]) = o1;
      }
    }
    if constexpr (KDT == DT_FP8)
      if (threadIdx.x < PF_TK) ksc[buf][threadIdx.x] = sstage;
  };

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();
  for (long long tile = 0; tile < ntiles; ++tile) {
    const int buf = (int)(tile & 1);
    if (tile + 1 < ntiles) gload(tile + 1);
    // per query, the lanes' shares of the tile's four subtiles, then one
    // reduce-scatter leaves lane (g, j) with key 16 g + j: a 256-byte store
    static_assert(PF_TK == 64, "four subtiles per tile");
    float P[QPW][4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      bf16x8_t Bf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        Bf[ks] = *(const bf16x8_t*)(&kt[buf][(16 * st + j) * ROWB + (GW * g + 8 * ks) * 2]);
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        P[qq][st] = partial_column<QH, KS>(f[qq], Bf);
        // materialised here, so the epilogue is not sunk below later subtiles
        // (which would keep their accumulators live: too many registers)
        asm volatile("" : "+v"(P[qq][st]));
      }
    }
    const int key = (int)tile * PF_TK + 16 * g + j;
#pragma unroll
    for (int qq = 0; qq < QPW; ++qq) {
      float v = reduce_scatter4(P[qq], g);
      if (tok[qq] && key < ncap) {
        if constexpr (KDT == DT_FP8) v *= ksc[buf][16 * g + j];
        __builtin_nontemporal_store(key < nvis[qq] ? v : -INFINITY, orow[qq] + key);
      }
    }
    if (tile + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }
  // entries past the workgroup's visible tiles
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    if (!tok[qq]) continue;
    for (long long key = ntiles * PF_TK + lane; key < N_cap; key += 64) orow[qq][key] = -INFINITY;
  }
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
bool index_mfma_supported(const IndexArgs& a) {
  if (a.q_dtype != DT_BF16) return false;
  if (a.k_dtype != DT_BF16 && a.k_dtype != DT_FP8) return false;
  if (!(a.H == 16 || a.H == 32 || a.H == 64)) return false;
  if (!(a.dI == 32 || a.dI == 64 || a.dI == 128)) return false;
  return true;
}

// waves of a kernel that fit on the whole device at once (cached per kernel)
static long long resident_waves(const void* kfn, int block) {
  static thread_local const void* last_fn = nullptr;
  static thread_local long long last = 0;
  if (kfn == last_fn) return last;
  int dev = 0, cus = 256, per_cu = 1;
  if (hipGetDevice(&dev) == hipSuccess)
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, block, 0) != hipSuccess || per_cu < 1)
    per_cu = 1;
  last_fn = kfn;
  last = (long long)cus * per_cu * (block / 64);
  return last;
}

static constexpr int PF_MIN_TQ = 8;   // query rows per sequence at which the LDS-tiled kernel is used
static constexpr int PF_QPW = 2;

// decode grid: at most one round of resident waves over the chip, shared by the
// query rows, a power of two per row (units then divide evenly at power-of-two
// caches: at 16 x 262,144 keys, 128 waves per row of 32 units each beat 192
// waves of 21 or 22 units by 2.5%), and enough waves per row that each wave's
// scores fit its LDS stage
static dim3 decode_grid(const IndexArgs& a, const void* kfn) {
  const long long waves = resident_waves(kfn, 256);
  const long long rows = (long long)a.B * a.Tq;
  const long long nunits = (a.N_cap + 16 * IDX_UNIT - 1) / (16 * IDX_UNIT);
  long long wpr = 1;
  while (2 * wpr <= waves / rows) wpr *= 2;
  wpr = max(wpr, (nunits * 16 * IDX_UNIT + IDX_STAGE - 1) / IDX_STAGE);
  wpr = min(wpr, nunits);
  return dim3((unsigned)((wpr + 3) / 4), (unsigned)a.Tq, (unsigned)a.B);
}

template <int QH>
static void launch_mx4(const IndexArgs& a, hipStream_t st) {
  auto kfn = index_mx4_decode<QH>;
  const dim3 grid = decode_grid(a, (const void*)kfn);
  const int flush_ok = (((uintptr_t)a.out) & 15u) == 0 && a.N_cap % (16 * IDX_UNIT) == 0;
  hipLaunchKernelGGL(kfn, grid, dim3(256), 0, st, (const uint16_t*)a.q, a.w, (const uint8_t*)a.K,
                     (const uint8_t*)a.K_scale, a.q_pos, a.Tq, a.N_cap, a.m, a.out, flush_ok);
}

template <int QH, int KS, int KDT>
static void launch_mfma(const IndexArgs& a, hipStream_t st) {
  const uint16_t* q = (const uint16_t*)a.q;
  if (a.Tq >= PF_MIN_TQ) {
    dim3 grid((unsigned)((a.Tq + 4 * PF_QPW - 1) / (4 * PF_QPW)), (unsigned)a.B);
    hipLaunchKernelGGL((index_mfma_prefill<QH, KS, KDT, PF_QPW>), grid, dim3(256), 0, st, q, a.w,
                       a.K, a.K_scale, a.q_pos, a.Tq, a.N_cap, a.m, a.out);
  } else {
    auto kfn = index_mfma_decode<QH, KS, KDT>;
    const dim3 grid = decode_grid(a, (const void*)kfn);
    // early flushes use 16-byte stores of whole units
    const int flush_ok = (((uintptr_t)a.out) & 15u) == 0 && a.N_cap % (16 * IDX_UNIT) == 0;
    hipLaunchKernelGGL((index_mfma_decode<QH, KS, KDT>), grid, dim3(256), 0, st, q, a.w, a.K,
                       a.K_scale, a.q_pos, a.Tq, a.N_cap, a.m, a.out, flush_ok);
  }
}

template <int QH, int KS>
static void launch_mfma_k(const IndexArgs& a, hipStream_t st) {
  if (a.k_dtype == DT_FP8) launch_mfma<QH, KS, DT_FP8>(a, st);
  else launch_mfma<QH, KS, DT_BF16>(a, st);
}

template <int QH>
static void launch_mfma_ks(const IndexArgs& a, hipStream_t st) {
  if (a.dI == 32) launch_mfma_k<QH, 1>(a, st);
  else if (a.dI == 64) launch_mfma_k<QH, 2>(a, st);
  else launch_mfma_k<QH, 4>(a, st);
}

// the MXFP4 matrix-core kernel: decode rows, 128-dim keys
static bool index_mx4_supported(const IndexArgs& a) {
  return a.k_dtype == DT_MX4 && a.q_dtype == DT_BF16 && a.dI == 128 && a.Tq < PF_MIN_TQ &&
         (a.H == 16 || a.H == 32 || a.H == 64) && (((uintptr_t)a.K) & 15u) == 0 &&
         (((uintptr_t)a.K_scale) & 3u) == 0 && (((uintptr_t)a.q) & 15u) == 0;
}

// the decode front: compress jobs beside the indexer (index_decode_front)
template <int QH, int KS, int KDT>
static void launch_front(const FrontJobs& fj, const IndexArgs& a, hipStream_t st) {
  auto kfn = index_decode_front<QH, KS, KDT>;
  // the indexer part's grid: the decode grid over every unit but the last
  const long long waves = resident_waves((const void*)kfn, 256);
  const long long nunits = a.N_cap / (16 * IDX_UNIT) - 1;
  long long wpr = 1;
  while (2 * wpr <= waves / a.B) wpr *= 2;
  wpr = std::max(wpr, (nunits * 16 * IDX_UNIT + IDX_STAGE - 1) / IDX_STAGE);
  wpr = std::min(wpr, nunits);
  const int gx = (int)((wpr + 3) / 4);
  const int flush_ok = (((uintptr_t)a.out) & 15u) == 0;   // (N_cap % 64 == 0: checked)
  hipLaunchKernelGGL(kfn, dim3((unsigned)((gx + 1) * a.B)), dim3(256), 0, st, fj, (const uint16_t*)a.q, a.w, a.K,
                     a.K_scale, a.q_pos, a.N_cap, a.m, a.out, flush_ok, gx, a.B);
}
template <int QH, int KS>
static void launch_front_k(const FrontJobs& fj, const IndexArgs& a, hipStream_t st) {
  if (a.k_dtype == DT_FP8) launch_front<QH, KS, DT_FP8>(fj, a, st);
  else launch_front<QH, KS, DT_BF16>(fj, a, st);
}
template <int QH>
static void launch_front_ks(const FrontJobs& fj, const IndexArgs& a, hipStream_t st) {
  if (a.dI == 32) launch_front_k<QH, 1>(fj, a, st);
  else if (a.dI == 64) launch_front_k<QH, 2>(fj, a, st);
  else launch_front_k<QH, 4>(fj, a, st);
}

// the decode front with MXFP4 keys (index_mx4_front)
template <int QH>
static void launch_front_mx4(const FrontJobs& fj, const IndexArgs& a, hipStream_t st) {
  auto kfn = index_mx4_front<QH>;
  const long long waves = resident_waves((const void*)kfn, 256);
  const long long nunits = a.N_cap / (16 * IDX_UNIT) - 1;
  long long wpr = 1;
  while (2 * wpr <= waves / a.B) wpr *= 2;
  wpr = std::max(wpr, (nunits * 16 * IDX_UNIT + IDX_STAGE - 1) / IDX_STAGE);
  wpr = std::min(wpr, nunits);
  const int gx = (int)((wpr + 3) / 4);
  const int flush_ok = (((uintptr_t)a.out) & 15u) == 0;
  hipLaunchKernelGGL(kfn, dim3((unsigned)((gx + 1) * a.B)), dim3(256), 0, st, fj, (const uint16_t*)a.q, a.w,
                     (const uint8_t*)a.K, (const uint8_t*)a.K_scale, a.q_pos, a.N_cap, a.m, a.out, flush_ok, gx,
                     a.B);
}

int launch_decode_front(const CompressArgs* jobs, int n_jobs, const IndexArgs& a, hipStream_t st,
                        const char** why) {
  *why = nullptr;
  auto no = [&](const char* w) {
    *why = w;
    return -1;
  };
  const bool mx4 = a.k_dtype == DT_MX4;
  if (mx4 ? !index_mx4_supported(a) : !index_mfma_supported(a))
    return no("the indexer shape has no matrix-core decode kernel");
  if (a.Tq != 1) return no("one query row per sequence");
  if (a.N_cap % (16 * IDX_UNIT) != 0 || a.N_cap < 2 * 16 * IDX_UNIT)
    return no("N_cap must be a multiple of 64, at least 128");
  if ((((uintptr_t)a.q) & 15u) != 0 || (((uintptr_t)a.K) & 15u) != 0)
    return no("q_I and K_I must be 16-byte aligned");
  if (n_jobs < 1 || n_jobs > FRONT_MAX_JOBS) return no("1 to 4 compress jobs");
  FrontJobs fj{};
  fj.n_jobs = n_jobs;
  fj.key_job = -1;
  // the key rows and their scales: only the key job may write there
  const size_t key_bytes = (size_t)a.B * (size_t)a.N_cap * (size_t)(mx4 ? a.dI / 2 : a.dI * (a.k_dtype == DT_FP8 ? 1 : 2));
  const size_t ks_bytes = (size_t)a.B * (size_t)a.N_cap * (mx4 ? (size_t)(a.dI / 32) : sizeof(float));
  auto inside = [](const void* p, const void* lo, size_t n) {
    return lo && (uintptr_t)p >= (uintptr_t)lo && (uintptr_t)p < (uintptr_t)lo + n;
  };
  for (int q = 0; q < n_jobs; ++q) {
    const CompressArgs& x = jobs[q];
    if (x.E != a.K && (inside(x.E, a.K, key_bytes) || inside(x.E_scale, a.K_scale, ks_bytes)))
      return no("a job other than the key job writes into K_I or K_scale");
    // bf16 or mixed rows beside either indexer; fp8 key rows beside the fp8
    // one, MXFP4 beside the MXFP4 one
    const bool fmt = x.out_dtype == DT_BF16 || x.out_dtype == DT_MIX || x.out_dtype == (mx4 ? DT_MX4 : DT_FP8);
    if (x.in_dtype != DT_BF16 || !fmt || !compress_wave_ok(x, mx4, true))
      return no("a compress job the wave-per-entry compressor does not cover (bf16 inputs in 16-byte pieces, "
                "at most 8 candidates, bf16 or mixed-row output, or the key format)");
    if (x.B != a.B) return no("every compress job has the indexer's batch");
    if (x.E == a.K) {
      if (fj.key_job >= 0) return no("one compress job writes the key rows");
      const bool scaled = a.k_dtype == DT_FP8 || mx4;
      if (x.out_dtype != a.k_dtype || x.c != a.dI || x.out_ring != 0 || x.out_bs != a.N_cap * (long long)a.dI ||
          (scaled && (const void*)x.E_scale != (const void*)a.K_scale))
        return no("the key job must write K_I's rows (and K_scale) in the indexer's layout");
      if (x.s_begin < a.N_cap - 16 * IDX_UNIT || x.s_end > a.N_cap)
        return no("the key job's entries must lie in the last 64 rows of K_I");
      fj.key_job = q;
    }
    fj.job[q] = make_compress_job(x, 1);
  }
  if (fj.key_job < 0) return no("no compress job writes K_I");
  if (mx4) {
    if (a.H == 16) launch_front_mx4<1>(fj, a, st);
    else if (a.H == 32) launch_front_mx4<2>(fj, a, st);
    else launch_front_mx4<4>(fj, a, st);
  } else if (a.H == 16) {
    launch_front_ks<1>(fj, a, st);
  } else if (a.H == 32) {
    launch_front_ks<2>(fj, a, st);
  } else {
    launch_front_ks<4>(fj, a, st);
  }
  return 0;
}

int launch_index_score(const IndexArgs& a, hipStream_t st) {
  if (index_mx4_supported(a)) {
    if (a.H == 16) launch_mx4<1>(a, st);
    else if (a.H == 32) launch_mx4<2>(a, st);
    else launch_mx4<4>(a, st);
  } else if (index_mfma_supported(a)) {
    if (a.H == 16) launch_mfma_ks<1>(a, st);
    else if (a.H == 32) launch_mfma_ks<2>(a, st);
    else launch_mfma_ks<4>(a, st);
  } else {
    dim3 grid((unsigned)((a.N_cap + 255) / 256), (unsigned)a.Tq, (unsigned)a.B);
    const size_t lds = (size_t)(a.H * a.dI + a.H) * sizeof(float);
#define CSA_IDX_VALU(QD, KD)                                                                   \
  hipLaunchKernelGGL((index_valu_kernel<QD, KD>), grid, dim3(256), lds, st, a.q, a.w, a.K,     \
                     a.K_scale, a.q_pos, a.Tq, a.H, a.dI, a.N_cap, a.m, a.out)
    if (a.q_dtype == DT_F32) {
      if (a.k_dtype == DT_F32) CSA_IDX_VALU(DT_F32, DT_F32);
      else if (a.k_dtype == DT_BF16) CSA_IDX_VALU(DT_F32, DT_BF16);
      else CSA_IDX_VALU(DT_F32, DT_FP8);
    } else {
      if (a.k_dtype == DT_F32) CSA_IDX_VALU(DT_BF16, DT_F32);
      else if (a.k_dtype == DT_BF16) CSA_IDX_VALU(DT_BF16, DT_BF16);
      else if (a.k_dtype == DT_FP8) CSA_IDX_VALU(DT_BF16, DT_FP8);
      else CSA_IDX_VALU(DT_BF16, DT_MX4);
    }
#undef CSA_IDX_VALU
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
