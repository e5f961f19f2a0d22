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
// scaling the key inside the ReLU.
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
      const float kv = load_key<KDT>(K, kb + d);
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

// sum over heads of w * ReLU(dot) for the key column of this lane, complete in every lane
template <int QH, int KS>
__device__ __forceinline__ float score_column(const IdxFrags<QH, KS>& f, const bf16x8_t (&Bf)[KS]) {
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
    for (int r = 0; r < 4; ++r) part += f.wv[mt][r] * fmaxf(acc[mt][r], 0.f);
  part += __shfl_xor(part, 16, 64);
  part += __shfl_xor(part, 32, 64);
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
// decode: few query rows, keys streamed from HBM straight into registers.
// Each wave owns kpw consecutive keys of one query row and walks them in
// subtiles of 16 keys with a prefetch ring of PF subtiles in flight.  Four
// subtiles form a group: every lane first sums its 16 head rows per subtile,
// then a reduce-scatter across the 4 lane groups (3 cross-lane adds) leaves
// lane (g, j) with the full score of key j of subtile g, so each group ends
// in one coalesced 256-byte store.
// ---------------------------------------------------------------------------
template <int KS, int KDT>
struct RawSub {                       // one lane's bytes of one key row for one subtile
  static constexpr int WORDS = (KDT == DT_FP8 ? 8 * KS : 16 * KS) / 4;
  uint32_t w[WORDS];
};

// Lane (g, j) reads row j of the subtile in 16-byte pieces at bytes 64 c + 16 g:
// load instruction c then covers 64 contiguous bytes of each of the 16 rows.
// The dims a lane ends up with per K-step are given by dec_dim below, and the
// query fragments follow the same order.
template <int KS, int KDT>
__device__ __forceinline__ void load_raw(RawSub<KS, KDT>& r, const void* __restrict__ K, size_t row,
                                         int g) {
  // Unconditional: the caller clamps row to a key of the sequence, and the
  // score of a slot past the end is never stored (a slot only feeds its own
  // key column), so no masking, and no select that would wait on the load.
  constexpr int BYTES = RawSub<KS, KDT>::WORDS * 4;   // bytes of this lane
  const uint8_t* base = (const uint8_t*)K + row * (size_t)(BYTES * 4);
  if constexpr (BYTES % 16 == 0) {
    const uint8_t* p = base + 16 * g;
#pragma unroll
    for (int c = 0; c < BYTES / 16; ++c) {   // streamed once: non-temporal
      const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)(p + 64 * c));
#pragma unroll
      for (int e = 0; e < 4; ++e) r.w[4 * c + e] = v[e];
    }
  } else {
    const u32x2_t v = *(const u32x2_t*)(base + BYTES * g);
    r.w[0] = v[0];
    r.w[1] = v[1];
  }
}

template <int KS, int KDT>
__device__ __forceinline__ void raw_to_frags(const RawSub<KS, KDT>& r, bf16x8_t (&Bf)[KS]) {
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    if constexpr (KDT == DT_FP8) {
      // 8 codes -> 8 bf16, exactly (gfx950 conversion, scale 1)
      bf16x2_t a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w[2 * ks], 1.0f, false);
      bf16x2_t b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w[2 * ks], 1.0f, true);
      bf16x2_t c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w[2 * ks + 1], 1.0f, false);
      bf16x2_t d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)r.w[2 * ks + 1], 1.0f, true);
      u32x4_t o;
      o[0] = __builtin_bit_cast(uint32_t, a); o[1] = __builtin_bit_cast(uint32_t, b);
      o[2] = __builtin_bit_cast(uint32_t, c); o[3] = __builtin_bit_cast(uint32_t, d);
      Bf[ks] = __builtin_bit_cast(bf16x8_t, o);
    } else {
      u32x4_t o;
      o[0] = r.w[4 * ks]; o[1] = r.w[4 * ks + 1]; o[2] = r.w[4 * ks + 2]; o[3] = r.w[4 * ks + 3];
      Bf[ks] = __builtin_bit_cast(bf16x8_t, o);
    }
  }
}

// this lane's share (its 4*QH head rows) of sum_h w * ReLU(dot) for its key column
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
    for (int r = 0; r < 4; ++r) part += f.wv[mt][r] * fmaxf(acc[mt][r], 0.f);
  return part;
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

template <int QH, int KS, int KDT>
__global__ __launch_bounds__(256) void index_mfma_decode(
    const uint16_t* __restrict__ q, const float* __restrict__ w, const void* __restrict__ K,
    const float* __restrict__ Ks, const int* __restrict__ q_pos, int Tq, long long N_cap, int m,
    int kpw, float* __restrict__ out) {
  constexpr int H = 16 * QH, DI = 32 * KS;
  constexpr int PF = 4;   // subtiles in flight per wave
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int b = blockIdx.z, t = blockIdx.y;
  const size_t qrow = (size_t)b * Tq + t;
  const long long k0 = ((long long)blockIdx.x * 4 + wave) * kpw;
  if (k0 >= N_cap) return;
  const long long k1 = min(k0 + (long long)kpw, N_cap);
  const int nst = (int)((k1 - k0 + 15) / 16);
  const long long i = q_pos[qrow];
  const long long nvis = min(N_cap, (i + 1) / m);

  IdxFrags<QH, KS> f;
  load_query_frags_dec<QH, KS, KDT>(f, q + qrow * (size_t)(H * DI), w + qrow * H, g, j);
  // Retire the query loads here, before the loop: an (empty) use of every
  // fragment makes the compiler wait for them at this point, so the loop's wait
  // counts are fixed by the key ring alone (otherwise every iteration waits for
  // all keys in flight, as the first one must for these loads).
#pragma unroll
  for (int mt = 0; mt < QH; ++mt) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" ::"v"(f.A[mt][ks]));
#pragma unroll
    for (int r = 0; r < 4; ++r) asm volatile("" ::"v"(f.wv[mt][r]));
  }
  const size_t kbase = (size_t)b * (size_t)N_cap;
  float* orow = out + qrow * (size_t)N_cap;

  // The key ring holds PF = 4 subtiles in flight (slot u of a group of four);
  // a slot is consumed, then refilled with the subtile one group later.
  RawSub<KS, KDT> ring[PF];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const long long key = k0 + 16 * p + j;
    load_raw<KS, KDT>(ring[p], K, kbase + (size_t)(key < k1 ? key : k0), g);
    __builtin_amdgcn_sched_barrier(0);   // issue in slot order, as the loop refills them
  }
  // Unscaled scores are staged in LDS and written once the wave's keys are all
  // read: stores share the memory counter with the loads (waiting for a key
  // would also wait for every store before it), and the (fp8) row scales and
  // the visibility mask are applied in that pass with coalesced loads.
  __shared__ __attribute__((aligned(16))) float stage[4][IDX_STAGE];
#pragma unroll 1
  for (int st0 = 0; st0 < nst; st0 += 4) {
    float P[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      static_assert(PF == 4, "slot u of each group");
      P[u] = partial_column_raw<QH, KS, KDT>(f, ring[u]);
      // the sum is materialised here, so the epilogue is not sunk below the
      // later subtiles (which would keep 64 accumulators live instead of 16)
      asm volatile("" : "+v"(P[u]));
      const long long nkey = k0 + 16LL * (st0 + u + PF) + j;
      load_raw<KS, KDT>(ring[u], K, kbase + (size_t)(nkey < k1 ? nkey : k0), g);
      // keep the next slot's conversions out of this one (they would wait on its load)
      __builtin_amdgcn_sched_barrier(0);
    }
    const float v = reduce_scatter4(P, g);
    if (k0 + 16LL * (st0 + g) + j < k1) stage[wave][16 * (st0 + g) + j] = v;
  }
  const int n = (int)(k1 - k0);
  float* dst = orow + k0;
  const float* srow = Ks + kbase + k0;
  const bool vec = (((uintptr_t)dst) & 15u) == 0 && (KDT != DT_FP8 || (((uintptr_t)srow) & 15u) == 0);
  const int nv = (int)max(0LL, min((long long)n, nvis - k0));   // visible keys of the wave
  for (int e = 4 * lane; e < n; e += 256) {
    if (vec && e + 4 <= n) {
      f32x4_t v = *(const f32x4_t*)&stage[wave][e];
      if constexpr (KDT == DT_FP8) {
        const f32x4_t s4 = __builtin_nontemporal_load((const f32x4_t*)(srow + e));
        v = v * s4;
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) v[c] = e + c < nv ? v[c] : -INFINITY;
      __builtin_nontemporal_store(v, (f32x4_t*)(dst + e));
    } else {
      for (int c = e; c < min(e + 4, n); ++c) {
        float v = stage[wave][c];
        if constexpr (KDT == DT_FP8) v *= srow[c];
        dst[c] = c < nv ? v : -INFINITY;
      }
    }
  }
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

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int b = blockIdx.y;
  const int t0 = blockIdx.x * (4 * QPW);

  // visible range of the whole workgroup
  long long kend = 0;
  for (int e = 0; e < 4 * QPW; ++e) {
    const int t = t0 + e;
    if (t < Tq) kend = max(kend, min(N_cap, ((long long)q_pos[(size_t)b * Tq + t] + 1) / m));
  }
  const long long ntiles = (kend + PF_TK - 1) / PF_TK;

  IdxFrags<QH, KS> f[QPW];
  long long nvis[QPW];
  bool tok[QPW];
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    const int t = t0 + wave * QPW + qq;
    tok[qq] = t < Tq;
    const size_t qrow = (size_t)b * Tq + (tok[qq] ? t : t0);
    load_query_frags<QH, KS>(f[qq], q + qrow * (size_t)(H * DI), w + qrow * H, g, j);
    nvis[qq] = min(N_cap, ((long long)q_pos[qrow] + 1) / m);
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
#pragma unroll
    for (int st = 0; st < PF_TK / 16; ++st) {
      bf16x8_t Bf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        Bf[ks] = *(const bf16x8_t*)(&kt[buf][(16 * st + j) * ROWB + (GW * g + 8 * ks) * 2]);
      const long long key = tile * PF_TK + 16 * st + j;
#pragma unroll
      for (int qq = 0; qq < QPW; ++qq) {
        float v = score_column<QH, KS>(f[qq], Bf);
        if (g == 0 && tok[qq] && key < N_cap) {
          if constexpr (KDT == DT_FP8) v *= ksc[buf][16 * st + j];
          const int t = t0 + wave * QPW + qq;
          out[((size_t)b * Tq + t) * (size_t)N_cap + key] = key < nvis[qq] ? v : -INFINITY;
        }
      }
    }
    if (tile + 1 < ntiles) lstore(buf ^ 1);
    __syncthreads();
  }
  // entries past the workgroup's visible tiles
#pragma unroll
  for (int qq = 0; qq < QPW; ++qq) {
    if (!tok[qq]) continue;
    const int t = t0 + wave * QPW + qq;
    float* orow = out + ((size_t)b * Tq + t) * (size_t)N_cap;
    for (long long key = ntiles * PF_TK + lane; key < N_cap; key += 64) orow[key] = -INFINITY;
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

template <int QH, int KS, int KDT>
static void launch_mfma(const IndexArgs& a, hipStream_t st) {
  const uint16_t* q = (const uint16_t*)a.q;
  if (a.Tq >= PF_MIN_TQ) {
    dim3 grid((unsigned)((a.Tq + 4 * PF_QPW - 1) / (4 * PF_QPW)), (unsigned)a.B);
    hipLaunchKernelGGL((index_mfma_prefill<QH, KS, KDT, PF_QPW>), grid, dim3(256), 0, st, q, a.w,
                       a.K, a.K_scale, a.q_pos, a.Tq, a.N_cap, a.m, a.out);
  } else {
    // one round of resident waves over the chip, each wave at least 64 keys
    auto kfn = index_mfma_decode<QH, KS, KDT>;
    const long long waves = resident_waves((const void*)kfn, 256);
    long long rows = (long long)a.B * a.Tq;
    long long kpw = (a.N_cap * rows + waves - 1) / waves;
    kpw = ((kpw + 63) / 64) * 64;
    if (kpw < 64) kpw = 64;
    if (kpw > IDX_STAGE) kpw = IDX_STAGE;   // a wave's scores fit its LDS stage
    long long nblk = (a.N_cap + 4 * kpw - 1) / (4 * kpw);
    dim3 grid((unsigned)nblk, (unsigned)a.Tq, (unsigned)a.B);
    hipLaunchKernelGGL((index_mfma_decode<QH, KS, KDT>), grid, dim3(256), 0, st, q, a.w, a.K,
                       a.K_scale, a.q_pos, a.Tq, a.N_cap, a.m, (int)kpw, a.out);
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

int launch_index_score(const IndexArgs& a, hipStream_t st) {
  if (index_mfma_supported(a)) {
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
      else CSA_IDX_VALU(DT_BF16, DT_FP8);
    }
#undef CSA_IDX_VALU
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
