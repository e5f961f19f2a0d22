// a1 — KV compressor: softmax pooling over overlapping (CSA) or disjoint (HCA)
// token blocks, then RMSNorm and partial RoPE, for gfx950.
//
// DeepSeek-V4 method page, section 3.3: each entry is a softmax-weighted sum of
// 2m candidates drawn from two overlapping index ranges (rate exactly 1/m);
// HCA uses m' >> m with no overlap; entries get RMSNorm and RoPE on their last
// dims.  Set a = the entry's own block [m s, m(s+1)), set b = the previous
// block [m(s-1), m s), both clipped to [0, T).
//
// One workgroup per (entry, sequence).  The workgroup is split into G
// candidate groups: group g pools every G-th candidate for all channels with
// an online softmax (running max, running sum, running weighted sum), and the
// G partial results are merged in LDS.  This keeps a 128-candidate HCA block
// from serialising 128 dependent loads per thread.  Reads are coalesced along
// the channel axis; HBM traffic is one pass over C and Z.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

static constexpr int COMP_THREADS = 512;
static constexpr int COMP_MAX_G = 8;
static constexpr int COMP_JU = 8;   // channels per thread whose loads are issued together

template <int IDT, int ODT>
__global__ __launch_bounds__(COMP_THREADS) void compress_kernel(
    const void* __restrict__ Ca, const void* __restrict__ Za, const void* __restrict__ Cb,
    const void* __restrict__ Zb, long long in_bs, long long tok_base, long long T, int c, int m,
    int overlap, long long s_begin, int G, const float* __restrict__ gamma, float eps, int rope_dim,
    RopeRatio rope, long long pos_stride, long long pos_offset, void* __restrict__ E,
    float* __restrict__ E_scale, long long out_bs, long long out_ring) {
  extern __shared__ float smem[];
  float* pmax = smem;                 // [G][c]
  float* psum = pmax + G * c;         // [G][c]
  float* pacc = psum + G * c;         // [G][c]
  float* row = pacc + G * c;          // [c]
  float* red = row + c;               // [COMP_THREADS / 64]

  const long long s = s_begin + blockIdx.x;
  const int b = blockIdx.y;
  const long long a_lo = (long long)m * s;
  const long long a_hi = min((long long)m * (s + 1), T);
  long long b_lo = 0, b_hi = 0;
  if (overlap) {
    b_lo = max((long long)m * (s - 1), 0LL);
    b_hi = min((long long)m * s, T);
  }
  const long long na = max(a_hi - a_lo, 0LL);
  const long long nb = max(b_hi - b_lo, 0LL);
  const long long ncand = na + nb;
  const size_t base = (size_t)b * (size_t)in_bs;

  const int tpg = COMP_THREADS / G;
  const int g = threadIdx.x / tpg;
  const int tg = threadIdx.x % tpg;

  // ---- partial online softmax over candidates g, g+G, g+2G, ...
  // COMP_JU channels per thread at a time, so their loads are all in flight
  // before any is used (one channel at a time, every channel costs a memory
  // latency, and at decode one workgroup per sequence is all the parallelism)
  for (int j0 = tg; j0 < c; j0 += tpg * COMP_JU) {
    float mx[COMP_JU], sum[COMP_JU], acc[COMP_JU];
#pragma unroll
    for (int u = 0; u < COMP_JU; ++u) {
      mx[u] = -INFINITY;
      sum[u] = 0.f;
      acc[u] = 0.f;
    }
#pragma unroll 2
    for (long long q = g; q < ncand; q += G) {
      const bool in_a = q < na;
      const long long tok = in_a ? a_lo + q : b_lo + (q - na);
      const size_t off0 = base + (size_t)(tok - tok_base) * (size_t)c;
      const void* Cp = in_a ? Ca : Cb;
      const void* Zp = in_a ? Za : Zb;
      float x[COMP_JU], z[COMP_JU];
#pragma unroll
      for (int u = 0; u < COMP_JU; ++u) {
        const int j = j0 + u * tpg;
        x[u] = j < c ? load_as_f32<IDT>(Cp, off0 + (size_t)j) : 0.f;
        z[u] = (j < c && Zp) ? load_as_f32<IDT>(Zp, off0 + (size_t)j) : 0.f;
      }
#pragma unroll
      for (int u = 0; u < COMP_JU; ++u) {
        if (z[u] > mx[u]) {
          const float r = __expf(mx[u] - z[u]);   // mx = -inf on the first candidate gives 0
          sum[u] = sum[u] * r + 1.f;
          acc[u] = acc[u] * r + x[u];
          mx[u] = z[u];
        } else {
          const float e = __expf(z[u] - mx[u]);
          sum[u] += e;
          acc[u] += e * x[u];
        }
      }
    }
#pragma unroll
    for (int u = 0; u < COMP_JU; ++u) {
      const int j = j0 + u * tpg;
      if (j < c) {
        pmax[g * c + j] = mx[u];
        psum[g * c + j] = sum[u];
        pacc[g * c + j] = acc[u];
      }
    }
  }
  __syncthreads();

  // ---- merge the G partials; pooled value per channel
  float ss = 0.f;
  for (int j = threadIdx.x; j < c; j += COMP_THREADS) {
    float M = -INFINITY;
    for (int q = 0; q < G; ++q) M = fmaxf(M, pmax[q * c + j]);
    float S = 0.f, A = 0.f;
    for (int q = 0; q < G; ++q) {
      const float mq = pmax[q * c + j];
      if (mq == -INFINITY) continue;      // group saw no candidate
      const float f = __expf(mq - M);
      S += psum[q * c + j] * f;
      A += pacc[q * c + j] * f;
    }
    const float v = S > 0.f ? A / S : 0.f;
    row[j] = v;
    ss += v * v;
  }

  // ---- RMSNorm over the c channels
  float rinv = 1.f;
  if (gamma) {
    const float tot = block_reduce<false>(ss, red);
    rinv = 1.f / sqrtf(tot / (float)c + eps);
  }
  __syncthreads();

  // ---- RoPE on the last rope_dim channels, pairs (2u, 2u+1); then store
  const long long pos = pos_stride * s + pos_offset;
  const long long orow = out_ring > 0 ? (s % out_ring) : s;
  const size_t obase = (size_t)b * (size_t)out_bs + (size_t)orow * (size_t)c;
  const int rbeg = c - rope_dim;
  float amax = 0.f;
  float outv[(1024 + COMP_THREADS - 1) / COMP_THREADS];
  int nv = 0;
  for (int j = threadIdx.x; j < c; j += COMP_THREADS, ++nv) {
    float v = row[j] * rinv * (gamma ? gamma[j] : 1.f);
    if (j >= rbeg) {
      const int u = (j - rbeg) >> 1;
      float cs, sn;
      rope_cos_sin(pos, u, rope, &cs, &sn);
      const float other = row[j ^ 1] * rinv * (gamma ? gamma[j ^ 1] : 1.f);
      v = (j & 1) ? (other * sn + v * cs) : (v * cs - other * sn);
    }
    outv[nv] = v;
    amax = fmaxf(amax, fabsf(v));
  }
  if constexpr (ODT == DT_FP8) {
    const float am = block_reduce<true>(amax, red);
    const float scale = am > 0.f ? am / 448.0f : 1.0f;
    nv = 0;
    for (int j = threadIdx.x; j < c; j += COMP_THREADS, ++nv)
      ((uint8_t*)E)[obase + j] = f32_to_e4m3(outv[nv] / scale);
    if (threadIdx.x == 0) E_scale[(size_t)b * (size_t)(out_bs / c) + (size_t)orow] = scale;
  } else {
    nv = 0;
    for (int j = threadIdx.x; j < c; j += COMP_THREADS, ++nv) store_from_f32<ODT>(E, obase + j, outv[nv]);
  }
}

int launch_compress(const CompressArgs& a, hipStream_t st) {
  const RopeRatio rope_rr = rope_ratio(a.rope_dim, a.rope_base);
  const int ncand_max = a.overlap ? 2 * a.m : a.m;
  int G = ncand_max < COMP_MAX_G ? ncand_max : COMP_MAX_G;
  if (G < 1) G = 1;
  const size_t lds = (size_t)(3 * G * a.c + a.c + COMP_THREADS / 64) * sizeof(float);
  dim3 grid((unsigned)(a.s_end - a.s_begin), (unsigned)a.B);
  dim3 block(COMP_THREADS);
#define CSA_COMP_LAUNCH(IDT, ODT)                                                                  \
  do {                                                                                             \
    auto kfn = compress_kernel<IDT, ODT>;                                                          \
    if (lds > 65536 &&                                                                             \
        hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize,         \
                            (int)lds) != hipSuccess)                                               \
      return -1;                                                                                   \
    hipLaunchKernelGGL(kfn, grid, block, lds, st, a.C_a, a.Z_a, a.C_b, a.Z_b, a.in_bs, a.tok_base, \
                       a.T, a.c, a.m, a.overlap, a.s_begin, G, a.gamma, a.eps, a.rope_dim,         \
                       rope_rr, a.pos_stride, a.pos_offset, a.E, a.E_scale, a.out_bs,          \
                       a.out_ring);                                                                \
  } while (0)
  if (a.in_dtype == DT_F32) {
    if (a.out_dtype == DT_F32) CSA_COMP_LAUNCH(DT_F32, DT_F32);
    else if (a.out_dtype == DT_BF16) CSA_COMP_LAUNCH(DT_F32, DT_BF16);
    else CSA_COMP_LAUNCH(DT_F32, DT_FP8);
  } else {
    if (a.out_dtype == DT_F32) CSA_COMP_LAUNCH(DT_BF16, DT_F32);
    else if (a.out_dtype == DT_BF16) CSA_COMP_LAUNCH(DT_BF16, DT_BF16);
    else CSA_COMP_LAUNCH(DT_BF16, DT_FP8);
  }
#undef CSA_COMP_LAUNCH
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
