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
//
// One launch runs a batch of independent jobs (blockIdx.z): a decode step's
// window row, KV entry and indexer key are each a few microseconds of memory
// and barrier latency, which overlap in one launch instead of adding up.  Each
// job's dtypes are chosen at run time (uniform per workgroup).
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

static constexpr int COMP_THREADS = 512;
static constexpr int COMP_MAX_G = 8;
static constexpr int COMP_JU = 8;   // channels per thread whose loads are issued together
static constexpr int COMP_MAX_JOBS = 8;

// one job's arguments as the kernel reads them (validated on the host)
struct CompressJob {
  const void *Ca, *Za, *Cb, *Zb;
  const float* gamma;
  void* E;
  float* E_scale;
  long long in_bs, tok_base, T, s_begin, n_entries, pos_stride, pos_offset, out_bs, out_ring;
  RopeRatio rope;
  float eps;
  int in_dtype, out_dtype, B, c, m, overlap, G, rope_dim;
};
struct CompressBatch {
  CompressJob job[COMP_MAX_JOBS];
};

template <int IDT, int ODT>
__device__ __forceinline__ void compress_entry(const CompressJob& J, float* smem) {
  const void* __restrict__ Ca = J.Ca;
  const void* __restrict__ Za = J.Za;
  const void* __restrict__ Cb = J.Cb;
  const void* __restrict__ Zb = J.Zb;
  const float* __restrict__ gamma = J.gamma;
  void* __restrict__ E = J.E;
  float* __restrict__ E_scale = J.E_scale;
  const long long in_bs = J.in_bs, tok_base = J.tok_base, T = J.T, s_begin = J.s_begin;
  const long long pos_stride = J.pos_stride, pos_offset = J.pos_offset, out_bs = J.out_bs;
  const long long out_ring = J.out_ring;
  const RopeRatio rope = J.rope;
  const float eps = J.eps;
  const int c = J.c, m = J.m, overlap = J.overlap, G = J.G, rope_dim = J.rope_dim;
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

  // gamma of this thread's output channels and of their RoPE partners, loaded
  // now so that their latency overlaps the candidates' (c <= 1024)
  constexpr int OPT = (1024 + COMP_THREADS - 1) / COMP_THREADS;
  const float* __restrict__ gsrc = gamma ? gamma : k_ones.v;
  float gj[OPT], gp[OPT];
#pragma unroll
  for (int i = 0; i < OPT; ++i) {
    const int j = min((int)threadIdx.x + i * COMP_THREADS, c - 1);
    gj[i] = gsrc[j];
    gp[i] = gsrc[min(j ^ 1, c - 1)];
  }

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
      // unconditional loads (channel clamped, a missing Z reads C), masked
      // afterwards: a guarded load becomes a branch with its own wait, and the
      // COMP_JU loads would then run one memory latency after another
      const void* Zq = Zp ? Zp : Cp;
      float x[COMP_JU], z[COMP_JU];
#pragma unroll
      for (int u = 0; u < COMP_JU; ++u) {
        const int j = min(j0 + u * tpg, c - 1);
        x[u] = load_as_f32<IDT>(Cp, off0 + (size_t)j);
        z[u] = load_as_f32<IDT>(Zq, off0 + (size_t)j);
      }
#pragma unroll
      for (int u = 0; u < COMP_JU; ++u) {
        const bool live = j0 + u * tpg < c;
        x[u] = live ? x[u] : 0.f;
        z[u] = (live && Zp) ? z[u] : 0.f;
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
    // all G partials read at once (group index clamped, the extra ones unused)
    float pm[COMP_MAX_G], ps[COMP_MAX_G], pa[COMP_MAX_G];
#pragma unroll
    for (int q = 0; q < COMP_MAX_G; ++q) {
      const int o = min(q, G - 1) * c + j;
      pm[q] = pmax[o];
      ps[q] = psum[o];
      pa[q] = pacc[o];
    }
    float M = -INFINITY;
#pragma unroll
    for (int q = 0; q < COMP_MAX_G; ++q)
      if (q < G) M = fmaxf(M, pm[q]);
    float S = 0.f, A = 0.f;
#pragma unroll
    for (int q = 0; q < COMP_MAX_G; ++q) {
      if (q >= G || pm[q] == -INFINITY) continue;   // no such group, or it saw no candidate
      const float f = __expf(pm[q] - M);
      S += ps[q] * f;
      A += pa[q] * f;
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
  float outv[OPT];
  int nv = 0;
  for (int j = threadIdx.x; j < c; j += COMP_THREADS, ++nv) {
    float v = row[j] * rinv * gj[nv];
    if (j >= rbeg) {
      const int u = (j - rbeg) >> 1;
      float cs, sn;
      rope_cos_sin(pos, u, rope, &cs, &sn);
      const float other = row[j ^ 1] * rinv * gp[nv];
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

__global__ __launch_bounds__(COMP_THREADS) void compress_kernel(const CompressBatch jb) {
  extern __shared__ float smem[];
  const CompressJob& J = jb.job[blockIdx.z];
  if ((long long)blockIdx.x >= J.n_entries || (int)blockIdx.y >= J.B) return;
  switch (J.in_dtype * 3 + J.out_dtype) {
    case DT_F32 * 3 + DT_F32: compress_entry<DT_F32, DT_F32>(J, smem); break;
    case DT_F32 * 3 + DT_BF16: compress_entry<DT_F32, DT_BF16>(J, smem); break;
    case DT_F32 * 3 + DT_FP8: compress_entry<DT_F32, DT_FP8>(J, smem); break;
    case DT_BF16 * 3 + DT_F32: compress_entry<DT_BF16, DT_F32>(J, smem); break;
    case DT_BF16 * 3 + DT_BF16: compress_entry<DT_BF16, DT_BF16>(J, smem); break;
    default: compress_entry<DT_BF16, DT_FP8>(J, smem); break;
  }
}

static size_t compress_lds_bytes(int G, int c) {
  return (size_t)(3 * G * c + c + COMP_THREADS / 64) * sizeof(float);
}

int launch_compress(const CompressArgs* a, int n_jobs, hipStream_t st) {
  if (n_jobs < 1 || n_jobs > COMP_MAX_JOBS) return -1;
  CompressBatch jb{};
  size_t lds = 0;
  long long gx = 1;
  int gy = 1;
  for (int q = 0; q < n_jobs; ++q) {
    const CompressArgs& x = a[q];
    const int ncand_max = x.overlap ? 2 * x.m : x.m;
    int G = ncand_max < COMP_MAX_G ? ncand_max : COMP_MAX_G;
    if (G < 1) G = 1;
    CompressJob& J = jb.job[q];
    J.Ca = x.C_a; J.Za = x.Z_a; J.Cb = x.C_b; J.Zb = x.Z_b;
    J.gamma = x.gamma; J.E = x.E; J.E_scale = x.E_scale;
    J.in_bs = x.in_bs; J.tok_base = x.tok_base; J.T = x.T; J.s_begin = x.s_begin;
    J.n_entries = x.s_end - x.s_begin;
    J.pos_stride = x.pos_stride; J.pos_offset = x.pos_offset;
    J.out_bs = x.out_bs; J.out_ring = x.out_ring;
    J.rope = rope_ratio(x.rope_dim, x.rope_base);
    J.eps = x.eps;
    J.in_dtype = x.in_dtype; J.out_dtype = x.out_dtype;
    J.B = x.B; J.c = x.c; J.m = x.m; J.overlap = x.overlap; J.G = G; J.rope_dim = x.rope_dim;
    const size_t l = compress_lds_bytes(G, x.c);
    if (l > lds) lds = l;
    if (J.n_entries > gx) gx = J.n_entries;
    if (x.B > gy) gy = x.B;
  }
  if (gx > 2147483647LL || gy > 65535) return -1;
  if (lds > 65536 && hipFuncSetAttribute((const void*)compress_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize,
                                         (int)lds) != hipSuccess)
    return -1;
  hipLaunchKernelGGL(compress_kernel, dim3((unsigned)gx, (unsigned)gy, (unsigned)n_jobs),
                     dim3(COMP_THREADS), lds, st, jb);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
