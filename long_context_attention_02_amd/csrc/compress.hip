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
// the channel axis; HBM traffic is one pass over C and Z.  With per-sequence
// token counts T_len, an entry whose block starts at or past T_len[b] does not
// exist in sequence b and its row is left as it was.
//
// One launch runs a batch of independent jobs (blockIdx.z): a decode step's
// window row, KV entry and indexer key are each a few microseconds of memory
// and barrier latency, which overlap in one launch instead of adding up.  Each
// job's dtypes are chosen at run time (uniform per workgroup).  Jobs of many
// entries (256 or more (sequence, entry) pairs, as in prefill) with at most 8
// candidates per entry (CSA m = 4, window rows) take the wave-per-entry kernel
// below instead: no LDS, no barriers.  The choice depends on the job alone, so
// a job gives the same result in any batch.
#include <algorithm>

#include "compress_wave.h"

namespace csa {

static constexpr int COMP_THREADS = 512;
static constexpr int COMP_MAX_G = 8;
static constexpr int COMP_JU = 8;   // channels per thread whose loads are issued together

struct CompressBatch {
  CompressJob job[COMP_MAX_JOBS];
};


// RMSNorm over the c channels of the pooled row (row[] in LDS; ss = this
// thread's share of the sum of squares), RoPE on the last rope_dim channels,
// then the store in the output format; NT threads, channel j in thread j mod NT
template <int ODT, int NT>
__device__ __forceinline__ void compress_store(const CompressJob& J, long long s, int b, const float* row,
                                               float ss, float* red, const float* gj, const float* gp) {
  constexpr int OPT = (1024 + NT - 1) / NT;
  void* __restrict__ E = J.E;
  float* __restrict__ E_scale = J.E_scale;
  const float* __restrict__ gamma = J.gamma;
  const long long pos_stride = J.pos_stride, pos_offset = J.pos_offset, out_bs = J.out_bs;
  const long long out_ring = J.out_ring;
  const RopeRatio rope = J.rope;
  const float eps = J.eps;
  const int c = J.c, rope_dim = J.rope_dim;
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
  for (int j = threadIdx.x; j < c; j += NT, ++nv) {
    float v = row[j] * rinv * gj[nv];
    if (j >= rbeg) {
      const int u = (j - rbeg) >> 1;
      float cs, sn;
      rope_cos_sin(pos, u, rope, &cs, &sn);
      const float other = row[j ^ 1] * rinv * gp[nv];
      v = (j & 1) ? (other * sn + v * cs) : (v * cs - other * sn);
    }
    outv[nv] = v;
    if (ODT != DT_MIX || j < rbeg) amax = fmaxf(amax, fabsf(v));   // mixed rows: the fp8 part only
  }
  if constexpr (ODT == DT_MIX) {
    // mixed row: e4m3 codes of channels [0, rbeg) under one row scale, bf16 of the rest
    const float am = block_reduce<true>(amax, red);
    const float scale = am > 0.f ? am / 448.0f : 1.0f;
    const size_t rowi = (size_t)b * (size_t)(out_bs / c) + (size_t)orow;
    uint8_t* rb = (uint8_t*)E + rowi * (size_t)(c + rope_dim);
    nv = 0;
    for (int j = threadIdx.x; j < c; j += NT, ++nv) {
      if (j < rbeg) rb[j] = f32_to_e4m3(outv[nv] / scale);
      else *(uint16_t*)(rb + rbeg + 2 * (j - rbeg)) = f32_to_bf16_bits(outv[nv]);
    }
    if (threadIdx.x == 0) E_scale[rowi] = scale;
  } else if constexpr (ODT == DT_FP8) {
    const float am = block_reduce<true>(amax, red);
    const float scale = am > 0.f ? am / 448.0f : 1.0f;
    nv = 0;
    for (int j = threadIdx.x; j < c; j += NT, ++nv)
      ((uint8_t*)E)[obase + j] = f32_to_e4m3(outv[nv] / scale);
    if (threadIdx.x == 0) E_scale[(size_t)b * (size_t)(out_bs / c) + (size_t)orow] = scale;
  } else if constexpr (ODT == DT_MX4) {
    // MXFP4: channel j sits in thread j (c % 32 == 0, so a 32-channel block is
    // 32 consecutive lanes of one wave): block maximum by lane exchange, codes,
    // the even channel's thread writes the byte of the pair, the block's first
    // thread its scale byte
    nv = 0;
    for (int j = threadIdx.x; j < c; j += NT, ++nv) {
      float a = fabsf(outv[nv]);
#pragma unroll
      for (int x = 1; x < 32; x <<= 1) a = fmaxf(a, __shfl_xor(a, x, 64));
      const int se = mx4_shared_exp(a);
      const uint32_t code = f32_to_e2m1(ldexpf(outv[nv], -se));
      const uint32_t other = (uint32_t)__shfl_xor((int)code, 1, 64);
      if ((j & 1) == 0) ((uint8_t*)E)[(obase + j) / 2] = (uint8_t)(code | (other << 4));
      if ((j & 31) == 0)
        ((uint8_t*)E_scale)[((size_t)b * (size_t)(out_bs / c) + (size_t)orow) * (size_t)(c / 32) + j / 32] =
            (uint8_t)(se + 127);
    }
  } else {
    nv = 0;
    for (int j = threadIdx.x; j < c; j += NT, ++nv) store_from_f32<ODT>(E, obase + j, outv[nv]);
  }
}

template <int IDT, int ODT>
__device__ __forceinline__ void compress_entry(const CompressJob& J, float* smem) {
  const void* __restrict__ Ca = J.Ca;
  const void* __restrict__ Za = J.Za;
  const void* __restrict__ Cb = J.Cb;
  const void* __restrict__ Zb = J.Zb;
  const float* __restrict__ gamma = J.gamma;
  void* __restrict__ E = J.E;
  float* __restrict__ E_scale = J.E_scale;
  const long long in_bs = J.in_bs, tok_base = J.tok_base, s_begin = J.s_begin;
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
  const long long T = seq_tokens(J, b);
  if ((long long)m * s >= T) return;   // no such entry in this sequence (whole workgroup)
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

  compress_store<ODT, COMP_THREADS>(J, s, b, row, ss, red, gj, gp);
}

__global__ __launch_bounds__(COMP_THREADS) void compress_kernel(const CompressBatch jb) {
  extern __shared__ float smem[];
  const CompressJob& J = jb.job[blockIdx.z];
  if ((long long)blockIdx.x >= J.n_entries || (int)blockIdx.y >= J.B) return;
  switch (J.in_dtype * 5 + J.out_dtype) {
    case DT_F32 * 5 + DT_F32: compress_entry<DT_F32, DT_F32>(J, smem); break;
    case DT_F32 * 5 + DT_BF16: compress_entry<DT_F32, DT_BF16>(J, smem); break;
    case DT_F32 * 5 + DT_FP8: compress_entry<DT_F32, DT_FP8>(J, smem); break;
    case DT_F32 * 5 + DT_MX4: compress_entry<DT_F32, DT_MX4>(J, smem); break;
    case DT_F32 * 5 + DT_MIX: compress_entry<DT_F32, DT_MIX>(J, smem); break;
    case DT_BF16 * 5 + DT_F32: compress_entry<DT_BF16, DT_F32>(J, smem); break;
    case DT_BF16 * 5 + DT_BF16: compress_entry<DT_BF16, DT_BF16>(J, smem); break;
    case DT_BF16 * 5 + DT_FP8: compress_entry<DT_BF16, DT_FP8>(J, smem); break;
    case DT_BF16 * 5 + DT_MX4: compress_entry<DT_BF16, DT_MX4>(J, smem); break;
    default: compress_entry<DT_BF16, DT_MIX>(J, smem); break;
  }
}

template <int MAXC>
__global__ __launch_bounds__(64 * COMPW_WAVES) void compress_wave_kernel(const CompressWaveBatch jb) {
  const int lane = threadIdx.x & 63;
  const long long item = (long long)blockIdx.x * COMPW_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (item >= jb.first[jb.n_jobs]) return;
  int q = 0;
  while (q + 1 < jb.n_jobs && item >= jb.first[q + 1]) ++q;
  const CompressJob& J = jb.job[q];
  const long long e = item - jb.first[q];
  const long long s = J.s_begin + e % J.n_entries;
  const int b = (int)(e / J.n_entries);
  switch (J.in_dtype * 5 + J.out_dtype) {
    case DT_F32 * 5 + DT_F32: compress_entry_wave<DT_F32, DT_F32, MAXC>(J, s, b, lane); break;
    case DT_F32 * 5 + DT_BF16: compress_entry_wave<DT_F32, DT_BF16, MAXC>(J, s, b, lane); break;
    case DT_F32 * 5 + DT_FP8: compress_entry_wave<DT_F32, DT_FP8, MAXC>(J, s, b, lane); break;
    case DT_BF16 * 5 + DT_F32: compress_entry_wave<DT_BF16, DT_F32, MAXC>(J, s, b, lane); break;
    case DT_BF16 * 5 + DT_BF16: compress_entry_wave<DT_BF16, DT_BF16, MAXC>(J, s, b, lane); break;
    default: compress_entry_wave<DT_BF16, DT_FP8, MAXC>(J, s, b, lane); break;
  }
}

// ---------------------------------------------------------------------------
// Wide kernel: one 1024-thread workgroup per (entry, sequence) for entries of
// many candidates (HCA blocks of m' = 128 tokens; also the few entries of a
// decode step).  Thread (token group tg, channel vector cv) owns 16-byte
// pieces (8 bf16 or 4 fp32 channels) of every TG-th candidate and issues the
// loads of up to COMPX_TPT candidates at once, so a 128-token block costs one
// memory latency rather than one per pair of candidates; each thread keeps an
// online softmax per channel, the TG partials of a channel merge in LDS, and
// the RMSNorm / RoPE / store epilogue is the one of the kernel above.
// ---------------------------------------------------------------------------
static constexpr int COMPX_THREADS = 1024;
static constexpr int COMPX_TPT = 4;    // candidates per thread whose loads are in flight together
static constexpr int COMPX_MAXTG = 16; // token groups (bounds the merge of a channel's partials)
// (1024 threads leave 128 VGPRs a thread; eight candidates in flight spilled)

template <int IDT, int ODT>
__device__ __forceinline__ void compress_entry_wide(const CompressJob& J, float* smem) {
  constexpr int VEC = IDT == DT_F32 ? 4 : 8;   // channels per 16-byte piece
  constexpr int ESZ = IDT == DT_F32 ? 4 : 2;
  const int c = J.c, m = J.m;
  const int ns = J.ns;                         // channel slices (1: whole rows)
  const int cs = c / ns;                       // channels of this workgroup (host: whole pieces)
  const int slice = ns > 1 ? (int)(blockIdx.x % (unsigned)ns) : 0;
  const long long ent = ns > 1 ? (long long)(blockIdx.x / (unsigned)ns) : (long long)blockIdx.x;
  const int c0 = slice * cs;
  const int CV = cs / VEC;                     // pieces per slice row (host: cs % VEC == 0, c <= 1024)
  const int TG = J.G;                          // token groups (host: wide_groups)
  const int b = blockIdx.y;
  long long s, T, tbase;
  if (J.T0) {   // append: the entries whose blocks complete with the new tokens
    const long long t0 = J.T0[b];
    s = t0 / m + J.s_begin + ent;
    T = t0 + J.n_new;
    if ((long long)m * (s + 1) > T) return;   // (whole workgroup)
    tbase = t0;
  } else {
    s = J.s_begin + ent;
    T = seq_tokens(J, b);
    if ((long long)m * s >= T) return;   // no such entry in this sequence (whole workgroup)
    tbase = J.tok_base;
  }
  if (J.out_rows > 0 && (J.out_ring > 0 ? s % J.out_ring : s) >= J.out_rows) return;
  const long long a_lo = (long long)m * s, a_hi = min((long long)m * (s + 1), T);
  long long b_lo = 0, b_hi = 0;
  if (J.overlap) {
    b_lo = max((long long)m * (s - 1), 0LL);
    b_hi = min((long long)m * s, T);
  }
  const long long na = max(a_hi - a_lo, 0LL), nb = max(b_hi - b_lo, 0LL);
  const long long ncand = na + nb;   // >= 1: the entry's block starts below T
  const size_t base = (size_t)b * (size_t)J.in_bs;
  const size_t rbase = (size_t)b * (size_t)J.r_bs;
  float* pm = smem;              // [TG][cs] running maxima
  float* ps = pm + TG * cs;      // [TG][cs] sums
  float* pa = ps + TG * cs;      // [TG][cs] weighted sums
  float* row = pa + TG * cs;     // [c]
  float* red = row + c;          // [16]

  // gamma of channel tid and of its RoPE partner, loaded with the candidates
  const float* __restrict__ gsrc = J.gamma ? J.gamma : k_ones.v;
  const int jc = min((int)threadIdx.x, c - 1);
  float gj[1] = {gsrc[jc]}, gp[1] = {gsrc[min(jc ^ 1, c - 1)]};

  const int tg = threadIdx.x / CV, cv = threadIdx.x % CV;
  if (tg < TG) {
    float mx[VEC], sum[VEC], acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      mx[e] = -INFINITY;
      sum[e] = 0.f;
      acc[e] = 0.f;
    }
    for (long long q0 = tg; q0 < ncand; q0 += (long long)TG * COMPX_TPT) {
      u32x4_t xc[COMPX_TPT], zc[COMPX_TPT];
      bool hz[COMPX_TPT];
#pragma unroll
      for (int u = 0; u < COMPX_TPT; ++u) {
        // unguarded loads (candidate clamped, a missing Z reads C); the extra ones unused
        const long long q = min(q0 + (long long)u * TG, ncand - 1);
        const bool in_a = q < na;
        const long long tok = in_a ? a_lo + q : b_lo + (q - na);
        // a token before the appended ones comes from the ring (append mode only)
        const bool from_ring = tok < tbase;
        const size_t off = (from_ring ? rbase + (size_t)(tok % J.in_ring) * (size_t)J.r_stride
                                      : base + (size_t)(tok - tbase) * (size_t)c) + (size_t)(c0 + cv * VEC);
        const char* Cp = (const char*)(from_ring ? (in_a ? J.rCa : J.rCb) : (in_a ? J.Ca : J.Cb)) + off * ESZ;
        const char* Zp0 = (const char*)(from_ring ? (in_a ? J.rZa : J.rZb) : (in_a ? J.Za : J.Zb));
        const char* Zp = Zp0 ? Zp0 + off * ESZ : nullptr;
        hz[u] = Zp != nullptr;
        xc[u] = *(const u32x4_t*)Cp;
        zc[u] = *(const u32x4_t*)(Zp ? Zp : Cp);
      }
      // the round's maximum first, then one rescale of the running sums
      float bm[VEC];
#pragma unroll
      for (int e = 0; e < VEC; ++e) bm[e] = mx[e];
#pragma unroll
      for (int u = 0; u < COMPX_TPT; ++u) {
        if (q0 + (long long)u * TG >= ncand) break;
        float z[VEC];
        unpack_piece<IDT>(zc[u], z);
#pragma unroll
        for (int e = 0; e < VEC; ++e) bm[e] = fmaxf(bm[e], hz[u] ? z[e] : 0.f);
      }
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float r = mx[e] == -INFINITY ? 0.f : __expf(mx[e] - bm[e]);
        sum[e] *= r;
        acc[e] *= r;
        mx[e] = bm[e];
      }
#pragma unroll
      for (int u = 0; u < COMPX_TPT; ++u) {
        if (q0 + (long long)u * TG >= ncand) break;
        float x[VEC], z[VEC];
        unpack_piece<IDT>(xc[u], x);
        unpack_piece<IDT>(zc[u], z);
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
          const float wgt = __expf((hz[u] ? z[e] : 0.f) - mx[e]);
          sum[e] += wgt;
          acc[e] += wgt * x[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      const int j = cv * VEC + e;
      pm[tg * cs + j] = mx[e];
      ps[tg * cs + j] = sum[e];
      pa[tg * cs + j] = acc[e];
    }
  }
  __syncthreads();

  // merge the TG partials of channel j = tid, in group order
  float ss = 0.f, v = 0.f;
  if ((int)threadIdx.x < cs) {
    const int j = threadIdx.x;
    float M = -INFINITY;
#pragma unroll 4
    for (int q = 0; q < TG; ++q) M = fmaxf(M, pm[q * cs + j]);
    float S = 0.f, A = 0.f;
#pragma unroll 4
    for (int q = 0; q < TG; ++q) {
      const float mq = pm[q * cs + j];
      const float f = mq == -INFINITY ? 0.f : __expf(mq - M);   // a group that saw no candidate adds 0
      S += ps[q * cs + j] * f;
      A += pa[q * cs + j] * f;
    }
    v = S > 0.f ? A / S : 0.f;
    ss = v * v;
  }
  if (ns == 1) {
    if ((int)threadIdx.x < c) row[threadIdx.x] = v;
    __syncthreads();   // row[] complete (the epilogue reads RoPE partners)
    compress_store<ODT, COMPX_THREADS>(J, s, b, row, ss, red, gj, gp);
    return;
  }
  // channel split: the slice's values and its sum of squares go to the
  // workspace (compress_finish_kernel adds the slices' sums in slice order).
  // Handing the row to a second kernel costs a launch; finishing it in the
  // last slice to arrive took device-scope fences, each a cache writeback that
  // cost more than the launch.
  const size_t slot = (size_t)b * (size_t)J.n_entries + (size_t)ent;
  if ((int)threadIdx.x < cs) J.ws_rows[slot * (size_t)c + c0 + threadIdx.x] = v;
  float w = ss;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) w += __shfl_xor(w, o, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = w;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int q = 0; q < (cs + 63) / 64; ++q) t += red[q];
    J.ws_ss[slot * (size_t)ns + slice] = t;
  }
}

// The rows of split entries: the pooled row from the workspace, the slices'
// sums of squares in slice order, then the RMSNorm / RoPE / store epilogue.
// One workgroup per (entry, sequence) of each split job (jobs on whole rows
// return at once).
template <int ODT>
__device__ __forceinline__ void compress_finish(const CompressJob& J, float* smem) {
  const int c = J.c, ns = J.ns, b = blockIdx.y;
  const long long ent = blockIdx.x;
  const long long s = J.s_begin + ent;
  if ((long long)J.m * s >= seq_tokens(J, b)) return;   // no such entry in this sequence (whole workgroup)
  if (J.out_rows > 0 && (J.out_ring > 0 ? s % J.out_ring : s) >= J.out_rows) return;
  float* row = smem;       // [c]
  float* red = row + c;    // [16]
  const size_t slot = (size_t)b * (size_t)J.n_entries + (size_t)ent;
  const float* __restrict__ gsrc = J.gamma ? J.gamma : k_ones.v;
  const int jc = min((int)threadIdx.x, c - 1);
  float gj[1] = {gsrc[jc]}, gp[1] = {gsrc[min(jc ^ 1, c - 1)]};
  if ((int)threadIdx.x < c) row[threadIdx.x] = J.ws_rows[slot * (size_t)c + threadIdx.x];
  float tot = 0.f;
  if (threadIdx.x == 0)
    for (int q = 0; q < ns; ++q) tot += J.ws_ss[slot * (size_t)ns + q];
  __syncthreads();
  compress_store<ODT, COMPX_THREADS>(J, s, b, row, tot, red, gj, gp);
}

__global__ __launch_bounds__(COMPX_THREADS) void compress_wide_kernel(const CompressBatch jb) {
  extern __shared__ float smem[];
  // the job is read where it lies, in the kernel-argument segment (jb is the only
  // argument, at offset 0): indexing the by-value batch with blockIdx.z made the
  // compiler copy all of it to scratch memory first
  (void)jb;
  const CompressJob& J = ((const CompressBatch*)__builtin_amdgcn_kernarg_segment_ptr())->job[blockIdx.z];
  if ((long long)blockIdx.x >= J.n_entries * J.ns || (int)blockIdx.y >= J.B) return;
  switch (J.in_dtype * 5 + J.out_dtype) {
    case DT_F32 * 5 + DT_F32: compress_entry_wide<DT_F32, DT_F32>(J, smem); break;
    case DT_F32 * 5 + DT_BF16: compress_entry_wide<DT_F32, DT_BF16>(J, smem); break;
    case DT_F32 * 5 + DT_FP8: compress_entry_wide<DT_F32, DT_FP8>(J, smem); break;
    case DT_F32 * 5 + DT_MX4: compress_entry_wide<DT_F32, DT_MX4>(J, smem); break;
    case DT_F32 * 5 + DT_MIX: compress_entry_wide<DT_F32, DT_MIX>(J, smem); break;
    case DT_BF16 * 5 + DT_F32: compress_entry_wide<DT_BF16, DT_F32>(J, smem); break;
    case DT_BF16 * 5 + DT_BF16: compress_entry_wide<DT_BF16, DT_BF16>(J, smem); break;
    case DT_BF16 * 5 + DT_FP8: compress_entry_wide<DT_BF16, DT_FP8>(J, smem); break;
    case DT_BF16 * 5 + DT_MX4: compress_entry_wide<DT_BF16, DT_MX4>(J, smem); break;
    default: compress_entry_wide<DT_BF16, DT_MIX>(J, smem); break;
  }
}

__global__ __launch_bounds__(COMPX_THREADS) void compress_finish_kernel(const CompressBatch jb) {
  extern __shared__ float smem[];
  (void)jb;
  const CompressJob& J = ((const CompressBatch*)__builtin_amdgcn_kernarg_segment_ptr())->job[blockIdx.z];
  if (J.ns == 1 || (long long)blockIdx.x >= J.n_entries || (int)blockIdx.y >= J.B) return;
  switch (J.out_dtype) {
    case DT_F32: compress_finish<DT_F32>(J, smem); break;
    case DT_BF16: compress_finish<DT_BF16>(J, smem); break;
    case DT_FP8: compress_finish<DT_FP8>(J, smem); break;
    case DT_MX4: compress_finish<DT_MX4>(J, smem); break;
    default: compress_finish<DT_MIX>(J, smem); break;
  }
}

static size_t compress_lds_bytes(int G, int c) {
  return (size_t)(3 * G * c + c + COMP_THREADS / 64) * sizeof(float);
}

CompressJob make_compress_job(const CompressArgs& x, int G) {
  CompressJob J{};
  J.Ca = x.C_a; J.Za = x.Z_a; J.Cb = x.C_b; J.Zb = x.Z_b;
  J.gamma = x.gamma; J.T_len = x.T_len; J.E = x.E; J.E_scale = x.E_scale;
  J.in_bs = x.in_bs; J.tok_base = x.tok_base; J.T = x.T; J.s_begin = x.s_begin;
  J.n_entries = x.s_end - x.s_begin;
  J.pos_stride = x.pos_stride; J.pos_offset = x.pos_offset;
  J.out_bs = x.out_bs; J.out_ring = x.out_ring;
  J.rope = rope_ratio(x.rope_dim, x.rope_base);
  J.eps = x.eps;
  J.in_dtype = x.in_dtype; J.out_dtype = x.out_dtype;
  J.B = x.B; J.c = x.c; J.m = x.m; J.overlap = x.overlap; J.G = G; J.rope_dim = x.rope_dim;
  J.ns = 1;
  return J;
}

// a job for the wave-per-entry kernel: few candidates per entry, whole 16-byte pieces
static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
// every input row starts 16-byte aligned (16-byte pieces of the channel axis)
static bool inputs_in_pieces(const CompressArgs& x) {
  const int vec = x.in_dtype == DT_F32 ? 4 : 8;
  return x.c % vec == 0 && aligned16(x.C_a) && (!x.C_b || aligned16(x.C_b)) && (!x.Z_a || aligned16(x.Z_a)) &&
         (!x.Z_b || aligned16(x.Z_b)) && (x.in_bs * (x.in_dtype == DT_F32 ? 4 : 2)) % 16 == 0;
}
// a job for the wide kernel: rows in 16-byte pieces (the choice depends on the
// job alone, so a job gives the same bytes in any batch)
static bool wide_job(const CompressArgs& x) { return x.c <= 1024 && inputs_in_pieces(x); }
// token groups of a wide job: enough for its candidates, at most COMPX_MAXTG
static int wide_groups(int c, int vec, int ncand_max) {
  return std::max(1, std::min(std::min(COMPX_THREADS / (c / vec), COMPX_MAXTG), ncand_max));
}
static bool wave_job(const CompressArgs& x);

// Channel slices of a wide job on the split path: entries of many candidates
// (HCA blocks) in a launch of few workgroups, where one workgroup per entry is
// bound by its own ALU work (every candidate's exponentials); 64-channel slices
// spread it over c / 64 workgroups.  1: whole rows.
static constexpr int COMPX_SLICE = 64;
static constexpr int COMPX_SPLIT_MAXTG = 32;     // token groups of a slice
static constexpr long long COMPX_SPLIT_ITEMS = 256;   // (sequence, entry) pairs at most
static int split_slices(const CompressArgs& x) {
  const int ncand_max = x.overlap ? 2 * x.m : x.m;
  const long long items = (long long)x.B * (x.s_end - x.s_begin);
  if (ncand_max < 64 || x.c % COMPX_SLICE != 0 || x.c < 2 * COMPX_SLICE || items > COMPX_SPLIT_ITEMS) return 1;
  return x.c / COMPX_SLICE;
}
static size_t ws_align(size_t x) { return (x + 255) / 256 * 256; }
size_t compress_workspace_bytes(const CompressArgs* a, int n_jobs) {
  size_t ss = 0, rows = 0;
  for (int q = 0; q < n_jobs; ++q) {
    const CompressArgs& x = a[q];
    if (wave_job(x) || !wide_job(x)) continue;
    const int ns = split_slices(x);
    if (ns == 1) continue;
    const size_t slots = (size_t)x.B * (size_t)(x.s_end - x.s_begin);
    ss += slots * ns;
    rows += slots * x.c;
  }
  if (ss == 0) return 0;
  return ws_align(ss * 4) + rows * 4;
}

bool compress_wave_ok(const CompressArgs& x, bool mx4_out, bool mix_out) {
  const int ncand_max = x.overlap ? 2 * x.m : x.m;
  const int vec = x.in_dtype == DT_F32 ? 4 : 8;
  // 16-byte pieces: every input row and (for bf16 output) every output row starts 16-byte aligned
  const bool in_al = inputs_in_pieces(x);
  // (MXFP4 and mixed output take the other kernels: another store format in the
  // wave kernel spilled registers; the decode front instantiates MXFP4 output
  // for bf16 inputs, whose 32-channel blocks are four whole pieces, stored as
  // 4-byte words)
  const bool mx4 = mx4_out && x.out_dtype == DT_MX4 && x.in_dtype == DT_BF16 && x.c % 32 == 0 &&
                   (((uintptr_t)x.E) & 3u) == 0 && x.out_bs % 8 == 0;
  // mixed rows of c + rope_dim bytes whose pieces stay whole: 8-byte code words,
  // 16-byte bf16 words
  const bool mix = mix_out && x.out_dtype == DT_MIX && x.in_dtype == DT_BF16 && x.rope_dim % 8 == 0 &&
                   aligned16(x.E) && (x.c + x.rope_dim) % 16 == 0 && (x.c - x.rope_dim) % 16 == 0;
  const bool out_al = (x.out_dtype != DT_BF16 || (aligned16(x.E) && x.out_bs % 8 == 0)) &&
                      (x.out_dtype != DT_MX4 || mx4) && (x.out_dtype != DT_MIX || mix);
  return ncand_max <= COMPW_MAXC && x.c % 8 == 0 && x.c <= 64 * COMPW_MAXP * vec &&
         x.rope_dim <= COMPW_MAXR && in_al && out_al;
}
static bool wave_job(const CompressArgs& x) {
  // a job of a few dozen entries (decode) is pure latency, where one workgroup per
  // entry is quicker; many entries (prefill) are throughput, where a wave each is
  const long long items = (long long)x.B * (x.s_end - x.s_begin);
  return items >= COMPW_MIN_ITEMS && compress_wave_ok(x);
}

int launch_compress(const CompressArgs* a, int n_jobs, hipStream_t st, void* ws, size_t ws_bytes) {
  if (n_jobs < 1 || n_jobs > COMP_MAX_JOBS) return -1;
  // jobs with few candidates per entry: one wave per entry, all in one launch
  CompressWaveBatch wb{};
  int nw = 0;
  for (int q = 0; q < n_jobs; ++q) {
    if (!wave_job(a[q])) continue;
    wb.job[nw] = make_compress_job(a[q], 1);
    wb.first[nw + 1] = wb.first[nw] + (long long)a[q].B * wb.job[nw].n_entries;
    ++nw;
  }
  if (nw > 0) {
    wb.n_jobs = nw;
    const long long blocks = (wb.first[nw] + COMPW_WAVES - 1) / COMPW_WAVES;
    if (blocks > 2147483647LL) return -1;
    hipLaunchKernelGGL(compress_wave_kernel<COMPW_MAXC>, dim3((unsigned)blocks), dim3(64 * COMPW_WAVES), 0,
                       st, wb);
  }
  // jobs whose rows come in 16-byte pieces: one 1024-thread workgroup per entry
  auto to_wide = [&](const CompressArgs& x) { return !wave_job(x) && wide_job(x); };
  {
    CompressBatch xb{};
    size_t lds = 0;
    long long gx = 1;
    int gy = 1;
    int nx = 0;
    // the split path's workspace: slice sums, then rows (compress_workspace_bytes)
    const size_t need = compress_workspace_bytes(a, n_jobs);
    const bool split = ws != nullptr && need > 0 && ws_bytes >= need;
    size_t o_rows = 0;
    if (split) {
      size_t ss = 0;
      for (int q = 0; q < n_jobs; ++q)
        if (to_wide(a[q]) && split_slices(a[q]) > 1)
          ss += (size_t)a[q].B * (size_t)(a[q].s_end - a[q].s_begin) * split_slices(a[q]);
      o_rows = ws_align(ss * 4);
    }
    size_t u_ss = 0, u_rows = 0;   // workspace elements taken so far
    long long fx = 0;              // entries of the largest split job
    size_t flds = 0;
    for (int q = 0; q < n_jobs; ++q) {
      if (!to_wide(a[q])) continue;
      const CompressArgs& x = a[q];
      const int vec = x.in_dtype == DT_F32 ? 4 : 8;
      const int ns = split ? split_slices(x) : 1;
      const int cs = x.c / ns;
      const int ncand_max = x.overlap ? 2 * x.m : x.m;
      const int TG = ns == 1 ? wide_groups(x.c, vec, ncand_max)
                             : std::max(1, std::min(std::min(COMPX_THREADS / (cs / vec), COMPX_SPLIT_MAXTG), ncand_max));
      xb.job[nx] = make_compress_job(x, TG);
      if (ns > 1) {
        const size_t slots = (size_t)x.B * (size_t)(x.s_end - x.s_begin);
        xb.job[nx].ns = ns;
        xb.job[nx].ws_ss = (float*)ws + u_ss;
        xb.job[nx].ws_rows = (float*)((char*)ws + o_rows) + u_rows;
        u_ss += slots * ns;
        u_rows += slots * x.c;
        fx = std::max(fx, xb.job[nx].n_entries);
        flds = std::max(flds, (size_t)(x.c + 16) * sizeof(float));
      }
      const size_t l = (size_t)(3 * TG * cs + x.c + 16) * sizeof(float);
      if (l > lds) lds = l;
      if (xb.job[nx].n_entries * ns > gx) gx = xb.job[nx].n_entries * ns;
      if (x.B > gy) gy = x.B;
      ++nx;
    }
    if (nx > 0) {
      if (gx > 2147483647LL || gy > 65535) return -1;
      if (lds > 65536 && hipFuncSetAttribute((const void*)compress_wide_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)lds) != hipSuccess)
        return -1;
      hipLaunchKernelGGL(compress_wide_kernel, dim3((unsigned)gx, (unsigned)gy, (unsigned)nx),
                         dim3(COMPX_THREADS), lds, st, xb);
      if (fx > 0)
        hipLaunchKernelGGL(compress_finish_kernel, dim3((unsigned)fx, (unsigned)gy, (unsigned)nx),
                           dim3(COMPX_THREADS), flds, st, xb);
    }
    if (nw + nx == n_jobs) return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  // the rest (rows not in 16-byte pieces): one 512-thread workgroup per entry
  CompressBatch jb{};
  size_t lds = 0;
  long long gx = 1;
  int gy = 1;
  int nb = 0;
  for (int q0 = 0; q0 < n_jobs; ++q0) {
    if (wave_job(a[q0]) || to_wide(a[q0])) continue;
    const int q = nb++;
    const CompressArgs& x = a[q0];
    const int ncand_max = x.overlap ? 2 * x.m : x.m;
    int G = ncand_max < COMP_MAX_G ? ncand_max : COMP_MAX_G;
    if (G < 1) G = 1;
    CompressJob& J = jb.job[q];
    J = make_compress_job(x, G);
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
  hipLaunchKernelGGL(compress_kernel, dim3((unsigned)gx, (unsigned)gy, (unsigned)nb),
                     dim3(COMP_THREADS), lds, st, jb);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

// ---------------------------------------------------------------------------
// Cache append (heterogeneous cache, method page section 3.5): the new tokens'
// window rows into the sliding-window ring, every CSA entry, indexer key and
// HCA entry whose block completes, then the new tokens' raw candidate rows
// into the tail ring of lcm(m, m') slots that the next append reads.
// ---------------------------------------------------------------------------
struct TailCopy {
  const uint16_t* src[10];   // Ca, Za, Cb, Zb, ICa, IZa, ICb, IZb, Ch, Zh: [B][n_new][width]
  int width[10], off[10];    // row width and offset within a tail slot (elements)
};

// block (u, b): the u-th of the last min(n_new, ring) new tokens of sequence b
__global__ __launch_bounds__(256) void tail_copy_kernel(const TailCopy tc, const int* __restrict__ T0,
                                                        uint16_t* __restrict__ tail, int n_new, int n_copy,
                                                        int ring, int TR) {
  const int b = blockIdx.y;
  const int r = n_new - n_copy + blockIdx.x;   // row among the new tokens
  const long long t = (long long)T0[b] + r;
  uint16_t* dst = tail + ((size_t)b * ring + (size_t)(t % ring)) * TR;
  for (int p = threadIdx.x; p < TR / 8; p += 256) {
    const int e = 8 * p;
    int k = 0;
#pragma unroll
    for (int q = 1; q < 10; ++q) k = e >= tc.off[q] ? q : k;
    const int w = tc.width[k];
    const uint16_t* src = tc.src[k] + ((size_t)b * n_new + r) * (size_t)w + (e - tc.off[k]);
    *(u32x4_t*)(dst + e) = *(const u32x4_t*)src;
  }
}

int launch_cache_append(const CacheAppendArgs& a, hipStream_t st) {
  const int c = a.c, dI = a.d_I, R = a.ring, TR = 6 * c + 4 * dI;
  const uint16_t* tail = (const uint16_t*)a.tail;
  auto job = [&](const void* Ca, const void* Za, const void* Cb, const void* Zb, int width, int m, int overlap,
                 const uint16_t* rCa, const uint16_t* rZa, const uint16_t* rCb, const uint16_t* rZb,
                 const float* gamma, int rope_dim, void* E, int out_dtype, float* E_scale, long long rows,
                 long long out_ring, long long s_begin, long long n_entries) {
    CompressArgs x{};
    x.C_a = Ca; x.Z_a = Za; x.C_b = Cb; x.Z_b = Zb; x.in_dtype = DT_BF16; x.B = a.B;
    x.R = a.n_new; x.in_bs = (long long)a.n_new * width; x.tok_base = 0; x.T = 1; x.T_len = nullptr;
    x.c = width; x.m = m; x.overlap = overlap; x.s_begin = 0; x.s_end = n_entries;
    x.gamma = gamma; x.eps = a.eps; x.rope_dim = rope_dim; x.rope_base = a.rope_base;
    x.pos_stride = m; x.pos_offset = 0; x.E = E; x.out_dtype = out_dtype; x.E_scale = E_scale;
    x.out_bs = rows * width; x.out_ring = out_ring;
    const int vec = 8;
    CompressJob J = make_compress_job(x, wide_groups(width, vec, overlap ? 2 * m : m));
    J.T0 = a.T0;
    J.n_new = a.n_new;
    J.s_begin = s_begin;
    J.rCa = rCa; J.rZa = rZa; J.rCb = rCb; J.rZb = rZb;
    J.r_stride = TR;
    J.r_bs = (long long)R * TR;
    J.in_ring = R;
    J.out_rows = out_ring > 0 ? 0 : rows;
    return J;
  };
  CompressBatch xb{};
  const long long n_win_rows = std::min<long long>(a.n_new, a.W_cap);
  xb.job[0] = job(a.Wraw, nullptr, nullptr, nullptr, c, 1, 0, nullptr, nullptr, nullptr, nullptr, a.gamma,
                  a.rope_dim, a.W, DT_BF16, nullptr, a.W_cap, a.W_cap, a.n_new - n_win_rows, n_win_rows);
  xb.job[1] = job(a.Ca, a.Za, a.Cb, a.Zb, c, a.m, 1, tail, tail + c, tail + 2 * c, tail + 3 * c, a.gamma,
                  a.rope_dim, a.E_csa, DT_BF16, nullptr, a.N_csa, 0, 0, a.n_new / a.m + 1);
  xb.job[2] = job(a.ICa, a.IZa, a.ICb, a.IZb, dI, a.m, 1, tail + 4 * c, tail + 4 * c + dI, tail + 4 * c + 2 * dI,
                  tail + 4 * c + 3 * dI, nullptr, 0, a.K_idx, a.k_dtype, (float*)a.K_scale, a.N_csa, 0, 0,
                  a.n_new / a.m + 1);
  xb.job[3] = job(a.Ch, a.Zh, nullptr, nullptr, c, a.m_hca, 0, tail + 4 * c + 4 * dI, tail + 5 * c + 4 * dI,
                  nullptr, nullptr, a.gamma, a.rope_dim, a.E_hca, DT_BF16, nullptr, a.N_hca, 0, 0,
                  a.n_new / a.m_hca + 1);
  // (window rows: pos_stride 1)
  xb.job[0].pos_stride = 1;
  long long gx = 1;
  size_t lds = 0;
  for (int q = 0; q < 4; ++q) {
    gx = std::max(gx, xb.job[q].n_entries);
    const int TG = xb.job[q].G;
    lds = std::max(lds, (size_t)(3 * TG * xb.job[q].c + xb.job[q].c + 16) * sizeof(float));
  }
  if (gx > 2147483647LL || a.B > 65535) return -1;
  if (lds > 65536 && hipFuncSetAttribute((const void*)compress_wide_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess)
    return -1;
  hipLaunchKernelGGL(compress_wide_kernel, dim3((unsigned)gx, (unsigned)a.B, 4u), dim3(COMPX_THREADS), lds, st,
                     xb);
  // the tail ring, after the compressions have read it
  TailCopy tc{};
  const void* src[10] = {a.Ca, a.Za, a.Cb, a.Zb, a.ICa, a.IZa, a.ICb, a.IZb, a.Ch, a.Zh};
  const int wid[10] = {c, c, c, c, dI, dI, dI, dI, c, c};
  int off = 0;
  for (int q = 0; q < 10; ++q) {
    tc.src[q] = (const uint16_t*)src[q];
    tc.width[q] = wid[q];
    tc.off[q] = off;
    off += wid[q];
  }
  const int n_copy = std::min(a.n_new, R);
  hipLaunchKernelGGL(tail_copy_kernel, dim3((unsigned)n_copy, (unsigned)a.B), dim3(256), 0, st, tc, a.T0,
                     (uint16_t*)a.tail, a.n_new, n_copy, R, TR);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
