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
// job's dtypes are chosen at run time (uniform per workgroup).  Jobs of many
// entries (256 or more (sequence, entry) pairs, as in prefill) with at most 8
// candidates per entry (CSA m = 4, window rows) take the wave-per-entry kernel
// below instead: no LDS, no barriers.  The choice depends on the job alone, so
// a job gives the same result in any batch.
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

// ---------------------------------------------------------------------------
// Wave-per-entry kernel: jobs whose entries have at most MAXC candidates (CSA
// with m <= MAXC / 2, window rows with m = 1) and c % 8 == 0.  One wave pools
// one (entry, sequence) of one job; a workgroup holds COMPW_WAVES of them.  A
// lane takes 16-byte pieces of the channel axis (8 bf16 or 4 fp32 channels):
// all candidate pieces of a lane are loaded at once, the softmax over the
// candidates runs in registers, and the RMSNorm sum and the fp8 row maximum are
// wave reductions (DPP and row swaps), so there is no LDS and no barrier.  A
// RoPE pair (2u, 2u + 1) lies inside one piece.
// ---------------------------------------------------------------------------
static constexpr int COMPW_WAVES = 4;   // entries per workgroup
static constexpr int COMPW_MAXP = 2;    // 16-byte pieces per lane: c <= 128 VEC
static constexpr int COMPW_MAXR = 128;  // rotated dims (one (cos, sin) per lane and half)
static constexpr int COMPW_MAXC = 8;    // candidates per entry (CSA m <= 4, window rows)
static constexpr long long COMPW_MIN_ITEMS = 256;   // (sequence, entry) pairs of a job

struct CompressWaveBatch {
  CompressJob job[COMP_MAX_JOBS];
  long long first[COMP_MAX_JOBS + 1];   // first item of each job (items: sequences x entries)
  int n_jobs;
};

template <int IDT>
__device__ __forceinline__ void unpack_piece(const u32x4_t v, float (&o)[IDT == DT_F32 ? 4 : 8]) {
  if constexpr (IDT == DT_F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) o[e] = __uint_as_float(v[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o[2 * e] = __uint_as_float(v[e] << 16);
      o[2 * e + 1] = __uint_as_float(v[e] & 0xffff0000u);
    }
  }
}

template <int IDT, int ODT, int MAXC>
__device__ __forceinline__ void compress_entry_wave(const CompressJob& J, long long s, int b, int lane) {
  constexpr int VEC = IDT == DT_F32 ? 4 : 8;   // channels per 16-byte piece
  constexpr int ESZ = IDT == DT_F32 ? 4 : 2;
  const int c = J.c, m = J.m;
  const long long a_lo = (long long)m * s, a_hi = min((long long)m * (s + 1), J.T);
  long long b_lo = 0, b_hi = 0;
  if (J.overlap) {
    b_lo = max((long long)m * (s - 1), 0LL);
    b_hi = min((long long)m * s, J.T);
  }
  const int na = (int)max(a_hi - a_lo, 0LL), nb = (int)max(b_hi - b_lo, 0LL);
  const int ncand = na + nb;   // <= MAXC (host), >= 1 (an entry < ceil(T / m) has a token)
  const size_t base = (size_t)b * (size_t)J.in_bs;
  const int npieces = c / VEC;
  const float* __restrict__ gsrc = J.gamma ? J.gamma : k_ones.v;

  float pooled[COMPW_MAXP][VEC];
  float ss = 0.f;
#pragma unroll
  for (int pi = 0; pi < COMPW_MAXP; ++pi) {
    if (64 * pi >= npieces) break;   // uniform
    const int piece = min(lane + 64 * pi, npieces - 1);   // clamped: extra lanes redo the last piece
    u32x4_t xc[MAXC], zc[MAXC];
    bool hz[MAXC];   // the candidate's set has logits (a missing Z means logits 0)
#pragma unroll
    for (int q = 0; q < MAXC; ++q) {
      const int qc = min(q, ncand - 1);   // unguarded loads, the extra ones unused
      const bool in_a = qc < na;
      const long long tok = in_a ? a_lo + qc : b_lo + (qc - na);
      const size_t off = (base + (size_t)(tok - J.tok_base) * (size_t)c + (size_t)piece * VEC) * ESZ;
      const char* Cp = (const char*)(in_a ? J.Ca : J.Cb);
      const char* Zp = (const char*)(in_a ? J.Za : J.Zb);
      hz[q] = Zp != nullptr;
      xc[q] = *(const u32x4_t*)(Cp + off);
      zc[q] = *(const u32x4_t*)((Zp ? Zp : Cp) + off);
    }
    float mx[VEC], sum[VEC], acc[VEC];
#pragma unroll
    for (int e = 0; e < VEC; ++e) mx[e] = -INFINITY;
#pragma unroll
    for (int q = 0; q < MAXC; ++q) {
      if (q >= ncand) break;
      float z[VEC];
      unpack_piece<IDT>(zc[q], z);
#pragma unroll
      for (int e = 0; e < VEC; ++e) mx[e] = fmaxf(mx[e], hz[q] ? z[e] : 0.f);
    }
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      sum[e] = 0.f;
      acc[e] = 0.f;
    }
#pragma unroll
    for (int q = 0; q < MAXC; ++q) {
      if (q >= ncand) break;
      float x[VEC], z[VEC];
      unpack_piece<IDT>(xc[q], x);
      unpack_piece<IDT>(zc[q], z);
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float w = __expf((hz[q] ? z[e] : 0.f) - mx[e]);
        sum[e] += w;
        acc[e] += w * x[e];
      }
    }
    const bool live = lane + 64 * pi < npieces;
#pragma unroll
    for (int e = 0; e < VEC; ++e) {
      pooled[pi][e] = sum[e] > 0.f ? acc[e] / sum[e] : 0.f;
      ss += live ? pooled[pi][e] * pooled[pi][e] : 0.f;
    }
  }

  float rinv = 1.f;
  if (J.gamma) rinv = 1.f / sqrtf(wave_reduce_f<false>(ss) / (float)c + J.eps);

  const long long pos = J.pos_stride * s + J.pos_offset;
  const long long orow = J.out_ring > 0 ? (s % J.out_ring) : s;
  const size_t obase = (size_t)b * (size_t)J.out_bs + (size_t)orow * (size_t)c;
  const int rbeg = c - J.rope_dim;
  // the entry's RoPE table: lane l holds the (cos, sin) of pairs l and 64 + l
  float rcs[2], rsn[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    rcs[h] = 1.f;
    rsn[h] = 0.f;
    if (lane + 64 * h < J.rope_dim / 2) rope_cos_sin(pos, lane + 64 * h, J.rope, &rcs[h], &rsn[h]);
  }
  float amax = 0.f;
#pragma unroll
  for (int pi = 0; pi < COMPW_MAXP; ++pi) {
    if (64 * pi >= npieces) break;
    const int piece = min(lane + 64 * pi, npieces - 1);
    const int j0 = piece * VEC;
#pragma unroll
    for (int e = 0; e < VEC; e += 2) {
      const int j = j0 + e;
      float v0 = pooled[pi][e] * rinv * gsrc[j], v1 = pooled[pi][e + 1] * rinv * gsrc[j + 1];
      // every lane takes part in the exchange (pairs outside the rotated dims read pair 0)
      const int u = j >= rbeg ? (j - rbeg) >> 1 : 0;
      const float c0 = __shfl(rcs[0], u & 63, 64), c1 = __shfl(rcs[1], u & 63, 64);
      const float s0 = __shfl(rsn[0], u & 63, 64), s1 = __shfl(rsn[1], u & 63, 64);
      if (j >= rbeg) {
        const float cs = u < 64 ? c0 : c1, sn = u < 64 ? s0 : s1;
        const float r0 = v0 * cs - v1 * sn, r1 = v0 * sn + v1 * cs;
        v0 = r0;
        v1 = r1;
      }
      pooled[pi][e] = v0;
      pooled[pi][e + 1] = v1;
      if (lane + 64 * pi < npieces) amax = fmaxf(amax, fmaxf(fabsf(v0), fabsf(v1)));
    }
  }
  float scale = 1.f;
  if constexpr (ODT == DT_FP8) {
    const float am = wave_reduce_f<true>(amax);
    scale = am > 0.f ? am / 448.0f : 1.0f;
    if (lane == 0) J.E_scale[(size_t)b * (size_t)(J.out_bs / c) + (size_t)orow] = scale;
  }
#pragma unroll
  for (int pi = 0; pi < COMPW_MAXP; ++pi) {
    if (64 * pi >= npieces) break;
    if (lane + 64 * pi >= npieces) continue;
    const size_t o = obase + (size_t)(lane + 64 * pi) * VEC;
    if constexpr (ODT == DT_BF16 && VEC == 8) {
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pack_bf16x2(pooled[pi][2 * e], pooled[pi][2 * e + 1]);
      *(u32x4_t*)((uint16_t*)J.E + o) = w;
    } else if constexpr (ODT == DT_FP8) {
#pragma unroll
      for (int e = 0; e < VEC; ++e) ((uint8_t*)J.E)[o + e] = f32_to_e4m3(pooled[pi][e] / scale);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) store_from_f32<ODT>(J.E, o + e, pooled[pi][e]);
    }
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
  switch (J.in_dtype * 3 + J.out_dtype) {
    case DT_F32 * 3 + DT_F32: compress_entry_wave<DT_F32, DT_F32, MAXC>(J, s, b, lane); break;
    case DT_F32 * 3 + DT_BF16: compress_entry_wave<DT_F32, DT_BF16, MAXC>(J, s, b, lane); break;
    case DT_F32 * 3 + DT_FP8: compress_entry_wave<DT_F32, DT_FP8, MAXC>(J, s, b, lane); break;
    case DT_BF16 * 3 + DT_F32: compress_entry_wave<DT_BF16, DT_F32, MAXC>(J, s, b, lane); break;
    case DT_BF16 * 3 + DT_BF16: compress_entry_wave<DT_BF16, DT_BF16, MAXC>(J, s, b, lane); break;
    default: compress_entry_wave<DT_BF16, DT_FP8, MAXC>(J, s, b, lane); break;
  }
}

static size_t compress_lds_bytes(int G, int c) {
  return (size_t)(3 * G * c + c + COMP_THREADS / 64) * sizeof(float);
}

static CompressJob make_job(const CompressArgs& x, int G) {
  CompressJob J{};
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
  return J;
}

// a job for the wave-per-entry kernel: few candidates per entry, whole 16-byte pieces
static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool wave_job(const CompressArgs& x) {
  const int ncand_max = x.overlap ? 2 * x.m : x.m;
  const int vec = x.in_dtype == DT_F32 ? 4 : 8;
  // 16-byte pieces: every input row and (for bf16 output) every output row starts 16-byte aligned
  const bool in_al = aligned16(x.C_a) && (!x.C_b || aligned16(x.C_b)) && (!x.Z_a || aligned16(x.Z_a)) &&
                     (!x.Z_b || aligned16(x.Z_b)) && (x.in_bs * (x.in_dtype == DT_F32 ? 4 : 2)) % 16 == 0;
  const bool out_al = x.out_dtype != DT_BF16 || (aligned16(x.E) && x.out_bs % 8 == 0);
  // a job of a few dozen entries (decode) is pure latency, where one workgroup per
  // entry is quicker; many entries (prefill) are throughput, where a wave each is
  const long long items = (long long)x.B * (x.s_end - x.s_begin);
  return items >= COMPW_MIN_ITEMS && ncand_max <= COMPW_MAXC && x.c % 8 == 0 &&
         x.c <= 64 * COMPW_MAXP * vec && x.rope_dim <= COMPW_MAXR && in_al && out_al;
}

int launch_compress(const CompressArgs* a, int n_jobs, hipStream_t st) {
  if (n_jobs < 1 || n_jobs > COMP_MAX_JOBS) return -1;
  // jobs with few candidates per entry: one wave per entry, all in one launch
  CompressWaveBatch wb{};
  int nw = 0;
  for (int q = 0; q < n_jobs; ++q) {
    if (!wave_job(a[q])) continue;
    wb.job[nw] = make_job(a[q], 1);
    wb.first[nw + 1] = wb.first[nw] + (long long)a[q].B * wb.job[nw].n_entries;
    ++nw;
  }
  if (nw > 0) {
    wb.n_jobs = nw;
    const long long blocks = (wb.first[nw] + COMPW_WAVES - 1) / COMPW_WAVES;
    if (blocks > 2147483647LL) return -1;
    hipLaunchKernelGGL(compress_wave_kernel<COMPW_MAXC>, dim3((unsigned)blocks), dim3(64 * COMPW_WAVES), 0,
                       st, wb);
    if (nw == n_jobs) return hipGetLastError() == hipSuccess ? 0 : -1;
  }
  // the rest (HCA blocks of many candidates): one workgroup per entry
  CompressBatch jb{};
  size_t lds = 0;
  long long gx = 1;
  int gy = 1;
  int nb = 0;
  for (int q0 = 0; q0 < n_jobs; ++q0) {
    if (wave_job(a[q0])) continue;
    const int q = nb++;
    const CompressArgs& x = a[q0];
    const int ncand_max = x.overlap ? 2 * x.m : x.m;
    int G = ncand_max < COMP_MAX_G ? ncand_max : COMP_MAX_G;
    if (G < 1) G = 1;
    CompressJob& J = jb.job[q];
    J = make_job(x, G);
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

}  // namespace csa
