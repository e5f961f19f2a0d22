// Wave-per-entry compressor: the job record the compress kernels read, and
// the device code that pools one (entry, sequence) of a job in one wave.
// Shared by the compressor's own kernels and by the decode-step front launch
// (index_score.hip), which runs the same arithmetic beside the indexer.
// DeepSeek-V4 method page, section 3.3 (softmax pooling of 2m overlapping
// candidates, RMSNorm and partial RoPE of each entry).
#pragma once

#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

static constexpr int COMP_MAX_JOBS = 8;   // jobs of one launch

// one job's arguments as the kernel reads them (validated on the host)
struct CompressJob {
  const void *Ca, *Za, *Cb, *Zb;
  const float* gamma;
  const int* T_len;   // per-sequence token counts (<= T), or NULL
  void* E;
  float* E_scale;
  long long in_bs, tok_base, T, s_begin, n_entries, pos_stride, pos_offset, out_bs, out_ring;
  RopeRatio rope;
  float eps;
  int in_dtype, out_dtype, B, c, m, overlap, G, rope_dim;
  // append mode (wide kernel only): T0[b] tokens were present before, n_new
  // arrive (rows of token T0[b] + r at row r of the inputs); entries whose
  // blocks complete are s = floor(T0[b] / m) + s_begin + blockIdx.x, those
  // with m (s + 1) <= T0[b] + n_new; candidates of earlier tokens are read from a ring of in_ring
  // token slots (token t at slot t mod in_ring, slot stride r_stride, batch
  // stride r_bs elements); output rows at or past out_rows are skipped
  const int* T0;
  const void *rCa, *rZa, *rCb, *rZb;
  long long n_new, r_stride, r_bs, out_rows;
  int in_ring;
  // channel split (wide kernel): ns workgroups per entry, each pooling c / ns
  // channels into slot b * n_entries + entry of the workspace arrays: the
  // entry's pooled row (ws_rows, c floats) and the slices' sums of squares
  // (ws_ss, ns floats); compress_finish_kernel then normalises and stores
  int ns;
  float *ws_ss, *ws_rows;
};

// tokens present in sequence b: T, or T_len[b] clamped to [0, T]
__device__ __forceinline__ long long seq_tokens(const CompressJob& J, int b) {
  return J.T_len ? min(J.T, max(0LL, (long long)J.T_len[b])) : J.T;
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
  const long long T = seq_tokens(J, b);
  if ((long long)m * s >= T) return;   // no such entry in this sequence (whole wave)
  const long long a_lo = (long long)m * s, a_hi = min((long long)m * (s + 1), T);
  long long b_lo = 0, b_hi = 0;
  if (J.overlap) {
    b_lo = max((long long)m * (s - 1), 0LL);
    b_hi = min((long long)m * s, T);
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
      // (mixed rows: the maximum of the fp8 part only)
      if (lane + 64 * pi < npieces && (ODT != DT_MIX || j < rbeg)) amax = fmaxf(amax, fmaxf(fabsf(v0), fabsf(v1)));
    }
  }
  float scale = 1.f;
  if constexpr (ODT == DT_FP8 || ODT == DT_MIX) {
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
    } else if constexpr (ODT == DT_MIX) {
      // mixed row (c + rope_dim bytes): e4m3 codes of channels [0, rbeg) under
      // the row scale, then bf16 of the rotated channels; a piece lies wholly
      // on one side (rope_dim % 8 == 0).  Used by the decode front only.
      static_assert(VEC == 8, "mixed rows from bf16 pieces");
      const int j0 = (lane + 64 * pi) * VEC;
      uint8_t* rb = (uint8_t*)J.E + ((size_t)b * (size_t)(J.out_bs / c) + (size_t)orow) * (size_t)(c + J.rope_dim);
      if (j0 < rbeg) {
        u32x2_t w2 = {0u, 0u};
#pragma unroll
        for (int e = 0; e < VEC; ++e) w2[e / 4] |= (uint32_t)f32_to_e4m3(pooled[pi][e] / scale) << (8 * (e % 4));
        *(u32x2_t*)(rb + j0) = w2;
      } else {
        u32x4_t w4;
#pragma unroll
        for (int e = 0; e < 4; ++e) w4[e] = pack_bf16x2(pooled[pi][2 * e], pooled[pi][2 * e + 1]);
        *(u32x4_t*)(rb + rbeg + 2 * (j0 - rbeg)) = w4;
      }
    } else if constexpr (ODT == DT_MX4) {
      // MXFP4 (OCP MX: E2M1 codes, one E8M0 scale per 32 channels): a block is
      // the 8-channel pieces of four consecutive lanes (c % 32 == 0, VEC = 8);
      // the block maximum by exchange within the four, the codes packed two per
      // byte (low nibble first), the block's first lane writes its scale byte.
      // Used by the decode front only (the wave kernel's other variants
      // would carry its registers).
      static_assert(VEC == 8, "MXFP4 output from bf16 pieces");
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < VEC; ++e) a = fmaxf(a, fabsf(pooled[pi][e]));
      a = fmaxf(a, __shfl_xor(a, 1, 64));
      a = fmaxf(a, __shfl_xor(a, 2, 64));
      const int se = mx4_shared_exp(a);
      uint32_t pk = 0;
#pragma unroll
      for (int e = 0; e < VEC; ++e) pk |= f32_to_e2m1(ldexpf(pooled[pi][e], -se)) << (4 * e);
      *(uint32_t*)((uint8_t*)J.E + o / 2) = pk;
      const int piece = lane + 64 * pi;
      if ((piece & 3) == 0)
        ((uint8_t*)J.E_scale)[((size_t)b * (size_t)(J.out_bs / c) + (size_t)orow) * (size_t)(c / 32) + piece / 4] =
            (uint8_t)(se + 127);
    } else {
#pragma unroll
      for (int e = 0; e < VEC; ++e) store_from_f32<ODT>(J.E, o + e, pooled[pi][e]);
    }
  }
}

// the job record of one compression (host): G token groups (wide kernel)
CompressJob make_compress_job(const CompressArgs& x, int G);
// true when the wave-per-entry arithmetic covers the job (any entry count);
// MXFP4 and mixed-row output only where the caller instantiates them (the
// decode front)
bool compress_wave_ok(const CompressArgs& x, bool mx4_out = false, bool mix_out = false);

}  // namespace csa
