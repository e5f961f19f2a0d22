// a4 / a5 — shared-KV multi-query attention over compressed entries, a sliding
// window and an attention sink, for gfx950.
//
// DeepSeek-V4 method page, section 3.3: core attention is MQA where each
// compressed entry is both key and value; RMSNorm on the query; partial RoPE
// on the last dims of query, entries and output, the output rotated again at
// position -i; a window of n_win uncompressed KV rows because a query cannot
// see its own block.  CSA attends to the top-k entries, HCA to every visible
// entry.  Report digest: learnable sink logits let a head's total attention
// weight fall below 1 (a sink adds e^sigma to the softmax denominator).
//
// Key slots of a query: slots [0, n_sel) are entries (idx[j] for CSA, j for
// HCA), slots [n_sel, n_sel + n_w) the window tokens i-n_w+1 .. i.
//
// Matrix-core kernel (bf16): a workgroup takes one query, 64 heads (16 per
// wave) and a contiguous range of key slots, staged 32 rows at a time in LDS.
//   S^T = KV . q^T  with v_mfma_f32_16x16x32_bf16, keys as M, heads as N, so a
//   lane ends with 4+4 key scores of ONE head: exactly the A operand layout of
//   P.V for that head (the contraction order over keys is permuted the same
//   way on both operands);
//   V is read transposed from row-major LDS with ds_read_b64_tr_b16;
//   an online softmax (running max / sum per head) rescales O per 32 keys.
// Decode queries split their slots across workgroups (fixed 128-slot ranges,
// independent of the batch) and a combine kernel merges the partial
// (max, sum, O) in a fixed order.
#include <type_traits>

#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

static constexpr int MQ_CH = 32;          // key rows per LDS chunk
static constexpr int MQ_SPLIT_KEYS = 128; // slots per workgroup when a query is split
static constexpr int MQ_SPLIT_BELOW_TQ = 16;
static constexpr int VALU_MAX_SLOTS = 8192;

struct QuerySlots {
  long long n_sel, n_w, win_lo, n_slots;
};

template <bool DENSE>
__device__ __forceinline__ QuerySlots query_slots(long long i, long long N_cap, int k, int m, int n_win) {
  QuerySlots s;
  s.n_sel = DENSE ? min(N_cap, (i + 1) / m) : (long long)k;
  s.n_w = min((long long)n_win, i + 1);
  s.win_lo = i - s.n_w + 1;
  s.n_slots = s.n_sel + s.n_w;
  return s;
}

// element offset of the row of a slot, or -1 for an empty slot
template <bool DENSE>
__device__ __forceinline__ long long slot_row(long long slot, const QuerySlots& qs,
                                              const int* __restrict__ idx_row, int b,
                                              long long N_cap, int W_cap, int d, bool* in_E) {
  if (slot < qs.n_sel) {
    long long e = DENSE ? slot : (long long)idx_row[slot];
    *in_E = true;
    if (e < 0 || e >= N_cap) return -1;
    return ((long long)b * N_cap + e) * d;
  }
  *in_E = false;
  const long long tau = qs.win_lo + (slot - qs.n_sel);
  return ((long long)b * W_cap + (tau % W_cap)) * d;
}

// Split partials in the workspace.  The output of (query row, split, head)
// divided by its softmax sum is a weighted mean of the value rows; it is stored
// times a power of two chosen from the row's own maximum magnitude (the
// maximum lands in [2^14, 2^15)), as the fp16 row part_o(ws)[((row * n_split +
// sp) * n_h + h) * D] (16-byte aligned rows).  The scaling is exact, so the row
// keeps 11 significant bits relative to its maximum whatever the magnitude of
// the values, and no finite input can saturate fp16.  The float records (max,
// sum, 1 / scale, 0) follow all rows, record u = (row * n_split + sp) * n_h + h
// at part_ml(...)[4 u].  n_units = (query rows) * n_split.
__device__ __forceinline__ _Float16* part_o(float* ws) { return (_Float16*)ws; }
__device__ __forceinline__ const _Float16* part_o(const float* ws) { return (const _Float16*)ws; }
__device__ __forceinline__ float* part_ml(float* ws, long long n_units, int n_h, int D) {
  return (float*)(part_o(ws) + (size_t)n_units * (size_t)n_h * (size_t)D);
}
__device__ __forceinline__ const float* part_ml(const float* ws, long long n_units, int n_h, int D) {
  return (const float*)(part_o(ws) + (size_t)n_units * (size_t)n_h * (size_t)D);
}
__device__ __forceinline__ _Float16 part_h(float x) {
  return (_Float16)fminf(fmaxf(x, -65504.f), 65504.f);   // a no-op once rows are scaled
}
// the power of two 2^(15 - k) for a row maximum amax = f 2^k (f in [0.5, 1)),
// exponent clamped to the normal range; 1 for a zero row
__device__ __forceinline__ float part_scale(float amax) {
  if (!(amax > 0.f)) return 1.f;
  const int k = (int)((__float_as_uint(amax) >> 23) & 0xff) - 126;
  const int e = min(max(15 - k + 127, 1), 254);
  return __uint_as_float((uint32_t)e << 23);
}
// 1 / part_scale (also a power of two, exact)
__device__ __forceinline__ float part_unscale(float sc) {
  const int e = (int)((__float_as_uint(sc) >> 23) & 0xff);
  return __uint_as_float((uint32_t)min(max(254 - e, 1), 254) << 23);
}
// 1 / l, or 0 for a split without visible keys (its O is 0)
__device__ __forceinline__ float part_inv(float l) { return l > 0.f ? 1.f / l : 0.f; }

// ---------------------------------------------------------------------------
// generic path (fp32 or bf16 storage): one workgroup per (query, head)
// ---------------------------------------------------------------------------
template <int DT, bool DENSE>
__global__ __launch_bounds__(256) void mqa_valu_kernel(
    const void* __restrict__ q, const float* __restrict__ gamma_q, float eps, const void* __restrict__ E,
    long long N_cap, const int* __restrict__ idx, int k, int m, const void* __restrict__ W, int W_cap,
    int n_win, const float* __restrict__ sink, const int* __restrict__ q_pos, int Tq, int n_h, int d,
    int rope_dim, RopeRatio rope, float scale, void* __restrict__ out) {
  extern __shared__ float sm[];
  float* qh = sm;                                  // [d]
  float* red = qh + d;                             // [4]
  float* pr = red + 4;                             // [VALU_MAX_SLOTS]
  long long* roff = (long long*)(pr + VALU_MAX_SLOTS);   // [VALU_MAX_SLOTS] (8-byte aligned: d, 4 even)
  const int h = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const size_t row = (size_t)b * Tq + t;
  const long long i = q_pos[row];
  const size_t qoff = (row * n_h + h) * (size_t)d;

  float ss = 0.f;
  for (int j = threadIdx.x; j < d; j += blockDim.x) {
    const float v = load_as_f32<DT>(q, qoff + j);
    qh[j] = v;
    ss += v * v;
  }
  const float rinv = 1.f / sqrtf(block_reduce<false>(ss, red) / (float)d + eps);
  for (int j = threadIdx.x; j < d; j += blockDim.x) qh[j] *= rinv * (gamma_q ? gamma_q[j] : 1.f);
  __syncthreads();
  for (int u = threadIdx.x; u < rope_dim / 2; u += blockDim.x) {
    const int j0 = d - rope_dim + 2 * u;
    float cs, sn;
    rope_cos_sin(i, u, rope, &cs, &sn);
    const float x0 = qh[j0], x1 = qh[j0 + 1];
    qh[j0] = x0 * cs - x1 * sn;
    qh[j0 + 1] = x0 * sn + x1 * cs;
  }
  __syncthreads();

  const QuerySlots qs = query_slots<DENSE>(i, N_cap, k, m, n_win);
  const int* idx_row = DENSE ? nullptr : idx + row * (size_t)k;
  float mx = -INFINITY;
  for (long long s = threadIdx.x; s < qs.n_slots; s += blockDim.x) {
    bool in_E;
    const long long off = slot_row<DENSE>(s, qs, idx_row, b, N_cap, W_cap, d, &in_E);
    roff[s] = in_E ? off : (off < 0 ? -1 : -2 - off);   // window rows encoded below -1
    float l = -INFINITY;
    if (off >= 0) {
      const void* base = in_E ? E : W;
      float dot = 0.f;
      for (int j = 0; j < d; ++j) dot += qh[j] * load_as_f32<DT>(base, (size_t)off + j);
      l = dot * scale;
    }
    pr[s] = l;
    mx = fmaxf(mx, l);
  }
  const float sig = sink ? sink[h] : -INFINITY;
  const float M = fmaxf(block_reduce<true>(mx, red), sig);
  float sum = 0.f;
  for (long long s = threadIdx.x; s < qs.n_slots; s += blockDim.x) {
    const float p = (pr[s] == -INFINITY) ? 0.f : __expf(pr[s] - M);
    pr[s] = p;
    sum += p;
  }
  float Z = block_reduce<false>(sum, red);
  if (sig != -INFINITY) Z += __expf(sig - M);
  const float inv = Z > 0.f ? 1.f / Z : 0.f;
  __syncthreads();

  for (int j = threadIdx.x; j < d; j += blockDim.x) {
    float o = 0.f;
    for (long long s = 0; s < qs.n_slots; ++s) {
      const long long ro = roff[s];
      if (ro == -1) continue;
      const float p = pr[s];
      o += p * (ro >= 0 ? load_as_f32<DT>(E, (size_t)ro + j) : load_as_f32<DT>(W, (size_t)(-2 - ro) + j));
    }
    qh[j] = o * inv;   // every thread finished reading qh before the barrier above
  }
  __syncthreads();
  for (int j = threadIdx.x; j < d; j += blockDim.x) {
    float v = qh[j];
    if (j >= d - rope_dim) {
      const int u = (j - (d - rope_dim)) >> 1;
      float cs, sn;
      rope_cos_sin(-i, u, rope, &cs, &sn);
      const float other = qh[j ^ 1];
      v = (j & 1) ? (other * sn + v * cs) : (v * cs - other * sn);
    }
    store_from_f32<DT>(out, qoff + j, v);
  }
}

// ---------------------------------------------------------------------------
// matrix-core path (bf16), D in {128, 256, 512}, n_h % 16 == 0
//
// Key slots are processed in groups of 128 held in LDS at once: all scores of
// the group first (the group maximum is then exact, so P needs no rescaling
// inside the group), then P.V.  Across groups (long slot lists, prefill) the
// reference maximum moves only when a group maximum exceeds it by more than 8
// (natural log units): P stays <= e^8 and O is rescaled rarely; the result is
// the same softmax, only the fp32 reference point differs.
//
// LDS layout: rows of D bf16, no padding; the 16-byte piece c of row r sits at
// piece position c ^ swz(r), swz(r) = ((r & 7) << 1) | ((r >> 3) & 1), which
// keeps the two read patterns conflict-free: 16 lanes reading the same piece
// of 16 consecutive rows (S^T operand) and 16 lanes reading two pieces of 4
// consecutive rows (transpose read of V).  Rows arrive with global_load_lds
// (16 bytes per lane; lane l fills piece position l of the wave's 1 KB window).
// ---------------------------------------------------------------------------
static constexpr int MQ_GROUP = 128;   // slots resident in LDS at once (4 chunks of 32)
static constexpr float MQ_REF_SLACK = 8.f;

__device__ __forceinline__ int mq_swz(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }

__device__ __forceinline__ uint32_t pack2_bf16_hw(float a, float b) {
  typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 v2bf;
  const v2bf v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32 (round to nearest even)
  return __builtin_bit_cast(uint32_t, v);
}

template <int D, bool DENSE, bool MULTI>
__global__ __launch_bounds__(256) void mqa_mfma_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ gamma_q, float eps,
    const uint16_t* __restrict__ E, long long N_cap, const int* __restrict__ idx, int k, int m,
    const uint16_t* __restrict__ W, int W_cap, int n_win, const float* __restrict__ sink,
    const int* __restrict__ q_pos, int Tq, int n_h, int rope_dim, RopeRatio rope, float scale,
    int kps, int n_split, long long n_units, uint16_t* __restrict__ out, float* __restrict__ ws) {
  constexpr int KS = D / 32;          // 8-dim chunks per lane group (S^T K-steps)
  constexpr int GW = D / 4;           // dims per lane group
  constexpr int NT = D / 16;          // 16-dim output tiles
  constexpr int RB = D * 2;           // row bytes
  constexpr int CPR = RB / 16;        // 16-byte pieces per row
  constexpr int RPI = 64 / CPR;       // rows per 1 KB load instruction
  constexpr int NKT = MQ_GROUP / 16;  // key tiles per group
  extern __shared__ __attribute__((aligned(16))) uint8_t kv[];   // MQ_GROUP * RB bytes
  __shared__ const uint16_t* srow[MQ_GROUP];   // row pointer of each slot (nullptr = empty)
  __shared__ float rope_cs[D];                 // (cos, sin) at i * theta_u, u < rope_dim / 2

  // ---- unit of work; the n_hg head groups of a unit are 8 workgroups apart (same XCD)
  const int n_hg = (n_h + 63) / 64;
  const long long L = blockIdx.x;
  const int hg = (int)((L / 8) % n_hg);
  const long long unit = (L / (8LL * n_hg)) * 8 + (L % 8);
  if (unit >= n_units) return;
  const int sp = (int)(unit % n_split);
  const size_t row = (size_t)(unit / n_split);
  const int b = (int)(row / Tq);
  const long long i = q_pos[row];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int h0 = 64 * hg + 16 * wave;
  const bool wact = h0 < n_h;
  const int hq = wact ? h0 + j : 0;

  for (int u = threadIdx.x; u < rope_dim / 2; u += 256)
    rope_cos_sin(i, u, rope, &rope_cs[2 * u], &rope_cs[2 * u + 1]);

  const QuerySlots qs = query_slots<DENSE>(i, N_cap, k, m, n_win);
  const int* idx_row = DENSE ? nullptr : idx + row * (size_t)k;
  const long long s0 = (long long)sp * kps;
  const long long s1 = min(s0 + (long long)kps, qs.n_slots);
  const uint16_t* dummy = E + (size_t)b * (size_t)N_cap * D;   // a valid row for empty slots
  __syncthreads();

  // ---- q^ = RoPE_i(RMSNorm(q)) as the B operand of S^T: head hq, dims GW*g + 8ks + e
  bf16x8_t qf[KS];
  {
    u32x4_t raw[KS];
    float ss = 0.f;
    const uint16_t* qp = q + (row * n_h + hq) * (size_t)D + GW * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      raw[ks] = *(const u32x4_t*)(qp + 8 * ks);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = __uint_as_float(raw[ks][e] << 16);
        const float x1 = __uint_as_float(raw[ks][e] & 0xffff0000u);
        ss += x0 * x0 + x1 * x1;
      }
    }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    const float rinv = 1.f / sqrtf(ss / (float)D + eps);
    const int rbeg = D - rope_dim;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4_t packed;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int dim = GW * g + 8 * ks + 2 * e;
        float v0 = __uint_as_float(raw[ks][e] << 16) * rinv * (gamma_q ? gamma_q[dim] : 1.f);
        float v1 = __uint_as_float(raw[ks][e] & 0xffff0000u) * rinv * (gamma_q ? gamma_q[dim + 1] : 1.f);
        if (dim >= rbeg) {
          const float cs = rope_cs[dim - rbeg], sn = rope_cs[dim - rbeg + 1];
          const float r0 = v0 * cs - v1 * sn, r1 = v0 * sn + v1 * cs;
          v0 = r0;
          v1 = r1;
        }
        packed[e] = pack2_bf16_hw(v0, v1);
      }
      qf[ks] = __builtin_bit_cast(bf16x8_t, packed);
    }
  }

  float m_run = -INFINITY, l_run = 0.f;    // softmax state of head hq (m_run: reference maximum)
  f32x4_t O[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) O[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  for (long long g0 = s0; g0 < s1; g0 += MQ_GROUP) {
    const int nrows = (int)min((long long)MQ_GROUP, s1 - g0);
    const int nch = (nrows + 31) / 32;                 // 32-row chunks holding slots
    // ---- resolve the group's slots, then copy their rows into LDS (swizzled pieces)
    if (threadIdx.x < MQ_GROUP) {
      const uint16_t* p = nullptr;
      if (threadIdx.x < nrows) {
        bool in_E;
        const long long off = slot_row<DENSE>(g0 + threadIdx.x, qs, idx_row, b, N_cap, W_cap, D, &in_E);
        if (off >= 0) p = (in_E ? E : W) + off;
      }
      srow[threadIdx.x] = p;
    }
    __syncthreads();
    for (int r0 = wave * RPI; r0 < nch * 32; r0 += 4 * RPI) {
      const int r = r0 + lane / CPR;
      const int c = (lane % CPR) ^ mq_swz(r);
      const uint16_t* p = srow[r];
      const uint8_t* src = (const uint8_t*)(p ? p : dummy) + 16 * c;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (__attribute__((address_space(3))) void*)(kv + r0 * RB), 16, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (wact) {
      // ---- phase 1: S^T for every key tile of the group (keys as M, heads as N).
      // K-step outer, 8 independent accumulators inner, so the LDS reads of a step
      // overlap.  Tiles past the group's rows read stale LDS; their scores are masked.
      f32x4_t S[NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) S[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        bf16x8_t a[NKT];
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt) {
          const int rr = 16 * kt + j;
          a[kt] = *(const bf16x8_t*)(kv + rr * RB + 16 * ((GW * g / 8 + ks) ^ mq_swz(rr)));
        }
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
          S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kt], qf[ks], S[kt], 0, 0, 0);
      }
      // lane (g, j): S[kt][r] = score of key 16 kt + 4 g + r for head hq
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int rr = 16 * kt + 4 * g + r;
          const bool ok = rr < nrows && srow[rr] != nullptr;
          S[kt][r] = ok ? S[kt][r] * scale : -INFINITY;
          mx = fmaxf(mx, S[kt][r]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      if constexpr (MULTI) {
        // move the reference maximum only when it would be exceeded by more than the slack
        if (__any(mx > m_run + MQ_REF_SLACK)) {
          const float m_new = (mx > m_run + MQ_REF_SLACK) ? mx : m_run;
          const float alpha = (m_run == -INFINITY) ? 0.f : __expf(m_run - m_new);
          l_run *= alpha;
          m_run = m_new;
          if (__any(alpha != 0.f)) {   // O is still zero while nothing has been accumulated
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float ar = __shfl(alpha, 4 * g + r, 64);
#pragma unroll
              for (int nt = 0; nt < NT; ++nt) O[nt][r] *= ar;
            }
          }
        }
      } else {
        m_run = mx;   // a single group: its maximum is the reference
      }
      float psum = 0.f;
      bf16x8_t pf[NKT / 2];
#pragma unroll
      for (int kk = 0; kk < NKT / 2; ++kk) {
        float p[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          p[r] = (S[2 * kk][r] == -INFINITY) ? 0.f : __expf(S[2 * kk][r] - m_run);
          p[4 + r] = (S[2 * kk + 1][r] == -INFINITY) ? 0.f : __expf(S[2 * kk + 1][r] - m_run);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) psum += p[e];
        u32x4_t pw;
        pw[0] = pack2_bf16_hw(p[0], p[1]);
        pw[1] = pack2_bf16_hw(p[2], p[3]);
        pw[2] = pack2_bf16_hw(p[4], p[5]);
        pw[3] = pack2_bf16_hw(p[6], p[7]);
        pf[kk] = __builtin_bit_cast(bf16x8_t, pw);
      }
      psum += __shfl_xor(psum, 16, 64);
      psum += __shfl_xor(psum, 32, 64);
      l_run += psum;
      // ---- phase 2: P (A operand: head j, keys {4g..4g+3, 16+4g..16+4g+3} of each
      // 32-key step) times V (transpose reads of the swizzled rows)
      const int half = 8 * (j & 1);
#pragma unroll
      for (int kk = 0; kk < NKT / 2; ++kk) {
        if (kk < nch) {
          const int tr0 = 32 * kk + 4 * g + (j >> 2), tr1 = tr0 + 16;
          const int sw0 = mq_swz(tr0), sw1 = mq_swz(tr1);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt) {
            const int pc = 2 * nt + ((j & 3) >> 1);
            const u32x2_t v0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4_t*)(kv + tr0 * RB + 16 * (pc ^ sw0) + half)));
            const u32x2_t v1 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) short4_t*)(kv + tr1 * RB + 16 * (pc ^ sw1) + half)));
            const u32x4_t vw = {v0[0], v0[1], v1[0], v1[1]};
            O[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[kk], __builtin_bit_cast(bf16x8_t, vw), O[nt], 0, 0, 0);
          }
        }
      }
    }
    __syncthreads();   // LDS rows and srow are rewritten by the next group
  }
  if (!wact) return;

  if (n_split == 1) {
    // ---- finish: sink, normalise, rotate the last rope_dim dims at -i, store
    const float sig = sink ? sink[hq] : -INFINITY;
    const float M = fmaxf(m_run, sig);
    float Z = 0.f;
    if (m_run != -INFINITY) Z += l_run * __expf(m_run - M);
    if (sig != -INFINITY) Z += __expf(sig - M);
    const float f = (Z > 0.f && m_run != -INFINITY) ? __expf(m_run - M) / Z : 0.f;
    float fr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) fr[r] = __shfl(f, 4 * g + r, 64);
    const int rbeg = D - rope_dim;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int dim = 16 * nt + j;
      float cs = 1.f, sn = 0.f;   // rotation at -i: cos(-x) = cos x, sin(-x) = -sin x
      if (dim >= rbeg) {
        cs = rope_cs[(dim - rbeg) & ~1];
        sn = -rope_cs[((dim - rbeg) & ~1) + 1];
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float v = O[nt][r] * fr[r];
        const float other = __shfl_xor(v, 1, 64);
        float o = v;
        if (dim >= rbeg) o = (dim & 1) ? (other * sn + v * cs) : (v * cs - other * sn);
        out[(row * n_h + h0 + 4 * g + r) * (size_t)D + dim] = f32_to_bf16_bits(o);
      }
    }
  } else {
    // ---- partial state: O / l_run scaled by a power of two, then the record
    const size_t pbase = (row * n_split + sp) * (size_t)n_h;
    float* ml = part_ml(ws, n_units, n_h, D);
    _Float16* wo = part_o(ws);
    const float li = part_inv(l_run);
    float lr[4], sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lr[r] = __shfl(li, 4 * g + r, 64);
      float a = 0.f;   // row maximum of head 4 g + r (its 16 lanes hold every dim)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) a = fmaxf(a, fabsf(O[nt][r] * lr[r]));
#pragma unroll
      for (int x = 1; x < 16; x <<= 1) a = fmaxf(a, __shfl_xor(a, x, 64));
      sc[r] = part_scale(a);
      lr[r] *= sc[r];
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        wo[(pbase + h0 + 4 * g + r) * D + 16 * nt + j] = part_h(O[nt][r] * lr[r]);
    // lane (0, j) writes the record of head h0 + j, whose scale lane group j / 4 holds
    const float s0 = __shfl(sc[0], 16 * (j >> 2), 64), s1 = __shfl(sc[1], 16 * (j >> 2), 64);
    const float s2 = __shfl(sc[2], 16 * (j >> 2), 64), s3 = __shfl(sc[3], 16 * (j >> 2), 64);
    const float sj = (j & 3) == 0 ? s0 : (j & 3) == 1 ? s1 : (j & 3) == 2 ? s2 : s3;
    if (g == 0)
      *(f32x4_t*)(ml + 4 * (pbase + hq)) = f32x4_t{m_run, l_run, part_unscale(sj), 0.f};
  }
}

// ---------------------------------------------------------------------------
// single-group kernel (every split holds <= 128 slots: decode).  Phase 1 as in
// the multi-group kernel (wave w: S^T of head tile w over the 128 slots); P
// goes to LDS; phase 2 gives wave w the output dims [w D/4, (w+1) D/4) of all
// 64 heads, so each transposed V fragment read from LDS feeds four MFMAs
// (one per head tile) and the accumulators are not live during phase 1.
// ---------------------------------------------------------------------------
template <int D, bool DENSE>
__global__ __launch_bounds__(256) void mqa_group_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ gamma_q, float eps,
    const uint16_t* __restrict__ E, long long N_cap, const int* __restrict__ idx, int k, int m,
    const uint16_t* __restrict__ W, int W_cap, int n_win, const float* __restrict__ sink,
    const int* __restrict__ q_pos, int Tq, int n_h, int rope_dim, RopeRatio rope, float scale,
    int kps, int n_split, long long n_units, uint16_t* __restrict__ out, float* __restrict__ ws) {
  constexpr int KS = D / 32, GW = D / 4, RB = D * 2, CPR = RB / 16, RPI = 64 / CPR;
  constexpr int NKT = MQ_GROUP / 16;   // key tiles (8)
  constexpr int NKK = MQ_GROUP / 32;   // 32-key MFMA steps of P.V (4)
  constexpr int NTW = D / 64;          // 16-dim output tiles per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t kv[];   // MQ_GROUP * RB bytes
  __shared__ const uint16_t* srow[MQ_GROUP];
  __shared__ float rope_cs[D];
  __shared__ u32x4_t pbuf[4][NKK][64];   // P fragments: [head tile][32-key step][lane]
  __shared__ float fstat[64], mstat[64], lstat[64];
  __shared__ float amx[4][64];           // split partials: per-wave row maxima of each head

  const int n_hg = (n_h + 63) / 64;
  const long long L = blockIdx.x;
  const int hg = (int)((L / 8) % n_hg);
  const long long unit = (L / (8LL * n_hg)) * 8 + (L % 8);
  if (unit >= n_units) return;
  const int sp = (int)(unit % n_split);
  const size_t row = (size_t)(unit / n_split);
  const int b = (int)(row / Tq);
  const long long i = q_pos[row];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int hbase = 64 * hg;
  const int ntiles = min(4, (n_h - hbase) / 16);   // valid head tiles of this workgroup
  const bool wact = wave < ntiles;
  const int hq = wact ? hbase + 16 * wave + j : 0;

  const QuerySlots qs = query_slots<DENSE>(i, N_cap, k, m, n_win);
  const int* idx_row = DENSE ? nullptr : idx + row * (size_t)k;
  const long long s0 = (long long)sp * kps;
  const long long s1 = min(s0 + (long long)kps, qs.n_slots);
  const int nrows = (int)max(0LL, min((long long)MQ_GROUP, s1 - s0));
  const int nch = (nrows + 31) / 32;
  const uint16_t* dummy = E + (size_t)b * (size_t)N_cap * D;

  for (int u = threadIdx.x; u < rope_dim / 2; u += 256)
    rope_cos_sin(i, u, rope, &rope_cs[2 * u], &rope_cs[2 * u + 1]);
  if (threadIdx.x < MQ_GROUP) {
    const uint16_t* p = nullptr;
    if (threadIdx.x < nrows) {
      bool in_E;
      const long long off = slot_row<DENSE>(s0 + threadIdx.x, qs, idx_row, b, N_cap, W_cap, D, &in_E);
      if (off >= 0) p = (in_E ? E : W) + off;
    }
    srow[threadIdx.x] = p;
  }
  __syncthreads();
  for (int r0 = wave * RPI; r0 < nch * 32; r0 += 4 * RPI) {
    const int r = r0 + lane / CPR;
    const int c = (lane % CPR) ^ mq_swz(r);
    const uint16_t* p = srow[r];
    const uint8_t* src = (const uint8_t*)(p ? p : dummy) + 16 * c;
    __builtin_amdgcn_global_load_lds((const void*)src,
                                     (__attribute__((address_space(3))) void*)(kv + r0 * RB), 16, 0, 0);
  }

  // ---- phase 1 (wave w = head tile w): q^, S^T over the group, softmax statistics, P
  if (wact) {
    bf16x8_t qf[KS];
    {
      u32x4_t raw[KS];
      float ss = 0.f;
      const uint16_t* qp = q + (row * n_h + hq) * (size_t)D + GW * g;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        raw[ks] = *(const u32x4_t*)(qp + 8 * ks);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x0 = __uint_as_float(raw[ks][e] << 16);
          const float x1 = __uint_as_float(raw[ks][e] & 0xffff0000u);
          ss += x0 * x0 + x1 * x1;
        }
      }
      ss += __shfl_xor(ss, 16, 64);
      ss += __shfl_xor(ss, 32, 64);
      const float rinv = 1.f / sqrtf(ss / (float)D + eps);
      const int rbeg = D - rope_dim;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        u32x4_t packed;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int dim = GW * g + 8 * ks + 2 * e;
          float v0 = __uint_as_float(raw[ks][e] << 16) * rinv * (gamma_q ? gamma_q[dim] : 1.f);
          float v1 = __uint_as_float(raw[ks][e] & 0xffff0000u) * rinv * (gamma_q ? gamma_q[dim + 1] : 1.f);
          if (dim >= rbeg) {
            const float cs = rope_cs[dim - rbeg], sn = rope_cs[dim - rbeg + 1];
            const float r0 = v0 * cs - v1 * sn, r1 = v0 * sn + v1 * cs;
            v0 = r0;
            v1 = r1;
          }
          packed[e] = pack2_bf16_hw(v0, v1);
        }
        qf[ks] = __builtin_bit_cast(bf16x8_t, packed);
      }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // (a) rows landed
    f32x4_t S[NKT];
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt) S[kt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8_t a[NKT];
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt) {
        const int rr = 16 * kt + j;
        a[kt] = *(const bf16x8_t*)(kv + rr * RB + 16 * ((GW * g / 8 + ks) ^ mq_swz(rr)));
      }
#pragma unroll
      for (int kt = 0; kt < NKT; ++kt)
        S[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[kt], qf[ks], S[kt], 0, 0, 0);
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rr = 16 * kt + 4 * g + r;
        const bool ok = rr < nrows && srow[rr] != nullptr;
        S[kt][r] = ok ? S[kt][r] * scale : -INFINITY;
        mx = fmaxf(mx, S[kt][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    float psum = 0.f;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      float p[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = (S[2 * kk][r] == -INFINITY) ? 0.f : __expf(S[2 * kk][r] - mx);
        p[4 + r] = (S[2 * kk + 1][r] == -INFINITY) ? 0.f : __expf(S[2 * kk + 1][r] - mx);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) psum += p[e];
      u32x4_t pw;
      pw[0] = pack2_bf16_hw(p[0], p[1]);
      pw[1] = pack2_bf16_hw(p[2], p[3]);
      pw[2] = pack2_bf16_hw(p[4], p[5]);
      pw[3] = pack2_bf16_hw(p[6], p[7]);
      pbuf[wave][kk][lane] = pw;
    }
    psum += __shfl_xor(psum, 16, 64);
    psum += __shfl_xor(psum, 32, 64);
    if (g == 0) {
      const int hl = 16 * wave + j;
      mstat[hl] = mx;
      lstat[hl] = psum;
      const float sig = sink ? sink[hq] : -INFINITY;
      const float M = fmaxf(mx, sig);
      float Z = 0.f;
      if (mx != -INFINITY) Z += psum * __expf(mx - M);
      if (sig != -INFINITY) Z += __expf(sig - M);
      fstat[hl] = (Z > 0.f && mx != -INFINITY) ? __expf(mx - M) / Z : 0.f;
    }
  } else {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();   // (a)
  }
  __syncthreads();     // (b) P and the statistics are visible

  // ---- phase 2 (wave w = output dims [w D/4, (w+1) D/4) of every head tile)
  f32x4_t O[4][NTW];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) O[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int dbase = wave * (D / 4);
  const int half = 8 * (j & 1);
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) {
    if (kk < nch) {
      const int tr0 = 32 * kk + 4 * g + (j >> 2), tr1 = tr0 + 16;
      const int sw0 = mq_swz(tr0), sw1 = mq_swz(tr1);
      bf16x8_t vf[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int pc = (dbase + 16 * nt) / 8 + ((j & 3) >> 1);
        const u32x2_t v0 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t*)(kv + tr0 * RB + 16 * (pc ^ sw0) + half)));
        const u32x2_t v1 = __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) short4_t*)(kv + tr1 * RB + 16 * (pc ^ sw1) + half)));
        const u32x4_t vw = {v0[0], v0[1], v1[0], v1[1]};
        vf[nt] = __builtin_bit_cast(bf16x8_t, vw);
      }
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        if (mt < ntiles) {
          const bf16x8_t pf = __builtin_bit_cast(bf16x8_t, pbuf[mt][kk][lane]);
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt)
            O[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, vf[nt], O[mt][nt], 0, 0, 0);
        }
      }
    }
  }

  // ---- output: lane (g, j) of tile (mt, nt) holds heads 16mt + 4g + r, dim dbase + 16nt + j
  const int rbeg = D - rope_dim;
  if (n_split == 1) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt >= ntiles) continue;
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int dim = dbase + 16 * nt + j;
        float cs = 1.f, sn = 0.f;   // rotation at -i: cos(-x) = cos x, sin(-x) = -sin x
        if (dim >= rbeg) {
          cs = rope_cs[(dim - rbeg) & ~1];
          sn = -rope_cs[((dim - rbeg) & ~1) + 1];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hl = 16 * mt + 4 * g + r;
          const float v = O[mt][nt][r] * fstat[hl];
          const float other = __shfl_xor(v, 1, 64);
          float o = v;
          if (dim >= rbeg) o = (dim & 1) ? (other * sn + v * cs) : (v * cs - other * sn);
          out[(row * n_h + hbase + hl) * (size_t)D + dim] = f32_to_bf16_bits(o);
        }
      }
    }
  } else {
    // O / l scaled by a power of two from the row maximum; a head's row spans the
    // four waves' dims, so their maxima meet in LDS
    const size_t pbase = (row * n_split + sp) * (size_t)n_h + hbase;
    _Float16* wo = part_o(ws);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float li = part_inv(lstat[16 * mt + 4 * g + r]);
        float a = 0.f;
        if (mt < ntiles) {
#pragma unroll
          for (int nt = 0; nt < NTW; ++nt) a = fmaxf(a, fabsf(O[mt][nt][r] * li));
        }
#pragma unroll
        for (int x = 1; x < 16; x <<= 1) a = fmaxf(a, __shfl_xor(a, x, 64));
        if (j == 0) amx[wave][16 * mt + 4 * g + r] = a;
      }
    }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt >= ntiles) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int hl = 16 * mt + 4 * g + r;
        const float sc = part_scale(fmaxf(fmaxf(amx[0][hl], amx[1][hl]), fmaxf(amx[2][hl], amx[3][hl])));
        const float li = part_inv(lstat[hl]) * sc;
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          wo[(pbase + hl) * D + dbase + 16 * nt + j] = part_h(O[mt][nt][r] * li);
      }
    }
    if (threadIdx.x < 16 * ntiles) {
      const int hl = threadIdx.x;
      const float sc = part_scale(fmaxf(fmaxf(amx[0][hl], amx[1][hl]), fmaxf(amx[2][hl], amx[3][hl])));
      float* ml = part_ml(ws, n_units, n_h, D);
      *(f32x4_t*)(ml + 4 * (pbase + hl)) = f32x4_t{mstat[hl], lstat[hl], part_unscale(sc), 0.f};
    }
  }
}

// ---------------------------------------------------------------------------
// decode kernel (few queries per sequence, heads a multiple of 16 per wave).
//
// A workgroup takes one query, a group of 16 HTW NW heads and a fixed range of
// at most MQ_DEC_TABLE key slots.  Wave w owns HTW 16-head tiles of the group
// (two, or one for decode at D = 512) over all D dims, so scores, softmax and P.V stay
// inside the wave and need no exchange.  The slots' rows stream through LDS 32 at a time: a ring of
// MQ_DEC_NBUF chunks filled with global_load_lds, MQ_DEC_NBUF - 1 chunks ahead,
// so each row is fetched from memory once per workgroup and then read from LDS
// by every wave.  Rows sit at a stride of 2D + 16 bytes: 16 lanes reading one
// 16-byte piece of 16 consecutive rows (the S^T operand) hit distinct banks,
// and the transposed reads of V take constant offsets along a row.  The
// range's selected entries are staged in LDS with the query loads, so a chunk's
// row addresses cost an LDS read, not a memory round trip.  The first chunk
// of a range skips the output rescale (O is still 0).  The split depends
// only on the slot count; a combine kernel merges split partials in order.
// ---------------------------------------------------------------------------
// key slots per workgroup (whole chunks), a function of the query's slot count
// only: 192 up to 1,536 slots, 160 above.  Both keep the decode grids near one
// workgroup per CU: the 1M CSA decode (1,152 slots, 16 sequences, 2 head
// groups) makes 192 workgroups, the 1M HCA decode (8,320 slots, 4 sequences,
// 1 head group) 208.  More ranges mean more split partials to merge.
static constexpr int MQ_DEC_SPLIT_LONG = 160;
static constexpr int MQ_DEC_SPLIT_SMALL = 192;
static constexpr long long MQ_DEC_SMALL_UPTO = 1536;
// slot table capacity of the decode ranges (the larger of the two range sizes)
static constexpr int MQ_DEC_TBL_SMALL = MQ_DEC_SPLIT_LONG > MQ_DEC_SPLIT_SMALL ? MQ_DEC_SPLIT_LONG : MQ_DEC_SPLIT_SMALL;
// With many queries per sequence (prefill) the queries give the parallelism:
// one range holds up to MQ_DEC_TABLE slots (the slot table's capacity), so a
// CSA query (k + n_win slots) is one workgroup and needs no combine.
static constexpr int MQ_DEC_TABLE = 2048;
static constexpr int MQ_DEC_NBUF = 3;      // LDS chunk ring
static constexpr int MQ_MIX_ROPE = 64;     // rotated (bf16) dims of a mixed row

// Workgroup barrier for LDS traffic only: this wave's LDS operations complete
// (lgkmcnt 0) and its vector-memory operations drop to at most VM outstanding
// (gfx9 s_waitcnt encoding; 63 = no wait), then s_barrier.  __syncthreads()
// would also drain every global_load_lds still in flight (vmcnt 0), which
// defeats the chunk prefetch.  The empty asm statements keep the compiler from
// moving memory accesses across the barrier.
template <int VM>
__device__ __forceinline__ void lds_sync() {
  static_assert(VM >= 0 && VM <= 63, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Sixteen transposed 64-bit LDS reads (ds_read_b64_tr_b16): eight 16-dim tiles
// at byte offsets 0, 32, ..., 224 from a0 (rows 4g..4g+3 of the chunk) and a1
// (rows 16+4g..), completed inside the statement.  The builtin form makes the
// compiler wait for every global_load_lds in flight (vmcnt 0) before the read,
// because it cannot tell the addresses apart from the prefetched chunks.
__device__ __forceinline__ void lds_read_tr16(uint32_t a0, uint32_t a1, u32x2_t (&r)[16]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %17\n\t"
      "ds_read_b64_tr_b16 %2, %16 offset:32\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:32\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:64\n\t"
      "ds_read_b64_tr_b16 %5, %17 offset:64\n\t"
      "ds_read_b64_tr_b16 %6, %16 offset:96\n\t"
      "ds_read_b64_tr_b16 %7, %17 offset:96\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:128\n\t"
      "ds_read_b64_tr_b16 %9, %17 offset:128\n\t"
      "ds_read_b64_tr_b16 %10, %16 offset:160\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:160\n\t"
      "ds_read_b64_tr_b16 %12, %16 offset:192\n\t"
      "ds_read_b64_tr_b16 %13, %17 offset:192\n\t"
      "ds_read_b64_tr_b16 %14, %16 offset:224\n\t"
      "ds_read_b64_tr_b16 %15, %17 offset:224\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
        "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(a0), "v"(a1)
      : "memory");
}

// The same for sixteen tiles (offsets 0 .. 480): one wait for two blocks of eight.
__device__ __forceinline__ void lds_read_tr32(uint32_t a0, uint32_t a1, u32x2_t (&r)[32]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %32\n\t"
      "ds_read_b64_tr_b16 %1, %33\n\t"
      "ds_read_b64_tr_b16 %2, %32 offset:32\n\t"
      "ds_read_b64_tr_b16 %3, %33 offset:32\n\t"
      "ds_read_b64_tr_b16 %4, %32 offset:64\n\t"
      "ds_read_b64_tr_b16 %5, %33 offset:64\n\t"
      "ds_read_b64_tr_b16 %6, %32 offset:96\n\t"
      "ds_read_b64_tr_b16 %7, %33 offset:96\n\t"
      "ds_read_b64_tr_b16 %8, %32 offset:128\n\t"
      "ds_read_b64_tr_b16 %9, %33 offset:128\n\t"
      "ds_read_b64_tr_b16 %10, %32 offset:160\n\t"
      "ds_read_b64_tr_b16 %11, %33 offset:160\n\t"
      "ds_read_b64_tr_b16 %12, %32 offset:192\n\t"
      "ds_read_b64_tr_b16 %13, %33 offset:192\n\t"
      "ds_read_b64_tr_b16 %14, %32 offset:224\n\t"
      "ds_read_b64_tr_b16 %15, %33 offset:224\n\t"
      "ds_read_b64_tr_b16 %16, %32 offset:256\n\t"
      "ds_read_b64_tr_b16 %17, %33 offset:256\n\t"
      "ds_read_b64_tr_b16 %18, %32 offset:288\n\t"
      "ds_read_b64_tr_b16 %19, %33 offset:288\n\t"
      "ds_read_b64_tr_b16 %20, %32 offset:320\n\t"
      "ds_read_b64_tr_b16 %21, %33 offset:320\n\t"
      "ds_read_b64_tr_b16 %22, %32 offset:352\n\t"
      "ds_read_b64_tr_b16 %23, %33 offset:352\n\t"
      "ds_read_b64_tr_b16 %24, %32 offset:384\n\t"
      "ds_read_b64_tr_b16 %25, %33 offset:384\n\t"
      "ds_read_b64_tr_b16 %26, %32 offset:416\n\t"
      "ds_read_b64_tr_b16 %27, %33 offset:416\n\t"
      "ds_read_b64_tr_b16 %28, %32 offset:448\n\t"
      "ds_read_b64_tr_b16 %29, %33 offset:448\n\t"
      "ds_read_b64_tr_b16 %30, %32 offset:480\n\t"
      "ds_read_b64_tr_b16 %31, %33 offset:480\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15]), "=&v"(r[16]), "=&v"(r[17]), "=&v"(r[18]), "=&v"(r[19]), "=&v"(r[20]), "=&v"(r[21]), "=&v"(r[22]), "=&v"(r[23]), "=&v"(r[24]), "=&v"(r[25]), "=&v"(r[26]), "=&v"(r[27]), "=&v"(r[28]), "=&v"(r[29]), "=&v"(r[30]), "=&v"(r[31])
      : "v"(a0), "v"(a1)
      : "memory");
}

// where the rows of one workgroup's slot range come from (all wave-uniform)
struct DecRows {
  const uint16_t* E_b;        // this sequence's entries
  const uint16_t* W_b;        // this sequence's window ring
  const uint16_t* dummy;      // a valid row, loaded for absent slots (their scores are masked)
  const float* Es_b;          // mixed rows: this sequence's entry row scales
  const float* Ws_b;          // mixed rows: this sequence's window row scales
  long long row_bytes;        // bytes per stored row (2 D, or D + rope_dim for mixed rows)
  long long s0;               // first slot of the range
  int n_rows;                 // slots in the range
  int n_sel;                  // of them, entry slots (the rest are window slots)
  int ring0;                  // ring row of the range's first window slot
  int W_cap;
  int N_cap;                  // entries per sequence, clamped to int
};

// row of slot `rel` of the range (e = its selected entry when sparse); *ok is
// false for an absent slot, whose row is the dummy.  Selects only, no branches:
// a divergent branch here would pull the selection loads into it, each with
// its own wait.
template <int D, bool DENSE, bool MIX = false>
__device__ __forceinline__ const uint16_t* dec_slot_row(int rel, int e, const DecRows& R, bool* ok,
                                                        float* rs = nullptr) {
  const bool in_rows = rel < R.n_rows;
  const bool is_sel = rel < R.n_sel;
  const long long ent = DENSE ? R.s0 + rel : (long long)e;
  const bool ent_ok = DENSE || (e >= 0 && e < R.N_cap);
  int ring = R.ring0 + (rel - R.n_sel);   // fewer window slots than ring rows: one wrap at most
  ring = ring >= R.W_cap ? ring - R.W_cap : ring;
  *ok = in_rows && (!is_sel || ent_ok);
  const long long rb = MIX ? R.row_bytes : 2LL * D;
  const uintptr_t pe = (uintptr_t)R.E_b + (uintptr_t)(max(ent, 0LL) * rb);
  const uintptr_t pw = (uintptr_t)R.W_b + (uintptr_t)((long long)max(ring, 0) * rb);
  if constexpr (MIX) {
    // the row's scale (unguarded loads at clamped rows, selected after)
    const float se = R.Es_b[max(min(ent, (long long)R.N_cap - 1), 0LL)];
    const float sw = R.Ws_b ? R.Ws_b[max(min(ring, R.W_cap - 1), 0)] : 1.f;
    *rs = !*ok ? 1.f : (is_sel ? se : sw);
  }
  return (const uint16_t*)(!*ok ? (uintptr_t)R.dummy : (is_sel ? pe : pw));
}

// start loading chunk c: rows RPW w .. RPW w + RPW - 1 of it are this wave's,
// their addresses read from the workgroup's slot table
// (mixed rows: cpr = row bytes / 16 pieces per row, rows at a stride of rbp bytes)
template <int D, int NW>
__device__ __forceinline__ void dec_issue(int c, const uint16_t* const* sptr, uint8_t* buf, int wave,
                                          int lane, int cpr = 2 * D / 16, int rbp = 2 * D + 16) {
  constexpr int RPW = MQ_CH / NW;
  const int rel0 = MQ_CH * c + RPW * wave;
  const uint16_t* p[RPW];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr) p[rr] = sptr[rel0 + rr];
#pragma unroll
  for (int rr = 0; rr < RPW; ++rr)
    if (lane < cpr)
      __builtin_amdgcn_global_load_lds((const void*)(p[rr] + 8 * lane),
                                       (__attribute__((address_space(3))) void*)(buf + (RPW * wave + rr) * rbp),
                                       16, 0, 0);
}

// the maximum and the sum of x over lanes l, l ^ 16, l ^ 32, l ^ 48 (the four
// lane groups of an MFMA tile column), with the gfx950 row swaps; each swap
// leaves a lane its own value and its partner's, in either order
__device__ __forceinline__ float quad_max(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// HTW: head tiles (16 heads each) per wave (host choice: dec_htw)
// MIX: entries and window rows are mixed rows (e4m3 codes of the first
// D - MQ_MIX_ROPE dims under a row scale, then bf16 of the MQ_MIX_ROPE rotated
// dims; scales in Es and Ws).  Their raw bytes stream through the LDS ring as
// the bf16 rows do; once a chunk has landed every thread widens its share of
// the codes into one bf16 chunk buffer (exact: every e4m3 value is a bf16
// value) and copies the rotated dims.  The row scale never rounds a stored
// value: the scores take it as s_key * (q . codes) + (q . rotated dims), the
// rotated share accumulated a second time on its own (the query with the other
// dims zeroed), and P.V as (p * s_key) . codes on the code dims and
// p . rotated on the rest, split at a 16-dim output tile boundary.
template <int D, bool DENSE, int NW, int TBL, int HTW, bool MIX = false>
__global__ __launch_bounds__(64 * NW) void mqa_decode_kernel(
    const uint16_t* __restrict__ q, const float* __restrict__ gamma_q, float eps,
    const uint16_t* __restrict__ E, long long N_cap, const int* __restrict__ idx, int k, int m,
    const uint16_t* __restrict__ W, int W_cap, int n_win, const float* __restrict__ sink,
    const int* __restrict__ q_pos, int Tq, int n_h, int rope_dim, RopeRatio rope, float scale,
    int kps, int n_split, long long n_units, uint16_t* __restrict__ out, float* __restrict__ ws,
    const float* __restrict__ Es, const float* __restrict__ Ws) {
  constexpr int KS = D / 32;          // S^T K-steps (8 dims per lane each)
  constexpr int NT = D / 16;          // 16-dim output tiles
  constexpr int RBP = 2 * D + 16;     // LDS row stride
  constexpr int RPW = MQ_CH / NW;     // rows each wave loads per chunk
  constexpr int CHB = MQ_CH * RBP;    // bytes per chunk
  constexpr int HG = 16 * HTW * NW;   // heads per workgroup
  constexpr int PF = MQ_DEC_NBUF - 1;
  constexpr int GPT = (D + 64 * NW - 1) / (64 * NW);   // gamma values per thread
  static_assert((PF - 1) * RPW <= 63, "vmcnt range");
  extern __shared__ __attribute__((aligned(16))) uint8_t kv[];   // MQ_DEC_NBUF * CHB
  __shared__ float rope_cs[D];   // (cos, sin) at position i of the pair starting at dim 2u; (1, 0) if not rotated
  __shared__ float gam[D];
  constexpr int NCH_MAX = TBL / MQ_CH;   // TBL: slot table capacity (a range's slots at most)
  static_assert(MQ_DEC_SPLIT_LONG % MQ_CH == 0 && MQ_DEC_SPLIT_SMALL % MQ_CH == 0 &&
                    TBL % MQ_CH == 0 && MQ_DEC_TBL_SMALL <= MQ_DEC_TABLE,
                "whole chunks per range");
  __shared__ const uint16_t* sptr[TBL];   // row of every slot of the range
  __shared__ __attribute__((aligned(16))) float sscale[MIX ? TBL : 4];  // mixed rows: each slot's row scale
  constexpr int NOPE = MIX ? D - MQ_MIX_ROPE : D;              // mixed rows: the e4m3 dims
  // lane group g feeds dims D/4 g + 8 ks .. of K-step ks: the rotated dims are those
  // of group 3 from K-step MIX_KS0 on, and whole 16-dim output tiles from NOPE on
  constexpr int MIX_KS0 = (D / 4 - (D - NOPE)) / 8;
  static_assert(!MIX || (MQ_MIX_ROPE <= D / 4 && MQ_MIX_ROPE % 16 == 0), "rotated dims in the last quarter");
  constexpr int RAW_ROW = MIX ? NOPE + 2 * MQ_MIX_ROPE : 2 * D;   // stored bytes per row
  constexpr int raw_rb = RAW_ROW + 16;                         // LDS ring row stride
  constexpr int raw_cpr = RAW_ROW / 16;                        // 16-byte pieces per row
  uint8_t* const convb = kv + MQ_DEC_NBUF * MQ_CH * raw_rb;   // mixed rows: the widened chunk
  __shared__ uint32_t smask[NCH_MAX];              // bit r of chunk c: slot 32 c + r exists
  __shared__ f32x4_t rs_tmp[NW * 8 * 64];   // per wave: eight output tiles, for the rare rescale

  // 32-bit index arithmetic (the host keeps the grid below 2^31 workgroups):
  // 64-bit divisions would put a few hundred instructions in front of the first load
  const unsigned n_hg = (unsigned)(n_h / HG);
  const unsigned L = blockIdx.x;
  const int hg = (int)((L / 8u) % n_hg);
  const unsigned unit = (L / (8u * n_hg)) * 8u + (L % 8u);
  if ((long long)unit >= n_units) return;
  const int sp = (int)(unit % (unsigned)n_split);
  const unsigned row32 = unit / (unsigned)n_split;
  const size_t row = row32;
  const int b = (int)(row32 / (unsigned)Tq);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, j = lane & 15;
  const int h0 = HG * hg + 16 * HTW * wave;   // first head of this wave
  const long long s0 = (long long)sp * kps;   // the range's first slot

  // The loads come first: the range's selection, the query pieces and gamma need
  // only the grid position, so their latency runs under the work on the query
  // position (its load, the slot counts, the RoPE table).  They are all used
  // before any chunk load is issued: a wait on an ordinary load issued before an
  // LDS-DMA load becomes a wait on every load in flight.
  constexpr int IPT = (TBL + 64 * NW - 1) / (64 * NW);
  int iv[IPT];
  if (!DENSE) {
    // bounded by the row's k selections only, so these loads need not wait for q_pos
    // unguarded loads (index clamped into the row, masked after): a guarded
    // load compiles to a branch with its own wait
    const int* idx_row = idx + row * (size_t)k;
    const int kcap = (int)max(0LL, min((long long)kps, (long long)k - s0));
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
      const int t = threadIdx.x + 64 * NW * e;
      const int v = idx_row[min(s0 + t, (long long)k - 1)];
      iv[e] = t < kcap ? v : -1;
    }
  }
  u32x4_t raw[HTW][KS];
#pragma unroll
  for (int ht = 0; ht < HTW; ++ht) {
    const uint16_t* qp = q + (row * n_h + h0 + 16 * ht + j) * (size_t)D + (D / 4) * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) raw[ht][ks] = *(const u32x4_t*)(qp + 8 * ks);
  }
  float gv[GPT];
#pragma unroll
  for (int e = 0; e < GPT; ++e) {
    const int t = threadIdx.x + 64 * NW * e;
    // unguarded: without gamma the load reads the query array (n_h >= 16 rows of
    // D bf16, so at least D floats) and the value is replaced by 1
    const float* gsrc = gamma_q ? gamma_q : (const float*)q;
    const float gl = gsrc[min(t, D - 1)];
    gv[e] = gamma_q ? gl : 1.f;
  }

  const long long i = q_pos[row];
  const QuerySlots qs = query_slots<DENSE>(i, N_cap, k, m, n_win);
  DecRows R;
  R.s0 = s0;
  R.n_rows = (int)max(0LL, min((long long)kps, qs.n_slots - R.s0));
  R.n_sel = (int)max(0LL, min((long long)R.n_rows, qs.n_sel - R.s0));
  R.row_bytes = RAW_ROW;
  R.E_b = (const uint16_t*)((const uint8_t*)E + (size_t)b * (size_t)N_cap * (size_t)R.row_bytes);
  R.W_b = W ? (const uint16_t*)((const uint8_t*)W + (size_t)b * (size_t)W_cap * (size_t)R.row_bytes) : nullptr;
  R.dummy = R.E_b;
  R.Es_b = MIX ? Es + (size_t)b * (size_t)N_cap : nullptr;
  R.Ws_b = (MIX && W) ? Ws + (size_t)b * (size_t)W_cap : nullptr;
  R.W_cap = W_cap;
  R.N_cap = (int)min(N_cap, 2147483647LL);
  R.ring0 = W_cap > 0 ? (int)((qs.win_lo + max(0LL, R.s0 - qs.n_sel)) % W_cap) : 0;
  const int nch = (R.n_rows + MQ_CH - 1) / MQ_CH;
  // the RoPE table needs the position alone, so it is built while the loads are in flight
  for (int t = threadIdx.x; t < D / 2; t += 64 * NW) {
    const int u = t - (D - rope_dim) / 2;
    float cs = 1.f, sn = 0.f;
    if (u >= 0) rope_cos_sin(i, u, rope, &cs, &sn);
    rope_cs[2 * t] = cs;
    rope_cs[2 * t + 1] = sn;
  }
  // slot table: thread t resolves slot t of the range once, for every wave
  // (straight-line code: no branch for the compiler to sink the selection
  // loads into, where each would get its own wait)
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const int t = threadIdx.x + 64 * NW * e;
    bool ok;
    float rs = 1.f;
    const uint16_t* p = dec_slot_row<D, DENSE, MIX>(t, DENSE ? 0 : iv[e], R, &ok, &rs);
    if (t < TBL) sptr[t] = p;
    if constexpr (MIX)
      if (t < TBL) sscale[t] = rs;
    const unsigned long long bal = __ballot(ok);
    if ((lane & 31) == 0 && (t >> 5) < NCH_MAX) smask[t >> 5] = (uint32_t)(bal >> (lane & 32));
  }
#pragma unroll
  for (int e = 0; e < GPT; ++e) {
    const int t = threadIdx.x + 64 * NW * e;
    if (t < D) gam[t] = gv[e];
  }
  float rinv[HTW];
#pragma unroll
  for (int ht = 0; ht < HTW; ++ht) {
    float ss = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x0 = __uint_as_float(raw[ht][ks][e] << 16);
        const float x1 = __uint_as_float(raw[ht][ks][e] & 0xffff0000u);
        ss += x0 * x0 + x1 * x1;
      }
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    rinv[ht] = 1.f / sqrtf(ss / (float)D + eps);
    // opaque to the compiler: the fp32 values unpacked for the sum are not kept
    // alive (twice the registers of the packed pieces) for the conversion below
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(raw[ht][ks]));
  }
  lds_sync<0>();   // selection, RoPE table and gamma visible
#pragma unroll
  for (int c = 0; c < PF; ++c)
    if (c < nch) dec_issue<D, NW>(c, sptr, kv + c * MQ_CH * raw_rb, wave, lane, raw_cpr, raw_rb);

  // q^ = RoPE_i(RMSNorm(q)) as bf16 B fragments of S^T: lane (g, j) holds head 16 ht + j,
  // dims (D/4) g + 8 ks + 0..7; the RoPE table holds (1, 0) for dims that are not rotated.
  // RoPE is linear, so the head's RMSNorm factor rinv moves onto its scores
  // (sc below): the fragments hold RoPE_i(gamma q), the same values up to the
  // common factor, and the bf16 rounding is relative either way.
  float sc[HTW];
#pragma unroll
  for (int ht = 0; ht < HTW; ++ht) sc[ht] = scale * rinv[ht];
  bf16x8_t qf[HTW][KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int d0 = (D / 4) * g + 8 * ks;
    const f32x4_t ga = *(const f32x4_t*)&gam[d0], gb = *(const f32x4_t*)&gam[d0 + 4];
    const f32x4_t ra = *(const f32x4_t*)&rope_cs[d0], rb = *(const f32x4_t*)&rope_cs[d0 + 4];
    const float gw[8] = {ga[0], ga[1], ga[2], ga[3], gb[0], gb[1], gb[2], gb[3]};
    const float rc[8] = {ra[0], ra[1], ra[2], ra[3], rb[0], rb[1], rb[2], rb[3]};
#pragma unroll
    for (int ht = 0; ht < HTW; ++ht) {
      u32x4_t packed;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float v0 = __uint_as_float(raw[ht][ks][e] << 16) * gw[2 * e];
        const float v1 = __uint_as_float(raw[ht][ks][e] & 0xffff0000u) * gw[2 * e + 1];
        const float cs = rc[2 * e], sn = rc[2 * e + 1];
        packed[e] = pack2_bf16_hw(v0 * cs - v1 * sn, v0 * sn + v1 * cs);
      }
      qf[ht][ks] = __builtin_bit_cast(bf16x8_t, packed);
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  f32x4_t O[HTW][NT];
#pragma unroll
  for (int ht = 0; ht < HTW; ++ht)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) O[ht][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float ref[HTW], lsum[HTW];   // of head 16 ht + j; lsum is this lane's share until the loop ends
#pragma unroll
  for (int ht = 0; ht < HTW; ++ht) {
    ref[ht] = -INFINITY;
    lsum[ht] = 0.f;
  }
  const int tr0 = 4 * g + (j >> 2), tr1 = tr0 + 16;

  for (int c = 0; c < nch; ++c) {
    // chunk c landed for every wave (later chunks may stay in flight); chunk c - 1 is consumed
    if (c + 1 < nch && PF >= 2) lds_sync<(PF >= 2 ? RPW : 0)>();
    else lds_sync<0>();
    const uint32_t vmask = smask[c];
    const uint8_t* kb = kv + (c % MQ_DEC_NBUF) * CHB;
    float skey[2][4];   // mixed rows: scales of keys 16 kt + 4 g + r of the chunk
    if constexpr (MIX) {
      // widen the landed chunk into the bf16 chunk buffer, 8 dims per piece: e4m3
      // codes to bf16 (exact), the rotated dims copied as they are
      const uint8_t* rawc = kv + (c % MQ_DEC_NBUF) * MQ_CH * raw_rb;
      constexpr int PPR = D / 8;
      for (int p = threadIdx.x; p < MQ_CH * PPR; p += 64 * NW) {
        const int rr = p / PPR, d0 = 8 * (p % PPR);
        u32x4_t o;
        if (d0 < NOPE) {
          const u32x2_t w = *(const u32x2_t*)(rawc + rr * raw_rb + d0);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], false);
            const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[h], true);
            o[2 * h] = pack2_bf16_hw(lo[0], lo[1]);
            o[2 * h + 1] = pack2_bf16_hw(hi[0], hi[1]);
          }
        } else {
          o = *(const u32x4_t*)(rawc + rr * raw_rb + NOPE + 2 * (d0 - NOPE));
        }
        *(u32x4_t*)(convb + rr * RBP + 2 * d0) = o;
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const f32x4_t v = *(const f32x4_t*)(&sscale[MQ_CH * c + 16 * kt + 4 * g]);
#pragma unroll
        for (int r = 0; r < 4; ++r) skey[kt][r] = v[r];
      }
      if (c + 1 < nch && PF >= 2) lds_sync<(PF >= 2 ? RPW : 0)>();
      else lds_sync<0>();
      kb = convb;
    }

    // S^T: 32 keys x 16 HTW heads over all D dims.  The key operands stream in
    // groups of four K-steps (both key tiles); a group's LDS reads are issued
    // before the previous group's MFMAs, so their latency hides behind them.
    f32x4_t S[2][HTW];
    f32x4_t Sr[2][MIX ? HTW : 1];   // mixed rows: the rotated dims' share of the scores
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int ht = 0; ht < HTW; ++ht) {
        S[kt][ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if constexpr (MIX) Sr[kt][ht] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      }
    constexpr int NGRP = KS / 4;
    static_assert(KS % 4 == 0, "K-steps in groups of four");
    bf16x8_t ka[2][8];
#pragma unroll
    for (int grp = 0; grp <= NGRP; ++grp) {
      if (grp < NGRP) {
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            ka[grp & 1][2 * u + kt] =
                *(const bf16x8_t*)(kb + (16 * kt + j) * RBP + 16 * ((D / 32) * g + 4 * grp + u));
      }
      __builtin_amdgcn_sched_barrier(0);
      if (grp > 0) {
        const int pg = grp - 1;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int ht = 0; ht < HTW; ++ht) {
              S[kt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[pg & 1][2 * u + kt], qf[ht][4 * pg + u],
                                                                  S[kt][ht], 0, 0, 0);
              if constexpr (MIX) {
                // the rotated dims' share alone: the query with every other dim zeroed
                // (lane group 3 holds the last quarter of the dims, the rotated ones
                // from K-step MIX_KS0 on)
                if (4 * pg + u >= MIX_KS0) {
                  const bf16x8_t qr = g == 3 ? qf[ht][4 * pg + u] : bf16x8_t{};
                  Sr[kt][ht] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[pg & 1][2 * u + kt], qr, Sr[kt][ht],
                                                                       0, 0, 0);
                }
              }
            }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MIX) {
      // score = s_key * (code share) + rotated share; the code share is the whole
      // fp32 sum minus the rotated one (fp32 sums: far below the bf16 inputs' precision)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ht = 0; ht < HTW; ++ht)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            S[kt][ht][r] = skey[kt][r] * (S[kt][ht][r] - Sr[kt][ht][r]) + Sr[kt][ht][r];
    }
    // the next chunk into the slot that chunk c - 1 left (every wave is past it);
    // issued after the scores, so a full load queue cannot hold them up
    if (c + PF < nch)
      dec_issue<D, NW>(c + PF, sptr, kv + ((c + PF) % MQ_DEC_NBUF) * MQ_CH * raw_rb, wave, lane, raw_cpr, raw_rb);

    // online softmax per head; the reference only moves when a chunk maximum
    // exceeds it by MQ_REF_SLACK, so O is rarely rescaled
    float alpha[HTW];
    bool moved = false;
    // FULL: every slot of the chunk exists (the common case), so no score is
    // masked and every score is finite: the per-score mask and -inf tests drop out
    auto softmax = [&](auto full_c) {
      constexpr bool FULL = decltype(full_c)::value;
#pragma unroll
      for (int ht = 0; ht < HTW; ++ht) {
        float cm = -INFINITY;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            if constexpr (FULL) {
              S[kt][ht][r] *= sc[ht];
            } else {
              const bool ok = (vmask >> (16 * kt + 4 * g + r)) & 1u;
              S[kt][ht][r] = ok ? S[kt][ht][r] * sc[ht] : -INFINITY;
            }
            cm = fmaxf(cm, S[kt][ht][r]);
          }
        cm = quad_max(cm);
        const float nr = (cm > ref[ht] + MQ_REF_SLACK) ? cm : ref[ht];
        alpha[ht] = (nr == ref[ht]) ? 1.f : (ref[ht] == -INFINITY ? 0.f : __expf(ref[ht] - nr));
        // while the reference is -inf every P so far was 0 and O is still 0
        moved |= nr != ref[ht] && ref[ht] != -INFINITY;
        float ps = 0.f;
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float e = (!FULL && S[kt][ht][r] == -INFINITY) ? 0.f : __expf(S[kt][ht][r] - nr);
            S[kt][ht][r] = e;
            ps += e;
          }
        // this lane's share of the head's sum; the four shares add up after the loop
        lsum[ht] = lsum[ht] * alpha[ht] + ps;
        ref[ht] = nr;
      }
    };
    if (vmask == 0xFFFFFFFFu) softmax(std::true_type{});
    else softmax(std::false_type{});
    if (__any(moved)) {
      // Rare (a chunk maximum passed the reference by MQ_REF_SLACK).  O is scaled
      // through this wave's LDS scratch, eight tiles at a time, so that on the
      // common path it only ever feeds the matrix cores and stays in AGPRs.
      f32x4_t* tw = rs_tmp + wave * 8 * 64;
#pragma unroll
      for (int ht = 0; ht < HTW; ++ht) {
        float a4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) a4[r] = __shfl(alpha[ht], 4 * g + r, 64);
#pragma unroll
        for (int n0 = 0; n0 < NT; n0 += 8) {
#pragma unroll
          for (int u = 0; u < 8; ++u) tw[u * 64 + lane] = O[ht][n0 + u];
          asm volatile("" ::: "memory");
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            f32x4_t v = tw[u * 64 + lane];
            v[0] *= a4[0];
            v[1] *= a4[1];
            v[2] *= a4[2];
            v[3] *= a4[3];
            tw[u * 64 + lane] = v;
          }
          asm volatile("" ::: "memory");
#pragma unroll
          for (int u = 0; u < 8; ++u) O[ht][n0 + u] = tw[u * 64 + lane];
          asm volatile("" ::: "memory");
        }
      }
    }
    bf16x8_t pf[HTW];
    bf16x8_t pfs[MIX ? HTW : 1];   // mixed rows: p times its key's scale, for the code dims
#pragma unroll
    for (int ht = 0; ht < HTW; ++ht) {
      u32x4_t pw;
      pw[0] = pack2_bf16_hw(S[0][ht][0], S[0][ht][1]);
      pw[1] = pack2_bf16_hw(S[0][ht][2], S[0][ht][3]);
      pw[2] = pack2_bf16_hw(S[1][ht][0], S[1][ht][1]);
      pw[3] = pack2_bf16_hw(S[1][ht][2], S[1][ht][3]);
      pf[ht] = __builtin_bit_cast(bf16x8_t, pw);
      if constexpr (MIX) {
        pw[0] = pack2_bf16_hw(S[0][ht][0] * skey[0][0], S[0][ht][1] * skey[0][1]);
        pw[1] = pack2_bf16_hw(S[0][ht][2] * skey[0][2], S[0][ht][3] * skey[0][3]);
        pw[2] = pack2_bf16_hw(S[1][ht][0] * skey[1][0], S[1][ht][1] * skey[1][1]);
        pw[3] = pack2_bf16_hw(S[1][ht][2] * skey[1][2], S[1][ht][3] * skey[1][3]);
        pfs[ht] = __builtin_bit_cast(bf16x8_t, pw);
      }
    }
    // P.V: V read transposed (keys 4g..4g+3 and 16+4g..16+4g+3 of column j of each tile)
    const uint32_t b0 = lds_addr(kb) + tr0 * RBP + 8 * (j & 3);
    const uint32_t b1 = lds_addr(kb) + tr1 * RBP + 8 * (j & 3);
    // sixteen tiles per wait where the registers allow (one head tile), else eight
    constexpr int TPW = (HTW == 1 && NT % 16 == 0) ? 16 : 8;
#pragma unroll
    for (int mb = 0; mb < NT / TPW; ++mb) {
      u32x2_t vr[2 * TPW];
      if constexpr (TPW == 16) lds_read_tr32(b0 + 512 * mb, b1 + 512 * mb, vr);
      else lds_read_tr16(b0 + 256 * mb, b1 + 256 * mb, vr);
#pragma unroll
      for (int u = 0; u < TPW; ++u) {
        const u32x4_t vw = {vr[2 * u][0], vr[2 * u][1], vr[2 * u + 1][0], vr[2 * u + 1][1]};
        const bf16x8_t vf = __builtin_bit_cast(bf16x8_t, vw);
#pragma unroll
        for (int ht = 0; ht < HTW; ++ht) {
          const bool code_tile = MIX && 16 * (TPW * mb + u) < NOPE;
          O[ht][TPW * mb + u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(code_tile ? pfs[MIX ? ht : 0] : pf[ht], vf,
                                                                        O[ht][TPW * mb + u], 0, 0, 0);
        }
      }
    }
  }

#pragma unroll
  for (int ht = 0; ht < HTW; ++ht) lsum[ht] = quad_sum(lsum[ht]);

  // ---- output: lane (g, j) of tile (ht, nt) holds heads h0 + 16 ht + 4 g + r, dim 16 nt + j.
  // Unsplit, the output row: O times the head's final factor, rotated at -i,
  // as bf16.  Split, the partial: O divided by the head's sum, as fp16, then
  // the (max, sum) pair.  Either goes out through LDS, so that every store
  // writes a whole 16-byte piece of one head's row (straight from the MFMA
  // layout a store instruction would write 32-byte pieces of four rows).  A
  // wave stages 16 heads x CW dims at a time (rows padded by 4 floats, so the
  // four lane groups hit distinct banks) in its own part of the chunk ring and
  // reads them back 8 dims per lane.
  const bool fin = n_split == 1;
  float fac[HTW];   // factor of head 16 ht + j
#pragma unroll
  for (int ht = 0; ht < HTW; ++ht) {
    if (fin) {
      const float sig = sink ? sink[h0 + 16 * ht + j] : -INFINITY;
      const float M = fmaxf(ref[ht], sig);
      float Z = 0.f;
      if (ref[ht] != -INFINITY) Z += lsum[ht] * __expf(ref[ht] - M);
      if (sig != -INFINITY) Z += __expf(sig - M);
      fac[ht] = (Z > 0.f && ref[ht] != -INFINITY) ? __expf(ref[ht] - M) / Z : 0.f;
    } else {
      fac[ht] = part_inv(lsum[ht]);
    }
  }
  {
    constexpr int CW = D >= 512 ? 256 : D / 2;   // dims per staged block
    constexpr int CRS = CW + 4;                  // staged row stride (floats)
    constexpr int LPH = CW / 8;                  // lanes per head row on the way out
    // (mixed rows: the host sizes the dynamic LDS to hold the staging as well)
    static_assert(MIX || 16 * CRS * 4 * NW <= MQ_DEC_NBUF * CHB, "staging fits the chunk ring");
    lds_sync<0>();   // every wave is done with the chunk ring
    float* stg = (float*)kv + wave * 16 * CRS;
    float pscale[HTW];   // split partials: scale of head 16 ht + j
    // FIN: compile-time copy of fin (one store loop each)
    auto write_out = [&](auto fin_c) {
      constexpr bool FIN = decltype(fin_c)::value;
      const size_t pb = FIN ? row * n_h + h0 : (row * n_split + sp) * (size_t)n_h + h0;
      uint16_t* dst = FIN ? out : (uint16_t*)part_o(ws);
#pragma unroll
      for (int ht = 0; ht < HTW; ++ht) {
        float fr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) fr[r] = __shfl(fac[ht], 4 * g + r, 64);
        if constexpr (!FIN) {
          // partial rows: scaled by a power of two from the row maximum (head 4 g + r:
          // the 16 lanes of group g hold all its dims); lane (0, j) keeps the scale of
          // head 16 ht + j for the record
          float sc[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float a = 0.f;
#pragma unroll
            for (int nt = 0; nt < D / 16; ++nt) a = fmaxf(a, fabsf(O[ht][nt][r] * fr[r]));
#pragma unroll
            for (int x = 1; x < 16; x <<= 1) a = fmaxf(a, __shfl_xor(a, x, 64));
            sc[r] = part_scale(a);
            fr[r] *= sc[r];
          }
          const int src = 16 * (j >> 2);
          const float s0 = __shfl(sc[0], src, 64), s1 = __shfl(sc[1], src, 64);
          const float s2 = __shfl(sc[2], src, 64), s3 = __shfl(sc[3], src, 64);
          pscale[ht] = (j & 3) == 0 ? s0 : (j & 3) == 1 ? s1 : (j & 3) == 2 ? s2 : s3;
        }
#pragma unroll
        for (int cb = 0; cb < D / CW; ++cb) {
#pragma unroll
          for (int nt = 0; nt < CW / 16; ++nt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              stg[(4 * g + r) * CRS + 16 * nt + j] = O[ht][cb * (CW / 16) + nt][r] * fr[r];
          // the writes of every lane land before any lane reads (and the reads below
          // finish before the next block's writes: their stores consume them first)
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
          asm volatile("" ::: "memory");
#pragma unroll
          for (int it = 0; it < 16 * CW / 512; ++it) {
            const int f = it * 64 + lane;   // 8-value piece of the 16 x CW block
            const int hh = f / LPH, c8 = f % LPH;
            const int d0 = cb * CW + 8 * c8;
            const f32x4_t v0 = *(const f32x4_t*)(stg + hh * CRS + 8 * c8);
            const f32x4_t v1 = *(const f32x4_t*)(stg + hh * CRS + 8 * c8 + 4);
            const float v[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
            u32x4_t pk;
            if constexpr (FIN) {
              // rotation at -i of the pairs (2u, 2u + 1): cos(-x) = cos x, sin(-x) = -sin x
              // ((1, 0) outside the rotated dims)
              const f32x4_t ra = *(const f32x4_t*)&rope_cs[d0], rb = *(const f32x4_t*)&rope_cs[d0 + 4];
              const float rc[8] = {ra[0], ra[1], ra[2], ra[3], rb[0], rb[1], rb[2], rb[3]};
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const float a = v[2 * e], bb = v[2 * e + 1], cs = rc[2 * e], sn = rc[2 * e + 1];
                pk[e] = (uint32_t)f32_to_bf16_bits(a * cs + bb * sn) |
                        ((uint32_t)f32_to_bf16_bits(bb * cs - a * sn) << 16);
              }
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                pk[e] = (uint32_t)__builtin_bit_cast(uint16_t, part_h(v[2 * e])) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, part_h(v[2 * e + 1])) << 16);
            }
            *(u32x4_t*)(dst + (pb + 16 * ht + hh) * D + d0) = pk;
          }
          asm volatile("" ::: "memory");
        }
      }
    };
    if (fin) write_out(std::true_type{});
    else write_out(std::false_type{});
    if (!fin) {
      const size_t pbs = (row * n_split + sp) * (size_t)n_h + h0;
      if (g == 0) {
        float* ml = part_ml(ws, n_units, n_h, D);
#pragma unroll
        for (int ht = 0; ht < HTW; ++ht)
          *(f32x4_t*)(ml + 4 * (pbs + 16 * ht + j)) = f32x4_t{ref[ht], lsum[ht], part_unscale(pscale[ht]), 0.f};
      }
    }
  }
}

// merge the split partial states of one (query, head): first the maximum M of
// every split's m (and the sink), then split s weighed by l_s exp(m_s - M) (its
// row holds O_s / l_s times 1 / u_s), summed in split order.  A block of CB
// splits' partials is loaded at once (one memory round trip for up to CB
// splits).  Lane l of each wave reads the record of split s0 + l % CB and
// forms its weight; readlane hands the weights to every lane.  Thread u owns
// output dims 2u, 2u + 1 (the launcher keeps D / 2 <= blockDim); every thread
// runs the split loop, so the wave reductions see full waves.
template <int CB>
__global__ __launch_bounds__(256) void mqa_combine_kernel(
    const float* __restrict__ ws, const float* __restrict__ sink, const int* __restrict__ q_pos,
    int Tq, int n_h, int D, int n_split, int rope_dim, RopeRatio rope, uint16_t* __restrict__ out) {
  static_assert(CB == 8 || CB == 64, "a block is a power of two of lanes");
  const int h = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const size_t row = (size_t)b * Tq + t;
  const long long i = q_pos[row];
  const float sig = sink ? sink[h] : -INFINITY;
  const _Float16* base = part_o(ws) + (row * n_split * (size_t)n_h + h) * D;   // O / l of split 0
  const size_t sstride = (size_t)n_h * D;
  const float* mlb = part_ml(ws, (long long)gridDim.z * Tq * n_split, n_h, D) + 4 * (row * n_split * (size_t)n_h + h);
  const size_t mstride = 4 * (size_t)n_h;
  const int rbeg = D - rope_dim;
  const bool has = (int)threadIdx.x < D / 2;
  const int d0 = has ? 2 * (int)threadIdx.x : 0;
  // every partial of a block in flight at once: unconditional loads (split index
  // clamped; the extra ones get weight 0), since a guarded load becomes a branch
  // with its own wait.  The first block's loads go out with the maximum's.
  uint32_t w[CB];
  auto load_block = [&](int s0) {
#pragma unroll
    for (int s = 0; s < CB; ++s) w[s] = *(const uint32_t*)(base + (size_t)min(s0 + s, n_split - 1) * sstride + d0);
  };
  load_block(0);
  // M over the splits and the sink.  The first 64 splits' whole records come
  // with it: for lanes below CB they are the first block's records below (lane
  // l holds split l), so that block needs no second, dependent load.
  float M = sig;
  f32x4_t rec0;
  for (int s0 = 0; s0 < n_split; s0 += 64) {
    const int sl = s0 + lane;
    const f32x4_t r = *(const f32x4_t*)(mlb + (size_t)min(sl, n_split - 1) * mstride);
    if (s0 == 0) rec0 = r;
    M = fmaxf(M, wave_reduce_f<true>(sl < n_split ? r[0] : -INFINITY));
  }
  float Z = (sig != -INFINITY) ? __expf(sig - M) : 0.f, o0 = 0.f, o1 = 0.f;
  for (int s0 = 0; s0 < n_split; s0 += CB) {
    if (s0 > 0) load_block(s0);
    const int sl = s0 + (lane & (CB - 1));
    const f32x4_t rec = s0 == 0 ? rec0 : *(const f32x4_t*)(mlb + (size_t)min(sl, n_split - 1) * mstride);
    const float f = (sl < n_split && rec[0] != -INFINITY) ? rec[1] * __expf(rec[0] - M) : 0.f;
    Z += wave_reduce_f<false>(lane < CB ? f : 0.f);
    const float gl = f * rec[2];
#pragma unroll
    for (int s = 0; s < CB; ++s) {
      const float gs = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(gl), s));
      o0 += (float)__builtin_bit_cast(_Float16, (uint16_t)(w[s] & 0xffffu)) * gs;
      o1 += (float)__builtin_bit_cast(_Float16, (uint16_t)(w[s] >> 16)) * gs;
    }
  }
  if (!has) return;
  const float inv = Z > 0.f ? 1.f / Z : 0.f;
  o0 *= inv;
  o1 *= inv;
  if (d0 >= rbeg) {
    float cs, sn;
    rope_cos_sin(-i, (d0 - rbeg) >> 1, rope, &cs, &sn);
    const float r0 = o0 * cs - o1 * sn, r1 = o0 * sn + o1 * cs;
    o0 = r0;
    o1 = r1;
  }
  const size_t ob = (row * n_h + h) * (size_t)D + d0;   // even: D is
  if ((((uintptr_t)out) & 3u) == 0) {
    *(uint32_t*)(out + ob) = (uint32_t)f32_to_bf16_bits(o0) | ((uint32_t)f32_to_bf16_bits(o1) << 16);
  } else {
    out[ob] = f32_to_bf16_bits(o0);
    out[ob + 1] = f32_to_bf16_bits(o1);
  }
}

// the combine launch: blocks of 8 splits up to 8, else of 64
static void launch_combine(const MqaArgs& a, int n_split, hipStream_t st) {
  const RopeRatio rope_rr = rope_ratio(a.rope_dim, a.rope_base);
  auto kfn = n_split <= 8 ? mqa_combine_kernel<8> : mqa_combine_kernel<64>;
  hipLaunchKernelGGL(kfn, dim3((unsigned)a.n_h, (unsigned)a.Tq, (unsigned)a.B), dim3(256), 0, st,
                     (const float*)a.ws, a.sink, a.q_pos, a.Tq, a.n_h, a.d, n_split, a.rope_dim, rope_rr,
                     (uint16_t*)a.out);
}

// ---------------------------------------------------------------------------
// dispatch
// ---------------------------------------------------------------------------
// the MFMA kernels read q, the entries and the window rows and write the
// output in 16-byte pieces
static bool mqa_aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool mqa_mfma_ok(const MqaArgs& a) {
  return (a.dtype == DT_BF16 || a.dtype == DT_MIX) && (a.d == 128 || a.d == 256 || a.d == 512) && a.n_h % 16 == 0 &&
         mqa_aligned16(a.q) && mqa_aligned16(a.E) && mqa_aligned16(a.W) && mqa_aligned16(a.out);
}

long long mqa_slots_max(const MqaArgs& a) {
  return (a.idx ? (long long)a.k : a.N_cap) + a.n_win;
}

// Head tiles (16 heads each) per wave of the streaming kernel.  Below D = 512
// the output accumulators of two tiles fit the register file next to the query
// fragments.  At D = 512 two tiles fill it (a few prologue values spill, none
// in the loop): prefill takes them, since each chunk read from LDS then feeds
// twice the heads and those reads bound the loop; decode keeps one tile and so
// twice the workgroups.
static int dec_htw(int Tq, int n_h, int d) {
  if (d < 512) return 2;
  return (Tq >= MQ_SPLIT_BELOW_TQ && n_h % 32 == 0) ? 2 : 1;
}

// the streaming kernel (mqa_decode_kernel) covers the shape: decode splits a
// query's slots over workgroups, prefill gives each query one range
static bool mqa_decode_ok(int Tq, int n_h, int d) {
  return n_h % (16 * dec_htw(Tq, n_h, d)) == 0;
}

// slots per workgroup and splits per query; depends on the shape only, never on B
static void mqa_split(int Tq, int n_h, int d, long long slots_max, int* kps, int* n_split) {
  if (mqa_decode_ok(Tq, n_h, d)) {
    if (Tq < MQ_SPLIT_BELOW_TQ) {
      // as many ranges as ranges of the nominal length take, each as long as a
      // balanced share rounded up to whole chunks (640 slots: 4 of 160, not
      // 3 of 192 and one of 64)
      const long long nom = slots_max <= MQ_DEC_SMALL_UPTO ? MQ_DEC_SPLIT_SMALL : MQ_DEC_SPLIT_LONG;
      const long long nsp = max(1LL, (slots_max + nom - 1) / nom);
      const long long share = (slots_max + nsp - 1) / nsp;
      *kps = (int)max((long long)MQ_CH, (share + MQ_CH - 1) / MQ_CH * MQ_CH);
    } else
      *kps = (int)min((long long)MQ_DEC_TABLE, max(1LL, (slots_max + MQ_CH - 1) / MQ_CH) * MQ_CH);
    *n_split = (int)max(1LL, (slots_max + *kps - 1) / *kps);
  } else if (Tq >= MQ_SPLIT_BELOW_TQ || slots_max <= MQ_SPLIT_KEYS) {
    long long s = ((slots_max + MQ_CH - 1) / MQ_CH) * MQ_CH;
    if (s > 2147483647LL) s = 2147483647LL;
    *kps = (int)(s > 0 ? s : MQ_CH);
    *n_split = 1;
  } else {
    *kps = MQ_SPLIT_KEYS;
    *n_split = (int)((slots_max + MQ_SPLIT_KEYS - 1) / MQ_SPLIT_KEYS);
  }
}

size_t mqa_workspace_bytes(int B, int Tq, int n_h, int d, long long n_slots_max, int dtype) {
  if (!((dtype == DT_BF16 || dtype == DT_MIX) && (d == 128 || d == 256 || d == 512) && n_h % 16 == 0)) return 0;
  int kps, n_split;
  mqa_split(Tq, n_h, d, n_slots_max, &kps, &n_split);
  if (n_split == 1) return 0;
  // per (query row, split, head): d fp16 outputs + a float record (max, sum, 1 / scale, 0)
  return (size_t)B * Tq * n_split * n_h * (size_t)(2 * d + 16);
}

template <int D, bool DENSE, bool MULTI>
static void launch_mfma_v(const MqaArgs& a, int kps, int n_split, hipStream_t st) {
  const RopeRatio rope_rr = rope_ratio(a.rope_dim, a.rope_base);
  const int n_hg = (a.n_h + 63) / 64;
  const long long units = (long long)a.B * a.Tq * n_split;
  const long long blocks = ((units + 7) / 8) * 8 * n_hg;
  const size_t lds = (size_t)MQ_GROUP * D * 2;
  auto kfn = MULTI ? mqa_mfma_kernel<D, DENSE, true> : mqa_group_kernel<D, DENSE>;
  if (lds > 65536)
    (void)hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kfn, dim3((unsigned)blocks), dim3(256), lds, st,
                     (const uint16_t*)a.q, a.gamma_q, a.eps, (const uint16_t*)a.E, a.N_cap, a.idx,
                     a.k, a.m, (const uint16_t*)a.W, a.W_cap, a.n_win, a.sink, a.q_pos, a.Tq, a.n_h,
                     a.rope_dim, rope_rr, a.scale, kps, n_split, units, (uint16_t*)a.out,
                     (float*)a.ws);
  if (n_split > 1) launch_combine(a, n_split, st);
}

// dynamic LDS of the streaming kernel: the chunk ring (raw mixed rows plus the
// widened chunk for mixed entries) and, reusing it, the output staging
template <int D, int NW, bool MIX>
static size_t decode_lds_bytes() {
  const size_t bf_row = 2 * D + 16;
  if (!MIX) return (size_t)MQ_DEC_NBUF * MQ_CH * bf_row;
  const size_t ring = (size_t)MQ_DEC_NBUF * MQ_CH * (D + MQ_MIX_ROPE + 16) + MQ_CH * bf_row;
  constexpr int CW = D >= 512 ? 256 : D / 2;
  const size_t stage = (size_t)16 * (CW + 4) * 4 * NW;
  return ring > stage ? ring : stage;
}

template <int D, bool DENSE, int NW, int HTW, bool MIX>
static void launch_decode_nw(const MqaArgs& a, int kps, int n_split, hipStream_t st) {
  const RopeRatio rope_rr = rope_ratio(a.rope_dim, a.rope_base);
  const int n_hg = a.n_h / (16 * HTW * NW);
  const long long units = (long long)a.B * a.Tq * n_split;
  const long long blocks = ((units + 7) / 8) * 8 * n_hg;
  const size_t lds = decode_lds_bytes<D, NW, MIX>();
  // the small slot table for decode ranges (<= 192 slots), the large one for prefill
  auto kfn = kps <= MQ_DEC_TBL_SMALL ? mqa_decode_kernel<D, DENSE, NW, MQ_DEC_TBL_SMALL, HTW, MIX>
                                     : mqa_decode_kernel<D, DENSE, NW, MQ_DEC_TABLE, HTW, MIX>;
  if (lds > 65536)
    (void)hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL(kfn, dim3((unsigned)blocks), dim3(64 * NW), lds, st,
                     (const uint16_t*)a.q, a.gamma_q, a.eps, (const uint16_t*)a.E, a.N_cap, a.idx,
                     a.k, a.m, (const uint16_t*)a.W, a.W_cap, a.n_win, a.sink, a.q_pos, a.Tq, a.n_h,
                     a.rope_dim, rope_rr, a.scale, kps, n_split, units, (uint16_t*)a.out,
                     (float*)a.ws, a.E_scale, a.W_scale);
  if (n_split > 1) launch_combine(a, n_split, st);
}

// waves per workgroup: as many head groups of one wave as divide n_h, up to four
template <int D, bool DENSE, int HTW, bool MIX>
static void launch_decode_w(const MqaArgs& a, int kps, int n_split, hipStream_t st) {
  constexpr int HW = 16 * HTW;
  if (a.n_h % (4 * HW) == 0) launch_decode_nw<D, DENSE, 4, HTW, MIX>(a, kps, n_split, st);
  else if (a.n_h % (2 * HW) == 0) launch_decode_nw<D, DENSE, 2, HTW, MIX>(a, kps, n_split, st);
  else launch_decode_nw<D, DENSE, 1, HTW, MIX>(a, kps, n_split, st);
}
template <int D, bool DENSE, bool MIX>
static void launch_decode(const MqaArgs& a, int kps, int n_split, hipStream_t st) {
  if constexpr (MIX) {
    // mixed rows keep one head tile per wave: with two, the second score and
    // weight sets they need do not fit the registers
    launch_decode_w<D, DENSE, 1, MIX>(a, kps, n_split, st);
  } else {
    if constexpr (D >= 512) {
      if (dec_htw(a.Tq, a.n_h, D) == 1) {
        launch_decode_w<D, DENSE, 1, MIX>(a, kps, n_split, st);
        return;
      }
    }
    launch_decode_w<D, DENSE, 2, MIX>(a, kps, n_split, st);
  }
}

template <int D, bool DENSE>
static void launch_mfma_d(const MqaArgs& a, int kps, int n_split, hipStream_t st) {
  if constexpr (D == 512) {
    if (a.dtype == DT_MIX) {
      launch_decode<D, DENSE, true>(a, kps, n_split, st);
      return;
    }
  }
  if (mqa_decode_ok(a.Tq, a.n_h, a.d)) launch_decode<D, DENSE, false>(a, kps, n_split, st);
  else if (kps <= MQ_GROUP) launch_mfma_v<D, DENSE, false>(a, kps, n_split, st);
  else launch_mfma_v<D, DENSE, true>(a, kps, n_split, st);
}

int launch_mqa(const MqaArgs& a, hipStream_t st, const char** why) {
  const RopeRatio rope_rr = rope_ratio(a.rope_dim, a.rope_base);
  const bool dense = a.idx == nullptr;
  const long long slots_max = mqa_slots_max(a);
  if (a.dtype == DT_MIX) {
    // mixed rows: the streaming kernel only
    if (a.d != 512 || !mqa_mfma_ok(a) || !mqa_decode_ok(a.Tq, a.n_h, a.d)) {
      *why = "mixed-precision entries need d = 512, n_h a multiple of 16 and 16-byte aligned q, E, W and out";
      return 4;
    }
    if (a.rope_dim != MQ_MIX_ROPE) {
      *why = "mixed-precision entries need rope_dim = 64 (the bf16 part of the row)";
      return 4;
    }
  }
  if (mqa_mfma_ok(a)) {
    int kps, n_split;
    mqa_split(a.Tq, a.n_h, a.d, slots_max, &kps, &n_split);
    if (n_split > 1 && a.ws_bytes < mqa_workspace_bytes(a.B, a.Tq, a.n_h, a.d, slots_max, a.dtype)) {
      *why = "workspace smaller than csa_mqa_workspace_size()";
      return 5;
    }
    if (n_split > 1 && ((uintptr_t)a.ws & 15u) != 0) {
      *why = "workspace must be 16-byte aligned";
      return 5;
    }
    if (mqa_decode_ok(a.Tq, a.n_h, a.d) &&
        (((long long)a.B * a.Tq * n_split + 7) / 8) * 8 * (a.n_h / 16) > 2147483647LL) {
      *why = "decode attention: more (query, split, head group) units than one grid holds";
      return 4;
    }
#define CSA_MQA_D(DV)                                                  \
  do {                                                                 \
    if (dense) launch_mfma_d<DV, true>(a, kps, n_split, st);           \
    else launch_mfma_d<DV, false>(a, kps, n_split, st);                \
  } while (0)
    if (a.d == 128) CSA_MQA_D(128);
    else if (a.d == 256) CSA_MQA_D(256);
    else CSA_MQA_D(512);
#undef CSA_MQA_D
  } else {
    if (slots_max > VALU_MAX_SLOTS) {
      *why = "the generic (fp32 / unaligned-shape) attention path holds at most 8192 key slots";
      return 4;
    }
    const size_t lds = (size_t)(a.d + 4 + VALU_MAX_SLOTS) * sizeof(float) + VALU_MAX_SLOTS * sizeof(long long);
    dim3 grid((unsigned)a.n_h, (unsigned)a.Tq, (unsigned)a.B);
#define CSA_MQA_VALU(DT, DN)                                                                        \
  do {                                                                                              \
    auto kfn = mqa_valu_kernel<DT, DN>;                                                             \
    if (hipFuncSetAttribute((const void*)kfn, hipFuncAttributeMaxDynamicSharedMemorySize,           \
                            (int)lds) != hipSuccess) {                                              \
      *why = "cannot reserve LDS for the generic attention kernel";                                 \
      return 6;                                                                                     \
    }                                                                                               \
    hipLaunchKernelGGL(kfn, grid, dim3(256), lds, st, a.q, a.gamma_q, a.eps, a.E, a.N_cap, a.idx, \
                       a.k, a.m, a.W, a.W_cap, a.n_win, a.sink, a.q_pos, a.Tq, a.n_h, a.d,          \
                       a.rope_dim, rope_rr, a.scale, a.out);                                    \
  } while (0)
    if (a.dtype == DT_F32) {
      if (dense) CSA_MQA_VALU(DT_F32, true); else CSA_MQA_VALU(DT_F32, false);
    } else {
      if (dense) CSA_MQA_VALU(DT_BF16, true); else CSA_MQA_VALU(DT_BF16, false);
    }
#undef CSA_MQA_VALU
  }
  if (hipGetLastError() != hipSuccess) {
    *why = "kernel launch failed";
    return 6;
  }
  return 0;
}

}  // namespace csa
