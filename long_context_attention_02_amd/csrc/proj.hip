// Grouped output projection of the attention outputs, for gfx950.
//
// DeepSeek-V4 method page, section 3.3: because c * n_h (all heads' outputs
// side by side) is large, the output projection is grouped -- each group of
// heads is projected down to d_g, the group results are concatenated and
// projected back to d.  Both stages are products C = A B^T of bf16 matrices
// with the contraction axis contiguous in both operands (the weights are
// output-major): stage 1 is a batch over the groups (group q reads columns
// [q W, (q+1) W) of the head outputs, W = n_h c / g, and writes columns
// [q d_g, (q+1) d_g) of the intermediate), stage 2 a single product.
//
// gemm_nt_kernel: a workgroup of four waves owns a BM x BN tile of C and walks
// K in steps of 64 through double-buffered LDS (rows padded by 16 bytes, so the
// 16 rows a lane group reads fall on distinct banks); each wave owns a
// (BM / WGM) x (BN / (4 / WGM)) sub-tile of 16 x 16 v_mfma_f32_16x16x32_bf16
// tiles.  Lane (g, j) feeds row j, dims 8 g .. 8 g + 7 of each 32-wide K step
// for both operands and receives C rows 4 g + r, column j.  Few rows (decode)
// take 16-row tiles and split K over workgroups; the splits write fp32
// partials that gemm_reduce_kernel sums in split order (deterministic).
#include <algorithm>

#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

static constexpr int GEMM_BK = 64;

template <int BM, int BN, int WGM>
__global__ __launch_bounds__(256) void gemm_nt_kernel(
    const uint16_t* __restrict__ A, long long lda, long long sA, const uint16_t* __restrict__ B,
    long long ldb, long long sB, uint16_t* __restrict__ C, long long ldc, long long sC,
    float* __restrict__ part, int M, int N, int K, int ksplit) {
  constexpr int BK = GEMM_BK;
  constexpr int WGN = 4 / WGM;
  constexpr int WM = BM / WGM, WN = BN / WGN;   // per-wave tile
  constexpr int TM = WM / 16, TN = WN / 16;     // 16 x 16 MFMA tiles per wave
  constexpr int RS = BK * 2 + 16;               // LDS row stride in bytes
  constexpr int PA = (BM * 8 + 255) / 256;      // 16-byte pieces of the A tile per thread
  constexpr int PB = (BN * 8 + 255) / 256;
  static_assert(TM >= 1 && TN >= 1, "a wave owns whole 16 x 16 tiles");
  __shared__ __attribute__((aligned(16))) uint8_t As[2][BM * RS];
  __shared__ __attribute__((aligned(16))) uint8_t Bs[2][BN * RS];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = lane >> 4, j = lane & 15;
  const int wm = wave / WGN, wn = wave % WGN;
  const int batch = blockIdx.z / ksplit, split = blockIdx.z % ksplit;
  const int m0 = blockIdx.y * BM, n0 = blockIdx.x * BN;
  A += (size_t)batch * (size_t)sA;
  B += (size_t)batch * (size_t)sB;
  // the K range of this split (whole 64-wide steps)
  const int nk_all = K / BK;
  const int k_lo = (int)((long long)nk_all * split / ksplit), k_hi = (int)((long long)nk_all * (split + 1) / ksplit);

  u32x4_t ra[PA], rb[PB];
  // rows past M (N) read row M - 1 (N - 1): their results are never stored
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int u = 0; u < PA; ++u) {
      const int p = threadIdx.x + 256 * u;
      const int r = min(p / 8, BM - 1), c = p % 8;
      const int row = min(m0 + r, M - 1);
      ra[u] = *(const u32x4_t*)(A + (size_t)row * (size_t)lda + k0 + 8 * c);
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int p = threadIdx.x + 256 * u;
      const int r = min(p / 8, BN - 1), c = p % 8;
      const int row = min(n0 + r, N - 1);
      rb[u] = *(const u32x4_t*)(B + (size_t)row * (size_t)ldb + k0 + 8 * c);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int u = 0; u < PA; ++u) {
      const int p = threadIdx.x + 256 * u;
      if (p < BM * 8) *(u32x4_t*)(&As[buf][(p / 8) * RS + 16 * (p % 8)]) = ra[u];
    }
#pragma unroll
    for (int u = 0; u < PB; ++u) {
      const int p = threadIdx.x + 256 * u;
      if (p < BN * 8) *(u32x4_t*)(&Bs[buf][(p / 8) * RS + 16 * (p % 8)]) = rb[u];
    }
  };

  f32x4_t acc[TM][TN];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  if (k_lo < k_hi) {
    gload(k_lo);
    lstore(0);
  }
  __syncthreads();
  for (int kt = k_lo; kt < k_hi; ++kt) {
    const int buf = (kt - k_lo) & 1;
    if (kt + 1 < k_hi) gload(kt + 1);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8_t af[TM], bfr[TN];
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
        af[tm] = *(const bf16x8_t*)(&As[buf][(wm * WM + 16 * tm + j) * RS + 2 * (32 * ks + 8 * g)]);
#pragma unroll
      for (int tn = 0; tn < TN; ++tn)
        bfr[tn] = *(const bf16x8_t*)(&Bs[buf][(wn * WN + 16 * tn + j) * RS + 2 * (32 * ks + 8 * g)]);
#pragma unroll
      for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int tn = 0; tn < TN; ++tn)
          acc[tm][tn] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tm], bfr[tn], acc[tm][tn], 0, 0, 0);
    }
    if (kt + 1 < k_hi) lstore(buf ^ 1);
    __syncthreads();
  }

  // lane (g, j) of tile (tm, tn): C rows m0 + wm WM + 16 tm + 4 g + r, column n0 + wn WN + 16 tn + j
#pragma unroll
  for (int tm = 0; tm < TM; ++tm)
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) {
      const int n = n0 + wn * WN + 16 * tn + j;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * WM + 16 * tm + 4 * g + r;
        if (m >= M || n >= N) continue;
        if (ksplit == 1)
          C[(size_t)batch * (size_t)sC + (size_t)m * (size_t)ldc + n] = f32_to_bf16_bits(acc[tm][tn][r]);
        else
          part[(((size_t)split * gridDim.z / ksplit + batch) * (size_t)M + m) * (size_t)N + n] = acc[tm][tn][r];
      }
    }
}

// C = the sum of the ksplit fp32 partials, in split order, rounded to bf16
__global__ __launch_bounds__(256) void gemm_reduce_kernel(const float* __restrict__ part,
                                                          uint16_t* __restrict__ C, long long ldc,
                                                          long long sC, int M, int N, int nbatch,
                                                          int ksplit) {
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long per = (long long)M * N;
  if (e >= per * nbatch) return;
  const int batch = (int)(e / per);
  const long long mn = e % per;
  const int m = (int)(mn / N), n = (int)(mn % N);
  float s = 0.f;
  for (int q = 0; q < ksplit; ++q) s += part[((size_t)q * nbatch + batch) * (size_t)per + (size_t)mn];
  C[(size_t)batch * (size_t)sC + (size_t)m * (size_t)ldc + n] = f32_to_bf16_bits(s);
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
static constexpr int GEMM_SMALL_M = 64;        // rows at or below which the 16-row tiles are used
static constexpr int GEMM_TARGET_WGS = 1024;   // workgroups a split-K launch aims for
static constexpr int GEMM_MIN_STEPS = 4;       // K steps per split at least

struct GemmShape {
  int M, N, K, nbatch;
};

// splits of K for the 16-row tiles: enough workgroups to stream the weights
static int gemm_splits(const GemmShape& s) {
  if (s.M > GEMM_SMALL_M) return 1;
  const long long tiles = (long long)((s.M + 15) / 16) * ((s.N + 127) / 128) * s.nbatch;
  long long q = (GEMM_TARGET_WGS + tiles - 1) / tiles;
  q = std::min<long long>(q, std::max(1, (s.K / GEMM_BK) / GEMM_MIN_STEPS));
  return (int)std::max<long long>(1, q);
}

static size_t gemm_part_bytes(const GemmShape& s) {
  const int q = gemm_splits(s);
  return q > 1 ? (size_t)q * s.nbatch * (size_t)s.M * (size_t)s.N * sizeof(float) : 0;
}

static void launch_gemm(const uint16_t* A, long long lda, long long sA, const uint16_t* B, long long ldb,
                        long long sB, uint16_t* C, long long ldc, long long sC, const GemmShape& s,
                        float* part, hipStream_t st) {
  if (s.M > GEMM_SMALL_M) {
    dim3 grid((unsigned)((s.N + 127) / 128), (unsigned)((s.M + 127) / 128), (unsigned)s.nbatch);
    hipLaunchKernelGGL((gemm_nt_kernel<128, 128, 2>), grid, dim3(256), 0, st, A, lda, sA, B, ldb, sB, C, ldc,
                       sC, (float*)nullptr, s.M, s.N, s.K, 1);
    return;
  }
  const int q = gemm_splits(s);
  dim3 grid((unsigned)((s.N + 127) / 128), (unsigned)((s.M + 15) / 16), (unsigned)(s.nbatch * q));
  hipLaunchKernelGGL((gemm_nt_kernel<16, 128, 1>), grid, dim3(256), 0, st, A, lda, sA, B, ldb, sB, C, ldc, sC,
                     part, s.M, s.N, s.K, q);
  if (q > 1) {
    const long long n = (long long)s.M * s.N * s.nbatch;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, part, C, ldc, sC,
                       s.M, s.N, s.nbatch, q);
  }
}

static GemmShape stage1(const ProjArgs& a) {
  return GemmShape{a.T, a.d_g, a.n_h * a.c / a.groups, a.groups};
}
static GemmShape stage2(const ProjArgs& a) { return GemmShape{a.T, a.d, a.groups * a.d_g, 1}; }

size_t proj_workspace_bytes(const ProjArgs& a) {
  const size_t p1 = gemm_part_bytes(stage1(a)), p2 = gemm_part_bytes(stage2(a));
  return p1 > p2 ? p1 : p2;   // the stages run one after the other on one stream
}

int launch_proj(const ProjArgs& a, hipStream_t st) {
  const int HC = a.n_h * a.c, W = HC / a.groups, Y = a.groups * a.d_g;
  // stage 1: group q, y[:, q d_g ..] = o[:, q W ..] W1[q]^T
  launch_gemm((const uint16_t*)a.o, HC, W, (const uint16_t*)a.W1, W, (long long)a.d_g * W, (uint16_t*)a.y, Y,
              a.d_g, stage1(a), (float*)a.ws, st);
  // stage 2: out = y W2^T
  launch_gemm((const uint16_t*)a.y, Y, 0, (const uint16_t*)a.W2, Y, 0, (uint16_t*)a.out, a.d, 0, stage2(a),
              (float*)a.ws, st);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
