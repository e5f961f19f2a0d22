// a3 — exact per-query top-k for gfx950.
//
// DeepSeek-V4 method page, section 3.3: the candidate set of a query is the
// top-k of its indexer scores (k = 512 / 1024 in the report digest).  Order:
// score descending, ties to the lower index; -0.0 equals +0.0.
//
// Every visible element becomes a unique 64-bit key
//     K64 = ord(score) << 32 | (0xFFFFFFFF - index)
// where ord() is the order-preserving map of a float onto uint32.  The k
// largest K64 are exactly the requested selection in the requested order, so
// an MSD radix select on K64 (11/11/10/11/11/10-bit digits, LDS histograms)
// finds the k-th largest key T without any tie special case, a single pass
// collects all K64 >= T, and a bitonic sort in LDS orders them.  No atomic
// decides anything but the (irrelevant) slot an element lands in before the
// sort, so the result is deterministic.
//
// Long rows with few queries (decode) run in two stages: workgroups first
// select the top-k of chunks of 16k elements (any global top-k element is in
// its chunk's top-k), then one workgroup per row selects from the union.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

static constexpr int TK_THREADS = 1024;
static constexpr int TK_KMAX = 2048;
static constexpr int TK_BINS = 2048;

struct RowSrc {        // elements of a score row; index = base + position
  const float* p;
  long long base;
  __device__ __forceinline__ uint64_t get(long long e) const {
    const uint32_t idx = (uint32_t)(base + e);
    return ((uint64_t)ord_key(p[e]) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
  }
};
struct KeySrc {        // explicit K64 candidates (0 = padding, below every real key)
  const uint64_t* p;
  __device__ __forceinline__ uint64_t get(long long e) const { return p[e]; }
};

struct TopkShared {
  uint32_t hist[TK_BINS];
  uint64_t buf[TK_KMAX];
  int wsum[TK_THREADS / 64];
  int digit, cum, cnt_d, count;
};

// exclusive prefix sum over the block (in thread order) of v; returns the sum before this thread
__device__ __forceinline__ int block_excl_scan(int v, int* wsum) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wid] = x;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wid; ++w) off += wsum[w];
  __syncthreads();
  return off + x - v;
}

// k largest K64 of n elements -> sh.buf[0 .. min(k,n)) sorted descending (when SORT)
template <class Src, bool SORT>
__device__ int select_topk(const Src& src, long long n, int k, TopkShared& sh) {
  const int tid = threadIdx.x;
  const int want = (int)min((long long)k, n);
  if (want <= 0) return 0;
  int need = want;
  uint64_t prefix = 0, pmask = 0;
  if (need < n) {
    const int shifts[6] = {53, 42, 32, 21, 10, 0};
    const int widths[6] = {11, 11, 10, 11, 11, 10};
    for (int pass = 0; pass < 6; ++pass) {
      const int shift = shifts[pass];
      const uint64_t dmask = (1ull << widths[pass]) - 1ull;
      for (int e = tid; e < TK_BINS; e += TK_THREADS) sh.hist[e] = 0u;
      __syncthreads();
      for (long long e = tid; e < n; e += TK_THREADS) {
        const uint64_t key = src.get(e);
        if ((key & pmask) == prefix) atomicAdd(&sh.hist[(key >> shift) & dmask], 1u);
      }
      __syncthreads();
      // bins in descending order; thread t holds bins 2047-2t and 2046-2t
      const int c0 = (int)sh.hist[TK_BINS - 1 - 2 * tid];
      const int c1 = (int)sh.hist[TK_BINS - 2 - 2 * tid];
      const int above = block_excl_scan(c0 + c1, sh.wsum);
      if (above < need && need <= above + c0 + c1) {
        if (need <= above + c0) {
          sh.digit = TK_BINS - 1 - 2 * tid; sh.cum = above; sh.cnt_d = c0;
        } else {
          sh.digit = TK_BINS - 2 - 2 * tid; sh.cum = above + c0; sh.cnt_d = c1;
        }
      }
      __syncthreads();
      prefix |= (uint64_t)sh.digit << shift;
      pmask |= dmask << shift;
      need -= sh.cum;
      const bool done = (sh.cnt_d == need);
      __syncthreads();
      if (done) break;
    }
  }
  // collect every key >= threshold (exactly `want` of them)
  if (tid == 0) sh.count = 0;
  __syncthreads();
  for (long long e = tid; e < n; e += TK_THREADS) {
    const uint64_t key = src.get(e);
    if (key >= prefix) {
      const int slot = atomicAdd(&sh.count, 1);
      if (slot < TK_KMAX) sh.buf[slot] = key;   // exactly `want` <= TK_KMAX keys qualify
    }
  }
  __syncthreads();
  if (SORT) {
    int P = 1;
    while (P < want) P <<= 1;
    for (int e = want + tid; e < P; e += TK_THREADS) sh.buf[e] = 0ull;
    for (int size = 2; size <= P; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        __syncthreads();
        for (int i = tid; i < P / 2; i += TK_THREADS) {
          const int lo = 2 * i - (i & (stride - 1));
          const int hi = lo + stride;
          const bool desc = (lo & size) == 0;
          const uint64_t x = sh.buf[lo], y = sh.buf[hi];
          if ((x < y) == desc) { sh.buf[lo] = y; sh.buf[hi] = x; }
        }
      }
    }
    __syncthreads();
  }
  return want;
}

__device__ __forceinline__ long long row_nvis(const int* q_pos, size_t row, long long N_cap, int m) {
  return min(N_cap, ((long long)q_pos[row] + 1) / m);
}

// one workgroup per query row: final, sorted selection
__global__ __launch_bounds__(TK_THREADS) void topk_rows_kernel(
    const float* __restrict__ I, const int* __restrict__ q_pos, long long N_cap, int m, int k,
    int* __restrict__ idx_out, float* __restrict__ val_out) {
  __shared__ TopkShared sh;
  const size_t row = blockIdx.x;
  const long long n = row_nvis(q_pos, row, N_cap, m);
  const float* rp = I + row * (size_t)N_cap;
  const int got = select_topk<RowSrc, true>(RowSrc{rp, 0}, n, k, sh);
  for (int e = threadIdx.x; e < k; e += TK_THREADS) {
    int idx = -1;
    float val = -INFINITY;
    if (e < got) {
      idx = (int)(0xFFFFFFFFu - (uint32_t)sh.buf[e]);
      val = rp[idx];
    }
    idx_out[row * (size_t)k + e] = idx;
    if (val_out) val_out[row * (size_t)k + e] = val;
  }
}

// stage 1: top-k of one chunk of one row, unsorted, padded with 0 keys
__global__ __launch_bounds__(TK_THREADS) void topk_chunk_kernel(
    const float* __restrict__ I, const int* __restrict__ q_pos, long long N_cap, int m, int k,
    long long chunk, int nchunks, uint64_t* __restrict__ cand) {
  __shared__ TopkShared sh;
  const size_t row = blockIdx.y;
  const int c = blockIdx.x;
  const long long n = row_nvis(q_pos, row, N_cap, m);
  const long long lo = (long long)c * chunk;
  const long long len = max(0LL, min(n, lo + chunk) - lo);
  int got = 0;
  if (len > 0) got = select_topk<RowSrc, false>(RowSrc{I + row * (size_t)N_cap + lo, lo}, len, k, sh);
  uint64_t* dst = cand + (row * (size_t)nchunks + c) * (size_t)k;
  for (int e = threadIdx.x; e < k; e += TK_THREADS) dst[e] = e < got ? sh.buf[e] : 0ull;
}

// stage 2: top-k over the union of the chunk selections of one row
__global__ __launch_bounds__(TK_THREADS) void topk_merge_kernel(
    const uint64_t* __restrict__ cand, const float* __restrict__ I, const int* __restrict__ q_pos,
    long long N_cap, int m, int k, int nchunks, int* __restrict__ idx_out,
    float* __restrict__ val_out) {
  __shared__ TopkShared sh;
  const size_t row = blockIdx.x;
  const long long n = row_nvis(q_pos, row, N_cap, m);
  const int want = (int)min((long long)k, n);
  const long long ncand = (long long)nchunks * k;
  // padding keys (0) rank below every real key and `want` never exceeds the real ones
  const int got = select_topk<KeySrc, true>(KeySrc{cand + row * (size_t)ncand}, ncand, want, sh);
  const float* rp = I + row * (size_t)N_cap;
  for (int e = threadIdx.x; e < k; e += TK_THREADS) {
    int idx = -1;
    float val = -INFINITY;
    if (e < got && e < want) {
      idx = (int)(0xFFFFFFFFu - (uint32_t)sh.buf[e]);
      val = rp[idx];
    }
    idx_out[row * (size_t)k + e] = idx;
    if (val_out) val_out[row * (size_t)k + e] = val;
  }
}

static bool topk_two_stage(long long rows, long long N_cap, int k, long long* chunk, int* nchunks) {
  const long long ch = 16LL * k;
  if (rows >= 512 || N_cap < 2 * ch) return false;
  *chunk = ch;
  *nchunks = (int)((N_cap + ch - 1) / ch);
  return true;
}

size_t topk_workspace_bytes(int B, int Tq, long long N_cap, int k) {
  long long chunk;
  int nchunks;
  const long long rows = (long long)B * Tq;
  if (!topk_two_stage(rows, N_cap, k, &chunk, &nchunks)) return 0;
  return (size_t)rows * (size_t)nchunks * (size_t)k * sizeof(uint64_t);
}

int launch_topk(const TopkArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.Tq;
  long long chunk;
  int nchunks;
  if (topk_two_stage(rows, a.N_cap, a.k, &chunk, &nchunks)) {
    uint64_t* cand = (uint64_t*)a.ws;
    hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)nchunks, (unsigned)rows), dim3(TK_THREADS),
                       0, st, a.I, a.q_pos, a.N_cap, a.m, a.k, chunk, nchunks, cand);
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(TK_THREADS), 0, st, cand, a.I,
                       a.q_pos, a.N_cap, a.m, a.k, nchunks, a.idx, a.val);
  } else {
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)rows), dim3(TK_THREADS), 0, st, a.I,
                       a.q_pos, a.N_cap, a.m, a.k, a.idx, a.val);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
