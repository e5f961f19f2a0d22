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
// an MSD radix select on K64 finds the k-th largest key T without any tie
// special case, one pass collects all K64 >= T, and a bitonic sort in LDS
// orders them.  No atomic decides anything but the slot an element lands in
// before the sort, so results are deterministic.
//
// The elements of a row (or chunk) are first copied into LDS once; on the way
// the block forms the AND and the OR of all keys, so the bits every key shares
// are skipped and the 11-bit digits start at the highest bit that differs.
// Long rows with few queries (decode) run in two stages: workgroups select
// the top-k of chunks of 16k elements (any global top-k element is in its
// chunk's top-k), then one workgroup per row selects from their union.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

static constexpr int TK_THREADS = 1024;
static constexpr int TK_KMAX = 2048;
static constexpr int TK_BINS = 2048;
static constexpr int TK_LDS_BYTES = 128 * 1024;           // element cache per workgroup
static constexpr int TK_CACHE32 = TK_LDS_BYTES / 4;       // score rows cached as ord keys
static constexpr int TK_CACHE64 = TK_LDS_BYTES / 8;       // K64 candidate lists

__device__ __forceinline__ uint64_t make_key(float score, uint32_t idx) {
  return ((uint64_t)ord_key(score) << 32) | (uint64_t)(0xFFFFFFFFu - idx);
}

struct RowSrc {        // scores in global memory; index = base + position
  const float* p;
  long long base;
  __device__ __forceinline__ uint64_t get(long long e) const { return make_key(p[e], (uint32_t)(base + e)); }
};
struct LdsRowSrc {     // ord keys cached in LDS; index = base + position
  const uint32_t* p;
  long long base;
  __device__ __forceinline__ uint64_t get(long long e) const {
    return ((uint64_t)p[e] << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(base + e));
  }
};
struct KeySrc {        // explicit K64 candidates, global or LDS (0 = padding, below every real key)
  const uint64_t* p;
  __device__ __forceinline__ uint64_t get(long long e) const { return p[e]; }
};

struct TopkShared {
  uint32_t hist[TK_BINS];
  uint64_t buf[TK_KMAX];
  uint64_t red_and[TK_THREADS / 64], red_or[TK_THREADS / 64];
  int wsum[TK_THREADS / 64];
  int digit, cum, cnt_d, count;
};

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, o, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), o, 64);
  return ((uint64_t)hi << 32) | lo;
}

// block-wide AND / OR of 64-bit values (every thread gets both)
__device__ __forceinline__ void block_and_or(uint64_t& a, uint64_t& o, TopkShared& sh) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) {
    a &= shfl_xor_u64(a, s);
    o |= shfl_xor_u64(o, s);
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) { sh.red_and[wid] = a; sh.red_or[wid] = o; }
  __syncthreads();
  a = ~0ull; o = 0ull;
  for (int w = 0; w < TK_THREADS / 64; ++w) { a &= sh.red_and[w]; o |= sh.red_or[w]; }
  __syncthreads();
}

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

// k largest K64 of n elements (whose AND / OR are k_and / k_or) -> sh.buf[0 .. min(k, n)),
// sorted descending when SORT.  Returns min(k, n).
template <class Src, bool SORT>
__device__ int select_topk(const Src& src, long long n, int k, uint64_t k_and, uint64_t k_or,
                           TopkShared& sh) {
  const int tid = threadIdx.x;
  const int want = (int)min((long long)k, n);
  if (want <= 0) return 0;
  uint64_t prefix = 0;
  if (want < n) {
    // bits shared by every key are already decided; digits start at the highest differing bit
    const uint64_t diff = k_and ^ k_or;            // nonzero: keys are unique and n > 1
    int top = 63 - __clzll((long long)diff);
    const uint64_t common = (top == 63) ? 0ull : ~((2ull << top) - 1ull);
    prefix = k_and & common;
    uint64_t pmask = common;
    int need = want;
    while (true) {
      const int width = top + 1 < 11 ? top + 1 : 11;
      const int shift = top + 1 - width;
      const uint64_t dmask = (1ull << width) - 1ull;
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
      const bool done = (sh.cnt_d == need) || shift == 0;
      __syncthreads();
      if (done) break;
      top = shift - 1;
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

// top-k of the scores p[0 .. n) (indices base + e): cached in LDS when they fit
template <bool SORT>
__device__ int select_row(const float* __restrict__ p, long long n, long long base, int k,
                          uint32_t* cache, bool use_cache, TopkShared& sh) {
  uint64_t a = ~0ull, o = 0ull;
  if (use_cache) {
    for (long long e = threadIdx.x; e < n; e += TK_THREADS) {
      const uint32_t ok = ord_key(p[e]);
      cache[e] = ok;
      const uint64_t key = ((uint64_t)ok << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)(base + e));
      a &= key;
      o |= key;
    }
    block_and_or(a, o, sh);   // its barriers also publish the cache
    return select_topk<LdsRowSrc, SORT>(LdsRowSrc{cache, base}, n, k, a, o, sh);
  }
  const RowSrc src{p, base};
  for (long long e = threadIdx.x; e < n; e += TK_THREADS) {
    const uint64_t key = src.get(e);
    a &= key;
    o |= key;
  }
  block_and_or(a, o, sh);
  return select_topk<RowSrc, SORT>(src, n, k, a, o, sh);
}

__device__ __forceinline__ long long row_nvis(const int* q_pos, size_t row, long long N_cap, int m) {
  return min(N_cap, ((long long)q_pos[row] + 1) / m);
}

// one workgroup per query row: final, sorted selection
__global__ __launch_bounds__(TK_THREADS) void topk_rows_kernel(
    const float* __restrict__ I, const int* __restrict__ q_pos, long long N_cap, int m, int k,
    int use_cache, int* __restrict__ idx_out, float* __restrict__ val_out) {
  __shared__ TopkShared sh;
  extern __shared__ uint32_t cache[];
  const size_t row = blockIdx.x;
  const long long n = row_nvis(q_pos, row, N_cap, m);
  const float* rp = I + row * (size_t)N_cap;
  const int got = select_row<true>(rp, n, 0, k, cache, use_cache != 0, sh);
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
    long long chunk, int nchunks, int use_cache, uint64_t* __restrict__ cand) {
  __shared__ TopkShared sh;
  extern __shared__ uint32_t cache[];
  const size_t row = blockIdx.y;
  const int c = blockIdx.x;
  const long long n = row_nvis(q_pos, row, N_cap, m);
  const long long lo = (long long)c * chunk;
  const long long len = max(0LL, min(n, lo + chunk) - lo);
  int got = 0;
  if (len > 0)
    got = select_row<false>(I + row * (size_t)N_cap + lo, len, lo, k, cache, use_cache != 0, sh);
  uint64_t* dst = cand + (row * (size_t)nchunks + c) * (size_t)k;
  for (int e = threadIdx.x; e < k; e += TK_THREADS) dst[e] = e < got ? sh.buf[e] : 0ull;
}

// stage 2: top-k over the union of the chunk selections of one row
__global__ __launch_bounds__(TK_THREADS) void topk_merge_kernel(
    const uint64_t* __restrict__ cand, const float* __restrict__ I, const int* __restrict__ q_pos,
    long long N_cap, int m, int k, int nchunks, int use_cache, int* __restrict__ idx_out,
    float* __restrict__ val_out) {
  __shared__ TopkShared sh;
  extern __shared__ uint64_t cache64[];
  const size_t row = blockIdx.x;
  const long long n = row_nvis(q_pos, row, N_cap, m);
  const int want = (int)min((long long)k, n);
  const long long ncand = (long long)nchunks * k;
  const uint64_t* cp = cand + row * (size_t)ncand;
  // padding keys (0) rank below every real key and `want` never exceeds the real ones
  uint64_t a = ~0ull, o = 0ull;
  int got;
  if (use_cache) {
    for (long long e = threadIdx.x; e < ncand; e += TK_THREADS) {
      const uint64_t key = cp[e];
      cache64[e] = key;
      a &= key;
      o |= key;
    }
    block_and_or(a, o, sh);
    got = select_topk<KeySrc, true>(KeySrc{cache64}, ncand, want, a, o, sh);
  } else {
    for (long long e = threadIdx.x; e < ncand; e += TK_THREADS) {
      a &= cp[e];
      o |= cp[e];
    }
    block_and_or(a, o, sh);
    got = select_topk<KeySrc, true>(KeySrc{cp}, ncand, want, a, o, sh);
  }
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

static bool set_lds(const void* kfn, size_t bytes) {
  return bytes <= 65536 ||
         hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) == hipSuccess;
}

int launch_topk(const TopkArgs& a, hipStream_t st) {
  const long long rows = (long long)a.B * a.Tq;
  long long chunk;
  int nchunks;
  if (topk_two_stage(rows, a.N_cap, a.k, &chunk, &nchunks)) {
    uint64_t* cand = (uint64_t*)a.ws;
    const bool c1 = chunk <= TK_CACHE32;
    const long long ncand = (long long)nchunks * a.k;
    const bool c2 = ncand <= TK_CACHE64;
    const size_t l1 = c1 ? (size_t)chunk * 4 : 0, l2 = c2 ? (size_t)ncand * 8 : 0;
    if (!set_lds((const void*)topk_chunk_kernel, l1) || !set_lds((const void*)topk_merge_kernel, l2))
      return -1;
    hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)nchunks, (unsigned)rows), dim3(TK_THREADS),
                       l1, st, a.I, a.q_pos, a.N_cap, a.m, a.k, chunk, nchunks, (int)c1, cand);
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(TK_THREADS), l2, st, cand, a.I,
                       a.q_pos, a.N_cap, a.m, a.k, nchunks, (int)c2, a.idx, a.val);
  } else {
    const bool c1 = a.N_cap <= TK_CACHE32;
    const size_t l1 = c1 ? (size_t)a.N_cap * 4 : 0;
    if (!set_lds((const void*)topk_rows_kernel, l1)) return -1;
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)rows), dim3(TK_THREADS), l1, st, a.I,
                       a.q_pos, a.N_cap, a.m, a.k, (int)c1, a.idx, a.val);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
