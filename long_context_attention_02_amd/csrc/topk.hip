// a3 — exact per-query top-k for gfx950.
//
// DeepSeek-V4 method page, section 3.3: the candidate set of a query is the
// top-k of its indexer scores (k = 512 / 1024 in the report digest).  Order:
// score descending, ties to the lower index; -0.0 equals +0.0.
//
// Every visible element has a unique 64-bit key
//     K64 = ord(score) << 32 | (0xFFFFFFFF - index)
// where ord() is the order-preserving map of a float onto uint32.  The k
// largest K64 are exactly the requested selection in the requested order.  An
// MSD radix select finds the threshold: 10-bit digits of the 32-bit score key
// first (LDS histograms, the digit located by one wave), and only when the k-th
// score is tied, further digits of the index half among the tied elements.
// One pass collects the k keys and a bitonic sort in LDS orders them.  No
// atomic decides anything but the slot an element lands in before the sort,
// so results are deterministic.
//
// The elements of a row (or chunk) are first copied into LDS once; on the way
// the block forms the AND and the OR of all score keys, so the bits every key
// shares are skipped and the digits start at the highest bit that differs.
// Long rows with few queries (decode) run in two stages: workgroups select
// the top-k of chunks of 16k elements (any global top-k element is in its
// chunk's top-k), then one workgroup per row selects from their union.
#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

static constexpr int TK_THREADS = 1024;
static constexpr int TK_KMAX = 2048;
static constexpr int TK_BINS = 1024;      // 10-bit digits
static constexpr int TK_LDS_BYTES = 128 * 1024;           // element cache per workgroup
static constexpr int TK_CACHE32 = TK_LDS_BYTES / 4;       // score rows cached as ord keys
static constexpr int TK_CACHE64 = TK_LDS_BYTES / 8;       // K64 candidate lists

// Element sources: hi(e) = ord(score), lo(e) = 0xFFFFFFFF - index.
struct LdsRowSrc {     // ord keys cached in LDS; index = base + position
  const uint32_t* p;
  long long base;
  __device__ __forceinline__ uint32_t hi(long long e) const { return p[e]; }
  __device__ __forceinline__ uint32_t lo(long long e) const { return 0xFFFFFFFFu - (uint32_t)(base + e); }
};
struct RowSrc {        // scores in global memory; index = base + position
  const float* p;
  long long base;
  __device__ __forceinline__ uint32_t hi(long long e) const { return ord_key(p[e]); }
  __device__ __forceinline__ uint32_t lo(long long e) const { return 0xFFFFFFFFu - (uint32_t)(base + e); }
};
struct KeySrc {        // explicit K64 candidates, global or LDS (0 = padding, below every real key)
  const uint64_t* p;
  __device__ __forceinline__ uint32_t hi(long long e) const { return (uint32_t)(p[e] >> 32); }
  __device__ __forceinline__ uint32_t lo(long long e) const { return (uint32_t)p[e]; }
};

struct TopkShared {
  uint32_t hist[2][TK_BINS];   // double-buffered: one is cleared while the other is read
  uint64_t buf[TK_KMAX];
  uint32_t red_and[TK_THREADS / 64], red_or[TK_THREADS / 64];
  int digit, cum, cnt_d, count;
};

// block-wide AND / OR of 32-bit values (every thread gets both)
__device__ __forceinline__ void block_and_or(uint32_t& a, uint32_t& o, TopkShared& sh) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) {
    a &= (uint32_t)__shfl_xor((int)a, s, 64);
    o |= (uint32_t)__shfl_xor((int)o, s, 64);
  }
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) { sh.red_and[wid] = a; sh.red_or[wid] = o; }
  __syncthreads();
  a = ~0u; o = 0u;
  for (int w = 0; w < TK_THREADS / 64; ++w) { a &= sh.red_and[w]; o |= sh.red_or[w]; }
}

// wave 0 finds the digit where the count from the top reaches `need` in hist
// (bins in descending order); writes sh.digit / cum / cnt_d
__device__ __forceinline__ void find_digit(const uint32_t* hist, int need, TopkShared& sh) {
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  constexpr int PER = TK_BINS / 64;           // bins per lane, lane 0 holds the top bins
  const int top = TK_BINS - 1 - PER * lane;
  int sum = 0;
#pragma unroll 8
  for (int q = 0; q < PER; ++q) sum += (int)hist[top - q];
  int incl = sum;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  const int above = incl - sum;
  if (above < need && need <= incl) {
    int run = above;
    for (int q = 0; q < PER; ++q) {
      const int c = (int)hist[top - q];
      if (need <= run + c) {
        sh.digit = top - q; sh.cum = run; sh.cnt_d = c;
        break;
      }
      run += c;
    }
  }
}

// Radix select on one 32-bit half of the keys among the elements whose other
// half / prefix matches.  HALF = 0: hi keys; HALF = 1: lo keys of the elements
// whose hi key equals hi_val.  Returns the decided bits in *prefix and the
// count still needed from the final group in *need; *tied reports whether the
// final group holds more elements than needed (only possible for HALF = 0).
template <class Src, int HALF>
__device__ void radix_half(const Src& src, long long n, uint32_t k_and, uint32_t k_or, uint32_t hi_val,
                           int& need, uint32_t& prefix, bool& tied, TopkShared& sh, int& hb) {
  const int tid = threadIdx.x;
  const uint32_t diff = k_and ^ k_or;
  tied = false;
  if (diff == 0u) {            // the whole group shares this half
    prefix = k_and;
    tied = true;               // every element of the group is equal here
    return;
  }
  int top = 31 - __clz((int)diff);
  const uint32_t common = (top == 31) ? 0u : ~((2u << top) - 1u);
  prefix = k_and & common;
  uint32_t pmask = common;
  // the buffer cleared for this pass is hist[hb]
  for (int e = tid; e < TK_BINS; e += TK_THREADS) sh.hist[hb][e] = 0u;
  __syncthreads();
  while (true) {
    const int width = top + 1 < 10 ? top + 1 : 10;
    const int shift = top + 1 - width;
    const uint32_t dmask = (1u << width) - 1u;
    uint32_t* hist = sh.hist[hb];
    for (long long e = tid; e < n; e += TK_THREADS) {
      const uint32_t h = src.hi(e);
      uint32_t key;
      if (HALF == 0) {
        key = h;
      } else {
        if (h != hi_val) continue;
        key = src.lo(e);
      }
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    // clear the other buffer for the next pass while this one is complete
    for (int e = tid; e < TK_BINS; e += TK_THREADS) sh.hist[hb ^ 1][e] = 0u;
    __syncthreads();
    find_digit(hist, need, sh);
    __syncthreads();
    prefix |= (uint32_t)sh.digit << shift;
    pmask |= dmask << shift;
    need -= sh.cum;
    hb ^= 1;
    if (sh.cnt_d == need) return;
    if (shift == 0) { tied = true; return; }
    top = shift - 1;
  }
}

// k largest K64 = hi << 32 | lo among n elements -> sh.buf[0 .. min(k, n)), sorted
// descending when SORT.  hi_and / hi_or: AND / OR of every element's hi key.
template <class Src, bool SORT>
__device__ int select_topk(const Src& src, long long n, int k, uint32_t hi_and, uint32_t hi_or,
                           TopkShared& sh) {
  const int tid = threadIdx.x;
  const int want = (int)min((long long)k, n);
  if (want <= 0) return 0;
  // threshold: select hi > thr_hi, plus hi == thr_hi with lo >= thr_lo
  uint32_t thr_hi = 0u, thr_lo = 0u;
  bool all_eq_hi = false;    // true: every element with hi == thr_hi's prefix group is taken
  if (want < n) {
    int need = want, hb = 0;
    bool tied;
    uint32_t pre;
    radix_half<Src, 0>(src, n, hi_and, hi_or, 0u, need, pre, tied, sh, hb);
    thr_hi = pre;
    if (!tied) {
      all_eq_hi = true;       // take every element whose hi >= pre (pre has zero low bits)
    } else {
      // ties on the full hi key: resolve among them by the lo key (the index)
      uint32_t l_and = ~0u, l_or = 0u;
      for (long long e = tid; e < n; e += TK_THREADS)
        if (src.hi(e) == thr_hi) { const uint32_t l = src.lo(e); l_and &= l; l_or |= l; }
      block_and_or(l_and, l_or, sh);
      __syncthreads();
      uint32_t lpre;
      bool t2;
      radix_half<Src, 1>(src, n, l_and, l_or, thr_hi, need, lpre, t2, sh, hb);
      thr_lo = lpre;
    }
  } else {
    all_eq_hi = true;
    thr_hi = 0u;
  }
  // collect every selected key (exactly `want` of them)
  if (tid == 0) sh.count = 0;
  __syncthreads();
  for (long long e = tid; e < n; e += TK_THREADS) {
    const uint32_t h = src.hi(e);
    bool take;
    if (all_eq_hi) take = h >= thr_hi;
    else take = h > thr_hi || (h == thr_hi && src.lo(e) >= thr_lo);
    if (take) {
      const int slot = atomicAdd(&sh.count, 1);
      if (slot < TK_KMAX) sh.buf[slot] = ((uint64_t)h << 32) | src.lo(e);
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
  uint32_t a = ~0u, o = 0u;
  if (use_cache) {
    const long long n4 = (((uintptr_t)p & 15u) == 0) ? (n & ~3LL) : 0;   // vector part if aligned
    for (long long e = 4LL * threadIdx.x; e < n4; e += 4LL * TK_THREADS) {
      const f32x4_t v = *(const f32x4_t*)(p + e);
      u32x4_t ok;
      ok[0] = ord_key(v[0]); ok[1] = ord_key(v[1]); ok[2] = ord_key(v[2]); ok[3] = ord_key(v[3]);
      *(u32x4_t*)(cache + e) = ok;
      a &= ok[0] & ok[1] & ok[2] & ok[3];
      o |= ok[0] | ok[1] | ok[2] | ok[3];
    }
    for (long long e = n4 + threadIdx.x; e < n; e += TK_THREADS) {
      const uint32_t ok = ord_key(p[e]);
      cache[e] = ok;
      a &= ok;
      o |= ok;
    }
    block_and_or(a, o, sh);   // its barrier also publishes the cache
    __syncthreads();
    return select_topk<LdsRowSrc, SORT>(LdsRowSrc{cache, base}, n, k, a, o, sh);
  }
  const RowSrc src{p, base};
  for (long long e = threadIdx.x; e < n; e += TK_THREADS) {
    const uint32_t ok = src.hi(e);
    a &= ok;
    o |= ok;
  }
  block_and_or(a, o, sh);
  __syncthreads();
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
  extern __shared__ __attribute__((aligned(16))) uint32_t cache[];
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
  extern __shared__ __attribute__((aligned(16))) uint32_t cache[];
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
  extern __shared__ __attribute__((aligned(16))) uint64_t cache64[];
  const size_t row = blockIdx.x;
  const long long n = row_nvis(q_pos, row, N_cap, m);
  const int want = (int)min((long long)k, n);
  const long long ncand = (long long)nchunks * k;
  const uint64_t* cp = cand + row * (size_t)ncand;
  // padding keys (0) rank below every real key and `want` never exceeds the real ones
  uint32_t a = ~0u, o = 0u;
  int got;
  if (use_cache) {
    for (long long e = threadIdx.x; e < ncand; e += TK_THREADS) {
      const uint64_t key = cp[e];
      cache64[e] = key;
      a &= (uint32_t)(key >> 32);
      o |= (uint32_t)(key >> 32);
    }
    block_and_or(a, o, sh);
    __syncthreads();
    got = select_topk<KeySrc, true>(KeySrc{cache64}, ncand, want, a, o, sh);
  } else {
    for (long long e = threadIdx.x; e < ncand; e += TK_THREADS) {
      a &= (uint32_t)(cp[e] >> 32);
      o |= (uint32_t)(cp[e] >> 32);
    }
    block_and_or(a, o, sh);
    __syncthreads();
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
