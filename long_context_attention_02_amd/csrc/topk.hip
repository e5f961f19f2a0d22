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
// One pass collects the k keys (one atomic per wave and group) and a bitonic sort orders
// them (lane shuffles for partners within a wave, LDS beyond).  No
// atomic decides anything but the slot an element lands in before the sort,
// so results are deterministic.
//
// The elements of a row (or chunk) are first copied into LDS once; on the way
// the block forms the AND and the OR of all score keys, so the bits every key
// shares are skipped and the digits start at the highest bit that differs.
// Long rows with few queries (decode) run in two stages over chunks of up to
// 16 k elements: workgroups keep the T largest keys of each chunk, sorted, with the
// chunk's (T+1)-th key as its threshold, then one workgroup per list places
// its keys in the merged order and checks the result against the thresholds
// (the sorted-list stages below; when the lists do not fit LDS, each chunk's
// top-k and a selection over their union instead).
#include <algorithm>
#include <cmath>

#include "csa_device.h"
#include "csa_internal.h"

namespace csa {

static constexpr int TK_THREADS = 1024;
static constexpr int TK_KMAX = 2048;
static constexpr int TK_BINS = 1024;      // 10-bit digits
static constexpr int TK_LDS_BYTES = 128 * 1024;           // element cache per workgroup
static constexpr int TK_CACHE32 = TK_LDS_BYTES / 4;       // score rows cached as ord keys
static constexpr int TK_CACHE64 = TK_LDS_BYTES / 8;       // K64 candidate lists
static constexpr int TK_LDU = 8;                          // global loads in flight per thread when caching

// Element sources: hi = ord(score), lo = 0xFFFFFFFF - index.  load<V>(e0)
// gives elements e0 .. e0 + V - 1 (V per thread and pass); sources held in LDS
// read V at once (their buffers are padded to 16 bytes, so a group that runs
// past n stays inside the allocation; such elements are masked by the caller).
struct LdsRowSrc {     // ord keys cached in LDS; index = base + position
  static constexpr int V = 4;
  const uint32_t* p;
  long long base;
  __device__ __forceinline__ void load(long long e0, uint32_t (&h)[V], uint32_t (&l)[V]) const {
    const u32x4_t q = *(const u32x4_t*)(p + e0);
#pragma unroll
    for (int v = 0; v < V; ++v) {
      h[v] = q[v];
      l[v] = 0xFFFFFFFFu - (uint32_t)(base + e0 + v);
    }
  }
};
struct RowSrc {        // scores in global memory; index = base + position
  static constexpr int V = 1;
  const float* p;
  long long base;
  __device__ __forceinline__ void load(long long e0, uint32_t (&h)[V], uint32_t (&l)[V]) const {
    h[0] = ord_key(p[e0]);
    l[0] = 0xFFFFFFFFu - (uint32_t)(base + e0);
  }
};
struct KeyLdsSrc {     // K64 candidates cached in LDS (0 = padding, below every real key)
  static constexpr int V = 2;
  const uint64_t* p;
  __device__ __forceinline__ void load(long long e0, uint32_t (&h)[V], uint32_t (&l)[V]) const {
    const u32x4_t q = *(const u32x4_t*)(p + e0);   // little endian: {lo0, hi0, lo1, hi1}
    l[0] = q[0]; h[0] = q[1];
    l[1] = q[2]; h[1] = q[3];
  }
};
struct KeySrc {        // K64 candidates in global memory
  static constexpr int V = 1;
  const uint64_t* p;
  __device__ __forceinline__ void load(long long e0, uint32_t (&h)[V], uint32_t (&l)[V]) const {
    const uint64_t x = p[e0];
    h[0] = (uint32_t)(x >> 32);
    l[0] = (uint32_t)x;
  }
};

struct TopkShared {
  uint32_t hist[2][TK_BINS];   // double-buffered: one is cleared while the other is read
  uint64_t buf[TK_KMAX];
  uint32_t red_and[TK_THREADS / 64], red_or[TK_THREADS / 64];
  int wcount[TK_THREADS / 64];
  int digit, cum, cnt_d, count;
};

// Wave-wide reductions: a butterfly inside each row of 16 lanes through DPP
// (quad permutes, half-row and row mirrors), then the four row results read
// as scalars.  Every lane gets the result.
template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, false));   // row_half_mirror
  v = op(v, (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, false));   // row_mirror
  const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return op(op(r0, r1), op(r2, r3));
}
struct OpAnd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a & b; } };
struct OpOr { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a | b; } };
struct OpMin { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a < b ? a : b; } };

// block-wide AND / OR of 32-bit values (every thread gets both)
__device__ __forceinline__ void block_and_or(uint32_t& a, uint32_t& o, TopkShared& sh) {
  a = wave_reduce_u32(a, OpAnd{});
  o = wave_reduce_u32(o, OpOr{});
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (lane == 0) { sh.red_and[wid] = a; sh.red_or[wid] = o; }
  __syncthreads();
  a = ~0u; o = 0u;
  for (int w = 0; w < TK_THREADS / 64; ++w) { a &= sh.red_and[w]; o |= sh.red_or[w]; }
}

// Lower bound for the selection: t = min over the threads that hold elements of
// each thread's largest hi key.  At least that many elements (one per such
// thread) have hi >= t, so when they are at least `want`, no element with
// hi < t can be among the k largest and t = 0 otherwise.  lmax = ~0u marks a
// thread without elements.
__device__ __forceinline__ uint32_t block_lower_bound(uint32_t lmax, int want, TopkShared& sh) {
  const bool has = lmax != ~0u;
  const uint32_t mn = wave_reduce_u32(has ? lmax : ~0u, OpMin{});
  const int cnt = __popcll(__ballot(has));
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();   // red_and / wcount may still be read by an earlier reduction
  if (lane == 0) { sh.red_and[wid] = mn; sh.wcount[wid] = cnt; }
  __syncthreads();
  uint32_t t = ~0u;
  int total = 0;
  for (int w = 0; w < TK_THREADS / 64; ++w) { t = min(t, sh.red_and[w]); total += sh.wcount[w]; }
  __syncthreads();   // the reads above finish before the next reduction reuses the buffers
  return (total >= want && total > 0) ? t : 0u;
}

// inclusive sum of v over lanes 0 .. lane: DPP row shifts inside each 16-lane row
// (lanes without a source add 0), then the totals of the rows below
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  const int t0 = __builtin_amdgcn_readlane(v, 15), t1 = __builtin_amdgcn_readlane(v, 31);
  const int t2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (threadIdx.x & 63) >> 4;
  return v + (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
}

// wave 0 finds the digit where the count from the top reaches `need` in hist
// (bins in descending order); writes sh.digit / cum / cnt_d.  Lane l holds the
// 16 bins just below TK_BINS - 16 l in registers.
__device__ __forceinline__ void find_digit(const uint32_t* hist, int need, TopkShared& sh) {
  static_assert(TK_BINS == 1024, "16 bins per lane");
  if (threadIdx.x >= 64) return;
  const int lane = threadIdx.x;
  const int lo_bin = TK_BINS - 16 * (lane + 1);      // lane's bins: lo_bin .. lo_bin + 15
  uint32_t c[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const u32x4_t v = *(const u32x4_t*)(hist + lo_bin + 4 * q);
    c[4 * q] = v[0]; c[4 * q + 1] = v[1]; c[4 * q + 2] = v[2]; c[4 * q + 3] = v[3];
  }
  int sum = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) sum += (int)c[q];
  // inclusive scan over the lanes: inside each 16-lane row by DPP row shifts
  // (lanes without a source add 0), then the totals of the rows above
  int incl = sum;
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x111, 0xF, 0xF, false);   // row_shr:1
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x112, 0xF, 0xF, false);   // row_shr:2
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x114, 0xF, 0xF, false);   // row_shr:4
  incl += __builtin_amdgcn_update_dpp(0, incl, 0x118, 0xF, 0xF, false);   // row_shr:8
  {
    const int t0 = __builtin_amdgcn_readlane(incl, 15), t1 = __builtin_amdgcn_readlane(incl, 31);
    const int t2 = __builtin_amdgcn_readlane(incl, 47);
    const int row = lane >> 4;
    incl += (row >= 1 ? t0 : 0) + (row >= 2 ? t1 : 0) + (row >= 3 ? t2 : 0);
  }
  const int above = incl - sum;
  if (above < need && need <= incl) {   // exactly one lane
    int run = above, dig = lo_bin, cum = above, cnt = 0;
    bool found = false;
#pragma unroll
    for (int q = 15; q >= 0; --q) {      // top bin first
      const int cq = (int)c[q];
      const bool hit = !found && need <= run + cq;
      if (hit) { dig = lo_bin + q; cum = run; cnt = cq; }
      found = found || hit;
      run += cq;
    }
    sh.digit = dig; sh.cum = cum; sh.cnt_d = cnt;
  }
}

// Radix select on one 32-bit half of the keys among the elements whose other
// half / prefix matches.  HALF = 0: hi keys; HALF = 1: lo keys of the elements
// whose hi key equals hi_val.  Returns the decided bits in *prefix and the
// count still needed from the final group in *need; *tied reports whether the
// final group holds more elements than needed (only possible for HALF = 0).
template <class Src, int HALF>
__device__ __forceinline__ void radix_half(const Src& src, long long n, uint32_t lb, uint32_t k_and, uint32_t k_or,
                           uint32_t hi_val, int& need, uint32_t& prefix, bool& tied, TopkShared& sh,
                           int& hb) {
  constexpr int V = Src::V;
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
    for (long long e0 = (long long)V * tid; e0 < n; e0 += (long long)V * TK_THREADS) {
      uint32_t h[V], l[V];
      src.load(e0, h, l);
      const int rem = (int)min(n - e0, (long long)V);
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const uint32_t key = HALF == 0 ? h[v] : l[v];
        unsigned ok = (unsigned)(v < rem) & (unsigned)(h[v] >= lb) & (unsigned)((key & pmask) == prefix);
        if (HALF == 1) ok &= (unsigned)(h[v] == hi_val);
        if (ok) atomicAdd(&hist[(key >> shift) & dmask], 1u);
      }
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

// value of lane (lane ^ M) for M < 64, in VALU only: DPP quad permutes (1, 2),
// a quad reversal then a half-row mirror (4), a row rotation by 8 (8), and the
// gfx950 row swaps (16, 32), which hand each lane its own value and its
// partner's
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, false);
}
template <int M>
__device__ __forceinline__ uint32_t xchg_u32(uint32_t v) {
  if constexpr (M == 1) return dpp_u32<0xB1>(v);                  // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return dpp_u32<0x4E>(v);             // quad_perm [2,3,0,1]
  else if constexpr (M == 4) return dpp_u32<0x141>(dpp_u32<0x1B>(v));   // [3,2,1,0], then i <-> 7 - i
  else if constexpr (M == 8) return dpp_u32<0x128>(v);            // row_ror:8
  else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (threadIdx.x & 16) ? r[0] : r[1];
  } else {
    static_assert(M == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (threadIdx.x & 32) ? r[0] : r[1];
  }
}

// one compare-exchange step of a descending bitonic sort at (size, stride):
// thread t holds element t.  Partners in other waves trade through one of two
// LDS buffers (alternating, so one barrier per step suffices: a buffer is
// rewritten only after the barrier of the step that follows its readers).
template <int STRIDE>
__device__ __forceinline__ uint64_t bitonic_step(uint64_t x, int t, bool desc, TopkShared& sh, int P,
                                                 int& par) {
  uint64_t y;
  if constexpr (STRIDE >= 64) {
    uint64_t* b = sh.buf + (par ? TK_THREADS : 0);
    if (t < P) b[t] = x;
    __syncthreads();
    y = t < P ? b[t ^ STRIDE] : 0ull;
    par ^= 1;
  } else {
    // a wave whose threads all lie past P holds no key: it skips the work
    // (wave-uniform, so the lane exchanges of the other waves see whole waves)
    if (__builtin_amdgcn_readfirstlane(t & ~63) >= P) return x;
    const uint32_t lo = xchg_u32<STRIDE>((uint32_t)x), hi = xchg_u32<STRIDE>((uint32_t)(x >> 32));
    y = ((uint64_t)hi << 32) | lo;
  }
  // the lower lane of a descending block keeps the larger key, the upper the
  // smaller; ascending blocks the other way round (one compare, one select)
  const bool take_max = ((t & STRIDE) == 0) == desc;
  return ((x > y) == take_max) ? x : y;
}

// all strides of one merge size, largest first (compile-time strides)
template <int STRIDE>
__device__ __forceinline__ uint64_t bitonic_merge(uint64_t x, int t, int size, bool desc, TopkShared& sh,
                                                  int P, int& par) {
  if (STRIDE < size) x = bitonic_step<STRIDE>(x, t, desc, sh, P, par);
  if constexpr (STRIDE > 1) x = bitonic_merge<STRIDE / 2>(x, t, size, desc, sh, P, par);
  return x;
}

// Bitonic sort of sh.buf[0 .. P), descending, P a power of two <= TK_THREADS:
// thread t holds element t; partners closer than 64 sit in the same wave and
// trade through lane permutes, farther ones through LDS.
__device__ __forceinline__ void sort_desc_regs(TopkShared& sh, int P) {
  static_assert(2 * TK_THREADS <= TK_KMAX, "two exchange buffers");
  const int t = threadIdx.x;
  uint64_t x = t < P ? sh.buf[t] : 0ull;   // each thread reads and later writes only slot t first
  int par = 0;
  for (int size = 2; size <= P; size <<= 1)
    x = bitonic_merge<TK_THREADS / 2>(x, t, size, (t & size) == 0, sh, P, par);   // block of t descending?
  __syncthreads();
  if (t < P) sh.buf[t] = x;
  __syncthreads();
}

// the same order for P up to TK_KMAX, every compare-exchange through LDS
__device__ __forceinline__ void sort_desc_lds(TopkShared& sh, int P) {
  const int tid = threadIdx.x;
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

// Collection of the selected keys into sh.buf (sh.count = 0 on entry).  A wave
// claims the slots for CG groups of V elements per thread (8 elements) with one
// LDS atomic, so the atomic's return latency is paid once per 8 elements; its
// lanes fill the range in ballot order (mbcnt rank).
template <int V>
__device__ __forceinline__ constexpr int tk_cg() { return V >= 8 ? 1 : 8 / V; }
template <int V>
__device__ __forceinline__ void collect_groups(const uint32_t (&h)[tk_cg<V>()][V], const uint32_t (&l)[tk_cg<V>()][V],
                                               const bool (&take)[tk_cg<V>()][V], TopkShared& sh) {
  constexpr int CG = tk_cg<V>();
  uint64_t bal[CG][V];
  int tot = 0;
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int v = 0; v < V; ++v) {
      bal[c][v] = __ballot(take[c][v]);
      tot += __popcll(bal[c][v]);
    }
  if (tot == 0) return;   // wave-uniform
  int off = 0;
  if ((threadIdx.x & 63) == 0) off = atomicAdd(&sh.count, tot);
  off = __builtin_amdgcn_readfirstlane(off);
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const int slot = off + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal[c][v] >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)bal[c][v], 0u));
      if (take[c][v] && slot < TK_KMAX) sh.buf[slot] = ((uint64_t)h[c][v] << 32) | l[c][v];
      off += __popcll(bal[c][v]);
    }
}

// every element (hi, lo) with take(hi, lo), n >= 1, CG groups at a time.  The loads are not guarded
// (a guarded load is a branch with its own wait): past the end they read the
// last group again, which is in bounds, and the count mask drops it.
template <class Src, class Take>
__device__ __forceinline__ void collect_if(const Src& src, long long n, Take take_fn, TopkShared& sh) {
  constexpr int V = Src::V, CG = tk_cg<V>();
  const long long step = (long long)V * TK_THREADS;
  const long long last = ((n - 1) / V) * V;   // start of the last group
  for (long long g0 = 0; g0 < n; g0 += CG * step) {
    uint32_t h[CG][V], l[CG][V];
    int rem[CG];
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      const long long e0 = g0 + c * step + (long long)V * threadIdx.x;
      src.load(min(e0, last), h[c], l[c]);
      rem[c] = (int)max(0LL, min(n - e0, (long long)V));
    }
    bool take[CG][V];
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int v = 0; v < V; ++v) take[c][v] = (v < rem[c]) && take_fn(h[c][v], l[c][v]);
    collect_groups<V>(h, l, take, sh);
  }
}

// every element with hi >= t (no tie to resolve)
template <class Src>
__device__ __forceinline__ void collect_ge(const Src& src, long long n, uint32_t t, TopkShared& sh) {
  collect_if(src, n, [t](uint32_t h, uint32_t) { return h >= t; }, sh);
}

// hi > thr_hi, plus hi == thr_hi with lo >= thr_lo (the k-th score is tied)
template <class Src>
__device__ __forceinline__ void collect_tied(const Src& src, long long n, uint32_t lb, uint32_t thr_hi, uint32_t thr_lo,
                             TopkShared& sh) {
  collect_if(src, n, [=](uint32_t h, uint32_t l) {
    return (h >= lb) & ((h > thr_hi) | ((h == thr_hi) & (l >= thr_lo)));
  }, sh);
}

// k largest K64 = hi << 32 | lo among n elements -> sh.buf[0 .. min(k, n)), sorted
// descending when SORT.  Only elements with hi >= lb take part (lb from
// block_lower_bound, which keeps at least min(k, n) of them); hi_and / hi_or:
// AND / OR of their hi keys.
template <class Src, bool SORT>
__device__ __forceinline__ int select_topk(const Src& src, long long n, uint32_t lb, int k, uint32_t hi_and,
                           uint32_t hi_or, TopkShared& sh) {
  constexpr int V = Src::V;
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
    radix_half<Src, 0>(src, n, lb, hi_and, hi_or, 0u, need, pre, tied, sh, hb);
    thr_hi = pre;
    if (!tied) {
      all_eq_hi = true;       // take every element whose hi >= pre (pre has zero low bits)
    } else {
      // ties on the full hi key: resolve among them by the lo key (the index)
      uint32_t l_and = ~0u, l_or = 0u;
      for (long long e0 = (long long)V * tid; e0 < n; e0 += (long long)V * TK_THREADS) {
        uint32_t h[V], l[V];
        src.load(e0, h, l);
        const int rem = (int)min(n - e0, (long long)V);
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const bool tie = (v < rem) & (h[v] == thr_hi);
          l_and &= tie ? l[v] : ~0u;
          l_or |= tie ? l[v] : 0u;
        }
      }
      block_and_or(l_and, l_or, sh);
      __syncthreads();
      uint32_t lpre;
      bool t2;
      radix_half<Src, 1>(src, n, lb, l_and, l_or, thr_hi, need, lpre, t2, sh, hb);
      thr_lo = lpre;
    }
  } else {
    all_eq_hi = true;
    thr_hi = 0u;
  }
  // collect every selected key (exactly `want` of them) in one pass: per
  // group of V elements a wave takes one range of slots with one LDS atomic
  // and its lanes fill it in ballot order.  The slot only decides where an
  // element sits before the sort (or before the merge's own exact selection),
  // so the result does not depend on the order in which waves get ranges.
  if (tid == 0) sh.count = 0;
  __syncthreads();
  if (all_eq_hi) collect_ge(src, n, max(thr_hi, lb), sh);   // (the radix only counted hi >= lb)
  else collect_tied(src, n, lb, thr_hi, thr_lo, sh);
  __syncthreads();
  if (SORT) {
    int P = 1;
    while (P < want) P <<= 1;
    for (int e = want + tid; e < P; e += TK_THREADS) sh.buf[e] = 0ull;
    __syncthreads();
    if (P <= TK_THREADS) sort_desc_regs(sh, P);
    else sort_desc_lds(sh, P);
  }
  return want;
}

// Sort of the cnt unique keys in sh.buf (cnt <= TK_THREADS) by rank: the
// place of a key is the number of keys above it, counted by S = TK_THREADS / P
// threads per key (P: cnt rounded up to a power of two, at least 16) and
// summed over those lanes; keys placed below want are written back in order.
// Cheaper than the bitonic sort for a few hundred keys (its work grows with
// cnt squared).  Reads past cnt stay inside sh.buf (cnt + 8 S <= TK_KMAX) and
// are masked.
__device__ __forceinline__ void sort_desc_rank(TopkShared& sh, int cnt, int P, int want) {
  const int tid = threadIdx.x;
  const int S = TK_THREADS / P;
  const int i = tid / S, part = tid - i * S;
  const uint64_t x = i < cnt ? sh.buf[i] : 0ull;
  int above = 0;
  for (int j0 = part; i < cnt && j0 < cnt; j0 += 8 * S) {
    uint64_t y[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) y[u] = sh.buf[j0 + u * S];   // eight reads in flight
#pragma unroll
    for (int u = 0; u < 8; ++u) above += (j0 + u * S < cnt && y[u] > x) ? 1 : 0;
  }
  for (int w = 1; w < S; w <<= 1) above += __shfl_xor(above, w, 64);
  __syncthreads();   // every read of the unsorted keys is done
  if (part == 0 && i < cnt && above < want) sh.buf[above] = x;
  __syncthreads();
}

// The want largest keys of a whole chunk of NV * 4 * TK_THREADS scores at p
// (16-byte aligned; indices base + e), sorted into sh.buf, with the scores
// held in registers (NV vectors of 4 per thread).  A bound b with at least
// want threads whose largest key is at or above it, so at least want
// elements, comes from two histogram passes over the thread maxima: the top
// 10 bits of the order key, then the next 10 inside the bin where the count
// from the top reaches want.  The elements at or above b are collected and,
// when they fit one sort (TK_THREADS), sorted; the first want are the answer.
// Returns want, or -1 when too many elements lie at or above b (heavy ties):
// the caller then runs the general selection.
template <int NV>
__device__ __forceinline__ int chunk_select_regs(const float* __restrict__ p, long long base, int want,
                                                 TopkShared& sh) {
  const int tid = threadIdx.x;
  for (int e = tid; e < 2 * TK_BINS; e += TK_THREADS) sh.hist[e / TK_BINS][e % TK_BINS] = 0u;
  if (tid == 0) sh.count = 0;
  f32x4_t v[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) v[u] = *(const f32x4_t*)(p + 4 * tid + 4 * TK_THREADS * u);
  uint32_t h[NV][4];
  uint32_t lmax = 0u;
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      h[u][q] = ord_key(v[u][q]);
      lmax = max(lmax, h[u][q]);
    }
  __syncthreads();   // the histograms are clear
  atomicAdd(&sh.hist[0][lmax >> 22], 1u);
  __syncthreads();
  find_digit(sh.hist[0], want, sh);
  __syncthreads();
  const uint32_t d1 = (uint32_t)sh.digit;
  const int need = want - sh.cum;
  if ((lmax >> 22) == d1) atomicAdd(&sh.hist[1][(lmax >> 12) & (TK_BINS - 1)], 1u);
  __syncthreads();
  find_digit(sh.hist[1], need, sh);
  __syncthreads();
  const uint32_t b = (d1 << 22) | ((uint32_t)sh.digit << 12);
  // collect every element at or above b: a thread's count, its place among the
  // wave's by an inclusive scan, one atomic per wave for the wave's range of slots
  int mine = 0;
#pragma unroll
  for (int u = 0; u < NV; ++u)
#pragma unroll
    for (int q = 0; q < 4; ++q) mine += h[u][q] >= b ? 1 : 0;
  const int incl = wave_incl_scan(mine);
  const int wtot = __builtin_amdgcn_readlane(incl, 63);
  if (wtot > 0) {   // wave-uniform
    int off = 0;
    if ((tid & 63) == 0) off = atomicAdd(&sh.count, wtot);
    off = __builtin_amdgcn_readfirstlane(off) + incl - mine;
#pragma unroll
    for (int u = 0; u < NV; ++u)
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (h[u][q] >= b) {
          if (off < TK_KMAX)
            sh.buf[off] = ((uint64_t)h[u][q] << 32) |
                          (0xFFFFFFFFu - (uint32_t)(base + 4 * tid + 4 * TK_THREADS * u + q));
          ++off;
        }
  }
  __syncthreads();
  const int cnt = sh.count;
  __syncthreads();   // every thread has the count before anything rewrites it
  if (cnt > TK_THREADS) return -1;
  int P = 16;
  while (P < cnt) P <<= 1;
  if (P <= 512) {
    sort_desc_rank(sh, cnt, P, want);
  } else {
    for (int e = cnt + tid; e < P; e += TK_THREADS) sh.buf[e] = 0ull;
    __syncthreads();
    sort_desc_regs(sh, P);
  }
  return want;
}

// top-k of the scores p[0 .. n) (indices base + e): cached in LDS when they fit
template <bool SORT>
__device__ __forceinline__ int select_row(const float* __restrict__ p, long long n, long long base, int k,
                          uint32_t* cache, bool use_cache, TopkShared& sh) {
  const int want = (int)min((long long)k, n);
  uint32_t a = ~0u, o = 0u, lmax = ~0u;
  if (use_cache) {
    const long long n4 = (((uintptr_t)p & 15u) == 0) ? (n & ~3LL) : 0;   // vector part if aligned
    // TK_LDU loads in flight per thread before any is used (one at a time, the
    // copy would take one memory latency per iteration)
    for (long long e = 4LL * threadIdx.x; e < n4; e += 4LL * TK_THREADS * TK_LDU) {
      f32x4_t v[TK_LDU];
#pragma unroll
      for (int u = 0; u < TK_LDU; ++u) {
        const long long eu = e + 4LL * TK_THREADS * u;
        if (eu < n4) v[u] = *(const f32x4_t*)(p + eu);
      }
#pragma unroll
      for (int u = 0; u < TK_LDU; ++u) {
        const long long eu = e + 4LL * TK_THREADS * u;
        if (eu < n4) {
          u32x4_t ok;
          ok[0] = ord_key(v[u][0]); ok[1] = ord_key(v[u][1]); ok[2] = ord_key(v[u][2]); ok[3] = ord_key(v[u][3]);
          *(u32x4_t*)(cache + eu) = ok;
          const uint32_t m4 = max(max(ok[0], ok[1]), max(ok[2], ok[3]));
          lmax = lmax == ~0u ? m4 : max(lmax, m4);
        }
      }
    }
    for (long long e = n4 + threadIdx.x; e < n; e += TK_THREADS) {
      const uint32_t ok = ord_key(p[e]);
      cache[e] = ok;
      lmax = lmax == ~0u ? ok : max(lmax, ok);
    }
    const uint32_t lb = block_lower_bound(lmax, want, sh);   // its barriers also publish the cache
    const LdsRowSrc src{cache, base};
    for (long long e0 = 4LL * threadIdx.x; e0 < n; e0 += 4LL * TK_THREADS) {
      uint32_t h[4], l[4];
      src.load(e0, h, l);
#pragma unroll
      for (int v = 0; v < 4; ++v)
        if (e0 + v < n && h[v] >= lb) { a &= h[v]; o |= h[v]; }
    }
    block_and_or(a, o, sh);
    __syncthreads();
    return select_topk<LdsRowSrc, SORT>(src, n, lb, k, a, o, sh);
  }
  const RowSrc src{p, base};
  for (long long e = threadIdx.x; e < n; e += TK_THREADS) {
    const uint32_t ok = ord_key(p[e]);
    a &= ok;
    o |= ok;
  }
  block_and_or(a, o, sh);
  __syncthreads();
  return select_topk<RowSrc, SORT>(src, n, 0u, k, a, o, sh);
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
    uint32_t lmax = ~0u;
    if ((ncand & 1) == 0) {   // rows start 16-byte aligned: two keys per load
      typedef unsigned long long u64x2_t __attribute__((ext_vector_type(2)));
      for (long long e = 2LL * threadIdx.x; e < ncand; e += 2LL * TK_THREADS * TK_LDU) {
        u64x2_t kk[TK_LDU];
#pragma unroll
        for (int u = 0; u < TK_LDU; ++u) {
          const long long eu = e + 2LL * TK_THREADS * u;
          if (eu < ncand) kk[u] = *(const u64x2_t*)(cp + eu);
        }
#pragma unroll
        for (int u = 0; u < TK_LDU; ++u) {
          const long long eu = e + 2LL * TK_THREADS * u;
          if (eu < ncand) {
            *(u64x2_t*)(cache64 + eu) = kk[u];
            const uint32_t m2 = max((uint32_t)(kk[u][0] >> 32), (uint32_t)(kk[u][1] >> 32));
            lmax = lmax == ~0u ? m2 : max(lmax, m2);
          }
        }
      }
    } else {
      for (long long e = threadIdx.x; e < ncand; e += TK_THREADS) {
        const uint64_t key = cp[e];
        cache64[e] = key;
        lmax = lmax == ~0u ? (uint32_t)(key >> 32) : max(lmax, (uint32_t)(key >> 32));
      }
    }
    // padding keys (0) only ever lower the bound
    const uint32_t lb = block_lower_bound(lmax, want, sh);
    const KeyLdsSrc src{cache64};
    if ((ncand & 1) == 0) {
      for (long long e0 = 2LL * threadIdx.x; e0 < ncand; e0 += 2LL * TK_THREADS) {
        uint32_t h[2], l[2];
        src.load(e0, h, l);
#pragma unroll
        for (int v = 0; v < 2; ++v)
          if (h[v] >= lb) { a &= h[v]; o |= h[v]; }
      }
    } else {
      for (long long e = threadIdx.x; e < ncand; e += TK_THREADS) {
        const uint32_t h = (uint32_t)(cache64[e] >> 32);
        if (h >= lb) { a &= h; o |= h; }
      }
    }
    block_and_or(a, o, sh);
    __syncthreads();
    got = select_topk<KeyLdsSrc, true>(src, ncand, lb, want, a, o, sh);
  } else {
    for (long long e = threadIdx.x; e < ncand; e += TK_THREADS) {
      a &= (uint32_t)(cp[e] >> 32);
      o |= (uint32_t)(cp[e] >> 32);
    }
    block_and_or(a, o, sh);
    __syncthreads();
    got = select_topk<KeySrc, true>(KeySrc{cp}, ncand, 0u, want, a, o, sh);
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

// ---------------------------------------------------------------------------
// Two stages with sorted lists.  A chunk (16 k elements, or shorter so that a
// row has 16 of them) holds on average k / nchunks of the row's top-k (the scores of a row are spread over its
// chunks), so stage 1 keeps only the T largest of each chunk, sorted, plus the
// (T+1)-th as the chunk's threshold, with T a few standard deviations above
// that mean.  Stage 2 places every listed key in the merged order directly
// (its place in its own list plus the keys above it in the other lists), one
// workgroup per list.  The result is exact when every chunk was reported whole
// (threshold 0) or the want-th merged key is above every threshold: any
// unreported element lies below its chunk's threshold.  Otherwise one
// workgroup selects from the whole row (a rare, slow path).
// ---------------------------------------------------------------------------
static constexpr int TK_LIST_KEYS = 8192;   // list keys of a row held in LDS by the merge

// stage 1: the T largest keys of one chunk, descending, padded with 0 to Tp,
// and the chunk's threshold (its (T+1)-th largest key, 0 if it has at most T).
// NV > 0: chunks of NV * 4 * TK_THREADS elements; whole, aligned chunks take
// the register path
template <int NV>
__global__ __launch_bounds__(TK_THREADS) void topk_chunk_sorted_kernel(
    const float* __restrict__ I, const int* __restrict__ q_pos, long long N_cap, int m, int T, int Tp,
    long long chunk, int nchunks, int use_cache, uint64_t* __restrict__ lists, uint64_t* __restrict__ thr) {
  __shared__ TopkShared sh;
  extern __shared__ __attribute__((aligned(16))) uint32_t cache[];
  const size_t row = blockIdx.y;
  const int c = blockIdx.x;
  const long long n = row_nvis(q_pos, row, N_cap, m);
  const long long lo = (long long)c * chunk;
  const long long len = max(0LL, min(n, lo + chunk) - lo);
  const float* cp = I + row * (size_t)N_cap + lo;
  int got = -1;
  if constexpr (NV > 0) {
    if (len == chunk && ((uintptr_t)cp & 15u) == 0 && T + 1 <= TK_THREADS) got = chunk_select_regs<NV>(cp, lo, T + 1, sh);
  }
  if (got < 0) got = len > 0 ? select_row<true>(cp, len, lo, T + 1, cache, use_cache != 0, sh) : 0;
  uint64_t* dst = lists + (row * (size_t)nchunks + c) * (size_t)Tp;
  for (int e = threadIdx.x; e < Tp; e += TK_THREADS) dst[e] = (e < got && e < T) ? sh.buf[e] : 0ull;
  if (threadIdx.x == 0) thr[row * (size_t)nchunks + c] = got > T ? sh.buf[T] : 0ull;
}

// number of keys of the descending list p[0 .. L) above x (GE: at or above)
template <bool GE>
__device__ __forceinline__ int count_above(const uint64_t* p, int L, uint64_t x) {
  int lo = 0, len = L;
  while (len > 0) {
    const int half = len >> 1;
    const uint64_t v = p[lo + half];
    if (GE ? (v >= x) : (v > x)) {
      lo += half + 1;
      len -= half + 1;
    } else {
      len = half;
    }
  }
  return lo;
}

struct OpAdd { __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a + b; } };

// stage 2: the k largest of the union of a row's sorted lists, one workgroup
// per (list, row).  Keys are unique and every real key is nonzero, so a key's
// place in the merged order is its place in its own list plus the number of
// keys above it in the other lists (binary searches in LDS); the workgroup
// writes the keys of its list whose place is below want.  All workgroups of a
// row reach the same exactness verdict from the same lists: the result is exact
// when every chunk was reported whole (threshold 0) or at least want keys of
// the union lie above the largest threshold (then no key a chunk left out can
// rank among the want largest).  Otherwise the row's first workgroup selects
// from the whole row and the others write nothing.
__global__ __launch_bounds__(TK_THREADS) void topk_rank_lists_kernel(
    const uint64_t* __restrict__ lists, const uint64_t* __restrict__ thr, const float* __restrict__ I,
    const int* __restrict__ q_pos, long long N_cap, int m, int k, int nchunks, int T, int Tp,
    int* __restrict__ idx_out, float* __restrict__ val_out) {
  __shared__ TopkShared sh;
  __shared__ int s_exact;
  extern __shared__ __attribute__((aligned(16))) uint64_t lds64[];   // nchunks * Tp keys, then Tp places
  const int own = blockIdx.x;
  const size_t row = blockIdx.y;
  const int tid = threadIdx.x;
  const long long n = row_nvis(q_pos, row, N_cap, m);
  const int want = (int)min((long long)k, n);
  const int tot = nchunks * Tp;
  uint64_t* A = lds64;
  int* place = (int*)(lds64 + tot);
  const uint64_t* lp = lists + row * (size_t)tot;
  // the thresholds: wave 0, one chunk per lane, loaded with the lists
  uint64_t tl = 0ull;
  if (tid < 64)
    for (int c = tid; c < nchunks; c += 64) tl = max(tl, thr[row * (size_t)nchunks + c]);
  for (int e = tid; e < tot; e += TK_THREADS) A[e] = lp[e];
  for (int e = tid; e < Tp; e += TK_THREADS) place[e] = e;
  __syncthreads();
  if (tid < 64) {
#pragma unroll
    for (int x = 1; x < 64; x <<= 1) {
      const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)tl, x, 64);
      const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(tl >> 32), x, 64);
      tl = max(tl, ((uint64_t)hi << 32) | lo);
    }
    uint32_t above = 0;
    if (tl != 0ull)
      for (int c = tid; c < nchunks; c += 64) above += (uint32_t)count_above<false>(A + (size_t)c * Tp, Tp, tl);
    above = wave_reduce_u32(above, OpAdd{});
    if (tid == 0) s_exact = (tl == 0ull || want == 0 || (int)above >= want) ? 1 : 0;
  }
  // places: thread (e = tid mod Tp, group tid / Tp) counts the keys above key e
  // of this list in lists group, group + G, ... (G = TK_THREADS / Tp groups; Tp
  // is a power of two), two fixed-step searches at a time, and adds the count
  // to the key's place once
  const uint64_t* mine = A + (size_t)own * Tp;
  if (Tp <= TK_THREADS) {
    const int G = TK_THREADS / Tp;
    const int e = tid & (Tp - 1), grp = tid / Tp;
    const uint64_t x = e < T ? mine[e] : 0ull;
    if (x != 0ull) {
      int cnt = 0;
      for (int l0 = grp; l0 < nchunks; l0 += 2 * G) {
        const int l1 = l0 + G;
        const uint64_t* p0 = A + (size_t)l0 * Tp;
        const uint64_t* p1 = A + (size_t)min(l1, nchunks - 1) * Tp;
        int c0 = 0, c1 = 0;
        for (int st = Tp >> 1; st > 0; st >>= 1) {
          const uint64_t v0 = p0[c0 + st - 1], v1 = p1[c1 + st - 1];
          c0 += v0 > x ? st : 0;
          c1 += v1 > x ? st : 0;
        }
        c0 += p0[c0] > x ? 1 : 0;
        c1 += p1[c1] > x ? 1 : 0;
        cnt += (l0 != own ? c0 : 0) + (l1 < nchunks && l1 != own ? c1 : 0);
      }
      if (cnt) atomicAdd(&place[e], cnt);
    }
  } else {
    // (element, other list) pairs spread over the threads
    const int others = nchunks - 1;
    for (int q = tid; q < T * others; q += TK_THREADS) {
      const int e = q / others, li = q - e * others;
      const int l = li + (li >= own ? 1 : 0);
      const uint64_t x = mine[e];
      if (x != 0ull) {
        const int c = count_above<false>(A + (size_t)l * Tp, Tp, x);
        if (c) atomicAdd(&place[e], c);
      }
    }
  }
  __syncthreads();
  const float* rp = I + row * (size_t)N_cap;
  if (s_exact) {
    for (int e = tid; e < T; e += TK_THREADS) {
      const uint64_t x = mine[e];
      const int r = place[e];
      if (x != 0ull && r < want) {
        const int idx = (int)(0xFFFFFFFFu - (uint32_t)x);
        idx_out[row * (size_t)k + r] = idx;
        if (val_out) val_out[row * (size_t)k + r] = rp[idx];
      }
    }
    // exact means the union holds at least want keys: places want .. k - 1 are empty
    if (own == 0)
      for (int e = want + tid; e < k; e += TK_THREADS) {
        idx_out[row * (size_t)k + e] = -1;
        if (val_out) val_out[row * (size_t)k + e] = -INFINITY;
      }
    return;
  }
  if (own != 0) return;   // uniform per workgroup
  const int got = select_row<true>(rp, n, 0, k, (uint32_t*)lds64, false, sh);
  for (int e = tid; e < k; e += TK_THREADS) {
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

static bool topk_two_stage(long long rows, long long N_cap, int k, long long* chunk, int* nchunks) {
  long long ch = 16LL * k;
  if (rows >= 512 || N_cap < 2 * ch) return false;
  // shorter chunks, down to 4 elements per thread, until a row has 16: more
  // workgroups for short rows and shorter lists to merge (depends on the row
  // length and k only, so a workspace sized for some rows serves fewer)
  while (ch / 2 >= 4LL * TK_THREADS && (N_cap + ch - 1) / ch < 16) ch /= 2;
  *chunk = ch;
  *nchunks = (int)((N_cap + ch - 1) / ch);
  return true;
}

// keys kept per chunk for the sorted-list stages: T (the chunk selects T + 1),
// list stride Tp; false when the lists do not fit the merge's LDS
static bool topk_lists(int k, int nchunks, int* T, int* Tp) {
  const double mean = (double)k / nchunks;
  const int est = (int)std::min<double>((double)k, std::ceil(mean + 6.0 * std::sqrt(mean) + 2.0));
  int p = 1;
  while (p < est) p <<= 1;
  *Tp = p;
  *T = p <= k ? p - 1 : k;   // a selection of T + 1 = p keys sorts in a power-of-two block
  if (*T < 1) *T = std::min(k, 1);
  return (long long)nchunks * p <= TK_LIST_KEYS && *T + 1 <= TK_KMAX;
}

size_t topk_workspace_bytes(int B, int Tq, long long N_cap, int k) {
  long long chunk;
  int nchunks, T, Tp;
  const long long rows = (long long)B * Tq;
  if (!topk_two_stage(rows, N_cap, k, &chunk, &nchunks)) return 0;
  if (topk_lists(k, nchunks, &T, &Tp))
    return (size_t)rows * (size_t)nchunks * ((size_t)Tp + 1) * sizeof(uint64_t);
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
  int T, Tp;
  if (topk_two_stage(rows, a.N_cap, a.k, &chunk, &nchunks) && topk_lists(a.k, nchunks, &T, &Tp)) {
    uint64_t* lists = (uint64_t*)a.ws;
    uint64_t* thr = lists + (size_t)rows * nchunks * Tp;
    const bool c1 = chunk <= TK_CACHE32;
    const size_t l1 = c1 ? ((size_t)chunk * 4 + 15) / 16 * 16 : 0;
    const size_t l2 = (size_t)nchunks * Tp * sizeof(uint64_t) + (size_t)Tp * sizeof(int);
    const long long per = 4LL * TK_THREADS;   // elements per register vector over the workgroup
    auto kfn = chunk == per ? topk_chunk_sorted_kernel<1>
             : chunk == 2 * per ? topk_chunk_sorted_kernel<2>
             : chunk == 4 * per ? topk_chunk_sorted_kernel<4>
             : chunk == 8 * per ? topk_chunk_sorted_kernel<8> : topk_chunk_sorted_kernel<0>;
    if (!set_lds((const void*)kfn, l1) || !set_lds((const void*)topk_rank_lists_kernel, l2)) return -1;
    hipLaunchKernelGGL(kfn, dim3((unsigned)nchunks, (unsigned)rows), dim3(TK_THREADS), l1, st,
                       a.I, a.q_pos, a.N_cap, a.m, T, Tp, chunk, nchunks, (int)c1, lists, thr);
    hipLaunchKernelGGL(topk_rank_lists_kernel, dim3((unsigned)nchunks, (unsigned)rows), dim3(TK_THREADS), l2, st,
                       lists, thr, a.I, a.q_pos, a.N_cap, a.m, a.k, nchunks, T, Tp, a.idx, a.val);
  } else if (topk_two_stage(rows, a.N_cap, a.k, &chunk, &nchunks)) {
    uint64_t* cand = (uint64_t*)a.ws;
    const bool c1 = chunk <= TK_CACHE32;
    const long long ncand = (long long)nchunks * a.k;
    const bool c2 = ncand <= TK_CACHE64;
    // caches padded to 16 bytes: vector reads of the last group stay inside them
    const size_t l1 = c1 ? ((size_t)chunk * 4 + 15) / 16 * 16 : 0, l2 = c2 ? ((size_t)ncand * 8 + 15) / 16 * 16 : 0;
    if (!set_lds((const void*)topk_chunk_kernel, l1) || !set_lds((const void*)topk_merge_kernel, l2))
      return -1;
    hipLaunchKernelGGL(topk_chunk_kernel, dim3((unsigned)nchunks, (unsigned)rows), dim3(TK_THREADS),
                       l1, st, a.I, a.q_pos, a.N_cap, a.m, a.k, chunk, nchunks, (int)c1, cand);
    hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)rows), dim3(TK_THREADS), l2, st, cand, a.I,
                       a.q_pos, a.N_cap, a.m, a.k, nchunks, (int)c2, a.idx, a.val);
  } else {
    const bool c1 = a.N_cap <= TK_CACHE32;
    const size_t l1 = c1 ? ((size_t)a.N_cap * 4 + 15) / 16 * 16 : 0;
    if (!set_lds((const void*)topk_rows_kernel, l1)) return -1;
    hipLaunchKernelGGL(topk_rows_kernel, dim3((unsigned)rows), dim3(TK_THREADS), l1, st, a.I,
                       a.q_pos, a.N_cap, a.m, a.k, (int)c1, a.idx, a.val);
  }
  return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace csa
