// C ABI of the CSA/HCA core (declared in include/csa.h).  Every entry point
// validates its arguments on the host first; on a non-OK status nothing has
// been enqueued and nothing written.  No device memory is allocated here.
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "../../include/csa.h"
#include "csa_internal.h"

// Device scratch of csa_sparse_mqa_noalloc: the split partials of attention,
// for callers that cannot allocate.  Every GPU the library runs on holds its own
// copy until the process ends.  In host code `scratch` names a host-side
// stand-in, never the device memory: host code uses the address that
// hipGetSymbolAddress returns for the current device (scratch_ptr below).
static __device__ __align__(256) unsigned char scratch[CSA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = 0;
  return CSA_OK;
}

bool dtype_valid(int dt) {
  return dt == CSA_F32 || dt == CSA_BF16 || dt == CSA_FP8_E4M3 || dt == CSA_MXFP4 || dt == CSA_KV_MIXED;
}

}  // namespace

// the checks of one compression (also every job of a batch); CSA_OK or the
// status of the first failure, with `who` naming the call in the message
static int check_compress(const csa_compress_job& j, const char* who) {
  const void *C_a = j.C_a, *C_b = j.C_b, *E = j.E;
  const float* gamma = j.gamma;
  const float* E_scale = j.E_scale;
  const int in_dtype = j.in_dtype, out_dtype = j.out_dtype, B = j.B, c = j.c, m = j.m;
  const int overlap = j.overlap, rope_dim = j.rope_dim;
  const long long R = j.R, in_batch_stride = j.in_batch_stride, tok_base = j.tok_base, T = j.T;
  const long long s_begin = j.s_begin, s_end = j.s_end, out_ring = j.out_ring;
  const long long out_batch_stride = j.out_batch_stride;
  const float eps = j.eps;
  if (!C_a || !E) return fail(CSA_E_NULL, "%s: C_a and E are required", who);
  if (overlap != 0 && overlap != 1) return fail(CSA_E_SHAPE, "%s: overlap must be 0 or 1", who);
  if (overlap && !C_b) return fail(CSA_E_NULL, "%s: C_b is required when overlap = 1", who);
  if (in_dtype != CSA_F32 && in_dtype != CSA_BF16)
    return fail(CSA_E_DTYPE, "%s: in_dtype must be F32 or BF16", who);
  if (!dtype_valid(out_dtype)) return fail(CSA_E_DTYPE, "%s: unknown out_dtype", who);
  if ((out_dtype == CSA_FP8_E4M3 || out_dtype == CSA_MXFP4 || out_dtype == CSA_KV_MIXED) && !E_scale)
    return fail(CSA_E_NULL, "%s: E_scale is required for FP8, MXFP4 and mixed output", who);
  if (out_dtype == CSA_KV_MIXED && (rope_dim % 8 || (c - rope_dim) % 8 || out_batch_stride % c))
    return fail(CSA_E_SHAPE, "%s: mixed rows need rope_dim and c - rope_dim multiples of 8 and "
                "out_batch_stride %% c == 0", who);
  if (out_dtype == CSA_MXFP4 && (c % 32 || out_batch_stride % c))
    return fail(CSA_E_SHAPE, "%s: MXFP4 output needs c %% 32 == 0 and out_batch_stride %% c == 0", who);
  if (B < 1 || R < 1 || c < 1 || m < 1 || T < 1)
    return fail(CSA_E_SHAPE, "%s: B, R, c, m and T must be >= 1", who);
  if (c > 1024) return fail(CSA_E_UNSUPPORTED, "%s: c = %d exceeds 1024", who, c);
  if (in_batch_stride < R * c)
    return fail(CSA_E_SHAPE, "%s: in_batch_stride %lld < R * c", who, in_batch_stride);
  if (tok_base < 0) return fail(CSA_E_SHAPE, "%s: tok_base < 0", who);
  if (s_begin < 0 || s_end < s_begin) return fail(CSA_E_SHAPE, "%s: bad entry range", who);
  const long long n_entries = (T + m - 1) / m;
  if (s_end > n_entries)
    return fail(CSA_E_SHAPE, "%s: s_end %lld > ceil(T/m) = %lld", who, s_end, n_entries);
  if (s_end - s_begin > 2147483647LL) return fail(CSA_E_UNSUPPORTED, "%s: too many entries", who);
  if (rope_dim < 0 || rope_dim > c || (rope_dim & 1) || ((c - rope_dim) & 1))
    return fail(CSA_E_SHAPE, "%s: rope_dim must be even, <= c, with c - rope_dim even", who);
  if (gamma && !(eps >= 0.f)) return fail(CSA_E_SHAPE, "%s: eps must be >= 0", who);
  if (out_ring < 0) return fail(CSA_E_SHAPE, "%s: out_ring < 0", who);
  if (out_ring > 0 && s_end - s_begin > out_ring)
    return fail(CSA_E_SHAPE, "%s: more entries than ring rows (rows would collide)", who);
  const long long rows_out = out_ring > 0 ? out_ring : s_end;
  if (out_batch_stride < rows_out * c && B > 1)
    return fail(CSA_E_SHAPE, "%s: out_batch_stride too small for the rows written", who);
  if (out_dtype == CSA_FP8_E4M3 && out_batch_stride % c)
    return fail(CSA_E_SHAPE, "%s: FP8 output needs out_batch_stride %% c == 0", who);
  if (s_end > s_begin) {
    // every candidate token < T of the requested entries must be among the given rows
    const long long first = overlap ? (m * (s_begin - 1) > 0 ? m * (s_begin - 1) : 0) : m * s_begin;
    const long long last = (m * s_end < T ? m * s_end : T) - 1;
    if (first < tok_base || last >= tok_base + R)
      return fail(CSA_E_SHAPE,
                  "%s: tokens [%lld, %lld] needed but rows hold [%lld, %lld)", who, first,
                  last, tok_base, tok_base + R);
  }
  return CSA_OK;
}

static csa::CompressArgs compress_args(const csa_compress_job& j) {
  return csa::CompressArgs{j.C_a, j.Z_a, j.C_b, j.Z_b, j.in_dtype, j.B, j.R, j.in_batch_stride,
                           j.tok_base, j.T, j.T_len, j.c, j.m, j.overlap, j.s_begin, j.s_end, j.gamma, j.eps,
                           j.rope_dim, j.rope_base, j.pos_stride, j.pos_offset, j.E, j.out_dtype,
                           j.E_scale, j.out_batch_stride, j.out_ring};
}

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_status_str(int status) {
  switch (status) {
    case CSA_OK: return "ok";
    case CSA_E_NULL: return "null pointer";
    case CSA_E_SHAPE: return "invalid shape or range";
    case CSA_E_DTYPE: return "invalid or unsupported dtype";
    case CSA_E_UNSUPPORTED: return "unsupported configuration";
    case CSA_E_WORKSPACE: return "workspace too small";
    case CSA_E_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* csa_last_error(void) { return g_err; }

int csa_compress(const void* C_a, const void* Z_a, const void* C_b, const void* Z_b, int in_dtype,
                 int B, long long R, long long in_batch_stride, long long tok_base, long long T,
                 const int* T_len, int c, int m, int overlap, long long s_begin, long long s_end,
                 const float* gamma, float eps, int rope_dim, float rope_base,
                 long long pos_stride, long long pos_offset,
                 void* E, int out_dtype, float* E_scale, long long out_batch_stride,
                 long long out_ring, void* stream) {
  const csa_compress_job j{C_a, Z_a, C_b, Z_b, in_dtype, B, R, in_batch_stride, tok_base, T, T_len, c, m,
                           overlap, s_begin, s_end, gamma, eps, rope_dim, rope_base, pos_stride,
                           pos_offset, E, out_dtype, E_scale, out_batch_stride, out_ring};
  const int st = check_compress(j, "csa_compress");
  if (st != CSA_OK) return st;
  if (s_end == s_begin) return ok();
  const csa::CompressArgs a = compress_args(j);
  if (csa::launch_compress(&a, 1, (hipStream_t)stream) != 0)
    return fail(CSA_E_HIP, "csa_compress: kernel launch failed");
  return ok();
}

int csa_compress_batch(const csa_compress_job* jobs, int n_jobs, void* workspace, size_t workspace_bytes,
                       void* stream) {
  if (!jobs) return fail(CSA_E_NULL, "csa_compress_batch: jobs is NULL");
  if (n_jobs < 1 || n_jobs > CSA_COMPRESS_MAX_JOBS)
    return fail(CSA_E_SHAPE, "csa_compress_batch: n_jobs = %d outside [1, %d]", n_jobs,
                CSA_COMPRESS_MAX_JOBS);
  csa::CompressArgs a[CSA_COMPRESS_MAX_JOBS];
  int n = 0;
  for (int q = 0; q < n_jobs; ++q) {
    char who[48];
    snprintf(who, sizeof(who), "csa_compress_batch: job %d", q);
    const int st = check_compress(jobs[q], who);
    if (st != CSA_OK) return st;
    if (jobs[q].s_end > jobs[q].s_begin) a[n++] = compress_args(jobs[q]);
  }
  if (workspace) {
    const size_t need = n > 0 ? csa::compress_workspace_bytes(a, n) : 0;
    if (workspace_bytes < need)
      return fail(CSA_E_WORKSPACE, "csa_compress_batch: workspace of %zu bytes, %zu needed", workspace_bytes,
                  need);
  }
  if (n > 0 && csa::launch_compress(a, n, (hipStream_t)stream, workspace, workspace_bytes) != 0)
    return fail(CSA_E_HIP, "csa_compress_batch: kernel launch failed");
  return ok();
}

size_t csa_compress_workspace_size(const csa_compress_job* jobs, int n_jobs) {
  if (!jobs || n_jobs < 1 || n_jobs > CSA_COMPRESS_MAX_JOBS) return 0;
  csa::CompressArgs a[CSA_COMPRESS_MAX_JOBS];
  int n = 0;
  for (int q = 0; q < n_jobs; ++q)
    if (check_compress(jobs[q], "csa_compress_workspace_size") == CSA_OK && jobs[q].s_end > jobs[q].s_begin)
      a[n++] = compress_args(jobs[q]);
  const size_t need = n > 0 ? csa::compress_workspace_bytes(a, n) : 0;
  ok();   // a failing job counts for nothing; it leaves no error behind
  return need;
}

}  // extern "C"

// the checks of csa_index_score's arguments (fn names the caller in the error)
static int check_index(const char* fn, const void* q_I, int q_dtype, const float* w_I, const void* K_I,
                       int k_dtype, const float* K_scale, const int* q_pos, int B, int Tq, int H_I, int d_I,
                       long long N_cap, int m, float* I_out) {
  if (!q_I || !w_I || !K_I || !q_pos || !I_out)
    return fail(CSA_E_NULL, "%s: q_I, w_I, K_I, q_pos and I_out are required", fn);
  if (q_dtype != CSA_F32 && q_dtype != CSA_BF16) return fail(CSA_E_DTYPE, "%s: q_dtype must be F32 or BF16", fn);
  if (!dtype_valid(k_dtype)) return fail(CSA_E_DTYPE, "%s: unknown k_dtype", fn);
  if (q_dtype == CSA_F32 && k_dtype != CSA_F32) return fail(CSA_E_DTYPE, "%s: F32 queries need F32 keys", fn);
  if (q_dtype == CSA_BF16 && k_dtype == CSA_F32)
    return fail(CSA_E_DTYPE, "%s: BF16 queries need BF16, FP8 or MXFP4 keys", fn);
  if ((k_dtype == CSA_FP8_E4M3 || k_dtype == CSA_MXFP4) && !K_scale)
    return fail(CSA_E_NULL, "%s: K_scale is required for FP8 and MXFP4 keys", fn);
  if (k_dtype == CSA_MXFP4 && d_I % 32) return fail(CSA_E_SHAPE, "%s: MXFP4 keys need d_I %% 32 == 0", fn);
  if (B < 1 || Tq < 1 || H_I < 1 || d_I < 1 || N_cap < 1 || m < 1)
    return fail(CSA_E_SHAPE, "%s: sizes must be >= 1", fn);
  if (H_I > 64 || d_I > 256 || H_I * (d_I + 1) > 16384)
    return fail(CSA_E_UNSUPPORTED, "%s: H_I <= 64 and d_I <= 256 are supported", fn);
  if (N_cap > 2147483647LL || (long long)B * Tq > 65535LL * 65535LL)
    return fail(CSA_E_UNSUPPORTED, "%s: N_cap must fit int32", fn);
  if (Tq > 65535 || B > 65535) return fail(CSA_E_UNSUPPORTED, "%s: B, Tq <= 65535", fn);
  return CSA_OK;
}

extern "C" {

int csa_index_score(const void* q_I, int q_dtype, const float* w_I,
                    const void* K_I, int k_dtype, const float* K_scale, const int* q_pos,
                    int B, int Tq, int H_I, int d_I, long long N_cap, int m,
                    float* I_out, void* stream) {
  const int st = check_index("csa_index_score", q_I, q_dtype, w_I, K_I, k_dtype, K_scale, q_pos, B, Tq, H_I, d_I,
                             N_cap, m, I_out);
  if (st != CSA_OK) return st;
  csa::IndexArgs a{q_I, q_dtype, w_I, K_I, k_dtype, K_scale, q_pos, B, Tq, H_I, d_I, N_cap, m, I_out};
  if (csa::launch_index_score(a, (hipStream_t)stream) != 0)
    return fail(CSA_E_HIP, "csa_index_score: kernel launch failed");
  return ok();
}

int csa_decode_front(const csa_compress_job* jobs, int n_jobs, const void* q_I, int q_dtype, const float* w_I,
                     const void* K_I, int k_dtype, const float* K_scale, const int* q_pos, int B, int H_I,
                     int d_I, long long N_cap, int m, float* I_out, void* stream) {
  if (!jobs) return fail(CSA_E_NULL, "csa_decode_front: jobs is NULL");
  if (n_jobs < 1 || n_jobs > CSA_DECODE_FRONT_MAX_JOBS)
    return fail(CSA_E_SHAPE, "csa_decode_front: n_jobs = %d outside [1, %d]", n_jobs, CSA_DECODE_FRONT_MAX_JOBS);
  csa::CompressArgs a[CSA_DECODE_FRONT_MAX_JOBS];
  for (int q = 0; q < n_jobs; ++q) {
    char who[48];
    snprintf(who, sizeof(who), "csa_decode_front: job %d", q);
    const int st = check_compress(jobs[q], who);
    if (st != CSA_OK) return st;
    if (jobs[q].s_end <= jobs[q].s_begin) return fail(CSA_E_SHAPE, "%s: no entries", who);
    a[q] = compress_args(jobs[q]);
  }
  const int st = check_index("csa_decode_front", q_I, q_dtype, w_I, K_I, k_dtype, K_scale, q_pos, B, 1, H_I, d_I,
                             N_cap, m, I_out);
  if (st != CSA_OK) return st;
  csa::IndexArgs ia{q_I, q_dtype, w_I, K_I, k_dtype, K_scale, q_pos, B, 1, H_I, d_I, N_cap, m, I_out};
  const char* why = nullptr;
  if (csa::launch_decode_front(a, n_jobs, ia, (hipStream_t)stream, &why) != 0)
    return fail(CSA_E_UNSUPPORTED, "csa_decode_front: %s", why ? why : "not covered");
  if (hipGetLastError() != hipSuccess) return fail(CSA_E_HIP, "csa_decode_front: kernel launch failed");
  return ok();
}

size_t csa_topk_workspace_size(int B, int Tq, long long N_cap, int k) {
  if (B < 1 || Tq < 1 || N_cap < 1 || k < 1) return 0;
  return csa::topk_workspace_bytes(B, Tq, N_cap, k);
}

int csa_topk(const float* I, const int* q_pos, int B, int Tq, long long N_cap, int m, int k,
             int* idx_out, float* val_out, void* workspace, size_t ws_bytes, void* stream) {
  if (!I || !q_pos || !idx_out) return fail(CSA_E_NULL, "csa_topk: I, q_pos and idx_out are required");
  if (B < 1 || Tq < 1 || N_cap < 1 || m < 1) return fail(CSA_E_SHAPE, "csa_topk: sizes must be >= 1");
  if (k < 1 || k > 2048) return fail(CSA_E_SHAPE, "csa_topk: k = %d outside [1, 2048]", k);
  if (N_cap > 2147483647LL) return fail(CSA_E_UNSUPPORTED, "csa_topk: N_cap must fit int32");
  if ((long long)B * Tq > 2147483647LL) return fail(CSA_E_UNSUPPORTED, "csa_topk: too many rows");
  const size_t need = csa::topk_workspace_bytes(B, Tq, N_cap, k);
  if (need > 0 && (!workspace || ws_bytes < need))
    return fail(CSA_E_WORKSPACE, "csa_topk: workspace of %zu bytes needed, %zu given", need, ws_bytes);
  csa::TopkArgs a{I, q_pos, B, Tq, N_cap, m, k, idx_out, val_out, workspace, ws_bytes};
  if (csa::launch_topk(a, (hipStream_t)stream) != 0)
    return fail(CSA_E_HIP, "csa_topk: kernel launch failed");
  return ok();
}

size_t csa_mqa_workspace_size(int B, int Tq, int n_h, int d, long long n_keys_max) {
  if (B < 1 || Tq < 1 || n_h < 1 || d < 1 || n_keys_max < 0) return 0;
  return csa::mqa_workspace_bytes(B, Tq, n_h, d, n_keys_max, CSA_BF16);
}

static int mqa_common(const char* fn, const void* q, const void* E, const float* E_scale, long long N_cap,
                      const void* W, const float* W_scale, int W_cap, int n_win, const int* q_pos, int B,
                      int Tq, int n_h, int d, int rope_dim, int dtype, void* out) {
  if (!q || !E || !q_pos || !out) return fail(CSA_E_NULL, "%s: q, E, q_pos and out are required", fn);
  if (dtype != CSA_F32 && dtype != CSA_BF16 && dtype != CSA_KV_MIXED)
    return fail(CSA_E_DTYPE, "%s: dtype must be F32, BF16 or KV_MIXED", fn);
  if (dtype == CSA_KV_MIXED && (!E_scale || (n_win > 0 && !W_scale)))
    return fail(CSA_E_NULL, "%s: KV_MIXED rows need E_scale (and W_scale with a window)", fn);
  if (B < 1 || Tq < 1 || n_h < 1 || d < 2 || N_cap < 1)
    return fail(CSA_E_SHAPE, "%s: sizes must be >= 1 (d >= 2)", fn);
  if (d & 1) return fail(CSA_E_SHAPE, "%s: d must be even", fn);
  if (d > 4096) return fail(CSA_E_UNSUPPORTED, "%s: d <= 4096", fn);
  if (rope_dim < 0 || rope_dim > d || (rope_dim & 1))
    return fail(CSA_E_SHAPE, "%s: rope_dim must be even and <= d", fn);
  if (n_win < 0) return fail(CSA_E_SHAPE, "%s: n_win < 0", fn);
  if (n_win > 0 && (!W || W_cap < n_win))
    return fail(W ? CSA_E_SHAPE : CSA_E_NULL, "%s: a window needs W with W_cap >= n_win", fn);
  if (Tq > 65535 || B > 65535 || n_h > 65535) return fail(CSA_E_UNSUPPORTED, "%s: B, Tq, n_h <= 65535", fn);
  return CSA_OK;
}

int csa_sparse_mqa(const void* q, const float* gamma_q, float eps, const void* E, const float* E_scale,
                   long long N_cap, const int* idx, int k, const void* W, const float* W_scale, int W_cap,
                   int n_win, const float* sink, const int* q_pos, int B, int Tq, int n_h, int d,
                   int rope_dim, float rope_base, float scale, int dtype, void* out, void* workspace,
                   size_t ws_bytes, void* stream) {
  int st = mqa_common("csa_sparse_mqa", q, E, E_scale, N_cap, W, W_scale, W_cap, n_win, q_pos, B, Tq, n_h,
                      d, rope_dim, dtype, out);
  if (st != CSA_OK) return st;
  if (!idx) return fail(CSA_E_NULL, "csa_sparse_mqa: idx is required");
  if (k < 1 || k > 65536) return fail(CSA_E_SHAPE, "csa_sparse_mqa: k outside [1, 65536]");
  csa::MqaArgs a{q, gamma_q, eps, E, E_scale, N_cap, idx, k, 1, W, W_scale, W_cap, n_win, sink, q_pos, B, Tq, n_h, d,
                 rope_dim, rope_base, scale, dtype, out, workspace, ws_bytes};
  const char* why = "";
  st = csa::launch_mqa(a, (hipStream_t)stream, &why);
  if (st != 0) return fail(st, "csa_sparse_mqa: %s", why);
  return ok();
}

int hca_dense_mqa(const void* q, const float* gamma_q, float eps, const void* E, const float* E_scale,
                  long long N_cap, int m, const void* W, const float* W_scale, int W_cap, int n_win,
                  const float* sink, const int* q_pos, int B, int Tq, int n_h, int d, int rope_dim,
                  float rope_base, float scale, int dtype, void* out, void* workspace, size_t ws_bytes,
                  void* stream) {
  int st = mqa_common("hca_dense_mqa", q, E, E_scale, N_cap, W, W_scale, W_cap, n_win, q_pos, B, Tq, n_h,
                      d, rope_dim, dtype, out);
  if (st != CSA_OK) return st;
  if (m < 1) return fail(CSA_E_SHAPE, "hca_dense_mqa: m must be >= 1");
  if (N_cap > 2147483647LL) return fail(CSA_E_UNSUPPORTED, "hca_dense_mqa: N_cap must fit int32");
  csa::MqaArgs a{q, gamma_q, eps, E, E_scale, N_cap, nullptr, 0, m, W, W_scale, W_cap, n_win, sink, q_pos, B, Tq, n_h,
                 d, rope_dim, rope_base, scale, dtype, out, workspace, ws_bytes};
  const char* why = "";
  st = csa::launch_mqa(a, (hipStream_t)stream, &why);
  if (st != 0) return fail(st, "hca_dense_mqa: %s", why);
  return ok();
}

int csa_cache_append(int B, const int* T0, int n_new, int c, int d_I, int m, int m_hca,
                     const void* C_a, const void* Z_a, const void* C_b, const void* Z_b,
                     const void* IC_a, const void* IZ_a, const void* IC_b, const void* IZ_b,
                     const void* C_h, const void* Z_h, const void* W_raw, void* tail,
                     void* E_csa, void* K_idx, void* K_scale, int k_dtype, long long N_csa,
                     void* E_hca, long long N_hca, void* W, int W_cap, const float* gamma, float eps,
                     int rope_dim, float rope_base, void* stream) {
  const char* fn = "csa_cache_append";
  const void* req[] = {T0, C_a, Z_a, C_b, Z_b, IC_a, IZ_a, IC_b, IZ_b, C_h, Z_h, W_raw, tail, E_csa, K_idx,
                       E_hca, W};
  for (const void* p : req)
    if (!p) return fail(CSA_E_NULL, "%s: every array argument except gamma and K_scale is required", fn);
  if (B < 1 || n_new < 1 || c < 8 || d_I < 8 || m < 1 || m_hca < 1 || N_csa < 1 || N_hca < 1 || W_cap < 1)
    return fail(CSA_E_SHAPE, "%s: sizes must be >= 1 (c, d_I >= 8)", fn);
  if (B > 65535) return fail(CSA_E_UNSUPPORTED, "%s: B <= 65535", fn);
  if (c % 8 || d_I % 8 || c > 1024 || d_I > 1024)
    return fail(CSA_E_UNSUPPORTED, "%s: c and d_I must be multiples of 8, at most 1024", fn);
  long long a = m, bb = m_hca;
  while (bb) { const long long t = a % bb; a = bb; bb = t; }
  const long long ring = (long long)m / a * m_hca;   // lcm(m, m')
  if (ring < 2LL * m || ring > 4096)
    return fail(CSA_E_UNSUPPORTED, "%s: lcm(m, m') must lie in [2 m, 4096]", fn);
  if (k_dtype != CSA_BF16 && k_dtype != CSA_FP8_E4M3 && k_dtype != CSA_MXFP4)
    return fail(CSA_E_DTYPE, "%s: k_dtype must be BF16, FP8_E4M3 or MXFP4", fn);
  if (k_dtype != CSA_BF16 && !K_scale) return fail(CSA_E_NULL, "%s: K_scale is required for FP8 and MXFP4 keys", fn);
  if (k_dtype == CSA_MXFP4 && d_I % 32) return fail(CSA_E_SHAPE, "%s: MXFP4 keys need d_I %% 32 == 0", fn);
  if (rope_dim < 0 || rope_dim > c || (rope_dim & 1) || ((c - rope_dim) & 1))
    return fail(CSA_E_SHAPE, "%s: rope_dim must be even and <= c", fn);
  if (gamma && !(eps >= 0.f)) return fail(CSA_E_SHAPE, "%s: eps must be >= 0", fn);
  const void* al[] = {C_a, Z_a, C_b, Z_b, IC_a, IZ_a, IC_b, IZ_b, C_h, Z_h, W_raw, tail};
  for (const void* p : al)
    if (((uintptr_t)p) & 15u) return fail(CSA_E_UNSUPPORTED, "%s: input arrays and tail must be 16-byte aligned", fn);
  csa::CacheAppendArgs x{B, T0, n_new, c, d_I, m, m_hca, (int)ring, C_a, Z_a, C_b, Z_b, IC_a, IZ_a, IC_b,
                         IZ_b, C_h, Z_h, W_raw, tail, E_csa, K_idx, K_scale, k_dtype, N_csa, E_hca, N_hca, W,
                         W_cap, gamma, eps, rope_dim, rope_base};
  if (csa::launch_cache_append(x, (hipStream_t)stream) != 0) return fail(CSA_E_HIP, "%s: kernel launch failed", fn);
  return ok();
}

static int proj_check(const char* fn, int T, int n_h, int c, int groups, int d_g, int d) {
  if (T < 1 || n_h < 1 || c < 1 || groups < 1 || d_g < 1 || d < 1)
    return fail(CSA_E_SHAPE, "%s: sizes must be >= 1", fn);
  const long long HC = (long long)n_h * c;
  if (HC % groups) return fail(CSA_E_SHAPE, "%s: n_h * c must be a multiple of groups", fn);
  if ((HC / groups) % 64 || ((long long)groups * d_g) % 64)
    return fail(CSA_E_UNSUPPORTED, "%s: n_h c / groups and groups d_g must be multiples of 64", fn);
  if (HC > 2147483647LL || (long long)groups * d_g > 2147483647LL || T > 65535 * 16)
    return fail(CSA_E_UNSUPPORTED, "%s: sizes beyond the supported range", fn);
  return CSA_OK;
}

size_t csa_out_proj_workspace_size(int T, int n_h, int c, int groups, int d_g, int d) {
  if (proj_check("csa_out_proj_workspace_size", T, n_h, c, groups, d_g, d) != CSA_OK) return 0;
  csa::ProjArgs a{nullptr, nullptr, nullptr, nullptr, nullptr, T, n_h, c, groups, d_g, d, nullptr, 0};
  return csa::proj_workspace_bytes(a);
}

int csa_grouped_out_proj(const void* o, const void* W1, const void* W2, void* y, void* out, int T, int n_h,
                         int c, int groups, int d_g, int d, void* workspace, size_t ws_bytes, void* stream) {
  const char* fn = "csa_grouped_out_proj";
  if (!o || !W1 || !W2 || !y || !out) return fail(CSA_E_NULL, "%s: o, W1, W2, y and out are required", fn);
  int st = proj_check(fn, T, n_h, c, groups, d_g, d);
  if (st != CSA_OK) return st;
  const void* ptrs[] = {o, W1, W2, y};
  for (const void* p : ptrs)
    if (((uintptr_t)p) & 15u) return fail(CSA_E_UNSUPPORTED, "%s: o, W1, W2 and y must be 16-byte aligned", fn);
  if (((uintptr_t)out) & 1u) return fail(CSA_E_SHAPE, "%s: out must be 2-byte aligned", fn);
  csa::ProjArgs a{o, W1, W2, y, out, T, n_h, c, groups, d_g, d, workspace, ws_bytes};
  const size_t need = csa::proj_workspace_bytes(a);
  if (need > 0 && (!workspace || ws_bytes < need || (((uintptr_t)workspace) & 15u)))
    return fail(CSA_E_WORKSPACE, "%s: a 16-byte aligned workspace of %zu bytes is needed, %zu given", fn, need,
                ws_bytes);
  if (csa::launch_proj(a, (hipStream_t)stream) != 0) return fail(CSA_E_HIP, "%s: kernel launch failed", fn);
  return ok();
}

}  // extern "C"

// ---------------------------------------------------------------------------
// the no-allocation variant of csa_sparse_mqa
// ---------------------------------------------------------------------------
namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// the device address of `scratch` on the current device, looked up once per
// device with that device current
int scratch_ptr(const char* fn, void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(CSA_E_HIP, "%s: no current HIP device", fn);
  if (dev >= kMaxDevices) return fail(CSA_E_UNSUPPORTED, "%s: device %d >= %d", fn, dev, kMaxDevices);
  std::call_once(g_scratch_once[dev], [dev]() {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev])
    return fail(CSA_E_HIP, "%s: hipGetSymbolAddress(scratch) failed on device %d: %s", fn, dev,
                hipGetErrorString(g_scratch_err[dev]));
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}
}  // namespace

extern "C" int csa_sparse_mqa_noalloc(const void* q, const float* gamma_q, float eps, const void* E,
                                      const float* E_scale, long long N_cap, const int* idx, int k,
                                      const void* W, const float* W_scale, int W_cap, int n_win,
                                      const float* sink, const int* q_pos, int B, int Tq, int n_h, int d,
                                      int rope_dim, float rope_base, float scale, int dtype, void* out,
                                      void* stream) {
  const char* fn = "csa_sparse_mqa_noalloc";
  int st = mqa_common(fn, q, E, E_scale, N_cap, W, W_scale, W_cap, n_win, q_pos, B, Tq, n_h, d, rope_dim,
                      dtype, out);
  if (st != CSA_OK) return st;
  if (!idx) return fail(CSA_E_NULL, "%s: idx is required", fn);
  if (k < 1 || k > 65536) return fail(CSA_E_SHAPE, "%s: k outside [1, 65536]", fn);
  const size_t need = csa_mqa_workspace_size(B, Tq, n_h, d, (long long)k + n_win);
  if (need > (size_t)CSA_NOALLOC_SCRATCH_BYTES)
    return fail(CSA_E_UNSUPPORTED,
                "%s: this call needs %zu bytes of split partials, more than the %u-byte static "
                "scratch; use csa_sparse_mqa with a workspace", fn, need, (unsigned)CSA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  if (need > 0 && (st = scratch_ptr(fn, &ws)) != CSA_OK) return st;
  csa::MqaArgs a{q, gamma_q, eps, E, E_scale, N_cap, idx, k, 1, W, W_scale, W_cap, n_win, sink, q_pos, B, Tq, n_h, d,
                 rope_dim, rope_base, scale, dtype, out, ws, need > 0 ? (size_t)CSA_NOALLOC_SCRATCH_BYTES : 0};
  const char* why = "";
  st = csa::launch_mqa(a, (hipStream_t)stream, &why);
  if (st != 0) return fail(st, "%s: %s", fn, why);
  return ok();
}
