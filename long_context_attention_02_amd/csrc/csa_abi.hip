// C ABI of the CSA/HCA core (declared in include/csa.h).  Every entry point
// validates its arguments on the host first; on a non-OK status nothing has
// been enqueued and nothing written.  No device memory is allocated here.
#include <stdarg.h>
#include <stdio.h>

#include "../../include/csa.h"
#include "csa_internal.h"

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

bool dtype_valid(int dt) { return dt == CSA_F32 || dt == CSA_BF16 || dt == CSA_FP8_E4M3; }

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
  if (out_dtype == CSA_FP8_E4M3 && !E_scale)
    return fail(CSA_E_NULL, "%s: E_scale is required for FP8 output", who);
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
                           j.tok_base, j.T, j.c, j.m, j.overlap, j.s_begin, j.s_end, j.gamma, j.eps,
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
                 int c, int m, int overlap, long long s_begin, long long s_end,
                 const float* gamma, float eps, int rope_dim, float rope_base,
                 long long pos_stride, long long pos_offset,
                 void* E, int out_dtype, float* E_scale, long long out_batch_stride,
                 long long out_ring, void* stream) {
  const csa_compress_job j{C_a, Z_a, C_b, Z_b, in_dtype, B, R, in_batch_stride, tok_base, T, c, m,
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

int csa_compress_batch(const csa_compress_job* jobs, int n_jobs, void* stream) {
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
  if (n > 0 && csa::launch_compress(a, n, (hipStream_t)stream) != 0)
    return fail(CSA_E_HIP, "csa_compress_batch: kernel launch failed");
  return ok();
}

int csa_index_score(const void* q_I, int q_dtype, const float* w_I,
                    const void* K_I, int k_dtype, const float* K_scale, const int* q_pos,
                    int B, int Tq, int H_I, int d_I, long long N_cap, int m,
                    float* I_out, void* stream) {
  if (!q_I || !w_I || !K_I || !q_pos || !I_out)
    return fail(CSA_E_NULL, "csa_index_score: q_I, w_I, K_I, q_pos and I_out are required");
  if (q_dtype != CSA_F32 && q_dtype != CSA_BF16)
    return fail(CSA_E_DTYPE, "csa_index_score: q_dtype must be F32 or BF16");
  if (!dtype_valid(k_dtype)) return fail(CSA_E_DTYPE, "csa_index_score: unknown k_dtype");
  if (q_dtype == CSA_F32 && k_dtype != CSA_F32)
    return fail(CSA_E_DTYPE, "csa_index_score: F32 queries need F32 keys");
  if (q_dtype == CSA_BF16 && k_dtype == CSA_F32)
    return fail(CSA_E_DTYPE, "csa_index_score: BF16 queries need BF16 or FP8 keys");
  if (k_dtype == CSA_FP8_E4M3 && !K_scale)
    return fail(CSA_E_NULL, "csa_index_score: K_scale is required for FP8 keys");
  if (B < 1 || Tq < 1 || H_I < 1 || d_I < 1 || N_cap < 1 || m < 1)
    return fail(CSA_E_SHAPE, "csa_index_score: sizes must be >= 1");
  if (H_I > 64 || d_I > 256 || H_I * (d_I + 1) > 16384)
    return fail(CSA_E_UNSUPPORTED, "csa_index_score: H_I <= 64 and d_I <= 256 are supported");
  if (N_cap > 2147483647LL || (long long)B * Tq > 65535LL * 65535LL)
    return fail(CSA_E_UNSUPPORTED, "csa_index_score: N_cap must fit int32");
  if (Tq > 65535 || B > 65535) return fail(CSA_E_UNSUPPORTED, "csa_index_score: B, Tq <= 65535");
  csa::IndexArgs a{q_I, q_dtype, w_I, K_I, k_dtype, K_scale, q_pos, B, Tq, H_I, d_I, N_cap, m, I_out};
  if (csa::launch_index_score(a, (hipStream_t)stream) != 0)
    return fail(CSA_E_HIP, "csa_index_score: kernel launch failed");
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

static int mqa_common(const char* fn, const void* q, const void* E, long long N_cap, const void* W,
                      int W_cap, int n_win, const int* q_pos, int B, int Tq, int n_h, int d,
                      int rope_dim, int dtype, void* out) {
  if (!q || !E || !q_pos || !out) return fail(CSA_E_NULL, "%s: q, E, q_pos and out are required", fn);
  if (dtype != CSA_F32 && dtype != CSA_BF16) return fail(CSA_E_DTYPE, "%s: dtype must be F32 or BF16", fn);
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

int csa_sparse_mqa(const void* q, const float* gamma_q, float eps, const void* E, long long N_cap,
                   const int* idx, int k, const void* W, int W_cap, int n_win, const float* sink,
                   const int* q_pos, int B, int Tq, int n_h, int d, int rope_dim, float rope_base,
                   float scale, int dtype, void* out, void* workspace, size_t ws_bytes,
                   void* stream) {
  int st = mqa_common("csa_sparse_mqa", q, E, N_cap, W, W_cap, n_win, q_pos, B, Tq, n_h, d,
                      rope_dim, dtype, out);
  if (st != CSA_OK) return st;
  if (!idx) return fail(CSA_E_NULL, "csa_sparse_mqa: idx is required");
  if (k < 1 || k > 65536) return fail(CSA_E_SHAPE, "csa_sparse_mqa: k outside [1, 65536]");
  csa::MqaArgs a{q, gamma_q, eps, E, N_cap, idx, k, 1, W, W_cap, n_win, sink, q_pos, B, Tq, n_h, d,
                 rope_dim, rope_base, scale, dtype, out, workspace, ws_bytes};
  const char* why = "";
  st = csa::launch_mqa(a, (hipStream_t)stream, &why);
  if (st != 0) return fail(st, "csa_sparse_mqa: %s", why);
  return ok();
}

int hca_dense_mqa(const void* q, const float* gamma_q, float eps, const void* E, long long N_cap,
                  int m, const void* W, int W_cap, int n_win, const float* sink,
                  const int* q_pos, int B, int Tq, int n_h, int d, int rope_dim, float rope_base,
                  float scale, int dtype, void* out, void* workspace, size_t ws_bytes,
                  void* stream) {
  int st = mqa_common("hca_dense_mqa", q, E, N_cap, W, W_cap, n_win, q_pos, B, Tq, n_h, d,
                      rope_dim, dtype, out);
  if (st != CSA_OK) return st;
  if (m < 1) return fail(CSA_E_SHAPE, "hca_dense_mqa: m must be >= 1");
  if (N_cap > 2147483647LL) return fail(CSA_E_UNSUPPORTED, "hca_dense_mqa: N_cap must fit int32");
  csa::MqaArgs a{q, gamma_q, eps, E, N_cap, nullptr, 0, m, W, W_cap, n_win, sink, q_pos, B, Tq, n_h,
                 d, rope_dim, rope_base, scale, dtype, out, workspace, ws_bytes};
  const char* why = "";
  st = csa::launch_mqa(a, (hipStream_t)stream, &why);
  if (st != 0) return fail(st, "hca_dense_mqa: %s", why);
  return ok();
}

}  // extern "C"
