/*
 * csa.h — C ABI of the CSA/HCA hybrid-attention core for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the DeepSeek-V4 method summary ("DeepSeek-V4: Towards
 * Highly Efficient Million-Token Context Intelligence", section 3.3 "CSA and
 * HCA hybrid attention"; section 3.5 for the state cache) and the technical
 * report digest ("DeepSeek V4 complete technical report", section "hybrid
 * attention: CSA + HCA": m = 4 / 128, top-k 512 / 1024, window 128, partial
 * RoPE on the last 64 dims, learnable sink logits).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every array argument is a DEVICE pointer owned by the caller, row-major,
 *    last dimension contiguous.  The library never allocates, frees,
 *    synchronises or prints.  Work is enqueued on `stream` (a hipStream_t
 *    passed as void*; NULL is the default stream) and returns immediately.
 *  - Arguments are validated on the host before anything is enqueued.  On a
 *    non-zero status nothing was launched and nothing was written;
 *    csa_last_error() then holds a thread-local description.  CSA_E_HIP means
 *    a launch itself failed.
 *  - Results are bitwise deterministic and do not depend on the batch size B:
 *    no atomics decide an arithmetic order, and any split of a reduction
 *    depends only on per-row sizes.
 *  - Floating-point arithmetic is fp32 (bf16 / fp8 operands are widened
 *    exactly); outputs are rounded to nearest even.
 *  - Data that the host cannot see (positions, indices, scales) is trusted
 *    as documented; out-of-range indices are skipped, never dereferenced.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 2

/* Storage types. CSA_FP8_E4M3 is OCP FP8 E4M3FN (max 448, no infinities). */
enum csa_dtype { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8_E4M3 = 2 };

enum csa_status {
  CSA_OK = 0,
  CSA_E_NULL = 1,        /* a required pointer is NULL                        */
  CSA_E_SHAPE = 2,       /* a size or index range is invalid                  */
  CSA_E_DTYPE = 3,       /* an unknown dtype or an unsupported dtype pairing  */
  CSA_E_UNSUPPORTED = 4, /* valid, but outside the shapes the kernels cover   */
  CSA_E_WORKSPACE = 5,   /* workspace missing or smaller than required        */
  CSA_E_HIP = 6          /* a HIP launch failed                               */
};

int csa_abi_version(void);
const char* csa_status_str(int status);
/* Description of the last non-OK status returned on the calling thread. */
const char* csa_last_error(void);

/*
 * a1 — KV compressor (method page §3.3: CSA computes two candidate sets and
 * two sets of compression logits; a softmax over 2m elements weights the sum;
 * the two index ranges overlap so the rate is exactly 1/m.  HCA uses a larger
 * m' without overlap.  RMSNorm on the entries, partial RoPE on their last
 * dims).
 *
 * For entry s in [s_begin, s_end) and channel j:
 *   candidates: set a = tokens [m s, m(s+1)) and, if overlap, set b = tokens
 *   [m(s-1), m s), both clipped to [0, T);
 *   alpha = softmax over the candidates of Z^x[tau, j];  E~ = sum alpha C^x[tau, j];
 *   if gamma: E^ = E~ * gamma[j] / sqrt(mean_j E~^2 + eps);
 *   if rope_dim: the last rope_dim channels, as pairs (2u, 2u+1), turn by the
 *   angle p_s * rope_base^(-2u/rope_dim), p_s = pos_stride * s + pos_offset.
 *
 *  C_a, Z_a, C_b, Z_b : [B][R][c] candidates / logits, dtype in_dtype (F32 or
 *      BF16), batch stride in_batch_stride elements.  Row r is token
 *      tok_base + r.  Z_a or Z_b may be NULL (all logits 0 = plain mean).
 *      C_b is required iff overlap.  Every candidate token < T of every
 *      requested entry must lie in [tok_base, tok_base + R).
 *  T        : tokens present (same for all B sequences); s_end <= ceil(T/m).
 *  E        : output [B][rows][c] of out_dtype (F32, BF16 or FP8_E4M3), batch
 *      stride out_batch_stride elements; entry s goes to row s, or to row
 *      s mod out_ring when out_ring > 0 (a sliding-window ring; then at most
 *      out_ring entries per call, so that no two write the same row).
 *  E_scale  : FP8_E4M3 only: fp32 per-row scale at
 *      E_scale[b * (out_batch_stride / c) + row] (row absmax / 448, or 1 for
 *      a zero row); codes are RNE(value / scale), saturated to +-448.
 */
int csa_compress(const void* C_a, const void* Z_a, const void* C_b, const void* Z_b, int in_dtype,
                 int B, long long R, long long in_batch_stride, long long tok_base, long long T,
                 int c, int m, int overlap, long long s_begin, long long s_end,
                 const float* gamma, float eps, int rope_dim, float rope_base,
                 long long pos_stride, long long pos_offset,
                 void* E, int out_dtype, float* E_scale, long long out_batch_stride,
                 long long out_ring, void* stream);

/*
 * a1, batched: n_jobs compressions in one kernel launch.  jobs[q] holds the
 * arguments of one csa_compress call, with the same meaning, layout and
 * checks; the results equal those of the n_jobs separate calls bit for bit.
 * One launch lets the jobs' memory and barrier latencies overlap: a decode
 * step compresses a window row, a KV entry and an indexer key, each a few
 * microseconds of latency for a few kilobytes of data.
 *
 *  jobs   : host array of n_jobs job descriptors, read during the call only.
 *  n_jobs : 1 .. CSA_COMPRESS_MAX_JOBS.
 *  Jobs must not write overlapping output rows (they run concurrently); a job
 *  with s_end == s_begin is a no-op.  Every job is checked before anything is
 *  launched; the first failing job's status is returned and csa_last_error()
 *  names its index.
 */
#define CSA_COMPRESS_MAX_JOBS 8
typedef struct csa_compress_job {
  const void *C_a, *Z_a, *C_b, *Z_b;
  int in_dtype;
  int B;
  long long R, in_batch_stride, tok_base, T;
  int c, m, overlap;
  long long s_begin, s_end;
  const float* gamma;
  float eps;
  int rope_dim;
  float rope_base;
  long long pos_stride, pos_offset;
  void* E;
  int out_dtype;
  float* E_scale;
  long long out_batch_stride, out_ring;
} csa_compress_job;
int csa_compress_batch(const csa_compress_job* jobs, int n_jobs, void* stream);

/*
 * a2 — lightning-indexer score (method page §3.3):
 *   I[b,t,s] = sum_h w_I[b,t,h] * ReLU(q_I[b,t,h,:] . K[b,s,:])  for s < n_vis,
 *   I[b,t,s] = -inf                                              for s >= n_vis,
 *   n_vis = min(N_cap, floor((q_pos[b,t] + 1) / m))  (a query cannot see its
 *   own block).
 *  q_I     : [B][Tq][H_I][d_I], q_dtype F32 or BF16.
 *  w_I     : [B][Tq][H_I] fp32 (any sign).
 *  K_I     : [B][N_cap][d_I]; k_dtype F32 (with q F32), BF16 (with q BF16) or
 *            FP8_E4M3 (with q BF16), then K = code * K_scale[b][s] and
 *            K_scale ([B][N_cap] fp32, every entry > 0) is required.
 *  q_pos   : [B][Tq] int32 absolute positions (>= 0).
 *  I_out   : [B][Tq][N_cap] fp32.
 *  Supported: H_I <= 64, d_I <= 256 (any); the matrix-core path covers
 *  H_I % 16 == 0 and d_I in {32, 64, 128} with BF16 queries.
 */
int csa_index_score(const void* q_I, int q_dtype, const float* w_I,
                    const void* K_I, int k_dtype, const float* K_scale, const int* q_pos,
                    int B, int Tq, int H_I, int d_I, long long N_cap, int m,
                    float* I_out, void* stream);

/*
 * a3 — per-query top-k (method page §3.3; k = 512 / 1024 in the report
 * digest).  For each row, the k_eff = min(k, n_vis) visible entries with the
 * largest score, ordered by score descending with ties to the lower index
 * (-0.0 equals +0.0); slots k_eff..k-1 hold -1 (and -inf in val_out).
 *  I       : [B][Tq][N_cap] fp32, finite on visible entries; entries >= n_vis
 *            are ignored whatever they hold.
 *  idx_out : [B][Tq][k] int32.  val_out: optional [B][Tq][k] fp32 (NULL = none).
 *  1 <= k <= 2048.  workspace: at least csa_topk_workspace_size(...) bytes
 *  (may be 0, then NULL is accepted).
 */
size_t csa_topk_workspace_size(int B, int Tq, long long N_cap, int k);
int csa_topk(const float* I, const int* q_pos, int B, int Tq, long long N_cap, int m, int k,
             int* idx_out, float* val_out, void* workspace, size_t ws_bytes, void* stream);

/*
 * a4 — CSA core attention: shared-KV MQA over the selected entries plus the
 * sliding window and the sink (method page §3.3; report digest: window 128,
 * learnable sink logits, partial RoPE with the output rotated at -i).
 *   q^_h = RoPE_i(RMSNorm_{gamma_q}(q_h))   (RMSNorm over d; rope on the last
 *           rope_dim dims at the query position i = q_pos[b,t]);
 *   keys = { E[b, idx[b,t,j]] : 0 <= idx < N_cap }  U  { W[b, tau mod W_cap] :
 *           tau in [max(0, i - n_win + 1), i] }   (every row is key and value);
 *   l_j = scale * q^_h . kv_j;  p_j = e^{l_j} / (e^{sink_h} + sum_j e^{l_j});
 *   o_h = sum_j p_j kv_j, then its last rope_dim dims turn by the angle at -i.
 *  q       : [B][Tq][n_h][d];  gamma_q: [d] fp32 or NULL (= 1).
 *  E       : [B][N_cap][d] entries stored after RMSNorm and RoPE.
 *  idx     : [B][Tq][k] int32 (-1 = empty slot).
 *  W       : [B][W_cap][d] window ring (token tau at row tau mod W_cap), NULL
 *            iff n_win == 0; W_cap >= n_win.
 *  sink    : [n_h] fp32 or NULL (no sink; -inf is also "no sink").
 *  dtype   : F32 or BF16 for q, E, W and out.  out: [B][Tq][n_h][d].
 *  No key and no sink gives a zero output row.
 *  Matrix-core path: BF16 with d in {128, 256, 512}, n_h a multiple of 16 and
 *  q, E, W and out 16-byte aligned; any other call takes the generic path,
 *  which holds at most 8192 key slots per query (CSA_E_UNSUPPORTED beyond).
 *  workspace: at least csa_mqa_workspace_size(B, Tq, n_h, d, k + n_win) bytes,
 *            16-byte aligned (split partials: per (query, split, head) the
 *            output over that split's keys divided by its softmax sum, as d
 *            fp16 values saturated at +-65504, then the fp32 (max, sum)
 *            pairs); contents on entry do not matter.
 */
size_t csa_mqa_workspace_size(int B, int Tq, int n_h, int d, long long n_keys_max);
int csa_sparse_mqa(const void* q, const float* gamma_q, float eps, const void* E, long long N_cap,
                   const int* idx, int k, const void* W, int W_cap, int n_win, const float* sink,
                   const int* q_pos, int B, int Tq, int n_h, int d, int rope_dim, float rope_base,
                   float scale, int dtype, void* out, void* workspace, size_t ws_bytes,
                   void* stream);

/*
 * a5 — HCA core attention (method page §3.3: larger m', no overlap, dense
 * attention, otherwise as CSA): as csa_sparse_mqa, with the selected set
 * replaced by every visible entry s < min(N_cap, floor((i + 1) / m)).
 * workspace: at least csa_mqa_workspace_size(B, Tq, n_h, d, N_cap + n_win).
 */
int hca_dense_mqa(const void* q, const float* gamma_q, float eps, const void* E, long long N_cap,
                  int m, const void* W, int W_cap, int n_win, const float* sink,
                  const int* q_pos, int B, int Tq, int n_h, int d, int rope_dim, float rope_base,
                  float scale, int dtype, void* out, void* workspace, size_t ws_bytes,
                  void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
