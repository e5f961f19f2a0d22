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

#define CSA_ABI_VERSION 6

/* Storage types. CSA_FP8_E4M3 is OCP FP8 E4M3FN (max 448, no infinities).
 * CSA_MXFP4 is OCP MXFP4: FP4 E2M1 codes (values 0, 0.5, 1, 1.5, 2, 3, 4, 6
 * and their negatives) packed two per byte, the even channel in the low
 * nibble, with one E8M0 scale byte (2^(byte - 127)) per 32 channels in a
 * separate array; quantised by the OCP MX rule (shared exponent
 * floor(log2(block max)) - 2, elements rounded to nearest even, saturating). */
enum csa_dtype { CSA_F32 = 0, CSA_BF16 = 1, CSA_FP8_E4M3 = 2, CSA_MXFP4 = 3, CSA_KV_MIXED = 4 };
/* CSA_KV_MIXED: KV rows (compressed entries and window rows) with the RoPE dims
 * in BF16 and the rest in FP8 (method page §3.3, storage of the KV entries):
 * of a row of c channels, the first c - rope_dim are e4m3fn codes under one
 * fp32 scale per row (absmax / 448 of those channels, in a separate array),
 * followed by the last rope_dim channels as bf16: c + rope_dim bytes per row
 * (576 instead of 1024 at c = 512, rope_dim = 64). */

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
 *  T        : tokens present, the same for every sequence, or an upper bound
 *      of the per-sequence counts when T_len is given; s_end <= ceil(T/m).
 *  T_len    : NULL, or a device array [B] int32 of per-sequence token counts
 *      (a batch of sequences with ragged tails; the method page's section 3.5
 *      keeps the tokens of a block that is not yet full in a state cache).
 *      Sequence b then has min(T, max(0, T_len[b])) tokens: candidates at or
 *      past it are absent, and an entry s with m s >= that count does not
 *      exist in sequence b and its output row is not written.
 *  E        : output [B][rows][c] of out_dtype (F32, BF16, FP8_E4M3 or MXFP4),
 *      batch stride out_batch_stride elements (channels); entry s goes to row
 *      s, or to row s mod out_ring when out_ring > 0 (a sliding-window ring;
 *      then at most out_ring entries per call, so that no two write the same
 *      row).  MXFP4 rows are c / 2 bytes (c % 32 == 0); KV_MIXED rows c +
 *      rope_dim bytes (rope_dim and c - rope_dim multiples of 8).
 *  E_scale  : FP8_E4M3: fp32 per-row scale at E_scale[b * (out_batch_stride /
 *      c) + row] (row absmax / 448, or 1 for a zero row); codes are
 *      RNE(value / scale), saturated to +-448.  MXFP4: the E8M0 block scales,
 *      bytes [B][rows][c / 32] (pass the byte array's address); the
 *      quantisation decisions are taken on the fp32 value.  KV_MIXED: the
 *      fp32 row scale of the e4m3 part, like FP8.  NULL otherwise.
 */
int csa_compress(const void* C_a, const void* Z_a, const void* C_b, const void* Z_b, int in_dtype,
                 int B, long long R, long long in_batch_stride, long long tok_base, long long T,
                 const int* T_len, int c, int m, int overlap, long long s_begin, long long s_end,
                 const float* gamma, float eps, int rope_dim, float rope_base,
                 long long pos_stride, long long pos_offset,
                 void* E, int out_dtype, float* E_scale, long long out_batch_stride,
                 long long out_ring, void* stream);

/*
 * a1, batched: n_jobs compressions in one kernel launch.  jobs[q] holds the
 * arguments of one csa_compress call, with the same meaning, layout and
 * checks.  One launch lets the jobs' memory and barrier latencies overlap: a
 * decode step compresses a window row, a KV entry and an indexer key, each a
 * few microseconds of latency for a few kilobytes of data.
 *
 *  jobs   : host array of n_jobs job descriptors, read during the call only.
 *  n_jobs : 1 .. CSA_COMPRESS_MAX_JOBS.
 *  workspace / workspace_bytes : NULL / 0, or device memory of at least
 *      csa_compress_workspace_size(jobs, n_jobs) bytes (any contents; owned by
 *      the caller).  Without it the results equal those of the n_jobs
 *      separate csa_compress calls bit for bit.  With it, jobs whose entries
 *      pool 64 or more candidates (HCA blocks) over at most 256 (sequence,
 *      entry) pairs spread each entry's channels over several workgroups (64
 *      channels each; a second kernel normalises and stores the rows): the
 *      same pooling summed in another order, so within rounding of the
 *      separate calls, and deterministic.  A workspace smaller than required
 *      is CSA_E_WORKSPACE.  Calls that share a workspace must not run
 *      concurrently.
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
  const int* T_len;
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
int csa_compress_batch(const csa_compress_job* jobs, int n_jobs, void* workspace, size_t workspace_bytes,
                       void* stream);
/* Workspace bytes csa_compress_batch takes for these jobs (0: none needed; a
 * job that fails the checks counts for nothing). */
size_t csa_compress_workspace_size(const csa_compress_job* jobs, int n_jobs);

/*
 * a2 — lightning-indexer score (method page §3.3):
 *   I[b,t,s] = sum_h w_I[b,t,h] * ReLU(q_I[b,t,h,:] . K[b,s,:])  for s < n_vis,
 *   I[b,t,s] = -inf                                              for s >= n_vis,
 *   n_vis = min(N_cap, floor((q_pos[b,t] + 1) / m))  (a query cannot see its
 *   own block).
 *  q_I     : [B][Tq][H_I][d_I], q_dtype F32 or BF16.
 *  w_I     : [B][Tq][H_I] fp32 (any sign).
 *  K_I     : [B][N_cap][d_I]; k_dtype F32 (with q F32), BF16 (with q BF16),
 *            FP8_E4M3 (with q BF16), then K = code * K_scale[b][s] and
 *            K_scale ([B][N_cap] fp32, every entry > 0) is required, or
 *            MXFP4 (with q BF16; d_I % 32 == 0): the FP4 query-key path of the
 *            method page's section 3.6 -- K_I holds [B][N_cap][d_I / 2] packed
 *            codes, K_scale the E8M0 bytes [B][N_cap][d_I / 32] (pass the byte
 *            array's address), and the query is quantised to MXFP4 by the same
 *            rule (per head, 32-dim blocks) before the products.
 *  q_pos   : [B][Tq] int32 absolute positions (>= 0).
 *  I_out   : [B][Tq][N_cap] fp32.
 *  Supported: H_I <= 64, d_I <= 256 (any); the matrix-core path covers
 *  H_I in {16, 32, 64} and d_I in {32, 64, 128} with BF16 queries (other
 *  head counts, e.g. 48, take the generic kernel); for MXFP4 keys it covers
 *  d_I = 128 with fewer than 8 queries per sequence (decode).
 */
int csa_index_score(const void* q_I, int q_dtype, const float* w_I,
                    const void* K_I, int k_dtype, const float* K_scale, const int* q_pos,
                    int B, int Tq, int H_I, int d_I, long long N_cap, int m,
                    float* I_out, void* stream);

/*
 * a1 + a2 of a decode step in one launch (method page §3.3: the step's new
 * compressed rows, then the indexer's scores over every visible entry).  The
 * compressions of jobs[] (csa_compress_batch's descriptors: typically the new
 * token's window row, the newest KV entry and the newest indexer key) run
 * beside the scoring of csa_index_score with Tq = 1, instead of in a launch of
 * their own in front of it.  Exactly one job writes the indexer's key rows
 * (its E is K_I, with K_I's layout: out_batch_stride = N_cap * d_I, no ring,
 * E_scale = K_scale for FP8 keys), and its entries lie in the last 64 rows of
 * K_I; the indexer scores the other rows while the job runs, and the wave that
 * wrote the key then scores those last 64 rows.  Other jobs must not write
 * memory the indexer reads: one whose E or E_scale starts inside K_I or
 * K_scale is refused (CSA_E_UNSUPPORTED).
 *  Arguments: as csa_compress_batch (jobs, n_jobs <= CSA_DECODE_FRONT_MAX_JOBS,
 *  no workspace) and csa_index_score (Tq = 1: q_I [B][1][H_I][d_I], w_I,
 *  q_pos [B][1], I_out [B][1][N_cap]).
 *  Results: I_out equals csa_index_score's on the same key rows bit for bit.
 *  The compressed rows come from the wave-per-entry compressor (one wave per
 *  entry: all candidates of a lane in flight, wave reductions), whose results
 *  agree with csa_compress_batch's to rounding (the RMSNorm sum and the
 *  pooling are added in another order); they are deterministic.
 *  Covered: BF16 queries; BF16 or FP8 keys with H_I in {16, 32, 64} and d_I
 *  in {32, 64, 128}, or MXFP4 keys with H_I in {16, 32, 64} and d_I = 128
 *  (K_scale the E8M0 bytes, 4-byte aligned); N_cap a multiple of 64, at least
 *  128; 16-byte aligned q_I and K_I; jobs with BF16 inputs in 16-byte pieces,
 *  at most 8 candidates per entry (m <= 4 with overlap, m <= 8 without),
 *  c % 8 == 0, BF16 output or the key format (FP8 beside FP8 keys, MXFP4 beside
 *  MXFP4 keys).  Anything else returns CSA_E_UNSUPPORTED with nothing launched,
 *  and the caller makes the two separate calls.
 */
#define CSA_DECODE_FRONT_MAX_JOBS 4
int csa_decode_front(const csa_compress_job* jobs, int n_jobs, const void* q_I, int q_dtype, const float* w_I,
                     const void* K_I, int k_dtype, const float* K_scale, const int* q_pos, int B, int H_I,
                     int d_I, long long N_cap, int m, float* I_out, void* stream);

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
 *  dtype   : F32 or BF16 for q, E, W and out; or KV_MIXED: q and out BF16,
 *            E and W mixed rows ([B][N_cap][d + rope_dim] and
 *            [B][W_cap][d + rope_dim] bytes) whose fp8 part is decoded as
 *            code * row scale, with the row scales in E_scale ([B][N_cap]
 *            fp32) and W_scale ([B][W_cap] fp32, NULL iff n_win == 0).
 *            E_scale and W_scale are ignored (may be NULL) for F32 and BF16.
 *            out: [B][Tq][n_h][d].
 *  No key and no sink gives a zero output row.
 *  Matrix-core path: BF16 with d in {128, 256, 512}, n_h a multiple of 16 and
 *  q, E, W and out 16-byte aligned; any other call takes the generic path,
 *  which holds at most 8192 key slots per query (CSA_E_UNSUPPORTED beyond).
 *  KV_MIXED runs on the matrix-core path only, at d = 512 with rope_dim = 64
 *  (the entry width and rotated share of the method page's models;
 *  CSA_E_UNSUPPORTED otherwise).  The stored values enter exactly: the row
 *  scale multiplies the code part of each score and each softmax weight, never
 *  a rounded copy of the row.
 *  workspace: at least csa_mqa_workspace_size(B, Tq, n_h, d, k + n_win) bytes,
 *            16-byte aligned (split partials: per (query, split, head) the
 *            output over that split's keys divided by its softmax sum and
 *            scaled by a power of two that puts the row's largest magnitude
 *            in [2^14, 2^15), as d fp16 values, then fp32 records (max, sum,
 *            1 / scale, 0); the scaling is exact, so any finite input keeps
 *            11 significant bits relative to the row's maximum and nothing
 *            saturates); contents on entry do not matter.
 */
size_t csa_mqa_workspace_size(int B, int Tq, int n_h, int d, long long n_keys_max);
int csa_sparse_mqa(const void* q, const float* gamma_q, float eps, const void* E, const float* E_scale,
                   long long N_cap, const int* idx, int k, const void* W, const float* W_scale, int W_cap,
                   int n_win, const float* sink, const int* q_pos, int B, int Tq, int n_h, int d,
                   int rope_dim, float rope_base, float scale, int dtype, void* out, void* workspace,
                   size_t ws_bytes, void* stream);

/*
 * a5 — HCA core attention (method page §3.3: larger m', no overlap, dense
 * attention, otherwise as CSA): as csa_sparse_mqa, with the selected set
 * replaced by every visible entry s < min(N_cap, floor((i + 1) / m)).
 * workspace: at least csa_mqa_workspace_size(B, Tq, n_h, d, N_cap + n_win).
 */
int hca_dense_mqa(const void* q, const float* gamma_q, float eps, const void* E, const float* E_scale,
                  long long N_cap, int m, const void* W, const float* W_scale, int W_cap, int n_win,
                  const float* sink, const int* q_pos, int B, int Tq, int n_h, int d, int rope_dim,
                  float rope_base, float scale, int dtype, void* out, void* workspace, size_t ws_bytes,
                  void* stream);

/*
 * Cache append (method page §3.5: the inference cache is heterogeneous -- a
 * classical cache whose blocks cover lcm(m, m') raw tokens holds the compressed
 * entries, and a state cache holds the sliding-window KV and the tokens of the
 * compression blocks that are not yet complete).  For every sequence b, the
 * n_new tokens T0[b] .. T0[b] + n_new - 1 arrive; in one call:
 *   - their window rows (RMSNorm with gamma, RoPE at the token's position) go
 *     to the sliding-window ring W (token t at row t mod W_cap; when n_new >
 *     W_cap only the last W_cap are written);
 *   - every CSA entry s with T0[b] < m (s + 1) <= T0[b] + n_new is compressed
 *     (overlapping, m; RMSNorm + RoPE at m s) into E_csa[b][s], and its indexer
 *     key (no norm, no RoPE) into K_idx[b][s] in k_dtype;
 *   - every HCA entry h with T0[b] < m' (h + 1) <= T0[b] + n_new is compressed
 *     (disjoint, m'; RMSNorm + RoPE at m' h) into E_hca[b][h];
 *   - the raw candidate rows of the last min(n_new, lcm(m, m')) new tokens go to
 *     the tail ring: tail[b][t mod lcm][...] holds, side by side, the token's
 *     C_a, Z_a, C_b, Z_b (c each), IC_a, IZ_a, IC_b, IZ_b (d_I each), C_h, Z_h
 *     (c each), 6 c + 4 d_I bf16 values.
 * Candidates of tokens before T0[b] are read from the tail ring, so a sequence's
 * appends must follow one another with the ring kept between them (T0[b] = 0
 * needs no ring contents).  The caches then equal the compression of the whole
 * sequence, entry by entry (appends in any chunking give the same bytes).
 *  T0      : [B] int32 on the device, tokens present before this append.
 *  C_a .. Z_h, W_raw : [B][n_new][c] (d_I for IC_*) bf16 rows of the new tokens.
 *  E_csa   : [B][N_csa][c] bf16;  K_idx: [B][N_csa][d_I] of k_dtype (BF16,
 *            FP8_E4M3 with K_scale fp32 [B][N_csa], or MXFP4 with K_scale
 *            E8M0 bytes [B][N_csa][d_I / 32]);  E_hca: [B][N_hca][c] bf16.
 *            Entries at or past the capacities are not written.
 *  W       : [B][W_cap][c] bf16;  gamma: [c] fp32 or NULL (1).
 *  Needs c, d_I multiples of 8 (at most 1024), lcm(m, m') in [2 m, 4096] and
 *  16-byte aligned inputs and tail.
 */
int csa_cache_append(int B, const int* T0, int n_new, int c, int d_I, int m, int m_hca,
                     const void* C_a, const void* Z_a, const void* C_b, const void* Z_b,
                     const void* IC_a, const void* IZ_a, const void* IC_b, const void* IZ_b,
                     const void* C_h, const void* Z_h, const void* W_raw, void* tail,
                     void* E_csa, void* K_idx, void* K_scale, int k_dtype, long long N_csa,
                     void* E_hca, long long N_hca, void* W, int W_cap, const float* gamma, float eps,
                     int rope_dim, float rope_base, void* stream);

/*
 * Grouped output projection of the attention outputs (method page §3.3:
 * because c * n_h is large, the output projection is grouped -- each group of
 * heads is projected down to d_g, the results are concatenated and projected
 * back to d).  For each of T rows (queries):
 *   y[t, q d_g + e] = sum_i o[t, q W + i] * W1[q, e, i]   (W = n_h c / groups;
 *                     group q is heads [q n_h / groups, (q+1) n_h / groups)),
 *   out[t, :]       = y[t, :] @ W2^T.
 *  o   : [T][n_h][c] bf16 (the attention output, e.g. B * Tq rows).
 *  W1  : [groups][d_g][W] bf16 (output-major: the input axis contiguous).
 *  W2  : [d][groups * d_g] bf16 (output-major).
 *  y   : [T][groups * d_g] bf16, written: the intermediate, rounded to bf16
 *        (RNE) from the fp32 sums before the second product reads it.
 *  out : [T][d] bf16, written (fp32 sums, RNE).
 *  Needs W % 64 == 0 and (groups d_g) % 64 == 0; o, W1, W2 and y 16-byte
 *  aligned (CSA_E_UNSUPPORTED otherwise).  Few rows (T <= 64) split the
 *  contraction over workgroups and need a workspace of
 *  csa_out_proj_workspace_size(...) bytes (16-byte aligned) for the fp32
 *  partials, which are summed in a fixed order: results do not depend on
 *  anything but the inputs.
 */
size_t csa_out_proj_workspace_size(int T, int n_h, int c, int groups, int d_g, int d);
int csa_grouped_out_proj(const void* o, const void* W1, const void* W2, void* y, void* out, int T,
                         int n_h, int c, int groups, int d_g, int d, void* workspace, size_t ws_bytes,
                         void* stream);

/*
 * csa_sparse_mqa without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (minus workspace and
 * ws_bytes), checks and results as csa_sparse_mqa, bit for bit.  The split
 * partials go to a static device array of CSA_NOALLOC_SCRATCH_BYTES that each
 * GPU holds from the library's first use on it until the process ends; the
 * call allocates and frees nothing.  A call whose partials need more than that
 * (csa_mqa_workspace_size(B, Tq, n_h, d, k + n_win) > CSA_NOALLOC_SCRATCH_BYTES;
 * the 1M-context decode of 16 sequences x 128 heads x 512 needs 12.8 MB)
 * returns CSA_E_UNSUPPORTED and launches nothing.  Every call on one GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other
 * streams, other threads) race on it and must be serialised by the caller.
 * Nothing in the array needs to hold any value on entry.
 */
#define CSA_NOALLOC_SCRATCH_BYTES (16u << 20)
int csa_sparse_mqa_noalloc(const void* q, const float* gamma_q, float eps, const void* E,
                           const float* E_scale, long long N_cap, const int* idx, int k, const void* W,
                           const float* W_scale, int W_cap, int n_win, const float* sink,
                           const int* q_pos, int B, int Tq, int n_h, int d, int rope_dim,
                           float rope_base, float scale, int dtype, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
