// Host-side launcher interfaces between the C ABI (csa_abi.hip) and the kernels.
// Arguments arrive here already validated.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa {

struct CompressArgs {
  const void *C_a, *Z_a, *C_b, *Z_b;
  int in_dtype;
  int B;
  long long R, in_bs, tok_base, T;
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
  long long out_bs, out_ring;
};
// n_jobs (1 .. 8) independent compressions in one launch.  ws / ws_bytes: the
// optional workspace of the channel-split path (compress_workspace_bytes; NULL:
// every job runs whole rows)
int launch_compress(const CompressArgs* a, int n_jobs, hipStream_t st, void* ws = nullptr, size_t ws_bytes = 0);
size_t compress_workspace_bytes(const CompressArgs* a, int n_jobs);

struct IndexArgs {
  const void* q;
  int q_dtype;
  const float* w;
  const void* K;
  int k_dtype;
  const float* K_scale;
  const int* q_pos;
  int B, Tq, H, dI;
  long long N_cap;
  int m;
  float* out;
};
// true when the matrix-core kernels cover the shape
bool index_mfma_supported(const IndexArgs& a);
int launch_index_score(const IndexArgs& a, hipStream_t st);
// compress jobs and the decode indexer in one launch (validated here: returns
// -1 with *why set when the combination is not covered, 0 once launched)
int launch_decode_front(const CompressArgs* jobs, int n_jobs, const IndexArgs& a, hipStream_t st,
                        const char** why);

struct TopkArgs {
  const float* I;
  const int* q_pos;
  int B, Tq;
  long long N_cap;
  int m, k;
  int* idx;
  float* val;
  void* ws;
  size_t ws_bytes;
};
size_t topk_workspace_bytes(int B, int Tq, long long N_cap, int k);
int launch_topk(const TopkArgs& a, hipStream_t st);

struct MqaArgs {
  const void* q;
  const float* gamma_q;
  float eps;
  const void* E;
  const float* E_scale;   // mixed entries: the row scales ([B][N_cap]); else NULL
  long long N_cap;
  const int* idx;   // NULL for dense
  int k;            // sparse slots
  int m;            // dense visibility
  const void* W;
  const float* W_scale;   // mixed window rows: the row scales ([B][W_cap]); else NULL
  int W_cap, n_win;
  const float* sink;
  const int* q_pos;
  int B, Tq, n_h, d, rope_dim;
  float rope_base, scale;
  int dtype;
  void* out;
  void* ws;
  size_t ws_bytes;
};
// maximum number of key slots one query can have
long long mqa_slots_max(const MqaArgs& a);
size_t mqa_workspace_bytes(int B, int Tq, int n_h, int d, long long n_slots_max, int dtype);
// returns 0 or a CSA status (UNSUPPORTED / HIP) and fills *why on failure
int launch_mqa(const MqaArgs& a, hipStream_t st, const char** why);

struct CacheAppendArgs {
  int B;
  const int* T0;    // [B] tokens present before the append (device)
  int n_new, c, d_I, m, m_hca, ring;
  const void *Ca, *Za, *Cb, *Zb, *ICa, *IZa, *ICb, *IZb, *Ch, *Zh, *Wraw;   // [B][n_new][width] bf16
  void* tail;       // [B][ring][6 c + 4 d_I] bf16
  void* E_csa;      // [B][N_csa][c] bf16
  void* K_idx;      // [B][N_csa][d_I] of k_dtype
  void* K_scale;
  int k_dtype;
  long long N_csa;
  void* E_hca;      // [B][N_hca][c] bf16
  long long N_hca;
  void* W;          // [B][W_cap][c] bf16
  int W_cap;
  const float* gamma;
  float eps;
  int rope_dim;
  float rope_base;
};
int launch_cache_append(const CacheAppendArgs& a, hipStream_t st);

struct ProjArgs {
  const void* o;    // [T][n_h c] bf16
  const void* W1;   // [groups][d_g][n_h c / groups] bf16
  const void* W2;   // [d][groups d_g] bf16
  void* y;          // [T][groups d_g] bf16 (intermediate, written)
  void* out;        // [T][d] bf16
  int T, n_h, c, groups, d_g, d;
  void* ws;
  size_t ws_bytes;
};
size_t proj_workspace_bytes(const ProjArgs& a);
int launch_proj(const ProjArgs& a, hipStream_t st);

}  // namespace csa
