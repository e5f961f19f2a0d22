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
// n_jobs (1 .. 8) independent compressions in one launch
int launch_compress(const CompressArgs* a, int n_jobs, hipStream_t st);

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
  long long N_cap;
  const int* idx;   // NULL for dense
  int k;            // sparse slots
  int m;            // dense visibility
  const void* W;
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

}  // namespace csa
