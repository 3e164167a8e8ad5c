// Internal interface between the C-ABI host code and the three kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace relay {

// sys_attn: one launch over (row block, chunk, KV head) workgroups.
struct SysArgs {
  const void* q;        // [T_q, H_q, d]
  const void* sys_k;    // [H_kv, L_s, d]
  const void* sys_v;    // [H_kv, ceil(L_s/16), d, 16]
  float* o_part;        // [n_chunks, T_q, H_q, d]
  float* lse_part;      // [n_chunks, T_q, H_q]
  int sys_len;
  int total_q;
  int num_q_heads;
  int group;            // g = H_q / H_kv
  int chunk_len;        // keys per chunk, multiple of 32
  int n_chunks;
  int row_blocks;       // ceil(T_q * g / rows per workgroup)
  int xcd_remap;        // 1: grid size is a multiple of 8 and ids are remapped per XCD
  float scale_log2;     // scale * log2(e)
};

// Tile configuration of sys_attn: rt row tiles (16 rows each) per wave, wk waves
// sharing the rows over different keys, wr row groups per workgroup.
struct SysConfig {
  int rt, wk, wr;
};

// The configuration used for M = T_q * g stacked query rows per KV head.
inline SysConfig sys_config(int M) {
  if (M <= 16) return {1, 8, 1};
  if (M <= 32) return {2, 4, 1};
  if (M <= 64) return {4, 2, 1};
  return {2, 1, 4};
}

// ctx_attn: one launch over (row block, split, KV head, request) workgroups.
struct CtxArgs {
  const void* q;             // [T_q, H_q, d]
  const void* ctx_k;         // [num_blocks, H_kv, 16, d]
  const void* ctx_v;         // [num_blocks, H_kv, d, 16]
  const int32_t* block_tables;
  const int32_t* ctx_lens;
  const int32_t* cu_q_lens;  // NULL: one query per request
  float* o_part;             // [max_splits, T_q, H_q, d]
  float* lse_part;           // [max_splits, T_q, H_q]
  int batch;
  int total_q;
  int num_q_heads;
  int num_kv_heads;
  int group;
  int num_blocks;
  int max_blocks_per_seq;
  int max_ctx_len;           // clamp for c_b (keeps splits inside the workspace)
  int split_len;             // keys per split, multiple of 32
  int max_splits;
  int row_blocks;            // ceil(max_q_len * g / rows per workgroup)
  float scale_log2;
};

struct CtxConfig {
  int rt, wr;  // row tiles per wave, waves (row groups) per workgroup
};

inline CtxConfig ctx_config(int rows_per_request) {
  if (rows_per_request <= 16) return {1, 1};
  if (rows_per_request <= 32) return {2, 1};
  if (rows_per_request <= 64) return {2, 2};
  return {2, 4};
}

// relay_fuse: LSE-weighted merge of two groups of partials per row.
//   group A (system): a_count partials, partial i of row r at a_o[i*rows + r].
//   group B (context): per-request count ceil(c_b / b_split_len) (capped at
//   b_count) when b_split_len > 0, else b_count.
struct FuseArgs {
  const float* a_o;
  const float* a_lse;
  const float* b_o;
  const float* b_lse;
  const int32_t* ctx_lens;
  const int32_t* cu_q_lens;
  void* out;
  float* lse_out;  // may be NULL
  long long n_rows;
  int num_q_heads;
  int batch;
  int a_count;
  int b_count;
  int b_split_len;
  int out_bf16;
};

hipError_t launch_sys_attn(const SysArgs& a, const SysConfig& c, int in_dtype, int head_dim,
                           int nwg, hipStream_t stream);
hipError_t launch_ctx_attn(const CtxArgs& a, const CtxConfig& c, int in_dtype, int head_dim,
                           int nwg, hipStream_t stream);
hipError_t launch_relay_fuse(const FuseArgs& a, int head_dim, int nwg, hipStream_t stream);

constexpr int kFuseRowsPerWg = 8;  // 256 threads, 32 lanes per row at d = 128

}  // namespace relay
