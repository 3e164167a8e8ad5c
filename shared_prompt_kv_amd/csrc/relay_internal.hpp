// Internal interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace relay {

// Optional timing of one launch: events the runtime stamps with the kernel's own start
// and end (hipExtLaunchKernelGGL), not with the time the launch is enqueued.
struct LaunchTiming {
  hipEvent_t start;
  hipEvent_t stop;
};

template <typename... KArgs, typename... Args>
inline void launch_kernel(void (*kernel)(KArgs...), dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                          const LaunchTiming* tm, Args... args) {
  if (tm && (tm->start || tm->stop))
    hipExtLaunchKernelGGL(kernel, grid, block, lds, s, tm->start, tm->stop, 0, args...);
  else
    hipLaunchKernelGGL(kernel, grid, block, lds, s, args...);
}

// sys_attn_tiled (large M): one launch over (row block, chunk, KV head) workgroups.
struct SysArgs {
  const void* q;        // [T_q, H_q, d]
  const void* sys_k;    // [H_kv, ceil(L_s/16), d/G, 16, G] key tiles
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
  // sys_attn_mfma only: the 64-key steps of all KV heads, head after head
  // (total_steps = H_kv * steps_per_head), are cut into `parts` equal runs; workgroup
  // (row block, part) streams its run, writing one partial per head it touches into
  // slot (part - first part of that head) < n_chunks.
  int steps_per_head;
  int total_steps;
  int parts;
  // sys_attn_mfma only: 1 = causal, query token t sees system keys 0..t only (the
  // prompt's own attention in the offline prefill; scale must be > 0)
  int causal;
};

// Tile configuration of sys_attn_tiled: rt row tiles (16 rows each) per wave, wk waves
// sharing the rows over different keys, wr row groups per workgroup.
struct SysConfig {
  int rt, wk, wr;
};

// Up to this many stacked query rows per KV head the system step streams together with
// the context step (HBM-bound, one stream per KV head); above it the matrix-core system
// kernel runs first (compute-bound).
constexpr int kStreamSysMaxRows = 64;

// The tiled kernel's configuration (it runs only above kStreamSysMaxRows stacked rows).
inline SysConfig sys_config(int) { return {2, 1, 4}; }

// stream_attn (stream_attn.hip): the system and context steps as one launch of equal
// contiguous step ranges, one per wave.
constexpr int kStreamWaves = 4;  // waves per workgroup

// Workgroups per CU a streaming instantiation is built for: two (two waves per SIMD,
// so one wave's arithmetic hides under the other's loads) wherever its registers fit
// 256 without spilling, else one.
constexpr int stream_wgs_per_cu(int elem_bytes, int head_dim, int rts, int rtc) {
  if (elem_bytes == 2) return (head_dim == 128 && rts == 4) ? 1 : 2;
  if (head_dim == 128) return (rts >= 2 || rtc == 2) ? 1 : 2;
  return rts == 4 ? 1 : 2;
}

// LDS of the system pieces' four-wave merge: two waves' states of one 16-row tile.
constexpr int stream_merge_lds_bytes(int head_dim) { return 2 * 64 * (2 + head_dim / 4) * 4; }

// Requests per streaming launch: their four LDS tables, the scan scratch and the merge
// area fit 64 KiB.
constexpr int kStreamMaxRequests = 2880;
static_assert(((4 * (4 * kStreamMaxRequests + 1 + 256) + 15) / 16) * 16 + stream_merge_lds_bytes(128) <= 65536,
              "streaming LDS over 64 KiB");

struct StreamArgs {
  const void* q;       // [T_q, H_q, d]
  int total_q;
  int num_q_heads;
  int num_kv_heads;
  int group;
  float scale_log2;    // scale * log2(e)
  // system streams: one per KV head over its M <= 64 stacked rows (sys_steps = 0: none)
  const void* sys_k;   // [H_kv, ceil(L_s/16), d/G, 16, G] key tiles
  const void* sys_v;   // [H_kv, ceil(L_s/16), d, 16]
  int sys_len;
  int sys_steps;       // ceil(L_s / 32)
  int M;               // stacked rows per KV head (T_q * g)
  float* sys_o;        // [H_kv ks + H_kv + workgroups slots][16 RTS rows][d]
  float* sys_lse;      // [slots][16 RTS]
  int* sys_desc;       // [H_kv][2]: first slot, number of pieces
  // context streams (request, KV head, row block) of requests [b_begin, b_begin + n_req)
  int ctx_on;
  const void* ctx_k;   // [num_blocks, H_kv, d/G, 16, G] key tiles
  const void* ctx_v;   // [num_blocks, H_kv, d, 16]
  const int32_t* block_tables;
  const int32_t* ctx_lens;
  const int32_t* cu_q_lens;  // NULL: one query per request
  int batch;
  int b_begin;
  int n_req;
  int num_blocks;
  int max_blocks_per_seq;
  int max_ctx_len;     // clamp for c_b
  int ctx_rb;          // row blocks (16 RTC rows each) per (request, KV head)
  long long slot_base; // first context slot of this launch's pieces
  float* ctx_o;        // [slots][16 RTC][d]
  float* ctx_lse;      // [slots][16 RTC]
  int* ctx_rowdesc;    // [T_q * H_q][4]: first slot, number of pieces, row in the piece
  // pieces at places fixed in advance, where the merge finds them without looking up
  // where they are: piece k < ks of KV head h's system stream in system slot h ks + k
  // (later ones in slot H_kv ks + h + w), piece j < kc of a context stream in slot j of
  // each of its rows, row_o[(r kc + j) d] (later ones in the stream slots above)
  float* row_o;
  float* row_lse;      // [T_q * H_q][kc]
  int ks, kc;
  int n_workers;       // waves of the launch (grid * kStreamWaves)
};

// The decode step's launch of matrix-core system workgroups (the first n_sys) beside the
// context streams' workgroups (stream_attn.hip).
struct CoArgs {
  SysArgs sys;
  StreamArgs str;
  int n_sys;
};
hipError_t launch_stream_sys(const CoArgs& a, int rtc, int grid, hipStream_t stream, const LaunchTiming* tm = nullptr);

// Workgroups of one streaming launch for this instantiation on a device with `cus` CUs.
inline int stream_grid(int cus, int elem_bytes, int head_dim, int rts, int rtc) {
  return cus * stream_wgs_per_cu(elem_bytes, head_dim, rts, rtc);
}

size_t stream_lds_bytes(int n_req, int ctx_on, int sys_on, int head_dim);
hipError_t launch_stream_attn(const StreamArgs& a, int rts, int rtc, int in_dtype, int head_dim, int grid,
                              hipStream_t stream, const LaunchTiming* tm = nullptr);

// Row tiles per context stream for up to R query rows per (request, KV head).
inline int ctx_rt_for(int rows_per_request) { return rows_per_request <= 16 ? 1 : 2; }

// relay_merge (relay_fuse.hip): each row's output from the pieces of its system stream
// (or the runs of the system kernel) and of its context stream.
struct MergeArgs {
  long long n_rows;    // T_q * H_q
  int num_q_heads;
  int group;
  // system part: 0 none, 1 stream pieces (sys_desc), 2 system-kernel runs (slot i of
  // row r at sys_o[(i n_rows + r) d], LSE = -inf marks an empty run)
  int sys_src;
  const float* sys_o;
  const float* sys_lse;
  const int* sys_desc;
  int sys_rows;        // rows per stream slot (16 RTS)
  long long sys_slots; // stream slots (clamp)
  int sys_runs;        // sys_src 2: run slots per row
  // context part: stream pieces located by ctx_rowdesc
  int ctx_on;
  const float* ctx_o;
  const float* ctx_lse;
  const int* ctx_rowdesc;
  int ctx_rows;        // rows per context slot (16 RTC)
  long long ctx_slots; // context slots (clamp)
  // pieces at fixed places (StreamArgs::row_o): the first ks system pieces of every KV
  // head, the first kc context pieces of every row
  const float* row_o;
  const float* row_lse;
  int ks, kc;
  void* out;
  float* lse_out;      // may be NULL
  int out_bf16;
};
hipError_t launch_relay_merge(const MergeArgs& a, int head_dim, hipStream_t stream, const LaunchTiming* tm = nullptr);
// Most pieces at fixed places per row (system and context together), which the merge
// reads with the descriptors; the most output rows a plan gives such places.
constexpr int kMaxRowSlots = 16;
constexpr long long kRowSlotRows = 4096;
inline int merge_threads(int head_dim, long long n_rows) {
  return n_rows >= 2LL * 256 * (256 / (head_dim / 4)) ? 256 : 64;
}

// relay_fuse: LSE-weighted merge of two groups of partials per row: group A
// (system chunks) a_count partials, partial i of row r at a_o[i*rows + r]; group B
// (context splits) likewise with b_count.  A partial with LSE = -inf is empty: its
// weight is 0 and its O is never used (it may be unwritten).
struct FuseArgs {
  const float* a_o;
  const float* a_lse;
  const float* b_o;
  const float* b_lse;
  void* out;
  float* lse_out;  // may be NULL
  long long n_rows;
  int a_count;
  int b_count;
  int a_sparse;    // group A slots may be empty (runs of the matrix-core system kernel)
  int out_bf16;
};

// relay_rope.hip: position embedding and KV append.
struct RopeArgs {
  const void* q_new;
  const void* k_new;
  const void* v_new;
  const float* cos_sin;  // [max_pos, head_dim]
  const int32_t* block_tables;
  const int32_t* ctx_lens;
  const int32_t* cu_q_lens;  // NULL: one token per request
  void* q_out;
  void* ctx_k;
  void* ctx_v;
  int batch, num_q_heads, num_kv_heads, head_dim, total_q;
  int max_blocks_per_seq, num_blocks, sys_len, max_pos, bf16;
};
hipError_t launch_rope_table(float* cos_sin, int max_pos, int d, double base, hipStream_t s);
hipError_t launch_rope_append(const RopeArgs& a, int max_q_len, hipStream_t s);
hipError_t launch_system_fill(const void* k_raw, const void* v_raw, const float* cos_sin, void* sys_k, void* sys_v,
                              int sys_len, int num_kv_heads, int d, int bf16, hipStream_t s);
hipError_t launch_rope_system(void* sys_k, const float* cos_sin, int sys_len, int num_kv_heads, int d, int bf16,
                              hipStream_t s);

hipError_t launch_sys_attn_tiled(const SysArgs& a, const SysConfig& c, int in_dtype, int head_dim,
                                 int nwg, hipStream_t stream, const LaunchTiming* tm = nullptr);

// sys_attn_mfma (bf16, head_dim 128): workgroups of kSysMfmaRows query rows; designed
// for two workgroups per CU (kSysMfmaSlots resident at once).
constexpr int kSysMfmaRows = 128;
// The decode system step as a launch of its own: one workgroup of kSysPPRows rows (eight
// waves in two groups half a step apart) per CU.
constexpr int kSysPPRows = 256;
constexpr int kSysMfmaSlots = 512;
constexpr int kSysMfmaStep = 64;
// Rates the decode plan weighs the system step's matrix-core time against the context
// step's memory time with (measured on MI355X: the system kernel at two workgroups per CU
// runs at about 0.9 PFLOP/s, the streaming launch at about 4.5 TB/s).
constexpr double kSysMfmaFlopsPerS = 0.9e15;
constexpr double kStreamBytesPerS = 4.5e12;
// Partials in which some row sees fewer than this many keys compute P.V with P split
// into bf16 hi + lo (two products): there single probabilities can be large and bf16
// rounding of P alone would cost up to 2^-9 of the output.  Where every row sees many
// keys the weight is spread over them and P is rounded once.
constexpr int kPSplitBelow = 256;
constexpr int kSysCausalRunsPerSlot = 4;  // causal plans: runs per resident workgroup slot

// The part (of `parts` equal runs over `total` steps) that holds step x.
inline __host__ __device__ int lean_part_of(long long x, int total, int parts) {
  return (int)(((x + 1) * parts + total - 1) / total) - 1;
}
hipError_t launch_sys_attn_mfma(const SysArgs& a, int nwg, hipStream_t stream, const LaunchTiming* tm = nullptr);
hipError_t launch_sys_attn_pp(const SysArgs& a, int nwg, hipStream_t stream, const LaunchTiming* tm = nullptr);
// relay_fuse workgroup size: one wave, or four once there are enough rows for two
// four-wave workgroups per CU (D/4 lanes per row).
inline int fuse_threads(int head_dim, long long n_rows) {
  return n_rows >= 2LL * 256 * (256 / (head_dim / 4)) ? 256 : 64;
}
inline int fuse_rows_per_wg(int head_dim, long long n_rows) { return fuse_threads(head_dim, n_rows) / (head_dim / 4); }
// Rows with many slots that may be empty (every context split past the first; group A
// slots when they are runs that need not touch a head): outputs of empty slots are
// skipped.  Chunks of the streaming system units always hold keys for every row.
inline bool fuse_skips_empty(const FuseArgs& a) {
  return (a.a_sparse ? a.a_count : 0) + (a.b_count > 1 ? a.b_count - 1 : 0) > 4;
}
hipError_t launch_relay_fuse(const FuseArgs& a, int head_dim, int nwg, hipStream_t stream);


}  // namespace relay
