/*
 * relay_attn.h - C ABI of librelay_attn.so: RelayAttention decode-time attention
 * on AMD Instinct MI355X (gfx950).
 *
 * RelayAttention (RelayAttention paper, abstract; atyun.com article, section
 * "RelayAttention"; linnk.ai summary, section "Abstract") computes causal decode
 * attention over a long system prompt shared by every request plus each request's
 * own context in three steps:
 *
 *   1. system attention  - every query row of the batch attends to the shared
 *      system KV cache alone; the cache is read from HBM once for the whole batch
 *      by stacking all query rows into one matrix-matrix product;
 *   2. context attention - each request attends to its own paged context KV alone;
 *   3. relay fusion      - the final output is a weighted average of the two
 *      intermediate outputs with non-negative weights that sum to one.  The pages
 *      fix nothing more about the weights; here they are alpha_sys = e^LSE_sys /
 *      (e^LSE_sys + e^LSE_ctx) and alpha_ctx = 1 - alpha_sys, the only such weights
 *      for which the result equals exact causal attention over [system; context].
 *
 * The system KV cache is separate from the context cache and filled before
 * serving; context positions follow the system prompt (atyun.com article, section
 * "RelayAttention").  The kernels take post-RoPE Q and K, so absolute positions
 * never enter; only the causal index inside the context does.
 *
 * ---------------------------------------------------------------------------
 * Conventions shared by every entry point
 * ---------------------------------------------------------------------------
 *  - All array arguments are DEVICE pointers (HIP device memory of the current
 *    device) unless marked "host".  Arrays are dense, row-major, with no padding
 *    beyond what the layouts below state.  Every pointer must be 16-byte aligned.
 *  - The caller owns every buffer.  The library allocates no device memory, keeps
 *    no pointer after a call returns, never synchronises the device and enqueues
 *    work only on `stream` (a hipStream_t; NULL = the legacy default stream).
 *    Results are valid once the stream's work has completed.
 *  - Return value: RELAY_OK (0) or a negative RELAY_ERR_* code.  Argument errors
 *    are detected on the host before anything is enqueued.  relay_last_error()
 *    returns a thread-local message describing the most recent failure.
 *  - Data-dependent preconditions (block ids in range, 1 <= n_b <= c_b <= the
 *    stated maxima) are the caller's; relay_validate() checks them on host copies.
 *    Kernels clamp indices so that violating them cannot read or write out of
 *    bounds, but the numbers are then unspecified.
 *  - Thread safety: the library's only process-wide state is written once per
 *    device and read atomically: the device's compute-unit count (it sizes the
 *    launches) and, for relay_attn_decode_noalloc, the device address of its static
 *    scratch.  No environment variable is read.  Concurrent calls on different
 *    streams with disjoint outputs and workspaces are safe; concurrent
 *    relay_attn_decode_noalloc calls on one device share its scratch and race.
 *
 * Notation: B requests; request b has n_b new query tokens (T_q = sum n_b) and a
 * context of c_b tokens that INCLUDES its n_b new tokens (their K/V are already in
 * the pages).  Query token t of request b (0 <= t < n_b) sits at context position
 * p = c_b - n_b + t and sees context keys 0..p and all system keys.  H_q query
 * heads, H_kv KV heads, g = H_q / H_kv; query head h uses KV head h / g.  d is the
 * head dimension, E the element size of in_dtype, L_s the system length.
 *
 * Layouts (E-byte elements unless stated):
 *   q            [T_q, H_q, d]               tokens of request b are rows
 *                                            cu_q_lens[b] .. cu_q_lens[b+1]-1
 *   sys_k        [H_kv, ceil(L_s/16), d/G, 16, G]  system keys in 16-key tiles,
 *                                            chunk-major, keys in slot order inside a
 *                                            chunk (below; the tail tile's padding keys
 *                                            are ignored)
 *   sys_v        [H_kv, ceil(L_s/16), d, 16] system values in 16-key tiles,
 *                                            dimension-major inside a tile (the
 *                                            tail tile's padding is ignored)
 *   ctx_k_pages  [num_blocks, H_kv, d/G, 16, G]  paged context keys, 16 tokens a
 *                                            page, chunk-major, keys in slot order
 *   ctx_v_pages  [num_blocks, H_kv, d, 16]   paged context values, dimension-major
 *                                            inside a page
 *   block_tables int32 [B, max_blocks_per_seq]  context token j of request b is
 *                                            key j%16 of page block_tables[b][j/16]
 *                                            (its K stored in slot slot(j%16));
 *                                            entries past ceil(c_b/16) are unused
 *   ctx_lens     int32 [B]                   c_b
 *   cu_q_lens    int32 [B+1] prefix sums of n_b (cu_q_lens[0] = 0), or NULL when
 *                every request has exactly one query token (then T_q = B)
 *   out          [T_q, H_q, d] of out_dtype
 *   LSE arrays   float32 [T_q, H_q], natural log of sum_j exp(scale * q.k_j);
 *                -inf marks an empty key set
 *   O partials   float32 [T_q, H_q, d]
 * Values are stored dimension-major (d before the 16 keys of a tile/page) so that
 * the keys a matrix-core lane reduces over are contiguous in memory.  Keys are stored
 * chunk-major: G = 16 / E elements (8 bf16, 4 fp32) make one 16-byte chunk, and a
 * tile/page holds chunk 0 of its 16 keys, then chunk 1, ...  Inside a chunk the keys
 * are in slot order: slot s holds key slot(s), where slot() exchanges keys 4..7 with
 * keys 8..11 (slot(r) = 0, 1, 2, 3, 8, 9, 10, 11, 4, 5, 6, 7, 12, 13, 14, 15 for
 * r = 0..15; it is its own inverse).  Element c of key r of a tile is at
 *     ((c / G) * 16 + slot(r)) * G + c % G.
 * The 64 lanes that load one matrix-core operand of a 16-key tile then read 1 KB of
 * contiguous memory, and slots 0..7 / 8..15 of a step's two pages are the score tiles
 * whose lanes hold 8 consecutive keys of one page.
 */
#ifndef RELAY_ATTN_H
#define RELAY_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RELAY_ATTN_ABI_VERSION 6  /* 3: keys in slot order inside each 16-byte chunk of a tile; plan
                                     fields of the streaming launch.  4: relay_attn_decode_timed
                                     takes kernel start/end event pairs.  5: relay_plan.sys_rows_per_wg.
                                     6: relay_plan.sys_row_slots, ctx_row_slots */

/* element types */
#define RELAY_F32 0  /* IEEE float32 */
#define RELAY_BF16 1 /* bfloat16 (bit pattern, round-to-nearest-even producers) */

/* return codes */
#define RELAY_OK 0
#define RELAY_ERR_INVALID (-1)     /* bad argument: NULL pointer, bad size, misaligned */
#define RELAY_ERR_UNSUPPORTED (-2) /* valid but unsupported: head_dim, block size, dtype */
#define RELAY_ERR_WORKSPACE (-3)   /* workspace smaller than relay_workspace_size() */
#define RELAY_ERR_HIP (-4)         /* a HIP launch failed; see relay_last_error() */
#define RELAY_ERR_DATA (-5)        /* relay_validate(): inconsistent host data */

/* Problem dimensions, passed by host pointer. */
typedef struct {
  int32_t batch;              /* B >= 1 */
  int32_t num_q_heads;        /* H_q, a multiple of num_kv_heads */
  int32_t num_kv_heads;       /* H_kv >= 1 */
  int32_t head_dim;           /* d: 64 or 128 */
  int32_t block_size;         /* context page size in tokens: must be 16 */
  int32_t max_blocks_per_seq; /* columns of block_tables */
  int32_t num_blocks;         /* pages in the context pool */
  int32_t total_q;            /* T_q = cu_q_lens[B] (== B when cu_q_lens is NULL) */
  int32_t max_q_len;          /* upper bound on n_b (1 when cu_q_lens is NULL) */
  int32_t max_ctx_len;        /* upper bound on c_b; sizes the split plan on the host */
  float scale;                /* softmax scale, e.g. 1/sqrt(d) */
  int32_t in_dtype;           /* RELAY_F32 or RELAY_BF16: q, K and V */
  int32_t out_dtype;          /* RELAY_F32 or RELAY_BF16: out of relay_attn_decode */
} relay_dims;

/* How a call is split into launches (for benchmarks and tests). */
typedef struct {
  int32_t sys_mode;            /* 0: no system step; 1: system streams inside the streaming launch
                                  (at most 64 stacked query rows per KV head); 2: the matrix-core
                                  system kernel runs first (bf16, head_dim 128; the system step
                                  alone); 3: the tiled system kernel runs first (fp32 or head_dim
                                  64); 4: the matrix-core system workgroups inside the first
                                  streaming launch, beside the context workgroups (the decode step,
                                  bf16, head_dim 128, more than 64 rows per KV head) */
  int32_t sys_row_tiles;       /* sys_mode 1: 16-row tiles of one system stream */
  int32_t sys_runs;            /* sys_mode 2, 3, 4: partial slots per row written by the system kernel */
  int32_t sys_wgs;             /* sys_mode 2, 3, 4: workgroups of the system kernel */
  int32_t ctx_row_tiles;       /* 16-row tiles of one context stream */
  int32_t ctx_row_blocks;      /* context streams per (request, KV head) */
  int32_t stream_waves;        /* waves of one streaming launch; each streams an equal share of the steps */
  int32_t stream_launches;     /* streaming launches (requests in groups of stream_max_requests) */
  int32_t stream_max_requests; /* requests per streaming launch */
  int32_t merge_wgs;           /* workgroups of the merge launch */
  int32_t launches;            /* kernel launches of one relay_attn_decode call */
  int32_t sys_rows_per_wg;     /* sys_mode 2, 4: stacked query rows per matrix-core system workgroup
                                  (128; 256 for the eight-wave kernel that sys_mode 2 uses when its
                                  row blocks fill) */
  int32_t sys_row_slots;       /* sys_mode 1: pieces of a KV head's system stream written to workspace
                                  slots fixed in advance (the merge reads those with the
                                  descriptors, in one memory round trip; later pieces cost it a
                                  second); from an estimate of the launch's steps (the context
                                  lengths are device data); 0 above 4096 output rows */
  int32_t ctx_row_slots;       /* the same for the pieces of a context stream (each row's own slots) */
} relay_plan;

/* ABI version compiled into the library (RELAY_ATTN_ABI_VERSION). */
int relay_abi_version(void);

/* Static string for a return code. */
const char* relay_strerror(int code);

/* Thread-local description of the most recent failure of this thread ("" if none). */
const char* relay_last_error(void);

/*
 * Bytes of device workspace that relay_attn_decode, relay_sys_attn and
 * relay_ctx_attn need for these dimensions and system length: the partial outputs
 * and log-sum-exps of the streaming launch's pieces (the first relay_plan.sys_row_slots
 * of each system stream and ctx_row_slots of each context stream at places fixed in
 * advance) and of the system kernel's runs, and descriptors of where each row's other
 * pieces are.  Returns 0 on invalid dims (see relay_last_error()).
 */
size_t relay_workspace_size(const relay_dims* dims, int32_t sys_len);

/* Fills *plan with the work split for these dims; RELAY_OK or an error code. */
int relay_get_plan(const relay_dims* dims, int32_t sys_len, relay_plan* plan);

/*
 * The whole RelayAttention decode step (RelayAttention paper page, Abstract: the
 * system KV read once per batch, then combined with each request's own attention;
 * atyun.com article, section "RelayAttention": the three steps and their exact
 * equivalence to attention over the concatenated cache): system attention (skipped
 * when sys_len == 0), context attention and relay fusion, written to out.  Equals
 * exact causal attention of each query row over its visible [system; context] keys.
 * Enqueued on `stream`: one streaming launch that runs the system and context steps
 * together (per group of at most relay_plan.stream_max_requests requests), then the
 * merge (2 launches for up to that many requests).  At most 64 query rows per KV head
 * take the system step as streams of the launch; more rows take it as matrix-core
 * workgroups of the launch's first group (bf16, head_dim 128), or as a system kernel
 * before it (3 launches: fp32 or head_dim 64).  relay_get_plan() says which.  workspace must hold relay_workspace_size(dims,
 * sys_len) bytes (256-byte aligned): the partial results and where they are; its
 * contents on entry are irrelevant (nothing in it needs to start at zero) and on
 * return unspecified.
 */
int relay_attn_decode(const relay_dims* dims, const void* q, const void* sys_k,
                      const void* sys_v, int32_t sys_len, const void* ctx_k_pages,
                      const void* ctx_v_pages, const int32_t* block_tables,
                      const int32_t* ctx_lens, const int32_t* cu_q_lens, void* out,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * relay_attn_decode with per-kernel timing: identical work, plus six events
 * (hipEvent_t handles created by the caller; any entry may be NULL) that the runtime
 * stamps with the start and the end of the kernels themselves (not with the time a
 * launch is enqueued): [0], [1] the separate system-attention kernel, [2], [3] the
 * streaming attention launch (the first one's start and the last one's end when the
 * requests take several), [4], [5] the merge.  Events of a kernel the call does not
 * launch (no separate system kernel when at most 64 query rows share a KV head; see
 * relay_get_plan) are left untouched.  For benchmarks; events must not be NULL.
 */
int relay_attn_decode_timed(const relay_dims* dims, const void* q, const void* sys_k,
                            const void* sys_v, int32_t sys_len, const void* ctx_k_pages,
                            const void* ctx_v_pages, const int32_t* block_tables,
                            const int32_t* ctx_lens, const int32_t* cu_q_lens, void* out,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events);

/*
 * relay_attn_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): identical
 * arguments and results, minus the workspace.  Its workspace is a static array of
 * RELAY_NOALLOC_SCRATCH_BYTES per device, held by the loaded library until the process
 * ends; nothing is allocated or freed, and no part of the array needs to start at
 * zero.  Every call on one device shares that device's array, which keeps the last
 * call's contents: calls that overlap on one device (other streams, other threads)
 * race and must be serialised by the caller.  Returns RELAY_ERR_WORKSPACE when
 * relay_workspace_size(dims, sys_len) exceeds RELAY_NOALLOC_SCRATCH_BYTES; errors
 * otherwise as relay_attn_decode.
 */
#define RELAY_NOALLOC_SCRATCH_BYTES (128u << 20)
int relay_attn_decode_noalloc(const relay_dims* dims, const void* q, const void* sys_k,
                              const void* sys_v, int32_t sys_len, const void* ctx_k_pages,
                              const void* ctx_v_pages, const int32_t* block_tables,
                              const int32_t* ctx_lens, const int32_t* cu_q_lens, void* out,
                              void* stream);

/*
 * System-attention step alone (atyun.com article, section "RelayAttention", first
 * step: every request's query rows against the shared system keys, the per-request
 * matrix-vector products grouped into matrix-matrix products; linnk.ai summary,
 * section "Deeper Inquiries"): for every query row, attention over the system keys
 * only.  o_sys: float32 [T_q, H_q, d]; lse_sys: float32 [T_q, H_q].  sys_len == 0
 * gives o_sys = 0 and lse_sys = -inf.  Enqueues the system step (the streaming
 * launch's system streams at <= 64 rows per KV head, else the matrix-core system
 * kernel) and the merge of its partials.
 */
int relay_sys_attn(const relay_dims* dims, const void* q, const void* sys_k, const void* sys_v,
                   int32_t sys_len, float* o_sys, float* lse_sys, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * The attention half of the offline system prefill.  RelayAttention fills the
 * system KV cache once, offline, before serving (atyun.com article, section
 * "RelayAttention"; the cost analysis there); the system prompt's own tokens then
 * need their causal attention over that cache, which is this call.  Query row
 * (t, h) -- prompt token t, query head h -- attends to system keys 0..min(t,
 * sys_len - 1) of KV head h / g, exactly.
 *   q:      [total_q, H_q, d], token t at position t, already position-embedded
 *           (relay_rope_append with sys_len = 0 does that);
 *   sys_k, sys_v: the system cache as for relay_attn_decode (relay_system_fill);
 *   out:    [total_q, H_q, d] of out_dtype (RELAY_F32 or RELAY_BF16);
 *   lse_out: float32 [total_q, H_q] (natural log, scale included), or NULL.
 * Only dims' total_q, num_q_heads, num_kv_heads, head_dim, in_dtype and scale
 * matter; the rest must pass the usual checks (e.g. batch 1, max_q_len =
 * max_ctx_len = total_q, ceil(total_q / 16) blocks).  Runs
 * the matrix-core system kernel with a causal mask, then relay_fuse (2 launches):
 * needs bf16 inputs, head_dim 128, more than 64 query rows per KV head (else
 * RELAY_ERR_UNSUPPORTED), sys_len >= 1 and scale > 0 (else RELAY_ERR_INVALID).
 * workspace: relay_prefill_workspace_size(dims, sys_len) bytes, 256-byte aligned,
 * contents irrelevant on entry.
 */
size_t relay_prefill_workspace_size(const relay_dims* dims, int32_t sys_len);
int relay_prefill_attn(const relay_dims* dims, const void* q, const void* sys_k, const void* sys_v,
                       int32_t sys_len, void* out, int32_t out_dtype, float* lse_out, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Context-attention step alone (atyun.com article, section "RelayAttention",
 * second step: each request against its own keys in the paged cache, as
 * PagedAttention does; linnk.ai summary, section "Abstract"): for every query row,
 * causal attention over its request's visible context keys only.  o_ctx / lse_ctx
 * as for relay_sys_attn.  Enqueues the streaming launch's context streams and the
 * merge of their pieces.
 */
int relay_ctx_attn(const relay_dims* dims, const void* q, const void* ctx_k_pages,
                   const void* ctx_v_pages, const int32_t* block_tables,
                   const int32_t* ctx_lens, const int32_t* cu_q_lens, float* o_ctx,
                   float* lse_ctx, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Relay fusion alone (atyun.com article, section "RelayAttention", third step: the
 * two intermediate outputs averaged with weights from their log-sum-exp normalisers;
 * linnk.ai summary, section "Abstract": a convex combination) over n_rows rows of
 * head_dim values: out = alpha_sys * o_sys + alpha_ctx * o_ctx with the LSE weights
 * above.
 * o_*: float32 [n_rows, head_dim]; lse_*: float32 [n_rows]; a part with LSE = -inf
 * has weight 0.  out: [n_rows, head_dim] of out_dtype.  lse_out (may be NULL):
 * float32 [n_rows], ln(e^lse_sys + e^lse_ctx).  head_dim: 64 or 128.
 */
int relay_fuse(int64_t n_rows, int32_t head_dim, const float* o_sys, const float* lse_sys,
               const float* o_ctx, const float* lse_ctx, void* out, int32_t out_dtype,
               float* lse_out, void* stream);

/*
 * Host-side check of the data-dependent preconditions on HOST copies of the
 * integer arrays: 1 <= n_b <= c_b <= max_ctx_len, n_b <= max_q_len,
 * ceil(c_b/16) <= max_blocks_per_seq, used block ids in [0, num_blocks), and
 * cu_q_lens consistent with total_q.  h_cu_q_lens may be NULL (n_b = 1).
 * RELAY_OK or RELAY_ERR_DATA / RELAY_ERR_INVALID; enqueues nothing.
 */
int relay_validate(const relay_dims* dims, const int32_t* h_block_tables,
                   const int32_t* h_ctx_lens, const int32_t* h_cu_q_lens, int32_t sys_len);

/*
 * ---- The step before the path: position embedding and KV append --------------
 *
 * The system K/V are prefilled offline at positions 0 .. L_s - 1; a request's own
 * tokens are placed after them, context token j at absolute position L_s + j
 * (atyun.com article, section "RelayAttention": context positions offset by the
 * system prompt's length; linnk.ai summary, section "Deeper Inquiries").  The
 * embedding is rotary (RoPE), rotate-half form: for i < d/2 the pair
 * (x[i], x[i + d/2]) is rotated by the angle p * base^(-2i/d), applied to queries and
 * keys, not values.
 */

/*
 * Builds the cos/sin table that relay_rope_append / relay_rope_system read:
 * cos_sin float32 [max_pos, head_dim], row p = cos(p f_i) for i < d/2, then
 * sin(p f_i), f_i = base^(-2i/d); angles reduced in fp64 on the device.  Caller
 * owns the buffer.  head_dim 64 or 128; max_pos >= 1; base > 0.
 */
int relay_rope_table(float* cos_sin, int32_t max_pos, int32_t head_dim, float base, void* stream);

/*
 * Appends a decode step's new tokens: for new token t of request b (rows
 * cu_q_lens[b] .. cu_q_lens[b+1]-1, or row b when cu_q_lens is NULL) at context
 * position p = c_b - n_b + t_local and absolute position sys_len + p:
 *   q_out[t, h]  = RoPE(q_new[t, h], sys_len + p)            h < H_q
 *   K page slot  = RoPE(k_new[t, hk], sys_len + p)           hk < H_kv
 *   V page slot  = v_new[t, hk]
 * at page block_tables[b][p / 16], slot p % 16 of ctx_k_pages [num_blocks, H_kv,
 * d/G, 16, G] / ctx_v_pages [num_blocks, H_kv, d, 16].  q_new / q_out [T_q, H_q, d] and
 * k_new / v_new [T_q, H_kv, d] are in_dtype (q_out may alias q_new).  ctx_lens
 * already include the new tokens.  cos_sin: relay_rope_table's table, max_pos rows;
 * a row whose position is >= max_pos, or whose page id is out of range, is not
 * written.  Then relay_attn_decode(q_out, ...) runs the relay path.
 */
int relay_rope_append(const relay_dims* dims, int32_t sys_len, const void* q_new,
                      const void* k_new, const void* v_new, const float* cos_sin,
                      int32_t max_pos, const int32_t* block_tables, const int32_t* ctx_lens,
                      const int32_t* cu_q_lens, void* q_out, void* ctx_k_pages,
                      void* ctx_v_pages, void* stream);

/*
 * The offline prefill's position embedding of the system keys: sys_k [H_kv,
 * ceil(L_s/16), d/G, 16, G] (in_dtype) rotated in place at positions 0 .. sys_len - 1
 * (padding keys untouched).  sys_len <= max_pos.
 */
int relay_rope_system(int32_t num_kv_heads, int32_t head_dim, int32_t sys_len, int32_t in_dtype,
                      void* sys_k, const float* cos_sin, int32_t max_pos, void* stream);

/*
 * The offline prefill's cache fill (the system K/V are filled before serving:
 * atyun.com article, section "RelayAttention"): the system prompt's keys and values
 * as a projection produces them, token-major k_raw / v_raw [L_s, H_kv, d] (in_dtype),
 * written into the system cache: sys_k [H_kv, ceil(L_s/16), d/G, 16, G] with RoPE
 * at positions 0 .. L_s - 1 and sys_v [H_kv, ceil(L_s/16), d, 16] (the tail tiles'
 * padding keys set to 0 in both).  cos_sin: relay_rope_table's table, sys_len <= max_pos.
 */
int relay_system_fill(int32_t num_kv_heads, int32_t head_dim, int32_t sys_len, int32_t in_dtype,
                      const void* k_raw, const void* v_raw, const float* cos_sin, int32_t max_pos,
                      void* sys_k, void* sys_v, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RELAY_ATTN_H */
