// C-ABI host layer of librelay_attn.so: argument checks, the work plan, workspace
// carving and the kernel launches.  Declarations and the contract of every entry
// point are in include/relay_attn.h.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/relay_attn.h"
#include "relay_internal.hpp"

namespace {

using relay::FuseArgs;
using relay::SysArgs;
using relay::SysConfig;

thread_local char g_err[512];

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

constexpr int kNumCUs = 256;  // MI355X
constexpr float kLog2e = 1.4426950408889634f;

int env_int(const char* name, int dflt) {
  const char* v = getenv(name);
  if (!v || !*v) return dflt;
  char* end = nullptr;
  long x = strtol(v, &end, 10);
  return (end && *end == 0 && x > 0 && x < (1L << 30)) ? (int)x : dflt;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// (head, chunk) groups from which system units take two row tiles (M <= 32).
constexpr long long kSysTwoTileGroups = 384;
int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }
int round_up32(long long x) { return (int)(((x + 31) / 32) * 32); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

struct Plan {
  int sys_mode = 0;  // 0: no system step, 1: streaming units, 2: matrix-core kernel
  int sys_mfma = 0;  // sys_mode 2: 1 = sys_attn_mfma (bf16, d = 128), 0 = sys_attn_tiled
  int causal = 0;    // the offline prefill's causal system attention (sys_attn_mfma only)
  SysConfig sc{};
  int sys_chunks = 0, sys_chunk_len = 0, sys_row_blocks = 0, sys_wgs = 0, xcd_remap = 0, sys_rt = 1;
  int sys_steps_per_head = 0, sys_total_steps = 0, sys_parts = 0;  // sys_attn_mfma
  int ctx_rt = 1, ctx_split_len = 0, ctx_max_splits = 0, ctx_row_blocks = 0, ctx_wgs = 0;
  int fuse_wgs = 0, launches = 0;
  size_t off_sys_o = 0, off_sys_lse = 0, off_ctx_o = 0, off_ctx_lse = 0, ws_bytes = 0;
};

int check_dims(const relay_dims* d, int32_t sys_len) {
  if (!d) return fail(RELAY_ERR_INVALID, "dims is NULL");
  if (d->batch < 1) return fail(RELAY_ERR_INVALID, "batch must be >= 1 (got %d)", d->batch);
  if (d->num_kv_heads < 1 || d->num_q_heads < 1 || d->num_q_heads % d->num_kv_heads)
    return fail(RELAY_ERR_INVALID, "num_q_heads (%d) must be a positive multiple of num_kv_heads (%d)",
                d->num_q_heads, d->num_kv_heads);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(RELAY_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", d->head_dim);
  if (d->block_size != 16)
    return fail(RELAY_ERR_UNSUPPORTED, "block_size %d unsupported (16)", d->block_size);
  if ((d->in_dtype != RELAY_F32 && d->in_dtype != RELAY_BF16) ||
      (d->out_dtype != RELAY_F32 && d->out_dtype != RELAY_BF16))
    return fail(RELAY_ERR_UNSUPPORTED, "dtype unsupported (in %d, out %d)", d->in_dtype, d->out_dtype);
  if (d->total_q < 1 || d->max_q_len < 1 || d->max_q_len > d->total_q)
    return fail(RELAY_ERR_INVALID, "total_q (%d) and max_q_len (%d) must satisfy 1 <= max_q_len <= total_q",
                d->total_q, d->max_q_len);
  if (d->max_ctx_len < 1 || d->max_ctx_len < d->max_q_len)
    return fail(RELAY_ERR_INVALID, "max_ctx_len (%d) must be >= max(1, max_q_len)", d->max_ctx_len);
  if (d->max_blocks_per_seq < ceil_div(d->max_ctx_len, 16))
    return fail(RELAY_ERR_INVALID, "max_blocks_per_seq (%d) < ceil(max_ctx_len/16) (%d)",
                d->max_blocks_per_seq, ceil_div(d->max_ctx_len, 16));
  if (d->num_blocks < 1) return fail(RELAY_ERR_INVALID, "num_blocks must be >= 1");
  if (!(isfinite(d->scale))) return fail(RELAY_ERR_INVALID, "scale must be finite");
  if (sys_len < 0) return fail(RELAY_ERR_INVALID, "sys_len must be >= 0 (got %d)", sys_len);
  const long long rows = (long long)d->total_q * d->num_q_heads;
  if (rows * d->head_dim > (1LL << 40) || (long long)sys_len * d->num_kv_heads > (1LL << 36) || (long long)d->total_q * (d->num_q_heads / d->num_kv_heads) > (1 << 30))
    return fail(RELAY_ERR_INVALID, "problem too large");
  return RELAY_OK;
}

int clamp_int(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

void make_plan(const relay_dims* d, int32_t sys_len, Plan* p, bool causal = false) {
  p->causal = causal ? 1 : 0;
  const int g = d->num_q_heads / d->num_kv_heads;
  const long long rows = (long long)d->total_q * d->num_q_heads;
  // ---- system step
  const int M = d->total_q * g;
  if (sys_len > 0) {
    if (M <= relay::kUnitMaxRows) {
      p->sys_mode = 1;
      const int chunk = round_up32(clamp_int(env_int("RELAY_SYS_CHUNK", 512), 32, 1 << 20));
      p->sys_chunk_len = chunk;
      p->sys_chunks = ceil_div(sys_len, chunk);
      const long long groups = (long long)d->num_kv_heads * p->sys_chunks;
      // Both 16-row tiles of M <= 32 rows in one unit (the chunk is read once, not once
      // per tile) when there are enough (head, chunk) groups to keep every workgroup
      // busy with such units; with few groups the smaller one-tile units balance better.
      // Measured crossover (Llama-30B shape, batch 32): 208 groups even, 416 and more
      // faster, 128 slower.
      p->sys_rt = (M > 16 && M <= 32 && groups >= kSysTwoTileGroups) ? 2 : 1;
      const int forced_rt = env_int("RELAY_SYS_ROW_TILES", 0);  // tuning: 1 or 2 tiles per unit
      if (forced_rt == 1 || forced_rt == 2) p->sys_rt = forced_rt;
      if (env_int("RELAY_KEY_LANES", 4) != 4) p->sys_rt = 1;  // two-tile units need four key lanes
      p->sys_row_blocks = ceil_div(M, 16 * p->sys_rt);
      p->sys_wgs = (int)(8LL * p->sys_row_blocks * ((groups + 7) / 8));
    } else if (d->in_dtype == RELAY_BF16 && d->head_dim == 128) {
      p->sys_mode = 2;
      p->sys_mfma = 1;
      p->sys_row_blocks = ceil_div(M, relay::kSysMfmaRows);
      // the 64-key steps of all heads, cut into `parts` equal runs so the row blocks
      // times the parts fill the resident workgroup slots once
      p->sys_steps_per_head = ceil_div(sys_len, relay::kSysMfmaStep);
      const long long S = (long long)p->sys_steps_per_head * d->num_kv_heads;
      p->sys_total_steps = (int)S;
      long long parts = relay::kSysMfmaSlots / p->sys_row_blocks;
      // causal: a row block's work grows with its tokens, so the runs are cut finer
      // and the workgroups of early row blocks, which finish first, free their slots
      if (causal) parts *= relay::kSysCausalRunsPerSlot;
      const int forced = env_int("RELAY_SYS_PARTS", 0);
      if (forced > 0) parts = forced;
      if (parts < 1) parts = 1;
      if (parts > S) parts = S;
      p->sys_parts = (int)parts;
      // slots: the most parts any one head is spread over
      int slots = 1;
      for (int h = 0; h < d->num_kv_heads; ++h) {
        const long long x0 = (long long)h * p->sys_steps_per_head;
        const long long x1 = x0 + p->sys_steps_per_head - 1;
        const int n = relay::lean_part_of(x1, (int)S, (int)parts) - relay::lean_part_of(x0, (int)S, (int)parts) + 1;
        if (n > slots) slots = n;
      }
      p->sys_chunks = slots;
      p->sys_chunk_len = (int)(((S + parts - 1) / parts) * relay::kSysMfmaStep);  // keys per part
      const long long wgs = (long long)p->sys_row_blocks * parts;
      p->sys_wgs = (int)((wgs + 7) / 8 * 8);
      p->xcd_remap = 1;
    } else {
      p->sys_mode = 2;
      p->sc = relay::sys_config(M);
      p->sys_row_blocks = ceil_div(M, p->sc.wr * p->sc.rt * 16);
      const int target = env_int("RELAY_SYS_TARGET_WGS", 2 * kNumCUs);
      int chunk = env_int("RELAY_SYS_CHUNK", 0);
      if (chunk <= 0) {
        const long long per = (long long)sys_len * d->num_kv_heads * p->sys_row_blocks / target;
        chunk = round_up32(per < 1 ? 1 : per);
        if (chunk < 32 * p->sc.wk) chunk = 32 * p->sc.wk;
      }
      p->sys_chunk_len = round_up32(chunk);
      p->sys_chunks = ceil_div(sys_len, p->sys_chunk_len);
      p->sys_wgs = p->sys_row_blocks * p->sys_chunks * d->num_kv_heads;
      p->xcd_remap = (p->sys_row_blocks > 1 && p->sys_wgs % 8 == 0) ? 1 : 0;
    }
  }
  // ---- context step
  const int R = d->max_q_len * g;
  p->ctx_rt = relay::ctx_rt_for(R);
  p->ctx_row_blocks = ceil_div(R, 16 * p->ctx_rt);
  // Context split: 512 keys while every context fits one split; 768 for longer contexts,
  // where 512 left many empty trailing splits (each a unit that only marks its rows
  // empty) and 768 measured 3-6% faster on the context step (Llama-3-8B GQA shape,
  // long-prompt multi-token shape).
  const int split = env_int("RELAY_CTX_SPLIT", d->max_ctx_len > 512 ? 768 : 512);
  p->ctx_split_len = round_up32(clamp_int(split, 32, 1024));
  p->ctx_max_splits = ceil_div(d->max_ctx_len, p->ctx_split_len);
  const long long cgroups = (long long)p->ctx_max_splits * d->num_kv_heads * d->batch;
  p->ctx_wgs = (int)(8LL * p->ctx_row_blocks * ((cgroups + 7) / 8));
  // ---- fusion
  p->fuse_wgs = ceil_div(rows, relay::fuse_rows_per_wg(d->head_dim, rows));
  p->launches = (p->sys_mode == 2 ? 3 : 2);
  // ---- workspace
  size_t off = 0;
  p->off_sys_o = off;
  off += align256((size_t)p->sys_chunks * rows * d->head_dim * sizeof(float));
  p->off_sys_lse = off;
  off += align256((size_t)p->sys_chunks * rows * sizeof(float));
  p->off_ctx_o = off;
  off += align256((size_t)p->ctx_max_splits * rows * d->head_dim * sizeof(float));
  p->off_ctx_lse = off;
  off += align256((size_t)p->ctx_max_splits * rows * sizeof(float));
  p->ws_bytes = off;
}

int grid_ok(long long n) { return n > 0 && n < (1LL << 31); }

int hip_fail(hipError_t e, const char* what) {
  return fail(RELAY_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int launch_sys_tiled(const relay_dims* d, const Plan& p, const void* q, const void* sys_k,
                     const void* sys_v, int32_t sys_len, char* ws, hipStream_t s) {
  if (!grid_ok(p.sys_wgs)) return fail(RELAY_ERR_INVALID, "system grid too large");
  SysArgs a;
  a.q = q;
  a.sys_k = sys_k;
  a.sys_v = sys_v;
  a.o_part = reinterpret_cast<float*>(ws + p.off_sys_o);
  a.lse_part = reinterpret_cast<float*>(ws + p.off_sys_lse);
  a.sys_len = sys_len;
  a.total_q = d->total_q;
  a.num_q_heads = d->num_q_heads;
  a.group = d->num_q_heads / d->num_kv_heads;
  a.chunk_len = p.sys_chunk_len;
  a.n_chunks = p.sys_chunks;
  a.row_blocks = p.sys_row_blocks;
  a.xcd_remap = p.xcd_remap;
  a.scale_log2 = d->scale * kLog2e;
  a.steps_per_head = p.sys_steps_per_head;
  a.total_steps = p.sys_total_steps;
  a.parts = p.sys_parts;
  a.causal = p.causal;
  hipError_t e = p.sys_mfma ? relay::launch_sys_attn_mfma(a, p.sys_wgs, s)
                            : relay::launch_sys_attn_tiled(a, p.sc, d->in_dtype, d->head_dim, p.sys_wgs, s);
  return e == hipSuccess ? RELAY_OK : hip_fail(e, "system attention launch");
}

// Launches single-wave units: what = relay::kUnitsSys / kUnitsCtx / kUnitsBoth.
int launch_units(const relay_dims* d, const Plan& p, int what, const void* q, const void* sys_k,
                 const void* sys_v, int32_t sys_len, const void* ck, const void* cv, const int32_t* bt,
                 const int32_t* cl, const int32_t* cu, char* ws, hipStream_t s) {
  relay::UnitArgs a{};
  a.q = q;
  a.total_q = d->total_q;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.group = d->num_q_heads / d->num_kv_heads;
  a.scale_log2 = d->scale * kLog2e;
  a.key_lanes = env_int("RELAY_KEY_LANES", 4);
  a.grid = env_int("RELAY_GRID", 0);

  if (what & relay::kUnitsSys) {
    a.sys_k = sys_k;
    a.sys_v = sys_v;
    a.sys_o = reinterpret_cast<float*>(ws + p.off_sys_o);
    a.sys_lse = reinterpret_cast<float*>(ws + p.off_sys_lse);
    a.sys_len = sys_len;
    a.sys_chunk_len = p.sys_chunk_len;
    a.sys_chunks = p.sys_chunks;
    a.sys_row_tiles = p.sys_row_blocks;
    a.sys_rt = p.sys_rt;
    a.n_sys_units = p.sys_wgs;
  }
  if (what & relay::kUnitsCtx) {
    a.ctx_k = ck;
    a.ctx_v = cv;
    a.block_tables = bt;
    a.ctx_lens = cl;
    a.cu_q_lens = cu;
    a.ctx_o = reinterpret_cast<float*>(ws + p.off_ctx_o);
    a.ctx_lse = reinterpret_cast<float*>(ws + p.off_ctx_lse);
    a.batch = d->batch;
    a.num_blocks = d->num_blocks;
    a.max_blocks_per_seq = d->max_blocks_per_seq;
    a.max_ctx_len = d->max_ctx_len;
    a.ctx_split_len = p.ctx_split_len;
    a.ctx_max_splits = p.ctx_max_splits;
    a.ctx_row_blocks = p.ctx_row_blocks;
    a.n_ctx_units = p.ctx_wgs;
  }
  if (!grid_ok((long long)a.n_sys_units + a.n_ctx_units)) return fail(RELAY_ERR_INVALID, "grid too large");
  hipError_t e = relay::launch_attn_units(a, p.ctx_rt, what, d->in_dtype, d->head_dim, s);
  return e == hipSuccess ? RELAY_OK : hip_fail(e, "attention units launch");
}

int launch_fuse(FuseArgs& a, int head_dim, hipStream_t s) {
  const long long per = relay::fuse_rows_per_wg(head_dim, a.n_rows);
  const long long nwg = (a.n_rows + per - 1) / per;
  if (!grid_ok(nwg)) return fail(RELAY_ERR_INVALID, "fusion grid too large");
  hipError_t e = relay::launch_relay_fuse(a, head_dim, (int)nwg, s);
  return e == hipSuccess ? RELAY_OK : hip_fail(e, "relay_fuse launch");
}

int check_ws(const Plan& p, void* ws, size_t bytes) {
  if (p.ws_bytes == 0) return RELAY_OK;
  if (!ws) return fail(RELAY_ERR_INVALID, "workspace is NULL");
  if (((uintptr_t)ws & 255u) != 0) return fail(RELAY_ERR_INVALID, "workspace must be 256-byte aligned");
  if (bytes < p.ws_bytes)
    return fail(RELAY_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", bytes, p.ws_bytes);
  return RELAY_OK;
}

// Records events[i] (a hipEvent_t, may be NULL) on the stream; no-op without events.
int record(void* const* events, int i, hipStream_t s) {
  if (!events || !events[i]) return RELAY_OK;
  hipError_t e = hipEventRecord(static_cast<hipEvent_t>(events[i]), s);
  return e == hipSuccess ? RELAY_OK : hip_fail(e, "hipEventRecord");
}

int check_q_layout(const relay_dims* d, const int32_t* cu) {
  if (!cu && (d->total_q != d->batch || d->max_q_len != 1))
    return fail(RELAY_ERR_INVALID, "cu_q_lens is NULL: total_q must equal batch and max_q_len must be 1");
  return RELAY_OK;
}

}  // namespace

extern "C" {

int relay_abi_version(void) { return RELAY_ATTN_ABI_VERSION; }

const char* relay_strerror(int code) {
  switch (code) {
    case RELAY_OK: return "ok";
    case RELAY_ERR_INVALID: return "invalid argument";
    case RELAY_ERR_UNSUPPORTED: return "unsupported configuration";
    case RELAY_ERR_WORKSPACE: return "workspace too small";
    case RELAY_ERR_HIP: return "HIP error";
    case RELAY_ERR_DATA: return "inconsistent data";
    default: return "unknown error";
  }
}

const char* relay_last_error(void) { return g_err; }

size_t relay_workspace_size(const relay_dims* dims, int32_t sys_len) {
  if (check_dims(dims, sys_len) != RELAY_OK) return 0;
  Plan p;
  make_plan(dims, sys_len, &p);
  return p.ws_bytes;
}

int relay_get_plan(const relay_dims* dims, int32_t sys_len, relay_plan* out) {
  int rc = check_dims(dims, sys_len);
  if (rc != RELAY_OK) return rc;
  if (!out) return fail(RELAY_ERR_INVALID, "plan is NULL");
  Plan p;
  make_plan(dims, sys_len, &p);
  out->sys_chunks = p.sys_chunks;
  out->sys_chunk_len = p.sys_chunk_len;
  out->sys_row_blocks = p.sys_row_blocks;
  out->sys_wgs = p.sys_wgs;
  out->ctx_split_len = p.ctx_split_len;
  out->ctx_max_splits = p.ctx_max_splits;
  out->ctx_row_blocks = p.ctx_row_blocks;
  out->ctx_wgs = p.ctx_wgs;
  out->fuse_wgs = p.fuse_wgs;
  out->sys_mode = p.sys_mode;
  out->launches = p.launches;
  return RELAY_OK;
}

static int decode_impl(const relay_dims* dims, const void* q, const void* sys_k, const void* sys_v,
                       int32_t sys_len, const void* ctx_k_pages, const void* ctx_v_pages,
                       const int32_t* block_tables, const int32_t* ctx_lens,
                       const int32_t* cu_q_lens, void* out, void* workspace,
                       size_t workspace_bytes, void* stream, void* const* events) {
  int rc = check_dims(dims, sys_len);
  if (rc != RELAY_OK) return rc;
  if ((rc = check_q_layout(dims, cu_q_lens)) != RELAY_OK) return rc;
  if (!q || !ctx_k_pages || !ctx_v_pages || !block_tables || !ctx_lens || !out)
    return fail(RELAY_ERR_INVALID, "NULL array argument");
  if (sys_len > 0 && (!sys_k || !sys_v)) return fail(RELAY_ERR_INVALID, "sys_k/sys_v NULL with sys_len > 0");
  if (!aligned16(q) || !aligned16(sys_k) || !aligned16(sys_v) || !aligned16(ctx_k_pages) ||
      !aligned16(ctx_v_pages) || !aligned16(out))
    return fail(RELAY_ERR_INVALID, "arrays must be 16-byte aligned");
  Plan p;
  make_plan(dims, sys_len, &p);
  if ((rc = check_ws(p, workspace, workspace_bytes)) != RELAY_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((rc = record(events, 0, s)) != RELAY_OK) return rc;
  int units = relay::kUnitsCtx;
  if (p.sys_mode == 2) {
    if ((rc = launch_sys_tiled(dims, p, q, sys_k, sys_v, sys_len, ws, s)) != RELAY_OK) return rc;
  } else if (p.sys_mode == 1) {
    units = relay::kUnitsBoth;  // both steps in one launch
  }
  if ((rc = record(events, 1, s)) != RELAY_OK) return rc;
  if ((rc = launch_units(dims, p, units, q, sys_k, sys_v, sys_len, ctx_k_pages, ctx_v_pages, block_tables,
                         ctx_lens, cu_q_lens, ws, s)) != RELAY_OK)
    return rc;
  if ((rc = record(events, 2, s)) != RELAY_OK) return rc;
  FuseArgs f{};
  f.a_o = reinterpret_cast<const float*>(ws + p.off_sys_o);
  f.a_lse = reinterpret_cast<const float*>(ws + p.off_sys_lse);
  f.a_count = p.sys_chunks;
  f.a_sparse = p.sys_mode == 2;
  f.b_o = reinterpret_cast<const float*>(ws + p.off_ctx_o);
  f.b_lse = reinterpret_cast<const float*>(ws + p.off_ctx_lse);
  f.b_count = p.ctx_max_splits;
  f.out = out;
  f.lse_out = nullptr;
  f.n_rows = (long long)dims->total_q * dims->num_q_heads;
  f.out_bf16 = dims->out_dtype == RELAY_BF16;
  if ((rc = launch_fuse(f, dims->head_dim, s)) != RELAY_OK) return rc;
  return record(events, 3, s);
}

int relay_attn_decode(const relay_dims* dims, const void* q, const void* sys_k, const void* sys_v,
                      int32_t sys_len, const void* ctx_k_pages, const void* ctx_v_pages,
                      const int32_t* block_tables, const int32_t* ctx_lens,
                      const int32_t* cu_q_lens, void* out, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return decode_impl(dims, q, sys_k, sys_v, sys_len, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens,
                     cu_q_lens, out, workspace, workspace_bytes, stream, nullptr);
}

int relay_attn_decode_timed(const relay_dims* dims, const void* q, const void* sys_k,
                            const void* sys_v, int32_t sys_len, const void* ctx_k_pages,
                            const void* ctx_v_pages, const int32_t* block_tables,
                            const int32_t* ctx_lens, const int32_t* cu_q_lens, void* out,
                            void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events) {
  if (!events) return fail(RELAY_ERR_INVALID, "events is NULL");
  return decode_impl(dims, q, sys_k, sys_v, sys_len, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens,
                     cu_q_lens, out, workspace, workspace_bytes, stream, events);
}



int relay_sys_attn(const relay_dims* dims, const void* q, const void* sys_k, const void* sys_v,
                   int32_t sys_len, float* o_sys, float* lse_sys, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims, sys_len);
  if (rc != RELAY_OK) return rc;
  if (!q || !o_sys || !lse_sys) return fail(RELAY_ERR_INVALID, "NULL array argument");
  if (sys_len > 0 && (!sys_k || !sys_v)) return fail(RELAY_ERR_INVALID, "sys_k/sys_v NULL with sys_len > 0");
  if (!aligned16(q) || !aligned16(sys_k) || !aligned16(sys_v) || !aligned16(o_sys))
    return fail(RELAY_ERR_INVALID, "arrays must be 16-byte aligned");
  Plan p;
  make_plan(dims, sys_len, &p);
  if ((rc = check_ws(p, workspace, workspace_bytes)) != RELAY_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (p.sys_mode == 2 && (rc = launch_sys_tiled(dims, p, q, sys_k, sys_v, sys_len, ws, s)) != RELAY_OK) return rc;
  if (p.sys_mode == 1 && (rc = launch_units(dims, p, relay::kUnitsSys, q, sys_k, sys_v, sys_len, nullptr, nullptr,
                                            nullptr, nullptr, nullptr, ws, s)) != RELAY_OK)
    return rc;
  FuseArgs f{};
  f.a_o = reinterpret_cast<const float*>(ws + p.off_sys_o);
  f.a_lse = reinterpret_cast<const float*>(ws + p.off_sys_lse);
  f.a_count = p.sys_chunks;
  f.a_sparse = p.sys_mode == 2;
  f.out = o_sys;
  f.lse_out = lse_sys;
  f.n_rows = (long long)dims->total_q * dims->num_q_heads;
  return launch_fuse(f, dims->head_dim, s);
}

size_t relay_prefill_workspace_size(const relay_dims* dims, int32_t sys_len) {
  if (check_dims(dims, sys_len) != RELAY_OK) return 0;
  Plan p;
  make_plan(dims, sys_len, &p, true);
  return p.ws_bytes;
}

int relay_prefill_attn(const relay_dims* dims, const void* q, const void* sys_k, const void* sys_v,
                       int32_t sys_len, void* out, int32_t out_dtype, float* lse_out, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims, sys_len);
  if (rc != RELAY_OK) return rc;
  if (!q || !sys_k || !sys_v || !out) return fail(RELAY_ERR_INVALID, "NULL array argument");
  if (sys_len < 1) return fail(RELAY_ERR_INVALID, "the prefill needs sys_len >= 1");
  if (!(dims->scale > 0.f)) return fail(RELAY_ERR_INVALID, "the prefill needs scale > 0");
  if (out_dtype != RELAY_F32 && out_dtype != RELAY_BF16) return fail(RELAY_ERR_UNSUPPORTED, "out_dtype %d", out_dtype);
  if (!aligned16(q) || !aligned16(sys_k) || !aligned16(sys_v) || !aligned16(out))
    return fail(RELAY_ERR_INVALID, "arrays must be 16-byte aligned");
  Plan p;
  make_plan(dims, sys_len, &p, true);
  if (!p.sys_mfma)
    return fail(RELAY_ERR_UNSUPPORTED, "the prefill runs on the matrix-core system kernel: bf16, head_dim 128 and "
                                       "more than %d query rows per KV head", relay::kUnitMaxRows);
  if ((rc = check_ws(p, workspace, workspace_bytes)) != RELAY_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((rc = launch_sys_tiled(dims, p, q, sys_k, sys_v, sys_len, ws, s)) != RELAY_OK) return rc;
  FuseArgs f{};
  f.a_o = reinterpret_cast<const float*>(ws + p.off_sys_o);
  f.a_lse = reinterpret_cast<const float*>(ws + p.off_sys_lse);
  f.a_count = p.sys_chunks;
  f.a_sparse = 1;  // causal runs past a row block's tokens are empty
  f.out = out;
  f.out_bf16 = out_dtype == RELAY_BF16;
  f.lse_out = lse_out;
  f.n_rows = (long long)dims->total_q * dims->num_q_heads;
  return launch_fuse(f, dims->head_dim, s);
}

int relay_ctx_attn(const relay_dims* dims, const void* q, const void* ctx_k_pages,
                   const void* ctx_v_pages, const int32_t* block_tables, const int32_t* ctx_lens,
                   const int32_t* cu_q_lens, float* o_ctx, float* lse_ctx, void* workspace,
                   size_t workspace_bytes, void* stream) {
  int rc = check_dims(dims, 0);
  if (rc != RELAY_OK) return rc;
  if ((rc = check_q_layout(dims, cu_q_lens)) != RELAY_OK) return rc;
  if (!q || !ctx_k_pages || !ctx_v_pages || !block_tables || !ctx_lens || !o_ctx || !lse_ctx)
    return fail(RELAY_ERR_INVALID, "NULL array argument");
  if (!aligned16(q) || !aligned16(ctx_k_pages) || !aligned16(ctx_v_pages) || !aligned16(o_ctx))
    return fail(RELAY_ERR_INVALID, "arrays must be 16-byte aligned");
  Plan p;
  make_plan(dims, 0, &p);
  if ((rc = check_ws(p, workspace, workspace_bytes)) != RELAY_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((rc = launch_units(dims, p, relay::kUnitsCtx, q, nullptr, nullptr, 0, ctx_k_pages, ctx_v_pages,
                         block_tables, ctx_lens, cu_q_lens, ws, s)) != RELAY_OK)
    return rc;
  FuseArgs f{};
  f.b_o = reinterpret_cast<const float*>(ws + p.off_ctx_o);
  f.b_lse = reinterpret_cast<const float*>(ws + p.off_ctx_lse);
  f.b_count = p.ctx_max_splits;
  f.out = o_ctx;
  f.lse_out = lse_ctx;
  f.n_rows = (long long)dims->total_q * dims->num_q_heads;
  return launch_fuse(f, dims->head_dim, s);
}

int relay_fuse(int64_t n_rows, int32_t head_dim, const float* o_sys, const float* lse_sys,
               const float* o_ctx, const float* lse_ctx, void* out, int32_t out_dtype,
               float* lse_out, void* stream) {
  if (n_rows < 0) return fail(RELAY_ERR_INVALID, "n_rows must be >= 0");
  if (head_dim != 64 && head_dim != 128)
    return fail(RELAY_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", head_dim);
  if (out_dtype != RELAY_F32 && out_dtype != RELAY_BF16)
    return fail(RELAY_ERR_UNSUPPORTED, "out_dtype %d unsupported", out_dtype);
  if (n_rows == 0) return RELAY_OK;
  if (!o_sys || !lse_sys || !o_ctx || !lse_ctx || !out) return fail(RELAY_ERR_INVALID, "NULL array argument");
  if (!aligned16(o_sys) || !aligned16(o_ctx) || !aligned16(out))
    return fail(RELAY_ERR_INVALID, "arrays must be 16-byte aligned");
  FuseArgs f{};
  f.a_o = o_sys;
  f.a_lse = lse_sys;
  f.a_count = 1;
  f.b_o = o_ctx;
  f.b_lse = lse_ctx;
  f.b_count = 1;
  f.out = out;
  f.lse_out = lse_out;
  f.n_rows = n_rows;
  f.out_bf16 = out_dtype == RELAY_BF16;
  return launch_fuse(f, head_dim, static_cast<hipStream_t>(stream));
}

int relay_validate(const relay_dims* dims, const int32_t* h_block_tables, const int32_t* h_ctx_lens,
                   const int32_t* h_cu_q_lens, int32_t sys_len) {
  int rc = check_dims(dims, sys_len);
  if (rc != RELAY_OK) return rc;
  if ((rc = check_q_layout(dims, h_cu_q_lens)) != RELAY_OK) return rc;
  if (!h_block_tables || !h_ctx_lens) return fail(RELAY_ERR_INVALID, "NULL host array");
  if (h_cu_q_lens && h_cu_q_lens[0] != 0) return fail(RELAY_ERR_DATA, "cu_q_lens[0] must be 0");
  if (h_cu_q_lens && h_cu_q_lens[dims->batch] != dims->total_q)
    return fail(RELAY_ERR_DATA, "cu_q_lens[B] = %d != total_q = %d", h_cu_q_lens[dims->batch], dims->total_q);
  for (int b = 0; b < dims->batch; ++b) {
    const int nb = h_cu_q_lens ? h_cu_q_lens[b + 1] - h_cu_q_lens[b] : 1;
    const int c = h_ctx_lens[b];
    if (nb < 1 || nb > dims->max_q_len)
      return fail(RELAY_ERR_DATA, "request %d: n_b = %d outside [1, max_q_len = %d]", b, nb, dims->max_q_len);
    if (c < nb || c > dims->max_ctx_len)
      return fail(RELAY_ERR_DATA, "request %d: ctx_len = %d outside [n_b = %d, max_ctx_len = %d]", b, c, nb,
                  dims->max_ctx_len);
    const int pages = (c + 15) / 16;
    for (int i = 0; i < pages; ++i) {
      const int blk = h_block_tables[(size_t)b * dims->max_blocks_per_seq + i];
      if (blk < 0 || blk >= dims->num_blocks)
        return fail(RELAY_ERR_DATA, "request %d: block_tables[%d] = %d outside [0, %d)", b, i, blk,
                    dims->num_blocks);
    }
  }
  return RELAY_OK;
}

int relay_rope_table(float* cos_sin, int32_t max_pos, int32_t head_dim, float base, void* stream) {
  if (head_dim != 64 && head_dim != 128)
    return fail(RELAY_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", head_dim);
  if (max_pos < 1 || !(base > 0.f) || !isfinite(base)) return fail(RELAY_ERR_INVALID, "max_pos >= 1 and base > 0 required");
  if (!cos_sin) return fail(RELAY_ERR_INVALID, "cos_sin is NULL");
  hipError_t e = relay::launch_rope_table(cos_sin, max_pos, head_dim, (double)base, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RELAY_OK : hip_fail(e, "rope table launch");
}

int relay_rope_append(const relay_dims* dims, int32_t sys_len, const void* q_new, const void* k_new,
                      const void* v_new, const float* cos_sin, int32_t max_pos, const int32_t* block_tables,
                      const int32_t* ctx_lens, const int32_t* cu_q_lens, void* q_out, void* ctx_k_pages,
                      void* ctx_v_pages, void* stream) {
  int rc = check_dims(dims, sys_len);
  if (rc != RELAY_OK) return rc;
  if ((rc = check_q_layout(dims, cu_q_lens)) != RELAY_OK) return rc;
  if (!q_new || !k_new || !v_new || !cos_sin || !block_tables || !ctx_lens || !q_out || !ctx_k_pages || !ctx_v_pages)
    return fail(RELAY_ERR_INVALID, "NULL array argument");
  if (max_pos < 1) return fail(RELAY_ERR_INVALID, "max_pos must be >= 1");
  if (dims->max_q_len > 65535 || dims->num_q_heads + dims->num_kv_heads > 65535)
    return fail(RELAY_ERR_INVALID, "too many tokens per request or heads for one launch");
  relay::RopeArgs a{};
  a.q_new = q_new;
  a.k_new = k_new;
  a.v_new = v_new;
  a.cos_sin = cos_sin;
  a.block_tables = block_tables;
  a.ctx_lens = ctx_lens;
  a.cu_q_lens = cu_q_lens;
  a.q_out = q_out;
  a.ctx_k = ctx_k_pages;
  a.ctx_v = ctx_v_pages;
  a.batch = dims->batch;
  a.num_q_heads = dims->num_q_heads;
  a.num_kv_heads = dims->num_kv_heads;
  a.head_dim = dims->head_dim;
  a.total_q = dims->total_q;
  a.max_blocks_per_seq = dims->max_blocks_per_seq;
  a.num_blocks = dims->num_blocks;
  a.sys_len = sys_len;
  a.max_pos = max_pos;
  a.bf16 = dims->in_dtype == RELAY_BF16;
  hipError_t e = relay::launch_rope_append(a, dims->max_q_len, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RELAY_OK : hip_fail(e, "rope append launch");
}

int relay_rope_system(int32_t num_kv_heads, int32_t head_dim, int32_t sys_len, int32_t in_dtype, void* sys_k,
                      const float* cos_sin, int32_t max_pos, void* stream) {
  if (head_dim != 64 && head_dim != 128)
    return fail(RELAY_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", head_dim);
  if (in_dtype != RELAY_F32 && in_dtype != RELAY_BF16) return fail(RELAY_ERR_UNSUPPORTED, "dtype %d unsupported", in_dtype);
  if (num_kv_heads < 1 || num_kv_heads > 65535 || sys_len < 0 || sys_len > max_pos)
    return fail(RELAY_ERR_INVALID, "need 1 <= num_kv_heads <= 65535 and 0 <= sys_len <= max_pos");
  if (sys_len == 0) return RELAY_OK;
  if (!sys_k || !cos_sin) return fail(RELAY_ERR_INVALID, "NULL array argument");
  hipError_t e = relay::launch_rope_system(sys_k, cos_sin, sys_len, num_kv_heads, head_dim, in_dtype == RELAY_BF16,
                                           static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RELAY_OK : hip_fail(e, "rope system launch");
}

int relay_system_fill(int32_t num_kv_heads, int32_t head_dim, int32_t sys_len, int32_t in_dtype, const void* k_raw,
                      const void* v_raw, const float* cos_sin, int32_t max_pos, void* sys_k, void* sys_v,
                      void* stream) {
  if (head_dim != 64 && head_dim != 128)
    return fail(RELAY_ERR_UNSUPPORTED, "head_dim %d unsupported (64 or 128)", head_dim);
  if (in_dtype != RELAY_F32 && in_dtype != RELAY_BF16) return fail(RELAY_ERR_UNSUPPORTED, "dtype %d unsupported", in_dtype);
  if (num_kv_heads < 1 || num_kv_heads > 65535 || sys_len < 0 || sys_len > max_pos)
    return fail(RELAY_ERR_INVALID, "need 1 <= num_kv_heads <= 65535 and 0 <= sys_len <= max_pos");
  if (sys_len == 0) return RELAY_OK;
  if (!k_raw || !v_raw || !cos_sin || !sys_k || !sys_v) return fail(RELAY_ERR_INVALID, "NULL array argument");
  hipError_t e = relay::launch_system_fill(k_raw, v_raw, cos_sin, sys_k, sys_v, sys_len, num_kv_heads, head_dim,
                                           in_dtype == RELAY_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? RELAY_OK : hip_fail(e, "system fill launch");
}

}  // extern "C"
