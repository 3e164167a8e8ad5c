// C-ABI host layer of librelay_attn.so: argument checks, the work plan, workspace
// carving and the kernel launches.  Declarations and the contract of every entry
// point are in include/relay_attn.h.
#include <math.h>
#include <atomic>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/relay_attn.h"
#include "relay_internal.hpp"

namespace {

using relay::FuseArgs;
using relay::MergeArgs;
using relay::StreamArgs;
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

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxDevices = 64;
constexpr int kDefaultCUs = 256;  // MI355X, assumed when no device can be queried (planning on a host)

// Compute units of the current device, queried once per device (a process-wide cache).
int device_cus() {
  static std::atomic<int> cached[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return kDefaultCUs;
  }
  if (dev < kMaxDevices) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) {
    (void)hipGetLastError();
    n = kDefaultCUs;
  }
  if (dev < kMaxDevices) cached[dev].store(n, std::memory_order_relaxed);
  return n;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }
int round_up32(long long x) { return (int)(((x + 31) / 32) * 32); }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// What a call computes.
enum Need { kDecode, kSysOnly, kCtxOnly, kPrefill };

struct Plan {
  int sys_mode = 0;  // 0: none, 1: system streams in the streaming launch, 2: sys_attn_mfma, 3: sys_attn_tiled
  int causal = 0;    // the offline prefill's causal system attention (sys_attn_mfma only)
  // sys_mode 1
  int rts = 0, sys_steps = 0;
  // sys_mode 2 / 3
  SysConfig sc{};
  int sys_chunks = 0, sys_chunk_len = 0, sys_row_blocks = 0, sys_wgs = 0, xcd_remap = 0;
  int sys_steps_per_head = 0, sys_total_steps = 0, sys_parts = 0;
  int sys_pp = 0;  // sys_mode 2: the two-group kernel (kSysPPRows rows, one workgroup per CU)
  // streaming launches
  int rtc = 1, ctx_rb = 1, grid = 0, workers = 0, chunk_req = 0, n_chunks = 0;
  long long sys_slots = 0, ctx_slots_per_chunk = 0, ctx_slots = 0;
  int merge_wgs = 0, launches = 0;
  int ks = 0, kc = 0;  // the rows' own slots for system and context pieces
  size_t off_sys_o = 0, off_sys_lse = 0, off_sys_desc = 0, off_ctx_o = 0, off_ctx_lse = 0, off_rowdesc = 0;
  size_t off_row_o = 0, off_row_lse = 0;
  size_t ws_bytes = 0;
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
  if (rows * d->head_dim > (1LL << 40) || (long long)sys_len * d->num_kv_heads > (1LL << 36) ||
      (long long)d->total_q * (d->num_q_heads / d->num_kv_heads) > (1 << 30) ||
      (long long)d->max_q_len * (d->num_q_heads / d->num_kv_heads) > (1 << 20))
    return fail(RELAY_ERR_INVALID, "problem too large");
  return RELAY_OK;
}

int clamp_int(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

// The system kernel's plan (M > 64 stacked rows per KV head).
// slots: workgroups of the system kernel resident at once (the launch is cut to fill them).
void plan_system_kernel(const relay_dims* d, int32_t sys_len, int M, Plan* p, long long slots = relay::kSysMfmaSlots,
                        bool pp = false) {
  if (d->in_dtype == RELAY_BF16 && d->head_dim == 128) {
    p->sys_mode = 2;
    p->sys_pp = pp && !p->causal ? 1 : 0;
    p->sys_row_blocks = ceil_div(M, p->sys_pp ? relay::kSysPPRows : relay::kSysMfmaRows);
    // the 64-key steps of all heads, cut into `parts` equal runs so the row blocks
    // times the parts fill the resident workgroup slots once
    p->sys_steps_per_head = ceil_div(sys_len, relay::kSysMfmaStep);
    const long long S = (long long)p->sys_steps_per_head * d->num_kv_heads;
    p->sys_total_steps = (int)S;
    long long parts = slots / p->sys_row_blocks;
    // causal: a row block's work grows with its tokens, so the runs are cut finer
    // and the workgroups of early row blocks, which finish first, free their slots
    if (p->causal) parts *= relay::kSysCausalRunsPerSlot;
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
    p->sys_mode = 3;
    p->sc = relay::sys_config(M);
    p->sys_row_blocks = ceil_div(M, p->sc.wr * p->sc.rt * 16);
    const long long target = 2LL * device_cus();
    const long long per = (long long)sys_len * d->num_kv_heads * p->sys_row_blocks / target;
    int chunk = round_up32(per < 1 ? 1 : per);
    if (chunk < 32 * p->sc.wk) chunk = 32 * p->sc.wk;
    p->sys_chunk_len = chunk;
    p->sys_chunks = ceil_div(sys_len, p->sys_chunk_len);
    p->sys_wgs = p->sys_row_blocks * p->sys_chunks * d->num_kv_heads;
    p->xcd_remap = (p->sys_row_blocks > 1 && p->sys_wgs % 8 == 0) ? 1 : 0;
  }
}

// Whether the system step as a launch of its own takes the two-group kernel (256 rows
// per workgroup, one per CU, about 10 % faster per row at config-5 sizes) rather than
// the four-wave one (128 rows, two per CU): yes unless the 256-row blocks would hold more
// than 10 % more padding rows than the 128-row ones.
bool pp_fills(int M) {
  const long long pp = (long long)relay::kSysPPRows * ceil_div(M, relay::kSysPPRows);
  const long long mf = (long long)relay::kSysMfmaRows * ceil_div(M, relay::kSysMfmaRows);
  return 10 * pp <= 11 * mf;
}

// Whether the decode step's matrix-core system workgroups should share the CUs with the
// context streams (one of each per CU) rather than run first at two per CU: yes unless
// the system step's matrix-core time exceeds twice the context step's memory time
// (then the co-run's halved matrix-core occupancy costs more than the overlap saves).
// The context bytes are estimated from max_ctx_len (the lengths are device data): half
// of it per request.
bool corun_pays(const relay_dims* d, int32_t sys_len) {
  const double sys_flops = 4.0 * d->num_q_heads * d->head_dim * (double)d->total_q * sys_len;
  const double ctx_bytes = 4.0 * d->num_kv_heads * d->head_dim * (double)d->batch * (d->max_ctx_len / 2.0 + 16.0);
  const double t_sys = sys_flops / relay::kSysMfmaFlopsPerS, t_ctx = ctx_bytes / relay::kStreamBytesPerS;
  return t_ctx > 0.5 * t_sys;
}

// Fills *p for dims and sys_len (need: what the call computes).  Returns RELAY_OK or
// an error for sizes one streaming launch cannot index.
int make_plan(const relay_dims* d, int32_t sys_len, Plan* p, Need need = kDecode) {
  p->causal = need == kPrefill ? 1 : 0;
  const int g = d->num_q_heads / d->num_kv_heads;
  const long long rows = (long long)d->total_q * d->num_q_heads;
  const int D = d->head_dim;
  const int M = d->total_q * g;
  size_t off = 0;
  if (need == kPrefill) {  // the causal system kernel and the merge of its runs
    plan_system_kernel(d, sys_len, M, p);
    p->off_sys_o = off;
    off += align256((size_t)p->sys_chunks * rows * D * sizeof(float));
    p->off_sys_lse = off;
    off += align256((size_t)p->sys_chunks * rows * sizeof(float));
    p->ws_bytes = off;
    p->launches = 2;
    return RELAY_OK;
  }
  // ---- system step
  if (sys_len > 0) {
    if (M <= relay::kStreamSysMaxRows) {
      p->sys_mode = 1;
      const int tiles = ceil_div(M, 16);
      p->rts = tiles <= 2 ? tiles : 4;
      p->sys_steps = ceil_div(sys_len, 32);
    } else if (need == kDecode && d->in_dtype == RELAY_BF16 && D == 128 && corun_pays(d, sys_len)) {
      // the matrix-core system workgroups inside the streaming launch, one per CU beside
      // one context workgroup per CU
      plan_system_kernel(d, sys_len, M, p, device_cus());
      p->sys_mode = 4;
    } else if (need != kPrefill && d->in_dtype == RELAY_BF16 && D == 128 && pp_fills(M)) {
      // a launch of its own: the two-group kernel, one workgroup per CU
      plan_system_kernel(d, sys_len, M, p, device_cus(), true);
    } else {
      plan_system_kernel(d, sys_len, M, p);
    }
  }
  // ---- context streams: (request, KV head, row block), requests in groups of at most
  // chunk_req per streaming launch so that a launch's step count fits 31 bits
  const long long R = (long long)d->max_q_len * g;
  p->rtc = relay::ctx_rt_for((int)R);
  p->ctx_rb = ceil_div(R, 16 * p->rtc);
  // one or two workgroups per CU (what the launch's instantiation is built for); one
  // per CU beside the system workgroups
  p->grid = p->sys_mode == 4 ? device_cus()
                             : relay::stream_grid(device_cus(), d->in_dtype == RELAY_BF16 ? 2 : 4, D, p->rts, p->rtc);
  p->workers = p->grid * relay::kStreamWaves;

  const int cap = d->max_ctx_len < d->max_blocks_per_seq * 16 ? d->max_ctx_len : d->max_blocks_per_seq * 16;
  const long long per_req = (long long)ceil_div(cap, 32) * d->num_kv_heads * p->ctx_rb;
  long long chunk = relay::kStreamMaxRequests;
  if (chunk > d->batch) chunk = d->batch;
  if (chunk * per_req > 0x7fffffffLL - 1) chunk = (0x7fffffffLL - 1) / per_req;
  if (p->sys_mode == 1 && (long long)d->num_kv_heads * p->sys_steps + chunk * per_req > 0x7fffffffLL)
    chunk = (0x7fffffffLL - (long long)d->num_kv_heads * p->sys_steps) / per_req;
  if (chunk < 1) return fail(RELAY_ERR_UNSUPPORTED, "one request's context is too long for a streaming launch");
  p->chunk_req = (int)chunk;
  p->n_chunks = ceil_div(d->batch, chunk);
  p->ctx_slots_per_chunk = chunk * d->num_kv_heads * p->ctx_rb + p->workers;
  p->ctx_slots = p->ctx_slots_per_chunk * p->n_chunks;
  // ---- the rows' own piece slots, which the merge reads without looking up where they
  // are: for up to kRowSlotRows rows (the system streams' shapes), where the merge waits
  // on memory latency, not bandwidth (with more rows, slots read in vain cost more than
  // the round trip they save).  Context: the most waves the longest stream can fall
  // into, with at least (system steps + one step per stream) / waves steps per wave, at
  // most four.  System streams: the most workgroups one KV head's steps fall into, for a
  // step count estimated from half the longest context per stream (the lengths are
  // device data), plus one; exact when the launch holds no context streams.  Pieces past
  // a row's own slots take the stream slots, and the merge a second round trip for them.
  const long long max_steps = ceil_div(cap, 32) > 1 ? ceil_div(cap, 32) : 1;
  const long long Ts = p->sys_mode == 1 ? (long long)d->num_kv_heads * p->sys_steps : 0;
  const bool row_slots = p->sys_mode <= 1 && rows <= relay::kRowSlotRows;
  if (row_slots && need != kSysOnly) {
    long long per_wave = (Ts + chunk * d->num_kv_heads) / p->workers;
    if (per_wave < 1) per_wave = 1;
    long long kc = (max_steps - 1 + per_wave - 1) / per_wave + 1;
    if (kc > max_steps) kc = max_steps;
    p->kc = (int)(kc < 4 ? kc : 4);
  }
  if (row_slots && p->sys_mode == 1) {
    const long long ss = p->sys_steps;
    long long T = Ts;
    if (need != kSysOnly) T += chunk * d->num_kv_heads * p->ctx_rb * ((max_steps + 1) / 2);
    const long long W = T < p->workers ? T : p->workers;
    auto part = [&](long long x) { return ((x + 1) * W + T - 1) / T - 1; };
    long long most = 1;
    for (int h = 0; h < d->num_kv_heads; ++h) {
      const long long n = part(h * ss + ss - 1) / relay::kStreamWaves - part(h * ss) / relay::kStreamWaves + 1;
      if (n > most) most = n;
    }
    if (need != kSysOnly) ++most;
    p->ks = (int)(most < relay::kMaxRowSlots - p->kc ? most : relay::kMaxRowSlots - p->kc);
  }
  // system stream slots: the fixed ones (KV head h's piece k < ks at h ks + k), then one
  // per (KV head, workgroup) pair a later piece can fall on (h + w)
  if (p->sys_mode == 1) p->sys_slots = (long long)d->num_kv_heads * (p->ks + 1) + p->grid;
  // ---- merge
  p->merge_wgs = ceil_div(rows, relay::merge_threads(D, rows) / (D / 4));
  p->launches = (p->sys_mode == 2 || p->sys_mode == 3 ? 1 : 0) + p->n_chunks + 1;
  // ---- workspace (fp32 partials, 256-byte aligned regions)
  if (p->sys_mode == 1) {
    p->off_sys_o = off;
    off += align256((size_t)p->sys_slots * 16 * p->rts * D * sizeof(float));
    p->off_sys_lse = off;
    off += align256((size_t)p->sys_slots * 16 * p->rts * sizeof(float));
    p->off_sys_desc = off;
    off += align256((size_t)d->num_kv_heads * 2 * sizeof(int));
  } else if (p->sys_mode >= 2) {
    p->off_sys_o = off;
    off += align256((size_t)p->sys_chunks * rows * D * sizeof(float));
    p->off_sys_lse = off;
    off += align256((size_t)p->sys_chunks * rows * sizeof(float));
  }
  p->off_ctx_o = off;
  off += align256((size_t)p->ctx_slots * 16 * p->rtc * D * sizeof(float));
  p->off_ctx_lse = off;
  off += align256((size_t)p->ctx_slots * 16 * p->rtc * sizeof(float));
  p->off_rowdesc = off;
  off += align256((size_t)rows * 4 * sizeof(int));
  p->off_row_o = off;
  off += align256((size_t)rows * p->kc * D * sizeof(float));
  p->off_row_lse = off;
  off += align256((size_t)rows * p->kc * sizeof(float));
  p->ws_bytes = off;
  return RELAY_OK;
}

int grid_ok(long long n) { return n > 0 && n < (1LL << 31); }

int hip_fail(hipError_t e, const char* what) {
  return fail(RELAY_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// The system kernel (sys_mode 2 or 3): one launch writing per-row run partials.
SysArgs system_args(const relay_dims* d, const Plan& p, const void* q, const void* sys_k, const void* sys_v,
                    int32_t sys_len, char* ws) {
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
  return a;
}

// The system kernel as a launch of its own (sys_mode 2, 3; sys_mode 4's workgroups when
// the system step runs alone).
int launch_sys_kernel(const relay_dims* d, const Plan& p, const void* q, const void* sys_k, const void* sys_v,
                      int32_t sys_len, char* ws, hipStream_t s, const relay::LaunchTiming* tm = nullptr) {
  if (!grid_ok(p.sys_wgs)) return fail(RELAY_ERR_INVALID, "system grid too large");
  const SysArgs a = system_args(d, p, q, sys_k, sys_v, sys_len, ws);
  hipError_t e = p.sys_mode == 3 ? relay::launch_sys_attn_tiled(a, p.sc, d->in_dtype, d->head_dim, p.sys_wgs, s, tm)
                 : p.sys_pp      ? relay::launch_sys_attn_pp(a, p.sys_wgs, s, tm)
                                 : relay::launch_sys_attn_mfma(a, p.sys_wgs, s, tm);
  return e == hipSuccess ? RELAY_OK : hip_fail(e, "system attention launch");
}

// The streaming launches: the system streams (sys_mode 1, with_sys) and the context
// streams (with_ctx) of every request group; co_sys (sys_mode 4): the system kernel's
// workgroups go with the first request group's launch.
int launch_streams(const relay_dims* d, const Plan& p, bool with_sys, bool with_ctx, const void* q,
                   const void* sys_k, const void* sys_v, int32_t sys_len, const void* ck, const void* cv,
                   const int32_t* bt, const int32_t* cl, const int32_t* cu, char* ws, hipStream_t s,
                   const relay::LaunchTiming* tm = nullptr, const SysArgs* co_sys = nullptr) {
  const bool sys = with_sys && p.sys_mode == 1;
  if (!sys && !with_ctx) return RELAY_OK;
  StreamArgs a{};
  a.q = q;
  a.total_q = d->total_q;
  a.num_q_heads = d->num_q_heads;
  a.num_kv_heads = d->num_kv_heads;
  a.group = d->num_q_heads / d->num_kv_heads;
  a.scale_log2 = d->scale * kLog2e;
  a.M = d->total_q * a.group;
  a.n_workers = p.workers;
  if (sys) {
    a.sys_k = sys_k;
    a.sys_v = sys_v;
    a.sys_len = sys_len;
    a.sys_steps = p.sys_steps;
    a.sys_o = reinterpret_cast<float*>(ws + p.off_sys_o);
    a.sys_lse = reinterpret_cast<float*>(ws + p.off_sys_lse);
    a.sys_desc = reinterpret_cast<int*>(ws + p.off_sys_desc);
  }
  a.ctx_on = with_ctx ? 1 : 0;
  a.ctx_k = ck;
  a.ctx_v = cv;
  a.block_tables = bt;
  a.ctx_lens = cl;
  a.cu_q_lens = cu;
  a.batch = d->batch;
  a.num_blocks = d->num_blocks;
  a.max_blocks_per_seq = d->max_blocks_per_seq;
  a.max_ctx_len = d->max_ctx_len;
  a.ctx_rb = p.ctx_rb;
  a.ctx_o = reinterpret_cast<float*>(ws + p.off_ctx_o);
  a.ctx_lse = reinterpret_cast<float*>(ws + p.off_ctx_lse);
  a.ctx_rowdesc = reinterpret_cast<int*>(ws + p.off_rowdesc);
  a.row_o = reinterpret_cast<float*>(ws + p.off_row_o);
  a.row_lse = reinterpret_cast<float*>(ws + p.off_row_lse);
  a.ks = p.ks;
  a.kc = p.kc;
  const int launches = with_ctx ? p.n_chunks : 1;
  for (int c = 0; c < launches; ++c) {
    StreamArgs ac = a;
    ac.b_begin = c * p.chunk_req;
    ac.n_req = with_ctx ? (d->batch - ac.b_begin < p.chunk_req ? d->batch - ac.b_begin : p.chunk_req) : 0;
    ac.slot_base = (long long)c * p.ctx_slots_per_chunk;
    if (c > 0) ac.sys_steps = 0;  // the system streams go with the first request group
    const int rts = ac.sys_steps > 0 ? p.rts : 0;
    // timing: the first launch's start and the last one's end
    const relay::LaunchTiming tc{tm && c == 0 ? tm->start : nullptr, tm && c == launches - 1 ? tm->stop : nullptr};
    hipError_t e;
    if (co_sys && c == 0) {
      if (!grid_ok((long long)p.sys_wgs + p.grid)) return fail(RELAY_ERR_INVALID, "grid too large");
      relay::CoArgs co;
      co.sys = *co_sys;
      co.str = ac;
      co.n_sys = p.sys_wgs;
      e = relay::launch_stream_sys(co, p.rtc, p.sys_wgs + p.grid, s, &tc);
    } else {
      e = relay::launch_stream_attn(ac, rts, p.rtc, d->in_dtype, d->head_dim, p.grid, s, &tc);
    }
    if (e != hipSuccess) return hip_fail(e, "streaming attention launch");
  }
  return RELAY_OK;
}

// The merge: every row's output (and LSE when lse_out is given) from its parts.
int launch_merge(const relay_dims* d, const Plan& p, bool with_sys, bool with_ctx, char* ws, void* out, int out_bf16,
                 float* lse_out, hipStream_t s, const relay::LaunchTiming* tm = nullptr) {
  MergeArgs m{};
  m.n_rows = (long long)d->total_q * d->num_q_heads;
  m.num_q_heads = d->num_q_heads;
  m.group = d->num_q_heads / d->num_kv_heads;
  if (with_sys && p.sys_mode == 1) {
    m.sys_src = 1;
    m.sys_o = reinterpret_cast<const float*>(ws + p.off_sys_o);
    m.sys_lse = reinterpret_cast<const float*>(ws + p.off_sys_lse);
    m.sys_desc = reinterpret_cast<const int*>(ws + p.off_sys_desc);
    m.sys_rows = 16 * p.rts;
    m.sys_slots = p.sys_slots;
  } else if (with_sys && p.sys_mode >= 2) {
    m.sys_src = 2;
    m.sys_o = reinterpret_cast<const float*>(ws + p.off_sys_o);
    m.sys_lse = reinterpret_cast<const float*>(ws + p.off_sys_lse);
    m.sys_runs = p.sys_chunks;
  }
  if (with_ctx) {
    m.ctx_on = 1;
    m.ctx_o = reinterpret_cast<const float*>(ws + p.off_ctx_o);
    m.ctx_lse = reinterpret_cast<const float*>(ws + p.off_ctx_lse);
    m.ctx_rowdesc = reinterpret_cast<const int*>(ws + p.off_rowdesc);
    m.ctx_rows = 16 * p.rtc;
    m.ctx_slots = p.ctx_slots;
  }
  // the kernel reads both descriptor arrays unconditionally: unused ones point at the
  // row descriptors (always part of the workspace)
  m.ctx_rowdesc = reinterpret_cast<const int*>(ws + p.off_rowdesc);
  if (m.sys_src != 1) m.sys_desc = m.ctx_rowdesc;
  m.row_o = reinterpret_cast<const float*>(ws + p.off_row_o);
  m.row_lse = reinterpret_cast<const float*>(ws + p.off_row_lse);
  m.ks = p.ks;
  m.kc = p.kc;
  m.out = out;
  m.lse_out = lse_out;
  m.out_bf16 = out_bf16;
  hipError_t e = relay::launch_relay_merge(m, d->head_dim, s, tm);
  return e == hipSuccess ? RELAY_OK : hip_fail(e, "merge launch");
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

// Launch timing from the caller's events: pair k is events[2 k] (kernel start) and
// events[2 k + 1] (kernel end); none without events.
relay::LaunchTiming timing_pair(void* const* events, int k) {
  if (!events) return relay::LaunchTiming{nullptr, nullptr};
  return relay::LaunchTiming{static_cast<hipEvent_t>(events[2 * k]), static_cast<hipEvent_t>(events[2 * k + 1])};
}

int check_q_layout(const relay_dims* d, const int32_t* cu) {
  if (!cu && (d->total_q != d->batch || d->max_q_len != 1))
    return fail(RELAY_ERR_INVALID, "cu_q_lens is NULL: total_q must equal batch and max_q_len must be 1");
  return RELAY_OK;
}

// ---- the allocation-free decode's scratch --------------------------------------------
//
// The workspace of relay_attn_decode_noalloc: one array per device, part of the loaded
// code object (each device the library runs on holds its own copy until the process
// ends).  Host code never uses the array's name as an address: the device address comes
// from hipGetSymbolAddress, once per device, with that device current.
static_assert(RELAY_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) char scratch[RELAY_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch_ptr[kMaxDevices];

// This device's scratch address, or nullptr (and the error recorded) on failure.
void* scratch_ptr() {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    hip_fail(e, "hipGetDevice");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(RELAY_ERR_UNSUPPORTED, "device %d: the allocation-free path serves devices 0..%d", dev, kMaxDevices - 1);
    return nullptr;
  }
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess || !p) {
    hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    return nullptr;
  }
  // racing first calls on one device store the same address
  g_scratch_ptr[dev].store(p, std::memory_order_release);
  return p;
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
  Plan p, pc, ps;
  if (make_plan(dims, sys_len, &p) != RELAY_OK) return 0;
  // relay_ctx_attn plans the context streams alone (two workgroups per CU), and
  // relay_sys_attn the system step alone
  if (make_plan(dims, 0, &pc) != RELAY_OK) return 0;
  if (make_plan(dims, sys_len, &ps, kSysOnly) != RELAY_OK) return 0;
  size_t b = p.ws_bytes > pc.ws_bytes ? p.ws_bytes : pc.ws_bytes;
  return b > ps.ws_bytes ? b : ps.ws_bytes;
}

int relay_get_plan(const relay_dims* dims, int32_t sys_len, relay_plan* out) {
  int rc = check_dims(dims, sys_len);
  if (rc != RELAY_OK) return rc;
  if (!out) return fail(RELAY_ERR_INVALID, "plan is NULL");
  Plan p;
  if ((rc = make_plan(dims, sys_len, &p)) != RELAY_OK) return rc;
  out->sys_mode = p.sys_mode;
  out->sys_row_tiles = p.rts;
  out->sys_runs = p.sys_mode >= 2 ? p.sys_chunks : 0;
  out->sys_wgs = p.sys_mode >= 2 ? p.sys_wgs : 0;
  out->ctx_row_tiles = p.rtc;
  out->ctx_row_blocks = p.ctx_rb;
  out->stream_waves = p.workers;
  out->stream_launches = p.n_chunks;
  out->stream_max_requests = p.chunk_req;
  out->merge_wgs = p.merge_wgs;
  out->launches = p.launches;
  out->sys_rows_per_wg = p.sys_mode == 2 || p.sys_mode == 4 ? (p.sys_pp ? relay::kSysPPRows : relay::kSysMfmaRows) : 0;
  out->sys_row_slots = p.ks;
  out->ctx_row_slots = p.kc;
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
  if ((rc = make_plan(dims, sys_len, &p)) != RELAY_OK) return rc;
  if ((rc = check_ws(p, workspace, workspace_bytes)) != RELAY_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const relay::LaunchTiming t_sys = timing_pair(events, 0), t_stream = timing_pair(events, 1),
                            t_merge = timing_pair(events, 2);
  if ((p.sys_mode == 2 || p.sys_mode == 3) &&
      (rc = launch_sys_kernel(dims, p, q, sys_k, sys_v, sys_len, ws, s, &t_sys)) != RELAY_OK)
    return rc;
  const SysArgs co = p.sys_mode == 4 ? system_args(dims, p, q, sys_k, sys_v, sys_len, ws) : SysArgs{};
  if ((rc = launch_streams(dims, p, true, true, q, sys_k, sys_v, sys_len, ctx_k_pages, ctx_v_pages, block_tables,
                           ctx_lens, cu_q_lens, ws, s, &t_stream, p.sys_mode == 4 ? &co : nullptr)) != RELAY_OK)
    return rc;
  return launch_merge(dims, p, sys_len > 0, true, ws, out, dims->out_dtype == RELAY_BF16, nullptr, s, &t_merge);
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

int relay_attn_decode_noalloc(const relay_dims* dims, const void* q, const void* sys_k, const void* sys_v,
                              int32_t sys_len, const void* ctx_k_pages, const void* ctx_v_pages,
                              const int32_t* block_tables, const int32_t* ctx_lens,
                              const int32_t* cu_q_lens, void* out, void* stream) {
  int rc = check_dims(dims, sys_len);
  if (rc != RELAY_OK) return rc;
  Plan p;
  if ((rc = make_plan(dims, sys_len, &p)) != RELAY_OK) return rc;
  if (p.ws_bytes > (size_t)RELAY_NOALLOC_SCRATCH_BYTES)
    return fail(RELAY_ERR_WORKSPACE, "the call needs %zu bytes of workspace; the allocation-free path holds %zu",
                p.ws_bytes, (size_t)RELAY_NOALLOC_SCRATCH_BYTES);
  void* ws = scratch_ptr();
  if (!ws) return RELAY_ERR_HIP;
  return decode_impl(dims, q, sys_k, sys_v, sys_len, ctx_k_pages, ctx_v_pages, block_tables, ctx_lens, cu_q_lens,
                     out, ws, (size_t)RELAY_NOALLOC_SCRATCH_BYTES, stream, nullptr);
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
  if ((rc = make_plan(dims, sys_len, &p, kSysOnly)) != RELAY_OK) return rc;
  if ((rc = check_ws(p, workspace, workspace_bytes)) != RELAY_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if (p.sys_mode >= 2) {
    if ((rc = launch_sys_kernel(dims, p, q, sys_k, sys_v, sys_len, ws, s)) != RELAY_OK) return rc;
  } else if (p.sys_mode == 1) {
    if ((rc = launch_streams(dims, p, true, false, q, sys_k, sys_v, sys_len, nullptr, nullptr, nullptr, nullptr,
                             nullptr, ws, s)) != RELAY_OK)
      return rc;
  }
  return launch_merge(dims, p, sys_len > 0, false, ws, o_sys, 0, lse_sys, s);
}

size_t relay_prefill_workspace_size(const relay_dims* dims, int32_t sys_len) {
  if (check_dims(dims, sys_len) != RELAY_OK) return 0;
  Plan p;
  if (make_plan(dims, sys_len, &p, kPrefill) != RELAY_OK) return 0;
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
  const int M = dims->total_q * (dims->num_q_heads / dims->num_kv_heads);
  if (dims->in_dtype != RELAY_BF16 || dims->head_dim != 128 || M <= relay::kStreamSysMaxRows)
    return fail(RELAY_ERR_UNSUPPORTED, "the prefill runs on the matrix-core system kernel: bf16, head_dim 128 and "
                                       "more than %d query rows per KV head", relay::kStreamSysMaxRows);
  Plan p;
  if ((rc = make_plan(dims, sys_len, &p, kPrefill)) != RELAY_OK) return rc;
  if ((rc = check_ws(p, workspace, workspace_bytes)) != RELAY_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((rc = launch_sys_kernel(dims, p, q, sys_k, sys_v, sys_len, ws, s)) != RELAY_OK) return rc;
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
  if ((rc = make_plan(dims, 0, &p)) != RELAY_OK) return rc;
  if ((rc = check_ws(p, workspace, workspace_bytes)) != RELAY_OK) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  if ((rc = launch_streams(dims, p, false, true, q, nullptr, nullptr, 0, ctx_k_pages, ctx_v_pages, block_tables,
                           ctx_lens, cu_q_lens, ws, s)) != RELAY_OK)
    return rc;
  return launch_merge(dims, p, false, true, ws, o_ctx, 0, lse_ctx, s);
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
