// stream_attn: RelayAttention's system-attention and context-attention steps as one
// equal-work streaming launch on gfx950.
//
// The work is a sequence of 32-key steps (two 16-key tiles or pages of K and V):
//
//   * system streams, one per KV head h: the shared system keys of h, for all
//     M = T_q * g query rows that use h stacked into one operand (at most 64 rows, one
//     to four 16-row tiles), so the system K/V leave HBM once for the whole batch
//     (RelayAttention paper page, Abstract; atyun.com article, section
//     "RelayAttention": the per-request matrix-vector products against the system
//     prompt become one matrix-matrix product);
//   * context streams, one per (request b, KV head h, row block): request b's own paged
//     context keys, for the g * n_b query rows of b that use h (causal: query token t
//     of b sits at context position c_b - n_b + t).
//
// System streams come first, then the context streams in (request, head, row block)
// order.  With T steps in all and W waves in the launch, wave v owns the contiguous
// steps [v T / W, (v + 1) T / W) (W = min(waves, T), so no range is empty): every wave
// moves the same number of K/V bytes.  The system steps owned by the four waves of a
// workgroup form one contiguous range, which the four stream together (wave k takes
// every fourth step from the k-th) and merge through LDS at the end of each KV head's
// part, so a system piece belongs to a workgroup, not a wave: four times fewer system
// partials to write and to merge.  Each wave then streams the context steps of its own
// range, with its next steps in flight across the boundaries between streams.  Two
// workgroups share a CU where the registers allow (two waves per SIMD).
//
// The part of a context stream that one wave processes is a piece, and so is the part
// of a system stream that one workgroup processes; each piece writes one partial (O
// normalised by its own sum, and its log-sum-exp) for the stream's rows.  The first
// pieces of a stream go to places fixed in advance: piece k < ks of KV head h's system
// stream to system slot h ks + k, piece j < kc of a context stream to slot j of each of
// its rows; later ones to slot (H_kv ks + h + w) of the system partials (w the
// workgroup) or slot (stream id + v) of the context partials (v the wave).  Pieces are
// ordered like their streams, so these slots are distinct.  The holder of a stream's
// first step also writes where the stream's pieces are (first slot and count), per KV
// head for system streams and per output row for context streams; the merge
// (relay_fuse.hip) reads those together with the fixed places and combines the pieces of
// a row with the same log-sum-exp identity that relay fusion uses.
#include "relay_device.hpp"
#include "relay_internal.hpp"
#include "sys_attn_mfma.hpp"

namespace relay {

namespace strm {
constexpr int kWaves = kStreamWaves;
constexpr int kWin = 32;  // steps per page-id window: one page id per lane, two per step
}  // namespace strm

__device__ __forceinline__ int ceil_steps(int keys) { return (keys + kStep - 1) / kStep; }

// Which wave of `parts` holds step x of `total` (waves hold [p total / parts, (p + 1)
// total / parts)).
__device__ __forceinline__ int part_of64(long long x, long long total, int parts) {
  return (int)(((x + 1) * parts + total - 1) / total) - 1;
}

// P enters P.V as bf16 hi + lo (two products).  A single bf16 rounding of P costs up
// to 2^-9 of each probability, and a key can hold half of a row's weight even among
// hundreds of keys (peaked logits), which alone exceeds 2e-3 on values of size 4; the
// second product costs matrix-core time that hides under the memory stream.
constexpr bool kStreamPSplit = true;

// Steps held in registers at once: two for bf16 with one row tile, or two row tiles
// at one workgroup per CU (the next step's loads are in flight while one computes),
// else one (fp32 steps are twice the bytes; more row tiles of queries and accumulators
// leave no room for a second step within the registers of the occupancy).
template <typename T, int RT, int OCC>
constexpr int stream_depth_of() {
  return (Elem<T>::kBytes == 2 && (RT <= 1 || (OCC == 1 && RT <= 2))) ? 2 : 1;
}

// ---- per-launch request tables (LDS) --------------------------------------------------
//
// For request i of the launch (b = b_begin + i): pre[i] = its first context step
// (exclusive prefix of its step counts; pre[n] = all context steps), clen[i] its clamped
// context length, qs[i] / nq[i] its query-row range.  Built by the whole workgroup.
struct ReqTables {
  int* pre;
  int* clen;
  int* qs;
  int* nq;
};

__device__ __forceinline__ int request_row_blocks(const StreamArgs& a, int nq, int rows_per_block) {
  return min((nq * a.group + rows_per_block - 1) / rows_per_block, a.ctx_rb);
}

template <int RTC>
__device__ void build_tables(const StreamArgs& a, const ReqTables& t, int* scratch) {
  constexpr int kThreads = kWave * strm::kWaves;
  const int n = a.n_req;
  const int tid = threadIdx.x;
  const int per = (n + kThreads - 1) / kThreads;
  const int i0 = min(tid * per, n), i1 = min(i0 + per, n);
  const int cap = min(a.max_ctx_len, a.max_blocks_per_seq * kTile);
  int sum = 0;
  for (int i = i0; i < i1; ++i) {
    const int b = a.b_begin + i;
    const int c = min(max(a.ctx_lens[b], 0), cap);
    int qs = b, nq = 1;
    if (a.cu_q_lens) {
      qs = min(max(a.cu_q_lens[b], 0), a.total_q);
      nq = min(max(a.cu_q_lens[b + 1] - qs, 0), a.total_q - qs);
    }
    // a context of length 0 (invalid data) still gets one fully masked step
    const int w = max(1, ceil_steps(c)) * a.num_kv_heads * request_row_blocks(a, nq, 16 * RTC);
    t.clen[i] = c;
    t.qs[i] = qs;
    t.nq[i] = nq;
    t.pre[i] = w;  // the weight, turned into the prefix below
    sum += w;
  }
  // inclusive scan of the thread sums: inside each wave by shuffles, then over the
  // wave totals (one barrier)
  const int lane = lane_id(), wave = tid / kWave;
  int incl = sum;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const int y = __shfl_up(incl, off, kWave);
    if (lane >= off) incl += y;
  }
  if (lane == kWave - 1) scratch[wave] = incl;
  __syncthreads();
  int base = 0, all = 0;
#pragma unroll
  for (int k = 0; k < strm::kWaves; ++k) {
    base += k < wave ? scratch[k] : 0;
    all += scratch[k];
  }
  int run = base + incl - sum;  // exclusive prefix of this thread's first request
  for (int i = i0; i < i1; ++i) {
    const int w = t.pre[i];
    t.pre[i] = run;
    run += w;
  }
  if (tid == kThreads - 1) t.pre[n] = all;
  __syncthreads();
}

// ---- one stream, one piece: depth-pipelined steps with fixed addresses ---------------

// Streams steps 0 .. nsteps - 1 (addr(s) gives step s's tiles, whose first key is
// key0 + s * key_stride); DEPTH steps in flight.
template <typename T, int D, int RT, bool PSPLIT, int DEPTH, class Addr>
__device__ __forceinline__ void run_steps(int nsteps, const u32x4 (&qf)[RT][StepK<T, D>::NCH], RowState<D> (&st_)[RT],
                                          int key0, int key_stride, int kv_len, const int (&last)[RT],
                                          float scale_log2, Addr&& addr) {
  const int q4 = lane_id() >> 4;
  auto issue = [&](StepK<T, D>& k, StepV<T, D>& v, int s) {
    const StepAddr ad = addr(s);
    issue_k(k, ad.ka, ad.kb);
    issue_v(v, ad.va, ad.vb);
  };
  auto run = [&](StepK<T, D>& k, StepV<T, D>& v, int s) {
    const int keyq = key0 + key_stride * s + 8 * q4;
    PStep<T> p[RT];
    step_scores<T, D, RT, PSPLIT>(k, qf, st_, keyq, kv_len, last, scale_log2, p);
    step_pv<T, D, RT, PSPLIT>(v, keyq, kv_len, st_, p);
  };
  if (nsteps <= 0) return;
  if constexpr (DEPTH >= 2) {
    // a ring of DEPTH steps: step s computes while the loads of s + 1 .. s + DEPTH - 1
    // are in flight; its registers then take the loads of s + DEPTH
    StepK<T, D> k[DEPTH];
    StepV<T, D> v[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (d < nsteps) issue(k[d], v[d], d);
    for (int s = 0; s < nsteps; s += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        if (s + d >= nsteps) break;
        run(k[d], v[d], s + d);
        if (s + d + DEPTH < nsteps) issue(k[d], v[d], s + d + DEPTH);
      }
    }
  } else {
    StepK<T, D> k;
    StepV<T, D> v;
    issue(k, v, 0);
    for (int s = 0; s < nsteps; ++s) {
      const int keyq = key0 + key_stride * s + 8 * q4;
      PStep<T> p[RT];
      step_scores<T, D, RT, PSPLIT>(k, qf, st_, keyq, kv_len, last, scale_log2, p);
      StepAddr ad;
      if (s + 1 < nsteps) {
        ad = addr(s + 1);
        issue_k(k, ad.ka, ad.kb);
      }
      step_pv<T, D, RT, PSPLIT>(v, keyq, kv_len, st_, p);
      if (s + 1 < nsteps) issue_v(v, ad.va, ad.vb);
    }
  }
}

// System piece: steps [j0, j1) of KV head h's stream, all M stacked rows (RTS tiles),
// streamed by the four waves of workgroup w (wave k takes steps j0 + k, j0 + k + 4, ...)
// and merged through LDS (mlds: stream_merge_lds_bytes of this workgroup).  Every wave
// of the workgroup calls it with the same arguments (it holds barriers).
template <typename T, int D, int RTS, int OCC>
__device__ void system_piece(const StreamArgs& a, int h, int j0, int j1, int w, int wk, int k, long long total,
                             int W, float* mlds) {
  constexpr int E = Elem<T>::kBytes;
  const int lane = lane_id(), r16 = lane & 15;
  u32x4 qf[RTS][StepK<T, D>::NCH];
  RowState<D> rs[RTS];
  int last[RTS];
#pragma unroll
  for (int rt = 0; rt < RTS; ++rt) {
    const int m = rt * 16 + r16;
    const int t = m / a.group, gi = m % a.group;
    const bool ok = m < a.M;
    load_q_tile<T, D>(qf[rt], a.q, ok ? (size_t)t * a.num_q_heads + (size_t)h * a.group + gi : 0, ok);
    rs[rt].init();
    last[rt] = a.sys_len - 1;
  }
  const int Ls = a.sys_len;
  const int key_end = min(j1 * kStep, Ls);
  const int ntile = (Ls + kTile - 1) / kTile;
  const char* kbase = static_cast<const char*>(a.sys_k) + (size_t)h * ntile * kTile * D * E;
  const char* vbase = static_cast<const char*>(a.sys_v) + (size_t)h * ntile * D * kTile * E;
  // this wave's steps: j0 + wk + 4 s; step j covers system tiles 2 j and 2 j + 1 (a tile
  // past the prompt's end repeats the previous one; its keys are masked)
  const int mine = j1 - j0 > wk ? (j1 - j0 - wk + strm::kWaves - 1) / strm::kWaves : 0;
  const int key0 = (j0 + wk) * kStep;
  auto addr = [&](int s) {
    const int ka = key0 + strm::kWaves * kStep * s;
    const int kb = ka + kTile < Ls ? ka + kTile : ka;
    StepAddr r;
    r.ka = kbase + (size_t)(ka / kTile) * kTile * D * E;
    r.kb = kbase + (size_t)(kb / kTile) * kTile * D * E;
    r.va = vbase + (size_t)(ka / kTile) * D * kTile * E;
    r.vb = vbase + (size_t)(kb / kTile) * D * kTile * E;
    return r;
  };
  constexpr int DEPTH = stream_depth_of<T, RTS, OCC>();
  run_steps<T, D, RTS, kStreamPSplit, DEPTH>(mine, qf, rs, key0, strm::kWaves * kStep, key_end, last, a.scale_log2,
                                              addr);
  // the four waves' states, one row tile at a time (fixed tree order: deterministic)
#pragma unroll
  for (int rt = 0; rt < RTS; ++rt)
    merge_key_lanes<D, 1, strm::kWaves>(*reinterpret_cast<RowState<D>(*)[1]>(&rs[rt]), wk, mlds);
  if (wk != 0) return;

  // piece k of the stream (k = w - the first piece's workgroup): fixed slot h ks + k while
  // k < ks, else slot H_kv ks + h + w
  const int slot = a.num_kv_heads * a.ks + h + w;
  const size_t base = k < a.ks ? (size_t)h * a.ks + k : (size_t)slot;
#pragma unroll
  for (int rt = 0; rt < RTS; ++rt) {
    const int m = rt * 16 + r16;
    float* orow = nullptr;
    float* lrow = nullptr;
    if (m < a.M) {
      const size_t r = base * (16 * RTS) + m;
      orow = a.sys_o + r * D;
      lrow = a.sys_lse + r;
    }
    store_row_tile(rs[rt], orow, lrow);
  }
  if (j0 == 0 && lane == 0) {
    // the workgroup holding the stream's last step: the wave holding it, over four
    const long long p0 = (long long)h * a.sys_steps;
    a.sys_desc[2 * h] = slot;
    a.sys_desc[2 * h + 1] = part_of64(p0 + a.sys_steps - 1, total, W) / strm::kWaves - w + 1;
  }
}

// ---- context: cross-stream streaming ----------------------------------------------------

// Page-id window: lane l describes step y0 + l / 2 of the wave's context range (its
// request, head, row block, step in the stream) and holds page l % 2 of that step.
struct CtxWin {
  long long y0;
  int i, h, rb, j, page;
};

template <int RTC>
__device__ __forceinline__ CtxWin ctx_window(const StreamArgs& a, const ReqTables& t, long long yw, long long y1) {
  CtxWin w;
  w.y0 = yw;
  const int lane = lane_id();
  const long long y = yw + (lane >> 1);
  int i = 0, h = 0, rb = 0, j = 0, page = 0;
  if (y < y1) {
    int lo = 0, hi = a.n_req;  // pre[lo] <= y < pre[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (t.pre[mid] <= y) lo = mid;
      else hi = mid;
    }
    i = lo;
    const int c = t.clen[i];
    const int steps = max(1, ceil_steps(c));
    const int off = (int)(y - t.pre[i]);
    const int k = off / steps;
    j = off - k * steps;
    const int rbs = request_row_blocks(a, t.nq[i], 16 * RTC);
    h = k / rbs;
    rb = k - h * rbs;
    const int npg = max(1, (c + kTile - 1) / kTile);
    const int pi = min(2 * j + (lane & 1), npg - 1);
    page = a.block_tables[(size_t)(a.b_begin + i) * a.max_blocks_per_seq + pi];
    page = min(max(page, 0), a.num_blocks - 1);
  }
  w.i = i;
  w.h = h;
  w.rb = rb;
  w.j = j;
  w.page = page;
  return w;
}

// One context step in registers: its K/V, the query rows of its stream, and where it is.
template <typename T, int D, int RTC>
struct CtxSlot {
  StepK<T, D> k;
  StepV<T, D> v;
  u32x4 q[RTC][StepK<T, D>::NCH];
  int i, h, rb, j;
};

// The piece being accumulated.
struct CtxPiece {
  int i, h, rb, j0, c, qs, nq;
};

// OWN: the launch may place context pieces in the rows' own slots (a.kc > 0); the
// launch beside the matrix-core system workgroups never does.
template <typename T, int D, int RTC, int OCC, bool OWN>
__device__ void context_range(const StreamArgs& a, const ReqTables& t, long long y0, long long y1, long long Ts,
                              int v, long long total, int W) {
  constexpr int E = Elem<T>::kBytes;
  constexpr int DEPTH = stream_depth_of<T, RTC, OCC>();
  constexpr int RPB = 16 * RTC;  // rows per block
  const int lane = lane_id(), q4 = lane >> 4, r16 = lane & 15;
  const size_t page_stride = (size_t)a.num_kv_heads * kTile * D * E;

  CtxWin wc = ctx_window<RTC>(a, t, y0, y1);
  // only the wave's first piece can start inside its stream: its index among the
  // stream's pieces (that stream's first step is launch step Ts + y0 - j, j the stream
  // step at y0)
  const int j_first = OWN ? v - part_of64(Ts + y0 - __builtin_amdgcn_readfirstlane(wc.j), total, W) : 0;
  CtxWin wn = (y0 + strm::kWin < y1) ? ctx_window<RTC>(a, t, y0 + strm::kWin, y1) : wc;

  auto issue = [&](CtxSlot<T, D, RTC>& s, long long y) {
    const CtxWin& w = (y < wc.y0 + strm::kWin) ? wc : wn;
    const int l = 2 * (int)(y - w.y0);
    s.i = __builtin_amdgcn_readlane(w.i, l);
    s.h = __builtin_amdgcn_readlane(w.h, l);
    s.rb = __builtin_amdgcn_readlane(w.rb, l);
    s.j = __builtin_amdgcn_readlane(w.j, l);
    const int pa = __builtin_amdgcn_readlane(w.page, l);
    const int pb = __builtin_amdgcn_readlane(w.page, l + 1);
    const char* kbase = static_cast<const char*>(a.ctx_k) + (size_t)s.h * kTile * D * E;
    const char* vbase = static_cast<const char*>(a.ctx_v) + (size_t)s.h * D * kTile * E;
    issue_k(s.k, kbase + (size_t)pa * page_stride, kbase + (size_t)pb * page_stride);
    issue_v(s.v, vbase + (size_t)pa * page_stride, vbase + (size_t)pb * page_stride);
    const int qs = t.qs[s.i], nq = t.nq[s.i];
#pragma unroll
    for (int rt = 0; rt < RTC; ++rt) {
      const int rl = s.rb * RPB + rt * 16 + r16;
      const bool ok = rl < nq * a.group;
      const int tl = rl / a.group, gi = rl - tl * a.group;
      load_q_tile<T, D>(s.q[rt], a.q, ok ? (size_t)(qs + tl) * a.num_q_heads + (size_t)s.h * a.group + gi : 0, ok);
    }
  };

  RowState<D> rs[RTC];
  int last[RTC];
  CtxPiece cur{-1, 0, 0, 0, 0, 0, 0};

  // the finished piece's partial (and, for a stream's first piece, where its pieces are):
  // piece j of the stream goes to slot j of each of its rows while j < kc, else to stream
  // slot s_id + v
  auto finish = [&]() {
    const int i = cur.i;
    const long long s_id = ((long long)i * a.num_kv_heads + cur.h) * a.ctx_rb + cur.rb;
    const long long slot = s_id + v + a.slot_base;
    const int steps = max(1, ceil_steps(cur.c));
    const int rbs = request_row_blocks(a, cur.nq, RPB);
    const long long p0 = Ts + t.pre[i] + (long long)(cur.h * rbs + cur.rb) * steps;
    const int pieces = part_of64(p0 + steps - 1, total, W) - v + 1;
    const int j = cur.j0 > 0 ? j_first : 0;
#pragma unroll
    for (int rt = 0; rt < RTC; ++rt) {
      const int rr = rt * 16 + r16;
      const int rl = cur.rb * RPB + rr;
      const bool ok = rl < cur.nq * a.group;
      float* orow = nullptr;
      float* lrow = nullptr;
      if (ok) {
        const bool own = OWN && j < a.kc;
        const int tl0 = rl / a.group, gi0 = rl - tl0 * a.group;
        const size_t oi0 = (size_t)(cur.qs + tl0) * a.num_q_heads + (size_t)cur.h * a.group + gi0;
        const size_t r = own ? oi0 * a.kc + j : (size_t)slot * RPB + rr;
        orow = (own ? a.row_o : a.ctx_o) + r * D;
        lrow = (own ? a.row_lse : a.ctx_lse) + r;
      }
      store_row_tile(rs[rt], orow, lrow);
      if (ok && cur.j0 == 0 && q4 == 0) {
        const int tl = rl / a.group, gi = rl - tl * a.group;
        const size_t orow_idx = (size_t)(cur.qs + tl) * a.num_q_heads + (size_t)cur.h * a.group + gi;
        *reinterpret_cast<int4*>(a.ctx_rowdesc + 4 * orow_idx) = int4{(int)slot, pieces, rr, 0};
      }
    }
  };

  // piece bookkeeping and the step's arithmetic
  auto compute = [&](CtxSlot<T, D, RTC>& s, long long y) {
    if (s.i != cur.i || s.h != cur.h || s.rb != cur.rb) {
      if (cur.i >= 0) finish();
      cur.i = s.i;
      cur.h = s.h;
      cur.rb = s.rb;
      cur.j0 = s.j;
      cur.c = t.clen[s.i];
      cur.qs = t.qs[s.i];
      cur.nq = t.nq[s.i];
#pragma unroll
      for (int rt = 0; rt < RTC; ++rt) {
        rs[rt].init();
        const int rl = cur.rb * RPB + rt * 16 + r16;
        last[rt] = rl < cur.nq * a.group ? cur.c - cur.nq + rl / a.group : -1;
      }
    }
    const int keyq = s.j * kStep + 8 * q4;
    PStep<T> p[RTC];
    step_scores<T, D, RTC, kStreamPSplit>(s.k, s.q, rs, keyq, cur.c, last, a.scale_log2, p);
    step_pv<T, D, RTC, kStreamPSplit>(s.v, keyq, cur.c, rs, p);
  };

  // windows advance as the computed step leaves the current one
  auto advance = [&](long long y) {
    if (y >= wc.y0 + strm::kWin) {
      wc = wn;
      if (wc.y0 + strm::kWin < y1) wn = ctx_window<RTC>(a, t, wc.y0 + strm::kWin, y1);
    }
  };

  if constexpr (DEPTH >= 2) {
    CtxSlot<T, D, RTC> sl[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d)
      if (y0 + d < y1) issue(sl[d], y0 + d);
    for (long long y = y0; y < y1; y += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        if (y + d >= y1) break;
        advance(y + d);
        compute(sl[d], y + d);
        if (y + d + DEPTH < y1) issue(sl[d], y + d + DEPTH);
      }
    }
  } else {
    CtxSlot<T, D, RTC> s0;
    issue(s0, y0);
    for (long long y = y0; y < y1; ++y) {
      advance(y);
      compute(s0, y);
      if (y + 1 < y1) issue(s0, y + 1);
    }
  }
  if (cur.i >= 0) finish();
}

// ---- the kernel ---------------------------------------------------------------------------

template <typename T, int D, int RTS, int RTC>
constexpr int stream_occ() {
  return stream_wgs_per_cu(Elem<T>::kBytes, D, RTS, RTC);
}

// LDS of one workgroup: the request tables (4 n + 1 ints), the scan scratch (one int per
// thread), then, 16-byte aligned, the system pieces' merge area.
__host__ __device__ constexpr size_t stream_tables_bytes(int n) {
  return (sizeof(int) * ((size_t)4 * n + 1 + (size_t)kWave * kStreamWaves) + 15) / 16 * 16;
}

// Streaming workgroup w of the launch's streaming workgroups (lds_tab: its LDS).
template <typename T, int D, int RTS, int RTC, bool OWN>
__device__ __forceinline__ void stream_workgroup(const StreamArgs& a, int w, int* lds_tab) {
  constexpr int OCC = stream_occ<T, D, RTS, RTC>();
  const int n = a.ctx_on ? a.n_req : 0;
  ReqTables t{lds_tab, lds_tab + n + 1, lds_tab + 2 * n + 1, lds_tab + 3 * n + 1};
  long long Tc = 0;
  if (a.ctx_on) {
    build_tables<RTC>(a, t, lds_tab + 4 * n + 1);
    Tc = t.pre[n];
  }
  const long long Ts = (RTS > 0) ? (long long)a.num_kv_heads * a.sys_steps : 0;
  const long long total = Ts + Tc;
  // with fewer steps than waves only the first `total` waves take part (one step each),
  // so that every wave of the partition holds at least one step and the pieces of a
  // stream sit on consecutive waves (and workgroups)
  const int W = total < a.n_workers ? (int)total : a.n_workers;
  const int wk = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
  const int v = w * strm::kWaves + wk;
  if (total == 0 || w * strm::kWaves >= W) return;  // uniform over the workgroup
  if constexpr (RTS > 0) {
    // the system steps of the workgroup's waves (all four take part, also a wave past W)
    const int vl = min(w * strm::kWaves + strm::kWaves - 1, W - 1);
    long long x = (long long)w * strm::kWaves * total / W;
    const long long X1 = (long long)(vl + 1) * total / W;
    const long long xs1 = X1 < Ts ? X1 : Ts;
    float* mlds = reinterpret_cast<float*>(reinterpret_cast<char*>(lds_tab) + stream_tables_bytes(n));
    while (x < xs1) {
      const int h = (int)(x / a.sys_steps);
      const int j0 = (int)(x - (long long)h * a.sys_steps);
      const int j1 = (int)((long long)j0 + (xs1 - x) < a.sys_steps ? j0 + (xs1 - x) : a.sys_steps);
      // only the workgroup's first piece can start inside a stream (k > 0)
      const int k = j0 > 0 ? w - part_of64((long long)h * a.sys_steps, total, W) / strm::kWaves : 0;
      system_piece<T, D, RTS, OCC>(a, h, j0, j1, w, wk, k, total, W, mlds);
      x += j1 - j0;
    }
  }
  if (v >= W) return;
  const long long x0 = (long long)v * total / W, x1 = (long long)(v + 1) * total / W;
  if (a.ctx_on && x1 > Ts) {
    const long long y0 = (x0 > Ts ? x0 : Ts) - Ts, y1 = x1 - Ts;
    context_range<T, D, RTC, OCC, OWN>(a, t, y0, y1, Ts, v, total, W);
  }
}

template <typename T, int D, int RTS, int RTC>
__global__ __launch_bounds__(kWave* strm::kWaves, (stream_occ<T, D, RTS, RTC>())) void stream_attn_kernel(
    StreamArgs a) {
  extern __shared__ int lds_tab[];
  stream_workgroup<T, D, RTS, RTC, true>(a, blockIdx.x, lds_tab);
}

// The decode step with more than 64 stacked rows per KV head (bf16, head_dim 128): the
// matrix-core system workgroups (the first a.n_sys of the launch, compute-bound) and the
// context streams' workgroups (memory-bound) in one launch, one of each per CU, so
// each CU's matrix cores and its memory stream work at the same time.
template <int RTC>
__global__ __launch_bounds__(kWave* strm::kWaves, 2) void stream_sys_kernel(CoArgs a) {
  extern __shared__ __attribute__((aligned(16))) int lds_tab[];
  if ((int)blockIdx.x < a.n_sys)
    sys_mfma_workgroup<false>(a.sys, blockIdx.x, a.n_sys, reinterpret_cast<char*>(lds_tab));
  else
    stream_workgroup<bf16_t, 128, 0, RTC, false>(a.str, blockIdx.x - a.n_sys, lds_tab);
}

hipError_t launch_stream_sys(const CoArgs& a, int rtc, int grid, hipStream_t s, const LaunchTiming* tm) {
  static_assert(stream_wgs_per_cu(2, 128, 0, 1) == 2 && stream_wgs_per_cu(2, 128, 0, 2) == 2,
                "the context workgroups are built for two per CU");
  if (rtc != 1 && rtc != 2) return hipErrorInvalidValue;
  const size_t lds = stream_lds_bytes(a.str.n_req, a.str.ctx_on, 0, 128);
  const uint32_t bytes = (uint32_t)(lds > kSysMfmaLds ? lds : kSysMfmaLds);
  if (rtc == 1) launch_kernel(stream_sys_kernel<1>, dim3(grid), dim3(kWave * strm::kWaves), bytes, s, tm, a);
  else launch_kernel(stream_sys_kernel<2>, dim3(grid), dim3(kWave * strm::kWaves), bytes, s, tm, a);
  return hipGetLastError();
}

size_t stream_lds_bytes(int n_req, int ctx_on, int sys_on, int head_dim) {
  const int n = ctx_on ? n_req : 0;
  return stream_tables_bytes(n) + (sys_on ? (size_t)stream_merge_lds_bytes(head_dim) : 0);
}

template <typename T, int D, int RTS, int RTC>
static hipError_t launch_stream_t(const StreamArgs& a, int grid, hipStream_t s, const LaunchTiming* tm) {
  const size_t lds = stream_lds_bytes(a.n_req, a.ctx_on, RTS > 0, D);
  launch_kernel(stream_attn_kernel<T, D, RTS, RTC>, dim3(grid), dim3(kWave * strm::kWaves), (uint32_t)lds, s, tm, a);
  return hipGetLastError();
}

template <typename T, int D, int RTS>
static hipError_t launch_stream_c(const StreamArgs& a, int rtc, int grid, hipStream_t s, const LaunchTiming* tm) {
  return rtc == 1 ? launch_stream_t<T, D, RTS, 1>(a, grid, s, tm) : launch_stream_t<T, D, RTS, 2>(a, grid, s, tm);
}

template <typename T, int D>
static hipError_t launch_stream_d(const StreamArgs& a, int rts, int rtc, int grid, hipStream_t s,
                                  const LaunchTiming* tm) {
  switch (rts) {
    case 0: return launch_stream_c<T, D, 0>(a, rtc, grid, s, tm);
    case 1: return launch_stream_c<T, D, 1>(a, rtc, grid, s, tm);
    case 2: return launch_stream_c<T, D, 2>(a, rtc, grid, s, tm);
    default: return launch_stream_c<T, D, 4>(a, rtc, grid, s, tm);
  }
}

hipError_t launch_stream_attn(const StreamArgs& a, int rts, int rtc, int in_dtype, int head_dim, int grid,
                              hipStream_t stream, const LaunchTiming* tm) {
  if ((rts != 0 && rts != 1 && rts != 2 && rts != 4) || (rtc != 1 && rtc != 2)) return hipErrorInvalidValue;
  if (in_dtype == 1)
    return head_dim == 64 ? launch_stream_d<bf16_t, 64>(a, rts, rtc, grid, stream, tm)
                          : launch_stream_d<bf16_t, 128>(a, rts, rtc, grid, stream, tm);
  return head_dim == 64 ? launch_stream_d<float, 64>(a, rts, rtc, grid, stream, tm)
                        : launch_stream_d<float, 128>(a, rts, rtc, grid, stream, tm);
}

}  // namespace relay
