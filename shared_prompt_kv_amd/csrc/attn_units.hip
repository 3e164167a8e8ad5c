// Streaming attention units for gfx950: RelayAttention's system-attention and
// context-attention steps as workgroup-sized work units.
//
// System unit (KV head h, key chunk, row unit of one or two 16-row tiles): the
// tiles hold 16 or 32 of the M = T_q * g query rows that use KV head h, stacked across
// all requests of the batch, so the system K/V of the chunk serve every request's
// query at once (RelayAttention paper, abstract; atyun.com article, section
// "RelayAttention": matrix-vector products against the system prompt grouped into
// matrix-matrix products).  When there are more rows than one unit holds, the row
// units of one chunk are separate units placed on the same XCD back to back, so the
// chunk leaves HBM once and the repeat reads hit that XCD's L2.
//
// Context unit (request b, KV head h, split, row block): causal attention of the
// request's g * n_b query rows over one fixed-length run of its paged context.
// Query token t sits at context position c_b - n_b + t.  The page ids of the whole
// split are fetched once, one per lane, and broadcast per step.  A unit whose split
// lies past the end of the context writes LSE = -inf for its rows, so relay_fuse
// can read every split slot without knowing the context lengths.
//
// A unit is one workgroup of WK waves (key lanes).  Key lane kl streams the 32-key
// steps (two pages) kl, kl+WK, ... of the unit, so a unit's critical path is 1/WK of its steps;
// the lanes' softmax states are merged through LDS (fixed order) and key lane 0
// writes one partial (O, LSE) per row.  sys_ctx_attn_kernel carries both kinds of
// unit in one launch (system units first: they are the longest), so the two steps
// overlap and the machine fills even when one step alone could not.
#include <atomic>

#include "relay_device.hpp"
#include "relay_internal.hpp"

namespace relay {

template <typename T, int D>
__device__ inline void load_q_tile(u32x4* qf, const void* q, size_t row_index, bool valid) {
  constexpr int E = Elem<T>::kBytes;
  const int q4 = lane_id() >> 4;
  const char* qp = static_cast<const char*>(q) + row_index * D * E;
#pragma unroll
  for (int kk = 0; kk < StepK<T, D>::NCH; ++kk)
    qf[kk] = valid ? ld16(qp + 64 * kk + 16 * q4) : u32x4{0u, 0u, 0u, 0u};
}

// SRT row tiles (16 rows each) per unit: 2 when M <= 32 and the system step is long
// enough to give every workgroup several units, so the chunk is read once for all 32
// rows; 1 otherwise (more, shorter units).
template <typename T, int D, int SRT, int WK>
__device__ __forceinline__ void sys_unit(const UnitArgs& a, int u, float* lds) {
  constexpr int E = Elem<T>::kBytes;
  const int lane = lane_id();
  const int kl = threadIdx.x / kWave;
  const int r16 = lane & 15;
  // unit id -> (row unit, chunk group): the row units of one chunk are 8 ids apart,
  // i.e. on the same XCD (workgroup i runs on XCD i % 8) and dispatched together.
  const int slot = u >> 3;
  const int ru = slot % a.sys_row_tiles;
  const int grp = (u & 7) + 8 * (slot / a.sys_row_tiles);
  const int chunk = grp % a.sys_chunks;
  const int h = grp / a.sys_chunks;
  if (h >= a.num_kv_heads) return;  // padding unit: uniform over the workgroup

  const int M = a.total_q * a.group;
  u32x4 qf[SRT][StepK<T, D>::NCH];
  RowState<D> st[SRT];
  int last[SRT];
  size_t qrow[SRT];
#pragma unroll
  for (int r = 0; r < SRT; ++r) {
    const int row = (ru * SRT + r) * 16 + r16;
    const int t = row / a.group, gi = row % a.group;
    qrow[r] = row < M ? (size_t)t * a.num_q_heads + (size_t)h * a.group + gi : ~(size_t)0;
    load_q_tile<T, D>(qf[r], a.q, qrow[r], row < M);
    st[r].init();
    last[r] = a.sys_len - 1;
  }

  const int Ls = a.sys_len;
  const int key_begin = chunk * a.sys_chunk_len;
  const int key_end = min(key_begin + a.sys_chunk_len, Ls);
  const int ntile = (Ls + kTile - 1) / kTile;
  // both caches are 16-key tiles, ntile per KV head (keys chunk-major, values dim-major)
  const char* kbase = static_cast<const char*>(a.sys_k) + (size_t)h * ntile * kTile * D * E;
  const char* vbase = static_cast<const char*>(a.sys_v) + (size_t)h * ntile * D * kTile * E;

  // step s covers system tiles key_begin/16 + 2s and + 2s + 1; a page past the end of
  // the keys re-reads the first, and keys past the end (the tail tile's padding slots,
  // in bounds) are masked
  const int npages = (key_end - key_begin + kTile - 1) / kTile;
  const int nsteps = (npages + 1) / 2;
  auto addr = [&](int st_) {
    const int ka = key_begin + 2 * kTile * st_;
    const int kb = ka + kTile < Ls ? ka + kTile : ka;
    StepAddr r;
    r.ka = kbase + (size_t)(ka / kTile) * kTile * D * E;
    r.kb = kbase + (size_t)(kb / kTile) * kTile * D * E;
    r.va = vbase + (size_t)(ka / kTile) * D * kTile * E;
    r.vb = vbase + (size_t)(kb / kTile) * D * kTile * E;
    return r;
  };
  if (key_end - key_begin < kPSplitBelow)
    stream_pipelined<T, D, SRT, WK, true>(kl, nsteps, qf, st, key_begin, key_end, last, a.scale_log2, addr);
  else
    stream_pipelined<T, D, SRT, WK, false>(kl, nsteps, qf, st, key_begin, key_end, last, a.scale_log2, addr);
  merge_key_lanes<D, SRT, WK>(st, kl, lds);

  if (kl == 0) {
#pragma unroll
    for (int r = 0; r < SRT; ++r) {
      float* orow = nullptr;
      float* lrow = nullptr;
      if (qrow[r] != ~(size_t)0) {
        const size_t rr = (size_t)chunk * a.total_q * a.num_q_heads + qrow[r];
        orow = a.sys_o + rr * D;
        lrow = a.sys_lse + rr;
      }
      store_row_tile(st[r], orow, lrow);
    }
  }
}

// Where a context unit's work is, read before the unit starts: the next unit's
// metadata loads are issued while the current unit streams, so a unit begins with
// its context length, query range and page ids already in registers.
struct CtxMeta {
  int raw;  // lane 0: context length; lanes 1, 2: the request's query-token range
            // (when cu_q_lens is given)
  int pt;   // this lane's page id (lane s holds the split's page s)
};

// Issues the metadata loads of context unit v (values are consumed later).  They are
// per-lane vector loads (lanes 0..2 read the request's length and query range), so
// their wait is the first use in the next unit, not the issue point.
__device__ __forceinline__ CtxMeta ctx_meta(const UnitArgs& a, int v) {
  CtxMeta m{0, 0};
  const int slot = v >> 3;
  const int grp = (v & 7) + 8 * (slot / a.ctx_row_blocks);
  const int per_split = a.batch * a.num_kv_heads;
  const int split = grp / per_split;
  if (split >= a.ctx_max_splits) return m;  // padding unit
  const int b = (grp % per_split) / a.num_kv_heads;
  // every lane loads (one vector load, in-bounds lane-dependent addresses): lane 0
  // the context length, lanes 1 and 2 the query range when there is one
  const int lane = lane_id();
  const int32_t* src = a.cu_q_lens ? (lane == 0 ? a.ctx_lens + b : a.cu_q_lens + min(b + lane - 1, a.batch))
                                   : a.ctx_lens + min(b + lane, a.batch - 1);
  m.raw = *src;
  // table entries of the split; entries past the context are read but never used
  const int pg_begin = split * (a.ctx_split_len / kTile);
  if (lane < a.ctx_split_len / kTile && pg_begin + lane < a.max_blocks_per_seq)
    m.pt = a.block_tables[(size_t)b * a.max_blocks_per_seq + pg_begin + lane];
  return m;
}

template <typename T, int D, int RT, int WK>
__device__ __forceinline__ void ctx_unit(const UnitArgs& a, int v, CtxMeta m, float* lds) {
  constexpr int E = Elem<T>::kBytes;
  constexpr int NCH = StepK<T, D>::NCH;
  const int lane = lane_id();
  const int kl = threadIdx.x / kWave;
  const int q4 = lane >> 4, r16 = lane & 15;
  // unit id -> (row block, group): the row blocks of one (request, head, split) are
  // 8 ids apart (same XCD).  Groups are split-major: with a grid-stride schedule,
  // every workgroup's first units are first splits (the longest, present for every
  // request), and no workgroup is tied to one split index.
  const int slot = v >> 3;
  const int rb = slot % a.ctx_row_blocks;
  const int grp = (v & 7) + 8 * (slot / a.ctx_row_blocks);
  const int per_split = a.batch * a.num_kv_heads;
  const int split = grp / per_split;
  const int h = grp % a.num_kv_heads;
  if (split >= a.ctx_max_splits) return;  // padding unit

  // Clamped per-request sizes: bad inputs cannot move an access out of bounds.
  const int cap = min(a.max_ctx_len, a.max_blocks_per_seq * kTile);
  const int c = min(max(__builtin_amdgcn_readlane(m.raw, 0), 0), cap);
  const int b = (grp % per_split) / a.num_kv_heads;
  int qs = b, nq = 1;
  if (a.cu_q_lens) {
    qs = min(max(__builtin_amdgcn_readlane(m.raw, 1), 0), a.total_q);
    nq = min(max(__builtin_amdgcn_readlane(m.raw, 2) - qs, 0), a.total_q - qs);
  }
  const int R = nq * a.group;
  const int row0 = rb * RT * 16;
  if (row0 >= R) return;  // no rows in this block: uniform over the workgroup
  const int key_begin = split * a.ctx_split_len;
  const int key_end = min(key_begin + a.ctx_split_len, c);

  size_t qrow[RT];
  int last[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row0 + rt * 16 + r16;
    const int tl = row / a.group, gi = row % a.group;
    qrow[rt] = (size_t)(qs + tl) * a.num_q_heads + (size_t)h * a.group + gi;
    last[rt] = row < R ? c - nq + tl : -1;
  }
  if (key_begin >= c) {  // split past the context: an empty partial
    if (kl == 0 && q4 == 0) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
        if (last[rt] >= 0) a.ctx_lse[(size_t)split * a.total_q * a.num_q_heads + qrow[rt]] = neg_inf();
    }
    return;
  }

  int pt = m.pt;
  u32x4 qf[RT][NCH];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) load_q_tile<T, D>(qf[rt], a.q, qrow[rt], last[rt] >= 0);
  pt = min(max(pt, 0), a.num_blocks - 1);
  RowState<D> st[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) st[rt].init();

  const size_t page_stride = (size_t)a.num_kv_heads * kTile * D * E;
  const char* kbase = static_cast<const char*>(a.ctx_k) + (size_t)h * kTile * D * E;
  const char* vbase = static_cast<const char*>(a.ctx_v) + (size_t)h * D * kTile * E;
  // step s covers the split's pages 2s and 2s + 1 (page ids broadcast from lane 2s,
  // 2s + 1); a page past the split's end re-reads the last one (its keys are masked)
  const int npages = (key_end - key_begin + kTile - 1) / kTile;
  const int nsteps = (npages + 1) / 2;
  auto addr = [&](int st_) {
    const int ba = __builtin_amdgcn_readlane(pt, 2 * st_);
    const int bb = __builtin_amdgcn_readlane(pt, min(2 * st_ + 1, npages - 1));
    StepAddr r;
    r.ka = kbase + (size_t)ba * page_stride;
    r.kb = kbase + (size_t)bb * page_stride;
    r.va = vbase + (size_t)ba * page_stride;
    r.vb = vbase + (size_t)bb * page_stride;
    return r;
  };
  // the unit's first row sees the fewest of its keys (causal bound c - n_b + t): P is
  // split when that row sees few, whatever the unit's length
  const int first_seen = min(key_end, c - nq + row0 / a.group + 1) - key_begin;
  if (first_seen < kPSplitBelow)
    stream_pipelined<T, D, RT, WK, true>(kl, nsteps, qf, st, key_begin, key_end, last, a.scale_log2, addr);
  else
    stream_pipelined<T, D, RT, WK, false>(kl, nsteps, qf, st, key_begin, key_end, last, a.scale_log2, addr);
  merge_key_lanes<D, RT, WK>(st, kl, lds);

  if (kl == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float* orow = nullptr;
      float* lrow = nullptr;
      if (last[rt] >= 0) {
        const size_t r = (size_t)split * a.total_q * a.num_q_heads + qrow[rt];
        orow = a.ctx_o + r * D;
        lrow = a.ctx_lse + r;
      }
      store_row_tile(st[rt], orow, lrow);
    }
  }
}

// Row tiles of the widest unit a kernel runs: its context row tiles, and with four key
// lanes also the two-tile system units.
template <int RT, int WK>
constexpr int merge_row_tiles() {
  return (WK == 4 && RT < 2) ? 2 : RT;
}

template <int D, int RT, int WK>
constexpr size_t units_lds_bytes() {
  return WK > 1 ? sizeof(float) * (size_t)(WK / 2) * kMergeSlot<D, merge_row_tiles<RT, WK>()> : 0;
}

// ---- scheduling ---------------------------------------------------------------------
//
// The kernels are persistent: the grid is sized to what the GPU holds at once, so no
// workgroup waits to be dispatched.  Units are numbered with system units first (the
// longest), then context units split-major.  Round k hands units [kG, kG + G) to the
// G workgroups rotated by 8k: workgroup w takes kG + (w + 8k) mod G.  Each round is a
// bijection, each unit stays on its workgroup's XCD (unit mod 8, G a multiple of 8),
// and no workgroup is tied to one row block or split for the whole launch.  The
// sequence is known in advance, so the next context unit's metadata loads are issued
// while the current unit streams.  (Barriers inside a unit are reached by every wave
// of the workgroup: the sequence depends on blockIdx only.)

constexpr int kNoUnit = 0x7fffffff;

// Metadata of unit u when it is a context unit (else nothing is loaded).
template <int WHAT>
__device__ __forceinline__ CtxMeta meta_for(const UnitArgs& a, int u, int ns, int total) {
  if ((WHAT & kUnitsCtx) && u >= ns && u < total) return ctx_meta(a, u - ns);
  return CtxMeta{0, 0};
}

template <typename T, int D, int RT, int WK, int WHAT>
__device__ __forceinline__ void run_units(const UnitArgs& a, float* lds) {
  const int ns = (WHAT & kUnitsSys) ? a.n_sys_units : 0;
  const int total = ns + ((WHAT & kUnitsCtx) ? a.n_ctx_units : 0);
  const int G = gridDim.x;
  int u = blockIdx.x < total ? (int)blockIdx.x : kNoUnit;
  int soff = (int)((blockIdx.x + 8) % G);
  int sbase = G;
  int un = sbase + soff < total ? sbase + soff : kNoUnit;
  CtxMeta m = meta_for<WHAT>(a, u, ns, total);
  while (u != kNoUnit) {
    const CtxMeta mn = meta_for<WHAT>(a, un, ns, total);
    if ((WHAT & kUnitsSys) && u < ns) {
      if (WK == 4 && a.sys_rt == 2) sys_unit<T, D, merge_row_tiles<1, WK>(), WK>(a, u, lds);
      else sys_unit<T, D, 1, WK>(a, u, lds);
    }
    else if (WHAT & kUnitsCtx) ctx_unit<T, D, RT, WK>(a, u - ns, m, lds);
    sbase += G;
    soff = (soff + 8) % G;
    u = un;
    un = sbase + soff < total ? sbase + soff : kNoUnit;
    m = mn;
  }
}

// Waves per SIMD the unit kernels are built for: two for bf16 (one or two row tiles fit
// 256 registers without spilling, and a second workgroup per CU keeps the memory
// streams of two units in flight), one for fp32 with one step in registers.
template <typename T, int RT>
constexpr int units_waves_per_simd() {
  return Elem<T>::kBytes == 2 ? 2 : stream_depth<T, RT>();
}

// The system-attention step alone (at most 64 stacked rows: row tiles as units).
template <typename T, int D, int WK>
__global__ __launch_bounds__(kWave* WK, (units_waves_per_simd<T, 1>())) void sys_attn_kernel(UnitArgs a) {
  extern __shared__ float lds[];
  run_units<T, D, 1, WK, kUnitsSys>(a, lds);
}

// The context-attention step alone.
template <typename T, int D, int RT, int WK>
__global__ __launch_bounds__(kWave* WK, (units_waves_per_simd<T, RT>())) void ctx_attn_kernel(UnitArgs a) {
  extern __shared__ float lds[];
  run_units<T, D, RT, WK, kUnitsCtx>(a, lds);
}

// Both steps in one launch.
template <typename T, int D, int RT, int WK>
__global__ __launch_bounds__(kWave* WK, (units_waves_per_simd<T, RT>())) void sys_ctx_attn_kernel(UnitArgs a) {
  extern __shared__ float lds[];
  run_units<T, D, RT, WK, kUnitsBoth>(a, lds);
}

// Workgroups of kernel `k` that one CU holds at once.
static int blocks_per_cu(const void* k, int threads, size_t lds) {
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, threads, lds) != hipSuccess || per_cu < 1)
    per_cu = 1;
  return per_cu;
}

template <typename T, int D, int RT, int WK>
static hipError_t launch_units_t(const UnitArgs& a, int what, hipStream_t s) {
  constexpr size_t lds = units_lds_bytes<D, RT, WK>();
  static_assert(lds <= 64 * 1024, "LDS budget");
  const void* k;
  int units;
  if (what == kUnitsSys) {
    k = reinterpret_cast<const void*>(&sys_attn_kernel<T, D, WK>);
    units = a.n_sys_units;
  } else if (what == kUnitsCtx) {
    k = reinterpret_cast<const void*>(&ctx_attn_kernel<T, D, RT, WK>);
    units = a.n_ctx_units;
  } else {
    k = reinterpret_cast<const void*>(&sys_ctx_attn_kernel<T, D, RT, WK>);
    units = a.n_sys_units + a.n_ctx_units;
  }
  // occupancy of each kernel, queried once
  static std::atomic<int> cached[4];
  int per_cu = cached[what].load(std::memory_order_relaxed);
  if (per_cu == 0) {
    per_cu = blocks_per_cu(k, kWave * WK, lds);
    cached[what].store(per_cu, std::memory_order_relaxed);
  }
  const long long cap = 256LL * per_cu;
  long long grid = a.grid > 0 ? a.grid : (units < cap ? units : cap);
  if (grid > units) grid = units;
  if (grid < 1) grid = 1;
  const dim3 g((unsigned)grid), b(kWave * WK);
  if (what == kUnitsSys)
    hipLaunchKernelGGL((sys_attn_kernel<T, D, WK>), g, b, lds, s, a);
  else if (what == kUnitsCtx)
    hipLaunchKernelGGL((ctx_attn_kernel<T, D, RT, WK>), g, b, lds, s, a);
  else
    hipLaunchKernelGGL((sys_ctx_attn_kernel<T, D, RT, WK>), g, b, lds, s, a);
  return hipGetLastError();
}

// Instantiated: 4 key lanes (8 for one row tile).
template <typename T, int D, int RT>
static hipError_t launch_units_w(const UnitArgs& a, int what, hipStream_t s) {
  if constexpr (RT == 1) {
    if (a.key_lanes == 8) return launch_units_t<T, D, RT, 8>(a, what, s);
  }
  return launch_units_t<T, D, RT, 4>(a, what, s);
}

template <typename T, int D>
static hipError_t launch_units_d(const UnitArgs& a, int rt, int what, hipStream_t s) {
  return rt == 1 ? launch_units_w<T, D, 1>(a, what, s) : launch_units_w<T, D, 2>(a, what, s);
}

hipError_t launch_attn_units(const UnitArgs& a, int ctx_rt, int what, int in_dtype, int head_dim,
                             hipStream_t stream) {
  if (a.key_lanes != 4 && a.key_lanes != 8) return hipErrorInvalidValue;
  if (in_dtype == 1) {
    return head_dim == 64 ? launch_units_d<bf16_t, 64>(a, ctx_rt, what, stream)
                          : launch_units_d<bf16_t, 128>(a, ctx_rt, what, stream);
  }
  return head_dim == 64 ? launch_units_d<float, 64>(a, ctx_rt, what, stream)
                        : launch_units_d<float, 128>(a, ctx_rt, what, stream);
}

}  // namespace relay
