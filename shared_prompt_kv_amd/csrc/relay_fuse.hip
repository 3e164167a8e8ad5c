// relay_fuse: RelayAttention's relay-fusion step on gfx950.
//
// The final output is a weighted average, with non-negative weights summing to one,
// of the system-attention and context-attention outputs (atyun.com article, section
// "RelayAttention"; a single
// fused elementwise kernel in the linnk.ai summary, section "Abstract").  With
// LSE_i = ln sum_{j in part i} e^{s_j}, the weights e^{LSE_i} / sum_k e^{LSE_k} are
// non-negative, sum to one, and make the result equal attention over the union of
// the parts.  The same identity merges any number of parts, so the pieces of the
// system and context streams (or the system kernel's runs) are merged here in one
// pass: one read of every partial row, one write of the output.
//
// Layout: D/4 lanes per row, each owning four consecutive dimensions (one 16-byte
// load per partial); one wave per workgroup when there are few rows, so a few hundred
// rows still spread over the CUs, four when there are many.  One pass: the LSEs and
// outputs of a batch of partials are loaded together (one memory latency per batch)
// and folded into a running (max, weight sum, weighted sum) that is rescaled when the
// max grows.  Few rows: bound by memory latency; many: by HBM bandwidth.
#include "relay_device.hpp"
#include "relay_internal.hpp"

namespace relay {

// SKIP_EMPTY: an output row is loaded only when its LSE is finite.  With many slots that
// may be empty (long contexts split many ways, system runs of the matrix-core kernel)
// a good share of them are, and their outputs need not be read; the LSEs of a batch are then
// awaited before its outputs are loaded (one more memory latency per batch, covered
// by the other rows' waves when there are many rows).  With a few slots, all of them
// live, the outputs are loaded together with the LSEs.
template <int D, int THREADS, bool SKIP_EMPTY>
__global__ __launch_bounds__(THREADS) void relay_fuse_kernel(FuseArgs a) {
  constexpr int LPR = D / 4;           // lanes per row
  constexpr int RPW = THREADS / LPR;   // rows per workgroup
  const long long row = (long long)blockIdx.x * RPW + threadIdx.x / LPR;
  if (row >= a.n_rows) return;
  const int c4 = threadIdx.x % LPR;

  // partial i < a_count is system chunk i, the rest are context splits
  const int n = a.a_count + a.b_count;
  auto lse_at = [&](int i) -> const float* {
    return i < a.a_count ? a.a_lse + (size_t)i * a.n_rows + row
                         : a.b_lse + (size_t)(i - a.a_count) * a.n_rows + row;
  };
  auto o_at = [&](int i) -> const f32x4* {
    const float* base = i < a.a_count ? a.a_o + ((size_t)i * a.n_rows + row) * D
                                      : a.b_o + ((size_t)(i - a.a_count) * a.n_rows + row) * D;
    return reinterpret_cast<const f32x4*>(base + 4 * c4);
  };
  // running state in the log2 domain: m = max LSE so far, z = sum of 2^(LSE_i - m),
  // acc = sum of 2^(LSE_i - m) O_i.  An empty partial (LSE = -inf) has weight 0 and
  // its O, possibly never written, is selected away rather than multiplied by 0.
  constexpr int kB = 8;
  float m = neg_inf(), z = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < n; i0 += kB) {
    float l[kB];
    f32x4 o[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int i = min(i0 + j, n - 1);
      l[j] = *lse_at(i) * kLog2e;
      if constexpr (!SKIP_EMPTY) o[j] = *o_at(i);
    }
    if constexpr (SKIP_EMPTY) {
#pragma unroll
      for (int j = 0; j < kB; ++j)
        o[j] = (i0 + j < n && l[j] != neg_inf()) ? *o_at(i0 + j) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float bm = m;
#pragma unroll
    for (int j = 0; j < kB; ++j)
      if (i0 + j < n) bm = fmaxf(bm, l[j]);
    if (bm == neg_inf()) continue;  // nothing live yet
    const float sc = fast_exp2(m - bm);  // 0 while m = -inf
    z *= sc;
    acc *= sc;
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const bool live = i0 + j < n && l[j] != neg_inf();
      const float w = live ? fast_exp2(l[j] - bm) : 0.f;
      z += w;
      const f32x4 wo = w * o[j];
      acc += live ? wo : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    m = bm;
  }
  acc *= (z > 0.f) ? 1.f / z : 0.f;
  if (a.out_bf16) {
    uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<char*>(a.out) + ((size_t)row * D + 4 * c4) * 2);
    o[0] = pack_bf16x2(acc.x, acc.y);
    o[1] = pack_bf16x2(acc.z, acc.w);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + (size_t)row * D + 4 * c4) = acc;
  }
  if (a.lse_out && c4 == 0) a.lse_out[row] = (z > 0.f) ? (m + __builtin_amdgcn_logf(z)) * kLn2 : neg_inf();
}

// relay_merge: the decode step's final output.  Row r = (token t, query head hq) uses
// KV head h = hq / g.  Its system part is the pieces of KV head h's system stream
// (stacked row t g + hq % g of each piece) or the runs of the system kernel (slots
// 0 .. sys_runs - 1, LSE = -inf for a run that holds no key of h); its context part is
// the pieces of its context stream.  All of them are merged in one pass with the weights
// e^{LSE_i} / sum_k e^{LSE_k}: the relay fusion over every partial at once.
//
// Where the pieces are: the first ks system pieces of a KV head and the first kc context
// pieces of a row sit at places known before anything is read (system slots h ks + k, the
// row's own slots row_o); so do the system kernel's runs.  Those are loaded together with the descriptors that say how many
// pieces there are (sys_desc for the KV head, ctx_rowdesc for the row): one memory round
// trip.  Only pieces past the row's own slots need the descriptors' first slots, and a
// second round trip.
struct MergeState {
  float m, z;  // log2-domain max LSE so far, and sum of 2^(LSE_i - m)
  f32x4 acc;   // sum of 2^(LSE_i - m) O_i
};

// Folds the partials marked live (natural-log LSEs l) into s; an empty or unused one,
// whose O may never have been written, is selected away rather than multiplied by 0.
template <int N>
__device__ __forceinline__ void merge_fold(MergeState& s, const float (&l)[N], const f32x4 (&o)[N],
                                           const bool (&live)[N]) {
  float l2[N];
  float bm = s.m;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    l2[j] = l[j] * kLog2e;
    if (live[j]) bm = fmaxf(bm, l2[j]);
  }
  if (bm == neg_inf()) return;        // nothing live yet
  const float sc = fast_exp2(s.m - bm);  // 0 while m = -inf
  s.z *= sc;
  s.acc *= sc;
#pragma unroll
  for (int j = 0; j < N; ++j) {
    const float w = live[j] ? fast_exp2(l2[j] - bm) : 0.f;
    s.z += w;
    const f32x4 wo = w * o[j];
    s.acc += live[j] ? wo : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  s.m = bm;
}

// KMAX >= ks + kc pieces at fixed places are loaded (indices clamped to the last real
// one) without waiting on anything: the loads of the first round trip are issued
// together.  Every pointer the kernel reads is valid (the host points the unused
// descriptors at the row descriptors).
template <int D, int THREADS, int KMAX>
__global__ __launch_bounds__(THREADS) void relay_merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 4;
  constexpr int RPW = THREADS / LPR;
  const long long row = (long long)blockIdx.x * RPW + threadIdx.x / LPR;
  if (row >= a.n_rows) return;
  const int c4 = threadIdx.x % LPR;
  const int t = (int)(row / a.num_q_heads), hq = (int)(row - (long long)t * a.num_q_heads);
  const int h = hq / a.group;
  const int m = t * a.group + (hq - h * a.group);  // stacked row of KV head h

  // ---- one round trip: the descriptors and the pieces at fixed places
  const int2 sd = *reinterpret_cast<const int2*>(a.sys_desc + 2 * h);
  const int4 cd = *reinterpret_cast<const int4*>(a.ctx_rowdesc + 4 * row);
  // fixed places: system slots h ks + k (row m of each), then this row's context slots
  const int K = a.ks + a.kc;
  float lr[KMAX > 0 ? KMAX : 1];
  f32x4 orr[KMAX > 0 ? KMAX : 1];
#pragma unroll
  for (int j = 0; j < KMAX; ++j) {
    const int q = min(j, K - 1);
    const bool sys = q < a.ks;
    const size_t r = sys ? ((size_t)h * a.ks + q) * a.sys_rows + m : (size_t)row * a.kc + (q - a.ks);
    lr[j] = (sys ? a.sys_lse : a.row_lse)[r];
    orr[j] = *reinterpret_cast<const f32x4*>((sys ? a.sys_o : a.row_o) + r * D + 4 * c4);
  }
  // how many pieces there are (clamped: stale or inconsistent descriptors cannot move a
  // read out of bounds)
  long long s_first = 0, c_first = 0;
  int s_count = 0, c_count = 0, c_row = 0;
  if (a.sys_src == 1) {
    s_first = min(max((long long)sd.x, 0LL), a.sys_slots - 1);
    s_count = (int)min(max((long long)sd.y, 0LL), a.sys_slots - s_first);
  }
  if (a.ctx_on) {
    c_first = min(max((long long)cd.x, 0LL), a.ctx_slots - 1);
    c_count = (int)min(max((long long)cd.y, 0LL), a.ctx_slots - c_first);
    c_row = min(max(cd.z, 0), a.ctx_rows - 1);
  }
  const int s_own = min(s_count, a.ks), c_own = min(c_count, a.kc);
  MergeState st{neg_inf(), 0.f, f32x4{0.f, 0.f, 0.f, 0.f}};
  if constexpr (KMAX > 0) {
    bool live[KMAX];
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
      live[j] = (j < a.ks ? j < s_own : j - a.ks < c_own) && lr[j] != neg_inf();
    merge_fold(st, lr, orr, live);
  }

  // ---- the rest: system pieces past the fixed slots, the system kernel's runs (their
  // places are fixed, but with many rows the merge is bound by bandwidth, not latency,
  // and they are read in as few batches as possible), context pieces past the row's
  // slots (in the stream slots the descriptors name)
  const int n_s = s_count - s_own, n_q = a.sys_src == 2 ? a.sys_runs : 0, n_c = c_count - c_own;
  const int n_over = n_s + n_q + n_c;
  auto over_at = [&](int i, const float** o) -> const float* {
    if (i < n_s) {
      const size_t r = (size_t)(s_first + s_own + i) * a.sys_rows + m;
      *o = a.sys_o + r * D;
      return a.sys_lse + r;
    }
    i -= n_s;
    if (i < n_q) {
      const size_t r = (size_t)i * a.n_rows + row;
      *o = a.sys_o + r * D;
      return a.sys_lse + r;
    }
    i -= n_q;
    const size_t r = (size_t)(c_first + c_own + i) * a.ctx_rows + c_row;
    *o = a.ctx_o + r * D;
    return a.ctx_lse + r;
  };
  constexpr int kB = 8;
  for (int i0 = 0; i0 < n_over; i0 += kB) {
    float l[kB];
    f32x4 o[kB];
    bool live[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const float* op;
      const float* lp = over_at(min(i0 + j, n_over - 1), &op);
      l[j] = *lp;
      o[j] = *reinterpret_cast<const f32x4*>(op + 4 * c4);
    }
#pragma unroll
    for (int j = 0; j < kB; ++j) live[j] = i0 + j < n_over && l[j] != neg_inf();
    merge_fold(st, l, o, live);
  }

  f32x4 acc = st.acc * ((st.z > 0.f) ? 1.f / st.z : 0.f);
  if (a.out_bf16) {
    uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<char*>(a.out) + ((size_t)row * D + 4 * c4) * 2);
    o[0] = pack_bf16x2(acc.x, acc.y);
    o[1] = pack_bf16x2(acc.z, acc.w);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + (size_t)row * D + 4 * c4) = acc;
  }
  if (a.lse_out && c4 == 0) a.lse_out[row] = (st.z > 0.f) ? (st.m + __builtin_amdgcn_logf(st.z)) * kLn2 : neg_inf();
}

// Instantiations: fixed places rounded up to 4, 8, 12 or 16 (none without them).
template <int D, int THREADS>
static void launch_merge_k(const MergeArgs& a, long long nwg, hipStream_t stream, const LaunchTiming* tm) {
  const int K = a.ks + a.kc;
  const dim3 g(nwg), b(THREADS);
  if (K == 0) launch_kernel(relay_merge_kernel<D, THREADS, 0>, g, b, 0, stream, tm, a);
  else if (K <= 4) launch_kernel(relay_merge_kernel<D, THREADS, 4>, g, b, 0, stream, tm, a);
  else if (K <= 8) launch_kernel(relay_merge_kernel<D, THREADS, 8>, g, b, 0, stream, tm, a);
  else if (K <= 12) launch_kernel(relay_merge_kernel<D, THREADS, 12>, g, b, 0, stream, tm, a);
  else launch_kernel(relay_merge_kernel<D, THREADS, kMaxRowSlots>, g, b, 0, stream, tm, a);
}

hipError_t launch_relay_merge(const MergeArgs& a, int head_dim, hipStream_t stream, const LaunchTiming* tm) {
  static_assert(kMaxRowSlots == 16, "row-slot instantiations");
  if (a.ks < 0 || a.kc < 0 || a.ks + a.kc > kMaxRowSlots || !a.sys_desc || !a.ctx_rowdesc)
    return hipErrorInvalidValue;
  const int threads = merge_threads(head_dim, a.n_rows);
  const long long per = threads / (head_dim / 4);
  const long long nwg = (a.n_rows + per - 1) / per;
  if (nwg < 1 || nwg >= (1LL << 31)) return hipErrorInvalidValue;
  if (head_dim == 64) {
    if (threads == 256) launch_merge_k<64, 256>(a, nwg, stream, tm);
    else launch_merge_k<64, 64>(a, nwg, stream, tm);
  } else {
    if (threads == 256) launch_merge_k<128, 256>(a, nwg, stream, tm);
    else launch_merge_k<128, 64>(a, nwg, stream, tm);
  }
  return hipGetLastError();
}

template <int D, bool SKIP>
static void launch_fuse_d(const FuseArgs& a, bool wide, int nwg, hipStream_t stream) {
  if (wide) hipLaunchKernelGGL((relay_fuse_kernel<D, 256, SKIP>), dim3(nwg), dim3(256), 0, stream, a);
  else hipLaunchKernelGGL((relay_fuse_kernel<D, 64, SKIP>), dim3(nwg), dim3(64), 0, stream, a);
}

hipError_t launch_relay_fuse(const FuseArgs& a, int head_dim, int nwg, hipStream_t stream) {
  const bool wide = fuse_threads(head_dim, a.n_rows) == 256;
  const bool skip = fuse_skips_empty(a);
  if (head_dim == 64) {
    if (skip) launch_fuse_d<64, true>(a, wide, nwg, stream);
    else launch_fuse_d<64, false>(a, wide, nwg, stream);
  } else {
    if (skip) launch_fuse_d<128, true>(a, wide, nwg, stream);
    else launch_fuse_d<128, false>(a, wide, nwg, stream);
  }
  return hipGetLastError();
}

}  // namespace relay
