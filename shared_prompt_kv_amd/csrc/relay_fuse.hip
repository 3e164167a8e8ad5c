// relay_fuse: RelayAttention's relay-fusion step on gfx950.
//
// The final output is a weighted average, with non-negative weights summing to one,
// of the system-attention and context-attention outputs (atyun.com article, section
// "RelayAttention"; a single
// fused elementwise kernel in the linnk.ai summary, section "Abstract").  With
// LSE_i = ln sum_{j in part i} e^{s_j}, the weights e^{LSE_i} / sum_k e^{LSE_k} are
// non-negative, sum to one, and make the result equal attention over the union of
// the parts.  The same identity merges any number of parts, so the per-chunk
// partials of sys_attn and the per-split partials of ctx_attn are merged here in one
// pass: one read of every partial row, one write of the output.
//
// Layout: D/4 lanes per row, each owning four consecutive dimensions (one 16-byte
// load per partial); one wave per workgroup when there are few rows, so a few hundred
// rows still spread over the CUs, four when there are many.  HBM-bound.  One pass: the LSEs and outputs of a batch of partials are
// loaded together (one memory latency per batch) and folded into a running
// (max, weight sum, weighted sum) that is rescaled when the max grows.
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
// KV head h = hq / g; its system part is the pieces of KV head h's system stream (stacked
// row t g + hq % g of each piece; stream_attn wrote where they are) or the runs of the
// system kernel (slots 0 .. sys_runs - 1, LSE = -inf for a run that holds no key of h),
// and its context part is the pieces of its context stream (ctx_rowdesc[r]: first
// slot, count, row in the piece).  All of them are merged in one pass with the weights
// e^{LSE_i} / sum_k e^{LSE_k}: the relay fusion over every partial at once.  Where the
// pieces are comes first (one memory round trip), then their LSEs and outputs together.
template <int D, int THREADS>
__global__ __launch_bounds__(THREADS) void relay_merge_kernel(MergeArgs a) {
  constexpr int LPR = D / 4;
  constexpr int RPW = THREADS / LPR;
  const long long row = (long long)blockIdx.x * RPW + threadIdx.x / LPR;
  if (row >= a.n_rows) return;
  const int c4 = threadIdx.x % LPR;
  const int t = (int)(row / a.num_q_heads), hq = (int)(row - (long long)t * a.num_q_heads);
  const int h = hq / a.group;
  const int m = t * a.group + (hq - h * a.group);  // stacked row of KV head h
  // where the pieces are (clamped: stale or inconsistent descriptors cannot move a read
  // out of bounds)
  long long s_first = 0, c_first = 0;
  int s_count = 0, c_count = 0, c_row = 0;
  if (a.sys_src == 1) {
    s_first = min(max((long long)a.sys_desc[2 * h], 0LL), a.sys_slots - 1);
    s_count = (int)min(max((long long)a.sys_desc[2 * h + 1], 0LL), a.sys_slots - s_first);
  } else if (a.sys_src == 2) {
    s_count = a.sys_runs;
  }
  if (a.ctx_on) {
    const int4 d = *reinterpret_cast<const int4*>(a.ctx_rowdesc + 4 * row);
    c_first = min(max((long long)d.x, 0LL), a.ctx_slots - 1);
    c_count = (int)min(max((long long)d.y, 0LL), a.ctx_slots - c_first);
    c_row = min(max(d.z, 0), a.ctx_rows - 1);
  }
  const int n = s_count + c_count;
  auto lse_at = [&](int i) -> const float* {
    if (i < s_count) {
      return a.sys_src == 1 ? a.sys_lse + (size_t)(s_first + i) * a.sys_rows + m
                            : a.sys_lse + (size_t)i * a.n_rows + row;
    }
    return a.ctx_lse + (size_t)(c_first + i - s_count) * a.ctx_rows + c_row;
  };
  auto o_at = [&](int i) -> const f32x4* {
    const float* base;
    if (i < s_count) {
      base = a.sys_src == 1 ? a.sys_o + ((size_t)(s_first + i) * a.sys_rows + m) * D
                            : a.sys_o + ((size_t)i * a.n_rows + row) * D;
    } else {
      base = a.ctx_o + ((size_t)(c_first + i - s_count) * a.ctx_rows + c_row) * D;
    }
    return reinterpret_cast<const f32x4*>(base + 4 * c4);
  };
  // running state in the log2 domain (as relay_fuse_kernel); an empty partial (LSE =
  // -inf) has weight 0 and its O is selected away
  constexpr int kB = 8;
  float mx = neg_inf(), z = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int i0 = 0; i0 < n; i0 += kB) {
    float l[kB];
    f32x4 o[kB];
#pragma unroll
    for (int j = 0; j < kB; ++j) {
      const int i = min(i0 + j, n - 1);
      l[j] = *lse_at(i) * kLog2e;
      o[j] = *o_at(i);
    }
    float bm = mx;
#pragma unroll
    for (int j = 0; j < kB; ++j)
      if (i0 + j < n) bm = fmaxf(bm, l[j]);
    if (bm == neg_inf()) continue;
    const float sc = fast_exp2(mx - bm);
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
    mx = bm;
  }
  acc *= (z > 0.f) ? 1.f / z : 0.f;
  if (a.out_bf16) {
    uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<char*>(a.out) + ((size_t)row * D + 4 * c4) * 2);
    o[0] = pack_bf16x2(acc.x, acc.y);
    o[1] = pack_bf16x2(acc.z, acc.w);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + (size_t)row * D + 4 * c4) = acc;
  }
  if (a.lse_out && c4 == 0) a.lse_out[row] = (z > 0.f) ? (mx + __builtin_amdgcn_logf(z)) * kLn2 : neg_inf();
}

hipError_t launch_relay_merge(const MergeArgs& a, int head_dim, hipStream_t stream, const LaunchTiming* tm) {
  const int threads = merge_threads(head_dim, a.n_rows);
  const long long per = threads / (head_dim / 4);
  const long long nwg = (a.n_rows + per - 1) / per;
  if (nwg < 1 || nwg >= (1LL << 31)) return hipErrorInvalidValue;
  if (head_dim == 64) {
    if (threads == 256) launch_kernel(relay_merge_kernel<64, 256>, dim3(nwg), dim3(256), 0, stream, tm, a);
    else launch_kernel(relay_merge_kernel<64, 64>, dim3(nwg), dim3(64), 0, stream, tm, a);
  } else {
    if (threads == 256) launch_kernel(relay_merge_kernel<128, 256>, dim3(nwg), dim3(256), 0, stream, tm, a);
    else launch_kernel(relay_merge_kernel<128, 64>, dim3(nwg), dim3(64), 0, stream, tm, a);
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
