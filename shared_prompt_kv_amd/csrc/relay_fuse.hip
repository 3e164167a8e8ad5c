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
