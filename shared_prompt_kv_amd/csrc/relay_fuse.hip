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
// load per partial); 256 threads per workgroup.  HBM-bound; the loads of a row's
// partials are issued in batches of four so a row costs few memory latencies.
#include "relay_device.hpp"
#include "relay_internal.hpp"

namespace relay {

template <int D>
__global__ __launch_bounds__(256) void relay_fuse_kernel(FuseArgs a) {
  constexpr int LPR = D / 4;         // lanes per row
  constexpr int RPW = 256 / LPR;     // rows per workgroup
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
  // pass 1: the largest LSE and a live partial (16 loads in flight per batch)
  constexpr int kL = 16;
  float mx = neg_inf();
  int live0 = -1;
  for (int i0 = 0; i0 < n; i0 += kL) {
    float l[kL];
#pragma unroll
    for (int j = 0; j < kL; ++j) l[j] = *lse_at(min(i0 + j, n - 1));
#pragma unroll
    for (int j = 0; j < kL; ++j) {
      if (i0 + j < n && l[j] != neg_inf()) {
        mx = fmaxf(mx, l[j]);
        if (live0 < 0) live0 = i0 + j;
      }
    }
  }
  // pass 2: the weighted sum, 8 output loads in flight per batch; an empty partial
  // (LSE = -inf, its O possibly never written) reads the live one instead, weight 0
  constexpr int kB = 8;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float z = 0.f;
  if (live0 >= 0) {
    for (int i0 = 0; i0 < n; i0 += kB) {
      float l[kB], w[kB];
      f32x4 o[kB];
#pragma unroll
      for (int j = 0; j < kB; ++j) l[j] = *lse_at(min(i0 + j, n - 1));
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        const bool live = i0 + j < n && l[j] != neg_inf();
        w[j] = live ? fast_exp2((l[j] - mx) * kLog2e) : 0.f;
        o[j] = *o_at(live ? i0 + j : live0);
      }
#pragma unroll
      for (int j = 0; j < kB; ++j) {
        z += w[j];
        acc += w[j] * o[j];
      }
    }
    acc *= 1.f / z;
  }
  if (a.out_bf16) {
    uint32_t* o = reinterpret_cast<uint32_t*>(static_cast<char*>(a.out) + ((size_t)row * D + 4 * c4) * 2);
    o[0] = pack_bf16x2(acc.x, acc.y);
    o[1] = pack_bf16x2(acc.z, acc.w);
  } else {
    *reinterpret_cast<f32x4*>(static_cast<float*>(a.out) + (size_t)row * D + 4 * c4) = acc;
  }
  if (a.lse_out && c4 == 0) a.lse_out[row] = (live0 < 0) ? neg_inf() : mx + __builtin_amdgcn_logf(z) * kLn2;
}

hipError_t launch_relay_fuse(const FuseArgs& a, int head_dim, int nwg, hipStream_t stream) {
  if (head_dim == 64)
    hipLaunchKernelGGL((relay_fuse_kernel<64>), dim3(nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((relay_fuse_kernel<128>), dim3(nwg), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace relay
