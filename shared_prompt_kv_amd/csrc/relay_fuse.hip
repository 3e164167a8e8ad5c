// relay_fuse: RelayAttention's relay-fusion step on gfx950.
//
// The final output is a convex combination of the system-attention and
// context-attention outputs (atyun.com article, section "RelayAttention"; a single
// fused elementwise kernel in the linnk.ai summary, section "Abstract").  With
// LSE_i = ln sum_{j in part i} e^{s_j}, the weights e^{LSE_i} / sum_k e^{LSE_k} are
// non-negative, sum to one, and make the result equal attention over the union of
// the parts.  The same identity merges any number of parts, so the per-chunk
// partials of sys_attn and the per-split partials of ctx_attn are merged here in one
// pass: one read of every partial row, one write of the output.
//
// Layout: D/4 lanes per row, each owning four consecutive dimensions (one 16-byte
// load per partial); 256 threads per workgroup.  HBM-bound.
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

  int nb = a.b_count;
  if (a.b_split_len > 0) {
    const int t = (int)(row / a.num_q_heads);
    int b = t;
    if (a.cu_q_lens) {  // last request whose first token is <= t
      int lo = 0, hi = a.batch - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (a.cu_q_lens[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      b = lo;
    }
    const int c = max(a.ctx_lens[b], 0);
    nb = min((c + a.b_split_len - 1) / a.b_split_len, a.b_count);
  }

  float m = neg_inf();
  for (int i = 0; i < a.a_count; ++i) m = fmaxf(m, a.a_lse[(size_t)i * a.n_rows + row]);
  for (int i = 0; i < nb; ++i) m = fmaxf(m, a.b_lse[(size_t)i * a.n_rows + row]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float z = 0.f;
  if (m != neg_inf()) {
    for (int i = 0; i < a.a_count; ++i) {
      const size_t r = (size_t)i * a.n_rows + row;
      const float w = fast_exp2((a.a_lse[r] - m) * kLog2e);
      z += w;
      acc += w * *reinterpret_cast<const f32x4*>(a.a_o + r * D + 4 * c4);
    }
    for (int i = 0; i < nb; ++i) {
      const size_t r = (size_t)i * a.n_rows + row;
      const float w = fast_exp2((a.b_lse[r] - m) * kLog2e);
      z += w;
      acc += w * *reinterpret_cast<const f32x4*>(a.b_o + r * D + 4 * c4);
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
  if (a.lse_out && c4 == 0) a.lse_out[row] = (m == neg_inf()) ? m : m + __builtin_amdgcn_logf(z) * kLn2;
}

hipError_t launch_relay_fuse(const FuseArgs& a, int head_dim, int nwg, hipStream_t stream) {
  if (head_dim == 64)
    hipLaunchKernelGGL((relay_fuse_kernel<64>), dim3(nwg), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((relay_fuse_kernel<128>), dim3(nwg), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace relay
