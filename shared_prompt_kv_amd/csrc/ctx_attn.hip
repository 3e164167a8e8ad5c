// ctx_attn: RelayAttention's context-attention step on gfx950.
//
// Each request attends to its own context alone, causally (atyun.com article,
// section "RelayAttention"; the context lives in a paged KV cache addressed through
// block tables, as in PagedAttention, linnk.ai summary, section "Abstract").  Query
// token t of request b sits at context position p = c_b - n_b + t and sees context
// keys 0..p.
//
// Work split: a workgroup owns (row block, split, KV head, request).  A split is a
// fixed run of context keys, so every workgroup streams at most split_len keys and
// long and short requests balance.  Its WR waves take disjoint groups of RT*16 of
// the request's g*n_b query rows and stream the same pages (the second and later
// reads hit the CU's L1), so each page leaves HBM once per request.  Both score and
// output products run on the matrix cores with rows padded to 16; the decode step
// stays bound by HBM, so P is fed to the output product as bf16 P_hi + P_lo (two
// MFMAs) at no cost in time, keeping fp32-level accuracy for short contexts whose
// few keys carry large softmax weights.  One split yields one partial (O, LSE) per row; relay_fuse
// merges the splits together with the system chunks.
#include "relay_device.hpp"
#include "relay_internal.hpp"

namespace relay {

template <typename T, int D, int RT, int WR>
__global__ __launch_bounds__(kWave* WR) void ctx_attn_kernel(CtxArgs a) {
  constexpr int NCH = D * Elem<T>::kBytes / 64;
  constexpr int E = Elem<T>::kBytes;
  const int lane = lane_id();
  const int rg = threadIdx.x / kWave;
  const int q4 = lane >> 4;
  const int r16 = lane & 15;

  int bid = blockIdx.x;
  const int rb = bid % a.row_blocks;
  bid /= a.row_blocks;
  const int split = bid % a.max_splits;
  bid /= a.max_splits;
  const int h = bid % a.num_kv_heads;
  const int b = bid / a.num_kv_heads;

  // Clamped per-request sizes: bad inputs cannot move an access out of bounds.
  const int cap = min(a.max_ctx_len, a.max_blocks_per_seq * kTile);
  const int c = min(max(a.ctx_lens[b], 0), cap);
  int qs = b, nq = 1;
  if (a.cu_q_lens) {
    qs = min(max(a.cu_q_lens[b], 0), a.total_q);
    nq = min(max(a.cu_q_lens[b + 1] - qs, 0), a.total_q - qs);
  }
  const int key_begin = split * a.split_len;
  if (key_begin >= c) return;
  const int key_end = min(key_begin + a.split_len, c);
  const int R = nq * a.group;
  const int row0 = (rb * WR + rg) * RT * 16;
  if (row0 >= R) return;

  u32x4 qf[RT][NCH];
  int prow[RT];
  size_t orow_idx[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row0 + rt * 16 + r16;
    if (row < R) {
      const int tl = row / a.group, i = row % a.group;
      const size_t r = (size_t)(qs + tl) * a.num_q_heads + (size_t)h * a.group + i;
      orow_idx[rt] = r;
      prow[rt] = c - nq + tl;
      const char* qp = static_cast<const char*>(a.q) + r * D * E;
#pragma unroll
      for (int kk = 0; kk < NCH; ++kk) qf[rt][kk] = ld16(qp + 64 * kk + 16 * q4);
    } else {
      orow_idx[rt] = ~(size_t)0;
      prow[rt] = -1;
#pragma unroll
      for (int kk = 0; kk < NCH; ++kk) qf[rt][kk] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  RowState<D> st[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) st[rt].init();

  const int32_t* bt = a.block_tables + (size_t)b * a.max_blocks_per_seq;
  const int npages = (c + kTile - 1) / kTile;
  const size_t page_stride = (size_t)a.num_kv_heads * kTile * D * E;  // bytes per page
  const char* kbase = static_cast<const char*>(a.ctx_k) + (size_t)h * kTile * D * E;
  const char* vbase = static_cast<const char*>(a.ctx_v) + (size_t)h * D * kTile * E;
  const int ja = step_key_a(r16), jb = step_key_b(r16);

  for (int key0 = key_begin; key0 < key_end; key0 += kStep) {
    const int pg0 = key0 / kTile;
    const int blk0 = min(max(bt[pg0], 0), a.num_blocks - 1);
    const int blk1 = (pg0 + 1 < npages) ? min(max(bt[pg0 + 1], 0), a.num_blocks - 1) : blk0;
    const char* ka = kbase + (size_t)(ja < kTile ? blk0 : blk1) * page_stride + (size_t)(ja % kTile) * D * E;
    const char* kb = kbase + (size_t)(jb < kTile ? blk0 : blk1) * page_stride + (size_t)(jb % kTile) * D * E;
    u32x4 kfa[NCH], kfb[NCH];
#pragma unroll
    for (int kk = 0; kk < NCH; ++kk) {
      kfa[kk] = ld16(ka + 64 * kk + 16 * q4);
      kfb[kk] = ld16(kb + 64 * kk + 16 * q4);
    }
    const char* vrow = vbase + (size_t)(q4 < 2 ? blk0 : blk1) * page_stride + (size_t)(8 * (q4 & 1)) * E;
    VFrag<T> vf[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) load_v(vf[t], vrow + (size_t)(16 * t + r16) * kTile * E);
    const int vkey = key0 + 8 * q4;
    const int nvalid = c - vkey;
    if (nvalid < 8) {
#pragma unroll
      for (int t = 0; t < D / 16; ++t) mask_v(vf[t], nvalid);
    }

#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < NCH; ++kk) {
        mfma_chunk(sa, kfa[kk], qf[rt][kk], T{});
        mfma_chunk(sb, kfb[kk], qf[rt][kk], T{});
      }
      float sc[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[i] = (vkey + i <= prow[rt]) ? sa[i] * a.scale_log2 : neg_inf();
        sc[4 + i] = (vkey + 4 + i <= prow[rt]) ? sb[i] * a.scale_log2 : neg_inf();
      }
      softmax_step(st[rt], sc);
      PFrag<T> pf;
      make_p<true>(pf, sc);
#pragma unroll
      for (int t = 0; t < D / 16; ++t) mfma_pv<true>(st[rt].o[t], vf[t], pf);
    }
  }

#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float* orow = nullptr;
    float* lrow = nullptr;
    if (orow_idx[rt] != ~(size_t)0) {
      const size_t r = (size_t)split * a.total_q * a.num_q_heads + orow_idx[rt];
      orow = a.o_part + r * D;
      lrow = a.lse_part + r;
    }
    store_row_tile(st[rt], orow, lrow);
  }
}

template <typename T, int D, int RT, int WR>
static hipError_t launch_ctx_t(const CtxArgs& a, int nwg, hipStream_t stream) {
  hipLaunchKernelGGL((ctx_attn_kernel<T, D, RT, WR>), dim3(nwg), dim3(kWave * WR), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_ctx_d(const CtxArgs& a, const CtxConfig& c, int nwg, hipStream_t s) {
  if (c.rt == 1) return launch_ctx_t<T, D, 1, 1>(a, nwg, s);
  if (c.wr == 1) return launch_ctx_t<T, D, 2, 1>(a, nwg, s);
  if (c.wr == 2) return launch_ctx_t<T, D, 2, 2>(a, nwg, s);
  return launch_ctx_t<T, D, 2, 4>(a, nwg, s);
}

hipError_t launch_ctx_attn(const CtxArgs& a, const CtxConfig& c, int in_dtype, int head_dim,
                           int nwg, hipStream_t stream) {
  if (in_dtype == 1) {
    return head_dim == 64 ? launch_ctx_d<bf16_t, 64>(a, c, nwg, stream)
                          : launch_ctx_d<bf16_t, 128>(a, c, nwg, stream);
  }
  return head_dim == 64 ? launch_ctx_d<float, 64>(a, c, nwg, stream)
                        : launch_ctx_d<float, 128>(a, c, nwg, stream);
}

}  // namespace relay
