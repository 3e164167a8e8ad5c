// sys_attn_tiled: RelayAttention's system-attention step on gfx950 for many stacked
// query rows (matrix-core-bound: large batch x GQA group).
//
// Every query row of the batch attends to the shared system KV cache alone
// (RelayAttention paper, abstract; atyun.com article, section "RelayAttention": the
// matrix-vector products against the system prompt of all requests become one
// matrix-matrix product, so the system K/V leave HBM once per batch).  For KV head
// h the M = T_q * g query rows that use it are stacked into one matrix and
// multiplied against the system keys on the matrix cores.
//
// Work split: the system keys of each KV head are cut into chunks; a workgroup owns
// (row block, chunk, KV head).  Inside it, WR row groups of RT*16 rows each and WK
// key lanes: wave (rg, kl) streams the 32-key steps kl, kl+WK, ... of the chunk for
// the rows of group rg.  With WK > 1 the waves of a row group merge their partial
// softmax states through LDS, so one chunk yields one partial (O, LSE) per row.
// Small batches (M <= 64) use WR = 1 and many key lanes: all waves share the rows
// and the chunk's K/V are read exactly once.  Large M uses several row groups over
// the same keys; their repeated K/V reads are served by the caches, and the grid is
// ordered so the workgroups that share a chunk run on the same XCD (one L2).
#include "relay_device.hpp"
#include "relay_internal.hpp"

namespace relay {

template <typename T, int D, int RT, int WK, int WR, bool PSPLIT>
__global__ __launch_bounds__(kWave* WK* WR) void sys_attn_tiled_kernel(SysArgs a) {
  constexpr int NCH = D * Elem<T>::kBytes / 64;  // 16-byte chunks per lane per row
  constexpr int E = Elem<T>::kBytes;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int rg = wave / WK;
  const int kl = wave % WK;
  const int q4 = lane >> 4;
  const int r16 = lane & 15;

  // XCD-aware order: consecutive logical ids (the row blocks sharing one chunk) are
  // placed on the same XCD.  Hardware assigns workgroup i to XCD i % 8.
  const int nwg = gridDim.x;
  int bid = blockIdx.x;
  if (a.xcd_remap) {
    const int per = nwg / 8;  // host guarantees nwg % 8 == 0 when remapping
    bid = (bid % 8) * per + bid / 8;
  }
  const int rb = bid % a.row_blocks;
  const int chunk = (bid / a.row_blocks) % a.n_chunks;
  const int h = bid / (a.row_blocks * a.n_chunks);

  const int M = a.total_q * a.group;
  const int row0 = (rb * WR + rg) * RT * 16;

  // Q^T fragments of this wave's row tiles (zero for padding rows).
  u32x4 qf[RT][NCH];
  int qrow[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int row = row0 + rt * 16 + r16;
    qrow[rt] = row;
    if (row < M) {
      const int t = row / a.group, i = row % a.group;
      const char* qp = static_cast<const char*>(a.q) +
                       ((size_t)t * a.num_q_heads + (size_t)h * a.group + i) * D * E;
#pragma unroll
      for (int kk = 0; kk < NCH; ++kk) qf[rt][kk] = ld16(qp + 64 * kk + 16 * q4);
    } else {
#pragma unroll
      for (int kk = 0; kk < NCH; ++kk) qf[rt][kk] = u32x4{0u, 0u, 0u, 0u};
    }
  }

  RowState<D> st[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) st[rt].init();

  const int Ls = a.sys_len;
  const int key_begin = chunk * a.chunk_len;
  const int key_end = min(key_begin + a.chunk_len, Ls);
  const int nsteps = (key_end - key_begin + kStep - 1) / kStep;
  const int ntile = (Ls + kTile - 1) / kTile;
  const char* kbase = static_cast<const char*>(a.sys_k) + (size_t)h * ntile * kTile * D * E;  // key tiles
  const char* vbase = static_cast<const char*>(a.sys_v) + (size_t)h * ntile * D * kTile * E;

  for (int s = kl; s < nsteps; s += WK) {
    const int key0 = key_begin + s * kStep;
    // keys of the two score tiles held by this lane's A-operand row
    const int ka = min(key0 + step_key_a(r16), Ls - 1);
    const int kb = min(key0 + step_key_b(r16), Ls - 1);
    u32x4 kfa[NCH], kfb[NCH];
#pragma unroll
    for (int kk = 0; kk < NCH; ++kk) {
      kfa[kk] = ld16(kbase + (size_t)(ka / kTile) * kTile * D * E + key_chunk_offset(key_slot(ka % kTile), 4 * kk + q4));
      kfb[kk] = ld16(kbase + (size_t)(kb / kTile) * kTile * D * E + key_chunk_offset(key_slot(kb % kTile), 4 * kk + q4));
    }
    // V^T fragments: keys key0 + 8*q4 .. +7 of every 16-dim tile
    const int vkey = key0 + 8 * q4;
    const int vtile = min(vkey / kTile, ntile - 1);
    const char* vrow = vbase + ((size_t)vtile * D * kTile + (vkey % kTile)) * E;
    VFrag<T> vf[D / 16];
#pragma unroll
    for (int t = 0; t < D / 16; ++t) load_v(vf[t], vrow + (size_t)(16 * t + r16) * kTile * E);
    const int nvalid = Ls - vkey;  // keys of this lane group that exist
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
        sc[i] = (vkey + i < Ls) ? sa[i] * a.scale_log2 : neg_inf();
        sc[4 + i] = (vkey + 4 + i < Ls) ? sb[i] * a.scale_log2 : neg_inf();
      }
      softmax_step(st[rt], sc);
      PFrag<T> pf;
      make_p<PSPLIT>(pf, sc);
#pragma unroll
      for (int t = 0; t < D / 16; ++t) mfma_pv<PSPLIT>(st[rt].o[t], vf[t], pf);
    }
  }

  // Merge the WK key lanes of each row group (fixed tree order: deterministic).
  if constexpr (WK > 1) {
    extern __shared__ float lds[];
    constexpr int kSlot = kWave * RT * (2 + D / 4);  // floats per slot
    for (int half = WK / 2; half >= 1; half /= 2) {
      __syncthreads();
      if (kl >= half && kl < 2 * half) {
        float* slot = lds + (size_t)(rg * (WK / 2) + (kl - half)) * kSlot;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          float* p = slot + rt * kWave * (2 + D / 4);
          p[lane] = st[rt].m;
          p[kWave + lane] = st[rt].l;
#pragma unroll
          for (int t = 0; t < D / 16; ++t)
            *reinterpret_cast<f32x4*>(p + 2 * kWave + (t * kWave + lane) * 4) = st[rt].o[t];
        }
      }
      __syncthreads();
      if (kl < half) {
        const float* slot = lds + (size_t)(rg * (WK / 2) + kl) * kSlot;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          const float* p = slot + rt * kWave * (2 + D / 4);
          f32x4 ob[D / 16];
#pragma unroll
          for (int t = 0; t < D / 16; ++t)
            ob[t] = *reinterpret_cast<const f32x4*>(p + 2 * kWave + (t * kWave + lane) * 4);
          merge_state(st[rt], p[lane], p[kWave + lane], ob);
        }
      }
    }
  }

  if (kl == 0) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const int row = qrow[rt];
      float* orow = nullptr;
      float* lrow = nullptr;
      if (row < M) {
        const int t = row / a.group, i = row % a.group;
        const size_t r = ((size_t)chunk * a.total_q + t) * a.num_q_heads + (size_t)h * a.group + i;
        orow = a.o_part + r * D;
        lrow = a.lse_part + r;
      }
      store_row_tile(st[rt], orow, lrow);
    }
  }
}

template <typename T, int D, int RT, int WK, int WR, bool PSPLIT>
static hipError_t launch_sys_t(const SysArgs& a, int nwg, hipStream_t stream, const LaunchTiming* tm) {
  constexpr size_t lds = (WK > 1) ? sizeof(float) * (size_t)WR * (WK / 2) * kWave * RT * (2 + D / 4) : 0;
  static_assert(lds <= 64 * 1024, "LDS budget");
  launch_kernel(sys_attn_tiled_kernel<T, D, RT, WK, WR, PSPLIT>, dim3(nwg), dim3(kWave * WK * WR), (uint32_t)lds,
                stream, tm, a);
  return hipGetLastError();
}

// The tiled kernel runs the system step for more than 64 stacked rows per KV head when
// the inputs are fp32 or head_dim is 64 (bf16 at head_dim 128 has sys_attn_mfma): row
// groups of 2 tiles, 4 per workgroup.  bf16 P goes to the output product as hi + lo: a
// single rounding costs up to 2^-9 of a probability, too much where one key holds much
// of a row's weight.
template <typename T, int D>
static hipError_t launch_sys_d(const SysArgs& a, const SysConfig& c, int nwg, hipStream_t s, const LaunchTiming* tm) {
  if (c.rt != 2 || c.wk != 1 || c.wr != 4) return hipErrorInvalidValue;
  return launch_sys_t<T, D, 2, 1, 4, true>(a, nwg, s, tm);
}

hipError_t launch_sys_attn_tiled(const SysArgs& a, const SysConfig& c, int in_dtype, int head_dim,
                                 int nwg, hipStream_t stream, const LaunchTiming* tm) {
  if (in_dtype == 1) {
    return head_dim == 64 ? launch_sys_d<bf16_t, 64>(a, c, nwg, stream, tm)
                          : launch_sys_d<bf16_t, 128>(a, c, nwg, stream, tm);
  }
  return head_dim == 64 ? launch_sys_d<float, 64>(a, c, nwg, stream, tm)
                        : launch_sys_d<float, 128>(a, c, nwg, stream, tm);
}

}  // namespace relay
