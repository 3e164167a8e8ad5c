// The step before the relay path on gfx950: rotary position embedding with context
// positions offset by the system length, and the append of a decode step's new
// tokens to the paged context cache.
//
// The system K/V are prefilled offline at positions 0 .. L_s - 1, so a request's own
// tokens are placed after them: context token j is at absolute position L_s + j
// (atyun.com article, section "RelayAttention"; linnk.ai summary, section "Deeper
// Inquiries").  The embedding is RoPE in rotate-half form (the Llama family's): for
// i < d/2 the pair (x[i], x[i + d/2]) is rotated by the angle p * base^(-2i/d).  The
// cos/sin of every (position, i) come from a table [max_pos, d] fp32 (cos in the
// first d/2 columns, sin in the last), built once by relay_rope_table with the angle
// reduced in fp64.
//
// Elementwise and HBM-bound (a few KB per token): d/2 lanes per (token, head) row,
// lane i rotating the pair (i, i + d/2), and kRopeThreads / (d/2) rows per workgroup
// (a prefill embeds thousands of tokens: one small workgroup per row would leave the
// launch bound by workgroup dispatch).
#include "relay_device.hpp"
#include "relay_internal.hpp"

namespace relay {

// Element index of head dimension c of key r (0..15) inside a 16-key tile of keys:
// tiles are chunk-major (16-byte chunks of 8 bf16 / 4 fp32 elements), keys in slot
// order (key_slot).
__device__ __forceinline__ size_t key_tile_elem(int r, int c, int bf16) {
  const int g = bf16 ? 8 : 4;
  return ((size_t)(c / g) * kTile + key_slot(r)) * g + c % g;
}

__device__ __forceinline__ float rope_load(const void* p, size_t i, int bf16) {
  if (bf16) return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  return static_cast<const float*>(p)[i];
}

__device__ __forceinline__ void rope_store(void* p, size_t i, float v, int bf16) {
  if (bf16) static_cast<__bf16*>(p)[i] = static_cast<__bf16>(v);  // round to nearest even
  else static_cast<float*>(p)[i] = v;
}

__global__ void rope_table_kernel(float* cos_sin, int max_pos, int d, double base) {
  const int pos = blockIdx.x;
  const int half = d / 2;
  for (int i = threadIdx.x; i < half; i += blockDim.x) {
    const double a = (double)pos * pow(base, -2.0 * i / d);
    cos_sin[(size_t)pos * d + i] = (float)cos(a);
    cos_sin[(size_t)pos * d + half + i] = (float)sin(a);
  }
}

constexpr int kRopeThreads = 256;

// New token t (row t of q_new) of request b sits at context position
// p = c_b - n_b + t_local, absolute position L_s + p.  Rows (heads of the token):
// row < H_q are query heads (rotated into q_out), the rest KV heads (K rotated and V
// copied into page block_tables[b][p / 16], slot p % 16).  Rows whose position or page
// is out of range are skipped (nothing written).
__global__ __launch_bounds__(kRopeThreads) void rope_append_kernel(RopeArgs a) {
  const int half = a.head_dim / 2, d = a.head_dim;
  const int b = blockIdx.x, tl = blockIdx.y;
  const int row = blockIdx.z * (kRopeThreads / half) + threadIdx.x / half;
  const int i = threadIdx.x % half;
  if (row >= a.num_q_heads + a.num_kv_heads) return;
  int qs = b, nq = 1;
  if (a.cu_q_lens) {
    qs = a.cu_q_lens[b];
    nq = a.cu_q_lens[b + 1] - qs;
  }
  if (tl >= nq || qs < 0 || qs + tl >= a.total_q) return;
  const int t = qs + tl;
  const int p = a.ctx_lens[b] - nq + tl;  // context position
  const long long pos = (long long)a.sys_len + p;
  if (p < 0 || pos >= a.max_pos) return;
  const float c = a.cos_sin[pos * d + i], s = a.cos_sin[pos * d + half + i];
  if (row < a.num_q_heads) {
    const size_t base = ((size_t)t * a.num_q_heads + row) * d;
    const float x1 = rope_load(a.q_new, base + i, a.bf16), x2 = rope_load(a.q_new, base + half + i, a.bf16);
    rope_store(a.q_out, base + i, x1 * c - x2 * s, a.bf16);
    rope_store(a.q_out, base + half + i, x2 * c + x1 * s, a.bf16);
    return;
  }
  const int hk = row - a.num_q_heads;
  if (p / kTile >= a.max_blocks_per_seq) return;
  const int page = a.block_tables[(size_t)b * a.max_blocks_per_seq + p / kTile];
  if (page < 0 || page >= a.num_blocks) return;
  const int slot = p % kTile;
  const size_t src = ((size_t)t * a.num_kv_heads + hk) * d;
  const float k1 = rope_load(a.k_new, src + i, a.bf16), k2 = rope_load(a.k_new, src + half + i, a.bf16);
  const size_t kdst = ((size_t)page * a.num_kv_heads + hk) * kTile * d;  // the page's key tile
  rope_store(a.ctx_k, kdst + key_tile_elem(slot, i, a.bf16), k1 * c - k2 * s, a.bf16);
  rope_store(a.ctx_k, kdst + key_tile_elem(slot, half + i, a.bf16), k2 * c + k1 * s, a.bf16);
  const size_t vdst = ((size_t)page * a.num_kv_heads + hk) * (size_t)d * kTile + slot;
  rope_store(a.ctx_v, vdst + (size_t)i * kTile, rope_load(a.v_new, src + i, a.bf16), a.bf16);
  rope_store(a.ctx_v, vdst + (size_t)(half + i) * kTile, rope_load(a.v_new, src + half + i, a.bf16), a.bf16);
}

// System keys (16-key tiles [H_kv, ceil(L_s/16), d/G, 16, G]) rotated in place at
// positions 0 .. L_s - 1 (the offline prefill's position embedding); kRopeThreads /
// (d/2) keys per workgroup.
__global__ __launch_bounds__(kRopeThreads) void rope_system_kernel(void* sys_k, const float* cos_sin, int sys_len,
                                                                   int d, int bf16) {
  const int half = d / 2, hk = blockIdx.y, i = threadIdx.x % half;
  const int j = blockIdx.x * (kRopeThreads / half) + threadIdx.x / half;
  if (j >= sys_len) return;
  const float c = cos_sin[(size_t)j * d + i], s = cos_sin[(size_t)j * d + half + i];
  const int ntile = (sys_len + kTile - 1) / kTile;
  const size_t base = ((size_t)hk * ntile + j / kTile) * kTile * d;
  const size_t e1 = base + key_tile_elem(j % kTile, i, bf16), e2 = base + key_tile_elem(j % kTile, half + i, bf16);
  const float x1 = rope_load(sys_k, e1, bf16), x2 = rope_load(sys_k, e2, bf16);
  rope_store(sys_k, e1, x1 * c - x2 * s, bf16);
  rope_store(sys_k, e2, x2 * c + x1 * s, bf16);
}

// The offline prefill's cache fill: the system prompt's keys and values, token-major
// as a projection produces them (k_raw / v_raw [L_s, H_kv, d]), into the system cache
// layouts: sys_k [H_kv, ceil(L_s/16), d/G, 16, G] (chunk-major 16-key tiles) with RoPE
// at position j, sys_v [H_kv, ceil(L_s/16), d, 16] (dimension-major 16-key tiles); the
// tail tiles' padding keys are written as 0.
__global__ __launch_bounds__(kRopeThreads) void system_fill_kernel(const void* k_raw, const void* v_raw,
                                                                   const float* cos_sin, void* sys_k, void* sys_v,
                                                                   int sys_len, int num_kv_heads, int d, int bf16) {
  const int half = d / 2, hk = blockIdx.y, i = threadIdx.x % half;
  const int j = blockIdx.x * (kRopeThreads / half) + threadIdx.x / half;
  const int ntile = (sys_len + kTile - 1) / kTile;
  if (j >= ntile * kTile) return;
  const size_t vt = ((size_t)hk * ntile + j / kTile) * (size_t)d * kTile + j % kTile;
  const size_t kt = ((size_t)hk * ntile + j / kTile) * (size_t)d * kTile;
  const size_t k_e1 = kt + key_tile_elem(j % kTile, i, bf16), k_e2 = kt + key_tile_elem(j % kTile, half + i, bf16);
  if (j >= sys_len) {  // padding keys of the tail tile (grid covers whole tiles)
    rope_store(sys_k, k_e1, 0.f, bf16);
    rope_store(sys_k, k_e2, 0.f, bf16);
    rope_store(sys_v, vt + (size_t)i * kTile, 0.f, bf16);
    rope_store(sys_v, vt + (size_t)(half + i) * kTile, 0.f, bf16);
    return;
  }
  const size_t src = ((size_t)j * num_kv_heads + hk) * d;
  const float c = cos_sin[(size_t)j * d + i], s = cos_sin[(size_t)j * d + half + i];
  const float k1 = rope_load(k_raw, src + i, bf16), k2 = rope_load(k_raw, src + half + i, bf16);
  rope_store(sys_k, k_e1, k1 * c - k2 * s, bf16);
  rope_store(sys_k, k_e2, k2 * c + k1 * s, bf16);
  rope_store(sys_v, vt + (size_t)i * kTile, rope_load(v_raw, src + i, bf16), bf16);
  rope_store(sys_v, vt + (size_t)(half + i) * kTile, rope_load(v_raw, src + half + i, bf16), bf16);
}

hipError_t launch_system_fill(const void* k_raw, const void* v_raw, const float* cos_sin, void* sys_k, void* sys_v,
                              int sys_len, int num_kv_heads, int d, int bf16, hipStream_t s) {
  const int padded = (sys_len + kTile - 1) / kTile * kTile;
  const int per = kRopeThreads / (d / 2);
  hipLaunchKernelGGL(system_fill_kernel, dim3((padded + per - 1) / per, num_kv_heads), dim3(kRopeThreads), 0, s,
                     k_raw, v_raw, cos_sin, sys_k, sys_v, sys_len, num_kv_heads, d, bf16);
  return hipGetLastError();
}

hipError_t launch_rope_table(float* cos_sin, int max_pos, int d, double base, hipStream_t s) {
  hipLaunchKernelGGL(rope_table_kernel, dim3(max_pos), dim3(64), 0, s, cos_sin, max_pos, d, base);
  return hipGetLastError();
}

hipError_t launch_rope_append(const RopeArgs& a, int max_q_len, hipStream_t s) {
  const int per = kRopeThreads / (a.head_dim / 2);
  hipLaunchKernelGGL(rope_append_kernel, dim3(a.batch, max_q_len, (a.num_q_heads + a.num_kv_heads + per - 1) / per),
                     dim3(kRopeThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_rope_system(void* sys_k, const float* cos_sin, int sys_len, int num_kv_heads, int d, int bf16,
                              hipStream_t s) {
  const int per = kRopeThreads / (d / 2);
  hipLaunchKernelGGL(rope_system_kernel, dim3((sys_len + per - 1) / per, num_kv_heads), dim3(kRopeThreads), 0, s,
                     sys_k, cos_sin, sys_len, d, bf16);
  return hipGetLastError();
}

}  // namespace relay
