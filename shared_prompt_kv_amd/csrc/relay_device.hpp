// Device building blocks of the RelayAttention decode kernels for gfx950 (CDNA4).
//
// Matrix-core mapping (one 64-lane wavefront, 16x16 output tiles):
//
//   * Scores are computed transposed, S^T = K Q^T: the A operand is 16 keys, the B
//     operand 16 query rows.  Lane l then holds scores of query row l%16 for keys
//     4*(l/16)+i, i = 0..3 (the 16x16 accumulator layout), so every per-row
//     softmax quantity lives in the lanes with the same l%16.
//   * Outputs are computed transposed too, O^T = V^T P^T: the A operand is 16
//     value dimensions, the B operand is P taken straight from the score
//     accumulators (no cross-lane shuffle), and the accumulator gives lane l the
//     outputs of row l%16 for dimensions 16*t + 4*(l/16) + i.
//   * One step covers 32 keys as two 16-key score tiles whose rows are permuted so
//     that lane group q = l/16 ends up with the scores of 8 consecutive keys
//     8q..8q+7 (tile A holds keys 8q+i, tile B keys 8q+4+i).  Those 8 keys are then
//     the reduction slice of lane group q in O^T = V^T P^T, and because values are
//     stored dimension-major in 16-key tiles, V^T for them is one contiguous
//     16-byte (bf16) or 32-byte (fp32) load.
//   * The reduction order inside one MFMA does not matter for the sum, so any
//     assignment of head dimensions (for S) or keys (for O) to the k slots is
//     valid as long as the A and B operands use the same one.  For product kk a
//     lane loads 16 bytes of its query row at byte offset 64*kk + 16*(l/16), and the
//     same head dimensions of its key: chunk 4*kk + l/16 of the key's 16-key tile,
//     which stores keys chunk-major (see key_chunk_offset).
//
// bf16 uses v_mfma_f32_16x16x32_bf16 (one 16-byte chunk = 8 elements per
// instruction); fp32 uses v_mfma_f32_16x16x4f32 (one chunk = 4 instructions).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace relay {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kStep = 32;   // keys per step
constexpr int kTile = 16;   // keys per page / per system V tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct bf16_t {};  // tag: storage is bfloat16 bit patterns

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kBytes = 4;
};
template <> struct Elem<bf16_t> {
  static constexpr int kBytes = 2;
};

__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

__device__ inline float neg_inf() { return -__builtin_inff(); }

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The values of lanes l and l^32 (permlane32 swap) and of l and l^16 (permlane16
// swap), exchanged in VALU without going through LDS (gfx950).
__device__ inline void swap32(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ inline void swap16(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// Max / sum over the four lane groups (lanes l, l^16, l^32, l^48) that hold the same row.
__device__ inline float row_max4(float v) {
  float a, b;
  swap32(v, a, b);
  swap16(fmaxf(a, b), a, b);
  return fmaxf(a, b);
}
__device__ inline float row_sum4(float v) {
  float a, b;
  swap32(v, a, b);
  swap16(a + b, a, b);
  return a + b;
}

// ---- matrix-core primitives ---------------------------------------------------------

// acc += A(chunk a) * B(chunk b) over the k slots carried by one 16-byte chunk.
__device__ inline void mfma_chunk(f32x4& acc, u32x4 a, u32x4 b, float) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), acc, 0, 0, 0);
}
__device__ inline void mfma_chunk(f32x4& acc, u32x4 a, u32x4 b, bf16_t) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}

// Value fragment: V^T for one 16-dimension tile and the 8 keys of this lane group.
template <typename T> struct VFrag;
template <> struct VFrag<bf16_t> {
  u32x4 c;  // 8 bf16 keys
};
template <> struct VFrag<float> {
  u32x4 c0, c1;  // 8 fp32 keys
};

// Probability fragment: the 8 probabilities of this lane's row for the same keys.
// For bf16, c holds P rounded to bf16 and lo the rounding residual P - c (also bf16),
// used when the product must keep fp32-level accuracy: O = V^T c + V^T lo.
template <typename T> struct PFrag;
template <> struct PFrag<bf16_t> {
  u32x4 c, lo;
};
template <> struct PFrag<float> {
  float p[8];
};

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  // Round to nearest even, both halves in one v_cvt_pk_bf16_f32 (gfx950).
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

__device__ inline float bf16_lo_as_float(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi_as_float(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <bool SPLIT>
__device__ inline void make_p(PFrag<bf16_t>& f, const float (&p)[8]) {
  f.c.x = pack_bf16x2(p[0], p[1]);
  f.c.y = pack_bf16x2(p[2], p[3]);
  f.c.z = pack_bf16x2(p[4], p[5]);
  f.c.w = pack_bf16x2(p[6], p[7]);
  if constexpr (SPLIT) {
    f.lo.x = pack_bf16x2(p[0] - bf16_lo_as_float(f.c.x), p[1] - bf16_hi_as_float(f.c.x));
    f.lo.y = pack_bf16x2(p[2] - bf16_lo_as_float(f.c.y), p[3] - bf16_hi_as_float(f.c.y));
    f.lo.z = pack_bf16x2(p[4] - bf16_lo_as_float(f.c.z), p[5] - bf16_hi_as_float(f.c.z));
    f.lo.w = pack_bf16x2(p[6] - bf16_lo_as_float(f.c.w), p[7] - bf16_hi_as_float(f.c.w));
  }
}
template <bool SPLIT>
__device__ inline void make_p(PFrag<float>& f, const float (&p)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.p[i] = p[i];
}

template <bool SPLIT>
__device__ inline void mfma_pv(f32x4& acc, const VFrag<bf16_t>& v, const PFrag<bf16_t>& p) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v.c),
                                                __builtin_bit_cast(bf16x8, p.c), acc, 0, 0, 0);
  if constexpr (SPLIT)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v.c),
                                                  __builtin_bit_cast(bf16x8, p.lo), acc, 0, 0, 0);
}
template <bool SPLIT>
__device__ inline void mfma_pv(f32x4& acc, const VFrag<float>& v, const PFrag<float>& p) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c0.x), p.p[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c0.y), p.p[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c0.z), p.p[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c0.w), p.p[3], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c1.x), p.p[4], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c1.y), p.p[5], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c1.z), p.p[6], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c1.w), p.p[7], acc, 0, 0, 0);
}

// Loads V^T[dim][k0..k0+7] from a dimension-major 16-key tile row (k0 in {0, 8}).
__device__ inline void load_v(VFrag<bf16_t>& f, const char* row_k0) { f.c = ld16(row_k0); }
__device__ inline void load_v(VFrag<float>& f, const char* row_k0) {
  f.c0 = ld16(row_k0);
  f.c1 = ld16(row_k0 + 16);
}

// Zeroes the keys of a value fragment whose index (0..7 within the lane group) is
// >= nvalid.  Poisoned (NaN) padding must not reach an output through 0 * NaN.
__device__ inline uint32_t keep_bf16_pair(uint32_t w, int k, int nvalid) {
  uint32_t lo = (k < nvalid) ? (w & 0xFFFFu) : 0u;
  uint32_t hi = (k + 1 < nvalid) ? (w & 0xFFFF0000u) : 0u;
  return lo | hi;
}
__device__ inline void mask_v(VFrag<bf16_t>& f, int nvalid) {
  f.c.x = keep_bf16_pair(f.c.x, 0, nvalid);
  f.c.y = keep_bf16_pair(f.c.y, 2, nvalid);
  f.c.z = keep_bf16_pair(f.c.z, 4, nvalid);
  f.c.w = keep_bf16_pair(f.c.w, 6, nvalid);
}
__device__ inline void mask_v(VFrag<float>& f, int nvalid) {
  f.c0.x = 0 < nvalid ? f.c0.x : 0u;
  f.c0.y = 1 < nvalid ? f.c0.y : 0u;
  f.c0.z = 2 < nvalid ? f.c0.z : 0u;
  f.c0.w = 3 < nvalid ? f.c0.w : 0u;
  f.c1.x = 4 < nvalid ? f.c1.x : 0u;
  f.c1.y = 5 < nvalid ? f.c1.y : 0u;
  f.c1.z = 6 < nvalid ? f.c1.z : 0u;
  f.c1.w = 7 < nvalid ? f.c1.w : 0u;
}

// Row permutation of the two 16-key score tiles of a 32-key step: A-operand row m
// of tile A holds key 8*(m/4) + m%4, of tile B key 8*(m/4) + 4 + m%4.
__device__ inline int step_key_a(int m) { return 8 * (m >> 2) + (m & 3); }
__device__ inline int step_key_b(int m) { return 8 * (m >> 2) + 4 + (m & 3); }

// ---- online softmax ------------------------------------------------------------------

// Running state of the 16 rows of one row tile, as held by one lane (row l%16).
template <int D>
struct RowState {
  static constexpr int kDT = D / 16;  // 16-dim output tiles
  float m;                            // running max of scaled scores (log2 domain)
  float l;                            // this lane's partial sum of 2^(s - m)
  f32x4 o[kDT];                       // O^T accumulators: dims 16*t + 4*(l/16) + i
  __device__ void init() {
    m = neg_inf();
    l = 0.f;
#pragma unroll
    for (int t = 0; t < kDT; ++t) o[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// Folds N scores (log2 domain, -inf = masked) into the state and returns their
// probabilities relative to the new running max.
template <int D, int N>
__device__ inline void softmax_step(RowState<D>& st, float (&s)[N]) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mx = fmaxf(mx, s[i]);
  mx = row_max4(mx);
  const float m_new = fmaxf(st.m, mx);
  const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
  const float alpha = fast_exp2(st.m - m_use);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    s[i] = fast_exp2(s[i] - m_use);
    sum += s[i];
  }
  st.l = st.l * alpha + sum;
#pragma unroll
  for (int t = 0; t < RowState<D>::kDT; ++t) st.o[t] *= alpha;
  st.m = m_new;
}

// Merges state b into a (both per-lane partial sums over the same rows).
template <int D>
__device__ inline void merge_state(RowState<D>& a, float mb, float lb, const f32x4* ob) {
  const float m_new = fmaxf(a.m, mb);
  const float m_use = (m_new == neg_inf()) ? 0.f : m_new;
  const float wa = fast_exp2(a.m - m_use);
  const float wb = fast_exp2(mb - m_use);
  a.l = a.l * wa + lb * wb;
#pragma unroll
  for (int t = 0; t < RowState<D>::kDT; ++t) a.o[t] = a.o[t] * wa + ob[t] * wb;
  a.m = m_new;
}

// Floats of LDS one wave's RT row states occupy in a key-lane merge.
template <int D, int RT>
constexpr int kMergeSlot = kWave * RT * (2 + D / 4);

// Merges the row states of WK waves (key lanes kl = 0..WK-1) that processed
// disjoint keys of the same rows, in a fixed tree order (deterministic); key lane 0
// ends with the merged state.  lds: (WK/2) * kMergeSlot<D, RT> floats for this group
// of waves.  Every wave of the workgroup must call it (it holds barriers).
template <int D, int RT, int WK>
__device__ inline void merge_key_lanes(RowState<D> (&st)[RT], int kl, float* lds) {
  if constexpr (WK > 1) {
    const int lane = lane_id();
    for (int half = WK / 2; half >= 1; half /= 2) {
      __syncthreads();
      if (kl >= half && kl < 2 * half) {
        float* slot = lds + (size_t)(kl - half) * kMergeSlot<D, RT>;
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
        const float* slot = lds + (size_t)kl * kMergeSlot<D, RT>;
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
}

// Writes a finished row tile: O = acc / l (0 when the row saw no key) and the
// natural-log LSE (-inf when empty).  o_row: this lane's row, or nullptr when the
// row is padding.
template <int D>
__device__ inline void store_row_tile(const RowState<D>& st, float* o_row, float* lse_row) {
  const int q = lane_id() >> 4;
  const float l = row_sum4(st.l);
  if (o_row == nullptr) return;
  const bool empty = !(l > 0.f);
  const float inv = empty ? 0.f : 1.f / l;
#pragma unroll
  for (int t = 0; t < RowState<D>::kDT; ++t) {
    f32x4 v = st.o[t] * inv;
    *reinterpret_cast<f32x4*>(o_row + 16 * t + 4 * q) = v;
  }
  if (q == 0) *lse_row = empty ? neg_inf() : (st.m + __builtin_amdgcn_logf(l)) * kLn2;
}

// ---- key tiles ------------------------------------------------------------------------
//
// A 16-key tile of keys is stored chunk-major, 16-byte chunk c of all its keys before
// chunk c + 1, and inside a chunk the keys are in slot order: slot s holds key
// key_slot(s), the key order with the middle two groups of four swapped (slots 0..7
// hold keys 0..3 and 8..11, slots 8..15 keys 4..7 and 12..15).  key_slot is its own
// inverse, so it also maps a key to its slot.

__device__ inline int key_slot(int r) { return (r & ~12) | ((r >> 1) & 4) | ((r << 1) & 8); }

// Byte offset of chunk c of the key in slot s of a key tile.
__device__ inline int key_chunk_offset(int s, int c) { return (c * kTile + s) * 16; }

// ---- two-page steps (32 keys) ----------------------------------------------------------
//
// A step covers pages a (keys k0..k0+15) and b (k0+16..k0+31).  Its two 16x16 score
// tiles take their 16 A-operand rows from slots 0..7 (tile A) and 8..15 (tile B) of
// both pages: row m of tile A is slot m % 8 of page a (m < 8) or b.  The score
// accumulators then give lane group q (lanes 16q..16q+15) the keys 8q..8q+3 of the
// step in tile A and 8q+4..8q+7 in tile B: 8 consecutive keys of one page, the k slots
// 8q..8q+7 of the P.V product, whose V^T is one 16-byte (bf16) read of the page's
// dimension-major tile.  A lane's loads for one chunk of tile A are the 8 slots of one
// page: 128 contiguous bytes, so every load reads whole cache lines.  One softmax
// update serves 32 keys.
//
// K and V are issued separately so a step can be pipelined with a single set of
// registers: once the score products have read K, the next step's K loads go out;
// once P.V has read V, the next step's V loads go out.

template <typename T, int D>
struct StepK {
  static constexpr int NCH = D * Elem<T>::kBytes / 64;
  u32x4 a[NCH], b[NCH];  // this lane's K chunks of score tiles A and B
};
// Loads the B operand of S^T = K Q^T for one 16-row tile: lane (r16, q) of product kk
// takes 16 bytes of its query row at byte offset 64 kk + 16 q (zeros for a padding row).
template <typename T, int D>
__device__ inline void load_q_tile(u32x4* qf, const void* q, size_t row_index, bool valid) {
  constexpr int E = Elem<T>::kBytes;
  const int q4 = lane_id() >> 4;
  const char* qp = static_cast<const char*>(q) + row_index * D * E;
#pragma unroll
  for (int kk = 0; kk < StepK<T, D>::NCH; ++kk)
    qf[kk] = valid ? ld16(qp + 64 * kk + 16 * q4) : u32x4{0u, 0u, 0u, 0u};
}

template <typename T, int D>
struct StepV {
  VFrag<T> v[D / 16];  // V^T of this lane group's 8 keys, per 16-dimension tile
};

// P of one row tile for a step: bf16 hi (+ residual lo) in the k-slot order above,
// or the 8 fp32 values.
template <typename T> struct PStep;
template <> struct PStep<bf16_t> {
  u32x4 c, lo;
};
template <> struct PStep<float> {
  float p[8];
};

template <bool SPLIT>
__device__ __forceinline__ void make_pstep(PStep<bf16_t>& f, const float (&p)[8]) {
  f.c.x = pack_bf16x2(p[0], p[1]);
  f.c.y = pack_bf16x2(p[2], p[3]);
  f.c.z = pack_bf16x2(p[4], p[5]);
  f.c.w = pack_bf16x2(p[6], p[7]);
  if constexpr (SPLIT) {
    f.lo.x = pack_bf16x2(p[0] - bf16_lo_as_float(f.c.x), p[1] - bf16_hi_as_float(f.c.x));
    f.lo.y = pack_bf16x2(p[2] - bf16_lo_as_float(f.c.y), p[3] - bf16_hi_as_float(f.c.y));
    f.lo.z = pack_bf16x2(p[4] - bf16_lo_as_float(f.c.z), p[5] - bf16_hi_as_float(f.c.z));
    f.lo.w = pack_bf16x2(p[6] - bf16_lo_as_float(f.c.w), p[7] - bf16_hi_as_float(f.c.w));
  }
}
template <bool SPLIT>
__device__ __forceinline__ void make_pstep(PStep<float>& f, const float (&p)[8]) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.p[i] = p[i];
}

template <bool SPLIT>
__device__ __forceinline__ void mfma_pstep(f32x4& acc, const VFrag<bf16_t>& v, const PStep<bf16_t>& p) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v.c), __builtin_bit_cast(bf16x8, p.c),
                                                acc, 0, 0, 0);
  if constexpr (SPLIT)
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, v.c), __builtin_bit_cast(bf16x8, p.lo),
                                                  acc, 0, 0, 0);
}
template <bool SPLIT>
__device__ __forceinline__ void mfma_pstep(f32x4& acc, const VFrag<float>& v, const PStep<float>& p) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c0.x), p.p[0], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c0.y), p.p[1], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c0.z), p.p[2], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c0.w), p.p[3], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c1.x), p.p[4], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c1.y), p.p[5], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c1.z), p.p[6], acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(v.c1.w), p.p[7], acc, 0, 0, 0);
}

// Issues the K loads of a step: kpa/kpb are the two pages' key tiles (page b may
// repeat page a past the end of the keys; its scores are masked).  Lane (r16, q) of
// product kk reads chunk 4 kk + q of slot r16 % 8 (tile A) and 8 + r16 % 8 (tile B).
template <typename T, int D>
__device__ __forceinline__ void issue_k(StepK<T, D>& f, const char* kpa, const char* kpb) {
  const int q4 = lane_id() >> 4, r16 = lane_id() & 15;
  const char* base = (r16 < 8 ? kpa : kpb) + key_chunk_offset(r16 & 7, q4);
#pragma unroll
  for (int kk = 0; kk < StepK<T, D>::NCH; ++kk) {
    f.a[kk] = ld16(base + 4 * kTile * 16 * kk);
    f.b[kk] = ld16(base + 4 * kTile * 16 * kk + 8 * 16);
  }
}

// Issues the V loads of a step: lane group q reads keys 8 (q % 2) .. + 7 of page a
// (q < 2) or b, dimension 16 t + r16, from the page's dimension-major tile.
template <typename T, int D>
__device__ __forceinline__ void issue_v(StepV<T, D>& f, const char* vpa, const char* vpb) {
  constexpr int E = Elem<T>::kBytes;
  const int q4 = lane_id() >> 4, r16 = lane_id() & 15;
  const char* base = (q4 < 2 ? vpa : vpb) + r16 * kTile * E + 8 * (q4 & 1) * E;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) load_v(f.v[t], base + 16 * t * kTile * E);
}

// Rows whose running maximum grew by more than this (log2 units) rescale their
// accumulators; otherwise probabilities are taken against the older, smaller
// reference and may reach 2^kLazyRescale.  The result is the same real number either
// way (the reference cancels in O = sum p v / sum p and in LSE = m + log2 l).
constexpr float kLazyRescale = 8.f;

template <int D, int N>
__device__ __forceinline__ void softmax_lazy(RowState<D>& st, float (&s)[N]) {
  float mx = s[0];
#pragma unroll
  for (int i = 1; i < N; ++i) mx = fmaxf(mx, s[i]);
  mx = row_max4(mx);
  const bool grow = mx > st.m + kLazyRescale;  // also true for the first live key (m = -inf)
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {  // wave-uniform
    const float m_new = grow ? mx : st.m;
    const float alpha = grow ? fast_exp2(st.m - m_new) : 1.f;
    st.l *= alpha;
#pragma unroll
    for (int t = 0; t < RowState<D>::kDT; ++t) st.o[t] *= alpha;
    st.m = m_new;
  }
  const float m_use = (st.m == neg_inf()) ? 0.f : st.m;
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    s[i] = fast_exp2(s[i] - m_use);
    sum += s[i];
  }
  st.l += sum;
}

// Scores of a step for every row tile, folded into the row states; P out.  keyq: key
// index of this lane group's first key (tile A holds keyq .. keyq + 3, tile B
// keyq + 4 .. keyq + 7); keys at or past kv_len do not exist; last[rt]: the last key the
// rows of tile rt may see.
template <typename T, int D, int RT, bool PSPLIT>
__device__ __forceinline__ void step_scores(const StepK<T, D>& k, const u32x4 (&qf)[RT][StepK<T, D>::NCH],
                                            RowState<D> (&st)[RT], int keyq, int kv_len, const int (&last)[RT],
                                            float scale_log2, PStep<T> (&p)[RT]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < StepK<T, D>::NCH; ++kk) {
      mfma_chunk(sa, k.a[kk], qf[rt][kk], T{});
      mfma_chunk(sb, k.b[kk], qf[rt][kk], T{});
    }
    const int lim = min(last[rt], kv_len - 1);
    float sc[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = (keyq + i <= lim) ? sa[i] * scale_log2 : neg_inf();
      sc[4 + i] = (keyq + 4 + i <= lim) ? sb[i] * scale_log2 : neg_inf();
    }
    softmax_lazy(st[rt], sc);
    make_pstep<PSPLIT>(p[rt], sc);
  }
}

// P.V of a step into every row tile's accumulators (values of keys at or past kv_len
// are zeroed first: poisoned padding must not reach an output through 0 * NaN).
template <typename T, int D, int RT, bool PSPLIT>
__device__ __forceinline__ void step_pv(StepV<T, D>& v, int keyq, int kv_len, RowState<D> (&st)[RT],
                                        const PStep<T> (&p)[RT]) {
  if (keyq + 8 > kv_len) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) mask_v(v.v[t], kv_len - keyq);
  }
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) mfma_pstep<PSPLIT>(st[rt].o[t], v.v[t], p[rt]);
  }
}

// Steps held in registers while streaming: 2 (the next step's loads are in flight
// while one computes) where it fits two waves per SIMD in 256 registers, bf16 with
// one row tile; else 1 (a single step whose K and V are reloaded as soon as read).
template <typename T, int RT>
constexpr int stream_depth() {
  return (Elem<T>::kBytes == 2 && RT == 1) ? 2 : 1;
}

// Page addresses of one step: the K and V tiles of pages a and b.
struct StepAddr {
  const char* ka;
  const char* kb;
  const char* va;
  const char* vb;
};

// Streams steps kl, kl + WK, ... < nsteps: K(s) -> scores -> issue K(next) ->
// V(s) -> P.V -> issue V(next).  addr(s) gives a step's page addresses.
template <typename T, int D, int RT, int WK, bool PSPLIT, class Addr>
__device__ __forceinline__ void stream_pipelined(int kl, int nsteps, const u32x4 (&qf)[RT][StepK<T, D>::NCH],
                                                 RowState<D> (&st)[RT], int key0, int kv_len,
                                                 const int (&last)[RT], float scale_log2, Addr&& addr) {
  if (kl >= nsteps) return;
  const int q4 = lane_id() >> 4;
  auto issue = [&](StepK<T, D>& k, StepV<T, D>& v, int s) {
    const StepAddr ad = addr(s);
    issue_k(k, ad.ka, ad.kb);
    issue_v(v, ad.va, ad.vb);
  };
  auto run = [&](StepK<T, D>& k, StepV<T, D>& v, int s) {
    const int keyq = key0 + 32 * s + 8 * q4;
    PStep<T> p[RT];
    step_scores<T, D, RT, PSPLIT>(k, qf, st, keyq, kv_len, last, scale_log2, p);
    step_pv<T, D, RT, PSPLIT>(v, keyq, kv_len, st, p);
  };
  if constexpr (stream_depth<T, RT>() == 2) {
    // two steps in registers: the loads of step s + WK are in flight while s computes
    StepK<T, D> k0, k1;
    StepV<T, D> v0, v1;
    issue(k0, v0, kl);
    if (kl + WK < nsteps) issue(k1, v1, kl + WK);
    for (int s = kl; s < nsteps; s += 2 * WK) {
      run(k0, v0, s);
      if (s + 2 * WK < nsteps) issue(k0, v0, s + 2 * WK);
      if (s + WK >= nsteps) break;
      run(k1, v1, s + WK);
      if (s + 3 * WK < nsteps) issue(k1, v1, s + 3 * WK);
    }
  } else {
    // one step in registers: K of the next step goes out once the scores have read K,
    // V once P.V has read V
    StepK<T, D> k;
    StepV<T, D> v;
    issue(k, v, kl);
    for (int s = kl; s < nsteps; s += WK) {
      const int sn = s + WK;
      const int keyq = key0 + 32 * s + 8 * q4;
      PStep<T> p[RT];
      step_scores<T, D, RT, PSPLIT>(k, qf, st, keyq, kv_len, last, scale_log2, p);
      StepAddr ad;
      if (sn < nsteps) {
        ad = addr(sn);
        issue_k(k, ad.ka, ad.kb);
      }
      step_pv<T, D, RT, PSPLIT>(v, keyq, kv_len, st, p);
      if (sn < nsteps) issue_v(v, ad.va, ad.vb);
    }
  }
}

}  // namespace relay
