// sys_attn_mfma.hpp: one workgroup of RelayAttention's system-attention step on the
// matrix cores of gfx950 (bf16 inputs, head_dim 128), shared by the system kernel
// (sys_attn_mfma.hip) and the streaming launch that runs it beside the context streams
// (stream_attn.hip).
//
// Every query row of the batch attends to the shared system KV cache alone, so for KV
// head h the M = T_q * g rows that use it form one matrix multiplied against the
// system keys (RelayAttention paper page, Abstract; atyun.com article, section
// "RelayAttention": the system K/V leave HBM once per batch).  With M in the
// thousands this is a dense contraction bound by the matrix cores.
//
// Workgroup = (128-row block, part of the keys of all heads), 4 waves of 32 rows
// each.  Its keys stream through LDS in 64-key steps, double-buffered: the next step's
// K and V tiles load straight into the other LDS buffer (global_load_lds) while the
// current one is computed; one wait and barrier per step.  Every wave reads each
// tile from LDS, so a tile leaves L2 once per workgroup.
//
// Matrix-core mapping (v_mfma_f32_32x32x16_bf16, 32x32 tiles):
//   * scores transposed, S^T = K Q^T: A = 32 keys x 16 dims from LDS, B = 16 dims x 32
//     query rows (registers).  Lane l then holds row l % 32 and keys
//     8 (j / 4) + 4 (l / 32) + j % 4, j = 0..15, of the 32-key block;
//   * outputs transposed, O^T = V^T P^T: B is P straight from the score
//     accumulators, 16 keys per product: k slots 0..3 hold keys 4 (l/32) + 0..3, slots
//     4..7 keys 8 + 4 (l/32) + 0..3 of the 16-key block; A is V^T with the same key
//     order, two 8-byte reads from the dimension-major LDS tile.
// The K tile sits in LDS chunk-major ([16-byte chunk][64 keys]), as the key cache
// stores its 16-key tiles, so a load instruction fetches whole 256-byte runs of the
// cache and a wave's operand read is 512 contiguous bytes per half wave; the V tile is
// XOR-swizzled in 16-byte chunks (by dim % 8) so its reads hit distinct banks.  Softmax uses a lazily moved reference (rows
// rescale only when their maximum grows by more than 2^8).
#pragma once

#include "relay_device.hpp"
#include "relay_internal.hpp"

namespace relay {

typedef float f32x16 __attribute__((ext_vector_type(16)));

// A decode 16-key block adds P's bf16 rounding residual when some row's largest probability in
// it exceeds 1 / kSplitShare of the row's running sum.
constexpr float kSplitShare = 32.f;

namespace mf {
constexpr int D = 128;
constexpr int kRowsPerWave = 32;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kKB = 64;                       // keys per step
constexpr int kTileBytes = kKB * D * 2;       // one K or V tile (bf16)
constexpr int kBufBytes = 2 * kTileBytes;     // K then V
constexpr int kChunks = kTileBytes / 16 / kThreads;  // 16-byte chunks per thread per tile
}  // namespace mf

static_assert(kSysMfmaRows == mf::kRowsPerWave * mf::kWaves, "rows per workgroup");
constexpr size_t kSysMfmaLds = 2 * (size_t)mf::kBufBytes;

__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// K rows are stored in LDS with the middle two 4-key groups of every 16 swapped (row
// 4..7 holds key 8..11 and row 8..11 key 4..7).  The score accumulators then give the
// lanes l / 32 = 0 the keys 0..7 and lanes l / 32 = 1 the keys 8..15 of each 16-key
// block, in order: exactly the k slots of the P.V product's B operand, so V^T for a
// lane is one contiguous 16-byte read of the dimension-major V tile.
__device__ __forceinline__ int mf_key_of_row(int row) {
  const int q = row & 15;
  return (row & ~15) + ((q >= 4 && q < 8) ? q + 4 : ((q >= 8 && q < 12) ? q - 4 : q));
}

// Offset of 16-byte chunk c of the key held by LDS row `row` (0..63) of a step, from
// the step's first key tile: key tiles are 16 keys x 256 bytes, chunk-major, and the
// key of LDS row r sits in slot r % 16 of its tile (mf_key_of_row and the tiles' slot
// order are the same swap).
__device__ __forceinline__ uint32_t mf_key_offset(int row, int c) {
  return (uint32_t)((row >> 4) * (kTile * mf::D * 2) + key_chunk_offset(row & 15, c));
}

// Issues the loads of the step whose first key is key0 straight into an LDS buffer
// (the NW waves of the workgroup share them): lane i of a wave's load lands at the
// instruction's LDS base + 16 i, so each lane fetches the global 16 bytes that belong
// at its position of the LDS layout (K: LDS position p holds chunk p / 64 of row
// p % 64).  K rows past the keys are clamped (their scores are masked); V tiles past
// the last are clamped (mf_zero_tail clears values of keys that do not exist).
template <int NW = mf::kWaves>
__device__ __forceinline__ void mf_issue(char* buf, const char* kbase, const char* vbase, int key0, int Ls,
                                         int ntile) {
  constexpr int kThreadsW = kWave * NW, kChunksW = mf::kTileBytes / 16 / kThreadsW;
  const int lane = lane_id(), wave = threadIdx.x / kWave;
#pragma unroll
  for (int j = 0; j < kChunksW; ++j) {
    const int base = kThreadsW * j + kWave * wave;  // first 16-byte position of this load
    const int p = base + lane;
    const int row = p & 63, c = p >> 6;
    const int key = min(key0 + mf_key_of_row(row), Ls - 1);
    const char* src = kbase + (size_t)(key / kTile) * (kTile * mf::D * 2) + key_chunk_offset(key_slot(key % kTile), c);
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(buf + base * 16), 16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kChunksW; ++j) {
    const int base = kThreadsW * j + kWave * wave;
    const int p = base + lane;
    const int d = p >> 3, c = (p & 7) ^ (d & 7);  // row d, 8-key chunk c of the 64
    const int tile = min(key0 / kTile + (c >> 1), ntile - 1);
    const char* src = vbase + (size_t)tile * (mf::D * kTile * 2) + d * (kTile * 2) + (c & 1) * 16;
    __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)(buf + mf::kTileBytes + base * 16), 16, 0, 0);
  }
}

// Per-lane byte offsets of one step's loads relative to its first key key0: both
// layouts hold 256 bytes per key (a 16-key tile of 128-dim bf16 keys or values is 4096
// bytes), and steps start at multiples of 64 keys, so every load of a step is
// base + 256 key0 + a constant of the lane.  Load j of a lane lands at LDS position
// p = 64 NW j + 64 wave + lane (NW waves): K row p % 64 = lane, chunk p / 64 = NW j +
// wave; V row d = 8 NW j + 8 wave + lane / 8, chunk (lane % 8) ^ (d % 8) with
// d % 8 = (lane / 8) % 8.  Both offsets are base + 256 NW j, so a lane keeps two bases.  Steps that end inside
// the prompt use these; the step holding the prompt's end goes through mf_issue
// (clamped rows).
struct MfLaneOffsets {
  uint32_t k, v;
};

__device__ __forceinline__ MfLaneOffsets mf_lane_offsets(int wave) {
  const int lane = lane_id();
  MfLaneOffsets o;
  o.k = mf_key_offset(lane, wave);
  const int d = 8 * wave + (lane >> 3), cv = (lane & 7) ^ (d & 7);
  o.v = (uint32_t)((cv >> 1) * (mf::D * kTile * 2) + d * (kTile * 2) + (cv & 1) * 16);
  return o;
}

template <int NW = mf::kWaves>
__device__ __forceinline__ void mf_issue_full(char* buf, const char* kstep, const char* vstep, int wave,
                                              const MfLaneOffsets& o) {
  constexpr int kThreadsW = kWave * NW, kChunksW = mf::kTileBytes / 16 / kThreadsW;
  static_assert(kChunksW * kThreadsW * 16 == mf::kTileBytes, "loads per tile");
#pragma unroll
  for (int j = 0; j < kChunksW; ++j) {
    const int base = kThreadsW * j + kWave * wave;
    __builtin_amdgcn_global_load_lds(kstep + o.k + 256 * NW * j, (lds_ptr_t)(buf + base * 16), 16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kChunksW; ++j) {
    const int base = kThreadsW * j + kWave * wave;
    __builtin_amdgcn_global_load_lds(vstep + o.v + 256 * NW * j, (lds_ptr_t)(buf + mf::kTileBytes + base * 16), 16,
                                     0, 0);
  }
}

// Zeroes the V values of keys [nvalid, 64) of a landed step (values of keys past the
// system prompt must not reach an output through 0 * NaN).
template <int NW = mf::kWaves>
__device__ __forceinline__ void mf_zero_tail(char* buf, int nvalid) {
  for (int i = threadIdx.x; i < mf::D * mf::kKB; i += kWave * NW) {
    const int d = i / mf::kKB, k = i % mf::kKB;
    if (k >= nvalid)
      *reinterpret_cast<uint16_t*>(buf + mf::kTileBytes + d * 128 + (((k >> 3) ^ (d & 7)) << 4) + (k & 7) * 2) = 0;
  }
}

// One workgroup of the system step: workgroup `block` of `nblocks` (hardware places
// workgroup i of a launch on XCD i % 8; the system workgroups are the first `nblocks`
// of their launch).  lds_raw: kSysMfmaLds bytes.  CAUSAL: the offline prefill's
// attention (query token t sees keys 0..t); its own instantiation, so the decode
// workgroups carry none of the masking.
template <bool CAUSAL>
__device__ __forceinline__ void sys_mfma_workgroup(const SysArgs& a, int block, int nblocks, char* lds_raw) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int r32 = lane & 31, hh = lane >> 5;
  const MfLaneOffsets lo_ = mf_lane_offsets(wave);

  // workgroup -> (row block, part).  Part p streams the 64-key steps
  // [p S / P, (p + 1) S / P) of the S = H_kv * steps_per_head steps of all heads
  // (every workgroup the same amount of work, whatever the head and row-block counts),
  // and every row block runs the same parts in step: the workgroups of one part are
  // consecutive ids, placed on one XCD (hardware puts workgroup i on XCD i % 8, the
  // remap gives each XCD a contiguous id range), so a K/V tile leaves HBM once and
  // the other row blocks read it from that XCD's L2.
  const int total = nblocks;
  int li = block;
  if (a.xcd_remap) li = (block & 7) * (total >> 3) + (block >> 3);
  // causal: a row block's work grows with its tokens, so the last row blocks (the
  // longest workgroups) are dispatched first
  const int rb = CAUSAL ? a.row_blocks - 1 - li % a.row_blocks : li % a.row_blocks;
  const int part = li / a.row_blocks;
  if (part >= a.parts) return;  // padding workgroup (whole workgroup)
  const int S = a.total_steps, P = a.parts, sph = a.steps_per_head;
  int sbeg = (int)((long long)part * S / P);
  const int send = (int)((long long)(part + 1) * S / P);

  const int Ls = a.sys_len;
  const int M = a.total_q * a.group;
  const int ntile = (Ls + kTile - 1) / kTile;
  // scores are taken scale-free with the sign folded in: s' = sign(scale) q.k (the
  // query's sign bits flipped once per segment: exact), and p = 2^(|scale| s' - m)
  const bool negative_scale = a.scale_log2 < 0.f;
  const float scale = negative_scale ? -a.scale_log2 : a.scale_log2;
  const int m = rb * kSysMfmaRows + wave * mf::kRowsPerWave + r32;  // this lane's stacked row
  const bool row_ok = m < M;
  const int t = m / a.group, gi = m % a.group;
  // causal: query token t sees keys 0..t; the workgroup's tokens span [t_lo, t_hi]
  const int t_lo = rb * kSysMfmaRows / a.group;
  const int t_hi = (min(rb * kSysMfmaRows + kSysMfmaRows, M) - 1) / a.group;

  // one segment per head the run touches: keys [ls0 * 64, min(ls1 * 64, Ls)) of head h
  while (sbeg < send) {
    const int h = sbeg / sph;
    const int ls0 = sbeg % sph;
    const int ls1 = min(sph, ls0 + (send - sbeg));
    sbeg += ls1 - ls0;
    const int key_begin = ls0 * mf::kKB;
    const int key_end = min(ls1 * mf::kKB, Ls);
    int nsteps = ls1 - ls0;
    // causal: steps no token of the workgroup sees are skipped (maybe all), and where
    // some token sees between 1 and kPSplitBelow - 1 of the segment's keys P is split
    bool psplit = false;
    if constexpr (CAUSAL) {
      const int seen = min(key_end, t_hi + 1) - key_begin;
      nsteps = seen > 0 ? (seen + mf::kKB - 1) / mf::kKB : 0;
      psplit = seen > 0 && t_lo + 1 - key_begin < kPSplitBelow;
    }
    const char* kbase = static_cast<const char*>(a.sys_k) + (size_t)h * ntile * kTile * mf::D * 2;
    const char* vbase = static_cast<const char*>(a.sys_v) + (size_t)h * ntile * mf::D * kTile * 2;

    // this lane's query row (B operand of S^T: 8 consecutive dims of 16 per product)
    const size_t qrow = (size_t)t * a.num_q_heads + (size_t)h * a.group + gi;
    u32x4 qf[mf::D / 16];
    {
      const char* qp = static_cast<const char*>(a.q) + qrow * mf::D * 2 + 16 * hh;
#pragma unroll
      for (int kk = 0; kk < mf::D / 16; ++kk) qf[kk] = row_ok ? ld16(qp + 32 * kk) : u32x4{0u, 0u, 0u, 0u};
      if (negative_scale) {
        const uint32_t sg = 0x80008000u;
#pragma unroll
        for (int kk = 0; kk < mf::D / 16; ++kk) qf[kk] ^= u32x4{sg, sg, sg, sg};
      }
    }

    f32x16 o[mf::D / 32];
#pragma unroll
    for (int db = 0; db < mf::D / 32; ++db) o[db] = f32x16{};
    float mrow = neg_inf(), lsum = 0.f;

    // loads of the step at key0 into buffer dst: plain offsets unless it holds the end
    auto issue = [&](char* dst, int key0) {
      if (!CAUSAL && key0 + mf::kKB <= Ls)  // (the causal kernel keeps the registers)
        mf_issue_full(dst, kbase + (size_t)key0 * (mf::D * 2), vbase + (size_t)key0 * (mf::D * 2), wave, lo_);
      else
        mf_issue(dst, kbase, vbase, key0, Ls, ntile);
    };

    if (nsteps > 0) {
      issue(lds_raw, key_begin);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }

    for (int s = 0; s < nsteps; ++s) {
      const int key0 = key_begin + s * mf::kKB;
      char* buf = lds_raw + (s & 1) * mf::kBufBytes;
      const bool partial = key0 + mf::kKB > Ls;  // the last step of the prompt
      if (partial) {  // clear V past the prompt's end
        mf_zero_tail(buf, Ls - key0);
        __syncthreads();
      }
      const bool more = s + 1 < nsteps;
      if (more) issue(lds_raw + ((s + 1) & 1) * mf::kBufBytes, key0 + mf::kKB);

      // ---- scores of the 64 keys (two 32-key blocks) from the K tile in LDS; lane (row,
      // hh) holds keys 32 kb2 + 16 (j / 8) + 8 hh + j % 8 as sc[16 kb2 + j].  Scale-free
      // with the scale's sign folded in; causal steps that token t_lo does not wholly see
      // mask keys past t (and past the prompt) to -inf, so their exponentials are 0 (scale
      // > 0).  Otherwise no masking: in the step holding the prompt's end, rows past it
      // hold copies of the last key (mf_issue clamps them), whose scores leave the
      // maximum unchanged, and their values are zero in LDS, so they add nothing to O;
      // only the row sum leaves them out.
      auto raw_scores = [&](float (&sc)[32]) {
        f32x16 sacc[2];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          sacc[kb2] = f32x16{};
          const char* krow = buf + (32 * kb2 + r32) * 16;  // LDS row 32 kb2 + r32, chunk-major
#pragma unroll
          for (int kk = 0; kk < mf::D / 16; ++kk) {
            const u32x4 ka = *reinterpret_cast<const u32x4*>(krow + (2 * kk + hh) * (mf::kKB * 16));
            sacc[kb2] = mfma32(ka, qf[kk], sacc[kb2]);
          }
        }
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
          for (int j = 0; j < 16; ++j) sc[16 * kb2 + j] = sacc[kb2][j];
        }
        if (CAUSAL && key0 + mf::kKB - 1 > t_lo) {
          const int lim_c = min(t + 1, Ls) - key0 - 8 * hh;
#pragma unroll
          for (int i = 0; i < 32; ++i)
            if (16 * (i >> 3) + (i & 7) >= lim_c) sc[i] = neg_inf();
        }
      };
      float sc[32];
      raw_scores(sc);
      // ---- online softmax on scale-free scores (lanes l and l ^ 32 hold the same row):
      // the reference m is kept scaled, p = 2^(|scale| s - m) is one FMA and an exp
      float mx = sc[0];
#pragma unroll
      for (int i = 1; i < 32; ++i) mx = fmaxf(mx, sc[i]);
      {
        float x, y;
        swap32(mx, x, y);
        mx = fmaxf(x, y) * scale;
      }
      const bool grow = mx > mrow + kLazyRescale;
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mx : mrow;
        const float alpha = grow ? fast_exp2(mrow - m_new) : 1.f;
        lsum *= alpha;
#pragma unroll
        for (int db = 0; db < mf::D / 32; ++db) o[db] *= alpha;
        mrow = m_new;
      }
      const float m_use = (mrow == neg_inf()) ? 0.f : mrow;
#pragma unroll
      for (int i = 0; i < 32; ++i) sc[i] = fast_exp2(__builtin_fmaf(sc[i], scale, -m_use));
      if (partial) {
        // score i of the lane is key 16 (i / 8) + 8 hh + i % 8 of the step; keys
        // [0, Ls - key0) exist
        const int lim_h = Ls - key0 - 8 * hh;
#pragma unroll
        for (int i = 0; i < 32; ++i) lsum += (16 * (i >> 3) + (i & 7) < lim_h) ? sc[i] : 0.f;
      } else {
#pragma unroll
        for (int i = 0; i < 32; ++i) lsum += sc[i];
      }
      // ---- O^T += V^T P^T per 16-key block kb: k slots 0..7 = keys 0..7 (lanes hh = 0),
      // 8..15 = keys 8..15 (hh = 1), i.e. sc[8 kb .. 8 kb + 7].  P enters as bf16; its
      // rounding costs up to 2^-9 of each probability.  Where that could matter, the
      // rounding residual lo = P - bf16(P) (also bf16) goes in as a second product:
      //  * causal segments that some token sees little of (psplit, known per segment);
      //  * decode 16-key blocks in which some row's largest probability exceeds
      //    1 / kSplitShare of the row's running sum, i.e. a key that may hold a large
      //    share of the row's weight.  Keys below that share round once: their errors
      //    are small and independent.
      const char* vt = buf + mf::kTileBytes;
      const int vsw = (hh ^ (r32 & 7)) << 4;  // V chunk 2 kb + hh of row d sits at (2 kb + hh) ^ (d % 8); d % 8 = r32 % 8
      // the row's running sum (both lane halves): a 16-key block needs the residual
      // product when one of its probabilities exceeds 1 / kSplitShare of it for some row.
      // No block of the step can when the step's largest probability, 2^(mx - m_use) (a
      // hair above every p of the step: the margin covers the rounding of the FMA in p),
      // does not: one test per step instead of one per block.
      float row_sum;
      {
        float la, lb;
        swap32(lsum, la, lb);
        row_sum = la + lb;
      }
      const bool any_big =
          CAUSAL || __builtin_amdgcn_ballot_w64(fast_exp2(mx - m_use) * (kSplitShare * 1.0039f) > row_sum) != 0;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const float* p = sc + 8 * kb;
        const u32x4 hi = u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                               pack_bf16x2(p[6], p[7])};
#pragma unroll
        for (int db = 0; db < mf::D / 32; ++db) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(vt + (32 * db + r32) * 128 + (((2 * kb) << 4) ^ vsw));
          o[db] = mfma32(v, hi, o[db]);
        }
        bool split;
        if constexpr (CAUSAL) {
          split = psplit;
        } else {
          split = false;
          if (any_big) {
            const float pm =
                fmaxf(fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3])), fmaxf(fmaxf(p[4], p[5]), fmaxf(p[6], p[7])));
            split = __builtin_amdgcn_ballot_w64(pm * kSplitShare > row_sum) != 0;
          }
        }
        if (split) {
          const u32x4 lo = u32x4{pack_bf16x2(p[0] - bf16_lo_as_float(hi[0]), p[1] - bf16_hi_as_float(hi[0])),
                                 pack_bf16x2(p[2] - bf16_lo_as_float(hi[1]), p[3] - bf16_hi_as_float(hi[1])),
                                 pack_bf16x2(p[4] - bf16_lo_as_float(hi[2]), p[5] - bf16_hi_as_float(hi[2])),
                                 pack_bf16x2(p[6] - bf16_lo_as_float(hi[3]), p[7] - bf16_hi_as_float(hi[3]))};
#pragma unroll
          for (int db = 0; db < mf::D / 32; ++db) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(vt + (32 * db + r32) * 128 + (((2 * kb) << 4) ^ vsw));
            o[db] = mfma32(v, lo, o[db]);
          }
        }
      }
      if (more) __builtin_amdgcn_s_waitcnt(0);  // the next step's tiles have landed
      __syncthreads();  // (also: the buffers are free for the next segment)
    }

    // ---- this segment's partial for the lane's row, in slot (part - first part of h);
    // the workgroup holding the head's first step also marks the head's unused slots
    // empty, so every slot < n_chunks of every row is written
    float lo, hi;
    swap32(lsum, lo, hi);
    const float ltot = lo + hi;
    if (row_ok) {
      const int first = lean_part_of((long long)h * sph, S, P);
      const size_t rows = (size_t)a.total_q * a.num_q_heads;
      const size_t r = (size_t)(part - first) * rows + qrow;
      const bool empty = !(ltot > 0.f);
      const float inv = empty ? 0.f : 1.f / ltot;
      float* orow = a.o_part + r * mf::D;
#pragma unroll
      for (int db = 0; db < mf::D / 32; ++db) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const f32x4 v = {o[db][4 * b] * inv, o[db][4 * b + 1] * inv, o[db][4 * b + 2] * inv,
                           o[db][4 * b + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * b + 4 * hh) = v;
        }
      }
      if (hh == 0) {
        a.lse_part[r] = empty ? neg_inf() : (mrow + __builtin_amdgcn_logf(ltot)) * kLn2;
        if (ls0 == 0) {
          const int used = lean_part_of((long long)(h + 1) * sph - 1, S, P) - first + 1;
          for (int sl = used; sl < a.n_chunks; ++sl) a.lse_part[(size_t)sl * rows + qrow] = neg_inf();
        }
      }
    }
  }
}

// ---- the decode system step as a launch of its own: one workgroup of 8 waves per CU,
// two groups of 4 half a step apart ------------------------------------------------------
//
// Per 64-key step a wave's work is matrix-core products (the scores S^T = K Q^T, and
// the previous step's O^T += V^T P^T) and then the softmax on the VALU, about equally
// long; two independent waves on a SIMD in the same phase leave one unit idle at a time.
// Here the eight waves of a workgroup (256 stacked rows, 32 per wave; waves w and w + 4
// share SIMD w % 4) run as two groups, the second one phase behind the first, with a
// workgroup barrier between phases: in every phase one wave of each SIMD issues
// matrix-core products while the other runs its softmax.  The phases of a wave:
//   M_s: O^T += V_{s-1}^T P_{s-1}^T (s > 0), then S_s^T = K_s Q^T (s < n);
//   V_s: the online softmax of S_s, giving P_s (bf16) and rescaling O when the row
//        maximum moved; the rounding residual of P_s, for the 16-key blocks that need
//        it (rare), goes into O here as well (V_s is in LDS);
// group 0 runs M_0 V_0 M_1 V_1 ... M_n in phases 0, 1, 2, ..., group 1 in phases 1, 2, ....
// Step s's K and V tiles are in LDS from phase 2 s (group 0's M_s) to phase 2 s + 3
// (group 1's M_{s+1}); four buffers, and step s + 4 is loaded from phase 2 s + 4 on, so
// each load has four phases (two steps) to land.
namespace pp {
constexpr int kWaves = 8;
constexpr int kThreads = kWave * kWaves;
constexpr int kRows = mf::kRowsPerWave * kWaves;  // stacked rows per workgroup
constexpr int kBufs = 4;
constexpr int kLoadsPerStep = 2 * (mf::kTileBytes / 16 / kThreads);  // per thread: K and V
}  // namespace pp
static_assert(kSysPPRows == pp::kRows, "rows per workgroup");
constexpr size_t kSysPPLds = (size_t)pp::kBufs * mf::kBufBytes;

// Waits until at most n of this wave's tile loads are in flight (n: loads issued after
// the step that must have landed), then joins the workgroup barrier.  The LDS reads
// before it have completed (so a buffer they read may be reloaded after it), and
// nothing in memory moves across it (the asm's memory clobber).
__device__ __forceinline__ void pp_sync(int later_steps) {
  static_assert(pp::kLoadsPerStep == 4, "vmcnt immediates below assume four loads per step");
  if (later_steps <= 0) asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if (later_steps == 1) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else if (later_steps == 2) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// The loads of the step at key0 for the two-group kernel (all eight waves), with the
// lane offsets of mf_lane_offsets.  A step that runs past the prompt's end reads its
// 16-key tiles clamped to the last one (whole tiles: no per-key arithmetic); the
// scores of keys past the end are masked and their values cleared in LDS.
__device__ __forceinline__ void pp_issue_clamped(char* buf, const char* kbase, const char* vbase, int t0, int ntile,
                                              int wave, uint32_t ok, uint32_t ov) {
  constexpr int kThreadsW = pp::kThreads, kChunksW = mf::kTileBytes / 16 / kThreadsW;
  const MfLaneOffsets o{ok, ov};
  const int lane = lane_id();
  // K: LDS row `lane` sits in tile lane / 16 of the step; V: chunk cv of the lane's row
  // is in tile cv / 2 (o.k and o.v hold those tile offsets for an unclamped step)
  const int tk = min(t0 + (lane >> 4), ntile - 1) - t0;
  const int d = 8 * wave + (lane >> 3), cv = (lane & 7) ^ (d & 7);
  const int tv = min(t0 + (cv >> 1), ntile - 1) - t0;
  const char* ks = kbase + (size_t)t0 * (kTile * mf::D * 2) + o.k + (tk - (lane >> 4)) * (kTile * mf::D * 2);
  const char* vs = vbase + (size_t)t0 * (kTile * mf::D * 2) + o.v + (tv - (cv >> 1)) * (kTile * mf::D * 2);
#pragma unroll
  for (int j = 0; j < kChunksW; ++j) {
    const int base = kThreadsW * j + kWave * wave;
    __builtin_amdgcn_global_load_lds(ks + 256 * pp::kWaves * j, (lds_ptr_t)(buf + base * 16), 16, 0, 0);
  }
#pragma unroll
  for (int j = 0; j < kChunksW; ++j) {
    const int base = kThreadsW * j + kWave * wave;
    __builtin_amdgcn_global_load_lds(vs + 256 * pp::kWaves * j, (lds_ptr_t)(buf + mf::kTileBytes + base * 16), 16, 0,
                                     0);
  }
}

__device__ __forceinline__ void pp_issue(char* buf, const char* kbase, const char* vbase, int key0, int ntile,
                                         int wave, const MfLaneOffsets& o) {
  const int t0 = key0 / kTile;
  if (t0 + mf::kKB / kTile <= ntile)
    mf_issue_full<pp::kWaves>(buf, kbase + (size_t)t0 * (kTile * mf::D * 2), vbase + (size_t)t0 * (kTile * mf::D * 2),
                              wave, o);
  else
    pp_issue_clamped(buf, kbase, vbase, t0, ntile, wave, o.k, o.v);
}

// Zeroes the V values of keys [nvalid, 64) of a landed step (two-group kernel).
__device__ __forceinline__ void pp_zero_tail(char* buf, int nvalid) { mf_zero_tail<pp::kWaves>(buf, nvalid); }

// Shapes the schedule of a block of 16 operand reads from LDS and the 16 products that
// use them: 8 reads ahead, then one product and one read at a time, so up to eight reads
// are in flight while the matrix cores work (the other wave of the SIMD is in its
// softmax and issues no products to cover the read latency).
__device__ __forceinline__ void pp_operand_pipeline() {
  __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // 8 LDS reads
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // a product
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);  // the last 8 products
}

// One workgroup of the decode system step (non-causal), workgroup `block` of `nblocks`:
// the same (row block, part) decomposition, partial slots and outputs as
// sys_mfma_workgroup, with pp::kRows rows per row block.  lds_raw: kSysPPLds bytes.
__device__ __forceinline__ void sys_pp_workgroup(const SysArgs& a, int block, int nblocks, char* lds_raw) {
  const int lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int grp = wave >> 2;
  const int r32 = lane & 31, hh = lane >> 5;
  const MfLaneOffsets lo_ = mf_lane_offsets(wave);

  int li = block;
  if (a.xcd_remap) li = (block & 7) * (nblocks >> 3) + (block >> 3);
  const int rb = li % a.row_blocks;
  const int part = li / a.row_blocks;
  if (part >= a.parts) return;  // padding workgroup (whole workgroup)
  const int S = a.total_steps, P = a.parts, sph = a.steps_per_head;
  int sbeg = (int)((long long)part * S / P);
  const int send = (int)((long long)(part + 1) * S / P);

  const int Ls = a.sys_len;
  const int M = a.total_q * a.group;
  const int ntile = (Ls + kTile - 1) / kTile;
  const bool negative_scale = a.scale_log2 < 0.f;
  const float scale = negative_scale ? -a.scale_log2 : a.scale_log2;
  const int m = rb * pp::kRows + wave * mf::kRowsPerWave + r32;  // this lane's stacked row
  const bool row_ok = m < M;
  const int t = m / a.group, gi = m % a.group;

  while (sbeg < send) {
    const int h = sbeg / sph;
    const int ls0 = sbeg % sph;
    const int ls1 = min(sph, ls0 + (send - sbeg));
    sbeg += ls1 - ls0;
    const int key_begin = ls0 * mf::kKB;
    const int n = ls1 - ls0;
    const char* kbase = static_cast<const char*>(a.sys_k) + (size_t)h * ntile * kTile * mf::D * 2;
    const char* vbase = static_cast<const char*>(a.sys_v) + (size_t)h * ntile * mf::D * kTile * 2;
    auto buf_of = [&](int s) { return lds_raw + (s % pp::kBufs) * mf::kBufBytes; };
    auto issue = [&](int s) { pp_issue(buf_of(s), kbase, vbase, key_begin + s * mf::kKB, ntile, wave, lo_); };
    // the highest step whose loads have been issued by the end of phase k: the first
    // kBufs at once, then step x at the start of phase 2 (x - kBufs) + 4
    auto last_issued = [&](int k) {
      const int x = k >= 4 ? k / 2 - 2 + pp::kBufs : pp::kBufs - 1;
      return min(n - 1, x);
    };

    const size_t qrow = (size_t)t * a.num_q_heads + (size_t)h * a.group + gi;
    u32x4 qf[mf::D / 16];
    {
      const char* qp = static_cast<const char*>(a.q) + qrow * mf::D * 2 + 16 * hh;
#pragma unroll
      for (int kk = 0; kk < mf::D / 16; ++kk) qf[kk] = row_ok ? ld16(qp + 32 * kk) : u32x4{0u, 0u, 0u, 0u};
      if (negative_scale) {
        const uint32_t sg = 0x80008000u;
#pragma unroll
        for (int kk = 0; kk < mf::D / 16; ++kk) qf[kk] ^= u32x4{sg, sg, sg, sg};
      }
    }
    f32x16 o[mf::D / 32];
#pragma unroll
    for (int db = 0; db < mf::D / 32; ++db) o[db] = f32x16{};
    float mrow = neg_inf(), lsum = 0.f;
    f32x16 sacc[2];  // S_s^T: from M_s to V_s
    u32x4 phi[4];    // P_s (bf16): from V_s to M_{s+1}

    // all earlier LDS reads of the buffers (the previous segment) are done: every wave
    // passed that segment's last barrier
    for (int s = 0; s < min(n, pp::kBufs); ++s) issue(s);
    pp_sync(last_issued(-1) - 0);  // step 0 has landed

    // global phase k: group 0 runs M_s in phase 2 s and V_s in 2 s + 1, group 1 one
    // phase later; every wave passes the same barriers
    auto start_phase = [&](int k) {
      if (k >= 4 && (k & 1) == 0) {
        const int x = k / 2 - 2 + pp::kBufs;
        if (x < n) issue(x);
      }
    };
    auto end_phase = [&](int k) {
      // the last step's V beyond the prompt's end is cleared once its loads have landed
      // (end of phase 2 n - 3) and before any wave reads it (phase 2 n: group 0's M_n);
      // its K is read in phases 2 n - 2 and 2 n - 1
      if (k == 2 * n - 2 && key_begin + n * mf::kKB > Ls)
        pp_zero_tail(buf_of(n - 1), Ls - (key_begin + (n - 1) * mf::kKB));
      // before phase k + 1 = 2 s (group 0's M_s), step s must have landed
      if ((k & 1) == 1) pp_sync(last_issued(k) - (k + 1) / 2);
      else asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    // M_s's scores (S_s^T = K_s Q^T), read from buffer `s` (M_n recomputes step n - 1's:
    // unused, but an unconditional product keeps the scores' registers simple)
    auto scores = [&](int s) {
      const char* krow = buf_of(s) + r32 * 16;
      sacc[0] = f32x16{};
      sacc[1] = f32x16{};
      // the two 32-key blocks' products alternate: consecutive products do not wait for
      // each other's accumulators
#pragma unroll
      for (int kk = 0; kk < mf::D / 16; ++kk) {
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2) {
          const u32x4 ka = *reinterpret_cast<const u32x4*>(krow + 32 * kb2 * 16 + (2 * kk + hh) * (mf::kKB * 16));
          sacc[kb2] = mfma32(ka, qf[kk], sacc[kb2]);
        }
      }
    };
    int k = 0;
    if (grp == 1) {  // group 1 waits out phase 0
      start_phase(k);
      end_phase(k);
      ++k;
    }
    start_phase(k);  // M_0
    scores(0);
    pp_operand_pipeline();
    end_phase(k);
    ++k;
    for (int s = 0; s < n; ++s) {
      start_phase(k);  // V_s
      const char* vt = buf_of(s) + mf::kTileBytes;
      const int vsw = (hh ^ (r32 & 7)) << 4;
      {
        // ---- V_s: online softmax of step s (as sys_mfma_workgroup)
        const int key0 = key_begin + s * mf::kKB;
        float sc[32];
#pragma unroll
        for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
          for (int j = 0; j < 16; ++j) sc[16 * kb2 + j] = sacc[kb2][j];
        if (key0 + mf::kKB > Ls) {
          // score i of the lane is key 16 (i / 8) + 8 hh + i % 8 of the step; keys
          // [0, Ls - key0) exist, the others (clamped tiles, padding) are masked
          const int lim_h = Ls - key0 - 8 * hh;
#pragma unroll
          for (int i = 0; i < 32; ++i)
            if (16 * (i >> 3) + (i & 7) >= lim_h) sc[i] = neg_inf();
        }
        float mx = sc[0];
#pragma unroll
        for (int i = 1; i < 32; ++i) mx = fmaxf(mx, sc[i]);
        {
          float x, y;
          swap32(mx, x, y);
          mx = fmaxf(x, y) * scale;
        }
        const bool grow = mx > mrow + kLazyRescale;
        if (__builtin_amdgcn_ballot_w64(grow) != 0) {
          const float m_new = grow ? mx : mrow;
          const float alpha = grow ? fast_exp2(mrow - m_new) : 1.f;
          lsum *= alpha;
#pragma unroll
          for (int db = 0; db < mf::D / 32; ++db) o[db] *= alpha;
          mrow = m_new;
        }
        const float m_use = (mrow == neg_inf()) ? 0.f : mrow;
#pragma unroll
        for (int i = 0; i < 32; ++i) sc[i] = fast_exp2(__builtin_fmaf(sc[i], scale, -m_use));
#pragma unroll
        for (int i = 0; i < 32; ++i) lsum += sc[i];
        float row_sum;
        {
          float la, lb;
          swap32(lsum, la, lb);
          row_sum = la + lb;
        }
        const bool any_big =
            __builtin_amdgcn_ballot_w64(fast_exp2(mx - m_use) * (kSplitShare * 1.0039f) > row_sum) != 0;
        const char* vt = buf_of(s) + mf::kTileBytes;
        const int vsw = (hh ^ (r32 & 7)) << 4;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const float* pb = sc + 8 * kb;
          phi[kb] = u32x4{pack_bf16x2(pb[0], pb[1]), pack_bf16x2(pb[2], pb[3]), pack_bf16x2(pb[4], pb[5]),
                          pack_bf16x2(pb[6], pb[7])};
          if (any_big) {
            const float pm = fmaxf(fmaxf(fmaxf(pb[0], pb[1]), fmaxf(pb[2], pb[3])),
                                   fmaxf(fmaxf(pb[4], pb[5]), fmaxf(pb[6], pb[7])));
            if (__builtin_amdgcn_ballot_w64(pm * kSplitShare > row_sum) != 0) {
              const u32x4 plo = {
                  pack_bf16x2(pb[0] - bf16_lo_as_float(phi[kb][0]), pb[1] - bf16_hi_as_float(phi[kb][0])),
                  pack_bf16x2(pb[2] - bf16_lo_as_float(phi[kb][1]), pb[3] - bf16_hi_as_float(phi[kb][1])),
                  pack_bf16x2(pb[4] - bf16_lo_as_float(phi[kb][2]), pb[5] - bf16_hi_as_float(phi[kb][2])),
                  pack_bf16x2(pb[6] - bf16_lo_as_float(phi[kb][3]), pb[7] - bf16_hi_as_float(phi[kb][3]))};
#pragma unroll
              for (int db = 0; db < mf::D / 32; ++db) {
                const u32x4 v =
                    *reinterpret_cast<const u32x4*>(vt + (32 * db + r32) * 128 + (((2 * kb) << 4) ^ vsw));
                o[db] = mfma32(v, plo, o[db]);
              }
            }
          }
        }
      }
      end_phase(k);
      ++k;
      start_phase(k);  // M_{s+1}: O^T += V_s^T P_s^T, then the scores of step s + 1
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int db = 0; db < mf::D / 32; ++db) {
          const u32x4 v = *reinterpret_cast<const u32x4*>(vt + (32 * db + r32) * 128 + (((2 * kb) << 4) ^ vsw));
          o[db] = mfma32(v, phi[kb], o[db]);
        }
      }
      pp_operand_pipeline();
      // (the scores' operand reads stay behind the products above)
      __builtin_amdgcn_sched_barrier(0);
      scores(s + 1 < n ? s + 1 : s);
      pp_operand_pipeline();
      end_phase(k);
      ++k;
    }
    if (grp == 0) {  // group 0 waits out phase 2 n + 1
      start_phase(k);
      end_phase(k);
    }

    // ---- this segment's partial for the lane's row (as sys_mfma_workgroup)
    float lo, hi;
    swap32(lsum, lo, hi);
    const float ltot = lo + hi;
    if (row_ok) {
      const int first = lean_part_of((long long)h * sph, S, P);
      const size_t rows = (size_t)a.total_q * a.num_q_heads;
      const size_t r = (size_t)(part - first) * rows + qrow;
      const bool empty = !(ltot > 0.f);
      const float inv = empty ? 0.f : 1.f / ltot;
      float* orow = a.o_part + r * mf::D;
#pragma unroll
      for (int db = 0; db < mf::D / 32; ++db) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const f32x4 v = {o[db][4 * b] * inv, o[db][4 * b + 1] * inv, o[db][4 * b + 2] * inv,
                           o[db][4 * b + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * b + 4 * hh) = v;
        }
      }
      if (hh == 0) {
        a.lse_part[r] = empty ? neg_inf() : (mrow + __builtin_amdgcn_logf(ltot)) * kLn2;
        if (ls0 == 0) {
          const int used = lean_part_of((long long)(h + 1) * sph - 1, S, P) - first + 1;
          for (int sl = used; sl < a.n_chunks; ++sl) a.lse_part[(size_t)sl * rows + qrow] = neg_inf();
        }
      }
    }
  }
}

}  // namespace relay
