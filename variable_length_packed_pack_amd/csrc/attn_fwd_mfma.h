// Tiled packed-attention forward on gfx950 matrix cores (device code).
//
// What is computed: for every sequence i and head h, out = softmax(scale *
// Q_i K_i^T) V_i over that sequence's own keys ("gigl.nn.packed_attention",
// module description and packed_attention; "PyCoRa", "Ragged Flash
// Attention": a tiled online softmax in which each workgroup looks up its
// sequence in grid_mapping and processes only that sequence's tokens).
//
// Work decomposition ("So you wanna CUDA Graph", "Scheduling without
// max_seqlen"): one workgroup per (tile slot, head), head fastest.  Slot s
// runs flat tile f = tile_order[s]; seq = grid_mapping[f]; local tile
// t = f - block_offsets[seq]; slots >= block_offsets[num_seqs] exit at once.
// With head fastest and workgroups dealt round-robin to the 8 XCDs, a head
// count that is a multiple of 8 keeps every tile of one (sequence, head) on
// one XCD, so its K/V stay in that XCD's L2.
//
// Per wavefront: 32 query rows.  Per inner step: BN keys staged in LDS.
// MFMA orientation (v_mfma_f32_32x32x16_{bf16,f16}, 64 lanes, lane = 32*hh + n):
//   A operand: lane holds row (lane & 31), k = 8*hh .. 8*hh+7.
//   B operand: lane holds column (lane & 31), k = 8*hh .. 8*hh+7.
//   C/D: lane holds column (lane & 31), rows 8*(r/4) + 4*hh + (r%4), r < 16.
// Scores are formed transposed, S^T = K Q^T (A = K from LDS, B = Q^T from
// registers), so each lane holds 16 keys of ONE query per 32-key block: the
// row max needs one exchange between the two half-waves and the row sum none
// (each half keeps a partial sum until the end).  The output is formed
// transposed too, O^T = V^T P^T, with P^T taken straight from the score
// registers as the B operand: the 8 P values a lane passes for k-step kk are
// keys 16*kk + 8*(j/4) + 4*hh + (j%4), j < 8, so V is stored transposed in LDS
// with the key order inside every 16-key group permuted to match (bits 2 and
// 3 of the key offset swapped); then each A operand is one 16-byte LDS read.
// Every per-query quantity (running max, sum, rescale factor) is lane-local.
//
// fp32 inputs use v_mfma_f32_32x32x2_f32 (A/B: one element per lane, k = hh)
// with the same S^T / O^T orientation; there V needs no transpose because
// each A operand is a single element.
//
// Masking: key rows past the sequence end are never read from memory (the
// 16-bit path re-reads the sequence's last row in their place, the fp32 path
// zero-fills), so nothing outside the sequence -- such as NaN in unused
// capacity rows, "So you wanna CUDA Graph", "Correctness tangent" -- can
// reach the result; their scores are set to -inf (probability 0); causal
// masking is bottom-right aligned in local positions (key j visible to query
// p iff j <= p + Lk - Lq).  Partial edge tiles are masked, never padded.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vlp_internal.h"

namespace vlp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

// 16-bit element traits: the MFMA and the fp32 -> element pack.
template <int DT> struct Half16;

template <> struct Half16<VLP_BF16> {
  static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  // Two floats -> packed pair, round to nearest even.
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    bf16x2_t p;
    p[0] = static_cast<__bf16>(x);
    p[1] = static_cast<__bf16>(y);
    return __builtin_bit_cast(uint32_t, p);
  }
};

template <> struct Half16<VLP_FP16> {
  static __device__ __forceinline__ f32x16_t mfma(u32x4_t a, u32x4_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f16x2_t p;
    p[0] = static_cast<_Float16>(x);
    p[1] = static_cast<_Float16>(y);
    return __builtin_bit_cast(uint32_t, p);
  }
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Swap bits 2 and 3 of a key offset: the slot a key occupies in the
// transposed V tile (see the header comment).
__device__ __forceinline__ int vslot(int key) {
  return (key & ~12) | ((key & 4) << 1) | ((key & 8) >> 1);
}

// Workgroup -> (sequence, local tile) through the ragged-grid metadata.
struct TileCoord {
  int seq, tile, head;
  int q_start, lq, k_start, lk;
};

__device__ __forceinline__ bool decode_workgroup(const AttnArgs& a, TileCoord& tc) {
  const int heads = a.heads;
  const int slot = static_cast<int>(blockIdx.x) / heads;
  tc.head = static_cast<int>(blockIdx.x) - slot * heads;
  const int g = a.num_blocks >= 0 ? a.num_blocks : a.block_offsets[a.num_seqs];
  if (slot >= g || slot >= a.grid_cap) return false;
  const int f = a.tile_order ? a.tile_order[slot] : slot;
  if (f < 0 || f >= a.grid_cap) return false;  // out-of-contract metadata: skip, never read past it
  tc.seq = a.grid_mapping[f];
  if (tc.seq < 0 || tc.seq >= a.num_seqs) return false;
  tc.tile = f - a.block_offsets[tc.seq];
  tc.q_start = a.cu_q[tc.seq];
  tc.lq = a.cu_q[tc.seq + 1] - tc.q_start;
  tc.k_start = a.cu_k[tc.seq];
  tc.lk = a.cu_k[tc.seq + 1] - tc.k_start;
  return true;
}

// Online-softmax step for one block of scores held as NS registers of 16
// values per lane (scores of one query row per lane; see the header comment).
// The reference max m (log2 units) moves lazily: only when some row of the
// wave meets a block max more than kRescaleLog2 above it are the running
// output and sum rescaled, for the whole wave at once.  Between rescales the
// probabilities exp2(s*c - m) may reach 2^kRescaleLog2, which the fp32 sum
// and the bf16/fp16/fp32 P operand hold without loss of range; the final
// normalisation uses the same m, so the result is the exact softmax.
// Overwrites s with the unnormalised probabilities; l is this half-wave's
// partial row sum.
constexpr float kRescaleLog2 = 8.0f;

template <int NS, int NA>
__device__ __forceinline__ void softmax_step(f32x16_t (&s)[NS], f32x16_t (&acc)[NA], float& m, float& l,
                                             float scale_log2) {
  // Four independent max / sum chains instead of one long dependent chain.
  float mx4[4] = {kNegInf, kNegInf, kNegInf, kNegInf};
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx4[r & 3] = fmaxf(mx4[r & 3], s[i][r]);
  float mx = fmaxf(fmaxf(mx4[0], mx4[1]), fmaxf(mx4[2], mx4[3]));
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float mt = mx * scale_log2;
  if (__builtin_amdgcn_ballot_w64(mt > m + kRescaleLog2)) {
    const float m_new = fmaxf(m, mt);
    const float alpha = m_new == kNegInf ? 1.0f : fast_exp2(m - m_new);
#pragma unroll
    for (int d = 0; d < NA; ++d)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[d][r] *= alpha;
    l *= alpha;
    m = m_new;
  }
  const float m_use = m == kNegInf ? 0.0f : m;
  float sum4[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = fast_exp2(__builtin_fmaf(s[i][r], scale_log2, -m_use));
      s[i][r] = p;
      sum4[r & 3] += p;
    }
  l += (sum4[0] + sum4[1]) + (sum4[2] + sum4[3]);
}

// Sets scores of invisible keys to -inf.  kb: first key of the block;
// row: this lane's local query row; diag = Lk - Lq.
template <int NS, bool CAUSAL>
__device__ __forceinline__ void mask_scores(f32x16_t (&s)[NS], int kb, int hh, int lk, int row, int diag) {
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kb + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
      bool vis = key < lk;
      if (CAUSAL) vis = vis && key <= row + diag;
      if (!vis) s[i][r] = kNegInf;
    }
}

// ---------------------------------------------------------------------------
// 16-bit inputs (bf16 / fp16)
//
// Pipeline per key block (BN keys): the block's K (row-major) and V
// (transposed) sit in one of two LDS buffers; while the waves run QK^T,
// softmax and PV on it, the next block is already in the other buffer and
// the one after is in flight from HBM into registers.  One workgroup barrier
// per block.  Waves whose rows see none of a block's keys (causal) skip its
// arithmetic but still share the loads and the barrier.
// ---------------------------------------------------------------------------
template <int DT, int D, int NW, int BN, bool CAUSAL>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_h16(const AttnArgs a) {
  static_assert(D % 32 == 0 || D == 16, "head_dim");
  static_assert(BN % 32 == 0, "block_n");
  using E = Half16<DT>;
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int KS = D / 16;                    // k-steps of QK^T
  constexpr int DT32 = (D + 31) / 32;           // 32-wide output column tiles
  constexpr int NS = BN / 32;                   // 32-key score tiles per block
  constexpr int KSTR = D + 8;                   // K tile row stride (elements)
  constexpr int VSTR = BN + 8;                  // transposed V row stride
  constexpr int DCH = D / 8;                    // 16-byte chunks per row
  constexpr int KTASKS = BN * DCH;              // 16-byte K chunks per block
  constexpr int KIT = (KTASKS + NT - 1) / NT;
  constexpr int VTASKS = (BN / 4) * DCH;        // (4 keys x 8 columns) V tasks per block
  constexpr int VIT = (VTASKS + NT - 1) / NT;

  __shared__ __attribute__((aligned(16))) uint16_t ks_lds[2][BN * KSTR];
  __shared__ __attribute__((aligned(16))) uint16_t vt_lds[2][(DT32 * 32) * VSTR];

  TileCoord tc;
  if (!decode_workgroup(a, tc)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int row0 = tc.tile * BM;
  const int tile_rows = min(BM, tc.lq - row0);
  const int wrow0 = row0 + 32 * wave;
  const int my_row = wrow0 + n;
  const bool row_ok = my_row < tc.lq;
  const int diag = tc.lk - tc.lq;
  const size_t rs = static_cast<size_t>(a.heads) * D;  // token row stride

  int kv_end = tc.lk;
  if (CAUSAL) kv_end = min(tc.lk, row0 + tile_rows + diag);
  if (kv_end < 0) kv_end = 0;
  const int nblocks = (kv_end + BN - 1) / BN;
  const bool wave_live = wrow0 < tc.lq;
  int wave_kv_end = tc.lk;
  if (CAUSAL) wave_kv_end = min(tc.lk, min(wrow0 + 32, tc.lq) + diag);

  // Q^T operand: this lane's query row, k-chunk hh of every 16-wide step.
  // Rows past the sequence end load the last real row instead (their
  // results are never stored), so every load is unconditional.
  u32x4_t qv[KS];
  {
    const int qrow = min(my_row, tc.lq - 1);
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                         (static_cast<size_t>(tc.q_start + qrow) * a.heads + tc.head) * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) qv[k] = *reinterpret_cast<const u32x4_t*>(qp + 16 * k + 8 * hh);
  }
  // Keep the Q loads ahead of the K/V prologue: if they were issued after it,
  // the wait for Q inside the loop would also wait out every K/V prefetch.
  __builtin_amdgcn_sched_barrier(0);

  f32x16_t acc[DT32];
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.0f;
  float m = kNegInf;
  float l = 0.0f;

  const uint16_t* kbase = static_cast<const uint16_t*>(a.k) +
                          (static_cast<size_t>(tc.k_start) * a.heads + tc.head) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v) +
                          (static_cast<size_t>(tc.k_start) * a.heads + tc.head) * D;

  // Register staging of one key block in 16-byte chunks.  Rows past the
  // sequence end load the sequence's last row instead: their scores are
  // masked to -inf (probability 0), so no value from outside the sequence is
  // ever read and every load is unconditional (no per-lane branches, which
  // keeps the compiler's load counting exact and the prefetch in flight).
  u32x4_t kpre[KIT];
  u32x4_t vpre[VIT][4];
  const int last_row = tc.lk - 1;
  auto load_block = [&](int kb) {
#pragma unroll
    for (int i = 0; i < KIT; ++i) {
      const int c = tid + i * NT;
      if (KTASKS % NT == 0 || c < KTASKS) {
        const int r = min(kb + c / DCH, last_row), col = c % DCH;
        kpre[i] = *reinterpret_cast<const u32x4_t*>(kbase + (size_t)r * rs + col * 8);
      }
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int c = tid + i * NT;
      if (VTASKS % NT == 0 || c < VTASKS) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = min(kb + 4 * (c / DCH) + j, last_row);
          vpre[i][j] = *reinterpret_cast<const u32x4_t*>(vbase + (size_t)key * rs + (c % DCH) * 8);
        }
      }
    }
  };
  auto store_block = [&](int buf) {
#pragma unroll
    for (int i = 0; i < KIT; ++i) {
      const int c = tid + i * NT;
      if (KTASKS % NT == 0 || c < KTASKS) {
        const int r = c / DCH, col = c % DCH;
        *reinterpret_cast<u32x4_t*>(&ks_lds[buf][r * KSTR + col * 8]) = kpre[i];
      }
    }
#pragma unroll
    for (int i = 0; i < VIT; ++i) {
      const int c = tid + i * NT;
      if (VTASKS % NT == 0 || c < VTASKS) {
        const int quad = c / DCH, col = c % DCH;
        const int slot = vslot(4 * quad);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const int sh = (e & 1) * 16;
          u32x2_t pk;
          pk[0] = ((vpre[i][0][w] >> sh) & 0xffffu) | (((vpre[i][1][w] >> sh) & 0xffffu) << 16);
          pk[1] = ((vpre[i][2][w] >> sh) & 0xffffu) | (((vpre[i][3][w] >> sh) & 0xffffu) << 16);
          *reinterpret_cast<u32x2_t*>(&vt_lds[buf][(col * 8 + e) * VSTR + slot]) = pk;
        }
      }
    }
  };

  // The loop sits inside this branch so that no path reaches it with the Q
  // loads still in flight (which would make every iteration wait for all
  // outstanding loads, prefetch included).  nblocks is uniform over the
  // workgroup, so the barriers inside are too.
  if (nblocks > 0) {
    load_block(0);
    store_block(0);
    if (nblocks > 1) load_block(BN);
    __syncthreads();

  for (int it = 0; it < nblocks; ++it) {
    const int buf = it & 1;
    const int kb = it * BN;
    if (wave_live && kb < wave_kv_end) {
      // S^T = K Q^T for NS tiles of 32 keys.
      f32x16_t s[NS];
#pragma unroll
      for (int i = 0; i < NS; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[i][r] = 0.0f;
#pragma unroll
        for (int k = 0; k < KS; ++k) {
          const u32x4_t kop =
              *reinterpret_cast<const u32x4_t*>(&ks_lds[buf][(32 * i + n) * KSTR + 16 * k + 8 * hh]);
          s[i] = E::mfma(kop, qv[k], s[i]);
        }
      }
      const bool need_mask = (kb + BN > tc.lk) || (CAUSAL && kb + BN - 1 > wrow0 + diag);
      if (need_mask) mask_scores<NS, CAUSAL>(s, kb, hh, tc.lk, my_row, diag);
      softmax_step<NS, DT32>(s, acc, m, l, a.scale_log2);

      // O^T += V^T P^T.
#pragma unroll
      for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          u32x4_t pop;
#pragma unroll
          for (int j = 0; j < 4; ++j) pop[j] = E::pack2(s[i][8 * kk + 2 * j], s[i][8 * kk + 2 * j + 1]);
#pragma unroll
          for (int d = 0; d < DT32; ++d) {
            const u32x4_t vop = *reinterpret_cast<const u32x4_t*>(
                &vt_lds[buf][(32 * d + n) * VSTR + 32 * i + 16 * kk + 8 * hh]);
            acc[d] = E::mfma(vop, pop, acc[d]);
          }
        }
    }
    if (it + 1 < nblocks) {
      store_block(buf ^ 1);                         // block it+1, loaded one block ago
      if (it + 2 < nblocks) load_block((it + 2) * BN);
    }
    __syncthreads();
  }
  }

  // Epilogue: normalise, round to the element type, store real rows only.
  const float l_tot = l + __shfl_xor(l, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* op = static_cast<uint16_t*>(a.out) +
                 (static_cast<size_t>(tc.q_start + my_row) * a.heads + tc.head) * D;
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * d + 8 * g + 4 * hh;
      if (col < D) {
        u32x2_t pk;
        pk[0] = E::pack2(acc[d][4 * g + 0] * inv, acc[d][4 * g + 1] * inv);
        pk[1] = E::pack2(acc[d][4 * g + 2] * inv, acc[d][4 * g + 3] * inv);
        *reinterpret_cast<u32x2_t*>(op + col) = pk;
      }
    }
  if (a.lse && hh == 0)
    a.lse[static_cast<size_t>(tc.head) * a.rows_q + tc.q_start + my_row] =
        l_tot > 0.0f ? (m + __log2f(l_tot)) * kLn2 : kNegInf;
}

// ---------------------------------------------------------------------------
// fp32 inputs
// ---------------------------------------------------------------------------
template <int D, int NW, int BN, bool CAUSAL>
__global__ __launch_bounds__(NW * 64) void attn_fwd_f32(const AttnArgs a) {
  static_assert(D % 16 == 0, "head_dim");
  static_assert(BN % 32 == 0, "block_n");
  constexpr int BM = 32 * NW;
  constexpr int NT = NW * 64;
  constexpr int HALF = D / 2;                   // d-values per half-wave
  constexpr int DT32 = (D + 31) / 32;
  constexpr int NS = BN / 32;
  constexpr int STR = D + 4;                    // row stride (floats)
  constexpr int DCH = D / 4;                    // 16-byte chunks per row

  __shared__ __attribute__((aligned(16))) float ks_lds[BN * STR];
  __shared__ __attribute__((aligned(16))) float vs_lds[BN * STR];

  TileCoord tc;
  if (!decode_workgroup(a, tc)) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int row0 = tc.tile * BM;
  const int tile_rows = min(BM, tc.lq - row0);
  const int wrow0 = row0 + 32 * wave;
  const int my_row = wrow0 + n;
  const bool row_ok = my_row < tc.lq;
  const int diag = tc.lk - tc.lq;
  const size_t rs = static_cast<size_t>(a.heads) * D;

  int kv_end = tc.lk;
  if (CAUSAL) kv_end = min(tc.lk, row0 + tile_rows + diag);
  if (kv_end < 0) kv_end = 0;
  const int nblocks = (kv_end + BN - 1) / BN;
  const bool wave_live = wrow0 < tc.lq;
  int wave_kv_end = tc.lk;
  if (CAUSAL) wave_kv_end = min(tc.lk, min(wrow0 + 32, tc.lq) + diag);

  // Q^T operand: contraction index d is split as d = hh * D/2 + step, so a
  // lane keeps the half hh of its query row.
  f32x4_t qv[HALF / 4];
  {
    const float* qp = static_cast<const float*>(a.q) +
                      (static_cast<size_t>(tc.q_start + my_row) * a.heads + tc.head) * D + hh * HALF;
#pragma unroll
    for (int j = 0; j < HALF / 4; ++j)
      qv[j] = row_ok ? *reinterpret_cast<const f32x4_t*>(qp + 4 * j) : f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  f32x16_t acc[DT32];
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.0f;
  float m = kNegInf;
  float l = 0.0f;

  const float* kbase = static_cast<const float*>(a.k) + (static_cast<size_t>(tc.k_start) * a.heads + tc.head) * D;
  const float* vbase = static_cast<const float*>(a.v) + (static_cast<size_t>(tc.k_start) * a.heads + tc.head) * D;

  for (int it = 0; it < nblocks; ++it) {
    const int kb = it * BN;
    __syncthreads();
    for (int c = tid; c < BN * DCH; c += NT) {
      const int r = c / DCH, col = c - (c / DCH) * DCH;
      f32x4_t kv = f32x4_t{0.f, 0.f, 0.f, 0.f}, vv = kv;
      if (kb + r < tc.lk) {
        kv = *reinterpret_cast<const f32x4_t*>(kbase + (size_t)(kb + r) * rs + col * 4);
        vv = *reinterpret_cast<const f32x4_t*>(vbase + (size_t)(kb + r) * rs + col * 4);
      }
      *reinterpret_cast<f32x4_t*>(&ks_lds[r * STR + col * 4]) = kv;
      *reinterpret_cast<f32x4_t*>(&vs_lds[r * STR + col * 4]) = vv;
    }
    __syncthreads();
    if (!wave_live || kb >= wave_kv_end) continue;

    f32x16_t s[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = 0.0f;
#pragma unroll
      for (int j = 0; j < HALF / 4; ++j) {
        const f32x4_t kop = *reinterpret_cast<const f32x4_t*>(&ks_lds[(32 * i + n) * STR + hh * HALF + 4 * j]);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(kop[e], qv[j][e], s[i], 0, 0, 0);
      }
    }
    const bool need_mask = (kb + BN > tc.lk) || (CAUSAL && kb + BN - 1 > wrow0 + diag);
    if (need_mask) mask_scores<NS, CAUSAL>(s, kb, hh, tc.lk, my_row, diag);
    softmax_step<NS, DT32>(s, acc, m, l, a.scale_log2);

    // O^T += V^T P^T, one key pair per MFMA: half hh supplies the key its
    // score register r holds.
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
#pragma unroll
        for (int d = 0; d < DT32; ++d) {
          const float vop = (32 * d + n < D) ? vs_lds[key * STR + 32 * d + n] : 0.0f;
          acc[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop, s[i][r], acc[d], 0, 0, 0);
        }
      }
  }

  const float l_tot = l + __shfl_xor(l, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float* op = static_cast<float*>(a.out) + (static_cast<size_t>(tc.q_start + my_row) * a.heads + tc.head) * D;
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * d + 8 * g + 4 * hh;
      if (col < D) {
        f32x4_t o;
        o[0] = acc[d][4 * g + 0] * inv;
        o[1] = acc[d][4 * g + 1] * inv;
        o[2] = acc[d][4 * g + 2] * inv;
        o[3] = acc[d][4 * g + 3] * inv;
        *reinterpret_cast<f32x4_t*>(op + col) = o;
      }
    }
  if (a.lse && hh == 0)
    a.lse[static_cast<size_t>(tc.head) * a.rows_q + tc.q_start + my_row] =
        l_tot > 0.0f ? (m + __log2f(l_tot)) * kLn2 : kNegInf;
}

}  // namespace vlp
