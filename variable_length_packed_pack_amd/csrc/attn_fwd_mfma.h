// Tiled packed-attention forward on gfx950 matrix cores (device code).
//
// What is computed: for every sequence i and head h, out = softmax(scale *
// Q_i K_i^T) V_i over that sequence's own keys ("gigl.nn.packed_attention",
// module description and packed_attention; "PyCoRa", "Ragged Flash
// Attention": a tiled online softmax in which each workgroup looks up its
// sequence in grid_mapping and processes only that sequence's tokens).
//
// Work decomposition ("So you wanna CUDA Graph", "Scheduling without
// max_seqlen"): one task per (tile slot, head), head fastest.  Slot s runs
// flat tile f = tile_order[s]; seq = grid_mapping[f]; local tile
// t = f - block_offsets[seq]; tasks of slots >= block_offsets[num_seqs] are
// not run.  On the static grid workgroup b runs task b; on the persistent
// grid a fixed worker count takes the tasks from per-XCD work queues that
// keep task t on XCD t % 8 (run_claimed_tasks).  With head fastest and
// workgroups dealt round-robin to the 8 XCDs, a head count that is a
// multiple of 8 keeps every tile of one (sequence, head) on one XCD, so its
// K/V stay in that XCD's L2.
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
// keys 16*kk + 8*(j/4) + 4*hh + (j%4), j < 8.  For 16-bit inputs the matching
// V^T operand comes from a row-major V tile through gfx950's transposing LDS
// read (see the 16-bit section).  Every per-query quantity (running max, sum,
// rescale factor) is lane-local.
//
// fp32 inputs use v_mfma_f32_32x32x2_f32 (A/B: one element per lane, k = hh)
// with the same S^T / O^T orientation; there V needs no transpose because
// each A operand is a single element.
//
// Masking: key rows past the sequence end are never read from memory (the
// 16-bit path's buffer loads return zeros past the sequence's last row, the
// fp32 path zero-fills), so nothing outside the sequence -- such as NaN in
// unused capacity rows, "So you wanna CUDA Graph", "Correctness tangent" --
// can reach the result; their scores are set to -inf (probability 0); causal
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

// Task -> (sequence, local tile, head) through the ragged-grid metadata.
struct TileCoord {
  int seq, tile, head;
  int q_start, lq, k_start, lk;
};

// Active tasks of a launch: (active tile slots) * heads, the slot count
// read on the device unless the host knows it.
__device__ __forceinline__ int active_tasks(const AttnArgs& a) {
  int g = a.num_blocks >= 0 ? a.num_blocks : a.block_offsets[a.num_seqs];
  g = min(g, a.grid_cap);
  return g > 0 ? g * a.heads : 0;
}

// Task t (< active_tasks) -> (tile slot, head).  The hardware deals
// workgroup t to XCD t % 8 and starts each XCD's workgroups in order (the
// persistent schedule's per-XCD queues keep that), so the decode decides
// which tiles share an XCD's L2 at a time.  Task t is head t % heads of slot
// t / heads -- each XCD interleaves its heads x, x + 8, ... slot by slot --
// except when an XCD has four or more heads (heads a multiple of 32): then
// it runs them one after another, each head's slots in longest-first order,
// so that the tiles resident on an XCD stream one head's K/V.  Measured on
// the skewed batch (32 heads): HBM reads 6.8 -> 5.5 GB per launch, kernel
// 3 % faster; on 16 heads the same order was 1.5 % slower, so two heads per
// XCD stay interleaved.
__device__ __forceinline__ bool decode_task(const AttnArgs& a, int task, TileCoord& tc) {
  const int heads = a.heads;
  int slot;
  if ((heads & 31) == 0) {
    int g = a.num_blocks >= 0 ? a.num_blocks : a.block_offsets[a.num_seqs];
    g = min(g, a.grid_cap);
    if (g <= 0) return false;
    const int i = task >> 3;
    const int j = i / g;
    slot = i - j * g;
    tc.head = (task & 7) + 8 * j;
  } else {
    slot = task / heads;
    tc.head = task - slot * heads;
  }
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

// Maximum over the two half-waves (lanes i and i + 32): v_permlane32_swap
// exchanges the halves of two registers in one VALU step, instead of a
// round trip through the LDS crossbar.
__device__ __forceinline__ float halves_max(float x) {
  float a = x, b = x;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  return fmaxf(a, b);
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
  mx = halves_max(mx);
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
// LDS tiles.  K and V of one key block are both kept row-major (key rows of
// D elements) in LDS, 16-byte chunks XOR-swizzled per row (chunk_swz) so
// that both operand reads below are free of bank conflicts:
//   * K as the A operand of S^T = K Q^T: lane (n, hh) reads row 32i+n, chunk
//     2k+hh with one ds_read_b128.
//   * V^T as the A operand of O^T = V^T P^T: gfx950's transposing LDS read
//     (ds_read_b64_tr_b16) gathers, within each group of 16 lanes, four key
//     rows x 16 columns and hands every lane four consecutive keys of one
//     column.  Two such reads give the eight keys 16kk + 4hh + {0..3, 8..11}
//     that this lane's P^T operand holds for k-step kk, so neither V nor P
//     is permuted anywhere.
// Tiles are filled by direct buffer-to-LDS loads (each lane moves one
// 16-byte chunk; 64 lanes fill 1 KB of LDS per instruction), so the block in
// flight occupies no registers.  The buffer descriptor of a key block ends at
// the sequence's last row, and the hardware returns zeros past it: no value
// outside the sequence -- NaN in unused capacity rows, "So you wanna CUDA
// Graph", "Correctness tangent" -- is ever read, and those keys' scores are
// masked to -inf.
//
// Pipeline: two LDS buffers; while the waves compute on block j, block j+1
// streams into the other buffer; one workgroup barrier per block.  The loop
// is unrolled by two so that every LDS access names its buffer statically.
// ---------------------------------------------------------------------------
typedef short i16x4_t __attribute__((ext_vector_type(4)));
#define VLP_LDS __attribute__((address_space(3)))

// Chunk swizzle of a tile row (chunks of 16 bytes, D/8 per row).
//   D = 128: a row is 256 bytes, all 64 banks.  Rows r..r+15 (K reads) must
//            take 16 different chunk slots, and rows 4m..4m+3 (transposed V
//            reads, 2 adjacent chunks each) must too.
//   D = 64:  two rows share the 64 banks; the even (odd) rows among 16
//            consecutive ones need distinct slots, and rows 4m, 4m+2 (and
//            4m+1, 4m+3) must land in different groups of four slots.
//   D <= 32: not swizzled (edge-case sizes).
template <int D>
__device__ __forceinline__ int chunk_swz(int row) {
  if constexpr (D == 128) {
    return ((row & 3) << 2) | ((row >> 2) & 3);
  } else if constexpr (D == 64) {
    const int x = (row >> 1) & 7;
    return ((x & 1) << 2) | (x & 2) | ((x >> 2) & 1);
  } else {
    return 0;
  }
}

// s_waitcnt with only the vector-memory counter constrained (to 0).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// One task (a tile of BM query rows of one head) of the 16-bit kernel.
// lds0 and lds1 are the workgroup's two LDS buffers of 2 * BN * D * 2 bytes.
template <int DT, int D, int NW, int BN, bool CAUSAL>
__device__ __forceinline__ void attn_fwd_h16_task(const AttnArgs& a, int task, char* lds0, char* lds1) {
  static_assert(D == 16 || D == 32 || D == 64 || D == 128, "head_dim");
  static_assert(BN % 32 == 0, "block_n");
  using E = Half16<DT>;
  constexpr int BM = 32 * NW;
  constexpr int KS = D / 16;           // k-steps of QK^T
  constexpr int DT32 = (D + 31) / 32;  // 32-wide output column tiles
  constexpr int NS = BN / 32;          // 32-key score tiles per block
  constexpr int RB = D * 2;            // bytes per tile row
  constexpr int CPR = D / 8;           // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;        // rows filled by one 1 KB direct load
  constexpr int LPT = BN / RPI;        // direct loads per tile
  static_assert(LPT % NW == 0, "tile loads must split evenly over the waves");
  constexpr int LPW = LPT / NW;        // direct loads per tile per wave
  constexpr int TILE = BN * RB;        // bytes of one K (or V) tile

  TileCoord tc;
  if (!decode_task(a, task, tc)) return;

  const int tid = task_tid();
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
  const int rs_bytes = a.kv_stride * 2;  // bytes between consecutive tokens of one head of k / v

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
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + static_cast<size_t>(tc.q_start + qrow) * a.q_stride +
                         static_cast<size_t>(tc.head) * D;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      qv[k] = *reinterpret_cast<const u32x4_t*>(qp + 16 * k + 8 * hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) qv[k][j] = flip_sign16x2(qv[k][j], a.negate_q);
    }
  }

  // Direct-load lane offsets (bytes, relative to the key block's first row):
  // load j of a tile fills rows j*RPI .. j*RPI+RPI-1; lane -> (row, slot),
  // and the slot holds logical chunk slot ^ chunk_swz(row).  K and V share
  // them.
  int voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int j = wave * LPW + i;
    const int r = j * RPI + lane / CPR;
    const int c = (lane % CPR) ^ chunk_swz<D>(r);
    voff[i] = r * rs_bytes + c * 16;
  }
  // K operand: row 32i+n, logical chunk 2k+hh (the row's swizzle depends on
  // n only, since 32 | 32i).
  int koff[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) koff[k] = n * RB + (((2 * k + hh) ^ chunk_swz<D>(n)) << 4);
  // V^T operand by transposing reads: lane = 16g + s; group g covers key
  // rows base + 0..3 (base = 32i + 16kk + 8e + 4(g>>1)) and columns
  // 32dt + 16(g&1) + 0..15; lane s points at row base + (s>>2), columns
  // +4(s&3) .. +4(s&3)+3.
  int vtoff[2][DT32];
  {
    const int g = lane >> 4, s = lane & 15;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 8 * e + 4 * (g >> 1) + (s >> 2);
#pragma unroll
      for (int dt = 0; dt < DT32; ++dt) {
        const int dcol = (32 * dt + 16 * (g & 1) + 4 * (s & 3)) & (D - 1);
        vtoff[e][dt] = r * RB + ((((dcol >> 3) ^ chunk_swz<D>(r)) << 4) | ((dcol & 7) * 2));
      }
    }
  }

  f32x16_t acc[DT32];
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.0f;
  float m = kNegInf;
  float l = 0.0f;

  const size_t kv_off = (static_cast<size_t>(tc.k_start) * a.kv_stride + static_cast<size_t>(tc.head) * D) * 2;
  const char* kseq = static_cast<const char*>(a.k) + kv_off;
  const char* vseq = static_cast<const char*>(a.v) + kv_off;

  // Stream key block [kb, kb + BN) of K and V into one LDS buffer.
  auto issue_block = [&](int kb, char* buf) {
    const int nrows = min(BN, tc.lk - kb);
    const int nrec = (nrows - 1) * rs_bytes + RB;
    const size_t boff = static_cast<size_t>(kb) * rs_bytes;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kseq + boff), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vseq + boff), 0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int j = wave * LPW + i;
      const int vo = voff[i];  // (a local copy: passing voff[i] directly drops the host-side kernel stub)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (VLP_LDS void*)(buf + j * 1024), 16, vo, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (VLP_LDS void*)(buf + TILE + j * 1024), 16, vo, 0, 0, 0);
    }
  };

  auto compute_block = [&](int kb, const char* buf) {
    if (!(wave_live && kb < wave_kv_end)) return;
    const char* kt = buf;
    const char* vt = buf + TILE;
    // S^T = K Q^T for NS tiles of 32 keys.
    // The NS accumulation chains are interleaved, k outermost.
    f32x16_t s[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k)
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const u32x4_t kop = *reinterpret_cast<const u32x4_t*>(kt + 32 * i * RB + koff[k]);
        s[i] = E::mfma(kop, qv[k], s[i]);
      }
    // Keep the K-operand reads QK_AHEAD MFMAs ahead of their use: an LDS
    // read takes several MFMA issue slots to return.
    constexpr int NQK = KS * NS;
    constexpr int QK_AHEAD = NQK < 4 ? NQK : 4;
    __builtin_amdgcn_sched_group_barrier(0x100, QK_AHEAD, 0);  // DS reads
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      if (t + QK_AHEAD < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next read
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
          const char* base = vt + (32 * i + 16 * kk) * RB;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VLP_LDS i16x4_t*)(base + vtoff[0][d]));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VLP_LDS i16x4_t*)(base + vtoff[1][d]));
          u32x4_t vop;
          vop[0] = __builtin_bit_cast(u32x2_t, lo)[0];
          vop[1] = __builtin_bit_cast(u32x2_t, lo)[1];
          vop[2] = __builtin_bit_cast(u32x2_t, hi)[0];
          vop[3] = __builtin_bit_cast(u32x2_t, hi)[1];
          acc[d] = E::mfma(vop, pop, acc[d]);
        }
      }
  };

  // nblocks is uniform over the workgroup, so every barrier below is too.
  if (nblocks > 0) {
    issue_block(0, lds0);
    wait_vmem_all();
    __syncthreads();
    for (int it = 0; it < nblocks; it += 2) {
      if (it + 1 < nblocks) issue_block((it + 1) * BN, lds1);
      compute_block(it * BN, lds0);
      wait_vmem_all();
      __syncthreads();
      if (it + 1 >= nblocks) break;
      if (it + 2 < nblocks) issue_block((it + 2) * BN, lds0);
      compute_block((it + 1) * BN, lds1);
      wait_vmem_all();
      __syncthreads();
    }
  }

  // Epilogue: normalise, round to the element type, store real rows only.
  const float l_tot = l + __shfl_xor(l, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  uint16_t* op = static_cast<uint16_t*>(a.out) + static_cast<size_t>(tc.q_start + my_row) * a.o_stride +
                 static_cast<size_t>(tc.head) * D;
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

// Static grid (PERSISTENT false): workgroup b runs task b, if it is active.
// Persistent grid: the workgroup runs the tasks it takes from the work
// queues (run_claimed_tasks).  The two are separate instantiations so that
// the static grid's kernel carries no loop.
template <int DT, int D, int NW, int BN, bool CAUSAL, bool PERSISTENT>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_h16(const AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds0[2 * BN * D * 2];  // buffer 0: K tile, V tile
  __shared__ __attribute__((aligned(1024))) char lds1[2 * BN * D * 2];  // buffer 1
  const int tasks = active_tasks(a);
  if constexpr (PERSISTENT) {
    int* mailbox = reinterpret_cast<int*>(lds0);
    run_claimed_tasks(tasks, a.task_counter, mailbox, [&](int task) __attribute__((always_inline)) {
      attn_fwd_h16_task<DT, D, NW, BN, CAUSAL>(task_args<AttnArgs>(), task, lds0, lds1);
    });
  } else {
    const int task = blockIdx.x;
    if (task < tasks) {
      attn_fwd_h16_task<DT, D, NW, BN, CAUSAL>(a, task, lds0, lds1);
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 inputs
//
// Same tile structure as the 16-bit path -- row-major K and V tiles filled
// by direct buffer-to-LDS loads (zeros past the sequence end), two LDS
// buffers, one barrier per key block -- with v_mfma_f32_32x32x2_f32, whose
// A and B operands are one element per lane (k = hh).  S^T = K Q^T: the
// contraction index d is split as d = hh*D/2 + step, so a lane keeps half of
// its query row and reads 16-byte K chunks.  O^T = V^T P^T: one key pair per
// MFMA, so each V^T operand is a single 4-byte read and V needs no
// transpose.  The chunk swizzle makes the K reads (16 consecutive rows, one
// chunk) and the V reads (32 consecutive columns of rows k and k+4) free of
// bank conflicts for rows of 256 bytes and more.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int chunk_swz_f32(int row) {
  if constexpr (D >= 64) {
    return (row & 3) | ((row & 4) << 1) | ((row & 8) >> 1);
  } else {
    return 0;
  }
}

// One task of the fp32 kernel; lds0 and lds1 hold 2 * BN * D * 4 bytes each.
template <int D, int NW, int BN, bool CAUSAL>
__device__ __forceinline__ void attn_fwd_f32_task(const AttnArgs& a, int task, char* lds0, char* lds1) {
  static_assert(D % 16 == 0, "head_dim");
  static_assert(BN % 32 == 0, "block_n");
  constexpr int BM = 32 * NW;
  constexpr int HALF = D / 2;           // d-values per half-wave
  constexpr int DT32 = (D + 31) / 32;   // 32-wide output column tiles
  constexpr int NS = BN / 32;           // 32-key score tiles per block
  constexpr int RB = D * 4;             // bytes per tile row
  constexpr int CPR = D / 4;            // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;         // rows filled by one 1 KB direct load
  constexpr int LPT = BN / RPI;         // direct loads per tile
  static_assert(LPT % NW == 0, "tile loads must split evenly over the waves");
  constexpr int LPW = LPT / NW;
  constexpr int TILE = BN * RB;

  TileCoord tc;
  if (!decode_task(a, task, tc)) return;

  const int tid = task_tid();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int row0 = tc.tile * BM;
  const int tile_rows = min(BM, tc.lq - row0);
  const int wrow0 = row0 + 32 * wave;
  const int my_row = wrow0 + n;
  const bool row_ok = my_row < tc.lq;
  const int diag = tc.lk - tc.lq;
  const int rs_bytes = a.kv_stride * 4;

  int kv_end = tc.lk;
  if (CAUSAL) kv_end = min(tc.lk, row0 + tile_rows + diag);
  if (kv_end < 0) kv_end = 0;
  const int nblocks = (kv_end + BN - 1) / BN;
  const bool wave_live = wrow0 < tc.lq;
  int wave_kv_end = tc.lk;
  if (CAUSAL) wave_kv_end = min(tc.lk, min(wrow0 + 32, tc.lq) + diag);

  // Q^T operand: half hh of this lane's query row (rows past the sequence
  // end load the last real row; their results are never stored).
  f32x4_t qv[HALF / 4];
  {
    const int qrow = min(my_row, tc.lq - 1);
    const float* qp = static_cast<const float*>(a.q) + static_cast<size_t>(tc.q_start + qrow) * a.q_stride +
                      static_cast<size_t>(tc.head) * D + hh * HALF;
#pragma unroll
    for (int j = 0; j < HALF / 4; ++j) {
      qv[j] = *reinterpret_cast<const f32x4_t*>(qp + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[j][e] = flip_sign(qv[j][e], a.negate_q);
    }
  }

  // Direct-load lane offsets (see the 16-bit path).
  int voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int j = wave * LPW + i;
    const int r = j * RPI + lane / CPR;
    const int c = (lane % CPR) ^ chunk_swz_f32<D>(r);
    voff[i] = r * rs_bytes + c * 16;
  }
  // K operand chunks: row 32i+n, logical chunk hh*HALF/4 + j.
  int koff[HALF / 4];
#pragma unroll
  for (int j = 0; j < HALF / 4; ++j) koff[j] = n * RB + (((hh * (HALF / 4) + j) ^ chunk_swz_f32<D>(n)) << 4);
  // V^T operand: row key, column 32d + n; the row's swizzle depends on key & 15,
  // which is 8(r>>2) + 4hh + (r&3) for score register r.
  const int vcol_chunk = n >> 2, vcol_byte = (n & 3) * 4;

  f32x16_t acc[DT32];
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.0f;
  float m = kNegInf;
  float l = 0.0f;

  const size_t kv_off = (static_cast<size_t>(tc.k_start) * a.kv_stride + static_cast<size_t>(tc.head) * D) * 4;
  const char* kseq = static_cast<const char*>(a.k) + kv_off;
  const char* vseq = static_cast<const char*>(a.v) + kv_off;

  auto issue_block = [&](int kb, char* buf) {
    const int nrows = min(BN, tc.lk - kb);
    const int nrec = (nrows - 1) * rs_bytes + RB;
    const size_t boff = static_cast<size_t>(kb) * rs_bytes;
    const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(kseq + boff), 0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(vseq + boff), 0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int j = wave * LPW + i;
      const int vo = voff[i];  // (a local copy: passing voff[i] directly drops the host-side kernel stub)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (VLP_LDS void*)(buf + j * 1024), 16, vo, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (VLP_LDS void*)(buf + TILE + j * 1024), 16, vo, 0, 0, 0);
    }
  };

  auto compute_block = [&](int kb, const char* buf) {
    if (!(wave_live && kb < wave_kv_end)) return;
    const char* kt = buf;
    const char* vt = buf + TILE;
    f32x16_t s[NS];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[i][r] = 0.0f;
#pragma unroll
      for (int j = 0; j < HALF / 4; ++j) {
        const f32x4_t kop = *reinterpret_cast<const f32x4_t*>(kt + 32 * i * RB + koff[j]);
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
        const char* vrow = vt + key * RB;
        const int sw = chunk_swz_f32<D>(key);
#pragma unroll
        for (int d = 0; d < DT32; ++d) {
          const float vop = (32 * d + n < D)
                                ? *reinterpret_cast<const float*>(vrow + (((8 * d + vcol_chunk) ^ sw) << 4) + vcol_byte)
                                : 0.0f;
          acc[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(vop, s[i][r], acc[d], 0, 0, 0);
        }
      }
  };

  if (nblocks > 0) {
    issue_block(0, lds0);
    wait_vmem_all();
    __syncthreads();
    for (int it = 0; it < nblocks; it += 2) {
      if (it + 1 < nblocks) issue_block((it + 1) * BN, lds1);
      compute_block(it * BN, lds0);
      wait_vmem_all();
      __syncthreads();
      if (it + 1 >= nblocks) break;
      if (it + 2 < nblocks) issue_block((it + 2) * BN, lds0);
      compute_block((it + 1) * BN, lds1);
      wait_vmem_all();
      __syncthreads();
    }
  }

  const float l_tot = l + __shfl_xor(l, 32);
  if (!row_ok) return;
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
  float* op = static_cast<float*>(a.out) + static_cast<size_t>(tc.q_start + my_row) * a.o_stride +
              static_cast<size_t>(tc.head) * D;
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

template <int D, int NW, int BN, bool CAUSAL, bool PERSISTENT>
__global__ __launch_bounds__(NW * 64, 2) void attn_fwd_f32(const AttnArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds0[2 * BN * D * 4];  // buffer 0: K tile, V tile
  __shared__ __attribute__((aligned(1024))) char lds1[2 * BN * D * 4];  // buffer 1
  const int tasks = active_tasks(a);
  if constexpr (PERSISTENT) {
    int* mailbox = reinterpret_cast<int*>(lds0);
    run_claimed_tasks(tasks, a.task_counter, mailbox, [&](int task) __attribute__((always_inline)) {
      attn_fwd_f32_task<D, NW, BN, CAUSAL>(task_args<AttnArgs>(), task, lds0, lds1);
    });
  } else {
    const int task = blockIdx.x;
    if (task < tasks) {
      attn_fwd_f32_task<D, NW, BN, CAUSAL>(a, task, lds0, lds1);
    }
  }
}

}  // namespace vlp
