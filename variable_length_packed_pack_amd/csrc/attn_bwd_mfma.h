// Tiled packed-attention backward on gfx950 matrix cores (device code).
//
// What is computed: the gradients of out = softmax(scale * Q_i K_i^T) V_i,
// per sequence i and head, given dO ("gigl.nn.packed_attention", "Why this
// exists": the packed path is trained through, with gradients from a
// backward kernel; "So you wanna CUDA Graph", "Correctness tangent": rows
// owned by no sequence get no gradient).  With P the softmax weights,
//   dV = P^T dO,  dP = dO V^T,  dS = P * (dP - delta),  delta = rowsum(dO * O),
//   dQ = scale * dS K,  dK = scale * dS^T Q.
// P is recomputed from the forward's log-sum-exp: P = exp2(s * scale*log2(e)
// - lse*log2(e)), so no score matrix is ever stored.
//
// Two kernels, no atomics, so every gradient is the same bit for bit from
// run to run and under any tile order:
//   * attn_bwd_dq_*   walks the query tiles of the forward's ragged grid
//     ("PyCoRa", "CoRa Metadata"; "So you wanna CUDA Graph", "Scheduling
//     without max_seqlen").  A wavefront keeps 32 query rows of Q and dO in
//     registers, streams the sequence's K/V blocks through LDS and
//     accumulates dQ.  It also writes, for every query row, delta and the
//     log-sum-exp in exp2 units (+inf for a row that sees no key, so that
//     its weights come out as exact zeros) into a workspace.
//   * attn_bwd_dkdv_* walks a ragged grid built over the KEY lengths.  A
//     wavefront keeps 32 key rows of K and V in registers, streams the
//     sequence's Q/dO blocks (with their delta and log-sum-exp) through LDS
//     and accumulates dK and dV.  Under the causal mask the first key tile of
//     a sequence is the one every query sees, so the grid's last-tile-first
//     order is mirrored within each sequence: the heaviest tiles still start
//     first.
//
// Both kernels reuse the forward's tile machinery (attn_fwd_mfma.h): 16-byte
// chunk-swizzled row-major LDS tiles filled by direct buffer-to-LDS loads
// (zeros past the sequence end), two LDS buffers with one barrier per block,
// the 32x32x16 MFMA orientation with the streamed tile as the A operand and
// the register-resident rows as the B operand, and the transposing LDS read
// for the second product.  Per block of streamed rows Y against resident
// rows X:
//   dQ kernel   (X = Q|dO, Y = K|V):  S^T = K Q^T, dP^T = V dO^T,
//               dQ^T += K^T dS^T  (K^T by transposing reads of the K tile).
//   dKdV kernel (X = K|V, Y = Q|dO):  S = Q K^T,   dP = dO V^T,
//               dV^T += dO^T P, dK^T += Q^T dS  (transposing reads of the
//               dO and Q tiles).
// In both, the lane holds one X row and 16 Y rows per 32-row Y tile, and the
// 8 values a lane passes as the B operand of k-step kk are Y rows
// 16kk + 8(j/4) + 4hh + (j%4), exactly the rows the two transposing reads
// deliver (see the forward's PV step).
#pragma once

#include "attn_fwd_mfma.h"

namespace vlp {

constexpr float kLog2e = 1.4426950408889634f;

// Task -> (sequence, local tile, head) for a backward launch.  KEY_GRID: the
// grid was built over the key lengths, and local tiles run in mirrored order.
// Tasks are laid out as in the forward (head fastest) and run as there: one
// per workgroup on the static grid, from the work queues on the persistent
// grid.
struct BwdTile {
  int seq, tile, head;
  int q_start, lq, k_start, lk;
};

__device__ __forceinline__ int bwd_active_tasks(const BwdArgs& a) {
  const int g = min(a.block_offsets[a.num_seqs], a.grid_cap);
  return g > 0 ? g * a.heads : 0;
}

template <bool KEY_GRID>
__device__ __forceinline__ bool decode_bwd(const BwdArgs& a, int task, BwdTile& t) {
  const int heads = a.heads;
  const int slot = task / heads;
  t.head = task - slot * heads;
  const int f = a.tile_order ? a.tile_order[slot] : slot;
  if (f < 0 || f >= a.grid_cap) return false;  // out-of-contract metadata: skip, never read past it
  t.seq = a.grid_mapping[f];
  if (t.seq < 0 || t.seq >= a.num_seqs) return false;
  t.tile = f - a.block_offsets[t.seq];
  if (KEY_GRID) t.tile = a.block_offsets[t.seq + 1] - a.block_offsets[t.seq] - 1 - t.tile;
  t.q_start = a.cu_q[t.seq];
  t.lq = a.cu_q[t.seq + 1] - t.q_start;
  t.k_start = a.cu_k[t.seq];
  t.lk = a.cu_k[t.seq + 1] - t.k_start;
  return true;
}

// Two packed 16-bit values -> floats.
template <int DT> struct Widen16;
template <> struct Widen16<VLP_BF16> {
  static __device__ __forceinline__ void get(uint32_t x, float& lo, float& hi) {
    lo = __uint_as_float(x << 16);
    hi = __uint_as_float(x & 0xffff0000u);
  }
};
template <> struct Widen16<VLP_FP16> {
  static __device__ __forceinline__ void get(uint32_t x, float& lo, float& hi) {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, x);
    lo = static_cast<float>(h[0]);
    hi = static_cast<float>(h[1]);
  }
};

// Two independent products over KS k-steps, issued as one alternating MFMA
// stream: acc_a[i] = Ya_i Xa^T and acc_b[i] = Yb_i Xb^T, where A = rows
// 32i + (lane&31) of the Y tile (chunk offsets yoff[k]) and B = this lane's
// resident row x[k].  One product of one 32-row tile alone would be a single
// chain of dependent MFMAs, each waiting for its predecessor's result; two
// products of NS tiles give 2*NS independent accumulators.  Operand reads
// are issued AHEAD MFMAs ahead of their use (an LDS read takes several MFMA
// issue slots to return).
template <int DT, int NS, int KS, int RB>
__device__ __forceinline__ void mma_rows2(const char* tile_a, const u32x4_t (&xa)[KS], f32x16_t (&acc_a)[NS],
                                          const char* tile_b, const u32x4_t (&xb)[KS], f32x16_t (&acc_b)[NS],
                                          const int (&yoff)[KS]) {
  using E = Half16<DT>;
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      acc_a[i][r] = 0.0f;
      acc_b[i][r] = 0.0f;
    }
#pragma unroll
  for (int k = 0; k < KS; ++k)
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const u32x4_t ya = *reinterpret_cast<const u32x4_t*>(tile_a + 32 * i * RB + yoff[k]);
      const u32x4_t yb = *reinterpret_cast<const u32x4_t*>(tile_b + 32 * i * RB + yoff[k]);
      acc_a[i] = E::mfma(ya, xa[k], acc_a[i]);
      acc_b[i] = E::mfma(yb, xb[k], acc_b[i]);
    }
  constexpr int NM = 2 * KS * NS;
  constexpr int AHEAD = NM < 4 ? NM : 4;
  __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);  // DS reads
#pragma unroll
  for (int t = 0; t < NM; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
    if (t + AHEAD < NM) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the next read
  }
}

// acc[d] += Y^T W: A = the Y tile read transposed (offsets ytoff, as the
// forward's V^T operand), B = the weights w (Y rows x this lane's X row),
// rounded to the element type.
template <int DT, int NS, int DT32, int RB>
__device__ __forceinline__ void mma_tr(const char* tile, const int (&ytoff)[2][DT32], const f32x16_t (&w)[NS],
                                       f32x16_t (&acc)[DT32]) {
  using E = Half16<DT>;
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      u32x4_t wop;
#pragma unroll
      for (int j = 0; j < 4; ++j) wop[j] = E::pack2(w[i][8 * kk + 2 * j], w[i][8 * kk + 2 * j + 1]);
#pragma unroll
      for (int d = 0; d < DT32; ++d) {
        const char* base = tile + (32 * i + 16 * kk) * RB;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VLP_LDS i16x4_t*)(base + ytoff[0][d]));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((VLP_LDS i16x4_t*)(base + ytoff[1][d]));
        u32x4_t yop;
        yop[0] = __builtin_bit_cast(u32x2_t, lo)[0];
        yop[1] = __builtin_bit_cast(u32x2_t, lo)[1];
        yop[2] = __builtin_bit_cast(u32x2_t, hi)[0];
        yop[3] = __builtin_bit_cast(u32x2_t, hi)[1];
        acc[d] = E::mfma(yop, wop, acc[d]);
      }
    }
  // Two transposing reads per MFMA, issued AHEAD MFMAs ahead.
  constexpr int NM = NS * 2 * DT32;
  constexpr int AHEAD = NM < 3 ? NM : 3;
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);
#pragma unroll
  for (int t = 0; t < NM; ++t) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (t + AHEAD < NM) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// Operand offsets shared by both kernels (bytes within one tile).
template <int D, int KS, int DT32, int RB>
__device__ __forceinline__ void tile_offsets(int lane, int (&yoff)[KS], int (&ytoff)[2][DT32]) {
  const int n = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int k = 0; k < KS; ++k) yoff[k] = n * RB + (((2 * k + hh) ^ chunk_swz<D>(n)) << 4);
  const int g = lane >> 4, s = lane & 15;
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int r = 8 * e + 4 * (g >> 1) + (s >> 2);
#pragma unroll
    for (int dt = 0; dt < DT32; ++dt) {
      const int dcol = (32 * dt + 16 * (g & 1) + 4 * (s & 3)) & (D - 1);
      ytoff[e][dt] = r * RB + ((((dcol >> 3) ^ chunk_swz<D>(r)) << 4) | ((dcol & 7) * 2));
    }
  }
}

// Direct-load lane offsets for a tile of rows with the given row stride.
template <int D, int LPW, int RPI, int CPR>
__device__ __forceinline__ void load_offsets(int wave, int lane, int rs_bytes, int (&voff)[LPW]) {
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int j = wave * LPW + i;
    const int r = j * RPI + lane / CPR;
    const int c = (lane % CPR) ^ chunk_swz<D>(r);
    voff[i] = r * rs_bytes + c * 16;
  }
}

// Store a transposed accumulator (lane: one row, d = 32dt + 8g + 4hh + 0..3)
// times `factor` as one row of D elements.
template <int DT, int D, int DT32>
__device__ __forceinline__ void store_row_t(uint16_t* rowp, const f32x16_t (&acc)[DT32], float factor, int hh) {
  using E = Half16<DT>;
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * d + 8 * g + 4 * hh;
      if (col < D) {
        u32x2_t pk;
        pk[0] = E::pack2(acc[d][4 * g + 0] * factor, acc[d][4 * g + 1] * factor);
        pk[1] = E::pack2(acc[d][4 * g + 2] * factor, acc[d][4 * g + 3] * factor);
        *reinterpret_cast<u32x2_t*>(rowp + col) = pk;
      }
    }
}

// ---------------------------------------------------------------------------
// dQ (and delta, lse in exp2 units) over the query tiles.
// ---------------------------------------------------------------------------
template <int DT, int D, int NW, int BN, bool CAUSAL>
__device__ __forceinline__ void attn_bwd_dq_h16_task(const BwdArgs& a, int task, char* lds0, char* lds1) {
  static_assert(D == 16 || D == 32 || D == 64 || D == 128, "head_dim");
  static_assert(BN % 32 == 0, "block_n");
  constexpr int BM = 32 * NW;
  constexpr int KS = D / 16;
  constexpr int DT32 = (D + 31) / 32;
  constexpr int NS = BN / 32;
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int LPT = BN / RPI;
  static_assert(LPT % NW == 0, "tile loads must split evenly over the waves");
  constexpr int LPW = LPT / NW;
  constexpr int TILE = BN * RB;

  BwdTile tc;
  if (!decode_bwd<false>(a, task, tc)) return;

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
  const int rs_bytes = a.kv_stride * 2;  // k / v tiles

  int kv_end = tc.lk;
  if (CAUSAL) kv_end = min(tc.lk, row0 + tile_rows + diag);
  if (kv_end < 0) kv_end = 0;
  const int nblocks = (kv_end + BN - 1) / BN;
  const bool wave_live = wrow0 < tc.lq;
  int wave_kv_end = tc.lk;
  if (CAUSAL) wave_kv_end = min(tc.lk, min(wrow0 + 32, tc.lq) + diag);

  // Resident rows: Q and dO of this lane's query (rows past the sequence end
  // repeat the last real row; their results are never stored).
  const int qrow = min(my_row, tc.lq - 1);
  const size_t qrow_g = static_cast<size_t>(tc.q_start + qrow), hoff = static_cast<size_t>(tc.head) * D;
  u32x4_t qv[KS], dov[KS];
  float delta;
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qrow_g * a.q_stride + hoff;
    const uint16_t* dop = static_cast<const uint16_t*>(a.dout) + qrow_g * a.do_stride + hoff;
    const uint16_t* op = static_cast<const uint16_t*>(a.out) + qrow_g * a.o_stride + hoff;
    float part = 0.0f;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      qv[k] = *reinterpret_cast<const u32x4_t*>(qp + 16 * k + 8 * hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) qv[k][j] = flip_sign16x2(qv[k][j], a.negate);
      dov[k] = *reinterpret_cast<const u32x4_t*>(dop + 16 * k + 8 * hh);
      const u32x4_t ov = *reinterpret_cast<const u32x4_t*>(op + 16 * k + 8 * hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float o0, o1, g0, g1;
        Widen16<DT>::get(ov[j], o0, o1);
        Widen16<DT>::get(dov[k][j], g0, g1);
        part = __builtin_fmaf(o0, g0, __builtin_fmaf(o1, g1, part));
      }
    }
    delta = part + __shfl_xor(part, 32);
  }
  const size_t sidx = static_cast<size_t>(tc.head) * a.rows_q + tc.q_start + qrow;
  const float lse = a.lse[sidx];
  const float lse2 = lse == kNegInf ? __builtin_inff() : lse * kLog2e;
  if (row_ok && hh == 0) {
    a.lse2[sidx] = lse2;
    a.delta[sidx] = delta;
  }

  int voff[LPW];
  load_offsets<D, LPW, RPI, CPR>(wave, lane, rs_bytes, voff);
  int yoff[KS], ytoff[2][DT32];
  tile_offsets<D, KS, DT32, RB>(lane, yoff, ytoff);

  f32x16_t acc[DT32];
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.0f;

  const size_t kv_off = (static_cast<size_t>(tc.k_start) * a.kv_stride + static_cast<size_t>(tc.head) * D) * 2;
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
    f32x16_t s[NS], dp[NS];
    mma_rows2<DT, NS, KS, RB>(kt, qv, s, vt, dov, dp, yoff);  // S^T = K Q^T, dP^T = V dO^T
    const bool need_mask = (kb + BN > tc.lk) || (CAUSAL && kb + BN - 1 > wrow0 + diag);
    if (need_mask) mask_scores<NS, CAUSAL>(s, kb, hh, tc.lk, my_row, diag);
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[i][r], a.scale_log2, -lse2));
        s[i][r] = p * (dp[i][r] - delta);  // dS^T
      }
    mma_tr<DT, NS, DT32, RB>(kt, ytoff, s, acc);  // dQ^T += K^T dS^T
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

  if (!row_ok) return;
  store_row_t<DT, D, DT32>(static_cast<uint16_t*>(a.dq) + qrow_g * a.dq_stride + hoff, acc, a.scale, hh);
}

template <int DT, int D, int NW, int BN, bool CAUSAL, bool PERSISTENT>
__global__ __launch_bounds__(NW * 64, 2) void attn_bwd_dq_h16(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds0[2 * (BN * D * 2)];  // buffer 0: K tile, V tile
  __shared__ __attribute__((aligned(1024))) char lds1[2 * (BN * D * 2)];  // buffer 1
  const int tasks = bwd_active_tasks(a);
  if constexpr (PERSISTENT) {
    int* mailbox = reinterpret_cast<int*>(lds0);
    run_claimed_tasks(tasks, a.task_counter, mailbox, [&](int task) __attribute__((always_inline)) {
      attn_bwd_dq_h16_task<DT, D, NW, BN, CAUSAL>(task_args<BwdArgs>(), task, lds0, lds1);
    });
  } else {
    const int task = blockIdx.x;
    if (task < tasks) {
      attn_bwd_dq_h16_task<DT, D, NW, BN, CAUSAL>(a, task, lds0, lds1);
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV over the key tiles.
// ---------------------------------------------------------------------------
template <int DT, int D, int NW, int BQ, bool CAUSAL>
__device__ __forceinline__ void attn_bwd_dkdv_h16_task(const BwdArgs& a, int task, char* lds0, char* lds1) {
  static_assert(D == 16 || D == 32 || D == 64 || D == 128, "head_dim");
  static_assert(BQ % 64 == 0, "4-byte direct loads move the row statistics 64 rows at a time");
  constexpr int BK = 32 * NW;
  constexpr int KS = D / 16;
  constexpr int DT32 = (D + 31) / 32;
  constexpr int NS = BQ / 32;
  constexpr int RB = D * 2;
  constexpr int CPR = D / 8;
  constexpr int RPI = 64 / CPR;
  constexpr int LPT = BQ / RPI;
  static_assert(LPT % NW == 0, "tile loads must split evenly over the waves");
  constexpr int LPW = LPT / NW;
  constexpr int TILE = BQ * RB;
  constexpr int STATS = 2 * TILE;  // lse2[BQ], then delta[BQ]

  BwdTile tc;
  if (!decode_bwd<true>(a, task, tc)) return;

  const int tid = task_tid();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int key0 = tc.tile * BK;
  const int wk0 = key0 + 32 * wave;
  const int my_key = wk0 + n;
  const bool key_ok = my_key < tc.lk;
  const int diag = tc.lk - tc.lq;
  const int rs_q = a.q_stride * 2, rs_do = a.do_stride * 2;  // q / dout tiles

  // Queries that see some key of this tile: p + diag >= key0 when causal.
  const int q_begin = CAUSAL ? max(0, key0 - diag) : 0;
  const int nblocks = tc.lq > q_begin ? (tc.lq - q_begin + BQ - 1) / BQ : 0;
  const bool wave_live = wk0 < tc.lk;
  const int wave_q_begin = CAUSAL ? max(0, wk0 - diag) : 0;

  // Resident rows: K and V of this lane's key.
  const int krow = min(my_key, tc.lk - 1);
  const size_t krow_g = static_cast<size_t>(tc.k_start + krow), hoff = static_cast<size_t>(tc.head) * D;
  const size_t kidx = krow_g * a.kv_stride + hoff;
  u32x4_t kv[KS], vv[KS];
  {
    const uint16_t* kp = static_cast<const uint16_t*>(a.k) + kidx;
    const uint16_t* vp = static_cast<const uint16_t*>(a.v) + kidx;
#pragma unroll
    for (int k = 0; k < KS; ++k) {
      kv[k] = *reinterpret_cast<const u32x4_t*>(kp + 16 * k + 8 * hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) kv[k][j] = flip_sign16x2(kv[k][j], a.negate);
      vv[k] = *reinterpret_cast<const u32x4_t*>(vp + 16 * k + 8 * hh);
    }
  }

  int voff[LPW], voff_do[LPW];
  load_offsets<D, LPW, RPI, CPR>(wave, lane, rs_q, voff);
  load_offsets<D, LPW, RPI, CPR>(wave, lane, rs_do, voff_do);
  int yoff[KS], ytoff[2][DT32];
  tile_offsets<D, KS, DT32, RB>(lane, yoff, ytoff);

  f32x16_t dk[DT32], dv[DT32];
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[d][r] = 0.0f;
      dv[d][r] = 0.0f;
    }

  const char* qseq = static_cast<const char*>(a.q) + (static_cast<size_t>(tc.q_start) * a.q_stride + hoff) * 2;
  const char* doseq = static_cast<const char*>(a.dout) + (static_cast<size_t>(tc.q_start) * a.do_stride + hoff) * 2;
  const size_t stat0 = static_cast<size_t>(tc.head) * a.rows_q + tc.q_start;

  auto issue_block = [&](int qb, char* buf) {
    const int nrows = min(BQ, tc.lq - qb);
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(qseq + static_cast<size_t>(qb) * rs_q), 0, (nrows - 1) * rs_q + RB, 0x00020000);
    const __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char*>(doseq + static_cast<size_t>(qb) * rs_do), 0, (nrows - 1) * rs_do + RB, 0x00020000);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int j = wave * LPW + i;
      const int vo = voff[i];  // (local copies: passing voff[i] directly drops the host-side kernel stub)
      const int vd = voff_do[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, (VLP_LDS void*)(buf + j * 1024), 16, vo, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (VLP_LDS void*)(buf + TILE + j * 1024), 16, vd, 0, 0, 0);
    }
    if (wave == 0) {
      // 64 lanes x 4 bytes per load: the block's lse2 and delta (zeros past
      // the end).
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(a.lse2 + stat0 + qb, 0, nrows * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t rdl = __builtin_amdgcn_make_buffer_rsrc(a.delta + stat0 + qb, 0, nrows * 4, 0x00020000);
#pragma unroll
      for (int j = 0; j < BQ / 64; ++j) {
        const int lo = lane * 4 + 256 * j;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (VLP_LDS void*)(buf + STATS + 256 * j), 4, lo, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rdl, (VLP_LDS void*)(buf + STATS + 4 * BQ + 256 * j), 4, lo, 0, 0, 0);
      }
    }
  };

  auto compute_block = [&](int qb, const char* buf) {
    if (!(wave_live && qb + BQ > wave_q_begin)) return;
    const char* qt = buf;
    const char* dot = buf + TILE;
    const float* st_l = reinterpret_cast<const float*>(buf + STATS);
    const float* st_d = st_l + BQ;
    const bool need_mask = (qb + BQ > tc.lq) || (CAUSAL && qb + diag < wk0 + 31);
    // Both 32-query sub-tiles' S and dP as one MFMA stream over four
    // accumulators (one wave per SIMD holds 2*NS score tiles next to the
    // resident rows and the AGPR accumulators), then the exponentials, then
    // the transposed products; per element and accumulator the same
    // operations in the same order as one sub-tile at a time (measured 4 %
    // faster on the Zipf batch).
    f32x16_t s[NS], dp[NS];
    mma_rows2<DT, NS, KS, RB>(qt, kv, s, dot, vv, dp, yoff);  // S = Q K^T, dP = dO V^T
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      // Masking in a pass of its own, skipped as a whole on blocks that need
      // none: folded into the exponential loop below, it was compiled into
      // per-element selects executed on every block (the backward ran ~20 %
      // slower).
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qb + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
          bool vis = q < tc.lq;
          if (CAUSAL) vis = vis && my_key <= q + diag;
          if (!vis) s[i][r] = kNegInf;
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qr = 32 * i + 8 * g + 4 * hh;  // rows qr .. qr+3 of the block
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(st_l + qr);
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(st_d + qr);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          const float sv = s[i][r];
          const float p = fast_exp2(__builtin_fmaf(sv, a.scale_log2, -l4[e]));
          s[i][r] = p;                        // P
          dp[i][r] = p * (dp[i][r] - d4[e]);  // dS
        }
      }
    }
    mma_tr<DT, NS, DT32, RB>(dot, ytoff, s, dv);  // dV^T += dO^T P
    mma_tr<DT, NS, DT32, RB>(qt, ytoff, dp, dk);  // dK^T += Q^T dS
  };

  if (nblocks > 0) {
    issue_block(q_begin, lds0);
    wait_vmem_all();
    __syncthreads();
    for (int it = 0; it < nblocks; it += 2) {
      if (it + 1 < nblocks) issue_block(q_begin + (it + 1) * BQ, lds1);
      compute_block(q_begin + it * BQ, lds0);
      wait_vmem_all();
      __syncthreads();
      if (it + 1 >= nblocks) break;
      if (it + 2 < nblocks) issue_block(q_begin + (it + 2) * BQ, lds0);
      compute_block(q_begin + (it + 1) * BQ, lds1);
      wait_vmem_all();
      __syncthreads();
    }
  }

  if (!key_ok) return;
  const size_t dkidx = krow_g * a.dkv_stride + hoff;
  store_row_t<DT, D, DT32>(static_cast<uint16_t*>(a.dk) + dkidx, dk, a.scale, hh);
  store_row_t<DT, D, DT32>(static_cast<uint16_t*>(a.dv) + dkidx, dv, 1.0f, hh);
}

template <int DT, int D, int NW, int BQ, bool CAUSAL, bool PERSISTENT>
__global__ __launch_bounds__(NW * 64, D == 128 ? 1 : 2) void attn_bwd_dkdv_h16(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds0[2 * (BQ * D * 2) + 8 * BQ];  // Q tile, dO tile, statistics
  __shared__ __attribute__((aligned(1024))) char lds1[2 * (BQ * D * 2) + 8 * BQ];
  const int tasks = bwd_active_tasks(a);
  if constexpr (PERSISTENT) {
    int* mailbox = reinterpret_cast<int*>(lds0);
    run_claimed_tasks(tasks, a.task_counter, mailbox, [&](int task) __attribute__((always_inline)) {
      attn_bwd_dkdv_h16_task<DT, D, NW, BQ, CAUSAL>(task_args<BwdArgs>(), task, lds0, lds1);
    });
  } else {
    const int task = blockIdx.x;
    if (task < tasks) {
      attn_bwd_dkdv_h16_task<DT, D, NW, BQ, CAUSAL>(a, task, lds0, lds1);
    }
  }
}

}  // namespace vlp
