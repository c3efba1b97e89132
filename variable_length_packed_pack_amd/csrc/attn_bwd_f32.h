// Tiled packed-attention backward for fp32 inputs (device code).
//
// The same two kernels and formulas as the 16-bit backward (attn_bwd_mfma.h)
// -- dQ over the query tiles (also writing delta and lse in exp2 units),
// dK/dV over the key tiles in mirrored longest-first order -- built on
// v_mfma_f32_32x32x2_f32 the way the fp32 forward is (attn_fwd_mfma.h): A and
// B operands are one element per lane with k = hh, so
//   * products contracting over d (S, dP) split d as hh*D/2 + step: a lane
//     keeps half of its resident row and reads 16-byte chunks of the
//     streamed tile;
//   * products contracting over the streamed rows (dQ^T += K^T dS^T, dV^T +=
//     dO^T P, dK^T += Q^T dS) take one streamed row per MFMA: the lane's own
//     score register supplies B, and A is a single 4-byte LDS read of that
//     row at column 32dt + (lane & 31), so no tile is transposed.
// Tiles are row-major, chunk-swizzled (chunk_swz_f32), filled by direct
// buffer-to-LDS loads that return zeros past the sequence end, two LDS
// buffers and one barrier per block.  Everything is fp32 end to end, as the
// graph transformer of "gigl.nn.packed_attention" ("Why this exists") runs it.
#pragma once

#include "attn_bwd_mfma.h"

namespace vlp {

// Rows of the lse2 / delta arrays staged per query block (one 4-byte direct
// load of 64 lanes each).
constexpr int kStatRows = 64;

// acc[i] = Y_i X^T: A = 16-byte chunks of row 32i + (lane&31) of the Y tile
// (chunk offsets yoff[j] cover this lane's half of d), B = the resident half
// row xv.
template <int NS, int HALF, int RB>
__device__ __forceinline__ void mma_rows_f32(const char* tile, const int (&yoff)[HALF / 4],
                                             const f32x4_t (&xv)[HALF / 4], f32x16_t (&acc)[NS]) {
#pragma unroll
  for (int i = 0; i < NS; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.0f;
#pragma unroll
    for (int j = 0; j < HALF / 4; ++j) {
      const f32x4_t yop = *reinterpret_cast<const f32x4_t*>(tile + 32 * i * RB + yoff[j]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[i] = __builtin_amdgcn_mfma_f32_32x32x2f32(yop[e], xv[j][e], acc[i], 0, 0, 0);
    }
  }
}

// acc[d] += Y^T W over the NS*32 streamed rows: one row pair per MFMA; half
// hh supplies the row its register r stands for.
template <int D, int NS, int DT32, int RB>
__device__ __forceinline__ void mma_cols_f32(const char* tile, const f32x16_t (&w)[NS], f32x16_t (&acc)[DT32],
                                             int n, int hh) {
  const int col_chunk = n >> 2, col_byte = (n & 3) * 4;
#pragma unroll
  for (int i = 0; i < NS; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
      const char* yrow = tile + row * RB;
      const int sw = chunk_swz_f32<D>(row);
#pragma unroll
      for (int d = 0; d < DT32; ++d) {
        const float yop = (32 * d + n < D)
                              ? *reinterpret_cast<const float*>(yrow + (((8 * d + col_chunk) ^ sw) << 4) + col_byte)
                              : 0.0f;
        acc[d] = __builtin_amdgcn_mfma_f32_32x32x2f32(yop, w[i][r], acc[d], 0, 0, 0);
      }
    }
}

template <int D, int DT32>
__device__ __forceinline__ void store_row_t_f32(float* rowp, const f32x16_t (&acc)[DT32], float factor, int hh) {
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int col = 32 * d + 8 * g + 4 * hh;
      if (col < D) {
        f32x4_t o;
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = acc[d][4 * g + e] * factor;
        *reinterpret_cast<f32x4_t*>(rowp + col) = o;
      }
    }
}

// Direct-load lane offsets for fp32 tiles.
template <int D, int LPW, int RPI, int CPR>
__device__ __forceinline__ void load_offsets_f32(int wave, int lane, int rs_bytes, int (&voff)[LPW]) {
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int j = wave * LPW + i;
    const int r = j * RPI + lane / CPR;
    const int c = (lane % CPR) ^ chunk_swz_f32<D>(r);
    voff[i] = r * rs_bytes + c * 16;
  }
}

// ---------------------------------------------------------------------------
// dQ (and delta, lse in exp2 units) over the query tiles, fp32.
// ---------------------------------------------------------------------------
template <int D, int NW, int BN, bool CAUSAL>
__device__ __forceinline__ void attn_bwd_dq_f32_task(const BwdArgs& a, int task, char* lds0, char* lds1) {
  static_assert(D % 16 == 0, "head_dim");
  static_assert(BN % 32 == 0, "block_n");
  constexpr int BM = 32 * NW;
  constexpr int HALF = D / 2;
  constexpr int DT32 = (D + 31) / 32;
  constexpr int NS = BN / 32;
  constexpr int RB = D * 4;
  constexpr int CPR = D / 4;
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
  const int rs_bytes = a.kv_stride * 4;  // k / v tiles

  int kv_end = tc.lk;
  if (CAUSAL) kv_end = min(tc.lk, row0 + tile_rows + diag);
  if (kv_end < 0) kv_end = 0;
  const int nblocks = (kv_end + BN - 1) / BN;
  const bool wave_live = wrow0 < tc.lq;
  int wave_kv_end = tc.lk;
  if (CAUSAL) wave_kv_end = min(tc.lk, min(wrow0 + 32, tc.lq) + diag);

  // Resident half rows of Q and dO; delta from the forward output row.
  const int qrow = min(my_row, tc.lq - 1);
  const size_t qrow_g = static_cast<size_t>(tc.q_start + qrow), hoff = static_cast<size_t>(tc.head) * D;
  f32x4_t qv[HALF / 4], dov[HALF / 4];
  float delta;
  {
    const float* qp = static_cast<const float*>(a.q) + qrow_g * a.q_stride + hoff + hh * HALF;
    const float* dop = static_cast<const float*>(a.dout) + qrow_g * a.do_stride + hoff + hh * HALF;
    const float* op = static_cast<const float*>(a.out) + qrow_g * a.o_stride + hoff + hh * HALF;
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < HALF / 4; ++j) {
      qv[j] = *reinterpret_cast<const f32x4_t*>(qp + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) qv[j][e] = flip_sign(qv[j][e], a.negate);
      dov[j] = *reinterpret_cast<const f32x4_t*>(dop + 4 * j);
      const f32x4_t ov = *reinterpret_cast<const f32x4_t*>(op + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) part = __builtin_fmaf(ov[e], dov[j][e], part);
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
  load_offsets_f32<D, LPW, RPI, CPR>(wave, lane, rs_bytes, voff);
  int koff[HALF / 4];
#pragma unroll
  for (int j = 0; j < HALF / 4; ++j) koff[j] = n * RB + (((hh * (HALF / 4) + j) ^ chunk_swz_f32<D>(n)) << 4);

  f32x16_t acc[DT32];
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[d][r] = 0.0f;

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
    f32x16_t s[NS], dp[NS];
    mma_rows_f32<NS, HALF, RB>(kt, koff, qv, s);   // S^T = K Q^T
    mma_rows_f32<NS, HALF, RB>(vt, koff, dov, dp);  // dP^T = V dO^T
    const bool need_mask = (kb + BN > tc.lk) || (CAUSAL && kb + BN - 1 > wrow0 + diag);
    if (need_mask) mask_scores<NS, CAUSAL>(s, kb, hh, tc.lk, my_row, diag);
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(__builtin_fmaf(s[i][r], a.scale_log2, -lse2));
        s[i][r] = p * (dp[i][r] - delta);  // dS^T
      }
    mma_cols_f32<D, NS, DT32, RB>(kt, s, acc, n, hh);  // dQ^T += K^T dS^T
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
  store_row_t_f32<D, DT32>(static_cast<float*>(a.dq) + qrow_g * a.dq_stride + hoff, acc, a.scale, hh);
}

template <int D, int NW, int BN, bool CAUSAL, bool PERSISTENT>
__global__ __launch_bounds__(NW * 64, 2) void attn_bwd_dq_f32(const BwdArgs a) {
  __shared__ __attribute__((aligned(1024))) char lds0[2 * (BN * D * 4)];  // buffer 0: K tile, V tile
  __shared__ __attribute__((aligned(1024))) char lds1[2 * (BN * D * 4)];  // buffer 1
  const int tasks = bwd_active_tasks(a);
  if constexpr (PERSISTENT) {
    int* mailbox = reinterpret_cast<int*>(lds0);
    run_claimed_tasks(tasks, a.task_counter, mailbox, [&](int task) __attribute__((always_inline)) {
      attn_bwd_dq_f32_task<D, NW, BN, CAUSAL>(task_args<BwdArgs>(), task, lds0, lds1);
    });
  } else {
    const int task = blockIdx.x;
    if (task < tasks) {
      attn_bwd_dq_f32_task<D, NW, BN, CAUSAL>(a, task, lds0, lds1);
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV over the key tiles, fp32.
// ---------------------------------------------------------------------------
template <int D, int NW, int BQ, bool CAUSAL>
__device__ __forceinline__ void attn_bwd_dkdv_f32_task(const BwdArgs& a, int task, char* lds0, char* lds1) {
  static_assert(D % 16 == 0, "head_dim");
  static_assert(BQ % 32 == 0 && BQ <= kStatRows, "query block");
  constexpr int BK = 32 * NW;
  constexpr int HALF = D / 2;
  constexpr int DT32 = (D + 31) / 32;
  constexpr int NS = BQ / 32;
  constexpr int RB = D * 4;
  constexpr int CPR = D / 4;
  constexpr int RPI = 64 / CPR;
  constexpr int LPT = BQ / RPI;
  static_assert(LPT % NW == 0, "tile loads must split evenly over the waves");
  constexpr int LPW = LPT / NW;
  constexpr int TILE = BQ * RB;
  constexpr int STATS = 2 * TILE;  // lse2[kStatRows], then delta[kStatRows]

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
  const int rs_q = a.q_stride * 4, rs_do = a.do_stride * 4;  // q / dout tiles

  const int q_begin = CAUSAL ? max(0, key0 - diag) : 0;
  const int nblocks = tc.lq > q_begin ? (tc.lq - q_begin + BQ - 1) / BQ : 0;
  const bool wave_live = wk0 < tc.lk;
  const int wave_q_begin = CAUSAL ? max(0, wk0 - diag) : 0;

  // Resident half rows of K and V.
  const int krow = min(my_key, tc.lk - 1);
  const size_t krow_g = static_cast<size_t>(tc.k_start + krow), hoff = static_cast<size_t>(tc.head) * D;
  const size_t kidx = krow_g * a.kv_stride + hoff;
  f32x4_t kv[HALF / 4], vv[HALF / 4];
  {
    const float* kp = static_cast<const float*>(a.k) + kidx + hh * HALF;
    const float* vp = static_cast<const float*>(a.v) + kidx + hh * HALF;
#pragma unroll
    for (int j = 0; j < HALF / 4; ++j) {
      kv[j] = *reinterpret_cast<const f32x4_t*>(kp + 4 * j);
#pragma unroll
      for (int e = 0; e < 4; ++e) kv[j][e] = flip_sign(kv[j][e], a.negate);
      vv[j] = *reinterpret_cast<const f32x4_t*>(vp + 4 * j);
    }
  }

  int voff[LPW], voff_do[LPW];
  load_offsets_f32<D, LPW, RPI, CPR>(wave, lane, rs_q, voff);
  load_offsets_f32<D, LPW, RPI, CPR>(wave, lane, rs_do, voff_do);
  int qoff[HALF / 4];
#pragma unroll
  for (int j = 0; j < HALF / 4; ++j) qoff[j] = n * RB + (((hh * (HALF / 4) + j) ^ chunk_swz_f32<D>(n)) << 4);

  f32x16_t dk[DT32], dv[DT32];
#pragma unroll
  for (int d = 0; d < DT32; ++d)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dk[d][r] = 0.0f;
      dv[d][r] = 0.0f;
    }

  const char* qseq = static_cast<const char*>(a.q) + (static_cast<size_t>(tc.q_start) * a.q_stride + hoff) * 4;
  const char* doseq = static_cast<const char*>(a.dout) + (static_cast<size_t>(tc.q_start) * a.do_stride + hoff) * 4;
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
      // 64 lanes x 4 bytes: the block's lse2 and delta (zeros past the end).
      const __amdgpu_buffer_rsrc_t rl = __builtin_amdgcn_make_buffer_rsrc(a.lse2 + stat0 + qb, 0, nrows * 4, 0x00020000);
      const __amdgpu_buffer_rsrc_t rdl = __builtin_amdgcn_make_buffer_rsrc(a.delta + stat0 + qb, 0, nrows * 4, 0x00020000);
      const int lo = lane * 4;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rl, (VLP_LDS void*)(buf + STATS), 4, lo, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rdl, (VLP_LDS void*)(buf + STATS + 4 * kStatRows), 4, lo, 0, 0, 0);
    }
  };

  auto compute_block = [&](int qb, const char* buf) {
    if (!(wave_live && qb + BQ > wave_q_begin)) return;
    const char* qt = buf;
    const char* dot = buf + TILE;
    const float* st_l = reinterpret_cast<const float*>(buf + STATS);
    const float* st_d = st_l + kStatRows;
    const bool need_mask = (qb + BQ > tc.lq) || (CAUSAL && qb + diag < wk0 + 31);
    // P and its dV product first, then dP: fewer score tiles live at once.
    f32x16_t s[NS], dp[NS];
    mma_rows_f32<NS, HALF, RB>(qt, qoff, kv, s);  // S = Q K^T
    // Masking in a pass of its own, skipped as a whole where no key of the
    // block needs it (see the 16-bit kernel).
    if (need_mask) {
#pragma unroll
      for (int i = 0; i < NS; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int q = qb + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
          bool vis = q < tc.lq;
          if (CAUSAL) vis = vis && my_key <= q + diag;
          if (!vis) s[i][r] = kNegInf;
        }
    }
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int qr = 32 * i + 8 * g + 4 * hh;  // rows qr .. qr+3 of the block
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(st_l + qr);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * g + e;
          s[i][r] = fast_exp2(__builtin_fmaf(s[i][r], a.scale_log2, -l4[e]));  // P
        }
      }
    mma_cols_f32<D, NS, DT32, RB>(dot, s, dv, n, hh);  // dV^T += dO^T P
    mma_rows_f32<NS, HALF, RB>(dot, qoff, vv, dp);     // dP = dO V^T
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(st_d + 32 * i + 8 * g + 4 * hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[i][4 * g + e] = s[i][4 * g + e] * (dp[i][4 * g + e] - d4[e]);  // dS
      }
    mma_cols_f32<D, NS, DT32, RB>(qt, dp, dk, n, hh);  // dK^T += Q^T dS
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
  store_row_t_f32<D, DT32>(static_cast<float*>(a.dk) + dkidx, dk, a.scale, hh);
  store_row_t_f32<D, DT32>(static_cast<float*>(a.dv) + dkidx, dv, 1.0f, hh);
}

template <int D, int NW, int BQ, bool CAUSAL, bool PERSISTENT>
__global__ __launch_bounds__(NW * 64, D >= 64 ? 1 : 2) void attn_bwd_dkdv_f32(const BwdArgs a) {
  // Per buffer: Q tile, dO tile, statistics.
  __shared__ __attribute__((aligned(1024))) char lds0[2 * (BQ * D * 4) + 8 * kStatRows];
  __shared__ __attribute__((aligned(1024))) char lds1[2 * (BQ * D * 4) + 8 * kStatRows];
  const int tasks = bwd_active_tasks(a);
  if constexpr (PERSISTENT) {
    int* mailbox = reinterpret_cast<int*>(lds0);
    run_claimed_tasks(tasks, a.task_counter, mailbox, [&](int task) __attribute__((always_inline)) {
      attn_bwd_dkdv_f32_task<D, NW, BQ, CAUSAL>(task_args<BwdArgs>(), task, lds0, lds1);
    });
  } else {
    const int task = blockIdx.x;
    if (task < tasks) {
      attn_bwd_dkdv_f32_task<D, NW, BQ, CAUSAL>(a, task, lds0, lds1);
    }
  }
}

}  // namespace vlp
