// Two-group ("ping-pong") tiled forward for 16-bit inputs at head_dim 128
// on gfx950 (device code).
//
// Same computation, operand layouts, LDS tile format and online softmax as
// attn_fwd_h16 (attn_fwd_mfma.h: per sequence and head, softmax(scale *
// Q_i K_i^T) V_i over the sequence's own keys, "PyCoRa", "Ragged Flash
// Attention"; tiles routed through grid_mapping / block_offsets), and the
// same per-row arithmetic in the same order, so both kernels give identical
// bits.  What changes is the schedule inside a workgroup:
//
//  * eight waves, 256 query rows per tile: waves 0-3 (group 0) and 4-7
//    (group 1), one wave of each group on every SIMD;
//  * a wave's work on key block j alternates between an MFMA phase M(j) --
//    PV of block j-1, then QK^T of block j -- and a VALU phase V(j) -- mask,
//    online softmax and the bf16/fp16 packing of P_j.  Group 0 runs M(j),
//    V(j) in period j; group 1 runs V(j-1), M(j).  So while group 0 issues
//    MFMAs group 1 does exponentials and the other way round: each SIMD holds
//    one wave of each kind instead of two waves that want the same unit at
//    once, and the MFMA-phase wave runs at raised issue priority.  Periods
//    end at a workgroup barrier; inside a period the two phases of the groups
//    settle into step by themselves (a barrier between them as well, forcing
//    the alternation, measured 0.5 % slower on the Zipf batch and 2 % on the
//    skewed one: it added the waves' skew twice per block);
//  * K and V tiles of 64 keys live in a ring of three LDS slots each, filled
//    by direct buffer-to-LDS loads.  In period i every wave issues its share
//    of K_{i+2} and V_{i+1}; both are first read in period i+2, and each wave
//    waits for them (vmcnt, counting only the newer loads) at the end of
//    period i+1, before the barrier that publishes them.  A ring slot is
//    refilled only after the barrier that ends its last reads (K_{i-1} and
//    V_{i-2} are last read in period i-1).  Blocks past the sequence's last
//    key get an empty buffer descriptor: those loads read no memory and
//    write zeros into a ring slot that is not used, so every wave issues the
//    same number of loads in every period and the vmcnt bound is a
//    constant;
//  * every barrier is reached by all eight waves the same number of times
//    (nblocks + 2 per task, nblocks uniform over the workgroup); waves whose
//    rows see fewer keys (causal) skip the MFMA and VALU work of those
//    blocks but not the barriers or the loads.
#pragma once

#include <type_traits>

#include "attn_fwd_mfma.h"

namespace vlp {

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every load in flight); LDS visibility of the direct loads is
// ordered by the explicit vmcnt waits before it.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt with only the vector-memory counter constrained (to <= N).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

// One task (256 query rows of one head).  k0..k2 and v0..v2 are the ring's
// LDS tiles of BN * D * 2 bytes each.
template <int DT, int D, int BN, bool CAUSAL>
__device__ __forceinline__ void attn_fwd_pingpong_task(const AttnArgs& a, int task, char* k0, char* k1, char* k2,
                                                       char* v0, char* v1, char* v2) {
  using E = Half16<DT>;
  constexpr int NW = 8;
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
  constexpr int NBUF = 3;
  char* const kr[NBUF] = {k0, k1, k2};
  char* const vr[NBUF] = {v0, v1, v2};

  TileCoord tc;
  if (!decode_task(a, task, tc)) return;

  const int tid = task_tid();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int row0 = tc.tile * BM;
  const int tile_rows = min(BM, tc.lq - row0);
  const int wrow0 = row0 + 32 * wave;
  const int my_row = wrow0 + n;
  const bool row_ok = my_row < tc.lq;
  const int diag = tc.lk - tc.lq;
  const int rs_bytes = a.kv_stride * 2;

  int kv_end = tc.lk;
  if (CAUSAL) kv_end = min(tc.lk, row0 + tile_rows + diag);
  if (kv_end < 0) kv_end = 0;
  const int nblocks = (kv_end + BN - 1) / BN;
  const bool wave_live = wrow0 < tc.lq;
  int wave_kv_end = tc.lk;
  if (CAUSAL) wave_kv_end = min(tc.lk, min(wrow0 + 32, tc.lq) + diag);
  // Key blocks this wave computes: a prefix of the workgroup's nblocks.
  const int wave_nb = wave_live ? min(nblocks, (max(wave_kv_end, 0) + BN - 1) / BN) : 0;

  // Q^T operand, direct-load lane offsets, K operand and transposing V^T
  // read offsets: exactly as in attn_fwd_h16_task.
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

  int voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int j = wave * LPW + i;
    const int r = j * RPI + lane / CPR;
    const int c = (lane % CPR) ^ chunk_swz<D>(r);
    voff[i] = r * rs_bytes + c * 16;
  }
  int koff[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) koff[k] = n * RB + (((2 * k + hh) ^ chunk_swz<D>(n)) << 4);
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
  f32x16_t s[NS];     // scores of the last QK block (written in M, read in V)
  u32x4_t p[NS][2];   // packed probabilities of the last softmaxed block (V -> next M)

  const size_t kv_off = (static_cast<size_t>(tc.k_start) * a.kv_stride + static_cast<size_t>(tc.head) * D) * 2;
  const char* kseq = static_cast<const char*>(a.k) + kv_off;
  const char* vseq = static_cast<const char*>(a.v) + kv_off;

  auto issue = [&](const char* seq, int j, char* buf) {
    // A block past the sequence's last key gets an empty buffer: its loads
    // read nothing and fill the (unused) tile with zeros, so every wave
    // issues the same loads in every slot.
    const int kb = j * BN;
    const int nrows = min(BN, tc.lk - kb);
    const int nrec = nrows > 0 ? (nrows - 1) * rs_bytes + RB : 0;
    const size_t boff = nrows > 0 ? static_cast<size_t>(kb) * rs_bytes : 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(seq + boff), 0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int jj = wave * LPW + i;
      const int vo = voff[i];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (VLP_LDS void*)(buf + jj * 1024), 16, vo, 0, 0, 0);
    }
  };

  // S^T = K Q^T for the key block in tile kt (MFMA phase).
  auto qk = [&](const char* kt) {
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
    constexpr int NQK = KS * NS;
    constexpr int QK_AHEAD = NQK < 4 ? NQK : 4;
    __builtin_amdgcn_sched_group_barrier(0x100, QK_AHEAD, 0);
#pragma unroll
    for (int t = 0; t < NQK; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (t + QK_AHEAD < NQK) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
  };

  // O^T += V^T P^T with the packed P of the previous block (MFMA phase).
  auto pv = [&](const char* vt) {
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
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
          acc[d] = E::mfma(vop, p[i][kk], acc[d]);
        }
    constexpr int NPV = NS * 2 * DT32;
    constexpr int PV_AHEAD = NPV < 4 ? NPV : 4;
    __builtin_amdgcn_sched_group_barrier(0x100, 2 * PV_AHEAD, 0);
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if (t + PV_AHEAD < NPV) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
  };

  // Mask, online softmax and packing of P for block j (VALU phase).
  auto softmax = [&](int j) {
    const int kb = j * BN;
    const bool need_mask = (kb + BN > tc.lk) || (CAUSAL && kb + BN - 1 > wrow0 + diag);
    if (need_mask) mask_scores<NS, CAUSAL>(s, kb, hh, tc.lk, my_row, diag);
    softmax_step<NS, DT32>(s, acc, m, l, a.scale_log2);
#pragma unroll
    for (int i = 0; i < NS; ++i)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) p[i][kk][jj] = E::pack2(s[i][8 * kk + 2 * jj], s[i][8 * kk + 2 * jj + 1]);
  };

  // Loads of period i, issued by every wave: K_{i+2} and V_{i+1} (R = i % 3
  // names the ring slots statically).  They may still be in flight at the
  // end of period i; everything older has landed by then (wait_older), in
  // time for the blocks' first use in period i+2.
  auto issue_pair = [&](auto rr, int i) {
    constexpr int R = decltype(rr)::value;
    issue(kseq, i + 2, kr[(R + 2) % NBUF]);
    issue(vseq, i + 1, vr[(R + 1) % NBUF]);
  };
  auto wait_older = [&]() { wait_vmem_le<2 * LPW>(); };

  if (nblocks > 0) {
    issue(kseq, 0, kr[0]);
    issue(kseq, 1, kr[1]);
    issue(vseq, 0, vr[0]);
  }
  wait_vmem_all();
  wg_barrier();
  if (nblocks > 0) {
    // Period j: group 0 runs M(j), V(j); group 1 runs V(j-1), M(j).  M(j) =
    // PV of block j-1, then QK of block j.  One barrier ends each period.
    auto mphase = [&](auto rr, int j) {
      constexpr int R = decltype(rr)::value;
      __builtin_amdgcn_s_setprio(1);
      if (j >= 1 && j - 1 < wave_nb) pv(vr[(R + 2) % NBUF]);
      if (j < wave_nb) qk(kr[R]);
      __builtin_amdgcn_s_setprio(0);
    };
    if (grp == 0) {
      auto body = [&](auto rr, int j) {
        mphase(rr, j);
        issue_pair(rr, j);
        if (j < wave_nb) softmax(j);
        wait_older();
        wg_barrier();
      };
      for (int j = 0; j <= nblocks; j += 3) {
        body(std::integral_constant<int, 0>{}, j);
        if (j + 1 > nblocks) break;
        body(std::integral_constant<int, 1>{}, j + 1);
        if (j + 2 > nblocks) break;
        body(std::integral_constant<int, 2>{}, j + 2);
      }
      wg_barrier();
    } else {
      issue_pair(std::integral_constant<int, 0>{}, 0);  // period 0: M(0) only
      mphase(std::integral_constant<int, 0>{}, 0);
      wait_older();
      wg_barrier();
      // Period j+1: the loads of period j+1, V(j), M(j+1).
      auto body = [&](auto rr, int j) {
        constexpr int R = decltype(rr)::value;
        issue_pair(std::integral_constant<int, (R + 1) % NBUF>{}, j + 1);
        if (j < wave_nb) softmax(j);
        mphase(std::integral_constant<int, (R + 1) % NBUF>{}, j + 1);
        wait_older();
        wg_barrier();
      };
      for (int j = 0; j < nblocks; j += 3) {
        body(std::integral_constant<int, 0>{}, j);
        if (j + 1 >= nblocks) break;
        body(std::integral_constant<int, 1>{}, j + 1);
        if (j + 2 >= nblocks) break;
        body(std::integral_constant<int, 2>{}, j + 2);
      }
      wg_barrier();
    }
  }

  // The last periods' loads (empty blocks past the end) may still be writing
  // LDS; none may outlive the task (the persistent grid reuses the ring).
  wait_vmem_all();

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

template <int DT, int D, int BN, bool CAUSAL, bool PERSISTENT>
__global__ __launch_bounds__(512, 1) void attn_fwd_h16_pingpong(const AttnArgs a) {
  // Three K and three V tiles, each its own array so that the compiler can
  // tell the ring slots apart (no wait for loads into other slots).
  __shared__ __attribute__((aligned(1024))) char k0[BN * D * 2];
  __shared__ __attribute__((aligned(1024))) char k1[BN * D * 2];
  __shared__ __attribute__((aligned(1024))) char k2[BN * D * 2];
  __shared__ __attribute__((aligned(1024))) char v0[BN * D * 2];
  __shared__ __attribute__((aligned(1024))) char v1[BN * D * 2];
  __shared__ __attribute__((aligned(1024))) char v2[BN * D * 2];
  const int tasks = active_tasks(a);
  if constexpr (PERSISTENT) {
    int* mailbox = reinterpret_cast<int*>(k0);
    run_claimed_tasks(tasks, a.task_counter, mailbox, [&](int task) __attribute__((always_inline)) {
      attn_fwd_pingpong_task<DT, D, BN, CAUSAL>(task_args<AttnArgs>(), task, k0, k1, k2, v0, v1, v2);
    });
  } else {
    const int task = blockIdx.x;
    if (task < tasks) attn_fwd_pingpong_task<DT, D, BN, CAUSAL>(a, task, k0, k1, k2, v0, v1, v2);
  }
}

}  // namespace vlp
