// Ragged matrix multiplication on gfx950 matrix cores.
//
// What is computed ("PyCoRa", "Ragged Matrix Multiplication"): every
// sequence of a packed batch is multiplied by its own weight matrix,
//   y[rows of sequence i] = x[rows of sequence i] W_i^T (+ b_i),
// with W_i in the [out_features, in_features] layout of a linear layer.  A
// weight shared by all sequences (sequence stride 0) is the packed linear
// layer of "gigl.nn.packed_attention" ("Why this exists": the projections run
// on the [num_tokens, dim] buffer, so no work is spent on padding).
//
// Work decomposition: the ragged grid of the attention ("PyCoRa", "CoRa
// Metadata") with 128-row tiles, times 128-column tiles of the output.  A
// workgroup looks its row tile up in grid_mapping / block_offsets and
// multiplies only that sequence's rows by that sequence's weight slice.
// Task t runs on XCD t % 8 (static grid: workgroup t, dealt round-robin to
// the XCDs; persistent grid: the per-XCD work queues).  The task mapping
// below gives each XCD whole row tiles, all their column tiles one after
// another, so a row tile of x is read from HBM once per XCD and then served
// by that XCD's L2.
//
// Per workgroup (4 wavefronts): output tile 128 rows x 128 columns, K in
// stages of 64 staged in LDS (double-buffered, direct buffer-to-LDS loads
// that return zeros past the sequence's last row or the last weight row).
// The product is formed transposed, C^T = W x^T, with v_mfma_f32_32x32x16:
//   A operand = W tile rows (lane: output column n, 8 consecutive k),
//   B operand = x tile rows (lane: token m, the same 8 k),
// both one 16-byte read of a row-major tile whose 16-byte chunks are XOR-
// swizzled per row (chunk_swz<64>: 128-byte rows, conflict-free for 32
// consecutive rows reading one chunk).  C^T leaves each lane holding one
// token's 4 consecutive output columns per register group, stored as one
// 8-byte write.  Each wavefront owns 64 columns x 64 tokens (2 x 2 MFMA
// tiles); fp32 accumulation, one rounding to the element type at the end.
#include "attn_fwd_mfma.h"

namespace vlp {

// Two packed 16-bit values -> floats.
template <int DT> __device__ __forceinline__ void widen_pair(uint32_t x, float& lo, float& hi);
template <> __device__ __forceinline__ void widen_pair<VLP_BF16>(uint32_t x, float& lo, float& hi) {
  lo = __uint_as_float(x << 16);
  hi = __uint_as_float(x & 0xffff0000u);
}
template <> __device__ __forceinline__ void widen_pair<VLP_FP16>(uint32_t x, float& lo, float& hi) {
  const f16x2_t h = __builtin_bit_cast(f16x2_t, x);
  lo = static_cast<float>(h[0]);
  hi = static_cast<float>(h[1]);
}

constexpr int kMmBK = 64;  // in_features per LDS stage

// BM token rows x BN output columns per workgroup, WGM x WGN wavefronts each
// owning (BM / WGM) tokens x (BN / WGN) columns.
template <int DT, bool BIAS, int BM, int BN, int WGM, int WGN>
__device__ __forceinline__ void ragged_matmul_task(const MatmulArgs& a, int task, char* lds0, char* lds1) {
  using E = Half16<DT>;
  constexpr int NW = WGM * WGN;
  constexpr int TM = BM / WGM, TN = BN / WGN;  // wave tile
  constexpr int MI = TM / 32, NI = TN / 32;    // 32 x 32 MFMA tiles per wave
  constexpr int RB = kMmBK * 2;                // bytes per tile row
  constexpr int CPR = RB / 16;                 // 16-byte chunks per row
  constexpr int RPI = 64 / CPR;                // rows per 1 KB direct load
  constexpr int LW = BN / RPI, LX = BM / RPI;  // loads per W / x tile
  static_assert((LW + LX) % NW == 0, "tile loads must split evenly over the waves");
  constexpr int LPW = (LW + LX) / NW;
  constexpr int TW = BN * RB, TX = BM * RB;    // tile bytes
  constexpr int STAGE = TW + TX;

  // Task -> (row slot, column tile), XCD-aware (see the header).
  const int l = task >> 3;
  const int nt = l % a.col_tiles;
  const int slot = (l / a.col_tiles) * 8 + (task & 7);
  const int g = a.block_offsets[a.num_seqs];
  if (slot >= g || slot >= a.grid_cap) return;
  const int seq = a.grid_mapping[slot];
  if (seq < 0 || seq >= a.num_seqs) return;
  const int tile = slot - a.block_offsets[seq];
  const int r_start = a.cu[seq];
  const int row0 = tile * BM;
  const int nrows = min(BM, a.cu[seq + 1] - r_start - row0);
  const int n0 = nt * BN;
  const int ncols = min(BN, a.n - n0);

  const int tid = task_tid();
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31;
  const int hh = lane >> 5;
  const int wn = wave % WGN;
  const int wm = wave / WGN;
  const int k_bytes = a.k * 2;

  // Direct loads: load j < LW fills W rows j*RPI.., the rest x rows; rows of
  // both are k_bytes apart, so the lane offsets have one form.
  int voff[LPW];
#pragma unroll
  for (int i = 0; i < LPW; ++i) {
    const int j = wave * LPW + i;
    const int r = (j < LW ? j : j - LW) * RPI + lane / CPR;
    voff[i] = r * k_bytes + (((lane % CPR) ^ chunk_swz<64>(r)) << 4);
  }
  // Operand offsets within a 32-row sub-tile: row (lane & 31), chunk 2ks + hh.
  int ooff[kMmBK / 16];
#pragma unroll
  for (int ks = 0; ks < kMmBK / 16; ++ks) ooff[ks] = n * RB + (((2 * ks + hh) ^ chunk_swz<64>(n)) << 4);

  const char* xrows = static_cast<const char*>(a.x) + (static_cast<size_t>(r_start) + row0) * k_bytes;
  const char* wrows = static_cast<const char*>(a.w) + (static_cast<size_t>(seq) * a.w_seq_stride +
                                                       static_cast<size_t>(n0) * a.k) * 2;
  const int x_rec = (nrows - 1) * k_bytes + RB;
  const int w_rec = (ncols - 1) * k_bytes + RB;

  auto issue_stage = [&](int kb, char* buf) {
    const __amdgpu_buffer_rsrc_t rw =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(wrows + kb * RB), 0, w_rec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rx =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(xrows + kb * RB), 0, x_rec, 0x00020000);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int j = wave * LPW + i;
      const int vo = voff[i];  // (a local copy: passing voff[i] directly drops the host-side kernel stub)
      if (j < LW)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rw, (VLP_LDS void*)(buf + j * 1024), 16, vo, 0, 0, 0);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (VLP_LDS void*)(buf + j * 1024), 16, vo, 0, 0, 0);
    }
  };

  f32x16_t acc[NI][MI];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < MI; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  auto compute_stage = [&](const char* buf) {
    const char* wt = buf + (TN * wn) * RB;
    const char* xt = buf + TW + (TM * wm) * RB;
#pragma unroll
    for (int ks = 0; ks < kMmBK / 16; ++ks) {
      u32x4_t aop[NI], bop[MI];
#pragma unroll
      for (int i = 0; i < NI; ++i) aop[i] = *reinterpret_cast<const u32x4_t*>(wt + 32 * i * RB + ooff[ks]);
#pragma unroll
      for (int j = 0; j < MI; ++j) bop[j] = *reinterpret_cast<const u32x4_t*>(xt + 32 * j * RB + ooff[ks]);
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int j = 0; j < MI; ++j) acc[i][j] = E::mfma(aop[i], bop[j], acc[i][j]);
    }
  };

  const int nstages = a.k / kMmBK;
  issue_stage(0, lds0);
  wait_vmem_all();
  __syncthreads();
  for (int it = 0; it < nstages; it += 2) {
    if (it + 1 < nstages) issue_stage(it + 1, lds1);
    compute_stage(lds0);
    wait_vmem_all();
    __syncthreads();
    if (it + 1 >= nstages) break;
    if (it + 2 < nstages) issue_stage(it + 2, lds0);
    compute_stage(lds1);
    wait_vmem_all();
    __syncthreads();
  }

  // Epilogue: lane holds token m = TM*wm + 32j + n and, per register group q,
  // output columns TN*wn + 32i + 8q + 4hh + 0..3.
  const char* bias_row =
      BIAS ? static_cast<const char*>(a.bias) + static_cast<size_t>(seq) * a.b_seq_stride * 2 : nullptr;
#pragma unroll
  for (int j = 0; j < MI; ++j) {
    const int m = TM * wm + 32 * j + n;
    if (m >= nrows) continue;
    uint16_t* yrow = static_cast<uint16_t*>(a.y) + (static_cast<size_t>(r_start) + row0 + m) * a.n + n0;
#pragma unroll
    for (int i = 0; i < NI; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = TN * wn + 32 * i + 8 * q + 4 * hh;
        if (col >= ncols) continue;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
        if (BIAS) {
          const u32x2_t bw = *reinterpret_cast<const u32x2_t*>(bias_row + static_cast<size_t>(n0 + col) * 2);
          float b0, b1, b2, b3;
          widen_pair<DT>(bw[0], b0, b1);
          widen_pair<DT>(bw[1], b2, b3);
          v[0] += b0;
          v[1] += b1;
          v[2] += b2;
          v[3] += b3;
        }
        u32x2_t pk;
        pk[0] = E::pack2(v[0], v[1]);
        pk[1] = E::pack2(v[2], v[3]);
        *reinterpret_cast<u32x2_t*>(yrow + col) = pk;
      }
  }
}

// Tasks below 8 * ceil(active slots / 8) * col_tiles run one per workgroup
// on the static grid and from the work queues on the persistent grid.
template <int DT, bool BIAS, int BM, int BN, int WGM, int WGN, bool PERSISTENT>
__global__ __launch_bounds__(WGM * WGN * 64, WGM * WGN == 4 ? 2 : 1) void ragged_matmul_h16(const MatmulArgs a) {
  constexpr int STAGE = (BN + BM) * kMmBK * 2;
  __shared__ __attribute__((aligned(1024))) char lds0[STAGE];  // W tile, x tile
  __shared__ __attribute__((aligned(1024))) char lds1[STAGE];
  const int g = min(a.block_offsets[a.num_seqs], a.grid_cap);
  const int tasks = g > 0 ? ((g + 7) & ~7) * a.col_tiles : 0;
  if constexpr (PERSISTENT) {
    int* mailbox = reinterpret_cast<int*>(lds0);
    run_claimed_tasks(tasks, a.task_counter, mailbox, [&](int task) __attribute__((always_inline)) {
      ragged_matmul_task<DT, BIAS, BM, BN, WGM, WGN>(task_args<MatmulArgs>(), task, lds0, lds1);
    });
  } else {
    const int task = blockIdx.x;
    if (task < tasks) {
      ragged_matmul_task<DT, BIAS, BM, BN, WGM, WGN>(a, task, lds0, lds1);
    }
  }
}

// Tile shape of the launch (the ragged grid's block_m is VLP_MATMUL_BLOCK_M).
constexpr int kMmBM = VLP_MATMUL_BLOCK_M;
constexpr int kMmBN = kMatmulBlockN;
constexpr int kMmWGM = kMatmulWavesM;
constexpr int kMmWGN = kMatmulWavesN;

namespace {

template <int DT, bool BIAS>
hipError_t go(const MatmulArgs& a, int64_t blocks, int32_t workers, hipStream_t s) {
  constexpr int threads = kMmWGM * kMmWGN * 64;
  const auto kernel = workers == kStaticGrid ? ragged_matmul_h16<DT, BIAS, kMmBM, kMmBN, kMmWGM, kMmWGN, false>
                                             : ragged_matmul_h16<DT, BIAS, kMmBM, kMmBN, kMmWGM, kMmWGN, true>;
  int64_t width = 0;
  const hipError_t e = launch_width(kernel, threads, blocks, workers, &width);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(width)), dim3(threads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ragged_matmul(int dtype, const MatmulArgs& a, bool bias, int64_t blocks, int32_t workers,
                                hipStream_t s) {
  if (blocks <= 0) return hipSuccess;
  switch (dtype) {
    case VLP_BF16: return bias ? go<VLP_BF16, true>(a, blocks, workers, s) : go<VLP_BF16, false>(a, blocks, workers, s);
    case VLP_FP16: return bias ? go<VLP_FP16, true>(a, blocks, workers, s) : go<VLP_FP16, false>(a, blocks, workers, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vlp
