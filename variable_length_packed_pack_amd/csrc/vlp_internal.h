// Internal declarations shared by the C-ABI layer (api.cpp) and the HIP
// translation units.  Not installed; the public surface is include/vlp.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/vlp.h"

namespace vlp {

// Arguments of one attention launch, passed by value to the kernels.
// Tile metadata follows "PyCoRa", "CoRa Metadata": flat tile f belongs to
// sequence grid_mapping[f] and is its local tile f - block_offsets[seq];
// workgroup slot s runs flat tile tile_order[s] (or s when tile_order is NULL).
struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;                  // [heads, rows_q] or nullptr
  const int32_t* cu_q;         // [num_seqs + 1] (unused in first-token mode)
  const int32_t* cu_k;         // [num_seqs + 1]
  const int32_t* grid_mapping; // [>= G]
  const int32_t* block_offsets;// [num_seqs + 1]
  const int32_t* tile_order;   // [>= G] or nullptr
  int32_t num_seqs;
  int32_t heads;
  int32_t rows_q;
  int32_t num_blocks;          // G when known on the host, -1: read block_offsets[num_seqs]
  int32_t grid_cap;            // entries of grid_mapping / tile_order (guards bad metadata)
  float scale_log2;            // |scale| * log2(e): scores go straight to exp2
  int32_t negate_q;            // 1 when scale < 0: q enters the products negated (see api.cpp)
  // Elements between consecutive tokens (a head's D elements are contiguous
  // and heads are D apart): heads * head_dim for contiguous tensors, more for
  // views into a fused projection output.
  int32_t q_stride;
  int32_t kv_stride;           // k and v
  int32_t o_stride;
  int32_t* task_counter;       // persistent launches: the queue counters (zero at launch)
  // Chunked first-token form only: per-chunk partial states
  // [chunks][heads][head_dim + 4] fp32 (m, l, two unused words, acc) and
  // per-(sequence, head) arrival counters [num_seqs][heads] (zero at launch).
  float* ft_partials;
  int32_t* ft_arrivals;
};

// Arguments of the two backward launches (the dQ kernel over the query
// grid, the dK/dV kernel over the key grid), passed by value.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;            // [heads, rows_q], from the forward
  float* lse2;                 // [heads, rows_q] workspace: lse * log2(e), +inf for keyless rows
  float* delta;                // [heads, rows_q] workspace: rowsum(dout * out)
  void* dq;
  void* dk;
  void* dv;
  const int32_t* cu_q;         // [num_seqs + 1]
  const int32_t* cu_k;         // [num_seqs + 1]
  const int32_t* grid_mapping; // grid of this launch (query grid or key grid)
  const int32_t* block_offsets;
  const int32_t* tile_order;
  int32_t num_seqs;
  int32_t heads;
  int32_t rows_q;
  int32_t grid_cap;
  float scale;                 // factor of dq and dk
  float scale_log2;            // |scale| * log2(e): scores -> exp2 units
  int32_t negate;              // 1 when scale < 0: the register-resident q (dq kernel) or k (dk/dv kernel)
                               // enters the score products negated
  // Elements between consecutive tokens, as in AttnArgs.
  int32_t q_stride;
  int32_t kv_stride;           // k and v
  int32_t o_stride;            // out
  int32_t do_stride;           // dout
  int32_t dq_stride;
  int32_t dkv_stride;          // dk and dv
  int32_t* task_counter;       // persistent launches: the queue counters (zero at launch)
};

// Ragged matrix multiplication tiles: VLP_MATMUL_BLOCK_M token rows x
// kMatmulBlockN output columns per workgroup, kMatmulWavesM x kMatmulWavesN
// wavefronts.
constexpr int kMatmulBlockN = 128;
constexpr int kMatmulWavesM = 2;
constexpr int kMatmulWavesN = 2;

// Arguments of one ragged matrix multiplication launch.
struct MatmulArgs {
  const void* x;               // [rows, k]
  const void* w;               // [num_seqs or 1, n, k]
  const void* bias;            // [num_seqs or 1, n] or nullptr
  void* y;                     // [rows, n]
  const int32_t* cu;           // [num_seqs + 1]
  const int32_t* grid_mapping; // ragged grid over cu with VLP_MATMUL_BLOCK_M rows per tile
  const int32_t* block_offsets;
  int32_t num_seqs;
  int32_t k;
  int32_t n;
  int32_t grid_cap;
  int32_t col_tiles;           // ceil(n / kMatmulBlockN)
  int64_t w_seq_stride;        // elements between sequences' weights (0: shared)
  int64_t b_seq_stride;        // elements between sequences' biases (0: shared)
  int32_t* task_counter;       // persistent launches: the queue counters (zero at launch)
};

// Launch width of a kernel over `tasks` tasks, for the two schedules of "So
// you wanna CUDA Graph" ("Graph overcapture: bound capacity-sized
// launches").  Static grid (workers == kStaticGrid): one workgroup per
// capacity task; tasks past the active count, read on the device, exit at
// once.  Persistent grid: a fixed worker count (kResident: as many
// workgroups of `kernel` as the device holds at once; > 0: at most that
// many) that takes the active tasks from a work queue (run_claimed_tasks).
constexpr int32_t kStaticGrid = 0;
constexpr int32_t kResident = -1;

template <typename Kernel>
inline hipError_t launch_width(Kernel kernel, int threads, int64_t tasks, int32_t workers, int64_t* width) {
  *width = tasks;
  if (workers == kStaticGrid) return hipSuccess;
  if (workers == kResident) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0);
    if (e != hipSuccess) return e;
    workers = per_cu > 0 && cus > 0 ? per_cu * cus : 1;
  }
  if (workers < *width) *width = workers;
  return hipSuccess;
}

// Persistent workgroups take the active tasks from work queues, one per XCD
// (nq = 8 of them; fewer, one per workgroup, when fewer than 8 workgroups
// run).  The hardware deals workgroup b to XCD b % 8 and, on the static
// grid, starts each XCD's workgroups in order; the queues do the same for
// the persistent grid: queue x holds the tasks t = x + nq*i in order of i,
// its first n_x tasks go to the n_x workgroups b = x + nq*i launched on XCD
// x, and each later one to the workgroup that claims it from counter[x] (a
// 256-byte line of its own, zero when the launch starts: the grid build
// that precedes every persistent launch on its stream clears it), as
// i = n_x + the counter's previous value.  A workgroup stops at its first
// claim past `tasks`, so every task runs exactly once and counter[x] ends at
// the number of tasks in queue x.  The longest-first order of the task list
// and the XCD a task's K/V (or rows of x) are cached on are what they are on
// the static grid.
//   The claim for the next task is issued as the current task starts, so
// its latency hides behind the task.  `mailbox` is an int in the kernel's
// own LDS (the first word of a tile buffer, so the persistent kernel needs
// no more LDS, and no lower occupancy, than the static one): between two
// tasks, with every wave past the task's LDS use, thread 0 posts the claim
// there, and every wave reads it before any wave starts the next task.  The
// task index is made wave-uniform, so the task's address arithmetic stays
// scalar.
constexpr int kTaskQueues = 8;
// Elements between two queue counters: one 256-byte line each.  Atomics on
// one line are serialised device-wide (about 10 ns apiece when every
// workgroup claims at once); on separate lines they proceed in parallel.
constexpr int kCounterStride = 64;

// The kernel's argument struct (its first argument, at the start of the
// kernel-argument segment), read through a pointer the compiler cannot see
// through: loads of the arguments stay next to their uses in each task
// instead of being hoisted out of the task loop into scalar registers held
// across it (which spilled to VGPR lanes).
template <typename Args>
__device__ __forceinline__ const Args& task_args() {
  auto p = __builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(p));
  return *(const Args*)p;
}

template <typename Fn>
__device__ __forceinline__ void run_claimed_tasks(int tasks, int32_t* counters, int* mailbox, Fn&& fn) {
  const int w = static_cast<int>(gridDim.x);
  const int nq = w < kTaskQueues ? w : kTaskQueues;  // every queue needs a worker
  const int x = static_cast<int>(blockIdx.x) % nq;
  const int n_x = (w - x + nq - 1) / nq;
  int task = static_cast<int>(blockIdx.x);
  while (task < tasks) {
    int claimed = 0;
    if (threadIdx.x == 0) claimed = atomicAdd(counters + x * kCounterStride, 1);
    fn(task);
    __syncthreads();  // the task's LDS traffic is over
    if (threadIdx.x == 0) *mailbox = x + nq * (n_x + claimed);
    __syncthreads();  // the claim is posted
    task = __builtin_amdgcn_readfirstlane(*mailbox);
    __syncthreads();  // and read by every wave before the LDS is reused
  }
}

// Sign flip of an operand held in registers, for a negative softmax scale:
// scale * (q . k) = |scale| * ((-q) . k) -- the flip negates every product
// exactly, and the sums differ from -(q . k) at most by the accumulation's
// rounding -- so the kernels run with |scale| and keep their running
// maximum order-preserving.  Two 16-bit values per 32-bit word.
__device__ __forceinline__ uint32_t flip_sign16x2(uint32_t x, bool on) { return on ? x ^ 0x80008000u : x; }
__device__ __forceinline__ float flip_sign(float x, bool on) { return on ? -x : x; }

// threadIdx.x behind an empty asm statement.  The task functions of the
// task-looping kernels derive their lane offsets from it, so those offsets
// are recomputed (a few instructions) for each task instead of being hoisted
// out of the task loop and held in registers across it.
__device__ __forceinline__ int task_tid() {
  int t = static_cast<int>(threadIdx.x);
  asm volatile("" : "+v"(t));
  return t;
}

// Kernel families and their tile shapes.  block_m is the query rows per
// workgroup tile; it is what the ragged grid is built with.
struct TileShape {
  int block_m;   // query rows per workgroup
  int block_n;   // keys per inner step
  int waves;     // wavefronts per workgroup
};

// Tile shape vlp_varlen_attn_fwd uses for (dtype, head_dim); block_m = 0 if
// the pair is not built.
TileShape attn_tile_shape(int dtype, int head_dim);

// Launch the tiled MFMA forward over `blocks` tasks (slots * heads); the
// launch width follows `workers` (see launch_width).
hipError_t launch_attn_bf16(const AttnArgs& a, int head_dim, bool causal, int64_t blocks,
                            int32_t workers, hipStream_t s);
hipError_t launch_attn_f16(const AttnArgs& a, int head_dim, bool causal, int64_t blocks,
                           int32_t workers, hipStream_t s);
hipError_t launch_attn_f32(const AttnArgs& a, int head_dim, bool causal, int64_t blocks,
                           int32_t workers, hipStream_t s);

enum class FirstTokenForm { kHeadParallel, kKeySplit, kChunked };

// First-token forward over `slots` tile slots: one wavefront per (sequence,
// head); or eight wavefronts per (sequence, head), each on an eighth of the
// keys (long sequences; see kFirstTokenSplitKeys); or, chunked, eight
// wavefronts per (chunk of kFirstTokenChunkKeys keys, head) with the grid
// built over the keys in chunks.
hipError_t launch_attn_first_token(int dtype, const AttnArgs& a, int head_dim, bool causal, FirstTokenForm form,
                                   int64_t slots, int32_t workers, hipStream_t s);

// First-token launches split each sequence's keys over eight wavefronts when
// the longest sequence (max_seqlen, or the mean length when no hint is
// given) has at least this many keys.
constexpr int64_t kFirstTokenSplitKeys = 1024;

// With a workspace (the device-grid entry points) and at least this many
// keys in the longest sequence, first-token launches take the chunked form:
// a grid over the keys with kFirstTokenChunkKeys keys per tile, one
// workgroup per (chunk, head), the partial states of a sequence merged by
// the workgroup that finishes last.
constexpr int64_t kFirstTokenChunkKeys = VLP_FIRST_TOKEN_CHUNK_KEYS;
constexpr int64_t kFirstTokenChunkMin = VLP_FIRST_TOKEN_CHUNK_MIN;
static_assert(kFirstTokenChunkKeys % 512 == 0, "a chunk splits into 64-key shares of eight waves");
static_assert(kFirstTokenChunkMin >= kFirstTokenChunkKeys, "a chunked launch has sequences of several chunks");

// Backward launches over `blocks` tasks each.
hipError_t launch_attn_bwd_dq_bf16(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                   int32_t workers, hipStream_t s);
hipError_t launch_attn_bwd_dkdv_bf16(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                     int32_t workers, hipStream_t s);
hipError_t launch_attn_bwd_dq_f16(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                  int32_t workers, hipStream_t s);
hipError_t launch_attn_bwd_dkdv_f16(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                    int32_t workers, hipStream_t s);
hipError_t launch_attn_bwd_dq_f32(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                  int32_t workers, hipStream_t s);
hipError_t launch_attn_bwd_dkdv_f32(const BwdArgs& a, int head_dim, bool causal, int64_t blocks,
                                    int32_t workers, hipStream_t s);

// Ragged matrix multiplication over `blocks` tasks.
hipError_t launch_ragged_matmul(int dtype, const MatmulArgs& a, bool bias, int64_t blocks,
                                int32_t workers, hipStream_t s);

// VLP_CHECK=1 debug validation: checks cu[0] == 0, non-decreasing steps,
// cu[num_seqs] <= max_total (and non-empty sequences if asked) on the device
// and waits; *flags != 0 reports a violation (allocates and synchronises:
// not for captured graphs).
hipError_t check_cu_seqlens(const int32_t* cu, int32_t num_seqs, int64_t max_total, bool require_nonempty,
                            hipStream_t s, int32_t* flags);

// Document ids -> cu_seqlens with a fixed capacity (one workgroup).
hipError_t launch_ids_to_cu(const int32_t* ids, int32_t num_tokens, int32_t max_seqs, int32_t* cu, int32_t* num_out,
                            hipStream_t s);

// Scratch of vlp_varlen_attn_fwd_noalloc: a file-scope device array of this
// many bytes on every GPU the library runs on; noalloc_scratch returns the
// current device's copy (its address is looked up once per device).
constexpr size_t kNoallocScratchBytes = VLP_NOALLOC_SCRATCH_BYTES;
hipError_t noalloc_scratch(void** ptr);

// Device ragged-grid build (one workgroup); also zeroes the kTaskQueues
// counters at task_counter (kCounterStride apart) when it is not null (the
// work queues of the persistent launch that follows), and zero_count ints
// at `zero` (counters of the launch that follows).
hipError_t launch_grid_build(const int32_t* cu_seqlens, int32_t num_seqs, int32_t block_m,
                             int32_t* block_offsets, int32_t* grid_mapping, int32_t* tile_order,
                             int64_t grid_cap, int32_t* task_counter, hipStream_t s, int32_t* zero = nullptr,
                             int32_t zero_count = 0);

}  // namespace vlp
