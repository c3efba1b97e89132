// First-token packed attention: one query per sequence.
//
// "gigl.nn.packed_attention", packed_attention with query_is_first_token:
// only each sequence's first token is queried (the anchor readout of the
// last layer); query row i belongs to sequence i and sees all of that
// sequence's keys (causal: only key 0, the query sits at position 0).
//
// The work is 4*Lk*D flops against 2*Lk*D*elt bytes of K/V per (sequence,
// head): bandwidth-bound, so no matrix cores.  One wavefront per (sequence,
// head), four heads per workgroup.  A key row of one head is split into
// 16-byte chunks over LPK lanes; the wave covers KPS = 64/LPK keys per step
// and U steps per round for memory parallelism: a wave's rounds form a chain
// of load latencies, so the longest sequences set the kernel's time, and
// U*KPS = 64 keys are kept in flight (U between 4 and 16, the register
// budget of the widest rows).  Each key slot keeps its own online-softmax
// state; slots merge at the end.  The dot products' cross-lane sums use DPP
// row permutations (group_sum).
// Sequences run in tile_order (longest first) through the same ragged-grid
// metadata as the tiled kernel, with one tile per sequence.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vlp_internal.h"

namespace vlp {
namespace {

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;
constexpr int kSplitWaves = 8;  // waves sharing one long sequence's keys in the key-split form

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT> struct Chunk;  // 16 bytes of one key row, widened to fp32

template <> struct Chunk<VLP_FP32> {
  static constexpr int N = 4;
  // Whole-vector bit casts only: this compiler reads element 0 when
  // __builtin_bit_cast is applied directly to a vector subscript.
  static __device__ __forceinline__ void widen(u32x4_t r, float (&x)[N]) {
    const f32x4_t f = __builtin_bit_cast(f32x4_t, r);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = f[i];
  }
  static __device__ __forceinline__ u32x4_t narrow(const float (&x)[N]) {
    f32x4_t f;
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = x[i];
    return __builtin_bit_cast(u32x4_t, f);
  }
};

template <> struct Chunk<VLP_BF16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void widen(u32x4_t r, float (&x)[N]) {
    const f32x4_t lo = __builtin_bit_cast(f32x4_t, r << 16);           // even elements
    const f32x4_t hi = __builtin_bit_cast(f32x4_t, r & 0xffff0000u);   // odd elements
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = lo[i];
      x[2 * i + 1] = hi[i];
    }
  }
  static __device__ __forceinline__ u32x4_t narrow(const float (&x)[N]) {
    u32x4_t r;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf16x2_t p;
      p[0] = static_cast<__bf16>(x[2 * i]);
      p[1] = static_cast<__bf16>(x[2 * i + 1]);
      r[i] = __builtin_bit_cast(uint32_t, p);
    }
    return r;
  }
};

template <> struct Chunk<VLP_FP16> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void widen(u32x4_t r, float (&x)[N]) {
    const f16x8_t h = __builtin_bit_cast(f16x8_t, r);
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = static_cast<float>(h[i]);
  }
  static __device__ __forceinline__ u32x4_t narrow(const float (&x)[N]) {
    f16x8_t h;
#pragma unroll
    for (int i = 0; i < 8; ++i) h[i] = static_cast<_Float16>(x[i]);
    return __builtin_bit_cast(u32x4_t, h);
  }
};

// Sum over groups of N consecutive lanes (N a power of two <= 64), the result
// in every lane of the group: DPP lane permutations within rows of 16 lanes
// (VALU operations, no round trip through the LDS crossbar) -- quad
// permutations for the lane xor 1 and xor 2 partners, then the half-row and
// row mirrors, which pair each lane with the other quad / half-row -- and a
// cross-lane shuffle beyond 16 lanes.  The additions pair the same lanes as
// an xor butterfly, so the sums are the butterfly's to the bit.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  if constexpr (N >= 4)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  if constexpr (N >= 8)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  if constexpr (N >= 16)
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
#pragma unroll
  for (int off = 16; off < N; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// Merge two online-softmax states (m in log2 units).
template <int N>
__device__ __forceinline__ void merge_state(float& m, float& l, float (&acc)[N], float mo, float lo,
                                            const float (&acco)[N]) {
  const float mn = fmaxf(m, mo);
  if (mn == kNegInf) return;  // both empty
  const float sa = __builtin_amdgcn_exp2f(m - mn);
  const float sb = __builtin_amdgcn_exp2f(mo - mn);
  l = l * sa + lo * sb;
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = acc[e] * sa + acco[e] * sb;
  m = mn;
}

// Online-softmax state of one wave over keys [kb, ke) of sequence `seq`,
// head `head` (kb, ke already cut to the visible keys).  On return every
// lane (grp, c) holds the state merged over the wave's KPS key slots for
// chunk c of the head's row.
template <int DT, int D>
__device__ __forceinline__ void first_token_keys(const AttnArgs& a, int seq, int head, int k_start, int kb, int ke,
                                                 float& m, float& l, float (&acc)[Chunk<DT>::N]) {
  using C = Chunk<DT>;
  constexpr int EPC = C::N;        // elements per 16-byte chunk
  constexpr int LPK = D / EPC;     // lanes per key row
  constexpr int KPS = 64 / LPK;    // keys per step
  constexpr int U = KPS >= 16 ? 4 : (KPS <= 4 ? 16 : 64 / KPS);  // steps per round (see the header)
  static_assert(LPK >= 1 && LPK <= 64 && (LPK & (LPK - 1)) == 0, "lanes per key");

  const int lane = task_tid() & 63;
  const int grp = lane / LPK;   // key slot within a step
  const int c = lane % LPK;     // chunk of the row

  float qf[EPC];
  {
    const char* qp = static_cast<const char*>(a.q) +
                     (static_cast<size_t>(seq) * a.q_stride + static_cast<size_t>(head) * D + c * EPC) * (16 / EPC);
    C::widen(*reinterpret_cast<const u32x4_t*>(qp), qf);
#pragma unroll
    for (int e = 0; e < EPC; ++e) qf[e] = flip_sign(qf[e], a.negate_q);
  }
  const size_t kv_off =
      (static_cast<size_t>(k_start) * a.kv_stride + static_cast<size_t>(head) * D + c * EPC) * (16 / EPC);
  const char* kp = static_cast<const char*>(a.k) + kv_off;
  const char* vp = static_cast<const char*>(a.v) + kv_off;
  const size_t row_bytes = static_cast<size_t>(a.kv_stride) * (16 / EPC);

  m = kNegInf;
  l = 0.0f;
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;

  for (int j0 = kb; j0 < ke; j0 += U * KPS) {
    u32x4_t kr[U], vr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * KPS + grp;
      kr[u] = u32x4_t{0, 0, 0, 0};
      vr[u] = kr[u];
      if (j < ke) {
        kr[u] = *reinterpret_cast<const u32x4_t*>(kp + j * row_bytes);
        vr[u] = *reinterpret_cast<const u32x4_t*>(vp + j * row_bytes);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int j = j0 + u * KPS + grp;
      float kf[EPC];
      C::widen(kr[u], kf);
      float dot = 0.0f;
#pragma unroll
      for (int e = 0; e < EPC; ++e) dot = __builtin_fmaf(qf[e], kf[e], dot);
      dot = group_sum<LPK>(dot);
      if (j < ke) {
        const float sc = dot * a.scale_log2;
        const float mn = fmaxf(m, sc);
        const float alpha = __builtin_amdgcn_exp2f(m - mn);
        const float p = __builtin_amdgcn_exp2f(sc - mn);
        float vf[EPC];
        C::widen(vr[u], vf);
        l = l * alpha + p;
#pragma unroll
        for (int e = 0; e < EPC; ++e) acc[e] = __builtin_fmaf(p, vf[e], acc[e] * alpha);
        m = mn;
      }
    }
  }

  // Merge the KPS key slots (lanes that differ in the grp bits).
#pragma unroll
  for (int off = LPK; off < 64; off <<= 1) {
    const float mo = __shfl_xor(m, off);
    const float lo = __shfl_xor(l, off);
    float acco[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acco[e] = __shfl_xor(acc[e], off);
    merge_state<EPC>(m, l, acc, mo, lo, acco);
  }
}

// Normalise a merged state and store the output chunk (lanes of key slot 0)
// and the log-sum-exp (lane 0).
template <int DT, int D>
__device__ __forceinline__ void first_token_store(const AttnArgs& a, int seq, int head, float m, float l,
                                                  const float (&acc)[Chunk<DT>::N]) {
  using C = Chunk<DT>;
  constexpr int EPC = C::N;
  constexpr int LPK = D / EPC;
  const int lane = task_tid() & 63;
  if (lane >= LPK) return;
  const int c = lane;
  const float inv = l > 0.0f ? 1.0f / l : 0.0f;
  float o[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) o[e] = acc[e] * inv;
  char* op = static_cast<char*>(a.out) +
             (static_cast<size_t>(seq) * a.o_stride + static_cast<size_t>(head) * D + c * EPC) * (16 / EPC);
  *reinterpret_cast<u32x4_t*>(op) = C::narrow(o);
  if (c == 0 && a.lse)
    a.lse[static_cast<size_t>(head) * a.rows_q + seq] = l > 0.0f ? (m + __log2f(l)) * kLn2 : kNegInf;
}

// Sequence and visible key count of tile slot `slot` (false: no such slot).
template <bool CAUSAL>
__device__ __forceinline__ bool first_token_decode(const AttnArgs& a, int slot, int& seq, int& k_start,
                                                   int& lk_vis) {
  const int f = a.tile_order ? a.tile_order[slot] : slot;
  if (f < 0 || f >= a.grid_cap) return false;
  seq = a.grid_mapping[f];
  if (seq < 0 || seq >= a.num_seqs) return false;
  k_start = a.cu_k[seq];
  const int lk = a.cu_k[seq + 1] - k_start;
  lk_vis = CAUSAL ? min(lk, 1) : lk;
  return true;
}

// One task of the head-parallel form: the wavefront's head of the sequence
// in tile slot `slot`, all of its keys.
template <int DT, int D, bool CAUSAL>
__device__ __forceinline__ void first_token_task(const AttnArgs& a, int slot, int head) {
  int seq, k_start, lk_vis;
  if (!first_token_decode<CAUSAL>(a, slot, seq, k_start, lk_vis)) return;
  float m, l, acc[Chunk<DT>::N];
  first_token_keys<DT, D>(a, seq, head, k_start, 0, lk_vis, m, l, acc);
  first_token_store<DT, D>(a, seq, head, m, l, acc);
}

// One task of the key-split form (long sequences): the kSplitWaves waves of
// the workgroup take consecutive equal shares of one head's keys (multiples
// of 64 keys), park their states in LDS, and wave 0 merges them in wave
// order.  A wave's keys are a chain of load latencies, so splitting a long
// sequence's keys shortens its chain (eight waves measured 18 % faster than
// four on the Zipf batch in first-token mode).
template <int DT, int D, bool CAUSAL>
__device__ __forceinline__ void first_token_split_task(const AttnArgs& a, int slot, int head,
                                                       float (*states)[64][Chunk<DT>::N + 2]) {
  constexpr int EPC = Chunk<DT>::N;
  int seq, k_start, lk_vis;
  if (!first_token_decode<CAUSAL>(a, slot, seq, k_start, lk_vis)) return;
  const int wave = __builtin_amdgcn_readfirstlane(task_tid() >> 6);
  const int lane = task_tid() & 63;
  const int share = ((lk_vis + kSplitWaves - 1) / kSplitWaves + 63) / 64 * 64;
  const int kb = min(lk_vis, wave * share), ke = min(lk_vis, kb + share);
  float m, l, acc[EPC];
  first_token_keys<DT, D>(a, seq, head, k_start, kb, ke, m, l, acc);
  states[wave][lane][0] = m;
  states[wave][lane][1] = l;
#pragma unroll
  for (int e = 0; e < EPC; ++e) states[wave][lane][2 + e] = acc[e];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) {
      float acco[EPC];
#pragma unroll
      for (int e = 0; e < EPC; ++e) acco[e] = states[w][lane][2 + e];
      merge_state<EPC>(m, l, acc, states[w][lane][0], states[w][lane][1], acco);
    }
    first_token_store<DT, D>(a, seq, head, m, l, acc);
  }
}

// One task of the chunked form (long sequences, with a workspace): the grid
// is built over the keys with kFirstTokenChunkKeys keys per tile, and the
// workgroup's kSplitWaves waves take consecutive shares of its chunk of one
// head's keys, merged in LDS by wave 0 as in the key-split form.  A sequence
// of one chunk is stored at once.  Otherwise wave 0 publishes the chunk's
// state in the workspace (ft_partials), and the workgroup that brings the
// (sequence, head)'s arrival counter to the chunk count merges every chunk's
// state in chunk order -- so the result does not depend on which one
// finishes last -- stores the output and clears the counter.  The
// device-scope fences order the state stores before the counter update and
// the counter read before the state loads (the XCDs' L2 caches are not
// coherent with one another within a launch).
template <int DT, int D>
__device__ __forceinline__ void first_token_chunk_task(const AttnArgs& a, int slot, int head,
                                                       float (*states)[64][Chunk<DT>::N + 2]) {
  constexpr int EPC = Chunk<DT>::N;
  constexpr int LPK = D / EPC;
  constexpr int STRIDE = D + 4;  // floats per published state: m, l, two unused, acc[D]
  const int f = a.tile_order ? a.tile_order[slot] : slot;
  if (f < 0 || f >= a.grid_cap) return;
  const int seq = a.grid_mapping[f];
  if (seq < 0 || seq >= a.num_seqs) return;
  const int first = a.block_offsets[seq];
  const int nchunks = a.block_offsets[seq + 1] - first;
  const int k_start = a.cu_k[seq];
  const int lk = a.cu_k[seq + 1] - k_start;
  const int cb = (f - first) * static_cast<int>(kFirstTokenChunkKeys);
  const int ce = min(lk, cb + static_cast<int>(kFirstTokenChunkKeys));
  const int wave = __builtin_amdgcn_readfirstlane(task_tid() >> 6);
  const int lane = task_tid() & 63;
  const int share = ((ce - cb + kSplitWaves - 1) / kSplitWaves + 63) / 64 * 64;
  const int kb = min(ce, cb + wave * share), ke = min(ce, kb + share);
  float m, l, acc[EPC];
  first_token_keys<DT, D>(a, seq, head, k_start, kb, ke, m, l, acc);
  states[wave][lane][0] = m;
  states[wave][lane][1] = l;
#pragma unroll
  for (int e = 0; e < EPC; ++e) states[wave][lane][2 + e] = acc[e];
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < kSplitWaves; ++w) {
    float acco[EPC];
#pragma unroll
    for (int e = 0; e < EPC; ++e) acco[e] = states[w][lane][2 + e];
    merge_state<EPC>(m, l, acc, states[w][lane][0], states[w][lane][1], acco);
  }
  if (nchunks == 1) {
    first_token_store<DT, D>(a, seq, head, m, l, acc);
    return;
  }
  const int c = lane % LPK;
  float* mine = a.ft_partials + (static_cast<size_t>(f) * a.heads + head) * STRIDE;
  if (lane < LPK) {
    f32x4_t* dst = reinterpret_cast<f32x4_t*>(mine + 4 + c * EPC);
#pragma unroll
    for (int v = 0; v < EPC / 4; ++v) dst[v] = f32x4_t{acc[4 * v], acc[4 * v + 1], acc[4 * v + 2], acc[4 * v + 3]};
    if (lane == 0) {
      mine[0] = m;
      mine[1] = l;
    }
  }
  __threadfence();
  int32_t* arrivals = a.ft_arrivals + static_cast<size_t>(seq) * a.heads + head;
  int before = 0;
  if (lane == 0) before = atomicAdd(arrivals, 1);
  before = __shfl(before, 0);
  if (before != nchunks - 1) return;
  __threadfence();
  m = kNegInf;
  l = 0.0f;
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
  for (int j = 0; j < nchunks; ++j) {
    const float* st = a.ft_partials + (static_cast<size_t>(first + j) * a.heads + head) * STRIDE;
    const f32x4_t* src = reinterpret_cast<const f32x4_t*>(st + 4 + c * EPC);
    float acco[EPC];
#pragma unroll
    for (int v = 0; v < EPC / 4; ++v) {
      const f32x4_t x = src[v];
#pragma unroll
      for (int e = 0; e < 4; ++e) acco[4 * v + e] = x[e];
    }
    merge_state<EPC>(m, l, acc, st[0], st[1], acco);
  }
  first_token_store<DT, D>(a, seq, head, m, l, acc);
  if (lane == 0) *arrivals = 0;
}

template <int DT, int D, bool PERSISTENT>
__global__ __launch_bounds__(64 * kSplitWaves) void attn_first_token_chunk_kernel(const AttnArgs a) {
  __shared__ float states[kSplitWaves][64][Chunk<DT>::N + 2];
  int g = a.num_blocks >= 0 ? a.num_blocks : a.block_offsets[a.num_seqs];
  g = min(g, a.grid_cap);
  const int tasks = g > 0 ? g * a.heads : 0;
  auto run = [&](int task) __attribute__((always_inline)) {
    const int slot = task / a.heads;
    first_token_chunk_task<DT, D>(a, slot, task - slot * a.heads, states);
  };
  if constexpr (PERSISTENT) {
    __shared__ int mailbox;
    run_claimed_tasks(tasks, a.task_counter, &mailbox, run);
  } else {
    const int task = blockIdx.x;
    if (task < tasks) run(task);
  }
}

template <int DT, int D>
hipError_t launch_chunked(const AttnArgs& a, int64_t slots, int32_t workers, hipStream_t s) {
  constexpr int threads = 64 * kSplitWaves;
  const auto kernel = workers == kStaticGrid ? attn_first_token_chunk_kernel<DT, D, false>
                                             : attn_first_token_chunk_kernel<DT, D, true>;
  int64_t width = 0;
  const hipError_t e = launch_width(kernel, threads, slots * a.heads, workers, &width);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(width)), dim3(threads), 0, s, a);
  return hipGetLastError();
}

// Head-parallel form (SPLIT false): task t = slot * head_groups + group,
// wave w of the workgroup takes head 4 * group + w (256 threads).  Key-split
// form: task t = slot * heads + head, all kSplitWaves waves on that head.  One task per
// workgroup on the static grid; tasks from the work queues on the
// persistent grid.
template <int DT, int D, bool CAUSAL, bool PERSISTENT, bool SPLIT>
__global__ __launch_bounds__(SPLIT ? 64 * kSplitWaves : 256) void attn_first_token_kernel(const AttnArgs a,
                                                                                        int head_groups) {
  const int wave = threadIdx.x >> 6;
  int g = a.num_blocks >= 0 ? a.num_blocks : a.block_offsets[a.num_seqs];
  g = min(g, a.grid_cap);
  const int tasks = g > 0 ? g * head_groups : 0;
  auto run = [&](int task) __attribute__((always_inline)) {
    const int slot = task / head_groups;
    if constexpr (SPLIT) {
      __shared__ float states[kSplitWaves][64][Chunk<DT>::N + 2];
      first_token_split_task<DT, D, CAUSAL>(a, slot, task - slot * head_groups, states);
    } else {
      const int head = (task - slot * head_groups) * 4 + wave;
      if (head < a.heads) first_token_task<DT, D, CAUSAL>(a, slot, head);
    }
  };
  if constexpr (PERSISTENT) {
    __shared__ int mailbox;
    run_claimed_tasks(tasks, a.task_counter, &mailbox, run);
  } else {
    const int task = blockIdx.x;
    if (task < tasks) run(task);
  }
}

template <int DT, int D, bool CAUSAL, bool SPLIT>
hipError_t launch_dt_d(const AttnArgs& a, int64_t slots, int32_t workers, hipStream_t s) {
  const int head_groups = SPLIT ? a.heads : (a.heads + 3) / 4;
  constexpr int threads = SPLIT ? 64 * kSplitWaves : 256;
  const auto kernel = workers == kStaticGrid ? attn_first_token_kernel<DT, D, CAUSAL, false, SPLIT>
                                             : attn_first_token_kernel<DT, D, CAUSAL, true, SPLIT>;
  int64_t width = 0;
  const hipError_t e = launch_width(kernel, threads, slots * head_groups, workers, &width);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(width)), dim3(threads), 0, s, a, head_groups);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_dt_dd(const AttnArgs& a, bool causal, FirstTokenForm form, int64_t slots, int32_t workers,
                        hipStream_t s) {
  if (form == FirstTokenForm::kChunked) return launch_chunked<DT, D>(a, slots, workers, s);
  if (form == FirstTokenForm::kKeySplit)
    return causal ? launch_dt_d<DT, D, true, true>(a, slots, workers, s)
                  : launch_dt_d<DT, D, false, true>(a, slots, workers, s);
  return causal ? launch_dt_d<DT, D, true, false>(a, slots, workers, s)
                : launch_dt_d<DT, D, false, false>(a, slots, workers, s);
}

template <int DT>
hipError_t launch_dt(const AttnArgs& a, int head_dim, bool causal, FirstTokenForm form, int64_t slots,
                     int32_t workers, hipStream_t s) {
  switch (head_dim) {
    case 16: return launch_dt_dd<DT, 16>(a, causal, form, slots, workers, s);
    case 32: return launch_dt_dd<DT, 32>(a, causal, form, slots, workers, s);
    case 64: return launch_dt_dd<DT, 64>(a, causal, form, slots, workers, s);
    case 128: return launch_dt_dd<DT, 128>(a, causal, form, slots, workers, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_attn_first_token(int dtype, const AttnArgs& a, int head_dim, bool causal, FirstTokenForm form,
                                   int64_t slots, int32_t workers, hipStream_t s) {
  if (slots <= 0) return hipSuccess;
  switch (dtype) {
    case VLP_FP32: return launch_dt<VLP_FP32>(a, head_dim, causal, form, slots, workers, s);
    case VLP_FP16: return launch_dt<VLP_FP16>(a, head_dim, causal, form, slots, workers, s);
    case VLP_BF16: return launch_dt<VLP_BF16>(a, head_dim, causal, form, slots, workers, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace vlp
