// C ABI of libvlp.so: host-side validation, workspace layout and dispatch.
//
// Every argument the host can see is checked before any HIP call; device
// buffer contents (cu_seqlens) are never read on the host (unless VLP_CHECK=1
// asks for a synchronous debug check), so the forward path enqueues work
// without synchronising ("gigl.nn.packed_attention":
// apart from the token count in pack_sequences, the packed path needs no
// host syncs; "So you wanna CUDA Graph", "Scheduling without max_seqlen":
// the launch is sized by G_cap, not by reading the lengths).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tile_config.h"
#include "vlp_internal.h"

namespace {

thread_local char g_hip_error[256] = "no HIP error recorded";

vlp_status hip_status(hipError_t e) {
  if (e == hipSuccess) return VLP_OK;
  snprintf(g_hip_error, sizeof(g_hip_error), "HIP error %d: %s", static_cast<int>(e), hipGetErrorString(e));
  return VLP_ERR_HIP;
}

constexpr int32_t kMfmaRateMaxBlocks = 1 << 16;
constexpr int32_t kMfmaRateMaxIters = 1 << 20;

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// VLP_CHECK=1 (any value but "0"): check device cu_seqlens contents before
// anything reads them (synchronous; a debugging aid).
bool debug_checks() {
  const char* v = getenv("VLP_CHECK");
  return v && v[0] && strcmp(v, "0") != 0;
}

vlp_status check_cu(const int32_t* cu, int32_t num_seqs, int64_t max_total, bool nonempty, hipStream_t s) {
  if (!cu || !debug_checks()) return VLP_OK;
  int32_t flags = 0;
  const vlp_status st = hip_status(vlp::check_cu_seqlens(cu, num_seqs, max_total, nonempty, s, &flags));
  if (st != VLP_OK) return st;
  return flags ? VLP_ERR_INVALID : VLP_OK;
}
inline size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Workspace layout of the device-built grid: [block_offsets | grid_mapping |
// tile_order | work-queue counters of a persistent launch], each 256-byte
// aligned.
struct GridWorkspace {
  size_t off_bo, off_gm, off_to, off_ctr, bytes;
};

GridWorkspace grid_workspace(int32_t num_seqs, int64_t cap) {
  GridWorkspace w;
  w.off_bo = 0;
  w.off_gm = round_up(sizeof(int32_t) * (static_cast<size_t>(num_seqs) + 1), 256);
  w.off_to = w.off_gm + round_up(sizeof(int32_t) * static_cast<size_t>(cap), 256);
  w.off_ctr = w.off_to + round_up(sizeof(int32_t) * static_cast<size_t>(cap), 256);
  w.bytes = w.off_ctr + sizeof(int32_t) * vlp::kTaskQueues * vlp::kCounterStride;
  return w;
}

struct Checked {
  int32_t block_m;
  int64_t grid_rows;  // rows the grid is sized for
  int32_t q_stride, kv_stride, o_stride;  // resolved token strides (elements)
};

inline int32_t element_bytes(int32_t dtype) { return dtype == VLP_FP32 ? 4 : 2; }

// Token stride (elements between consecutive tokens) of a [rows, heads,
// head_dim] operand whose heads are head_dim apart: 0 means contiguous.
// Rows must start 16-byte aligned (the kernels move 16-byte chunks), and a
// 64-row block must stay addressable with 32-bit byte offsets.
vlp_status resolve_stride(int64_t stride, int32_t heads, int32_t head_dim, int32_t elt, int32_t* out) {
  const int64_t row = static_cast<int64_t>(heads) * head_dim;
  if (stride == 0) stride = row;
  if (stride < row || (stride * elt) % 16 != 0) return VLP_ERR_INVALID;
  if (stride * elt > (int64_t{1} << 24)) return VLP_ERR_OVERFLOW;
  *out = static_cast<int32_t>(stride);
  return VLP_OK;
}

// Shared validation of the forward arguments; fills the tile size and the
// resolved strides.
vlp_status check_forward(int32_t dtype, const void* q, const void* k, const void* v,
                         const int32_t* cu_q, const int32_t* cu_k, int32_t num_seqs, int64_t rows_q,
                         int64_t total_k, int32_t heads, int32_t head_dim, int64_t q_stride, int64_t kv_stride,
                         int64_t out_stride, int32_t max_seqlen, float scale, int32_t causal, int32_t first_token,
                         const void* out, Checked* c) {
  if (!q || !k || !v || !out || !cu_k) return VLP_ERR_NULL;
  if (!first_token && !cu_q) return VLP_ERR_NULL;
  if (dtype != VLP_FP32 && dtype != VLP_FP16 && dtype != VLP_BF16) return VLP_ERR_UNSUPPORTED;
  if (!vlp::head_dim_built(head_dim)) return VLP_ERR_UNSUPPORTED;
  if (num_seqs < 1 || heads < 1 || rows_q < 0 || total_k < 0 || max_seqlen < 0) return VLP_ERR_INVALID;
  if ((causal != 0 && causal != 1) || (first_token != 0 && first_token != 1)) return VLP_ERR_INVALID;
  if (!isfinite(scale)) return VLP_ERR_INVALID;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out)) return VLP_ERR_INVALID;
  if (first_token && rows_q != num_seqs) return VLP_ERR_INVALID;
  if (rows_q > INT32_MAX || total_k > INT32_MAX) return VLP_ERR_OVERFLOW;
  if (rows_q * static_cast<int64_t>(heads) > INT32_MAX) return VLP_ERR_OVERFLOW;
  c->block_m = vlp_kernel_block_m(dtype, head_dim, causal, first_token, num_seqs, rows_q, max_seqlen);
  if (c->block_m < 1) return VLP_ERR_UNSUPPORTED;
  c->grid_rows = first_token ? num_seqs : rows_q;
  const int32_t elt = element_bytes(dtype);
  vlp_status st = resolve_stride(q_stride, heads, head_dim, elt, &c->q_stride);
  if (st == VLP_OK) st = resolve_stride(kv_stride, heads, head_dim, elt, &c->kv_stride);
  if (st == VLP_OK) st = resolve_stride(out_stride, heads, head_dim, elt, &c->o_stride);
  return st;
}

// Factor taking raw scores to exp2 units.  Masked scores are -inf and must
// map to -inf, which -inf * 0 would not: a zero scale is replaced by the
// smallest normal float, which leaves every finite score at (nearly) 0, so
// exp2 returns exactly 1 and the weights are exactly uniform, as for scale 0.
// A negative scale runs as |scale| with the register-resident operand of the
// score products negated (negate_q / negate), which keeps every kernel's
// running maximum order-preserving: scale * s = |scale| * (-s).
float exp2_factor(float scale) {
  const float mag = fabsf(scale);
  return mag > 0.0f ? mag * 1.4426950408889634f : 1.17549435e-38f;
}

vlp::AttnArgs make_args(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
                        int32_t num_seqs, int64_t rows_q, int32_t heads, float scale, void* out, float* lse,
                        const Checked& c) {
  vlp::AttnArgs a{};
  a.q_stride = c.q_stride;
  a.kv_stride = c.kv_stride;
  a.o_stride = c.o_stride;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.lse = lse;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.num_seqs = num_seqs;
  a.heads = heads;
  a.rows_q = static_cast<int32_t>(rows_q);
  a.num_blocks = -1;
  a.scale_log2 = exp2_factor(scale);
  a.negate_q = scale < 0.0f ? 1 : 0;
  return a;
}

vlp_status enqueue(int32_t dtype, const vlp::AttnArgs& a, int32_t head_dim, int32_t causal, int32_t first_token,
                   int64_t slots, int32_t workers, vlp::FirstTokenForm form, hipStream_t s) {
  if (slots <= 0) return VLP_OK;
  if (first_token)
    return hip_status(vlp::launch_attn_first_token(dtype, a, head_dim, causal != 0, form, slots, workers, s));
  const int64_t blocks = slots * a.heads;
  if (blocks > INT32_MAX) return VLP_ERR_OVERFLOW;
  switch (dtype) {
    case VLP_BF16: return hip_status(vlp::launch_attn_bf16(a, head_dim, causal != 0, blocks, workers, s));
    case VLP_FP16: return hip_status(vlp::launch_attn_f16(a, head_dim, causal != 0, blocks, workers, s));
    default: return hip_status(vlp::launch_attn_f32(a, head_dim, causal != 0, blocks, workers, s));
  }
}

// Key count that decides the first-token form: the keys a query sees in the
// longest sequence -- one when causal (the query sits at position 0), else
// the max_seqlen hint, or the mean sequence length when there is none.
int64_t long_keys(int32_t causal, int32_t max_seqlen, int64_t total_k, int32_t num_seqs) {
  if (causal) return 1;
  return max_seqlen > 0 ? max_seqlen : total_k / num_seqs;
}

// Form of a first-token launch; the chunked form needs a workspace (its
// partial states), so the cached-grid entry point never takes it.
vlp::FirstTokenForm first_token_form(int32_t causal, int32_t max_seqlen, int64_t total_k, int32_t num_seqs,
                                     bool with_workspace) {
  const int64_t keys = long_keys(causal, max_seqlen, total_k, num_seqs);
  if (with_workspace && keys >= vlp::kFirstTokenChunkMin) return vlp::FirstTokenForm::kChunked;
  return keys >= vlp::kFirstTokenSplitKeys ? vlp::FirstTokenForm::kKeySplit : vlp::FirstTokenForm::kHeadParallel;
}

// Workspace of the device-grid forward: the grid (GridWorkspace) and, for
// the chunked first-token form, per-(sequence, head) arrival counters and
// the per-(chunk, head) partial states, each 256-byte aligned.
struct FwdWorkspace {
  GridWorkspace grid;
  int32_t block_m;           // rows (keys, chunked form) per tile of the grid
  int64_t cap;               // grid capacity
  vlp::FirstTokenForm form;
  size_t off_arrivals, off_partials, bytes;
};

vlp_status fwd_workspace(const Checked& c, int32_t num_seqs, int64_t total_k, int32_t heads, int32_t head_dim,
                         int32_t causal, int32_t first_token, int32_t max_seqlen, FwdWorkspace* w) {
  w->form = first_token ? first_token_form(causal, max_seqlen, total_k, num_seqs, true)
                        : vlp::FirstTokenForm::kHeadParallel;
  const bool chunked = first_token && w->form == vlp::FirstTokenForm::kChunked;
  w->block_m = chunked ? static_cast<int32_t>(vlp::kFirstTokenChunkKeys) : c.block_m;
  w->cap = vlp_grid_capacity(chunked ? total_k : c.grid_rows, num_seqs, w->block_m);
  if (w->cap > INT32_MAX || w->cap * heads > INT32_MAX) return VLP_ERR_OVERFLOW;
  w->grid = grid_workspace(num_seqs, w->cap);
  w->off_arrivals = w->off_partials = w->bytes = w->grid.bytes;
  if (chunked) {
    w->off_arrivals = round_up(w->grid.bytes, 256);
    w->off_partials = w->off_arrivals + round_up(sizeof(int32_t) * static_cast<size_t>(num_seqs) * heads, 256);
    w->bytes = w->off_partials + sizeof(float) * static_cast<size_t>(w->cap) * heads * (head_dim + 4);
  }
  return VLP_OK;
}

// The launch-width argument of the persistent entry points: 0 asks for the
// resident workgroup count, a positive value caps the width; negative values
// are out of contract.
vlp_status persistent_workers(int32_t num_workers, int32_t* workers) {
  if (num_workers < 0) return VLP_ERR_INVALID;
  *workers = num_workers == 0 ? vlp::kResident : num_workers;
  return VLP_OK;
}

// Workspace of the backward: [lse2 | delta | query grid | key grid], each
// 256-byte aligned; lse2 and delta are fp32 [heads, rows_q].
struct BwdWorkspace {
  size_t off_lse2, off_delta, off_qgrid, off_kgrid, bytes;
  int64_t cap_q, cap_k;
  GridWorkspace qg, kg;
};

BwdWorkspace bwd_workspace(int32_t num_seqs, int64_t rows_q, int64_t total_k, int32_t heads, int32_t block) {
  BwdWorkspace w;
  const size_t stats = round_up(sizeof(float) * static_cast<size_t>(heads) * static_cast<size_t>(rows_q), 256);
  w.cap_q = vlp_grid_capacity(rows_q, num_seqs, block);
  w.cap_k = vlp_grid_capacity(total_k, num_seqs, VLP_BWD_BLOCK_K);
  w.qg = grid_workspace(num_seqs, w.cap_q);
  w.kg = grid_workspace(num_seqs, w.cap_k);
  w.off_lse2 = 0;
  w.off_delta = stats;
  w.off_qgrid = 2 * stats;
  w.off_kgrid = w.off_qgrid + w.qg.bytes;
  w.bytes = w.off_kgrid + w.kg.bytes;
  return w;
}

vlp_status launch_bwd(int32_t dtype, bool dkdv, const vlp::BwdArgs& a, int32_t head_dim, bool causal,
                      int64_t blocks, int32_t workers, hipStream_t s) {
  if (blocks <= 0) return VLP_OK;
  if (blocks > INT32_MAX) return VLP_ERR_OVERFLOW;
  switch (dtype) {
    case VLP_BF16:
      return hip_status(dkdv ? vlp::launch_attn_bwd_dkdv_bf16(a, head_dim, causal, blocks, workers, s)
                             : vlp::launch_attn_bwd_dq_bf16(a, head_dim, causal, blocks, workers, s));
    case VLP_FP16:
      return hip_status(dkdv ? vlp::launch_attn_bwd_dkdv_f16(a, head_dim, causal, blocks, workers, s)
                             : vlp::launch_attn_bwd_dq_f16(a, head_dim, causal, blocks, workers, s));
    default:
      return hip_status(dkdv ? vlp::launch_attn_bwd_dkdv_f32(a, head_dim, causal, blocks, workers, s)
                             : vlp::launch_attn_bwd_dq_f32(a, head_dim, causal, blocks, workers, s));
  }
}

}  // namespace

extern "C" int32_t vlp_kernel_block_m(int32_t dtype, int32_t head_dim, int32_t causal, int32_t first_token,
                                      int32_t num_seqs, int64_t rows_q, int32_t max_seqlen) {
  (void)causal;
  (void)num_seqs;
  (void)rows_q;
  (void)max_seqlen;
  if (dtype != VLP_FP32 && dtype != VLP_FP16 && dtype != VLP_BF16) return -1;
  if (!vlp::head_dim_built(head_dim)) return -1;
  if (first_token) return VLP_FIRST_TOKEN_BLOCK_M;
  return vlp::fwd_block_m(dtype, head_dim);
}

extern "C" int32_t vlp_bwd_block_m(int32_t dtype, int32_t head_dim, int32_t causal) {
  (void)causal;
  if (dtype != VLP_FP32 && dtype != VLP_FP16 && dtype != VLP_BF16) return -1;
  if (!vlp::head_dim_built(head_dim)) return -1;
  return 32 * vlp::tile_waves(dtype, head_dim);
}

extern "C" vlp_status vlp_varlen_attn_workspace_size(int32_t num_seqs, int64_t rows_q, int32_t block_m,
                                                     size_t* bytes) {
  if (!bytes) return VLP_ERR_NULL;
  if (num_seqs < 1 || rows_q < 0 || block_m < 1) return VLP_ERR_INVALID;
  const int64_t cap = vlp_grid_capacity(rows_q, num_seqs, block_m);
  *bytes = grid_workspace(num_seqs, cap).bytes;
  return VLP_OK;
}

extern "C" vlp_status vlp_varlen_attn_fwd_workspace_size(int32_t dtype, int32_t num_seqs, int64_t rows_q,
                                                         int64_t total_k, int32_t heads, int32_t head_dim,
                                                         int32_t max_seqlen, int32_t causal,
                                                         int32_t query_is_first_token, size_t* bytes) {
  if (!bytes) return VLP_ERR_NULL;
  if (dtype != VLP_FP32 && dtype != VLP_FP16 && dtype != VLP_BF16) return VLP_ERR_UNSUPPORTED;
  if (!vlp::head_dim_built(head_dim)) return VLP_ERR_UNSUPPORTED;
  if (num_seqs < 1 || heads < 1 || rows_q < 0 || total_k < 0 || max_seqlen < 0) return VLP_ERR_INVALID;
  if ((causal != 0 && causal != 1) || (query_is_first_token != 0 && query_is_first_token != 1))
    return VLP_ERR_INVALID;
  if (rows_q > INT32_MAX || total_k > INT32_MAX) return VLP_ERR_OVERFLOW;
  Checked c{};
  c.block_m = vlp_kernel_block_m(dtype, head_dim, causal, query_is_first_token, num_seqs, rows_q, max_seqlen);
  c.grid_rows = query_is_first_token ? num_seqs : rows_q;
  FwdWorkspace fw{};
  const vlp_status st =
      fwd_workspace(c, num_seqs, total_k, heads, head_dim, causal, query_is_first_token, max_seqlen, &fw);
  if (st != VLP_OK) return st;
  *bytes = fw.bytes;
  return VLP_OK;
}

extern "C" vlp_status vlp_build_ragged_grid_device(const int32_t* cu_seqlens, int32_t num_seqs, int32_t block_m,
                                                   int32_t* block_offsets, int32_t* grid_mapping,
                                                   int32_t* tile_order, int64_t grid_cap, void* stream) {
  if (!cu_seqlens || !block_offsets || !grid_mapping || !tile_order) return VLP_ERR_NULL;
  if (num_seqs < 1 || block_m < 1 || grid_cap < 0 || grid_cap > INT32_MAX) return VLP_ERR_INVALID;
  return hip_status(vlp::launch_grid_build(cu_seqlens, num_seqs, block_m, block_offsets, grid_mapping, tile_order,
                                           grid_cap, nullptr, static_cast<hipStream_t>(stream)));
}

namespace {

vlp_status fwd_device_grid(int32_t dtype, const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t rows_q, int64_t total_k,
                           int32_t heads, int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride,
                           int64_t out_row_stride, int32_t max_seqlen, float scale, int32_t causal,
                           int32_t query_is_first_token, void* out, float* lse, void* workspace,
                           size_t workspace_bytes, int32_t workers, void* stream, bool debug_check = true) {
  Checked c{};
  vlp_status st = check_forward(dtype, q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, total_k, heads,
                                head_dim, q_row_stride, kv_row_stride, out_row_stride, max_seqlen, scale, causal,
                                query_is_first_token, out, &c);
  if (st != VLP_OK) return st;
  if (!workspace) return VLP_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return VLP_ERR_INVALID;
  FwdWorkspace fw{};
  st = fwd_workspace(c, num_seqs, total_k, heads, head_dim, causal, query_is_first_token, max_seqlen, &fw);
  if (st != VLP_OK) return st;
  if (workspace_bytes < fw.bytes) return VLP_ERR_CAPACITY;
  const int64_t cap = fw.cap;
  if (cap == 0) return VLP_OK;

  const GridWorkspace& w = fw.grid;
  char* base = static_cast<char*>(workspace);
  int32_t* bo = reinterpret_cast<int32_t*>(base + w.off_bo);
  int32_t* gm = reinterpret_cast<int32_t*>(base + w.off_gm);
  int32_t* to = reinterpret_cast<int32_t*>(base + w.off_to);
  int32_t* ctr = workers == vlp::kStaticGrid ? nullptr : reinterpret_cast<int32_t*>(base + w.off_ctr);
  const bool chunked = query_is_first_token && fw.form == vlp::FirstTokenForm::kChunked;
  int32_t* arrivals = chunked ? reinterpret_cast<int32_t*>(base + fw.off_arrivals) : nullptr;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (debug_check) {
    if (!query_is_first_token) st = check_cu(cu_seqlens_q, num_seqs, rows_q, false, s);
    if (st == VLP_OK) st = check_cu(cu_seqlens_k, num_seqs, total_k, query_is_first_token != 0, s);
    if (st != VLP_OK) return st;
  }
  const int32_t* grid_cu = query_is_first_token ? cu_seqlens_k : cu_seqlens_q;
  // The grid build also clears the chunked form's arrival counters, so the
  // sequence stays free of memsets (capture-safe).
  st = hip_status(vlp::launch_grid_build(grid_cu, num_seqs, fw.block_m, bo, gm, to, cap, ctr, s, arrivals,
                                         chunked ? num_seqs * heads : 0));
  if (st != VLP_OK) return st;

  vlp::AttnArgs a = make_args(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, heads, scale, out, lse, c);
  a.task_counter = ctr;
  a.grid_mapping = gm;
  a.block_offsets = bo;
  a.tile_order = to;
  a.grid_cap = static_cast<int32_t>(cap);
  a.ft_arrivals = arrivals;
  a.ft_partials = chunked ? reinterpret_cast<float*>(base + fw.off_partials) : nullptr;
  return enqueue(dtype, a, head_dim, causal, query_is_first_token, cap, workers, fw.form, s);
}

}  // namespace

extern "C" vlp_status vlp_varlen_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                          int32_t num_seqs, int64_t rows_q, int64_t total_k, int32_t heads,
                                          int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride,
                                          int64_t out_row_stride, int32_t max_seqlen, float scale, int32_t causal,
                                          int32_t query_is_first_token, void* out, float* lse, void* workspace,
                                          size_t workspace_bytes, void* stream) {
  return fwd_device_grid(dtype, q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, total_k, heads, head_dim,
                         q_row_stride, kv_row_stride, out_row_stride, max_seqlen, scale, causal,
                         query_is_first_token, out, lse, workspace, workspace_bytes, vlp::kStaticGrid, stream);
}

extern "C" vlp_status vlp_varlen_attn_fwd_noalloc(int32_t dtype, const void* q, const void* k, const void* v,
                                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                                  int32_t num_seqs, int64_t rows_q, int64_t total_k, int32_t heads,
                                                  int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride,
                                                  int64_t out_row_stride, int32_t max_seqlen, float scale,
                                                  int32_t causal, int32_t query_is_first_token, void* out,
                                                  float* lse, void* stream) {
  // Sizes first, on the host: a request beyond the scratch is refused before
  // any HIP call.
  Checked c{};
  const vlp_status st = check_forward(dtype, q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, total_k, heads,
                                      head_dim, q_row_stride, kv_row_stride, out_row_stride, max_seqlen, scale,
                                      causal, query_is_first_token, out, &c);
  if (st != VLP_OK) return st;
  FwdWorkspace fw{};
  const vlp_status wst = fwd_workspace(c, num_seqs, total_k, heads, head_dim, causal, query_is_first_token,
                                       max_seqlen, &fw);
  if (wst != VLP_OK) return wst;
  if (fw.bytes > vlp::kNoallocScratchBytes) return VLP_ERR_CAPACITY;
  if (fw.cap == 0) return VLP_OK;
  void* scratch = nullptr;
  const vlp_status sst = hip_status(vlp::noalloc_scratch(&scratch));
  if (sst != VLP_OK) return sst;
  // The static grid rewrites every metadata entry it reads (the grid build
  // fills all grid_cap slots and clears the chunked first-token form's
  // counters), so nothing in the scratch needs clearing here.
  return fwd_device_grid(dtype, q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, total_k, heads, head_dim,
                         q_row_stride, kv_row_stride, out_row_stride, max_seqlen, scale, causal,
                         query_is_first_token, out, lse, scratch, vlp::kNoallocScratchBytes, vlp::kStaticGrid,
                         stream, /*debug_check=*/false);
}

extern "C" vlp_status vlp_varlen_attn_fwd_persistent(
    int32_t dtype, const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
    const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t rows_q, int64_t total_k, int32_t heads, int32_t head_dim,
    int64_t q_row_stride, int64_t kv_row_stride, int64_t out_row_stride, int32_t max_seqlen, float scale,
    int32_t causal, int32_t query_is_first_token, void* out, float* lse, void* workspace, size_t workspace_bytes,
    int32_t num_workers, void* stream) {
  int32_t workers = 0;
  const vlp_status st = persistent_workers(num_workers, &workers);
  if (st != VLP_OK) return st;
  return fwd_device_grid(dtype, q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, total_k, heads, head_dim,
                         q_row_stride, kv_row_stride, out_row_stride, max_seqlen, scale, causal,
                         query_is_first_token, out, lse, workspace, workspace_bytes, workers, stream);
}

extern "C" vlp_status vlp_varlen_attn_fwd_grid(int32_t dtype, const void* q, const void* k, const void* v,
                                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                               int32_t num_seqs, int64_t rows_q, int64_t total_k, int32_t heads,
                                               int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride,
                                               int64_t out_row_stride, int32_t max_seqlen, float scale,
                                               int32_t causal, int32_t query_is_first_token, void* out, float* lse,
                                               const int32_t* grid_mapping, const int32_t* block_offsets,
                                               const int32_t* tile_order, int64_t num_blocks, int32_t block_m,
                                               void* stream) {
  Checked c{};
  vlp_status st = check_forward(dtype, q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, total_k, heads,
                                head_dim, q_row_stride, kv_row_stride, out_row_stride, max_seqlen, scale, causal,
                                query_is_first_token, out, &c);
  if (st != VLP_OK) return st;
  if (!grid_mapping || !block_offsets) return VLP_ERR_NULL;
  if (num_blocks < 0 || block_m != c.block_m) return VLP_ERR_INVALID;
  if (num_blocks > INT32_MAX || num_blocks * heads > INT32_MAX) return VLP_ERR_OVERFLOW;
  vlp::AttnArgs a = make_args(q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, heads, scale, out, lse, c);
  a.grid_mapping = grid_mapping;
  a.block_offsets = block_offsets;
  a.tile_order = tile_order;
  a.num_blocks = static_cast<int32_t>(num_blocks);
  a.grid_cap = static_cast<int32_t>(num_blocks);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!query_is_first_token) st = check_cu(cu_seqlens_q, num_seqs, rows_q, false, s);
  if (st == VLP_OK) st = check_cu(cu_seqlens_k, num_seqs, total_k, query_is_first_token != 0, s);
  if (st != VLP_OK) return st;
  return enqueue(dtype, a, head_dim, causal, query_is_first_token, num_blocks, vlp::kStaticGrid,
                 first_token_form(causal, max_seqlen, total_k, num_seqs, false), s);
}

#ifndef VLP_SOURCE_HASH
#define VLP_SOURCE_HASH "unknown"
#endif

namespace vlp {
hipError_t launch_mfma_rate(int dtype, int blocks, int iters, float* sink, hipStream_t s);
double mfma_rate_flops(int dtype, int blocks, int iters);
}  // namespace vlp

extern "C" vlp_status vlp_mfma_rate(int32_t dtype, int32_t blocks, int32_t iters, float* sink, double* flops,
                                    void* stream) {
  if (dtype != VLP_FP32 && dtype != VLP_FP16 && dtype != VLP_BF16) return VLP_ERR_UNSUPPORTED;
  if (!sink || !flops) return VLP_ERR_NULL;
  if (blocks < 1 || blocks > kMfmaRateMaxBlocks || iters < 1 || iters > kMfmaRateMaxIters) return VLP_ERR_INVALID;
  *flops = vlp::mfma_rate_flops(dtype, blocks, iters);
  return hip_status(vlp::launch_mfma_rate(dtype, blocks, iters, sink, static_cast<hipStream_t>(stream)));
}

extern "C" const char* vlp_build_info(void) { return "csrc=" VLP_SOURCE_HASH " arch=gfx950"; }

extern "C" const char* vlp_status_string(vlp_status status) {
  switch (status) {
    case VLP_OK: return "VLP_OK";
    case VLP_ERR_NULL: return "VLP_ERR_NULL: a required pointer is NULL";
    case VLP_ERR_INVALID: return "VLP_ERR_INVALID: an argument is out of contract";
    case VLP_ERR_UNSUPPORTED: return "VLP_ERR_UNSUPPORTED: dtype, head_dim or mode not built";
    case VLP_ERR_CAPACITY: return "VLP_ERR_CAPACITY: an output or workspace buffer is too small";
    case VLP_ERR_OVERFLOW: return "VLP_ERR_OVERFLOW: a count does not fit in int32";
    case VLP_ERR_HIP: return g_hip_error;
    default: return "unknown vlp status";
  }
}

extern "C" vlp_status vlp_varlen_attn_bwd_workspace_size(int32_t num_seqs, int64_t rows_q, int64_t total_k,
                                                         int32_t heads, int32_t block_m, size_t* bytes) {
  if (!bytes) return VLP_ERR_NULL;
  if (num_seqs < 1 || rows_q < 0 || total_k < 0 || heads < 1 || block_m < 1) return VLP_ERR_INVALID;
  if (rows_q > INT32_MAX || total_k > INT32_MAX) return VLP_ERR_OVERFLOW;
  *bytes = bwd_workspace(num_seqs, rows_q, total_k, heads, block_m).bytes;
  return VLP_OK;
}

namespace {

// Shared validation of the backward arguments (the forward's plus the
// gradient buffers).
struct BwdStrides {
  int64_t q, kv, out, dout, dq, dkv;  // as passed (0 = contiguous)
};

vlp_status check_backward(int32_t dtype, const void* q, const void* k, const void* v, const void* out,
                          const void* dout, const float* lse, const int32_t* cu_q, const int32_t* cu_k,
                          int32_t num_seqs, int64_t rows_q, int64_t total_k, int32_t heads, int32_t head_dim,
                          const BwdStrides& sd, int32_t max_seqlen, float scale, int32_t causal, const void* dq,
                          const void* dk, const void* dv, Checked* c, int32_t* do_stride, int32_t* dq_stride,
                          int32_t* dkv_stride) {
  vlp_status st = check_forward(dtype, q, k, v, cu_q, cu_k, num_seqs, rows_q, total_k, heads, head_dim, sd.q, sd.kv,
                                sd.out, max_seqlen, scale, causal, 0, out, c);
  if (st != VLP_OK) return st;
  if (!dout || !lse || !dq || !dk || !dv) return VLP_ERR_NULL;
  if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
      (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return VLP_ERR_INVALID;
  if (rows_q * heads > INT32_MAX || total_k * heads > INT32_MAX) return VLP_ERR_OVERFLOW;
  c->block_m = vlp_bwd_block_m(dtype, head_dim, causal);  // the query grid of the dQ kernel
  if (c->block_m < 1) return VLP_ERR_UNSUPPORTED;
  const int32_t elt = element_bytes(dtype);
  st = resolve_stride(sd.dout, heads, head_dim, elt, do_stride);
  if (st == VLP_OK) st = resolve_stride(sd.dq, heads, head_dim, elt, dq_stride);
  if (st == VLP_OK) st = resolve_stride(sd.dkv, heads, head_dim, elt, dkv_stride);
  return st;
}

vlp::BwdArgs make_bwd_args(const void* q, const void* k, const void* v, const void* out, const void* dout,
                           const float* lse, const int32_t* cu_q, const int32_t* cu_k, int32_t num_seqs,
                           int64_t rows_q, int32_t heads, float scale, void* dq, void* dk, void* dv,
                           float* row_stats, const Checked& c, int32_t do_stride, int32_t dq_stride,
                           int32_t dkv_stride) {
  vlp::BwdArgs a{};
  a.q_stride = c.q_stride;
  a.kv_stride = c.kv_stride;
  a.o_stride = c.o_stride;
  a.do_stride = do_stride;
  a.dq_stride = dq_stride;
  a.dkv_stride = dkv_stride;
  a.q = q;
  a.k = k;
  a.v = v;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.lse2 = row_stats;
  a.delta = row_stats + static_cast<size_t>(heads) * static_cast<size_t>(rows_q);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.num_seqs = num_seqs;
  a.heads = heads;
  a.rows_q = static_cast<int32_t>(rows_q);
  a.scale = scale;
  a.scale_log2 = exp2_factor(scale);
  a.negate = scale < 0.0f ? 1 : 0;
  return a;
}

}  // namespace

namespace {

vlp_status bwd_device_grid(int32_t dtype, const void* q, const void* k, const void* v, const void* out,
                           const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                           const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t rows_q, int64_t total_k,
                           int32_t heads, int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride,
                           int64_t out_row_stride, int64_t dout_row_stride, int64_t dq_row_stride,
                           int64_t dkv_row_stride, int32_t max_seqlen, float scale, int32_t causal, void* dq,
                           void* dk, void* dv, void* workspace, size_t workspace_bytes, int32_t workers,
                           void* stream) {
  Checked c{};
  int32_t do_stride = 0, dq_stride = 0, dkv_stride = 0;
  const BwdStrides sd{q_row_stride, kv_row_stride, out_row_stride, dout_row_stride, dq_row_stride, dkv_row_stride};
  vlp_status st = check_backward(dtype, q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q,
                                 total_k, heads, head_dim, sd, max_seqlen, scale, causal, dq, dk, dv, &c, &do_stride,
                                 &dq_stride, &dkv_stride);
  if (st != VLP_OK) return st;
  if (!workspace) return VLP_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return VLP_ERR_INVALID;
  const BwdWorkspace w = bwd_workspace(num_seqs, rows_q, total_k, heads, c.block_m);
  if (w.cap_q * heads > INT32_MAX || w.cap_k * heads > INT32_MAX) return VLP_ERR_OVERFLOW;
  if (workspace_bytes < w.bytes) return VLP_ERR_CAPACITY;

  char* base = static_cast<char*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = check_cu(cu_seqlens_q, num_seqs, rows_q, false, s);
  if (st == VLP_OK) st = check_cu(cu_seqlens_k, num_seqs, total_k, false, s);
  if (st != VLP_OK) return st;
  vlp::BwdArgs a = make_bwd_args(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, heads,
                                 scale, dq, dk, dv, reinterpret_cast<float*>(base + w.off_lse2), c, do_stride,
                                 dq_stride, dkv_stride);
  a.delta = reinterpret_cast<float*>(base + w.off_delta);

  // dQ over the query grid first: it also writes lse2 and delta, which the
  // dK/dV launch (same stream) reads.
  if (w.cap_q > 0) {
    char* g = base + w.off_qgrid;
    int32_t* bo = reinterpret_cast<int32_t*>(g + w.qg.off_bo);
    int32_t* gm = reinterpret_cast<int32_t*>(g + w.qg.off_gm);
    int32_t* to = reinterpret_cast<int32_t*>(g + w.qg.off_to);
    int32_t* ctr = workers == vlp::kStaticGrid ? nullptr : reinterpret_cast<int32_t*>(g + w.qg.off_ctr);
    st = hip_status(vlp::launch_grid_build(cu_seqlens_q, num_seqs, c.block_m, bo, gm, to, w.cap_q, ctr, s));
    if (st != VLP_OK) return st;
    a.task_counter = ctr;
    a.grid_mapping = gm;
    a.block_offsets = bo;
    a.tile_order = to;
    a.grid_cap = static_cast<int32_t>(w.cap_q);
    st = launch_bwd(dtype, false, a, head_dim, causal != 0, w.cap_q * heads, workers, s);
    if (st != VLP_OK) return st;
  }
  if (w.cap_k > 0) {
    char* g = base + w.off_kgrid;
    int32_t* bo = reinterpret_cast<int32_t*>(g + w.kg.off_bo);
    int32_t* gm = reinterpret_cast<int32_t*>(g + w.kg.off_gm);
    int32_t* to = reinterpret_cast<int32_t*>(g + w.kg.off_to);
    int32_t* ctr = workers == vlp::kStaticGrid ? nullptr : reinterpret_cast<int32_t*>(g + w.kg.off_ctr);
    st = hip_status(vlp::launch_grid_build(cu_seqlens_k, num_seqs, VLP_BWD_BLOCK_K, bo, gm, to, w.cap_k, ctr, s));
    if (st != VLP_OK) return st;
    a.task_counter = ctr;
    a.grid_mapping = gm;
    a.block_offsets = bo;
    a.tile_order = to;
    a.grid_cap = static_cast<int32_t>(w.cap_k);
    st = launch_bwd(dtype, true, a, head_dim, causal != 0, w.cap_k * heads, workers, s);
  }
  return st;
}

}  // namespace

extern "C" vlp_status vlp_varlen_attn_bwd(int32_t dtype, const void* q, const void* k, const void* v,
                                          const void* out, const void* dout, const float* lse,
                                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                          int32_t num_seqs, int64_t rows_q, int64_t total_k, int32_t heads,
                                          int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride,
                                          int64_t out_row_stride, int64_t dout_row_stride, int64_t dq_row_stride,
                                          int64_t dkv_row_stride, int32_t max_seqlen, float scale, int32_t causal,
                                          void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                          void* stream) {
  return bwd_device_grid(dtype, q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, total_k,
                         heads, head_dim, q_row_stride, kv_row_stride, out_row_stride, dout_row_stride,
                         dq_row_stride, dkv_row_stride, max_seqlen, scale, causal, dq, dk, dv, workspace,
                         workspace_bytes, vlp::kStaticGrid, stream);
}

extern "C" vlp_status vlp_varlen_attn_bwd_persistent(
    int32_t dtype, const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t rows_q, int64_t total_k,
    int32_t heads, int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride, int64_t out_row_stride,
    int64_t dout_row_stride, int64_t dq_row_stride, int64_t dkv_row_stride, int32_t max_seqlen, float scale,
    int32_t causal, void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, int32_t num_workers,
    void* stream) {
  int32_t workers = 0;
  const vlp_status st = persistent_workers(num_workers, &workers);
  if (st != VLP_OK) return st;
  return bwd_device_grid(dtype, q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, total_k,
                         heads, head_dim, q_row_stride, kv_row_stride, out_row_stride, dout_row_stride,
                         dq_row_stride, dkv_row_stride, max_seqlen, scale, causal, dq, dk, dv, workspace,
                         workspace_bytes, workers, stream);
}

extern "C" vlp_status vlp_varlen_attn_bwd_grid(
    int32_t dtype, const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t rows_q, int64_t total_k,
    int32_t heads, int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride, int64_t out_row_stride,
    int64_t dout_row_stride, int64_t dq_row_stride, int64_t dkv_row_stride, int32_t max_seqlen, float scale,
    int32_t causal, void* dq, void* dk, void* dv,
    const int32_t* q_grid_mapping, const int32_t* q_block_offsets, const int32_t* q_tile_order,
    int64_t q_num_blocks, const int32_t* k_grid_mapping, const int32_t* k_block_offsets,
    const int32_t* k_tile_order, int64_t k_num_blocks, int32_t block_m, float* row_stats, int32_t phases,
    void* stream) {
  Checked c{};
  int32_t do_stride = 0, dq_stride = 0, dkv_stride = 0;
  const BwdStrides sd{q_row_stride, kv_row_stride, out_row_stride, dout_row_stride, dq_row_stride, dkv_row_stride};
  vlp_status st = check_backward(dtype, q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q,
                                 total_k, heads, head_dim, sd, max_seqlen, scale, causal, dq, dk, dv, &c, &do_stride,
                                 &dq_stride, &dkv_stride);
  if (st != VLP_OK) return st;
  if (phases < 1 || phases > 3) return VLP_ERR_INVALID;
  const bool run_dq = (phases & VLP_BWD_DQ) != 0, run_dkdv = (phases & VLP_BWD_DKDV) != 0;
  if (!row_stats) return VLP_ERR_NULL;
  if (run_dq && (!q_grid_mapping || !q_block_offsets)) return VLP_ERR_NULL;
  if (run_dkdv && (!k_grid_mapping || !k_block_offsets)) return VLP_ERR_NULL;
  if ((reinterpret_cast<uintptr_t>(row_stats) & 3u) != 0) return VLP_ERR_INVALID;
  if (block_m != c.block_m || (run_dq && q_num_blocks < 0) || (run_dkdv && k_num_blocks < 0)) return VLP_ERR_INVALID;
  if ((run_dq && q_num_blocks * heads > INT32_MAX) || (run_dkdv && k_num_blocks * heads > INT32_MAX))
    return VLP_ERR_OVERFLOW;
  hipStream_t s = static_cast<hipStream_t>(stream);
  st = check_cu(cu_seqlens_q, num_seqs, rows_q, false, s);
  if (st == VLP_OK) st = check_cu(cu_seqlens_k, num_seqs, total_k, false, s);
  if (st != VLP_OK) return st;
  vlp::BwdArgs a = make_bwd_args(q, k, v, out, dout, lse, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, heads,
                                 scale, dq, dk, dv, row_stats, c, do_stride, dq_stride, dkv_stride);
  if (run_dq) {
    a.grid_mapping = q_grid_mapping;
    a.block_offsets = q_block_offsets;
    a.tile_order = q_tile_order;
    a.grid_cap = static_cast<int32_t>(q_num_blocks);
    st = launch_bwd(dtype, false, a, head_dim, causal != 0, q_num_blocks * heads, vlp::kStaticGrid, s);
    if (st != VLP_OK) return st;
  }
  if (run_dkdv) {
    a.grid_mapping = k_grid_mapping;
    a.block_offsets = k_block_offsets;
    a.tile_order = k_tile_order;
    a.grid_cap = static_cast<int32_t>(k_num_blocks);
    st = launch_bwd(dtype, true, a, head_dim, causal != 0, k_num_blocks * heads, vlp::kStaticGrid, s);
  }
  return st;
}

extern "C" vlp_status vlp_ragged_matmul_workspace_size(int32_t num_seqs, int64_t rows, size_t* bytes) {
  if (!bytes) return VLP_ERR_NULL;
  if (num_seqs < 1 || rows < 0) return VLP_ERR_INVALID;
  *bytes = grid_workspace(num_seqs, vlp_grid_capacity(rows, num_seqs, VLP_MATMUL_BLOCK_M)).bytes;
  return VLP_OK;
}

namespace {

vlp_status matmul_device_grid(int32_t dtype, const void* x, const void* weight, const void* bias,
                              const int32_t* cu_seqlens, int32_t num_seqs, int64_t rows, int32_t in_features,
                              int32_t out_features, int64_t weight_seq_stride, int64_t bias_seq_stride, void* y,
                              void* workspace, size_t workspace_bytes, int32_t workers, void* stream) {
  if (!x || !weight || !cu_seqlens || !y || !workspace) return VLP_ERR_NULL;
  if (dtype != VLP_FP32 && dtype != VLP_FP16 && dtype != VLP_BF16) return VLP_ERR_UNSUPPORTED;
  if (dtype == VLP_FP32) return VLP_ERR_UNSUPPORTED;
  if (num_seqs < 1 || rows < 0) return VLP_ERR_INVALID;
  if (in_features < 64 || in_features > 65536 || in_features % 64 != 0) return VLP_ERR_INVALID;
  if (out_features < 4 || out_features > 65536 || out_features % 4 != 0) return VLP_ERR_INVALID;
  if (weight_seq_stride < 0 || weight_seq_stride % 8 != 0) return VLP_ERR_INVALID;
  if (bias && (bias_seq_stride < 0 || bias_seq_stride % 4 != 0)) return VLP_ERR_INVALID;
  if (!aligned16(x) || !aligned16(weight) || !aligned16(y) || (bias && !aligned16(bias))) return VLP_ERR_INVALID;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return VLP_ERR_INVALID;
  if (rows > INT32_MAX) return VLP_ERR_OVERFLOW;
  const int64_t cap = vlp_grid_capacity(rows, num_seqs, VLP_MATMUL_BLOCK_M);
  const int64_t col_tiles = (out_features + vlp::kMatmulBlockN - 1) / vlp::kMatmulBlockN;
  const int64_t blocks = (cap + 7) / 8 * 8 * col_tiles;
  if (cap > INT32_MAX || blocks > INT32_MAX) return VLP_ERR_OVERFLOW;
  const GridWorkspace w = grid_workspace(num_seqs, cap);
  if (workspace_bytes < w.bytes) return VLP_ERR_CAPACITY;
  if (cap == 0) return VLP_OK;

  char* base = static_cast<char*>(workspace);
  int32_t* bo = reinterpret_cast<int32_t*>(base + w.off_bo);
  int32_t* gm = reinterpret_cast<int32_t*>(base + w.off_gm);
  int32_t* to = reinterpret_cast<int32_t*>(base + w.off_to);
  int32_t* ctr = workers == vlp::kStaticGrid ? nullptr : reinterpret_cast<int32_t*>(base + w.off_ctr);
  hipStream_t s = static_cast<hipStream_t>(stream);
  vlp_status st = check_cu(cu_seqlens, num_seqs, rows, false, s);
  if (st != VLP_OK) return st;
  st = hip_status(vlp::launch_grid_build(cu_seqlens, num_seqs, VLP_MATMUL_BLOCK_M, bo, gm, to, cap, ctr, s));
  if (st != VLP_OK) return st;
  vlp::MatmulArgs a{};
  a.task_counter = ctr;
  a.x = x;
  a.w = weight;
  a.bias = bias;
  a.y = y;
  a.cu = cu_seqlens;
  a.grid_mapping = gm;
  a.block_offsets = bo;
  a.num_seqs = num_seqs;
  a.k = in_features;
  a.n = out_features;
  a.grid_cap = static_cast<int32_t>(cap);
  a.col_tiles = static_cast<int32_t>(col_tiles);
  a.w_seq_stride = weight_seq_stride;
  a.b_seq_stride = bias_seq_stride;
  return hip_status(vlp::launch_ragged_matmul(dtype, a, bias != nullptr, blocks, workers, s));
}

}  // namespace

extern "C" vlp_status vlp_ragged_matmul(int32_t dtype, const void* x, const void* weight, const void* bias,
                                        const int32_t* cu_seqlens, int32_t num_seqs, int64_t rows,
                                        int32_t in_features, int32_t out_features, int64_t weight_seq_stride,
                                        int64_t bias_seq_stride, void* y, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  return matmul_device_grid(dtype, x, weight, bias, cu_seqlens, num_seqs, rows, in_features, out_features,
                            weight_seq_stride, bias_seq_stride, y, workspace, workspace_bytes, vlp::kStaticGrid,
                            stream);
}

extern "C" vlp_status vlp_ragged_matmul_persistent(int32_t dtype, const void* x, const void* weight,
                                                   const void* bias, const int32_t* cu_seqlens, int32_t num_seqs,
                                                   int64_t rows, int32_t in_features, int32_t out_features,
                                                   int64_t weight_seq_stride, int64_t bias_seq_stride, void* y,
                                                   void* workspace, size_t workspace_bytes, int32_t num_workers,
                                                   void* stream) {
  int32_t workers = 0;
  const vlp_status st = persistent_workers(num_workers, &workers);
  if (st != VLP_OK) return st;
  return matmul_device_grid(dtype, x, weight, bias, cu_seqlens, num_seqs, rows, in_features, out_features,
                            weight_seq_stride, bias_seq_stride, y, workspace, workspace_bytes, workers, stream);
}

extern "C" vlp_status vlp_cu_seqlens_from_ids(const int32_t* ids, int64_t num_tokens, int32_t max_seqs,
                                              int32_t* cu_seqlens, int32_t* num_seqs, void* stream) {
  if (!cu_seqlens || !num_seqs || (num_tokens > 0 && !ids)) return VLP_ERR_NULL;
  if (num_tokens < 0 || max_seqs < 1) return VLP_ERR_INVALID;
  if (num_tokens > INT32_MAX) return VLP_ERR_OVERFLOW;
  return hip_status(vlp::launch_ids_to_cu(ids, static_cast<int32_t>(num_tokens), max_seqs, cu_seqlens, num_seqs,
                                          static_cast<hipStream_t>(stream)));
}
