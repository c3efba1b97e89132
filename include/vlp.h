/*
 * vlp.h -- packed variable-length attention (forward and gradients) for AMD
 * Instinct MI355X (gfx950): the C ABI of libvlp.so.
 *
 * The operation: a batch of B sequences is packed token-major into one buffer
 * [num_tokens, heads, head_dim]; sequence i occupies rows
 * [cu_seqlens[i], cu_seqlens[i+1]) and attends only to itself.  Sources:
 *   - "gigl.nn.packed_attention": the module description ("each sequence
 *     attends only to itself, with boundaries given by cu_seqlens"), "Data
 *     flow of a packed forward", "Constraints", "Example", and the
 *     packed_attention entry (query_is_first_token).
 *   - "PyCoRa: A PyTorch implementation of CoRa Ragged Tensors": "The Data
 *     Structure", "CoRa Metadata" (grid_mapping, block_offsets) and "Ragged
 *     Flash Attention" (tiled online softmax routed through grid_mapping).
 *   - "So you wanna CUDA Graph" (attention-gym): "What are ragged kernels?"
 *     (the cu_seqlens convention), "Terminology time" (capacity tails),
 *     "Scheduling without max_seqlen" (flat tile list, its decode and the
 *     launch capacity G_cap), "Correctness tangent" (inactive rows).
 *   - "DanLing NestedTensor", section 3.3 "Attention through packed blocks"
 *     (token-major q/k/v, separate query and key boundaries).
 *
 * Conventions shared by every entry point:
 *   - All functions are non-throwing and reentrant and keep no pointer after
 *     they return.  The caller owns every buffer.
 *   - "host" pointers are ordinary CPU memory; "device" pointers are HIP
 *     device memory on the current device.
 *   - Device entry points only enqueue work on `stream` (a hipStream_t passed
 *     as void*, NULL = the null stream); they never synchronise and never read
 *     device memory on the host, so the values in device buffers (cu_seqlens
 *     in particular) are NOT validated.  Out-of-contract values are undefined
 *     behaviour: boundaries beyond the rows of q, k or v (say, a
 *     cross-attention batch's key boundaries passed as its query boundaries)
 *     make the kernels read and write outside those buffers, which faults the
 *     GPU.  Every argument the host can see is validated before any HIP call,
 *     and a failed check returns a status without touching the GPU.
 *   - Debugging aid: with VLP_CHECK=1 in the environment, the attention,
 *     gradient and ragged-matmul entry points first check the cu_seqlens
 *     contents on the device (cu[0] == 0, non-decreasing, cu[num_seqs] no
 *     more than the rows of the buffer; in first-token mode every sequence
 *     non-empty), wait for that check, and return VLP_ERR_INVALID on a
 *     violation before any other kernel reads the values.  It allocates and
 *     synchronises, so it is not for captured graphs or timed runs.
 */
#ifndef VLP_H_
#define VLP_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t vlp_status;

enum {
  VLP_OK = 0,
  VLP_ERR_NULL = 1,        /* a required pointer is NULL                   */
  VLP_ERR_INVALID = 2,     /* an argument value is out of contract         */
  VLP_ERR_UNSUPPORTED = 3, /* dtype / head_dim / mode not built            */
  VLP_ERR_CAPACITY = 4,    /* an output or workspace buffer is too small   */
  VLP_ERR_OVERFLOW = 5,    /* a count does not fit in int32                */
  VLP_ERR_HIP = 6          /* a HIP runtime call failed (kernel launch)    */
};

/* Element types of q, k, v and out. */
enum { VLP_FP32 = 0, VLP_FP16 = 1, VLP_BF16 = 2 };

/*
 * vlp_pack_sequences -- lengths -> flat_index, cu_seqlens (all host memory).
 *
 * "gigl.nn.packed_attention", "Data flow of a packed forward" and "Example":
 * cu_seqlens[0] = 0, cu_seqlens[i+1] = cu_seqlens[i] + lengths[i]; the packed
 * buffer is padded_grid.flatten()[flat_index], where flat_index lists the
 * row-major positions i*max_seq_len + j (j < lengths[i]) of the real tokens of
 * the padded grid [num_seqs, max_seq_len], sequence after sequence.
 * Example: lengths {3,1,2}, max_seq_len 3 -> flat_index {0,1,2,3,6,7},
 * cu_seqlens {0,3,4,6}.
 *
 *   lengths      host int32 [num_seqs]; each in [1, max_seq_len]
 *                ("Every sequence must contain at least one token").
 *   num_seqs     >= 1.
 *   max_seq_len  >= 1, the padded grid's row length.
 *   flat_index   host int64 [flat_index_cap], or NULL to query the size only.
 *   cu_seqlens   host int32 [num_seqs + 1], always written on success and on
 *                VLP_ERR_CAPACITY.
 *   num_tokens   host int64*, receives sum(lengths) (the one host-visible
 *                count the packing needs).
 * Errors: NULL lengths / cu_seqlens / num_tokens -> VLP_ERR_NULL; num_seqs < 1,
 * max_seq_len < 1, a length < 1 or > max_seq_len -> VLP_ERR_INVALID; total >
 * INT32_MAX ("cu_seqlens is int32, so the token count must fit in int32") ->
 * VLP_ERR_OVERFLOW; flat_index != NULL and flat_index_cap < total ->
 * VLP_ERR_CAPACITY (cu_seqlens and num_tokens still filled in).
 */
vlp_status vlp_pack_sequences(const int32_t* lengths, int32_t num_seqs, int32_t max_seq_len,
                              int64_t* flat_index, int64_t flat_index_cap,
                              int32_t* cu_seqlens, int64_t* num_tokens);

/*
 * vlp_grid_capacity -- G_cap(T, N, C) = M + floor((T - M) / C), M = min(T, N).
 *
 * "So you wanna CUDA Graph", "Scheduling without max_seqlen": an upper bound
 * on the number of active tiles for any split of at most T tokens over at
 * most N sequences, usable as a launch size without reading cu_seqlens.
 * Returns -1 if total_tokens < 0, num_seqs < 0 or block_m < 1.
 */
int64_t vlp_grid_capacity(int64_t total_tokens, int32_t num_seqs, int32_t block_m);

/*
 * vlp_build_ragged_grid -- CoRa-style tile metadata on the host.
 *
 * "PyCoRa", "CoRa Metadata" and "So you wanna CUDA Graph", "Scheduling
 * without max_seqlen":
 *   block_offsets[0] = 0, block_offsets[i+1] = block_offsets[i]
 *       + ceil(len_i / block_m), len_i = cu_seqlens[i+1] - cu_seqlens[i]
 *       (the ceiling restarts at every sequence; block_offsets[B] = G, the
 *       number of active tiles);
 *   grid_mapping[f] = the sequence i with block_offsets[i] <= f <
 *       block_offsets[i+1] (zero-length sequences own no tile);
 *   tile_order[s] = the flat tile run by the s-th launched tile slot, longest
 *       sequence first: sequences by length descending (ties: lower index
 *       first), each with its tiles from the last local tile down to tile 0.
 *
 *   cu_seqlens     host int32 [num_seqs + 1]: cu[0] == 0, non-decreasing.
 *   block_offsets  host int32 [num_seqs + 1].
 *   grid_mapping, tile_order  host int32 [grid_cap] (either may be NULL to
 *                  skip it).
 *   num_blocks     host int64*, receives G.
 * Errors: NULL cu_seqlens / block_offsets / num_blocks -> VLP_ERR_NULL;
 * num_seqs < 1, block_m < 1, cu[0] != 0 or decreasing cu -> VLP_ERR_INVALID;
 * G > grid_cap -> VLP_ERR_CAPACITY (block_offsets and num_blocks filled in).
 */
vlp_status vlp_build_ragged_grid(const int32_t* cu_seqlens, int32_t num_seqs, int32_t block_m,
                                 int32_t* block_offsets, int32_t* grid_mapping,
                                 int32_t* tile_order, int64_t grid_cap, int64_t* num_blocks);

/*
 * vlp_build_ragged_grid_device -- the same metadata, built on the GPU from a
 * device cu_seqlens without any host read (one workgroup, enqueued on
 * `stream`).  Bit-identical to vlp_build_ragged_grid whenever num_seqs <=
 * VLP_DEVICE_SORT_MAX_SEQS; above that the device tile_order is the natural
 * order 0..G-1 (block_offsets and grid_mapping are unaffected).
 *
 *   cu_seqlens     device int32 [num_seqs + 1].
 *   block_offsets  device int32 [num_seqs + 1].
 *   grid_mapping, tile_order  device int32 [grid_cap]; entries >= G are set
 *                  to -1.
 *   grid_cap       must be >= G; pass vlp_grid_capacity(T, num_seqs, block_m)
 *                  with T >= cu_seqlens[num_seqs] to be safe.  Tiles beyond
 *                  grid_cap are dropped (undefined metadata), not detected.
 * Errors: NULL pointers -> VLP_ERR_NULL; num_seqs < 1, block_m < 1, grid_cap <
 * 0 -> VLP_ERR_INVALID; launch failure -> VLP_ERR_HIP.
 */
#define VLP_DEVICE_SORT_MAX_SEQS 4096
vlp_status vlp_build_ragged_grid_device(const int32_t* cu_seqlens, int32_t num_seqs, int32_t block_m,
                                        int32_t* block_offsets, int32_t* grid_mapping,
                                        int32_t* tile_order, int64_t grid_cap, void* stream);

/*
 * vlp_kernel_block_m -- the query rows per tile (the C of the ragged grid)
 * that vlp_varlen_attn_fwd uses for these arguments, or -1 if the combination
 * is unsupported.  A grid passed to vlp_varlen_attn_fwd_grid must be built
 * with this block_m.  In first-token mode every sequence is one tile, and the
 * value returned is VLP_FIRST_TOKEN_BLOCK_M (a grid over cu_seqlens_k with
 * this block_m has exactly one tile per non-empty sequence).
 *   max_seqlen  a hint (0 = unknown); the choice never affects correctness.
 */
#define VLP_FIRST_TOKEN_BLOCK_M (1 << 30)
int32_t vlp_kernel_block_m(int32_t dtype, int32_t head_dim, int32_t causal,
                           int32_t query_is_first_token, int32_t num_seqs,
                           int64_t rows_q, int32_t max_seqlen);

/*
 * vlp_bwd_block_m -- the query rows per tile of the backward pass's dq phase
 * (the block_m of its query grid; see vlp_varlen_attn_bwd_grid), or -1 if
 * the dtype / head_dim combination is unsupported.  It may differ from the
 * forward's vlp_kernel_block_m (the forward runs 256-row tiles for 16-bit
 * inputs at head_dim 128, the dq kernel 128-row tiles).  The tiling is the
 * same ragged grid ("PyCoRa", "Ragged Flash Attention"; "So you wanna CUDA
 * Graph", "Scheduling without max_seqlen").
 */
int32_t vlp_bwd_block_m(int32_t dtype, int32_t head_dim, int32_t causal);

/*
 * vlp_varlen_attn_workspace_size -- bytes of device workspace that
 * vlp_varlen_attn_fwd(_persistent) needs for the device-built grid
 * (block_offsets, grid_mapping, tile_order for G_cap(rows, num_seqs,
 * block_m) tiles, where rows = rows_q, or num_seqs in first-token mode) and
 * the persistent schedule's work-queue counters.  Enough for every launch
 * except first-token mode over long sequences (the chunked form, see
 * vlp_varlen_attn_fwd_workspace_size, which covers every case).
 * Errors: NULL bytes -> VLP_ERR_NULL; num_seqs < 1, rows_q < 0, block_m < 1
 * -> VLP_ERR_INVALID.
 */
vlp_status vlp_varlen_attn_workspace_size(int32_t num_seqs, int64_t rows_q, int32_t block_m,
                                          size_t* bytes);

/* Keys per tile of the chunked first-token form, and the longest-sequence
 * key count from which the device-grid entry points take that form. */
#define VLP_FIRST_TOKEN_CHUNK_KEYS 4096
#define VLP_FIRST_TOKEN_CHUNK_MIN 8192

/*
 * vlp_varlen_attn_fwd_workspace_size -- exact bytes of device workspace that
 * vlp_varlen_attn_fwd(_persistent) needs for these arguments (each means
 * what it means there).  In first-token mode without the causal mask, when
 * the longest sequence (max_seqlen, or the mean length when it is 0) has at
 * least VLP_FIRST_TOKEN_CHUNK_MIN keys, the forward takes its chunked form
 * ("gigl.nn.packed_attention", packed_attention with query_is_first_token:
 * one query per sequence, every key of the sequence): the grid is built over
 * the keys, VLP_FIRST_TOKEN_CHUNK_KEYS per tile, one workgroup per (tile,
 * head), and the workspace also
 * holds the partial softmax states of every (tile, head) -- (head_dim + 4)
 * floats each -- and one arrival counter per (sequence, head).
 * Errors: NULL bytes -> VLP_ERR_NULL; dtype or head_dim not built ->
 * VLP_ERR_UNSUPPORTED; num_seqs < 1, heads < 1, negative counts, causal or
 * query_is_first_token not 0/1 -> VLP_ERR_INVALID; rows beyond int32 or a
 * grid of more than int32 (tile, head) tasks -> VLP_ERR_OVERFLOW.
 */
vlp_status vlp_varlen_attn_fwd_workspace_size(int32_t dtype, int32_t num_seqs, int64_t rows_q, int64_t total_k,
                                              int32_t heads, int32_t head_dim, int32_t max_seqlen,
                                              int32_t causal, int32_t query_is_first_token, size_t* bytes);

/*
 * vlp_varlen_attn_fwd -- packed attention forward, out = softmax(scale q k^T) v
 * within each sequence, plus the log-sum-exp of every query row.
 *
 * "gigl.nn.packed_attention" (packed_attention; "Example"), "PyCoRa" ("Ragged
 * Flash Attention"), "DanLing NestedTensor" 3.3 ("Attention through packed
 * blocks": the output takes the query structure; query and key lengths may
 * differ).  Enqueues, on `stream`, the device grid build into `workspace`
 * (no host read of cu_seqlens) and one attention launch of
 * G_cap * heads workgroups in which surplus tiles exit at once (the static
 * grid; vlp_varlen_attn_fwd_persistent launches fewer).
 *
 *   dtype          VLP_FP32, VLP_FP16 or VLP_BF16 for q, k, v and out; the
 *                  contractions accumulate in fp32, the softmax runs in fp32.
 *   q              device [rows_q, heads, head_dim]; in first-token mode
 *                  rows_q == num_seqs and row i is the query of sequence i
 *                  (the page's query[cu_seqlens[:-1]]).
 *   k, v           device [total_k, heads, head_dim].
 *   cu_seqlens_q   device int32 [num_seqs + 1] (ignored, may be NULL, in
 *                  first-token mode).
 *   cu_seqlens_k   device int32 [num_seqs + 1]; cu[0] = 0, non-decreasing,
 *                  cu[B] <= total_k.  Zero-length sequences are allowed
 *                  (capacity tails [0, .., L, L, L]) except in first-token
 *                  mode, where every sequence needs a key.
 *   num_seqs       B >= 1.
 *   rows_q         physical query rows (>= cu_seqlens_q[B]); rows not owned
 *                  by a sequence are never written.
 *   total_k        physical key rows.
 *   heads, head_dim  heads >= 1; head_dim in {16, 32, 64, 128} ("head_dim must
 *                  be a multiple of 8"; these four are built).
 *   q_row_stride, kv_row_stride, out_row_stride
 *                  elements between consecutive tokens of q, of k and v (one
 *                  stride shared by both), and of out; within a token the
 *                  heads are head_dim elements apart and each head's
 *                  head_dim elements are contiguous.  0 = heads * head_dim
 *                  (contiguous).  Larger strides take views into a fused
 *                  projection output, e.g. q, k, v = qkv.view(T, 3, H, D)
 *                  .unbind(1) with stride 3 * H * D ("PyCoRa", "Ragged Flash
 *                  Attention": the attention module passes such unbound
 *                  views).  Each must be >= heads * head_dim, give 16-byte
 *                  aligned rows, and stride * element size <= 2^24 bytes.
 *   max_seqlen     a hint (0 = unknown); never needed for correctness.
 *   scale          any finite softmax scale (usually 1/sqrt(head_dim)).  A
 *                  negative scale runs as |scale| with q's sign flipped in
 *                  the score products (scale * s = |scale| * (-s)).
 *   causal         0/1: key j of a sequence is visible to its query at local
 *                  position p iff j <= p + (Lk - Lq) (bottom-right aligned).
 *   query_is_first_token  0/1: one query per sequence, at local position 0.
 *   out            device [rows_q, heads, head_dim] in dtype.
 *   lse            device fp32 [heads, rows_q] or NULL: natural-log
 *                  log-sum-exp of the scaled scores; -inf (and a zero output
 *                  row) for a query that sees no key.
 *   workspace      device, >= vlp_varlen_attn_fwd_workspace_size bytes,
 *                  256-byte aligned; overwritten.
 * q, k, v and out must be 16-byte aligned.
 * Errors: NULL q/k/v/out/cu_seqlens_k/workspace (or cu_seqlens_q outside
 * first-token mode) -> VLP_ERR_NULL; dtype or head_dim not built ->
 * VLP_ERR_UNSUPPORTED; num_seqs < 1, heads < 1, rows_q < 0, total_k < 0,
 * non-finite scale, misaligned pointers, a stride below heads *
 * head_dim or not giving 16-byte aligned rows, rows_q != num_seqs in
 * first-token mode -> VLP_ERR_INVALID; rows or rows*heads beyond int32, a
 * stride beyond 2^24 bytes -> VLP_ERR_OVERFLOW; small workspace ->
 * VLP_ERR_CAPACITY; launch failure -> VLP_ERR_HIP.
 */
vlp_status vlp_varlen_attn_fwd(int32_t dtype, const void* q, const void* k, const void* v,
                               const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                               int32_t num_seqs, int64_t rows_q, int64_t total_k,
                               int32_t heads, int32_t head_dim, int64_t q_row_stride,
                               int64_t kv_row_stride, int64_t out_row_stride, int32_t max_seqlen,
                               float scale, int32_t causal, int32_t query_is_first_token,
                               void* out, float* lse, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * vlp_varlen_attn_fwd_grid -- the same forward with caller-supplied, cached
 * tile metadata ("PyCoRa", "CoRa Metadata": computed once and cached).
 *
 *   grid_mapping, block_offsets, tile_order  device int32, as produced by
 *                  vlp_build_ragged_grid(_device) for cu_seqlens_q (or, in
 *                  first-token mode, cu_seqlens_k) with `block_m`.
 *   tile_order     may be NULL: flat tiles then run in natural order.
 *   num_blocks     G, the number of active tiles; exactly G * heads
 *                  workgroups are launched.
 *   block_m        must equal vlp_kernel_block_m(...) for these arguments.
 * Errors: as vlp_varlen_attn_fwd (workspace not used), plus NULL grid_mapping
 * / block_offsets -> VLP_ERR_NULL, num_blocks < 0 or a block_m mismatch ->
 * VLP_ERR_INVALID, num_blocks * heads beyond int32 -> VLP_ERR_OVERFLOW.
 */
vlp_status vlp_varlen_attn_fwd_grid(int32_t dtype, const void* q, const void* k, const void* v,
                                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                    int32_t num_seqs, int64_t rows_q, int64_t total_k,
                                    int32_t heads, int32_t head_dim, int64_t q_row_stride,
                                    int64_t kv_row_stride, int64_t out_row_stride, int32_t max_seqlen,
                                    float scale, int32_t causal, int32_t query_is_first_token,
                                    void* out, float* lse,
                                    const int32_t* grid_mapping, const int32_t* block_offsets,
                                    const int32_t* tile_order, int64_t num_blocks, int32_t block_m,
                                    void* stream);

/* Bytes of the library-owned device scratch of vlp_varlen_attn_fwd_noalloc
 * (one copy per GPU, held until the process ends). */
#define VLP_NOALLOC_SCRATCH_BYTES (4u << 20)

/*
 * vlp_varlen_attn_fwd_noalloc -- vlp_varlen_attn_fwd without a workspace
 * argument and without any allocation, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  The tile metadata the device grid build
 * writes (vlp_varlen_attn_workspace_size bytes for these sizes) goes into a
 * file-scope device array of VLP_NOALLOC_SCRATCH_BYTES bytes inside the
 * library instead, whose address on the current device is looked up once
 * (hipGetSymbolAddress) on the first call there.  Same kernels, same
 * arguments (minus workspace) and bit-identical results as
 * vlp_varlen_attn_fwd on the static grid; nothing in the scratch has to
 * start at zero (every entry the kernels read is rewritten by the grid build
 * of the same call).  All calls on one GPU share its scratch: calls that may
 * overlap on one GPU (different streams without ordering between them) race
 * and must not be made.  VLP_CHECK=1 is not honoured here (the check
 * allocates and synchronises).
 * Errors: as vlp_varlen_attn_fwd; metadata larger than
 * VLP_NOALLOC_SCRATCH_BYTES (about a million tile slots) -> VLP_ERR_CAPACITY,
 * checked on the host before any HIP call; a failed symbol lookup ->
 * VLP_ERR_HIP.
 */
vlp_status vlp_varlen_attn_fwd_noalloc(int32_t dtype, const void* q, const void* k, const void* v,
                                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                       int32_t num_seqs, int64_t rows_q, int64_t total_k,
                                       int32_t heads, int32_t head_dim, int64_t q_row_stride,
                                       int64_t kv_row_stride, int64_t out_row_stride, int32_t max_seqlen,
                                       float scale, int32_t causal, int32_t query_is_first_token,
                                       void* out, float* lse, void* stream);

/*
 * vlp_varlen_attn_fwd_persistent -- vlp_varlen_attn_fwd with the persistent
 * schedule of "So you wanna CUDA Graph" ("Graph overcapture: bound
 * capacity-sized launches"): instead of one workgroup per capacity task
 * (G_cap(rows_q, num_seqs, block_m) * heads, the surplus exiting at once),
 * min(capacity tasks, W) workgroups are launched and they take the ACTIVE
 * tasks (block_offsets[num_seqs] * heads, read on the device) from work
 * queues in device memory (one per XCD, in longest-first order, cleared by
 * the grid build that precedes the launch), so a launch recorded for a large
 * token capacity launches no more workgroups than the device holds.  Every
 * argument means what it means for vlp_varlen_attn_fwd (the workspace also
 * holds the queue counters: calls that share a workspace must not overlap),
 * and the results are bit-identical to it (each task computes the same
 * values).
 *
 *   num_workers    W; 0 = the number of workgroups of the kernel the device
 *                  holds at once (compute units x workgroups per unit);
 *                  > 0 = at most that many (8 or more keep every task on
 *                  the XCD the static grid would run it on).
 * Errors: as vlp_varlen_attn_fwd, plus num_workers < 0 -> VLP_ERR_INVALID.
 */
vlp_status vlp_varlen_attn_fwd_persistent(int32_t dtype, const void* q, const void* k, const void* v,
                                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                          int32_t num_seqs, int64_t rows_q, int64_t total_k,
                                          int32_t heads, int32_t head_dim, int64_t q_row_stride,
                                          int64_t kv_row_stride, int64_t out_row_stride,
                                          int32_t max_seqlen, float scale, int32_t causal,
                                          int32_t query_is_first_token, void* out, float* lse,
                                          void* workspace, size_t workspace_bytes, int32_t num_workers,
                                          void* stream);

/*
 * Key rows per tile of the key grid that the dk/dv kernel of the backward
 * walks (for every dtype and head_dim).
 */
#define VLP_BWD_BLOCK_K 64

/*
 * vlp_varlen_attn_bwd_workspace_size -- bytes of device workspace that
 * vlp_varlen_attn_bwd(_persistent) needs: two fp32 [heads, rows_q] row
 * statistics plus a device-built grid over the query lengths and one over
 * the key lengths (G_cap(rows_q, num_seqs, block_m) and G_cap(total_k,
 * num_seqs, VLP_BWD_BLOCK_K) tiles, each with its work-queue counters),
 * block_m = vlp_bwd_block_m(dtype, head_dim, causal).
 * Errors: NULL bytes -> VLP_ERR_NULL; num_seqs < 1, rows_q < 0, total_k < 0,
 * heads < 1, block_m < 1 -> VLP_ERR_INVALID; rows beyond int32 ->
 * VLP_ERR_OVERFLOW.
 */
vlp_status vlp_varlen_attn_bwd_workspace_size(int32_t num_seqs, int64_t rows_q, int64_t total_k, int32_t heads,
                                              int32_t block_m, size_t* bytes);

/*
 * vlp_varlen_attn_bwd -- gradients of vlp_varlen_attn_fwd with respect to q,
 * k and v, given the output gradient dout.
 *
 * "gigl.nn.packed_attention", "Why this exists" (the packed attention is
 * trained through; a backward kernel supplies its gradients) and "So you
 * wanna CUDA Graph", "Correctness tangent" (gradients of inactive rows may
 * stay undefined).  The pages give no backward algorithm; what is computed is
 * the derivative of the forward: per sequence and head, with P its softmax
 * weights, dv = P^T dout, dS = P * (dout v^T - rowsum(dout * out)),
 * dq = scale * dS k, dk = scale * dS^T q.  Enqueues on `stream` two device
 * grid builds and two kernels (dq over query tiles, then dk/dv over key
 * tiles); no atomics, so the result is bitwise reproducible.
 *
 *   dtype          VLP_FP32, VLP_FP16 or VLP_BF16; fp32 accumulation,
 *                  gradients rounded to dtype.
 *   q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, rows_q, total_k, heads,
 *   head_dim, q_row_stride, kv_row_stride, out_row_stride, max_seqlen,
 *   scale, causal  as for vlp_varlen_attn_fwd (no first-token mode).
 *   dout_row_stride, dq_row_stride, dkv_row_stride
 *                  token strides of dout, of dq, and of dk and dv (one
 *                  stride shared by both), with the same rules; views into
 *                  one fused gradient buffer are allowed.
 *   out            device [rows_q, heads, head_dim], the forward's output.
 *   dout           device [rows_q, heads, head_dim], gradient of the output.
 *   lse            device fp32 [heads, rows_q], the forward's log-sum-exp.
 *   dq             device [rows_q, heads, head_dim]: rows owned by a sequence
 *                  are written (zeros for a query that sees no key); other
 *                  rows are never written.
 *   dk, dv         device [total_k, heads, head_dim]: rows owned by a
 *                  sequence are written (zeros for a key that no query sees);
 *                  other rows are never written.
 *   workspace      device, >= vlp_varlen_attn_bwd_workspace_size bytes,
 *                  256-byte aligned; overwritten.
 * q, k, v, out, dout, dq, dk and dv must be 16-byte aligned, lse 4-byte.
 * dq, dk and dv must not overlap any input or each other's elements (they
 * may be disjoint views into one buffer).
 * Errors: as vlp_varlen_attn_fwd, plus NULL dout/lse/dq/dk/dv/workspace ->
 * VLP_ERR_NULL, misaligned dout/dq/dk/dv/lse/workspace -> VLP_ERR_INVALID,
 * small workspace -> VLP_ERR_CAPACITY.
 */
vlp_status vlp_varlen_attn_bwd(int32_t dtype, const void* q, const void* k, const void* v, const void* out,
                               const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t rows_q, int64_t total_k,
                               int32_t heads, int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride,
                               int64_t out_row_stride, int64_t dout_row_stride, int64_t dq_row_stride,
                               int64_t dkv_row_stride, int32_t max_seqlen, float scale, int32_t causal,
                               void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * vlp_varlen_attn_bwd_persistent -- vlp_varlen_attn_bwd with the persistent
 * schedule (see vlp_varlen_attn_fwd_persistent): each of the two gradient
 * launches has min(its capacity tasks, W) workgroups taking its active
 * tasks from its own work queues.  Arguments and results (bit-identical) as for
 * vlp_varlen_attn_bwd; num_workers as for vlp_varlen_attn_fwd_persistent,
 * W counted per launch.
 * Errors: as vlp_varlen_attn_bwd, plus num_workers < 0 -> VLP_ERR_INVALID.
 */
vlp_status vlp_varlen_attn_bwd_persistent(int32_t dtype, const void* q, const void* k, const void* v,
                                          const void* out, const void* dout, const float* lse,
                                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                          int32_t num_seqs, int64_t rows_q, int64_t total_k, int32_t heads,
                                          int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride,
                                          int64_t out_row_stride, int64_t dout_row_stride,
                                          int64_t dq_row_stride, int64_t dkv_row_stride, int32_t max_seqlen,
                                          float scale, int32_t causal, void* dq, void* dk, void* dv,
                                          void* workspace, size_t workspace_bytes, int32_t num_workers,
                                          void* stream);

/*
 * vlp_varlen_attn_bwd_grid -- the same gradients with caller-supplied, cached
 * tile metadata ("PyCoRa", "CoRa Metadata": computed once and cached) and a
 * caller-owned row-statistics buffer, run in one or both phases.
 *
 *   q_grid_mapping, q_block_offsets, q_tile_order, q_num_blocks
 *                  the ragged grid of cu_seqlens_q, as built by
 *                  vlp_build_ragged_grid(_device) with block_m (tile_order
 *                  may be NULL: natural order); q_num_blocks * heads
 *                  workgroups run the dq phase.
 *   k_grid_mapping, k_block_offsets, k_tile_order, k_num_blocks
 *                  the ragged grid of cu_seqlens_k built with block_m =
 *                  VLP_BWD_BLOCK_K; k_num_blocks * heads workgroups run the
 *                  dk/dv phase.
 *   block_m        the query grid's; must equal vlp_bwd_block_m(dtype,
 *                  head_dim, causal).
 *   row_stats      device fp32 [2, heads, rows_q], 4-byte aligned: written by
 *                  the dq phase (the log-sum-exp in base-2 units and
 *                  rowsum(dout * out) of every owned query row), read by the
 *                  dk/dv phase.
 *   phases         VLP_BWD_DQ, VLP_BWD_DKDV or both (dq first).  The dk/dv
 *                  phase alone needs row_stats from an earlier dq phase on
 *                  the same inputs.
 * Errors: as vlp_varlen_attn_bwd (no workspace), plus NULL row_stats or a
 * NULL grid of a requested phase -> VLP_ERR_NULL; phases outside 1..3, a
 * block_m mismatch, negative block counts, misaligned row_stats ->
 * VLP_ERR_INVALID; block counts * heads beyond int32 -> VLP_ERR_OVERFLOW.
 */
#define VLP_BWD_DQ 1
#define VLP_BWD_DKDV 2
vlp_status vlp_varlen_attn_bwd_grid(int32_t dtype, const void* q, const void* k, const void* v, const void* out,
                                    const void* dout, const float* lse, const int32_t* cu_seqlens_q,
                                    const int32_t* cu_seqlens_k, int32_t num_seqs, int64_t rows_q, int64_t total_k,
                                    int32_t heads, int32_t head_dim, int64_t q_row_stride, int64_t kv_row_stride,
                                    int64_t out_row_stride, int64_t dout_row_stride, int64_t dq_row_stride,
                                    int64_t dkv_row_stride, int32_t max_seqlen, float scale,
                                    int32_t causal, void* dq, void* dk, void* dv, const int32_t* q_grid_mapping,
                                    const int32_t* q_block_offsets, const int32_t* q_tile_order,
                                    int64_t q_num_blocks, const int32_t* k_grid_mapping,
                                    const int32_t* k_block_offsets, const int32_t* k_tile_order,
                                    int64_t k_num_blocks, int32_t block_m, float* row_stats, int32_t phases,
                                    void* stream);

/*
 * Token rows per tile of the ragged grid that vlp_ragged_matmul walks.
 */
#define VLP_MATMUL_BLOCK_M 128

/*
 * vlp_ragged_matmul_workspace_size -- bytes of device workspace that
 * vlp_ragged_matmul(_persistent) needs (its device-built grid: G_cap(rows,
 * num_seqs, VLP_MATMUL_BLOCK_M) tiles, and work-queue counters).
 * Errors: NULL bytes -> VLP_ERR_NULL; num_seqs < 1, rows < 0 ->
 * VLP_ERR_INVALID.
 */
vlp_status vlp_ragged_matmul_workspace_size(int32_t num_seqs, int64_t rows, size_t* bytes);

/*
 * vlp_ragged_matmul -- y = x W_i^T (+ b_i) on the rows of every sequence i
 * of a packed batch.
 *
 * "PyCoRa", "Ragged Matrix Multiplication": each sequence is multiplied by
 * its own weight matrix, thread blocks finding their sequence through the
 * ragged-grid metadata ("CoRa Metadata").  With weight_seq_stride = 0 every
 * sequence shares one weight: the packed linear layer of
 * "gigl.nn.packed_attention" ("Why this exists").  Enqueues on `stream` the
 * device grid build and one launch; no host read of cu_seqlens.
 *
 *   dtype          VLP_BF16 or VLP_FP16 (VLP_FP32 -> VLP_ERR_UNSUPPORTED);
 *                  fp32 accumulation, y rounded to dtype once.
 *   x              device [rows, in_features], contiguous.
 *   weight         device; sequence i's matrix is [out_features,
 *                  in_features] row-major (a linear layer's weight) at
 *                  weight + i * weight_seq_stride elements.
 *   bias           device or NULL; sequence i's bias is out_features
 *                  elements at bias + i * bias_seq_stride.
 *   cu_seqlens     device int32 [num_seqs + 1]: cu[0] = 0, non-decreasing,
 *                  cu[B] <= rows; zero-length sequences allowed.
 *   rows           physical rows of x and y; rows not owned by a sequence
 *                  are never written.
 *   in_features    a multiple of 64 in [64, 65536].
 *   out_features   a multiple of 4 in [4, 65536].
 *   weight_seq_stride, bias_seq_stride  >= 0; 0 = shared; multiples of 8
 *                  (weight) and 4 (bias) elements.
 *   y              device [rows, out_features], contiguous; must not overlap
 *                  x, weight or bias.
 *   workspace      device, >= vlp_ragged_matmul_workspace_size bytes,
 *                  256-byte aligned; overwritten.
 * x, weight, bias and y must be 16-byte aligned.
 * Errors: NULL x/weight/cu_seqlens/y/workspace -> VLP_ERR_NULL; dtype not
 * built -> VLP_ERR_UNSUPPORTED; num_seqs < 1, rows < 0, feature counts out of
 * range or not multiples, negative or misaligned strides, misaligned pointers
 * -> VLP_ERR_INVALID; rows beyond int32 or a grid beyond int32 workgroups ->
 * VLP_ERR_OVERFLOW; small workspace -> VLP_ERR_CAPACITY; launch failure ->
 * VLP_ERR_HIP.
 */
vlp_status vlp_ragged_matmul(int32_t dtype, const void* x, const void* weight, const void* bias,
                             const int32_t* cu_seqlens, int32_t num_seqs, int64_t rows, int32_t in_features,
                             int32_t out_features, int64_t weight_seq_stride, int64_t bias_seq_stride, void* y,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * vlp_ragged_matmul_persistent -- vlp_ragged_matmul with the persistent
 * schedule (see vlp_varlen_attn_fwd_persistent): min(capacity tasks, W)
 * workgroups take the (row tile, column tile) tasks of the active rows from
 * work queues.  Arguments and results (bit-identical) as for vlp_ragged_matmul;
 * num_workers as for vlp_varlen_attn_fwd_persistent.
 * Errors: as vlp_ragged_matmul, plus num_workers < 0 -> VLP_ERR_INVALID.
 */
vlp_status vlp_ragged_matmul_persistent(int32_t dtype, const void* x, const void* weight, const void* bias,
                                        const int32_t* cu_seqlens, int32_t num_seqs, int64_t rows,
                                        int32_t in_features, int32_t out_features, int64_t weight_seq_stride,
                                        int64_t bias_seq_stride, void* y, void* workspace,
                                        size_t workspace_bytes, int32_t num_workers, void* stream);

/*
 * vlp_cu_seqlens_from_ids -- cu_seqlens of the runs of equal document ids in
 * one packed sequence, built on the GPU (one workgroup, enqueued on `stream`,
 * no host read).
 *
 * A query attending only to keys of its own document (the sample-id mask of
 * one packed sequence) is varlen attention over the runs ("DanLing
 * NestedTensor" 3.3: varlen kernels take the segment boundaries).  Tokens of
 * a document must be contiguous: a change of id between neighbouring tokens
 * starts a new sequence, so an id that comes back after another document
 * starts a separate sequence.  The result has a fixed capacity ("So you
 * wanna CUDA Graph", "Terminology time"): cu_seqlens[0..n-1] are the run
 * starts, cu_seqlens[n..max_seqs] = num_tokens (zero-length sequences that
 * every kernel here skips), so it can be passed on with num_seqs = max_seqs.
 *
 *   ids            device int32 [num_tokens] (may be NULL when num_tokens is 0).
 *   max_seqs       >= 1, the capacity.
 *   cu_seqlens     device int32 [max_seqs + 1].
 *   num_seqs       device int32 [1]: receives the number of runs n.  If n >
 *                  max_seqs only the first max_seqs starts are written and
 *                  cu_seqlens must not be used.
 * Errors: NULL cu_seqlens / num_seqs (or ids with num_tokens > 0) ->
 * VLP_ERR_NULL; num_tokens < 0, max_seqs < 1 -> VLP_ERR_INVALID; num_tokens
 * beyond int32 -> VLP_ERR_OVERFLOW; launch failure -> VLP_ERR_HIP.
 */
vlp_status vlp_cu_seqlens_from_ids(const int32_t* ids, int64_t num_tokens, int32_t max_seqs, int32_t* cu_seqlens,
                                   int32_t* num_seqs, void* stream);

/*
 * vlp_mfma_rate -- the matrix-core rate at the running clock, the measured
 * ceiling beside the datasheet peak for roofline reporting (not an operation
 * of the pages: a calibration launch for measurement tools).  One launch of
 * `blocks` workgroups of eight waves (two per SIMD; one workgroup per CU at
 * a time); every wave runs `iters` rounds of four
 * independent products with the instruction the attention kernels use for
 * `dtype` (32x32x16 bf16 / fp16, 32x32x2 fp32) on register operands, with no
 * memory traffic until each thread writes one float of its sums to `sink`.
 * The caller times it on `stream` and divides *flops by the time.
 *
 *   dtype   VLP_FP32, VLP_FP16 or VLP_BF16.
 *   blocks  1 .. 65536 (the CU count keeps every SIMD busy).
 *   iters   1 .. 1,048,576.
 *   sink    device float [blocks * 512], overwritten (values meaningless).
 *   flops   host double: receives the flop count of the launch
 *           (2 * 32 * 32 * K per product, K = 16 for 16-bit and 2 for fp32).
 * Errors: other dtype -> VLP_ERR_UNSUPPORTED; NULL sink or flops ->
 * VLP_ERR_NULL; blocks or iters out of range -> VLP_ERR_INVALID; launch
 * failure -> VLP_ERR_HIP.
 */
vlp_status vlp_mfma_rate(int32_t dtype, int32_t blocks, int32_t iters, float* sink, double* flops, void* stream);

/* vlp_build_info -- a static string "csrc=<hash> arch=gfx950" naming the
 * sources this library was built from: <hash> is the first 16 hex digits of
 * a SHA-256 over the library's source files and this header (the build
 * computes it; see variable_length_packed_pack_amd/build.py, source_hash).
 * Callers compare it with the hash of the sources they hold to make sure a
 * prebuilt library is not stale.  Never fails; the string is owned by the
 * library. */
const char* vlp_build_info(void);

/* vlp_status_string -- a static, human-readable name for a status code; for
 * VLP_ERR_HIP, the text of the last HIP error seen on this thread. */
const char* vlp_status_string(vlp_status status);

#ifdef __cplusplus
}
#endif

#endif /* VLP_H_ */
