/*
 * mla_decode.h -- C ABI of an MI355X (gfx950) library for multi-head latent
 * attention (MLA) decode over a paged latent KV cache, split along the key
 * axis into segments whose base-2 partials are merged into the output plus a
 * natural-log LSE.
 *
 * Pages this interface follows (cited by page title and section):
 *  - vLLM API page "vllm.v1.attention.ops.rocm_aiter_mla_merge": module
 *    description (segment partition tiles_per_segment =
 *    cdiv(seq_len, NUM_SEGMENTS * TILE_SIZE); base-2 partials; natural-log LSE
 *    for a later cross-rank merge) and merge_mla_segments_triton (partials
 *    [T, H, S, 512], output [T, H, 512] in out_dtype, lse [T, H] fp32).
 *  - Source page "rocm_aiter_mla.py" (vLLM AITER MLA backend):
 *    _segmented_mla_page_size (TILE = min(128, largest power-of-two divisor of
 *    the block)), _forward_segmented_dcp_verify (q = [q_nope(512) || q_pe(64)],
 *    cache viewed as [blocks, page, 576], kv_descale scales the cache, causal
 *    rows of a multi-token query block), dcp_local_verify_row_lens (row t of a
 *    qlen-token block sees positions [0, seq_len - qlen + t]) and
 *    _expand_page_indices_kernel (block table strides come from the caller).
 *  - vLLM API page "vllm.v1.attention.backends.mla.rocm_aiter_mla_sparse":
 *    ROCMAiterMLASparseImpl.__init__ (sinks are fp32, one per head) and
 *    _forward_mla (sink folded in after the merge with logaddexp).
 *
 * Conventions
 *  - Every pointer named "device" is GPU memory owned by the caller; the
 *    library never allocates, frees or retains it.  "stream" is a hipStream_t
 *    (NULL = the legacy default stream).  Calls are stream-ordered and
 *    asynchronous: no call reads device memory on the host or synchronises, so
 *    every launch is graph-capturable.
 *  - All argument checking happens on the host before any launch.  On error
 *    nothing is launched and a negative status is returned; mla_last_error()
 *    gives a message (thread-local).
 *  - Device-side metadata (seq_lens, qo_indptr, block ids) cannot be checked
 *    without a sync.  The kernels clamp it so that no access leaves the
 *    buffers the descriptor describes; a request whose metadata is out of range
 *    produces NaN in its outputs instead.
 */
#ifndef MLA_DECODE_H_
#define MLA_DECODE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1) /* shape, stride, alignment, NULL, tile or S */
#define MLA_ERR_UNSUPPORTED (-2) /* head count > 128 or a dtype pair not offered */
#define MLA_ERR_WORKSPACE (-3)   /* workspace missing or too small */
#define MLA_ERR_HIP (-4)         /* launch failed; message carries the HIP error */

/* Element types. */
#define MLA_DTYPE_BF16 1
#define MLA_DTYPE_FP8_E4M3 2 /* OCP float8 e4m3 "fn" (max 448, no inf) */
#define MLA_DTYPE_FP16 3     /* output only */
#define MLA_DTYPE_FP32 4     /* output only */

#define MLA_HEAD_DIM 576     /* kv_lora_rank 512 + rope 64 */
#define MLA_KV_LORA_RANK 512 /* V is the first 512 dims of each cache row */
#define MLA_MAX_HEADS 128
#define MLA_MAX_SEGMENTS 256
#define MLA_MAX_TILE 128

/* How mla_decode splits the key axis (mla_problem.schedule). */
#define MLA_SCHEDULE_SEGMENTS 0 /* the segment partition of the merge page's module
                                   description, S = num_segments (0 = the planner's S) */
#define MLA_SCHEDULE_BALANCED 1 /* equal key ranges per workgroup (num_segments must be 0) */

/*
 * One decode batch.  Set struct_size = sizeof(mla_problem); zero-fill unused
 * fields.  Rows of a request: its qlen new query tokens x num_heads.
 */
typedef struct mla_problem {
  size_t struct_size;

  int32_t num_tokens;   /* T: query tokens in the batch (sum of qlen) */
  int32_t num_heads;    /* H: 1..128 */
  int32_t num_reqs;     /* R: requests */
  int32_t head_dim;     /* must be 576 */
  int32_t kv_lora_rank; /* must be 512 */

  /* q: device [T, H, 576] of q_dtype.  Element strides; the last dim is
   * contiguous.  Base 16-byte aligned, strides multiples of 16 bytes. */
  const void* q;
  int32_t q_dtype; /* MLA_DTYPE_BF16 or MLA_DTYPE_FP8_E4M3: equal to kv_dtype, or
                      BF16 with an FP8 cache (then q is quantised in the load path,
                      see q_pe below) */
  int64_t q_stride_token;
  int64_t q_stride_head;
  const float* q_scale; /* device fp32 scalar: real q = code * q_scale; NULL = 1 */

  /* Paged cache: device [num_blocks, block_size, 576] of kv_dtype, contiguous,
   * 16-byte aligned.  Row j of request r lives in block
   * block_table[r, j / block_size] at offset j % block_size. */
  const void* kv_cache;
  int32_t kv_dtype;      /* MLA_DTYPE_BF16 or MLA_DTYPE_FP8_E4M3 */
  int32_t block_size;    /* >= 1 */
  int64_t num_blocks;    /* >= 1 */
  const float* kv_scale; /* device fp32 scalar: real row = code * kv_scale; NULL = 1 */

  /* block_table: device int32, element strides (a view: both strides used). */
  const int32_t* block_table;
  int64_t bt_stride_row;
  int64_t bt_stride_col;
  int32_t max_blocks_per_req; /* columns of the table; >= cdiv(max_seq_len, block_size) */

  /* seq_lens: device int32 [R], KV length of each request including its new
   * tokens.  qo_indptr: device int32 [R+1] (query tokens of request r are
   * [qo_indptr[r], qo_indptr[r+1])), or NULL for one token per request (T == R). */
  const int32_t* seq_lens;
  const int32_t* qo_indptr;

  /* Host-side bounds (no device read is ever made for them). */
  int32_t max_qlen;     /* >= every qlen; 1 when qo_indptr is NULL */
  int32_t max_seq_len;  /* >= every seq_len */
  int64_t sum_seq_lens; /* optional hint for the planner (0 = assume R * max_seq_len) */

  int32_t causal;      /* nonzero: row i of a qlen block sees seq_len - qlen + i + 1 keys */
  float softmax_scale; /* scores = softmax_scale * (q . row) over all 576 dims */
  int32_t tile_size;   /* 0 = min(128, largest power-of-two divisor of block_size);
                          else a power of two <= 128 dividing block_size */
  int32_t num_segments; /* S >= 1; mla_decode also accepts 0: the planner picks S
                           (mla_resolve_num_segments), or the balanced split
                           when schedule == MLA_SCHEDULE_BALANCED */
  int32_t max_workgroups; /* balanced split: at most this many workgroups
                             (0 = as many as the device holds at once), e.g.
                             to leave compute units to concurrent work */

  /* Ragged page lists (NULL = the 2-D table above).  When set, device int32
   * [R+1], non-decreasing: the pages of request r are
   * block_table[(bt_indptr[r] + i) * bt_stride_col] for i < bt_indptr[r+1] -
   * bt_indptr[r] (bt_stride_row and max_blocks_per_req are then unused), and a
   * seq_len past that count times block_size is reported as NaN like a length
   * past the table.  With block_size 1 this is the index stream of the sparse
   * MLA page's decode (vLLM API page "rocm_aiter_mla_sparse",
   * ROCMAiterMLASparseImpl.forward_mqa / _forward_mla: one request per query
   * token, paged_kv_indptr / paged_kv_indices over a [rows, 1, 576] cache). */
  const int32_t* bt_indptr;

  /* The q prologue of the sparse MLA page's forward_mqa (q arrives as the
   * pair (ql_nope, q_pe); the fp8 path concatenates and quantises it with the
   * layer's q scale before the decode), fused into the decode's q load:
   *  - q_pe set: q holds the 512 latent dims [T, H, 512] (q strides, head
   *    stride >= 512) and q_pe the 64 rope dims, device [T, H, 64] of q_dtype
   *    with element strides q_pe_stride_token / q_pe_stride_head (last dim
   *    contiguous, rows 16-byte aligned).  NULL: q is [T, H, 576].
   *  - q_dtype BF16 with an FP8 cache: each q value x becomes the e4m3 code of
   *    x / q_scale (IEEE single division, then saturated to +-448 and rounded
   *    to nearest even), whose dequantised value code * q_scale enters the
   *    scores; q_scale NULL = 1. */
  const void* q_pe;
  int64_t q_pe_stride_token;
  int64_t q_pe_stride_head;

  /* mla_decode only: MLA_SCHEDULE_SEGMENTS (0, the segment partition) or
   * MLA_SCHEDULE_BALANCED (1, see mla_decode).  The segment entry points
   * require 0. */
  int32_t schedule;
} mla_problem;

/*
 * Host-only check of a descriptor (no GPU call).  Returns MLA_OK or an error.
 * require_segments: nonzero -> num_segments must be >= 1.
 */
int mla_validate(const mla_problem* p, int require_segments);

/*
 * Segment partials.  Partition (per request, from its seq_len): TILE as
 * above, tps = cdiv(seq_len, S * TILE); segment s covers positions
 * [s*tps*TILE, min((s+1)*tps*TILE, seq_len)) and is valid iff its start is
 * < seq_len.  For every query row (t, h) and valid segment s, with
 * x_j = softmax_scale * log2(e) * (q . row_j) over the positions j of the
 * segment that the row sees:
 *   segm_max[t,h,s]    = max_j x_j                           (base 2)
 *   segm_expsum[t,h,s] = sum_j 2^(x_j - segm_max)
 *   segm_output[t,h,s] = sum_j 2^(x_j - segm_max) * V_j       (unnormalised,
 *                        dequantised units, V_j = row_j[0:512])
 * A valid segment with no visible position (causal) is (0 vector, -inf, 0).
 * Slots of invalid segments are left untouched.
 * Buffers (device fp32, contiguous): segm_output [T, H, S, 512],
 * segm_max [T, H, S], segm_expsum [T, H, S].
 */
int mla_decode_segments(const mla_problem* p, float* segm_output, float* segm_max,
                        float* segm_expsum, void* stream);

/*
 * Merge of segment partials.  part_lens: device int32 [T], the length the
 * partition of token t was built from (its request's seq_len).  For each (t, h)
 * over the valid segments: M = max_s m_s, L = sum_s l_s 2^(m_s - M),
 * out = sum_s acc_s 2^(m_s - M) / L, lse = ln2 * (M + log2 L).  A row with no
 * key gets out = 0, lse = -inf.  With sinks (device fp32 [H], or NULL):
 * lse' = logaddexp(lse, sink[h]), out' = out * exp(lse - lse') (0 for rows
 * without keys).  out: device [T, H, 512] of out_dtype (BF16 rounded to
 * nearest even, FP16 or FP32), lse: device fp32 [T, H].  Contiguous.
 */
int mla_merge_segments(const float* segm_output, const float* segm_max, const float* segm_expsum,
                       const int32_t* part_lens, int32_t num_tokens, int32_t num_heads,
                       int32_t num_segments, int32_t kv_lora_rank, int32_t tile_size,
                       const float* sinks, void* out, int32_t out_dtype, float* lse,
                       void* stream);

/*
 * Cross-shard combine for decode context parallelism (the cross-rank merge
 * that consumes the natural-log LSE of the merge page's module description;
 * vLLM API page "rocm_aiter_mla" DCP decode routing: token t of a request on
 * shard t % W, partial outputs merged by LSE).  Shard w computed (out_w, lse_w)
 * over its keys with mla_decode (without sinks).  For each (t, h):
 *   lse = ln sum_w e^(lse_w)            (shards with lse_w = -inf add nothing)
 *   out = sum_w out_w e^(lse_w - lse)
 * then, with sinks (device fp32 [H] or NULL), once for the whole row:
 *   lse' = logaddexp(lse, sink[h]), out' = out e^(lse - lse')
 * A row that no shard saw gets out = 0, lse = -inf (or the sink); a NaN lse_w
 * makes the row NaN.
 *  shard_out: device [W, T, H, 512] of in_dtype (BF16, FP16 or FP32),
 *             contiguous, 16-byte aligned;  shard_lse: device fp32 [W, T, H].
 *  out: device [T, H, 512] of out_dtype;  lse: device fp32 [T, H].
 *  1 <= num_shards <= 64.  One stream-ordered launch, no allocation.
 */
int mla_combine_lse(const void* shard_out, int32_t in_dtype, const float* shard_lse, int32_t num_shards,
                    int32_t num_tokens, int32_t num_heads, const float* sinks, void* out,
                    int32_t out_dtype, float* lse, void* stream);

/*
 * Fused decode: out [T, H, 512] and lse [T, H] in two stream-ordered
 * launches, partial results living in the caller's workspace
 * (>= mla_decode_workspace_bytes(p) bytes, 256-byte aligned; its contents on
 * entry do not matter).  sinks / out / out_dtype / lse as for
 * mla_merge_segments.
 *  - schedule MLA_SCHEDULE_SEGMENTS: the segment partition above with
 *    S = num_segments, or with the planner's S (mla_resolve_num_segments) when
 *    num_segments == 0, then the merge (the results of
 *    mla_decode_segments + mla_merge_segments with that S: bit for bit with
 *    an fp32 output; with a 16-bit output the fused call keeps its partials
 *    in bf16, a rounding of the size of the output's own).
 *  - schedule MLA_SCHEDULE_BALANCED (num_segments must be 0): a balanced
 *    split of the key axis.  The batch's work is
 *    one sequence of units (request, row chunk, tile of TT keys) that is cut
 *    into equal ranges, one per workgroup, so every compute unit streams the
 *    same number of cache rows whatever the lengths.  A (request, row chunk)
 *    inside one range is finished by the first launch; one cut by a range
 *    boundary is merged by the second from per-piece base-2 partials (the
 *    same merge rule as above; bf16 partials for a 16-bit output).  The
 *    result equals the segment schedule's up to floating-point rounding.
 */
int mla_decode(const mla_problem* p, const float* sinks, void* out, int32_t out_dtype, float* lse,
               void* workspace, size_t workspace_bytes, void* stream);

/*
 * One of the two launches of mla_decode, for callers that schedule them
 * separately (e.g. to place other work between them, or to time them):
 * stage 1 streams the cache (and, with num_segments == 0, finishes the rows
 * whose keys fell in one workgroup), stage 2 merges.  Stage 2 must follow
 * stage 1 on the same workspace.  Arguments as for mla_decode.
 */
int mla_decode_stage(const mla_problem* p, const float* sinks, void* out, int32_t out_dtype, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t stage, void* stream);

/*
 * mla_decode without a workspace argument, for callers that cannot allocate
 * device memory (code under graph capture, serving loops that must not call
 * the allocator, harnesses that forbid it).  The partials live in a static
 * device array of MLA_NO_ALLOC_SCRATCH_BYTES that the library holds on every
 * GPU it runs on until the process ends; nothing is allocated or freed.  The
 * caller still passes q, the cache and the outputs.  160 MiB holds the
 * balanced split's partials for any batch on a 256-CU MI355X (at most
 * 32768 rows x 2 pieces x 2056 B, plus 16 B per query token); a segment partition needs
 * T * H * S * 2056 B.  A batch whose mla_decode_workspace_bytes exceeds the
 * scratch size fails with MLA_ERR_WORKSPACE before any launch.  All calls on one GPU share the one
 * array: calls that overlap on a GPU (concurrent streams, threads) race and
 * must be ordered by the caller.  Other arguments as for mla_decode.
 */
#define MLA_NO_ALLOC_SCRATCH_BYTES ((size_t)160 << 20)
int mla_decode_no_alloc(const mla_problem* p, const float* sinks, void* out, int32_t out_dtype, float* lse,
                        void* stream);

/* Workspace mla_decode needs for p.  Returns 0 and sets *bytes, or an error. */
int mla_decode_workspace_bytes(const mla_problem* p, size_t* bytes);

/* The balanced split mla_decode uses for p (schedule MLA_SCHEDULE_BALANCED): workgroups,
 * query rows per workgroup and keys per unit (TT).  Returns 1 and fills the
 * outputs (each may be NULL); 0 when p uses the segment partition instead;
 * or an error. */
int mla_split_plan(const mla_problem* p, int32_t* workgroups, int32_t* rows_per_workgroup,
                   int32_t* unit_keys);

/* The S mla_decode uses for p under MLA_SCHEDULE_SEGMENTS: the planner's S
 * when num_segments == 0 (host only after the first call on a device: reads
 * the CU count once), else p->num_segments.  Returns S >= 1 or an error. */
int mla_resolve_num_segments(const mla_problem* p);

/* Planner (pure host): S so that request x segment work items fill num_cus
 * compute units; clamped to [1, min(MLA_MAX_SEGMENTS, cdiv(max_seq_len, TILE))]. */
int mla_plan_num_segments(int32_t num_reqs, int32_t max_seq_len, int64_t sum_seq_lens,
                          int32_t num_heads, int32_t max_qlen, int32_t tile_size,
                          int32_t kv_dtype, int32_t num_cus);

/* TILE for a block size (min(128, largest power-of-two divisor)); error if < 1. */
int mla_tile_size_for_block(int32_t block_size);

/* Host partition of one request: writes the valid segments' [start, end) into
 * starts/ends (capacity num_segments each, may be NULL) and returns their count. */
int mla_segment_bounds(int32_t seq_len, int32_t num_segments, int32_t tile_size,
                       int32_t* starts, int32_t* ends);

const char* mla_status_string(int status);
const char* mla_last_error(void);
int mla_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MLA_DECODE_H_ */
