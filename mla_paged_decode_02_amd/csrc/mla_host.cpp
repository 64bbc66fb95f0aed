// Host side of the MLA decode library: argument checks, segment planner,
// workspace layout and the C ABI entry points declared in mla_decode.h.
//
// Nothing here reads device memory or synchronises; every entry point checks
// its arguments completely before the first launch.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include <hip/hip_runtime_api.h>

#include "mla_decode.h"
#include "mla_internal.h"

static_assert(mla::kScratchBytes == MLA_NO_ALLOC_SCRATCH_BYTES, "static scratch size of the header");

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }
int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// [backend page "rocm_aiter_mla.py", _segmented_mla_page_size]: the largest
// power of two dividing the block, capped at 128.
int tile_rule(int block_size) {
  int t = 1;
  while (t < MLA_MAX_TILE && block_size % (2 * t) == 0) t *= 2;
  return t;
}

int resolved_tile(const mla_problem* p) { return p->tile_size ? p->tile_size : tile_rule(p->block_size); }

int elem_bytes(int dtype) { return dtype == MLA_DTYPE_BF16 ? 2 : 1; }

// Compute units of the current device, read once per device.
int device_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

int validate(const mla_problem* p, bool require_segments) {
  if (!p) return fail(MLA_ERR_INVALID_ARG, "problem descriptor is NULL");
  if (p->struct_size < sizeof(mla_problem))
    return fail(MLA_ERR_INVALID_ARG, "struct_size %zu < sizeof(mla_problem) %zu", p->struct_size,
                sizeof(mla_problem));
  if (p->head_dim != MLA_HEAD_DIM) return fail(MLA_ERR_INVALID_ARG, "head_dim must be 576, got %d", p->head_dim);
  if (p->kv_lora_rank != MLA_KV_LORA_RANK)
    return fail(MLA_ERR_INVALID_ARG, "kv_lora_rank must be 512, got %d", p->kv_lora_rank);
  if (p->num_heads < 1) return fail(MLA_ERR_INVALID_ARG, "num_heads must be >= 1, got %d", p->num_heads);
  if (p->num_heads > MLA_MAX_HEADS)
    return fail(MLA_ERR_UNSUPPORTED, "num_heads %d > %d is not supported", p->num_heads, MLA_MAX_HEADS);
  if (p->num_tokens < 0 || p->num_reqs < 0)
    return fail(MLA_ERR_INVALID_ARG, "num_tokens / num_reqs must be >= 0 (got %d, %d)", p->num_tokens, p->num_reqs);
  if (p->q_dtype != MLA_DTYPE_BF16 && p->q_dtype != MLA_DTYPE_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "q dtype %d not supported (bf16 or fp8-e4m3)", p->q_dtype);
  if (p->kv_dtype != MLA_DTYPE_BF16 && p->kv_dtype != MLA_DTYPE_FP8_E4M3)
    return fail(MLA_ERR_UNSUPPORTED, "kv_cache dtype %d not supported (bf16 or fp8-e4m3)", p->kv_dtype);
  if (p->q_dtype != p->kv_dtype && !(p->q_dtype == MLA_DTYPE_BF16 && p->kv_dtype == MLA_DTYPE_FP8_E4M3))
    return fail(MLA_ERR_UNSUPPORTED, "q dtype %d and kv_cache dtype %d must match (or bf16 q with an fp8 cache)",
                p->q_dtype, p->kv_dtype);
  if (p->block_size < 1) return fail(MLA_ERR_INVALID_ARG, "block_size must be >= 1, got %d", p->block_size);
  if (p->num_blocks < 1) return fail(MLA_ERR_INVALID_ARG, "num_blocks must be >= 1");
  if ((int64_t)p->num_blocks * p->block_size >= ((int64_t)1 << 31))
    return fail(MLA_ERR_UNSUPPORTED, "cache holds %lld rows; at most 2^31 - 1 are addressable",
                (long long)((int64_t)p->num_blocks * p->block_size));
  if (p->tile_size != 0) {
    if (!is_pow2(p->tile_size) || p->tile_size > MLA_MAX_TILE || p->block_size % p->tile_size != 0)
      return fail(MLA_ERR_INVALID_ARG,
                  "tile_size %d must be a power of two <= 128 dividing block_size %d", p->tile_size,
                  p->block_size);
  }
  if (p->schedule != MLA_SCHEDULE_SEGMENTS && p->schedule != MLA_SCHEDULE_BALANCED)
    return fail(MLA_ERR_INVALID_ARG, "schedule must be MLA_SCHEDULE_SEGMENTS (0) or MLA_SCHEDULE_BALANCED (1), got %d",
                p->schedule);
  if (require_segments && p->schedule != MLA_SCHEDULE_SEGMENTS)
    return fail(MLA_ERR_INVALID_ARG, "the segment entry points take schedule MLA_SCHEDULE_SEGMENTS (0)");
  if (p->schedule == MLA_SCHEDULE_BALANCED && p->num_segments != 0)
    return fail(MLA_ERR_INVALID_ARG, "schedule MLA_SCHEDULE_BALANCED takes num_segments 0, got %d", p->num_segments);
  if (require_segments ? p->num_segments < 1 : p->num_segments < 0)
    return fail(MLA_ERR_INVALID_ARG, "num_segments must be >= %d, got %d", require_segments ? 1 : 0,
                p->num_segments);
  if (p->num_segments > MLA_MAX_SEGMENTS)
    return fail(MLA_ERR_INVALID_ARG, "num_segments %d > %d", p->num_segments, MLA_MAX_SEGMENTS);
  if (p->max_workgroups < 0)
    return fail(MLA_ERR_INVALID_ARG, "max_workgroups must be >= 0, got %d", p->max_workgroups);
  if (p->max_seq_len < 0) return fail(MLA_ERR_INVALID_ARG, "max_seq_len must be >= 0");
  if (p->qo_indptr == nullptr) {
    if (p->num_tokens != p->num_reqs)
      return fail(MLA_ERR_INVALID_ARG, "without qo_indptr num_tokens (%d) must equal num_reqs (%d)",
                  p->num_tokens, p->num_reqs);
    if (p->num_tokens > 0 && p->max_qlen != 1)
      return fail(MLA_ERR_INVALID_ARG, "without qo_indptr max_qlen must be 1, got %d", p->max_qlen);
  } else if (p->num_tokens > 0 && p->max_qlen < 1) {
    return fail(MLA_ERR_INVALID_ARG, "max_qlen must be >= 1, got %d", p->max_qlen);
  }
  if (p->max_qlen < 0 || (int64_t)p->max_qlen * p->num_heads > 4096)
    return fail(MLA_ERR_UNSUPPORTED, "max_qlen %d x num_heads %d exceeds 4096 query rows per request",
                p->max_qlen, p->num_heads);
  if (!(p->softmax_scale == p->softmax_scale) || p->softmax_scale <= 0.f)
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be a positive number");
  if (p->num_tokens == 0) return MLA_OK;  // nothing will be launched or read

  if (!p->q) return fail(MLA_ERR_INVALID_ARG, "q is NULL");
  if (!p->kv_cache) return fail(MLA_ERR_INVALID_ARG, "kv_cache is NULL");
  if (!p->block_table) return fail(MLA_ERR_INVALID_ARG, "block_table is NULL");
  if (!p->seq_lens) return fail(MLA_ERR_INVALID_ARG, "seq_lens is NULL");
  if (p->num_reqs < 1) return fail(MLA_ERR_INVALID_ARG, "num_reqs must be >= 1 when num_tokens > 0");
  const int eb = elem_bytes(p->q_dtype);
  if (!aligned16(p->q) || !aligned16(p->kv_cache))
    return fail(MLA_ERR_INVALID_ARG, "q and kv_cache must be 16-byte aligned");
  const int q_width = p->q_pe ? MLA_KV_LORA_RANK : MLA_HEAD_DIM;
  if (p->q_stride_head < q_width || p->q_stride_token < 0 || (p->q_stride_head * eb) % 16 != 0 ||
      (p->q_stride_token * eb) % 16 != 0)
    return fail(MLA_ERR_INVALID_ARG,
                "q strides (token %lld, head %lld elements) must be >= 0 / >= %d and multiples of 16 bytes",
                (long long)p->q_stride_token, (long long)p->q_stride_head, q_width);
  if (p->q_pe) {
    if (!aligned16(p->q_pe)) return fail(MLA_ERR_INVALID_ARG, "q_pe must be 16-byte aligned");
    if (p->q_pe_stride_head < MLA_HEAD_DIM - MLA_KV_LORA_RANK || p->q_pe_stride_token < 0 ||
        (p->q_pe_stride_head * eb) % 16 != 0 || (p->q_pe_stride_token * eb) % 16 != 0)
      return fail(MLA_ERR_INVALID_ARG,
                  "q_pe strides (token %lld, head %lld elements) must be >= 0 / >= 64 and multiples of 16 bytes",
                  (long long)p->q_pe_stride_token, (long long)p->q_pe_stride_head);
  }
  if (!p->bt_indptr) {
    if (p->max_blocks_per_req < 1) return fail(MLA_ERR_INVALID_ARG, "max_blocks_per_req must be >= 1");
    if (cdiv64(p->max_seq_len, p->block_size) > p->max_blocks_per_req)
      return fail(MLA_ERR_INVALID_ARG, "max_seq_len %d needs %lld blocks but the table has %d columns",
                  p->max_seq_len, (long long)cdiv64(p->max_seq_len, p->block_size), p->max_blocks_per_req);
    if ((int64_t)p->max_blocks_per_req * p->block_size >= ((int64_t)1 << 31))
      return fail(MLA_ERR_UNSUPPORTED, "block table spans more than 2^31 positions");
  }
  if (p->bt_stride_col < 1 || p->bt_stride_row < 0)
    return fail(MLA_ERR_INVALID_ARG, "block_table strides must be row >= 0, col >= 1");
  return MLA_OK;
}

// Tiles a piece of gathered rows (pages shorter than a tile) holds at least
// (while at least half the slots stay busy): each piece pays a query load, a
// page-window load and its first tile's round trip, and every extra piece is
// one more partial for the merge.  Measured on 52 index streams of 2048 keys
// at 16 heads (128 tiles per request): 10-12 pieces per request beat 19 by
// 9-10% of the step under both schedules; at 128 heads in fp8 (64 tiles) 4
// pieces beat 8.
constexpr int64_t kMinGatherTiles = 12;

int plan_segments(int num_reqs, int max_seq_len, int64_t sum_seq_lens, int num_heads, int max_qlen,
                  int tile, int kv_dtype, int num_cus) {
  if (num_reqs < 1 || max_seq_len < 1) return 1;
  const mla::SegmentShape sh = mla::segment_shape(kv_dtype == MLA_DTYPE_FP8_E4M3, num_heads,
                                                  max_qlen < 1 ? 1 : max_qlen, tile);
  // Workgroups a CU holds at once (the LDS ring decides).
  const int per_cu = mla::wgs_per_cu(sh.fp8, sh.waves, sh.rows_per_wave);
  const int64_t slots = (int64_t)(num_cus > 0 ? num_cus : 256) * per_cu;
  const int64_t total = sum_seq_lens > 0 ? sum_seq_lens : (int64_t)num_reqs * max_seq_len;
  // Segments sized so the longest request's pieces match one slot's share of
  // all keys: uniform batches get floor(slots / (R * chunks)).
  int64_t S = (int64_t)max_seq_len * slots / ((int64_t)sh.chunks * total);
  const int64_t max_useful = cdiv64(max_seq_len, tile);
  if (S > max_useful) S = max_useful;
  if (!sh.contig) {
    // gathered tiles: at least kMinGatherTiles tiles per segment, down to half
    // the slots
    int64_t cap = max_seq_len / ((int64_t)kMinGatherTiles * mla::tile_tokens(sh.fp8, sh.waves, sh.rows_per_wave));
    if (cap < (S + 1) / 2) cap = (S + 1) / 2;
    if (S > cap) S = cap;
  }
  if (S > MLA_MAX_SEGMENTS) S = MLA_MAX_SEGMENTS;
  if (S < 1) S = 1;
  return (int)S;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// Balanced split of the fused decode (MLA_SCHEDULE_BALANCED): the split kernel's
// shape and workgroup count.  grid_wgs == 0 means "use the segment formula"
// (the unit count would not fit 32 bits).
struct SplitPlan {
  mla::SegmentShape sh;
  int rows_wg, tt, grid_wgs;
};

SplitPlan plan_split(const mla_problem* p, int tile) {
  SplitPlan sp;
  const int max_qlen = p->qo_indptr ? p->max_qlen : 1;
  sp.sh = mla::segment_shape(p->kv_dtype == MLA_DTYPE_FP8_E4M3, p->num_heads, max_qlen, tile);
  sp.rows_wg = 16 * sp.sh.waves * sp.sh.rows_per_wave;
  sp.tt = mla::tile_tokens(sp.sh.fp8, sp.sh.waves, sp.sh.rows_per_wave);
  const int64_t chunks = cdiv64((int64_t)max_qlen * p->num_heads, sp.rows_wg);
  const int64_t max_units = (int64_t)p->num_reqs * chunks * cdiv64(p->max_seq_len > 0 ? p->max_seq_len : 1, sp.tt);
  if (max_units >= ((int64_t)1 << 31)) { sp.grid_wgs = 0; return sp; }
  // Units the batch holds at most (exact up to one tile per request when the
  // caller gives the summed lengths).
  const int64_t est = p->sum_seq_lens > 0 ? chunks * (cdiv64(p->sum_seq_lens, sp.tt) + p->num_reqs) : max_units;
  // (k-split waves: one workgroup holds ks waves' rings)
  const int64_t slots =
      (int64_t)device_cus() * mla::wgs_per_cu(sp.sh.fp8, sp.sh.waves, sp.sh.rows_per_wave) / sp.sh.ks;
  int64_t G = slots < est ? slots : est;
  // Gathered tiles: every piece pays its query load, its page window and its
  // first tile's round trip, so pieces keep at least kMinGatherTiles tiles,
  // down to half the slots.
  const int64_t busy = G;  // workgroups the batch could keep busy
  if (!sp.sh.contig) {
    int64_t cap = est / kMinGatherTiles;
    if (cap < slots / 2) cap = slots / 2;
    if (G > cap) G = cap;
  }
  // A batch of equal jobs (every request the same length and query count):
  // k workgroups per (request, row chunk) give every workgroup one piece.  A
  // workgroup that moves to a second piece restarts its stream (the query load
  // and the first tiles' round trips; with gathered tiles also the page
  // window).  For the stream-bound one-row-group shape, and for gathered
  // tiles, that costs more than leaving up to a quarter of the slots idle
  // (measured ~6% of the stream kernel at 52 x 16K, and 22% of the step for
  // 52 index streams of 2048 keys at 128 heads); contiguous shapes with more
  // row groups lean on the CUs' LDS and matrix units and give up at most 1/8.
  const int64_t jobs = (int64_t)p->num_reqs * chunks;
  const bool uniform = p->sum_seq_lens > 0 && p->sum_seq_lens == (int64_t)p->num_reqs * p->max_seq_len &&
                       (int64_t)p->num_tokens == (int64_t)p->num_reqs * max_qlen;
  if (uniform && busy == slots && jobs <= G) {
    const int64_t k = G / jobs;
    const bool loose = sp.sh.ks > 1 || !sp.sh.contig;
    const int64_t num = loose ? 3 : 7, den = loose ? 4 : 8;
    if (den * k * jobs >= num * G) G = k * jobs;
  }
  if (p->max_workgroups > 0 && G > p->max_workgroups) G = p->max_workgroups;
  if (G < 1) G = 1;
  sp.grid_wgs = (int)G;
  return sp;
}

struct SplitWs {
  size_t out_off, max_off, sum_off, off_off, rec_off, total;
};

SplitWs split_ws(const SplitPlan& sp, int num_reqs, int num_tokens) {
  SplitWs w;
  const size_t rows = (size_t)sp.grid_wgs * 2 * sp.rows_wg;
  w.out_off = 0;
  w.max_off = align256(rows * MLA_KV_LORA_RANK * sizeof(float));  // fp32 (or bf16) piece partials
  w.sum_off = w.max_off + align256(rows * sizeof(float));
  w.off_off = w.sum_off + align256(rows * sizeof(float));
  w.rec_off = w.off_off + align256((size_t)(num_reqs + 1) * sizeof(int32_t));
  // per-token records (16 B each) and their flag, used with query ranges
  w.total = w.rec_off + align256(((size_t)num_tokens + 1) * 4 * sizeof(int32_t));
  return w;
}

struct WsLayout {
  size_t out_off, max_off, sum_off, total;
};

WsLayout ws_layout(int T, int H, int S) {
  WsLayout w;
  const size_t rows = (size_t)T * H * S;
  w.out_off = 0;
  w.max_off = align256(rows * MLA_KV_LORA_RANK * sizeof(float));
  w.sum_off = w.max_off + align256(rows * sizeof(float));
  w.total = w.sum_off + align256(rows * sizeof(float));
  return w;
}

mla::SegmentLaunch make_launch(const mla_problem* p, int tile, int S, float* so, float* sm, float* ss) {
  mla::SegmentLaunch a;
  memset(&a, 0, sizeof(a));
  a.q = p->q;
  a.q_stride_token = p->q_stride_token;
  a.q_stride_head = p->q_stride_head;
  a.q_pe = p->q_pe;
  a.q_pe_stride_token = p->q_pe_stride_token;
  a.q_pe_stride_head = p->q_pe_stride_head;
  a.q_bf16 = p->q_dtype == MLA_DTYPE_BF16 && p->kv_dtype == MLA_DTYPE_FP8_E4M3;
  a.q_scale = p->q_scale;
  a.kv = static_cast<const char*>(p->kv_cache);
  a.num_blocks = p->num_blocks;
  a.block_size = p->block_size;
  a.kv_scale = p->kv_scale;
  a.block_table = p->block_table;
  a.bt_stride_row = p->bt_stride_row;
  a.bt_stride_col = p->bt_stride_col;
  a.bt_cols = p->max_blocks_per_req;
  a.bt_indptr = p->bt_indptr;
  a.seq_lens = p->seq_lens;
  a.qo_indptr = p->qo_indptr;
  a.num_tokens = p->num_tokens;
  a.num_heads = p->num_heads;
  a.num_reqs = p->num_reqs;
  a.max_qlen = p->qo_indptr ? p->max_qlen : 1;
  a.causal = p->causal ? 1 : 0;
  a.tile = tile;
  a.num_segments = S;
  a.softmax_scale = p->softmax_scale;
  a.seg_out = so;
  a.seg_max = sm;
  a.seg_sum = ss;
  return a;
}

int out_code(int out_dtype) {
  switch (out_dtype) {
    case MLA_DTYPE_BF16: return 0;
    case MLA_DTYPE_FP16: return 1;
    case MLA_DTYPE_FP32: return 2;
    default: return -1;
  }
}

int hip_fail(hipError_t e, const char* what) {
  return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int mla_version(void) { return 1; }

const char* mla_status_string(int status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    default: return "MLA_ERR_UNKNOWN";
  }
}

const char* mla_last_error(void) { return g_last_error.c_str(); }

int mla_tile_size_for_block(int32_t block_size) {
  if (block_size < 1) return fail(MLA_ERR_INVALID_ARG, "block_size must be >= 1, got %d", block_size);
  return tile_rule(block_size);
}

int mla_segment_bounds(int32_t seq_len, int32_t num_segments, int32_t tile_size, int32_t* starts,
                       int32_t* ends) {
  if (num_segments < 1 || tile_size < 1)
    return fail(MLA_ERR_INVALID_ARG, "num_segments and tile_size must be >= 1");
  if (seq_len <= 0) return 0;
  // [merge page, module description]: tiles_per_segment = cdiv(seq_len, S * TILE).
  const int64_t span = cdiv64(seq_len, (int64_t)num_segments * tile_size) * tile_size;
  int count = 0;
  for (int s = 0; s < num_segments; ++s) {
    const int64_t a = (int64_t)s * span;
    if (a >= seq_len) break;
    if (starts) starts[count] = (int32_t)a;
    if (ends) ends[count] = (int32_t)(a + span < seq_len ? a + span : seq_len);
    ++count;
  }
  return count;
}

int mla_plan_num_segments(int32_t num_reqs, int32_t max_seq_len, int64_t sum_seq_lens, int32_t num_heads,
                          int32_t max_qlen, int32_t tile_size, int32_t kv_dtype, int32_t num_cus) {
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS) return fail(MLA_ERR_INVALID_ARG, "num_heads out of range");
  if (tile_size < 1 || !is_pow2(tile_size) || tile_size > MLA_MAX_TILE)
    return fail(MLA_ERR_INVALID_ARG, "tile_size must be a power of two in [1, 128]");
  return plan_segments(num_reqs, max_seq_len, sum_seq_lens, num_heads, max_qlen, tile_size, kv_dtype, num_cus);
}

int mla_validate(const mla_problem* p, int require_segments) { return validate(p, require_segments != 0); }

int mla_resolve_num_segments(const mla_problem* p) {
  int st = validate(p, false);
  if (st != MLA_OK) return st;
  if (p->num_segments > 0) return p->num_segments;
  return plan_segments(p->num_reqs, p->max_seq_len, p->sum_seq_lens, p->num_heads,
                       p->qo_indptr ? p->max_qlen : 1, resolved_tile(p), p->kv_dtype, device_cus());
}

int mla_decode_workspace_bytes(const mla_problem* p, size_t* bytes) {
  if (!bytes) return fail(MLA_ERR_INVALID_ARG, "bytes is NULL");
  const int st = validate(p, false);
  if (st != MLA_OK) return st;
  if (p->schedule == MLA_SCHEDULE_BALANCED) {
    const SplitPlan sp = plan_split(p, resolved_tile(p));
    if (sp.grid_wgs > 0) {
      *bytes = split_ws(sp, p->num_reqs, p->num_tokens).total;
      return MLA_OK;
    }
  }
  const int S = mla_resolve_num_segments(p);
  if (S < 0) return S;
  *bytes = ws_layout(p->num_tokens, p->num_heads, S).total;
  return MLA_OK;
}

int mla_split_plan(const mla_problem* p, int32_t* workgroups, int32_t* rows_per_workgroup,
                   int32_t* unit_keys) {
  const int st = validate(p, false);
  if (st != MLA_OK) return st;
  if (p->schedule != MLA_SCHEDULE_BALANCED) return 0;
  const SplitPlan sp = plan_split(p, resolved_tile(p));
  if (sp.grid_wgs <= 0) return 0;
  if (workgroups) *workgroups = sp.grid_wgs;
  if (rows_per_workgroup) *rows_per_workgroup = sp.rows_wg;
  if (unit_keys) *unit_keys = sp.tt;
  return 1;
}

int mla_decode_segments(const mla_problem* p, float* segm_output, float* segm_max, float* segm_expsum,
                        void* stream) {
  int st = validate(p, true);
  if (st != MLA_OK) return st;
  if (p->num_tokens == 0) return MLA_OK;
  if (!segm_output || !segm_max || !segm_expsum)
    return fail(MLA_ERR_INVALID_ARG, "segment output buffers must not be NULL");
  if (!aligned16(segm_output)) return fail(MLA_ERR_INVALID_ARG, "segm_output must be 16-byte aligned");
  const int tile = resolved_tile(p);
  mla::SegmentLaunch a = make_launch(p, tile, p->num_segments, segm_output, segm_max, segm_expsum);
  const mla::SegmentShape sh =
      mla::segment_shape(p->kv_dtype == MLA_DTYPE_FP8_E4M3, p->num_heads, a.max_qlen, tile);
  hipError_t e = mla::launch_segments(a, sh, 0, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "segment kernel launch");
  return MLA_OK;
}

int mla_merge_segments(const float* segm_output, const float* segm_max, const float* segm_expsum,
                       const int32_t* part_lens, int32_t num_tokens, int32_t num_heads, int32_t num_segments,
                       int32_t kv_lora_rank, int32_t tile_size, const float* sinks, void* out,
                       int32_t out_dtype, float* lse, void* stream) {
  if (num_tokens < 0) return fail(MLA_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS)
    return fail(num_heads < 1 ? MLA_ERR_INVALID_ARG : MLA_ERR_UNSUPPORTED, "num_heads %d out of [1, 128]",
                num_heads);
  if (num_segments < 1 || num_segments > MLA_MAX_SEGMENTS)
    return fail(MLA_ERR_INVALID_ARG, "num_segments %d out of [1, %d]", num_segments, MLA_MAX_SEGMENTS);
  if (kv_lora_rank != MLA_KV_LORA_RANK) return fail(MLA_ERR_INVALID_ARG, "kv_lora_rank must be 512");
  if (tile_size < 1 || !is_pow2(tile_size) || tile_size > MLA_MAX_TILE)
    return fail(MLA_ERR_INVALID_ARG, "tile_size %d must be a power of two in [1, 128]", tile_size);
  const int oc = out_code(out_dtype);
  if (oc < 0) return fail(MLA_ERR_UNSUPPORTED, "out_dtype %d not supported (bf16, fp16, fp32)", out_dtype);
  if (num_tokens == 0) return MLA_OK;
  if (!segm_output || !segm_max || !segm_expsum || !part_lens || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "merge buffers must not be NULL");
  if (!aligned16(segm_output) || !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "segm_output and out must be 16-byte aligned");
  mla::MergeLaunch m;
  memset(&m, 0, sizeof(m));
  m.seg_out = segm_output;
  m.seg_max = segm_max;
  m.seg_sum = segm_expsum;
  m.part_lens = part_lens;
  m.num_tokens = num_tokens;
  m.num_heads = num_heads;
  m.num_segments = num_segments;
  m.tile = tile_size;
  m.sinks = sinks;
  m.out = out;
  m.out_dtype = oc;
  m.lse = lse;
  hipError_t e = mla::launch_merge(m, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  return MLA_OK;
}

int mla_combine_lse(const void* shard_out, int32_t in_dtype, const float* shard_lse, int32_t num_shards,
                    int32_t num_tokens, int32_t num_heads, const float* sinks, void* out, int32_t out_dtype,
                    float* lse, void* stream) {
  if (num_shards < 1 || num_shards > 64) return fail(MLA_ERR_INVALID_ARG, "num_shards %d out of [1, 64]", num_shards);
  if (num_tokens < 0) return fail(MLA_ERR_INVALID_ARG, "num_tokens must be >= 0");
  if (num_heads < 1 || num_heads > MLA_MAX_HEADS)
    return fail(num_heads < 1 ? MLA_ERR_INVALID_ARG : MLA_ERR_UNSUPPORTED, "num_heads %d out of [1, 128]",
                num_heads);
  const int ic = out_code(in_dtype), oc = out_code(out_dtype);
  if (ic < 0) return fail(MLA_ERR_UNSUPPORTED, "in_dtype %d not supported (bf16, fp16, fp32)", in_dtype);
  if (oc < 0) return fail(MLA_ERR_UNSUPPORTED, "out_dtype %d not supported (bf16, fp16, fp32)", out_dtype);
  if (num_tokens == 0) return MLA_OK;
  if (!shard_out || !shard_lse || !out || !lse) return fail(MLA_ERR_INVALID_ARG, "combine buffers must not be NULL");
  if (!aligned16(shard_out) || !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "shard_out and out must be 16-byte aligned");
  mla::CombineLaunch c;
  memset(&c, 0, sizeof(c));
  c.shard_out = shard_out;
  c.shard_lse = shard_lse;
  c.in_dtype = ic;
  c.num_shards = num_shards;
  c.num_tokens = num_tokens;
  c.num_heads = num_heads;
  c.sinks = sinks;
  c.out = out;
  c.out_dtype = oc;
  c.lse = lse;
  hipError_t e = mla::launch_combine(c, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "combine kernel launch");
  return MLA_OK;
}

namespace {

// Both stages of the fused decode; stage 1 = the key stream, stage 2 = the
// merge, 3 = both.
int decode_stages(const mla_problem* p, const float* sinks, void* out, int32_t out_dtype, float* lse,
                  void* workspace, size_t workspace_bytes, int stages, void* stream) {
  int st = validate(p, false);
  if (st != MLA_OK) return st;
  const int oc = out_code(out_dtype);
  if (oc < 0) return fail(MLA_ERR_UNSUPPORTED, "out_dtype %d not supported (bf16, fp16, fp32)", out_dtype);
  if (stages < 1 || stages > 3) return fail(MLA_ERR_INVALID_ARG, "stages must be 1, 2 or 3, got %d", stages);
  if (p->num_tokens == 0) return MLA_OK;
  if (!out || !lse) return fail(MLA_ERR_INVALID_ARG, "out and lse must not be NULL");
  if (!aligned16(out)) return fail(MLA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  const int tile = resolved_tile(p);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
    return fail(MLA_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);

  if (p->schedule == MLA_SCHEDULE_BALANCED) {
    const SplitPlan sp = plan_split(p, tile);
    if (sp.grid_wgs > 0) {
      const SplitWs w = split_ws(sp, p->num_reqs, p->num_tokens);
      if (!workspace || workspace_bytes < w.total)
        return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                    workspace ? workspace_bytes : (size_t)0);
      // piece partials: fp32 for fp32 outputs, else bf16 in the same region
      float* so = reinterpret_cast<float*>(ws + w.out_off);
      uint16_t* po = reinterpret_cast<uint16_t*>(ws + w.out_off);
      float* sm = reinterpret_cast<float*>(ws + w.max_off);
      float* ss = reinterpret_cast<float*>(ws + w.sum_off);
      int32_t* offs = reinterpret_cast<int32_t*>(ws + w.off_off);
      int32_t* recs = p->qo_indptr ? reinterpret_cast<int32_t*>(ws + w.rec_off) : nullptr;
      if (stages & 1) {
        mla::SegmentLaunch a = make_launch(p, tile, 1, so, sm, ss);
        a.piece_out = po;
        a.piece_bf16 = oc != 2;
        a.out = out;
        a.out_dtype = oc;
        a.lse = lse;
        a.sinks = sinks;
        a.unit_offsets = offs;
        a.tok_rec = recs;
        hipError_t e = mla::launch_segments(a, sp.sh, sp.grid_wgs, hs);
        if (e != hipSuccess) return hip_fail(e, "split kernel launch");
      }
      if (stages & 2) {
        mla::MergeLaunch m;
        memset(&m, 0, sizeof(m));
        m.seg_out = so;
        m.piece_out = po;
        m.piece_bf16 = oc != 2;
        m.seg_max = sm;
        m.seg_sum = ss;
        m.seq_lens = p->seq_lens;
        m.qo_indptr = p->qo_indptr;
        m.num_reqs = p->num_reqs;
        m.max_qlen = p->qo_indptr ? p->max_qlen : 1;
        m.num_tokens = p->num_tokens;
        m.num_heads = p->num_heads;
        m.num_segments = 1;
        m.tile = tile;
        m.sinks = sinks;
        m.out = out;
        m.out_dtype = oc;
        m.lse = lse;
        m.unit_offsets = offs;
        m.tok_rec = recs;
        m.rows_wg = sp.rows_wg;
        m.tt = sp.tt;
        m.grid_wgs = sp.grid_wgs;
        hipError_t e = mla::launch_merge(m, hs);
        if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
      }
      return MLA_OK;
    }
  }

  const int S = mla_resolve_num_segments(p);
  if (S < 0) return S;
  const WsLayout w = ws_layout(p->num_tokens, p->num_heads, S);
  if (!workspace || workspace_bytes < w.total)
    return fail(MLA_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", w.total,
                workspace ? workspace_bytes : (size_t)0);
  float* so = reinterpret_cast<float*>(ws + w.out_off);
  float* sm = reinterpret_cast<float*>(ws + w.max_off);
  float* ss = reinterpret_cast<float*>(ws + w.sum_off);
  // the fused call's partials: bf16 for a 16-bit output, else fp32
  const bool piece_bf16 = oc != 2;
  if (stages & 1) {
    mla::SegmentLaunch a = make_launch(p, tile, S, so, sm, ss);
    a.piece_out = reinterpret_cast<uint16_t*>(so);
    a.piece_bf16 = piece_bf16;
    const mla::SegmentShape sh =
        mla::segment_shape(p->kv_dtype == MLA_DTYPE_FP8_E4M3, p->num_heads, a.max_qlen, tile);
    hipError_t e = mla::launch_segments(a, sh, 0, hs);
    if (e != hipSuccess) return hip_fail(e, "segment kernel launch");
  }
  if (stages & 2) {
    mla::MergeLaunch m;
    memset(&m, 0, sizeof(m));
    m.seg_out = so;
    m.piece_out = reinterpret_cast<const uint16_t*>(so);
    m.piece_bf16 = piece_bf16;
    m.seg_max = sm;
    m.seg_sum = ss;
    m.part_lens = nullptr;
    m.seq_lens = p->seq_lens;
    m.qo_indptr = p->qo_indptr;
    m.num_reqs = p->num_reqs;
    m.max_qlen = p->qo_indptr ? p->max_qlen : 1;
    m.num_tokens = p->num_tokens;
    m.num_heads = p->num_heads;
    m.num_segments = S;
    m.tile = tile;
    m.sinks = sinks;
    m.out = out;
    m.out_dtype = oc;
    m.lse = lse;
    hipError_t e = mla::launch_merge(m, hs);
    if (e != hipSuccess) return hip_fail(e, "merge kernel launch");
  }
  return MLA_OK;
}

}  // namespace

int mla_decode(const mla_problem* p, const float* sinks, void* out, int32_t out_dtype, float* lse,
               void* workspace, size_t workspace_bytes, void* stream) {
  return decode_stages(p, sinks, out, out_dtype, lse, workspace, workspace_bytes, 3, stream);
}

int mla_decode_no_alloc(const mla_problem* p, const float* sinks, void* out, int32_t out_dtype, float* lse,
                        void* stream) {
  size_t need = 0;
  int st = mla_decode_workspace_bytes(p, &need);
  if (st != MLA_OK) return st;
  if (need > mla::kScratchBytes)
    return fail(MLA_ERR_WORKSPACE, "mla_decode_no_alloc: the batch needs %zu bytes of scratch; the static scratch holds %zu",
                need, mla::kScratchBytes);
  if (p->num_tokens == 0) return decode_stages(p, sinks, out, out_dtype, lse, nullptr, 0, 3, stream);
  void* ws = nullptr;
  hipError_t e = mla::scratch_buffer(&ws);
  if (e != hipSuccess) return hip_fail(e, "static scratch address");
  return decode_stages(p, sinks, out, out_dtype, lse, ws, mla::kScratchBytes, 3, stream);
}

int mla_decode_stage(const mla_problem* p, const float* sinks, void* out, int32_t out_dtype, float* lse,
                     void* workspace, size_t workspace_bytes, int32_t stage, void* stream) {
  if (stage != 1 && stage != 2) return fail(MLA_ERR_INVALID_ARG, "stage must be 1 or 2, got %d", stage);
  return decode_stages(p, sinks, out, out_dtype, lse, workspace, workspace_bytes, stage, stream);
}

}  // extern "C"
