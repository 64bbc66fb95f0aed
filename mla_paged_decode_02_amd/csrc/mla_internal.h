// Internal interface between the host side (argument checks, planning) and the
// HIP kernels.  Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace mla {

constexpr int kHeadDim = 576;
constexpr int kKvRank = 512;
// Tokens per LDS tile of the segment kernel: 16 for bf16 with one wave per
// workgroup (so four workgroups share a CU's LDS), else 32.
constexpr int tile_tokens(bool fp8, int waves) { return (!fp8 && waves == 1) ? 16 : 32; }
// LDS ring bytes per workgroup for a given wave count.
constexpr int ring_bytes(int waves) { return waves == 1 ? 36864 : waves == 2 ? 73728 : 147456; }
// Workgroups of that size one CU holds at once (LDS-bound).
constexpr int wgs_per_cu(int waves) { return 147456 / ring_bytes(waves); }

struct SegmentLaunch {
  // query
  const void* q;
  int64_t q_stride_token, q_stride_head;  // elements
  const float* q_scale;                   // nullable
  // cache
  const char* kv;
  int64_t num_blocks;
  int32_t block_size;
  const float* kv_scale;  // nullable
  const int32_t* block_table;
  int64_t bt_stride_row, bt_stride_col;
  int32_t bt_cols;
  const int32_t* seq_lens;
  const int32_t* qo_indptr;  // nullable -> one token per request
  int32_t num_tokens, num_heads, num_reqs, max_qlen;
  int32_t causal, tile, num_segments;
  float softmax_scale;
  // outputs
  float* seg_out;
  float* seg_max;
  float* seg_sum;
};

struct MergeLaunch {
  const float* seg_out;
  const float* seg_max;
  const float* seg_sum;
  const int32_t* part_lens;  // [T] or NULL -> derive from seq_lens / qo_indptr
  const int32_t* seq_lens;
  const int32_t* qo_indptr;  // nullable
  int32_t num_reqs;
  int32_t num_tokens, num_heads, num_segments, tile;
  const float* sinks;  // nullable
  void* out;
  int32_t out_dtype;
  float* lse;
};

// Kernel shape chosen by the host for a decode batch.
struct SegmentShape {
  bool fp8;
  int waves;          // waves per workgroup (1..4)
  int rows_per_wave;  // 16-row groups per wave (1 or 2)
  int chunks;         // row chunks per (request, segment)
  bool contig;        // TILE >= tile tokens: an LDS tile is one contiguous run of rows
};

SegmentShape segment_shape(bool fp8, int num_heads, int max_qlen, int tile);

hipError_t launch_segments(const SegmentLaunch& a, const SegmentShape& sh, hipStream_t stream);
hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream);

}  // namespace mla
