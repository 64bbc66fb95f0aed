// Internal interface between the host side (argument checks, planning) and the
// HIP kernels.  Not part of the public ABI.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace mla {

constexpr int kHeadDim = 576;
constexpr int kKvRank = 512;
// Launch shape of the segment kernel per (dtype, waves per workgroup, 16-row
// groups per wave):
//  tt   tokens per LDS tile (bf16 16 except with two waves: 18 KiB tiles,
//       so a ring holds enough of them in flight; fp8 32),
//  ring LDS ring bytes per workgroup,
//  occ  waves per SIMD the kernel's registers are sized for (2 caps a wave
//       at 256 registers; 1 allows 512, which two row groups need).
struct ShapeCfg {
  int tt;
  int ring;
  int occ;
};
constexpr ShapeCfg shape_cfg(bool fp8, int waves, int rg) {
  // One wave: four workgroups per CU, one wave per SIMD, 2-slot ring.
  // Four waves: two workgroups per CU (two waves per SIMD hide each other's
  // LDS and MFMA latency; measured 1.9x faster than one 144 KiB workgroup).
  // Eight waves: one workgroup, two waves per SIMD.
  // Two row groups per wave (the wide fp8 body, 32 rows per wave): one wave
  // per SIMD, rings of 2, 4 or 8 32-token tiles (4, 2 or 1 workgroups per CU).
  return rg == 2 ? (waves == 1 ? ShapeCfg{32, 36864, 1}
                    : waves == 2 ? ShapeCfg{32, 73728, 1} : ShapeCfg{32, 147456, 1})
       : waves == 1 ? ShapeCfg{fp8 ? 32 : 16, 36864, 1}
       : waves == 2 ? ShapeCfg{32, 73728, 1}
       : waves == 4 ? ShapeCfg{fp8 ? 32 : 16, 73728, 2}
                    : ShapeCfg{fp8 ? 32 : 16, 147456, 2};
}
constexpr int tile_tokens(bool fp8, int waves, int rg) { return shape_cfg(fp8, waves, rg).tt; }
// Workgroups one CU holds at once: bound by LDS and by wave slots.
constexpr int wgs_per_cu(bool fp8, int waves, int rg) {
  return (147456 / shape_cfg(fp8, waves, rg).ring) < (4 * shape_cfg(fp8, waves, rg).occ / waves)
             ? (147456 / shape_cfg(fp8, waves, rg).ring)
             : (4 * shape_cfg(fp8, waves, rg).occ / waves);
}

struct SegmentLaunch {
  // query
  const void* q;
  int64_t q_stride_token, q_stride_head;  // elements
  const float* q_scale;                   // nullable
  const void* q_pe;                       // nullable: rope dims in their own tensor
  int64_t q_pe_stride_token, q_pe_stride_head;
  int32_t q_bf16;                         // bf16 q with an fp8 cache: quantise on load
  // cache
  const char* kv;
  int64_t num_blocks;
  int32_t block_size;
  const float* kv_scale;  // nullable
  const int32_t* block_table;
  int64_t bt_stride_row, bt_stride_col;
  int32_t bt_cols;
  const int32_t* bt_indptr;  // nullable: ragged page lists (block_table is then flat)
  const int32_t* seq_lens;
  const int32_t* qo_indptr;  // nullable -> one token per request
  int32_t num_tokens, num_heads, num_reqs, max_qlen;
  int32_t causal, tile, num_segments;
  float softmax_scale;
  // partial outputs: fp32 at seg_out, or, with piece_bf16 (the fused call
  // with a 16-bit output), bf16 at piece_out (the same memory); seg_max /
  // seg_sum in fp32 either way
  float* seg_out;
  unsigned short* piece_out;
  int32_t piece_bf16;
  float* seg_max;
  float* seg_sum;
  // split kernel: finished rows go straight to the output
  void* out;
  int32_t out_dtype;  // 0 bf16, 1 fp16, 2 fp32
  float* lse;
  const float* sinks;     // nullable
  int32_t* unit_offsets;  // [num_reqs + 1]: unit offset of each request, then the total
  int32_t* tok_rec;       // nullable: [T + 1][4] per-token records for the merge, then a flag
};

struct MergeLaunch {
  const float* seg_out;             // fp32 partials
  const unsigned short* piece_out;  // bf16 partials (piece_bf16), the same memory
  int32_t piece_bf16;
  const float* seg_max;
  const float* seg_sum;
  const int32_t* part_lens;  // [T] or NULL -> derive from seq_lens / qo_indptr
  const int32_t* seq_lens;
  const int32_t* qo_indptr;  // nullable
  int32_t num_reqs, max_qlen;
  int32_t num_tokens, num_heads, num_segments, tile;
  const float* sinks;  // nullable
  void* out;
  int32_t out_dtype;
  float* lse;
  // balanced split pieces (unit_offsets != NULL): rows per workgroup, tile
  // tokens and workgroup count of the split kernel that wrote them
  const int32_t* unit_offsets;
  const int32_t* tok_rec;  // nullable: the split kernel's per-token records
  int32_t rows_wg, tt, grid_wgs;
};

struct CombineLaunch {
  const void* shard_out;  // [W, T, H, 512]
  const float* shard_lse; // [W, T, H]
  int32_t in_dtype;       // 0 bf16, 1 fp16, 2 fp32
  int32_t num_shards, num_tokens, num_heads;
  const float* sinks;     // nullable
  void* out;
  int32_t out_dtype;
  float* lse;
};

// Kernel shape chosen by the host for a decode batch.
struct SegmentShape {
  bool fp8;
  int waves;          // waves per workgroup (1, 2, 4 or 8)
  int rows_per_wave;  // 16-row groups per wave (2: the wide fp8 body, one 32-row block)
  int chunks;         // row chunks per (request, segment)
  bool contig;        // TILE >= tile tokens: an LDS tile is one contiguous run of rows
  int ks;             // balanced split: k-split waves per workgroup (1 = none)
};

// Balanced split with one 16-row group: four waves per workgroup share every
// piece tile by tile and combine at its end, one workgroup per CU (the same
// four waves per CU as four one-wave workgroups, a quarter of the pieces).
constexpr int kSplitKs = 4;
constexpr int split_ks(int waves, int rg, bool contig) {
  return (waves == 1 && rg == 1 && contig) ? kSplitKs : 1;
}

SegmentShape segment_shape(bool fp8, int num_heads, int max_qlen, int tile);

// split_wgs > 0: the balanced split kernel on that many workgroups; else the
// segment kernel on (num_segments, num_reqs, chunks).
hipError_t launch_segments(const SegmentLaunch& a, const SegmentShape& sh, int split_wgs, hipStream_t stream);
hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream);
hipError_t launch_combine(const CombineLaunch& a, hipStream_t stream);

// The library's static device scratch (mla_decode_no_alloc): its size, and
// its device address on the current device.
constexpr size_t kScratchBytes = (size_t)160 << 20;
hipError_t scratch_buffer(void** ptr);

}  // namespace mla
