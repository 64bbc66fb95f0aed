// HIP kernels for MLA paged decode on gfx950 (MI355X).
//
// Segment kernel: one workgroup per (request, segment, row chunk).  A row is
// one (query token, head) pair of the request; a wave owns 16 rows.  All waves
// of a workgroup stream the segment's 576-wide cache rows HBM -> LDS once,
// 32 tokens per tile, through direct global->LDS loads into a ring of tiles,
// and every wave computes its rows against each tile:
//
//   S^T[token, row] = K . Q^T    MFMA 16x16x32 (bf16, or fp8 x fp8)
//   base-2 online softmax        exp2, max over the tile via lane shuffles
//   O^T[dim, row]  += V^T . P^T  MFMA 16x16x32 bf16; V^T comes straight from
//                                the row-major tile with the LDS transpose
//                                reads (ds_read_b64_tr_b16 / _tr_b8)
//
// The same tile bytes serve as K (all 576 dims) and V (the first 512), as the
// AITER MLA backend's segmented call does (source page "rocm_aiter_mla.py",
// _forward_segmented_dcp_verify: one [blocks, page, 576] cache view, latent
// rank 512 + rope 64).  No head count is folded into 16-head pseudo-batches:
// every row of a request reads the tile from LDS, so the cache bytes of a
// request leave HBM once per segment regardless of the head count.
//
// Partials are base 2 and unnormalised; the merge kernel turns them into the
// output and a natural-log LSE (vLLM API page
// "vllm.v1.attention.ops.rocm_aiter_mla_merge", merge_mla_segments_triton)
// and folds in optional per-head sinks (vLLM API page
// "vllm.v1.attention.backends.mla.rocm_aiter_mla_sparse", _forward_mla).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>
#include <utility>
#include <vector>

#include "mla_internal.h"

namespace mla {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Buffer resource word 3 for raw (untyped) buffer accesses on gfx9-family parts.
constexpr int kBufferFlags = 0x00020000;
// The cache-row stream loads are non-temporal ("nt": each row is read once per
// piece), which measured ~10% faster than the default policy.
// The softmax reference max moves only past kLazy base-2 units, and p is
// taken relative to (reference - kBias), so p <= 2^(kLazy + kBias) = 2^8.
// bf16 P keeps fp32's range (lazy 8, no bias).  fp8 P is rounded to e4m3,
// whose smallest step is 2^-9: lazy 6 and a bias of 2 keep p <= 256 < 448
// while weights down to 2^-12 of the reference stay representable (host
// simulation on N(0,1) data: under 1% of tiles rescale).
template <bool FP8>
struct Lazy {
  static constexpr float kLazy = FP8 ? 6.0f : 8.0f;
  static constexpr float kBias = FP8 ? 2.0f : 0.0f;
};

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Wait until at most `ahead` tiles of this wave's DMA loads are in flight.
template <int PER_TILE, int MAX_AHEAD>
__device__ __forceinline__ void wait_tiles(int ahead) {
  if constexpr (MAX_AHEAD >= 6) { if (ahead >= 6) { wait_vmcnt<(6 * PER_TILE < 63 ? 6 * PER_TILE : 63)>(); return; } }
  if constexpr (MAX_AHEAD >= 5) { if (ahead == 5) { wait_vmcnt<(5 * PER_TILE < 63 ? 5 * PER_TILE : 63)>(); return; } }
  if constexpr (MAX_AHEAD >= 4) { if (ahead == 4) { wait_vmcnt<(4 * PER_TILE < 63 ? 4 * PER_TILE : 63)>(); return; } }
  if constexpr (MAX_AHEAD >= 3) { if (ahead == 3) { wait_vmcnt<(3 * PER_TILE < 63 ? 3 * PER_TILE : 63)>(); return; } }
  if constexpr (MAX_AHEAD >= 2) { if (ahead == 2) { wait_vmcnt<(2 * PER_TILE < 63 ? 2 * PER_TILE : 63)>(); return; } }
  if constexpr (MAX_AHEAD >= 1) { if (ahead == 1) { wait_vmcnt<(PER_TILE < 63 ? PER_TILE : 63)>(); return; } }
  wait_vmcnt<0>();
}

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Byte address in LDS of a __shared__ object (what M0 takes for LDS DMA).
__device__ __forceinline__ unsigned lds_address(const void* shared_ptr) {
  return (unsigned)(uintptr_t)(const LDS_AS void*)shared_ptr;
}

// Buffer resource (V#) over `bytes` bytes at `base`, no stride, raw access.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(a >> 32) & 0xffffu));
  r[2] = __builtin_amdgcn_readfirstlane(bytes);
  r[3] = kBufferFlags;
  return r;
}

// One 16-byte-per-lane load from a buffer straight into LDS (64 lanes fill
// 1 KiB at lds_addr), non-temporal.  Written as inline assembly on purpose:
// the kernels track these loads themselves with explicit vmcnt waits on the
// ring slot they read, and the compiler, which cannot tell ring slots apart,
// would otherwise make every LDS read and barrier wait for all of them.
// M0 is set here for every load; kernels that use this have no other M0 user.
__device__ __forceinline__ void dma_lds16(i32x4 rsrc, unsigned lds_addr, int voff, int soff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, %3 offen nt lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc),
        "s"(__builtin_amdgcn_readfirstlane(soff))
      : "memory", "m0");
}

// One 4-byte-per-lane load from a buffer straight into LDS (64 lanes fill
// 256 B at lds_addr).  Tracked by the kernels' own vmcnt waits, like dma_lds16.
__device__ __forceinline__ void dma_lds4(i32x4 rsrc, unsigned lds_addr, int voff) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dword %1, %2, %3 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc),
        "s"(__builtin_amdgcn_readfirstlane(0))
      : "memory", "m0");
}

// One 16-byte-per-lane load from a 64-bit address per lane straight into LDS
// (64 lanes fill 1 KiB at lds_addr): the gather path's row loads, which may
// lie anywhere in the cache.  Tracked by the kernels' own vmcnt waits.
__device__ __forceinline__ void dma_lds16_gather(unsigned lds_addr, const void* src) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "global_load_lds_dwordx4 %1, off"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(src)
      : "memory", "m0");
}

// Page-table entries a gathering workgroup keeps in LDS at a time.
constexpr int kIdxCap = 256;

// LDS tile layout (32 tokens).  The 512 latent dims (also V) and the 64 rope
// dims of a row live in two regions so that one DMA instruction (64 lanes x
// 16 B) covers whole rows:
//   bf16: V region 32 x 1024 B, rope region 32 x 128 B at +32 KiB
//   fp8 : V region 32 x  512 B, rope region 32 x  64 B at +16 KiB
// 16-byte chunks are XOR-swizzled per row.  In the V region chunk c of row r
// sits at c ^ swz_v(r), chosen so that the K reads (16 rows per 16-lane pass),
// the 16-bit transpose reads (8 rows x 2 chunks) and the 8-bit transpose reads
// (16 rows) meet no LDS bank conflict.  fp8 (512 B rows): (((r & 7) << 1) |
// bit 3 of r), flipped in bit 0 for the second 16-row block.  bf16 (1024 B
// rows): ((r & 7) << 1), flipped in bit 0 for the second block; rows r and
// r + 8 share a chunk position there, which the LDS serves without conflict
// (rows 8 KiB apart), while the fp8 pattern costs a second cycle per read at
// this pitch (both measured with the LDS bank-conflict counter on gfx950).
// Rope chunks use swz_r(r) = (r >> 1) & 7 (bf16) or (r >> 2) & 3 (fp8),
// distinct within each group of rows one read touches.
template <bool FP8>
struct KvFmt;
template <>
struct KvFmt<false> {  // bf16
  static constexpr int kRowBytes = 1152;   // in the cache
  static constexpr int kVPitch = 1024;     // LDS V region row pitch
  static constexpr int kRopePitch = 128;   // LDS rope region row pitch
  static constexpr int kVChunks = 64;
  static constexpr int kRopeChunks = 8;
  __device__ static int swz_r(int r) { return (r >> 1) & 7; }
  __device__ static int swz_v(int r) { return ((r & 7) << 1) ^ ((r >> 4) & 1); }
};
template <>
struct KvFmt<true> {  // fp8
  static constexpr int kRowBytes = 576;
  static constexpr int kVPitch = 512;
  static constexpr int kRopePitch = 64;
  static constexpr int kVChunks = 32;
  static constexpr int kRopeChunks = 4;
  __device__ static int swz_r(int r) { return (r >> 2) & 3; }
  __device__ static int swz_v(int r) { return ((((r & 7) << 1) | ((r >> 3) & 1)) ^ ((r >> 4) & 1)); }
};

// Max over the four 16-lane rows of a wave (lanes n, n + 16, n + 32, n + 48).
// gfx950's lane swaps run on the VALU: v_permlane32_swap pairs lanes l and
// l ^ 32, v_permlane16_swap pairs lanes l and l ^ 16 (with both operands the
// same value, the two results are the value and its partner's), so the
// reduction needs no LDS round trip.
__device__ __forceinline__ float wave_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ bf16x8 to_bf16x8(const float (&p)[8]) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (__bf16)p[i];
  return r;
}

// 8 fp8-e4m3 codes (two dwords) -> 8 bf16 values (exact: e4m3 fits in bf16).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 v) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

// ---------------------------------------------------------------------------
// Segment kernel
// ---------------------------------------------------------------------------
// Hides a value from the optimiser for one use site: offsets derived from it
// are recomputed where needed instead of being hoisted out of the tile loop
// into dozens of long-lived registers.
__device__ __forceinline__ int opaque(int v) {
  asm volatile("" : "+v"(v));
  return v;
}

template <typename T>
__device__ __forceinline__ T lds_load(const char* base, int off) {
  return *(const LDS_AS T*)(base + off);
}

// One piece of work for a workgroup: the query rows [row0, row0 + rows per
// workgroup) of request r (rows are (token, head) pairs, token-major) against
// the request's key positions [seg_start, seg_end).
struct Piece {
  int r, t0, qlen, L;
  int row0;
  int seg_start, seg_end;
  int mode;        // kOutSegment, kOutFinal or kOutSplit
  int s;           // segment index (kOutSegment)
  int64_t prow0;   // first partial row of the piece (kOutSplit)
  int phase;       // k-split waves: the wave that takes the piece's first tile
};

// Where request r's pages start in the block table, and how many positions
// they cover: row r of the 2-D table, or (ragged lists) the flat range
// [bt_indptr[r], bt_indptr[r+1]).  Uniform loads of read-only data.
__device__ __forceinline__ void page_list(const SegmentLaunch& p, int r, int64_t* base, int* cap) {
  if (p.bt_indptr) {
    const __attribute__((address_space(4))) int* ip = (const __attribute__((address_space(4))) int*)p.bt_indptr;
    const int a = ip[r], b = ip[r + 1];
    *base = (int64_t)a * p.bt_stride_col;
    const int64_t c = (int64_t)(b - a) * p.block_size;
    *cap = c < 0 ? 0 : (c > 0x7fffffff ? 0x7fffffff : (int)c);
  } else {
    *base = (int64_t)r * p.bt_stride_row;
    *cap = p.bt_cols * p.block_size;
  }
}
// Where a piece's result goes:
//  segment: base-2 partials of segment s at [t, h, s] of the segment buffers;
//  final:   the piece is a whole (request, row chunk): normalised output and
//           natural-log LSE (sinks folded in) written directly;
//  split:   base-2 partials at rows prow0 + local row of the split buffers.
constexpr int kOutSegment = 0, kOutFinal = 1, kOutSplit = 2;

template <bool FP8, int TT>
struct TileGeom {
  using F = KvFmt<FP8>;
  static constexpr int kTileBytes = TT * F::kRowBytes;  // bf16 36864 / 18432, fp8 18432
};

__device__ __forceinline__ float logaddexp_f(float a, float b) {
  const float mx = fmaxf(a, b);
  return (mx == -INFINITY) ? -INFINITY : mx + log1pf(expf(-fabsf(a - b)));
}

__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;  // NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (unsigned short)(u >> 16);
}

// Streams one piece through the LDS ring and writes its result.  NW waves x
// RG row groups of 16 rows per workgroup; TT tokens per LDS tile (16 or 32;
// fp8 always uses 32); OCC waves per SIMD the register allocation must allow
// (2 caps a wave at 256 registers).  Every wave of the workgroup calls it with
// the same piece (it holds workgroup barriers).
template <bool FP8, int NW, int RG, int NBUF, bool CONTIG, int TT, int OCC, int KS = 1, bool QB = false>
__device__ __forceinline__ void run_piece(const SegmentLaunch& p,
                                          char (*lds)[TileGeom<FP8, TT>::kTileBytes], unsigned lds_u32,
                                          int* idx_buf, const Piece& pc) {
  using F = KvFmt<FP8>;
  static_assert(TT == 32 || (TT == 16 && !FP8), "tile shape");
  constexpr int kNB = TT / 16;                         // 16-token blocks per tile
  constexpr int kRowBytes = F::kRowBytes;
  constexpr int kVRegion = TT * F::kVPitch;
  constexpr int kTileBytes = TT * kRowBytes;
  constexpr int kRowsPerV = 1024 / F::kVPitch;         // rows per V-region DMA instruction
  constexpr int kNIV = TT / kRowsPerV;                 // V-region DMA instructions
  constexpr int kNI = kTileBytes / 1024;               // all DMA instructions per tile
  constexpr int kNIw = kNIV / NW + (kNI - kNIV) / NW;   // per wave, lower bound
  constexpr int kRowsWG = 16 * RG * NW;
  static_assert(kTileBytes % 1024 == 0, "tile must be whole DMA instructions");

  const int lane = threadIdx.x & 63;
  // k-split waves (KS > 1) all take the one row group: their wave index
  // (kw below) picks tiles, not rows.
  const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wave
  const int rgw = wave;                                              // this wave's row group
  const int g = lane >> 4;
  const int n = lane & 15;

  const int r = pc.r, t0 = pc.t0, qlen = pc.qlen, L = pc.L;
  const int H = p.num_heads;
  const int M = qlen * H;
  const int row0 = pc.row0;
  // A length past the block table is reported as NaN; rows beyond the table
  // are never read.
  int64_t bt_base;
  int cap;
  page_list(p, r, &bt_base, &cap);
  bt_base = __builtin_amdgcn_readfirstlane((int)(bt_base & 0xffffffff)) |
            ((int64_t)__builtin_amdgcn_readfirstlane((int)(bt_base >> 32)) << 32);
  cap = __builtin_amdgcn_readfirstlane(cap);
  bool bad = L > cap;
  const int seg_start = pc.seg_start;
  const int seg_end = pc.seg_end;

  // The workgroup's last row decides how far its rows can see.
  const int last_row = min(row0 + kRowsWG, M) - 1;
  const int lim_wg = p.causal ? (L - qlen + last_row / H + 1) : L;
  const int eff_end = min(min(seg_end, lim_wg), cap);
  const int ntiles = eff_end > seg_start ? cdiv(eff_end - seg_start, TT) : 0;

  // ---- this lane's query rows (one per row group) ----
  int ti[RG], hh[RG], end_row[RG];
  bool rok[RG];
#pragma unroll
  for (int q = 0; q < RG; ++q) {
    const int row = row0 + (rgw * RG + q) * 16 + n;
    rok[q] = row < M;
    ti[q] = rok[q] ? row / H : 0;
    hh[q] = rok[q] ? row - ti[q] * H : 0;
    const int lim = rok[q] ? (p.causal ? max(0, L - qlen + ti[q] + 1) : L) : 0;
    end_row[q] = min(seg_end, lim);
  }
  const bool wave_has_rows = row0 + rgw * RG * 16 < M;
  // Keys every valid row of this wave's row group sees (and the piece
  // streams): tiles below it need no mask.
  int end_min[RG];
#pragma unroll
  for (int q = 0; q < RG; ++q) {
    int v = rok[q] ? end_row[q] : 0x7fffffff;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = min(v, __shfl_xor(v, off));
    end_min[q] = min(__builtin_amdgcn_readfirstlane(v), eff_end);
  }

  // fp8 four-wave workgroups whose chunk leaves a wave without rows (48
  // heads): that wave issues every DMA instruction of a tile, so the waves
  // that compute issue none.  (Eight waves would need more than vmcnt's 63
  // outstanding loads in one wave; the bf16 variant spills.)
  constexpr bool kProd = FP8 && CONTIG && KS == 1 && NW == 4;
  // fp8 rows are 576 bytes, so every odd row starts half a 128-byte line in,
  // and loading each row's latent and rope apart makes the tile's 18 DMA
  // instructions touch 176 lines for its 144 (a plain DMA stream measured
  // 5.9 TB/s that way, 6.8 TB/s over whole lines).  A lone wave (NW 1) loads
  // whole lines instead and restores the layout with one exchange of 64
  // chunks per tile (line_fix), before it reads the tile.  (The four-wave
  // body's producer wave doing the same measured 3% slower at 48 heads when
  // it exchanged tile k before the barrier that releases it, and no faster
  // when it exchanged tile k+1 while the others computed on tile k: there the
  // waves' own tile work, not the memory path, sets the pace.)
  constexpr bool kLineDma = FP8 && CONTIG && NW == 1;
  const int active_waves = cdiv(min(M - row0, kRowsWG), 16 * RG);
  const bool prod_mode = kProd && active_waves < NW;
  const bool is_producer = prod_mode && wave == NW - 1;

  const float qs = p.q_scale ? *p.q_scale : 1.0f;
  const float ks = p.kv_scale ? *p.kv_scale : 1.0f;
  const float sl2 = p.softmax_scale * kLog2e * qs * ks;

  // ---- Q^T operand ----
  // bf16: lane (g, n) holds row n, dims 32c + 8g .. +7 for c = 0..17.
  // fp8:  latent dims 128c + 32g .. +31 for c = 0..3 (16x16x128 MFMA) and
  //       rope dims 512 + 32c + 8g .. +7 for c = 0..1 (16x16x32 MFMA).
  typedef bf16x8 QBf[FP8 ? 1 : RG][FP8 ? 1 : 18];
  typedef i32x8 QLat[FP8 ? RG : 1][4];
  typedef long QRope[FP8 ? RG : 1][2];
  // q as one [T, H, 576] tensor, or as q_nope [T, H, 512] + q_pe [T, H, 64];
  // bf16 q with an fp8 cache is quantised here (code = e4m3 RNE of
  // sat(q / q_scale)), the q prologue of the sparse page's forward_mqa.
  auto load_q = [&](QBf& qop, QLat& qlat, QRope& qrope) {
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      const int64_t tok = t0 + ti[q];
      const int64_t qoff = tok * p.q_stride_token + (int64_t)hh[q] * p.q_stride_head;
      const int64_t poff = p.q_pe ? tok * p.q_pe_stride_token + (int64_t)hh[q] * p.q_pe_stride_head
                                  : qoff + kKvRank;
      if constexpr (FP8) {
        if constexpr (!QB) {
          const uint8_t* qb = (const uint8_t*)p.q + qoff;
          const uint8_t* qr = (const uint8_t*)(p.q_pe ? p.q_pe : p.q) + poff;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const u32x4 lo = rok[q] ? *(const u32x4*)(qb + 128 * c + 32 * g) : u32x4{0, 0, 0, 0};
            const u32x4 hi = rok[q] ? *(const u32x4*)(qb + 128 * c + 32 * g + 16) : u32x4{0, 0, 0, 0};
            qlat[q][c] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
#pragma unroll
          for (int c = 0; c < 2; ++c) qrope[q][c] = rok[q] ? *(const long*)(qr + 32 * c + 8 * g) : 0;
        } else {
          const unsigned short* qb = (const unsigned short*)p.q + qoff;
          const unsigned short* qr = (const unsigned short*)(p.q_pe ? p.q_pe : p.q) + poff;
          const float qs_div = p.q_scale ? *p.q_scale : 1.0f;
          // 8 bf16 values -> 8 e4m3 codes (two dwords)
          auto quant8 = [&](const unsigned short* src) -> u32x2 {
            const u32x4 v = rok[q] ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
            float f[8];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              f[2 * i] = __uint_as_float(v[i] << 16);
              f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const float y = __fdiv_rn(f[i], qs_div);
              f[i] = y != y ? y : fminf(fmaxf(y, -448.f), 448.f);
            }
            u32x2 r;
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              int w = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * k], f[4 * k + 1], 0, false);
              w = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * k + 2], f[4 * k + 3], w, true);
              r[k] = (unsigned)w;
            }
            return r;
          };
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            i32x8 x;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
              const u32x2 w = quant8(qb + 128 * c + 32 * g + 8 * k);
              x[2 * k] = (int)w[0];
              x[2 * k + 1] = (int)w[1];
            }
            qlat[q][c] = x;
          }
#pragma unroll
          for (int c = 0; c < 2; ++c) qrope[q][c] = __builtin_bit_cast(long, quant8(qr + 32 * c + 8 * g));
        }
      } else {
        const __bf16* qb = (const __bf16*)p.q + qoff;
        const __bf16* qr = (const __bf16*)(p.q_pe ? p.q_pe : p.q) + poff;
#pragma unroll
        for (int c = 0; c < 18; ++c) {
          const __bf16* qp = c < 16 ? qb + 32 * c + 8 * g : qr + 32 * (c - 16) + 8 * g;
          const u32x4 v = rok[q] ? *(const u32x4*)qp : u32x4{0, 0, 0, 0};
          qop[q][c] = __builtin_bit_cast(bf16x8, v);
        }
      }
    }
  };


  // ---- DMA of one 32-token tile into ring slot b ----
  // V region: instruction i of this wave fills V row index vi = wave + NW*i
  // (bf16: tile row vi, 64 chunks; fp8: rows 2vi and 2vi+1, 32 chunks each).
  // Rope region: bf16 4 instructions of 8 rows, fp8 2 of 16 rows.  Lane
  // lambda writes LDS byte 16*lambda of its instruction's 1 KiB and loads the
  // logical chunk the swizzle stores there.  Rows at or past the tile's valid
  // count load tile row 0 instead (finite data that the softmax masks).
  constexpr int kNIR = kNI - kNIV;  // rope instructions per tile
  static_assert(kNIV % NW == 0, "V rows split evenly over the waves");
  constexpr int kVPerWave = kNIV / NW;
  constexpr int kRopePerWaveMax = (kNIR + NW - 1) / NW;
  constexpr int kRowsPerRope = 64 / F::kRopeChunks;
  const int lane16 = 16 * lane;
  const int v_half = lane / F::kVChunks;  // fp8: which of the instruction's two rows
  const int v_cpos = lane % F::kVChunks;
  const int rope_row_in = lane / F::kRopeChunks;
  const int rope_cpos = lane % F::kRopeChunks;
  // Whole-line fp8 tiles (kLineDma): the lane parts of the DMA offsets.  V
  // instructions: (16 c) ^ (32 half) swizzled, plus 576 for the odd row; the
  // row's rope chunk for the four displaced lanes.  Ninth-line instructions:
  // lane 8i + e takes byte 16e of pair i's ninth line, as row 2i+1's latent
  // chunk 28 + e (e < 4) or its rope chunk (e - 4) ^ swz_r (swz_r(2a+1) =
  // ((lane >> 4) & 3) for a = 8ri + lane / 8).
  const int lkey = (16 * v_cpos) ^ (32 * v_half);
  const int h576 = v_half ? kRowBytes : 0;
  const int rkey512 = kKvRank + 16 * (lane & 3);
  const int lane4 = lane >> 2;
  const int l8off = 2 * kRowBytes * (lane >> 3) +
                    ((lane & 7) < 4 ? kRowBytes + 16 * (28 + (lane & 7))
                                    : kRowBytes + kKvRank + 16 * (((lane & 7) - 4) ^ ((lane >> 4) & 3)));

  // Gathered tiles: a window of the request's page-table entries in LDS,
  // starting at page idx_pg0.  Every wave calls load_idx at the same tile;
  // it waits for all of the wave's loads (the window is refilled at most once
  // per kIdxCap pages).  Entries past the table repeat its last one.
  int idx_pg0 = 0x7fffffff / 2;
  auto issue_idx = [&](int pg) {
    const int npages = max(cap / p.block_size, 1);
    const int64_t stride = p.bt_stride_col;
    const i32x4 trs = make_rsrc(p.block_table + bt_base,
                                (int)min((int64_t)0x7fffffff, ((int64_t)(npages - 1) * stride + 1) * 4));
    for (int i = wave; i < kIdxCap / 64; i += NW) {
      const int e = min(pg + i * 64 + lane, npages - 1);
      dma_lds4(trs, lds_address(idx_buf) + (unsigned)(i * 256), (int)((int64_t)e * stride * 4));
    }
  };
  auto load_idx = [&](int pg) {
    __syncthreads();  // every wave is done with the previous window
    issue_idx(pg);
    wait_vmcnt<0>();
    __syncthreads();
    idx_pg0 = pg;
  };

  // Contiguous tiles: a scalar cursor over the page table.  A wave issues its
  // tiles in order, KS * TT keys apart, so the page index and the offset in
  // the page advance by addition; the page number is reloaded only when the
  // page changes.  A call for any other tile locates it by division.
  int cur_start = -1, cur_blk_i = 0, cur_in = 0, cached_blk_i = -1;
  int64_t cached_off = 0;  // byte offset of the cached page's first row
  auto issue_tile = [&](int k, int b) {
    const int tile_start = seg_start + k * TT;
    const int nvalid = min(TT, eff_end - tile_start);
    const unsigned lbase = lds_u32 + (unsigned)(b * kTileBytes);
    if constexpr (CONTIG) {
      if (tile_start != cur_start) {
        cur_blk_i = tile_start / p.block_size;
        cur_in = tile_start - cur_blk_i * p.block_size;
      }
      if (cur_blk_i != cached_blk_i) {
        // Uniform address, read-only table: a scalar load through the constant
        // address space, so no vector-memory wait drains the DMA stream.
        int blk = ((const __attribute__((address_space(4))) int*)p.block_table)
            [bt_base + (int64_t)cur_blk_i * p.bt_stride_col];
        if (blk < 0 || blk >= p.num_blocks) { blk = 0; bad = true; }
        cached_off = (int64_t)blk * p.block_size * kRowBytes;
        cached_blk_i = cur_blk_i;
      }
      // Buffer descriptor over the tile's rows (a guard: no offset below
      // leaves them; whole-line fp8 tiles cover only the valid rows, and
      // what lies past them loads as zeros, finite data the softmax masks);
      // per instruction a scalar row offset plus one 32-bit per-lane chunk
      // offset.
      const i32x4 rsrc = make_rsrc(p.kv + cached_off + (int64_t)cur_in * kRowBytes, (kLineDma ? nvalid : TT) * kRowBytes);
      const int key16 = opaque(lane16);
      // Otherwise rows at or past the valid count load tile row 0; a full
      // tile needs no clamp.
      auto dma_all = [&](auto full_tag) {
        constexpr bool kFull = decltype(full_tag)::value;
        auto clamp = [&](int row) { return kFull ? row : (row < nvalid ? row : 0); };
        auto dma_v = [&](int vi) {
          int voff, soff;
          // (the producer's lane offsets are formed per instruction, not held
          // for all of a tile's rows)
          auto keep = [&](int v) { return kProd ? opaque(v) : v; };
          if constexpr (!FP8) {
            soff = clamp(vi) * kRowBytes;
            voff = key16 ^ (16 * F::swz_v(vi));
          } else if constexpr (kLineDma) {
            // rows 2vi and 2vi+1 are the tile's bytes 1152 vi .. +1151, nine
            // 128-byte lines; this instruction reads the first eight whole:
            // row 2vi's latent and rope, and row 2vi+1's latent chunks 0-27.
            // The four lanes whose slots hold row 2vi+1's chunks 28-31 (lane
            // group 8 + (7 ^ (so >> 2))) load row 2vi's rope instead (rope
            // chunk (c - 28) ^ swz_r for slot c), for line_fix to exchange
            // with the rope region.  The row offset is the scalar soff; the
            // descriptor ends at the tile's valid rows (past them: zeros).
            const int se = F::swz_v(2 * vi), so = se ^ 2;
            const int nrm = (lkey ^ (16 * se)) + h576;
            const int exc = rkey512 ^ (16 * ((so & 3) ^ F::swz_r(2 * vi)));
            voff = lane4 == 8 + (7 ^ (so >> 2)) ? exc : nrm;
            soff = 2 * vi * kRowBytes;
          } else {
            // rows 2vi (lanes 0-31) and 2vi+1 (lanes 32-63); F::swz_v(2vi+1) = F::swz_v(2vi) ^ 2
            const int row = 2 * vi + keep(v_half);
            soff = 0;
            voff = clamp(row) * kRowBytes + (keep((16 * v_cpos) ^ (32 * v_half)) ^ (16 * F::swz_v(2 * vi)));
          }
          dma_lds16(rsrc, lbase + vi * 1024, voff, soff);
        };
        auto dma_r = [&](int ri) {
          if constexpr (kLineDma) {
            // the ninth line of row pairs 8ri .. 8ri+7 (row 2a+1's latent
            // chunks 28-31, then its rope) into the rope slots of rows 2a
            // (the latent chunks, for line_fix) and 2a+1
            dma_lds16(rsrc, lbase + (kNIV + ri) * 1024, l8off, 16 * kRowBytes * ri);
          } else {
            const int row = ri * kRowsPerRope + rope_row_in;
            const int voff = clamp(row) * kRowBytes + kKvRank * (FP8 ? 1 : 2) + 16 * (rope_cpos ^ F::swz_r(row));
            dma_lds16(rsrc, lbase + (kNIV + ri) * 1024, voff, 0);
          }
        };
        if (prod_mode) {
          // A wave without rows issues the whole tile; the others none.
          if (is_producer) {
#pragma unroll
            for (int vi = 0; vi < kNIV; ++vi) dma_v(vi);
#pragma unroll
            for (int ri = 0; ri < kNIR; ++ri) dma_r(ri);
          }
        } else {
#pragma unroll
          for (int i = 0; i < kVPerWave; ++i) dma_v(wave + NW * i);
#pragma unroll
          for (int i = 0; i < kRopePerWaveMax; ++i)
            if (wave + NW * i < kNIR) dma_r(wave + NW * i);
        }
      };
      dma_all(std::false_type{});
      // Advance the cursor to this wave's next tile.
      cur_start = tile_start + KS * TT;
      cur_in += KS * TT;
      while (cur_in >= p.block_size) { cur_in -= p.block_size; ++cur_blk_i; }
    } else {
      // Rows of a tile span several pages.  The page entries come from a
      // window of kIdxCap table entries in LDS, refilled (one full wait) when
      // a tile reaches past it, so no table load waits inside the stream.
      const int pg_first = tile_start / p.block_size;
      const int pg_last = (tile_start + max(nvalid, 1) - 1) / p.block_size;
      if (pg_first < idx_pg0 || pg_last >= idx_pg0 + kIdxCap) load_idx(pg_first);
      // Lane j < TT of every wave resolves tile row j to its cache row (rows
      // past the valid count resolve to tile row 0); the DMA instructions take
      // the rows they need across lanes (a lane read for a row the whole
      // instruction, or half of it, shares; a lane shuffle for per-lane rows),
      // so no LDS round trip and no barrier per tile.
      int phys = 0;
      bool pbad = false;
      if (lane < TT) {
        const int j = tile_start + (lane < nvalid ? lane : 0);
        // pages of a power-of-two size (1 for index streams) divide by a shift
        const int blk_i = (p.block_size & (p.block_size - 1)) == 0 ? j >> __builtin_ctz(p.block_size)
                                                                     : j / p.block_size;
        const int blk = idx_buf[blk_i - idx_pg0];
        pbad = blk < 0 || blk >= p.num_blocks;
        phys = pbad ? 0 : blk * p.block_size + (j - blk_i * p.block_size);
      }
      if (__ballot(pbad)) bad = true;
      auto row_base = [&](int pr) -> const char* { return p.kv + (int64_t)pr * kRowBytes; };
#pragma unroll
      for (int i = 0; i < kVPerWave; ++i) {
        const int vi = wave + NW * i;
        const char* src;
        if constexpr (!FP8) {
          const int pr = __builtin_amdgcn_readlane(phys, vi);
          src = row_base(pr) + (unsigned)(lane16 ^ (16 * F::swz_v(vi)));
        } else {
          // rows 2vi (lanes 0-31) and 2vi+1 (lanes 32-63)
          const int p0 = __builtin_amdgcn_readlane(phys, 2 * vi);
          const int p1 = __builtin_amdgcn_readlane(phys, 2 * vi + 1);
          const int row = 2 * vi + v_half;
          src = row_base(v_half ? p1 : p0) + 16 * (v_cpos ^ F::swz_v(row));
        }
        dma_lds16_gather(lbase + vi * 1024, src);
      }
#pragma unroll
      for (int i = 0; i < kRopePerWaveMax; ++i) {
        const int ri = wave + NW * i;
        if (ri < kNIR) {
          const int row = ri * kRowsPerRope + rope_row_in;
          const int pr = __shfl(phys, row);
          const char* src = row_base(pr) + kKvRank * (FP8 ? 1 : 2) + 16 * (rope_cpos ^ F::swz_r(row));
          dma_lds16_gather(lbase + (kNIV + ri) * 1024, src);
        }
      }
    }
  };

  // The exchange that completes a whole-line tile: lane (a, q) swaps row
  // 2a+1's latent slot 28+q (which the DMA filled with row 2a's rope) with
  // row 2a's rope slot q (filled with row 2a+1's latent chunk 28+q).
  auto line_fix = [&](const char* buf) {
    const int a = lane >> 2, q = lane & 3;
    const int x = 1024 * a + 512 + 16 * ((28 + q) ^ F::swz_v(2 * a + 1));
    const int y = kVRegion + 2 * a * F::kRopePitch + 16 * q;
    LDS_AS u32x4* px = (LDS_AS u32x4*)(buf + x);
    LDS_AS u32x4* py = (LDS_AS u32x4*)(buf + y);
    const u32x4 vx = *px, vy = *py;
    *px = vy;
    *py = vx;
  };

  // Per-lane LDS read geometry (see the layout note above KvFmt).
  // K reads: lane (g, t = n) reads tile row 16b + n.
  int kv_base[2], kv_x[2], kr_base[2], kr_x[2];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int lrow = 16 * b + n;
    kv_base[b] = lrow * F::kVPitch;
    kr_base[b] = kVRegion + lrow * F::kRopePitch;
    if constexpr (FP8) {
      // latent: logical chunks 8c + 2g (+1); rope: chunk 2c + g/2, half g & 1
      kv_x[b] = (2 * g) ^ F::swz_v(lrow);
      kr_x[b] = (g >> 1) ^ F::swz_r(lrow);
      kr_base[b] += 8 * (g & 1);
    } else {
      // logical chunk 4c + g
      kv_x[b] = g ^ F::swz_v(lrow);
      kr_x[b] = g ^ F::swz_r(lrow);
    }
  }
  // V^T transpose reads.
  int vt_base[2], vt_x[2];
  if constexpr (FP8) {
    // address lane 16g + 2e + j: k-slot e = (block e/4, A-row 4g + e%4), dims 16db + 8j
    const int e = (lane >> 1) & 7, j = lane & 1;
    const int vrow = 16 * (e >> 2) + 4 * g + (e & 3);
    vt_base[0] = vrow * F::kVPitch + 8 * j;
    vt_x[0] = F::swz_v(vrow);
    vt_base[1] = vt_x[1] = 0;
  } else {
    // address lane 16g + 4i + j: A-row 4g + i of block 0 / 1, dims 16db + 4j
    const int i4 = (lane >> 2) & 3, j = lane & 3;
#pragma unroll
    for (int rd = 0; rd < 2; ++rd) {
      const int vrow = 16 * rd + 4 * g + i4;
      vt_base[rd] = vrow * F::kVPitch + 8 * (j & 1);
      vt_x[rd] = (j >> 1) ^ F::swz_v(vrow);
    }
  }

  // ---- per-tile steps ----
  // LDS operands are prefetched several MFMA steps ahead: one MFMA issues every
  // 16-32 cycles, while an LDS read takes ~100-200 cycles to return.  (Kernels
  // sized for two waves per SIMD have half the registers: shallower there.)
  // (bf16 with two waves per SIMD: K operands two steps ahead and Vt operands
  // four, which keeps the Q, S and accumulator registers clear of spills in
  // the tile loop.)
  constexpr int kPF = OCC == 2 ? (FP8 ? 4 : 2) : 8;
  constexpr int kPFL = OCC == 2 ? 2 : 4;
  constexpr int kPFV = OCC == 2 ? 4 : 8;
  typedef typename std::conditional<kNB == 2, bf16x8, i16x4>::type POp;
  typedef typename std::conditional<FP8, i32x2, POp>::type VRaw;
  typedef f32x4 Acc[RG][32];
  typedef f32x4 SBlk[RG][2];
  // P^T operand of one row group (the layout of the S^T accumulator, so it
  // needs no data movement): bf16 values, or e4m3 codes packed in a long.
  struct PVal {
    POp pb[RG];
    long pb8[FP8 ? RG : 1];
  };

  // S^T = K . Q^T for the tile's 16-token blocks.
  auto qk_tile = [&](const char* buf, const QBf& qop, const QLat& qlat, const QRope& qrope, SBlk& sblk) {
    int kvb[2], kvx[2], krb[2], krx[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      kvb[b] = opaque(kv_base[b]); kvx[b] = opaque(kv_x[b]);
      krb[b] = opaque(kr_base[b]); krx[b] = opaque(kr_x[b]);
    }
#pragma unroll
    for (int q = 0; q < RG; ++q) sblk[q][0] = sblk[q][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (FP8) {
      // latent: 4 x (16x16x128 f8f6f4) per block; steps (c, b), c = 0..3
      // (8 c) ^ x = 16 (c / 2) + (8 (c % 2)) ^ x for x < 16: two per-lane
      // bases per block and half, the rest an immediate offset.
      int kl2[kNB][2][2];
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          kl2[b][e][0] = kvb[b] + 16 * ((8 * e) ^ kvx[b]);
          kl2[b][e][1] = kvb[b] + 16 * ((8 * e) ^ (kvx[b] ^ 1));
        }
      auto lat_load = [&](int st) -> i32x8 {
        const int c = st / kNB, b = st % kNB;
        const u32x4 lo = lds_load<u32x4>(buf, kl2[b][c & 1][0] + 256 * (c >> 1));
        const u32x4 hi = lds_load<u32x4>(buf, kl2[b][c & 1][1] + 256 * (c >> 1));
        return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      constexpr int kLat = 4 * kNB;
      i32x8 kl[kPFL];
#pragma unroll
      for (int i = 0; i < kPFL; ++i) kl[i] = lat_load(i);
#pragma unroll
      for (int st = 0; st < kLat; ++st) {
        const i32x8 cur = kl[st % kPFL];
        if (st + kPFL < kLat) kl[st % kPFL] = lat_load(st + kPFL);
        const int c = st / kNB, b = st % kNB;
#pragma unroll
        for (int q = 0; q < RG; ++q)
          sblk[q][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(cur, qlat[q][c], sblk[q][b], 0, 0,
                                                                         0, 127, 0, 127);
        __builtin_amdgcn_sched_barrier(0);
      }
      // rope: 2 x (16x16x32 fp8) per block
#pragma unroll
      for (int c = 0; c < 2; ++c) {
#pragma unroll
        for (int b = 0; b < kNB; ++b) {
          const long a = lds_load<long>(buf, krb[b] + 16 * ((2 * c) ^ krx[b]));
#pragma unroll
          for (int q = 0; q < RG; ++q)
            sblk[q][b] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(a, qrope[q][c], sblk[q][b], 0, 0, 0);
        }
      }
    } else {
      // 18 * kNB (chunk, block) steps of 16x16x32 bf16
      constexpr int kSteps = 18 * kNB;
      // (4 c) ^ kvx = 16 (c / 4) + (4 (c % 4)) ^ kvx for c < 16: four per-lane
      // bases per block, the rest an immediate offset.
      int kb4[kNB][4];
#pragma unroll
      for (int b = 0; b < kNB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) kb4[b][e] = kvb[b] + 16 * ((4 * e) ^ kvx[b]);
      auto k_off = [&](int st) {
        const int c = st / kNB, b = st % kNB;
        if (c < 16) return kb4[b][c & 3] + 256 * (c >> 2);
        return krb[b] + 16 * ((4 * (c - 16)) ^ krx[b]);
      };
      bf16x8 kop[kPF];
#pragma unroll
      for (int i = 0; i < kPF; ++i) kop[i] = lds_load<bf16x8>(buf, k_off(i));
#pragma unroll
      for (int st = 0; st < kSteps; ++st) {
        const bf16x8 cur = kop[st % kPF];
        if (st + kPF < kSteps) kop[st % kPF] = lds_load<bf16x8>(buf, k_off(st + kPF));
        const int c = st / kNB, b = st % kNB;
#pragma unroll
        for (int q = 0; q < RG; ++q)
          sblk[q][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qop[q][c], sblk[q][b], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // Base-2 online softmax per row over one tile.  The reference max m_run
  // only moves when the tile max exceeds it by more than kLazy, and
  // p = 2^(x - (m_run - kBias)) <= 2^8; m_true tracks the exact max and the
  // end rescales to it once.  l sums the exact p, lh (fp8) the e4m3-rounded
  // p the product uses.  Returns whether this lane's rows need the
  // accumulator rescaled by alpha.
  auto softmax_tile = [&](const SBlk& sblk, int tile_start, float (&m_run)[RG], float (&m_true)[RG],
                          float (&l_run)[RG], float (&lh_run)[RG], PVal& pv_out, float (&alpha)[RG]) -> bool {
    bool rescale = false;
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      float x[4 * kNB];
      float mloc = -INFINITY;
      if (tile_start + TT <= end_min[q]) {
#pragma unroll
        for (int i = 0; i < 4 * kNB; ++i) {
          x[i] = sblk[q][i >> 2][i & 3] * sl2;
          mloc = fmaxf(mloc, x[i]);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 4 * kNB; ++i) {
          // score slot i: block i/4, A-row 4g + i%4
          const int tok = tile_start + 16 * (i >> 2) + 4 * g + (i & 3);
          const float v = (tok < end_row[q]) ? sblk[q][i >> 2][i & 3] * sl2 : -INFINITY;
          x[i] = v;
          mloc = fmaxf(mloc, v);
        }
      }
      mloc = wave_max(mloc);
      m_true[q] = fmaxf(m_true[q], mloc);
      const float m_new = (mloc > m_run[q] + Lazy<FP8>::kLazy) ? mloc : m_run[q];
      alpha[q] = 1.f;
      float pv[4 * kNB];
      const bool live = m_new != -INFINITY;
      if (!live) {
#pragma unroll
        for (int i = 0; i < 4 * kNB; ++i) pv[i] = 0.f;
      } else {
        alpha[q] = __builtin_amdgcn_exp2f(m_run[q] - m_new);
        const float m_ref = m_new - Lazy<FP8>::kBias;
#pragma unroll
        for (int i = 0; i < 4 * kNB; ++i) pv[i] = __builtin_amdgcn_exp2f(x[i] - m_ref);
      }
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4 * kNB; ++i) psum += pv[i];
      if (live) l_run[q] = l_run[q] * alpha[q] + psum;
      if constexpr (FP8) {
        // P^T in e4m3 for the fp8 P.V product (p <= 2^8 = 256 < 448).
        // e4m3 flushes p < 2^-10 to zero, so the product's weights can sum
        // to less than the exact exp-sum l.  lh accumulates the rounded
        // weights; the end of the piece rescales the accumulator by l / lh,
        // so the output is the average under the weights the product used
        // (a constant V stays exact) while l, and with it the LSE, stays the
        // exact sum.
        int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[0], pv[1], 0, false);
        w0 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[2], pv[3], w0, true);
        int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[4], pv[5], 0, false);
        w1 = __builtin_amdgcn_cvt_pk_fp8_f32(pv[6], pv[7], w1, true);
        pv_out.pb8[q] = (long)(unsigned)w0 | ((long)(unsigned)w1 << 32);
        const f32x2 r0 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, false), r1 = __builtin_amdgcn_cvt_pk_f32_fp8(w0, true);
        const f32x2 r2 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, false), r3 = __builtin_amdgcn_cvt_pk_f32_fp8(w1, true);
        const float hsum = ((r0[0] + r0[1]) + (r1[0] + r1[1])) + ((r2[0] + r2[1]) + (r3[0] + r3[1]));
        if (live) lh_run[q] = lh_run[q] * alpha[q] + hsum;
      }
      m_run[q] = m_new;
      rescale |= alpha[q] != 1.f;
      if constexpr (FP8) {
      } else if constexpr (kNB == 2) {
        pv_out.pb[q] = to_bf16x8(pv);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) pv_out.pb[q][i] = __builtin_bit_cast(short, (__bf16)pv[i]);
      }
    }
    return rescale;
  };

  // acc *= alpha, one accumulator group at a time: keeps the AGPR -> VGPR ->
  // AGPR round trip to four registers.  One wave per SIMD (OCC 1) keeps the
  // accumulators in AGPRs; there the empty asm redefines the group in its
  // AGPRs inside this rarely taken branch, as without it the compiler copies
  // every accumulator to VGPRs at the top of each tile, on the path that does
  // not rescale as well (bf16 at 16 heads: 1.1 us of 157 per step; the fp8
  // body, with half the tiles, measured no gain).  With two waves per SIMD
  // they live in VGPRs, and pinning them to AGPRs would split the register
  // budget and spill.
  auto rescale_acc = [&](Acc& acc, const float (&alpha)[RG]) {
#pragma unroll
    for (int q = 0; q < RG; ++q)
#pragma unroll
      for (int d = 0; d < 32; ++d) {
        if constexpr (OCC == 1 && !FP8) asm volatile("" : "+a"(acc[q][d]));
        acc[q][d] *= alpha[q];
        __builtin_amdgcn_sched_barrier(0);
      }
  };

  // O^T += V^T . P^T over 32 dim blocks of 16, operands prefetched kPFV ahead.
  auto pv_tile = [&](const char* buf, Acc& acc, const PVal& pvv) {
    int vtb[2], vtx[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) { vtb[b] = opaque(vt_base[b]); vtx[b] = opaque(vt_x[b]); }
    // The swizzle (vtx < 16) only touches the low four chunk bits, so the
    // chunk splits into an immediate offset plus a per-lane part that repeats:
    // with one 16-token block (2 db) ^ vtx = 16 (db / 8) + (2 (db % 8)) ^ vtx,
    // for fp8 db ^ vtx = 16 (db / 16) + (db % 16) ^ vtx.  The per-lane bases
    // are formed once per tile instead of an address per read.
    const char* vb8[kNB == 1 ? 8 : 1];
    const char* vb16[FP8 ? 16 : 1];
    if constexpr (kNB == 1) {
#pragma unroll
      for (int d = 0; d < 8; ++d) vb8[d] = buf + vtb[0] + 16 * ((2 * d) ^ vtx[0]);
    } else if constexpr (FP8) {
#pragma unroll
      for (int d = 0; d < 16; ++d) vb16[d] = buf + vtb[0] + 16 * (d ^ vtx[0]);
    }
    auto v_load = [&](int db) -> VRaw {
      if constexpr (kNB == 1) {
        // one 16-token block: k-slots 4g..4g+3 from a single transpose read
        return __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(vb8[db & 7] + 256 * (db >> 3)));
      } else if constexpr (FP8) {
        // logical chunk db, half j
        return __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(vb16[db & 15] + 256 * (db >> 4)));
      } else {
        // logical chunk 2db + j/2, half j & 1
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS i16x4*)(buf + vtb[0] + 16 * ((2 * db) ^ vtx[0])));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS i16x4*)(buf + vtb[1] + 16 * ((2 * db) ^ vtx[1])));
        return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    };
    VRaw vop[kPFV];
#pragma unroll
    for (int i = 0; i < kPFV; ++i) vop[i] = v_load(i);
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const VRaw cur = vop[db % kPFV];
      if (db + kPFV < 32) vop[db % kPFV] = v_load(db + kPFV);
      if constexpr (kNB == 1) {
#pragma unroll
        for (int q = 0; q < RG; ++q)
          acc[q][db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(cur, pvv.pb[q], acc[q][db], 0, 0, 0);
      } else if constexpr (FP8) {
        const long va = __builtin_bit_cast(long, cur);
#pragma unroll
        for (int q = 0; q < RG; ++q)
          acc[q][db] = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(va, pvv.pb8[q], acc[q][db], 0, 0, 0);
      } else {
#pragma unroll
        for (int q = 0; q < RG; ++q)
          acc[q][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, pvv.pb[q], acc[q][db], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- the piece's result ----
  // acc holds sum_j 2^(x_j - m_true) V_j in code units for each row, l_tot
  // the matching sum of weights (already reduced over the lanes of a row).
  // The dim blocks db0 .. db0 + ND - 1 of every row are stored (ND = 32 unless
  // k-split waves share the store); the row statistics only if with_stats.
  auto write_result = [&](const auto& acc, const float (&l_tot_in)[RG], const float (&m_fin)[RG], bool bad_all,
                          int db0, bool with_stats) {
    constexpr int ND = sizeof(acc[0]) / sizeof(f32x4);
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      const float l_tot = l_tot_in[q];
      if (!rok[q]) continue;
      // One store loop for every destination: values acc * mult, as fp32 or
      // as 16-bit (bf16 rounded to nearest even, or fp16).
      float mult, stat0, stat1;
      float* stat0_p;
      float* stat1_p;
      char* dst;
      int kind;  // 0 bf16, 1 fp16, 2 fp32
      if (pc.mode == kOutFinal) {
        // Normalised output and natural-log LSE; an optional sink joins the
        // softmax as one more logit with a zero value.
        const bool has = m_fin[q] > -INFINITY;
        float lse = has ? kLn2 * (m_fin[q] + __log2f(l_tot)) : -INFINITY;
        mult = has ? ks / l_tot : 0.f;
        if (p.sinks) {
          const float nl = logaddexp_f(lse, p.sinks[hh[q]]);
          mult = has ? mult * expf(lse - nl) : 0.f;
          lse = nl;
        }
        if (bad_all) { lse = __builtin_nanf(""); mult = __builtin_nanf(""); }
        const int64_t orow = (int64_t)(t0 + ti[q]) * H + hh[q];
        kind = p.out_dtype;
        dst = (char*)p.out + (orow * kKvRank + 16 * db0 + 4 * g) * (kind == 2 ? 4 : 2);
        stat0 = lse;
        stat0_p = p.lse + orow;
        stat1 = 0.f;
        stat1_p = nullptr;
      } else {
        // partials in fp32, or in bf16 when the fused call's output is
        // 16-bit (a rounding of the size that output takes anyway)
        const int64_t slot = pc.mode == kOutSegment
                                 ? ((int64_t)(t0 + ti[q]) * H + hh[q]) * p.num_segments + pc.s
                                 : pc.prow0 + (rgw * RG + q) * 16 + n;
        mult = ks;
        if (!p.piece_bf16) {
          kind = 2;
          dst = (char*)(p.seg_out + slot * kKvRank + 16 * db0 + 4 * g);
        } else {
          kind = 0;
          dst = (char*)(p.piece_out + slot * kKvRank + 16 * db0 + 4 * g);
        }
        stat0 = bad_all ? __builtin_nanf("") : m_fin[q];
        stat0_p = p.seg_max + slot;
        stat1 = l_tot;
        stat1_p = p.seg_sum + slot;
      }
#pragma unroll
      for (int db = 0; db < ND; ++db) {
        const f32x4 o = acc[q][db] * mult;
        if (kind == 2) {
          *(f32x4*)(dst + 64 * db) = o;
        } else {
          u32x2 v;
          if (kind == 0) {
            v[0] = (unsigned)f32_to_bf16_rne(o[0]) | ((unsigned)f32_to_bf16_rne(o[1]) << 16);
            v[1] = (unsigned)f32_to_bf16_rne(o[2]) | ((unsigned)f32_to_bf16_rne(o[3]) << 16);
          } else {
            v[0] = (unsigned)__builtin_bit_cast(unsigned short, (_Float16)o[0]) |
                   ((unsigned)__builtin_bit_cast(unsigned short, (_Float16)o[1]) << 16);
            v[1] = (unsigned)__builtin_bit_cast(unsigned short, (_Float16)o[2]) |
                   ((unsigned)__builtin_bit_cast(unsigned short, (_Float16)o[3]) << 16);
          }
          *(u32x2*)(dst + 32 * db) = v;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (with_stats && g == 0) {
        *stat0_p = stat0;
        if (stat1_p) *stat1_p = stat1;
      }
    }
  };

  {
    // ---- every wave: QK, softmax and P.V of its own rows, tile after tile ----
    // k-split waves (KS > 1): wave kw takes tiles first, first + KS, ... of
    // the piece in its own ring slots kw * NBUF ..; pc.phase rotates the
    // first tile so that the waves share a workgroup's pieces evenly.
    static_assert(KS == 1 || (NW == 1 && RG == 1 && CONTIG && NBUF > 1 && 32 % KS == 0),
                  "k-split waves: one row group over contiguous tiles");
    const int kw = KS > 1 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : 0;
    const int first = KS > 1 ? (kw - pc.phase + KS) % KS : 0;
    const int nloc = ntiles > first ? (ntiles - first + KS - 1) / KS : 0;
    const int slot0 = kw * NBUF;
    auto tile_of = [&](int k) { return first + KS * k; };
    QBf qop;
    QLat qlat;
    QRope qrope;
    load_q(qop, qlat, qrope);
    // Gathered tiles: the first page window loads in the same round trip as q
    // (the previous piece ended with a barrier, so nobody reads the window).
    const bool early_idx = !CONTIG && ntiles > 0;
    if (early_idx) issue_idx(seg_start / p.block_size);
    wait_vmcnt<0>();  // q is in registers before the DMA stream starts
    if (early_idx) {
      __syncthreads();
      idx_pg0 = seg_start / p.block_size;
    }
    Acc acc;
#pragma unroll
    for (int q = 0; q < RG; ++q)
#pragma unroll
      for (int d = 0; d < 32; ++d) acc[q][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[RG], m_true[RG], l_run[RG], lh_run[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q) { m_run[q] = m_true[q] = -INFINITY; l_run[q] = lh_run[q] = 0.f; }

#pragma unroll
    for (int k = 0; k < NBUF - 1; ++k)
      if (k < nloc) issue_tile(tile_of(k), slot0 + k);

    for (int k = 0; k < nloc; ++k) {
      if constexpr (NBUF == 1) {
        // Single slot: load, wait, compute; other waves on the SIMD overlap.
        if (k > 0) __syncthreads();  // every wave is done with the slot
        issue_tile(k, 0);
        wait_vmcnt<0>();
        __syncthreads();
      } else if constexpr (NW == 1) {
        // A lone wave owns its ring: the slot of tile k-1 is free as soon as
        // its reads returned, so the next tile is issued before waiting for
        // tile k and NBUF tiles are in flight during the wait.
        if (k + NBUF - 1 < nloc) issue_tile(tile_of(k + NBUF - 1), slot0 + (k + NBUF - 1) % NBUF);
        wait_tiles<kNIw, NBUF - 1>(min(NBUF - 1, nloc - 1 - k));
      } else {
        if (is_producer) wait_tiles<kNI, (NBUF >= 2 ? NBUF - 2 : 0)>(min(NBUF - 2, ntiles - 1 - k));
        else wait_tiles<kNIw, (NBUF >= 2 ? NBUF - 2 : 0)>(min(NBUF - 2, ntiles - 1 - k));
        __syncthreads();
        if (k + NBUF - 1 < ntiles) issue_tile(k + NBUF - 1, (k + NBUF - 1) % NBUF);
      }
      if (!wave_has_rows) continue;
      const char* buf = lds[slot0 + k % NBUF];
      if constexpr (kLineDma) line_fix(buf);
      SBlk sblk;
      qk_tile(buf, qop, qlat, qrope, sblk);
      PVal pvv;
      float alpha[RG];
      const bool resc = softmax_tile(sblk, seg_start + tile_of(k) * TT, m_run, m_true, l_run, lh_run, pvv, alpha);
      if (__ballot(resc)) rescale_acc(acc, alpha);
      __builtin_amdgcn_sched_barrier(0);
      pv_tile(buf, acc, pvv);
    }

    // Final exact-max correction of the lazily rescaled state (and, for
    // fp8, the l / lh weight correction of the e4m3-rounded P).
    float l_tot[RG];
#pragma unroll
    for (int q = 0; q < RG; ++q) {
      // p was taken relative to m_run - kBias; rescale to the exact max
      const float f0 = (m_true[q] == -INFINITY)
                           ? 1.f
                           : __builtin_amdgcn_exp2f((m_run[q] - Lazy<FP8>::kBias) - m_true[q]);
      float f = f0;
      l_tot[q] = l_run[q] + __shfl_xor(l_run[q], 16);
      l_tot[q] += __shfl_xor(l_tot[q], 32);
      if constexpr (FP8) {
        float lh = lh_run[q] + __shfl_xor(lh_run[q], 16);
        lh += __shfl_xor(lh, 32);
        if (lh > 0.f) f *= l_tot[q] / lh;
      }
      l_tot[q] *= f0;
#pragma unroll
      for (int d = 0; d < 32; ++d) {
        acc[q][d] *= f;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    bad = __syncthreads_or(bad ? 1 : 0) != 0;
    if constexpr (KS == 1) {
      write_result(acc, l_tot, m_true, bad, 0, true);
    } else {
      // Combine the k-split waves' states: each leaves its rows' max and sum
      // and its accumulator (scaled to its own max) in its ring slots (whose
      // DMA and reads are complete); then wave kw sums dim blocks
      // kDB * kw .. + kDB - 1 over the waves, each weighted by 2^(m_w - M)
      // for the common max M, and stores them.
      __shared__ float ks_stat[KS][2][16];
      constexpr int kDB = 32 / KS;
      char* own = &lds[slot0][0];
      if (g == 0) {
        ks_stat[kw][0][n] = m_true[0];
        ks_stat[kw][1][n] = l_tot[0];
      }
#pragma unroll
      for (int db = 0; db < 32; ++db) *(LDS_AS f32x4*)(own + 1024 * db + 16 * lane) = acc[0][db];
      __syncthreads();
      float m_all = -INFINITY;
#pragma unroll
      for (int w = 0; w < KS; ++w) m_all = fmaxf(m_all, ks_stat[w][0][n]);
      float fw[KS];
      float l_all = 0.f;
#pragma unroll
      for (int w = 0; w < KS; ++w) {
        const float mw = ks_stat[w][0][n];
        fw[w] = mw == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw - m_all);
        l_all += fw[w] * ks_stat[w][1][n];
      }
      f32x4 comb[1][kDB];
#pragma unroll
      for (int j = 0; j < kDB; ++j) {
        comb[0][j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int w = 0; w < KS; ++w)
          comb[0][j] += fw[w] * lds_load<f32x4>(&lds[w * NBUF][0], 1024 * (kDB * kw + j) + 16 * lane);
      }
      const float lt[1] = {l_all};
      const float mf[1] = {m_all};
      write_result(comb, lt, mf, bad, kDB * kw, kw == 0);
      __syncthreads();  // every wave is done with the others' slots
    }
  }
}

// ---------------------------------------------------------------------------
// Wide waves (fp8): 32 query rows per wave
// ---------------------------------------------------------------------------
// A wave owns 32 rows (token, head) and works on 32x32 blocks:
//   S^T[token, row] = K . Q^T     v_mfma_scale_f32_32x32x64_f8f6f4: 8 latent
//                                 steps of 64 dims + 1 rope step per tile
//   O^T[dim, row]  += V^T . P^T   v_mfma_f32_32x32x16_fp8: 16 blocks of 32
//                                 dims x 2 steps of 16 tokens per tile
// Every K or V byte a wave reads from LDS feeds 32 rows (the 16-row shapes
// feed 16), and the accumulator (512 dims x 32 rows: 256 registers per lane)
// fits the AGPRs at one wave per SIMD.  The LDS tile keeps the regions of
// KvFmt<true> (V rows of 512 B, rope rows of 64 B at +16 KiB) with its own V
// swizzle, swz_w.
//
// Lane layouts (checked on gfx950 with a lane probe):
//  32x32x64 f8f6f4: A lane l = row l%32, k 32(l/32)..+31; B lane l = column
//    l%32, k 32(l/32)..+31; D lane l, register r = row 8(r/4)+4(l/32)+r%4,
//    column l%32.  32x32x16 fp8: the same with k 8(l/32)..+7.
//  ds_read_b64_tr_b8: each lane of a 16-lane group reads 8 bytes (row
//    lane/2 of an 8 x 16-byte block, half lane%2); lane n of the group gets
//    byte n of the block's rows 0..7.
// So the S^T accumulator (tokens 8(r/4)+4(l/32)+r%4 of column l%32) is the
// P^T operand of the two 16-token steps as it stands (registers 8s..8s+7 for
// step s), and the V^T reads fetch the same token order.

// Chunk swizzle of the wide tile's V region (16-byte chunk c of row r sits at
// c ^ swz_w(r)): a bijection of r's low four bits, so the 16 rows one K read
// serves at once land in 16 distinct bank groups; its bits 3..1 are a
// bijection of (r1, r0, r3), so the 8 rows of a transpose-read group (r2
// fixed) land in 8 distinct 32-byte bank pairs.
__device__ __forceinline__ int swz_w(int r) {
  return (((r >> 1) & 1) << 3) | ((r & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// One step of S^T = K . Q^T (64 dims, e4m3 x e4m3): v_mfma_f32_32x32x64_f8f6f4
// written with its result in VGPRs.  At one wave per SIMD the compiler gives
// every MFMA it emits an AGPR result, and the 512-dim accumulator already
// takes all 256 AGPRs.  The steps of one tile chain through the same
// registers (exact overlap of the accumulator needs no wait states); the
// last step ends with the wait states a VALU read of its result needs
// (24 >= the compiler's own for this MFMA), so the result may be read by any
// instruction after it.  Each step opens with the 2 wait states an MFMA
// operand written by a VALU instruction needs.
template <bool FIRST, bool LAST>
__device__ __forceinline__ void qk_step_w32(f32x16& s, const i32x8& k, const i32x8& q) {
  if constexpr (FIRST && LAST) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0\n\ts_nop 15\n\ts_nop 7"
                 : "=&v"(s) : "v"(k), "v"(q));
  } else if constexpr (FIRST) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "v"(q));
  } else if constexpr (LAST) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 7"
                 : "+v"(s) : "v"(k), "v"(q));
  } else {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+v"(s) : "v"(k), "v"(q));
  }
}

// One P.V step O^T += 2^e V^T . P^T (64 tokens, e4m3, E8M0 scale 2^e of the
// P^T columns, V^T unscaled), v_mfma_scale_f32_32x32x64_f8f6f4 on an AGPR
// accumulator, written as assembly so that it keeps its place among the DMA
// and LDS instructions the stream puts between the steps.  It opens with the
// 2 wait states an operand written by a VALU instruction needs; an
// accumulator chained from the previous step on the same registers needs
// none.  mfma_settle_w32 gives the wait states a read of the last result
// needs.
__device__ __forceinline__ void pv_step_w32(f32x16& acc, const i32x8& v, const i32x8& pt, int scale_a,
                                            int scale_b) {
  asm volatile("s_nop 1\n\tv_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
               : "+a"(acc)
               : "v"(v), "v"(pt), "v"(scale_a), "v"(scale_b));
}
__device__ __forceinline__ void mfma_settle_w32() { asm volatile("s_nop 15\n\ts_nop 7"); }

// A wide wave's result for its row (lane l holds row l % 32): register r of
// dim block d holds dim 32 d + 8 (r / 4) + 4 h + r % 4 (h = l / 32); stored
// times mult at dst as fp32 (kind 2), bf16 (0) or fp16 (1), one store loop
// per kind (the kind is chosen outside the loop).
__device__ __forceinline__ void store_w32(const f32x16 (&acc)[16], int h, float mult, char* dst, int kind) {
  auto store_all = [&](auto kind_tag) {
    constexpr int K = decltype(kind_tag)::value;
#pragma unroll
    for (int d = 0; d < 16; ++d) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int dim = 32 * d + 8 * q + 4 * h;
        const f32x4 o = f32x4{acc[d][4 * q], acc[d][4 * q + 1], acc[d][4 * q + 2], acc[d][4 * q + 3]} * mult;
        if constexpr (K == 2) {
          *(f32x4*)(dst + 4 * dim) = o;
        } else {
          u32x2 v;
          if constexpr (K == 0) {
            v[0] = (unsigned)f32_to_bf16_rne(o[0]) | ((unsigned)f32_to_bf16_rne(o[1]) << 16);
            v[1] = (unsigned)f32_to_bf16_rne(o[2]) | ((unsigned)f32_to_bf16_rne(o[3]) << 16);
          } else {
            v[0] = (unsigned)__builtin_bit_cast(unsigned short, (_Float16)o[0]) |
                   ((unsigned)__builtin_bit_cast(unsigned short, (_Float16)o[1]) << 16);
            v[1] = (unsigned)__builtin_bit_cast(unsigned short, (_Float16)o[2]) |
                   ((unsigned)__builtin_bit_cast(unsigned short, (_Float16)o[3]) << 16);
          }
          *(u32x2*)(dst + 2 * dim) = v;
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (kind == 2) store_all(std::integral_constant<int, 2>{});
  else if (kind == 0) store_all(std::integral_constant<int, 0>{});
  else store_all(std::integral_constant<int, 1>{});
}

template <typename F, int... C>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, C...>) {
  (f(std::integral_constant<int, C>{}), ...);
}

template <int NW, int NBUF, bool QB>
__device__ __forceinline__ void run_piece_w32(const SegmentLaunch& p, char (*lds)[18432], unsigned lds_u32,
                                              const Piece& pc) {
  constexpr int TT = 32;                        // tokens per DMA tile (ring slot)
  constexpr int kRowBytes = 576;
  constexpr int kTileBytes = TT * kRowBytes;
  constexpr int kVRegion = TT * 512;
  constexpr int kRowsWG = 32 * NW;
  constexpr int kNI = 18;                       // DMA instructions per tile: 16 V (2 rows) + 2 rope (16 rows)
  constexpr int kNIw = kNI / NW;                // per wave, lower bound
  constexpr int kVw = 16 / NW;                  // V instructions per wave
  static_assert(kTileBytes == 18432, "fp8 32-token tiles");
  static_assert(NW == 2 || NW == 4, "the wide body runs two or four waves");
  static_assert(NBUF >= 3, "a tile in the P.V phase, one in the QK phase, and one in flight");

  const int lane = threadIdx.x & 63;
  const int wave = NW == 1 ? 0 : __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 31;  // the lane's query row in the wave
  const int h = lane >> 5;

  const int r = pc.r, t0 = pc.t0, qlen = pc.qlen, L = pc.L;
  const int H = p.num_heads;
  const int M = qlen * H;
  const int row0 = pc.row0;
  int64_t bt_base;
  int cap;
  page_list(p, r, &bt_base, &cap);
  bt_base = __builtin_amdgcn_readfirstlane((int)(bt_base & 0xffffffff)) |
            ((int64_t)__builtin_amdgcn_readfirstlane((int)(bt_base >> 32)) << 32);
  cap = __builtin_amdgcn_readfirstlane(cap);
  bool bad = L > cap;
  const int seg_start = pc.seg_start;
  const int seg_end = pc.seg_end;
  const int last_row = min(row0 + kRowsWG, M) - 1;
  const int lim_wg = p.causal ? (L - qlen + last_row / H + 1) : L;
  const int eff_end = min(min(seg_end, lim_wg), cap);
  const int ntiles = eff_end > seg_start ? cdiv(eff_end - seg_start, TT) : 0;

  // The lane's query row (lanes l and l + 32 hold the same row).
  const int row = row0 + wave * 32 + j;
  const bool rok = row < M;
  const int ti = rok ? row / H : 0;
  const int hh = rok ? row - ti * H : 0;
  const int lim = rok ? (p.causal ? max(0, L - qlen + ti + 1) : L) : 0;
  const int end_row = min(seg_end, lim);
  int end_min;  // keys every valid row of the wave sees: steps below need no mask
  {
    int v = rok ? end_row : 0x7fffffff;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = min(v, __shfl_xor(v, off));
    end_min = min(__builtin_amdgcn_readfirstlane(v), eff_end);
  }

  const float qs = p.q_scale ? *p.q_scale : 1.0f;
  const float ks = p.kv_scale ? *p.kv_scale : 1.0f;
  const float sl2 = p.softmax_scale * kLog2e * qs * ks;

  // ---- Q^T operand: lane (j, h) holds row j's dims 64c + 32h .. +31 (c = 8: rope) ----
  i32x8 qop[9];
  {
    const int64_t tok = t0 + ti;
    const int64_t qoff = tok * p.q_stride_token + (int64_t)hh * p.q_stride_head;
    const int64_t poff = p.q_pe ? tok * p.q_pe_stride_token + (int64_t)hh * p.q_pe_stride_head : qoff + kKvRank;
    if constexpr (!QB) {
      const uint8_t* qb = (const uint8_t*)p.q + qoff;
      const uint8_t* qr = (const uint8_t*)(p.q_pe ? p.q_pe : p.q) + poff;
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        const uint8_t* src = c < 8 ? qb + 64 * c + 32 * h : qr + 32 * h;
        const u32x4 lo = rok ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
        const u32x4 hi = rok ? *(const u32x4*)(src + 16) : u32x4{0, 0, 0, 0};
        qop[c] = __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
    } else {
      // bf16 q quantised here: code = e4m3 RNE of sat(q / q_scale)
      const unsigned short* qb = (const unsigned short*)p.q + qoff;
      const unsigned short* qr = (const unsigned short*)(p.q_pe ? p.q_pe : p.q) + poff;
      auto quant8 = [&](const unsigned short* src) -> u32x2 {
        const u32x4 v = rok ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = __uint_as_float(v[i] << 16);
          f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float y = __fdiv_rn(f[i], qs);
          f[i] = y != y ? y : fminf(fmaxf(y, -448.f), 448.f);
        }
        u32x2 o;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          int w = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * k], f[4 * k + 1], 0, false);
          w = __builtin_amdgcn_cvt_pk_fp8_f32(f[4 * k + 2], f[4 * k + 3], w, true);
          o[k] = (unsigned)w;
        }
        return o;
      };
#pragma unroll
      for (int c = 0; c < 9; ++c) {
        const unsigned short* src = c < 8 ? qb + 64 * c + 32 * h : qr + 32 * h;
        i32x8 x;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const u32x2 w = quant8(src + 8 * k);
          x[2 * k] = (int)w[0];
          x[2 * k + 1] = (int)w[1];
        }
        qop[c] = x;
      }
    }
  }

  // ---- DMA of one tile into ring slot b ----
  // Instruction i < kVw of wave w fills V rows 2m and 2m + 1, m = kVw w + i
  // (lanes 0-31 row 2m, lanes 32-63 row 2m + 1): lane l writes physical
  // chunk l % 32 and loads the logical chunk the swizzle puts there.  With
  // r = 2m + hb, chunk c ^ swz_w(r) = (c ^ 4 hb) ^ g(m) for the scalar
  // g(m) = 8 (m & 1) | 2 ((m >> 2) & 1) | ((m >> 1) & 1), so a lane's offset
  // is its fixed part u_v (XOR) the scalar 16 g(m), plus its row part h_v,
  // with the scalar row offset 1152 m in soffset.  Instruction kVw of waves
  // 0 and 1 fills rope rows 16w .. 16w + 15 (4 lanes per 64-byte row, chunk
  // c at c ^ ((row / 4) % 4)): the lane part r_v plus the scalar 9216 w.
  // The buffer descriptor covers the tile's valid rows only, so rows at or
  // past the valid count read as zeros (finite data the softmax masks) and a
  // tile past the piece's end (every offset out of range) fetches nothing.
  // tile_setup resolves the tile's page through a scalar cursor over the
  // page table (its scalar load is waited for there, before any LDS read is
  // in flight); dma_ins issues one of the wave's instructions, so the stream
  // spreads them over the P.V MFMAs.
  constexpr int kNDw = kVw + 1;  // instruction slots per wave (the rope one is empty for waves 2 and 3)
  constexpr int kNIo = kVw + (NW == 2 ? 1 : 0);  // instructions per tile of waves 2 and 3 (NW 2: of all)
  const int hb = lane >> 5;
  const int u_v = 16 * ((lane & 31) ^ (4 * hb));
  const int h_v = hb * kRowBytes;
  const int r_v = (lane >> 2) * kRowBytes + kKvRank + 16 * ((lane & 3) ^ ((lane >> 4) & 3));
  int cur_start = -1, cur_blk_i = 0, cur_in = 0, cached_blk_i = -1;
  int64_t cached_off = 0;
  // The next page's table entry is loaded when a page is entered, so the
  // scalar load is long back when the stream reaches that page.
  int pf_i = -1, pf_blk = 0;
  const int npages_tab = cap / p.block_size;
  auto table_entry = [&](int i) {
    return ((const __attribute__((address_space(4))) int*)p.block_table)[bt_base + (int64_t)i * p.bt_stride_col];
  };
  i32x4 t_rsrc;
  unsigned t_lbase = 0;
  auto tile_setup = [&](int k, int b) {
    t_lbase = lds_u32 + (unsigned)(b * kTileBytes);
    if (k >= ntiles) {
      t_rsrc = make_rsrc(p.kv, 0);  // past the piece: fetches nothing
      return;
    }
    const int tile_start = seg_start + k * TT;
    const int nvalid = min(TT, eff_end - tile_start);
    if (tile_start != cur_start) {
      cur_blk_i = tile_start / p.block_size;
      cur_in = tile_start - cur_blk_i * p.block_size;
    }
    if (cur_blk_i != cached_blk_i) {
      int blk = cur_blk_i == pf_i ? pf_blk : table_entry(cur_blk_i);
      if (blk < 0 || blk >= p.num_blocks) { blk = 0; bad = true; }
      cached_off = (int64_t)blk * p.block_size * kRowBytes;
      cached_blk_i = cur_blk_i;
      pf_i = cur_blk_i + 1 < npages_tab ? cur_blk_i + 1 : -1;
      if (pf_i >= 0) pf_blk = table_entry(pf_i);
    }
    t_rsrc = make_rsrc(p.kv + cached_off + (int64_t)cur_in * kRowBytes, nvalid * kRowBytes);
    cur_start = tile_start + TT;
    cur_in += TT;
    while (cur_in >= p.block_size) { cur_in -= p.block_size; ++cur_blk_i; }
  };
  auto dma_ins = [&](int i) {
    if (i < kVw) {
      const int m = kVw * wave + i;
      const int gm = 8 * (m & 1) | 2 * ((m >> 2) & 1) | ((m >> 1) & 1);
      dma_lds16(t_rsrc, t_lbase + m * 1024, (u_v ^ (16 * gm)) + h_v, 1152 * m);
    } else if (wave < 2) {
      dma_lds16(t_rsrc, t_lbase + kVRegion + wave * 1024, r_v, 9216 * wave);
    }
  };
  auto issue_tile = [&](int k, int b) {
    tile_setup(k, b);
#pragma unroll
    for (int i = 0; i < kNDw; ++i) dma_ins(i);
  };
  // Wait until at most `n` tile issues after the one awaited are in flight
  // (every issue, real or empty, is the same instructions).
  auto wait_issues = [&](auto n_tag) {
    constexpr int n = decltype(n_tag)::value;
    if (NW == 2 || wave >= 2) wait_vmcnt<n * kNIo>();
    else wait_vmcnt<n * kNDw>();
  };

  // ---- LDS reads ----
  // K: lane (token j, half h) reads the 32 bytes 64c + 32h .. +31 of row j
  // (logical chunks 4c + 2h, 4c + 2h + 1); the swizzle makes that chunk
  // pair (4 (c & 3) ^ (2h ^ swz_w(j))) (+1), i.e. byte offset
  // (k_b ^ 64 (c & 3)) + 256 (c >> 2) and that ^ 16.  The rope step reads the
  // rope row.
  const int k_b = j * 512 + 16 * ((2 * h) ^ swz_w(j));
  const int k_r = kVRegion + j * 64 + 16 * ((2 * h) ^ ((j >> 2) & 3));
  auto load_k = [&](const char* buf, int c) -> i32x8 {
    int o0, o1;
    if (c < 8) {
      o0 = (k_b ^ (64 * (c & 3))) + 256 * (c >> 2);
      o1 = o0 ^ 16;
    } else {
      o0 = k_r;
      o1 = k_r ^ 16;
    }
    const u32x4 lo = lds_load<u32x4>(buf, o0);
    const u32x4 hi = lds_load<u32x4>(buf, o1);
    return __builtin_bit_cast(i32x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  // V^T for dim block d: k-slot 32h' + 8q + e (q = 0, 1) of lane group G
  // (h' = G / 2) is token 16q + 8 (e / 4) + 4h' + e % 4, the token order of
  // the P^T operand below; k-slots 32h' + 16 .. +31 are zero.  Group G reads
  // dims 32d + 16 (G % 2) .. +15 of row e = (lane / 2) % 8, half lane % 2:
  // chunk (2 (d & 7) | (G & 1)) ^ swz_w(tv) at byte (v_b ^ 32 (d & 7)) +
  // 256 (d >> 3), and 16 tokens on at +8192.
  int v_b;
  {
    const int G = lane >> 4, e = (lane >> 1) & 7, jb = lane & 1;
    const int tv = 8 * (e >> 2) + 4 * (G >> 1) + (e & 3);
    v_b = tv * 512 + 16 * ((G & 1) ^ swz_w(tv)) + 8 * jb;
  }
  auto load_v = [&](const char* buf, int d, i32x8& v) {
    const int off = (v_b ^ (32 * (d & 7))) + 256 * (d >> 3);
    const i32x2 a = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(buf + off));
    const i32x2 b = __builtin_amdgcn_ds_read_tr8_b64_v2i32((LDS_AS i32x2*)(buf + off + 8192));
    v[0] = a[0]; v[1] = a[1]; v[2] = b[0]; v[3] = b[1];
  };

  // ---- the stream ----
  // The accumulator holds sum 2^(x - (m0 - kBias)) V over the keys so far,
  // m0 the row's reference: P is e4m3 of p = 2^(x - (m_run - kBias)) <= 2^8
  // with an integer running reference m_run that moves (to the ceiling of
  // the tile max) only past kLazy, and the P.V MFMA scales P by the E8M0
  // factor 2^(m_run - m0).  So the accumulator is only ever written by MFMAs
  // and needs no rescaling.  (The scaled MFMA takes 64 tokens: a 32-token
  // tile fills k-slots 0-15 of each lane half and zeros the rest, at half
  // the MFMA rate, so that three tiles of the ring stay in flight.)  m0 is
  // the ceiling of the row's first maximum; a row whose maximum later climbs
  // more than 64 units above it (far inside the E8M0 range, and keeping
  // 2^e V P inside fp32) sends the workgroup through the piece again with m0
  // the ceiling of the exact maximum (second pass).
  //
  // Software pipeline, one iteration per tile k (S(k) = its scores, computed
  // by the previous iteration):
  //   A  wait until tile k+1 has landed, then a barrier (every wave's share
  //      of it is in, and every wave is done with tile k-1's slot); resolve
  //      the page of tile k+NBUF-1;
  //   B  the QK MFMAs of tile k+1, with the softmax of S(k) (VALU) between
  //      them;
  //   C  the P.V MFMAs of tile k, with the DMA instructions of tile k+NBUF-1
  //      (into tile k-1's slot) between them.
  // The matrix pipe runs the MFMAs of a phase while the wave issues the
  // phase's other work.  Tiles past the piece's end are issued as empty
  // loads, so every wait counts the same instructions.
  wait_vmcnt<0>();  // q is in registers before the DMA stream starts
  f32x16 acc[16];
  float m_true = -INFINITY, m_run = -INFINITY, m0 = -INFINITY, l_run = 0.f, lh_run = 0.f;
  float m0_fixed = -INFINITY;  // second pass: the reference from the first pass's exact max
  constexpr int kPK = 3;       // K operands in flight ahead of their MFMA
  constexpr int kPV = 4;       // V^T operands in flight ahead of their MFMA
  // V^T and P^T operands keep their upper four registers at zero
  i32x8 vq[kPV];
#pragma unroll
  for (int i = 0; i < kPV; ++i) vq[i] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  i32x8 pop = i32x8{0, 0, 0, 0, 0, 0, 0, 0};

  // QK of one tile as 9 chained steps; between step c and c+1 the caller's
  // work(c) (c = 0..8) is issued, and work(-1) before the first.
  auto qk_tile = [&](const char* buf, f32x16& s, auto&& work) {
    i32x8 kq[kPK];
#pragma unroll
    for (int i = 0; i < kPK; ++i) kq[i] = load_k(buf, i);
    work(std::integral_constant<int, -1>{});
    __builtin_amdgcn_sched_barrier(0);
    auto step = [&](auto c_tag) {
      constexpr int c = decltype(c_tag)::value;
      const i32x8 cur = kq[c % kPK];
      if constexpr (c + kPK < 9) kq[c % kPK] = load_k(buf, c + kPK);
      qk_step_w32<c == 0, c == 8>(s, cur, qop[c]);
      work(c_tag);
      __builtin_amdgcn_sched_barrier(0);
    };
    step(std::integral_constant<int, 0>{});
    step(std::integral_constant<int, 1>{});
    step(std::integral_constant<int, 2>{});
    step(std::integral_constant<int, 3>{});
    step(std::integral_constant<int, 4>{});
    step(std::integral_constant<int, 5>{});
    step(std::integral_constant<int, 6>{});
    step(std::integral_constant<int, 7>{});
    step(std::integral_constant<int, 8>{});
  };
  auto no_work = [](auto) {};

  bool ovf = false;
  // One iteration of the pipeline for tile k: S(k) in s_cur, S(k+1) into s_next.
  auto iteration = [&](int k, const f32x16& s_cur, f32x16& s_next) {
    const bool has_next = k + 1 < ntiles;
    // ---- A ----
    wait_issues(std::integral_constant<int, NBUF - 3>{});  // tile k+1 in
    if constexpr (NW > 1) __syncthreads();
    tile_setup(k + NBUF - 1, (k + NBUF - 1) % NBUF);
    __builtin_amdgcn_sched_barrier(0);

    // ---- B: softmax of S(k) between the QK steps of tile k+1 ----
    // Register r of S holds token 8 (r / 4) + 4h + r % 4 of the tile (the
    // row's other 16 are in lane l ^ 32).
    const int tile_start = seg_start + k * TT;
    const int vis = end_row - tile_start - 4 * h;  // register r is visible iff 8 (r / 4) + r % 4 < vis
    float x[16];
    float mloc = -INFINITY;
    float e = 0.f, m_ref = 0.f, psum = 0.f, hsum = 0.f;
    int w[4];
    auto softmax_part = [&](auto c_tag) {
      constexpr int c = decltype(c_tag)::value;
      if constexpr (c == -1) {
        if (tile_start + TT <= end_min) {
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = s_cur[i];
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = (8 * (i >> 2) + (i & 3)) < vis ? s_cur[i] : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, x[i]);
      } else if constexpr (c == 0) {
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
        mloc = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])) * sl2;
        m_true = fmaxf(m_true, mloc);
        if (mloc > m_run + Lazy<true>::kLazy) m_run = ceilf(mloc);
        if (m0 == -INFINITY) m0 = m_run;
        const bool live = m_run != -INFINITY;
        e = live ? m_run - m0 : 0.f;  // an integer >= 0
        ovf |= e > 64.f;              // keeps 2^e V P (and l) far inside fp32
        // p = 2^(s sl2 - m_ref); a row without a visible key yet has every
        // score at -inf and takes m_ref 0 (p = 0)
        m_ref = live ? m_run - Lazy<true>::kBias : 0.f;
      } else if constexpr (c >= 1 && c <= 4) {
#pragma unroll
        for (int i = 4 * (c - 1); i < 4 * c; ++i) x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sl2, -m_ref));
      } else if constexpr (c == 6) {
        // P^T in e4m3: k-slot 32h + 4m + i (byte 4m + i) is token 8m + 4h + i,
        // register 4m + i
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          w[q] = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * q], x[4 * q + 1], 0, false);
          w[q] = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * q + 2], x[4 * q + 3], w[q], true);
        }
      }
    };
    // The row sums (exact p, and p as rounded to e4m3) go between the P.V
    // steps.
    auto sums_part = [&](int d) {
      if (d == 1) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = x[i] + x[i + 8];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] += t[i + 4];
        psum = (t[0] + t[2]) + (t[1] + t[3]);
      } else if (d == 3) {
        float t[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8(w[q], false), b = __builtin_amdgcn_cvt_pk_f32_fp8(w[q], true);
          t[q] = (a[0] + a[1]) + (b[0] + b[1]);
        }
        hsum = (t[0] + t[1]) + (t[2] + t[3]);
      } else if (d == 5) {
        const float se = __builtin_amdgcn_exp2f(e);  // exact: e is a small integer
        l_run += se * psum;
        lh_run += se * hsum;
      }
    };
    if (has_next) {
      qk_tile(lds[(k + 1) % NBUF], s_next, softmax_part);
    } else {
      softmax_part(std::integral_constant<int, -1>{});
      softmax_part(std::integral_constant<int, 0>{});
      softmax_part(std::integral_constant<int, 1>{});
      softmax_part(std::integral_constant<int, 2>{});
      softmax_part(std::integral_constant<int, 3>{});
      softmax_part(std::integral_constant<int, 4>{});
      softmax_part(std::integral_constant<int, 6>{});
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) pop[q] = w[q];
    const int scale_b = 127 + (int)fminf(e, 64.f);  // E8M0 2^e per row
    const int scale_a = opaque(127);                // E8M0 1 for V^T
    __builtin_amdgcn_sched_barrier(0);

    // ---- C: O^T += 2^e V^T . P^T over 16 dim blocks, with the DMA of tile
    // k+NBUF-1 between them ----
    const char* buf = lds[k % NBUF];
#pragma unroll
    for (int i = 0; i < kPV; ++i) load_v(buf, i, vq[i]);
#pragma unroll
    for (int d = 0; d < 16; ++d) {
      const i32x8 cur = vq[d % kPV];
      if (d + kPV < 16) load_v(buf, d + kPV, vq[d % kPV]);
      pv_step_w32(acc[d], cur, pop, scale_a, scale_b);
#pragma unroll
      for (int i = 0; i < kNDw; ++i)
        if (i * 16 / kNDw == d) dma_ins(i);
      sums_part(d);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] = f32x16{};
    m_true = -INFINITY;
    m_run = m0 = m0_fixed;
    l_run = lh_run = 0.f;
    ovf = false;
    cur_start = -1;
    cached_blk_i = -1;
    pf_i = -1;
    if (ntiles > 0) {
#pragma unroll
      for (int k = 0; k < NBUF - 1; ++k) issue_tile(k, k);
      f32x16 s_a, s_b;
      wait_issues(std::integral_constant<int, NBUF - 2>{});  // tile 0 in
      if constexpr (NW > 1) __syncthreads();
      qk_tile(lds[0], s_a, no_work);
      // two iterations per trip, so S(k) and S(k+1) alternate between s_a
      // and s_b without copies
      for (int k = 0; k < ntiles; ++k) {
        iteration(k, s_a, s_b);
        s_a = s_b;
      }
      wait_vmcnt<0>();  // the empty issues past the end have landed
    }
    mfma_settle_w32();  // the accumulator is read (or cleared) after this
    if (__syncthreads_or(ovf ? 1 : 0) == 0) break;
    // some row outran the reference's range: again, from the exact maximum
    m0_fixed = ceilf(m_true);
  }

  // ---- the piece's result ----
  // Row totals over the two lanes of a row; the accumulator and l refer to
  // m0 - kBias: rescale to the exact max, and by l / lh for the rounded P.
  auto pair_sum = [](float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
  };
  float l_tot = pair_sum(l_run);
  const float lh_tot = pair_sum(lh_run);
  const float f0 = (m_true == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f((m0 - Lazy<true>::kBias) - m_true);
  const float fo = lh_tot > 0.f ? f0 * (l_tot / lh_tot) : f0;
  l_tot *= f0;
  bad = __syncthreads_or(bad ? 1 : 0) != 0;
  if (!rok) return;
  float mult, stat0;
  char* dst;
  float* stat0_p;
  float* stat1_p = nullptr;
  int kind;  // 0 bf16, 1 fp16, 2 fp32
  if (pc.mode == kOutFinal) {
    // normalised output and natural-log LSE; a sink joins as one more logit
    // with a zero value
    const bool has = m_true > -INFINITY;
    float lse = has ? kLn2 * (m_true + __log2f(l_tot)) : -INFINITY;
    mult = has ? ks / l_tot : 0.f;
    if (p.sinks) {
      const float nl = logaddexp_f(lse, p.sinks[hh]);
      mult = has ? mult * expf(lse - nl) : 0.f;
      lse = nl;
    }
    if (bad) { lse = __builtin_nanf(""); mult = __builtin_nanf(""); }
    const int64_t orow = (int64_t)(t0 + ti) * H + hh;
    kind = p.out_dtype;
    dst = (char*)p.out + orow * kKvRank * (kind == 2 ? 4 : 2);
    stat0 = lse;
    stat0_p = p.lse + orow;
  } else {
    const int64_t slot = pc.mode == kOutSegment ? ((int64_t)(t0 + ti) * H + hh) * p.num_segments + pc.s
                                                : pc.prow0 + wave * 32 + j;
    mult = ks;
    // partials in fp32, or in bf16 when the fused call's output is 16-bit
    if (!p.piece_bf16) {
      kind = 2;
      dst = (char*)(p.seg_out + slot * kKvRank);
    } else {
      kind = 0;
      dst = (char*)(p.piece_out + slot * kKvRank);
    }
    stat0 = bad ? __builtin_nanf("") : m_true;
    stat0_p = p.seg_max + slot;
    stat1_p = p.seg_sum + slot;
  }
  mult *= fo;
  store_w32(acc, h, mult, dst, kind);
  if (h == 0) {
    *stat0_p = stat0;
    if (stat1_p) *stat1_p = l_tot;
  }
}

// ---------------------------------------------------------------------------
// Wide waves (bf16): 32 query rows per wave
// ---------------------------------------------------------------------------
// The bf16 counterpart of the wide fp8 body.  A wave owns 32 rows and works on
// 32x32 blocks with v_mfma_f32_32x32x16_bf16 (A lane l = row l%32, k
// 8(l/32)..+7; B lane l = column l%32, the same k; D as for the fp8 body):
//   S^T[token, row] = K . Q^T     32 latent steps of 16 dims + 4 rope steps
//   O^T[dim, row]  += V^T . P^T   16 blocks of 32 dims x 2 steps of 16 tokens
// Q^T takes 144 registers per lane and the accumulator the 256 AGPRs.  Each
// K or V byte a wave reads from LDS feeds 32 rows (the 16-row bf16 shapes
// feed 16), and both products run on the full-rate 32x32x16 instruction.
//
// The tile (32 tokens, 36 KiB) keeps the regions of KvFmt<false> (V rows of
// 1024 B, rope rows of 128 B at +32 KiB, rope chunks swizzled by swz_r) with
// its own V swizzle: chunk c of row r sits at c ^ swz_b(r).  swz_b's low four
// bits are a bijection of r's, so the 16 rows one K read serves per pass land
// in 16 distinct bank groups; a 16-bit transpose read serves 4 rows x 4
// chunks per 32-lane pass, and those rows (r & 3 distinct) land in distinct
// chunk quads.
//
// Softmax: P^T = bf16 of p = 2^(x - m0) for a fixed reference m0 per row, the
// ceiling of the row's first maximum.  bf16 keeps fp32's exponent range, so p
// needs no running rescale while the row's maximum stays within kBound of m0
// (p <= 2^kBound); a row that climbs further sends the workgroup through the
// piece again with m0 the ceiling of the exact maximum (second pass), as in
// the fp8 body.  The accumulator is only ever written by MFMAs.
__device__ __forceinline__ int swz_b(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }

// One step of S^T = K . Q^T (16 dims, bf16), result in VGPRs; wait states as
// for qk_step_w32.
template <bool FIRST, bool LAST>
__device__ __forceinline__ void qk_step_w32b(f32x16& s, const bf16x8& k, const bf16x8& q) {
  static_assert(!(FIRST && LAST), "a tile has 36 steps");
  if constexpr (FIRST) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(s) : "v"(k), "v"(q));
  } else if constexpr (LAST) {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0\n\ts_nop 15\n\ts_nop 7"
                 : "+v"(s) : "v"(k), "v"(q));
  } else {
    asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(s) : "v"(k), "v"(q));
  }
}

// One P.V step O^T += V^T . P^T (16 tokens, bf16) on an AGPR accumulator;
// wait states as for pv_step_w32.
__device__ __forceinline__ void pv_step_w32b(f32x16& acc, const bf16x8& v, const bf16x8& pt) {
  asm volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(pt));
}

template <int NW, int NBUF>
__device__ __forceinline__ void run_piece_w32b(const SegmentLaunch& p, char (*lds)[36864], unsigned lds_u32,
                                               const Piece& pc) {
  constexpr int TT = 32;                  // tokens per DMA tile (ring slot)
  constexpr int kRowBytes = 1152;
  constexpr int kTileBytes = TT * kRowBytes;
  constexpr int kVRegion = TT * 1024;
  constexpr int kRowsWG = 32 * NW;
  constexpr int kVw = TT / NW;            // V rows per wave per tile (one instruction each)
  constexpr int kRw = 4 / NW;             // rope instructions (8 rows each) per wave per tile
  constexpr int kNDw = kVw + kRw;         // DMA instructions per wave per tile
  constexpr float kBound = 32.f;          // p <= 2^kBound before a second pass
  static_assert(kTileBytes == 36864, "bf16 32-token tiles");
  static_assert(NW == 2 || NW == 4, "the wide body runs two or four waves");
  static_assert(NBUF >= 3, "a tile in the P.V phase, one in the QK phase, and one in flight");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int j = lane & 31;  // the lane's query row in the wave
  const int h = lane >> 5;

  const int r = pc.r, t0 = pc.t0, qlen = pc.qlen, L = pc.L;
  const int H = p.num_heads;
  const int M = qlen * H;
  const int row0 = pc.row0;
  int64_t bt_base;
  int cap;
  page_list(p, r, &bt_base, &cap);
  bt_base = __builtin_amdgcn_readfirstlane((int)(bt_base & 0xffffffff)) |
            ((int64_t)__builtin_amdgcn_readfirstlane((int)(bt_base >> 32)) << 32);
  cap = __builtin_amdgcn_readfirstlane(cap);
  bool bad = L > cap;
  const int seg_start = pc.seg_start;
  const int seg_end = pc.seg_end;
  const int last_row = min(row0 + kRowsWG, M) - 1;
  const int lim_wg = p.causal ? (L - qlen + last_row / H + 1) : L;
  const int eff_end = min(min(seg_end, lim_wg), cap);
  const int ntiles = eff_end > seg_start ? cdiv(eff_end - seg_start, TT) : 0;

  // The lane's query row (lanes l and l + 32 hold the same row).
  const int row = row0 + wave * 32 + j;
  const bool rok = row < M;
  const int ti = rok ? row / H : 0;
  const int hh = rok ? row - ti * H : 0;
  const int lim = rok ? (p.causal ? max(0, L - qlen + ti + 1) : L) : 0;
  const int end_row = min(seg_end, lim);
  int end_min;  // keys every valid row of the wave sees: tiles below need no mask
  {
    int v = rok ? end_row : 0x7fffffff;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) v = min(v, __shfl_xor(v, off));
    end_min = min(__builtin_amdgcn_readfirstlane(v), eff_end);
  }

  const float qs = p.q_scale ? *p.q_scale : 1.0f;
  const float ks = p.kv_scale ? *p.kv_scale : 1.0f;
  const float sl2 = p.softmax_scale * kLog2e * qs * ks;

  // ---- Q^T operand: lane (j, h) holds row j's dims 16c + 8h .. +7 (c >= 32: rope) ----
  bf16x8 qop[36];
  {
    const int64_t tok = t0 + ti;
    const int64_t qoff = tok * p.q_stride_token + (int64_t)hh * p.q_stride_head;
    const int64_t poff = p.q_pe ? tok * p.q_pe_stride_token + (int64_t)hh * p.q_pe_stride_head : qoff + kKvRank;
    const __bf16* qb = (const __bf16*)p.q + qoff;
    const __bf16* qr = (const __bf16*)(p.q_pe ? p.q_pe : p.q) + poff;
#pragma unroll
    for (int c = 0; c < 36; ++c) {
      const __bf16* src = c < 32 ? qb + 16 * c + 8 * h : qr + 16 * (c - 32) + 8 * h;
      const u32x4 v = rok ? *(const u32x4*)src : u32x4{0, 0, 0, 0};
      qop[c] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // ---- DMA of one tile into ring slot b ----
  // Instruction i < kVw of wave w fills V row m = kVw w + i: lane l writes
  // physical chunk l and loads logical chunk l ^ swz_b(m) (the scalar row
  // offset 1152 m in soffset).  Instruction kVw + i fills rope rows 8n ..
  // 8n + 7, n = kRw w + i: lane l writes chunk l % 8 of row 8n + l / 8 and
  // loads logical chunk (l % 8) ^ swz_r(8n + l / 8) = (l % 8) ^ (l / 16) ^
  // 4 (n % 2).  The buffer descriptor covers the tile's valid rows only (rows
  // past them read as zeros, which the softmax masks; a tile past the piece's
  // end fetches nothing).  tile_setup resolves the tile's page through a
  // scalar cursor over the page table; dma_ins issues one instruction, so the
  // stream spreads them over the P.V MFMAs.
  const int u_v = 16 * lane;
  const int r_v = (lane >> 3) * kRowBytes + kKvRank * 2 + 16 * ((lane & 7) ^ (lane >> 4));
  int cur_start = -1, cur_blk_i = 0, cur_in = 0, cached_blk_i = -1;
  int64_t cached_off = 0;
  int pf_i = -1, pf_blk = 0;
  const int npages_tab = cap / p.block_size;
  auto table_entry = [&](int i) {
    return ((const __attribute__((address_space(4))) int*)p.block_table)[bt_base + (int64_t)i * p.bt_stride_col];
  };
  i32x4 t_rsrc;
  unsigned t_lbase = 0;
  auto tile_setup = [&](int k, int b) {
    t_lbase = lds_u32 + (unsigned)(b * kTileBytes);
    if (k >= ntiles) {
      t_rsrc = make_rsrc(p.kv, 0);  // past the piece: fetches nothing
      return;
    }
    const int tile_start = seg_start + k * TT;
    const int nvalid = min(TT, eff_end - tile_start);
    if (tile_start != cur_start) {
      cur_blk_i = tile_start / p.block_size;
      cur_in = tile_start - cur_blk_i * p.block_size;
    }
    if (cur_blk_i != cached_blk_i) {
      int blk = cur_blk_i == pf_i ? pf_blk : table_entry(cur_blk_i);
      if (blk < 0 || blk >= p.num_blocks) { blk = 0; bad = true; }
      cached_off = (int64_t)blk * p.block_size * kRowBytes;
      cached_blk_i = cur_blk_i;
      pf_i = cur_blk_i + 1 < npages_tab ? cur_blk_i + 1 : -1;
      if (pf_i >= 0) pf_blk = table_entry(pf_i);
    }
    t_rsrc = make_rsrc(p.kv + cached_off + (int64_t)cur_in * kRowBytes, nvalid * kRowBytes);
    cur_start = tile_start + TT;
    cur_in += TT;
    while (cur_in >= p.block_size) { cur_in -= p.block_size; ++cur_blk_i; }
  };
  auto dma_ins = [&](int i) {
    if (i < kVw) {
      const int m = kVw * wave + i;
      dma_lds16(t_rsrc, t_lbase + m * 1024, u_v ^ (16 * swz_b(m)), kRowBytes * m);
    } else {
      const int n = kRw * wave + (i - kVw);
      dma_lds16(t_rsrc, t_lbase + kVRegion + n * 1024, r_v ^ (64 * (n & 1)), 8 * kRowBytes * n);
    }
  };
  auto issue_tile = [&](int k, int b) {
    tile_setup(k, b);
#pragma unroll
    for (int i = 0; i < kNDw; ++i) dma_ins(i);
  };
  // Wait until at most `n` tile issues after the one awaited are in flight
  // (every wave issues the same kNDw instructions per tile, real or empty).
  auto wait_issues = [&](auto n_tag) {
    constexpr int n = decltype(n_tag)::value;
    wait_vmcnt<n * kNDw>();
  };

  // ---- LDS reads ----
  // K: lane (token j, half h) reads the 16 bytes of dims 16c + 8h .. +7 of
  // row j, logical chunk 2c + h: byte (k_b ^ 32 (c & 7)) + 256 (c >> 3) in
  // the V region, k_r ^ 32 (c - 32) in the rope region.
  const int k_b = j * 1024 + 16 * (h ^ swz_b(j));
  const int k_r = kVRegion + j * 128 + 16 * (h ^ KvFmt<false>::swz_r(j));
  auto load_k = [&](const char* buf, int c) -> bf16x8 {
    const int off = c < 32 ? (k_b ^ (32 * (c & 7))) + 256 * (c >> 3) : k_r ^ (32 * (c - 32));
    return lds_load<bf16x8>(buf, off);
  };
  // V^T for dim block d, step s: k-slots 0-3 of lane half h' are tokens
  // 16s + 4h' + e and k-slots 4-7 tokens 16s + 8 + 4h' + e (e = 0..3): the
  // token order of the P^T operand below.  Lane 4i + jj of 16-lane group G
  // (h' = G / 2) reads row 16s + 4h' + i (then + 8), dims 32d + 16 (G % 2) +
  // 4jj .. +3: logical chunk 4d + 2 (G % 2) + jj / 2, half jj % 2.  Row + 8
  // flips bit 1 of swz_b, row + 16 leaves it.
  int v_b;
  {
    const int G = lane >> 4, i = (lane >> 2) & 3, jj = lane & 3;
    const int ra = 4 * (G >> 1) + i;
    v_b = ra * 1024 + 8 * (jj & 1) + 16 * ((2 * (G & 1) + (jj >> 1)) ^ swz_b(ra));
  }
  auto load_v = [&](const char* buf, int d, int s) -> bf16x8 {
    const int oa = (v_b ^ (64 * (d & 3))) + 256 * (d >> 2) + 16384 * s;
    const int ob = ((v_b ^ 32) ^ (64 * (d & 3))) + 256 * (d >> 2) + 16384 * s + 8192;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(buf + oa));
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4*)(buf + ob));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
  };

  // ---- the stream ----
  // Software pipeline, one iteration per tile k (S(k) computed by the
  // previous iteration), as in the fp8 body:
  //   A  wait until tile k+1 has landed, then a barrier; resolve the page of
  //      tile k+NBUF-1;
  //   B  the QK MFMAs of tile k+1, with the softmax of S(k) between them;
  //   C  the P.V MFMAs of tile k, with the DMA of tile k+NBUF-1 (into tile
  //      k-1's slot) between them.
  wait_vmcnt<0>();  // q is in registers before the DMA stream starts
  f32x16 acc[16];
  float m_true = -INFINITY, m0 = -INFINITY, l_run = 0.f;
  float m0_fixed = -INFINITY;  // second pass: the reference from the first pass's exact max
  constexpr int kPK = 3;       // K operands in flight ahead of their MFMA
  constexpr int kPV = 4;       // V^T operands in flight ahead of their MFMA

  // QK of one tile as 36 chained steps; between step c and c+1 the caller's
  // work(c) is issued, and work(-1) before the first.
  auto qk_tile = [&](const char* buf, f32x16& s, auto&& work) {
    bf16x8 kq[kPK];
#pragma unroll
    for (int i = 0; i < kPK; ++i) kq[i] = load_k(buf, i);
    work(std::integral_constant<int, -1>{});
    __builtin_amdgcn_sched_barrier(0);
    auto step = [&](auto c_tag) {
      constexpr int c = decltype(c_tag)::value;
      const bf16x8 cur = kq[c % kPK];
      if constexpr (c + kPK < 36) kq[c % kPK] = load_k(buf, c + kPK);
      qk_step_w32b<c == 0, c == 35>(s, cur, qop[c]);
      work(c_tag);
      __builtin_amdgcn_sched_barrier(0);
    };
    unroll_seq(step, std::make_integer_sequence<int, 36>{});
  };
  auto no_work = [](auto) {};

  bool ovf = false;
  auto iteration = [&](int k, const f32x16& s_cur, f32x16& s_next) {
    const bool has_next = k + 1 < ntiles;
    // ---- A ----
    wait_issues(std::integral_constant<int, NBUF - 3>{});  // tile k+1 in
    __syncthreads();
    tile_setup(k + NBUF - 1, (k + NBUF - 1) % NBUF);
    __builtin_amdgcn_sched_barrier(0);

    // ---- B: softmax of S(k) between the QK steps of tile k+1 ----
    // Register r of S holds token 8 (r / 4) + 4h + r % 4 of the tile (the
    // row's other 16 are in lane l ^ 32).
    const int tile_start = seg_start + k * TT;
    const int vis = end_row - tile_start - 4 * h;  // register r is visible iff 8 (r / 4) + r % 4 < vis
    float x[16];
    float mloc = -INFINITY, m_ref = 0.f;
    bf16x8 pop[2];
    auto softmax_part = [&](auto c_tag) {
      constexpr int c = decltype(c_tag)::value;
      if constexpr (c == -1) {
        if (tile_start + TT <= end_min) {
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = s_cur[i];
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) x[i] = (8 * (i >> 2) + (i & 3)) < vis ? s_cur[i] : -INFINITY;
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) mloc = fmaxf(mloc, x[i]);
      } else if constexpr (c == 0) {
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(mloc), __float_as_uint(mloc), false, false);
        mloc = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1])) * sl2;
        m_true = fmaxf(m_true, mloc);
        if (m0 == -INFINITY && mloc > -INFINITY) m0 = ceilf(mloc);
        ovf |= mloc > m0 + kBound;
        // p = 2^(s sl2 - m_ref); a row without a visible key yet has every
        // score at -inf and takes m_ref 0 (p = 0)
        m_ref = m0 > -INFINITY ? m0 : 0.f;
      } else if constexpr (c >= 1 && c <= 4) {
#pragma unroll
        for (int i = 4 * (c - 1); i < 4 * c; ++i) x[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[i], sl2, -m_ref));
      } else if constexpr (c == 6) {
        // P^T of step s: k-slot e is register 8s + e (token 16s + 8 (e / 4) + 4h + e % 4)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
          for (int e = 0; e < 8; ++e) pop[s][e] = (__bf16)x[8 * s + e];
      } else if constexpr (c == 8) {
        float t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) t[i] = x[i] + x[i + 8];
#pragma unroll
        for (int i = 0; i < 4; ++i) t[i] += t[i + 4];
        l_run += (t[0] + t[2]) + (t[1] + t[3]);
      }
    };
    if (has_next) {
      qk_tile(lds[(k + 1) % NBUF], s_next, softmax_part);
    } else {
      softmax_part(std::integral_constant<int, -1>{});
      softmax_part(std::integral_constant<int, 0>{});
      softmax_part(std::integral_constant<int, 1>{});
      softmax_part(std::integral_constant<int, 2>{});
      softmax_part(std::integral_constant<int, 3>{});
      softmax_part(std::integral_constant<int, 4>{});
      softmax_part(std::integral_constant<int, 6>{});
      softmax_part(std::integral_constant<int, 8>{});
    }
    __builtin_amdgcn_sched_barrier(0);

    // ---- C: O^T += V^T . P^T over 16 dim blocks x 2 token steps, with the
    // DMA of tile k+NBUF-1 between them ----
    const char* buf = lds[k % NBUF];
    bf16x8 vq[kPV];
#pragma unroll
    for (int i = 0; i < kPV; ++i) vq[i] = load_v(buf, i >> 1, i & 1);
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const bf16x8 cur = vq[t % kPV];
      if (t + kPV < 32) vq[t % kPV] = load_v(buf, (t + kPV) >> 1, (t + kPV) & 1);
      pv_step_w32b(acc[t >> 1], cur, pop[t & 1]);
#pragma unroll
      for (int i = 0; i < kNDw; ++i)
        if (i * 32 / kNDw == t) dma_ins(i);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int d = 0; d < 16; ++d) acc[d] = f32x16{};
    m_true = -INFINITY;
    m0 = m0_fixed;
    l_run = 0.f;
    ovf = false;
    cur_start = -1;
    cached_blk_i = -1;
    pf_i = -1;
    if (ntiles > 0) {
#pragma unroll
      for (int k = 0; k < NBUF - 1; ++k) issue_tile(k, k);
      f32x16 s_a, s_b;
      wait_issues(std::integral_constant<int, NBUF - 2>{});  // tile 0 in
      __syncthreads();
      qk_tile(lds[0], s_a, no_work);
      for (int k = 0; k < ntiles; ++k) {
        iteration(k, s_a, s_b);
        s_a = s_b;
      }
      wait_vmcnt<0>();  // the empty issues past the end have landed
    }
    mfma_settle_w32();  // the accumulator is read (or cleared) after this
    if (__syncthreads_or(ovf ? 1 : 0) == 0) break;
    // some row outran the reference's range: again, from the exact maximum
    m0_fixed = ceilf(m_true);
  }

  // ---- the piece's result ----
  // Row totals over the two lanes of a row; the accumulator and l refer to
  // m0: rescale to the exact max.
  auto pair_sum = [](float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(a[0]) + __uint_as_float(a[1]);
  };
  float l_tot = pair_sum(l_run);
  const float f0 = (m_true == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m0 - m_true);
  l_tot *= f0;
  bad = __syncthreads_or(bad ? 1 : 0) != 0;
  if (!rok) return;
  float mult, stat0;
  char* dst;
  float* stat0_p;
  float* stat1_p = nullptr;
  int kind;  // 0 bf16, 1 fp16, 2 fp32
  if (pc.mode == kOutFinal) {
    // normalised output and natural-log LSE; a sink joins as one more logit
    // with a zero value
    const bool has = m_true > -INFINITY;
    float lse = has ? kLn2 * (m_true + __log2f(l_tot)) : -INFINITY;
    mult = has ? ks / l_tot : 0.f;
    if (p.sinks) {
      const float nl = logaddexp_f(lse, p.sinks[hh]);
      mult = has ? mult * expf(lse - nl) : 0.f;
      lse = nl;
    }
    if (bad) { lse = __builtin_nanf(""); mult = __builtin_nanf(""); }
    const int64_t orow = (int64_t)(t0 + ti) * H + hh;
    kind = p.out_dtype;
    dst = (char*)p.out + orow * kKvRank * (kind == 2 ? 4 : 2);
    stat0 = lse;
    stat0_p = p.lse + orow;
  } else {
    const int64_t slot = pc.mode == kOutSegment ? ((int64_t)(t0 + ti) * H + hh) * p.num_segments + pc.s
                                                : pc.prow0 + wave * 32 + j;
    mult = ks;
    if (!p.piece_bf16) {
      kind = 2;
      dst = (char*)(p.seg_out + slot * kKvRank);
    } else {
      kind = 0;
      dst = (char*)(p.piece_out + slot * kKvRank);
    }
    stat0 = bad ? __builtin_nanf("") : m_true;
    stat0_p = p.seg_max + slot;
    stat1_p = p.seg_sum + slot;
  }
  mult *= f0;
  store_w32(acc, h, mult, dst, kind);
  if (h == 0) {
    *stat0_p = stat0;
    if (stat1_p) *stat1_p = l_tot;
  }
}

// Two 16-row groups per wave run as a wide body (contiguous tiles).
template <bool FP8, int RG, bool CONTIG>
constexpr bool kWide = RG == 2 && CONTIG;

// Segment kernel: one workgroup per (segment, request, row chunk); the key
// partition is the segment formula of the merge page's module description
// (span = cdiv(len, S * TILE) * TILE; segment s = [s * span, min((s+1) * span, len))).
template <bool FP8, int NW, int RG, int NBUF, bool CONTIG, int TT, int OCC, bool QB>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(OCC, 8))) void segment_kernel(
    SegmentLaunch p) {
  __shared__ __attribute__((aligned(1024))) char lds[NBUF][TileGeom<FP8, TT>::kTileBytes];
  __shared__ int idx_buf[CONTIG ? 1 : kIdxCap];
  constexpr int kRowsWG = 16 * RG * NW;
  const int s = blockIdx.x;
  const int r = blockIdx.y;
  const int chunk = blockIdx.z;
  int t0 = r, qlen = 1;
  if (p.qo_indptr) {
    const int64_t a = p.qo_indptr[r], b = p.qo_indptr[r + 1];
    if (a < 0 || b < a || b - a > p.max_qlen || b > p.num_tokens) {
      // Malformed request: the batch tokens its range names get NaN
      // statistics in this segment's slot (the merge then reports NaN for
      // them, as for a length past the block table) instead of partials
      // that were never written.
      if (chunk == 0) {
        const int64_t lo = a < 0 ? 0 : a;
        const int64_t hi = b > p.num_tokens ? p.num_tokens : b;
        for (int64_t i = lo * p.num_heads + threadIdx.x; i < hi * p.num_heads; i += blockDim.x)
          p.seg_max[i * p.num_segments + s] = __builtin_nanf("");
      }
      return;
    }
    t0 = (int)a;
    qlen = (int)(b - a);
  }
  const int row0 = chunk * kRowsWG;
  if (row0 >= qlen * p.num_heads) return;
  const int L = p.seq_lens[r];
  if (L <= 0) return;  // no valid segment
  const int span = cdiv(L, p.num_segments * p.tile) * p.tile;
  const int seg_start = s * span;
  if (seg_start >= L) return;  // invalid segment: its slot is never read
  Piece pc;
  pc.r = r; pc.t0 = t0; pc.qlen = qlen; pc.L = L; pc.row0 = row0;
  pc.seg_start = seg_start; pc.seg_end = min(seg_start + span, L);
  pc.mode = kOutSegment; pc.s = s; pc.prow0 = 0; pc.phase = 0;
  if constexpr (kWide<FP8, RG, CONTIG> && FP8)
    run_piece_w32<NW, NBUF, QB>(p, lds, lds_address(&lds[0][0]), pc);
  else if constexpr (kWide<FP8, RG, CONTIG>)
    run_piece_w32b<NW, NBUF>(p, lds, lds_address(&lds[0][0]), pc);
  else
    run_piece<FP8, NW, RG, NBUF, CONTIG, TT, OCC, 1, QB>(p, lds, lds_address(&lds[0][0]), idx_buf, pc);
}

// Work units of request r for a workgroup shape of rows_wg rows and TT-token
// tiles: (row chunks) x (tiles of its keys).  0 for an empty or malformed
// request (the merge writes its empty rows).
__device__ __forceinline__ int request_units(const SegmentLaunch& p, int r, int rows_wg, int tt, int* t0_out,
                                             int* qlen_out, int* len_out) {
  int t0 = r, qlen = 1;
  if (p.qo_indptr) {
    t0 = p.qo_indptr[r];
    qlen = p.qo_indptr[r + 1] - t0;
  }
  const int L = p.seq_lens[r];
  *t0_out = t0; *qlen_out = qlen; *len_out = L;
  if (t0 < 0 || qlen <= 0 || qlen > p.max_qlen || t0 + qlen > p.num_tokens || L <= 0) return 0;
  return cdiv(qlen * p.num_heads, rows_wg) * cdiv(L, tt);
}

// Per-token records for the merge, written by one wave of the split kernel
// (lane = request): for each query token t of the request, {first token of
// the request, its unit offset, units per row chunk (0: no keys), total units
// W} at tok_rec[4 t].  With them a merge wave finds its pieces, or that its
// row was finished, in one load instead of a search over the query ranges.
// They are only complete when the ranges tile the tokens: every qlen in
// [0, max_qlen] here, and qo_indptr[0] == 0, qo_indptr[R] == T checked by the
// caller, which then sets the flag word tok_rec[4 T]; otherwise the merge
// searches.  Returns whether this lane's request passed its check.
__device__ __forceinline__ bool write_token_records(const SegmentLaunch& p, bool real, int t0, int ql, int units,
                                                    int offset, int W, int rows_wg) {
  const bool ok = !real || (ql >= 0 && ql <= p.max_qlen);
  const int n = (real && ok) ? ql : 0;
  const int chunks = n > 0 ? cdiv(n * p.num_heads, rows_wg) : 1;
  const i32x4 rec = {t0, offset, units > 0 ? units / chunks : 0, W};
  for (int j = 0; __ballot(j < n); ++j) {
    const int t = t0 + j;
    if (j < n && t >= 0 && t < p.num_tokens) *(i32x4*)(p.tok_rec + 4 * (int64_t)t) = rec;
  }
  return ok;
}

// Logical index of physical workgroup b of G when workgroup b runs on XCD
// b % 8: XCD x holds logical indices [x q + min(x, r), ...) for G = 8 q + r,
// in dispatch order (a bijection of [0, G)).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_major(int b, int G) {
  const int x = b % kXcds, i = b / kXcds, q = G / kXcds, r = G % kXcds;
  return x * q + min(x, r) + i;
}

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Balanced split kernel (the fused decode's first stage).  The work of the
// whole batch is laid out as one sequence of units, request by request, row
// chunk by row chunk, tile by tile; workgroup g of G takes units
// [g W / G, (g+1) W / G), so every workgroup streams the same number of tiles
// whatever the lengths.  A (request, row chunk) whose tiles all fall in one
// workgroup is finished there (output and LSE written); one cut by a range
// boundary leaves base-2 partials in the workgroup's slot 0 (its first piece)
// or slot 1 (its last piece) for the merge.  Workgroup 0 also stores the
// per-request unit offsets the merge uses to find the pieces.
// With KS > 1 k-split waves a workgroup's KS waves share each of its pieces
// tile by tile (one row group) and combine their states at the piece's end,
// so a workgroup covers KS times the units with the same number of pieces.
template <bool FP8, int NW, int RG, int NBUF, bool CONTIG, int TT, int OCC, int KS, bool QB>
__global__ __launch_bounds__(64 * NW * KS) __attribute__((amdgpu_waves_per_eu(OCC, 8))) void split_kernel(
    SegmentLaunch p) {
  __shared__ __attribute__((aligned(1024))) char lds[KS * NBUF][TileGeom<FP8, TT>::kTileBytes];
  __shared__ int idx_buf[CONTIG ? 1 : kIdxCap];
  constexpr int kRowsWG = 16 * RG * NW;
  const int lane = threadIdx.x & 63;
  const int R = p.num_reqs;
  const int G = gridDim.x;
  // XCD-aware order: the dispatcher deals workgroups to the 8 XCDs in turn,
  // so logical ranges are numbered XCD by XCD.  Neighbouring ranges (the
  // pieces of one request, which load the same q rows) then share an L2.
  const int gw = xcd_major(blockIdx.x, G);

  // The first 64 requests' units, first tokens, query counts and lengths,
  // one request per lane, loaded once: with at most 64 requests the two scans
  // below and the piece loop read them from registers instead of reloading
  // them one dependent round trip after another.
  int u_l = 0, t0_l = 0, ql_l = 0, L_l = 0;
  if (lane < R) u_l = request_units(p, lane, kRowsWG, TT, &t0_l, &ql_l, &L_l);

  // Total units W (every wave computes the same values).
  int W = 0;
  for (int i = 0; i < R; i += 64) {
    int t0, ql, L;
    const int u = i == 0 ? u_l : ((i + lane < R) ? request_units(p, i + lane, kRowsWG, TT, &t0, &ql, &L) : 0);
    W += __shfl(wave_incl_scan(u), 63);
  }
  // Lane shuffles read as divergent to the compiler: make the uniform values
  // scalar so the tile loop's geometry stays in scalar registers.
  W = __builtin_amdgcn_readfirstlane(W);
  const int64_t s_g = ((int64_t)gw * W) / G;
  const int64_t e_g = ((int64_t)(gw + 1) * W) / G;

  // First request whose units reach past s_g, and its unit offset; workgroup 0
  // records every offset (and W) for the merge, and with query ranges one
  // record per token (see write_token_records).
  int r = -1;
  int base = 0;
  int carry = 0;
  const bool recorder = gw == 0 && threadIdx.x < 64;
  bool ranges_ok = true;
  for (int i = 0; i < R; i += 64) {
    int t0 = t0_l, ql = ql_l, L = L_l;
    const int u = i == 0 ? u_l : ((i + lane < R) ? request_units(p, i + lane, kRowsWG, TT, &t0, &ql, &L) : 0);
    const int incl = wave_incl_scan(u);
    const int excl = carry + incl - u;
    if (recorder && i + lane < R) p.unit_offsets[i + lane] = excl;
    if (recorder && p.tok_rec) ranges_ok &= write_token_records(p, i + lane < R, t0, ql, u, excl, W, kRowsWG);
    if (r < 0) {
      const unsigned long long hit = __ballot(u > 0 && excl <= s_g && s_g < (int64_t)excl + u);
      if (hit) {
        const int j = __builtin_ctzll(hit);
        r = i + j;
        base = __shfl(excl, j);
      }
    }
    carry = __builtin_amdgcn_readfirstlane(carry + __shfl(incl, 63));
  }
  if (recorder && p.tok_rec) {
    // valid only if the ranges tile [0, T) (qo_indptr[0] == 0 and
    // qo_indptr[R] == T on top of the per-request checks)
    const bool ok = __ballot(!ranges_ok) == 0 && p.qo_indptr[0] == 0 && p.qo_indptr[R] == p.num_tokens;
    if (lane == 0) p.tok_rec[4 * p.num_tokens] = ok ? 1 : 0;
  }
  if (recorder && lane == 0) p.unit_offsets[R] = W;
  r = __builtin_amdgcn_readfirstlane(r);
  base = __builtin_amdgcn_readfirstlane(base);
  if (s_g >= e_g || r < 0) return;

  // The first request's fields come from the registers above (read once, as
  // scalars, so they are not held through the tile loop); a workgroup that
  // moves on to further requests loads theirs.
  int t0, qlen, L, units;
  if (r < 64) {
    units = __builtin_amdgcn_readlane(u_l, r);
    t0 = __builtin_amdgcn_readlane(t0_l, r);
    qlen = __builtin_amdgcn_readlane(ql_l, r);
    L = __builtin_amdgcn_readlane(L_l, r);
  } else {
    units = request_units(p, r, kRowsWG, TT, &t0, &qlen, &L);
  }
  int64_t pos = s_g;
  int loaded = r;  // the request whose fields t0, qlen, L, units hold
  while (pos < e_g && r < R) {
    if (r != loaded) {
      units = request_units(p, r, kRowsWG, TT, &t0, &qlen, &L);
      loaded = r;
    }
    if (pos >= base + units) {  // past this request (or it has no units)
      base += units;
      ++r;
      continue;
    }
    const int nt = cdiv(L, TT);
    const int local = (int)(pos - base);
    const int c = local / nt;
    const int a = local - c * nt;
    const int b = (int)min((int64_t)nt, (int64_t)a + (e_g - pos));
    Piece pc;
    pc.r = r; pc.t0 = t0; pc.qlen = qlen; pc.L = L;
    pc.row0 = c * kRowsWG;
    pc.seg_start = a * TT;
    pc.seg_end = min(b * TT, L);
    pc.mode = (a == 0 && b == nt) ? kOutFinal : kOutSplit;
    pc.s = 0;
    pc.prow0 = ((int64_t)gw * 2 + (pos == s_g ? 0 : 1)) * kRowsWG;
    pc.phase = (int)((pos - s_g) % KS);
    if constexpr (kWide<FP8, RG, CONTIG> && FP8)
      run_piece_w32<NW, NBUF, QB>(p, lds, lds_address(&lds[0][0]), pc);
    else if constexpr (kWide<FP8, RG, CONTIG>)
      run_piece_w32b<NW, NBUF>(p, lds, lds_address(&lds[0][0]), pc);
    else
      run_piece<FP8, NW, RG, NBUF, CONTIG, TT, OCC, KS, QB>(p, lds, lds_address(&lds[0][0]), idx_buf, pc);
    pos += b - a;
  }
}

// ---------------------------------------------------------------------------
// Merge kernel
// ---------------------------------------------------------------------------
// floor(num / den) for 0 <= num < 2^48 and 0 < den < 2^31, through one fp64
// division instead of a 64-bit integer division (a long instruction
// sequence that also costs registers): the correctly rounded quotient is
// within 2^-36 of num / den, which is an integer (then returned exactly) or
// at least 1 / den from one.
__device__ __forceinline__ int floor_div_exact(int64_t num, int64_t den) {
  return (int)__builtin_floor((double)num / (double)den);
}

// Request of token t: the largest r with qo_indptr[r] <= t, found 64 entries
// at a time (one load per lane and a ballot per level: one level for fewer
// than 64 requests, two below 4096).
__device__ __forceinline__ int request_of_token(const int32_t* qo_indptr, int num_reqs, int t) {
  const int lane = threadIdx.x & 63;
  int lo = 0, span = num_reqs + 1;
  while (span > 1) {
    const int step = cdiv(span, 64);
    const int idx = lo + lane * step;
    const bool ok = lane * step < span && qo_indptr[idx] <= t;
    const unsigned long long mask = __ballot(ok);
    const int j = mask ? 63 - __builtin_clzll(mask) : 0;
    lo += j * step;
    span = min(step, num_reqs + 1 - lo);
  }
  return min(lo, num_reqs - 1);
}

// Merge kernel: one wave per (token, head) row; lane covers dims
// [8 lane, 8 lane + 8).  The row's piece statistics (one piece per lane) and
// the data of its first 16 pieces are loaded together; the weights
// 2^(m_i - M) follow once the statistics are in, and longer rows stream
// further blocks of 16 pieces.
//
// Segment pieces (SPLIT false): the valid segments of part_lens[t] (or of the
// token's request length), contiguous at [t, h, 0..nv).
// SPLIT: the pieces are those of the balanced split kernel.  The row's
// (request, row chunk) covers units [P, P + nt) of the batch's unit sequence;
// the workgroups g_first..g_last holding them left partials in slot 1 of
// g_first when that workgroup began before P, else in slot 0.  With more
// workgroups than units some ranges are empty; those wrote nothing and are
// skipped.  A row whose units all fell in one workgroup was finished there and
// is skipped here; an empty row gets O = 0 and LSE = -inf (or its sink).
// BLK: pieces in flight per step.  Their registers set the occupancy, so rows
// that usually have at most 12 pieces take 4-piece steps with five waves per
// SIMD (measured faster than one 16-piece step at two waves up to 9 pieces;
// six waves spill); the rest take 16-piece steps.
template <int OUT, bool SPLIT, int BLK>  // OUT: 0 bf16, 1 fp16, 2 fp32
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(BLK <= 4 ? 5 : 2, 8)))
void merge_kernel(MergeLaunch p) {
  constexpr int kBlk = BLK;
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= (int64_t)p.num_tokens * p.num_heads) return;
  const int t = (int)(row / p.num_heads);
  const int h = (int)(row - (int64_t)t * p.num_heads);
  const int S = p.num_segments;

  // The split kernel's token record, when its flag says the records are
  // complete: the row's request start, unit offset and units per chunk in one
  // load.  Else the request is found by searching the query ranges.
  i32x4 rec = {0, 0, 0, 0};
  bool have_rec = false;
  if constexpr (SPLIT) {
    if (p.tok_rec) {
      rec = *(const i32x4*)(p.tok_rec + 4 * (int64_t)t);
      have_rec = p.tok_rec[4 * (int64_t)p.num_tokens] != 0;
    }
  }
  int req = t;
  bool malformed = false;
  if (!have_rec && (SPLIT || !p.part_lens) && p.qo_indptr) {
    req = request_of_token(p.qo_indptr, p.num_reqs, t);
    // A request whose query range is malformed gets NaN rows (the stream
    // kernels computed nothing for it); so does a token outside every range.
    const int64_t a = p.qo_indptr[req], b = p.qo_indptr[req + 1];
    malformed = a < 0 || b < a || b - a > p.max_qlen || b > p.num_tokens || t < a || t >= b;
  }
  int nv = 0;
  const int64_t base = row * S;
  // split pieces: rows of the piece buffers (below 2 G rows_wg, so 32-bit)
  int row_i0 = 0, first_row = 0, stride = 0, gf = 0, W = 1, G = 1;
  if (malformed) {
  } else if constexpr (SPLIT) {
    int t0, P0, nt;  // the request's first token, unit offset, units per row chunk
    if (have_rec) {
      t0 = rec[0];
      P0 = rec[1];
      nt = rec[2];
      W = rec[3];
    } else {
      t0 = p.qo_indptr ? p.qo_indptr[req] : req;
      const int qlen = p.qo_indptr ? p.qo_indptr[req + 1] - t0 : 1;
      P0 = p.unit_offsets[req];
      const int units = p.unit_offsets[req + 1] - P0;
      W = p.unit_offsets[p.num_reqs];
      const int chunks = cdiv(qlen * p.num_heads, p.rows_wg);
      nt = units > 0 ? units / chunks : 0;
    }
    const int rr = (t - t0) * p.num_heads + h;  // row within the request
    const int c = rr / p.rows_wg, local = rr - c * p.rows_wg;
    if (nt > 0 && W > 0) {
      const int P = P0 + c * nt;
      G = p.grid_wgs;
      gf = floor_div_exact(((int64_t)P + 1) * G - 1, W);
      const int gl = floor_div_exact(((int64_t)P + nt) * G - 1, W);
      if (gf == gl) return;  // finished by the split kernel
      nv = gl - gf + 1;
      const int start_f = floor_div_exact((int64_t)gf * W, G);
      row_i0 = (gf * 2 + (start_f < P ? 1 : 0)) * p.rows_wg + local;
      first_row = (gf * 2) * p.rows_wg + local;
      stride = 2 * p.rows_wg;
    }
  } else {
    const int L = p.part_lens ? p.part_lens[t] : p.seq_lens[req];
    if (L > 0) {
      const int span = cdiv(L, S * p.tile) * p.tile;
      nv = min(S, cdiv(L, span));
    }
  }
  // Row index of piece i in the partial buffers, and whether it exists.
  auto prow = [&](int i) -> int64_t {
    if constexpr (SPLIT) return (int64_t)(i == 0 ? row_i0 : first_row + i * stride);
    return base + i;
  };
  auto present = [&](int i) -> bool {
    if constexpr (SPLIT) {
      const int64_t g = gf + i;
      return floor_div_exact((g + 1) * W, G) > floor_div_exact(g * W, G);
    }
    return true;
  };
  // dims 8 lane .. 8 lane + 7 of piece row pr (fp32, or bf16 partials)
  const bool bf16_pieces = p.piece_bf16 != 0;
  auto load_piece = [&](int64_t pr, f32x4& lo, f32x4& hi) {
    if (bf16_pieces) {
      const u32x4 b = *(const u32x4*)(p.piece_out + pr * kKvRank + 8 * lane);
      lo = f32x4{__uint_as_float(b[0] << 16), __uint_as_float(b[0] & 0xffff0000u),
                 __uint_as_float(b[1] << 16), __uint_as_float(b[1] & 0xffff0000u)};
      hi = f32x4{__uint_as_float(b[2] << 16), __uint_as_float(b[2] & 0xffff0000u),
                 __uint_as_float(b[3] << 16), __uint_as_float(b[3] & 0xffff0000u)};
    } else {
      const float* src = p.seg_out + pr * kKvRank + 8 * lane;
      lo = *(const f32x4*)(src);
      hi = *(const f32x4*)(src + 4);
    }
  };
  auto load_block = [&](f32x4 (&v)[2 * kBlk], int j0, unsigned long long pmask, int cnt) {
#pragma unroll
    for (int u = 0; u < kBlk; ++u) {
      if (j0 + u < cnt && ((pmask >> (j0 + u)) & 1ull)) {
        load_piece(prow(j0 + u), v[2 * u], v[2 * u + 1]);
      } else {
        v[2 * u] = v[2 * u + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float M = -INFINITY, Lsum = 0.f;
  bool nan_seen = malformed;
  if (malformed) {
  } else if (nv <= 64) {
    // Common case: statistics of every piece in one load per lane, issued with
    // the first block's data.
    const bool pres = lane < nv && present(lane);
    const unsigned long long pmask = __ballot(pres);
    const float m = pres ? p.seg_max[prow(lane)] : -INFINITY;
    const float l = pres ? p.seg_sum[prow(lane)] : 0.f;
    f32x4 v[2 * kBlk];
    load_block(v, 0, pmask, nv);
    nan_seen = __ballot(m != m) != 0;
    M = m;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    const float wgt = (m > -INFINITY) ? exp2f(m - M) : 0.f;
    Lsum = l * wgt;
    for (int j0 = 0; j0 < nv; j0 += kBlk) {
      if (j0 > 0) load_block(v, j0, pmask, nv);
#pragma unroll
      for (int u = 0; u < kBlk; ++u) {
        const float wu = __shfl(wgt, (j0 + u) & 63);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[e] += wu * v[2 * u][e];
          acc[4 + e] += wu * v[2 * u + 1][e];
        }
      }
    }
  } else {
    // Long rows: the maximum first, then blocks of 64 pieces.
    for (int s0 = 0; s0 < nv; s0 += 64) {
      const int i = s0 + lane;
      const float m = (i < nv && present(i)) ? p.seg_max[prow(i)] : -INFINITY;
      nan_seen |= (m != m);
      M = fmaxf(M, m);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    nan_seen = __ballot(nan_seen) != 0;
    for (int s0 = 0; s0 < nv; s0 += 64) {
      const int i = s0 + lane;
      const bool pres = i < nv && present(i);
      const unsigned long long pmask = __ballot(pres);
      float wgt = 0.f;
      if (pres) {
        const float m = p.seg_max[prow(i)];
        wgt = (m > -INFINITY) ? exp2f(m - M) : 0.f;
        Lsum += p.seg_sum[prow(i)] * wgt;
      }
      const int cnt = min(64, nv - s0);
      for (int j0 = 0; j0 < cnt; j0 += kBlk) {
        f32x4 v[2 * kBlk];
#pragma unroll
        for (int u = 0; u < kBlk; ++u) {
          if (j0 + u < cnt && ((pmask >> (j0 + u)) & 1ull)) {
            load_piece(prow(s0 + j0 + u), v[2 * u], v[2 * u + 1]);
          } else {
            v[2 * u] = v[2 * u + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
        }
#pragma unroll
        for (int u = 0; u < kBlk; ++u) {
          const float wu = __shfl(wgt, (j0 + u) & 63);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[e] += wu * v[2 * u][e];
            acc[4 + e] += wu * v[2 * u + 1][e];
          }
        }
      }
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) Lsum += __shfl_xor(Lsum, o);
  const bool has = M > -INFINITY;
  float lse, scale;
  if (has) {
    lse = kLn2 * (M + log2f(Lsum));
    scale = 1.0f / Lsum;
  } else {
    lse = -INFINITY;
    scale = 0.f;
  }
  if (p.sinks) {
    const float nl = logaddexp_f(lse, p.sinks[h]);
    scale = has ? scale * expf(lse - nl) : 0.f;
    lse = nl;
  }
  if (nan_seen) { lse = __builtin_nanf(""); scale = __builtin_nanf(""); }
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = has ? acc[i] * scale : (nan_seen ? scale : 0.f);

  const int64_t orow = row * kKvRank + 8 * lane;
  if constexpr (OUT == 0) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = (unsigned)f32_to_bf16_rne(o[2 * i]) | ((unsigned)f32_to_bf16_rne(o[2 * i + 1]) << 16);
    *(u32x4*)((unsigned short*)p.out + orow) = v;
  } else if constexpr (OUT == 1) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const _Float16 a = (_Float16)o[2 * i], b = (_Float16)o[2 * i + 1];
      v[i] = (unsigned)__builtin_bit_cast(unsigned short, a) | ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
    }
    *(u32x4*)((unsigned short*)p.out + orow) = v;
  } else {
    f32x4* dst = (f32x4*)((float*)p.out + orow);
    dst[0] = f32x4{o[0], o[1], o[2], o[3]};
    dst[1] = f32x4{o[4], o[5], o[6], o[7]};
  }
  if (lane == 0) p.lse[row] = lse;
}

// ---------------------------------------------------------------------------
// Cross-shard combine (decode context parallelism)
// ---------------------------------------------------------------------------
// One wave per (token, head) row; lane w < W holds shard w's LSE, and lane l
// covers dims [8 l, 8 l + 8) of the output.  Natural-log weights
// e^(lse_w - lse) on the shard outputs, then the sink once per row.
template <int IN, int OUT>  // 0 bf16, 1 fp16, 2 fp32
__global__ __launch_bounds__(256) void combine_kernel(CombineLaunch p) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = (int64_t)p.num_tokens * p.num_heads;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int h = (int)(row % p.num_heads);
  const int W = p.num_shards;
  const float lw = lane < W ? p.shard_lse[(int64_t)lane * rows + row] : -INFINITY;
  const bool nan_seen = __ballot(lw != lw) != 0;
  float M = lw;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  const bool has = M > -INFINITY;
  const float wgt = (has && lw > -INFINITY) ? expf(lw - M) : 0.f;
  float S = wgt;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) S += __shfl_xor(S, o);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int w = 0; w < W; ++w) {
    const float ww = __shfl(wgt, w);
    if (ww == 0.f) continue;  // uniform: an empty shard adds nothing
    const int64_t base = ((int64_t)w * rows + row) * kKvRank + 8 * lane;
    float v[8];
    if constexpr (IN == 2) {
      const f32x4 a = *(const f32x4*)((const float*)p.shard_out + base);
      const f32x4 b = *(const f32x4*)((const float*)p.shard_out + base + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) { v[i] = a[i]; v[4 + i] = b[i]; }
    } else {
      const u32x4 u = *(const u32x4*)((const unsigned short*)p.shard_out + base);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const unsigned short lo = (unsigned short)(u[i] & 0xffff), hi = (unsigned short)(u[i] >> 16);
        if constexpr (IN == 0) {
          v[2 * i] = __uint_as_float((unsigned)lo << 16);
          v[2 * i + 1] = __uint_as_float((unsigned)hi << 16);
        } else {
          v[2 * i] = (float)__builtin_bit_cast(_Float16, lo);
          v[2 * i + 1] = (float)__builtin_bit_cast(_Float16, hi);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += ww * v[i];
  }
  float lse = has ? M + logf(S) : -INFINITY;
  float scale = has ? 1.0f / S : 0.f;
  if (p.sinks) {
    const float nl = logaddexp_f(lse, p.sinks[h]);
    scale = has ? scale * expf(lse - nl) : 0.f;
    lse = nl;
  }
  if (nan_seen) { lse = __builtin_nanf(""); scale = __builtin_nanf(""); }
  float o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = has ? acc[i] * scale : (nan_seen ? scale : 0.f);
  const int64_t orow = row * kKvRank + 8 * lane;
  if constexpr (OUT == 2) {
    f32x4* dst = (f32x4*)((float*)p.out + orow);
    dst[0] = f32x4{o[0], o[1], o[2], o[3]};
    dst[1] = f32x4{o[4], o[5], o[6], o[7]};
  } else {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (OUT == 0) {
        v[i] = (unsigned)f32_to_bf16_rne(o[2 * i]) | ((unsigned)f32_to_bf16_rne(o[2 * i + 1]) << 16);
      } else {
        const _Float16 a = (_Float16)o[2 * i], b = (_Float16)o[2 * i + 1];
        v[i] = (unsigned)__builtin_bit_cast(unsigned short, a) | ((unsigned)__builtin_bit_cast(unsigned short, b) << 16);
      }
    }
    *(u32x4*)((unsigned short*)p.out + orow) = v;
  }
  if (lane == 0) p.lse[row] = lse;
}

template <bool FP8, int NW, int RG, bool CONTIG, bool QB>
hipError_t launch_seg(const SegmentLaunch& a, int chunks, hipStream_t stream) {
  constexpr ShapeCfg kCfg = shape_cfg(FP8, NW, RG);
  constexpr int kTT = kCfg.tt;
  constexpr int kTileBytes = kTT * (FP8 ? 576 : 1152);
  constexpr int kRing = kCfg.ring / kTileBytes;
  dim3 grid(a.num_segments, a.num_reqs, chunks);
  hipLaunchKernelGGL((segment_kernel<FP8, NW, RG, kRing, CONTIG, kTT, kCfg.occ, QB>), grid, dim3(64 * NW), 0,
                     stream, a);
  return hipGetLastError();
}

template <bool FP8, int NW, int RG, bool CONTIG, int KS, bool QB>
hipError_t launch_split(const SegmentLaunch& a, int grid_wgs, hipStream_t stream) {
  constexpr ShapeCfg kCfg = shape_cfg(FP8, NW, RG);
  constexpr int kTT = kCfg.tt;
  constexpr int kTileBytes = kTT * (FP8 ? 576 : 1152);
  constexpr int kRing = kCfg.ring / kTileBytes;
  hipLaunchKernelGGL((split_kernel<FP8, NW, RG, kRing, CONTIG, kTT, kCfg.occ, KS, QB>), dim3(grid_wgs),
                     dim3(64 * NW * KS), 0, stream, a);
  return hipGetLastError();
}

template <bool FP8, int NW, int RG, bool CONTIG, bool QB = false>
hipError_t launch_any(const SegmentLaunch& a, const SegmentShape& sh, int split_wgs, hipStream_t stream) {
  if (split_wgs <= 0) return launch_seg<FP8, NW, RG, CONTIG, QB>(a, sh.chunks, stream);
  if constexpr (NW == 1 && RG == 1 && CONTIG) {
    if (sh.ks == kSplitKs) return launch_split<FP8, NW, RG, CONTIG, kSplitKs, QB>(a, split_wgs, stream);
  }
  return launch_split<FP8, NW, RG, CONTIG, 1, QB>(a, split_wgs, stream);
}

// QB: bf16 q quantised in the q load (fp8 cache).
template <bool FP8, bool CONTIG, bool QB = false>
hipError_t launch_seg_shape(const SegmentLaunch& a, const SegmentShape& sh, int split_wgs, hipStream_t stream) {
  if constexpr (FP8 && CONTIG) {
    if (sh.rows_per_wave == 2) {  // wide waves: 32 rows each
      return launch_any<true, 2, 2, true, QB>(a, sh, split_wgs, stream);
    }
  }
  if constexpr (!FP8 && CONTIG) {
    if (sh.rows_per_wave == 2) return launch_any<false, 4, 2, true>(a, sh, split_wgs, stream);
  }
  switch (sh.waves) {
    case 1: return launch_any<FP8, 1, 1, CONTIG, QB>(a, sh, split_wgs, stream);
    case 2: return launch_any<FP8, 2, 1, CONTIG, QB>(a, sh, split_wgs, stream);
    case 4: return launch_any<FP8, 4, 1, CONTIG, QB>(a, sh, split_wgs, stream);
    default: return launch_any<FP8, 8, 1, CONTIG, QB>(a, sh, split_wgs, stream);
  }
}

// Scratch for callers that cannot allocate (mla_decode_no_alloc): the fused
// decode's partials and unit offsets.  Every GPU holds its own copy until
// the process ends; calls that overlap on one GPU share it and race.
static __device__ __align__(256) char scratch[kScratchBytes];

}  // namespace

hipError_t scratch_buffer(void** ptr) {
  // The device address of `scratch` on the current device, looked up once per
  // device (the host-side name of the array is not a device address).
  static std::mutex mu;
  static std::vector<void*> addr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

SegmentShape segment_shape(bool fp8, int num_heads, int max_qlen, int tile) {
  SegmentShape sh;
  sh.fp8 = fp8;
  sh.rows_per_wave = 1;
  const int groups = (max_qlen * num_heads + 15) / 16;
  if (fp8 && groups == 4 && tile >= 32) {
    // 49-64 rows per chunk: two wide waves of 32 rows over contiguous
    // 32-token tiles, two workgroups per CU.  (Measured at 52 x 16K: faster
    // than four 16-row waves at 64 heads; slower at 48 heads, where the
    // second wide wave would carry 16 empty rows, and with four wide waves
    // for 96-head verify blocks.)
    sh.rows_per_wave = 2;
    sh.waves = 2;
    const int rows_wg = 32 * sh.waves;
    sh.chunks = (max_qlen * num_heads + rows_wg - 1) / rows_wg;
    sh.contig = true;
    sh.ks = 1;
    return sh;
  }
  if (!fp8 && groups >= 5 && tile >= 32) {
    // more than 64 rows per chunk: four wide bf16 waves of 32 rows over
    // contiguous 32-token tiles, one workgroup per CU
    sh.rows_per_wave = 2;
    sh.waves = 4;
    const int rows_wg = 32 * sh.waves;
    sh.chunks = (max_qlen * num_heads + rows_wg - 1) / rows_wg;
    sh.contig = true;
    sh.ks = 1;
    return sh;
  }
  // groups of 16 rows -> waves per workgroup
  if (groups <= 1)      { sh.waves = 1; }
  else if (groups == 2) { sh.waves = 2; }
  else if (groups <= 4) { sh.waves = 4; }
  else                  { sh.waves = 8; }
  const int rows_wg = 16 * sh.rows_per_wave * sh.waves;
  sh.chunks = (max_qlen * num_heads + rows_wg - 1) / rows_wg;
  sh.contig = tile >= tile_tokens(fp8, sh.waves, sh.rows_per_wave);
  sh.ks = split_ks(sh.waves, sh.rows_per_wave, sh.contig);
  return sh;
}

hipError_t launch_segments(const SegmentLaunch& a, const SegmentShape& sh, int split_wgs, hipStream_t stream) {
  if (sh.fp8) {
    if (a.q_bf16)
      return sh.contig ? launch_seg_shape<true, true, true>(a, sh, split_wgs, stream)
                       : launch_seg_shape<true, false, true>(a, sh, split_wgs, stream);
    return sh.contig ? launch_seg_shape<true, true>(a, sh, split_wgs, stream)
                     : launch_seg_shape<true, false>(a, sh, split_wgs, stream);
  }
  return sh.contig ? launch_seg_shape<false, true>(a, sh, split_wgs, stream)
                   : launch_seg_shape<false, false>(a, sh, split_wgs, stream);
}

template <bool SPLIT, int BLK>
void launch_merge_t(const MergeLaunch& a, dim3 grid, hipStream_t stream) {
  switch (a.out_dtype) {
    case 0: hipLaunchKernelGGL((merge_kernel<0, SPLIT, BLK>), grid, dim3(256), 0, stream, a); break;
    case 1: hipLaunchKernelGGL((merge_kernel<1, SPLIT, BLK>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((merge_kernel<2, SPLIT, BLK>), grid, dim3(256), 0, stream, a); break;
  }
}

// Pieces a row usually has: the segment count, or for split pieces the
// workgroups per request (+2 when a request's range does not start and end on
// workgroup boundaries).
template <bool SPLIT>
void launch_merge_b(const MergeLaunch& a, dim3 grid, hipStream_t stream) {
  int est = a.num_segments;
  if (SPLIT) {
    const int r = a.num_reqs > 0 ? a.num_reqs : 1;
    est = a.grid_wgs / r + (a.grid_wgs % r ? 2 : 0);
  }
  if (est <= 12) launch_merge_t<SPLIT, 4>(a, grid, stream);
  else launch_merge_t<SPLIT, 16>(a, grid, stream);
}

template <int IN>
void launch_combine_t(const CombineLaunch& a, dim3 grid, hipStream_t stream) {
  switch (a.out_dtype) {
    case 0: hipLaunchKernelGGL((combine_kernel<IN, 0>), grid, dim3(256), 0, stream, a); break;
    case 1: hipLaunchKernelGGL((combine_kernel<IN, 1>), grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL((combine_kernel<IN, 2>), grid, dim3(256), 0, stream, a); break;
  }
}

hipError_t launch_combine(const CombineLaunch& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_tokens * a.num_heads;
  dim3 grid((unsigned)((rows + 3) / 4));
  switch (a.in_dtype) {
    case 0: launch_combine_t<0>(a, grid, stream); break;
    case 1: launch_combine_t<1>(a, grid, stream); break;
    default: launch_combine_t<2>(a, grid, stream); break;
  }
  return hipGetLastError();
}

hipError_t launch_merge(const MergeLaunch& a, hipStream_t stream) {
  const int64_t rows = (int64_t)a.num_tokens * a.num_heads;
  dim3 grid((unsigned)((rows + 3) / 4));
  if (a.unit_offsets) launch_merge_b<true>(a, grid, stream);
  else launch_merge_b<false>(a, grid, stream);
  return hipGetLastError();
}

}  // namespace mla
