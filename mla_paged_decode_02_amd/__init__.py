"""Thin Python binding of the MLA paged-decode HIP library (libmla_decode.so).

Argument marshalling only: every step of the decode runs in the library's HIP
kernels.  torch is used for device memory and streams.  The names mirror the C
ABI in include/mla_decode.h:

* ``decode_segments``  -> mla_decode_segments  (base-2 partials per segment)
* ``merge_segments``   -> mla_merge_segments   (output + natural-log LSE, sinks)
* ``decode``           -> mla_decode           (both, partials in a workspace)

plus the host helpers ``tile_size_for_block``, ``segment_bounds``,
``plan_num_segments``, ``resolve_num_segments``, ``validate``.

The library must be built (``python -m mla_paged_decode_02_amd.build``); there
is no fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "lib", "libmla_decode.so")

MLA_OK = 0
MLA_ERR_INVALID_ARG = -1
MLA_ERR_UNSUPPORTED = -2
MLA_ERR_WORKSPACE = -3
MLA_ERR_HIP = -4

MLA_DTYPE_BF16 = 1
MLA_DTYPE_FP8_E4M3 = 2
MLA_DTYPE_FP16 = 3
MLA_DTYPE_FP32 = 4

MLA_SCHEDULE_SEGMENTS = 0
MLA_SCHEDULE_BALANCED = 1
_SCHEDULES = {"segments": MLA_SCHEDULE_SEGMENTS, "balanced": MLA_SCHEDULE_BALANCED}

HEAD_DIM = 576
KV_LORA_RANK = 512


class MlaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class MlaProblem(ctypes.Structure):
    _fields_ = [
        ("struct_size", ctypes.c_size_t),
        ("num_tokens", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_reqs", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("kv_lora_rank", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("q_dtype", ctypes.c_int32),
        ("q_stride_token", ctypes.c_int64),
        ("q_stride_head", ctypes.c_int64),
        ("q_scale", ctypes.c_void_p),
        ("kv_cache", ctypes.c_void_p),
        ("kv_dtype", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("kv_scale", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("bt_stride_row", ctypes.c_int64),
        ("bt_stride_col", ctypes.c_int64),
        ("max_blocks_per_req", ctypes.c_int32),
        ("seq_lens", ctypes.c_void_p),
        ("qo_indptr", ctypes.c_void_p),
        ("max_qlen", ctypes.c_int32),
        ("max_seq_len", ctypes.c_int32),
        ("sum_seq_lens", ctypes.c_int64),
        ("causal", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("tile_size", ctypes.c_int32),
        ("num_segments", ctypes.c_int32),
        ("max_workgroups", ctypes.c_int32),
        ("bt_indptr", ctypes.c_void_p),
        ("q_pe", ctypes.c_void_p),
        ("q_pe_stride_token", ctypes.c_int64),
        ("q_pe_stride_head", ctypes.c_int64),
        ("schedule", ctypes.c_int32),
    ]


_lib = None

EXPORTED = (
    "mla_validate", "mla_decode_segments", "mla_merge_segments", "mla_decode",
    "mla_decode_workspace_bytes", "mla_resolve_num_segments", "mla_plan_num_segments",
    "mla_tile_size_for_block", "mla_segment_bounds", "mla_status_string", "mla_last_error",
    "mla_version", "mla_decode_stage", "mla_split_plan", "mla_combine_lse", "mla_decode_no_alloc",
)

# Size of the library's static device scratch (mla_decode_no_alloc).
NO_ALLOC_SCRATCH_BYTES = 160 << 20


def lib() -> ctypes.CDLL:
    """Load the HIP library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m mla_paged_decode_02_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(MlaProblem)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    L.mla_validate.argtypes = [P, ctypes.c_int]
    L.mla_decode_segments.argtypes = [P, vp, vp, vp, vp]
    L.mla_merge_segments.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, vp, vp, i32, vp, vp]
    L.mla_decode.argtypes = [P, vp, vp, i32, vp, vp, sz, vp]
    L.mla_decode_stage.argtypes = [P, vp, vp, i32, vp, vp, sz, i32, vp]
    L.mla_decode_no_alloc.argtypes = [P, vp, vp, i32, vp, vp]
    L.mla_combine_lse.argtypes = [vp, i32, vp, i32, i32, i32, vp, vp, i32, vp, vp]
    L.mla_split_plan.argtypes = [P, ctypes.POINTER(i32), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.mla_decode_workspace_bytes.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    L.mla_resolve_num_segments.argtypes = [P]
    L.mla_plan_num_segments.argtypes = [i32, i32, i64, i32, i32, i32, i32, i32]
    L.mla_tile_size_for_block.argtypes = [i32]
    L.mla_segment_bounds.argtypes = [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.mla_status_string.argtypes = [ctypes.c_int]
    L.mla_status_string.restype = ctypes.c_char_p
    L.mla_last_error.argtypes = []
    L.mla_last_error.restype = ctypes.c_char_p
    L.mla_version.argtypes = []
    for f in ("mla_validate", "mla_decode_segments", "mla_merge_segments", "mla_decode",
              "mla_decode_workspace_bytes", "mla_resolve_num_segments", "mla_plan_num_segments",
              "mla_tile_size_for_block", "mla_segment_bounds", "mla_version", "mla_decode_stage",
              "mla_split_plan", "mla_combine_lse", "mla_decode_no_alloc"):
        getattr(L, f).restype = ctypes.c_int
    _lib = L
    return L


def _status_name(status: int) -> str:
    try:
        return lib().mla_status_string(status).decode()
    except ImportError:
        return str(status)


def _check(status: int) -> int:
    if status < 0:
        raise MlaError(status, lib().mla_last_error().decode())
    return status


# ------------------------------------------------------------------ helpers --

def tile_size_for_block(block_size: int) -> int:
    return _check(lib().mla_tile_size_for_block(int(block_size)))


def segment_bounds(seq_len: int, num_segments: int, tile_size: int) -> list[tuple[int, int]]:
    n = max(int(num_segments), 1)
    starts = (ctypes.c_int32 * n)()
    ends = (ctypes.c_int32 * n)()
    cnt = _check(lib().mla_segment_bounds(int(seq_len), int(num_segments), int(tile_size), starts, ends))
    return [(starts[i], ends[i]) for i in range(cnt)]


def plan_num_segments(num_reqs: int, max_seq_len: int, num_heads: int, *, max_qlen: int = 1,
                      tile_size: int = 64, kv_dtype: str = "bf16", num_cus: int = 256,
                      sum_seq_lens: int = 0) -> int:
    code = MLA_DTYPE_FP8_E4M3 if kv_dtype.startswith("fp8") else MLA_DTYPE_BF16
    return _check(lib().mla_plan_num_segments(int(num_reqs), int(max_seq_len), int(sum_seq_lens),
                                              int(num_heads), int(max_qlen), int(tile_size), code,
                                              int(num_cus)))


def _dtype_code(t: torch.Tensor, name: str) -> int:
    if t.dtype == torch.bfloat16:
        return MLA_DTYPE_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return MLA_DTYPE_FP8_E4M3
    raise ValueError(f"{name} must be bfloat16 or float8_e4m3fn (uint8 holding e4m3 codes), got {t.dtype}")


def _out_code(dtype: torch.dtype) -> int:
    return {torch.bfloat16: MLA_DTYPE_BF16, torch.float16: MLA_DTYPE_FP16,
            torch.float32: MLA_DTYPE_FP32}[dtype]


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def check_sinks(sinks: Optional[torch.Tensor], num_heads: int) -> None:
    """Sink contract of the sparse MLA backend page (ROCMAiterMLASparseImpl.__init__)."""
    if sinks is None:
        return
    if sinks.dtype != torch.float32:
        raise ValueError(f"ROCm AITER MLA sinks must be float32, got {sinks.dtype}")
    if sinks.ndim != 1 or sinks.numel() != num_heads:
        raise ValueError(f"ROCm AITER MLA sinks must have shape ({num_heads},), got {tuple(sinks.shape)}")
    if not sinks.is_contiguous():
        raise ValueError("ROCm AITER MLA sinks must be contiguous")


def make_problem(q: torch.Tensor, kv_cache: torch.Tensor, block_table: torch.Tensor,
                 seq_lens: torch.Tensor, *, softmax_scale: float, max_seq_len: int,
                 qo_indptr: Optional[torch.Tensor] = None, max_qlen: Optional[int] = None,
                 causal: bool = False, q_scale: Optional[torch.Tensor] = None,
                 kv_scale: Optional[torch.Tensor] = None, tile_size: int = 0,
                 num_segments: int = 0, sum_seq_lens: int = 0, max_workgroups: int = 0,
                 bt_indptr: Optional[torch.Tensor] = None, q_pe: Optional[torch.Tensor] = None,
                 schedule: str = "segments") -> MlaProblem:
    """Fill an ``mla_problem`` from tensors.  Host ints (max_seq_len, max_qlen)
    are passed by the caller so nothing is read back from the device.

    With ``bt_indptr`` (int32 [R+1]) the block table is one flat int32 list and
    request r's pages are ``block_table[bt_indptr[r]:bt_indptr[r+1]]``; with
    block_size 1 that is a per-token index stream (sparse decode).

    With ``q_pe`` ([T, H, 64]) q holds only the 512 latent dims ([T, H, 512]):
    the (ql_nope, q_pe) pair of the MLA layer, concatenated in the q load.  A
    bf16 q with an fp8 cache is quantised in the q load with ``q_scale``.

    ``schedule`` picks how ``decode`` splits the key axis: "segments" (the
    segment partition with ``num_segments``, 0 = the planner's S) or
    "balanced" (equal key ranges per workgroup; ``num_segments`` must be 0)."""
    if schedule not in _SCHEDULES:
        raise ValueError(f"schedule must be one of {sorted(_SCHEDULES)}, got {schedule!r}")
    width = KV_LORA_RANK if q_pe is not None else HEAD_DIM
    if q.ndim != 3 or q.shape[-1] != width or q.stride(-1) != 1:
        raise ValueError(f"q must be [T, H, {width}] with a contiguous last dim, got {tuple(q.shape)}")
    if q_pe is not None and (q_pe.ndim != 3 or tuple(q_pe.shape) != (q.shape[0], q.shape[1], HEAD_DIM - KV_LORA_RANK)
                             or q_pe.stride(-1) != 1 or q_pe.dtype != q.dtype):
        raise ValueError(f"q_pe must be [T, H, 64] of q's dtype with a contiguous last dim, got "
                         f"{tuple(q_pe.shape)} {q_pe.dtype}")
    if kv_cache.ndim != 3 or kv_cache.shape[-1] != HEAD_DIM or not kv_cache.is_contiguous():
        raise ValueError(f"kv_cache must be a contiguous [blocks, page, 576] tensor, got {tuple(kv_cache.shape)}")
    qd, kd = _dtype_code(q, "q"), _dtype_code(kv_cache, "kv_cache")
    if qd != kd and not (qd == MLA_DTYPE_BF16 and kd == MLA_DTYPE_FP8_E4M3):
        raise ValueError(f"q dtype {q.dtype} and kv_cache dtype {kv_cache.dtype} must match "
                         "(bf16 with bf16, fp8 with fp8; a bf16 q with an fp8 cache is quantised in the q load)")
    if block_table.dtype != torch.int32 or seq_lens.dtype != torch.int32:
        raise ValueError("block_table and seq_lens must be int32")
    if bt_indptr is not None:
        if bt_indptr.dtype != torch.int32 or bt_indptr.shape != (seq_lens.shape[0] + 1,):
            raise ValueError("bt_indptr must be int32 [num_reqs + 1]")
        if block_table.ndim != 1:
            raise ValueError("with bt_indptr the block table is one flat int32 list")
    elif block_table.ndim != 2:
        raise ValueError("block_table must be int32 [num_reqs, max_blocks_per_req]")
    if qo_indptr is not None and qo_indptr.dtype != torch.int32:
        raise ValueError("qo_indptr must be int32")
    for name, s in (("q_scale", q_scale), ("kv_scale", kv_scale)):
        if s is not None and (s.dtype != torch.float32 or s.numel() != 1):
            raise ValueError(f"{name} must be a one-element float32 tensor")
    T, H = q.shape[0], q.shape[1]
    p = MlaProblem()
    p.struct_size = ctypes.sizeof(MlaProblem)
    p.num_tokens, p.num_heads, p.num_reqs = T, H, seq_lens.shape[0]
    p.head_dim, p.kv_lora_rank = HEAD_DIM, KV_LORA_RANK
    p.q, p.q_dtype = _ptr(q), qd
    p.q_stride_token, p.q_stride_head = q.stride(0), q.stride(1)
    p.q_scale = _ptr(q_scale)
    if q_pe is not None:
        p.q_pe = _ptr(q_pe)
        p.q_pe_stride_token, p.q_pe_stride_head = q_pe.stride(0), q_pe.stride(1)
    p.kv_cache, p.kv_dtype = _ptr(kv_cache), kd
    p.block_size, p.num_blocks = kv_cache.shape[1], kv_cache.shape[0]
    p.kv_scale = _ptr(kv_scale)
    p.block_table = _ptr(block_table)
    if bt_indptr is not None:
        p.bt_stride_row, p.bt_stride_col = 0, block_table.stride(0)
        p.max_blocks_per_req = 0
        p.bt_indptr = _ptr(bt_indptr)
    else:
        p.bt_stride_row, p.bt_stride_col = block_table.stride(0), block_table.stride(1)
        p.max_blocks_per_req = block_table.shape[1]
    p.seq_lens = _ptr(seq_lens)
    p.qo_indptr = _ptr(qo_indptr)
    p.max_qlen = 1 if qo_indptr is None else int(max_qlen if max_qlen is not None else 1)
    p.max_seq_len = int(max_seq_len)
    p.sum_seq_lens = int(sum_seq_lens)
    p.causal = 1 if causal else 0
    p.softmax_scale = float(softmax_scale)
    p.tile_size = int(tile_size)
    p.num_segments = int(num_segments)
    p.max_workgroups = int(max_workgroups)
    p.schedule = _SCHEDULES[schedule]
    return p


def validate(p: MlaProblem, require_segments: bool = True) -> None:
    _check(lib().mla_validate(ctypes.byref(p), 1 if require_segments else 0))


def resolve_num_segments(p: MlaProblem) -> int:
    return _check(lib().mla_resolve_num_segments(ctypes.byref(p)))


def split_plan(p: MlaProblem):
    """(workgroups, rows per workgroup, keys per unit) of the balanced split
    ``decode`` uses for p, or None when p uses the segment partition."""
    g, rw, tt = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    used = _check(lib().mla_split_plan(ctypes.byref(p), ctypes.byref(g), ctypes.byref(rw), ctypes.byref(tt)))
    return (g.value, rw.value, tt.value) if used else None


def workspace_bytes(p: MlaProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().mla_decode_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return n.value


# --------------------------------------------------------------- entry points

def decode_segments(q, kv_cache, block_table, seq_lens, *, softmax_scale: float, num_segments: int,
                    max_seq_len: int, qo_indptr=None, max_qlen=None, causal=False, q_scale=None,
                    kv_scale=None, tile_size: int = 0, sum_seq_lens: int = 0, segm_output=None,
                    segm_max=None, segm_expsum=None, bt_indptr=None, q_pe=None, stream=None):
    """Base-2 partials [T, H, S, 512], [T, H, S], [T, H, S] (fp32).  Slots of
    segments that hold no position are left as allocated (uninitialised)."""
    p = make_problem(q, kv_cache, block_table, seq_lens, softmax_scale=softmax_scale,
                     max_seq_len=max_seq_len, qo_indptr=qo_indptr, max_qlen=max_qlen, causal=causal,
                     q_scale=q_scale, kv_scale=kv_scale, tile_size=tile_size, num_segments=num_segments,
                     sum_seq_lens=sum_seq_lens, bt_indptr=bt_indptr, q_pe=q_pe)
    T, H, S = q.shape[0], q.shape[1], int(num_segments)
    dev = q.device
    if segm_output is None:
        segm_output = torch.empty((T, H, S, KV_LORA_RANK), dtype=torch.float32, device=dev)
    if segm_max is None:
        segm_max = torch.empty((T, H, S), dtype=torch.float32, device=dev)
    if segm_expsum is None:
        segm_expsum = torch.empty((T, H, S), dtype=torch.float32, device=dev)
    for t, shp in ((segm_output, (T, H, S, KV_LORA_RANK)), (segm_max, (T, H, S)), (segm_expsum, (T, H, S))):
        if tuple(t.shape) != shp or t.dtype != torch.float32 or not t.is_contiguous():
            raise ValueError(f"partials buffer must be contiguous float32 {shp}, got {tuple(t.shape)}")
    _check(lib().mla_decode_segments(ctypes.byref(p), _ptr(segm_output), _ptr(segm_max),
                                     _ptr(segm_expsum), _stream(stream)))
    return segm_output, segm_max, segm_expsum


def merge_segments(segm_output, segm_max, segm_expsum, part_lens, tile_size: int, *, sinks=None,
                   out_dtype=torch.bfloat16, out=None, lse=None, stream=None):
    """Output [T, H, 512] (out_dtype) and natural-log LSE [T, H] fp32."""
    T, H, S, D = segm_output.shape
    check_sinks(sinks, H)
    if part_lens.dtype != torch.int32 or part_lens.shape != (T,):
        raise ValueError("part_lens must be int32 [T]")
    if out is None:
        out = torch.empty((T, H, D), dtype=out_dtype, device=segm_output.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=segm_output.device)
    _check(lib().mla_merge_segments(_ptr(segm_output), _ptr(segm_max), _ptr(segm_expsum),
                                    _ptr(part_lens), T, H, S, D, int(tile_size), _ptr(sinks),
                                    _ptr(out), _out_code(out.dtype), _ptr(lse), _stream(stream)))
    return out, lse


def decode(q, kv_cache, block_table, seq_lens, *, softmax_scale: float, max_seq_len: int,
           qo_indptr=None, max_qlen=None, causal=False, q_scale=None, kv_scale=None, sinks=None,
           tile_size: int = 0, num_segments: int = 0, sum_seq_lens: int = 0, max_workgroups: int = 0,
           out_dtype=torch.bfloat16, out=None, lse=None, workspace=None, bt_indptr=None, q_pe=None,
           schedule: str = "segments", stream=None):
    """Fused decode: returns (out [T, H, 512], lse [T, H]).  schedule
    "segments" uses the segment partition (num_segments 0 = the planner's S),
    "balanced" the balanced split."""
    p = make_problem(q, kv_cache, block_table, seq_lens, softmax_scale=softmax_scale,
                     max_seq_len=max_seq_len, qo_indptr=qo_indptr, max_qlen=max_qlen, causal=causal,
                     q_scale=q_scale, kv_scale=kv_scale, tile_size=tile_size,
                     num_segments=num_segments, sum_seq_lens=sum_seq_lens, max_workgroups=max_workgroups,
                     bt_indptr=bt_indptr, q_pe=q_pe, schedule=schedule)
    T, H = q.shape[0], q.shape[1]
    check_sinks(sinks, H)
    if out is None:
        out = torch.empty((T, H, KV_LORA_RANK), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=q.device)
    need = workspace_bytes(p)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    _check(lib().mla_decode(ctypes.byref(p), _ptr(sinks), _ptr(out), _out_code(out.dtype), _ptr(lse),
                            _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(stream)))
    return out, lse


def decode_no_alloc(q, kv_cache, block_table, seq_lens, *, softmax_scale: float, max_seq_len: int, out, lse,
                    qo_indptr=None, max_qlen=None, causal=False, q_scale=None, kv_scale=None, sinks=None,
                    tile_size: int = 0, num_segments: int = 0, sum_seq_lens: int = 0, max_workgroups: int = 0,
                    bt_indptr=None, q_pe=None, schedule: str = "segments", stream=None):
    """mla_decode_no_alloc: the fused decode with the library's static device
    scratch instead of a workspace (out [T, H, 512] and lse [T, H] are given
    by the caller; nothing is allocated).  Calls on one GPU share the scratch
    and must not overlap."""
    p = make_problem(q, kv_cache, block_table, seq_lens, softmax_scale=softmax_scale,
                     max_seq_len=max_seq_len, qo_indptr=qo_indptr, max_qlen=max_qlen, causal=causal,
                     q_scale=q_scale, kv_scale=kv_scale, tile_size=tile_size,
                     num_segments=num_segments, sum_seq_lens=sum_seq_lens, max_workgroups=max_workgroups,
                     bt_indptr=bt_indptr, q_pe=q_pe, schedule=schedule)
    check_sinks(sinks, q.shape[1])
    _check(lib().mla_decode_no_alloc(ctypes.byref(p), _ptr(sinks), _ptr(out), _out_code(out.dtype), _ptr(lse),
                                     _stream(stream)))
    return out, lse


def combine_lse(shard_out, shard_lse, *, sinks=None, out_dtype=torch.bfloat16, out=None, lse=None,
                stream=None):
    """Cross-shard combine (decode context parallelism): shard_out
    [W, T, H, 512] (bf16 / fp16 / fp32) and shard_lse [W, T, H] fp32 from W
    sink-free decodes of disjoint key shards -> (out [T, H, 512], lse [T, H]),
    with the sinks applied once to the combined rows."""
    if shard_out.ndim != 4 or shard_out.shape[-1] != KV_LORA_RANK or not shard_out.is_contiguous():
        raise ValueError(f"shard_out must be a contiguous [W, T, H, 512] tensor, got {tuple(shard_out.shape)}")
    W, T, H, _ = shard_out.shape
    if shard_lse.shape != (W, T, H) or shard_lse.dtype != torch.float32 or not shard_lse.is_contiguous():
        raise ValueError("shard_lse must be a contiguous float32 [W, T, H] tensor")
    check_sinks(sinks, H)
    if out is None:
        out = torch.empty((T, H, KV_LORA_RANK), dtype=out_dtype, device=shard_out.device)
    if lse is None:
        lse = torch.empty((T, H), dtype=torch.float32, device=shard_out.device)
    _check(lib().mla_combine_lse(_ptr(shard_out), _out_code(shard_out.dtype), _ptr(shard_lse), W, T, H,
                                 _ptr(sinks), _ptr(out), _out_code(out.dtype), _ptr(lse), _stream(stream)))
    return out, lse


class Decoder:
    """A prepared ``mla_decode`` call for a fixed batch layout.

    The descriptor, segment count, workspace and outputs are set up once; each
    ``run()`` is one C call (no per-call Python argument processing), which is
    what a serving loop re-issues every step.  The tensors passed here must stay
    alive and keep their addresses; their contents may change between runs.
    """

    def __init__(self, q, kv_cache, block_table, seq_lens, *, softmax_scale: float, max_seq_len: int,
                 qo_indptr=None, max_qlen=None, causal=False, q_scale=None, kv_scale=None, sinks=None,
                 tile_size: int = 0, num_segments: int = 0, sum_seq_lens: int = 0,
                 max_workgroups: int = 0, out_dtype=torch.bfloat16, bt_indptr=None, out=None, lse=None,
                 q_pe=None, schedule: str = "segments"):
        self.p = make_problem(q, kv_cache, block_table, seq_lens, softmax_scale=softmax_scale,
                              max_seq_len=max_seq_len, qo_indptr=qo_indptr, max_qlen=max_qlen,
                              causal=causal, q_scale=q_scale, kv_scale=kv_scale, tile_size=tile_size,
                              num_segments=num_segments, sum_seq_lens=sum_seq_lens,
                              max_workgroups=max_workgroups, bt_indptr=bt_indptr, q_pe=q_pe,
                              schedule=schedule)
        check_sinks(sinks, q.shape[1])
        # The balanced split (split_workgroups > 0), or the segment partition
        # with the resolved S (the planner's when num_segments == 0).
        self.split = split_plan(self.p)
        self.split_workgroups = self.split[0] if self.split else 0
        self.num_segments = 0 if self.split else resolve_num_segments(self.p)
        self.p.num_segments = self.num_segments
        T, H = q.shape[0], q.shape[1]
        # out / lse may be given (e.g. one shard's slice of a stacked buffer)
        self.out = torch.empty((T, H, KV_LORA_RANK), dtype=out_dtype, device=q.device) if out is None else out
        self.lse = torch.empty((T, H), dtype=torch.float32, device=q.device) if lse is None else lse
        if tuple(self.out.shape) != (T, H, KV_LORA_RANK) or not self.out.is_contiguous() or \
                tuple(self.lse.shape) != (T, H) or self.lse.dtype != torch.float32 or not self.lse.is_contiguous():
            raise ValueError("out must be a contiguous [T, H, 512] tensor and lse a contiguous float32 [T, H]")
        out_dtype = self.out.dtype
        self.workspace = torch.empty(max(workspace_bytes(self.p), 256), dtype=torch.uint8, device=q.device)
        self._keep = (q, kv_cache, block_table, seq_lens, qo_indptr, q_scale, kv_scale, sinks, bt_indptr, q_pe)
        self._fn = lib().mla_decode
        self._args = (ctypes.byref(self.p), _ptr(sinks), _ptr(self.out), _out_code(out_dtype), _ptr(self.lse),
                      _ptr(self.workspace), self.workspace.numel())

    def run(self, stream=None):
        _check(self._fn(*self._args, _stream(stream)))
        return self.out, self.lse

    def run_stage(self, stage: int, stream=None):
        """One of the two launches of ``run`` (1: cache stream, 2: merge)."""
        _check(lib().mla_decode_stage(*self._args, int(stage), _stream(stream)))
        return self.out, self.lse
