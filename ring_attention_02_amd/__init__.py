"""MI355X-native blockwise ring attention: thin Python binding of libringattn.so.

Every function here only marshals arguments for the C ABI declared in
``include/ringattn.h``; all the work runs in the library (host index code in
C++, attention / merge / decode in HIP kernels for gfx950).  PyTorch is used
for device memory and streams only.  Importing this package fails loudly
when the library has not been built (``python ring_attention_02_amd/build.py``):
there is no fallback implementation.
"""

import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libringattn.so")

CP_OK, CP_EINVAL, CP_EDTYPE, CP_EUNSUPPORTED, CP_EHIP = 0, 1, 2, 3, 4
CP_BF16, CP_F32 = 0, 1
CP_MASK_NONE, CP_MASK_CAUSAL = 0, 1
FULL, DIAG, SKIP = 0, 1, 2
ABI_VERSION = 3

# Every symbol include/ringattn.h declares.
EXPORTED = ("cp_abi_version", "cp_status_string", "cp_last_error", "cp_partition",
            "cp_slot_mapping", "cp_classify", "ring_attn_step", "lse_merge",
            "split_kv_decode_workspace", "split_kv_decode", "ring_stage_copy",
            "ring_attn_step_jobs", "split_kv_decode_paged", "ring_attn_step_varlen",
            "cp_gather_rows", "cp_reorg_index", "cp_ring_schedule", "split_kv_decode_noalloc")


class RingAttnError(RuntimeError):
    def __init__(self, status, func, detail):
        super().__init__(f"{func}: status {status} ({detail})")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python ring_attention_02_amd/build.py`")

_lib = ctypes.CDLL(LIB_PATH)
_i32, _i64, _f32, _vp, _sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t
_pi64, _pi32 = ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)

_lib.cp_abi_version.restype = _i32
_lib.cp_abi_version.argtypes = []
_lib.cp_status_string.restype = ctypes.c_char_p
_lib.cp_status_string.argtypes = [_i32]
_lib.cp_last_error.restype = ctypes.c_char_p
_lib.cp_last_error.argtypes = []
_lib.cp_partition.restype = _i32
_lib.cp_partition.argtypes = [_vp, _i32, _i32, _i32, _vp, _pi64, _vp, _pi64]
_lib.cp_slot_mapping.restype = _i32
_lib.cp_slot_mapping.argtypes = [_vp, _i64, _i32, _i32, _i32, _i32, _vp, _i64, _vp, _vp]
_lib.cp_classify.restype = _i32
_lib.cp_classify.argtypes = [_i64, _i64, _i64, _i64, _i32, _pi32]
_lib.cp_reorg_index.restype = _i32
_lib.cp_reorg_index.argtypes = [_vp, _i32, _i32, _i32, _i32, _i32, _vp, _pi64, _vp, _i64]
_lib.cp_ring_schedule.restype = _i32
_lib.cp_ring_schedule.argtypes = [_i32, _i32, _vp, _vp]
_lib.ring_attn_step.restype = _i32
_lib.ring_attn_step.argtypes = [_vp, _vp, _vp, _i32, _i32, _i64, _i64, _i32, _i32, _i32, _i32,
                                _i64, _i64, _i32, _f32, _i32, _vp, _vp, _pi32, _vp]
_lib.lse_merge.restype = _i32
_lib.lse_merge.argtypes = [_vp, _vp, _i32, _i64, _i32, _vp, _i32, _vp, _vp]
_lib.split_kv_decode_workspace.restype = _sz
_lib.split_kv_decode_workspace.argtypes = [_i32, _i32, _i32, _i32, _i32, _i64]
_lib.split_kv_decode.restype = _i32
_lib.split_kv_decode.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i64, _vp, _i32, _i32, _i32,
                                 _i32, _f32, _vp, _vp, _vp, _sz, _vp]
_lib.split_kv_decode_noalloc.restype = _i32
_lib.split_kv_decode_noalloc.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i64, _vp, _i32, _i32, _i32,
                                         _i32, _f32, _vp, _vp, _vp]
_lib.split_kv_decode_paged.restype = _i32
_lib.split_kv_decode_paged.argtypes = [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _vp, _i32, _vp,
                                       _i32, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _sz, _vp]
_lib.ring_attn_step_varlen.restype = _i32
_lib.ring_attn_step_varlen.argtypes = [_vp, _vp, _vp, _i32, _i32, _vp, _vp, _vp, _vp, _i32,
                                       _i32, _i32, _i32, _i32, _f32, _i32, _vp, _vp, _vp]
_lib.cp_gather_rows.restype = _i32
_lib.cp_gather_rows.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp]
_lib.ring_stage_copy.restype = _i32
_lib.ring_stage_copy.argtypes = [_vp, _vp, _vp, _i32, _vp]


class _KvSegment(ctypes.Structure):          # cp_kv_segment_t
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("sk", ctypes.c_int64),
                ("k_pos0", ctypes.c_int64)]


class _AttnJob(ctypes.Structure):            # cp_attn_job_t
    _fields_ = [("q", ctypes.c_void_p), ("o", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("q_pos0", ctypes.c_int64), ("accumulate", ctypes.c_int32),
                ("n_segments", ctypes.c_int32), ("segments", _KvSegment * 4)]


class _Copy(ctypes.Structure):                # cp_copy_t
    _fields_ = [("dst", ctypes.c_void_p), ("src", ctypes.c_void_p), ("bytes", ctypes.c_int64)]


_lib.ring_attn_step_jobs.restype = _i32
_lib.ring_attn_step_jobs.argtypes = [_vp, _i32, _vp, _i32, _i32, _i32, _i64, _i32, _i32, _i32,
                                     _i32, _i32, _f32, _vp]
MAX_JOBS, MAX_SEGMENTS, MAX_FORWARD = 4, 4, 4

if _lib.cp_abi_version() != ABI_VERSION:
    raise ImportError(f"libringattn ABI {_lib.cp_abi_version()} != binding ABI {ABI_VERSION}")


def lib():
    """The loaded ctypes library (for ABI-level tests)."""
    return _lib


def last_error():
    return _lib.cp_last_error().decode()


def _check(status, func):
    if status != CP_OK:
        raise RingAttnError(status, func, last_error() or _lib.cp_status_string(status).decode())


def _np_ptr(a):
    return ctypes.c_void_p(a.ctypes.data) if a is not None and a.size else None


# ---------------------------------------------------------------------------
# host index functions
# ---------------------------------------------------------------------------

def partition(seq_lens, cp_size, rank):
    """Head-tail (zigzag) partition: (local token ids of `rank`, restore index)."""
    lens = np.ascontiguousarray(seq_lens, dtype=np.int64)
    llen, rlen = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(_lib.cp_partition(_np_ptr(lens), len(lens), cp_size, rank, None, ctypes.byref(llen),
                             None, ctypes.byref(rlen)), "cp_partition")
    local = np.empty(llen.value, dtype=np.int64)
    restore = np.empty(rlen.value, dtype=np.int64)
    _check(_lib.cp_partition(_np_ptr(lens), len(lens), cp_size, rank, _np_ptr(local),
                             ctypes.byref(llen), _np_ptr(restore), ctypes.byref(rlen)),
           "cp_partition")
    return local, restore


def slot_mapping(positions, block_size, interleave, pcp_size, dcp_size, block_table=None):
    """Interleaved virtual-block placement: (device int32[n], slot int64[n])."""
    pos = np.ascontiguousarray(positions, dtype=np.int64)
    dev = np.empty(pos.size, dtype=np.int32)
    slot = np.empty(pos.size, dtype=np.int64)
    table = None if block_table is None else np.ascontiguousarray(block_table, dtype=np.int32)
    _check(_lib.cp_slot_mapping(_np_ptr(pos), pos.size, block_size, interleave, pcp_size,
                                dcp_size, _np_ptr(table), 0 if table is None else table.size,
                                _np_ptr(dev), _np_ptr(slot)), "cp_slot_mapping")
    return dev, slot


def reorg_index(seq_lens, block_size, interleave, pcp_size, dcp_size):
    """Rows of an all-gathered KV buffer in request order: (src_idx int64[sum L],
    dev_lens int64[W, num_reqs])."""
    lens = np.ascontiguousarray(seq_lens, dtype=np.int64)
    n = ctypes.c_int64(0)
    W = pcp_size * dcp_size
    dev_lens = np.zeros((W, lens.size), dtype=np.int64)
    _check(_lib.cp_reorg_index(_np_ptr(lens), lens.size, block_size, interleave, pcp_size, dcp_size,
                               None, ctypes.byref(n), _np_ptr(dev_lens), dev_lens.size),
           "cp_reorg_index")
    src = np.empty(n.value, dtype=np.int64)
    if n.value:
        _check(_lib.cp_reorg_index(_np_ptr(lens), lens.size, block_size, interleave, pcp_size,
                                   dcp_size, _np_ptr(src), ctypes.byref(n), None, 0), "cp_reorg_index")
    return src, dev_lens


def ring_schedule(cp_size, rank):
    """Ring order of `rank`: (src_rank int32[cp], parts int32[cp, 2]) -- the rank
    whose K/V block it computes with at each step, and that block's head and
    tail sequence parts under the head-tail partition."""
    src = np.empty(cp_size, dtype=np.int32)
    parts = np.empty((cp_size, 2), dtype=np.int32)
    _check(_lib.cp_ring_schedule(rank, cp_size, _np_ptr(src), _np_ptr(parts)), "cp_ring_schedule")
    return src, parts


def classify(q_pos0, sq, k_pos0, sk, causal=True):
    out = ctypes.c_int32(-1)
    _check(_lib.cp_classify(q_pos0, sq, k_pos0, sk, CP_MASK_CAUSAL if causal else CP_MASK_NONE,
                            ctypes.byref(out)), "cp_classify")
    return out.value


# ---------------------------------------------------------------------------
# device functions (torch tensors: memory and streams only)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return CP_BF16
    if t.dtype == torch.float32:
        return CP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev_ptr(t, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def ring_attn_step(q, k, v, o, lse, q_pos0=0, k_pos0=0, causal=True, scale=None,
                   accumulate=False, stream=None):
    """One (Q chunk, KV block) ring step; returns the pair's class (FULL/DIAG/SKIP).

    q [B,Sq,Hq,Dqk], k [B,Sk,Hkv,Dqk], v [B,Sk,Hkv,Dv] (bf16 or float32);
    o [B,Sq,Hq,Dv] float32 and lse [B,Sq,Hq] float32 are written (or merged
    into when accumulate=True).
    """
    torch = _torch()
    B, Sq, Hq, Dqk = q.shape
    Bk, Sk, Hkv, Dk = k.shape
    Dv = v.shape[3]
    if Bk != B or Dk != Dqk or tuple(v.shape[:3]) != (B, Sk, Hkv):
        raise ValueError("q/k/v shapes do not agree")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k and v must share a dtype")
    if tuple(o.shape) != (B, Sq, Hq, Dv) or o.dtype != torch.float32:
        raise ValueError("o must be float32 [B, Sq, Hq, Dv]")
    if tuple(lse.shape) != (B, Sq, Hq) or lse.dtype != torch.float32:
        raise ValueError("lse must be float32 [B, Sq, Hq]")
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    cls = ctypes.c_int32(-1)
    _check(_lib.ring_attn_step(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"),
                               _dtype_code(q), B, Sq, Sk, Hq, Hkv, Dqk, Dv, int(q_pos0),
                               int(k_pos0), CP_MASK_CAUSAL if causal else CP_MASK_NONE,
                               float(scale), 1 if accumulate else 0, _dev_ptr(o, "o"),
                               _dev_ptr(lse, "lse"), ctypes.byref(cls), _stream_handle(stream)),
           "ring_attn_step")
    return cls.value


def ring_attn_step_jobs(jobs, causal=True, scale=None, stream=None, forward=()):
    """One launch for up to 4 query chunks, each over up to 4 K/V segments.

    jobs: list of dicts with q [B,Sq,Hq,Dqk] (bf16), o [B,Sq,Hq,Dv] / lse [B,Sq,Hq]
    (float32), q_pos0, accumulate, and segments = [(k, v, k_pos0), ...] with
    k [B,Sk,Hkv,Dqk], v [B,Sk,Hkv,Dv].  Every job's result is attention over
    the union of its segments' keys, written to (or LSE-merged into) o / lse.
    forward: up to 4 (dst, src) pairs of equally sized contiguous GPU tensors
    that the same launch copies while it computes (the block passed on
    around the ring); no dst may overlap anything else the launch touches.
    """
    torch = _torch()
    if not 1 <= len(jobs) <= MAX_JOBS:
        raise ValueError(f"ring_attn_step_jobs takes 1..{MAX_JOBS} jobs")
    q0 = jobs[0]["q"]
    B, Sq, Hq, Dqk = q0.shape
    Hkv, Dv = None, jobs[0]["o"].shape[3]
    arr = (_AttnJob * len(jobs))()
    for i, jb in enumerate(jobs):
        q, o, lse = jb["q"], jb["o"], jb["lse"]
        if tuple(q.shape) != (B, Sq, Hq, Dqk) or q.dtype != torch.bfloat16:
            raise ValueError("all jobs need bf16 q of one shape [B, Sq, Hq, Dqk]")
        if tuple(o.shape) != (B, Sq, Hq, Dv) or o.dtype != torch.float32:
            raise ValueError("o must be float32 [B, Sq, Hq, Dv]")
        if tuple(lse.shape) != (B, Sq, Hq) or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [B, Sq, Hq]")
        segs = jb.get("segments", [])
        if len(segs) > MAX_SEGMENTS:
            raise ValueError(f"at most {MAX_SEGMENTS} segments per job")
        arr[i].q, arr[i].o, arr[i].lse = (_dev_ptr(q, "q").value, _dev_ptr(o, "o").value,
                                          _dev_ptr(lse, "lse").value)
        arr[i].q_pos0 = int(jb.get("q_pos0", 0))
        arr[i].accumulate = 1 if jb.get("accumulate", False) else 0
        arr[i].n_segments = len(segs)
        for j, (k, v, k_pos0) in enumerate(segs):
            if k.shape[0] != B or k.shape[3] != Dqk or tuple(v.shape[:3]) != tuple(k.shape[:3]) \
                    or v.shape[3] != Dv or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
                raise ValueError("segment k/v shapes or dtypes do not agree with q / o")
            Hkv = k.shape[2] if Hkv is None else Hkv
            if k.shape[2] != Hkv:
                raise ValueError("all segments need the same kv heads")
            arr[i].segments[j] = _KvSegment(_dev_ptr(k, "k").value, _dev_ptr(v, "v").value,
                                            k.shape[1], int(k_pos0))
    if Hkv is None:
        Hkv = Hq
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    if len(forward) > MAX_FORWARD:
        raise ValueError(f"at most {MAX_FORWARD} forwarded ranges")
    fwd = (_Copy * max(1, len(forward)))()
    for i, (dst, src) in enumerate(forward):
        nbytes = dst.numel() * dst.element_size()
        if nbytes != src.numel() * src.element_size():
            raise ValueError("forward: dst and src sizes differ")
        fwd[i] = _Copy(_dev_ptr(dst, "forward dst").value, _dev_ptr(src, "forward src").value, nbytes)
    _check(_lib.ring_attn_step_jobs(ctypes.cast(arr, ctypes.c_void_p), len(jobs),
                                    ctypes.cast(fwd, ctypes.c_void_p), len(forward), CP_BF16, B, Sq,
                                    Hq, Hkv, Dqk, Dv, CP_MASK_CAUSAL if causal else CP_MASK_NONE,
                                    float(scale), _stream_handle(stream)), "ring_attn_step_jobs")


def lse_merge(o_parts, lse_parts, o_out=None, lse_out=None, out_dtype=None, stream=None):
    """Merge partials o_parts [n, ..., Dv] / lse_parts [n, ...]; returns (o, lse)."""
    torch = _torch()
    n = o_parts.shape[0]
    dv = o_parts.shape[-1]
    rows_shape = tuple(o_parts.shape[1:-1])
    if tuple(lse_parts.shape) != (n, *rows_shape):
        raise ValueError("lse_parts shape does not match o_parts")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("partials must be float32")
    rows = int(np.prod(rows_shape)) if rows_shape else 1
    out_dtype = out_dtype or torch.float32
    if o_out is None:
        o_out = torch.empty((*rows_shape, dv), dtype=out_dtype, device=o_parts.device)
    if lse_out is None:
        lse_out = torch.empty(rows_shape, dtype=torch.float32, device=o_parts.device)
    _check(_lib.lse_merge(_dev_ptr(o_parts, "o_parts"), _dev_ptr(lse_parts, "lse_parts"), n, rows,
                          dv, _dev_ptr(o_out, "o_out"), _dtype_code(o_out),
                          _dev_ptr(lse_out, "lse_out"), _stream_handle(stream)), "lse_merge")
    return o_out, lse_out


def split_kv_decode_workspace(n_shards, batch, hq, hkv, d_v, t_shard):
    return int(_lib.split_kv_decode_workspace(n_shards, batch, hq, hkv, d_v, t_shard))


def split_kv_decode(q, k_shards, v_shards, shard_lens=None, scale=None, o_parts=None,
                    lse_parts=None, workspace=None, stream=None):
    """Per-shard decode partials: q [B,Hq,D], shards [S,B,T,Hkv,D] -> (o_parts, lse_parts)."""
    torch = _torch()
    B, Hq, Dqk = q.shape
    S, Bk, T, Hkv, Dk = k_shards.shape
    Dv = v_shards.shape[4]
    if Bk != B or Dk != Dqk or tuple(v_shards.shape[:4]) != (S, B, T, Hkv):
        raise ValueError("q / shard shapes do not agree")
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    if o_parts is None:
        o_parts = torch.empty((S, B, Hq, Dv), dtype=torch.float32, device=q.device)
    if lse_parts is None:
        lse_parts = torch.empty((S, B, Hq), dtype=torch.float32, device=q.device)
    ws_need = split_kv_decode_workspace(S, B, Hq, Hkv, Dv, T)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    lens_ptr = None
    if shard_lens is not None:
        if shard_lens.dtype != torch.int64 or tuple(shard_lens.shape) != (S, B):
            raise ValueError("shard_lens must be int64 [n_shards, batch]")
        lens_ptr = _dev_ptr(shard_lens, "shard_lens")
    _check(_lib.split_kv_decode(_dev_ptr(q, "q"), _dev_ptr(k_shards, "k_shards"),
                                _dev_ptr(v_shards, "v_shards"), _dtype_code(q), S, B, T, lens_ptr,
                                Hq, Hkv, Dqk, Dv, float(scale), _dev_ptr(o_parts, "o_parts"),
                                _dev_ptr(lse_parts, "lse_parts"),
                                None if workspace is None else _dev_ptr(workspace, "workspace"),
                                0 if workspace is None else workspace.numel() * workspace.element_size(),
                                _stream_handle(stream)), "split_kv_decode")
    return o_parts, lse_parts


def split_kv_decode_noalloc(q, k_shards, v_shards, o_parts, lse_parts, shard_lens=None, scale=None,
                            stream=None):
    """split_kv_decode into caller-given o_parts / lse_parts, with the key-split
    partials in the library's static scratch array: the call allocates nothing."""
    B, Hq, Dqk = q.shape
    S, Bk, T, Hkv, Dk = k_shards.shape
    Dv = v_shards.shape[4]
    if Bk != B or Dk != Dqk or tuple(v_shards.shape[:4]) != (S, B, T, Hkv):
        raise ValueError("q / shard shapes do not agree")
    if tuple(o_parts.shape) != (S, B, Hq, Dv) or tuple(lse_parts.shape) != (S, B, Hq):
        raise ValueError("o_parts must be [S, B, Hq, Dv] and lse_parts [S, B, Hq]")
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    lens_ptr = None
    if shard_lens is not None:
        if tuple(shard_lens.shape) != (S, B):
            raise ValueError("shard_lens must be int64 [n_shards, batch]")
        lens_ptr = _dev_ptr(shard_lens, "shard_lens")
    _check(_lib.split_kv_decode_noalloc(_dev_ptr(q, "q"), _dev_ptr(k_shards, "k_shards"),
                                        _dev_ptr(v_shards, "v_shards"), _dtype_code(q), S, B, T, lens_ptr,
                                        Hq, Hkv, Dqk, Dv, float(scale), _dev_ptr(o_parts, "o_parts"),
                                        _dev_ptr(lse_parts, "lse_parts"), _stream_handle(stream)),
           "split_kv_decode_noalloc")
    return o_parts, lse_parts


def split_kv_decode_paged(q, k_pool, v_pool, block_tables, shard_lens, scale=None, o_parts=None,
                          lse_parts=None, workspace=None, stream=None):
    """Per-shard decode partials over paged caches.

    q [B,Hq,D]; k_pool / v_pool [S, num_blocks, block_size, Hkv, D] (one pool
    per shard); block_tables int32 [S, B, max_blocks] (physical block of each
    logical block); shard_lens int64 [S, B].  Returns (o_parts [S,B,Hq,Dv],
    lse_parts [S,B,Hq]).
    """
    torch = _torch()
    B, Hq, Dqk = q.shape
    S, NB, BS, Hkv, Dk = k_pool.shape
    Dv = v_pool.shape[4]
    if Dk != Dqk or tuple(v_pool.shape[:4]) != (S, NB, BS, Hkv):
        raise ValueError("q / pool shapes do not agree")
    if block_tables.dtype != torch.int32 or block_tables.dim() != 3 or \
            tuple(block_tables.shape[:2]) != (S, B):
        raise ValueError("block_tables must be int32 [n_shards, batch, max_blocks]")
    if shard_lens.dtype != torch.int64 or tuple(shard_lens.shape) != (S, B):
        raise ValueError("shard_lens must be int64 [n_shards, batch]")
    MB = block_tables.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    if o_parts is None:
        o_parts = torch.empty((S, B, Hq, Dv), dtype=torch.float32, device=q.device)
    if lse_parts is None:
        lse_parts = torch.empty((S, B, Hq), dtype=torch.float32, device=q.device)
    ws_need = split_kv_decode_workspace(S, B, Hq, Hkv, Dv, MB * BS)
    if workspace is None and ws_need:
        workspace = torch.empty(ws_need, dtype=torch.uint8, device=q.device)
    _check(_lib.split_kv_decode_paged(
        _dev_ptr(q, "q"), _dev_ptr(k_pool, "k_pool"), _dev_ptr(v_pool, "v_pool"), _dtype_code(q), S, B,
        NB, BS, _dev_ptr(block_tables, "block_tables"), MB, _dev_ptr(shard_lens, "shard_lens"), Hq, Hkv,
        Dqk, Dv, float(scale), _dev_ptr(o_parts, "o_parts"), _dev_ptr(lse_parts, "lse_parts"),
        None if workspace is None else _dev_ptr(workspace, "workspace"),
        0 if workspace is None else workspace.numel() * workspace.element_size(),
        _stream_handle(stream)), "split_kv_decode_paged")
    return o_parts, lse_parts


def ring_attn_step_varlen(q, k, v, cu_seqlens_q, cu_seqlens_k, q_pos0, k_pos0, o=None, lse=None,
                          causal=True, scale=None, accumulate=False, stream=None):
    """One ring step for packed requests: q [Tq,Hq,Dqk], k [Tk,Hkv,Dqk], v [Tk,Hkv,Dv] (bf16);
    cu_seqlens_* / *_pos0 are host int64 sequences (per request).  Returns (o, lse) with
    o [Tq,Hq,Dv] and lse [Tq,Hq] float32 (written, or LSE-merged when accumulate)."""
    torch = _torch()
    Tq, Hq, Dqk = q.shape
    Tk, Hkv, Dk = k.shape
    Dv = v.shape[2]
    if Dk != Dqk or tuple(v.shape[:2]) != (Tk, Hkv):
        raise ValueError("q / k / v shapes do not agree")
    cq = np.ascontiguousarray(cu_seqlens_q, dtype=np.int64)
    ck = np.ascontiguousarray(cu_seqlens_k, dtype=np.int64)
    pq = np.ascontiguousarray(q_pos0, dtype=np.int64)
    pk = np.ascontiguousarray(k_pos0, dtype=np.int64)
    n = pq.size
    if cq.size != n + 1 or ck.size != n + 1 or pk.size != n:
        raise ValueError("cu_seqlens need n_req + 1 entries, positions n_req")
    if cq[-1] > Tq or ck[-1] > Tk:
        raise ValueError("cu_seqlens run past the packed tensors")
    if o is None:
        o = torch.empty((Tq, Hq, Dv), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((Tq, Hq), dtype=torch.float32, device=q.device)
    if tuple(o.shape) != (Tq, Hq, Dv) or tuple(lse.shape) != (Tq, Hq):
        raise ValueError("o / lse shapes do not agree with q")
    if scale is None:
        scale = 1.0 / math.sqrt(Dqk)
    _check(_lib.ring_attn_step_varlen(_dev_ptr(q, "q"), _dev_ptr(k, "k"), _dev_ptr(v, "v"), _dtype_code(q),
                                      n, _np_ptr(cq), _np_ptr(ck), _np_ptr(pq), _np_ptr(pk), Hq, Hkv,
                                      Dqk, Dv, CP_MASK_CAUSAL if causal else CP_MASK_NONE, float(scale),
                                      1 if accumulate else 0, _dev_ptr(o, "o"), _dev_ptr(lse, "lse"),
                                      _stream_handle(stream)), "ring_attn_step_varlen")
    return o, lse


def gather_rows(src, idx, dst=None, stream=None):
    """dst[i] = src[idx[i]] along dim 0 on the device (idx: int64 GPU tensor)."""
    torch = _torch()
    n = idx.numel()
    if idx.dtype != torch.int64:
        raise ValueError("idx must be int64")
    if dst is None:
        dst = torch.empty((n, *src.shape[1:]), dtype=src.dtype, device=src.device)
    row_bytes = src[0].numel() * src.element_size() if src.shape[0] else dst[0].numel() * dst.element_size()
    if tuple(dst.shape[1:]) != tuple(src.shape[1:]) or dst.shape[0] != n or dst.dtype != src.dtype:
        raise ValueError("dst must be [len(idx), *src.shape[1:]] of src's dtype")
    _check(_lib.cp_gather_rows(_dev_ptr(dst, "dst"), _dev_ptr(src, "src"), _dev_ptr(idx, "idx"), n,
                               src.shape[0], row_bytes, _stream_handle(stream)), "cp_gather_rows")
    return dst


def stage_copy(pairs, stream=None):
    """Copy each (dst, src) pair of equally sized contiguous GPU tensors in one launch."""
    n = len(pairs)
    dsts = (ctypes.c_void_p * n)()
    srcs = (ctypes.c_void_p * n)()
    nbytes = (ctypes.c_int64 * n)()
    for i, (dst, src) in enumerate(pairs):
        if dst.numel() * dst.element_size() != src.numel() * src.element_size():
            raise ValueError("stage_copy: piece sizes differ")
        dsts[i] = _dev_ptr(dst, "dst").value
        srcs[i] = _dev_ptr(src, "src").value
        nbytes[i] = dst.numel() * dst.element_size()
    _check(_lib.ring_stage_copy(dsts, srcs, nbytes, n, _stream_handle(stream)), "ring_stage_copy")


from .ring import ZigzagRing, segmented_prefill, noncausal_ring_sweep  # noqa: E402

__all__ = ["partition", "slot_mapping", "reorg_index", "ring_schedule", "classify", "ring_attn_step", "ring_attn_step_jobs",
           "lse_merge", "stage_copy",
           "split_kv_decode", "split_kv_decode_workspace", "split_kv_decode_paged",
           "split_kv_decode_noalloc",
           "ring_attn_step_varlen", "gather_rows", "ZigzagRing", "segmented_prefill",
           "noncausal_ring_sweep", "RingAttnError", "FULL", "DIAG", "SKIP", "EXPORTED", "lib",
           "last_error"]
