"""ctypes binding of libmapflow.so (include/mapflow.h).

Argument marshalling only: every step of the path runs in the HIP kernels of
the library.  Torch tensors supply device memory and the current stream.
The binding refuses to work without the built library: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmapflow.so")

MF_OK, MF_ERR_INVALID, MF_ERR_UNSUPPORTED, MF_ERR_CAPACITY, MF_ERR_HIP, MF_ERR_WORKSPACE = range(6)
MF_F32, MF_BF16 = 0, 1
MF_MAX_KEYS = 40448
MF_MAX_LAYERS = 256
MF_MAX_RECEIVERS = 4
EXPORTS = ("mf_plan", "mf_block_stats", "mf_block_stats_workspace_size",
           "mf_compress_workspace_size", "mf_compress_blocks",
           "mf_mapped_attn_v", "mf_mapped_attn_v_multi", "mf_prefix_block_hashes", "mf_map_cache_create",
           "mf_map_cache_destroy", "mf_map_cache_insert", "mf_map_cache_lookup", "mf_map_cache_release",
           "mf_map_cache_splice", "mf_map_cache_get_stats", "mf_headmix_workspace_size", "mf_headmix_gram",
           "mf_headmix_solve", "mf_status_string", "mf_last_error_message", "mf_version",
           "mf_debug_force_portable", "mf_compress_blocks_noalloc", "mf_mapped_split_workspace_size",
           "mf_mapped_attn_v_split", "mf_mfma_probe")
# stages mf_debug_force_portable can send to their portable twins
FORCE_PORTABLE = {"stats": 0x1, "select": 0x2, "extract": 0x4, "mapped": 0x8}

_i32p = ctypes.POINTER(ctypes.c_int32)


class PlanInfo(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("block", ctypes.c_int32),
                ("total_rowblocks", ctypes.c_int32), ("max_colblocks", ctypes.c_int32),
                ("total_q", ctypes.c_int32), ("total_k", ctypes.c_int32),
                ("max_k_len", ctypes.c_int32), ("plan_len", ctypes.c_int32)]


class BatchC(ctypes.Structure):
    _fields_ = [("info", PlanInfo), ("cu_seqlens_q", ctypes.c_void_p),
                ("cu_seqlens_k", ctypes.c_void_p), ("q_pos0", ctypes.c_void_p),
                ("plan", ctypes.c_void_p)]


class SenderDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("num_layers", ctypes.c_int32),
                ("H_s", ctypes.c_int32), ("H_kv_s", ctypes.c_int32),
                ("d", ctypes.c_int32), ("B", ctypes.c_int32), ("sm_scale", ctypes.c_float),
                ("layer_stride_q", ctypes.c_int64), ("layer_stride_k", ctypes.c_int64)]


class ReceiverDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("num_layers", ctypes.c_int32),
                ("sender_layers", ctypes.c_int32), ("layer_map", _i32p),
                ("H_s", ctypes.c_int32), ("H_r", ctypes.c_int32), ("H_kv_r", ctypes.c_int32),
                ("d", ctypes.c_int32), ("B", ctypes.c_int32),
                ("layer_stride_v", ctypes.c_int64), ("layer_stride_o", ctypes.c_int64),
                ("block_table", ctypes.c_void_p), ("page_size", ctypes.c_int32),
                ("max_pages", ctypes.c_int32), ("num_pages", ctypes.c_int64),
                ("csr_capacity", ctypes.c_int64)]


class HeadmixDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("B", ctypes.c_int32), ("num_layers", ctypes.c_int32),
                ("sender_layers", ctypes.c_int32), ("layer_map", _i32p), ("H_s", ctypes.c_int32),
                ("H_r", ctypes.c_int32), ("sender_capacity", ctypes.c_int64),
                ("receiver_capacity", ctypes.c_int64)]


class MapCacheDesc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("num_layers", ctypes.c_int32), ("H_s", ctypes.c_int32),
                ("B", ctypes.c_int32)]


class MapCacheStats(ctypes.Structure):
    _fields_ = [("entries", ctypes.c_int64), ("pinned_entries", ctypes.c_int64),
                ("bytes_used", ctypes.c_int64), ("bytes_capacity", ctypes.c_int64),
                ("blocks_hit", ctypes.c_int64), ("blocks_missed", ctypes.c_int64),
                ("evictions", ctypes.c_int64)]


class MapflowError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


_lib = None


def _status_name(s: int) -> str:
    names = ["MF_OK", "MF_ERR_INVALID", "MF_ERR_UNSUPPORTED", "MF_ERR_CAPACITY", "MF_ERR_HIP", "MF_ERR_WORKSPACE"]
    return names[s] if 0 <= s < len(names) else f"status {s}"


def lib():
    """Load libmapflow.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m cross_model_attention_mf_amd.build_lib`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    L.mf_plan.argtypes = [_i32p, _i32p, _i32p, i32, i32, _i32p, i64, ctypes.POINTER(PlanInfo)]
    L.mf_block_stats.argtypes = [ctypes.POINTER(SenderDesc), ctypes.POINTER(BatchC), vp, vp, vp, vp, vp, sz, vp]
    L.mf_block_stats_workspace_size.argtypes = [ctypes.POINTER(SenderDesc), ctypes.POINTER(BatchC)]
    L.mf_block_stats_workspace_size.restype = sz
    L.mf_compress_workspace_size.argtypes = [ctypes.POINTER(SenderDesc), ctypes.POINTER(BatchC)]
    L.mf_compress_workspace_size.restype = sz
    L.mf_compress_blocks.argtypes = [ctypes.POINTER(SenderDesc), ctypes.POINTER(BatchC), vp, vp, vp, vp,
                                     ctypes.c_float, vp, vp, vp, i64, ctypes.POINTER(i64), vp, sz, vp]
    L.mf_compress_blocks_noalloc.argtypes = [ctypes.POINTER(SenderDesc), ctypes.POINTER(BatchC), vp, vp, vp, vp,
                                             ctypes.c_float, vp, vp, vp, i64, ctypes.POINTER(i64), vp]
    L.mf_mapped_attn_v.argtypes = [ctypes.POINTER(ReceiverDesc), ctypes.POINTER(BatchC), vp, vp, vp, vp,
                                   vp, vp, vp]
    L.mf_mapped_attn_v_multi.argtypes = [ctypes.POINTER(ctypes.POINTER(ReceiverDesc)), ctypes.c_int,
                                         ctypes.POINTER(BatchC), vp, vp, vp, ctypes.POINTER(vp),
                                         ctypes.POINTER(vp), ctypes.POINTER(vp), vp]
    L.mf_mfma_probe.argtypes = [vp, i32, i32, i32, vp]
    L.mf_mfma_probe.restype = ctypes.c_int
    L.mf_mapped_split_workspace_size.argtypes = [ctypes.POINTER(ReceiverDesc), ctypes.POINTER(BatchC)]
    L.mf_mapped_split_workspace_size.restype = sz
    L.mf_mapped_attn_v_split.argtypes = [ctypes.POINTER(ReceiverDesc), ctypes.POINTER(BatchC), vp, vp, vp, vp,
                                         vp, vp, vp, sz, vp]
    u64p = ctypes.POINTER(ctypes.c_uint64)
    L.mf_prefix_block_hashes.argtypes = [_i32p, i64, i32, ctypes.c_uint64, u64p]
    L.mf_prefix_block_hashes.restype = i64
    L.mf_map_cache_create.argtypes = [ctypes.POINTER(MapCacheDesc), vp, sz, ctypes.POINTER(vp)]
    L.mf_map_cache_destroy.argtypes = [vp]
    L.mf_map_cache_destroy.restype = None
    L.mf_map_cache_insert.argtypes = [vp, u64p, i32, _i32p, i32, i32, vp, vp, vp]
    L.mf_map_cache_lookup.argtypes = [vp, u64p, i32]
    L.mf_map_cache_lookup.restype = i32
    L.mf_map_cache_release.argtypes = [vp, u64p, i32]
    L.mf_map_cache_release.restype = None
    L.mf_map_cache_splice.argtypes = [vp, u64p, i32, i32, _i32p, i32, i32, vp, vp, vp, vp, vp, i64,
                                      ctypes.POINTER(i64), vp]
    L.mf_map_cache_get_stats.argtypes = [vp, ctypes.POINTER(MapCacheStats)]
    L.mf_headmix_workspace_size.argtypes = [ctypes.POINTER(HeadmixDesc), ctypes.POINTER(BatchC)]
    L.mf_headmix_workspace_size.restype = sz
    L.mf_headmix_gram.argtypes = [ctypes.POINTER(HeadmixDesc), ctypes.POINTER(BatchC), vp, vp, vp, vp, vp, vp,
                                  vp, vp, vp, sz, vp]
    L.mf_headmix_solve.argtypes = [ctypes.POINTER(HeadmixDesc), vp, vp, ctypes.c_double, vp, vp, vp]
    for f in ("mf_plan", "mf_block_stats", "mf_compress_blocks", "mf_mapped_attn_v", "mf_mapped_attn_v_multi",
              "mf_mapped_attn_v_split",
              "mf_map_cache_create", "mf_map_cache_insert", "mf_map_cache_splice", "mf_map_cache_get_stats",
              "mf_headmix_gram", "mf_headmix_solve"):
        getattr(L, f).restype = ctypes.c_int
    L.mf_status_string.argtypes = [ctypes.c_int]
    L.mf_status_string.restype = ctypes.c_char_p
    L.mf_last_error_message.restype = ctypes.c_char_p
    L.mf_version.restype = ctypes.c_char_p
    L.mf_debug_force_portable.argtypes = [ctypes.c_uint32]
    L.mf_debug_force_portable.restype = ctypes.c_uint32
    _lib = L
    return L


class force_portable:
    """Context manager (tests only): calls inside it run the named stages
    ("stats", "select", "extract", "mapped") on their portable twin kernels."""

    def __init__(self, *stages: str):
        self.mask = 0
        for s in stages:
            self.mask |= FORCE_PORTABLE[s]

    def __enter__(self):
        self.prev = int(lib().mf_debug_force_portable(self.mask))
        return self

    def __exit__(self, *exc):
        lib().mf_debug_force_portable(self.prev)
        return False


def _check(status: int):
    if status != MF_OK:
        raise MapflowError(status, lib().mf_last_error_message().decode())


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def dtype_code(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return MF_BF16
    if t == torch.float32:
        return MF_F32
    raise ValueError(f"unsupported dtype {t}")


def _as_i32(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def plan(cu_seqlens_q: Sequence[int], cu_seqlens_k: Sequence[int],
         q_pos0: Optional[Sequence[int]], B: int):
    """mf_plan on host arrays -> (PlanInfo, int32 plan array)."""
    L = lib()
    cq, ck = _as_i32(cu_seqlens_q), _as_i32(cu_seqlens_k)
    p0 = None if q_pos0 is None else _as_i32(q_pos0)
    ns = cq.shape[0] - 1
    info = PlanInfo()
    args = (cq.ctypes.data_as(_i32p), ck.ctypes.data_as(_i32p),
            None if p0 is None else p0.ctypes.data_as(_i32p), ns, B)
    st = L.mf_plan(*args, None, 0, ctypes.byref(info))
    if st not in (MF_OK, MF_ERR_CAPACITY):
        _check(st)
    buf = np.zeros(max(info.plan_len, 1), dtype=np.int32)
    _check(L.mf_plan(*args, buf.ctypes.data_as(_i32p), buf.shape[0], ctypes.byref(info)))
    return info, buf[: info.plan_len]


class Batch:
    """A packed batch on the device: cu_seqlens, chunk starts and the plan."""

    def __init__(self, cu_seqlens_q, cu_seqlens_k, q_pos0, B: int, device="cuda"):
        self.info, h_plan = plan(cu_seqlens_q, cu_seqlens_k, q_pos0, B)
        self.B = B
        self.cu_q = torch.from_numpy(_as_i32(cu_seqlens_q)).to(device)
        self.cu_k = torch.from_numpy(_as_i32(cu_seqlens_k)).to(device)
        self.q_pos0 = None if q_pos0 is None else torch.from_numpy(_as_i32(q_pos0)).to(device)
        self.plan = torch.from_numpy(h_plan.copy() if h_plan.size else np.zeros(1, np.int32)).to(device)
        self.c = BatchC(self.info, _ptr(self.cu_q), _ptr(self.cu_k), _ptr(self.q_pos0), _ptr(self.plan))

    @property
    def total_rowblocks(self) -> int:
        return self.info.total_rowblocks

    @property
    def max_colblocks(self) -> int:
        return self.info.max_colblocks


def sender_desc(q: torch.Tensor, k: torch.Tensor, B: int, sm_scale: float = 0.0) -> SenderDesc:
    """q [L, Tq, H, d] (or [Tq, H, d]), k [L, Tk, H_kv, d]; contiguous."""
    if q.dim() == 3:
        q, k = q[None], k[None]
    L_, _, H, d = q.shape
    return SenderDesc(dtype_code(q.dtype), L_, H, k.shape[2], d, B, sm_scale,
                      q[0].numel(), k[0].numel())


def block_stats_workspace_size(desc: SenderDesc, batch: Batch) -> int:
    return int(lib().mf_block_stats_workspace_size(ctypes.byref(desc), ctypes.byref(batch.c)))


def block_stats(desc: SenderDesc, batch: Batch, q, k, row_lse, block_mass, workspace=None, stream=None):
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(lib().mf_block_stats(ctypes.byref(desc), ctypes.byref(batch.c), _ptr(q), _ptr(k),
                                _ptr(row_lse), _ptr(block_mass), _ptr(workspace), ws_bytes,
                                _stream(stream)))


def compress_workspace_size(desc: SenderDesc, batch: Batch) -> int:
    return int(lib().mf_compress_workspace_size(ctypes.byref(desc), ctypes.byref(batch.c)))


def compress_blocks(desc: SenderDesc, batch: Batch, q, k, row_lse, block_mass, tau: float,
                    row_ptr, col_idx, values, capacity: int, workspace, sync_count: bool = True,
                    stream=None) -> Optional[int]:
    """Returns the kept-block count when sync_count (one stream sync), else None."""
    nnz = ctypes.c_int64(-1)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = lib().mf_compress_blocks(ctypes.byref(desc), ctypes.byref(batch.c), _ptr(q), _ptr(k),
                                  _ptr(row_lse), _ptr(block_mass), float(tau), _ptr(row_ptr),
                                  _ptr(col_idx), _ptr(values), int(capacity),
                                  ctypes.byref(nnz) if sync_count else None, _ptr(workspace),
                                  ws_bytes, _stream(stream))
    _check(st)
    return int(nnz.value) if sync_count else None


def compress_blocks_noalloc(desc: SenderDesc, batch: Batch, q, k, row_lse, block_mass, tau: float,
                            row_ptr, col_idx, values, capacity: int, sync_count: bool = True,
                            stream=None) -> Optional[int]:
    """compress_blocks without a workspace: the library's static per-GPU
    scratch stands in for it (calls that overlap on one GPU race)."""
    nnz = ctypes.c_int64(-1)
    st = lib().mf_compress_blocks_noalloc(ctypes.byref(desc), ctypes.byref(batch.c), _ptr(q), _ptr(k),
                                          _ptr(row_lse), _ptr(block_mass), float(tau), _ptr(row_ptr),
                                          _ptr(col_idx), _ptr(values), int(capacity),
                                          ctypes.byref(nnz) if sync_count else None, _stream(stream))
    _check(st)
    return int(nnz.value) if sync_count else None


STATIC_SCRATCH_BYTES = 16 << 20   # MF_STATIC_SCRATCH_BYTES


def receiver_desc(v: torch.Tensor, H_s: int, H_r: int, d: int, B: int, layer_map: Sequence[int],
                  sender_layers: int, o_layer_stride: int, csr_capacity: int, block_table=None,
                  page_size: int = 0, v_layer_stride: Optional[int] = None):
    """v: [L, Tk, H_kv_r, d] packed or [L, pages, page_size, H_kv_r, d] paged."""
    lm = _as_i32(layer_map)
    paged = block_table is not None
    H_kv_r = v.shape[-2]
    num_pages = v.shape[1] if paged else 0
    max_pages = block_table.shape[1] if paged else 0
    desc = ReceiverDesc(dtype_code(v.dtype), lm.shape[0], sender_layers, lm.ctypes.data_as(_i32p),
                        H_s, H_r, H_kv_r, d, B,
                        v[0].numel() if v_layer_stride is None else v_layer_stride, o_layer_stride,
                        _ptr(block_table), page_size, max_pages, num_pages, csr_capacity)
    desc._keep = lm  # the layer map must outlive the descriptor
    return desc


def mapped_attn_v(desc: ReceiverDesc, batch: Batch, row_ptr, col_idx, values, W, v, o, stream=None):
    _check(lib().mf_mapped_attn_v(ctypes.byref(desc), ctypes.byref(batch.c), _ptr(row_ptr),
                                  _ptr(col_idx), _ptr(values), _ptr(W), _ptr(v), _ptr(o),
                                  _stream(stream)))


def mfma_probe(out, nblocks: int, iters: int, with_vector: bool, stream=None):
    _check(lib().mf_mfma_probe(_ptr(out), nblocks, iters, int(with_vector), _stream(stream)))


def mapped_split_workspace_size(desc: ReceiverDesc, batch: Batch) -> int:
    return int(lib().mf_mapped_split_workspace_size(ctypes.byref(desc), ctypes.byref(batch.c)))


def mapped_attn_v_split(desc: ReceiverDesc, batch: Batch, row_ptr, col_idx, values, W, v, o, workspace,
                        stream=None):
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mf_mapped_attn_v_split(ctypes.byref(desc), ctypes.byref(batch.c), _ptr(row_ptr),
                                        _ptr(col_idx), _ptr(values), _ptr(W), _ptr(v), _ptr(o),
                                        _ptr(workspace), ws, _stream(stream)))


def mapped_attn_v_multi(descs: Sequence[ReceiverDesc], batch: Batch, row_ptr, col_idx, values,
                        Ws, vs, os_, stream=None):
    """Several receivers of one CSR in one call: descs[k], Ws[k], vs[k], os_[k] as in
    mapped_attn_v."""
    n = len(descs)
    dp = (ctypes.POINTER(ReceiverDesc) * n)(*[ctypes.pointer(d) for d in descs])
    wp = (ctypes.c_void_p * n)(*[_ptr(w) for w in Ws])
    vp_ = (ctypes.c_void_p * n)(*[_ptr(x) for x in vs])
    op = (ctypes.c_void_p * n)(*[_ptr(x) for x in os_])
    _check(lib().mf_mapped_attn_v_multi(dp, n, ctypes.byref(batch.c), _ptr(row_ptr), _ptr(col_idx),
                                        _ptr(values), wp, vp_, op, _stream(stream)))


def headmix_desc(dtype: torch.dtype, B: int, layer_map: Sequence[int], sender_layers: int, H_s: int, H_r: int,
                 sender_capacity: int, receiver_capacity: int) -> HeadmixDesc:
    lm = _as_i32(layer_map)
    desc = HeadmixDesc(dtype_code(dtype), B, lm.shape[0], sender_layers, lm.ctypes.data_as(_i32p), H_s, H_r,
                       sender_capacity, receiver_capacity)
    desc._keep = lm  # the layer map must outlive the descriptor
    return desc


def headmix_workspace_size(desc: HeadmixDesc, batch: Batch) -> int:
    return int(lib().mf_headmix_workspace_size(ctypes.byref(desc), ctypes.byref(batch.c)))


def headmix_gram(desc: HeadmixDesc, batch: Batch, s_row_ptr, s_col_idx, s_values, r_row_ptr, r_col_idx, r_values,
                 gram, cross, workspace, stream=None):
    ws = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().mf_headmix_gram(ctypes.byref(desc), ctypes.byref(batch.c), _ptr(s_row_ptr), _ptr(s_col_idx),
                                 _ptr(s_values), _ptr(r_row_ptr), _ptr(r_col_idx), _ptr(r_values), _ptr(gram),
                                 _ptr(cross), _ptr(workspace), ws, _stream(stream)))


def headmix_solve(desc: HeadmixDesc, gram, cross, lam: float, W, dropped=None, stream=None):
    _check(lib().mf_headmix_solve(ctypes.byref(desc), _ptr(gram), _ptr(cross), float(lam), _ptr(W), _ptr(dropped),
                                  _stream(stream)))


def prefix_block_hashes(tokens, B: int, parent: int = 0) -> np.ndarray:
    """Chained block keys of a token sequence (one per full block of B)."""
    t = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
    out = np.zeros(max(len(t) // B, 1), dtype=np.uint64)
    n = lib().mf_prefix_block_hashes(t.ctypes.data_as(_i32p), len(t), int(B), int(parent),
                                     out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64)))
    if n < 0:
        raise MapflowError(MF_ERR_INVALID, "mf_prefix_block_hashes: bad arguments")
    return out[:n]


class MapCache:
    """Prefix cache of compressed maps in a device pool (a uint8 CUDA tensor the
    object keeps alive)."""

    def __init__(self, dtype: torch.dtype, num_layers: int, H_s: int, B: int, pool_bytes: int,
                 device=None):
        self.pool = torch.empty(pool_bytes, dtype=torch.uint8, device=device or "cuda")
        self.desc = MapCacheDesc(dtype_code(dtype), num_layers, H_s, B)
        h = ctypes.c_void_p()
        _check(lib().mf_map_cache_create(ctypes.byref(self.desc), _ptr(self.pool), pool_bytes, ctypes.byref(h)))
        self.h = h
        self._destroy = lib().mf_map_cache_destroy  # kept for interpreter shutdown

    def close(self):
        if getattr(self, "h", None):
            self._destroy(self.h)
            self.h = None

    __del__ = close

    @staticmethod
    def _u64(keys):
        k = np.ascontiguousarray(np.asarray(keys, dtype=np.uint64))
        return k, k.ctypes.data_as(ctypes.POINTER(ctypes.c_uint64))

    def insert(self, keys, row_ptr_host: np.ndarray, total_rb: int, rb_first: int, col_idx, values, stream=None):
        k, kp = self._u64(keys)
        rp = np.ascontiguousarray(np.asarray(row_ptr_host, dtype=np.int32))
        _check(lib().mf_map_cache_insert(self.h, kp, len(k), rp.ctypes.data_as(_i32p), int(total_rb), int(rb_first),
                                         _ptr(col_idx), _ptr(values), _stream(stream)))

    def lookup(self, keys) -> int:
        k, kp = self._u64(keys)
        return int(lib().mf_map_cache_lookup(self.h, kp, len(k)))

    def release(self, keys, m: int):
        k, kp = self._u64(keys)
        lib().mf_map_cache_release(self.h, kp, int(m))

    def splice(self, keys, m: int, n_blocks: int, suffix_row_ptr_host, suffix_total_rb: int, suffix_rb_first: int,
               suffix_col_idx, suffix_values, row_ptr_out, col_idx_out, values_out, stream=None) -> int:
        k, kp = self._u64(keys if len(keys) else [0])
        rp = np.ascontiguousarray(np.asarray(suffix_row_ptr_host if suffix_row_ptr_host is not None else [0],
                                             dtype=np.int32))
        nnz = ctypes.c_int64(-1)
        cap = col_idx_out.numel() if col_idx_out is not None else 0
        _check(lib().mf_map_cache_splice(self.h, kp, int(m), int(n_blocks), rp.ctypes.data_as(_i32p),
                                         int(suffix_total_rb), int(suffix_rb_first), _ptr(suffix_col_idx),
                                         _ptr(suffix_values), _ptr(row_ptr_out), _ptr(col_idx_out),
                                         _ptr(values_out), cap, ctypes.byref(nnz), _stream(stream)))
        return int(nnz.value)

    def stats(self) -> dict:
        st = MapCacheStats()
        _check(lib().mf_map_cache_get_stats(self.h, ctypes.byref(st)))
        return {f: getattr(st, f) for f, _ in MapCacheStats._fields_}
