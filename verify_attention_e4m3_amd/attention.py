"""Thin Python binding over libattn.so (C ABI in include/attn.h).

Argument marshalling only: every step of the attention runs in the HIP kernels of the
library. torch supplies device memory and streams. The library is loaded on first use from
this package directory; if it is missing the call raises - there is no other code path.

Names follow the C ABI: ``Plan`` wraps ``attn_plan``; ``Plan.run`` calls ``attn_run`` then
``attn_combine`` on the current torch stream; ``WorkspaceBank`` keeps the per-stream FP32
split workspaces (grow-only, older buffers stay alive for graphs that captured them), as the
DFlash2 long-batch design note describes for its workspace bank ("Why the single-request
optimization was missing from concurrent decode").
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libattn.so")

ATTN_ABI_VERSION = 1
ATTN_OK, ATTN_E_INVALID, ATTN_E_UNSUPPORTED, ATTN_E_HIP, ATTN_E_WORKSPACE, ATTN_E_STATIC_WORKSPACE = range(6)
ATTN_STATIC_WORKSPACE_BYTES = 64 << 20
ATTN_KV_E4M3, ATTN_KV_FP16, ATTN_KV_E5M2 = 1, 2, 3
ATTN_DEVICE_HOST_ONLY = -1
ATTN_MAX_GEOMETRIES = 8

KV_DTYPES = {"e4m3": ATTN_KV_E4M3, "fp16": ATTN_KV_FP16, "e5m2": ATTN_KV_E5M2}
ELEM_BYTES = {"e4m3": 1, "fp16": 2, "e5m2": 1}


class attn_geometry(ctypes.Structure):
    _fields_ = [("kv_dtype", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("max_q_len", ctypes.c_int32),
                ("max_rows", ctypes.c_int32)]


class attn_caps(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("max_batch", ctypes.c_int32),
                ("accumulation_bits", ctypes.c_int32), ("page_alignment", ctypes.c_int32),
                ("stride_alignment", ctypes.c_int32), ("max_seq_len", ctypes.c_int32),
                ("num_geometries", ctypes.c_int32), ("geometries", attn_geometry * ATTN_MAX_GEOMETRIES)]


class attn_desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("kv_dtype", ctypes.c_int32), ("q_len", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("max_seq_len", ctypes.c_int32), ("batch_capacity", ctypes.c_int32),
                ("k_page_stride", ctypes.c_int64), ("k_token_stride", ctypes.c_int64),
                ("k_head_stride", ctypes.c_int64), ("v_page_stride", ctypes.c_int64),
                ("v_token_stride", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
                ("sm_scale", ctypes.c_float), ("causal", ctypes.c_int32)]


class attn_plan_info(ctypes.Structure):
    _fields_ = [("num_cus", ctypes.c_int32), ("split_cap", ctypes.c_int32), ("partition_max", ctypes.c_int32),
                ("partition_min", ctypes.c_int32),
                ("partition_align", ctypes.c_int32), ("grid_splits", ctypes.c_int32), ("rows", ctypes.c_int32),
                ("split_bytes", ctypes.c_size_t), ("workspace_bytes", ctypes.c_size_t)]


class attn_args(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p),
                ("num_pages", ctypes.c_int64), ("block_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("k_scale", ctypes.c_void_p), ("v_scale", ctypes.c_void_p), ("workspace", ctypes.c_void_p),
                ("workspace_bytes", ctypes.c_size_t), ("out", ctypes.c_void_p), ("batch", ctypes.c_int32)]


class attn_prefill_desc(ctypes.Structure):
    _fields_ = [("abi_version", ctypes.c_uint32), ("q_len", ctypes.c_int32), ("kv_len", ctypes.c_int32),
                ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("q_token_stride", ctypes.c_int64), ("q_head_stride", ctypes.c_int64),
                ("k_token_stride", ctypes.c_int64), ("k_head_stride", ctypes.c_int64),
                ("v_token_stride", ctypes.c_int64), ("v_head_stride", ctypes.c_int64),
                ("o_token_stride", ctypes.c_int64), ("o_head_stride", ctypes.c_int64),
                ("sm_scale", ctypes.c_float), ("causal", ctypes.c_int32)]


EXPORTS = {
    "attn_get_capabilities": (ctypes.c_int, [ctypes.POINTER(attn_caps)]),
    "attn_plan": (ctypes.c_int, [ctypes.POINTER(attn_desc), ctypes.c_int, ctypes.POINTER(ctypes.c_void_p),
                                 ctypes.POINTER(ctypes.c_size_t)]),
    "attn_plan_destroy": (None, [ctypes.c_void_p]),
    "attn_plan_get_info": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(attn_plan_info)]),
    "attn_plan_workspace_bytes": (ctypes.c_size_t, [ctypes.c_void_p, ctypes.c_int32]),
    "attn_plan_splits": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                        ctypes.POINTER(ctypes.c_int32)]),
    "attn_run": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(attn_args), ctypes.c_void_p]),
    "attn_combine": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(attn_args), ctypes.c_void_p]),
    "attn_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "attn_prefill": (ctypes.c_int, [ctypes.POINTER(attn_prefill_desc), ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "attn_run_static": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(attn_args), ctypes.c_void_p]),
}

_lib = None
_lib_lock = threading.Lock()


class AttnError(RuntimeError):
    def __init__(self, call: str, status: int):
        self.status = status
        super().__init__(f"{call} failed: {status_string(status)} (status {status})")


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    with _lib_lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                                   "`python -m verify_attention_e4m3_amd.build`")
            handle = ctypes.CDLL(LIB_PATH)
            for name, (res, args) in EXPORTS.items():
                fn = getattr(handle, name)
                fn.restype = res
                fn.argtypes = args
            _lib = handle
        return _lib


def status_string(status: int) -> str:
    return lib().attn_status_string(status).decode()


def _check(call: str, status: int):
    if status != ATTN_OK:
        raise AttnError(call, status)


def capabilities() -> dict:
    caps = attn_caps()
    _check("attn_get_capabilities", lib().attn_get_capabilities(ctypes.byref(caps)))
    return dict(abi_version=caps.abi_version, max_batch=caps.max_batch,
                accumulation_bits=caps.accumulation_bits, page_alignment=caps.page_alignment,
                stride_alignment=caps.stride_alignment, max_seq_len=caps.max_seq_len,
                geometries=[dict(kv_dtype=g.kv_dtype, head_dim=g.head_dim, max_q_len=g.max_q_len,
                                 max_rows=g.max_rows) for g in caps.geometries[:caps.num_geometries]])


def contiguous_strides(page_size: int, num_kv_heads: int, head_dim: int, kv_dtype: str):
    """Byte strides (page, token, head) of a contiguous [pages][page_size][Hkv][D] cache."""
    e = ELEM_BYTES[kv_dtype]
    return (page_size * num_kv_heads * head_dim * e, num_kv_heads * head_dim * e, head_dim * e)


def _ptr(x) -> int:
    return x if isinstance(x, int) else x.data_ptr()


class Plan:
    """An immutable attention contract (``attn_plan``) for one device."""

    def __init__(self, *, q_len: int, num_q_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                 max_seq_len: int, batch_capacity: int, max_pages_per_seq: Optional[int] = None,
                 kv_dtype: str = "e4m3", k_strides=None, v_strides=None, sm_scale: float = 0.0,
                 causal: bool = True, device=None, abi_version: int = ATTN_ABI_VERSION):
        if max_pages_per_seq is None:
            max_pages_per_seq = -(-max_seq_len // page_size) if page_size > 0 else 1
        default = contiguous_strides(page_size, num_kv_heads, head_dim, kv_dtype) if kv_dtype in ELEM_BYTES \
            else (8, 8, 8)
        ks = tuple(k_strides) if k_strides is not None else default
        vs = tuple(v_strides) if v_strides is not None else default
        d = attn_desc(abi_version, KV_DTYPES.get(kv_dtype, 0), q_len, num_q_heads, num_kv_heads, head_dim,
                      page_size, max_pages_per_seq, max_seq_len, batch_capacity, ks[0], ks[1], ks[2],
                      vs[0], vs[1], vs[2], sm_scale, 1 if causal else 0)
        if device is None or device == ATTN_DEVICE_HOST_ONLY:
            dev_index = ATTN_DEVICE_HOST_ONLY
            self.device = None
        else:
            self.device = torch.device(device)
            dev_index = self.device.index if self.device.index is not None else torch.cuda.current_device()
            self.device = torch.device("cuda", dev_index)
        handle = ctypes.c_void_p()
        ws = ctypes.c_size_t()
        _check("attn_plan", lib().attn_plan(ctypes.byref(d), dev_index, ctypes.byref(handle), ctypes.byref(ws)))
        self._handle = handle
        self.desc = d
        self.kv_dtype = kv_dtype
        self.q_len, self.num_q_heads, self.num_kv_heads, self.head_dim = q_len, num_q_heads, num_kv_heads, head_dim
        self.page_size, self.max_seq_len, self.batch_capacity = page_size, max_seq_len, batch_capacity
        self.max_pages_per_seq = max_pages_per_seq
        self.causal = causal
        self.workspace_bytes_capacity = ws.value
        info = attn_plan_info()
        _check("attn_plan_get_info", lib().attn_plan_get_info(handle, ctypes.byref(info)))
        self.info = {f: getattr(info, f) for f, _ in attn_plan_info._fields_}
        self.contract = (kv_dtype, q_len, num_q_heads, num_kv_heads, head_dim, page_size, max_seq_len,
                         self.info["split_bytes"], self.info["grid_splits"])

    def __del__(self):
        h = getattr(self, "_handle", None)
        if h is not None and h.value and _lib is not None:
            _lib.attn_plan_destroy(h)
            self._handle = None

    @property
    def handle(self):
        return self._handle

    def splits(self, seq_len: int):
        """(num_splits, partition_len) of the plan's split policy for one row length."""
        ns, pl = ctypes.c_int32(), ctypes.c_int32()
        _check("attn_plan_splits", lib().attn_plan_splits(self._handle, seq_len, ctypes.byref(ns), ctypes.byref(pl)))
        return ns.value, pl.value

    def workspace_bytes(self, batch: int) -> int:
        return int(lib().attn_plan_workspace_bytes(self._handle, batch))

    def make_args(self, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, out, workspace,
                  num_pages: Optional[int] = None, batch: Optional[int] = None) -> attn_args:
        """Pack device buffers (torch tensors, or raw device addresses for the caches) into attn_args."""
        if batch is None:
            batch = q.shape[0]
        if num_pages is None:
            num_pages = k_cache.shape[0]
        ws_ptr = 0 if workspace is None else workspace.data_ptr()
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        return attn_args(_ptr(q), _ptr(k_cache), _ptr(v_cache), int(num_pages), _ptr(block_table), _ptr(seq_lens),
                         _ptr(k_scale), _ptr(v_scale), ws_ptr, ws_bytes, _ptr(out), int(batch))

    def cache_extent_bytes(self, num_pages: int, strides) -> int:
        """Bytes from a cache base that the kernels may touch for `num_pages` pages with byte
        strides (page, token, head): the last byte of the last head row of the last page."""
        ps, ts, hs = strides
        return (num_pages - 1) * ps + (self.page_size - 1) * ts + (self.num_kv_heads - 1) * hs + \
            self.head_dim * ELEM_BYTES[self.kv_dtype]

    def _validate_caches(self, k_cache, v_cache, k_scale, v_scale, num_pages):
        strides = {"k_cache": (self.desc.k_page_stride, self.desc.k_token_stride, self.desc.k_head_stride),
                   "v_cache": (self.desc.v_page_stride, self.desc.v_token_stride, self.desc.v_head_stride)}
        for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
            if isinstance(t, int):
                continue                       # a raw device address: the caller vouches for its extent
            if t.device != self.device:
                raise ValueError(f"{name} is on {t.device}, the plan on {self.device}")
            need = self.cache_extent_bytes(num_pages, strides[name])
            have = t.numel() * t.element_size()
            if have < need:
                raise ValueError(f"{name} holds {have} bytes; {num_pages} pages at the plan's strides need {need}")
        for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
            if t.dtype != torch.float32 or t.numel() < 1 or t.device != self.device:
                raise ValueError(f"{name} must be a float32 device tensor on {self.device}")

    def _validate(self, q, block_table, seq_lens, out):
        B = q.shape[0]
        for name, t in (("q", q), ("out", out), ("block_table", block_table), ("seq_lens", seq_lens)):
            if t.device != self.device:
                raise ValueError(f"{name} is on {t.device}, the plan on {self.device}")
        want = (B, self.q_len, self.num_q_heads, self.head_dim)
        if q.dtype != torch.float16 or tuple(q.shape) != want or not q.is_contiguous():
            raise ValueError(f"q must be contiguous float16 {want}")
        if out.dtype != torch.float16 or tuple(out.shape) != want or not out.is_contiguous():
            raise ValueError(f"out must be contiguous float16 {want}")
        if block_table.dtype != torch.int32 or tuple(block_table.shape) != (B, self.max_pages_per_seq) or \
                not block_table.is_contiguous():
            raise ValueError(f"block_table must be contiguous int32 ({B}, {self.max_pages_per_seq})")
        if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,) or not seq_lens.is_contiguous():
            raise ValueError(f"seq_lens must be contiguous int32 ({B},)")

    def split(self, args: attn_args, stream=None):
        """attn_run on `stream` (default: torch's current stream of the plan's device)."""
        _check("attn_run", lib().attn_run(self._handle, ctypes.byref(args), self._stream(stream)))

    def combine(self, args: attn_args, stream=None):
        """attn_combine on `stream` (default: torch's current stream of the plan's device)."""
        _check("attn_combine", lib().attn_combine(self._handle, ctypes.byref(args), self._stream(stream)))

    def run_static(self, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, *, out=None,
                   num_pages: Optional[int] = None, stream=None):
        """attn_run_static: the whole attention with the library's static split workspace (no
        workspace tensor; calls that overlap on one GPU race on that array). Returns ``out``."""
        if self.device is None:
            raise RuntimeError("host-only plan cannot run")
        if out is None:
            out = torch.empty_like(q)
        self._validate(q, block_table, seq_lens, out)
        if num_pages is None and isinstance(k_cache, int):
            raise ValueError("num_pages is required when the caches are raw device addresses")
        self._validate_caches(k_cache, v_cache, k_scale, v_scale, k_cache.shape[0] if num_pages is None else num_pages)
        args = self.make_args(q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, out, None,
                              num_pages=num_pages)
        _check("attn_run_static", lib().attn_run_static(self._handle, ctypes.byref(args), self._stream(stream)))
        return out

    def _stream(self, stream):
        if stream is None:
            stream = torch.cuda.current_stream(self.device)
        return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))

    def run(self, q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, *, out=None, workspace=None,
            num_pages: Optional[int] = None, stream=None, bank: Optional["WorkspaceBank"] = None):
        """Attention for the batch in ``q``: attn_run then attn_combine; returns ``out``."""
        if self.device is None:
            raise RuntimeError("host-only plan cannot run")
        if out is None:
            out = torch.empty_like(q)
        self._validate(q, block_table, seq_lens, out)
        if num_pages is None and isinstance(k_cache, int):
            raise ValueError("num_pages is required when the caches are raw device addresses")
        self._validate_caches(k_cache, v_cache, k_scale, v_scale, k_cache.shape[0] if num_pages is None else num_pages)
        if workspace is None:
            workspace = (bank or default_bank()).get(self, q.shape[0], stream)
        args = self.make_args(q, k_cache, v_cache, block_table, seq_lens, k_scale, v_scale, out, workspace,
                              num_pages=num_pages)
        self.split(args, stream)
        self.combine(args, stream)
        return out


class WorkspaceBank:
    """FP32 split workspaces keyed by (device, stream, plan contract).

    A request-major panel set is sized by ``Plan.workspace_bytes(batch)``. Buffers only grow;
    a replaced buffer is kept alive because a captured graph may still reference it. Streams
    never share a buffer.
    """

    def __init__(self):
        self._bufs = {}
        self._retired = []
        self._lock = threading.Lock()

    def get(self, plan: Plan, batch: int, stream=None) -> torch.Tensor:
        if stream is None:
            stream = torch.cuda.current_stream(plan.device)
        key = (str(plan.device), int(stream.cuda_stream if hasattr(stream, "cuda_stream") else stream), plan.contract)
        need = plan.workspace_bytes(batch)
        with self._lock:
            buf = self._bufs.get(key)
            if buf is None or buf.numel() * 4 < need:
                if buf is not None:
                    self._retired.append(buf)
                # 256-byte aligned: torch's caching allocator hands out 512-byte aligned blocks
                buf = torch.empty((need + 3) // 4, dtype=torch.float32, device=plan.device)
                self._bufs[key] = buf
            return buf

    def buffers(self):
        with self._lock:
            return list(self._bufs.values()) + list(self._retired)


_default_bank = None


def default_bank() -> WorkspaceBank:
    global _default_bank
    if _default_bank is None:
        _default_bank = WorkspaceBank()
    return _default_bank


def prefill_desc(q, k, v, out, *, causal: bool = True, sm_scale: float = 0.0,
                 abi_version: int = ATTN_ABI_VERSION) -> attn_prefill_desc:
    """attn_prefill_desc for [tokens][heads][D] views (element strides taken from the tensors)."""
    return attn_prefill_desc(abi_version, q.shape[0], k.shape[0], q.shape[1], k.shape[1], q.shape[2],
                             q.stride(0), q.stride(1), k.stride(0), k.stride(1), v.stride(0), v.stride(1),
                             out.stride(0), out.stride(1), sm_scale, 1 if causal else 0)


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, out: Optional[torch.Tensor] = None,
            causal: bool = True, sm_scale: float = 0.0, stream=None) -> torch.Tensor:
    """attn_prefill on FP16 q [q_len][Hq][D], k / v [kv_len][Hkv][D] (any element strides with a
    unit dim stride); the queries are the last q_len positions of the kv_len-token sequence."""
    if out is None:
        out = torch.empty_like(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        if t.dtype != torch.float16 or t.dim() != 3 or t.stride(2) != 1:
            raise ValueError(f"{name} must be a float16 [tokens][heads][D] view with unit dim stride")
    if k.shape != v.shape or out.shape != q.shape or q.shape[2] != k.shape[2]:
        raise ValueError("shape mismatch between q, k, v and out")
    d = prefill_desc(q, k, v, out, causal=causal, sm_scale=sm_scale)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    st = ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))
    _check("attn_prefill", lib().attn_prefill(ctypes.byref(d), q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                              out.data_ptr(), st))
    return out
