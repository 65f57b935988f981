"""Thin ctypes binding over libkvq.so (include/kvq.h).

Argument marshalling only: torch tensors are used for device memory and the
current HIP stream; every step of store / decode runs in the library's HIP
kernels. There is no fallback: if libkvq.so is missing or a call fails, an
exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os
from ctypes import POINTER, byref, c_char_p, c_double, c_float, c_int32, c_int64, c_size_t, c_void_p

import numpy as np
import torch

# KVQ_LIB_PATH names another build of the same library (the host-sanitizer
# build the CPU tests load); by default the in-tree libkvq.so
LIB_PATH = os.environ.get("KVQ_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvq.so")

DTYPES = {"e4m3": 1, "e5m2": 2, "mx16": 3, "nvfp4": 4}
SCALE_MODES = {"tensor": 0, "head": 1, "kivi": 2}
KINDS = {"gqa": 0, "mla": 1}
STATUS = {0: "KVQ_OK", -1: "KVQ_ERR_ARG", -2: "KVQ_ERR_UNSUPPORTED", -3: "KVQ_ERR_SIZE", -4: "KVQ_ERR_HIP",
          -5: "KVQ_ERR_WORKSPACE"}


class KVQError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_lib().kvq_status_string(status).decode()})")


class CacheDesc(ctypes.Structure):
    _fields_ = [("dtype", c_int32), ("kind", c_int32), ("num_kv_heads", c_int32), ("head_dim", c_int32),
                ("v_dim", c_int32), ("page_size", c_int32), ("num_pages", c_int64), ("scale_mode", c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [(n, c_size_t) for n in (
        "k_codes_offset", "k_codes_bytes", "v_codes_offset", "v_codes_bytes",
        "k_scales_offset", "k_scales_bytes", "v_scales_offset", "v_scales_bytes",
        "scratch_offset", "scratch_bytes", "total_bytes")]


_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.kvq_status_string.argtypes = [c_int32]
        L.kvq_status_string.restype = c_char_p
        L.kvq_bytes_per_token.argtypes = [POINTER(CacheDesc), POINTER(c_double)]
        L.kvq_bytes_per_token.restype = c_int32
        L.kvq_alloc_pages.argtypes = [POINTER(CacheDesc), c_void_p, c_size_t, POINTER(c_size_t), POINTER(c_void_p)]
        L.kvq_alloc_pages.restype = c_int32
        L.kvq_cache_layout.argtypes = [c_void_p, POINTER(Layout)]
        L.kvq_cache_layout.restype = c_int32
        L.kvq_free_handle.argtypes = [c_void_p]
        L.kvq_free_handle.restype = None
        L.kvq_compute_scale.argtypes = [c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_void_p]
        L.kvq_compute_scale.restype = c_int32
        L.kvq_store.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p]
        L.kvq_store.restype = c_int32
        L.kvq_decode_workspace_bytes.argtypes = [c_void_p, c_int32, c_int32, c_int32]
        L.kvq_decode_workspace_bytes.restype = c_size_t
        L.kvq_decode.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_int32,
                                 c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.kvq_decode.restype = c_int32
        L.kvq_decode_noalloc.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_int32, c_void_p,
                                         c_int32, c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]
        L.kvq_decode_noalloc.restype = c_int32
        L.kvq_decode_append.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_int32,
                                        c_void_p, c_int32, c_float, c_void_p, c_void_p, c_void_p, c_void_p,
                                        c_void_p, c_size_t, c_void_p]
        L.kvq_decode_append.restype = c_int32
        L.kvq_decode_fp8q.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_int32, c_void_p, c_int32,
                                      c_float, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                      c_void_p]
        L.kvq_decode_fp8q.restype = c_int32
        L.kvq_decode_append_fp8q.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p,
                                             c_int32, c_void_p, c_int32, c_float, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.kvq_decode_append_fp8q.restype = c_int32
        L.kvq_compute_q_scale.argtypes = [c_void_p, c_void_p, c_int64, c_int32, c_void_p, c_void_p]
        L.kvq_compute_q_scale.restype = c_int32
        L.kvq_dequantize_prev_kv.argtypes = [c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p]
        L.kvq_dequantize_prev_kv.restype = c_int32
        L.kvq_extend_attention.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
                                           c_void_p, c_void_p, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                           c_int32, c_int32, c_int32, c_int32, c_float, c_void_p, c_void_p, c_void_p]
        L.kvq_extend_attention.restype = c_int32
        L.kvq_testing_set_split_target.argtypes = [c_void_p, c_int32]
        L.kvq_testing_set_split_target.restype = c_int32
        L.kvq_profile_enable.argtypes = [c_int32]
        L.kvq_profile_enable.restype = c_int32
        L.kvq_profile_read.argtypes = [c_char_p, POINTER(c_double), POINTER(c_int64)]
        L.kvq_profile_read.restype = c_int32
        _LIB = L
    return _LIB


def library():
    """The loaded ctypes library (raises if libkvq.so is not built)."""
    return _lib()


def _check(status: int, what: str):
    if status != 0:
        raise KVQError(status, what)


def _ptr(t):
    return None if t is None else c_void_p(t.data_ptr())


def _stream(device) -> c_void_p:
    return c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _tensor(t, name: str, dtype, dev, shape=None, numel=None, min_numel=None, dim=None):
    """Raise ValueError unless t is a contiguous `dtype` tensor on `dev` with
    the given shape / element count. The C ABI sees raw pointers only, so a
    tensor on the wrong device or too small must be stopped here."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor, got {type(t).__name__}")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if t.device != dev:
        raise ValueError(f"{name}: on {t.device}, the cache is on {dev}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: not contiguous")
    if dim is not None and t.dim() != dim:
        raise ValueError(f"{name}: {t.dim()} dimensions, expected {dim}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name}: {t.numel()} elements, expected {numel}")
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError(f"{name}: {t.numel()} elements, at least {min_numel} needed")
    return t


def _require_gpu(dev):
    """The kernels read device memory only: refuse a cache that is not on a GPU
    (checked after the arguments, so argument errors are reported first)."""
    if dev.type != "cuda":
        raise ValueError(f"the cache memory is on {dev}; the HIP kernels need GPU memory")


def _row_elems(cache: "Cache") -> int:
    """BF16 elements of one token's K (or V) input row: Hkv * D (GQA), D (MLA)."""
    d = cache.desc
    return d.num_kv_heads * d.head_dim if d.kind == KINDS["gqa"] else d.head_dim


def make_desc(dtype: str, kind: str, num_kv_heads: int, head_dim: int, v_dim: int, page_size: int,
              num_pages: int, scale_per_head: bool = False, scale_mode: str | None = None) -> CacheDesc:
    """scale_mode: "tensor", "head" (same as scale_per_head=True) or "kivi"
    (FP8 K scales per channel, V scales per token)."""
    mode = SCALE_MODES[scale_mode] if scale_mode is not None else (1 if scale_per_head else 0)
    return CacheDesc(DTYPES[dtype], KINDS[kind], num_kv_heads, head_dim, v_dim, page_size, num_pages,
                     mode)


def kvq_bytes_per_token(desc: CacheDesc) -> float:
    out = c_double()
    _check(_lib().kvq_bytes_per_token(byref(desc), byref(out)), "kvq_bytes_per_token")
    return out.value


class Cache:
    """One layer's quantized cache bound into a caller-owned uint8 device tensor."""

    def __init__(self, desc: CacheDesc, memory: torch.Tensor):
        self.desc = desc
        self.memory = memory
        h = c_void_p()
        need = c_size_t()
        _check(_lib().kvq_alloc_pages(byref(desc), c_void_p(memory.data_ptr()), memory.numel(), byref(need),
                                      byref(h)), "kvq_alloc_pages")
        self.handle = h
        lay = Layout()
        _check(_lib().kvq_cache_layout(h, byref(lay)), "kvq_cache_layout")
        self.layout = lay

    def view(self, name: str) -> torch.Tensor:
        """uint8 view of one buffer: k_codes, v_codes, k_scales, v_scales."""
        off = getattr(self.layout, name + "_offset")
        n = getattr(self.layout, name + "_bytes")
        return self.memory[off:off + n]

    @property
    def device(self):
        return self.memory.device

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and _LIB is not None:
            _LIB.kvq_free_handle(h)
            self.handle = None


def kvq_alloc_pages(dtype: str, kind: str, num_kv_heads: int, head_dim: int, v_dim: int, page_size: int,
                    num_pages: int, device="cuda", fill: int | None = None, scale_per_head: bool = False,
                    scale_mode: str | None = None) -> Cache:
    desc = make_desc(dtype, kind, num_kv_heads, head_dim, v_dim, page_size, num_pages, scale_per_head, scale_mode)
    need = c_size_t()
    _check(_lib().kvq_alloc_pages(byref(desc), None, 0, byref(need), None), "kvq_alloc_pages(query)")
    mem = torch.empty(need.value, dtype=torch.uint8, device=device)
    if fill is not None:
        mem.fill_(fill)
    return Cache(desc, mem)


def _dev_f32(x, device, n=1):
    """A device fp32 scale array of at least n values (1 per tensor, Hkv per
    head, Hkv * D KIVI channel scales); host values are flattened."""
    if x is None:
        return None
    if not isinstance(x, torch.Tensor):
        x = torch.tensor(np.asarray(x, dtype=np.float32).reshape(-1).tolist(), dtype=torch.float32, device=device)
    return _tensor(x, "scale", torch.float32, device, min_numel=n)


def _n_scales(cache: "Cache", which: str = "k") -> int:
    """Floats of a k_scale / v_scale argument: 1, Hkv (per head), Hkv * D
    (KIVI K channel scales; KIVI V scales live in the cache, none passed)."""
    d = cache.desc
    if d.scale_mode == SCALE_MODES["kivi"]:
        return d.num_kv_heads * d.head_dim if which == "k" else 0
    return d.num_kv_heads if d.scale_mode == SCALE_MODES["head"] else 1


def kvq_compute_scale(cache: Cache, x0: torch.Tensor, x1: torch.Tensor | None = None,
                      out: torch.Tensor | None = None) -> torch.Tensor:
    dev = cache.device
    _tensor(x0, "x0", torch.bfloat16, dev)
    if x1 is not None:
        _tensor(x1, "x1", torch.bfloat16, dev)
    if out is None:
        out = torch.empty(_n_scales(cache), dtype=torch.float32, device=dev)
    _tensor(out, "out", torch.float32, dev, min_numel=_n_scales(cache))
    _require_gpu(dev)
    _check(_lib().kvq_compute_scale(cache.handle, _ptr(x0), x0.numel(), _ptr(x1), 0 if x1 is None else x1.numel(),
                                    _ptr(out), _stream(dev)), "kvq_compute_scale")
    return out


def kvq_store(cache: Cache, k: torch.Tensor, v: torch.Tensor | None, slot_mapping: torch.Tensor,
              k_scale=None, v_scale=None) -> None:
    dev = cache.device
    _tensor(slot_mapping, "slot_mapping", torch.int64, dev, dim=1)
    n = slot_mapping.numel() * _row_elems(cache)
    _tensor(k, "k", torch.bfloat16, dev, numel=n)
    if cache.desc.kind == KINDS["gqa"]:
        _tensor(v, "v", torch.bfloat16, dev, numel=n)
    elif v is not None:
        raise ValueError("v: an MLA cache takes latent rows in k only")
    ks, vs = _dev_f32(k_scale, dev, _n_scales(cache)), _dev_f32(v_scale, dev, _n_scales(cache, "v"))
    _require_gpu(dev)
    _check(_lib().kvq_store(cache.handle, _ptr(k), _ptr(v), _ptr(slot_mapping), slot_mapping.numel(), _ptr(ks),
                            _ptr(vs), _stream(dev)), "kvq_store")


def kvq_decode_workspace_bytes(cache: Cache, batch: int, num_q_heads: int, max_seq_len: int) -> int:
    return int(_lib().kvq_decode_workspace_bytes(cache.handle, batch, num_q_heads, max_seq_len))


def _decode_call(name: str, cache: Cache, k_new, v_new, q, page_table, seq_lens, max_seq_len, sm_scale,
                 q_scale, k_scale, v_scale, out, lse, workspace):
    """Checks every tensor argument of one decode entry point, allocates what
    the caller left out, and calls it. Returns (out, lse)."""
    dev, d = cache.device, cache.desc
    _tensor(q, "q", torch.bfloat16, dev, dim=3)
    B, Hq, Dq = q.shape
    if Dq != d.head_dim:
        raise ValueError(f"q: head dim {Dq}, the cache holds {d.head_dim}")
    if int(max_seq_len) < 0:
        raise ValueError("max_seq_len must be >= 0")
    _tensor(page_table, "page_table", torch.int32, dev, dim=2)
    if page_table.shape[0] < B:
        raise ValueError(f"page_table: {page_table.shape[0]} rows for a batch of {B}")
    _tensor(seq_lens, "seq_lens", torch.int32, dev, numel=B)
    append = name in ("kvq_decode_append", "kvq_decode_append_fp8q")
    if append:
        _tensor(k_new, "k_new", torch.bfloat16, dev, numel=B * _row_elems(cache))
        if d.kind == KINDS["gqa"]:
            _tensor(v_new, "v_new", torch.bfloat16, dev, numel=B * _row_elems(cache))
        elif v_new is not None:
            raise ValueError("v_new: an MLA cache appends latent rows in k_new only")
    if out is None:
        out = torch.empty((B, Hq, d.v_dim), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((B, Hq), dtype=torch.float32, device=dev)
    _tensor(out, "out", torch.float32, dev, shape=(B, Hq, d.v_dim))
    _tensor(lse, "lse", torch.float32, dev, shape=(B, Hq))
    noalloc = name == "kvq_decode_noalloc"
    need = 0 if noalloc else kvq_decode_workspace_bytes(cache, B, Hq, max_seq_len)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    if workspace is not None:
        if noalloc:
            raise ValueError("workspace: kvq_decode_noalloc uses the library's own")
        _tensor(workspace, "workspace", torch.uint8, dev, min_numel=need)
    ks, vs = _dev_f32(k_scale, dev, _n_scales(cache)), _dev_f32(v_scale, dev, _n_scales(cache, "v"))
    fp8q = name.endswith("_fp8q")
    qs = _dev_f32(q_scale, dev, _n_q_scales(cache, Hq)) if fp8q else None
    _require_gpu(dev)
    head = (cache.handle,) + ((_ptr(k_new), _ptr(v_new)) if append else ())
    mid = (_ptr(q), B, Hq, _ptr(page_table), page_table.shape[1], _ptr(seq_lens), int(max_seq_len), float(sm_scale))
    scales = ((_ptr(qs),) if fp8q else ()) + (_ptr(ks), _ptr(vs))
    tail = (_ptr(out), _ptr(lse)) + (() if noalloc else (_ptr(workspace), 0 if workspace is None else
                                                           workspace.numel())) + (_stream(dev),)
    _check(getattr(_lib(), name)(*head, *mid, *scales, *tail), name)
    return out, lse


def kvq_decode(cache: Cache, q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int,
               sm_scale: float, k_scale=None, v_scale=None, out=None, lse=None, workspace=None):
    """Returns (out fp32 [B, Hq, Dv], lse fp32 [B, Hq])."""
    return _decode_call("kvq_decode", cache, None, None, q, page_table, seq_lens, max_seq_len, sm_scale, None,
                        k_scale, v_scale, out, lse, workspace)


def kvq_decode_noalloc(cache: Cache, q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                       max_seq_len: int, sm_scale: float, k_scale=None, v_scale=None, out=None, lse=None):
    """kvq_decode with the split partials in the library's static device
    workspace (no device allocation by the library; pass out and lse to keep
    this binding from allocating them). Calls that overlap on one GPU race.
    Returns (out fp32 [B, Hq, Dv], lse fp32 [B, Hq])."""
    return _decode_call("kvq_decode_noalloc", cache, None, None, q, page_table, seq_lens, max_seq_len, sm_scale,
                        None, k_scale, v_scale, out, lse, None)


def kvq_decode_append(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor | None, q: torch.Tensor,
                      page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float,
                      k_scale=None, v_scale=None, out=None, lse=None, workspace=None):
    """Append the token at position seq_lens[b]-1 of every sequence (k_new, v_new:
    [B, Hkv, D] BF16; MLA: k_new [B, 576], v_new None) and decode, in one
    launch. Returns (out fp32 [B, Hq, Dv], lse fp32 [B, Hq])."""
    return _decode_call("kvq_decode_append", cache, k_new, v_new, q, page_table, seq_lens, max_seq_len, sm_scale,
                        None, k_scale, v_scale, out, lse, workspace)


def _n_q_scales(cache: Cache, num_q_heads: int) -> int:
    """Floats of a q_scale argument: Hq with per-head scales, else 1."""
    return num_q_heads if cache.desc.scale_mode == SCALE_MODES["head"] else 1


def kvq_compute_q_scale(cache: Cache, q: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """E4M3 query scales (amax / 448, per tensor or per query head as the
    cache's scale mode) from a calibration batch q [tokens, Hq, D] BF16."""
    dev = cache.device
    _tensor(q, "q", torch.bfloat16, dev, dim=3)
    if q.shape[2] != cache.desc.head_dim:
        raise ValueError(f"q: head dim {q.shape[2]}, the cache holds {cache.desc.head_dim}")
    if out is None:
        out = torch.empty(_n_q_scales(cache, q.shape[1]), dtype=torch.float32, device=dev)
    _tensor(out, "out", torch.float32, dev, min_numel=_n_q_scales(cache, q.shape[1]))
    _require_gpu(dev)
    _check(_lib().kvq_compute_q_scale(cache.handle, _ptr(q), q.shape[0], q.shape[1], _ptr(out), _stream(dev)),
           "kvq_compute_q_scale")
    return out


def kvq_decode_fp8q(cache: Cache, q: torch.Tensor, page_table: torch.Tensor, seq_lens: torch.Tensor,
                    max_seq_len: int, sm_scale: float, q_scale=None, k_scale=None, v_scale=None, out=None, lse=None,
                    workspace=None):
    """kvq_decode with Q rounded to E4M3 (q / q_scale) and QK^T on FP8 matrix
    cores. Returns (out fp32 [B, Hq, D], lse fp32 [B, Hq])."""
    return _decode_call("kvq_decode_fp8q", cache, None, None, q, page_table, seq_lens, max_seq_len, sm_scale,
                        q_scale, k_scale, v_scale, out, lse, workspace)


def kvq_decode_append_fp8q(cache: Cache, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                           page_table: torch.Tensor, seq_lens: torch.Tensor, max_seq_len: int, sm_scale: float,
                           q_scale=None, k_scale=None, v_scale=None, out=None, lse=None, workspace=None):
    """kvq_decode_append followed by kvq_decode_fp8q, in one launch."""
    return _decode_call("kvq_decode_append_fp8q", cache, k_new, v_new, q, page_table, seq_lens, max_seq_len,
                        sm_scale, q_scale, k_scale, v_scale, out, lse, workspace)


def kvq_dequantize_prev_kv(cache: Cache, pages: torch.Tensor, k_scale_out=None, v_scale_out=None, g=None,
                           dq_k: torch.Tensor | None = None, dq_v: torch.Tensor | None = None):
    """FP4 pages -> E4M3 rows (uint8). Returns (dq_k, dq_v): GQA
    [n, Hkv, P, D] each; MLA (dq_k [n, P, Dk], None)."""
    dev, d = cache.device, cache.desc
    _tensor(pages, "pages", torch.int32, dev, dim=1)
    n = pages.numel()
    shape = (n, d.num_kv_heads, d.page_size, d.head_dim) if d.kind == KINDS["gqa"] else (n, d.page_size, d.head_dim)
    if dq_k is None:
        dq_k = torch.empty(shape, dtype=torch.uint8, device=dev)
    if dq_v is None and d.kind == KINDS["gqa"]:
        dq_v = torch.empty(shape, dtype=torch.uint8, device=dev)
    _tensor(dq_k, "dq_k", torch.uint8, dev, min_numel=math.prod(shape))
    if d.kind == KINDS["gqa"]:
        _tensor(dq_v, "dq_v", torch.uint8, dev, min_numel=math.prod(shape))
    elif dq_v is not None:
        raise ValueError("dq_v: an MLA cache dequantizes its latent rows into dq_k only")
    # the scale tensors stay referenced until the launch: a temporary freed
    # inside the argument list would hand its block to the next one
    gd, ksd, vsd = _dev_f32(g, dev), _dev_f32(k_scale_out, dev), _dev_f32(v_scale_out, dev)
    _require_gpu(dev)
    _check(_lib().kvq_dequantize_prev_kv(cache.handle, _ptr(pages), n, _ptr(gd), _ptr(ksd), _ptr(vsd),
                                         _ptr(dq_k), _ptr(dq_v), _stream(dev)), "kvq_dequantize_prev_kv")
    return dq_k, dq_v


def kvq_extend_attention(q: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, cu_q: torch.Tensor,
                         prefix_len: torch.Tensor, dq_k: torch.Tensor | None, dq_v: torch.Tensor | None,
                         page_off: torch.Tensor, s_k, s_v, max_chunk: int, sm_scale: float, out=None, lse=None):
    """Chunk rows attend to their E4M3 prefix workspace rows and causally to
    the chunk's BF16 K/V. Returns (out fp32 [Nq, Hq, D], lse fp32 [Nq, Hq])."""
    dev = q.device
    _tensor(q, "q", torch.bfloat16, dev, dim=3)
    nq, hq, d = q.shape
    _tensor(k_new, "k_new", torch.bfloat16, dev, dim=3)
    hkv = k_new.shape[1]
    _tensor(k_new, "k_new", torch.bfloat16, dev, shape=(nq, hkv, d))
    _tensor(v_new, "v_new", torch.bfloat16, dev, shape=(nq, hkv, d))
    _tensor(prefix_len, "prefix_len", torch.int32, dev, dim=1)
    batch = prefix_len.numel()
    _tensor(cu_q, "cu_q", torch.int32, dev, numel=batch + 1)
    _tensor(page_off, "page_off", torch.int32, dev, numel=batch)
    n_pages, page_size = (0, 16) if dq_k is None else (dq_k.shape[0], dq_k.shape[2])
    if dq_k is not None:
        _tensor(dq_k, "dq_k", torch.uint8, dev, dim=4)
        _tensor(dq_k, "dq_k", torch.uint8, dev, shape=(n_pages, hkv, page_size, d))
        _tensor(dq_v, "dq_v", torch.uint8, dev, shape=(n_pages, hkv, page_size, d))
    elif dq_v is not None:
        raise ValueError("dq_v given without dq_k")
    if out is None:
        out = torch.empty((nq, hq, d), dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty((nq, hq), dtype=torch.float32, device=dev)
    _tensor(out, "out", torch.float32, dev, shape=(nq, hq, d))
    _tensor(lse, "lse", torch.float32, dev, shape=(nq, hq))
    skd, svd = _dev_f32(s_k, dev), _dev_f32(s_v, dev)
    _require_gpu(dev)
    _check(_lib().kvq_extend_attention(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(cu_q), nq, _ptr(prefix_len),
                                       _ptr(dq_k), _ptr(dq_v), _ptr(page_off), n_pages, _ptr(skd), _ptr(svd),
                                       batch, hq, hkv, d, page_size, int(max_chunk), float(sm_scale),
                                       _ptr(out), _ptr(lse), _stream(dev)), "kvq_extend_attention")
    return out, lse


def set_split_target(cache: Cache, target_wgs: int) -> None:
    """Test and tuning hook (include/kvq_testing.h): aim this cache's decode
    split planner at `target_wgs` workgroups per launch; 0 restores the
    default. The workspace query and every decode call on the cache follow it."""
    _check(_lib().kvq_testing_set_split_target(cache.handle, int(target_wgs)), "kvq_testing_set_split_target")


class split_target:
    """Context manager: set_split_target(cache, target) inside, the default after."""

    def __init__(self, cache: Cache, target_wgs: int):
        self.cache, self.target = cache, int(target_wgs)

    def __enter__(self):
        set_split_target(self.cache, self.target)
        return self.cache

    def __exit__(self, *exc):
        set_split_target(self.cache, 0)
        return False


def kvq_profile_enable(on: bool = True) -> None:
    """Bracket every library kernel launch with HIP events (instrumentation)."""
    _check(_lib().kvq_profile_enable(1 if on else 0), "kvq_profile_enable")


def kvq_profile_read(kernel: str) -> tuple[float, int]:
    """(summed device ms, launches) of one kernel family since the last read:
    "store", "decode", "merge", "amax", "dequant_prev" or "extend"."""
    ms, n = c_double(), c_int64()
    _check(_lib().kvq_profile_read(kernel.encode(), byref(ms), byref(n)), "kvq_profile_read")
    return ms.value, n.value
