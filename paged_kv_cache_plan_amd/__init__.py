"""Batch attention over a paged KV cache for AMD Instinct MI355X (gfx950).

A thin ctypes binding over ``libpka.so`` (C ABI in ``include/pka.h``).  This
module only marshals arguments: PyTorch provides device memory and the
stream; every step of planning and attention runs in the library.  There is
no fallback: if the library is missing or a tensor is not on a GPU, calls
raise.

    plan = Plan(qo_indptr, kv_indptr, kv_indices, kv_last_page_len,
                num_qo_heads, num_kv_heads, head_dim, page_size, causal=True,
                num_pages=pool.shape[0], device=q.device)
    o, lse = plan.run(q, paged_kv)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpka.so")

PKA_OK = 0
PKA_ERR_INVALID_ARG = 1
PKA_ERR_UNSUPPORTED = 2
PKA_ERR_WORKSPACE = 3
PKA_ERR_HIP = 4

PKA_DISABLE_SPLIT_KV = 0x1
PKA_OUT_FP32 = 0x2
PKA_RAGGED_KV = 0x4
PKA_GRAPH_STABLE = 0x8
PKA_MIXED_BATCH = 0x10
PKA_MIXED_TWO_LAUNCHES = 0x20

PKA_KERNEL_PREFILL = 0
PKA_KERNEL_DECODE = 1
PKA_KERNEL_MIXED = 2

EXPORTED = ["pka_last_error", "pka_plan_workspace_size", "pka_plan_create", "pka_plan_get_info",
            "pka_plan_host_image", "pka_run", "pka_run_ragged", "pka_merge_states",
            "pka_debug_gather", "pka_plan_destroy", "pka_get_batch_indices_positions",
            "pka_append_paged_kv", "pka_run_paged_strided", "pka_merge_states_strided",
            "pka_plan_update", "pka_run_noalloc", "pka_cascade_workspace_size", "pka_cascade_create",
            "pka_cascade_run", "pka_cascade_destroy"]


class PlanInfo(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("num_units", ctypes.c_int32),
                ("num_merge_groups", ctypes.c_int32), ("num_partial_rows", ctypes.c_int32),
                ("block_rows", ctypes.c_int32), ("kv_chunk", ctypes.c_int32),
                ("batch", ctypes.c_int32), ("nnz_pages", ctypes.c_int32),
                ("total_q", ctypes.c_int64), ("total_kv", ctypes.c_int64),
                ("int_ws_bytes", ctypes.c_int64), ("float_ws_bytes", ctypes.c_int64),
                ("num_workers", ctypes.c_int32), ("num_queues", ctypes.c_int32),
                ("prefill_cus", ctypes.c_int32), ("decode_cus", ctypes.c_int32)]

    def as_dict(self):
        return {k: getattr(self, k) for k, _ in self._fields_}


class PkaError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"pka error {code}: {msg}")
        self.code = code


_lib = None


def load_library(path: Optional[str] = None):
    """Load libpka.so and declare its signatures (no GPU needed to load).

    ``path`` (or the PKA_LIBRARY environment variable) selects another build
    of the library, such as the host-only planner library built under the
    host sanitizers; signatures of functions a library lacks are skipped, and
    calling one raises AttributeError."""
    global _lib
    if _lib is not None:
        return _lib
    path = path or os.environ.get("PKA_LIBRARY") or LIB_PATH
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m paged_kv_cache_plan_amd.build`")
    L = ctypes.CDLL(path)
    i32p = ctypes.POINTER(ctypes.c_int32)
    vp, i32, u32, szp = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.POINTER(ctypes.c_size_t)
    i64, f32, sz = ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    c_int = ctypes.c_int
    sigs = {
        "pka_last_error": (ctypes.c_char_p, []),
        "pka_plan_workspace_size": (c_int, [i32p, i32p, i32p, i32, i32, i32, i32, i32, i32, u32, szp, szp]),
        "pka_plan_create": (c_int, [i32p, i32p, i32p, i32p, i32, i32, i32, i32, i32, i32, i32, i32, f32, u32,
                                    vp, sz, vp, sz, vp, ctypes.POINTER(vp)]),
        "pka_plan_get_info": (c_int, [vp, ctypes.POINTER(PlanInfo)]),
        "pka_plan_host_image": (c_int, [i32p, i32p, i32p, i32p, i32, i32, i32, i32, i32, i32, i32, i32, u32, vp,
                                        sz, ctypes.POINTER(PlanInfo)]),
        "pka_run": (c_int, [vp, vp, vp, vp, vp, vp]),
        "pka_run_noalloc": (c_int, [vp, vp, vp, vp, vp, vp]),
        "pka_run_ragged": (c_int, [vp, vp, vp, vp, vp, vp, vp]),
        "pka_merge_states": (c_int, [vp, vp, i64, i32, i32, i32, vp, vp, u32, vp]),
        "pka_debug_gather": (c_int, [vp, vp, vp, vp, vp]),
        "pka_merge_states_strided": (c_int, [vp, vp, i64, i32, i32, i32, i64, i64, i64, i64, vp, vp, u32, vp]),
        "pka_run_paged_strided": (c_int, [vp, vp, vp, vp, i64, i64, i64, vp, vp, vp]),
        "pka_get_batch_indices_positions": (c_int, [vp, vp, i32, i32, vp, vp, vp]),
        "pka_append_paged_kv": (c_int, [vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, vp, vp, i32, vp]),
        "pka_plan_update": (c_int, [vp, i32p, i32p, i32p, i32p, i32, i32, vp]),
        "pka_plan_destroy": (None, [vp]),
        "pka_cascade_workspace_size": (c_int, [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, u32, szp, szp]),
        "pka_cascade_create": (c_int, [i32, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, f32, u32, vp, sz,
                                       vp, sz, vp, ctypes.POINTER(vp)]),
        "pka_cascade_run": (c_int, [vp, vp, vp, vp, vp, vp]),
        "pka_cascade_destroy": (None, [vp]),
    }
    for name, (res, args) in sigs.items():
        try:
            fn = getattr(L, name)
        except AttributeError:
            continue
        fn.restype, fn.argtypes = res, args
    _lib = L
    return L


def _check(code):
    if code != PKA_OK:
        raise PkaError(code, _lib.pka_last_error().decode(errors="replace"))


def _host_i32(x):
    """A contiguous host int32 tensor (kept alive by the caller) and its pointer."""
    import torch
    if x is None:
        return None, None
    t = torch.as_tensor(x)
    if t.device.type != "cpu":
        raise ValueError("plan arrays are host tensors")
    t = t.to(torch.int32).contiguous()
    return t, ctypes.cast(t.data_ptr(), ctypes.POINTER(ctypes.c_int32))


def _dev_ptr(t, name, dtype=None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace_size(qo_indptr, kv_indptr, kv_last_page_len, num_qo_heads, num_kv_heads, head_dim,
                   page_size, causal=True, flags=0):
    L = load_library()
    qo, qo_p = _host_i32(qo_indptr)
    kv, kv_p = _host_i32(kv_indptr)
    last, last_p = _host_i32(kv_last_page_len)
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(L.pka_plan_workspace_size(qo_p, kv_p, last_p, qo.numel() - 1, num_qo_heads, num_kv_heads,
                                     head_dim, page_size, int(bool(causal)), flags,
                                     ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def plan_host_image(qo_indptr, kv_indptr, kv_indices, kv_last_page_len, num_qo_heads, num_kv_heads,
                    head_dim, page_size, causal=True, num_pages=None, flags=0):
    """Run the host planner only; returns (int32 tensor image, PlanInfo dict)."""
    import torch
    L = load_library()
    qo, qo_p = _host_i32(qo_indptr)
    kv, kv_p = _host_i32(kv_indptr)
    idx, idx_p = _host_i32(kv_indices)
    last, last_p = _host_i32(kv_last_page_len)
    B = qo.numel() - 1
    nnz = 0 if idx is None else idx.numel()
    if num_pages is None:
        num_pages = int(idx.max()) + 1 if nnz else 0
    info = PlanInfo()
    _check(L.pka_plan_host_image(qo_p, kv_p, idx_p, last_p, B, nnz, num_pages, num_qo_heads,
                                 num_kv_heads, head_dim, page_size, int(bool(causal)), flags, None, 0,
                                 ctypes.byref(info)))
    img = torch.zeros(info.int_ws_bytes // 4, dtype=torch.int32)
    _check(L.pka_plan_host_image(qo_p, kv_p, idx_p, last_p, B, nnz, num_pages, num_qo_heads,
                                 num_kv_heads, head_dim, page_size, int(bool(causal)), flags,
                                 ctypes.c_void_p(img.data_ptr()), img.numel() * 4, ctypes.byref(info)))
    return img, info.as_dict()


class IoShape:
    """What a plan fixes about the tensors of a run."""

    def __init__(self, total_q, num_qo_heads, num_kv_heads, head_dim, page_size, num_pages, total_kv, out_fp32):
        self.total_q, self.num_qo_heads, self.num_kv_heads = total_q, num_qo_heads, num_kv_heads
        self.head_dim, self.page_size, self.num_pages = head_dim, page_size, num_pages
        self.total_kv, self.out_fp32 = total_kv, out_fp32


def check_io(s, q, o, lse, paged_kv=None, k=None, v=None, k_cache=None, v_cache=None):
    """Check the tensors of a run against the plan before any pointer reaches
    the library (the C ABI sees raw pointers and cannot): a wrong shape or
    dtype would make the kernels read or write out of bounds.  Row counts may
    exceed the plan's (a graph-stable plan runs on buffers sized for its
    largest batch); the rows past the planned ones are not touched.  Raises
    ValueError."""
    import torch
    Hq, Hkv, D = s.num_qo_heads, s.num_kv_heads, s.head_dim

    def rows_ok(t, n, tail, dtype):
        return t.dim() == 1 + len(tail) and t.shape[0] >= n and tuple(t.shape[1:]) == tail and t.dtype == dtype

    if not rows_ok(q, s.total_q, (Hq, D), torch.bfloat16):
        raise ValueError(f"q must be bf16 [>= {s.total_q}, {Hq}, {D}], got {q.dtype} {tuple(q.shape)}")
    want_o = torch.float32 if s.out_fp32 else torch.bfloat16
    if not rows_ok(o, s.total_q, (Hq, D), want_o):
        raise ValueError(f"o must be {want_o} [>= {s.total_q}, {Hq}, {D}] (the plan's output dtype), "
                         f"got {o.dtype} {tuple(o.shape)}")
    if lse is not None and not rows_ok(lse, s.total_q, (Hq,), torch.float32):
        raise ValueError(f"lse must be float32 [>= {s.total_q}, {Hq}], got {lse.dtype} {tuple(lse.shape)}")
    if paged_kv is not None:
        if not rows_ok(paged_kv, s.num_pages, (2, s.page_size, Hkv, D), torch.bfloat16):
            raise ValueError(f"paged_kv must be bf16 [>= {s.num_pages} pages, 2, {s.page_size}, {Hkv}, {D}] "
                             f"(the plan's pool), got {paged_kv.dtype} {tuple(paged_kv.shape)}")
    for name, t in (("k", k), ("v", v)):
        if t is not None and not rows_ok(t, s.total_kv, (Hkv, D), torch.bfloat16):
            raise ValueError(f"{name} must be bf16 [>= {s.total_kv}, {Hkv}, {D}], got {t.dtype} {tuple(t.shape)}")
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        if t is not None and t.shape[0] < s.num_pages:
            raise ValueError(f"{name} holds {t.shape[0]} pages; the plan was made for {s.num_pages}")

class Plan:
    """A planned batch: device workspaces plus the library-owned plan handle.

    Index arrays are host tensors (copied during the call).  The plan uploads
    its work arrays with one asynchronous copy on ``stream`` (default: the
    current stream) and does not synchronise.  ``graph_stable`` plans enqueue
    the same launches for every batch, so a captured run can be replayed
    after ``update``; size their workspaces for the largest batch with
    ``int_ws_bytes`` / ``float_ws_bytes`` (at least what this batch needs is
    allocated).  ``mixed`` plans a batch of prefill and decode requests as
    one launch whose workgroups serve both kinds, one after the other;
    ``mixed_two_launches`` as two concurrent launches over a split of the
    compute units.
    """

    def __init__(self, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, num_qo_heads,
                 num_kv_heads, head_dim, page_size=1, causal=True, sm_scale=None,
                 num_pages=None, ragged=False, disable_split_kv=False, out_fp32=False,
                 device=None, stream=None, graph_stable=False, int_ws_bytes=0, float_ws_bytes=0,
                 mixed=False, mixed_two_launches=False):
        import torch
        L = load_library()
        self._lib = L
        self._handle = ctypes.c_void_p()
        flags = (PKA_RAGGED_KV if ragged else 0) | (PKA_DISABLE_SPLIT_KV if disable_split_kv else 0) \
            | (PKA_OUT_FP32 if out_fp32 else 0) | (PKA_GRAPH_STABLE if graph_stable else 0) \
            | (PKA_MIXED_BATCH if (mixed or mixed_two_launches) else 0) \
            | (PKA_MIXED_TWO_LAUNCHES if mixed_two_launches else 0)
        self.flags = flags
        self.num_qo_heads, self.num_kv_heads, self.head_dim = num_qo_heads, num_kv_heads, head_dim
        self.page_size = page_size
        self.out_fp32 = out_fp32
        self.ragged = ragged
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        if dev.type != "cuda":
            raise ValueError("Plan needs a GPU device")
        qo, qo_p = _host_i32(qo_indptr)
        kv, kv_p = _host_i32(kv_indptr)
        idx, idx_p = (None, None) if ragged else _host_i32(kv_indices)
        last, last_p = (None, None) if ragged else _host_i32(kv_last_page_len)
        B = qo.numel() - 1
        nnz = 0 if idx is None else idx.numel()
        if num_pages is None:
            num_pages = (int(idx.max()) + 1) if nnz else 0
        self.num_pages = 0 if ragged else int(num_pages)
        a, b = ctypes.c_size_t(), ctypes.c_size_t()
        _check(L.pka_plan_workspace_size(qo_p, kv_p, last_p, B, num_qo_heads, num_kv_heads, head_dim,
                                         page_size, int(bool(causal)), flags, ctypes.byref(a),
                                         ctypes.byref(b)))
        ia, fb = max(a.value, int(int_ws_bytes)), max(b.value, int(float_ws_bytes))
        self.int_ws = torch.empty(ia, dtype=torch.uint8, device=dev)
        self.float_ws = torch.empty(fb, dtype=torch.uint8, device=dev)
        self._stream = stream if stream is not None else torch.cuda.current_stream(dev)
        _check(L.pka_plan_create(qo_p, kv_p, idx_p, last_p, B, nnz, num_pages, num_qo_heads,
                                 num_kv_heads, head_dim, page_size, int(bool(causal)),
                                 float(sm_scale) if sm_scale else 0.0, flags,
                                 ctypes.c_void_p(self.int_ws.data_ptr()), ia,
                                 ctypes.c_void_p(self.float_ws.data_ptr()), fb,
                                 _stream_ptr(self._stream), ctypes.byref(self._handle)))
        info = PlanInfo()
        _check(L.pka_plan_get_info(self._handle, ctypes.byref(info)))
        self.info = info.as_dict()
        self.total_q = info.total_q
        self.device = dev

    def update(self, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, stream=None):
        """Plan another batch into this plan's workspaces (pka_plan_update)."""
        qo, qo_p = _host_i32(qo_indptr)
        kv, kv_p = _host_i32(kv_indptr)
        idx, idx_p = (None, None) if self.ragged else _host_i32(kv_indices)
        last, last_p = (None, None) if self.ragged else _host_i32(kv_last_page_len)
        nnz = 0 if idx is None else idx.numel()
        _check(self._lib.pka_plan_update(self._handle, qo_p, kv_p, idx_p, last_p, qo.numel() - 1, nnz,
                                         _stream_ptr(stream if stream is not None else self._stream)))
        info = PlanInfo()
        _check(self._lib.pka_plan_get_info(self._handle, ctypes.byref(info)))
        self.info = info.as_dict()
        self.total_q = info.total_q

    def _outputs(self, q, o, lse):
        import torch
        shape = (self.total_q, self.num_qo_heads, self.head_dim)
        if o is None:
            o = torch.empty(shape, dtype=torch.float32 if self.out_fp32 else torch.bfloat16, device=q.device)
        if lse is None:
            lse = torch.empty(shape[:2], dtype=torch.float32, device=q.device)
        return o, lse

    def _io_shape(self):
        return IoShape(self.total_q, self.num_qo_heads, self.num_kv_heads, self.head_dim, self.page_size,
                       self.num_pages, int(self.info["total_kv"]), self.out_fp32)

    def run(self, q, paged_kv, o=None, lse=None, stream=None):
        """Attention over the paged KV cache; returns (o, lse)."""
        import torch
        if self.ragged:
            raise ValueError("plan was made for ragged K/V: use run_ragged")
        o, lse = self._outputs(q, o, lse)
        check_io(self._io_shape(), q, o, lse, paged_kv=paged_kv)
        _check(self._lib.pka_run(self._handle, _dev_ptr(q, "q", torch.bfloat16),
                                 _dev_ptr(paged_kv, "paged_kv", torch.bfloat16),
                                 _dev_ptr(o, "o"), _dev_ptr(lse, "lse", torch.float32),
                                 _stream_ptr(stream)))
        return o, lse

    def run_noalloc(self, q, paged_kv, o, lse=None, stream=None):
        """pka_run_noalloc: as run, with the split-KV partial states in the
        library's static device scratch; o (and lse) must be given, so that
        the call allocates nothing.  Calls that overlap on one GPU race."""
        import torch
        if self.ragged:
            raise ValueError("plan was made for ragged K/V: use run_ragged")
        if o is None:
            raise ValueError("run_noalloc allocates nothing: pass o (and lse)")
        check_io(self._io_shape(), q, o, lse, paged_kv=paged_kv)
        _check(self._lib.pka_run_noalloc(self._handle, _dev_ptr(q, "q", torch.bfloat16),
                                         _dev_ptr(paged_kv, "paged_kv", torch.bfloat16),
                                         _dev_ptr(o, "o"), _dev_ptr(lse, "lse", torch.float32),
                                         _stream_ptr(stream)))
        return o, lse

    def run_ragged(self, q, k, v, o=None, lse=None, stream=None):
        """Attention over ragged dense K/V; returns (o, lse)."""
        import torch
        if not self.ragged:
            raise ValueError("plan was made for a paged KV cache: use run")
        o, lse = self._outputs(q, o, lse)
        check_io(self._io_shape(), q, o, lse, k=k, v=v)
        _check(self._lib.pka_run_ragged(self._handle, _dev_ptr(q, "q", torch.bfloat16),
                                        _dev_ptr(k, "k", torch.bfloat16), _dev_ptr(v, "v", torch.bfloat16),
                                        _dev_ptr(o, "o"), _dev_ptr(lse, "lse", torch.float32),
                                        _stream_ptr(stream)))
        return o, lse

    def run_strided(self, q, k_cache, v_cache, o=None, lse=None, stream=None):
        """Attention over a paged KV cache held in strided views.

        k_cache and v_cache are bf16 GPU tensors viewed as [num_pages,
        page_size, Hkv, D] with the last dimension contiguous and any other
        strides: for example pool[:, 0] of an NHD pool, an HND pool
        [num_pages, 2, Hkv, ps, D] as pool[:, 0].permute(0, 2, 1, 3), or two
        separate K and V pools.  Returns (o, lse)."""
        import torch
        if self.ragged:
            raise ValueError("plan was made for ragged K/V: use run_ragged")
        for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
            if not t.is_cuda or t.dtype != torch.bfloat16:
                raise ValueError(f"{name} must be a bf16 GPU tensor")
            if t.dim() != 4 or tuple(t.shape[1:]) != (self.page_size, self.num_kv_heads, self.head_dim):
                raise ValueError(f"{name} must be viewed as [num_pages, page_size, Hkv, D]")
            if t.stride(3) != 1:
                raise ValueError(f"{name}: the head_dim axis must be contiguous")
        if k_cache.stride() != v_cache.stride():
            raise ValueError("k_cache and v_cache must have the same strides")
        o, lse = self._outputs(q, o, lse)
        check_io(self._io_shape(), q, o, lse, k_cache=k_cache, v_cache=v_cache)
        ps_, ss, hs = k_cache.stride(0), k_cache.stride(1), k_cache.stride(2)
        _check(self._lib.pka_run_paged_strided(self._handle, _dev_ptr(q, "q", torch.bfloat16),
                                               ctypes.c_void_p(k_cache.data_ptr()),
                                               ctypes.c_void_p(v_cache.data_ptr()), ps_, ss, hs,
                                               _dev_ptr(o, "o"), _dev_ptr(lse, "lse", torch.float32),
                                               _stream_ptr(stream)))
        return o, lse

    def debug_gather(self, paged_kv, stream=None):
        """Dense copies (k, v) of the KV rows the page table selects."""
        import torch
        n = int(self.info["total_kv"])
        k = torch.empty((n, self.num_kv_heads, self.head_dim), dtype=torch.bfloat16, device=paged_kv.device)
        v = torch.empty_like(k)
        _check(self._lib.pka_debug_gather(self._handle, _dev_ptr(paged_kv, "paged_kv", torch.bfloat16),
                                          _dev_ptr(k, "k"), _dev_ptr(v, "v"), _stream_ptr(stream)))
        return k, v

    def close(self):
        if getattr(self, "_handle", None) is not None and self._handle.value:
            import torch
            torch.cuda.synchronize(self.device)
            self._lib.pka_plan_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def merge_states(v, s, out_fp32=True, stream=None):
    """Merge attention states: v fp32 [n, S, H, D], s fp32 [n, S, H] (base 2)."""
    import torch
    L = load_library()
    n, S, H, D = v.shape
    if tuple(s.shape) != (n, S, H):
        raise ValueError("s must be [n, S, H]")
    v_out = torch.empty((n, H, D), dtype=torch.float32 if out_fp32 else torch.bfloat16, device=v.device)
    s_out = torch.empty((n, H), dtype=torch.float32, device=v.device)
    _check(L.pka_merge_states(_dev_ptr(v, "v", torch.float32), _dev_ptr(s, "s", torch.float32), n, S, H, D,
                              _dev_ptr(v_out, "v_out"), _dev_ptr(s_out, "s_out"),
                              PKA_OUT_FP32 if out_fp32 else 0, _stream_ptr(stream)))
    return v_out, s_out


def merge_states_levels(v, s, out_fp32=False, stream=None):
    """Merge states stored level-major: v fp32 [S, n, H, D], s fp32 [S, n, H]
    (each contiguous) -> (v_out [n, H, D], s_out [n, H])."""
    import torch
    L = load_library()
    S, n, H, D = v.shape
    if tuple(s.shape) != (S, n, H) or not v.is_contiguous() or not s.is_contiguous():
        raise ValueError("v must be contiguous [S, n, H, D] and s contiguous [S, n, H]")
    v_out = torch.empty((n, H, D), dtype=torch.float32 if out_fp32 else torch.bfloat16, device=v.device)
    s_out = torch.empty((n, H), dtype=torch.float32, device=v.device)
    _check(L.pka_merge_states_strided(_dev_ptr(v, "v", torch.float32), _dev_ptr(s, "s", torch.float32), n, S, H, D,
                                      H * D, n * H * D, H, n * H, _dev_ptr(v_out, "v_out"),
                                      _dev_ptr(s_out, "s_out"), PKA_OUT_FP32 if out_fp32 else 0,
                                      _stream_ptr(stream)))
    return v_out, s_out


class _LevelArrays:
    pass


def _level_arrays(levels):
    """Host int32 copies of every level's four arrays, kept alive on the
    returned object, with the int32* [num_levels] pointer arrays and the
    per-level batch and nnz_pages counts that pka_cascade_* take."""
    import torch
    n = len(levels)
    r = _LevelArrays()
    names = ("qo_indptr", "kv_indptr", "kv_indices", "kv_last_page_len")
    for k, name in enumerate(names):
        ts, arr = [], (ctypes.POINTER(ctypes.c_int32) * max(n, 1))()
        for i, lev in enumerate(levels):
            if len(lev) != 4:
                raise ValueError("a level is (qo_indptr, kv_indptr, kv_indices, kv_last_page_len)")
            t, ptr = _host_i32(lev[k])
            ts.append(t)
            arr[i] = ptr
        setattr(r, name, ts)
        setattr(r, ("qo", "kvp", "kvi", "last")[k], arr)
    r.batch = (ctypes.c_int32 * max(n, 1))(*[t.numel() - 1 for t in r.qo_indptr])
    r.nnz = (ctypes.c_int32 * max(n, 1))(*[t.numel() for t in r.kv_indices])
    return r


def cascade_workspace_size(levels, num_qo_heads, num_kv_heads, head_dim, page_size, causal=True, out_fp32=False,
                           disable_split_kv=False):
    """(int_ws_bytes, float_ws_bytes) a cascade over ``levels`` needs
    (pka_cascade_workspace_size: host only, no GPU)."""
    L = load_library()
    lv = _level_arrays(levels)
    flags = (PKA_OUT_FP32 if out_fp32 else 0) | (PKA_DISABLE_SPLIT_KV if disable_split_kv else 0)
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    _check(L.pka_cascade_workspace_size(len(levels), lv.qo, lv.kvp, lv.last, lv.batch, num_qo_heads, num_kv_heads,
                                        head_dim, page_size, int(bool(causal)), flags, ctypes.byref(a),
                                        ctypes.byref(b)))
    return a.value, b.value


class Cascade:
    """Multi-level cascade attention over one paged KV pool (pka_cascade_*;
    FlashInfer documentation, "flashinfer.cascade: Cascade Attention" and
    "Multi-level Cascade Inference Data Layout").

    ``levels`` is a list of (qo_indptr, kv_indptr, kv_indices,
    kv_last_page_len) host arrays: level l groups the same total_q query rows
    into contiguous groups (its qo_indptr) that share the keys of its page
    table.  A query attends to the concatenation of its groups' keys, level 0
    first; only the last level is masked (bottom-right causal when
    ``causal``), so each request's last-level keys must include its own query
    tokens.  The library plans every level into its share of the two device
    workspaces allocated here, and a run merges the levels' states.
    """

    def __init__(self, levels, num_qo_heads, num_kv_heads, head_dim, page_size, causal=True, sm_scale=-1.0,
                 num_pages=None, out_fp32=False, disable_split_kv=False, device=None, stream=None):
        import torch
        L = load_library()
        self._lib = L
        self._handle = ctypes.c_void_p()
        n = len(levels)
        if n < 1:
            raise ValueError("at least one level")
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        if dev.type != "cuda":
            raise ValueError("Cascade needs a GPU device")
        lv = _level_arrays(levels)
        if num_pages is None:
            num_pages = max((int(t.max()) + 1 for t in lv.kv_indices if t.numel()), default=0)
        flags = (PKA_OUT_FP32 if out_fp32 else 0) | (PKA_DISABLE_SPLIT_KV if disable_split_kv else 0)
        a, b = ctypes.c_size_t(), ctypes.c_size_t()
        _check(L.pka_cascade_workspace_size(n, lv.qo, lv.kvp, lv.last, lv.batch, num_qo_heads, num_kv_heads, head_dim,
                                            page_size, int(bool(causal)), flags, ctypes.byref(a), ctypes.byref(b)))
        self.int_ws = torch.empty(max(a.value, 256), dtype=torch.uint8, device=dev)
        self.float_ws = torch.empty(max(b.value, 256), dtype=torch.uint8, device=dev)
        self._stream = stream if stream is not None else torch.cuda.current_stream(dev)
        _check(L.pka_cascade_create(n, lv.qo, lv.kvp, lv.kvi, lv.last, lv.batch, lv.nnz, int(num_pages), num_qo_heads,
                                    num_kv_heads, head_dim, page_size, int(bool(causal)),
                                    float(sm_scale) if sm_scale and sm_scale > 0 else 0.0, flags,
                                    ctypes.c_void_p(self.int_ws.data_ptr()), self.int_ws.numel(),
                                    ctypes.c_void_p(self.float_ws.data_ptr()), self.float_ws.numel(),
                                    _stream_ptr(self._stream), ctypes.byref(self._handle)))
        self.total_q = int(lv.qo_indptr[0][-1]) if lv.qo_indptr[0].numel() else 0
        self.num_qo_heads, self.head_dim, self.out_fp32 = num_qo_heads, head_dim, out_fp32
        self.device = dev

    def run(self, q, paged_kv, o=None, lse=None, stream=None):
        """Returns (o, lse) of the cascade."""
        import torch
        shape = (self.total_q, self.num_qo_heads, self.head_dim)
        if o is None:
            o = torch.empty(shape, dtype=torch.float32 if self.out_fp32 else torch.bfloat16, device=q.device)
        if lse is None:
            lse = torch.empty(shape[:2], dtype=torch.float32, device=q.device)
        if tuple(q.shape) != shape or q.dtype != torch.bfloat16:
            raise ValueError(f"q must be bf16 {list(shape)}, got {q.dtype} {tuple(q.shape)}")
        if tuple(o.shape) != shape or o.dtype != (torch.float32 if self.out_fp32 else torch.bfloat16):
            raise ValueError("o does not match the cascade's output shape and dtype")
        if tuple(lse.shape) != shape[:2] or lse.dtype != torch.float32:
            raise ValueError("lse must be float32 [total_q, Hq]")
        _check(self._lib.pka_cascade_run(self._handle, _dev_ptr(q, "q", torch.bfloat16),
                                         _dev_ptr(paged_kv, "paged_kv", torch.bfloat16), _dev_ptr(o, "o"),
                                         _dev_ptr(lse, "lse", torch.float32), _stream_ptr(stream)))
        return o, lse

    def close(self):
        if getattr(self, "_handle", None) is not None and self._handle.value:
            import torch
            torch.cuda.synchronize(self.device)
            self._lib.pka_cascade_destroy(self._handle)
            self._handle = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def get_batch_indices_positions(append_indptr, seq_lens, nnz, stream=None):
    """Request and position of every appended token (device int32 [nnz] each).

    append_indptr int32 [batch+1] and seq_lens int32 [batch] (lengths after
    the append) are GPU tensors; nnz = append_indptr[batch]."""
    import torch
    L = load_library()
    batch = seq_lens.numel()
    if append_indptr.numel() != batch + 1:
        raise ValueError("append_indptr must have batch + 1 entries")
    bi = torch.empty(nnz, dtype=torch.int32, device=seq_lens.device)
    pos = torch.empty(nnz, dtype=torch.int32, device=seq_lens.device)
    _check(L.pka_get_batch_indices_positions(_dev_ptr(append_indptr, "append_indptr", torch.int32),
                                             _dev_ptr(seq_lens, "seq_lens", torch.int32), batch, nnz,
                                             _dev_ptr(bi, "batch_indices"), _dev_ptr(pos, "positions"),
                                             _stream_ptr(stream)))
    return bi, pos


def append_paged_kv(append_k, append_v, batch_indices, positions, paged_kv, kv_indices, kv_indptr,
                    stream=None):
    """Write appended K/V rows (bf16 [nnz, Hkv, D]) into paged_kv
    (bf16 [num_pages, 2, ps, Hkv, D]) in place, through the page table."""
    import torch
    L = load_library()
    nnz, Hkv, D = append_k.shape
    if tuple(append_v.shape) != (nnz, Hkv, D):
        raise ValueError("append_v must match append_k")
    num_pages, two, ps, Hkv2, D2 = paged_kv.shape
    if two != 2 or Hkv2 != Hkv or D2 != D:
        raise ValueError("paged_kv must be [num_pages, 2, page_size, Hkv, D] matching the appended rows")
    if batch_indices.numel() != nnz or positions.numel() != nnz:
        raise ValueError("batch_indices and positions must have nnz entries")
    _check(L.pka_append_paged_kv(_dev_ptr(append_k, "append_k", torch.bfloat16),
                                 _dev_ptr(append_v, "append_v", torch.bfloat16),
                                 _dev_ptr(batch_indices, "batch_indices", torch.int32),
                                 _dev_ptr(positions, "positions", torch.int32), nnz,
                                 _dev_ptr(paged_kv, "paged_kv", torch.bfloat16), num_pages, ps, Hkv, D,
                                 _dev_ptr(kv_indices, "kv_indices", torch.int32),
                                 _dev_ptr(kv_indptr, "kv_indptr", torch.int32), kv_indptr.numel() - 1,
                                 _stream_ptr(stream)))

