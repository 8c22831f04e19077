"""Flexible-mask flash attention (forward and backward) for MI355X (gfx950).

A thin ctypes binding over ``libffa.so`` (C ABI declared in ``include/ffa.h``).
Python marshals arguments only: validation of the slices, planning and every
step of the computation run in the library and its HIP kernels.  PyTorch is used
for device memory and streams.  There is no fallback: if the library is missing
or cannot be loaded, every entry point raises.

API (names follow the pages):
  flex_flash_attn_fwd(q, k, v, q_ranges, k_ranges, attn_type_map, sink=None,
                      softmax_scale=None, softcap=0.0, sink_layout="sh")
      MagiAttention's single-GPU FFA interface on packed THD tensors
      q [Tq,Hq,D], k/v [Tk,Hkv,D] (bf16 or fp16; D 16, 32, 64 or 128) ->
      (out [Tq,Hq,D], lse [Tq,Hq] fp32); mask types 0-3, optional sink
      logits and soft-capping.
  flex_flash_attn_bwd(dout, q, k, v, out, lse, q_ranges, k_ranges, attn_type_map, ...)
      its gradients (dq, dk, dv[, dsink]).
  flex_flash_attn_func(...)  the same forward as a torch.autograd.Function.
  flex_total_attention(q, k, lse, q_ranges, k_ranges, attn_type_map, ...)
      attention probabilities summed over the queries, [Tk, Hq].
  flash_attention(q, k, v, causal=False, sm_scale=None, ...)
      FlagAttention's dense contract on [B,H,M,D] tensors (GQA, bottom-right
      causal), differentiable; returns out, or the 5-tuple (out, lse [B,Hq,M],
      total [B,Hq,N], None, None) when an auxiliary flag is set.
  flash_attention_split_kv(q, k, v, causal=False, sm_scale=None, num_splits=0, ...)
      FlagAttention's forward-only long-KV entry: partial (out, lse) per key
      chunk, merged by a second kernel with a global logsumexp.
  Plan(...)  a reusable host plan (ffa_plan) with its device metadata.

Streams.  A plan may be used on several streams: its metadata is uploaded once
per device and other streams wait for that upload; each (device, stream) pair
gets its own workspace, so calls on different streams never share scratch.
Calls on one stream are ordered by the stream.
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from collections import OrderedDict
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "FFAError",
    "Plan",
    "flex_flash_attn_fwd",
    "flex_flash_attn_bwd",
    "flex_flash_attn_func",
    "flex_total_attention",
    "flash_attention",
    "flash_attention_split_kv",
    "load_library",
    "library_path",
    "FULL",
    "INVCAUSAL",
    "BICAUSAL",
    "CAUSAL",
]

FULL = 0
CAUSAL = 1
INVCAUSAL = 2  # row i of a slice starts at ks + (i - qs): top-left aligned
BICAUSAL = 3   # both bounds move with the row: a band (sliding window)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libffa.so")
_lib = None
_lib_lock = threading.Lock()

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_f32 = ctypes.c_float


class FFAError(RuntimeError):
    def __init__(self, status: int, what: str, detail: str = ""):
        self.status = status
        super().__init__(f"{what}: status {status} ({detail})" if detail else f"{what}: status {status}")


class PlanOpts(ctypes.Structure):
    _fields_ = [("split_tiles", _i32), ("max_splits", _i32), ("num_cus", _i32), ("flags", ctypes.c_uint32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("meta_bytes", _i64),
        ("workspace_bytes", _i64),
        ("visible_pairs", _i64),
        ("computed_pairs", _i64),
        ("num_items", _i32),
        ("num_runs", _i32),
        ("num_combine", _i32),
        ("num_split_items", _i32),
        ("heads_per_item", _i32),
        ("rows_per_item", _i32),
        ("block_n", _i32),
        ("max_item_tiles", _i32),
        ("total_tiles", _i64),
        ("bwd_workspace_bytes", _i64),
        ("dq_tiles", _i64),
        ("kv_tiles", _i64),
        ("num_dq_items", _i32),
        ("num_kv_items", _i32),
    ]


class AttnExtras(ctypes.Structure):
    """ffa_attn_extras: optional sink logits (and their gradient) and softcap."""
    _fields_ = [("sink", _vp), ("dsink", _vp), ("sink_sb", _i64), ("sink_st", _i64), ("sink_ss", _i64),
                ("sink_sh", _i64), ("n_sink", _i32), ("softcap", _f32), ("dtype", _i32), ("flags", _i32)]


# (name, restype, argtypes) of every function in include/ffa.h
_SIGNATURES = [
    ("ffa_abi_version", _i32, []),
    ("ffa_status_string", ctypes.c_char_p, [_i32]),
    ("ffa_last_error", ctypes.c_char_p, []),
    ("ffa_plan", _i32, [_vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(PlanOpts),
                        ctypes.POINTER(_vp)]),
    ("ffa_plan_info_get", _i32, [_vp, ctypes.POINTER(PlanInfo)]),
    ("ffa_plan_sizes", _i32, [_vp, ctypes.POINTER(_sz), ctypes.POINTER(_sz)]),
    ("ffa_plan_upload", _i32, [_vp, _vp, _sz, _vp]),
    ("ffa_plan_export", _i32, [_vp, _vp, _sz]),
    ("ffa_fwd", _i32, [_vp, _vp, _i32,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _f32, ctypes.POINTER(AttnExtras), _vp, _sz, _vp]),
    ("ffa_fwd_noalloc", _i32, [_vp, _vp, _i32,
                               _vp, _i64, _i64, _i64,
                               _vp, _i64, _i64, _i64,
                               _vp, _i64, _i64, _i64,
                               _vp, _i64, _i64, _i64,
                               _vp, _i64, _i64, _i64,
                               _f32, ctypes.POINTER(AttnExtras), _vp]),
    ("ffa_combine", _i32, [_vp, _vp, _i32,
                           _vp, _i64, _i64, _i64,
                           _vp, _i64, _i64, _i64,
                           ctypes.POINTER(AttnExtras), _vp, _sz, _vp]),
    ("ffa_bwd", _i32, [_vp, _vp, _i32,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _vp, _i64, _i64, _i64,
                       _f32, ctypes.POINTER(AttnExtras), _vp, _sz, _vp]),
    ("ffa_total_attention", _i32, [_vp, _vp, _i32,
                                   _vp, _i64, _i64, _i64,
                                   _vp, _i64, _i64, _i64,
                                   _vp, _i64, _i64, _i64,
                                   _vp, _i64, _i64, _i64,
                                   _f32, ctypes.POINTER(AttnExtras), _vp, _sz, _vp]),
    ("ffa_plan_destroy", None, [_vp]),
]

ABI_VERSION = 3
EXTRAS_ROUNDED_NORM = 1
PLAN_NATURAL_ORDER = 1
PLAN_BACKWARD = 2


def library_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libffa.so (built by ``python -m flexible_mask_flash_amd.build``); raise if absent."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise FFAError(-1, "libffa.so is not built",
                           f"expected {_LIB_PATH}; run `python -m flexible_mask_flash_amd.build`")
        lib = ctypes.CDLL(_LIB_PATH)
        for name, res, args in _SIGNATURES:
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        if lib.ffa_abi_version() != ABI_VERSION:
            raise FFAError(-1, "libffa.so ABI mismatch", f"{lib.ffa_abi_version()} != {ABI_VERSION}")
        _lib = lib
        return lib


def _check(status: int, what: str):
    if status != 0:
        lib = load_library()
        detail = lib.ffa_last_error().decode(errors="replace")
        name = lib.ffa_status_string(status).decode(errors="replace")
        raise FFAError(status, what, f"{name}: {detail}")


def _host_i32(x, shape_tail) -> np.ndarray:
    """Ranges / types as a contiguous host int32 array (device tensors are copied: this syncs)."""
    try:
        import torch

        if isinstance(x, torch.Tensor):
            x = x.detach().to("cpu").numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int64))
    a = a.reshape((-1,) + shape_tail) if a.size else np.zeros((0,) + shape_tail, dtype=np.int64)
    if a.size and (a.min() < -(2 ** 31) or a.max() >= 2 ** 31):
        raise ValueError("range values do not fit int32")
    return np.ascontiguousarray(a.astype(np.int32))


class Plan:
    """A validated work plan for one mask and problem shape (ffa_plan)."""

    def __init__(self, q_ranges, k_ranges, mask_types, total_q: int, total_k: int, heads_q: int,
                 heads_kv: int, head_dim: int, split_tiles: int = 0, max_splits: int = 0,
                 num_cus: int = 0, natural_order: bool = False, backward: bool = False):
        lib = load_library()
        qr = _host_i32(q_ranges, (2,))
        kr = _host_i32(k_ranges, (2,))
        ty = _host_i32(mask_types, ())
        if not (qr.shape[0] == kr.shape[0] == ty.shape[0]):
            raise ValueError("q_ranges, k_ranges and mask types must have the same number of slices")
        self.q_ranges, self.k_ranges, self.mask_types = qr, kr, ty
        self.total_q, self.total_k = int(total_q), int(total_k)
        self.heads_q, self.heads_kv, self.head_dim = int(heads_q), int(heads_kv), int(head_dim)
        self.backward = bool(backward)
        flags = (PLAN_NATURAL_ORDER if natural_order else 0) | (PLAN_BACKWARD if backward else 0)
        opts = PlanOpts(int(split_tiles), int(max_splits), int(num_cus), flags)
        h = _vp()
        st = lib.ffa_plan(qr.ctypes.data if qr.size else None, kr.ctypes.data if kr.size else None,
                          ty.ctypes.data if ty.size else None, int(qr.shape[0]), self.total_q, self.total_k,
                          self.heads_q, self.heads_kv, self.head_dim, ctypes.byref(opts), ctypes.byref(h))
        _check(st, "ffa_plan")
        self._h = h
        inf = PlanInfo()
        _check(lib.ffa_plan_info_get(self._h, ctypes.byref(inf)), "ffa_plan_info_get")
        self.info = {name: getattr(inf, name) for name, _ in PlanInfo._fields_}
        # Device state.  The metadata is uploaded once per device; a stream other than
        # the one that uploaded it waits on the upload's event before its first use.
        # Workspaces hold per-call scratch (split partials, backward row terms), so each
        # (device, stream) pair gets its own: calls on different streams never share one.
        self._meta = {}  # device index -> (torch int32 tensor, upload stream, event)
        self._ws = {}    # (device index, stream handle) -> torch uint8 tensor
        self._bws = {}   # (device index, stream handle) -> torch uint8 tensor (backward)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and _lib is not None:
            _lib.ffa_plan_destroy(h)
            self._h = None

    @property
    def handle(self):
        return self._h

    def meta_host(self) -> np.ndarray:
        """The plan metadata as the device sees it (ffa_plan_export)."""
        lib = load_library()
        n = int(self.info["meta_bytes"])
        buf = np.zeros(n // 4, dtype=np.int32)
        _check(lib.ffa_plan_export(self._h, buf.ctypes.data, n), "ffa_plan_export")
        return buf

    def sizes(self):
        """(meta_bytes, workspace_bytes) from ffa_plan_sizes."""
        mb, wb = _sz(), _sz()
        _check(load_library().ffa_plan_sizes(self._h, ctypes.byref(mb), ctypes.byref(wb)), "ffa_plan_sizes")
        return int(mb.value), int(wb.value)

    def device_meta(self, device, stream=None):
        """Device copy of the metadata (ffa_plan_upload), uploaded once per device; a
        later use on another stream is ordered after the upload."""
        import torch

        dev = torch.device(device)
        key = dev.index if dev.index is not None else torch.cuda.current_device()
        s = torch.cuda.current_stream(key) if stream is None else stream
        ent = self._meta.get(key)
        if ent is None:
            n = int(self.info["meta_bytes"])
            t = torch.empty(max(1, n // 4), dtype=torch.int32, device=torch.device("cuda", key))
            _check(load_library().ffa_plan_upload(self._h, t.data_ptr(), n, s.cuda_stream), "ffa_plan_upload")
            ev = torch.cuda.Event()
            ev.record(s)
            ent = (t, s.cuda_stream, ev)
            self._meta[key] = ent
        elif ent[1] != s.cuda_stream:
            s.wait_event(ent[2])
            ent[0].record_stream(s)
        return ent[0]

    def _scratch(self, cache, need: int, device):
        import torch

        if need == 0:
            return None, 0
        dev = torch.device(device)
        idx = dev.index if dev.index is not None else torch.cuda.current_device()
        key = (idx, torch.cuda.current_stream(idx).cuda_stream)
        t = cache.get(key)
        if t is None or t.numel() < need:
            with torch.cuda.device(idx):
                t = torch.empty(need, dtype=torch.uint8, device=torch.device("cuda", idx))
            cache[key] = t
        return t, need

    def workspace(self, device, batch: int = 1):
        """Split-K workspace of this plan for the current stream of `device`."""
        return self._scratch(self._ws, int(self.info["workspace_bytes"]) * int(batch), device)

    def bwd_workspace(self, device, batch: int = 1):
        """Backward workspace of this plan for the current stream of `device`."""
        return self._scratch(self._bws, int(self.info["bwd_workspace_bytes"]) * int(batch), device)


_plan_cache: "OrderedDict[tuple, Plan]" = OrderedDict()
_PLAN_CACHE_MAX = 16


def _cached_plan(qr, kr, ty, tq, tk, hq, hkv, d, split_tiles, backward: bool = False,
                 max_splits: int = 0) -> Plan:
    key = (qr.tobytes(), kr.tobytes(), ty.tobytes(), tq, tk, hq, hkv, d, split_tiles, bool(backward), max_splits)
    p = _plan_cache.get(key)
    if p is None:
        p = Plan(qr, kr, ty, tq, tk, hq, hkv, d, split_tiles=split_tiles, max_splits=max_splits,
                 backward=backward)
        _plan_cache[key] = p
        if len(_plan_cache) > _PLAN_CACHE_MAX:
            _plan_cache.popitem(last=False)
    else:
        _plan_cache.move_to_end(key)
    return p


def _require_bf16_cuda(name, t, ndim, dtype=None):
    """A device tensor of `ndim` dims, bfloat16 or float16 (the same as `dtype` when given)."""
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if t.dtype not in (torch.bfloat16, torch.float16):
        raise TypeError(f"{name} must be bfloat16 or float16, got {t.dtype}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must have the dtype of q ({dtype}), got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have a contiguous head_dim")


def make_extras(sink=None, sink_layout: str = "sh", softcap: float = 0.0, dsink=None, total_q=None, heads_q=None,
                dtype=None, rounded_norm: bool = False):
    """ffa_attn_extras for a sink tensor (fp32 device; layout "sh" [S, Hq] or "ssh" [Tq, S, Hq]),
    a softcap, the element dtype (torch.float16 selects the fp16 kernels) and the forward's
    rounded-weight normalisation (FFA_EXTRAS_ROUNDED_NORM); None for plain bfloat16 attention."""
    import torch

    f16 = dtype == torch.float16
    if sink is None and not softcap and not f16 and not rounded_norm:
        return None
    ex = AttnExtras()
    ex.softcap = float(softcap or 0.0)
    ex.dtype = 1 if f16 else 0
    ex.flags = EXTRAS_ROUNDED_NORM if rounded_norm else 0
    if sink is not None:
        if not isinstance(sink, torch.Tensor) or sink.dtype != torch.float32 or not sink.is_cuda:
            raise TypeError("sink must be a float32 device tensor")
        if sink_layout == "sh":
            if sink.dim() != 2 or (heads_q is not None and sink.shape[1] != heads_q):
                raise ValueError("sink layout 'sh' needs [S_sink, Hq]")
            ex.sink_st, ex.sink_ss, ex.sink_sh = 0, sink.stride(0), sink.stride(1)
            ex.n_sink = sink.shape[0]
        elif sink_layout == "ssh":
            if sink.dim() != 3 or (heads_q is not None and sink.shape[2] != heads_q) or \
                    (total_q is not None and sink.shape[0] != total_q):
                raise ValueError("sink layout 'ssh' needs [Tq, S_sink, Hq]")
            ex.sink_st, ex.sink_ss, ex.sink_sh = sink.stride(0), sink.stride(1), sink.stride(2)
            ex.n_sink = sink.shape[1]
        else:
            raise ValueError(f"unknown sink layout {sink_layout!r}")
        ex.sink = sink.data_ptr()
        if dsink is not None:
            if dsink.shape != sink.shape or dsink.stride() != sink.stride() or dsink.dtype != torch.float32:
                raise ValueError("dsink must match sink in shape, strides and dtype")
            ex.dsink = dsink.data_ptr()
    return ex


def run_fwd(plan: Plan, q, k, v, out, lse, strides, batch: int, softmax_scale: float, extras=None):
    """Call ffa_fwd.  strides: dict of (sb, st, sh) per tensor, in elements."""
    import torch

    dev = q.device
    s = torch.cuda.current_stream(dev)
    meta = plan.device_meta(dev, s)
    ws, ws_bytes = plan.workspace(dev, batch)
    lib = load_library()
    qs, ks, vs, os_, ls = strides["q"], strides["k"], strides["v"], strides["out"], strides["lse"]
    st = lib.ffa_fwd(plan.handle, meta.data_ptr(), int(batch),
                     q.data_ptr(), *qs,
                     k.data_ptr(), *ks,
                     v.data_ptr(), *vs,
                     out.data_ptr(), *os_,
                     lse.data_ptr(), *ls,
                     float(softmax_scale), ctypes.byref(extras) if extras is not None else None,
                     ws.data_ptr() if ws is not None else None, ws_bytes, s.cuda_stream)
    _check(st, "ffa_fwd")


def run_fwd_noalloc(plan: Plan, q, k, v, out, lse, strides, batch: int, softmax_scale: float, extras=None):
    """Call ffa_fwd_noalloc: ffa_fwd without a workspace argument (split partials go to
    the library's own device scratch; nothing is allocated by the call).  Raises
    FFAError (status 7) when the plan's partials exceed that scratch."""
    import torch

    dev = q.device
    s = torch.cuda.current_stream(dev)
    meta = plan.device_meta(dev, s)
    qs, ks, vs, os_, ls = strides["q"], strides["k"], strides["v"], strides["out"], strides["lse"]
    st = load_library().ffa_fwd_noalloc(plan.handle, meta.data_ptr(), int(batch), q.data_ptr(), *qs,
                                        k.data_ptr(), *ks, v.data_ptr(), *vs, out.data_ptr(), *os_,
                                        lse.data_ptr(), *ls, float(softmax_scale),
                                        ctypes.byref(extras) if extras is not None else None, s.cuda_stream)
    _check(st, "ffa_fwd_noalloc")


def run_combine(plan: Plan, out, lse, strides, batch: int, extras=None):
    """Call ffa_combine: merge the split partials the last ffa_fwd with this plan left in
    its workspace (on the current stream).  strides: (sb, st, sh) for "out" and "lse"."""
    import torch

    dev = out.device
    s = torch.cuda.current_stream(dev)
    meta = plan.device_meta(dev, s)
    ws, ws_bytes = plan.workspace(dev, batch)
    st = load_library().ffa_combine(plan.handle, meta.data_ptr(), int(batch), out.data_ptr(), *strides["out"],
                                    lse.data_ptr(), *strides["lse"],
                                    ctypes.byref(extras) if extras is not None else None,
                                    ws.data_ptr() if ws is not None else None, ws_bytes, s.cuda_stream)
    _check(st, "ffa_combine")


def flex_flash_attn_fwd(q, k, v, q_ranges, k_ranges, attn_type_map, sink=None,
                        softmax_scale: Optional[float] = None, softcap: float = 0.0,
                        plan: Optional[Plan] = None, split_tiles: int = 0, sink_layout: str = "sh",
                        rounded_norm: bool = False):
    """Forward of flexible-mask attention on packed THD tensors -> (out, lse).

    q [Tq,Hq,D], k/v [Tk,Hkv,D] bf16 or fp16 device tensors (head_dim contiguous);
    q_ranges / k_ranges int32 [S,2], attn_type_map int32 [S] (0 full, 1 causal,
    2 inverse causal, 3 bi-causal), host or device (device ranges are copied to
    the host, which synchronises).  Optional: sink, fp32 logits [S_sink, Hq]
    ("sh") or [Tq, S_sink, Hq] ("ssh") that join each row's softmax denominator
    without a value; softcap > 0 maps a scaled score s to softcap*tanh(s/softcap).
    Returns out [Tq,Hq,D] bf16 and lse [Tq,Hq] fp32 (natural log, sinks included;
    -inf and a zero output for rows that see no key and no sink).  rounded_norm: divide
    out by the sum of the 16-bit rounded weights its P.V uses (a convex combination of
    value rows; ~6-9% slower), see FFA_EXTRAS_ROUNDED_NORM.
    """
    import torch

    _require_bf16_cuda("q", q, 3)
    _require_bf16_cuda("k", k, 3, q.dtype)
    _require_bf16_cuda("v", v, 3, q.dtype)
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    if v.shape != k.shape or dk != d:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    if plan is None:
        qr = _host_i32(q_ranges, (2,))
        kr = _host_i32(k_ranges, (2,))
        ty = _host_i32(attn_type_map, ())
        plan = _cached_plan(qr, kr, ty, tq, tk, hq, hkv, d, split_tiles)
    elif (plan.total_q, plan.total_k, plan.heads_q, plan.heads_kv, plan.head_dim) != (tq, tk, hq, hkv, d):
        raise ValueError("plan was built for another shape")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    out = torch.empty((tq, hq, d), dtype=q.dtype, device=q.device)
    lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
    strides = {
        "q": (0, q.stride(0), q.stride(1)),
        "k": (0, k.stride(0), k.stride(1)),
        "v": (0, v.stride(0), v.stride(1)),
        "out": (0, out.stride(0), out.stride(1)),
        "lse": (0, lse.stride(0), lse.stride(1)),
    }
    ex = make_extras(sink, sink_layout, softcap, total_q=tq, heads_q=hq, dtype=q.dtype, rounded_norm=rounded_norm)
    run_fwd(plan, q, k, v, out, lse, strides, 1, scale, ex)
    return out, lse


def run_bwd(plan: Plan, t: dict, strides: dict, batch: int, softmax_scale: float, extras=None):
    """Call ffa_bwd.  t: tensors q k v out lse dout dq dk dv; strides: (sb, st, sh) each."""
    import torch

    if not plan.backward:
        raise ValueError("the plan was built without backward=True")
    dev = t["q"].device
    s = torch.cuda.current_stream(dev)
    meta = plan.device_meta(dev, s)
    ws, ws_bytes = plan.bwd_workspace(dev, batch)
    lib = load_library()
    args = []
    for name in ("q", "k", "v", "out", "lse", "dout", "dq", "dk", "dv"):
        args += [t[name].data_ptr(), *strides[name]]
    st = lib.ffa_bwd(plan.handle, meta.data_ptr(), int(batch), *args, float(softmax_scale),
                     ctypes.byref(extras) if extras is not None else None,
                     ws.data_ptr() if ws is not None else None, ws_bytes, s.cuda_stream)
    _check(st, "ffa_bwd")


def _thd_strides(x):
    return (0, x.stride(0), x.stride(1))


def run_total(plan: Plan, q, k, lse, total, strides: dict, batch: int, softmax_scale: float, extras=None):
    """Call ffa_total_attention.  strides: (sb, st, sh) for q, k, lse and total (total: (b, key, head))."""
    import torch

    if not plan.backward:
        raise ValueError("total attention needs a plan built with backward=True (key-major worklist)")
    dev = q.device
    s = torch.cuda.current_stream(dev)
    meta = plan.device_meta(dev, s)
    ws, ws_bytes = plan.bwd_workspace(dev, batch)
    st = load_library().ffa_total_attention(
        plan.handle, meta.data_ptr(), int(batch), q.data_ptr(), *strides["q"], k.data_ptr(), *strides["k"],
        lse.data_ptr(), *strides["lse"], total.data_ptr(), *strides["total"], float(softmax_scale),
        ctypes.byref(extras) if extras is not None else None, ws.data_ptr() if ws is not None else None, ws_bytes,
        s.cuda_stream)
    _check(st, "ffa_total_attention")


def flex_total_attention(q, k, lse, q_ranges, k_ranges, attn_type_map, softmax_scale: Optional[float] = None,
                         sink=None, sink_layout: str = "sh", softcap: float = 0.0):
    """Attention probabilities summed over the query axis, per key and query head -> [Tk, Hq] fp32.

    q [Tq,Hq,D], k [Tk,Hkv,D] bf16 and the forward's lse [Tq,Hq] (with the same
    sink / softcap); FlagAttention's `total` (user guide, "FlashAttention") on
    packed THD tensors.
    """
    import torch

    _require_bf16_cuda("q", q, 3)
    _require_bf16_cuda("k", k, 3, q.dtype)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if lse.dtype != torch.float32 or tuple(lse.shape) != (tq, hq):
        raise ValueError("lse must be float32 [Tq, Hq]")
    plan = _cached_plan(_host_i32(q_ranges, (2,)), _host_i32(k_ranges, (2,)), _host_i32(attn_type_map, ()),
                        tq, tk, hq, hkv, d, 0, backward=True)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    total = torch.empty((tk, hq), dtype=torch.float32, device=q.device)
    strides = {"q": _thd_strides(q), "k": _thd_strides(k), "lse": _thd_strides(lse), "total": _thd_strides(total)}
    run_total(plan, q, k, lse, total, strides, 1, scale, make_extras(sink, sink_layout, softcap, total_q=tq,
                                                                     heads_q=hq, dtype=q.dtype))
    return total


def flex_flash_attn_bwd(dout, q, k, v, out, lse, q_ranges, k_ranges, attn_type_map,
                        softmax_scale: Optional[float] = None, plan: Optional[Plan] = None, sink=None,
                        sink_layout: str = "sh", softcap: float = 0.0):
    """Gradients (dq, dk, dv) of flex_flash_attn_fwd for the upstream gradient dout.

    q [Tq,Hq,D], k/v [Tk,Hkv,D], out/dout [Tq,Hq,D] bf16 and lse [Tq,Hq] fp32
    (the forward's outputs, with the same sink / softcap) on the device; returns
    bf16 tensors shaped like q, k and v, and the fp32 gradient of sink as a
    fourth result when sink is given.  Every step runs in the library's HIP kernels.
    """
    import torch

    for name, x in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _require_bf16_cuda(name, x, 3, q.dtype)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    if v.shape != k.shape or out.shape != q.shape or dout.shape != q.shape or k.shape[2] != d:
        raise ValueError("shape mismatch")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (tq, hq) or lse.device != q.device:
        raise ValueError("lse must be float32 [Tq, Hq] on the device of q")
    if plan is None:
        plan = _cached_plan(_host_i32(q_ranges, (2,)), _host_i32(k_ranges, (2,)), _host_i32(attn_type_map, ()),
                            tq, tk, hq, hkv, d, 0, backward=True)
    elif (plan.total_q, plan.total_k, plan.heads_q, plan.heads_kv, plan.head_dim) != (tq, tk, hq, hkv, d):
        raise ValueError("plan was built for another shape")
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    dq = torch.empty((tq, hq, d), dtype=q.dtype, device=q.device)
    dk = torch.empty((tk, hkv, d), dtype=q.dtype, device=q.device)
    dv = torch.empty((tk, hkv, d), dtype=q.dtype, device=q.device)
    t = {"q": q, "k": k, "v": v, "out": out, "lse": lse, "dout": dout, "dq": dq, "dk": dk, "dv": dv}
    strides = {n: _thd_strides(x) for n, x in t.items()}
    dsink = torch.empty_like(sink) if sink is not None else None
    ex = make_extras(sink, sink_layout, softcap, dsink=dsink, total_q=tq, heads_q=hq, dtype=q.dtype)
    run_bwd(plan, t, strides, 1, scale, ex)
    if sink is not None:
        return dq, dk, dv, dsink
    return dq, dk, dv


def _autograd_function():
    import torch

    class _FlexAttn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, sink, plan, scale, sink_layout, softcap):
            tq, hq, d = q.shape
            out = torch.empty((tq, hq, d), dtype=q.dtype, device=q.device)
            lse = torch.empty((tq, hq), dtype=torch.float32, device=q.device)
            strides = {"q": _thd_strides(q), "k": _thd_strides(k), "v": _thd_strides(v),
                       "out": _thd_strides(out), "lse": _thd_strides(lse)}
            sk = sink.detach() if sink is not None else None
            run_fwd(plan, q, k, v, out, lse, strides, 1, scale, make_extras(sk, sink_layout, softcap,
                                                                           total_q=tq, heads_q=hq, dtype=q.dtype))
            ctx.save_for_backward(q, k, v, out, lse, sk)
            ctx.plan, ctx.scale, ctx.sink_layout, ctx.softcap = plan, scale, sink_layout, softcap
            ctx.mark_non_differentiable(lse)
            return out, lse

        @staticmethod
        def backward(ctx, dout, _dlse):
            q, k, v, out, lse, sink = ctx.saved_tensors
            if dout.stride(-1) != 1 or dout.dtype != q.dtype:
                dout = dout.to(q.dtype).contiguous()
            g = flex_flash_attn_bwd(dout, q, k, v, out, lse, None, None, None, ctx.scale, plan=ctx.plan,
                                    sink=sink, sink_layout=ctx.sink_layout, softcap=ctx.softcap)
            dsink = g[3] if sink is not None else None
            return g[0], g[1], g[2], dsink, None, None, None, None

    return _FlexAttn


_FLEX_FN = None


def flex_flash_attn_func(q, k, v, q_ranges, k_ranges, attn_type_map, sink=None,
                         softmax_scale: Optional[float] = None, softcap: float = 0.0, sink_layout: str = "sh"):
    """Differentiable flexible-mask attention -> (out, lse).

    Same arguments and results as flex_flash_attn_fwd; gradients flow to q, k,
    v and sink through out (lse is returned without a gradient).  The backward
    runs ffa_bwd on a plan built with the backward worklists.
    """
    global _FLEX_FN
    for name, x in (("q", q), ("k", k), ("v", v)):
        _require_bf16_cuda(name, x, 3)
    tq, hq, d = q.shape
    tk, hkv, dk = k.shape
    if v.shape != k.shape or dk != d:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    plan = _cached_plan(_host_i32(q_ranges, (2,)), _host_i32(k_ranges, (2,)), _host_i32(attn_type_map, ()),
                        tq, tk, hq, hkv, d, 0, backward=True)
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if _FLEX_FN is None:
        _FLEX_FN = _autograd_function()
    return _FLEX_FN.apply(q, k, v, sink, plan, scale, sink_layout, float(softcap or 0.0))


def _bhmd_strides(x):
    """(batch, token, head) element strides of a [B, H, T, D] (or [B, H, T]) tensor."""
    return (x.stride(0), x.stride(2), x.stride(1))


_FLASH_FN = None


def _flash_function():
    import torch

    class _FlashAttn(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, plan, scale):
            b, hq, m, d = q.shape
            out = torch.empty((b, hq, m, d), dtype=q.dtype, device=q.device)
            lse = torch.empty((b, hq, m), dtype=torch.float32, device=q.device)
            strides = {n: _bhmd_strides(x) for n, x in (("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse))}
            run_fwd(plan, q, k, v, out, lse, strides, b, scale, make_extras(dtype=q.dtype))
            ctx.save_for_backward(q, k, v, out, lse)
            ctx.plan, ctx.scale = plan, scale
            ctx.mark_non_differentiable(lse)
            return out, lse

        @staticmethod
        def backward(ctx, dout, _dlse):
            q, k, v, out, lse = ctx.saved_tensors
            if dout.stride(-1) != 1 or dout.dtype != q.dtype:
                dout = dout.to(q.dtype).contiguous()
            dq = torch.empty(q.shape, dtype=q.dtype, device=q.device)
            dk = torch.empty(k.shape, dtype=q.dtype, device=q.device)
            dv = torch.empty(v.shape, dtype=q.dtype, device=q.device)
            t = {"q": q, "k": k, "v": v, "out": out, "lse": lse, "dout": dout, "dq": dq, "dk": dk, "dv": dv}
            run_bwd(ctx.plan, t, {n: _bhmd_strides(x) for n, x in t.items()}, q.shape[0], ctx.scale,
                    make_extras(dtype=q.dtype))
            return dq, dk, dv, None, None

    return _FlashAttn


def flash_attention(q, k, v, causal: bool = False, sm_scale: Optional[float] = None, dropout_p: float = 0.0,
                    return_log_normalizer: bool = False, return_total_attention: bool = False,
                    return_seed_offset: bool = False, split_tiles: int = 0):
    """FlagAttention-style dense attention on [B, H, M, D] tensors, differentiable.

    q [B,Hq,M,D], k/v [B,Hkv,N,D] bf16; Hq % Hkv == 0; causal is bottom-right
    aligned.  Every batch element is one slice of a shared plan; the kernels
    read the [B,H,M,D] layout through strides (no copies).  Gradients flow to
    q, k and v through out (ffa_bwd).  With an auxiliary flag set it returns
    (out, lse [B,Hq,M] or None, total [B,Hq,N] or None, None, None); total is
    the attention probabilities summed over the query axis.
    """
    import torch

    global _FLASH_FN
    if dropout_p:
        raise NotImplementedError("dropout is not supported")
    if return_seed_offset:
        raise NotImplementedError("return_seed_offset needs dropout, which is not supported")
    _require_bf16_cuda("q", q, 4)
    _require_bf16_cuda("k", k, 4, q.dtype)
    _require_bf16_cuda("v", v, 4, q.dtype)
    b, hq, m, d = q.shape
    bk, hkv, n, dk = k.shape
    if v.shape != k.shape or bk != b or dk != d:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    ty = CAUSAL if causal else FULL
    need_bwd = return_total_attention or (torch.is_grad_enabled() and
                                          any(x.requires_grad for x in (q, k, v)))
    plan = _cached_plan(np.array([[0, m]], np.int32), np.array([[0, n]], np.int32), np.array([ty], np.int32),
                        m, n, hq, hkv, d, split_tiles, backward=need_bwd)
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    if _FLASH_FN is None:
        _FLASH_FN = _flash_function()
    out, lse = _FLASH_FN.apply(q, k, v, plan, scale)
    if not (return_log_normalizer or return_total_attention):
        return out
    total = None
    if return_total_attention:
        total = torch.empty((b, hq, n), dtype=torch.float32, device=q.device)
        strides = {"q": _bhmd_strides(q), "k": _bhmd_strides(k), "lse": _bhmd_strides(lse),
                   "total": _bhmd_strides(total)}
        run_total(plan, q.detach(), k.detach(), lse, total, strides, b, scale, make_extras(dtype=q.dtype))
    return out, (lse if return_log_normalizer else None), total, None, None


KEY_TILE = 64  # keys per key tile of the forward kernel (the unit of split_tiles)


def flash_attention_split_kv(q, k, v, causal: bool = False, sm_scale: Optional[float] = None,
                             num_splits: int = 0, return_log_normalizer: bool = False):
    """Forward-only attention over a long key axis, on [B, H, M, D] tensors.

    q [B,Hq,M,D], k/v [B,Hkv,N,D] bf16 or fp16; Hq % Hkv == 0; D in {16, 32, 64,
    128}; causal is bottom-right aligned.  The key axis of each query tile is cut
    into chunks; every chunk writes a float32 partial output and log-normalizer,
    and a second kernel (ffa_combine) merges them with a global logsumexp
    (FlagAttention user guide, "Split-KV and paged attention").  num_splits: 0
    lets the planner choose (it splits only when the work cannot fill the
    device), 1 never splits, n > 1 cuts the longest key range into n chunks of
    ceil(N / 64 / n) key tiles of 64 keys (shorter causal ranges into fewer).
    Returns out [B,Hq,M,D], or (out, lse [B,Hq,M]) with return_log_normalizer.
    Nothing here is differentiable.
    """
    import torch

    _require_bf16_cuda("q", q, 4)
    _require_bf16_cuda("k", k, 4, q.dtype)
    _require_bf16_cuda("v", v, 4, q.dtype)
    b, hq, m, d = q.shape
    bk, hkv, n, dk = k.shape
    if v.shape != k.shape or bk != b or dk != d:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} k {tuple(k.shape)} v {tuple(v.shape)}")
    num_splits = int(num_splits)
    if num_splits < 0:
        raise ValueError("num_splits must be >= 0")
    if num_splits == 0:
        split_tiles, max_splits = 0, 0
    elif num_splits == 1:
        split_tiles, max_splits = -1, 0
    else:
        n_tiles = max(1, -(-n // KEY_TILE))
        split_tiles, max_splits = max(1, -(-n_tiles // num_splits)), num_splits
    ty = CAUSAL if causal else FULL
    plan = _cached_plan(np.array([[0, m]], np.int32), np.array([[0, n]], np.int32), np.array([ty], np.int32),
                        m, n, hq, hkv, d, split_tiles, max_splits=max_splits)
    scale = 1.0 / math.sqrt(d) if sm_scale is None else float(sm_scale)
    with torch.no_grad():
        out = torch.empty((b, hq, m, d), dtype=q.dtype, device=q.device)
        lse = torch.empty((b, hq, m), dtype=torch.float32, device=q.device)
        strides = {nm: _bhmd_strides(x) for nm, x in (("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse))}
        run_fwd(plan, q.detach(), k.detach(), v.detach(), out, lse, strides, b, scale, make_extras(dtype=q.dtype))
    return (out, lse) if return_log_normalizer else out
