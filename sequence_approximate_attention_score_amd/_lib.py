"""ctypes binding of ``libapbv.so`` (argument marshalling only).

Every step of the hot path runs in the library's HIP kernels; this module checks that torch
tensors have the dtype, shape and strides the C ABI assumes, converts them into device
pointers, allocates outputs the caller did not provide (torch is the device-memory and
stream plumbing) and raises ``ApbvError`` on a non-zero status.
Importing it fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libapbv.so")

APBV_OK, APBV_EINVAL, APBV_EUNSUPPORTED, APBV_EWORKSPACE, APBV_EHIP = 0, 1, 2, 3, 4
MAX_BLOCKS = 64

EXPORTED = ["apbv_score_select_workspace", "apbv_score_select", "apbv_gather_passing",
            "apbv_approx_attn_prefill", "apbv_query_forward_workspace", "apbv_query_forward",
            "apbv_num_buckets", "apbv_schedule", "apbv_attn_tile_rows", "apbv_status_str",
            "apbv_last_error", "apbv_version", "apbv_prefill_layer", "apbv_prefill_layer_plan",
            "apbv_score_select_noalloc", "apbv_layer_workspace", "apbv_layer_forward"]


class ApbvError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class _Layout(ctypes.Structure):
    _fields_ = [("n_blocks", ctypes.c_int32), ("block_starts", ctypes.POINTER(ctypes.c_int32)),
                ("l_anchor", ctypes.c_int32), ("l_query", ctypes.c_int32), ("l_pass", ctypes.c_int32),
                ("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("scale", ctypes.c_float), ("zigzag", ctypes.c_int32),
                ("q_row_stride", ctypes.c_int64), ("kv_row_stride", ctypes.c_int64)]


_VP, _I32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
_LP = ctypes.POINTER(_Layout)

_IO_FIELDS = ["q_anchor", "k_anchor", "v_anchor", "q_ctx", "k_ctx", "v_ctx", "q_query",
              "k_query", "v_query", "scores", "sel", "k_pre", "v_pre", "anchor_out",
              "anchor_lse", "out", "lse", "query_out", "query_lse", "workspace"]


class _LayerIO(ctypes.Structure):
    _fields_ = [(f, _VP) for f in _IO_FIELDS] + [("workspace_bytes", _SZ)]
_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first "
                               "(python -m sequence_approximate_attention_score_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "apbv_score_select_workspace": (_I32, [_LP, ctypes.POINTER(_SZ)]),
            "apbv_score_select": (_I32, [_LP, _VP, _VP, _VP, _VP, _VP, _SZ, _VP]),
            "apbv_score_select_noalloc": (_I32, [_LP, _VP, _VP, _VP, _VP, _VP]),
            "apbv_gather_passing": (_I32, [_LP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP]),
            "apbv_approx_attn_prefill": (_I32, [_LP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _I32, _I32, _VP]),
            "apbv_query_forward_workspace": (_I32, [_LP, ctypes.POINTER(_SZ)]),
            "apbv_query_forward": (_I32, [_LP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                                          _SZ, _VP]),
            "apbv_prefill_layer": (_I32, [_LP] + [_VP] * 13 + [_SZ] + [_VP] * 4 + [_I32]),
            "apbv_layer_workspace": (_I32, [_LP, ctypes.POINTER(_SZ)]),
            "apbv_layer_forward": (_I32, [_LP, ctypes.POINTER(_LayerIO), _VP]),
            "apbv_prefill_layer_plan": (_I32, [_LP, _I32, ctypes.POINTER(_I32),
                                               ctypes.POINTER(_I32)]),
            "apbv_num_buckets": (_I32, [_LP]),
            "apbv_schedule": (_I32, [_LP, _I32, _I32, _VP, _I32, ctypes.POINTER(_I32)]),
            "apbv_attn_tile_rows": (_I32, [_I32]),
            "apbv_status_str": (ctypes.c_char_p, [_I32]),
            "apbv_last_error": (ctypes.c_char_p, []),
            "apbv_version": (ctypes.c_char_p, []),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int, where: str) -> None:
    if status != APBV_OK:
        L = lib()
        raise ApbvError(status, where, f"{L.apbv_status_str(status).decode()}: "
                                       f"{L.apbv_last_error().decode()}")


class Layout:
    """Host-side layout of one problem (mirrors ``apbv_layout``)."""

    def __init__(self, block_starts, *, l_anchor: int, l_query: int, l_pass: int, hq: int,
                 hkv: int, head_dim: int, scale: float = 0.0, zigzag: bool = True,
                 q_row_stride: int = 0, kv_row_stride: int = 0):
        bs = np.ascontiguousarray(np.asarray(block_starts, dtype=np.int32))
        self._bs = bs
        self.block_starts = bs
        self.n_blocks = int(bs.size - 1)
        self.l_anchor, self.l_query, self.l_pass = int(l_anchor), int(l_query), int(l_pass)
        self.hq, self.hkv, self.head_dim = int(hq), int(hkv), int(head_dim)
        self.n_tokens = int(bs[-1]) if bs.size else 0
        self.pre_rows = self.l_anchor + self.n_blocks * self.l_pass
        self.q_stride = int(q_row_stride) or self.hq * self.head_dim
        self.kv_stride = int(kv_row_stride) or self.hkv * self.head_dim
        self.c = _Layout(self.n_blocks, bs.ctypes.data_as(ctypes.POINTER(ctypes.c_int32)),
                         self.l_anchor, self.l_query, self.l_pass, self.hq, self.hkv,
                         self.head_dim, float(scale), int(bool(zigzag)), int(q_row_stride),
                         int(kv_row_stride))

    def ref(self):
        return ctypes.byref(self.c)


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _arg(t, name: str, dtype, rows: int, row_elems: int, row_stride: int | None = None,
         required: bool = True):
    """Check tensor argument ``name`` against what the C ABI assumes: ``dtype``, ``rows`` rows
    of ``row_elems`` contiguous elements, rows ``row_stride`` elements apart (default: packed).
    Returns (name, tensor or None); ``_pointers`` checks the device and takes the addresses."""
    import torch
    if t is None:
        if required:
            raise ValueError(f"{name} is required for this layout")
        return name, None
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    stride = row_elems if row_stride is None else row_stride
    inner = int(np.prod(t.shape[1:])) if t.dim() > 1 else (1 if t.dim() == 1 else 0)
    if t.dim() < 1 or t.shape[0] != rows or inner != row_elems:
        raise ValueError(f"{name} must hold {rows} rows of {row_elems} elements, got shape "
                         f"{tuple(t.shape)}")
    if rows > 0 and row_elems > 0:
        ok = rows == 1 or t.stride(0) == stride
        step = 1
        for dim in range(t.dim() - 1, 0, -1):       # inner dims packed (size-1 dims: any stride)
            ok = ok and (t.shape[dim] == 1 or t.stride(dim) == step)
            step *= int(t.shape[dim])
        if not ok:
            raise ValueError(f"{name} rows must be contiguous and {stride} elements apart, "
                             f"got strides {tuple(t.stride())}")
    return name, t


def _pointers(*args):
    """Device addresses of checked arguments; all tensors must sit on one CUDA device."""
    dev = None
    for name, t in args:
        if t is None:
            continue
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be a CUDA tensor")
        if dev is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}, other arguments on {dev}")
        dev = t.device
    return tuple(None if t is None else t.data_ptr() for _, t in args)


def _stream(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def num_buckets(layout: Layout) -> int:
    n = lib().apbv_num_buckets(layout.ref())
    if n < 0:
        _check(APBV_EINVAL, "apbv_num_buckets")
    return n


def attn_tile_rows(head_dim: int) -> int:
    return lib().apbv_attn_tile_rows(head_dim)


def schedule(layout: Layout, range_begin: int = 0, range_end: int = 0) -> np.ndarray:
    """Work units of the attention launch as an int32 array [units, 4] (host only)."""
    L = lib()
    cnt = _I32(0)
    _check(L.apbv_schedule(layout.ref(), range_begin, range_end, None, 0, ctypes.byref(cnt)),
           "apbv_schedule")
    out = np.zeros((cnt.value, 4), np.int32)
    _check(L.apbv_schedule(layout.ref(), range_begin, range_end, out.ctypes.data_as(_VP),
                           cnt.value, ctypes.byref(cnt)), "apbv_schedule")
    return out


def score_select_workspace(layout: Layout) -> int:
    n = _SZ(0)
    _check(lib().apbv_score_select_workspace(layout.ref(), ctypes.byref(n)),
           "apbv_score_select_workspace")
    return n.value


def score_select(layout: Layout, q_query, k_ctx, *, scores=None, sel=None, workspace=None,
                 want_scores: bool = True):
    """Step 1 (scores + top-l_p). Returns (scores or None, sel)."""
    import torch
    dev = k_ctx.device
    if want_scores and scores is None:
        scores = torch.empty((layout.hkv, layout.n_tokens), dtype=torch.float32, device=dev)
    if sel is None:
        sel = torch.empty((layout.n_blocks, layout.hkv, layout.l_pass), dtype=torch.int32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(score_select_workspace(layout), 256), dtype=torch.uint8, device=dev)
    L, d = layout, layout.head_dim
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    args = _pointers(
        _arg(q_query, "q_query", bf, L.l_query, L.hq * d, required=L.l_query > 0),
        _arg(k_ctx, "k_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(scores, "scores", f32, L.hkv, L.n_tokens, required=False),
        _arg(sel, "sel", i32, L.n_blocks, L.hkv * L.l_pass),
        _arg(workspace, "workspace", torch.uint8, workspace.numel(), 1))
    _check(lib().apbv_score_select(L.ref(), *args, workspace.numel(), _stream(dev)),
           "apbv_score_select")
    return scores, sel


def score_select_noalloc(layout: Layout, q_query, k_ctx, *, scores=None, sel=None,
                         want_scores: bool = True):
    """Step 1 through the allocation-free entry point (the library's per-device scratch in
    place of a workspace). Returns (scores or None, sel)."""
    import torch
    dev = k_ctx.device
    if want_scores and scores is None:
        scores = torch.empty((layout.hkv, layout.n_tokens), dtype=torch.float32, device=dev)
    if sel is None:
        sel = torch.empty((layout.n_blocks, layout.hkv, layout.l_pass), dtype=torch.int32, device=dev)
    L, d = layout, layout.head_dim
    bf, i32, f32 = torch.bfloat16, torch.int32, torch.float32
    args = _pointers(
        _arg(q_query, "q_query", bf, L.l_query, L.hq * d, required=L.l_query > 0),
        _arg(k_ctx, "k_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(scores, "scores", f32, L.hkv, L.n_tokens, required=False),
        _arg(sel, "sel", i32, L.n_blocks, L.hkv * L.l_pass))
    _check(lib().apbv_score_select_noalloc(L.ref(), *args, _stream(dev)),
           "apbv_score_select_noalloc")
    return scores, sel


def gather_passing(layout: Layout, k_anchor, v_anchor, k_ctx, v_ctx, sel, *, k_pre=None,
                   v_pre=None, sel_errors=None):
    """Step 2 (anchor + passing prefix per KV head). Returns (k_pre, v_pre). ``sel_errors``
    (an int32 tensor of one element, zeroed by the caller) receives the count of ``sel``
    entries outside their own block."""
    import torch
    shape = (layout.hkv, layout.pre_rows, layout.head_dim)
    if k_pre is None:
        k_pre = torch.empty(shape, dtype=torch.bfloat16, device=k_ctx.device)
    if v_pre is None:
        v_pre = torch.empty(shape, dtype=torch.bfloat16, device=k_ctx.device)
    L, d, bf = layout, layout.head_dim, torch.bfloat16
    has_anchor = L.l_anchor > 0
    args = _pointers(
        _arg(k_anchor, "k_anchor", bf, L.l_anchor, L.hkv * d, required=has_anchor),
        _arg(v_anchor, "v_anchor", bf, L.l_anchor, L.hkv * d, required=has_anchor),
        _arg(k_ctx, "k_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(v_ctx, "v_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(sel, "sel", torch.int32, L.n_blocks, L.hkv * L.l_pass),
        _arg(k_pre, "k_pre", bf, L.hkv, L.pre_rows * d),
        _arg(v_pre, "v_pre", bf, L.hkv, L.pre_rows * d),
        _arg(sel_errors, "sel_errors", torch.int32, 1, 1, required=False))
    _check(lib().apbv_gather_passing(L.ref(), *args, _stream(k_ctx.device)),
           "apbv_gather_passing")
    return k_pre, v_pre


def approx_attn_prefill(layout: Layout, q_ctx, k_pre, v_pre, k_ctx, v_ctx, *, out=None, lse=None,
                        want_lse: bool = False, range_begin: int = 0, range_end: int = 0):
    """Step 3 (attention over [anchor | passing | causal local]). Returns (out, lse or None)."""
    import torch
    if out is None:
        out = torch.empty((layout.n_tokens, layout.hq, layout.head_dim), dtype=torch.bfloat16,
                          device=q_ctx.device)
    if want_lse and lse is None:
        lse = torch.empty((layout.hq, layout.n_tokens), dtype=torch.float32, device=q_ctx.device)
    L, d, bf = layout, layout.head_dim, torch.bfloat16
    has_pre = L.pre_rows > 0
    args = _pointers(
        _arg(q_ctx, "q_ctx", bf, L.n_tokens, L.hq * d, L.q_stride),
        _arg(k_pre, "k_pre", bf, L.hkv, L.pre_rows * d, required=has_pre),
        _arg(v_pre, "v_pre", bf, L.hkv, L.pre_rows * d, required=has_pre),
        _arg(k_ctx, "k_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(v_ctx, "v_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(out, "out", bf, L.n_tokens, L.hq * d),
        _arg(lse, "lse", torch.float32, L.hq, L.n_tokens, required=False))
    _check(lib().apbv_approx_attn_prefill(L.ref(), *args, range_begin, range_end,
                                          _stream(q_ctx.device)), "apbv_approx_attn_prefill")
    return out, lse


def query_forward_workspace(layout: Layout) -> int:
    n = _SZ(0)
    _check(lib().apbv_query_forward_workspace(layout.ref(), ctypes.byref(n)),
           "apbv_query_forward_workspace")
    return n.value


def query_forward(layout: Layout, q_query, k_query, v_query, k_anchor, v_anchor, k_ctx, v_ctx, *,
                  out=None, lse=None, want_lse: bool = False, workspace=None):
    """Rows of the query block over [anchor | all context | causal query]. Returns
    (out [l_q, hq, d] bf16, lse [hq, l_q] fp32 or None)."""
    import torch
    dev = k_ctx.device
    if out is None:
        out = torch.empty((layout.l_query, layout.hq, layout.head_dim), dtype=torch.bfloat16,
                          device=dev)
    if want_lse and lse is None:
        lse = torch.empty((layout.hq, layout.l_query), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(query_forward_workspace(layout), 256), dtype=torch.uint8,
                                device=dev)
    L, d, bf = layout, layout.head_dim, torch.bfloat16
    any_q, has_anchor = L.l_query > 0, L.l_anchor > 0
    args = _pointers(
        _arg(q_query, "q_query", bf, L.l_query, L.hq * d, required=any_q),
        _arg(k_query, "k_query", bf, L.l_query, L.hkv * d, required=any_q),
        _arg(v_query, "v_query", bf, L.l_query, L.hkv * d, required=any_q),
        _arg(k_anchor, "k_anchor", bf, L.l_anchor, L.hkv * d, required=has_anchor),
        _arg(v_anchor, "v_anchor", bf, L.l_anchor, L.hkv * d, required=has_anchor),
        _arg(k_ctx, "k_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(v_ctx, "v_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(out, "out", bf, L.l_query, L.hq * d),
        _arg(lse, "lse", torch.float32, L.hq, L.l_query, required=False),
        _arg(workspace, "workspace", torch.uint8, workspace.numel(), 1))
    _check(lib().apbv_query_forward(L.ref(), *args, workspace.numel(), _stream(dev)),
           "apbv_query_forward")
    return out, lse


def prefill_layer_plan(layout: Layout, compute_units: int) -> tuple[int, int]:
    """(late, early) of the two-stream layer: attention of buckets [late, n_buckets) runs
    after the selections of blocks [0, early) only (host only)."""
    late, early = _I32(0), _I32(0)
    _check(lib().apbv_prefill_layer_plan(layout.ref(), compute_units, ctypes.byref(late),
                                         ctypes.byref(early)), "apbv_prefill_layer_plan")
    return late.value, early.value


_layer_events: dict = {}


def _events(dev):
    """Two events of the device for apbv_prefill_layer (created once per device and kept
    alive; layer calls on one device from several threads at once must not share them)."""
    import torch
    key = torch.device(dev).index or 0
    if key not in _layer_events:
        evs = (torch.cuda.Event(), torch.cuda.Event())
        for e in evs:
            e.record(torch.cuda.current_stream(dev))   # creates the underlying event
        _layer_events[key] = evs
    return _layer_events[key]


def prefill_layer(layout: Layout, q_query, q_ctx, k_ctx, v_ctx, k_anchor, v_anchor, *,
                  aux_stream=None, scores=None, sel=None, k_pre=None, v_pre=None, out=None,
                  lse=None, want_scores: bool = False, want_lse: bool = False, workspace=None,
                  compute_units: int = 0):
    """Steps 1-3 of one layer in one call; with ``aux_stream`` (a torch.cuda.Stream of the
    same device) the selection and gather of later blocks overlap attention, split for
    ``compute_units`` CUs (0: the device's). Returns (out, lse or None, sel, scores or None)."""
    import torch
    dev = k_ctx.device
    L, d, bf = layout, layout.head_dim, torch.bfloat16
    if want_scores and scores is None:
        scores = torch.empty((L.hkv, L.n_tokens), dtype=torch.float32, device=dev)
    if sel is None:
        sel = torch.empty((L.n_blocks, L.hkv, L.l_pass), dtype=torch.int32, device=dev)
    shape = (L.hkv, L.pre_rows, d)
    if k_pre is None:
        k_pre = torch.empty(shape, dtype=bf, device=dev)
    if v_pre is None:
        v_pre = torch.empty(shape, dtype=bf, device=dev)
    if out is None:
        out = torch.empty((L.n_tokens, L.hq, d), dtype=bf, device=dev)
    if want_lse and lse is None:
        lse = torch.empty((L.hq, L.n_tokens), dtype=torch.float32, device=dev)
    if workspace is None:
        workspace = torch.empty(max(score_select_workspace(layout), 256), dtype=torch.uint8,
                                device=dev)
    has_anchor, has_pre = L.l_anchor > 0, L.pre_rows > 0
    args = _pointers(
        _arg(q_query, "q_query", bf, L.l_query, L.hq * d, required=L.l_query > 0),
        _arg(q_ctx, "q_ctx", bf, L.n_tokens, L.hq * d, L.q_stride),
        _arg(k_ctx, "k_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(v_ctx, "v_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(k_anchor, "k_anchor", bf, L.l_anchor, L.hkv * d, required=has_anchor),
        _arg(v_anchor, "v_anchor", bf, L.l_anchor, L.hkv * d, required=has_anchor),
        _arg(scores, "scores", torch.float32, L.hkv, L.n_tokens, required=False),
        _arg(sel, "sel", torch.int32, L.n_blocks, L.hkv * L.l_pass),
        _arg(k_pre, "k_pre", bf, L.hkv, L.pre_rows * d, required=has_pre),
        _arg(v_pre, "v_pre", bf, L.hkv, L.pre_rows * d, required=has_pre),
        _arg(out, "out", bf, L.n_tokens, L.hq * d),
        _arg(lse, "lse", torch.float32, L.hq, L.n_tokens, required=False),
        _arg(workspace, "workspace", torch.uint8, workspace.numel(), 1))
    aux = ready = done = None
    if aux_stream is not None:
        if aux_stream.device != dev:
            raise ValueError("aux_stream must be a stream of the tensors' device")
        aux = aux_stream.cuda_stream
        ready, done = (e.cuda_event for e in _events(dev))
    _check(lib().apbv_prefill_layer(L.ref(), *args[:12], args[12], workspace.numel(),
                                    _stream(dev), aux, ready, done, int(compute_units)),
           "apbv_prefill_layer")
    return out, lse, sel, scores


def layer_workspace(layout: Layout) -> int:
    n = _SZ(0)
    _check(lib().apbv_layer_workspace(layout.ref(), ctypes.byref(n)), "apbv_layer_workspace")
    return n.value


def layer_forward(layout: Layout, *, q_anchor, k_anchor, v_anchor, q_ctx, k_ctx, v_ctx,
                  q_query, k_query, v_query, anchor_rows: bool = True, query_rows: bool = True,
                  want_lse: bool = False, want_scores: bool = False, workspace=None):
    """Every row of one layer in one call on the current stream: anchor rows (dense causal
    over the anchor), context rows (score/select, gather, approximate attention) and query
    rows (exact over the whole sequence). Returns a dict with ``anchor_out``, ``out``,
    ``query_out`` (None when skipped), their lse (``anchor_lse``, ``lse``, ``query_lse``;
    None unless ``want_lse``), ``sel``, ``k_pre``, ``v_pre`` and ``scores``."""
    import torch
    dev = k_ctx.device
    L, d, bf, f32 = layout, layout.head_dim, torch.bfloat16, torch.float32
    do_anchor = anchor_rows and L.l_anchor > 0
    do_query = query_rows and L.l_query > 0

    def new(shape, dtype, cond=True):
        return torch.empty(shape, dtype=dtype, device=dev) if cond else None

    r = dict(
        anchor_out=new((L.l_anchor, L.hq, d), bf, do_anchor),
        anchor_lse=new((L.hq, L.l_anchor), f32, do_anchor and want_lse),
        out=new((L.n_tokens, L.hq, d), bf),
        lse=new((L.hq, L.n_tokens), f32, want_lse),
        query_out=new((L.l_query, L.hq, d), bf, do_query),
        query_lse=new((L.hq, L.l_query), f32, do_query and want_lse),
        sel=new((L.n_blocks, L.hkv, L.l_pass), torch.int32),
        k_pre=new((L.hkv, L.pre_rows, d), bf),
        v_pre=new((L.hkv, L.pre_rows, d), bf),
        scores=new((L.hkv, L.n_tokens), f32, want_scores))
    if workspace is None:
        workspace = torch.empty(max(layer_workspace(layout), 256), dtype=torch.uint8,
                                device=dev)
    has_anchor, has_pre = L.l_anchor > 0, L.pre_rows > 0
    checked = [
        _arg(q_anchor, "q_anchor", bf, L.l_anchor, L.hq * d, required=do_anchor),
        _arg(k_anchor, "k_anchor", bf, L.l_anchor, L.hkv * d, required=has_anchor),
        _arg(v_anchor, "v_anchor", bf, L.l_anchor, L.hkv * d, required=has_anchor),
        _arg(q_ctx, "q_ctx", bf, L.n_tokens, L.hq * d, L.q_stride),
        _arg(k_ctx, "k_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(v_ctx, "v_ctx", bf, L.n_tokens, L.hkv * d, L.kv_stride),
        _arg(q_query, "q_query", bf, L.l_query, L.hq * d, required=L.l_query > 0),
        _arg(k_query, "k_query", bf, L.l_query, L.hkv * d, required=do_query),
        _arg(v_query, "v_query", bf, L.l_query, L.hkv * d, required=do_query),
        _arg(r["scores"], "scores", f32, L.hkv, L.n_tokens, required=False),
        _arg(r["sel"], "sel", torch.int32, L.n_blocks, L.hkv * L.l_pass),
        _arg(r["k_pre"], "k_pre", bf, L.hkv, L.pre_rows * d, required=has_pre),
        _arg(r["v_pre"], "v_pre", bf, L.hkv, L.pre_rows * d, required=has_pre),
        _arg(r["anchor_out"], "anchor_out", bf, L.l_anchor, L.hq * d, required=False),
        _arg(r["anchor_lse"], "anchor_lse", f32, L.hq, L.l_anchor, required=False),
        _arg(r["out"], "out", bf, L.n_tokens, L.hq * d),
        _arg(r["lse"], "lse", f32, L.hq, L.n_tokens, required=False),
        _arg(r["query_out"], "query_out", bf, L.l_query, L.hq * d, required=False),
        _arg(r["query_lse"], "query_lse", f32, L.hq, L.l_query, required=False),
        _arg(workspace, "workspace", torch.uint8, workspace.numel(), 1)]
    io = _LayerIO(*_pointers(*checked), workspace.numel())
    _check(lib().apbv_layer_forward(L.ref(), ctypes.byref(io), _stream(dev)),
           "apbv_layer_forward")
    return r


def version() -> str:
    return lib().apbv_version().decode()
