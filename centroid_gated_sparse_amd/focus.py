"""Python binding of libfocus.so: the C ABI of include/focus.h, called with
torch tensors.  Argument marshalling only — every step of the path runs in
the library's HIP kernels.  Raises if the library has not been built or a
call returns an error status.

The call names match the C ABI: focus_route, focus_route_project,
focus_bucket, focus_check_buckets, focus_attn_fwd (+ focus_attn_fwd_part), focus_attn_bwd,
focus_sinkhorn, focus_gated_attn_fwd, focus_dense_causal_fwd.  ``focus_forward`` chains
the three calls and allocates outputs and workspaces with torch.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

LIB_PATH = Path(__file__).resolve().parent / "libfocus.so"

FOCUS_F32 = 0
FOCUS_BF16 = 1
PART_PREPARE = 1
PART_GROUP = 2
PART_WINDOW = 4
PART_ALL = 7
CHECK_WORKSPACE_BYTES = 256  # FOCUS_CHECK_WORKSPACE_BYTES

# exported symbols (all declared in include/focus.h)
SYMBOLS = (
    "focus_status_string", "focus_last_error", "focus_abi_version",
    "focus_route", "focus_route_project", "focus_num_subbuckets", "focus_bucket_workspace_bytes",
    "focus_bucket",
    "focus_bucket_noalloc",
    "focus_attn_fwd_workspace_bytes", "focus_attn_workspace_bytes", "focus_check_buckets",
    "focus_attn_fwd", "focus_attn_fwd_part",
    "focus_dense_workspace_bytes", "focus_dense_causal_fwd",
    "focus_attn_bwd_workspace_bytes", "focus_attn_bwd",
    "focus_sinkhorn_workspace_bytes", "focus_sinkhorn", "focus_gated_attn_workspace_bytes",
    "focus_gated_attn_fwd",
)

_lib = None


class FocusError(RuntimeError):
    def __init__(self, call: str, status: int, detail: str):
        super().__init__(f"{call} failed: {status_string(status)} ({detail})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libfocus.so once; raise if it is missing (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m "
                           "centroid_gated_sparse_amd.build` (hipcc, gfx950)")
    L = ctypes.CDLL(str(LIB_PATH))
    P, i32, i64, sz, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                            ctypes.c_size_t, ctypes.c_float)
    L.focus_status_string.argtypes = [ctypes.c_int]
    L.focus_status_string.restype = ctypes.c_char_p
    L.focus_last_error.argtypes = []
    L.focus_last_error.restype = ctypes.c_char_p
    L.focus_abi_version.argtypes = []
    L.focus_abi_version.restype = i32
    L.focus_route.argtypes = [P, P, i32, i64, i32, i32, i32, P, P, P]
    L.focus_route_project.argtypes = [P, ctypes.c_int, i64, i32, P, P, i32, i32, i32, i32,
                                      P, P, P, P]
    L.focus_num_subbuckets.argtypes = [i32, i32]
    L.focus_num_subbuckets.restype = i32
    L.focus_bucket_workspace_bytes.argtypes = [i32, i64, i32, i32]
    L.focus_bucket_workspace_bytes.restype = sz
    L.focus_bucket.argtypes = [P, i32, i64, i32, i32, P, P, P, P, sz, P]
    L.focus_bucket_noalloc.argtypes = [P, i32, i64, i32, i32, P, P, P, P]
    for name in ("focus_attn_fwd_workspace_bytes", "focus_attn_workspace_bytes"):
        getattr(L, name).argtypes = [ctypes.c_int, i32, i32, i64, i32, i32, i32]
        getattr(L, name).restype = sz
    L.focus_check_buckets.argtypes = [P, P, P, P, i32, i64, i32, i32, P, sz, P]
    attn = [P, P, P, ctypes.c_int, i32, i32, i64, i32, P, P, P, P, i32, i32, i64, f32,
            P, P, P, sz]
    L.focus_attn_fwd.argtypes = attn + [P]
    L.focus_attn_fwd_part.argtypes = attn + [i32, P]
    L.focus_dense_workspace_bytes.argtypes = [ctypes.c_int, i32, i64, i32]
    L.focus_dense_workspace_bytes.restype = sz
    L.focus_dense_causal_fwd.argtypes = [P, P, P, ctypes.c_int, i32, i32, i64, i32, f32,
                                         P, P, P, sz, P]
    L.focus_attn_bwd_workspace_bytes.argtypes = [ctypes.c_int, i32, i32, i64, i32, i32, i32]
    L.focus_attn_bwd_workspace_bytes.restype = sz
    L.focus_attn_bwd.argtypes = [P, P, P, P, P, P, ctypes.c_int, i32, i32, i64, i32, P, P, P, P,
                                 i32, i32, i64, f32, P, P, P, P, sz, P]
    L.focus_sinkhorn_workspace_bytes.argtypes = [i32, i64]
    L.focus_sinkhorn_workspace_bytes.restype = sz
    L.focus_sinkhorn.argtypes = [P, P, i32, i64, i32, i32, i32, P, P, sz, P]
    L.focus_gated_attn_workspace_bytes.argtypes = [i32, i64, i32, i32]
    L.focus_gated_attn_workspace_bytes.restype = sz
    L.focus_gated_attn_fwd.argtypes = [P, P, P, ctypes.c_int, i32, i32, i64, i32, P, i32, i64,
                                       f32, f32, P, P, P, sz, P]
    for name in ("focus_route", "focus_route_project", "focus_bucket", "focus_bucket_noalloc",
                 "focus_check_buckets",
                 "focus_attn_fwd",
                 "focus_attn_fwd_part", "focus_dense_causal_fwd", "focus_attn_bwd",
                 "focus_sinkhorn", "focus_gated_attn_fwd"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def status_string(status: int) -> str:
    return lib().focus_status_string(status).decode()


def _check(call: str, status: int) -> None:
    if status != 0:
        raise FocusError(call, status, lib().focus_last_error().decode())


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int:
    import torch

    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return FOCUS_BF16
    if t.dtype == torch.float32:
        return FOCUS_F32
    raise TypeError(f"inputs must be bfloat16 or float32, got {t.dtype}")


def _need(cond: bool, msg: str) -> None:
    if not cond:
        raise ValueError(msg)


# ----------------------------------------------------------------------------
# the C ABI, one function each

def focus_route(r, centroids, topk: int, groups=None, gmask=None, stream=None):
    """r fp32 [H, n, 16], centroids fp32 [H, K, 16] -> (groups int32 [H, n, topk],
    gmask int32 [H, n] holding the uint32 bit patterns)."""
    import torch

    H, n, dg = r.shape
    K = centroids.shape[1]
    if groups is None:
        groups = torch.empty((H, n, topk), dtype=torch.int32, device=r.device)
    if gmask is None:
        gmask = torch.empty((H, n), dtype=torch.int32, device=r.device)
    _check("focus_route", lib().focus_route(_ptr(r), _ptr(centroids), H, n, dg, K, topk,
                                            _ptr(groups), _ptr(gmask), _stream(stream)))
    return groups, gmask


def focus_route_project(x, Wt, centroids, topk: int, groups=None, gmask=None, r=None,
                        want_r: bool = False, stream=None):
    """x [n, d_model] (bf16 or fp32), Wt fp32 [d_model, 16] (row e: the 16 weights of
    hidden feature e), centroids fp32 [H, K, 16]
    -> (groups int32 [H, n, topk], gmask int32 [H, n], r fp32 [n, 16] or None).
    r is written when given or when want_r is set."""
    import torch

    n, dm = x.shape
    H, K, dg = centroids.shape
    _need(tuple(Wt.shape) == (dm, dg), f"Wt must be [{dm}, {dg}], got {tuple(Wt.shape)}")
    if groups is None:
        groups = torch.empty((H, n, topk), dtype=torch.int32, device=x.device)
    if gmask is None:
        gmask = torch.empty((H, n), dtype=torch.int32, device=x.device)
    if r is None and want_r:
        r = torch.empty((n, dg), dtype=torch.float32, device=x.device)
    _check("focus_route_project", lib().focus_route_project(
        _ptr(x), _dtype_code(x), n, dm, _ptr(Wt), _ptr(centroids), H, dg, K, topk,
        _ptr(groups), _ptr(gmask), _ptr(r), _stream(stream)))
    return groups, gmask, r


def focus_num_subbuckets(K: int, topk: int) -> int:
    """Sub-buckets per routing head: every (group, lower-set code)."""
    return int(lib().focus_num_subbuckets(K, topk))


def focus_bucket_workspace_bytes(H: int, n: int, K: int, topk: int) -> int:
    return int(lib().focus_bucket_workspace_bytes(H, n, K, topk))


def focus_bucket(groups, K: int, offsets=None, tokens=None, slot_entry=None, workspace=None,
                 stream=None):
    """groups int32 [H, n, topk] -> (offsets [H, focus_num_subbuckets(K, topk) + 1],
    tokens [H, n*topk], slot_entry [H, n, topk]), all int32."""
    import torch

    H, n, topk = groups.shape
    dev = groups.device
    nsb = focus_num_subbuckets(K, topk)
    if offsets is None:
        offsets = torch.empty((H, nsb + 1), dtype=torch.int32, device=dev)
    if tokens is None:
        tokens = torch.empty((H, n * topk), dtype=torch.int32, device=dev)
    if slot_entry is None:
        slot_entry = torch.empty((H, n, topk), dtype=torch.int32, device=dev)
    need = focus_bucket_workspace_bytes(H, n, K, topk)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    _check("focus_bucket", lib().focus_bucket(_ptr(groups), H, n, K, topk, _ptr(offsets),
                                              _ptr(tokens), _ptr(slot_entry), _ptr(workspace),
                                              workspace.numel(), _stream(stream)))
    return offsets, tokens, slot_entry


BUCKET_NOALLOC_SCRATCH_BYTES = 16 << 20  # FOCUS_BUCKET_NOALLOC_SCRATCH_BYTES


def focus_bucket_noalloc(groups, K: int, offsets=None, tokens=None, slot_entry=None,
                         stream=None):
    """focus_bucket without a workspace (the library's fixed per-device
    scratch holds the counts).  The C call allocates nothing; this wrapper
    allocates only the outputs that are not passed in."""
    import torch

    H, n, topk = groups.shape
    dev = groups.device
    if offsets is None:
        offsets = torch.empty((H, focus_num_subbuckets(K, topk) + 1), dtype=torch.int32,
                              device=dev)
    if tokens is None:
        tokens = torch.empty((H, n * topk), dtype=torch.int32, device=dev)
    if slot_entry is None:
        slot_entry = torch.empty((H, n, topk), dtype=torch.int32, device=dev)
    _check("focus_bucket_noalloc", lib().focus_bucket_noalloc(
        _ptr(groups), H, n, K, topk, _ptr(offsets), _ptr(tokens), _ptr(slot_entry),
        _stream(stream)))
    return offsets, tokens, slot_entry


def focus_attn_fwd_workspace_bytes(dtype_code: int, Hq: int, Hkv: int, n: int, d: int, K: int,
                                   topk: int) -> int:
    return int(lib().focus_attn_fwd_workspace_bytes(dtype_code, Hq, Hkv, n, d, K, topk))


def focus_attn_workspace_bytes(dtype_code: int, Hq: int, Hkv: int, n: int, d: int, K: int,
                               topk: int) -> int:
    """The same query as focus_attn_fwd_workspace_bytes, under its earlier name."""
    return int(lib().focus_attn_workspace_bytes(dtype_code, Hq, Hkv, n, d, K, topk))


def focus_check_buckets(gmask, offsets, tokens, slot_entry, K: int, workspace=None,
                        stream=None) -> None:
    """Raise FocusError (INVALID_ARGUMENT) unless (offsets, tokens, slot_entry)
    is the bucketing of the routing behind gmask; waits for the stream."""
    import torch

    H, n, topk = slot_entry.shape
    if workspace is None:
        workspace = torch.empty(CHECK_WORKSPACE_BYTES, dtype=torch.uint8, device=gmask.device)
    _check("focus_check_buckets", lib().focus_check_buckets(
        _ptr(gmask), _ptr(offsets), _ptr(tokens), _ptr(slot_entry), H, n, K, topk,
        _ptr(workspace), workspace.numel(), _stream(stream)))


def focus_attn_fwd_part(q, k, v, gmask, offsets, tokens, slot_entry, K: int, window: int,
                        scale: float, out, lse, workspace, parts: int = PART_ALL,
                        stream=None):
    Hq, n, d = q.shape
    Hkv = k.shape[0]
    topk = slot_entry.shape[2]
    _check("focus_attn_fwd_part", lib().focus_attn_fwd_part(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), Hq, Hkv, n, d, _ptr(gmask),
        _ptr(offsets), _ptr(tokens), _ptr(slot_entry), K, topk, int(window), float(scale),
        _ptr(out), _ptr(lse), _ptr(workspace), workspace.numel(), int(parts),
        _stream(stream)))
    return out, lse


def focus_attn_fwd(q, k, v, gmask, offsets, tokens, slot_entry, K: int, window: int,
                   scale: float, out=None, lse=None, workspace=None, stream=None):
    """q [Hq, n, d], k/v [Hkv, n, d] (bf16 or fp32) -> (out [Hq, n, d], lse fp32 [Hq, n])."""
    import torch

    Hq, n, d = q.shape
    Hkv = k.shape[0]
    topk = slot_entry.shape[2]
    _need(q.dtype == k.dtype == v.dtype, "q, k, v must share a dtype")
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, n), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = focus_attn_fwd_workspace_bytes(_dtype_code(q), Hq, Hkv, n, d, K, topk)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("focus_attn_fwd", lib().focus_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), Hq, Hkv, n, d, _ptr(gmask), _ptr(offsets),
        _ptr(tokens), _ptr(slot_entry), K, topk, int(window), float(scale), _ptr(out),
        _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def focus_dense_workspace_bytes(dtype_code: int, Hkv: int, n: int, d: int) -> int:
    return int(lib().focus_dense_workspace_bytes(dtype_code, Hkv, n, d))


def focus_dense_causal_fwd(q, k, v, scale: float, out=None, lse=None, workspace=None,
                           stream=None):
    import torch

    Hq, n, d = q.shape
    Hkv = k.shape[0]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, n), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = focus_dense_workspace_bytes(_dtype_code(q), Hkv, n, d)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("focus_dense_causal_fwd", lib().focus_dense_causal_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), Hq, Hkv, n, d, float(scale), _ptr(out),
        _ptr(lse), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out, lse


def focus_attn_bwd_workspace_bytes(dtype_code: int, Hq: int, Hkv: int, n: int, d: int,
                                   K: int, topk: int) -> int:
    return int(lib().focus_attn_bwd_workspace_bytes(dtype_code, Hq, Hkv, n, d, K, topk))


def focus_attn_bwd(q, k, v, out, lse, dout, gmask, offsets, tokens, slot_entry, K: int,
                   window: int, scale: float, dq=None, dk=None, dv=None, workspace=None,
                   stream=None):
    """Gradients of focus_attn_fwd: q, out, dout bf16 [Hq, n, d]; k, v bf16 [Hkv, n, d];
    lse fp32 [Hq, n]; the routing and buckets of the forward.
    Returns (dq [Hq, n, d], dk [Hkv, n, d], dv [Hkv, n, d]) in bf16."""
    import torch

    Hq, n, d = q.shape
    Hkv = k.shape[0]
    topk = slot_entry.shape[2]
    if dq is None:
        dq = torch.empty_like(q)
    if dk is None:
        dk = torch.empty_like(k)
    if dv is None:
        dv = torch.empty_like(v)
    if workspace is None:
        need = focus_attn_bwd_workspace_bytes(_dtype_code(q), Hq, Hkv, n, d, K, topk)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("focus_attn_bwd", lib().focus_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(dout), _dtype_code(q), Hq, Hkv,
        n, d, _ptr(gmask), _ptr(offsets), _ptr(tokens), _ptr(slot_entry), K, topk,
        int(window), float(scale), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return dq, dk, dv


def focus_sinkhorn(r, centroids, iters: int, assign=None, workspace=None, stream=None):
    """r fp32 [H, n, 16], centroids fp32 [H, K, 16] -> assign fp32 [H, n, K]."""
    import torch

    H, n, dg = r.shape
    K = centroids.shape[1]
    if assign is None:
        assign = torch.empty((H, n, K), dtype=torch.float32, device=r.device)
    if workspace is None:
        need = int(lib().focus_sinkhorn_workspace_bytes(H, n))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=r.device)
    _check("focus_sinkhorn", lib().focus_sinkhorn(
        _ptr(r), _ptr(centroids), H, n, dg, K, int(iters), _ptr(assign), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return assign


def focus_gated_attn_fwd(q, k, v, assign, window: int, lam: float, scale: float, out=None,
                         lse=None, workspace=None, stream=None):
    """Training-mode gated dense causal attention -> (out bf16 [Hq, n, d], lse fp32 [Hq, n])."""
    import torch

    Hq, n, d = q.shape
    Hkv = k.shape[0]
    K = assign.shape[2]
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((Hq, n), dtype=torch.float32, device=q.device)
    if workspace is None:
        need = int(lib().focus_gated_attn_workspace_bytes(Hkv, n, d, K))
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check("focus_gated_attn_fwd", lib().focus_gated_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _dtype_code(q), Hq, Hkv, n, d, _ptr(assign), K,
        int(window), float(lam), float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
        workspace.numel(), _stream(stream)))
    return out, lse


def focus_forward(q, k, v, r, centroids, topk: int, window: int, scale: float | None = None,
                  stream=None):
    """route -> bucket -> attention, allocating everything with torch.
    Returns dict(out, lse, groups, gmask, offsets, tokens, slot_entry)."""
    K = centroids.shape[1]
    if scale is None:
        scale = q.shape[-1] ** -0.5
    groups, gmask = focus_route(r, centroids, topk, stream=stream)
    offsets, tokens, slot_entry = focus_bucket(groups, K, stream=stream)
    out, lse = focus_attn_fwd(q, k, v, gmask, offsets, tokens, slot_entry, K, window, scale,
                              stream=stream)
    return dict(out=out, lse=lse, groups=groups, gmask=gmask, offsets=offsets,
                tokens=tokens, slot_entry=slot_entry)


# ----------------------------------------------------------------------------
# autograd: q, k, v get the gradients of focus_attn_fwd (the routing is a
# hard choice and gets none)

def _autograd_function():
    import torch

    class FocusAttention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, r, centroids, topk, window, scale):
            q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
            res = focus_forward(q, k, v, r, centroids, topk, window, scale)
            ctx.save_for_backward(q, k, v, res["out"], res["lse"], res["gmask"],
                                  res["offsets"], res["tokens"], res["slot_entry"])
            ctx.K = centroids.shape[1]
            ctx.window = window
            ctx.scale = scale
            return res["out"]

        @staticmethod
        def backward(ctx, dout):
            q, k, v, out, lse, gmask, offsets, tokens, slot_entry = ctx.saved_tensors
            dq, dk, dv = focus_attn_bwd(q, k, v, out, lse, dout.contiguous(), gmask, offsets,
                                        tokens, slot_entry, ctx.K, ctx.window, ctx.scale)
            return dq, dk, dv, None, None, None, None, None

    return FocusAttention


_FocusAttention = None


def focus_attention(q, k, v, r, centroids, topk: int, window: int, scale: float | None = None):
    """Differentiable Focus attention (bf16): out = focus_attn_fwd(...), and
    backward through focus_attn_bwd.  q [Hq, n, d], k/v [Hkv, n, d],
    r fp32 [Hkv, n, 16], centroids fp32 [Hkv, K, 16]."""
    global _FocusAttention
    if _FocusAttention is None:
        _FocusAttention = _autograd_function()
    if scale is None:
        scale = q.shape[-1] ** -0.5
    return _FocusAttention.apply(q, k, v, r, centroids, int(topk), int(window), float(scale))
