"""CPU oracle for the Focus attention forward path.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package.  The product library
(``centroid_gated_sparse_amd``) never imports it, and it imports nothing from
the product.

The arithmetic lives in ``focus_oracle.c`` (plain C, built with gcc
``-O2 -ffp-contract=off -fopenmp``); this module only builds it, marshals
numpy arrays into it and returns numpy arrays.  Every function cites the
passage of the Focus pages it follows in the C source.

Pins: every function here is checked against values fixed by the pages and by
mathematics (closed forms, library softmax on special cases, brute force on
tiny inputs) in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "focus_oracle.c"
_LIB_PATH = _HERE / "libfocus_oracle.so"
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-fPIC",
           "-shared", "-std=c11", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> Path:
    """Compile the oracle with gcc into ``oracle/libfocus_oracle.so``."""
    if force or not _LIB_PATH.exists():
        tmp = _LIB_PATH.with_suffix(".so.tmp")
        cmd = ["gcc", *_CFLAGS, str(_SRC), "-o", str(tmp), "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # The mutation test points this at a deliberately broken copy.
    override = os.environ.get("FOCUS_ORACLE_LIB")
    if override:
        lib = ctypes.CDLL(override)
    else:
        if not _LIB_PATH.exists():
            build(force=True)
        lib = ctypes.CDLL(str(_LIB_PATH))
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.oracle_route.argtypes = [P, P, i32, i64, i32, i32, i32, P, P]
    lib.oracle_bucket.argtypes = [P, i32, i64, i32, i32, P, P, P]
    lib.oracle_num_subbuckets.argtypes = [i32, i32]
    lib.oracle_num_subbuckets.restype = i32
    lib.oracle_attn_rows.argtypes = [P, i32, P, P, i32, i32, i32, i64, i32, P, i32, i32,
                                     i64, f64, P, P, i64, P, P, P, i32]
    lib.oracle_pair_counts.argtypes = [P, i32, i64, i32, i32, i64, P]
    lib.oracle_project.argtypes = [P, i32, i64, i32, P, P]
    lib.oracle_attn_bwd_rows.argtypes = [P, P, P, P, i32, i32, i32, i64, i32, P, i32, i32,
                                         i64, f64, P, P, i64, P, i32]
    lib.oracle_attn_bwd.argtypes = [P, P, P, P, i32, i32, i32, i64, i32, P, i32, i32, i64,
                                    f64, P, P, P, i32]
    lib.oracle_sinkhorn.argtypes = [P, P, i32, i64, i32, i32, i32, P]
    lib.oracle_gated_attn_rows.argtypes = [P, P, P, i32, i32, i32, i64, i32, P, i32, i64, f64,
                                           f64, P, P, i64, P, P, i32]
    for f in (lib.oracle_route, lib.oracle_bucket, lib.oracle_attn_rows,
              lib.oracle_pair_counts, lib.oracle_project, lib.oracle_attn_bwd_rows,
              lib.oracle_attn_bwd, lib.oracle_sinkhorn, lib.oracle_gated_attn_rows):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    assert a.flags["C_CONTIGUOUS"]
    return ctypes.c_void_p(a.ctypes.data)


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def route(r: np.ndarray, centroids: np.ndarray, topk: int):
    """Top-k groups of every token.

    r: float32 [H, n, d_g]; centroids: float32 [H, K, d_g].
    Returns (groups int32 [H, n, topk] in score order, gmask uint32 [H, n]).
    """
    r = np.ascontiguousarray(r, dtype=np.float32)
    c = np.ascontiguousarray(centroids, dtype=np.float32)
    H, n, dg = r.shape
    K = c.shape[1]
    assert c.shape == (H, K, dg)
    groups = np.empty((H, n, topk), np.int32)
    gmask = np.empty((H, n), np.uint32)
    _check(_load().oracle_route(_ptr(r), _ptr(c), H, n, dg, K, topk,
                                _ptr(groups), _ptr(gmask)), "route")
    return groups, gmask


def project(x: np.ndarray, W: np.ndarray) -> np.ndarray:
    """Routing projection r = W x of every token, in the fixed fp32 order.

    x: [n, d_model] float32, or uint16 bf16 bit patterns; W: float32 [16, d_model].
    Returns r float32 [n, 16].
    """
    is_bf16 = x.dtype == np.uint16
    x = np.ascontiguousarray(x)
    W = np.ascontiguousarray(W, dtype=np.float32)
    n, dm = x.shape
    assert W.shape == (16, dm)
    r = np.empty((n, 16), np.float32)
    _check(_load().oracle_project(_ptr(x), int(is_bf16), n, dm, _ptr(W), _ptr(r)), "project")
    return r


def route_project(x: np.ndarray, W: np.ndarray, centroids: np.ndarray, topk: int):
    """Projection shared by all routing heads, then each head's top-k.

    Returns (r float32 [n, 16], groups int32 [H, n, topk], gmask uint32 [H, n]).
    """
    r = project(x, W)
    H = centroids.shape[0]
    rh = np.ascontiguousarray(np.broadcast_to(r, (H,) + r.shape))
    groups, gmask = route(rh, centroids, topk)
    return r, groups, gmask


def num_subbuckets(K: int, topk: int) -> int:
    """Sub-buckets per routing head: every (group, lower-set code)."""
    return int(_load().oracle_num_subbuckets(int(K), int(topk)))


def bucket(groups: np.ndarray, K: int):
    """Per-head stable bucketing of (token, group) entries.

    Sub-buckets are (group, lower-set code) pairs, num_subbuckets(K, topk)
    per head.  Returns (offsets int32 [H, num_subbuckets + 1],
    tokens int32 [H, n*topk], slot_entry int32 [H, n, topk]).
    """
    groups = np.ascontiguousarray(groups, dtype=np.int32)
    H, n, topk = groups.shape
    nsb = num_subbuckets(K, topk)
    offsets = np.empty((H, nsb + 1), np.int32)
    tokens = np.empty((H, n * topk), np.int32)
    slot_entry = np.empty((H, n, topk), np.int32)
    _check(_load().oracle_bucket(_ptr(groups), H, n, K, topk, _ptr(offsets),
                                 _ptr(tokens), _ptr(slot_entry)), "bucket")
    return offsets, tokens, slot_entry


def _as_raw(x) -> tuple[np.ndarray, int]:
    """Accept float32 arrays, or bf16 given as uint16 bit patterns."""
    a = np.ascontiguousarray(x)
    if a.dtype == np.float32:
        return a, 0
    if a.dtype == np.uint16:
        return a, 1
    raise TypeError(f"oracle attention takes float32 or bf16 bits (uint16), got {a.dtype}")


def attn_rows(q, k, v, groups: np.ndarray, K: int, window: int, scale: float,
              row_head: np.ndarray, row_pos: np.ndarray, nthreads: int = 0,
              num_q_heads: int | None = None):
    """Exact softmax over A(i) for the listed (query head, row) pairs.

    q: [Hq, n, d], or [rows, d] holding just the listed rows' queries (then
    pass num_q_heads); k, v: [Hkv, n, d] (float32, or uint16 holding bf16
    bits); groups: int32 [Hkv, n, topk].
    Returns (o float64 [rows, d], lse float64 [rows], count int64 [rows]).
    """
    qa, qb = _as_raw(q)
    ka, kb = _as_raw(k)
    va, vb = _as_raw(v)
    assert qb == kb == vb
    Hkv, n, d = ka.shape
    q_per_row = qa.ndim == 2
    if q_per_row:
        assert num_q_heads is not None and qa.shape == (len(row_head), d)
        Hq = int(num_q_heads)
    else:
        Hq = qa.shape[0]
        assert qa.shape == (Hq, n, d)
    assert ka.shape == (Hkv, n, d) and va.shape == (Hkv, n, d)
    groups = np.ascontiguousarray(groups, dtype=np.int32)
    assert groups.shape[:2] == (Hkv, n)
    topk = groups.shape[2]
    rh = np.ascontiguousarray(row_head, dtype=np.int32)
    rp = np.ascontiguousarray(row_pos, dtype=np.int64)
    nrows = rh.shape[0]
    o = np.empty((nrows, d), np.float64)
    lse = np.empty(nrows, np.float64)
    cnt = np.empty(nrows, np.int64)
    _check(_load().oracle_attn_rows(_ptr(qa), int(q_per_row), _ptr(ka), _ptr(va), qb, Hq,
                                    Hkv, n, d,
                                    _ptr(groups), K, topk, int(window), float(scale),
                                    _ptr(rh), _ptr(rp), nrows, _ptr(o), _ptr(lse),
                                    _ptr(cnt), int(nthreads)), "attn_rows")
    return o, lse, cnt


def attn_full(q, k, v, groups: np.ndarray, K: int, window: int, scale: float,
              nthreads: int = 0):
    """Every row of every query head: (o [Hq, n, d], lse [Hq, n], count [Hq, n])."""
    qa, _ = _as_raw(q)
    Hq, n, d = qa.shape
    rh = np.repeat(np.arange(Hq, dtype=np.int32), n)
    rp = np.tile(np.arange(n, dtype=np.int64), Hq)
    o, lse, cnt = attn_rows(q, k, v, groups, K, window, scale, rh, rp, nthreads)
    return o.reshape(Hq, n, d), lse.reshape(Hq, n), cnt.reshape(Hq, n)


def pair_counts(groups: np.ndarray, K: int, window: int) -> np.ndarray:
    """|A(i)| for every routing head and row: int64 [H, n]."""
    groups = np.ascontiguousarray(groups, dtype=np.int32)
    H, n, topk = groups.shape
    out = np.empty((H, n), np.int64)
    _check(_load().oracle_pair_counts(_ptr(groups), H, n, K, topk, int(window),
                                      _ptr(out)), "pair_counts")
    return out


def attn_bwd(q, k, v, dout, groups: np.ndarray, K: int, window: int, scale: float,
             nthreads: int = 0):
    """Gradients of the exact softmax over A(i) with respect to q, k and v,
    given the output gradient dout [Hq, n, d] (same dtype convention as q).
    Returns (dq [Hq, n, d], dk [Hkv, n, d], dv [Hkv, n, d]), float64."""
    qa, qb = _as_raw(q)
    ka, kb = _as_raw(k)
    va, vb = _as_raw(v)
    da, db = _as_raw(dout)
    assert qb == kb == vb == db
    Hq, n, d = qa.shape
    Hkv = ka.shape[0]
    assert ka.shape == va.shape == (Hkv, n, d) and da.shape == qa.shape
    groups = np.ascontiguousarray(groups, dtype=np.int32)
    assert groups.shape[:2] == (Hkv, n)
    topk = groups.shape[2]
    dq = np.empty((Hq, n, d), np.float64)
    dk = np.empty((Hkv, n, d), np.float64)
    dv = np.empty((Hkv, n, d), np.float64)
    _check(_load().oracle_attn_bwd(_ptr(qa), _ptr(ka), _ptr(va), _ptr(da), qb, Hq, Hkv, n,
                                   d, _ptr(groups), K, topk, int(window), float(scale),
                                   _ptr(dq), _ptr(dk), _ptr(dv), int(nthreads)), "attn_bwd")
    return dq, dk, dv


def attn_bwd_rows(q, k, v, dout, groups: np.ndarray, K: int, window: int, scale: float,
                  row_head: np.ndarray, row_pos: np.ndarray, nthreads: int = 0):
    """dq of the listed (query head, position) rows: float64 [rows, d]."""
    qa, qb = _as_raw(q)
    ka, kb = _as_raw(k)
    va, vb = _as_raw(v)
    da, db = _as_raw(dout)
    assert qb == kb == vb == db
    Hq, n, d = qa.shape
    Hkv = ka.shape[0]
    groups = np.ascontiguousarray(groups, dtype=np.int32)
    topk = groups.shape[2]
    rh = np.ascontiguousarray(row_head, dtype=np.int32)
    rp = np.ascontiguousarray(row_pos, dtype=np.int64)
    dq = np.empty((rh.shape[0], d), np.float64)
    _check(_load().oracle_attn_bwd_rows(_ptr(qa), _ptr(ka), _ptr(va), _ptr(da), qb, Hq, Hkv,
                                        n, d, _ptr(groups), K, topk, int(window),
                                        float(scale), _ptr(rh), _ptr(rp), rh.shape[0],
                                        _ptr(dq), int(nthreads)), "attn_bwd_rows")
    return dq


def sinkhorn(r: np.ndarray, centroids: np.ndarray, iters: int) -> np.ndarray:
    """Sinkhorn soft assignment of every token to the groups: float64
    [H, n, K], rows summing to 1 and columns approaching n/K."""
    r = np.ascontiguousarray(r, dtype=np.float32)
    c = np.ascontiguousarray(centroids, dtype=np.float32)
    H, n, dg = r.shape
    K = c.shape[1]
    A = np.empty((H, n, K), np.float64)
    _check(_load().oracle_sinkhorn(_ptr(r), _ptr(c), H, n, dg, K, int(iters), _ptr(A)),
           "sinkhorn")
    return A


def gated_attn_rows(q, k, v, A: np.ndarray, window: int, lam: float, scale: float,
                    row_head: np.ndarray, row_pos: np.ndarray, nthreads: int = 0):
    """Training-mode gated dense causal attention of the listed rows.
    A: float64 [Hkv, n, K] assignment.  Returns (o [rows, d], lse [rows])."""
    qa, qb = _as_raw(q)
    ka, kb = _as_raw(k)
    va, vb = _as_raw(v)
    assert qb == kb == vb
    Hq, n, d = qa.shape
    Hkv = ka.shape[0]
    A = np.ascontiguousarray(A, dtype=np.float64)
    assert A.shape[:2] == (Hkv, n)
    K = A.shape[2]
    rh = np.ascontiguousarray(row_head, dtype=np.int32)
    rp = np.ascontiguousarray(row_pos, dtype=np.int64)
    o = np.empty((rh.shape[0], d), np.float64)
    lse = np.empty(rh.shape[0], np.float64)
    _check(_load().oracle_gated_attn_rows(_ptr(qa), _ptr(ka), _ptr(va), qb, Hq, Hkv, n, d,
                                          _ptr(A), K, int(window), float(lam), float(scale),
                                          _ptr(rh), _ptr(rp), rh.shape[0], _ptr(o), _ptr(lse),
                                          int(nthreads)), "gated_attn_rows")
    return o, lse
