"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/focus.h declares, and rejects bad arguments before
anything is launched."""
import ctypes
import re
from pathlib import Path

import pytest

from centroid_gated_sparse_amd import focus as F

ROOT = Path(__file__).resolve().parents[1]
HEADER = (ROOT / "include" / "focus.h").read_text()


def declared_functions():
    body = re.sub(r"/\*.*?\*/", "", HEADER, flags=re.S)
    return sorted(set(re.findall(r"\b(focus_[a-z0-9_]+)\s*\(", body)))


@pytest.fixture(scope="module")
def L():
    if not F.LIB_PATH.exists():
        from centroid_gated_sparse_amd.build import build
        build()
    return F.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert len(names) == 22
    for name in names:
        assert hasattr(L, name), name
    assert set(names) == set(F.SYMBOLS)


def test_status_strings_and_version(L):
    assert L.focus_abi_version() == 1
    for code, text in [(0, "FOCUS_OK"), (1, "FOCUS_ERR_INVALID_ARGUMENT"),
                       (2, "FOCUS_ERR_UNSUPPORTED"), (3, "FOCUS_ERR_WORKSPACE"),
                       (4, "FOCUS_ERR_HIP"), (99, "FOCUS_ERR_UNKNOWN")]:
        assert F.status_string(code) == text


def test_workspace_sizes(L):
    # sub-buckets: group g of K holds 1, 1 + g, 1 + g + C(g, 2) or
    # 1 + g + C(g, 2) + C(g, 3) lower-set codes at top-1, top-2, top-3 (and
    # top-4 or more above K = 16), and top-4 or more up to K = 16
    assert F.focus_num_subbuckets(8, 1) == 8
    assert F.focus_num_subbuckets(8, 2) == 8 + 28
    assert F.focus_num_subbuckets(8, 3) == 8 + 28 + 56
    assert F.focus_num_subbuckets(8, 4) == F.focus_num_subbuckets(8, 6) == 8 + 28 + 56 + 70
    assert F.focus_num_subbuckets(16, 5) == 16 + 120 + 560 + 1820
    assert F.focus_num_subbuckets(17, 4) == 17 + 136 + 680
    assert F.focus_num_subbuckets(32, 4) == 32 + 496 + 4960
    assert F.focus_num_subbuckets(0, 1) == F.focus_num_subbuckets(4, 5) == 0
    assert F.focus_num_subbuckets(33, 2) == 0
    # bucket: one int per (head, sub-bucket, 512-token chunk)
    assert F.focus_bucket_workspace_bytes(8, 1 << 20, 8, 2) == 8 * 36 * 2048 * 4
    assert F.focus_bucket_workspace_bytes(1, 10, 0, 1) == 0
    # attention: at least the partials of every (query head, entry), O in
    # the I/O dtype and the LSE in fp32, plus the bucket-order K and V^T
    n, hq, hkv, d, K, k = 131072, 32, 8, 128, 4, 2
    ws = F.focus_attn_workspace_bytes(F.FOCUS_BF16, hq, hkv, n, d, K, k)
    assert ws >= hq * n * k * (d * 2 + 4) + 2 * hkv * n * k * d * 2
    assert ws < 2 * hq * n * k * (d * 2 + 4) + 4 * hkv * (n * k + n) * d * 2
    ws32 = F.focus_attn_workspace_bytes(F.FOCUS_F32, hq, hkv, n, d, K, k)
    assert ws32 >= hq * n * k * (d + 1) * 4
    assert F.focus_attn_workspace_bytes(F.FOCUS_BF16, hq, hkv, n, 96, K, k) == 0
    assert F.focus_attn_workspace_bytes(F.FOCUS_BF16, 6, 4, n, d, K, k) == 0
    assert F.focus_dense_workspace_bytes(F.FOCUS_F32, 2, 512, 64) > 0
    # the workspace query under both of its names
    for args in [(F.FOCUS_BF16, hq, hkv, n, d, K, k), (F.FOCUS_F32, 2, 2, 512, 64, 4, 1),
                 (F.FOCUS_BF16, hq, hkv, n, 96, K, k)]:
        assert F.focus_attn_fwd_workspace_bytes(*args) == F.focus_attn_workspace_bytes(*args)


# An aligned non-null address.  Every call below carries at least one invalid
# argument, so the library returns before launching anything.  As a guard
# against a validation regression turning one of them into a launch on a fake
# address, these tests only run where no GPU is visible.
FAKE = 1 << 20
no_gpu = pytest.mark.skipif(
    __import__("conftest").gpu_available(),
    reason="fake-pointer validation tests run only where no GPU is visible")


@no_gpu
def test_route_rejects_bad_arguments(L):
    call = lambda *a: L.focus_route(*a)
    ok = (FAKE, FAKE, 2, 100, 16, 4, 2, FAKE, FAKE, None)
    assert call(None, *ok[1:]) == 1
    assert call(FAKE + 4, *ok[1:]) == 1            # misaligned
    assert call(*ok[:4], 8, *ok[5:]) == 2          # d_g != 16
    assert call(*ok[:5], 33, 2, *ok[7:]) == 2      # K > 32
    assert call(*ok[:5], 4, 5, *ok[7:]) == 1       # topk > K
    assert call(*ok[:3], 0, *ok[4:]) == 1          # n < 1
    assert call(*ok[:5], 4, 0, *ok[7:]) == 1       # topk < 1
    assert b"topk" in L.focus_last_error()


@no_gpu
def test_route_project_rejects_bad_arguments(L):
    f = L.focus_route_project
    # x, xdt, n, d_model, Wt, centroids, H, d_g, K, topk, groups, gmask, r, stream
    ok = [FAKE, F.FOCUS_BF16, 100, 768, FAKE, FAKE, 4, 16, 8, 2, FAKE, FAKE, None, None]

    def call(**over):
        a = list(ok)
        for i, v in over.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a0=None) == 1                      # x null
    assert call(a4=FAKE + 4) == 1                  # Wt misaligned
    assert call(a12=FAKE + 8) == 1                 # r given but misaligned
    assert call(a1=3) == 1                         # dtype
    assert call(a2=0) == 1                         # n < 1
    assert call(a3=0) == 1                         # d_model < 1
    assert call(a6=0) == 1                         # H < 1
    assert call(a7=8) == 2                         # d_g != 16
    assert call(a8=33) == 2                        # K > 32
    assert call(a9=9) == 1                         # topk > K
    assert call(a9=0) == 1
    assert b"topk" in L.focus_last_error()


@no_gpu
def test_bucket_rejects_bad_arguments(L):
    ok = [FAKE, 2, 100, 4, 2, FAKE, FAKE, FAKE, FAKE, 1 << 30, None]
    bad = list(ok); bad[8] = None
    assert L.focus_bucket(*bad) == 3               # missing workspace
    bad = list(ok); bad[9] = 16
    assert L.focus_bucket(*bad) == 3               # short workspace
    bad = list(ok); bad[2] = 1 << 31
    assert L.focus_bucket(*bad) == 1               # n * topk > INT32_MAX
    bad = list(ok); bad[3] = 40
    assert L.focus_bucket(*bad) == 2


def _attn_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, dt=F.FOCUS_BF16, Hq=8, Hkv=2, n=256, d=128, gmask=FAKE,
             offsets=FAKE, tokens=FAKE, slot=FAKE, K=4, topk=2, window=16, scale=0.088,
             out=FAKE, lse=FAKE, ws=FAKE, wsb=1 << 40, parts=7, stream=None)
    a.update(over)
    return list(a.values())


@no_gpu
def test_attn_rejects_bad_arguments(L):
    f = L.focus_attn_fwd_part
    assert f(*_attn_args(Hq=7)) == 1               # Hq % Hkv
    assert f(*_attn_args(d=96)) == 2
    assert f(*_attn_args(window=-1)) == 1
    assert f(*_attn_args(topk=5)) == 1
    assert f(*_attn_args(K=33, topk=2)) == 2
    assert f(*_attn_args(q=None)) == 1
    assert f(*_attn_args(out=FAKE + 8)) == 1
    assert f(*_attn_args(wsb=64)) == 3
    assert f(*_attn_args(parts=0)) == 1
    assert f(*_attn_args(parts=8)) == 1
    assert f(*_attn_args(scale=0.0)) == 1
    assert f(*_attn_args(dt=5)) == 1
    d = L.focus_dense_causal_fwd
    assert d(FAKE, FAKE, FAKE, 1, 8, 3, 256, 128, 0.1, FAKE, FAKE, FAKE, 1 << 30, None) == 1
    assert d(FAKE, FAKE, FAKE, 1, 8, 2, 256, 64, 0.1, FAKE, FAKE, None, 0, None) == 3


def _bwd_args(**over):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, lse=FAKE, dout=FAKE, dt=F.FOCUS_BF16, Hq=8,
             Hkv=2, n=256, d=128, gmask=FAKE, offsets=FAKE, tokens=FAKE, slot=FAKE, K=4,
             topk=2, window=16, scale=0.088, dq=FAKE, dk=FAKE, dv=FAKE, ws=FAKE,
             wsb=1 << 40, stream=None)
    a.update(over)
    return list(a.values())


@no_gpu
def test_attn_bwd_rejects_bad_arguments(L):
    f = L.focus_attn_bwd
    assert f(*_bwd_args(dt=F.FOCUS_F32)) == 2          # bf16 only
    assert f(*_bwd_args(d=96)) == 2
    assert f(*_bwd_args(Hq=7)) == 1                    # Hq % Hkv
    assert f(*_bwd_args(dout=None)) == 1
    assert f(*_bwd_args(lse=FAKE + 4)) == 1
    assert f(*_bwd_args(dv=None)) == 1
    assert f(*_bwd_args(window=-1)) == 1
    assert f(*_bwd_args(topk=5)) == 1
    assert f(*_bwd_args(wsb=64)) == 3
    assert F.focus_attn_bwd_workspace_bytes(F.FOCUS_F32, 8, 2, 256, 128, 4, 2) == 0
    ws = F.focus_attn_bwd_workspace_bytes(F.FOCUS_BF16, 8, 2, 256, 128, 4, 2)
    # at least the fp32 partials of every row and entry
    assert ws >= 4 * 128 * (8 * 256 + 2 * 2 * 256 + 8 * 512 + 2 * 2 * 512)


@no_gpu
def test_training_forward_rejects_bad_arguments(L):
    s = L.focus_sinkhorn
    ok = [FAKE, FAKE, 2, 100, 16, 4, 3, FAKE, FAKE, 1 << 30, None]
    bad = list(ok); bad[6] = 0
    assert s(*bad) == 1                                # iters < 1
    bad = list(ok); bad[4] = 8
    assert s(*bad) == 2                                # d_g != 16
    bad = list(ok); bad[5] = 33
    assert s(*bad) == 2
    bad = list(ok); bad[9] = 8
    assert s(*bad) == 3                                # short workspace
    g = L.focus_gated_attn_fwd
    okg = [FAKE, FAKE, FAKE, F.FOCUS_BF16, 8, 2, 256, 128, FAKE, 4, 16, 1.5, 0.088, FAKE, FAKE,
           FAKE, 1 << 30, None]
    bad = list(okg); bad[3] = F.FOCUS_F32
    assert g(*bad) == 2
    bad = list(okg); bad[11] = float("nan")
    assert g(*bad) == 1
    bad = list(okg); bad[8] = None
    assert g(*bad) == 1
    bad = list(okg); bad[9] = 40
    assert g(*bad) == 2
    bad = list(okg); bad[16] = 8
    assert g(*bad) == 3                                # short workspace


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(F, "_lib", None)
    monkeypatch.setattr(F, "LIB_PATH", tmp_path / "missing.so")
    with pytest.raises(RuntimeError, match="not built"):
        F.lib()


@no_gpu
def test_check_buckets_rejects_bad_arguments(L):
    # gmask, offsets, tokens, slot_entry, H, n, K, topk, workspace, bytes, stream
    ok = [FAKE, FAKE, FAKE, FAKE, 8, 1000, 8, 2, FAKE, F.CHECK_WORKSPACE_BYTES, None]

    def call(**over):
        a = list(ok)
        for i, v in over.items():
            a[int(i[1:])] = v
        return L.focus_check_buckets(*a)

    assert call(a0=None) == 1                      # gmask null
    assert call(a2=FAKE + 4) == 1                  # tokens misaligned
    assert call(a4=0) == 1                         # H < 1
    assert call(a5=0) == 1                         # n < 1
    assert call(a6=33) == 2                        # K > 32
    assert call(a7=9) == 1                         # topk > K
    assert call(a5=1 << 31) == 1                   # n * topk > INT32_MAX
    assert call(a8=None) == 3                      # no workspace
    assert call(a9=F.CHECK_WORKSPACE_BYTES - 1) == 3


@no_gpu
def test_bucket_noalloc_rejects_bad_arguments(L):
    # groups, H, n, K, topk, offsets, tokens, slot_entry, stream
    ok = [FAKE, 2, 100, 4, 2, FAKE, FAKE, FAKE, None]
    bad = list(ok); bad[0] = None
    assert L.focus_bucket_noalloc(*bad) == 1       # groups null
    bad = list(ok); bad[4] = 5
    assert L.focus_bucket_noalloc(*bad) == 1       # topk > K
    bad = list(ok); bad[3] = 40
    assert L.focus_bucket_noalloc(*bad) == 2       # K > 32
    bad = list(ok); bad[2] = 1 << 31
    assert L.focus_bucket_noalloc(*bad) == 1       # n * topk > INT32_MAX
    # beyond the fixed scratch: 8 heads of 1M tokens at K = 32 need 66 MiB of counts
    big = [FAKE, 8, 1 << 20, 32, 2, FAKE, FAKE, FAKE, None]
    assert F.focus_bucket_workspace_bytes(8, 1 << 20, 32, 2) > F.BUCKET_NOALLOC_SCRATCH_BYTES
    assert L.focus_bucket_noalloc(*big) == 3
    assert b"scratch" in L.focus_last_error()
