"""The bucketing check (focus_check_buckets, and FOCUS_DEBUG=1 in front of
focus_attn_fwd / focus_attn_bwd): consistent buckets pass; each kind of
inconsistency is reported as INVALID_ARGUMENT before any kernel reads rows
through the buckets.  The corrupted arrays only ever reach the checking
kernels, which range-test every value before using it as an index."""
import numpy as np
import pytest
import torch

from centroid_gated_sparse_amd import focus as F
from centroid_gated_sparse_amd.workloads import Workload, qkv_inputs, routing_inputs

pytestmark = pytest.mark.gpu
DEV = "cuda"


def log(msg):
    print(msg, flush=True)


def routed(wl, seed):
    c, r, _ = routing_inputs(wl, seed)
    groups, gmask = F.focus_route(torch.from_numpy(r).to(DEV), torch.from_numpy(c).to(DEV),
                                  wl.topk)
    offsets, tokens, slot_entry = F.focus_bucket(groups, wl.K)
    torch.cuda.synchronize()
    return c, r, gmask, offsets, tokens, slot_entry


def expect_invalid(fn, what):
    with pytest.raises(F.FocusError) as ei:
        fn()
    assert ei.value.status == 1, what
    log(f"  {what}: {ei.value}")
    return str(ei.value)


def corruptions(wl, gmask, offsets, tokens, slot_entry):
    """(name, expected word in the message, gmask, offsets, tokens, slot_entry)."""
    E = wl.n * wl.topk
    off = offsets.cpu().numpy()
    tok = tokens.cpu().numpy()
    # the first sub-bucket of head 0 with at least two entries
    sb = int(np.nonzero(np.diff(off[0]) >= 2)[0][0])
    a = int(off[0, sb])
    out = []

    def case(name, word, gm=None, of=None, tk=None, se=None):
        out.append((name, word, gmask if gm is None else gm, offsets if of is None else of,
                    tokens if tk is None else tk, slot_entry if se is None else se))

    t = tokens.clone(); t[0, a], t[0, a + 1] = tokens[0, a + 1], tokens[0, a]
    case("two entries of a sub-bucket swapped", "tokens", tk=t)
    t = tokens.clone(); t[1, E // 2] = wl.n + 5
    case("a position past the sequence", "tokens", tk=t)
    t = tokens.clone(); t[0, E - 1] = -1
    case("a negative position", "tokens", tk=t)
    t = tokens.clone(); t[0, E - 1] = 2 ** 31 - 1
    case("the largest int32 position", "tokens", tk=t)
    s = slot_entry.clone(); s[0, 3, 0], s[0, 4, 0] = slot_entry[0, 4, 0], slot_entry[0, 3, 0]
    case("slot entries of two tokens swapped", "slot_entry", se=s)
    s = slot_entry.clone(); s[1, wl.n - 1, wl.topk - 1] = E + 100
    case("a slot entry past the entries", "slot_entry", se=s)
    s = slot_entry.clone(); s[0, 0, 0] = -7
    case("a negative slot entry", "slot_entry", se=s)
    o = offsets.clone(); o[0, -1] = E - 1
    case("offsets not ending at n * topk", "offsets", of=o)
    o = offsets.clone(); o[1, 1] = E
    case("offsets decreasing", "offsets", of=o)
    o = offsets.clone(); o[0, 0] = 3
    case("offsets not starting at 0", "offsets", of=o)
    o = offsets.clone(); o[0, sb + 1] += 1   # the next sub-bucket's first entry joins sb
    case("an entry moved to the previous sub-bucket", "", of=o)
    m = gmask.clone(); m[0, 10] = gmask[0, 10] ^ 1
    case("a group bit flipped", "groups", gm=m)
    g0 = int(gmask[1, 0].item()) & 0xFFFFFFFF
    extra = next(g for g in range(wl.K) if not (g0 >> g) & 1)
    m = gmask.clone(); m[1, 0] = np.int32(np.uint32(g0 | (1 << extra)).view(np.int32))
    case("a token holding an extra group", "groups", gm=m)
    return out


CASES = [
    Workload("check_k8_top2", 1500, 4, 2, 64, 8, 2, 32, "bf16", qkv_std=0.125),
    Workload("check_k4_top1", 900, 2, 2, 128, 4, 1, 16, "bf16", qkv_std=0.09),
    Workload("check_k16_top3", 1100, 4, 2, 64, 16, 3, 8, "bf16", qkv_std=0.125),
    Workload("check_k8_top4", 1000, 2, 2, 64, 8, 4, 16, "bf16", qkv_std=0.125),
    Workload("check_k16_top5", 900, 2, 2, 64, 16, 5, 16, "bf16", qkv_std=0.125),
    Workload("check_k20_top4", 900, 2, 2, 64, 20, 4, 16, "bf16", qkv_std=0.125),
]


@pytest.mark.parametrize("wl", CASES, ids=lambda w: w.name)
def test_check_buckets_entry_point(wl):
    log(f"bucket check {wl.name}")
    _, _, gmask, offsets, tokens, slot_entry = routed(wl, 515)
    F.focus_check_buckets(gmask, offsets, tokens, slot_entry, wl.K)
    for name, word, gm, of, tk, se in corruptions(wl, gmask, offsets, tokens, slot_entry):
        msg = expect_invalid(lambda: F.focus_check_buckets(gm, of, tk, se, wl.K), name)
        assert word in msg, (name, msg)
    # the valid buckets still pass after the failures (the flag is cleared per call)
    F.focus_check_buckets(gmask, offsets, tokens, slot_entry, wl.K)


def test_debug_mode_guards_forward_and_backward(monkeypatch):
    wl = CASES[0]
    log(f"FOCUS_DEBUG forward/backward {wl.name}")
    c, r, gmask, offsets, tokens, slot_entry = routed(wl, 616)
    q, k, v = qkv_inputs(wl, 616, DEV)
    ref_out, ref_lse = F.focus_attn_fwd(q, k, v, gmask, offsets, tokens, slot_entry, wl.K,
                                        wl.window, wl.scale)
    torch.cuda.synchronize()
    monkeypatch.setenv("FOCUS_DEBUG", "1")
    out, lse = F.focus_attn_fwd(q, k, v, gmask, offsets, tokens, slot_entry, wl.K, wl.window,
                                wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(lse, ref_lse)
    dout = torch.randn_like(q)
    F.focus_attn_bwd(q, k, v, out, lse, dout, gmask, offsets, tokens, slot_entry, wl.K,
                     wl.window, wl.scale)
    torch.cuda.synchronize()
    for name, _, gm, of, tk, se in corruptions(wl, gmask, offsets, tokens, slot_entry):
        sentinel = torch.full_like(out, 7.0)
        expect_invalid(lambda: F.focus_attn_fwd(q, k, v, gm, of, tk, se, wl.K, wl.window,
                                                wl.scale, out=sentinel), "forward: " + name)
        torch.cuda.synchronize()
        assert bool((sentinel == 7.0).all()), "nothing may run after a failed check"
        expect_invalid(lambda: F.focus_attn_bwd(q, k, v, out, lse, dout, gm, of, tk, se, wl.K,
                                                wl.window, wl.scale), "backward: " + name)
    monkeypatch.delenv("FOCUS_DEBUG")
    # switched off again: the same call goes through unchecked on valid input
    out2, _ = F.focus_attn_fwd(q, k, v, gmask, offsets, tokens, slot_entry, wl.K, wl.window,
                               wl.scale)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref_out)
