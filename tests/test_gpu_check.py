"""GPU tests of moe_check_routing, the layer's debug check of a routing
table and its group offsets: ids outside [0, E), a token naming one expert
twice, and offsets that are not the exclusive prefix of the local group
sizes (first slot per expert, clamped to the row capacity) that moe_permute
writes.  The expected offsets come from the oracle's permute; the expected
range and repeat bits from their definitions on the table."""
import sys

import numpy as np
import pytest
import torch

from mixture_experts_layer_50_amd import binding as B
from oracle import moe_oracle as O

pytestmark = pytest.mark.gpu

RANGE, REPEAT, OFFSETS = 1, 2, 4


def _announce(name):
    print(f"\n[gpu case] {name}", flush=True)
    sys.stdout.flush()


def _expected_bits(idx, E):
    bits = 0
    if np.any((idx < 0) | (idx >= E)):
        bits |= RANGE
    k = idx.shape[1]
    if any(np.any(idx[:, :j] == idx[:, j:j + 1]) for j in range(1, k)):
        bits |= REPEAT
    return bits


def _check(s, idx_dev, offsets_dev, flags=None):
    if flags is None:
        flags = torch.zeros(1, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(B.workspace_size(s, "check_routing"), 256), dtype=torch.uint8,
                     device="cuda")
    B.moe_check_routing(s, idx_dev, offsets_dev, flags, ws)
    torch.cuda.synchronize()
    return int(flags.item()), flags


def _table(T, E, k, seed, bad=True):
    rng = np.random.default_rng(seed)
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    if bad:
        idx[T // 3, 0] = E + 2             # out of range, high
        idx[T - 1, k - 1] = -1             # out of range, negative, in the last token
        idx[1, 1] = idx[1, 0]              # a repeat
    return idx


@pytest.mark.parametrize("T,E,k,e_lo,e_hi,R_cap", [
    (300, 16, 4, 0, 16, 0),
    (300, 16, 4, 4, 12, 0),
    (1000, 64, 6, 8, 40, 2000),            # the capacity clamps the offsets
    (4096, 128, 8, 0, 128, 0),
    (77, 512, 32, 100, 356, 0),
])
def test_check_routing_table_and_offsets(T, E, k, e_lo, e_hi, R_cap):
    _announce(f"check_routing T={T} E={E} k={k} local=[{e_lo},{e_hi}) R_cap={R_cap}")
    s = B.MoEShape.make(T, 64, E, k, 64, e_lo=e_lo, e_hi=e_hi, R_cap=R_cap)
    for bad in (False, True):
        idx = _table(T, E, k, seed=T + E + k, bad=bad)
        ref = O.permute(idx, None, E, e_lo, e_hi, R_cap or None)
        off = ref["offsets"].astype(np.int32)
        idx_dev = torch.from_numpy(idx).cuda()
        want = _expected_bits(idx, E)
        assert want == ((RANGE | REPEAT) if bad else 0)
        # the table alone, then with the oracle's offsets: no offsets bit
        assert _check(s, idx_dev, None)[0] == want
        assert _check(s, idx_dev, torch.from_numpy(off).cuda())[0] == want
        # moe_permute's own offsets agree with the check too
        off_gpu = torch.empty(e_hi - e_lo + 1, dtype=torch.int32, device="cuda")
        perm = torch.empty(s.rows_cap, dtype=torch.int32, device="cuda")
        inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
        wsp = torch.empty(max(B.workspace_size(s, "permute"), 256), dtype=torch.uint8,
                          device="cuda")
        B.moe_permute(s, idx_dev, None, off_gpu, perm, inv, None, wsp)
        assert _check(s, idx_dev, off_gpu)[0] == want
        # corrupted offsets: one middle entry, the last entry, a nonzero start
        for i, delta in ((len(off) // 2, 1), (len(off) - 1, -1), (0, 1)):
            o2 = off.copy()
            o2[i] += delta
            assert _check(s, idx_dev, torch.from_numpy(o2).cuda())[0] == want | OFFSETS, (i, delta)
    if R_cap:
        # the unclamped prefix differs from what the permute writes
        raw = np.concatenate([[0], np.cumsum(ref["counts"])]).astype(np.int32)
        assert raw[-1] > R_cap
        assert _check(s, idx_dev, torch.from_numpy(raw).cuda())[0] == want | OFFSETS


def test_check_routing_router_output_and_sticky_bits():
    _announce("check_routing router output")
    T, d, E, k, I = 512, 128, 32, 4, 64
    s = B.MoEShape.make(T, d, E, k, I)
    g = torch.Generator().manual_seed(7)
    x = (torch.randn(T, d, generator=g) * 0.5).to(torch.bfloat16).cuda()
    wr = (torch.randn(d, E, generator=g) * 0.1).to(torch.bfloat16).cuda()
    logits = torch.empty(T, E, dtype=torch.float32, device="cuda")
    idx = torch.empty(T, k, dtype=torch.int32, device="cuda")
    w = torch.empty(T, k, dtype=torch.float32, device="cuda")
    B.moe_route(s, x, wr, None, logits, idx, w)
    off = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.empty(T * k, dtype=torch.int32, device="cuda")
    inv = torch.empty(T * k, dtype=torch.int32, device="cuda")
    wsp = torch.empty(max(B.workspace_size(s, "permute"), 256), dtype=torch.uint8, device="cuda")
    B.moe_permute(s, idx, None, off, perm, inv, None, wsp)
    bits, flags = _check(s, idx, off)
    assert bits == 0                       # the router's table is always clean
    # bits only accumulate: a bad table's bits stay after a clean check
    bad = idx.clone()
    bad[5, 2] = E
    assert _check(s, bad, None, flags)[0] == RANGE
    assert _check(s, idx, off, flags)[0] == RANGE
