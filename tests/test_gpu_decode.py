"""Decode parity: the HIP path (through the C ABI) against the fp64 oracle,
element by element on the same seeded inputs, plus metamorphic equalities
that must hold bit for bit (gathers, routing, masking)."""
import numpy as np
import pytest
import torch

from tests.gpu_harness import (TOL_BF16, TOL_F32, oracle_rows, row_rel_err, run_decode, to_np, upload)
from workloads import config_8b_decode, config_long_layer, config_serving_mix, config_tiny_f32, decode_workload

pytestmark = pytest.mark.gpu


def _check(w, tol, seqs=None, poison=False):
    dw = upload(w, poison=poison)
    got = to_np(run_decode(dw))
    seqs = list(range(w.S)) if seqs is None else seqs
    ref = np.concatenate(oracle_rows(w, seqs))
    err = row_rel_err(got[seqs], ref)
    assert np.isfinite(got).all()
    assert err <= tol, f"{w.name}: max row-relative error {err:.3e} > {tol}"
    return dw, got, err


def test_tiny_f32_decode():
    _check(config_tiny_f32(), TOL_F32)


def test_8b_decode_shared_base():
    _check(config_8b_decode(), TOL_BF16)


SMALL = [
    # (Hq, Hkv, group_sizes, context_lens, ranks, shared_l, theta)
    (32, 8, (4,), (1,), (16,) * 4, True, 5e5),
    (32, 8, (4,), (15,), (16,) * 4, True, 5e5),
    (32, 8, (4,), (17,), (16,) * 4, True, 5e5),
    (32, 8, (4,), (33,), (16,) * 4, True, 0.0),
    (32, 8, (4,), (1000,), (16,) * 4, True, 5e5),
    (32, 8, (2, 1, 3), (129, 16, 700), (16,) * 6, True, 1e4),
    (16, 8, (8,), (300,), (32,) * 8, False, 5e5),  # G=2, 8 agents/tile
    (8, 8, (5,), (77,), (8,) * 5, False, 5e5),  # G=1
    (8, 8, (12,), (300,), (16,) * 12, False, 5e5),  # G=1, 12 agents: row tiles of 8 and 4 over one base
    (32, 8, (3,), (400,), (16, 32, 8), False, 5e5),  # separate pools of different ranks in one tile
    (64, 8, (3,), (260,), (64,) * 3, False, 5e5),  # G=8: 2 agents per tile -> 2 row tiles
    (128, 8, (2,), (200,), (16, 16), False, 5e5),  # G=16: 1 agent per tile
    (32, 8, (6,), (513,), (64,) * 6, False, 5e5),  # 2 row tiles at r=64
    (32, 8, (1,) * 5, (31, 64, 257, 1500, 4097), (8, 16, 32, 64, 8), False, 5e5),  # mixed ranks
    (32, 4, (4,), (5000,), (16,) * 4, True, 5e5),
    (32, 8, (4,), (700,), (64,) * 4, True, 5e5),  # one shared pool at r=64: its rows in slot 0, the rest empty
    (32, 8, (4,), (301,), (32,) * 4, True, 0.0),  # the same at r=32, no rotary
    # several groups with 8 or more splits: splits dealt over the XCDs by
    # (group + split), group and split counts padded to multiples of 8
    (16, 4, (1, 2, 1), (6000, 2500, 4200), (16, 32, 16, 8), False, 5e5),  # 3 groups, 12 splits of 512
    (4, 4, (10, 1), (5000, 3000), (16,) * 11, False, 5e5),  # 2 groups, 2 row tiles, 10 splits of 512
    (4, 1, (2,), (16000,), (16, 16), True, 5e5),  # one KV head: 63 splits of 256 (the 64-split combine)
    (260, 260, (1,), (40,), (16,), True, 5e5),  # more than 255 KV heads (their count takes 16 bits of a packed argument)
]


@pytest.mark.parametrize("case", SMALL, ids=[f"c{i}" for i in range(len(SMALL))])
def test_small_decode_variants(case):
    Hq, Hkv, gs, tl, ranks, shared, theta = case
    w = decode_workload(name="small", Hq=Hq, Hkv=Hkv, group_sizes=gs, context_lens=tl, ranks=ranks,
                        shared_l=shared, theta=theta, seed=11)
    _check(w, TOL_BF16)


def test_tiny_f32_variants():
    for theta, gs, tl, d in ((5e5, (3,), (100,), 64), (0.0, (1, 2), (16, 65), 64), (1e4, (2,), (1,), 64),
                             (5e5, (2, 1), (130, 47), 128)):
        w = decode_workload(name="f32v", dtype="f32", Hq=8, Hkv=4, d=d, theta=theta, group_sizes=gs,
                            context_lens=tl, ranks=(8,) * sum(gs), shared_l=False, seed=3)
        _check(w, TOL_F32)


def test_poison_unreachable_memory_is_ignored():
    """NaN in spare blocks, in slots past each context end and in pool rows no
    agent reads leaves every output bit-identical and finite."""
    w = decode_workload(name="poison", group_sizes=(3, 1), context_lens=(70, 33), ranks=(16, 32, 8, 64),
                        shared_l=False, spare_blocks=7, seed=5)
    clean = to_np(run_decode(upload(w, poison=False)))
    dirty = to_np(run_decode(upload(w, poison=True)))
    assert np.isfinite(dirty).all()
    assert np.array_equal(clean, dirty)


def test_paged_shuffle_and_determinism_bit_exact():
    """Shuffled physical blocks give the same bits as contiguous ones (the
    gather is exact and the arithmetic order depends on token positions
    only); two runs give identical bits."""
    kw = dict(name="meta", group_sizes=(4, 2), context_lens=(3000, 517), ranks=(16,) * 6, shared_l=True, seed=9)
    a = to_np(run_decode(upload(decode_workload(shuffle=True, **kw))))
    b = to_np(run_decode(upload(decode_workload(shuffle=False, **kw))))
    assert np.array_equal(a, b)
    dw = upload(decode_workload(shuffle=True, **kw))
    assert np.array_equal(to_np(run_decode(dw)), to_np(run_decode(dw)))


def test_grouped_equals_ungrouped_within_tolerance_and_routing():
    """A group sharing one base gives the same result as the same sequences
    each in their own group (split sizes differ, so within tolerance), and
    swapping two agents' adapters swaps their output rows exactly."""
    kw = dict(name="grp", context_lens=(900,), ranks=(16,) * 4, shared_l=True, seed=4)
    w = decode_workload(group_sizes=(4,), **kw)
    dw = upload(w)
    g = to_np(run_decode(dw))
    dw.group_offsets = None
    u = to_np(run_decode(dw))
    assert row_rel_err(u, g) < 1e-2
    dw = upload(w)
    base = to_np(run_decode(dw))
    perm = torch.tensor([1, 0, 2, 3], device="cuda")
    dw.bk_ptrs = dw.bk_ptrs[perm].contiguous()
    dw.bv_ptrs = dw.bv_ptrs[perm].contiguous()
    dw.agent_ids = torch.tensor([1, 0, 2, 3], dtype=torch.int32, device="cuda")
    sw = to_np(run_decode(dw))
    assert np.array_equal(sw, base)


def test_long_context_layer_full_size():
    """One layer of the 32-layer long-context workload (T=32768, 8 agents,
    per-agent r=64), all 8 sequences against the oracle."""
    _check(config_long_layer(0), TOL_BF16)


def test_serving_mix_full_size_sampled():
    """The 64-request serving mix runs whole on the GPU; the oracle checks a
    seeded sample of 8 requests (including the longest and shortest)."""
    w = config_serving_mix()
    lens = np.array([w.context_len(s) for s in range(w.S)])
    rng = np.random.default_rng(1)
    pick = sorted(set([int(lens.argmax()), int(lens.argmin())] + rng.choice(w.S, 6, replace=False).tolist()))
    _check(w, TOL_BF16, seqs=pick)


def test_workspace_contents_do_not_matter():
    """Split records are fully rewritten by each call: a workspace full of NaN
    bytes, or one left over from a call with other shapes, gives the same bits
    as a zeroed one. Groups of different lengths make some rows finish in the
    main kernel while others are combined."""
    from tests.gpu_harness import decode_workspace

    w = decode_workload(name="ws", group_sizes=(2, 1, 3), context_lens=(700, 16, 2500), ranks=(16,) * 6,
                        shared_l=True, seed=12)
    dw = upload(w)
    ws = decode_workspace(dw)
    ref = to_np(run_decode(dw, workspace=ws))
    ws.fill_(0xFF)  # every float is NaN
    assert np.array_equal(to_np(run_decode(dw, workspace=ws)), ref)
    other = upload(decode_workload(name="ws2", group_sizes=(4,), context_lens=(5000,), ranks=(16,) * 4, seed=13))
    n = max(decode_workspace(other).numel(), ws.numel())
    big = torch.zeros(n, dtype=torch.uint8, device="cuda")
    run_decode(other, workspace=big)
    assert np.array_equal(to_np(run_decode(dw, workspace=big)), ref)
