"""Adapter-absent paths on the GPU against the fp64 oracle: calls without a
key adapter (b_k NULL: adapters on q and v only), without a value adapter,
without any adapter, and batches in which some sequences have no agent
(id -1). Plus exact equalities: an absent adapter gives the same bits as a
zero one, and an agent-less sequence in a mixed batch the same bits as in a
call without adapters."""
import numpy as np
import pytest
import torch

from tests.gpu_harness import (TOL_BF16, TOL_F32, oracle_rows, row_rel_err, run_decode, run_prefill, to_np,
                               upload)
from workloads import config_8b_decode, decode_workload, prefill_workload

pytestmark = pytest.mark.gpu

MODES = ("v", "k", "none")


def _check_decode(w, tol):
    print(f"[case] decode {w.name} adapt={w.adapt} S={w.S}", flush=True)
    got = to_np(run_decode(upload(w)))
    ref = np.concatenate(oracle_rows(w, range(w.S)))
    assert np.isfinite(got).all()
    err = row_rel_err(got, ref)
    assert err <= tol, f"{w.name}/{w.adapt}: max row-relative error {err:.3e} > {tol}"
    return got


@pytest.mark.parametrize("mode", MODES)
def test_8b_decode_full_size(mode):
    """The 8B-shaped decode (T=8192, 4 agents on one base, shared-A r=16) with
    the given adapters, all four sequences against the oracle."""
    w = config_8b_decode()
    w.adapt = mode
    _check_decode(w, TOL_BF16)


SMALL = [
    # (Hq, Hkv, group_sizes, context_lens, ranks, shared_l)
    (32, 8, (4,), (1,), (16,) * 4, True),
    (32, 8, (4,), (700,), (16,) * 4, True),
    (16, 8, (8,), (300,), (32,) * 8, False),  # G=2, 8 agents per tile
    (64, 8, (3,), (260,), (64,) * 3, False),  # 2 row tiles at r=64
    (32, 8, (1,) * 4, (31, 257, 1500, 4097), (8, 16, 32, 64), False),  # mixed ranks, splits
    (32, 4, (2, 3), (5000, 17), (16,) * 5, True),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("case", SMALL, ids=[f"c{i}" for i in range(len(SMALL))])
def test_small_decode(case, mode):
    Hq, Hkv, gs, tl, ranks, shared = case
    w = decode_workload(name="absent", Hq=Hq, Hkv=Hkv, group_sizes=gs, context_lens=tl, ranks=ranks,
                        shared_l=shared, theta=5e5, seed=31, adapt=mode)
    _check_decode(w, TOL_BF16)


@pytest.mark.parametrize("theta", (5e5, 0.0))  # 0: the adapter score as L_k . (B_k q), no rebuilt key
@pytest.mark.parametrize("mode", MODES)
def test_f32_decode(mode, theta):
    w = decode_workload(name="absent_f32", dtype="f32", Hq=8, Hkv=4, d=64, theta=theta, group_sizes=(3,),
                        context_lens=(100,), ranks=(8,) * 3, shared_l=False, seed=3, adapt=mode)
    _check_decode(w, TOL_F32)


AGENTLESS = [
    # (group_sizes, context_lens, agent_of_seq, ranks, shared_l)
    ((4,), (900,), (-1, 0, 1, 2), (16,) * 3, True),        # lead is slot 1
    ((4,), (900,), (-1, 0, -1, 1), (16, 32), False),       # separate pools, slot 0 agentless
    ((4,), (333,), (-1, -1, -1, -1), (16,), True),         # a tile with no adapter at all
    ((2, 3), (40, 2100), (0, -1, -1, 1, 2), (16, 16, 16), True),
    ((1,) * 4, (64, 17, 3000, 5), (-1, 2, -1, 0), (8, 64, 16), False),
]


@pytest.mark.parametrize("mode", ("kv", "v"))
@pytest.mark.parametrize("case", AGENTLESS, ids=[f"a{i}" for i in range(len(AGENTLESS))])
def test_agentless_sequences_in_decode(case, mode):
    gs, tl, agents, ranks, shared = case
    w = decode_workload(name="agentless", group_sizes=gs, context_lens=tl, agent_of_seq=agents, ranks=ranks,
                        shared_l=shared, seed=17, adapt=mode)
    _check_decode(w, TOL_BF16)


@pytest.mark.parametrize("theta", (5e5, 0.0))
def test_agentless_f32_decode(theta):
    w = decode_workload(name="agentless_f32", dtype="f32", Hq=8, Hkv=4, d=64, theta=theta, group_sizes=(3,),
                        context_lens=(70,), agent_of_seq=(1, -1, 0), ranks=(8, 8), shared_l=False, seed=4)
    _check_decode(w, TOL_F32)


def test_absent_adapter_equals_zero_adapter_bit_exact():
    """b_k = b_v = NULL gives the same bits as zero B matrices at the same
    launch plan (the adapter products add exact zeros), and so does b_k =
    NULL against a zero B_k with B_v kept."""
    kw = dict(name="zero", group_sizes=(4,), context_lens=(1500,), ranks=(16,) * 4, shared_l=True, seed=6)
    full = upload(decode_workload(**kw))
    for b in full.bk:
        b.zero_()
    zero_k = to_np(run_decode(full))
    for b in full.bv:
        b.zero_()
    zero_kv = to_np(run_decode(full))
    dw = upload(decode_workload(adapt="v", **kw))
    assert np.array_equal(to_np(run_decode(dw)), zero_k)
    dw = upload(decode_workload(adapt="none", **kw))  # max_rank 0 plans as rank 16
    assert np.array_equal(to_np(run_decode(dw)), zero_kv)


def test_agentless_row_matches_call_without_adapters_bit_exact():
    """An agent-less sequence batched with adapted ones gets the same bits as
    in a call without any adapter (max_rank 0 plans as 16: same launch)."""
    kw = dict(name="mixed", group_sizes=(4,), context_lens=(2000,), ranks=(16,) * 3, shared_l=True, seed=8)
    mixed = to_np(run_decode(upload(decode_workload(agent_of_seq=(0, -1, 1, 2), **kw))))
    dw = upload(decode_workload(agent_of_seq=(0, -1, 1, 2), adapt="none", **kw))  # plans as rank 16
    plain = to_np(run_decode(dw))
    assert np.array_equal(mixed[1], plain[1])


def _check_prefill(w, q_rows=None):
    print(f"[case] prefill {w.name} adapt={w.adapt} S={w.S}", flush=True)
    got = to_np(run_prefill(upload(w)))
    qo = w.q_offsets()
    assert np.isfinite(got).all()
    refs = oracle_rows(w, range(w.S), q_rows)
    for s, ref in enumerate(refs):
        rows = np.arange(qo[s + 1] - qo[s]) if q_rows is None else np.asarray(q_rows[s])
        err = row_rel_err(got[qo[s] + rows], ref)
        assert err <= TOL_BF16, f"{w.name}/{w.adapt} seq {s}: max row-relative error {err:.3e}"


PREFILL = [
    # (Hq, Hkv, prefix, q_lens, rank, agents)
    (32, 8, 0, (17, 40), 16, None),
    (32, 8, 128, (64, 65, 3), 32, None),
    (32, 8, 32, (70,), 64, None),
    (16, 8, 16, (90, 5), 16, (1, -1)),
    (32, 8, 256, (200, 31, 9), 16, (-1, 0, 2)),
    (32, 8, 48, (70, 33), 64, (-1, 1)),  # rank 64: values rebuilt in the kernel, one sequence agent-less
]


@pytest.mark.parametrize("mode", ("kv",) + MODES)
@pytest.mark.parametrize("case", PREFILL, ids=[f"p{i}" for i in range(len(PREFILL))])
def test_small_prefill(case, mode):
    Hq, Hkv, prefix, q_lens, rank, agents = case
    if mode == "kv" and agents is None:
        pytest.skip("covered by the prefill parity tests")
    w = prefill_workload(name="absent_prefill", Hq=Hq, Hkv=Hkv, prefix=prefix, q_lens=q_lens, rank=rank,
                         theta=5e5, seed=23, adapt=mode, agents=agents)
    _check_prefill(w)


@pytest.mark.parametrize("mode", ("v", "none"))
def test_prefill_chunk_full_size_sampled_rows(mode):
    """The full prefill chunk (4 x 512 tokens after the 8192-token prefix)
    without key adapters / without adapters; 24 sampled rows per agent."""
    from workloads import config_prefill

    w = config_prefill()
    w.adapt = mode
    rng = np.random.default_rng(5)
    picks = {s: sorted(set([0, 63, 64, 511] + rng.choice(512, 20, replace=False).tolist())) for s in range(w.S)}
    _check_prefill(w, q_rows=picks)


def test_prefill_absent_equals_zero_bit_exact():
    kw = dict(name="pzero", prefix=64, q_lens=(50, 33), rank=16, seed=9)
    full = upload(prefill_workload(**kw))
    for b in full.bk + full.bv:
        b.zero_()
    zero = to_np(run_prefill(full))
    dw = upload(prefill_workload(adapt="none", **kw))
    assert np.array_equal(to_np(run_prefill(dw)), zero)
    torch.cuda.synchronize()
