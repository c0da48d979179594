"""Activation positions on the GPU against the fp64 oracle: tokens before a
sequence's adapter_start keep the base key and value (an activated adapter
acts from its invocation point on). Covers starts at 0, inside a cache block,
on block and split edges, past the context, different starts in one row
tile, shared and separate low-rank pools, the fp32 decode and the prefill
chunk; plus exact equalities with the paths that have no adapter at all."""
import numpy as np
import pytest
import torch

from tests.gpu_harness import (TOL_BF16, TOL_F32, oracle_rows, row_rel_err, run_decode, run_prefill, to_np,
                               upload)
from workloads import config_8b_decode, config_prefill, decode_workload, prefill_workload

pytestmark = pytest.mark.gpu


def _check_decode(w, tol):
    print(f"[case] decode {w.name} starts={[sq.adapter_start for sq in w.seqs]}", flush=True)
    got = to_np(run_decode(upload(w)))
    ref = np.concatenate(oracle_rows(w, range(w.S)))
    assert np.isfinite(got).all()
    err = row_rel_err(got, ref)
    assert err <= tol, f"{w.name}: max row-relative error {err:.3e} > {tol}"
    return got


def test_8b_decode_full_size_mixed_starts():
    """The 8B-shaped decode (T=8192, 4 agents on one base) with the four
    agents activated at 0, mid-context, near the end and never."""
    w = config_8b_decode()
    for sq, st in zip(w.seqs, (0, 4100, 8000, 8192)):
        sq.adapter_start = st
    _check_decode(w, TOL_BF16)


SMALL = [
    # (Hq, Hkv, group_sizes, context_lens, ranks, shared_l, starts)
    (32, 8, (4,), (700,), (16,) * 4, True, (0, 5, 16, 699)),
    (32, 8, (4,), (700,), (16,) * 4, True, (300, 300, 300, 300)),
    (32, 8, (4,), (40,), (16,) * 4, True, (1000, 17, 39, 40)),
    (16, 8, (8,), (300,), (32,) * 8, False, (0, 31, 32, 33, 64, 200, 299, 500)),
    (64, 8, (3,), (260,), (64,) * 3, False, (100, 0, 259)),
    (32, 8, (1,) * 4, (31, 257, 1500, 4097), (8, 16, 32, 64), False, (7, 256, 1024, 4000)),
    (32, 4, (2, 3), (5000, 17), (16,) * 5, True, (2048, 4095, 16, 0, 9)),
]


@pytest.mark.parametrize("mode", ("kv", "v", "k"))
@pytest.mark.parametrize("case", SMALL, ids=[f"c{i}" for i in range(len(SMALL))])
def test_small_decode(case, mode):
    Hq, Hkv, gs, tl, ranks, shared, starts = case
    w = decode_workload(name="act", Hq=Hq, Hkv=Hkv, group_sizes=gs, context_lens=tl, ranks=ranks, shared_l=shared,
                        theta=5e5, seed=41, adapt=mode, adapter_starts=starts)
    _check_decode(w, TOL_BF16)


def test_agentless_and_starts_together():
    w = decode_workload(name="act_mixed", group_sizes=(4,), context_lens=(900,), agent_of_seq=(-1, 0, 1, 2),
                        ranks=(16,) * 3, shared_l=True, seed=43, adapter_starts=(0, 450, 0, 899))
    _check_decode(w, TOL_BF16)


@pytest.mark.parametrize("theta", (5e5, 0.0))  # 0: the adapter score as L_k . (B_k q), no rebuilt key
def test_f32_decode(theta):
    w = decode_workload(name="act_f32", dtype="f32", Hq=8, Hkv=4, d=64, theta=theta, group_sizes=(3,),
                        context_lens=(150,), ranks=(8,) * 3, shared_l=False, seed=5, adapter_starts=(0, 70, 64))
    _check_decode(w, TOL_F32)


def test_start_zero_and_start_past_context_bit_exact():
    """Starts of 0 give the same bits as no start array; starts at or past
    every context give the same bits as a call without adapters."""
    kw = dict(name="act_eq", group_sizes=(4,), context_lens=(1500,), ranks=(16,) * 4, shared_l=True, seed=7)
    plain = to_np(run_decode(upload(decode_workload(**kw))))
    dw = upload(decode_workload(**kw))
    dw.adapter_start = torch.zeros(4, dtype=torch.int32, device="cuda")
    assert np.array_equal(to_np(run_decode(dw)), plain)
    none = to_np(run_decode(upload(decode_workload(adapt="none", **kw))))
    late = to_np(run_decode(upload(decode_workload(adapter_starts=(1500, 1500, 9999, 1 << 30), **kw))))
    assert np.array_equal(late, none)


def _check_prefill(w, q_rows=None):
    print(f"[case] prefill {w.name} starts={[sq.adapter_start for sq in w.seqs]}", flush=True)
    got = to_np(run_prefill(upload(w)))
    qo = w.q_offsets()
    assert np.isfinite(got).all()
    for s, ref in enumerate(oracle_rows(w, range(w.S), q_rows)):
        rows = np.arange(qo[s + 1] - qo[s]) if q_rows is None else np.asarray(q_rows[s])
        err = row_rel_err(got[qo[s] + rows], ref)
        assert err <= TOL_BF16, f"{w.name} seq {s}: max row-relative error {err:.3e}"


PREFILL = [
    # (prefix, q_lens, rank, starts)
    (128, (64, 65, 3), 32, (0, 100, 191)),
    (256, (200, 31, 9), 16, (256, 64, 300)),
    (64, (90,), 64, (70,)),
    (0, (17, 40), 16, (10, 100)),
]


@pytest.mark.parametrize("mode", ("kv", "v", "k"))
@pytest.mark.parametrize("case", PREFILL, ids=[f"p{i}" for i in range(len(PREFILL))])
def test_small_prefill(case, mode):
    prefix, q_lens, rank, starts = case
    w = prefill_workload(name="act_prefill", prefix=prefix, q_lens=q_lens, rank=rank, theta=5e5, seed=29, adapt=mode,
                         adapter_starts=starts)
    _check_prefill(w)


def test_prefill_chunk_full_size_activated_at_the_chunk():
    """The full prefill chunk with each agent's adapter activated where its
    own 512 tokens begin (the shared 8192-token prefix keeps the base cache),
    and one agent activated mid-chunk; 24 sampled rows per agent."""
    w = config_prefill()
    for sq, st in zip(w.seqs, (8192, 8192, 8192 + 200, 4000)):
        sq.adapter_start = st
    rng = np.random.default_rng(6)
    picks = {s: sorted(set([0, 199, 200, 201, 511] + rng.choice(512, 19, replace=False).tolist())) for s in range(w.S)}
    _check_prefill(w, q_rows=picks)
