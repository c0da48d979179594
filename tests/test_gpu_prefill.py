"""Prefill parity: the HIP prefill kernel (through the C ABI) against the fp64
oracle on the same seeded inputs, including the pipeline in which the
low-rank rows of the new tokens come from lr_cache_build on the GPU while
the oracle computes them as X A in fp64."""
import numpy as np
import pytest
import torch

import oracle
import shared_base_kv_amd as lra
from tests.gpu_harness import TOL_BF16, oracle_rows, row_rel_err, run_prefill, to_np, upload
from workloads import BLOCK, bf16_bits, build_inputs, config_prefill, config_prefill_r64, prefill_workload

pytestmark = pytest.mark.gpu


def _check(w, q_rows=None, poison=False):
    dw = upload(w, poison=poison)
    got = to_np(run_prefill(dw))
    qo = w.q_offsets()
    assert np.isfinite(got).all()
    seqs = list(range(w.S))
    refs = oracle_rows(w, seqs, q_rows)
    for s, ref in zip(seqs, refs):
        rows = np.arange(qo[s + 1] - qo[s]) if q_rows is None else np.asarray(q_rows[s])
        err = row_rel_err(got[qo[s] + rows], ref)
        assert err <= TOL_BF16, f"{w.name} seq {s}: max row-relative error {err:.3e}"
    return got


def test_prefill_chunk_full_size_sampled_rows():
    """4 agents x 512 new tokens after the shared 8192-token prefix, all rows
    computed on the GPU; the oracle checks 40 rows per agent (first, last,
    tile edges and a seeded sample)."""
    w = config_prefill()
    rng = np.random.default_rng(3)
    picks = {}
    for s in range(w.S):
        base = [0, 1, 31, 32, 33, 255, 256, 510, 511]
        picks[s] = sorted(set(base + rng.choice(512, 31, replace=False).tolist()))
    _check(w, q_rows=picks)


def test_prefill_chunk_rank64_full_size_sampled_rows():
    """The same chunk at rank 64, where the kernel rebuilds the values in LDS
    instead of accumulating P L_v; 20 rows per agent."""
    w = config_prefill_r64()
    rng = np.random.default_rng(4)
    picks = {}
    for s in range(w.S):
        base = [0, 63, 64, 255, 256, 511]
        picks[s] = sorted(set(base + rng.choice(512, 14, replace=False).tolist()))
    _check(w, q_rows=picks)


SMALL = [
    # (Hq, Hkv, prefix, q_lens, rank, theta)
    (32, 8, 0, (1,), 16, 5e5),
    (32, 8, 0, (17, 40), 16, 5e5),
    (32, 8, 16, (1, 15, 33), 16, 1e4),
    (32, 8, 64, (100,), 16, 0.0),
    (32, 8, 128, (64, 65, 3), 32, 5e5),
    (32, 8, 32, (70,), 64, 5e5),
    (32, 8, 48, (50, 9), 8, 5e5),
    (8, 8, 32, (300,), 16, 5e5),    # G=1: 256 tokens per tile, two tiles
    (16, 8, 16, (90,), 16, 5e5),    # G=2
    (64, 8, 16, (40,), 16, 5e5),    # G=8
    (128, 8, 16, (20,), 16, 5e5),   # G=16
    (32, 4, 256, (200, 31), 16, 5e5),
]


@pytest.mark.parametrize("case", SMALL, ids=[f"c{i}" for i in range(len(SMALL))])
def test_small_prefill_variants(case):
    Hq, Hkv, prefix, q_lens, rank, theta = case
    w = prefill_workload(name="small_prefill", Hq=Hq, Hkv=Hkv, prefix=prefix, q_lens=q_lens, rank=rank,
                         theta=theta, seed=21)
    _check(w)


def test_prefill_poison_unreachable_memory_is_ignored():
    w = prefill_workload(name="poison_prefill", prefix=32, q_lens=(21, 7), rank=16, spare_blocks=5, seed=8)
    clean = to_np(run_prefill(upload(w, poison=False)))
    dirty = to_np(run_prefill(upload(w, poison=True)))
    assert np.isfinite(dirty).all()
    assert np.array_equal(clean, dirty)


def test_prefill_matches_decode_rows():
    """Prefill row i equals a decode step at T = prefix + i + 1 (causality on
    the GPU, across the two kernels, within tolerance)."""
    from tests.gpu_harness import run_decode
    from workloads.device import upload as up

    w = prefill_workload(name="pd", prefix=48, q_lens=(37,), rank=16, seed=30)
    dw = up(w)
    pre = to_np(run_prefill(dw))
    for i in (0, 5, 17, 36):
        # decode over the first 48 + i + 1 tokens of the same pools with query row i
        dd = up(w)
        dd.q = dw.q[i : i + 1].contiguous()
        dd.context_lens = torch.tensor([48 + i + 1], dtype=torch.int32, device="cuda")
        dd.group_offsets = None
        dd.max_context_len = 48 + i + 1
        dec = to_np(run_decode(dd))
        assert row_rel_err(dec[0], pre[i]) < 1e-2


def test_build_then_prefill_pipeline():
    """The low-rank rows of each agent's new tokens are produced on the GPU by
    lr_cache_build (X_a A_k into the key-chunked L_k pool, X_a A_v into the
    rank-major L_v pool) and then read by the prefill kernel. The oracle runs
    the same pipeline in fp64 with L = X_a A unrounded."""
    w = prefill_workload(name="pipe", prefix=64, q_lens=(48, 29), rank=16, seed=40)
    dw = upload(w)
    hidden = 512
    Xs = [build_inputs(w.seqs[a].q_len, hidden, 16, seed=50 + a)[0] for a in range(w.S)]
    Ak = build_inputs(1, hidden, 16, seed=60, sigma_a=1.0 / np.sqrt(hidden))[1]
    Av = build_inputs(1, hidden, 16, seed=61, sigma_a=1.0 / np.sqrt(hidden))[1]
    dev = lambda x: torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    for a in range(w.S):
        seg = w.segments[1 + a]
        slots = (seg.blocks.astype(np.int64)[:, None] * BLOCK + np.arange(BLOCK)[None, :]).reshape(-1)[: seg.T]
        sm = torch.from_numpy(slots).cuda()
        ws = torch.zeros(lra.lr_cache_build_workspace_size(seg.T, hidden, 16), dtype=torch.uint8, device="cuda")
        lra.lr_cache_build(dev(Xs[a]), dev(Ak), dw.lk_pools[0], ws, slot_mapping=sm, l_layout=lra.LRA_L_KEY_CHUNKED,
                           ldl=16)
        lra.lr_cache_build(dev(Xs[a]), dev(Av), dw.lv_pools[0], ws, slot_mapping=sm, l_layout=lra.LRA_L_RANK_MAJOR)
    got = to_np(run_prefill(dw))
    qo = w.q_offsets()
    for a in range(w.S):
        lg = w.logical(a)
        n = w.seqs[a].q_len
        lg["lk"][-n:] = oracle.lr_cache_build(Xs[a], Ak)
        lg["lv"][-n:] = oracle.lr_cache_build(Xs[a], Av)
        ref = oracle.lora_attention(**lg, sm_scale=w.sm_scale, theta=w.theta)
        assert row_rel_err(got[qo[a] : qo[a + 1]], ref) <= TOL_BF16
