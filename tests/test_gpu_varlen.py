"""Decode rows and prefill chunks in one launch (lora_attn_varlen) on the GPU:
each row is bit-identical to what the separate decode and prefill calls
write for it (same split plan and query tiling), and within tolerance of the
fp64 oracle. Covers both adapters, one or none, separate low-rank pools with
activation positions and an agent-less sequence, higher ranks, a prefill-only
and a decode-only batch, and the 8B-shaped serving step (the 4-agent decode
on its 8192-token base plus the 4 x 512-token prefill chunk)."""
import numpy as np
import pytest
import torch

import shared_base_kv_amd as lra
from tests.gpu_harness import TOL_BF16, oracle_rows, row_rel_err, to_np
from workloads import config_mixed_step, mixed_workload
from workloads.device import upload

pytestmark = pytest.mark.gpu


def _n_groups(dw, S_dec):
    return dw.group_offsets.numel() - 1 if dw.group_offsets is not None else S_dec


def run_varlen(dw, S_dec, out=None):
    w = dw.w
    n = lra.lora_attn_varlen_workspace_size(w.S, S_dec, _n_groups(dw, S_dec), w.Hq, w.Hkv, w.d, dw.max_rank,
                                            dw.max_context_len, lra.LRA_BF16)
    ws = torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")
    out = dw.new_out() if out is None else out
    lra.lora_attn_varlen(dw.q, dw.k_base, dw.v_base, dw.block_tables, dw.context_lens, dw.max_context_len,
                         dw.cu_q_lens, dw.max_q_len, S_dec, dw.group_offsets, dw.agent_ids, dw.lk_ptrs, dw.lv_ptrs,
                         dw.bk_ptrs, dw.bv_ptrs, dw.ranks, dw.max_rank, w.n_agents, w.Hkv, w.sm_scale, w.theta, out, ws,
                         adapter_start=dw.adapter_start)
    torch.cuda.synchronize()
    return out


def run_separate(dw, S_dec):
    """The decode call on sequences 0 .. S_dec - 1 and the prefill call on the
    rest, with the same context and query-length bounds as the varlen call."""
    w = dw.w
    out = dw.new_out()
    cut = lambda t, lo, hi=None: None if t is None else t[lo:hi]  # noqa: E731
    if S_dec:
        n = lra.lora_attn_decode_workspace_size(S_dec, _n_groups(dw, S_dec), w.Hq, w.Hkv, w.d, dw.max_rank,
                                                dw.max_context_len, lra.LRA_BF16)
        ws = torch.zeros(max(n, 256), dtype=torch.uint8, device="cuda")
        od = torch.zeros_like(out[:S_dec])
        lra.lora_attn_decode(dw.q[:S_dec].contiguous(), dw.k_base, dw.v_base, dw.block_tables[:S_dec].contiguous(),
                             dw.context_lens[:S_dec].contiguous(), dw.max_context_len, dw.group_offsets,
                             cut(dw.agent_ids, 0, S_dec), dw.lk_ptrs, dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs, dw.ranks,
                             dw.max_rank, w.n_agents, w.Hkv, w.sm_scale, w.theta, od, ws,
                             adapter_start=cut(dw.adapter_start, 0, S_dec))
        out[:S_dec] = od
    if S_dec < w.S:
        cu = (dw.cu_q_lens[S_dec:] - S_dec).contiguous()
        op = torch.zeros_like(out[S_dec:])
        lra.lora_attn_prefill(dw.q[S_dec:].contiguous(), dw.k_base, dw.v_base, dw.block_tables[S_dec:].contiguous(),
                              dw.context_lens[S_dec:].contiguous(), dw.max_context_len, cu, dw.max_q_len,
                              cut(dw.agent_ids, S_dec), dw.lk_ptrs, dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs, dw.ranks,
                              dw.max_rank, w.n_agents, w.Hkv, w.sm_scale, w.theta, op,
                              adapter_start=cut(dw.adapter_start, S_dec))
        out[S_dec:] = op
    torch.cuda.synchronize()
    return out


def _check(w, S_dec, oracle=True, n_rows=12, seed=3):
    print(f"[case] varlen {w.name} S={w.S} S_dec={S_dec} adapt={w.adapt}", flush=True)
    dw = upload(w)
    got = run_varlen(dw, S_dec)
    sep = run_separate(dw, S_dec)
    assert torch.isfinite(got.float()).all()
    assert torch.equal(got, sep), "varlen rows differ from the separate calls' rows"
    if not oracle:
        return
    g = to_np(got)
    qo = w.q_offsets()
    rng = np.random.default_rng(seed)
    picks = {}
    for s in range(w.S):
        nq = qo[s + 1] - qo[s]
        picks[s] = sorted(set([0, nq - 1] + rng.choice(nq, min(nq, n_rows), replace=False).tolist()))
    for s, ref in enumerate(oracle_rows(w, range(w.S), picks)):
        err = row_rel_err(g[qo[s] + np.asarray(picks[s])], ref)
        assert err <= TOL_BF16, f"{w.name} seq {s}: max row-relative error {err:.3e}"


@pytest.mark.parametrize("adapt", ("kv", "v", "k", "none"))
def test_mixed_small(adapt):
    _check(mixed_workload(name="mixed", adapt=adapt, seed=11), S_dec=4)


def test_separate_pools_starts_and_agentless():
    w = mixed_workload(name="mixed_sep", Hq=16, Hkv=8, dec_group_sizes=(3, 2), dec_context_lens=(700, 257),
                       prefix=128, q_lens=(90, 17), ranks=(32, 32, 32), shared_l=False,
                       dec_agents=(0, 1, -1, 2, 0), pre_agents=(1, 2),
                       adapter_starts=(0, 300, 0, 100, 999, 64, 0), seed=12)
    _check(w, S_dec=5)


def test_rank64_two_groups():
    w = mixed_workload(name="mixed_r64", dec_group_sizes=(2, 2), dec_context_lens=(4097, 33), prefix=512,
                       q_lens=(65, 260), ranks=(64, 64), seed=13)
    _check(w, S_dec=4)


def test_prefill_only_and_decode_only():
    w = mixed_workload(name="mixed_pre_only", dec_group_sizes=(), dec_context_lens=(), prefix=256, q_lens=(40, 130),
                       seed=14)
    _check(w, S_dec=0)
    w = mixed_workload(name="mixed_dec_only", dec_group_sizes=(4,), dec_context_lens=(2000,), q_lens=(), seed=15)
    _check(w, S_dec=4)


def test_8b_serving_step():
    """The 8B-shaped serving step the benchmark times: bit-identical to the
    two separate calls; 12 sampled rows per sequence against the oracle."""
    _check(config_mixed_step(), S_dec=4, n_rows=10)
