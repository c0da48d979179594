"""lora_attn_decode_noalloc (the decode call for callers that cannot
allocate): through the C ABI, its output equals lora_attn_decode's on the
same inputs, bit for bit (same kernels, same launch plan) and so within the
bf16 parity bound, over two calls in a row whose second is smaller than the
first (the fixed array still holds the first call's records, none of which
the second may read)."""
import pytest
import torch

import shared_base_kv_amd as lra
from tests.gpu_harness import TOL_BF16, row_rel_err, run_decode, to_np, upload
from workloads import config_8b_decode, decode_workload

pytestmark = pytest.mark.gpu


def _noalloc(dw):
    w = dw.w
    out = torch.full(dw.q.shape, 7.0, dtype=dw.torch_dtype, device=dw.q.device)
    lra.lora_attn_decode_noalloc(dw.q, dw.k_base, dw.v_base, dw.block_tables, dw.context_lens, dw.max_context_len,
                                 dw.group_offsets, dw.agent_ids, dw.lk_ptrs, dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs,
                                 dw.ranks, dw.max_rank, w.n_agents, w.Hkv, w.sm_scale, w.theta, out,
                                 adapter_start=dw.adapter_start)
    torch.cuda.synchronize()
    return out


def test_noalloc_matches_decode_two_calls():
    cases = (config_8b_decode(),
             decode_workload(name="noalloc_small", group_sizes=(2, 1), context_lens=(700, 130), ranks=(16, 32, 8),
                             shared_l=False, theta=5e5, seed=4))
    for i, w in enumerate(cases):
        print(f"[case] noalloc call {i}: {w.name} S={w.S} T={[w.context_len(s) for s in range(w.S)]}", flush=True)
        dw = upload(w)
        got = _noalloc(dw)
        ref = run_decode(dw)
        assert torch.isfinite(got.float()).all(), i
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), i
        assert row_rel_err(to_np(got), to_np(ref)) <= TOL_BF16, i
