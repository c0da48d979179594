"""liblra_debug.so: the kernels of liblra.so behind device-side input checks.
Valid calls give results bit-identical to liblra.so; each kind of bad
device-side input is reported as LRA_ERR_INVALID_ARG before any attention
kernel runs, so the output buffer keeps its sentinel value. The bad inputs
never reach an attention kernel: the check kernel reads every table only at
indices it has bounded."""
import pytest
import torch

import shared_base_kv_amd as lra
from shared_base_kv_amd import binding as B
from tests.gpu_harness import run_decode, run_prefill, upload
from tests.test_gpu_varlen import run_varlen
from workloads import decode_workload, mixed_workload, prefill_workload

pytestmark = pytest.mark.gpu

SENTINEL = 7.0


@pytest.fixture
def use_debug(monkeypatch):
    """Route the binding's wrappers through liblra_debug.so for one test."""
    B.load()

    def switch():
        monkeypatch.setattr(B, "_lib", B.load_debug())

    return switch


def _decode_w():
    # two groups of two sequences sharing a base each, four agents
    return decode_workload(name="dbg", Hq=32, Hkv=8, group_sizes=(2, 2), context_lens=(300, 700),
                           ranks=(16,) * 4, shared_l=False, theta=5e5, seed=5)


def test_valid_calls_match_release(use_debug):
    dw = upload(_decode_w())
    pw = upload(prefill_workload(name="dbgp", prefix=256, q_lens=(100, 37), rank=16, seed=6))
    mw = upload(mixed_workload(name="dbgm", seed=7))
    ref = (run_decode(dw), run_prefill(pw), run_varlen(mw, 4))
    use_debug()
    got = (run_decode(dw), run_prefill(pw), run_varlen(mw, 4))
    for r, g, name in zip(ref, got, ("decode", "prefill", "varlen")):
        print(f"[case] debug library, valid {name}", flush=True)
        assert torch.equal(r, g), name


def _bad_decode(dw, fragment):
    out = torch.full(dw.q.shape, SENTINEL, dtype=dw.torch_dtype, device="cuda")
    with pytest.raises(lra.LraError) as e:
        run_decode(dw, out=out)
    assert e.value.code == B.LRA_ERR_INVALID_ARG
    assert fragment in str(e.value), str(e.value)
    assert bool((out == SENTINEL).all()), "an attention kernel ran on bad input"


def _set(t, idx, value):
    t[idx] = value
    torch.cuda.synchronize()


DECODE_CASES = {
    "context_too_long": ("context length", lambda dw: _set(dw.context_lens, 3, dw.max_context_len + 1)),
    "context_zero": ("context length", lambda dw: _set(dw.context_lens, 2, 0)),
    "negative_block": ("negative physical block id", lambda dw: _set(dw.block_tables, (3, 5), -1)),
    "agent_id": ("agent id", lambda dw: _set(dw.agent_ids, 1, 4)),
    "agent_below": ("agent id", lambda dw: _set(dw.agent_ids, 1, -2)),
    "rank": ("agent rank", lambda dw: _set(dw.ranks, 2, 17)),
    "rank_not_multiple_of_8": ("agent rank", lambda dw: _set(dw.ranks, 2, 12)),
    "null_pool": ("null low-rank pool", lambda dw: _set(dw.lk_ptrs, 0, 0)),
    "group_offsets": ("group_offsets", lambda dw: _set(dw.group_offsets, 1, 0)),
    "group_context": ("differ in context length", lambda dw: _set(dw.context_lens, 1, 299)),
    "group_blocks": ("block-table row", lambda dw: _set(dw.block_tables, (1, 2), int(dw.block_tables[1, 2]) + 1)),
}


@pytest.mark.parametrize("case", sorted(DECODE_CASES))
def test_bad_decode_input_is_reported(use_debug, case):
    fragment, spoil = DECODE_CASES[case]
    print(f"[case] debug library, decode with {case}", flush=True)
    dw = upload(_decode_w())
    spoil(dw)
    use_debug()
    _bad_decode(dw, fragment)


def test_negative_adapter_start_is_reported(use_debug):
    dw = upload(_decode_w())
    dw.adapter_start = torch.zeros(dw.w.S, dtype=torch.int32, device="cuda")
    _set(dw.adapter_start, 0, -5)
    use_debug()
    _bad_decode(dw, "adapter_start")


def test_bad_prefill_query_count_is_reported(use_debug):
    print("[case] debug library, prefill with a query count above its context", flush=True)
    pw = upload(prefill_workload(name="dbgp", prefix=0, q_lens=(64, 64), rank=16, seed=8))
    # chunk 0 claims 96 queries on a 64-token context (chunk 1 keeps 32)
    _set(pw.cu_q_lens, 1, 96)
    use_debug()
    out = torch.full(pw.q.shape, SENTINEL, dtype=pw.torch_dtype, device="cuda")
    with pytest.raises(lra.LraError) as e:
        run_prefill(pw, out=out)
    assert e.value.code == B.LRA_ERR_INVALID_ARG and "query count" in str(e.value)
    assert bool((out == SENTINEL).all())


def test_varlen_decode_rows_are_checked(use_debug):
    """Decode sequence s of a varlen call owns query row s: cu_q_lens[s] must
    equal s up to s = S_dec (else prefill rows would overlap decode rows)."""
    print("[case] debug library, varlen with a decode row offset moved", flush=True)
    mw = upload(mixed_workload(name="dbgm", seed=9))
    _set(mw.cu_q_lens, 2, 3)
    use_debug()
    out = torch.full(mw.q.shape, SENTINEL, dtype=mw.torch_dtype, device="cuda")
    with pytest.raises(lra.LraError) as e:
        run_varlen(mw, 4, out=out)
    assert e.value.code == B.LRA_ERR_INVALID_ARG
    assert "decode part" in str(e.value) and "cu_q_lens" in str(e.value), str(e.value)
    assert bool((out == SENTINEL).all())


def test_bad_varlen_input_is_reported(use_debug):
    print("[case] debug library, varlen with a bad agent id in the prefill part", flush=True)
    mw = upload(mixed_workload(name="dbgm", seed=9))
    _set(mw.agent_ids, mw.w.S - 1, 99)
    use_debug()
    with pytest.raises(lra.LraError) as e:
        run_varlen(mw, 4)
    assert e.value.code == B.LRA_ERR_INVALID_ARG
    assert "prefill part" in str(e.value) and "agent id" in str(e.value)


def test_build_workspace_counters_checked(use_debug):
    """The cache build's tile counters must be zero on entry (the workspace is
    zero-filled before first use); the debug library reports a nonzero one
    before the build runs, leaving L untouched."""
    import numpy as np

    from workloads import bf16_bits, build_inputs

    print("[case] debug library, cache build with a nonzero tile counter", flush=True)
    X, A = build_inputs(64, 1024, 16, seed=3)
    dev = lambda x: torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()  # noqa: E731
    ws = torch.zeros(lra.lr_cache_build_workspace_size(64, 1024, 16), dtype=torch.uint8, device="cuda")
    ws[8:12] = 1  # counter 2
    L = torch.full((64, 16), SENTINEL, dtype=torch.bfloat16, device="cuda")
    use_debug()
    with pytest.raises(lra.LraError) as e:
        lra.lr_cache_build(dev(X), dev(A), L, ws)
        torch.cuda.synchronize()
    assert e.value.code == B.LRA_ERR_WORKSPACE and "counter 2" in str(e.value), str(e.value)
    assert bool((L == SENTINEL).all())
