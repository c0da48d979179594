"""The seeded generator: bf16 rounding and the paged scatter it hands to the
library (gathering pools back through the block tables must give the
logical rows the oracle reads)."""
import numpy as np
import torch

from workloads import BLOCK, bf16_bits, decode_workload, prefill_workload, round_bf16
from workloads.synth import _bits_rne


def test_round_bf16_matches_torch_rne():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-20, 20, 100000),
                        np.array([0.0, -0.0, 1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, np.inf, -np.inf], np.float32)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    got = round_bf16(x)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    assert np.array_equal(bf16_bits(got), torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))
    fin = np.isfinite(x)
    assert np.array_equal(_bits_rne(x[fin].copy()), bf16_bits(got[fin]))


def _gather_check(w, poison):
    kpool, vpool, lkp, lvp = w.host_pools(poison=poison)
    bt = w.block_tables()
    to32 = (lambda b: (b.astype(np.uint32) << 16).view(np.float32)) if w.dtype == "bf16" else (lambda b: b)
    for s in range(w.S):
        lg = w.logical(s)
        T = w.context_len(s)
        nblk = -(-T // BLOCK)
        ids = bt[s, :nblk]
        k = to32(kpool[ids]).transpose(0, 2, 1, 3).reshape(nblk * BLOCK, w.Hkv, w.d)[:T]
        v = to32(vpool[ids]).transpose(0, 3, 1, 2).reshape(nblk * BLOCK, w.Hkv, w.d)[:T]
        p = w.pool_of_agent[w.seqs[s].agent]
        lk = to32(lkp[p][ids]).transpose(0, 2, 1, 3).reshape(nblk * BLOCK, -1)[:T]
        lv = to32(lvp[p][ids]).transpose(0, 2, 1).reshape(nblk * BLOCK, -1)[:T]
        assert np.array_equal(k, lg["kb"]) and np.array_equal(v, lg["vb"])
        assert np.array_equal(lk, lg["lk"]) and np.array_equal(lv, lg["lv"])
        if poison and T % BLOCK:
            assert np.isnan(to32(kpool[ids[-1]])[:, T % BLOCK :, :]).all()


def test_paged_scatter_roundtrip_decode():
    w = decode_workload(Hq=8, Hkv=2, d=16, group_sizes=(3, 1, 2), context_lens=(37, 16, 5),
                        ranks=(8, 16, 8, 32), shared_l=False, agent_of_seq=[0, 1, 2, 3, 1, 0], spare_blocks=3)
    _gather_check(w, poison=False)
    _gather_check(w, poison=True)


def test_paged_scatter_roundtrip_prefill_and_f32():
    w = prefill_workload(Hq=4, Hkv=2, d=8, prefix=32, q_lens=(5, 17), rank=8)
    _gather_check(w, poison=True)
    w = decode_workload(dtype="f32", Hq=4, Hkv=4, d=8, group_sizes=(2,), context_lens=(20,), ranks=(8, 8),
                        shared_l=False, shuffle=False, theta=0.0)
    _gather_check(w, poison=False)


def test_group_members_share_base_rows():
    w = decode_workload(Hq=8, Hkv=2, d=16, group_sizes=(3,), context_lens=(40,), ranks=(16,) * 3)
    a, b = w.logical(0), w.logical(2)
    assert np.array_equal(a["kb"], b["kb"]) and np.array_equal(a["lk"], b["lk"])
    assert not np.array_equal(a["bk"], b["bk"])
