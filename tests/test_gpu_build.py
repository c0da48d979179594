"""lr_cache_build parity: L = X A on the GPU against the fp64 oracle, and the
paged stores (token-major and rank-major through a slot mapping) bit-exact
against the dense result."""
import numpy as np
import pytest
import torch

import oracle
import shared_base_kv_amd as lra
from tests.gpu_harness import TOL_BF16, row_rel_err
from workloads import bf16_bits, build_inputs

pytestmark = pytest.mark.gpu


def _dev_bf16(x):
    return torch.from_numpy(bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()


def _build(X, A, ws=None, **kw):
    n, hidden = X.shape
    ncols = A.shape[1]
    if ws is None:
        ws = torch.zeros(max(lra.lr_cache_build_workspace_size(n, hidden, ncols), 16), dtype=torch.uint8,
                         device="cuda")
    L = kw.pop("L", None)
    if L is None:
        L = torch.full((n, ncols), float("nan"), dtype=torch.bfloat16, device="cuda")
    lra.lr_cache_build(_dev_bf16(X), _dev_bf16(A), L, ws, **kw)
    torch.cuda.synchronize()
    return L


# hidden past 4096 takes several staging rounds (8200: three, the last 8 wide); 20 columns give
# lda % 8 != 0 (the element-wise staging path); 40 columns end in a partial column tile
@pytest.mark.parametrize("shape", [(512, 4096, 16), (512, 4096, 32), (1, 4096, 16), (37, 520, 8), (300, 2048, 200),
                                   (70, 8200, 20), (33, 5000, 40)])
def test_build_matches_oracle(shape):
    n, hidden, ncols = shape
    X, A = build_inputs(n, hidden, ncols, seed=n + ncols)
    L = _build(X, A).float().cpu().numpy()
    ref = oracle.lr_cache_build(X, A)
    assert row_rel_err(L, ref) <= TOL_BF16
    # diagnostic bound: one fp32 sum + one rounding keeps nearly all elements at
    # RNE(fp64), except values on a bf16 rounding midpoint to within fp32
    # precision, which the summation order decides either way
    rne = torch.from_numpy(ref).float().to(torch.bfloat16).float().numpy()
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    off_mid = np.abs(np.abs(ref - rne) - ulp / 2) > 1e-3 * ulp
    rate = float((L == rne)[off_mid].mean())
    print(f"[rne] {shape}: {rate:.4f} of off-midpoint elements equal RNE(fp64)", flush=True)
    assert rate >= 0.99


def test_build_paged_stores_bit_exact():
    n, hidden, r = 70, 1024, 16
    X, A = build_inputs(n, hidden, r, seed=2)
    dense = _build(X, A)
    nb = 12
    rng = np.random.default_rng(0)
    slots = rng.permutation(nb * 16)[:n].astype(np.int64)
    slots[5] = -1  # skipped row
    sm = torch.from_numpy(slots).cuda()
    tok = torch.zeros((nb, 16, r), dtype=torch.bfloat16, device="cuda")
    _build(X, A, L=tok, slot_mapping=sm, l_layout=lra.LRA_L_TOKEN_MAJOR, ldl=r)
    rk = torch.zeros((nb, r, 16), dtype=torch.bfloat16, device="cuda")
    _build(X, A, L=rk, slot_mapping=sm, l_layout=lra.LRA_L_RANK_MAJOR)
    ch = torch.zeros((nb, r // 8, 16, 8), dtype=torch.bfloat16, device="cuda")
    _build(X, A, L=ch, slot_mapping=sm, l_layout=lra.LRA_L_KEY_CHUNKED)
    d = dense.view(torch.int16).cpu().numpy()
    t = tok.view(torch.int16).cpu().numpy().reshape(nb * 16, r)
    k = rk.view(torch.int16).cpu().numpy().transpose(0, 2, 1).reshape(nb * 16, r)
    # key-chunked: rank j of slot s at block s/16, ((j/8)*16 + s%16)*8 + j%8
    c = ch.view(torch.int16).cpu().numpy().transpose(0, 2, 1, 3).reshape(nb * 16, r)
    for i, s in enumerate(slots):
        if s < 0:
            continue
        assert np.array_equal(t[s], d[i]) and np.array_equal(k[s], d[i]) and np.array_equal(c[s], d[i])
    written = set(int(s) for s in slots if s >= 0)
    untouched = [s for s in range(nb * 16) if s not in written]
    assert not t[untouched].any() and not k[untouched].any() and not c[untouched].any()


def _multi_case(n, hidden, ranks, seed):
    """X, the side-by-side A of every (agent, k/v) group, group columns and layouts."""
    widths = [r for r in ranks for _ in (0, 1)]  # agent a: A_k then A_v
    cols = np.concatenate([[0], np.cumsum(widths)]).astype(np.int32).tolist()
    X, A = build_inputs(n, hidden, cols[-1], seed=seed)
    lays = [lra.LRA_L_KEY_CHUNKED, lra.LRA_L_RANK_MAJOR] * len(ranks)
    return X, A, cols, lays, widths


@pytest.mark.parametrize("shape", [(512, 4096, (16, 16, 16, 16)), (300, 2048, (16, 8, 32, 64, 8)), (5, 520, (8,))])
def test_multi_build_equals_single_builds_bit_exact(shape):
    """Every group's pool rows from one multi-group build are bit-identical to
    a separate lr_cache_build of that group's columns, and within the bf16
    bound of the oracle's X A_g; skipped and unwritten slots stay untouched."""
    n, hidden, ranks = shape
    X, A, cols, lays, widths = _multi_case(n, hidden, ranks, seed=n + hidden)
    nb = -(-n // 16) + 3
    rng = np.random.default_rng(1)
    slots = rng.permutation(nb * 16)[:n].astype(np.int64)
    if n > 3:
        slots[3] = -1
    sm = torch.from_numpy(slots).cuda()
    Xd, Ad = _dev_bf16(X), _dev_bf16(A)

    def pools():
        return [torch.zeros((nb, w // 8, 16, 8) if lay == lra.LRA_L_KEY_CHUNKED else (nb, w, 16),
                            dtype=torch.bfloat16, device="cuda") for w, lay in zip(widths, lays)]

    multi = pools()
    ws = torch.zeros(lra.lr_cache_build_workspace_size(n, hidden, cols[-1]), dtype=torch.uint8, device="cuda")
    lra.lr_cache_build_multi(Xd, Ad, cols, multi, lays, sm, ws)
    single = pools()
    for g, (w, lay) in enumerate(zip(widths, lays)):
        wsg = torch.zeros(lra.lr_cache_build_workspace_size(n, hidden, w), dtype=torch.uint8, device="cuda")
        lra.lr_cache_build(Xd, Ad[:, cols[g]:cols[g + 1]], single[g], wsg, slot_mapping=sm, l_layout=lay, ldl=w,
                           n_cols=w)
    torch.cuda.synchronize()
    refs = oracle.lr_cache_build_multi(X, A, cols)
    for g, (w, lay) in enumerate(zip(widths, lays)):
        m = multi[g].view(torch.int16).cpu().numpy()
        assert np.array_equal(m, single[g].view(torch.int16).cpu().numpy()), g

        def rows_of(x):
            if lay == lra.LRA_L_KEY_CHUNKED:
                return x.transpose(0, 2, 1, 3).reshape(nb * 16, w)
            return x.transpose(0, 2, 1).reshape(nb * 16, w)

        rows = rows_of(m)
        got = rows_of(multi[g].float().cpu().numpy())
        keep = slots >= 0
        assert row_rel_err(got[slots[keep]], refs[g][keep]) <= TOL_BF16, g
        untouched = sorted(set(range(nb * 16)) - set(int(s) for s in slots[keep]))
        assert not rows[untouched].any(), g


def test_build_reuses_workspace_across_calls():
    """Twelve builds in a row, of changing data and sizes, on one workspace
    (zero-filled once): every result matches the oracle and is bit-identical
    to the same build on a freshly zero-filled workspace, and the tile
    counters are back at zero after each call (no slice reads another call's
    partial sums or counts)."""
    big = lra.lr_cache_build_workspace_size(512, 4096, 64)
    ws = torch.zeros(big, dtype=torch.uint8, device="cuda")
    shapes = [(512, 4096, 16), (300, 2048, 64), (17, 4096, 8), (512, 4096, 64), (64, 1032, 40), (1, 4096, 16)] * 2
    for i, (n, hidden, ncols) in enumerate(shapes):
        X, A = build_inputs(n, hidden, ncols, seed=1000 + i)
        print(f"[case] build {i}: n={n} hidden={hidden} cols={ncols}", flush=True)
        L = _build(X, A, ws=ws)
        fresh = _build(X, A)
        assert torch.equal(L.view(torch.int16), fresh.view(torch.int16)), i
        assert row_rel_err(L.float().cpu().numpy(), oracle.lr_cache_build(X, A)) <= TOL_BF16, i
        assert not ws[:4096].any(), i
