"""Checks that pin the fp64 oracle to facts outside itself.

Each ``pin_*`` takes the oracle module and raises AssertionError on a
mismatch. They are run as tests against the real oracle
(test_oracle_pins.py) and against deliberately broken copies of it
(test_oracle_mutations.py), which must each fail at least one pin.

Kinds of pin used (the pages print no worked example or error bound):
closed forms worked by hand (tests/golden/hand_tiny.json), special cases
that reduce to a library routine (torch's scaled_dot_product_attention in
float64 on the CPU, numpy matmul), invariants of the mathematics (rotation
identities, causal truncation, linearity) and brute force on tiny inputs.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand_case(rng, T=9, Hq=4, Hkv=2, d=8, r=3, nq=1, scale_b=0.3):
    return dict(
        q=rng.standard_normal((nq, Hq, d)),
        kb=rng.standard_normal((T, Hkv, d)),
        vb=rng.standard_normal((T, Hkv, d)),
        lk=rng.standard_normal((T, r)),
        lv=rng.standard_normal((T, r)),
        bk=scale_b * rng.standard_normal((r, Hkv * d)),
        bv=scale_b * rng.standard_normal((r, Hkv * d)),
    )


# --------------------------------------------------------------- rotary pins
def pin_rope_d2_closed_form(o):
    """d=2 has one frequency, theta**0 = 1: the plain 2x2 rotation by n rad."""
    for theta in (10000.0, 5e5):
        for n in (0, 1, 3, 1000, 32767):
            y = o.rope_rotate(np.array([[1.0, 0.0]]), np.array([n]), theta)[0]
            assert np.allclose(y, [math.cos(n), math.sin(n)], atol=1e-12), (theta, n, y)
            y = o.rope_rotate(np.array([[0.0, 1.0]]), np.array([n]), theta)[0]
            assert np.allclose(y, [-math.sin(n), math.cos(n)], atol=1e-12), (theta, n, y)


def pin_rope_pairing_d4(o):
    """d=4, theta=100: pair 0 turns by n rad, pair 1 by n*100**(-1/2) = 0.1n rad;
    dimension i pairs with i + d/2."""
    n = 7
    y = o.rope_rotate(np.array([[0.0, 1.0, 0.0, 0.0]]), np.array([n]), 100.0)[0]
    assert np.allclose(y, [0.0, math.cos(0.1 * n), 0.0, math.sin(0.1 * n)], atol=1e-12), y
    y = o.rope_rotate(np.array([[0.0, 0.0, 1.0, 0.0]]), np.array([n]), 100.0)[0]
    assert np.allclose(y, [-math.sin(n), 0.0, math.cos(n), 0.0], atol=1e-12), y


def pin_rope_invariants(o):
    """Rotations: identity at 0, norm of each pair kept, relative-position
    property (R_m x).(R_n y) = x.(R_{n-m} y), identity when theta == 0."""
    rng = np.random.default_rng(1)
    d, theta = 16, 1e4
    x = rng.standard_normal((1, d))
    y = rng.standard_normal((1, d))
    assert np.allclose(o.rope_rotate(x, np.array([0]), theta), x, atol=1e-14)
    assert np.array_equal(o.rope_rotate(x, np.array([5]), 0.0), x)
    z = o.rope_rotate(x, np.array([123]), theta)
    pn = lambda v: v[0, : d // 2] ** 2 + v[0, d // 2 :] ** 2  # noqa: E731
    assert np.allclose(pn(z), pn(x), atol=1e-12)
    for m, n in ((3, 10), (100, 40), (0, 31000)):
        lhs = (o.rope_rotate(x, np.array([m]), theta) @ o.rope_rotate(y, np.array([n]), theta).T)[0, 0]
        rhs = (x @ o.rope_rotate(y, np.array([n - m]), theta).T)[0, 0]
        assert abs(lhs - rhs) < 1e-9, (m, n, lhs, rhs)


# ----------------------------------------------------------- attention pins
def _sdpa(q, K, V, positions, sm_scale):
    """torch's scaled_dot_product_attention in float64 on the CPU, with KV
    heads repeated G times and an explicit causal mask."""
    import torch

    nq, Hq, d = q.shape
    T, Hkv, _ = K.shape
    G = Hq // Hkv
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2)))  # [Hq, nq, d]
    kt = torch.from_numpy(np.ascontiguousarray(K.transpose(1, 0, 2))).repeat_interleave(G, dim=0)
    vt = torch.from_numpy(np.ascontiguousarray(V.transpose(1, 0, 2))).repeat_interleave(G, dim=0)
    mask = torch.from_numpy(np.arange(T)[None, :] <= np.asarray(positions)[:, None])
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=sm_scale)
    return out.numpy().transpose(1, 0, 2)


def pin_zero_adapter_is_sdpa(o):
    """B = 0 reduces to plain attention over the base cache: equals torch SDPA
    (fp64, CPU) for decode and for a causal prefill chunk, with GQA."""
    rng = np.random.default_rng(2)
    for nq, theta in ((1, 0.0), (1, 5e5), (5, 1e4)):
        c = _rand_case(rng, T=13, nq=nq)
        c["bk"][:] = 0.0
        c["bv"][:] = 0.0
        sc = 0.37
        got = o.lora_attention(**c, sm_scale=sc, theta=theta)
        pos = np.arange(13 - nq, 13)
        ref = _sdpa(c["q"], c["kb"], c["vb"], pos, sc)
        assert np.allclose(got, ref, atol=1e-12, rtol=0), np.abs(got - ref).max()


def pin_adapter_matches_sdpa_on_built_cache(o):
    """With rotary off, the cache is kb + lk bk and vb + lv bv (numpy matmul);
    attention over it equals SDPA. Pins the adapter's head slicing: B column
    h*d + i feeds KV head h, dimension i."""
    rng = np.random.default_rng(3)
    c = _rand_case(rng, T=11, Hq=6, Hkv=3, d=4, r=2, nq=3)
    T, Hkv, d = c["kb"].shape
    K = c["kb"] + (c["lk"] @ c["bk"]).reshape(T, Hkv, d)
    V = c["vb"] + (c["lv"] @ c["bv"]).reshape(T, Hkv, d)
    got = o.lora_attention(**c, sm_scale=0.5, theta=0.0)
    ref = _sdpa(c["q"], K, V, np.arange(T - 3, T), 0.5)
    assert np.allclose(got, ref, atol=1e-12, rtol=0), np.abs(got - ref).max()


def pin_absent_adapters_sdpa(o):
    """A projection without an adapter (B None) keeps its base cache: with no
    adapter at all the result is SDPA over (kb, vb); with only a value adapter
    it is SDPA over (kb, vb + lv bv), unaffected by the rotary base (rotary
    acts on the key adapter alone); with only a key adapter and rotary off it
    is SDPA over (kb + lk bk, vb)."""
    rng = np.random.default_rng(10)
    for nq in (1, 4):
        c = _rand_case(rng, T=12, Hq=6, Hkv=3, d=4, r=2, nq=nq)
        T, Hkv, d = c["kb"].shape
        pos = np.arange(T - nq, T)
        K_ad = c["kb"] + (c["lk"] @ c["bk"]).reshape(T, Hkv, d)
        V_ad = c["vb"] + (c["lv"] @ c["bv"]).reshape(T, Hkv, d)
        cases = (
            (dict(c, lk=None, lv=None, bk=None, bv=None), 5e5, c["kb"], c["vb"]),
            (dict(c, lk=None, bk=None), 5e5, c["kb"], V_ad),
            (dict(c, lv=None, bv=None), 0.0, K_ad, c["vb"]),
        )
        for args, theta, K, V in cases:
            got = o.lora_attention(**args, sm_scale=0.45, theta=theta)
            ref = _sdpa(c["q"], K, V, pos, 0.45)
            assert np.allclose(got, ref, atol=1e-12, rtol=0), (nq, theta, np.abs(got - ref).max())


def pin_adapter_start(o):
    """Activation position a: start 0 is the full adapter, start T is the base
    cache alone (SDPA over kb, vb), and in between the cache is kb, vb on
    rows n < a and kb + lk bk, vb + lv bv on rows n >= a (rotary off, SDPA);
    with rotary on, the rows from a on still carry their rotation at their
    own absolute position (equal to the full oracle there)."""
    rng = np.random.default_rng(12)
    c = _rand_case(rng, T=12, Hq=6, Hkv=3, d=4, r=2, nq=3)
    T, Hkv, d = c["kb"].shape
    pos = np.arange(T - 3, T)
    full = o.lora_attention(**c, sm_scale=0.5, theta=1e4)
    assert np.array_equal(o.lora_attention(**c, sm_scale=0.5, theta=1e4, adapter_start=0), full)
    base = o.lora_attention(**c, sm_scale=0.5, theta=1e4, adapter_start=T)
    assert np.allclose(base, _sdpa(c["q"], c["kb"], c["vb"], pos, 0.5), atol=1e-12, rtol=0)
    for a in (1, 5, 11):
        K = c["kb"].copy()
        V = c["vb"].copy()
        K[a:] += (c["lk"][a:] @ c["bk"]).reshape(-1, Hkv, d)
        V[a:] += (c["lv"][a:] @ c["bv"]).reshape(-1, Hkv, d)
        got = o.lora_attention(**c, sm_scale=0.5, theta=0.0, adapter_start=a)
        assert np.allclose(got, _sdpa(c["q"], K, V, pos, 0.5), atol=1e-12, rtol=0), a
        Kf, Vf = o.materialise_kv(c["kb"], c["vb"], c["lk"], c["lv"], c["bk"], c["bv"], 1e4)
        Ka, Va = o.materialise_kv(c["kb"], c["vb"], c["lk"], c["lv"], c["bk"], c["bv"], 1e4, a)
        assert np.array_equal(Ka[a:], Kf[a:]) and np.array_equal(Va[a:], Vf[a:])
        assert np.array_equal(Ka[:a], c["kb"][:a]) and np.array_equal(Va[:a], c["vb"][:a])


def pin_uniform_scores_mean(o):
    """q = 0 gives equal weights: out = mean_n V[n] = mean(vb) + mean(lv) bv."""
    rng = np.random.default_rng(4)
    c = _rand_case(rng, T=10)
    c["q"][:] = 0.0
    got = o.lora_attention(**c, sm_scale=1.0, theta=5e5)
    T, Hkv, d = c["kb"].shape
    meanv = c["vb"].mean(axis=0) + (c["lv"].mean(axis=0) @ c["bv"]).reshape(Hkv, d)
    G = c["q"].shape[1] // Hkv
    assert np.allclose(got[0], np.repeat(meanv, G, axis=0), atol=1e-13)


def pin_single_key(o):
    """T = 1: softmax over one key is 1, out = vb[0] + lv[0] bv for every head."""
    rng = np.random.default_rng(5)
    c = _rand_case(rng, T=1)
    got = o.lora_attention(**c, sm_scale=0.3, theta=5e5)
    Hkv, d = c["kb"].shape[1:]
    v0 = c["vb"][0] + (c["lv"][0] @ c["bv"]).reshape(Hkv, d)
    G = c["q"].shape[1] // Hkv
    assert np.allclose(got[0], np.repeat(v0, G, axis=0), atol=1e-14)


def pin_dominant_key(o):
    """A score far above the rest puts all weight on that key: the output is
    that key's full value row (its own adapter term included), not a neighbour's."""
    rng = np.random.default_rng(6)
    T, Hq, Hkv, d, r = 8, 2, 1, 4, 2
    c = _rand_case(rng, T=T, Hq=Hq, Hkv=Hkv, d=d, r=r)
    c["kb"][:] = 0.0
    c["lk"][:] = 0.0
    c["bk"][:] = 0.0
    star = 5
    c["kb"][star, 0, 0] = 1.0
    c["q"][:] = 0.0
    c["q"][0, :, 0] = 200.0
    got = o.lora_attention(**c, sm_scale=1.0, theta=0.0)
    vstar = c["vb"][star, 0] + c["lv"][star] @ c["bv"]
    assert np.allclose(got[0, 0], vstar, atol=1e-10), (got[0, 0], vstar)


def pin_prefill_rows_equal_truncated_decode(o):
    """Causality: prefill row i (position P + i) equals a decode step over the
    first P + i + 1 tokens."""
    rng = np.random.default_rng(7)
    c = _rand_case(rng, T=12, nq=4)
    full = o.lora_attention(**c, sm_scale=0.4, theta=1e4)
    for i in range(4):
        n = 12 - 4 + i + 1
        sub = {k: (v[:n] if k in ("kb", "vb", "lk", "lv") else v) for k, v in c.items()}
        sub["q"] = c["q"][i : i + 1]
        dec = o.lora_attention(**sub, sm_scale=0.4, theta=1e4)
        assert np.allclose(full[i], dec[0], atol=1e-13), i


def pin_hand_golden(o):
    """Closed forms worked by hand (tests/golden/hand_tiny.json)."""
    with open(os.path.join(GOLDEN, "hand_tiny.json")) as f:
        cases = json.load(f)["cases"]
    for cs in cases:
        arr = {k: np.array(cs[k], dtype=np.float64) for k in ("q", "kb", "vb", "lk", "lv", "bk", "bv")}
        got = o.lora_attention(**arr, sm_scale=1 / math.sqrt(2), theta=cs["theta"])
        assert np.allclose(got, np.array(cs["expected"]), atol=1e-12), (cs["name"], got)


def _brute(q, kb, vb, lk, lv, bk, bv, sm_scale, theta):
    """Scalar loops straight from the definition (tiny sizes only)."""
    nq, Hq, d = q.shape
    T, Hkv, _ = kb.shape
    r = lk.shape[1]
    G = Hq // Hkv
    half = d // 2
    K = [[[0.0] * d for _ in range(Hkv)] for _ in range(T)]
    V = [[[0.0] * d for _ in range(Hkv)] for _ in range(T)]
    for n in range(T):
        for h in range(Hkv):
            a = [sum(lk[n][k] * bk[k][h * d + i] for k in range(r)) for i in range(d)]
            av = [sum(lv[n][k] * bv[k][h * d + i] for k in range(r)) for i in range(d)]
            rot = list(a)
            if theta:
                for i in range(half):
                    w = n * theta ** (-2.0 * i / d)
                    rot[i] = a[i] * math.cos(w) - a[i + half] * math.sin(w)
                    rot[i + half] = a[i + half] * math.cos(w) + a[i] * math.sin(w)
            for i in range(d):
                K[n][h][i] = kb[n][h][i] + rot[i]
                V[n][h][i] = vb[n][h][i] + av[i]
    out = np.zeros((nq, Hq, d))
    for qi in range(nq):
        p = T - nq + qi
        for j in range(Hq):
            h = j // G
            s = [sm_scale * sum(q[qi][j][i] * K[n][h][i] for i in range(d)) for n in range(p + 1)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = sum(e)
            for i in range(d):
                out[qi][j][i] = sum(e[n] / z * V[n][h][i] for n in range(p + 1))
    return out


def pin_bruteforce_tiny(o):
    """Vectorised oracle equals scalar loops on tiny inputs (T<=8, d=4, r<=2;
    Hq=2 over one KV head, and Hq=4 over two KV heads, where B column h*d + i
    must feed head h), with and without rotary, decode and causal prefill."""
    rng = np.random.default_rng(8)
    for T, r, nq, theta, Hq, Hkv in ((1, 1, 1, 0.0, 2, 1), (5, 2, 1, 1e4, 2, 1), (8, 2, 3, 5e5, 2, 1),
                                     (7, 1, 7, 10.0, 2, 1), (6, 2, 2, 1e4, 4, 2), (5, 2, 1, 0.0, 4, 2),
                                     (4, 1, 4, 100.0, 2, 2)):
        c = _rand_case(rng, T=T, Hq=Hq, Hkv=Hkv, d=4, r=r, nq=nq, scale_b=1.0)
        got = o.lora_attention(**c, sm_scale=0.6, theta=theta)
        ref = _brute(**c, sm_scale=0.6, theta=theta)
        assert np.allclose(got, ref, atol=1e-12, rtol=0), (T, r, nq, theta, Hkv, np.abs(got - ref).max())


def _rot_complex(x, n, theta):
    """Rotary embedding of the rows x [T, d] at positions n [T], written as a
    complex product: pair (i, i + d/2) is the number x_i + j x_{i+d/2}, turned
    by exp(j n theta^(-2i/d)). Independent of the oracle's rotate-half code."""
    x = np.asarray(x, np.float64)
    if theta == 0:
        return x.copy()
    h = x.shape[-1] // 2
    z = x[:, :h] + 1j * x[:, h:]
    w = np.exp(1j * np.outer(np.asarray(n, np.float64), np.power(float(theta), -np.arange(h) / h)))
    zr = z * w
    return np.concatenate([zr.real, zr.imag], axis=-1)


def _reordered(c, sm_scale, theta, positions):
    """Attention in the reordered form, never building full-dimension adapter
    keys or values per head of the query: per query row j (KV head h) the
    score splits as q.K_base[n] + q.rope_n(L_k[n] B_k), and the output as
    P V_base + (P L_v) B_v, with the rank-space sum P L_v taken before B_v."""
    q, kb, vb, lk, lv, bk, bv = (np.asarray(c[k], np.float64) for k in ("q", "kb", "vb", "lk", "lv", "bk", "bv"))
    nq, Hq, d = q.shape
    T, Hkv, _ = kb.shape
    G = Hq // Hkv
    out = np.zeros((nq, Hq, d))
    for j in range(Hq):
        h = j // G
        bk_h, bv_h = bk[:, h * d:(h + 1) * d], bv[:, h * d:(h + 1) * d]
        ad_key = _rot_complex(lk @ bk_h, np.arange(T), theta)  # [T, d]
        for i in range(nq):
            p = int(positions[i])
            s = sm_scale * (kb[: p + 1, h] @ q[i, j] + ad_key[: p + 1] @ q[i, j])
            e = np.exp(s - s.max())
            P = e / e.sum()
            out[i, j] = P @ vb[: p + 1, h] + (P @ lv[: p + 1]) @ bv_h
    return out


def pin_reorder_equals_materialised(o):
    """The reordered form P V_base + (P L_v) B_v, with scores q.K_base +
    q.rope(L_k B_k) (LRAgent abstract: attention reordered so the low-rank
    cache is never expanded), equals attention over the materialised K, V, for
    decode and causal prefill rows, GQA with two KV heads, rotary on and off."""
    rng = np.random.default_rng(13)
    for nq, theta, r in ((1, 0.0, 3), (1, 5e5, 2), (4, 1e4, 3), (2, 10.0, 1)):
        c = _rand_case(rng, T=10, Hq=4, Hkv=2, d=8, r=r, nq=nq, scale_b=0.7)
        pos = np.arange(10 - nq, 10)
        ref = _reordered(c, 0.45, theta, pos)
        K, V = o.materialise_kv(c["kb"], c["vb"], c["lk"], c["lv"], c["bk"], c["bv"], theta)
        got = o.attend(np.asarray(c["q"], np.float64), pos, K, V, 0.45)
        assert np.allclose(got, ref, atol=1e-12, rtol=0), (nq, theta, np.abs(got - ref).max())
        full = o.lora_attention(**c, sm_scale=0.45, theta=theta)
        assert np.allclose(full, ref, atol=1e-12, rtol=0), (nq, theta, np.abs(full - ref).max())


def pin_shared_base_unchanged(o):
    """Several agents over one base cache (LRAgent abstract: the base component
    is shared; PReCache abstract): each agent's result over the shared base
    arrays equals its result over a private copy of the base, exactly, in
    either order of the agents, with one shared low-rank cache or one per
    agent; the shared base arrays are left as they were."""
    rng = np.random.default_rng(14)
    T, Hq, Hkv, d, r = 11, 4, 2, 8, 3
    kb = rng.standard_normal((T, Hkv, d))
    vb = rng.standard_normal((T, Hkv, d))
    kb0, vb0 = kb.copy(), vb.copy()
    lk_sh, lv_sh = rng.standard_normal((T, r)), rng.standard_normal((T, r))
    agents = []
    for a in range(3):
        own = a % 2 == 1
        agents.append(dict(q=rng.standard_normal((2, Hq, d)),
                           lk=rng.standard_normal((T, r)) if own else lk_sh,
                           lv=rng.standard_normal((T, r)) if own else lv_sh,
                           bk=0.5 * rng.standard_normal((r, Hkv * d)), bv=0.5 * rng.standard_normal((r, Hkv * d))))
    private = [o.lora_attention(kb=kb0.copy(), vb=vb0.copy(), **ag, sm_scale=0.4, theta=1e4) for ag in agents]
    for order in ((0, 1, 2), (2, 1, 0)):
        for a in order:
            got = o.lora_attention(kb=kb, vb=vb, **agents[a], sm_scale=0.4, theta=1e4)
            assert np.array_equal(got, private[a]), (order, a)
        assert np.array_equal(kb, kb0) and np.array_equal(vb, vb0), order


# --------------------------------------------------------- cache-build pins
def pin_lr_cache_build(o):
    """L = X A: equals numpy matmul, scalar loops on a tiny case, and X when A = I."""
    rng = np.random.default_rng(9)
    X = rng.standard_normal((5, 7))
    A = rng.standard_normal((7, 3))
    L = o.lr_cache_build(X, A)
    ref = [[sum(X[i][k] * A[k][c] for k in range(7)) for c in range(3)] for i in range(5)]
    assert np.allclose(L, ref, atol=1e-13)
    assert np.array_equal(o.lr_cache_build(X, np.eye(7)), X)


def pin_lr_cache_build_multi(o):
    """Groups of uneven width each equal X times their own slice of A, by
    scalar loops, and together cover every column once."""
    rng = np.random.default_rng(11)
    X = rng.standard_normal((4, 6))
    A = rng.standard_normal((6, 7))
    cols = [0, 2, 3, 7]
    parts = o.lr_cache_build_multi(X, A, cols)
    assert len(parts) == 3
    for g, P in enumerate(parts):
        c0, c1 = cols[g], cols[g + 1]
        assert P.shape == (4, c1 - c0)
        ref = [[sum(X[i][k] * A[k][c] for k in range(6)) for c in range(c0, c1)] for i in range(4)]
        assert np.allclose(P, ref, atol=1e-13), g


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
