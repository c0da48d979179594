"""Seeded synthetic inputs for shared-base + low-rank KV attention.

This module serves both the fp64 oracle (logical, unpaged arrays) and the GPU
library (paged pools, block tables, pointer tables). It holds draws and data
layout only: normal draws, round-to-nearest-even to bf16, and the scatter of
logical token rows into paged pools. No attention, rotation or product of
the method is computed here.

Draw recipe (everything from ``numpy.random.default_rng`` children of one
``SeedSequence(seed)``, spawned in this fixed order):

1. queries ``q``                         ~ N(0, 1)
2. one child per agent: ``B_k`` then ``B_v``  ~ N(0, 0.1 / sqrt(r_a))  (sigma)
3. one child per segment: base ``K`` then base ``V`` ~ N(0, 1), then for each
   low-rank pool the segment writes (in pool order) ``L_k`` then ``L_v`` ~ N(0, 1)
4. the layout child: a permutation of the physical block ids (or identity)

Draws are float32; for bf16 workloads each value is rounded to nearest-even
bf16 once, and the oracle reads exactly the rounded value.

Layouts handed to the library (block size 16):
- ``k_base``  [NB, Hkv, 16, d]   token rows of one (block, head) contiguous
- ``v_base``  [NB, Hkv, d, 16]   the 16 tokens of one (block, head, dim) contiguous
- ``L_k`` pool [NB, r/8, 16, 8]  chunks of 8 ranks (rank j of slot t at ((j/8)*16 + t)*8 + j%8)
- ``L_v`` pool [NB, r, 16]       rank-major (16 tokens of one rank contiguous)
- ``B_k``, ``B_v`` per agent [r, Hkv*d], column h*d + i
"""
from __future__ import annotations

import concurrent.futures as cf
import math
import os
from dataclasses import dataclass, field

import numpy as np

BLOCK = 16


def round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the round-to-nearest-even bf16 value."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    out = ((u + r) & np.uint32(0xFFFF0000)).view(np.float32)
    nan = np.isnan(x)
    if nan.any():
        out = out.copy()
        out[nan] = np.nan
    return out


def bf16_bits(x_rounded: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    return (np.ascontiguousarray(x_rounded, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bits_rne(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (round to nearest even) of finite float32 draws, in place."""
    u = x.view(np.uint32)
    t = u >> 16
    t &= 1
    t += np.uint32(0x7FFF)
    t += u
    t >>= 16
    return t.astype(np.uint16)


def _normal(rng: np.random.Generator, shape, sigma: float, dtype: str, bits: bool = False) -> np.ndarray:
    """N(0, sigma) draws as float32; bf16 workloads round once to bf16.
    With ``bits`` a bf16 draw is returned as its uint16 bit pattern."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    if dtype != "bf16":
        return x
    b = _bits_rne(x)
    if bits:
        return b
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Segment:
    """A run of tokens with its own base K/V rows and low-rank rows per pool."""

    T: int
    pools: tuple  # pool ids this segment writes rows for
    seed: np.random.SeedSequence = None
    blocks: np.ndarray = None  # physical block ids (filled by the layout step)


@dataclass
class SeqSpec:
    segments: tuple  # segment ids, in token order
    agent: int
    q_len: int = 1  # decode: 1; prefill: number of new query tokens
    adapter_start: int = 0  # first token position that carries the adapter terms


@dataclass
class Workload:
    name: str
    dtype: str  # "f32" | "bf16"
    Hq: int
    Hkv: int
    d: int
    theta: float  # 0 => no rotary embedding on the adapter term
    ranks: list  # rank per agent
    pool_of_agent: list  # low-rank pool id read by each agent
    pool_rank: list  # rank per pool
    segments: list
    seqs: list
    group_offsets: list = None  # decode grouping, or None
    seed: int = 0
    shuffle: bool = True
    spare_blocks: int = 0  # unused physical blocks (poison targets)
    prefill: bool = False
    sm_scale: float = None
    # projections that carry an adapter: "kv" (both), "v" (value only: no key
    # adapter), "k" (key only) or "none". A sequence whose agent is -1 has no
    # adapter in any case. Draws do not depend on this field.
    adapt: str = "kv"
    _cache: dict = field(default_factory=dict, repr=False)

    # ------------------------------------------------------------------ draws
    def __post_init__(self):
        if self.sm_scale is None:
            self.sm_scale = 1.0 / math.sqrt(self.d)
        for sq in self.seqs:
            for sid in sq.segments[:-1]:
                assert self.segments[sid].T % BLOCK == 0, "only a sequence's last segment may end mid-block"
        root = np.random.SeedSequence(self.seed)
        n_children = 1 + len(self.ranks) + len(self.segments) + 1
        ch = root.spawn(n_children)
        self._q_seed = ch[0]
        self._b_seeds = ch[1 : 1 + len(self.ranks)]
        for i, seg in enumerate(self.segments):
            seg.seed = ch[1 + len(self.ranks) + i]
        self._layout_seed = ch[-1]
        nb = sum(-(-seg.T // BLOCK) for seg in self.segments)
        self.num_blocks = nb + self.spare_blocks
        lay = np.random.default_rng(self._layout_seed)
        perm = lay.permutation(self.num_blocks) if self.shuffle else np.arange(self.num_blocks)
        pos = 0
        for seg in self.segments:
            n = -(-seg.T // BLOCK)
            seg.blocks = perm[pos : pos + n].astype(np.int32)
            pos += n
        self.spare = perm[pos:].astype(np.int32)

    @property
    def S(self) -> int:
        return len(self.seqs)

    @property
    def n_agents(self) -> int:
        return len(self.ranks)

    def context_len(self, s: int) -> int:
        return sum(self.segments[i].T for i in self.seqs[s].segments)

    def q_all(self) -> np.ndarray:
        if "q" not in self._cache:
            nq = sum(sq.q_len for sq in self.seqs)
            rng = np.random.default_rng(self._q_seed)
            self._cache["q"] = _normal(rng, (nq, self.Hq, self.d), 1.0, self.dtype)
        return self._cache["q"]

    def adapter(self, a: int):
        """(B_k, B_v) of agent a, each [r_a, Hkv*d]."""
        key = ("B", a)
        if key not in self._cache:
            r = self.ranks[a]
            rng = np.random.default_rng(self._b_seeds[a])
            sig = 0.1 / math.sqrt(r)
            bk = _normal(rng, (r, self.Hkv * self.d), sig, self.dtype)
            bv = _normal(rng, (r, self.Hkv * self.d), sig, self.dtype)
            self._cache[key] = (bk, bv)
        return self._cache[key]

    def segment_data(self, sid: int, bits: bool = False):
        """Logical rows of one segment: kb, vb [T, Hkv, d]; lk, lv: {pool: [T, r]}.
        With ``bits`` (bf16 only) the arrays hold uint16 bit patterns."""
        seg = self.segments[sid]
        rng = np.random.default_rng(seg.seed)
        kb = _normal(rng, (seg.T, self.Hkv, self.d), 1.0, self.dtype, bits)
        vb = _normal(rng, (seg.T, self.Hkv, self.d), 1.0, self.dtype, bits)
        lk, lv = {}, {}
        for p in seg.pools:
            lk[p] = _normal(rng, (seg.T, self.pool_rank[p]), 1.0, self.dtype, bits)
            lv[p] = _normal(rng, (seg.T, self.pool_rank[p]), 1.0, self.dtype, bits)
        return kb, vb, lk, lv

    def q_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum([sq.q_len for sq in self.seqs])]).astype(np.int32)

    @property
    def has_k(self) -> bool:
        return "k" in self.adapt

    @property
    def has_v(self) -> bool:
        return "v" in self.adapt

    def logical(self, s: int) -> dict:
        """Unpaged float64 arrays of sequence s, as the oracle consumes them
        (None for the low-rank rows and B of a projection without an adapter)."""
        sq = self.seqs[s]
        parts = [self.segment_data(i) for i in sq.segments]
        kb = np.concatenate([p[0] for p in parts]).astype(np.float64)
        vb = np.concatenate([p[1] for p in parts]).astype(np.float64)
        qo = self.q_offsets()
        q = self.q_all()[qo[s] : qo[s + 1]].astype(np.float64)
        out = dict(q=q, kb=kb, vb=vb, lk=None, lv=None, bk=None, bv=None, adapter_start=sq.adapter_start)
        if sq.agent >= 0:
            pool = self.pool_of_agent[sq.agent]
            bk, bv = self.adapter(sq.agent)
            if self.has_k:
                out["lk"] = np.concatenate([p[2][pool] for p in parts]).astype(np.float64)
                out["bk"] = bk.astype(np.float64)
            if self.has_v:
                out["lv"] = np.concatenate([p[3][pool] for p in parts]).astype(np.float64)
                out["bv"] = bv.astype(np.float64)
        return out

    # ----------------------------------------------------------------- layout
    def block_tables(self) -> np.ndarray:
        rows = [np.concatenate([self.segments[i].blocks for i in sq.segments]) for sq in self.seqs]
        mb = max(len(r) for r in rows)
        bt = np.zeros((self.S, mb), dtype=np.int32)
        for s, r in enumerate(rows):
            bt[s, : len(r)] = r
        return bt

    def host_pools(self, poison: bool = False):
        """Paged pools as numpy arrays in the library's storage type.

        bf16 pools are uint16 bit patterns. Unwritten storage (spare blocks,
        slots past a segment's end, pool rows no agent writes) is NaN when
        ``poison`` is set, zero otherwise.
        """
        nb, H, d = self.num_blocks, self.Hkv, self.d
        st = np.uint16 if self.dtype == "bf16" else np.float32
        fill = (0x7FC0 if st == np.uint16 else np.nan) if poison else 0
        kpool = np.full((nb, H, BLOCK, d), fill, dtype=st)
        vpool = np.full((nb, H, d, BLOCK), fill, dtype=st)
        assert all(r % 8 == 0 for r in self.pool_rank), "low-rank pools hold chunks of 8 ranks"
        lkp = [np.full((nb, r // 8, BLOCK, 8), fill, dtype=st) for r in self.pool_rank]
        lvp = [np.full((nb, r, BLOCK), fill, dtype=st) for r in self.pool_rank]
        bits = st == np.uint16

        def fill_segment(sid):
            seg = self.segments[sid]
            kb, vb, lk, lv = self.segment_data(sid, bits=bits)
            nfull = seg.T // BLOCK
            rem = seg.T - nfull * BLOCK
            pad = (-seg.T) % BLOCK

            def blocks_of(x):  # [T, ...] -> [nblk, 16, ...] zero-padded tail
                if pad:
                    x = np.concatenate([x, np.zeros((pad,) + x.shape[1:], x.dtype)])
                return x.reshape((-1, BLOCK) + x.shape[1:])

            kbb = blocks_of(kb).transpose(0, 2, 1, 3)  # [nblk, H, 16, d]
            vbb = blocks_of(vb).transpose(0, 2, 3, 1)  # [nblk, H, d, 16]
            ids = seg.blocks
            if nfull:
                kpool[ids[:nfull]] = kbb[:nfull]
                vpool[ids[:nfull]] = vbb[:nfull]
            if rem:
                kpool[ids[nfull], :, :rem, :] = kbb[nfull, :, :rem, :]
                vpool[ids[nfull], :, :, :rem] = vbb[nfull, :, :, :rem]
            for p in seg.pools:
                lkb = blocks_of(lk[p])  # [nblk, 16, r] -> [nblk, r/8, 16, 8]
                lkb = lkb.reshape(lkb.shape[0], BLOCK, -1, 8).transpose(0, 2, 1, 3)
                lvb = blocks_of(lv[p]).transpose(0, 2, 1)  # [nblk, r, 16]
                if nfull:
                    lkp[p][ids[:nfull]] = lkb[:nfull]
                    lvp[p][ids[:nfull]] = lvb[:nfull]
                if rem:
                    lkp[p][ids[nfull], :, :rem, :] = lkb[nfull, :, :rem, :]
                    lvp[p][ids[nfull], :, :rem] = lvb[nfull, :, :rem]

        # segments own disjoint blocks, so they fill in parallel
        workers = max(1, min(16, len(os.sched_getaffinity(0)), len(self.segments)))
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            list(ex.map(fill_segment, range(len(self.segments))))
        return kpool, vpool, lkp, lvp

    def host_adapters(self):
        st = np.uint16 if self.dtype == "bf16" else np.float32
        conv = bf16_bits if st == np.uint16 else (lambda x: np.ascontiguousarray(x, np.float32))
        return [tuple(conv(m) for m in self.adapter(a)) for a in range(self.n_agents)]

    def host_q(self):
        q = self.q_all()
        return bf16_bits(q) if self.dtype == "bf16" else q


# ---------------------------------------------------------------------------
# The five workloads (plus parametrised small variants for the tests)
# ---------------------------------------------------------------------------


def decode_workload(
    name="decode",
    dtype="bf16",
    Hq=32,
    Hkv=8,
    d=128,
    theta=5e5,
    group_sizes=(4,),
    context_lens=(8192,),
    ranks=(16, 16, 16, 16),
    shared_l=True,
    agent_of_seq=None,
    shuffle=True,
    spare_blocks=0,
    seed=0,
    adapt="kv",
    adapter_starts=None,
):
    """Decode batch: groups of sequences; each group shares one base context.

    ``shared_l`` gives every agent one low-rank pool (shared-A adapters);
    otherwise each agent has its own pool. Sequence i of the flattened groups
    belongs to agent ``agent_of_seq[i]`` (default: i; -1: no adapter).
    """
    S = sum(group_sizes)
    agent_of_seq = list(agent_of_seq) if agent_of_seq is not None else list(range(S))
    n_agents = len(ranks)
    if shared_l:
        assert len(set(ranks)) == 1
        pool_of_agent, pool_rank = [0] * n_agents, [ranks[0]]
    else:
        pool_of_agent, pool_rank = list(range(n_agents)), list(ranks)
    segments, seqs, go = [], [], [0]
    s = 0
    for g, (gs, T) in enumerate(zip(group_sizes, context_lens)):
        pools = sorted({pool_of_agent[agent_of_seq[s + i]] for i in range(gs) if agent_of_seq[s + i] >= 0})
        segments.append(Segment(T=T, pools=tuple(pools)))
        for i in range(gs):
            st = 0 if adapter_starts is None else int(adapter_starts[s + i])
            seqs.append(SeqSpec(segments=(g,), agent=agent_of_seq[s + i], adapter_start=st))
        s += gs
        go.append(s)
    return Workload(
        name=name, dtype=dtype, Hq=Hq, Hkv=Hkv, d=d, theta=theta, ranks=list(ranks),
        pool_of_agent=pool_of_agent, pool_rank=pool_rank, segments=segments, seqs=seqs,
        group_offsets=go, seed=seed, shuffle=shuffle, spare_blocks=spare_blocks, adapt=adapt,
    )


def config_tiny_f32(seed=0):
    """Tiny fp32 decode: 4 q heads = 4 KV heads, d=64, T=256, r=8, 2 agents
    sharing one base, one low-rank pool per agent, no rotary, contiguous cache."""
    return decode_workload(
        name="tiny_f32_decode", dtype="f32", Hq=4, Hkv=4, d=64, theta=0.0, group_sizes=(2,),
        context_lens=(256,), ranks=(8, 8), shared_l=False, shuffle=False, seed=seed,
    )


def config_8b_decode(seed=0):
    """8B-shaped single-layer decode: 32 q / 8 KV heads, d=128, T=8192, 4 agents
    sharing one base and one shared-A low-rank pool (r=16), rotary theta 5e5,
    shuffled 16-token blocks, bf16."""
    return decode_workload(
        name="8b_decode_shared_base", dtype="bf16", Hq=32, Hkv=8, d=128, theta=5e5,
        group_sizes=(4,), context_lens=(8192,), ranks=(16, 16, 16, 16), shared_l=True, seed=seed,
    )


def prefill_workload(
    name="prefill",
    dtype="bf16",
    Hq=32,
    Hkv=8,
    d=128,
    theta=5e5,
    prefix=8192,
    q_lens=(512, 512, 512, 512),
    rank=16,
    shuffle=True,
    spare_blocks=0,
    seed=0,
    adapt="kv",
    agents=None,
    adapter_starts=None,
):
    """Prefill chunks: each agent appends ``q_lens[a]`` new tokens after one
    shared prefix; one shared-A low-rank pool; agent a's new rows live in its
    own blocks. Query i of agent a sits at position prefix + i. ``agents``
    gives the agent of each chunk (default: chunk a is agent a; -1: no
    adapter)."""
    A = len(q_lens)
    agents = list(range(A)) if agents is None else list(agents)
    segments = []
    if prefix:
        assert prefix % BLOCK == 0
        segments.append(Segment(T=prefix, pools=(0,)))
    base = len(segments)
    for a in range(A):
        segments.append(Segment(T=q_lens[a], pools=(0,)))
    starts = [0] * A if adapter_starts is None else [int(x) for x in adapter_starts]
    seqs = [SeqSpec(segments=((0,) if prefix else ()) + (base + a,), agent=agents[a], q_len=q_lens[a],
                    adapter_start=starts[a]) for a in range(A)]
    return Workload(
        name=name, dtype=dtype, Hq=Hq, Hkv=Hkv, d=d, theta=theta, ranks=[rank] * A,
        pool_of_agent=[0] * A, pool_rank=[rank], segments=segments, seqs=seqs,
        seed=seed, shuffle=shuffle, spare_blocks=spare_blocks, prefill=True, adapt=adapt,
    )


def config_prefill(seed=0):
    """Prefill chunk: 8B-shaped layer, 4 agents x 512 new tokens after an
    8192-token shared prefix, shared-A r=16, bf16."""
    return prefill_workload(name="8b_prefill_chunk", seed=seed)


def config_prefill_r64(seed=0):
    """The prefill chunk at rank 64 (shared-A r=64), the largest rank the
    pages sweep."""
    return prefill_workload(name="8b_prefill_chunk_r64", rank=64, seed=seed)


def mixed_workload(
    name="mixed",
    dtype="bf16",
    Hq=32,
    Hkv=8,
    d=128,
    theta=5e5,
    dec_group_sizes=(4,),
    dec_context_lens=(1500,),
    prefix=256,
    q_lens=(100, 37, 300),
    ranks=(16, 16, 16, 16),
    shared_l=True,
    dec_agents=None,
    pre_agents=None,
    shuffle=True,
    seed=0,
    adapt="kv",
    adapter_starts=None,
):
    """Decode groups followed by prefill chunks over one set of paged pools
    (the varlen call's batch). Decode sequences come first (one query each,
    grouped: each group shares one base context); then one prefill chunk per
    ``q_lens`` entry, all after one shared ``prefix``. Decode sequence i is
    agent ``dec_agents[i]`` (default i mod the agent count), chunk j agent
    ``pre_agents[j]`` (default j mod the agent count); -1: no adapter.
    ``adapter_starts`` covers all sequences, decode ones first."""
    n_agents = len(ranks)
    S_dec = sum(dec_group_sizes)
    dec_agents = [i % n_agents for i in range(S_dec)] if dec_agents is None else list(dec_agents)
    pre_agents = [j % n_agents for j in range(len(q_lens))] if pre_agents is None else list(pre_agents)
    if shared_l:
        assert len(set(ranks)) == 1
        pool_of_agent, pool_rank = [0] * n_agents, [ranks[0]]
    else:
        pool_of_agent, pool_rank = list(range(n_agents)), list(ranks)
    pools_of = lambda ags: tuple(sorted({pool_of_agent[a] for a in ags if a >= 0}))  # noqa: E731
    starts = [0] * (S_dec + len(q_lens)) if adapter_starts is None else [int(x) for x in adapter_starts]
    segments, seqs, go = [], [], [0]
    s = 0
    for g, (gs, T) in enumerate(zip(dec_group_sizes, dec_context_lens)):
        segments.append(Segment(T=T, pools=pools_of(dec_agents[s : s + gs])))
        for i in range(gs):
            seqs.append(SeqSpec(segments=(g,), agent=dec_agents[s + i], adapter_start=starts[s + i]))
        s += gs
        go.append(s)
    pre = ()
    if prefix:
        assert prefix % BLOCK == 0
        segments.append(Segment(T=prefix, pools=pools_of(pre_agents)))
        pre = (len(segments) - 1,)
    for j, ql in enumerate(q_lens):
        segments.append(Segment(T=ql, pools=pools_of([pre_agents[j]])))
        seqs.append(SeqSpec(segments=pre + (len(segments) - 1,), agent=pre_agents[j], q_len=ql,
                            adapter_start=starts[S_dec + j]))
    return Workload(
        name=name, dtype=dtype, Hq=Hq, Hkv=Hkv, d=d, theta=theta, ranks=list(ranks),
        pool_of_agent=pool_of_agent, pool_rank=pool_rank, segments=segments, seqs=seqs,
        group_offsets=go if S_dec else None, seed=seed, shuffle=shuffle, adapt=adapt,
    )


def config_mixed_step(seed=0):
    """One serving step of the 8B-shaped layer: the 4-agent decode on its
    8192-token shared base plus the prefill chunk (4 agents x 512 new tokens
    after an 8192-token shared prefix), shared-A r=16, bf16."""
    return mixed_workload(name="8b_decode_plus_prefill_chunk", dec_group_sizes=(4,), dec_context_lens=(8192,),
                          prefix=8192, q_lens=(512, 512, 512, 512), ranks=(16, 16, 16, 16), seed=seed)


def build_inputs(n_tokens=512, hidden=4096, n_cols=16, seed=0, sigma_a=1.0 / 64):
    """X [n, hidden] ~ N(0,1) and A [hidden, n_cols] ~ N(0, sigma_a), bf16-rounded."""
    root = np.random.SeedSequence(seed)
    cx, ca = root.spawn(2)
    X = _normal(np.random.default_rng(cx), (n_tokens, hidden), 1.0, "bf16")
    A = _normal(np.random.default_rng(ca), (hidden, n_cols), sigma_a, "bf16")
    return X, A


def config_long_layer(layer: int, seed=0):
    """One layer of the 32-layer long-context decode: T=32768, 8 agents sharing
    one base, per-agent low-rank pools at r=64, one decode token per agent."""
    return decode_workload(
        name=f"long_ctx_layer{layer}", dtype="bf16", Hq=32, Hkv=8, d=128, theta=5e5,
        group_sizes=(8,), context_lens=(32768,), ranks=(64,) * 8, shared_l=False,
        seed=int(np.random.SeedSequence([seed, layer]).generate_state(1)[0]),
    )


def config_serving_mix(seed=0, n_req=64, n_agents=16, tmin=1024, tmax=32768):
    """Concurrent-serving mix: 64 decode requests over 16 agents (4 each, in
    seeded shuffled order), T ~ U{1024..32768}, per-agent rank from
    {8,16,32,64}, each request with its own base and shuffled blocks."""
    rng = np.random.default_rng(np.random.SeedSequence([seed, 5]))
    lens = rng.integers(tmin, tmax + 1, size=n_req)
    ranks = rng.choice([8, 16, 32, 64], size=n_agents)
    agents = np.repeat(np.arange(n_agents), n_req // n_agents)
    rng.shuffle(agents)
    return decode_workload(
        name="serving_mix", dtype="bf16", Hq=32, Hkv=8, d=128, theta=5e5,
        group_sizes=(1,) * n_req, context_lens=tuple(int(t) for t in lens),
        ranks=tuple(int(r) for r in ranks), shared_l=False, agent_of_seq=agents.tolist(), seed=seed,
    )
