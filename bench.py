#!/usr/bin/env python3
"""Benchmark of the shared-base + low-rank KV attention hot path on one MI355X.

Prints ONE JSON line. The headline (``value``) is decode tokens/s of the
8B-shaped single-layer decode (32 q / 8 KV heads, d=128, T=8192, 4 agents
sharing one base and one shared-A r=16 low-rank cache, rotary theta 5e5,
shuffled 16-token blocks, bf16): one step = one lora_attn_decode call
serving the 4 agents' decode tokens. Inputs are resident in HBM before the
timed region; the base and low-rank pools are rotated over enough copies to
exceed the 256 MB last-level cache, so every step streams from HBM.

``roofline`` is for the decode kernel: algorithmic bytes per launch (each
distinct buffer once: base K/V, shared L_k/L_v, the 4 agents' B_k/B_v, q,
out, block table) divided by the kernel's mean duration from HIP events
around each launch in the timed region. ``traffic`` comes from the committed
rocprofv3 counter summary when it was taken on the current kernel source.

Other legs (same JSON line, under "legs"): the prefill chunk with its
low-rank cache build (and the chunk's attention at rank 64), the 32-layer long-context decode, the 64-request
serving mix, the tiny fp32 decode, the 8B decode and prefill chunk
without a key adapter (b_k NULL) and without adapters, and the low-rank
caches of 4 agents built from one segment's hidden states in one call, and one
serving step (the 8B decode plus the prefill chunk) as one varlen launch
against the two separate calls. ``cpu_baseline``
times the fp64 oracle on the host on a bounded sample of the headline
workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
MALL_BYTES = 256 << 20
PROFILES = os.path.join(ROOT, "profiles")


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--legs", default="decode,prefill,prefill64,long,mix,tiny,qv,base,act,lrmulti,varlen")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (counter calibration) and exit")
    return ap.parse_args()


# ---------------------------------------------------------------- timing
def _timed(launch, K, W, n_copies):
    """Run W untimed then exactly K timed launches (launch(i) uses copy
    i % n_copies), back to back between two HIP events on the launch stream.
    The GPU is kept busy with a spin kernel while the host enqueues, so the K
    launches run back to back and the event interval holds GPU time only.
    Returns the mean time per launch in ms (kernel time plus the gap
    between dependent launches; no per-launch event overhead)."""
    import torch

    for i in range(W):
        launch(i % n_copies)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e6) + K * 200000)
    t0.record()
    for i in range(K):
        launch(i % n_copies)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / K


def _per_launch_us(launch, n, n_copies):
    """Per-launch times (us) of n back-to-back launches, each between two
    events on the launch stream (so each includes its launch gap, as the mean
    of _timed does): median, p10, p90."""
    import torch

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    torch.cuda._sleep(int(2e6) + n * 200000)
    for i in range(n):
        ev[i].record()
        launch(i % n_copies)
    ev[n].record()
    torch.cuda.synchronize()
    d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(n))
    q = lambda f: round(d[min(n - 1, int(round(f * (n - 1))))], 2)  # noqa: E731
    return {"median": q(0.5), "p10": q(0.1), "p90": q(0.9), "launches": n,
            "note": "each launch between two events of its own; the event records add about 2.5 us per launch, "
                    "so ms_per_step (one event pair around all launches) is the throughput figure"}


def hbm_measured():
    """Measured HBM ceilings on this device, beside the published peak: a
    4 GiB fp32 read (torch sum) and a 4 GiB copy (torch copy_), best of 5."""
    import torch

    n = 1 << 30
    x = torch.ones(n, dtype=torch.float32, device="cuda")
    y = torch.empty_like(x)
    out = {}
    for name, fn, nbytes in (("read_GBps", lambda: x.sum(), 4 * n), ("copy_GBps", lambda: y.copy_(x), 8 * n)):
        fn()
        best = None
        for _ in range(5):
            t0 = torch.cuda.Event(enable_timing=True)
            t1 = torch.cuda.Event(enable_timing=True)
            t0.record()
            fn()
            t1.record()
            torch.cuda.synchronize()
            ms = t0.elapsed_time(t1)
            best = ms if best is None else min(best, ms)
        out[name] = round(nbytes / (best / 1e3) / 1e9, 1)
    del x, y
    torch.cuda.empty_cache()
    out["how"] = ("torch sum over 4 GiB fp32 (read) and copy_ of 4 GiB (read + write), best of 5; torch's own "
                  "kernels, a lower bound on the attainable bandwidth; roofline.peak stays the published 8 TB/s")
    return out


def _p(t):
    """Device address of a tensor, 0 (NULL) for an absent one."""
    return 0 if t is None else t.data_ptr()


def _decode_caller(dw, ws_bytes):
    """Pre-marshalled C call of lora_attn_decode for each pool copy."""
    import torch

    import shared_base_kv_amd as lra

    lib = lra.load()
    w = dw.w
    ws = torch.zeros(max(ws_bytes, 256), dtype=torch.uint8, device="cuda")
    out = dw.new_out()
    ng = dw.group_offsets.numel() - 1
    code = lra.LRA_BF16 if w.dtype == "bf16" else lra.LRA_F32
    stream = torch.cuda.current_stream().cuda_stream
    copies = dw.copies if hasattr(dw, "copies") else [(dw.k_base, dw.v_base, dw.lk_ptrs, dw.lv_ptrs)]
    argsets = []
    for kb, vb, lkp, lvp in copies:
        argsets.append((dw.q.data_ptr(), kb.data_ptr(), vb.data_ptr(), dw.block_tables.data_ptr(),
                        dw.block_tables.shape[1], dw.context_lens.data_ptr(), dw.max_context_len,
                        dw.group_offsets.data_ptr(), ng, _p(dw.agent_ids), _p(dw.adapter_start), _p(lkp), _p(lvp),
                        _p(dw.bk_ptrs), _p(dw.bv_ptrs), _p(dw.ranks), dw.max_rank, w.S,
                        w.n_agents, w.Hq, w.Hkv, w.d, 16, w.sm_scale, w.theta, code, out.data_ptr(),
                        ws.data_ptr(), ws.numel(), stream))

    def launch(i):
        rc = lib.lora_attn_decode(*argsets[i])
        if rc:
            raise lra.LraError(rc, lra.lra_last_error())

    return launch, out, ws, len(argsets)


def _replicate(dw, min_bytes):
    """Extra device copies of the base and low-rank pools so the rotation
    over copies exceeds the last-level cache."""
    import torch

    per = dw.k_base.nbytes + dw.v_base.nbytes + sum(t.nbytes for t in dw.lk_pools + dw.lv_pools)
    n = max(1, -(-min_bytes // per))
    copies = [(dw.k_base, dw.v_base, dw.lk_ptrs, dw.lv_ptrs)]
    keep = []
    for _ in range(n - 1):
        kb, vb = dw.k_base.clone(), dw.v_base.clone()
        lks = [t.clone() for t in dw.lk_pools]
        lvs = [t.clone() for t in dw.lv_pools]
        w = dw.w
        lkp = torch.tensor([lks[w.pool_of_agent[a]].data_ptr() for a in range(w.n_agents)], dtype=torch.int64,
                           device="cuda") if w.has_k else None
        lvp = torch.tensor([lvs[w.pool_of_agent[a]].data_ptr() for a in range(w.n_agents)], dtype=torch.int64,
                           device="cuda") if w.has_v else None
        keep += [lks, lvs]
        copies.append((kb, vb, lkp, lvp))
    dw.copies = copies
    dw._keep = keep
    return n


def decode_bytes(w):
    """Algorithmic bytes of one decode step: every distinct buffer once (the
    low-rank rows and B matrices of present adapters only)."""
    es = 2 if w.dtype == "bf16" else 4
    n_proj = int(w.has_k) + int(w.has_v)
    tok_groups = sum(w.segments[i].T for i in range(len(w.segments)))
    base = tok_groups * w.Hkv * w.d * es * 2
    # low-rank rows from the earliest activation position among the sequences
    # that read a (segment, pool) pair
    first = {}
    for sq in w.seqs:
        if sq.agent < 0:
            continue
        off = 0
        for sid in sq.segments:
            key = (sid, w.pool_of_agent[sq.agent])
            first[key] = min(first.get(key, 1 << 60), max(0, sq.adapter_start - off))
            off += w.segments[sid].T
    lr = sum(max(0, w.segments[sid].T - st) * w.pool_rank[p] for (sid, p), st in first.items()) * es * n_proj
    used_agents = sorted({sq.agent for sq in w.seqs if sq.agent >= 0})
    bmat = sum(w.ranks[a] * w.Hkv * w.d * es * n_proj for a in used_agents)
    qo = w.S * w.Hq * w.d * es * 2
    tables = sum(-(-w.context_len(s) // 16) for s in range(w.S)) * 4 + w.S * 4 * 2
    return base + lr + bmat + qo + tables


def decode_flops(w):
    """Algorithmic FLOPs of one decode step over visible pairs: adapter key
    rebuild, QK, PV, P L_v and the final C B_v."""
    f = 0
    for s in range(w.S):
        T = w.context_len(s)
        a = w.seqs[s].agent
        rk = w.ranks[a] if (a >= 0 and w.has_k) else 0
        rv = w.ranks[a] if (a >= 0 and w.has_v) else 0
        Ta = max(0, T - max(0, w.seqs[s].adapter_start))  # tokens carrying adapter terms
        f += 2 * Ta * rk * w.Hkv * w.d  # rebuild L_k B_k (per agent, per KV head)
        f += 2 * T * w.Hq * w.d * 2  # QK and PV
        f += 2 * Ta * w.Hq * rv  # P L_v
        f += 2 * w.Hq * rv * w.d  # C B_v
    return f


# every source the decode kernels are compiled from
DECODE_SOURCES = ("decode_bf16.hip", "decode_bf16_kv.hip", "decode_bf16_body.h", "decode_bf16_body.inc",
                  "device_common.h", "internal.h")


def decode_source_sha256():
    h = hashlib.sha256()
    for name in DECODE_SOURCES:
        h.update(name.encode())
        h.update(open(os.path.join(ROOT, "shared_base_kv_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def _traffic():
    """HBM bytes per decode call from the committed counter summary, or None
    if the counters were taken on another version of the decode sources."""
    path = os.path.join(PROFILES, "decode_8b_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_source_sha256") != decode_source_sha256():
        return None
    return rec.get("bytes_per_launch")


# ------------------------------------------------------------------ legs
def leg_decode(K, W, adapt="kv", starts=None):
    """The 8B-shaped decode; ``adapt`` "v" drops the key adapter (b_k NULL),
    "none" both adapters; ``starts`` sets the agents' activation positions."""
    from workloads import config_8b_decode
    from workloads.device import upload

    import shared_base_kv_amd as lra

    w = config_8b_decode()
    w.adapt = adapt
    for i, st in enumerate(starts or ()):
        w.seqs[i].adapter_start = st
    dw = upload(w)
    ncopy = _replicate(dw, 2 * MALL_BYTES)
    wsb = lra.lora_attn_decode_workspace_size(w.S, 1, w.Hq, w.Hkv, w.d, dw.max_rank, dw.max_context_len, lra.LRA_BF16)
    launch, _, _, n = _decode_caller(dw, wsb)
    step_ms = _timed(launch, K, W, n)
    per_launch = _per_launch_us(launch, max(K, 50), n)
    nbytes = decode_bytes(w)
    return dict(w=w, step_ms=step_ms, kernel_ms=step_ms, bytes=nbytes, flops=decode_flops(w), tokens=w.S,
                copies=ncopy, per_launch_us=per_launch)


def leg_long(K, W):
    """32-layer long-context decode: 32 independent layer calls per step."""
    import concurrent.futures as cf

    import torch

    import shared_base_kv_amd as lra
    from workloads import config_long_layer
    from workloads.device import upload

    layers = [config_long_layer(i) for i in range(32)]
    with cf.ThreadPoolExecutor(max_workers=8) as ex:
        pools = list(ex.map(lambda w: w.host_pools(), layers))
    dws = []
    for i in range(len(layers)):
        dws.append(upload(layers[i], host_pools=pools[i]))
        pools[i] = None
    wsb = lra.lora_attn_decode_workspace_size(8, 1, 32, 8, 128, 64, 32768, lra.LRA_BF16)
    calls = [_decode_caller(dw, wsb) for dw in dws]

    def launch(i):
        for c in calls:
            c[0](0)

    step_ms = _timed(launch, max(2, K // 8), min(W, 2), 1)
    nbytes = sum(decode_bytes(w) for w in layers)
    flops = sum(decode_flops(w) for w in layers)
    del dws, calls
    torch.cuda.empty_cache()
    return dict(step_ms=step_ms, layer_ms=step_ms / 32, bytes=nbytes, flops=flops, tokens=8)


def leg_mix(K, W):
    import torch

    import shared_base_kv_amd as lra
    from workloads import config_serving_mix
    from workloads.device import upload

    w = config_serving_mix()
    dw = upload(w)
    wsb = lra.lora_attn_decode_workspace_size(w.S, w.S, w.Hq, w.Hkv, w.d, dw.max_rank, dw.max_context_len,
                                              lra.LRA_BF16)
    launch, _, _, n = _decode_caller(dw, wsb)
    step_ms = _timed(launch, max(4, K // 4), W, n)
    out = dict(step_ms=step_ms, kernel_ms=step_ms, bytes=decode_bytes(w), flops=decode_flops(w), tokens=w.S,
               total_context=int(sum(w.context_len(s) for s in range(w.S))))
    del dw
    torch.cuda.empty_cache()
    return out


def leg_tiny(K, W):
    import shared_base_kv_amd as lra
    from workloads import config_tiny_f32
    from workloads.device import upload

    w = config_tiny_f32()
    dw = upload(w)
    launch, _, _, n = _decode_caller(dw, 0)
    step_ms = _timed(launch, K, W, n)
    return dict(step_ms=step_ms, kernel_ms=step_ms, tokens=w.S)


def leg_prefill(K, W):
    """Prefill chunk: lr_cache_build for the 4 agents' new tokens (X_a A_k and
    X_a A_v into the paged pools), then lora_attn_prefill."""
    import torch

    import shared_base_kv_amd as lra
    from workloads import bf16_bits, build_inputs, config_prefill
    from workloads.device import upload

    w = config_prefill()
    dw = upload(w)
    # build inputs: X_a [512, 4096] per agent, A_k and A_v [4096, 16]
    dev = lambda x: torch.from_numpy(bf16_bits(x).view("int16")).view(torch.bfloat16).cuda()  # noqa: E731
    Xs = [dev(build_inputs(512, 4096, 16, seed=100 + a)[0]) for a in range(4)]
    Ak = dev(build_inputs(1, 4096, 16, seed=200)[1])
    Av = dev(build_inputs(1, 4096, 16, seed=201)[1])
    slots = []
    for a in range(4):
        seg = w.segments[1 + a]
        ids = torch.from_numpy(seg.blocks.astype("int64"))
        slots.append((ids[:, None] * 16 + torch.arange(16)[None, :]).reshape(-1)[: seg.T].cuda())
    bws = torch.zeros(lra.lr_cache_build_workspace_size(512, 4096, 16), dtype=torch.uint8, device="cuda")
    out = dw.new_out()

    def build_all():
        for a in range(4):
            lra.lr_cache_build(Xs[a], Ak, dw.lk_pools[0], bws, slot_mapping=slots[a], l_layout=lra.LRA_L_KEY_CHUNKED,
                               ldl=16)
            lra.lr_cache_build(Xs[a], Av, dw.lv_pools[0], bws, slot_mapping=slots[a], l_layout=lra.LRA_L_RANK_MAJOR)

    def prefill():
        lra.lora_attn_prefill(dw.q, dw.k_base, dw.v_base, dw.block_tables, dw.context_lens, dw.max_context_len,
                              dw.cu_q_lens, dw.max_q_len, dw.agent_ids, dw.lk_ptrs, dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs,
                              dw.ranks, dw.max_rank, w.n_agents, w.Hkv, w.sm_scale, w.theta, out,
                              adapter_start=dw.adapter_start)

    kk = max(4, K // 5)
    b_kern = _timed(lambda i: build_all(), kk, 2, 1)
    p_kern = _timed(lambda i: prefill(), kk, 2, 1)
    flops = prefill_flops(w)
    return dict(build_ms=b_kern, prefill_ms=p_kern, flops=flops,
                tokens=sum(sq.q_len for sq in w.seqs), build_bytes=4 * 2 * (512 * 4096 * 2 + 4096 * 16 * 2 + 512 * 16 * 2))


def leg_prefill_absent(K, W, adapt, starts=None, config=None):
    """The prefill chunk's attention alone with absent adapters or
    activation positions (or another chunk configuration)."""
    from workloads import config_prefill
    from workloads.device import upload

    import shared_base_kv_amd as lra

    w = (config or config_prefill)()
    w.adapt = adapt
    for i, st in enumerate(starts or ()):
        w.seqs[i].adapter_start = st
    dw = upload(w)
    out = dw.new_out()

    def prefill():
        lra.lora_attn_prefill(dw.q, dw.k_base, dw.v_base, dw.block_tables, dw.context_lens, dw.max_context_len,
                              dw.cu_q_lens, dw.max_q_len, dw.agent_ids, dw.lk_ptrs, dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs,
                              dw.ranks, dw.max_rank, w.n_agents, w.Hkv, w.sm_scale, w.theta, out,
                              adapter_start=dw.adapter_start)

    ms = _timed(lambda i: prefill(), max(4, K // 5), 2, 1)
    return dict(prefill_ms=ms, flops=prefill_flops(w), tokens=sum(sq.q_len for sq in w.seqs))


def leg_varlen(K, W):
    """One serving step of the 8B-shaped layer (the 4-agent decode on its
    8192-token base plus the 4 x 512-token prefill chunk): one
    lora_attn_varlen call against lora_attn_decode followed by
    lora_attn_prefill, with the same context and query-length bounds."""
    import torch

    import shared_base_kv_amd as lra
    from workloads import config_mixed_step
    from workloads.device import upload

    w = config_mixed_step()
    dw = upload(w)
    S_dec = 4
    out = dw.new_out()
    ng = dw.group_offsets.numel() - 1
    wsv = torch.zeros(max(256, lra.lora_attn_varlen_workspace_size(w.S, S_dec, ng, w.Hq, w.Hkv, w.d, dw.max_rank,
                                                                   dw.max_context_len, lra.LRA_BF16)),
                      dtype=torch.uint8, device="cuda")
    wsd = torch.zeros(max(256, lra.lora_attn_decode_workspace_size(S_dec, ng, w.Hq, w.Hkv, w.d, dw.max_rank,
                                                                   dw.max_context_len, lra.LRA_BF16)),
                      dtype=torch.uint8, device="cuda")
    qd, qp = dw.q[:S_dec].contiguous(), dw.q[S_dec:].contiguous()
    btd, btp = dw.block_tables[:S_dec].contiguous(), dw.block_tables[S_dec:].contiguous()
    cd, cp = dw.context_lens[:S_dec].contiguous(), dw.context_lens[S_dec:].contiguous()
    agd, agp = dw.agent_ids[:S_dec].contiguous(), dw.agent_ids[S_dec:].contiguous()
    cup = (dw.cu_q_lens[S_dec:] - S_dec).contiguous()
    od, op = out[:S_dec].clone(), out[S_dec:].clone()

    def unified():
        lra.lora_attn_varlen(dw.q, dw.k_base, dw.v_base, dw.block_tables, dw.context_lens, dw.max_context_len,
                             dw.cu_q_lens, dw.max_q_len, S_dec, dw.group_offsets, dw.agent_ids, dw.lk_ptrs, dw.lv_ptrs,
                             dw.bk_ptrs, dw.bv_ptrs, dw.ranks, dw.max_rank, w.n_agents, w.Hkv, w.sm_scale, w.theta,
                             out, wsv)

    def separate():
        lra.lora_attn_decode(qd, dw.k_base, dw.v_base, btd, cd, dw.max_context_len, dw.group_offsets, agd, dw.lk_ptrs,
                             dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs, dw.ranks, dw.max_rank, w.n_agents, w.Hkv, w.sm_scale,
                             w.theta, od, wsd)
        lra.lora_attn_prefill(qp, dw.k_base, dw.v_base, btp, cp, dw.max_context_len, cup, dw.max_q_len, agp,
                              dw.lk_ptrs, dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs, dw.ranks, dw.max_rank, w.n_agents, w.Hkv,
                              w.sm_scale, w.theta, op)

    def prefill_via_varlen():  # the prefill part alone through the varlen entry point
        lra.lora_attn_varlen(qp, dw.k_base, dw.v_base, btp, cp, dw.max_context_len, cup, dw.max_q_len, 0, None, agp,
                             dw.lk_ptrs, dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs, dw.ranks, dw.max_rank, w.n_agents, w.Hkv,
                             w.sm_scale, w.theta, op, None)

    def prefill_alone():
        lra.lora_attn_prefill(qp, dw.k_base, dw.v_base, btp, cp, dw.max_context_len, cup, dw.max_q_len, agp,
                              dw.lk_ptrs, dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs, dw.ranks, dw.max_rank, w.n_agents, w.Hkv,
                              w.sm_scale, w.theta, op)

    # the four are timed in turn, three rounds, best of each (so no one of
    # them is favoured by the order or by the clock's drift)
    kk = max(4, K // 5)
    best = {}
    for _ in range(3):
        for name, fn in (("uni", unified), ("sep", separate), ("pv", prefill_via_varlen), ("pa", prefill_alone)):
            t = _timed(lambda i, fn=fn: fn(), kk, 2, 1)
            best[name] = min(best.get(name, t), t)
    t_uni, t_sep, t_pv, t_pa = best["uni"], best["sep"], best["pv"], best["pa"]
    return dict(unified_ms=t_uni, separate_ms=t_sep, prefill_varlen_ms=t_pv, prefill_ms=t_pa,
                tokens=int(dw.cu_q_lens[-1].item()), flops=prefill_flops(w), w=w)


def leg_lr_multi(K, W, n_agents=4, rank=16):
    """Low-rank caches of every agent from one segment's hidden states: X
    [512, 4096] against the 2 * n_agents adapters' A (r=16 each) side by side,
    one lr_cache_build_multi call into 2 * n_agents paged pools, against the
    same rows built by one lr_cache_build call per adapter."""
    import torch

    import shared_base_kv_amd as lra
    from workloads import bf16_bits, build_inputs

    n, hidden = 512, 4096
    ncols = 2 * n_agents * rank
    X, A = build_inputs(n, hidden, ncols, seed=300)
    dev = lambda x: torch.from_numpy(bf16_bits(x).view("int16")).view(torch.bfloat16).cuda()  # noqa: E731
    Xd, Ad = dev(X), dev(A)
    nb = n // 16 + 8
    slots = torch.randperm(nb * 16, generator=torch.Generator().manual_seed(1))[:n].cuda()
    cols = [rank * g for g in range(2 * n_agents + 1)]
    lays = [lra.LRA_L_KEY_CHUNKED, lra.LRA_L_RANK_MAJOR] * n_agents
    pools = [torch.zeros((nb, rank // 8, 16, 8) if l == lra.LRA_L_KEY_CHUNKED else (nb, rank, 16),
                         dtype=torch.bfloat16, device="cuda") for l in lays]
    ws = torch.zeros(lra.lr_cache_build_workspace_size(n, hidden, ncols), dtype=torch.uint8, device="cuda")
    ws1 = torch.zeros(lra.lr_cache_build_workspace_size(n, hidden, rank), dtype=torch.uint8, device="cuda")

    def multi():
        lra.lr_cache_build_multi(Xd, Ad, cols, pools, lays, slots, ws)

    def singles():
        for g in range(2 * n_agents):
            lra.lr_cache_build(Xd, Ad[:, cols[g]:cols[g + 1]], pools[g], ws1, slot_mapping=slots, l_layout=lays[g],
                               ldl=rank, n_cols=rank)

    kk = max(10, K)
    ms_multi = _timed(lambda i: multi(), kk, 3, 1)
    ms_single = _timed(lambda i: singles(), kk, 3, 1)
    nbytes = n * hidden * 2 + hidden * ncols * 2 + n * ncols * 2 + n * 8  # X once, A, L rows, slot mapping
    return dict(ms_multi=ms_multi, ms_single=ms_single, bytes=nbytes, n_groups=2 * n_agents, n_cols=ncols)


def prefill_flops(w):
    """Visible-pair FLOPs of the prefill chunk: QK, PV, P L_v over causal pairs,
    the adapter key rebuild once per token, and C B_v per row (adapter terms
    of present adapters only)."""
    f = 0
    for s, sq in enumerate(w.seqs):
        T = w.context_len(s)
        rk = w.ranks[sq.agent] if (sq.agent >= 0 and w.has_k) else 0
        rv = w.ranks[sq.agent] if (sq.agent >= 0 and w.has_v) else 0
        nq = sq.q_len
        st = max(0, sq.adapter_start)
        pairs = sum(T - nq + i + 1 for i in range(nq))
        pairs_ad = sum(max(0, T - nq + i + 1 - st) for i in range(nq))  # visible pairs with an adapted key
        f += pairs * w.Hq * 2 * w.d * 2 + pairs_ad * w.Hq * 2 * rv
        f += 2 * max(0, T - st) * rk * w.Hkv * w.d
        f += 2 * nq * w.Hq * rv * w.d
    return f


# ------------------------------------------------------------- baseline
def cpu_baseline(seconds):
    import numpy as np

    import oracle
    from workloads import config_8b_decode

    try:
        from threadpoolctl import threadpool_info

        blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max([i.get("num_threads", 1) for i in blas] or [1])
        vendor = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in blas})) or "unknown"
    except Exception:
        threads, vendor = 1, "unknown"
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "unknown")
    except OSError:
        pass
    w = config_8b_decode()
    logical = [w.logical(s) for s in range(w.S)]
    done = 0
    t0 = time.perf_counter()
    while True:
        for lg in logical:
            oracle.lora_attention(**lg, sm_scale=w.sm_scale, theta=w.theta)
            done += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"fp64 oracle on the 8B-shaped decode workload: {done} sequence decodes "
                      f"({done // w.S} full 4-agent steps) in {dt:.1f} s, BLAS threads={threads}, "
                      f"host cpus={len(os.sched_getaffinity(0))}",
            "cpu_model": model, "blas": vendor}


def main():
    args = _args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: this library has no multi-GPU path "
              "(DESIGN.md describes how it would shard). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    torch.cuda.set_device(0)
    if args.calibrate_copy_mib:
        # a plain copy of known size: HBM counters per dispatch should read
        # this many bytes fetched and written
        n = args.calibrate_copy_mib << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": n, "launches": 5}))
        return
    legs = set(args.legs.split(","))
    K, W = args.steps, args.warmup

    torch.cuda.synchronize()
    log = lambda m: print(f"[bench] {m}", file=sys.stderr, flush=True)  # noqa: E731
    head = leg_decode(K, W)
    log(f"decode leg done: {head['kernel_ms'] * 1e3:.2f} us/launch")
    w = head["w"]
    step_s = head["step_ms"] / 1e3
    kern_s = head["kernel_ms"] / 1e3
    achieved = head["bytes"] / kern_s / 1e9
    traffic = _traffic()
    res = {
        "metric": "LoRA-attn decode tokens/s (8B-shaped layer, 4 agents, shared base, T=8192)",
        "value": round(head["tokens"] / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(head["step_ms"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) base/low-rank caches, N(0,0.1/sqrt(r)) adapters)",
        "config": {"workload": "8b_decode_shared_base", "Hq": 32, "Hkv": 8, "head_dim": 128, "context": 8192,
                   "agents": 4, "rank": 16, "shared_a": True, "rope_theta": 5e5, "block_size": 16,
                   "pool_copies_rotated": head["copies"]},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_bf16_kernel<16, 4, true, true, false> + decode_bf16_combine<32>", "algorithmic_bytes_per_launch": head["bytes"],
                     "ms_per_launch": round(head["kernel_ms"], 5)},
        "per_launch_us": head["per_launch_us"],
    }
    try:
        res["hbm_measured"] = hbm_measured()
    except Exception as e:  # a measurement aid, never the product path
        res["hbm_measured"] = {"error": str(e)[:200]}
    extra = {}
    if "prefill" in legs:
        try:
            p = leg_prefill(K, W)
            tf = p["flops"] / (p["prefill_ms"] / 1e3) / 1e12
            extra["prefill_chunk"] = {
                "prefill_tokens_per_s": round(p["tokens"] / (p["prefill_ms"] / 1e3), 1),
                "prefill_ms": round(p["prefill_ms"], 4), "tflops": round(tf, 2),
                "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                             "frac": round(tf / BF16_PEAK_TFLOPS, 4), "algorithmic_flops": p["flops"]},
                "lr_cache_build_ms_8_calls": round(p["build_ms"], 4),
                "lr_cache_build_GBps": round(p["build_bytes"] / (p["build_ms"] / 1e3) / 1e9, 1),
            }
        except Exception as e:  # prefill not available
            extra["prefill_chunk"] = {"error": str(e)[:200]}
        log("prefill leg done")
    if "prefill64" in legs:
        from workloads import config_prefill_r64
        p = leg_prefill_absent(K, W, "kv", config=config_prefill_r64)
        tf = p["flops"] / (p["prefill_ms"] / 1e3) / 1e12
        extra["prefill_chunk_rank64"] = {
            "prefill_tokens_per_s": round(p["tokens"] / (p["prefill_ms"] / 1e3), 1),
            "prefill_ms": round(p["prefill_ms"], 4), "tflops": round(tf, 2),
            "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4), "algorithmic_flops": p["flops"]}
        log("rank-64 prefill leg done")
    if "long" in legs:
        lo = leg_long(K, W)
        extra["long_ctx_32_layers"] = {
            "tokens_per_s": round(lo["tokens"] / (lo["step_ms"] / 1e3), 1), "ms_per_step": round(lo["step_ms"], 4),
            "GBps": round(lo["bytes"] / (lo["step_ms"] / 1e3) / 1e9, 1),
            "hbm_frac": round(lo["bytes"] / (lo["step_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "tflops": round(lo["flops"] / (lo["step_ms"] / 1e3) / 1e12, 2), "bytes_per_step": lo["bytes"]}
        log("long-context leg done")
    if "mix" in legs:
        mx = leg_mix(K, W)
        extra["serving_mix_64"] = {
            "tokens_per_s": round(mx["tokens"] / (mx["step_ms"] / 1e3), 1), "ms_per_step": round(mx["step_ms"], 4),
            "kernel_ms": round(mx["kernel_ms"], 4),
            "GBps": round(mx["bytes"] / (mx["kernel_ms"] / 1e3) / 1e9, 1),
            "hbm_frac": round(mx["bytes"] / (mx["kernel_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "bytes_per_step": mx["bytes"], "total_context": mx["total_context"]}
        log("serving-mix leg done")
    for leg, adapt in (("qv", "v"), ("base", "none")):
        if leg not in legs:
            continue
        d = leg_decode(K, W, adapt)
        gbs = d["bytes"] / (d["kernel_ms"] / 1e3) / 1e9
        extra[f"decode_{'no_key_adapter' if adapt == 'v' else 'no_adapter'}"] = {
            "tokens_per_s": round(d["tokens"] / (d["step_ms"] / 1e3), 1),
            "us_per_launch": round(d["kernel_ms"] * 1e3, 2), "GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": d["bytes"]}
        # the prefill chunk with the same adapters
        p = leg_prefill_absent(K, W, adapt)
        tf = p["flops"] / (p["prefill_ms"] / 1e3) / 1e12
        extra[f"prefill_{'no_key_adapter' if adapt == 'v' else 'no_adapter'}"] = {
            "prefill_tokens_per_s": round(p["tokens"] / (p["prefill_ms"] / 1e3), 1),
            "prefill_ms": round(p["prefill_ms"], 4), "tflops": round(tf, 2),
            "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4), "algorithmic_flops": p["flops"]}
        log(f"{leg} legs done")
    if "act" in legs:
        # activated adapters: the 8B decode with the agents invoked for the
        # last 512 tokens, and the prefill chunk with each agent activated at
        # its own 512 new tokens (the shared prefix keeps the base cache)
        d = leg_decode(K, W, "kv", starts=[8192 - 512] * 4)
        gbs = d["bytes"] / (d["kernel_ms"] / 1e3) / 1e9
        extra["decode_activated_last_512"] = {
            "tokens_per_s": round(d["tokens"] / (d["step_ms"] / 1e3), 1),
            "us_per_launch": round(d["kernel_ms"] * 1e3, 2), "GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes_per_launch": d["bytes"]}
        # the prefill chunk with each agent activated at its new tokens
        p = leg_prefill_absent(K, W, "kv", starts=[8192] * 4)
        tf = p["flops"] / (p["prefill_ms"] / 1e3) / 1e12
        extra["prefill_activated_at_chunk"] = {
            "prefill_tokens_per_s": round(p["tokens"] / (p["prefill_ms"] / 1e3), 1),
            "prefill_ms": round(p["prefill_ms"], 4), "tflops": round(tf, 2),
            "mfma_frac": round(tf / BF16_PEAK_TFLOPS, 4), "algorithmic_flops": p["flops"]}
        log("activation legs done")
    if "lrmulti" in legs:
        lm = leg_lr_multi(K, W)
        gbs = lm["bytes"] / (lm["ms_multi"] / 1e3) / 1e9
        extra["lr_cache_build_multi_4_agents"] = {
            "us_per_call": round(lm["ms_multi"] * 1e3, 2), "groups": lm["n_groups"], "n_cols": lm["n_cols"],
            "us_per_adapter_calls": round(lm["ms_single"] * 1e3, 2), "GBps": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4), "algorithmic_bytes": lm["bytes"]}
        log("multi-adapter cache build leg done")
    if "varlen" in legs:
        vl = leg_varlen(K, W)
        extra["varlen_serving_step"] = {
            "tokens": vl["tokens"], "unified_ms": round(vl["unified_ms"], 4), "separate_ms": round(vl["separate_ms"], 4),
            "tokens_per_s": round(vl["tokens"] / (vl["unified_ms"] / 1e3), 1),
            "saved_us": round((vl["separate_ms"] - vl["unified_ms"]) * 1e3, 2),
            "prefill_part_alone_ms": round(vl["prefill_ms"], 4),
            "prefill_part_through_varlen_ms": round(vl["prefill_varlen_ms"], 4)}
        log("varlen leg done")
    if "tiny" in legs:
        ti = leg_tiny(K, W)
        extra["tiny_f32"] = {"us_per_step": round(ti["step_ms"] * 1e3, 2), "kernel_us": round(ti["kernel_ms"] * 1e3, 2)}
    res["legs"] = extra
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
