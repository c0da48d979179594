"""Helpers shared by the GPU tests: run the library through its C ABI on a
seeded workload and compare with the fp64 oracle."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import shared_base_kv_amd as lra
from workloads.device import upload  # noqa: F401

TOL_F32 = 1e-5  # fp32 inputs and arithmetic
TOL_BF16 = 2e-2  # bf16 inputs, fp32 accumulation


def dtype_code(w):
    return lra.LRA_BF16 if w.dtype == "bf16" else lra.LRA_F32


def decode_workspace(dw):
    w = dw.w
    ng = dw.group_offsets.numel() - 1 if dw.group_offsets is not None else w.S
    n = lra.lora_attn_decode_workspace_size(w.S, ng, w.Hq, w.Hkv, w.d, dw.max_rank, dw.max_context_len, dtype_code(w))
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=dw.q.device)


def run_decode(dw, workspace=None, out=None):
    w = dw.w
    ws = decode_workspace(dw) if workspace is None else workspace
    out = dw.new_out() if out is None else out
    lra.lora_attn_decode(dw.q, dw.k_base, dw.v_base, dw.block_tables, dw.context_lens, dw.max_context_len,
                         dw.group_offsets, dw.agent_ids, dw.lk_ptrs, dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs, dw.ranks,
                         dw.max_rank, w.n_agents, w.Hkv, w.sm_scale, w.theta, out, ws, adapter_start=dw.adapter_start)
    torch.cuda.synchronize()
    return out


def run_prefill(dw, out=None):
    w = dw.w
    out = dw.new_out() if out is None else out
    lra.lora_attn_prefill(dw.q, dw.k_base, dw.v_base, dw.block_tables, dw.context_lens, dw.max_context_len,
                          dw.cu_q_lens, dw.max_q_len, dw.agent_ids, dw.lk_ptrs, dw.lv_ptrs, dw.bk_ptrs, dw.bv_ptrs,
                          dw.ranks, dw.max_rank, w.n_agents, w.Hkv, w.sm_scale, w.theta, out,
                          adapter_start=dw.adapter_start)
    torch.cuda.synchronize()
    return out


def oracle_rows(w, seqs, q_rows=None):
    """fp64 oracle output of the given sequences; q_rows optionally picks
    query rows per sequence (prefill sampling)."""
    outs = []
    for s in seqs:
        lg = w.logical(s)
        T = lg["kb"].shape[0]
        nq = lg["q"].shape[0]
        if q_rows is None:
            outs.append(oracle.lora_attention(**lg, sm_scale=w.sm_scale, theta=w.theta))
        else:
            rows = np.asarray(q_rows[s])
            pos = T - nq + rows
            K, V = oracle.materialise_kv(lg["kb"], lg["vb"], lg["lk"], lg["lv"], lg["bk"], lg["bv"], w.theta,
                                         lg["adapter_start"])
            outs.append(oracle.attend(lg["q"][rows], pos, K, V, w.sm_scale))
    return outs


def to_np(t):
    return t.float().cpu().numpy().astype(np.float64)


def row_rel_err(got, ref):
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows = last axis)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return float((num / den).max())
