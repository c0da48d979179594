"""Upload a seeded Workload to device memory in the library's layout.

Data movement only: the pools, tables and pointer arrays the C ABI takes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

from .synth import Workload


def _t(x: np.ndarray, dev, dtype_code: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if dtype_code == "bf16":
        t = t.view(torch.bfloat16)  # int16 bit patterns -> bf16
    return t.to(dev)


def _u16(x: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(x).view(np.int16)


@dataclass
class DeviceWorkload:
    w: Workload
    q: torch.Tensor
    k_base: torch.Tensor
    v_base: torch.Tensor
    block_tables: torch.Tensor
    context_lens: torch.Tensor
    group_offsets: torch.Tensor
    agent_ids: torch.Tensor  # None without any adapter
    adapter_start: torch.Tensor  # int32 [S] activation positions, None when all are 0
    lk_pools: list
    lv_pools: list
    bk: list
    bv: list
    lk_ptrs: torch.Tensor  # pointer tables: None for a projection without an adapter
    lv_ptrs: torch.Tensor
    bk_ptrs: torch.Tensor
    bv_ptrs: torch.Tensor
    ranks: torch.Tensor  # None without any adapter
    cu_q_lens: torch.Tensor
    max_context_len: int
    max_q_len: int
    max_rank: int

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.w.dtype == "bf16" else torch.float32

    def new_out(self):
        return torch.empty(self.q.shape, dtype=self.torch_dtype, device=self.q.device)


def upload(w: Workload, device="cuda", poison: bool = False, host_pools=None) -> DeviceWorkload:
    dev = torch.device(device)
    kpool, vpool, lkp, lvp = host_pools if host_pools is not None else w.host_pools(poison=poison)
    conv = _u16 if w.dtype == "bf16" else (lambda x: x)
    k_base = _t(conv(kpool), dev, w.dtype)
    v_base = _t(conv(vpool), dev, w.dtype)
    lk_pools = [_t(conv(p), dev, w.dtype) for p in lkp]
    lv_pools = [_t(conv(p), dev, w.dtype) for p in lvp]
    ads = w.host_adapters()
    bk = [_t(conv(a[0]), dev, w.dtype) for a in ads]
    bv = [_t(conv(a[1]), dev, w.dtype) for a in ads]
    q = _t(conv(w.host_q()), dev, w.dtype)
    i32 = lambda x: torch.tensor(np.asarray(x, dtype=np.int32), device=dev)  # noqa: E731
    ptrs = lambda ts: torch.tensor([t.data_ptr() for t in ts], dtype=torch.int64, device=dev)  # noqa: E731
    lk_of_agent = [lk_pools[w.pool_of_agent[a]] for a in range(w.n_agents)]
    lv_of_agent = [lv_pools[w.pool_of_agent[a]] for a in range(w.n_agents)]
    ctx = [w.context_len(s) for s in range(w.S)]
    adapted = w.has_k or w.has_v
    # a projection without an adapter passes NULL pointer tables; with no
    # adapter at all the agent ids and ranks are not passed either
    return DeviceWorkload(
        w=w, q=q, k_base=k_base, v_base=v_base,
        block_tables=i32(w.block_tables()), context_lens=i32(ctx),
        group_offsets=i32(w.group_offsets) if w.group_offsets is not None else None,
        agent_ids=i32([sq.agent for sq in w.seqs]) if adapted else None,
        adapter_start=(i32([sq.adapter_start for sq in w.seqs])
                       if adapted and any(sq.adapter_start for sq in w.seqs) else None),
        lk_pools=lk_pools, lv_pools=lv_pools, bk=bk, bv=bv,
        lk_ptrs=ptrs(lk_of_agent) if w.has_k else None, lv_ptrs=ptrs(lv_of_agent) if w.has_v else None,
        bk_ptrs=ptrs(bk) if w.has_k else None, bv_ptrs=ptrs(bv) if w.has_v else None,
        ranks=i32(w.ranks) if adapted else None, cu_q_lens=i32(w.q_offsets()),
        max_context_len=max(ctx), max_q_len=max(sq.q_len for sq in w.seqs),
        max_rank=max(w.ranks) if adapted else 0,
    )
