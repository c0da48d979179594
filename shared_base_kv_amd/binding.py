"""ctypes binding of liblra.so (include/lra.h). Argument marshalling only.

Functions keep the C names. Device buffers may be torch tensors (their
data_ptr() is passed) or integer device addresses. ``stream`` defaults to
torch's current stream on the current device. Every failure raises
``LraError`` with the library's message; there is no fallback path: if the
library is not built, loading raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblra.so")
# the same kernels with the device-side input checks (LRA_DEBUG_CHECKS)
DEBUG_LIB_PATH = os.path.join(HERE, "liblra_debug.so")

LRA_OK = 0
LRA_ERR_INVALID_ARG = -1
LRA_ERR_UNSUPPORTED = -2
LRA_ERR_WORKSPACE = -3
LRA_ERR_LAUNCH = -4
LRA_F32 = 0
LRA_BF16 = 1
LRA_L_TOKEN_MAJOR = 0
LRA_L_RANK_MAJOR = 1
LRA_L_KEY_CHUNKED = 2

EXPORTS = (
    "lra_version",
    "lra_last_error",
    "lr_cache_build_workspace_size",
    "lr_cache_build",
    "lr_cache_build_multi",
    "lora_attn_decode_workspace_size",
    "lora_attn_decode",
    "lora_attn_decode_noalloc",
    "lora_attn_prefill_workspace_size",
    "lora_attn_prefill",
    "lora_attn_varlen_workspace_size",
    "lora_attn_varlen",
)


class LraError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"lra error {code}: {msg}")
        self.code = code


_lib = None
_p = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_f32 = ctypes.c_float
_sz = ctypes.c_size_t


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """The library every wrapper below calls (loaded once)."""
    global _lib
    if _lib is None:
        _lib = _open(path)
    return _lib


_dlib = None


def load_debug() -> ctypes.CDLL:
    """liblra_debug.so, for direct C calls: each attention call first checks
    the device-side inputs (and synchronises its stream). The wrappers below
    keep using load()."""
    global _dlib
    if _dlib is None:
        _dlib = _open(DEBUG_LIB_PATH)
    return _dlib


def _open(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run python -m shared_base_kv_amd.build")
    lib = ctypes.CDLL(path)
    lib.lra_version.restype = ctypes.c_int
    lib.lra_version.argtypes = []
    lib.lra_last_error.restype = ctypes.c_char_p
    lib.lra_last_error.argtypes = []
    lib.lr_cache_build_workspace_size.restype = _sz
    lib.lr_cache_build_workspace_size.argtypes = [_i32, _i32, _i32]
    lib.lr_cache_build.restype = ctypes.c_int
    lib.lr_cache_build.argtypes = [_p, _i64, _p, _i64, _p, _i64, _p, _i32, _i32, _i32, _i32, _i32, _p, _sz, _p]
    lib.lr_cache_build_multi.restype = ctypes.c_int
    lib.lr_cache_build_multi.argtypes = [_p, _i64, _p, _i64, _i32, _p, _p, _p, _p, _i32, _i32, _i32, _i32, _p, _sz, _p]
    size8 = [_i32] * 8
    lib.lora_attn_decode_workspace_size.restype = _sz
    lib.lora_attn_decode_workspace_size.argtypes = size8
    attn = [_p, _p, _p, _p, _i32, _p, _i32, _p, _i32, _p, _p, _p, _p, _p, _p, _p, _i32, _i32, _i32,
            _i32, _i32, _i32, _i32, _f32, _f32, _i32, _p, _p, _sz, _p]
    lib.lora_attn_decode.restype = ctypes.c_int
    lib.lora_attn_decode.argtypes = attn
    lib.lora_attn_decode_noalloc.restype = ctypes.c_int
    lib.lora_attn_decode_noalloc.argtypes = attn[:-3] + [_p]  # no workspace, workspace_bytes
    lib.lora_attn_prefill_workspace_size.restype = _sz
    lib.lora_attn_prefill_workspace_size.argtypes = size8
    lib.lora_attn_prefill.restype = ctypes.c_int
    lib.lora_attn_prefill.argtypes = attn
    lib.lora_attn_varlen_workspace_size.restype = _sz
    lib.lora_attn_varlen_workspace_size.argtypes = [_i32] * 9
    lib.lora_attn_varlen.restype = ctypes.c_int
    lib.lora_attn_varlen.argtypes = [_p, _p, _p, _p, _i32, _p, _i32, _p, _i32, _i32, _i32, _p, _i32, _p, _p, _p, _p,
                                     _p, _p, _p, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _f32, _i32, _p, _p, _sz, _p]
    return lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch

    return torch.cuda.current_stream().cuda_stream


def _check(rc: int):
    if rc != LRA_OK:
        raise LraError(rc, load().lra_last_error().decode())


def _dtype_code(t) -> int:
    import torch

    if t.dtype == torch.bfloat16:
        return LRA_BF16
    if t.dtype == torch.float32:
        return LRA_F32
    raise LraError(LRA_ERR_UNSUPPORTED, f"dtype {t.dtype}")


def lra_version() -> int:
    return load().lra_version()


def lra_last_error() -> str:
    return load().lra_last_error().decode()


def lr_cache_build_workspace_size(n_tokens: int, hidden: int, n_cols: int) -> int:
    return load().lr_cache_build_workspace_size(n_tokens, hidden, n_cols)


def lr_cache_build(X, A, L, workspace, *, slot_mapping=None, l_layout=LRA_L_TOKEN_MAJOR, ldl=None, n_cols=None,
                   stream=None):
    """L = X A. X [n, hidden] and A [hidden, n_cols] bf16 tensors (row strides
    taken from the tensors); L a bf16 tensor: dense [n, >=n_cols] or a paged
    pool addressed through ``slot_mapping`` (int64 [n]). ``workspace``: at
    least lr_cache_build_workspace_size(n, hidden, n_cols) bytes, zero-filled
    before its first use (each call leaves its counters zero again)."""
    n, hidden = X.shape
    n_cols = A.shape[1] if n_cols is None else n_cols
    if ldl is None:
        ldl = L.stride(0) if (slot_mapping is None or l_layout == LRA_L_TOKEN_MAJOR) and L.dim() == 2 else n_cols
    _check(load().lr_cache_build(_ptr(X), X.stride(0), _ptr(A), A.stride(0), _ptr(L), ldl, _ptr(slot_mapping),
                                 l_layout, n, hidden, n_cols, _dtype_code(X), _ptr(workspace),
                                 workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                 _stream(stream)))


def lr_cache_build_multi(X, A, group_cols, group_pools, group_layouts, slot_mapping, workspace, stream=None):
    """Every group's low-rank rows from one pass over X: columns
    group_cols[g]:group_cols[g+1] of X A go to pool group_pools[g] (a bf16
    tensor or device address) in layout group_layouts[g], through the int64
    slot mapping. X [n, hidden] and A [hidden, n_cols] bf16 tensors."""
    n, hidden = X.shape
    ng = len(group_pools)
    cols = (ctypes.c_int32 * (ng + 1))(*group_cols)
    pools = (ctypes.c_void_p * ng)(*[_ptr(p) for p in group_pools])
    lays = (ctypes.c_int32 * ng)(*group_layouts)
    _check(load().lr_cache_build_multi(_ptr(X), X.stride(0), _ptr(A), A.stride(0), ng, cols, pools, lays,
                                       _ptr(slot_mapping), n, hidden, int(group_cols[-1]), _dtype_code(X),
                                       _ptr(workspace),
                                       workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                       _stream(stream)))


def lora_attn_decode_workspace_size(S, num_groups, Hq, Hkv, d, max_rank, max_context_len, dtype) -> int:
    return load().lora_attn_decode_workspace_size(S, num_groups, Hq, Hkv, d, max_rank, max_context_len, dtype)


def lora_attn_decode(q, k_base, v_base, block_tables, context_lens, max_context_len, group_offsets, agent_ids,
                     l_k_pools, l_v_pools, b_k, b_v, ranks, max_rank, n_agents, Hkv, sm_scale, rope_theta, out,
                     workspace, stream=None, adapter_start=None):
    """Decode step. q/out [S, Hq, d]; pools and tables as in include/lra.h;
    l_k_pools, l_v_pools, b_k, b_v are int64 device tensors of addresses
    (None: that adapter is absent); adapter_start an int32 [S] tensor or None."""
    S, Hq, d = q.shape
    num_groups = (group_offsets.numel() - 1) if group_offsets is not None else S
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().lora_attn_decode(
        _ptr(q), _ptr(k_base), _ptr(v_base), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        max_context_len, _ptr(group_offsets), num_groups, _ptr(agent_ids), _ptr(adapter_start), _ptr(l_k_pools),
        _ptr(l_v_pools),
        _ptr(b_k), _ptr(b_v), _ptr(ranks), max_rank, S, n_agents, Hq, Hkv, d, 16, sm_scale, rope_theta,
        _dtype_code(q), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


def lora_attn_decode_noalloc(q, k_base, v_base, block_tables, context_lens, max_context_len, group_offsets, agent_ids,
                             l_k_pools, l_v_pools, b_k, b_v, ranks, max_rank, n_agents, Hkv, sm_scale, rope_theta, out,
                             stream=None, adapter_start=None):
    """lora_attn_decode without a workspace: the split records go to the
    library's fixed 16 MiB device array (calls overlapping on one GPU race)."""
    S, Hq, d = q.shape
    num_groups = (group_offsets.numel() - 1) if group_offsets is not None else S
    _check(load().lora_attn_decode_noalloc(
        _ptr(q), _ptr(k_base), _ptr(v_base), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        max_context_len, _ptr(group_offsets), num_groups, _ptr(agent_ids), _ptr(adapter_start), _ptr(l_k_pools),
        _ptr(l_v_pools), _ptr(b_k), _ptr(b_v), _ptr(ranks), max_rank, S, n_agents, Hq, Hkv, d, 16, sm_scale,
        rope_theta, _dtype_code(q), _ptr(out), _stream(stream)))


def lora_attn_prefill_workspace_size(S, Hq, Hkv, d, max_rank, max_q_len, max_context_len, dtype) -> int:
    return load().lora_attn_prefill_workspace_size(S, Hq, Hkv, d, max_rank, max_q_len, max_context_len, dtype)


def lora_attn_prefill(q, k_base, v_base, block_tables, context_lens, max_context_len, cu_q_lens, max_q_len,
                      agent_ids, l_k_pools, l_v_pools, b_k, b_v, ranks, max_rank, n_agents, Hkv, sm_scale,
                      rope_theta, out, workspace=None, stream=None, adapter_start=None):
    """Prefill chunks. q/out [sum q_len, Hq, d]; cu_q_lens int32 [S+1]."""
    _, Hq, d = q.shape
    S = cu_q_lens.numel() - 1
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().lora_attn_prefill(
        _ptr(q), _ptr(k_base), _ptr(v_base), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        max_context_len, _ptr(cu_q_lens), max_q_len, _ptr(agent_ids), _ptr(adapter_start), _ptr(l_k_pools),
        _ptr(l_v_pools),
        _ptr(b_k), _ptr(b_v), _ptr(ranks), max_rank, S, n_agents, Hq, Hkv, d, 16, sm_scale, rope_theta,
        _dtype_code(q), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))


def lora_attn_varlen_workspace_size(S, S_dec, num_groups, Hq, Hkv, d, max_rank, max_context_len, dtype) -> int:
    return load().lora_attn_varlen_workspace_size(S, S_dec, num_groups, Hq, Hkv, d, max_rank, max_context_len, dtype)


def lora_attn_varlen(q, k_base, v_base, block_tables, context_lens, max_context_len, cu_q_lens, max_q_len, S_dec,
                     group_offsets, agent_ids, l_k_pools, l_v_pools, b_k, b_v, ranks, max_rank, n_agents, Hkv,
                     sm_scale, rope_theta, out, workspace, stream=None, adapter_start=None):
    """Decode rows (sequences 0 .. S_dec - 1, one query row each) and prefill
    chunks (the rest) in one launch. q/out [cu_q_lens[S], Hq, d]; cu_q_lens
    int32 [S+1] over all sequences (cu_q_lens[s] = s for s <= S_dec);
    group_offsets over the decode sequences or None."""
    _, Hq, d = q.shape
    S = cu_q_lens.numel() - 1
    num_groups = (group_offsets.numel() - 1) if group_offsets is not None else S_dec
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().lora_attn_varlen(
        _ptr(q), _ptr(k_base), _ptr(v_base), _ptr(block_tables), block_tables.shape[1], _ptr(context_lens),
        max_context_len, _ptr(cu_q_lens), max_q_len, S, S_dec, _ptr(group_offsets), num_groups, _ptr(agent_ids),
        _ptr(adapter_start), _ptr(l_k_pools), _ptr(l_v_pools), _ptr(b_k), _ptr(b_v), _ptr(ranks), max_rank, n_agents,
        Hq, Hkv, d, 16, sm_scale, rope_theta, _dtype_code(q), _ptr(out), _ptr(workspace), ws_bytes, _stream(stream)))
