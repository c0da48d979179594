"""The C-ABI library on the host: it loads, exports every symbol the header
declares, and rejects bad arguments before any HIP call (so these run
without a GPU). Fake device addresses are never dereferenced: each call
fails validation first."""
import ctypes
import os
import re

import pytest

import shared_base_kv_amd as lra
from shared_base_kv_amd import binding as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "lra.h")
FAKE = 0x10000  # 16-byte aligned, never touched


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b([a-z_0-9]+)\s*\(", src)) - {"defined"})


def test_exports_every_declared_symbol():
    lib = lra.load()
    names = _declared()
    assert set(names) == set(B.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_version_matches_header():
    m = re.search(r"#define LRA_VERSION (\d+)", open(HEADER).read())
    assert lra.lra_version() == int(m.group(1))


def _decode(**over):
    args = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, max_blocks=512, ctx=FAKE, max_ctx=8192, go=FAKE, ng=1, ag=FAKE,
                act=None, lk=FAKE, lv=FAKE, bk=FAKE, bv=FAKE, ranks=FAKE, max_rank=16, S=4, NA=4, Hq=32, Hkv=8, d=128, bs=16,
                sc=0.088, theta=5e5, dtype=lra.LRA_BF16, out=FAKE, ws=FAKE, wsb=1 << 30, stream=None)
    args.update(over)
    rc = lra.load().lora_attn_decode(*args.values())
    return rc, lra.lra_last_error()


@pytest.mark.parametrize("over,code,frag", [
    (dict(q=None), B.LRA_ERR_INVALID_ARG, "null"),
    (dict(out=None), B.LRA_ERR_INVALID_ARG, "null"),
    (dict(q=FAKE + 2), B.LRA_ERR_INVALID_ARG, "aligned"),
    (dict(Hq=30), B.LRA_ERR_INVALID_ARG, "multiple"),
    (dict(Hq=8 * 17), B.LRA_ERR_UNSUPPORTED, "16 query heads"),
    (dict(Hq=65536, Hkv=65536), B.LRA_ERR_UNSUPPORTED, "65535 KV heads"),
    (dict(d=64), B.LRA_ERR_UNSUPPORTED, "d = 128"),
    (dict(dtype=7), B.LRA_ERR_UNSUPPORTED, "dtype"),
    (dict(max_rank=65), B.LRA_ERR_UNSUPPORTED, "max_rank"),
    (dict(max_rank=0), B.LRA_ERR_INVALID_ARG, "max_rank"),
    (dict(max_rank=-1), B.LRA_ERR_UNSUPPORTED, "max_rank"),
    (dict(bk=None, bv=None), B.LRA_ERR_INVALID_ARG, "max_rank must be 0"),
    (dict(lk=None), B.LRA_ERR_INVALID_ARG, "l_k_pools"),
    (dict(bk=None, lk=None, lv=None), B.LRA_ERR_INVALID_ARG, "l_v_pools"),
    (dict(ag=None), B.LRA_ERR_INVALID_ARG, "agent_ids"),
    (dict(bv=None, ranks=None), B.LRA_ERR_INVALID_ARG, "ranks"),
    # without adapters the agent and low-rank arguments may be NULL: the
    # call gets past them to the workspace check
    (dict(bk=None, bv=None, lk=None, lv=None, ag=None, ranks=None, max_rank=0, NA=0, wsb=100),
     B.LRA_ERR_WORKSPACE, "workspace"),
    (dict(bk=None, lk=None, wsb=100), B.LRA_ERR_WORKSPACE, "workspace"),
    (dict(bs=32), B.LRA_ERR_UNSUPPORTED, "block_size"),
    (dict(max_blocks=10), B.LRA_ERR_INVALID_ARG, "max_blocks"),
    (dict(ng=5), B.LRA_ERR_INVALID_ARG, "num_groups"),
    (dict(NA=0), B.LRA_ERR_INVALID_ARG, "N_agents"),
    (dict(wsb=100), B.LRA_ERR_WORKSPACE, "workspace"),
    (dict(ws=None), B.LRA_ERR_WORKSPACE, "workspace"),
    (dict(theta=-1.0), B.LRA_ERR_INVALID_ARG, "rope_theta"),
    (dict(sc=float("inf")), B.LRA_ERR_INVALID_ARG, "sm_scale"),
])
def test_decode_rejects_bad_arguments(over, code, frag):
    rc, msg = _decode(**over)
    assert rc == code, msg
    assert frag in msg


def test_empty_batch_is_a_no_op():
    rc, msg = _decode(S=0)
    assert rc == B.LRA_OK and msg == ""


def test_decode_workspace_is_small_and_bounded():
    """Workspace holds split partials only: O(splits * rows * (d + r + 4))
    floats, bounded as the context grows, never O(T * d)."""
    f = lra.lora_attn_decode_workspace_size
    small = f(4, 1, 32, 8, 128, 16, 8192, lra.LRA_BF16)
    assert 0 < small < 8 * 1024 * 1024
    sizes = [f(8, 1, 32, 8, 128, 64, T, lra.LRA_BF16) for T in (4096, 32768, 1 << 20, 1 << 24)]
    bound = 8 * 2 * 64 * 16 * (4 + 128) * 4
    assert max(sizes) <= bound
    assert sizes[-1] < (1 << 24) * 128 * 2
    assert f(4, 1, 32, 8, 128, 16, 8192, lra.LRA_F32) == 0  # fp32 path has no split
    assert f(4, 1, 30, 8, 128, 16, 8192, lra.LRA_BF16) == 0  # invalid sizes -> 0
    assert f(4, 1, 32, 8, 128, 0, 8192, lra.LRA_BF16) == small  # no adapter plans as rank 16


def test_build_rejects_bad_arguments():
    lib = lra.load()
    call = lambda **o: lib.lr_cache_build(*dict(dict(X=FAKE, ldx=4096, A=FAKE, lda=16, L=FAKE, ldl=16, slot=None,  # noqa: E731
                                                     lay=0, n=512, hidden=4096, ncols=16, dtype=lra.LRA_BF16,
                                                     ws=FAKE, wsb=1 << 30, stream=None), **o).values())
    assert call(dtype=lra.LRA_F32) == B.LRA_ERR_UNSUPPORTED
    assert call(X=None) == B.LRA_ERR_INVALID_ARG
    assert call(hidden=4100, ldx=4100) == B.LRA_ERR_UNSUPPORTED
    assert call(ncols=600, lda=600, ldl=600) == B.LRA_ERR_UNSUPPORTED
    assert call(lay=1) == B.LRA_ERR_INVALID_ARG  # rank-major needs a slot mapping
    assert call(ldl=8) == B.LRA_ERR_INVALID_ARG
    assert call(n=0) == B.LRA_OK
    assert call(ws=None) == B.LRA_ERR_WORKSPACE  # hidden 4096 is summed in 8 slices
    assert call(wsb=4096) == B.LRA_ERR_WORKSPACE


def test_build_workspace_size():
    """Counters (4096 bytes) plus one fp32 16x16 partial per tile and slice of
    512 hidden values; nothing when the hidden size fits one slice."""
    f = lra.lr_cache_build_workspace_size
    assert f(512, 4096, 16) == 4096 + 32 * 1 * 8 * 1024
    assert f(512, 4096, 128) == 4096 + 32 * 8 * 8 * 1024
    assert f(37, 520, 8) == 4096 + 3 * 1 * 2 * 1024
    assert f(5000, 512, 16) == 0 and f(1, 8, 1) == 0
    # at most 1024 tiles' partials (larger builds run in several launches)
    assert f(1 << 16, 4096, 512) == 4096 + 1024 * 8 * 1024
    assert f(-1, 4096, 16) == 0 and f(4, 4096, 600) == 0


def test_prefill_rejects_bad_arguments():
    lib = lra.load()
    base = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, max_blocks=600, ctx=FAKE, max_ctx=8704, cu=FAKE, mq=512, ag=FAKE,
                act=None, lk=FAKE, lv=FAKE, bk=FAKE, bv=FAKE, ranks=FAKE, max_rank=16, S=4, NA=4, Hq=32, Hkv=8, d=128, bs=16,
                sc=0.088, theta=5e5, dtype=lra.LRA_BF16, out=FAKE, ws=None, wsb=0, stream=None)
    call = lambda **o: lib.lora_attn_prefill(*dict(base, **o).values())  # noqa: E731
    assert call(dtype=lra.LRA_F32) == B.LRA_ERR_UNSUPPORTED
    assert call(cu=None) == B.LRA_ERR_INVALID_ARG
    assert call(mq=0) == B.LRA_ERR_INVALID_ARG
    assert call(mq=9000) == B.LRA_ERR_INVALID_ARG
    assert call(S=0) == B.LRA_OK
    assert call(bk=None, bv=None) == B.LRA_ERR_INVALID_ARG  # max_rank must be 0 without adapters
    assert call(bv=None, lv=None, lk=None) == B.LRA_ERR_INVALID_ARG
    assert call(ag=None) == B.LRA_ERR_INVALID_ARG


def test_multi_build_rejects_bad_group_tables():
    import ctypes

    lib = lra.load()

    def call(cols=(0, 16, 32), pools=(FAKE, FAKE), lays=(0, 1), slot=FAKE, ncols=32, **o):
        ng = len(pools)
        c = (ctypes.c_int32 * len(cols))(*cols)
        p = (ctypes.c_void_p * ng)(*pools)
        la = (ctypes.c_int32 * len(lays))(*lays)
        args = dict(X=FAKE, ldx=4096, A=FAKE, lda=ncols, ng=o.pop("ng", ng), cols=c, pools=p, lays=la, slot=slot,
                    n=512, hidden=4096, ncols=ncols, dtype=lra.LRA_BF16, ws=FAKE, wsb=o.pop("wsb", 1 << 30),
                    stream=None)
        args.update(o)
        return lib.lr_cache_build_multi(*args.values())

    assert call(cols=(0, 16, 30)) == B.LRA_ERR_INVALID_ARG  # does not end at n_cols
    assert call(cols=(0, 0, 32)) == B.LRA_ERR_INVALID_ARG  # empty group
    assert call(pools=(FAKE, None)) == B.LRA_ERR_INVALID_ARG
    assert call(lays=(0, 5)) == B.LRA_ERR_INVALID_ARG
    assert call(slot=None) == B.LRA_ERR_INVALID_ARG
    assert call(ng=0) == B.LRA_ERR_UNSUPPORTED
    assert call(ng=65) == B.LRA_ERR_UNSUPPORTED
    assert call(dtype=lra.LRA_F32) == B.LRA_ERR_UNSUPPORTED
    assert call(n=0) == B.LRA_OK



def test_varlen_rejects_bad_arguments():
    """The mixed decode + prefill call validates both parts before launching;
    every case here fails (or is a no-op) on the host without touching memory."""
    lib = lra.load()
    base = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, max_blocks=600, ctx=FAKE, max_ctx=8704, cu=FAKE, mq=512, S=8,
                S_dec=4, go=FAKE, ng=1, ag=FAKE, act=None, lk=FAKE, lv=FAKE, bk=FAKE, bv=FAKE, ranks=FAKE,
                max_rank=16, NA=4, Hq=32, Hkv=8, d=128, bs=16, sc=0.088, theta=5e5, dtype=lra.LRA_BF16, out=FAKE,
                ws=FAKE, wsb=1 << 30, stream=None)
    call = lambda **o: lib.lora_attn_varlen(*dict(base, **o).values())  # noqa: E731
    assert call(S_dec=9) == B.LRA_ERR_INVALID_ARG
    assert call(S_dec=-1) == B.LRA_ERR_INVALID_ARG
    assert call(dtype=lra.LRA_F32) == B.LRA_ERR_UNSUPPORTED
    assert call(ng=5) == B.LRA_ERR_INVALID_ARG  # more groups than decode sequences
    assert call(cu=None) == B.LRA_ERR_INVALID_ARG  # prefill part without cu_q_lens
    assert call(mq=0) == B.LRA_ERR_INVALID_ARG
    assert call(wsb=100) == B.LRA_ERR_WORKSPACE  # the decode part's split records
    assert call(q=FAKE + 2) == B.LRA_ERR_INVALID_ARG
    assert call(bs=32) == B.LRA_ERR_UNSUPPORTED
    assert call(bk=None, bv=None) == B.LRA_ERR_INVALID_ARG  # max_rank must be 0 without adapters
    assert call(S=0, S_dec=0) == B.LRA_OK
    f = lra.lora_attn_varlen_workspace_size
    assert f(8, 4, 1, 32, 8, 128, 16, 8192, lra.LRA_BF16) == lra.lora_attn_decode_workspace_size(
        4, 1, 32, 8, 128, 16, 8192, lra.LRA_BF16)
    assert f(8, 0, 1, 32, 8, 128, 16, 8192, lra.LRA_BF16) == 0  # prefill only: no split records
    assert f(8, 9, 1, 32, 8, 128, 16, 8192, lra.LRA_BF16) == 0


def test_debug_library_exports_and_validates_like_release():
    """liblra_debug.so (the same kernels, device-side input checks) exports
    every declared symbol and rejects bad host arguments exactly as liblra.so
    does, before any HIP call."""
    dbg = B.load_debug()
    for n in _declared():
        assert hasattr(dbg, n), n
    assert dbg.lra_version() == lra.lra_version()
    for over in (dict(q=None), dict(Hq=30), dict(d=64), dict(max_rank=65), dict(lk=None)):
        args = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, max_blocks=512, ctx=FAKE, max_ctx=8192, go=FAKE, ng=1, ag=FAKE,
                    act=None, lk=FAKE, lv=FAKE, bk=FAKE, bv=FAKE, ranks=FAKE, max_rank=16, S=4, NA=4, Hq=32, Hkv=8,
                    d=128, bs=16, sc=0.088, theta=5e5, dtype=lra.LRA_BF16, out=FAKE, ws=FAKE, wsb=1 << 30,
                    stream=None)
        args.update(over)
        rc_r = lra.load().lora_attn_decode(*args.values())
        rc_d = dbg.lora_attn_decode(*args.values())
        assert rc_r == rc_d != 0, over
        assert lra.lra_last_error() == dbg.lra_last_error().decode(), over


def test_decode_noalloc_rejects_before_any_hip_call():
    """The allocation-free decode checks its arguments as lora_attn_decode
    does, and rejects a call whose split records exceed its fixed 16 MiB
    array, all before any HIP call (fake addresses are never touched)."""
    lib = lra.load()
    base = dict(q=FAKE, k=FAKE, v=FAKE, bt=FAKE, max_blocks=2048, ctx=FAKE, max_ctx=32768, go=None, ng=64, ag=FAKE,
                act=None, lk=FAKE, lv=FAKE, bk=FAKE, bv=FAKE, ranks=FAKE, max_rank=64, S=64, NA=16, Hq=32, Hkv=8, d=128,
                bs=16, sc=0.088, theta=5e5, dtype=lra.LRA_BF16, out=FAKE, stream=None)
    call = lambda **o: (lib.lora_attn_decode_noalloc(*dict(base, **o).values()), lra.lra_last_error())  # noqa: E731
    need = lra.lora_attn_decode_workspace_size(64, 64, 32, 8, 128, 64, 32768, lra.LRA_BF16)
    assert need > 16 << 20
    rc, msg = call()
    assert rc == B.LRA_ERR_UNSUPPORTED and "fixed scratch" in msg, msg
    rc, msg = call(q=None, S=4, ng=4, max_ctx=8192)
    assert rc == B.LRA_ERR_INVALID_ARG and "null" in msg, msg
    rc, msg = call(Hq=30, S=4, ng=4, max_ctx=8192)
    assert rc == B.LRA_ERR_INVALID_ARG, msg
