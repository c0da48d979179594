"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
catch every one: a pin set that lets a dropped term, a wrong sign or index,
or a transposed operand through is too weak."""
import numpy as np
import pytest

from oracle import lra_oracle as O
from tests.oracle_pins import ALL_PINS

_orig_rope = O.rope_rotate
_orig_attend = O.attend
_orig_adapter = O.adapter_term
_orig_mat = O.materialise_kv
_orig_multi = O.lr_cache_build_multi


def _rope_sign(x, positions, theta):
    return _orig_rope(x, -np.asarray(positions), theta)


def _rope_pos_shift(x, positions, theta):
    return _orig_rope(x, np.asarray(positions) + 1, theta)


def _rope_adjacent_pairs(x, positions, theta):
    x = np.asarray(x, np.float64)
    if theta == 0:
        return x.copy()
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    return _orig_rope(x[..., perm], positions, theta)[..., inv]


def _rope_freq(x, positions, theta):
    x = np.asarray(x, np.float64)
    if theta == 0:
        return x.copy()
    d = x.shape[-1]
    ang = np.asarray(positions, np.float64)[:, None] * np.power(theta, -np.arange(d // 2) / d)[None, :]
    shape = (ang.shape[0],) + (1,) * (x.ndim - 2) + (d // 2,)
    c, s = np.cos(ang).reshape(shape), np.sin(ang).reshape(shape)
    x1, x2 = x[..., : d // 2], x[..., d // 2 :]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def _adapter_head_major(l_rows, b, Hkv, d):
    return (np.asarray(l_rows) @ np.asarray(b)).reshape(-1, d, Hkv).transpose(0, 2, 1)


def _drop_v_adapter(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    K, _ = _orig_mat(kb, vb, lk, lv, bk, bv, theta, adapter_start)
    return K, np.asarray(vb, np.float64).copy()


def _drop_k_adapter(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    _, V = _orig_mat(kb, vb, lk, lv, bk, bv, theta, adapter_start)
    return np.asarray(kb, np.float64).copy(), V


def _rope_on_v_too(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    K, V = _orig_mat(kb, vb, lk, lv, bk, bv, theta, adapter_start)
    T, Hkv, d = kb.shape
    v_ad = V - vb
    return K, vb + O.rope_rotate(v_ad, np.arange(T), theta)


def _absent_key_drops_value(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    K, V = _orig_mat(kb, vb, lk, lv, bk, bv, theta, adapter_start)
    return K, (np.asarray(vb, np.float64).copy() if bk is None else V)


def _absent_key_rotates_base(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    K, V = _orig_mat(kb, vb, lk, lv, bk, bv, theta, adapter_start)
    if bk is None:
        K = O.rope_rotate(np.asarray(kb, np.float64), np.arange(kb.shape[0]), theta)
    return K, V


def _absent_value_drops_key(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    K, V = _orig_mat(kb, vb, lk, lv, bk, bv, theta, adapter_start)
    return (np.asarray(kb, np.float64).copy() if bv is None else K), V


def _start_off_by_one(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    return _orig_mat(kb, vb, lk, lv, bk, bv, theta, adapter_start + 1 if adapter_start else 0)


def _start_keys_only(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    K, _ = _orig_mat(kb, vb, lk, lv, bk, bv, theta, adapter_start)
    _, V = _orig_mat(kb, vb, lk, lv, bk, bv, theta, 0)
    return K, V


def _start_shifts_rotation(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    T, Hkv, d = kb.shape
    K, V = _orig_mat(kb, vb, lk, lv, bk, bv, theta, adapter_start)
    if bk is not None and adapter_start:
        a = adapter_start
        k_ad = O.adapter_term(lk, bk, Hkv, d)[a:]
        K = K.copy()
        K[a:] = np.asarray(kb, np.float64)[a:] + O.rope_rotate(k_ad, np.arange(T - a), theta)
    return K, V


def _base_updated_in_place(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    """Adds the adapter terms into the caller's base arrays (an aliasing
    mistake: the next agent over the same base sees this agent's terms)."""
    K, V = _orig_mat(kb, vb, lk, lv, bk, bv, theta, adapter_start)
    if isinstance(kb, np.ndarray) and kb.dtype == np.float64:
        kb += K - kb
        vb += V - vb
        return kb, vb
    return K, V


def _value_adapter_rank_reversed(kb, vb, lk, lv, bk, bv, theta, adapter_start=0):
    """Pairs rank k of L_v with row r-1-k of B_v (a transposed operand)."""
    return _orig_mat(kb, vb, lk, lv, bk, None if bv is None else np.asarray(bv)[::-1], theta, adapter_start)


def _adapter_head_swapped(l_rows, b, Hkv, d):
    """Feeds KV head h from the columns of head Hkv-1-h."""
    return _orig_adapter(l_rows, b, Hkv, d)[:, ::-1, :]


def _gqa_modulo(j, Hq, Hkv):
    return j % Hkv


def _causal_exclusive(q, positions, K, V, sm_scale):
    return _orig_attend(q, np.maximum(np.asarray(positions) - 1, 0), K, V, sm_scale)


def _no_scale(q, positions, K, V, sm_scale):
    return _orig_attend(q, positions, K, V, 1.0)


def _multi_shifted(X, A, group_cols):
    L = _orig_multi(X, A, group_cols)
    return [L[0]] + [np.roll(P, 1, axis=1) for P in L[1:]]


def _build_transposed(X, A):
    return (np.asarray(A, np.float64).T @ np.asarray(X, np.float64).T).T[:, ::-1]


MUTATIONS = {
    "rope_sign": ("rope_rotate", _rope_sign),
    "rope_position_shift": ("rope_rotate", _rope_pos_shift),
    "rope_adjacent_pairs": ("rope_rotate", _rope_adjacent_pairs),
    "rope_frequency_exponent": ("rope_rotate", _rope_freq),
    "adapter_head_major_columns": ("adapter_term", _adapter_head_major),
    "drop_value_adapter": ("materialise_kv", _drop_v_adapter),
    "drop_key_adapter": ("materialise_kv", _drop_k_adapter),
    "rotate_value_adapter": ("materialise_kv", _rope_on_v_too),
    "absent_key_adapter_drops_value_adapter": ("materialise_kv", _absent_key_drops_value),
    "absent_key_adapter_rotates_base_keys": ("materialise_kv", _absent_key_rotates_base),
    "absent_value_adapter_drops_key_adapter": ("materialise_kv", _absent_value_drops_key),
    "adapter_start_off_by_one": ("materialise_kv", _start_off_by_one),
    "adapter_start_on_keys_only": ("materialise_kv", _start_keys_only),
    "adapter_start_rotation_relative": ("materialise_kv", _start_shifts_rotation),
    "gqa_modulo_mapping": ("kv_head_of", _gqa_modulo),
    "base_updated_in_place": ("materialise_kv", _base_updated_in_place),
    "value_adapter_rank_reversed": ("materialise_kv", _value_adapter_rank_reversed),
    "adapter_heads_swapped": ("adapter_term", _adapter_head_swapped),
    "causal_off_by_one": ("attend", _causal_exclusive),
    "missing_softmax_scale": ("attend", _no_scale),
    "build_columns_reversed": ("lr_cache_build", _build_transposed),
    "multi_build_group_columns_shifted": ("lr_cache_build_multi", _multi_shifted),
}


def _failing_pins(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(O)
        except AssertionError:
            failed.append(pin.__name__)
    return failed


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    assert _failing_pins(name, monkeypatch), f"no pin catches mutation {name}"


# pins that must each catch a particular planted mistake on their own
OWN_CATCH = [
    ("pin_reorder_equals_materialised", "value_adapter_rank_reversed"),
    ("pin_reorder_equals_materialised", "rotate_value_adapter"),
    ("pin_shared_base_unchanged", "base_updated_in_place"),
    ("pin_bruteforce_tiny", "adapter_heads_swapped"),
    ("pin_bruteforce_tiny", "adapter_head_major_columns"),
]


@pytest.mark.parametrize("pin,name", OWN_CATCH, ids=[f"{p}-{m}" for p, m in OWN_CATCH])
def test_pin_catches_its_mutation(pin, name, monkeypatch):
    assert pin in _failing_pins(name, monkeypatch)
