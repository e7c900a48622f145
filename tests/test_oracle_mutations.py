"""Planted mistakes in the CPU oracle must each fail at least one pin.

Each mutation replaces one piece of ``oracle.qift_oracle`` (on the CPU, via
monkeypatch) with a plausible slip: a wrong sign or index, a dropped term, a
transposed operand, the wrong rounding. The pins of ``test_oracle_pins.py``
are then run; the test passes only if some pin raises.
"""
import math

import numpy as np
import pytest

from oracle import qift_oracle as O
import test_oracle_pins as P


def _wrong_sign_hadamard(B):
    H = np.ones((1, 1), dtype=np.int64)
    base = np.array([[1, -1], [1, 1]], dtype=np.int64)
    while H.shape[0] < B:
        H = np.kron(base, H)
    return H


def _unnormalized_rotate(x, B):
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    Hm = O.hadamard(B).astype(np.float64)
    return (x.reshape(-1, K // B, B) @ Hm).reshape(x.shape)


def _strided_blocks_rotate(x, B):
    # blocks taken as every (K/B)-th feature instead of contiguous runs
    x = np.asarray(x, dtype=np.float64)
    K = x.shape[-1]
    Q = O.hadamard(B).astype(np.float64) / math.sqrt(B)
    xb = x.reshape(-1, B, K // B).swapaxes(1, 2)
    return (xb @ Q).swapaxes(1, 2).reshape(x.shape)


def _round_half_up_quant(xr32):
    xr32 = np.asarray(xr32, dtype=np.float32)
    R, K = xr32.shape
    q = np.zeros((R, K), dtype=np.int8)
    s = np.zeros(R, dtype=np.float32)
    for r in range(R):
        a = np.float32(np.max(np.abs(xr32[r])))
        if a == 0:
            continue
        s[r] = a / np.float32(7)
        q[r] = np.clip(np.floor(xr32[r] / s[r] + np.float32(0.5)), -7, 7)
    return q, s


def _wrong_divisor_quant(xr32):
    xr32 = np.asarray(xr32, dtype=np.float32)
    R, K = xr32.shape
    q = np.zeros((R, K), dtype=np.int8)
    s = np.zeros(R, dtype=np.float32)
    for r in range(R):
        a = np.float32(np.max(np.abs(xr32[r])))
        if a == 0:
            continue
        s[r] = a / np.float32(8)
        q[r] = np.clip(np.rint(xr32[r] / s[r]), -7, 7)
    return q, s


def _unclamped_quant(xr32):
    xr32 = np.asarray(xr32, dtype=np.float32)
    R, K = xr32.shape
    q = np.zeros((R, K), dtype=np.int64)
    s = np.zeros(R, dtype=np.float32)
    for r in range(R):
        sr = np.float32(np.max(np.abs(xr32[r]))) / np.float32(7)
        if sr == 0:
            continue
        s[r] = sr
        q[r] = np.rint(xr32[r] / sr)
    return q, s


def _zero_rule_on_absmax_quant(xr32):
    xr32 = np.asarray(xr32, dtype=np.float32)
    R, K = xr32.shape
    q = np.zeros((R, K), dtype=np.int64)
    s = np.zeros(R, dtype=np.float32)
    for r in range(R):
        a = np.float32(np.max(np.abs(xr32[r])))
        if a == 0:
            continue
        s[r] = a / np.float32(7)
        with np.errstate(divide="ignore", invalid="ignore"):
            q[r] = np.nan_to_num(np.clip(np.rint(xr32[r] / s[r]), -7, 7))
    return q, s


def _int4_weight_round_half_up(wr32, s_stored):
    w = wr32.astype(np.float32)
    s = s_stored.astype(np.float32)
    q = np.zeros(w.shape, dtype=np.int64)
    for n in range(w.shape[0]):
        if s[n] == 0:
            continue
        q[n] = np.clip(np.floor(w[n] / s[n] + np.float32(0.5)), -7, 7).astype(np.int64)
    return q


def _transposed_int_matmul(q, lv):
    a = np.asarray(q, dtype=np.float64) @ np.asarray(lv, dtype=np.float64)
    return np.rint(a).astype(np.int64)


def _natural_bit_offset(i):
    return 2 * i


def _swapped_pack_int4(q):
    q = np.asarray(q, dtype=np.int64)
    nib = (q & 0xF).astype(np.uint8)
    return (nib[..., 1::2] | (nib[..., 0::2] << 4)).astype(np.uint8)


def _tiled_index_group_row_swapped(Np, W):
    n = np.arange(Np)[:, None]
    w = np.arange(W)[None, :]
    r, i = n // 16, n % 16
    c, rem = w // 16, w % 16
    g, j = rem // 4, rem % 4
    uc = np.minimum(16, W - 16 * c)
    return c * 256 * (Np // 16) + r * 16 * uc + (16 * i + g) * 4 + j


def _gaussian_mse_cross_term_sign(levels, s=1.0):
    pts = sorted(float(v) * s for v in levels)
    edges = [-math.inf] + [(pts[i] + pts[i + 1]) / 2 for i in range(len(pts) - 1)] + [math.inf]
    total = 0.0
    for c, a, b in zip(pts, edges[:-1], edges[1:]):
        P_ = O._Phi(b) - O._Phi(a)
        aphi = 0.0 if math.isinf(a) else a * O._phi(a)
        bphi = 0.0 if math.isinf(b) else b * O._phi(b)
        total += P_ + aphi - bphi + 2.0 * c * (O._phi(a) - O._phi(b)) + c * c * P_
    return total


def _lloyd_wrong_centroid(n_levels=4, iters=2000, tol=1e-13):
    pts = list(np.linspace(-1.5, 1.5, n_levels))
    for _ in range(iters):
        edges = [-math.inf] + [(pts[i] + pts[i + 1]) / 2 for i in range(n_levels - 1)] + [math.inf]
        new = [(O._phi(a) - O._phi(b)) for a, b in zip(edges[:-1], edges[1:])]
        pts = new
    return np.array(pts)


def _table_preference_negative_first(table):
    t = O.check_table(table)
    return tuple(sorted(range(4), key=lambda c: (abs(t[c]), t[c] > 0, c)))


def _row_abs_error(w32, s, kind, table=None):
    w32 = np.asarray(w32, dtype=np.float32)[None, :]
    sv = np.asarray([s])
    if kind == "int4":
        lv = O.int4_weight_codes(w32, sv).astype(np.float64)
    else:
        lv = O._kind_levels(kind, table)[0][O.nearest_codes(w32, sv, kind, table)]
    return float(np.sum(np.abs(w32.astype(np.float64) - lv * float(sv[0]))))


def _attention_not_rotated_back(q, k_codes, k_scales, v_codes, v_scales, B, softmax_scale):
    q = np.asarray(q, dtype=np.float64)
    kd = np.asarray(k_codes, np.float64) * np.asarray(k_scales, np.float64)[..., None]
    vd = np.asarray(v_codes, np.float64) * np.asarray(v_scales, np.float64)[..., None]
    s = np.einsum("shd,sthd->sht", O.rotate(q, B), kd) * float(softmax_scale)
    p = np.exp(s - s.max(axis=2, keepdims=True))
    p /= p.sum(axis=2, keepdims=True)
    return np.einsum("sht,sthd->shd", p, vd)


def _attention_query_unrotated(q, k_codes, k_scales, v_codes, v_scales, B, softmax_scale):
    q = np.asarray(q, dtype=np.float64)
    kd = np.asarray(k_codes, np.float64) * np.asarray(k_scales, np.float64)[..., None]
    vd = np.asarray(v_codes, np.float64) * np.asarray(v_scales, np.float64)[..., None]
    s = np.einsum("shd,sthd->sht", q, kd) * float(softmax_scale)
    p = np.exp(s - s.max(axis=2, keepdims=True))
    p /= p.sum(axis=2, keepdims=True)
    return O.rotate(np.einsum("sht,sthd->shd", p, vd), B)


def _gptq_columns_variant(sign=1.0, divide=True):
    def cols(wr32, s, U, dead, kind, table=None):
        w = np.asarray(wr32, dtype=np.float32).astype(np.float64)
        w[:, dead] = 0.0
        N, K = w.shape
        sd = np.asarray(s).astype(np.float64)
        codes = np.zeros((N, K), dtype=np.int64)
        for k in range(K):
            col32 = w[:, k].astype(np.float32)[:, None]
            if kind == "int4":
                c = O.int4_weight_codes(col32, s)[:, 0]
                deq = c.astype(np.float64) * sd
            else:
                c = O.nearest_codes(col32, s, kind, table)[:, 0]
                deq = O._kind_levels(kind, table)[0][c] * sd
            codes[:, k] = c
            err = (w[:, k] - deq) / (U[k, k] if divide else 1.0)
            w[:, k + 1:] -= sign * np.outer(err, U[k, k + 1:])
        return codes
    return cols


def _gptq_factor_lower(H):
    return np.linalg.cholesky(np.linalg.inv(H))


def _gptq_factor_without_inverse(H):
    return np.linalg.cholesky(H).T


def _gptq_hessian_absolute_damping(X, B, damp):
    xr = O.rotate(X, B)
    H = xr.T @ xr
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    return H + float(damp) * np.eye(H.shape[0]), dead


def _gptq_hessian_unrotated(X, B, damp):
    X = np.asarray(X, dtype=np.float64)
    H = X.T @ X
    dead = np.diag(H) == 0
    H[dead, dead] = 1.0
    return H + float(damp) * float(np.mean(np.diag(H))) * np.eye(H.shape[0]), dead


def _kinds_with(kind, **over):
    d = {k: dict(v) for k, v in O.LEVEL_KINDS.items()}
    d[kind].update(over)
    return d


def _asym_params_not_widened(wr32, scale_dtype):
    w = np.asarray(wr32, dtype=np.float32)
    lo, hi = w.min(axis=1), w.max(axis=1)
    s = O._store_scale(((hi - lo) / np.float32(3)).astype(np.float32), scale_dtype)
    z = np.zeros(w.shape[0], dtype=np.int64)
    for n in range(w.shape[0]):
        if s[n] != 0:
            z[n] = int(np.clip(np.rint(np.float32(-lo[n]) / np.float32(s[n])), 0, 3))
    return s, z


def _asym_params_zero_point_sign(wr32, scale_dtype):
    s, z = _real_asym_params(wr32, scale_dtype)
    return s, np.clip(-z, 0, 3)


def _asym_params_divisor_4(wr32, scale_dtype):
    w = np.asarray(wr32, dtype=np.float32)
    lo = np.minimum(w.min(axis=1), np.float32(0))
    hi = np.maximum(w.max(axis=1), np.float32(0))
    s = O._store_scale(((hi - lo) / np.float32(4)).astype(np.float32), scale_dtype)
    z = np.zeros(w.shape[0], dtype=np.int64)
    for n in range(w.shape[0]):
        if s[n] != 0:
            z[n] = int(np.clip(np.rint(np.float32(-lo[n]) / np.float32(s[n])), 0, 3))
    return s, z


def _asym_codes_round_half_up(wr32, s_stored, z):
    w = np.asarray(wr32, dtype=np.float32)
    c = np.zeros(w.shape, dtype=np.int64)
    for n in range(w.shape[0]):
        sn = np.float32(s_stored[n])
        if sn != 0:
            c[n] = np.clip(np.floor(w[n] / sn + np.float32(0.5)).astype(np.int64) + int(z[n]), 0, 3)
    return c


def _linear_asym_without_zero_point(q, s_a, codes, s_w, kind, table=None):
    if kind == "asym":
        s, _ = O.split_asym_scales(s_w)
        acc = _real_int_matmul(q, np.asarray(codes, np.int64))
        return acc, acc * np.asarray(s_a, np.float64)[:, None] * np.asarray(s, np.float64)[None, :]
    return _real_linear(q, s_a, codes, s_w, kind, table)


_real_asym_params = O.asym_minmax_params
_real_int_matmul = O.int_matmul
_real_linear = O.linear


MUTATIONS = {
    "hadamard_wrong_sign": [("hadamard", _wrong_sign_hadamard)],
    "rotate_unnormalized": [("rotate", _unnormalized_rotate)],
    "rotate_strided_blocks": [("rotate", _strided_blocks_rotate)],
    "act_round_half_up": [("quant_sym4", _round_half_up_quant)],
    "act_divisor_8": [("quant_sym4", _wrong_divisor_quant)],
    "act_no_clamp": [("quant_sym4", _unclamped_quant)],
    "int4_weight_round_half_up": [("int4_weight_codes", _int4_weight_round_half_up)],
    "act_zero_rule_on_absmax": [("quant_sym4", _zero_rule_on_absmax_quant)],
    "ties_to_outer": [("_PREFERENCE", {"mnz": (1, 2, 0, 3), "pot": (1, 3, 0, 2)})],
    "ties_to_negative": [("_PREFERENCE", {"mnz": (3, 0, 2, 1), "pot": (2, 0, 3, 1)})],
    "pot_shift_sign_swapped": [("LEVEL_KINDS", _kinds_with("pot", code_to_int=(1, -4, -1, 4)))],
    "mnz_sorted_mapping": [("LEVEL_KINDS", _kinds_with("mnz", code_to_int=(-3, -1, 1, 3)))],
    "mnz_kappa_dropped": [("LEVEL_KINDS", _kinds_with("mnz", kappa=1.0))],
    "mnz_scale_divisor_2": [("LEVEL_KINDS", _kinds_with("mnz", outer=2.0))],
    "matmul_transposed": [("int_matmul", _transposed_int_matmul)],
    "pack2_natural_order": [("bit_offset_2b", _natural_bit_offset)],
    "pack4_nibbles_swapped": [("pack_int4", _swapped_pack_int4)],
    "tile_group_and_row_swapped": [("_tiled_index", _tiled_index_group_row_swapped)],
    "mse_cross_term_sign": [("gaussian_mse", _gaussian_mse_cross_term_sign)],
    "lloyd_unnormalized_centroid": [("lloyd_gaussian", _lloyd_wrong_centroid)],
    "table_ties_to_negative": [("table_preference", _table_preference_negative_first)],
    "mse_grid_32": [("MSE_GRID", 32)],
    "mse_rule_abs_error": [("row_sq_error", _row_abs_error)],
    "attention_not_rotated_back": [("kv4_attention_decode", _attention_not_rotated_back)],
    "attention_query_unrotated": [("kv4_attention_decode", _attention_query_unrotated)],
    "gptq_update_sign": [("gptq_columns", _gptq_columns_variant(sign=-1.0))],
    "gptq_error_not_divided": [("gptq_columns", _gptq_columns_variant(divide=False))],
    "gptq_factor_lower": [("gptq_factor", _gptq_factor_lower)],
    "gptq_factor_without_inverse": [("gptq_factor", _gptq_factor_without_inverse)],
    "gptq_damping_absolute": [("gptq_hessian", _gptq_hessian_absolute_damping)],
    "gptq_hessian_unrotated": [("gptq_hessian", _gptq_hessian_unrotated)],
    "asym_range_not_widened_to_zero": [("asym_minmax_params", _asym_params_not_widened)],
    "asym_zero_point_sign": [("asym_minmax_params", _asym_params_zero_point_sign)],
    "asym_step_divisor_4": [("asym_minmax_params", _asym_params_divisor_4)],
    "asym_codes_round_half_up": [("asym_codes", _asym_codes_round_half_up)],
    "asym_linear_without_zero_point": [("linear", _linear_asym_without_zero_point)],
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    for attr, repl in MUTATIONS[name]:
        monkeypatch.setattr(O, attr, repl)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except Exception as e:  # an assertion, or a shape error from a transposed operand
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutation {name} passed every pin"
