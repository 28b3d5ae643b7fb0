"""Plant plausible mistakes in the oracle (on the CPU) and check that the pins
in test_oracle.py catch every one of them."""
import dataclasses

import numpy as np
import pytest

from oracle import mla_oracle as O
from tests import test_oracle as P

_rope = O.rope
_attend = O.attend_head
_hkv = O.head_keys_values
_pq = O.project_queries
_out = O.output_projection
_ckv = O.compress_kv


_freqs = O.rope_freqs
_scale = O.softmax_scale


def _rope_sign(x, pos, base, theta=None):
    return _rope(x, -np.asarray(pos), base, theta)


def _rope_freq(x, pos, base, theta=None):
    # frequency base^(-k/d_R) instead of base^(-2k/d_R)
    d = np.asarray(x).shape[-1]
    return _rope(x, pos, base ** 0.5, theta) if d > 2 else _rope(x, pos, base, theta)


def _yarn_ramp_inverted(dims):
    # interpolate the fast pairs and keep the slow ones
    th = _freqs(dataclasses.replace(dims, yarn_factor=1.0))
    got = _freqs(dims)
    return th * th / got if O.yarn_on(dims) else got


def _yarn_ramp_in_index(dims):
    # the blend weight linear in the pair index k between the (real-valued)
    # pairs that turn beta_fast and beta_slow times, instead of linear in r_k
    if not O.yarn_on(dims):
        return _freqs(dims)
    d_r = dims.d_rope
    k = np.arange(d_r // 2, dtype=np.float64)
    theta = np.power(float(dims.rope_base), -2.0 * k / d_r)
    L = float(dims.yarn_orig_len)
    k_at = lambda r: (d_r / 2.0) * np.log(L / (2.0 * np.pi * r)) / np.log(float(dims.rope_base))
    k_fast, k_slow = k_at(float(dims.yarn_beta_fast)), k_at(float(dims.yarn_beta_slow))
    gamma = np.clip((k_slow - k) / (k_slow - k_fast), 0.0, 1.0)
    return (1.0 - gamma) * theta / float(dims.yarn_factor) + gamma * theta


def _yarn_no_temperature(dims):
    return 1.0 / np.sqrt(dims.d_nope + dims.d_rope)


def _yarn_temperature_unsquared(dims):
    s = _scale(dims)
    return s / (0.1 * np.log(dims.yarn_factor) + 1.0) if O.yarn_on(dims) else s


def _rope_halfsplit_pairs_wrong(x, pos, base, theta=None):
    # rotate (x[k], x[k+1]) over overlapping pairs: a wrong index
    x = np.asarray(x, dtype=np.float64)
    y = np.roll(x, 1, axis=-1)
    return np.roll(_rope(y, pos, base, theta), -1, axis=-1)


def _attend_drop_rope(q_c_i, q_r_i, qpos, k_c_i, k_r, v_i, scale, return_probs=False):
    return _attend(q_c_i, np.zeros_like(q_r_i), qpos, k_c_i, k_r, v_i, scale, return_probs)


def _attend_strict_mask(q_c_i, q_r_i, qpos, k_c_i, k_r, v_i, scale, return_probs=False):
    return _attend(q_c_i, q_r_i, np.asarray(qpos) - 1, k_c_i, k_r, v_i, scale, return_probs)


def _attend_no_mask(q_c_i, q_r_i, qpos, k_c_i, k_r, v_i, scale, return_probs=False):
    L = np.asarray(k_r).shape[0]
    return _attend(q_c_i, q_r_i, np.full_like(np.asarray(qpos), L - 1), k_c_i, k_r, v_i, scale, return_probs)


def _attend_wrong_axis(q_c_i, q_r_i, qpos, k_c_i, k_r, v_i, scale, return_probs=False):
    s = (q_c_i @ k_c_i.T + q_r_i @ k_r.T) * scale
    L = s.shape[1]
    vis = np.arange(L)[None, :] <= np.asarray(qpos)[:, None]
    e = np.where(vis, np.exp(s - s.max()), 0.0)
    p = e / e.sum(axis=0, keepdims=True).clip(1e-300)
    o = p @ v_i
    return (o, p) if return_probs else o


def _attend_transposed_key(q_c_i, q_r_i, qpos, k_c_i, k_r, v_i, scale, return_probs=False):
    # scores against k_R without the content key (k_C dropped)
    return _attend(np.zeros_like(q_c_i), q_r_i, qpos, k_c_i, k_r, v_i, scale, return_probs)


def _hkv_values_from_uk(W, c_kv, i, dims):
    k, v = _hkv(W, c_kv, i, dims)
    if dims.d_v == dims.d_nope:
        return k, k
    w = np.asarray(W["w_uk"], dtype=np.float64)[i * dims.d_nope:(i + 1) * dims.d_nope]
    kk = np.asarray(c_kv) @ w.T
    return k, np.resize(kk, v.shape)


def _hkv_strided_heads(W, c_kv, i, dims):
    w_uk = np.asarray(W["w_uk"], dtype=np.float64)[i::dims.n_heads][:dims.d_nope]
    w_uv = np.asarray(W["w_uv"], dtype=np.float64)[i::dims.n_heads][:dims.d_v]
    c = np.asarray(c_kv, dtype=np.float64)
    return c @ w_uk.T, c @ w_uv.T


def _pq_qr_head_split(W, h, pos, dims):
    q_c, q_r = _pq(W, h, pos, dims)
    T = q_r.shape[0]
    c_q = np.asarray(h, dtype=np.float64) @ np.asarray(W["w_dq"], dtype=np.float64).T
    raw = (c_q @ np.asarray(W["w_qr"], dtype=np.float64).T).reshape(T, dims.d_rope, dims.n_heads).transpose(0, 2, 1)
    return q_c, O.rope(raw, np.asarray(pos)[:, None], dims.rope_base)


def _pq_no_rope(W, h, pos, dims):
    q_c, _ = _pq(W, h, pos, dims)
    T = q_c.shape[0]
    c_q = np.asarray(h, dtype=np.float64) @ np.asarray(W["w_dq"], dtype=np.float64).T
    return q_c, (c_q @ np.asarray(W["w_qr"], dtype=np.float64).T).reshape(T, dims.n_heads, dims.d_rope)


def _out_head_order(W, o):
    o = np.asarray(o, dtype=np.float64)
    return o.transpose(0, 2, 1).reshape(o.shape[0], -1) @ np.asarray(W["w_o"], dtype=np.float64).T


def _ckv_kr_unroped(W, h, pos, dims):
    c, _ = _ckv(W, h, pos, dims)
    return c, np.asarray(h, dtype=np.float64) @ np.asarray(W["w_kr"], dtype=np.float64).T


_dec8 = O.e4m3_decode
_enc8 = O.e4m3_encode
_quant = O.quantize_latent


def _e4m3_bias8(codes):
    # the exponent bias of the other common 8-bit format (8 instead of 7)
    return _dec8(codes) / 2.0


def _e4m3_truncate(x):
    # truncation towards zero instead of round to nearest even
    x = np.asarray(x, dtype=np.float64)
    mags = O.e4m3_decode(np.arange(127))
    a = np.minimum(np.abs(x), O.E4M3_MAX)
    code = np.clip(np.searchsorted(mags, a, side="right") - 1, 0, 126)
    return np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)


def _quant_scale_240(c_kv):
    # scale against 240 (another format's largest value) instead of 448
    codes, scales = _quant(np.asarray(c_kv) * (240.0 / 448.0))
    return codes, scales * (448.0 / 240.0)


def _quant_group_64(c_kv):
    # groups of 64 columns, one scale each, but the stored scale of the first
    c = np.asarray(c_kv, dtype=np.float64)
    T, d_c = c.shape
    g = c.reshape(T, d_c // 64, 64)
    sc = O.fp8_group_scale(np.max(np.abs(g), axis=2))
    codes = _enc8(g / sc[:, :, None]).reshape(T, d_c)
    return codes, sc[:, ::2]


def _quant_scale_amax(c_kv):
    # scale = max|x| / 448 (the group maximum maps to 448 exactly), not a
    # power of two
    c = np.asarray(c_kv, dtype=np.float64)
    T, d_c = c.shape
    g = c.reshape(T, d_c // 128, 128)
    amax = np.max(np.abs(g), axis=2)
    sc = np.where(amax > 0, amax / 448.0, 1.0)
    return _enc8(g / sc[:, :, None]).reshape(T, d_c), sc


def _quant_scale_floor(c_kv):
    # the power of two at or below max|x| / 448 (the group maximum can then
    # exceed 448 and saturates)
    c = np.asarray(c_kv, dtype=np.float64)
    T, d_c = c.shape
    g = c.reshape(T, d_c // 128, 128)
    amax = np.max(np.abs(g), axis=2)
    with np.errstate(divide="ignore"):
        sc = np.where(amax > 0, 2.0 ** np.floor(np.log2(np.where(amax > 0, amax, 1.0) / 448.0)), 1.0)
    return _enc8(g / sc[:, :, None]).reshape(T, d_c), sc


def _bf16_truncate(x):
    # drop the low bits instead of rounding to nearest
    f, e = np.frexp(np.asarray(x, dtype=np.float64))
    return np.ldexp(np.trunc(f * 256.0) / 256.0, e)


def _bf16_skipped(x):
    # quantise the float64 value (no bf16 rounding first)
    return np.asarray(x, dtype=np.float64)


_qgroups = O.quantize_groups
_deqw = O.dequantize_weight_blocks


def _quant_scale_per_token(x):
    # one scale per token row (its largest magnitude) instead of one per group
    x = np.asarray(x, dtype=np.float64)
    codes, scales = _qgroups(x)
    amax = np.max(np.abs(x), axis=1, keepdims=True)
    sc = np.repeat(O.fp8_group_scale(amax), scales.shape[1], axis=1)
    g = x.reshape(x.shape[0], -1, 128)
    return _enc8(g / sc[:, :, None]).reshape(x.shape), sc


def _weight_scale_row_blocks_only(codes, scales):
    # the first column block's scale for the whole row block
    sc = np.asarray(scales, dtype=np.float64)
    return _deqw(codes, np.repeat(sc[:, :1], sc.shape[1], axis=1))


MUTATIONS = {
    "rope_sign": ("rope", _rope_sign),
    "rope_frequency": ("rope", _rope_freq),
    "rope_pairs": ("rope", _rope_halfsplit_pairs_wrong),
    "scale_dh_only": ("softmax_scale", lambda d: 1.0 / np.sqrt(d.d_nope)),
    "scale_missing": ("softmax_scale", lambda d: 1.0),
    "drop_rope_score": ("attend_head", _attend_drop_rope),
    "drop_content_score": ("attend_head", _attend_transposed_key),
    "mask_strict": ("attend_head", _attend_strict_mask),
    "mask_missing": ("attend_head", _attend_no_mask),
    "softmax_axis": ("attend_head", _attend_wrong_axis),
    "values_from_uk": ("head_keys_values", _hkv_values_from_uk),
    "heads_strided": ("head_keys_values", _hkv_strided_heads),
    "qr_head_split": ("project_queries", _pq_qr_head_split),
    "q_no_rope": ("project_queries", _pq_no_rope),
    "output_head_order": ("output_projection", _out_head_order),
    "k_no_rope": ("compress_kv", _ckv_kr_unroped),
    "yarn_ramp_inverted": ("rope_freqs", _yarn_ramp_inverted),
    "yarn_ramp_in_index": ("rope_freqs", _yarn_ramp_in_index),
    "yarn_no_interpolation": ("rope_freqs", lambda d: _freqs(dataclasses.replace(d, yarn_factor=1.0))),
    "yarn_no_temperature": ("softmax_scale", _yarn_no_temperature),
    "yarn_temperature_unsquared": ("softmax_scale", _yarn_temperature_unsquared),
    "e4m3_bias8": ("e4m3_decode", _e4m3_bias8),
    "e4m3_truncate": ("e4m3_encode", _e4m3_truncate),
    "fp8_scale_240": ("quantize_latent", _quant_scale_240),
    "fp8_group_64": ("quantize_latent", _quant_group_64),
    "fp8_scale_amax_over_448": ("quantize_latent", _quant_scale_amax),
    "fp8_scale_rounded_down": ("quantize_latent", _quant_scale_floor),
    "bf16_truncate": ("round_bf16", _bf16_truncate),
    "fp8_input_not_bf16": ("round_bf16", _bf16_skipped),
    "fp8_act_scale_per_token": ("quantize_groups", _quant_scale_per_token),
    "fp8_weight_scale_per_row_block": ("dequantize_weight_blocks", _weight_scale_row_blocks_only),
    "fp8_activation_unquantised": ("fp8_activation", lambda x: np.asarray(x, dtype=np.float64)),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    attr, fn = MUTATIONS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        if pin is P.pin_brute_force:
            continue  # the scalar brute force is a restatement; real pins must catch it
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception as e:  # AssertionError, or a shape error the mistake causes
            caught.append((pin.__name__, type(e).__name__))
    assert caught, f"mutation {name} passed every pin"
