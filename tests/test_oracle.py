"""Pins for the CPU oracle (no GPU).

Each pin ties the oracle to something other than itself: a closed form, an
identity, a library routine (PyTorch's scaled_dot_product_attention), the
rotation properties of RoPE, the dimensions the pages print, or a scalar brute
force.  ``test_oracle_mutations.py`` plants plausible mistakes in the oracle and
checks that these pins catch each one.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from mla_inputs import TINY, DSV3, Dims, draw_weights, make_workload
from oracle import mla_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
SMALL = Dims(d_model=48, n_heads=3, d_nope=8, d_rope=6, d_v=5, d_c=12, d_cq=10)


def _weights(dims, seed=0):
    rng = np.random.Generator(np.random.PCG64(seed))
    f32, _ = draw_weights(rng, dims, bf16=False)
    return {k: v.astype(np.float64) for k, v in f32.items()}


def _h(T, dims, seed=1):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal((T, dims.d_model))


# ---------------------------------------------------------------------------
# Pin functions (plain, so the mutation test can re-run them)
# ---------------------------------------------------------------------------

def pin_absorbed_equals_plain(dims=TINY, L=20, n_q=3, seed=3):
    """P1: weight absorption (decode in latent space) equals the literal form."""
    W = _weights(dims, seed)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    cache = rng.standard_normal((L - n_q, dims.d_row))
    h = rng.standard_normal((n_q, dims.d_model))
    a = O.decode(dims, W, h, cache)
    b = O.decode_absorbed(dims, W, h, cache)
    err = np.max(np.abs(a["u"] - b["u"])) / np.max(np.abs(b["u"]))
    assert err <= 1e-12, err
    erro = np.max(np.abs(a["o"] - b["o"])) / np.max(np.abs(b["o"]))
    assert erro <= 1e-12, erro


def pin_softmax_rows(dims=TINY, L=17):
    """P2: every probability row sums to one and masked entries are zero."""
    W = _weights(dims, 5)
    r = O.prefill(dims, W, _h(L, dims, 6), return_probs=True)
    for i, p in r["probs"].items():
        assert np.allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
        assert np.all(p[np.triu_indices(L, k=1)] == 0.0)
        assert np.all(p >= 0)


def pin_causal(dims=TINY, L=16, t=9):
    """P3: changing tokens after t leaves outputs up to t bitwise unchanged."""
    W = _weights(dims, 7)
    h = _h(L, dims, 8)
    h2 = h.copy()
    h2[t + 1:] += np.random.Generator(np.random.PCG64(9)).standard_normal(h2[t + 1:].shape)
    a = O.prefill(dims, W, h)["u"]
    b = O.prefill(dims, W, h2)["u"]
    assert np.array_equal(a[:t + 1], b[:t + 1])
    assert not np.allclose(a[t + 1:], b[t + 1:])


def pin_single_key(dims=TINY):
    """P5: at position 0 the only visible key has probability one, so
    u_0 = W_O [W_UV,i c_KV,0]_i."""
    W = _weights(dims, 11)
    h = _h(5, dims, 12)
    r = O.prefill(dims, W, h)
    c0 = W["w_dkv"] @ h[0]
    expect = W["w_o"] @ (W["w_uv"] @ c0)
    assert np.allclose(r["u"][0], expect, rtol=1e-12, atol=1e-12)


def pin_zero_query(dims=TINY, L=11):
    """P6: with W_UQ = W_QR = 0 every score is zero, so each output is the mean
    of the values visible to it."""
    W = _weights(dims, 13)
    W["w_uq"][:] = 0
    W["w_qr"][:] = 0
    h = _h(L, dims, 14)
    r = O.prefill(dims, W, h)
    c = h @ W["w_dkv"].T
    v = (c @ W["w_uv"].T).reshape(L, dims.n_heads, dims.d_v)
    mean = np.cumsum(v, axis=0) / np.arange(1, L + 1)[:, None, None]
    assert np.allclose(r["o"], mean, rtol=1e-12, atol=1e-12)


def pin_head_isolation(dims=TINY, L=9):
    """Head slicing: with W_UQ = 0 and W_QR zero outside head k's rows, every
    head but k attends uniformly, and head k does not."""
    for k in range(dims.n_heads):
        W = _weights(dims, 15 + k)
        W["w_uq"][:] = 0
        keep = W["w_qr"][k * dims.d_rope:(k + 1) * dims.d_rope].copy() * 8.0
        W["w_qr"][:] = 0
        W["w_qr"][k * dims.d_rope:(k + 1) * dims.d_rope] = keep
        r = O.prefill(dims, W, _h(L, dims, 30 + k), return_probs=True)
        for i, p in r["probs"].items():
            uniform = np.tril(np.ones((L, L))) / np.arange(1, L + 1)[:, None]
            if i == k:
                assert not np.allclose(p, uniform, atol=1e-6)
            else:
                assert np.allclose(p, uniform, rtol=0, atol=1e-14)
    # the same for the content query through W_UQ
    for k in range(dims.n_heads):
        W = _weights(dims, 40 + k)
        W["w_qr"][:] = 0
        keep = W["w_uq"][k * dims.d_nope:(k + 1) * dims.d_nope].copy() * 8.0
        W["w_uq"][:] = 0
        W["w_uq"][k * dims.d_nope:(k + 1) * dims.d_nope] = keep
        r = O.prefill(dims, W, _h(L, dims, 50 + k), return_probs=True)
        for i, p in r["probs"].items():
            uniform = np.tril(np.ones((L, L))) / np.arange(1, L + 1)[:, None]
            assert (not np.allclose(p, uniform, atol=1e-6)) if i == k else np.allclose(p, uniform, atol=1e-14)


def pin_mha_special_case(dims=None, L=13):
    """P7: with d_c = d_model, W_DKV = I and W_KR = W_QR = 0, MLA is causal
    multi-head attention with Q = W_UQ W_DQ h, K = W_UK h, V = W_UV h; compare
    with PyTorch's scaled_dot_product_attention in float64, then W_O."""
    d = dims or Dims(d_model=24, n_heads=3, d_nope=8, d_rope=4, d_v=6, d_c=24, d_cq=16)
    W = _weights(d, 21)
    W["w_dkv"] = np.eye(d.d_c)
    W["w_kr"][:] = 0
    W["w_qr"][:] = 0
    h = _h(L, d, 22)
    got = O.prefill(d, W, h)["u"]
    th = torch.from_numpy(h)
    Q = th @ torch.from_numpy(W["w_dq"]).T @ torch.from_numpy(W["w_uq"]).T
    K = th @ torch.from_numpy(W["w_uk"]).T
    V = th @ torch.from_numpy(W["w_uv"]).T
    q = Q.reshape(L, d.n_heads, d.d_nope).transpose(0, 1).unsqueeze(0)
    k = K.reshape(L, d.n_heads, d.d_nope).transpose(0, 1).unsqueeze(0)
    v = V.reshape(L, d.n_heads, d.d_v).transpose(0, 1).unsqueeze(0)
    o = torch.nn.functional.scaled_dot_product_attention(
        q, k, v, is_causal=True, scale=1.0 / math.sqrt(d.d_nope + d.d_rope))
    ref = o.squeeze(0).transpose(0, 1).reshape(L, -1) @ torch.from_numpy(W["w_o"]).T
    assert np.allclose(got, ref.numpy(), rtol=1e-11, atol=1e-12)


def pin_rope_rotation():
    """P8: explicit rotation at d_R = 2 (angle = position), the frequency at
    d_R = 4, identity at position 0, norm preservation, and the relative
    property RoPE(x,m).RoPE(y,n) = f(m-n)."""
    for p in (0, 1, 3, 17):
        assert np.allclose(O.rope(np.array([1.0, 0.0]), p, 10000.0), [math.cos(p), math.sin(p)], atol=1e-15)
        assert np.allclose(O.rope(np.array([0.0, 1.0]), p, 10000.0), [-math.sin(p), math.cos(p)], atol=1e-15)
    th1 = 10000.0 ** (-0.5)
    got = O.rope(np.array([0.0, 0.0, 1.0, 0.0]), 5, 10000.0)
    assert np.allclose(got, [0.0, 0.0, math.cos(5 * th1), math.sin(5 * th1)], atol=1e-15)
    rng = np.random.Generator(np.random.PCG64(4))
    x = rng.standard_normal(16)
    y = rng.standard_normal(16)
    assert np.array_equal(O.rope(x, 0, 10000.0), x)
    assert np.isclose(np.linalg.norm(O.rope(x, 123, 10000.0)), np.linalg.norm(x), rtol=1e-14)
    d1 = O.rope(x, 40, 10000.0) @ O.rope(y, 30, 10000.0)
    d2 = O.rope(x, 1010, 10000.0) @ O.rope(y, 1000, 10000.0)
    assert np.isclose(d1, d2, rtol=1e-10)
    assert not np.isclose(d1, O.rope(x, 41, 10000.0) @ O.rope(y, 30, 10000.0), rtol=1e-6)


def pin_rope_in_scores():
    """RoPE acts on both the query (at its position t) and the key (at its
    position j): with no content score (W_UQ = 0), d_R = 2 and the same token
    at positions 0 and 1, the scores at t = 1 are a.R(-1)b and a.b with
    a = W_QR,i c_Q, b = W_KR h and R the textbook 2x2 rotation, so the
    probability of key 0 has a closed form."""
    d = Dims(d_model=12, n_heads=2, d_nope=4, d_rope=2, d_v=3, d_c=5, d_cq=6)
    W = _weights(d, 27)
    W["w_uq"][:] = 0
    x = _h(1, d, 28)[0]
    r = O.prefill(d, W, np.stack([x, x]), return_probs=True)
    scale = 1.0 / math.sqrt(d.d_nope + d.d_rope)
    b = W["w_kr"] @ x
    rot = lambda ang: np.array([[math.cos(ang), -math.sin(ang)], [math.sin(ang), math.cos(ang)]])
    for i in range(d.n_heads):
        a = W["w_qr"][2 * i:2 * i + 2] @ (W["w_dq"] @ x)
        s0 = a @ rot(-1.0) @ b * scale
        s1 = a @ b * scale
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert abs(r["probs"][i][1, 0] - p0) <= 1e-14, (r["probs"][i][1, 0], p0)


def pin_yarn_frequencies():
    """YaRN (highlight 13 of the V3 highlights page): pairs that turn at most
    beta_slow times over the original context rotate at theta/s, i.e. as
    plain RoPE at position p/s; pairs that turn at least beta_fast times keep
    theta; the blend in between lies between the two, and less interpolation
    goes to faster pairs.  For DeepSeek-V3 (d_R 64, base 10^4, L 4096,
    s 40, 1, 32) the pair k turns 4096 * 10^(-k/8) / (2 pi) times: pairs
    0..10 turn at least 32 times, pairs 23..31 at most once."""
    import dataclasses
    rng = np.random.Generator(np.random.PCG64(31))
    x = rng.standard_normal(16)
    slow = dataclasses.replace(TINY, yarn_factor=40.0, yarn_orig_len=1)            # every pair slow
    fast = dataclasses.replace(TINY, yarn_factor=40.0, yarn_orig_len=10 ** 12)     # every pair fast
    for p in (0, 1, 7, 300, 5000):
        got = O.rope(x, p, TINY.rope_base, O.rope_freqs(slow))
        assert np.allclose(got, O.rope(x, p / 40.0, TINY.rope_base), rtol=0, atol=1e-12)
        assert np.array_equal(O.rope(x, p, TINY.rope_base, O.rope_freqs(fast)), O.rope(x, p, TINY.rope_base))
    ds = dataclasses.replace(DSV3, yarn_factor=40.0)
    th = 10000.0 ** (-2.0 * np.arange(32) / 64)
    ratio = O.rope_freqs(ds) / th
    assert np.allclose(ratio[:11], 1.0, rtol=0, atol=1e-15)
    assert np.allclose(ratio[23:], 1.0 / 40.0, rtol=1e-15, atol=0)
    mid = ratio[11:23]
    assert np.all((mid > 1.0 / 40.0) & (mid < 1.0)) and np.all(np.diff(ratio) <= 1e-15)
    # relative-position property survives the new frequencies
    y = rng.standard_normal(64)
    z = rng.standard_normal(64)
    f = O.rope_freqs(ds)
    d1 = O.rope(y, 9000, 1.0, f) @ O.rope(z, 8000, 1.0, f)
    d2 = O.rope(y, 131000, 1.0, f) @ O.rope(z, 130000, 1.0, f)
    assert np.isclose(d1, d2, rtol=1e-8)


def pin_yarn_in_scores():
    """YaRN through the whole prefill: as pin_rope_in_scores, with every pair
    slow (the angle per position becomes 1/s) and the logits multiplied by
    the temperature factor (0.1 ln s + 1)^2."""
    import dataclasses
    d = dataclasses.replace(Dims(d_model=12, n_heads=2, d_nope=4, d_rope=2, d_v=3, d_c=5, d_cq=6),
                            yarn_factor=40.0, yarn_orig_len=1)
    W = _weights(d, 29)
    W["w_uq"][:] = 0
    x = _h(1, d, 30)[0]
    r = O.prefill(d, W, np.stack([x, x]), return_probs=True)
    scale = (0.1 * math.log(40.0) + 1.0) ** 2 / math.sqrt(d.d_nope + d.d_rope)
    b = W["w_kr"] @ x
    rot = lambda ang: np.array([[math.cos(ang), -math.sin(ang)], [math.sin(ang), math.cos(ang)]])
    for i in range(d.n_heads):
        a = W["w_qr"][2 * i:2 * i + 2] @ (W["w_dq"] @ x)
        s0 = a @ rot(-1.0 / 40.0) @ b * scale
        s1 = a @ b * scale
        p0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert abs(r["probs"][i][1, 0] - p0) <= 1e-14, (r["probs"][i][1, 0], p0)


def pin_yarn_blend_hand_worked():
    """YaRN's blend inside the ramp, against values worked by hand from the
    method's definition (tests/golden/yarn_blend_hand_worked.json, V3
    highlights page, highlight 13): pairs 11 and 16 of DeepSeek-V3 (d_R 64,
    base 10^4, 4K original context, s 40) and one pair over a 100-token
    original context.  A ramp linear in the pair index instead of in the
    rotation count r_k moves pair 16 from 0.00199 to 0.0055."""
    import dataclasses
    g = json.load(open(os.path.join(GOLDEN, "yarn_blend_hand_worked.json")))
    for c in g["cases"]:
        d = dataclasses.replace(Dims(d_model=8, n_heads=1, d_nope=2, d_rope=c["d_rope"], d_v=2, d_c=4, d_cq=4),
                                rope_base=c["rope_base"], yarn_factor=c["yarn_factor"],
                                yarn_orig_len=c["yarn_orig_len"], yarn_beta_slow=c["yarn_beta_slow"],
                                yarn_beta_fast=c["yarn_beta_fast"])
        got = O.rope_freqs(d)[c["pair"]]
        assert abs(got - c["theta_blended"]) <= 1e-8 * c["theta_blended"], (c["name"], got, c["theta_blended"])


def pin_prefill_decode_agree(dims=TINY, L=24, steps=5):
    """P9: a prefill of L followed by decode steps equals one longer prefill."""
    W = _weights(dims, 23)
    h = _h(L + steps, dims, 24)
    full = O.prefill(dims, W, h)
    r = O.prefill(dims, W, h[:L])
    rows = np.concatenate([r["c_kv"], r["k_r"]], axis=1)
    for s in range(steps):
        d = O.decode(dims, W, h[L + s:L + s + 1], rows)
        assert np.allclose(d["u"][0], full["u"][L + s], rtol=1e-12, atol=1e-12)
        rows = np.concatenate([rows, d["row_new"]], axis=0)
    # two query tokens at once (causal between themselves)
    d2 = O.decode(dims, W, h[L:L + 2], np.concatenate([r["c_kv"], r["k_r"]], axis=1))
    assert np.allclose(d2["u"], full["u"][L:L + 2], rtol=1e-12, atol=1e-12)


def pin_brute_force(dims=SMALL, L=4):
    """Scalar-loop MLA on a micro case, written independently of numpy's
    vectorised reshapes."""
    W = _weights(dims, 25)
    h = _h(L, dims, 26)
    got = O.prefill(dims, W, h)["u"]

    def mv(M, x):
        return [sum(M[r][c] * x[c] for c in range(len(x))) for r in range(len(M))]

    def rot(x, p):
        out = list(x)
        for k in range(len(x) // 2):
            a = p * dims.rope_base ** (-2.0 * k / len(x))
            out[2 * k] = x[2 * k] * math.cos(a) - x[2 * k + 1] * math.sin(a)
            out[2 * k + 1] = x[2 * k] * math.sin(a) + x[2 * k + 1] * math.cos(a)
        return out

    Wl = {k: v.tolist() for k, v in W.items()}
    hs = h.tolist()
    ckv = [mv(Wl["w_dkv"], hs[t]) for t in range(L)]
    kr = [rot(mv(Wl["w_kr"], hs[t]), t) for t in range(L)]
    for t in range(L):
        cq = mv(Wl["w_dq"], hs[t])
        qc_all = mv(Wl["w_uq"], cq)
        qr_all = mv(Wl["w_qr"], cq)
        ocat = []
        for i in range(dims.n_heads):
            qc = qc_all[i * dims.d_nope:(i + 1) * dims.d_nope]
            qr = rot(qr_all[i * dims.d_rope:(i + 1) * dims.d_rope], t)
            scores, vals = [], []
            for j in range(t + 1):
                kc = mv(Wl["w_uk"][i * dims.d_nope:(i + 1) * dims.d_nope], ckv[j])
                v = mv(Wl["w_uv"][i * dims.d_v:(i + 1) * dims.d_v], ckv[j])
                s = sum(a * b for a, b in zip(qc + qr, kc + kr[j])) / math.sqrt(dims.d_nope + dims.d_rope)
                scores.append(s)
                vals.append(v)
            mx = max(scores)
            ex = [math.exp(s - mx) for s in scores]
            z = sum(ex)
            ocat += [sum(ex[j] / z * vals[j][c] for j in range(t + 1)) for c in range(dims.d_v)]
        u = mv(Wl["w_o"], ocat)
        assert np.allclose(got[t], u, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------
# FP8 latent cache
# ---------------------------------------------------------------------------

def pin_e4m3_definition():
    """E4M3 values from the OCP 8-bit floating-point definition, worked by
    hand: bias 7, three mantissa bits, exponent field 0 for subnormals,
    S.1111.111 the only NaN, largest finite 448."""
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
             0x30: 0.5, 0x38: 1.0, 0x39: 1.125, 0x3F: 1.875, 0x40: 2.0, 0x58: 16.0, 0x7E: 448.0,
             0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in table.items():
        got = O.e4m3_decode(c)
        assert got == v and np.signbit(got) == np.signbit(v), (hex(c), got, v)
    vals = O.e4m3_decode(np.arange(256))
    assert np.isnan(vals[0x7F]) and np.isnan(vals[0xFF]) and np.sum(np.isnan(vals)) == 2
    assert np.max(vals[~np.isnan(vals)]) == O.E4M3_MAX


def pin_e4m3_rounding():
    """Encoding: every finite code round-trips; a value halfway between two
    neighbours goes to the one with the even code; just off the midpoint it
    goes to the nearer; beyond 448 it saturates."""
    vals = O.e4m3_decode(np.arange(256))
    fin = np.where(~np.isnan(vals))[0]
    assert np.array_equal(O.e4m3_encode(vals[fin]), fin.astype(np.uint8))
    mags = O.e4m3_decode(np.arange(127))
    mid = (mags[:-1] + mags[1:]) / 2
    even = np.where(np.arange(126) % 2 == 0, np.arange(126), np.arange(1, 127))
    assert np.array_equal(O.e4m3_encode(mid), even.astype(np.uint8))
    assert np.array_equal(O.e4m3_encode(mid * (1 - 1e-9)), np.arange(126).astype(np.uint8))
    assert np.array_equal(O.e4m3_encode(mid * (1 + 1e-9)), np.arange(1, 127).astype(np.uint8))
    assert O.e4m3_encode(1000.0) == 0x7E and O.e4m3_encode(-470.0) == 0xFE
    # 1.0625 lies halfway between 1 (0x38) and 1.125 (0x39): the even code
    assert O.e4m3_encode(1.0625) == 0x38 and O.e4m3_encode(1.1875) == 0x3A


def pin_e4m3_library():
    """The codec against PyTorch's float8_e4m3fn (a library implementation
    of the same format): every code's value, and the codes of random values
    within range."""
    codes = np.arange(256)
    ref = torch.tensor(codes, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)) and np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    x = np.random.Generator(np.random.PCG64(41)).standard_normal(20000).astype(np.float32) * 60
    x = np.clip(x, -448, 448)
    ref_codes = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(O.e4m3_encode(x.astype(np.float64)), ref_codes)


def pin_quantize_latent_hand_worked():
    """One row of four 128-column groups, codes worked out by hand from the
    E4M3 definition (1 sign, 4 exponent bits with bias 7, 3 mantissa bits).
    Group 0, max |x| = 3.0: scale 2^-7 (448 * 2^-7 = 3.5 >= 3, 448 * 2^-8 =
    1.75 < 3); x / scale: 3.0 -> 384 = 1.5 * 2^8 -> 0x7C, 1.0 -> 128 ->
    0x70, 0.1 -> 12.8 -> 13 = 1.625 * 8 -> 0x55, -0.3 -> -38.4 -> -40 ->
    0xE2, 13.5 / 128 -> 13.5, a tie between 13 (odd code) and 14 -> 0x56,
    0.01 / 128 -> 0.01 = 5.12 * 2^-9 (subnormal) -> 0x05.  Group 1, max |x|
    = 7.0 exactly: scale 2^-6 (448 * 2^-6 = 7), 7 -> 448 -> 0x7E, -7 ->
    0xFE, 0.5 -> 32 -> 0x60.  Group 2, max |x| = 7 (1 + 2^-20), just past
    448 * 2^-6: scale 2^-5 and that value -> 224 (1 + 2^-20) -> 224 ->
    0x76.  Group 3, all zero: scale 1, codes 0."""
    c = np.zeros((1, 512))
    c[0, :7] = [3.0, 1.0, 0.1, -0.3, 0.0, 13.5 / 128, 0.01 / 128]
    c[0, 128:131] = [7.0, -7.0, 0.5]
    c[0, 256] = 7.0 * (1 + 2.0 ** -20)
    codes, scales = O.quantize_latent(c)
    assert scales.tolist() == [[2.0 ** -7, 2.0 ** -6, 2.0 ** -5, 1.0]]
    assert codes[0, :7].tolist() == [0x7C, 0x70, 0x55, 0xE2, 0x00, 0x56, 0x05]
    assert codes[0, 128:131].tolist() == [0x7E, 0xFE, 0x60]
    assert codes[0, 256] == 0x76
    rest = np.ones(512, dtype=bool)
    rest[[0, 1, 2, 3, 4, 5, 6, 128, 129, 130, 256]] = False
    assert np.all(codes[0, rest] == 0)


def pin_quantize_latent_bound():
    """On random groups spanning many magnitudes: each scale is a power of
    two and the smallest with 448 s >= max|x| (so 224 s < max|x|), and every
    dequantised value lies within half a code step of the input,
    |x' - x| <= s * max(2^-4 |x/s|, 2^-10) (normal and subnormal spacing);
    an all-zero group stays zero."""
    rng = np.random.Generator(np.random.PCG64(43))
    c = rng.standard_normal((7, 256)) * np.exp(rng.standard_normal((7, 1)) * 3)
    c[3, 128:] = 0.0
    codes, scales = O.quantize_latent(c)
    assert codes.shape == (7, 256) and scales.shape == (7, 2)
    deq = O.e4m3_decode(codes).reshape(7, 2, 128) * scales[:, :, None]
    g = c.reshape(7, 2, 128)
    amax = np.max(np.abs(g), axis=2)
    mant, _ = np.frexp(scales)
    assert np.all(mant == 0.5)                                   # powers of two
    live = amax > 0
    assert np.all(448.0 * scales[live] >= amax[live]) and np.all(224.0 * scales[live] < amax[live])
    assert scales[3, 1] == 1.0
    bound = scales[:, :, None] * np.maximum(2.0 ** -4 * np.abs(g) / scales[:, :, None], 2.0 ** -10)
    assert np.all(np.abs(deq - g) <= bound * (1 + 1e-12))
    assert np.all(deq[3, 1] == 0.0)


def pin_fp8_row_layout():
    """A stored FP8 row, assembled byte by byte here: codes, k_R in bf16,
    then the little-endian fp32 scales; 656 bytes for DeepSeek-V3 widths."""
    assert O.fp8_row_bytes(DSV3) == 512 + 128 + 16
    d = Dims(d_model=8, n_heads=1, d_nope=2, d_rope=2, d_v=2, d_c=128, d_cq=4)
    row = np.zeros(O.fp8_row_bytes(d), dtype=np.uint8)
    row[0] = 0x38          # 1.0
    row[127] = 0xC0        # -2.0
    row[128:130] = np.frombuffer(np.float32(3.0).tobytes()[2:], dtype=np.uint8)     # bf16 3.0
    row[130:132] = np.frombuffer(np.float32(-0.5).tobytes()[2:], dtype=np.uint8)    # bf16 -0.5
    row[132:136] = np.frombuffer(np.float32(0.25).tobytes(), dtype=np.uint8)        # scale
    got = O.dequantize_fp8_rows(row[None], d)[0]
    assert got.shape == (130,)
    assert got[0] == 0.25 and got[127] == -0.5 and np.all(got[1:127] == 0)
    assert got[128] == 3.0 and got[129] == -0.5


def pin_round_bf16():
    """bfloat16 rounding against PyTorch's float32 -> bfloat16 cast (round
    to nearest even) on float32 values, ties included: 1 + 2^-8 lies halfway
    between 1 and 1 + 2^-7 and goes to 1; 1 + 3 * 2^-8 goes to 1 + 2^-6."""
    import torch
    rng = np.random.Generator(np.random.PCG64(46))
    x = (rng.standard_normal(4000) * np.exp(rng.standard_normal(4000) * 4)).astype(np.float32)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, -(1 + 2.0 ** -8), 3 * (1 + 2.0 ** -8), 0.0], dtype=np.float32)
    x = np.concatenate([x, ties])
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = O.round_bf16(x.astype(np.float64))
    assert np.array_equal(got, want)
    assert got[-5] == 1.0 and got[-4] == 1 + 2.0 ** -6


def pin_decode_fp8_new_rows():
    """With an FP8 cache the new tokens attend to their own c_KV in quantised
    form: a one-token sequence (only its own key) gives o_i = W_UV,i c_KV',
    c_KV' the quantise-dequantise of c_KV rounded to bfloat16."""
    d = dataclasses_replace(TINY, d_c=128)
    W = _weights(d, 44)
    x = _h(1, d, 45)
    r = O.decode(d, W, x, np.zeros((0, d.d_row)), cache_fp8=True)
    c = x @ W["w_dkv"].T
    c16 = torch_bf16(c)
    codes, scales = O.quantize_latent(c16)
    cq = O.e4m3_decode(codes) * np.repeat(scales, 128, axis=1)
    for i in range(d.n_heads):
        v = W["w_uv"][i * d.d_v:(i + 1) * d.d_v] @ cq[0]
        assert np.allclose(r["o"][0, i], v, rtol=1e-13, atol=1e-13)
    assert not np.allclose(cq, c, rtol=1e-6, atol=0)   # the quantisation is visible


def torch_bf16(x):
    """float64 -> bfloat16 -> float64 by PyTorch (through float32; the values
    here are far from any double-rounding case at that precision)."""
    import torch
    return torch.from_numpy(np.asarray(x, dtype=np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def dataclasses_replace(d, **kw):
    import dataclasses
    return dataclasses.replace(d, **kw)


# ---------------------------------------------------------------------------
# Block-scaled FP8 projections
# ---------------------------------------------------------------------------

def _torch_e4m3_values(codes):
    """Values of E4M3 codes by PyTorch's float8_e4m3fn."""
    return torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def pin_weight_blocks_layout():
    """A [130][256] weight of codes 0x38 (1.0) under scales [[1, 2], [4, 8]]:
    element (r, c) takes the scale of block (r // 128, c // 128), the last
    row block holding two rows; and random codes and scales against
    PyTorch's E4M3 values times a scale expanded block by block here."""
    codes = np.full((130, 256), 0x38, dtype=np.uint8)
    sc = np.array([[1.0, 2.0], [4.0, 8.0]])
    w = O.dequantize_weight_blocks(codes, sc)
    assert w[0, 0] == 1 and w[127, 127] == 1 and w[0, 128] == 2 and w[0, 255] == 2
    assert w[128, 0] == 4 and w[129, 127] == 4 and w[128, 128] == 8 and w[129, 255] == 8
    rng = np.random.Generator(np.random.PCG64(51))
    codes = rng.integers(0, 256, (200, 384)).astype(np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x38        # no NaN codes
    sc = np.ldexp(1.0, rng.integers(-12, 3, (2, 3)))
    ref = _torch_e4m3_values(codes)
    for rb in range(2):
        for cb in range(3):
            ref[rb * 128:(rb + 1) * 128, cb * 128:(cb + 1) * 128] *= sc[rb, cb]
    assert np.array_equal(O.dequantize_weight_blocks(codes, sc), ref)


def pin_activation_groups_per_row():
    """Activation groups run along a token's row: row 0 is 1e-3 in columns
    0..127 and 100 in 128..255, row 1 the other way round.  Worked by hand:
    100 = 0.78125 * 2^7 needs 2^-2 (448 / 4 = 112 >= 100, 448 / 8 = 56 <
    100); 1e-3 = 0.512 * 2^-9 needs 2^-18 (448 * 2^-18 = 1.709e-3, half that
    falls short).  Each value is then a multiple of a code: 100 / 2^-2 = 400
    lies halfway between the codes 384 (mantissa 100) and 416 (101) and goes
    to the even 384, so 100 -> 96; 1e-3 / 2^-18 = 262.144 -> 256, so
    1e-3 -> 2^-10."""
    x = np.zeros((2, 256))
    x[0, :128], x[0, 128:] = 1e-3, 100.0
    x[1, :128], x[1, 128:] = 100.0, 1e-3
    codes, scales = O.quantize_groups(x)
    assert scales.tolist() == [[2.0 ** -18, 0.25], [0.25, 2.0 ** -18]]
    deq = O.fp8_activation(x)
    assert np.all(deq[0, :128] == 2.0 ** -10) and np.all(deq[0, 128:] == 96.0)
    assert np.all(deq[1, :128] == 96.0) and np.all(deq[1, 128:] == 2.0 ** -10)


def _brute_quant(row):
    """Quantise-dequantise one row in groups of 128 without the oracle: the
    scale 2^ceil(log2(max|x| / 448)) (the smallest power of two s with
    448 s >= max|x|), codes by PyTorch's E4M3 cast of x / s."""
    out = []
    for g in range(0, len(row), 128):
        grp = row[g:g + 128]
        amax = max(abs(v) for v in grp)
        s = 2.0 ** math.ceil(math.log2(amax / 448.0)) if amax > 0 else 1.0
        q = torch.tensor([v / s for v in grp], dtype=torch.float64).to(torch.float32).to(torch.float8_e4m3fn)
        out += [float(v) * s for v in q.double().tolist()]
    return out


def pin_fp8_projections_brute_force(dims=TINY, L=3):
    """FP8 projections on a micro case by scalar loops: W_DQ, W_DKV, W_KR
    and W_O from E4M3 codes and block scales (PyTorch's E4M3 values), the
    hidden state quantised per token and 128 columns before the down
    projections, the attention output rounded to bfloat16 (PyTorch) and
    quantised the same way before W_O; the other projections in float64.
    Then the decode of the last token against a cache of the first L-1 rows
    gives the prefill's last row."""
    W = _weights(dims, 52)
    wl = make_workload(1, dims=dims, weights_fp8=True)
    for n, (codes, sc) in wl.weights_fp8.items():
        vals = _torch_e4m3_values(codes)
        for r in range(vals.shape[0]):
            for cb in range(vals.shape[1] // 128):
                vals[r, cb * 128:(cb + 1) * 128] *= sc[r // 128, cb]
        W[n] = vals
    h = _h(L, dims, 53) * 3.0
    got = O.prefill(dims, W, h, weights_fp8=True)

    def mv(M, x):
        return [sum(M[r][c] * x[c] for c in range(len(x))) for r in range(len(M))]

    def rot(x, p):
        out = list(x)
        for k in range(len(x) // 2):
            a = p * dims.rope_base ** (-2.0 * k / len(x))
            out[2 * k] = x[2 * k] * math.cos(a) - x[2 * k + 1] * math.sin(a)
            out[2 * k + 1] = x[2 * k] * math.sin(a) + x[2 * k + 1] * math.cos(a)
        return out

    Wl = {k: v.tolist() for k, v in W.items()}
    hq = [_brute_quant(h[t].tolist()) for t in range(L)]
    ckv = [mv(Wl["w_dkv"], hq[t]) for t in range(L)]
    kr = [rot(mv(Wl["w_kr"], hq[t]), t) for t in range(L)]
    for t in range(L):
        cq = mv(Wl["w_dq"], hq[t])
        qc_all, qr_all = mv(Wl["w_uq"], cq), mv(Wl["w_qr"], cq)
        ocat = []
        for i in range(dims.n_heads):
            qc = qc_all[i * dims.d_nope:(i + 1) * dims.d_nope]
            qr = rot(qr_all[i * dims.d_rope:(i + 1) * dims.d_rope], t)
            scores, vals = [], []
            for j in range(t + 1):
                kc = mv(Wl["w_uk"][i * dims.d_nope:(i + 1) * dims.d_nope], ckv[j])
                v = mv(Wl["w_uv"][i * dims.d_v:(i + 1) * dims.d_v], ckv[j])
                scores.append(sum(a * b for a, b in zip(qc + qr, kc + kr[j])) / math.sqrt(dims.d_nope + dims.d_rope))
                vals.append(v)
            mx = max(scores)
            ex = [math.exp(s - mx) for s in scores]
            z = sum(ex)
            ocat += [sum(ex[j] / z * vals[j][c] for j in range(t + 1)) for c in range(dims.d_v)]
        o16 = torch.tensor(ocat, dtype=torch.float64).to(torch.bfloat16).double().tolist()
        u = mv(Wl["w_o"], _brute_quant(o16))
        assert np.allclose(got["u"][t], u, rtol=1e-10, atol=1e-12)
        assert np.allclose(got["c_kv"][t], ckv[t], rtol=1e-11, atol=1e-12)
    rows = np.concatenate([got["c_kv"][:L - 1], got["k_r"][:L - 1]], axis=1)
    dec = O.decode(dims, W, h[L - 1:], rows, weights_fp8=True)
    assert np.allclose(dec["u"][0], got["u"][L - 1], rtol=1e-10, atol=1e-12)


ALL_PINS = [pin_absorbed_equals_plain, pin_softmax_rows, pin_causal, pin_single_key,
            pin_zero_query, pin_head_isolation, pin_mha_special_case, pin_rope_rotation, pin_rope_in_scores,
            pin_yarn_frequencies, pin_yarn_in_scores, pin_yarn_blend_hand_worked, pin_prefill_decode_agree,
            pin_e4m3_definition, pin_e4m3_rounding, pin_e4m3_library, pin_quantize_latent_hand_worked,
            pin_quantize_latent_bound,
            pin_fp8_row_layout, pin_round_bf16, pin_decode_fp8_new_rows, pin_brute_force,
            pin_weight_blocks_layout, pin_activation_groups_per_row, pin_fp8_projections_brute_force]


# ---------------------------------------------------------------------------
# Tests
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_random_shapes(seed):
    rng = np.random.Generator(np.random.PCG64(100 + seed))
    dr = 2 * int(rng.integers(1, 5))
    d = Dims(d_model=int(rng.integers(8, 40)), n_heads=int(rng.integers(1, 5)),
             d_nope=int(rng.integers(2, 12)), d_rope=dr, d_v=int(rng.integers(2, 12)),
             d_c=int(rng.integers(4, 24)), d_cq=int(rng.integers(4, 24)))
    pin_absorbed_equals_plain(d, L=int(rng.integers(3, 30)), n_q=int(rng.integers(1, 3)), seed=seed)


def test_cache_size_closed_form():
    """P4: the cache holds only c_KV and k_R: (d_c + d_R) elements per token,
    against a key and a value per head for MHA.  Dimensions from the pages."""
    g = json.load(open(os.path.join(GOLDEN, "dsv3_mla_dims.json")))
    d = Dims(d_model=g["d_model"], n_heads=g["n_heads"], d_nope=g["d_head"], d_rope=g["d_rope"],
             d_v=g["d_head"], d_c=g["d_c"], d_cq=g["d_cq"])
    assert d == DSV3
    e = g["expected"]
    assert O.cache_elements_per_token(d) == e["mla_cache_elements_per_token"]
    assert O.mha_elements_per_token(d) == e["mha_cache_elements_per_token"]
    assert 2 * O.cache_elements_per_token(d) == e["mla_cache_bytes_per_token_bf16"]
    assert 2 * O.cache_elements_per_token(d) * g["n_layers"] == e["mla_cache_bytes_per_token_61_layers_bf16"]
    assert O.cache_elements_per_token(TINY) == 80 and O.mha_elements_per_token(TINY) == 256
    # and the oracle's decode really only needs those rows: the new row it
    # returns has exactly that width
    W = _weights(TINY, 1)
    r = O.decode(TINY, W, _h(1, TINY), np.zeros((3, TINY.d_row)))
    assert r["row_new"].shape == (1, O.cache_elements_per_token(TINY))


def test_tiny_workload_end_to_end():
    """The tiny workload's prefill + 8 decode steps agree with one 72-token
    prefill on the workload's own seeded inputs."""
    wl = make_workload(1)
    d = wl.dims
    W = {k: v.astype(np.float64) for k, v in wl.weights_f32.items()}
    h = wl.h_f32[0].astype(np.float64)
    full = O.prefill(d, W, h)
    r = O.prefill(d, W, h[:wl.seq_len])
    rows = np.concatenate([r["c_kv"], r["k_r"]], axis=1)
    assert np.allclose(r["u"], full["u"][:wl.seq_len], rtol=1e-12, atol=1e-12)
    for s in range(wl.n_steps):
        t = wl.seq_len + s
        dd = O.decode(d, W, h[t:t + 1], rows)
        rows = np.concatenate([rows, dd["row_new"]], axis=0)
        assert np.allclose(dd["u"][0], full["u"][t], rtol=1e-12, atol=1e-12)


def test_head_subset_matches_full():
    W = _weights(TINY, 2)
    h = _h(12, TINY, 3)
    full = O.prefill(TINY, W, h)
    part = O.prefill(TINY, W, h, rows=[0, 5, 11], heads=[1, 3])
    assert part["u"] is None
    assert np.allclose(part["o"][:, [1, 3]], full["o"][[0, 5, 11]][:, [1, 3]], rtol=1e-13, atol=1e-14)
