"""Plain CPU oracle for DeepSeek-V3 Multi-head Latent Attention (MLA).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or links
this module: only the tests, ``__graft_entry__.smoke()`` and the cpu_baseline
leg of ``bench.py`` use it.  It shares no code with the HIP library; the only
module both sides consume is ``mla_inputs`` (seeded draws, no arithmetic of the
method).

Everything is float64 numpy and follows the non-absorbed MLA equations in the
order the pages write them:
  "DeepSeek V3 technical paper, close reading" notes (hk.pswp.cn), section 2.1
  "Multi-Head Latent Attention", items "Key and Value compression", "Query
  compression" and "attention computation";
  the V3 technical-report summary (cooktownmusic.com), "hyperparameters"
  paragraph, for the dimensions;
  the same section 2.1, "advantages of MLA", for what the cache holds.

Readings of passages the pages leave open (their sub- and superscripts were
lost in extraction):
  * the RoPE key k_R is one vector per token shared by all heads (the cache
    holds only c_KV and k_R); the RoPE query q_R is split per head;
  * RoPE rotates interleaved pairs (2k, 2k+1) by p * base^(-2k/d_R), with p the
    0-based position in the sequence;
  * attention is causal: query at position t sees keys 0..t;
  * the softmax scale is 1/sqrt(d_h + d_R) (d_h the per-head content width);
  * YaRN (V3 highlights page, highlight 13: "scale 40, base 1, factor 32"
    with garbled names) is read as the YaRN method with s = 40,
    beta_slow = 1, beta_fast = 32 over a 4K original context: per-pair
    frequencies blended linearly in the pair's rotation count, and the
    logits divided by the temperature t with sqrt(1/t) = 0.1 ln s + 1;
  * head i owns the i-th contiguous slice of each up-projection output and of
    W_O's input;
  * weights are stored [out][in] because the pages write W*h;
  * decode appends the new tokens first: the n_q queries of a sequence with L
    tokens sit at positions L-n_q..L-1.

Pins (tests/test_oracle.py): absorbed == non-absorbed form; softmax rows sum
to 1; causal invariance; the closed-form cache size; single-key and
zero-query closed forms; the plain-MHA special case against PyTorch's
scaled_dot_product_attention; RoPE rotation properties; prefill + decode ==
longer prefill; a scalar brute force on a micro case.  The RoPE pairing
convention (interleaved versus half-split) is a reading the mathematics does
not fix: any pairing passes the rotation pins, so that one choice is parity
unpinned beyond agreement of the two sides on the same reading.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "rope", "rope_freqs", "yarn_on", "compress_kv", "project_queries", "head_keys_values", "attend_head",
    "output_projection", "prefill", "decode", "decode_absorbed",
    "cache_elements_per_token", "mha_elements_per_token", "softmax_scale",
    "E4M3_MAX", "FP8_GROUP", "e4m3_decode", "e4m3_encode", "round_bf16", "fp8_group_scale", "quantize_latent",
    "fp8_row_bytes",
    "dequantize_fp8_rows",
    "FP8_WEIGHTS", "quantize_groups", "dequantize_groups", "fp8_activation", "dequantize_weight_blocks",
]


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# RoPE (section 2.1: "ROPE(W_KR h)" and "ROPE(W_QR c_Q)")
# ---------------------------------------------------------------------------

def yarn_on(dims):
    return dims.yarn_factor not in (0.0, 1.0)


def rope_freqs(dims):
    """Angular frequency of each rotated pair k = 0..d_R/2-1.

    Plain RoPE: theta_k = base^(-2k/d_R).  With YaRN (named, with its
    constants, in highlight 13 of the V3 highlights page; the steps are those
    of the YaRN method's "NTK-by-parts" interpolation): pair k turns
    r_k = L_orig * theta_k / (2 pi) times over the original context; pairs
    that turn fewer than beta_slow times are interpolated (theta_k / s), pairs
    that turn more than beta_fast times are kept, and in between the two
    frequencies are blended linearly in r_k."""
    d_r = dims.d_rope
    k = np.arange(d_r // 2, dtype=np.float64)
    theta = np.power(float(dims.rope_base), -2.0 * k / d_r)
    if not yarn_on(dims):
        return theta
    s = float(dims.yarn_factor)
    r = float(dims.yarn_orig_len) * theta / (2.0 * np.pi)
    lo, hi = float(dims.yarn_beta_slow), float(dims.yarn_beta_fast)
    gamma = np.clip((r - lo) / (hi - lo), 0.0, 1.0)   # 0: interpolate, 1: keep
    return (1.0 - gamma) * (theta / s) + gamma * theta


def _yarn_theta(dims):
    """The YaRN frequencies, or None for plain RoPE (rope() then forms
    base^(-2k/d_R) itself)."""
    return rope_freqs(dims) if yarn_on(dims) else None


def rope(x, pos, base, theta=None):
    """Rotate interleaved pairs (x[2k], x[2k+1]) by angle pos * theta_k, with
    theta_k = base^(-2k/d_R) unless the frequencies are given.

    x: [..., d_R]; pos: integer array broadcastable to x.shape[:-1]."""
    x = _f64(x)
    d_r = x.shape[-1]
    if theta is None:
        k = np.arange(d_r // 2, dtype=np.float64)
        theta = np.power(float(base), -2.0 * k / d_r)
    ang = _f64(pos)[..., None] * _f64(theta)
    c, s = np.cos(ang), np.sin(ang)
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def softmax_scale(dims):
    """1/sqrt(d_h + d_R): section 2.1, attention computation.  With YaRN the
    logits are further divided by the method's temperature t, where
    sqrt(1/t) = 0.1 ln(s) + 1."""
    scale = 1.0 / np.sqrt(dims.d_nope + dims.d_rope)
    if yarn_on(dims):
        scale *= (0.1 * np.log(float(dims.yarn_factor)) + 1.0) ** 2
    return scale


# ---------------------------------------------------------------------------
# Key/value compression (section 2.1, "Key and Value compression")
# ---------------------------------------------------------------------------

def compress_kv(W, h, pos, dims):
    """c_KV = W_DKV h and k_R = RoPE(W_KR h) for tokens h [T][d_model] at
    positions pos [T].  These two are the whole cached row."""
    h = _f64(h)
    c_kv = h @ _f64(W["w_dkv"]).T
    k_r = rope(h @ _f64(W["w_kr"]).T, pos, dims.rope_base, _yarn_theta(dims))
    return c_kv, k_r


def head_keys_values(W, c_kv, i, dims):
    """Head i's content keys k_C = W_UK c_KV and values v_C = W_UV c_KV
    (rows i*d_h..(i+1)*d_h of the up-projections)."""
    w_uk_i = _f64(W["w_uk"])[i * dims.d_nope:(i + 1) * dims.d_nope]
    w_uv_i = _f64(W["w_uv"])[i * dims.d_v:(i + 1) * dims.d_v]
    c_kv = _f64(c_kv)
    return c_kv @ w_uk_i.T, c_kv @ w_uv_i.T


# ---------------------------------------------------------------------------
# Query compression (section 2.1, "Query compression")
# ---------------------------------------------------------------------------

def project_queries(W, h, pos, dims):
    """c_Q = W_DQ h; q_C = W_UQ c_Q split into heads; q_R = RoPE(W_QR c_Q)
    split into heads.  Returns q_C [T][n_h][d_h], q_R [T][n_h][d_R]."""
    h = _f64(h)
    T = h.shape[0]
    c_q = h @ _f64(W["w_dq"]).T
    q_c = (c_q @ _f64(W["w_uq"]).T).reshape(T, dims.n_heads, dims.d_nope)
    q_r_raw = (c_q @ _f64(W["w_qr"]).T).reshape(T, dims.n_heads, dims.d_rope)
    q_r = rope(q_r_raw, _f64(pos)[:, None], dims.rope_base, _yarn_theta(dims))
    return q_c, q_r


# ---------------------------------------------------------------------------
# Attention (section 2.1, "attention computation")
# ---------------------------------------------------------------------------

def attend_head(q_c_i, q_r_i, qpos, k_c_i, k_r, v_i, scale, return_probs=False):
    """o_{t,i} = sum_{j<=t} softmax_j((q_{t,i} . k_{j,i}) * scale) v_{j,i}
    with q = [q_C; q_R] and k = [k_C; k_R].

    q_c_i [T][d_h], q_r_i [T][d_R], qpos [T]; k_c_i [L][d_h], k_r [L][d_R],
    v_i [L][d_v].  The full score row is formed, masked, and normalised in one
    piece (no online softmax)."""
    s = (_f64(q_c_i) @ _f64(k_c_i).T + _f64(q_r_i) @ _f64(k_r).T) * scale
    L = s.shape[1]
    visible = np.arange(L)[None, :] <= np.asarray(qpos)[:, None]
    s = np.where(visible, s, -np.inf)
    m = np.max(s, axis=1, keepdims=True)
    e = np.exp(s - m)
    p = e / np.sum(e, axis=1, keepdims=True)
    o = p @ _f64(v_i)
    return (o, p) if return_probs else o


def output_projection(W, o):
    """u_t = W_O [o_{t,1}; ...; o_{t,n_h}]; o is [T][n_h][d_v]."""
    o = _f64(o)
    return o.reshape(o.shape[0], -1) @ _f64(W["w_o"]).T


# ---------------------------------------------------------------------------
# One sequence end to end
# ---------------------------------------------------------------------------

def _heads(dims, heads):
    return range(dims.n_heads) if heads is None else heads


def prefill(dims, W, h, rows=None, heads=None, return_probs=False, weights_fp8=False):
    """Causal MLA over one whole sequence h [L][d_model] (positions 0..L-1).

    rows: query positions to evaluate (default all); heads: heads to evaluate
    (default all; u is only formed when all heads are).  Returns a dict with
    u [R][d_model] (or None), o [R][n_h][d_v] (zeros for skipped heads),
    and the cache rows c_kv [L][d_c], k_r [L][d_R].  weights_fp8: the
    projections of FP8_WEIGHTS are FP8 products (W holds their dequantised
    weights, dequantize_weight_blocks); their inputs, h and the attention
    output o, enter as fp8_activation of themselves."""
    h = _f64(h)
    L = h.shape[0]
    pos = np.arange(L)
    hp = fp8_activation(h) if weights_fp8 else h
    c_kv, k_r = compress_kv(W, hp, pos, dims)
    qpos = pos if rows is None else np.asarray(rows)
    q_c, q_r = project_queries(W, hp[qpos], qpos, dims)
    scale = softmax_scale(dims)
    o = np.zeros((len(qpos), dims.n_heads, dims.d_v))
    probs = {}
    for i in _heads(dims, heads):
        k_c_i, v_i = head_keys_values(W, c_kv, i, dims)
        res = attend_head(q_c[:, i], q_r[:, i], qpos, k_c_i, k_r, v_i, scale, return_probs)
        if return_probs:
            o[:, i], probs[i] = res
        else:
            o[:, i] = res
    u = None
    if heads is None:
        u = output_projection(W, fp8_activation(round_bf16(o.reshape(o.shape[0], -1))) if weights_fp8 else o)
    out = dict(u=u, o=o, c_kv=c_kv, k_r=k_r)
    if return_probs:
        out["probs"] = probs
    return out


def decode(dims, W, h, cache_rows, heads=None, cache_fp8=False, weights_fp8=False):
    """n_q new tokens h [n_q][d_model] appended to one sequence whose first
    cached rows ``cache_rows`` [L-n_q][d_c+d_R] (each [c_KV || k_R]) are given.
    The new tokens take positions L-n_q..L-1 and query i sees keys
    0..L-n_q+i.  Returns u [n_q][d_model] (None when heads is a subset),
    o [n_q][n_h][d_v] and the new cache rows [n_q][d_c+d_R] (before any
    quantisation).  cache_fp8: the cache holds c_KV in FP8 (E4M3 with a scale
    per group of FP8_GROUP columns), so the new tokens' c_KV is attended in
    its quantised form, as every cached row is (``cache_rows`` are then the
    dequantised rows, dequantize_fp8_rows).  The quantiser reads c_KV
    rounded to bfloat16, the type the compression produces in a bf16 layer
    (the FP8 cache exists for bf16 layers only), so that a code is decided
    from the value the layer holds, not from its float64 form.
    weights_fp8: as in prefill, the FP8_WEIGHTS projections read
    fp8_activation(h) and fp8_activation(o rounded to bfloat16)."""
    h = _f64(h)
    cache_rows = _f64(cache_rows)
    n_q = h.shape[0]
    L = cache_rows.shape[0] + n_q
    qpos = np.arange(L - n_q, L)
    if weights_fp8:
        h = fp8_activation(h)
    c_new, kr_new = compress_kv(W, h, qpos, dims)
    c_att = c_new
    if cache_fp8:
        codes, scales = quantize_latent(round_bf16(c_new))
        c_att = _dequantize_latent(codes, scales)
    c_kv = np.concatenate([cache_rows[:, :dims.d_c], c_att], axis=0)
    k_r = np.concatenate([cache_rows[:, dims.d_c:], kr_new], axis=0)
    q_c, q_r = project_queries(W, h, qpos, dims)
    scale = softmax_scale(dims)
    o = np.zeros((n_q, dims.n_heads, dims.d_v))
    for i in _heads(dims, heads):
        k_c_i, v_i = head_keys_values(W, c_kv, i, dims)
        o[:, i] = attend_head(q_c[:, i], q_r[:, i], qpos, k_c_i, k_r, v_i, scale)
    u = None
    if heads is None:
        u = output_projection(W, fp8_activation(round_bf16(o.reshape(o.shape[0], -1))) if weights_fp8 else o)
    return dict(u=u, o=o, row_new=np.concatenate([c_new, kr_new], axis=1))


def decode_absorbed(dims, W, h, cache_rows):
    """The same decode computed in latent space, used only to pin the
    non-absorbed form above: by associativity q_C,i . (W_UK,i c_KV) equals
    (W_UK,i^T q_C,i) . c_KV, and sum_j p_j W_UV,i c_KV,j equals
    W_UV,i sum_j p_j c_KV,j."""
    h = _f64(h)
    cache_rows = _f64(cache_rows)
    n_q = h.shape[0]
    L = cache_rows.shape[0] + n_q
    qpos = np.arange(L - n_q, L)
    c_new, kr_new = compress_kv(W, h, qpos, dims)
    rows = np.concatenate([cache_rows, np.concatenate([c_new, kr_new], axis=1)], axis=0)
    q_c, q_r = project_queries(W, h, qpos, dims)
    w_uk = _f64(W["w_uk"]).reshape(dims.n_heads, dims.d_nope, dims.d_c)
    w_uv = _f64(W["w_uv"]).reshape(dims.n_heads, dims.d_v, dims.d_c)
    scale = softmax_scale(dims)
    o = np.zeros((n_q, dims.n_heads, dims.d_v))
    for t in range(n_q):
        for i in range(dims.n_heads):
            q_lat = w_uk[i].T @ q_c[t, i]                  # [d_c]
            q_full = np.concatenate([q_lat, q_r[t, i]])    # [d_c + d_R]
            n_vis = qpos[t] + 1
            s = rows[:n_vis] @ q_full * scale
            p = np.exp(s - s.max())
            p /= p.sum()
            o_lat = p @ rows[:n_vis, :dims.d_c]
            o[t, i] = w_uv[i] @ o_lat
    return dict(u=output_projection(W, o), o=o)


# ---------------------------------------------------------------------------
# Cache size (section 2.1, "advantages of MLA": only c_KV and k_R are cached)
# ---------------------------------------------------------------------------

def cache_elements_per_token(dims):
    """Elements cached per token and layer by MLA: c_KV plus the shared k_R."""
    return dims.d_c + dims.d_rope


def mha_elements_per_token(dims):
    """Elements a standard multi-head attention caches: a key and a value per head."""
    return 2 * dims.n_heads * dims.d_nope


# ---------------------------------------------------------------------------
# FP8 latent cache (the FP8 framework of the V3 technical-report summary,
# "FP8 training framework" paragraph and figure 7: values kept in FP8 with
# fine-grained scaling, a scale per small group of elements, the group of 128
# elements the figure's accumulation interval gives; the 18-highlights page,
# highlight 5, FP8 for computation and storage).  Reading: a cached row keeps
# c_KV as E4M3 codes with one fp32 scale per FP8_GROUP consecutive columns,
# and k_R in the layer dtype.  The pages do not say how a scale is chosen;
# here it is the smallest power of two s with 448 s >= the group's largest
# magnitude (an all-zero group takes 1; s is kept at or above 2^-126, the
# smallest normal fp32), so that no value saturates and code * s is exact.
# ---------------------------------------------------------------------------

E4M3_MAX = 448.0
FP8_GROUP = 128


def e4m3_decode(codes):
    """Values of E4M3 codes (OCP 8-bit floating point, E4M3: 1 sign, 4
    exponent bits with bias 7, 3 mantissa bits; exponent field 0 encodes
    subnormals m/8 * 2^-6; S.1111.111 is NaN; there is no infinity)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.power(2.0, e - 7))
    mag = np.where((e == 15) & ((c & 7) == 7), np.nan, mag)
    return sign * mag


def _e4m3_magnitudes():
    return e4m3_decode(np.arange(127))   # codes 0..126: every finite non-negative value, increasing


def e4m3_encode(x):
    """Nearest E4M3 code to each value, ties to the even code (round to
    nearest even); magnitudes beyond 448 saturate to 448 (reading: the
    format has no infinity and the quantiser never exceeds 448); NaN maps to
    the NaN code; the sign of zero is kept."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    mags = _e4m3_magnitudes()
    hi = np.clip(np.searchsorted(mags, a, side="left"), 0, 126)   # first value >= a
    lo = np.clip(hi - 1, 0, 126)
    d_lo, d_hi = a - mags[lo], mags[hi] - a
    code = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    code = np.where(tie, np.where(lo % 2 == 0, lo, hi), code)
    code = np.where(np.signbit(x), code | 0x80, code)
    code = np.where(np.isnan(x), 0x7F, code)
    return code.astype(np.uint8)


def round_bf16(x):
    """Nearest bfloat16 value (8 significant bits) to each value, ties to
    even (values in bfloat16's normal range)."""
    f, e = np.frexp(_f64(x))                 # x = f * 2^e, 0.5 <= |f| < 1
    return np.ldexp(np.round(f * 256.0) / 256.0, e)   # np.round: half to even


def fp8_group_scale(amax):
    """Smallest power of two s >= 2^-126 with 448 s >= amax (1 when amax is
    0), for each group maximum in ``amax``."""
    a = _f64(amax)
    # amax = f * 2^e with 0.5 <= f < 1; 448 * 2^(e-10) = 0.4375 * 2^e < amax,
    # so s is 2^(e-9) (448 * 2^(e-9) = 0.875 * 2^e) or, if that is short, 2^(e-8)
    f, e = np.frexp(a)
    s = np.ldexp(1.0, e - 9)
    s = np.where(E4M3_MAX * s >= a, s, 2.0 * s)
    s = np.maximum(s, 2.0 ** -126)
    return np.where(a > 0, s, 1.0)


def quantize_groups(x):
    """Rows [T][K] (K a multiple of FP8_GROUP) -> (codes [T][K] uint8,
    scales [T][K/FP8_GROUP]): per group of FP8_GROUP consecutive columns of
    a row, scale = fp8_group_scale(max|x|) and each value takes the E4M3
    code nearest to x / scale."""
    c = _f64(x)
    T, K = c.shape
    g = c.reshape(T, K // FP8_GROUP, FP8_GROUP)
    amax = np.max(np.abs(g), axis=2)
    scales = fp8_group_scale(amax)
    codes = e4m3_encode(g / scales[:, :, None]).reshape(T, K)
    return codes, scales


def dequantize_groups(codes, scales):
    """Inverse of quantize_groups: each code's value times its group's scale."""
    T, K = codes.shape
    v = e4m3_decode(codes).reshape(T, K // FP8_GROUP, FP8_GROUP) * _f64(scales)[:, :, None]
    return v.reshape(T, K)


def quantize_latent(c_kv):
    """c_KV rows [T][d_c] -> (codes, scales): quantize_groups over the latent
    columns (a scale per FP8_GROUP columns of each row)."""
    return quantize_groups(c_kv)


def _dequantize_latent(codes, scales):
    return dequantize_groups(codes, scales)


def fp8_row_bytes(dims):
    """Bytes of one FP8 cache row: d_c codes, d_R bf16 values of k_R, and
    d_c / FP8_GROUP fp32 scales, in that order."""
    return dims.d_c + 2 * dims.d_rope + 4 * (dims.d_c // FP8_GROUP)


def dequantize_fp8_rows(rows, dims):
    """Cache rows as stored ([T][fp8_row_bytes] uint8, little-endian) ->
    [T][d_c + d_R] float64: codes times their group's scale, then k_R."""
    r = np.ascontiguousarray(np.asarray(rows, dtype=np.uint8))
    T = r.shape[0]
    d_c, d_r = dims.d_c, dims.d_rope
    codes = r[:, :d_c]
    kr_bits = r[:, d_c:d_c + 2 * d_r].copy().view(np.uint16).astype(np.uint32)
    k_r = (kr_bits << np.uint32(16)).view(np.float32).astype(np.float64)
    scales = r[:, d_c + 2 * d_r:].copy().view(np.float32).astype(np.float64)
    return np.concatenate([_dequantize_latent(codes, scales), k_r.reshape(T, d_r)], axis=1)


# ---------------------------------------------------------------------------
# FP8 projections: block-scaled GEMMs (the FP8 framework of the V3
# technical-report summary, "FP8 training framework" paragraph and figures 6
# and 7; the CSDN blog, "FP8 mixed-precision training framework": the GEMMs
# take FP8 inputs and produce higher-precision outputs, activations and
# weights are scaled in blocks, and figure 7 gives 128 elements as the
# interval of high-precision accumulation).  Readings: an activation is
# scaled per token and per group of FP8_GROUP consecutive input columns (one
# scale per accumulation interval of each row); a weight per block of
# FP8_GROUP output rows by FP8_GROUP input columns; scales are powers of two
# chosen as for the latent cache (fp8_group_scale); the products are exact
# and accumulate in at least fp32, so the result is the plain product of the
# dequantised operands.  The FP8 projections are those between the model's
# hidden width and the latent or head space that read the hidden state or
# write the layer output: W_DQ, W_DKV, W_KR and W_O (FP8_WEIGHTS); the
# up-projections W_UQ, W_QR, W_UK and W_UV, which act inside the latent and
# head space, keep the layer dtype.  An activation is quantised from the
# value the layer holds in bfloat16 (h as given; o rounded to bfloat16), as
# for the latent cache.
# ---------------------------------------------------------------------------

FP8_WEIGHTS = ("w_dq", "w_dkv", "w_kr", "w_o")


def fp8_activation(x):
    """The values an FP8 product reads for activations x [T][K]: the
    dequantised quantize_groups(x)."""
    codes, scales = quantize_groups(x)
    return dequantize_groups(codes, scales)


def dequantize_weight_blocks(codes, scales):
    """Weight codes [N][K] (uint8 E4M3) with one scale per block of FP8_GROUP
    rows by FP8_GROUP columns (scales [ceil(N/FP8_GROUP)][K/FP8_GROUP];
    the last row block may be short) -> [N][K] float64 values."""
    c = np.asarray(codes)
    N, K = c.shape
    sc = _f64(scales)
    rb = np.arange(N) // FP8_GROUP
    cb = np.arange(K) // FP8_GROUP
    return e4m3_decode(c) * sc[rb[:, None], cb[None, :]]
