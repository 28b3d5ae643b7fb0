"""Seeded synthetic inputs for the MLA workloads.

This module only draws numbers and lays them out; it holds none of the
attention arithmetic.  Both the CPU oracle (through the tests) and the GPU
path (through the binding, tests and bench) consume what it returns, and
neither side imports the other.

Recipe (shared by every workload):
  * one numpy ``Generator(PCG64(1000 + workload_id))`` per workload;
  * draw order: W_DQ, W_UQ, W_QR, W_DKV, W_KR, W_UK, W_UV, W_O, then h, then
    the per-sequence cache lengths (ragged workload only), then the cached
    latent rows; the block permutation (paged workload only) comes from a
    stream of its own, ``PCG64(1000 + workload_id + 7919)``, so it is the
    same whether or not the rows are drawn on the host (the benchmark draws
    the rows of its large workloads on the device: ``cache_rows=False``);
  * weights are N(0, 1/fan_in) with fan_in the input dimension, hidden states
    N(0, 1), cached latent rows N(0, 1) for both the c_KV and the k_R columns;
  * values are drawn as float32 and rounded to bfloat16 with
    round-to-nearest-even for the bf16 workloads.  The float32 view of the
    rounded values (``*_f32``) is exactly what the device receives.

Dimensions follow DeepSeek-V3 as the pages give them (hidden 7168, 128 heads
of 128, KV latent 512, query latent 1536: the V3 summary page,
"hyperparameters" paragraph, and the "18 highlights" page, highlight 2); the
decoupled RoPE width 64 is not on the pages and is taken from the workload
description.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "Dims", "TINY", "DSV3", "Workload", "WORKLOADS", "make_workload",
    "bf16_round", "bf16_bits_to_f32", "WEIGHT_NAMES", "weight_shapes",
    "draw_weights", "scatter_paged", "block_table_rows", "FP8_WEIGHT_NAMES", "fp8_weight_blocks",
]


@dataclass(frozen=True)
class Dims:
    d_model: int
    n_heads: int
    d_nope: int   # per-head width of the up-projected (content) query/key
    d_rope: int   # width of the decoupled RoPE query/key
    d_v: int      # per-head value width
    d_c: int      # KV latent width
    d_cq: int     # query latent width
    rope_base: float = 10000.0
    # YaRN context extension (factor 1: plain RoPE).  The V3 highlights page
    # (highlight 13) names YaRN with the constants 40, 1 and 32, read as the
    # scale factor s, beta_slow and beta_fast, over the 4K pre-training
    # context the same passage extends to 128K.
    yarn_factor: float = 1.0
    yarn_orig_len: int = 4096
    yarn_beta_slow: float = 1.0
    yarn_beta_fast: float = 32.0

    @property
    def d_row(self) -> int:
        """Width of one cached row: [c_KV || k_R]."""
        return self.d_c + self.d_rope


TINY = Dims(d_model=256, n_heads=4, d_nope=32, d_rope=16, d_v=32, d_c=64, d_cq=96)
DSV3 = Dims(d_model=7168, n_heads=128, d_nope=128, d_rope=64, d_v=128, d_c=512, d_cq=1536)

WEIGHT_NAMES = ("w_dq", "w_uq", "w_qr", "w_dkv", "w_kr", "w_uk", "w_uv", "w_o")


def weight_shapes(d: Dims) -> Dict[str, tuple]:
    """[out][in] shapes; the pages write every projection as W·x."""
    return {
        "w_dq": (d.d_cq, d.d_model),
        "w_uq": (d.n_heads * d.d_nope, d.d_cq),
        "w_qr": (d.n_heads * d.d_rope, d.d_cq),
        "w_dkv": (d.d_c, d.d_model),
        "w_kr": (d.d_rope, d.d_model),
        "w_uk": (d.n_heads * d.d_nope, d.d_c),
        "w_uv": (d.n_heads * d.d_v, d.d_c),
        "w_o": (d.d_model, d.n_heads * d.d_v),
    }


# ----------------------------------------------------------------------------
# bf16 rounding (input preparation only)
# ----------------------------------------------------------------------------

def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round-to-nearest-even.

    Inputs are finite by construction (normal draws)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _normal(rng: np.random.Generator, shape, scale: float, bf16: bool, chunk: int = 1 << 24):
    """Draw N(0, scale^2) as float32 (in fixed-size chunks so that very large
    arrays never need a float64 temporary).  Returns (f32 values, bf16 bits or None)."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    bits = np.empty(n, dtype=np.uint16) if bf16 else None
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = rng.standard_normal(e - s, dtype=np.float32)
        if scale != 1.0:
            v *= np.float32(scale)
        if bf16:
            b = bf16_round(v)
            bits[s:e] = b
            out[s:e] = bf16_bits_to_f32(b)
        else:
            out[s:e] = v
    out = out.reshape(shape)
    if bits is not None:
        bits = bits.reshape(shape)
    return out, bits


def draw_weights(rng: np.random.Generator, d: Dims, bf16: bool):
    f32, bits = {}, {}
    for name, shp in weight_shapes(d).items():
        v, b = _normal(rng, shp, 1.0 / np.sqrt(shp[1]), bf16)
        f32[name] = v
        bits[name] = b
    return f32, bits


# ----------------------------------------------------------------------------
# Workloads
# ----------------------------------------------------------------------------

@dataclass
class Workload:
    """One seeded synthetic workload.

    kind == "prefill": h is [B][L][d_model]; the whole sequence is new.
    kind == "decode":  h is [B][n_q][d_model]; sequence b has ``lens[b]``
        tokens after the n_q new ones are appended, so its first
        ``lens[b] - n_q`` cached rows are given in ``cache_f32[b]``.
    kind == "prefill+decode": tiny end-to-end check; h is [B][L + n_steps][d_model];
        the first L tokens are prefilled, then one token per decode step.
    """
    wid: int
    name: str
    dims: Dims
    dtype: str                      # "fp32" or "bf16"
    kind: str
    batch: int
    seq_len: int = 0                # prefill length
    n_q: int = 0                    # decode query tokens per sequence
    n_steps: int = 0                # decode steps after the prefill (tiny)
    lens: Optional[np.ndarray] = None          # [B] int32, lengths after append
    weights_f32: Dict[str, np.ndarray] = field(default_factory=dict)
    weights_bits: Dict[str, Optional[np.ndarray]] = field(default_factory=dict)
    h_f32: Optional[np.ndarray] = None
    h_bits: Optional[np.ndarray] = None
    cache_f32: Optional[List[np.ndarray]] = None   # per sequence [lens[b]-n_q][d_row]
    cache_bits: Optional[List[np.ndarray]] = None
    paged: bool = False
    block_size: int = 64
    block_perm: Optional[np.ndarray] = None        # physical block id of logical block k
    cache_fp8: bool = False                        # cached rows in the FP8 layout
    cache_fp8_rows: Optional[List[np.ndarray]] = None   # per sequence [lens[b]-n_q][row bytes] uint8
    # block-scaled FP8 projections: (E4M3 codes [out][in] uint8, float32
    # scales [ceil(out/128)][in/128]) by weight name (FP8_WEIGHT_NAMES)
    weights_fp8: Optional[Dict[str, tuple]] = None

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"


WORKLOADS = {
    1: dict(name="tiny-fp32-prefill64+decode8", dims=TINY, dtype="fp32", kind="prefill+decode",
            batch=1, seq_len=64, n_steps=8),
    2: dict(name="dsv3-decode-b32-len4096", dims=DSV3, dtype="bf16", kind="decode",
            batch=32, n_q=1, uniform_len=4096),
    3: dict(name="dsv3-prefill-b1-len4096", dims=DSV3, dtype="bf16", kind="prefill",
            batch=1, seq_len=4096),
    4: dict(name="dsv3-decode-b128-ragged32k-paged64", dims=DSV3, dtype="bf16", kind="decode",
            batch=128, n_q=1, ragged_max=32768, paged=True, block_size=64),
    5: dict(name="dsv3-decode-b4-len131072-nq2", dims=DSV3, dtype="bf16", kind="decode",
            batch=4, n_q=2, uniform_len=131072),
}


FP8_GROUP = 128   # columns of c_KV per scale in the FP8 cache rows


def fp8_cache_rows(rng: np.random.Generator, n: int, d_c: int, d_rope: int, chunk: int = 1 << 16) -> np.ndarray:
    """n cached rows in the FP8 cache layout, [n][d_c + 2*d_rope + 4*d_c/128]
    uint8: E4M3 codes of c_KV, k_R as bf16 bits, then one float32 scale per
    128 columns (little-endian).  Input data only: per row and group a scale
    2^-7, 2^-6 or 2^-5 is drawn uniformly (scales of the FP8 cache are powers
    of two) and the codes are those of N(0,1) draws divided by it (clamped
    to +-448), cast by PyTorch's float8_e4m3fn conversion; k_R is N(0,1)
    rounded to bf16.  The dequantised c_KV is then close to N(0,1), as in
    the bf16 workloads."""
    import torch
    G = d_c // FP8_GROUP
    out = np.empty((n, d_c + 2 * d_rope + 4 * G), dtype=np.uint8)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        m = e - s
        x = rng.standard_normal((m, d_c), dtype=np.float32)
        sc = np.ldexp(np.float32(1.0), rng.integers(-7, -4, (m, G))).astype(np.float32)
        q = np.clip(x.reshape(m, G, FP8_GROUP) / sc[:, :, None], -448.0, 448.0).reshape(m, d_c)
        out[s:e, :d_c] = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
        _, kr_bits = _normal(rng, (m, d_rope), 1.0, True)
        out[s:e, d_c:d_c + 2 * d_rope] = kr_bits.view(np.uint8).reshape(m, 2 * d_rope)
        out[s:e, d_c + 2 * d_rope:] = sc.view(np.uint8).reshape(m, 4 * G)
    return out


FP8_WEIGHT_NAMES = ("w_dq", "w_dkv", "w_kr", "w_o")   # the projections that may be block-scaled FP8


def fp8_weight_blocks(rng: np.random.Generator, shape, std: float, chunk_rows: int = 1024):
    """A weight [out][in] as E4M3 codes with one float32 scale per block of
    128 rows by 128 columns.  Input data only: per block a scale
    2^(e0 + d), d drawn uniformly from {-1, 0, 1} and 2^e0 the power of two
    nearest to std/32 (scales of FP8 weights are powers of two), and the
    codes are those of N(0, std^2) draws divided by their block's scale
    (clamped to +-448), cast by PyTorch's float8_e4m3fn conversion.  The
    dequantised weight is then close to N(0, std^2)."""
    import torch
    N, K = shape
    nb, kb = (N + 127) // 128, K // 128
    e0 = int(np.round(np.log2(std / 32.0)))
    scales = np.ldexp(np.float32(1.0), e0 + rng.integers(-1, 2, (nb, kb))).astype(np.float32)
    codes = np.empty((N, K), dtype=np.uint8)
    for r0 in range(0, N, chunk_rows):
        r1 = min(N, r0 + chunk_rows)
        x = rng.standard_normal((r1 - r0, K), dtype=np.float32) * np.float32(std)
        sc = np.repeat(scales, 128, axis=0)[r0:r1]            # each row's block scales [rows][kb]
        q = np.clip(x.reshape(r1 - r0, kb, 128) / sc[:, :, None], -448.0, 448.0).reshape(r1 - r0, K)
        codes[r0:r1] = torch.from_numpy(np.ascontiguousarray(q, dtype=np.float32)).to(
            torch.float8_e4m3fn).view(torch.uint8).numpy()
    return codes, scales


def make_workload(wid: int, *, dims: Optional[Dims] = None, batch: Optional[int] = None,
                  seq_len: Optional[int] = None, uniform_len: Optional[int] = None,
                  ragged_max: Optional[int] = None, n_q: Optional[int] = None,
                  paged: Optional[bool] = None, block_size: Optional[int] = None,
                  dtype: Optional[str] = None, seed: Optional[int] = None,
                  n_steps: Optional[int] = None, lengths=None, cache_rows: bool = True,
                  cache_fp8: bool = False, weights_fp8: bool = False) -> Workload:
    """Build workload ``wid`` (1..5).  Keyword overrides shrink or reshape it
    for tests; the seed stays 1000 + wid unless given.  ``lengths`` (decode
    workloads) fixes every sequence's cache length after the append (and the
    batch).  ``cache_fp8`` (decode workloads) gives the cached rows in the
    FP8 cache layout (``cache_fp8_rows``, fp8_cache_rows) instead of bf16.
    ``weights_fp8`` adds the FP8 projections (``weights_fp8``,
    fp8_weight_blocks) from a stream of their own,
    ``PCG64(1000 + workload_id + 4481)``, so every other draw is unchanged."""
    spec = dict(WORKLOADS[wid])
    d = dims or spec["dims"]
    dt = dtype or spec["dtype"]
    bf16 = dt == "bf16"
    kind = spec["kind"]
    rng = np.random.Generator(np.random.PCG64(1000 + wid if seed is None else seed))
    B = batch if batch is not None else spec["batch"]
    if lengths is not None:
        B = len(lengths)
    wl = Workload(wid=wid, name=spec["name"], dims=d, dtype=dt, kind=kind, batch=B)
    wl.weights_f32, wl.weights_bits = draw_weights(rng, d, bf16)
    if weights_fp8:
        frng = np.random.Generator(np.random.PCG64((1000 + wid if seed is None else seed) + 4481))
        shp = weight_shapes(d)
        wl.weights_fp8 = {n: fp8_weight_blocks(frng, shp[n], 1.0 / np.sqrt(shp[n][1])) for n in FP8_WEIGHT_NAMES}

    if kind == "prefill":
        L = seq_len if seq_len is not None else spec["seq_len"]
        wl.seq_len = L
        wl.h_f32, wl.h_bits = _normal(rng, (B, L, d.d_model), 1.0, bf16)
        return wl

    if kind == "prefill+decode":
        L = seq_len if seq_len is not None else spec["seq_len"]
        ns = n_steps if n_steps is not None else spec["n_steps"]
        wl.seq_len, wl.n_steps, wl.n_q = L, ns, 1
        wl.h_f32, wl.h_bits = _normal(rng, (B, L + ns, d.d_model), 1.0, bf16)
        wl.paged = bool(paged) if paged is not None else False
        wl.block_size = block_size or 64
        return wl

    # decode
    nq = n_q if n_q is not None else spec["n_q"]
    wl.n_q = nq
    wl.h_f32, wl.h_bits = _normal(rng, (B, nq, d.d_model), 1.0, bf16)
    rmax = ragged_max if ragged_max is not None else spec.get("ragged_max")
    ulen = uniform_len if uniform_len is not None else spec.get("uniform_len")
    if lengths is not None:
        lens = np.maximum(np.asarray(lengths, dtype=np.int64), nq)
    elif rmax is not None and uniform_len is None:
        # integers, both ends inclusive; at least n_q so the new tokens fit
        lens = rng.integers(low=1, high=rmax, size=B, endpoint=True).astype(np.int64)
        lens = np.maximum(lens, nq)
    else:
        lens = np.full(B, ulen, dtype=np.int64)
    wl.lens = lens.astype(np.int32)
    wl.cache_fp8 = cache_fp8
    if cache_rows and cache_fp8:
        wl.cache_fp8_rows = [fp8_cache_rows(rng, int(lens[b]) - nq, d.d_c, d.d_rope) for b in range(B)]
    elif cache_rows:
        cf, cb = [], []
        for b in range(B):
            v, bb = _normal(rng, (int(lens[b]) - nq, d.d_row), 1.0, bf16)
            cf.append(v)
            cb.append(bb)
        wl.cache_f32, wl.cache_bits = cf, cb
    wl.paged = bool(spec.get("paged", False)) if paged is None else bool(paged)
    wl.block_size = block_size or spec.get("block_size", 64)
    if wl.paged:
        nblk = int(sum((int(l) + wl.block_size - 1) // wl.block_size for l in lens))
        prng = np.random.Generator(np.random.PCG64((1000 + wid if seed is None else seed) + 7919))
        wl.block_perm = prng.permutation(nblk).astype(np.int32)
    return wl


# ----------------------------------------------------------------------------
# Paged layout helpers (pure index bookkeeping)
# ----------------------------------------------------------------------------

def block_table_rows(lens: np.ndarray, block_size: int, perm: np.ndarray, max_blocks: int) -> np.ndarray:
    """Block table [B][max_blocks] int32: logical block k of sequence b is
    physical block perm[offset_b + k]; unused entries are -1."""
    B = len(lens)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        nb = (int(lens[b]) + block_size - 1) // block_size
        table[b, :nb] = perm[off:off + nb]
        off += nb
    return table


def scatter_paged(rows_per_seq: List[np.ndarray], lens: np.ndarray, block_size: int,
                  table: np.ndarray, n_blocks: int, d_row: int, dtype) -> np.ndarray:
    """Place each sequence's rows into a pool [n_blocks*block_size][d_row]
    following ``table``.  Rows past the given ones are left zero."""
    pool = np.zeros((n_blocks * block_size, d_row), dtype=dtype)
    for b, rows in enumerate(rows_per_seq):
        n = rows.shape[0]
        pos = np.arange(n)
        phys = table[b, pos // block_size].astype(np.int64) * block_size + pos % block_size
        pool[phys] = rows
    return pool
