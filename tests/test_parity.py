"""GPU parity: libmla (through the C ABI) against the CPU oracle on the same
seeded inputs, element by element.  fp32: max-abs <= 1e-4; bf16: relative
Frobenius <= 2e-2 and max-abs <= 5e-2."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_inputs import Dims, DSV3, TINY, make_workload
from oracle import mla_oracle as O

from tests.gpu_harness import (CacheBuf, Timer, assert_close, decode_cache, layer_for, oracle_decode_seq,
                               run_decode, say, upload, weights64)

pytestmark = pytest.mark.gpu


def _prefill_check(wl, layer, paged=False, rows=None, want_o=False):
    """Run mla_prefill on wl (kind prefill) and compare u, o and the cache rows."""
    d, bf16 = wl.dims, wl.bf16
    B, L = wl.batch, wl.seq_len
    h = upload(wl.h_f32, wl.h_bits, bf16)
    if paged:
        bs = 64
        nb = (L + bs - 1) // bs
        perm = np.random.Generator(np.random.PCG64(5)).permutation(B * nb).astype(np.int32)
        table = perm.reshape(B, nb)
        pool = torch.zeros(B * nb * bs, d.d_row, dtype=layer.tdtype, device="cuda")
        cache = CacheBuf.paged(pool, bs, table)
    else:
        cache = layer.new_cache(B, L)
    say(f"prefill {wl.name} B={B} L={L} paged={paged}")
    u, o = layer.prefill(h, cache, want_o=True)
    torch.cuda.synchronize()
    W = weights64(wl)
    for b in range(B):
        with Timer(f"oracle prefill b={b}"):
            ref = O.prefill(d, W, wl.h_f32[b].astype(np.float64), rows=rows)
        sel = np.arange(L) if rows is None else np.asarray(rows)
        if ref["u"] is not None:
            assert_close(u[b, torch.from_numpy(sel).cuda()], ref["u"], bf16, f"u b={b}")
        assert_close(o.view(B, L, d.n_heads, d.d_v)[b, torch.from_numpy(sel).cuda()], ref["o"], bf16, f"o b={b}")
        got_rows = cache.read_rows(b, np.arange(L))
        ref_rows = np.concatenate([ref["c_kv"], ref["k_r"]], axis=1)
        assert_close(got_rows, ref_rows, bf16, f"cache rows b={b}")
    return u, o, cache


def test_tiny_fp32_prefill_then_decode():
    """Workload 1: 64-token prefill, then 8 single-token decode steps, fp32."""
    wl = make_workload(1)
    d = wl.dims
    layer = layer_for(wl)
    W = weights64(wl)
    h_all = wl.h_f32[0].astype(np.float64)
    full = O.prefill(d, W, h_all)
    for paged in (False, True):
        L, steps = wl.seq_len, wl.n_steps
        total = L + steps
        if paged:
            bs = 16
            nb = (total + bs - 1) // bs
            table = np.random.Generator(np.random.PCG64(3)).permutation(nb).astype(np.int32).reshape(1, nb)
            pool = torch.zeros(nb * bs, d.d_row, dtype=torch.float32, device="cuda")
            cache = CacheBuf.paged(pool, bs, table)
        else:
            cache = layer.new_cache(1, total)
        say(f"tiny prefill paged={paged}")
        h = torch.from_numpy(wl.h_f32[:, :L]).cuda()
        u = layer.prefill(h, cache)
        torch.cuda.synchronize()
        assert_close(u[0], full["u"][:L], False, "tiny prefill u")
        ref_rows = np.concatenate([full["c_kv"], full["k_r"]], axis=1)
        assert_close(cache.read_rows(0, np.arange(L)), ref_rows[:L], False, "tiny prefill cache rows")
        for s in range(steps):
            t = L + s
            say(f"tiny decode step {s} paged={paged}")
            hs = torch.from_numpy(wl.h_f32[:, t:t + 1]).cuda()
            lens = torch.tensor([t + 1], dtype=torch.int32, device="cuda")
            u1 = layer.decode(hs, lens, total, cache)
            torch.cuda.synchronize()
            assert_close(u1[0, 0], full["u"][t], False, f"tiny decode u step {s}")
        assert_close(cache.read_rows(0, np.arange(total)), ref_rows, False, "tiny cache after decode")


@pytest.mark.parametrize("B,L", [(1, 64), (2, 200), (1, 1), (3, 37), (2, 8), (1, 520), (1, 261), (1, 200), (1, 150), (1, 240)])
def test_dsv3_prefill_small(B, L):
    """DeepSeek-V3 shapes, bf16, small sequences with ragged tiles."""
    wl = make_workload(3, batch=B, seq_len=L)
    layer = layer_for(wl)
    _prefill_check(wl, layer)


@pytest.mark.parametrize("B,L,tb", [(1, 520, 100), (2, 264, 70)])
def test_dsv3_prefill_large_logit_spread(B, L, tb):
    """The hidden state of one token (tb, in the last sequence) scaled by 16:
    for later queries its key scores far above the first keys (by more than
    the flash kernel's fixed-reference range in many heads), so their
    workgroups run the second pass (reference = each row's maximum); they
    match the oracle like every other row.  The scaled token's own query row is left
    out: scaled twice (query and key), its scores reach magnitudes where
    rounding q and k to bf16 already moves the softmax weights by more than
    the bf16 bounds, whatever the attention kernel does."""
    from mla_inputs import bf16_bits_to_f32, bf16_round
    wl = make_workload(3, batch=B, seq_len=L)
    sb = B - 1   # the scaled token sits in the last sequence
    big = bf16_round(wl.h_f32[sb][tb] * 16.0)
    wl.h_bits[sb][tb] = big
    wl.h_f32[sb][tb] = bf16_bits_to_f32(big)
    layer = layer_for(wl)
    d = wl.dims
    h = upload(wl.h_f32, wl.h_bits, True)
    say(f"prefill with large logit spread B={B} L={L} token {tb} of sequence {sb}")
    u, o = layer.prefill(h, layer.new_cache(B, L), want_o=True)
    torch.cuda.synchronize()
    from tests.gpu_harness import BF16_MAX_ABS, BF16_REL_FROB, err
    for b in range(B):
        keep = np.setdiff1d(np.arange(L), [tb]) if b == sb else np.arange(L)
        with Timer(f"oracle prefill b={b}"):
            ref = O.prefill(d, weights64(wl), wl.h_f32[b].astype(np.float64), rows=keep)
        sel = torch.from_numpy(keep).cuda()
        for what, got, r in (("u", u[b, sel], ref["u"]), ("o", o.view(B, L, d.n_heads, d.d_v)[b, sel], ref["o"])):
            # the scaled key raises the outputs' magnitude, so the max-abs
            # bound is taken relative to max(1, max|oracle|)
            e = err(got, r)
            mag = max(1.0, float(np.max(np.abs(r))))
            say(f"{what} b={b}: max_abs={e.max_abs:.3e} (max|ref|={mag:.1f}) rel_frob={e.rel_frob:.3e}")
            assert e.rel_frob <= BF16_REL_FROB and e.max_abs <= BF16_MAX_ABS * mag, (what, b, e)


def test_dsv3_prefill_paged():
    wl = make_workload(3, batch=2, seq_len=130)
    layer = layer_for(wl)
    _prefill_check(wl, layer, paged=True)


@pytest.mark.parametrize("B,L,nq", [(4, 300, 1), (2, 33, 1), (3, 1, 1), (2, 500, 2), (2, 2, 2), (1, 97, 3),
                                     (20, 50, 1), (11, 40, 3), (4, 260, 4), (2, 900, 8)])
def test_dsv3_decode_small(B, L, nq):
    """DeepSeek-V3 shapes, bf16 decode against a contiguous latent cache.  20
    tokens leave the second 16-token block of the one-launch query path and of
    the combine partly empty; 33 tokens take the separate up-projection and
    absorption GEMMs; 4 and 8 query tokens per sequence are multi-token
    verification steps (causal among the new tokens)."""
    wl = make_workload(2, batch=B, uniform_len=L, n_q=nq)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"decode B={B} L={L} n_q={nq}")
    u, o = run_decode(wl, layer, cache)
    d = wl.dims
    for b in range(B):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b}")
        assert_close(o.view(B, nq, d.n_heads, d.d_v)[b], ref["o"], True, f"o b={b}")
        got_new = cache.read_rows(b, np.arange(L - nq, L))
        assert_close(got_new, ref["row_new"], True, f"new cache rows b={b}")


@pytest.mark.parametrize("B,L,nq", [(100, 300, 2), (96, 200, 1)])
def test_dsv3_decode_96_to_255_tokens(B, L, nq):
    """200 and 96 new tokens in one decode call: W_O runs on the 256x256-tile
    kernel split eight ways over k (one tile row, its rows past the token
    count clamped and not stored) and the ordered reduce; the other products
    keep their kernels.  Sequences at both ends and one inside against the
    oracle."""
    wl = make_workload(2, batch=B, uniform_len=L, n_q=nq)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"decode B={B} L={L} n_q={nq} ({B * nq} tokens)")
    u, o = run_decode(wl, layer, cache)
    d = wl.dims
    for b in (0, B // 2 + 7, B - 1):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b}")
        assert_close(o.view(B, nq, d.n_heads, d.d_v)[b], ref["o"], True, f"o b={b}")
        got_new = cache.read_rows(b, np.arange(L - nq, L))
        assert_close(got_new, ref["row_new"], True, f"new cache rows b={b}")


# DeepSeek-V3 latent and head widths with 20 heads and a narrower model:
# head counts off the multiples of 8 that the workgroup-to-XCD maps assume,
# fewer query rows (20) than a 64-row decode workgroup, a W_O input width
# (2560) below the streaming GEMM's range, and the flash kernel's mapping for
# head counts not divisible by 8.
ODD_HEADS = Dims(d_model=1024, n_heads=20, d_nope=128, d_rope=64, d_v=128, d_c=512, d_cq=1536)


@pytest.mark.parametrize("B,L,nq", [(5, 150, 1), (3, 90, 2)])
def test_dsv3_widths_odd_head_count_decode(B, L, nq):
    wl = make_workload(2, dims=ODD_HEADS, batch=B, uniform_len=L, n_q=nq)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"decode 20 heads B={B} L={L} n_q={nq}")
    u, o = run_decode(wl, layer, cache)
    d = wl.dims
    for b in range(B):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b}")
        assert_close(o.view(B, nq, d.n_heads, d.d_v)[b], ref["o"], True, f"o b={b}")


def test_dsv3_widths_odd_head_count_prefill():
    wl = make_workload(3, dims=ODD_HEADS, batch=2, seq_len=100)
    layer = layer_for(wl)
    _prefill_check(wl, layer)


@pytest.mark.parametrize("block_size", [64, 32, 16, 96])
def test_dsv3_decode_ragged_paged_small(block_size):
    """Ragged lengths, paged blocks in a permuted order (block sizes that are
    and are not multiples of the 32-row cache tile)."""
    wl = make_workload(4, batch=6, ragged_max=700, block_size=block_size)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"ragged paged decode lens={wl.lens.tolist()}")
    u, o = run_decode(wl, layer, cache)
    for b in range(wl.batch):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b} len={wl.lens[b]}")


def test_dsv3_decode_large_logit_spread():
    """Cached rows scaled by 64 late in a split: their scores exceed the
    split's first-tile reference by far more than 2^32, so those workgroups
    run their second pass (reference = each row's maximum); all rows still
    match the oracle."""
    from mla_inputs import bf16_bits_to_f32, bf16_round
    wl = make_workload(2, batch=32, uniform_len=300)
    for b, pos, src in ((0, 40, 3), (5, 100, 7), (9, 250, 2)):
        big = bf16_round(bf16_bits_to_f32(wl.cache_bits[b][src]) * 64.0)
        wl.cache_bits[b][pos] = big
        wl.cache_f32[b][pos] = bf16_bits_to_f32(big)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say("decode with large logit spread B=32 L=300")
    u, o = run_decode(wl, layer, cache)
    d = wl.dims
    from tests.gpu_harness import BF16_MAX_ABS, BF16_REL_FROB, err
    for b in (0, 5, 9, 1):
        ref = oracle_decode_seq(wl, b)
        for what, got, r in (("u", u[b], ref["u"]), ("o", o.view(wl.batch, 1, d.n_heads, d.d_v)[b], ref["o"])):
            # the scaled rows raise the outputs' magnitude, so the max-abs
            # bound is taken relative to max(1, max|oracle|)
            e = err(got, r)
            mag = max(1.0, float(np.max(np.abs(r))))
            say(f"{what} b={b}: max_abs={e.max_abs:.3e} (max|ref|={mag:.1f}) rel_frob={e.rel_frob:.3e}")
            assert e.rel_frob <= BF16_REL_FROB and e.max_abs <= BF16_MAX_ABS * mag, (what, b, e)


# YaRN long-context RoPE (highlight 13 of the V3 highlights page: s = 40,
# beta_slow = 1, beta_fast = 32 over the 4K original context).  The library
# forms the blended frequencies and the softmax temperature on the host; the
# kernels are the plain-RoPE ones.
YARN_DS = dataclasses.replace(DSV3, yarn_factor=40.0)
YARN_TINY = dataclasses.replace(TINY, yarn_factor=40.0, yarn_orig_len=32)


def test_yarn_tiny_fp32_prefill():
    """fp32, 64 positions over a 32-token original context (every regime of
    the blend occurs among the 8 pairs)."""
    wl = make_workload(1, dims=YARN_TINY)
    layer = layer_for(wl)
    W = weights64(wl)
    h = wl.h_f32[0, :wl.seq_len].astype(np.float64)
    plain = O.prefill(TINY, W, h)["u"]
    assert not np.allclose(O.prefill(YARN_TINY, W, h)["u"], plain, rtol=1e-3, atol=1e-3)
    wl.h_f32, wl.h_bits = wl.h_f32[:, :wl.seq_len], (None if wl.h_bits is None else wl.h_bits[:, :wl.seq_len])
    _prefill_check(wl, layer)


def test_yarn_dsv3_prefill_small():
    wl = make_workload(3, dims=YARN_DS, batch=1, seq_len=300)
    layer = layer_for(wl)
    _prefill_check(wl, layer)


def test_yarn_dsv3_decode_ragged_paged():
    """YaRN with ragged lengths over a paged cache in a permuted block order."""
    wl = make_workload(4, dims=YARN_DS, batch=5, ragged_max=5000, block_size=64)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"yarn ragged paged decode lens={wl.lens.tolist()}")
    u, o = run_decode(wl, layer, cache)
    for b in range(wl.batch):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b} len={wl.lens[b]}")
        L = int(wl.lens[b])
        assert_close(cache.read_rows(b, np.arange(L - 1, L)), ref["row_new"], True, f"new row b={b}")


@pytest.mark.parametrize("B,L,nq", [(1, 4600, 2), (3, 700, 1)])
def test_yarn_dsv3_decode(B, L, nq):
    """Decode with positions past the 4K original context (the new tokens'
    RoPE key and query rotate at the blended frequencies)."""
    wl = make_workload(2, dims=YARN_DS, batch=B, uniform_len=L, n_q=nq)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"yarn decode B={B} L={L} n_q={nq}")
    u, o = run_decode(wl, layer, cache)
    d = wl.dims
    for b in range(B):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b}")
        assert_close(o.view(B, nq, d.n_heads, d.d_v)[b], ref["o"], True, f"o b={b}")
        got_new = cache.read_rows(b, np.arange(L - nq, L))
        assert_close(got_new, ref["row_new"], True, f"new cache rows b={b}")


def _mixed_lengths(n_long, long_len, n_short, short_max, seed):
    """n_long sequences of long_len rows and n_short of 1..short_max rows, in
    a seeded random order."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = [long_len] * n_long + [int(x) for x in rng.integers(1, short_max, n_short, endpoint=True)]
    return [lens[i] for i in rng.permutation(len(lens))]


@pytest.mark.parametrize("n_long,long_len,n_short,short_max,paged", [
    (8, 4000, 56, 40, True),     # 128-row workgroups, paged
    (4, 3000, 16, 50, False),    # 64-row workgroups (at most 32 sequences), contiguous
])
def test_dsv3_decode_mixed_lengths(n_long, long_len, n_short, short_max, paged):
    """The split plan deals the batch's cached tiles out evenly, so one
    workgroup's share can hold the end of a long sequence, several whole
    short ones and the start of the next: every sequence still matches the
    oracle (all short ones, and three long ones)."""
    lens = _mixed_lengths(n_long, long_len, n_short, short_max, seed=17)
    wl = make_workload(4 if paged else 2, lengths=lens, paged=paged)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"mixed-length decode B={wl.batch} paged={paged} lens={wl.lens.tolist()}")
    u, o = run_decode(wl, layer, cache)
    longs = [b for b in range(wl.batch) if wl.lens[b] == long_len][:3]
    for b in range(wl.batch):
        if wl.lens[b] == long_len and b not in longs:
            continue
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b} len={wl.lens[b]}")


def test_decode_stale_nan_workspace():
    """Workspace bytes left by earlier calls never reach the result: every
    workspace byte is set to 0xFF (NaN in bf16 and fp32) before a decode of
    short and long sequences, whose outputs still match the oracle."""
    from head_latent_attention_18_amd import libmla as LM
    lens = _mixed_lengths(2, 3000, 10, 60, seed=4)
    wl = make_workload(2, lengths=lens)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    ml = int(wl.lens.max())
    nbytes = LM.mla_workspace_size(layer.cfg, LM.MLA_OP_DECODE, wl.batch, wl.n_q, ml)
    layer.workspace("decode", nbytes, torch.device("cuda")).fill_(255)
    torch.cuda.synchronize()
    say(f"decode over a NaN-filled workspace lens={wl.lens.tolist()}")
    u, o = run_decode(wl, layer, cache, max_len=ml)
    for b in range(wl.batch):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b} len={wl.lens[b]}")
