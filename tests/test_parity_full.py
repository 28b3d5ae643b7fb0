"""GPU parity at the full DeepSeek-V3 workload sizes, in the launch
configuration bench.py times, on outputs the oracle can compute one by one:
whole sequences (decode), sampled rows (prefill) and sampled heads (128K
decode).  Same tolerances as test_parity (bf16: relative Frobenius <= 2e-2,
max-abs <= 5e-2)."""
import dataclasses

import numpy as np
import pytest
import torch

from mla_inputs import DSV3, make_workload
from oracle import mla_oracle as O

from tests.gpu_harness import Timer, assert_close, decode_cache, layer_for, run_decode, say, upload, weights64

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def _decode_seq_check(wl, u, o, cache, seqs, heads=None):
    d = wl.dims
    W = weights64(wl)
    B, nq = wl.batch, wl.n_q
    for b in seqs:
        with Timer(f"oracle decode b={b} len={wl.lens[b]} heads={'all' if heads is None else heads}"):
            ref = O.decode(d, W, wl.h_f32[b].astype(np.float64), wl.cache_f32[b].astype(np.float64), heads=heads)
        ob = o.view(B, nq, d.n_heads, d.d_v)[b]
        if heads is None:
            assert_close(u[b], ref["u"], True, f"u b={b}")
            assert_close(ob, ref["o"], True, f"o b={b}")
        else:
            hsel = torch.tensor(heads, device=ob.device)
            assert_close(ob.index_select(1, hsel), ref["o"][:, heads], True, f"o b={b} heads={heads}")
        L = int(wl.lens[b])
        assert_close(cache.read_rows(b, np.arange(L - nq, L)), ref["row_new"], True, f"new rows b={b}")


def test_full_decode_b32_len4096():
    """DeepSeek-V3 decode, batch 32, cache length 4096 (the benchmarked step)."""
    wl = make_workload(2)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say("full decode b32 len4096")
    u, o = run_decode(wl, layer, cache)
    _decode_seq_check(wl, u, o, cache, seqs=[0, 13, 31])


def test_full_prefill_len4096_sampled_rows():
    """DeepSeek-V3 causal prefill of 4096 tokens; rows at tile edges, the ends
    and random positions; every cache row."""
    wl = make_workload(3)
    d = wl.dims
    layer = layer_for(wl)
    L = wl.seq_len
    h = upload(wl.h_f32, wl.h_bits, True)
    cache = layer.new_cache(1, L)
    say("full prefill len4096")
    u, o = layer.prefill(h, cache, want_o=True)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(77))
    rows = sorted(set([0, 1, 2, 15, 16, 63, 64, 65, 127, 128, 255, 256, 257, 511, 1023, 2047, 2048, 4094, 4095]
                      + rng.integers(0, L, 13).tolist()))
    with Timer("oracle prefill (sampled rows)"):
        ref = O.prefill(d, weights64(wl), wl.h_f32[0].astype(np.float64), rows=rows)
    sel = torch.tensor(rows, device="cuda")
    assert_close(u[0].index_select(0, sel), ref["u"], True, "u sampled rows")
    assert_close(o.view(L, d.n_heads, d.d_v).index_select(0, sel), ref["o"], True, "o sampled rows")
    assert_close(cache.read_rows(0, np.arange(L)), np.concatenate([ref["c_kv"], ref["k_r"]], axis=1), True,
                 "all cache rows")


@pytest.mark.parametrize("fp8w", [False, True])
def test_prefill_len4000_sampled_rows(fp8w):
    """4000 tokens, bf16 and FP8 projections: every 256x256-tile product has
    a partial last row of tiles (3840..3999) and the flash kernel a partial
    last query block; rows of the first and last row tiles and random ones."""
    wl = make_workload(3, seq_len=4000, weights_fp8=fp8w)
    d = wl.dims
    layer = layer_for(wl)
    L = wl.seq_len
    h = upload(wl.h_f32, wl.h_bits, True)
    cache = layer.new_cache(1, L)
    say(f"prefill len4000 fp8w={fp8w}")
    u = layer.prefill(h, cache)
    torch.cuda.synchronize()
    rng = np.random.Generator(np.random.PCG64(78))
    rows = sorted(set([0, 255, 256, 3839, 3840, 3841, 3998, 3999] + rng.integers(0, L, 8).tolist()))
    with Timer("oracle prefill (sampled rows)"):
        ref = O.prefill(d, weights64(wl), wl.h_f32[0].astype(np.float64), rows=rows, weights_fp8=fp8w)
    sel = torch.tensor(rows, device="cuda")
    assert_close(u[0].index_select(0, sel), ref["u"], True, "u sampled rows")


def test_full_decode_ragged_paged_b128():
    """128 sequences, lengths uniform in [1, 32768], paged 64-row blocks in a
    permuted order: the shortest, the longest and random sequences in full."""
    with Timer("draw ragged workload"):
        wl = make_workload(4)
    layer = layer_for(wl)
    with Timer("build paged cache"):
        cache = decode_cache(wl, layer)
    say(f"ragged paged decode sum(len)={int(wl.lens.sum())} max={int(wl.lens.max())}")
    u, o = run_decode(wl, layer, cache)
    order = np.argsort(wl.lens)
    rng = np.random.Generator(np.random.PCG64(78))
    seqs = sorted(set([int(order[0]), int(order[1]), int(order[-1])] + rng.integers(0, wl.batch, 3).tolist()))
    _decode_seq_check(wl, u, o, cache, seqs=seqs)


@pytest.mark.parametrize("yarn", [False, True], ids=["rope", "yarn40"])
def test_full_decode_len131072_nq2(yarn):
    """Four sequences of 128K, two new tokens each (causal between them): one
    sequence in full, sampled heads of the others.  The YaRN case is the
    configuration the V3 highlights page runs at 128K (highlight 13: s = 40,
    beta_slow = 1, beta_fast = 32 over the 4K original context)."""
    with Timer("draw 128K workload"):
        wl = make_workload(5, dims=dataclasses.replace(DSV3, yarn_factor=40.0) if yarn else None)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say("128K decode n_q=2")
    u, o = run_decode(wl, layer, cache)
    _decode_seq_check(wl, u, o, cache, seqs=[3])
    _decode_seq_check(wl, u, o, cache, seqs=[0, 1, 2], heads=[0, 57, 127])


def _fp8_full(wid, seqs, heads_seqs=(), heads=None):
    with Timer(f"draw workload {wid} (FP8 cache)"):
        wl = make_workload(wid, cache_fp8=True)
    layer = layer_for(wl)
    with Timer("build cache"):
        cache = decode_cache(wl, layer)
    say(f"fp8 full decode workload {wid}")
    u, o = run_decode(wl, layer, cache)
    d = wl.dims
    B, nq = wl.batch, wl.n_q
    for b in list(seqs) + list(heads_seqs):
        hs = heads if b in heads_seqs else None
        with Timer(f"oracle fp8 decode b={b} len={wl.lens[b]}"):
            ref = O.decode(d, weights64(wl), wl.h_f32[b].astype(np.float64),
                           O.dequantize_fp8_rows(wl.cache_fp8_rows[b], d), heads=hs, cache_fp8=True)
        ob = o.view(B, nq, d.n_heads, d.d_v)[b]
        if hs is None:
            assert_close(u[b], ref["u"], True, f"fp8 u b={b}")
            assert_close(ob, ref["o"], True, f"fp8 o b={b}")
        else:
            hsel = torch.tensor(hs, device=ob.device)
            assert_close(ob.index_select(1, hsel), ref["o"][:, hs], True, f"fp8 o b={b} heads={hs}")


def test_full_fp8_decode_b32_len4096():
    _fp8_full(2, seqs=[0, 31])


def test_full_fp8_decode_ragged_paged_b128():
    wl_lens = make_workload(4, cache_rows=False).lens
    order = np.argsort(wl_lens)
    _fp8_full(4, seqs=sorted({int(order[0]), int(order[-1]), 64}))


def test_full_fp8_decode_len131072_nq2():
    _fp8_full(5, seqs=[1], heads_seqs=[0, 3], heads=[0, 127])
