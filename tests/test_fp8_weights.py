"""GPU parity of the block-scaled FP8 projections: W_DQ, W_DKV, W_KR and W_O
as E4M3 codes with a power-of-two scale per 128x128 block, h and the
attention output quantised per token and 128 columns, scaled FP8 MFMAs.
Decode goes through the weight-streaming kernel (every token-count variant
up to 128) and, beyond 128 tokens, the 256x256 tiles; prefill through both.
The oracle applies the same reading; both sides quantise from bf16 values,
so a code can differ only where the two sides' bf16 values differ.  Bounds
as for bf16 (relative Frobenius <= 2e-2, max-abs <= 5e-2)."""
import numpy as np
import pytest
import torch

from mla_inputs import make_workload
from oracle import mla_oracle as O

from tests.gpu_harness import (Timer, assert_close, assert_fp8_rows, decode_cache, layer_for, oracle_decode_seq,
                               run_decode, say, upload, weights64)

pytestmark = pytest.mark.gpu


# B * n_q tokens: 4 and 6 (16-row blocks), 20 (32), 64 (64), 128 (128 rows),
# 132 (the 256x256 tiles with a partial tile), 600 (a 300-token chunk per
# sequence: the up-projected form)
@pytest.mark.parametrize("B,L,nq", [(4, 300, 1), (3, 97, 2), (20, 50, 1), (64, 40, 1), (128, 20, 1), (33, 70, 4),
                                    (2, 700, 300)])
def test_fp8w_decode(B, L, nq):
    wl = make_workload(2, batch=B, uniform_len=L, n_q=nq, weights_fp8=True)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"fp8-weight decode B={B} L={L} n_q={nq}")
    u, o = run_decode(wl, layer, cache)
    d = wl.dims
    for b in sorted({0, B // 2, B - 1}):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b}")
        assert_close(o.view(B, nq, d.n_heads, d.d_v)[b], ref["o"], True, f"o b={b}")
        assert_close(cache.read_rows(b, np.arange(L - nq, L)), ref["row_new"], True, f"new rows b={b}")


def test_fp8w_decode_ragged_paged_fp8_cache():
    """FP8 projections and the FP8 latent cache together, ragged and paged."""
    wl = make_workload(4, batch=5, ragged_max=700, cache_fp8=True, weights_fp8=True)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"fp8-weight fp8-cache ragged decode lens={wl.lens.tolist()}")
    u, _ = run_decode(wl, layer, cache)
    for b in range(wl.batch):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b} len={wl.lens[b]}")
        L = int(wl.lens[b])
        assert_fp8_rows(cache.read_rows(b, np.arange(L - 1, L)), ref["row_new"], wl.dims, f"new row b={b}")


# 64 and 100 tokens stream the weights; 300 and 2 x 200 take the 256x256
# tiles (a partial tile each)
@pytest.mark.parametrize("B,L", [(1, 64), (1, 100), (1, 300), (2, 200)])
def test_fp8w_prefill(B, L):
    wl = make_workload(3, batch=B, seq_len=L, weights_fp8=True)
    d = wl.dims
    layer = layer_for(wl)
    h = upload(wl.h_f32, wl.h_bits, True)
    cache = layer.new_cache(B, L)
    say(f"fp8-weight prefill B={B} L={L}")
    u, o = layer.prefill(h, cache, want_o=True)
    torch.cuda.synchronize()
    W = weights64(wl)
    for b in range(B):
        with Timer(f"oracle prefill b={b}"):
            ref = O.prefill(d, W, wl.h_f32[b].astype(np.float64), weights_fp8=True)
        assert_close(u[b], ref["u"], True, f"u b={b}")
        assert_close(o.view(B, L, d.n_heads, d.d_v)[b], ref["o"], True, f"o b={b}")
        assert_close(cache.read_rows(b, np.arange(L)), np.concatenate([ref["c_kv"], ref["k_r"]], axis=1), True,
                     f"cache rows b={b}")


def test_fp8w_prefill_then_decode():
    """Prefill of 200 tokens, then two decode steps on the rows it wrote."""
    L0, steps = 200, 2
    wl = make_workload(3, batch=1, seq_len=L0 + steps, weights_fp8=True)
    d = wl.dims
    layer = layer_for(wl)
    W = weights64(wl)
    h = upload(wl.h_f32, wl.h_bits, True)
    cache = layer.new_cache(1, L0 + steps)
    layer.prefill(h[:, :L0].contiguous(), cache)
    torch.cuda.synchronize()
    with Timer("oracle prefill"):
        full = O.prefill(d, W, wl.h_f32[0].astype(np.float64), weights_fp8=True)
    rows = np.concatenate([full["c_kv"], full["k_r"]], axis=1)
    for s in range(steps):
        t = L0 + s
        lens = torch.tensor([t + 1], dtype=torch.int32, device="cuda")
        u1 = layer.decode(h[:, t:t + 1].contiguous(), lens, L0 + steps, cache)
        torch.cuda.synchronize()
        assert_close(u1[0], full["u"][t:t + 1], True, f"decode step {s} u")


@pytest.mark.slow
def test_fp8w_full_decode_b32_len4096():
    """The benchmarked decode step (batch 32, cache 4096) with FP8
    projections: whole sequences."""
    wl = make_workload(2, weights_fp8=True)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say("fp8-weight full decode b32 len4096")
    u, o = run_decode(wl, layer, cache)
    for b in (0, 31):
        with Timer(f"oracle decode b={b}"):
            ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b}")


@pytest.mark.slow
def test_fp8w_full_prefill_len4096_sampled_rows():
    """The benchmarked prefill (4096 tokens) with FP8 projections: sampled
    rows and every cache row."""
    wl = make_workload(3, weights_fp8=True)
    d = wl.dims
    layer = layer_for(wl)
    L = wl.seq_len
    h = upload(wl.h_f32, wl.h_bits, True)
    cache = layer.new_cache(1, L)
    say("fp8-weight full prefill len4096")
    u = layer.prefill(h, cache)
    torch.cuda.synchronize()
    rows = [0, 1, 255, 256, 257, 2047, 4095, 1234, 3333]
    with Timer("oracle prefill (sampled rows)"):
        ref = O.prefill(d, weights64(wl), wl.h_f32[0].astype(np.float64), rows=rows, weights_fp8=True)
    sel = torch.tensor(rows, device="cuda")
    assert_close(u[0].index_select(0, sel), ref["u"], True, "u sampled rows")
    assert_close(cache.read_rows(0, np.arange(L)), np.concatenate([ref["c_kv"], ref["k_r"]], axis=1), True,
                 "all cache rows")
