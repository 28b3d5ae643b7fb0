"""GPU parity of the FP8 latent cache (E4M3 codes with a float32 scale per
128 columns of c_KV, k_R in bf16): decode reading FP8 rows and appending its
own, prefill writing FP8 rows, and decode after prefill, against the oracle
(which dequantises the same stored rows, and quantises the new rows itself).
Outputs: bf16 bounds (relative Frobenius <= 2e-2, max-abs <= 5e-2); rows
written by the GPU: within the quantisation bound of the oracle's rows."""
import numpy as np
import pytest
import torch

from mla_inputs import make_workload
from oracle import mla_oracle as O

from tests.gpu_harness import (Timer, assert_close, assert_fp8_rows, decode_cache, layer_for, oracle_decode_seq,
                               run_decode, say, upload, weights64)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B,L,nq", [(4, 300, 1), (3, 97, 2), (2, 900, 8), (20, 50, 1), (33, 70, 1)])
def test_fp8_decode_small(B, L, nq):
    wl = make_workload(2, batch=B, uniform_len=L, n_q=nq, cache_fp8=True)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"fp8 decode B={B} L={L} n_q={nq}")
    u, o = run_decode(wl, layer, cache)
    d = wl.dims
    for b in range(B):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b}")
        assert_close(o.view(B, nq, d.n_heads, d.d_v)[b], ref["o"], True, f"o b={b}")
        assert_fp8_rows(cache.read_rows(b, np.arange(L - nq, L)), ref["row_new"], d, f"new rows b={b}")


@pytest.mark.parametrize("block_size", [64, 32])
def test_fp8_decode_ragged_paged(block_size):
    wl = make_workload(4, batch=6, ragged_max=700, block_size=block_size, cache_fp8=True)
    layer = layer_for(wl)
    cache = decode_cache(wl, layer)
    say(f"fp8 ragged paged decode lens={wl.lens.tolist()} block={block_size}")
    u, o = run_decode(wl, layer, cache)
    for b in range(wl.batch):
        ref = oracle_decode_seq(wl, b)
        assert_close(u[b], ref["u"], True, f"u b={b} len={wl.lens[b]}")


def test_fp8_decode_mixed_lengths_deterministic():
    """Short and long sequences packed into workgroups' shares; two runs are
    bitwise equal."""
    rng = np.random.Generator(np.random.PCG64(19))
    lens = [3000] * 3 + [int(x) for x in rng.integers(1, 60, 20)]
    lens = [lens[i] for i in rng.permutation(len(lens))]
    wl = make_workload(4, lengths=lens, cache_fp8=True)
    layer = layer_for(wl)
    say(f"fp8 mixed-length decode lens={wl.lens.tolist()}")
    u1, _ = run_decode(wl, layer, decode_cache(wl, layer))
    u2, _ = run_decode(wl, layer, decode_cache(wl, layer))
    assert torch.equal(u1, u2)
    for b in range(wl.batch):
        if wl.lens[b] == 3000 and b % 2:
            continue
        ref = oracle_decode_seq(wl, b)
        assert_close(u1[b], ref["u"], True, f"u b={b} len={wl.lens[b]}")


def test_fp8_prefill_then_decode():
    """Prefill of 300 tokens into an FP8 cache (the attention of the prefill
    itself uses the unquantised latent), then three decode steps reading the
    FP8 rows the prefill wrote.  The oracle quantises its own rows, from
    their bf16 values as the layer does."""
    L0, steps = 300, 3
    wl = make_workload(3, batch=1, seq_len=L0 + steps)
    wl.cache_fp8 = True
    d = wl.dims
    layer = layer_for(wl)
    W = weights64(wl)
    h = upload(wl.h_f32, wl.h_bits, True)
    cache = layer.new_cache(1, L0 + steps)
    say("fp8 prefill 300")
    u = layer.prefill(h[:, :L0].contiguous(), cache)
    torch.cuda.synchronize()
    with Timer("oracle prefill"):
        full = O.prefill(d, W, wl.h_f32[0].astype(np.float64))
    assert_close(u[0], full["u"][:L0], True, "prefill u")
    assert_fp8_rows(cache.read_rows(0, np.arange(L0)), np.concatenate([full["c_kv"], full["k_r"]], axis=1)[:L0],
                    d, "prefill rows")
    codes, scales = O.quantize_latent(O.round_bf16(full["c_kv"]))   # codes decided from the bf16 latent
    cq = O.e4m3_decode(codes) * np.repeat(scales, O.FP8_GROUP, axis=1)
    rows_oracle = np.concatenate([cq, full["k_r"]], axis=1)
    for s in range(steps):
        t = L0 + s
        lens = torch.tensor([t + 1], dtype=torch.int32, device="cuda")
        u1 = layer.decode(h[:, t:t + 1].contiguous(), lens, L0 + steps, cache)
        torch.cuda.synchronize()
        ref = O.decode(d, W, wl.h_f32[0, t:t + 1].astype(np.float64), rows_oracle[:t], cache_fp8=True)
        assert_close(u1[0], ref["u"], True, f"decode step {s} u")
