"""mla_decode_noalloc (the decode entry point that allocates nothing: its
workspace is a device array inside the library) against mla_decode on the
same inputs, through the C ABI: two calls in a row, the second smaller, each
bitwise equal to mla_decode and within the bf16 bounds of the oracle."""
import numpy as np
import pytest
import torch

from head_latent_attention_18_amd import libmla as L
from mla_inputs import make_workload

from tests.gpu_harness import assert_close, decode_cache, layer_for, oracle_decode_seq, say, upload

pytestmark = pytest.mark.gpu


def test_noalloc_matches_decode_two_calls():
    for B, Lc, nq in ((24, 2100, 1), (5, 300, 2)):
        wl = make_workload(2, batch=B, uniform_len=Lc, n_q=nq)
        layer = layer_for(wl)
        h = upload(wl.h_f32, wl.h_bits, True)
        lens_host = wl.lens.astype(np.int32)
        lens = torch.from_numpy(lens_host).cuda()
        cache_ref, cache_na = decode_cache(wl, layer), decode_cache(wl, layer)
        say(f"no-alloc decode B={B} L={Lc} n_q={nq}")
        u_ref = layer.decode(h, lens, Lc, cache_ref, lens_host=lens_host)
        u_na = torch.empty_like(u_ref)
        L.mla_decode_noalloc(layer.cfg, layer.cw, h, B, nq, lens, Lc, cache_na.desc, u_na, None,
                             cache_lens_host=lens_host)
        torch.cuda.synchronize()
        assert torch.equal(u_na, u_ref), "no-alloc decode differs from mla_decode"
        assert torch.equal(cache_na.pool, cache_ref.pool), "appended cache rows differ"
        for b in (0, B - 1):
            ref = oracle_decode_seq(wl, b)
            assert_close(u_na[b], ref["u"], True, f"no-alloc u b={b}")
