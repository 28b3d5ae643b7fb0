"""Thin helpers over the ctypes binding: device buffers (torch), cache
descriptors and workspaces.  No arithmetic of the method happens here."""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import libmla as L


def upload(f32: np.ndarray, bits: Optional[np.ndarray], bf16: bool, device="cuda") -> torch.Tensor:
    """Host array -> device tensor holding exactly the given values."""
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(f32, dtype=np.float32)).to(device)


class CacheBuf:
    """A latent cache pool plus its descriptor (contiguous or paged)."""

    def __init__(self, pool: torch.Tensor, desc: L.mla_cache, table: Optional[torch.Tensor] = None,
                 table_host: Optional[np.ndarray] = None, block_size: int = 0, max_len: int = 0):
        self.pool, self.desc, self.table, self.table_host = pool, desc, table, table_host
        self.block_size, self.max_len = block_size, max_len

    @staticmethod
    def contiguous(d_row: int, tdtype, batch: int, max_len: int, device="cuda") -> "CacheBuf":
        """d_row: elements per row of tdtype (FP8 rows: bytes, tdtype uint8)."""
        pool = torch.zeros(batch * max_len, d_row, dtype=tdtype, device=device)
        return CacheBuf(pool, L.make_cache(pool, max_len=max_len), max_len=max_len)

    @staticmethod
    def paged(pool: torch.Tensor, block_size: int, table_host: np.ndarray, device="cuda") -> "CacheBuf":
        table = torch.from_numpy(np.ascontiguousarray(table_host, dtype=np.int32)).to(device)
        n_blocks = pool.shape[0] // block_size
        desc = L.make_cache(pool, block_size=block_size, n_blocks=n_blocks, block_table=table,
                            max_blocks_per_seq=table_host.shape[1])
        return CacheBuf(pool, desc, table, table_host, block_size=block_size)

    def row_index(self, b: int, positions: np.ndarray) -> np.ndarray:
        positions = np.asarray(positions, dtype=np.int64)
        if self.table_host is None:
            return b * self.max_len + positions
        blk = self.table_host[b, positions // self.block_size].astype(np.int64)
        return blk * self.block_size + positions % self.block_size

    def read_rows(self, b: int, positions) -> torch.Tensor:
        idx = torch.from_numpy(self.row_index(b, positions)).to(self.pool.device)
        return self.pool.index_select(0, idx)


class MlaLayer:
    """One MLA layer's weights on the device and the libmla calls on them."""

    def __init__(self, dims, dtype: str, weights: Dict[str, torch.Tensor], cache: str = "layer",
                 scales: Optional[Dict[str, torch.Tensor]] = None):
        """scales (by weight name): the block scales of FP8 projections,
        whose weights are then E4M3 codes (MLA_WEIGHTS_FP8_BLOCK)."""
        self.dims, self.dtype, self.cache = dims, dtype, cache
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.weights, self.scales = weights, scales
        self.cfg = L.make_config(dims, dtype, cache, "fp8" if scales else "layer")
        # a cache row: d_row elements of the layer dtype, or the FP8 row's bytes
        self.row_width = L.mla_cache_bytes_per_token(self.cfg) if cache == "fp8" else dims.d_row
        self.cache_tdtype = torch.uint8 if cache == "fp8" else self.tdtype
        self.cw = L.make_weights(weights, scales)
        self._ws: Dict[str, torch.Tensor] = {}

    @classmethod
    def from_host(cls, dims, dtype: str, weights_f32: Dict[str, np.ndarray],
                  weights_bits: Dict[str, Optional[np.ndarray]], device="cuda", cache: str = "layer",
                  weights_fp8: Optional[Dict[str, tuple]] = None) -> "MlaLayer":
        """weights_fp8: (E4M3 codes, block scales) by weight name for the FP8
        projections; those replace the layer-dtype weights of the same name."""
        bf16 = dtype == "bf16"
        w = {k: upload(weights_f32[k], weights_bits.get(k), bf16, device) for k in L.WEIGHT_NAMES}
        scales = None
        if weights_fp8:
            scales = {}
            for k, (codes, sc) in weights_fp8.items():
                w[k] = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).to(device)
                scales[k] = torch.from_numpy(np.ascontiguousarray(sc, dtype=np.float32)).to(device)
        return cls(dims, dtype, w, cache, scales)

    def workspace(self, key: str, nbytes: int, device) -> torch.Tensor:
        ws = self._ws.get(key)
        if ws is None or ws.numel() < nbytes:
            ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._ws[key] = ws
        return ws

    def new_cache(self, batch: int, max_len: int, device="cuda") -> CacheBuf:
        return CacheBuf.contiguous(self.row_width, self.cache_tdtype, batch, max_len, device)

    def prefill(self, h: torch.Tensor, cache: CacheBuf, want_o: bool = False, stream=None):
        B, S, _ = h.shape
        u = torch.empty(B, S, self.dims.d_model, dtype=self.tdtype, device=h.device)
        o = torch.empty(B * S, self.dims.n_heads, self.dims.d_v, dtype=self.tdtype, device=h.device) if want_o else None
        nbytes = L.mla_workspace_size(self.cfg, L.MLA_OP_PREFILL, B, S, 0)
        ws = self.workspace("prefill", nbytes, h.device)
        L.mla_prefill(self.cfg, self.cw, h, B, S, cache.desc, u, o, ws, ws.numel(), stream)
        return (u, o) if want_o else u

    def decode(self, h: torch.Tensor, lens: torch.Tensor, max_len: int, cache: CacheBuf, want_o: bool = False,
               stream=None, u: Optional[torch.Tensor] = None, lens_host=None):
        B, nq, _ = h.shape
        if u is None:
            u = torch.empty(B, nq, self.dims.d_model, dtype=self.tdtype, device=h.device)
        o = torch.empty(B * nq, self.dims.n_heads, self.dims.d_v, dtype=self.tdtype, device=h.device) if want_o else None
        nbytes = L.mla_workspace_size(self.cfg, L.MLA_OP_DECODE, B, nq, max_len)
        ws = self.workspace("decode", nbytes, h.device)
        L.mla_decode(self.cfg, self.cw, h, B, nq, lens, max_len, cache.desc, u, o, ws, ws.numel(), stream,
                     cache_lens_host=lens_host)
        return (u, o) if want_o else u

    def compress_kv(self, h: torch.Tensor, seq_idx: torch.Tensor, pos: torch.Tensor, batch: int, cache: CacheBuf,
                    stream=None):
        n = h.shape[0]
        nbytes = L.mla_workspace_size(self.cfg, L.MLA_OP_COMPRESS, 1, n, 0)
        ws = self.workspace("compress", nbytes, h.device) if nbytes else None
        L.mla_compress_kv(self.cfg, self.cw, h, n, seq_idx, pos, batch, cache.desc, ws,
                          ws.numel() if ws is not None else 0, stream)


def cache_from_rows(rows_per_seq, lens, d_row: int, bf16: bool, paged: bool = False, block_size: int = 64,
                    perm=None, max_len: Optional[int] = None, device="cuda") -> CacheBuf:
    """Device cache whose sequence b starts with the given rows (host arrays:
    bf16 bit patterns as uint16, float32, or FP8 rows as uint8 bytes with
    d_row the row's bytes).  Positions after them are zero.  Paged: logical
    block k of sequence b is physical block perm[offset_b + k]."""
    lens = np.asarray(lens, dtype=np.int64)
    B = len(rows_per_seq)
    raw = rows_per_seq[0].dtype == np.uint8
    np_dtype = np.uint8 if raw else (np.uint16 if bf16 else np.float32)
    if not paged:
        ml = int(max_len or lens.max())
        pool = np.zeros((B * ml, d_row), dtype=np_dtype)
        for b in range(B):
            pool[b * ml: b * ml + rows_per_seq[b].shape[0]] = rows_per_seq[b]
        t = torch.from_numpy(pool).to(device) if raw else upload(pool, pool, bf16, device)
        return CacheBuf(t, L.make_cache(t, max_len=ml), max_len=ml)
    bs = block_size
    nblk = [(int(l) + bs - 1) // bs for l in lens]
    if perm is None:
        perm = np.arange(sum(nblk), dtype=np.int32)
    max_blocks = max(nblk)
    if max_len:
        max_blocks = max(max_blocks, (int(max_len) + bs - 1) // bs)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    off = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[off:off + nblk[b]]
        off += nblk[b]
    pool = np.zeros((len(perm) * bs, d_row), dtype=np_dtype)
    for b in range(B):
        n = rows_per_seq[b].shape[0]
        pos = np.arange(n)
        phys = table[b, pos // bs].astype(np.int64) * bs + pos % bs
        pool[phys] = rows_per_seq[b]
    t = torch.from_numpy(pool).to(device) if raw else upload(pool, pool, bf16, device)
    return CacheBuf.paged(t, bs, table, device)
