"""Seeded synthetic inputs for the eviction pass.

This module holds the input recipe only -- random caches, calibration
statistics and positions with the shapes of the workloads the source pages
describe (Qwen3-8B-shaped caches: 36 layers x 8 KV / 32 query heads,
head_dim 128, 32K context; a uniform head_dim 256 model; a paged batch).  It
contains none of the method's arithmetic; the test-suite and the benchmark
feed the same bytes to the HIP library and to the CPU oracle.

Recipe (the same for every workload):
* K and V: N(0, 1) times a per-(layer, KV head, channel) scale drawn as
  exp(N(0, 0.5^2)); K and V have separate scales.  Stored as fp16 (round to
  nearest even) or q8_0 (per block of 32 values: scale d = amax/127 stored as
  fp16, q = round-half-away-from-zero(x / d) clamped to [-127, 127]).
* Statistics per (layer, query head, frequency pair): mean-query magnitude
  lognormal(0, 1), phase uniform in [0, 2*pi), norm-term weight equal to the
  magnitude times U[0, 1).
* Positions 0..n-1.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

KV_F16 = 0
KV_Q8_0 = 1


def pow2_offsets(max_exp: int):
    """{1, 2, 4, ..., 2^max_exp}."""
    return [1 << e for e in range(max_exp + 1)]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    L: int
    Hkv: int
    Hq: int
    hd: int
    n: int
    k_type: int
    v_type: int
    offsets: tuple
    budget: int
    sink: int
    window: int
    seed: int
    theta: float = 1e6
    # paged batch only
    n_seq: int = 0
    len_lo: int = 0
    len_hi: int = 0
    budget_frac: float = 0.0
    append: int = 0

    @property
    def G(self):
        return self.Hq // self.Hkv


WORKLOADS = {
    # 1 layer x 1 KV head x 4 query heads, hd 128, 4096 tokens, fp16, 50% budget.
    "tiny_1x1_4k_f16": Workload("tiny_1x1_4k_f16", 1, 1, 4, 128, 4096, KV_F16, KV_F16,
                                tuple(pow2_offsets(12)), 2048, 4, 512, 0),
    # One Qwen3-8B-shaped layer: 8 KV / 32 query heads, 32768 tokens, fp16, 25% budget.
    "qwen3_8b_layer_32k_f16": Workload("qwen3_8b_layer_32k_f16", 1, 8, 32, 128, 32768, KV_F16,
                                       KV_F16, tuple(pow2_offsets(15)), 8192, 4, 512, 1),
    # Full Qwen3-8B-shaped cache: 36 x 8 KV heads, 32768 tokens, q8_0 K / fp16 V, 25%.
    "qwen3_8b_full_32k_q8": Workload("qwen3_8b_full_32k_q8", 36, 8, 32, 128, 32768, KV_Q8_0,
                                     KV_F16, tuple(pow2_offsets(15)), 8192, 0, 512, 2),
    # Uniform head_dim 256: 48 layers x 4 KV / 16 query heads, 131072 tokens, fp16, 10%.
    "hd256_48x4_128k_f16": Workload("hd256_48x4_128k_f16", 48, 4, 16, 256, 131072, KV_F16,
                                    KV_F16, tuple(pow2_offsets(17)), 13107, 4, 1024, 3),
    # Paged batch: 16 sequences of 8K..64K tokens, 16-token blocks in shuffled physical
    # order, Qwen3-8B shape, q8_0 K / fp16 V, 30% budget, a pass every 128 appended tokens.
    "paged16_qwen3_8b_q8": Workload("paged16_qwen3_8b_q8", 36, 8, 32, 128, 0, KV_Q8_0, KV_F16,
                                    tuple(pow2_offsets(16)), 0, 0, 512, 4, n_seq=16,
                                    len_lo=8192, len_hi=65536, budget_frac=0.3, append=128),
}


def row_bytes(kv_type: int, hd: int) -> int:
    if kv_type == KV_F16:
        return 2 * hd
    if kv_type == KV_Q8_0:
        return 34 * (hd // 32)
    raise ValueError(kv_type)


# --------------------------------------------------------------------------
# Calibration statistics (host, fp32 [L][Hq][F])
# --------------------------------------------------------------------------

def gen_stats(L: int, Hq: int, hd: int, seed: int):
    rng = np.random.Generator(np.random.PCG64(seed * 7919 + 17))
    F = hd // 2
    mag = rng.lognormal(0.0, 1.0, size=(L, Hq, F))
    phase = rng.uniform(0.0, 2.0 * math.pi, size=(L, Hq, F))
    w = mag * rng.uniform(0.0, 1.0, size=(L, Hq, F))
    q_re = (mag * np.cos(phase)).astype(np.float32)
    q_im = (mag * np.sin(phase)).astype(np.float32)
    return q_re, q_im, w.astype(np.float32)


# --------------------------------------------------------------------------
# Storage encodings of synthetic values
# --------------------------------------------------------------------------

def encode_q8_0(x: torch.Tensor) -> torch.Tensor:
    """x: float32 [..., hd] -> uint8 [..., hd/32*34] (q8_0 blocks)."""
    shp = x.shape
    hd = shp[-1]
    nb = hd // 32
    xb = x.reshape(-1, nb, 32)
    amax = xb.abs().amax(dim=-1, keepdim=True)
    d16 = (amax / 127.0).to(torch.float16)
    d = d16.to(torch.float32)
    safe = torch.where(d > 0, d, torch.ones_like(d))
    t = xb / safe
    q = torch.sign(t) * torch.floor(t.abs() + 0.5)
    q = torch.where(d > 0, q, torch.zeros_like(q)).clamp_(-127, 127).to(torch.int8)
    out = torch.empty(xb.shape[0], nb, 34, dtype=torch.uint8, device=x.device)
    out[:, :, 0:2] = d16.view(torch.uint8).reshape(-1, nb, 2)
    out[:, :, 2:] = q.view(torch.uint8)
    return out.reshape(*shp[:-1], nb * 34)


def encode(x: torch.Tensor, kv_type: int) -> torch.Tensor:
    """float32 [..., hd] -> uint8 rows in the given storage type."""
    if kv_type == KV_F16:
        return x.to(torch.float16).view(torch.uint8)
    if kv_type == KV_Q8_0:
        return encode_q8_0(x)
    raise ValueError(kv_type)


# --------------------------------------------------------------------------
# Caches
# --------------------------------------------------------------------------

def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def gen_values(shape, hd, gen, device, scale):
    """N(0,1) [.., hd] times a per-channel scale [hd]."""
    x = torch.randn(*shape, hd, generator=gen, device=device, dtype=torch.float32)
    return x * scale


def gen_cache(L: int, Hkv: int, hd: int, cap: int, n: int, k_type: int, v_type: int, seed: int,
              device="cpu"):
    """Contiguous cache: K, V uint8 [L, Hkv, cap, row_bytes]; pos int32 [L, Hkv, cap].

    Rows n..cap-1 are zero.  Generated a layer at a time (all KV heads of the
    layer at once) to bound temporaries and the number of device launches.
    """
    device = torch.device(device)
    gen = _gen(device, seed * 1000003 + 1)
    kb, vb = row_bytes(k_type, hd), row_bytes(v_type, hd)
    k = torch.zeros(L, Hkv, cap, kb, dtype=torch.uint8, device=device)
    v = torch.zeros(L, Hkv, cap, vb, dtype=torch.uint8, device=device)
    ks = torch.exp(0.5 * torch.randn(L, Hkv, 1, hd, generator=gen, device=device))
    vs = torch.exp(0.5 * torch.randn(L, Hkv, 1, hd, generator=gen, device=device))
    for l in range(L):
        if n > 0:
            k[l, :, :n] = encode(gen_values((Hkv, n), hd, gen, device, ks[l]), k_type)
            v[l, :, :n] = encode(gen_values((Hkv, n), hd, gen, device, vs[l]), v_type)
    pos = torch.zeros(L, Hkv, cap, dtype=torch.int32, device=device)
    pos[:, :, :n] = torch.arange(n, dtype=torch.int32, device=device)
    return k, v, pos


def make_case(wl: Workload, device="cpu", n=None, cap=None, L=None):
    """Stats (host numpy) and a contiguous cache (torch on `device`) for a workload.

    n, cap, L override the workload's sizes (smaller parity cases).
    """
    n = wl.n if n is None else n
    cap = n if cap is None else cap
    L = wl.L if L is None else L
    q_re, q_im, w = gen_stats(L, wl.Hq, wl.hd, wl.seed)
    k, v, pos = gen_cache(L, wl.Hkv, wl.hd, cap, n, wl.k_type, wl.v_type, wl.seed, device)
    return dict(q_re=q_re, q_im=q_im, w=w, k=k, v=v, pos=pos, n=n, cap=cap, L=L)


# --------------------------------------------------------------------------
# Paged batch
# --------------------------------------------------------------------------

BLOCK = 16


def paged_lengths(wl: Workload):
    """Per-sequence context lengths L_s ~ U{len_lo..len_hi}, seed per sequence."""
    out = []
    for s in range(wl.n_seq):
        rng = np.random.Generator(np.random.PCG64(wl.seed * 1000 + s))
        out.append(int(rng.integers(wl.len_lo, wl.len_hi + 1)))
    return out


def shuffled_blocks(n_blocks: int, seed: int):
    rng = np.random.Generator(np.random.PCG64(seed * 31 + 5))
    return rng.permutation(n_blocks).astype(np.int32)


def gen_paged(L: int, Hkv: int, hd: int, k_type: int, v_type: int, lens, seed: int,
              device="cpu", extra_blocks: int = 0):
    """Paged cache for sequences of the given lengths.

    Pools [L][n_blocks][Hkv][16][row_bytes] (K, V) and [L][n_blocks][Hkv][16]
    (positions 0..n-1); each sequence's blocks are a slice of one seeded random
    permutation of the physical blocks.  block_table: int32 [n_seq][max_blocks]
    (unused entries -1).  `extra_blocks` leaves room for appended tokens.
    """
    device = torch.device(device)
    kb, vb = row_bytes(k_type, hd), row_bytes(v_type, hd)
    nblk = [(n + extra_blocks * BLOCK + BLOCK - 1) // BLOCK for n in lens]
    total = sum(nblk)
    perm = torch.from_numpy(shuffled_blocks(total, seed)).to(device)
    max_blocks = max(nblk)
    bt = torch.full((len(lens), max_blocks), -1, dtype=torch.int32, device=device)
    k_pool = torch.zeros(L, total, Hkv, BLOCK, kb, dtype=torch.uint8, device=device)
    v_pool = torch.zeros(L, total, Hkv, BLOCK, vb, dtype=torch.uint8, device=device)
    p_pool = torch.zeros(L, total, Hkv, BLOCK, dtype=torch.int32, device=device)
    start = 0
    for s, n in enumerate(lens):
        blocks = perm[start:start + nblk[s]]
        start += nblk[s]
        bt[s, :nblk[s]] = blocks
        cap = nblk[s] * BLOCK
        k, v, pos = gen_cache(L, Hkv, hd, cap, n, k_type, v_type, seed * 1000 + s, device)
        # [L][Hkv][cap][rb] -> [L][blk][Hkv][16][rb]
        k_pool[:, blocks] = k.view(L, Hkv, nblk[s], BLOCK, kb).transpose(1, 2)
        v_pool[:, blocks] = v.view(L, Hkv, nblk[s], BLOCK, vb).transpose(1, 2)
        p_pool[:, blocks] = pos.view(L, Hkv, nblk[s], BLOCK).transpose(1, 2)
    return dict(k_pool=k_pool, v_pool=v_pool, pos_pool=p_pool, block_table=bt, lens=list(lens),
                n_blocks=total)


def paged_rows(pool: torch.Tensor, bt_row: torch.Tensor, n: int) -> torch.Tensor:
    """Logical rows 0..n-1 of one sequence: [L][Hkv][n][...] from a pool."""
    nb = (n + BLOCK - 1) // BLOCK
    blocks = bt_row[:nb].long()
    x = pool[:, blocks]  # [L][nb][Hkv][16][...]
    x = x.transpose(1, 2).reshape(pool.shape[0], pool.shape[2], nb * BLOCK, *pool.shape[4:])
    return x[:, :, :n]


def append_paged(pg: dict, s: int, n: int, m: int, first_pos: int, L: int, Hkv: int, hd: int,
                 k_type: int, v_type: int, seed: int):
    """Write m fresh rows (same recipe as gen_cache) at logical rows n..n+m-1 of
    sequence s, with positions first_pos, first_pos+1, ... (decode appends)."""
    pools = pg["k_pool"], pg["v_pool"], pg["pos_pool"]
    device = pools[0].device
    k, v, _ = gen_cache(L, Hkv, hd, m, m, k_type, v_type, seed, device)
    r = torch.arange(n, n + m, device=device)
    blk = pg["block_table"][s].to(device).long()[r >> 4]
    within = r & (BLOCK - 1)
    pos = (first_pos + torch.arange(m, device=device, dtype=torch.int32))
    # advanced indices around a slice put the row dimension first: [m][L][Hkv][...]
    pools[0][:, blk, :, within] = k.permute(2, 0, 1, 3)
    pools[1][:, blk, :, within] = v.permute(2, 0, 1, 3)
    pools[2][:, blk, :, within] = pos.view(m, 1, 1).expand(m, L, Hkv)


# --------------------------------------------------------------------------
# Calibration query streams
# --------------------------------------------------------------------------

# name -> (layers, query heads, head_dim, tokens, dtype): a Qwen3-8B-shaped
# stream of pre-RoPE query rows, the size of one calibration sample (the
# llama.cpp page suggests 512-2K tokens per sample).
CALIB_WORKLOADS = {
    "calib_qwen3_8b_2k_f32": (36, 32, 128, 2048, torch.float32),
}


def gen_query_stream(L: int, Hq: int, hd: int, T: int, dtype, seed: int, device):
    """Per layer a device tensor [T, Hq*hd]: a fixed per-(head, dim) mean direction
    (lognormal size, uniform phase per pair) plus N(0,1) noise per token."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    F = hd // 2
    out = []
    for _ in range(L):
        mag = torch.exp(torch.randn(Hq, F, generator=g))
        ph = torch.rand(Hq, F, generator=g) * (2 * np.pi)
        mean = torch.cat([mag * torch.cos(ph), mag * torch.sin(ph)], dim=1)  # [Hq, hd]
        noise = torch.randn(T, Hq, hd, generator=g)
        out.append((noise + mean).reshape(T, Hq * hd).to(dtype).to(device))
    return out

