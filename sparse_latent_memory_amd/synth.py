"""Seeded synthetic inputs for the MSA hot path.

This module only draws inputs; it computes none of the method's steps.
Both the HIP library's tests/benchmarks and the CPU oracle's tests take
their inputs from here.

Workloads (sizes of the pages' scenarios; the pages publish no value
statistics, so values are standard normal):

1. tiny: 64 docs x 512 tokens, fp32, pool 64, router 4 x 64, 16 query
   tokens, top-4, decode GQA 8/2 x 64 with 128 local tokens.
2. routing layer shaped like a 4B-parameter backbone: 2048 docs with
   lengths uniform in [256, 1024], bf16, pool 64, router 8 x 128, a
   256-token query prefill, top-16, decode GQA 32/8 x 128, 2048 local.
3. 16M-token bank: 32768 docs, lognormal lengths (mean 512, sigma 1,
   clipped to [64, 8192]), bf16, router 8 x 128, 8 queries of one token,
   top-16, one planted needle per query at cosine 0.6.
4. 100M-token bank: 195,313 docs x 512 tokens, pool 64 (1,562,504 pooled
   rows), bf16, router 8 x 128, one query token, top-16, 4096 local
   tokens, GQA 32/8 x 128.
5. interleaved multi-hop: 50M-token bank, lognormal lengths (mean 1024,
   sigma 1.25, clipped to [64, 65536]), 64 queries x 3 rounds of top-8,
   4096 local tokens, context capped at 16384.

Banks of configs 3-5 are drawn directly in pooled space: each pooled row of
a chunk with n tokens is N(0, 1/n), which is the exact distribution of the
mean of n iid N(0, 1) tokens (RoPE maps an isotropic Gaussian to itself).

Seeds: every tensor is drawn in blocks of 2^16 rows, block b of tensor t of
config c seeded from SeedSequence([0x4D5341, c, t, b]), so any block can be
regenerated on its own and the result does not depend on the device.
"""

from dataclasses import dataclass, field, replace

import numpy as np
import torch

SEED_TAG = 0x4D5341
BLOCK_ROWS = 1 << 16

# tensor ids used in the seed sequence
T_LENGTHS, T_KR, T_K, T_V, T_QR, T_Q, T_LOCK, T_LOCV, T_NEEDLE = range(9)

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    n_docs: int                 # for "until" lengths: 0 (drawn until total_tokens)
    lengths: str                # "fixed" | "uniform" | "lognormal"
    len_a: float                # fixed length / uniform low / lognormal mean
    len_b: float = 0.0          # uniform high / lognormal sigma
    len_lo: int = 1
    len_hi: int = 1 << 30
    total_tokens: int = 0       # lognormal drawn until this many tokens (config 5)
    pool: int = 64
    dtype: str = "bf16"
    n_router_heads: int = 8
    router_dim: int = 128
    n_q_heads: int = 32
    n_kv_heads: int = 8
    head_dim: int = 128
    batch: int = 1
    q_tokens: int = 1
    top_k: int = 16
    local_len: int = 4096
    rounds: int = 1
    ctx_cap: int = 0            # 0: no cap on [memory ; local]
    needle: bool = False
    raw: bool = True            # raw tokens (pooled by the library) vs pooled space
    rope_theta: float = 1.0e6
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]


CONFIGS = {
    1: Config(1, "tiny-32K-fp32", 64, "fixed", 512, pool=64, dtype="f32",
              n_router_heads=4, router_dim=64, n_q_heads=8, n_kv_heads=2, head_dim=64,
              batch=1, q_tokens=16, top_k=4, local_len=128),
    2: Config(2, "routing-layer-1M-bf16", 2048, "uniform", 256, 1024, pool=64,
              batch=1, q_tokens=256, top_k=16, local_len=2048),
    3: Config(3, "bank-16M-needles", 32768, "lognormal", 512, 1.0, len_lo=64, len_hi=8192,
              batch=8, q_tokens=1, top_k=16, local_len=4096, needle=True, raw=False),
    4: Config(4, "bank-100M-decode", 195313, "fixed", 512, batch=1, q_tokens=1, top_k=16,
              local_len=4096, raw=False),
    5: Config(5, "interleave-50M-multihop", 0, "lognormal", 1024, 1.25, len_lo=64,
              len_hi=65536, total_tokens=50_000_000, batch=64, q_tokens=1, top_k=8,
              local_len=4096, rounds=3, ctx_cap=16384, raw=False),
}


def config(cid, **overrides):
    """The named workload, optionally with fields replaced (smaller test cases)."""
    cfg = CONFIGS[cid]
    return replace(cfg, **overrides) if overrides else cfg


# --------------------------------------------------------------------------
# seeds and raw draws
# --------------------------------------------------------------------------

def seed_of(cid, tensor_id, block=0, step=0):
    ss = np.random.SeedSequence([SEED_TAG, cid, tensor_id, block, step])
    return int(ss.generate_state(1, np.uint64)[0] & ((1 << 63) - 1))


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal_rows(cid, tensor_id, n_rows, row_shape, device, step=0):
    """n_rows x row_shape standard normals (fp32), block-seeded."""
    out = torch.empty((n_rows,) + tuple(row_shape), dtype=torch.float32, device=device)
    for b, r0 in enumerate(range(0, n_rows, BLOCK_ROWS)):
        r1 = min(r0 + BLOCK_ROWS, n_rows)
        g = _gen(device, seed_of(cid, tensor_id, b, step))
        out[r0:r1] = torch.randn((r1 - r0,) + tuple(row_shape), generator=g,
                                 device=device, dtype=torch.float32)
    return out


# --------------------------------------------------------------------------
# document lengths and offsets
# --------------------------------------------------------------------------

def doc_lengths(cfg):
    """Token count of every document (int64 numpy array)."""
    rng = np.random.Generator(np.random.PCG64(seed_of(cfg.cid, T_LENGTHS)))
    if cfg.lengths == "fixed":
        return np.full(cfg.n_docs, int(cfg.len_a), dtype=np.int64)
    if cfg.lengths == "uniform":
        return rng.integers(int(cfg.len_a), int(cfg.len_b) + 1, size=cfg.n_docs).astype(np.int64)
    if cfg.lengths == "lognormal":
        mu = np.log(cfg.len_a) - cfg.len_b ** 2 / 2.0

        def draw(n):
            x = np.rint(rng.lognormal(mu, cfg.len_b, size=n))
            return np.clip(x, cfg.len_lo, cfg.len_hi).astype(np.int64)

        if cfg.total_tokens:
            chunks, total = [], 0
            while total < cfg.total_tokens:
                c = draw(1 << 16)
                chunks.append(c)
                total += int(c.sum())
            lens = np.concatenate(chunks)
            n = int(np.searchsorted(np.cumsum(lens), cfg.total_tokens) + 1)
            return lens[:n]
        return draw(cfg.n_docs)
    raise ValueError(cfg.lengths)


def token_offsets(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def chunk_counts(lens, pool_size):
    """Pooled rows per document (ceil(L/P)): a shape, not a method step."""
    lens = np.asarray(lens, dtype=np.int64)
    return -(-lens // pool_size)


def row_offsets(lens, pool_size):
    return np.concatenate([[0], np.cumsum(chunk_counts(lens, pool_size))]).astype(np.int64)


# --------------------------------------------------------------------------
# banks
# --------------------------------------------------------------------------

def raw_bank(cfg, lens=None, device="cpu"):
    """Raw per-token K, V (pre-RoPE) [T, Hkv, D] and Kr [T, Hr, dr] in the
    storage dtype, plus token offsets (int64, on device)."""
    lens = doc_lengths(cfg) if lens is None else np.asarray(lens, dtype=np.int64)
    n_tok = int(lens.sum())
    dt = cfg.torch_dtype
    k = _normal_rows(cfg.cid, T_K, n_tok, (cfg.n_kv_heads, cfg.head_dim), device).to(dt)
    v = _normal_rows(cfg.cid, T_V, n_tok, (cfg.n_kv_heads, cfg.head_dim), device).to(dt)
    kr = _normal_rows(cfg.cid, T_KR, n_tok, (cfg.n_router_heads, cfg.router_dim), device).to(dt)
    off = torch.as_tensor(token_offsets(lens), device=device)
    return {"k": k, "v": v, "kr": kr, "doc_tok_off": off, "lens": lens}


def _pooled_rows(cfg, tensor_id, lens, row_shape, device, out=None, host_out=None):
    """Pooled-space rows: chunk of n tokens ~ N(0, 1/n), in storage dtype."""
    counts = chunk_counts(lens, cfg.pool)
    n_pool = int(counts.sum())
    # tokens in each pooled row: full chunks P, the tail chunk L - (C-1)P
    ntok = np.full(n_pool, cfg.pool, dtype=np.int64)
    tails = np.cumsum(counts) - 1
    ntok[tails] = lens - (counts - 1) * cfg.pool
    inv_sd = torch.as_tensor(1.0 / np.sqrt(ntok), dtype=torch.float32)
    dt = cfg.torch_dtype
    if out is None and host_out is None:
        out = torch.empty((n_pool,) + tuple(row_shape), dtype=dt, device=device)
    tgt = out if out is not None else host_out
    for b, r0 in enumerate(range(0, n_pool, BLOCK_ROWS)):
        r1 = min(r0 + BLOCK_ROWS, n_pool)
        g = _gen(device, seed_of(cfg.cid, tensor_id, b))
        x = torch.randn((r1 - r0,) + tuple(row_shape), generator=g, device=device,
                        dtype=torch.float32)
        sd = inv_sd[r0:r1].to(device).reshape((-1,) + (1,) * len(row_shape))
        tgt[r0:r1].copy_((x * sd).to(dt))
    return tgt


def pooled_router_bank(cfg, lens, device="cpu"):
    """Kr_bar [n_pool, Hr, dr] drawn in pooled space."""
    return _pooled_rows(cfg, T_KR, lens, (cfg.n_router_heads, cfg.router_dim), device)


def tile_router_bank(kr, pad_value=0.0):
    """A row-major router bank [n, Hr, dr] re-laid out in the library's tiled
    order: whole 16-row tiles, each storing its rows' 16-byte pieces
    piece-major.  A permutation of the elements (padding rows = pad_value);
    returned as [ceil(n/16)*16, Hr, dr] so that it indexes like the rows."""
    n, hr, dr = kr.shape
    pe = 16 // kr.element_size()
    nt = -(-n // 16)
    rows = torch.full((nt * 16, hr, dr), pad_value, dtype=kr.dtype, device=kr.device)
    rows[:n] = kr
    return rows.view(nt, 16, hr * dr // pe, pe).permute(0, 2, 1, 3).contiguous().view(nt * 16, hr, dr)


def untile_router_bank(kt, n):
    """Inverse of tile_router_bank: the first n rows, row-major."""
    rows16, hr, dr = kt.shape
    pe = 16 // kt.element_size()
    nt = rows16 // 16
    return kt.view(nt, hr * dr // pe, 16, pe).permute(0, 2, 1, 3).contiguous().view(rows16, hr, dr)[:n]


def pooled_content_bank(cfg, lens, device="cpu", pin=False):
    """K_bar/V_bar [n_pool, 2, Hkv, D] drawn in pooled space.  With pin=True
    the result lives in pinned host memory (drawn on `device` block by block)."""
    shape = (2, cfg.n_kv_heads, cfg.head_dim)
    if pin:
        n_pool = int(chunk_counts(lens, cfg.pool).sum())
        host = torch.empty((n_pool,) + shape, dtype=cfg.torch_dtype, pin_memory=True)
        return _pooled_rows(cfg, T_K, lens, shape, device, host_out=host)
    return _pooled_rows(cfg, T_K, lens, shape, device)


# --------------------------------------------------------------------------
# queries and local context
# --------------------------------------------------------------------------

def router_queries(cfg, step=0, device="cpu"):
    """Qr [B, Tq, Hr, dr] in storage dtype."""
    x = _normal_rows(cfg.cid, T_QR, cfg.batch * cfg.q_tokens,
                     (cfg.n_router_heads, cfg.router_dim), device, step)
    return x.reshape(cfg.batch, cfg.q_tokens, cfg.n_router_heads, cfg.router_dim).to(cfg.torch_dtype)


def decode_queries(cfg, step=0, device="cpu"):
    """q [B, Hq, D] (before RoPE) in storage dtype."""
    x = _normal_rows(cfg.cid, T_Q, cfg.batch, (cfg.n_q_heads, cfg.head_dim), device, step)
    return x.to(cfg.torch_dtype)


def prefill_queries(cfg, step=0, device="cpu"):
    """q [B, Tq, Hq, D] (before RoPE) for a block of query tokens, in
    storage dtype."""
    x = _normal_rows(cfg.cid, T_Q, cfg.batch * cfg.q_tokens, (cfg.n_q_heads, cfg.head_dim), device, step + 1000)
    return x.reshape(cfg.batch, cfg.q_tokens, cfg.n_q_heads, cfg.head_dim).to(cfg.torch_dtype)


def local_context(cfg, cap=None, device="cpu"):
    """Local K (before RoPE) and V [B, T_cap, Hkv, D]; every query holds
    cfg.local_len tokens."""
    cap = cfg.local_len if cap is None else cap
    shape = (cfg.n_kv_heads, cfg.head_dim)
    k = _normal_rows(cfg.cid, T_LOCK, cfg.batch * cap, shape, device)
    v = _normal_rows(cfg.cid, T_LOCV, cfg.batch * cap, shape, device)
    k = k.reshape(cfg.batch, cap, *shape).to(cfg.torch_dtype)
    v = v.reshape(cfg.batch, cap, *shape).to(cfg.torch_dtype)
    return k, v


# --------------------------------------------------------------------------
# planted needles (routing stand-in for needle-in-a-haystack retrieval)
# --------------------------------------------------------------------------

def plant_needles(cfg, qr, kr_pooled, row_off, cosine=0.6, scale=0.125):
    """For each query b (token 0) pick a distinct random document and one of
    its pooled rows, and overwrite that row so that per router head it equals
    scale * (cosine * q_unit + sqrt(1 - cosine^2) * u) with u a random unit
    vector orthogonal to q_unit.  Returns the needle document ids (numpy).
    Operates in place on kr_pooled (any device)."""
    rng = np.random.Generator(np.random.PCG64(seed_of(cfg.cid, T_NEEDLE)))
    n_docs = len(row_off) - 1
    docs = rng.choice(n_docs, size=qr.shape[0], replace=False)
    q = qr[:, 0].to(torch.float64).cpu().numpy()          # [B, Hr, dr]
    side = np.sqrt(1.0 - cosine * cosine)
    for b, d in enumerate(docs):
        r0, r1 = int(row_off[d]), int(row_off[d + 1])
        row = r0 + int(rng.integers(0, r1 - r0))
        new = np.empty(q.shape[1:], dtype=np.float64)
        for h in range(q.shape[1]):
            qu = q[b, h] / np.linalg.norm(q[b, h])
            u = rng.standard_normal(q.shape[2])
            u -= (u @ qu) * qu
            u /= np.linalg.norm(u)
            new[h] = scale * (cosine * qu + side * u)
        kr_pooled[row] = torch.as_tensor(new, dtype=torch.float32).to(kr_pooled.dtype).to(kr_pooled.device)
    return docs
