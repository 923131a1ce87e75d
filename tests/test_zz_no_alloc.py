"""msa_sparse_decode_noalloc (the decode entry point that allocates nothing
and keeps its split partials in the library's static scratch) against
msa_sparse_decode with a caller workspace, through the C ABI: two calls in a
row, the second with smaller sizes, for bf16 (matrix-core attention) and
fp32 (split-KV kernel).  Both run the same kernels on the same plan, so the
outputs must agree to the decode tolerance and are in fact identical."""

import numpy as np
import pytest
import torch

import oracle
import sparse_latent_memory_amd as msa
from parity_util import check_decode, np64, storage
from sparse_latent_memory_amd import _lib

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    _lib.load()


def _inputs(seed, b, hq, hkv, d, mem_cap, loc_cap, dtype):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(b, hq, d, generator=g).to(dtype)
    mem = torch.randn(b, mem_cap, 2, hkv, d, generator=g).to(dtype)
    lk = torch.randn(b, loc_cap, hkv, d, generator=g).to(dtype)
    lv = torch.randn(b, loc_cap, hkv, d, generator=g).to(dtype)
    mem_len = torch.randint(0, mem_cap + 1, (b,), generator=g, dtype=torch.int32)
    loc_len = torch.randint(1, loc_cap + 1, (b,), generator=g, dtype=torch.int32)
    pos = torch.randint(0, 4096, (b,), generator=g, dtype=torch.int32)
    return q, mem, mem_len, lk, lv, loc_len, pos


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_decode_matches_workspace_decode(dtype):
    shapes = [(8, 32, 8, 128, 1024, 4096), (2, 16, 2, 64, 96, 300)]   # the second call is smaller
    for n, (b, hq, hkv, d, mem_cap, loc_cap) in enumerate(shapes):
        print(f"\n[case] noalloc decode call {n}: B={b} Hq={hq} Hkv={hkv} D={d} mem {mem_cap} local {loc_cap} {dtype}",
              flush=True)
        q, mem, mem_len, lk, lv, loc_len, pos = [t.to(DEV) for t in _inputs(n, b, hq, hkv, d, mem_cap, loc_cap,
                                                                             dtype)]
        ref, ref_lse = msa.sparse_decode(q, mem, mem_len, lk, lv, loc_len, pos, 1e6)
        out = torch.full_like(ref, float("nan"))
        lse = torch.full_like(ref_lse, float("nan"))
        got, got_lse = msa.sparse_decode_noalloc(q, mem, mem_len, lk, lv, loc_len, pos, 1e6, out, lse)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        check_decode(np64(got), np64(ref), dtype, f"noalloc call {n}")
        assert torch.equal(got, ref) and torch.equal(got_lse, ref_lse), f"noalloc call {n}: not identical"
        if n == 1:      # the smaller call also against the oracle
            ro, _ = oracle.decode(np64(q), np64(mem), np64(mem_len), np64(lk), np64(lv), np64(loc_len), np64(pos),
                                  1e6, None, storage(dtype))
            check_decode(np64(got), ro, dtype, "noalloc vs oracle")
