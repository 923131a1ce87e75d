"""The reference streaming read that bench.py times beside the bank scan
reads every byte of the whole tiles it is given, once: the XOR of its
per-thread folds equals the XOR of the buffer (computed on the CPU)."""

import sys

import numpy as np
import pytest
import torch

from sparse_latent_memory_amd import readref

pytestmark = pytest.mark.gpu


def _say(msg):
    print(f"[gpu] {msg}", file=sys.stderr, flush=True)


@pytest.mark.parametrize("grid,nt", [(1, True), (7, False), (7, True), (64, True)])
def test_read_reference_folds_every_byte(grid, nt):
    g = torch.Generator().manual_seed(grid * 2 + nt)
    n_words = 37 * 32768 // 4 + 1000                  # 37 whole tiles and a ragged tail it must skip
    host = torch.randint(-2**31, 2**31 - 1, (n_words,), generator=g, dtype=torch.int64).to(torch.int32)
    buf = host.to("cuda")
    _say(f"readref: 37 tiles + tail, grid {grid}, nontemporal {nt}")
    sink, n_bytes = readref.read_tiles(buf, grid, nontemporal=nt)
    torch.cuda.synchronize()
    assert n_bytes == 37 * 32768
    want = np.bitwise_xor.reduce(host[:n_bytes // 4].numpy().view(np.uint32).reshape(-1, 4), axis=0)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    assert np.array_equal(got, want)
