"""Host-side logic of bench.py that needs no GPU: the CPU baseline's
whole-step timing (the oracle over scoring, top-k, the encode batch and the
decode step) on a small bank of the headline workload's shape."""

import numpy as np
import torch

import bench
from sparse_latent_memory_amd import synth


def test_cpu_baseline_times_the_whole_step_oracle():
    cfg = synth.config(4, n_docs=600)
    lens = synth.doc_lengths(cfg)
    pool_off = synth.row_offsets(lens, cfg.pool)
    kr = synth.pooled_router_bank(cfg, lens, device="cpu")
    qr = synth.router_queries(cfg, step=0, device="cpu")
    enc = synth.config(4, n_docs=4)
    enc_lens = synth.doc_lengths(enc)
    enc_bank = synth.raw_bank(enc, lens=enc_lens, device="cpu")
    lk, lv = synth.local_context(cfg, device="cpu")
    k = cfg.top_k
    mem_cap = k * (512 // cfg.pool)
    g = torch.Generator().manual_seed(3)
    mem = torch.randn((cfg.batch, mem_cap, 2, cfg.n_kv_heads, cfg.head_dim), generator=g).to(cfg.torch_dtype)
    full = lambda v: torch.full((cfg.batch,), v, dtype=torch.int32)
    step_in = {"enc_bank": enc_bank, "enc_tok_off": synth.row_offsets(enc_lens, 1), "enc_pool": enc.pool,
               "rope_theta": cfg.rope_theta, "k": k, "q": synth.decode_queries(cfg, step=0, device="cpu"),
               "mem_kv": mem, "mem_len": full(mem_cap), "local_k": lk, "local_v": lv,
               "local_len": full(cfg.local_len), "pos": full(k)}
    r = bench.cpu_baseline(cfg, kr, pool_off, qr, 0.05, step_in)
    assert r["kind"] == "oracle" and r["cores"] == 1 and r["unit"] == "bank tokens/s"
    c = r["step_components_s"]
    assert set(c) == {"step_s", "scoring_s", "topk_s", "encode_batch_s", "decode_s"}
    assert all(v >= 0 for v in c.values())
    # the step time is the sum of its parts; the rate is the whole bank over it
    assert np.isclose(c["step_s"], c["scoring_s"] + c["topk_s"] + c["encode_batch_s"] + c["decode_s"], rtol=1e-3,
                      atol=1e-3)
    n_docs = len(pool_off) - 1
    assert np.isclose(r["value"], n_docs * 512 * cfg.batch / c["step_s"], rtol=2e-3)
    # the whole step is slower than its scoring alone
    assert r["value"] <= r["scoring_only_value"] * 1.001


def test_scan_traffic_record_is_current_and_guarded(tmp_path, monkeypatch):
    import json
    with open(bench.TRAFFIC_RECORD) as f:
        good = json.load(f)
    # the committed record is used exactly when it was taken on the current
    # scan sources, and then its bytes are close to the bank's
    rec = bench.measured_traffic(bench.SCAN_KERNEL)
    if good["source_sha256"] == bench.source_digest(bench.SCAN_SOURCES):
        assert rec is not None and 1.0 <= rec / 3_200_010_240 < 1.05
    else:
        assert rec is None
    # a record of other sources, or of another kernel, is not used
    stale = dict(good, source_sha256="0" * 64)
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(stale))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(path))
    assert bench.measured_traffic(bench.SCAN_KERNEL) is None
    path.write_text(json.dumps(good))
    assert bench.measured_traffic("some_other_kernel<1>") is None
    assert bench.measured_traffic(bench.SCAN_KERNEL) == good["hbm_bytes_per_launch"]
