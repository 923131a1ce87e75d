"""Host-side checks of the C ABI: libmsa.so loads, exports every function
include/msa.h declares, the ctypes structs have the C layout, and invalid
arguments are rejected before anything touches a GPU."""

import ctypes
import os
import re
import shutil
import subprocess

import pytest
import torch  # noqa: F401  (load torch's HIP runtime before libmsa)

from sparse_latent_memory_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "msa.h")


def _declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(msa_[a-z_]+)\s*\(", text, re.M)))


def test_library_built_and_exports_every_declared_symbol():
    lib = _lib.load()
    declared = _declared_functions()
    assert set(declared) == set(_lib.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", _lib.LIB_PATH], capture_output=True, text=True).stdout
        exported = set(re.findall(r" T (msa_\w+)$", out, re.M))
        assert set(declared) <= exported


def test_read_reference_library_exports_its_declared_symbol_and_checks_arguments():
    """libmsa_readref.so (the streaming-read reference bench.py times beside
    the scan) exports what include/msa_readref.h declares and refuses bad
    arguments before any launch."""
    from sparse_latent_memory_amd import readref
    text = open(os.path.join(ROOT, "include", "msa_readref.h")).read()
    declared = set(re.findall(r"^\s*int\s+(msa_\w+)\s*\(", text, re.M))
    assert declared == set(readref.EXPORTS)
    lib = readref.load()
    for name in declared:
        assert hasattr(lib, name), name
    f = lib.msa_ref_read_tiles
    sink, buf = ctypes.c_void_p(256), ctypes.c_void_p(4096)   # never dereferenced: every call is refused
    assert f(None, 32768, 1, 1, sink, None, None, None) == -1
    assert f(buf, 32768, 1, 1, None, None, None, None) == -1
    assert f(buf, 32768 + 16, 1, 1, sink, None, None, None) == -1      # not whole tiles
    assert f(buf, 0, 1, 1, sink, None, None, None) == -1
    assert f(buf, 32768, 0, 1, sink, None, None, None) == -1           # empty grid
    assert f(ctypes.c_void_p(4100), 32768, 1, 1, sink, None, None, None) == -1   # misaligned


def test_doc_map_size_and_argument_checks():
    """msa_doc_map_bytes: n_tiles int32 then, 256-byte aligned, n_tiles
    uint32; msa_doc_map refuses NULL pointers, bad counts and a short or
    misaligned buffer before launching anything."""
    lib = _lib.load()
    assert lib.msa_doc_map_bytes(0) == 0
    assert lib.msa_doc_map_bytes(17) == 512                 # 2 tiles: 8 B -> 256, twice
    assert lib.msa_doc_map_bytes(16 * 64) == 512            # 64 tiles: 256 B each
    assert lib.msa_doc_map_bytes(16 * 65) == 1024
    off, buf = ctypes.c_void_p(4096), ctypes.c_void_p(8192)  # never dereferenced: every call is refused
    assert lib.msa_doc_map(None, 4, 100, buf, 4096, None) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_doc_map(off, 4, 100, None, 4096, None) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_doc_map(off, 0, 100, buf, 4096, None) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_doc_map(off, 101, 100, buf, 4096, None) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_doc_map(off, 4, 100, buf, 256, None) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_doc_map(off, 4, 100, ctypes.c_void_p(8200), 4096, None) == _lib.MSA_ERR_INVALID_ARG
    assert b"doc_map" in lib.msa_last_error()


def test_version():
    assert _lib.load().msa_version() == 100


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_ctypes_struct_layout_matches_c(tmp_path):
    structs = {"msa_pool_args": _lib.PoolArgs, "msa_route_args": _lib.RouteArgs,
               "msa_decode_args": _lib.DecodeArgs, "msa_attend_args": _lib.AttendArgs}
    lines = ['#include <stdio.h>', '#include <stddef.h>', f'#include "{HEADER}"', "int main(void) {"]
    for cname, cls in structs.items():
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for fname, _ in cls._fields_:
            lines.append(f'  printf("{cname} {fname} %zu\\n", offsetof({cname}, {fname}));')
    lines.append("  return 0; }")
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c11", "-Wall", "-Werror", str(src), "-o", str(exe)], check=True)
    got = {}
    for line in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.splitlines():
        s, f, v = line.split()
        got[(s, f)] = int(v)
    for cname, cls in structs.items():
        assert got[(cname, "size")] == ctypes.sizeof(cls), cname
        for fname, _ in cls._fields_:
            assert got[(cname, fname)] == getattr(cls, fname).offset, (cname, fname)


def test_workspace_size_functions():
    lib = _lib.load()
    # one token per query: per-document parts (a stride of 4 queries) and per-tile continuations
    assert lib.msa_route_workspace_bytes(1, 1, 1, 8, 128, 195313, 1562504, 16) >= 16 * 195313 + 16 * 97657
    # several tokens: one score per bank row and query
    assert lib.msa_route_workspace_bytes(1, 1, 2, 8, 128, 195313, 1562504, 16) >= 4 * 1562504
    assert lib.msa_route_workspace_bytes(1, 0, 1, 8, 128, 10, 10, 1) == 0          # batch 0
    assert lib.msa_route_workspace_bytes(7, 1, 1, 8, 128, 10, 10, 1) == 0          # bad dtype
    assert lib.msa_route_workspace_bytes(1, 1, 1, 8, 128, 10, 9, 1) == 0           # n_pool < n_docs
    assert lib.msa_decode_workspace_bytes(1, 32, 128, 128, 4096) > 0
    assert lib.msa_decode_workspace_bytes(1, 32, 96, 128, 4096) == 0               # head_dim 96
    assert lib.msa_decode_workspace_bytes(1, 32, 128, -1, 4096) == 0


# --------------------------------------------------------------------------
# error paths: every call below must fail validation, before any HIP call.
# They pass host addresses, so they only run where no GPU is visible.
# --------------------------------------------------------------------------
no_gpu = pytest.mark.skipif(torch.cuda.device_count() > 0,
                            reason="error-path calls pass host pointers; run them without a GPU")

_buf = ctypes.create_string_buffer(1 << 16)
_B = ctypes.addressof(_buf) + (-ctypes.addressof(_buf) % 256)   # 256-byte aligned host address


def _p(off=0):
    return ctypes.c_void_p(_B + off)


def _pool_args(**kw):
    a = _lib.PoolArgs(dtype=1, n_docs=2, n_tokens=100, n_pool=4, pool_size=64, n_kv_heads=8, head_dim=128,
                      n_router_heads=8, router_dim=128, rope_theta=1e6, doc_tok_off=_p(), doc_pool_off=_p(),
                      k=_p(), v=_p(), kr=_p(), kv_pooled=_p(), kr_pooled=_p())
    for k, v in kw.items():
        setattr(a, k, v)
    return a


def _call_pool(a):
    lib = _lib.load()
    return lib.msa_pool_encode(ctypes.byref(a), None), lib.msa_last_error().decode()


@no_gpu
@pytest.mark.parametrize("field,value,code", [
    ("dtype", 5, _lib.MSA_ERR_INVALID_ARG),
    ("n_docs", 0, _lib.MSA_ERR_INVALID_ARG),
    ("pool_size", 0, _lib.MSA_ERR_INVALID_ARG),
    ("head_dim", 96, _lib.MSA_ERR_UNSUPPORTED),
    ("router_dim", 256, _lib.MSA_ERR_UNSUPPORTED),
    ("rope_theta", 0.0, _lib.MSA_ERR_INVALID_ARG),
    ("n_pool", 1000, _lib.MSA_ERR_INVALID_ARG),
    ("k", None, _lib.MSA_ERR_INVALID_ARG),
    ("kv_pooled", ctypes.c_void_p(_B + 8), _lib.MSA_ERR_INVALID_ARG),   # misaligned
    ("kr_layout", 2, _lib.MSA_ERR_INVALID_ARG),
    ("kr_row_base", -1, _lib.MSA_ERR_INVALID_ARG),
])
def test_pool_rejects_bad_arguments(field, value, code):
    status, msg = _call_pool(_pool_args(**{field: value}))
    assert status == code, msg
    assert msg.startswith("msa_pool_encode")


@no_gpu
def test_tiled_router_bank_needs_bf16_and_a_matrix_core_shape():
    status, msg = _call_pool(_pool_args(dtype=0, kr_layout=_lib.MSA_KR_TILED))
    assert status == _lib.MSA_ERR_UNSUPPORTED and "bf16" in msg
    lib = _lib.load()
    for kw in ({"dtype": 0}, {"n_router_heads": 16, "router_dim": 128}, {"n_router_heads": 32, "router_dim": 64}):
        a = _route_args(kr_layout=_lib.MSA_KR_TILED, **kw)
        assert lib.msa_route(ctypes.byref(a), None) == _lib.MSA_ERR_UNSUPPORTED, lib.msa_last_error()
        assert b"tiled" in lib.msa_last_error()
    a = _route_args(kr_layout=2)
    assert lib.msa_route(ctypes.byref(a), None) == _lib.MSA_ERR_INVALID_ARG


@no_gpu
def test_binding_checks_router_bank_sizes():
    """An undersized bank buffer is refused by the binding before any call
    (the library cannot see a raw pointer's extent)."""
    import sparse_latent_memory_amd as msa
    bf = torch.bfloat16
    qr = torch.zeros(1, 1, 8, 128, dtype=bf)
    off = torch.tensor([0, 20], dtype=torch.int64)
    with pytest.raises(ValueError, match="n_pool is required"):
        msa.route(qr, torch.zeros(32, 8, 128, dtype=bf), off, 1, kr_layout="tiled")
    with pytest.raises(ValueError, match="need"):
        msa.route(qr, torch.zeros(20, 8, 128, dtype=bf), off, 1, kr_layout="tiled", n_pool=20)
    with pytest.raises(ValueError, match="kr_layout must be"):
        msa.route(qr, torch.zeros(20, 8, 128, dtype=bf), off, 1, kr_layout="cols")
    k = torch.zeros(100, 8, 128, dtype=bf)
    with pytest.raises(ValueError, match="kr_pooled holds"):
        msa.pool_encode(k, k, k, off, off, 64, 1e6, 2, kr_pooled=torch.zeros(16, 8, 128, dtype=bf),
                        kr_layout="tiled", kr_row_base=15)


@no_gpu
def test_null_args_rejected():
    lib = _lib.load()
    assert lib.msa_pool_encode(None, None) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_route(None, None) == _lib.MSA_ERR_INVALID_ARG
    assert lib.msa_sparse_decode(None, None) == _lib.MSA_ERR_INVALID_ARG
    assert b"NULL" in lib.msa_last_error()


def _route_args(**kw):
    a = _lib.RouteArgs(dtype=1, batch=1, q_tokens=1, n_router_heads=8, router_dim=128, top_k=4, n_docs=10,
                       n_pool=20, qr=_p(), kr_pooled=_p(), doc_pool_off=_p(), doc_scores=_p(), topk_idx=_p(),
                       topk_score=_p(), workspace=_p(), workspace_bytes=16)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@no_gpu
@pytest.mark.parametrize("kw,code", [
    ({"top_k": 11}, _lib.MSA_ERR_INVALID_ARG),                  # k > n_docs
    ({"top_k": 0}, _lib.MSA_ERR_INVALID_ARG),
    ({"n_docs": 5000, "n_pool": 6000, "top_k": 4097}, _lib.MSA_ERR_UNSUPPORTED),
    ({"router_dim": 96}, _lib.MSA_ERR_UNSUPPORTED),
    ({"n_router_heads": 3}, _lib.MSA_ERR_UNSUPPORTED),
    ({"n_pool": 5}, _lib.MSA_ERR_INVALID_ARG),                  # fewer rows than documents
    ({"qr": None}, _lib.MSA_ERR_INVALID_ARG),
    ({}, _lib.MSA_ERR_WORKSPACE),                               # 16 bytes is too small
    ({"workspace": None}, _lib.MSA_ERR_WORKSPACE),
])
def test_route_rejects_bad_arguments(kw, code):
    lib = _lib.load()
    a = _route_args(**kw)
    assert lib.msa_route(ctypes.byref(a), None) == code, lib.msa_last_error()


@no_gpu
def test_route_assembly_arguments_checked_before_launch():
    lib = _lib.load()
    need = lib.msa_route_workspace_bytes(1, 1, 1, 8, 128, 10, 20, 4)
    assert need < len(_buf) - 256
    a = _route_args(workspace_bytes=need, host_kv=_p())          # assembly without its buffers
    assert lib.msa_route(ctypes.byref(a), None) == _lib.MSA_ERR_INVALID_ARG
    assert b"assembly" in lib.msa_last_error()
    lens = (ctypes.c_int32 * 1)(99)
    a = _route_args(workspace_bytes=need, host_kv=_p(), host_doc_pool_off=_p(), mem_kv=_p(), mem_len=_p(),
                    host_topk_idx=_p(), host_mem_len=ctypes.cast(lens, ctypes.c_void_p), kv_dtype=1,
                    n_kv_heads=8, head_dim=128, mem_cap=10, append=1)
    assert lib.msa_route(ctypes.byref(a), None) == _lib.MSA_ERR_INVALID_ARG   # 99 > mem_cap
    assert b"host_mem_len" in lib.msa_last_error()
    a.kv_dtype = 9
    assert lib.msa_route(ctypes.byref(a), None) == _lib.MSA_ERR_INVALID_ARG
    assert b"kv_dtype" in lib.msa_last_error()


def _assemble_args(**kw):
    a = _lib.AssembleArgs(batch=1, top_k=4, n_docs=10, kv_dtype=1, n_pool=20, topk_idx=_p(), doc_pool_off=_p(),
                          host_kv=_p(), host_doc_pool_off=_p(), n_kv_heads=8, head_dim=128, mem_cap=10, append=0,
                          gather_mode=_lib.MSA_GATHER_COPIES, mem_kv=_p(), mem_len=_p(), host_topk_idx=_p(),
                          host_mem_len=_p(), workspace=_p(), workspace_bytes=16)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@no_gpu
@pytest.mark.parametrize("kw,code,msg", [
    ({"batch": 0}, _lib.MSA_ERR_INVALID_ARG, b"batch"),
    ({"topk_idx": None}, _lib.MSA_ERR_INVALID_ARG, b"topk_idx"),
    ({"top_k": 11}, _lib.MSA_ERR_INVALID_ARG, b"top_k"),           # more than n_docs
    ({"n_pool": 9}, _lib.MSA_ERR_INVALID_ARG, b"n_pool"),
    ({"gather_mode": 7}, _lib.MSA_ERR_INVALID_ARG, b"gather_mode"),
    ({"mem_kv": None}, _lib.MSA_ERR_INVALID_ARG, b"assembly needs"),
    ({"host_topk_idx": None}, _lib.MSA_ERR_INVALID_ARG, b"copy assembly"),
    ({"kv_dtype": 3}, _lib.MSA_ERR_INVALID_ARG, b"kv_dtype"),
    ({"mem_cap": -1}, _lib.MSA_ERR_INVALID_ARG, b"mem_cap"),
    ({"gather_mode": _lib.MSA_GATHER_KERNEL}, _lib.MSA_ERR_INVALID_ARG, b"device-mapped"),   # plain host address
])
def test_assemble_rejects_bad_arguments(kw, code, msg):
    lib = _lib.load()
    a = _assemble_args(**kw)
    assert lib.msa_assemble(ctypes.byref(a), None) == code, lib.msa_last_error()
    assert msg in lib.msa_last_error()
    assert lib.msa_assemble(None, None) == _lib.MSA_ERR_INVALID_ARG


@no_gpu
def test_assemble_checks_appended_lengths_and_sizes_its_workspace():
    lib = _lib.load()
    lens = (ctypes.c_int32 * 1)(11)
    a = _assemble_args(append=1, host_mem_len=ctypes.cast(lens, ctypes.c_void_p))
    assert lib.msa_assemble(ctypes.byref(a), None) == _lib.MSA_ERR_INVALID_ARG     # 11 > mem_cap
    assert b"host_mem_len" in lib.msa_last_error()
    assert lib.msa_assemble_workspace_bytes(64, 8) >= 64 * 8 * 16               # one 16-byte plan entry per rank
    assert lib.msa_assemble_workspace_bytes(0, 8) == 0


def _decode_args(**kw):
    a = _lib.DecodeArgs(dtype=1, batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, mem_cap=128, local_cap=64,
                        q=_p(), mem_kv=_p(), mem_len=_p(), local_k=_p(), local_v=_p(), local_len=_p(),
                        pos_offset=_p(), rope_theta=1e6, softmax_scale=0.0, out=_p(), lse=None, workspace=_p(),
                        workspace_bytes=16)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@no_gpu
@pytest.mark.parametrize("kw,code", [
    ({"n_q_heads": 30}, _lib.MSA_ERR_INVALID_ARG),              # not a multiple of Hkv
    ({"n_q_heads": 72}, _lib.MSA_ERR_UNSUPPORTED),              # 9 query heads per KV head
    ({"head_dim": 80}, _lib.MSA_ERR_UNSUPPORTED),
    ({"mem_kv": None}, _lib.MSA_ERR_INVALID_ARG),               # mem_cap > 0 needs memory
    ({"local_v": None}, _lib.MSA_ERR_INVALID_ARG),
    ({"rope_theta": -1.0}, _lib.MSA_ERR_INVALID_ARG),
    ({"local_k": ctypes.c_void_p(_B + 4)}, _lib.MSA_ERR_INVALID_ARG),
    ({"q": ctypes.c_void_p(_B + 8)}, _lib.MSA_ERR_INVALID_ARG),   # bf16 query not 16-byte aligned
    ({"out": ctypes.c_void_p(_B + 2)}, _lib.MSA_ERR_INVALID_ARG),  # bf16 output not 16-byte aligned
    ({"dtype": 0, "q": ctypes.c_void_p(_B + 4)}, _lib.MSA_ERR_WORKSPACE),   # fp32 takes any 4-byte alignment
    ({}, _lib.MSA_ERR_WORKSPACE),
])
def test_decode_rejects_bad_arguments(kw, code):
    lib = _lib.load()
    a = _decode_args(**kw)
    assert lib.msa_sparse_decode(ctypes.byref(a), None) == code, lib.msa_last_error()


@no_gpu
def test_decode_noalloc_refuses_partials_beyond_its_static_scratch():
    """msa_sparse_decode_noalloc keeps the split partials in a 64 MiB static
    array: sizes that need more are refused before any launch (128 queries
    of 32 heads over 16,384 keys need 65 MiB), and the caller's workspace
    fields are ignored rather than used."""
    lib = _lib.load()
    assert lib.msa_decode_workspace_bytes(128, 32, 128, 12288, 4096) > (64 << 20)
    a = _decode_args(batch=128, mem_cap=12288, local_cap=4096, workspace=None, workspace_bytes=0)
    assert lib.msa_sparse_decode_noalloc(ctypes.byref(a), None) == _lib.MSA_ERR_WORKSPACE
    assert b"static scratch" in lib.msa_last_error()
    a = _decode_args(batch=128, mem_cap=12288, local_cap=4096, workspace=_p(), workspace_bytes=1 << 40)
    assert lib.msa_sparse_decode_noalloc(ctypes.byref(a), None) == _lib.MSA_ERR_WORKSPACE
    a = _decode_args(n_q_heads=30)
    assert lib.msa_sparse_decode_noalloc(ctypes.byref(a), None) == _lib.MSA_ERR_INVALID_ARG
    assert b"msa_sparse_decode_noalloc" in lib.msa_last_error()


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load(str(tmp_path / "missing" / "libmsa.so"))


def _attend_args(**kw):
    a = _lib.AttendArgs(dtype=1, batch=1, q_tokens=4, n_q_heads=32, n_kv_heads=8, head_dim=128, mem_cap=128,
                        local_cap=64, q=_p(), mem_kv=_p(), mem_len=_p(), local_k=_p(), local_v=_p(), local_len=_p(),
                        pos_offset=_p(), rope_theta=1e6, softmax_scale=0.0, out=_p(), lse=None, workspace=_p(),
                        workspace_bytes=16)
    for k, v in kw.items():
        setattr(a, k, v)
    return a


@no_gpu
@pytest.mark.parametrize("kw,code", [
    ({"dtype": 0}, _lib.MSA_ERR_UNSUPPORTED),                   # fp32: bf16 only
    ({"dtype": 5}, _lib.MSA_ERR_INVALID_ARG),
    ({"q_tokens": 0}, _lib.MSA_ERR_INVALID_ARG),
    ({"n_q_heads": 30}, _lib.MSA_ERR_INVALID_ARG),              # not a multiple of Hkv
    ({"n_q_heads": 136}, _lib.MSA_ERR_UNSUPPORTED),             # 17 query heads per KV head
    ({"head_dim": 80}, _lib.MSA_ERR_UNSUPPORTED),
    ({"mem_kv": None}, _lib.MSA_ERR_INVALID_ARG),               # mem_cap > 0 needs memory
    ({"local_k": None}, _lib.MSA_ERR_INVALID_ARG),
    ({"rope_theta": 0.0}, _lib.MSA_ERR_INVALID_ARG),
    ({"q": ctypes.c_void_p(_B + 8)}, _lib.MSA_ERR_INVALID_ARG),  # misaligned query
    ({}, _lib.MSA_ERR_WORKSPACE),
])
def test_attend_rejects_bad_arguments(kw, code):
    lib = _lib.load()
    a = _attend_args(**kw)
    assert lib.msa_sparse_attend(ctypes.byref(a), None) == code, lib.msa_last_error()


def test_attend_workspace_size():
    lib = _lib.load()
    assert lib.msa_attend_workspace_bytes(1, 256, 32, 8, 128, 256, 2048) > 0
    assert lib.msa_attend_workspace_bytes(64, 1, 32, 8, 128, 12288, 4096) > 0
    assert lib.msa_attend_workspace_bytes(1, 0, 32, 8, 128, 256, 2048) == 0      # no tokens
    assert lib.msa_attend_workspace_bytes(1, 4, 34, 8, 128, 256, 2048) == 0      # Hq not a multiple of Hkv
    assert lib.msa_attend_workspace_bytes(1, 4, 32, 8, 96, 256, 2048) == 0       # head dim



def test_binding_checks_route_output_sizes():
    """Route outputs that cannot hold what the call writes (B x n_docs scores,
    B x k ids and scores) are refused by the binding before any call: the
    library sees only their addresses."""
    import sparse_latent_memory_amd as msa
    bf = torch.bfloat16
    qr = torch.zeros(2, 1, 8, 128, dtype=bf)
    kr = torch.zeros(20, 8, 128, dtype=bf)
    off = torch.tensor([0, 5, 20], dtype=torch.int64)
    with pytest.raises(ValueError, match="doc_scores must be torch.float32 with at least 4"):
        msa.route(qr, kr, off, 1, doc_scores=torch.zeros(3))
    with pytest.raises(ValueError, match="doc_scores must be torch.float32"):
        msa.route(qr, kr, off, 1, doc_scores=torch.zeros(4, dtype=torch.float64))
    with pytest.raises(ValueError, match="topk_idx must be torch.int32 with at least 4"):
        msa.route(qr, kr, off, 2, topk_idx=torch.zeros(2, 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="topk_score must be torch.float32 with at least 2"):
        msa.route(qr, kr, off, 1, topk_score=torch.zeros(1))


def test_binding_refuses_host_tensors_for_device_arguments():
    """A CPU tensor passed where the library takes device memory is refused
    by the binding before any call, with the argument named; pooled outputs
    may be pinned CPU tensors, but not pageable ones."""
    import sparse_latent_memory_amd as msa
    f, i32, i64 = torch.float32, torch.int32, torch.int64
    k = torch.zeros(8, 1, 64, dtype=f)
    off = torch.tensor([0, 8], dtype=i64)
    with pytest.raises(ValueError, match="doc_tok_off must be a CUDA"):
        msa.pool_encode(k, k, k, off, torch.tensor([0, 1], dtype=i64), 8, 1e4, 1)
    with pytest.raises(ValueError, match="qr must be a CUDA"):
        msa.route(torch.zeros(1, 1, 1, 64, dtype=f), k, off, 1)
    lens = torch.ones(1, dtype=i32)
    with pytest.raises(ValueError, match="q must be a CUDA"):
        msa.sparse_decode(torch.zeros(1, 1, 64, dtype=f), None, None, torch.zeros(1, 4, 1, 64, dtype=f),
                          torch.zeros(1, 4, 1, 64, dtype=f), lens, lens, 1e4)
    with pytest.raises(ValueError, match="q must be a CUDA"):
        msa.sparse_attend(torch.zeros(1, 1, 1, 64, dtype=torch.bfloat16), None, None,
                          torch.zeros(1, 4, 1, 64, dtype=torch.bfloat16), torch.zeros(1, 4, 1, 64,
                          dtype=torch.bfloat16), lens, lens, 1e4)
    with pytest.raises(ValueError, match="must be contiguous"):
        _lib._hptr(torch.zeros(4, 4).t(), "x")
    with pytest.raises(ValueError, match="not pinned"):
        _lib._dptr(torch.zeros(4), "kv_pooled", pinned_ok=True)
    with pytest.raises(ValueError, match="pinned CPU tensor"):
        _lib._hptr(torch.zeros(4), "host_kv", pinned=True)
    assert _lib._hptr(torch.zeros(4), "host_doc_pool_off") is not None


def test_tiled_bank_helpers_follow_the_declared_layout():
    """synth.tile_router_bank puts element e of row j at
    16*E*(j/16) + 8*(16*(e/8) + j%16) + e%8, as msa.h declares for
    MSA_KR_TILED, and untile_router_bank inverts it."""
    from sparse_latent_memory_amd import synth
    for n, hr, dr in [(37, 2, 64), (16, 8, 128), (1, 1, 64)]:
        e_row = hr * dr
        ids = (torch.arange(n * e_row, dtype=torch.int32) % 30011).to(torch.int16)
        bank = ids.view(n, hr, dr).view(torch.bfloat16)
        flat = synth.tile_router_bank(bank, pad_value=-1.0).view(torch.int16).view(-1)
        assert flat.numel() == -(-n // 16) * 16 * e_row
        j = torch.arange(n).view(n, 1)
        e = torch.arange(e_row).view(1, e_row)
        off = 16 * e_row * (j // 16) + 8 * (16 * (e // 8) + j % 16) + e % 8
        assert torch.equal(flat[off.reshape(-1)], ids)
        back = synth.untile_router_bank(synth.tile_router_bank(bank), n)
        assert torch.equal(back.view(torch.int16), bank.view(torch.int16))
    assert msa_bank_rows(37) == (37, 48)


def msa_bank_rows(n):
    import sparse_latent_memory_amd as msa
    return msa.bank_rows(n, "rows"), msa.bank_rows(n, "tiled")
