"""ctypes binding of libmsa (include/msa.h): argument marshalling only.

Every step of the hot path runs in the HIP library; this module turns torch
tensors into the C structs of msa.h, allocates outputs the caller did not
pass (PyTorch is the device-memory and stream provider), and raises
MSAError on a non-zero status.  If libmsa.so is missing it raises; there is
no other implementation to fall back to.
"""

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmsa.so")

MSA_OK, MSA_ERR_INVALID_ARG, MSA_ERR_UNSUPPORTED, MSA_ERR_WORKSPACE, MSA_ERR_CAPACITY, MSA_ERR_HIP = 0, -1, -2, -3, -4, -5
MSA_F32, MSA_BF16 = 0, 1
MSA_GATHER_COPIES, MSA_GATHER_KERNEL = 0, 1
MSA_KR_ROWS, MSA_KR_TILED = 0, 1
_KR_LAYOUT = {"rows": MSA_KR_ROWS, "tiled": MSA_KR_TILED}

_DTYPE = {torch.float32: MSA_F32, torch.bfloat16: MSA_BF16}

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64


class MSAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"libmsa status {status}: {message}")
        self.status = status


class PoolArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", I32), ("n_docs", I32), ("n_tokens", I64), ("n_pool", I64),
        ("pool_size", I32), ("n_kv_heads", I32), ("head_dim", I32), ("n_router_heads", I32),
        ("router_dim", I32), ("kr_layout", I32), ("rope_theta", ctypes.c_double),
        ("doc_tok_off", P), ("doc_pool_off", P), ("k", P), ("v", P), ("kr", P),
        ("kv_pooled", P), ("kr_pooled", P), ("kr_row_base", I64),
    ]


class RouteArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", I32), ("batch", I32), ("q_tokens", I32), ("n_router_heads", I32),
        ("router_dim", I32), ("top_k", I32), ("n_docs", I32), ("kr_layout", I32), ("n_pool", I64),
        ("qr", P), ("kr_pooled", P), ("doc_pool_off", P), ("doc_scores", P), ("topk_idx", P),
        ("topk_score", P), ("workspace", P), ("workspace_bytes", ctypes.c_size_t),
        ("host_kv", P), ("host_doc_pool_off", P), ("kv_dtype", I32), ("n_kv_heads", I32), ("head_dim", I32),
        ("mem_cap", I32), ("append", I32), ("gather_mode", I32), ("mem_kv", P), ("mem_len", P), ("host_topk_idx", P),
        ("host_mem_len", P), ("host_mem_docs", P), ("copy_stream", P),
        ("prof_event_begin", P), ("prof_event_end", P), ("doc_map", P),
    ]


class AssembleArgs(ctypes.Structure):
    _fields_ = [
        ("batch", I32), ("top_k", I32), ("n_docs", I32), ("kv_dtype", I32), ("n_pool", I64),
        ("topk_idx", P), ("doc_pool_off", P), ("host_kv", P), ("host_doc_pool_off", P),
        ("n_kv_heads", I32), ("head_dim", I32), ("mem_cap", I32), ("append", I32), ("gather_mode", I32),
        ("reserved0", I32), ("mem_kv", P), ("mem_len", P), ("host_topk_idx", P), ("host_mem_len", P),
        ("host_mem_docs", P), ("copy_stream", P), ("workspace", P), ("workspace_bytes", ctypes.c_size_t),
    ]


class DecodeArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", I32), ("batch", I32), ("n_q_heads", I32), ("n_kv_heads", I32), ("head_dim", I32),
        ("mem_cap", I32), ("local_cap", I32), ("reserved0", I32),
        ("q", P), ("mem_kv", P), ("mem_len", P), ("local_k", P), ("local_v", P), ("local_len", P),
        ("pos_offset", P), ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
        ("reserved1", I32), ("out", P), ("lse", P), ("workspace", P), ("workspace_bytes", ctypes.c_size_t),
        ("prof_event_begin", P), ("prof_event_end", P),
    ]


class AttendArgs(ctypes.Structure):
    _fields_ = [
        ("dtype", I32), ("batch", I32), ("q_tokens", I32), ("n_q_heads", I32), ("n_kv_heads", I32),
        ("head_dim", I32), ("mem_cap", I32), ("local_cap", I32),
        ("q", P), ("mem_kv", P), ("mem_len", P), ("local_k", P), ("local_v", P), ("local_len", P),
        ("pos_offset", P), ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
        ("reserved0", I32), ("out", P), ("lse", P), ("workspace", P), ("workspace_bytes", ctypes.c_size_t),
        ("prof_event_begin", P), ("prof_event_end", P),
    ]


EXPORTS = ("msa_pool_encode", "msa_route", "msa_route_workspace_bytes", "msa_assemble", "msa_assemble_workspace_bytes",
           "msa_doc_map_bytes", "msa_doc_map",
           "msa_sparse_decode", "msa_sparse_decode_noalloc",
           "msa_decode_workspace_bytes", "msa_sparse_attend", "msa_attend_workspace_bytes", "msa_last_error",
           "msa_version")

_lib = None


def load(path=None):
    """Load libmsa.so (after torch, so both share torch's HIP runtime)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"libmsa.so is not built ({p}); run `python -m sparse_latent_memory_amd.build` "
                           "or __graft_entry__.build()")
    lib = ctypes.CDLL(p)
    lib.msa_pool_encode.argtypes = [ctypes.POINTER(PoolArgs), P]
    lib.msa_pool_encode.restype = ctypes.c_int
    lib.msa_route.argtypes = [ctypes.POINTER(RouteArgs), P]
    lib.msa_route.restype = ctypes.c_int
    lib.msa_sparse_decode.argtypes = [ctypes.POINTER(DecodeArgs), P]
    lib.msa_sparse_decode.restype = ctypes.c_int
    lib.msa_sparse_decode_noalloc.argtypes = [ctypes.POINTER(DecodeArgs), P]
    lib.msa_sparse_decode_noalloc.restype = ctypes.c_int
    lib.msa_assemble.argtypes = [ctypes.POINTER(AssembleArgs), P]
    lib.msa_assemble.restype = ctypes.c_int
    lib.msa_assemble_workspace_bytes.argtypes = [I32, I32]
    lib.msa_assemble_workspace_bytes.restype = ctypes.c_size_t
    lib.msa_route_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I64, I32]
    lib.msa_route_workspace_bytes.restype = ctypes.c_size_t
    lib.msa_doc_map_bytes.argtypes = [I64]
    lib.msa_doc_map_bytes.restype = ctypes.c_size_t
    lib.msa_doc_map.argtypes = [P, I32, I64, P, ctypes.c_size_t, P]
    lib.msa_doc_map.restype = ctypes.c_int
    lib.msa_decode_workspace_bytes.argtypes = [I32, I32, I32, I32, I32]
    lib.msa_decode_workspace_bytes.restype = ctypes.c_size_t
    lib.msa_sparse_attend.argtypes = [ctypes.POINTER(AttendArgs), P]
    lib.msa_sparse_attend.restype = ctypes.c_int
    lib.msa_attend_workspace_bytes.argtypes = [I32, I32, I32, I32, I32, I32, I32]
    lib.msa_attend_workspace_bytes.restype = ctypes.c_size_t
    lib.msa_last_error.argtypes = []
    lib.msa_last_error.restype = ctypes.c_char_p
    lib.msa_version.argtypes = []
    lib.msa_version.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def _check(status):
    if status != MSA_OK:
        raise MSAError(status, load().msa_last_error().decode(errors="replace"))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dptr(t, name, pinned_ok=False):
    """Pointer to a dense device tensor (or, where the library allows it, a
    pinned CPU tensor); anything else is refused here, before it could reach
    a kernel as an address the GPU cannot map."""
    if t is None:
        return None
    if not (t.is_cuda or (pinned_ok and t.device.type == "cpu" and t.is_pinned())):
        raise ValueError(f"{name} must be a {'CUDA or pinned CPU' if pinned_ok else 'CUDA'} tensor, "
                         f"got one on {t.device}{' (not pinned)' if t.device.type == 'cpu' else ''}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _ptr(t)


def _hptr(t, name, pinned=False):
    """Pointer to a dense CPU tensor (pinned where the library maps it)."""
    if t is None:
        return None
    if t.device.type != "cpu" or (pinned and not t.is_pinned()):
        raise ValueError(f"{name} must be a {'pinned ' if pinned else ''}CPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return _ptr(t)


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def dtype_code(dtype):
    try:
        return _DTYPE[dtype]
    except KeyError:
        raise ValueError(f"unsupported dtype {dtype}; libmsa takes float32 or bfloat16") from None


# --------------------------------------------------------------------------
# stage 1
# --------------------------------------------------------------------------

def _layout_code(kr_layout):
    try:
        return _KR_LAYOUT[kr_layout]
    except KeyError:
        raise ValueError(f"kr_layout must be 'rows' or 'tiled', got {kr_layout!r}") from None


def bank_rows(n_rows, kr_layout="rows"):
    """Rows a router-bank buffer holds for n_rows rows: the tiled layout
    stores whole 16-row tiles."""
    return -(-n_rows // 16) * 16 if _layout_code(kr_layout) == MSA_KR_TILED else n_rows


def pool_encode(k, v, kr, doc_tok_off, doc_pool_off, pool_size, rope_theta, n_pool,
                kv_pooled=None, kr_pooled=None, stream=None, kr_layout="rows", kr_row_base=0):
    """msa_pool_encode.  k, v: [T, Hkv, D]; kr: [T, Hr, dr] (device, same
    dtype); offsets: int64 device [n_docs+1].  The outputs may be device
    tensors or pinned CPU tensors (written straight over the host link).
    kr_pooled is the router bank in `kr_layout` ("rows" or "tiled"); this
    call writes its rows kr_row_base .. kr_row_base + n_pool.  Returns
    (kv_pooled, kr_pooled)."""
    n_tok, hkv, d = k.shape
    _, hr, dr = kr.shape
    lay = _layout_code(kr_layout)
    if kv_pooled is None:
        kv_pooled = torch.empty((n_pool, 2, hkv, d), dtype=k.dtype, device=k.device)
    if kr_pooled is None:
        kr_pooled = torch.empty((bank_rows(kr_row_base + n_pool, kr_layout), hr, dr), dtype=k.dtype,
                                device=k.device)
    if kv_pooled.numel() < n_pool * 2 * hkv * d:
        raise ValueError(f"kv_pooled holds {kv_pooled.numel()} elements, {n_pool} rows need {n_pool * 2 * hkv * d}")
    need = bank_rows(kr_row_base + n_pool, kr_layout) * hr * dr
    if kr_pooled.numel() < need:
        raise ValueError(f"kr_pooled holds {kr_pooled.numel()} elements, rows up to {kr_row_base + n_pool} in the "
                         f"{kr_layout} layout need {need}")
    a = PoolArgs(dtype=dtype_code(k.dtype), n_docs=doc_tok_off.numel() - 1, n_tokens=n_tok, n_pool=n_pool,
                 pool_size=pool_size, n_kv_heads=hkv, head_dim=d, n_router_heads=hr, router_dim=dr,
                 rope_theta=float(rope_theta), doc_tok_off=_dptr(doc_tok_off, "doc_tok_off"),
                 doc_pool_off=_dptr(doc_pool_off, "doc_pool_off"), k=_dptr(k, "k"), v=_dptr(v, "v"),
                 kr=_dptr(kr, "kr"), kv_pooled=_dptr(kv_pooled, "kv_pooled", pinned_ok=True),
                 kr_pooled=_dptr(kr_pooled, "kr_pooled", pinned_ok=True), kr_layout=lay,
                 kr_row_base=kr_row_base)
    _check(load().msa_pool_encode(ctypes.byref(a), _stream(stream)))
    return kv_pooled, kr_pooled


# --------------------------------------------------------------------------
# stage 2
# --------------------------------------------------------------------------

def route_workspace_bytes(dtype, batch, q_tokens, n_router_heads, router_dim, n_docs, n_pool, top_k):
    return int(load().msa_route_workspace_bytes(dtype_code(dtype), batch, q_tokens, n_router_heads,
                                                router_dim, n_docs, n_pool, top_k))


class Assembly:
    """Buffers of the optional context-assembly part of msa_route.

    mode "kernel" (MSA_GATHER_KERNEL) or "copies" (MSA_GATHER_COPIES)."""

    def __init__(self, host_kv, host_doc_pool_off, mem_kv, mem_len, host_topk_idx, host_mem_len,
                 host_mem_docs=None, append=False, copy_stream=None, mode="kernel"):
        if mode not in ("kernel", "copies"):
            raise ValueError(f"assembly mode {mode!r}")
        self.mode = mode
        self.host_kv = host_kv
        self.host_doc_pool_off = host_doc_pool_off
        self.mem_kv = mem_kv
        self.mem_len = mem_len
        self.host_topk_idx = host_topk_idx
        self.host_mem_len = host_mem_len
        self.host_mem_docs = host_mem_docs
        self.append = append
        self.copy_stream = copy_stream

    @classmethod
    def allocate(cls, host_kv, host_doc_pool_off, batch, top_k, mem_cap, device, copy_stream=None,
                 mode="kernel"):
        _, two, hkv, d = host_kv.shape
        mem_kv = torch.zeros((batch, mem_cap, two, hkv, d), dtype=host_kv.dtype, device=device)
        return cls(host_kv, host_doc_pool_off, mem_kv, torch.zeros(batch, dtype=torch.int32, device=device),
                   torch.zeros((batch, top_k), dtype=torch.int32, pin_memory=True),
                   torch.zeros(batch, dtype=torch.int32, pin_memory=True),
                   torch.zeros(batch, dtype=torch.int32, pin_memory=True), copy_stream=copy_stream, mode=mode)


def _fill_assembly(a, asm, stream):
    """The assembly fields of RouteArgs / AssembleArgs from an Assembly.  The
    checked fields are kept on the Assembly and reused while its tensors
    (objects, addresses and shapes), mode and append flag stay the same: the
    checks cost a route call ~4 us of host time before its first launch."""
    key = (asm.mode, asm.append, id(asm.host_kv), asm.host_kv.data_ptr(), asm.host_kv.shape,
           id(asm.host_doc_pool_off), asm.host_doc_pool_off.data_ptr(), id(asm.mem_kv), asm.mem_kv.data_ptr(),
           asm.mem_kv.shape, id(asm.mem_len), asm.mem_len.data_ptr(), id(asm.host_topk_idx),
           id(asm.host_mem_len), id(asm.host_mem_docs))
    cached = getattr(asm, "_marshalled", None)
    if cached is None or cached[0] != key:
        f = type(a)()
        _check_assembly_fields(f, asm)
        cached = (key, {n: getattr(f, n) for n in _ASSEMBLY_FIELDS})
        asm._marshalled = cached
    for n, v in cached[1].items():
        setattr(a, n, v)
    cs = asm.copy_stream if asm.copy_stream is not None else stream
    a.copy_stream = _stream(cs)


_ASSEMBLY_FIELDS = ("host_kv", "host_doc_pool_off", "kv_dtype", "n_kv_heads", "head_dim", "mem_cap", "append",
                    "gather_mode", "mem_kv", "mem_len", "host_topk_idx", "host_mem_len", "host_mem_docs")


def _check_assembly_fields(a, asm):
    a.host_kv = _hptr(asm.host_kv, "host_kv", pinned=asm.mode == "kernel")
    a.host_doc_pool_off = _hptr(asm.host_doc_pool_off, "host_doc_pool_off")
    a.kv_dtype = dtype_code(asm.host_kv.dtype)
    a.n_kv_heads = asm.host_kv.shape[2]
    a.head_dim = asm.host_kv.shape[3]
    a.mem_cap = asm.mem_kv.shape[1]
    a.append = 1 if asm.append else 0
    a.gather_mode = MSA_GATHER_KERNEL if asm.mode == "kernel" else MSA_GATHER_COPIES
    a.mem_kv = _dptr(asm.mem_kv, "mem_kv")
    a.mem_len = _dptr(asm.mem_len, "mem_len")
    a.host_topk_idx = _hptr(asm.host_topk_idx, "host_topk_idx")
    a.host_mem_len = _hptr(asm.host_mem_len, "host_mem_len")
    a.host_mem_docs = _hptr(asm.host_mem_docs, "host_mem_docs")


def assemble_workspace_bytes(batch, top_k):
    return int(load().msa_assemble_workspace_bytes(batch, top_k))


def assemble(topk_idx, doc_pool_off, assembly, workspace=None, stream=None):
    """msa_assemble: copy the documents topk_idx [B, k] (int32 device, rank
    order) name into assembly.mem_kv, as msa_route's assembly does.
    doc_pool_off: int64 device [n_docs+1] (the kernel mode reads it there).
    Returns assembly.mem_len."""
    b, k = topk_idx.shape
    n_docs = doc_pool_off.numel() - 1
    a = AssembleArgs(batch=b, top_k=k, n_docs=n_docs, n_pool=assembly.host_kv.shape[0],
                     topk_idx=_dptr(topk_idx, "topk_idx"), doc_pool_off=_dptr(doc_pool_off, "doc_pool_off"))
    _fill_assembly(a, assembly, stream)
    if assembly.mode == "kernel":
        if workspace is None:
            workspace = torch.empty(max(assemble_workspace_bytes(b, k), 16), dtype=torch.uint8,
                                    device=topk_idx.device)
        a.workspace = _dptr(workspace, "workspace")
        a.workspace_bytes = workspace.numel()
    _check(load().msa_assemble(ctypes.byref(a), _stream(stream)))
    return assembly.mem_len


def _route_args(b, tq, hr, dr, q_dtype, dev, kr_pooled, doc_pool_off, top_k, doc_scores, topk_idx, topk_score,
                workspace, assembly, stream, kr_layout, n_pool, doc_map, qr=None):
    """RouteArgs (without the profiling events; without the query when qr is
    None), with the checks msa_route's pointers need: outputs and buffers
    the kernels write must hold what the call writes (checked first), then
    every pointer's placement, the query's first.  Returns (args,
    doc_scores, topk_idx, topk_score, workspace)."""
    lay = _layout_code(kr_layout)
    if n_pool is None:
        if lay == MSA_KR_TILED:
            raise ValueError("n_pool is required with the tiled layout")
        n_pool = kr_pooled.shape[0]
    if kr_pooled.numel() < bank_rows(n_pool, kr_layout) * hr * dr:
        raise ValueError(f"kr_pooled holds {kr_pooled.numel()} elements, {n_pool} rows in the {kr_layout} layout "
                         f"need {bank_rows(n_pool, kr_layout) * hr * dr}")
    n_docs = doc_pool_off.numel() - 1
    if doc_scores is None:
        doc_scores = torch.empty((b, n_docs), dtype=torch.float32, device=dev)
    if topk_idx is None:
        topk_idx = torch.empty((b, top_k), dtype=torch.int32, device=dev)
    if topk_score is None:
        topk_score = torch.empty((b, top_k), dtype=torch.float32, device=dev)
    for t, name, dt, n in ((doc_scores, "doc_scores", torch.float32, b * n_docs),
                           (topk_idx, "topk_idx", torch.int32, b * top_k),
                           (topk_score, "topk_score", torch.float32, b * top_k)):
        if t.dtype != dt or t.numel() < n:
            raise ValueError(f"{name} must be {dt} with at least {n} elements, got {t.dtype} with {t.numel()}")
    if workspace is None:
        nbytes = route_workspace_bytes(q_dtype, b, tq, hr, dr, n_docs, n_pool, top_k)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    a = RouteArgs(dtype=dtype_code(q_dtype), batch=b, q_tokens=tq, n_router_heads=hr, router_dim=dr,
                  top_k=top_k, n_docs=n_docs, n_pool=n_pool, qr=None if qr is None else _dptr(qr, "qr"),
                  kr_pooled=_dptr(kr_pooled, "kr_pooled"),
                  doc_pool_off=_dptr(doc_pool_off, "doc_pool_off"), doc_scores=_dptr(doc_scores, "doc_scores"),
                  topk_idx=_dptr(topk_idx, "topk_idx"), topk_score=_dptr(topk_score, "topk_score"),
                  workspace=_dptr(workspace, "workspace"),
                  workspace_bytes=workspace.numel() * workspace.element_size(), kr_layout=lay)
    if assembly is not None:
        _fill_assembly(a, assembly, stream)
    if doc_map is not None:
        if doc_map.numel() * doc_map.element_size() < doc_map_bytes(n_pool):
            raise ValueError(f"doc_map holds {doc_map.numel() * doc_map.element_size()} bytes, "
                             f"{doc_map_bytes(n_pool)} needed")
        a.doc_map = _dptr(doc_map, "doc_map")
    return a, doc_scores, topk_idx, topk_score, workspace


def route(qr, kr_pooled, doc_pool_off, top_k, doc_scores=None, topk_idx=None, topk_score=None,
          workspace=None, assembly=None, stream=None, prof_events=None, kr_layout="rows", n_pool=None,
          doc_map=None):
    """msa_route.  qr: [B, Tq, Hr, dr]; kr_pooled: the router bank in
    `kr_layout` ("rows": [n_pool, Hr, dr]; "tiled": whole 16-row tiles,
    n_pool given); doc_pool_off: int64 device [n_docs+1]; doc_map: optional,
    doc_map(doc_pool_off, n_pool)'s output for these offsets.  Returns
    (topk_idx, topk_score, doc_scores)."""
    b, tq, hr, dr = qr.shape
    a, doc_scores, topk_idx, topk_score, _ = _route_args(b, tq, hr, dr, qr.dtype, qr.device, kr_pooled,
                                                         doc_pool_off, top_k, doc_scores, topk_idx, topk_score,
                                                         workspace, assembly, stream, kr_layout, n_pool, doc_map,
                                                         qr=qr)
    if prof_events is not None:
        a.prof_event_begin, a.prof_event_end = prof_events
    _check(load().msa_route(ctypes.byref(a), _stream(stream)))
    return topk_idx, topk_score, doc_scores


class RouteCall:
    """msa_route with every argument but the query bound once, for serving
    loops whose bank, outputs, workspace, document map and assembly stay the
    same from call to call: route()'s checks and marshalling run here, once,
    and each call checks the query (shape, dtype, placement) and sets its
    pointer - about 1 us of host time before the first launch instead of
    ~7 us.  The bound tensors are kept alive; an Assembly is bound as it is
    at construction (tensors, mode, append flag).  Calls reuse one argument
    block: one thread at a time.  Calling it returns (topk_idx, topk_score,
    doc_scores)."""

    def __init__(self, q_shape, q_dtype, kr_pooled, doc_pool_off, top_k, doc_scores=None, topk_idx=None,
                 topk_score=None, workspace=None, assembly=None, kr_layout="rows", n_pool=None, doc_map=None):
        b, tq, hr, dr = q_shape
        dev = kr_pooled.device
        (self._a, self.doc_scores, self.topk_idx, self.topk_score,
         self.workspace) = _route_args(b, tq, hr, dr, q_dtype, dev, kr_pooled, doc_pool_off, top_k, doc_scores,
                                       topk_idx, topk_score, workspace, assembly, None, kr_layout, n_pool, doc_map)
        self._bound = (kr_pooled, doc_pool_off, doc_map, assembly)
        self._shape = (b, tq, hr, dr)
        self._dtype = q_dtype
        self._copy_stream = None if assembly is None else assembly.copy_stream
        self._assembly = assembly is not None
        self._fn = load().msa_route

    def __call__(self, qr, stream=None, prof_events=None):
        if tuple(qr.shape) != self._shape or qr.dtype != self._dtype:
            raise ValueError(f"qr must be {self._dtype} {list(self._shape)}, got {qr.dtype} {list(qr.shape)}")
        a = self._a
        a.qr = _dptr(qr, "qr")
        if self._assembly:
            a.copy_stream = _stream(self._copy_stream if self._copy_stream is not None else stream)
        a.prof_event_begin, a.prof_event_end = prof_events if prof_events is not None else (None, None)
        _check(self._fn(ctypes.byref(a), _stream(stream)))
        return self.topk_idx, self.topk_score, self.doc_scores


def doc_map_bytes(n_pool):
    return int(load().msa_doc_map_bytes(n_pool))


def doc_map(doc_pool_off, n_pool, out=None, stream=None):
    """msa_doc_map: the document map of a bank (doc_pool_off int64 device
    [n_docs+1]) into `out` (uint8 device, doc_map_bytes(n_pool) bytes), for
    route(..., doc_map=...).  Returns out."""
    n_docs = doc_pool_off.numel() - 1
    nbytes = doc_map_bytes(n_pool)
    if out is None:
        out = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=doc_pool_off.device)
    _check(load().msa_doc_map(_dptr(doc_pool_off, "doc_pool_off"), n_docs, n_pool, _dptr(out, "doc_map"),
                              out.numel() * out.element_size(), _stream(stream)))
    return out


# --------------------------------------------------------------------------
# stage 3
# --------------------------------------------------------------------------

def decode_workspace_bytes(batch, n_q_heads, head_dim, mem_cap, local_cap):
    return int(load().msa_decode_workspace_bytes(batch, n_q_heads, head_dim, mem_cap, local_cap))


def _decode_struct(q, mem_kv, mem_len, local_k, local_v, local_len, pos_offset, rope_theta, out, lse,
                   softmax_scale, want_lse, prof_events):
    b, hq, d = q.shape
    _, t_cap, hkv, _ = local_k.shape
    m_cap = 0 if mem_kv is None else mem_kv.shape[1]
    if out is None:
        out = torch.empty((b, hq, d), dtype=q.dtype, device=q.device)
    if lse is None and want_lse:
        lse = torch.empty((b, hq), dtype=torch.float32, device=q.device)
    a = DecodeArgs(dtype=dtype_code(q.dtype), batch=b, n_q_heads=hq, n_kv_heads=hkv, head_dim=d, mem_cap=m_cap,
                   local_cap=t_cap, q=_dptr(q, "q"), mem_kv=_dptr(mem_kv, "mem_kv"), mem_len=_dptr(mem_len, "mem_len"),
                   local_k=_dptr(local_k, "local_k"), local_v=_dptr(local_v, "local_v"),
                   local_len=_dptr(local_len, "local_len"), pos_offset=_dptr(pos_offset, "pos_offset"),
                   rope_theta=float(rope_theta), softmax_scale=float(softmax_scale), out=_dptr(out, "out"),
                   lse=_dptr(lse, "lse"))
    if prof_events is not None:
        a.prof_event_begin, a.prof_event_end = prof_events
    return a, out, lse


def sparse_decode(q, mem_kv, mem_len, local_k, local_v, local_len, pos_offset, rope_theta,
                  out=None, lse=None, workspace=None, softmax_scale=0.0, want_lse=True, stream=None,
                  prof_events=None):
    """msa_sparse_decode.  q: [B, Hq, D]; mem_kv: [B, M_cap, 2, Hkv, D] (or
    None); local_k/v: [B, T_cap, Hkv, D]; mem_len, local_len, pos_offset:
    int32 device [B].  Returns (out, lse)."""
    a, out, lse = _decode_struct(q, mem_kv, mem_len, local_k, local_v, local_len, pos_offset, rope_theta, out, lse,
                                 softmax_scale, want_lse, prof_events)
    if workspace is None:
        nbytes = decode_workspace_bytes(a.batch, a.n_q_heads, a.head_dim, a.mem_cap, a.local_cap)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=q.device)
    a.workspace = _dptr(workspace, "workspace")
    a.workspace_bytes = workspace.numel()
    _check(load().msa_sparse_decode(ctypes.byref(a), _stream(stream)))
    return out, lse


def sparse_decode_noalloc(q, mem_kv, mem_len, local_k, local_v, local_len, pos_offset, rope_theta, out, lse=None,
                          softmax_scale=0.0, stream=None):
    """msa_sparse_decode_noalloc: msa_sparse_decode with the library's static
    scratch in place of a workspace.  The caller passes every output (out,
    and lse or None), so nothing is allocated here either.  Returns
    (out, lse)."""
    a, out, lse = _decode_struct(q, mem_kv, mem_len, local_k, local_v, local_len, pos_offset, rope_theta, out, lse,
                                 softmax_scale, False, None)
    _check(load().msa_sparse_decode_noalloc(ctypes.byref(a), _stream(stream)))
    return out, lse


def attend_workspace_bytes(batch, q_tokens, n_q_heads, n_kv_heads, head_dim, mem_cap, local_cap):
    return int(load().msa_attend_workspace_bytes(batch, q_tokens, n_q_heads, n_kv_heads, head_dim, mem_cap,
                                                 local_cap))


def sparse_attend(q, mem_kv, mem_len, local_k, local_v, local_len, pos_offset, rope_theta,
                  out=None, lse=None, workspace=None, softmax_scale=0.0, want_lse=True, stream=None,
                  prof_events=None):
    """msa_sparse_attend.  q: [B, Tq, Hq, D], the last Tq local tokens of
    each query; mem_kv: [B, M_cap, 2, Hkv, D] (or None); local_k/v:
    [B, T_cap, Hkv, D]; mem_len, local_len, pos_offset: int32 device [B].
    Returns (out [B, Tq, Hq, D], lse [B, Tq, Hq])."""
    b, tq, hq, d = q.shape
    _, t_cap, hkv, _ = local_k.shape
    m_cap = 0 if mem_kv is None else mem_kv.shape[1]
    dev = q.device
    if out is None:
        out = torch.empty((b, tq, hq, d), dtype=q.dtype, device=dev)
    if lse is None and want_lse:
        lse = torch.empty((b, tq, hq), dtype=torch.float32, device=dev)
    if workspace is None:
        nbytes = attend_workspace_bytes(b, tq, hq, hkv, d, m_cap, t_cap)
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=dev)
    a = AttendArgs(dtype=dtype_code(q.dtype), batch=b, q_tokens=tq, n_q_heads=hq, n_kv_heads=hkv, head_dim=d,
                   mem_cap=m_cap, local_cap=t_cap, q=_dptr(q, "q"), mem_kv=_dptr(mem_kv, "mem_kv"),
                   mem_len=_dptr(mem_len, "mem_len"), local_k=_dptr(local_k, "local_k"),
                   local_v=_dptr(local_v, "local_v"), local_len=_dptr(local_len, "local_len"),
                   pos_offset=_dptr(pos_offset, "pos_offset"), rope_theta=float(rope_theta),
                   softmax_scale=float(softmax_scale), out=_dptr(out, "out"), lse=_dptr(lse, "lse"),
                   workspace=_dptr(workspace, "workspace"), workspace_bytes=workspace.numel())
    if prof_events is not None:
        a.prof_event_begin, a.prof_event_end = prof_events
    _check(load().msa_sparse_attend(ctypes.byref(a), _stream(stream)))
    return out, lse

