"""Memory interleave: repeated route -> expand -> generate rounds, pipelined.

The method's memory interleaving runs rounds of routing over the bank,
appending the selected documents' pooled K/V to a query's memory, and
generating over the grown context ("EverMind Releases Memory-Sparse
Attention Code for Long-Context AI Models", section "Core Contributions";
the content tier is fetched from host memory when selected, "EverMind-AI/MSA:
Memory Sparse Attention for 100M-Token Contexts", section "How MSA compresses
and routes documents").  Each round's work is three library calls; here they
run on three streams so that the host link (assembly) and HBM (scoring,
decode) work at once:

  stream S   msa_route for round n (scan and top-k, no assembly)
  stream G   msa_assemble for round n (appending; from row 0 at a group's
             first round), then a copy of the memory lengths for round n
  stream D   msa_sparse_decode for round n over that copy

While the host link carries round n's documents, S scores round n + 1 and
D decodes round n - 1.  Round n + 1's scoring does not depend on round n
(its query is given); its assembly appends after round n's, in G's order.
Groups of rounds (one memory per group, reset at its first round) alternate
between two memory buffers, so a group's first assembly can overlap the
previous group's last decode.  Events order the streams: S refills a top-k
buffer after G has read it, G refills a length copy after D has read it and
a memory buffer after D's last decode of it.  Only scheduling lives here;
every step is a call into libmsa.
"""

import ctypes
import os

import torch

from . import _lib

_HIP_EVENT_DISABLE_TIMING = 0x2
_HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


class _Event:
    """A hipEvent_t for ordering streams of one device: no timing and no
    system-scope fence (a device-scope release is all another stream of the
    same device needs)."""

    _hip = None

    def __init__(self):
        if _Event._hip is None:
            hip = ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipStreamWaitEvent.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            _Event._hip = hip
        self.ev = ctypes.c_void_p()
        flags = _HIP_EVENT_DISABLE_TIMING | _HIP_EVENT_DISABLE_SYSTEM_FENCE
        if _Event._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), flags) != 0:
            raise RuntimeError("hipEventCreateWithFlags failed")

    def record(self, stream):
        if _Event._hip.hipEventRecord(self.ev, ctypes.c_void_p(stream.cuda_stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def wait(self, stream):
        """`stream` waits for this event's latest record."""
        if _Event._hip.hipStreamWaitEvent(ctypes.c_void_p(stream.cuda_stream), self.ev, 0) != 0:
            raise RuntimeError("hipStreamWaitEvent failed")

    def __del__(self):
        if self.ev and _Event._hip is not None:
            _Event._hip.hipEventDestroy(self.ev)


class InterleavePipeline:
    """Pipelined interleave rounds for a batch of queries over one bank.

    bank, doc_pool_off (device int64), route_kw: msa_route's router bank and
    its keywords (kr_layout, n_pool, doc_map); host_kv (pinned), host_off
    (CPU int64): the content tier; local_k/local_v/local_len: the queries'
    local context (device); mem_cap: memory rows per query.  Buffers are
    allocated once here; run() only enqueues library calls."""

    def __init__(self, bank, doc_pool_off, route_kw, host_kv, host_off, batch, top_k, mem_cap, local_k, local_v,
                 local_len, rope_theta, n_q_heads):
        dev = doc_pool_off.device
        self.bank, self.off, self.route_kw = bank, doc_pool_off, route_kw
        self.k, self.batch = top_k, batch
        self.local = (local_k, local_v, local_len)
        self.rope_theta = rope_theta
        n_docs = doc_pool_off.numel() - 1
        n_pool = route_kw.get("n_pool", bank.shape[0])
        hr, dr = bank.shape[1], bank.shape[2]
        hkv, d = host_kv.shape[2], host_kv.shape[3]
        self.S, self.G, self.D = torch.cuda.Stream(), torch.cuda.Stream(), torch.cuda.Stream()
        self.mems = [_lib.Assembly.allocate(host_kv, host_off, batch, top_k, mem_cap, dev) for _ in range(2)]
        self.tki = [torch.empty((batch, top_k), dtype=torch.int32, device=dev) for _ in range(2)]
        self.tks = torch.empty((batch, top_k), dtype=torch.float32, device=dev)
        self.dsc = torch.empty((batch, n_docs), dtype=torch.float32, device=dev)
        self.snap = [torch.empty(batch, dtype=torch.int32, device=dev) for _ in range(2)]
        self.rws = torch.empty(max(_lib.route_workspace_bytes(bank.dtype, batch, 1, hr, dr, n_docs, n_pool, top_k), 16),
                               dtype=torch.uint8, device=dev)
        self.aws = torch.empty(max(_lib.assemble_workspace_bytes(batch, top_k), 16), dtype=torch.uint8, device=dev)
        self.dws = torch.empty(max(_lib.decode_workspace_bytes(batch, n_q_heads, d, mem_cap, local_k.shape[1]), 16),
                               dtype=torch.uint8, device=dev)
        self.out = torch.empty((batch, n_q_heads, d), dtype=host_kv.dtype, device=dev)
        self.lse = torch.empty((batch, n_q_heads), dtype=torch.float32, device=dev)
        self.e_sel, self.e_asm, self.e_dec, self.e_free = ([_Event() for _ in range(2)] for _ in range(4))
        self.n = 0          # rounds enqueued so far (orders the buffer reuse)
        self.group = 0      # groups of rounds started so far

    def run(self, qrs, qs, pos, keep=None):
        """Enqueue one group of rounds: round r routes qrs[r] ([B, 1, Hr, dr]),
        appends its top-k documents to the group's memory (empty before the
        first round) and decodes qs[r] ([B, Hq, D]) with position offsets
        pos[r] (int32 device [B]).  keep: an optional list; each round's
        (decode output, memory lengths, top-k ids) are copied into new
        tensors on D and appended to it.  Returns the Assembly holding the
        group's memory (valid once the streams have drained)."""
        S, G, D = self.S, self.G, self.D
        g = self.group
        self.group += 1
        m = self.mems[g % 2]
        lk, lv, ll = self.local
        for r in range(len(qrs)):
            n = self.n
            self.n += 1
            j = n % 2
            if n >= 2:
                self.e_asm[j].wait(S)                  # G has read tki[j] (round n - 2)
            _lib.route(qrs[r], self.bank, self.off, self.k, self.dsc, self.tki[j], self.tks, self.rws, stream=S,
                       **self.route_kw)
            self.e_sel[j].record(S)
            self.e_sel[j].wait(G)
            if r == 0 and g >= 2:
                self.e_free[g % 2].wait(G)             # D is done with this memory buffer (group g - 2)
            if n >= 2:
                self.e_dec[j].wait(G)                  # D has read snap[j] (round n - 2)
            m.append = r > 0
            _lib.assemble(self.tki[j], self.off, m, workspace=self.aws, stream=G)
            with torch.cuda.stream(G):
                self.snap[j].copy_(m.mem_len)
                kept_idx = self.tki[j].clone() if keep is not None else None
            self.e_asm[j].record(G)
            self.e_asm[j].wait(D)
            _lib.sparse_decode(qs[r], m.mem_kv, self.snap[j], lk, lv, ll, pos[r], self.rope_theta, self.out, self.lse,
                               self.dws, stream=D)
            if keep is not None:
                with torch.cuda.stream(D):
                    keep.append((self.out.clone(), self.snap[j].clone(), kept_idx))
            self.e_dec[j].record(D)
            if r == len(qrs) - 1:
                self.e_free[g % 2].record(D)
        return m
