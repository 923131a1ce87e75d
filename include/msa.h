/*
 * msa.h - C ABI of libmsa, the MI355X (gfx950) hot path of Memory Sparse
 * Attention (MSA).
 *
 * The three calls follow the method's three inference stages as described
 * in "EverMind Releases Memory-Sparse Attention Code for Long-Context AI
 * Models" (toolmesh.ai), section "Architectural Design and Inference", and
 * in "EverMind-AI/MSA: Memory Sparse Attention for 100M-Token Contexts"
 * (hysenlabs.com), section "How MSA compresses and routes documents":
 *
 *   msa_pool_encode   - offline memory encoding: chunk-mean pooling of each
 *                       document's K / V / Kr, positions restarting per doc.
 *   msa_route         - online routing and context assembly: cosine scores
 *                       of the projected query Qr against the pooled router
 *                       keys, mean over heads, max over tokens, max per
 *                       document, top-k; optionally copies the selected
 *                       documents' pooled K/V from pinned host memory.
 *   msa_sparse_decode - sparse generation: one attention step over the
 *                       assembled memory followed by the query's local K/V,
 *                       with the query position offset by k.
 *   msa_sparse_attend - the same for a block of query tokens (prefill
 *                       through the sparse context), causal over the local
 *                       tokens.
 *
 * Conventions shared by every call
 * --------------------------------
 * - Ownership: the caller owns every buffer (device memory, pinned host
 *   memory from hipHostMalloc, workspaces).  The library allocates and
 *   frees no memory.  Its only internal objects are per-thread HIP events.
 * - Pointers marked "device" are device memory on the current HIP device;
 *   "pinned host" pointers come from hipHostMalloc (or an equivalent pinned
 *   allocation); "host" pointers are ordinary host memory.
 * - Streams are hipStream_t values passed as void*; NULL is the default
 *   stream.  Every call enqueues its work on `stream` and returns without
 *   waiting, except msa_route with assembly (see there).
 * - Dense row-major layouts; shapes are given outermost first.  Element
 *   type of the float tensors is `dtype` (MSA_F32 or MSA_BF16); offsets are
 *   int64, lengths and indices int32, scores fp32.
 * - Errors: every argument is checked before anything is enqueued; a
 *   non-zero return means nothing was enqueued (MSA_ERR_CAPACITY in
 *   msa_route is the one documented exception).  Device-resident values
 *   (offsets, lengths) cannot be checked on the host: kernels clamp every
 *   index derived from them into the buffers they are given, so a bad value
 *   yields wrong numbers, never an out-of-bounds access.  msa_last_error()
 *   returns a thread-local message for the last non-OK return.  No C++
 *   exception crosses the ABI.  Calls are re-entrant across threads.
 * - Supported shapes: head_dim and router_dim in {64, 128}; n_q_heads a
 *   multiple of n_kv_heads; 1 <= top_k <= min(n_docs, 4096).
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MSA_OK = 0,
  MSA_ERR_INVALID_ARG = -1, /* null pointer, bad size, inconsistent shape  */
  MSA_ERR_UNSUPPORTED = -2, /* valid but not implemented (head_dim, top_k)  */
  MSA_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required  */
  MSA_ERR_CAPACITY = -4,    /* reserved; assembly drops what does not fit  */
  MSA_ERR_HIP = -5          /* a HIP runtime call or kernel launch failed  */
} msa_status;

typedef enum { MSA_F32 = 0, MSA_BF16 = 1 } msa_dtype;

/* ------------------------------------------------------------------------
 * Layouts of the pooled router-key bank Kr_bar (E = Hr * dr elements a row).
 *
 *  MSA_KR_ROWS (0): row-major [n_pool, Hr, dr]; the buffer holds n_pool rows.
 *  MSA_KR_TILED (1), bf16 only: rows are grouped in tiles of 16 and a tile
 *    stores its rows' 16-byte pieces piece-major: element e of row j is at
 *    element offset 16*E*(j/16) + 8*(16*(e/8) + j%16) + e%8.  The buffer
 *    holds ceil(rows/16) whole tiles (16 * E * 2 bytes each); the padding
 *    rows of the last tile are never written by msa_pool_encode and never
 *    reach a score in msa_route, whatever they hold.  In this order every
 *    matrix-core operand load of the scan reads 1 KiB of contiguous memory.
 *    The layout is a storage order of this library, not of the method: the
 *    scores are identical, bit for bit, to those of the row-major bank.
 * ------------------------------------------------------------------------ */
typedef enum { MSA_KR_ROWS = 0, MSA_KR_TILED = 1 } msa_kr_layout;

/* ------------------------------------------------------------------------
 * Stage 1 - offline memory encoding.
 *
 * For document d with L_d = doc_tok_off[d+1] - doc_tok_off[d] tokens and
 * chunk c covering its tokens [c*P, min((c+1)*P, L_d)) (n_c tokens):
 *   K_bar = mean over the chunk of RoPE(K_t, t - doc_tok_off[d])
 *   V_bar = mean of V_t,   Kr_bar = mean of Kr_t
 * written to pooled row doc_pool_off[d] + c.  RoPE is the rotate-half form:
 * pair (j, j + D/2) of a head is rotated by angle p * theta^(-2j/D).
 * Positions restart at zero in every document (document-wise RoPE, same
 * sources as above; "Key Technical Details" of "MSA (Memory Sparse
 * Attention) - An Open-Source Answer to AI's Memory Bottleneck").
 * Only K is rotated; V and Kr are averaged as given.  Accumulation is fp32,
 * the result is rounded to nearest-even into `dtype`.  Kr_bar of pooled row
 * j goes to bank row kr_row_base + j of kr_pooled, stored in kr_layout
 * (MSA_KR_TILED needs bf16); kv_pooled is always row-major, row j.
 * Either output may be pinned host memory (hipHostMalloc, or torch's
 * pin_memory) instead of device memory: the kernel then writes the pooled
 * rows through the buffer's device mapping, straight over the host link -
 * this is how a large bank streams its pooled K/V into the host-resident
 * content tier while the next batch is encoded.  Pageable host memory and
 * another device's memory are rejected (MSA_ERR_INVALID_ARG) before any
 * launch.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t dtype;            /* msa_dtype of k, v, kr and both outputs       */
  int32_t n_docs;           /* >= 1                                         */
  int64_t n_tokens;         /* = doc_tok_off[n_docs]                        */
  int64_t n_pool;           /* = doc_pool_off[n_docs]                       */
  int32_t pool_size;        /* P >= 1                                       */
  int32_t n_kv_heads;       /* Hkv >= 1                                     */
  int32_t head_dim;         /* D in {64, 128}                               */
  int32_t n_router_heads;   /* Hr >= 1                                      */
  int32_t router_dim;       /* dr in {64, 128}                              */
  int32_t kr_layout;        /* msa_kr_layout of kr_pooled                   */
  double rope_theta;        /* > 0                                          */
  const int64_t *doc_tok_off;  /* device [n_docs+1], non-decreasing, from 0 */
  const int64_t *doc_pool_off; /* device [n_docs+1], prefix of ceil(L_d/P)  */
  const void *k;            /* device [n_tokens, Hkv, D], K before RoPE     */
  const void *v;            /* device [n_tokens, Hkv, D]                    */
  const void *kr;           /* device [n_tokens, Hr, dr]                    */
  void *kv_pooled;          /* out [n_pool, 2, Hkv, D]: K_bar, V_bar; device
                               or pinned host memory                        */
  void *kr_pooled;          /* out: the router bank, in kr_layout; device or
                               pinned host.  Row j of this call is written to
                               bank row kr_row_base + j                     */
  int64_t kr_row_base;      /* >= 0: first bank row of this call (a batch of
                               a bank encoded in pieces)                    */
} msa_pool_args;

int msa_pool_encode(const msa_pool_args *args, void *stream);

/* ------------------------------------------------------------------------
 * Stage 2 - online routing and context assembly.
 *
 * For query b, token t, pooled row j:
 *   s[b,t,j]  = (1/Hr) * sum_h cos(Qr[b,t,h], Kr_bar[j,h]),
 *               cos(x, y) = <x,y> / (max(|x|,1e-8) * max(|y|,1e-8))
 *   Dsc[b,d]  = max over t and over the rows j of document d of s[b,t,j]
 *   top-k     = the k documents with the largest Dsc[b,.], ties to the
 *               lower document id, in that order.
 * Sources: as for stage 1, whose routing paragraph defines the score as a
 * cosine averaged over router heads, then its maximum over tokens, and the
 * selection as the k best documents.
 * doc_scores is always written.  Arithmetic: bf16 inputs are multiplied in
 * the matrix cores with fp32 accumulation.  With at most 8 query tokens in
 * the call the normalised query is split into two bf16 terms (about 16
 * mantissa bits); with more it is rounded once to bf16 (relative error at
 * most 2^-9 per element, so a score moves by at most ~2e-3 and in practice
 * by ~1e-5).  fp32 inputs use fp32 vector arithmetic.
 *
 * Assembly (when host_kv != NULL): the selected documents' pooled rows
 * host_kv[doc_pool_off[d] .. doc_pool_off[d+1]) are copied, in rank order,
 * into mem_kv[b, L0 ...] where L0 is the current length when `append` is set
 * and 0 otherwise.  A document that does not fit in mem_cap rows is dropped
 * together with every lower-ranked one.  After the call, mem_len[b] is the
 * new length, and a later msa_sparse_decode on `stream` sees the memory.
 * The content tier is not in HBM: it is "fetched when selected" from host
 * memory, as the sources describe the tiered storage.  Two modes:
 *  MSA_GATHER_COPIES (0): BLOCKS the calling thread until the top-k indices
 *    are in host_topk_idx, enqueues one hipMemcpyAsync per document on
 *    copy_stream, writes host_mem_len / host_mem_docs (current length read
 *    from host_mem_len when appending), copies the lengths to mem_len and
 *    makes `stream` wait for the copies.  host_kv may be any pinned memory.
 *  MSA_GATHER_KERNEL (1): fully asynchronous.  The top-k kernel plans the
 *    copies on the device (current length read from mem_len when
 *    appending) and a gather kernel on `stream` reads the selected rows
 *    straight from host_kv, which must be device-mapped pinned memory
 *    (hipHostMalloc; checked with hipHostGetDevicePointer).  host_topk_idx,
 *    host_mem_len, host_mem_docs and copy_stream are unused (may be NULL).
 * In both modes host_kv must hold n_pool rows.  The host buffers of the copy
 * mode must not be modified until `stream` has passed this call.
 * ------------------------------------------------------------------------ */
typedef enum { MSA_GATHER_COPIES = 0, MSA_GATHER_KERNEL = 1 } msa_gather_mode;

typedef struct {
  int32_t dtype;            /* msa_dtype of qr and kr_pooled                */
  int32_t batch;            /* B >= 1 independent queries                   */
  int32_t q_tokens;         /* Tq >= 1 tokens per query                     */
  int32_t n_router_heads;   /* Hr                                           */
  int32_t router_dim;       /* dr in {64, 128}                              */
  int32_t top_k;            /* 1 <= k <= min(n_docs, 4096)                  */
  int32_t n_docs;
  int32_t kr_layout;        /* msa_kr_layout of kr_pooled; TILED needs bf16
                               and dr 64 with Hr <= 16 or dr 128 with Hr <= 8
                               (else MSA_ERR_UNSUPPORTED)                   */
  int64_t n_pool;           /* = doc_pool_off[n_docs]                       */
  const void *qr;           /* device [B, Tq, Hr, dr]                       */
  const void *kr_pooled;    /* device, n_pool rows in kr_layout             */
  const int64_t *doc_pool_off; /* device [n_docs+1]; every doc >= 1 row     */
  float *doc_scores;        /* device out [B, n_docs]                       */
  int32_t *topk_idx;        /* device out [B, k]                            */
  float *topk_score;        /* device out [B, k]                            */
  void *workspace;          /* device, msa_route_workspace_bytes() bytes    */
  size_t workspace_bytes;
  /* context assembly; all NULL / 0 to skip */
  const void *host_kv;              /* pinned host [n_pool, 2, Hkv, D]      */
  const int64_t *host_doc_pool_off; /* host [n_docs+1], same as device copy */
  int32_t kv_dtype;                 /* msa_dtype of host_kv and mem_kv      */
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t mem_cap;                  /* rows per query in mem_kv             */
  int32_t append;                   /* 1: append after the current length   */
  int32_t gather_mode;              /* msa_gather_mode                      */
  void *mem_kv;                     /* device [B, mem_cap, 2, Hkv, D]       */
  int32_t *mem_len;                 /* device [B]: out; in when appending   */
                                    /*   in MSA_GATHER_KERNEL mode          */
  int32_t *host_topk_idx;           /* pinned host out [B, k]     (copies)  */
  int32_t *host_mem_len;            /* pinned host in/out [B]     (copies)  */
  int32_t *host_mem_docs;           /* pinned host out [B]; opt.  (copies)  */
  void *copy_stream;                /* hipStream_t for the copies (copies)  */
  /* profiling, optional: existing hipEvent_t values attached to the
   * bank-scan kernel's dispatch (hipExtLaunchKernel): they record its start
   * and its end, and add no packet to the queue; NULL to skip */
  void *prof_event_begin;
  void *prof_event_end;
  /* optional: the document map of doc_pool_off from msa_doc_map (below),
   * used by the document path instead of building it in the workspace on
   * every call; 16-byte aligned.  NULL to build it per call. */
  const void *doc_map;
} msa_route_args;

int msa_route(const msa_route_args *args, void *stream);

/* Workspace for msa_route, in bytes (0 on invalid sizes). */
size_t msa_route_workspace_bytes(int32_t dtype, int32_t batch, int32_t q_tokens,
                                 int32_t n_router_heads, int32_t router_dim,
                                 int32_t n_docs, int64_t n_pool, int32_t top_k);

/* ------------------------------------------------------------------------
 * Context assembly as a call of its own: the assembly part of msa_route
 * for top-k ids it (or anything else) produced earlier.  Same sources and
 * the same rule as msa_route's assembly: the documents topk_idx[b, 0..k)
 * in rank order while they fit after the current length (append) or from
 * row 0; an id outside [0, n_docs) ends query b's list.  mem_len[b] is the
 * new length.
 * Splitting routing from assembly lets the content of one routing round
 * cross the host link while the next round is scored: call msa_route
 * without assembly for round r+1 and msa_assemble for round r (the sources'
 * "fetched when selected" tier, overlapped with scoring).
 *  MSA_GATHER_KERNEL: a plan kernel and the gather kernel on `stream`, fully
 *    asynchronous; host_kv device-mapped pinned memory; needs the
 *    workspace (msa_assemble_workspace_bytes) and doc_pool_off on the device.
 *  MSA_GATHER_COPIES: BLOCKS the calling thread until topk_idx (read on
 *    `stream`, after the work already queued there) is in host_topk_idx,
 *    then one hipMemcpyAsync per document on copy_stream; `stream` waits for
 *    the copies.  Uses host_doc_pool_off; no workspace.  Any pinned host_kv.
 * Errors as for msa_route's assembly arguments, plus batch >= 1,
 * 1 <= top_k <= min(n_docs, 4096) and a NULL topk_idx.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t batch;                    /* B >= 1                               */
  int32_t top_k;                    /* k ids per query                      */
  int32_t n_docs;
  int32_t kv_dtype;                 /* msa_dtype of host_kv and mem_kv      */
  int64_t n_pool;                   /* = doc_pool_off[n_docs]               */
  const int32_t *topk_idx;          /* device [B, k], rank order            */
  const int64_t *doc_pool_off;      /* device [n_docs+1] (kernel mode)      */
  const void *host_kv;              /* pinned host [n_pool, 2, Hkv, D]      */
  const int64_t *host_doc_pool_off; /* host [n_docs+1] (copies mode)        */
  int32_t n_kv_heads;
  int32_t head_dim;
  int32_t mem_cap;                  /* rows per query in mem_kv             */
  int32_t append;                   /* 1: append after the current length   */
  int32_t gather_mode;              /* msa_gather_mode                      */
  int32_t reserved0;
  void *mem_kv;                     /* device [B, mem_cap, 2, Hkv, D]       */
  int32_t *mem_len;                 /* device [B]: out; in when appending   */
                                    /*   in MSA_GATHER_KERNEL mode          */
  int32_t *host_topk_idx;           /* pinned host out [B, k]     (copies)  */
  int32_t *host_mem_len;            /* pinned host in/out [B]     (copies)  */
  int32_t *host_mem_docs;           /* pinned host out [B]; opt.  (copies)  */
  void *copy_stream;                /* hipStream_t for the copies (copies)  */
  void *workspace;                  /* device (kernel mode)                 */
  size_t workspace_bytes;
} msa_assemble_args;

int msa_assemble(const msa_assemble_args *args, void *stream);

/* Workspace for msa_assemble in the kernel mode (the copy plan), in bytes
 * (0 on invalid sizes). */
size_t msa_assemble_workspace_bytes(int32_t batch, int32_t top_k);

/* Document map of a router bank: an optional input of msa_route.
 * The document path of msa_route (one token per query on the matrix-core
 * scans) reduces each 16-row tile of the bank per document inside the scan;
 * for that it needs, per tile t (n_tiles = ceil(n_pool / 16)), the document
 * holding row 16 t and a bit per row 16 t + r (r < 16) that starts a
 * document or is row n_pool.  This depends on doc_pool_off alone (the
 * document-per-row reading of the routing passage quoted above), so a bank
 * routed many times can build it once: msa_doc_map writes it to doc_map,
 * device memory of msa_doc_map_bytes(n_pool) bytes, 16-byte aligned (layout:
 * n_tiles int32 document numbers, then, at the next multiple of 256 bytes,
 * n_tiles uint32 row masks), enqueued on `stream`.  The map describes exactly
 * the offsets it was built from; routing with a map of other offsets gives
 * wrong scores.  Returns MSA_ERR_INVALID_ARG for NULL pointers, n_docs < 1,
 * n_pool < n_docs or too small a buffer (nothing enqueued). */
size_t msa_doc_map_bytes(int64_t n_pool);
int msa_doc_map(const int64_t *doc_pool_off, int32_t n_docs, int64_t n_pool, void *doc_map,
                size_t doc_map_bytes, void *stream);

/* ------------------------------------------------------------------------
 * Stage 3 - one sparse decode-attention step.
 *
 * For query b with o = pos_offset[b], T = local_len[b], M = mem_len[b]:
 *   q'   = RoPE(q[b,h], o + T - 1)
 *   keys = [ K_bar rows mem_kv[b, 0..M, 0]  (used as stored: already
 *            rotated per document by msa_pool_encode) ;
 *            RoPE(local_k[b,i], o + i) for i < T ]
 *   vals = [ mem_kv[b, 0..M, 1] ; local_v[b, 0..T] ]
 *   out[b,h] = softmax(scale * keys[:, g] . q') . vals[:, g],
 *   g = h / (Hq/Hkv),  lse[b,h] = logsumexp of the logits.
 * The offset o is the number of retrieved documents k in the method's
 * global RoPE (order: background, then query, then generation), same
 * sources as above.  A query with no keys gets out = 0, lse = -inf.
 * M and T are clamped to [0, mem_cap] and [0, local_cap].  fp32 softmax and
 * accumulation; out is rounded to nearest-even into `dtype`.  bf16 runs
 * msa_sparse_attend's matrix-core kernel with one query token (same
 * arithmetic as described there) and needs q and out 16-byte aligned
 * (MSA_ERR_INVALID_ARG otherwise); fp32 runs a split-KV kernel in fp32
 * vector arithmetic.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t dtype;            /* msa_dtype of q, mem_kv, local_k/v, out       */
  int32_t batch;
  int32_t n_q_heads;        /* Hq, multiple of Hkv                          */
  int32_t n_kv_heads;       /* Hkv                                          */
  int32_t head_dim;         /* D in {64, 128}                               */
  int32_t mem_cap;          /* >= 0                                         */
  int32_t local_cap;        /* >= 0                                         */
  int32_t reserved0;
  const void *q;            /* device [B, Hq, D], before RoPE               */
  const void *mem_kv;       /* device [B, mem_cap, 2, Hkv, D]; NULL if cap 0 */
  const int32_t *mem_len;   /* device [B]                                   */
  const void *local_k;      /* device [B, local_cap, Hkv, D], before RoPE   */
  const void *local_v;      /* device [B, local_cap, Hkv, D]                */
  const int32_t *local_len; /* device [B]                                   */
  const int32_t *pos_offset;/* device [B]                                   */
  double rope_theta;        /* > 0                                          */
  float softmax_scale;      /* <= 0 selects 1/sqrt(D)                       */
  int32_t reserved1;
  void *out;                /* device out [B, Hq, D]                        */
  float *lse;               /* device out [B, Hq]; may be NULL              */
  void *workspace;          /* device, msa_decode_workspace_bytes() bytes   */
  size_t workspace_bytes;
  /* profiling, optional: existing hipEvent_t values attached to the
   * attention kernel's dispatch (its start and end; the split merge
   * follows); NULL to skip */
  void *prof_event_begin;
  void *prof_event_end;
} msa_decode_args;

int msa_sparse_decode(const msa_decode_args *args, void *stream);

/* Workspace for msa_sparse_decode, in bytes (0 on invalid sizes). */
size_t msa_decode_workspace_bytes(int32_t batch, int32_t n_q_heads, int32_t head_dim,
                                  int32_t mem_cap, int32_t local_cap);

/* msa_sparse_decode for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation and kernels, with the split partials in
 * a static device array of the library (64 MiB, one per device, held until
 * the process ends) instead of a workspace.  args->workspace and
 * args->workspace_bytes are ignored; the call allocates nothing.  A call
 * whose partials exceed 64 MiB (msa_decode_workspace_bytes() > 64 MiB for
 * its sizes) returns MSA_ERR_WORKSPACE and enqueues nothing.  Every call on
 * one device uses the same array: calls whose execution overlaps on one
 * device (different streams, no ordering between them) race and give wrong
 * results; calls ordered on one stream are safe.  Other arguments,
 * validation and errors as for msa_sparse_decode. */
int msa_sparse_decode_noalloc(const msa_decode_args *args, void *stream);

/* ------------------------------------------------------------------------
 * Stage 3 for a block of query tokens - prefill through the sparse context.
 *
 * The Tq query tokens of query b are the LAST Tq tokens of its local context
 * (their K/V are already in local_k/local_v).  With o = pos_offset[b],
 * T = local_len[b], M = mem_len[b], token t sits at local index
 * i_t = T - Tq + t and position o + i_t:
 *   q'[t,h]  = RoPE(q[b,t,h], o + i_t)
 *   keys     = [ mem_kv[b, 0..M, 0] (as stored) ; RoPE(local_k[b,i], o + i) ]
 *   token t sees every memory row and the local tokens i <= i_t (causal)
 *   out[b,t,h] = softmax(scale * keys[:, g] . q'[t,h]) . vals[:, g] over
 *                the keys it sees; lse[b,t,h] their log-sum-exp.
 * With Tq = 1 this is msa_sparse_decode's step.  Sources as for stage 3; the
 * pages order the context background, then query, then generation, and do
 * not spell out the block form: the causal block over the local context is
 * this library's reading.  A token that sees no key gets out = 0,
 * lse = -inf (also when T < Tq leaves it without local tokens).
 * bf16 only: q, K and V enter v_mfma_f32_16x16x32_bf16 /
 * v_mfma_f32_16x16x16bf16_1k with fp32 accumulation; the rotated query is
 * split into two bf16 terms, rotated local keys and the softmax weights are
 * rounded to bf16 once; softmax statistics are fp32.
 * Validation as for msa_sparse_decode, plus batch, q_tokens >= 1,
 * Hq / Hkv <= 16; fp32 returns MSA_ERR_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
typedef struct {
  int32_t dtype;            /* MSA_BF16                                     */
  int32_t batch;
  int32_t q_tokens;         /* Tq >= 1                                      */
  int32_t n_q_heads;        /* Hq, multiple of Hkv, Hq/Hkv <= 16            */
  int32_t n_kv_heads;       /* Hkv                                          */
  int32_t head_dim;         /* D in {64, 128}                               */
  int32_t mem_cap;          /* >= 0                                         */
  int32_t local_cap;        /* >= 0                                         */
  const void *q;            /* device [B, Tq, Hq, D], before RoPE           */
  const void *mem_kv;       /* device [B, mem_cap, 2, Hkv, D]; NULL if cap 0 */
  const int32_t *mem_len;   /* device [B]                                   */
  const void *local_k;      /* device [B, local_cap, Hkv, D], before RoPE   */
  const void *local_v;      /* device [B, local_cap, Hkv, D]                */
  const int32_t *local_len; /* device [B], including the Tq query tokens    */
  const int32_t *pos_offset;/* device [B]                                   */
  double rope_theta;        /* > 0                                          */
  float softmax_scale;      /* <= 0 selects 1/sqrt(D)                       */
  int32_t reserved0;
  void *out;                /* device out [B, Tq, Hq, D], 16-byte aligned   */
  float *lse;               /* device out [B, Tq, Hq]; may be NULL          */
  void *workspace;          /* device, msa_attend_workspace_bytes() bytes   */
  size_t workspace_bytes;
  /* profiling, optional: existing hipEvent_t values attached to the
   * attention kernel's dispatch (its start and end; the split merge
   * follows); NULL to skip */
  void *prof_event_begin;
  void *prof_event_end;
} msa_attend_args;

int msa_sparse_attend(const msa_attend_args *args, void *stream);

/* Workspace for msa_sparse_attend, in bytes (0 on invalid sizes). */
size_t msa_attend_workspace_bytes(int32_t batch, int32_t q_tokens, int32_t n_q_heads, int32_t n_kv_heads,
                                  int32_t head_dim, int32_t mem_cap, int32_t local_cap);

/* Thread-local description of the last non-OK return on this thread. */
const char *msa_last_error(void);

/* Library version, MAJOR * 10000 + MINOR * 100 + PATCH. */
int msa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MSA_H */
