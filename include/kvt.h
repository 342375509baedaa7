/*
 * kvt.h -- C ABI of libkvt: the tiered KV-cache hot path on MI355X (gfx950).
 *
 * Paged K/V lives partly in pinned, device-mapped host memory and partly in HBM.  The library
 * moves blocks between the tiers and runs attention over them:
 *
 *   kvt_sub_block_ptrs   build src/dst/size pointer tables        (host, pure)
 *   kvt_swap_blocks      batched block copy driven by those tables (host<->HBM)
 *   kvt_index_topk       score a pooled indexer plane in HBM, select the top-k blocks
 *   kvt_select_positions expand selected pooled blocks into token positions (+ write-head tail)
 *   kvt_gather_blocks    copy only the selected blocks' K/V rows host -> HBM
 *   kvt_stage_tail       copy a sequence's host-resident rows into an HBM staging buffer
 *   kvt_attn_decode      GQA decode attention over gathered K/V
 *   kvt_gather_attn_decode  the gather and the decode attention in one pass
 *   kvt_sparse_attend_rows  many query rows, each over its own selection of cache positions
 *   kvt_sparse_attend_rows_auto  the same, staging the used pages first when that reads less
 *   kvt_stage_pages      copy a sequence's pages (via its block table) into HBM in logical order
 *   kvt_attn_prefill     causal (or full) prefill attention over an HBM head + tail
 *   kvt_attn_prefill_range      the same attention as resumable passes over key ranges
 *   kvt_attn_prefill_pipelined  tail staging in arena buckets overlapped with the attention
 *   kvt_attn_prefill_chain      the same over a chain of layers, prefetching the next layer
 *   kvt_attn_prefill_auto       stage the tail, pipeline it or read it in place, by a time model
 *   kvt_worker_*         an ordered, event-timed asynchronous transfer queue around the swap
 *   kvt_paged_write      append new K/V (and raw key) rows into paged planes via a block table
 *   kvt_copy_page        duplicate a page's first rows (host planes on the CPU, pooled on device)
 *   kvt_pool_rebuild     recompute the pooled keys of the blocks an append touched
 *
 * Sources (page titles; each entry point names the section it follows):
 *   [vLLM-CPU] vLLM fork, "v1/kv_offload/cpu/gpu_worker.py" (CPU offloading worker)
 *   [QSA-KVO]  "QSA KV cache host-RAM offload for ExLlamaV3" (qsa-kv-offload.patch)
 *   [llama-T]  "llama/cuda: tiered KV cache (--kv-vram-cells)", llama.cpp PR #319
 *   [exl3-DMA] vllm-exl3 patch "vllm-exl3-host-dma.patch" (prefill DMA streaming into VRAM slots)
 *
 * Conventions (all entry points):
 *   - The caller owns every buffer.  The library allocates nothing on the hot path; where an
 *     op needs scratch, the caller passes a workspace sized by the matching *_ws_bytes call.
 *     (The transfer worker is the exception: it owns pools of streams, events and pinned
 *     descriptor tables, which grow on first need or up front through kvt_worker_reserve.)
 *   - "device pointer" = an address a gfx950 kernel may dereference: HBM from hipMalloc /
 *     torch, or pinned host memory from kvt_host_alloc (its device alias).  "host-mapped"
 *     planes are such device aliases of pinned host memory; kernels read them over PCIe.
 *   - Every compute entry point only ENQUEUES work on `stream` (a hipStream_t; NULL = the
 *     legacy default stream) and returns.  Inputs, tables and outputs must stay valid, and
 *     must not be written by anyone else, until the stream has passed the op.  Ordering against
 *     other streams (e.g. a store must wait for the writes it reads) is the caller's job.
 *   - Errors: argument checks happen on the host before anything is enqueued; a failing check
 *     returns a negative status and enqueues nothing.  Nothing aborts or throws across the
 *     ABI.  kvt_last_error() returns a message for the last failure on the calling thread.
 *   - ABI evolution is append-only: new parameters go into new entry points, and
 *     kvt_abi_version() is bumped on any addition.
 */
#ifndef KVT_H
#define KVT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVT_ABI_VERSION 16

/* status codes */
#define KVT_OK 0
#define KVT_EINVAL (-1)       /* bad argument (shape, count, null pointer, skip >= bpc ...) */
#define KVT_ERANGE (-2)       /* an index or count outside what the buffers hold */
#define KVT_EALIGN (-3)       /* an address or size misaligned for the requested path */
#define KVT_EOVERLAP (-4)     /* overlapping copy ranges (only when validation is asked for) */
#define KVT_ENOMEM (-5)       /* pinned host allocation failed */
#define KVT_EUNSUPPORTED (-6) /* a valid request the library does not implement */
#define KVT_EHIP (-7)         /* a HIP runtime call failed; kvt_last_error() has its text */

/* copy direction and mechanism */
#define KVT_H2D 0
#define KVT_D2H 1
#define KVT_COPY_AUTO 0    /* the kernel when sizes are multiples of 8 and pages are below the
                             threshold (default: no limit), else RUNTIME */
#define KVT_COPY_KERNEL 1  /* wavefront loads/stores through the host mapping */
#define KVT_COPY_SDMA 2    /* the DMA copy engines driven through HSA, one engine copy per
                             run of adjacent descriptors (<= 4 MiB pieces), round-robin over
                             the engines; waits on the calling thread (kvt_swap_blocks and
                             kvt_stage_tail; see kvt_swap_blocks) */
#define KVT_COPY_RUNTIME 3 /* HIP's copy calls (hipMemcpyBatchAsync, else hipMemcpyAsync per
                             descriptor); the runtime picks the engine per copy and serves
                             page-sized copies with its blit kernel */

/* element formats */
#define KVT_F16 1
#define KVT_BF16 2
#define KVT_Q8_0 3 /* 32-value blocks: fp16 scale (2 bytes, little-endian) + 32 int8; x = scale*q */

/* kvt_host_alloc flags */
#define KVT_HOST_COHERENT 0u       /* fine-grained: GPU reads bypass caching of host data */
#define KVT_HOST_NONCOHERENT 1u    /* coarse-grained mapping */
#define KVT_HOST_WRITECOMBINED 2u  /* write-combined on the CPU side (host writes, GPU reads) */

int kvt_abi_version(void);
const char *kvt_last_error(void);

/* ----------------------------------------------------------------------------------------
 * Host tier.  [QSA-KVO] CacheLayer_qsa_offload.alloc/free: K/V planes live in pinned,
 * device-mapped host memory that kernels reach through a device alias.  The page registers
 * an anonymous mapping; this library allocates pinned memory instead (registering memory
 * that already exists is not available on every ROCm host), with the same result: one slab,
 * zero-filled, usable by host code through *host_ptr and by kernels through *dev_ptr.
 *   bytes    > 0
 *   flags    KVT_HOST_* (one of)
 *   host_ptr receives the host address; dev_ptr the device alias (equal on ROCm with UVA).
 * Returns KVT_ENOMEM when the allocation fails (the page's fallback rule: the caller may
 * then keep the data in pageable memory and use SDMA copies).
 * kvt_host_free releases a slab from kvt_host_alloc; every device use must have completed.
 * ---------------------------------------------------------------------------------------- */
int kvt_host_alloc(size_t bytes, unsigned flags, void **host_ptr, void **dev_ptr);
int kvt_host_free(void *host_ptr);

/* ----------------------------------------------------------------------------------------
 * S1  pointer tables.  [vLLM-CPU] compute_sub_block_ptrs, _fill_direct_ops, transfer_async.
 * A tensor row (block) b holds `bpc` sub-blocks ("pages") of page_bytes each; sub-block j of
 * block b starts at  base + b*row_stride + j*page_bytes.  The pointers of block_ids[0..n_ids)
 * are listed block-major and the run [skip, skip + n_out) is written to out[0..n_out).
 *   bpc >= 1, 0 <= skip < bpc, n_out <= n_ids*bpc - skip, block_ids[i] >= 0.
 * With bpc == 1 (the GPU side of a transfer) out[i] = base + block_ids[i]*row_stride.
 * Pure host code: touches no device.  Errors: KVT_EINVAL, KVT_ERANGE.
 * kvt_chunks_consumed(n, skip, bpc) = ceil((n + skip) / bpc): how many chunk-side blocks a
 * run of n sub-blocks starting `skip` into its first block uses.
 * ---------------------------------------------------------------------------------------- */
int kvt_sub_block_ptrs(uint64_t base, uint64_t row_stride, uint64_t page_bytes,
                       const int64_t *block_ids, int64_t n_ids, int32_t bpc, int32_t skip,
                       uint64_t *out, int64_t n_out);
int64_t kvt_chunks_consumed(int64_t n, int32_t skip, int32_t bpc);

/* ----------------------------------------------------------------------------------------
 * S2  batched swap.  [vLLM-CPU] transfer_async -> swap_blocks_batch(src, dst, sizes):
 *   for i < n: copy sizes[i] bytes from address src[i] to address dst[i].
 * src, dst, sizes: u64 tables of n entries in pinned host memory from kvt_host_alloc (the
 *   SDMA path reads them on the host, the kernel path through their device alias; pass the
 *   host pointer -- it is the same address on ROCm).  Table entries are device addresses.
 * dir:  KVT_H2D (load) or KVT_D2H (store); selects which AUTO threshold applies.
 * mode: KVT_COPY_AUTO / KERNEL / SDMA / RUNTIME.  The kernel path needs every size to be a
 *   multiple of 8 (else KVT_EALIGN); 16-byte aligned addresses take the wide path, 8-byte
 *   aligned ones an 8-byte path, anything else a byte path.
 *   SDMA is synchronous with respect to the calling thread: the call waits for the work
 *   already queued on the stream, submits the engine copies (descriptors that continue the
 *   previous one on both sides go as one copy, cut into pieces of at most 4 MiB), round-robin
 *   over the engines kvt_copy_engines(dir) counts, waits for them and returns, so work queued
 *   afterwards sees them.  Host addresses must be pinned memory from kvt_host_alloc (or
 *   hipHostMalloc).  Not allowed while the stream is being captured into a graph
 *   (KVT_EUNSUPPORTED).  Every engine copy has a completion signal of its own (value 1), at
 *   most 256 in flight, waited for oldest first.  A signal that cannot be created, or a copy
 *   that cannot be submitted, returns KVT_EHIP after the copies already submitted are done.
 * Destination ranges must be pairwise disjoint and disjoint from all sources; the order of
 * the copies is unspecified.  Zero sizes are no-ops.  n == 0 enqueues nothing.
 * ---------------------------------------------------------------------------------------- */
int kvt_swap_blocks(const uint64_t *src, const uint64_t *dst, const uint64_t *sizes, int64_t n,
                    int32_t dir, int32_t mode, void *stream);
/* AUTO switches to RUNTIME at pages >= threshold bytes (per direction); returns the old value. */
uint64_t kvt_set_copy_threshold(int32_t dir, uint64_t bytes);
/* The number of DMA engines KVT_COPY_SDMA spreads its copies over on the current device for
 * direction dir (those the runtime reports available; 0: none reported, the runtime then
 * picks an engine per copy), or a negative status. */
int kvt_copy_engines(int32_t dir);

/* ----------------------------------------------------------------------------------------
 * S3+S4  index scoring and top-k selection.  [QSA-KVO] CacheLayer_qsa_offload docstring and
 * InferParams.qsa_kv_offload: the pooled indexer plane stays in HBM and is scored in full on
 * every step; a top-k selection of blocks decides which K/V rows are read from host memory.
 *   pooled  device fp16 [n_blocks][dim]  (one pooled key per KV block)
 *   q_idx   device fp16 [n_sel][dim]     (one index query per selection head)
 *   score s[h][b] = sum_{d=0..dim-1} q_idx[h][d]*pooled[b][d], evaluated in fp64 in index
 *   order (each fp16 product is exact in fp64, so the value is fully determined).
 *   ids     device int32 [n_sel][k]: per head the k best blocks -- larger score first, equal
 *           scores by lower block id, NaN after every number -- written in ascending id
 *           order; when k > n_blocks the trailing slots hold -1.
 *   scores  optional device fp64 [n_sel][n_blocks] copy of every score (NULL to skip).
 *   ws      device workspace of kvt_index_topk_ws_bytes(n_blocks, n_sel, k) bytes.
 * Limits: 1 <= k <= 2048, dim a multiple of 8 and <= 256, 1 <= n_sel <= 32.
 * ---------------------------------------------------------------------------------------- */
size_t kvt_index_topk_ws_bytes(int64_t n_blocks, int32_t n_sel, int32_t k);
int kvt_index_topk(const void *pooled, int64_t n_blocks, int32_t dim, const void *q_idx,
                   int32_t n_sel, int32_t k, int32_t *ids, double *scores, void *ws,
                   size_t ws_bytes, void *stream);

/* ----------------------------------------------------------------------------------------
 * S4 selection geometry.  [QSA-KVO] indexer: each pooled key covers cr tokens, a row selects
 * block_topk pooled blocks, and reads their cr*block_topk token positions plus the tokens at
 * the write head that no complete pooled block covers yet, -1 padded to
 * K_pad = ceil((block_topk*cr + cr - 1) / 32) * 32 (2080 for block_topk 512, cr 4).
 *   ids        device int32 [n_sel][k]: selected pooled-block ids, ascending, -1 only at the end
 *              (kvt_index_topk's output over the n_tok / cr complete blocks)
 *   positions  device int32 [n_sel][k_pad]: for the v valid ids, positions id*cr + 0..cr-1 in
 *              order; then cr*floor(n_tok/cr) .. n_tok-1; then -1.  Ascending up to the first -1.
 * Limits: k_pad >= k*cr + cr - 1, n_tok < 2^31.  Feed positions to kvt_gather_attn_decode (or
 * kvt_gather_blocks) with bt = 1, k = k_pad, n_blocks = n_tok and per-token strides.
 * ---------------------------------------------------------------------------------------- */
int kvt_select_positions(const int32_t *ids, int32_t n_sel, int32_t k, int32_t cr, int64_t n_tok,
                         int32_t k_pad, int32_t *positions, void *stream);

/* ----------------------------------------------------------------------------------------
 * S5  top-k gather.  [QSA-KVO] sparse_attend / CacheLayer_qsa_offload: only the selected
 * blocks' K/V rows cross the host link, so the bytes read per step do not depend on context;
 * the gather reaches the planes through a base pointer plus computed offsets.
 *   k_plane, v_plane  device pointers (normally host-mapped).  Token r (0 <= r < bt) of
 *                     physical block p, head h, starts at
 *                         plane + p*block_stride + h*head_stride + r*token_stride   (bytes)
 *                     and holds hd elements of elem_bytes.  Token-major [token][head][dim]:
 *                     (bt*kvh*hd*eb, hd*eb, kvh*hd*eb); block-local head-major
 *                     [block][head][token][dim]: (kvh*bt*hd*eb, bt*hd*eb, hd*eb).
 *   n_blocks          physical blocks the planes hold; logical block b lives in physical block
 *                     block_table[b] (identity when block_table is NULL).
 *   ids               device int32 [kvh][k], e.g. kvt_index_topk's output.
 *   k_out, v_out      device [kvh][k*bt][hd] elements: out[h][i*bt + r] = token r of block
 *                     phys(ids[h][i]), head h.
 * Slots with ids < 0, or whose block lies outside [0, n_blocks), are skipped (left untouched).
 * hd*elem_bytes and the three strides must be multiples of 16, bases 16-byte aligned.
 * ---------------------------------------------------------------------------------------- */
int kvt_gather_blocks(const void *k_plane, const void *v_plane, int64_t n_blocks, int32_t kvh,
                      int32_t hd, int32_t elem_bytes, int64_t block_stride, int64_t head_stride,
                      int64_t token_stride, const int32_t *block_table, int32_t bt,
                      const int32_t *ids, int32_t k, void *k_out, void *v_out, void *stream);

/* ----------------------------------------------------------------------------------------
 * S7  tail staging.  [llama-T] commit text: when an attention op reaches the host tail, the
 * used host rows are copied into a VRAM staging buffer once per op, and the op reads that.
 *   staging[(r - row_begin)*row_bytes ...] = plane[r*row_bytes ...]  for r in [row_begin, row_end)
 *   plane: device pointer (host-mapped), staging: device (HBM); mode KVT_COPY_*: KERNEL is
 *   the wide-load kernel over one span; AUTO and RUNTIME are one hipMemcpyAsync, which the
 *   runtime runs on a copy engine at staging sizes (and which graph capture records); SDMA
 *   is the engine mode of kvt_swap_blocks over the one range (4 MiB pieces round-robin over
 *   the engines, synchronous with respect to the calling thread, not capturable).
 * ---------------------------------------------------------------------------------------- */
int kvt_stage_tail(const void *plane, int64_t row_bytes, int64_t row_begin, int64_t row_end,
                   void *staging, int32_t mode, void *stream);

/* ----------------------------------------------------------------------------------------
 * S6  decode attention.  [QSA-KVO] qsa_sparse_attend_rows_staged: q head i reads KV head
 * i / (n_qh/kvh); softmax over the head's keys; partial (o, m, l) folded with the online-
 * softmax rule.
 *   q      device [n_qh][hd], dtype KVT_BF16 or KVT_F16
 *   k, v   device [kvh][n_kv][hd], same dtype (kvt_gather_blocks' layout)
 *   n_valid optional device int32 [kvh]: keys j < n_valid[h] take part (NULL = all n_kv)
 *   out    device fp32 [n_qh][hd]:  o_i = sum_j e^(l_j - m) v_j / sum_j e^(l_j - m),
 *          l_j = scale * q_i.k_j; a head with no valid key gets 0.
 *   ws     device workspace of kvt_attn_decode_ws_bytes(n_qh, hd, n_kv) bytes.
 * Limits: hd == 128, n_qh/kvh <= 16.  Deterministic: fixed split and merge order.
 * ---------------------------------------------------------------------------------------- */
size_t kvt_attn_decode_ws_bytes(int32_t n_qh, int32_t hd, int64_t n_kv);
int kvt_attn_decode(const void *q, int32_t n_qh, int32_t kvh, int32_t hd, int32_t dtype,
                    const void *k, const void *v, int64_t n_kv, const int32_t *n_valid,
                    float scale, float *out, void *ws, size_t ws_bytes, void *stream);

/* ----------------------------------------------------------------------------------------
 * S5+S6 in one pass.  [QSA-KVO] sparse_attend / qsa_sparse_attend_rows_staged: decode reads
 * the selected blocks' K/V through base pointers and computed offsets.  Each 64-key chunk's
 * rows cross the host link straight into the wavefront that attends them, so the attention
 * runs under the transfer instead of after it.
 *   q, n_qh, kvh, hd, dtype, scale, out, ws   as kvt_attn_decode, with n_kv = k*bt
 *                     (ws: kvt_attn_decode_ws_bytes(n_qh, hd, k*bt) bytes)
 *   k_plane ... k     as kvt_gather_blocks, with elem_bytes = 2: key j (j < k*bt) of head h
 *                     is token j % bt of slot j / bt of that head's selection
 *   k_out, v_out      optional device [kvh][k*bt][hd] (both or neither): when given they
 *                     receive exactly what kvt_gather_blocks writes (skipped slots untouched)
 * Keys of slots that kvt_gather_blocks skips (id < 0, block outside [0, n_blocks)) take no
 * part.  With such slots only at the end of each head's list, out is bit-identical to
 * kvt_gather_blocks followed by kvt_attn_decode with n_valid[h] = bt * (valid slots of h):
 * the same chunks, the same arithmetic, the same merge.
 * Limits: hd == 128, n_qh/kvh <= 16, n_blocks >= 1, k*bt < 2^31 - 64; strides multiples of
 * 16, q, planes and outputs 16-byte aligned.
 * ---------------------------------------------------------------------------------------- */
int kvt_gather_attn_decode(const void *q, int32_t n_qh, int32_t kvh, int32_t hd, int32_t dtype,
                           const void *k_plane, const void *v_plane, int64_t n_blocks,
                           int64_t block_stride, int64_t head_stride, int64_t token_stride,
                           const int32_t *block_table, int32_t bt, const int32_t *ids, int32_t k,
                           void *k_out, void *v_out, float scale, float *out, void *ws,
                           size_t ws_bytes, void *stream);

/* ----------------------------------------------------------------------------------------
 * kvt_gather_attn_decode without a workspace, for callers that cannot allocate device memory
 * (code under graph capture, tight serving loops, harnesses that forbid allocation).
 * Arguments, results and limits as kvt_gather_attn_decode, minus ws / ws_bytes: the split
 * partials go to a scratch array inside the library, one per GPU, of
 * kvt_gather_attn_decode_noalloc_max_bytes() bytes (4 MiB), held until the process ends.
 * The call allocates nothing.  It needs n_qh * ceil(k*bt / 64) * (hd + 2) * 4 bytes of it
 * (1.06 MB for 64 query heads and 32 blocks of 64 tokens); more returns KVT_ERANGE and
 * enqueues nothing.  Every call on one GPU uses the same scratch, and each call writes every
 * partial it reads, so nothing carries over between calls; but calls that can run at the
 * same time on one GPU (on different streams) race on it and must be ordered by the caller.
 * ---------------------------------------------------------------------------------------- */
size_t kvt_gather_attn_decode_noalloc_max_bytes(void);
int kvt_gather_attn_decode_noalloc(const void *q, int32_t n_qh, int32_t kvh, int32_t hd,
                                   int32_t dtype, const void *k_plane, const void *v_plane,
                                   int64_t n_blocks, int64_t block_stride, int64_t head_stride,
                                   int64_t token_stride, const int32_t *block_table, int32_t bt,
                                   const int32_t *ids, int32_t k, void *k_out, void *v_out,
                                   float scale, float *out, void *stream);

/* ----------------------------------------------------------------------------------------
 * Sparse attention over per-row selections.  [QSA-KVO] qsa_sparse_attend_rows: query row r
 * (R rows of n_qh heads, e.g. the tokens of a prefill chunk) attends the cache positions
 * positions[r][0..k_pad) (logical token positions; -1 pads), the same selection for every
 * head; query head i reads KV head i / (n_qh/kvh).  Each row's result is the decode
 * attention of kvt_attn_decode over its valid positions, in the same fp32 arithmetic.
 *   q       device [rows][n_qh][hd], dtype KVT_BF16 / KVT_F16;  out: device fp32, same shape
 *   planes  k_plane, v_plane: device pointers (host-mapped or HBM) of n_rows token rows;
 *           head h of physical row x at plane + x*row_stride + h*head_stride
 *           (head_stride*(kvh-1) + hd*2 <= row_stride; strides multiples of 16)
 *   block_table  NULL: positions are physical rows.  Else device int32, row r's entries at
 *           block_table + r*table_row_stride (0 = one table for all rows), table_cols of
 *           them; position p -> physical row block_table[p / page_size]*page_size + p % page_size
 *   A position takes part when it is >= 0, below table_cols*page_size (n_rows without a
 *   table), its table entry is >= 0 and the physical row is below n_rows.
 *   ws      device workspace of kvt_sparse_attend_rows_ws_bytes(rows, n_qh, kvh, k_pad)
 * Limits: hd == 128, n_qh/kvh <= 16, rows <= 65535, n_rows < 2^31.  Deterministic.
 *
 * kvt_staging_worthwhile: [QSA-KVO] qsa_staging_worthwhile -- nonzero when
 *   rows * k_pad > 2 * pages_used * page_size (the direct reads would exceed twice the history).
 * kvt_stage_pages: page block_table[p] of k_plane (and v_plane) -> page p of k_out (v_out),
 *   p < n_used, pages of page_bytes (a multiple of 16); entries outside [0, n_pages) leave
 *   their page untouched.  v_plane and v_out both given or both NULL.
 * kvt_sparse_attend_rows_auto: one sequence (one block table for every row), dense pages of
 *   page_size rows (n_rows a multiple of page_size), positions below pages_used*page_size.
 *   When kvt_staging_worthwhile(rows, k_pad, pages_used, page_size) holds and staging_k and
 *   staging_v (device, staging_bytes each) hold pages_used pages, the pages are staged with
 *   kvt_stage_pages and the rows attend the HBM copy; otherwise they read in place.  The
 *   output is bit-identical either way.  *staged (optional, host) receives which was taken.
 * ---------------------------------------------------------------------------------------- */
size_t kvt_sparse_attend_rows_ws_bytes(int32_t rows, int32_t n_qh, int32_t kvh, int32_t k_pad);
int kvt_sparse_attend_rows(const void *q, int32_t rows, int32_t n_qh, int32_t kvh, int32_t hd,
                           int32_t dtype, const void *k_plane, const void *v_plane,
                           int64_t n_rows, int64_t row_stride, int64_t head_stride,
                           const int32_t *block_table, int32_t table_cols,
                           int64_t table_row_stride, int32_t page_size, const int32_t *positions,
                           int32_t k_pad, float scale, float *out, void *ws, size_t ws_bytes,
                           void *stream);
int kvt_staging_worthwhile(int64_t rows, int64_t k_pad, int64_t pages_used, int64_t page_size);
int kvt_stage_pages(const void *k_plane, const void *v_plane, int64_t page_bytes,
                    const int32_t *block_table, int32_t n_used, int64_t n_pages, void *k_out,
                    void *v_out, void *stream);
int kvt_sparse_attend_rows_auto(const void *q, int32_t rows, int32_t n_qh, int32_t kvh,
                                int32_t hd, int32_t dtype, const void *k_plane,
                                const void *v_plane, int64_t n_rows, int64_t row_stride,
                                int64_t head_stride, const int32_t *block_table,
                                int32_t pages_used, int32_t page_size, const int32_t *positions,
                                int32_t k_pad, float scale, float *out, void *ws,
                                size_t ws_bytes, void *staging_k, void *staging_v,
                                size_t staging_bytes, int32_t *staged, void *stream);

/* ----------------------------------------------------------------------------------------
 * S8  prefill attention over a tiered cache.  [llama-T]: cells [0, n_head) live in HBM, the
 * rest in host memory (read in place, or staged into HBM first by kvt_stage_tail); the output
 * is the same, bit for bit, whichever way the tail is reached.
 *   q      device fp16 [n_q][n_qh][hd]; query row t is at position q_pos0 + t
 *   row r of K (and V) lives at k_head + r*row_bytes for r < n_head, else at
 *          k_tail + (r - n_head)*row_bytes; a row is kvh heads x hd values in kv_format
 *          (KVT_Q8_0: hd/32 blocks of 34 bytes per head, head-major)
 *   causal nonzero: row t sees keys j <= q_pos0 + t (j < n_kv); zero: all n_kv keys
 *   out    device fp32 [n_q][n_qh][hd]
 *   kv_format KVT_Q8_0, KVT_F16 or KVT_BF16.  q8_0 values are dequantised to fp16 (one
 *          rounding) and fp16 values used as stored, on fp16 MFMA.  bf16 values are used as
 *          stored, on bf16 MFMA, over their whole range: the fp16 query is split into two
 *          bf16 parts whose sum is exact, and the fp32 probabilities into two bf16 parts
 *          (16 significant bits), so each product is taken twice (about 1.6x the time).
 * Limits: hd == 128, n_qh/kvh in {1, 2, 4, 8}, scale > 0; q and out 16-byte aligned,
 * K/V pointers 8-byte aligned.  Deterministic: the same inputs give the same bits, however
 * the rows are split between head and tail.
 * ---------------------------------------------------------------------------------------- */
int kvt_attn_prefill(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh, int32_t kvh,
                     int32_t hd, const void *k_head, const void *v_head, int64_t n_head,
                     const void *k_tail, const void *v_tail, int64_t n_kv, int32_t kv_format,
                     int32_t causal, float scale, float *out, void *stream);

/* ----------------------------------------------------------------------------------------
 * S8 for short chunks.  [llama-T] also stages the tail for decode steps in the host tier; a
 * chunk of few queries (one, for a decode step) gives kvt_attn_prefill only query tiles x kvh
 * workgroups, each walking the whole key range.  kvt_attn_prefill_splitk computes the same
 * attention with the key range split across workgroups at fixed 64-key tile boundaries: each
 * split keeps its (o, m, l) in the workspace and a merge folds the splits in split order.
 * Arguments as kvt_attn_prefill, plus ws: device workspace of
 * kvt_attn_prefill_splitk_ws_bytes(n_q, n_qh, kvh, n_kv) bytes (0 when no split is taken).
 * Splits are chosen to put about one workgroup on every CU (at least 8 tiles each); with one
 * split the call is kvt_attn_prefill, bit for bit.  Deterministic, and independent of n_head
 * (head/tail placement) like kvt_attn_prefill.
 * ---------------------------------------------------------------------------------------- */
size_t kvt_attn_prefill_splitk_ws_bytes(int64_t n_q, int32_t n_qh, int32_t kvh, int64_t n_kv);
int kvt_attn_prefill_splitk(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                            int32_t kvh, int32_t hd, const void *k_head, const void *v_head,
                            int64_t n_head, const void *k_tail, const void *v_tail, int64_t n_kv,
                            int32_t kv_format, int32_t causal, float scale, void *ws,
                            size_t ws_bytes, float *out, void *stream);

/* ----------------------------------------------------------------------------------------
 * S8 as resumable passes.  [QSA-KVO] staged attention folds bucket partials with the online-
 * softmax rule; here a pass over keys [key_begin, key_end) continues from the running
 * (o, m, l) of the previous pass, kept in `state` in exact fp32, so any split into passes
 * gives the same bits as kvt_attn_prefill (the tiles, their order and the arithmetic are the
 * same).  Arguments as kvt_attn_prefill, plus:
 *   key_begin, key_end  multiples of 64 (key_end may be n_kv); passes must cover [0, n_kv) in
 *                       order, each starting where the last ended.  The first pass
 *                       (key_begin == 0) starts a fresh state; the last (key_end == n_kv)
 *                       writes `out`, the others write only `state`.
 *   state               device, kvt_attn_prefill_state_bytes(n_q, n_qh, kvh) bytes, owned by
 *                       the caller; opaque layout; may be NULL for a single pass [0, n_kv).
 * Rows a pass reads through k_tail/v_tail must be valid during that pass only: a pass over
 * [key_begin, key_end) touches no row outside that range.
 * ---------------------------------------------------------------------------------------- */
size_t kvt_attn_prefill_state_bytes(int64_t n_q, int32_t n_qh, int32_t kvh);
int kvt_attn_prefill_range(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                           int32_t kvh, int32_t hd, const void *k_head, const void *v_head,
                           int64_t n_head, const void *k_tail, const void *v_tail, int64_t n_kv,
                           int32_t kv_format, int32_t causal, float scale, int64_t key_begin,
                           int64_t key_end, void *state, size_t state_bytes, float *out,
                           void *stream);

/* ----------------------------------------------------------------------------------------
 * S7+S8 overlapped.  [llama-T] stages the used host rows into VRAM once per op; [QSA-KVO]
 * stages in arena-sized buckets and overlaps the copy of one bucket with attention on the
 * previous.  Here: `stream` attends the HBM head (whole 64-key tiles) while `copy_stream`
 * copies the first bucket of host rows into one half of the arena; then each bucket is
 * attended from its arena half while the next bucket is copied into the other half.
 *   k_host, v_host      device aliases of the host tail: row r >= n_head at
 *                       k_host + (r - n_head)*row_bytes (row_bytes = kvh*136 for q8_0 and
 *                       kvh*256 for fp16 / bf16, at hd 128)
 *   arena_k, arena_v    device (HBM), arena_rows rows each (>= 128); buckets are
 *                       floor(arena_rows/2 / 64)*64 keys
 *   state               as kvt_attn_prefill_range (required)
 *   stream, copy_stream two different streams; the copies wait for everything enqueued on
 *                       `stream` before the call, and `stream` waits for each copy it reads,
 *                       so the op is ordered on `stream` like any other call.
 * The output equals kvt_attn_prefill's bit for bit.  The library keeps six events per host
 * thread (created on the first call on a device, then reused); calls from one thread are
 * ordered through them, so two calls on one thread must use the same `stream`.
 * Limits: as kvt_attn_prefill.
 * ---------------------------------------------------------------------------------------- */
int kvt_attn_prefill_pipelined(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh,
                               int32_t kvh, int32_t hd, const void *k_head, const void *v_head,
                               int64_t n_head, const void *k_host, const void *v_host,
                               int64_t n_kv, int32_t kv_format, int32_t causal, float scale,
                               void *arena_k, void *arena_v, int64_t arena_rows, void *state,
                               size_t state_bytes, float *out, void *stream, void *copy_stream);

/* ----------------------------------------------------------------------------------------
 * S7+S8 overlapped across layers.  [exl3-DMA]'s prefill streaming copies the next layer's
 * first batches into VRAM slots while the current layer runs.  kvt_attn_prefill_pipelined exposes the
 * copy of its first bucket whenever the HBM head is too short to hide it; in a chain of calls,
 * one per layer, each call can copy the next call's first host rows behind its own copies:
 *   next_k_host, next_v_host, next_arena_k, next_arena_v, next_arena_rows
 *                       the next call's k_host, v_host, arena_k, arena_v and arena_rows
 *   next_rows           host rows [0, next_rows) of the next call's planes (its rows
 *                       n_head ...) to copy into the start of its arena; 0 = no prefetch.
 *                       At most one bucket of the next arena.  Those rows must be final when
 *                       this call is enqueued; rows written later (this chunk's own keys, say)
 *                       are left to the next call.
 *   staged_rows         how many rows the previous call prefetched for this one (0 = none).
 *                       Must equal that call's next_rows, with the same planes and arena, and
 *                       fit this call's first bucket; else KVT_EINVAL and nothing enqueued.
 * Everything else as kvt_attn_prefill_pipelined, whose calls also take part: each call to
 * either entry point ends the previous prefetch of its thread, used or not, even when it
 * fails its checks.  Calls of a chain come from one host thread, in order, on the same
 * `stream`.  The prefetch waits for everything enqueued on `stream` before this call (the
 * previous layer's passes over the next arena), so the next arena must not overlap this
 * call's arena (KVT_EINVAL) and must not be read by anything this call reads: two arenas,
 * alternating between layers, are enough.  Outputs equal kvt_attn_prefill's bit for bit.
 * ---------------------------------------------------------------------------------------- */
int kvt_attn_prefill_chain(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh, int32_t kvh,
                           int32_t hd, const void *k_head, const void *v_head, int64_t n_head,
                           const void *k_host, const void *v_host, int64_t n_kv,
                           int32_t kv_format, int32_t causal, float scale, void *arena_k,
                           void *arena_v, int64_t arena_rows, int64_t staged_rows,
                           const void *next_k_host, const void *next_v_host, int64_t next_rows,
                           void *next_arena_k, void *next_arena_v, int64_t next_arena_rows,
                           void *state, size_t state_bytes, float *out, void *stream,
                           void *copy_stream);

/* ----------------------------------------------------------------------------------------
 * S7+S8 with the choice made by the library.  [exl3-DMA] decides per chunk whether host
 * memory is read in place or copied over first, by the chunk's token count (its minimum-token
 * rule for the DMA path); [llama-T] stages the tail once per op.  For attention over a tiered
 * cache the deciding quantity is time, not tokens: a short chunk has few workgroups, which
 * wait on scattered head slices across the link when reading in place, while the attention
 * itself is short, so copying the tail first (contiguously, at the link rate) pays; a long
 * chunk hides in-place reads or bucket copies behind its attention.
 *
 * kvt_attn_prefill_plan (host only, no device work) returns the plan, or a negative status:
 *   KVT_PREFILL_IN_PLACE   the tail is read where it lies (through the host mapping)
 *   KVT_PREFILL_STAGED     the whole tail is first copied into the arena (kvt_stage_tail,
 *                          mode AUTO, on `stream`), then attended from HBM
 *   KVT_PREFILL_PIPELINED  the tail copied in arena buckets on copy_stream while the previous
 *                          bucket is attended, as kvt_attn_prefill_pipelined
 * Rule.  No tail rows, or n_q == 0: IN_PLACE.  With two_streams nonzero and arena_rows >= 128:
 * STAGED when arena_rows >= n_kv - n_head and the modelled attention time is below a quarter
 * of the modelled staging time (too short to hide much), else PIPELINED.  With one stream:
 * STAGED when arena_rows >= n_kv - n_head and the modelled attention time is below the
 * modelled staging time, else IN_PLACE.  The model: staging
 * 2*(n_kv - n_head)*row_bytes at 56 GB/s; attention 4*hd*n_qh*pairs flop at 0.85 (q8_0), 0.98
 * (fp16) or 0.61 (bf16) PFLOP/s, pairs being the (query, key) pairs visited (causal: row t
 * sees min(n_kv, q_pos0 + t + 1) keys).  Every plan runs the attention in the key splits
 * kvt_attn_prefill_splitk takes for (n_q, n_qh, kvh, n_kv) -- s of them, one when the chunk's
 * own workgroups fill the chip; the pipelined plan carries each split's state from bucket to
 * bucket and merges the splits after the last.
 *
 * kvt_attn_prefill_auto: computes the plan (two_streams = stream and copy_stream differ;
 * arena_rows counts as 0 when arena_k or arena_v is NULL), writes it to *plan (optional,
 * host) and runs it.  Arguments as kvt_attn_prefill_pipelined, with ws (device,
 * kvt_attn_prefill_auto_ws_bytes(n_q, n_qh, kvh, n_kv) bytes, 4-byte aligned) serving as the
 * split-K workspace or the pipelined state; arena_k / arena_v may be NULL (no staging).
 *   conv, conv_bytes  optional (NULL, 0): device, 16-byte aligned, at least
 *          kvt_attn_prefill_conv_bytes(n_head, kvh, arena_rows, kv_format) bytes (0 unless
 *          the cache is q8_0).  Given that, a q8_0 cache on the pipelined plan has its rows
 *          converted to fp16 once -- the head at the start, each bucket as it lands in the
 *          arena -- and every pass runs on fp16 rows, when the modelled attention outlasts
 *          the conversion (the time it moves the cache's bytes at 4 TB/s).  The fp16 values are the
 *          ones the q8_0 kernel dequantises to, so the output is the same either way.
 * Output: kvt_attn_prefill_splitk's bits (kvt_attn_prefill's when s == 1), whichever plan is
 * taken and however the rows are split between head and tail.  A PIPELINED plan carries
 * kvt_attn_prefill_pipelined's thread rules (one stream per thread; it ends a pending chain
 * prefetch).  Limits: as kvt_attn_prefill.
 * ---------------------------------------------------------------------------------------- */
#define KVT_PREFILL_IN_PLACE 0
#define KVT_PREFILL_STAGED 1
#define KVT_PREFILL_PIPELINED 2
int kvt_attn_prefill_plan(int64_t n_q, int64_t q_pos0, int32_t n_qh, int32_t kvh, int64_t n_head,
                          int64_t n_kv, int32_t kv_format, int32_t causal, int64_t arena_rows,
                          int32_t two_streams);
size_t kvt_attn_prefill_auto_ws_bytes(int64_t n_q, int32_t n_qh, int32_t kvh, int64_t n_kv);
size_t kvt_attn_prefill_conv_bytes(int64_t n_head, int32_t kvh, int64_t arena_rows,
                                   int32_t kv_format);
int kvt_attn_prefill_auto(const void *q, int64_t n_q, int64_t q_pos0, int32_t n_qh, int32_t kvh,
                          int32_t hd, const void *k_head, const void *v_head, int64_t n_head,
                          const void *k_host, const void *v_host, int64_t n_kv,
                          int32_t kv_format, int32_t causal, float scale, void *arena_k,
                          void *arena_v, int64_t arena_rows, void *ws, size_t ws_bytes,
                          void *conv, size_t conv_bytes, float *out, int32_t *plan,
                          void *stream, void *copy_stream);

/* ----------------------------------------------------------------------------------------
 * Transfer worker.  [vLLM-CPU] SingleDirectionOffloadingHandler: transfer_async,
 * get_finished, wait, shutdown.  One worker per direction (KVT_H2D loads, KVT_D2H stores)
 * keeps the transfers submitted to it in order.  kvt_worker_create takes the copy mode AUTO,
 * KERNEL or RUNTIME (SDMA waits on the host, which a worker never does: KVT_EUNSUPPORTED).
 *   - kvt_worker_submit copies the caller's src/dst/sizes tables (host memory, any kind) into
 *     a pooled pinned buffer, so the caller may reuse its tables as soon as it returns; takes
 *     a stream and two timing events from the worker's pools; makes that stream wait for all
 *     work enqueued so far on `compute_stream` (NULL = legacy default stream) and for the end
 *     of the previous transfer of this worker; then enqueues start event, kvt_swap_blocks
 *     (mode from create; same table rules) and end event.  job_id is the caller's tag and
 *     must not match a job still pending in this worker (KVT_EINVAL).  n == 0 is allowed
 *     (an ordering-only job of 0 bytes).
 *   - kvt_worker_get_finished reports, oldest first, up to `max` jobs whose end event has
 *     passed, stopping at the first one still running (completion is reported in submission
 *     order): job_ids[i], bytes[i] (sum of its sizes) and seconds[i] (start->end event time).
 *     bytes / seconds may be NULL.  A reported job's stream, events and buffer return to the
 *     pools.  *n_out receives the count.
 *   - kvt_worker_wait blocks the calling thread until the transfers of job_ids[0..n) have
 *     finished; ids that are unknown or already reported are skipped.  It reports nothing.
 *   - kvt_worker_pending returns how many jobs are submitted and not yet reported (or < 0).
 *   - kvt_worker_reserve grows the pools to hold `jobs` transfers in flight whose tables have
 *     up to `entries` rows each, so later submits within that allocate nothing.
 *   - kvt_worker_destroy (shutdown) waits for the pending jobs in order, releases the pools
 *     and frees the worker.  If a wait fails, the later jobs are not waited for and that
 *     error is returned (the worker is freed all the same).
 * A worker belongs to the device current at create; its calls are thread-safe.  Errors:
 * KVT_EINVAL (arguments), KVT_ENOMEM (pinned allocation), KVT_EHIP, or kvt_swap_blocks's own.
 * ---------------------------------------------------------------------------------------- */
typedef struct kvt_worker kvt_worker;
int kvt_worker_create(int32_t dir, int32_t mode, kvt_worker **out);
int kvt_worker_reserve(kvt_worker *w, int32_t jobs, int64_t entries);
int kvt_worker_submit(kvt_worker *w, int64_t job_id, const uint64_t *src, const uint64_t *dst,
                      const uint64_t *sizes, int64_t n, void *compute_stream);
int kvt_worker_get_finished(kvt_worker *w, int64_t *job_ids, uint64_t *bytes, double *seconds,
                            int32_t max, int32_t *n_out);
int kvt_worker_wait(kvt_worker *w, const int64_t *job_ids, int32_t n);
int kvt_worker_pending(kvt_worker *w);
int kvt_worker_destroy(kvt_worker *w);

/* ----------------------------------------------------------------------------------------
 * Paged writes.  [QSA-KVO] CacheLayer_qsa_offload docstring: new tokens reach the host-
 * resident K/V planes (and the indexer's raw key plane) through the paged cache update, which
 * addresses them by base pointer plus offsets.  The update's source is not on the page; this
 * is the plain paged-cache rule.  Each plane is dense pages [n_pages][page_size][row_bytes];
 * token t of sequence b (position p = cache_seqlens[b] + t) goes to row p % page_size of page
 * block_table[b*pages_per_seq + p / page_size]:
 *   dst[i] + (page*page_size + p % page_size)*row_bytes[i]  <-  src[i] + (b*seq + t)*row_bytes[i]
 *   src, dst, row_bytes: host arrays of n_planes (1..4) entries.  src[i]: device rows
 *     [bsz][seq][row_bytes[i]] (HBM); dst[i]: device pointer of the plane (host-mapped or HBM).
 *   cache_seqlens: device int32 [bsz] (the tokens each sequence holds before this write);
 *   block_table: device int32 [bsz][pages_per_seq].
 * Rows whose sequence length is negative, whose page slot is >= pages_per_seq or whose page
 * id lies outside [0, n_pages) are skipped.  Two tokens must not map to the same row.
 * row_bytes % 16 == 0, planes 16-byte aligned.  Errors: KVT_EINVAL, KVT_EALIGN, KVT_ERANGE.
 * ---------------------------------------------------------------------------------------- */
int kvt_paged_write(const void *const *src, void *const *dst, const int64_t *row_bytes,
                    int32_t n_planes, int32_t bsz, int32_t seq, const int32_t *cache_seqlens,
                    const int32_t *block_table, int32_t pages_per_seq, int32_t page_size,
                    int64_t n_pages, void *stream);

/* ----------------------------------------------------------------------------------------
 * Page copy.  [QSA-KVO] CacheLayer_qsa_offload.copy_page: after draining `stream` (a page
 * being read may still wait on a queued write, and one being written may still be under a
 * read), the first num_tokens rows of page from_page of each host plane are copied to page
 * to_page on the CPU (memmove), leaving the host link to the attention gather; then the
 * page's first ceil(num_tokens / cr) pooled rows are copied on the device, enqueued on stream.
 *   src_host, dst_host, row_bytes: host arrays of n_planes (0..4) entries; planes are dense
 *     pages [n_pages][page_size][row_bytes[i]] given by their host addresses.
 *   src_pooled, dst_pooled: device planes [n_pages][page_size/cr][pooled_row_bytes], or both
 *     NULL to skip.  cr must divide page_size.
 * Blocks the calling thread until the stream is idle; not for use under graph capture.
 * ---------------------------------------------------------------------------------------- */
int kvt_copy_page(const void *const *src_host, void *const *dst_host, const int64_t *row_bytes,
                  int32_t n_planes, int64_t from_page, int64_t to_page, int32_t page_size,
                  int32_t num_tokens, const void *src_pooled, void *dst_pooled,
                  int64_t pooled_row_bytes, int32_t cr, void *stream);

/* ----------------------------------------------------------------------------------------
 * Pool rebuild at the write head.  [QSA-KVO] CacheLayer_qsa_offload docstring: the raw key
 * plane is read only around the write head, where the pool kernel rebuilds the pooled blocks
 * an append touched.  The page does not give the pooling function; here a block's pooled key
 * is the mean of the raw key rows it holds, per element: the rows' exact sum (fp64), divided
 * by their count, rounded once to fp16 (to nearest, ties to even; NaN gives 0x7E00).
 *   Call after kvt_paged_write has placed the raw rows of an append of seq tokens, with the
 *   same cache_seqlens (the lengths before the append) and block table.  For sequence b,
 *   len = cache_seqlens[b] (< 0: skipped); blocks j = len/cr ... (len+seq-1)/cr are rebuilt,
 *   each from rows [j*cr, min(j*cr + cr, len + seq)) -- the write head's partial block from
 *   the rows it has so far.  Block j lies in page block_table[b][(j*cr) / page_size]
 *   (skipped when that slot is past pages_per_seq or the entry is outside [0, n_pages)).
 *   raw_k   fp16 [n_pages][page_size][dim], device pointer (host-mapped or HBM)
 *   pooled  fp16 [n_pages][page_size/cr][dim], device pointer (HBM); pooled row
 *           ((j*cr) % page_size) / cr of the block's page is written, no other
 * Limits: 1 <= cr <= 512, cr divides page_size; planes 2-byte aligned.  Enqueued on stream.
 * ---------------------------------------------------------------------------------------- */
int kvt_pool_rebuild(const void *raw_k, void *pooled, int32_t dim, int32_t bsz, int32_t seq,
                     const int32_t *cache_seqlens, const int32_t *block_table,
                     int32_t pages_per_seq, int32_t page_size, int32_t cr, int64_t n_pages,
                     void *stream);

/* ----------------------------------------------------------------------------------------
 * Workspace sizes by operation: one entry point over the *_ws_bytes / *_state_bytes calls
 * above, for callers that size buffers generically.  dims per op:
 *   KVT_OP_INDEX_TOPK     {n_blocks, n_sel, k}          = kvt_index_topk_ws_bytes
 *   KVT_OP_ATTN_DECODE    {n_qh, hd, n_kv}              = kvt_attn_decode_ws_bytes (also the
 *                                                          fused pass, with n_kv = k * bt)
 *   KVT_OP_SPARSE_ROWS    {rows, n_qh, kvh, k_pad}      = kvt_sparse_attend_rows_ws_bytes
 *   KVT_OP_PREFILL_STATE  {n_q, n_qh, kvh}              = kvt_attn_prefill_state_bytes
 *   KVT_OP_NONE_NEEDED    any dims                      = 0 (swap, gather, staging, single-pass
 *                                                          prefill take no workspace)
 * Returns 0 as well for an unknown op, a wrong dims count or a dimension outside its type;
 * kvt_last_error() then names the problem.
 * ---------------------------------------------------------------------------------------- */
#define KVT_OP_NONE_NEEDED 0
#define KVT_OP_INDEX_TOPK 1
#define KVT_OP_ATTN_DECODE 2
#define KVT_OP_SPARSE_ROWS 3
#define KVT_OP_PREFILL_STATE 4
size_t kvt_workspace_bytes(int32_t op, const int64_t *dims, int32_t n_dims);

#ifdef __cplusplus
}
#endif
#endif /* KVT_H */
