/*
 * mla_decode.h -- C ABI of the MI355X (gfx950) library for Multi-head Latent
 * Attention (MLA) decoding over a paged latent KV cache.
 *
 * The operation (FlashMLA pages):
 *   - "FlashMLA: DeepSeek's efficient MLA decoding kernel" (geoz.com.cn), usage
 *     example section: metadata is computed once per decode step from
 *     cache_seqlens, s_q*h_q/h_kv and h_kv, then the decode call runs once per
 *     layer with q, the layer's KV cache, block_table, cache_seqlens and d_v and
 *     returns o and lse; the cache is paged in 64-token blocks (main features).
 *   - "FlashMLA attention kernel source walk-through: the 656-byte KV cache"
 *     (bjdmk.com.cn): scheduling section (a small kernel spreads
 *     (request, KV block range) units over all compute units ahead of time; the
 *     main kernel only follows it; long sequences are split and merged; the
 *     metadata can be reused while shapes and lengths are unchanged); decode
 *     call example (get_mla_metadata also takes h_q, is_fp8 and topk, and the
 *     decode call takes is_fp8 and indices); data-loading section (the 656-byte
 *     FP8 token); combine section (each split leaves a partial o and lse).
 *   - agentlenshq.com FlashMLA summary, technical details: indices is a 3-D
 *     int32 tensor and -1 entries are ignored.
 *
 * Model: one KV head (h_kv = 1); each token stores a 576-dim latent that is K;
 * its first 512 dims are V.  For query row (b, s, h):
 *   T = [0, cache_seqlens[b]) (dense), or the non-(-1) entries of
 *       indices[b, s, 0:topk] (sparse; logical positions, looked up through
 *       block_table; duplicates count with multiplicity);
 *   o = softmax(softmax_scale * q K_T^T) V_T,  lse = ln sum exp(softmax_scale * q K_T^T).
 *   An empty T gives o = 0 and lse = -inf.  Decoding is non-causal.
 *
 * Memory: every pointer argument of the compute calls is a device pointer into
 * memory the caller owns; the library allocates nothing per call and keeps no
 * per-call state.  All tensors are dense, row-major, naturally aligned (16-byte
 * aligned bases for q, kvcache, o and the workspace).
 *
 * Errors: every call returns MLA_OK (0) or a negative MLA_ERR_* code.  When a
 * call returns an error that the host detected, nothing was launched;
 * mla_last_error() then describes the failure (thread-local string).  Faults
 * inside kernels (a precondition broken, see below) surface at the caller's
 * next stream synchronisation.  No C++ exception crosses this interface.
 *
 * Streams: compute calls are asynchronous on the given hipStream_t (NULL = the
 * default stream) and do not synchronise the host.
 */
#ifndef MLA_DECODE_H
#define MLA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_API __attribute__((visibility("default")))

#define MLA_OK 0
#define MLA_ERR_INVALID_ARG (-1)         /* null pointer, non-positive size, inconsistent arguments */
#define MLA_ERR_UNSUPPORTED (-2)         /* d_qk != 576, d_v != 512, h_kv != 1 */
#define MLA_ERR_BUFFER_TOO_SMALL (-3)    /* metadata or workspace smaller than the size call reported */
#define MLA_ERR_HIP (-4)                 /* a HIP runtime call or kernel launch failed */

#define MLA_PAGE_TOKENS 64
#define MLA_D_QK 576
#define MLA_D_V 512
#define MLA_FP8_TOKEN_BYTES 656

/*
 * Sizes of the two caller-owned scratch buffers for one (B, s_q, h_q, topk,
 * num_workers) shape.
 *   B            requests (>= 1)
 *   s_q, h_q     query tokens per request and query heads (>= 1)
 *   h_kv         KV heads; must be 1
 *   topk         0 = dense decode; > 0 = sparse decode with topk index slots
 *   num_workers  KV workers the schedule spreads tiles over; 0 = automatic
 *                (one per compute unit of the current device; this makes a
 *                HIP device query)
 * On success *metadata_bytes holds the metadata size, *workspace_bytes the split
 * workspace size (partial outputs and lse of split sequences), and
 * *num_workers_out (may be NULL) the worker count actually used.
 */
MLA_API int mla_get_metadata_size(int B, int s_q, int h_q, int h_kv, int topk, int num_workers,
                                  size_t* metadata_bytes, size_t* workspace_bytes, int* num_workers_out);

/*
 * Scheduler: spreads the (request, KV tile range) work of a decode step over
 * num_workers workers (one launch of a single-workgroup kernel on `stream`).
 *   cache_seqlens  device int32 [B], tokens cached per request (>= 0)
 *   is_fp8         1 if the cache will be the 656-byte FP8 layout, else 0 (checked
 *                  to be 0 or 1).  The split rule is the same for both caches
 *                  (measured: the cache type did not change the best split):
 *                  the finest balanced split, one workgroup per compute unit,
 *                  with splits of at least 4 tiles (256 tokens or index slots)
 *                  for streams of more than 64 query rows and 2 tiles otherwise
 *   metadata       device buffer of metadata_bytes (>= the size call's value);
 *                  written entirely by the kernel
 * The metadata stays valid for every layer's decode call while cache_seqlens,
 * B, s_q, h_q, topk, is_fp8 and num_workers are unchanged; reusing it after a
 * length change gives wrong results (not detected).  It also holds one arrival
 * counter per (stream, 64-row tile), zeroed here, that merging decode calls
 * (mla_set_merge_mode) use and leave at zero: merging decode calls that share
 * one metadata buffer must therefore not run at the same time (issue them on
 * one stream, as the layers of a step are).
 */
MLA_API int mla_get_metadata(const int32_t* cache_seqlens, int B, int s_q, int h_q, int h_kv, int topk, int is_fp8,
                             int num_workers, int32_t* metadata, size_t metadata_bytes, void* stream);

/*
 * Decode: split-KV attention over the paged cache, then the lse combine of
 * split sequences.
 *   q              device bf16 [B, s_q, h_q, 576]
 *   kvcache        device; bf16 [num_blocks, 64, 576] when is_fp8 == 0, else
 *                  uint8 [num_blocks, 64, 656]: bytes 0..511 e4m3fn codes
 *                  (byte d = dim d), 512..527 four little-endian fp32 scales
 *                  (scale t covers dims [128 t, 128 t + 128)), 528..655 dims
 *                  512..575 as little-endian bf16.  An element decodes to
 *                  bf16_rne(fp32_rne(e4m3(code) * scale)).
 *   block_table    device int32 [B, max_blocks]; logical token j of request b is
 *                  row j % 64 of page block_table[b, j / 64]
 *   cache_seqlens  device int32 [B] (the same values the metadata was built from)
 *   softmax_scale  <= 0 selects 1 / sqrt(576)
 *   metadata       from mla_get_metadata with the same shape and num_workers;
 *                  read, and in the merging mode (mla_set_merge_mode) its
 *                  arrival counters are updated and left at zero
 *   indices        device int32 [B, s_q, topk] when topk > 0, else NULL
 *   causal         0 or 1; 1 (dense only, else MLA_ERR_INVALID_ARG) masks the
 *                  attention of speculative query tokens: the s_q query tokens
 *                  are the last s_q cache positions, so query token s sees
 *                  positions j <= seqlen_b - s_q + s (none when negative: o = 0,
 *                  lse = -inf).  The usage example of "FlashMLA: DeepSeek's
 *                  efficient MLA decoding kernel" passes causal=True for
 *                  autoregressive decoding.
 *   workspace      device buffer of workspace_bytes (>= the size call's value);
 *                  no initial contents needed.  A split row that attends no
 *                  token writes only its lse (-inf), not its partial output,
 *                  and the combine gives it weight 0
 *   o              device bf16 [B, s_q, h_q, 512] (output)
 *   lse            device fp32 [B, s_q, h_q] (output, natural log)
 * Preconditions not checked on the device: indices in {-1} U [0, seqlen_b);
 * block_table entries read for a request (the first ceil(seqlen_b / 64), or
 * those its indices reach) lie in [0, num_blocks); buffers do not overlap.
 * Tokens that no query row attends (page tails, unused pages, skipped slots)
 * are never read and may hold any bytes, NaN included.
 */
MLA_API int mla_decode_with_kvcache(const void* q, const void* kvcache, int64_t num_blocks, const int32_t* block_table,
                                    int max_blocks, const int32_t* cache_seqlens, int B, int s_q, int h_q, int h_kv,
                                    int d_qk, int d_v, float softmax_scale, int32_t* metadata,
                                    size_t metadata_bytes, int num_workers, const int32_t* indices, int topk,
                                    int is_fp8, int causal, void* workspace, size_t workspace_bytes, void* o,
                                    float* lse, void* stream);

/*
 * Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  The same computation, arguments and errors as
 * mla_decode_with_kvcache, without the workspace arguments: the split workspace
 * (partial outputs and their lse) lives in a static device array of
 * MLA_NOALLOC_SCRATCH_BYTES inside the library, one copy per GPU, held until the
 * process ends.  The caller still passes the inputs, the metadata and o / lse.
 * Shapes whose workspace (mla_get_metadata_size's workspace_bytes) exceeds
 * MLA_NOALLOC_SCRATCH_BYTES are refused with MLA_ERR_UNSUPPORTED before any
 * launch.  The call never allocates: the array's device address is looked up
 * (hipGetSymbolAddress) on the first call on each device and kept.  Every call
 * on one GPU shares that GPU's array, so calls that overlap in time on one GPU
 * (concurrent streams, several host threads) race and give wrong results;
 * calls ordered on one stream are safe.  Nothing in the array needs clearing
 * between calls: each call writes every workspace value it uses.
 */
#define MLA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
MLA_API int mla_decode_with_kvcache_noalloc(const void* q, const void* kvcache, int64_t num_blocks,
                                            const int32_t* block_table, int max_blocks, const int32_t* cache_seqlens,
                                            int B, int s_q, int h_q, int h_kv, int d_qk, int d_v, float softmax_scale,
                                            int32_t* metadata, size_t metadata_bytes, int num_workers,
                                            const int32_t* indices, int topk, int is_fp8, int causal, void* o,
                                            float* lse, void* stream);

/*
 * Sparse prefill: token-sparse attention of many query tokens over one
 * contiguous latent KV sequence ("FlashMLA" summary on agentlenshq.com, usage
 * section, the sparse prefill call flash_mla_sparse_fwd(q, kv, indices, ...):
 * a query tensor, the KV and a 3-D index tensor naming the KV tokens each query
 * token attends; zhouruolin.cn FlashMLA page, test section, sparse prefill).
 * The pages leave the rest open; this call reads it plainly: BF16 KV, one KV
 * head, and per query row s the same rule as sparse decoding,
 *   o = softmax(softmax_scale * q K_T^T) V_T,  lse = ln sum exp(softmax_scale * q K_T^T),
 * with T the non-(-1) entries of indices[s, 0:topk] (duplicates count with
 * multiplicity; an empty T gives o = 0, lse = -inf).
 *   q          device bf16 [s_q, h_q, 576]
 *   kv         device bf16 [s_kv, 576] (token j = row j; h_kv = 1)
 *   indices    device int32 [s_q, topk], entries in {-1} U [0, s_kv) (not
 *              checked on the device)
 *   o, lse     device bf16 [s_q, h_q, 512] and fp32 [s_q, h_q] (outputs)
 *   workspace  device buffer of the size call's workspace_bytes: the call
 *              writes the sequence's page table and the schedule there, then
 *              runs the sparse decode path on it (four launches on `stream`)
 * num_workers and softmax_scale as for mla_decode_with_kvcache.  Errors as for
 * the other calls; nothing is launched when one is returned.
 */
MLA_API int mla_sparse_prefill_workspace_size(int s_q, int h_q, int h_kv, int64_t s_kv, int topk, int num_workers,
                                              size_t* workspace_bytes, int* num_workers_out);
MLA_API int mla_sparse_prefill(const void* q, const void* kv, int64_t s_kv, const int32_t* indices, int s_q, int h_q,
                               int h_kv, int topk, int d_qk, int d_v, float softmax_scale, int num_workers,
                               void* workspace, size_t workspace_bytes, void* o, float* lse, void* stream);

/* Thread-local, NUL-terminated description of this thread's last failed call ("" if none). */
MLA_API const char* mla_last_error(void);

/*
 * Where a decode call merges the partial results of split streams (FlashMLA
 * source walk-through, combine section: split results are folded by their lse
 * in a combine step, whose launch gap the pages' kernels hide by overlapping
 * the two kernels).  Modes, for the calling thread's later decode calls:
 *   MLA_MERGE_OFF  (default) the combine kernel, launched after the decode
 *                  kernel on the same stream
 *   MLA_MERGE_ON   the decode kernel merges, where the host can prove that no
 *                  stream has more than 4 splits (sparse: from topk and the
 *                  worker count; dense: from max_blocks; otherwise the combine
 *                  kernel runs): each split writes its partial output through to
 *                  memory and counts itself in on the metadata's arrival counter
 *                  of its 64-row tile; the last split of the tile to arrive
 *                  merges the stream's splits and writes o and lse, and no
 *                  combine kernel is launched.  On MI355X this measured 1-9 us
 *                  slower per call than the combine kernel on every shape tried
 *                  (small calls included: its device-coherent writes, the count
 *                  and the merge's reads are serial memory round trips), so it
 *                  is an option, not the default.
 * Results are bit-identical in both modes.  Returns MLA_ERR_INVALID_ARG for any
 * other value.
 */
#define MLA_MERGE_OFF 0
#define MLA_MERGE_ON 1
MLA_API int mla_set_merge_mode(int mode);

/*
 * Bench hook: timing of the split-KV decode kernel alone.  While set on the
 * calling thread (both non-NULL hipEvent_t handles created by the caller),
 * each mla_decode_with_kvcache call records `start` on its stream right before
 * the decode kernel and `stop` right after it, ahead of the combine launch.
 * Passing NULL for both clears the hook.  Returns MLA_ERR_INVALID_ARG when
 * exactly one of the two is NULL.  The events stay owned by the caller.
 */
MLA_API int mla_set_decode_kernel_events(void* start, void* stop);

/*
 * Test hook: the FP8 -> bf16 decode the decode kernel applies, exported for
 * bit-exact checking.  tokens: device uint8 [n, 656]; out: device bf16
 * [n, 576] = the decoded 512 dims followed by the 64 RoPE dims copied verbatim.
 */
MLA_API int mla_debug_dequant_fp8(const uint8_t* tokens, int64_t n, void* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_DECODE_H */
