/*
 * ring_attention_chunk.h -- C ABI of the MI355X (gfx950) ring-attention library.
 *
 * The library computes one device's share of ring attention on one GPU: the
 * local queries attend to a list of key/value chunks that are already resident
 * in device memory, visited in list order (the ring order). Three calls follow
 * the exercise page "systems-distributed-ring-attention-online-softmax"
 * (problem statement): per-chunk online-softmax statistics, the merge of two
 * statistics, and the whole ring pass with one normalisation at the end.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - All pointers to tensors are DEVICE pointers owned by the caller. The
 *    library allocates no device memory. Host pointers (descriptor arrays)
 *    need to stay valid only for the duration of the call: the descriptor
 *    tables reach the device as kernel arguments of small copy kernels,
 *    which the runtime captures when each launch is enqueued, so nothing
 *    reads host memory after a call returns (no host-to-device memcpy, no
 *    pinned staging).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL means the
 *    default stream). A status of RA_OK means the work was enqueued; faults
 *    inside kernels surface at the caller's next synchronisation.
 *  - Every argument is validated on the host before any HIP call. On error a
 *    call returns a nonzero status, enqueues nothing, and leaves a message for
 *    ra_last_error() (per host thread). Calls never abort or print.
 *  - Scores are s = scale * <q, k>, in natural-log units; scale must be finite
 *    and > 0 (1/sqrt(head_dim) is the usual choice).
 *  - Element types: RA_BF16 inputs use bf16 matrix cores with fp32
 *    accumulation; RA_F32 inputs use fp32 matrix cores. All statistics and
 *    outputs are fp32.
 *  - head_dim is 1..128; q_heads must be a multiple of kv_heads (query head h
 *    reads key/value head h / (q_heads / kv_heads)).
 *  - Global positions (every position a chunk or query segment describes)
 *    must lie in [0, 2^31 - 2]; the total number of keys must be < 2^31.
 *
 * Layouts
 * -------
 *  q          [batch, q_heads, q_len, head_dim], contiguous, element type dtype.
 *  chunk      per chunk: key row j of batch b, kv head h starts at element
 *             b*stride_b + h*stride_h + j*stride_s of `k` (and of `v`, which
 *             shares the strides); the head_dim elements of a row are
 *             contiguous. A chunk can therefore be a slice of a larger
 *             [batch, kv_heads, n, head_dim] buffer without a copy.
 *  u, out     [batch, q_heads, q_len, head_dim] fp32, contiguous.
 *  l, m, lse  [batch, q_heads, q_len] fp32, contiguous.
 *  Output buffers must not overlap any input.
 */
#ifndef RING_ATTENTION_CHUNK_H
#define RING_ATTENTION_CHUNK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum ra_status {
  RA_OK = 0,
  RA_ERR_NULL = 1,        /* a required pointer is NULL                        */
  RA_ERR_SHAPE = 2,       /* sizes, strides, offsets or lengths are invalid    */
  RA_ERR_DTYPE = 3,       /* unknown element type                              */
  RA_ERR_UNSUPPORTED = 4, /* valid request outside what the kernels implement  */
  RA_ERR_HIP = 5,         /* the HIP runtime refused a copy or a launch        */
  RA_ERR_WORKSPACE = 6    /* workspace missing or smaller than required        */
};

enum ra_dtype { RA_F32 = 0, RA_BF16 = 1 };

/* One key/value chunk: keys whose global positions form the progression
 * global_offset + pos_stride * j, j = 0..len-1 ("Ring Attention: Distributed
 * Reads with Online Softmax", section "Causal masks depend on global
 * positions": shard metadata carries global positions). pos_stride 1 (or 0,
 * read as 1) is a contiguous run; pos_stride P is a striped shard, whose keys
 * are every P-th token of the sequence (glossary "ring attention",
 * paragraph Variants: striped attention). Memory strides are in elements;
 * stride_s >= head_dim. */
typedef struct ra_kv_chunk {
  const void* k;
  const void* v;
  int64_t len;           /* keys in this chunk, >= 0 (0 contributes nothing) */
  int64_t global_offset; /* global position of the chunk's first key         */
  int64_t stride_b;
  int64_t stride_h;
  int64_t stride_s;
  int64_t pos_stride;    /* position step between consecutive keys, >= 0     */
} ra_kv_chunk;

/* A run of local query rows whose global positions are global_offset +
 * pos_stride * i (pos_stride 0 is read as 1). A contiguous share is one
 * segment with step 1; a paired early/late ("zigzag") share is two; a striped
 * share is one segment with step P. */
typedef struct ra_q_segment {
  int64_t len;
  int64_t global_offset;
  int64_t pos_stride;
} ra_q_segment;

/* attention_chunk_stats(query, key_chunk, value_chunk) -> (u, l, m).
 * Exercise page, problem statement and hint 1: for every query row, the
 * un-normalised weighted value sum u, the un-normalised softmax denominator l
 * and the row-wise maximum score m over this one chunk, computed as if it were
 * the only chunk (no mask). u is relative to m: u = sum_j exp(s_j - m) v_j,
 * l = sum_j exp(s_j - m). A chunk of length 0 yields (0, 0, -inf).
 * Writes u [B,Hq,q_len,d], l and m [B,Hq,q_len].
 *  workspace   optional device buffer (NULL, or 256-byte aligned) of
 *              workspace_bytes. With at least ra_chunk_stats_workspace_bytes(...)
 *              bytes, a grid too small to fill the GPU is completed by cutting
 *              the chunk's keys into ranges whose partial statistics are merged
 *              afterwards on `stream`; with less (or NULL) the call runs
 *              uncut. The results agree to rounding either way; for a given
 *              shape and workspace they are bit-identical from run to run. */
int ra_attention_chunk_stats(int dtype, int batch, int q_heads, int kv_heads, int head_dim,
                             const void* q, int64_t q_len, const ra_kv_chunk* chunk,
                             float scale, float* u, float* l, float* m,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Device workspace, in bytes, with which ra_attention_chunk_stats cuts the
 * keys into ranges for this shape: fp32 partial statistics, (head_dim + 2)
 * values per row and range. 0 when the query rows fill the GPU on their own
 * (a multiple of 256 otherwise). */
size_t ra_chunk_stats_workspace_bytes(int batch, int q_heads, int head_dim, int64_t q_len, int64_t chunk_len);

/* merge_chunk_stats(acc, chunk), in place on acc.
 * Exercise page, hint 2 ("rescale to the shared new max"): with
 * m' = max(m_acc, m_chunk), both sides are multiplied by exp(own_max - m')
 * before adding: l' = a l_acc + b l_chunk, u' = a u_acc + b u_chunk, m' as
 * above. Two -inf maxima give the identity (0, 0, -inf). rows is the number of
 * (batch, head, query) rows; u has head_dim floats per row. acc_* are read and
 * overwritten; the chunk arrays must not overlap them. */
int ra_merge_chunk_stats(int64_t rows, int head_dim, float* acc_u, float* acc_l, float* acc_m,
                         const float* u, const float* l, const float* m, void* stream);

/* Device workspace, in bytes, that ra_ring_attention needs for this shape:
 * the chunk descriptor and query segment tables and, when the query tiles
 * alone cannot fill the GPU, room for per-key-range partial statistics
 * (fp32, (head_dim + 2) values per row and range). A multiple of 256. */
size_t ra_ring_workspace_bytes(int batch, int q_heads, int head_dim, int64_t q_len, int64_t total_keys,
                               int n_chunks, int n_q_segments);

/* ring_attention(query, key_chunks, value_chunks, q_global_offset,
 * kv_global_offsets, causal) -> normalised output.
 * Exercise page, problem statement: the result equals ordinary softmax
 * attention over the concatenation of the chunks in list order, for any split
 * of that sequence into chunks; the blog post's "A simple forward schedule"
 * keeps one running (m, l, u) per query across all chunks and divides u / l
 * once at the end. With causal != 0 a key is allowed for a query when its
 * global position is <= the query's (section "Causal masks depend on global
 * positions"). Rows with no allowed key give out = 0 and lse = -inf.
 *  q_segments  host array of n_q_segments runs whose lengths sum to q_len
 *              (n_q_segments >= 1); positions matter only when causal.
 *  chunks      host array of n_chunks descriptors in ring order (n_chunks >= 0).
 *  workspace   device buffer of >= ra_ring_workspace_bytes(batch, q_heads,
 *              head_dim, q_len, total_keys, n_chunks, n_q_segments) bytes,
 *              256-byte aligned, where total_keys is the sum of the chunk
 *              lengths; the descriptor tables are copied there on `stream`
 *              (stream-ordered) and partial statistics may be written there,
 *              so two calls on one stream may share it, calls on different
 *              streams may not.
 *  out         [B,Hq,q_len,d] fp32; lse [B,Hq,q_len] fp32 or NULL.
 * For a fixed ordered key sequence the output is bit-identical for every split
 * of that sequence into chunks and from run to run. */
int ra_ring_attention(int dtype, int batch, int q_heads, int kv_heads, int head_dim,
                      const void* q, const ra_q_segment* q_segments, int n_q_segments,
                      const ra_kv_chunk* chunks, int n_chunks, int causal, float scale,
                      void* workspace, size_t workspace_bytes, float* out, float* lse,
                      void* stream);

/* Size, in bytes, of the device array that ra_ring_attention_noalloc uses as
 * its workspace (one per GPU, held until the process ends). */
#define RA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/* ra_ring_attention for callers that cannot allocate device memory or pass a
 * workspace: code under HIP stream capture, tight serving loops, harnesses
 * that forbid allocation. Same arguments, meaning and results as
 * ra_ring_attention (bit-identical output and lse), without the workspace:
 * the descriptor tables and key-range partials go to a file-scope device
 * array of RA_NOALLOC_SCRATCH_BYTES that each GPU the library runs on holds
 * until the process ends. The call allocates nothing (no hipMalloc, hipFree
 * or allocating library routine, no host allocation). The first call on a
 * device, with that device current, looks up the array's address there
 * (hipGetSymbolAddress); make that first call outside stream capture.
 * Returns RA_ERR_WORKSPACE, before any HIP call, when the tables and
 * key-range partials of the call exceed RA_NOALLOC_SCRATCH_BYTES (they never
 * exceed ra_ring_workspace_bytes(...) for the call).
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind; each call writes every byte it reads on its own stream first, so
 * nothing needs clearing, but calls that overlap on one GPU (on different
 * streams, or from several host threads) race and must be serialised by the
 * caller. The stream must belong to the current device. */
int ra_ring_attention_noalloc(int dtype, int batch, int q_heads, int kv_heads, int head_dim,
                              const void* q, const ra_q_segment* q_segments, int n_q_segments,
                              const ra_kv_chunk* chunks, int n_chunks, int causal, float scale,
                              float* out, float* lse, void* stream);

/* Device workspace, in bytes, that ra_ring_attention_block_sparse needs for
 * this shape and a block mask of n_qblocks x n_kblocks: that of
 * ra_ring_attention, plus the mask packed one bit per block and, per query
 * tile, the list of key tiles to visit. A multiple of 256. */
size_t ra_block_sparse_workspace_bytes(int batch, int q_heads, int head_dim, int64_t q_len, int64_t total_keys,
                                       int n_chunks, int n_q_segments, int64_t n_qblocks, int64_t n_kblocks);

/* ring_attention under a block-sparse mask.
 * "Ring Attention: Distributed Reads with Online Softmax", section "What is
 * preserved, what is distributed?": the method composes with tiled kernels
 * and sparse patterns. The pages give no pattern; here it is a block mask over
 * GLOBAL positions (like the causal mask, section "Causal masks depend on
 * global positions"), so it means the same on every device and for every
 * split of the keys into chunks: positions fall into query blocks of block_q
 * and key blocks of block_k positions, and a key at position k is allowed for
 * a query at position p when block_mask[p / block_q][k / block_k] != 0 and,
 * with causal != 0, k <= p. The result is ordinary attention restricted to the
 * allowed keys; rows with none give out = 0 and lse = -inf.
 *  block_mask  DEVICE pointer, row-major bytes [n_qblocks][n_kblocks] (any
 *              nonzero byte allows the block pair), read on `stream` during
 *              the call; every query and key position must lie below
 *              n_qblocks * block_q and n_kblocks * block_k.
 *  block_q, block_k  powers of two, 1 .. 2^30.
 *  workspace   >= ra_block_sparse_workspace_bytes(...) bytes, 256-byte
 *              aligned: the descriptor tables, the packed mask and the key
 *              tiles each query tile visits are built there on `stream`.
 * Other arguments as for ra_ring_attention. Key tiles with no allowed pair for
 * any query of a workgroup are not visited; visited tiles are masked per key.
 * For a fixed ordered key sequence the output is bit-identical for every split
 * of it into chunks, and with an all-ones mask it is ra_ring_attention's. */
int ra_ring_attention_block_sparse(int dtype, int batch, int q_heads, int kv_heads, int head_dim,
                                   const void* q, const ra_q_segment* q_segments, int n_q_segments,
                                   const ra_kv_chunk* chunks, int n_chunks, int causal, float scale,
                                   const uint8_t* block_mask, int64_t n_qblocks, int64_t n_kblocks,
                                   int64_t block_q, int64_t block_k, void* workspace, size_t workspace_bytes,
                                   float* out, float* lse, void* stream);

/* Device workspace, in bytes, that ra_ring_attention_backward needs: the
 * chunk and query segment tables, the query and key positions (4 bytes per
 * query row and per key, built on the device), per-32-row position bounds,
 * delta (fp32 per (batch, head, query) row) and, when the query rows alone
 * cannot fill the GPU, fp32 partial dq of up to 8 key ranges. A multiple of
 * 256. */
size_t ra_ring_backward_workspace_bytes(int batch, int q_heads, int head_dim, int64_t q_len, int64_t total_keys,
                                        int n_chunks, int n_q_segments);

/* Gradients of ring_attention for this device's share.
 * "Ring Attention: Distributed Reads with Online Softmax", section "Backward
 * must aggregate shared dependencies": the local queries contribute gradients
 * to the keys and values of every chunk they attend to; these are summed per
 * key and returned per chunk, for the chunk's owner to add to the
 * contributions of the other devices. Probabilities are recomputed from the
 * forward's lse with the same scale and the same global-position causal mask.
 * With p_ij = exp(scale <q_i, k_j> - lse_i) over allowed pairs and
 * delta_i = <dout_i, out_i>:
 *   dv_j = sum_i p_ij dout_i,  ds_ij = p_ij (<dout_i, v_j> - delta_i),
 *   dq_i = scale sum_j ds_ij k_j,  dk_j = scale sum_i ds_ij q_i,
 * where the sums over i run over every query head sharing k_j's head (GQA).
 *  dtype       RA_BF16 only (bf16 matrix cores, fp32 accumulation); other
 *              types return RA_ERR_UNSUPPORTED. head_dim is a multiple of 8
 *              (8 .. 128).
 *  q, dout     [B,Hq,q_len,d] bf16; out [B,Hq,q_len,d] fp32 and lse
 *              [B,Hq,q_len] fp32 as ra_ring_attention returned them for the
 *              same inputs (lse must not be NULL there).
 *  q_segments, chunks, causal, scale: as for ra_ring_attention; rows of
 *              every chunk must be 16-byte aligned.
 *  dq          [B,Hq,q_len,d] fp32 (written).
 *  dk, dv      [B,Hkv,total_keys,d] fp32 (written): key j of the
 *              concatenated chunk list in list order, so chunk c's gradient
 *              is the slice of its keys. Every row is written, zero for keys
 *              no local query sees.
 *  workspace   >= ra_ring_backward_workspace_bytes(...) bytes, 256-byte
 *              aligned; tables are written there on `stream`.
 * Outputs must not overlap inputs. The result is bit-identical from run to
 * run (no atomics; every sum in a fixed order). */
int ra_ring_attention_backward(int dtype, int batch, int q_heads, int kv_heads, int head_dim,
                               const void* q, const ra_q_segment* q_segments, int n_q_segments,
                               const ra_kv_chunk* chunks, int n_chunks, int causal, float scale,
                               const float* out, const float* lse, const void* dout,
                               void* workspace, size_t workspace_bytes,
                               float* dq, float* dk, float* dv, void* stream);

/* Measurement aid, outside the pages' API: device time of the attention
 * kernels themselves. While enabled, every ra_ring_attention and
 * ra_attention_chunk_stats call records a pair of HIP events on its stream,
 * immediately before and after its attention kernel (the key-range combine
 * of ra_ring_attention is outside the pair); up to 512 pairs are kept.
 * Each ra_ring_attention_backward call records two pairs: one around its
 * dK/dV kernel and one around its dQ kernel.
 * ra_kernel_timer(1) creates the events on first use (the only resources the
 * library ever creates; they live until the process ends), clears the kept
 * pairs and enables recording; ra_kernel_timer(0) disables it.
 * ra_kernel_timer_read waits for the kept pairs, writes the sum of their
 * durations in milliseconds and their number, and clears them. Not
 * thread-safe; meant for one benchmarking thread. */
int ra_kernel_timer(int enable);
int ra_kernel_timer_read(float* total_ms, int* count);

/* Static, human-readable name of a status code. */
const char* ra_status_string(int status);

/* Message describing the last failed call on this host thread ("" if none). */
const char* ra_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RING_ATTENTION_CHUNK_H */
