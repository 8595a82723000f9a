/*
 * pa.h -- C ABI of the paged KV-cache decode library (libpa.so) for AMD
 * Instinct MI355X (gfx950).
 *
 * The method: a sequence's K/V live in fixed-size physical blocks of a shared
 * pool, found through a per-sequence block table (logical block -> physical
 * block).  Attention itself is unchanged; only where the rows are stored
 * changes, and the kernel follows the table (page "vLLM：把 KV 缓存当成虚拟
 * 内存", section "破除误解"; page "放下账簿，打开源码", sections
 * "PagedAttention：虚实分离，按需取用" and "注意力计算的改写").  Blocks are
 * taken lazily, shared by fork / prefix sharing with reference counts, and
 * copied on the first write into a shared block (page "Lazy Allocation 与
 * Copy-on-Write 在 LLM 推理系统中的应用", sections 3.3 and 4.4; page "第 6 章
 * 缓存管理：把显存当操作系统来管", section "块表长什么样").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pool layout (K and V alike): contiguous [num_blocks][num_kv_heads]
 *   [block_size][head_dim] elements of the pool element type (the dtype, or
 *   8-bit E4M3 codes for a quantised pool).  Token position `pos`
 *   of a sequence lives in physical block table[pos / block_size] at offset
 *   pos % block_size; its slot is block * block_size + offset.
 * - Device pointers are caller-owned (e.g. torch tensors) and must be 16-byte
 *   aligned.  The library never allocates device memory; the split-K
 *   workspace is passed in by the caller.
 * - Kernels run asynchronously on `hip_stream` (NULL = the null stream), in
 *   the order the calls are made.  A step that copies blocks and writes new
 *   tokens must call pa_copy_blocks before pa_reshape_and_cache on the same
 *   stream (copies of a step land before its writes).
 * - Argument, shape and dtype checks happen on the host before any launch and
 *   return a negative status with nothing launched.  A failed launch returns
 *   PA_ERR_HIP.  Device-side values (block ids, slots, context lengths) are not
 *   validated on the host; the kernels never access memory outside the pools,
 *   tables or buffers for out-of-range values, but the numbers they produce
 *   for such inputs are unspecified (see each call).
 * - Supported shapes: dtype f32, f16 or bf16; head_dim 64 or 128; block_size
 *   16 or 32; num_q_heads a multiple of num_kv_heads with group
 *   G = num_q_heads / num_kv_heads <= 16 (<= 8 for f32 or head_dim 64).
 *   8-bit pools: f16 or bf16 dtype, head_dim 128.
 *
 * Thread safety: the kernel entry points are reentrant.  An allocator handle
 * must not be used from two threads at once.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PA_OK = 0,
  PA_ERR_ARG = -1,       /* null pointer, misalignment, value out of range */
  PA_ERR_DTYPE = -2,     /* unknown dtype */
  PA_ERR_SHAPE = -3,     /* unsupported head_dim / block_size / group size */
  PA_ERR_OOM = -4,       /* allocator: not enough free blocks (state unchanged) */
  PA_ERR_REFCOUNT = -5,  /* allocator: refcount would go below zero */
  PA_ERR_NOT_FOUND = -6, /* allocator: unknown sequence id */
  PA_ERR_HIP = -7,       /* a HIP launch or runtime call failed */
  PA_ERR_SWAPPED = -8,   /* allocator: the sequence is swapped out to the host */
  PA_ERR_SCRATCH = -9    /* pa_decode_noalloc: the call needs more scratch than
                            PA_NOALLOC_SCRATCH_BYTES (nothing launched) */
} pa_status;

typedef enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2 } pa_dtype;

/* Element type of the pools: the dtype itself, or E4M3 8-bit floats (OCP
 * "fn" variant: bias 7, no infinity, 0x7F/0xFF NaN, largest 448) scaled per
 * pool.  A quantised cache trades accuracy for capacity and bandwidth (page
 * "第 6 章 缓存管理", section "缓存的边界"). */
typedef enum { PA_KV_SAME = 0, PA_KV_FP8_E4M3 = 1 } pa_kv_dtype;

/* Shape of one K pool and one V pool (both have this shape). */
typedef struct {
  int32_t num_blocks;   /* physical blocks NB >= 1 */
  int32_t block_size;   /* tokens per block BS: 16 or 32 */
  int32_t num_kv_heads; /* Hkv >= 1 */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t dtype;        /* pa_dtype of q, out and new K/V rows (and of the pools
                           when kv_dtype is PA_KV_SAME) */
  int32_t kv_dtype;     /* pa_kv_dtype of the pools */
  float k_scale;        /* PA_KV_FP8_E4M3: a K element's value is its code's
                           value times k_scale (finite, > 0); ignored otherwise */
  float v_scale;        /* the same for V */
} pa_pool_desc;

/* Library version of this ABI (bumped on incompatible change). */
int32_t pa_abi_version(void);

/* Static string naming a status code. */
const char* pa_status_string(int32_t status);

/* ------------------------------------------------------------------------
 * Decode attention (one new query token per sequence).
 *
 * For sequence i, q head h and its kv head g = h / G, with ctx = context_lens[i]
 * tokens at positions 0..ctx-1 found through block_tables[i]:
 *     out[i][h] = sum_t softmax_t(scale * <q[i][h], K[t][g]>) * V[t][g]
 * accumulated in fp32 and rounded once (round to nearest even) to the
 * dtype.  context_lens count every token the query attends to, including the
 * token being decoded, whose K/V must already be written (pa_reshape_and_cache
 * before pa_decode on the same stream).
 *
 * Work split (split-K).  Each kernel splits every sequence's positions into
 * pieces and merges the pieces' fp32 (max, sum, unnormalised output) with a
 * log-sum-exp rescale in a second kernel:
 *  - grid split: one workgroup per (sequence, kv head, partition of
 *    `partition_tokens` consecutive positions); a sequence with a single
 *    partition is written to `out` directly;
 *  - stream split (matrix-core kernel, up to 4096 sequences): all 16-token
 *    tiles of the batch, in (kv head, sequence, position) order, are divided
 *    evenly among a fixed set of waves (one 4-wave workgroup per CU); a
 *    (sequence, kv head) inside one wave's share is written directly.
 *
 *   q             device, [num_seqs][num_q_heads][head_dim], dtype
 *   k_pool/v_pool device, pool layout above
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries past
 *                 ceil(ctx / BS) are never read (any padding value is fine)
 *   context_lens  device int32 [num_seqs]; a value <= 0 yields an all-zero
 *                 output row; values are clamped to max_context_len and to
 *                 max_blocks_per_seq * BS
 *   max_context_len  host bound >= every context_lens[i]; sizes the grid
 *                 without a device->host copy
 *   scale         softmax scale (typically 1 / sqrt(head_dim))
 *   out           device, [num_seqs][num_q_heads][head_dim], dtype
 *   workspace     device, >= pa_decode_workspace_bytes(...) bytes, 16-byte
 *                 aligned; may be NULL when that size is 0.  Split-K scratch,
 *                 except that the stream split keeps its balance state (see
 *                 pa_set_decode_balance) in the first 4352 bytes between
 *                 calls: any contents on entry are valid input (a header it
 *                 does not recognise means the even cut).  Reusing one
 *                 workspace across calls lets the balance adapt.
 *   partition_tokens  multiple of 16 and of block_size, in [16, 4096];
 *                 0 selects the default (512).  Sizes the grid split's
 *                 partitions, and under PA_PATH_AUTO decides whether a small
 *                 pass fits one partition (see pa_set_decode_path); unused
 *                 by the stream split.
 *   sliding_window  0: none.  W > 0: the query (position ctx - 1) attends only
 *                 positions max(0, ctx - W) .. ctx - 1 (its own and the W - 1
 *                 before it); table entries of blocks wholly below that are
 *                 never read (they may be PA_NO_BLOCK).  < 0: PA_ERR_ARG.
 *   status        device int32, or NULL.  When a table entry inside a
 *                 sequence's attended range names a block outside [0,
 *                 num_blocks), the call ORs PA_STATUS_BAD_BLOCK into it; it
 *                 never clears it (the caller zeroes it before the call and
 *                 reads it after).  A wrong table otherwise gives plausible
 *                 wrong numbers with no signal at all (page "vLLM：把 KV 缓存当成
 *                 虚拟内存", section "KV 的体积从哪来，页表如何把它切开").
 * 8-bit pools: K and V elements are dequantised as code value * k_scale /
 * v_scale (k_scale folded into the score scale, v_scale into the output).
 * Block ids outside [0, num_blocks) are skipped (those tokens do not take
 * part; `status` reports them); the output is then unspecified but no access
 * leaves the pool.
 * ------------------------------------------------------------------------ */
/* Bit of the status word: a block id outside the pool inside an attended
 * range (pa_decode*, pa_prefill). */
#define PA_STATUS_BAD_BLOCK 1

/* Workspace bytes pa_decode may need for these arguments: the largest need
 * of the kernels that can run this shape under any path setting (so the
 * setting may change without a new workspace).  0 when none is needed or the
 * arguments are invalid (pa_decode then reports the error). */
size_t pa_decode_workspace_bytes(const pa_pool_desc* pool, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_context_len,
                                 int32_t partition_tokens);

pa_status pa_decode(const void* q, const void* k_pool, const void* v_pool,
                    const pa_pool_desc* pool, const int32_t* block_tables,
                    int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t max_context_len, float scale,
                    int32_t sliding_window, void* out, void* workspace,
                    size_t workspace_bytes, int32_t partition_tokens, int32_t* status,
                    void* hip_stream);

/* The two passes of pa_decode, callable one at a time (same arguments, same
 * path setting, same stream; pa_decode == pa_decode_partition then
 * pa_decode_reduce).  The partition pass writes every row it can finish
 * alone, including the all-zero rows of empty sequences (context_lens <= 0),
 * on every kernel; the reduce pass finishes the rows the partition pass left
 * in the workspace, and does nothing when the grid split has one partition. */
pa_status pa_decode_partition(const void* q, const void* k_pool, const void* v_pool,
                              const pa_pool_desc* pool, const int32_t* block_tables,
                              int32_t max_blocks_per_seq, const int32_t* context_lens,
                              int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                              float scale, int32_t sliding_window, void* out, void* workspace,
                              size_t workspace_bytes, int32_t partition_tokens, int32_t* status,
                              void* hip_stream);

pa_status pa_decode_reduce(const void* q, const void* k_pool, const void* v_pool,
                           const pa_pool_desc* pool, const int32_t* block_tables,
                           int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                           float scale, int32_t sliding_window, void* out, void* workspace,
                           size_t workspace_bytes, int32_t partition_tokens, int32_t* status,
                           void* hip_stream);

/* pa_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and kernels as
 * pa_decode (bit-identical output for the same cut of the stream split, e.g.
 * with pa_set_decode_balance(0)), minus workspace and workspace_bytes: the
 * split-K workspace is a static device array of PA_NOALLOC_SCRATCH_BYTES that
 * the library holds on each device it runs on until the process ends.  The
 * call allocates nothing.  It runs on the current device (hip_stream must
 * belong to it); its first call on a device looks up that device's copy of
 * the array (PA_ERR_HIP if that fails).  Returns PA_ERR_SCRATCH, with nothing
 * launched, when the shape needs more workspace than the array holds
 * (pa_decode_workspace_bytes bounds the need).  Every call on one device
 * uses the same array: calls that can overlap on one device (different
 * streams without ordering between them) race and must not be made; calls
 * on one stream are ordered and safe.  Nothing in the array needs to start
 * at zero: stale contents from an earlier call are at most the stream
 * split's balance state, which every call on the device shares. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
pa_status pa_decode_noalloc(const void* q, const void* k_pool, const void* v_pool,
                            const pa_pool_desc* pool, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* context_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                            float scale, int32_t sliding_window, void* out,
                            int32_t partition_tokens, int32_t* status, void* hip_stream);

/* Decode kernel family.  PA_PATH_AUTO: the matrix-core kernels for 16-bit
 * and 8-bit pools with head_dim 128 and G = num_q_heads / num_kv_heads in
 * [1, 16], the vector kernel otherwise; among the matrix-core kernels, the
 * grid split for a small single-partition pass (max_context_len <=
 * partition_tokens and num_seqs * num_kv_heads * ceil(max_context_len / 16)
 * at most 80 tiles per stream wave: no reduce pass is needed and the
 * hardware's workgroup dispatch balances it), else the stream split when the
 * batch has at most 4096 sequences, else the grid split.  PA_PATH_MFMA /
 * PA_PATH_VALU force one family (PA_ERR_SHAPE if it does not support the
 * shape), PA_PATH_MFMA taking the stream split up to 4096 sequences;
 * PA_PATH_MFMA_GRID forces the grid split.  Results agree up to the order of
 * the fp32 merges.  Process-wide setting; returns the previous value (-1 for
 * an unknown path, which leaves the setting unchanged). */
typedef enum {
  PA_PATH_AUTO = 0,
  PA_PATH_VALU = 1,
  PA_PATH_MFMA = 2,
  PA_PATH_MFMA_GRID = 3
} pa_decode_path;
int32_t pa_set_decode_path(int32_t path);

/* Run-time balance of the stream split (the block loop and cross-partition
 * merge of page "放下账簿，打开源码", section "注意力计算的改写", cut over the
 * GPU's dies).  The stream split cuts the batch's tiles into one chunk per
 * XCD (each XCD with its own L2; the count is queried from the device, 8 on
 * a whole MI355X); the dies do not run equally fast, so with balancing on
 * (1, the default; used with 8 XCDs) each partition pass of at least 80 tiles per
 * wave records how long each chunk's slowest wave took, and the next reduce
 * pass moves each chunk's share of the next call's tiles halfway towards its
 * measured rate (shares kept within 1/16 .. 3/16).  The state lives in the
 * first 4352 bytes of the workspace (of the static array for
 * pa_decode_noalloc), so it carries over only between calls that share one.
 * The cut changes where the fp32 merges fall: outputs of two calls then
 * agree up to the order of those merges, not bit for bit.  With balancing
 * off (0) the cut is even and repeated calls are bit-identical.
 * Process-wide setting; returns the previous value (-1 for a value other
 * than 0 or 1, which leaves the setting unchanged). */
int32_t pa_set_decode_balance(int32_t on);

/* ------------------------------------------------------------------------
 * Chunked prefill attention: a step that runs a chunk of each sequence's
 * prompt tokens, after their K/V have been written to the cache
 * (pa_reshape_and_cache before pa_prefill on the same stream).  Prefill
 * writes every prompt token's K/V; a long prompt may be cut into chunks run
 * between decode steps (page "附录：Lazy Allocation 与 Copy-on-Write 在 LLM 推理
 * 系统中的应用" §2.1; page "vLLM：把 KV 缓存当成虚拟内存", section "KV 的体积从哪
 * 来，页表如何把它切开").
 *
 * Sequence i's chunk is query rows a = query_start[i] .. b - 1 (b =
 * query_start[i+1], n = b - a), its tokens at positions ctx - n .. ctx - 1
 * with ctx = context_lens[i] (the length after the chunk).  Row a + j, q
 * head h, kv head g = h / G attends to positions 0 .. ctx - n + j:
 *     out[a+j][h] = sum_{p <= ctx-n+j} softmax_p(scale * <q[a+j][h], K[p][g]>) * V[p][g]
 * in fp32, rounded once (RNE) to the dtype.  A row whose position is
 * negative (ctx < n) is all zeros.  With sliding_window W > 0 a row at
 * position p attends only positions max(0, p - W + 1) .. p.
 *
 *   q, out        device [num_tokens][num_q_heads][head_dim], dtype
 *   query_start   device int32 [num_seqs + 1], non-decreasing; a sequence
 *                 whose rows fall outside [0, num_tokens) is skipped
 *   context_lens  device int32 [num_seqs], clamped like pa_decode's
 *   max_query_len host bound >= every n; rows past it are not computed
 *   max_context_len, block_tables, max_blocks_per_seq, scale: as pa_decode
 * Supported: f16/bf16 dtype (16-bit or 8-bit pools), head_dim 128, G in
 * {1, 2, 4, 8, 16} (PA_ERR_SHAPE otherwise).  No workspace; one kernel
 * launch.  status: as pa_decode's (a block outside the pool inside the keys
 * some row of the chunk attends).
 * ------------------------------------------------------------------------ */
pa_status pa_prefill(const void* q, const void* k_pool, const void* v_pool,
                     const pa_pool_desc* pool, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* query_start,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_tokens,
                     int32_t num_q_heads, int32_t max_query_len, int32_t max_context_len,
                     float scale, int32_t sliding_window, void* out, int32_t* status,
                     void* hip_stream);

/* Prefill kernel.  PA_PREFILL_LDS: the K/V tiles of a 32-key step are loaded
 * through registers into LDS (8-bit codes widened on the way).
 * PA_PREFILL_DMA: the tiles go from memory straight into LDS (8-bit codes
 * into a code stage, then widened into a 16-bit stage by the waves that
 * loaded them) and the P.V operands are read from it transposed.
 * PA_PREFILL_AUTO: the faster of the two on the measured workloads, the DMA
 * kernel for 16-bit and 8-bit pools.  Both paths take every pool type and
 * shape pa_prefill accepts; results agree up to the order of fp32 sums.
 * Process-wide; returns the previous value (-1 for an unknown path, which
 * leaves the setting unchanged). */
typedef enum { PA_PREFILL_AUTO = 0, PA_PREFILL_LDS = 1, PA_PREFILL_DMA = 2 } pa_prefill_path;
int32_t pa_set_prefill_path(int32_t path);

/* ------------------------------------------------------------------------
 * Cache write: decode appends each new token's K/V to the cache (page
 * "Lazy Allocation 与 Copy-on-Write 在 LLM 推理系统中的应用", section 2.1), at
 * the slot its block table gives.  For every t with slot = slot_mapping[t]
 * >= 0 and every kv head h:
 *     k_pool[slot / BS][h][slot % BS][:] = k[t][h][:]   (same for v)
 * Bit-exact copy into a pool of the dtype.  Into an 8-bit pool each element
 * x is stored as the E4M3 code nearest to clamp(x * (1 / k_scale), -448,
 * 448) (products and the reciprocal in fp32, ties to the even code; NaN
 * stays NaN); v with v_scale.  Slots < 0 are skipped; slots >= num_blocks *
 * BS are skipped too (never written).  Two tokens with the same slot race.
 *   k, v          device, [num_tokens][num_kv_heads][head_dim], dtype
 *   slot_mapping  device int64 [num_tokens]
 * ------------------------------------------------------------------------ */
pa_status pa_reshape_and_cache(const void* k, const void* v, const int64_t* slot_mapping,
                               int32_t num_tokens, void* k_pool, void* v_pool,
                               const pa_pool_desc* pool, void* hip_stream);

/* ------------------------------------------------------------------------
 * Block-table upkeep on the device.  A decode step changes each sequence's
 * table in at most the entries its new positions fall in: a fresh block when
 * a position starts a logical block (lazy allocation), and the repointed last
 * block when the first position copies a shared block (copy-on-write); both
 * are the block of the position's slot (page "放下账簿，打开源码", section
 * "PagedAttention：虚实分离，按需取用": the table maps a position's logical
 * block to the physical block its slot lies in).  So device-resident tables
 * can follow a step from the step's slots alone, without uploading them.
 * For each row i < num_seqs and each t < tokens_per_seq, with pos =
 * new_lens[i] - tokens_per_seq + t and slot = slot_mapping[i *
 * tokens_per_seq + t]:
 *     block_tables[i][pos / block_size] = slot / block_size   (slot >= 0,
 *         pos >= 0 and pos / block_size < max_blocks_per_seq; else skipped)
 *     context_lens[i] = new_lens[i]
 * The arguments are exactly what pa_seq_append_batch(seqs, num_seqs,
 * tokens_per_seq) returns for the sequences of those rows (slots_out,
 * lens_out), copied to the device.  Entries the step does not touch keep
 * their values, so the rows must hold the sequences' tables from before the
 * step (any other change, e.g. a fork, a free, a swap-in or a window trim,
 * needs the rows rebuilt, e.g. from pa_build_tables).  Writes are plain
 * stores: rows shared by two entries of one call race.
 *   slot_mapping  device int64 [num_seqs * tokens_per_seq]
 *   new_lens      device int32 [num_seqs]
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq] (updated)
 *   context_lens  device int32 [num_seqs] (written)
 *   block_size    power of two in [1, 65536] (the allocator's)
 * ------------------------------------------------------------------------ */
pa_status pa_update_tables(const int64_t* slot_mapping, const int32_t* new_lens, int32_t num_seqs,
                           int32_t tokens_per_seq, int32_t block_size, int32_t* block_tables,
                           int32_t max_blocks_per_seq, int32_t* context_lens, void* hip_stream);

/* ------------------------------------------------------------------------
 * Copy-on-write block copy: before the first write into a block that other
 * sequences still share, the writer gets a private copy (page "Lazy
 * Allocation 与 Copy-on-Write 在 LLM 推理系统中的应用", section 4.4; page
 * "第 6 章 缓存管理：把显存当操作系统来管", section "块表长什么样").  For each
 * pair p: k_pool[dst] = k_pool[src] and v_pool[dst] = v_pool[src], whole
 * blocks (all kv heads, all slots).  Bit-exact.  The pairs of one call run
 * concurrently, so no dst may be a src or a dst of another pair of the same
 * call.  The pairs of one pa_seq_append_batch call always satisfy this, and
 * so do pairs gathered from several appends of an allocator without the
 * prefix cache (a copied block keeps a holder).  With the prefix cache on,
 * pairs from separate pa_seq_append / pa_seq_append_tokens calls may chain
 * (a cached block copied by its last holder is evictable at once, and a
 * later append may take it as its copy's destination): give each such append
 * its own call, in order.  Pairs with an id outside [0, num_blocks) are
 * skipped.
 *   pairs  device int32 [num_pairs][2] = (src, dst)
 * ------------------------------------------------------------------------ */
pa_status pa_copy_blocks(void* k_pool, void* v_pool, const pa_pool_desc* pool,
                         const int32_t* pairs, int32_t num_pairs, void* hip_stream);

/* ------------------------------------------------------------------------
 * Host block allocator (no device memory; host arrays only).
 *
 * Free pool: a FIFO seeded with `initial_free_order` (NULL = 0..NB-1).
 * Allocation pops the front; freeing a sequence walks its table in logical
 * order and appends every block whose refcount reaches zero at the back.
 *
 * pa_seq_append writes positions len..len+n-1 of a sequence.  A position that
 * starts a logical block takes a fresh block (lazy allocation).  If the first
 * position falls inside the last block and that block's refcount is > 1, the
 * writer first gets a copy: a fresh block dst, the pair (src, dst) is
 * returned for pa_copy_blocks, src's refcount drops by one and the table
 * points at dst (the last holder writes in place; page "Lazy Allocation 与
 * Copy-on-Write ...", section 4.4).  At most one pair per call.  If the free
 * pool cannot supply every block the call needs it returns PA_ERR_OOM and
 * changes nothing.
 *
 * pa_seq_fork: the child gets a copy of the parent's table and length; every
 * block's refcount goes up by one (no KV moves; page "vLLM：把 KV 缓存当成虚拟
 * 内存", section "碎片从哪里来").
 * pa_seq_share_prefix: a new sequence whose first ceil(n / BS) table entries
 * are src's, refcounts +1, length n (0 <= n <= src length; page "第 6 章
 * 缓存管理：把显存当操作系统来管", section "块表长什么样").
 * pa_seq_free: refcount -1 on each block; zero -> back to the free pool
 * (or, for a cached block, to the evictable list; see the prefix cache).
 * Sequence ids are assigned 0, 1, 2, ... in creation order, never reused.
 * ------------------------------------------------------------------------ */
typedef struct pa_alloc pa_alloc;

/* Table entry of a block a sliding window released (pa_seq_trim_window). */
#define PA_NO_BLOCK (-2147483647 - 1)

pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                          const int32_t* initial_free_order, pa_alloc** out);
void pa_alloc_destroy(pa_alloc* a);

pa_status pa_seq_create(pa_alloc* a, int64_t* seq_out);
/* slots_out: host int64 [n_tokens]; cow_pair_out: host int32 [2]; num_cow_out: 0 or 1 */
pa_status pa_seq_append(pa_alloc* a, int64_t seq, int32_t n_tokens, int64_t* slots_out,
                        int32_t* cow_pair_out, int32_t* num_cow_out);
/* One decode step for many sequences: appends n_tokens to each of seqs[0..n)
 * in order.  slots_out [n * n_tokens]; pairs_out [n][2]; *num_pairs_out =
 * pairs written; lens_out [n] (may be NULL) = each sequence's new length.  The pairs are independent (no dst is another pair's src or
 * dst), so one pa_copy_blocks call can run them all: a cached block whose
 * last holder copies it is held back from the evictable list until the
 * step's last append, and joins it then, in the order of release.  Each
 * append must fit what is available when it runs (held blocks excluded).
 * All or nothing: on PA_ERR_OOM nothing changes.  A sequence named twice is
 * PA_ERR_ARG. */
pa_status pa_seq_append_batch(pa_alloc* a, const int64_t* seqs, int32_t n, int32_t n_tokens,
                              int64_t* slots_out, int32_t* pairs_out, int32_t* num_pairs_out,
                              int32_t* lens_out);
pa_status pa_seq_fork(pa_alloc* a, int64_t parent, int64_t* child_out);
pa_status pa_seq_share_prefix(pa_alloc* a, int64_t src, int32_t n_tokens, int64_t* seq_out);
pa_status pa_seq_free(pa_alloc* a, int64_t seq);
/* Length and table of one sequence: table_out [capacity] (may be NULL);
 * *num_blocks_out = its number of blocks (PA_ERR_ARG if > capacity and
 * table_out is non-NULL). */
pa_status pa_seq_info(const pa_alloc* a, int64_t seq, int32_t* len_out, int32_t* table_out,
                      int32_t capacity, int32_t* num_blocks_out);
/* Block tables of seqs[0..n) padded with -1: tables_out [n][max_blocks],
 * lens_out [n].  PA_ERR_ARG if a sequence has more than max_blocks blocks. */
pa_status pa_build_tables(const pa_alloc* a, const int64_t* seqs, int32_t n, int32_t max_blocks,
                          int32_t* tables_out, int32_t* lens_out);
/* Free-pool size, the free pool front to back (free_list_out [NB] or NULL)
 * and every block's refcount (refcounts_out [NB] or NULL). */
pa_status pa_alloc_query(const pa_alloc* a, int32_t* num_free, int32_t* free_list_out,
                         int32_t* refcounts_out);
/* Counters: lazy block allocations and CoW copies since creation, live
 * sequences, blocks with refcount > 1. */
pa_status pa_alloc_stats(const pa_alloc* a, int64_t* lazy_allocs, int64_t* cow_copies,
                         int32_t* live_seqs, int32_t* shared_blocks);
/* PA_OK if refcount == in-degree over all tables, a block is in the free
 * pool iff its refcount is 0 and it is not cached, in the evictable list iff
 * its refcount is 0 and it is cached, neither list has duplicates, the cache
 * index and the cached blocks agree, and every table has ceil(len / BS)
 * entries; PA_ERR_REFCOUNT otherwise. */
pa_status pa_alloc_check_invariants(const pa_alloc* a);

/* ------------------------------------------------------------------------
 * Prefix cache.  A prefix many requests share (a system prompt) stays in
 * memory as cached blocks kept out of the free pool, and a later request with
 * the same prefix takes them instead of computing that prefill (page "vLLM：
 * 把 KV 缓存当成虚拟内存", sections "碎片从哪里来" and "KV 的体积从哪来，页表如何
 * 把它切开"; page "放下账簿，打开源码", section "写时复制与前缀缓存").  When
 * memory runs out, cached blocks are dropped least recently used first and
 * recomputed when needed (page "第 6 章 缓存管理", section "缓存放不下的时候").
 *
 * Rules:
 *  - only full blocks whose token ids are known are cached, under the whole
 *    token prefix up to the block's end (a chained 64-bit hash; the block's
 *    own tokens and its parent's hash are compared on a hit);
 *  - pa_seq_append_tokens caches each block it fills, unless that prefix is
 *    already cached under another block (the first registration stays);
 *    pa_seq_append and pa_seq_append_batch carry no ids and cache nothing
 *    from the first position they write onwards;
 *  - pa_seq_create_prefix walks the prompt's full blocks from the start and
 *    takes each cached one (refcount + 1) up to the first miss, at most
 *    n_tokens - 1 tokens (one prompt token is always left to compute); the
 *    sequence's length is the hit length; the caller appends the rest;
 *  - a cached block whose count drops to zero is evictable: released
 *    sequences' cached blocks enter a least-recently-used list from the
 *    sequence's last block to its first; a hit takes a block back out;
 *  - new blocks come from the free pool, else by evicting the least recently
 *    used evictable block (PA_ERR_OOM only when both are short);
 *  - a cached block is never written: an append whose first position falls
 *    in one copies it first (a CoW pair, as for a shared block).
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t lookup_tokens;     /* prompt tokens looked up */
  int64_t hit_tokens;        /* of which found cached */
  int64_t evictions;         /* cached blocks dropped for new data */
  int32_t cached_blocks;     /* blocks currently cached */
  int32_t evictable_blocks;  /* cached with refcount 0 */
  int32_t pinned_blocks;     /* cached with refcount > 0 */
} pa_prefix_stats;

/* Turns the cache on; PA_ERR_ARG once any sequence exists. */
pa_status pa_alloc_enable_prefix_cache(pa_alloc* a);
/* A new sequence for a prompt of n_tokens ids (host int32); *hit_tokens_out
 * = tokens found cached.  PA_ERR_ARG if the cache is off. */
pa_status pa_seq_create_prefix(pa_alloc* a, const int32_t* tokens, int32_t n_tokens,
                               int64_t* seq_out, int32_t* hit_tokens_out);
/* pa_seq_append with the new positions' token ids (host int32 [n_tokens]). */
pa_status pa_seq_append_tokens(pa_alloc* a, int64_t seq, const int32_t* tokens, int32_t n_tokens,
                               int64_t* slots_out, int32_t* cow_pair_out, int32_t* num_cow_out);
pa_status pa_prefix_cache_stats(const pa_alloc* a, pa_prefix_stats* out);
/* Evictable blocks, least recently used first (evictable_out [NB] or NULL). */
pa_status pa_prefix_cache_query(const pa_alloc* a, int32_t* evictable_out, int32_t* num_out);

/* ------------------------------------------------------------------------
 * Sliding window.  With a window of W positions, the newest token (position
 * len - 1) and every later one attend only positions >= len - W, so a block
 * whose positions all lie below len - W is never read again (page "vLLM：把
 * KV 缓存当成虚拟内存": sliding windows change how long K/V live).
 * pa_seq_trim_window drops the sequence's reference to each such block
 * (released as pa_seq_free releases: free pool, or evictable if cached) and
 * leaves PA_NO_BLOCK in its table entry; the table keeps its length, so
 * entry j still maps positions j * BS ...  Attention with the same window
 * never reads those entries.  Holes are skipped by every other call; a fork
 * copies them; pa_seq_share_prefix of a prefix that includes one returns
 * PA_ERR_ARG.  *released_out (may be NULL) = entries that became holes.
 * PA_ERR_ARG for window <= 0; PA_ERR_SWAPPED for a swapped-out sequence.
 * ------------------------------------------------------------------------ */
pa_status pa_seq_trim_window(pa_alloc* a, int64_t seq, int32_t window, int32_t* released_out);

/* ------------------------------------------------------------------------
 * Swapping (preemption).  A preempted sequence's KV moves to host memory and
 * comes back later, block by block, not as one contiguous buffer (page
 * "vLLM：把 KV 缓存当成虚拟内存", section "碎片从哪里来"; page "第 6 章 缓存管理",
 * section "缓存放不下的时候", on moving cold cache to CPU memory).
 *
 * The host side is a second pool pair (K and V) of num_host_blocks blocks of
 * the device pool's block shape, [NHB][Hkv][BS][D] each, in pinned host
 * memory; the allocator keeps its free list (FIFO, ids 0.. in order at
 * start).
 *  - pa_seq_swap_out: the blocks only this sequence holds (refcount 1) get
 *    host blocks from the front of the host list, in logical order, and are
 *    released like pa_seq_free releases them (free pool, or evictable if
 *    cached).  Blocks it shares stay on the device with its reference kept.
 *    pairs_out [capacity][2] = (device block, host block); these copies must
 *    run (pa_swap_blocks, PA_SWAP_OUT) before the released blocks are
 *    written again.  PA_ERR_OOM if the host list is short (nothing changes).
 *  - A swapped-out sequence can only be swapped in, freed or inspected:
 *    other calls on it return PA_ERR_SWAPPED.  pa_seq_info reports a host
 *    entry h as -(h + 1).  Freeing it returns its host blocks to the back of
 *    the host list in logical order.
 *  - pa_seq_swap_in: each host entry gets a device block the way an append
 *    takes one (free pool front, else eviction of a cached block), in
 *    logical order; pairs_out = (host block, device block), to be copied
 *    (PA_SWAP_IN) before the sequence is read; the host blocks go back to
 *    the host list in logical order.  The new blocks are private and not
 *    cached.  PA_ERR_OOM if the device is short (nothing changes);
 *    PA_ERR_ARG if the sequence is not swapped out.
 * capacity must cover the sequence's block count (pa_seq_info), else
 * PA_ERR_ARG before any change.
 * ------------------------------------------------------------------------ */
typedef struct {
  int64_t swap_outs;     /* sequences swapped out (preemptions) */
  int64_t swap_ins;
  int64_t blocks_out;    /* blocks moved device -> host */
  int64_t blocks_in;
  int32_t swapped_seqs;  /* sequences on the host now */
  int32_t host_free;     /* free host blocks */
} pa_swap_stats;

/* Turns swapping on with a host pool of num_host_blocks blocks (once). */
pa_status pa_alloc_enable_swap(pa_alloc* a, int32_t num_host_blocks);
pa_status pa_seq_swap_out(pa_alloc* a, int64_t seq, int32_t* pairs_out, int32_t capacity,
                          int32_t* num_pairs_out);
pa_status pa_seq_swap_in(pa_alloc* a, int64_t seq, int32_t* pairs_out, int32_t capacity,
                         int32_t* num_pairs_out);
/* Counters, and the host free list front to back (host_free_out [NHB] or NULL). */
pa_status pa_swap_query(const pa_alloc* a, pa_swap_stats* stats, int32_t* host_free_out);

typedef enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 } pa_swap_direction;

/* Copies whole blocks between the device pools and the host pools (both K and
 * V): PA_SWAP_OUT copies device block p[0] to host block p[1] for each pair p
 * of pairs (device int32 [num_pairs][2]); PA_SWAP_IN copies host block p[0]
 * to device block p[1].  The host pools must be pinned host allocations
 * (hipHostMalloc, or torch's pin_memory) of num_host_blocks blocks of the
 * device pools' block shape; the kernel reads or writes them directly over
 * the host link.  Pairs with an id out of range are skipped; every
 * destination block must be distinct.  PA_ERR_ARG for null or misaligned
 * pointers, host pointers that are not pinned host memory, or num_pairs
 * beyond 65535.  Asynchronous on the stream: the host pool is complete (out)
 * or may be reused (in) once the stream has passed the call. */
pa_status pa_swap_blocks(void* k_pool, void* v_pool, void* k_host, void* v_host,
                         int32_t num_host_blocks, const pa_pool_desc* pool, const int32_t* pairs,
                         int32_t num_pairs, int32_t direction, void* hip_stream);

/* ------------------------------------------------------------------------
 * Read ceiling of the decode access pattern (a measurement aid).  Decode
 * reads every attended K/V row once per step and is bound by memory (page
 * "vLLM：把 KV 缓存当成虚拟内存", section "KV 的体积从哪来，页表如何把它切开"),
 * in tiles scattered over the pool.  This call reads a list of such tiles
 * and does nothing else with them: 4-wave workgroups, each wave a contiguous
 * run of the list (wave rank r of W: tiles [n r / W, n (r + 1) / W)), 32
 * 16-byte loads in flight per wave, each tile's offset read one tile ahead
 * (one offset for both pools' tiles when two are given).
 * With W = 4 per compute unit it is the decode stream kernel's work split,
 * and its rate over a step's tiles is what that split allows; with W = n
 * (one tile per wave) it is the rate of the tiles alone.
 *   pool          device bytes [pool_bytes], 16-byte aligned; pool_bytes
 *                 below 2^32
 *   pool2         a second pool of pool_bytes, or NULL: each tile is then
 *                 read from both pools at the same offset (as the decode
 *                 kernel reads the K and V tiles of one (block, kv head))
 *   tile_offsets  device uint32 [num_tiles]: tile t is the tile_bytes bytes
 *                 at byte offset tile_offsets[t] of pool (and of pool2), a
 *                 multiple of 16 (bytes past pool_bytes read as zeros)
 *   tile_bytes    1024, 2048 or 4096
 *   num_waves     W, a positive multiple of 4 up to 2^24, or 0 for 4 per
 *                 compute unit (the decode stream split's grid)
 *   out           device uint32 [out_len]: out[r] = the XOR of every 32-bit
 *                 word wave r read (of both pools); out_len >= W
 *   waves         host int32, or NULL: receives W
 * PA_ERR_ARG for a null or misaligned pointer, a size out of range or an
 * out_len below W; PA_ERR_HIP when the device cannot be queried.  Runs
 * asynchronously on the stream; allocates nothing. */
pa_status pa_probe_tile_reads(const void* pool, const void* pool2, uint64_t pool_bytes,
                              const uint32_t* tile_offsets, int64_t num_tiles, int32_t tile_bytes,
                              int32_t num_waves, uint32_t* out, int32_t out_len, int32_t* waves,
                              void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
