/*
 * rpa.h -- ragged paged attention forward for AMD Instinct MI355X (gfx950).
 *
 * One call computes, for every query token of a step, causal (optionally
 * sliding-window) grouped-query attention over that token's sequence, whose
 * keys and values live in fixed-size pages found through a per-sequence page
 * table.  The step's query tokens of all sequences are flattened into one
 * array, with per-sequence metadata giving their structure ("TPU Deep Dive",
 * chapter 8, "Continuous batching with static shapes": flattened token batch,
 * true lengths handled inside the kernel, decode / prefill / mixed steps).
 *
 * The operation (the pages' method, read plainly):
 *   For sequence s with q_len = cu_q_lens[s+1] - cu_q_lens[s] and kv_len =
 *   kv_lens[s], query row r sits at position p = kv_len - q_len + r (the step's
 *   tokens are the last q_len of the sequence: chunked prefill on a cached
 *   prefix, "Pallas Kernel: vLLM on TPU ...", environment section).  Key t of
 *   the sequence is slot t % page_size of page page_table[s][t / page_size]
 *   (same page, S3: KV in 128-token blocks).  Query head h reads KV head
 *   h / G with G = num_q_heads / num_kv_heads ("TPU Deep Dive", chapter 4:
 *   several query heads share a KV head).  Key j is visible from position p iff
 *   j <= p and, when window W > 0, j >= p - W + 1 (a key is wanted by the W
 *   queries that follow it, "Chasing speed of light on TPU v6e", section
 *   Attention).  Then
 *       out[row, h, :] = sum_j softmax_j(scale * q[row, h, :] . k_j) * v_j
 *   over the visible keys: the two per-head products of footnote 5 of that
 *   section, with fp32 softmax accumulators (its footnote 6).
 *
 * Data types are fixed: bf16 tensors, int32 metadata, fp32 accumulation,
 * bf16 output rounded to nearest even.
 *
 * Threading: a context is not thread-safe (one host thread at a time).
 * Every call that takes a stream only enqueues work on it and returns.
 */
#ifndef RPA_H
#define RPA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes.  No exception or abort crosses this interface. */
enum {
  RPA_OK = 0,
  RPA_ERR_INVALID_ARG = -1, /* a pointer, size or metadata value is invalid   */
  RPA_ERR_UNSUPPORTED = -2, /* head_dim / head ratio without a compiled kernel */
  RPA_ERR_OOM = -3,         /* device or pinned host allocation failed         */
  RPA_ERR_HIP = -4          /* a HIP runtime call or kernel launch failed      */
};

typedef struct rpa_ctx rpa_ctx;

/* Shapes fixed for the lifetime of a context. */
typedef struct rpa_config {
  int32_t num_q_heads;       /* Hq >= 1                                         */
  int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0                          */
  int32_t head_dim;          /* D: 64, 128, 256 or 512                          */
  int32_t page_size;         /* B: tokens per page, >= 1                        */
  int32_t max_num_seqs;      /* most sequences of one call                      */
  int32_t max_pages_per_seq; /* row stride of page_table, >= 1                  */
  int64_t max_q_tokens;      /* most query tokens of one call                   */
} rpa_config;
/* Page size and speed: the kernels read a run of keys that lies in one page
 * through one buffer (a whole prefill tile or decode chunk when B is a
 * multiple of 32 or 64 keys, a 16-key run or one wave's rows of a prefill
 * tile when B is a multiple of 16, or of 4 at D = 256 and 512); any other B
 * works with a page lookup per lane, about 7-18 % slower. */

/*
 * rpa_create -- validate `cfg` and allocate a context (host memory only; the
 * device work-list and split-KV workspace are allocated on first use, on the
 * device that is current then, and grow as needed).
 * Returns RPA_OK and *out_ctx, RPA_ERR_INVALID_ARG for a bad config or null
 * pointer, RPA_ERR_UNSUPPORTED for a head_dim without a compiled kernel.
 */
int rpa_create(const rpa_config* cfg, rpa_ctx** out_ctx);

/*
 * rpa_forward -- one ragged paged attention call (the operation above).
 *
 *   q          device, bf16 [T, Hq, D] row-major, T = cu_q_lens[num_seqs]
 *   k_pages    device, bf16 [P, page_size, Hkv, D] row-major (P pages)
 *   v_pages    device, bf16 [P, page_size, Hkv, D] row-major
 *   page_table device, int32 [num_seqs, max_pages_per_seq] row-major; entries
 *              past ceil(kv_len / page_size) are never read, nor (W > 0) the
 *              entries of pages that hold only keys before the window of the
 *              sequence's first query token (keys < kv_len - q_len - W + 1)
 *   cu_q_lens  HOST, int32 [num_seqs + 1]; cu[0] = 0, non-decreasing
 *   kv_lens    HOST, int32 [num_seqs]; q_len <= kv_len, ceil(kv_len / B) <=
 *              max_pages_per_seq; kv_len includes this step's tokens, whose K/V
 *              must already be in their pages
 *   num_seqs   0 <= num_seqs <= max_num_seqs
 *   window     0: full causal; W > 0: keys p - W + 1 .. p; negative is an error
 *   scale      finite positive multiplier of q.k before the softmax (usually
 *              1/sqrt(D)); zero, negative or non-finite is an error
 *   out        device, bf16 [T, Hq, D]; must not overlap q
 *   stream     a hipStream_t (NULL = the null stream)
 *
 * Host arrays are read before the call returns and may be freed afterwards.
 * Device buffers are owned by the caller and must stay valid until the
 * enqueued work has completed.  Page slots past kv_len, slots of keys before
 * the window of a sequence's first query token, and the pool's other pages
 * may hold anything (even NaN): they are never read into the result.
 * Every argument check runs on the host before anything is enqueued: a call
 * that returns an error has enqueued nothing.  A call without query tokens
 * (cu_q_lens[num_seqs] == 0) enqueues nothing and returns RPA_OK once its
 * metadata has passed; its device pointers may then be NULL (as torch gives
 * for empty tensors).  Page-table *values* are device data and are not
 * checked.  Returns RPA_OK, RPA_ERR_INVALID_ARG, RPA_ERR_OOM
 * or RPA_ERR_HIP; rpa_last_error() then holds a message.
 *
 * Ordering: the calls of one context run in the order they are made, also
 * when they are made on different streams (a call on another stream than
 * the previous call first waits, on the device, for that call to finish).
 *
 * Work lists: the context keeps the work list of each metadata key
 * (cu_q_lens, kv_lens, window, bf16 or fp8 cache) it has seen recently in
 * device buffers of its own, written once when the key is first seen and
 * never overwritten; up to 8 keys that no capture has used are kept (least
 * recently used first out, after its last call has finished).
 *
 * Stream capture: a call may be captured into a HIP graph (for example the
 * attention of every layer of a step, replayed as one graph) when the context
 * has already run a call with the same cu_q_lens, kv_lens and window, so that
 * its work list is on the device; the captured call enqueues only kernels
 * (and, for a mixed step, the fork and join of its second stream) and records
 * no kernel timing.  A capture that would need a new work list returns
 * RPA_ERR_INVALID_ARG.  The work list, split workspace and fp8 staging pool
 * that a capture used stay allocated and unchanged -- later calls with any
 * other metadata use other buffers -- until rpa_release_captured() or
 * rpa_destroy(), so a graph may be replayed at any time before then.  The
 * caller orders replays against the context's eager calls (both use the
 * same split workspace), as for any graph launch, and replays of graphs that
 * captured the same metadata must not overlap in time.
 */
int rpa_forward(rpa_ctx* ctx, const void* q, const void* k_pages, const void* v_pages,
                const int32_t* page_table, const int32_t* cu_q_lens, const int32_t* kv_lens,
                int32_t num_seqs, int32_t window, float scale, void* out, void* stream);

/*
 * rpa_forward_noalloc -- rpa_forward for callers that cannot allocate
 * device memory: code in tight serving loops and harnesses that forbid
 * hipMalloc.  It allocates nothing on the device and creates no stream or
 * event: the call's work list and split-KV partials go into one device
 * array that the library holds for the life of the process (per GPU, at
 * most RPA_NOALLOC_SCRATCH_BYTES), the list is copied there from host memory
 * on `stream` by every call, and every kernel runs on `stream` (split groups
 * are merged by a separate merge kernel).  The result equals rpa_forward's.
 *
 * Arguments, checks and errors as for rpa_forward, plus RPA_ERR_INVALID_ARG
 * when the call's work list and partials exceed the scratch size (the message
 * gives both sizes; a larger RPA_OPT_DECODE_SPLIT_KEYS means fewer partials)
 * and when `stream` is being captured (the per-call copy from host memory
 * cannot be replayed; use rpa_forward under capture).  Every call on a GPU
 * uses that GPU's one scratch array: calls that overlap in time on one GPU
 * (from any context or thread, or on two streams) race and must be ordered
 * by the caller; the library does not order these calls against the
 * context's other calls either.
 */
#define RPA_NOALLOC_SCRATCH_BYTES (32u << 20)
int rpa_forward_noalloc(rpa_ctx* ctx, const void* q, const void* k_pages, const void* v_pages,
                        const int32_t* page_table, const int32_t* cu_q_lens, const int32_t* kv_lens,
                        int32_t num_seqs, int32_t window, float scale, void* out, void* stream);

/*
 * rpa_forward_append -- write the step's new keys and values into their
 * pages, then the same attention as rpa_forward, in one call.  The pages'
 * kernel takes the step's new tokens into the paged cache within the
 * attention call ("TPU Deep Dive", chapter 8, ragged paged attention).
 *
 *   k_new, v_new  device, bf16 [T, Hkv, D] row-major (16-byte aligned): row t
 *                 holds the new token at flattened query index t, i.e.
 *                 position p = kv_len_s - q_len_s + (t - cu_q_lens[s]) of its
 *                 sequence s; it is written to slot p % page_size of page
 *                 page_table[s][p / page_size] of k_pages / v_pages
 *   k_pages, v_pages  as for rpa_forward but written: the slots of the step's
 *                 tokens are overwritten with k_new / v_new, every other byte
 *                 is left as it was; the two must be distinct buffers, and
 *                 k_new / v_new must not overlap them
 *   all other arguments as for rpa_forward (kv_len counts the new tokens)
 *
 * The rows are written on `stream` within the call, and every product of
 * the call sees them.  A sequence whose new tokens all sit in one decode
 * item (rpa_work_item.self_append) has them written by the decode kernel
 * itself: the wave that reads the 32-key chunk holding a new key writes that
 * key's rows just before it reads the chunk.  With a bf16 cache the prefill
 * kernel takes the keys of a prefill sequence's new tokens straight from
 * k_new / v_new (the key of position p is row cu_q_lens[s] + p - (kv_len -
 * q_len) there) and each query tile's workgroup writes its own tokens' rows
 * into their slots after its products, so no workgroup of the call reads
 * those slots -- when every prefill sequence's first new position (kv_len -
 * q_len) is a multiple of the keys the kernel loads per buffer run (a key
 * tile, or one wave's rows of it: 4 to 64 keys by head size and page size;
 * always for prefills without prior context) and the prefill launch holds
 * at most two workgroups per slot of the device.  The rows of every other
 * sequence (fp8 caches, a sequence's tokens spread over several decode
 * items, the other prefill launches) are written by a copy kernel that runs
 * before the attention kernels.  Page slots of different tokens must be distinct (a page table
 * that maps two positions to one slot leaves either row there).  Errors as
 * for rpa_forward, plus RPA_ERR_INVALID_ARG for a NULL k_new / v_new (in a
 * call with query tokens) or k_pages == v_pages.
 */
int rpa_forward_append(rpa_ctx* ctx, const void* q, const void* k_new, const void* v_new, void* k_pages,
                       void* v_pages, const int32_t* page_table, const int32_t* cu_q_lens,
                       const int32_t* kv_lens, int32_t num_seqs, int32_t window, float scale, void* out,
                       void* stream);

/*
 * rpa_forward_fp8 -- rpa_forward over a KV cache held in fp8.  Holding KV in
 * fp8 halves the cache read that dominates decode and long contexts ("TPU
 * Deep Dive", chapter 7, quantization levers) and doubles the tokens a cache
 * holds ("Pallas Kernel: vLLM on TPU ...", S5).  The pages fix neither the
 * fp8 format nor the scale layout; here every element is one byte in the OCP
 * FP8 E4M3 format (sign, 4 exponent bits of bias 7, 3 mantissa bits,
 * subnormals, NaN at 0x7f / 0xff, no infinity; largest value 448), and K and
 * V each have one float32 scale per KV head: element (page, slot, g, i)
 * stands for e4m3(byte) * scale[g].
 *
 *   k_pages, v_pages  device, uint8 [P, page_size, Hkv, D] row-major (16-byte
 *                 aligned), E4M3 bytes; bytes past a sequence's kv_len and
 *                 pages it does not reach are never read into the result
 *   k_scales, v_scales  device, float32 [Hkv], finite (read by the kernels;
 *                 the caller keeps them valid until the work is done)
 *   all other arguments as for rpa_forward (q and out stay bf16)
 *
 * The work is planned as for rpa_forward.  The split-KV decode kernel reads
 * the bytes itself and converts them to bf16 exactly in registers (the K
 * scale joins the score scale, the V scale the output weight).  The
 * sequences the prefill kernel serves take one of two routes
 * (RPA_OPT_FP8_STAGE; by default chosen by head size): the prefill kernel
 * loads each E4M3 tile into LDS and converts it there exactly (the scales
 * applied as in the decode kernel), or a staging kernel first converts
 * their pages to bf16 (value times scale, rounded to nearest even) in a
 * pool the context owns (grown on demand, like the split workspace), which
 * the prefill kernel then reads through the pool's own page table; all run
 * on `stream`.  With RPA_OPT_PATH = 3 every token goes through the decode
 * kernel instead (no staging).  Errors as for rpa_forward, plus
 * RPA_ERR_INVALID_ARG for a NULL scale array.
 */
int rpa_forward_fp8(rpa_ctx* ctx, const void* q, const void* k_pages, const void* v_pages, const float* k_scales,
                    const float* v_scales, const int32_t* page_table, const int32_t* cu_q_lens,
                    const int32_t* kv_lens, int32_t num_seqs, int32_t window, float scale, void* out,
                    void* stream);

/*
 * rpa_forward_fp8_append -- rpa_forward_append for an fp8 cache: the step's
 * new keys and values (bf16, as for rpa_forward_append) are quantized into
 * their page slots, then the attention of rpa_forward_fp8 runs, in one call
 * (the pages' kernel writes the new tokens' K/V within the attention call:
 * "TPU Deep Dive", chapter 8).  Each new element x of KV head g is stored
 * as the E4M3 byte nearest to x / scale[g] (the division in float32; ties to
 * an even last mantissa bit; magnitudes beyond 448 stored as +-448; NaN as
 * 0x7f).  Arguments as for rpa_forward_fp8 plus k_new / v_new; errors as for
 * rpa_forward_append and rpa_forward_fp8.
 */
int rpa_forward_fp8_append(rpa_ctx* ctx, const void* q, const void* k_new, const void* v_new, void* k_pages,
                           void* v_pages, const float* k_scales, const float* v_scales, const int32_t* page_table,
                           const int32_t* cu_q_lens, const int32_t* kv_lens, int32_t num_seqs, int32_t window,
                           float scale, void* out, void* stream);

/* rpa_destroy -- free a context (NULL-safe).  The caller must first make sure
 * no work enqueued with it is still running, and must not replay a graph
 * that captured one of its calls afterwards. */
void rpa_destroy(rpa_ctx* ctx);

/*
 * rpa_release_captured -- declare that no graph holding a captured call of
 * this context will be replayed again (and none is running).  The work
 * lists, workspaces and staging pools that captures pinned become ordinary
 * cache entries again (evictable; retired pools are freed).  Returns RPA_OK,
 * RPA_ERR_INVALID_ARG for a NULL context, or RPA_ERR_HIP.
 */
int rpa_release_captured(rpa_ctx* ctx);

/* rpa_status_string -- static text of a status code. */
const char* rpa_status_string(int status);

/* rpa_last_error -- message of the context's last failing call ("" if none). */
const char* rpa_last_error(const rpa_ctx* ctx);

/*
 * Tuning options (rpa_set_option).  Every option changes only how the work is
 * scheduled, never what is computed: block sizes change scheduling, not
 * arithmetic ("Chasing speed of light on TPU v6e", footnote 6 of section
 * Attention; "Pallas Kernel: vLLM on TPU ...", S7).
 */
enum {
  RPA_OPT_DECODE_SPLIT_KEYS = 1, /* keys per split of a decode item; 0 = automatic
                                    (a positive value is rounded up to 32)      */
  RPA_OPT_PATH = 2,              /* 0 automatic, 1 every sequence through the
                                    prefill kernel, 2 decode kernel wherever the
                                    rows of a sequence fit one decode item,
                                    3 every token through the decode kernel
                                    (longer sequences in chunks of
                                    decode-item rows; with G > 16 the
                                    prefill kernel keeps them)                  */
  RPA_OPT_DECODE_MAX_ROWS = 4,   /* most q_len * G rows of a sequence that the
                                    decode kernels take (items of up to 16 rows
                                    run the one-block decode kernel, of 17..32
                                    the two-block one; head size 512: at most
                                    16); 0 (default) = the tuning table: 16 for
                                    a bf16 cache, 32 for an fp8 cache          */
  RPA_OPT_DECODE_WAVES = 5,      /* waves per decode workgroup: 0 automatic
                                    (4), 4, 8 (head size 512 always runs 4)     */
  RPA_OPT_KERNEL_TIMING = 6,     /* n > 0: time up to n launches per kernel kind
                                    (see rpa_kernel_times); 0 = off (default),
                                    n <= 65536                                  */
  RPA_OPT_XCD_GROUPS = 7,        /* prefill launch order: runs of 4 neighbouring
                                    tiles go to the same one of X chiplets
                                    (workgroup b runs on chiplet b mod X; MI355X
                                    has 8, the default); 0 or 1 = plain
                                    longest-first order; <= 64                  */
  RPA_OPT_FUSED_MERGE = 8,       /* 1 (default): the decode split that
                                    finishes last merges its group's
                                    partials; 0: a separate merge kernel does
                                    (same result).  Prefill splits are always
                                    merged by the merge kernel (a tile's rows
                                    spread over several workgroups)             */
  RPA_OPT_PREFILL_SPLIT_KEYS = 9, /* keys per split of a long prefill item: 0 =
                                    automatic (split only when the longest item
                                    exceeds the average work of a compute unit
                                    by half), -1 = never split, > 0 = split every
                                    item longer than 1.5x this many keys (rounded
                                    up to 256, at least 512 for items of full
                                    tiles); <= 2^30                              */
  RPA_OPT_CONCURRENT = 10,       /* 1 (default): when a step has both decode
                                    and prefill items, the decode kernel runs
                                    on a second stream of
                                    the context, forked from and joined back
                                    into the caller's stream; 0: both kernels
                                    on the caller's stream                      */
  RPA_OPT_FP8_STAGE = 11         /* fp8 calls with prefill items: 1 a staging
                                    kernel first converts the pages those
                                    items read into a bf16 pool (value times
                                    scale, rounded to bf16) that the bf16
                                    prefill kernel reads; 0 the prefill kernel
                                    loads the E4M3 tiles (half the bytes) and
                                    converts them to bf16 in LDS itself; 2
                                    (default) by head size: 0 for 64 and 256,
                                    whose tiles leave room to convert the next
                                    tile while the current one is used, 1 for
                                    128 and 512                                  */
};
/* Returns RPA_OK or RPA_ERR_INVALID_ARG (unknown option or bad value). */
int rpa_set_option(rpa_ctx* ctx, int32_t option, int64_t value);

/*
 * Kernel timing.  With RPA_OPT_KERNEL_TIMING = n, every rpa_forward records a
 * pair of HIP timing events on its stream directly before and after each
 * kernel it launches, for the first n launches of each kind since the last
 * read.  The events only mark the stream: results are unchanged.
 *
 * rpa_kernel_times -- wait for the recorded launches of `kind` to finish and
 * copy their durations in milliseconds (GPU time between the two events, in
 * launch order) to ms[0 .. min(count, capacity)), set *count to the number
 * recorded, and clear the record of that kind.  `ms` is host memory owned by
 * the caller (may be NULL when capacity is 0).  Returns RPA_OK,
 * RPA_ERR_INVALID_ARG (null ctx/count, bad kind, negative capacity) or
 * RPA_ERR_HIP.
 */
enum { RPA_KERNEL_PREFILL = 0, RPA_KERNEL_DECODE = 1, RPA_KERNEL_MERGE = 2, RPA_KERNEL_APPEND = 3,
       RPA_KERNEL_STAGE = 4 /* rpa_forward_fp8: fp8 pages converted for the prefill kernel */,
       RPA_KERNEL_DECODE2 = 5 /* the two-block (17..32-row) decode kernel */ };
int rpa_kernel_times(rpa_ctx* ctx, int32_t kind, float* ms, int32_t capacity, int32_t* count);

/*
 * Measured-peak probes (diagnostics; no attention arithmetic).  The metric
 * asks for each kernel's throughput against the published peaks and, as a
 * diagnostic, against what the device measurably sustains: these two kernels
 * measure that.  Both enqueue one launch on `stream` (a hipStream_t, NULL for
 * the default stream) and return at once; time them with events on that stream.
 *
 * rpa_probe_read -- stream `bytes` bytes of device memory at `src` (16-byte
 * aligned, bytes a positive multiple of 16) through the compute units: each
 * of `workgroups` (1 .. 65536) workgroups of `threads` threads (256 or 1024)
 * reads one contiguous slice with 16-byte loads, `loads_in_flight` of them
 * per thread at a time (4, 8 or 16; with 256 threads also 32), and every
 * thread writes one 32-bit fold of what it read to `sink` (device memory of
 * workgroups * threads uint32, caller-owned).  Swept over its shapes, the
 * best case for moving that many bytes from HBM into the chip.
 *
 * rpa_probe_mfma -- `workgroups` (1 .. 65536) workgroups of 512 threads, each
 * wave running 4 independent chains of `iterations` (>= 1)
 * v_mfma_f32_32x32x16_bf16 (the prefill kernel's instruction) on register
 * operands; work = workgroups * 8 * iterations * 4 * 32768 FLOP.  Every thread
 * writes one float to `sink` (device memory of workgroups * 512 floats).
 *
 * Return RPA_OK, RPA_ERR_INVALID_ARG (bad pointer or size; nothing enqueued)
 * or RPA_ERR_HIP (launch failure).
 */
int rpa_probe_read(const void* src, int64_t bytes, int32_t workgroups, int32_t threads, int32_t loads_in_flight,
                   void* sink, void* stream);
int rpa_probe_mfma(int32_t workgroups, int32_t iterations, void* sink, void* stream);

/*
 * rpa_probe_e4m3 -- convert `count` (a multiple of 8, 8 .. 2^30) OCP FP8 E4M3
 * bytes at device `src` to bf16 at device `dst` (2 * count bytes), with the
 * conversion rpa_forward_fp8's kernel applies to the cache bytes, on
 * `stream`, asynchronously.  A check of that conversion on its own: every
 * E4M3 value is exact in bf16.  Returns RPA_ERR_INVALID_ARG for NULL pointers
 * or a bad count, RPA_ERR_HIP if the launch fails.
 */
int rpa_probe_e4m3(const void* src, void* dst, int64_t count, void* stream);

/*
 * Planner introspection (host only, no device call).  The host builds the
 * work list that the kernels consume: one item per (sequence, KV head, query
 * tile, key range), the GPU form of the per-sequence metadata the pages'
 * kernel reads ("TPU Deep Dive", chapter 8).
 */
typedef struct rpa_work_item {
  int32_t seq;          /* sequence index                                          */
  int32_t kv_head;      /* KV head g; query heads g*G .. g*G+G-1                   */
  int32_t q_start;      /* first flattened query token of the item                 */
  int32_t q_count;      /* query tokens in the item                                */
  int32_t q_pos0;       /* position of token q_start in its sequence               */
  int32_t kv_begin;     /* first key of the item's range (inclusive)               */
  int32_t kv_end;       /* end of the range (exclusive), <= kv_len                 */
  int32_t split_group;  /* -1: writes the output; else index of its merge group    */
  int32_t split_index;  /* 0 .. num_splits-1 within the group                      */
  int32_t num_splits;   /* splits in the group (1 when split_group == -1)          */
  int32_t partial_base; /* first partial-result slot of the group                  */
  int32_t kind;         /* 0: prefill kernel item, 1: decode kernel item (<= 16
                           rows), 2: two-block decode kernel item (17..32 rows);
                           a split group has the kind of its splits               */
  int32_t self_append;  /* 1: in an appending call with a bf16 cache the item
                           writes K/V rows of new tokens itself: a decode item
                           holding every new token of its sequence (the split
                           whose key range holds them), or split 0 of a
                           prefill item (its own query tokens' rows, KV head
                           kv_head) when the call's prefill launch takes the
                           new rows (see rpa_forward_append); 0: the copy
                           kernel writes them                                */
  int32_t new_pos0;     /* position of the sequence's first new token
                           (kv_len - q_len): an appending call's prefill
                           kernel reads keys from it on from k_new / v_new  */
} rpa_work_item;

typedef struct rpa_plan_info {
  int32_t num_prefill_items;
  int32_t num_decode_items;
  int32_t num_split_groups;
  int32_t num_partials;     /* partial-result slots used (16 rows of d floats each;
                               a prefill split takes prefill_rows / 16 of them)    */
  int32_t prefill_rows;     /* query rows (tokens x grouped heads) per prefill tile */
  int32_t decode_split_keys;/* keys per decode split chosen                         */
  int64_t visible_pairs;    /* visible (query, key) pairs per query head            */
  int32_t prefill_split_keys;/* keys per prefill split chosen, 0 when none split    */
  int32_t reserved;
} rpa_plan_info;

/*
 * rpa_plan -- build the work list for the given metadata without launching.
 * Writes *info and, when items != NULL, up to `capacity` items (prefill items
 * first, then decode items, each in launch order).  Same checks as
 * rpa_forward on the metadata.  Returns RPA_OK or RPA_ERR_INVALID_ARG.
 */
int rpa_plan(rpa_ctx* ctx, const int32_t* cu_q_lens, const int32_t* kv_lens, int32_t num_seqs,
             int32_t window, rpa_plan_info* info, rpa_work_item* items, int32_t capacity);

#ifdef __cplusplus
}
#endif

#endif /* RPA_H */
