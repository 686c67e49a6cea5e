/*
 * pkv.h - paged KV cache and paged decode attention for AMD MI355X (gfx950).
 *
 * A C ABI over plain pointers and sizes.  Device pointers are HIP device
 * memory owned by the caller; the library never allocates or frees device
 * memory and never synchronises a stream.  Every GPU call is asynchronous on
 * the stream it is given (NULL = the default stream).  Host-side argument
 * checks return PKV_ERR_INVALID / PKV_ERR_UNSUPPORTED and set a thread-local
 * message readable with pkv_last_error(); nothing is launched then.
 * Values that live in device memory (table entries, context lengths, slots,
 * copy pairs) are not inspected on the host by the GPU calls; the kernels
 * clamp table entries and skip out-of-range slots and pairs so that a bad
 * value never reads or writes outside the pool, but the numbers they produce
 * for such input are unspecified.  pkv_check_* validate host copies.
 *
 * What the library computes comes from three web pages on the KV cache:
 *   [KVP]  "KV Cache 原理与 PagedAttention" (notebook.any.me.uk)
 *   [BJD]  the bjdmk.com.cn article on KV-cache management (news/6246348)
 *   [AWA]  aiworkagent.org, Transformer architecture, question 17
 * Each declaration names the section it follows.
 *
 * ---------------------------------------------------------------------------
 * Pool layout (this library's choice; the pages fix only the logical
 * structure: fixed-size physical blocks in a preallocated pool, reached
 * through per-sequence block tables - [KVP] §三 工作方式, [AWA]
 * PagedAttention 的关键数据结构).
 *
 *   L = num_layers, NB = num_blocks, B = block_size, H = num_kv_heads,
 *   D = head_dim, e = element bytes (2 for bf16, 1 for fp8-e5m2 and int8),
 *   X = 16 / e (elements per 16-byte piece).
 *
 *   The pool is one caller-owned device buffer split into regions, each
 *   starting at a multiple of 256 bytes from the base, in this order:
 *     K        [L][NB][H][tile]      tile = B*D elements
 *     V        [L][NB][H][tile]
 *     K scales [L][NB][H][B] float   (PKV_KV_INT8: per token and head)
 *              [L][H][D] float       (PKV_KV_INT8_CHANNEL, PKV_KV_INT4,
 *                                     PKV_KV_INT8_KCHANNEL_VTENSOR)
 *     V scales as the K scales (none for PKV_KV_INT8_KCHANNEL_VTENSOR)
 *   Other storage types have no scale regions.
 *   Inside a K tile, element (token t, dim d) is at
 *       ((d / X) * B + t) * X + d % X
 *   i.e. the tile is D/X runs of B 16-byte pieces: the 16 bytes of dims
 *   [X*c, X*c+X) of consecutive tokens are adjacent, so a wavefront reads a
 *   whole 16-token block in fully contiguous 1 KB loads.
 *   Inside a V tile, element (t, d) is at
 *       ((t / 4) * D + d) * 4 + t % 4
 *   i.e. groups of 4 consecutive tokens are stored dim by dim, so the
 *   4 tokens x 1 dim operand of the P.V matrix-core step is one 4e-byte
 *   word and 16 consecutive dims are one contiguous run.
 *   INT4 (two codes per byte, stored as code + 8; a tile is B*D/2 bytes)
 *   has its own placement, in 4-bit nibbles from the tile start, with
 *   P = D / 8 bytes per piece and nibble n of a 32-bit little-endian word
 *   at bits 4n .. 4n+3:
 *     K (t, d):  2 * ((j * B + t) * P + 4 * kk) + n
 *                kk = d / 32, j = (d % 32) / 8, i = d % 8,
 *                n = 4 * (i % 2) + i / 2
 *     V (t, d):  2 * ((g * 16 + m) * P + 4 * (c / 2)) + n
 *                g = t / 4, r = t % 4, c = d / 16, m = d % 16,
 *                n = 4 * (r % 2) + 2 * (r / 2) + c % 2
 *   so that one word widens to the bf16 pairs a matrix-core operand takes
 *   with a mask and an OR, and every V byte belongs to one token.
 *   A slot is block * B + t.  Requirements: D in {64, 128}; B in {8, 16,
 *   32}.
 *
 * Query, output: q is bf16 [S][Hq][D], out is fp32 [S][Hq][D], both dense.
 * Block tables: int32 [S][W], row-major; entry i of row s is the physical
 * block of logical block i of sequence s.  Only entries i < ceil(ctx_s / B)
 * are read.  Context lengths: int32 [S], counting the token being decoded.
 * GQA: query head h reads KV head h / (Hq / H) ([KVP] §一 GQA / MQA).
 * ------------------------------------------------------------------------- */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_ERR_INVALID = -1,        /* bad argument (message in pkv_last_error) */
  PKV_ERR_UNSUPPORTED = -2,    /* valid but not built (e.g. head_dim 96)   */
  PKV_ERR_OUT_OF_BLOCKS = -3,  /* block manager: pool exhausted, no change */
  PKV_ERR_HIP = -4             /* a HIP runtime call failed                */
} pkv_status;

typedef enum {
  PKV_KV_BF16 = 0,       /* K/V stored as bf16                               */
  PKV_KV_FP8_E5M2 = 1,   /* OCP e5m2, one fp32 scale per tensor ([KVP] §四)  */
  PKV_KV_INT8 = 2,       /* symmetric int8, one fp32 scale per (token, head)
                            for K and for V ([BJD] §5.2 量化粒度)             */
  PKV_KV_INT8_TENSOR = 3,  /* int8 codes, one calibrated fp32 scale for all
                              of K and one for V, passed with each call like
                              the fp8 scales ([KVP] §四 INT8 per-tensor;
                              [BJD] §5.2 per-tensor)                        */
  PKV_KV_INT8_CHANNEL = 4, /* int8 codes, one calibrated fp32 scale per
                              (layer, KV head, dim) for K and for V, kept in
                              the pool's scale regions, which the caller
                              fills ([KVP] §四 per-channel; [BJD] §5.2)     */
  PKV_KV_INT4 = 5,         /* symmetric 4-bit codes clamp(round(x / s), -7,
                              7) under calibrated per-(layer, KV head, dim)
                              scales kept as for PKV_KV_INT8_CHANNEL: a
                              quarter of bf16's bytes ([KVP] §四 INT4 KV,
                              which needs calibration)                      */
  PKV_KV_INT8_KCHANNEL_VTENSOR = 6 /* int8 codes, K and V at different
                              granularities ([BJD] §5.2: K, the more
                              sensitive, per channel; V coarser): K under
                              calibrated per-(layer, KV head, dim) scales in
                              the pool's K scale region, V under one
                              calibrated scale per tensor passed with each
                              call (pkv_kv_scales.v_scale)                  */
} pkv_kv_dtype;

typedef struct {
  int32_t num_layers;
  int32_t num_blocks;     /* physical blocks per layer                      */
  int32_t block_size;     /* tokens per block, B                            */
  int32_t num_kv_heads;   /* H                                              */
  int32_t head_dim;       /* D                                              */
  int32_t kv_dtype;       /* pkv_kv_dtype                                   */
} pkv_pool_config;

/* Filled by kv_pool_create; plain data, may be copied freely.  Pointers are
 * device addresses inside the caller's buffer.  k_scale / v_scale: for
 * PKV_KV_INT8 the per-(token, head) scales [L][NB][H][B] the cache write
 * fills; for PKV_KV_INT8_CHANNEL and PKV_KV_INT4 the per-channel scales
 * [L][H][D] the caller writes before caching or decoding a layer (element
 * (l, h, d) at (l * H + h) * D + d); for PKV_KV_INT8_KCHANNEL_VTENSOR
 * k_scale as for PKV_KV_INT8_CHANNEL and v_scale NULL; NULL otherwise. */
typedef struct {
  pkv_pool_config cfg;
  void* base;
  uint64_t bytes;
  void* k;
  void* v;
  float* k_scale;
  float* v_scale;
  uint64_t tile_bytes;    /* B * D * e (B * D / 2 for INT4)                  */
  uint64_t layer_bytes;   /* NB * H * tile_bytes: one layer of K (or of V)   */
} pkv_pool;

/* Per-tensor scales of PKV_KV_FP8_E5M2 and PKV_KV_INT8_TENSOR storage, and
 * the V scale (v_scale only) of PKV_KV_INT8_KCHANNEL_VTENSOR: stored = value
 * / scale, value = stored * scale ([KVP] §四: FP8 / INT8 KV with a scale).
 * Those read must be positive and finite (PKV_ERR_INVALID otherwise); the
 * others are not read.  NULL means 1.0 and 1.0. */
typedef struct {
  float k_scale;
  float v_scale;
} pkv_kv_scales;

/* Thread-local message for the last failed call on this thread ("" if none).
 * Error reporting is this library's own; the pages say nothing about it. */
const char* pkv_last_error(void);

/* ------------------------------------------------------------- pool sizing */

/* Bytes of device memory a pool with this configuration needs (regions and
 * their 256-byte alignment included); 0 if the configuration is invalid.
 * The K/V payload is 2 * L * NB * B * H * D * e bytes: the KV-size formula of
 * [KVP] §一 显存占用公式 applied to NB*B token slots per layer. */
uint64_t kv_pool_bytes(const pkv_pool_config* cfg);

/* Largest num_blocks whose pool fits in budget_bytes (cfg->num_blocks is
 * ignored); -1 if the rest of the configuration is invalid.  Sizing the pool
 * from a memory budget follows [BJD] §7.2 显存容量估算 and the
 * gpu-memory-utilization setting of [KVP] §四. */
int64_t kv_pool_num_blocks_for_budget(const pkv_pool_config* cfg, uint64_t budget_bytes);

/* Describe a pool living in dev_mem (device, >= kv_pool_bytes(cfg) bytes,
 * 256-byte aligned): the preallocated pool of fixed-size physical blocks
 * ([AWA] KV Memory Pool; [KVP] §三 工作方式 steps 1-3).  Host only: records
 * pointers, touches no memory. */
pkv_status kv_pool_create(const pkv_pool_config* cfg, void* dev_mem, uint64_t bytes,
                          pkv_pool* out);

/* ------------------------------------------------------------- cache write */

/* Write the K and V of num_tokens new tokens into their slots of one layer
 * ([KVP] §一: each step computes only the newest token's K and V and appends
 * them to the cache; §三 工作方式: the append goes to the slot the block table
 * names).
 *   key, value    device, bf16 [num_tokens][H][D]
 *   slot_mapping  device, int64 [num_tokens]; slot = block * B + t; a
 *                 negative slot (padding) or one >= NB*B writes nothing
 *   scales        host; fp8: stored = e5m2_rne_sat(fp32(x / scale)); NULL=1
 * int8 storage computes per (token, head): scale = fp32(absmax) / 127,
 * code = clamp(rint_even(fp32(x / scale)), -127, 127) (0 if absmax is 0) and
 * writes the scale beside the codes.  INT8_TENSOR uses the same code formula
 * with scales' k_scale / v_scale (positive and finite for fp8 and INT8_TENSOR,
 * PKV_ERR_INVALID otherwise, as for the decode calls);
 * INT8_CHANNEL with the pool's channel scales of this layer (a scale of 0
 * gives code 0); INT8_KCHANNEL_VTENSOR K with the pool's K channel scales,
 * V with scales' v_scale.  Two tokens with the same slot in one call race
 * (pkv_check_slots rejects that). */
pkv_status reshape_and_cache(const pkv_pool* pool, int32_t layer, const void* key,
                             const void* value, const int64_t* slot_mapping,
                             int32_t num_tokens, const pkv_kv_scales* scales,
                             hipStream_t stream);

/* Copy-on-write split: for each row (src, dst) of pairs (device, int64
 * [num_pairs][2]) copy physical block src to dst in every layer - K tile, V
 * tile and int8 scale rows - byte for byte ([BJD] §3.2 Copy-on-Write: the
 * shared block is copied before the writer's table is repointed).  A pair
 * with an index outside [0, NB) is skipped.  A dst that is also some pair's
 * src, or repeated, races (pkv_check_pairs rejects that). */
pkv_status copy_blocks(const pkv_pool* pool, const int64_t* pairs, int32_t num_pairs,
                       hipStream_t stream);

/* Offload and restore: for each row (src, dst) of pairs (device, int64
 * [num_pairs][2]) copy block src of pool `from` to block dst of pool `to` in
 * every layer - K tile, V tile and int8 scale rows - byte for byte.  The
 * bjdmk.com.cn article, §6.1, moves the KV blocks of preempted or idle
 * requests to CPU memory and brings them back when the request is scheduled
 * again (aiworkagent.org question 17, 进阶 item 5: offloading cold KV).  The
 * two pools must have the same configuration apart from num_blocks
 * (PKV_ERR_INVALID otherwise).  Either may live in device memory or in pinned
 * host memory (hipHostMalloc, torch pin_memory) described with
 * kv_pool_create: one kernel reads and writes both directly, host memory
 * through its device mapping; pageable host memory is refused with
 * PKV_ERR_INVALID before any launch.  A pair with src outside [0, from NB) or
 * dst outside [0, to NB) is skipped; a repeated dst races.  Asynchronous on
 * stream: host memory written by a swap-out is complete once the stream is. */
pkv_status swap_blocks(const pkv_pool* from, const pkv_pool* to, const int64_t* pairs, int32_t num_pairs,
                       hipStream_t stream);

/* ------------------------------------------------------------- decode */

/* Workspace bytes paged_attn_decode needs for these sizes on the current
 * device (0 when partition_size is 0: the single-pass form needs none).  The
 * split form's grid is sized to the device's compute units, so a workspace
 * sized on one device model may not fit another.  The pages are silent on
 * splitting a context across workgroups; this scratch (partial softmax
 * states and row counters) is the library's own. */
uint64_t paged_attn_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                    int32_t table_width, int32_t block_size,
                                    int32_t partition_size);

/* Decode attention for one layer: for every sequence s and query head h,
 *   out[s][h] = softmax(scale * q[s][h] . K_s^T) V_s
 * over the ctx_s cached tokens of KV head h / G, gathered through the block
 * table ([BJD] §2.1 for the formula; [KVP] §三 工作方式 step 4 for the gather;
 * [KVP] §一 for the GQA grouping).  Stored 8-bit and 4-bit codes are
 * converted exactly and their scales applied in fp32 ([KVP] §四: dequantise
 * before compute): per-tensor and per-(token, head) K scales multiply the
 * logits, per-channel K scales are folded into the query (q' = q * s_k held
 * as two bf16 parts, hi and lo, ~16 significant bits; the split form folds
 * each query as it loads it, the single-pass forms in a first pass that
 * stages q' in out's rows, so out must not alias q), V scales multiply p
 * (per token) or the output (per tensor, per channel).  ctx_s == 0 gives a
 * zero row.  Arithmetic: bf16 q, fp32 accumulation and softmax; p meets V as
 * two bf16 parts (~16 bits of p) for bf16 storage and in the single-pass
 * form, while the split form meets 8-bit codes (converted exactly to fp16)
 * and 4-bit codes (the exact fp16 values u * 2^-24 or u * 2^-20 of u = code +
 * 8, the scale and 8 * sum(p) taken back exactly after the products) with p
 * rounded to one fp16 (<= 2^-11 relative).  A stored inf or
 * NaN in V gives a non-finite output element (inf may surface as NaN).
 *   out           device fp32 [S][Hq][D]
 *   q             device bf16 [S][Hq][D]
 *   block_tables  device int32 [S][table_width]
 *   context_lens  device int32 [S], each <= table_width * B
 *   kv_dtype      must equal pool->cfg.kv_dtype
 *   kv_scales     host; the per-tensor scales of fp8 and INT8-per-tensor
 *                 storage and the V scale of INT8_KCHANNEL_VTENSOR (NULL =
 *                 1.0), positive and finite; the rest is not read
 *   partition_size 0: single pass, one workgroup per (sequence, KV head), no
 *                 workspace (INT4: one query per sequence through the
 *                 paged_attn_prefill kernel).  Otherwise the split-context form, a positive
 *                 multiple of 32: the work of all sequences and heads is cut
 *                 into equal ranges, one per wavefront of a grid sized to the
 *                 GPU; each range yields one partial result per
 *                 (sequence, KV head) it covers, and the wavefront that
 *                 completes a sequence's KV head merges its partials.  A
 *                 wavefront carries its running softmax across multiples of
 *                 partition_size, which is the same as merging fixed-length
 *                 partitions in order, so the result does not depend on the
 *                 partition size; the size only selects this form.  Too
 *                 many (sequence, KV head) rows for one call (a partial
 *                 buffer over 4 GiB) is PKV_ERR_INVALID.  Needs a device
 *                 workspace of paged_attn_workspace_bytes bytes, 256-byte
 *                 aligned; its contents are scratch (no initialisation
 *                 needed).  Calls sharing a workspace must not overlap in
 *                 time (same stream, or ordered by events).
 * Hq must be a multiple of H. */
pkv_status paged_attn_decode(float* out, const void* q, const pkv_pool* pool, int32_t layer,
                             const int32_t* block_tables, int32_t table_width,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t num_q_heads, float scale, int32_t kv_dtype,
                             const pkv_kv_scales* kv_scales, int32_t partition_size,
                             void* workspace, uint64_t workspace_bytes, hipStream_t stream);

/* Paged prefill: causal attention of a chunk of new tokens per sequence over
 * its cached context.  Sequence s brings n_s = query_start[s+1] -
 * query_start[s] new tokens, the last n_s of its context_lens[s] positions,
 * whose K/V are already in the pool (reshape_and_cache); new token k sits at
 * position ctx_s - n_s + k and attends to positions 0 .. ctx_s - n_s + k,
 * itself included.  This is the prefill that prefix caching leaves to do: the
 * cached prompt prefix is reused and only the rest is computed ([BJD] §4.1;
 * [KVP] §五); a whole prompt is the case n_s = ctx_s, a decode step the case
 * n_s = 1.  Every storage type of the pool, with the arithmetic of
 * paged_attn_decode's single-pass form (INT4 and per-channel INT8: the K
 * channel scales are folded into the query first), except that INT8 per
 * (token, head) and per tensor take q.K in fp16: the codes as 1152 + c
 * (exact) and the query as fp16(q * 2^-8), exact for 2^-6 <= |q| <= 2^23
 * (smaller elements keep an absolute precision of 2^-17; the shift trades
 * those for queries up to 2^23 that fp16 could not hold unshifted), and INT8
 * per tensor and per channel take P.V in fp16, the codes as 1152 + c and p
 * as two fp16 parts.
 *   out           device fp32 [T][Hq][D], T = num_queries = query_start[S]
 *   q             device bf16 [T][Hq][D]
 *   query_start   device int32 [S + 1], non-decreasing, query_start[0] = 0
 *   max_query_len host; >= every n_s (it sizes the grid: spans of 64
 *                 (token, head) pairs per KV head).  Of a chunk longer than
 *                 it, only the first max_query_len tokens are computed (at
 *                 their positions in the whole chunk); the rows of the later
 *                 ones are left unwritten.
 *   block_tables, context_lens, kv_scales as for paged_attn_decode.
 * A query whose position would be negative (n_s > ctx_s) gets a zero row.
 * For per-channel scales, out must not alias q (the folded query is staged
 * in out's rows first). */
pkv_status paged_attn_prefill(float* out, const void* q, const pkv_pool* pool, int32_t layer,
                              const int32_t* block_tables, int32_t table_width, const int32_t* context_lens,
                              const int32_t* query_start, int32_t num_seqs, int32_t num_queries,
                              int32_t max_query_len, int32_t num_q_heads, float scale, int32_t kv_dtype,
                              const pkv_kv_scales* kv_scales, hipStream_t stream);

/* paged_attn_prefill with options (flags; 0 is paged_attn_prefill itself).
 * The pages fix no precision for the products of the softmax weights with
 * V ([KVP] §四 and [BJD] §5 speak only of the KV storage types), so the
 * prefill offers a faster reading beside its default:
 * PKV_PREFILL_P_ONE_PART: each weight p meets V rounded once - to bf16, or
 * to fp16 where V enters the products as fp16 (INT8 per tensor, per
 * channel) - instead of as hi + lo parts, which halves the matrix-core
 * products of P.V (a third of all the products of a step).  The softmax
 * denominator is then the sum of the rounded weights (INT8 per token-head,
 * whose weights carry the V scale: of the unrounded ones), so with u =
 * 2^-8 (bf16) or 2^-11 (fp16) an output element moves by at most about
 * u * (max - min) of the V values its query attends (INT8 per token-head:
 * u * max |V|) beyond the default's error.  Unknown flag bits:
 * PKV_ERR_INVALID.  Arguments, layouts and the other errors as for
 * paged_attn_prefill. */
#define PKV_PREFILL_P_ONE_PART 1u
pkv_status paged_attn_prefill_ex(float* out, const void* q, const pkv_pool* pool, int32_t layer,
                                 const int32_t* block_tables, int32_t table_width, const int32_t* context_lens,
                                 const int32_t* query_start, int32_t num_seqs, int32_t num_queries,
                                 int32_t max_query_len, int32_t num_q_heads, float scale, int32_t kv_dtype,
                                 const pkv_kv_scales* kv_scales, uint32_t flags, hipStream_t stream);

/* One decode step with its cache write in the same launch: for each sequence s
 * with ctx_s > 0, the new token's K and V (key, value: device bf16
 * [S][H][D], 16-byte aligned) are stored at position ctx_s - 1 - the slot the
 * block table names - exactly as reshape_and_cache would store them (same
 * quantisation), and the decode of paged_attn_decode over ctx_s tokens,
 * including that one, is computed.  The result and the pool afterwards equal
 * reshape_and_cache with those slots followed by paged_attn_decode ([KVP] §一:
 * the step computes only K_t, V_t and appends them; §三 工作方式 steps 3-4).
 * The token's block must not be shared with another sequence (copy_blocks
 * first).  Split-context form only: partition_size > 0, else
 * PKV_ERR_UNSUPPORTED.  Other arguments as for paged_attn_decode; kv_scales
 * also give the fp8 encoding scales. */
pkv_status paged_attn_decode_append(float* out, const void* q, const pkv_pool* pool, int32_t layer,
                                    const void* key, const void* value, const int32_t* block_tables,
                                    int32_t table_width, const int32_t* context_lens, int32_t num_seqs,
                                    int32_t num_q_heads, float scale, int32_t kv_dtype,
                                    const pkv_kv_scales* kv_scales, int32_t partition_size, void* workspace,
                                    uint64_t workspace_bytes, hipStream_t stream);

/* Every argument of a decode call in one block, for the options the two
 * calls above do not take.  Fields as for paged_attn_decode_append (key and
 * value NULL for the plain decode), plus:
 *   sliding_window  0: attend to the whole context.  w > 0: attend only to
 *                   the last w positions, [max(0, ctx - w), ctx) - the
 *                   sliding-window KV of "Transformer 架构" (aiworkagent.org)
 *                   question 17, 进阶 item 3 (keep only the most recent N
 *                   tokens).  Blocks that lie wholly before that range are
 *                   never read: their table entries may name any block, e.g.
 *                   one already given back to the pool.  Works in both forms
 *                   (partition_size 0 or > 0); the workspace size does not
 *                   depend on it.  Negative: PKV_ERR_INVALID. */
typedef struct {
  float* out;                  /* device, [S][Hq][D] fp32 */
  const void* q;               /* device, [S][Hq][D] bf16 */
  const pkv_pool* pool;        /* host */
  int32_t layer;
  const void* key;             /* device [S][Hkv][D] bf16 or NULL (appending form when set) */
  const void* value;           /* device, set exactly when key is */
  const int32_t* block_tables; /* device, [S][table_width] */
  int32_t table_width;
  const int32_t* context_lens; /* device, [S] */
  int32_t num_seqs;
  int32_t num_q_heads;
  float scale;
  int32_t kv_dtype;
  const pkv_kv_scales* kv_scales; /* host, or NULL */
  int32_t partition_size;
  int32_t sliding_window;
  void* workspace;             /* device */
  uint64_t workspace_bytes;
  uint32_t flags;              /* 0, or PKV_DECODE_KEEP_KV_CACHED (other bits: PKV_ERR_INVALID) */
} pkv_decode_args;

/* pkv_decode_args.flags.  The split form loads K/V tiles with the
 * non-temporal hint by default: when each sequence's blocks are its own,
 * every tile is read once per call, and streaming it keeps the reused lines
 * (queries, tables, partials) in the L2 and the MALL.  When tables share
 * blocks - sequences forked from one prompt, a cached prefix reused by many
 * requests ([BJD] §3.1, §3.2) - and the call is not
 * paged_attn_decode_shared_prefix, PKV_DECODE_KEEP_KV_CACHED loads them with
 * the default policy, so that the other readers of a shared block find it
 * in the caches.  Results are identical either way; paged_attn_decode and
 * paged_attn_decode_append stream. */
#define PKV_DECODE_KEEP_KV_CACHED 1u

/* Decode with every option: same behaviour, ownership and errors as
 * paged_attn_decode (key == NULL) or paged_attn_decode_append (key set);
 * PKV_ERR_INVALID for a NULL args or a key without a value. */
pkv_status paged_attn_decode_ex(const pkv_decode_args* args, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * decode as paged_attn_decode_ex (plain or appending form, sliding window,
 * every storage type; identical results), with the split form's workspace
 * taken from a static device array of 32 MiB (33554432 bytes) that the
 * library holds on every GPU it runs on until the process ends.  The
 * workspace and workspace_bytes fields are ignored; the caller passes only
 * inputs and outputs.  Nothing is allocated and no allocating routine is
 * called (the array's device address is looked up once per device, on the
 * first call made with that device current).  A call whose split form would
 * need more than 32 MiB - (rows + waves) partial slots of (D / 16) KiB plus
 * 256 bytes each, rows = S * Hkv * ceil(G / 16), waves = 4 per compute unit -
 * returns PKV_ERR_INVALID before any launch (e.g. D = 128: about 2,900 rows
 * with 1,024 waves).  The array keeps the last call's contents; nothing in it
 * needs clearing.  Calls that overlap in time on one GPU share the array and
 * race: order them on one stream or with events. */
pkv_status paged_attn_decode_noalloc(const pkv_decode_args* args, hipStream_t stream);

/* Decode of a batch whose sequences share a cached prompt prefix.  Requests
 * that start with one prompt have tables naming the same physical blocks for
 * it ([BJD] §3.1), and a prompt shared by many requests is held once ([BJD]
 * §3.2: a 1500-token system prompt for 200 concurrent requests).  The result
 * is paged_attn_decode_ex's for tables whose first prefix_len / B entries
 * are prefix_table; the pages describe the sharing of the blocks, not how
 * attention over them is computed.  Here the shared blocks are read once
 * per KV head for the whole batch instead of once per sequence:
 *   1. the split-context form attends each sequence's own positions
 *      [prefix_len, ctx_s) and keeps every output row's softmax state;
 *   2. a second launch attends, per KV head, the prefix positions
 *      [0, min(ctx_s, prefix_len)) of all (sequence, query head) pairs
 *      together - their queries are the columns of the matrix-core products,
 *      as paged_attn_prefill's tokens are; a workgroup's four waves share
 *      its columns and split the prefix's keys - and merges the partial
 *      states with the first pass's rows (exact softmax merge, fp32).
 *   args          as for paged_attn_decode_ex (plain or appending form, every
 *                 storage type); partition_size must be positive and
 *                 sliding_window 0, else PKV_ERR_UNSUPPORTED; the workspace
 *                 (256-byte aligned, scratch) must hold
 *                 paged_attn_shared_prefix_workspace_bytes bytes.
 *   prefix_table  device int32 [prefix_len / B]: the physical blocks of
 *                 positions [0, prefix_len), read for every sequence in place
 *                 of the first prefix_len / B entries of its own table row
 *                 (those are not read and may hold anything).
 *   prefix_len    >= 0 and a multiple of B (else PKV_ERR_INVALID); 0 is
 *                 paged_attn_decode_ex.
 * A sequence with ctx_s <= prefix_len attends its first ctx_s positions,
 * all in the prefix; in the appending form nothing is written for it (its
 * new token would land in a shared block, which a caller copies first).
 * Arithmetic: the split form's for each sequence's own positions,
 * paged_attn_prefill's (single-pass decode arithmetic) for the prefix.
 * Launches: the split kernel, the query fold for storage with K channel
 * scales, the prefix pass; asynchronous on `stream`. */
pkv_status paged_attn_decode_shared_prefix(const pkv_decode_args* args, const int32_t* prefix_table,
                                           int32_t prefix_len, hipStream_t stream);

/* Workspace bytes paged_attn_decode_shared_prefix needs on the current
 * device for any batch of at most num_seqs sequences (the split form's
 * workspace, each row's softmax state, and the folded query for storage
 * with K channel scales); 0 for sizes that are invalid or too large for one
 * call. */
uint64_t paged_attn_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                                  int32_t head_dim, int32_t table_width, int32_t block_size,
                                                  int32_t kv_dtype, int32_t prefix_len);

/* ------------------------------------------------------------- host checks
 * Validators over HOST copies of device inputs, for callers that want to
 * rule out racing or out-of-range values before a launch.  Return PKV_OK or
 * PKV_ERR_INVALID with a message naming the first bad entry.  The pages say
 * nothing about validation; what is checked follows from the layout above:
 *   pkv_check_slots   every slot in [0, num_slots) or negative (padding),
 *                     no slot twice;
 *   pkv_check_pairs   src and dst in [0, num_blocks), no dst twice, no dst
 *                     that is also a src;
 *   pkv_check_tables  each context length in [0, table_width * block_size]
 *                     and the first ceil(ctx / B) entries of its row in
 *                     [0, num_blocks). */
pkv_status pkv_check_slots(const int64_t* slots, int32_t n, int64_t num_slots);
pkv_status pkv_check_pairs(const int64_t* pairs, int32_t n, int32_t num_blocks);
pkv_status pkv_check_tables(const int32_t* tables, const int32_t* context_lens, int32_t num_seqs,
                            int32_t table_width, int32_t block_size, int32_t num_blocks);

/* ------------------------------------------------------------- block manager
 * Host-only bookkeeping of the pool ([KVP] §三 工作方式 steps 1-3: blocks
 * handed out on demand and reused; [AWA] KV Memory Pool; [BJD] §3.1-3.2
 * sharing and copy-on-write).  Rules fixed by this library:
 *  - free blocks form a FIFO; the caller gives the initial order (a
 *    permutation of 0..NB-1, or NULL for 0..NB-1); allocation pops the front,
 *    blocks whose count drops to 0 are pushed to the back in table order;
 *  - a sequence of n tokens holds ceil(n / B) blocks;
 *  - appending to a sequence of length n writes position n: if n % B == 0 a
 *    new block is appended; else if the last block is shared (count > 1) a
 *    new block dst is taken, (src, dst) is reported for copy_blocks, src's
 *    count drops by one and dst replaces it in this table; the slot is
 *    table[n / B] * B + n % B;
 *  - a batch append handles sequences in the order given and is all or
 *    nothing: if the pool cannot supply every block it needs, it returns
 *    PKV_ERR_OUT_OF_BLOCKS, counts one failed allocation, changes nothing.
 * Not thread-safe: one manager per thread, or external locking. */
typedef struct pkv_bm pkv_bm;

/* A manager of num_blocks blocks of block_size tokens, all free, in the
 * given FIFO order ([AWA] KV Memory Pool: fixed-size blocks preallocated and
 * handed to sequences on demand).  *out receives it; free with
 * kv_bm_destroy (host memory only; the pages are silent on teardown). */
pkv_status kv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* initial_order,
                        pkv_bm** out);
void kv_bm_destroy(pkv_bm* bm);
/* New sequence holding ctx_len tokens (ceil(ctx_len / B) fresh blocks; [KVP]
 * §三 工作方式 step 2: its block table maps logical block i to physical
 * block p). */
pkv_status kv_bm_add_seq(pkv_bm* bm, int32_t seq, int32_t ctx_len);
/* child shares all of parent's blocks (counts + 1) and its length ([BJD]
 * §3.1: two requests with the same prefix point their tables at the same
 * physical blocks; §3.2: the share holds until one of them writes). */
pkv_status kv_bm_fork(pkv_bm* bm, int32_t parent, int32_t child);
/* Append one token to each of seqs[0..n) (host arrays).  slots: int64 [n]
 * out; cow_pairs: int64 [n][2] out; *num_pairs: pairs written ([KVP] §三
 * 工作方式 step 3: a new block only when the last one is full; [BJD] §3.2
 * copy-on-write of a shared last block). */
pkv_status kv_bm_append(pkv_bm* bm, const int32_t* seqs, int32_t n, int64_t* slots,
                        int64_t* cow_pairs, int32_t* num_pairs);
/* Drop a sequence: each of its blocks loses one reference and returns to
 * the free FIFO at 0 ([KVP] §三 工作方式 step 3: blocks are released when
 * done and the pool reuses them). */
pkv_status kv_bm_free_seq(pkv_bm* bm, int32_t seq);
/* Rows of tables (host int32 [n][width]) for seqs[0..n), padded with 0, and
 * their lengths (context_lens may be NULL) - the per-sequence block tables
 * of [AWA] PagedAttention 的关键数据结构, for upload before a decode. */
pkv_status kv_bm_block_tables(const pkv_bm* bm, const int32_t* seqs, int32_t n, int32_t* tables,
                              int32_t width, int32_t* context_lens);
/* used = blocks referenced by some table; total = NB ([KVP] §六 cache usage);
 * failed_allocs = calls refused for lack of blocks ([KVP] §六 preemptions). */
pkv_status kv_bm_stats(const pkv_bm* bm, int32_t* used, int32_t* total, int64_t* failed_allocs);
/* Reference count of one block: the number of tables naming it (the
 * sharing count [BJD] §3.2's copy-on-write decision reads); for tests and
 * leak checks; -1 for a block outside [0, NB). */
int32_t kv_bm_ref_count(const pkv_bm* bm, int32_t block);

/* Prefix caching ([BJD] §4.1: a request whose prompt starts like an earlier
 * one reuses that prompt's KV blocks and skips their prefill; §4.3: only an
 * exact, position-aligned prefix qualifies).  Rules fixed by this library:
 *  - a full block i of a prompt (tokens [iB, (i+1)B)) has the key
 *    SHA-256(key(i-1) || its B token ids as little-endian int32), key(-1) =
 *    32 zero bytes, so a key names the whole prefix up to that block;
 *  - kv_bm_add_seq_tokens reuses, for the longest run of leading full blocks
 *    whose keys are cached and which lie wholly before the prompt's last
 *    token (at most (n - 1) / B blocks), those blocks (count + 1, also when
 *    they were free); every other block is fresh, and each fresh full block
 *    becomes the cached holder of its key (the previous holder, if any, loses
 *    it); the partial last block and blocks filled later by appends are never
 *    cached; *cached_tokens = reused blocks * B < n, the prefix whose KV is
 *    already in the pool: the caller computes the rest, which always holds
 *    at least the last prompt token (its forward pass yields the first new
 *    token, and its K/V never lands in a block another sequence shares);
 *  - a cached block whose count drops to 0 keeps its key and content while
 *    it waits on the free FIFO; it leaves the cache only when allocation
 *    takes it, so the least recently freed cached block is evicted first;
 *  - all or nothing, like the other calls: PKV_ERR_OUT_OF_BLOCKS with no
 *    change when the free blocks cannot cover the fresh ones.
 * The caller must write the KV of fresh blocks before another request can
 * reuse them (same stream order as the decode that follows). */
pkv_status kv_bm_add_seq_tokens(pkv_bm* bm, int32_t seq, const int32_t* tokens, int32_t n,
                                int32_t* cached_tokens);
/* Lookups (blocks eligible for reuse, as above) and hits of
 * kv_bm_add_seq_tokens so far ([KVP] §六 hit rate) and the number of keys
 * currently cached. */
pkv_status kv_bm_prefix_stats(const pkv_bm* bm, int64_t* lookups, int64_t* hits, int32_t* cached_blocks);
/* The key of a block: SHA-256 of parent (32 bytes; NULL = zeros) followed by
 * tokens[0..n) as little-endian int32 (host arrays; out: 32 bytes) - the
 * prefix hash of [BJD] §4.1 (the pages name no hash function; SHA-256 is this
 * library's choice). */
pkv_status kv_bm_block_key(const uint8_t* parent, const int32_t* tokens, int32_t n, uint8_t* out);

/* Radix-tree prefix cache, the alternative to the hash chain above ([BJD]
 * §4.2: the cached KV forms a tree over token sequences; a request reuses
 * its longest matching prefix, also a partial one, and computes and inserts
 * the rest; under memory pressure the least recently used leaves go first,
 * so shared prefixes outlive the branches using them).  A manager uses one
 * of the two caches: the first successful call picks it, and a call of the
 * other kind then returns PKV_ERR_UNSUPPORTED.  With paged storage a node is
 * a full prompt block: its B token ids, under the node of the block before
 * it (block 0 under the root).  Rules fixed by this library:
 *  - matching walks from the root through the child whose B tokens equal
 *    the prompt's next block, while that block lies wholly before the
 *    prompt's last token (which is always computed, as above); in the first
 *    block not matched whole, the child sharing the longest run of leading
 *    tokens (capped at the last token; the earliest inserted among equals)
 *    gives l > 0 further tokens: the sequence gets a fresh block there and
 *    copy_pair = (that child, the fresh block), which the caller copies
 *    (copy_blocks) before computing tokens from *cached_tokens on, so the
 *    copy carries the l matched tokens' K/V; else copy_pair = (-1, -1);
 *    *cached_tokens = B * (whole blocks matched) + l < n;
 *  - fresh blocks come from the free FIFO (blocks outside the tree) while it
 *    has any, else by evicting the tree leaf nobody references that was used
 *    longest ago (then the deeper, then the lower block id); a block is used
 *    when matched (whole or as the copy source) and when a kv_bm_free_seq
 *    drops its count to 0 - a tree block at count 0 stays in the tree, its
 *    K/V intact, until evicted; every kv_bm_free_seq and every successful
 *    kv_bm_add_seq_radix is one tick of that clock;
 *  - the prompt's fresh full blocks are inserted in order as a chain under
 *    the last block matched whole; a block whose tokens a sibling already
 *    holds (only when the last token cut a whole match short) and the blocks
 *    after it are not inserted; partial last blocks and appended tokens are
 *    never cached;
 *  - all or nothing: PKV_ERR_OUT_OF_BLOCKS with no change when the free FIFO
 *    and the evictable tree blocks (those nobody references, less the ones
 *    this request matches) cannot cover the fresh blocks;
 *  - kv_bm_stats counts tree blocks nobody references as free.
 * tokens: host int32 [n]; copy_pair: host int64 [2], required. */
pkv_status kv_bm_add_seq_radix(pkv_bm* bm, int32_t seq, const int32_t* tokens, int32_t n,
                               int32_t* cached_tokens, int64_t* copy_pair);
/* Tokens eligible for reuse and tokens reused by kv_bm_add_seq_radix so far
 * ([KVP] §六 hit rate, per token), the blocks in the tree, and those of them
 * nobody references (evictable). */
pkv_status kv_bm_radix_stats(const pkv_bm* bm, int64_t* lookup_tokens, int64_t* hit_tokens, int32_t* cached_blocks,
                             int32_t* idle_blocks);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
