/*
 * moe.h -- C ABI of libmoe: the routed-expert MoE layer forward for MI355X
 * (gfx950), with a VRAM expert cache over a pinned host expert pool.
 *
 * The operation.  FreeToken keeps the full expert pool in host memory and
 * treats VRAM as a cache of experts ("FreeToken github moe: Setup Guide &
 * MoE Runtime Comparison", introduction; "FreeToken Inference Engine: 3x
 * Speed Boost for MoE Models", section "From Static Allocation to Dynamic
 * Scheduling").  Expert banks are ggml blocks of the standard types
 * (Q4_0, Q4_1, Q5_0, Q5_1, Q8_0) or the K-quants Q4_K, Q5_K in one GPU slot
 * pool of a single type (FreeToken fork README, "Quant types" and "Known
 * limits"); decode and prefill use different kernel families there (matrix
 * x vector for decode, matrix x matrix for prefill, same section).  One
 * layer forward is:
 *   logits -> softmax -> top-k (ties to the lower expert id) -> renormalise
 *   -> expert id to slot -> group (token, expert) pairs by expert
 *   -> per pair: h = silu(Wg x) * (Wu x), y = Wd h  -> out[t] = sum_j w_tj y_tj
 *
 * Conventions (all entry points).
 *  - Return value: MOE_OK (0) or a negative MOE_ERR_* code.  An unsupported
 *    block type is an error, never a silently empty result (the fork README,
 *    "What else changed", describes the bug where an unknown type returned
 *    uninitialised memory and a block-size query returned 0).
 *    moe_last_error() returns a thread-local message naming the offending
 *    argument, layer, expert or type.
 *  - Pointers: "device" pointers are HIP device memory of the context's
 *    device (for example torch tensors' data_ptr()); "host" pointers are
 *    ordinary process memory.  The caller owns every buffer and every
 *    stream; the library never allocates device memory in a compute call.
 *    Streams are hipStream_t values passed as void* (NULL = default stream).
 *  - All shape, type and alignment checks run on the host before any
 *    launch.  Compute calls are stream ordered and do not synchronise, so
 *    on success outputs are valid once the stream reaches the call.
 *  - A fault that only the device can see (an expert whose slot is -1, that
 *    is not resident) sets the context's sticky device error word and
 *    writes NaN to that expert's outputs; moe_ctx_check() reports it.
 *  - Shapes: H and I must be multiples of 256 (eight 32-weight blocks);
 *    1 <= k <= E <= 1024.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ------------------------------------------------------------------ codes */
enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,
  MOE_ERR_UNSUPPORTED_QTYPE = -2,
  MOE_ERR_MIXED_QTYPE = -3,
  MOE_ERR_ALIGNMENT = -4,
  MOE_ERR_WORKSPACE = -5,
  MOE_ERR_NOT_RESIDENT = -6,
  MOE_ERR_NOT_PINNED = -7,
  MOE_ERR_CAPACITY = -8,
  MOE_ERR_HIP = -9
};

/* Block types, numbered as in ggml's type enum. */
enum {
  MOE_QTYPE_Q4_0 = 2,
  MOE_QTYPE_Q4_1 = 3,
  MOE_QTYPE_Q5_0 = 6,
  MOE_QTYPE_Q5_1 = 7,
  MOE_QTYPE_Q8_0 = 8,
  MOE_QTYPE_Q4_K = 12,
  MOE_QTYPE_Q5_K = 13
};

/* Activation dtypes. */
enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 };

/* Expert FFN kernel families: matrix x vector decode with fp32 activations
 * and fp32 accumulation, or grouped matrix x matrix prefill with bf16
 * operands on the matrix cores and fp32 accumulation (fork README, "Quant
 * types": separate decode and prefill kernels per block type). */
enum { MOE_MODE_DECODE = 0, MOE_MODE_PREFILL = 1, MOE_MODE_DECODE_Q8A = 2 };
/* MOE_MODE_DECODE_Q8A: decode with 8-bit activations against the raw
 * 4- or 8-bit weight codes (the fork README's W4A8 decode scheme, section
 * "DeepSeek-V4-Flash", which states that it cannot agree bit for bit with
 * a float reference).  x (fp32) and then the h rows are quantised per
 * block of 32: s = max|v| / 127, code = v / s rounded half away from zero
 * (both divisions in fp32; s = 0 gives codes 0); every block dot product is
 * an exact integer sum of code products scaled by d * s in fp32.  Q4_0 and
 * Q8_0 banks only (others -> MOE_ERR_UNSUPPORTED_QTYPE), T*k <= 1024.  The
 * workspace (moe_expert_ffn_workspace_size) also holds the quantised rows. */

/* What cache_decode_layer does with an expert that is not in VRAM:
 * MOE_MISS_COPY copies it in (it becomes resident); MOE_MISS_HOST computes
 * its FFN on the host cores from the pinned pool (it stays out of the
 * cache); MOE_MISS_QSTAR splits each layer's misses between the two;
 * MOE_MISS_HOST_COPY computes it on the host and copies it in behind. */
enum { MOE_MISS_COPY = 0, MOE_MISS_HOST = 1, MOE_MISS_QSTAR = 2, MOE_MISS_HOST_COPY = 3 };

typedef struct moe_ctx moe_ctx;
typedef struct moe_cache moe_cache;

/* Thread-local description of the last error of this thread ("" if none). */
const char* moe_last_error(void);

/* ---------------------------------------------------------------- context
 * moe_ctx_create: binds device `device`, allocates the 4-byte device error
 * word, and creates a second stream (default priority, non-blocking) with
 * two events: decode batches of 32 or more tokens run the matrix-core
 * experts' kernels there, forked from and joined back into the caller's
 * stream within the call (this also holds under HIP graph capture).  Calls
 * that share a context are issued from one host thread at a time.
 * moe_ctx_check: waits for `stream`, reads and clears the error word;
 * returns MOE_ERR_NOT_RESIDENT if a kernel met a slot of -1 since the last
 * check (the message names the expert).  moe_ctx_destroy frees the word,
 * the stream and the events. */
int moe_ctx_create(int device, moe_ctx** out);
int moe_ctx_destroy(moe_ctx* ctx);
int moe_ctx_check(moe_ctx* ctx, void* stream);

/* Per-kernel timing for profiling.  moe_ctx_set_timing(ctx, 1) makes every
 * later launch of this context carry a start and a stop HIP event bound to
 * the launch itself (hipExtLaunchKernel), so their elapsed time is the
 * kernel's execution on its stream (launches inside a stream capture are
 * not timed); enabling or disabling discards earlier records.  moe_ctx_kernel_time waits for the
 * recorded launches of `kernel` (names: "router_logits", "topk", "permute",
 * "ffn_gateup", "ffn_down", "combine", "dequant", "topk_permute",
 * "permute_count", "permute_scan", "permute_scatter", "quant_act",
 * "ffn_gateup_mfma", "ffn_down_mfma") and
 * returns their number
 * and summed duration in milliseconds. */
int moe_ctx_set_timing(moe_ctx* ctx, int enable);
int moe_ctx_kernel_time(moe_ctx* ctx, const char* kernel, int* count,
                        double* total_ms);

/* ------------------------------------------------------------ block types
 * The standard ggml types (fork README, "Quant types"), 32 weights per
 * block, fields little endian in this order:
 * Q8_0: fp16 d, 32 int8 q (34 B), w = d*q.
 * Q4_0: fp16 d, 16 nibble bytes (18 B), w = d*(q-8), q in 0..15.
 * Q4_1: fp16 d, fp16 m, 16 nibble bytes (20 B), w = d*q + m, q in 0..15.
 * Q5_0: fp16 d, 4 bytes of fifth bits, 16 nibble bytes (22 B),
 *       w = d*(q-16), q in 0..31.
 * Q5_1: fp16 d, fp16 m, 4 bytes of fifth bits, 16 nibble bytes (24 B),
 *       w = d*q + m, q in 0..31.
 * Nibble byte j holds element j (low nibble) and element j+16 (high
 * nibble); bit j of the little-endian fifth-bit word is bit 4 of element j.
 * The K-quant Q4_K (the fork README's "K-quants" row) is a super-block of
 * 256 weights (144 B): fp16 d, fp16 dmin, 12 bytes of 6-bit scale and min
 * codes of its 8 sub-blocks of 32 (sub-block j < 4: scale = byte j & 63,
 * min = byte j+4 & 63; j >= 4: scale = (byte j+4 & 15) | (byte j-4 >> 6)
 * << 4, min = (byte j+4 >> 4) | (byte j >> 6) << 4), 128 nibble bytes
 * (bytes 32i..32i+31: sub-block 2i low nibbles, 2i+1 high, element l in
 * byte 32i + l); weight l of sub-block j = d * scale_j * q - dmin * min_j.
 * moe_qtype_info reports its super-block (256, 144).
 * Q5_K is Q4_K with a fifth code bit (176 B): fp16 d, fp16 dmin, the same
 * 12 scale bytes, 32 bytes qh, 128 nibble bytes as in Q4_K; bit j of qh
 * byte l is bit 4 of element l of sub-block j, so q in 0..31 and weight l
 * of sub-block j = d * scale_j * q - dmin * min_j; super-block (256, 176).
 * Unknown qtype -> MOE_ERR_UNSUPPORTED_QTYPE and the outputs untouched. */
int moe_qtype_info(int qtype, int* block_elems, int* block_bytes);

/* -------------------------------------------------------------- packing
 * Device layout of one expert slot (same byte count as the ggml blocks):
 * gate [I rows][H], up [I rows][H], down [H rows][I], each matrix row-major
 * by rows, each row a sequence of groups of 8 blocks; a group is the 8
 * blocks' quant bytes (ggml order, 8*32 B for Q8_0, 8*16 B otherwise),
 * then for Q5_0 / Q5_1 their 8 fifth-bit words (32 B), then their 8 fp16
 * scales d (16 B), then for Q4_1 / Q5_1 their 8 fp16 offsets m (16 B), so
 * every group is 16-B aligned.  A Q4_K group is one super-block (144 B):
 * its 8 sub-blocks' 16 quant bytes each (nibble order as above: byte j
 * holds elements j and j+16 of the sub-block), the 12 scale bytes, d, dmin.
 * A Q5_K group (176 B) is the same with the 8 sub-blocks' fifth-bit words
 * (32 B, bit j for element j, as in Q5_0) between the quant bytes and the
 * scale bytes.
 * The pinned host pool holds experts in this same layout, so staging an
 * expert into VRAM is one verbatim copy ("FreeToken Inference Engine",
 * FTW paragraph: load straight into the engine's layout, no repacking).
 *
 * moe_slot_bytes: bytes of one expert slot.
 * moe_pack_expert (host): ggml blocks of gate [I][H/32], up [I][H/32],
 * down [H][I/32] (host memory) -> `dst` (host memory, dst_bytes >= slot).
 * moe_pack_matrix (host): one [rows][cols/32] block matrix -> device layout. */
int moe_slot_bytes(int qtype, int H, int I, size_t* out_bytes);
int moe_pack_expert(int qtype, int H, int I, const void* gate_blocks,
                    const void* up_blocks, const void* down_blocks, void* dst,
                    size_t dst_bytes);
int moe_pack_matrix(int qtype, int rows, int cols, const void* blocks,
                    void* dst, size_t dst_bytes);

/* ----------------------------------------------------------------- route
 * Router softmax and top-k with renormalisation, for T tokens.
 *   x          device, [T][H] in x_dtype (ignored when logits_in != NULL)
 *   router_w   device fp32 [E][H] (row e maps hidden -> logit e)
 *   bias       device fp32 [E] added to the logits, or NULL
 *   logits_in  device fp32 [T][E] given logits, or NULL to compute x.Wr^T
 *   logits_out device fp32 [T][E]: the logits the selection used (bias
 *              included); required when the logits are computed from x,
 *              optional (may be NULL) with logits_in
 *   topk_ids   device int32 [T][k]: the k largest logits, ordered by
 *              (logit desc, id asc); equal logits go to the lower id
 *   topk_w     device fp32 [T][k]: softmax probabilities of the chosen
 *              experts renormalised to sum 1
 * Selection is decided on the fp32 logits. */
int moe_route(moe_ctx* ctx, const void* x, int x_dtype, const float* router_w,
              const float* bias, const float* logits_in, int T, int H, int E,
              int k, float* logits_out, int32_t* topk_ids, float* topk_w,
              void* stream);

/* --------------------------------------------------------------- permute
 * Groups the P = T*k pairs p = t*k + j by expert, stably (pair order kept
 * inside an expert).  All device int32:
 *   expert_offsets [E+1]: exclusive prefix sum of per-expert pair counts
 *   sorted_pairs   [P]  : pairs of expert e at [offsets[e], offsets[e+1])
 *   pair_pos       [P]  : inverse: sorted_pairs[pair_pos[p]] == p
 *   active         [E+1]: active[0] = number of experts with pairs, then
 *                         those expert ids ascending
 * ws: device workspace (4-byte aligned) of moe_permute_workspace_size()
 * bytes, 0 up to P = 4096 pairs and 2 x chunks x E x 4 above (chunks of
 * 512 pairs), used for the per-chunk expert counts and bases of a grouping
 * spread over many workgroups.  A NULL or smaller workspace selects the single-
 * workgroup grouping instead: same results, slower for large P. */
int moe_permute_workspace_size(int T, int k, int E, size_t* bytes);
/* moe_route_permute: moe_route followed by moe_permute with the top-k and
 * the grouping in one launch, for decode-sized batches (T*k <= 4096;
 * larger batches run the separate kernels, with ws as for moe_permute).
 * Same arguments and results. */
int moe_route_permute_workspace_size(int T, int k, int E, size_t* bytes);
int moe_route_permute(moe_ctx* ctx, const void* x, int x_dtype,
                      const float* router_w, const float* bias,
                      const float* logits_in, int T, int H, int E, int k,
                      float* logits_out, int32_t* topk_ids, float* topk_w,
                      int32_t* expert_offsets, int32_t* sorted_pairs,
                      int32_t* pair_pos, int32_t* active, void* ws,
                      size_t ws_bytes, void* stream);
int moe_permute(moe_ctx* ctx, const int32_t* topk_ids, int T, int k, int E,
                int32_t* expert_offsets, int32_t* sorted_pairs,
                int32_t* pair_pos, int32_t* active, void* ws, size_t ws_bytes,
                void* stream);

/* ------------------------------------------------------------ expert FFN
 * For every active expert e (or only those with expert_mask[e] != 0) and
 * every pair p of e: y_pairs[p] = Wd_e (silu(Wg_e x_t) * (Wu_e x_t)),
 * t = p / k, with the expert's weights at pool_base + slot*slot_bytes,
 * slot = slot_table[e] (the expert-id -> slot indirection over one slot
 * pool, fork README "Known limits").  A slot of -1 (or outside the pool)
 * sets the device error word and fills that expert's y rows with NaN.
 * Experts masked out are skipped and their y rows left as they were. */
typedef struct moe_ffn_args {
  const void* pool_base;          /* device: slot pool */
  size_t slot_bytes;              /* bytes per slot (moe_slot_bytes) */
  int n_slots;                    /* slots in the pool; a slot outside
                                     [0, n_slots) counts as not resident */
  int qtype;                      /* MOE_QTYPE_* of every slot */
  int H, I;                       /* hidden, intermediate */
  int T, k, E;                    /* tokens, experts per token, experts */
  const int32_t* slot_table;      /* device [E]: slot of expert e or -1 */
  const void* x;                  /* device [T][H] in x_dtype */
  int x_dtype;                    /* MOE_DTYPE_F32 (decode) or _BF16 */
  const int32_t* expert_offsets;  /* device [E+1] from moe_permute */
  const int32_t* sorted_pairs;    /* device [T*k] from moe_permute */
  const int32_t* active;          /* device [E+1] from moe_permute */
  const int32_t* expert_mask;     /* device [E] or NULL (= all) */
  float* y_pairs;                 /* device fp32 [T*k][H], pair order */
  int mode;                       /* MOE_MODE_DECODE, _PREFILL or _DECODE_Q8A */
  void* ws;                       /* device workspace (256-B aligned) */
  size_t ws_bytes;
  const float* topk_w;            /* device [T][k]; with out: fused combine */
  float* out;                     /* device fp32 [T][H] or NULL: when set,
                                     the call also writes out as
                                     moe_combine would (needs no mask) */
} moe_ffn_args;

int moe_expert_ffn_workspace_size(const moe_ffn_args* args, size_t* bytes);
int moe_expert_ffn(moe_ctx* ctx, const moe_ffn_args* args, void* stream);

/* ---------------------------------------------------- decode layer, fused
 * One decode layer: the results of moe_route_permute (router logits, top-k,
 * grouping) followed by moe_expert_ffn with the combine (args.topk_w and
 * args.out set), in fewer launches.  For T*k <= 64 the top-k and the
 * grouping run inside the gate/up kernel, every workgroup selecting from the
 * logits it needs anyway (three launches with computed logits, two with
 * logits_in); larger batches run the two calls.  Arguments are those of the
 * two calls: args.x (fp32, args.mode = MOE_MODE_DECODE, no expert_mask) is
 * also the router input; router_w/bias/logits_in/logits_out/topk_ids as in
 * moe_route; args.topk_w, args.expert_offsets, args.sorted_pairs,
 * args.active and pair_pos receive the routing results (this call writes
 * through those args pointers, which moe_expert_ffn only reads); args.out
 * receives the layer output.  Errors as in the two calls. */
int moe_decode_layer(moe_ctx* ctx, const moe_ffn_args* args,
                     const float* router_w, const float* bias,
                     const float* logits_in, float* logits_out,
                     int32_t* topk_ids, int32_t* pair_pos, void* stream);

/* moe_decode_layer_static: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The same layer as moe_decode_layer, through the same
 * kernels and with the same results, but args.ws / args.ws_bytes are
 * ignored: the workspace is a static device array of the library,
 * moe_static_scratch_bytes() bytes (8 MiB) on each GPU it runs on, held
 * until the process ends.  The caller still passes every input and output.
 * The call allocates nothing (no hipMalloc, hipFree or allocating library
 * routine; with the context's kernel timing switched on the timer may
 * create events).  It needs T*k*I*4 bytes of workspace (the decode h rows);
 * more -> MOE_ERR_WORKSPACE, checked on the host before any launch.  Every
 * call on one GPU shares that GPU's array and leaves its contents as they
 * were, so calls that overlap on one GPU (on different streams, or from
 * different threads) race: order them on one stream.  Nothing in the array
 * needs to start at zero (every element read is first written by the same
 * call).  Errors otherwise as moe_decode_layer. */
size_t moe_static_scratch_bytes(void);
int moe_decode_layer_static(moe_ctx* ctx, const moe_ffn_args* args,
                            const float* router_w, const float* bias,
                            const float* logits_in, float* logits_out,
                            int32_t* topk_ids, int32_t* pair_pos,
                            void* stream);

/* --------------------------------------------------------------- combine
 * out[t][:] = sum over j ascending of topk_w[t][j] * y_pairs[t*k + j][:]
 * (device fp32; out [T][H]). */
int moe_combine(moe_ctx* ctx, const float* y_pairs, const float* topk_w,
                int T, int k, int H, float* out, void* stream);

/* ------------------------------------------------------------ dequantise
 * One packed matrix (device layout above, rows x cols) -> device `out`
 * [rows][cols] as fp32 (exact d*q) or bf16 (round to nearest even of that
 * fp32), through the same block decoding the FFN kernels use. */
int moe_dequantize(moe_ctx* ctx, int qtype, const void* packed, int rows,
                   int cols, int out_dtype, void* out, void* stream);

/* ---------------------------------------------------------- expert cache
 * A global LRU over (layer, expert) keys (fork README, "About": global LRU
 * expert caching; setup guide: a shared LRU follows token-level routing
 * locality) backed by a device slot pool, with the full pool in pinned host
 * memory.  Only missing experts move over PCIe ("FreeToken Inference
 * Engine: 3x Speed Boost for MoE Models", "RTX 5090 Benchmark").
 *   d_pool   device, (n_slots + 2) * slot_bytes, caller-owned.  At most
 *            n_slots keys are resident; free slots are reused oldest-first,
 *            so a copy lands in a slot released two evictions earlier
 *            (ping-pong staging) after that slot's last reader finished.
 *   h_pool   host pinned memory (hipHostMalloc / torch pin_memory),
 *            experts [L][E] in the device slot layout, caller-owned;
 *            memory that is not pinned -> MOE_ERR_NOT_PINNED.
 * The device slot table (int32 [L][E], -1 = absent) is owned by the cache;
 * cache_slot_table_device() returns it (row `layer` is the slot_table of
 * moe_expert_ffn).  The cache starts empty.
 *
 * cache_slot_table_lookup (host): applies n ids of one layer in order.  A
 * resident key is a hit and becomes most recently used.  A missing key is
 * inserted at once, evicting the least recently used key that was not
 * looked up earlier in this call; it gets a destination slot but its bytes
 * are not there yet: call prefetch_expert for every listed miss before the
 * FFN.  slots_out[i] = slot of ids[i]; miss_ids lists the misses in order
 * without repeats (may be NULL); *n_miss = their number.
 * MOE_ERR_CAPACITY if the call names more distinct experts than n_slots
 * (the cache is then unchanged).  Every lookup must be followed by
 * cache_mark_layer_done before the next lookup.
 *
 * prefetch_expert: for a key listed as a miss, copies its bytes from the
 * pinned pool into its slot with hipMemcpyAsync on copy_stream (after the
 * slot's previous reader, recorded by cache_mark_layer_done, has finished),
 * makes compute_stream wait for the copy, and writes the key's slot (and
 * -1 for the key it evicted) into the device table in compute_stream
 * order.  A key already resident returns its slot with no copy.
 * *slot_out (may be NULL) = the slot.
 *
 * cache_mark_layer_done: records on compute_stream the point after which the
 * slots of the last lookup are no longer read (enqueue it after the layer's
 * FFN), and ends that lookup.
 *
 * cache_slot_table_resize: changes the capacity to n_slots while the cache
 * is in use, with no restart ("FreeToken Inference Engine: 3x Speed Boost
 * for MoE Models", "Dynamic Cache Adjustment Experiments": the expert cache
 * is resized at run time).  The n_slots most recently used keys stay
 * resident; the others are evicted.  d_pool is the device pool to use from now on,
 * (n_slots + 2) * slot_bytes, caller-owned, 16-byte aligned; NULL or the
 * current pool resizes in place (the allocation must then hold
 * (n_slots + 2) slots: shrinking always fits).  Kept experts move on
 * device (slot_move_kernel on `stream`): into a new pool all of them, in
 * place only those whose slot is past the new end.  The call waits for the
 * device (every earlier reader of the pool and every expert copy) before the
 * moves and for `stream` after them, so on return the old pool is no longer
 * used and may be freed.  It allocates a small temporary device buffer for
 * the move list.  Between a lookup and its cache_mark_layer_done (or with
 * copies not yet issued by prefetch_expert) -> MOE_ERR_INVALID_ARG; the
 * cache is unchanged on any error.  Hit and miss counts carry over. */
int cache_slot_table_create(int L, int E, int n_slots, int qtype, int H, int I,
                            void* d_pool, const void* h_pool, moe_cache** out);
int cache_slot_table_lookup(moe_cache* c, int layer, const int32_t* ids,
                            int n, int32_t* slots_out, int32_t* miss_ids,
                            int* n_miss);
const int32_t* cache_slot_table_device(moe_cache* c);
int cache_slot_table_stats(moe_cache* c, int64_t* hits, int64_t* misses);
int cache_slot_table_destroy(moe_cache* c);
int prefetch_expert(moe_cache* c, int layer, int expert, void* copy_stream,
                    void* compute_stream, int32_t* slot_out);
int cache_mark_layer_done(moe_cache* c, int layer, void* compute_stream);
int cache_slot_table_resize(moe_cache* c, int n_slots, void* d_pool,
                            void* stream);

/* cache_decode_layer: one decode layer of `layer` through the cache, the
 * sequence above in one host call: moe_route_permute on compute_stream (x
 * fp32 [T][H] device; router_w/bias/logits_in/logits_out/topk_ids/topk_w/
 * expert_offsets/sorted_pairs/pair_pos/active as there), the routed ids
 * written by the routing kernel itself into coherent pinned staging owned
 * by the cache, followed by a flag word (the host waits for the flag, not
 * for the kernel's end, bounded by an event on the kernel: a layer's
 * misses are known only once it has routed), the LRU lookup,
 * then moe_expert_ffn on the resident experts while prefetch_expert copies
 * the misses on copy_stream, moe_expert_ffn on the misses once they land,
 * moe_combine into out (device fp32 [T][H]) and cache_mark_layer_done.
 * With no miss the FFN and the combine are one call.  y_pairs and ws as in
 * moe_expert_ffn.  T*k <= 1024.  The staging is allocated with the cache,
 * so the call allocates nothing.  Errors as in the calls it makes. */
int cache_decode_layer(moe_cache* c, moe_ctx* ctx, int layer, const float* x,
                       const float* router_w, const float* bias,
                       const float* logits_in, int T, int k,
                       float* logits_out, int32_t* topk_ids, float* topk_w,
                       int32_t* expert_offsets, int32_t* sorted_pairs,
                       int32_t* pair_pos, int32_t* active, float* y_pairs,
                       void* ws, size_t ws_bytes, float* out,
                       void* copy_stream, void* compute_stream);

/* ------------------------------------------------- prefill layer streaming
 * Dual buffering for long prompts ("FreeToken Inference Engine: 3x Speed
 * Boost for MoE Models", "Dual-Buffering to Solve the Prefill Bottleneck"):
 * a prompt touches nearly every expert of every layer, so every layer's
 * experts cross PCIe, and the next layer's copy overlaps the current
 * layer's compute.
 *   d_bufs   device, 2 * E * slot_bytes, caller-owned, 16-byte aligned: two
 *            buffers of one layer's E experts (expert e in slot e).
 *   h_pool   pinned host memory, experts [L][E] in the device slot layout
 *            (the expert cache's host pool layout), caller-owned; not
 *            pinned -> MOE_ERR_NOT_PINNED.
 * The stream object owns an identity slot table, four events and two HSA
 * signals.
 *
 * prefill_stream_layer: one layer's forward with its experts streamed.  If
 * no buffer holds `layer` it is copied now (a demand load, counted) into
 * the buffer the previous call did not use.  moe_route_permute then runs on
 * compute_stream (router_w/bias/logits_in/logits_out/topk_ids/pair_pos and
 * route_ws as there; its other outputs go to args.topk_w,
 * args.expert_offsets, args.sorted_pairs, args.active), compute_stream
 * waits for the layer's copy, and moe_expert_ffn with the combine runs out
 * of the buffer (args as in moe_expert_ffn with args.topk_w and args.out
 * set and no expert_mask; args.pool_base, slot_bytes, n_slots and
 * slot_table are ignored, and args.H, I, E and qtype must equal the
 * stream's).  Then layer + 1, if it exists and is not held, is copied into
 * the other buffer, after the last layer that read that buffer has
 * finished on its compute stream.  Calls in layer order keep PCIe busy back
 * to back; any order is correct.  Errors as in the calls it makes.
 * The copies are HSA asynchronous copies (DMA engines, completion signals
 * waited for on the host), which enter no HIP queue and so overlap the
 * compute whatever hardware queues HIP gives the streams; copy_stream is
 * then unused, and the call blocks the host until its layer's copy has
 * landed and until the previous call's layer has finished (before it
 * issues the next copy).  Such calls cannot be captured in a HIP graph.
 * Where the HSA runtime is unavailable, or MOE_STREAM_HIP_COPY is set to
 * a nonzero value when the stream is created, the copies are
 * hipMemcpyAsync calls on copy_stream ordered by events instead, and the
 * call does not block.  Either way d_bufs and h_pool must outlive
 * prefill_stream_destroy, which waits for every copy.
 *
 * prefill_stream_stats: layer copies issued in total and how many of them
 * were demand loads (not prefetched by the previous call). */
typedef struct moe_prefill_stream moe_prefill_stream;
int prefill_stream_create(int L, int E, int qtype, int H, int I, void* d_bufs,
                          const void* h_pool, moe_prefill_stream** out);
int prefill_stream_layer(moe_prefill_stream* s, moe_ctx* ctx, int layer,
                         const moe_ffn_args* args, const float* router_w,
                         const float* bias, const float* logits_in,
                         float* logits_out, int32_t* topk_ids,
                         int32_t* pair_pos, void* route_ws,
                         size_t route_ws_bytes, void* copy_stream,
                         void* compute_stream);
int prefill_stream_stats(moe_prefill_stream* s, int64_t* loads,
                         int64_t* demand_loads);
int prefill_stream_destroy(moe_prefill_stream* s);

/* ------------------------------------------------------ host executor
 * moe_host_expert_ffn: the expert FFN of n tokens computed on the host
 * cores, reading one expert where it already is, in pinned host memory
 * ("FreeToken Inference Engine: 3x Speed Boost for MoE Models", "Q*
 * Strategy: Intelligently Choosing Where to Compute": a missing expert is
 * either moved to the GPU or computed on the CPU).  slot: host, one expert
 * in the device slot layout (moe_pack_expert); x: host fp32 [n][H]; y: host
 * fp32 [n][H], written.  h = silu(Wg x) * (Wu x) and y = Wd h accumulate
 * in fp32.  threads: worker threads including the caller (0 = all
 * hardware threads but four, at least one); vector: 1 uses AVX-512 when
 * the CPU has it, 0 plain C++.  Errors: MOE_ERR_UNSUPPORTED_QTYPE,
 * MOE_ERR_INVALID_ARG.
 * moe_host_has_avx512: 1 when the AVX-512 path is available. */
int moe_host_expert_ffn(int qtype, int H, int I, const void* slot,
                        const float* x, int n, float* y, int threads,
                        int vector);
int moe_host_has_avx512(void);

/* ------------------------------------------- misses on the host (Q*)
 * On a miss FreeToken either moves the expert to the GPU or computes it on
 * the CPU, choosing per batch of missing experts from the measured PCIe
 * bandwidth and RAM speed ("FreeToken Inference Engine: 3x Speed Boost for
 * MoE Models", "Q* Strategy: Intelligently Choosing Where to Compute").
 *
 * cache_set_miss_policy: the policy of later cache_decode_layer calls
 * (MOE_MISS_*; default MOE_MISS_COPY) and the host threads of the host
 * executor, caller included (0 = all hardware threads but four, at
 * least one).  The first policy
 * other than MOE_MISS_COPY allocates the staging it needs (pinned and
 * device, kCtlStagePairs = 1024 rows of H floats each, and host scratch);
 * MOE_MISS_QSTAR first measures both rates (a few expert-sized copies and
 * host FFNs).  Calling it between layers is allowed.
 *
 * In cache_decode_layer, for each layer: the missing experts are found in
 * the order the router named them; MOE_MISS_HOST sends all to the host,
 * MOE_MISS_QSTAR sends the last m, where m minimises
 * max((n - m) B / r_copy, m B / r_host + 20 us) (n missing experts of B
 * bytes; r_copy and r_host running estimates of the copy and host
 * executor rates, updated every layer), the fewest on a tie.  A host
 * expert is not inserted into the cache (its lookup is a miss and changes
 * nothing); the layer's tokens are read back, the host computes its rows
 * while the GPU runs the resident and copied experts, and the rows are
 * copied back into y_pairs before the combine.
 *
 * MOE_MISS_HOST_COPY (not on the pages; it keeps the cache learning while
 * the host takes the misses): this layer computes every missing expert on
 * the host; the first ones (router order), up to 8 background copies in
 * flight, are also inserted and copied as with MOE_MISS_COPY, but with
 * nothing on compute_stream waiting for them: through the HSA runtime's
 * asynchronous copy with a completion signal the host polls (so no packet
 * on any stream's hardware queue waits for the copy), or on copy_stream if
 * that cannot be set up; the rest are left out of the cache as with
 * MOE_MISS_HOST.  A later hit on an expert whose copy has not completed
 * (checked on the host at lookup) is computed on the host as well.  Use
 * one copy_stream per cache.  Leaving this policy (for another) waits for
 * every background copy; until then use cache_decode_layer only.
 *
 * cache_miss_stats: experts copied and computed on the host so far, and
 * the current rate estimates (GB/s; 0 before any measurement).
 * cache_last_misses: the experts the last cache_decode_layer copied and
 * computed on the host (arrays of at least E entries, may be NULL); the
 * first *n_host_only (may be NULL) host experts were misses left out of
 * the cache, the others (MOE_MISS_HOST_COPY) were also copied or are
 * resident with their copy still in flight. */
int cache_set_miss_policy(moe_cache* c, int policy, int host_threads);
int cache_miss_stats(moe_cache* c, int64_t* copied, int64_t* host,
                     double* pcie_gbs, double* host_gbs);
int cache_last_misses(moe_cache* c, int32_t* copy_ids, int* n_copy,
                      int32_t* host_ids, int* n_host, int* n_host_only);

/* ------------------------------------------------------- bank type check
 * One block type for every expert bank: the slot pool is one allocation
 * indexed with a single row stride, so mixed types would read every block
 * at the wrong offset and must be refused, naming the layers (fork README,
 * "Known limits").  qtypes: host int [L][n_per_layer] (e.g. gate, up, down
 * per layer).  On success *out_qtype is the common type; otherwise
 * MOE_ERR_MIXED_QTYPE (message lists the layers that differ from layer 0)
 * or MOE_ERR_UNSUPPORTED_QTYPE. */
int moe_check_bank_types(int L, int n_per_layer, const int* qtypes,
                         int* out_qtype);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
