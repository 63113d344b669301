/*
 * moe.h -- C ABI of the MI355X (gfx950) quantized Mixture-of-Experts FFN block.
 *
 * The block (one MoE layer of a Gemma-4-26B-A4B-style model, as the
 * TurboFieldfare pages describe it):
 *   - an 8-bit affine router projects each activation row to n_experts logits
 *     (router kept at 8 bits: ai-heartland review "TurboFieldfareとは",
 *     system-design summary; rebasdaily article, MLX affine 4-bit paragraph);
 *   - the top_k experts per row are picked (8 of 128: blog-mushroom article
 *     "TurboFieldfare: Gemma 4 26B on an 8 GB MacBook", section "Why 26B Fits
 *     in 2 GB") and weighted by a softmax over the picked logits;
 *   - each picked expert is a GeGLU FFN over MLX affine 4-bit weights (group
 *     64 along the input dimension, bf16 scale and bias per group; same
 *     passages);
 *   - an always-on shared expert runs beside them and the two paths merge
 *     (blog-mushroom article, "Why 26B Fits in 2 GB", per-token flow);
 *   - prefill runs in chunks of rows so that one fetched expert serves every
 *     row of the chunk routed to it (same section; paperfeed digest
 *     "drumih/turbo-fieldfare", "How it works").
 *
 * Conventions for every entry point:
 *   - Device pointers point to HIP device memory (allocated by the caller,
 *     e.g. through PyTorch). Host pointers are named *_host.
 *   - `stream` is a hipStream_t passed as void*. Work is enqueued on it;
 *     nothing is synchronised unless stated. Pointers must stay valid until
 *     the stream has reached the enqueued work.
 *   - The library allocates no device memory. Scratch space comes from the
 *     caller's workspace `ws` of `ws_bytes` bytes (>= moe_workspace_bytes()).
 *     The workspace must be zero-filled once before its first use
 *     (moe_workspace_init). Every call leaves it ready for the next one: the
 *     arrival counters are back at zero, and the whole-block decode keeps a
 *     call counter (epoch) there that tags its hand-off words, so the
 *     workspace must not be overwritten between calls.
 *     Calls that overlap in time need separate workspaces.
 *   - Arguments are validated before anything is enqueued; a failing check
 *     returns a negative moe_status and launches nothing. No C++ exception
 *     crosses this interface.
 *   - A slot-table entry that names a blob outside the pool is not followed:
 *     the kernel records MOE_DEVERR_BAD_SLOT in the library's device error
 *     word and treats that expert's output as zero; moe_check_device_error()
 *     reports it.
 */
#ifndef QMOE_MOE_H_
#define QMOE_MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,       /* null pointer, bad enum, rows < 0, misaligned pointer */
  MOE_ERR_UNSUPPORTED_SHAPE = -2, /* a dimension not a multiple of 64, top_k out of range, ... */
  MOE_ERR_WORKSPACE = -3,         /* ws_bytes < moe_workspace_bytes(...) */
  MOE_ERR_HIP = -4,               /* a HIP runtime call failed (launch, copy, sync) */
  MOE_ERR_DEVICE_CHECK = -5       /* a kernel recorded an error in the device error word */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* device error word values (bit flags) */
#define MOE_DEVERR_BAD_SLOT 1u      /* a slot-table entry named a blob outside the pool */
#define MOE_DEVERR_BAD_EXPERT_ID 2u /* an expert id outside [0, n_experts) (e.g. NaN logits) */
#define MOE_DEVERR_SYNC_TIMEOUT 4u  /* a fused-decode wait gave up; re-initialise the workspace */

/* Slot-table entry that leaves an expert out of a prefill call on purpose (see
 * moe_expert_ffn_prefill_chunk): no flag, its outputs are not written. */
#define MOE_SLOT_SKIP 0xFFFFFFFFu

/* Shape of one MoE layer. d_model, d_ff, d_ff_shared: multiples of 64, d_model and
 * d_ff_shared at most 6144; n_experts: 64, 128 or 256; 1 <= top_k <= min(n_experts, 16);
 * group must be 64; rows * top_k < 65536 per call. Anything else returns
 * MOE_ERR_UNSUPPORTED_SHAPE. Gemma-4-26B-A4B-like: {2816, 704, 2112, 128, 8, 64}. */
typedef struct {
  int32_t d_model, d_ff, d_ff_shared, n_experts, top_k, group;
} moe_shape;

/*
 * One layer's weights, all device memory owned by the caller.
 *   pool        base of the HBM-resident packed-expert pool: n_blobs blobs of
 *               blob_stride bytes each (blob_stride >= moe_expert_blob_bytes(),
 *               multiple of 256). The pages keep 128 fixed-size page-aligned
 *               expert blobs per layer file and bind sub-regions of them
 *               (blog-mushroom article, model-file-layout section); here the
 *               pool holds the blobs of every layer in HBM.
 *   slot_table  [n_experts] uint32: expert id -> blob index in the pool (the
 *               per-layer slot table the kernels read; any placement gives the
 *               same results).
 *   router_blob packed 8-bit router [n_experts x d_model] (moe_pack_matrix8).
 *   shared_blob packed shared expert: gate [d_ff_shared x d_model], up (same),
 *               down [d_model x d_ff_shared], each moe_pack_matrix4, back to back.
 * An expert blob is gate [d_ff x d_model] | up [d_ff x d_model] |
 * down [d_model x d_ff], each packed with moe_pack_matrix4, back to back.
 */
typedef struct {
  const uint8_t* pool;
  uint64_t blob_stride;
  uint64_t n_blobs;
  const uint32_t* slot_table;
  const uint8_t* router_blob;
  const uint8_t* shared_blob;
} moe_layer;

/* ------------------------------------------------------------------ sizes */

/* Bytes of workspace any entry point below needs for `rows` activation rows. */
size_t moe_workspace_bytes(const moe_shape* shape, int32_t rows);

/* Zero-fills a workspace (a hipMemsetAsync enqueued on `stream`). Required once per
 * workspace, before its first use. Call it outside HIP graph capture: a replayed
 * memset node would also reset the fused decode's call counter while stale
 * hand-off words keep their tags. */
moe_status moe_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Packed sizes (bytes) of a 4-bit / 8-bit matrix [rows x cols], of one routed
 * expert blob (before stride padding), of the shared-expert blob and of the
 * router blob. 0 if the shape is unsupported. */
uint64_t moe_matrix4_bytes(int32_t rows, int32_t cols);
uint64_t moe_matrix8_bytes(int32_t rows, int32_t cols);
uint64_t moe_expert_blob_bytes(const moe_shape* shape);
uint64_t moe_shared_blob_bytes(const moe_shape* shape);
uint64_t moe_router_blob_bytes(const moe_shape* shape);

/* ------------------------------------------------------------------ packer (host, CPU only) */

/*
 * Canonical (MLX-style) format of a quantized matrix W[rows x cols], w = s*q + b:
 *   q_host  4-bit: uint8 [rows][cols/2], element 2j in the low nibble of byte j;
 *           8-bit: uint8 [rows][cols]
 *   s_host, b_host  uint16 bf16 bit patterns [rows][cols/64]
 * Device format written to out_host (moe_matrix{4,8}_bytes bytes): tiles of
 * 64 rows x 64 columns, row-block major then group; each 4-bit tile holds the
 * codes (2048 B, laid out so that lane r of a wavefront reads row r with
 * 16-byte loads and one 32-bit word yields four bf16 pairs) followed by the
 * 64 (s, b) pairs (256 B). rows and cols must be multiples of 64.
 * The unpackers invert the packers bit-exactly.
 */
moe_status moe_pack_matrix4(const uint8_t* q_host, const uint16_t* s_host, const uint16_t* b_host, int32_t rows,
                            int32_t cols, uint8_t* out_host);
moe_status moe_pack_matrix8(const uint8_t* q_host, const uint16_t* s_host, const uint16_t* b_host, int32_t rows,
                            int32_t cols, uint8_t* out_host);
moe_status moe_unpack_matrix4(const uint8_t* in_host, int32_t rows, int32_t cols, uint8_t* q_host, uint16_t* s_host,
                              uint16_t* b_host);
moe_status moe_unpack_matrix8(const uint8_t* in_host, int32_t rows, int32_t cols, uint8_t* q_host, uint16_t* s_host,
                              uint16_t* b_host);

/* ------------------------------------------------------------------ the block's steps */

/*
 * Router + top-k + softmax for `rows` rows of x ([rows][d_model], dtype MOE_F32
 * or MOE_BF16, 16-byte aligned). Defining passages: the router scores every
 * expert and the top 8 of 128 run per token and layer (blog-mushroom article
 * "TurboFieldfare: Gemma 4 26B on an 8 GB MacBook", section "Why 26B Fits in
 * 2 GB"); the router weights stay 8-bit affine while the experts are 4-bit
 * (rebasdaily article, section "不是把模型塞小，而是边用边取"; ai-heartland review,
 * section "TurboFieldfareとは", quantisation summary). The pages give no pick
 * weighting; the softmax over the picked logits is the reading taken here.
 *   logit[r][e] = sum_i (s*q + b)[e][i] * x[r][i] + logit_offset[e]
 * accumulated in fp64 (every product exact), so the top-k set is decided on
 * logits within ~1e-12 of exact. Picks ordered by (logit desc, expert id asc).
 *   topk_idx [rows][top_k] int32, topk_w [rows][top_k] float (softmax of the
 *   picked logits), logits [rows][n_experts] double (optional, may be NULL),
 *   logit_offset [n_experts] float (optional, NULL = 0).
 */
moe_status moe_router_topk(const moe_shape* shape, const moe_layer* layer, const void* x, moe_dtype x_dtype,
                           int32_t rows, const float* logit_offset, int32_t* topk_idx, float* topk_w,
                           double* logits, void* ws, size_t ws_bytes, void* stream);

/*
 * Token-to-expert grouping (prefill): the rows*top_k (row, slot) pairs, pair
 * id = row*top_k + slot, stably sorted by expert id (a counting sort). It serves
 * the pages' chunked prefill, where one fetched expert serves every row of the
 * chunk routed to it (blog-mushroom article, section "Why 26B Fits in 2 GB",
 * prefill paragraph; paperfeed digest "drumih/turbo-fieldfare", "How it works"):
 *   count [n_experts], offset [n_experts+1] (exclusive prefix sum of count),
 *   perm [rows*top_k] (pair id at each sorted position),
 *   inv_perm [rows*top_k] (sorted position of each pair). Bit-exact.
 * An id outside [0, n_experts) is recorded as MOE_DEVERR_BAD_EXPERT_ID and its
 * pair is left out: count/offset/perm cover the other pairs (perm entries from
 * offset[n_experts] on are not written) and its inv_perm is -1.
 */
moe_status moe_group_by_expert(const moe_shape* shape, const int32_t* topk_idx, int32_t rows, int32_t* count,
                               int32_t* offset, int32_t* perm, int32_t* inv_perm, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * Routed experts for ONE decode row x [d_model]: for each slot j < top_k,
 *   expert_out[j][:] = W_down (gelu_tanh(W_gate x) * (W_up x)) of expert topk_idx[j]
 * (unweighted), fp32 [top_k][d_model]. 4-bit dequant is fused into the GEMVs.
 * Defining passages: each selected expert's blob runs on the GPU per token
 * (blog-mushroom article, section "Why 26B Fits in 2 GB", per-token flow); the
 * experts are MLX affine 4-bit with group 64 and bf16 scale and bias (ai-heartland
 * review, section "TurboFieldfareとは", quantisation summary). The pages name no
 * activation; GeGLU with tanh-GELU on the gate is the reading taken here.
 * topk_idx is device memory [top_k]; ids outside [0, n_experts) or slot entries
 * outside the pool set the device error word and give zero outputs. A slot whose
 * expert's table entry is MOE_SLOT_SKIP is left out without a flag: its row of
 * expert_out keeps its contents. Decode through an expert cache runs this call twice
 * on disjoint slots: the picks already resident while the misses are copied in, then
 * the misses (see moe_shared_expert_decode).
 */
moe_status moe_expert_ffn_decode(const moe_shape* shape, const moe_layer* layer, const void* x, moe_dtype x_dtype,
                                 const int32_t* topk_idx, float* expert_out, void* ws, size_t ws_bytes,
                                 void* stream);

/*
 * Routed experts for a prefill chunk of `rows` rows, grouped by expert
 * (offset, perm from moe_group_by_expert): for sorted position j with pair
 * id p = perm[j], row r = p / top_k, expert e = the expert whose range holds j,
 *   expert_out[j][:] = E_e(x[r]) (unweighted), fp32 [rows*top_k][d_model].
 * Defining passages: prefill runs in chunks of up to 128 rows (256 optional) so
 * that one fetched expert serves every row routed to it (blog-mushroom article,
 * section "Why 26B Fits in 2 GB"; paperfeed digest "drumih/turbo-fieldfare",
 * "How it works"; ai-heartland review, section "OpenAI互換サーバーと、速度に効くつまみ").
 * Every expert's weights are read once per 64-row tile of its rows; the 4-bit
 * codes enter the matrix cores exactly and the group scale and bias are applied
 * per group in fp32 afterwards. An expert whose slot-table entry is
 * MOE_SLOT_SKIP is left out without a flag: the rows of its pairs in expert_out
 * keep their contents. Prefill through an expert cache smaller than a chunk's
 * experts runs this call once per group of resident experts, each pass with a
 * table that names that group and skips the rest (the passes write disjoint rows);
 * the router, the grouping and moe_combine run once.
 */
moe_status moe_expert_ffn_prefill_chunk(const moe_shape* shape, const moe_layer* layer, const void* x,
                                        moe_dtype x_dtype, int32_t rows, const int32_t* offset,
                                        const int32_t* perm, float* expert_out, void* ws, size_t ws_bytes,
                                        void* stream);

/*
 * Shared expert + weighted combine. Defining passage: an always-on shared expert
 * runs beside the routed experts and the two paths merge (blog-mushroom article,
 * section "Why 26B Fits in 2 GB", per-token flow); the shared expert is one of the
 * resident weights (same section). The shared expert's weight is 1 and the
 * routed outputs are weighted by topk_w (the reading taken here):
 *   y[r][:] = S(x[r]) + sum_{j<top_k} topk_w[r][j] * E_j
 * where E_j = expert_out[inv_perm[r*top_k + j]] (prefill, inv_perm != NULL) or
 * expert_out[r*top_k + j] (inv_perm == NULL; decode has rows == 1), summed in
 * slot order. y fp32 [rows][d_model]. If residual_bf16 is not NULL it is a
 * bf16 [rows][d_model] in/out buffer: residual = bf16_rne(fp32(residual) + y)
 * (the residual add between stacked layers). It may be the buffer x itself
 * (bf16 x): every read of x precedes the residual store, here and in the
 * fused layer calls below. expert_out and y must be 16-byte aligned and
 * residual_bf16 8-byte aligned (MOE_ERR_INVALID_ARG otherwise; rows of
 * d_model elements keep every row aligned).
 */
moe_status moe_combine(const moe_shape* shape, const moe_layer* layer, const void* x, moe_dtype x_dtype,
                       int32_t rows, const float* expert_out, const int32_t* inv_perm, const float* topk_w,
                       float* y, uint16_t* residual_bf16, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_combine for ONE decode row (inv_perm NULL) in two calls, so that other work can
 * run between the shared expert and the combine. The pages run the shared-expert
 * branch while the reads of the routed experts that missed the cache complete
 * (blog-mushroom article, section "Why 26B Fits in 2 GB", per-token flow): here
 * moe_shared_expert_decode goes first on the compute stream, the copies of the misses
 * on another, and moe_combine_decode after the routed experts.
 *   moe_shared_expert_decode: the shared expert of x (bf16 or fp32 [d_model]) into the
 *     workspace; nothing else is written.
 *   moe_combine_decode: y [d_model] = S(x) + sum_j topk_w[j] * expert_out[j] and the
 *     residual store, as moe_combine; expert_out [top_k][d_model] unweighted.
 * The pair gives y and residual bit-identical to moe_combine on the same inputs, if no
 * call between them on the same workspace runs a shared expert or a whole-layer call
 * (the routed-expert calls do not touch the shared expert's part of the workspace).
 * Errors: as moe_combine; moe_combine_decode takes no layer and no x.
 */
moe_status moe_shared_expert_decode(const moe_shape* shape, const moe_layer* layer, const void* x,
                                    moe_dtype x_dtype, void* ws, size_t ws_bytes, void* stream);
moe_status moe_combine_decode(const moe_shape* shape, const float* expert_out, const float* topk_w, float* y,
                              uint16_t* residual_bf16, void* ws, size_t ws_bytes, void* stream);

/*
 * Whole block for one decode row, fused: router + top-k + routed experts +
 * shared expert + combine (+ optional residual), the same results as the four
 * calls above (the per-token flow of the blog-mushroom article, section "Why 26B
 * Fits in 2 GB": router, picks, shared expert while the picked experts arrive,
 * merge). topk_idx/topk_w [top_k], y [d_model]; expert_out [top_k][d_model]
 * receives the unweighted routed outputs. Runs as one launch when the grid fits
 * the device at once (the workspace's call counter tags the hand-off words, so the
 * workspace must not be written between calls), else as three launches.
 */
moe_status moe_layer_decode(const moe_shape* shape, const moe_layer* layer, const void* x, moe_dtype x_dtype,
                            const float* logit_offset, int32_t* topk_idx, float* topk_w, float* expert_out,
                            float* y, uint16_t* residual_bf16, void* ws, size_t ws_bytes, void* stream);

/*
 * One decode row through n_layers stacked blocks (layers[l]: host array of each layer's
 * weights, every layer of the same shape), with the residual add between them:
 *   x_{l+1} = bf16_rne(fp32(x_l) + y_l),  y_l = the block of layer l on x_l.
 * x is bf16 [d_model], in: x_0, out: x_{n_layers}. The pages run the 30 MoE layers of
 * a token one after another (blog-mushroom article "TurboFieldfare: Gemma 4 26B on an
 * 8 GB MacBook", section "Why 26B Fits in 2 GB"); their decode step spends a third of
 * its time waiting between command buffers (same article, decode-step breakdown table
 * in section 实测数据). Here the whole stack is one launch when the shape fits the
 * whole-block decode kernel and n_layers <= 32: each workgroup keeps its item from layer
 * to layer and streams the next layer's routing-independent weights while the previous
 * layer finishes; otherwise the layers run one call each. Same results as n_layers calls
 * of moe_layer_decode with residual_bf16 = x.
 *   logit_offsets  host array [n_layers] of device [n_experts] offsets, or NULL (none)
 *   topk_idx, topk_w  [n_layers][top_k];  expert_out [n_layers][top_k][d_model],
 *   y [n_layers][d_model] fp32 and x_layers [n_layers][d_model] bf16 (each layer's input)
 *   may be NULL. The workspace is moe_workspace_bytes(shape, 1), as for moe_layer_decode
 *   (and shares its call counter).
 * Errors: those of moe_layer_decode for x and every layer; MOE_ERR_INVALID_ARG for
 * layers NULL, n_layers < 0, topk_idx or topk_w NULL, or a non-NULL expert_out, y or
 * x_layers not 16-byte aligned. n_layers = 0 returns MOE_OK and launches nothing.
 */
moe_status moe_stack_decode(const moe_shape* shape, const moe_layer* layers, int32_t n_layers, uint16_t* x,
                            const float* const* logit_offsets, int32_t* topk_idx, float* topk_w, float* expert_out,
                            float* y, uint16_t* x_layers, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_layer_decode for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc. It takes no
 * workspace: its scratch is a static device array of the library (5 MiB per GPU the
 * library runs on, held until the process ends), found once per device with
 * hipGetSymbolAddress. It calls no hipMalloc, hipFree or allocating routine. Same
 * arguments and results as moe_layer_decode without ws/ws_bytes; the caller still
 * owns every input and output.
 *   - Shapes past the scratch's maximum (d_model 3072, d_ff 768, d_ff_shared 2560,
 *     n_experts 256, top_k 16) return MOE_ERR_WORKSPACE and launch nothing.
 *   - Every call on one GPU shares that GPU's scratch and finds it as the previous
 *     call left it: calls that overlap in time on one GPU (several streams or host
 *     threads at once) race and give wrong results. Calls in stream order are safe,
 *     for any mix of shapes.
 *   - The first call on a device enqueues a clear of the scratch (a fill kernel) on
 *     `stream` before its work; a call captured into a HIP graph before any
 *     uncaptured call has cleared it captures the clear too, so each replay starts
 *     clean. After moe_check_device_error reports MOE_DEVERR_SYNC_TIMEOUT, the next
 *     call clears it again.
 */
moe_status moe_layer_decode_noalloc(const moe_shape* shape, const moe_layer* layer, const void* x, moe_dtype x_dtype,
                                    const float* logit_offset, int32_t* topk_idx, float* topk_w, float* expert_out,
                                    float* y, uint16_t* residual_bf16, void* stream);

/*
 * Whole block for a prefill chunk: router + top-k, grouping, grouped expert
 * GEMMs, shared expert and combine (+ optional residual), the pages' chunked
 * prefill (blog-mushroom article, section "Why 26B Fits in 2 GB"; paperfeed digest
 * "drumih/turbo-fieldfare", "How it works"). Outputs as the separate calls (with
 * the alignment moe_combine asks for); count/offset/perm/inv_perm as
 * moe_group_by_expert.
 */
moe_status moe_layer_prefill(const moe_shape* shape, const moe_layer* layer, const void* x, moe_dtype x_dtype,
                             int32_t rows, const float* logit_offset, int32_t* topk_idx, float* topk_w,
                             int32_t* count, int32_t* offset, int32_t* perm, int32_t* inv_perm,
                             float* expert_out, float* y, uint16_t* residual_bf16, void* ws, size_t ws_bytes,
                             void* stream);

/* ------------------------------------------------------------------ tiered expert residency */

/*
 * An HBM cache of expert blobs in front of a slower tier, per layer (the pages'
 * per-layer 16-slot LFU cache with misses read in on demand: blog-mushroom
 * article "TurboFieldfare: Gemma 4 26B on an 8 GB MacBook", section "Why 26B
 * Fits in 2 GB", per-token flow; paperfeed digest "drumih/turbo-fieldfare",
 * "How it works"). The slow tier is pinned host memory.
 *
 * Memory, all owned by the caller:
 *   host_pool     pinned host memory (e.g. hipHostMalloc, torch pin_memory):
 *                 n_layers * n_experts blobs of blob_stride bytes, layer-major;
 *                 blob (l, e) at host_pool + (l * n_experts + e) * blob_stride.
 *   device_slots  device memory, n_layers * slots blobs: layer l's slots start at
 *                 device_slots + l * slots * blob_stride.
 *   slot_tables   device [n_layers][n_experts] uint32, kept up to date by the
 *                 cache: the slot of each resident expert, `slots` for the others.
 * Layer l then runs through a moe_layer with pool = its slots, n_blobs = slots and
 * slot_table = slot_tables + l * n_experts, once its picks are resident.
 *
 * With device_slots and slot_tables both NULL the cache tracks the policy alone
 * (no HIP calls; host_pool and blob_stride are ignored), for tests of the policy.
 * moe_cache_create synchronises the device (it writes the initial tables); the
 * cache's host state is allocated with new and pinned memory: it is the only
 * allocation the library makes, and moe_cache_destroy frees it.
 */
typedef struct moe_expert_cache moe_expert_cache;

moe_status moe_cache_create(int32_t n_layers, int32_t n_experts, int32_t slots, uint64_t blob_stride,
                            const uint8_t* host_pool, uint8_t* device_slots, uint32_t* slot_tables,
                            moe_expert_cache** cache);

/*
 * Makes the experts idx_host[0..n) of `layer` resident (n <= slots; ids in range).
 * Every request counts once toward its expert's frequency. A hit reuses the slot;
 * a miss takes a never-used slot, else the slot of the resident expert with the
 * smallest (frequency, last use, id) that this request does not name, and enqueues
 * on `stream` the host-to-device copy of the blob and then of the layer's updated
 * slot table. Kernels enqueued on the same stream afterwards see the experts in
 * place; work enqueued earlier on it that used an evicted slot has run first.
 * slot_host (nullable) [n] receives each request's slot, n_misses (nullable) the
 * number of misses of this call. Host-side bookkeeping happens before return.
 */
moe_status moe_cache_acquire(moe_expert_cache* cache, int32_t layer, const int32_t* idx_host, int32_t n,
                             int32_t* slot_host, int32_t* n_misses, void* stream);

/*
 * One decode row of `layer` through the cache, on `stream` (the pages' per-token flow:
 * blog-mushroom article, section "Why 26B Fits in 2 GB"): the router; its picks read
 * back to the host (the call waits for `stream` there); the cache makes them resident
 * (moe_cache_acquire); the routed experts, the shared expert and the combine, with
 * y and the residual store as moe_combine gives them on a resident pool. With
 * copy_stream non-NULL the misses are copied on copy_stream, which first waits for the
 * work already on `stream`, while `stream` runs the shared expert
 * (moe_shared_expert_decode) and the picks that hit (moe_expert_ffn_decode over a table
 * that skips the misses); `stream` then waits for the copies, runs the misses and the
 * combine (moe_combine_decode). With copy_stream NULL, or when every pick is resident,
 * the copies (if any) go first on `stream`, then moe_expert_ffn_decode and moe_combine.
 *   router_blob, shared_blob  the layer's resident router and shared-expert blobs
 *   x, x_dtype, logit_offset, topk_idx, topk_w, expert_out, y, residual_bf16  as
 *                 moe_layer_decode (the routed experts come from the cache's slots)
 *   pass_tables   device [2][n_experts] uint32 the call writes (NULL allowed without
 *                 copy_stream); ws: moe_workspace_bytes(shape, 1)
 * Errors: MOE_ERR_INVALID_ARG for a policy-only cache, a layer out of range, a shape
 * whose n_experts differs from the cache's, top_k above the slots, blobs larger than
 * the cache's stride, or copy_stream without pass_tables; the errors of the calls it
 * makes (it stops at the first).
 */
moe_status moe_cache_decode(moe_expert_cache* cache, int32_t layer, const moe_shape* shape,
                            const uint8_t* router_blob, const uint8_t* shared_blob, const void* x, moe_dtype x_dtype,
                            const float* logit_offset, int32_t* topk_idx, float* topk_w, float* expert_out,
                            float* y, uint16_t* residual_bf16, uint32_t* pass_tables, void* ws, size_t ws_bytes,
                            void* stream, void* copy_stream);

/*
 * The same cache with its policy on the device: moe_cache_decode then applies the
 * policy to the router's picks in a one-thread kernel and copies the misses with a
 * kernel that reads the host tier through its device mapping, all in stream order on
 * `stream`, so a decode row never waits for the host and can be captured in a graph.
 * The policy is the one above, with a request counter per layer (the order it gives
 * within a layer is the same).
 *   device_state  device memory of moe_cache_device_state_bytes(...) bytes (256-byte
 *                 aligned), owned by the caller; it holds the frequencies, the slots'
 *                 experts and last uses, the counters and the last request's misses
 *   host_pool     pinned host memory that is mapped on the device (hipHostMalloc,
 *                 torch pin_memory); MOE_ERR_INVALID_ARG if it is not
 * Creation initialises the state and the slot tables on `stream` and waits for it.
 * moe_cache_decode ignores copy_stream and pass_tables on such a cache;
 * moe_cache_acquire and moe_cache_lookup return MOE_ERR_INVALID_ARG (the policy is not
 * on the host); moe_cache_stats synchronises the device and reads the counters. Decode
 * rows of one cache must be enqueued on one stream (the requests are applied in stream
 * order). moe_cache_device_state_bytes returns 0 for invalid sizes.
 */
uint64_t moe_cache_device_state_bytes(int32_t n_layers, int32_t n_experts, int32_t slots);
moe_status moe_cache_create_device(int32_t n_layers, int32_t n_experts, int32_t slots, uint64_t blob_stride,
                                   const uint8_t* host_pool, uint8_t* device_slots, uint32_t* slot_tables,
                                   void* device_state, uint64_t state_bytes, void* stream,
                                   moe_expert_cache** cache);

/* The slot of each expert idx_host[0..n) of `layer` as the cache stands (-1: not
 * resident), without counting a request or changing anything; host-side only. A
 * following moe_cache_acquire naming these experts keeps every resident one in its
 * slot, so this tells the caller which picks hit before their misses are copied. */
moe_status moe_cache_lookup(const moe_expert_cache* cache, int32_t layer, const int32_t* idx_host, int32_t n,
                            int32_t* slot_host);

/* Totals since creation: requests that hit, requests that missed, bytes copied. */
moe_status moe_cache_stats(const moe_expert_cache* cache, uint64_t* hits, uint64_t* misses, uint64_t* bytes_copied);

/* Waits for the cache's own pending copies, then frees its host state. */
moe_status moe_cache_destroy(moe_expert_cache* cache);

/* ------------------------------------------------------------------ errors */

const char* moe_status_string(moe_status status);

/* Synchronises `stream`, reads and clears the device error word of the
 * current device. Returns MOE_OK, or MOE_ERR_DEVICE_CHECK with the flags in
 * *flags (may be NULL). */
moe_status moe_check_device_error(void* stream, uint32_t* flags);

#ifdef __cplusplus
}
#endif

#endif /* QMOE_MOE_H_ */
