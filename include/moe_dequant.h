/*
 * moe_dequant.h -- C ABI of a gfx950 (MI355X) library for the per-token Mixture-of-Experts
 * expert computation over affine group-quantised weights.
 *
 * What it computes (per token, per layer):
 *   n      = RMSNorm(x) if the layer has a norm weight, else x
 *   logits = W_r n (+ logit_bias);  p = softmax(logits) over all E experts
 *   idx    = the K largest logits (descending; equal logits -> lower index first)
 *   w_k    = p[idx_k] / sum_j p[idx_j]
 *   y_k    = W_down[idx_k] (silu(W_gate[idx_k] n) * (W_up[idx_k] n)),  silu(z) = z/(1+e^-z)
 *   out    = sum_k w_k y_k (+ x with MOE_FLAG_RESIDUAL)
 * with every expert weight stored as codes q (2 or 4 bits) and one bf16 (scale, bias)
 * pair per group of 64 inputs, w = q * scale + bias.
 *
 * Sources.  The Flash-MoE web pages define the affine dequantisation (nibble*scale+bias)
 * and its FMA rewrite fma(nibble, scale*x, bias*x), the 4-bit and 2-bit expert matvec
 * kernels, the two-pass RMSNorm and the MoE combine as a weighted sum of expert outputs
 * (lilting.ch, "397Bパラメータモデルを48GB MacBookで動かすFlash-MoE", section "Metal
 * Compute Shaders", kernel table and the paragraph after it); 512 experts per layer with
 * 4 active per token (same page, model-architecture section); about 6.75 MB per 4-bit
 * expert and 27 MB per token (same page, SSD expert streaming section); the tiered
 * hot-4-bit / cold-2-bit expert store (nzkcom.pages.dev, "flash-moe-romance-vs-utility",
 * adopted-optimisations table).  The pages leave the router normalisation, top-K rule,
 * SwiGLU form, RMSNorm epsilon placement, group size, code order and scale dtype open;
 * this library takes the plain readings written above and in the format section below.
 *
 * Conventions (all entry points):
 *   - Every device buffer is allocated, owned and freed by the caller; the library never
 *     allocates device memory and never synchronises a compute stream.  Its state: a
 *     thread-local error message; per device, one side stream and two events that the first
 *     batched moe_expert_ffn call creates (kept until the process ends); and the host objects
 *     of the expert cache, which the caller creates and destroys.  moe_check_experts, a host
 *     check, copies the table synchronously.
 *   - Compute calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  They validate every argument the host can see first; on any failure they
 *     return a non-zero moe_status and enqueue nothing.  Device faults surface at the
 *     caller's next synchronisation.
 *   - "device" pointers must point to memory of the current HIP device; "host" pointers
 *     to ordinary host memory.
 *   - Supported shapes: hidden H and intermediate I are multiples of 64 with
 *     64 <= H <= 8192 and 64 <= I <= 8192; 1 <= E <= 2048; 1 <= K <= min(E, 8); and the
 *     down projection's staged activations must fit in LDS: K * I <= 36864.
 */
#ifndef MOE_DEQUANT_H
#define MOE_DEQUANT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_GROUP 64        /* quantisation group length along the input dimension */
#define MOE_MAX_TOPK 8
#define MOE_MAX_EXPERTS 2048
#define MOE_MAX_DIM 8192
#define MOE_MAX_K_TIMES_I 36864
#define MOE_BLOB_ALIGN 256  /* required alignment of expert blobs and plane offsets */

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL */
    MOE_ERR_SHAPE = 2,       /* a dimension or count is outside the supported range */
    MOE_ERR_DTYPE = 3,       /* unknown moe_dtype */
    MOE_ERR_BITS = 4,        /* bits not in {2, 4} */
    MOE_ERR_ALIGN = 5,       /* a pointer lacks the documented alignment */
    MOE_ERR_WORKSPACE = 6,   /* workspace NULL or smaller than moe_workspace_bytes() */
    MOE_ERR_LAUNCH = 7,      /* the HIP runtime refused a kernel launch */
    MOE_ERR_UNSUPPORTED = 8, /* valid request this build does not implement */
    MOE_ERR_BUFFER = 9,      /* an output buffer is too small */
    MOE_ERR_DEVICE = 10      /* no usable gfx950 device / HIP runtime error */
} moe_status;

typedef enum moe_dtype {
    MOE_F32 = 0,   /* IEEE binary32 */
    MOE_BF16 = 1   /* bfloat16 bits, uint16 little-endian */
} moe_dtype;

/* ------------------------------------------------------------------------------------
 * Packed format.
 *
 * Matrix with R rows (outputs) and C columns (inputs), C a multiple of 64, bits b:
 *   code plane : R*C*b/8 bytes, row-major.  Code (r, c) is in byte r*(C*b/8) + (c*b)/8
 *                at bit offset (c*b) % 8: the lowest bits hold the lowest column.
 *   sb plane   : R*(C/64) pairs of bf16; pair (r, g) at uint16 index 2*(r*(C/64) + g),
 *                scale first, then bias.  w[r][c] = code(r,c) * scale(r, c/64) + bias(r, c/64).
 * Expert blob (gate and up are I x H, down is H x I), planes in this order, each starting
 * at an offset rounded up to 256 bytes, total size rounded up to 256 bytes:
 *   gate.codes, gate.sb, up.codes, up.sb, down.codes, down.sb
 * At H = 4096, I = 1024 a 4-bit blob is 7,077,888 bytes (6.75 MiB) and a 2-bit blob
 * 3,932,160 bytes; no padding occurs at those shapes.
 * ------------------------------------------------------------------------------------ */

/* One entry per expert of a layer, in DEVICE memory (the kernels select experts there).
 * blob: device address of the expert's packed blob, 256-byte aligned.
 * bits: 2 or 4.  Experts of one layer may mix widths (tiered store).  A value other than
 *       2 is read as 4; moe_check_experts() validates a table on the host. */
typedef struct moe_expert_desc {
    uint64_t blob;
    uint32_t bits;
    uint32_t reserved;   /* must be 0 */
} moe_expert_desc;

typedef struct moe_dims {
    int32_t hidden;      /* H */
    int32_t inter;       /* I (expert intermediate size) */
    int32_t n_experts;   /* E */
    int32_t top_k;       /* K */
} moe_dims;

/* One layer: a HOST struct holding DEVICE pointers. */
typedef struct moe_layer {
    const void *router;              /* device [E][H] row-major, router_dtype; 16-byte aligned */
    int32_t router_dtype;            /* MOE_F32 or MOE_BF16 */
    float norm_eps;                  /* RMSNorm epsilon, added to mean(x^2) inside the sqrt */
    const float *logit_bias;         /* device [E] fp32 added to the logits, or NULL */
    const uint16_t *norm_w;          /* device [H] bf16 RMSNorm weight, or NULL for no norm */
    const moe_expert_desc *experts;  /* device [E] */
} moe_layer;

/* --------------------------------------------------------------------------- errors */

/* Static string naming a status code. */
const char *moe_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none).  Valid until the next
 * call on this thread. */
const char *moe_last_error(void);

/* Library version string. */
const char *moe_version(void);

/* --------------------------------------------------------------------------- format (host only) */

/* Bytes of one code plane / one sb plane / one expert blob; 0 for unsupported arguments
 * (rows, cols or dims < 1, cols or dims not multiples of 64, bits not in {2,4}). */
size_t moe_packed_codes_bytes(int rows, int cols, int bits);
size_t moe_packed_sb_bytes(int rows, int cols);
size_t moe_packed_expert_bytes(int hidden, int inter, int bits);

/* Byte offsets of the six planes inside one expert blob, in the order listed above.
 * off: host [6].  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_BITS. */
int moe_expert_plane_offsets(int hidden, int inter, int bits, size_t off[6]);

/* Pack one R x C matrix.  codes: host [R*C], one code per byte (must be < 2^bits);
 * scale, bias: host [R*(C/64)] bf16.  Writes codes_out (host, codes_out_bytes >=
 * moe_packed_codes_bytes) and sb_out (host, sb_out_bytes >= moe_packed_sb_bytes).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_BITS (also for a code >= 2^bits),
 * MOE_ERR_BUFFER. */
int moe_pack_matrix(const uint8_t *codes, const uint16_t *scale, const uint16_t *bias,
                    int rows, int cols, int bits,
                    uint8_t *codes_out, size_t codes_out_bytes,
                    uint16_t *sb_out, size_t sb_out_bytes);

/* Inverse of moe_pack_matrix (host buffers; codes [R*C], scale/bias [R*(C/64)]). */
int moe_unpack_matrix(const uint8_t *codes_in, const uint16_t *sb_in, int rows, int cols, int bits,
                      uint8_t *codes, uint16_t *scale, uint16_t *bias);

/* Pack a whole expert: matrices in the order gate (I x H), up (I x H), down (H x I), each
 * given as (codes, scale, bias) host arrays as for moe_pack_matrix.  Writes the blob,
 * padding included, to blob_out (host, blob_out_bytes >= moe_packed_expert_bytes). */
int moe_pack_expert(const uint8_t *const codes[3], const uint16_t *const scale[3],
                    const uint16_t *const bias[3], int hidden, int inter, int bits,
                    void *blob_out, size_t blob_out_bytes);

/* Quantise real weights into the packed format (device in, device out; the step before the
 * packer): per row r and group g of 64 columns, lo and hi = min and max of the 64 weights,
 *   scale = bf16((hi - lo) / (2^bits - 1)),  bias = bf16(lo),
 *   code  = nearest integer (ties to even) to (w - bias) / scale, clamped to [0, 2^bits - 1],
 *           and 0 where the bf16 scale is 0,
 * every step in fp32 with the stored bf16 pair.  The pages name an MLX 4-bit affine base
 * (tomo3141592653.github.io, "iPhone 17 Proで400Bパラメータ LLM を動かす「flash-moe」",
 * section "ハイブリッド量子化") and the form w = q * scale + bias (lilting.ch, "397Bパラメータ
 * モデルを48GB MacBookで動かすFlash-MoE", section "Metal Compute Shaders"), not the rounding;
 * this is the plain reading.
 *   w      device [rows][cols], w_dtype (MOE_F32 or MOE_BF16), finite values, 16-byte aligned
 *   codes  device code plane, moe_packed_codes_bytes(rows, cols, bits) bytes, 16-byte aligned
 *   sb     device (scale, bias) plane, moe_packed_sb_bytes(rows, cols) bytes, 4-byte aligned
 * The planes are the layout above: gate, up and down of an expert quantised into the offsets of
 * moe_expert_plane_offsets make a blob.  Asynchronous on `stream`.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (rows < 1, cols not a positive multiple of 64),
 * MOE_ERR_DTYPE, MOE_ERR_BITS, MOE_ERR_ALIGN, MOE_ERR_LAUNCH. */
int moe_quantize_matrix(const void *w, int w_dtype, int rows, int cols, int bits, uint8_t *codes,
                        uint16_t *sb, void *stream);

/* --------------------------------------------------------------------------- tiered store policy */
/* The pages keep the experts a model uses often at 4 bits and store the rest at 2 bits
 * (nzkcom.pages.dev, "flash-moe-romance-vs-utility", adopted-optimisation table; an MLX 4-bit
 * base: tomo3141592653.github.io, "iPhone 17 Proで400Bパラメータ LLM を動かす「flash-moe」",
 * section "ハイブリッド量子化"), without saying how use is measured or how a 2-bit expert is made.
 * The three calls below are the plain reading: count routing selections over a token stream,
 * rank the experts by count, requantise the cold ones from their base blobs.  All device in,
 * device out, asynchronous on `stream`. */

/* counts[e] += number of entries of idx equal to e, for e in [0, n_experts); entries outside that
 * range are not counted.  Accumulates, so a token stream may span many calls: zero counts
 * before the first.  Counts wrap modulo 2^32.
 *   idx    device [n] int32, e.g. the [T][K] routing indices moe_route writes (n = T * K)
 *   counts device [n_experts] uint32
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (n < 0, n_experts outside [1, MOE_MAX_EXPERTS]),
 * MOE_ERR_ALIGN, MOE_ERR_LAUNCH. */
int moe_expert_usage(const int32_t *idx, int n, int n_experts, uint32_t *counts, void *stream);

/* order = the experts ranked by counts, largest first; equal counts rank the lower expert index
 * first.  The first n entries of order are the hot set of size n.
 *   counts device [n_experts] uint32;  order device [n_experts] int32 (a permutation)
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_LAUNCH. */
int moe_hot_order(const uint32_t *counts, int n_experts, int32_t *order, void *stream);

/* Re-tier a layer: the experts order[0 .. n_hot-1] are hot and keep their base blobs; the expert
 * of rank r >= n_hot is cold: each of its three matrices is dequantised from its base blob (any
 * width, w = q * scale + bias in fp32) and quantised again at cold_bits with the rounding of
 * moe_quantize_matrix, into the cold blob at store + (r - n_hot) * moe_packed_expert_bytes(H, I,
 * cold_bits).  Then tiered[e] = base[e] for a hot expert and {its cold blob, cold_bits} for a
 * cold one.
 *   dims   host; hidden, inter, n_experts of the layer (top_k is only validated)
 *   base   device [n_experts] descriptor table of the base blobs (validate it with
 *          moe_check_experts; its blobs are read, not changed)
 *   order  device [n_experts] int32, a permutation of the experts (as moe_hot_order writes);
 *          an entry outside [0, n_experts) is skipped (its slot stays unwritten)
 *   store  device, 256-byte aligned, store_bytes >= (n_experts - n_hot) cold blobs; it must not
 *          overlap the base blobs
 *   tiered device [n_experts] descriptor table, written after every cold blob; it may be base
 *          itself (re-tiering in place)
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_BITS, MOE_ERR_ALIGN, MOE_ERR_BUFFER (store too
 * small), MOE_ERR_LAUNCH. */
int moe_retier(const moe_dims *dims, const moe_expert_desc *base, const int32_t *order, int n_hot,
               int cold_bits, void *store, size_t store_bytes, moe_expert_desc *tiered, void *stream);

/* --------------------------------------------------------------------------- expert cache */
/* For stores larger than device memory: the experts stay in host memory and a cache of slots in
 * device memory holds the recently used ones.  The pages stream each selected expert from SSD once
 * routing is known and let the OS page cache keep recently read experts (lilting.ch, "397Bパラメータ
 * モデルを48GB MacBookで動かすFlash-MoE", section "コア技術: SSDエキスパートストリーミング"); here a
 * routing step's indices, copied to the host, drive host-to-device copies of the missing experts
 * into least recently used slots.  A step: moe_route -> copy idx to the host -> moe_cache_fetch ->
 * moe_expert_ffn with the cache's table as the layer's experts -> moe_combine.
 * A cache object is host state; calls on one cache must not overlap (serialise them). */
typedef struct moe_expert_cache moe_expert_cache;

#define MOE_CACHE_DRY_RUN 1u   /* policy only: no copies and no device writes (planning, host tests) */

/* Create a cache.
 *   dims          host; hidden, inter, n_experts (E), top_k of the layer
 *   host_experts  HOST [E]: blob = host address of expert e's packed blob, bits 2 or 4, reserved 0.
 *                 The list is copied; the blobs are read by later fetches and must stay valid and
 *                 unchanged until moe_cache_destroy.  Allocate them pinned (hipHostMalloc) so the
 *                 copies are asynchronous DMA.
 *   slots         device, n_slots * slot_bytes bytes, 256-byte aligned; slot_bytes a multiple of 256
 *                 and at least the largest expert blob (moe_packed_expert_bytes)
 *   n_slots       in [top_k, 2^20]
 *   table         device [E] descriptor table for the expert kernels (the moe_layer's experts).
 *                 Create enqueues on `stream` a fill marking every expert absent (blob 0); from then
 *                 on entry e is {its slot, its bits} while e is resident and blob 0 otherwise.  The
 *                 expert kernels give a zero output row for an absent expert (moe_check_experts,
 *                 which requires blobs, does not apply to such a table).
 *   flags         0 or MOE_CACHE_DRY_RUN (then slots, table and stream are not used and may be NULL)
 *   cache         out: the new cache, or NULL on error
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_BITS, MOE_ERR_ALIGN, MOE_ERR_BUFFER (slot too small),
 * MOE_ERR_UNSUPPORTED (flags), MOE_ERR_LAUNCH. */
int moe_cache_create(const moe_dims *dims, const moe_expert_desc *host_experts, void *slots,
                     size_t slot_bytes, int n_slots, moe_expert_desc *table, unsigned flags,
                     void *stream, moe_expert_cache **cache);

/* Make resident every distinct expert named in idx (HOST [n] int32, e.g. one routing step's [T][K]
 * indices; entries outside [0, E) are ignored).  First every such expert already resident is a
 * hit and becomes most recently used; then each missing one (in first-occurrence order) takes the
 * lowest free slot or, with none free, the slot used least recently among those this call has not
 * touched (equal times: the lower slot), evicting its expert.  Each miss enqueues a host-to-device
 * copy of the blob into its slot, then one small kernel writes the changed table entries (evicted
 * experts become absent), all on `stream` after the work already there: kernels enqueued earlier
 * still see a slot's previous expert.  misses (out, may be NULL): this call's misses.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE (n < 0, or more distinct experts than slots: nothing
 * changes), MOE_ERR_LAUNCH (an enqueue failed; the cache is then unusable: destroy it). */
int moe_cache_fetch(moe_expert_cache *cache, const int32_t *idx, int n, void *stream, int *misses);

/* Totals since creation: distinct-expert hits and misses, bytes copied to the device.  Any output
 * may be NULL.  Errors: MOE_ERR_NULL. */
int moe_cache_stats(const moe_expert_cache *cache, uint64_t *hits, uint64_t *misses, uint64_t *bytes);

/* Slot holding `expert`, -1 when it is not resident, -2 for a NULL cache or an expert outside
 * [0, E). */
int moe_cache_slot(const moe_expert_cache *cache, int expert);

/* Device-side policy: the same policy as moe_cache_fetch, run by a kernel on device indices, with
 * the missing blobs copied by a kernel that reads the pinned host store directly (zero-copy loads
 * at the host link's rate), so a routing step needs no host round trip:
 *   moe_route -> moe_cache_fetch_device -> moe_expert_ffn with the cache's table -> moe_combine.
 * moe_cache_device_state_bytes: bytes of device state for this cache (0: the device policy does not
 *   apply: a dry-run cache, or more than 2048 slots).
 * moe_cache_attach_device: copies the cache's residency so far into `state` (device, 256-byte
 *   aligned, state_bytes >= moe_cache_device_state_bytes) and synchronises `stream`.  From then on
 *   the policy state lives on the device: moe_cache_fetch is refused (MOE_ERR_UNSUPPORTED), and
 *   moe_cache_stats and moe_cache_slot read the device state (synchronous copies, so call them after
 *   the fetches they should see have completed).  Every host blob must be pinned memory the device
 *   can read (hipHostMalloc, or a pinned torch tensor): MOE_ERR_UNSUPPORTED otherwise.  Errors:
 *   MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_UNSUPPORTED, MOE_ERR_DEVICE.
 * moe_cache_fetch_device: idx device [n] int32 (entries outside [0, E) ignored).  Enqueues on
 *   `stream` one single-workgroup policy kernel (which also rewrites the changed table entries) and
 *   one copy kernel; calls on one cache must be stream-ordered.  A step naming more distinct experts
 *   than slots changes nothing and is counted (moe_cache_device_refused).  Errors: MOE_ERR_NULL,
 *   MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_UNSUPPORTED (not attached), MOE_ERR_LAUNCH.
 * moe_cache_device_refused: refused steps so far (synchronous read), -1 when not attached. */
size_t moe_cache_device_state_bytes(const moe_expert_cache *cache);
int moe_cache_attach_device(moe_expert_cache *cache, void *state, size_t state_bytes, void *stream);
int moe_cache_fetch_device(moe_expert_cache *cache, const int32_t *idx, int n, void *stream);
int moe_cache_device_refused(const moe_expert_cache *cache);

/* Free the cache's host state (device memory belongs to the caller; pending copies read host
 * blobs, so synchronise the stream before freeing those).  NULL is ignored. */
void moe_cache_destroy(moe_expert_cache *cache);

/* --------------------------------------------------------------------------- test hook */
/* Failure handling test hook: of the launch steps that compute calls make from now on (each kernel
 * launch, or group of launches, that the call checks), the next `after` proceed and the `count`
 * after them are refused before anything is enqueued, returning MOE_ERR_LAUNCH with a message
 * naming the injection.  (0, 0) switches it off.  Process-wide; tests only.
 * Errors: MOE_ERR_SHAPE (a negative argument). */
int moe_debug_inject_launch_failure(int after, int count);

/* Copy a device descriptor table to the host (synchronously, on the null stream) and
 * check it: non-NULL, 256-byte aligned blobs, bits in {2,4}, reserved == 0.
 * Errors: MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_BITS, MOE_ERR_SHAPE, MOE_ERR_DEVICE. */
int moe_check_experts(const moe_expert_desc *experts_dev, int n_experts);

/* --------------------------------------------------------------------------- workspace */

#define MOE_OP_ROUTE 1
#define MOE_OP_EXPERT_FFN 2
#define MOE_OP_LAYER_DECODE 3

/* Device workspace bytes needed by one call of `op` with these dims and T tokens
 * (n_layers for MOE_OP_LAYER_DECODE).  0 for unsupported arguments.  For MOE_OP_ROUTE and
 * MOE_OP_EXPERT_FFN the workspace is scratch: its contents need no initialisation and are
 * undefined after the call.  A MOE_OP_LAYER_DECODE workspace carries state from one
 * moe_layer_decode call to the next (a launch counter and hand-over words of the two-launch
 * layer schedule): zero-fill it once before its first moe_layer_decode call, and again
 * before going back to moe_layer_decode after using the same memory for anything else.
 * A moe_layer_decode call that returned MOE_ERR_LAUNCH may have run only part of a layer's launches:
 * zero-fill its workspace again before the next moe_layer_decode call.
 * Calls sharing a workspace must be ordered (same stream, or synchronised); two calls that
 * may run concurrently need separate workspaces. */
size_t moe_workspace_bytes(int op, const moe_dims *dims, int T, int n_layers);

/* --------------------------------------------------------------------------- compute */

/* Router for T tokens: steps n, logits, softmax, top-K and renormalisation above.
 *   x      device [T][H], x_dtype, 16-byte aligned
 *   idx    device [T][K] int32, descending weight (ties: lower expert index first)
 *   w      device [T][K] fp32 renormalised weights (each row sums to 1)
 *   logits device [T][E] fp32 pre-softmax logits (bias included), or NULL
 * For T >= 64 with a bf16 router (H a multiple of 256) the logits come from MFMA tiles; with a norm
 * weight the normalised rows are first written to the workspace after the logits (the size from
 * moe_workspace_bytes includes them; a smaller workspace that still holds the logits makes the
 * matvec router normalise in registers instead).  While the tiles are fewer than 256 the tiles'
 * K range is split across 2 to 8 workgroups, whose partial logit rows follow the normalised rows in
 * the workspace and are summed in split order by the top-K step (without room for them the tiles
 * run unsplit; the logits may then differ in the last bits).
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE,
 * MOE_ERR_LAUNCH. */
int moe_route(const moe_dims *dims, const moe_layer *layer, const void *x, int x_dtype, int T,
              int32_t *idx, float *w, float *logits, void *ws, size_t ws_bytes, void *stream);

/* Expert FFN for T tokens and the K experts each token selected:
 *   y[t][k] = W_down[e] (silu(W_gate[e] n_t) * (W_up[e] n_t)),  e = idx[t][k]
 *   x   device [T][H] x_dtype (normalised inside when the layer has a norm weight)
 *   idx device [T][K] int32; an entry outside [0, E) gives a zero row of y
 *   y   device [T][K][H] fp32
 * The kernels are chosen by T (moe_expert_ffn_path below names them):
 *   T < 8, and T <= 24 when the shared-read path does not apply: MOE_FFN_PER_TOKEN;
 *   8 <= T <= 16 with T*K <= 64: MOE_FFN_SHARED (measured on a 4096 x 1024, 512-expert top-4 layer:
 *     within 2 % of the per-token kernels at 8-10 tokens with distinct experts, up to 9 % faster when
 *     tokens share experts, faster on every routing from 12 tokens);
 *   T > 24: MOE_FFN_GROUPED (T*K <= 32768).
 * Errors as moe_route, and MOE_ERR_UNSUPPORTED when T*K exceeds 32768 above 24 tokens. */
int moe_expert_ffn(const moe_dims *dims, const moe_layer *layer, const void *x, int x_dtype, int T,
                   const int32_t *idx, float *y, void *ws, size_t ws_bytes, void *stream);

/* moe_expert_ffn with the kernels chosen by the caller (same arguments, results equal within the
 * parity tolerance whatever the path; moe_workspace_bytes(MOE_OP_EXPERT_FFN) covers every path
 * that can take T):
 *   MOE_FFN_AUTO       the choice moe_expert_ffn makes.
 *   MOE_FFN_PER_TOKEN  T <= 24: the decode matvec kernels, all K experts in one launch per phase,
 *                      one grid row per token; every token streams the experts it selected.
 *   MOE_FFN_SHARED     2 <= T <= 16 and T*K <= 64 (and the staged rows fit in LDS: 8 rows (4 when
 *                      T <= 4) of H and of I inputs at 2.25 bytes per input, and 8 bytes per
 *                      expert): each distinct expert of idx is streamed once for all (token, slot)
 *                      pairs that chose it, its workgroups staging those pairs' activations.  Three
 *                      launches: the T rows (normalised when the layer has a norm weight) converted
 *                      once to the kernels' 16-bit fixed-point layout, then gate/up and down, which
 *                      find the distinct experts themselves (no grouping pass).  An expert chosen by more than 16
 *                      pairs (8 when T <= 4; only possible when tokens repeat experts within their
 *                      K) is streamed once per 16 (8) pairs.  Motivation: the nzkcom.pages.dev page
 *                      "flash-moe-romance-vs-utility", section on admitting geek romance, table of
 *                      rejected optimisations, multi-token-prediction row: MoE decoding pays expert
 *                      I/O per token, so several tokens gain only when they share the reads.
 *   MOE_FFN_GROUPED    2 <= T, T*K <= 32768: the T*K (token, slot) pairs are grouped by expert;
 *                      experts with more than 8 tokens run the grouped dequant-GEMM (MFMA) kernels,
 *                      the others integer dot-product kernels over their staged tokens.  The MFMA
 *                      kernels run on a second stream of the device, forked from `stream` with an
 *                      event and joined back to it before the call returns (graph capture follows
 *                      the fork); the library creates that stream on the first grouped call on a
 *                      device and keeps it until the process ends.
 * Errors as moe_expert_ffn; MOE_ERR_UNSUPPORTED for an unknown path or a T the path cannot take. */
#define MOE_FFN_AUTO 0
#define MOE_FFN_PER_TOKEN 1
#define MOE_FFN_SHARED 2
#define MOE_FFN_GROUPED 3
int moe_expert_ffn_path(const moe_dims *dims, const moe_layer *layer, const void *x, int x_dtype, int T,
                        const int32_t *idx, float *y, void *ws, size_t ws_bytes, int path, void *stream);

/* Weighted combine: out[t][c] = sum_k w[t][k] * y[t][k][c] (+ residual[t][c]).
 *   y device [T][K][H] fp32, w device [T][K] fp32, residual device [T][H] fp32 or NULL,
 *   out device [T][H] fp32 (may alias residual).  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE,
 *   MOE_ERR_LAUNCH. */
int moe_combine(const float *y, const float *w, int T, int K, int H, const float *residual,
                float *out, void *stream);

#define MOE_FLAG_RESIDUAL 1u          /* out = x + MoE(x) (pre-norm residual block) */
#define MOE_FLAG_SEPARATE_KERNELS 2u  /* run each layer as three kernels (router, gate/up, down) */
#define MOE_FLAG_SINGLE_LAUNCH 4u     /* run each layer as one launch of a persistent grid */

/* One decode token through n_layers layers (1 <= n_layers <= 4096); layer l's output is
 * layer l+1's input.  Per layer: [RMSNorm] -> router -> top-K -> gate/up/SwiGLU for all K
 * experts -> down projection + weighted combine (+ residual).
 * By default a layer is two kernel launches: router and gate/up run as two groups of
 * workgroups of one grid, the logits passing between them through the workspace (see
 * moe_workspace_bytes for its zero-fill rule), then the down + combine kernel.  The gate/up
 * workgroups only wait for router workgroups started before them, and the wait is bounded: if it
 * ever runs out, the workspace's error word becomes nonzero and this and every later call with
 * that workspace write NaN outputs until it is zero-filled again.  MOE_FLAG_SEPARATE_KERNELS
 * selects three launches per layer (router, gate/up, down); MOE_FLAG_SINGLE_LAUNCH one launch of a
 * grid whose workgroups each compute router rows, gate/up and down units, handing the logits and h
 * over through the workspace (the grid is sized to what the device can hold resident at once; every
 * wait is bounded as above).  Same arithmetic in all three, except that the single launch hands h
 * over truncated to 19 mantissa bits (a relative change below 2^-19).  The flags exclude each other.
 *   layers host [n_layers]
 *   x      device [H] x_dtype (input of the first layer), 16-byte aligned
 *   out    device [H] fp32 output of the last layer
 *   idx    device [n_layers][K] int32, or NULL
 *   w      device [n_layers][K] fp32, or NULL
 * Errors as moe_route (MOE_ERR_UNSUPPORTED for unknown flags). */
int moe_layer_decode(const moe_dims *dims, const moe_layer *layers, int n_layers, const void *x,
                     int x_dtype, unsigned flags, float *out, int32_t *idx, float *w,
                     void *ws, size_t ws_bytes, void *stream);

/* For callers that cannot allocate (code under HIP graph capture, serving loops that forbid
 * allocation): moe_layer_decode with its workspace in a device array the library holds, one per
 * device, MOE_STATIC_SCRATCH_BYTES (256 KiB) large, so the caller passes inputs and outputs only and
 * the call allocates nothing.  The array starts zeroed and keeps the state of the last call on the
 * device (launch counter, hand-over words); calls on one device that may overlap (different streams
 * without ordering) race on it and must not be issued.  Unlike moe_layer_decode, a timed-out wait
 * makes only the call it happens in write NaN outputs.  Arguments as moe_layer_decode.
 * Errors as moe_layer_decode; MOE_ERR_WORKSPACE when the dims need more than the array holds
 * (moe_workspace_bytes(MOE_OP_LAYER_DECODE, ...) > MOE_STATIC_SCRATCH_BYTES), MOE_ERR_DEVICE when the
 * array's device address cannot be obtained. */
#define MOE_STATIC_SCRATCH_BYTES (1u << 18)
int moe_layer_decode_static(const moe_dims *dims, const moe_layer *layers, int n_layers, const void *x,
                            int x_dtype, unsigned flags, float *out, int32_t *idx, float *w, void *stream);

/* moe_layer_decode with per-kernel timing, the library's counterpart of the pages' per-layer
 * timing breakdown (lilting.ch page, "遅延GPU実行" section, per-layer time table).  It runs the
 * schedule `flags` selects, kernel j of the call (in issue order) getting the start/stop pair
 * events[2j], events[2j+1]:
 *   default (two launches per layer): 4*n_layers events; layer l's router + gate/up launch is
 *           kernel 2l and its down kernel 2l+1;
 *   MOE_FLAG_SINGLE_LAUNCH: 2*n_layers events; layer l's launch is kernel l;
 *   MOE_FLAG_SEPARATE_KERNELS: 6*n_layers events; layer l's router, gate/up and down kernels are
 *           kernels 3l, 3l+1, 3l+2.
 * Each kernel is launched through hipExtLaunchKernel with its pair, which the runtime stamps with
 * the dispatch's own start and end, so hipEventElapsedTime(events[2j], events[2j+1]) is kernel
 * j's execution time without the gaps between kernels.  The events are hipEvent_t created by the
 * caller on the current device.  The call cannot be captured into a graph (MOE_ERR_UNSUPPORTED
 * while `stream` is capturing).
 * Other arguments and errors as moe_layer_decode (MOE_ERR_NULL when events or one of its
 * entries is NULL). */
int moe_layer_decode_timed(const moe_dims *dims, const moe_layer *layers, int n_layers, const void *x,
                           int x_dtype, unsigned flags, float *out, int32_t *idx, float *w,
                           void *ws, size_t ws_bytes, void *stream, void *const *events);

/* --------------------------------------------------------------------------- measurement */

/* Read-stream reference for the HBM roofline, not part of the expert path: reads the `bytes`
 * bytes at `buf` once with 16-byte non-temporal loads from every compute unit (the access
 * pattern of the expert weight stream) and XORs every dword into *sink, one atomic per
 * wavefront.  The benchmark times it over a buffer far larger than the caches to report the
 * measured read bandwidth beside the nominal peak.
 *   buf   device, 16-byte aligned, caller-owned
 *   bytes a positive multiple of 16
 *   sink  device uint32, 4-byte aligned; zero it first to get the XOR of the data
 * Errors: MOE_ERR_NULL, MOE_ERR_ALIGN, MOE_ERR_SHAPE, MOE_ERR_LAUNCH. */
int moe_stream_read(const void *buf, size_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DEQUANT_H */
