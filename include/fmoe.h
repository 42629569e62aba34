/*
 * fmoe.h -- C ABI of libfmoe: the quantized Mixture-of-Experts expert forward at
 * decode time, for AMD Instinct MI355X (gfx950).
 *
 * What the library computes comes from the Flash-MoE pages:
 *  [P1] "397B MoE en MacBook: Motor Flash-MoE a 4,4 t/s" (aibit.im)
 *  [P2] "Flash-MoE: Ausfuehren eines 397B-Parameter-Qwen-Modells auf dem MacBook
 *       Pro mit reinem C/Metal" (openclawradar.com)
 * Per layer it takes the hidden state, picks K of the layer's experts by softmax
 * top-K ([P2] "Pipeline-Leistung"; 512 experts, K=4 plus one shared expert in
 * [P2] "Technische Implementierung"), runs each chosen expert's SwiGLU
 * feed-forward on 4-bit or 2-bit group-affine quantized weights
 * (weight = code*scale + bias, evaluated as fma(code, scale*x, bias*x):
 * [P1] "2. Kernel de desquantizacion optimizado con FMA", [P2]
 * "FMA-optimierter Dequant-Kernel"), and combines the outputs with their routing
 * weights, the sigmoid-gated shared expert and the residual ([P2]
 * "Metal-Compute-Shader": fused MoE combination + residual + sigmoid gate).
 *
 * ---------------------------------------------------------------- conventions
 * Pointers. Every array argument of an entry point that enqueues GPU work is a
 * DEVICE pointer (HBM, e.g. hipMalloc or a torch tensor's data_ptr()); the pack
 * and unpack helpers without "_device" in their name take HOST pointers. fp32
 * arrays are row-major and contiguous and must be 16-byte aligned; quantized
 * blobs and workspaces must be 256-byte aligned.
 *
 * Ownership. The caller allocates and frees everything: blobs, activations and
 * workspaces. The library never allocates or frees device memory; its only
 * device state is the static workspace of fmoe_moe_layer_noalloc. Blobs are
 * read-only during a call.
 *
 * Asynchrony. A device entry point validates its arguments on the host, enqueues
 * its kernels on `stream` (a hipStream_t; NULL means the null stream) and
 * returns. It never synchronises, so it can be captured in a HIP graph. Results
 * are valid once the caller has synchronised the stream; a device fault surfaces
 * there, not as a status.
 *
 * Errors. Validation is synchronous and complete before the first launch: on
 * any status other than FMOE_OK nothing was enqueued and no output was written.
 * FMOE_ERR_LAUNCH reports a launch the HIP runtime refused (earlier kernels of
 * the same call may have been enqueued). No C++ exception crosses this ABI.
 *
 * Determinism. Identical inputs give bitwise identical outputs and routing:
 * every reduction runs in a fixed order and no floating-point atomics are used.
 *
 * Re-entrancy. Calls are re-entrant; calls that may run concurrently need
 * distinct workspaces and outputs.
 *
 * Supported set. bits in {4, 2}; group == 64; every quantized matrix has cols a
 * multiple of 256 from 256 to 4096 (so hidden and inter are such multiples: 768,
 * 1536, 3072, ... as well as the powers of two) and rows >= 1; 1 <= top_k <=
 * FMOE_MAX_TOPK; 1 <= n_experts <= FMOE_MAX_EXPERTS; 1 <= n_tokens <=
 * FMOE_MAX_TOKENS. The tuned shape is hidden 4096, inter 1024, 512 experts, top_k 4.
 * (A row's 64-column groups are spread one per lane over a wavefront, so 4096
 * columns is the widest row; widths that are not powers of two leave some lanes
 * of a row's segment idle.)
 *
 * ---------------------------------------------------------------- blob layout
 * A quantized matrix W [rows][cols] is stored as `rows` row records. A row
 * record holds cols/64 groups of 64 codes and, after the codes, one 32-bit
 * word per group: (bf16 scale << 16) | bf16 bias.
 *   4-bit: record = [first halves of all groups: 16 B each]
 *                   [second halves of all groups: 16 B each][scale/bias words]
 *          (36 bytes per group). In the 16-byte half h of group g, byte k of
 *          32-bit word w holds column 64g+32h+8w+k in its low nibble and column
 *          64g+32h+8w+4+k in its high nibble.
 *   2-bit: record = [groups: 16 B each][scale/bias words] (20 bytes per group).
 *          Byte k of word w of group g holds column 64g+16w+4q+k in bits 2q..2q+1.
 * An expert blob is [gate row 0][up row 0][gate row 1][up row 1]...
 * [gate row inter-1][up row inter-1] (records over hidden columns) followed by
 * the `hidden` row records of down (records over inter columns). A bank of
 * experts is n_experts expert blobs at a stride of fmoe_expert_bytes().
 * Use the pack functions; the layout may change between library versions.
 */
#ifndef FMOE_H_
#define FMOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FMOE_GROUP 64
#define FMOE_MAX_TOPK 16
#define FMOE_MAX_TOKENS 256
#define FMOE_MAX_EXPERTS 1024

typedef enum fmoe_status {
  FMOE_OK = 0,
  FMOE_ERR_NULL = 1,      /* a required pointer is NULL                                   */
  FMOE_ERR_SHAPE = 2,     /* rows/cols/hidden/inter/group unsupported or inconsistent     */
  FMOE_ERR_ALIGN = 3,     /* fp32 array not 16-B aligned, or blob not 256-B aligned       */
  FMOE_ERR_BITS = 4,      /* bits not 4 (q4 entry), not 2 (q2 entry), not in {2,4} else  */
  FMOE_ERR_ROUTING = 5,   /* top_k < 1, top_k > n_experts, top_k > FMOE_MAX_TOPK,
                             or n_experts outside [1, FMOE_MAX_EXPERTS]                    */
  FMOE_ERR_BATCH = 6,     /* n_tokens < 1 or n_tokens > FMOE_MAX_TOKENS, or n_layers < 1  */
  FMOE_ERR_WORKSPACE = 7, /* workspace NULL or smaller than the matching *_bytes() query  */
  FMOE_ERR_LAUNCH = 8,    /* the HIP runtime refused a kernel launch                      */
  FMOE_ERR_ALIAS = 9      /* an input aliases an output or the workspace it must not      */
} fmoe_status;

/* One packed quantized matrix (see "blob layout"). */
typedef struct fmoe_qmat {
  const void *blob; /* device, 256-B aligned, fmoe_qmat_bytes(bits, rows, cols, group) bytes */
  int32_t rows, cols, bits, group;
} fmoe_qmat;

/* One packed SwiGLU expert: gate and up [inter][hidden], down [hidden][inter]. */
typedef struct fmoe_expert {
  const void *blob; /* device, 256-B aligned, fmoe_expert_bytes(bits, hidden, inter, group) */
  int32_t hidden, inter, bits, group;
} fmoe_expert;

/* One MoE layer. */
typedef struct fmoe_layer {
  const float *router;      /* device fp32 [n_experts][hidden], row-major                   */
  const float *shared_gate; /* device fp32 [hidden]; the shared expert's gate is
                               sigmoid(shared_gate . x). Ignored when shared == NULL.      */
  const void *bank;         /* device: n_experts expert blobs, stride fmoe_expert_bytes()   */
  const void *shared;       /* device: one expert blob, or NULL for a layer without a
                               shared expert                                               */
  int32_t n_experts, top_k, hidden, inter, bits, group;
} fmoe_layer;

/* ------------------------------------------------------------------ sizes */

/* Bytes of one packed matrix; 0 if the arguments are outside the supported set. */
size_t fmoe_qmat_bytes(int bits, int rows, int cols, int group);
/* Bytes of one packed expert (4, 4096, 1024, 64 -> 7,077,888 = 6.75 MiB); 0 if unsupported. */
size_t fmoe_expert_bytes(int bits, int hidden, int inter, int group);
/* Workspace of fmoe_expert_ffn for one token; 0 if unsupported. */
size_t fmoe_expert_workspace_bytes(const fmoe_expert *E);
/* Workspace of fmoe_moe_layer for n_tokens tokens; 0 if unsupported. */
size_t fmoe_workspace_bytes(const fmoe_layer *L, int n_tokens);
/* Workspace of fmoe_moe_stack for n_tokens tokens (every layer shaped like L); 0 if unsupported. */
size_t fmoe_stack_workspace_bytes(const fmoe_layer *L, int n_tokens);

/* ------------------------------------------------------------------ packing
 * Canonical input (host or device, as named): codes uint8 [rows][cols], one
 * unsigned code in [0, 2^bits) per element (higher bits must be zero, else
 * FMOE_ERR_SHAPE from the host packers; the device packers mask them off);
 * scale and bias uint16 [rows][cols/group], bf16 bit patterns. blob_out
 * receives fmoe_qmat_bytes() bytes. */
fmoe_status fmoe_pack_qmat(int bits, int rows, int cols, int group, const uint8_t *codes,
                           const uint16_t *scale, const uint16_t *bias, void *blob_out);
fmoe_status fmoe_unpack_qmat(int bits, int rows, int cols, int group, const void *blob,
                             uint8_t *codes, uint16_t *scale, uint16_t *bias);
/* codes/scale/bias[0..2] = gate [inter][hidden], up [inter][hidden], down [hidden][inter]. */
fmoe_status fmoe_pack_expert(int bits, int hidden, int inter, int group, const uint8_t *const codes[3],
                             const uint16_t *const scale[3], const uint16_t *const bias[3],
                             void *blob_out);
fmoe_status fmoe_unpack_expert(int bits, int hidden, int inter, int group, const void *blob,
                               uint8_t *const codes[3], uint16_t *const scale[3],
                               uint16_t *const bias[3]);
/* Device twins: all pointers are device pointers; work is enqueued on `stream`. */
fmoe_status fmoe_pack_qmat_device(int bits, int rows, int cols, int group, const uint8_t *codes,
                                  const uint16_t *scale, const uint16_t *bias, void *blob_out,
                                  void *stream);
fmoe_status fmoe_pack_expert_device(int bits, int hidden, int inter, int group,
                                    const uint8_t *const codes[3], const uint16_t *const scale[3],
                                    const uint16_t *const bias[3], void *blob_out, void *stream);

/* ------------------------------------------------------------------ compute */

/* y[r] = sum_c (code[r][c]*scale[r][c/64] + bias[r][c/64]) * x[c] for a 4-bit matrix
 * ([P2] "FMA-optimierter Dequant-Kernel"; [P2] "Metal-Compute-Shader": 4-bit dequantized
 * matrix-vector multiplication). x: device fp32 [cols]; y: device fp32 [rows], must not
 * overlap x. FMOE_ERR_BITS unless W->bits == 4. */
fmoe_status fmoe_q4_matvec(const fmoe_qmat *W, const float *x, float *y, void *stream);
/* The same for a 2-bit matrix ([P2] "Metal-Compute-Shader": 2-bit dequantized matvec).
 * FMOE_ERR_BITS unless W->bits == 2. */
fmoe_status fmoe_q2_matvec(const fmoe_qmat *W, const float *x, float *y, void *stream);

/* Comparison aid: y = W x for a matrix of either bit width (W->bits), with the
 * per-weight arithmetic in one of four forms, c the code, s and b its group's scale
 * and bias: form 0 naive, w = c*s + b then w*x accumulated; form 1 the recast
 * fma(c, s*x, b*x) per weight ([P1] "2. Kernel de desquantizacion optimizado con
 * FMA", [P2] "FMA-optimierter Dequant-Kernel"); form 2 group-factored,
 * s * sum c*x + b * sum x per 64-column group (the form of fmoe_q4_matvec and every
 * other call); form 3 a per-(row, group) table of c*s + b in LDS read per weight
 * (the GPU dequant lookup table of [P1] "Lo que descartaron"). One row iteration per
 * wavefront. Results agree with fmoe_q4_matvec / fmoe_q2_matvec up to fp32
 * rounding (summation order and form differ). Arguments and errors as
 * fmoe_q4_matvec, without the bit-width restriction; FMOE_ERR_SHAPE if form is
 * outside 0..3. */
fmoe_status fmoe_qmatvec_form(const fmoe_qmat *W, const float *x, float *y, int form, void *stream);

/* One SwiGLU expert on one token: out = down( silu(gate x) * (up x) ), silu(z) = z/(1+e^-z)
 * ([P2] "Metal-Compute-Shader": fused SwiGLU activation). x: device fp32 [hidden];
 * out: device fp32 [hidden], must not overlap x; ws: device, >= fmoe_expert_workspace_bytes. */
fmoe_status fmoe_expert_ffn(const fmoe_expert *E, const float *x, float *out, void *ws, size_t ws_bytes,
                            void *stream);

/* Comparison aid: fmoe_expert_ffn with the per-weight arithmetic of every projection in
 * form `form` (0 naive, 1 fma recast, 2 group-factored, 3 table in LDS; as
 * fmoe_qmatvec_form): the fused gate/up + SwiGLU kernel, then the down projection as
 * fmoe_qmatvec_form does it. Results agree with fmoe_expert_ffn up to fp32 rounding.
 * Arguments and errors as fmoe_expert_ffn; FMOE_ERR_SHAPE if form is outside 0..3. */
fmoe_status fmoe_expert_ffn_form(const fmoe_expert *E, const float *x, float *out, void *ws, size_t ws_bytes,
                                 int form, void *stream);

/* One MoE layer for n_tokens independent tokens t:
 *   logits = router x_t; p = softmax(logits); T = the top_k experts by p (descending,
 *   lower index first on a tie); w_j = p[T_j] / sum_{i in T} p[i];
 *   out_t = residual_t + sum_j w_j E_{T_j}(x_t) + sigmoid(shared_gate . x_t) E_shared(x_t)
 * ([P2] "Pipeline-Leistung", "Technische Implementierung", "Metal-Compute-Shader").
 * x, residual, out: device fp32 [n_tokens][hidden]; out may equal residual (in-place
 * residual update) but must not overlap it otherwise, nor overlap x or ws. topk_idx
 * (int32) and topk_w (fp32): device [n_tokens][top_k] or NULL; neither may overlap the
 * other, x, residual, out or ws. ws: device, >= fmoe_workspace_bytes(L, n_tokens).
 * FMOE_ERR_ALIAS for any overlap named here.
 * With n_tokens > 1 the tokens are grouped by expert: the router, the shared expert and
 * each distinct chosen expert are read from HBM once per call and applied to every token
 * that uses them (results equal the one-token definition above, per token). */
fmoe_status fmoe_moe_layer(const fmoe_layer *L, int n_tokens, const float *x, const float *residual,
                           float *out, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                           void *stream);

/* Comparison aid: fmoe_moe_layer for one token with the per-weight arithmetic of every
 * expert projection (the routed and shared experts' gate/up and down) in dequant form
 * `form` (0 naive, 1 fma recast, 2 group-factored, 3 table in LDS; as fmoe_qmatvec_form).
 * The router, top-K and combine are fmoe_moe_layer's; the gate/up kernel takes x in fp32
 * instead of the digit form its library build uses ([P1] "2. Kernel de desquantizacion
 * optimizado con FMA", [P1] "Lo que descartaron"). Results agree with fmoe_moe_layer up
 * to fp32 rounding. Arguments and errors as fmoe_moe_layer with n_tokens = 1;
 * FMOE_ERR_SHAPE if form is outside 0..3 or the layer is not hidden 4096, inter 1024 with
 * at most 512 experts; FMOE_ERR_ROUTING unless top_k == 4. */
fmoe_status fmoe_moe_layer_form(const fmoe_layer *L, const float *x, const float *residual, float *out,
                                int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, int form,
                                void *stream);

/* Diagnostic form of fmoe_moe_layer for per-kernel timing: enqueues only some of
 * the layer's kernels, in order. One token -- bit 0: router and the shared-expert
 * gate sigma; bit 1: routing + routed and shared-expert gate/up; bit 2: routed and
 * shared-expert down + combine. Several tokens -- bit 0: router and the input
 * preparation; bit 1: routing and grouping with the routed and shared-expert
 * gate/up; bit 2: routed and shared-expert down, then combine. phases == 7 is
 * fmoe_moe_layer. A kernel reads what the
 * previous ones left in ws, so partial calls are meaningful only after a full
 * call with the same ws and inputs. FMOE_ERR_BATCH if phases is outside 1..7;
 * otherwise the arguments and errors of fmoe_moe_layer. */
fmoe_status fmoe_moe_layer_phases(const fmoe_layer *L, int n_tokens, const float *x, const float *residual,
                                  float *out, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                                  int phases, void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): fmoe_moe_layer with its
 * workspace in a static device array that the library holds on every GPU it runs
 * on, FMOE_NOALLOC_SCRATCH_BYTES (4 MiB) per GPU, kept until the process ends,
 * instead of a caller's ws. The call allocates and frees nothing. Every call on one
 * GPU shares that GPU's array, so calls that may overlap on one GPU (other streams,
 * other threads) race and give undefined results; calls on one stream are ordered.
 * FMOE_ERR_WORKSPACE if fmoe_workspace_bytes(L, n_tokens) exceeds the array (at
 * hidden 4096, inter 1024, 512 experts and top_k 4: above 32 tokens);
 * FMOE_ERR_LAUNCH if the array's device address cannot be looked up; otherwise the
 * arguments, results and errors of fmoe_moe_layer. */
#define FMOE_NOALLOC_SCRATCH_BYTES (4u << 20)
fmoe_status fmoe_moe_layer_noalloc(const fmoe_layer *L, int n_tokens, const float *x, const float *residual,
                                   float *out, int32_t *topk_idx, float *topk_w, void *stream);

/* ------------------------------------------------------------------ host-memory expert tier
 * The pages stream the routed experts from SSD and let the operating system's
 * page cache keep the recently used ones in memory ([P1] "1. Streaming de
 * expertos desde SSD + 'Confia en el SO'", [P2] "SSD-Experten-Streaming"). Here
 * the slow tier is host memory: a layer's routed expert bank lives in host memory
 * (fmoe_layer.bank is then a HOST pointer, best pinned: hipHostMalloc or a pinned
 * torch tensor, so that the copies are DMA transfers), and an HBM cache of n_slots
 * expert blobs holds the most recently used (layer, expert) pairs. The router,
 * the shared-expert gate vector and the shared expert stay in device memory.
 *
 * fmoe_cache_device_bytes: bytes of the caller's device buffer for a cache of
 * n_slots blobs of experts with this shape and up to n_experts experts per layer
 * (the slots, a table of blob addresses and the state of the policy when it runs on
 * the GPU: 16 bytes per slot and 8 KB); 0 if unsupported.
 * fmoe_cache_create: the cache over that buffer (256-B aligned, device_bytes at
 * least the above). The library allocates the host bookkeeping here and, at the
 * first tiered call, two small pinned host buffers (the routing read-back and the
 * address table), all released by fmoe_cache_destroy; no device memory.
 * FMOE_ERR_WORKSPACE if n_slots < 1 or the buffer is too small, FMOE_ERR_ROUTING for
 * n_experts outside 1..FMOE_MAX_EXPERTS; a tiered call returns FMOE_ERR_LAUNCH if
 * the pinned host buffers cannot be allocated.
 * fmoe_cache_plan: the cache's policy step alone (host only, no device work): for
 * n distinct experts of layer `layer`, slot_out[i] is the slot that holds expert
 * experts[i] after the call and miss_out[i] 1 when it had to be (re)filled. A hit
 * refreshes the slot; a miss takes the first empty slot, else the least recently
 * used slot that the call does not need (ties: the lower slot). FMOE_ERR_ROUTING
 * for an expert outside 0..n_experts-1 or a repeated one, FMOE_ERR_WORKSPACE if n
 * exceeds the slots (nothing changes then). It updates the bookkeeping as a tiered
 * call does but copies nothing, so a later tiered call would take the planned
 * experts as resident: it is for inspecting the policy on a cache that no tiered
 * call uses.
 * fmoe_moe_layer_tiered: fmoe_moe_layer with L->bank in host memory, any n_tokens
 * (the tokens grouped by expert, as fmoe_moe_layer does for several): the router
 * and top-K run on the GPU; the call then synchronises `stream` once to read the
 * routing, plans the batch's distinct experts (ascending id) through the cache,
 * copies the missing blobs from host memory into their slots (on `stream`), and
 * enqueues the experts and the combine, which read the blobs from their slots.
 * Results equal fmoe_moe_layer's for several tokens (one token takes the same
 * grouped kernels here, so it matches fmoe_moe_layer up to rounding). ws >= fmoe_tiered_workspace_bytes(L, n_tokens);
 * the batch's distinct experts must fit the slots (FMOE_ERR_WORKSPACE, found after
 * the routing: the routing outputs are then written, nothing else). Calls on one
 * cache must be serialised on one stream. Otherwise the arguments and errors of
 * fmoe_moe_layer; FMOE_ERR_SHAPE if L does not match the cache's shape. */
typedef struct fmoe_cache fmoe_cache;
size_t fmoe_cache_device_bytes(int bits, int hidden, int inter, int group, int n_experts, int n_slots);
fmoe_status fmoe_cache_create(int bits, int hidden, int inter, int group, int n_experts, int n_slots,
                              void *device_buf, size_t device_bytes, fmoe_cache **out);
void fmoe_cache_destroy(fmoe_cache *c);
/* Counters since creation: expert lookups, hits, misses, bytes copied from host memory. */
fmoe_status fmoe_cache_get_stats(const fmoe_cache *c, int64_t *lookups, int64_t *hits, int64_t *misses,
                                 int64_t *bytes_copied);
fmoe_status fmoe_cache_plan(fmoe_cache *c, int layer, const int32_t *experts, int n, int32_t *slot_out,
                            int32_t *miss_out);
size_t fmoe_tiered_workspace_bytes(const fmoe_layer *L, int n_tokens);
fmoe_status fmoe_moe_layer_tiered(fmoe_cache *c, int layer, const fmoe_layer *L, int n_tokens, const float *x,
                                  const float *residual, float *out, int32_t *topk_idx, float *topk_w, void *ws,
                                  size_t ws_bytes, void *stream);
/* fmoe_moe_layer_tiered_device: the same layer and the same policy, run on the GPU,
 * with no host synchronisation (it can be captured in a graph). After the router and
 * top-K, one kernel plans the call's distinct experts (ascending id) through the
 * cache's state, which lives in the cache's device buffer, writes the chosen
 * experts' slot addresses and the list of misses; a second kernel copies each
 * missing blob from L->bank, read directly over the bus (L->bank must be pinned host
 * memory the device can address: hipHostMalloc or a pinned torch tensor); then the
 * experts and the combine, as fmoe_moe_layer_tiered for several tokens, and with the
 * one-token kernels of fmoe_moe_layer for one token (the routed blobs read through the
 * cache's table). For the same sequence of calls the slots, counters and routing equal
 * the host policy's, the results too for several tokens (to rounding for one token,
 * where the host-planned call takes the grouped kernels). A cache is driven by one
 * policy: FMOE_ERR_SHAPE if fmoe_cache_plan or fmoe_moe_layer_tiered used it before
 * (and they return FMOE_ERR_SHAPE on a cache this call used). The first such call on
 * a cache initialises its device state (every slot empty) on `stream` and must not be
 * captured (FMOE_ERR_WORKSPACE if `stream` is capturing then); later calls may be.
 * fmoe_cache_get_stats on such a cache synchronises the device and reads the counters
 * back (call it outside graph capture). FMOE_ERR_WORKSPACE if n_slots exceeds 65536 or is below
 * min(n_tokens * top_k, n_experts) (every call's experts must fit; checked on the host,
 * before anything is enqueued); FMOE_ERR_LAUNCH if L->bank is not device-addressable
 * host memory. Otherwise the arguments and errors of fmoe_moe_layer_tiered. */
fmoe_status fmoe_moe_layer_tiered_device(fmoe_cache *c, int layer, const fmoe_layer *L, int n_tokens,
                                         const float *x, const float *residual, float *out, int32_t *topk_idx,
                                         float *topk_w, void *ws, size_t ws_bytes, void *stream);

/* RMS scaling without a learned weight, two stages (sum of squares, then apply)
 * ([P2] "Metal-Compute-Shader": RMS normalization, two-stage):
 *   x_t = h_t / sqrt(sum_i h_t[i]^2 / hidden + eps). h, x: device fp32 [n_tokens][hidden];
 * x may equal h. */
fmoe_status fmoe_rms_scale(const float *h, float *x, int n_tokens, int hidden, float eps, void *stream);

/* A stack of MoE layers with RMS scaling between them, all enqueued without a host
 * synchronisation ([P2] "Verzoegerte GPU-Experten-Berechnung": the expert forward,
 * combine and norm run on the GPU and feed the next layer directly):
 *   h_0 = h0;  for l: x_l = rms_scale(h_l, eps); h_{l+1} = moe_layer(layers[l], x_l, residual = h_l)
 * h0, h_out: device fp32 [n_tokens][hidden] (h_out may equal h0). h_all: device fp32
 * [n_layers][n_tokens][hidden] receiving every h_{l+1}, or NULL. topk_idx / topk_w: device
 * [n_layers][n_tokens][top_k], or NULL. None of h0 (h_out), h_all, topk_idx, topk_w and ws
 * may overlap another (FMOE_ERR_ALIAS), except h_out == h0. Every layer must share hidden, inter, bits, group,
 * top_k and n_experts with layers[0]. ws >= fmoe_stack_workspace_bytes(&layers[0], n_tokens). */
fmoe_status fmoe_moe_stack(const fmoe_layer *layers, int n_layers, int n_tokens, const float *h0,
                           float *h_out, float *h_all, int32_t *topk_idx, float *topk_w, float eps,
                           void *ws, size_t ws_bytes, void *stream);

/* Diagnostic form of fmoe_moe_stack (no h_all or routing outputs): the kernels of
 * layer trace_layer stamp the device clock (100 MHz, the same counter in every
 * workgroup) into trace, a device uint64 array [3][FMOE_TRACE_BLOCKS][FMOE_TRACE_SLOTS]
 * owned and zeroed by the caller. Entry [k][b][s] is stamp s of workgroup b of kernel k.
 * One token (n_tokens == 1): kernel 0 router and shared-expert gate, 1 routing + routed
 * and shared-expert gate/up, 2 routed and shared-expert down + combine; stamp 0 start;
 * 1 its inputs in LDS (x; for kernel 2 the routing and h); 2 (kernel 1, routed
 * workgroups) the routing known; 3 end of its first wavefront.
 * Several tokens (the grouped layer): kernel 0 router + token preparation (stamps 0
 * start, 3 end), 1 the persistent gate/up kernel (0 start; 1 the routing derived, when
 * the workgroup meets a routed item; 2 + i end of its item i for i < 5; 7 end), 2 the
 * down kernel (0 start, 3 end; workgroups past the last token block stamp nothing);
 * the routing and combine kernels are not stamped. Stamps not taken stay 0; workgroups from FMOE_TRACE_BLOCKS on are not
 * recorded. Results equal fmoe_moe_stack's. FMOE_ERR_NULL if trace is NULL,
 * FMOE_ERR_BATCH unless 0 <= trace_layer < n_layers, FMOE_ERR_ALIAS if trace overlaps
 * ws; otherwise the arguments and errors of fmoe_moe_stack. */
#define FMOE_TRACE_BLOCKS 4096
#define FMOE_TRACE_SLOTS 8
fmoe_status fmoe_moe_stack_trace(const fmoe_layer *layers, int n_layers, int n_tokens, const float *h0,
                                 float *h_out, float eps, void *ws, size_t ws_bytes, uint64_t *trace,
                                 int trace_layer, void *stream);

/* Measurement aid, not a step of the method: the HBM read rate this GPU reaches, to
 * report beside the nominal peak. Streams the bytes bytes of buf (device, 16-B
 * aligned, bytes a multiple of 16) with 16-byte non-temporal loads, several in flight
 * per thread, and folds the XOR of all its 32-bit words into *out (device uint32,
 * 4-B aligned): *out ^= w_0 ^ w_1 ^ ... (atomically, so calls accumulate). bytes == 0
 * launches one workgroup that reads nothing (an empty kernel, for timing launch gaps)
 * and leaves *out unchanged. FMOE_ERR_NULL if out is NULL, or buf is NULL with
 * bytes > 0; FMOE_ERR_ALIGN for a misaligned buf or out or bytes not a multiple of 16;
 * FMOE_ERR_ALIAS if out lies inside the buffer. */
fmoe_status fmoe_read_xor(const void *buf, size_t bytes, uint32_t *out, void *stream);

/* Human-readable text of a status (static storage). */
const char *fmoe_status_string(fmoe_status s);

/* Library version as major*10000 + minor*100 + patch. */
int fmoe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FMOE_H_ */
