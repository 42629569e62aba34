// api.cpp -- the extern "C" entry points of libfmoe (include/fmoe.h): argument
// validation on the host, workspace carving, and launch sequencing. No device
// memory is allocated, no stream is synchronised, and no exception escapes.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include "../../include/fmoe.h"
#include "forms.h"
#include "kernels.h"
#include "layout.h"
#include "pack.h"

using namespace fmoe;

namespace {

bool al16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool al256(const void *p) { return ((uintptr_t)p & 255u) == 0; }
bool overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + nb && b0 < a0 + na;
}
hipStream_t as_stream(void *s) { return (hipStream_t)s; }

fmoe_status check_qmat(const fmoe_qmat *W, int want_bits) {
  if (!W || !W->blob) return FMOE_ERR_NULL;
  if (want_bits && W->bits != want_bits) return FMOE_ERR_BITS;
  if (!bits_ok(W->bits)) return FMOE_ERR_BITS;
  if (W->group != kGroup || !cols_ok(W->cols) || W->rows < 1) return FMOE_ERR_SHAPE;
  if (!al256(W->blob)) return FMOE_ERR_ALIGN;
  return FMOE_OK;
}

fmoe_status check_expert_shape(int bits, int hidden, int inter, int group) {
  if (!bits_ok(bits)) return FMOE_ERR_BITS;
  if (group != kGroup || !cols_ok(hidden) || !cols_ok(inter)) return FMOE_ERR_SHAPE;
  return FMOE_OK;
}

fmoe_status check_layer(const fmoe_layer *L) {
  if (!L || !L->router || !L->bank) return FMOE_ERR_NULL;
  if (L->shared && !L->shared_gate) return FMOE_ERR_NULL;
  fmoe_status st = check_expert_shape(L->bits, L->hidden, L->inter, L->group);
  if (st != FMOE_OK) return st;
  if (L->n_experts < 1 || L->n_experts > kMaxExperts || L->top_k < 1 || L->top_k > kMaxTopK ||
      L->top_k > L->n_experts)
    return FMOE_ERR_ROUTING;
  if (!al16(L->router) || !al256(L->bank) || (L->shared && (!al256(L->shared) || !al16(L->shared_gate))))
    return FMOE_ERR_ALIGN;
  return FMOE_OK;
}

bool same_shape(const fmoe_layer *a, const fmoe_layer *b) {
  return a->n_experts == b->n_experts && a->top_k == b->top_k && a->hidden == b->hidden &&
         a->inter == b->inter && a->bits == b->bits && a->group == b->group &&
         (a->shared == nullptr) == (b->shared == nullptr);
}

fmoe_status matvec_common(const fmoe_qmat *W, const float *x, float *y, void *stream, int bits) {
  fmoe_status st = check_qmat(W, bits);
  if (st != FMOE_OK) return st;
  if (!x || !y) return FMOE_ERR_NULL;
  if (!al16(x) || !al16(y)) return FMOE_ERR_ALIGN;
  if (overlap(x, sizeof(float) * (size_t)W->cols, y, sizeof(float) * (size_t)W->rows)) return FMOE_ERR_ALIAS;
  hipError_t e = launch_qmatvec(W->bits, (const uint8_t *)W->blob, W->rows, W->cols, x, y, as_stream(stream));
  return e == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
}

// Enqueue one layer for n_tokens tokens (arguments already validated): the
// one-token kernels for a single token, the grouped kernels for several.
// rms_eps >= 0: the layer input is rms_scale(x, rms_eps), computed inside the layer's kernels.
// trace: device-clock stamps of the one-token kernels (layout in fmoe.h), or null.
fmoe_status layer_enqueue(const fmoe_layer *L, int B, const float *x, float rms_eps, const float *residual,
                          float *out, int32_t *topk_idx, float *topk_w, uint8_t *ws, hipStream_t s,
                          int phases = 7, uint64_t *trace = nullptr) {
  const LayerWs w = layer_ws(B, L->n_experts, L->top_k, L->hidden, L->inter);
  const int H = L->hidden, I = L->inter, E = L->n_experts, K = L->top_k;
  if (B > 1) {
    GroupArgs g{};
    g.router = L->router;
    g.gvec = L->shared ? L->shared_gate : nullptr;
    g.bank = (const uint8_t *)L->bank;
    g.shared = (const uint8_t *)L->shared;
    g.stride = expert_bytes(L->bits, H, I);
    g.gu_bytes = gateup_bytes(L->bits, H, I);
    g.E = E;
    g.K = K;
    g.H = H;
    g.I = I;
    g.B = B;
    g.bits = L->bits;
    g.x = x;
    g.rms_eps = rms_eps;
    g.residual = residual;
    g.out = out;
    g.out_idx = topk_idx;
    g.out_w = topk_w;
    g.logits = (float *)(ws + w.logits);
    g.sigma = (float *)(ws + w.sigma);
    g.gdot = (float *)(ws + w.gdot);
    g.idx = (int32_t *)(ws + w.topk_idx);
    g.w = (float *)(ws + w.topk_w);
    g.xq = (uint8_t *)(ws + w.xq);
    g.xsum = (float *)(ws + w.xsum);
    g.xinv = (float *)(ws + w.xinv);
    g.hq = (uint8_t *)(ws + w.hq);
    g.hsum = (float *)(ws + w.hsum);
    g.d_shared = (float *)(ws + w.d_shared);
    g.partial = (float *)(ws + w.partial);
    g.groups = (int32_t *)(ws + w.groups);
    return launch_group(g, s, phases) == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
  }
  for (int t = 0; t < B; ++t) {
    LayerArgs a{};
    a.router = L->router;
    a.shared_gate = L->shared_gate;
    a.bank = (const uint8_t *)L->bank;
    a.shared = (const uint8_t *)L->shared;
    a.E = E;
    a.K = K;
    a.H = H;
    a.I = I;
    a.bits = L->bits;
    a.expert_stride = expert_bytes(L->bits, H, I);
    a.gateup_bytes = gateup_bytes(L->bits, H, I);
    a.x = x + (size_t)t * H;
    a.rms_eps = rms_eps;
    a.residual = residual + (size_t)t * H;
    a.out = out + (size_t)t * H;
    a.topk_idx_out = topk_idx ? topk_idx + (size_t)t * K : nullptr;
    a.topk_w_out = topk_w ? topk_w + (size_t)t * K : nullptr;
    a.logits = (float *)(ws + w.logits) + (size_t)t * logit_stride(E);
    a.sigma = (float *)(ws + w.sigma) + t;
    a.ws_idx = (int32_t *)(ws + w.topk_idx) + (size_t)t * K;
    a.ws_w = (float *)(ws + w.topk_w) + (size_t)t * K;
    a.h_shared = (float *)(ws + w.h_shared) + (size_t)t * I;
    a.h_routed = (float *)(ws + w.h_routed) + (size_t)t * K * I;
    a.d_shared = (float *)(ws + w.d_shared) + (size_t)t * H;
    a.xdig = (uint32_t *)(ws + w.xdig);
    a.trace = trace;
    if (launch_layer(a, s, phases) != hipSuccess) return FMOE_ERR_LAUNCH;
  }
  return FMOE_OK;
}

}  // namespace

extern "C" {

size_t fmoe_qmat_bytes(int bits, int rows, int cols, int group) {
  if (!bits_ok(bits) || group != kGroup || !cols_ok(cols) || rows < 1) return 0;
  return qmat_bytes(bits, rows, cols);
}

size_t fmoe_expert_bytes(int bits, int hidden, int inter, int group) {
  if (check_expert_shape(bits, hidden, inter, group) != FMOE_OK) return 0;
  return expert_bytes(bits, hidden, inter);
}

size_t fmoe_expert_workspace_bytes(const fmoe_expert *E) {
  if (!E || check_expert_shape(E->bits, E->hidden, E->inter, E->group) != FMOE_OK) return 0;
  return round_up(sizeof(float) * (size_t)E->inter, 256);
}

size_t fmoe_workspace_bytes(const fmoe_layer *L, int n_tokens) {
  if (!L || check_expert_shape(L->bits, L->hidden, L->inter, L->group) != FMOE_OK) return 0;
  if (n_tokens < 1 || n_tokens > kMaxTokens || L->top_k < 1 || L->top_k > kMaxTopK || L->n_experts < 1 ||
      L->n_experts > kMaxExperts)
    return 0;
  return layer_ws(n_tokens, L->n_experts, L->top_k, L->hidden, L->inter).total;
}

size_t fmoe_stack_workspace_bytes(const fmoe_layer *L, int n_tokens) {
  if (fmoe_workspace_bytes(L, n_tokens) == 0) return 0;
  return stack_ws(n_tokens, L->n_experts, L->top_k, L->hidden, L->inter).total;
}

fmoe_status fmoe_pack_qmat(int bits, int rows, int cols, int group, const uint8_t *codes, const uint16_t *scale,
                           const uint16_t *bias, void *blob_out) {
  if (!codes || !scale || !bias || !blob_out) return FMOE_ERR_NULL;
  if (!bits_ok(bits)) return FMOE_ERR_BITS;
  if (group != kGroup || !cols_ok(cols) || rows < 1) return FMOE_ERR_SHAPE;
  const size_t total = qmat_bytes(bits, rows, cols), rb = row_bytes(bits, cols);
  uint8_t *blob = (uint8_t *)blob_out;
  memset(blob + (size_t)rows * rb, 0, total - (size_t)rows * rb);
  if (!pack_matrix(bits, rows, cols, codes, scale, bias, blob, rb, 0)) return FMOE_ERR_SHAPE;
  return FMOE_OK;
}

fmoe_status fmoe_unpack_qmat(int bits, int rows, int cols, int group, const void *blob, uint8_t *codes,
                             uint16_t *scale, uint16_t *bias) {
  if (!codes || !scale || !bias || !blob) return FMOE_ERR_NULL;
  if (!bits_ok(bits)) return FMOE_ERR_BITS;
  if (group != kGroup || !cols_ok(cols) || rows < 1) return FMOE_ERR_SHAPE;
  unpack_matrix(bits, rows, cols, (const uint8_t *)blob, row_bytes(bits, cols), 0, codes, scale, bias);
  return FMOE_OK;
}

fmoe_status fmoe_pack_expert(int bits, int hidden, int inter, int group, const uint8_t *const codes[3],
                             const uint16_t *const scale[3], const uint16_t *const bias[3], void *blob_out) {
  if (!codes || !scale || !bias || !blob_out) return FMOE_ERR_NULL;
  for (int i = 0; i < 3; ++i)
    if (!codes[i] || !scale[i] || !bias[i]) return FMOE_ERR_NULL;
  fmoe_status st = check_expert_shape(bits, hidden, inter, group);
  if (st != FMOE_OK) return st;
  uint8_t *blob = (uint8_t *)blob_out;
  const size_t rbh = row_bytes(bits, hidden), rbi = row_bytes(bits, inter);
  const size_t gub = gateup_bytes(bits, hidden, inter), total = expert_bytes(bits, hidden, inter);
  memset(blob + 2 * (size_t)inter * rbh, 0, gub - 2 * (size_t)inter * rbh);
  memset(blob + gub + (size_t)hidden * rbi, 0, total - gub - (size_t)hidden * rbi);
  if (!pack_matrix(bits, inter, hidden, codes[0], scale[0], bias[0], blob, 2 * rbh, 0) ||
      !pack_matrix(bits, inter, hidden, codes[1], scale[1], bias[1], blob, 2 * rbh, rbh) ||
      !pack_matrix(bits, hidden, inter, codes[2], scale[2], bias[2], blob, rbi, gub))
    return FMOE_ERR_SHAPE;
  return FMOE_OK;
}

fmoe_status fmoe_unpack_expert(int bits, int hidden, int inter, int group, const void *blob,
                               uint8_t *const codes[3], uint16_t *const scale[3], uint16_t *const bias[3]) {
  if (!codes || !scale || !bias || !blob) return FMOE_ERR_NULL;
  for (int i = 0; i < 3; ++i)
    if (!codes[i] || !scale[i] || !bias[i]) return FMOE_ERR_NULL;
  fmoe_status st = check_expert_shape(bits, hidden, inter, group);
  if (st != FMOE_OK) return st;
  const uint8_t *b = (const uint8_t *)blob;
  const size_t rbh = row_bytes(bits, hidden), rbi = row_bytes(bits, inter);
  const size_t gub = gateup_bytes(bits, hidden, inter);
  unpack_matrix(bits, inter, hidden, b, 2 * rbh, 0, codes[0], scale[0], bias[0]);
  unpack_matrix(bits, inter, hidden, b, 2 * rbh, rbh, codes[1], scale[1], bias[1]);
  unpack_matrix(bits, hidden, inter, b, rbi, gub, codes[2], scale[2], bias[2]);
  return FMOE_OK;
}

fmoe_status fmoe_pack_qmat_device(int bits, int rows, int cols, int group, const uint8_t *codes,
                                  const uint16_t *scale, const uint16_t *bias, void *blob_out, void *stream) {
  if (!codes || !scale || !bias || !blob_out) return FMOE_ERR_NULL;
  if (!bits_ok(bits)) return FMOE_ERR_BITS;
  if (group != kGroup || !cols_ok(cols) || rows < 1) return FMOE_ERR_SHAPE;
  if (!al16(codes) || !al256(blob_out)) return FMOE_ERR_ALIGN;
  hipError_t e = launch_pack_matrix(bits, rows, cols, codes, scale, bias, (uint8_t *)blob_out,
                                    row_bytes(bits, cols), 0, as_stream(stream));
  return e == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
}

fmoe_status fmoe_pack_expert_device(int bits, int hidden, int inter, int group, const uint8_t *const codes[3],
                                    const uint16_t *const scale[3], const uint16_t *const bias[3],
                                    void *blob_out, void *stream) {
  if (!codes || !scale || !bias || !blob_out) return FMOE_ERR_NULL;
  for (int i = 0; i < 3; ++i)
    if (!codes[i] || !scale[i] || !bias[i]) return FMOE_ERR_NULL;
  fmoe_status st = check_expert_shape(bits, hidden, inter, group);
  if (st != FMOE_OK) return st;
  for (int i = 0; i < 3; ++i)
    if (!al16(codes[i])) return FMOE_ERR_ALIGN;
  if (!al256(blob_out)) return FMOE_ERR_ALIGN;
  uint8_t *blob = (uint8_t *)blob_out;
  const size_t rbh = row_bytes(bits, hidden), rbi = row_bytes(bits, inter);
  const size_t gub = gateup_bytes(bits, hidden, inter);
  hipStream_t s = as_stream(stream);
  if (launch_pack_matrix(bits, inter, hidden, codes[0], scale[0], bias[0], blob, 2 * rbh, 0, s) != hipSuccess ||
      launch_pack_matrix(bits, inter, hidden, codes[1], scale[1], bias[1], blob, 2 * rbh, rbh, s) != hipSuccess ||
      launch_pack_matrix(bits, hidden, inter, codes[2], scale[2], bias[2], blob, rbi, gub, s) != hipSuccess)
    return FMOE_ERR_LAUNCH;
  return FMOE_OK;
}

fmoe_status fmoe_q4_matvec(const fmoe_qmat *W, const float *x, float *y, void *stream) {
  return matvec_common(W, x, y, stream, 4);
}

fmoe_status fmoe_q2_matvec(const fmoe_qmat *W, const float *x, float *y, void *stream) {
  return matvec_common(W, x, y, stream, 2);
}

fmoe_status fmoe_expert_ffn(const fmoe_expert *E, const float *x, float *out, void *ws, size_t ws_bytes,
                            void *stream) {
  if (!E || !E->blob || !x || !out) return FMOE_ERR_NULL;
  fmoe_status st = check_expert_shape(E->bits, E->hidden, E->inter, E->group);
  if (st != FMOE_OK) return st;
  if (!al256(E->blob) || !al16(x) || !al16(out)) return FMOE_ERR_ALIGN;
  const size_t need = fmoe_expert_workspace_bytes(E);
  if (!ws || ws_bytes < need) return FMOE_ERR_WORKSPACE;
  if (!al256(ws)) return FMOE_ERR_ALIGN;
  const size_t xb = sizeof(float) * (size_t)E->hidden;
  if (overlap(x, xb, out, xb) || overlap(out, xb, ws, need) || overlap(x, xb, ws, need)) return FMOE_ERR_ALIAS;
  const uint8_t *blob = (const uint8_t *)E->blob;
  hipStream_t s = as_stream(stream);
  float *h = (float *)ws;
  if (launch_expert_gateup(E->bits, blob, E->hidden, E->inter, x, h, s) != hipSuccess) return FMOE_ERR_LAUNCH;
  if (launch_qmatvec(E->bits, blob + gateup_bytes(E->bits, E->hidden, E->inter), E->hidden, E->inter, h, out, s) !=
      hipSuccess)
    return FMOE_ERR_LAUNCH;
  return FMOE_OK;
}

fmoe_status fmoe_moe_layer(const fmoe_layer *L, int n_tokens, const float *x, const float *residual, float *out,
                           int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  return fmoe_moe_layer_phases(L, n_tokens, x, residual, out, topk_idx, topk_w, ws, ws_bytes, 7, stream);
}

fmoe_status fmoe_moe_layer_phases(const fmoe_layer *L, int n_tokens, const float *x, const float *residual,
                                  float *out, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                                  int phases, void *stream) {
  if (phases < 1 || phases > 7) return FMOE_ERR_BATCH;
  fmoe_status st = check_layer(L);
  if (st != FMOE_OK) return st;
  if (!x || !residual || !out) return FMOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > kMaxTokens) return FMOE_ERR_BATCH;
  if (!al16(x) || !al16(residual) || !al16(out) || (topk_idx && !al16(topk_idx)) || (topk_w && !al16(topk_w)))
    return FMOE_ERR_ALIGN;
  const size_t need = fmoe_workspace_bytes(L, n_tokens);
  if (!ws || ws_bytes < need) return FMOE_ERR_WORKSPACE;
  if (!al256(ws)) return FMOE_ERR_ALIGN;
  const size_t ab = sizeof(float) * (size_t)n_tokens * L->hidden;
  const size_t kb = sizeof(float) * (size_t)n_tokens * L->top_k;
  if (overlap(out, ab, x, ab) || overlap(out, ab, ws, need) || overlap(x, ab, ws, need) ||
      overlap(residual, ab, ws, need) || overlap(topk_idx, kb, ws, need) || overlap(topk_w, kb, ws, need) ||
      overlap(topk_idx, kb, out, ab) || overlap(topk_w, kb, out, ab) || overlap(topk_idx, kb, topk_w, kb))
    return FMOE_ERR_ALIAS;
  return layer_enqueue(L, n_tokens, x, -1.f, residual, out, topk_idx, topk_w, (uint8_t *)ws, as_stream(stream),
                       phases);
}

fmoe_status fmoe_rms_scale(const float *h, float *x, int n_tokens, int hidden, float eps, void *stream) {
  if (!h || !x) return FMOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > kMaxTokens) return FMOE_ERR_BATCH;
  if (hidden < 1) return FMOE_ERR_SHAPE;
  if (!al16(h) || !al16(x)) return FMOE_ERR_ALIGN;
  const size_t b = sizeof(float) * (size_t)n_tokens * hidden;
  if (h != x && overlap(h, b, x, b)) return FMOE_ERR_ALIAS;
  return launch_rms(h, x, n_tokens, hidden, eps, as_stream(stream)) == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
}

static_assert(FMOE_TRACE_BLOCKS == kTraceBlocks && FMOE_TRACE_SLOTS == kTraceSlots, "the kernels' stamp layout");

// fmoe_moe_stack, with the stamps of layer trace_layer's kernels in trace (null: none)
static fmoe_status stack_enqueue(const fmoe_layer *layers, int n_layers, int n_tokens, const float *h0,
                                 float *h_out, float *h_all, int32_t *topk_idx, float *topk_w, float eps, void *ws,
                                 size_t ws_bytes, void *stream, uint64_t *trace, int trace_layer) {
  if (!layers) return FMOE_ERR_NULL;
  if (n_layers < 1) return FMOE_ERR_BATCH;
  for (int l = 0; l < n_layers; ++l) {
    fmoe_status st = check_layer(&layers[l]);
    if (st != FMOE_OK) return st;
    if (!same_shape(&layers[0], &layers[l])) return FMOE_ERR_SHAPE;
  }
  if (!h0 || !h_out) return FMOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > kMaxTokens) return FMOE_ERR_BATCH;
  if (!al16(h0) || !al16(h_out) || (h_all && !al16(h_all)) || (topk_idx && !al16(topk_idx)) ||
      (topk_w && !al16(topk_w)))
    return FMOE_ERR_ALIGN;
  const fmoe_layer *L0 = &layers[0];
  const size_t need = fmoe_stack_workspace_bytes(L0, n_tokens);
  if (!ws || ws_bytes < need) return FMOE_ERR_WORKSPACE;
  if (!al256(ws)) return FMOE_ERR_ALIGN;
  const int H = L0->hidden, K = L0->top_k, B = n_tokens;
  const size_t hb = sizeof(float) * (size_t)B * H;
  const size_t kb = sizeof(float) * (size_t)n_layers * B * K;
  if (overlap(h0, hb, ws, need) || overlap(h_out, hb, ws, need) || overlap(h_all, hb * n_layers, ws, need) ||
      overlap(h_all, hb * n_layers, h0, hb) || overlap(h_all, hb * n_layers, h_out, hb) ||
      overlap(topk_idx, kb, ws, need) || overlap(topk_w, kb, ws, need) || overlap(topk_idx, kb, topk_w, kb))
    return FMOE_ERR_ALIAS;
  const StackWs sw = stack_ws(B, L0->n_experts, K, H, L0->inter);
  uint8_t *w = (uint8_t *)ws;
  float *ping[2] = {(float *)(w + sw.ha), (float *)(w + sw.hb)};
  hipStream_t s = as_stream(stream);
  const float *cur = h0;
  for (int l = 0; l < n_layers; ++l) {
    // x_l = rms_scale(h_l) is formed inside the layer's kernels from h_l itself
    float *nxt;
    if (h_all)
      nxt = h_all + (size_t)l * B * H;
    else if (l == n_layers - 1)
      nxt = h_out;
    else
      nxt = ping[l & 1];
    fmoe_status st = layer_enqueue(&layers[l], B, cur, eps, cur, nxt, topk_idx ? topk_idx + (size_t)l * B * K : nullptr,
                                   topk_w ? topk_w + (size_t)l * B * K : nullptr, w + sw.layer, s, 7,
                                   l == trace_layer ? trace : nullptr);
    if (st != FMOE_OK) return st;
    cur = nxt;
  }
  if (h_all && hipMemcpyAsync(h_out, cur, hb, hipMemcpyDeviceToDevice, s) != hipSuccess) return FMOE_ERR_LAUNCH;
  return FMOE_OK;
}

fmoe_status fmoe_moe_stack(const fmoe_layer *layers, int n_layers, int n_tokens, const float *h0, float *h_out,
                           float *h_all, int32_t *topk_idx, float *topk_w, float eps, void *ws, size_t ws_bytes,
                           void *stream) {
  return stack_enqueue(layers, n_layers, n_tokens, h0, h_out, h_all, topk_idx, topk_w, eps, ws, ws_bytes, stream,
                       nullptr, -1);
}

fmoe_status fmoe_moe_stack_trace(const fmoe_layer *layers, int n_layers, int n_tokens, const float *h0,
                                 float *h_out, float eps, void *ws, size_t ws_bytes, uint64_t *trace,
                                 int trace_layer, void *stream) {
  if (!trace) return FMOE_ERR_NULL;
  if (n_tokens != 1 || trace_layer < 0 || trace_layer >= n_layers) return FMOE_ERR_BATCH;
  if ((uintptr_t)trace % 8) return FMOE_ERR_ALIGN;
  if (ws && overlap(trace, sizeof(uint64_t) * 3 * FMOE_TRACE_BLOCKS * FMOE_TRACE_SLOTS, ws, ws_bytes))
    return FMOE_ERR_ALIAS;
  return stack_enqueue(layers, n_layers, n_tokens, h0, h_out, nullptr, nullptr, nullptr, eps, ws, ws_bytes, stream,
                       trace, trace_layer);
}

fmoe_status fmoe_qmatvec_form(const fmoe_qmat *W, const float *x, float *y, int form, void *stream) {
  if (!W) return FMOE_ERR_NULL;
  if (form < 0 || form >= kForms) return FMOE_ERR_SHAPE;
  fmoe_status st = check_qmat(W, W->bits);
  if (st != FMOE_OK) return st;
  if (!x || !y) return FMOE_ERR_NULL;
  if (!al16(x) || !al16(y)) return FMOE_ERR_ALIGN;
  if (overlap(x, sizeof(float) * (size_t)W->cols, y, sizeof(float) * (size_t)W->rows)) return FMOE_ERR_ALIAS;
  hipError_t e = launch_qmatvec_form(W->bits, form, (const uint8_t *)W->blob, W->rows, W->cols, x, y, as_stream(stream));
  return e == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
}

fmoe_status fmoe_read_xor(const void *buf, size_t bytes, uint32_t *out, void *stream) {
  if (!out || (bytes > 0 && !buf)) return FMOE_ERR_NULL;
  if (bytes % 16 || (bytes > 0 && !al16(buf)) || (uintptr_t)out % 4) return FMOE_ERR_ALIGN;
  if (bytes > 0 && overlap(out, sizeof(uint32_t), buf, bytes)) return FMOE_ERR_ALIAS;
  return launch_read_xor(buf, bytes, out, as_stream(stream)) == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
}

const char *fmoe_status_string(fmoe_status s) {
  switch (s) {
    case FMOE_OK: return "ok";
    case FMOE_ERR_NULL: return "a required pointer is NULL";
    case FMOE_ERR_SHAPE: return "unsupported or inconsistent shape, group size or code value";
    case FMOE_ERR_ALIGN: return "misaligned pointer (fp32 arrays need 16 B, blobs and workspaces 256 B)";
    case FMOE_ERR_BITS: return "unsupported or mismatched bit width";
    case FMOE_ERR_ROUTING: return "top_k or n_experts out of range";
    case FMOE_ERR_BATCH: return "n_tokens or n_layers out of range";
    case FMOE_ERR_WORKSPACE: return "workspace missing or too small";
    case FMOE_ERR_LAUNCH: return "the HIP runtime refused a kernel launch";
    case FMOE_ERR_ALIAS: return "an input overlaps an output or the workspace";
  }
  return "unknown status";
}

int fmoe_version(void) { return 100; }

}  // extern "C"
