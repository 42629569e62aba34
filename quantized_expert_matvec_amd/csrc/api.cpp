// api.cpp -- the extern "C" entry points of libfmoe (include/fmoe.h): argument
// validation on the host, workspace carving, and launch sequencing. No device
// memory is allocated, no stream is synchronised, and no exception escapes.
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <unordered_map>
#include <vector>

#include "../../include/fmoe.h"
#include "expert_cache.h"
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

// The arguments of the grouped kernels for one layer (workspace carved as layer_ws(grouped)).
GroupArgs group_args(const fmoe_layer *L, int B, const float *x, float rms_eps, const float *residual, float *out,
                     int32_t *topk_idx, float *topk_w, uint8_t *ws) {
  const LayerWs w = layer_ws(B, L->n_experts, L->top_k, L->hidden, L->inter, true);
  const int H = L->hidden, I = L->inter, E = L->n_experts, K = L->top_k;
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
  g.logit_parts = router_parts(E, B, H);
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
  g.expert_ptr = nullptr;
  return g;
}

// Enqueue one layer for n_tokens tokens (arguments already validated): the
// one-token kernels for a single token, the grouped kernels for several.
// rms_eps >= 0: the layer input is rms_scale(x, rms_eps), computed inside the layer's kernels.
// trace: device-clock stamps of the layer's kernels (layout in fmoe.h), or null.
// form >= 0 (one token): the dequant-form build of the layer kernels (launch_layer_form),
// with x in fp32 in the workspace's d_shared region, which the one-token kernels leave unused.
// The one-token kernels' arguments for token x of layer L (workspace ws laid out by
// layer_ws for one token).
LayerArgs one_token_args(const fmoe_layer *L, const float *x, float rms_eps, const float *residual, float *out,
                         int32_t *topk_idx, float *topk_w, uint8_t *ws) {
  const LayerWs w = layer_ws(1, L->n_experts, L->top_k, L->hidden, L->inter, false);
  const int H = L->hidden, I = L->inter;
  LayerArgs a{};
  a.router = L->router;
  a.shared_gate = L->shared_gate;
  a.bank = (const uint8_t *)L->bank;
  a.shared = (const uint8_t *)L->shared;
  a.E = L->n_experts;
  a.K = L->top_k;
  a.H = H;
  a.I = I;
  a.bits = L->bits;
  a.expert_stride = expert_bytes(L->bits, H, I);
  a.gateup_bytes = gateup_bytes(L->bits, H, I);
  a.x = x;
  a.rms_eps = rms_eps;
  a.residual = residual;
  a.out = out;
  a.topk_idx_out = topk_idx;
  a.topk_w_out = topk_w;
  a.logits = (float *)(ws + w.logits);
  a.sigma = (float *)(ws + w.sigma);
  a.ws_idx = (int32_t *)(ws + w.topk_idx);
  a.ws_w = (float *)(ws + w.topk_w);
  a.h_shared = (float *)(ws + w.h_shared);
  a.h_routed = (float *)(ws + w.h_routed);
  a.d_shared = (float *)(ws + w.d_shared);
  a.xdig = (uint32_t *)(ws + w.xdig);
  return a;
}

fmoe_status layer_enqueue(const fmoe_layer *L, int B, const float *x, float rms_eps, const float *residual,
                          float *out, int32_t *topk_idx, float *topk_w, uint8_t *ws, hipStream_t s,
                          int phases = 7, uint64_t *trace = nullptr, int form = -1) {
  if (B > 1) {
    GroupArgs g = group_args(L, B, x, rms_eps, residual, out, topk_idx, topk_w, ws);
    g.trace = trace;
    return launch_group(g, s, phases) == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
  }
  LayerArgs a = one_token_args(L, x, rms_eps, residual, out, topk_idx, topk_w, ws);
  a.trace = trace;
  if (form >= 0) {
    a.xs = a.d_shared;  // (the workspace's d_shared region holds x in fp32 for the form builds)
    return launch_layer_form(a, form, s) == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
  }
  return launch_layer(a, s, phases) == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
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
  return layer_ws(n_tokens, L->n_experts, L->top_k, L->hidden, L->inter, n_tokens > 1).total;
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

fmoe_status fmoe_expert_ffn_form(const fmoe_expert *E, const float *x, float *out, void *ws, size_t ws_bytes, int form,
                                 void *stream) {
  if (!E || !E->blob || !x || !out) return FMOE_ERR_NULL;
  if (form < 0 || form >= kForms) return FMOE_ERR_SHAPE;
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
  if (launch_expert_gateup_form(E->bits, form, blob, E->hidden, E->inter, x, h, s) != hipSuccess)
    return FMOE_ERR_LAUNCH;
  if (launch_qmatvec_form(E->bits, form, blob + gateup_bytes(E->bits, E->hidden, E->inter), E->hidden, E->inter, h, out,
                          s) != hipSuccess)
    return FMOE_ERR_LAUNCH;
  return FMOE_OK;
}

fmoe_status fmoe_moe_layer(const fmoe_layer *L, int n_tokens, const float *x, const float *residual, float *out,
                           int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  return fmoe_moe_layer_phases(L, n_tokens, x, residual, out, topk_idx, topk_w, ws, ws_bytes, 7, stream);
}

// the checks of fmoe_moe_layer (status FMOE_OK: the call may be enqueued)
static fmoe_status check_layer_call(const fmoe_layer *L, int n_tokens, const float *x, const float *residual,
                                    float *out, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes) {
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
      overlap(topk_idx, kb, out, ab) || overlap(topk_w, kb, out, ab) || overlap(topk_idx, kb, topk_w, kb) ||
      (residual != out && overlap(residual, ab, out, ab)) || overlap(topk_idx, kb, residual, ab) ||
      overlap(topk_w, kb, residual, ab) || overlap(topk_idx, kb, x, ab) || overlap(topk_w, kb, x, ab))
    return FMOE_ERR_ALIAS;
  return FMOE_OK;
}

fmoe_status fmoe_moe_layer_phases(const fmoe_layer *L, int n_tokens, const float *x, const float *residual,
                                  float *out, int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes,
                                  int phases, void *stream) {
  if (phases < 1 || phases > 7) return FMOE_ERR_BATCH;
  const fmoe_status st = check_layer_call(L, n_tokens, x, residual, out, topk_idx, topk_w, ws, ws_bytes);
  if (st != FMOE_OK) return st;
  return layer_enqueue(L, n_tokens, x, -1.f, residual, out, topk_idx, topk_w, (uint8_t *)ws, as_stream(stream),
                       phases);
}

fmoe_status fmoe_moe_layer_form(const fmoe_layer *L, const float *x, const float *residual, float *out,
                                int32_t *topk_idx, float *topk_w, void *ws, size_t ws_bytes, int form, void *stream) {
  if (form < 0 || form >= kForms) return FMOE_ERR_SHAPE;
  const fmoe_status st = check_layer_call(L, 1, x, residual, out, topk_idx, topk_w, ws, ws_bytes);
  if (st != FMOE_OK) return st;
  if (L->hidden != 4096 || L->inter != 1024 || L->n_experts > 512) return FMOE_ERR_SHAPE;
  if (L->top_k != 4) return FMOE_ERR_ROUTING;
  return layer_enqueue(L, 1, x, -1.f, residual, out, topk_idx, topk_w, (uint8_t *)ws, as_stream(stream), 7, nullptr,
                       form);
}

fmoe_status fmoe_moe_layer_noalloc(const fmoe_layer *L, int n_tokens, const float *x, const float *residual,
                                   float *out, int32_t *topk_idx, float *topk_w, void *stream) {
  fmoe_status st = check_layer(L);
  if (st != FMOE_OK) return st;
  if (!x || !residual || !out) return FMOE_ERR_NULL;
  if (n_tokens < 1 || n_tokens > kMaxTokens) return FMOE_ERR_BATCH;
  const size_t need = fmoe_workspace_bytes(L, n_tokens);
  if (need > kScratchBytes) return FMOE_ERR_WORKSPACE;
  void *ws = nullptr;
  if (scratch_device_ptr(&ws) != hipSuccess) return FMOE_ERR_LAUNCH;
  // the full validation of fmoe_moe_layer, with the static workspace as ws
  return fmoe_moe_layer_phases(L, n_tokens, x, residual, out, topk_idx, topk_w, ws, kScratchBytes, 7, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ host-memory expert tier

// The cache: n_slots expert blobs and a table of expert blob addresses in the
// caller's device buffer; the slot bookkeeping, and pinned host staging for the
// routing read-back and the address table, on the host.
struct fmoe_cache {
  int bits, hidden, inter, n_experts, n_slots;
  size_t stride;                 // bytes per expert blob
  uint8_t *slots;                // device: n_slots blobs
  const uint8_t **table;         // device: [n_experts] blob addresses
  const uint8_t **table_host;    // pinned host mirror of table
  int32_t *idx_host;             // pinned host: routing read-back [kMaxTokens * kMaxTopK]
  fmoe::ExpertCache lru;
  int64_t lookups = 0, bytes = 0;
  // where the policy runs: 0 not yet, 1 on the host (lru), 2 on the device (the state below)
  int mode = 0;
  bool dev_init = false;         // the device state initialised (by the first device-policy call)
  fmoe::TierHdr *hdr;            // device: counters and the current call's copy count
  int64_t *key;                  // device: [n_slots] (layer, expert) held, -1 empty
  uint64_t *last;                // device: [n_slots] last use
  int32_t *jobs;                 // device: [2 * kMaxExperts] the current call's copies
  std::unordered_map<const void *, const void *> bank_dev;  // host bank -> its device-visible address
  fmoe_cache(int n) : lru(n) {}
};

namespace {
size_t cache_table_offset(int bits, int hidden, int inter, int n_slots) {
  return round_up((size_t)n_slots * expert_bytes(bits, hidden, inter), 256);
}
// the device policy's state, after the table: header, keys, last uses, copy jobs
struct CacheState {
  size_t hdr, key, last, jobs, end;
};
CacheState cache_state(int bits, int hidden, int inter, int n_experts, int n_slots) {
  CacheState c;
  c.hdr = cache_table_offset(bits, hidden, inter, n_slots) + round_up(sizeof(void *) * (size_t)n_experts, 256);
  c.key = c.hdr + round_up(sizeof(fmoe::TierHdr), 256);
  c.last = c.key + round_up(sizeof(int64_t) * (size_t)n_slots, 256);
  c.jobs = c.last + round_up(sizeof(uint64_t) * (size_t)n_slots, 256);
  c.end = c.jobs + round_up(sizeof(int32_t) * 2 * kMaxExperts, 256);
  return c;
}
}  // namespace

extern "C" {

size_t fmoe_cache_device_bytes(int bits, int hidden, int inter, int group, int n_experts, int n_slots) {
  if (check_expert_shape(bits, hidden, inter, group) != FMOE_OK || n_slots < 1 || n_experts < 1 ||
      n_experts > kMaxExperts)
    return 0;
  return cache_state(bits, hidden, inter, n_experts, n_slots).end;
}

fmoe_status fmoe_cache_create(int bits, int hidden, int inter, int group, int n_experts, int n_slots,
                              void *device_buf, size_t device_bytes, fmoe_cache **out) {
  if (!out || !device_buf) return FMOE_ERR_NULL;
  *out = nullptr;
  fmoe_status st = check_expert_shape(bits, hidden, inter, group);
  if (st != FMOE_OK) return st;
  if (n_experts < 1 || n_experts > kMaxExperts) return FMOE_ERR_ROUTING;
  if (n_slots < 1) return FMOE_ERR_WORKSPACE;
  if (!al256(device_buf)) return FMOE_ERR_ALIGN;
  if (device_bytes < fmoe_cache_device_bytes(bits, hidden, inter, group, n_experts, n_slots))
    return FMOE_ERR_WORKSPACE;
  fmoe_cache *c = new (std::nothrow) fmoe_cache(n_slots);
  if (!c) return FMOE_ERR_WORKSPACE;
  c->bits = bits;
  c->hidden = hidden;
  c->inter = inter;
  c->n_experts = n_experts;
  c->n_slots = n_slots;
  c->stride = expert_bytes(bits, hidden, inter);
  c->slots = (uint8_t *)device_buf;
  c->table = (const uint8_t **)((uint8_t *)device_buf + cache_table_offset(bits, hidden, inter, n_slots));
  c->table_host = nullptr;  // (pinned host buffers: allocated by the first tiered call)
  c->idx_host = nullptr;
  const CacheState cs = cache_state(bits, hidden, inter, n_experts, n_slots);
  uint8_t *b = (uint8_t *)device_buf;
  c->hdr = (fmoe::TierHdr *)(b + cs.hdr);
  c->key = (int64_t *)(b + cs.key);
  c->last = (uint64_t *)(b + cs.last);
  c->jobs = (int32_t *)(b + cs.jobs);
  *out = c;
  return FMOE_OK;
}

void fmoe_cache_destroy(fmoe_cache *c) {
  if (!c) return;
  if (c->table_host) (void)hipHostFree((void *)c->table_host);
  if (c->idx_host) (void)hipHostFree(c->idx_host);
  delete c;
}

fmoe_status fmoe_cache_get_stats(const fmoe_cache *c, int64_t *lookups, int64_t *hits, int64_t *misses,
                                 int64_t *bytes_copied) {
  if (!c) return FMOE_ERR_NULL;
  if (c->mode == 2) {
    fmoe::TierHdr h;
    if (hipDeviceSynchronize() != hipSuccess || hipMemcpy(&h, c->hdr, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess)
      return FMOE_ERR_LAUNCH;
    if (lookups) *lookups = h.lookups;
    if (hits) *hits = h.hits;
    if (misses) *misses = h.misses;
    if (bytes_copied) *bytes_copied = h.bytes;
    return FMOE_OK;
  }
  if (lookups) *lookups = c->lookups;
  if (hits) *hits = c->lru.hits();
  if (misses) *misses = c->lru.misses();
  if (bytes_copied) *bytes_copied = c->bytes;
  return FMOE_OK;
}

fmoe_status fmoe_cache_plan(fmoe_cache *c, int layer, const int32_t *experts, int n, int32_t *slot_out,
                            int32_t *miss_out) {
  if (!c || !experts || !slot_out || !miss_out) return FMOE_ERR_NULL;
  if (c->mode == 2) return FMOE_ERR_SHAPE;  // (the cache's policy runs on the device)
  if (layer < 0 || n < 1) return FMOE_ERR_BATCH;
  std::vector<int32_t> sorted(experts, experts + n);
  std::sort(sorted.begin(), sorted.end());
  for (int i = 0; i < n; ++i)
    if (sorted[i] < 0 || sorted[i] >= c->n_experts || (i > 0 && sorted[i] == sorted[i - 1])) return FMOE_ERR_ROUTING;
  if (n > c->n_slots) return FMOE_ERR_WORKSPACE;
  c->lookups += n;
  c->mode = 1;
  return c->lru.plan(layer, experts, n, slot_out, miss_out) ? FMOE_OK : FMOE_ERR_WORKSPACE;
}

size_t fmoe_tiered_workspace_bytes(const fmoe_layer *L, int n_tokens) {
  if (fmoe_workspace_bytes(L, n_tokens) == 0) return 0;
  const size_t g = layer_ws(n_tokens, L->n_experts, L->top_k, L->hidden, L->inter, true).total;
  // (one token: either kernels' workspace, for the two policies' calls)
  return n_tokens == 1 ? std::max(g, layer_ws(1, L->n_experts, L->top_k, L->hidden, L->inter, false).total) : g;
}

}  // extern "C"

namespace {
// The arguments of a tiered layer call (either policy).
fmoe_status tiered_check(const fmoe_cache *c, int layer, const fmoe_layer *L, int n_tokens, const float *x,
                         const float *residual, const float *out, const int32_t *topk_idx, const float *topk_w,
                         const void *ws, size_t ws_bytes) {
  if (!c) return FMOE_ERR_NULL;
  fmoe_status st = check_layer(L);
  if (st != FMOE_OK) return st;
  if (L->bits != c->bits || L->hidden != c->hidden || L->inter != c->inter || L->n_experts > c->n_experts)
    return FMOE_ERR_SHAPE;
  if (!x || !residual || !out) return FMOE_ERR_NULL;
  if (layer < 0 || n_tokens < 1 || n_tokens > kMaxTokens) return FMOE_ERR_BATCH;
  if (!al16(x) || !al16(residual) || !al16(out) || (topk_idx && !al16(topk_idx)) || (topk_w && !al16(topk_w)))
    return FMOE_ERR_ALIGN;
  const size_t need = fmoe_tiered_workspace_bytes(L, n_tokens);
  if (!ws || ws_bytes < need) return FMOE_ERR_WORKSPACE;
  if (!al256(ws)) return FMOE_ERR_ALIGN;
  const size_t ab = sizeof(float) * (size_t)n_tokens * L->hidden;
  const size_t kb = sizeof(float) * (size_t)n_tokens * L->top_k;
  if (overlap(out, ab, x, ab) || overlap(out, ab, ws, need) || overlap(x, ab, ws, need) ||
      overlap(residual, ab, ws, need) || overlap(topk_idx, kb, ws, need) || overlap(topk_w, kb, ws, need) ||
      overlap(topk_idx, kb, out, ab) || overlap(topk_w, kb, out, ab) || overlap(topk_idx, kb, topk_w, kb) ||
      (residual != out && overlap(residual, ab, out, ab)) || overlap(topk_idx, kb, residual, ab) ||
      overlap(topk_w, kb, residual, ab) || overlap(topk_idx, kb, x, ab) || overlap(topk_w, kb, x, ab))
    return FMOE_ERR_ALIAS;
  return FMOE_OK;
}
}  // namespace

extern "C" {

fmoe_status fmoe_moe_layer_tiered(fmoe_cache *c, int layer, const fmoe_layer *L, int n_tokens, const float *x,
                                  const float *residual, float *out, int32_t *topk_idx, float *topk_w, void *ws,
                                  size_t ws_bytes, void *stream) {
  fmoe_status st = tiered_check(c, layer, L, n_tokens, x, residual, out, topk_idx, topk_w, ws, ws_bytes);
  if (st != FMOE_OK) return st;
  if (c->mode == 2) return FMOE_ERR_SHAPE;  // (the cache's policy runs on the device)
  c->mode = 1;
  if (!c->table_host) {
    if (hipHostMalloc((void **)&c->table_host, sizeof(void *) * (size_t)c->n_experts, hipHostMallocDefault) !=
        hipSuccess) {
      c->table_host = nullptr;
      return FMOE_ERR_LAUNCH;
    }
    for (int e = 0; e < c->n_experts; ++e) c->table_host[e] = nullptr;
  }
  if (!c->idx_host &&
      hipHostMalloc((void **)&c->idx_host, sizeof(int32_t) * kMaxTokens * kMaxTopK, hipHostMallocDefault) !=
          hipSuccess) {
    c->idx_host = nullptr;
    return FMOE_ERR_LAUNCH;
  }
  hipStream_t s = as_stream(stream);
  GroupArgs g = group_args(L, n_tokens, x, -1.f, residual, out, topk_idx, topk_w, (uint8_t *)ws);
  g.expert_ptr = c->table;
  // 1. the routing on the GPU, read back (the one host synchronisation of the call)
  if (launch_group_route(g, s) != hipSuccess) return FMOE_ERR_LAUNCH;
  const int S = n_tokens * L->top_k;
  if (hipMemcpyAsync(c->idx_host, g.idx, sizeof(int32_t) * S, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return FMOE_ERR_LAUNCH;
  // 2. the distinct experts, in ascending id; their slots; the missing blobs copied in
  std::vector<int32_t> ex(c->idx_host, c->idx_host + S);
  std::sort(ex.begin(), ex.end());
  ex.erase(std::unique(ex.begin(), ex.end()), ex.end());
  const int n = (int)ex.size();
  if (n > c->n_slots) return FMOE_ERR_WORKSPACE;  // (checked before anything is copied)
  std::vector<int32_t> slot(n), miss(n);
  c->lookups += n;
  if (!c->lru.plan(layer, ex.data(), n, slot.data(), miss.data())) return FMOE_ERR_WORKSPACE;
  const uint8_t *host_bank = (const uint8_t *)L->bank;
  for (int i = 0; i < n; ++i) {
    uint8_t *dst = c->slots + (size_t)slot[i] * c->stride;
    c->table_host[ex[i]] = dst;
    if (miss[i]) {
      if (hipMemcpyAsync(dst, host_bank + (size_t)ex[i] * c->stride, c->stride, hipMemcpyHostToDevice, s) !=
          hipSuccess)
        return FMOE_ERR_LAUNCH;
      c->bytes += (int64_t)c->stride;
    }
  }
  if (hipMemcpyAsync((void *)c->table, (const void *)c->table_host, sizeof(void *) * (size_t)L->n_experts,
                     hipMemcpyHostToDevice, s) != hipSuccess)
    return FMOE_ERR_LAUNCH;
  // 3. the experts from their slots, and the combine
  return launch_group_experts(g, s) == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
}

fmoe_status fmoe_moe_layer_tiered_device(fmoe_cache *c, int layer, const fmoe_layer *L, int n_tokens,
                                         const float *x, const float *residual, float *out, int32_t *topk_idx,
                                         float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  fmoe_status st = tiered_check(c, layer, L, n_tokens, x, residual, out, topk_idx, topk_w, ws, ws_bytes);
  if (st != FMOE_OK) return st;
  if (c->mode == 1) return FMOE_ERR_SHAPE;  // (the cache's policy runs on the host)
  const int S = n_tokens * L->top_k;
  if (c->n_slots > kMaxTierSlots || std::min(S, L->n_experts) > c->n_slots) return FMOE_ERR_WORKSPACE;
  // the bank's device-visible address, looked up once per bank (so that calls under
  // graph capture make no runtime query)
  const void *bank = nullptr;
  const auto it = c->bank_dev.find(L->bank);
  if (it != c->bank_dev.end()) {
    bank = it->second;
  } else {
    void *d = nullptr;
    if (hipHostGetDevicePointer(&d, (void *)L->bank, 0) != hipSuccess || !d) {
      (void)hipGetLastError();  // (not left for the next launch check to report)
      return FMOE_ERR_LAUNCH;
    }
    c->bank_dev[L->bank] = d;
    bank = d;
  }
  hipStream_t s = as_stream(stream);
  if (!c->dev_init) {
    // the first call initialises the state (every slot empty, counters zero): not
    // inside a graph capture, whose replays would each start from an empty cache
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cap) != hipSuccess) return FMOE_ERR_LAUNCH;
    if (cap != hipStreamCaptureStatusNone) return FMOE_ERR_WORKSPACE;
    if (launch_tier_init(c->hdr, c->key, c->n_slots, s) != hipSuccess) return FMOE_ERR_LAUNCH;
    c->dev_init = true;
  }
  c->mode = 2;
  TierPlanArgs p{};
  p.S = S;
  p.E = L->n_experts;
  p.layer = layer;
  p.n_slots = c->n_slots;
  p.stride = c->stride;
  p.slots = c->slots;
  p.table = c->table;
  p.key = c->key;
  p.last = c->last;
  p.hdr = c->hdr;
  p.jobs = c->jobs;
  if (n_tokens == 1) {
    // one token: the one-token kernels, the routed experts through the table: the
    // router, the top-K alone, the plan and its copies, then gate/up and down
    LayerArgs a = one_token_args(L, x, -1.f, residual, out, topk_idx, topk_w, (uint8_t *)ws);
    a.bank = c->slots;  // (read only where no routed expert is chosen yet: any valid blob)
    a.expert_ptr = c->table;
    p.idx = a.ws_idx;
    if (launch_layer(a, s, 1) != hipSuccess || launch_route1(a.logits, a.E, a.K, a.ws_idx, a.ws_w, s) != hipSuccess ||
        launch_tier_plan(p, s) != hipSuccess ||
        launch_tier_copy(c->hdr, c->jobs, (const uint8_t *)bank, c->slots, c->stride, s) != hipSuccess)
      return FMOE_ERR_LAUNCH;
    return launch_layer_ptr(a, s, 6) == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
  }
  GroupArgs g = group_args(L, n_tokens, x, -1.f, residual, out, topk_idx, topk_w, (uint8_t *)ws);
  g.expert_ptr = c->table;
  // the routing, the plan and the copies it needs, then the experts from their slots
  p.idx = g.idx;
  if (launch_group_route(g, s) != hipSuccess || launch_tier_plan(p, s) != hipSuccess ||
      launch_tier_copy(c->hdr, c->jobs, (const uint8_t *)bank, c->slots, c->stride, s) != hipSuccess)
    return FMOE_ERR_LAUNCH;
  return launch_group_experts(g, s) == hipSuccess ? FMOE_OK : FMOE_ERR_LAUNCH;
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

static_assert(FMOE_NOALLOC_SCRATCH_BYTES == kScratchBytes, "the static workspace size");
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
      overlap(topk_idx, kb, ws, need) || overlap(topk_w, kb, ws, need) || overlap(topk_idx, kb, topk_w, kb) ||
      overlap(topk_idx, kb, h0, hb) || overlap(topk_idx, kb, h_out, hb) || overlap(topk_idx, kb, h_all, hb * n_layers) ||
      overlap(topk_w, kb, h0, hb) || overlap(topk_w, kb, h_out, hb) || overlap(topk_w, kb, h_all, hb * n_layers))
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
  if (trace_layer < 0 || trace_layer >= n_layers) return FMOE_ERR_BATCH;
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
