// kernels.h -- host-side launchers of the HIP kernels (kernels.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fmoe {

// y[r] = sum_c W[r][c] x[c] for a packed matrix (row records at blob + r * row_bytes).
hipError_t launch_qmatvec(int bits, const uint8_t *blob, int rows, int cols, const float *x, float *y,
                          hipStream_t s);

// h[r] = silu(gate_r . x) * (up_r . x) for one expert's interleaved gate/up region.
hipError_t launch_expert_gateup(int bits, const uint8_t *gateup, int hidden, int inter, const float *x,
                                float *h, hipStream_t s);

// Everything one MoE layer needs for one token.
struct LayerArgs {
  const float *router;       // [E][H]
  const float *shared_gate;  // [H] or null (no shared expert)
  const uint8_t *bank;       // E expert blobs
  const uint8_t *shared;     // one expert blob or null
  int E, K, H, I, bits;
  size_t expert_stride;      // bytes per expert blob
  size_t gateup_bytes;       // offset of the down region inside an expert blob
  const float *x;            // [H]
  float rms_eps;             // >= 0: the layer input is rms_scale(x, rms_eps); < 0: x as given
  const float *residual;     // [H]
  float *out;                // [H]
  int32_t *topk_idx_out;     // [K] or null
  float *topk_w_out;         // [K] or null
  // workspace (device)
  float *logits;             // [E] (16-byte aligned, padded to a multiple of 4)
  float *sigma;              // [1]
  int32_t *ws_idx;           // [K]
  float *ws_w;               // [K]
  float *h_shared;           // [I]
  float *h_routed;           // [K][I]
  float *d_shared;           // [H]
  uint32_t *xdig;            // [H/64][kDigStride] x in digit form (router kernel -> gate/up kernel)
  float *xs;                 // null, or [H]: x in fp32 as well (the dequant-form builds of the gate/up kernel)
  // optional per-workgroup timestamps (device, 100 MHz clock) for profiling:
  // [phase][kTraceBlocks workgroups][kTraceSlots]; null in normal use
  uint64_t *trace;
  // launch_layer_ptr: routed expert e's blob at expert_ptr[e] (device array [E]; entries
  // needed only for the chosen experts); bank then only needs one readable blob
  const uint8_t *const *expert_ptr;
};
constexpr int kTraceSlots = 8;
constexpr int kTraceBlocks = 4096;  // workgroups recorded per phase

// One MoE layer for B > 1 tokens grouped by expert (device pointers).
struct GroupArgs {
  const float *router;
  const float *gvec;         // null: no shared expert
  const uint8_t *bank;
  const uint8_t *shared;     // null: no shared expert
  size_t stride, gu_bytes;
  int E, K, H, I, B, bits;
  const float *x;
  float rms_eps;             // >= 0: each token's x is RMS-scaled first
  const float *residual;
  float *out;
  int32_t *out_idx;          // [B][K] or null
  float *out_w;              // [B][K] or null
  // workspace
  float *logits;             // [logit_parts][B][logit_stride(E)] router rows . x, before the RMS factor
  int logit_parts;           // slabs to add (router_parts)
  float *sigma;              // [B]
  float *gdot;               // [B]        gate vector . x, before the RMS factor
  int32_t *idx;              // [B][K]
  float *w;                  // [B][K]
  uint8_t *xq;               // [B][3][H]  x in integer form: three signed 8-bit digit planes
  float *xsum;               // [B][H/64][2] per group: the factor f, the sum of x
  float *xinv;               // [B]        RMS factor of x (1 without RMS scaling)
  uint8_t *hq;               // [S+B][3][I] h (routed slots, then shared tokens), as xq
  float *hsum;               // [S+B][I/64][2]
  float *d_shared;           // [B][H]
  float *partial;            // [S][H]
  int32_t *groups;           // D, NB, token blocks {expert, n, 4 slots}[S]; S = B*K
  // null: expert e's blob is bank + e * stride; else expert_ptr[e] (device array
  // [E], entries needed only for the experts the batch chooses)
  const uint8_t *const *expert_ptr;
  int n_router_blocks;       // g1
  // optional per-workgroup timestamps (device, 100 MHz clock) for profiling, as
  // LayerArgs::trace: [0] router + token preparation, [1] gate/up, [2] down; null in normal use
  uint64_t *trace;
};

// The grouped layer: four launches (router + input preparation; routing,
// grouping and the gate/up of the distinct experts and the shared expert; their
// down projections; combine). phases: bit 0 the first, bit 1 the second, bit 2
// the last two.
hipError_t launch_group(const GroupArgs &a, hipStream_t s, int phases = 7);
// The same layer in two parts around a host step: the router, input preparation
// and every token's top-K (idx, w, sigma and the caller's outputs); then the
// grouping, the gate/up and down of the chosen and shared experts, and the
// combine (expert blobs through a.expert_ptr when it is set).
hipError_t launch_group_route(const GroupArgs &a, hipStream_t s);
hipError_t launch_group_experts(const GroupArgs &a, hipStream_t s);

// Router + sigmoid gate + shared gate/up; routing + routed gate/up + shared down;
// down + weighted combine + residual. Three launches, no host synchronisation.
// phases: bit p set = enqueue kernel p+1 (7 = the whole layer).
hipError_t launch_layer(const LayerArgs &a, hipStream_t s, int phases = 7);
// Phases 2 and 3 (or any of the three) with the routed experts through a.expert_ptr.
hipError_t launch_layer_ptr(const LayerArgs &a, hipStream_t s, int phases);
// One token's top-K from the router kernel's logits into idx / w (K entries each).
hipError_t launch_route1(const float *logits, int E, int K, int32_t *idx, float *w, hipStream_t s);
// The same layer (one token, hidden 4096, inter 1024, top_k <= 4, n_experts <= 512) with
// the per-weight arithmetic of its gate/up and down projections in dequant form `form`
// (forms.h); a.xs must hold H floats of workspace.
hipError_t launch_layer_form(const LayerArgs &a, int form, hipStream_t s);

// x_t = h_t / sqrt(mean(h_t^2) + eps) for B tokens of width H.
hipError_t launch_rms(const float *h, float *x, int B, int H, float eps, hipStream_t s);
// *out ^= XOR of the 32-bit words of buf (bytes a multiple of 16); bytes == 0: an empty kernel
hipError_t launch_read_xor(const void *buf, size_t bytes, uint32_t *out, hipStream_t s);

// Device address of the current device's static workspace (kScratchBytes bytes,
// scratch.hip), looked up once per device.
hipError_t scratch_device_ptr(void **out);

// The host-memory expert tier's cache state in device memory, for the policy run
// on the GPU (tier_kernels.hip): per slot the (layer, expert) key it holds (-1:
// empty) and its last-use clock; the counters; the copies the current call needs.
struct TierHdr {
  uint64_t clock, call;
  int64_t lookups, hits, misses, bytes;
  int32_t njobs, pad;
};
struct TierPlanArgs {
  const int32_t *idx;      // [S] the call's routing (expert of each slot)
  int S, E, layer, n_slots;
  size_t stride;           // bytes per expert blob
  uint8_t *slots;          // n_slots blobs
  const uint8_t **table;   // [E] blob address of each chosen expert (written)
  int64_t *key;            // [n_slots]
  uint64_t *last;          // [n_slots]
  TierHdr *hdr;
  int32_t *jobs;           // [2 * kMaxExperts]: (slot, expert) of each miss, in the call's order
};
// The state of an empty cache: every key -1, the header zero.
hipError_t launch_tier_init(TierHdr *hdr, int64_t *key, int n_slots, hipStream_t s);
// One workgroup: the least-recently-used plan of one call (the rules of the host
// policy, expert_cache.h), the table of the chosen experts' blobs and the copy jobs.
hipError_t launch_tier_plan(const TierPlanArgs &a, hipStream_t s);
// The copies the plan asked for, read straight from the pinned host bank
// (host_bank: its device-visible address).
hipError_t launch_tier_copy(const TierHdr *hdr, const int32_t *jobs, const uint8_t *host_bank, uint8_t *slots,
                            size_t stride, hipStream_t s);

// Device packer: record r of the matrix goes to blob + rec_offset + r * rec_stride.
hipError_t launch_pack_matrix(int bits, int rows, int cols, const uint8_t *codes, const uint16_t *scale,
                              const uint16_t *bias, uint8_t *blob, size_t rec_stride, size_t rec_offset,
                              hipStream_t s);

}  // namespace fmoe
