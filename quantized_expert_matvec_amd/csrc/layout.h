// layout.h -- sizes and offsets of the library's packed weight layout and of
// its workspaces (host-side arithmetic shared by the packers and the launchers).
//
// A quantized matrix is a sequence of row records. A record holds cols/64
// groups of 64 codes followed by one 32-bit word per group,
// (bf16 scale << 16) | bf16 bias:
//   4-bit: [group halves 0: 16 B each][group halves 1: 16 B each][words]  (36 B/group)
//   2-bit: [groups: 16 B each][words]                                    (20 B/group)
// so that the 64 lanes of a wavefront, one group each, read every 16-byte
// piece of a row with one contiguous 128-bit load per lane.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace fmoe {

constexpr int kGroup = 64;
constexpr int kWave = 64;
constexpr int kBlock = 256;  // threads per block everywhere: 4 wavefronts
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 1024;
constexpr int kMaxTokens = 256;
constexpr int kMaxTierSlots = 65536;  // slots of a cache whose policy runs on the GPU
constexpr int kDigStride = 52;  // u32 words per 64-column group of x in digit form
constexpr size_t kScratchBytes = (size_t)4 << 20;  // static workspace of fmoe_moe_layer_noalloc (per GPU)

inline bool bits_ok(int bits) { return bits == 2 || bits == 4; }
// Columns of a quantized matrix: a multiple of 256 (four 64-column groups) up to
// 4096, so that a row's groups fit one wavefront (one group per lane).
inline bool cols_ok(int cols) { return cols >= 256 && cols <= 4096 && cols % 256 == 0; }
inline int ilog2(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}

// bytes of one group inside a row record: its codes plus its scale/bias word
inline size_t group_bytes(int bits) { return bits == 4 ? 36 : 20; }
inline size_t code_bytes(int bits) { return bits == 4 ? 32 : 16; }
inline size_t row_bytes(int bits, int cols) { return (size_t)(cols / kGroup) * group_bytes(bits); }
inline size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline size_t qmat_bytes(int bits, int rows, int cols) {
  return round_up((size_t)rows * row_bytes(bits, cols), 256);
}
// gate/up region of an expert: 2*inter interleaved records over hidden columns
inline size_t gateup_bytes(int bits, int hidden, int inter) {
  return round_up((size_t)2 * inter * row_bytes(bits, hidden), 256);
}
inline size_t down_bytes(int bits, int hidden, int inter) {
  return round_up((size_t)hidden * row_bytes(bits, inter), 256);
}
inline size_t expert_bytes(int bits, int hidden, int inter) {
  return gateup_bytes(bits, hidden, inter) + down_bytes(bits, hidden, inter);
}

// Logits of one token in the workspace: E floats, padded to a multiple of 4 (the
// routing reads them with 16-byte loads).
constexpr int logit_stride(int E) { return (E + 3) & ~3; }

// The router of the grouped kernels. From kRouterTileMin tokens it runs in tiles of
// kRt experts x kRt tokens on the matrix cores, each tile's columns split into
// router_parts() parts (separate workgroups) so that about 256 workgroups share
// it; part p writes its partial dot products to logit slab p ([B][logit_stride(E)]
// each) and the routing adds the slabs in order (all requested at once). Below
// kRouterTileMin tokens: one slab, from workgroups that hold router rows in
// registers. Measured per layer (60-layer q4 stack, same build): 8 tokens 68.0
// tiled against 67.4 row-held, 16 tokens 99.1 / 100.6, 24 tokens 125.2 / 132.1,
// 32 tokens 152.2 / 164.0, 48 tokens 206.0 / 224.5 us.
constexpr int kRouterTileMin = 16;
constexpr int kRt = 16;
constexpr int kRouterMaxParts = 4;
__host__ __device__ inline bool router_tiled(int B) { return B >= kRouterTileMin; }
__host__ __device__ inline int router_tiles(int E, int B) { return ((E + kRt - 1) / kRt) * ((B + kRt - 1) / kRt); }
// parts: the largest power of two up to kRouterMaxParts with tiles x parts <= 256
// whose column share per wavefront (hidden / 4 / parts) is a whole number of
// 32-column steps
__host__ __device__ inline int router_parts(int E, int B, int hidden) {
  if (!router_tiled(B)) return 1;
  const int tiles = router_tiles(E, B), steps = hidden / 128;
  int p = 1;
  while (p < kRouterMaxParts && tiles * 2 * p <= 256 && steps % (2 * p) == 0) p *= 2;
  return p;
}

// Workspace of one MoE layer for B tokens (all offsets 256-B aligned).
struct LayerWs {
  size_t logits;    // fp32 [parts][B][logit_stride(E)] (parts: router_parts; 1 for one token)
  size_t sigma;     // fp32 [B]
  size_t topk_idx;  // int32 [B][K]
  size_t topk_w;    // fp32 [B][K]
  size_t h_shared;  // B == 1: fp32 [inter]
  size_t h_routed;  // B == 1: fp32 [K][inter]
  size_t d_shared;  // fp32 [B][hidden]  sigma * shared-expert output
  size_t xdig;      // B == 1: u32 [hidden/64][kDigStride] x as signed base-16 digits per group (+ factor, sum)
  // B > 1 only (tokens grouped by expert):
  size_t partial;   // fp32 [B][K][hidden]  w * routed-expert output, per (token, slot)
  size_t groups;    // int32 [2 + 6 S], S = B*K: the number of distinct experts, the number of
                    // token blocks, and per token block {expert, number of slots, 4 slots} [6 S]
  size_t xq;        // int8 [B][3][hidden]     the input in integer form: three digit planes
  size_t xsum;      // fp32 [B][hidden/64][2]  per group: its factor f and the sum of x
  size_t xinv;      // fp32 [B]                its RMS factor
  size_t gdot;      // fp32 [B]                g . x before the RMS factor
  size_t hq;        // int8 [S + B][3][inter]  the SwiGLU outputs in the same form
  size_t hsum;      // fp32 [S + B][inter/64][2] per group: factor f and sum
  size_t total;
};

// grouped: the workspace of the grouped kernels (B > 1, or any B for the
// host-memory expert tier); otherwise that of the one-token kernels.
inline LayerWs layer_ws(int B, int E, int K, int hidden, int inter, bool grouped) {
  LayerWs w{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = round_up(o + bytes, 256);
    return at;
  };
  w.logits = take(sizeof(float) * (size_t)(grouped ? router_parts(E, B, hidden) : 1) * B * logit_stride(E));
  w.sigma = take(sizeof(float) * (size_t)B);
  w.topk_idx = take(sizeof(int32_t) * (size_t)B * K);
  w.topk_w = take(sizeof(float) * (size_t)B * K);
  const bool one = !grouped;
  w.h_shared = take(one ? sizeof(float) * (size_t)inter : 0);
  w.h_routed = take(one ? sizeof(float) * (size_t)K * inter : 0);
  w.d_shared = take(sizeof(float) * (size_t)B * hidden);
  w.xdig = take(one ? sizeof(uint32_t) * kDigStride * (size_t)(hidden / 64) : 0);
  const size_t S = (size_t)B * K;
  w.partial = take(grouped ? sizeof(float) * S * hidden : 0);
  w.groups = take(grouped ? sizeof(int32_t) * (6 * S + 2) : 0);
  w.xq = take(grouped ? 3 * (size_t)B * hidden : 0);
  w.xsum = take(grouped ? 2 * sizeof(float) * (size_t)B * (hidden / 64) : 0);
  w.xinv = take(grouped ? sizeof(float) * (size_t)B : 0);
  w.gdot = take(grouped ? sizeof(float) * (size_t)B : 0);
  w.hq = take(grouped ? 3 * (S + B) * inter : 0);
  w.hsum = take(grouped ? 2 * sizeof(float) * (S + B) * (inter / 64) : 0);
  w.total = o;
  return w;
}

// Workspace of a layer stack: x [B][H], two h buffers [B][H], then one layer workspace.
struct StackWs {
  size_t x, ha, hb, layer, total;
  LayerWs lw;
};

inline StackWs stack_ws(int B, int E, int K, int hidden, int inter) {
  StackWs s{};
  size_t hb = round_up(sizeof(float) * (size_t)B * hidden, 256);
  s.x = 0;
  s.ha = hb;
  s.hb = 2 * hb;
  s.layer = 3 * hb;
  s.lw = layer_ws(B, E, K, hidden, inter, B > 1);
  s.total = s.layer + s.lw.total;
  return s;
}

}  // namespace fmoe
