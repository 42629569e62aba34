// grouped_kernels.h -- the MoE layer for B > 1 tokens, with the tokens grouped
// by expert: every weight row of the layer (router, shared expert, each
// distinct routed expert) is read from HBM once per layer-step and applied to
// all the tokens that use it. Included by kernels_q4.hip / kernels_q2.hip after
// layer_kernels.h, which instantiate group_b<BITS>.
//
// Several tokens against one weight row make a (skinny) dense contraction, so
// the quantized experts run on the matrix cores, on exact integer products:
// v_mfma_i32_16x16x64_i8 with
//   B operand = 16 weight rows x 64 columns (one group) of codes, each code c
//               (BITS bits) as the byte c: a mask (and a shift) of the packed
//               code words puts 16 codes of a row in a lane, in column order;
//   A operand = 16 rows = 4 tokens x {d0, d1, d2, 0}: a group of 64 values v_j
//               (x, or h) is held as v_j = f X_j, X_j an integer with
//               |X_j| <= 2^22 (the group's largest |v_j| scaled just below 2^22,
//               f a power of two), written with three signed base-256 digits,
//               X = d0 + 256 d1 + 65536 d2;
//   D (int32) = per (token digit, weight row) the exact sum over the group.
// Per (row, group) the epilogue applies the group-factored dequantization
//   sum_j (c_j s + b) v_j = s f (D0 + 256 D1 + 65536 D2) + b sum_j v_j
// with the fp32 group sum of v formed when v is prepared. The only roundings
// are those of the X_j (at most 2^-22 of the group's largest magnitude) and of
// the fp32 combination.
//
// Four launches (above 8 tokens, the top-K kernel, and above 64 slots the grouping
// kernel, before g2):
//   g1  router rows . x of every token (fp32 rows held in registers, VALU, the
//       tokens' x through LDS), unscaled; other workgroups prepare each token's
//       x for the matrix cores: RMS factor, per group the digit planes, the
//       factor f and the sum of x
//   g2  gate/up + SwiGLU of (shared expert or distinct expert, one group of 64
//       gate/up pairs = 128 rows, one 16-row tile per wavefront) for all the
//       tokens / slots using it; writes h (one whole group per item) in the same
//       integer form. The routed workgroups first derive the routing themselves
//       (top-K of every token, the distinct experts in ascending id and, for
//       each, the ascending list of the slots (token t, choice k; slot = t*K + k)
//       routed to it); the shared expert's workgroups need none and stream at once
//   g3  down of (shared expert or distinct expert, 128 or 256 rows): per token
//       sigma * (D_s h) into d_shared, per slot w * (D h) into partial[slot]
//   g4  out = residual + the K per-slot outputs in slot order + sigma * shared
#pragma once

#include <algorithm>
#include <type_traits>

#include "layer_kernels.h"

namespace fmoe {
namespace dev {

// Slots (token, choice) that the gate/up kernel's own routing handles (one thread
// per slot): batches with more, or with more than kRouteTokens tokens, take their
// top-Ks from the top-K kernel before it (k_topk); the gate/up workgroups then group
// at most 64 slots themselves (group_from_idx), and read the table the grouping
// kernel (k_group) writes for more.
// Every gate/up workgroup that routes for itself reads all the batch's logits
// (B x the router's slabs x 2 KB): from 16 tokens that traffic, and the top-Ks
// of two tokens per wavefront, cost more than the two extra launches (same-build
// layer times on the 60-layer q4 stack, in-kernel against routing kernels: 8
// tokens 69.5 / 70.9 us, 16 tokens 100.2 / 95.6, 32 tokens 156.3 / 144.6, 64
// tokens 261.5 / 232.8).
constexpr int kRouteTokens = 8;
constexpr int kRouteSlots = kRouteTokens * kMaxTopK;  // 128: every batch of at most kRouteTokens tokens
// Tokens per work item: one MFMA row block (4 rows each: hi, mid, lo, 0). An
// expert used by more tokens (the shared expert, mostly) gives several items,
// which run on different compute units and re-read its rows (from the caches).
constexpr int kTokBlock = 4;
// Batches of up to kDownOneTile tokens run the down kernel with one 128-row tile per
// workgroup (more, smaller workgroups: the last ones end sooner), larger ones with two
// tiles per staging of h (60-layer q4 stack, one tile against two: 8 tokens 60.4 / 62.9
// us per layer, 12 tokens 74.0 / 74.7, 16 tokens 84.3 / 84.4).
constexpr int kDownOneTile = 16;
constexpr int kParts = 3;       // signed 8-bit digit planes of a value's integer form
constexpr int kGThreads = 512;  // workgroup of the matrix-core kernels: 8 wavefronts
constexpr int kGWaves = kGThreads / kWave;
constexpr int kMaxNG = 64;      // groups per row (4096 columns)
// groups per weight chunk (16 rows x 8 groups; 16 groups a chunk measured slower:
// 4 tokens 46.4 against 42.7 us per layer, 16 tokens 95.2 against 89.0)
constexpr int kChunkGroups = 8;
constexpr int kWaveLds = 16 * (2 * kChunkGroups * 16 + 16) + 16 * (kChunkGroups + 1) * 4;  // LDS bytes per wavefront for a weight chunk

typedef __attribute__((ext_vector_type(4))) int i32x4_t;

// Profiling hook: thread 0 of the workgroup stamps the device clock into stamp
// slot of kernel k's rows of the trace (null in normal use).
__device__ __forceinline__ void gtrace(const GroupArgs &a, int k, int slot) {
  trace_mark(a.trace ? a.trace + (size_t)k * kTraceBlocks * kTraceSlots : nullptr, slot);
}

// ------------------------------------------------------------------ integer form

// The shift k of a group whose largest magnitude is amax (< 2^e): values are
// scaled by 2^k = 2^(22 - e), so that every X_j = round(v_j 2^k) has |X_j| <= 2^22.
__device__ __forceinline__ int group_shift(float amax) {
  int e;
  frexpf(amax, &e);  // (e = 0 for amax = 0)
  return 22 - e;
}
// The three signed base-256 digits of X = round(v 2^k): byte p of the result is
// d_p (two's complement); adding 128 to every digit first keeps the word positive.
__device__ __forceinline__ uint32_t digits3(float v, int k) {
  const int X = (int)rintf(ldexpf(v, k));
  return (uint32_t)(X + 0x808080) ^ 0x808080u;
}
// The group's factor f = 2^-k; NaN when the group holds a non-finite value.
__device__ __forceinline__ float group_factor(float amax, int k) {
  return amax <= 3.402823466e38f ? ldexpf(1.f, -k) : __int_as_float(0x7FC00000);
}
// Largest magnitude over the 8 consecutive lanes of a segment, as float bits
// (non-negative floats order as integers; NaN above infinity), in every lane.
__device__ __forceinline__ int seg_max8_bits(float v) {
  int m = __float_as_int(fabsf(v));
  m = max(m, dpp_i<0xB1, 0xF>(m, 0));   // lanes i, i^1
  m = max(m, dpp_i<0x4E, 0xF>(m, 0));   // i, i^2
  m = max(m, dpp_i<0x141, 0xF>(m, 0));  // row_half_mirror: i, 7-i
  return m;
}

// One group of one weight row as held by lane (row, q): the 16 codes of columns
// 16q .. 16q + 15 (4-bit: words 2q and 2q + 1 of the group; 2-bit: word q), and
// the (scale, bias) word.
struct MCodes {
  uint32_t c0, c1, sb;
};

// The lane's B operand for the group: its 16 codes as bytes, byte j the code of
// column 16q + j. (A operand bytes j of lane (row, q) take the same columns:
// the matrix cores pair A and B bytes of the same k-block and position.)
template <int BITS>
__device__ __forceinline__ i32x4_t mfma_codes(const MCodes &m) {
  i32x4_t b;
  if constexpr (BITS == 4) {
    // word w: byte b's low nibble is column 8w + b, its high nibble 8w + 4 + b
    b[0] = (int)(m.c0 & 0x0F0F0F0Fu);
    b[1] = (int)((m.c0 >> 4) & 0x0F0F0F0Fu);
    b[2] = (int)(m.c1 & 0x0F0F0F0Fu);
    b[3] = (int)((m.c1 >> 4) & 0x0F0F0F0Fu);
  } else {
    // byte b's field f (bits 2f, 2f + 1) is column 16q + 4f + b
    b[0] = (int)(m.c0 & 0x03030303u);
    b[1] = (int)((m.c0 >> 2) & 0x03030303u);
    b[2] = (int)((m.c0 >> 4) & 0x03030303u);
    b[3] = (int)((m.c0 >> 6) & 0x03030303u);
  }
  return b;
}

// ------------------------------------------------------------------ matrix-core rows

// Workgroup-cooperative (kGThreads threads): NTILE tiles of 16 rows per
// wavefront (tile i: rows rec0 + i * tile_stride + r * RB, r = 0..15; records of
// ng groups, RB bytes) against T <= kTokBlock vectors tokv[u] of a prepared
// source: digit plane k (0..2) at xq_base + (3 vec + k) * ng * 64 (bytes); per
// group (f, sum v) at xs_base + 2 (vec * ng + g). The vectors are staged in LDS
// once (xl: XL + 16 bytes, each vector NGP groups wide; xsl: kTokBlock * NGP + 1
// entries, zero for the groups past ng). As each tile ends, lane (n = lane % 16,
// u = lane / 16) holds in y row n of the tile for token u (meaningless for
// u >= T). Contains barriers: every thread of the workgroup calls it with the
// same T.
//
// Weights stream in chunks of CG groups. A wavefront loads a chunk of its 16
// rows with 16-byte loads over whole 16 CG-byte spans of each row (each load
// instruction covers complete cache lines), keeps DEPTH chunks in flight, and
// passes each chunk through its own LDS region (wl: kWaveLds bytes), from
// which lane (n, q) reads the codes of k-block q of row n. The loop has no
// branches around its loads (its last round, which requests nothing, is a
// separate copy), so every wait is exact; the empty asm statements keep the
// optimiser from moving the loads (and the reads of their results) away from
// where the pipeline needs them. A row of ng < NGP groups runs as NGP groups:
// the groups past ng load group ng - 1 (and its neighbour's scale/bias) again,
// and their factor f and sum are zero, so they add exactly 0. FULL: ng == NGP
// (the group count is then a compile-time constant).
template <int BITS, int NGP, int NTILE = 1, bool FULL = true>
struct MfmaRows {
  static constexpr int CG = NGP < kChunkGroups ? NGP : kChunkGroups;        // groups per chunk
  static constexpr int NC = NGP / CG;                 // chunks per row
  static constexpr int NCT = NTILE * NC;              // chunks of the whole stream
  // chunks in flight per wavefront: one (the next chunk is requested as the
  // current one is taken). A chunk is 16 rows x CG groups in 128-byte pieces of 16
  // records; with more of them outstanding the stream got slower, not faster
  // (60-layer q4 stack, per layer: 4 tokens 47.1 / 44.7 / 43.9 us with 4 / 2 / 1
  // chunks in flight, 16 tokens 95.9 / 91.2 / 88.9 us; 8 chunks 50.0 / 100.6 us)
  static constexpr int DEPTH = 1;
  static constexpr int HALVES = BITS == 4 ? 2 : 1;    // 16-byte code units per group
  static constexpr int NI = 16 * HALVES * CG / kWave; // 16-byte code loads per lane per chunk
  static constexpr int SBW = CG / 4;                  // scale/bias words per lane per chunk
  static constexpr int RS = 16 * HALVES * CG + 16;    // LDS bytes per row of codes (padded)
  static constexpr int SBS = CG + 1;                  // LDS words per row of scale/bias (padded)
  static constexpr int VS = NGP * 64 + 16;            // LDS bytes per staged vector (padded)
  static constexpr int XL = kParts * kTokBlock * VS;  // LDS bytes of staged x (a spare 16 B follow)
  static_assert(NGP <= kMaxNG, "row width");
  static_assert(16 * RS + 64 * SBS <= kWaveLds, "chunk fits the wavefront's LDS region");
  static_assert(NCT % DEPTH == 0, "whole rounds of chunks");
  static_assert((NC & (NC - 1)) == 0, "chunks per row: a power of two");
  static_assert(kTokBlock * NGP <= kGThreads, "one group sum per thread");

  struct Chunk {
    uint4 c[NI];
    uint32_t s[SBW];
  };

  float y;
  int ng;  // groups per row (<= NGP; a multiple of 4)

  // this lane's share of a chunk: code unit u = 64 k + lane is (row, half, group)
  // = (u / (HALVES CG), u / CG % HALVES, u % CG), at goff + 16 (group); scale/bias:
  // row lane / 4, groups SBW (lane % 4) .. + SBW - 1 of the chunk, at gsoff + 4 (group)
  int goff[NI], loff[NI], gj, gsoff, gsg, lsoff;
  // where lane (n, q) reads group j of the chunk in its LDS region
  int rcode, rsb;

  __device__ __forceinline__ void offsets() {
    const int lane = lane_id();
    const int q = lane >> 4, i = lane & 15;
    const int RB = ng * gbytes<BITS>();
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int u = kWave * k + lane;
      const int j = u % CG, rh = u / CG;
      const int r = rh / HALVES, h = rh % HALVES;
      goff[k] = r * RB + 16 * h * ng;
      loff[k] = r * RS + 16 * (h * CG + j);
    }
    gj = lane % CG;  // the group within the chunk, the same for every k (CG divides 64)
    const int sr = lane >> 2, sp = lane & 3;
    gsoff = sr * RB + 16 * HALVES * ng;
    gsg = SBW * sp;
    lsoff = 16 * RS + 4 * (sr * SBS + SBW * sp);
    rcode = BITS == 4 ? i * RS + 16 * (q >> 1) * CG + 8 * (q & 1) : i * RS + 4 * q;
    rsb = 16 * RS + 4 * i * SBS;
  }

  // chunk c of the stream: chunk c % NC of tile c / NC (tile rows tile_stride
  // bytes after the previous tile's)
  __device__ __forceinline__ void load_chunk(const uint8_t *__restrict__ rec0, size_t tile_stride, int c,
                                             Chunk &k) const {
    const uint8_t *r = rec0 + (size_t)(c / NC) * tile_stride;
    const int g0 = (c % NC) * CG;
#pragma unroll
    for (int t = 0; t < NI; ++t)
      k.c[t] = *reinterpret_cast<const uint4 *>(r + goff[t] + 16 * min(g0 + gj, ng - 1));
    if constexpr (SBW == 2) {
      // (ng is even: a pair past ng re-reads the last pair of the row)
      const uint2 v = *reinterpret_cast<const uint2 *>(r + gsoff + 4 * min(g0 + gsg, ng - 2));
      k.s[0] = v.x;
      k.s[1] = v.y;
    } else {
      k.s[0] = *reinterpret_cast<const uint32_t *>(r + gsoff + 4 * min(g0 + gsg, ng - 1));
    }
  }

  // one batch of staging loads: 16-byte units e0 + k kGThreads of the
  // 3 T ng 4 (vector 3u + plane, unit); past the end, a clamped unit whose store
  // goes to the spare slot at XL. One batch covers four tokens: a single memory
  // round trip.
  static constexpr int kBatch = (kParts * kTokBlock * NGP * 4 + kGThreads - 1) / kGThreads;
  __device__ __forceinline__ static void load_batch(const uint8_t *__restrict__ xq_base, const int *tokv, int units,
                                                    int ng, int e0, uint4 (&xv)[kBatch], int (&xdst)[kBatch]) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int ee = e0 + k * kGThreads;
      const int e = min(ee, units - 1);
      const int vv = e / (ng * 4), rr = e - vv * (ng * 4);
      const int vu = vv / kParts, vk = vv - kParts * vu;
      xv[k] = *reinterpret_cast<const uint4 *>(xq_base + ((size_t)(kParts * tokv[vu] + vk) * ng) * 64 + 16 * rr);
      xdst[k] = ee < units ? vv * VS + 16 * rr : XL;
    }
  }

  // An item's staging data in registers: its vectors' group factors and sums
  // (one float2 per thread; zero for the groups past ng) and its digit planes
  // (one batch covers kTokBlock tokens), with their LDS destinations.
  struct XAhead {
    uint4 xv[kBatch];
    int xdst[kBatch];
    float2 sv;
    int sdst;
    bool szero;
  };
  static_assert(kBatch * kGThreads >= kParts * kTokBlock * NGP * 4, "one batch stages an item");
  // request the staging data of an item of T tokens whose vector indices are in tv
  __device__ __forceinline__ static void stage_request(const uint8_t *__restrict__ xq_base,
                                                       const float *__restrict__ xs_base, const int *tv, int T,
                                                       int ng, XAhead &ah) {
    const int e = min((int)threadIdx.x, T * NGP - 1);
    const int u = e / NGP, gl = e - u * NGP;
    ah.sv = reinterpret_cast<const float2 *>(xs_base)[(size_t)tv[u] * ng + min(gl, ng - 1)];
    ah.szero = gl >= ng;
    ah.sdst = (int)threadIdx.x < T * NGP ? u * NGP + gl : kTokBlock * NGP;
    load_batch(xq_base, tv, kParts * T * ng * 4, ng, threadIdx.x, ah.xv, ah.xdst);
  }

  // rec0: record of the wavefront's first row of its first tile (the NTILE tiles
  // of 16 rows lie tile_stride bytes apart); wl: its LDS region; tokv: an LDS
  // table of kTokBlock vector indices, which fill(u) (run by thread u < T first)
  // writes; after() runs on every thread right after x is requested, to request
  // what the caller's epilogue needs; tile_done(tile) runs on every thread as
  // each tile's stream ends, with its rows in y.
  // AHEAD (a persistent caller, x staged per item): *have says that ah holds this
  // item's staging data already; filln(u) (thread u < Tn) writes the next item's
  // vector indices into tokn, and halfway through the last round of chunks (whose
  // slots then hold no more requests) the next item's staging data is requested
  // into ah, when there is a next item (Tn > 0), so that it arrives while this
  // item's stream ends; *have = Tn > 0. (Requesting this item's again when there
  // was none made the workgroup's last epilogue barrier wait for a needless
  // round trip: 1.1 us per layer at 16 tokens.)
  template <bool PRE, bool AHEAD = false, typename Fill, typename After, typename TileDone,
            typename FillN = void (*)(int)>
  __device__ __forceinline__ void run(int ngroups, const uint8_t *__restrict__ rec0, size_t tile_stride,
                                      const uint8_t *__restrict__ xq_base, const float *__restrict__ xs_base, int T,
                                      int *tokv, Fill fill, After after, TileDone tile_done, uint8_t *xl,
                                      float2 *xsl, uint8_t *wl, XAhead *ah = nullptr, bool *have = nullptr,
                                      int Tn = 0, int *tokn = nullptr, FillN filln = nullptr) {
    static_assert(!(PRE && AHEAD), "a staged batch needs no staging ahead");
    const int lane = lane_id();
    const int q = lane >> 4;  // k-block of the A / B operands; token of D
    const int i = lane & 15;  // A row (4 token + part) / weight row of B and D
    y = 0.f;
    ng = FULL ? NGP : ngroups;
    offsets();
    // per-token tables (tokv, ...) from values the caller requested earlier
    if ((int)threadIdx.x < T) fill((int)threadIdx.x);
    if constexpr (AHEAD) {
      if ((int)threadIdx.x < Tn) filln((int)threadIdx.x);
    }
    __syncthreads();  // tokv (tokn) written; earlier reads of xl / xsl are done
    Chunk ring[DEPTH];
    int aoff, xoff;
    if constexpr (PRE) {
      // x is staged already, every token of the batch in token order (vector
      // 3 t + part, group sums at t NGP): the whole prologue goes out at once, and
      // an A row reads its token's vector
      after();
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        load_chunk(rec0, tile_stride, d, ring[d]);
        asm volatile("" ::: "memory");
      }
      aoff = (kParts * tokv[min(i >> 2, T - 1)] + min(i & 3, kParts - 1)) * VS + q * 16;
      xoff = tokv[min(q, T - 1)] * NGP;
    } else {
      // Requests in the order they are needed: x (its group factors and sums,
      // then its digit planes: 3 T ng 4 16-byte units) and the caller's epilogue
      // values; the first weight chunk; once x is in LDS (a wavefront issues in
      // order, and a long queue of weight requests ahead of the staging stores
      // would hold them up), the rest of the first DEPTH chunks. The parts move in
      // batches (loads of a batch before its stores); stores are unconditional
      // (lanes past the end write a spare slot: xl at XL, xsl at kTokBlock * NGP),
      // so that the optimiser keeps a batch's loads together.
      XAhead own;
      XAhead &st = AHEAD ? *ah : own;
      if (!AHEAD || !*have) stage_request(xq_base, xs_base, tokv, T, ng, st);  // (uniform)
      after();
      // narrow rows stage little x: then the whole prologue goes out at once
      constexpr int EARLY = NGP <= 16 ? DEPTH : 1;
#pragma unroll
      for (int d = 0; d < EARLY; ++d) {
        load_chunk(rec0, tile_stride, d, ring[d]);
        asm volatile("" ::: "memory");
      }
      {
        const float2 v = st.sv;  // (through locals: a direct struct copy kept st in scratch memory)
        xsl[st.sdst] = st.szero ? make_float2(0.f, 0.f) : v;
      }
#pragma unroll
      for (int k = 0; k < kBatch; ++k) {
        const uint4 v = st.xv[k];
        *reinterpret_cast<uint4 *>(xl + st.xdst[k]) = v;
      }
      __syncthreads();
#pragma unroll
      for (int d = EARLY; d < DEPTH; ++d) {
        load_chunk(rec0, tile_stride, d, ring[d]);
        asm volatile("" ::: "memory");  // the loop's issue order (each chunk's loads together)
      }
      // A row i: token min(i / 4, T - 1), digit plane min(i % 4, 2) (rows past T
      // and the fourth row of a token feed D rows that are never read); X: token
      // min(q, T - 1)
      aoff = (kParts * min(i >> 2, T - 1) + min(i & 3, kParts - 1)) * VS + q * 16;
      xoff = min(q, T - 1) * NGP;
    }
    // chunk c from ring slot d; then (if REFILL) slot d requests chunk c + DEPTH
    auto step = [&](auto refill, int c, Chunk &slot) {
      // chunk c arrives here; into this wavefront's LDS region (the reads of
      // the previous chunk were issued before, and LDS keeps a wavefront's order)
#pragma unroll
      for (int t = 0; t < NI; ++t) {
        asm volatile("" : "+v"(slot.c[t].x), "+v"(slot.c[t].y), "+v"(slot.c[t].z), "+v"(slot.c[t].w));
        *reinterpret_cast<uint4 *>(wl + loff[t]) = slot.c[t];
      }
#pragma unroll
      for (int t = 0; t < SBW; ++t) {
        asm volatile("" : "+v"(slot.s[t]));
        *reinterpret_cast<uint32_t *>(wl + lsoff + 4 * t) = slot.s[t];
      }
      if constexpr (decltype(refill)::value) {
        load_chunk(rec0, tile_stride, c + DEPTH, slot);
        asm volatile("" ::: "memory");
      }
#pragma unroll 4
      for (int j = 0; j < CG; ++j) {
        const int g = (c % NC) * CG + j;
        MCodes m;
        if constexpr (BITS == 4) {
          const uint2 v = *reinterpret_cast<const uint2 *>(wl + rcode + 16 * j);
          m.c0 = v.x;
          m.c1 = v.y;
        } else {
          m.c0 = *reinterpret_cast<const uint32_t *>(wl + rcode + 16 * j);
          m.c1 = 0;
        }
        m.sb = *reinterpret_cast<const uint32_t *>(wl + rsb + 4 * j);
        const i32x4_t b = mfma_codes<BITS>(m);
        const i32x4_t A = *reinterpret_cast<const i32x4_t *>(xl + aoff + g * 64);
        i32x4_t dd = {0, 0, 0, 0};
        dd = __builtin_amdgcn_mfma_i32_16x16x64_i8(A, b, dd, 0, 0, 0);
        // D rows 4q .. 4q + 2 of this lane: token q's three digit sums (exact);
        // their value sum_j c_j X_j, the low two digits in 32-bit integers
        const int lo = dd[0] + 256 * dd[1];
        const float S = fmaf((float)dd[2], 65536.f, (float)lo);
        const float2 F = xsl[xoff + g];  // (f, sum v) of token q's group
        y = fmaf(scale_of(m.sb) * F.x, S, fmaf(bias_of(m.sb), F.y, y));
      }
      if (c % NC == NC - 1) {  // (uniform) the tile's last chunk
        tile_done(c / NC);
        y = 0.f;
      }
    };
    // every round but the last refills its slots; the last round requests
    // nothing, so no loads are left in flight when the stream ends
#pragma unroll 1
    for (int cb = 0; cb < NCT - DEPTH; cb += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) step(std::true_type{}, cb + d, ring[d]);
    }
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      step(std::false_type{}, NCT - DEPTH + d, ring[d]);
      if constexpr (AHEAD) {
        if (d == (DEPTH - 1) / 2) {
          if (Tn > 0) {  // (uniform: no next item, no request)
            stage_request(xq_base, xs_base, tokn, Tn, ng, *ah);
            asm volatile("" ::: "memory");
          }
          *have = Tn > 0;
        }
      }
    }
  }
};

// ------------------------------------------------------------------ g1

// g1: workgroups [0, n_router_blocks): router rows against every token's x,
// unscaled (each row split over router_split() wavefronts, two rows per
// workgroup, so that 512 rows take 256 compute units). Workgroups
// n_router_blocks + t: token t's x for the matrix cores (RMS factor xinv; per
// group the three digit planes, the factor f and the sum of x) and its gate dot
// product g . x (unscaled).
constexpr int kG1Chunk = 4;  // tokens whose x is staged in LDS at a time
template <int NGH>
__host__ __device__ constexpr int g1_rows_per_block() {
  return kWavesPerBlock / router_split<NGH>();
}

// From kRouterTileMin tokens the router runs on the matrix cores instead
// (router_tile below): every workgroup of the row-held form reads every token's x.

typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// One part of one tile of the router on the matrix cores: for 16 experts x 16
// tokens, the dot products R_e . x_t over the part's columns (fp32, unscaled),
// with v_mfma_f32_16x16x4_f32 (fp32 products, fp32 sums), into logit slab p.
// Lane l holds A[l % 16][k] and B[k][l % 16] for k = l / 16: with two float4
// loads per operand the lane covers columns c + 8 (l / 16) .. + 7 of its expert's
// row and of its token, and eight MFMAs take them in turn (the same column order
// on both sides). The four wavefronts take a quarter of the part's columns each;
// their partial tiles are added in LDS in wavefront order, so the result does not
// depend on timing. Workgroups that share router rows (same expert tile and part)
// run on one XCD (the dispatcher places workgroup b on XCD b % 8; with a multiple
// of 8 such units, unit u goes to XCD u % 8), so each XCD's L2 serves those rows to
// all token tiles after one read. part: 4 x 256 floats of LDS.
__device__ __forceinline__ void router_tile(const GroupArgs &a, float (*part)[kRt * kRt]) {
  const int lane = lane_id(), wv = wave_in_block();
  const int P = a.logit_parts;
  const int n_units = ((a.E + kRt - 1) / kRt) * P, n_tt = (a.B + kRt - 1) / kRt;
  const int b = blockIdx.x;
  int un, tt;  // unit = (expert tile, part), token tile
  if (n_units % 8 == 0) {
    const int x = b % 8, s = b / 8;
    un = x + 8 * (s / n_tt);
    tt = s % n_tt;
  } else {
    un = b / n_tt;
    tt = b % n_tt;
  }
  const int rt = un / P, pt = un % P;
  const int H = a.H, HP = H / P;  // the part's columns
  const int e0 = rt * kRt, t0 = tt * kRt;
  const int cw = pt * HP + wv * (HP / kWavesPerBlock) + 8 * (lane >> 4);  // this lane's first column
  const float4 *rp = reinterpret_cast<const float4 *>(a.router + (size_t)min(e0 + (lane & 15), a.E - 1) * H + cw);
  const float4 *xp = reinterpret_cast<const float4 *>(a.x + (size_t)min(t0 + (lane & 15), a.B - 1) * H + cw);
  const int steps = HP / kWavesPerBlock / 32;  // 32 columns per step (router_parts keeps it whole, >= 1)
  constexpr int U = 8;                        // steps in flight (128 KB per workgroup)
  float4 ra[U][2], xa[U][2];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int nx = min(u, steps - 1);
    ra[u][0] = rp[8 * nx];
    ra[u][1] = rp[8 * nx + 1];
    xa[u][0] = xp[8 * nx];
    xa[u][1] = xp[8 * nx + 1];
  }
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  for (int st = 0; st < steps; st += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (st + u >= steps) break;  // (uniform)
      const float4 r0 = ra[u][0], r1 = ra[u][1], x0 = xa[u][0], x1 = xa[u][1];
      if (st + U < steps) {  // (uniform: no requests past the part's last step)
        const int nx = min(st + U + u, steps - 1);  // (past the end: the last step again, unused)
        ra[u][0] = rp[8 * nx];
        ra[u][1] = rp[8 * nx + 1];
        xa[u][0] = xp[8 * nx];
        xa[u][1] = xp[8 * nx + 1];
      }
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r0.x, x0.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r0.y, x0.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r0.z, x0.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r0.w, x0.w, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r1.x, x1.x, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r1.y, x1.y, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r1.z, x1.z, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(r1.w, x1.w, acc, 0, 0, 0);
    }
  }
  // lane l holds D[4 (l / 16) + j][l % 16]: expert e0 + 4 (l / 16) + j, token t0 + l % 16
#pragma unroll
  for (int j = 0; j < 4; ++j) part[wv][64 * j + lane] = acc[j];
  __syncthreads();
  const int o = threadIdx.x;  // (kBlock = 256 = the tile's outputs)
  const float d = ((part[0][o] + part[1][o]) + part[2][o]) + part[3][o];
  const int l = o & 63, j = o >> 6;
  const int e = e0 + 4 * (l >> 4) + j, t = t0 + (l & 15);
  if (e < a.E && t < a.B) a.logits[((size_t)pt * a.B + t) * logit_stride(a.E) + e] = d;
}

// Input preparation of token t for the matrix cores (RMS factor xinv; per group
// the three digit planes, the factor f and the sum of x) and its gate dot
// product g . x (unscaled), by one workgroup. part: 2 x kWavesPerBlock floats of LDS.
__device__ __forceinline__ void g1_prep(const GroupArgs &a, int t, float (*part)[kWavesPerBlock]) {
  const int lane = lane_id();
  const int wv = wave_in_block();
  const int ng = a.H / kGroup, H = a.H;
  const bool rms = a.rms_eps >= 0.f;
  const float *xt = a.x + (size_t)t * H;
  const float *gv = a.gvec ? a.gvec : a.x;  // (read but unused without a shared expert)
  const int UNITS = ng * 8;  // 8 consecutive columns each: unit u = columns 8u .. 8u + 7
  float ss = 0.f, gd = 0.f;
  for (int u0 = 0; u0 < UNITS; u0 += kBlock) {
    const int u = u0 + threadIdx.x;
    const bool ok = u < UNITS;
    const int uc = ok ? u : UNITS - 1;
    const int g = uc >> 3;
    const int c = 8 * uc;
    const float4 v0 = *reinterpret_cast<const float4 *>(xt + c);
    const float4 v1 = *reinterpret_cast<const float4 *>(xt + c + 4);
    const float4 g0 = *reinterpret_cast<const float4 *>(gv + c);
    const float4 g1 = *reinterpret_cast<const float4 *>(gv + c + 4);
    const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    const float gw[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    float sum = 0.f, amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      sum += f[j];
      amax = __int_as_float(max(__float_as_int(amax), __float_as_int(fabsf(f[j]))));
      if (ok) {
        ss = fmaf(f[j], f[j], ss);
        gd = fmaf(gw[j], f[j], gd);
      }
    }
    // the group's 8 units are 8 consecutive threads
    sum = seg_allreduce<8>(sum);
    const float gmax = __int_as_float(seg_max8_bits(amax));
    const int k = group_shift(gmax);
    uint32_t d[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) d[j] = digits3(f[j], k);
    if (ok) {
      uint8_t *dst = a.xq + ((size_t)(kParts * t) * ng + g) * 64 + 8 * (uc & 7);
#pragma unroll
      for (int p = 0; p < kParts; ++p) {
        const int sh = 8 * p;
        const uint2 w = {((d[0] >> sh) & 0xFFu) | ((d[1] >> sh) & 0xFFu) << 8 | ((d[2] >> sh) & 0xFFu) << 16 |
                             ((d[3] >> sh) & 0xFFu) << 24,
                         ((d[4] >> sh) & 0xFFu) | ((d[5] >> sh) & 0xFFu) << 8 | ((d[6] >> sh) & 0xFFu) << 16 |
                             ((d[7] >> sh) & 0xFFu) << 24};
        *reinterpret_cast<uint2 *>(dst + (size_t)p * ng * 64) = w;
      }
      if ((uc & 7) == 0) reinterpret_cast<float2 *>(a.xsum)[(size_t)t * ng + g] = make_float2(group_factor(gmax, k), sum);
    }
  }
  ss = seg_reduce<kWave>(ss);
  gd = seg_reduce<kWave>(gd);
  if (lane == kWave - 1) {
    part[0][wv] = ss;
    part[1][wv] = gd;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    a.xinv[t] = rms ? rms_inv(part[0], H, a.rms_eps) : 1.f;
    if (a.gvec) {
      float d = part[1][0];
#pragma unroll
      for (int i = 1; i < kWavesPerBlock; ++i) d += part[1][i];
      a.gdot[t] = d;
    }
  }
}

template <int BITS, int NGHP>
__global__ __launch_bounds__(kBlock) void k_g1(const GroupArgs a) {
  constexpr int SPLIT = router_split<NGHP>();
  constexpr int NTW = NGHP / 4 / SPLIT;                      // float4 per lane of a wavefront's part of a row, at most
  constexpr int RPB = g1_rows_per_block<NGHP>();
  constexpr int C4 = (kG1Chunk * NGHP * 16 + kBlock - 1) / kBlock;
  const int ng = a.H / kGroup, H = a.H, nt = ng / 4;
  const int CF4 = kG1Chunk * H / 4;                          // float4 of a chunk of tokens
  __shared__ float part[2][kWavesPerBlock];
  __shared__ uint32_t xc[kG1Chunk * NGHP * kGroup];          // a chunk of tokens' x (fp32 bits)
  __shared__ float dp[kWavesPerBlock][kMaxTokens];           // per wavefront: its part of each token's dot
  const int lane = lane_id();
  const int wv = wave_in_block();
  gtrace(a, 0, 0);
  if ((int)blockIdx.x >= a.n_router_blocks) {
    g1_prep(a, blockIdx.x - a.n_router_blocks, part);
    gtrace(a, 0, 3);
    return;
  }
  // ---- router rows: a wavefront holds its part of one fp32 row in registers;
  // the tokens' x vectors pass through LDS kG1Chunk at a time (the next
  // chunk's loads in flight while the current one is used). The dot products
  // are written unscaled: the RMS factor of each token (xinv, from the
  // preparation workgroups) is applied by the routing.
  const int half = wv % SPLIT;
  const int row = (int)blockIdx.x * RPB + wv / SPLIT;
  const int rr = min(row, a.E - 1);
  const int per = (nt + SPLIT - 1) / SPLIT;  // chunks of 256 columns per part
  const int t0 = per * half, tn = min(per, nt - t0);  // this part's chunks (tn >= 1)
  const float4 *src = reinterpret_cast<const float4 *>(a.router + (size_t)rr * H) + 64 * t0;
  float4 wr[NTW];
#pragma unroll
  for (int q = 0; q < NTW; ++q) wr[q] = src[lane + 64 * min(q, tn - 1)];
  Staged<C4> nx;
  stage_load(a.x, min(kG1Chunk, a.B) * (H / 4), nx);
#pragma unroll 1
  for (int c = 0; c < a.B; c += kG1Chunk) {
    __syncthreads();  // the previous chunk's reads are done
    stage_copy(nx, CF4, xc);
    __syncthreads();
    // the next chunk, if any (uniform)
    if (c + kG1Chunk < a.B) {
      const int cn = c + kG1Chunk;
      stage_load(a.x + (size_t)cn * H, min(kG1Chunk, a.B - cn) * (H / 4), nx);
      asm volatile("" ::: "memory");
    }
#pragma unroll
    for (int tt = 0; tt < kG1Chunk; ++tt) {
      const float4 *xv4 = reinterpret_cast<const float4 *>(xc) + tt * (H / 4) + 64 * t0;
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < NTW; ++q) {
        if (q < tn) {  // (uniform)
          const float4 xv = xv4[lane + 64 * q];
          acc = fmaf(wr[q].x, xv.x, acc);
          acc = fmaf(wr[q].y, xv.y, acc);
          acc = fmaf(wr[q].z, xv.z, acc);
          acc = fmaf(wr[q].w, xv.w, acc);
        }
      }
      const float d = seg_reduce<kWave>(acc);
      if (lane == kWave - 1 && c + tt < a.B) dp[wv][c + tt] = d;
    }
  }
  __syncthreads();
  // the parts of each row, added in order
  for (int i = threadIdx.x; i < RPB * a.B; i += kBlock) {
    const int r = i / a.B, t = i - r * a.B;
    float d = dp[SPLIT * r][t];
#pragma unroll
    for (int h = 1; h < SPLIT; ++h) d += dp[SPLIT * r + h][t];
    const int rw = (int)blockIdx.x * RPB + r;
    if (rw < a.E) a.logits[(size_t)t * logit_stride(a.E) + rw] = d;
  }
  gtrace(a, 0, 3);
}

// g1, for batches of kRouterTileMin tokens or more: workgroups [0,
// n_router_blocks) compute the router in parts of 16 x 16 tiles on the matrix
// cores (router_tile), workgroups n_router_blocks + t prepare token t (g1_prep).
template <int BITS>
__global__ __launch_bounds__(kBlock) void k_g1t(const GroupArgs a) {
  static_assert(kBlock == kRt * kRt && kWavesPerBlock == 4, "one output per thread, four column quarters");
  __shared__ float part[2][kWavesPerBlock];
  __shared__ float tile[kWavesPerBlock][kRt * kRt];
  gtrace(a, 0, 0);
  if ((int)blockIdx.x >= a.n_router_blocks)
    g1_prep(a, blockIdx.x - a.n_router_blocks, part);
  else
    router_tile(a, tile);
  gtrace(a, 0, 3);
}

// ------------------------------------------------------------------ g2, g3

// The grouping table G (int32, in the workspace), written by the routing:
//   G[0] = D, the number of distinct routed experts; G[1] = NB, the number of
//   routed token blocks;
//   G[2 + kBlkInts k ..]: token block k < NB = {expert, number of slots n
//   (1..kTokBlock), its slots (slot = token * K + choice)}. The distinct experts
//   come in ascending id, their slots in ascending order, an expert's blocks
//   consecutive. One record holds all a down-projection workgroup needs.
constexpr int kBlkInts = 2 + kTokBlock;
__host__ __device__ constexpr int g_size(int S) { return 2 + kBlkInts * S; }

// One work item: up to kTokBlock tokens of one expert.
struct GroupItem {
  int expert;  // -1: the shared expert
  int q0;      // routed: offset of its slots in the block table; shared: first token
  int n;       // slots / tokens (1..kTokBlock)
};

// ------------------------------------------------------------------ routing

// LDS scratch of block_route (it lives in the x staging buffer, which is free
// until staging starts).
template <int NW>  // wavefronts holding slots (slots 64 v .. 64 v + 63)
struct RouteLdsT {
  unsigned long long mask[NW][kMaxExperts];  // [v][e]: lanes of wavefront v routed to e
  int sidx[64 * NW];                         // expert of each slot
  int eoff[kMaxExperts];                     // list offset of each present expert
  int wtot[kGWaves];
  TopkLds tk[kGWaves];                       // each wavefront's top-K scratch
};
using RouteLds = RouteLdsT<kRouteSlots / kWave>;  // every routed-in-kernel batch (kRouteSlots slots)

// The top-K of every token of the batch (wavefront t % 8 takes token t, two
// tokens per pass, all their loads requested together), from its unscaled logits
// with the weights taken after its RMS factor: sidx[t K + j] = choice j of token t
// (LDS). The writer workgroup also stores the routing (idx, w, sigma, the
// caller's outputs). No barrier: the caller synchronises before reading sidx.
__device__ __forceinline__ void route_topk(const GroupArgs &a, int *sidx, TopkLds (&tks)[kGWaves], bool writer) {
  const int lane = lane_id();
  const int wave = wave_in_block();
  // token t's routing from its top-K (lane j < K: choice j): slot experts, and
  // the writer's outputs
  auto publish = [&](int t, int mi, float mw, float inv, float gd) {
    if (lane < a.K) {
      const int s = t * a.K + lane;
      sidx[s] = mi;
      if (writer) {
        a.idx[s] = mi;
        a.w[s] = mw;
        if (a.out_idx) a.out_idx[s] = mi;
        if (a.out_w) a.out_w[s] = mw;
      }
    }
    if (writer && lane == 0 && a.gvec) a.sigma[t] = 1.f / (1.f + expf(-gd * inv));
  };
  TopkLds &tk = tks[wave];
  if (a.E <= 512) {
    // wavefront v: tokens v, v + 8, ...; two tokens per pass, all their loads
    // (logits in the top-K's layout, RMS factor, gate dot) requested together
    for (int t0 = wave; t0 < a.B; t0 += 2 * kGWaves) {
      const int t1 = min(t0 + kGWaves, a.B - 1);  // (past the end: a repeat, unused)
      float v0[8], v1[8];
      const size_t ps = (size_t)a.B * logit_stride(a.E);  // (slab stride)
      load_logits<8>(a.logits + (size_t)t0 * logit_stride(a.E), a.E, v0, a.logit_parts, ps);
      load_logits<8>(a.logits + (size_t)t1 * logit_stride(a.E), a.E, v1, a.logit_parts, ps);
      const float inv0 = a.xinv[t0], inv1 = a.xinv[t1];
      const float gd0 = a.gvec ? a.gdot[t0] : 0.f, gd1 = a.gvec ? a.gdot[t1] : 0.f;
      int key[8], mi;
      float mw;
      logit_keys<8>(v0, a.E, key);
      wave_topk<8>(key, a.K, inv0, tk, mi, mw);
      publish(t0, mi, mw, inv0, gd0);
      if (t0 + kGWaves < a.B) {
        logit_keys<8>(v1, a.E, key);
        wave_topk<8>(key, a.K, inv1, tk, mi, mw);
        publish(t1, mi, mw, inv1, gd1);
      }
    }
  } else {
    for (int t = wave; t < a.B; t += kGWaves) {
      const float inv = a.xinv[t];
      const float gd = a.gvec ? a.gdot[t] : 0.f;
      int mi;
      float mw;
      wave_topk_lds(a.logits + (size_t)t * logit_stride(a.E), a.E, a.K, inv, tk, mi, mw, a.logit_parts,
                    (size_t)a.B * logit_stride(a.E));
      publish(t, mi, mw, inv, gd);
    }
  }
}

// Top-K of every token and the grouping of the S = B*K slots by expert, by one
// workgroup of kGThreads threads, deterministic whatever the thread timing:
//  - top-K of each token (route_topk);
//  - mask[v][e] = the lanes of wavefront v (slots 64v ..) routed to expert e (LDS
//    atomic ORs: the result does not depend on their order); a slot's position in
//    its expert's list = the set bits below it, in its own and earlier wavefronts:
//    ascending slot order within each list;
//  - the distinct experts in ascending id, with the offsets of their lists and of
//    their token blocks, from one workgroup scan over the experts (two per thread).
// On return blk[kBlkInts k ..] holds the token blocks (LDS; slotl[0..S) the
// lists, as scratch); returns NB. The writer workgroup also stores the routing
// (idx, w, sigma, the caller's outputs) and the table G.
template <int NW>
__device__ __forceinline__ int block_route(const GroupArgs &a, RouteLdsT<NW> &R, int *slotl, int *blk, bool writer) {
  static_assert(kRouteSlots <= kGThreads, "one thread per slot");
  static_assert(kMaxExperts <= 2 * kGThreads, "two experts per thread in the scan");
  const int lane = lane_id();
  const int wave = wave_in_block();
  const int S = a.B * a.K;
  const int nwl = (S + kWave - 1) / kWave;  // wavefronts holding slots
  for (int i = threadIdx.x; i < nwl * a.E; i += kGThreads) R.mask[i / a.E][i % a.E] = 0ull;
  route_topk(a, R.sidx, R.tk, writer);
  __syncthreads();
  const int s = threadIdx.x;
  const bool live = s < S;
  const int e = live ? R.sidx[s] : 0;
  if (live) atomicOr(&R.mask[wave][e], 1ull << lane);
  __syncthreads();
  int pos = 0;
  if (live) {
    pos = __popcll(R.mask[wave][e] & ((1ull << lane) - 1ull));
    for (int v = 0; v < wave; ++v) pos += __popcll(R.mask[v][e]);
  }
  // experts 2x and 2x + 1 of thread x: slot counts and token blocks, then an
  // integer scan of (present experts | slots << 11 | token blocks << 21)
  const int e0 = 2 * (int)threadIdx.x, e1 = e0 + 1;
  int n0 = 0, n1 = 0;
  for (int v = 0; v < nwl; ++v) {
    n0 += e0 < a.E ? __popcll(R.mask[v][e0]) : 0;
    n1 += e1 < a.E ? __popcll(R.mask[v][e1]) : 0;
  }
  const int p0 = n0 > 0, p1 = n1 > 0;
  const int nb0 = (n0 + kTokBlock - 1) / kTokBlock, nb1 = (n1 + kTokBlock - 1) / kTokBlock;
  const int mine = (p0 + p1) | (n0 + n1) << 11 | (nb0 + nb1) << 21;
  int v = mine;
  v += dpp_i<0x111, 0xF>(v, 0);  // row_shr:1
  v += dpp_i<0x112, 0xF>(v, 0);  // row_shr:2
  v += dpp_i<0x114, 0xF>(v, 0);  // row_shr:4
  v += dpp_i<0x118, 0xF>(v, 0);  // row_shr:8
  v += dpp_i<0x142, 0xA>(v, 0);  // row_bcast:15
  v += dpp_i<0x143, 0xC>(v, 0);  // row_bcast:31
  if (lane == kWave - 1) R.wtot[wave] = v;
  __syncthreads();
  int base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kGWaves; ++w) {
    base += w < wave ? R.wtot[w] : 0;
    tot += R.wtot[w];
  }
  const int ex = base + v - mine;  // exclusive prefix of this thread
  const int o0 = (ex >> 11) & 1023, b0 = ex >> 21;
  const int D = tot & 2047, NB = tot >> 21;
  if (p0) R.eoff[e0] = o0;
  if (p1) R.eoff[e1] = o0 + n0;
  __syncthreads();
  if (live) slotl[R.eoff[e] + pos] = s;
  __syncthreads();
  // token blocks of the two experts, with their slots
  for (int k = 0; k < nb0; ++k) {
    const int n = min(kTokBlock, n0 - kTokBlock * k), q = o0 + kTokBlock * k;
    int *r = blk + kBlkInts * (b0 + k);
    r[0] = e0;
    r[1] = n;
#pragma unroll
    for (int u = 0; u < kTokBlock; ++u) r[2 + u] = slotl[q + min(u, n - 1)];
  }
  for (int k = 0; k < nb1; ++k) {
    const int n = min(kTokBlock, n1 - kTokBlock * k), q = o0 + n0 + kTokBlock * k;
    int *r = blk + kBlkInts * (b0 + nb0 + k);
    r[0] = e1;
    r[1] = n;
#pragma unroll
    for (int u = 0; u < kTokBlock; ++u) r[2 + u] = slotl[q + min(u, n - 1)];
  }
  __syncthreads();
  if (writer) {
    int32_t *G = a.groups;
    if (threadIdx.x == 0) {
      G[0] = D;
      G[1] = NB;
    }
    for (int k = threadIdx.x; k < kBlkInts * NB; k += kGThreads) G[2 + k] = blk[k];
  }
  return NB;
}

// LDS scratch of route_small.
struct __attribute__((aligned(16))) RouteSmallLds {
  int sidx[kWave];  // expert of each slot (16-byte aligned: read four at a time)
  int sorted[kWave];  // the slots in (expert, slot) order
  int info[kWave];  // per sorted position: its slot's list index k | expert << 8 | slots in its block << 24
  int nb;
  TopkLds tk[kGWaves];
};

// The routing of a batch of S <= 64 slots, with the same result as block_route
// (the table G and blk: the distinct experts in ascending id, each expert's slots
// in ascending order cut into token blocks of up to kTokBlock, the blocks in that
// order), with one wavefront doing the grouping instead of a scan over every
// expert: after the top-Ks, lane s of wavefront 0 holds slot s and counts, over
// all slots, those of a lower expert, those of its own and those of its own below
// it (its index k in its expert's list); its rank under the key (expert, slot) is
// the first count plus k, and it opens a token block when k is a multiple of
// kTokBlock. The slots are placed in rank order in LDS, and each
// block-opening position writes its block, numbered by the block-opening
// positions below it. Returns NB.
// The grouping alone, from the slots' experts in R.sidx (S <= 64; written and
// synchronised by the caller); the writer stores the table G. Returns NB.
__device__ __forceinline__ int group_ranked(const GroupArgs &a, RouteSmallLds &R, int *blk, bool writer) {
  const int lane = lane_id();
  const int S = a.B * a.K;
  if (wave_in_block() == 0) {
    const bool live = lane < S;
    const int e = live ? R.sidx[lane] : kMaxExperts;
    // every lane reads the slots' experts four at a time (the same LDS words for
    // all lanes: broadcasts); slots past S read as kMaxExperts, above every expert
    int lower = 0, same = 0, k = 0;
    for (int j0 = 0; j0 < S; j0 += 4) {  // (uniform)
      const int4 q = *reinterpret_cast<const int4 *>(R.sidx + j0);
      const int ej[4] = {q.x, j0 + 1 < S ? q.y : kMaxExperts, j0 + 2 < S ? q.z : kMaxExperts,
                         j0 + 3 < S ? q.w : kMaxExperts};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        lower += ej[u] < e ? 1 : 0;
        same += ej[u] == e ? 1 : 0;
        k += ej[u] == e && j0 + u < lane ? 1 : 0;  // index of the slot in its expert's list
      }
    }
    const int rank = lower + k;  // position of the slot under the key (expert, slot)
    const unsigned long long first = __ballot(live && k == 0);  // one slot per distinct expert
    if (live) {
      const bool opens = k % kTokBlock == 0;
      R.sorted[rank] = lane;
      R.info[rank] = opens ? (k | e << 8 | min(kTokBlock, same - k) << 24) : -1;
    }
    wave_lds_fence();
    // lane p: sorted position p
    const int inf = lane < S ? R.info[lane] : -1;
    const bool opens = inf >= 0;
    const unsigned long long bm = __ballot(opens);
    const int nb = __popcll(bm);
    if (opens) {
      const int b = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u));
      const int n = inf >> 24, ex = (inf >> 8) & 0xFFFF;
      int rec[kBlkInts];
      rec[0] = ex;
      rec[1] = n;
#pragma unroll
      for (int u = 0; u < kTokBlock; ++u) rec[2 + u] = R.sorted[lane + min(u, n - 1)];
#pragma unroll
      for (int i = 0; i < kBlkInts; ++i) blk[kBlkInts * b + i] = rec[i];
      if (writer) {
#pragma unroll
        for (int i = 0; i < kBlkInts; ++i) a.groups[2 + kBlkInts * b + i] = rec[i];
      }
    }
    if (lane == 0) {
      R.nb = nb;
      if (writer) {
        a.groups[0] = __popcll(first);
        a.groups[1] = nb;
      }
    }
  }
  __syncthreads();
  return R.nb;
}

__device__ __forceinline__ int route_small(const GroupArgs &a, RouteSmallLds &R, int *blk, bool writer) {
  static_assert(kTokBlock * kMaxTopK <= kWave, "every batch of at most kTokBlock tokens: one slot per lane");
  route_topk(a, R.sidx, R.tk, writer);
  __syncthreads();
  return group_ranked(a, R, blk, writer);
}

// The grouping of at most 64 slots from the routing kernel's indices (a.idx).
__device__ __forceinline__ int group_from_idx(const GroupArgs &a, RouteSmallLds &R, int *blk, bool writer) {
  const int S = a.B * a.K;
  if ((int)threadIdx.x < S) R.sidx[threadIdx.x] = a.idx[threadIdx.x];
  __syncthreads();
  return group_ranked(a, R, blk, writer);
}

// ------------------------------------------------------------------ routing kernels (large batches)

// k_topk: the routing of every token, one wavefront per token: the top-K of its
// unscaled logits with the weights taken after its RMS factor (as block_route),
// into idx / w (and the caller's outputs), and its shared-expert gate sigma.
template <int BITS>
__global__ __launch_bounds__(kGThreads) void k_topk(const GroupArgs a) {
  __shared__ TopkLds tks[kGWaves];
  const int t = (int)blockIdx.x * kGWaves + wave_in_block();
  if (t >= a.B) return;  // (uniform over the wavefront)
  const int lane = lane_id();
  const float inv = a.xinv[t];
  const float gd = a.gvec ? a.gdot[t] : 0.f;
  int mi;
  float mw;
  wave_topk_lds(a.logits + (size_t)t * logit_stride(a.E), a.E, a.K, inv, tks[wave_in_block()], mi, mw,
                a.logit_parts, (size_t)a.B * logit_stride(a.E));
  if (lane < a.K) {  // lane j stores choice j
    const int s = t * a.K + lane;
    a.idx[s] = mi;
    a.w[s] = mw;
    if (a.out_idx) a.out_idx[s] = mi;
    if (a.out_w) a.out_w[s] = mw;
  }
  if (lane == 0 && a.gvec) a.sigma[t] = 1.f / (1.f + expf(-gd * inv));
}

// k_group: one workgroup groups the S = B K slots by expert into the table G
// (layout above): per expert its slots in ascending order, the experts in
// ascending id, each expert's list cut into token blocks of up to kTokBlock.
// Deterministic whatever the thread timing: the counts come from LDS atomic adds
// (their order does not matter), and a slot's place in its expert's list is the
// number of lower slots with the same expert, taken 512 slots at a time from
// per-wavefront 64-bit masks (as in block_route), plus the expert's running
// count over the earlier rounds.
struct GroupLds {
  unsigned long long mask[kGWaves][kMaxExperts];
  int cnt[kMaxExperts], eoff[kMaxExperts], boff[kMaxExperts], run[kMaxExperts];
  int slotl[kMaxTokens * kMaxTopK];
  int wtot[kGWaves];
};
template <int BITS>
__global__ __launch_bounds__(kGThreads) void k_group(const GroupArgs a) {
  static_assert(kMaxExperts <= 2 * kGThreads, "two experts per thread in the scan");
  __shared__ GroupLds R;
  const int lane = lane_id(), wave = wave_in_block();
  const int S = a.B * a.K, E = a.E;
  for (int e = threadIdx.x; e < E; e += kGThreads) {
    R.cnt[e] = 0;
    R.run[e] = 0;
  }
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += kGThreads) atomicAdd(&R.cnt[a.idx[s]], 1);
  __syncthreads();
  // experts 2x and 2x + 1 of thread x: slot counts and token blocks, then integer
  // scans of two words, (present experts | slots << 11) and token blocks
  const int e0 = 2 * (int)threadIdx.x, e1 = e0 + 1;
  const int n0 = e0 < E ? R.cnt[e0] : 0, n1 = e1 < E ? R.cnt[e1] : 0;
  const int nb0 = (n0 + kTokBlock - 1) / kTokBlock, nb1 = (n1 + kTokBlock - 1) / kTokBlock;
  int v1 = (n0 > 0) + (n1 > 0) + ((n0 + n1) << 11);  // present experts (< 2048), slots (<= 4096)
  int v2 = nb0 + nb1;                                // token blocks
  const int m1 = v1, m2 = v2;
  v1 += dpp_i<0x111, 0xF>(v1, 0);
  v2 += dpp_i<0x111, 0xF>(v2, 0);
  v1 += dpp_i<0x112, 0xF>(v1, 0);
  v2 += dpp_i<0x112, 0xF>(v2, 0);
  v1 += dpp_i<0x114, 0xF>(v1, 0);
  v2 += dpp_i<0x114, 0xF>(v2, 0);
  v1 += dpp_i<0x118, 0xF>(v1, 0);
  v2 += dpp_i<0x118, 0xF>(v2, 0);
  v1 += dpp_i<0x142, 0xA>(v1, 0);
  v2 += dpp_i<0x142, 0xA>(v2, 0);
  v1 += dpp_i<0x143, 0xC>(v1, 0);
  v2 += dpp_i<0x143, 0xC>(v2, 0);
  __shared__ int wtot2[kGWaves];
  if (lane == kWave - 1) {
    R.wtot[wave] = v1;
    wtot2[wave] = v2;
  }
  __syncthreads();
  int base1 = 0, base2 = 0, tot1 = 0, tot2 = 0;
#pragma unroll
  for (int w = 0; w < kGWaves; ++w) {
    base1 += w < wave ? R.wtot[w] : 0;
    base2 += w < wave ? wtot2[w] : 0;
    tot1 += R.wtot[w];
    tot2 += wtot2[w];
  }
  const int ex1 = base1 + v1 - m1, ex2 = base2 + v2 - m2;  // exclusive prefixes
  const int o0 = ex1 >> 11;
  if (e0 < E) {
    R.eoff[e0] = o0;
    R.boff[e0] = ex2;
  }
  if (e1 < E) {
    R.eoff[e1] = o0 + n0;
    R.boff[e1] = ex2 + nb0;
  }
  // each slot's place in its expert's list, 512 slots per round
  for (int r0 = 0; r0 < S; r0 += kGThreads) {
    for (int i = threadIdx.x; i < kGWaves * E; i += kGThreads) R.mask[i / E][i % E] = 0ull;
    __syncthreads();
    const int s = r0 + (int)threadIdx.x;
    const bool live = s < S;
    const int e = live ? a.idx[s] : 0;
    if (live) atomicOr(&R.mask[wave][e], 1ull << lane);
    __syncthreads();
    if (live) {
      int pos = R.eoff[e] + R.run[e] + __popcll(R.mask[wave][e] & ((1ull << lane) - 1ull));
      for (int v = 0; v < wave; ++v) pos += __popcll(R.mask[v][e]);
      R.slotl[pos] = s;
    }
    __syncthreads();
    for (int x = threadIdx.x; x < E; x += kGThreads) {
      int add = 0;
#pragma unroll
      for (int v = 0; v < kGWaves; ++v) add += __popcll(R.mask[v][x]);
      R.run[x] += add;
    }
    __syncthreads();
  }
  // the token blocks of the two experts, with their slots
  int32_t *G = a.groups;
  if (threadIdx.x == 0) {
    G[0] = tot1 & 2047;
    G[1] = tot2;
  }
  for (int k = 0; k < nb0; ++k) {
    const int n = min(kTokBlock, n0 - kTokBlock * k), q = R.eoff[e0] + kTokBlock * k;
    int32_t *r = G + 2 + kBlkInts * (ex2 + k);
    r[0] = e0;
    r[1] = n;
#pragma unroll
    for (int u = 0; u < kTokBlock; ++u) r[2 + u] = R.slotl[q + min(u, n - 1)];
  }
  for (int k = 0; k < nb1; ++k) {
    const int n = min(kTokBlock, n1 - kTokBlock * k), q = R.eoff[e0] + n0 + kTokBlock * k;
    int32_t *r = G + 2 + kBlkInts * (ex2 + nb0 + k);
    r[0] = e1;
    r[1] = n;
#pragma unroll
    for (int u = 0; u < kTokBlock; ++u) r[2 + u] = R.slotl[q + min(u, n - 1)];
  }
}

// g2: gate/up + SwiGLU of 128 interleaved rows (64 pairs = group gi of the
// inter dimension) of one item's expert, for the item's tokens / slots.
// Wavefront w holds rows 16w .. 16w + 15. h vectors: slot s at index s,
// shared-expert token t at index S + t. TABLE: the routing kernels have written
// the routing and the grouping table already (large batches); IDX: the top-K kernel
// has written the routing and every workgroup groups the slots (at most 64) itself;
// otherwise every workgroup derives both when it meets its first routed item
// (route_small for batches of at most kTokBlock tokens, block_route for the others).
template <int BITS, int NGH, bool PRE, bool FULL, bool TABLE, bool IDX = false>
__global__ __launch_bounds__(kGThreads) void k_g2(const GroupArgs a) {
  // (NGH: the hidden groups ng rounded up to a power of two; FULL: ng == NGH)
  const int ng = FULL ? NGH : a.H / kGroup, ngi = a.I / kGroup;
  const size_t RB = (size_t)ng * gbytes<BITS>();
  // staged x, and before it the routing scratch
  constexpr size_t kXlBytes = MfmaRows<BITS, NGH>::XL + 16 > sizeof(RouteLds) ? MfmaRows<BITS, NGH>::XL + 16
                                                                               : sizeof(RouteLds);
  __shared__ __attribute__((aligned(16))) uint8_t xl[kXlBytes];
  __shared__ float2 xsl[kTokBlock * NGH + 1];
  __shared__ float2 hpart[kGWaves][kTokBlock];
  __shared__ __attribute__((aligned(16))) uint8_t wlds[kGWaves][kWaveLds];
  __shared__ int slotl[kRouteSlots], blk[kBlkInts * kRouteSlots];
  __shared__ int tokv[kTokBlock], hvl[kTokBlock], tokn[kTokBlock];
  static_assert(sizeof(RouteLds) <= sizeof(xl), "routing scratch fits the staging buffer");
  const bool sh = a.shared != nullptr;
  const int S = a.B * a.K;
  const int lane = lane_id(), wv = wave_in_block();
  const int n = lane & 15, qq = lane >> 4;
  // Work items: (token block, group gi of 64 gate/up pairs); first the shared
  // expert's token blocks (if any), then the routed ones. Persistent workgroups
  // take items in grid stride; a workgroup derives the routing (every one the
  // same; the one that meets the first routed item first publishes it) when it
  // meets its first routed item, so the shared expert's items stream at once.
  gtrace(a, 1, 0);
  const int sh_items = sh ? (a.B + kTokBlock - 1) / kTokBlock * ngi : 0;
  const int max_items = sh_items + S * ngi;
  const bool writer = (int)blockIdx.x == sh_items % (int)gridDim.x;
  int NB = -1;  // routing not derived yet
  // the token blocks {expert, n, slots}: in LDS (derived here) or the table in memory
  const int *btab = TABLE ? a.groups + 2 : blk;
  // A batch of at most kTokBlock tokens: every item's tokens are among them, so
  // their x is staged once, now, by the wavefronts past the batch's tokens
  // (wavefront t < B derives token t's top-K meanwhile), in token order; the
  // routing scratch then lives in the wavefronts' chunk regions instead of xl.
  using MR = MfmaRows<BITS, NGH, 1, FULL>;
  constexpr bool pre = PRE;  // (launched for batches of at most kTokBlock tokens)
  static_assert(sizeof(RouteSmallLds) <= sizeof(wlds), "routing scratch of a small batch fits the chunk regions");
  static_assert(sizeof(RouteSmallLds) <= sizeof(xl), "grouping scratch fits the staging buffer");
  if (pre && wv >= a.B) {  // (B <= kTokBlock < kGWaves: at least four such wavefronts)
    const int nst = (kGWaves - a.B) * kWave, st = (int)threadIdx.x - a.B * kWave;
    const int units = kParts * a.B * ng * 4;
    constexpr int kB = 12;
    for (int e0 = st; e0 < units; e0 += kB * nst) {
      uint4 v[kB];
      int dst[kB];
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const int ee = e0 + k * nst;
        const int e = min(ee, units - 1);
        const int vv = e / (ng * 4), rr = e - vv * (ng * 4);
        v[k] = *reinterpret_cast<const uint4 *>(a.xq + (size_t)vv * ng * 64 + 16 * rr);
        dst[k] = ee < units ? vv * MR::VS + 16 * rr : MR::XL;
      }
      asm volatile("" ::: "memory");
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const uint4 t = v[k];  // (through a local: a direct struct copy kept v in scratch memory)
        *reinterpret_cast<uint4 *>(xl + dst[k]) = t;
      }
    }
    // group sums of token u at u NGH + g, zero for the groups past ng
    for (int e = st; e < a.B * NGH; e += nst) {
      const int u = e / NGH, g = e - u * NGH;
      xsl[e] = g < ng ? reinterpret_cast<const float2 *>(a.xsum)[(size_t)u * ng + g] : make_float2(0.f, 0.f);
    }
  }
  // (items staged one by one) the next item's x is requested during this item's
  // last chunks, when its tokens are known: any next shared item, a routed one
  // once the routing is derived
  typename MR::XAhead ahead;
  bool have = false;
  int done = 0;  // items finished (for the trace)
  for (int item = blockIdx.x; item < max_items; item += gridDim.x) {
    GroupItem it;
    int gi;
    if (item < sh_items) {
      gi = item % ngi;
      it.expert = -1;
      it.q0 = kTokBlock * (item / ngi);
      it.n = min(kTokBlock, a.B - it.q0);
    } else {
      if (NB < 0) {
        if constexpr (TABLE)
          NB = __builtin_amdgcn_readfirstlane(a.groups[1]);
        else if constexpr (IDX)
          NB = group_from_idx(a, *reinterpret_cast<RouteSmallLds *>(xl), blk, writer);
        else if constexpr (PRE)
          NB = route_small(a, *reinterpret_cast<RouteSmallLds *>(&wlds[0][0]), blk, writer);
        else
          NB = block_route(a, *reinterpret_cast<RouteLds *>(xl), slotl, blk, writer);
        gtrace(a, 1, 1);
      }
      const int kb = (item - sh_items) / ngi;
      if (kb >= NB) break;  // (uniform) later items are past the last block
      gi = (item - sh_items) % ngi;
      // (uniform values: kept in scalar registers)
      it.expert = __builtin_amdgcn_readfirstlane(btab[kBlkInts * kb]);
      it.n = __builtin_amdgcn_readfirstlane(btab[kBlkInts * kb + 1]);
      it.q0 = kBlkInts * kb + 2;
    }
    const int T = it.n;
    const uint8_t *base = it.expert < 0  ? a.shared
                          : a.expert_ptr ? a.expert_ptr[it.expert]
                                         : a.bank + (size_t)it.expert * a.stride;
    const uint8_t *rec0 = base + (size_t)(128 * gi + 16 * __builtin_amdgcn_readfirstlane(wv)) * RB;
    // thread u < T: slot of item token u (unused for the shared expert, whose
    // item tokens are tokens q0 + u)
    const int sl = btab[it.expert < 0 ? 0 : it.q0 + min((int)threadIdx.x, T - 1)];
    // tables: the token whose x item token u takes, the index of its h vector
    auto fill = [&](int u) {
      tokv[u] = it.expert < 0 ? it.q0 + u : sl / a.K;
      hvl[u] = it.expert < 0 ? S + it.q0 + u : sl;
    };
    float tinv;  // RMS factor of the token of this lane's D rows
    auto after = [&]() { tinv = a.xinv[tokv[min(qq, T - 1)]]; };
    // the next item of this workgroup: its token count (0: not known yet, or none)
    // and where its tokens come from
    int Tn = 0, nq0 = 0;
    bool nsh = false;
    if constexpr (!PRE) {
      const int nitem = item + (int)gridDim.x;
      if (nitem < sh_items) {
        nsh = true;
        nq0 = kTokBlock * (nitem / ngi);
        Tn = min(kTokBlock, a.B - nq0);
      } else if (nitem < max_items && NB >= 0) {
        const int kbn = (nitem - sh_items) / ngi;
        if (kbn < NB) {
          nq0 = kBlkInts * kbn + 2;
          Tn = __builtin_amdgcn_readfirstlane(btab[kBlkInts * kbn + 1]);
        }
      }
    }
    auto filln = [&](int u) { tokn[u] = nsh ? nq0 + u : btab[nq0 + u] / a.K; };
    float y = 0.f;
    MR M;
    M.template run<PRE, !PRE>(ng, rec0, 0, a.xq, a.xsum, T, tokv, fill, after, [&](int) { y = M.y; }, xl, xsl,
                              wlds[wv], &ahead, &have, Tn, tokn, filln);
    // h = silu(gate) * up: gate rows are even, up rows odd (adjacent lanes); the
    // item's 64 pairs are one whole group of h (pair 8 wv + n / 2)
    float hv = 0.f;
    {
      const float yv = y * tinv;
      const float up = dpp_f<0xB1, 0xF>(yv, 0.f);  // partner row (quad_perm [1,0,3,2])
      if ((n & 1) == 0 && qq < T) hv = silu(yv) * up;
    }
    // per token: the group's sum of h and largest magnitude, over the even lanes
    // of each 16-lane row (odd lanes hold 0), then the wavefronts in order
    {
      float r = hv;
      int m = __float_as_int(fabsf(hv));
      r += dpp_f<0xB1, 0xF>(r, 0.f);  // lanes n, n^1
      m = max(m, dpp_i<0xB1, 0xF>(m, 0));
      r += dpp_f<0x4E, 0xF>(r, 0.f);  // n, n^2
      m = max(m, dpp_i<0x4E, 0xF>(m, 0));
      r += dpp_f<0x141, 0xF>(r, 0.f);  // row_half_mirror: n, 7-n
      m = max(m, dpp_i<0x141, 0xF>(m, 0));
      r += dpp_f<0x140, 0xF>(r, 0.f);  // row_mirror: n, 15-n
      m = max(m, dpp_i<0x140, 0xF>(m, 0));
      if (n == 0 && qq < T) hpart[wv][qq] = make_float2(r, __int_as_float(m));
    }
    // the h vector indices this thread stores to, read before the barrier: after it,
    // wavefront 0 may already be filling hvl with the next item's
    const int hv_lane = hvl[min(qq, T - 1)];
    const int hv_thr = hvl[min((int)threadIdx.x, T - 1)];
    __syncthreads();
    // h of this lane in integer form (its token's group shift), and per token the
    // group's factor and sum
    {
      const int u = min(qq, T - 1);
      int mb = __float_as_int(hpart[0][u].y);
#pragma unroll
      for (int v = 1; v < kGWaves; ++v) mb = max(mb, __float_as_int(hpart[v][u].y));
      const int k = group_shift(__int_as_float(mb));
      if ((n & 1) == 0 && qq < T) {
        const uint32_t d = digits3(hv, k);
        uint8_t *dst = a.hq + (size_t)(kParts * hv_lane) * a.I + 64 * gi + 8 * wv + (n >> 1);
#pragma unroll
        for (int p = 0; p < kParts; ++p) dst[(size_t)p * a.I] = (uint8_t)(d >> (8 * p));
      }
    }
    if ((int)threadIdx.x < T) {
      const int u = threadIdx.x;
      float sum = hpart[0][u].x;
      int mb = __float_as_int(hpart[0][u].y);
#pragma unroll
      for (int v = 1; v < kGWaves; ++v) {
        sum += hpart[v][u].x;
        mb = max(mb, __float_as_int(hpart[v][u].y));
      }
      const float amax = __int_as_float(mb);
      reinterpret_cast<float2 *>(a.hsum)[(size_t)hv_thr * ngi + gi] = make_float2(group_factor(amax, group_shift(amax)), sum);
    }
    if (done < 5) gtrace(a, 1, 2 + done);
    ++done;
  }
  gtrace(a, 1, 7);
}

// g3: down of 128 TILES rows (part rb: TILES tiles of 128, each wavefront 16
// rows of each) of one item's expert for the item's tokens / slots, from one
// staging of h: shared: d_shared[t][row] = sigma[t] * row . h_shared[t]; routed:
// partial[slot][row] = w[slot] * row . h[slot]. Workgroups: the shared
// expert's token blocks, then one per possible routed token block (those past
// G[1] exit at once), each times the H / (128 TILES) row parts. Two tiles per
// staging halve the staging overhead when there are many token blocks; with
// few, one tile per workgroup spreads the rows over more compute units.
template <int BITS, int NGI, int kG3Tiles, bool FULL>
__global__ __launch_bounds__(kGThreads) void k_g3(const GroupArgs a) {
  // (NGI: the inter groups ngi rounded up to a power of two; FULL: ngi == NGI)
  const int ngi = FULL ? NGI : a.I / kGroup;
  const size_t RB = (size_t)ngi * gbytes<BITS>();
  __shared__ __attribute__((aligned(16))) uint8_t xl[MfmaRows<BITS, NGI, kG3Tiles>::XL + 16];
  __shared__ float2 xsl[kTokBlock * NGI + 1];
  __shared__ __attribute__((aligned(16))) uint8_t wlds[kGWaves][kWaveLds];
  __shared__ int tokv[kTokBlock], oidx[kTokBlock];
  const int per = a.H / (128 * kG3Tiles);
  const bool sh = a.shared != nullptr;
  const int S = a.B * a.K;
  const int shb = sh ? (a.B + kTokBlock - 1) / kTokBlock : 0;
  const int ib = blockIdx.x / per, rb = blockIdx.x % per;
  const int32_t *G = a.groups;
  GroupItem it;
  if (ib < shb) {
    it.expert = -1;
    it.q0 = kTokBlock * ib;
    it.n = min(kTokBlock, a.B - it.q0);
  } else {
    const int kb = ib - shb;
    // (requested together with the slots below: one round trip)
    const int nb = G[1];
    it.expert = G[2 + kBlkInts * kb];
    it.n = G[2 + kBlkInts * kb + 1];
    it.q0 = 2 + kBlkInts * kb + 2;
    if (kb >= nb) return;  // uniform over the workgroup
  }
  gtrace(a, 2, 0);
  const int T = it.n;
  const int lane = lane_id(), wv = wave_in_block();
  const int n = lane & 15, qq = lane >> 4;
  const uint8_t *base = (it.expert < 0  ? a.shared
                         : a.expert_ptr ? a.expert_ptr[it.expert]
                                        : a.bank + (size_t)it.expert * a.stride) +
                        a.gu_bytes;
  const int row0 = 128 * kG3Tiles * rb + 16 * wv;  // this wavefront's first row of tile 0
  const uint8_t *rec0 = base + (size_t)row0 * RB;
  float *const outp = it.expert < 0 ? a.d_shared : a.partial;
  const float *const scl = it.expert < 0 ? a.sigma : a.w;
  const int sl = G[it.expert < 0 ? 0 : it.q0 + min((int)threadIdx.x, T - 1)];
  // tables: the h vector of item token u, and its output row (token or slot)
  auto fill = [&](int u) {
    tokv[u] = it.expert < 0 ? S + it.q0 + u : sl;
    oidx[u] = it.expert < 0 ? it.q0 + u : sl;
  };
  float osc;  // sigma (shared) or routing weight of this lane's D rows
  auto after = [&]() { osc = scl[oidx[min(qq, T - 1)]]; };
  MfmaRows<BITS, NGI, kG3Tiles, FULL> M;
  auto done = [&](int tile) {
    if (qq < T) outp[(size_t)oidx[qq] * a.H + row0 + 128 * tile + n] = osc * M.y;
  };
  M.template run<false>(ngi, rec0, (size_t)128 * RB, a.hq, a.hsum, T, tokv, fill, after, done, xl, xsl, wlds[wv]);
  gtrace(a, 2, 3);
}

// g4: out[t] = residual[t] + sum_k partial[t*K + k] (k ascending) + d_shared[t];
// KM: 8 for top_k <= 8, else kMaxTopK
template <int BITS, int KM>
__global__ __launch_bounds__(kBlock) void k_g4(const GroupArgs a) {
  const int f = blockIdx.x * kBlock + threadIdx.x;  // float4 index into [B][H]
  const int h4 = a.H / 4;
  if (f >= a.B * h4) return;
  const int t = f / h4, i = f - t * h4;
  // every load issued before the first add (clamped choices past K are not added)
  float4 p[KM];
#pragma unroll
  for (int k = 0; k < KM; ++k)
    p[k] = reinterpret_cast<const float4 *>(a.partial)[(size_t)(t * a.K + min(k, a.K - 1)) * h4 + i];
  const float4 q = reinterpret_cast<const float4 *>(a.shared ? a.d_shared : a.residual)[f];
  float4 o = reinterpret_cast<const float4 *>(a.residual)[f];
#pragma unroll
  for (int k = 0; k < KM; ++k) {
    if (k < a.K) {
      o.x += p[k].x;
      o.y += p[k].y;
      o.z += p[k].z;
      o.w += p[k].w;
    }
  }
  if (a.shared) {
    o.x += q.x;
    o.y += q.y;
    o.z += q.z;
    o.w += q.w;
  }
  reinterpret_cast<float4 *>(a.out)[f] = o;
}

// Compute units of the current device (cached per device): the persistent
// gate/up kernel runs one workgroup per compute unit (its LDS admits one).
inline int cu_count() {
  static int cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

// Launches of the grouped layer; NGH and NGI are the hidden and inter group
// counts rounded up to powers of two (the router and gate/up kernels depend on
// the first, the down kernel on the second).
template <int BITS>
struct GroupDispatch {
  // router + token preparation (sets a.n_router_blocks)
  template <int NGH>
  static void launch_g1(GroupArgs &a, hipStream_t s) {
    if (router_tiled(a.B)) {
      a.n_router_blocks = router_tiles(a.E, a.B) * a.logit_parts;
      hipLaunchKernelGGL(k_g1t<BITS>, dim3(a.n_router_blocks + a.B), dim3(kBlock), 0, s, a);
    } else {
      a.n_router_blocks = (a.E + g1_rows_per_block<NGH>() - 1) / g1_rows_per_block<NGH>();
      hipLaunchKernelGGL((k_g1<BITS, NGH>), dim3(a.n_router_blocks + a.B), dim3(kBlock), 0, s, a);
    }
  }

  static void launch_topk(const GroupArgs &a, hipStream_t s) {
    const dim3 grid((a.B + kGWaves - 1) / kGWaves);
    hipLaunchKernelGGL(k_topk<BITS>, grid, dim3(kGThreads), 0, s, a);
  }

  template <int NGH>
  static hipError_t front(GroupArgs a, hipStream_t s, int phases) {
    const bool sh = a.shared != nullptr;
    const int S = a.B * a.K;
    const int shb = sh ? (a.B + kTokBlock - 1) / kTokBlock : 0;  // shared token blocks
    if (phases & 1) launch_g1<NGH>(a, s);
    if (phases & 2) {
      const dim3 grid(std::min((shb + S) * (a.I / kGroup), cu_count()));
      const bool full = a.H == NGH * kGroup;
      if (S > kRouteSlots || a.B > kRouteTokens) {
        // large batches: the top-K kernel first; with at most 64 slots every gate/up
        // workgroup groups them itself from the indices (one wavefront's ranking),
        // else the grouping kernel writes the table first
        launch_topk(a, s);
        if (S <= kWave) {
          if (full)
            hipLaunchKernelGGL((k_g2<BITS, NGH, false, true, false, true>), grid, dim3(kGThreads), 0, s, a);
          else
            hipLaunchKernelGGL((k_g2<BITS, NGH, false, false, false, true>), grid, dim3(kGThreads), 0, s, a);
        } else {
          hipLaunchKernelGGL(k_group<BITS>, dim3(1), dim3(kGThreads), 0, s, a);
          if (full)
            hipLaunchKernelGGL((k_g2<BITS, NGH, false, true, true>), grid, dim3(kGThreads), 0, s, a);
          else
            hipLaunchKernelGGL((k_g2<BITS, NGH, false, false, true>), grid, dim3(kGThreads), 0, s, a);
        }
      } else if (a.B <= kTokBlock && full) {
        hipLaunchKernelGGL((k_g2<BITS, NGH, true, true, false>), grid, dim3(kGThreads), 0, s, a);
      } else if (a.B <= kTokBlock) {
        hipLaunchKernelGGL((k_g2<BITS, NGH, true, false, false>), grid, dim3(kGThreads), 0, s, a);
      } else if (full) {
        hipLaunchKernelGGL((k_g2<BITS, NGH, false, true, false>), grid, dim3(kGThreads), 0, s, a);
      } else {
        hipLaunchKernelGGL((k_g2<BITS, NGH, false, false, false>), grid, dim3(kGThreads), 0, s, a);
      }
    }
    return hipGetLastError();
  }

  template <int NGI>
  static hipError_t back(const GroupArgs &a, hipStream_t s, int phases) {
    const bool sh = a.shared != nullptr;
    const int S = a.B * a.K;
    const int shb = sh ? (a.B + kTokBlock - 1) / kTokBlock : 0;
    const int n4 = (a.B * (a.H / 4) + kBlock - 1) / kBlock;
    if (phases & 4) {
      const bool full = a.I == NGI * kGroup;
      const dim3 g1((shb + S) * (a.H / 128)), g2((shb + S) * (a.H / 256));
      if (a.B <= kDownOneTile && full)
        hipLaunchKernelGGL((k_g3<BITS, NGI, 1, true>), g1, dim3(kGThreads), 0, s, a);
      else if (a.B <= kDownOneTile)
        hipLaunchKernelGGL((k_g3<BITS, NGI, 1, false>), g1, dim3(kGThreads), 0, s, a);
      else if (full)
        hipLaunchKernelGGL((k_g3<BITS, NGI, 2, true>), g2, dim3(kGThreads), 0, s, a);
      else
        hipLaunchKernelGGL((k_g3<BITS, NGI, 2, false>), g2, dim3(kGThreads), 0, s, a);
      if (a.K <= 8)
        hipLaunchKernelGGL((k_g4<BITS, 8>), dim3(n4), dim3(kBlock), 0, s, a);
      else
        hipLaunchKernelGGL((k_g4<BITS, kMaxTopK>), dim3(n4), dim3(kBlock), 0, s, a);
    }
    return hipGetLastError();
  }
};

// The layer around a host step (see launch_group_route / launch_group_experts):
// the routing kernels always, the gate/up from the table.
template <int BITS>
struct SplitDispatch {
  template <int NGH>
  static hipError_t route(GroupArgs a, hipStream_t s) {
    GroupDispatch<BITS>::template launch_g1<NGH>(a, s);
    GroupDispatch<BITS>::launch_topk(a, s);
    return hipGetLastError();
  }
  template <int NGH>
  static hipError_t gateup(const GroupArgs &a, hipStream_t s) {
    const bool sh = a.shared != nullptr;
    const int S = a.B * a.K;
    const int shb = sh ? (a.B + kTokBlock - 1) / kTokBlock : 0;
    const dim3 grid(std::min((shb + S) * (a.I / kGroup), cu_count()));
    hipLaunchKernelGGL(k_group<BITS>, dim3(1), dim3(kGThreads), 0, s, a);
    if (a.H == NGH * kGroup)
      hipLaunchKernelGGL((k_g2<BITS, NGH, false, true, true>), grid, dim3(kGThreads), 0, s, a);
    else
      hipLaunchKernelGGL((k_g2<BITS, NGH, false, false, true>), grid, dim3(kGThreads), 0, s, a);
    return hipGetLastError();
  }
};

template <int BITS>
hipError_t group_route_b(const GroupArgs &a, hipStream_t s) {
  FMOE_NG_SWITCH(pad_groups(a.H / kGroup), SplitDispatch<BITS>::template route, a, s)
}

template <int BITS>
hipError_t group_experts_b(const GroupArgs &a, hipStream_t s) {
  hipError_t e;
  switch (pad_groups(a.H / kGroup)) {
    case 4: e = SplitDispatch<BITS>::template gateup<4>(a, s); break;
    case 8: e = SplitDispatch<BITS>::template gateup<8>(a, s); break;
    case 16: e = SplitDispatch<BITS>::template gateup<16>(a, s); break;
    case 32: e = SplitDispatch<BITS>::template gateup<32>(a, s); break;
    case 64: e = SplitDispatch<BITS>::template gateup<64>(a, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  FMOE_NG_SWITCH(pad_groups(a.I / kGroup), GroupDispatch<BITS>::template back, a, s, 4)
}

template <int BITS>
hipError_t group_front(const GroupArgs &a, hipStream_t s, int phases) {
  FMOE_NG_SWITCH(pad_groups(a.H / kGroup), GroupDispatch<BITS>::template front, a, s, phases)
}

template <int BITS>
hipError_t group_b(const GroupArgs &a, hipStream_t s, int phases) {
  const hipError_t e = group_front<BITS>(a, s, phases);
  if (e != hipSuccess) return e;
  FMOE_NG_SWITCH(pad_groups(a.I / kGroup), GroupDispatch<BITS>::template back, a, s, phases)
}

}  // namespace dev
}  // namespace fmoe
