// grouped_kernels.h -- the MoE layer for B > 1 tokens, with the tokens grouped
// by expert: every weight row of the layer (router, shared expert, each
// distinct routed expert) is read from HBM once per layer-step and applied to
// all the tokens that use it. Included by kernels_q4.hip / kernels_q2.hip after
// layer_kernels.h, which instantiate group_b<BITS>.
//
// Several tokens against one weight row make a (skinny) dense contraction, so
// the quantized experts run on the matrix cores: v_mfma_f32_16x16x32_bf16 with
//   B operand = 16 weight rows x 32 columns of codes, each code c (BITS bits) as
//               the exact bf16 value 1 + c / 2^BITS (c in the top mantissa bits,
//               so the constant 1 stays small next to the code's part);
//   A operand = 16 rows = 4 tokens x {hi, mid, lo, 0}, where hi = bf16(x),
//               mid = bf16(x - hi), lo = bf16(x - hi - mid): three bf16 parts
//               that add up to the fp32 x exactly (in the normal range);
//   D (fp32)  = per (token part, weight row) the sum over 32 columns.
// Two MFMAs cover a 64-column group; per (row, group) the epilogue applies the
// affine dequantization in the group-factored form
//   sum_j (c_j s + b) x_j = 2^BITS s * (sum_j (1 + c_j / 2^BITS) x'_j - sum_j x'_j) + b sum_j x_j
// where x' = hi + mid + lo is the value the matrix cores saw: the constant is
// taken off with the sum of x' itself, the bias with the fp32 group sum of x.
// Both sums are formed when x (or h) is prepared.
//
// Five launches:
//   g1  router logits and sigmoid(g . x) of every token (fp32 rows, VALU, the
//       tokens' x staged through LDS); other workgroups prepare each token's x
//       for the matrix cores: RMS factor, per-group sums, bf16 parts
//   g2r one workgroup: top-K of every token, then the distinct experts in
//       order of first use and, for each, the ascending list of the slots
//       (token t, choice k; slot = t*K + k) routed to it
//   g2  gate/up + SwiGLU of (shared expert or distinct expert, one group of 64
//       gate/up pairs = 128 rows, one 16-row tile per wavefront) for all the
//       tokens / slots using it; writes h as bf16 parts plus its group sums
//   g3  down of (shared expert or distinct expert, 128 rows): per token
//       sigma * (D_s h) into d_shared, per slot w * (D h) into partial[slot]
//   g4  out = residual + the K per-slot outputs in slot order + sigma * shared
#pragma once

#include "layer_kernels.h"

namespace fmoe {
namespace dev {

constexpr int kRouteThreads = 1024;
constexpr int kMaxSlots = kMaxTokens * kMaxTopK;
static_assert(kMaxSlots <= kRouteThreads, "one routing thread per slot");
constexpr int kRouterTok = 8;  // tokens whose fp32 x the router stages in LDS at a time
constexpr int kTokBlock = 16;  // tokens per pass over the weights
constexpr int kTokPass = 4;    // tokens per MFMA row block (4 rows each: hi, mid, lo, 0)
constexpr int kParts = 3;      // bf16 parts of an fp32 value
constexpr int kGThreads = 512;  // workgroup of the matrix-core kernels: 8 wavefronts
constexpr int kGWaves = kGThreads / kWave;
constexpr int kWaveLds = 16 * (2 * 8 * 16 + 16) + 16 * 9 * 4;  // LDS bytes per wavefront for a weight chunk
constexpr int kXBudget = 96 * 1024;                          // LDS bytes for staged x
constexpr int kXLds = kXBudget + kParts * kTokBlock * 16;    // plus 16 B of padding per vector
static_assert(kXBudget >= kParts * kTokBlock * 8 * 128, "x chunks of at least 8 groups");

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

// ------------------------------------------------------------------ bf16 and MFMA order

// bf16 bits of a finite float, round to nearest even.
__device__ __forceinline__ uint32_t bf16_bits(float v) {
  const uint32_t b = __float_as_uint(v);
  return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ float bf16_float(uint32_t h) { return __uint_as_float(h << 16); }

// v = bf16(p[0]) + bf16(p[1]) + bf16(p[2]) (exactly, for v in the normal range);
// rep = that sum as a float.
__device__ __forceinline__ void bf16_split3(float v, uint32_t (&p)[3], float &rep) {
  p[0] = bf16_bits(v);
  const float r1 = v - bf16_float(p[0]);
  p[1] = bf16_bits(r1);
  p[2] = bf16_bits(r1 - bf16_float(p[1]));
  rep = bf16_float(p[0]) + (bf16_float(p[1]) + bf16_float(p[2]));
}

// The MFMA order of a group's 64 columns: MFMA m (0, 1) takes from k-block q
// (0..3) the 8 consecutive columns starting at mfma_col(q, m), matching which
// packed codes lane (row, q) holds (see MCodes).
template <int BITS>
__device__ __forceinline__ int mfma_col(int q, int m) {
  return BITS == 4 ? 32 * (q >> 1) + 8 * (2 * (q & 1) + m) : 16 * q + 8 * m;
}
// Position (0..63) of column c of a group in MFMA order.
template <int BITS>
__device__ __forceinline__ int mfma_pos(int c) {
  int q, m;
  if constexpr (BITS == 4) {
    const int w = (c >> 3) & 3;
    q = 2 * (c >> 5) + (w >> 1);
    m = w & 1;
  } else {
    q = c >> 4;
    m = (c >> 3) & 1;
  }
  return (m * 4 + q) * 8 + (c & 7);
}

// One group of one weight row as held by lane (row, q): 16 codes for 4-bit (two
// words, one per MFMA; bytes 8 (q & 1) .. + 7 of half q >> 1 of the group),
// 16 codes for 2-bit (one word: word q of the group), and the (scale, bias) word.
struct MCodes {
  uint32_t c0, c1, sb;
};

// Four low bytes of bf16 values (0x80 | code in the top mantissa bits) in v ->
// two dwords of bf16 pairs: the high byte 0x3F above each (value 1 + c / 2^BITS);
// v_perm_b32 selects bytes 0..3 from v and 4..7 from the constant.
__device__ __forceinline__ void bf16_pairs(uint32_t v, uint32_t &p0, uint32_t &p1) {
  constexpr uint32_t K = 0x3F3F3F3Fu;
  p0 = __builtin_amdgcn_perm(K, v, 0x04010400u);
  p1 = __builtin_amdgcn_perm(K, v, 0x04030402u);
}

// The B operands of the group's two MFMAs (8 codes each, in column order).
template <int BITS>
__device__ __forceinline__ void mfma_codes(const MCodes &m, uint4 &u0, uint4 &u1) {
  // each byte's code moved to bits 6..(7 - BITS) of its byte, with bit 7 set
  // (the low bit of the bf16 exponent of 1.0)
  constexpr uint32_t E = 0x80808080u;
  if constexpr (BITS == 4) {
    bf16_pairs(((m.c0 << 3) & 0x78787878u) | E, u0.x, u0.y);
    bf16_pairs(((m.c0 >> 1) & 0x78787878u) | E, u0.z, u0.w);
    bf16_pairs(((m.c1 << 3) & 0x78787878u) | E, u1.x, u1.y);
    bf16_pairs(((m.c1 >> 1) & 0x78787878u) | E, u1.z, u1.w);
  } else {
    bf16_pairs(((m.c0 << 5) & 0x60606060u) | E, u0.x, u0.y);
    bf16_pairs(((m.c0 << 3) & 0x60606060u) | E, u0.z, u0.w);
    bf16_pairs(((m.c0 << 1) & 0x60606060u) | E, u1.x, u1.y);
    bf16_pairs(((m.c0 >> 1) & 0x60606060u) | E, u1.z, u1.w);
  }
}

// ------------------------------------------------------------------ matrix-core rows

// Workgroup-cooperative (kGThreads threads): one 16-row tile per wavefront
// (rows rec0 + r * RB, r = 0..15) against T <= kTokBlock vectors vec_of(u) of
// a prepared source: part k (0..2) at xq_base + (3 vec + k) * NG * 64; per
// group (sum x, sum x') at xs_base + 2 (vec * NG + g). The vectors are staged
// in LDS (xl: kXLds bytes, xsl: kTokBlock * NG entries) in chunks of as many
// groups as fit the budget: all of them for up to 4 tokens at NG = 64. On
// return lane (n = lane % 16, qq = lane / 16) holds in y[p] row n for token
// u = 4p + qq (meaningless for u >= T). Contains barriers: every thread of the
// workgroup calls it with the same T.
//
// Weights stream in chunks of CG groups. A wavefront loads a chunk of its 16
// rows with 16-byte loads over whole 16 CG-byte spans of each row (each load
// instruction covers complete cache lines), keeps DEPTH chunks in flight, and
// passes each chunk through its own LDS region (wl: kWaveLds bytes), from
// which lane (n, q) reads the codes of k-block q of row n. The loop has no
// branches around its loads, so every wait is exact; the empty asm statements
// keep the optimiser from moving the loads (and the reads of their results)
// away from where the pipeline needs them.
template <int BITS, int NG>
struct MfmaRows {
  static constexpr int CG = NG < 8 ? NG : 8;          // groups per chunk
  static constexpr int NC = NG / CG;                  // chunks per row
  static constexpr int DEPTH = NC < 2 ? NC : 2;       // chunks in flight
  static constexpr int HALVES = BITS == 4 ? 2 : 1;    // 16-byte code units per group
  static constexpr int NI = 16 * HALVES * CG / kWave; // 16-byte code loads per lane per chunk
  static constexpr int SBW = CG / 4;                  // scale/bias words per lane per chunk
  static constexpr int RB = NG * gbytes<BITS>();      // bytes per row record
  static constexpr int SBO = 16 * HALVES * NG;        // scale/bias words within a record
  static constexpr int RS = 16 * HALVES * CG + 16;    // LDS bytes per row of codes (padded)
  static constexpr int SBS = CG + 1;                  // LDS words per row of scale/bias (padded)
  static_assert(16 * RS + 64 * SBS <= kWaveLds, "chunk fits the wavefront's LDS region");
  static_assert(NC % DEPTH == 0, "whole rounds of chunks");

  struct Chunk {
    uint4 c[NI];
    uint32_t s[SBW];
  };

  float y[kTokBlock / kTokPass];

  template <typename VecOf>
  __device__ __forceinline__ static void stage(const uint16_t *__restrict__ xq_base, const float *__restrict__ xs_base,
                                               int T, VecOf vec_of, int g0, int gc, int vs, uint8_t *xl,
                                               float2 *xsl) {
    __syncthreads();  // earlier reads of xl / xsl are done
    const int units = kParts * T * gc * 8;  // 16-byte units; vector v = 3u + k: token u, part k
    for (int e = threadIdx.x; e < units; e += kGThreads) {
      const int v = e / (gc * 8), r = e - v * (gc * 8);
      const int gl = r >> 3, k16 = r & 7;
      const int vu = v / kParts, vk = v - kParts * vu;
      const uint16_t *src = xq_base + ((size_t)(kParts * vec_of(vu) + vk) * NG + g0 + gl) * 64 + 8 * k16;
      *reinterpret_cast<uint4 *>(xl + v * vs + gl * 128 + k16 * 16) = *reinterpret_cast<const uint4 *>(src);
    }
    for (int e = threadIdx.x; e < T * gc; e += kGThreads) {
      const int u = e / gc, gl = e - u * gc;
      xsl[u * NG + gl] = reinterpret_cast<const float2 *>(xs_base)[(size_t)vec_of(u) * NG + g0 + gl];
    }
    __syncthreads();
  }

  template <int NP, bool WHOLE, typename VecOf>
  __device__ __forceinline__ void loop(const uint8_t *__restrict__ rec0, const uint16_t *__restrict__ xq_base,
                                       const float *__restrict__ xs_base, int T, VecOf vec_of, int gc, int vs,
                                       uint8_t *xl, float2 *xsl, uint8_t *wl) {
    const int lane = lane_id();
    const int q = lane >> 4;  // k-block of the A / B operands; token of D
    const int i = lane & 15;  // A row (4 token + part) / weight row of B and D
    int aoff[NP], xoff[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int ua = min(kTokPass * p + (i >> 2), T - 1), ka = min(i & 3, kParts - 1);
      aoff[p] = (kParts * ua + ka) * vs + q * 16;
      xoff[p] = min(kTokPass * p + q, T - 1) * NG;
    }
    // this lane's share of a chunk: code unit u = 64 k + lane is (row, half, group)
    // = (u / (HALVES CG), u / CG % HALVES, u % CG); scale/bias: row lane / 4, words
    // SBW (lane % 4) .. + SBW - 1
    int goff[NI], loff[NI];
#pragma unroll
    for (int k = 0; k < NI; ++k) {
      const int u = kWave * k + lane;
      const int j = u % CG, rh = u / CG;
      const int r = rh / HALVES, h = rh % HALVES;
      goff[k] = r * RB + 16 * (h * NG + j);
      loff[k] = r * RS + 16 * (h * CG + j);
    }
    const int sr = lane >> 2, sp = lane & 3;
    const int gsoff = sr * RB + SBO + 4 * SBW * sp;
    const int lsoff = 16 * RS + 4 * (sr * SBS + SBW * sp);
    // where lane (n = i, q) reads group j of the chunk in wl
    const int rcode = BITS == 4 ? i * RS + 16 * (q >> 1) * CG + 8 * (q & 1) : i * RS + 4 * q;
    const int rsb = 16 * RS + 4 * i * SBS;

    auto load_chunk = [&](int c, Chunk &k) {
#pragma unroll
      for (int t = 0; t < NI; ++t) k.c[t] = *reinterpret_cast<const uint4 *>(rec0 + goff[t] + 16 * CG * c);
      if constexpr (SBW == 2) {
        const uint2 v = *reinterpret_cast<const uint2 *>(rec0 + gsoff + 4 * CG * c);
        k.s[0] = v.x;
        k.s[1] = v.y;
      } else {
        k.s[0] = *reinterpret_cast<const uint32_t *>(rec0 + gsoff + 4 * CG * c);
      }
    };
    Chunk ring[DEPTH];
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      load_chunk(d, ring[d]);
      asm volatile("" ::: "memory");
    }
#pragma unroll 1
    for (int cb = 0; cb < NC; cb += DEPTH) {
#pragma unroll
      for (int d = 0; d < DEPTH; ++d) {
        const int c = cb + d;
        if (!WHOLE && c > 0 && ((c * CG) & (gc - 1)) == 0) stage(xq_base, xs_base, T, vec_of, c * CG, gc, vs, xl, xsl);
        // chunk c arrives here; into this wavefront's LDS region (the reads of
        // the previous chunk were issued before, and LDS keeps a wavefront's order)
#pragma unroll
        for (int t = 0; t < NI; ++t) {
          asm volatile("" : "+v"(ring[d].c[t].x), "+v"(ring[d].c[t].y), "+v"(ring[d].c[t].z), "+v"(ring[d].c[t].w));
          *reinterpret_cast<uint4 *>(wl + loff[t]) = ring[d].c[t];
        }
#pragma unroll
        for (int t = 0; t < SBW; ++t) {
          asm volatile("" : "+v"(ring[d].s[t]));
          *reinterpret_cast<uint32_t *>(wl + lsoff + 4 * t) = ring[d].s[t];
        }
        // refill (a clamped chunk past the end)
        load_chunk(min(c + DEPTH, NC - 1), ring[d]);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int j = 0; j < CG; ++j) {
          const int g = c * CG + j;
          const int gl = WHOLE ? g : (g & (gc - 1));
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
          uint4 u0, u1;
          mfma_codes<BITS>(m, u0, u1);
          const float s = scale_of(m.sb) * (float)(1 << BITS);  // exact (power of two)
          const float ns = -s;
          const float bi = bias_of(m.sb);
          const bf16x8_t b0 = __builtin_bit_cast(bf16x8_t, u0), b1 = __builtin_bit_cast(bf16x8_t, u1);
#pragma unroll
          for (int p = 0; p < NP; ++p) {
            const uint8_t *src = xl + aoff[p] + gl * 128;
            const bf16x8_t A0 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(src));
            const bf16x8_t A1 = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const uint4 *>(src + 64));
            const float2 X = xsl[xoff[p] + gl];
            f32x4_t dd = {0.f, 0.f, 0.f, 0.f};
            dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, b0, dd, 0, 0, 0);
            dd = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, b1, dd, 0, 0, 0);
            y[p] = fmaf(s, dd[0] + (dd[1] + dd[2]), fmaf(ns, X.y, fmaf(bi, X.x, y[p])));
          }
        }
      }
    }
  }

  // rec0: record of the wavefront's first row; wl: its LDS region
  template <typename VecOf>
  __device__ __forceinline__ void run(const uint8_t *__restrict__ rec0, const uint16_t *__restrict__ xq_base,
                                      const float *__restrict__ xs_base, int T, VecOf vec_of, uint8_t *xl,
                                      float2 *xsl, uint8_t *wl) {
    int gc = NG;  // groups per staged chunk of x (a power of two, a multiple of CG)
    while (gc > CG && kParts * T * gc * 128 > kXBudget) gc >>= 1;
    const int vs = gc * 128 + 16;  // LDS bytes per staged vector
#pragma unroll
    for (int p = 0; p < kTokBlock / kTokPass; ++p) y[p] = 0.f;
    stage(xq_base, xs_base, T, vec_of, 0, gc, vs, xl, xsl);
    const int np = (T + kTokPass - 1) / kTokPass;
    const bool whole = gc == NG;
    if (np == 1) {
      if (whole)
        loop<1, true>(rec0, xq_base, xs_base, T, vec_of, gc, vs, xl, xsl, wl);
      else
        loop<1, false>(rec0, xq_base, xs_base, T, vec_of, gc, vs, xl, xsl, wl);
    } else if (np == 2) {
      if (whole)
        loop<2, true>(rec0, xq_base, xs_base, T, vec_of, gc, vs, xl, xsl, wl);
      else
        loop<2, false>(rec0, xq_base, xs_base, T, vec_of, gc, vs, xl, xsl, wl);
    } else if (np == 3) {
      if (whole)
        loop<3, true>(rec0, xq_base, xs_base, T, vec_of, gc, vs, xl, xsl, wl);
      else
        loop<3, false>(rec0, xq_base, xs_base, T, vec_of, gc, vs, xl, xsl, wl);
    } else {
      if (whole)
        loop<4, true>(rec0, xq_base, xs_base, T, vec_of, gc, vs, xl, xsl, wl);
      else
        loop<4, false>(rec0, xq_base, xs_base, T, vec_of, gc, vs, xl, xsl, wl);
    }
  }
};

// ------------------------------------------------------------------ g1

// g1: workgroups [0, n_router_blocks): router rows (one fp32 row per
// wavefront; row E is the gate vector) for every token. Workgroups
// n_router_blocks + t: token t's x for the matrix cores (RMS factor, per-group
// sums of x, hi/lo bf16 parts in MFMA order).
template <int BITS, int NGH>
__global__ __launch_bounds__(kBlock) void k_g1(const GroupArgs a) {
  constexpr int NT = NGH / 4;
  constexpr int H = NGH * kGroup;
  __shared__ float xl[kRouterTok][NGH * kXPad];
  __shared__ float part[kRouterTok][kWavesPerBlock];
  const int lane = lane_id();
  const bool rms = a.rms_eps >= 0.f;
  if ((int)blockIdx.x >= a.n_router_blocks) {
    // ---- input preparation of token t
    const int t = blockIdx.x - a.n_router_blocks;
    const float *xt = a.x + (size_t)t * H;
    constexpr int UNITS = NGH * 8;  // 8 columns each, in MFMA order: unit = 8g + 4m + q
    float ss = 0.f;
    for (int u0 = 0; u0 < UNITS; u0 += kBlock) {
      const int u = u0 + threadIdx.x;
      const bool ok = u < UNITS;
      const int uc = ok ? u : UNITS - 1;
      const int g = uc >> 3, mq = uc & 7;
      const int c = 64 * g + mfma_col<BITS>(mq & 3, mq >> 2);
      const float4 v0 = *reinterpret_cast<const float4 *>(xt + c);
      const float4 v1 = *reinterpret_cast<const float4 *>(xt + c + 4);
      const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      uint32_t pt[8][3];
      float sum = 0.f, rep = 0.f;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        float r;
        bf16_split3(f[j], pt[j], r);
        sum += f[j];
        rep += r;
        if (ok) ss = fmaf(f[j], f[j], ss);
      }
      // group sums: the group's 8 units are 8 consecutive threads
      sum = seg_allreduce<8>(sum);
      rep = seg_allreduce<8>(rep);
      if (ok) {
        uint16_t *dst = a.xq + ((size_t)(kParts * t) * NGH + g) * 64 + 8 * mq;
#pragma unroll
        for (int k = 0; k < kParts; ++k) {
          const uint4 v4 = {pt[0][k] | pt[1][k] << 16, pt[2][k] | pt[3][k] << 16, pt[4][k] | pt[5][k] << 16,
                            pt[6][k] | pt[7][k] << 16};
          *reinterpret_cast<uint4 *>(dst + (size_t)k * NGH * 64) = v4;
        }
        if (mq == 0) reinterpret_cast<float2 *>(a.xsum)[(size_t)t * NGH + g] = make_float2(sum, rep);
      }
    }
    ss = seg_reduce<kWave>(ss);
    if (lane == kWave - 1) part[0][wave_in_block()] = ss;
    __syncthreads();
    if (threadIdx.x == 0) a.xinv[t] = rms ? rms_inv(part[0], H, a.rms_eps) : 1.f;
    return;
  }
  // ---- router rows
  const int n_rows = a.E + (a.gvec ? 1 : 0);
  const int row = blockIdx.x * kWavesPerBlock + wave_in_block();
  const int rr = min(row, n_rows - 1);
  const float *src = rr == a.E ? a.gvec : a.router + (size_t)rr * H;
  float4 wr[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) wr[t] = reinterpret_cast<const float4 *>(src)[lane + 64 * t];
  for (int t0 = 0; t0 < a.B; t0 += kRouterTok) {
    const int nt = min(kRouterTok, a.B - t0);
    if (t0 > 0) __syncthreads();  // the previous chunk's reads of xl are done
    for (int j = 0; j < nt; ++j) {
      if (rms)
        stage_vec<NGH, true>(a.x + (size_t)(t0 + j) * H, xl[j], part[j]);
      else
        stage_vec<NGH, false>(a.x + (size_t)(t0 + j) * H, xl[j], part[j]);
    }
    __syncthreads();
    for (int j = 0; j < nt; ++j) {
      const float inv = rms ? rms_inv(part[j], H, a.rms_eps) : 1.f;
      float acc = 0.f;
#pragma unroll
      for (int q = 0; q < NT; ++q) {
        const float4 xv = *reinterpret_cast<const float4 *>(&xl[j][lds_index(4 * lane + 256 * q)]);
        acc = fmaf(wr[q].x, xv.x * inv, acc);
        acc = fmaf(wr[q].y, xv.y * inv, acc);
        acc = fmaf(wr[q].z, xv.z * inv, acc);
        acc = fmaf(wr[q].w, xv.w * inv, acc);
      }
      const float d = seg_reduce<kWave>(acc);
      if (lane == kWave - 1 && row < n_rows) {
        if (row == a.E)
          a.sigma[t0 + j] = 1.f / (1.f + expf(-d));
        else
          a.logits[(size_t)(t0 + j) * a.E + row] = d;
      }
    }
  }
}

// ------------------------------------------------------------------ g2r

// g2r: one workgroup of kRouteThreads. Top-K of each token (one wavefront per
// token), then the grouping, deterministic whatever the thread timing:
//  - first[e] = the lowest slot routed to expert e (an atomic minimum);
//  - the slots with first[e] == slot lead their expert; the leaders, in slot
//    order, number the distinct experts 0..D-1;
//  - every slot's position in its expert's list = the number of lower slots
//    routed to the same expert, so each list is in ascending slot order.
template <int BITS>  // (instantiated per bit width, like the rest of the layer)
__global__ __launch_bounds__(kRouteThreads) void k_g2r(const GroupArgs a) {
  constexpr int NW = kRouteThreads / kWave;
  __shared__ int first[kMaxExperts];
  __shared__ int sidx[kMaxSlots];
  __shared__ int rank_of[kMaxSlots];
  __shared__ int cnt[kMaxSlots];
  __shared__ int off[kMaxSlots + 1];
  __shared__ int wsum[NW];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int S = a.B * a.K;
  for (int t = wave; t < a.B; t += NW) {
    int idx[kMaxTopK];
    float w[kMaxTopK];
    wave_topk_lds(a.logits + (size_t)t * a.E, a.E, a.K, idx, w);
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j == lane && j < a.K) {
        const int s = t * a.K + j;
        a.idx[s] = idx[j];
        a.w[s] = w[j];
        if (a.out_idx) a.out_idx[s] = idx[j];
        if (a.out_w) a.out_w[s] = w[j];
        sidx[s] = idx[j];
      }
  }
  for (int e = threadIdx.x; e < a.E; e += kRouteThreads) first[e] = 0x7FFFFFFF;
  __syncthreads();
  const int s = threadIdx.x;
  if (s < S) atomicMin(&first[sidx[s]], s);
  __syncthreads();
  const bool lead = s < S && first[sidx[s]] == s;
  const unsigned long long bl = __ballot(lead);
  if (lane == 0) wsum[wave] = __popcll(bl);
  __syncthreads();
  int before = 0, D = 0;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    before += v < wave ? wsum[v] : 0;
    D += wsum[v];
  }
  const int rank = before + __popcll(bl & ((1ull << lane) - 1ull));
  if (lead) {
    rank_of[s] = rank;
    cnt[rank] = 0;
  }
  __syncthreads();
  int r = 0, pos = 0;
  if (s < S) {
    const int e = sidx[s];
    r = rank_of[first[e]];
    for (int q = first[e]; q < s; ++q) pos += sidx[q] == e;
    atomicAdd(&cnt[r], 1);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int o = 0;
    for (int q = 0; q < D; ++q) {
      off[q] = o;
      o += cnt[q];
    }
    off[D] = o;
  }
  __syncthreads();
  int32_t *G = a.groups;
  if (threadIdx.x == 0) G[0] = D;
  if (lead) G[1 + rank] = sidx[s];
  if ((int)threadIdx.x <= D) G[1 + S + threadIdx.x] = off[threadIdx.x];
  if (s < S) G[1 + S + (S + 1) + off[r] + pos] = s;
}

// ------------------------------------------------------------------ g2, g3

// Work of one owner: the shared expert (owner 0 when there is one; its tokens
// 0..B-1) or distinct expert d (its slot list).
struct GroupItem {
  int expert;  // -1: the shared expert
  int q0, n;   // slot-list range (routed) or tokens 0..B-1 (shared)
};

// false if the owner does not exist (past the D distinct experts)
__device__ __forceinline__ bool group_item(const GroupArgs &a, int owner, GroupItem &it) {
  const int S = a.B * a.K;
  const bool sh = a.shared != nullptr;
  if (sh && owner == 0) {
    it.expert = -1;
    it.q0 = 0;
    it.n = a.B;
    return true;
  }
  const int d = owner - (sh ? 1 : 0);
  const int32_t *G = a.groups;
  if (d >= G[0]) return false;
  it.expert = G[1 + d];
  it.q0 = G[1 + S + d];
  it.n = G[1 + S + d + 1] - it.q0;
  return true;
}

// g2: gate/up + SwiGLU of 128 interleaved rows (64 pairs = group gi of the
// inter dimension) of one owner, for all its tokens / slots. Wavefront w holds
// rows 16w .. 16w + 15. h vectors: slot s at index s, shared-expert token t at
// index S + t.
template <int BITS, int NGH, int NGI>
__global__ __launch_bounds__(kGThreads) void k_g2(const GroupArgs a) {
  constexpr size_t RB = (size_t)NGH * gbytes<BITS>();
  __shared__ __attribute__((aligned(16))) uint8_t xl[kXLds];
  __shared__ float2 xsl[kTokBlock * NGH];
  __shared__ float2 hpart[kGWaves][kTokBlock];
  __shared__ __attribute__((aligned(16))) uint8_t wlds[kGWaves][kWaveLds];
  GroupItem it;
  const int owner = blockIdx.x / NGI, gi = blockIdx.x % NGI;
  if (!group_item(a, owner, it)) return;  // uniform over the workgroup
  const int S = a.B * a.K;
  const int lane = lane_id(), wv = wave_in_block();
  const int n = lane & 15, qq = lane >> 4;
  const uint8_t *base = it.expert < 0 ? a.shared : a.bank + (size_t)it.expert * a.stride;
  const uint8_t *rec0 = base + (size_t)(128 * gi + 16 * wv) * RB;
  const int32_t *slots = a.groups + 1 + S + (S + 1);
  for (int tb = 0; tb < it.n; tb += kTokBlock) {
    const int T = min(kTokBlock, it.n - tb);
    // the token whose x item token u takes, and the index of its h vector
    auto xtok = [&](int u) { return it.expert < 0 ? tb + u : slots[it.q0 + tb + u] / a.K; };
    auto hvec = [&](int u) { return it.expert < 0 ? S + tb + u : slots[it.q0 + tb + u]; };
    MfmaRows<BITS, NGH> M;
    M.run(rec0, a.xq, a.xsum, T, xtok, xl, xsl, wlds[wv]);
    // h = silu(gate) * up: gate rows are even, up rows odd (adjacent lanes)
    float hs[kTokBlock / kTokPass] = {}, hr[kTokBlock / kTokPass] = {};
#pragma unroll
    for (int p = 0; p < kTokBlock / kTokPass; ++p) {
      const int u = kTokPass * p + qq;
      const float inv = u < T ? a.xinv[xtok(u)] : 0.f;
      const float yv = M.y[p] * inv;
      const float up = dpp_f<0xB1, 0xF>(yv, 0.f);  // partner row (quad_perm [1,0,3,2])
      if ((n & 1) == 0 && u < T) {
        const float h = silu(yv) * up;
        const int pl = 8 * wv + (n >> 1);  // pair within the group
        uint16_t *dst = a.hq + (size_t)(kParts * hvec(u)) * a.I + 64 * gi + mfma_pos<BITS>(pl);
        uint32_t pt[3];
        float r;
        bf16_split3(h, pt, r);
#pragma unroll
        for (int k = 0; k < kParts; ++k) dst[(size_t)k * a.I] = (uint16_t)pt[k];
        hs[p] += h;
        hr[p] += r;
      }
    }
    // group sums of h: the even lanes of each 16-lane row (odd lanes hold 0), then
    // the wavefronts in order
#pragma unroll
    for (int p = 0; p < kTokBlock / kTokPass; ++p) {
      float r = hs[p], e = hr[p];
      r += dpp_f<0xB1, 0xF>(r, 0.f);   // lanes n, n^1
      e += dpp_f<0xB1, 0xF>(e, 0.f);
      r += dpp_f<0x4E, 0xF>(r, 0.f);   // n, n^2
      e += dpp_f<0x4E, 0xF>(e, 0.f);
      r += dpp_f<0x141, 0xF>(r, 0.f);  // row_half_mirror: n, 7-n
      e += dpp_f<0x141, 0xF>(e, 0.f);
      r += dpp_f<0x140, 0xF>(r, 0.f);  // row_mirror: n, 15-n
      e += dpp_f<0x140, 0xF>(e, 0.f);
      const int u = kTokPass * p + qq;
      if (n == 0 && u < T) hpart[wv][u] = make_float2(r, e);
    }
    __syncthreads();
    if ((int)threadIdx.x < T) {
      const int u = threadIdx.x;
      float2 t = hpart[0][u];
#pragma unroll
      for (int v = 1; v < kGWaves; ++v) {
        t.x += hpart[v][u].x;
        t.y += hpart[v][u].y;
      }
      reinterpret_cast<float2 *>(a.hsum)[(size_t)hvec(u) * NGI + gi] = t;
    }
  }
}

// g3: down of 128 rows (part rb) of one owner for all its tokens / slots:
// shared: d_shared[t][row] = sigma[t] * row . h_shared[t]; routed:
// partial[slot][row] = w[slot] * row . h[slot]. Wavefront w holds rows 16w .. +15.
template <int BITS, int NGI>
__global__ __launch_bounds__(kGThreads) void k_g3(const GroupArgs a) {
  constexpr size_t RB = (size_t)NGI * gbytes<BITS>();
  __shared__ __attribute__((aligned(16))) uint8_t xl[kXLds];
  __shared__ float2 xsl[kTokBlock * NGI];
  __shared__ __attribute__((aligned(16))) uint8_t wlds[kGWaves][kWaveLds];
  const int per = a.H / 128;
  GroupItem it;
  const int owner = blockIdx.x / per, rb = blockIdx.x % per;
  if (!group_item(a, owner, it)) return;
  const int S = a.B * a.K;
  const int lane = lane_id(), wv = wave_in_block();
  const int n = lane & 15, qq = lane >> 4;
  const uint8_t *base = (it.expert < 0 ? a.shared : a.bank + (size_t)it.expert * a.stride) + a.gu_bytes;
  const int row = 128 * rb + 16 * wv + n;
  const uint8_t *rec0 = base + (size_t)(128 * rb + 16 * wv) * RB;
  const int32_t *slots = a.groups + 1 + S + (S + 1);
  for (int tb = 0; tb < it.n; tb += kTokBlock) {
    const int T = min(kTokBlock, it.n - tb);
    auto hvec = [&](int u) { return it.expert < 0 ? S + tb + u : slots[it.q0 + tb + u]; };
    MfmaRows<BITS, NGI> M;
    M.run(rec0, a.hq, a.hsum, T, hvec, xl, xsl, wlds[wv]);
#pragma unroll
    for (int p = 0; p < kTokBlock / kTokPass; ++p) {
      const int u = kTokPass * p + qq;
      if (u < T) {
        if (it.expert < 0) {
          a.d_shared[(size_t)(tb + u) * a.H + row] = a.sigma[tb + u] * M.y[p];
        } else {
          const int slot = slots[it.q0 + tb + u];
          a.partial[(size_t)slot * a.H + row] = a.w[slot] * M.y[p];
        }
      }
    }
  }
}

// g4: out[t] = residual[t] + sum_k partial[t*K + k] (k ascending) + d_shared[t]
template <int BITS>
__global__ __launch_bounds__(kBlock) void k_g4(const GroupArgs a) {
  const int f = blockIdx.x * kBlock + threadIdx.x;  // float4 index into [B][H]
  const int h4 = a.H / 4;
  if (f >= a.B * h4) return;
  const int t = f / h4, i = f - t * h4;
  float4 o = reinterpret_cast<const float4 *>(a.residual)[f];
  for (int k = 0; k < a.K; ++k) {
    const float4 p = reinterpret_cast<const float4 *>(a.partial)[(size_t)(t * a.K + k) * h4 + i];
    o.x += p.x;
    o.y += p.y;
    o.z += p.z;
    o.w += p.w;
  }
  if (a.shared) {
    const float4 q = reinterpret_cast<const float4 *>(a.d_shared)[f];
    o.x += q.x;
    o.y += q.y;
    o.z += q.z;
    o.w += q.w;
  }
  reinterpret_cast<float4 *>(a.out)[f] = o;
}

template <int BITS>
struct GroupDispatch {
  template <int NGH, int NGI>
  static hipError_t layer(GroupArgs a, hipStream_t s, int phases) {
    const bool sh = a.shared != nullptr;
    const int S = a.B * a.K;
    const int owners = (S < a.E ? S : a.E) + (sh ? 1 : 0);
    a.n_router_blocks = blocks_for(a.E + (sh ? 1 : 0));
    const int n4 = (a.B * (a.H / 4) + kBlock - 1) / kBlock;
    if (phases & 1)
      hipLaunchKernelGGL((k_g1<BITS, NGH>), dim3(a.n_router_blocks + a.B), dim3(kBlock), 0, s, a);
    if (phases & 2) {
      hipLaunchKernelGGL(k_g2r<BITS>, dim3(1), dim3(kRouteThreads), 0, s, a);
      hipLaunchKernelGGL((k_g2<BITS, NGH, NGI>), dim3(owners * NGI), dim3(kGThreads), 0, s, a);
    }
    if (phases & 4) {
      hipLaunchKernelGGL((k_g3<BITS, NGI>), dim3(owners * (a.H / 128)), dim3(kGThreads), 0, s, a);
      hipLaunchKernelGGL(k_g4<BITS>, dim3(n4), dim3(kBlock), 0, s, a);
    }
    return hipGetLastError();
  }

  template <int NGH>
  static hipError_t layer_h(const GroupArgs &a, hipStream_t s, int phases) {
    switch (a.I / kGroup) {
      case 4: return layer<NGH, 4>(a, s, phases);
      case 8: return layer<NGH, 8>(a, s, phases);
      case 16: return layer<NGH, 16>(a, s, phases);
      case 32: return layer<NGH, 32>(a, s, phases);
      case 64: return layer<NGH, 64>(a, s, phases);
      default: return hipErrorInvalidValue;
    }
  }
};

template <int BITS>
hipError_t group_b(const GroupArgs &a, hipStream_t s, int phases) {
  FMOE_NG_SWITCH(a.H / kGroup, GroupDispatch<BITS>::template layer_h, a, s, phases)
}

}  // namespace dev
}  // namespace fmoe
