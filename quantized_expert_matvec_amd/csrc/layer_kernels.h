// layer_kernels.h -- templated HIP kernels of the MoE layer (one token) and their
// host-side dispatch. Included by one translation unit per bit width
// (kernels_q4.hip, kernels_q2.hip), which instantiate the *_b<BITS> entries.
//
// A layer is three launches:
//   phase 1  router logits (RMS scaling of the incoming h fused), x in digit
//            form for phase 2, sigmoid(g . x)
//   phase 2  top-K (re-derived by one wavefront of every routed block from the
//            logits), routed gate/up + SwiGLU; shared expert gate/up + SwiGLU in
//            blocks of their own, which need no routing
//   phase 3  routed and shared down + weighted combine + residual
// Each block has one role. Loads go out in the order they are needed (what the
// block must wait for first, then the weights), every group of loads before the
// first use of any of them; a block stages the vector it needs in LDS once (one
// coalesced read instead of one per wavefront; padded rows of 68 floats make the
// per-lane 128-bit slice reads conflict-free). The row count per wavefront is
// fixed at compile time so the code is straight-line and the compiler cannot
// sink loads toward their uses.
#pragma once

#include "device.h"
#include "kernels.h"

namespace fmoe {
namespace dev {

constexpr int kXPad = 68;               // LDS floats per 64-value group (4 floats of padding)
constexpr int kWavesPerBlock = kBlock / kWave;

__device__ __forceinline__ int wave_in_block() { return threadIdx.x >> 6; }
__device__ __forceinline__ int lds_index(int c) { return (c >> 6) * kXPad + (c & 63); }

// Two-step staging, so that a wavefront can issue the vector's loads before its
// weight loads (memory counters complete in order: waiting for the vector then
// does not wait for the weights). N4 = float4s per thread.
template <int N4>
struct Staged {
  float4 v[N4];
};

// The loads are unconditional (indices clamped to the vector), so that no branch
// hides them from the compiler's memory-counter bookkeeping: waiting for them
// then does not also wait for loads issued after them.
template <int N4, int BS = kBlock>
__device__ __forceinline__ void stage_load(const float *__restrict__ src, int nf4, Staged<N4> &st) {
#pragma unroll
  for (int k = 0; k < N4; ++k) {
    const int f = min((int)threadIdx.x + BS * k, nf4 - 1);
    st.v[k] = reinterpret_cast<const float4 *>(src)[f];
  }
}

// Store into padded LDS rows; with SUMSQ, the block's sum of squares of the
// vector is formed in a fixed order (each thread over its float4s, DPP within the
// wavefront): part[] receives one partial per wavefront, which rms_inv adds in
// order after the caller's barrier.
template <int N4, bool SUMSQ, int BS = kBlock>
__device__ __forceinline__ void stage_store(const Staged<N4> &st, int nf4, float *lds, float *part) {
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < N4; ++k) {
    const int f = threadIdx.x + BS * k;
    if (f < nf4) {
      const float4 v = st.v[k];
      *reinterpret_cast<float4 *>(&lds[lds_index(4 * f)]) = v;
      if constexpr (SUMSQ) ss += (v.x * v.x + v.y * v.y) + (v.z * v.z + v.w * v.w);
    }
  }
  if constexpr (SUMSQ) {
    ss = seg_reduce<kWave>(ss);
    if (lane_id() == kWave - 1) part[wave_in_block()] = ss;
  }
}

// Store into padded LDS rows, and each 64-value group's sum into gsum[]: a
// thread's float4 sum ((x + y) + (z + w)), then DPP over the 16 consecutive
// threads that hold the group (nf4 a multiple of 16, BS of 64).
template <int N4, int BS>
__device__ __forceinline__ void stage_store_gsum(const Staged<N4> &st, int nf4, float *lds, float *gsum) {
#pragma unroll
  for (int k = 0; k < N4; ++k) {
    const int f = threadIdx.x + BS * k;
    const float4 v = st.v[k];
    if (f < nf4) *reinterpret_cast<float4 *>(&lds[lds_index(4 * f)]) = v;
    const float t = seg_reduce<16>((v.x + v.y) + (v.z + v.w));
    if (f < nf4 && seg_last<16>(lane_id())) gsum[f >> 4] = t;
  }
}

// Lane's slice x[64g .. 64g+63] from padded LDS, with its sum given.
__device__ __forceinline__ void read_slice_sum(const float *lds, int g, float sum, XSlice &xs) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 t = *reinterpret_cast<const float4 *>(&lds[g * kXPad + 4 * i]);
    xs.v[4 * i] = t.x;
    xs.v[4 * i + 1] = t.y;
    xs.v[4 * i + 2] = t.z;
    xs.v[4 * i + 3] = t.w;
  }
  xs.sum = sum;
}

// Store into unpadded LDS (a plain copy of nf4 16-byte units).
template <int N4>
__device__ __forceinline__ void stage_copy(const Staged<N4> &st, int nf4, uint32_t *lds) {
#pragma unroll
  for (int k = 0; k < N4; ++k) {
    const int f = threadIdx.x + kBlock * k;
    if (f < nf4) {
      const float4 v = st.v[k];  // (through a local: a direct struct copy kept st in scratch memory)
      reinterpret_cast<float4 *>(lds)[f] = v;
    }
  }
}

// RMS factor 1/sqrt(mean(x^2) + eps) from the wavefront partials (after the barrier).
__device__ __forceinline__ float rms_inv(const float *part, int n, float eps) {
  float t = 0.f;
#pragma unroll
  for (int i = 0; i < kWavesPerBlock; ++i) t += part[i];
  return 1.f / sqrtf(t / (float)n + eps);
}

// Lane's slice x[64g .. 64g+63] from padded LDS, times `scale`.
__device__ __forceinline__ void read_slice(const float *lds, int g, float scale, XSlice &xs) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 t = *reinterpret_cast<const float4 *>(&lds[g * kXPad + 4 * i]);
    xs.v[4 * i] = t.x * scale;
    xs.v[4 * i + 1] = t.y * scale;
    xs.v[4 * i + 2] = t.z * scale;
    xs.v[4 * i + 3] = t.w * scale;
  }
  xs.sum = tree_sum64(xs.v);
}

// Profiling hook: thread 0 of a workgroup records the device clock at a point.
__device__ __forceinline__ void trace_mark(uint64_t *tr, int slot) {
  if (tr && threadIdx.x == 0 && blockIdx.x < (unsigned)kTraceBlocks)
    tr[(size_t)blockIdx.x * kTraceSlots + slot] = __builtin_amdgcn_s_memrealtime();
}

// ------------------------------------------------------------------ dequant forms

// The per-weight arithmetic of a group's partial sum in one of four forms, for the
// comparison entry points (fmoe_qmatvec_form, fmoe_expert_ffn_form,
// fmoe_moe_layer_form). Pages cited: [P1] "397B MoE en MacBook: Motor Flash-MoE a
// 4,4 t/s" (aibit.im); [P2] "Flash-MoE: Ausfuehren eines 397B-Parameter-Qwen-Modells
// auf dem MacBook Pro mit reinem C/Metal" (openclawradar.com). With c_j the code of
// column j of a 64-column group, s and b the group's scale and bias:
//   0 naive:     w_j = c_j s + b, then acc += w_j x_j (two fused multiply-adds);
//   1 recast:    acc += fma(c_j, s x_j, b x_j), the per-weight form of
//                [P1] "2. Kernel de desquantización optimizado con FMA" and
//                [P2] "FMA-optimierter Dequant-Kernel" (s x_j and b x_j formed per weight);
//   2 factored:  s * sum_j c_j x_j + b * sum_j x_j (group_partial, the library's form);
//   3 table:     w_j = T[c_j] from a per-(row, group) table T[c] = c s + b that each
//                lane writes to its own LDS row (kLutStride floats), then acc += w_j x_j:
//                the GPU dequant lookup table that [P1] "Lo que descartaron" lists as slower.
constexpr int kLutStride = 17;  // LDS floats per lane's table (16 entries, padded)

// code of column j of the lane's group, as stored: 4-bit -- word j / 8 of the
// group's eight words, low nibble of byte j % 4 for j % 8 < 4, else its high
// nibble; 2-bit -- word j / 16, field (j / 4) % 4 of byte j % 4.
template <int BITS>
__device__ __forceinline__ uint32_t code_of(const Chunk<BITS> &c, int j);
template <>
__device__ __forceinline__ uint32_t code_of<4>(const Chunk<4> &c, int j) {
  const uint32_t w[8] = {c.a.x, c.a.y, c.a.z, c.a.w, c.b.x, c.b.y, c.b.z, c.b.w};
  const int hw = j / 8, r = j % 8;
  return (w[hw] >> (8 * (r % 4) + 4 * (r / 4))) & 15u;
}
template <>
__device__ __forceinline__ uint32_t code_of<2>(const Chunk<2> &c, int j) {
  const uint32_t w[4] = {c.a.x, c.a.y, c.a.z, c.a.w};
  const int wd = j / 16, q = (j / 4) % 4, b = j % 4;
  return (w[wd] >> (8 * b + 2 * q)) & 3u;
}

template <int BITS, int FORM>
__device__ __forceinline__ float partial_form(const Chunk<BITS> &c, uint32_t sb, const XSlice &xs, float *lut) {
  const float s = scale_of(sb), b = bias_of(sb);
  if constexpr (FORM == 2) {
    return group_partial<BITS>(c, sb, xs);
  } else if constexpr (FORM == 3) {
#pragma unroll
    for (int k = 0; k < (1 << BITS); ++k) lut[k] = fmaf((float)k, s, b);
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) acc = fmaf(lut[code_of<BITS>(c, j)], xs.v[j], acc);
    return acc;
  } else {
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const float cj = (float)code_of<BITS>(c, j);
      if constexpr (FORM == 0)
        acc = fmaf(fmaf(cj, s, b), xs.v[j], acc);
      else
        acc += fmaf(cj, s * xs.v[j], b * xs.v[j]);
    }
    return acc;
  }
}

// ------------------------------------------------------------------ row work

// Weight registers of ITERS row iterations of one wavefront (a segment of NGP
// lanes per row of ng groups, ng <= NGP; the lanes past ng add 0, see pad_groups).
template <int BITS, int NGP, int ITERS>
struct RowLoads {
  Chunk<BITS> c[ITERS];
  uint32_t sb[ITERS];
  bool live;  // this lane's group exists
  // rows row0 + i*RPI + sub (clamped to rows-1) of a matrix of ng-group records
  __device__ __forceinline__ void issue(const uint8_t *__restrict__ blob, int ng, int rows, int row0) {
    constexpr int RPI = kWave / NGP;
    const size_t RB = (size_t)ng * gbytes<BITS>();
    const int lane = lane_id();
    const int g = lane & (NGP - 1), sub = lane / NGP;
    live = g < ng;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int row = min(row0 + i * RPI + sub, rows - 1);
      load_group<BITS>(blob + (size_t)row * RB, ng, min(g, ng - 1), c[i], sb[i]);
    }
    __builtin_amdgcn_sched_barrier(0);  // (as in PairLoads::issue)
  }
  // y[row] = alpha * row . x
  __device__ __forceinline__ void finish(const XSlice &xs, float *__restrict__ y, int rows, int row0,
                                         float alpha) const {
    constexpr int RPI = kWave / NGP;
    const int lane = lane_id();
    const int sub = lane / NGP;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const float p = seg_reduce<NGP>(live ? group_partial<BITS>(c[i], sb[i], xs) : 0.f);
      const int row = row0 + i * RPI + sub;
      if (seg_last<NGP>(lane) && row < rows) y[row] = alpha * p;
    }
  }
};

// Row pairs of an interleaved gate/up region (records 2r and 2r+1), rows of ng groups.
template <int BITS, int NGP, int ITERS>
struct PairLoads {
  Chunk<BITS> cg[ITERS], cu[ITERS];
  uint32_t sg[ITERS], su[ITERS];
  bool live;  // this lane's group exists
  __device__ __forceinline__ void issue(const uint8_t *__restrict__ gu, int ng, int pair0) {
    constexpr int RPI = kWave / NGP;
    const size_t RB = (size_t)ng * gbytes<BITS>();
    const int lane = lane_id();
    const int g = lane & (NGP - 1), sub = lane / NGP;
    live = g < ng;
    const int gl = min(g, ng - 1);
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const uint8_t *rec = gu + (size_t)(2 * (pair0 + i * RPI + sub)) * RB;
      load_group<BITS>(rec, ng, gl, cg[i], sg[i]);
      load_group<BITS>(rec + RB, ng, gl, cu[i], su[i]);
    }
    // every load goes out before the first use of a loaded word (otherwise the
    // scheduler can hoist that use between the loads, and its wait stalls the rest)
    __builtin_amdgcn_sched_barrier(0);
  }
  // h[r] = silu(gate_r . x) * (up_r . x)
  __device__ __forceinline__ void finish(const XSlice &xs, float *__restrict__ h, int pair0) const {
    constexpr int RPI = kWave / NGP;
    const int lane = lane_id();
    const int sub = lane / NGP;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const float pg = seg_reduce<NGP>(live ? group_partial<BITS>(cg[i], sg[i], xs) : 0.f);
      const float pu = seg_reduce<NGP>(live ? group_partial<BITS>(cu[i], su[i], xs) : 0.f);
      if (seg_last<NGP>(lane)) h[pair0 + i * RPI + sub] = silu(pg) * pu;
    }
  }
  // the same with the per-weight arithmetic in form FORM (tab: this lane's LDS table row)
  template <int FORM>
  __device__ __forceinline__ void finish_form(const XSlice &xs, float *__restrict__ h, int pair0, float *tab) const {
    constexpr int RPI = kWave / NGP;
    const int lane = lane_id();
    const int sub = lane / NGP;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const float pg = seg_reduce<NGP>(live ? partial_form<BITS, FORM>(cg[i], sg[i], xs, tab) : 0.f);
      const float pu = seg_reduce<NGP>(live ? partial_form<BITS, FORM>(cu[i], su[i], xs, tab) : 0.f);
      if (seg_last<NGP>(lane)) h[pair0 + i * RPI + sub] = silu(pg) * pu;
    }
  }
  // the same from the digit form of x
  __device__ __forceinline__ void finish_dig(const XDig &xd, float *__restrict__ h, int pair0) const {
    constexpr int RPI = kWave / NGP;
    const int lane = lane_id();
    const int sub = lane / NGP;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const float pg = seg_reduce<NGP>(live ? group_partial_dig<BITS>(cg[i], sg[i], xd) : 0.f);
      const float pu = seg_reduce<NGP>(live ? group_partial_dig<BITS>(cu[i], su[i], xd) : 0.f);
      if (seg_last<NGP>(lane)) h[pair0 + i * RPI + sub] = silu(pg) * pu;
    }
  }
};

// Order-preserving integer key of a float: a > b (as floats) <=> key(a) > key(b)
// (as signed integers). key(-inf) = 0x807FFFFF; every key is above INT_MIN.
__device__ __forceinline__ int order_key(float f) {
  const int b = __float_as_int(f);
  return b >= 0 ? b : b ^ 0x7FFFFFFF;
}
__device__ __forceinline__ float key_value(int k) { return __int_as_float(k >= 0 ? k : k ^ 0x7FFFFFFF); }

// Top-K of E logits by one wavefront, exactly under the order (value
// descending, index ascending). Values are compared as order-preserving integer
// keys (NaN logits count as -inf); lane l holds the VPL consecutive elements
// VPL l .. VPL l + VPL - 1, so a lower lane means a lower index, and padding
// elements (e >= E) hold INT_MIN, below every real key.
__device__ __forceinline__ int wave_max_i(int g) {
  constexpr int kGone = (int)0x80000000;
  g = max(g, dpp_i<0xB1, 0xF>(g, kGone));
  g = max(g, dpp_i<0x4E, 0xF>(g, kGone));
  g = max(g, dpp_i<0x141, 0xF>(g, kGone));
  g = max(g, dpp_i<0x140, 0xF>(g, kGone));
  g = max(g, dpp_i<0x142, 0xA>(g, kGone));
  g = max(g, dpp_i<0x143, 0xC>(g, kGone));
  return __builtin_amdgcn_readlane(g, 63);
}

__device__ __forceinline__ int wave_min_i(int g) {
  constexpr int kTop = 0x7FFFFFFF;
  g = min(g, dpp_i<0xB1, 0xF>(g, kTop));
  g = min(g, dpp_i<0x4E, 0xF>(g, kTop));
  g = min(g, dpp_i<0x141, 0xF>(g, kTop));
  g = min(g, dpp_i<0x140, 0xF>(g, kTop));
  g = min(g, dpp_i<0x142, 0xA>(g, kTop));
  g = min(g, dpp_i<0x143, 0xC>(g, kTop));
  return __builtin_amdgcn_readlane(g, 63);
}

// the lane's maximum key and its first position
template <int VPL>
__device__ __forceinline__ void lane_max(const int (&key)[VPL], int &m1, int &p1) {
  m1 = key[0];
  p1 = 0;
#pragma unroll
  for (int m = 1; m < VPL; ++m) {
    const bool gt = key[m] > m1;
    p1 = gt ? m : p1;
    m1 = gt ? key[m] : m1;
  }
}

// Orders one wavefront's LDS writes before its later LDS reads of what other
// lanes wrote (without it the compiler may forward a lane's own stored value).
__device__ __forceinline__ void wave_lds_fence() { __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

// LDS scratch of one wavefront's top-K.
struct TopkLds {
  int m[kWave];        // each lane's maximum key; later the candidates' keys
  int ci[kWave];       // the candidates' indices
  int widx[kMaxTopK];  // the K choices in order: index, key
  int wkey[kMaxTopK];
};

// Exact rank of candidate i among the first C in S (keys S.m, indices S.ci).
__device__ __forceinline__ int candidate_rank(const TopkLds &S, int C, int ck, int cx) {
  int r = 0;
  for (int j = 0; j < C; ++j) {
    const int k = S.m[j];
    r += (k > ck || (k == ck && S.ci[j] < cx)) ? 1 : 0;
  }
  return r;
}

// The general top K (1 <= K <= kMaxTopK) at a cost that does not grow with K:
//  1. each lane's maximum key m1 (first position p1 among equal keys) and its
//     second key m2;
//  2. each lane ranks its maximum among the 64 by the number of greater lane
//     maxima (broadcast LDS reads, four lanes a read);
//  3. the lanes ranked below K write their element to that rank's slot; when
//     exactly K of them did, each finds its own write there (no two share a rank:
//     no tie among them) and no lane's second key reaches the K-th of them, those
//     K lane maxima are the top K, in rank order;
//  4. otherwise the candidates are every key at or above T, the least lane
//     maximum ranked below K: at least K lane maxima reach T, so the top K are
//     among them. At most 64 candidates are ranked exactly among themselves (value
//     descending, index ascending); beyond that (many equal keys) K rounds take
//     the wavefront maximum, lowest index first, one at a time.
// Slot j of S.widx / S.wkey receives choice j. key may be modified.
template <int VPL>
__device__ __forceinline__ void topk_rank(int (&key)[VPL], int K, TopkLds &S) {
  constexpr int kGone = (int)0x80000000;
  const int lane = lane_id();
  int m1, p1, m2 = kGone;
  lane_max<VPL>(key, m1, p1);
#pragma unroll
  for (int m = 0; m < VPL; ++m) m2 = m == p1 ? m2 : max(m2, key[m]);
  S.m[lane] = m1;
  wave_lds_fence();
  int r = 0;
#pragma unroll
  for (int j = 0; j < kWave / 4; ++j) {
    const int4 q = reinterpret_cast<const int4 *>(S.m)[j];
    r += (q.x > m1 ? 1 : 0) + (q.y > m1 ? 1 : 0) + (q.z > m1 ? 1 : 0) + (q.w > m1 ? 1 : 0);
  }
  const bool win = r < K;
  const int me = VPL * lane + p1;
  if (win) {
    S.widx[r] = me;
    S.wkey[r] = m1;
  }
  wave_lds_fence();
  const bool clash = win && S.widx[r] != me;
  bool fast = __popcll(__ballot(win)) == K && __ballot(clash) == 0ull;
  if (fast) fast = __ballot(m2 >= S.wkey[K - 1]) == 0ull;
  if (!fast) {
    // T: the least lane maximum ranked below K
    const int t = wave_min_i(win ? m1 : 0x7FFFFFFF);
    int c = 0;
#pragma unroll
    for (int m = 0; m < VPL; ++m) c += key[m] >= t ? 1 : 0;
    int off = 0, C = 0;
#pragma unroll
    for (int b = 0; b < 5; ++b) {  // (c <= VPL <= 16)
      const unsigned long long bm = __ballot((c >> b) & 1);
      off += (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bm, 0u)) << b;
      C += __popcll(bm) << b;
    }
    if (C <= kWave) {
#pragma unroll
      for (int m = 0; m < VPL; ++m) {
        if (key[m] >= t) {
          S.m[off] = key[m];
          S.ci[off] = VPL * lane + m;
          ++off;
        }
      }
      wave_lds_fence();
      if (lane < C) {
        const int ck = S.m[lane], cx = S.ci[lane];
        const int rk = candidate_rank(S, C, ck, cx);
        if (rk < K) {
          S.widx[rk] = cx;
          S.wkey[rk] = ck;
        }
      }
    } else {
      for (int j = 0; j < K; ++j) {
        int b, p;
        lane_max<VPL>(key, b, p);
        const int g = wave_max_i(b);
        const int L = __ffsll((long long)__ballot(b == g)) - 1;
        const int pl = __builtin_amdgcn_readlane(p, L);
        if (lane == 0) {
          S.widx[j] = VPL * L + pl;
          S.wkey[j] = g;
        }
#pragma unroll
        for (int m = 0; m < VPL; ++m) key[m] = (lane == L && m == pl) ? kGone : key[m];
      }
    }
  }
}

// Small K (at most kRoundsTopK): K rounds of the wavefront maximum over the lane
// maxima, each taking every lane that equals it, need no exchange through LDS and
// cost about one cross-lane reduction a round (on gfx950 ~110 cycles, which is why
// it stops at small K). The picks are the top K exactly when no round matched two
// lanes (no tie among lane maxima) and no lane holds a second key at or above the
// last pick (then no element below a lane maximum can belong to the top K, nor tie
// with the last pick); otherwise returns false and writes nothing. On success,
// slot j of S.widx / S.wkey holds pick j (the lane of a pick writes it).
constexpr int kRoundsTopK = 4;
template <int VPL>
__device__ __forceinline__ bool topk_rounds(const int (&key)[VPL], int K, TopkLds &S) {
  constexpr int kGone = (int)0x80000000;
  const int lane = lane_id();
  int m1 = key[0];
#pragma unroll
  for (int m = 1; m < VPL; ++m) m1 = max(m1, key[m]);
  int v = m1, myr = -1, last = kGone;
  unsigned long long multi = 0ull;
  for (int j = 0; j < K; ++j) {
    const int g = wave_max_i(v);
    const bool hit = v == g;
    const unsigned long long bm = __ballot(hit);
    multi |= bm & (bm - 1ull);  // (nonzero when more than one lane matched)
    myr = hit ? j : myr;
    v = hit ? kGone : v;
    last = g;
  }
  int c = 0;
#pragma unroll
  for (int m = 0; m < VPL; ++m) c += key[m] >= last ? 1 : 0;
  if (multi != 0ull || __ballot(c > 1) != 0ull) return false;
  if (myr >= 0) {
    int p = VPL - 1;  // the maximum's (only) position
#pragma unroll
    for (int m = VPL - 2; m >= 0; --m) p = key[m] == m1 ? m : p;
    S.widx[myr] = VPL * lane + p;
    S.wkey[myr] = m1;
  }
  return true;
}

// The top K (1 <= K <= kMaxTopK) of the wavefront's keys, exactly under the order
// (value descending, index ascending): topk_rounds for small K, else (or when it
// cannot decide) topk_rank. Then lane j < K holds choice j: my_idx, and its
// renormalised softmax weight my_w = exp((l_j - l_0) lscale) / sum_{i<K}
// exp((l_i - l_0) lscale) (renormalising over the chosen K cancels the full softmax
// denominator), the sum taken in choice order by every lane; lanes j >= K get 0 and
// 0. The logits may be held unscaled: lscale > 0 is the factor that turns them into
// the true logits (it does not change the order). key may be modified.
template <int VPL>
__device__ __forceinline__ void wave_topk(int (&key)[VPL], int K, float lscale, TopkLds &S, int &my_idx,
                                          float &my_w) {
  const int lane = lane_id();
  if (!(K <= kRoundsTopK && topk_rounds<VPL>(key, K, S))) topk_rank<VPL>(key, K, S);  // (uniform)
  wave_lds_fence();
  // weights, the sum in choice order
  const float l0 = key_value(S.wkey[0]);
  float sum = 0.f;
  for (int j = 0; j < K; ++j) sum += __expf((key_value(S.wkey[j]) - l0) * lscale);
  const float inv = 1.f / sum;
  my_idx = 0;
  my_w = 0.f;
  if (lane < K) {
    my_idx = S.widx[lane];
    my_w = __expf((key_value(S.wkey[lane]) - l0) * lscale) * inv;
  }
}

// lane l's VPL consecutive logits, with 16-byte loads (clamped to the row; lg
// 16-byte aligned and readable up to E rounded up to 4; the caller turns the
// values into keys, those past E into the lowest key): one load instruction of
// the wavefront covers whole cache lines, where VPL-strided 4-byte loads would
// touch VPL times as many lines per instruction.
template <int VPL>
__device__ __forceinline__ void load_logits(const float *lg, int E, float (&v)[VPL], int parts = 1,
                                            size_t pstride = 0) {
  const int lane = lane_id();
  const float4 *l4 = reinterpret_cast<const float4 *>(lg);
#pragma unroll
  for (int q = 0; q < VPL / 4; ++q) {
    const int i = min(VPL / 4 * lane + q, (E + 3) / 4 - 1);
    float4 t = l4[i];
    if (parts > 1) {
      // slabs of a split router, all requested at once (past the last: the last
      // again, not added), then added in slab order (every reader the same)
      float4 u[kRouterMaxParts - 1];
#pragma unroll
      for (int p = 1; p < kRouterMaxParts; ++p)
        u[p - 1] = reinterpret_cast<const float4 *>(lg + min(p, parts - 1) * pstride)[i];
#pragma unroll
      for (int p = 1; p < kRouterMaxParts; ++p) {
        if (p < parts) {
          t.x += u[p - 1].x;
          t.y += u[p - 1].y;
          t.z += u[p - 1].z;
          t.w += u[p - 1].w;
        }
      }
    }
    v[4 * q] = t.x;
    v[4 * q + 1] = t.y;
    v[4 * q + 2] = t.z;
    v[4 * q + 3] = t.w;
  }
}

template <int VPL>
__device__ __forceinline__ void logit_keys(const float (&v)[VPL], int E, int (&key)[VPL]) {
  const int lane = lane_id();
#pragma unroll
  for (int m = 0; m < VPL; ++m) {
    const float t = v[m];
    key[m] = VPL * lane + m < E ? order_key(t == t ? t : -INFINITY) : (int)0x80000000;
  }
}

// top-K of E <= kMaxExperts logits in memory (LDS or global); see wave_topk
__device__ __forceinline__ void wave_topk_lds(const float *lg, int E, int K, float lscale, TopkLds &S, int &my_idx,
                                              float &my_w, int parts = 1, size_t pstride = 0) {
  if (E <= 512) {
    float v[8];
    int key[8];
    load_logits<8>(lg, E, v, parts, pstride);
    logit_keys<8>(v, E, key);
    wave_topk<8>(key, K, lscale, S, my_idx, my_w);
  } else {
    float v[16];
    int key[16];
    load_logits<16>(lg, E, v, parts, pstride);
    logit_keys<16>(v, E, key);
    wave_topk<16>(key, K, lscale, S, my_idx, my_w);
  }
}

// Block-wide top-K: one wavefront computes it from the logits in LDS and
// publishes it through LDS (sidx, sw: lane j writes choice j); contains one
// barrier, after which every thread reads the result from sidx / sw. Workgroup b
// uses wavefront b % 4, so that the workgroups sharing a CU do not all compute it
// on the same SIMD.
__device__ __forceinline__ void block_topk(const float *lg, int E, int K, TopkLds &S, int *sidx, float *sw) {
  if (wave_in_block() == (int)(blockIdx.x % kWavesPerBlock)) {
    // the rest of the workgroup waits on this wavefront: let it win the SIMD's
    // issue arbitration against co-resident wavefronts of other workgroups
    __builtin_amdgcn_s_setprio(3);
    int mi;
    float mw;
    wave_topk_lds(lg, E, K, 1.f, S, mi, mw);
    __builtin_amdgcn_s_setprio(0);
    if (lane_id() < K) {
      sidx[lane_id()] = mi;
      sw[lane_id()] = mw;
    }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ standalone kernels

template <int BITS, int NGP, int ITERS>
__global__ __launch_bounds__(kBlock) void k_qmatvec(const uint8_t *__restrict__ blob, int ng, int rows,
                                                     const float *__restrict__ x, float *__restrict__ y) {
  __shared__ float xl[NGP * kXPad];
  constexpr int X4 = (NGP * 16 + kBlock - 1) / kBlock;
  const int row0 = wave_id() * ITERS * (kWave / NGP);
  Staged<X4> xst;
  stage_load(x, ng * 16, xst);
  RowLoads<BITS, NGP, ITERS> L;
  if (row0 < rows) L.issue(blob, ng, rows, row0);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<X4, false>(xst, ng * 16, xl, nullptr);
  __syncthreads();
  if (row0 >= rows) return;
  XSlice xs;
  read_slice(xl, min(lane_id() & (NGP - 1), ng - 1), 1.f, xs);
  L.finish(xs, y, rows, row0, 1.f);
}

template <int BITS, int NGP, int ITERS>
__global__ __launch_bounds__(kBlock) void k_expert_gateup(const uint8_t *__restrict__ gu, int ng, int inter,
                                                           const float *__restrict__ x, float *__restrict__ h) {
  __shared__ float xl[NGP * kXPad];
  constexpr int X4 = (NGP * 16 + kBlock - 1) / kBlock;
  const int pair0 = wave_id() * ITERS * (kWave / NGP);
  Staged<X4> xst;
  stage_load(x, ng * 16, xst);
  PairLoads<BITS, NGP, ITERS> P;
  if (pair0 < inter) P.issue(gu, ng, pair0);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<X4, false>(xst, ng * 16, xl, nullptr);
  __syncthreads();
  if (pair0 >= inter) return;
  XSlice xs;
  read_slice(xl, min(lane_id() & (NGP - 1), ng - 1), 1.f, xs);
  P.finish(xs, h, pair0);
}

// ------------------------------------------------------------------ layer kernels

// gate/up pair iterations per wavefront (routed and shared): four above four
// slots, which halves the routed workgroups so that they are all resident at once
// (3 per compute unit; at top-10, 1,280 workgroups with two pairs each ran in two
// rounds); and routed down row iterations per wavefront by the padded top_k: two
// above four slots (measured,
// top-10 layer: 12.8 us for the down kernel against 14.9 with one row per
// wavefront, whose workgroups each stage all of h for a quarter of the rows)
__host__ __device__ constexpr int gateup_iters(int K) { return K <= 4 ? 2 : 4; }
__host__ __device__ constexpr int down_iters(int kpad) { return kpad <= 4 ? 4 : 2; }
// Slots per down lane group for top_k slots: top_k rounded up to a power of two, or
// 12 for 9..12 slots when a row's lane groups then fill whole wavefronts (12 x the
// inter groups a multiple of 64, at most 32 groups: inter 1024 or 2048), which spares
// a quarter of the lanes' loads and arithmetic at top_k 10 against 16 slots.
__host__ __device__ constexpr int down_slots(int K, int ngi_pad) {
  return K <= 1 ? 1 : K <= 2 ? 2 : K <= 4 ? 4 : K <= 8 ? 8 : (K <= 12 && (ngi_pad == 16 || ngi_pad == 32)) ? 12 : 16;
}
constexpr int kP3Block = 256;      // threads per down + combine workgroup
constexpr int kP3Waves = kP3Block / kWave;

struct Phase1Args {
  const float *router;
  const float *gvec;  // null: no shared expert
  int E;
  int bits;           // code width of the experts (digit word order)
  const float *x;
  float rms_eps;  // >= 0: x is RMS-scaled first
  float *logits;
  float *sigma;
  uint32_t *xdig;     // [hidden/64][kDigStride] x in digit form
  int ng;             // hidden / 64
  int n_prep_blocks;  // workgroups before the router's: x in digit form, then the gate
  float *xs;          // null, or [hidden]: x (RMS-scaled) in fp32 too, for the form variants of phase 2
  uint64_t *trace;
};

// Group g of the layer input in digit form (lanes = the group's 64 columns), from
// the staged raw vector and its RMS factor inv: X_j = round(h_j 2^k), with k such
// that the group's largest |h_j| lies below 2^22; f = inv 2^-k, sum x = inv sum h.
// A non-finite value in the group makes f and the sum NaN.
template <int BITS>
__device__ __forceinline__ void write_digits(const float *xl, int g, float inv, uint32_t *ybuf,
                                             uint32_t *__restrict__ dst) {
  const int lane = lane_id();
  const float h = xl[lds_index(kGroup * g + lane)];
  const float amax = __int_as_float(wave_max_i(__float_as_int(fabsf(h))));
  int e;
  frexpf(amax, &e);  // amax < 2^e (e = 0 for amax = 0)
  const int k = 22 - e;
  const int X = (int)rintf(ldexpf(h, k));
  ybuf[lane] = (uint32_t)(X + 0x888888) ^ 0x888888u;  // nibble p = digit p + 8, then two's complement
  const float sh = seg_allreduce<kWave>(h);
  const bool finite = amax <= 3.402823466e38f;
  if (lane < kDigWords) {
    const int w = lane / kDigits, p = lane % kDigits;
    uint32_t word = 0;
#pragma unroll
    for (int n = 0; n < 8; ++n) word |= ((ybuf[digit_column<BITS>(w, n)] >> (4 * p)) & 15u) << (4 * n);
    dst[g * kDigStride + lane] = word;
  } else if (lane < kDigStride) {
    const float v = lane == kDigWords ? ldexpf(inv, -k) : lane == kDigWords + 1 ? inv * sh : 0.f;
    dst[g * kDigStride + lane] = __float_as_uint(finite || lane >= kDigWords + 2 ? v : __int_as_float(0x7FC00000));
  }
}

// Phase 1: the router. Each fp32 router row is split over router_split()
// wavefronts of a workgroup (part h: lane l covers columns 4l + 256t + 0..3 for
// the chunks t in [h c, (h+1) c), c = ceil(nt / SPLIT), nt = hidden / 256), so
// that the 8 MB of rows spread over every compute unit (512 rows: one workgroup
// per compute unit); the parts' sums are added in order. The workgroups before
// the router's write x in digit form for the gate/up kernel, and the last of them
// computes the shared expert's gate sigmoid(g . x).
template <int NGHP>
constexpr int router_split() {
  return NGHP / 4 >= 2 ? 2 : 1;
}
template <int NGHP>
__global__ __launch_bounds__(kBlock) void k_phase1(const Phase1Args a) {
  constexpr int X4 = (NGHP * 16 + kBlock - 1) / kBlock;
  constexpr int SPLIT = router_split<NGHP>();
  constexpr int NTW = NGHP / 4 / SPLIT;  // float4 per lane of a wavefront's part of the row, at most
  __shared__ float xl[NGHP * kXPad];
  __shared__ float part[kWavesPerBlock];
  __shared__ float dpart[kWavesPerBlock];
  __shared__ uint32_t ybuf[kWavesPerBlock][kWave];
  const int ng = a.ng, H = ng * kGroup, nt = ng / 4;
  const int lane = lane_id();
  const bool rms = a.rms_eps >= 0.f;
  trace_mark(a.trace, 0);
  const int wv = wave_in_block();
  if ((int)blockIdx.x < a.n_prep_blocks) {
    // The workgroups before the router's: x in digit form, one 64-column group per
    // wavefront, then one for the shared expert's gate sigma = sigmoid(g . x) --
    // beside the router rows, off their path. Dispatched first, so that their x
    // requests do not queue behind a router workgroup's rows on the same compute
    // unit. (The second vector's loads are unconditional: the gate vector in the
    // gate's workgroup, x again in the others.)
    const int g = (int)blockIdx.x * kWavesPerBlock + wv;
    const bool gate = a.gvec != nullptr && (int)blockIdx.x == (ng + kWavesPerBlock - 1) / kWavesPerBlock;
    Staged<X4> xst, gst;
    stage_load(a.x, ng * 16, xst);
    stage_load(gate ? a.gvec : a.x, ng * 16, gst);
    if (rms)
      stage_store<X4, true>(xst, ng * 16, xl, part);
    else
      stage_store<X4, false>(xst, ng * 16, xl, part);
    __syncthreads();
    const float inv = rms ? rms_inv(part, H, a.rms_eps) : 1.f;
    if (gate) {  // (uniform over the workgroup)
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < X4; ++k) {
        const int f = threadIdx.x + kBlock * k;
        if (f < ng * 16) {
          const float4 xv = *reinterpret_cast<const float4 *>(&xl[lds_index(4 * f)]);
          const float4 gv = gst.v[k];
          acc = fmaf(gv.x, xv.x, acc);
          acc = fmaf(gv.y, xv.y, acc);
          acc = fmaf(gv.z, xv.z, acc);
          acc = fmaf(gv.w, xv.w, acc);
        }
      }
      acc = seg_reduce<kWave>(acc);
      if (lane == kWave - 1) dpart[wv] = acc;
      __syncthreads();
      if (threadIdx.x == 0) {
        float d = dpart[0];
#pragma unroll
        for (int i = 1; i < kWavesPerBlock; ++i) d += dpart[i];
        *a.sigma = 1.f / (1.f + expf(-d * inv));
      }
    } else if (g < ng) {
      if (a.bits == 4)
        write_digits<4>(xl, g, inv, ybuf[wv], a.xdig);
      else
        write_digits<2>(xl, g, inv, ybuf[wv], a.xdig);
      if (a.xs) a.xs[kGroup * g + lane] = xl[lds_index(kGroup * g + lane)] * inv;
    }
    trace_mark(a.trace, 3);
    return;
  }
  const int n_rows = a.E;
  const int half = wv % SPLIT;
  const int row = ((int)blockIdx.x - a.n_prep_blocks) * (kWavesPerBlock / SPLIT) + wv / SPLIT;
  const int rr = min(row, n_rows - 1);
  const int per = (nt + SPLIT - 1) / SPLIT;  // chunks of 256 columns per part
  const int t0 = per * half, tn = min(per, nt - t0);  // this part's chunks (tn >= 1)
  const float4 *src = reinterpret_cast<const float4 *>(a.router + (size_t)rr * H);
  Staged<X4> xst;
  stage_load(a.x, ng * 16, xst);
  float4 w[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) w[t] = src[lane + 64 * (t0 + min(t, tn - 1))];
  __builtin_amdgcn_sched_barrier(0);
  if (rms)
    stage_store<X4, true>(xst, ng * 16, xl, part);
  else
    stage_store<X4, false>(xst, ng * 16, xl, part);
  __syncthreads();
  trace_mark(a.trace, 1);
  const float inv = rms ? rms_inv(part, H, a.rms_eps) : 1.f;
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    if (t < tn) {  // (uniform)
      const float4 xv = *reinterpret_cast<const float4 *>(&xl[lds_index(4 * lane + 256 * (t0 + t))]);
      acc = fmaf(w[t].x, xv.x * inv, acc);
      acc = fmaf(w[t].y, xv.y * inv, acc);
      acc = fmaf(w[t].z, xv.z * inv, acc);
      acc = fmaf(w[t].w, xv.w * inv, acc);
    }
  }
  float d = seg_reduce<kWave>(acc);
  if constexpr (SPLIT > 1) {
    if (lane == kWave - 1) dpart[wv] = d;
    __syncthreads();
    d = dpart[wv - half];
#pragma unroll
    for (int h = 1; h < SPLIT; ++h) d += dpart[wv - half + h];
  }
  if (lane == kWave - 1 && half == 0 && row < n_rows) a.logits[row] = d;
  trace_mark(a.trace, 3);
}

struct Phase2Args {
  const float *logits;
  int E, K;
  const uint8_t *bank;
  size_t stride;
  const uint32_t *xdig;  // x in digit form, [hidden/64][kDigStride]
  int ng;                // hidden / 64
  int I;
  float *h_routed;
  int32_t *ws_idx;
  float *ws_w;
  int32_t *out_idx;
  float *out_w;
  int waves_per_slot;
  int n_routed_blocks;
  const uint8_t *shared_gu;  // null: no shared expert
  float *h_shared;
  const float *xs;           // the form variants (FORM >= 0): x in fp32 [hidden] instead of xdig
  uint64_t *trace;
  const uint8_t *const *expert_ptr;  // PTR builds: expert e's blob at expert_ptr[e] (the tier's table)
};

// Phase 2. Routed blocks stage the logits and x (in digit form), derive the
// top-K (one wavefront per block), then run gate/up + SwiGLU of their slot's
// expert. Shared blocks run the shared expert's gate/up + SwiGLU: it does not
// depend on the routing, so its weights stream while the routed blocks are still
// choosing. x arrives in the digit form the router kernel wrote (RMS factor
// included), so this kernel reads no raw x. GI: gate/up pair iterations per
// wavefront (gateup_iters(top_k)). FORM >= 0 (comparison builds): x in fp32
// (a.xs) and the per-weight arithmetic of partial_form<FORM> instead of the digit
// form's integer dot products.
template <int BITS, int NGHP, int GI, int FORM = -1, bool PTR = false>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void k_phase2(const Phase2Args a) {
  // the blob of routed expert e: in the bank, or (PTR) where the table says
  auto blob = [&](int e) -> const uint8_t * {
    if constexpr (PTR)
      return a.expert_ptr[e];
    else
      return a.bank + (size_t)e * a.stride;
  };
  constexpr int RPIH = kWave / NGHP;
  constexpr bool DIG = FORM < 0;
  constexpr int D4 = DIG ? (NGHP * kDigStride / 4 + kBlock - 1) / kBlock : (NGHP * 16 + kBlock - 1) / kBlock;
  const int NF4 = DIG ? a.ng * kDigStride / 4 : a.ng * 16;  // 16-byte units of x's staged form
  __shared__ uint32_t xdl[DIG ? NGHP * kDigStride : 1];
  __shared__ float xfl[DIG ? 1 : NGHP * kXPad];
  __shared__ float lut[FORM == 3 ? kBlock * kLutStride : 1];
  __shared__ __align__(16) float lg[kMaxExperts];
  __shared__ int sidx[kMaxTopK];
  __shared__ float sw[kMaxTopK];
  __shared__ TopkLds tks;
  const int lane = lane_id();
  const float *xsrc = DIG ? reinterpret_cast<const float *>(a.xdig) : a.xs;
  auto x_store = [&](const Staged<D4> &st) {
    if constexpr (DIG)
      stage_copy(st, NF4, xdl);
    else
      stage_store<D4, false>(st, NF4, xfl, nullptr);
  };
  auto finish = [&](const PairLoads<BITS, NGHP, GI> &P, float *h, int pair0) {
    const int g = min(lane & (NGHP - 1), a.ng - 1);
    if constexpr (DIG) {
      XDig xd;
      read_digits(xdl, g, xd);
      P.finish_dig(xd, h, pair0);
    } else {
      XSlice xs;
      read_slice(xfl, g, 1.f, xs);
      P.template finish_form<DIG ? 0 : FORM>(xs, h, pair0, FORM == 3 ? lut + threadIdx.x * kLutStride : lut);
    }
  };
  trace_mark(a.trace, 0);
  if ((int)blockIdx.x < a.n_routed_blocks) {
    // a workgroup serves one slot (waves_per_slot is a multiple of 4) and needs
    // only the first slot+1 winners: the rounds stop there, so the workgroups of
    // the early slots start streaming before the last winner is known. The
    // workgroup that publishes the routing is one of the last slot's (all K).
    const int bslot = min((int)(blockIdx.x * kWavesPerBlock) / a.waves_per_slot, a.K - 1);
    const int wv = blockIdx.x * kWavesPerBlock + wave_in_block();
    const int slot = min(wv / a.waves_per_slot, a.K - 1);
    const int pair0 = (wv % a.waves_per_slot) * GI * RPIH;
    const bool active = wv < a.waves_per_slot * a.K;
    PairLoads<BITS, NGHP, GI> P;
    if (a.E <= 512) {
      // One wavefront (b % 4, so that the workgroups sharing a CU use different
      // SIMDs) requests the logits in the top-K's layout before its share of x,
      // waits for the logits only and derives the routing while x is still
      // arriving; every wavefront then stores its share of x. (Each branch issues
      // its own loads, in a fixed order, so that no wait joins the two.)
      Staged<D4> xst;
      if (wave_in_block() == (int)(blockIdx.x % kWavesPerBlock)) {
        float lv[8];
        load_logits<8>(a.logits, a.E, lv);
        __builtin_amdgcn_sched_barrier(0);
        stage_load(xsrc, NF4, xst);
        __builtin_amdgcn_sched_barrier(0);
        int key[8];
        logit_keys<8>(lv, a.E, key);
        // the rest of the workgroup waits on this wavefront: let it win the
        // SIMD's issue arbitration against co-resident wavefronts of other workgroups
        __builtin_amdgcn_s_setprio(3);
        int mi;
        float mw;
        wave_topk<8>(key, bslot + 1, 1.f, tks, mi, mw);
        __builtin_amdgcn_s_setprio(0);
        if (lane <= bslot) {
          sidx[lane] = mi;
          sw[lane] = mw;
        }
      } else {
        stage_load(xsrc, NF4, xst);
      }
      // the routing is published before x is staged: the weight requests go out as
      // soon as the top-K is known, and the staging then waits for x only (its
      // loads went out first)
      __syncthreads();
      trace_mark(a.trace, 2);
      // unconditional, so that the staging's wait counts the x loads only (every
      // routed wavefront is active: waves_per_slot * K is a whole number of
      // workgroups, and each wavefront's pairs lie inside its expert)
      P.issue(blob(sidx[slot]), a.ng, pair0);
      x_store(xst);
      __syncthreads();
      trace_mark(a.trace, 1);
    } else {
      for (int i = threadIdx.x; i < a.E; i += kBlock) lg[i] = a.logits[i];
      Staged<D4> xst;
      stage_load(xsrc, NF4, xst);
      x_store(xst);
      __syncthreads();
      trace_mark(a.trace, 1);
      block_topk(lg, a.E, bslot + 1, tks, sidx, sw);
      trace_mark(a.trace, 2);
      if (active) P.issue(blob(sidx[slot]), a.ng, pair0);
    }
    if (wv == (a.K - 1) * a.waves_per_slot && lane < a.K) {
      const int sel = sidx[lane];
      const float ws = sw[lane];
      a.ws_idx[lane] = sel;
      a.ws_w[lane] = ws;
      if (a.out_idx) a.out_idx[lane] = sel;
      if (a.out_w) a.out_w[lane] = ws;
    }
    if (active) finish(P, a.h_routed + (size_t)slot * a.I, pair0);
    trace_mark(a.trace, 3);
    return;
  }
  // shared expert gate/up
  const int wv = (blockIdx.x - a.n_routed_blocks) * kWavesPerBlock + wave_in_block();
  const int pair0 = wv * GI * RPIH;
  // x first (its loads complete before the weights', so the staging does not
  // wait for them), then the weights
  Staged<D4> xst;
  stage_load(xsrc, NF4, xst);
  __builtin_amdgcn_sched_barrier(0);
  PairLoads<BITS, NGHP, GI> P;
  if (pair0 < a.I) P.issue(a.shared_gu, a.ng, pair0);
  x_store(xst);
  __syncthreads();
  trace_mark(a.trace, 1);
  if (pair0 < a.I) finish(P, a.h_shared, pair0);
  trace_mark(a.trace, 3);
}

// Down partials of one slot for ITERS rows, reading that slot's h group from LDS
// as the code words are used (eight or sixteen values at a time) instead of
// holding the whole 64-value slice in registers: gp[i] = scale_i * sum_j c_ij h_j
// + bias_i * hsum, in exactly the order of group_partial (the same accumulators,
// code words ascending).
template <int BITS, int ITERS, int SPL>
__device__ __forceinline__ void stream_partials(const Chunk<BITS> (&c)[ITERS][SPL], const uint32_t (&sb)[ITERS][SPL],
                                                int m, const float *hx, float hsum, float (&gp)[ITERS]) {
  if constexpr (BITS == 4) {
    float a0[ITERS], a1[ITERS];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) a0[i] = a1[i] = 0.f;
#pragma unroll
    for (int hw = 0; hw < 8; ++hw) {
      const float4 v0 = *reinterpret_cast<const float4 *>(hx + 8 * hw);
      const float4 v1 = *reinterpret_cast<const float4 *>(hx + 8 * hw + 4);
#pragma unroll
      for (int i = 0; i < ITERS; ++i) {
        const uint4 &q = hw < 4 ? c[i][m].a : c[i][m].b;
        const int w = hw & 3;
        const uint32_t d = w == 0 ? q.x : w == 1 ? q.y : w == 2 ? q.z : q.w;
        const uint32_t lo = opaque(d & 0x0F0F0F0Fu);
        const uint32_t hi = opaque(d & 0xF0F0F0F0u);
        a0[i] = fmaf(ub0(lo), v0.x, a0[i]);
        a0[i] = fmaf(ub1(lo), v0.y, a0[i]);
        a0[i] = fmaf(ub2(lo), v0.z, a0[i]);
        a0[i] = fmaf(ub3(lo), v0.w, a0[i]);
        a1[i] = fmaf(ub0(hi), v1.x, a1[i]);
        a1[i] = fmaf(ub1(hi), v1.y, a1[i]);
        a1[i] = fmaf(ub2(hi), v1.z, a1[i]);
        a1[i] = fmaf(ub3(hi), v1.w, a1[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i)
      gp[i] = fmaf(scale_of(sb[i][m]), fmaf(a1[i], 0.0625f, a0[i]), bias_of(sb[i][m]) * hsum);
  } else {
    float a[ITERS][4];
#pragma unroll
    for (int i = 0; i < ITERS; ++i) a[i][0] = a[i][1] = a[i][2] = a[i][3] = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float4 v[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const float4 *>(hx + 16 * w + 4 * q);
#pragma unroll
      for (int i = 0; i < ITERS; ++i) {
        const uint4 &cq = c[i][m].a;
        const uint32_t d = w == 0 ? cq.x : w == 1 ? cq.y : w == 2 ? cq.z : cq.w;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t mk = opaque(d & (0x03030303u << (2 * q)));
          a[i][q] = fmaf(ub0(mk), v[q].x, a[i][q]);
          a[i][q] = fmaf(ub1(mk), v[q].y, a[i][q]);
          a[i][q] = fmaf(ub2(mk), v[q].z, a[i][q]);
          a[i][q] = fmaf(ub3(mk), v[q].w, a[i][q]);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const float dot = fmaf(a[i][3], 0.015625f, fmaf(a[i][2], 0.0625f, fmaf(a[i][1], 0.25f, a[i][0])));
      gp[i] = fmaf(scale_of(sb[i][m]), dot, bias_of(sb[i][m]) * hsum);
    }
  }
}

struct Phase3Args {
  const uint8_t *bank;
  size_t stride, gu_bytes;
  const int32_t *idx;
  const float *w;
  int K;
  const float *h_routed;      // [K][I]
  int I, H;
  const uint8_t *shared_down; // null: no shared expert
  const float *h_shared;      // [I]
  const float *sigma;
  const float *residual;
  float *out;
  uint64_t *trace;
  const uint8_t *const *expert_ptr;  // PTR builds: expert e's blob at expert_ptr[e] (the tier's table)
};

// Phase 3: out_i = residual_i + sum_k w_k (down_k . h_k)_i + sigma (down_s . h_s)_i.
// Routed: lanes are (slot k, group j) pairs, so one cross-lane sum adds the K
// experts' weighted partials of a row together; each lane keeps its slot's h
// slice. KPAD = down_slots(top_k, NGIP) (top_k rounded up to a power of two, or 12), NGIP = the inter groups ngi
// rounded up to a power of two (lanes of slots past top_k or groups past ngi stay
// idle). The routed h vectors are staged in LDS when they fit (KPAD * NGIP <=
// 128), group j of slot k in row k ngi + j. Shared: the same wavefront's rows,
// NGIP lanes per row; its weights do not depend on the routing and are requested
// first. A wavefront passes its shared results from the shared lanes to the
// combining lanes through LDS.
// FORM >= 0 (comparison builds, at most four slots): the per-weight arithmetic of
// partial_form<FORM> instead of group_partial.
template <int BITS, int NGIP, int KPAD, int FORM = -1, bool PTR = false>
__global__ __launch_bounds__(kP3Block) void k_phase3(const Phase3Args a) {
  constexpr int kP3Iters = down_iters(KPAD);
  constexpr int SLOTS = KPAD * NGIP;
  constexpr int SEG = SLOTS < kWave ? SLOTS : kWave;  // lanes per row
  constexpr int SPL = SLOTS / SEG;                     // slots per lane
  constexpr int RPI = kWave / SEG;
  constexpr int RPW = kP3Iters * RPI;                  // rows per wavefront
  constexpr int RPII = kWave / NGIP;                   // shared-down rows per iteration
  constexpr int SIT = (RPW + RPII - 1) / RPII;         // shared-down iterations
  // routed h staged in LDS when it fits (up to 68 KB above four slots); above four
  // slots the partials stream h (stream_partials, from LDS or, unstaged, from the
  // cache hierarchy) instead of holding a lane's SPL slices in registers
  constexpr bool STAGE = KPAD * NGIP <= (KPAD <= 4 ? 128 : 256);
  constexpr bool STREAM = KPAD >= 8;
  static_assert(FORM < 0 || !STREAM, "the form builds take at most four slots");
  const int ngi = a.I / kGroup;
  const size_t RB = (size_t)ngi * gbytes<BITS>();
  __shared__ float hl[STAGE ? KPAD * NGIP * kXPad : 1];
  __shared__ float hs[NGIP * kXPad];
  __shared__ float hlsum[STAGE ? KPAD * NGIP : 1];  // per-group sums of the staged h
  __shared__ float hssum[NGIP];
  __shared__ float dsh[kP3Waves * RPW];
  __shared__ float lut[FORM == 3 ? kP3Block * kLutStride : 1];
  // a group's partial sum in this build's form
  auto gpart = [&](const Chunk<BITS> &c, uint32_t sb, const XSlice &xs) {
    if constexpr (FORM < 0)
      return group_partial<BITS>(c, sb, xs);
    else
      return partial_form<BITS, FORM>(c, sb, xs, FORM == 3 ? lut + threadIdx.x * kLutStride : lut);
  };
  trace_mark(a.trace, 0);
  const int lane = lane_id();
  const int sub = lane / SEG;
  const int row0 = ((int)blockIdx.x * kP3Waves + wave_in_block()) * RPW;
  const bool sh = a.shared_down != nullptr;
  // requested first, all independent of each other: the routing of each slot, the
  // residual of this lane's rows and sigma (used only after the dot products),
  // the h vectors, and the shared expert's down rows
  int sel[SPL];
  float wk[SPL];
  int grp[SPL], kk[SPL];
  bool act[SPL];
#pragma unroll
  for (int m = 0; m < SPL; ++m) {
    const int slot = (lane % SEG) + kWave * m;
    const int k = slot / NGIP;
    grp[m] = min(slot % NGIP, ngi - 1);
    act[m] = k < a.K && slot % NGIP < ngi && row0 < a.H;
    kk[m] = k < a.K ? k : 0;
    sel[m] = a.idx[kk[m]];
    wk[m] = k < a.K ? a.w[kk[m]] : 0.f;
  }
  float res[kP3Iters];
#pragma unroll
  for (int i = 0; i < kP3Iters; ++i) res[i] = a.residual[min(row0 + i * RPI + sub, a.H - 1)];
  const float sig = *a.sigma;  // (a workspace value; unused without a shared expert)
  constexpr int H4 = STAGE ? (KPAD * NGIP * 16 + kP3Block - 1) / kP3Block : 1;
  constexpr int S4 = (NGIP * 16 + kP3Block - 1) / kP3Block;
  Staged<H4> hst;
  if constexpr (STAGE) stage_load<H4, kP3Block>(a.h_routed, a.K * a.I / 4, hst);
  // without a shared expert these loads read the routed expert 0 instead (valid
  // memory, results unused): unconditional loads keep the memory-counter waits exact
  Staged<S4> sst;
  stage_load<S4, kP3Block>(sh ? a.h_shared : a.h_routed, ngi * 16, sst);
  __builtin_amdgcn_sched_barrier(0);  // every h load goes out before any weight load
  const uint8_t *sdown = sh ? a.shared_down : a.bank + a.gu_bytes;
  // shared rows: NGIP lanes per row; with fewer rows per wavefront than a load
  // covers, the spare lanes repeat this wavefront's rows (the same cache lines)
  const int ssub = RPW < RPII ? (lane / NGIP) % RPW : lane / NGIP;
  const int sg = min(lane & (NGIP - 1), ngi - 1);
  const bool slive = (lane & (NGIP - 1)) < ngi;
  Chunk<BITS> cs[SIT];
  uint32_t ss[SIT];
#pragma unroll
  for (int q = 0; q < SIT; ++q) {
    const int row = min(row0 + q * RPII + ssub, a.H - 1);
    load_group<BITS>(sdown + (size_t)row * RB, ngi, sg, cs[q], ss[q]);
  }
  __builtin_amdgcn_sched_barrier(0);  // the shared rows go out before the routing is needed
  const uint8_t *base[SPL];
#pragma unroll
  for (int m = 0; m < SPL; ++m) {
    asm volatile("" : "+v"(sel[m]));  // (keeps the address arithmetic, and its wait, here)
    if constexpr (PTR)
      base[m] = a.expert_ptr[sel[m]] + a.gu_bytes;
    else
      base[m] = a.bank + (size_t)sel[m] * a.stride + a.gu_bytes;
  }
  Chunk<BITS> c[kP3Iters][SPL];
  uint32_t sb[kP3Iters][SPL];
#pragma unroll
  for (int i = 0; i < kP3Iters; ++i) {
    const int row = min(row0 + i * RPI + sub, a.H - 1);
    // unconditional (inactive slots reload slot 0's rows, unused), as above
#pragma unroll
    for (int m = 0; m < SPL; ++m) load_group<BITS>(base[m] + (size_t)row * RB, ngi, grp[m], c[i][m], sb[i][m]);
  }
  __builtin_amdgcn_sched_barrier(0);  // the h vectors were requested before the weights
  if constexpr (STAGE) stage_store_gsum<H4, kP3Block>(hst, a.K * a.I / 4, hl, hlsum);
  stage_store_gsum<S4, kP3Block>(sst, ngi * 16, hs, hssum);
  __syncthreads();
  trace_mark(a.trace, 1);
  if (row0 >= a.H) return;
  if (sh) {
    XSlice xs;
    read_slice_sum(hs, sg, hssum[sg], xs);
#pragma unroll
    for (int q = 0; q < SIT; ++q) {
      const float p = seg_reduce<NGIP>(slive ? gpart(cs[q], ss[q], xs) : 0.f);
      const int r = q * RPII + ssub;  // row within this wavefront's rows
      if (seg_last<NGIP>(lane) && r < RPW) dsh[wave_in_block() * RPW + r] = sig * p;
    }
  }
  float pr[kP3Iters];  // this lane's weighted routed partial of each row
#pragma unroll
  for (int i = 0; i < kP3Iters; ++i) pr[i] = 0.f;
  if constexpr (STREAM) {
#pragma unroll
    for (int m = 0; m < SPL; ++m) {
      const int row = kk[m] * ngi + grp[m];
      float gp[kP3Iters];
      if constexpr (STAGE) {
        stream_partials<BITS, kP3Iters, SPL>(c, sb, m, hl + row * kXPad, hlsum[row], gp);
      } else {
        const float *hx = a.h_routed + (size_t)kk[m] * a.I + kGroup * grp[m];
        float hsum;
        {
          XSlice t;  // (one slice at a time: its sum, then its values again as used)
          load_xslice(hx, t);
          hsum = t.sum;
        }
        stream_partials<BITS, kP3Iters, SPL>(c, sb, m, hx, hsum, gp);
      }
#pragma unroll
      for (int i = 0; i < kP3Iters; ++i)
        if (act[m]) pr[i] = fmaf(wk[m], gp[i], pr[i]);
    }
  } else {
    XSlice xs[SPL];
    if constexpr (STAGE) {
#pragma unroll
      for (int m = 0; m < SPL; ++m) read_slice_sum(hl, kk[m] * ngi + grp[m], hlsum[kk[m] * ngi + grp[m]], xs[m]);
    } else {
#pragma unroll
      for (int m = 0; m < SPL; ++m) load_xslice(a.h_routed + (size_t)kk[m] * a.I + kGroup * grp[m], xs[m]);
    }
#pragma unroll
    for (int i = 0; i < kP3Iters; ++i)
#pragma unroll
      for (int m = 0; m < SPL; ++m)
        if (act[m]) pr[i] = fmaf(wk[m], gpart(c[i][m], sb[i][m], xs[m]), pr[i]);
  }
#pragma unroll
  for (int i = 0; i < kP3Iters; ++i) {
    const float p = seg_reduce<SEG>(pr[i]);
    const int row = row0 + i * RPI + sub;
    if (seg_last<SEG>(lane) && row < a.H) {
      float o = res[i] + p;
      if (sh) o += dsh[wave_in_block() * RPW + i * RPI + sub];
      a.out[row] = o;
    }
  }
  trace_mark(a.trace, 3);
}

// ------------------------------------------------------------------ host dispatch

#define FMOE_NG_SWITCH(ng, FN, ...)          \
  switch (ng) {                              \
    case 4: return FN<4>(__VA_ARGS__);       \
    case 8: return FN<8>(__VA_ARGS__);       \
    case 16: return FN<16>(__VA_ARGS__);     \
    case 32: return FN<32>(__VA_ARGS__);     \
    case 64: return FN<64>(__VA_ARGS__);     \
    default: return hipErrorInvalidValue;    \
  }

inline int blocks_for(long waves) { return (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock); }

// Launch geometry of one layer's three kernels (NGH, NGI: the hidden and inter
// group counts rounded up to powers of two).
template <int BITS, int NGH, int NGI>
struct LayerGeom {
  static constexpr int RPIH = kWave / NGH;
  int n1r, n2r, n2s, n3, wps, kpad;
  __host__ LayerGeom(const LayerArgs &L, int bits) {
    const bool sh = L.shared != nullptr;
    n1r = (L.E + kWavesPerBlock / router_split<NGH>() - 1) / (kWavesPerBlock / router_split<NGH>());
    const int GI = gateup_iters(L.K);
    wps = (L.I / RPIH + GI - 1) / GI;
    n2r = blocks_for((long)wps * L.K);
    n2s = sh ? blocks_for(wps) : 0;
    kpad = down_slots(L.K, NGI);
    const int DI = down_iters(kpad);
    const int slots = kpad * NGI;
    const int seg = slots < kWave ? slots : kWave;
    const long w3 = ((long)L.H / (kWave / seg) + DI - 1) / DI;
    n3 = (int)((w3 + kP3Waves - 1) / kP3Waves);
  }
};

template <int BITS>
struct Dispatch {
  template <int NGP>
  static hipError_t qmatvec(const uint8_t *blob, int ng, int rows, const float *x, float *y, hipStream_t s) {
    constexpr int RPI = kWave / NGP;
    const long iters = (rows + RPI - 1) / RPI;
    // Enough wavefronts to cover every SIMD several times over; more rows per
    // wavefront only once there is work to spare.
    if (iters >= 4L * 4096)
      hipLaunchKernelGGL((k_qmatvec<BITS, NGP, 4>), dim3(blocks_for((iters + 3) / 4)), dim3(kBlock), 0, s, blob, ng,
                         rows, x, y);
    else if (iters >= 2L * 2048)
      hipLaunchKernelGGL((k_qmatvec<BITS, NGP, 2>), dim3(blocks_for((iters + 1) / 2)), dim3(kBlock), 0, s, blob, ng,
                         rows, x, y);
    else
      hipLaunchKernelGGL((k_qmatvec<BITS, NGP, 1>), dim3(blocks_for(iters)), dim3(kBlock), 0, s, blob, ng, rows, x,
                         y);
    return hipGetLastError();
  }

  template <int NGP>
  static hipError_t gateup(const uint8_t *gu, int ng, int inter, const float *x, float *h, hipStream_t s) {
    constexpr int RPI = kWave / NGP;
    const long waves = inter / RPI;
    hipLaunchKernelGGL((k_expert_gateup<BITS, NGP, 1>), dim3(blocks_for(waves)), dim3(kBlock), 0, s, gu, ng, inter, x,
                       h);
    return hipGetLastError();
  }

  template <int NGH, int NGI, int KPAD, int FORM = -1, bool PTR = false>
  static hipError_t phase3(const LayerArgs &L, const LayerGeom<BITS, NGH, NGI> &G, hipStream_t s) {
    Phase3Args p3{};
    p3.bank = L.bank;
    p3.stride = L.expert_stride;
    p3.gu_bytes = L.gateup_bytes;
    p3.idx = L.ws_idx;
    p3.w = L.ws_w;
    p3.K = L.K;
    p3.h_routed = L.h_routed;
    p3.I = L.I;
    p3.H = L.H;
    p3.shared_down = L.shared ? L.shared + L.gateup_bytes : nullptr;
    p3.h_shared = L.h_shared;
    p3.sigma = L.sigma;
    p3.residual = L.residual;
    p3.out = L.out;
    p3.trace = L.trace ? L.trace + (size_t)2 * kTraceBlocks * kTraceSlots : nullptr;
    p3.expert_ptr = L.expert_ptr;
    hipLaunchKernelGGL((k_phase3<BITS, NGI, KPAD, FORM, PTR>), dim3(G.n3), dim3(kP3Block), 0, s, p3);
    return hipGetLastError();
  }

  template <int NGH, int NGI>
  static hipError_t phase1(const LayerArgs &L, const LayerGeom<BITS, NGH, NGI> &G, hipStream_t s) {
    const bool has_shared = L.shared != nullptr;
    Phase1Args p1{};
    p1.router = L.router;
    p1.gvec = has_shared ? L.shared_gate : nullptr;
    p1.E = L.E;
    p1.bits = BITS;
    p1.x = L.x;
    p1.rms_eps = L.rms_eps;
    p1.logits = L.logits;
    p1.sigma = L.sigma;
    p1.xdig = L.xdig;
    p1.ng = L.H / kGroup;
    p1.n_prep_blocks = (p1.ng + kWavesPerBlock - 1) / kWavesPerBlock + (has_shared ? 1 : 0);
    p1.xs = L.xs;
    p1.trace = L.trace;
    // before the router's workgroups: one per four 64-column groups of x (digit
    // form), then one for the shared expert's gate
    hipLaunchKernelGGL((k_phase1<NGH>), dim3(G.n1r + p1.n_prep_blocks), dim3(kBlock), 0, s, p1);
    return hipGetLastError();
  }

  template <int NGH, int NGI, int FORM = -1, bool PTR = false>
  static hipError_t phase2(const LayerArgs &L, const LayerGeom<BITS, NGH, NGI> &G, hipStream_t s) {
    const bool has_shared = L.shared != nullptr;
    Phase2Args p2{};
    p2.logits = L.logits;
    p2.E = L.E;
    p2.K = L.K;
    p2.bank = L.bank;
    p2.stride = L.expert_stride;
    p2.xdig = L.xdig;
    p2.ng = L.H / kGroup;
    p2.I = L.I;
    p2.h_routed = L.h_routed;
    p2.ws_idx = L.ws_idx;
    p2.ws_w = L.ws_w;
    p2.out_idx = L.topk_idx_out;
    p2.out_w = L.topk_w_out;
    p2.waves_per_slot = G.wps;
    p2.n_routed_blocks = G.n2r;
    p2.shared_gu = has_shared ? L.shared : nullptr;
    p2.h_shared = L.h_shared;
    p2.xs = L.xs;
    p2.trace = L.trace ? L.trace + (size_t)kTraceBlocks * kTraceSlots : nullptr;
    p2.expert_ptr = L.expert_ptr;
    static_assert(gateup_iters(4) == 2 && gateup_iters(5) == 4, "the builds below");
    const dim3 grid(G.n2r + G.n2s);
    if (L.K <= 4)
      hipLaunchKernelGGL((k_phase2<BITS, NGH, 2, FORM, PTR>), grid, dim3(kBlock), 0, s, p2);
    else if constexpr (FORM < 0)
      hipLaunchKernelGGL((k_phase2<BITS, NGH, 4, -1, PTR>), grid, dim3(kBlock), 0, s, p2);
    else
      return hipErrorInvalidValue;  // (the form builds take at most four slots)
    return hipGetLastError();
  }

  template <int NGH, int NGI, bool PTR = false>
  static hipError_t phase3k(const LayerArgs &L, const LayerGeom<BITS, NGH, NGI> &G, hipStream_t s) {
    if (L.K <= 1) return phase3<NGH, NGI, 1, -1, PTR>(L, G, s);
    if (L.K <= 2) return phase3<NGH, NGI, 2, -1, PTR>(L, G, s);
    if (L.K <= 4) return phase3<NGH, NGI, 4, -1, PTR>(L, G, s);
    if (L.K <= 8) return phase3<NGH, NGI, 8, -1, PTR>(L, G, s);
    if constexpr (down_slots(12, NGI) == 12) {
      if (L.K <= 12) return phase3<NGH, NGI, 12, -1, PTR>(L, G, s);
    }
    return phase3<NGH, NGI, 16, -1, PTR>(L, G, s);
  }

  // PTR: the routed experts' blobs through L.expert_ptr (the tier's table)
  template <int NGH, int NGI, bool PTR = false>
  static hipError_t layer(const LayerArgs &L, hipStream_t s, int phases) {
    const LayerGeom<BITS, NGH, NGI> G(L, BITS);
    hipError_t err = hipSuccess;
    if (phases & 1) err = phase1<NGH, NGI>(L, G, s);
    if (err == hipSuccess && (phases & 2)) err = phase2<NGH, NGI, -1, PTR>(L, G, s);
    if (err == hipSuccess && (phases & 4)) err = phase3k<NGH, NGI, PTR>(L, G, s);
    return err;
  }

  template <int NGH, bool PTR = false>
  static hipError_t layer_h(const LayerArgs &L, hipStream_t s, int phases) {
    switch (pad_groups(L.I / kGroup)) {
      case 4: return layer<NGH, 4, PTR>(L, s, phases);
      case 8: return layer<NGH, 8, PTR>(L, s, phases);
      case 16: return layer<NGH, 16, PTR>(L, s, phases);
      case 32: return layer<NGH, 32, PTR>(L, s, phases);
      case 64: return layer<NGH, 64, PTR>(L, s, phases);
      default: return hipErrorInvalidValue;
    }
  }
};

template <int BITS>
hipError_t qmatvec_b(const uint8_t *blob, int rows, int cols, const float *x, float *y, hipStream_t s) {
  FMOE_NG_SWITCH(pad_groups(cols / kGroup), Dispatch<BITS>::template qmatvec, blob, cols / kGroup, rows, x, y, s)
}

template <int BITS>
hipError_t gateup_b(const uint8_t *gu, int hidden, int inter, const float *x, float *h, hipStream_t s) {
  FMOE_NG_SWITCH(pad_groups(hidden / kGroup), Dispatch<BITS>::template gateup, gu, hidden / kGroup, inter, x, h, s)
}

template <int BITS>
hipError_t layer_b(const LayerArgs &L, hipStream_t s, int phases) {
  FMOE_NG_SWITCH(pad_groups(L.H / kGroup), Dispatch<BITS>::template layer_h, L, s, phases)
}

// The layer's kernels with the routed experts' blobs through L.expert_ptr.
template <int BITS>
hipError_t layer_ptr_b(const LayerArgs &L, hipStream_t s, int phases) {
  switch (pad_groups(L.H / kGroup)) {
    case 4: return Dispatch<BITS>::template layer_h<4, true>(L, s, phases);
    case 8: return Dispatch<BITS>::template layer_h<8, true>(L, s, phases);
    case 16: return Dispatch<BITS>::template layer_h<16, true>(L, s, phases);
    case 32: return Dispatch<BITS>::template layer_h<32, true>(L, s, phases);
    case 64: return Dispatch<BITS>::template layer_h<64, true>(L, s, phases);
    default: return hipErrorInvalidValue;
  }
}

// One token's routing alone (its top-K from the router kernel's logits, which carry
// the RMS factor already): ws_idx / ws_w, as the gate/up kernel derives them.
template <int BITS>
__global__ __launch_bounds__(kWave) void k_route1(const float *logits, int E, int K, int32_t *idx, float *w) {
  __shared__ TopkLds tk;
  int mi;
  float mw;
  wave_topk_lds(logits, E, K, 1.f, tk, mi, mw);
  if (lane_id() < K) {
    idx[lane_id()] = mi;
    w[lane_id()] = mw;
  }
}

template <int BITS>
hipError_t route1_b(const float *logits, int E, int K, int32_t *idx, float *w, hipStream_t s) {
  hipLaunchKernelGGL(k_route1<BITS>, dim3(1), dim3(kWave), 0, s, logits, E, K, idx, w);
  return hipGetLastError();
}

}  // namespace dev
}  // namespace fmoe
