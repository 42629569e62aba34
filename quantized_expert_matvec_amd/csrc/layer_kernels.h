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

// ------------------------------------------------------------------ row work

// Weight registers of ITERS row iterations of one wavefront (NG lanes per row).
template <int BITS, int NG, int ITERS>
struct RowLoads {
  Chunk<BITS> c[ITERS];
  uint32_t sb[ITERS];
  // rows row0 + i*RPI + sub (clamped to rows-1) of a matrix with records of RB bytes
  __device__ __forceinline__ void issue(const uint8_t *__restrict__ blob, int rows, int row0) {
    constexpr int RPI = kWave / NG;
    constexpr size_t RB = (size_t)NG * gbytes<BITS>();
    const int lane = lane_id();
    const int g = lane & (NG - 1), sub = lane / NG;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const int row = min(row0 + i * RPI + sub, rows - 1);
      load_group<BITS, NG>(blob + (size_t)row * RB, g, c[i], sb[i]);
    }
    __builtin_amdgcn_sched_barrier(0);  // (as in PairLoads::issue)
  }
  // y[row] = alpha * row . x
  __device__ __forceinline__ void finish(const XSlice &xs, float *__restrict__ y, int rows, int row0,
                                         float alpha) const {
    constexpr int RPI = kWave / NG;
    const int lane = lane_id();
    const int sub = lane / NG;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const float p = seg_reduce<NG>(group_partial<BITS>(c[i], sb[i], xs));
      const int row = row0 + i * RPI + sub;
      if (seg_last<NG>(lane) && row < rows) y[row] = alpha * p;
    }
  }
};

// Row pairs of an interleaved gate/up region (records 2r and 2r+1).
template <int BITS, int NG, int ITERS>
struct PairLoads {
  Chunk<BITS> cg[ITERS], cu[ITERS];
  uint32_t sg[ITERS], su[ITERS];
  __device__ __forceinline__ void issue(const uint8_t *__restrict__ gu, int pair0) {
    constexpr int RPI = kWave / NG;
    constexpr size_t RB = (size_t)NG * gbytes<BITS>();
    const int lane = lane_id();
    const int g = lane & (NG - 1), sub = lane / NG;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const uint8_t *rec = gu + (size_t)(2 * (pair0 + i * RPI + sub)) * RB;
      load_group<BITS, NG>(rec, g, cg[i], sg[i]);
      load_group<BITS, NG>(rec + RB, g, cu[i], su[i]);
    }
    // every load goes out before the first use of a loaded word (otherwise the
    // scheduler can hoist that use between the loads, and its wait stalls the rest)
    __builtin_amdgcn_sched_barrier(0);
  }
  // h[r] = silu(gate_r . x) * (up_r . x)
  __device__ __forceinline__ void finish(const XSlice &xs, float *__restrict__ h, int pair0) const {
    constexpr int RPI = kWave / NG;
    const int lane = lane_id();
    const int sub = lane / NG;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const float pg = seg_reduce<NG>(group_partial<BITS>(cg[i], sg[i], xs));
      const float pu = seg_reduce<NG>(group_partial<BITS>(cu[i], su[i], xs));
      if (seg_last<NG>(lane)) h[pair0 + i * RPI + sub] = silu(pg) * pu;
    }
  }
  // the same from the digit form of x
  __device__ __forceinline__ void finish_dig(const XDig &xd, float *__restrict__ h, int pair0) const {
    constexpr int RPI = kWave / NG;
    const int lane = lane_id();
    const int sub = lane / NG;
#pragma unroll
    for (int i = 0; i < ITERS; ++i) {
      const float pg = seg_reduce<NG>(group_partial_dig<BITS>(cg[i], sg[i], xd));
      const float pu = seg_reduce<NG>(group_partial_dig<BITS>(cu[i], su[i], xd));
      if (seg_last<NG>(lane)) h[pair0 + i * RPI + sub] = silu(pg) * pu;
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
//
// Fast path: each lane's maximum (first position among equal keys) and second
// key; K rounds over the 64 lane maxima (wavefront maximum, lowest lane holding
// it) give the K best lane maxima in order, and they are the top K of all
// elements when no second key reaches the K-th of them. Otherwise (a lane holding
// two of the top K, or a tie at the boundary) K full rounds run: each lane's
// maximum over its remaining keys, the wavefront maximum, the lowest lane holding
// it and that lane's first position holding it; the chosen key is retired.
//
// Then the renormalised softmax weights of the chosen K,
// w_j = exp(l_j - l_0) / sum (renormalising over the chosen K cancels the full
// softmax denominator). The logits may be held unscaled: lscale > 0 is the
// factor that turns them into the true logits (it does not change the order), so
// w_j = exp((l_j - l_0) * lscale) / sum. Results are wavefront-uniform.
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

template <int VPL>
__device__ __forceinline__ void wave_topk_keys(int (&key)[VPL], int K, int *idx, float *w, float lscale) {
  constexpr int kGone = (int)0x80000000;
  const int lane = lane_id();
  int m1, p1, m2 = kGone;
  lane_max<VPL>(key, m1, p1);
#pragma unroll
  for (int m = 0; m < VPL; ++m) m2 = m == p1 ? m2 : max(m2, key[m]);
  int a = m1, T = kGone;
  float lv[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    idx[j] = 0;
    lv[j] = 0.f;
    if (j < K) {
      const int g = wave_max_i(a);
      const int L = __ffsll((long long)__ballot(a == g)) - 1;
      idx[j] = VPL * L + __builtin_amdgcn_readlane(p1, L);
      lv[j] = key_value(g);
      a = lane == L ? kGone : a;
      T = g;
    }
  }
  if (wave_max_i(m2) >= T) {
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) {
      if (j < K) {
        int b, p;
        lane_max<VPL>(key, b, p);
        const int g = wave_max_i(b);
        const int L = __ffsll((long long)__ballot(b == g)) - 1;
        const int pl = __builtin_amdgcn_readlane(p, L);
        idx[j] = VPL * L + pl;
        lv[j] = key_value(g);
#pragma unroll
        for (int m = 0; m < VPL; ++m) key[m] = (lane == L && m == pl) ? kGone : key[m];
      }
    }
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) {
    w[j] = 0.f;
    if (j < K) {
      w[j] = __expf((lv[j] - lv[0]) * lscale);
      sum += w[j];
    }
  }
  const float inv = 1.f / sum;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) w[j] *= inv;
}

// lane l's VPL consecutive logits, with 16-byte loads (clamped to the row; lg
// 16-byte aligned and readable up to E rounded up to 4; the caller turns the
// values into keys, those past E into the lowest key): one load instruction of
// the wavefront covers whole cache lines, where VPL-strided 4-byte loads would
// touch VPL times as many lines per instruction.
template <int VPL>
__device__ __forceinline__ void load_logits(const float *lg, int E, float (&v)[VPL]) {
  const int lane = lane_id();
  const float4 *l4 = reinterpret_cast<const float4 *>(lg);
#pragma unroll
  for (int q = 0; q < VPL / 4; ++q) {
    const float4 t = l4[min(VPL / 4 * lane + q, (E + 3) / 4 - 1)];
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

// top-K of E <= kMaxExperts logits in memory (LDS or global)
__device__ __forceinline__ void wave_topk_lds(const float *lg, int E, int K, int *idx, float *w,
                                              float lscale = 1.f) {
  if (E <= 512) {
    float v[8];
    int key[8];
    load_logits<8>(lg, E, v);
    logit_keys<8>(v, E, key);
    wave_topk_keys<8>(key, K, idx, w, lscale);
  } else {
    float v[16];
    int key[16];
    load_logits<16>(lg, E, v);
    logit_keys<16>(v, E, key);
    wave_topk_keys<16>(key, K, idx, w, lscale);
  }
}

// Block-wide top-K: one wavefront computes it from the logits in LDS and
// publishes it through LDS (sidx, sw); contains one barrier, after which every
// thread reads the result from sidx / sw. (Results are not copied back into
// per-thread arrays: indexing those by a runtime slot would put them in scratch
// memory.) Workgroup b uses wavefront b % 4, so that the workgroups sharing a CU
// do not all compute it on the same SIMD. (Measured: splitting the rounds over
// the four wavefronts, with one barrier per round, is slower.)
__device__ __forceinline__ void block_topk(const float *lg, int E, int K, int *sidx, float *sw) {
  if (wave_in_block() == (int)(blockIdx.x % kWavesPerBlock)) {
    // the rest of the workgroup waits on this wavefront: let it win the SIMD's
    // issue arbitration against co-resident wavefronts of other workgroups
    __builtin_amdgcn_s_setprio(3);
    int idx[kMaxTopK];
    float w[kMaxTopK];
    wave_topk_lds(lg, E, K, idx, w);
    __builtin_amdgcn_s_setprio(0);
    const int lane = lane_id();
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j)
      if (j == lane) {
        sidx[j] = idx[j];
        sw[j] = w[j];
      }
  }
  __syncthreads();
}

// ------------------------------------------------------------------ standalone kernels

template <int BITS, int NG, int ITERS>
__global__ __launch_bounds__(kBlock) void k_qmatvec(const uint8_t *__restrict__ blob, int rows,
                                                     const float *__restrict__ x, float *__restrict__ y) {
  __shared__ float xl[NG * kXPad];
  constexpr int X4 = (NG * 16 + kBlock - 1) / kBlock;
  const int row0 = wave_id() * ITERS * (kWave / NG);
  Staged<X4> xst;
  stage_load(x, NG * 16, xst);
  RowLoads<BITS, NG, ITERS> L;
  if (row0 < rows) L.issue(blob, rows, row0);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<X4, false>(xst, NG * 16, xl, nullptr);
  __syncthreads();
  if (row0 >= rows) return;
  XSlice xs;
  read_slice(xl, lane_id() & (NG - 1), 1.f, xs);
  L.finish(xs, y, rows, row0, 1.f);
}

template <int BITS, int NG, int ITERS>
__global__ __launch_bounds__(kBlock) void k_expert_gateup(const uint8_t *__restrict__ gu, int inter,
                                                           const float *__restrict__ x, float *__restrict__ h) {
  __shared__ float xl[NG * kXPad];
  constexpr int X4 = (NG * 16 + kBlock - 1) / kBlock;
  const int pair0 = wave_id() * ITERS * (kWave / NG);
  Staged<X4> xst;
  stage_load(x, NG * 16, xst);
  PairLoads<BITS, NG, ITERS> P;
  if (pair0 < inter) P.issue(gu, pair0);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<X4, false>(xst, NG * 16, xl, nullptr);
  __syncthreads();
  if (pair0 >= inter) return;
  XSlice xs;
  read_slice(xl, lane_id() & (NG - 1), 1.f, xs);
  P.finish(xs, h, pair0);
}

// ------------------------------------------------------------------ layer kernels

constexpr int kP2GateUpIters = 2;  // gate/up pair iterations per wavefront (routed and shared)
constexpr int kP3Iters = 4;        // routed down row iterations per wavefront
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
  int n_prep_blocks;  // workgroups before the router's: x in digit form, then the gate
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
// wavefronts of a workgroup (half h: lane l covers columns 4l + 256t + 0..3 for
// t in [h NT/2, (h+1) NT/2)), so that the 8 MB of rows spread over every compute
// unit (512 rows: one workgroup per compute unit); the halves' sums are added in
// order. The workgroups before the router's write x in digit form for the gate/up
// kernel, and the last of them computes the shared expert's gate sigmoid(g . x).
template <int NGH>
constexpr int router_split() {
  return NGH / 4 >= 2 ? 2 : 1;
}
template <int NGH>
__global__ __launch_bounds__(kBlock) void k_phase1(const Phase1Args a) {
  constexpr int NT = NGH / 4;  // hidden / 256
  constexpr int H = NGH * kGroup;
  constexpr int X4 = (NGH * 16 + kBlock - 1) / kBlock;
  constexpr int SPLIT = router_split<NGH>();
  constexpr int NTW = NT / SPLIT;  // float4 per lane of this wavefront's part of the row
  __shared__ float xl[NGH * kXPad];
  __shared__ float part[kWavesPerBlock];
  __shared__ float dpart[kWavesPerBlock];
  __shared__ uint32_t ybuf[kWavesPerBlock][kWave];
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
    const bool gate = a.gvec != nullptr && (int)blockIdx.x == (NGH + kWavesPerBlock - 1) / kWavesPerBlock;
    Staged<X4> xst, gst;
    stage_load(a.x, NGH * 16, xst);
    stage_load(gate ? a.gvec : a.x, NGH * 16, gst);
    if (rms)
      stage_store<X4, true>(xst, NGH * 16, xl, part);
    else
      stage_store<X4, false>(xst, NGH * 16, xl, part);
    __syncthreads();
    const float inv = rms ? rms_inv(part, H, a.rms_eps) : 1.f;
    if (gate) {  // (uniform over the workgroup)
      float acc = 0.f;
#pragma unroll
      for (int k = 0; k < X4; ++k) {
        const int f = threadIdx.x + kBlock * k;
        if (f < NGH * 16) {
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
    } else if (g < NGH) {
      if (a.bits == 4)
        write_digits<4>(xl, g, inv, ybuf[wv], a.xdig);
      else
        write_digits<2>(xl, g, inv, ybuf[wv], a.xdig);
    }
    trace_mark(a.trace, 3);
    return;
  }
  const int n_rows = a.E;
  const int half = wv % SPLIT;
  const int row = ((int)blockIdx.x - a.n_prep_blocks) * (kWavesPerBlock / SPLIT) + wv / SPLIT;
  const int rr = min(row, n_rows - 1);
  const float *src = a.router + (size_t)rr * H + 256 * NTW * half;
  Staged<X4> xst;
  stage_load(a.x, NGH * 16, xst);
  float4 w[NTW];
#pragma unroll
  for (int t = 0; t < NTW; ++t) w[t] = reinterpret_cast<const float4 *>(src)[lane + 64 * t];
  __builtin_amdgcn_sched_barrier(0);
  if (rms)
    stage_store<X4, true>(xst, NGH * 16, xl, part);
  else
    stage_store<X4, false>(xst, NGH * 16, xl, part);
  __syncthreads();
  trace_mark(a.trace, 1);
  const float inv = rms ? rms_inv(part, H, a.rms_eps) : 1.f;
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < NTW; ++t) {
    const float4 xv = *reinterpret_cast<const float4 *>(&xl[lds_index(4 * lane + 256 * (t + NTW * half))]);
    acc = fmaf(w[t].x, xv.x * inv, acc);
    acc = fmaf(w[t].y, xv.y * inv, acc);
    acc = fmaf(w[t].z, xv.z * inv, acc);
    acc = fmaf(w[t].w, xv.w * inv, acc);
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
  uint64_t *trace;
};

// Phase 2. Routed blocks stage the logits and x (in digit form), derive the
// top-K (one wavefront per block), then run gate/up + SwiGLU of their slot's
// expert. Shared blocks run the shared expert's gate/up + SwiGLU: it does not
// depend on the routing, so its weights stream while the routed blocks are still
// choosing. x arrives in the digit form the router kernel wrote (RMS factor
// included), so this kernel reads no raw x.
template <int BITS, int NGH>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(3))) void k_phase2(const Phase2Args a) {
  constexpr int RPIH = kWave / NGH;
  constexpr int NF4 = NGH * kDigStride / 4;  // 16-byte units of the digit form
  constexpr int D4 = (NF4 + kBlock - 1) / kBlock;
  __shared__ uint32_t xdl[NGH * kDigStride];
  __shared__ __align__(16) float lg[kMaxExperts];
  __shared__ int sidx[kMaxTopK];
  __shared__ float sw[kMaxTopK];
  const int lane = lane_id();
  const float *xsrc = reinterpret_cast<const float *>(a.xdig);
  trace_mark(a.trace, 0);
  if ((int)blockIdx.x < a.n_routed_blocks) {
    // a workgroup serves one slot (waves_per_slot is a multiple of 4) and needs
    // only the first slot+1 winners: the rounds stop there, so the workgroups of
    // the early slots start streaming before the last winner is known. The
    // workgroup that publishes the routing is one of the last slot's (all K).
    const int bslot = min((int)(blockIdx.x * kWavesPerBlock) / a.waves_per_slot, a.K - 1);
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
        int key[8], idx[kMaxTopK];
        float w[kMaxTopK];
        logit_keys<8>(lv, a.E, key);
        // the rest of the workgroup waits on this wavefront: let it win the
        // SIMD's issue arbitration against co-resident wavefronts of other workgroups
        __builtin_amdgcn_s_setprio(3);
        wave_topk_keys<8>(key, bslot + 1, idx, w, 1.f);
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int j = 0; j < kMaxTopK; ++j)
          if (j == lane) {
            sidx[j] = idx[j];
            sw[j] = w[j];
          }
      } else {
        stage_load(xsrc, NF4, xst);
      }
      stage_copy(xst, NF4, xdl);
      __syncthreads();
      trace_mark(a.trace, 1);
    } else {
      for (int i = threadIdx.x; i < a.E; i += kBlock) lg[i] = a.logits[i];
      Staged<D4> xst;
      stage_load(xsrc, NF4, xst);
      stage_copy(xst, NF4, xdl);
      __syncthreads();
      trace_mark(a.trace, 1);
      block_topk(lg, a.E, bslot + 1, sidx, sw);
    }
    trace_mark(a.trace, 2);
    const int wv = blockIdx.x * kWavesPerBlock + wave_in_block();
    const int slot = min(wv / a.waves_per_slot, a.K - 1);
    const int pair0 = (wv % a.waves_per_slot) * kP2GateUpIters * RPIH;
    const bool active = wv < a.waves_per_slot * a.K;
    PairLoads<BITS, NGH, kP2GateUpIters> P;
    if (active) P.issue(a.bank + (size_t)sidx[slot] * a.stride, pair0);
    if (wv == (a.K - 1) * a.waves_per_slot && lane < a.K) {
      const int sel = sidx[lane];
      const float ws = sw[lane];
      a.ws_idx[lane] = sel;
      a.ws_w[lane] = ws;
      if (a.out_idx) a.out_idx[lane] = sel;
      if (a.out_w) a.out_w[lane] = ws;
    }
    if (active) {
      XDig xd;
      read_digits(xdl, lane & (NGH - 1), xd);
      P.finish_dig(xd, a.h_routed + (size_t)slot * a.I, pair0);
    }
    trace_mark(a.trace, 3);
    return;
  }
  // shared expert gate/up
  const int wv = (blockIdx.x - a.n_routed_blocks) * kWavesPerBlock + wave_in_block();
  const int pair0 = wv * kP2GateUpIters * RPIH;
  // x first (its loads complete before the weights', so the staging does not
  // wait for them), then the weights
  Staged<D4> xst;
  stage_load(xsrc, NF4, xst);
  __builtin_amdgcn_sched_barrier(0);
  PairLoads<BITS, NGH, kP2GateUpIters> P;
  if (pair0 < a.I) P.issue(a.shared_gu, pair0);
  stage_copy(xst, NF4, xdl);
  __syncthreads();
  trace_mark(a.trace, 1);
  if (pair0 < a.I) {
    XDig xd;
    read_digits(xdl, lane & (NGH - 1), xd);
    P.finish_dig(xd, a.h_shared, pair0);
  }
  trace_mark(a.trace, 3);
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
};

// Phase 3: out_i = residual_i + sum_k w_k (down_k . h_k)_i + sigma (down_s . h_s)_i.
// Routed: lanes are (slot k, group j) pairs, so one cross-lane sum adds the K
// experts' weighted partials of a row together; each lane keeps its slot's h
// slice. KPAD = top_k rounded up to a power of two (slots beyond top_k stay
// idle). The routed h vectors are staged in LDS when they fit (KPAD * inter <=
// 8192). Shared: the same wavefront's rows, NGI lanes per row; its weights do not
// depend on the routing and are requested first. A wavefront passes its shared
// results from the shared lanes to the combining lanes through LDS.
template <int BITS, int NGI, int KPAD>
__global__ __launch_bounds__(kP3Block) void k_phase3(const Phase3Args a) {
  constexpr int SLOTS = KPAD * NGI;
  constexpr int SEG = SLOTS < kWave ? SLOTS : kWave;  // lanes per row
  constexpr int SPL = SLOTS / SEG;                     // slots per lane
  constexpr int RPI = kWave / SEG;
  constexpr int RPW = kP3Iters * RPI;                  // rows per wavefront
  constexpr int RPII = kWave / NGI;                    // shared-down rows per iteration
  constexpr int SIT = (RPW + RPII - 1) / RPII;         // shared-down iterations
  constexpr size_t RB = (size_t)NGI * gbytes<BITS>();
  constexpr bool STAGE = KPAD * NGI <= 128;
  __shared__ float hl[STAGE ? KPAD * NGI * kXPad : 1];
  __shared__ float hs[NGI * kXPad];
  __shared__ float hlsum[STAGE ? KPAD * NGI : 1];  // per-group sums of the staged h
  __shared__ float hssum[NGI];
  __shared__ float dsh[kP3Waves * RPW];
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
    const int k = slot / NGI;
    grp[m] = slot % NGI;
    act[m] = k < a.K && row0 < a.H;
    kk[m] = k < a.K ? k : 0;
    sel[m] = a.idx[kk[m]];
    wk[m] = k < a.K ? a.w[kk[m]] : 0.f;
  }
  float res[kP3Iters];
#pragma unroll
  for (int i = 0; i < kP3Iters; ++i) res[i] = a.residual[min(row0 + i * RPI + sub, a.H - 1)];
  const float sig = *a.sigma;  // (a workspace value; unused without a shared expert)
  constexpr int H4 = STAGE ? (KPAD * NGI * 16 + kP3Block - 1) / kP3Block : 1;
  constexpr int S4 = (NGI * 16 + kP3Block - 1) / kP3Block;
  Staged<H4> hst;
  if constexpr (STAGE) stage_load<H4, kP3Block>(a.h_routed, a.K * a.I / 4, hst);
  // without a shared expert these loads read the routed expert 0 instead (valid
  // memory, results unused): unconditional loads keep the memory-counter waits exact
  Staged<S4> sst;
  stage_load<S4, kP3Block>(sh ? a.h_shared : a.h_routed, NGI * 16, sst);
  __builtin_amdgcn_sched_barrier(0);  // every h load goes out before any weight load
  const uint8_t *sdown = sh ? a.shared_down : a.bank + a.gu_bytes;
  // shared rows: NGI lanes per row; with fewer rows per wavefront than a load
  // covers, the spare lanes repeat this wavefront's rows (the same cache lines)
  const int ssub = RPW < RPII ? (lane / NGI) % RPW : lane / NGI, sg = lane & (NGI - 1);
  Chunk<BITS> cs[SIT];
  uint32_t ss[SIT];
#pragma unroll
  for (int q = 0; q < SIT; ++q) {
    const int row = min(row0 + q * RPII + ssub, a.H - 1);
    load_group<BITS, NGI>(sdown + (size_t)row * RB, sg, cs[q], ss[q]);
  }
  __builtin_amdgcn_sched_barrier(0);  // the shared rows go out before the routing is needed
  const uint8_t *base[SPL];
#pragma unroll
  for (int m = 0; m < SPL; ++m) {
    asm volatile("" : "+v"(sel[m]));  // (keeps the address arithmetic, and its wait, here)
    base[m] = a.bank + (size_t)sel[m] * a.stride + a.gu_bytes;
  }
  Chunk<BITS> c[kP3Iters][SPL];
  uint32_t sb[kP3Iters][SPL];
#pragma unroll
  for (int i = 0; i < kP3Iters; ++i) {
    const int row = min(row0 + i * RPI + sub, a.H - 1);
    // unconditional (inactive slots reload slot 0's rows, unused), as above
#pragma unroll
    for (int m = 0; m < SPL; ++m) load_group<BITS, NGI>(base[m] + (size_t)row * RB, grp[m], c[i][m], sb[i][m]);
  }
  __builtin_amdgcn_sched_barrier(0);  // the h vectors were requested before the weights
  if constexpr (STAGE) stage_store_gsum<H4, kP3Block>(hst, a.K * a.I / 4, hl, hlsum);
  stage_store_gsum<S4, kP3Block>(sst, NGI * 16, hs, hssum);
  __syncthreads();
  trace_mark(a.trace, 1);
  if (row0 >= a.H) return;
  if (sh) {
    XSlice xs;
    read_slice_sum(hs, sg, hssum[sg], xs);
#pragma unroll
    for (int q = 0; q < SIT; ++q) {
      const float p = seg_reduce<NGI>(group_partial<BITS>(cs[q], ss[q], xs));
      const int r = q * RPII + ssub;  // row within this wavefront's rows
      if (seg_last<NGI>(lane) && r < RPW) dsh[wave_in_block() * RPW + r] = sig * p;
    }
  }
  XSlice xs[SPL];
  if constexpr (STAGE) {
#pragma unroll
    for (int m = 0; m < SPL; ++m) read_slice_sum(hl, kk[m] * NGI + grp[m], hlsum[kk[m] * NGI + grp[m]], xs[m]);
  } else {
#pragma unroll
    for (int m = 0; m < SPL; ++m) load_xslice(a.h_routed + (size_t)kk[m] * a.I + kGroup * grp[m], xs[m]);
  }
#pragma unroll
  for (int i = 0; i < kP3Iters; ++i) {
    float p = 0.f;
#pragma unroll
    for (int m = 0; m < SPL; ++m)
      if (act[m]) p = fmaf(wk[m], group_partial<BITS>(c[i][m], sb[i][m], xs[m]), p);
    p = seg_reduce<SEG>(p);
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

// Launch geometry of one layer's three kernels.
template <int NGH, int NGI>
struct LayerGeom {
  static constexpr int RPIH = kWave / NGH, RPII = kWave / NGI;
  int n1r, n1s, n2r, n2s, n3, wps, kpad;
  size_t rbh, rbi;
  __host__ LayerGeom(const LayerArgs &L, int bits) {
    const bool sh = L.shared != nullptr;
    rbh = (size_t)NGH * (bits == 4 ? 36 : 20);
    rbi = (size_t)NGI * (bits == 4 ? 36 : 20);
    n1r = (L.E + kWavesPerBlock / router_split<NGH>() - 1) / (kWavesPerBlock / router_split<NGH>());
    n1s = 0;
    wps = (L.I / RPIH + kP2GateUpIters - 1) / kP2GateUpIters;
    n2r = blocks_for((long)wps * L.K);
    n2s = sh ? blocks_for(wps) : 0;
    kpad = 1;
    while (kpad < L.K) kpad <<= 1;
    const int slots = kpad * NGI;
    const int seg = slots < kWave ? slots : kWave;
    const long w3 = ((long)L.H / (kWave / seg) + kP3Iters - 1) / kP3Iters;
    n3 = (int)((w3 + kP3Waves - 1) / kP3Waves);
  }
};

template <int BITS>
struct Dispatch {
  template <int NG>
  static hipError_t qmatvec(const uint8_t *blob, int rows, const float *x, float *y, hipStream_t s) {
    constexpr int RPI = kWave / NG;
    const long iters = (rows + RPI - 1) / RPI;
    // Enough wavefronts to cover every SIMD several times over; more rows per
    // wavefront only once there is work to spare.
    if (iters >= 4L * 4096)
      hipLaunchKernelGGL((k_qmatvec<BITS, NG, 4>), dim3(blocks_for((iters + 3) / 4)), dim3(kBlock), 0, s, blob, rows,
                         x, y);
    else if (iters >= 2L * 2048)
      hipLaunchKernelGGL((k_qmatvec<BITS, NG, 2>), dim3(blocks_for((iters + 1) / 2)), dim3(kBlock), 0, s, blob, rows,
                         x, y);
    else
      hipLaunchKernelGGL((k_qmatvec<BITS, NG, 1>), dim3(blocks_for(iters)), dim3(kBlock), 0, s, blob, rows, x, y);
    return hipGetLastError();
  }

  template <int NG>
  static hipError_t gateup(const uint8_t *gu, int inter, const float *x, float *h, hipStream_t s) {
    constexpr int RPI = kWave / NG;
    const long waves = inter / RPI;
    hipLaunchKernelGGL((k_expert_gateup<BITS, NG, 1>), dim3(blocks_for(waves)), dim3(kBlock), 0, s, gu, inter, x, h);
    return hipGetLastError();
  }

  template <int NGH, int NGI, int KPAD>
  static hipError_t phase3(const LayerArgs &L, const LayerGeom<NGH, NGI> &G, hipStream_t s) {
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
    hipLaunchKernelGGL((k_phase3<BITS, NGI, KPAD>), dim3(G.n3), dim3(kP3Block), 0, s, p3);
    return hipGetLastError();
  }

  template <int NGH, int NGI>
  static hipError_t phase1(const LayerArgs &L, const LayerGeom<NGH, NGI> &G, hipStream_t s) {
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
    p1.n_prep_blocks = (NGH + kWavesPerBlock - 1) / kWavesPerBlock + (has_shared ? 1 : 0);
    p1.trace = L.trace;
    // before the router's workgroups: one per four 64-column groups of x (digit
    // form), then one for the shared expert's gate
    hipLaunchKernelGGL((k_phase1<NGH>), dim3(G.n1r + p1.n_prep_blocks), dim3(kBlock), 0, s, p1);
    return hipGetLastError();
  }

  template <int NGH, int NGI>
  static hipError_t phase2(const LayerArgs &L, const LayerGeom<NGH, NGI> &G, hipStream_t s) {
    const bool has_shared = L.shared != nullptr;
    Phase2Args p2{};
    p2.logits = L.logits;
    p2.E = L.E;
    p2.K = L.K;
    p2.bank = L.bank;
    p2.stride = L.expert_stride;
    p2.xdig = L.xdig;
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
    p2.trace = L.trace ? L.trace + (size_t)kTraceBlocks * kTraceSlots : nullptr;
    hipLaunchKernelGGL((k_phase2<BITS, NGH>), dim3(G.n2r + G.n2s), dim3(kBlock), 0, s, p2);
    return hipGetLastError();
  }

  template <int NGH, int NGI>
  static hipError_t phase3k(const LayerArgs &L, const LayerGeom<NGH, NGI> &G, hipStream_t s) {
    if (L.K <= 1) return phase3<NGH, NGI, 1>(L, G, s);
    if (L.K <= 2) return phase3<NGH, NGI, 2>(L, G, s);
    if (L.K <= 4) return phase3<NGH, NGI, 4>(L, G, s);
    return phase3<NGH, NGI, 8>(L, G, s);
  }

  template <int NGH, int NGI>
  static hipError_t layer(const LayerArgs &L, hipStream_t s, int phases) {
    const LayerGeom<NGH, NGI> G(L, BITS);
    hipError_t err = hipSuccess;
    if (phases & 1) err = phase1<NGH, NGI>(L, G, s);
    if (err == hipSuccess && (phases & 2)) err = phase2<NGH, NGI>(L, G, s);
    if (err == hipSuccess && (phases & 4)) err = phase3k<NGH, NGI>(L, G, s);
    return err;
  }

  template <int NGH>
  static hipError_t layer_h(const LayerArgs &L, hipStream_t s, int phases) {
    switch (L.I / kGroup) {
      case 4: return layer<NGH, 4>(L, s, phases);
      case 8: return layer<NGH, 8>(L, s, phases);
      case 16: return layer<NGH, 16>(L, s, phases);
      case 32: return layer<NGH, 32>(L, s, phases);
      case 64: return layer<NGH, 64>(L, s, phases);
      default: return hipErrorInvalidValue;
    }
  }
};

template <int BITS>
hipError_t qmatvec_b(const uint8_t *blob, int rows, int cols, const float *x, float *y, hipStream_t s) {
  FMOE_NG_SWITCH(cols / kGroup, Dispatch<BITS>::template qmatvec, blob, rows, x, y, s)
}

template <int BITS>
hipError_t gateup_b(const uint8_t *gu, int hidden, int inter, const float *x, float *h, hipStream_t s) {
  FMOE_NG_SWITCH(hidden / kGroup, Dispatch<BITS>::template gateup, gu, inter, x, h, s)
}

template <int BITS>
hipError_t layer_b(const LayerArgs &L, hipStream_t s, int phases) {
  FMOE_NG_SWITCH(L.H / kGroup, Dispatch<BITS>::template layer_h, L, s, phases)
}

}  // namespace dev
}  // namespace fmoe
