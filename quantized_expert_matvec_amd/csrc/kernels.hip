// kernels.hip -- HIP kernels for gfx950 (MI355X) of the quantized MoE expert
// forward at batch 1.
//
// Work mapping. Every quantized matrix is processed with one 64-column group per
// lane: lane g of a row segment loads the group's codes with 128-bit loads
// (two for 4-bit, one for 2-bit; consecutive lanes read consecutive 16-byte
// pieces, so each load instruction of a wavefront covers a contiguous span) and
// its (scale, bias) word, and keeps the matching 64 values of the input vector
// in registers for every row it visits. A row of `cols` columns occupies
// cols/64 lanes; a wavefront covers 64/(cols/64) rows per iteration, and a
// butterfly of cross-lane adds over those lanes finishes each row.
//
// Arithmetic. The pages recast (code*scale + bias)*x as
// fma(code, scale*x, bias*x) ("397B MoE en MacBook: Motor Flash-MoE a 4,4 t/s",
// section "2. Kernel de desquantizacion optimizado con FMA"; German page
// "Flash-MoE: Ausfuehren eines 397B-Parameter-Qwen-Modells auf dem MacBook Pro
// mit reinem C/Metal", section "FMA-optimierter Dequant-Kernel"). Here the same
// identity is applied per group: scale is constant over a group, so
//   sum_j (c_j*scale + bias) x_j = scale * sum_j c_j x_j + bias * sum_j x_j,
// with sum_j x_j computed once per lane. Each code costs one byte-to-float
// conversion and one FMA; a mask of the packed word puts four codes in byte
// lanes (the high nibbles as 16*c, the 2-bit fields as 4^q*c), each such field
// accumulates on its own, and the exact powers of two 1/16 and 4^-q are applied
// once per group.
// Everything is fp32 with a fixed reduction order (bitwise deterministic).
#include <hip/hip_runtime.h>
#include <math.h>

#include "kernels.h"
#include "layout.h"

namespace fmoe {
namespace {

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ float scale_of(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float bias_of(uint32_t w) { return __uint_as_float(w << 16); }

// Hide a masked word from the optimiser so that it does not fold the mask into
// the byte extraction: the backend then selects one v_cvt_f32_ubyte{0..3} per code
// (a bitfield extract followed by a convert would cost two instructions).
__device__ __forceinline__ uint32_t opaque(uint32_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

__device__ __forceinline__ float ub0(uint32_t v) { return (float)(v & 0xFFu); }
__device__ __forceinline__ float ub1(uint32_t v) { return (float)((v >> 8) & 0xFFu); }
__device__ __forceinline__ float ub2(uint32_t v) { return (float)((v >> 16) & 0xFFu); }
__device__ __forceinline__ float ub3(uint32_t v) { return (float)(v >> 24); }

template <int BITS>
struct Chunk;
template <>
struct Chunk<4> {
  uint4 a, b;  // first and second 16-byte half of the group
};
template <>
struct Chunk<2> {
  uint4 a;
};

// One lane's 64 input values for its group. The packing puts column 64g+i of
// group g at unpack position i (4-bit: word i/8, low nibble of byte i%4 for
// i%8 < 4, else high nibble; 2-bit: word i/16, field (i%16)/4, byte i%4), so the
// slice is simply x[64g .. 64g+63] in order.
struct XSlice {
  float v[64];
  float sum;  // plain sum of the 64 values (the bias term's factor)
};

template <int BITS>
__device__ __forceinline__ void load_xslice(const float *__restrict__ xg, XSlice &s) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 t = reinterpret_cast<const float4 *>(xg)[i];
    s.v[4 * i] = t.x;
    s.v[4 * i + 1] = t.y;
    s.v[4 * i + 2] = t.z;
    s.v[4 * i + 3] = t.w;
  }
  float acc = 0.f;
#pragma unroll
  for (int c = 0; c < 64; ++c) acc += s.v[c];
  s.sum = acc;
}

__device__ __forceinline__ float dot_codes(const Chunk<4> &c, const float *v) {
  const uint32_t d[8] = {c.a.x, c.a.y, c.a.z, c.a.w, c.b.x, c.b.y, c.b.z, c.b.w};
  float a0 = 0.f, a1 = 0.f;
#pragma unroll
  for (int hw = 0; hw < 8; ++hw) {
    const uint32_t lo = opaque(d[hw] & 0x0F0F0F0Fu);
    const uint32_t hi = opaque(d[hw] & 0xF0F0F0F0u);
    a0 = fmaf(ub0(lo), v[hw * 8 + 0], a0);
    a0 = fmaf(ub1(lo), v[hw * 8 + 1], a0);
    a0 = fmaf(ub2(lo), v[hw * 8 + 2], a0);
    a0 = fmaf(ub3(lo), v[hw * 8 + 3], a0);
    a1 = fmaf(ub0(hi), v[hw * 8 + 4], a1);
    a1 = fmaf(ub1(hi), v[hw * 8 + 5], a1);
    a1 = fmaf(ub2(hi), v[hw * 8 + 6], a1);
    a1 = fmaf(ub3(hi), v[hw * 8 + 7], a1);
  }
  return fmaf(a1, 0.0625f, a0);  // high nibbles were read as 16*c
}

__device__ __forceinline__ float dot_codes(const Chunk<2> &c, const float *v) {
  const uint32_t d[4] = {c.a.x, c.a.y, c.a.z, c.a.w};
  float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int w = 0; w < 4; ++w)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t m = opaque(d[w] & (0x03030303u << (2 * q)));
      a[q] = fmaf(ub0(m), v[(w * 4 + q) * 4 + 0], a[q]);
      a[q] = fmaf(ub1(m), v[(w * 4 + q) * 4 + 1], a[q]);
      a[q] = fmaf(ub2(m), v[(w * 4 + q) * 4 + 2], a[q]);
      a[q] = fmaf(ub3(m), v[(w * 4 + q) * 4 + 3], a[q]);
    }
  // field q was read as 4^q * c
  return fmaf(a[3], 0.015625f, fmaf(a[2], 0.0625f, fmaf(a[1], 0.25f, a[0])));
}

template <int BITS>
__device__ __forceinline__ void load_group(const uint8_t *__restrict__ rec, int ng, int g, Chunk<BITS> &c,
                                           uint32_t &sb) {
  if constexpr (BITS == 4) {
    c.a = *reinterpret_cast<const uint4 *>(rec + 16 * g);
    c.b = *reinterpret_cast<const uint4 *>(rec + 16 * (ng + g));
    sb = *reinterpret_cast<const uint32_t *>(rec + 32 * ng + 4 * g);
  } else {
    c.a = *reinterpret_cast<const uint4 *>(rec + 16 * g);
    sb = *reinterpret_cast<const uint32_t *>(rec + 16 * ng + 4 * g);
  }
}

// scale * sum c x + bias * sum x over the lane's group
template <int BITS>
__device__ __forceinline__ float group_partial(const Chunk<BITS> &c, uint32_t sb, const XSlice &xs) {
  const float d = dot_codes(c, xs.v);
  return fmaf(scale_of(sb), d, bias_of(sb) * xs.sum);
}

// Sum over aligned segments of `width` lanes (width a power of two <= 64); every
// lane of a segment receives the segment's sum, always in the same order.
__device__ __forceinline__ float seg_sum(float v, int width) {
  for (int o = width >> 1; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return (int)(blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6)); }

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

template <int BITS>
constexpr int gbytes() {
  return BITS == 4 ? 36 : 20;
}

// ------------------------------------------------------------------ row work

// Rows [row0, row0 + ITERS*rpi) of a packed matrix times x; y[row] = alpha * dot.
template <int BITS, int ITERS>
__device__ __forceinline__ void matvec_rows(const uint8_t *__restrict__ blob, int rows, int ng,
                                            const float *__restrict__ x, float *__restrict__ y, float alpha,
                                            int row0) {
  const int lane = lane_id();
  const int g = lane & (ng - 1);
  const int sub = lane / ng;
  const int rpi = kWave / ng;
  const size_t rb = (size_t)ng * gbytes<BITS>();
  XSlice xs;
  load_xslice<BITS>(x + kGroup * g, xs);
  Chunk<BITS> c[ITERS];
  uint32_t sb[ITERS];
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int row = min(row0 + i * rpi + sub, rows - 1);
    load_group<BITS>(blob + (size_t)row * rb, ng, g, c[i], sb[i]);
  }
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const float p = seg_sum(group_partial<BITS>(c[i], sb[i], xs), ng);
    const int row = row0 + i * rpi + sub;
    if (g == 0 && row < rows) y[row] = alpha * p;
  }
}

// Row pairs [pair0, pair0 + ITERS*rpi) of an interleaved gate/up region:
// h[r] = silu(gate_r . x) * (up_r . x).
template <int BITS, int ITERS>
__device__ __forceinline__ void gateup_pairs(const uint8_t *__restrict__ gu, int ng,
                                             const float *__restrict__ x, float *__restrict__ h, int pair0) {
  const int lane = lane_id();
  const int g = lane & (ng - 1);
  const int sub = lane / ng;
  const int rpi = kWave / ng;
  const size_t rb = (size_t)ng * gbytes<BITS>();
  XSlice xs;
  load_xslice<BITS>(x + kGroup * g, xs);
  Chunk<BITS> cg[ITERS], cu[ITERS];
  uint32_t sg[ITERS], su[ITERS];
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const int r = pair0 + i * rpi + sub;
    const uint8_t *rec = gu + (size_t)(2 * r) * rb;
    load_group<BITS>(rec, ng, g, cg[i], sg[i]);
    load_group<BITS>(rec + rb, ng, g, cu[i], su[i]);
  }
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const float pg = seg_sum(group_partial<BITS>(cg[i], sg[i], xs), ng);
    const float pu = seg_sum(group_partial<BITS>(cu[i], su[i], xs), ng);
    if (g == 0) h[pair0 + i * rpi + sub] = silu(pg) * pu;
  }
}

// One fp32 router row per call: lane l covers columns 4l + 256t + (0..3).
__device__ __forceinline__ float router_row_dot(const float *__restrict__ row, const float4 *xr, int nt) {
  const int lane = lane_id();
  float4 w[16];
#pragma unroll
  for (int t = 0; t < 16; ++t)
    if (t < nt) w[t] = reinterpret_cast<const float4 *>(row)[lane + 64 * t];
  float acc = 0.f;
#pragma unroll
  for (int t = 0; t < 16; ++t)
    if (t < nt) {
      acc = fmaf(w[t].x, xr[t].x, acc);
      acc = fmaf(w[t].y, xr[t].y, acc);
      acc = fmaf(w[t].z, xr[t].z, acc);
      acc = fmaf(w[t].w, xr[t].w, acc);
    }
  return seg_sum(acc, kWave);
}

// Top-K of E logits, computed redundantly by a whole wavefront (no barrier):
// K rounds of "largest remaining value, lower index on a tie". Also returns the
// renormalised softmax weights of the chosen K: w_j = exp(l_j - l_0) / sum.
// NaN logits are treated as -inf.
template <int MAXK>
__device__ __forceinline__ void wave_topk(const float *__restrict__ logits, int E, int K, int *idx, float *w) {
  const int lane = lane_id();
  float v[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) {
    const int e = lane + 64 * m;
    float t = -INFINITY;
    if (e < E) {
      t = logits[e];
      if (t != t) t = -INFINITY;
    }
    v[m] = t;
  }
  uint32_t taken = 0;
  float lv[MAXK];
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    if (j >= K) break;
    float bv = -INFINITY;
    int bi = 0x7FFFFFFF;
#pragma unroll
    for (int m = 0; m < 16; ++m) {
      const int e = lane + 64 * m;
      if (e < E && !(taken & (1u << m)) && (v[m] > bv || (v[m] == bv && e < bi))) {
        bv = v[m];
        bi = e;
      }
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      const float ov = __shfl_xor(bv, o);
      const int oi = __shfl_xor(bi, o);
      if (ov > bv || (ov == bv && oi < bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
    idx[j] = bi;
    lv[j] = bv;
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    if (j >= K) break;
    w[j] = expf(lv[j] - lv[0]);
    sum += w[j];
  }
#pragma unroll
  for (int j = 0; j < MAXK; ++j) {
    if (j >= K) break;
    w[j] = w[j] / sum;
  }
}

// ------------------------------------------------------------------ kernels

template <int BITS, int ITERS>
__global__ __launch_bounds__(kBlock) void k_qmatvec(const uint8_t *__restrict__ blob, int rows, int ng,
                                                     const float *__restrict__ x, float *__restrict__ y) {
  const int rpi = kWave / ng;
  const int row0 = wave_id() * ITERS * rpi;
  if (row0 >= rows) return;
  matvec_rows<BITS, ITERS>(blob, rows, ng, x, y, 1.f, row0);
}

template <int BITS, int ITERS>
__global__ __launch_bounds__(kBlock) void k_expert_gateup(const uint8_t *__restrict__ gu, int inter, int ng,
                                                           const float *__restrict__ x, float *__restrict__ h) {
  const int rpi = kWave / ng;
  const int pair0 = wave_id() * ITERS * rpi;
  if (pair0 >= inter) return;
  gateup_pairs<BITS, ITERS>(gu, ng, x, h, pair0);
}

constexpr int kP1GateUpIters = 2;   // gate/up pairs per iteration-group in phase 1
constexpr int kP2GateUpIters = 2;   // routed gate/up
constexpr int kP2DownIters = 4;     // shared down rows
constexpr int kP3Iters = 4;         // down + combine

struct Phase1Args {
  const float *router;
  const float *gvec;  // null: no shared expert
  int E, H, nt;       // nt = H / 256
  const float *x;
  float *logits;
  float *sigma;
  const uint8_t *shared_gu;  // null: no shared expert
  int I, ngh;
  float *h_shared;
  int n_router_waves;
};

// Phase 1: router logits (one row per wave), sigmoid(g . x) (one more wave) and
// the shared expert's gate/up + SwiGLU (independent of routing).
template <int BITS>
__global__ __launch_bounds__(kBlock) void k_phase1(const Phase1Args a) {
  const int wv = wave_id();
  if (wv < a.n_router_waves) {
    float4 xr[16];
#pragma unroll
    for (int t = 0; t < 16; ++t)
      if (t < a.nt) xr[t] = reinterpret_cast<const float4 *>(a.x)[lane_id() + 64 * t];
    const bool is_gate = wv == a.E;
    const float *row = is_gate ? a.gvec : a.router + (size_t)wv * a.H;
    const float d = router_row_dot(row, xr, a.nt);
    if (lane_id() == 0) {
      if (is_gate)
        *a.sigma = 1.f / (1.f + expf(-d));
      else
        a.logits[wv] = d;
    }
    return;
  }
  if (!a.shared_gu) return;
  const int w2 = wv - a.n_router_waves;
  const int pair0 = w2 * kP1GateUpIters * (kWave / a.ngh);
  if (pair0 >= a.I) return;
  gateup_pairs<BITS, kP1GateUpIters>(a.shared_gu, a.ngh, a.x, a.h_shared, pair0);
}

struct Phase2Args {
  const float *logits;
  int E, K;
  const uint8_t *bank;
  size_t stride;
  const float *x;
  int I, ngh;
  float *h_routed;
  int32_t *ws_idx;
  float *ws_w;
  int32_t *out_idx;
  float *out_w;
  int waves_per_slot;
  int n_routed_waves;
  // shared expert's down projection (null: none)
  const uint8_t *shared_down;
  int H, ngi;
  const float *h_shared;
  const float *sigma;
  float *d_shared;
};

// Phase 2: every routed wave re-derives the top-K from the logits, then runs
// gate/up + SwiGLU of its slot's expert; the remaining waves run the shared
// expert's down projection (scaled by its sigmoid gate).
template <int BITS>
__global__ __launch_bounds__(kBlock) void k_phase2(const Phase2Args a) {
  const int wv = wave_id();
  if (wv < a.n_routed_waves) {
    int idx[kMaxTopK] = {0, 0, 0, 0, 0, 0, 0, 0};
    float w[kMaxTopK] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    wave_topk<kMaxTopK>(a.logits, a.E, a.K, idx, w);
    if (wv == 0 && lane_id() < a.K) {
      const int j = lane_id();
      int sel = idx[0];
      float ws = w[0];
#pragma unroll
      for (int t = 1; t < kMaxTopK; ++t)
        if (t == j) {
          sel = idx[t];
          ws = w[t];
        }
      a.ws_idx[j] = sel;
      a.ws_w[j] = ws;
      if (a.out_idx) a.out_idx[j] = sel;
      if (a.out_w) a.out_w[j] = ws;
    }
    const int slot = wv / a.waves_per_slot;
    const int pair0 = (wv % a.waves_per_slot) * kP2GateUpIters * (kWave / a.ngh);
    int e = idx[0];
#pragma unroll
    for (int t = 1; t < kMaxTopK; ++t)
      if (t == slot) e = idx[t];
    const uint8_t *gu = a.bank + (size_t)e * a.stride;
    gateup_pairs<BITS, kP2GateUpIters>(gu, a.ngh, a.x, a.h_routed + (size_t)slot * a.I, pair0);
    return;
  }
  if (!a.shared_down) return;
  const int w2 = wv - a.n_routed_waves;
  const int row0 = w2 * kP2DownIters * (kWave / a.ngi);
  if (row0 >= a.H) return;
  matvec_rows<BITS, kP2DownIters>(a.shared_down, a.H, a.ngi, a.h_shared, a.d_shared, *a.sigma, row0);
}

struct Phase3Args {
  const uint8_t *bank;
  size_t stride, gu_bytes;
  const int32_t *idx;
  const float *w;
  int K, kpad;
  const float *h_routed;  // [K][I]
  int I, ngi, H;
  const float *d_shared;  // [H] or null
  const float *residual;
  float *out;
};

// Phase 3: out_i = residual_i + sum_k w_k (down_k . h_k)_i + d_shared_i.
// Lanes are (slot k, group j) pairs, so one cross-lane sum adds the K experts'
// weighted partials of a row together; each lane keeps its slot's h slice.
template <int BITS, int SPL>
__global__ __launch_bounds__(kBlock) void k_phase3(const Phase3Args a) {
  const int lane = lane_id();
  const int slots = a.kpad * a.ngi;               // power of two
  const int seg = slots < kWave ? slots : kWave;  // lanes per row
  const int rpi = kWave / seg;
  const int sub = lane / seg;
  const int row0 = wave_id() * kP3Iters * rpi;
  if (row0 >= a.H) return;
  const size_t rb = (size_t)a.ngi * gbytes<BITS>();
  XSlice xs[SPL];
  const uint8_t *base[SPL];
  float wk[SPL];
  int grp[SPL];
  bool act[SPL];
#pragma unroll
  for (int m = 0; m < SPL; ++m) {
    const int slot = (lane % seg) + kWave * m;
    const int k = slot / a.ngi;
    grp[m] = slot % a.ngi;
    act[m] = k < a.K;
    const int kk = act[m] ? k : 0;
    base[m] = a.bank + (size_t)a.idx[kk] * a.stride + a.gu_bytes;
    wk[m] = act[m] ? a.w[kk] : 0.f;
    load_xslice<BITS>(a.h_routed + (size_t)kk * a.I + kGroup * grp[m], xs[m]);
  }
  Chunk<BITS> c[kP3Iters][SPL];
  uint32_t sb[kP3Iters][SPL];
#pragma unroll
  for (int i = 0; i < kP3Iters; ++i) {
    const int row = min(row0 + i * rpi + sub, a.H - 1);
#pragma unroll
    for (int m = 0; m < SPL; ++m)
      if (act[m]) load_group<BITS>(base[m] + (size_t)row * rb, a.ngi, grp[m], c[i][m], sb[i][m]);
  }
#pragma unroll
  for (int i = 0; i < kP3Iters; ++i) {
    float p = 0.f;
#pragma unroll
    for (int m = 0; m < SPL; ++m)
      if (act[m]) p = fmaf(wk[m], group_partial<BITS>(c[i][m], sb[i][m], xs[m]), p);
    p = seg_sum(p, seg);
    const int row = row0 + i * rpi + sub;
    if ((lane % seg) == 0 && row < a.H) {
      float o = a.residual[row] + p;
      if (a.d_shared) o += a.d_shared[row];
      a.out[row] = o;
    }
  }
}

// Two-stage RMS scaling, one block per token.
__global__ __launch_bounds__(kBlock) void k_rms(const float *__restrict__ h, float *__restrict__ x, int H,
                                                 float eps) {
  __shared__ float part[kBlock / kWave];
  const float *ht = h + (size_t)blockIdx.x * H;
  float *xt = x + (size_t)blockIdx.x * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += kBlock) ss = fmaf(ht[i], ht[i], ss);
  ss = seg_sum(ss, kWave);
  if (lane_id() == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kBlock / kWave; ++i) tot += part[i];
  const float r = sqrtf(tot / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += kBlock) xt[i] = ht[i] / r;
}

// Device packer: one thread per (row, group).
template <int BITS>
__global__ __launch_bounds__(kBlock) void k_pack(int rows, int ng, const uint8_t *__restrict__ codes,
                                                  const uint16_t *__restrict__ scale,
                                                  const uint16_t *__restrict__ bias, uint8_t *__restrict__ blob,
                                                  size_t rec_stride, size_t rec_offset) {
  const size_t t = (size_t)blockIdx.x * kBlock + threadIdx.x;
  if (t >= (size_t)rows * ng) return;
  const int r = (int)(t / ng), g = (int)(t % ng);
  const uint8_t *cg = codes + (size_t)r * ng * kGroup + (size_t)g * kGroup;
  uint8_t *rec = blob + rec_offset + (size_t)r * rec_stride;
  uint32_t cw[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t v = reinterpret_cast<const uint32_t *>(cg)[i];
    cw[i] = v;
  }
  auto code = [&](int c) -> uint32_t { return (cw[c >> 2] >> (8 * (c & 3))) & ((1u << BITS) - 1u); };
  if constexpr (BITS == 4) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t o[4];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t word = 0;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int c = 32 * h + 8 * w + k;
          word |= (code(c) | (code(c + 4) << 4)) << (8 * k);
        }
        o[w] = word;
      }
      *reinterpret_cast<uint4 *>(rec + (size_t)h * ng * 16 + (size_t)g * 16) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  } else {
    uint32_t o[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        uint32_t byte = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) byte |= code(16 * w + 4 * q + k) << (2 * q);
        word |= byte << (8 * k);
      }
      o[w] = word;
    }
    *reinterpret_cast<uint4 *>(rec + (size_t)g * 16) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  const size_t sbi = (size_t)r * ng + g;
  *reinterpret_cast<uint32_t *>(rec + (size_t)ng * (BITS == 4 ? 32 : 16) + 4 * g) =
      ((uint32_t)scale[sbi] << 16) | bias[sbi];
}

inline int blocks_for_waves(long waves) { return (int)((waves + (kBlock / kWave) - 1) / (kBlock / kWave)); }

template <int BITS>
hipError_t qmatvec_impl(const uint8_t *blob, int rows, int cols, const float *x, float *y, hipStream_t s) {
  const int ng = cols / kGroup;
  const int rpi = kWave / ng;
  const long iters = (rows + rpi - 1) / rpi;
  // Prefer enough wavefronts to cover every SIMD several times over; more rows
  // per wavefront only once there is work to spare.
  if (iters >= 4L * 4096) {
    hipLaunchKernelGGL((k_qmatvec<BITS, 4>), dim3(blocks_for_waves((iters + 3) / 4)), dim3(kBlock), 0, s, blob,
                       rows, ng, x, y);
  } else if (iters >= 2L * 2048) {
    hipLaunchKernelGGL((k_qmatvec<BITS, 2>), dim3(blocks_for_waves((iters + 1) / 2)), dim3(kBlock), 0, s, blob,
                       rows, ng, x, y);
  } else {
    hipLaunchKernelGGL((k_qmatvec<BITS, 1>), dim3(blocks_for_waves(iters)), dim3(kBlock), 0, s, blob, rows, ng,
                       x, y);
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t layer_impl(const LayerArgs &L, hipStream_t s) {
  const int ngh = L.H / kGroup, ngi = L.I / kGroup;
  const bool has_shared = L.shared != nullptr;
  // ---- phase 1
  Phase1Args p1{};
  p1.router = L.router;
  p1.gvec = has_shared ? L.shared_gate : nullptr;
  p1.E = L.E;
  p1.H = L.H;
  p1.nt = L.H / 256;
  p1.x = L.x;
  p1.logits = L.logits;
  p1.sigma = L.sigma;
  p1.shared_gu = has_shared ? L.shared : nullptr;
  p1.I = L.I;
  p1.ngh = ngh;
  p1.h_shared = L.h_shared;
  p1.n_router_waves = L.E + (has_shared ? 1 : 0);
  const int rpi_h = kWave / ngh;
  const long w1 = p1.n_router_waves + (has_shared ? (L.I / rpi_h + kP1GateUpIters - 1) / kP1GateUpIters : 0);
  hipLaunchKernelGGL((k_phase1<BITS>), dim3(blocks_for_waves(w1)), dim3(kBlock), 0, s, p1);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  // ---- phase 2
  Phase2Args p2{};
  p2.logits = L.logits;
  p2.E = L.E;
  p2.K = L.K;
  p2.bank = L.bank;
  p2.stride = L.expert_stride;
  p2.x = L.x;
  p2.I = L.I;
  p2.ngh = ngh;
  p2.h_routed = L.h_routed;
  p2.ws_idx = L.ws_idx;
  p2.ws_w = L.ws_w;
  p2.out_idx = L.topk_idx_out;
  p2.out_w = L.topk_w_out;
  p2.waves_per_slot = (L.I / rpi_h + kP2GateUpIters - 1) / kP2GateUpIters;
  p2.n_routed_waves = p2.waves_per_slot * L.K;
  p2.shared_down = has_shared ? L.shared + L.gateup_bytes : nullptr;
  p2.H = L.H;
  p2.ngi = ngi;
  p2.h_shared = L.h_shared;
  p2.sigma = L.sigma;
  p2.d_shared = L.d_shared;
  const int rpi_i = kWave / ngi;
  const long w2 = p2.n_routed_waves +
                  (has_shared ? (L.H / rpi_i + kP2DownIters - 1) / kP2DownIters : 0);
  hipLaunchKernelGGL((k_phase2<BITS>), dim3(blocks_for_waves(w2)), dim3(kBlock), 0, s, p2);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  // ---- phase 3
  Phase3Args p3{};
  p3.bank = L.bank;
  p3.stride = L.expert_stride;
  p3.gu_bytes = L.gateup_bytes;
  p3.idx = L.ws_idx;
  p3.w = L.ws_w;
  p3.K = L.K;
  int kpad = 1;
  while (kpad < L.K) kpad <<= 1;
  p3.kpad = kpad;
  p3.h_routed = L.h_routed;
  p3.I = L.I;
  p3.ngi = ngi;
  p3.H = L.H;
  p3.d_shared = has_shared ? L.d_shared : nullptr;
  p3.residual = L.residual;
  p3.out = L.out;
  const int slots = kpad * ngi;
  const int seg = slots < kWave ? slots : kWave;
  const int spl = slots / seg;
  const long w3 = ((long)L.H / (kWave / seg) + kP3Iters - 1) / kP3Iters;
  const dim3 g3(blocks_for_waves(w3));
  switch (spl) {
    case 1: hipLaunchKernelGGL((k_phase3<BITS, 1>), g3, dim3(kBlock), 0, s, p3); break;
    case 2: hipLaunchKernelGGL((k_phase3<BITS, 2>), g3, dim3(kBlock), 0, s, p3); break;
    case 4: hipLaunchKernelGGL((k_phase3<BITS, 4>), g3, dim3(kBlock), 0, s, p3); break;
    default: hipLaunchKernelGGL((k_phase3<BITS, 8>), g3, dim3(kBlock), 0, s, p3); break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qmatvec(int bits, const uint8_t *blob, int rows, int cols, const float *x, float *y,
                          hipStream_t s) {
  return bits == 4 ? qmatvec_impl<4>(blob, rows, cols, x, y, s) : qmatvec_impl<2>(blob, rows, cols, x, y, s);
}

hipError_t launch_expert_gateup(int bits, const uint8_t *gu, int hidden, int inter, const float *x, float *h,
                                hipStream_t s) {
  const int ng = hidden / kGroup;
  const int rpi = kWave / ng;
  const long waves = (inter / rpi + 1) / 2;
  if (bits == 4)
    hipLaunchKernelGGL((k_expert_gateup<4, 2>), dim3(blocks_for_waves(waves)), dim3(kBlock), 0, s, gu, inter, ng,
                       x, h);
  else
    hipLaunchKernelGGL((k_expert_gateup<2, 2>), dim3(blocks_for_waves(waves)), dim3(kBlock), 0, s, gu, inter, ng,
                       x, h);
  return hipGetLastError();
}

hipError_t launch_layer(const LayerArgs &a, hipStream_t s) {
  return a.bits == 4 ? layer_impl<4>(a, s) : layer_impl<2>(a, s);
}

hipError_t launch_rms(const float *h, float *x, int B, int H, float eps, hipStream_t s) {
  hipLaunchKernelGGL(k_rms, dim3(B), dim3(kBlock), 0, s, h, x, H, eps);
  return hipGetLastError();
}

hipError_t launch_pack_matrix(int bits, int rows, int cols, const uint8_t *codes, const uint16_t *scale,
                              const uint16_t *bias, uint8_t *blob, size_t rec_stride, size_t rec_offset,
                              hipStream_t s) {
  const int ng = cols / kGroup;
  const size_t n = (size_t)rows * ng;
  const dim3 grid((unsigned)((n + kBlock - 1) / kBlock));
  if (bits == 4)
    hipLaunchKernelGGL(k_pack<4>, grid, dim3(kBlock), 0, s, rows, ng, codes, scale, bias, blob, rec_stride,
                       rec_offset);
  else
    hipLaunchKernelGGL(k_pack<2>, grid, dim3(kBlock), 0, s, rows, ng, codes, scale, bias, blob, rec_stride,
                       rec_offset);
  return hipGetLastError();
}

}  // namespace fmoe
