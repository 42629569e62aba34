// kernels_forms.hip -- the standalone dequantized matvec y = W x in four forms of
// the per-weight arithmetic, to compare them on this GPU. Pages cited:
//   [P1] "397B MoE en MacBook: Motor Flash-MoE a 4,4 t/s" (aibit.im)
//   [P2] "Flash-MoE: Ausfuehren eines 397B-Parameter-Qwen-Modells auf dem MacBook
//        Pro mit reinem C/Metal" (openclawradar.com)
// With c_j the code of column j of a 64-column group, s and b the group's scale
// and bias:
//   0 naive:     w_j = c_j s + b, then acc += w_j x_j (two fused multiply-adds);
//   1 recast:    acc += fma(c_j, s x_j, b x_j), the per-weight form of
//                [P1] "2. Kernel de desquantización optimizado con FMA" and
//                [P2] "FMA-optimierter Dequant-Kernel" (s x_j and b x_j formed per weight);
//   2 factored:  s * sum_j c_j x_j + b * sum_j x_j, the form every other kernel of
//                the library uses (one multiply-add per weight);
//   3 table:     w_j = T[c_j] from a per-(row, group) table T[c] = c s + b that each
//                lane writes to its own LDS row, then acc += w_j x_j: the GPU dequant
//                lookup table that [P1] "Lo que descartaron" lists as slower.
// One row per 64 / NGP lanes (NGP: the groups per row rounded up to a power of
// two), a lane per group, and 1, 2 or 4 row iterations per
// wavefront chosen by the matrix height, as in the library's matvec (form 2 is
// that kernel); x staged once per workgroup. The expert's fused gate/up + SwiGLU
// kernel comes in the same four forms, so that a whole expert (gate/up, then the
// down projection as a matvec) can run in each.
#include "forms.h"
#include "kernels.h"
#include "layer_kernels.h"

namespace fmoe {
namespace dev {
namespace {

template <int BITS, int NGP, int ITERS, int FORM>
__global__ __launch_bounds__(kBlock) void k_qmatvec_form(const uint8_t *__restrict__ blob, int ng, int rows,
                                                          const float *__restrict__ x, float *__restrict__ y) {
  constexpr int RPI = kWave / NGP;
  __shared__ float xl[NGP * kXPad];
  __shared__ float lut[FORM == 3 ? kBlock * kLutStride : 1];
  constexpr int X4 = (NGP * 16 + kBlock - 1) / kBlock;
  const int lane = lane_id();
  const int row0 = wave_id() * ITERS * RPI;
  Staged<X4> xst;
  stage_load(x, ng * 16, xst);
  RowLoads<BITS, NGP, ITERS> L;
  if (row0 < rows) L.issue(blob, ng, rows, row0);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<X4, false>(xst, ng * 16, xl, nullptr);
  __syncthreads();
  if (row0 >= rows) return;
  XSlice xs;
  read_slice(xl, min(lane & (NGP - 1), ng - 1), 1.f, xs);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const float p = seg_reduce<NGP>(
        L.live ? partial_form<BITS, FORM>(L.c[i], L.sb[i], xs, FORM == 3 ? lut + threadIdx.x * kLutStride : lut)
               : 0.f);
    const int row = row0 + i * RPI + lane / NGP;
    if (seg_last<NGP>(lane) && row < rows) y[row] = p;
  }
}

// The expert's fused gate/up + SwiGLU (h[r] = silu(gate_r . x) * (up_r . x)) with the
// per-weight arithmetic in form FORM: the library's gate/up kernel for one expert with
// its partial sums replaced (form 2 is that kernel's arithmetic).
template <int BITS, int NGP, int FORM>
__global__ __launch_bounds__(kBlock) void k_expert_gateup_form(const uint8_t *__restrict__ gu, int ng, int inter,
                                                                const float *__restrict__ x, float *__restrict__ h) {
  constexpr int RPI = kWave / NGP;
  __shared__ float xl[NGP * kXPad];
  __shared__ float lut[FORM == 3 ? kBlock * kLutStride : 1];
  constexpr int X4 = (NGP * 16 + kBlock - 1) / kBlock;
  const int lane = lane_id();
  const int pair0 = wave_id() * RPI;
  Staged<X4> xst;
  stage_load(x, ng * 16, xst);
  PairLoads<BITS, NGP, 1> P;
  if (pair0 < inter) P.issue(gu, ng, pair0);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<X4, false>(xst, ng * 16, xl, nullptr);
  __syncthreads();
  if (pair0 >= inter) return;
  XSlice xs;
  read_slice(xl, min(lane & (NGP - 1), ng - 1), 1.f, xs);
  float *tab = FORM == 3 ? lut + threadIdx.x * kLutStride : lut;
  const float pg = seg_reduce<NGP>(P.live ? partial_form<BITS, FORM>(P.cg[0], P.sg[0], xs, tab) : 0.f);
  const float pu = seg_reduce<NGP>(P.live ? partial_form<BITS, FORM>(P.cu[0], P.su[0], xs, tab) : 0.f);
  if (seg_last<NGP>(lane)) h[pair0 + lane / NGP] = silu(pg) * pu;
}

template <int BITS, int NGP>
hipError_t launch_gateup(int form, const uint8_t *gu, int ng, int inter, const float *x, float *h, hipStream_t s) {
  const dim3 grid(blocks_for(inter / (kWave / NGP))), block(kBlock);
  switch (form) {
    case 0: hipLaunchKernelGGL((k_expert_gateup_form<BITS, NGP, 0>), grid, block, 0, s, gu, ng, inter, x, h); break;
    case 1: hipLaunchKernelGGL((k_expert_gateup_form<BITS, NGP, 1>), grid, block, 0, s, gu, ng, inter, x, h); break;
    case 2: hipLaunchKernelGGL((k_expert_gateup_form<BITS, NGP, 2>), grid, block, 0, s, gu, ng, inter, x, h); break;
    default: hipLaunchKernelGGL((k_expert_gateup_form<BITS, NGP, 3>), grid, block, 0, s, gu, ng, inter, x, h); break;
  }
  return hipGetLastError();
}

template <int BITS>
hipError_t launch_gateup_bits(int form, const uint8_t *gu, int hidden, int inter, const float *x, float *h,
                              hipStream_t s) {
  const int ng = hidden / kGroup;
  switch (pad_groups(ng)) {
    case 4: return launch_gateup<BITS, 4>(form, gu, ng, inter, x, h, s);
    case 8: return launch_gateup<BITS, 8>(form, gu, ng, inter, x, h, s);
    case 16: return launch_gateup<BITS, 16>(form, gu, ng, inter, x, h, s);
    case 32: return launch_gateup<BITS, 32>(form, gu, ng, inter, x, h, s);
    case 64: return launch_gateup<BITS, 64>(form, gu, ng, inter, x, h, s);
    default: return hipErrorInvalidValue;
  }
}

template <int BITS, int NGP, int ITERS>
hipError_t launch_it(int form, const uint8_t *blob, int ng, int rows, const float *x, float *y, hipStream_t s) {
  const long iters = (rows + kWave / NGP - 1) / (kWave / NGP);
  const dim3 grid(blocks_for((iters + ITERS - 1) / ITERS));
  const dim3 block(kBlock);
  switch (form) {
    case 0: hipLaunchKernelGGL((k_qmatvec_form<BITS, NGP, ITERS, 0>), grid, block, 0, s, blob, ng, rows, x, y); break;
    case 1: hipLaunchKernelGGL((k_qmatvec_form<BITS, NGP, ITERS, 1>), grid, block, 0, s, blob, ng, rows, x, y); break;
    case 2: hipLaunchKernelGGL((k_qmatvec_form<BITS, NGP, ITERS, 2>), grid, block, 0, s, blob, ng, rows, x, y); break;
    default: hipLaunchKernelGGL((k_qmatvec_form<BITS, NGP, ITERS, 3>), grid, block, 0, s, blob, ng, rows, x, y); break;
  }
  return hipGetLastError();
}

// row iterations per wavefront as the library's matvec chooses them
template <int BITS, int NGP>
hipError_t launch_ng(int form, const uint8_t *blob, int ng, int rows, const float *x, float *y, hipStream_t s) {
  const long iters = (rows + kWave / NGP - 1) / (kWave / NGP);
  if (iters >= 4L * 4096) return launch_it<BITS, NGP, 4>(form, blob, ng, rows, x, y, s);
  if (iters >= 2L * 2048) return launch_it<BITS, NGP, 2>(form, blob, ng, rows, x, y, s);
  return launch_it<BITS, NGP, 1>(form, blob, ng, rows, x, y, s);
}

template <int BITS>
hipError_t launch_bits(int form, const uint8_t *blob, int rows, int cols, const float *x, float *y, hipStream_t s) {
  const int ng = cols / kGroup;
  switch (pad_groups(ng)) {
    case 4: return launch_ng<BITS, 4>(form, blob, ng, rows, x, y, s);
    case 8: return launch_ng<BITS, 8>(form, blob, ng, rows, x, y, s);
    case 16: return launch_ng<BITS, 16>(form, blob, ng, rows, x, y, s);
    case 32: return launch_ng<BITS, 32>(form, blob, ng, rows, x, y, s);
    case 64: return launch_ng<BITS, 64>(form, blob, ng, rows, x, y, s);
    default: return hipErrorInvalidValue;
  }
}

// The one-token layer at hidden 4096, inter 1024, top-4 with the gate/up and down
// arithmetic in form FORM (the router kernel as in the library, writing x in fp32 too).
template <int BITS, int FORM>
hipError_t layer_form_it(const LayerArgs &L, hipStream_t s) {
  using D = Dispatch<BITS>;
  const LayerGeom<BITS, 64, 16> G(L, BITS);
  hipError_t e = D::template phase1<64, 16>(L, G, s);
  if (e == hipSuccess) e = D::template phase2<64, 16, FORM>(L, G, s);
  if (e == hipSuccess) e = D::template phase3<64, 16, 4, FORM>(L, G, s);
  return e;
}

template <int BITS>
hipError_t layer_form_bits(const LayerArgs &L, int form, hipStream_t s) {
  switch (form) {
    case 0: return layer_form_it<BITS, 0>(L, s);
    case 1: return layer_form_it<BITS, 1>(L, s);
    case 2: return layer_form_it<BITS, 2>(L, s);
    default: return layer_form_it<BITS, 3>(L, s);
  }
}

}  // namespace
}  // namespace dev

hipError_t launch_layer_form(const LayerArgs &a, int form, hipStream_t s) {
  if (a.H != 4096 || a.I != 1024 || a.K != 4 || a.E > 512 || !a.xs || form < 0 || form >= kForms)
    return hipErrorInvalidValue;
  return a.bits == 4 ? dev::layer_form_bits<4>(a, form, s) : dev::layer_form_bits<2>(a, form, s);
}

hipError_t launch_qmatvec_form(int bits, int form, const uint8_t *blob, int rows, int cols, const float *x, float *y,
                               hipStream_t s) {
  return bits == 4 ? dev::launch_bits<4>(form, blob, rows, cols, x, y, s)
                   : dev::launch_bits<2>(form, blob, rows, cols, x, y, s);
}

hipError_t launch_expert_gateup_form(int bits, int form, const uint8_t *gu, int hidden, int inter, const float *x,
                                     float *h, hipStream_t s) {
  return bits == 4 ? dev::launch_gateup_bits<4>(form, gu, hidden, inter, x, h, s)
                   : dev::launch_gateup_bits<2>(form, gu, hidden, inter, x, h, s);
}

}  // namespace fmoe
