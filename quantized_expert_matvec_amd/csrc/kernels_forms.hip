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
// One row per 64 / NG lanes, a lane per group, and 1, 2 or 4 row iterations per
// wavefront chosen by the matrix height, as in the library's matvec (form 2 is
// that kernel); x staged once per workgroup.
#include "forms.h"
#include "layer_kernels.h"

namespace fmoe {
namespace dev {
namespace {

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

template <int BITS, int NG, int ITERS, int FORM>
__global__ __launch_bounds__(kBlock) void k_qmatvec_form(const uint8_t *__restrict__ blob, int rows,
                                                          const float *__restrict__ x, float *__restrict__ y) {
  constexpr int RPI = kWave / NG;
  __shared__ float xl[NG * kXPad];
  __shared__ float lut[FORM == 3 ? kBlock * kLutStride : 1];
  constexpr int X4 = (NG * 16 + kBlock - 1) / kBlock;
  const int lane = lane_id();
  const int row0 = wave_id() * ITERS * RPI;
  Staged<X4> xst;
  stage_load(x, NG * 16, xst);
  RowLoads<BITS, NG, ITERS> L;
  if (row0 < rows) L.issue(blob, rows, row0);
  __builtin_amdgcn_sched_barrier(0);
  stage_store<X4, false>(xst, NG * 16, xl, nullptr);
  __syncthreads();
  if (row0 >= rows) return;
  XSlice xs;
  read_slice(xl, lane & (NG - 1), 1.f, xs);
#pragma unroll
  for (int i = 0; i < ITERS; ++i) {
    const float p = seg_reduce<NG>(
        partial_form<BITS, FORM>(L.c[i], L.sb[i], xs, FORM == 3 ? lut + threadIdx.x * kLutStride : lut));
    const int row = row0 + i * RPI + lane / NG;
    if (seg_last<NG>(lane) && row < rows) y[row] = p;
  }
}

template <int BITS, int NG, int ITERS>
hipError_t launch_it(int form, const uint8_t *blob, int rows, const float *x, float *y, hipStream_t s) {
  const long iters = (rows + kWave / NG - 1) / (kWave / NG);
  const dim3 grid(blocks_for((iters + ITERS - 1) / ITERS));
  const dim3 block(kBlock);
  switch (form) {
    case 0: hipLaunchKernelGGL((k_qmatvec_form<BITS, NG, ITERS, 0>), grid, block, 0, s, blob, rows, x, y); break;
    case 1: hipLaunchKernelGGL((k_qmatvec_form<BITS, NG, ITERS, 1>), grid, block, 0, s, blob, rows, x, y); break;
    case 2: hipLaunchKernelGGL((k_qmatvec_form<BITS, NG, ITERS, 2>), grid, block, 0, s, blob, rows, x, y); break;
    default: hipLaunchKernelGGL((k_qmatvec_form<BITS, NG, ITERS, 3>), grid, block, 0, s, blob, rows, x, y); break;
  }
  return hipGetLastError();
}

// row iterations per wavefront as the library's matvec chooses them
template <int BITS, int NG>
hipError_t launch_ng(int form, const uint8_t *blob, int rows, const float *x, float *y, hipStream_t s) {
  const long iters = (rows + kWave / NG - 1) / (kWave / NG);
  if (iters >= 4L * 4096) return launch_it<BITS, NG, 4>(form, blob, rows, x, y, s);
  if (iters >= 2L * 2048) return launch_it<BITS, NG, 2>(form, blob, rows, x, y, s);
  return launch_it<BITS, NG, 1>(form, blob, rows, x, y, s);
}

template <int BITS>
hipError_t launch_bits(int form, const uint8_t *blob, int rows, int cols, const float *x, float *y, hipStream_t s) {
  switch (cols / kGroup) {
    case 4: return launch_ng<BITS, 4>(form, blob, rows, x, y, s);
    case 8: return launch_ng<BITS, 8>(form, blob, rows, x, y, s);
    case 16: return launch_ng<BITS, 16>(form, blob, rows, x, y, s);
    case 32: return launch_ng<BITS, 32>(form, blob, rows, x, y, s);
    case 64: return launch_ng<BITS, 64>(form, blob, rows, x, y, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace
}  // namespace dev

hipError_t launch_qmatvec_form(int bits, int form, const uint8_t *blob, int rows, int cols, const float *x, float *y,
                               hipStream_t s) {
  return bits == 4 ? dev::launch_bits<4>(form, blob, rows, cols, x, y, s)
                   : dev::launch_bits<2>(form, blob, rows, cols, x, y, s);
}

}  // namespace fmoe
