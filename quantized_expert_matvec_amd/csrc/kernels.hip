// kernels.hip -- the small kernels (RMS scaling, device packer) and the
// launchers that dispatch on the bit width to kernels_q4.hip / kernels_q2.hip.
#include <hip/hip_runtime.h>

#include "device.h"
#include "kernels.h"
#include "layout.h"

namespace fmoe {
namespace dev {
template <int BITS>
hipError_t qmatvec_b(const uint8_t *, int, int, const float *, float *, hipStream_t);
template <int BITS>
hipError_t gateup_b(const uint8_t *, int, int, const float *, float *, hipStream_t);
template <int BITS>
hipError_t layer_b(const LayerArgs &, hipStream_t, int);
extern template hipError_t qmatvec_b<4>(const uint8_t *, int, int, const float *, float *, hipStream_t);
extern template hipError_t qmatvec_b<2>(const uint8_t *, int, int, const float *, float *, hipStream_t);
extern template hipError_t gateup_b<4>(const uint8_t *, int, int, const float *, float *, hipStream_t);
extern template hipError_t gateup_b<2>(const uint8_t *, int, int, const float *, float *, hipStream_t);
extern template hipError_t layer_b<4>(const LayerArgs &, hipStream_t, int);
extern template hipError_t layer_b<2>(const LayerArgs &, hipStream_t, int);
template <int BITS>
hipError_t layer_ptr_b(const LayerArgs &, hipStream_t, int);
extern template hipError_t layer_ptr_b<4>(const LayerArgs &, hipStream_t, int);
extern template hipError_t layer_ptr_b<2>(const LayerArgs &, hipStream_t, int);
template <int BITS>
hipError_t route1_b(const float *, int, int, int32_t *, float *, hipStream_t);
extern template hipError_t route1_b<4>(const float *, int, int, int32_t *, float *, hipStream_t);
template <int BITS>
hipError_t group_b(const GroupArgs &, hipStream_t, int);
extern template hipError_t group_b<4>(const GroupArgs &, hipStream_t, int);
extern template hipError_t group_b<2>(const GroupArgs &, hipStream_t, int);
template <int BITS>
hipError_t group_route_b(const GroupArgs &, hipStream_t);
template <int BITS>
hipError_t group_experts_b(const GroupArgs &, hipStream_t);
extern template hipError_t group_route_b<4>(const GroupArgs &, hipStream_t);
extern template hipError_t group_route_b<2>(const GroupArgs &, hipStream_t);
extern template hipError_t group_experts_b<4>(const GroupArgs &, hipStream_t);
extern template hipError_t group_experts_b<2>(const GroupArgs &, hipStream_t);

namespace {

// Two-stage RMS scaling, one block per token.
__global__ __launch_bounds__(kBlock) void k_rms(const float *__restrict__ h, float *__restrict__ x, int H,
                                                 float eps) {
  __shared__ float part[kBlock / kWave];
  const float *ht = h + (size_t)blockIdx.x * H;
  float *xt = x + (size_t)blockIdx.x * H;
  float ss = 0.f;
  for (int i = threadIdx.x; i < H; i += kBlock) ss = fmaf(ht[i], ht[i], ss);
  ss = seg_reduce<kWave>(ss);
  if (lane_id() == kWave - 1) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kBlock / kWave; ++i) tot += part[i];
  const float r = sqrtf(tot / (float)H + eps);
  for (int i = threadIdx.x; i < H; i += kBlock) xt[i] = ht[i] / r;
}

// Streaming read: the XOR of every 32-bit word of n16 16-byte units, folded into
// *out with one atomic per workgroup. Grid-stride over the units with
// kReadUnroll independent non-temporal loads in flight per thread; an empty
// buffer makes an empty kernel.
constexpr int kReadUnroll = 8;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(kBlock) void k_read_xor(const u32x4 *__restrict__ p, size_t n16,
                                                      uint32_t *__restrict__ out) {
  __shared__ uint32_t part[kBlock / kWave];
  const size_t stride = (size_t)gridDim.x * kBlock;
  size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x;
  uint32_t acc = 0;
  // rounds of kReadUnroll loads, all requested before any is used; in the last round
  // the loads past the end re-read the last unit (not folded in), so that a buffer that
  // takes one round per thread is one burst whatever its size
  for (; i < n16; i += kReadUnroll * stride) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k) {
      const size_t j = i + k * stride;
      v[k] = __builtin_nontemporal_load(p + (j < n16 ? j : n16 - 1));
    }
#pragma unroll
    for (int k = 0; k < kReadUnroll; ++k)
      if (i + k * stride < n16) acc ^= (v[k].x ^ v[k].y) ^ (v[k].z ^ v[k].w);
  }
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) acc ^= (uint32_t)__shfl_xor((int)acc, m);
  if (lane_id() == 0) part[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
#pragma unroll
    for (int w = 0; w < kBlock / kWave; ++w) t ^= part[w];
    if (t) atomicXor(out, t);
  }
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

}  // namespace
}  // namespace dev

hipError_t launch_qmatvec(int bits, const uint8_t *blob, int rows, int cols, const float *x, float *y,
                          hipStream_t s) {
  return bits == 4 ? dev::qmatvec_b<4>(blob, rows, cols, x, y, s) : dev::qmatvec_b<2>(blob, rows, cols, x, y, s);
}

hipError_t launch_expert_gateup(int bits, const uint8_t *gu, int hidden, int inter, const float *x, float *h,
                                hipStream_t s) {
  return bits == 4 ? dev::gateup_b<4>(gu, hidden, inter, x, h, s) : dev::gateup_b<2>(gu, hidden, inter, x, h, s);
}

hipError_t launch_read_xor(const void *buf, size_t bytes, uint32_t *out, hipStream_t s) {
  const size_t n16 = bytes / 16;
  const size_t per = (size_t)kBlock * dev::kReadUnroll;
  const size_t want = (n16 + per - 1) / per;
  const int grid = (int)(want < 1 ? 1 : want > 2048 ? 2048 : want);
  hipLaunchKernelGGL(dev::k_read_xor, dim3(grid), dim3(kBlock), 0, s, reinterpret_cast<const dev::u32x4 *>(buf), n16,
                     out);
  return hipGetLastError();
}

hipError_t launch_layer(const LayerArgs &a, hipStream_t s, int phases) {
  return a.bits == 4 ? dev::layer_b<4>(a, s, phases) : dev::layer_b<2>(a, s, phases);
}

hipError_t launch_layer_ptr(const LayerArgs &a, hipStream_t s, int phases) {
  return a.bits == 4 ? dev::layer_ptr_b<4>(a, s, phases) : dev::layer_ptr_b<2>(a, s, phases);
}

hipError_t launch_route1(const float *logits, int E, int K, int32_t *idx, float *w, hipStream_t s) {
  return dev::route1_b<4>(logits, E, K, idx, w, s);
}

hipError_t launch_group(const GroupArgs &a, hipStream_t s, int phases) {
  return a.bits == 4 ? dev::group_b<4>(a, s, phases) : dev::group_b<2>(a, s, phases);
}

hipError_t launch_group_route(const GroupArgs &a, hipStream_t s) {
  return a.bits == 4 ? dev::group_route_b<4>(a, s) : dev::group_route_b<2>(a, s);
}

hipError_t launch_group_experts(const GroupArgs &a, hipStream_t s) {
  return a.bits == 4 ? dev::group_experts_b<4>(a, s) : dev::group_experts_b<2>(a, s);
}

hipError_t launch_rms(const float *h, float *x, int B, int H, float eps, hipStream_t s) {
  hipLaunchKernelGGL(dev::k_rms, dim3(B), dim3(kBlock), 0, s, h, x, H, eps);
  return hipGetLastError();
}

hipError_t launch_pack_matrix(int bits, int rows, int cols, const uint8_t *codes, const uint16_t *scale,
                              const uint16_t *bias, uint8_t *blob, size_t rec_stride, size_t rec_offset,
                              hipStream_t s) {
  const int ng = cols / kGroup;
  const size_t n = (size_t)rows * ng;
  const dim3 grid((unsigned)((n + kBlock - 1) / kBlock));
  if (bits == 4)
    hipLaunchKernelGGL(dev::k_pack<4>, grid, dim3(kBlock), 0, s, rows, ng, codes, scale, bias, blob, rec_stride,
                       rec_offset);
  else
    hipLaunchKernelGGL(dev::k_pack<2>, grid, dim3(kBlock), 0, s, rows, ng, codes, scale, bias, blob, rec_stride,
                       rec_offset);
  return hipGetLastError();
}

}  // namespace fmoe
