// synth_dev.hip -- device twin of synth.c for bulk fills of large resident
// expert banks. It draws the same splitmix64 words and repeats the same integer
// and fp64 steps as the host generator, so a code or a scale/bias pair drawn
// here equals the host's bit for bit (built with contraction off). It writes
// the canonical layout (one uint8 per code; bf16 bit patterns), never the
// library's packed layout. Normals are drawn on the host only.
#include <hip/hip_runtime.h>
#include <stdint.h>

#pragma clang fp contract(off)

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t word(uint64_t key, uint64_t n) { return mix(key + (n + 1) * kGamma); }

__device__ __forceinline__ uint16_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__global__ void codes_kernel(uint64_t key, int bits, int64_t n, uint8_t* out) {
  const int per = 64 / bits;
  const uint64_t mask = (1u << bits) - 1u;
  const int64_t nw = (n + per - 1) / per;
  for (int64_t w = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; w < nw;
       w += (int64_t)gridDim.x * blockDim.x) {
    uint64_t v = word(key, (uint64_t)w);
    int64_t base = w * per;
    int lim = (n - base) < per ? (int)(n - base) : per;
    if (lim == per && bits == 4) {
      // 16 codes -> four 32-bit stores (base is a multiple of 16 bytes).
      uint32_t o[4];
      for (int q = 0; q < 4; ++q) {
        uint32_t acc = 0;
        for (int i = 0; i < 4; ++i) acc |= (uint32_t)((v >> (4 * (4 * q + i))) & 15u) << (8 * i);
        o[q] = acc;
      }
      *reinterpret_cast<uint4*>(out + base) = make_uint4(o[0], o[1], o[2], o[3]);
    } else if (lim == per && bits == 2) {
      uint32_t o[8];
      for (int q = 0; q < 8; ++q) {
        uint32_t acc = 0;
        for (int i = 0; i < 4; ++i) acc |= (uint32_t)((v >> (2 * (4 * q + i))) & 3u) << (8 * i);
        o[q] = acc;
      }
      *reinterpret_cast<uint4*>(out + base) = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(out + base + 16) = make_uint4(o[4], o[5], o[6], o[7]);
    } else {
      for (int i = 0; i < lim; ++i) out[base + i] = (uint8_t)((v >> (bits * i)) & mask);
    }
  }
}

__global__ void scale_bias_kernel(uint64_t key, int64_t n, double lo, double hi, double bmul,
                                  double spread, uint16_t* scale, uint16_t* bias) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    uint64_t v = word(key, (uint64_t)i);
    double u1 = (double)(v >> 40) * 0x1p-24;
    double u2 = (double)((v >> 16) & 0xFFFFFFu) * 0x1p-24;
    double width = __dsub_rn(hi, lo);
    double s = __dmul_rn(width, u1);
    s = __dadd_rn(lo, s);
    uint16_t sb = bf16_rne(__double2float_rn(s));
    double sd = (double)__uint_as_float((uint32_t)sb << 16);
    double t = __dmul_rn(__dmul_rn(2.0, spread), u2);
    t = __dsub_rn(t, spread);
    t = __dadd_rn(1.0, t);
    double b = __dmul_rn(-bmul, sd);
    b = __dmul_rn(b, t);
    scale[i] = sb;
    bias[i] = bf16_rne(__double2float_rn(b));
  }
}

int grid_for(int64_t items) {
  int64_t g = (items + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace

extern "C" int synd_codes(uint64_t key, int bits, int64_t n, uint8_t* out, void* stream) {
  if (bits != 2 && bits != 4) return -1;
  if ((reinterpret_cast<uintptr_t>(out) & 15u) != 0) return -2;
  const int per = 64 / bits;
  hipLaunchKernelGGL(codes_kernel, dim3(grid_for((n + per - 1) / per)), dim3(256), 0,
                     (hipStream_t)stream, key, bits, n, out);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

extern "C" int synd_scale_bias(uint64_t key, int64_t n, double lo, double hi, double bmul,
                               double spread, uint16_t* scale, uint16_t* bias, void* stream) {
  hipLaunchKernelGGL(scale_bias_kernel, dim3(grid_for(n)), dim3(256), 0, (hipStream_t)stream, key, n,
                     lo, hi, bmul, spread, scale, bias);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}
