// device.h -- device helpers shared by the HIP kernels of libfmoe (gfx950).
//
// Work mapping. Every quantized matrix is processed with one 64-column group per
// lane: lane g of a row segment loads the group's codes with 128-bit loads
// (two for 4-bit, one for 2-bit; consecutive lanes read consecutive 16-byte
// pieces, so each load instruction of a wavefront covers a contiguous span) and
// its (scale, bias) word, and keeps the matching 64 values of the input vector
// in registers for every row it visits. A row of `cols` columns has ng = cols/64
// groups and occupies NGP lanes (ng rounded up to a power of two, pad_groups); a
// wavefront covers 64/NGP rows per iteration, and DPP cross-lane adds over those
// lanes finish each row.
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
// once per group. Everything is fp32 with a fixed reduction order (bitwise
// deterministic). The one-token gate/up takes sum_j c_j x_j on exact integer dot
// products instead (the digit form of x, further below).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "layout.h"

namespace fmoe {
namespace dev {

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

template <int BITS>
constexpr int gbytes() {
  return BITS == 4 ? 36 : 20;
}

// One lane's 64 input values for its group. The packing puts column 64g+i of
// group g at unpack position i (4-bit: word i/8, low nibble of byte i%4 for
// i%8 < 4, else high nibble; 2-bit: word i/16, field (i%16)/4, byte i%4), so the
// slice is simply x[64g .. 64g+63] in order.
struct XSlice {
  float v[64];
  float sum;  // sum of the 64 values (the bias term's factor)
};

// Pairwise sum of 64 values (fixed order, depth 6).
__device__ __forceinline__ float tree_sum64(const float *v) {
  float t[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) t[i] = v[2 * i] + v[2 * i + 1];
#pragma unroll
  for (int w = 16; w > 0; w >>= 1)
#pragma unroll
    for (int i = 0; i < w; ++i) t[i] = t[2 * i] + t[2 * i + 1];
  return t[0];
}

__device__ __forceinline__ void load_xslice(const float *__restrict__ xg, XSlice &s) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 t = reinterpret_cast<const float4 *>(xg)[i];
    s.v[4 * i] = t.x;
    s.v[4 * i + 1] = t.y;
    s.v[4 * i + 2] = t.z;
    s.v[4 * i + 3] = t.w;
  }
  s.sum = tree_sum64(s.v);
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

// Loads of group g (g < ng) from one row record of ng groups.
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

// Row widths. A row of ng groups (ng = cols / 64, any value 4 .. 64: cols a
// multiple of 256 up to 4096) occupies a segment of NGP lanes, NGP the power of
// two at or above ng; lane g < ng holds group g. The lanes past ng load group
// ng - 1 again (the same bytes, no extra traffic) and see an input of zeros (the
// staged vector is zero past ng groups), so they add exactly 0 to the row.
__host__ __device__ constexpr int pad_groups(int ng) { return ng <= 4 ? 4 : ng <= 8 ? 8 : ng <= 16 ? 16 : ng <= 32 ? 32 : 64; }

// scale * sum c x + bias * sum x over the lane's group
template <int BITS>
__device__ __forceinline__ float group_partial(const Chunk<BITS> &c, uint32_t sb, const XSlice &xs) {
  const float d = dot_codes(c, xs.v);
  return fmaf(scale_of(sb), d, bias_of(sb) * xs.sum);
}

// ------------------------------------------------------------------ integer digits of x
//
// The one-token gate/up evaluates the same per-group identity with exact
// integer dot products. A 64-column group of x is held as x_j = f * X_j, X_j an
// integer with |X_j| <= 2^22 (the group's largest |x_j| scaled just below
// 2^22), written with 6 signed base-16 digits d_p in [-8, 7], X = sum_p d_p 16^p.
// A digit word holds digit p of the 8 columns whose codes share one 32-bit code
// word, nibble n of the digit word for code nibble n, so that one
// v_dot8_i32_i4 of a code word and a digit word adds the 8 products code * digit
// exactly. 4-bit codes enter as c - 8 (the nibbles xor 8, two's complement), so
//   sum_j c_j x_j = f * sum_p 16^p sum_j (c_j - 8) d_jp + 8 sum_j x_j;
// 2-bit codes (0..3, non-negative as signed nibbles) enter as they are, after a
// mask spreads each code word into two words of 4-bit fields. The only
// roundings are those of X_j (at most 2^-22 of the group's largest |x_j|) and of
// the final fp32 combination.
constexpr int kDigits = 6;
constexpr int kDigWords = 8 * kDigits;     // digit words of a group
static_assert(kDigStride == kDigWords + 4, "per group: digit words, f, sum x, two spare words");

// Column (within the group) of nibble n of code word k. 4-bit: word k holds
// columns 8k .. 8k+7, byte b's low nibble column 8k+b, its high nibble 8k+4+b.
// 2-bit: packed word u = k/2 holds columns 16u .. 16u+15, byte b's field q
// column 16u+4q+b; the mask keeps fields 0 and 2 of every byte in nibbles
// (k even), the mask after a shift by two fields 1 and 3 (k odd).
template <int BITS>
__device__ __forceinline__ int digit_column(int k, int n) {
  if constexpr (BITS == 4) return 8 * k + (n >> 1) + 4 * (n & 1);
  return 16 * (k >> 1) + 4 * (k & 1) + 8 * (n & 1) + (n >> 1);
}

struct XDig {
  uint32_t d[kDigWords];  // digit word p of code word k at d[kDigits k + p]
  float f;                // x_j = f * X_j
  float sx;               // sum_j x_j
};

__device__ __forceinline__ void read_digits(const uint32_t *lds, int g, XDig &xd) {
  const uint4 *src = reinterpret_cast<const uint4 *>(lds + g * kDigStride);
#pragma unroll
  for (int i = 0; i < kDigWords / 4; ++i) {
    const uint4 t = src[i];
    xd.d[4 * i] = t.x;
    xd.d[4 * i + 1] = t.y;
    xd.d[4 * i + 2] = t.z;
    xd.d[4 * i + 3] = t.w;
  }
  const float2 fs = *reinterpret_cast<const float2 *>(lds + g * kDigStride + kDigWords);
  xd.f = fs.x;
  xd.sx = fs.y;
}

// sum_p 16^p acc_p (the low four digits exactly in 32-bit integers)
__device__ __forceinline__ float digit_sum(const int (&acc)[kDigits]) {
  const int lo = acc[0] + 16 * acc[1] + 256 * acc[2] + 4096 * acc[3];
  const int hi = acc[4] + 16 * acc[5];
  return fmaf((float)hi, 65536.f, (float)lo);
}

// scale * sum c x + bias * sum x over the lane's group, from the digit form of x
template <int BITS>
__device__ __forceinline__ float group_partial_dig(const Chunk<BITS> &c, uint32_t sb, const XDig &xd) {
  int acc[kDigits];
#pragma unroll
  for (int p = 0; p < kDigits; ++p) acc[p] = 0;
  if constexpr (BITS == 4) {
    const uint32_t w[8] = {c.a.x, c.a.y, c.a.z, c.a.w, c.b.x, c.b.y, c.b.z, c.b.w};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int cs = (int)(w[k] ^ 0x88888888u);
#pragma unroll
      for (int p = 0; p < kDigits; ++p) acc[p] = __builtin_amdgcn_sdot8(cs, (int)xd.d[kDigits * k + p], acc[p], false);
    }
    const float s = scale_of(sb);
    return fmaf(s * xd.f, digit_sum(acc), fmaf(8.f, s, bias_of(sb)) * xd.sx);
  } else {
    const uint32_t w[4] = {c.a.x, c.a.y, c.a.z, c.a.w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int n0 = (int)(w[u] & 0x33333333u), n1 = (int)((w[u] >> 2) & 0x33333333u);
#pragma unroll
      for (int p = 0; p < kDigits; ++p) {
        acc[p] = __builtin_amdgcn_sdot8(n0, (int)xd.d[kDigits * (2 * u) + p], acc[p], false);
        acc[p] = __builtin_amdgcn_sdot8(n1, (int)xd.d[kDigits * (2 * u + 1) + p], acc[p], false);
      }
    }
    return fmaf(scale_of(sb) * xd.f, digit_sum(acc), bias_of(sb) * xd.sx);
  }
}

// ------------------------------------------------------------------ cross-lane

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
__device__ __forceinline__ int wave_id() { return (int)(blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6)); }

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_f(float v, float old) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWS, 0xF, false));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_i(int v, int old) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWS, 0xF, false);
}

// Cross-lane sums with DPP. After seg_reduce<W>, the last lane of every aligned
// segment of W lanes holds the segment's sum (every lane of it for W <= 16).
// Steps: quad xor 1, quad xor 2, half-row mirror, row mirror (all lanes of a row
// of 16 then hold the row sum), then row broadcasts 15 and 31 across rows.
template <int W>
__device__ __forceinline__ float seg_reduce(float v) {
  if constexpr (W >= 2) v += dpp_f<0xB1, 0xF>(v, 0.f);
  if constexpr (W >= 4) v += dpp_f<0x4E, 0xF>(v, 0.f);
  if constexpr (W >= 8) v += dpp_f<0x141, 0xF>(v, 0.f);
  if constexpr (W >= 16) v += dpp_f<0x140, 0xF>(v, 0.f);
  if constexpr (W >= 32) v += dpp_f<0x142, 0xA>(v, 0.f);
  if constexpr (W >= 64) v += dpp_f<0x143, 0xC>(v, 0.f);
  return v;
}

// The segment's sum in every lane of the segment.
template <int W>
__device__ __forceinline__ float seg_allreduce(float v) {
  v = seg_reduce<W>(v);
  if constexpr (W == 64) return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
  if constexpr (W == 32) {
    const float lo = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 31));
    const float hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
    return lane_id() < 32 ? lo : hi;
  }
  return v;
}

// The lane that holds a segment's sum after seg_reduce.
template <int W>
__device__ __forceinline__ bool seg_last(int lane) {
  return (lane & (W - 1)) == W - 1;
}

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

inline int blocks_for_waves(long waves) { return (int)((waves + (kBlock / kWave) - 1) / (kBlock / kWave)); }

}  // namespace dev
}  // namespace fmoe
