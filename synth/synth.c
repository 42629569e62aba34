/*
 * synth.c -- seeded, counter-based synthetic inputs for the quantized MoE
 * expert forward (host side).
 *
 * This module only draws numbers. It holds none of the method's arithmetic:
 * no dequantization, no dot products, no routing. Both the fp64 oracle and the
 * GPU library consume what it produces, in the canonical layout:
 *   codes  uint8  [rows][cols]        one unsigned code per element
 *   scale  uint16 [rows][cols/group]  bf16 bit pattern
 *   bias   uint16 [rows][cols/group]  bf16 bit pattern
 *   dense  float  [n]                 fp32 values
 *
 * Generator: splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
 * number generators", OOPSLA 2014; the 64-bit finalizer constants are the ones
 * Vigna publishes for splitmix64). Output n of the stream seeded with state k is
 * mix(k + (n + 1) * GAMMA), so any element can be drawn on its own. A stream key
 * is derived from (seed, a, b, c) by chaining that same step, which lets any
 * expert of any layer be regenerated independently of every other one.
 *
 * The device twin (synth_dev.hip) repeats the integer and fp64 steps for codes
 * and scale/bias exactly; both are built without floating-point contraction so
 * that the two agree bit for bit.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define SYN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t syn_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* n-th output (0-based) of the splitmix64 stream whose state starts at key. */
uint64_t syn_word(uint64_t key, uint64_t n) { return syn_mix(key + (n + 1) * SYN_GAMMA); }

/* Stream key for the tensor identified by (a, b, c) under a master seed. */
uint64_t syn_stream(uint64_t seed, uint64_t a, uint64_t b, uint64_t c) {
  uint64_t k = syn_word(seed, a);
  k = syn_word(k, b);
  return syn_word(k, c);
}

/* Round-to-nearest-even fp32 -> bf16 bit pattern (inputs here are finite). */
static inline uint16_t syn_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

static inline float syn_bf16_decode(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

/* Unsigned codes of `bits` (2 or 4) bits each, element e of a row-major
 * [rows][cols] tensor taken from word e / (64 / bits), least significant
 * field first. */
int syn_codes(uint64_t key, int bits, int64_t n, uint8_t *out) {
  if (bits != 2 && bits != 4) return -1;
  const int per = 64 / bits;
  const uint64_t mask = (1u << bits) - 1u;
  int64_t nw = (n + per - 1) / per;
#pragma omp parallel for schedule(static)
  for (int64_t w = 0; w < nw; ++w) {
    uint64_t v = syn_word(key, (uint64_t)w);
    int64_t base = w * per;
    int lim = (n - base) < per ? (int)(n - base) : per;
    for (int i = 0; i < lim; ++i) out[base + i] = (uint8_t)((v >> (bits * i)) & mask);
  }
  return 0;
}

/* Per-group scale and bias, one splitmix64 word per (row, group) pair:
 *   u1 = bits 40..63 / 2^24, u2 = bits 16..39 / 2^24
 *   scale = bf16(fp32(lo + (hi - lo) * u1))
 *   bias  = bf16(fp32(-bmul * scale_decoded * (1 + (2 * spread * u2 - spread))))
 * Each fp64 step is a separately rounded operation (no fused multiply-add). */
int syn_scale_bias(uint64_t key, int64_t n, double lo, double hi, double bmul, double spread,
                   uint16_t *scale, uint16_t *bias) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t v = syn_word(key, (uint64_t)i);
    double u1 = (double)(v >> 40) * 0x1p-24;
    double u2 = (double)((v >> 16) & 0xFFFFFFu) * 0x1p-24;
    double width = hi - lo;
    double s = width * u1;
    s = lo + s;
    uint16_t sb = syn_bf16_rne((float)s);
    double sd = (double)syn_bf16_decode(sb);
    double t = (2.0 * spread) * u2;
    t = t - spread;
    t = 1.0 + t;
    double b = (-bmul) * sd;
    b = b * t;
    scale[i] = sb;
    bias[i] = syn_bf16_rne((float)b);
  }
  return 0;
}

/* Normal(0, std) via Box-Muller in fp64 from words 2i and 2i+1, rounded to fp32. */
int syn_normal(uint64_t key, int64_t n, double std, float *out) {
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t w1 = syn_word(key, 2 * (uint64_t)i);
    uint64_t w2 = syn_word(key, 2 * (uint64_t)i + 1);
    double u1 = (double)((w1 >> 11) + 1) * 0x1p-53; /* (0, 1] */
    double u2 = (double)(w2 >> 11) * 0x1p-53;       /* [0, 1) */
    double r = sqrt(-2.0 * log(u1));
    double z = r * cos(two_pi * u2);
    out[i] = (float)(z * std);
  }
  return 0;
}

/* Uniform [lo, hi) floats from 24-bit fractions. */
int syn_uniform(uint64_t key, int64_t n, double lo, double hi, float *out) {
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    uint64_t v = syn_word(key, (uint64_t)i);
    double u = (double)(v >> 40) * 0x1p-24;
    double t = (hi - lo) * u;
    out[i] = (float)(lo + t);
  }
  return 0;
}
