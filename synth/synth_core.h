/*
 * Seeded synthetic inputs: the element generators.
 *
 * Test and benchmark infrastructure, not part of the MoE layer: it holds no
 * step of the method. Every element of every tensor is a pure function of
 * (key, flat index), so the host build (synth_host.c) and the device build
 * (synth_dev.hip) produce the same bytes, in any chunking and any order.
 *
 * Generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable
 * pseudorandom number generators", OOPSLA 2014; constants as published by
 * Vigna for java.util.SplittableRandom). Element n of a stream with key k is
 * mix64(k + (n + 1) * golden_gamma).
 *
 * Distributions (all floating point in single f32 operations, no fused
 * multiply-add, so both builds round identically; compile with
 * -ffp-contract=off):
 *   normal(sigma): Irwin-Hall sum of the four 16-bit lanes of one draw,
 *       centred: s = sum - 131070, value = f32(s) * c with the f32 constant
 *       c = sigma * sqrt(3) / 65536 supplied by the caller (unit variance
 *       before scaling, bounded at +-3.46 sigma).
 *   uniform(lo, hi): t = top 24 bits / 2^24 (exact), value = lo + w * t with
 *       w = hi - lo given as an f32 (one multiply, one add).
 *   int8 uniform on [-127, 127]: draw mod 255 - 127.
 *   raw byte (e2m1 code pairs): top 8 bits of the draw.
 *   e8m0 byte uniform on [127 + emin, 127 + emax]: 127 + emin + draw mod span.
 * Storage roundings: f32 -> bf16 and f32 -> fp16 round to nearest even
 * (finite, normal inputs only; the generated ranges never leave them).
 */
#ifndef SYNTH_CORE_H
#define SYNTH_CORE_H

#include <stdint.h>

#if defined(__HIPCC__)
#define SYN_FN __host__ __device__ static inline
#else
#define SYN_FN static inline
#endif

#define SYN_GAMMA 0x9E3779B97F4A7C15ull

SYN_FN uint64_t syn_mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

/* Draw n of the stream keyed by `key`. */
SYN_FN uint64_t syn_draw(uint64_t key, uint64_t n) {
  return syn_mix64(key + (n + 1ull) * SYN_GAMMA);
}

/* Stream key for (seed, tensor tag, sub-index such as an expert or a sample). */
SYN_FN uint64_t syn_key(uint64_t seed, uint32_t tag, uint32_t index) {
  uint64_t k = syn_mix64(seed * SYN_GAMMA + 0x632BE59BD9B4E019ull);
  return syn_mix64(k ^ (((uint64_t)tag << 32) | (uint64_t)index));
}

SYN_FN uint32_t syn_f32_bits(float f) {
  union { float f; uint32_t u; } v;
  v.f = f;
  return v.u;
}

SYN_FN float syn_normal(uint64_t x, float c) {
  int32_t s = (int32_t)(x & 0xFFFFu) + (int32_t)((x >> 16) & 0xFFFFu) +
              (int32_t)((x >> 32) & 0xFFFFu) + (int32_t)(x >> 48) - 131070;
  return (float)s * c;
}

SYN_FN float syn_uniform(uint64_t x, float lo, float width) {
  float t = (float)(uint32_t)(x >> 40) * 5.9604644775390625e-08f; /* 2^-24 */
  float m = width * t;
  return lo + m;
}

SYN_FN uint16_t syn_to_bf16(float f) {
  uint32_t u = syn_f32_bits(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* f32 -> fp16, round to nearest even; normal fp16 range only. */
SYN_FN uint16_t syn_to_f16(float f) {
  uint32_t u = syn_f32_bits(f);
  uint32_t sign = (u >> 16) & 0x8000u;
  int32_t e = (int32_t)((u >> 23) & 0xFF) - 127 + 15;
  uint32_t m = u & 0x7FFFFFu;
  uint32_t h = ((uint32_t)e << 10) | (m >> 13);
  uint32_t rest = m & 0x1FFFu;
  if (rest > 0x1000u || (rest == 0x1000u && (h & 1u))) h += 1u;
  return (uint16_t)(sign | h);
}

SYN_FN int8_t syn_i8(uint64_t x) { return (int8_t)((int32_t)(x % 255ull) - 127); }

SYN_FN uint8_t syn_byte(uint64_t x) { return (uint8_t)(x >> 56); }

SYN_FN uint8_t syn_e8m0(uint64_t x, int32_t emin, int32_t emax) {
  return (uint8_t)(127 + emin + (int32_t)(x % (uint64_t)(emax - emin + 1)));
}

/* Encodings a tensor can be filled with. */
enum {
  SYN_F32_NORMAL = 0,   /* float,    p0 = c (sigma*sqrt(3)/65536)  */
  SYN_BF16_NORMAL = 1,  /* uint16,   p0 = c                        */
  SYN_F32_UNIFORM = 2,  /* float,    p0 = lo, p1 = hi - lo         */
  SYN_BF16_UNIFORM = 3, /* uint16,   p0 = lo, p1 = hi - lo         */
  SYN_F16_UNIFORM = 4,  /* uint16,   p0 = lo, p1 = hi - lo         */
  SYN_I8_UNIFORM = 5,   /* int8,     [-127, 127]                   */
  SYN_BYTES = 6,        /* uint8,    raw byte (two e2m1 codes)     */
  SYN_E8M0 = 7          /* uint8,    i0 = emin, i1 = emax          */
};

SYN_FN int syn_elem_bytes(int kind) {
  switch (kind) {
    case SYN_F32_NORMAL: case SYN_F32_UNIFORM: return 4;
    case SYN_BF16_NORMAL: case SYN_BF16_UNIFORM: case SYN_F16_UNIFORM: return 2;
    default: return 1;
  }
}

/* Writes element n of the stream (key, kind) to out[i]. */
SYN_FN void syn_put(void* out, uint64_t i, int kind, uint64_t key, uint64_t n, float p0,
                    float p1, int32_t i0, int32_t i1) {
  uint64_t x = syn_draw(key, n);
  switch (kind) {
    case SYN_F32_NORMAL: ((float*)out)[i] = syn_normal(x, p0); break;
    case SYN_BF16_NORMAL: ((uint16_t*)out)[i] = syn_to_bf16(syn_normal(x, p0)); break;
    case SYN_F32_UNIFORM: ((float*)out)[i] = syn_uniform(x, p0, p1); break;
    case SYN_BF16_UNIFORM: ((uint16_t*)out)[i] = syn_to_bf16(syn_uniform(x, p0, p1)); break;
    case SYN_F16_UNIFORM: ((uint16_t*)out)[i] = syn_to_f16(syn_uniform(x, p0, p1)); break;
    case SYN_I8_UNIFORM: ((int8_t*)out)[i] = syn_i8(x); break;
    case SYN_BYTES: ((uint8_t*)out)[i] = syn_byte(x); break;
    case SYN_E8M0: ((uint8_t*)out)[i] = syn_e8m0(x, i0, i1); break;
    default: break;
  }
}

#endif /* SYNTH_CORE_H */
