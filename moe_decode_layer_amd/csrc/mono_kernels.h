/*
 * libmonolayer device code for gfx950 (CDNA4, wave64): phases, kernels and launch templates.
 * Included by the per-format translation units; nothing here is instantiated on its own.
 *
 * The layer-half step is written as phases (device functions). The unfused entry points run
 * each phase as its own kernel; the fused entry point runs every phase in ONE persistent launch
 * (one workgroup per compute unit) with no grid barrier: workgroups hand values to each other
 * tagged with the launch epoch and the readers poll for the tag. Every output element has a
 * fixed decomposition (one wave per dot product, fixed lane mapping, fixed reduction tree),
 * independent of which workgroup computes it, so the fused and unfused paths give identical
 * bytes.
 *
 * The step is a chain of HBM-bound matrix-vector products (1 to 8 activation rows against
 * weights read once), so it runs on the vector ALUs: each lane streams 16-byte weight vectors
 * (1 KB per wave per step, coalesced), a wave keeps a whole row's loads in flight, weights are
 * decoded once per vector into packed bf16 pairs (exact for bf16, Q8_0 and e2m1 values) and
 * every activation row consumes them with v_dot2_f32_bf16 (exact products, f32 sums).
 * Activations live in LDS. Reductions use DPP. The one dense product of the step, the shared
 * expert's gate/up at several rows, runs on the matrix cores (v_mfma_f32_16x16x32_bf16).
 *
 * Data that crosses workgroups inside the fused launch (mix partials, router logits, hidden rows,
 * down outputs at several rows, carry partials) is written with device-coherent (sc1) stores,
 * each value with the launch tag beside it, and read with device-coherent loads that poll
 * until the tag is current. No cache write-back or invalidation is needed.
 *
 * Steps and rounding points follow the ds4 page "v41: fuse the single-box decode glue (HC, MoE,
 * attention)" ("What" and its HC and router/shared-expert commits); the fused launch follows K2
 * of the SGLang page "[AMD][V4.1] Mono kernel framework ... DeepSeek-V4.1 decode layers" (figure
 * "DeepSeek-V4.1 layer on mono"), the load order of the lm-sys page "Add the AMD low-latency
 * kernels section" (Layer diagram: mHC mix weights and the shared expert early, routed experts
 * after routing) and the post -> next-pre carry of the SGLang page "[DeepSeek-V4] Add
 * mhc_fused_post_pre kernel" ("Motivation").
 */
#ifndef MONOLAYER_KERNELS_H
#define MONOLAYER_KERNELS_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mono_internal.h"

namespace mono {

enum { F32 = MONO_F32, BF16 = MONO_BF16, Q8 = MONO_Q8_0, FP4 = MONO_MXFP4 };

constexpr int kMaxUnion = kMaxRows * kMaxTopK;
constexpr int kRG = 4; /* consecutive down-projection rows per task */
constexpr int kMaxStaged = 160; /* hidden rows staged at once (80 KB / 512 B at least) */
constexpr uint32_t kHidShared = 0x80000000u;
constexpr int kSliceMax = 32; /* hidden positions per workgroup whose expand inputs sit in LDS */

/* ------------------------------------------------------------------------------------------
 * Number formats */

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

/* f32 -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32). */
__device__ __forceinline__ uint32_t f2bf(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

/* Two f32 -> packed bf16 pair (lo in the low half), round to nearest even. */
__device__ __forceinline__ uint32_t f2bf2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

template <int ACT>
__device__ __forceinline__ float act_round(float v) {
  return ACT == F32 ? v : bf2f(f2bf(v));
}

template <int ACT>
__device__ __forceinline__ float act_ld(const void* p, size_t i) {
  if (ACT == F32) return static_cast<const float*>(p)[i];
  return bf2f(static_cast<const uint16_t*>(p)[i]);
}

/* Stores v (already rounded to the act type). */
template <int ACT>
__device__ __forceinline__ void act_st(void* p, size_t i, float v) {
  if (ACT == F32)
    static_cast<float*>(p)[i] = v;
  else
    static_cast<uint16_t*>(p)[i] = (uint16_t)f2bf(v);
}

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

/* e8m0 scale 2^(e-127). */
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
  if (e == 0) return __uint_as_float(0x00400000u);
  if (e == 255) return __uint_as_float(0x7FC00000u);
  return __uint_as_float(e << 23);
}

/* MXFP8 round trip of a value v of a block whose shared exponent is X [vLLM "[ROCm][Perf][GLM-5]
 * Fused sparse-layer decode via AITER MonoKernel", Details, Numerics: activations of the MXFP4
 * experts quantised to MXFP8]. READING: the OCP MX v1.0 conversion with E4M3 elements: v / 2^X
 * rounded to the nearest E4M3 number (3 mantissa bits; below 2^-6 the subnormal spacing 2^-9),
 * ties to even, magnitudes above 448 clamped to 448, then times 2^X. Every step is exact in f32
 * except the one rounding (rintf rounds to nearest even). */
__device__ __forceinline__ float mx8_rt(float v, int X) {
  const float t = ldexpf(v, -X);
  const uint32_t eb = __float_as_uint(t) >> 23 & 0xFFu; /* biased exponent of |t| */
  const int qe = eb < 121u ? -9 : (int)eb - 130;         /* log2 of the E4M3 spacing at |t| */
  float r = ldexpf(rintf(ldexpf(t, -qe)), qe);
  r = fminf(fmaxf(r, -448.0f), 448.0f);
  return ldexpf(r, X);
}

/* MXFP8 round trip, in place, of one block of 32 bf16 values (64 bytes of LDS). The shared
 * exponent is X = floor(log2 max|v|) - 8, clamped to [-127, 127] (bf16 magnitudes order as
 * integers, and the exponent field of the largest is floor(log2) + 127). An all-zero block is
 * left as it is. The results are exact in bf16 (4 significant bits times a power of two). */
__device__ __forceinline__ void mx8_block_lds(uint8_t* b) {
  uint4* q = reinterpret_cast<uint4*>(b);
  uint32_t w[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 v = q[i];
    w[4 * i] = v.x;
    w[4 * i + 1] = v.y;
    w[4 * i + 2] = v.z;
    w[4 * i + 3] = v.w;
  }
  uint32_t mx = 0;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    mx = max(mx, w[j] & 0x7FFFu);
    mx = max(mx, (w[j] >> 16) & 0x7FFFu);
  }
  if (mx == 0) return;
  int X = (int)(mx >> 7) - 127 - 8;
  X = X < -127 ? -127 : (X > 127 ? 127 : X);
#pragma unroll
  for (int j = 0; j < 16; ++j)
    w[j] = f2bf2(mx8_rt(bf2f(w[j] & 0xFFFFu), X), mx8_rt(bf2f(w[j] >> 16), X));
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
}

/* c + a.lo * b.lo + a.hi * b.hi for packed bf16 pairs. */
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

/* ------------------------------------------------------------------------------------------
 * Device-coherent accesses for data shared between workgroups of one launch */

template <typename T>
__device__ __forceinline__ T ld_coh(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void st_coh(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

/* Tagged hidden-row value: bf16 bits | tag << 16 (uint32) or f32 bits | tag << 32 (uint64). */
template <int ACT>
__device__ __forceinline__ void hid_store(void* base, size_t i, float v, uint32_t tag) {
  if (ACT == F32)
    st_coh(static_cast<uint64_t*>(base) + i, ((uint64_t)tag << 32) | __float_as_uint(v));
  else
    st_coh(static_cast<uint32_t*>(base) + i, (tag << 16) | f2bf(v));
}

/* Device-coherent (sc1) loads issued as buffer loads: unlike atomic loads they are ordinary
 * memory operations, so a wave keeps many in flight. Offsets are bytes inside the region the
 * resource covers; reads past its end return 0. */
typedef unsigned int v4u_t __attribute__((ext_vector_type(4)));
typedef unsigned int v2u_t __attribute__((ext_vector_type(2)));
constexpr int kCohPolicy = 16; /* sc1: device scope */

__device__ __forceinline__ __amdgpu_buffer_rsrc_t coh_region(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}
__device__ __forceinline__ uint4 coh_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v4u_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCohPolicy);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ uint2 coh_b64(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const v2u_t v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kCohPolicy);
  return make_uint2(v[0], v[1]);
}

/* Copies n tagged values (value bits | tag << 32, uint64) at src into LDS as floats at dst with
 * the whole workgroup, two values per 16-byte coherent load, B loads per thread in flight. With
 * check, a pair whose tags are not yet `tag` is loaded again (bounded by spin ticks); returns
 * false (uniform) on expiry. */
template <int B>
__device__ __forceinline__ bool coh_copy_tagged_to_lds(const uint64_t* src, int n, float* dst,
                                                       bool check, uint32_t tag, uint32_t spin,
                                                       int* flag) {
  const int tid = threadIdx.x;
  const __amdgpu_buffer_rsrc_t r = coh_region(src, (size_t)n * 8);
  const int npair = (n + 1) / 2;
  if (tid == 0) *flag = 1;
  __syncthreads();
  bool ok = true;
  for (int v0 = 0; v0 < npair; v0 += B * kBlock) {
    uint4 buf[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int v = v0 + b * kBlock + tid; /* past the end: a repeated pair, unused */
      buf[b] = coh_b128(r, (uint32_t)(v < npair ? v : npair - 1) * 16u);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int v = v0 + b * kBlock + tid;
      if (v >= npair) continue;
      const bool two = 2 * v + 1 < n;
      if (check && (buf[b].y != tag || (two && buf[b].w != tag))) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (buf[b].y != tag || (two && buf[b].w != tag)) {
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_sleep(1);
          buf[b] = coh_b128(r, (uint32_t)v * 16u);
          if (__builtin_amdgcn_s_memrealtime() - t0 > spin) {
            ok = false;
            break;
          }
        }
      }
      dst[2 * v] = __uint_as_float(buf[b].x);
      if (two) dst[2 * v + 1] = __uint_as_float(buf[b].z);
    }
  }
  if (!ok) *flag = 0;
  __syncthreads();
  return *flag != 0;
}

/* Waits until this wave's memory operations have completed (and orders the compiler). */
__device__ __forceinline__ void drain() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }


/* ------------------------------------------------------------------------------------------
 * Wave reductions (DPP butterflies inside each row of 16 lanes, then the four row sums). Must
 * be called with all 64 lanes active; every lane returns the same value. */

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, false);
}

__device__ __forceinline__ float readlane(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dpp<0xB1>(v);  /* quad_perm [1,0,3,2] */
  v += dpp<0x4E>(v);  /* quad_perm [2,3,0,1] */
  v += dpp<0x141>(v); /* row_half_mirror */
  v += dpp<0x140>(v); /* row_mirror */
  return (readlane(v, 0) + readlane(v, 16)) + (readlane(v, 32) + readlane(v, 48));
}

/* ------------------------------------------------------------------------------------------
 * Weight streaming. A step of a row covers 64 lanes x 16 bytes (1 KB): 4 f32, 8 bf16, 16 Q8_0
 * or 32 MXFP4 values per lane, so lane L of step s holds elements [(64 s + L) * EL, + EL).
 * CH_GU / CH_DN: steps a wave keeps in flight per row in the gate/up and down phases. */

template <int FMT> struct Fmt;
template <> struct Fmt<F32> { static constexpr int EL = 4, CH_GU = 8, CH_DN = 4, PAIRS = 0; };
template <> struct Fmt<BF16> { static constexpr int EL = 8, CH_GU = 10, CH_DN = 4, PAIRS = 4; };
template <> struct Fmt<Q8> { static constexpr int EL = 16, CH_GU = 5, CH_DN = 2, PAIRS = 8; };
template <> struct Fmt<FP4> { static constexpr int EL = 32, CH_GU = 3, CH_DN = 1, PAIRS = 16; };
/* Routed tasks of the fused launch at several rows when the expert serves one row (the common
 * case): GB hidden rows per gate/up task and DG down rows per down task, so that a wave keeps
 * 16-20 KB of weights in flight whatever the format. */
template <int FMT> struct Wide;
template <> struct Wide<F32> { static constexpr int GB = 1, DG = 4; };
template <> struct Wide<BF16> { static constexpr int GB = 1, DG = 4; };
template <> struct Wide<Q8> { static constexpr int GB = 2, DG = 8; };
template <> struct Wide<FP4> { static constexpr int GB = 4, DG = 16; };

__host__ __device__ constexpr size_t row_vbytes(int fmt, size_t k) {
  return fmt == F32 ? 4 * k : fmt == BF16 ? 2 * k : fmt == Q8 ? k : k / 2;
}
__host__ __device__ constexpr size_t row_sbytes(int fmt, size_t k) {
  return fmt == Q8 ? (k / 32) * 2 : fmt == FP4 ? k / 32 : 0;
}

/* Buffer resource over one weight row (a wave-uniform address, so the resource lives in scalar
 * registers): loads past `bytes` return zeros in hardware, so the weight loads need no bounds
 * branch and a wave issues all of a chunk's loads before it waits for any. */
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const uint8_t* row, size_t bytes) {
  /* readfirstlane returns int: go through uint32_t so the low word is not sign-extended */
  const uint64_t a = reinterpret_cast<uint64_t>(row);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32));
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  const uint64_t u = ((uint64_t)hi << 32) | (uint64_t)lo;
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(u), (short)0, (int)bytes,
                                           0x00020000);
}

/* Loads step s of a Q8_0 or MXFP4 row for this lane, with its block scale (zeros past the end
 * of the row). */
template <int FMT>
__device__ __forceinline__ void wload(__amdgpu_buffer_rsrc_t vr, __amdgpu_buffer_rsrc_t sr, int s,
                                      int lane, uint4& v, uint32_t& sc) {
  const int q = s * 64 + lane;
  const v4u_t x = __builtin_amdgcn_raw_buffer_load_b128(vr, q * 16, 0, 0);
  v = make_uint4(x[0], x[1], x[2], x[3]);
  if (FMT == Q8) sc = __builtin_amdgcn_raw_buffer_load_b16(sr, (q * Fmt<FMT>::EL / 32) * 2, 0, 0);
  else sc = __builtin_amdgcn_raw_buffer_load_b8(sr, q * Fmt<FMT>::EL / 32, 0, 0);
}

/* Exact decode of one 16-byte weight vector into packed bf16 pairs (element 2m in the low
 * half of pair m) and its block scale. Q8_0: each int8 q converts to f32 exactly, and the top 16
 * bits of that f32 are the exact bf16 of q (|q| <= 128 needs 8 significant bits). MXFP4: each byte converts to
 * a bf16 pair (low nibble first) with unit scale; the e8m0 scale multiplies the partial sum. */
template <int FMT>
__device__ __forceinline__ void decode(const uint4& v, uint32_t sc, uint32_t (&w)[Fmt<FMT>::PAIRS],
                                       float& scale) {
  if constexpr (FMT == BF16) {
    w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    scale = 1.0f;
  } else if constexpr (FMT == Q8) {
    /* one sign-extending byte-to-float conversion per value */
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float f0 = (float)(int)(int8_t)d[i];
      const float f1 = (float)(int)(int8_t)(d[i] >> 8);
      const float f2 = (float)(int)(int8_t)(d[i] >> 16);
      const float f3 = (float)(int)(int8_t)(d[i] >> 24);
      w[2 * i] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
      w[2 * i + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
    scale = f16_to_f32(sc);
  } else if constexpr (FMT == FP4) {
    const uint32_t d[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 0));
      w[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 1));
      w[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 2));
      w[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d[i], 1.0f, 3));
    }
    scale = e8m0_to_f32(sc);
  }
}

/* acc + scale * (pairs . bf16 activations k .. k + 2 PAIRS - 1 of one LDS row). */
/* acc + scale * (weight pairs . activations[k, k + EL)) for one lane. */
template <int FMT>
__device__ __forceinline__ float dot_pairs(const uint32_t (&w)[Fmt<FMT>::PAIRS], float scale,
                                           const void* arow, int k, float acc) {
  constexpr int P = Fmt<FMT>::PAIRS;
  const uint16_t* a = static_cast<const uint16_t*>(arow) + k;
  if constexpr (FMT == BF16) {
    const uint4 x = *reinterpret_cast<const uint4*>(a);
    acc = dot2bf(w[0], x.x, acc);
    acc = dot2bf(w[1], x.y, acc);
    acc = dot2bf(w[2], x.z, acc);
    acc = dot2bf(w[3], x.w, acc);
    return acc;
  } else {
    float part = 0.0f;
#pragma unroll
    for (int c = 0; c < P / 4; ++c) {
      const uint4 x = *reinterpret_cast<const uint4*>(a + 8 * c);
      part = dot2bf(w[4 * c + 0], x.x, part);
      part = dot2bf(w[4 * c + 1], x.y, part);
      part = dot2bf(w[4 * c + 2], x.z, part);
      part = dot2bf(w[4 * c + 3], x.w, part);
    }
    return fmaf(scale, part, acc);
  }
}

/* f32 weights against f32 activations (the all-f32 workload). */
__device__ __forceinline__ float dot_f32(const uint4& v, const void* arow, int k, float acc) {
  const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(arow) + k);
  acc = fmaf(__uint_as_float(v.x), x.x, acc);
  acc = fmaf(__uint_as_float(v.y), x.y, acc);
  acc = fmaf(__uint_as_float(v.z), x.z, acc);
  acc = fmaf(__uint_as_float(v.w), x.w, acc);
  return acc;
}

/* Weight registers of CH steps of NR rows (one chunk of a wave task). */
template <int FMT, int NR, int CH>
struct WRegs {
  uint4 v[NR][CH];
  uint32_t sc[NR][CH];
};

template <int FMT, int NR, int CH>
__device__ __forceinline__ void wregs_load(WRegs<FMT, NR, CH>& W, const uint8_t* const (&vrow)[NR],
                                           const uint8_t* const (&srow)[NR], int K, int s0) {
  const int lane = threadIdx.x & 63;
  if constexpr (FMT == Q8 || FMT == FP4) {
    /* the decode would otherwise be sunk into a bounds branch per load, one load in flight */
    const size_t vb = row_vbytes(FMT, K), sb = row_sbytes(FMT, K);
    __amdgpu_buffer_rsrc_t vr[NR], sr[NR];
#pragma unroll
    for (int m = 0; m < NR; ++m) {
      vr[m] = row_rsrc(vrow[m], vb);
      sr[m] = row_rsrc(srow[m], sb);
    }
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int m = 0; m < NR; ++m) wload<FMT>(vr[m], sr[m], s0 + c, lane, W.v[m][c], W.sc[m][c]);
  } else {
    constexpr int EL = Fmt<FMT>::EL;
    const int nsteps = (K + 64 * EL - 1) / (64 * EL);
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        const int q = (s0 + c) * 64 + lane;
        if (s0 + c < nsteps && q * EL < K)
          W.v[m][c] = *reinterpret_cast<const uint4*>(vrow[m] + (size_t)q * 16);
        else
          W.v[m][c] = make_uint4(0, 0, 0, 0);
        W.sc[m][c] = 0;
      }
  }
}

/* acc[m][r] += (chunk of row m) . act_r for every r in `mask` (per-lane partials); with one
 * row every task row is used, so the row test is dropped. */
template <int FMT, int ACT, int RMAX, int NR, int CH>
__device__ __forceinline__ void wregs_dot(const WRegs<FMT, NR, CH>& W, int K, int s0,
                                          const void* const (&arow)[RMAX], uint32_t mask,
                                          float (&acc)[NR][RMAX]) {
  constexpr int EL = Fmt<FMT>::EL;
  const int lane = threadIdx.x & 63;
  const int nsteps = (K + 64 * EL - 1) / (64 * EL);
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int k = ((s0 + c) * 64 + lane) * EL;
    if (s0 + c < nsteps && k < K) {
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        if constexpr (FMT == F32) {
#pragma unroll
          for (int r = 0; r < RMAX; ++r)
            if (RMAX == 1 || (mask & (1u << r))) acc[m][r] = dot_f32(W.v[m][c], arow[r], k, acc[m][r]);
        } else {
          uint32_t w[Fmt<FMT>::PAIRS];
          float scale;
          decode<FMT>(W.v[m][c], W.sc[m][c], w, scale);
#pragma unroll
          for (int r = 0; r < RMAX; ++r)
            if (RMAX == 1 || (mask & (1u << r))) acc[m][r] = dot_pairs<FMT>(w, scale, arow[r], k, acc[m][r]);
        }
      }
    }
  }
}

/* acc[m][r] += row_m . act_r over K elements, CH steps of all NR rows in flight at a time. */
template <int FMT, int ACT, int RMAX, int NR, int CH>
__device__ __forceinline__ void dot_rows(const uint8_t* const (&vrow)[NR],
                                         const uint8_t* const (&srow)[NR], int K,
                                         const void* const (&arow)[RMAX], uint32_t mask,
                                         float (&acc)[NR][RMAX], int s_begin = 0) {
  constexpr int EL = Fmt<FMT>::EL;
  const int nsteps = (K + 64 * EL - 1) / (64 * EL);
  for (int s0 = s_begin; s0 < nsteps; s0 += CH) {
    WRegs<FMT, NR, CH> W;
    wregs_load(W, vrow, srow, K, s0);
    wregs_dot<FMT, ACT, RMAX, NR, CH>(W, K, s0, arow, mask, acc);
  }
}

/* ------------------------------------------------------------------------------------------
 * Workgroup shared memory */

struct Smem {
  alignas(16) uint8_t big[kLdsActBytes]; /* act rows [R][H] + norm weight [H]; down phase:
                                            staged hidden rows, then y and block values */
  float raw[kMaxRows][kNCarry];
  float mixes[kMaxRows][kNMix];
  float pre[kMaxRows][4];
  float post[kMaxRows][4];
  float comb[kMaxRows][16];
  float hcs[4];
  float hcb[kNMix];
  float red[kWaves][kMaxRows];
  float rsum[kMaxRows];
  int sel_e[kMaxRows][kMaxTopK];
  float sel_w[kMaxRows][kMaxTopK];
  int U[kMaxUnion + 1];
  uint32_t umask[kMaxUnion + 1];
  int8_t uslot[kMaxUnion + 1][kMaxRows];
  uint16_t voff[kMaxUnion + 1][kMaxRows]; /* staged hidden row offset per (item, row), 16 B */
  uint32_t ubits[kMaxExperts / 32]; /* plan: selected experts as a bitmap */
  int ubase[kMaxExperts / 32];       /* plan: distinct experts before each bitmap word */
  uint32_t vsrc[kMaxStaged]; /* staged hidden rows: source offset (flag: shared), */
  uint16_t vdst[kMaxStaged]; /* LDS offset in 16 B, */
  uint16_t vlen[kMaxStaged]; /* length in 16 B */
  int nv;
  int sel_ok;      /* cleared when a select wave's logits did not arrive */
  int shared_next; /* next shared-expert gate/up task of this workgroup (fused launch) */
  int routed_next; /* next routed gate/up task of this workgroup (fused launch) */
  int down_next;   /* next down block of the current staged group (fused launch, several rows),
                      or next down task of the one-row flow */
  int em_q0, em_q1, em_u1; /* several rows: this workgroup's down stretch [q0, q1) and the end
                              of its first staged group, found with the plan */
  int lg_ready;   /* one row: wave 0 has gathered the logits (or given up waiting) */
  int plan_ready; /* one row: 0 not yet, 1 the plan is built, 2 the logits did not arrive */
  int stage_state[kMaxUnion + 1]; /* one-row flow: item staged? 0 no, 1 being staged, 2 yes,
                                     3 its hidden rows did not arrive */
  int nU;
  int flag;
  uint64_t epoch;
  int trace_on;
  int state_in_lds;
  float bias[kMaxExperts];
  float wnext[kNMix * 4 * kSliceMax]; /* next mix weights of the slice [24][4][hs]; before
                                         the down phase, the collapse's sums of squares */
  float sslice[kMaxRows * 4 * kSliceMax]; /* input state of the slice [R][4][hs] */
  float cred[kMaxGrid];                  /* carry reduction: one partial per workgroup */
  uint32_t spin;
  int skip_phase;
};

/* ------------------------------------------------------------------------------------------
 * Ordering between the workgroups of the fused launch. There is no grid barrier: every value a
 * workgroup publishes for others (mix partials, router logits, hidden rows, carry partials)
 * is stored with a tag of the launch beside it, and the reader waits until the tags are
 * current. The tag comes from the launch epoch: the first thing every workgroup does is add 1
 * to a start counter (one of 8, by blockIdx % 8) and keep the old value. Group g has
 * n_g = ceil((grid - g) / 8) workgroups, so every launch advances counter g by exactly n_g, and
 * since launches on one workspace run one after another (stream order), every workgroup of the
 * N-th launch reads an old value in [N n_g, (N + 1) n_g): epoch = old / n_g = N, whatever the
 * order in which the workgroups start or finish, and also after a launch that ended early.
 * Waits are bounded: on expiry the error word is set and the workgroup returns; the error word
 * stays set until mono_workspace_init. Fault injection: workgroup fault_wg withholds its values
 * at fault_phase. */

__device__ __forceinline__ uint64_t* start_counter(const Params& p, int group) {
  return reinterpret_cast<uint64_t*>(p.ctl + CTL_START64 + group * kStartStride);
}

__device__ __forceinline__ void report_timeout(const Params& p, int phase) {
  uint32_t* e = p.ctl + CTL_ERR;
  if (atomicCAS(&e[0], 0u, 1u) == 0u) {
    st_coh(&e[1], (uint32_t)phase);
    st_coh(&e[2], (uint32_t)blockIdx.x);
  }
  atomicAdd(&e[3], 1u);
}

/* Takes this workgroup's place in the launch (the epoch, above) and reads the debug words, once
 * per launch (made visible to the workgroup by the next __syncthreads). */
__device__ __forceinline__ void bar_setup(const Params& p, Smem& sm) {
  if (threadIdx.x == 0) {
    const uint32_t g = blockIdx.x % kBarGroups;
    const uint64_t n = ((uint64_t)gridDim.x - g + kBarGroups - 1) / kBarGroups;
    const uint64_t old = __hip_atomic_fetch_add(start_counter(p, (int)g), (uint64_t)1,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.epoch = old / n;
    sm.trace_on = ld_coh(p.ctl + CTL_TRACE) != 0u;
    const uint32_t spin = ld_coh(p.ctl + CTL_SPIN);
    const uint32_t fwg = ld_coh(p.ctl + CTL_FAULT_WG), fph = ld_coh(p.ctl + CTL_FAULT_PHASE);
    sm.spin = spin ? spin : kDefaultSpin;
    sm.skip_phase = (int32_t)fwg == (int32_t)blockIdx.x ? (int)fph : -1;
  }
}

/* Last-arriver election of a plain (non-persistent) launch: one counter that every launch
 * advances by exactly its grid size, so the arrival that makes it a multiple of the grid size
 * is the last of this launch. All threads get the answer. */
__device__ __forceinline__ bool arrive_last_single(const Params& p, Smem& sm) {
  drain();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint64_t a = __hip_atomic_fetch_add(reinterpret_cast<uint64_t*>(p.ctl + CTL_XEND64),
                                              (uint64_t)1, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    sm.flag = ((a + 1) % gridDim.x) == 0 ? 1 : 0;
  }
  __syncthreads();
  return sm.flag != 0;
}

__device__ __forceinline__ void stamp(const Params& p, bool on, int slot, int thread = 0) {
  if (on && (int)threadIdx.x == thread)
    p.trace[(size_t)blockIdx.x * kTraceSlots + slot] = __builtin_amdgcn_s_memrealtime();
}

/* Race shaker (debug mode; off unless mono_workspace_set_jitter set a nonzero limit for the
 * workspace): this wave waits a pseudo-random number of real-time ticks below p.jitter (at most
 * MONO_JITTER_MAX_TICKS), drawn from the seed, the launch epoch, the workgroup, the wave and
 * `salt` through the lowbias32 integer hash (C. Wellons). The delays at the phase boundaries
 * reorder both the workgroups' publications and the waves' task claims inside a workgroup. The
 * results of a launch do not depend on the timing of its waves, so any difference under the
 * shaker is a race. Off, it costs a test of a kernel argument per boundary (none inside the
 * task loops). */
__device__ __forceinline__ void shake(const Params& p, const Smem& sm, uint32_t salt) {
  if (p.jitter == 0u) return;
  const uint32_t J = p.jitter < MONO_JITTER_MAX_TICKS ? p.jitter : MONO_JITTER_MAX_TICKS;
  uint32_t h = p.jseed + 0x9E3779B9u * (uint32_t)(sm.epoch + 1) + 0x85EBCA6Bu * blockIdx.x +
               0xC2B2AE35u * (threadIdx.x >> 6) + 0x27D4EB2Fu * salt;
  h ^= h >> 16;
  h *= 0x7FEB352Du;
  h ^= h >> 15;
  h *= 0x846CA68Bu;
  h ^= h >> 16;
  h = __builtin_amdgcn_readfirstlane(h);
  const uint64_t d = h % J, t0 = __builtin_amdgcn_s_memrealtime();
  while (__builtin_amdgcn_s_memrealtime() - t0 < d) __builtin_amdgcn_s_sleep(4);
}

/* Task order for phases with fewer tasks than waves: consecutive tasks go to different compute
 * units first (task t -> workgroup t % G, wave t / G). */
__device__ __forceinline__ int wave_major_id() {
  return (threadIdx.x >> 6) * gridDim.x + blockIdx.x;
}

/* ------------------------------------------------------------------------------------------
 * Phase: mix partials [ds4 HC fusion commit: rms_norm_mix over the 4 x H row; SGLang fused
 * post/pre page: pre-norm GEMM partials + RMS square-sum partials]. Chunk t (256 consecutive
 * elements of the flattened row) is one wave task: part[t][r][j] = W_mix[j] . s over the chunk,
 * part[t][r][24] = sum s^2 over the chunk. */
template <int ACT, int RMAX>
__device__ __forceinline__ void ph_mix_partials(const Params& p, uint32_t tag, bool skip) {
  const int n = 4 * p.H, nch = (n + kMixChunk - 1) / kMixChunk;
  const int lane = threadIdx.x & 63;
  const int nwt = gridDim.x * kWaves;
  /* task = (chunk, row, group of kMixGroup outputs; the last group also takes the sum of
   * squares), so a wave loads kMixGroup weight rows and reduces at most kMixGroup + 1 sums.
   * A lane takes positions base + 256 h + 0..3 for the halves h of the chunk that exist (n is a
   * multiple of 256, so the last chunk may have one half only) */
  constexpr int NG = kNMix / kMixGroup, NH = kMixChunk / 256;
  for (int t = wave_major_id(); t < nch * p.R * NG; t += nwt) {
    const int g = t % NG, ch = t / NG / p.R, r = t / NG % p.R;
    const int base = ch * kMixChunk + lane * 4;
    float4 w[NH][kMixGroup];
    float s[NH][4];
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const int b = base + 256 * h;
      const bool in = ch * kMixChunk + 256 * h < n; /* uniform */
#pragma unroll
      for (int j = 0; j < kMixGroup; ++j)
        w[h][j] = in ? *reinterpret_cast<const float4*>(p.w_mix + (size_t)(g * kMixGroup + j) * n + b)
                     : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      if (!in) {
        s[h][0] = s[h][1] = s[h][2] = s[h][3] = 0.0f;
      } else if (ACT == F32) {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(p.state) +
                                                          (size_t)r * n + b);
        s[h][0] = v.x; s[h][1] = v.y; s[h][2] = v.z; s[h][3] = v.w;
      } else {
        const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.state) +
                                                        (size_t)r * n + b);
        s[h][0] = bf2f(v.x & 0xFFFFu); s[h][1] = bf2f(v.x >> 16);
        s[h][2] = bf2f(v.y & 0xFFFFu); s[h][3] = bf2f(v.y >> 16);
      }
    }
    uint64_t* out = p.mix_part + ((size_t)ch * p.R + r) * kNCarry;
#pragma unroll
    for (int j = 0; j < kMixGroup; ++j) {
      float a = 0.0f;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        a = fmaf(w[h][j].x, s[h][0], a);
        a = fmaf(w[h][j].y, s[h][1], a);
        a = fmaf(w[h][j].z, s[h][2], a);
        a = fmaf(w[h][j].w, s[h][3], a);
      }
      const float tot = wave_sum(a);
      if (lane == 0 && !skip)
        st_coh(out + g * kMixGroup + j, ((uint64_t)tag << 32) | __float_as_uint(tot));
    }
    if (g != NG - 1) continue;
    float ss = 0.0f;
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      ss = fmaf(s[h][0], s[h][0], ss);
      ss = fmaf(s[h][1], s[h][1], ss);
      ss = fmaf(s[h][2], s[h][2], ss);
      ss = fmaf(s[h][3], s[h][3], ss);
    }
    const float tot = wave_sum(ss);
    if (lane == 0 && !skip) st_coh(out + kNMix, ((uint64_t)tag << 32) | __float_as_uint(tot));
  }
}

/* ------------------------------------------------------------------------------------------
 * Prologue of the pre side: hc parameters and the norm weight into LDS (the norm weight sits
 * after the R activation rows in sm.big). */
template <int ACT>
__device__ __forceinline__ void load_pre_params(const Params& p, Smem& sm, int t0 = 0) {
  const int tid = threadIdx.x;
  if (tid < 3) sm.hcs[tid] = p.hc_scale[tid];
  if (tid < kNMix) sm.hcb[tid] = p.hc_base[tid];
  const size_t ab = ACT == F32 ? 4 : 2;
  const size_t rows = (size_t)p.R * p.H * ab, wbytes = (size_t)p.H * ab;
  const uint4* s = static_cast<const uint4*>(p.w_norm);
  uint4* d = reinterpret_cast<uint4*>(sm.big + rows);
  /* the copies run on threads t0 .. kBlock - 1 */
  const int ct = tid - t0, nt = kBlock - t0;
  if (ct < 0) {
    if (tid == 0) sm.state_in_lds = rows + wbytes + 4 * rows <= (size_t)kLdsActBytes ? 1 : 0;
    return;
  }
  for (size_t i = ct; i < wbytes / 16; i += nt) d[i] = s[i];
  /* the state rows too when they fit after the norm weight (one row does: 40 KB at H 5120) */
  const size_t sbytes = 4 * rows;
  const bool fits = rows + wbytes + sbytes <= (size_t)kLdsActBytes;
  if (fits) {
    const uint4* ss = static_cast<const uint4*>(p.state);
    uint4* sd = reinterpret_cast<uint4*>(sm.big + rows + wbytes);
    for (size_t i = ct; i < sbytes / 16; i += nt) sd[i] = ss[i];
  }
  if (ct == 0) sm.state_in_lds = fits ? 1 : 0;
}

/* When the state rows do not fit in LDS, the collapse of every workgroup reads the whole state
 * from memory. While the mix partials of the other workgroups are still on their way, each
 * workgroup touches its 1/32 share of the state (its rank among the workgroups w with the same
 * w % 8, which run on one XCD and share its L2), so that the collapse finds the state in L2. */
template <int ACT>
__device__ __forceinline__ void warm_state(const Params& p, const Smem& sm) {
  if (sm.state_in_lds) return;
  const size_t n16 = (size_t)p.R * 4 * p.H * (ACT == F32 ? 4 : 2) / 16;
  const int ranks = ((int)gridDim.x + kBarGroups - 1) / kBarGroups;
  const int rank = (int)blockIdx.x / kBarGroups;
  const size_t per = (n16 + ranks - 1) / ranks, i0 = rank * per;
  const size_t i1 = i0 + per < n16 ? i0 + per : n16;
  uint32_t acc = 0;
  for (size_t i = i0 + threadIdx.x; i < i1; i += kBlock)
    acc ^= static_cast<const uint4*>(p.state)[i].x;
  asm volatile("" ::"v"(acc)); /* the loads are issued and complete here; the value is unused */
}

/* Router bias into LDS (read by the select of every workgroup). */
__device__ __forceinline__ void load_bias(const Params& p, Smem& sm) {
  for (int e = threadIdx.x; e < p.E; e += kBlock) sm.bias[e] = p.bias[e];
}

/* ------------------------------------------------------------------------------------------
 * Phase: mHC pre side for all rows, run by one whole workgroup (redundantly by every
 * workgroup of the fused launch): mixes from the partials (or the carry); split / Sinkhorn;
 * collapse; weighted RMSNorm. The norm rows are left in sm.big as act values.
 * READING (mHC, not on the pages): pre = sigmoid(a0 m[i] + b[i]); post = 2 sigmoid(a1 m[4+i]
 * + b[4+i]); comb = Sinkhorn on exp(a2 m[8+4i+j] + b[8+4i+j] - max), rows then columns.
 * Needs load_pre_params first (and a __syncthreads between). */
template <int ACT, int RMAX>
__device__ __forceinline__ bool ph_hc_pre(const Params& p, Smem& sm, bool write_out, bool check,
                                          uint32_t tag) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = p.R, H = p.H, n = 4 * H, nch = (n + kMixChunk - 1) / kMixChunk;
  constexpr int VE = ACT == F32 ? 4 : 8; /* elements per 16-byte state load */
  const size_t ab = ACT == F32 ? 4 : 2;
  /* raw mix sums: the tagged partials [chunk][row][25] are copied into LDS with contiguous
   * 16-byte coherent loads (in the fused launch once their tags are current: no grid barrier),
   * then summed per (row, output) */
  float* part = reinterpret_cast<float*>(sm.big); /* free until x is written below */
  if (!p.carry_in) {
    /* one round of loads per thread when it covers every pair (up to 8 rows at H 5120) */
    const int np = nch * R * kNCarry;
    const bool got =
        np <= 2 * 8 * kBlock
            ? coh_copy_tagged_to_lds<8>(p.mix_part, np, part, check, tag, sm.spin, &sm.flag)
            : coh_copy_tagged_to_lds<16>(p.mix_part, np, part, check, tag, sm.spin, &sm.flag);
    if (!got) {
      if (threadIdx.x == 0) report_timeout(p, PH_MIX);
      return false;
    }
  }
  __syncthreads();
  if constexpr (RMAX == 1) {
    /* one row: a wave per output, lanes taking chunks t = lane + 64 m */
    for (int q = wave; q < R * kNCarry; q += kWaves) {
      const int r = q / kNCarry, j = q % kNCarry;
      float v = 0.0f;
      if (p.carry_in) {
        if (lane == 0) v = p.carry_in[r * kNCarry + j];
      } else {
        for (int t = lane; t < nch; t += 64) v += part[((size_t)t * R + r) * kNCarry + j];
      }
      const float tot = wave_sum(v);
      if (lane == 0) sm.raw[r][j] = tot;
    }
  } else {
    /* several rows: a thread per (row, output), summing the chunks in chunk order (the
     * 150-200 sums run side by side instead of 19-25 wave reductions one after another) */
    for (int q = tid; q < R * kNCarry; q += kBlock) {
      const int r = q / kNCarry, j = q % kNCarry;
      float v = 0.0f;
      if (p.carry_in) {
        v = p.carry_in[r * kNCarry + j];
      } else {
        for (int t = 0; t < nch; ++t) v += part[(size_t)t * R * kNCarry + q];
      }
      sm.raw[r][j] = v;
    }
  }
  __syncthreads();
  stamp(p, sm.trace_on != 0, 14);
  if (tid < R * kNMix) {
    const int r = tid / kNMix, j = tid % kNMix;
    const float den = sqrtf(sm.raw[r][kNMix] / (float)n + p.eps_hc);
    const float m = sm.raw[r][j] / den;
    sm.mixes[r][j] = m;
    if (write_out && p.mixes) p.mixes[r * kNMix + j] = m;
  }
  __syncthreads();
  stamp(p, sm.trace_on != 0, 15);
  /* pre / post gates: one thread each */
  if (tid < R * 8) {
    const int r = tid >> 3, g = tid & 7;
    const float* m = sm.mixes[r];
    if (g < 4) {
      const float v = 1.0f / (1.0f + expf(-(sm.hcs[0] * m[g] + sm.hcb[g])));
      sm.pre[r][g] = v;
      if (write_out) p.pre[r * 4 + g] = v;
    } else {
      const int i = g - 4;
      const float v = 2.0f / (1.0f + expf(-(sm.hcs[1] * m[4 + i] + sm.hcb[4 + i])));
      sm.post[r][i] = v;
      if (write_out) p.post[r * 4 + i] = v;
    }
  }
  __syncthreads();
  stamp(p, sm.trace_on != 0, 16);
  /* collapse: x = bf16(sum_i pre_i state_i), in chunks of VE consecutive positions with
   * 16-byte loads of the four streams, and the sum of squares of the rounded x */
  if constexpr (RMAX == 1) {
    /* one row: one thread per chunk; sums of squares per wave, then in wave order */
    float ss[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) ss[r] = 0.0f;
    constexpr int RB = 1;
    for (int c = tid; c < H / VE; c += kBlock) {
#pragma unroll
      for (int r0 = 0; r0 < RMAX; r0 += RB) {
        if (r0 >= R) break;
        uint4 sv[RB][4];
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
          if (r0 + rr >= R) break;
          const uint8_t* sbase = sm.state_in_lds
                                     ? sm.big + ((size_t)R + 1) * H * ab
                                     : static_cast<const uint8_t*>(p.state);
          const uint8_t* base = sbase + ((size_t)(r0 + rr) * n + (size_t)c * VE) * ab;
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sv[rr][i] = *reinterpret_cast<const uint4*>(base + (size_t)i * H * ab);
        }
#pragma unroll
        for (int rr = 0; rr < RB; ++rr) {
          const int r = r0 + rr;
          if (r >= R) break;
          const float p0 = sm.pre[r][0], p1 = sm.pre[r][1], p2 = sm.pre[r][2], p3 = sm.pre[r][3];
          const uint32_t a0[4] = {sv[rr][0].x, sv[rr][0].y, sv[rr][0].z, sv[rr][0].w};
          const uint32_t a1[4] = {sv[rr][1].x, sv[rr][1].y, sv[rr][1].z, sv[rr][1].w};
          const uint32_t a2[4] = {sv[rr][2].x, sv[rr][2].y, sv[rr][2].z, sv[rr][2].w};
          const uint32_t a3[4] = {sv[rr][3].x, sv[rr][3].y, sv[rr][3].z, sv[rr][3].w};
          uint32_t xo[4];
          float xf[2];
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            float v0, v1, v2, v3;
            if (ACT == F32) {
              v0 = __uint_as_float(a0[e]); v1 = __uint_as_float(a1[e]);
              v2 = __uint_as_float(a2[e]); v3 = __uint_as_float(a3[e]);
            } else {
              const int sh = (e & 1) ? 16 : 0;
              v0 = bf2f((a0[e >> 1] >> sh) & 0xFFFFu); v1 = bf2f((a1[e >> 1] >> sh) & 0xFFFFu);
              v2 = bf2f((a2[e >> 1] >> sh) & 0xFFFFu); v3 = bf2f((a3[e >> 1] >> sh) & 0xFFFFu);
            }
            float a = p0 * v0;
            a = fmaf(p1, v1, a);
            a = fmaf(p2, v2, a);
            a = fmaf(p3, v3, a);
            if (ACT == F32) {
              xo[e] = __float_as_uint(a);
              ss[r] = fmaf(a, a, ss[r]);
            } else {
              xf[e & 1] = a;
              if (e & 1) {
                const uint32_t pr = f2bf2(xf[0], xf[1]);
                xo[e >> 1] = pr;
                const float x0 = bf2f(pr & 0xFFFFu), x1 = bf2f(pr >> 16);
                ss[r] = fmaf(x0, x0, ss[r]);
                ss[r] = fmaf(x1, x1, ss[r]);
              }
            }
          }
          const uint4 xv = make_uint4(xo[0], xo[1], xo[2], xo[3]);
          const size_t byte = ((size_t)r * H + (size_t)c * VE) * ab;
          *reinterpret_cast<uint4*>(sm.big + byte) = xv;
          if (write_out && p.x) *reinterpret_cast<uint4*>(static_cast<uint8_t*>(p.x) + byte) = xv;
        }
      }
    }
    stamp(p, sm.trace_on != 0, 17);
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r >= R) break;
      const float t = wave_sum(ss[r]);
      if (lane == 0) sm.red[wave][r] = t;
    }
    __syncthreads();
    if (tid < R) {
      float t = 0.0f;
      for (int w = 0; w < kWaves; ++w) t += sm.red[w][tid];
      sm.rsum[tid] = t;
    }
    __syncthreads();
  } else {
    /* several rows: kBlock / R threads per row, each taking chunks of its row with CB chunks'
     * loads in flight at once (every thread has at most two rounds at H 5120); sums of squares
     * per thread, then per row in thread order */
    {
      const int tpr = kBlock / R, r = tid / tpr, lt = tid % tpr, nchunk = H / VE;
      constexpr int CB = 5;
      float ss = 0.0f;
      if (r < R) {
        const uint8_t* sbase = sm.state_in_lds ? sm.big + ((size_t)R + 1) * H * ab
                                               : static_cast<const uint8_t*>(p.state);
        const float p0 = sm.pre[r][0], p1 = sm.pre[r][1], p2 = sm.pre[r][2], p3 = sm.pre[r][3];
        for (int c0 = lt; c0 < nchunk; c0 += CB * tpr) {
          uint4 sv[CB][4];
#pragma unroll
          for (int b = 0; b < CB; ++b) {
            const int c = c0 + b * tpr, cc = c < nchunk ? c : nchunk - 1; /* cc: unused repeat */
            const uint8_t* base = sbase + ((size_t)r * n + (size_t)cc * VE) * ab;
#pragma unroll
            for (int i = 0; i < 4; ++i)
              sv[b][i] = *reinterpret_cast<const uint4*>(base + (size_t)i * H * ab);
          }
#pragma unroll
          for (int b = 0; b < CB; ++b) {
            const int c = c0 + b * tpr;
            if (c >= nchunk) break;
            const uint32_t a0[4] = {sv[b][0].x, sv[b][0].y, sv[b][0].z, sv[b][0].w};
            const uint32_t a1[4] = {sv[b][1].x, sv[b][1].y, sv[b][1].z, sv[b][1].w};
            const uint32_t a2[4] = {sv[b][2].x, sv[b][2].y, sv[b][2].z, sv[b][2].w};
            const uint32_t a3[4] = {sv[b][3].x, sv[b][3].y, sv[b][3].z, sv[b][3].w};
            uint32_t xo[4];
            float xf[2];
#pragma unroll
            for (int e = 0; e < VE; ++e) {
              float v0, v1, v2, v3;
              if (ACT == F32) {
                v0 = __uint_as_float(a0[e]); v1 = __uint_as_float(a1[e]);
                v2 = __uint_as_float(a2[e]); v3 = __uint_as_float(a3[e]);
              } else {
                const int sh = (e & 1) ? 16 : 0;
                v0 = bf2f((a0[e >> 1] >> sh) & 0xFFFFu); v1 = bf2f((a1[e >> 1] >> sh) & 0xFFFFu);
                v2 = bf2f((a2[e >> 1] >> sh) & 0xFFFFu); v3 = bf2f((a3[e >> 1] >> sh) & 0xFFFFu);
              }
              float a = p0 * v0;
              a = fmaf(p1, v1, a);
              a = fmaf(p2, v2, a);
              a = fmaf(p3, v3, a);
              if (ACT == F32) {
                xo[e] = __float_as_uint(a);
                ss = fmaf(a, a, ss);
              } else {
                xf[e & 1] = a;
                if (e & 1) {
                  const uint32_t pr = f2bf2(xf[0], xf[1]);
                  xo[e >> 1] = pr;
                  const float x0 = bf2f(pr & 0xFFFFu), x1 = bf2f(pr >> 16);
                  ss = fmaf(x0, x0, ss);
                  ss = fmaf(x1, x1, ss);
                }
              }
            }
            const uint4 xv = make_uint4(xo[0], xo[1], xo[2], xo[3]);
            const size_t byte = ((size_t)r * H + (size_t)c * VE) * ab;
            *reinterpret_cast<uint4*>(sm.big + byte) = xv;
            if (write_out && p.x) *reinterpret_cast<uint4*>(static_cast<uint8_t*>(p.x) + byte) = xv;
          }
        }
      }
      stamp(p, sm.trace_on != 0, 17);
      static_assert(kNMix * 4 * kSliceMax >= kBlock, "one sum per thread");
      float* ssp = sm.wnext; /* free until the slice is loaded for the expand */
      ssp[tid] = ss;
      __syncthreads();
      for (int q = wave; q < R; q += kWaves) {
        float t = 0.0f;
        for (int i = lane; i < tpr; i += 64) t += ssp[q * tpr + i];
        t = wave_sum(t);
        if (lane == 0) sm.rsum[q] = t;
      }
      __syncthreads();
    }
  }
  stamp(p, sm.trace_on != 0, 18);
  /* weighted RMSNorm: norm = bf16(x * (1 / sqrt(mean(x^2) + eps)) * w), VE positions per
   * thread */
  const uint8_t* wn = sm.big + (size_t)R * H * ab;
  for (int r = 0; r < R; ++r) {
    const float inv = 1.0f / sqrtf(sm.rsum[r] / (float)H + p.eps_norm);
    for (int c = tid; c < H / VE; c += kBlock) {
      const size_t byte = ((size_t)r * H + (size_t)c * VE) * ab;
      const uint4 xv = *reinterpret_cast<const uint4*>(sm.big + byte);
      const uint4 wv = *reinterpret_cast<const uint4*>(wn + (size_t)c * VE * ab);
      const uint32_t xa[4] = {xv.x, xv.y, xv.z, xv.w}, wa[4] = {wv.x, wv.y, wv.z, wv.w};
      uint32_t o[4];
      float vf = 0.0f;
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        float xb, w;
        if (ACT == F32) {
          xb = __uint_as_float(xa[e]);
          w = __uint_as_float(wa[e]);
        } else {
          const int sh = (e & 1) ? 16 : 0;
          xb = bf2f((xa[e >> 1] >> sh) & 0xFFFFu);
          w = bf2f((wa[e >> 1] >> sh) & 0xFFFFu);
        }
        const float v = xb * inv * w;
        if (ACT == F32)
          o[e] = __float_as_uint(v);
        else if (e & 1)
          o[e >> 1] = f2bf2(vf, v);
        else
          vf = v;
      }
      const uint4 ov = make_uint4(o[0], o[1], o[2], o[3]);
      *reinterpret_cast<uint4*>(sm.big + byte) = ov;
      if (write_out) *reinterpret_cast<uint4*>(static_cast<uint8_t*>(p.norm) + byte) = ov;
    }
  }
  __syncthreads();
  return true;
}

/* comb = Sinkhorn(exp(a2 m[8 + 4 i + j] + b[8 + 4 i + j] - max)) for every row, run by waves
 * 0 .. (R + 3) / 4 - 1 with no workgroup barrier (comb is first read by the expand). Needs the
 * mixes in LDS. */
__device__ __forceinline__ void ph_sinkhorn(const Params& p, Smem& sm, bool write_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, R = p.R;
  /* Sinkhorn: 16 lanes per row hold M[i][j] at lane 16 (r % 4) + 4 i + j; row sums with quad
   * butterflies, column sums with two rotations inside the 16-lane row (each lane associates
   * its column sum in its own fixed order); each normalisation multiplies by the hardware
   * reciprocal of the sum */
  if (wave < (R + 3) / 4) {
    const int r = wave * 4 + (lane >> 4), q = lane & 15;
    const bool live = r < R;
    const float* m = sm.mixes[live ? r : 0];
    const float L = sm.hcs[2] * m[8 + q] + sm.hcb[8 + q];
    float mx = fmaxf(L, dpp<0xB1>(L));
    mx = fmaxf(mx, dpp<0x4E>(mx));
    mx = fmaxf(mx, dpp<0x124>(mx)); /* row_ror:4 */
    mx = fmaxf(mx, dpp<0x128>(mx)); /* row_ror:8 */
    float M = expf(L - mx);
    for (int it = 0; it < p.iters; ++it) {
      float rs = M + dpp<0xB1>(M);
      rs = rs + dpp<0x4E>(rs);
      M = M * __builtin_amdgcn_rcpf(rs);
      float cs = M + dpp<0x124>(M);
      cs = cs + dpp<0x128>(cs);
      M = M * __builtin_amdgcn_rcpf(cs);
    }
    if (live) {
      sm.comb[r][q] = M;
      if (write_out) p.comb[r * 16 + q] = M;
    }
  }
}

/* Copies R act rows [R][H] from global memory into sm.big. */
template <int ACT>
__device__ __forceinline__ void load_act_rows(const void* src, int R, int H, Smem& sm) {
  const size_t bytes = (size_t)R * H * (ACT == F32 ? 4 : 2);
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(sm.big);
  for (size_t i = threadIdx.x; i < bytes / 16; i += kBlock) d[i] = s[i];
  __syncthreads();
}

template <int ACT, int RMAX>
__device__ __forceinline__ void act_rows_ptrs(const Params& p, const Smem& sm,
                                              const void* (&arow)[RMAX]) {
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
    arow[r] = sm.big + (size_t)(r < p.R ? r : 0) * p.H * (ACT == F32 ? 4 : 2);
}

/* MXFP8 round trip, in place, of the R bf16 activation rows at the start of sm.big (blocks of 32
 * along H, one per thread at a time). Whole workgroup; the caller places the barriers. */
template <int ACT>
__device__ __forceinline__ void mx8_act_rows(const Params& p, Smem& sm) {
  if constexpr (ACT == BF16) {
    const int nb = p.R * p.H / 32;
    for (int b = threadIdx.x; b < nb; b += kBlock) mx8_block_lds(sm.big + (size_t)b * 64);
  }
}

/* ------------------------------------------------------------------------------------------
 * Phase: router logits [ds4 router commit: the F32 logits matvec]. One wave per expert row,
 * rows spread over compute units first; the fused launch loads each wave's first row before
 * it gathers the mix partials. */
typedef WRegs<F32, 1, kRouterCh> RouterRegs;

/* Router task of this wave. A row of H values has nsteps steps of 256 values. When
 * ceil(E / grid) <= 7 and each expert's steps fit kRouterCh per wave over its share of the
 * waves 1 .. 7, expert e goes to workgroup e % grid and its steps are spread over those waves
 * (local): every wave adds up its steps, the workgroup sums the wave parts in wave order and
 * stores one tagged logit per (row, expert). Otherwise each wave walks whole rows
 * e = wave_major_id() + n * waves in chunks of kRouterCh steps. In the local case wave 0 has no
 * steps, so its polls do not queue behind early loads. */
struct RouterTask {
  bool local;
  int per, nw; /* local: experts per workgroup, waves per expert */
  int e, s0, cnt;
};

__device__ __forceinline__ RouterTask router_task(const Params& p) {
  RouterTask t;
  const int nsteps = (p.H + 255) / 256;
  t.per = (p.E + (int)gridDim.x - 1) / (int)gridDim.x;
  t.nw = t.per <= kWaves - 1 ? (kWaves - 1) / t.per : 1;
  const int spw = (nsteps + t.nw - 1) / t.nw;
  t.local = t.per <= kWaves - 1 && spw <= kRouterCh;
  const int wave = threadIdx.x >> 6;
  if (t.local) {
    const int j = (wave - 1) / t.nw, sub = (wave - 1) % t.nw;
    t.e = wave > 0 && j < t.per ? (int)blockIdx.x + j * (int)gridDim.x : p.E;
    t.s0 = wave > 0 ? sub * spw : 0;
    t.cnt = wave > 0 ? max(0, min(spw, nsteps - t.s0)) : 0;
  } else {
    t.e = wave_major_id();
    t.s0 = 0;
    t.cnt = min(kRouterCh, nsteps);
  }
  return t;
}

/* Loads steps s0 .. s0 + cnt - 1 (cnt <= kRouterCh) of f32 router row e; the other registers
 * are zero. */
__device__ __forceinline__ void router_load(const Params& p, int e, int s0, int cnt, RouterRegs& W) {
  const int lane = threadIdx.x & 63;
  const uint4* row = reinterpret_cast<const uint4*>(p.w_router + (size_t)e * p.H);
#pragma unroll
  for (int c = 0; c < kRouterCh; ++c) {
    const int q = (s0 + c) * 64 + lane; /* 16-byte unit: f32 values 4 q .. 4 q + 3 */
    W.v[0][c] = c < cnt && q * 4 < p.H ? row[q] : make_uint4(0, 0, 0, 0);
    W.sc[0][c] = 0;
  }
}

/* Issues the loads of this wave's first router chunk (the task order of ph_router). */
__device__ __forceinline__ void router_prefetch(const Params& p, RouterRegs& W) {
  const RouterTask t = router_task(p);
  if (t.e < p.E) router_load(p, t.e, t.s0, t.cnt, W);
}

/* acc[r] += steps s0 .. s0 + cnt - 1 of one f32 router row (in W) . act row r. Values past H
 * are zero in W and read a valid act address. */
template <int ACT, int RMAX>
__device__ __forceinline__ void router_dot(const RouterRegs& W, int s0, int cnt, int H,
                                           const void* const (&arow)[RMAX], uint32_t mask,
                                           float (&acc)[RMAX]) {
  constexpr int EL = 4;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int c = 0; c < kRouterCh; ++c) {
    if (c >= cnt) break;
    const int k = min(((s0 + c) * 64 + lane) * EL, H - EL);
    const float w0 = __uint_as_float(W.v[0][c].x), w1 = __uint_as_float(W.v[0][c].y);
    const float w2 = __uint_as_float(W.v[0][c].z), w3 = __uint_as_float(W.v[0][c].w);
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (RMAX > 1 && !(mask & (1u << r))) continue;
      float x0, x1, x2, x3;
      if constexpr (ACT == F32) {
        const float4 x = *reinterpret_cast<const float4*>(static_cast<const float*>(arow[r]) + k);
        x0 = x.x; x1 = x.y; x2 = x.z; x3 = x.w;
      } else {
        const uint2 x = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(arow[r]) + k);
        x0 = bf2f(x.x & 0xFFFFu); x1 = bf2f(x.x >> 16);
        x2 = bf2f(x.y & 0xFFFFu); x3 = bf2f(x.y >> 16);
      }
      float a = acc[r];
      a = fmaf(w0, x0, a);
      a = fmaf(w1, x1, a);
      a = fmaf(w2, x2, a);
      a = fmaf(w3, x3, a);
      acc[r] = a;
    }
  }
}

/* Tagged store of one router logit: value bits in the low word, tag in the high word. */
__device__ __forceinline__ void store_logit(const Params& p, int r, int e, float v, uint32_t tag) {
  st_coh(p.lgp + (size_t)r * p.E + e, ((uint64_t)tag << 32) | __float_as_uint(v));
}

/* Every expert's logit is stored once per row as a tagged value (tag = the launch epoch + 1 in
 * the fused launch, 0 otherwise); the select waits for the tags, so no grid barrier separates
 * the router from the select. The sum over a row has a fixed order (steps in a wave, then
 * waves in order), so every reader sees the same logits. In the local case every wave of the
 * workgroup passes one __syncthreads here. With skip (fault injection) nothing is stored. */
template <int ACT, int RMAX, bool PRE>
__device__ __forceinline__ void ph_router(const Params& p, Smem& sm, const RouterRegs& pre,
                                          uint32_t tag, bool skip) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, tid = threadIdx.x;
  const void* arow[RMAX];
  act_rows_ptrs<ACT, RMAX>(p, sm, arow);
  const uint32_t mask = (1u << p.R) - 1u;
  const int nsteps = (p.H + 255) / 256;
  const RouterTask t = router_task(p);
  /* the first router wave: wave 1 in the local case, else wave 0 */
  const int tw = t.local ? 64 : 0;
  stamp(p, sm.trace_on != 0, 22, tw);
  if (t.local) {
    float acc[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) acc[r] = 0.0f;
    if (t.e < p.E) {
      if (PRE) {
        router_dot<ACT, RMAX>(pre, t.s0, t.cnt, p.H, arow, mask, acc);
      } else {
        RouterRegs W;
        router_load(p, t.e, t.s0, t.cnt, W);
        router_dot<ACT, RMAX>(W, t.s0, t.cnt, p.H, arow, mask, acc);
      }
    }
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r >= p.R) break;
      const float v = wave_sum(acc[r]);
      if (lane == 0 && wave > 0) sm.red[wave][r] = v;
    }
    __syncthreads();
    /* thread (j, r) sums the parts of expert slot j, row r in wave order */
    if (tid < t.per * p.R) {
      const int j = tid / p.R, r = tid % p.R, e = (int)blockIdx.x + j * (int)gridDim.x;
      if (e < p.E) {
        float v = 0.0f;
        for (int w = 1 + j * t.nw; w < 1 + (j + 1) * t.nw; ++w) v += sm.red[w][r];
        if (!skip) store_logit(p, r, e, v, tag);
      }
    }
    stamp(p, sm.trace_on != 0, 23, 0);
    return;
  }
  const int nwt = gridDim.x * kWaves;
  for (int e = wave_major_id(); e < p.E; e += nwt) {
    float acc[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) acc[r] = 0.0f;
    for (int s0 = 0; s0 < nsteps; s0 += kRouterCh) {
      const int cnt = min(kRouterCh, nsteps - s0);
      if (PRE && s0 == 0 && e == wave_major_id()) {
        router_dot<ACT, RMAX>(pre, 0, cnt, p.H, arow, mask, acc);
      } else {
        RouterRegs W;
        router_load(p, e, s0, cnt, W);
        router_dot<ACT, RMAX>(W, s0, cnt, p.H, arow, mask, acc);
      }
    }
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r >= p.R) break;
      const float v = wave_sum(acc[r]);
      if (lane == 0 && !skip) store_logit(p, r, e, v, tag);
    }
  }
}

/* ------------------------------------------------------------------------------------------
 * Phase: select, run by one whole workgroup for all rows [ds4 router commit: sqrt(softplus),
 * the bias, the canonical (score descending, index ascending) top-k, normalised weights, the
 * clamp, the row division and the scale as separately rounded ops; tie-order commit].
 * One wave per row; lane L holds experts L, L + 64, ... as 64-bit keys (ordered biased score in
 * the high word, complement of the index in the low word), so the largest key is the highest
 * score and, among equal scores, the smallest index; k rounds of a DPP wave maximum pick the
 * experts in canonical order. READING: the clamp floor is 2^-14; the bias steers selection
 * only (the weights gather the unbiased scores). */
__device__ __forceinline__ uint32_t ord_f32(float f) {
  if (f != f) return 0u; /* NaN ranks last */
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

/* softplus(z) = max(z, 0) + log1p(exp(-|z|)) in f32. log1p(t) for t in (0, 1] uses the
 * correction log(u) * t / (u - 1) with u = 1 + t rounded (exact where u == 1: log1p(t) = t to
 * f32 precision), which keeps the relative error near that of log. */
__device__ __forceinline__ float softplus_f32(float z) {
  const float t = expf(-fabsf(z));
  const float u = 1.0f + t;
  const float l = u == 1.0f ? t : __logf(u) * (t / (u - 1.0f));
  return fmaxf(z, 0.0f) + l;
}

/* Largest unsigned value over the wave, uniform. */
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u<0xB1>(v));
  v = max(v, dpp_u<0x4E>(v));
  v = max(v, dpp_u<0x141>(v));
  v = max(v, dpp_u<0x140>(v));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

/* Compare-exchange of two (hi, lo, s) entries so that entry a holds the larger key. */
__device__ __forceinline__ void key_cx(uint32_t& ah, uint32_t& al, float& as, uint32_t& bh,
                                       uint32_t& bl, float& bs) {
  const bool sw = bh > ah || (bh == ah && bl > al);
  const uint32_t th = sw ? bh : ah, tl = sw ? bl : al;
  const float ts = sw ? bs : as;
  bh = sw ? ah : bh;
  bl = sw ? al : bl;
  bs = sw ? as : bs;
  ah = th;
  al = tl;
  as = ts;
}

/* Top-k of one row by the 64-bit key (ord(s + bias) << 32) | ~e: biased score descending, then
 * expert index ascending [ds4 page, tie-order commit]. Each lane sorts its PER candidates once;
 * a round takes the largest head over the wave (high word, then low word among the lanes that
 * hold it) and the owning lane pops its head. */
/* Logits of row r for this lane's experts e = lane + 64 c. With check, waits (bounded) until
 * every one carries `tag`; returns false on expiry (uniform over the wave). */
template <int PER>
__device__ __forceinline__ bool gather_logits(const Params& p, const Smem& sm, int r, bool check,
                                              uint32_t tag, float (&z)[PER]) {
  const int lane = threadIdx.x & 63, E = p.E;
  const __amdgpu_buffer_rsrc_t lg = coh_region(p.lgp + (size_t)r * E, (size_t)E * 8);
  uint2 v[PER];
  bool need[PER];
  /* every load is issued (a valid repeated address when not needed), so all are in flight
   * together */
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int e = lane + 64 * c;
    need[c] = e < E;
    v[c] = coh_b64(lg, (uint32_t)(e < E ? e : E - 1) * 8u);
    if (!need[c]) v[c] = make_uint2(0u, tag);
  }
  bool ok = true;
  if (check) {
    auto pending = [&]() {
      bool any = false;
#pragma unroll
      for (int c = 0; c < PER; ++c) any |= need[c] && v[c].y != tag;
      return any;
    };
    if (__ballot(pending()) != 0ull) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__ballot(pending()) != 0ull) {
        __builtin_amdgcn_s_sleep(1);
#pragma unroll
        for (int c = 0; c < PER; ++c)
          if (need[c] && v[c].y != tag) v[c] = coh_b64(lg, (uint32_t)(lane + 64 * c) * 8u);
        if (__builtin_amdgcn_s_memrealtime() - t0 > sm.spin) {
          ok = false;
          break;
        }
      }
    }
  }
#pragma unroll
  for (int c = 0; c < PER; ++c) z[c] = need[c] ? __uint_as_float(v[c].x) : 0.0f;
  return ok;
}

/* Top-k of one row by the 64-bit key (ord(s + bias) << 32) | ~e: biased score descending, then
 * expert index ascending [ds4 page, tie-order commit]. Each lane sorts its PER candidates once;
 * a round takes the largest head over the wave (high word, then low word among the lanes that
 * hold it) and the owning lane pops its head. Returns false when the logits did not arrive. */
template <int PER>
__device__ __forceinline__ bool select_row(const Params& p, Smem& sm, int r, bool write_out,
                                           bool check, uint32_t tag, int& e_lane, float& s_lane) {
  const int lane = threadIdx.x & 63, E = p.E, K = p.K;
  uint32_t kh[PER], kl[PER];
  float sv[PER], zs[PER], bz[PER];
  /* the lane's biases, read from LDS while the logits are still in flight */
#pragma unroll
  for (int c = 0; c < PER; ++c) bz[c] = lane + 64 * c < E ? sm.bias[lane + 64 * c] : 0.0f;
  const bool gathered = gather_logits<PER>(p, sm, r, check, tag, zs);
  if (lane == 0) __hip_atomic_store(&sm.lg_ready, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  if (!gathered) return false;
  stamp(p, sm.trace_on != 0, 24);
#pragma unroll
  for (int c = 0; c < PER; ++c) {
    const int e = lane + 64 * c;
    kh[c] = 0u;
    kl[c] = 0u;
    sv[c] = 0.0f;
    if (e < E) {
      const float z = zs[c];
      if (write_out) p.logits[(size_t)r * E + e] = z;
      const float sc = sqrtf(softplus_f32(z));
      kh[c] = ord_f32(sc + bz[c]);
      kl[c] = 0xFFFFFFFFu - (uint32_t)e;
      sv[c] = sc;
    }
  }
  stamp(p, sm.trace_on != 0, 19);
  /* odd-even transposition sort, descending */
#pragma unroll
  for (int ph = 0; ph < PER; ++ph)
#pragma unroll
    for (int c = ph & 1; c + 1 < PER; c += 2)
      key_cx(kh[c], kl[c], sv[c], kh[c + 1], kl[c + 1], sv[c + 1]);
  for (int j = 0; j < K; ++j) {
    const uint32_t mh = wave_max_u32(kh[0]);
    /* the low word decides only between lanes that share the highest score */
    const uint64_t top = __ballot(kh[0] == mh);
    const uint32_t ml = __popcll(top) == 1
                            ? (uint32_t)__builtin_amdgcn_readlane((int)kl[0], (int)__builtin_ctzll(top))
                            : wave_max_u32(kh[0] == mh ? kl[0] : 0u);
    const bool win = kh[0] == mh && kl[0] == ml;
    const uint64_t who = __ballot(win);
    const float s_win = readlane(sv[0], (int)__builtin_ctzll(who));
    if (lane == 0) sm.sel_e[r][j] = (int)(0xFFFFFFFFu - ml);
    if (lane == j) { /* pick j also stays in lane j */
      e_lane = (int)(0xFFFFFFFFu - ml);
      s_lane = s_win;
    }
    if (win) {
#pragma unroll
      for (int c = 0; c + 1 < PER; ++c) {
        kh[c] = kh[c + 1];
        kl[c] = kl[c + 1];
        sv[c] = sv[c + 1];
      }
      kh[PER - 1] = 0u;
      kl[PER - 1] = 0u;
      sv[PER - 1] = 0.0f;
    }
  }
  return true;
}

/* Routing weights of row r by the wave that selected it, pick j in lane j (e_lane, s_lane):
 * sum = f32 sum of the picked scores in pick order, c = max(sum, 2^-14), w_j = (s_j / c) rho
 * [ds4 router commit: sum, clamp, divide and scale as separate rounded ops]. */
__device__ __forceinline__ void select_weights(const Params& p, Smem& sm, int r, int e_lane,
                                               float s_lane, bool write_out) {
  const int lane = threadIdx.x & 63, K = p.K;
  float sum = 0.0f;
  for (int j = 0; j < K; ++j) sum += readlane(s_lane, j);
  const float c = fmaxf(sum, 6.103515625e-05f); /* 2^-14 */
  if (lane < K) {
    const float w = (s_lane / c) * p.rho;
    sm.sel_w[r][lane] = w;
    if (write_out) {
      p.idx[r * K + lane] = e_lane;
      p.weights[r * K + lane] = w;
    }
  }
}

/* Select, part 1: waves 0 .. min(R, 8) - 1 take rows r = wave, wave + 8, ... Needs sm.sel_ok
 * set to 1 beforehand (made visible by a __syncthreads); no workgroup barrier inside, so other
 * waves may do independent work meanwhile. */
__device__ __forceinline__ void select_rows(const Params& p, Smem& sm, bool write_out, bool check,
                                            uint32_t tag) {
  const int wave = threadIdx.x >> 6;
  for (int r = wave; r < p.R; r += kWaves) {
    int e_l;
    float s_l;
    const bool ok = p.E <= 256 ? select_row<4>(p, sm, r, write_out, check, tag, e_l, s_l)
                               : select_row<kMaxExperts / 64>(p, sm, r, write_out, check, tag,
                                                              e_l, s_l);
    if (ok) select_weights(p, sm, r, e_l, s_l, write_out);
    if (!ok && (threadIdx.x & 63) == 0) sm.sel_ok = 0;
  }
}

/* Select, part 2 (after a __syncthreads that follows part 1; the weights are in sm.sel_w).
 * Returns false (after reporting once) when some row's logits did not arrive in time. */
__device__ __forceinline__ bool select_finish(const Params& p, Smem& sm, bool write_out) {
  (void)write_out;
  if (sm.sel_ok == 0) {
    if (threadIdx.x == 0) report_timeout(p, PH_ROUTER);
    return false;
  }
  __syncthreads();
  return true;
}

__device__ __forceinline__ bool ph_select(const Params& p, Smem& sm, bool write_out, bool check,
                                          uint32_t tag) {
  if (threadIdx.x == 0) sm.sel_ok = 1;
  __syncthreads();
  select_rows(p, sm, write_out, check, tag);
  __syncthreads();
  return select_finish(p, sm, write_out);
}

/* Reads a caller-provided selection (idx, weights) into sm.sel_*; indices are clamped into
 * [0, E) so a bad index cannot address outside the expert arrays. */
__device__ __forceinline__ void load_selection(const Params& p, Smem& sm) {
  const int tid = threadIdx.x;
  if (tid < p.R * p.K) {
    const int r = tid / p.K, j = tid % p.K;
    int e = p.idx_in[tid];
    e = e < 0 ? 0 : (e >= p.E ? p.E - 1 : e);
    sm.sel_e[r][j] = e;
    sm.sel_w[r][j] = p.w_in[tid];
  }
  __syncthreads();
}

/* Plan: the distinct selected experts in ascending order (each is streamed once for all the
 * rows that chose it), with the rows that use it and the slot j it fills in each row. Item nU
 * is the shared expert (every row). Built by wave 0 alone from a bitmap of the selected
 * experts (LDS operations of one wave complete in order); every wave sees it after the
 * __syncthreads at the end. */
/* One-row plan, by one wave: its k experts are distinct, so the plan is their ascending order;
 * lane q < k holds pick q (expert e_lane) and ranks it among them (the same result as the
 * bitmap walk of plan_wave). */
__device__ __forceinline__ void plan_one_row(const Params& p, Smem& sm, int e_lane) {
  {
    const int lane = threadIdx.x & 63, K = p.K;
    const int e = lane < K ? e_lane : 0x7FFFFFFF;
    int rank = 0;
    for (int t = 0; t < K; ++t) rank += __builtin_amdgcn_readlane(e, t) < e ? 1 : 0;
    for (int q = lane; q < (K + 1) * kMaxRows; q += 64) sm.uslot[q / kMaxRows][q % kMaxRows] = -1;
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup"); /* the -1s land before the slots */
    if (lane < K) {
      sm.U[rank] = e;
      sm.umask[rank] = 1u;
      sm.uslot[rank][0] = (int8_t)lane;
    }
    if (lane == 0) {
      sm.umask[K] = 1u;
      sm.uslot[K][0] = (int8_t)K;
      sm.nU = K;
    }
  }
}

/* One-row finish of the select in the fused launch, by wave 0 with pick j in lane j
 * (e_lane, s_lane): the weights, then the plan. */
__device__ __forceinline__ void finish_one_row(const Params& p, Smem& sm, int e_lane,
                                               float s_lane, bool write_out) {
  select_weights(p, sm, 0, e_lane, s_lane, write_out);
  plan_one_row(p, sm, e_lane);
}

__device__ __forceinline__ void plan_wave(const Params& p, Smem& sm) {
  if (p.R == 1) {
    const int lane = threadIdx.x & 63;
    plan_one_row(p, sm, lane < p.K ? sm.sel_e[0][lane] : 0);
    return;
  }
  {
    const int lane = threadIdx.x & 63, R = p.R, K = p.K, RK = p.R * p.K;
    constexpr int NW = kMaxExperts / 32;
    if (lane < NW) sm.ubits[lane] = 0u;
    for (int q = lane; q < RK; q += 64) {
      const int e = sm.sel_e[q / K][q % K];
      atomicOr(&sm.ubits[e >> 5], 1u << (e & 31));
    }
    uint32_t w = lane < NW ? sm.ubits[lane] : 0u;
    const int c = __popc(w);
    int incl = c;
#pragma unroll
    for (int d = 1; d < NW; d <<= 1) {
      const int t = __shfl_up(incl, d);
      if (lane >= d) incl += t;
    }
    const int base = incl - c;
    const int nU = __shfl(incl, NW - 1);
    if (lane < NW) {
      sm.ubase[lane] = base;
      int k = base;
      while (w) {
        sm.U[k++] = lane * 32 + (__ffs(w) - 1);
        w &= w - 1u;
      }
    }
    for (int q = lane; q < (nU + 1) * kMaxRows; q += 64) sm.uslot[q / kMaxRows][q % kMaxRows] = -1;
    for (int u = lane; u <= nU; u += 64) sm.umask[u] = 0u;
    for (int q = lane; q < RK; q += 64) {
      const int r = q / K, j = q % K, e = sm.sel_e[r][j];
      const int u = sm.ubase[e >> 5] + __popc(sm.ubits[e >> 5] & ((1u << (e & 31)) - 1u));
      sm.uslot[u][r] = (int8_t)j;
      atomicOr(&sm.umask[u], 1u << r);
    }
    for (int r = lane; r < R; r += 64) sm.uslot[nU][r] = (int8_t)K;
    if (lane == 0) {
      sm.umask[nU] = (1u << R) - 1u;
      sm.nU = nU;
    }
  }
}

/* plan_wave by wave 0, then a workgroup barrier. */
__device__ __forceinline__ void ph_plan(const Params& p, Smem& sm) {
  if (threadIdx.x < 64) plan_wave(p, sm);
  __syncthreads();
}

/* ------------------------------------------------------------------------------------------
 * Phase: gate/up + SwiGLU [ds4 router/shared commit: both matvecs, gate/up rounded to BF16
 * before SwiGLU and the product after it]. Task (expert, intermediate row i): one wave streams
 * gate row i and up row i once and applies them to every row that chose the expert.
 * READING: routed experts use the shared expert's rounding points. */
/* Gate row i and up row i of expert e (and their scale rows). */
template <int FMT>
__device__ __forceinline__ void gu_rows(const Params& p, const Mat& m, int e, int i, int inter,
                                        const uint8_t* (&vr)[2], const uint8_t* (&sr)[2]) {
  const size_t vb = row_vbytes(FMT, p.H), sb = row_sbytes(FMT, p.H);
  const size_t row = (size_t)e * inter + i;
  vr[0] = m.gate + row * vb;
  vr[1] = m.up + row * vb;
  sr[0] = m.gate_s ? m.gate_s + row * sb : nullptr;
  sr[1] = m.up_s ? m.up_s + row * sb : nullptr;
}

/* SwiGLU of hidden row i from the per-lane partial sums of gate (acc[0]) and up (acc[1]). */
template <int ACT, int RMAX>
__device__ __forceinline__ void gu_store(const Params& p, const Smem& sm, float (&acc)[2][RMAX],
                                         int i, uint32_t mask, int u, bool is_shared,
                                         uint32_t htag, bool hskip) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (!(mask & (1u << r))) continue;
    const float g = act_round<ACT>(wave_sum(acc[0][r]));
    const float uu = act_round<ACT>(wave_sum(acc[1][r]));
    const float h = act_round<ACT>(g / (1.0f + expf(-g)) * uu);
    if (lane == 0 && !hskip) {
      if (is_shared)
        hid_store<ACT>(p.h_shared, (size_t)r * p.Is + i, h, htag);
      else
        hid_store<ACT>(p.h_routed, ((size_t)r * p.K + sm.uslot[u][r]) * p.I + i, h, htag);
    }
  }
}

template <int ACT, int FMT, int RMAX>
__device__ __forceinline__ void gateup_task(const Params& p, const Smem& sm, const Mat& m,
                                            int e, int i, int inter, uint32_t mask, int u,
                                            bool is_shared, uint32_t htag, bool hskip) {
  const int H = p.H;
  const uint8_t* vr[2];
  const uint8_t* sr[2];
  gu_rows<FMT>(p, m, e, i, inter, vr, sr);
  const void* arow[RMAX];
  act_rows_ptrs<ACT, RMAX>(p, sm, arow);
  float acc[2][RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) acc[0][r] = acc[1][r] = 0.0f;
  dot_rows<FMT, ACT, RMAX, 2, Fmt<FMT>::CH_GU>(vr, sr, H, arow, mask, acc);
  gu_store<ACT, RMAX>(p, sm, acc, i, mask, u, is_shared, htag, hskip);
}

/* ------------------------------------------------------------------------------------------
 * Shared-expert gate/up at several rows on the matrix cores. Every row uses the shared expert,
 * so its gate/up is a small dense product [2 Is x H] x [H x R]. A workgroup takes tiles of 8
 * hidden rows: 16 weight rows (8 gate, 8 up) against the R activation rows (columns; the 16 - R
 * spare columns read row 0 and are dropped), with v_mfma_f32_16x16x32_bf16. Its 8 waves split
 * H into 8 ranges of 32-wide steps and the partial tiles are summed in LDS in wave order.
 * Operand layout (checked on the device): lane l gives A row l % 16 and B column l % 16, with
 * k = 32 s + 8 (l / 16) .. + 7; it gets D rows 4 (l / 16) + i, column l % 16. Q8_0 and MXFP4
 * weights decode exactly to bf16 and their block scale (one per 32-wide step and row)
 * multiplies each step's product before it is accumulated. */
typedef __bf16 mfma_bf16x8 __attribute__((ext_vector_type(8)));
typedef float mfma_f32x4 __attribute__((ext_vector_type(4)));
constexpr int kMfmaPass = 20; /* steps whose weight loads a wave keeps in flight at once */

__device__ __forceinline__ uint32_t smfma_scratch_off(const Params& p) {
  return (uint32_t)(((size_t)(p.R + 1) * p.H * 2 + 255) / 256 * 256);
}

/* The matrix-core path needs bf16 activations, 8-row tiles and its LDS scratch (the partial
 * tiles of 8 waves and their block scales) after the activation rows and norm weight. */
template <int ACT>
__device__ __forceinline__ bool smfma_fits(const Params& p) {
  return ACT == BF16 && p.R > 1 && p.Is > 0 && p.Is % 8 == 0 &&
         smfma_scratch_off(p) + 8 * 64 * 16 + 8 * kMfmaPass * 16 * 4 <= (uint32_t)kLdsActBytes;
}

/* Weight values k .. k + 7 of one row as bf16 (exact), and the row's block scale source. */
template <int SFMT>
__device__ __forceinline__ mfma_bf16x8 smfma_a(const uint8_t* row, int k) {
  mfma_bf16x8 a;
  if constexpr (SFMT == BF16) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + (size_t)k * 2);
    a = __builtin_bit_cast(mfma_bf16x8, v);
  } else if constexpr (SFMT == Q8) {
    const uint2 v = *reinterpret_cast<const uint2*>(row + k);
    const uint32_t d[2] = {v.x, v.y};
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const float f0 = (float)(int)(int8_t)d[i];
      const float f1 = (float)(int)(int8_t)(d[i] >> 8);
      const float f2 = (float)(int)(int8_t)(d[i] >> 16);
      const float f3 = (float)(int)(int8_t)(d[i] >> 24);
      w[2 * i] = __builtin_amdgcn_perm(__float_as_uint(f1), __float_as_uint(f0), 0x07060302u);
      w[2 * i + 1] = __builtin_amdgcn_perm(__float_as_uint(f3), __float_as_uint(f2), 0x07060302u);
    }
    a = __builtin_bit_cast(mfma_bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  } else {
    const uint32_t d = *reinterpret_cast<const uint32_t*>(row + k / 2);
    const uint32_t w0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 0));
    const uint32_t w1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 1));
    const uint32_t w2 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 2));
    const uint32_t w3 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(d, 1.0f, 3));
    a = __builtin_bit_cast(mfma_bf16x8, make_uint4(w0, w1, w2, w3));
  }
  return a;
}

template <int SFMT>
__device__ __forceinline__ float smfma_scale(const uint8_t* srow, int step) {
  if constexpr (SFMT == Q8) return f16_to_f32(reinterpret_cast<const uint16_t*>(srow)[step]);
  else return e8m0_to_f32(srow[step]);
}

template <int SFMT>
__device__ __forceinline__ void shared_gu_mfma(const Params& p, Smem& sm, uint32_t htag,
                                               bool hskip) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int S = p.H / 32, ks0 = wave * S / kWaves, ks1 = (wave + 1) * S / kWaves;
  const size_t vb = row_vbytes(SFMT, p.H), sb = row_sbytes(SFMT, p.H);
  float* red = reinterpret_cast<float*>(sm.big + smfma_scratch_off(p)); /* [8][64][4] */
  float* scl = red + kWaves * 64 * 4; /* [8 waves][kMfmaPass][16 rows] */
  const int NT = p.Is / 8;
  const int m = lane % 16, grp = lane / 16;
  const int n = lane % 16 < p.R ? lane % 16 : 0;
  const uint16_t* arow = reinterpret_cast<const uint16_t*>(sm.big) + (size_t)n * p.H;
  for (int tile = blockIdx.x; tile < NT; tile += gridDim.x) {
    const int i0 = tile * 8;
    const size_t wr = (size_t)(i0 + (m & 7));
    const uint8_t* row = (m < 8 ? p.shared.gate : p.shared.up) + wr * vb;
    mfma_f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int s0 = ks0; s0 < ks1; s0 += kMfmaPass) {
      const int ns = ks1 - s0 < kMfmaPass ? ks1 - s0 : kMfmaPass;
      /* block scales of the tile's 16 rows for these steps (lane q: row q % 16, step q / 16),
       * loaded before the weights so that they reach LDS while the weights are in flight */
      constexpr int NSC = SFMT != BF16 ? (16 * kMfmaPass + 63) / 64 : 1;
      float sv[NSC];
      if constexpr (SFMT != BF16) {
#pragma unroll
        for (int t = 0; t < NSC; ++t) {
          const int q = lane + 64 * t, rr = q % 16, j = q / 16 < ns ? q / 16 : ns - 1;
          const uint8_t* srow = (rr < 8 ? p.shared.gate_s : p.shared.up_s) + (size_t)(i0 + (rr & 7)) * sb;
          sv[t] = smfma_scale<SFMT>(srow, s0 + j);
        }
      }
      uint4 a[kMfmaPass];
#pragma unroll
      for (int j = 0; j < kMfmaPass; ++j) /* past ns a step repeats the last one, unused */
        a[j] = __builtin_bit_cast(uint4, smfma_a<SFMT>(row, (s0 + (j < ns ? j : ns - 1)) * 32 + 8 * grp));
      if constexpr (SFMT != BF16) {
        /* [step][row] in this wave's LDS */
#pragma unroll
        for (int t = 0; t < NSC; ++t) {
          const int q = lane + 64 * t;
          if (q < 16 * ns) scl[(wave * kMfmaPass + q / 16) * 16 + q % 16] = sv[t];
        }
        /* the same wave reads them below: its LDS writes complete first */
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      }
#pragma unroll
      for (int j = 0; j < kMfmaPass; ++j) {
        if (j < ns) {
          const int k = (s0 + j) * 32 + 8 * grp;
          const mfma_bf16x8 av = __builtin_bit_cast(mfma_bf16x8, a[j]);
          const mfma_bf16x8 b =
              __builtin_bit_cast(mfma_bf16x8, *reinterpret_cast<const uint4*>(arow + k));
          if constexpr (SFMT == BF16) {
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b, acc, 0, 0, 0);
          } else {
            const mfma_f32x4 zero = {0.0f, 0.0f, 0.0f, 0.0f};
            const mfma_f32x4 t = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b, zero, 0, 0, 0);
            const float* sc = scl + (wave * kMfmaPass + j) * 16 + 4 * grp;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = fmaf(sc[i], t[i], acc[i]);
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(wave * 64 + lane) * 4 + i] = acc[i];
    __syncthreads();
    if (wave == 0) {
      float d[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float t = 0.0f;
        for (int w = 0; w < kWaves; ++w) t += red[(w * 64 + lane) * 4 + i];
        d[i] = t;
      }
      /* lanes 0-31 hold gate rows 0-7, lanes 32-63 the matching up rows */
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float up = __shfl(d[i], lane + 32);
        const int rowh = 4 * grp + i, col = lane % 16;
        if (lane < 32 && col < p.R && !hskip) {
          const float g = act_round<BF16>(d[i]);
          const float u = act_round<BF16>(up);
          const float h = act_round<BF16>(g / (1.0f + expf(-g)) * u);
          hid_store<BF16>(p.h_shared, (size_t)col * p.Is + i0 + rowh, h, htag);
        }
      }
    }
    __syncthreads();
  }
}

/* Shared-expert gate/up: Is tasks spread over compute units first. */
template <int ACT, int SFMT, int RMAX>
__device__ __forceinline__ void ph_gateup_shared(const Params& p, Smem& sm) {
  if (p.Is <= 0) return;
  if (RMAX > 1 && smfma_fits<ACT>(p)) {
    shared_gu_mfma<SFMT>(p, sm, 0u, false);
    return;
  }
  const int nwt = gridDim.x * kWaves;
  const uint32_t mask = (1u << p.R) - 1u;
  for (int i = wave_major_id(); i < p.Is; i += nwt)
    gateup_task<ACT, SFMT, RMAX>(p, sm, p.shared, 0, i, p.Is, mask, 0, true, 0u, false);
}

/* A value the whole wave holds alike, moved to a scalar register, so that branches on it are
 * scalar branches rather than per-lane masks. */
__device__ __forceinline__ uint32_t uniform(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}

/* Next task index of this wave from an LDS counter: all 64 lanes add 1 and lane 0's old value
 * (a multiple of 64) is read back uniformly, so there is no divergent branch in the loop. */
__device__ __forceinline__ int claim(int* counter) {
  return __builtin_amdgcn_readfirstlane(atomicAdd(counter, 1)) / 64;
}

/* Shared-expert gate/up in the fused launch: workgroup g owns rows g, g + grid, ...; its waves
 * claim them one at a time from an LDS counter (sm.shared_next, zeroed beforehand), so a wave
 * that also selects joins when it is done. */
template <int ACT, int SFMT, int RMAX>
__device__ __forceinline__ void ph_gateup_shared_claim(const Params& p, Smem& sm, uint32_t htag,
                                                       bool hskip) {
  if (p.Is <= 0) return;
  if (RMAX > 1 && smfma_fits<ACT>(p)) {
    shared_gu_mfma<SFMT>(p, sm, htag, hskip);
    return;
  }
  const uint32_t mask = (1u << p.R) - 1u;
  for (;;) {
    const int i = (int)blockIdx.x + claim(&sm.shared_next) * (int)gridDim.x;
    if (i >= p.Is) break;
    gateup_task<ACT, SFMT, RMAX>(p, sm, p.shared, 0, i, p.Is, mask, 0, true, htag, hskip);
  }
}

template <int ACT, int NA, int GB>
__device__ __forceinline__ void gu_wide_store(const Params& p, const Smem& sm,
                                              float (&acc)[2 * GB][NA], int u, int i0,
                                              const int (&rows)[NA], uint32_t htag, bool hskip);

/* GB consecutive hidden rows i0 .. of routed expert u for the NA rows in `mask` (NA = its
 * population): the 2 GB gate and up weight rows stream at once. */
template <int ACT, int FMT, int NA, int GB>
__device__ __forceinline__ void gu_wide(const Params& p, const Smem& sm, int u, int i0,
                                        uint32_t mask, uint32_t htag, bool hskip) {
  int rows[NA];
  uint32_t m = mask;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    rows[a] = __builtin_ctz(m);
    m &= m - 1u;
  }
  const uint8_t* vr[2 * GB];
  const uint8_t* sr[2 * GB];
#pragma unroll
  for (int g = 0; g < GB; ++g) {
    const uint8_t* v2[2];
    const uint8_t* s2[2];
    gu_rows<FMT>(p, p.routed, sm.U[u], i0 + g, p.I, v2, s2);
    vr[2 * g] = v2[0];
    vr[2 * g + 1] = v2[1];
    sr[2 * g] = s2[0];
    sr[2 * g + 1] = s2[1];
  }
  const void* arow[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) arow[a] = sm.big + (size_t)rows[a] * p.H * (ACT == F32 ? 4 : 2);
  float acc[2 * GB][NA];
#pragma unroll
  for (int k = 0; k < 2 * GB; ++k)
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[k][a] = 0.0f;
  dot_rows<FMT, ACT, NA, 2 * GB, Fmt<FMT>::CH_GU>(vr, sr, p.H, arow, (1u << NA) - 1u, acc);
  gu_wide_store<ACT, NA, GB>(p, sm, acc, u, i0, rows, htag, hskip);
}

/* SwiGLU of hidden rows i0 .. i0 + GB - 1 of item u for rows[0 .. NA) from the per-lane partial
 * sums of their gate (acc[2 g]) and up (acc[2 g + 1]) rows; lane g stores hidden row i0 + g,
 * one coalesced store per row. */
template <int ACT, int NA, int GB>
__device__ __forceinline__ void gu_wide_store(const Params& p, const Smem& sm,
                                              float (&acc)[2 * GB][NA], int u, int i0,
                                              const int (&rows)[NA], uint32_t htag, bool hskip) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int r = rows[a];
    float hv = 0.0f;
#pragma unroll
    for (int g = 0; g < GB; ++g) {
      const float gg = act_round<ACT>(wave_sum(acc[2 * g][a]));
      const float uu = act_round<ACT>(wave_sum(acc[2 * g + 1][a]));
      const float h = act_round<ACT>(gg / (1.0f + expf(-gg)) * uu);
      if (lane == g) hv = h;
    }
    if (lane < GB && !hskip)
      hid_store<ACT>(p.h_routed, ((size_t)r * p.K + sm.uslot[u][r]) * p.I + i0 + lane, hv, htag);
  }
}

/* Routed gate/up: workgroup b owns one task of every round of grid tasks (expert-major order,
 * see gu_task), so at any moment the grid streams one contiguous stretch of rows; its waves
 * claim them one at a time, so a wave that runs ahead takes more and the workgroup's waves end
 * together. At several rows a
 * task is GB consecutive hidden rows of one expert: when one or two rows use the expert, all
 * 2 GB weight rows stream at once against them; otherwise the rows go one by one for every row
 * that uses the expert. Every hidden value comes from the same per-row dot product either way. */
/* Task of the n-th routed gate/up claim of this workgroup: round n covers tasks n grid ..
 * (n + 1) grid - 1 (expert-major, so experts complete in order), and within a round the
 * workgroup's slot rotates by 37 per round, so one workgroup's rows do not keep the same
 * address residues (and HBM channels) from round to round. */
__device__ __forceinline__ int gu_task(int n) {
  const int G = gridDim.x;
  return n * G + (int)(((unsigned)blockIdx.x + 37u * (unsigned)n) % (unsigned)G);
}

/* Routed gate/up at several rows for Q8_0 and MXFP4 rows that fit one chunk: tasks of GB / 2
 * hidden rows, software-pipelined over two register buffers, so a wave issues the loads of its
 * next task before it computes the current one and waits only for the current one's loads
 * (every load is issued unconditionally: past the last task a wave loads through an empty
 * resource, which returns zeros without touching memory). */
template <int ACT, int FMT, int RMAX>
__device__ __forceinline__ void gu_pipelined(const Params& p, Smem& sm, uint32_t htag,
                                             bool hskip) {
  constexpr int GBp = Wide<FMT>::GB / 2, NR = 2 * GBp, CH = Fmt<FMT>::CH_GU;
  const int lane = threadIdx.x & 63;
  const int nb = p.I / GBp, T = sm.nU * nb;
  const size_t vb = row_vbytes(FMT, p.H), sb = row_sbytes(FMT, p.H);
  auto next = [&]() -> int { return gu_task(claim(&sm.routed_next)); };
  auto load = [&](WRegs<FMT, NR, CH>& W, int t) {
    const bool live = t < T;
    const int tt = live ? t : 0;
    const int u = tt / nb, i0 = (tt % nb) * GBp;
#pragma unroll
    for (int g = 0; g < GBp; ++g) {
      const uint8_t* vr[2];
      const uint8_t* sr[2];
      gu_rows<FMT>(p, p.routed, sm.U[u], i0 + g, p.I, vr, sr);
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const __amdgpu_buffer_rsrc_t rv = row_rsrc(vr[h], live ? vb : 0);
        const __amdgpu_buffer_rsrc_t rs = row_rsrc(sr[h], live ? sb : 0);
#pragma unroll
        for (int c = 0; c < CH; ++c)
          wload<FMT>(rv, rs, c, lane, W.v[2 * g + h][c], W.sc[2 * g + h][c]);
      }
    }
  };
  auto compute = [&](const WRegs<FMT, NR, CH>& W, int t) {
    const int u = t / nb, i0 = (t % nb) * GBp;
    const uint32_t mask = uniform(sm.umask[u]);
    const int n = __popc(mask);
    const size_t ab = ACT == F32 ? 4 : 2;
    if (n == 1) {
      const int rows[1] = {__builtin_ctz(mask)};
      const void* arow[1] = {sm.big + (size_t)rows[0] * p.H * ab};
      float acc[NR][1];
#pragma unroll
      for (int k = 0; k < NR; ++k) acc[k][0] = 0.0f;
      wregs_dot<FMT, ACT, 1, NR, CH>(W, p.H, 0, arow, 1u, acc);
      gu_wide_store<ACT, 1, GBp>(p, sm, acc, u, i0, rows, htag, hskip);
    } else if (n == 2) {
      const int r0 = __builtin_ctz(mask);
      const int rows[2] = {r0, __builtin_ctz(mask & (mask - 1u))};
      const void* arow[2] = {sm.big + (size_t)rows[0] * p.H * ab,
                             sm.big + (size_t)rows[1] * p.H * ab};
      float acc[NR][2];
#pragma unroll
      for (int k = 0; k < NR; ++k) acc[k][0] = acc[k][1] = 0.0f;
      wregs_dot<FMT, ACT, 2, NR, CH>(W, p.H, 0, arow, 3u, acc);
      gu_wide_store<ACT, 2, GBp>(p, sm, acc, u, i0, rows, htag, hskip);
    } else {
      const void* arow[RMAX];
      act_rows_ptrs<ACT, RMAX>(p, sm, arow);
      float acc[NR][RMAX];
#pragma unroll
      for (int k = 0; k < NR; ++k)
#pragma unroll
        for (int r = 0; r < RMAX; ++r) acc[k][r] = 0.0f;
      wregs_dot<FMT, ACT, RMAX, NR, CH>(W, p.H, 0, arow, mask, acc);
#pragma unroll
      for (int g = 0; g < GBp; ++g) {
        float a2[2][RMAX];
#pragma unroll
        for (int r = 0; r < RMAX; ++r) {
          a2[0][r] = acc[2 * g][r];
          a2[1][r] = acc[2 * g + 1][r];
        }
        gu_store<ACT, RMAX>(p, sm, a2, i0 + g, mask, u, false, htag, hskip);
      }
    }
  };
  WRegs<FMT, NR, CH> A, B;
  int tA = next();
  load(A, tA);
  while (tA < T) {
    const int tB = next();
    load(B, tB);
    compute(A, tA);
    if (tB >= T) break;
    tA = next();
    load(A, tA);
    compute(B, tB);
  }
}

template <int ACT, int RFMT, int RMAX>
__device__ __forceinline__ void ph_gateup_routed(const Params& p, Smem& sm, uint32_t htag,
                                                 bool hskip) {
  if constexpr (RMAX > 1 && (RFMT == Q8 || RFMT == FP4)) {
    if (p.H <= 64 * Fmt<RFMT>::EL * Fmt<RFMT>::CH_GU) {
      gu_pipelined<ACT, RFMT, RMAX>(p, sm, htag, hskip);
      return;
    }
  }
  constexpr int GB = RMAX > 1 ? Wide<RFMT>::GB : 1;
  const int nb = p.I / GB;
  const int T = sm.nU * nb;
  auto next = [&]() -> int { return gu_task(claim(&sm.routed_next)); };
  for (int t = next(); t < T; t = next()) {
    const int u = t / nb, i0 = (t % nb) * GB;
    const uint32_t mask = uniform(sm.umask[u]);
    const int n = __popc(mask);
    if (RMAX > 1 && n == 1)
      gu_wide<ACT, RFMT, 1, GB>(p, sm, u, i0, mask, htag, hskip);
    else if (RMAX > 1 && n == 2)
      gu_wide<ACT, RFMT, 2, GB>(p, sm, u, i0, mask, htag, hskip);
    else
#pragma unroll 1
      for (int g = 0; g < GB; ++g)
        gateup_task<ACT, RFMT, RMAX>(p, sm, p.routed, sm.U[u], i0 + g, p.I, mask, u, false, htag,
                                     hskip);
  }
}

/* ------------------------------------------------------------------------------------------
 * Phase: down projections, routed sum, shared rounding and block for the workgroup's slice of
 * hidden rows [ds4 router/shared commit: the down projection rounded on its store, the routed +
 * shared sum and its rounding]. The hidden rows of the selected experts are staged in LDS in
 * groups; task (item, group of 4 consecutive output rows) is one wave. y values land in LDS;
 * then per (h, r): routed = f32 sum_j w_j y_j (selection order), shared = bf16(y_s),
 * block = bf16(routed + shared). Leaves block in sm for the expand. */
struct DownGeo {
  int h0, nh, hs;
  float* y;   /* [hs][R][K + 1] */
  float* blk; /* [hs][R] */
};

__device__ __forceinline__ DownGeo down_geo(const Params& p, Smem& sm) {
  DownGeo g;
  g.hs = (p.H + p.nslice - 1) / p.nslice;
  g.h0 = blockIdx.x * g.hs;
  g.nh = p.H - g.h0 < g.hs ? p.H - g.h0 : g.hs;
  if (g.nh < 0) g.nh = 0;
  g.y = reinterpret_cast<float*>(sm.big + kLdsHidBytes);
  g.blk = g.y + (size_t)g.hs * p.R * (p.K + 1);
  return g;
}

template <int ACT, int FMT>
__device__ __forceinline__ void down_rows(const Params& p, const DownGeo& g, const Mat& m, int e,
                                          int inter, int q, const uint8_t* (&vr)[kRG],
                                          const uint8_t* (&sr)[kRG]) {
  const size_t vb = row_vbytes(FMT, inter), sb = row_sbytes(FMT, inter);
#pragma unroll
  for (int c = 0; c < kRG; ++c) {
    int hl = q * kRG + c;
    if (hl >= g.nh) hl = g.nh - 1; /* duplicate a valid row; its result is discarded */
    const size_t row = (size_t)e * p.H + g.h0 + hl;
    vr[c] = m.down + row * vb;
    sr[c] = m.down_s ? m.down_s + row * sb : nullptr;
  }
}

template <int ACT, int FMT, int RMAX>
__device__ __forceinline__ void down_task(const Params& p, const Smem& sm, const DownGeo& g,
                                          const Mat& m, int e, int inter, int item, int q,
                                          bool is_shared,
                                          const WRegs<FMT, kRG, Fmt<FMT>::CH_DN>& pre,
                                          bool use_pre) {
  const int lane = threadIdx.x & 63;
  constexpr int CH = Fmt<FMT>::CH_DN;
  const uint8_t* vr[kRG];
  const uint8_t* sr[kRG];
  down_rows<ACT, FMT>(p, g, m, e, inter, q, vr, sr);
  const uint32_t mask = uniform(sm.umask[item]);
  const void* arow[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
    arow[r] = sm.big + (size_t)((mask & (1u << r)) ? sm.voff[item][r] : 0) * 16;
  float acc[kRG][RMAX];
#pragma unroll
  for (int c = 0; c < kRG; ++c)
#pragma unroll
    for (int r = 0; r < RMAX; ++r) acc[c][r] = 0.0f;
  if (use_pre) {
    wregs_dot<FMT, ACT, RMAX, kRG, CH>(pre, inter, 0, arow, mask, acc);
    dot_rows<FMT, ACT, RMAX, kRG, CH>(vr, sr, inter, arow, mask, acc, CH);
  } else {
    dot_rows<FMT, ACT, RMAX, kRG, CH>(vr, sr, inter, arow, mask, acc);
  }
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (!(mask & (1u << r))) continue;
    const int slot = is_shared ? p.K : sm.uslot[item][r];
#pragma unroll
    for (int c = 0; c < kRG; ++c) {
      const float t = wave_sum(acc[c][r]);
      const int hl = q * kRG + c;
      if (lane == 0 && hl < g.nh) g.y[((size_t)hl * p.R + r) * (p.K + 1) + slot] = t;
    }
  }
}

/* Items [first, last) whose hidden rows fit in the staging area (bytes and list entries). */
/* Order of the down phase's items: the shared expert first (its hidden rows are complete
 * earliest), then the distinct routed experts in ascending order. */
__device__ __forceinline__ int down_item(const Params& p, const Smem& sm, int k) {
  return p.Is > 0 ? (k == 0 ? sm.nU : k - 1) : k;
}

/* End of the group of items [k0, end): as many as fit the staging area next to used0 bytes and
 * count0 rows already listed, at most max_items. Each wave computes it on its own, 64 items at a
 * time (one per lane, inclusive prefix sums of bytes and rows, the first item that overflows by
 * ballot), so no lane waits on a chain of LDS reads; the result is uniform. */
__device__ __forceinline__ int down_group_end(const Params& p, const Smem& sm, int k0, size_t ab,
                                              int max_items, size_t used0 = 0, int count0 = 0) {
  const int nU = sm.nU, n_items = nU + (p.Is > 0 ? 1 : 0), lane = threadIdx.x & 63;
  const int kend = min(n_items, k0 + max_items);
  uint32_t used = (uint32_t)used0;
  int count = count0;
  for (int c0 = k0; c0 < kend; c0 += 64) {
    const int k = c0 + lane;
    uint32_t need = 0u;
    int rows = 0;
    if (k < kend) {
      const int item = down_item(p, sm, k);
      rows = __popc(sm.umask[item]);
      need = (uint32_t)((size_t)rows * (item == nU ? p.Is : p.I) * ab);
    }
    uint32_t pn = need;
    int pr = rows;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t tn = __shfl_up(pn, d);
      const int tr = __shfl_up(pr, d);
      if (lane >= d) {
        pn += tn;
        pr += tr;
      }
    }
    /* the first item always fits an empty area; rows already listed (count0) may leave none */
    const bool first_item = k == k0 && count0 == 0;
    const bool over = k < kend && !first_item &&
                      (used + pn > (uint32_t)kLdsHidBytes || count + pr > kMaxStaged);
    const uint64_t ov = __ballot(over);
    if (ov != 0ull) return c0 + (int)__builtin_ctzll(ov);
    used += __shfl(pn, 63);
    count += __shfl(pr, 63);
  }
  return kend;
}

/* Hidden-position slice of the workgroup for the down projections and the expand. */
struct Slice {
  int h0, nh, hs;
  bool lds; /* the slice's state and next mix weights were copied into LDS */
};

__device__ __forceinline__ Slice slice_of(const Params& p) {
  Slice c;
  c.hs = (p.H + p.nslice - 1) / p.nslice;
  c.h0 = blockIdx.x * c.hs;
  c.nh = p.H - c.h0 < c.hs ? p.H - c.h0 : c.hs;
  if (c.nh < 0) c.nh = 0;
  c.lds = c.hs <= kSliceMax;
  return c;
}

/* Loads of the slice's input state [R][4][nh] and next mix weights [24][4][nh] into registers
 * (issued early so that their latency overlaps other waiting), then stored into LDS by
 * slice_store. Element e of the flat list: state first, then weights. */
constexpr int kSliceRegs = (kMaxRows * 4 * kSliceMax + kNMix * 4 * kSliceMax + kBlock - 1) / kBlock;
struct SliceRegs {
  float v[kSliceRegs];
};

template <int ACT>
__device__ __forceinline__ void slice_prefetch(const Params& p, const Slice& c, SliceRegs& sr) {
  if (!c.lds) return;
  const int tid = threadIdx.x, nh = c.nh, H = p.H;
  const int ns = p.R * 4 * nh, nw = p.w_mix_next ? kNMix * 4 * nh : 0;
#pragma unroll
  for (int k = 0; k < kSliceRegs; ++k) {
    const int e = tid + k * kBlock;
    sr.v[k] = 0.0f;
    if (e < ns) {
      const int hl = e % nh, ri = e / nh; /* ri = r * 4 + i */
      sr.v[k] = act_ld<ACT>(p.state, (size_t)ri * H + c.h0 + hl);
    } else if (e < ns + nw) {
      const int f = e - ns, hl = f % nh, ji = f / nh; /* ji = j * 4 + i */
      sr.v[k] = p.w_mix_next[(size_t)ji * H + c.h0 + hl];
    }
  }
}

__device__ __forceinline__ void slice_store(const Params& p, const Slice& c, Smem& sm,
                                            const SliceRegs& sr) {
  if (!c.lds) return;
  const int tid = threadIdx.x, nh = c.nh;
  const int ns = p.R * 4 * nh, nw = p.w_mix_next ? kNMix * 4 * nh : 0;
#pragma unroll
  for (int k = 0; k < kSliceRegs; ++k) {
    const int e = tid + k * kBlock;
    if (e < ns)
      sm.sslice[(e / nh) * kSliceMax + e % nh] = sr.v[k];
    else if (e < ns + nw)
      sm.wnext[((e - ns) / nh) * kSliceMax + (e - ns) % nh] = sr.v[k];
  }
}

/* Staging list of the items of positions [first, last) in down_item order (optionally led by
 * the shared expert): for every (item, row
 * that uses it), in item-major
 * order, the source of the hidden row (routed [R][K][I] or shared [R][Is]), its LDS offset and
 * length in 16-byte units, and sm.voff. One wave scans the items 64 at a time. */
__device__ __forceinline__ void stage_list_wave(const Params& p, Smem& sm, int first, int last,
                                                size_t ab, bool lead_shared = false) {
  {
    const int lane = threadIdx.x & 63, nU = sm.nU;
    /* with lead_shared the shared expert (position 0) comes before positions [first, last) */
    const int lead = lead_shared ? 1 : 0, n = lead + (last - first);
    int nv = 0;
    uint32_t off = 0;
    for (int k0 = 0; k0 < n; k0 += 64) {
      const int v0 = k0 + lane;
      const bool live = v0 < n;
      const int pos = v0 < lead ? 0 : first + v0 - lead;
      const int it = live ? down_item(p, sm, pos) : 0;
      const uint32_t m = live ? sm.umask[it] : 0u;
      const bool sh = it == nU;
      const uint32_t vl = (uint32_t)((size_t)(sh ? p.Is : p.I) * ab / 16);
      const int rows = __popc(m);
      int pr = rows;
      uint32_t pb = (uint32_t)rows * vl;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int tr = __shfl_up(pr, d);
        const uint32_t tb = __shfl_up(pb, d);
        if (lane >= d) {
          pr += tr;
          pb += tb;
        }
      }
      if (live) {
        int v = nv + pr - rows;
        uint32_t o = off + pb - (uint32_t)rows * vl;
        for (int r = 0; r < p.R; ++r)
          if (m & (1u << r)) {
            sm.voff[it][r] = (uint16_t)o;
            /* source: first element of the hidden row (tagged buffers) */
            sm.vsrc[v] = sh ? (uint32_t)(kHidShared | ((size_t)r * p.Is))
                            : (uint32_t)(((size_t)r * p.K + sm.uslot[it][r]) * p.I);
            sm.vdst[v] = (uint16_t)o;
            sm.vlen[v] = (uint16_t)vl;
            ++v;
            o += vl;
          }
      }
      nv += __shfl(pr, 63);
      off += __shfl(pb, 63);
    }
    if (lane == 0) sm.nv = nv;
  }
}

/* stage_list_wave by wave 0, then a workgroup barrier. */
__device__ __forceinline__ void stage_list(const Params& p, Smem& sm, int first, int last,
                                           size_t ab, bool lead_shared = false) {
  if (threadIdx.x < 64) stage_list_wave(p, sm, first, last, ab, lead_shared);
  __syncthreads();
}

/* Copies the listed hidden rows into LDS, dropping their tags: wave w takes rows w, w + 8, ...;
 * a 16-byte LDS chunk (8 bf16 or 4 f32 values) comes from 32 bytes of tagged values (two
 * coherent 16-byte loads); each lane keeps up to 4 chunks in flight before storing them. With
 * check, a chunk whose tags are not yet `tag` is loaded again (bounded wait); on expiry the
 * function reports once and returns false for the whole workgroup. */
template <int ACT>
__device__ __forceinline__ bool stage_copy(const Params& p, Smem& sm, bool check, uint32_t tag,
                                           bool mx_shared) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int TB = ACT == F32 ? 8 : 4; /* tagged bytes per value */
  constexpr int EPC = ACT == F32 ? 4 : 8; /* values per 16-byte LDS chunk */
  /* one resource over the routed and then the shared hidden rows (consecutive workspace
   * regions), so every load of a round uses the same scalar resource */
  const uint8_t* hbase = static_cast<const uint8_t*>(p.h_routed);
  const uint32_t sh_off = (uint32_t)(static_cast<const uint8_t*>(p.h_shared) - hbase);
  const __amdgpu_buffer_rsrc_t hr =
      coh_region(hbase, (size_t)sh_off + (size_t)p.R * (p.Is > 0 ? p.Is : 1) * TB);
  if (threadIdx.x == 0) sm.sel_ok = 1;
  __syncthreads();
  const int nv = sm.nv;
  int v = wave, ch = lane;
  while (v < nv && ch >= (int)sm.vlen[v]) {
    v += kWaves;
    ch = lane;
  }
  bool ok = true;
  constexpr int B = 4;
  while (__ballot(v < nv) != 0ull) {
    uint4 lo[B], hi[B];
    uint32_t dst[B], src[B];
    /* addresses first, then all loads of the round back to back (a lane without a chunk
     * repeats its first one, unused), then the tag checks */
#pragma unroll
    for (int b = 0; b < B; ++b) {
      dst[b] = 0xFFFFFFFFu;
      src[b] = 0u;
      if (v < nv) {
        const uint32_t s0 = sm.vsrc[v];
        const uint32_t e0 = s0 & ~kHidShared;
        src[b] = ((s0 & kHidShared) ? sh_off : 0u) + (e0 + (uint32_t)ch * EPC) * TB;
        dst[b] = (uint32_t)sm.vdst[v] + ch;
        ch += 64;
        while (v < nv && ch >= (int)sm.vlen[v]) {
          v += kWaves;
          ch = lane;
        }
      }
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const uint32_t o = dst[b] != 0xFFFFFFFFu ? src[b] : src[0];
      lo[b] = coh_b128(hr, o);
      hi[b] = coh_b128(hr, o + 16);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      if (dst[b] == 0xFFFFFFFFu) continue;
      if (check) {
        auto stale = [&]() {
          if (ACT == F32)
            return lo[b].y != tag || lo[b].w != tag || hi[b].y != tag || hi[b].w != tag;
          const uint32_t w0 = lo[b].x & lo[b].y & lo[b].z & lo[b].w & hi[b].x & hi[b].y & hi[b].z & hi[b].w;
          const uint32_t w1 = lo[b].x | lo[b].y | lo[b].z | lo[b].w | hi[b].x | hi[b].y | hi[b].z | hi[b].w;
          return (w0 >> 16) != tag || (w1 >> 16) != tag;
        };
        if (stale()) {
          const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
          while (stale()) {
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_sleep(1);
            lo[b] = coh_b128(hr, src[b]);
            hi[b] = coh_b128(hr, src[b] + 16);
            if (__builtin_amdgcn_s_memrealtime() - t0 > sm.spin) {
              ok = false;
              break;
            }
          }
        }
      }
      uint4 o;
      if (ACT == F32) {
        o = make_uint4(lo[b].x, lo[b].z, hi[b].x, hi[b].z);
      } else {
        o = make_uint4((lo[b].x & 0xFFFFu) | (lo[b].y << 16), (lo[b].z & 0xFFFFu) | (lo[b].w << 16),
                       (hi[b].x & 0xFFFFu) | (hi[b].y << 16), (hi[b].z & 0xFFFFu) | (hi[b].w << 16));
      }
      reinterpret_cast<uint4*>(sm.big)[dst[b]] = o;
    }
  }
  if (!ok) sm.sel_ok = 0;
  __syncthreads();
  if (sm.sel_ok == 0) {
    if (threadIdx.x == 0) report_timeout(p, PH_GATEUP);
    return false;
  }
  /* MXFP8 activations: the hidden rows entering MXFP4 down projections (the routed ones, and the
   * shared one when mx_shared) take their round trip in place */
  if (ACT == BF16 && p.aq8) {
    for (int u = wave; u < nv; u += kWaves) {
      if ((sm.vsrc[u] & kHidShared) && !mx_shared) continue;
      const int nblk = sm.vlen[u] / 4;
      for (int b = lane; b < nblk; b += 64) mx8_block_lds(sm.big + (size_t)sm.vdst[u] * 16 + b * 64);
    }
    __syncthreads();
  }
  return true;
}

/* Per (h, r) of the slice, from y [hs][R][K + 1] in LDS: routed = f32 sum_j w_j y_j in
 * selection order, shared = rounded y_s, block = rounded (routed + shared); block also to LDS
 * for the expand. Whole workgroup. */
template <int ACT>
__device__ __forceinline__ void down_combine(const Params& p, Smem& sm, const DownGeo& g) {
  const int R = p.R;
  for (int q = threadIdx.x; q < g.nh * R; q += kBlock) {
    const int hl = q / R, r = q % R;
    const float* y = g.y + ((size_t)hl * R + r) * (p.K + 1);
    float routed = 0.0f;
    for (int j = 0; j < p.K; ++j) routed = fmaf(sm.sel_w[r][j], y[j], routed);
    const float shared = p.Is > 0 ? act_round<ACT>(y[p.K]) : 0.0f;
    const float blk = act_round<ACT>(routed + shared);
    const size_t o = (size_t)r * p.H + g.h0 + hl;
    if (p.routed_out) p.routed_out[o] = routed;
    if (p.shared_out) act_st<ACT>(p.shared_out, o, shared);
    if (p.block) act_st<ACT>(p.block, o, blk);
    g.blk[q] = blk;
  }
  __syncthreads();
}

/* ------------------------------------------------------------------------------------------
 * One-row down phase of the fused launch as a flow: a wave that runs out of gate/up tasks goes
 * straight on to down tasks (item, kFlowRows rows of the slice) claimed from an LDS counter, while
 * other waves still finish their gate/up rows. Each item's hidden row is staged in LDS, behind
 * the activation row, by the first wave that needs it (an LDS compare-and-swap elects it);
 * other waves needing the item wait on its LDS state. Used when every item fits at once. */

/* LDS byte offset of the hidden rows of the item at down position k. */
__device__ __forceinline__ uint32_t flow_off(const Params& p, int k, size_t ab) {
  const size_t base = ((size_t)p.R * p.H * ab + 15) / 16 * 16;
  if (p.Is > 0) return (uint32_t)(k == 0 ? base : base + (size_t)p.Is * ab + (size_t)(k - 1) * p.I * ab);
  return (uint32_t)(base + (size_t)k * p.I * ab);
}

__device__ __forceinline__ bool flow_fits(const Params& p, const Smem& sm, size_t ab) {
  const int n_items = sm.nU + (p.Is > 0 ? 1 : 0);
  return p.R == 1 && flow_off(p, n_items, ab) <= (uint32_t)kLdsHidBytes;
}

/* One wave copies the hidden row of item `item` (one row) into LDS at byte offset `off`,
 * dropping the tags, each 16-byte chunk polled (bounded) until its tags are `tag`. */
template <int ACT>
__device__ __forceinline__ bool flow_stage(const Params& p, Smem& sm, int item, uint32_t off,
                                           uint32_t tag, bool mx) {
  const int lane = threadIdx.x & 63, nU = sm.nU;
  constexpr int TB = ACT == F32 ? 8 : 4, EPC = ACT == F32 ? 4 : 8;
  const bool sh = item == nU;
  const int inter = sh ? p.Is : p.I;
  const int r = __builtin_ctz(sm.umask[item]);
  const size_t src0 = sh ? (size_t)r * p.Is : ((size_t)r * p.K + sm.uslot[item][r]) * p.I;
  const __amdgpu_buffer_rsrc_t rs =
      sh ? coh_region(p.h_shared, (size_t)p.R * p.Is * TB)
         : coh_region(p.h_routed, (size_t)p.R * p.K * p.I * TB);
  const int nch = inter / EPC; /* 16-byte LDS chunks */
  bool ok = true;
  constexpr int B = 8;
  for (int c0 = 0; c0 < nch; c0 += B * 64) {
    uint4 lo[B], hi[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = c0 + b * 64 + lane, cc = c < nch ? c : nch - 1; /* cc: unused repeat */
      const uint32_t o = (uint32_t)((src0 + (size_t)cc * EPC) * TB);
      lo[b] = coh_b128(rs, o);
      hi[b] = coh_b128(rs, o + 16);
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = c0 + b * 64 + lane;
      if (c >= nch) continue;
      auto stale = [&]() {
        if (ACT == F32)
          return lo[b].y != tag || lo[b].w != tag || hi[b].y != tag || hi[b].w != tag;
        const uint32_t w0 = lo[b].x & lo[b].y & lo[b].z & lo[b].w & hi[b].x & hi[b].y & hi[b].z & hi[b].w;
        const uint32_t w1 = lo[b].x | lo[b].y | lo[b].z | lo[b].w | hi[b].x | hi[b].y | hi[b].z | hi[b].w;
        return (w0 >> 16) != tag || (w1 >> 16) != tag;
      };
      if (stale()) {
        const uint32_t o = (uint32_t)((src0 + (size_t)c * EPC) * TB);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (stale()) {
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_sleep(1);
          lo[b] = coh_b128(rs, o);
          hi[b] = coh_b128(rs, o + 16);
          if (__builtin_amdgcn_s_memrealtime() - t0 > sm.spin) {
            ok = false;
            break;
          }
        }
      }
      uint4 v;
      if (ACT == F32)
        v = make_uint4(lo[b].x, lo[b].z, hi[b].x, hi[b].z);
      else
        v = make_uint4((lo[b].x & 0xFFFFu) | (lo[b].y << 16), (lo[b].z & 0xFFFFu) | (lo[b].w << 16),
                       (hi[b].x & 0xFFFFu) | (hi[b].y << 16), (hi[b].z & 0xFFFFu) | (hi[b].w << 16));
      *reinterpret_cast<uint4*>(sm.big + off + (size_t)c * 16) = v;
    }
  }
  if (ACT == BF16 && mx) {
    /* MXFP8 round trip of the staged row (its down projection is MXFP4); the lanes read chunks
     * other lanes wrote, so the fences order the LDS accesses */
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
    for (int b = lane; b < inter / 32; b += 64) mx8_block_lds(sm.big + off + (size_t)b * 64);
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  }
  return __ballot(!ok) == 0ull;
}

/* One flow task: down rows h_lo .. h_lo + nr - 1 of the slice (nr <= kFlowRows; the rest repeat
 * the last row and are not stored) of item `item` against its staged hidden row; y into LDS. */
constexpr int kFlowRows = 8;

template <int ACT, int FMT>
__device__ __forceinline__ void flow_task(const Params& p, const Smem& sm, const DownGeo& g,
                                          const Mat& m, int e, int inter, int item, int h_lo,
                                          int nr, bool is_shared) {
  const int lane = threadIdx.x & 63;
  const size_t vb = row_vbytes(FMT, inter), sb = row_sbytes(FMT, inter);
  const uint8_t* vr[kFlowRows];
  const uint8_t* sr[kFlowRows];
#pragma unroll
  for (int c = 0; c < kFlowRows; ++c) {
    const size_t row = (size_t)e * p.H + g.h0 + h_lo + (c < nr ? c : nr - 1);
    vr[c] = m.down + row * vb;
    sr[c] = m.down_s ? m.down_s + row * sb : nullptr;
  }
  const int r = __builtin_ctz(uniform(sm.umask[item]));
  const void* arow[1] = {sm.big + (size_t)sm.voff[item][r] * 16};
  float acc[kFlowRows][1];
#pragma unroll
  for (int c = 0; c < kFlowRows; ++c) acc[c][0] = 0.0f;
  dot_rows<FMT, ACT, 1, kFlowRows, Fmt<FMT>::CH_DN>(vr, sr, inter, arow, 1u, acc);
  const int slot = is_shared ? p.K : sm.uslot[item][r];
#pragma unroll
  for (int c = 0; c < kFlowRows; ++c) {
    const float t = wave_sum(acc[c][0]);
    if (lane == 0 && c < nr) g.y[((size_t)(h_lo + c) * p.R + r) * (p.K + 1) + slot] = t;
  }
}

/* The down tasks of this wave (no workgroup barrier inside). Returns false when some item's
 * hidden row did not arrive in time (the caller reports once per workgroup). */
template <int ACT, int RFMT, int SFMT>
__device__ __forceinline__ bool ph_down_flow(const Params& p, Smem& sm, uint32_t htag) {
  const DownGeo g = down_geo(p, sm);
  const int nU = sm.nU, n_items = nU + (p.Is > 0 ? 1 : 0);
  const size_t ab = ACT == F32 ? 4 : 2;
  const int nq = (g.nh + kFlowRows - 1) / kFlowRows, ntask = n_items * nq;
  bool ok = true;
  for (;;) {
    const int d = claim(&sm.down_next);
    if (d >= ntask) break;
    const int k = d / nq, q = d % nq, it = down_item(p, sm, k);
    /* all lanes try; lane 0's attempt is the first, and its old value says who stages */
    const int st = __builtin_amdgcn_readfirstlane(atomicCAS(&sm.stage_state[k], 0, 1));
    if (st == 0) {
      const uint32_t off = flow_off(p, k, ab);
      const bool got =
          ok && flow_stage<ACT>(p, sm, it, off, htag, p.aq8 && (it != nU || SFMT == FP4));
      if ((threadIdx.x & 63) == 0) {
        sm.voff[it][__builtin_ctz(sm.umask[it])] = (uint16_t)(off / 16);
        __hip_atomic_store(&sm.stage_state[k], got ? 2 : 3, __ATOMIC_RELEASE,
                           __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      if (!got) ok = false;
    } else {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int v;
      while ((v = __builtin_amdgcn_readfirstlane(__hip_atomic_load(
                  &sm.stage_state[k], __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP))) == 1) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > 4ull * sm.spin) break;
      }
      if (v != 2) ok = false;
    }
    if (!ok) continue; /* drain the remaining tasks without work */
    const int h_lo = q * kFlowRows, nr = g.nh - h_lo < kFlowRows ? g.nh - h_lo : kFlowRows;
    if (it == nU)
      flow_task<ACT, SFMT>(p, sm, g, p.shared, 0, p.Is, it, h_lo, nr, true);
    else
      flow_task<ACT, RFMT>(p, sm, g, p.routed, sm.U[it], p.I, it, h_lo, nr, false);
  }
  return ok;
}

/* Items are processed in groups (down_item order); each group's hidden rows are staged in LDS,
 * then its tasks (item, kRG output rows of the slice) run one per wave. In the fused launch the
 * first group holds at most kFusedGroupItems items and every staging waits (bounded) for the
 * tags of this launch: no grid barrier separates gate/up from down, so a workgroup starts on the
 * first items while others still finish their gate/up rows. Before a group is staged, each wave
 * issues the weight loads of its first routed task (one row). */
constexpr int kFusedGroupItems = 3;

template <int ACT, int RFMT, int SFMT, int RMAX, bool FUSED>
__device__ __forceinline__ bool ph_down(const Params& p, Smem& sm, uint32_t htag) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const DownGeo g = down_geo(p, sm);
  const int nU = sm.nU, R = p.R;
  const size_t ab = ACT == F32 ? 4 : 2;
  const int nq = (g.nh + kRG - 1) / kRG;
  constexpr int CHR = Fmt<RFMT>::CH_DN;
  const int n_items = nU + (p.Is > 0 ? 1 : 0);
  WRegs<SFMT, kRG, Fmt<SFMT>::CH_DN> none;
  const Slice c = slice_of(p);
  SliceRegs sreg;
  if (FUSED) slice_prefetch<ACT>(p, c, sreg);
  int k0 = 0;
  while (k0 < n_items) {
    /* fused: a small first group (ready earliest), then groups as large as the staging area */
    const int k1 = down_group_end(p, sm, k0, ab, FUSED && k0 == 0 ? kFusedGroupItems : n_items);
    if (k0 > 0) __syncthreads(); /* the previous group's tasks are done with the staging area */
    stage_list(p, sm, k0, k1, ab);
    const int ntask = (k1 - k0) * nq;
    WRegs<RFMT, kRG, CHR> pre;
    bool have_pre = false;
    /* (one row, bf16 weights: the other formats' decode needs the registers) */
    if (RMAX == 1 && RFMT == BF16 && wave < ntask) {
      const int it = down_item(p, sm, k0 + wave / nq);
      if (it != nU) {
        const uint8_t* vr[kRG];
        const uint8_t* sr[kRG];
        down_rows<ACT, RFMT>(p, g, p.routed, sm.U[it], p.I, wave % nq, vr, sr);
        wregs_load(pre, vr, sr, p.I, 0);
        have_pre = true;
      }
    }
    if (!stage_copy<ACT>(p, sm, FUSED, htag, SFMT == FP4)) return false;
    if (FUSED && k0 == 0) {
      slice_store(p, c, sm, sreg);
      stamp(p, sm.trace_on != 0, 21);
      shake(p, sm, 21);
    }
    for (int t = wave; t < ntask; t += kWaves) {
      const int it = down_item(p, sm, k0 + t / nq), q = t % nq;
      if (it == nU)
        down_task<ACT, SFMT, RMAX>(p, sm, g, p.shared, 0, p.Is, it, q, true, none, false);
      else
        down_task<ACT, RFMT, RMAX>(p, sm, g, p.routed, sm.U[it], p.I, it, q, false, pre,
                                   have_pre && t == wave);
    }
    k0 = k1;
  }
  __syncthreads();
  down_combine<ACT>(p, sm, g);
  return true;
}

/* ------------------------------------------------------------------------------------------
 * Down phase of the fused launch at several rows. The shared expert is used by every row, so
 * its down rows cost R dot products per weight: each workgroup takes the shared rows of its own
 * hidden-position slice, as the per-slice down phase does. The routed down rows of all
 * distinct experts form one list of (expert, DG consecutive output rows) blocks, and workgroup
 * w takes an equal contiguous stretch of it, so a workgroup stages in LDS only the hidden rows
 * of the one or two experts its stretch touches (polling their tags) instead of all of them.
 * Every output y[r][slot][h] is published tagged; each workgroup then gathers the y values of
 * its slice and forms routed, shared and block as the per-slice down phase does. Each y value
 * comes from the same per-row dot product as there, so the results are the same bits. */

/* Down rows hb .. hb + nr - 1 of expert e (nr <= kRG; the rest repeat the last row). */
template <int FMT>
__device__ __forceinline__ void em_rows(const Params& p, const Mat& m, int e, int inter, int hb,
                                        int nr, const uint8_t* (&vr)[kRG],
                                        const uint8_t* (&sr)[kRG]) {
  const size_t vb = row_vbytes(FMT, inter), sb = row_sbytes(FMT, inter);
#pragma unroll
  for (int c = 0; c < kRG; ++c) {
    const size_t row = (size_t)e * p.H + hb + (c < nr ? c : nr - 1);
    vr[c] = m.down + row * vb;
    sr[c] = m.down_s ? m.down_s + row * sb : nullptr;
  }
}

/* Publishes y[r][slot][hb + c] (value bits | tag << 32), c < nr, for every row r that uses
 * item `item`, from the per-lane partial sums of the quad's rows. */
template <int RMAX>
__device__ __forceinline__ void em_store(const Params& p, const Smem& sm, float (&acc)[kRG][RMAX],
                                         uint32_t mask, int item, int hb, int nr, bool is_shared,
                                         int Kp, uint32_t tag) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (!(mask & (1u << r))) continue;
    const int slot = is_shared ? p.K : sm.uslot[item][r];
#pragma unroll
    for (int c = 0; c < kRG; ++c) {
      const float t = wave_sum(acc[c][r]);
      if (lane == c && c < nr)
        st_coh(p.y_part + ((size_t)r * Kp + slot) * p.H + hb + c,
               ((uint64_t)tag << 32) | __float_as_uint(t));
    }
  }
}

template <int RMAX>
__device__ __forceinline__ void em_arows(const Smem& sm, int item, uint32_t mask,
                                         const void* (&arow)[RMAX]) {
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
    arow[r] = sm.big + (size_t)((mask & (1u << r)) ? sm.voff[item][r] : 0) * 16;
}

/* One quad: down rows hb .. hb + nr - 1 of item `item` against its staged hidden rows. */
template <int ACT, int FMT, int RMAX>
__device__ __forceinline__ void em_down_task(const Params& p, const Smem& sm, const Mat& m, int e,
                                             int inter, int item, int hb, int nr, bool is_shared,
                                             int Kp, uint32_t tag) {
  constexpr int CH = Fmt<FMT>::CH_DN;
  const uint8_t* vr[kRG];
  const uint8_t* sr[kRG];
  em_rows<FMT>(p, m, e, inter, hb, nr, vr, sr);
  const uint32_t mask = uniform(sm.umask[item]);
  const void* arow[RMAX];
  em_arows<RMAX>(sm, item, mask, arow);
  float acc[kRG][RMAX];
#pragma unroll
  for (int c = 0; c < kRG; ++c)
#pragma unroll
    for (int r = 0; r < RMAX; ++r) acc[c][r] = 0.0f;
  dot_rows<FMT, ACT, RMAX, kRG, CH>(vr, sr, inter, arow, mask, acc);
  em_store<RMAX>(p, sm, acc, mask, item, hb, nr, is_shared, Kp, tag);
}

template <int NA, int DG>
__device__ __forceinline__ void dn_store(const Params& p, const Smem& sm, float (&acc)[DG][NA],
                                         int it, int hb, const int (&rows)[NA], int Kp,
                                         uint32_t tag);

/* DG down rows from hb of routed item `it` for the NA rows in `mask` (NA = its population),
 * streamed at once against their staged hidden rows; publishes y[r][slot][hb + c]. */
template <int ACT, int FMT, int NA, int DG>
__device__ __forceinline__ void dn_wide(const Params& p, const Smem& sm, int it, int hb,
                                        uint32_t mask, int Kp, uint32_t tag) {
  const int lane = threadIdx.x & 63;
  int rows[NA];
  uint32_t m = mask;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    rows[a] = __builtin_ctz(m);
    m &= m - 1u;
  }
  const int e = sm.U[it];
  const size_t vb = row_vbytes(FMT, p.I), sb = row_sbytes(FMT, p.I);
  const uint8_t* vr[DG];
  const uint8_t* sr[DG];
#pragma unroll
  for (int c = 0; c < DG; ++c) {
    const size_t row = (size_t)e * p.H + hb + c;
    vr[c] = p.routed.down + row * vb;
    sr[c] = p.routed.down_s ? p.routed.down_s + row * sb : nullptr;
  }
  const void* arow[NA];
#pragma unroll
  for (int a = 0; a < NA; ++a) arow[a] = sm.big + (size_t)sm.voff[it][rows[a]] * 16;
  float acc[DG][NA];
#pragma unroll
  for (int c = 0; c < DG; ++c)
#pragma unroll
    for (int a = 0; a < NA; ++a) acc[c][a] = 0.0f;
  dot_rows<FMT, ACT, NA, DG, Fmt<FMT>::CH_DN>(vr, sr, p.I, arow, (1u << NA) - 1u, acc);
  dn_store<NA, DG>(p, sm, acc, it, hb, rows, Kp, tag);
}

/* Publishes y[r][slot][hb + c] for the NA rows of item `it` from the per-lane partial sums of
 * its DG down rows (lane c stores row c: one coalesced store per row). */
template <int NA, int DG>
__device__ __forceinline__ void dn_store(const Params& p, const Smem& sm, float (&acc)[DG][NA],
                                         int it, int hb, const int (&rows)[NA], int Kp,
                                         uint32_t tag) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int a = 0; a < NA; ++a) {
    const int r = rows[a], slot = sm.uslot[it][r];
    float v = 0.0f;
#pragma unroll
    for (int c = 0; c < DG; ++c) {
      const float t = wave_sum(acc[c][a]);
      if (lane == c) v = t;
    }
    if (lane < DG)
      st_coh(p.y_part + ((size_t)r * Kp + slot) * p.H + hb + lane,
             ((uint64_t)tag << 32) | __float_as_uint(v));
  }
}

/* Routed down blocks at several rows for Q8_0 and MXFP4 rows that fit one chunk: blocks of
 * DG / 2 rows, software-pipelined over two register buffers (as the gate/up phase does); loads
 * past the last block go through an empty resource and read nothing. */
template <int ACT, int FMT, int RMAX>
__device__ __forceinline__ void dn_pipelined(const Params& p, Smem& sm, int qa, int qb, int nqi,
                                             int Kp, uint32_t tag) {
  constexpr int DGp = Wide<FMT>::DG / 2, CH = Fmt<FMT>::CH_DN;
  const int lane = threadIdx.x & 63;
  const size_t vb = row_vbytes(FMT, p.I), sb = row_sbytes(FMT, p.I);
  /* block q of DG rows = half-blocks 2 q and 2 q + 1 */
  const int ha = 2 * qa, hbnd = 2 * qb;
  auto next = [&]() -> int { return ha + claim(&sm.down_next); };
  auto load = [&](WRegs<FMT, DGp, CH>& W, int t) {
    const bool live = t < hbnd;
    const int tt = live ? t : ha;
    const int it = (tt / 2) / nqi, h0 = ((tt / 2) % nqi) * (2 * DGp) + (tt % 2) * DGp;
    const int e = sm.U[it];
#pragma unroll
    for (int c = 0; c < DGp; ++c) {
      const size_t row = (size_t)e * p.H + h0 + c;
      const __amdgpu_buffer_rsrc_t rv = row_rsrc(p.routed.down + row * vb, live ? vb : 0);
      const __amdgpu_buffer_rsrc_t rs = row_rsrc(p.routed.down_s + row * sb, live ? sb : 0);
#pragma unroll
      for (int k = 0; k < CH; ++k) wload<FMT>(rv, rs, k, lane, W.v[c][k], W.sc[c][k]);
    }
  };
  auto compute = [&](const WRegs<FMT, DGp, CH>& W, int t) {
    const int it = (t / 2) / nqi, h0 = ((t / 2) % nqi) * (2 * DGp) + (t % 2) * DGp;
    const uint32_t mask = uniform(sm.umask[it]);
    const int n = __popc(mask);
    if (n == 1) {
      const int rows[1] = {__builtin_ctz(mask)};
      const void* arow[1] = {sm.big + (size_t)sm.voff[it][rows[0]] * 16};
      float acc[DGp][1];
#pragma unroll
      for (int c = 0; c < DGp; ++c) acc[c][0] = 0.0f;
      wregs_dot<FMT, ACT, 1, DGp, CH>(W, p.I, 0, arow, 1u, acc);
      dn_store<1, DGp>(p, sm, acc, it, h0, rows, Kp, tag);
    } else if (n == 2) {
      const int rows[2] = {__builtin_ctz(mask), __builtin_ctz(mask & (mask - 1u))};
      const void* arow[2] = {sm.big + (size_t)sm.voff[it][rows[0]] * 16,
                             sm.big + (size_t)sm.voff[it][rows[1]] * 16};
      float acc[DGp][2];
#pragma unroll
      for (int c = 0; c < DGp; ++c) acc[c][0] = acc[c][1] = 0.0f;
      wregs_dot<FMT, ACT, 2, DGp, CH>(W, p.I, 0, arow, 3u, acc);
      dn_store<2, DGp>(p, sm, acc, it, h0, rows, Kp, tag);
    } else {
      /* three or more rows (rare): the general loop, which reads its rows again */
#pragma unroll 1
      for (int h = h0; h < h0 + DGp; h += kRG)
        em_down_task<ACT, FMT, RMAX>(p, sm, p.routed, sm.U[it], p.I, it, h, kRG, false, Kp, tag);
    }
  };
  WRegs<FMT, DGp, CH> A, B;
  int tA = next();
  load(A, tA);
  while (tA < hbnd) {
    const int tB = next();
    load(B, tB);
    compute(A, tA);
    if (tB >= hbnd) break;
    tA = next();
    load(A, tA);
    compute(B, tB);
  }
}

/* The routed blocks [qa, qb) of the staged group (block q: DG down rows from (q % nqi) DG of
 * the expert q / nqi), claimed one at a time by the waves. When one or two rows use the expert,
 * the DG rows stream at once against their hidden rows; otherwise they go kRG at a time for
 * every row that uses it. sm.down_next must be zero and visible to every wave. */
template <int ACT, int FMT, int RMAX>
__device__ __forceinline__ void em_routed_blocks(const Params& p, Smem& sm, int qa, int qb,
                                                 int nqi, int Kp, uint32_t tag) {
  constexpr int DG = Wide<FMT>::DG;
  if constexpr (FMT == Q8 || FMT == FP4) {
    if (p.I <= 64 * Fmt<FMT>::EL * Fmt<FMT>::CH_DN) {
      dn_pipelined<ACT, FMT, RMAX>(p, sm, qa, qb, nqi, Kp, tag);
      return;
    }
  }
  for (int q = qa + claim(&sm.down_next); q < qb; q = qa + claim(&sm.down_next)) {
    const int it = q / nqi, hb = (q % nqi) * DG;
    const uint32_t mask = uniform(sm.umask[it]);
    const int n = __popc(mask);
    if (n == 1) {
      dn_wide<ACT, FMT, 1, DG>(p, sm, it, hb, mask, Kp, tag);
    } else if (n == 2) {
      dn_wide<ACT, FMT, 2, DG>(p, sm, it, hb, mask, Kp, tag);
    } else {
#pragma unroll 1
      for (int h = hb; h < hb + DG; h += kRG)
        em_down_task<ACT, FMT, RMAX>(p, sm, p.routed, sm.U[it], p.I, it, h, kRG, false, Kp, tag);
    }
  }
}

/* Gathers the tagged y values of the slice (y_part is [R][Kp][H]) into LDS at dst as floats,
 * [nh][R][Kp], polling (bounded) until each carries `tag`. Whole workgroup; returns false
 * (uniform) on expiry. */
__device__ __forceinline__ bool em_gather_y(const Params& p, Smem& sm, int h0, int nh, int Kp,
                                            float* dst, uint32_t tag) {
  const int tid = threadIdx.x;
  const int n = nh * p.R * Kp;
  const __amdgpu_buffer_rsrc_t yr = coh_region(p.y_part, (size_t)p.R * Kp * p.H * 8);
  int ok = 1;
  constexpr int B = 4;
  for (int v0 = 0; v0 < n; v0 += B * kBlock) {
    uint2 b[B];
    uint32_t off[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int v = v0 + k * kBlock + tid; /* v = (r Kp + slot) nh + hl */
      const int vv = v < n ? v : n - 1; /* past the end: a repeated value, unused */
      off[k] = (uint32_t)(((size_t)(vv / nh) * p.H + h0 + vv % nh) * 8);
      b[k] = coh_b64(yr, off[k]);
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int v = v0 + k * kBlock + tid;
      if (v >= n) continue;
      if (b[k].y != tag) {
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        while (b[k].y != tag) {
          asm volatile("" ::: "memory");
          __builtin_amdgcn_s_sleep(1);
          b[k] = coh_b64(yr, off[k]);
          if (__builtin_amdgcn_s_memrealtime() - t0 > sm.spin) {
            ok = 0;
            break;
          }
        }
      }
      const int rs = v / nh, hl = v % nh; /* rs = r Kp + slot */
      dst[((size_t)hl * p.R + rs / Kp) * Kp + rs % Kp] = __uint_as_float(b[k].x);
    }
  }
  const bool all = __syncthreads_and(ok) != 0;
  if (!all && tid == 0) report_timeout(p, PH_GATEUP);
  return all;
}

/* Relative cost of a routed down block by the number of rows that use its expert: the wide
 * path streams the rows once for one or two rows; more rows take the general path. */
__device__ __forceinline__ uint32_t em_cost(int n) { return n == 1 ? 2u : n == 2 ? 3u : 2u + n; }

/* Workgroup b's stretch [q0, q1) of the nU * nqi routed blocks: the list is cut at the blocks
 * whose cost prefix first reaches b / grid and (b + 1) / grid of the total, so every workgroup
 * gets the same cost and the stretches tile the list. One wave, one lane per item
 * (nU <= kMaxUnion = 128: two items per lane), prefix sums and ballots; 32-bit arithmetic (the
 * total cost is at most 10 nqi nU, and times the grid it stays below 2^32). */
__device__ __forceinline__ void em_stretch(const Smem& sm, int nqi, int& q0, int& q1) {
  static_assert(kMaxUnion <= 128, "em_stretch covers two items per lane");
  const int nU = sm.nU, G = gridDim.x, b = blockIdx.x, lane = threadIdx.x & 63;
  uint32_t w[2], incl[2], carry = 0u;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = lane + 64 * h;
    w[h] = u < nU ? em_cost(__popc(sm.umask[u])) : 0u;
    uint32_t x = w[h] * (uint32_t)nqi;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t t = __shfl_up(x, d);
      if (lane >= d) x += t;
    }
    incl[h] = carry + x;
    carry += __shfl(x, 63);
  }
  const uint32_t W = carry;
  const uint32_t c0 = W * (uint32_t)b / (uint32_t)G, c1 = W * (uint32_t)(b + 1) / (uint32_t)G;
  /* the first item whose inclusive prefix exceeds c; the block is u nqi + ceil((c - P) / w) */
  auto cut = [&](uint32_t c) -> int {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int u = lane + 64 * h;
      const uint64_t hit = __ballot(u < nU && c < incl[h]);
      if (hit != 0ull) {
        const int src = (int)__builtin_ctzll(hit);
        const uint32_t wu = (uint32_t)__shfl((int)w[h], src);
        const uint32_t P = (uint32_t)__shfl((int)incl[h], src) - wu * (uint32_t)nqi;
        return (64 * h + src) * nqi + (int)((c - P + wu - 1u) / wu);
      }
    }
    return nU * nqi;
  };
  q0 = cut(c0);
  q1 = cut(c1);
}

/* After the plan, by wave 0 while the other waves start the gate/up phase (which leaves these
 * LDS fields alone): the workgroup's down stretch, the end of its first staged group and that
 * group's staging list, so that the down phase starts with the copy. The other waves read them
 * after the barrier at the start of ph_down_em. */
template <int ACT, int RFMT>
__device__ __forceinline__ void em_prepare(const Params& p, Smem& sm) {
  const int nqi = p.H / Wide<RFMT>::DG, off = p.Is > 0 ? 1 : 0;
  const size_t ab = ACT == F32 ? 4 : 2;
  int q0, q1;
  em_stretch(sm, nqi, q0, q1);
  const int u = q0 / nqi, uend = q1 > q0 ? (q1 - 1) / nqi + 1 : u;
  const bool has_sh = p.Is > 0 && slice_of(p).nh > 0;
  const int u1 = u < uend ? down_group_end(p, sm, u + off, ab, uend - u,
                                           has_sh ? (size_t)p.R * p.Is * ab : 0, has_sh ? p.R : 0) -
                                off
                          : u;
  stage_list_wave(p, sm, u + off, u1 + off, ab, has_sh);
  if ((threadIdx.x & 63) == 0) {
    sm.em_q0 = q0;
    sm.em_q1 = q1;
    sm.em_u1 = u1;
    sm.down_next = 0;
  }
}

template <int ACT, int RFMT, int SFMT, int RMAX>
__device__ __forceinline__ bool ph_down_em(const Params& p, Smem& sm, uint32_t htag) {
  const int tid = threadIdx.x, wave = tid >> 6, R = p.R;
  const uint32_t tag = (uint32_t)(sm.epoch + 1);
  const int nU = sm.nU, Kp = p.K + (p.Is > 0 ? 1 : 0), off = p.Is > 0 ? 1 : 0;
  const size_t ab = ACT == F32 ? 4 : 2;
  const int nqi = p.H / Wide<RFMT>::DG; /* routed down blocks per expert */
  const Slice c = slice_of(p);
  SliceRegs sreg;
  slice_prefetch<ACT>(p, c, sreg);
  /* this workgroup's stretch of routed blocks, from em_prepare (wave 0): every wave is done
   * with its gate/up rows after this barrier, and sees what wave 0 wrote */
  __syncthreads();
  const int q0 = sm.em_q0, q1 = sm.em_q1;
  int u = q0 / nqi;
  const int uend = q1 > q0 ? (q1 - 1) / nqi + 1 : u;
  /* the first staged group holds the shared expert's hidden rows (for this workgroup's slice of
   * its down rows, complete since before the select) and as many routed items as fit beside
   * them; the waves take the shared rows first, then claim routed blocks */
  const bool has_sh = p.Is > 0 && c.nh > 0;
  bool first = true;
  while (u < uend || (first && has_sh)) {
    const bool with_sh = first && has_sh;
    int u1;
    if (first) {
      u1 = sm.em_u1; /* listed by em_prepare; sm.down_next is zero */
    } else {
      u1 = u < uend ? down_group_end(p, sm, u + off, ab, uend - u) - off : u;
      __syncthreads(); /* the previous items' tasks are done with the staging area */
      if (tid == 0) sm.down_next = 0; /* visible after stage_list's barrier */
      stage_list(p, sm, u + off, u1 + off, ab, false);
    }
    if (!stage_copy<ACT>(p, sm, true, htag, SFMT == FP4)) return false;
    if (first) {
      slice_store(p, c, sm, sreg);
      stamp(p, sm.trace_on != 0, 21);
      shake(p, sm, 21);
      first = false;
    }
    if (with_sh) {
      for (int t = wave; t * kRG < c.nh; t += kWaves) {
        const int nr = c.nh - t * kRG < kRG ? c.nh - t * kRG : kRG;
        em_down_task<ACT, SFMT, RMAX>(p, sm, p.shared, 0, p.Is, nU, c.h0 + t * kRG, nr, true,
                                      Kp, tag);
      }
      stamp(p, sm.trace_on != 0, 20);
      shake(p, sm, 20);
    }
    const int qa = q0 > u * nqi ? q0 : u * nqi, qb = q1 < u1 * nqi ? q1 : u1 * nqi;
    if (qa < qb) em_routed_blocks<ACT, RFMT, RMAX>(p, sm, qa, qb, nqi, Kp, tag);
    u = u1;
  }
  if (first) slice_store(p, c, sm, sreg);
  stamp(p, sm.trace_on != 0, 10);
  shake(p, sm, 10);
  const DownGeo g = down_geo(p, sm);
  if (!em_gather_y(p, sm, g.h0, g.nh, Kp, g.y, tag)) return false;
  for (int q = tid; q < g.nh * R; q += kBlock) {
    const int hl = q / R, r = q % R;
    const float* y = g.y + ((size_t)hl * R + r) * Kp;
    float routed = 0.0f;
    for (int j = 0; j < p.K; ++j) routed = fmaf(sm.sel_w[r][j], y[j], routed);
    const float shared = p.Is > 0 ? act_round<ACT>(y[p.K]) : 0.0f;
    const float blk = act_round<ACT>(routed + shared);
    const size_t o = (size_t)r * p.H + g.h0 + hl;
    if (p.routed_out) p.routed_out[o] = routed;
    if (p.shared_out) act_st<ACT>(p.shared_out, o, shared);
    if (p.block) act_st<ACT>(p.block, o, blk);
    g.blk[q] = blk;
  }
  __syncthreads();
  return true;
}

/* ------------------------------------------------------------------------------------------
 * Phase: expand + carry for the workgroup's slice [ds4 HC fusion commit: post/comb expand +
 * BF16; SGLang fused post/pre page: bf16 residual materialisation + next pre-norm GEMM
 * partials + RMS square-sum partials]. new[i][h] = bf16(post_i block[h] + sum_j comb[i][j]
 * state_j[h]). The carry is taken on the rounded new state: every workgroup writes its 25 R
 * partial sums, each tagged with the launch epoch; output q of the carry is then summed over
 * the workgroups in a fixed order (reduce_carry). */
/* Carry output q (row q / 25, output q % 25) = sum over the grid's tagged partials, in the
 * order: lane L adds workgroups L, L + 64, ... in turn, then a wave sum. With check, waits
 * (bounded) until every partial carries `tag`. Whole workgroup; returns false on expiry. */
__device__ __forceinline__ bool reduce_carry(const Params& p, Smem& sm, int q, bool check,
                                             uint32_t tag) {
  const int tid = threadIdx.x, G = gridDim.x;
  const __amdgpu_buffer_rsrc_t cp =
      coh_region(p.carry_part, (size_t)p.R * kNCarry * G * 8);
  int ok = 1;
  for (int w = tid; w < G; w += kBlock) {
    const uint32_t off = (uint32_t)(((size_t)q * G + w) * 8);
    uint2 v = coh_b64(cp, off);
    if (check && v.y != tag) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (v.y != tag) {
        __builtin_amdgcn_s_sleep(2);
        v = coh_b64(cp, off);
        if (__builtin_amdgcn_s_memrealtime() - t0 > sm.spin) {
          ok = 0;
          break;
        }
      }
    }
    sm.cred[w] = __uint_as_float(v.x);
  }
  const bool all = __syncthreads_and(ok) != 0;
  if (!all && tid == 0) report_timeout(p, PH_END);
  if (tid < 64) {
    float t = 0.0f;
    for (int w = tid; w < G; w += 64) t += sm.cred[w];
    t = wave_sum(t);
    if (tid == 0 && all) {
      p.carry_out[q] = t;
      if (p.carry_ws) p.carry_ws[q] = t;
    }
  }
  __syncthreads();
  return all;
}

/* When the new state overwrites the input (state_out == state), no workgroup may store its
 * slice before every workgroup has read the whole input (mix partials and collapse): each
 * workgroup publishes the launch tag in pre_done[wg] after its collapse, and the expand waits
 * (bounded) until all of them carry it. Whole workgroup; returns false on expiry. */
/* Every carry output by the last workgroup of the per-stage expand to arrive (all partials are
 * complete): wave w takes outputs q = w, w + 8, ..., with reduce_carry's arithmetic (lane L adds
 * workgroups L, L + 64, ... in turn, then the wave sum), so the per-stage and fused launches
 * give the same bits; the outputs proceed side by side instead of one workgroup reduction
 * (two barriers and a round of loads) after another. */
__device__ __forceinline__ void reduce_carry_waves(const Params& p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, G = gridDim.x;
  const int NQ = p.R * kNCarry;
  constexpr int QB = 4, KW = (kMaxGrid + 63) / 64; /* outputs per round, loads per output */
  const __amdgpu_buffer_rsrc_t cp = coh_region(p.carry_part, (size_t)NQ * G * 8);
  for (int q0 = wave; q0 < NQ; q0 += kWaves * QB) {
    /* all loads of the round first (past the end: a repeated valid address, unused) */
    uint32_t v[QB][KW];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int q = q0 + b * kWaves < NQ ? q0 + b * kWaves : q0;
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        if (64 * k >= G) break; /* uniform */
        const int w = lane + 64 * k < G ? lane + 64 * k : lane;
        v[b][k] = coh_b64(cp, (uint32_t)(((size_t)q * G + w) * 8)).x;
      }
    }
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const int q = q0 + b * kWaves;
      if (q >= NQ) break;
      float t = 0.0f;
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        if (64 * k >= G) break; /* uniform */
        if (lane + 64 * k < G) t += __uint_as_float(v[b][k]);
      }
      t = wave_sum(t);
      if (lane == 0) {
        p.carry_out[q] = t;
        if (p.carry_ws) p.carry_ws[q] = t;
      }
    }
  }
}

__device__ __forceinline__ bool wait_pre_done(const Params& p, Smem& sm, uint32_t tag) {
  const int G = gridDim.x;
  const __amdgpu_buffer_rsrc_t rs = coh_region(p.pre_done, (size_t)G * 8);
  int ok = 1;
  for (int w = threadIdx.x; w < G; w += kBlock) {
    uint2 v = coh_b64(rs, (uint32_t)w * 8u);
    if (v.x != tag) {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (v.x != tag) {
        __builtin_amdgcn_s_sleep(2);
        v = coh_b64(rs, (uint32_t)w * 8u);
        if (__builtin_amdgcn_s_memrealtime() - t0 > sm.spin) {
          ok = 0;
          break;
        }
      }
    }
  }
  const bool all = __syncthreads_and(ok) != 0;
  if (!all && threadIdx.x == 0) report_timeout(p, PH_END);
  return all;
}

template <int ACT, int RMAX, bool FUSED>
__device__ __forceinline__ void ph_expand(const Params& p, Smem& sm, const float* blk) {
  const int tid = threadIdx.x;
  if (FUSED && p.state_out == p.state && !wait_pre_done(p, sm, (uint32_t)(sm.epoch + 1)))
    return;
  const Slice c = slice_of(p);
  const int h0 = c.h0, nh = c.nh;
  const int R = p.R, H = p.H, n = 4 * H;
  /* new state: one thread per hidden position reads all 4 streams and writes all 4, so the
   * output may alias the input */
  float* nvb = reinterpret_cast<float*>(sm.big); /* [nh][R][4] */
  for (int hl = tid; hl < nh; hl += kBlock) {
    const int h = h0 + hl;
    for (int r = 0; r < R; ++r) {
      const size_t sb = (size_t)r * n + h;
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        sv[i] = c.lds ? sm.sslice[(r * 4 + i) * kSliceMax + hl]
                      : act_ld<ACT>(p.state, sb + (size_t)i * H);
      const float b = blk[hl * R + r];
      float nv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = sm.post[r][i] * b;
        a = fmaf(sm.comb[r][4 * i + 0], sv[0], a);
        a = fmaf(sm.comb[r][4 * i + 1], sv[1], a);
        a = fmaf(sm.comb[r][4 * i + 2], sv[2], a);
        a = fmaf(sm.comb[r][4 * i + 3], sv[3], a);
        nv[i] = act_round<ACT>(a);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        act_st<ACT>(p.state_out, sb + (size_t)i * H, nv[i]);
        nvb[(hl * R + r) * 4 + i] = nv[i];
      }
    }
  }
  if (p.w_mix_next == nullptr) return;
  stamp(p, sm.trace_on != 0, 12);
  shake(p, sm, 12);
  __syncthreads();
  /* carry partials of this slice: cp[j][r][hl] = sum_i W_next[j][i H + h] new[r][i] (j < 24),
   * cp[24][r][hl] = sum_i new[r][i]^2; then summed over hl in order */
  float* cpl = nvb + (size_t)nh * R * 4; /* [25][R][nh] */
  for (int q = tid; q < nh * kNCarry; q += kBlock) {
    const int hl = q % nh, j = q / nh, h = h0 + hl;
    float w[4];
    if (j < kNMix) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = c.lds ? sm.wnext[(j * 4 + i) * kSliceMax + hl]
                     : p.w_mix_next[(size_t)j * n + (size_t)i * H + h];
    }
    for (int r = 0; r < R; ++r) {
      const float* v = nvb + (hl * R + r) * 4;
      float a;
      if (j < kNMix) {
        a = w[0] * v[0];
        a = fmaf(w[1], v[1], a);
        a = fmaf(w[2], v[2], a);
        a = fmaf(w[3], v[3], a);
      } else {
        a = v[0] * v[0];
        a = fmaf(v[1], v[1], a);
        a = fmaf(v[2], v[2], a);
        a = fmaf(v[3], v[3], a);
      }
      cpl[((size_t)j * R + r) * nh + hl] = a;
    }
  }
  __syncthreads();
  const uint32_t tag = FUSED ? (uint32_t)(sm.epoch + 1) : 0u;
  if (tid < R * kNCarry) {
    const int j = tid % kNCarry, r = tid / kNCarry;
    const float* cl = cpl + ((size_t)j * R + r) * nh;
    float t = 0.0f;
    for (int hl = 0; hl < nh; ++hl) t += cl[hl];
    /* partial (q = tid, workgroup) at [q][grid]: value in the low word, tag in the high word */
    st_coh(reinterpret_cast<uint64_t*>(p.carry_part) + (size_t)tid * gridDim.x + blockIdx.x,
           ((uint64_t)tag << 32) | __float_as_uint(t));
  }
  if (FUSED) {
    for (int q = blockIdx.x; q < R * kNCarry; q += gridDim.x)
      if (!reduce_carry(p, sm, q, true, tag)) return;
  } else if (arrive_last_single(p, sm)) {
    reduce_carry_waves(p);
  }
}

/* ------------------------------------------------------------------------------------------
 * Kernels */

template <int ACT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_mix_partials(Params p) {
  ph_mix_partials<ACT, RMAX>(p, 0u, false);
}

template <int ACT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_hc_pre(Params p) {
  __shared__ Smem sm;
  if (threadIdx.x == 0) sm.trace_on = 0;
  load_pre_params<ACT>(p, sm);
  __syncthreads();
  ph_hc_pre<ACT, RMAX>(p, sm, true, false, 0u);
  ph_sinkhorn(p, sm, true);
}

template <int ACT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_router_logits(Params p) {
  __shared__ Smem sm;
  if (threadIdx.x == 0) sm.trace_on = 0;
  load_act_rows<ACT>(p.norm_in, p.R, p.H, sm);
  RouterRegs none;
  ph_router<ACT, RMAX, false>(p, sm, none, 0u, false);
}

template <int UNUSED>
__global__ void __launch_bounds__(kBlock) k_select(Params p) {
  __shared__ Smem sm;
  if (threadIdx.x == 0) sm.trace_on = 0;
  load_bias(p, sm);
  __syncthreads();
  ph_select(p, sm, true, false, 0u);
}

template <int ACT, int RFMT, int SFMT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_gateup(Params p) {
  __shared__ Smem sm;
  if (threadIdx.x == 0) {
    sm.trace_on = 0;
    sm.routed_next = 0; /* read after ph_plan's barrier */
  }
  load_act_rows<ACT>(p.norm_in, p.R, p.H, sm);
  load_selection(p, sm);
  ph_plan(p, sm);
  /* MXFP8 activations: the MXFP4 experts see the round trip of the norm rows, the others the
   * rows themselves (the routed experts are MXFP4 in this mode) */
  if (p.aq8 && SFMT == FP4) {
    mx8_act_rows<ACT>(p, sm);
    __syncthreads();
  }
  ph_gateup_shared<ACT, SFMT, RMAX>(p, sm);
  if (p.aq8 && SFMT != FP4) {
    __syncthreads();
    mx8_act_rows<ACT>(p, sm);
    __syncthreads();
  }
  ph_gateup_routed<ACT, RFMT, RMAX>(p, sm, 0u, false);
}

template <int ACT, int RFMT, int SFMT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_down(Params p) {
  __shared__ Smem sm;
  if (threadIdx.x == 0) sm.trace_on = 0;
  load_selection(p, sm);
  ph_plan(p, sm);
  ph_down<ACT, RFMT, SFMT, RMAX, false>(p, sm, 0u);
}

template <int ACT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_expand(Params p) {
  __shared__ Smem sm;
  if (threadIdx.x == 0) sm.trace_on = 0;
  const int tid = threadIdx.x;
  if (tid < p.R * 4) sm.post[tid / 4][tid % 4] = p.post_in[tid];
  if (tid < p.R * 16) sm.comb[tid / 16][tid % 16] = p.comb_in[tid];
  const int hs = (p.H + p.nslice - 1) / p.nslice, h0 = blockIdx.x * hs;
  int nh = p.H - h0 < hs ? p.H - h0 : hs;
  if (nh < 0) nh = 0;
  float* blk = reinterpret_cast<float*>(sm.big + kLdsHidBytes);
  {
    const Slice c = slice_of(p);
    SliceRegs sreg;
    slice_prefetch<ACT>(p, c, sreg);
    slice_store(p, c, sm, sreg);
  }
  for (int q = tid; q < nh * p.R; q += kBlock) {
    const int hl = q / p.R, r = q % p.R;
    blk[q] = act_ld<ACT>(p.block_in, (size_t)r * p.H + h0 + hl);
  }
  __syncthreads();
  ph_expand<ACT, RMAX, false>(p, sm, blk);
}

/* The whole layer half in one persistent launch (one workgroup per compute unit), with no grid
 * barrier: every value one workgroup hands to another carries this launch's tag and the reader
 * polls for it (bounded).
 *   mix partials (tagged) | pre side in every workgroup (gathers the partials) | router logits
 *   (tagged) beside Sinkhorn | select of every row (gathers the parts) while free waves claim
 *   the shared expert's gate/up rows | plan | routed gate/up strided over the grid (tagged
 *   hidden rows) | down in groups staged as their hidden rows arrive, block | expand + carry
 *   partials (tagged; workgroup q sums carry output q over the grid).
 * Trace slots: 0 start, 1 mix partials, 2 pre-side inputs ready, 3 pre side, 4 router,
 * 5 shared gate/up, 6 select rows, 7 select finished, 8 plan, 9 routed gate/up,
 * 10 routed down (several rows), 11 down + block, 12 expand, 13 carry; 14-18 inside the pre
 * side, 19 select scores, 20 shared down (several rows), 21 first down group staged, 22 router
 * start (first router wave), 23 router logits stored, 24 logits gathered, 25-31 gate/up end of
 * waves 1-7. */
template <int ACT, int RFMT, int SFMT, int RMAX>
__global__ void __launch_bounds__(kBlock, 1) k_ffn_layer(Params p) {
  __shared__ Smem sm;
  bar_setup(p, sm);
  __syncthreads();
  const bool tr = sm.trace_on != 0;
  stamp(p, tr, 0);
  shake(p, sm, 0);
  /* values exchanged between workgroups carry this launch's tag: no grid barrier */
  const uint32_t tag = (uint32_t)(sm.epoch + 1);
  RouterRegs rpre;
  int t0 = 0; /* waves below t0 / 64 have a mix-partial task; the others copy the pre inputs */
  if (!p.carry_in) {
    const int ntask = ((4 * p.H + kMixChunk - 1) / kMixChunk) * p.R * (kNMix / kMixGroup);
    const int busy = ntask > (int)blockIdx.x ? (ntask - (int)blockIdx.x + (int)gridDim.x - 1) / (int)gridDim.x : 0;
    t0 = busy < kWaves ? busy * 64 : 0;
    ph_mix_partials<ACT, RMAX>(p, tag, sm.skip_phase == PH_MIX);
    stamp(p, tr, 1);
    shake(p, sm, 1);
  }
  router_prefetch(p, rpre);
  load_pre_params<ACT>(p, sm, t0);
  load_bias(p, sm);
  for (int i = threadIdx.x; i <= kMaxUnion; i += kBlock) sm.stage_state[i] = 0;
  if (threadIdx.x == 0) {
    sm.sel_ok = 1;
    sm.lg_ready = 0;
    sm.plan_ready = 0;
    sm.shared_next = 0;
    sm.routed_next = 0;
    sm.down_next = 0;
  }
  __syncthreads();
  stamp(p, tr, 2);
  shake(p, sm, 2);
  if (!p.carry_in) warm_state<ACT>(p, sm);
  if (!ph_hc_pre<ACT, RMAX>(p, sm, blockIdx.x == 0, true, tag)) return;
  if (p.state_out == p.state) { /* in place: tell the expands this workgroup is done reading */
    __syncthreads();
    if (threadIdx.x == 0) st_coh(p.pre_done + blockIdx.x, (uint64_t)tag);
  }
  stamp(p, tr, 3);
  shake(p, sm, 3);
  /* router logits (waves 1 ..), then the select (waves 0 .. R - 1, polling the tagged logits)
   * beside the shared expert's gate/up rows, claimed by whichever waves are free */
  ph_router<ACT, RMAX, true>(p, sm, rpre, tag, sm.skip_phase == PH_ROUTER);
  stamp(p, tr, 4);
  shake(p, sm, 4);
  ph_sinkhorn(p, sm, blockIdx.x == 0); /* comb is needed only by the expand */
  /* MXFP8 activations with an MXFP4 shared expert: every expert sees the round trip of the norm
   * rows, so it replaces them once the router has read them */
  if (p.aq8 && SFMT == FP4) {
    __syncthreads();
    mx8_act_rows<ACT>(p, sm);
    __syncthreads();
  }
  /* hidden rows carry a 16-bit tag of this launch (never 0, the value the init leaves) */
  const uint32_t htag = (uint32_t)(sm.epoch % 65535u) + 1u;
  const bool hskip = sm.skip_phase == PH_GATEUP; /* fault injection: store no hidden rows */
  if (RMAX == 1) {
    /* one row: wave 0 selects while the other waves take the shared expert's rows, which they
     * start once wave 0 has gathered the logits: their loads would otherwise queue ahead of its
     * polls (bounded wait; wave 0 sets the flag whether or not the logits arrived) */
    if (threadIdx.x < 64) {
      /* wave 0 selects, finishes the select and builds the plan with pick j held in lane j,
       * without waiting for the other waves' shared rows, then publishes the plan through
       * sm.plan_ready (1 ready, 2 the logits did not arrive) */
      int e_l = 0;
      float s_l = 0.0f;
      const bool ok =
          p.E <= 256 ? select_row<4>(p, sm, 0, blockIdx.x == 0, true, tag, e_l, s_l)
                     : select_row<kMaxExperts / 64>(p, sm, 0, blockIdx.x == 0, true, tag, e_l, s_l);
      if (!ok && threadIdx.x == 0) report_timeout(p, PH_ROUTER);
      stamp(p, tr, 7);
      if (ok) finish_one_row(p, sm, e_l, s_l, blockIdx.x == 0);
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
      if (threadIdx.x == 0)
        __hip_atomic_store(&sm.plan_ready, ok ? 1 : 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      stamp(p, tr, 8);
    } else {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(&sm.lg_ready, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0 &&
             __builtin_amdgcn_s_memrealtime() - t0 <= sm.spin)
        __builtin_amdgcn_s_sleep(2);
    }
    stamp(p, tr, 6);
    ph_gateup_shared_claim<ACT, SFMT, RMAX>(p, sm, htag, hskip);
    stamp(p, tr, 5);
    /* bounded wait for the plan (usually ready by now). Wave 0 sets the flag at most a few
     * microseconds after its own bounded gather ends, so with twice the limit every wave sees
     * the same value; on a failed select all waves return. */
    {
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      int st;
      while ((st = __hip_atomic_load(&sm.plan_ready, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP)) == 0 &&
             __builtin_amdgcn_s_memrealtime() - t0 <= 2ull * sm.spin)
        __builtin_amdgcn_s_sleep(1);
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      if (st != 1) return;
    }
    /* MXFP8 activations, shared expert not MXFP4: the routed rows see the round trip of the
     * norm row, after every wave is done with the shared rows */
    if (p.aq8 && SFMT != FP4) {
      __syncthreads();
      mx8_act_rows<ACT>(p, sm);
      __syncthreads();
    }
    shake(p, sm, 8);
  } else {
    /* several rows: most waves select, so the shared rows go first, while the logits arrive */
    ph_gateup_shared_claim<ACT, SFMT, RMAX>(p, sm, htag, hskip);
    stamp(p, tr, 5);
    select_rows(p, sm, blockIdx.x == 0, true, tag);
    stamp(p, tr, 6);
  }
  if constexpr (RMAX > 1) {
    __syncthreads();
    if (!select_finish(p, sm, blockIdx.x == 0)) return;
    stamp(p, tr, 7);
    shake(p, sm, 7);
    /* MXFP8 activations, shared expert not MXFP4: the round trip of the norm rows for the
     * routed gate/up (every wave is done with the shared rows; ph_plan's barrier follows) */
    if (p.aq8 && SFMT != FP4) mx8_act_rows<ACT>(p, sm);
    ph_plan(p, sm);
    /* wave 0 prepares the down phase while the others start the gate/up rows; it reads the
     * plan only after the plan's barrier (lanes of one wave exchange LDS values only across a
     * barrier or fence: without one the compiler may schedule one lane's load before another
     * lane's store) */
    if (threadIdx.x < 64) em_prepare<ACT, RFMT>(p, sm);
    stamp(p, tr, 8);
    shake(p, sm, 8);
  }
  ph_gateup_routed<ACT, RFMT, RMAX>(p, sm, htag, hskip);
  stamp(p, tr, 9);
  shake(p, sm, 9);
  /* end of each other wave's gate/up rows: slots 25 .. 31 */
  if (tr && (threadIdx.x & 63) == 0 && threadIdx.x > 0)
    p.trace[(size_t)blockIdx.x * kTraceSlots + 24 + (threadIdx.x >> 6)] =
        __builtin_amdgcn_s_memrealtime();
  if constexpr (RMAX > 1) {
    if (!ph_down_em<ACT, RFMT, SFMT, RMAX>(p, sm, htag)) return;
  } else {
    if (flow_fits(p, sm, ACT == F32 ? 4 : 2)) {
      const Slice c = slice_of(p);
      SliceRegs sreg;
      slice_prefetch<ACT>(p, c, sreg);
      const bool ok = ph_down_flow<ACT, RFMT, SFMT>(p, sm, htag);
      if (__syncthreads_or(!ok)) {
        if (threadIdx.x == 0) report_timeout(p, PH_GATEUP);
        return;
      }
      slice_store(p, c, sm, sreg);
      down_combine<ACT>(p, sm, down_geo(p, sm));
    } else if (!ph_down<ACT, RFMT, SFMT, RMAX, true>(p, sm, htag)) {
      return;
    }
  }
  stamp(p, tr, 11);
  shake(p, sm, 11);
  const DownGeo g = down_geo(p, sm);
  ph_expand<ACT, RMAX, true>(p, sm, g.blk);
  stamp(p, tr, 13);
}

/* ------------------------------------------------------------------------------------------
 * Launch templates */

#define MONO_LAUNCH(KERNEL, GRID)                                                      \
  do {                                                                                 \
    hipLaunchKernelGGL((KERNEL), dim3(GRID), dim3(kBlock), 0, st, p);                  \
    return (int)hipGetLastError();                                                     \
  } while (0)

template <int ACT, int RFMT, int SFMT, int RMAX>
int launch_fmt(Kernel k, const Params& p, int grid, hipStream_t st) {
  switch (k) {
    case K_GATEUP: MONO_LAUNCH((k_gateup<ACT, RFMT, SFMT, RMAX>), grid);
    case K_DOWN: MONO_LAUNCH((k_down<ACT, RFMT, SFMT, RMAX>), grid);
    case K_FFN_LAYER: MONO_LAUNCH((k_ffn_layer<ACT, RFMT, SFMT, RMAX>), grid);
    default: return (int)hipErrorInvalidValue;
  }
}

/* Workgroups of the fused launch one compute unit holds at once (its LDS and registers). */
template <int ACT, int RFMT, int SFMT, int RMAX>
int occ_fmt() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_ffn_layer<ACT, RFMT, SFMT, RMAX>, kBlock,
                                                   0) != hipSuccess)
    return -1;
  return n;
}

/* Explicit instantiation of one (activation, routed format, shared format) combination for one
 * and for several rows (used by the per-format translation units). */
#define MONO_INSTANTIATE(A, RF, SF)                                                    \
  template int launch_fmt<A, RF, SF, 1>(Kernel, const Params&, int, hipStream_t);      \
  template int launch_fmt<A, RF, SF, kMaxRows>(Kernel, const Params&, int, hipStream_t); \
  template int occ_fmt<A, RF, SF, 1>();                                                \
  template int occ_fmt<A, RF, SF, kMaxRows>();

}  // namespace mono

#endif /* MONOLAYER_KERNELS_H */
