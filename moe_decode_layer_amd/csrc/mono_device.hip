/*
 * libmonolayer device code for gfx950 (CDNA4, wave64).
 *
 * The layer-half step is written as phases (device functions). The unfused
 * entry points run each phase as its own kernel; the fused entry point runs
 * all phases in ONE persistent launch, separated by device-wide barriers. A
 * phase computes every output element with a fixed decomposition (one wave
 * per dot product, fixed lane mapping, fixed reduction tree), independent of
 * which workgroup runs it, so the fused and the unfused paths produce
 * identical bytes.
 *
 * The work is a chain of HBM-bound matrix-vector products (1 to 8 activation
 * rows against weights read once), so it runs on the vector ALUs: every lane
 * streams 16-byte weight vectors (1 KB per wave per step, coalesced), keeps a
 * whole row's loads in flight, dequantises in registers and reduces with DPP.
 * Activations live in LDS. MFMA is not used: at these widths it cannot pay.
 *
 * Steps and rounding points follow the ds4 page "v41: fuse the single-box
 * decode glue (HC, MoE, attention)" ("What" and its HC / router / shared
 * expert commits); the fused launch follows K2 of the SGLang page "[AMD][V4.1]
 * Mono kernel framework ... DeepSeek-V4.1 decode layers" (figure "DeepSeek-V4.1
 * layer on mono") and the post -> next-pre carry of the SGLang page
 * "[DeepSeek-V4] Add mhc_fused_post_pre kernel" ("Motivation").
 */
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mono_internal.h"

namespace mono {

enum { F32 = MONO_F32, BF16 = MONO_BF16, Q8 = MONO_Q8_0, FP4 = MONO_MXFP4 };

constexpr int kSelKeys = 1024;   /* (row, expert) candidates ranked at once by the select */
constexpr int kMaxUnion = kMaxRows * kMaxTopK;
constexpr int kRG = 4;           /* consecutive down-projection rows per task */

/* ------------------------------------------------------------------------------------------
 * Number formats */

__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

/* f32 -> bf16 bits, round to nearest even (NaN stays NaN). */
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x7FFFFFu)) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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

/* Four consecutive act values starting at i (i a multiple of 4). */
template <int ACT>
__device__ __forceinline__ void act_ld4(const void* p, size_t i, float (&o)[4]) {
  if (ACT == F32) {
    float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  } else {
    uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p) + i);
    o[0] = bf2f(v.x & 0xFFFFu); o[1] = bf2f(v.x >> 16);
    o[2] = bf2f(v.y & 0xFFFFu); o[3] = bf2f(v.y >> 16);
  }
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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

/* c + a.lo * b.lo + a.hi * b.hi for packed bf16 pairs. */
__device__ __forceinline__ float dot2bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

/* ------------------------------------------------------------------------------------------
 * Wave reductions (DPP butterflies inside each row of 16 lanes, then the four row sums). Must
 * be called with all 64 lanes active; every lane returns the same value. */

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
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
 * or 32 MXFP4 values per lane, so lane L of step s holds elements [(64 s + L) * EL, + EL). */

template <int FMT> struct Fmt;
template <> struct Fmt<F32> { static constexpr int EL = 4, CH_GU = 8, CH_DN = 4; };
template <> struct Fmt<BF16> { static constexpr int EL = 8, CH_GU = 10, CH_DN = 4; };
template <> struct Fmt<Q8> { static constexpr int EL = 16, CH_GU = 5, CH_DN = 2; };
template <> struct Fmt<FP4> { static constexpr int EL = 32, CH_GU = 3, CH_DN = 1; };

__host__ __device__ constexpr size_t row_vbytes(int fmt, size_t k) {
  return fmt == F32 ? 4 * k : fmt == BF16 ? 2 * k : fmt == Q8 ? k : k / 2;
}
__host__ __device__ constexpr size_t row_sbytes(int fmt, size_t k) {
  return fmt == Q8 ? (k / 32) * 2 : fmt == FP4 ? k / 32 : 0;
}

template <int FMT>
__device__ __forceinline__ void wload(const uint8_t* vrow, const uint8_t* srow, int s, int lane,
                                      int K, uint4& v, uint32_t& sc) {
  const int q = s * 64 + lane;
  const int k = q * Fmt<FMT>::EL;
  if (k < K) {
    v = *reinterpret_cast<const uint4*>(vrow + (size_t)q * 16);
    if (FMT == Q8) sc = *reinterpret_cast<const uint16_t*>(srow + (k / 32) * 2);
    if (FMT == FP4) sc = srow[k / 32];
  } else {
    v = make_uint4(0, 0, 0, 0);
    sc = 0;
  }
}

/* acc + (weights of one step) . (act values k .. k + EL - 1 of one LDS row). */
template <int FMT, int ACT>
__device__ __forceinline__ float vdot(const uint4& v, uint32_t sc, const void* arow, int k,
                                      float acc) {
  if (FMT == F32) {
    float x[4];
    act_ld4<ACT>(arow, k, x);
    acc = fmaf(__uint_as_float(v.x), x[0], acc);
    acc = fmaf(__uint_as_float(v.y), x[1], acc);
    acc = fmaf(__uint_as_float(v.z), x[2], acc);
    acc = fmaf(__uint_as_float(v.w), x[3], acc);
    return acc;
  } else if (FMT == BF16) {
    const uint4 x = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(arow) + k);
    acc = dot2bf(v.x, x.x, acc);
    acc = dot2bf(v.y, x.y, acc);
    acc = dot2bf(v.z, x.z, acc);
    acc = dot2bf(v.w, x.w, acc);
    return acc;
  } else if (FMT == Q8) {
    const uint16_t* a = static_cast<const uint16_t*>(arow) + k;
    const uint4 x0 = *reinterpret_cast<const uint4*>(a);
    const uint4 x1 = *reinterpret_cast<const uint4*>(a + 8);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    const uint32_t xa[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    float part = 0.0f;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const float q = (float)(int8_t)((w[b >> 2] >> (8 * (b & 3))) & 0xFFu);
      const uint32_t xw = xa[b >> 1];
      const float xv = (b & 1) ? __uint_as_float(xw & 0xFFFF0000u) : __uint_as_float(xw << 16);
      part = fmaf(q, xv, part);
    }
    return fmaf(f16_to_f32(sc), part, acc);
  } else {
    const uint16_t* a = static_cast<const uint16_t*>(arow) + k;
    uint32_t xa[16];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 t = *reinterpret_cast<const uint4*>(a + 8 * c);
      xa[4 * c] = t.x; xa[4 * c + 1] = t.y; xa[4 * c + 2] = t.z; xa[4 * c + 3] = t.w;
    }
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float part = 0.0f;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      /* byte b holds elements 2b (low nibble) and 2b + 1 (high nibble) */
      float2 f;
      switch (b & 3) {
        case 0: { auto t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[b >> 2], 1.0f, 0); f = make_float2(t[0], t[1]); break; }
        case 1: { auto t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[b >> 2], 1.0f, 1); f = make_float2(t[0], t[1]); break; }
        case 2: { auto t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[b >> 2], 1.0f, 2); f = make_float2(t[0], t[1]); break; }
        default: { auto t = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[b >> 2], 1.0f, 3); f = make_float2(t[0], t[1]); break; }
      }
      const uint32_t xw = xa[b];
      part = fmaf(f.x, __uint_as_float(xw << 16), part);
      part = fmaf(f.y, __uint_as_float(xw & 0xFFFF0000u), part);
    }
    return fmaf(e8m0_to_f32(sc), part, acc);
  }
}

/* acc[m][r] += row_m . act_r for m < NR and every r in `mask`, over K elements. Every lane
 * keeps CH steps of all NR rows in flight before it computes. Per-lane partials only; the
 * caller reduces across the wave. */
template <int FMT, int ACT, int RMAX, int NR, int CH>
__device__ __forceinline__ void dot_rows(const uint8_t* const (&vrow)[NR],
                                         const uint8_t* const (&srow)[NR], int K,
                                         const void* const (&arow)[RMAX], uint32_t mask,
                                         float (&acc)[NR][RMAX]) {
  constexpr int EL = Fmt<FMT>::EL;
  const int lane = threadIdx.x & 63;
  const int nsteps = (K + 64 * EL - 1) / (64 * EL);
  for (int s0 = 0; s0 < nsteps; s0 += CH) {
    uint4 v[NR][CH];
    uint32_t sc[NR][CH];
#pragma unroll
    for (int c = 0; c < CH; ++c)
#pragma unroll
      for (int m = 0; m < NR; ++m) {
        if (s0 + c < nsteps)
          wload<FMT>(vrow[m], srow[m], s0 + c, lane, K, v[m][c], sc[m][c]);
        else {
          v[m][c] = make_uint4(0, 0, 0, 0);
          sc[m][c] = 0;
        }
      }
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      const int k = ((s0 + c) * 64 + lane) * EL;
      if (s0 + c < nsteps && k < K) {
#pragma unroll
        for (int r = 0; r < RMAX; ++r)
          if (mask & (1u << r))
#pragma unroll
            for (int m = 0; m < NR; ++m)
              acc[m][r] = vdot<FMT, ACT>(v[m][c], sc[m][c], arow[r], k, acc[m][r]);
      }
    }
  }
}

/* ------------------------------------------------------------------------------------------
 * Workgroup shared memory */

struct Smem {
  alignas(16) uint8_t big[kLdsActBytes]; /* act rows [R][H]; down phase: hidden rows + y */
  float raw[kMaxRows][kNCarry];
  float mixes[kMaxRows][kNMix];
  float pre[kMaxRows][4];
  float post[kMaxRows][4];
  float comb[kMaxRows][16];
  float red[kWaves][kMaxRows * kNCarry];
  float rsum[kMaxRows];
  uint64_t keys[kSelKeys];
  float sval[kSelKeys];
  int sel_e[kMaxRows][kMaxTopK];
  float sel_s[kMaxRows][kMaxTopK];
  float sel_w[kMaxRows][kMaxTopK];
  int U[kMaxUnion + 1];
  uint32_t umask[kMaxUnion + 1];
  int8_t uslot[kMaxUnion + 1][kMaxRows];
  uint16_t voff[kMaxUnion + 1][kMaxRows]; /* staged hidden row offset per (item, row), 16 B */
  uint8_t used[kMaxExperts];
  int nU;
  int flag;
};

/* ------------------------------------------------------------------------------------------
 * Device-wide barrier with a bounded wait. Generation counting: the last workgroup to arrive
 * resets the count and advances the generation; the others spin on the generation. Arrivals
 * release at agent scope, the waiters acquire after they see the new generation. On expiry the
 * error word is set and every thread of the workgroup returns false. */

__device__ __forceinline__ uint32_t spin_limit(const Params& p) {
  uint32_t l = __hip_atomic_load(&p.ctl[CTL_SPIN], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return l ? l : kDefaultSpin;
}

__device__ void report_timeout(const Params& p, int phase) {
  uint32_t* e = p.ctl + CTL_ERR;
  if (atomicCAS(&e[0], 0u, 1u) == 0u) {
    __hip_atomic_store(&e[1], (uint32_t)phase, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&e[2], (uint32_t)blockIdx.x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  atomicAdd(&e[3], 1u);
}

__device__ bool grid_barrier(const Params& p, Smem& sm, int phase) {
  __builtin_amdgcn_s_waitcnt(0); /* this wave's stores have reached the cache */
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t* cnt = p.ctl + CTL_BAR_COUNT;
    uint32_t* gen = p.ctl + CTL_BAR_GEN;
    const uint32_t nwg = gridDim.x;
    const uint32_t g = __hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool skip =
        (int32_t)p.ctl[CTL_FAULT_WG] == (int32_t)blockIdx.x && (int32_t)p.ctl[CTL_FAULT_PHASE] == phase;
    int ok = 1;
    bool last = false;
    if (!skip) {
      const uint32_t a = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      if (a == nwg - 1) {
        last = true;
        __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_fetch_add(gen, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    if (!last) {
      const uint32_t lim = spin_limit(p);
      const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
      while (__hip_atomic_load(gen, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == g) {
        __builtin_amdgcn_s_sleep(1);
        if (__builtin_amdgcn_s_memrealtime() - t0 > lim) {
          report_timeout(p, phase);
          ok = 0;
          break;
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    sm.flag = ok;
  }
  __syncthreads();
  return sm.flag != 0;
}

/* ------------------------------------------------------------------------------------------
 * Phase: mix partials [ds4 HC fusion commit: rms_norm_mix over the 4 x H row; SGLang fused
 * post/pre page: pre-norm GEMM partials + RMS square-sum partials]. Chunk t (256 consecutive
 * elements of the flattened row) is one wave task: part[t][r][j] = W_mix[j] . s over the chunk,
 * part[t][r][24] = sum s^2 over the chunk. */
template <int ACT, int RMAX>
__device__ void ph_mix_partials(const Params& p) {
  const int n = 4 * p.H, nch = n / kMixChunk;
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWaves + (threadIdx.x >> 6), nwt = gridDim.x * kWaves;
  for (int t = gw; t < nch; t += nwt) {
    const int base = t * kMixChunk + lane * 4;
    float s[RMAX][4];
    float ss[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r < p.R) {
        act_ld4<ACT>(p.state, (size_t)r * n + base, s[r]);
      } else {
        s[r][0] = s[r][1] = s[r][2] = s[r][3] = 0.0f;
      }
      ss[r] = s[r][0] * s[r][0];
      ss[r] = fmaf(s[r][1], s[r][1], ss[r]);
      ss[r] = fmaf(s[r][2], s[r][2], ss[r]);
      ss[r] = fmaf(s[r][3], s[r][3], ss[r]);
    }
    float4 w[kNMix];
#pragma unroll
    for (int j = 0; j < kNMix; ++j)
      w[j] = *reinterpret_cast<const float4*>(p.w_mix + (size_t)j * n + base);
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r >= p.R) break;
      float* out = p.mix_part + ((size_t)t * p.R + r) * kNCarry;
#pragma unroll
      for (int j = 0; j < kNMix; ++j) {
        float a = w[j].x * s[r][0];
        a = fmaf(w[j].y, s[r][1], a);
        a = fmaf(w[j].z, s[r][2], a);
        a = fmaf(w[j].w, s[r][3], a);
        const float tot = wave_sum(a);
        if (lane == 0) out[j] = tot;
      }
      const float tot = wave_sum(ss[r]);
      if (lane == 0) out[kNMix] = tot;
    }
  }
}

/* ------------------------------------------------------------------------------------------
 * Phase: mHC pre side for all rows, run by one whole workgroup (redundantly by every workgroup
 * of the fused launch). mixes from the partials (or the carry); split / Sinkhorn; collapse;
 * weighted RMSNorm. The norm rows are left in sm.big as act values.
 * READING (mHC, not on the pages): pre = sigmoid(a0 m[i] + b[i]); post = 2 sigmoid(a1 m[4+i]
 * + b[4+i]); comb = Sinkhorn on exp(a2 m[8+4i+j] + b[8+4i+j] - max), rows then columns. */
template <int ACT, int RMAX>
__device__ void ph_hc_pre(const Params& p, Smem& sm, bool write_out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int R = p.R, H = p.H, n = 4 * H, nch = n / kMixChunk;
  if (tid < R * kNCarry) {
    const int r = tid / kNCarry, j = tid % kNCarry;
    float v;
    if (p.carry_in) {
      v = p.carry_in[r * kNCarry + j];
    } else {
      v = 0.0f;
      for (int t = 0; t < nch; ++t) v += p.mix_part[((size_t)t * R + r) * kNCarry + j];
    }
    sm.raw[r][j] = v;
  }
  __syncthreads();
  if (tid < R * kNMix) {
    const int r = tid / kNMix, j = tid % kNMix;
    const float den = sqrtf(sm.raw[r][kNMix] / (float)n + p.eps_hc);
    const float m = sm.raw[r][j] / den;
    sm.mixes[r][j] = m;
    if (write_out && p.mixes) p.mixes[r * kNMix + j] = m;
  }
  __syncthreads();
  if (tid < R) {
    const int r = tid;
    const float a0 = p.hc_scale[0], a1 = p.hc_scale[1], a2 = p.hc_scale[2];
    const float* m = sm.mixes[r];
    const float* b = p.hc_base;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sm.pre[r][i] = 1.0f / (1.0f + expf(-(a0 * m[i] + b[i])));
      sm.post[r][i] = 2.0f / (1.0f + expf(-(a1 * m[4 + i] + b[4 + i])));
    }
    float M[16];
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      M[q] = a2 * m[8 + q] + b[8 + q];
      mx = fmaxf(mx, M[q]);
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) M[q] = expf(M[q] - mx);
    for (int it = 0; it < p.iters; ++it) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s = ((M[4 * i] + M[4 * i + 1]) + M[4 * i + 2]) + M[4 * i + 3];
#pragma unroll
        for (int j = 0; j < 4; ++j) M[4 * i + j] = M[4 * i + j] / s;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float s = ((M[j] + M[4 + j]) + M[8 + j]) + M[12 + j];
#pragma unroll
        for (int i = 0; i < 4; ++i) M[4 * i + j] = M[4 * i + j] / s;
      }
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) sm.comb[r][q] = M[q];
    if (write_out) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p.pre[r * 4 + i] = sm.pre[r][i];
        p.post[r * 4 + i] = sm.post[r][i];
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) p.comb[r * 16 + q] = M[q];
    }
  }
  __syncthreads();
  /* collapse: x = bf16(sum_i pre_i state_i); sum of squares of the rounded x */
  float ss[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    ss[r] = 0.0f;
    if (r >= R) continue;
    const float p0 = sm.pre[r][0], p1 = sm.pre[r][1], p2 = sm.pre[r][2], p3 = sm.pre[r][3];
    for (int h = tid; h < H; h += kBlock) {
      const size_t b = (size_t)r * n + h;
      float a = p0 * act_ld<ACT>(p.state, b);
      a = fmaf(p1, act_ld<ACT>(p.state, b + H), a);
      a = fmaf(p2, act_ld<ACT>(p.state, b + 2 * (size_t)H), a);
      a = fmaf(p3, act_ld<ACT>(p.state, b + 3 * (size_t)H), a);
      const float xb = act_round<ACT>(a);
      act_st<ACT>(sm.big, (size_t)r * H + h, xb);
      if (write_out && p.x) act_st<ACT>(p.x, (size_t)r * H + h, xb);
      ss[r] = fmaf(xb, xb, ss[r]);
    }
  }
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
  /* weighted RMSNorm: norm = bf16(x / sqrt(mean(x^2) + eps) * w) */
  for (int r = 0; r < R; ++r) {
    const float den = sqrtf(sm.rsum[r] / (float)H + p.eps_norm);
    for (int h = tid; h < H; h += kBlock) {
      const float xb = act_ld<ACT>(sm.big, (size_t)r * H + h);
      const float v = act_round<ACT>(xb / den * act_ld<ACT>(p.w_norm, h));
      act_st<ACT>(sm.big, (size_t)r * H + h, v);
      if (write_out) act_st<ACT>(p.norm, (size_t)r * H + h, v);
    }
  }
  __syncthreads();
}

/* Copies R act rows [R][H] from global memory into sm.big. */
template <int ACT>
__device__ void load_act_rows(const void* src, int R, int H, Smem& sm) {
  const size_t bytes = (size_t)R * H * (ACT == F32 ? 4 : 2);
  const uint4* s = static_cast<const uint4*>(src);
  uint4* d = reinterpret_cast<uint4*>(sm.big);
  for (size_t i = threadIdx.x; i < bytes / 16; i += kBlock) d[i] = s[i];
  __syncthreads();
}

/* ------------------------------------------------------------------------------------------
 * Phase: router logits [ds4 router commit: the F32 logits matvec]. One wave per expert row. */
template <int ACT, int RMAX>
__device__ void ph_router(const Params& p, const Smem& sm) {
  const int lane = threadIdx.x & 63;
  const int gw = blockIdx.x * kWaves + (threadIdx.x >> 6), nwt = gridDim.x * kWaves;
  const void* arow[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
    arow[r] = sm.big + (size_t)(r < p.R ? r : 0) * p.H * (ACT == F32 ? 4 : 2);
  const uint32_t mask = (1u << p.R) - 1u;
  for (int e = gw; e < p.E; e += nwt) {
    const uint8_t* vr[1] = {reinterpret_cast<const uint8_t*>(p.w_router + (size_t)e * p.H)};
    const uint8_t* sr[1] = {nullptr};
    float acc[1][RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) acc[0][r] = 0.0f;
    dot_rows<F32, ACT, RMAX, 1, 10>(vr, sr, p.H, arow, mask, acc);
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
      if (r >= p.R) break;
      const float t = wave_sum(acc[0][r]);
      if (lane == 0) p.logits[(size_t)r * p.E + e] = t;
    }
  }
}

/* ------------------------------------------------------------------------------------------
 * Phase: select, run by one whole workgroup for all rows [ds4 router commit: sqrt(softplus),
 * the bias, the canonical (score descending, index ascending) top-k, normalised weights, the
 * clamp, the row division and the scale as separately rounded ops; tie-order commit].
 * Each candidate's rank is the number of candidates with a larger 64-bit key
 * (ordered biased score, then the complement of the index), so ties order by ascending index and
 * every rank is unique. READING: the clamp floor is 2^-14 and the bias steers selection only. */
__device__ __forceinline__ uint32_t ord_f32(float f) {
  if (f != f) return 0u; /* NaN ranks last */
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

template <int RMAX>
__device__ void ph_select(const Params& p, Smem& sm, bool write_out) {
  const int tid = threadIdx.x, R = p.R, E = p.E, K = p.K;
  const int rows_per = kSelKeys / E > 0 ? kSelKeys / E : 1;
  for (int r0 = 0; r0 < R; r0 += rows_per) {
    const int nb = (R - r0) < rows_per ? (R - r0) : rows_per;
    for (int c = tid; c < nb * E; c += kBlock) {
      const int r = r0 + c / E, e = c % E;
      const float z = p.logits[(size_t)r * E + e];
      const float sp = z > 0.0f ? z + log1pf(expf(-z)) : log1pf(expf(z));
      const float s = sqrtf(sp);
      const float beta = s + p.bias[e];
      sm.keys[c] = ((uint64_t)ord_f32(beta) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
      sm.sval[c] = s;
    }
    __syncthreads();
    for (int c = tid; c < nb * E; c += kBlock) {
      const int rl = c / E;
      const uint64_t key = sm.keys[c];
      const uint64_t* row = sm.keys + rl * E;
      int rank = 0;
      for (int q = 0; q < E; ++q) rank += row[q] > key ? 1 : 0;
      if (rank < K) {
        sm.sel_e[r0 + rl][rank] = c % E;
        sm.sel_s[r0 + rl][rank] = sm.sval[c];
      }
    }
    __syncthreads();
  }
  if (tid < R) {
    const int r = tid;
    float sum = 0.0f;
    for (int j = 0; j < K; ++j) sum += sm.sel_s[r][j];
    const float c = fmaxf(sum, 6.103515625e-05f); /* 2^-14 */
    for (int j = 0; j < K; ++j) {
      const float w = (sm.sel_s[r][j] / c) * p.rho;
      sm.sel_w[r][j] = w;
      if (write_out) {
        p.idx[r * K + j] = sm.sel_e[r][j];
        p.weights[r * K + j] = w;
      }
    }
  }
  __syncthreads();
}

/* Reads a caller-provided selection (idx, weights) into sm.sel_*; indices are clamped into
 * [0, E) so a bad index cannot address outside the expert arrays. */
__device__ void load_selection(const Params& p, Smem& sm) {
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
 * is the shared expert (every row). */
__device__ void ph_plan(const Params& p, Smem& sm) {
  const int tid = threadIdx.x, R = p.R, K = p.K, E = p.E;
  for (int e = tid; e < E; e += kBlock) sm.used[e] = 0;
  __syncthreads();
  if (tid < R * K) sm.used[sm.sel_e[tid / K][tid % K]] = 1;
  __syncthreads();
  if (tid < 64) {
    int base = 0;
    for (int e0 = 0; e0 < E; e0 += 64) {
      const int e = e0 + tid;
      const bool u = e < E && sm.used[e];
      const uint64_t bal = __ballot(u);
      if (u) sm.U[base + __popcll(bal & ((1ull << tid) - 1ull))] = e;
      base += __popcll(bal);
    }
    if (tid == 0) sm.nU = base;
  }
  __syncthreads();
  const int nU = sm.nU;
  for (int q = tid; q < (nU + 1) * kMaxRows; q += kBlock) {
    const int u = q / kMaxRows, r = q % kMaxRows;
    int slot = -1;
    if (r < R) {
      if (u == nU) {
        slot = K;
      } else {
        for (int j = 0; j < K; ++j)
          if (sm.sel_e[r][j] == sm.U[u]) slot = j;
      }
    }
    sm.uslot[u][r] = (int8_t)slot;
  }
  __syncthreads();
  if (tid <= nU) {
    uint32_t m = 0;
    for (int r = 0; r < R; ++r)
      if (sm.uslot[tid][r] >= 0) m |= 1u << r;
    sm.umask[tid] = m;
  }
  __syncthreads();
}

/* ------------------------------------------------------------------------------------------
 * Phase: gate/up + SwiGLU [ds4 router/shared commit: both matvecs, gate/up rounded to BF16
 * before SwiGLU and the product after it]. Task (item u, intermediate row i): one wave streams
 * gate row i and up row i once and applies them to every row that selected the expert.
 * READING: routed experts use the shared expert's rounding points. */
template <int ACT, int FMT, int RMAX>
__device__ __forceinline__ void gateup_task(const Params& p, const Smem& sm, const Mat& m,
                                            int e, int i, int inter, uint32_t mask, int u,
                                            bool is_shared) {
  const int H = p.H, lane = threadIdx.x & 63;
  const size_t vb = row_vbytes(FMT, H), sb = row_sbytes(FMT, H);
  const size_t row = (size_t)e * inter + i;
  const uint8_t* vr[2] = {m.gate + row * vb, m.up + row * vb};
  const uint8_t* sr[2] = {m.gate_s ? m.gate_s + row * sb : nullptr,
                          m.up_s ? m.up_s + row * sb : nullptr};
  const void* arow[RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
    arow[r] = sm.big + (size_t)(r < p.R ? r : 0) * H * (ACT == F32 ? 4 : 2);
  float acc[2][RMAX];
#pragma unroll
  for (int r = 0; r < RMAX; ++r) acc[0][r] = acc[1][r] = 0.0f;
  dot_rows<FMT, ACT, RMAX, 2, Fmt<FMT>::CH_GU>(vr, sr, H, arow, mask, acc);
#pragma unroll
  for (int r = 0; r < RMAX; ++r) {
    if (!(mask & (1u << r))) continue;
    const float g = act_round<ACT>(wave_sum(acc[0][r]));
    const float uu = act_round<ACT>(wave_sum(acc[1][r]));
    const float h = act_round<ACT>(g / (1.0f + expf(-g)) * uu);
    if (lane == 0) {
      if (is_shared)
        act_st<ACT>(p.h_shared, (size_t)r * p.Is + i, h);
      else
        act_st<ACT>(p.h_routed, ((size_t)r * p.K + sm.uslot[u][r]) * p.I + i, h);
    }
  }
}

template <int ACT, int RFMT, int SFMT, int RMAX>
__device__ void ph_gateup(const Params& p, const Smem& sm) {
  const int nU = sm.nU;
  const long T = (long)nU * p.I + p.Is;
  const long gw = blockIdx.x * kWaves + (threadIdx.x >> 6), nwt = (long)gridDim.x * kWaves;
  const long t0 = T * gw / nwt, t1 = T * (gw + 1) / nwt;
  for (long t = t0; t < t1; ++t) {
    if (t < (long)nU * p.I) {
      const int u = (int)(t / p.I), i = (int)(t % p.I);
      gateup_task<ACT, RFMT, RMAX>(p, sm, p.routed, sm.U[u], i, p.I, sm.umask[u], u, false);
    } else {
      const int i = (int)(t - (long)nU * p.I);
      gateup_task<ACT, SFMT, RMAX>(p, sm, p.shared, 0, i, p.Is, sm.umask[nU], nU, true);
    }
  }
}

/* ------------------------------------------------------------------------------------------
 * Phase: down projections, routed sum, shared rounding and block for the workgroup's slice of
 * hidden rows [ds4 router/shared commit: the down projection rounded on its store, the routed +
 * shared sum and its rounding]. The hidden rows of the selected experts are staged in LDS in
 * groups; task (item, group of 4 consecutive output rows) is one wave. y values land in LDS;
 * then per (h, r): routed = f32 sum_j w_j y_j (selection order), shared = bf16(y_s),
 * block = bf16(routed + shared). Leaves block in sm (y region) for the expand. */
struct DownGeo {
  int h0, nh;
  size_t hid_bytes; /* LDS bytes for staged hidden rows */
  float* y;         /* [nh][R][K + 1] */
  float* blk;       /* [nh][R] */
};

template <int ACT>
__device__ __forceinline__ DownGeo down_geo(const Params& p, Smem& sm) {
  DownGeo g;
  const int hs = (p.H + p.nslice - 1) / p.nslice;
  g.h0 = blockIdx.x * hs;
  g.nh = p.H - g.h0 < hs ? p.H - g.h0 : hs;
  if (g.nh < 0) g.nh = 0;
  g.hid_bytes = kLdsHidBytes;
  g.y = reinterpret_cast<float*>(sm.big + kLdsHidBytes);
  g.blk = g.y + (size_t)hs * p.R * (p.K + 1);
  return g;
}

template <int ACT, int FMT, int RMAX>
__device__ __forceinline__ void down_task(const Params& p, const Smem& sm, const DownGeo& g,
                                          const Mat& m, int e, int inter, int item, int q,
                                          bool is_shared) {
  const int lane = threadIdx.x & 63;
  const size_t vb = row_vbytes(FMT, inter), sb = row_sbytes(FMT, inter);
  const uint8_t* vr[kRG];
  const uint8_t* sr[kRG];
#pragma unroll
  for (int c = 0; c < kRG; ++c) {
    int hl = q * kRG + c;
    if (hl >= g.nh) hl = g.nh - 1; /* duplicate a valid row; its result is discarded */
    const size_t row = (size_t)e * p.H + g.h0 + hl;
    vr[c] = m.down + row * vb;
    sr[c] = m.down_s ? m.down_s + row * sb : nullptr;
  }
  const uint32_t mask = sm.umask[item];
  const void* arow[RMAX];
  const size_t ab = ACT == F32 ? 4 : 2;
#pragma unroll
  for (int r = 0; r < RMAX; ++r)
    arow[r] = sm.big + (size_t)((mask & (1u << r)) ? sm.voff[item][r] : 0) * 16;
  float acc[kRG][RMAX];
#pragma unroll
  for (int c = 0; c < kRG; ++c)
#pragma unroll
    for (int r = 0; r < RMAX; ++r) acc[c][r] = 0.0f;
  dot_rows<FMT, ACT, RMAX, kRG, Fmt<FMT>::CH_DN>(vr, sr, inter, arow, mask, acc);
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

template <int ACT, int RFMT, int SFMT, int RMAX>
__device__ void ph_down(const Params& p, Smem& sm) {
  const int tid = threadIdx.x, wave = tid >> 6;
  const DownGeo g = down_geo<ACT>(p, sm);
  const int nU = sm.nU, R = p.R;
  const size_t ab = ACT == F32 ? 4 : 2;
  const int nq = (g.nh + kRG - 1) / kRG;
  int item = 0;
  while (item <= nU) {
    /* a group of items [first, last) whose hidden rows fit in the staging area */
    const int first = item;
    size_t used = 0;
    while (item <= nU) {
      const int inter = item == nU ? p.Is : p.I;
      const size_t need = (size_t)__popc(sm.umask[item]) * inter * ab;
      if (item > first && used + need > g.hid_bytes) break;
      used += need;
      ++item;
    }
    const int last = item;
    __syncthreads(); /* previous group's tasks are done with the staging area */
    if (tid == 0) {
      size_t off = 0;
      for (int it = first; it < last; ++it) {
        const int inter = it == nU ? p.Is : p.I;
        for (int r = 0; r < R; ++r)
          if (sm.umask[it] & (1u << r)) {
            sm.voff[it][r] = (uint16_t)(off / 16);
            off += (size_t)inter * ab;
          }
      }
    }
    __syncthreads();
    for (int it = first; it < last; ++it) {
      const int inter = it == nU ? p.Is : p.I;
      const size_t vbytes = (size_t)inter * ab;
      for (int r = 0; r < R; ++r) {
        if (!(sm.umask[it] & (1u << r))) continue;
        const uint8_t* src =
            it == nU ? static_cast<const uint8_t*>(p.h_shared) + (size_t)r * vbytes
                     : static_cast<const uint8_t*>(p.h_routed) +
                           ((size_t)r * p.K + sm.uslot[it][r]) * vbytes;
        uint8_t* dst = sm.big + (size_t)sm.voff[it][r] * 16;
        for (size_t b = (size_t)tid * 16; b < vbytes; b += (size_t)kBlock * 16)
          *reinterpret_cast<uint4*>(dst + b) = *reinterpret_cast<const uint4*>(src + b);
      }
    }
    __syncthreads();
    const int ntask = (last - first) * nq;
    for (int t = wave; t < ntask; t += kWaves) {
      const int it = first + t / nq, q = t % nq;
      if (it == nU) {
        if (p.Is > 0 && sm.umask[it]) down_task<ACT, SFMT, RMAX>(p, sm, g, p.shared, 0, p.Is, it, q, true);
      } else {
        down_task<ACT, RFMT, RMAX>(p, sm, g, p.routed, sm.U[it], p.I, it, q, false);
      }
    }
    __syncthreads();
  }
  /* combine */
  for (int q = tid; q < g.nh * R; q += kBlock) {
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
 * Phase: expand + carry for the workgroup's slice [ds4 HC fusion commit: post/comb expand +
 * BF16; SGLang fused post/pre page: bf16 residual materialisation + next pre-norm GEMM partials
 * + RMS square-sum partials]. new[i][h] = bf16(post_i block[h] + sum_j comb[i][j] state_j[h]).
 * The carry is taken on the rounded new state; per-workgroup partials are summed in workgroup
 * order by the last workgroup to finish. */
template <int ACT, int RMAX>
__device__ void ph_expand(const Params& p, Smem& sm, const float* blk) {
  const int tid = threadIdx.x;
  const int hs = (p.H + p.nslice - 1) / p.nslice;
  const int h0 = blockIdx.x * hs;
  int nh = p.H - h0 < hs ? p.H - h0 : hs;
  if (nh < 0) nh = 0;
  const int R = p.R, H = p.H, n = 4 * H;
  /* new state: one thread per hidden position reads all 4 streams and writes all 4, so the
   * output may alias the input */
  float* nvb = reinterpret_cast<float*>(sm.big); /* [nh][R][4] */
  for (int hl = tid; hl < nh; hl += kBlock) {
    const int h = h0 + hl;
    for (int r = 0; r < R; ++r) {
      const size_t sb = (size_t)r * n + h;
      const float s0 = act_ld<ACT>(p.state, sb), s1 = act_ld<ACT>(p.state, sb + H);
      const float s2 = act_ld<ACT>(p.state, sb + 2 * (size_t)H);
      const float s3 = act_ld<ACT>(p.state, sb + 3 * (size_t)H);
      const float b = blk[hl * R + r];
      float nv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float a = sm.post[r][i] * b;
        a = fmaf(sm.comb[r][4 * i + 0], s0, a);
        a = fmaf(sm.comb[r][4 * i + 1], s1, a);
        a = fmaf(sm.comb[r][4 * i + 2], s2, a);
        a = fmaf(sm.comb[r][4 * i + 3], s3, a);
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
  __syncthreads();
  /* carry partials of this slice: cp[j][r][hl] = sum_i W_next[j][i H + h] new[r][i] (j < 24),
   * cp[24][r][hl] = sum_i new[r][i]^2; then summed over hl in order */
  float* cp = nvb + (size_t)nh * R * 4; /* [25][R][nh] */
  for (int q = tid; q < nh * kNCarry; q += kBlock) {
    const int hl = q % nh, j = q / nh, h = h0 + hl;
    float w[4];
    if (j < kNMix) {
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = p.w_mix_next[(size_t)j * n + (size_t)i * H + h];
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
      cp[((size_t)j * R + r) * nh + hl] = a;
    }
  }
  __syncthreads();
  if (tid < R * kNCarry) {
    const int j = tid % kNCarry, r = tid / kNCarry;
    const float* c = cp + ((size_t)j * R + r) * nh;
    float t = 0.0f;
    for (int hl = 0; hl < nh; ++hl) t += c[hl];
    p.carry_part[(size_t)blockIdx.x * R * kNCarry + tid] = t;
  }
  /* the last workgroup to finish sums the partials in workgroup order */
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (tid == 0) {
    const uint32_t a = __hip_atomic_fetch_add(p.ctl + CTL_CARRY_COUNT, 1u, __ATOMIC_ACQ_REL,
                                              __HIP_MEMORY_SCOPE_AGENT);
    const bool last = a == gridDim.x - 1;
    if (last)
      __hip_atomic_store(p.ctl + CTL_CARRY_COUNT, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.flag = last ? 1 : 0;
  }
  __syncthreads();
  if (sm.flag && tid < R * kNCarry) {
    float t = 0.0f;
    for (int w = 0; w < (int)gridDim.x; ++w)
      t += __hip_atomic_load(p.carry_part + (size_t)w * R * kNCarry + tid, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    p.carry_out[tid] = t;
    if (p.carry_ws) p.carry_ws[tid] = t;
  }
}

/* ------------------------------------------------------------------------------------------
 * Kernels */

template <int ACT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_mix_partials(Params p) {
  ph_mix_partials<ACT, RMAX>(p);
}

template <int ACT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_hc_pre(Params p) {
  __shared__ Smem sm;
  ph_hc_pre<ACT, RMAX>(p, sm, true);
}

template <int ACT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_router_logits(Params p) {
  __shared__ Smem sm;
  load_act_rows<ACT>(p.norm_in, p.R, p.H, sm);
  ph_router<ACT, RMAX>(p, sm);
}

template <int RMAX>
__global__ void __launch_bounds__(kBlock) k_select(Params p) {
  __shared__ Smem sm;
  ph_select<RMAX>(p, sm, true);
}

template <int ACT, int RFMT, int SFMT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_gateup(Params p) {
  __shared__ Smem sm;
  load_act_rows<ACT>(p.norm_in, p.R, p.H, sm);
  load_selection(p, sm);
  ph_plan(p, sm);
  ph_gateup<ACT, RFMT, SFMT, RMAX>(p, sm);
}

template <int ACT, int RFMT, int SFMT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_down(Params p) {
  __shared__ Smem sm;
  load_selection(p, sm);
  ph_plan(p, sm);
  ph_down<ACT, RFMT, SFMT, RMAX>(p, sm);
}

template <int ACT, int RMAX>
__global__ void __launch_bounds__(kBlock) k_expand(Params p) {
  __shared__ Smem sm;
  const int tid = threadIdx.x;
  if (tid < p.R * 4) {
    sm.post[tid / 4][tid % 4] = p.post_in[tid];
  }
  if (tid < p.R * 16) sm.comb[tid / 16][tid % 16] = p.comb_in[tid];
  const int hs = (p.H + p.nslice - 1) / p.nslice, h0 = blockIdx.x * hs;
  int nh = p.H - h0 < hs ? p.H - h0 : hs;
  if (nh < 0) nh = 0;
  float* blk = reinterpret_cast<float*>(sm.big + kLdsHidBytes);
  for (int q = tid; q < nh * p.R; q += kBlock) {
    const int hl = q / p.R, r = q % p.R;
    blk[q] = act_ld<ACT>(p.block_in, (size_t)r * p.H + h0 + hl);
  }
  __syncthreads();
  ph_expand<ACT, RMAX>(p, sm, blk);
}

/* The whole layer half in one persistent launch (one workgroup per compute unit). */
template <int ACT, int RFMT, int SFMT, int RMAX>
__global__ void __launch_bounds__(kBlock, 1) k_ffn_layer(Params p) {
  __shared__ Smem sm;
  if (!p.carry_in) {
    ph_mix_partials<ACT, RMAX>(p);
    if (!grid_barrier(p, sm, PH_MIX)) return;
  }
  ph_hc_pre<ACT, RMAX>(p, sm, blockIdx.x == 0);
  ph_router<ACT, RMAX>(p, sm);
  if (!grid_barrier(p, sm, PH_ROUTER)) return;
  ph_select<RMAX>(p, sm, blockIdx.x == 0);
  ph_plan(p, sm);
  ph_gateup<ACT, RFMT, SFMT, RMAX>(p, sm);
  if (!grid_barrier(p, sm, PH_GATEUP)) return;
  ph_down<ACT, RFMT, SFMT, RMAX>(p, sm);
  const DownGeo g = down_geo<ACT>(p, sm);
  ph_expand<ACT, RMAX>(p, sm, g.blk);
}

__global__ void k_ws_init(uint32_t* ctl) {
  const int t = threadIdx.x;
  if (t < CTL_WORDS) ctl[t] = (t == CTL_FAULT_WG) ? 0xFFFFFFFFu : 0u;
}

__global__ void k_ws_debug(uint32_t* ctl, uint32_t spin, uint32_t fwg, uint32_t fph) {
  if (threadIdx.x == 0) {
    ctl[CTL_SPIN] = spin;
    ctl[CTL_FAULT_WG] = fwg;
    ctl[CTL_FAULT_PHASE] = fph;
  }
}

/* ------------------------------------------------------------------------------------------
 * Host-side dispatch */

#define MONO_LAUNCH(KERNEL, GRID)                                                      \
  do {                                                                                 \
    hipLaunchKernelGGL((KERNEL), dim3(GRID), dim3(kBlock), 0, st, p);                  \
    return (int)hipGetLastError();                                                     \
  } while (0)

template <int ACT, int RFMT, int SFMT, int RMAX>
static int launch_fmt(Kernel k, const Params& p, int grid, hipStream_t st) {
  switch (k) {
    case K_GATEUP: MONO_LAUNCH((k_gateup<ACT, RFMT, SFMT, RMAX>), grid);
    case K_DOWN: MONO_LAUNCH((k_down<ACT, RFMT, SFMT, RMAX>), grid);
    case K_FFN_LAYER: MONO_LAUNCH((k_ffn_layer<ACT, RFMT, SFMT, RMAX>), grid);
    default: return (int)hipErrorInvalidValue;
  }
}

template <int ACT, int RMAX>
static int launch_act(Kernel k, const Params& p, int rfmt, int sfmt, int grid, hipStream_t st) {
  switch (k) {
    case K_MIX_PARTIALS: MONO_LAUNCH((k_mix_partials<ACT, RMAX>), grid);
    case K_HC_PRE: MONO_LAUNCH((k_hc_pre<ACT, RMAX>), 1);
    case K_ROUTER_LOGITS: MONO_LAUNCH((k_router_logits<ACT, RMAX>), grid);
    case K_SELECT: MONO_LAUNCH((k_select<RMAX>), 1);
    case K_EXPAND: MONO_LAUNCH((k_expand<ACT, RMAX>), grid);
    default: break;
  }
  if constexpr (ACT == F32) {
    if (rfmt == F32 && sfmt == F32) return launch_fmt<ACT, F32, F32, RMAX>(k, p, grid, st);
    return (int)hipErrorInvalidValue;
  } else {
#define MONO_FMT_CASE(RF, SF) \
  if (rfmt == RF && sfmt == SF) return launch_fmt<ACT, RF, SF, RMAX>(k, p, grid, st);
  MONO_FMT_CASE(BF16, BF16)
  MONO_FMT_CASE(BF16, Q8)
  MONO_FMT_CASE(BF16, FP4)
  MONO_FMT_CASE(Q8, BF16)
  MONO_FMT_CASE(Q8, Q8)
  MONO_FMT_CASE(Q8, FP4)
  MONO_FMT_CASE(FP4, BF16)
  MONO_FMT_CASE(FP4, Q8)
  MONO_FMT_CASE(FP4, FP4)
#undef MONO_FMT_CASE
    return (int)hipErrorInvalidValue;
  }
}

int launch(Kernel k, const Params& p, int act, int rfmt, int sfmt, int grid, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (k == K_WS_INIT) {
    hipLaunchKernelGGL(k_ws_init, dim3(1), dim3(64), 0, st, p.ctl);
    return (int)hipGetLastError();
  }
  const bool one = p.R <= 1;
  if (act == F32)
    return one ? launch_act<F32, 1>(k, p, rfmt, sfmt, grid, st)
               : launch_act<F32, kMaxRows>(k, p, rfmt, sfmt, grid, st);
  return one ? launch_act<BF16, 1>(k, p, rfmt, sfmt, grid, st)
             : launch_act<BF16, kMaxRows>(k, p, rfmt, sfmt, grid, st);
}

int launch_debug(uint32_t* ctl, uint32_t spin, uint32_t fwg, uint32_t fph, void* stream) {
  hipLaunchKernelGGL(k_ws_debug, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ctl,
                     spin, fwg, fph);
  return (int)hipGetLastError();
}

int grid_size_for_device(int device) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
    return 0;
  return cus < kMaxGrid ? cus : kMaxGrid;
}

}  // namespace mono
