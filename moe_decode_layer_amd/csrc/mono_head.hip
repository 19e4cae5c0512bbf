/*
 * Model tail: the deferred post of the last layer half is closed by collapsing its new HC state
 * to one row for the output head, without a split [ds4 single-box commit: the logits' collapse
 * and the output norm reuse the collapse kernel without a split; SGLang fused post/pre page,
 * Modifications: the final FFN post deferred to the model tail].
 *   m[i]   = (W_head[i] . s) / sqrt(mean(s^2) + eps_hc)   over the flattened row s (4H values)
 *   pre[i] = sigmoid(a m[i] + b[i])                      (the pre half of the split only)
 *   x      = act(sum_i pre[i] state_i)
 *   norm   = act(x (1 / sqrt(mean(x^2) + eps_norm)) w_norm)
 * One workgroup per row: a pass over the row for the sum of squares and the four head dot
 * products, a pass for x and its sum of squares, and a pass that recomputes x from the state
 * (the same f32 operations, so the same bits) for the norm instead of holding x in LDS. Every
 * sum has a fixed order: each thread adds its own elements in order, then a wave sum, then the
 * waves in order. HBM-bound and small: 4H + 16H/|act| bytes per row plus W_head once.
 */
#include "mono_kernels.h"

namespace mono {

struct HeadParams {
  int H;
  float eps_hc, eps_norm;
  const void* state;
  const float* w_head;
  const float* head_scale;
  const float* head_base;
  const void* w_norm;
  float* pre;
  void* x;
  void* norm;
};

/* The EL act values of a 16-byte unit as floats. */
template <int ACT>
__device__ __forceinline__ void head_unpack(const uint4& u, float (&v)[ACT == F32 ? 4 : 8]) {
  const uint32_t a[4] = {u.x, u.y, u.z, u.w};
  if constexpr (ACT == F32) {
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = __uint_as_float(a[e]);
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = bf2f((a[e >> 1] >> ((e & 1) * 16)) & 0xFFFFu);
  }
}

/* x of unit u (EL consecutive positions): act(pre0 s0 + pre1 s1 + pre2 s2 + pre3 s3). */
template <int ACT>
__device__ __forceinline__ void head_collapse(const uint4* srow, int hu, int u, const float (&pw)[4],
                                              float (&x)[ACT == F32 ? 4 : 8]) {
  constexpr int EL = ACT == F32 ? 4 : 8;
  float s[4][EL];
#pragma unroll
  for (int i = 0; i < 4; ++i) head_unpack<ACT>(srow[(size_t)i * hu + u], s[i]);
#pragma unroll
  for (int e = 0; e < EL; ++e) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(pw[i], s[i][e], acc);
    x[e] = act_round<ACT>(acc);
  }
}

template <int ACT>
__device__ __forceinline__ uint4 head_pack(const float (&v)[ACT == F32 ? 4 : 8]) {
  if constexpr (ACT == F32)
    return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]),
                      __float_as_uint(v[3]));
  else
    return make_uint4(f2bf2(v[0], v[1]), f2bf2(v[2], v[3]), f2bf2(v[4], v[5]), f2bf2(v[6], v[7]));
}

template <int ACT>
__global__ void __launch_bounds__(kBlock) k_hc_head(HeadParams q) {
  constexpr int EL = ACT == F32 ? 4 : 8;
  constexpr size_t AB = ACT == F32 ? 4 : 2;
  __shared__ float red[kWaves][5];
  __shared__ float sh[5];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, r = blockIdx.x;
  const int H = q.H, n = 4 * H, nu = n / EL, hu = H / EL;
  const uint4* srow = reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(q.state) +
                                                     (size_t)r * n * AB);
  /* pass 1: sum of squares and the four head dot products */
  float ss = 0.0f, acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int u = tid; u < nu; u += kBlock) {
    float v[EL];
    head_unpack<ACT>(srow[u], v);
#pragma unroll
    for (int e = 0; e < EL; ++e) ss = fmaf(v[e], v[e], ss);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4* w = reinterpret_cast<const float4*>(q.w_head + (size_t)i * n + (size_t)u * EL);
#pragma unroll
      for (int c = 0; c < EL / 4; ++c) {
        const float4 wv = w[c];
        float a = acc[i];
        a = fmaf(wv.x, v[4 * c], a);
        a = fmaf(wv.y, v[4 * c + 1], a);
        a = fmaf(wv.z, v[4 * c + 2], a);
        a = fmaf(wv.w, v[4 * c + 3], a);
        acc[i] = a;
      }
    }
  }
  ss = wave_sum(ss);
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = wave_sum(acc[i]);
  if (lane == 0) {
    red[wave][0] = ss;
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][1 + i] = acc[i];
  }
  __syncthreads();
  if (tid < 4) {
    float S = 0.0f, A = 0.0f;
    for (int w = 0; w < kWaves; ++w) {
      S += red[w][0];
      A += red[w][1 + tid];
    }
    const float m = A / sqrtf(S / (float)n + q.eps_hc);
    const float v = 1.0f / (1.0f + expf(-(q.head_scale[0] * m + q.head_base[tid])));
    sh[tid] = v;
    if (q.pre) q.pre[r * 4 + tid] = v;
  }
  __syncthreads();
  const float pw[4] = {sh[0], sh[1], sh[2], sh[3]};
  /* pass 2: x and the sum of squares of the rounded x */
  float sx = 0.0f;
  for (int u = tid; u < hu; u += kBlock) {
    float x[EL];
    head_collapse<ACT>(srow, hu, u, pw, x);
#pragma unroll
    for (int e = 0; e < EL; ++e) sx = fmaf(x[e], x[e], sx);
    if (q.x)
      reinterpret_cast<uint4*>(static_cast<uint8_t*>(q.x) + (size_t)r * H * AB)[u] =
          head_pack<ACT>(x);
  }
  sx = wave_sum(sx);
  if (lane == 0) red[wave][0] = sx;
  __syncthreads();
  if (tid == 0) {
    float S = 0.0f;
    for (int w = 0; w < kWaves; ++w) S += red[w][0];
    sh[4] = 1.0f / sqrtf(S / (float)H + q.eps_norm);
  }
  __syncthreads();
  const float inv = sh[4];
  /* pass 3: norm = act(x * inv * w) */
  const uint4* wrow = static_cast<const uint4*>(q.w_norm);
  uint4* orow = reinterpret_cast<uint4*>(static_cast<uint8_t*>(q.norm) + (size_t)r * H * AB);
  for (int u = tid; u < hu; u += kBlock) {
    float x[EL], w[EL];
    head_collapse<ACT>(srow, hu, u, pw, x);
    head_unpack<ACT>(wrow[u], w);
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] = x[e] * inv * w[e];
    orow[u] = head_pack<ACT>(x);
  }
}

int launch_head(int act, int rows, int H, float eps_hc, float eps_norm, const void* state,
                const float* w_head, const float* head_scale, const float* head_base,
                const void* w_norm, float* pre, void* x, void* norm, void* stream) {
  HeadParams q;
  q.H = H;
  q.eps_hc = eps_hc;
  q.eps_norm = eps_norm;
  q.state = state;
  q.w_head = w_head;
  q.head_scale = head_scale;
  q.head_base = head_base;
  q.w_norm = w_norm;
  q.pre = pre;
  q.x = x;
  q.norm = norm;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (act == F32)
    hipLaunchKernelGGL(k_hc_head<F32>, dim3(rows), dim3(kBlock), 0, st, q);
  else
    hipLaunchKernelGGL(k_hc_head<BF16>, dim3(rows), dim3(kBlock), 0, st, q);
  return (int)hipGetLastError();
}

}  // namespace mono
