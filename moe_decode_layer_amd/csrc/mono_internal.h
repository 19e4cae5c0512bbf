/*
 * libmonolayer internals shared by the device code (mono_kernels.h) and the
 * host code (mono_api.cpp): kernel parameter block, workspace layout, limits.
 */
#ifndef MONOLAYER_INTERNAL_H
#define MONOLAYER_INTERNAL_H

#include <stddef.h>
#include <stdint.h>

#include "../../include/mono.h"

namespace mono {

constexpr int kBlock = 512;          /* threads per workgroup, every kernel */
constexpr int kWaves = kBlock / 64;  /* wave64 */
constexpr int kMaxRows = 8;
constexpr int kMaxTopK = 16;
constexpr int kMaxExperts = 512;
constexpr int kNMix = 24;            /* 4 pre + 4 post + 16 comb */
constexpr int kNCarry = kNMix + 1;   /* raw mix sums + sum of squares */
constexpr int kMixChunk = 512;       /* flattened HC-row elements per mix partial (a multiple of 256) */
constexpr int kMixGroup = 6;         /* mix outputs per mix-partial task (24 = 4 groups) */
constexpr int kMaxGrid = 1024;       /* upper bound on persistent workgroups (workspace sizing) */
constexpr int kLdsActBytes = 114688; /* LDS for the activation rows of the matvec phases */
constexpr int kLdsHidBytes = 81920;  /* of which: staged SwiGLU hidden rows in the down phase */
constexpr uint32_t kDefaultSpin = 200000000u; /* 2 s of the 100 MHz real-time counter */

/* Control words at the head of the workspace (u32 indices). */
enum {
  CTL_ERR = 8,       /* 4 words: flag, phase, workgroup, count */
  CTL_SPIN = 16,     /* bounded-wait limit in real-time ticks (0 = default) */
  CTL_FAULT_WG = 17, /* workgroup that withholds its published values (-1 = none) */
  CTL_FAULT_PHASE = 18,
  CTL_TRACE = 19,    /* nonzero: the fused launch records per-phase timestamps */
  CTL_XEND64 = 60,   /* uint64 arrival counter of the unfused expand (last-arriver election) */
  CTL_START64 = 128, /* uint64 launch-start counters of the fused launch, one per group of
                        workgroups (blockIdx % 8), each in its own 256-byte block */
  CTL_WORDS = 128 + 8 * 64
};
constexpr int kStartStride = 64; /* u32 words between two start counters */

/* Points where the fused launch's workgroups exchange values (reported in the error word and
 * named by fault injection); PH_END is the expand's wait and the carry reduction. */
enum { PH_MIX = 1, PH_ROUTER = 2, PH_GATEUP = 3, PH_END = 4 };
constexpr int kBarGroups = 8; /* one start counter per group of workgroups (blockIdx % 8) */

struct Mat {
  int fmt;
  const uint8_t* gate;
  const uint8_t* up;
  const uint8_t* down;
  const uint8_t* gate_s;
  const uint8_t* up_s;
  const uint8_t* down_s;
};

/* Everything a kernel needs. Inputs of a phase are read through these pointers, so the fused
 * launch points them into the workspace and the unfused calls at the caller's buffers. */
struct Params {
  int R, H, E, K, I, Is, iters, nslice;
  float rho, eps_hc, eps_norm;
  int aq8; /* MXFP8 round trip of the activations entering the MXFP4 experts (routed is MXFP4) */
  uint32_t jitter, jseed; /* race shaker of the fused launch: largest delay in ticks (0 = off) */
  /* weights */
  const float* w_mix;
  const float* hc_scale;
  const float* hc_base;
  const void* w_norm;
  const float* w_router;
  const float* bias;
  const float* w_mix_next;
  Mat routed, shared;
  /* step inputs */
  const void* state;
  const float* carry_in;
  const void* norm_in;  /* router / experts input when not produced in-kernel */
  const int32_t* idx_in;
  const float* w_in;
  const void* block_in;
  const float* post_in;
  const float* comb_in;
  /* outputs */
  float* mixes;
  float* pre;
  float* post;
  float* comb;
  void* x;
  void* norm;
  float* logits;
  int32_t* idx;
  float* weights;
  void* h_routed;    /* [R][K][I] tagged hidden rows of the selected experts */
  void* h_shared;    /* [R][Is] tagged hidden rows of the shared expert */
  void* shared_out;
  float* routed_out;
  void* block;
  void* state_out;
  float* carry_out;
  float* carry_ws;   /* workspace copy of the carry */
  /* workspace scratch */
  uint64_t* mix_part; /* [nchunk][R][25] tagged mix partial sums: value bits | tag << 32 */
  float* carry_part; /* [R * 25][grid] tagged partials: value bits | epoch tag << 32 */
  uint64_t* pre_done; /* [grid] launch tag of each workgroup once it has read all of the state */
  uint64_t* y_part;   /* [R][Kp][H] tagged down-projection outputs, Kp = K + (shared expert ? 1
                       * : 0), slot K the shared expert */
  uint64_t* lgp;     /* [R][E] tagged router logits (same format) */
  uint64_t* trace;   /* [grid][32] real-time stamps */
  size_t tag_words; /* u64 words from carry_part through lgp cleared by the workspace init */
  uint32_t* ctl;
};

/* Workspace layout (byte offsets, 256-byte aligned regions). */
struct WsLayout {
  size_t ctl, mix_part, carry_part, pre_done, y_part, lgp, lgp_end, mixes, pre, post, comb, x, norm, logits, idx, weights,
      h_routed, h_shared, shared, routed, block, carry, trace, total;
};

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

/* Router steps (of 256 f32 values) a wave holds in registers at once. */
constexpr int kRouterCh = 4;

/* Phase timestamps per workgroup in the trace region. */
constexpr int kTraceSlots = 32;

inline WsLayout ws_layout(const mono_shape& s) {
  const size_t R = s.rows > 0 ? s.rows : 1, H = s.hidden, E = s.n_experts, k = s.top_k,
               I = s.inter, Is = s.shared_inter;
  const size_t ab = s.act == MONO_F32 ? 4 : 2;
  const size_t nchunk = (4 * H + kMixChunk - 1) / kMixChunk;
  WsLayout L;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  L.ctl = take(CTL_WORDS * 4);
  L.carry_part = take((size_t)kMaxGrid * R * kNCarry * 8);
  L.pre_done = take((size_t)kMaxGrid * 8);
  L.y_part = take(R * (k + 1) * H * 8);
  L.mix_part = take(nchunk * R * kNCarry * 8);
  L.lgp = take(R * E * 8);
  /* hidden rows, tagged: each value with the launch tag beside it (bf16 | tag16 << 16 in a
   * uint32, or f32 | tag32 << 32 in a uint64) */
  L.h_routed = take(R * k * I * ab * 2);
  L.h_shared = take(R * (Is > 0 ? Is : 1) * ab * 2);
  L.lgp_end = o; /* the workspace init clears [carry_part, lgp_end) */
  L.mixes = take(R * kNMix * 4);
  L.pre = take(R * 4 * 4);
  L.post = take(R * 4 * 4);
  L.comb = take(R * 16 * 4);
  L.x = take(R * H * ab);
  L.norm = take(R * H * ab);
  L.logits = take(R * E * 4);
  L.idx = take(R * k * 4);
  L.weights = take(R * k * 4);
  L.shared = take(R * H * ab);
  L.routed = take(R * H * 4);
  L.block = take(R * H * ab);
  L.carry = take(R * kNCarry * 4);
  L.trace = take((size_t)kMaxGrid * kTraceSlots * 8);
  L.total = o;
  return L;
}

/* Launchers (mono_launch.hip). Each returns a hipError_t as int. */
enum Kernel {
  K_MIX_PARTIALS,
  K_HC_PRE,
  K_ROUTER_LOGITS,
  K_SELECT,
  K_GATEUP,
  K_DOWN,
  K_EXPAND,
  K_FFN_LAYER,
  K_WS_INIT,
  K_WS_DEBUG
};
int launch(Kernel k, const Params& p, int act, int rfmt, int sfmt, int grid, void* stream);
/* Sets the thread's mono_last_error() text (printf format). */
void set_last_error(const char* fmt, ...);
int grid_size_for_device(int device);
/* Workgroups of the fused launch for (act, routed format, shared format, rows > 1) that one
 * compute unit holds at once (hipOccupancyMaxActiveBlocksPerMultiprocessor), or -1 for a
 * combination that is not instantiated. */
int max_active_persistent(int act, int rfmt, int sfmt, int rows);

}  // namespace mono

#endif /* MONOLAYER_INTERNAL_H */
