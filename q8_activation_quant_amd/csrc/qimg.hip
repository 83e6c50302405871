// qimg.hip — shared Q8_1 activation image: fused producers and Q4_0 MMVQ readers for gfx950.
//
// Sources (web pages; cited by title and section):
//   [P1] "Share temporary Q8_1 activation images" (llama.cpp fork, PR #117): Overview,
//        Coverage, GLU producer evidence.
//   [P2] "r49 - A-quantize prepass shared-A dedup: consecutive-window memoization":
//        section 1 Background, section 2 Principle.
//   [P3] "qwen3_5 CUDA: a captured bucket's padding rows no longer go through the routed
//        experts" (TensorFold PR #1047): What this changes, Receipt.
//
// Kernels
//   emit_kernel<OP,JW>       producers, per live row (RMS: a few rows each split over several
//                            workgroups that all take the same row sum; element-wise ops: row
//                            slices): (RMS reduction) -> f32 output -> per 32-block Q8_1
//                            quantization, all in one pass.
//   mmvq_tiled_kernel<N,M,G> ordinary Q4_0 x Q8_1 readers on the matrix cores
//                            (v_mfma_i32_16x16x64_i8) over tiled weights, the live image rows as
//                            columns; M = 2: block-dot export; M = 3, 4: Q8_0, Q4_1 weights.
//   mmq_kernel               prefill reader for many image rows (v_mfma_i32_32x32x32_i8).
//   mmvq_routed_kernel<KU,S> routed readers: the plan of the live pairs built by every
//                            workgroup (in LDS; S: at most 64 pairs, in registers by a wave-wide
//                            sort), then (expert, pass, tile) units streamed in two K halves.
//   moe_router_kernel, moe_topk_kernel, moe_combine_kernel: the rest of a routed MoE FFN.
//   tile_weights_kernel<F>   one-time reordering of standard Q4_0 / Q8_0 / Q4_1 planes into
//                            reader tiles.
//   eval_math_kernel<FN>     the producers' scalar math over ranges of f32 inputs (a check hook).
//
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off (no fast-math), so every float
// operation written here is one IEEE binary32 operation with round-to-nearest-even; f32
// division and square root are the correctly rounded ones.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <type_traits>
#include <string.h>
#include <mutex>

#include "qimg.h"

namespace {

// ---------------------------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint32_t h) {
  return __half2float(__ushort_as_half((unsigned short)(h & 0xffffu)));
}
// f32 -> fp16, round-to-nearest-even, subnormals kept. The empty asm makes f an opaque f32
// register: without it the compiler folds a conversion of a product, fp16(a * b), into one
// mixed-precision multiply-add (v_fma_mix) that rounds the exact product once, straight to
// fp16, instead of rounding it to f32 first; the two differ when the f32 product is an fp16
// tie (the image's s = fp16(f32(sum * d)) is specified with both roundings).
__device__ __forceinline__ uint32_t f2h(float f) {
  asm volatile("" : "+v"(f));
  return (uint32_t)__half_as_ushort(__float2half_rn(f));
}

__device__ __forceinline__ int clamp_live(const int32_t* live_rows, int rows, int* clamped) {
  int live = rows;
  if (live_rows) {
    live = *live_rows;
    if (live < 0 || live > rows) {
      if (clamped) *clamped = 1;
      live = live < 0 ? 0 : rows;
    }
  }
  return live;
}

// Cross-lane moves without LDS: DPP (quad_perm, row mirrors) within a 16-lane row, and the
// gfx950 permlane swaps across rows. pair_sum_* return v(l) + v(partner) where the partner set
// pairs lanes exactly as a balanced pairwise tree over lane index needs when every lane of a
// group already holds that group's value (the sum of a pair is the same in both lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_n(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xb1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4e;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8 lanes
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16 lanes
__device__ __forceinline__ float pair_sum_rows(float v) {  // lanes l and l ^ 16
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float pair_sum_halves(float v) {  // lanes l and l ^ 32
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// Balanced pairwise tree over the 64 lanes in lane order (every lane receives the total).
__device__ __forceinline__ float wave_tree_sum(float v) {
  v = v + dpp_f<kDppXor1>(v);
  v = v + dpp_f<kDppXor2>(v);
  v = v + dpp_f<kDppHalfMirror>(v);
  v = v + dpp_f<kDppMirror>(v);
  v = pair_sum_rows(v);
  return pair_sum_halves(v);
}

// XOR over the 64 lanes (every lane receives it)
__device__ __forceinline__ uint32_t wave_xor(uint32_t v) {
  v ^= (uint32_t)dpp_n<kDppXor1>((int)v);
  v ^= (uint32_t)dpp_n<kDppXor2>((int)v);
  v ^= (uint32_t)dpp_n<kDppHalfMirror>((int)v);
  v ^= (uint32_t)dpp_n<kDppMirror>((int)v);
  const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // lanes l and l ^ 16
  v = r[0] ^ r[1];
  const auto h = __builtin_amdgcn_permlane32_swap(v, v, false, false);  // lanes l and l ^ 32
  return h[0] ^ h[1];
}

// balanced pairwise tree over a lane's JW values (JW a power of two)
template <int JW>
__device__ __forceinline__ float tree_sum(float (&v)[JW]) {
#pragma unroll
  for (int w = JW; w > 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  }
  return v[0];
}

// exp_q: Cody-Waite reduction by ln 2 split into a 12-bit-short high part and an f32 low part,
// degree-7 Taylor polynomial of e^r with coefficients 1/k! rounded to f32 (Horner, fma), then
// scaling by 2^n. NaN passes through, x > 88.8 gives +inf, x < -86 gives +0 (no subnormal
// results). The GLU pages give the activation formulas but no exp; this fixed sequence makes
// the f32 producer output a function of its inputs alone.
__device__ __forceinline__ float exp_q(float x) {
  if (x != x) return x;
  if (x > 88.8f) return __builtin_huge_valf();
  if (x < -86.0f) return 0.0f;
  constexpr float kLog2e = 0x1.715476p+0f;   // log2(e) rounded to f32
  constexpr float kLn2Hi = 0x1.62ep-1f;      // ln 2 to f32, low 12 significand bits cleared
  constexpr float kLn2Lo = 0x1.0bfbe8p-15f;  // f32 nearest ln 2 - kLn2Hi
  const float n = __builtin_rintf(x * kLog2e);
  float r = __builtin_fmaf(-n, kLn2Hi, x);
  r = __builtin_fmaf(-n, kLn2Lo, r);
  float p = (float)(1.0 / 5040.0);
  p = __builtin_fmaf(p, r, (float)(1.0 / 720.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 120.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 24.0));
  p = __builtin_fmaf(p, r, (float)(1.0 / 6.0));
  p = __builtin_fmaf(p, r, 0.5f);
  p = __builtin_fmaf(p, r, 1.0f);
  p = __builtin_fmaf(p, r, 1.0f);
  return __builtin_ldexpf(p, (int)n);
}

// erfc_q(z), z >= 0: Numerical Recipes' Chebyshev fit "erfcc" (fractional error < 1.2e-7):
// erfc(z) = t * exp(-z^2 - 1.26551223 + t*P(t)), t = 1/(1 + z/2), P by Horner with fma.
__device__ __forceinline__ float erfc_q(float z) {
  const float t = 1.0f / (1.0f + 0.5f * z);
  float p = 0.17087277f;
  p = __builtin_fmaf(p, t, -0.82215223f);
  p = __builtin_fmaf(p, t, 1.48851587f);
  p = __builtin_fmaf(p, t, -1.13520398f);
  p = __builtin_fmaf(p, t, 0.27886807f);
  p = __builtin_fmaf(p, t, -0.18628806f);
  p = __builtin_fmaf(p, t, 0.09678418f);
  p = __builtin_fmaf(p, t, 0.37409196f);
  p = __builtin_fmaf(p, t, 1.00002368f);
  p = __builtin_fmaf(p, t, -1.26551223f);
  const float arg = __builtin_fmaf(-z, z, p);
  return t * exp_q(arg);
}

// [P1] Coverage: F32 SwiGLU and GeGLU-erf producers keep their formulas.
//   SwiGLU    act(g) = g / (1 + exp(-g))
//   GeGLU-erf act(g) = (0.5 g) * (1 + erf(g / sqrt 2)), 1 + erf(z) = erfc(-z) (z < 0)
//                                                               or 2 - erfc(z) (z >= 0)
__device__ __forceinline__ float swiglu_act(float g) {
  const float e = exp_q(-g);
  const float den = 1.0f + e;
  return g / den;
}
__device__ __forceinline__ float geglu_erf_act(float g) {
  constexpr float kSqrtHalf = 0x1.6a09e6p-1f;  // 1/sqrt(2) rounded to f32
  const float z = g * kSqrtHalf;
  const float ope = (z < 0.0f) ? erfc_q(-z) : 2.0f - erfc_q(z);
  return (0.5f * g) * ope;
}

// Device router and top-k ("qwen3_5 CUDA: a captured bucket's padding rows no longer go through
// the routed experts", What this changes: router and top-k read the live count; padding rows
// get no picks and their outputs stay unwritten).
//
// Router: logits[t][e] = x[t] . W[e] over K for live rows, in the order of the RMS sum of
// squares with products: leaf c (4 elements) = fma(x3,w3, fma(x2,w2, fma(x1,w1, x0*w0)));
// lane l owns leaves c = l + 64 j, j < Jp (next power of two >= ceil(K/256), missing leaves
// +0), summed by a pairwise tree over j; the 64 lane sums by a pairwise tree (wave_tree_sum).
// One workgroup per (block of EB experts, group of RT rows, RT = 8 or 1): wave w holds leaves j in
// [w JW, (w+1) JW) of every row and expert (JW = Jp / W), sums them by the lower levels of the
// tree, and the W wave partials are combined through LDS by its top levels; the (expert, row)
// dots are then finished by the waves in turn. The activations of the rows are loaded once per
// workgroup and shared by its EB experts; all loads of a wave go out together.
struct RouterArgs {
  const float* x;  // [bucket][ldx]
  int64_t ldx;
  const float* w;  // [E][K]
  const int32_t* live_rows;
  float* logits;   // [bucket][ldl]
  int64_t ldl;
  int32_t rows, E, K;
};

template <int JW, int EB, int RT>
__global__ __launch_bounds__(1024) void moe_router_kernel(RouterArgs a) {
  static_assert(RT == 8 || RT == 1, "rows per workgroup");
  const int live = clamp_live(a.live_rows, a.rows, nullptr);
  const int t0 = blockIdx.y * RT;
  if (t0 >= live) return;
  extern __shared__ __align__(16) unsigned char smem[];
  float* part = reinterpret_cast<float*>(smem);  // [W][EB][RT][64]
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int e0 = blockIdx.x * EB;
  const int ne = a.E - e0 < EB ? a.E - e0 : EB;
  const int nt = live - t0 < RT ? live - t0 : RT;
  const int C = a.K >> 2;
  // leaves past K re-read leaf 0 (in bounds) and count as +0; experts past E re-read expert e0
  // and rows past the live count re-read row t0 (their results are not stored). All 8 rows'
  // activation leaves are loaded at once (one round trip) unless the rows are long (more than
  // 2 leaves per lane), then row by row.
  constexpr int XT = RT == 1 ? 1 : (EB > 1 || JW <= 2) ? 8 : 1;
  float4 wv[EB][JW], xv[XT][JW];
  auto load_x = [&](int t, float4 (&dst)[JW]) {
    const float* xr = a.x + (int64_t)(t0 + (t < nt ? t : 0)) * a.ldx;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int c = lane + 64 * (w * JW + jj);
      dst[jj] = *reinterpret_cast<const float4*>(xr + 4 * (c < C ? c : 0));
    }
  };
#pragma unroll
  for (int b = 0; b < EB; ++b) {
    const float* wr = a.w + (int64_t)(e0 + (b < ne ? b : 0)) * a.K;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int c = lane + 64 * (w * JW + jj);
      wv[b][jj] = *reinterpret_cast<const float4*>(wr + 4 * (c < C ? c : 0));
    }
  }
  if constexpr (XT == 8) {
#pragma unroll
    for (int t = 0; t < 8; ++t) load_x(t, xv[t]);
  } else if constexpr (RT == 1) {
    load_x(0, xv[0]);
  }
#pragma unroll
  for (int b = 0; b < EB; ++b)
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      if constexpr (XT == 1 && RT == 8) {
        if (t >= nt) break;
        load_x(t, xv[0]);
      }
      float leaf[JW];
#pragma unroll
      for (int jj = 0; jj < JW; ++jj) {
        const int c = lane + 64 * (w * JW + jj);
        const float4 q = wv[b][jj], v = xv[XT == 8 ? t : 0][jj];
        leaf[jj] = c < C ? __builtin_fmaf(v.w, q.w, __builtin_fmaf(v.z, q.z,
                                          __builtin_fmaf(v.y, q.y, v.x * q.x)))
                         : 0.0f;
      }
      part[((w * EB + b) * RT + t) * 64 + lane] = tree_sum<JW>(leaf);
    }
  __syncthreads();
  for (int q = w; q < EB * RT; q += W) {
    const int b = q / RT, t = q % RT;
    if (b < ne && t < nt) {
      float v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = i < W ? part[((i * EB + b) * RT + t) * 64 + lane] : 0.0f;
      for (int n = W; n > 1; n >>= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
          if (i < n / 2) v[i] = v[2 * i] + v[2 * i + 1];
      const float sum = wave_tree_sum(v[0]);
      if (lane == 0) a.logits[(int64_t)(t0 + t) * a.ldl + e0 + b] = sum;
    }
  }
}

// Top-k: one wave per live row. Each lane keeps the best of its own experts not yet taken as
// a 64-bit key (order-preserving bits of the logit, -0 made +0, then the complemented id, so
// equal logits rank the lower id first) and every round takes the wave maximum of the keys
// by DPP and permlane moves; only the winning lane rescans its experts. Routing weights: the
// softmax over the selected logits, e_r = exp_q(l_r - l_0), s = e_0 + e_1 + ... in ascending
// r from +0, w_r = e_r / s. Lane r keeps pick r.
struct TopkArgs {
  const float* logits;  // [bucket][ldl]
  int64_t ldl;
  const int32_t* live_rows;
  int32_t* ids;         // [bucket][k]
  float* w;             // [bucket][k] or null
  int32_t rows, E, k;
};

__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t u = __float_as_uint(v == 0.0f ? 0.0f : v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
template <int CTRL>
__device__ __forceinline__ void key_max_dpp(uint32_t& hi, uint32_t& lo) {
  const uint32_t oh = (uint32_t)dpp_n<CTRL>((int)hi), ol = (uint32_t)dpp_n<CTRL>((int)lo);
  if (oh > hi || (oh == hi && ol > lo)) {
    hi = oh;
    lo = ol;
  }
}
__device__ __forceinline__ void key_max_pair(uint32_t& hi, uint32_t& lo, bool halves) {
  const auto h = halves ? __builtin_amdgcn_permlane32_swap(hi, hi, false, false)
                        : __builtin_amdgcn_permlane16_swap(hi, hi, false, false);
  const auto l = halves ? __builtin_amdgcn_permlane32_swap(lo, lo, false, false)
                        : __builtin_amdgcn_permlane16_swap(lo, lo, false, false);
  const bool second = h[1] > h[0] || (h[1] == h[0] && l[1] > l[0]);
  hi = second ? h[1] : h[0];
  lo = second ? l[1] : l[0];
}

// PER keys per lane: E <= 64 PER (the launch picks the smallest power of two that holds E)
template <int PER>
__global__ __launch_bounds__(64) void moe_topk_kernel(TopkArgs a) {
  const int t = blockIdx.x;
  if (t >= clamp_live(a.live_rows, a.rows, nullptr)) return;
  const int lane = threadIdx.x;
  constexpr int kPer = PER;
  const float* lr = a.logits + (int64_t)t * a.ldl;
  uint32_t key[kPer];
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const int e = lane + 64 * i;
    // unconditional in-bounds load; 0 (below every logit's key) where there is no expert
    const float v = lr[e < a.E ? e : 0];
    key[i] = order_key(v) & (e < a.E ? 0xffffffffu : 0u);
  }
  // this lane's best: slot bi with key bk (the largest; ties to the lower slot = lower id)
  int bi = 0;
  uint32_t bk = 0;
  auto local_best = [&]() {
    bi = 0;
    bk = key[0];
#pragma unroll
    for (int i = 1; i < kPer; ++i)
      if (key[i] > bk) {
        bk = key[i];
        bi = i;
      }
  };
  local_best();
  int my_id = 0;
  float my_l = 0.0f;
  for (int r = 0; r < a.k; ++r) {
    uint32_t hi = bk, lo = ~(uint32_t)(lane + 64 * bi);
    key_max_dpp<kDppXor1>(hi, lo);
    key_max_dpp<kDppXor2>(hi, lo);
    key_max_dpp<kDppHalfMirror>(hi, lo);
    key_max_dpp<kDppMirror>(hi, lo);
    key_max_pair(hi, lo, false);
    key_max_pair(hi, lo, true);
    const int id = (int)~lo;
    if (lane == r) {
      my_id = id;
      const uint32_t u = (hi & 0x80000000u) ? (hi & 0x7fffffffu) : ~hi;
      my_l = __uint_as_float(u);
    }
    if ((id & 63) == lane) {  // the winner's lane takes it and rescans
#pragma unroll
      for (int i = 0; i < kPer; ++i)
        if (i == (id >> 6)) key[i] = 0u;
      local_best();
    }
  }
  if (lane < a.k) a.ids[(int64_t)t * a.k + lane] = my_id;
  if (a.w) {
    const float m = __shfl(my_l, 0, 64);
    const float ev = exp_q(my_l - m);
    float sum = 0.0f;
    for (int r = 0; r < a.k; ++r)
      sum = sum + __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(ev), r));
    if (lane < a.k) a.w[(int64_t)t * a.k + lane] = ev / sum;
  }
}

// MoE combine ("qwen3_5 CUDA: a captured bucket's padding rows no longer go through the
// routed experts", What this changes: only live rows are combined, padding output rows stay
// unwritten). out[t][n] = sum over slots s (ascending) whose expert id is in [0, E) of
// w[t][s] * x[t][s][n], one f32 fma per slot from +0. Grid (ceil(N/1024), bucket); a thread
// owns 4 consecutive n. The x rows of up to 8 slots are loaded before any is used.
struct CombineArgs {
  const float* x;          // [bucket][top_k][ld_pair]
  int64_t ld_pair;
  const float* w;          // [bucket][top_k]
  const int32_t* ids;      // [bucket][top_k]
  const int32_t* live_rows;
  float* out;              // [bucket][ldo]
  int64_t ldo;
  int32_t rows, top_k, E, N;
};

__global__ __launch_bounds__(256) void moe_combine_kernel(CombineArgs c) {
  const int t = blockIdx.y;
  if (t >= clamp_live(c.live_rows, c.rows, nullptr)) return;
  const int n4 = blockIdx.x * 256 + threadIdx.x;
  if (4 * n4 >= c.N) return;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int s0 = 0; s0 < c.top_k; s0 += 8) {
    float4 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {  // slots past top_k re-read the last slot (unused)
      const int s = s0 + j < c.top_k ? s0 + j : c.top_k - 1;
      v[j] = *reinterpret_cast<const float4*>(c.x + (int64_t)(t * c.top_k + s) * c.ld_pair + 4 * n4);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int p = t * c.top_k + s0 + j;
      if (s0 + j < c.top_k && c.ids[p] >= 0 && c.ids[p] < c.E) {
        const float wp = c.w[p];
        acc.x = __builtin_fmaf(wp, v[j].x, acc.x);
        acc.y = __builtin_fmaf(wp, v[j].y, acc.y);
        acc.z = __builtin_fmaf(wp, v[j].z, acc.z);
        acc.w = __builtin_fmaf(wp, v[j].w, acc.w);
      }
    }
  }
  *reinterpret_cast<float4*>(c.out + (int64_t)t * c.ldo + 4 * n4) = acc;
}

// The other GLU variants ([P1] Coverage: F32 ReGLU, GeGLU, GeGLU-quick, SwiGLU-OAI and
// SwiGLU-clamp producers keep their formulas and alpha/limit parameters).
//   ReGLU        act(g) = max(g, 0)  (g > 0 ? g : 0)
//   GeGLU        act(g) = 0.5 g (1 + tanh(sqrt(2/pi) (g + 0.044715 g^3))), evaluated through
//                0.5 (1 + tanh z) = 1 / (1 + exp(-2 z)) as g / (1 + exp_q(-c2 (g + 0.044715 g^3))),
//                c2 = 2 sqrt(2/pi) (no cancellation for either sign of g)
//   GeGLU-quick  act(g) = g sigmoid(1.702 g)
//   SwiGLU-OAI   g' = min(g, limit), u' = clamp(u, -limit, limit), y = g' sigmoid(alpha g') (u' + 1)
//   SwiGLU-clamp g' = min(g, limit), u' = clamp(u, -limit, limit), y = silu(g') u'
__device__ __forceinline__ float g_sigmoid(float g, float c) {
  const float e = exp_q(-(c * g));
  const float den = 1.0f + e;
  return g / den;
}
__device__ __forceinline__ float reglu_act(float g) { return g > 0.0f ? g : 0.0f; }
__device__ __forceinline__ float geglu_tanh_act(float g) {
  constexpr float kC2 = 0x1.988454p+0f;      // 2 sqrt(2/pi) rounded to f32
  constexpr float kCubic = 0x1.6e4e26p-5f;   // 0.044715 rounded to f32
  const float g3 = (g * g) * g;
  const float inner = g + kCubic * g3;
  const float e = exp_q(-(kC2 * inner));
  const float den = 1.0f + e;
  return g / den;
}
__device__ __forceinline__ float geglu_quick_act(float g) {
  return g_sigmoid(g, 0x1.b3b646p+0f);  // 1.702 rounded to f32
}

// ---------------------------------------------------------------------------------------------
// Producer: workgroups of live rows (RMS: a whole row, or for few rows the same row in several
// workgroups that each take the whole row's sum and finish a share of it; element-wise ops: row
// slices of up to kEltWaves waves).
// Element mapping: leaf c covers elements 4c..4c+3; lane l of wave w holds leaves
// c = l + 64 j for j in [w*JW, (w+1)*JW). A 32-element block is 8 consecutive leaves, i.e. 8
// consecutive lanes at the same j, so the block amax and code sum are 3-step lane reductions.
// RMS sum of squares (the fixed order, independent of the wave count): leaf value
// fma(x3,x3, fma(x2,x2, fma(x1,x1, x0*x0))); per lane a balanced pairwise tree over j (padded
// to a power of two Jp with zeros), whose top levels are taken across waves through LDS; then
// a balanced pairwise tree over the 64 lanes (xor butterfly, masks 1..32).
// ---------------------------------------------------------------------------------------------
enum : int {
  OP_RMS = 0, OP_SWIGLU = 1, OP_GEGLU = 2, OP_QUANT = 3,
  OP_REGLU = 4, OP_GEGLU_TANH = 5, OP_GEGLU_QUICK = 6, OP_SWIGLU_OAI = 7, OP_SWIGLU_CLAMP = 8
};
constexpr bool is_glu(int op) { return op != OP_RMS && op != OP_QUANT; }

// y for one element of a GLU producer: act(g) * u, or the clamped forms
template <int OP>
__device__ __forceinline__ float glu_pair(float g, float u, float alpha, float limit) {
  if constexpr (OP == OP_SWIGLU) return swiglu_act(g) * u;
  else if constexpr (OP == OP_GEGLU) return geglu_erf_act(g) * u;
  else if constexpr (OP == OP_REGLU) return reglu_act(g) * u;
  else if constexpr (OP == OP_GEGLU_TANH) return geglu_tanh_act(g) * u;
  else if constexpr (OP == OP_GEGLU_QUICK) return geglu_quick_act(g) * u;
  else {
    const float gg = g < limit ? g : limit;
    const float uu = u < -limit ? -limit : (u > limit ? limit : u);
    if constexpr (OP == OP_SWIGLU_OAI) return g_sigmoid(gg, alpha) * (uu + 1.0f);
    else return swiglu_act(gg) * uu;
  }
}

// Element-wise evaluation of the activation math above over a range of f32 bit patterns:
// out[i] = f(x) with x the float whose bits are first + i (mod 2^32). It runs the same inlined
// device functions the producers run, so every f32 input can be compared with a host
// evaluation of the same operation sequence.
// Two more functions cover the correctly rounded divisions and square root the producers rely
// on: 1/sqrt(x) (the RMS scale) and 1/(x/127) (the quantizer's scale and its reciprocal).
// The quantizer's block scale d = x/127 on its own and the f32 -> fp16 conversion of its
// stored halves (result bits in the low 16 bits of the output word) are the last two.
// Then the other GLU activations: ReGLU, GeGLU (tanh form), GeGLU-quick and the gate factor
// of SwiGLU-OAI at alpha 1.702, limit 7 (its output times (0 + 1)).
enum : int { MATH_EXP = 0, MATH_ERFC = 1, MATH_SWIGLU = 2, MATH_GEGLU = 3, MATH_RSQRT = 4,
             MATH_QSCALE = 5, MATH_QDIV = 6, MATH_F2H = 7, MATH_REGLU = 8, MATH_GEGLU_TANH = 9,
             MATH_GEGLU_QUICK = 10, MATH_OAI_GATE = 11 };

template <int FN>
__global__ __launch_bounds__(256) void eval_math_kernel(uint32_t first, int64_t n, float* out) {
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) {
    const float x = __builtin_bit_cast(float, first + (uint32_t)i);
    float v;
    if constexpr (FN == MATH_EXP) v = exp_q(x);
    else if constexpr (FN == MATH_ERFC) v = erfc_q(x);
    else if constexpr (FN == MATH_SWIGLU) v = swiglu_act(x);
    else if constexpr (FN == MATH_GEGLU) v = geglu_erf_act(x);
    else if constexpr (FN == MATH_RSQRT) v = 1.0f / __builtin_sqrtf(x);
    else if constexpr (FN == MATH_QSCALE) v = 1.0f / (x / 127.0f);
    else if constexpr (FN == MATH_QDIV) v = x / 127.0f;
    else if constexpr (FN == MATH_F2H) v = __builtin_bit_cast(float, f2h(x));
    else if constexpr (FN == MATH_REGLU) v = reglu_act(x);
    else if constexpr (FN == MATH_GEGLU_TANH) v = geglu_tanh_act(x);
    else if constexpr (FN == MATH_GEGLU_QUICK) v = geglu_quick_act(x);
    else v = glu_pair<OP_SWIGLU_OAI>(x, 0.0f, 1.702f, 7.0f);
    out[i] = v;
  }
}

struct EmitArgs {
  const float* a;      // rms: x; glu: gate; quant: y
  int64_t lda;
  const float* b;      // rms: gamma (may be null); glu: up
  int64_t ldb;
  float* y;            // f32 output (null for quant-only)
  int64_t ldy;
  uint8_t* codes;      // image codes plane (null: no image)
  uint32_t* ds;        // image ds plane
  const int32_t* live_rows;
  int32_t rows, K, Kb, RB;
  int32_t live_mul;    // rows per live count unit: 1, or top_k for per-slot (pair) rows
  float eps;
  const float* beta;   // rms: added after gamma (may be null)
  float scale;         // rms: final factor (1 keeps the value)
  float alpha, limit;  // SwiGLU-OAI / SwiGLU-clamp parameters
};

__device__ __forceinline__ void quantize_leaf(const float4 y, int row, int blk, int lane,
                                              const EmitArgs& p) {
  float amax = fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w)));
  // group of 8 lanes: max is exact in any order
  amax = fmaxf(amax, dpp_f<kDppXor1>(amax));
  amax = fmaxf(amax, dpp_f<kDppXor2>(amax));
  amax = fmaxf(amax, dpp_f<kDppHalfMirror>(amax));
  uint32_t packed = 0, dsw = 0;
  int sum = 0;
  const float d = amax / 127.0f;
  const float id = 1.0f / d;
  const bool zero = (amax == 0.0f) || !(__builtin_fabsf(id) < __builtin_huge_valf());
  if (!zero) {
    const int c0 = (int)__builtin_roundf(y.x * id);
    const int c1 = (int)__builtin_roundf(y.y * id);
    const int c2 = (int)__builtin_roundf(y.z * id);
    const int c3 = (int)__builtin_roundf(y.w * id);
    packed = (uint32_t)(c0 & 0xff) | ((uint32_t)(c1 & 0xff) << 8) |
             ((uint32_t)(c2 & 0xff) << 16) | ((uint32_t)(c3 & 0xff) << 24);
    sum = c0 + c1 + c2 + c3;
  }
  sum += dpp_n<kDppXor1>(sum);
  sum += dpp_n<kDppXor2>(sum);
  sum += dpp_n<kDppHalfMirror>(sum);
  if (!zero) dsw = f2h(d) | (f2h((float)sum * d) << 16);
  const int64_t blk_idx = (int64_t)row * p.RB + blk;
  reinterpret_cast<uint32_t*>(p.codes)[blk_idx * 8 + (lane & 7)] = packed;
  if ((lane & 7) == 0) p.ds[blk_idx] = dsw;
}

template <int OP, int JW>
__global__ __launch_bounds__(1024) void emit_kernel(EmitArgs p) {
  const int row = blockIdx.x;
  // padding rows (past the live count, in units of live_mul rows) stay untouched
  if (row >= clamp_live(p.live_rows, p.rows / p.live_mul, nullptr) * p.live_mul) return;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int C = p.K >> 2;
  // leaves of this workgroup: the whole row (RMS, whose sum needs it), or slice blockIdx.y of
  // W * 64 * JW leaves (the element-wise producers and the quantizer)
  const int c_off = OP == OP_RMS ? 0 : blockIdx.y * (W * 64 * JW);
  const float* arow = p.a + (int64_t)row * p.lda;
  // RMS rows split over gridDim.y workgroups: each sums the whole row (in the same order, so
  // every one gets the same scale) and normalizes, stores and quantizes only its share of the
  // leaf groups (64 leaves, one wave's jj-th), so that the per-element work of a few rows is
  // spread over many CUs
  const int gps = OP == OP_RMS ? (W * JW) / (int)gridDim.y : 0;  // leaf groups per share
  const int g_lo = gps * (int)blockIdx.y;
  auto mine = [&](int jj) { return OP != OP_RMS || (unsigned)(w * JW + jj - g_lo) < (unsigned)gps; };

  // all input loads of the row go out at once (in bounds: leaves past K re-read leaf 0 and
  // are zeroed): x (or gate, or y) and gamma (or up)
  float4 v[JW], u[JW], bt[JW];
  const float* brow = is_glu(OP) ? p.b + (int64_t)row * p.ldb : p.b;
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
    const int c = c_off + lane + 64 * (w * JW + jj);
    const int cc = c < C ? c : 0;
    v[jj] = *reinterpret_cast<const float4*>(arow + 4 * cc);
    if (c >= C) v[jj] = make_float4(0, 0, 0, 0);
    if (OP != OP_QUANT && brow && mine(jj)) u[jj] = *reinterpret_cast<const float4*>(brow + 4 * cc);
    if (OP == OP_RMS && p.beta && mine(jj)) bt[jj] = *reinterpret_cast<const float4*>(p.beta + 4 * cc);
  }

  if constexpr (OP == OP_RMS) {
    __shared__ float part[16][64];
    float leaf[JW];
#pragma unroll
    for (int jj = 0; jj < JW; ++jj)
      leaf[jj] = __builtin_fmaf(v[jj].w, v[jj].w,
                 __builtin_fmaf(v[jj].z, v[jj].z,
                 __builtin_fmaf(v[jj].y, v[jj].y, v[jj].x * v[jj].x)));
    part[w][lane] = tree_sum<JW>(leaf);
    __syncthreads();
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = i < W ? part[i][lane] : 0.0f;
    for (int n = W; n > 1; n >>= 1)
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (i < n / 2) t[i] = t[2 * i] + t[2 * i + 1];
    const float S = wave_tree_sum(t[0]);
    const float mean = S / (float)p.K;
    const float r = 1.0f / __builtin_sqrtf(mean + p.eps);
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      if (!mine(jj)) continue;
      const int c = c_off + lane + 64 * (w * JW + jj);
      float4 y;
      y.x = v[jj].x * r; y.y = v[jj].y * r; y.z = v[jj].z * r; y.w = v[jj].w * r;
      if (p.b && c < C) {
        const float4 g = u[jj];
        y.x = y.x * g.x; y.y = y.y * g.y; y.z = y.z * g.z; y.w = y.w * g.w;
      }
      if (p.beta && c < C) {  // RMS+MUL+ADD
        const float4 b = bt[jj];
        y.x = y.x + b.x; y.y = y.y + b.y; y.z = y.z + b.z; y.w = y.w + b.w;
      }
      // RMS+SCALE (a scale of 1 leaves every value unchanged)
      y.x = y.x * p.scale; y.y = y.y * p.scale; y.z = y.z * p.scale; y.w = y.w * p.scale;
      v[jj] = y;
    }
  } else if constexpr (is_glu(OP)) {
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int c = c_off + lane + 64 * (w * JW + jj);
      if (c < C) {
        const float4 uu = u[jj];
        float4 y;
        y.x = glu_pair<OP>(v[jj].x, uu.x, p.alpha, p.limit);
        y.y = glu_pair<OP>(v[jj].y, uu.y, p.alpha, p.limit);
        y.z = glu_pair<OP>(v[jj].z, uu.z, p.alpha, p.limit);
        y.w = glu_pair<OP>(v[jj].w, uu.w, p.alpha, p.limit);
        v[jj] = y;
      }
    }
  }

  // every original F32 store remains ([P1] Coverage)
  if constexpr (OP != OP_QUANT) {
    float* yrow = p.y + (int64_t)row * p.ldy;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int c = c_off + lane + 64 * (w * JW + jj);
      if (c < C && mine(jj)) *reinterpret_cast<float4*>(yrow + 4 * c) = v[jj];
    }
  }

  if (p.codes) {
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int blk = (c_off >> 3) + 8 * (w * JW + jj) + (lane >> 3);
      if (blk < p.Kb && mine(jj)) quantize_leaf(v[jj], row, blk, lane, p);  // whole 8-lane groups agree
    }
    // row padding blocks [Kb, RB) are zero bytes (written by the row's last slice)
    const int npad = blockIdx.y + 1 == gridDim.y ? p.RB - p.Kb : 0;
    uint32_t* cw = reinterpret_cast<uint32_t*>(p.codes) + ((int64_t)row * p.RB + p.Kb) * 8;
    for (int i = threadIdx.x; i < npad * 9; i += blockDim.x) {
      if (i < npad * 8) cw[i] = 0u;
      else p.ds[(int64_t)row * p.RB + p.Kb + (i - npad * 8)] = 0u;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Readers: Q4_0 x Q8_1 mat-vec on the matrix cores.
//
// Weights are read in a tiled Q4_0 order made once by qimg_q4_0_tile: the rows of a reader are
// cut into 16-row tiles and the K axis into chunks of 4 blocks; chunk (tile, s) is 1 KB of
// codes, lane l holding the 16 bytes of block 4 s + (l >> 4) of row (l & 15), then 128 B of
// fp16 scales in the same lane order. One wave load instruction thus moves 1 KB of contiguous
// weights, 16 bytes per lane (narrower or scattered loads run at a fraction of HBM bandwidth on
// this part).
//
// Dot products: v_mfma_i32_16x16x64_i8, D[m][n] = sum_k A[m][k] B[k][n], where lane l supplies
// A row (l & 15) and B column (l & 15) over k-group (l >> 4) (16 values each) and receives
// D rows 4 (l >> 4) .. +3 of column (l & 15).
//   B: the lane's own weight block, low nibbles (elements 0..15) in one MFMA and high nibbles
//      (elements 16..31) in a second one that accumulates onto the first.
//   A: block-diagonal over the four k-groups: row m carries image column 4 tg + (m & 3) of the
//      block in k-group (m >> 2), zero elsewhere.
// So D[4 g + v][n] of lane (n, g) is the block integer dot of its own block with image column
// 4 tg + v: the lane then applies its block scale, acc += d_w * (d_a * sumi - 8 s_a), summing
// its chunks in K order; the four k-group lanes of a row are added (lanes n, n+16: then with
// n+32), then the waves' K ranges in ascending wave order. The sum for one output does not
// depend on the other columns, the live count or the tiles of the workgroup.
//
// Image columns (live image rows; a routed expert's live pairs) are staged in LDS per pass of
// up to 8: codes [block][column][32], d_a and -8 s_a as f32 [block][8].
// ---------------------------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned v4u __attribute__((ext_vector_type(4)));

// Buffer resource word 3 for raw (untyped) buffer loads on this GPU family: 32-bit data
// format, no swizzle, no index stride. Offsets at or past num_records read as zero.
constexpr int kBufferFlags = 0x00020000;
// Cache policy of the weight loads: nontemporal (each weight byte is read once per launch; the
// streams run 5-10% faster than with the default policy)
constexpr int kNt = 2;

constexpr int kWaves = 8;  // routed readers
constexpr int kOrdWaves = 8;  // ordinary readers

typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4h as_v4h(uint64_t x) { return __builtin_bit_cast(v4h, x); }

struct ReaderDesc {
  const uint8_t* qs;  // tiled codes (1 KB per chunk)
  const uint16_t* d;  // tiled scales (64 per chunk)
  float* out;
  int64_t ld;         // ordinary: per image row; routed: per pair
  int32_t N;          // rows
  int32_t tiles;      // ceil(N / 16): tiles per expert
};

// Division of values in [0, 2^31) by a divisor fixed for a launch, as a multiply-high, an add
// and a shift (Granlund and Montgomery, "Division by invariant integers using multiplication",
// 1994): for 1 <= d < 2^31 with s = ceil(log2 d) and m = floor(2^32 (2^s - d) / d) + 1,
// floor(n / d) = (mulhi(n, m) + n) >> s; the sum stays below 2^32 since mulhi(n, m) <= n.
struct FastDiv {
  uint32_t m, s;
};
inline FastDiv fast_div(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  return FastDiv{(uint32_t)((((uint64_t)1 << 32) * ((1ull << s) - d)) / d + 1), s};
}
__device__ __forceinline__ int fdiv(int n, FastDiv f) {
  return (int)((__umulhi((uint32_t)n, f.m) + (uint32_t)n) >> f.s);
}

struct ReadArgs {
  ReaderDesc r[QIMG_MAX_READERS];
  int32_t tile_start[QIMG_MAX_READERS + 1];  // tile prefix over readers (within one expert)
  const uint8_t* codes;
  const uint32_t* ds;
  const int32_t* live_rows;
  const int32_t* ids;  // routed: [bucket][top_k]
  int32_t* ws;         // routed: plan workspace
  int32_t* sumi;       // debug: block dots of reader 0, [rows][N][Kb]
  int32_t n_readers, RB, Kb, KC, rows, top_k, E;
  int32_t img_div;      // routed: image row of pair p is p / img_div (top_k: token rows; 1: per slot)
  int32_t tiles_total;  // tiles per expert summed over readers
  // ordinary readers: work is split over the workgroups in half tiles (8 weight rows), so that
  // every workgroup streams the same number of bytes; half_start is the prefix over readers of
  // ceil(N / 8)
  int32_t half_start[QIMG_MAX_READERS + 1];
  int32_t halves_total;
  int32_t half_q, half_r;  // halves_total = half_q * workgroups + half_r (half_r < workgroups)
  int32_t tp;           // image columns per LDS pass (8, 4, 2 or 1)
  int32_t tp_log2;      // log2(tp)
  int32_t lds_zero, lds_red;  // byte offsets (codes at 0)
  int32_t lds_raw;      // ordinary: raw image scale words (d_a | s_a << 16)
  int32_t raw_wave;     // ordinary, 8 columns per pass: raw word bytes per wave
  // routed readers
  int32_t lds_plan;     // byte offset of the plan arrays
  int32_t slots;        // staged (expert, pass) segments per batch
  int32_t slot_bytes;   // LDS code bytes per staged segment
  int32_t lds_da, lds_ms;  // byte offsets of the staged f32 d_a and -8 s_a, [slots][4 KC][8]
  int32_t lds_xo;          // byte offset of the half-unit carry slots, [8 waves][64] float2
  int32_t halves, khalf;   // units cut in two K halves at chunk khalf (halves 2), or whole
  int32_t pairs_cap;    // bucket * top_k
  FastDiv fd_grid, fd_tiles;  // division by the workgroup count and by tiles_total
};

// Staging of image columns [c0, c0 + nc) in LDS for the ordinary readers, all 4 KC blocks, by
// direct global-to-LDS copies (no registers): codes into [4 KC][tp][32] at LDS 0 as 1 KB wave
// instructions (16 bytes per lane), raw scale words (d_a | s_a << 16, used as they are) at
// lds_raw as 256-byte instructions: [4 KC][tp], or with 8 columns per pass per wave (below).
// Wave w issues code instructions w, w + 8, ... Items past the end of a region copy an
// in-bounds image address into the region's padding; blocks past K/32 copy the row's last
// block (the weight tiles hold d_w = 0 there, which is what makes them contribute nothing).
typedef __attribute__((address_space(3))) void* lds_void_ptr;

// One direct global-to-LDS copy per lane, to LDS byte address lds + lane * bytes (lds must be
// the same in all lanes). Issued as inline assembly so that the compiler's wait-count pass does
// not track it (it would otherwise wait for every outstanding load before each later LDS read
// inside the streaming loop); callers issue these before any other vector memory load and
// wait for them with an explicit vmcnt, which is exact because that counter retires in order.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(lds_void_ptr)p);
}
__device__ __forceinline__ void dma_b128(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void* g, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
               :: "v"(g), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ int stage_code_insts(const ReadArgs& p) { return (4 * p.KC * p.tp * 2 + 63) / 64; }
// Staging by the waves for themselves: with 8 image columns per pass a code copy instruction
// is exactly one chunk (4 blocks x 8 columns x 32 bytes), and wave w streams chunks w, w + 8,
// ...; when the scale words are copied the same way (below), every wave stages exactly what
// it reads and needs no barrier before streaming.
__device__ __forceinline__ bool stage_own(const ReadArgs& p) { return p.tp == 8; }
__device__ __forceinline__ int stage_word_insts(const ReadArgs& p) { return (4 * p.KC * p.tp + 63) / 64; }

__device__ __forceinline__ void stage_dma_issue(const ReadArgs& p, unsigned char* smem, int c0, int nc,
                                                int w, int lane) {
  const int TP = p.tp;
  const int nci = stage_code_insts(p), nwi = stage_word_insts(p);
  const int L = p.tp_log2;
  for (int k = w; k < nci; k += kOrdWaves) {
    const int i = 64 * k + lane;
    const int half = i & 1, c = (i >> 1) & (TP - 1), b = i >> (1 + L);
    const int row = c0 + (c < nc ? c : 0);
    const int bs = b < p.Kb ? b : p.Kb - 1;
    dma_b128(p.codes + ((int64_t)row * p.RB + bs) * 32 + 16 * half, lds_addr(smem + 1024 * k));
  }
  if (stage_own(p)) {
    // the scale words of the wave's own chunks of steps 2 j (lanes 0..31) and 2 j + 1 (lanes
    // 32..63), 32 words per chunk ([block of the chunk][column]), so that the words of the
    // wave's step st sit at lds_raw + w raw_wave + 128 st (a chunk past the end copies the
    // first one's words again; they are not used)
    for (int j = 0; w + 2 * kOrdWaves * j < p.KC; ++j) {
      const int ca = w + 2 * kOrdWaves * j, cb = ca + kOrdWaves;
      const int ch = lane < 32 || cb >= p.KC ? ca : cb;
      const int i = lane & 31, c = i & 7, b = 4 * ch + (i >> 3);
      const int row = c0 + (c < nc ? c : 0);
      const int bs = b < p.Kb ? b : p.Kb - 1;
      dma_b32(p.ds + (int64_t)row * p.RB + bs, lds_addr(smem + p.lds_raw + w * p.raw_wave + 256 * j));
    }
    return;
  }
  for (int k = w; k < nwi; k += kOrdWaves) {
    const int i = 64 * k + lane;
    const int c = i & (TP - 1), b = i >> L;
    const int row = c0 + (c < nc ? c : 0);
    const int bs = b < p.Kb ? b : p.Kb - 1;
    dma_b32(p.ds + (int64_t)row * p.RB + bs, lds_addr(smem + p.lds_raw + 256 * k));
  }
}

// The 32-byte zero slot that the A operands of lanes outside their k-group (or past the
// columns) read. Every wave writes it before its own first read (the same zeros in all waves).
__device__ __forceinline__ void stage_zero(const ReadArgs& p, unsigned char* smem, int lane) {
  if (lane < 8) reinterpret_cast<uint32_t*>(smem + p.lds_zero)[lane] = 0u;
}

// s_waitcnt on the vector memory counter alone (expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup i runs on XCD i % 8, each
// with its own L2). xcd_rank renumbers them so that each XCD's workgroups take a contiguous run
// of the work (ranks [start of XCD, next XCD)): work split by rank is then balanced across the
// XCDs and neighbouring tiles share an L2. A bijection of [0, G).
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_rank(int i, int G) {
  const int x = i % kXcds, q = G / kXcds, r = G % kXcds;
  return x * q + (x < r ? x : r) + i / kXcds;
}

// Weight loads in flight per wave: a ring of D slots of one chunk of NTM tiles each (D - 1 in
// flight while one is computed); deeper rings measured slower for NTM >= 2.
constexpr int ring_depth(int ntm) { return ntm == 1 ? 4 : 2; }

// MODE: 0 Q4_0 readers, 2 Q4_0 block-dot export, 3 Q8_0 readers, 4 Q4_1 readers. NTG: token
// groups of 4 image columns per pass (1 when a pass has at most 4 columns).
template <int NTM, int MODE, int NTG>
__global__ __launch_bounds__(kOrdWaves * 64) void mmvq_tiled_kernel(ReadArgs p) {
  constexpr bool DOTS = MODE == 2;
  constexpr int FMT = MODE == 3 ? 1 : MODE == 4 ? 2 : 0;    // weight format: Q4_0, Q8_0, Q4_1
  constexpr uint32_t kCodeBytes = FMT == 1 ? 2048u : 1024u;  // codes per chunk
  constexpr uint32_t kScaleBytes = FMT == 2 ? 256u : 128u;   // scales (Q4_1: d | m) per chunk
  // vector memory instructions per chunk and tile that are certain to be issued, which the
  // staging wait counts (it may undercount, never overcount): the block-dot export does not
  // use the weight scales, and the compiler drops their loads
  constexpr int kLoads = (FMT == 1 ? 2 : 1) + (DOTS ? 0 : 1);
  extern __shared__ __align__(16) unsigned char smem[];
  // weight loads in flight per wave: a ring of D slots, each one chunk of NTM tiles
  constexpr int D = ring_depth(NTM);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave index (uniform)
  const int n = lane & 15, g = lane >> 4;
  const int KC = p.KC, TP = p.tp;
  const int live = DOTS ? p.rows : clamp_live(p.live_rows, p.rows, nullptr);
  const int wgi = xcd_rank(blockIdx.x, gridDim.x);
  // this workgroup's half tiles [h0, h1) = [floor(H i / G), floor(H (i + 1) / G)) in 32-bit
  // arithmetic (H = q G + r, r i < G^2); a slot is one tile, whole or one of its halves
  // (the divisions go through the vector ALU: the results are made wave-uniform again)
  const uint32_t G = gridDim.x;
  const int h0 = __builtin_amdgcn_readfirstlane(p.half_q * wgi + (int)((uint32_t)p.half_r * (uint32_t)wgi / G));
  const int h1 = __builtin_amdgcn_readfirstlane(p.half_q * (wgi + 1) +
                                                (int)((uint32_t)p.half_r * (uint32_t)(wgi + 1) / G));
  float* red = reinterpret_cast<float*>(smem + p.lds_red);

  const int ncols = live;
  if (ncols == 0 || h0 >= h1) return;

  for (int c0 = 0; c0 < ncols; c0 += TP) {
    const int nc = ncols - c0 < TP ? ncols - c0 : TP;
    // A operand of this lane (row m = n of the MFMA's A, k-group g) for token group tg: the
    // 32 staged bytes of image column 4 tg + (m & 3), block 4 cs + g, at
    // a_base + cs * a_step (low half, high half 16 bytes on), or the 32-byte zero slot
    // (a_step = 0) when the row is outside the lane's k-group or past the columns.
    const int m = n;
    // The scale products go through f16 matrix-core products, exact in f32 (an f16 product
    // has 22 significant bits): per token group the d_a d_w outer product of the chunk's
    // blocks (A: d_a of image column 4 tg + (m & 3), block 4 cs + g, in k slot 4 g of row m
    // when the row is in the lane's k-group, as for the codes; B: d_w of the lane's row and
    // block in k slot 4 g), which lands in the lanes exactly as the block dots do; and per
    // chunk the sums over its 4 blocks of s_a d_w (A: s_a of column 2 (m >> 2) + (m & 3) for
    // m & 3 < 2, block 4 cs + g, in k slot 4 g: the sums land where the epilogue's lane
    // reduction leaves each column)
    // slot 4 g), accumulated over K. Their raw words (d_a | s_a << 16) are read in place, at
    // base + idx * step with idx = the wave's step (8 columns per pass) or the chunk.
    const bool own = stage_own(p);
    const int wrd_base = own ? p.lds_raw + w * p.raw_wave + 4 * 8 * g : p.lds_raw + 4 * TP * g;
    const int wrd_step = own ? 128 : 16 * TP;
    int a_base[2], a_step[2], da_base[2], da_step[2];
#pragma unroll
    for (int tg = 0; tg < 2; ++tg) {
      const int col = 4 * tg + (m & 3);
      const bool on = (m >> 2) == g && col < nc;
      a_base[tg] = on ? (g * TP + col) * 32 : p.lds_zero;
      a_step[tg] = on ? 4 * TP * 32 : 0;
      da_base[tg] = on ? wrd_base + 4 * col : p.lds_zero;
      da_step[tg] = on ? wrd_step : 0;
    }
    const int s_col = 2 * (m >> 2) + (m & 3);
    const bool s_on = (m & 3) < 2 && s_col < nc;
    const int sa_base = s_on ? wrd_base + 4 * s_col + 2 : p.lds_zero;
    const int sa_step = s_on ? wrd_step : 0;
    for (int hb = h0; hb < h1;) {
      // the next NTM slots: slot t is tile lt[t] of reader rr[t], rows [lo[t], hi[t]) of it
      int rr[NTM], lts[NTM], lo[NTM], hi[NTM];
      int nt = 0, hn = hb;
#pragma unroll
      for (int t = 0; t < NTM; ++t) {
        if (hn < h1) {
          int ri = 0;
          while (ri + 1 < p.n_readers && hn >= p.half_start[ri + 1]) ++ri;
          const int lh = hn - p.half_start[ri];
          const bool both = (lh & 1) == 0 && hn + 1 < h1 && hn + 1 < p.half_start[ri + 1];
          rr[t] = ri;
          lts[t] = lh >> 1;
          lo[t] = 8 * (lh & 1);
          hi[t] = both ? 16 : lo[t] + 8;
          hn += both ? 2 : 1;
          ++nt;
        } else {  // idle slots (t > 0 here) re-read the last slot
          const int u = t > 0 ? t - 1 : 0;
          rr[t] = rr[u];
          lts[t] = lts[u];
          lo[t] = lo[u];
          hi[t] = hi[u];
        }
      }
      // per slot: buffer resources over its reader's code and scale planes, the byte offsets
      // of its first chunk (the same in every lane), and the lane's offset in a chunk: 16 bytes
      // per lane (row n, block g) as laid out; in a half slot the lanes of the other half read
      // the lines of this half again (no traffic of their own; their rows are not stored)
      __amdgpu_buffer_rsrc_t rq[NTM], rd[NTM];
      uint32_t oq[NTM], od[NTM], lq[NTM];
      int rl[NTM];
#pragma unroll
      for (int t = 0; t < NTM; ++t) {
        const int ri = rr[t], lt = lts[t];
        rl[t] = lt * 16 + n;  // this lane's weight row in reader ri
        lq[t] = 16u * (uint32_t)(16 * g + (hi[t] - lo[t] == 16 ? n : (lo[t] | (n & 7))));
        const uint32_t chunk0 = (uint32_t)lt * (uint32_t)KC;
        const uint32_t chunks = (uint32_t)p.r[ri].tiles * (uint32_t)KC;
        rq[t] = __builtin_amdgcn_make_buffer_rsrc((void*)p.r[ri].qs, (short)0, (int)(chunks * kCodeBytes),
                                                  kBufferFlags);
        rd[t] = __builtin_amdgcn_make_buffer_rsrc((void*)p.r[ri].d, (short)0, (int)(chunks * kScaleBytes),
                                                  kBufferFlags);
        oq[t] = chunk0 * kCodeBytes;
        od[t] = chunk0 * kScaleBytes;
      }
      float acc[NTM][8];
      v4f sacc[NTM];  // sum over blocks of s_a d_w (Q4_1: of s_a m_w): lane (n, g) column 4 g + v
#pragma unroll
      for (int t = 0; t < NTM; ++t) {
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[t][v] = 0.0f;
        sacc[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
      }

      uint4 q[D][NTM], q2[FMT == 1 ? D : 1][NTM];  // q2: Q8_0's second 16 bytes per block
      // the weight scales as loaded (16 bits; Q4_1 d | m << 16): kept at the loaded width, so
      // that nothing is computed from a slot between its load and its use (a widening at the
      // loop latch made the compiler wait there for every load in flight)
      using ScaleT = typename std::conditional<FMT == 2, uint32_t, uint16_t>::type;
      ScaleT dsc[D][NTM];
      // chunks of this wave: w, w + 8, w + 16, ... (the workgroup's waves read 8 consecutive
      // chunks of a tile at each step)
      const int nst = (KC - w + kOrdWaves - 1) / kOrdWaves;
      auto chunk_of = [&](int st) { return w + kOrdWaves * st; };
      // Every slot is loaded unconditionally (a conditional load would keep the slot's stale
      // value alive and defeat the exact wait counts); a slot past the wave's last chunk
      // repeats that chunk (its lines are in flight or cached), never used. The chunk part of
      // the address is the same in every lane.
      auto load = [&](int j, int st) {
        const uint32_t cs = (uint32_t)chunk_of(st < nst ? st : nst - 1);
#pragma unroll
        for (int t = 0; t < NTM; ++t) {
          const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rq[t], lq[t], oq[t] + cs * kCodeBytes, kNt);
          q[j][t] = make_uint4(x.x, x.y, x.z, x.w);
          if constexpr (FMT == 1) {
            const v4u x2 = __builtin_amdgcn_raw_buffer_load_b128(rq[t], lq[t], oq[t] + cs * kCodeBytes + 1024u, kNt);
            q2[j][t] = make_uint4(x2.x, x2.y, x2.z, x2.w);
          }
          if constexpr (FMT == 2)
            dsc[j][t] = __builtin_amdgcn_raw_buffer_load_b32(rd[t], lq[t] >> 2, od[t] + cs * kScaleBytes, kNt);
          else
            dsc[j][t] = __builtin_amdgcn_raw_buffer_load_b16(rd[t], lq[t] >> 3, od[t] + cs * kScaleBytes, kNt);
        }
      };
      // One chunk of NTM tiles: all matrix-core products first (for every tile slot; an idle
      // slot repeats the last tile and its sums are never stored), then the scaling, so no
      // VALU instruction waits on a product issued just before it.
      auto compute = [&](int j, int cs, int st) {
        v4i blo[NTM], bhi[NTM];
        v4h bw[NTM], bm[NTM];  // (d_w, 0, 0, 0) and (m_w, 0, 0, 0) at k slot 4 g
#pragma unroll
        for (int t = 0; t < NTM; ++t) {
          if constexpr (FMT == 1) {  // Q8_0: elements 0..15 and 16..31 are the two 16-byte halves
            blo[t][0] = (int)q[j][t].x; blo[t][1] = (int)q[j][t].y;
            blo[t][2] = (int)q[j][t].z; blo[t][3] = (int)q[j][t].w;
            bhi[t][0] = (int)q2[j][t].x; bhi[t][1] = (int)q2[j][t].y;
            bhi[t][2] = (int)q2[j][t].z; bhi[t][3] = (int)q2[j][t].w;
          } else {
            blo[t][0] = (int)(q[j][t].x & 0x0f0f0f0fu);
            blo[t][1] = (int)(q[j][t].y & 0x0f0f0f0fu);
            blo[t][2] = (int)(q[j][t].z & 0x0f0f0f0fu);
            blo[t][3] = (int)(q[j][t].w & 0x0f0f0f0fu);
            bhi[t][0] = (int)((q[j][t].x >> 4) & 0x0f0f0f0fu);
            bhi[t][1] = (int)((q[j][t].y >> 4) & 0x0f0f0f0fu);
            bhi[t][2] = (int)((q[j][t].z >> 4) & 0x0f0f0f0fu);
            bhi[t][3] = (int)((q[j][t].w >> 4) & 0x0f0f0f0fu);
          }
          bw[t] = as_v4h((uint64_t)((uint32_t)dsc[j][t] & 0xffffu));
          bm[t] = as_v4h((uint64_t)((uint32_t)dsc[j][t] >> 16));
        }
        const int blk = 4 * cs + g;  // this lane's block
        const int idx = own ? st : cs;
        v4i dd[NTG][NTM];
        v4f dwda[NTG][NTM];
#pragma unroll
        for (int tg = 0; tg < NTG; ++tg) {
          const unsigned char* ap = smem + a_base[tg] + cs * a_step[tg];
          const v4i alo = *reinterpret_cast<const v4i*>(ap);
          const v4i ahi = *reinterpret_cast<const v4i*>(ap + 16);
          const v4h ada = as_v4h((uint64_t)*reinterpret_cast<const uint16_t*>(smem + da_base[tg] + idx * da_step[tg]));
#pragma unroll
          for (int t = 0; t < NTM; ++t) {
            const v4i zero = {0, 0, 0, 0};
            dd[tg][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo, blo[t], zero, 0, 0, 0);
            dd[tg][t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi, bhi[t], dd[tg][t], 0, 0, 0);
            if constexpr (!DOTS)
              dwda[tg][t] = __builtin_amdgcn_mfma_f32_16x16x16f16(ada, bw[t], v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
          }
        }
        if constexpr (!DOTS && FMT != 1) {
          const v4h asa = as_v4h((uint64_t)*reinterpret_cast<const uint16_t*>(smem + sa_base + idx * sa_step));
#pragma unroll
          for (int t = 0; t < NTM; ++t)
            sacc[t] = __builtin_amdgcn_mfma_f32_16x16x16f16(asa, FMT == 2 ? bm[t] : bw[t], sacc[t], 0, 0, 0);
        }
#pragma unroll
        for (int tg = 0; tg < NTG; ++tg) {
#pragma unroll
          for (int t = 0; t < NTM; ++t) {
            const v4i d = dd[tg][t];
            if constexpr (DOTS) {
              if (t < nt && n >= lo[t] && n < hi[t] && rl[t] < p.r[0].N && blk < p.Kb) {
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                  const int col = c0 + 4 * tg + v;
                  if (4 * tg + v < nc)
                    p.sumi[((int64_t)col * p.r[0].N + rl[t]) * p.Kb + blk] = d[v];
                }
              }
            } else {  // (d_w d_a) sumi
#pragma unroll
              for (int v = 0; v < 4; ++v)
                acc[t][4 * tg + v] = __builtin_fmaf(dwda[tg][t][v], (float)d[v], acc[t][4 * tg + v]);
            }
          }
        }
      };
      // Stage the image columns (first tile group of a column pass): the copies go out before
      // the wave's first weight loads, and the wait below covers the copies alone.
      // (the copies and the first loads go out at wave priority 2, so that a wave issuing them is
      // not held behind the other waves' work: same-box A/B 10.53 against 10.67 us on the GLU
      // workload, within 0.5% elsewhere)
      const bool stage = hb == h0;
      if (stage) {
        if (c0 > 0) __syncthreads();  // every wave is done with the previous pass's columns
        __builtin_amdgcn_s_setprio(2);
        stage_dma_issue(p, smem, c0, nc, w, lane);
      }
      if (nst > 0) {
#pragma unroll
        for (int j = 0; j < D - 1; ++j) load(j, j);
        __builtin_amdgcn_s_setprio(0);
        if (stage) wait_vmcnt<(D - 1) * NTM * kLoads>();
      } else if (stage) {
        __builtin_amdgcn_s_setprio(0);
        wait_vmcnt<0>();
      }
      if (stage) {
        stage_zero(p, smem, lane);
        if (!own) __syncthreads();
      }
      for (int base = 0; base < nst; base += D) {
#pragma unroll
        for (int j = 0; j < D; ++j) {
          load((j + D - 1) % D, base + j + D - 1);
          if (base + j < nst) compute(j, chunk_of(base + j), base + j);
          __builtin_amdgcn_sched_barrier(0);  // keep each step's LDS operands local to it
        }
      }
      if constexpr (!DOTS) {
        // The four k-group lanes of a row, reduced and scattered: a swap of the lanes 32 apart
        // carries columns c and c + 4 at once (lanes g < 2 keep column c, g >= 2 column c + 4,
        // summed over g and g + 2), then a swap of the lanes 16 apart carries two of those
        // (lane g ends with columns 2 g and 2 g + 1, summed over all four); then the s_a term
        // of those columns: -8 sum d_w s_a (Q4_0) or + sum m_w s_a (Q4_1).
        float part[NTM][2];
#pragma unroll
        for (int t = 0; t < NTM; ++t) {
          float h[4];
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[t][c]),
                                                              __float_as_uint(acc[t][c + 4]), false, false);
            h[c] = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
          }
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(h[c]),
                                                              __float_as_uint(h[c + 2]), false, false);
            part[t][c] = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
            if constexpr (FMT != 1) part[t][c] = __builtin_fmaf(FMT == 2 ? 1.0f : -8.0f, sacc[t][c], part[t][c]);
          }
        }
        // lane (n, g) stores columns 2g, 2g+1 of its row for each slot
#pragma unroll
        for (int t = 0; t < NTM; ++t)
          if (t < nt)
            *reinterpret_cast<float2*>(red + ((w * NTM + t) * 16 + n) * 8 + 2 * g) = make_float2(part[t][0], part[t][1]);
        __syncthreads();
        for (int o = threadIdx.x; o < nt * 128; o += blockDim.x) {
          const int t = o >> 7, nn = (o >> 3) & 15, col = o & 7;
          int ri = rr[0], lt = lts[0], rlo = lo[0], rhi = hi[0];
#pragma unroll
          for (int u = 1; u < NTM; ++u)
            if (t == u) ri = rr[u], lt = lts[u], rlo = lo[u], rhi = hi[u];
          if (col < nc && nn >= rlo && nn < rhi) {
            const int row = lt * 16 + nn;
            if (row < p.r[ri].N) {
              float s = red[(t * 16 + nn) * 8 + col];
              for (int ww = 1; ww < kOrdWaves; ++ww) s = s + red[((ww * NTM + t) * 16 + nn) * 8 + col];
              p.r[ri].out[(int64_t)(c0 + col) * p.r[ri].ld + row] = s;
            }
          }
        }
        // the cross-wave sums are reused by the next slot group or column pass, if any
        if (hn < h1 || c0 + TP < ncols) __syncthreads();
      }
      hb = hn;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Prefill readers (many image rows: a prompt's tokens): Q4_0 x Q8_1 on v_mfma_i32_32x32x32_i8,
// one 32-value block per product, so every block's int32 dot gets its own scales
// ("r49 - A-quantize prepass shared-A dedup", section 2 Principle: the activation is
// quantized once and every projection that reads it shares that one image).
//
// A workgroup computes 64 weight rows (4 tiles of 16) x 64 image rows with 4 waves, each 32
// weight rows x 32 image rows. Product orientation: A = weights (32 rows), B = image codes (32
// image rows). Per 4-block chunk the image rows' codes and scale words and the weight tiles'
// codes and scales are copied into LDS by direct global-to-LDS copies (double buffered: the next
// chunk's copies are in flight during the products), so nothing is staged through registers;
// then per block one product and the scaling acc += d_w (d_a sumi - 8 s_a). Image rows past
// the live count, rows past N and blocks past K/32 contribute nothing and are not stored. Every
// LDS operand read is 16 bytes per lane and falls on distinct banks (an image row's 16-byte
// pieces are stored in an order permuted by the row), and the reader tiles made for the mat-vec
// readers serve as they are.
// ---------------------------------------------------------------------------------------------
constexpr int kMmqWaves = 4;
constexpr int kMmqMinRows = 64;  // Q4_0 readers of this many image rows or more use this kernel
typedef long v1l;
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// The scales go through f16 products (exact in f32): per block the outer product
// d_w[row] d_a[image row] (one non-zero k slot on the weight side), and per chunk the sums over
// its 4 blocks of d_w s_a, accumulated over K by the matrix core. Each (image row, weight row,
// block) then costs a convert and one fma:
//   acc += (d_w d_a) sumi;     out = acc - 8 sum_b d_w s_a.
__global__ __launch_bounds__(kMmqWaves * 64, 2) void mmq_kernel(ReadArgs p) {
  // A chunk's operands are copied into LDS by direct global-to-LDS copies, double buffered (the
  // next chunk's copies are in flight while a chunk is computed). Image codes, [buf][row][8
  // pieces of 16 bytes]: piece P of local row r sits at position P ^ (r & 7), so that the product
  // operand reads (16 bytes per lane, 8 lanes per bank cycle: 8 consecutive rows, one piece
  // each) fall on distinct banks.
  __shared__ __align__(16) uint8_t s_img[2][64 * 128];
  // image scale words d_a | s_a << 16, [buf][row][block]
  __shared__ __align__(16) uint32_t s_isc[2][64][4];
  // the workgroup's 4 weight tiles of a chunk: codes in their tiled order ([lane (row, block)]
  // [16 bytes]) and scales d_w [block][row]
  __shared__ __align__(16) uint32_t s_wt[kMmqWaves][2][256];
  __shared__ __align__(16) uint16_t s_wsc[kMmqWaves][2][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int live = clamp_live(p.live_rows, p.rows, nullptr);
  const int c0 = blockIdx.y * 64;
  if (c0 >= live) return;  // whole workgroup
  const int KC = p.KC;
  // weight tile t of the workgroup is tile 4 blockIdx.x + t (tiles past the end repeat the last
  // one; nothing is stored for them); wave w copies tile w, and computes weight rows
  // 32 (w >> 1) .. + 31 (tiles 2 (w >> 1) and 2 (w >> 1) + 1) x image rows 32 (w & 1) .. + 31
  auto tile_of = [&](int t, int& ri, int& lt) {
    const int tr = blockIdx.x * kMmqWaves + t;
    const int tile = tr < p.tiles_total ? tr : p.tiles_total - 1;
    ri = 0;
    while (ri + 1 < p.n_readers && tile >= p.tile_start[ri + 1]) ++ri;
    lt = tile - p.tile_start[ri];
    return tr < p.tiles_total;
  };
  int cri, clt;
  tile_of(w, cri, clt);
  const uint8_t* wq = p.r[cri].qs + ((int64_t)clt * KC * 64 + lane) * 16;
  const uint8_t* wdp = reinterpret_cast<const uint8_t*>(p.r[cri].d + (int64_t)clt * KC * 64) + 4 * (lane & 31);

  // The copies of one chunk, 5 per wave: local image rows 16 w + 8 i + (lane >> 3), i < 2 (lane
  // position lane & 7 of its row gets piece (lane & 7) ^ (lane >> 3)); the scale words of local
  // image rows 16 w + (lane >> 2), block lane & 3; weight tile w's codes (1 KB) and scales (128
  // bytes, lanes < 32). Image rows past the live count copy the last live row and blocks past
  // K/32 the row's last block (finite scales; the weight tiles hold d_w = 0 there, and the
  // outputs of those image rows are not stored).
  const uint8_t* csrc[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int lr = 16 * w + 8 * i + (lane >> 3);
    const int row = c0 + lr < live ? c0 + lr : live - 1;
    csrc[i] = p.codes + ((size_t)row * p.RB) * 32 + 16 * ((lane & 7) ^ (lr & 7));
  }
  const int srow = c0 + 16 * w + (lane >> 2) < live ? c0 + 16 * w + (lane >> 2) : live - 1;
  const uint32_t* ssrc = p.ds + (size_t)srow * p.RB;
  // LDS byte addresses (wave-uniform) of this wave's copy destinations in buffer 0
  const uint32_t l_img = lds_addr(&s_img[0][(16 * w) * 128]), l_isc = lds_addr(&s_isc[0][16 * w][0]);
  const uint32_t l_wt = lds_addr(&s_wt[w][0][0]), l_wsc = lds_addr(&s_wsc[w][0][0]);
  auto copy_chunk = [&](int s, int q) {
    dma_b128(csrc[0] + (size_t)s * 128, l_img + q * (64 * 128));
    dma_b128(csrc[1] + (size_t)s * 128, l_img + q * (64 * 128) + 1024);
    const int blk = 4 * s + (lane & 3) < p.Kb ? 4 * s + (lane & 3) : p.Kb - 1;
    dma_b32(ssrc + blk, l_isc + q * (64 * 16));
    dma_b128(wq + (int64_t)s * 1024, l_wt + q * 1024);
    if (lane < 32) dma_b32(wdp + (int64_t)s * 128, l_wsc + q * 128);
  };

  // Products on v_mfma_i32_32x32x32_i8, one block each: lane (i, h) = (lane & 31, lane >> 5)
  // holds elements 16 h .. 16 h + 15 of the block, i.e. image piece 2 b + h of image row i and
  // the low (h = 0) or high (h = 1) nibbles of weight row i's 16 block bytes (byte k holds
  // elements k and k + 16). D[8 u + 4 h + v][i] lands in lane (i, h), register 4 u + v.
  const int i32 = lane & 31, h = lane >> 5;
  const int wr = w >> 1, wc = w & 1;
  const int tt = 2 * wr + (i32 >> 4), r16 = i32 & 15;  // this lane's weight tile and row in it
  const int ir = 32 * wc + i32;                          // this lane's local image row
  const uint32_t a_img = ir * 128 + 16 * (h ^ (ir & 7));  // block b: a_img ^ (32 b)
  // Scale products (f16, exact in f32) on v_mfma_f32_32x32x8_f16, k group h holding blocks 2 h and
  // 2 h + 1 as (d_a, s_a, d_a, s_a) on the image side; the weight side is, per block b, d_w in
  // slot 2 (b & 1) of group b >> 1 (the d_w d_a outer product), and per chunk (0, d_w, 0, d_w)
  // in both groups (the chunk's sum of d_w s_a).
  float acc[16];
  v16f sacc;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    acc[k] = 0.0f;
    sacc[k] = 0.0f;
  }

  copy_chunk(0, 0);
  wait_vmcnt<0>();
  __syncthreads();
  for (int s = 0; s < KC; ++s) {
    const int q = s & 1;
    // Wave priorities (s_setprio, within the SIMD's arbitration): the next chunk's copies go out
    // at priority 2, each block's scaling runs at 1, the rest at 0, so that a wave reaching its
    // copies or its vector work is not held behind the other waves' instructions (same-box A/B:
    // 168 against 177 us on the prompt workload)
    if (s + 1 < KC) {
      __builtin_amdgcn_s_setprio(2);
      copy_chunk(s + 1, q ^ 1);
      __builtin_amdgcn_s_setprio(0);
    }
    const uint64_t wsw = (uint64_t)s_wsc[tt][q][32 * h + r16] | ((uint64_t)s_wsc[tt][q][32 * h + 16 + r16] << 32);
    const uint64_t dav = *reinterpret_cast<const uint64_t*>(&s_isc[q][ir][2 * h]);
    sacc = __builtin_amdgcn_mfma_f32_32x32x8f16(as_v4h(wsw << 16), as_v4h(dav), sacc, 0, 0, 0);
    // the LDS operands of block b are read one block ahead (two operand sets, ping-pong); the
    // products and scaling of each block stay in a scheduling region of their own
    struct Ops { uint4 wb; uint4 ib; };
    auto ops = [&](int b, Ops& o) {
      o.wb = *reinterpret_cast<const uint4*>(&s_wt[tt][q][(16 * b + r16) * 4]);
      o.ib = *reinterpret_cast<const uint4*>(&s_img[q][a_img ^ (32u * b)]);
    };
    auto block = [&](const Ops& o, int b) {
      const uint64_t dwb = h == (b >> 1) ? (wsw & (b & 1 ? 0xffffffff00000000ull : 0xffffffffull)) : 0ull;
      const int sh = 4 * h;
      const v4i a = {(int)((o.wb.x >> sh) & 0x0f0f0f0fu), (int)((o.wb.y >> sh) & 0x0f0f0f0fu),
                     (int)((o.wb.z >> sh) & 0x0f0f0f0fu), (int)((o.wb.w >> sh) & 0x0f0f0f0fu)};
      const v4i bb = {(int)o.ib.x, (int)o.ib.y, (int)o.ib.z, (int)o.ib.w};
      v16i zero;
      v16f fzero;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        zero[k] = 0;
        fzero[k] = 0.0f;
      }
      const v16i dd = __builtin_amdgcn_mfma_i32_32x32x32_i8(a, bb, zero, 0, 0, 0);
      const v16f dwda = __builtin_amdgcn_mfma_f32_32x32x8f16(as_v4h(dwb), as_v4h(dav), fzero, 0, 0, 0);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int k = 0; k < 16; ++k) acc[k] = __builtin_fmaf(dwda[k], (float)dd[k], acc[k]);
      __builtin_amdgcn_s_setprio(0);
      // the block's scaling is done here (not sunk below the next blocks' products)
#pragma unroll
      for (int k = 0; k < 16; k += 4)
        asm volatile("" : "+v"(acc[k]), "+v"(acc[k + 1]), "+v"(acc[k + 2]), "+v"(acc[k + 3]));
    };
    Ops oa;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      ops(b, oa);
      block(oa, b);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next chunk's copies have landed (nothing else in the loop uses the counter)
    if (s + 1 < KC) wait_vmcnt<0>();
    __syncthreads();
  }
  // lane (i, h), register 4 u + v: weight row 8 u + 4 h + v of the wave's 32 (tile 2 wr + (u >> 1)),
  // image row 32 wc + i
  const int col = c0 + 32 * wc + i32;
  if (col >= live) return;
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    int ri, lt;
    if (!tile_of(2 * wr + half, ri, lt)) continue;
    const ReaderDesc& r = p.r[ri];
    float* o = r.out + (int64_t)col * r.ld;
#pragma unroll
    for (int u = 2 * half; u < 2 * half + 2; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int row = lt * 16 + 8 * (u & 1) + 4 * h + v;
        if (row < r.N) o[row] = __builtin_fmaf(-8.0f, sacc[4 * u + v], acc[4 * u + v]);
      }
  }
}

// ---------------------------------------------------------------------------------------------
// Routed readers (MUL_MAT_ID).
//
// Plan ([P3] What this changes: only the live rows' pairs are planned; padding ids are never
// used). Every workgroup reads the live pairs' expert ids into LDS and counts them per expert
// (LDS atomics); one scan gives each expert's pair offset and the first of its work units. The
// members of an expert in ascending pair order come from a scan of the ids with wave ballots
// (no sort): a wave walks the ids 64 at a time and places each match at its rank. The plan is
// exported to the workspace: the members of each segment (a pass of up to TP pairs of one
// expert) by the workgroup holding the segment's first unit, as it stages it; the counts,
// offsets and error word by workgroup 0 at the end.
//
// Work. A unit is one 16-row tile (over the concatenated readers) of one active expert for one
// pass of up to TP of its pairs; units are ordered by (expert, pass, tile), and an (expert,
// pass) is a segment of T units, T = tiles per expert. Workgroup i takes units
// [U i / G, U (i + 1) / G) in batches of up to `slots` segments, whose image columns it stages
// in LDS (all K blocks). Each unit is cut along K into two halves at a chunk fixed by K (or kept
// whole when K is too short), and the batch's half-units are split contiguously over the waves.
// A wave streams its half-units one tile at a time, KU chunks per load, two loads in flight; the
// loads of the next half-unit go out before the current one ends, so the stream does not drain.
// After the last chunk of a half the four k-group lanes of each row are summed; the two half
// sums are added (through an LDS carry slot when two waves hold them) and stored. The sum for a
// pair depends only on its image row and expert (each half's chunks in K order, the fixed lane
// tree, then first + second): not on the other pairs, the live count or the schedule.
// ---------------------------------------------------------------------------------------------
constexpr int kRoutedMaxSlots = 4;
constexpr int kRoutedKu = 2;  // chunks per load of a routed wave; two loads in flight

// Inclusive prefix sum over the 64 lanes in lane order, by DPP moves: shifts by 1, 2, 4 and 8
// lanes within each row of 16, then the last lane of row 0 into row 1 and of row 2 into row 3
// (row_bcast:15), then the last lane of row 1 into rows 2 and 3 (row_bcast:31). A lane whose
// source lies outside the move's rows adds 0.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);
  return v;
}

// Pairs of expert e with ranks [lo, hi) in ascending pair order (rank r goes to dst[r - lo]),
// found by one wave's ballots over the live pairs' expert ids sid[] (padded with -1 to a
// multiple of 256 entries, 16-byte aligned): lane l reads pairs 4 l .. 4 l + 3 of each run of
// 256, and a match's rank counts the matches of the lower lanes and of its lower pairs in the
// lane.
__device__ __forceinline__ void ballot_members(const int32_t* sid, int P, int e, int lo, int hi,
                                               int32_t* dst, int lane) {
  int base = 0;
  const uint64_t below = (1ull << lane) - 1ull;
  for (int c0 = 0; c0 < P && base < hi; c0 += 256) {
    const int4 v = *reinterpret_cast<const int4*>(sid + c0 + 4 * lane);
    const bool m0 = v.x == e, m1 = v.y == e, m2 = v.z == e, m3 = v.w == e;
    const uint64_t b0 = __ballot(m0), b1 = __ballot(m1), b2 = __ballot(m2), b3 = __ballot(m3);
    int r = base + __popcll(b0 & below) + __popcll(b1 & below) + __popcll(b2 & below) + __popcll(b3 & below);
    const int pi = c0 + 4 * lane;
    if (m0) { if (r >= lo && r < hi) dst[r - lo] = pi; ++r; }
    if (m1) { if (r >= lo && r < hi) dst[r - lo] = pi + 1; ++r; }
    if (m2) { if (r >= lo && r < hi) dst[r - lo] = pi + 2; ++r; }
    if (m3 && r >= lo && r < hi) dst[r - lo] = pi + 3;
    base += __popcll(b0) + __popcll(b1) + __popcll(b2) + __popcll(b3);
  }
}

// The value of lane l ^ J (J a power of two up to 32): DPP within rows of 16 (xor 4 and 8 as
// two mirrors each), permlane swaps across rows. A swap returns the lane's own value and its
// partner's; the partner's is the one that differs (keys below are distinct across lanes).
constexpr int kDppQuadRev = 0x1b;  // quad_perm [3,2,1,0]
template <int J>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  if constexpr (J == 1) {
    return (uint32_t)dpp_n<kDppXor1>((int)v);
  } else if constexpr (J == 2) {
    return (uint32_t)dpp_n<kDppXor2>((int)v);
  } else if constexpr (J == 4) {
    return (uint32_t)dpp_n<kDppQuadRev>(dpp_n<kDppHalfMirror>((int)v));
  } else if constexpr (J == 8) {
    return (uint32_t)dpp_n<kDppHalfMirror>(dpp_n<kDppMirror>((int)v));
  } else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return r[0] != v ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return r[0] != v ? r[0] : r[1];
  }
}
// One compare-exchange of a bitonic sort network over the 64 lanes (block size K, distance J):
// the lower lane of a pair keeps the smaller key in ascending blocks, the larger in descending.
template <int K, int J>
__device__ __forceinline__ void bitonic_step(uint32_t& key, int lane) {
  const uint32_t o = lane_xor<J>(key);
  const bool keep_min = ((lane & J) == 0) == ((lane & K) == 0);
  key = keep_min ? (key < o ? key : o) : (key > o ? key : o);
}
// Ascending sort of one distinct 32-bit key per lane over the wave.
__device__ __forceinline__ uint32_t wave_sort64(uint32_t key, int lane) {
  bitonic_step<2, 1>(key, lane);
  bitonic_step<4, 2>(key, lane);
  bitonic_step<4, 1>(key, lane);
  bitonic_step<8, 4>(key, lane);
  bitonic_step<8, 2>(key, lane);
  bitonic_step<8, 1>(key, lane);
  bitonic_step<16, 8>(key, lane);
  bitonic_step<16, 4>(key, lane);
  bitonic_step<16, 2>(key, lane);
  bitonic_step<16, 1>(key, lane);
  bitonic_step<32, 16>(key, lane);
  bitonic_step<32, 8>(key, lane);
  bitonic_step<32, 4>(key, lane);
  bitonic_step<32, 2>(key, lane);
  bitonic_step<32, 1>(key, lane);
  bitonic_step<64, 32>(key, lane);
  bitonic_step<64, 16>(key, lane);
  bitonic_step<64, 8>(key, lane);
  bitonic_step<64, 4>(key, lane);
  bitonic_step<64, 2>(key, lane);
  bitonic_step<64, 1>(key, lane);
  return key;
}

template <int KU, bool SMALL>
__global__ __launch_bounds__(kWaves * 64) void mmvq_routed_kernel(ReadArgs p) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ __align__(16) int sh_wave[2][kWaves];  // per-wave totals of the plan scans
  __shared__ int sh_misc[4];                  // bad-id flag, segments, unused, unused
  __shared__ int sh_seg[kRoutedMaxSlots][4];  // start unit, expert, columns, pass
  __shared__ int sh_mem[kRoutedMaxSlots][8];  // pair ids of a segment's columns
  __shared__ int sh_row[kRoutedMaxSlots][8];  // and their image rows
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int n = lane & 15, g = lane >> 4;
  const int E = p.E, T = p.tiles_total, TP = p.tp, KC = p.KC;
  // The ids are read over the whole bucket (its buffer holds bucket x top_k entries) and before
  // the live count, so that their loads do not wait for it; entries of padding rows are masked
  // off below and never used. Buffer loads read 0 past the bucket's pairs; every load goes out,
  // so that the waits for them are exact. SMALL: pair lane of each wave; otherwise pairs
  // tid + 512 j (pairs_cap <= 8 * 512).
  const __amdgpu_buffer_rsrc_t rid =
      __builtin_amdgcn_make_buffer_rsrc((void*)p.ids, (short)0, p.pairs_cap * 4, kBufferFlags);
  int idv[SMALL ? 1 : 8];
#pragma unroll
  for (int j = 0; j < (SMALL ? 1 : 8); ++j)
    idv[j] = (int)__builtin_amdgcn_raw_buffer_load_b32(rid, 4u * (uint32_t)((SMALL ? lane : tid) + 512 * j), 0u, 0);
  int clamped = 0;
  const int live = clamp_live(p.live_rows, p.rows, &clamped);
  const int P = live * p.top_k;     // <= rows * top_k = pairs_cap
  const int Pp = (P + 255) & ~255;  // sid entries the member ballots read (runs of 256)

  const int sid_n = (p.pairs_cap + 255) & ~255;
  int32_t* sid = reinterpret_cast<int32_t*>(smem + p.lds_plan);  // [sid_n]: expert of a live pair or -1
  int32_t* cnt = sid + sid_n;                                      // [E] live pairs per expert
  int32_t* off = cnt + E;                                          // [E + 1] pair offsets
  int32_t* pps = off + E + 1;                                      // [E + 1] first segment

  // ---- plan ----
  // A launch of at most 64 pairs (SMALL: bucket * top_k <= 64) keeps its plan in registers:
  // every wave sorts the keys
  // (expert << 6 | pair) of the live pairs across its lanes (lanes past P and ids out of range
  // sort last), so the sorted order lists each expert's pairs in ascending pair order, and the
  // segments (runs of up to TP pairs of one expert) follow from ballots over it: no LDS plan,
  // atomic or barrier before the staging. Larger launches count per expert in LDS.
  constexpr bool small = SMALL;
  int s_e = 0, s_pair = 0, s_first = 0, s_seg = -1, s_count = 0, s_valid_n = 0;
  bool s_valid = false, s_start = false, s_bad = false;
  if (tid < 8) reinterpret_cast<uint32_t*>(smem + p.lds_zero)[tid] = 0u;  // the 32-byte zero slot
  if constexpr (small) {
    const int id = idv[0];
    const bool ok = lane < P && (uint32_t)id < (uint32_t)E;
    s_bad = __ballot(lane < P && !ok) != 0ull;
    const uint32_t key = wave_sort64(((uint32_t)(ok ? id : 0xfffff) << 6) | (uint32_t)lane, lane);
    s_e = (int)(key >> 6);
    s_pair = (int)(key & 63u);
    s_valid = s_e < E;
    const int prev = __builtin_amdgcn_ds_bpermute(((lane + 63) & 63) << 2, s_e);
    const uint64_t le = ~0ull >> (63 - lane);  // lanes 0 .. lane
    const uint64_t chg = __ballot(s_valid && (lane == 0 || prev != s_e));
    s_first = s_valid ? 63 - __builtin_clzll((chg & le) | 1ull) : lane;  // first lane of the expert
    s_start = s_valid && ((lane - s_first) & (TP - 1)) == 0;
    const uint64_t smask = __ballot(s_start);
    s_count = __popcll(smask);  // segments
    s_seg = __popcll(smask & le) - 1;
    s_valid_n = __popcll(__ballot(s_valid));
    // the plan's members (ascending by expert, then pair): one wave of the grid stores them
    if (blockIdx.x == 0 && w == 0 && s_valid) p.ws[4 + 2 * E + 1 + lane] = s_pair;
  } else {
    for (int e = tid; e < E; e += kWaves * 64) cnt[e] = 0;
    if (tid < 4) sh_misc[tid] = 0;
    __syncthreads();
    {
      const int nj = (Pp + 511) >> 9;
      bool bad = false;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (j < nj) {
          const int pi = tid + 512 * j, id = idv[j];
          const bool ok = pi < P && (uint32_t)id < (uint32_t)E;
          bad |= pi < P && !ok;
          if (pi < Pp) sid[pi] = ok ? id : -1;
          if (ok) atomicAdd(&cnt[id], 1);
        }
      }
      if (bad) sh_misc[0] = 1;
    }
    __syncthreads();
    {  // thread t: experts t and t + 512 (E <= 1024)
      const int ea = tid, eb = tid + kWaves * 64;
      const int ca = ea < E ? cnt[ea] : 0, cb = eb < E ? cnt[eb] : 0;
      // pairs in the low 16 bits, segments (passes of up to TP pairs) in the high 16: each total
      // is at most the pair count (<= 4096), so no carry crosses
      const int va = ca | (((ca + TP - 1) >> p.tp_log2) << 16);
      const int vb = cb | (((cb + TP - 1) >> p.tp_log2) << 16);
      const int ia = wave_incl_scan(va), ib = wave_incl_scan(vb);
      if (lane == 63) {
        sh_wave[0][w] = ia;
        sh_wave[1][w] = ib;
      }
      __syncthreads();
      int xa = 0, xb = 0, ta = 0, tb = 0;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const int a = sh_wave[0][i], b = sh_wave[1][i];
        xa += i < w ? a : 0;
        xb += i < w ? b : 0;
        ta += a;
        tb += b;
      }
      const int pa = xa + ia - va, pb = ta + xb + ib - vb;  // before experts ea and eb
      if (ea < E) {
        off[ea] = pa & 0xffff;
        pps[ea] = (int)((uint32_t)pa >> 16);
      }
      if (eb < E) {
        off[eb] = pb & 0xffff;
        pps[eb] = (int)((uint32_t)pb >> 16);
      }
      if (tid == 0) {
        const uint32_t tot = (uint32_t)(ta + tb);
        off[E] = (int)(tot & 0xffffu);
        pps[E] = (int)(tot >> 16);
        sh_misc[1] = (int)(tot >> 16);
      }
    }
    __syncthreads();
  }

  // ---- work ----
  // values read from LDS that are the same in every lane are made wave-uniform, so that the
  // reader descriptors they select are fetched with scalar loads
  auto uni = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
  // every segment holds T units (its tiles), so segment s covers units [s T, s T + T)
  const int U = (small ? s_count : uni(sh_misc[1])) * T;
  const int G = gridDim.x;
  const int wr = xcd_rank(blockIdx.x, G);
  // [u0, u1) = [floor(U wr / G), floor(U (wr + 1) / G)) in 32-bit arithmetic (U = q G + r,
  // r (wr + 1) <= G^2)
  const int uq = fdiv(U, p.fd_grid), urm = U - uq * G;
  const int u0 = uq * wr + fdiv(urm * wr, p.fd_grid), u1 = uq * (wr + 1) + fdiv(urm * (wr + 1), p.fd_grid);
  const int nb = 4 * KC;               // staged blocks per segment (K padded to chunks)
  const int ncode = nb * TP * 2;       // 16-byte code items per slot: [nb][TP][2]
  const int nds = nb * 8;              // scale items per slot: [nb][column slot of 8]
  float* const daA = reinterpret_cast<float*>(smem + p.lds_da);  // [slots][nds]
  float* const msA = reinterpret_cast<float*>(smem + p.lds_ms);  // [slots][nds]
  for (int ub = u0; ub < u1;) {
    // this batch: segments [s_lo, s_lo + ns), units [ub, ue)
    const int s_lo = fdiv(ub, p.fd_tiles), s_last = fdiv(u1 - 1, p.fd_tiles);
    const int ns = s_last - s_lo + 1 < p.slots ? s_last - s_lo + 1 : p.slots;
    const int ue = (s_lo + ns) * T < u1 ? (s_lo + ns) * T : u1;
    if constexpr (small) {
      // the batch's segments and their members from the sorted keys: every wave writes the
      // same values and reads back only what it wrote itself, so no barrier is needed
#pragma unroll
      for (int k = 0; k < kRoutedMaxSlots; ++k) {
        if (k < ns) {
          const uint64_t m = __ballot(s_start && s_seg == s_lo + k);
          const int sk = (int)__builtin_ctzll(m | (1ull << 63));  // the segment's first lane
          const int e = __builtin_amdgcn_readlane(s_e, sk);
          const int pass = (sk - __builtin_amdgcn_readlane(s_first, sk)) >> p.tp_log2;
          const int left = __popcll(__ballot(s_valid && s_e == e)) - pass * TP;
          if (lane == 0) {
            sh_seg[k][0] = (s_lo + k) * T;
            sh_seg[k][1] = e;
            sh_seg[k][2] = left < TP ? left : TP;
            sh_seg[k][3] = pass;
          }
        } else if (lane == 0) {
          sh_seg[k][0] = 0x7fffffff;
        }
      }
      const int kk = s_seg - s_lo;
      if (s_valid && kk >= 0 && kk < ns) {
        const int c = (lane - s_first) & (TP - 1);
        sh_mem[kk][c] = s_pair;
        sh_row[kk][c] = s_pair / p.img_div;
      }
    } else {
      {  // the batch's segments, found by the threads of their experts
        auto find = [&](int e) {
          const int a0 = pps[e], a1 = pps[e + 1];
          const int sa = a0 > s_lo ? a0 : s_lo, sb = a1 < s_lo + ns ? a1 : s_lo + ns;
          for (int sg = sa; sg < sb; ++sg) {
            const int k = sg - s_lo, pass = sg - a0;
            const int left = cnt[e] - pass * TP;
            sh_seg[k][0] = sg * T;
            sh_seg[k][1] = e;
            sh_seg[k][2] = left < TP ? left : TP;
            sh_seg[k][3] = pass;
          }
        };
        if (tid < E) find(tid);
        if (tid + kWaves * 64 < E) find(tid + kWaves * 64);
        if (tid < kRoutedMaxSlots && tid >= ns) sh_seg[tid][0] = 0x7fffffff;
      }
      __syncthreads();
      // members of the batch's segments (wave k: segment k) and their image rows
      if (w < ns) {
        const int e = uni(sh_seg[w][1]), nc = uni(sh_seg[w][2]), lo = uni(sh_seg[w][3]) * TP;
        ballot_members(sid, P, e, lo, lo + nc, sh_mem[w], lane);
        if (lane < nc) sh_row[w][lane] = sh_mem[w][lane] / p.img_div;
      }
      __syncthreads();
    }
    const int seg0 = s_lo * T;
    auto seg_of = [&](int u) {  // segment index in the batch of unit u (u in [ub, ue))
      return (u >= seg0 + T ? 1 : 0) + (u >= seg0 + 2 * T ? 1 : 0) + (u >= seg0 + 3 * T ? 1 : 0);
    };

    // ---- this wave's work of the batch: the first loads go out with the staging ----
    // With p.halves == 2 every unit is cut at chunk H = p.khalf (a multiple of KU fixed by K)
    // into two half-units, 2 u and 2 u + 1, each summed on its own (chunks in order, then the
    // lane tree); a pair's output is the first half's sum plus the second's. The wave takes
    // half-units [ha, hb) of the batch, so that the work of the workgroup splits over its waves
    // in steps of half a unit. With p.halves == 1 (K too short to cut), H = KC.
    const int halves = p.halves, H = p.khalf;
    const int h_lo = halves * ub, hm = halves * (ue - ub);
    auto hstart = [&](int v) { return h_lo + (int)(((int64_t)hm * v) >> 3); };
    static_assert(kWaves == 8, "work split by shifts");
    const int ha = hstart(w), hb = hstart(w + 1);
    struct Cursor {
      int hu, u, k, kb, ke;  // half-unit, unit, slot, next chunk, end chunk
    };
    auto start = [&](int hu, Cursor& c) {
      c.hu = hu;
      c.u = halves == 2 ? hu >> 1 : hu;
      const bool second = halves == 2 && (hu & 1);
      c.k = seg_of(c.u);
      c.kb = second ? H : 0;
      c.ke = second ? KC : H;
    };
    auto reader_of = [&](int tt) {  // reader of tile tt of an expert
      int ri = 0;
      while (ri + 1 < p.n_readers && tt >= p.tile_start[ri + 1]) ++ri;
      return ri;
    };
    // load cursor: buffer resources over the unit's reader planes and the lane's offsets in its
    // first chunk. A wave past its last unit (or without units) loads through empty resources:
    // the loads read zeros and touch no memory; their values are never used.
    __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.r[0].qs, (short)0, 0, kBufferFlags);
    __amdgpu_buffer_rsrc_t rd = __builtin_amdgcn_make_buffer_rsrc((void*)p.r[0].d, (short)0, 0, kBufferFlags);
    uint32_t vq = 0, vd = 0;
    int crow = 0, cri = 0;  // compute cursor: output row of this lane, reader
    auto bind_load = [&](const Cursor& c) {
      const int e = uni(sh_seg[c.k][1]);
      const int tt = c.u - uni(sh_seg[c.k][0]);  // tile in the segment
      const int ri = reader_of(tt);
      const uint32_t chunks = (uint32_t)E * (uint32_t)p.r[ri].tiles * (uint32_t)KC;
      const uint32_t chunk0 = ((uint32_t)e * (uint32_t)p.r[ri].tiles + (uint32_t)(tt - p.tile_start[ri])) * (uint32_t)KC;
      rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.r[ri].qs, (short)0, (int)(chunks * 1024u), kBufferFlags);
      rd = __builtin_amdgcn_make_buffer_rsrc((void*)p.r[ri].d, (short)0, (int)(chunks * 128u), kBufferFlags);
      vq = chunk0 * 1024u + 16u * (uint32_t)lane;
      vd = chunk0 * 128u + 4u * (uint32_t)(lane >> 1);
    };
    auto bind_compute = [&](const Cursor& c) {
      const int tt = c.u - uni(sh_seg[c.k][0]);
      cri = reader_of(tt);
      crow = (tt - p.tile_start[cri]) * 16 + n;
    };
    Cursor lc{0, 0, 0, 0, 0}, cc{0, 0, 0, 0, 0};
    bool ldone = ha >= hb;
    if (!ldone) {
      start(ha, lc);
      bind_load(lc);
    }
    auto advance_load = [&]() {
      if (ldone) return;
      lc.kb += KU;
      if (lc.kb >= lc.ke) {
        if (lc.hu + 1 < hb) {
          const int pu = lc.u;
          start(lc.hu + 1, lc);
          if (lc.u != pu) bind_load(lc);  // the second half of a unit keeps its planes
        } else {
          ldone = true;
          rq = __builtin_amdgcn_make_buffer_rsrc((void*)p.r[0].qs, (short)0, 0, kBufferFlags);
          rd = __builtin_amdgcn_make_buffer_rsrc((void*)p.r[0].d, (short)0, 0, kBufferFlags);
        }
      }
    };
    // one load: KU chunks of codes and their scales, the scales as the 32-bit word that holds
    // the lane's fp16 d_w and its neighbour's (lane pairs read the same word), so that every
    // loop-carried value is a whole register: 16-bit values would be packed in pairs where the
    // loop paths merge, and that packing waits for nearly every load in flight. Chunks past the
    // half-unit's last repeat it (in flight or cached; not used).
    uint4 qa[KU], qb[KU];
    uint32_t da_[KU], db_[KU];
    auto load = [&](uint4 (&q)[KU], uint32_t (&d)[KU]) {
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const uint32_t cs = (uint32_t)(lc.kb + u < lc.ke ? lc.kb + u : lc.ke - 1);
        const v4u x = __builtin_amdgcn_raw_buffer_load_b128(rq, vq + cs * 1024u, 0u, kNt);
        q[u] = make_uint4(x.x, x.y, x.z, x.w);
        d[u] = __builtin_amdgcn_raw_buffer_load_b32(rd, vd + cs * 128u, 0u, kNt);
      }
    };
    // The plan's members of each segment whose first unit this workgroup holds (so every
    // segment is exported by exactly one workgroup), stored ahead of the staging copies: the
    // staging wait below then covers these stores as well, and no barrier waits for them.
    if (!small && w < ns) {
      const int st = uni(sh_seg[w][0]);
      if (st >= ub && st < ue) {
        const int e = uni(sh_seg[w][1]), nc = uni(sh_seg[w][2]), lo = uni(sh_seg[w][3]) * TP;
        if (lane < nc) p.ws[4 + 2 * E + 1 + off[e] + lo + lane] = sh_mem[w][lane];
      }
    }
    // Stage the batch by direct global-to-LDS copies (no registers). Codes: 1 KB per wave
    // instruction into [4 KC][TP][32] per slot (lane l: half l & 1 of column (l >> 1) & (TP - 1)
    // of block i >> (1 + log2 TP), i = 64 q + l for instruction q). Scales: the raw words
    // d_a | s_a << 16, 256 bytes per instruction into the -8 s_a array [slot][4 KC][8] (lane l:
    // column l & 7), converted in place by the lane that copied them once its copies have
    // landed. A column past the segment's members copies column 0 and a block past K/32 the
    // row's last block: finite values the reader never uses, or multiplies by d_w = 0. Order:
    // copies, then the wave's first two weight loads, then one explicit wait that leaves
    // exactly those weight loads in flight (the counter retires in order).
    {
      // image rows of this lane's code column and scale column in each slot, 16 bits each
      // (rows < 4096), two slots per word; a column past the members takes column 0's row
      const int ccol = (lane >> 1) & (TP - 1), dcol = lane & 7;
      uint32_t rc01 = 0, rc23 = 0, rd01 = 0, rd23 = 0;
#pragma unroll
      for (int k = 0; k < kRoutedMaxSlots; ++k) {
        if (k < ns) {
          const int nck = sh_seg[k][2];
          const uint32_t vc = (uint32_t)sh_row[k][ccol < nck ? ccol : 0];
          const uint32_t vs = (uint32_t)sh_row[k][dcol < nck ? dcol : 0];
          if (k < 2) {
            rc01 |= vc << (16 * k);
            rd01 |= vs << (16 * k);
          } else {
            rc23 |= vc << (16 * (k - 2));
            rd23 |= vs << (16 * (k - 2));
          }
        }
      }
      auto row_of = [](uint32_t w01, uint32_t w23, int k) {
        return ((k & 2 ? w23 : w01) >> (16 * (k & 1))) & 0xffffu;
      };
      const int Kb = p.Kb;
      {  // codes: this wave's instructions w, w + 8, ... of the batch, slot by slot
        const int ipk = (ncode + 63) >> 6;  // copy instructions per slot
        const int half = lane & 1, bl = lane >> (1 + p.tp_log2);
        const int bstep = 64 >> (1 + p.tp_log2);  // blocks per instruction
        int k = 0, q = w;
        while (k < ns && q >= ipk) {
          q -= ipk;
          ++k;
        }
        while (k < ns) {
          const int b = q * bstep + bl;
          const uint32_t irow = row_of(rc01, rc23, k);
          const uint32_t bs = (uint32_t)(b < Kb ? b : Kb - 1);
          if (64 * q + lane < ncode)
            dma_b128(p.codes + ((irow * (uint32_t)p.RB + bs) * 32u + 16u * half),
                     lds_addr(smem + k * p.slot_bytes + 1024 * q));
          q += kWaves;
          while (k < ns && q >= ipk) {
            q -= ipk;
            ++k;
          }
        }
      }
      const int nit = ns * nds, nid = (nit + 63) >> 6;
      for (int q = w; q < nid; q += kWaves) {  // raw scale words, flat over the batch's slots
        const int f = 64 * q + lane;
        const int k = (f >= nds ? 1 : 0) + (f >= 2 * nds ? 1 : 0) + (f >= 3 * nds ? 1 : 0);
        const int b = (f - k * nds) >> 3;
        const uint32_t irow = row_of(rd01, rd23, k);
        const uint32_t bs = (uint32_t)(b < Kb ? b : Kb - 1);
        if (f < nit) dma_b32(p.ds + (irow * (uint32_t)p.RB + bs), lds_addr(msA + 64 * q));
      }
      // the last copy has been issued (a marker in the assembly for the wait-count check; the
      // clobber keeps the weight loads after it)
      asm volatile("; routed staging copies issued" ::: "memory");
      load(qa, da_);
      advance_load();
      load(qb, db_);
      advance_load();
      wait_vmcnt<4 * KU>();
      for (int q = w; q < nid; q += kWaves) {
        const int f = 64 * q + lane;
        if (f < nit) {
          const uint32_t x = __float_as_uint(msA[f]);
          daA[f] = h2f(x);
          msA[f] = -8.0f * h2f(x >> 16);
        }
      }
    }
    __syncthreads();

    // ---- stream this wave's half-units ----
    // A unit whose halves fall to two waves: the first half's owner leaves its sums in its
    // carry slot (LDS, float2 per lane); the second half's owner keeps its own sums and the
    // unit's store targets, and adds the two after the batch's last barrier.
    float2* const xo = reinterpret_cast<float2*>(smem + p.lds_xo);  // [kWaves][64]
    bool pend = false;
    float pend0 = 0.0f, pend1 = 0.0f;
    float* pend_out0 = nullptr;
    float* pend_out1 = nullptr;
    if (ha < hb) {
      start(ha, cc);
      bind_compute(cc);
      float acc[8];
#pragma unroll
      for (int v = 0; v < 8; ++v) acc[v] = 0.0f;
      float carry0 = 0.0f, carry1 = 0.0f;  // first-half sums of the current unit
      // A operand of this lane for token group tg (row m = n of the product's A, k-group g):
      // the staged 32 bytes of column 4 tg + (n & 3), block 4 cs + g, at a_base + cs a_step
      // (low half, high half 16 bytes on), or the 32-byte zero slot (a_step = 0) when the row
      // is outside the lane's k-group or past the segment's columns
      int a_base[2], a_step[2];
      auto bind_a = [&](const Cursor& c) {
        const int nc = uni(sh_seg[c.k][2]);
#pragma unroll
        for (int tg = 0; tg < 2; ++tg) {
          const int col = 4 * tg + (n & 3);
          const bool on = (n >> 2) == g && col < nc;
          a_base[tg] = on ? c.k * p.slot_bytes + (g * TP + col) * 32 : p.lds_zero;
          a_step[tg] = on ? 4 * TP * 32 : 0;
        }
      };
      bind_a(cc);
      const int dsh = 16 * (lane & 1);  // this lane's half of a scale word
      // One step for NTG token groups (1: up to 4 columns, 2: up to 8): every matrix-core
      // product and LDS operand of the step first, then the scaling, so that no vector
      // instruction waits on a product issued just before it. The sums are those of a chunk-by-
      // chunk loop: each acc element still takes its chunks in order.
      auto compute_ntg = [&](auto ntg_c, const uint4 (&q)[KU], const uint32_t (&d)[KU]) {
        constexpr int NTG = decltype(ntg_c)::value;
        const float* daL = daA + cc.k * nds;
        const float* msL = msA + cc.k * nds;
        v4i dd[KU][NTG];
        float4 da4[KU][NTG], ms4[KU][NTG];
#pragma unroll
        for (int u = 0; u < KU; ++u) {
          const int cs = cc.kb + u;
          if (cs >= cc.ke) break;
          v4i blo, bhi;
          blo[0] = (int)(q[u].x & 0x0f0f0f0fu);
          blo[1] = (int)(q[u].y & 0x0f0f0f0fu);
          blo[2] = (int)(q[u].z & 0x0f0f0f0fu);
          blo[3] = (int)(q[u].w & 0x0f0f0f0fu);
          bhi[0] = (int)((q[u].x >> 4) & 0x0f0f0f0fu);
          bhi[1] = (int)((q[u].y >> 4) & 0x0f0f0f0fu);
          bhi[2] = (int)((q[u].z >> 4) & 0x0f0f0f0fu);
          bhi[3] = (int)((q[u].w >> 4) & 0x0f0f0f0fu);
          const int blk = 4 * cs + g;
#pragma unroll
          for (int tg = 0; tg < NTG; ++tg) {
            const unsigned char* ap = smem + a_base[tg] + cs * a_step[tg];
            const v4i alo = *reinterpret_cast<const v4i*>(ap);
            const v4i ahi = *reinterpret_cast<const v4i*>(ap + 16);
            da4[u][tg] = *reinterpret_cast<const float4*>(daL + blk * 8 + 4 * tg);
            ms4[u][tg] = *reinterpret_cast<const float4*>(msL + blk * 8 + 4 * tg);
            const v4i zero = {0, 0, 0, 0};
            dd[u][tg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(alo, blo, zero, 0, 0, 0);
            dd[u][tg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(ahi, bhi, dd[u][tg], 0, 0, 0);
          }
        }
        // the scaling at wave priority 1 (a wave with its products in hand goes first: same-box
        // A/B, padded bucket live 128 35.1 against 35.9 us, live 113 34.4 against 34.7)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int u = 0; u < KU; ++u) {
          if (cc.kb + u >= cc.ke) break;
          const float dw = h2f(d[u] >> dsh);
#pragma unroll
          for (int tg = 0; tg < NTG; ++tg) {
            const v4i x = dd[u][tg];
            const float4 a4 = da4[u][tg], m4 = ms4[u][tg];
            acc[4 * tg + 0] = __builtin_fmaf(dw, __builtin_fmaf(a4.x, (float)x[0], m4.x), acc[4 * tg + 0]);
            acc[4 * tg + 1] = __builtin_fmaf(dw, __builtin_fmaf(a4.y, (float)x[1], m4.y), acc[4 * tg + 1]);
            acc[4 * tg + 2] = __builtin_fmaf(dw, __builtin_fmaf(a4.z, (float)x[2], m4.z), acc[4 * tg + 2]);
            acc[4 * tg + 3] = __builtin_fmaf(dw, __builtin_fmaf(a4.w, (float)x[3], m4.w), acc[4 * tg + 3]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      };
      auto compute = [&](const uint4 (&q)[KU], const uint32_t (&d)[KU]) {
        if (uni(sh_seg[cc.k][2]) > 4)
          compute_ntg(std::integral_constant<int, 2>{}, q, d);
        else
          compute_ntg(std::integral_constant<int, 1>{}, q, d);
      };
      // after a compute step: at the end of a half-unit, sum the k-group lanes; at the end of
      // a unit store (or hand over), and move the compute cursor to the next half-unit
      auto finish_step = [&]() {
        cc.kb += KU;
        if (cc.kb < cc.ke) return;
        // the four k-group lanes of a row, reduced and scattered: a swap of the lanes 32 apart
        // carries columns c and c + 4 at once (lanes g < 2 keep column c, g >= 2 column c + 4,
        // summed over g and g + 2), then a swap of the lanes 16 apart carries two of those, so
        // lane g ends with columns 2 g and 2 g + 1 summed over all four
        float h[4], v2[2];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[c]), __float_as_uint(acc[c + 4]),
                                                            false, false);
          h[c] = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(h[c]), __float_as_uint(h[c + 2]),
                                                            false, false);
          v2[c] = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
        }
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[v] = 0.0f;
        const bool first = halves == 2 && (cc.hu & 1) == 0;
        const bool next = cc.hu + 1 < hb;
        if (first) {
          if (next) {  // the second half follows in this wave
            carry0 = v2[0];
            carry1 = v2[1];
          } else {
            xo[w * 64 + lane] = make_float2(v2[0], v2[1]);
          }
        } else {
          const bool own_first = halves == 1 || cc.hu - 1 >= ha;
          float o0 = v2[0], o1 = v2[1];
          if (halves == 2 && own_first) {
            o0 = carry0 + o0;
            o1 = carry1 + o1;
          }
          const int nc = uni(sh_seg[cc.k][2]);
          const bool row_ok = crow < p.r[cri].N;
          float* const out = p.r[cri].out + crow;
          const int64_t ld = p.r[cri].ld;
          float* const t0 = row_ok && 2 * g < nc ? out + (int64_t)sh_mem[cc.k][2 * g] * ld : nullptr;
          float* const t1 = row_ok && 2 * g + 1 < nc ? out + (int64_t)sh_mem[cc.k][2 * g + 1] * ld : nullptr;
          if (own_first) {
            if (t0) *t0 = o0;
            if (t1) *t1 = o1;
          } else {  // the first half belongs to an earlier wave: add after the barrier
            pend = true;
            pend0 = o0;
            pend1 = o1;
            pend_out0 = t0;
            pend_out1 = t1;
          }
        }
        if (next) {
          const int pu = cc.u;
          start(cc.hu + 1, cc);
          if (cc.u != pu) {
            bind_compute(cc);
            bind_a(cc);
          }
        }
      };
      // steps of this wave: H / KU per first half, ceil((KC - H) / KU) per second half (with
      // one half per unit, ceil(KC / KU))
      int S;
      if (halves == 2) {
        const int n0 = (hb + 1) / 2 - (ha + 1) / 2;  // even half-units in [ha, hb)
        S = n0 * (H / KU) + (hb - ha - n0) * ((KC - H + KU - 1) / KU);
      } else {
        S = (hb - ha) * ((KC + KU - 1) / KU);
      }
      for (int st = 0; st < S; st += 2) {
        compute(qa, da_);
        finish_step();
        load(qa, da_);
        advance_load();
        if (st + 1 < S) {
          compute(qb, db_);
          finish_step();
        }
        load(qb, db_);  // unconditional: a load past the wave's last half-unit reads nothing
        advance_load();
      }
    }
    // the trailing repeated loads land before the next batch reuses their registers (without
    // this the compiler waits for every load at the start of each batch's streaming, the
    // first included)
    wait_vmcnt<0>();
    __syncthreads();
    if (pend) {  // the first half's sums: from the last wave before this one with work
      int v = w - 1;
      while (v > 0 && hstart(v) == hstart(v + 1)) --v;
      const float2 x = xo[v * 64 + lane];
      if (pend_out0) *pend_out0 = x.x + pend0;
      if (pend_out1) *pend_out1 = x.y + pend1;
    }
    ub = ue;
  }
  // The rest of the plan, exported after the last barrier (a global store before a barrier
  // makes that barrier wait for every load in flight): workgroup 0 the counts, offsets and
  // error word (the members went out with each batch's staging).
  if (blockIdx.x == 0) {
    int32_t* counts = p.ws + 4;
    int32_t* offsets = counts + E;
    if constexpr (small) {
      // lower bound of expert e in the sorted keys: a binary search over the lanes (every lane
      // searches, so that every source lane of the permutes is active)
      auto lb = [&](int e) {
        int lo = 0;
#pragma unroll
        for (int st = 32; st > 0; st >>= 1)
          if (__builtin_amdgcn_ds_bpermute((lo + st - 1) << 2, s_e) < e) lo += st;
        return __builtin_amdgcn_ds_bpermute(lo << 2, s_e) < e ? lo + 1 : lo;
      };
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int e = tid + kWaves * 64 * i, ec = e < E ? e : E;
        const int a = lb(ec), b = lb(ec + 1);
        if (e < E) {
          counts[e] = b - a;
          offsets[e] = a;
        }
      }
    } else {
      for (int e = tid; e < E; e += blockDim.x) {
        counts[e] = cnt[e];
        offsets[e] = off[e];
      }
    }
    if (tid == 0) {
      const bool bad = small ? s_bad : sh_misc[0] != 0;
      p.ws[0] = (bad ? QIMG_ERR_EXPERT_RANGE : 0) | (clamped ? QIMG_ERR_LIVE_CLAMPED : 0);
      p.ws[1] = P;
      p.ws[2] = 0;
      p.ws[3] = 0;
      offsets[E] = small ? s_valid_n : off[E];
    }
  }
}

// Plain streaming read of a contiguous buffer (the measured ceiling of the readers): workgroup
// i reads pieces [i per, (i + 1) per) of 1 KB, its wave w pieces w, w + 8, ... with four loads
// in flight; loads past the wave's last piece go to an out-of-range offset (no memory access).
constexpr int kCeilWaves = 8, kCeilDepth = 4, kCeilGrid = 256;
static_assert(kCeilGrid * kCeilWaves == QIMG_CEILING_SINK_WORDS, "one sink word per wave");
__global__ __launch_bounds__(kCeilWaves * 64) void read_ceiling_kernel(const uint8_t* buf, uint32_t pieces,
                                                                       uint32_t* sink) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t per = (pieces + gridDim.x - 1) / gridDim.x;
  const uint32_t c0 = blockIdx.x * per;
  const uint32_t c1 = c0 + per < pieces ? c0 + per : pieces;
  const int n = c0 + w < c1 ? (int)((c1 - c0 - w + kCeilWaves - 1) / kCeilWaves) : 0;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc((void*)buf, (short)0, (int)(pieces * 1024u), kBufferFlags);
  auto off = [&](int j) {
    return j < n ? (c0 + w + (uint32_t)kCeilWaves * (uint32_t)j) * 1024u + 16u * lane : 0x80000000u;
  };
  v4u q[kCeilDepth];
#pragma unroll
  for (int j = 0; j < kCeilDepth; ++j) q[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off(j), 0u, kNt);
  uint32_t acc = 0;
  for (int b = 0; b < n; b += kCeilDepth) {
#pragma unroll
    for (int j = 0; j < kCeilDepth; ++j) {
      acc ^= q[j].x ^ q[j].y ^ q[j].z ^ q[j].w;
      q[j] = __builtin_amdgcn_raw_buffer_load_b128(rs, off(b + kCeilDepth + j), 0u, kNt);
    }
  }
#pragma unroll
  for (int j = 0; j < kCeilDepth; ++j) acc ^= q[j].x;  // the last loads (zeros) land before the exit
  acc = wave_xor(acc);
  if (lane == 0) sink[blockIdx.x * kCeilWaves + w] = acc;
}

// Standard planes -> tiled order (see the reader notes above). Rows and blocks past N and
// K/32 are written as zeros, so tiles and chunks are always whole. FMT 0 Q4_0 and 2 Q4_1:
// 1 KB of codes per chunk (lane l: the 16 bytes of block 4 s + l/16 of row l%16); Q8_0:
// 2 KB, the first 16 bytes of every lane's block, then the second 16. Scales after all codes:
// fp16 d (Q4_0, Q8_0) or the 32-bit word d | m << 16 (Q4_1), lane order.
template <int FMT>
__global__ void tile_weights_kernel(const uint8_t* __restrict__ qs, const uint16_t* __restrict__ d,
                                    const uint16_t* __restrict__ m, int N, int Kb, int KC, int tiles,
                                    int E, uint8_t* __restrict__ tq, uint8_t* __restrict__ tsc) {
  const int64_t total = (int64_t)E * tiles * KC * 64;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int lane = (int)(o & 63);
    const int64_t c = o >> 6;
    const int s = (int)(c % KC);
    const int64_t et = c / KC;
    const int tile = (int)(et % tiles);
    const int64_t e = et / tiles;
    const int row = tile * 16 + (lane & 15);
    const int blk = 4 * s + (lane >> 4);
    const bool in = row < N && blk < Kb;
    const int64_t src = (e * N + row) * Kb + blk;
    if constexpr (FMT == 1) {
      uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
      if (in) {
        v0 = reinterpret_cast<const uint4*>(qs)[2 * src];
        v1 = reinterpret_cast<const uint4*>(qs)[2 * src + 1];
      }
      reinterpret_cast<uint4*>(tq)[(2 * c) * 64 + lane] = v0;
      reinterpret_cast<uint4*>(tq)[(2 * c + 1) * 64 + lane] = v1;
    } else {
      reinterpret_cast<uint4*>(tq)[o] = in ? reinterpret_cast<const uint4*>(qs)[src] : make_uint4(0, 0, 0, 0);
    }
    if constexpr (FMT == 2)
      reinterpret_cast<uint32_t*>(tsc)[o] = in ? ((uint32_t)d[src] | ((uint32_t)m[src] << 16)) : 0u;
    else
      reinterpret_cast<uint16_t*>(tsc)[o] = in ? d[src] : (uint16_t)0;
  }
}

// host helpers
// ---------------------------------------------------------------------------------------------
inline bool al16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
inline bool al(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

struct Span {
  uintptr_t lo, hi;
};
inline Span span(const void* p, int64_t bytes) {
  return Span{(uintptr_t)p, (uintptr_t)p + (uintptr_t)(bytes > 0 ? bytes : 0)};
}
inline bool overlap(Span a, Span b) {
  return a.lo != a.hi && b.lo != b.hi && a.lo < b.hi && b.lo < a.hi;
}
inline int64_t rows_extent(int64_t rows, int64_t ld, int64_t width, int64_t elem) {
  return rows <= 0 ? 0 : ((rows - 1) * ld + width) * elem;
}

inline int check_k(int32_t K) {
  if (K <= 0 || K % 32 != 0) return QIMG_EINVAL;
  if (K > QIMG_MAX_K) return QIMG_EUNSUPPORTED;
  return QIMG_OK;
}

inline int32_t row_blocks(int32_t K) { return ((K / 32 + 15) / 16) * 16; }

inline int launch_status() {
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? QIMG_OK : QIMG_EHIP;
}

// Producer launch shape: Jp = next power of two >= ceil(K/256) leaf slots per lane;
// W = min(kRmsWaves, max(1, Jp/2)) waves, or Jp/8 where that is more, JW = Jp / W slots per
// lane (at most 8).
// The element-wise producers and the quantizer need no row-wide value: their rows are cut into
// slices of at most kEltWaves waves x 64 lanes x 1 leaf (256 elements a wave), one workgroup each.
constexpr int kRmsSplitWgs = 256;  // RMS rows are split while rows x shares stay within this
constexpr int kRmsWaves = 8;       // RMS producer waves per workgroup, up to K = 16384
constexpr int kEltWaves = 4;       // waves per workgroup of the element-wise producers

int launch_emit(int op, EmitArgs& a, hipStream_t s) {
  const int J = (a.K + 255) / 256;
  int W, JW, S = 1;
  if (op == OP_RMS) {
    int Jp = 1;
    while (Jp < J) Jp <<= 1;
    // 8 waves of 2 to 8 leaves per lane (the sum's order does not depend on the split); 16
    // waves only where a lane would otherwise hold more than 8 leaves (K above 16384)
    W = Jp / 2;
    if (W < 1) W = 1;
    if (W > kRmsWaves) W = kRmsWaves;
    if (Jp / W > 8) W = Jp / 8;
    JW = Jp / W;
    // few rows: split each row's per-element work over S workgroups (powers of two, at least
    // one leaf group each, at most kRmsSplitWgs workgroups in all)
    const int groups = W * JW;
    while (S * 2 <= groups && (int64_t)a.rows * S * 2 <= kRmsSplitWgs) S *= 2;
  } else {
    W = J < kEltWaves ? J : kEltWaves;
    JW = 1;
    S = (J + W - 1) / W;
  }
  dim3 grid(a.rows, S), block(W * 64);
#define QIMG_EMIT_CASE(OPV, JWV) \
  if (op == OPV && JW == JWV) { hipLaunchKernelGGL((emit_kernel<OPV, JWV>), grid, block, 0, s, a); return launch_status(); }
  // RMS rows are whole rows (JW leaves per lane); the element-wise ops use slices with JW = 1
  QIMG_EMIT_CASE(OP_RMS, 1) QIMG_EMIT_CASE(OP_RMS, 2) QIMG_EMIT_CASE(OP_RMS, 4) QIMG_EMIT_CASE(OP_RMS, 8)
  QIMG_EMIT_CASE(OP_SWIGLU, 1)
  QIMG_EMIT_CASE(OP_GEGLU, 1)
  QIMG_EMIT_CASE(OP_QUANT, 1)
  QIMG_EMIT_CASE(OP_REGLU, 1)
  QIMG_EMIT_CASE(OP_GEGLU_TANH, 1)
  QIMG_EMIT_CASE(OP_GEGLU_QUICK, 1)
  QIMG_EMIT_CASE(OP_SWIGLU_OAI, 1)
  QIMG_EMIT_CASE(OP_SWIGLU_CLAMP, 1)
#undef QIMG_EMIT_CASE
  return QIMG_EUNSUPPORTED;
}


inline int cu_count() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

inline int64_t tiled_chunks(int32_t N, int32_t K, int32_t E) {
  const int64_t tiles = (N + 15) / 16, KC = (K / 32 + 3) / 4;
  return (int64_t)E * tiles * KC;
}

constexpr int kMaxLds = 156 * 1024;  // dynamic LDS; 4 KB left for static arrays (160 KB per workgroup)

struct ReadPlan {
  int grid, ntm, lds;
};

// LDS layout of the ordinary reader: staged codes [4 KC][tp][32] (padded to whole 1 KB copy
// instructions), raw scale words (d_a | s_a << 16) [4 KC][tp] (padded to 256 B instructions),
// or with 8 columns per pass 32 words per step in a run per wave, a 32-byte zero slot,
// cross-wave sums [waves][ntm][16][8] f32. tp is the widest of 8, 4, 2, 1 image columns per
// pass that fits.
inline bool plan_lds(ReadArgs& a, int ntm, int* total) {
  const int nb = 4 * a.KC;
  for (int tp : {8, 4, 2, 1}) {
    if (tp > 1 && tp / 2 >= a.rows) continue;  // a narrower pass holds every image row
    const int codes = (nb * tp * 2 + 63) / 64 * 1024;
    int raw = (nb * tp + 63) / 64 * 256;
    a.raw_wave = 0;
    if (tp == 8) {  // per-wave runs of 32 words per step (see stage_own)
      const int steps = (a.KC + kOrdWaves - 1) / kOrdWaves;
      a.raw_wave = (steps + 1) / 2 * 256;
      raw = kOrdWaves * a.raw_wave;
    }
    const int red = kOrdWaves * ntm * 16 * 8 * 4;
    const int t = codes + raw + 32 + red;
    if (t <= kMaxLds) {
      a.tp = tp;
      a.tp_log2 = tp == 8 ? 3 : tp == 4 ? 2 : tp == 2 ? 1 : 0;
      a.lds_raw = codes;
      a.lds_zero = codes + raw;
      a.lds_red = a.lds_zero + 32;
      *total = t;
      return true;
    }
  }
  return false;
}

template <int MODE, int NTG>
int launch_read_g(ReadArgs& a, int grid, int ntm, int lds, hipStream_t s) {
  const void* fn = ntm == 1 ? (const void*)mmvq_tiled_kernel<1, MODE, NTG>
                 : ntm == 2 ? (const void*)mmvq_tiled_kernel<2, MODE, NTG>
                 : ntm == 3 ? (const void*)mmvq_tiled_kernel<3, MODE, NTG>
                            : (const void*)mmvq_tiled_kernel<4, MODE, NTG>;
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return QIMG_EHIP;
  dim3 g(grid), b(kOrdWaves * 64);
  if (ntm == 1) hipLaunchKernelGGL((mmvq_tiled_kernel<1, MODE, NTG>), g, b, lds, s, a);
  else if (ntm == 2) hipLaunchKernelGGL((mmvq_tiled_kernel<2, MODE, NTG>), g, b, lds, s, a);
  else if (ntm == 3) hipLaunchKernelGGL((mmvq_tiled_kernel<3, MODE, NTG>), g, b, lds, s, a);
  else hipLaunchKernelGGL((mmvq_tiled_kernel<4, MODE, NTG>), g, b, lds, s, a);
  return launch_status();
}

// One token group when no pass can hold more than 4 image columns.
template <int MODE>
int launch_read(ReadArgs& a, int grid, int ntm, int lds, hipStream_t s) {
  const int max_cols = a.rows < a.tp ? a.rows : a.tp;
  return max_cols <= 4 ? launch_read_g<MODE, 1>(a, grid, ntm, lds, s)
                       : launch_read_g<MODE, 2>(a, grid, ntm, lds, s);
}

inline int ntm_for(int64_t tiles_per_wg) {
  return tiles_per_wg <= 1 ? 1 : tiles_per_wg <= 2 ? 2 : tiles_per_wg <= 3 ? 3 : 4;
}

// Ordinary readers: one workgroup per CU (fewer when there are fewer half tiles); each takes an
// equal contiguous run of half tiles (8 weight rows) over the concatenated readers, so that no
// workgroup streams more than its share (640 tiles on 256 CUs: 2.5 tiles each, not 3 and 2).
template <int MODE>
int run_ordinary(ReadArgs& a, hipStream_t s) {
  int halves = 0;
  for (int i = 0; i < a.n_readers; ++i) {
    a.half_start[i] = halves;
    halves += (a.r[i].N + 7) / 8;
  }
  a.half_start[a.n_readers] = halves;
  a.halves_total = halves;
  a.tiles_total = a.tile_start[a.n_readers];
  int G = cu_count();
  if (halves < G) G = halves;
  a.half_q = halves / G;
  a.half_r = halves % G;
  // the most slots (whole or half tiles) any workgroup's run of half tiles covers, as the
  // kernel walks it
  int most = 1;
  for (int wg = 0; wg < G; ++wg) {
    const int h0 = a.half_q * wg + (int)((uint32_t)a.half_r * (uint32_t)wg / (uint32_t)G);
    const int h1 = a.half_q * (wg + 1) + (int)((uint32_t)a.half_r * (uint32_t)(wg + 1) / (uint32_t)G);
    int slots = 0, ri = 0;
    for (int h = h0; h < h1; ++slots) {
      while (ri + 1 < a.n_readers && h >= a.half_start[ri + 1]) ++ri;
      const int lh = h - a.half_start[ri];
      h += ((lh & 1) == 0 && h + 1 < h1 && h + 1 < a.half_start[ri + 1]) ? 2 : 1;
    }
    if (slots > most) most = slots;
  }
  const int ntm = ntm_for(most);
  int lds = 0;
  if (!plan_lds(a, ntm, &lds)) return QIMG_EUNSUPPORTED;
  return launch_read<MODE>(a, G, ntm, lds, s);
}

// Routed readers: one workgroup per CU over the (expert, pass, tile) units. LDS: the codes of
// `slots` staged segments, [4 KC][tp][32] each, then their f32 d_a and -8 s_a, [slot][4 KC][8]
// each, the 32-byte zero slot, the half-unit carry slots, then the plan arrays sid[pairs, padded to
// 256] (expert of each live pair), cnt[E], off[E+1], pps[E+1] (first segment of each expert).
constexpr int kXoBytes = kWaves * 64 * 8;
int run_routed(ReadArgs& a, int pairs_cap, hipStream_t s) {
  const int tiles = a.tile_start[a.n_readers];
  a.tiles_total = tiles;
  a.pairs_cap = pairs_cap;
  if ((int64_t)(pairs_cap + a.E) * tiles > 0x7fffffff) return QIMG_EUNSUPPORTED;
  // the weight loads address a reader's planes with 32-bit offsets
  for (int i = 0; i < a.n_readers; ++i)
    if ((int64_t)a.E * a.r[i].tiles * a.KC * 1024 > 0x7fffffff) return QIMG_EUNSUPPORTED;
  for (int i = a.n_readers + 1; i <= QIMG_MAX_READERS; ++i) a.tile_start[i] = 0x7fffffff;
  // a launch of at most 64 pairs keeps its plan in registers (no LDS plan arrays)
  const bool small = pairs_cap <= 64;
  const int plan = small ? 0 : 4 * (((pairs_cap + 255) & ~255) + 3 * a.E + 2);
  const int nb = 4 * a.KC;
  // the widest column pass that leaves room for two staged segments, else for one
  int lds = -1;
  for (int need : {2, 1}) {
    for (int tp : {8, 4, 2, 1}) {
      const int slot = nb * tp * 32 + nb * 64;
      int slots = (kMaxLds - 32 - kXoBytes - plan) / slot;
      if (slots > kRoutedMaxSlots) slots = kRoutedMaxSlots;
      if (slots >= need) {
        a.tp = tp;
        a.tp_log2 = tp == 8 ? 3 : tp == 4 ? 2 : tp == 2 ? 1 : 0;
        a.slots = slots;
        a.slot_bytes = nb * tp * 32;
        a.lds_da = slots * a.slot_bytes;
        a.lds_ms = a.lds_da + slots * nb * 32;
        a.lds_zero = a.lds_ms + slots * nb * 32;
        a.lds_xo = a.lds_zero + 32;
        a.lds_plan = a.lds_xo + kXoBytes;
        lds = a.lds_plan + plan;
        break;
      }
    }
    if (lds >= 0) break;
  }
  if (lds < 0) return QIMG_EUNSUPPORTED;
  // K halves: the first a whole number of loads (KU chunks), about half of K; no cut when the
  // second half would be empty
  const int H = kRoutedKu * ((a.KC + 2 * kRoutedKu - 1) / (2 * kRoutedKu));
  a.halves = H < a.KC ? 2 : 1;
  a.khalf = H < a.KC ? H : a.KC;
  const int G = cu_count();
  a.fd_grid = fast_div((uint32_t)G);
  a.fd_tiles = fast_div((uint32_t)tiles);
  const void* fn = small ? (const void*)mmvq_routed_kernel<kRoutedKu, true>
                         : (const void*)mmvq_routed_kernel<kRoutedKu, false>;
  if (lds > 64 * 1024 &&
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
    return QIMG_EHIP;
  if (small)
    hipLaunchKernelGGL((mmvq_routed_kernel<kRoutedKu, true>), dim3(G), dim3(kWaves * 64), lds, s, a);
  else
    hipLaunchKernelGGL((mmvq_routed_kernel<kRoutedKu, false>), dim3(G), dim3(kWaves * 64), lds, s, a);
  return launch_status();
}

// Plan memory of the allocation-free routed reader: one array per GPU (each device holds its
// own copy until the process ends) with room for the routed workspace of the largest call the
// routed readers take (QIMG_MAX_ROUTED_PAIRS pairs, QIMG_MAX_EXPERTS experts). In host code the
// name is a host-side stand-in, not a device address: the kernels get the address that
// hipGetSymbolAddress returns for the current device, kept per device below.
constexpr int kScratchWords = 6400;
static_assert(4 + 2 * QIMG_MAX_EXPERTS + 1 + QIMG_MAX_ROUTED_PAIRS <= kScratchWords, "scratch plan size");
static __device__ __align__(256) int32_t scratch[kScratchWords];
static_assert(sizeof(scratch) == QIMG_NOALLOC_SCRATCH_BYTES, "documented scratch size");

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's `scratch`, looked up once per device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QIMG_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return QIMG_EHIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return QIMG_OK;
}

}  // namespace

// =============================================================================================
// C ABI
// =============================================================================================
extern "C" {

const char* qimg_strerror(int status) {
  switch (status) {
    case QIMG_OK: return "ok";
    case QIMG_EINVAL: return "invalid argument (null pointer, bad size or op)";
    case QIMG_EALIGN: return "misaligned plane base or stride";
    case QIMG_EALIAS: return "an output overlaps an input or another output";
    case QIMG_EUNSUPPORTED: return "shape outside the supported range";
    case QIMG_EWORKSPACE: return "routed workspace missing or too small";
    case QIMG_EHIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int qimg_abi_version(void) { return QIMG_ABI_VERSION; }

int32_t qimg_row_blocks(int32_t K) { return check_k(K) == QIMG_OK ? row_blocks(K) : 0; }

int64_t qimg_image_bytes(int32_t rows, int32_t K) {
  if (rows < 0 || check_k(K) != QIMG_OK) return 0;
  return (int64_t)rows * row_blocks(K) * 36;
}

struct EmitExtra {  // producer parameters beyond the common ones
  const float* beta = nullptr;
  float scale = 1.0f, alpha = 0.0f, limit = 0.0f;
};

static int emit_common(int op, const float* a, int64_t lda, const float* b, int64_t ldb,
                       int b_rows, float eps, int32_t rows, const int32_t* live_rows, int32_t K,
                       float* y, int64_t ldy, void* img, void* stream, int32_t live_mul = 1,
                       EmitExtra ex = EmitExtra{}) {
  int st = check_k(K);
  if (st) return st;
  if (rows < 0) return QIMG_EINVAL;
  if (rows == 0) return QIMG_OK;
  if (!a || (op != OP_QUANT && !y) || (op == OP_QUANT && !img)) return QIMG_EINVAL;
  if (is_glu(op) && !b) return QIMG_EINVAL;
  if (lda < K || (op != OP_QUANT && ldy < K) || (b && b_rows > 1 && ldb < K)) return QIMG_EINVAL;
  if (!al16(a) || lda % 4 || (b && (!al16(b) || (b_rows > 1 && ldb % 4))) ||
      (y && (!al16(y) || ldy % 4)) || (img && !al16(img)) || (live_rows && !al(live_rows, 4)) ||
      (ex.beta && !al16(ex.beta)))
    return QIMG_EALIGN;
  const int64_t ib = qimg_image_bytes(rows, K);
  const Span sa = span(a, rows_extent(rows, lda, K, 4));
  const Span sb = b ? span(b, b_rows > 1 ? rows_extent(rows, ldb, K, 4) : (int64_t)K * 4) : Span{0, 0};
  const Span sy = y ? span(y, rows_extent(rows, ldy, K, 4)) : Span{0, 0};
  const Span si = img ? span(img, ib) : Span{0, 0};
  const Span sl = live_rows ? span(live_rows, 4) : Span{0, 0};
  const Span sbeta = ex.beta ? span(ex.beta, (int64_t)K * 4) : Span{0, 0};
  if (overlap(sy, sa) || overlap(sy, sb) || overlap(sy, sl) || overlap(sy, sbeta) ||
      overlap(si, sl) || overlap(sy, si))
    return QIMG_EALIAS;
  // an image over the producer's own inputs: emission declined, the original two steps run
  const bool decline = overlap(si, sa) || overlap(si, sb) || overlap(si, sbeta);
  if (decline && op == OP_QUANT) return QIMG_EALIAS;  // the quantizer's input is y itself

  EmitArgs e{};
  e.a = a; e.lda = lda; e.b = b; e.ldb = ldb; e.y = y; e.ldy = ldy;
  const int RB = row_blocks(K);
  uint8_t* codes = (uint8_t*)img;
  uint32_t* ds = img ? (uint32_t*)((uint8_t*)img + (size_t)rows * RB * 32) : nullptr;
  e.codes = decline ? nullptr : codes;
  e.ds = decline ? nullptr : ds;
  e.live_rows = live_rows; e.rows = rows; e.K = K; e.Kb = K / 32; e.RB = RB; e.eps = eps;
  e.live_mul = live_mul;
  e.beta = ex.beta; e.scale = ex.scale; e.alpha = ex.alpha; e.limit = ex.limit;
  st = launch_emit(op, e, (hipStream_t)stream);
  if (st || !decline) return st;
  EmitArgs q{};
  q.a = y; q.lda = ldy; q.codes = codes; q.ds = ds;
  q.live_rows = live_rows; q.rows = rows; q.K = K; q.Kb = K / 32; q.RB = RB;
  q.live_mul = live_mul; q.scale = 1.0f;
  return launch_emit(OP_QUANT, q, (hipStream_t)stream);
}

int qimg_emit_rmsnorm(const float* x, int64_t ldx, const float* gamma, float eps, int32_t rows,
                      const int32_t* live_rows, int32_t K, float* y, int64_t ldy, void* img,
                      void* stream) {
  return emit_common(OP_RMS, x, ldx, gamma, 0, 1, eps, rows, live_rows, K, y, ldy, img, stream);
}

// kernel op of a public GLU op; params: whether the op takes alpha/limit. -1: unknown op.
static int glu_kop(int32_t op, bool* params) {
  *params = false;
  switch (op) {
    case QIMG_GLU_SWIGLU: return OP_SWIGLU;
    case QIMG_GLU_GEGLU_ERF: return OP_GEGLU;
    case QIMG_GLU_REGLU: return OP_REGLU;
    case QIMG_GLU_GEGLU: return OP_GEGLU_TANH;
    case QIMG_GLU_GEGLU_QUICK: return OP_GEGLU_QUICK;
    case QIMG_GLU_SWIGLU_OAI: *params = true; return OP_SWIGLU_OAI;
    case QIMG_GLU_SWIGLU_CLAMP: *params = true; return OP_SWIGLU_CLAMP;
    default: return -1;
  }
}

int qimg_emit_rmsnorm_ex(const float* x, int64_t ldx, const float* gamma, const float* beta,
                         float scale, float eps, int32_t rows, const int32_t* live_rows,
                         int32_t K, float* y, int64_t ldy, void* img, void* stream) {
  if (!(scale == scale) || __builtin_isinf(scale)) return QIMG_EINVAL;
  EmitExtra ex;
  ex.beta = beta;
  ex.scale = scale;
  return emit_common(OP_RMS, x, ldx, gamma, 0, 1, eps, rows, live_rows, K, y, ldy, img, stream, 1, ex);
}

int qimg_emit_glu_ex(int32_t op, float alpha, float limit, const float* gate, int64_t ldg,
                     const float* up, int64_t ldu, int32_t rows, const int32_t* live_rows,
                     int32_t K, float* y, int64_t ldy, void* img, void* stream) {
  bool params;
  const int kop = glu_kop(op, &params);
  if (kop < 0) return QIMG_EINVAL;
  if (params && (!(alpha == alpha) || __builtin_isinf(alpha) || !(limit >= 0.0f))) return QIMG_EINVAL;
  EmitExtra ex;
  ex.alpha = alpha;
  ex.limit = limit;
  return emit_common(kop, gate, ldg, up, ldu, 2, 0.0f, rows, live_rows, K, y, ldy, img, stream, 1, ex);
}

int qimg_emit_glu(int32_t op, const float* gate, int64_t ldg, const float* up, int64_t ldu,
                  int32_t rows, const int32_t* live_rows, int32_t K, float* y, int64_t ldy,
                  void* img, void* stream) {
  bool params;
  const int kop = glu_kop(op, &params);
  if (kop < 0 || params) return QIMG_EINVAL;
  // gate and up may be the two halves of one packed row (they must not overlap each other's
  // elements, which packed halves do not)
  return emit_common(kop, gate, ldg, up, ldu, 2, 0.0f, rows, live_rows, K, y, ldy, img, stream);
}

int qimg_emit_glu_per_slot(int32_t op, const float* gate, int64_t ldg, const float* up,
                           int64_t ldu, int32_t bucket, int32_t top_k, const int32_t* live_rows,
                           int32_t K, float* y, int64_t ldy, void* img, void* stream) {
  bool params;
  const int kop = glu_kop(op, &params);
  if (kop < 0 || params) return QIMG_EINVAL;
  if (bucket < 0 || top_k <= 0) return QIMG_EINVAL;
  if ((int64_t)bucket * top_k > QIMG_MAX_ROUTED_PAIRS) return QIMG_EUNSUPPORTED;
  return emit_common(kop, gate, ldg, up, ldu, 2, 0.0f, bucket * top_k, live_rows, K, y, ldy, img,
                     stream, top_k);
}

int qimg_quantize_q8_1(const float* y, int64_t ldy, int32_t rows, const int32_t* live_rows,
                       int32_t K, void* img, void* stream) {
  return emit_common(OP_QUANT, y, ldy, nullptr, 0, 0, 0.0f, rows, live_rows, K, nullptr, 0, img,
                     stream);
}


static int64_t tiled_bytes_fmt(int fmt, int32_t N, int32_t K, int32_t E) {
  if (N <= 0 || E <= 0 || check_k(K) != QIMG_OK) return 0;
  return tiled_chunks(N, K, E) * (fmt == 1 ? 2048 + 128 : fmt == 2 ? 1024 + 256 : 1024 + 128);
}

static int tile_common(int fmt, const void* qs, const void* d, const void* m, int32_t N, int32_t K,
                       int32_t E, void* tiled, void* stream) {
  int st = check_k(K);
  if (st) return st;
  if (!qs || !d || (fmt == 2 && !m) || !tiled || N <= 0 || E <= 0) return QIMG_EINVAL;
  if (!al16(qs) || !al(d, 2) || (m && !al(m, 2)) || !al16(tiled)) return QIMG_EALIGN;
  const int Kb = K / 32;
  const int64_t chunks = tiled_chunks(N, K, E);
  const int64_t cbytes = fmt == 1 ? 2048 : 1024;
  const Span so = span(tiled, tiled_bytes_fmt(fmt, N, K, E));
  const int64_t blocks_in = (int64_t)E * N * Kb;
  if (overlap(so, span(qs, blocks_in * (fmt == 1 ? 32 : 16))) || overlap(so, span(d, blocks_in * 2)) ||
      (m && overlap(so, span(m, blocks_in * 2))))
    return QIMG_EALIAS;
  const int64_t total = chunks * 64;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  const int KC = (Kb + 3) / 4, tiles = (N + 15) / 16;
  uint8_t* tq = (uint8_t*)tiled;
  uint8_t* tsc = tq + chunks * cbytes;
  hipStream_t s = (hipStream_t)stream;
  const dim3 g((unsigned)blocks), b(256);
  if (fmt == 1)
    hipLaunchKernelGGL(tile_weights_kernel<1>, g, b, 0, s, (const uint8_t*)qs, (const uint16_t*)d, nullptr, N, Kb, KC, tiles, E, tq, tsc);
  else if (fmt == 2)
    hipLaunchKernelGGL(tile_weights_kernel<2>, g, b, 0, s, (const uint8_t*)qs, (const uint16_t*)d, (const uint16_t*)m, N, Kb, KC, tiles, E, tq, tsc);
  else
    hipLaunchKernelGGL(tile_weights_kernel<0>, g, b, 0, s, (const uint8_t*)qs, (const uint16_t*)d, nullptr, N, Kb, KC, tiles, E, tq, tsc);
  return launch_status();
}

int64_t qimg_q4_0_tiled_bytes(int32_t N, int32_t K, int32_t E) { return tiled_bytes_fmt(0, N, K, E); }
int64_t qimg_q8_0_tiled_bytes(int32_t N, int32_t K, int32_t E) { return tiled_bytes_fmt(1, N, K, E); }
int64_t qimg_q4_1_tiled_bytes(int32_t N, int32_t K, int32_t E) { return tiled_bytes_fmt(2, N, K, E); }

int qimg_q4_0_tile(const void* qs, const void* d, int32_t N, int32_t K, int32_t E, void* tiled,
                   void* stream) {
  return tile_common(0, qs, d, nullptr, N, K, E, tiled, stream);
}
int qimg_q8_0_tile(const void* qs, const void* d, int32_t N, int32_t K, int32_t E, void* tiled,
                   void* stream) {
  return tile_common(1, qs, d, nullptr, N, K, E, tiled, stream);
}
int qimg_q4_1_tile(const void* qs, const void* d, const void* m, int32_t N, int32_t K, int32_t E,
                   void* tiled, void* stream) {
  return tile_common(2, qs, d, m, N, K, E, tiled, stream);
}

static int check_image(const void* img) {
  if (!img) return QIMG_EINVAL;
  if (!al16(img)) return QIMG_EALIGN;
  return QIMG_OK;
}

static void fill_common(ReadArgs& a, const void* img, int32_t rows, int32_t K) {
  const int RB = row_blocks(K);
  a.codes = (const uint8_t*)img;
  a.ds = (const uint32_t*)((const uint8_t*)img + (size_t)rows * RB * 32);
  a.RB = RB;
  a.Kb = K / 32;
  a.KC = (K / 32 + 3) / 4;
  a.rows = rows;
}

static int ordinary_common(int fmt, const qimg_q4_0_reader* readers, int32_t n_readers,
                           const void* img, int32_t rows, const int32_t* live_rows, int32_t K,
                           void* stream) {
  int st = check_k(K);
  if (st) return st;
  if (!readers || n_readers < 1 || n_readers > QIMG_MAX_READERS || rows < 0) return QIMG_EINVAL;
  if (rows == 0) return QIMG_OK;
  if ((st = check_image(img))) return st;
  if (live_rows && !al(live_rows, 4)) return QIMG_EALIGN;
  const Span si = span(img, qimg_image_bytes(rows, K));
  const Span sl = live_rows ? span(live_rows, 4) : Span{0, 0};
  Span outs[QIMG_MAX_READERS];
  for (int i = 0; i < n_readers; ++i) {
    const qimg_q4_0_reader& r = readers[i];
    if (!r.w || !r.out || r.N <= 0 || r.ldo < r.N) return QIMG_EINVAL;
    // the mat-vec readers address a reader's code plane with 32-bit buffer offsets
    if (tiled_chunks(r.N, K, 1) * (fmt == 1 ? 2048 : 1024) > (int64_t)0xffffffff) return QIMG_EUNSUPPORTED;
    if (!al16(r.w) || !al(r.out, 4)) return QIMG_EALIGN;
    outs[i] = span(r.out, rows_extent(rows, r.ldo, r.N, 4));
    for (int j = 0; j < n_readers; ++j)
      if (overlap(outs[i], span(readers[j].w, tiled_bytes_fmt(fmt == 3 ? 0 : fmt, readers[j].N, K, 1))))
        return QIMG_EALIAS;
    if (overlap(outs[i], si) || overlap(outs[i], sl)) return QIMG_EALIAS;
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j])) return QIMG_EALIAS;
  }
  ReadArgs a{};
  int tiles = 0;
  for (int i = 0; i < n_readers; ++i) {
    const qimg_q4_0_reader& r = readers[i];
    const int64_t ch = tiled_chunks(r.N, K, 1);
    a.r[i] = ReaderDesc{(const uint8_t*)r.w,
                        (const uint16_t*)((const uint8_t*)r.w + ch * (fmt == 1 ? 2048 : 1024)),
                        r.out, r.ldo, r.N, (r.N + 15) / 16};
    a.tile_start[i] = tiles;
    tiles += (r.N + 15) / 16;
  }
  a.tile_start[n_readers] = tiles;
  fill_common(a, img, rows, K);
  a.live_rows = live_rows;
  a.n_readers = n_readers;
  a.top_k = 1;
  if (fmt == 1) return run_ordinary<3>(a, (hipStream_t)stream);
  if (fmt == 2) return run_ordinary<4>(a, (hipStream_t)stream);
  if (fmt == 3 || (fmt == 0 && rows >= kMmqMinRows)) {  // prefill: the many-row reader
    a.tiles_total = tiles;
    const dim3 grid((unsigned)((tiles + kMmqWaves - 1) / kMmqWaves), (unsigned)((rows + 63) / 64));
    hipLaunchKernelGGL(mmq_kernel, grid, dim3(kMmqWaves * 64), 0, (hipStream_t)stream, a);
    return launch_status();
  }
  return run_ordinary<0>(a, (hipStream_t)stream);
}

int mmvq_q4_0_q8_1(const qimg_q4_0_reader* readers, int32_t n_readers, const void* img,
                   int32_t rows, const int32_t* live_rows, int32_t K, void* stream) {
  return ordinary_common(0, readers, n_readers, img, rows, live_rows, K, stream);
}
int mmq_q4_0_q8_1(const qimg_q4_0_reader* readers, int32_t n_readers, const void* img,
                  int32_t rows, const int32_t* live_rows, int32_t K, void* stream) {
  return ordinary_common(3, readers, n_readers, img, rows, live_rows, K, stream);
}
int mmvq_q8_0_q8_1(const qimg_q4_0_reader* readers, int32_t n_readers, const void* img,
                   int32_t rows, const int32_t* live_rows, int32_t K, void* stream) {
  return ordinary_common(1, readers, n_readers, img, rows, live_rows, K, stream);
}
int mmvq_q4_1_q8_1(const qimg_q4_0_reader* readers, int32_t n_readers, const void* img,
                   int32_t rows, const int32_t* live_rows, int32_t K, void* stream) {
  return ordinary_common(2, readers, n_readers, img, rows, live_rows, K, stream);
}

size_t mmvq_id_workspace_bytes(int32_t bucket, int32_t top_k, int32_t E) {
  if (bucket < 0 || top_k <= 0 || E <= 0) return 0;
  const size_t words = 4 + (size_t)E + (size_t)E + 1 + (size_t)bucket * top_k;
  return (words * 4 + 255) & ~(size_t)255;
}

// per_slot = 0: the image holds one row per token (pair p reads row p / top_k);
// per_slot = 1: one row per (token, slot) pair (pair p reads row p).
static int routed_common(const qimg_q4_0_expert_reader* readers, int32_t n_readers, int32_t E,
                         const void* img, const int32_t* ids, int32_t bucket, int32_t top_k,
                         const int32_t* live_rows, int32_t K, void* workspace,
                         size_t workspace_bytes, int per_slot, void* stream) {
  int st = check_k(K);
  if (st) return st;
  if (!readers || n_readers < 1 || n_readers > QIMG_MAX_READERS || E <= 0 || bucket < 0 ||
      top_k <= 0 || !ids)
    return QIMG_EINVAL;
  if (bucket == 0) return QIMG_OK;
  if ((st = check_image(img))) return st;
  if (!workspace || workspace_bytes < mmvq_id_workspace_bytes(bucket, top_k, E))
    return QIMG_EWORKSPACE;
  if (!al16(workspace) || !al(ids, 4) || (live_rows && !al(live_rows, 4))) return QIMG_EALIGN;
  const int64_t pairs = (int64_t)bucket * top_k;
  if (pairs > QIMG_MAX_ROUTED_PAIRS || E > QIMG_MAX_EXPERTS) return QIMG_EUNSUPPORTED;
  const int32_t img_rows = per_slot ? (int32_t)pairs : bucket;
  const Span si = span(img, qimg_image_bytes(img_rows, K));
  const Span sids = span(ids, pairs * 4);
  const Span sl = live_rows ? span(live_rows, 4) : Span{0, 0};
  const Span sw = span(workspace, (int64_t)mmvq_id_workspace_bytes(bucket, top_k, E));
  if (overlap(sw, si) || overlap(sw, sids) || overlap(sw, sl)) return QIMG_EALIAS;
  Span outs[QIMG_MAX_READERS];
  for (int i = 0; i < n_readers; ++i) {
    const qimg_q4_0_expert_reader& r = readers[i];
    if (!r.w || !r.out || r.N <= 0 || r.ld_pair < r.N) return QIMG_EINVAL;
    if (!al16(r.w) || !al(r.out, 4)) return QIMG_EALIGN;
    outs[i] = span(r.out, rows_extent(pairs, r.ld_pair, r.N, 4));
    for (int j = 0; j < n_readers; ++j)
      if (overlap(outs[i], span(readers[j].w, qimg_q4_0_tiled_bytes(readers[j].N, K, E))))
        return QIMG_EALIAS;
    if (overlap(outs[i], si) || overlap(outs[i], sids) || overlap(outs[i], sl) ||
        overlap(outs[i], sw))
      return QIMG_EALIAS;
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j])) return QIMG_EALIAS;
  }
  ReadArgs a{};
  int tiles = 0;
  for (int i = 0; i < n_readers; ++i) {
    const qimg_q4_0_expert_reader& r = readers[i];
    const int64_t ch = tiled_chunks(r.N, K, E);
    a.r[i] = ReaderDesc{(const uint8_t*)r.w, (const uint16_t*)((const uint8_t*)r.w + ch * 1024),
                        r.out, r.ld_pair, r.N, (r.N + 15) / 16};
    a.tile_start[i] = tiles;
    tiles += (r.N + 15) / 16;
  }
  a.tile_start[n_readers] = tiles;
  fill_common(a, img, img_rows, K);
  a.rows = bucket;
  a.live_rows = live_rows;
  a.ids = ids;
  a.ws = (int32_t*)workspace;
  a.n_readers = n_readers;
  a.top_k = top_k;
  a.img_div = per_slot ? 1 : top_k;
  a.E = E;
  return run_routed(a, (int)pairs, (hipStream_t)stream);
}

int mmvq_id_q4_0_q8_1(const qimg_q4_0_expert_reader* readers, int32_t n_readers, int32_t E,
                      const void* img, const int32_t* ids, int32_t bucket, int32_t top_k,
                      const int32_t* live_rows, int32_t K, void* workspace,
                      size_t workspace_bytes, void* stream) {
  return routed_common(readers, n_readers, E, img, ids, bucket, top_k, live_rows, K, workspace,
                       workspace_bytes, 0, stream);
}

int mmvq_id_q4_0_q8_1_per_slot(const qimg_q4_0_expert_reader* readers, int32_t n_readers,
                               int32_t E, const void* img, const int32_t* ids, int32_t bucket,
                               int32_t top_k, const int32_t* live_rows, int32_t K,
                               void* workspace, size_t workspace_bytes, void* stream) {
  return routed_common(readers, n_readers, E, img, ids, bucket, top_k, live_rows, K, workspace,
                       workspace_bytes, 1, stream);
}

int mmvq_id_q4_0_q8_1_noalloc(const qimg_q4_0_expert_reader* readers, int32_t n_readers, int32_t E,
                              const void* img, const int32_t* ids, int32_t bucket, int32_t top_k,
                              const int32_t* live_rows, int32_t K, void* stream) {
  if (!readers || n_readers < 1 || n_readers > QIMG_MAX_READERS || E <= 0 || bucket < 0 ||
      top_k <= 0 || !ids)
    return QIMG_EINVAL;
  if (bucket == 0) return QIMG_OK;
  if ((int64_t)bucket * top_k > QIMG_MAX_ROUTED_PAIRS || E > QIMG_MAX_EXPERTS ||
      mmvq_id_workspace_bytes(bucket, top_k, E) > sizeof(scratch))
    return QIMG_EUNSUPPORTED;
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st) return st;
  return routed_common(readers, n_readers, E, img, ids, bucket, top_k, live_rows, K, ws,
                       sizeof(scratch), 0, stream);
}

// logits[t][e] = x[t] . w[e] for live rows t in the router's fixed order (the router and the
// extra f32 reader run this one kernel)
static int f32_rows_dot(const float* x, int64_t ldx, const float* w, int32_t E, int32_t bucket,
                        const int32_t* live_rows, int32_t K, float* logits, int64_t ldl, void* stream) {
  int st = check_k(K);
  if (st) return st;
  if (!x || !w || !logits || E <= 0 || bucket < 0 || ldx < K || ldl < E) return QIMG_EINVAL;
  if (bucket == 0) return QIMG_OK;
  if (!al16(x) || ldx % 4 || !al16(w) || !al(logits, 4) || (live_rows && !al(live_rows, 4)))
    return QIMG_EALIGN;
  const Span so = span(logits, rows_extent(bucket, ldl, E, 4));
  if (overlap(so, span(x, rows_extent(bucket, ldx, K, 4))) || overlap(so, span(w, (int64_t)E * K * 4)) ||
      (live_rows && overlap(so, span(live_rows, 4))))
    return QIMG_EALIAS;
  RouterArgs a{x, ldx, w, live_rows, logits, ldl, bucket, E, K};
  // the RMS producer's shape: Jp leaves per lane over W = min(16, max(1, Jp/2)) waves
  const int J = (K + 255) / 256;
  int Jp = 1;
  while (Jp < J) Jp <<= 1;
  int W = Jp / 2;
  if (W < 1) W = 1;
  if (W > 16) W = 16;
  const int JW = Jp / W;
  // experts per workgroup: 4 for buckets of many rows (each workgroup then loads its rows'
  // activations once for 4 experts) while the wave partials fit in 64 KB of LDS, else 1
  const int EB = (W <= 8 && bucket > 16) ? 4 : 1;
  // rows per workgroup: 8 (sharing each expert's weight loads), or 1 when that leaves fewer
  // than 128 workgroups (few experts or outputs: a lone row of a long dot is then one
  // workgroup's work instead of eight rows in turn). The sums are the same either way.
  const int RT = (EB == 1 && (int64_t)E * ((bucket + 7) / 8) < 128) ? 1 : 8;
  const size_t lds = (size_t)W * EB * RT * 64 * 4;
  const dim3 grid((unsigned)((E + EB - 1) / EB), (unsigned)((bucket + RT - 1) / RT)), block((unsigned)(W * 64));
  hipStream_t s = (hipStream_t)stream;
  if (EB == 4) {
    switch (JW) {
      case 1: hipLaunchKernelGGL((moe_router_kernel<1, 4, 8>), grid, block, lds, s, a); break;
      case 2: hipLaunchKernelGGL((moe_router_kernel<2, 4, 8>), grid, block, lds, s, a); break;
      default: return QIMG_EUNSUPPORTED;  // W <= 8 gives JW <= 2
    }
  } else if (RT == 8) {
    switch (JW) {
      case 1: hipLaunchKernelGGL((moe_router_kernel<1, 1, 8>), grid, block, lds, s, a); break;
      case 2: hipLaunchKernelGGL((moe_router_kernel<2, 1, 8>), grid, block, lds, s, a); break;
      case 4: hipLaunchKernelGGL((moe_router_kernel<4, 1, 8>), grid, block, lds, s, a); break;
      case 8: hipLaunchKernelGGL((moe_router_kernel<8, 1, 8>), grid, block, lds, s, a); break;
      default: return QIMG_EUNSUPPORTED;
    }
  } else {
    switch (JW) {
      case 1: hipLaunchKernelGGL((moe_router_kernel<1, 1, 1>), grid, block, lds, s, a); break;
      case 2: hipLaunchKernelGGL((moe_router_kernel<2, 1, 1>), grid, block, lds, s, a); break;
      case 4: hipLaunchKernelGGL((moe_router_kernel<4, 1, 1>), grid, block, lds, s, a); break;
      case 8: hipLaunchKernelGGL((moe_router_kernel<8, 1, 1>), grid, block, lds, s, a); break;
      default: return QIMG_EUNSUPPORTED;
    }
  }
  return launch_status();
}

int qimg_moe_router(const float* x, int64_t ldx, const float* w, int32_t E, int32_t bucket,
                    const int32_t* live_rows, int32_t K, float* logits, int64_t ldl, void* stream) {
  return f32_rows_dot(x, ldx, w, E, bucket, live_rows, K, logits, ldl, stream);
}

int qimg_f32_reader(const float* y, int64_t ldy, const float* v, int32_t N, int32_t rows,
                    const int32_t* live_rows, int32_t K, float* out, int64_t ldo, void* stream) {
  return f32_rows_dot(y, ldy, v, N, rows, live_rows, K, out, ldo, stream);
}

int qimg_moe_topk(const float* logits, int64_t ldl, int32_t E, int32_t bucket,
                  const int32_t* live_rows, int32_t top_k, int32_t* ids, float* weights,
                  void* stream) {
  if (!logits || !ids || E <= 0 || bucket < 0 || top_k <= 0 || top_k > E || ldl < E)
    return QIMG_EINVAL;
  if (E > QIMG_MAX_EXPERTS || top_k > QIMG_MAX_TOPK) return QIMG_EUNSUPPORTED;
  if (bucket == 0) return QIMG_OK;
  if (!al(logits, 4) || !al(ids, 4) || (weights && !al(weights, 4)) || (live_rows && !al(live_rows, 4)))
    return QIMG_EALIGN;
  const Span sl = span(logits, rows_extent(bucket, ldl, E, 4));
  const Span si = span(ids, (int64_t)bucket * top_k * 4);
  const Span sw = weights ? span(weights, (int64_t)bucket * top_k * 4) : Span{0, 0};
  const Span sv = live_rows ? span(live_rows, 4) : Span{0, 0};
  if (overlap(si, sl) || overlap(si, sv) || overlap(sw, sl) || overlap(sw, sv) || overlap(si, sw))
    return QIMG_EALIAS;
  TopkArgs a{logits, ldl, live_rows, ids, weights, bucket, E, top_k};
  const dim3 grid((unsigned)bucket), block(64);
  hipStream_t st = (hipStream_t)stream;
  static_assert(QIMG_MAX_EXPERTS <= 64 * 16, "top-k keys per lane");
  if (E <= 64) hipLaunchKernelGGL(moe_topk_kernel<1>, grid, block, 0, st, a);
  else if (E <= 128) hipLaunchKernelGGL(moe_topk_kernel<2>, grid, block, 0, st, a);
  else if (E <= 256) hipLaunchKernelGGL(moe_topk_kernel<4>, grid, block, 0, st, a);
  else if (E <= 512) hipLaunchKernelGGL(moe_topk_kernel<8>, grid, block, 0, st, a);
  else hipLaunchKernelGGL(moe_topk_kernel<16>, grid, block, 0, st, a);
  return launch_status();
}

int qimg_moe_combine(const float* x, int64_t ld_pair, const float* weights, const int32_t* ids,
                     int32_t E, int32_t bucket, int32_t top_k, const int32_t* live_rows,
                     int32_t N, float* out, int64_t ldo, void* stream) {
  if (bucket < 0 || top_k <= 0 || E <= 0 || N <= 0 || !x || !weights || !ids || !out ||
      ld_pair < N || ldo < N)
    return QIMG_EINVAL;
  if (bucket == 0) return QIMG_OK;
  if (N % 4) return QIMG_EUNSUPPORTED;
  if (!al16(x) || ld_pair % 4 || !al16(out) || ldo % 4 || !al(weights, 4) || !al(ids, 4) ||
      (live_rows && !al(live_rows, 4)))
    return QIMG_EALIGN;
  const int64_t pairs = (int64_t)bucket * top_k;
  const Span so = span(out, rows_extent(bucket, ldo, N, 4));
  if (overlap(so, span(x, rows_extent(pairs, ld_pair, N, 4))) || overlap(so, span(weights, pairs * 4)) ||
      overlap(so, span(ids, pairs * 4)) || (live_rows && overlap(so, span(live_rows, 4))))
    return QIMG_EALIAS;
  CombineArgs c{x, ld_pair, weights, ids, live_rows, out, ldo, bucket, top_k, E, N};
  const dim3 grid((unsigned)((N / 4 + 255) / 256), (unsigned)bucket);
  hipLaunchKernelGGL(moe_combine_kernel, grid, dim3(256), 0, (hipStream_t)stream, c);
  return launch_status();
}

int mmvq_q4_0_q8_1_blockdots(const qimg_q4_0_reader* reader, const void* img, int32_t rows,
                             int32_t K, int32_t* sumi, void* stream) {
  int st = check_k(K);
  if (st) return st;
  if (!reader || !sumi || rows < 0 || !reader->w || reader->N <= 0) return QIMG_EINVAL;
  if (rows == 0) return QIMG_OK;
  if ((st = check_image(img))) return st;
  if (!al16(reader->w) || !al(sumi, 4)) return QIMG_EALIGN;
  const int Kb = K / 32;
  const Span ss = span(sumi, (int64_t)rows * reader->N * Kb * 4);
  if (overlap(ss, span(img, qimg_image_bytes(rows, K))) ||
      overlap(ss, span(reader->w, qimg_q4_0_tiled_bytes(reader->N, K, 1))))
    return QIMG_EALIAS;
  ReadArgs a{};
  const int64_t ch = tiled_chunks(reader->N, K, 1);
  a.r[0] = ReaderDesc{(const uint8_t*)reader->w, (const uint16_t*)((const uint8_t*)reader->w + ch * 1024),
                      nullptr, 0, reader->N, (reader->N + 15) / 16};
  a.tile_start[0] = 0;
  a.tile_start[1] = (reader->N + 15) / 16;
  fill_common(a, img, rows, K);
  a.sumi = sumi;
  a.n_readers = 1;
  a.top_k = 1;
  return run_ordinary<2>(a, (hipStream_t)stream);
}

int qimg_eval_math(int32_t fn, uint32_t first_bits, int64_t n, float* out, void* stream) {
  if (fn < MATH_EXP || fn > MATH_OAI_GATE || n < 0 || n > ((int64_t)1 << 32)) return QIMG_EINVAL;
  if (n == 0) return QIMG_OK;
  if (!out) return QIMG_EINVAL;
  if (!al(out, 4)) return QIMG_EALIGN;
  const int64_t wgs = (n + 255) / 256;
  const dim3 grid((unsigned)(wgs < 8192 ? wgs : 8192));
  hipStream_t s = (hipStream_t)stream;
  switch (fn) {
    case MATH_EXP: eval_math_kernel<MATH_EXP><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    case MATH_ERFC: eval_math_kernel<MATH_ERFC><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    case MATH_SWIGLU: eval_math_kernel<MATH_SWIGLU><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    case MATH_GEGLU: eval_math_kernel<MATH_GEGLU><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    case MATH_RSQRT: eval_math_kernel<MATH_RSQRT><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    case MATH_QSCALE: eval_math_kernel<MATH_QSCALE><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    case MATH_QDIV: eval_math_kernel<MATH_QDIV><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    case MATH_F2H: eval_math_kernel<MATH_F2H><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    case MATH_REGLU: eval_math_kernel<MATH_REGLU><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    case MATH_GEGLU_TANH: eval_math_kernel<MATH_GEGLU_TANH><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    case MATH_GEGLU_QUICK: eval_math_kernel<MATH_GEGLU_QUICK><<<grid, 256, 0, s>>>(first_bits, n, out); break;
    default: eval_math_kernel<MATH_OAI_GATE><<<grid, 256, 0, s>>>(first_bits, n, out); break;
  }
  return launch_status();
}

int qimg_read_ceiling(const void* buf, int64_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 1024 || bytes >= ((int64_t)1 << 31)) return QIMG_EINVAL;
  if (!al16(buf) || !al(sink, 4)) return QIMG_EALIGN;
  if (overlap(span(buf, bytes), span(sink, QIMG_CEILING_SINK_WORDS * 4))) return QIMG_EALIAS;
  hipLaunchKernelGGL(read_ceiling_kernel, dim3(kCeilGrid), dim3(kCeilWaves * 64), 0, (hipStream_t)stream,
                     (const uint8_t*)buf, (uint32_t)(bytes / 1024), sink);
  return launch_status();
}

}  // extern "C"
