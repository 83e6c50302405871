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
//   emit_kernel<OP,JW>   one workgroup per live row: (RMS reduction) -> f32 output -> per
//                        32-block Q8_1 quantization, all in one pass over the row.
//   mmvq_kernel<LPR,NWM> Q4_0 x Q8_1 readers. A lane owns one 32-weight block column of the
//                        K axis and keeps that block of every image column it serves in VGPRs;
//                        the workgroup then streams weight rows (16-byte block loads, adjacent
//                        lanes on adjacent blocks) and reduces per-lane block terms with a
//                        transpose-butterfly and a fixed cross-wave sum. Ordinary readers take
//                        the live image rows as columns; routed readers take the live pairs of
//                        one expert, found by a stable scan of the ids in the same launch.
//   blockdots_kernel     debug export of the per-block integer dots (same device dot code).
//
// Build: hipcc --offload-arch=gfx950 -O3 -ffp-contract=off (no fast-math), so every float
// operation written here is one IEEE binary32 operation with round-to-nearest-even; f32
// division and square root are the correctly rounded ones.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>
#include <string.h>

#include "qimg.h"

namespace {

// ---------------------------------------------------------------------------------------------
// small device helpers
// ---------------------------------------------------------------------------------------------
__device__ __forceinline__ float h2f(uint32_t h) {
  return __half2float(__ushort_as_half((unsigned short)(h & 0xffffu)));
}
__device__ __forceinline__ uint32_t f2h(float f) {  // round-to-nearest-even, subnormals kept
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

// Q4_0 block: 16 bytes, byte j = element j (low nibble) | element j+16 (high nibble).
// Activation block: 32 int8 codes as 8 dwords (elements 0..15 in a[0..3], 16..31 in a[4..7]).
// sumi = sum_j lo_j * c_j + hi_j * c_{j+16}, with v_dot4 (signed; nibbles are 0..15).
__device__ __forceinline__ void unpack_q4(const uint4 q, uint32_t (&lo)[4], uint32_t (&hi)[4]) {
  lo[0] = q.x & 0x0f0f0f0fu; hi[0] = (q.x >> 4) & 0x0f0f0f0fu;
  lo[1] = q.y & 0x0f0f0f0fu; hi[1] = (q.y >> 4) & 0x0f0f0f0fu;
  lo[2] = q.z & 0x0f0f0f0fu; hi[2] = (q.z >> 4) & 0x0f0f0f0fu;
  lo[3] = q.w & 0x0f0f0f0fu; hi[3] = (q.w >> 4) & 0x0f0f0f0fu;
}
__device__ __forceinline__ int block_sumi(const uint32_t (&lo)[4], const uint32_t (&hi)[4],
                                          const int32_t* a) {
  int s = 0;
  s = __builtin_amdgcn_sdot4((int)lo[0], a[0], s, false);
  s = __builtin_amdgcn_sdot4((int)lo[1], a[1], s, false);
  s = __builtin_amdgcn_sdot4((int)lo[2], a[2], s, false);
  s = __builtin_amdgcn_sdot4((int)lo[3], a[3], s, false);
  s = __builtin_amdgcn_sdot4((int)hi[0], a[4], s, false);
  s = __builtin_amdgcn_sdot4((int)hi[1], a[5], s, false);
  s = __builtin_amdgcn_sdot4((int)hi[2], a[6], s, false);
  s = __builtin_amdgcn_sdot4((int)hi[3], a[7], s, false);
  return s;
}

// ---------------------------------------------------------------------------------------------
// Producer: one workgroup per live row.
// Element mapping: leaf c covers elements 4c..4c+3; lane l of wave w holds leaves
// c = l + 64 j for j in [w*JW, (w+1)*JW). A 32-element block is 8 consecutive leaves, i.e. 8
// consecutive lanes at the same j, so the block amax and code sum are 3-step lane reductions.
// RMS sum of squares (the fixed order, independent of the wave count): leaf value
// fma(x3,x3, fma(x2,x2, fma(x1,x1, x0*x0))); per lane a balanced pairwise tree over j (padded
// to a power of two Jp with zeros), whose top levels are taken across waves through LDS; then
// a balanced pairwise tree over the 64 lanes (xor butterfly, masks 1..32).
// ---------------------------------------------------------------------------------------------
enum : int { OP_RMS = 0, OP_SWIGLU = 1, OP_GEGLU = 2, OP_QUANT = 3 };

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
  float eps;
};

template <int JW>
__device__ __forceinline__ float tree_sum(float (&v)[JW]) {
#pragma unroll
  for (int w = JW; w > 1; w >>= 1) {
#pragma unroll
    for (int i = 0; i < w / 2; ++i) v[i] = v[2 * i] + v[2 * i + 1];
  }
  return v[0];
}

__device__ __forceinline__ void quantize_leaf(const float4 y, int row, int blk, int lane,
                                              const EmitArgs& p) {
  float amax = fmaxf(fmaxf(fabsf(y.x), fabsf(y.y)), fmaxf(fabsf(y.z), fabsf(y.w)));
  amax = fmaxf(amax, __shfl_xor(amax, 1, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 2, 64));
  amax = fmaxf(amax, __shfl_xor(amax, 4, 64));
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
  sum += __shfl_xor(sum, 1, 64);
  sum += __shfl_xor(sum, 2, 64);
  sum += __shfl_xor(sum, 4, 64);
  if (!zero) dsw = f2h(d) | (f2h((float)sum * d) << 16);
  const int64_t blk_idx = (int64_t)row * p.RB + blk;
  reinterpret_cast<uint32_t*>(p.codes)[blk_idx * 8 + (lane & 7)] = packed;
  if ((lane & 7) == 0) p.ds[blk_idx] = dsw;
}

template <int OP, int JW>
__global__ __launch_bounds__(1024) void emit_kernel(EmitArgs p) {
  const int row = blockIdx.x;
  if (row >= clamp_live(p.live_rows, p.rows, nullptr)) return;  // padding rows: untouched
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int W = blockDim.x >> 6;
  const int C = p.K >> 2;
  const float* arow = p.a + (int64_t)row * p.lda;

  float4 v[JW];
#pragma unroll
  for (int jj = 0; jj < JW; ++jj) {
    const int c = lane + 64 * (w * JW + jj);
    v[jj] = c < C ? *reinterpret_cast<const float4*>(arow + 4 * c) : make_float4(0, 0, 0, 0);
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
    float S = t[0];
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) S = S + __shfl_xor(S, m, 64);
    const float mean = S / (float)p.K;
    const float r = 1.0f / __builtin_sqrtf(mean + p.eps);
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int c = lane + 64 * (w * JW + jj);
      float4 y;
      y.x = v[jj].x * r; y.y = v[jj].y * r; y.z = v[jj].z * r; y.w = v[jj].w * r;
      if (p.b && c < C) {
        const float4 g = *reinterpret_cast<const float4*>(p.b + 4 * c);
        y.x = y.x * g.x; y.y = y.y * g.y; y.z = y.z * g.z; y.w = y.w * g.w;
      }
      v[jj] = y;
    }
  } else if constexpr (OP == OP_SWIGLU || OP == OP_GEGLU) {
    const float* brow = p.b + (int64_t)row * p.ldb;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int c = lane + 64 * (w * JW + jj);
      if (c < C) {
        const float4 u = *reinterpret_cast<const float4*>(brow + 4 * c);
        float4 y;
        if constexpr (OP == OP_SWIGLU) {
          y.x = swiglu_act(v[jj].x) * u.x; y.y = swiglu_act(v[jj].y) * u.y;
          y.z = swiglu_act(v[jj].z) * u.z; y.w = swiglu_act(v[jj].w) * u.w;
        } else {
          y.x = geglu_erf_act(v[jj].x) * u.x; y.y = geglu_erf_act(v[jj].y) * u.y;
          y.z = geglu_erf_act(v[jj].z) * u.z; y.w = geglu_erf_act(v[jj].w) * u.w;
        }
        v[jj] = y;
      }
    }
  }

  // every original F32 store remains ([P1] Coverage)
  if constexpr (OP != OP_QUANT) {
    float* yrow = p.y + (int64_t)row * p.ldy;
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int c = lane + 64 * (w * JW + jj);
      if (c < C) *reinterpret_cast<float4*>(yrow + 4 * c) = v[jj];
    }
  }

  if (p.codes) {
#pragma unroll
    for (int jj = 0; jj < JW; ++jj) {
      const int blk = 8 * (w * JW + jj) + (lane >> 3);
      if (blk < p.Kb) quantize_leaf(v[jj], row, blk, lane, p);  // whole 8-lane groups agree
    }
    // row padding blocks [Kb, RB) are zero bytes
    const int npad = p.RB - p.Kb;
    uint32_t* cw = reinterpret_cast<uint32_t*>(p.codes) + ((int64_t)row * p.RB + p.Kb) * 8;
    for (int i = threadIdx.x; i < npad * 9; i += blockDim.x) {
      if (i < npad * 8) cw[i] = 0u;
      else p.ds[(int64_t)row * p.RB + p.Kb + (i - npad * 8)] = 0u;
    }
  }
}

// ---------------------------------------------------------------------------------------------
// Readers
// ---------------------------------------------------------------------------------------------
struct ReaderDesc {
  const uint8_t* qs;
  const uint16_t* d;
  float* out;
  int64_t ld;   // ordinary: ldo per image row; routed: ld_pair per pair
  int32_t N;
  int32_t pad;
};

struct MmvqArgs {
  ReaderDesc r[QIMG_MAX_READERS];
  int32_t tile_start[QIMG_MAX_READERS + 1];  // tile prefix over readers (per expert if routed)
  const uint8_t* codes;
  const uint32_t* ds;
  const int32_t* live_rows;
  const int32_t* ids;   // routed only
  int32_t* ws;          // routed only: plan workspace
  int32_t n_readers, RB, Kb, rows, TR, top_k, E, routed;
};

// Transpose-butterfly over LPR lanes of V values per lane. At the level of mask M a lane
// keeps the half of its values selected by its lane bit M and adds the partner's copy of that
// half, so after log2(LPR) levels lane bl of the segment holds the complete sums of values
// [bl*V/LPR, (bl+1)*V/LPR) (V >= LPR), or of value bl/(LPR/V) (V < LPR; the remaining levels
// are plain butterflies). Every value is summed over the lanes by the same tree.
template <int M, int N>
__device__ __forceinline__ void tbfly(float* v, int lane) {
  if constexpr (M > 0) {
    if constexpr (N > 1) {
      constexpr int H = N / 2;
      const bool up = (lane & M) != 0;
#pragma unroll
      for (int i = 0; i < H; ++i) {
        const float send = up ? v[i] : v[i + H];
        const float keep = up ? v[i + H] : v[i];
        v[i] = keep + __shfl_xor(send, M, 64);
      }
      tbfly<M / 2, H>(v, lane);
    } else {
      v[0] = v[0] + __shfl_xor(v[0], M, 64);
      tbfly<M / 2, 1>(v, lane);
    }
  }
}

constexpr int kGroup = 4;  // weight rows per lane between two reductions

// One pass of a row tile against up to CT image columns cols[c0 .. c0+ncols).
// red: LDS [NW][TR*CT]. Writes the finished outputs.
template <int LPR, int CT>
__device__ __forceinline__ void reader_pass(const MmvqArgs& p, const ReaderDesc& R,
                                            const uint8_t* __restrict__ qs,
                                            const uint16_t* __restrict__ dw_plane, int n0,
                                            int n_end, const int32_t* cols, int c0, int ncols,
                                            float* red) {
  constexpr int RPW = 64 / LPR;
  constexpr int V = kGroup * CT;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int NW = blockDim.x >> 6;
  const int r = lane / LPR;
  const int bl = lane % LPR;
  const int blk = w * LPR + bl;
  const bool act = blk < p.Kb;
  const int Kb = p.Kb;

  // this lane's activation block for each column, kept in VGPRs for the whole tile
  int32_t a[CT][8];
  float da[CT], ms[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[c][i] = 0;
    da[c] = 0.0f;
    ms[c] = 0.0f;
    if (act && c < ncols) {
      const int col = cols[c0 + c];
      const int irow = p.routed ? col / p.top_k : col;
      const int64_t bi = (int64_t)irow * p.RB + blk;
      const int4 lo = reinterpret_cast<const int4*>(p.codes)[bi * 2];
      const int4 hi = reinterpret_cast<const int4*>(p.codes)[bi * 2 + 1];
      a[c][0] = lo.x; a[c][1] = lo.y; a[c][2] = lo.z; a[c][3] = lo.w;
      a[c][4] = hi.x; a[c][5] = hi.y; a[c][6] = hi.z; a[c][7] = hi.w;
      const uint32_t dsw = p.ds[bi];
      da[c] = h2f(dsw);
      ms[c] = -8.0f * h2f(dsw >> 16);
    }
  }

  const int nrows = n_end - n0;
  for (int g0 = 0; g0 < nrows; g0 += kGroup * RPW) {
    float acc[V];
#pragma unroll
    for (int s = 0; s < kGroup; ++s) {
      const int n = n0 + g0 + s * RPW + r;
      uint4 q = make_uint4(0, 0, 0, 0);
      float dwf = 0.0f;
      if (act && n < n_end) {
        const int64_t wi = (int64_t)n * Kb + blk;
        q = reinterpret_cast<const uint4*>(qs)[wi];
        dwf = h2f(dw_plane[wi]);
      }
      uint32_t lo[4], hi[4];
      unpack_q4(q, lo, hi);
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        const int si = block_sumi(lo, hi, a[c]);
        const float x = __builtin_fmaf(da[c], (float)si, ms[c]);  // d_a*sumi - 8*s_a
        acc[s * CT + c] = dwf * x;
      }
    }
    tbfly<LPR / 2, V>(acc, lane);
    // scatter this lane's finished values into the per-wave LDS slots
    float* rw = red + (int64_t)w * (p.TR * CT);
    if constexpr (V >= LPR) {
      constexpr int PER = V / LPR;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const int vi = bl * PER + i;
        const int s = vi / CT, c = vi % CT;
        rw[(g0 + s * RPW + r) * CT + c] = acc[i];
      }
    } else {
      constexpr int DUP = LPR / V;
      if (bl % DUP == 0) {
        const int vi = bl / DUP;
        const int s = vi / CT, c = vi % CT;
        rw[(g0 + s * RPW + r) * CT + c] = acc[0];
      }
    }
  }
  __syncthreads();
  // fixed cross-wave order: ascending wave index
  for (int o = threadIdx.x; o < nrows * CT; o += blockDim.x) {
    const int c = o % CT;
    if (c >= ncols) continue;
    float t = red[o];
    for (int ww = 1; ww < NW; ++ww) t = t + red[(int64_t)ww * (p.TR * CT) + o];
    const int n = n0 + o / CT;
    const int col = cols[c0 + c];
    R.out[(int64_t)col * R.ld + n] = t;
  }
  __syncthreads();
}

template <int LPR>
__device__ __forceinline__ void reader_columns(const MmvqArgs& p, const ReaderDesc& R,
                                               const uint8_t* qs, const uint16_t* dwp, int n0,
                                               int n_end, const int32_t* cols, int ncols,
                                               float* red) {
  for (int c0 = 0; c0 < ncols; c0 += 8) {
    const int ct = ncols - c0 < 8 ? ncols - c0 : 8;
    if (ct > 4) reader_pass<LPR, 8>(p, R, qs, dwp, n0, n_end, cols, c0, ct, red);
    else if (ct > 2) reader_pass<LPR, 4>(p, R, qs, dwp, n0, n_end, cols, c0, ct, red);
    else if (ct > 1) reader_pass<LPR, 2>(p, R, qs, dwp, n0, n_end, cols, c0, ct, red);
    else reader_pass<LPR, 1>(p, R, qs, dwp, n0, n_end, cols, c0, ct, red);
  }
}

// Dynamic LDS: int32 cols[max_cols] then float red[NW][TR*8].
template <int LPR, int NWM>
__global__ __launch_bounds__(NWM * 64) void mmvq_kernel(MmvqArgs p, int max_cols) {
  extern __shared__ __align__(16) unsigned char smem[];
  int32_t* cols = reinterpret_cast<int32_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + ((max_cols * 4 + 15) & ~15));
  __shared__ int wave_cnt[16];
  __shared__ int red_i[4];

  int clamped = 0;
  const int live = clamp_live(p.live_rows, p.rows, &clamped);
  const int tiles = p.tile_start[p.n_readers];
  const int unit = blockIdx.x / tiles;  // expert (routed) or 0
  const int tile = blockIdx.x % tiles;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, NW = blockDim.x >> 6;

  int ncols;
  if (!p.routed) {
    ncols = live;
    for (int i = threadIdx.x; i < live; i += blockDim.x) cols[i] = i;
    __syncthreads();
  } else {
    // Stable scan of the live pairs for this expert ([P3] What this changes: only the first
    // live rows' pairs are planned; padding rows' ids are never read).
    const int e = unit;
    const int P = live * p.top_k;
    if (threadIdx.x < 4) red_i[threadIdx.x] = 0;
    __syncthreads();
    int n_lt = 0, n_valid = 0, n_bad = 0, base = 0;
    for (int p0 = 0; p0 < P; p0 += blockDim.x) {
      const int pi = p0 + threadIdx.x;
      const int id = pi < P ? p.ids[pi] : -1;
      const bool valid = pi < P && id >= 0 && id < p.E;
      n_bad += (pi < P && !valid) ? 1 : 0;
      n_valid += valid ? 1 : 0;
      n_lt += (valid && id < e) ? 1 : 0;
      const bool match = valid && id == e;
      const unsigned long long bal = __ballot(match);
      const int rank = __popcll(bal & ((1ull << lane) - 1ull));
      if (lane == 0) wave_cnt[w] = __popcll(bal);
      __syncthreads();
      int pre = 0, tot = 0;
      for (int i = 0; i < NW; ++i) {
        pre += i < w ? wave_cnt[i] : 0;
        tot += wave_cnt[i];
      }
      if (match) cols[base + pre + rank] = pi;
      base += tot;
      __syncthreads();
    }
    ncols = base;
    if (tile == 0) {
      atomicAdd(&red_i[0], n_lt);
      atomicAdd(&red_i[1], n_valid);
      atomicAdd(&red_i[2], n_bad);
      __syncthreads();
      const int off = red_i[0];
      int32_t* counts = p.ws + 4;
      int32_t* offsets = counts + p.E;
      int32_t* members = offsets + p.E + 1;
      if (threadIdx.x == 0) {
        counts[e] = ncols;
        offsets[e] = off;
      }
      for (int i = threadIdx.x; i < ncols; i += blockDim.x) members[off + i] = cols[i];
      if (e == 0 && threadIdx.x == 0) {
        p.ws[0] = (red_i[2] ? QIMG_ERR_EXPERT_RANGE : 0) | (clamped ? QIMG_ERR_LIVE_CLAMPED : 0);
        p.ws[1] = P;
        p.ws[2] = 0;
        p.ws[3] = 0;
        offsets[p.E] = red_i[1];
      }
    }
  }
  if (ncols == 0) return;

  int ri = 0;
  while (ri + 1 < p.n_readers && tile >= p.tile_start[ri + 1]) ++ri;
  const ReaderDesc& R = p.r[ri];
  const int n0 = (tile - p.tile_start[ri]) * p.TR;
  const int n_end = n0 + p.TR < R.N ? n0 + p.TR : R.N;
  const int64_t eoff = (int64_t)unit * R.N * p.Kb;  // expert offset in blocks (0 if ordinary)
  reader_columns<LPR>(p, R, R.qs + eoff * 16, R.d + eoff, n0, n_end, cols, ncols, red);
}

__global__ void blockdots_kernel(const uint8_t* __restrict__ qs, int N, int Kb,
                                 const uint8_t* __restrict__ codes, int RB, int rows,
                                 int32_t* __restrict__ sumi) {
  const int64_t total = (int64_t)rows * N * Kb;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = i / ((int64_t)N * Kb);
    const int64_t rem = i % ((int64_t)N * Kb);
    const int64_t n = rem / Kb, b = rem % Kb;
    const uint4 q = reinterpret_cast<const uint4*>(qs)[n * Kb + b];
    const int4* ab = reinterpret_cast<const int4*>(codes) + (t * RB + b) * 2;
    const int4 lo = ab[0], hi = ab[1];
    const int32_t a[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    uint32_t l4[4], h4[4];
    unpack_q4(q, l4, h4);
    sumi[i] = block_sumi(l4, h4, a);
  }
}

// ---------------------------------------------------------------------------------------------
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
// W = min(16, max(1, Jp/2)) waves, JW = Jp / W slots per lane.
int launch_emit(int op, EmitArgs& a, hipStream_t s) {
  const int J = (a.K + 255) / 256;
  int Jp = 1;
  while (Jp < J) Jp <<= 1;
  int W = Jp / 2;
  if (W < 1) W = 1;
  if (W > 16) W = 16;
  const int JW = Jp / W;
  dim3 grid(a.rows), block(W * 64);
#define QIMG_EMIT_CASE(OPV, JWV) \
  if (op == OPV && JW == JWV) { hipLaunchKernelGGL((emit_kernel<OPV, JWV>), grid, block, 0, s, a); return launch_status(); }
#define QIMG_EMIT_OP(OPV) QIMG_EMIT_CASE(OPV, 1) QIMG_EMIT_CASE(OPV, 2) QIMG_EMIT_CASE(OPV, 4) QIMG_EMIT_CASE(OPV, 8)
  QIMG_EMIT_OP(OP_RMS)
  QIMG_EMIT_OP(OP_SWIGLU)
  QIMG_EMIT_OP(OP_GEGLU)
  QIMG_EMIT_OP(OP_QUANT)
#undef QIMG_EMIT_OP
#undef QIMG_EMIT_CASE
  return QIMG_EUNSUPPORTED;
}

struct ReaderShape {
  int LPR, NW, TR;
};

// Lanes per row segment: the candidate in {64, 32, 16} that leaves the fewest idle lanes on
// the K axis (ties go to the wider segment); NW = waves covering K.
ReaderShape reader_shape(int Kb, int64_t rows_per_unit, int64_t units) {
  ReaderShape s{64, 0, 0};
  int best = 1 << 30;
  for (int lpr : {64, 32, 16}) {
    const int nw = (Kb + lpr - 1) / lpr;
    const int waste = nw * lpr - Kb;
    if (nw <= 16 && waste < best) {
      best = waste;
      s.LPR = lpr;
      s.NW = nw;
    }
  }
  const int grp = kGroup * (64 / s.LPR);
  // rows per workgroup tile: aim at ~1024 busy workgroups for ordinary readers, ~16 tiles per
  // expert for routed ones; a multiple of the reduction group, at most 64 rows.
  int64_t want = units > 1 ? rows_per_unit / 16 : rows_per_unit / 1024;
  int tr = grp;
  while (tr * 2 <= want && tr * 2 <= 64) tr *= 2;
  s.TR = tr;
  return s;
}

int launch_mmvq(MmvqArgs& a, int units, int max_cols, hipStream_t s, const ReaderShape& sh) {
  const size_t lds = (size_t)((max_cols * 4 + 15) & ~15) + (size_t)sh.NW * sh.TR * 8 * 4;
  if (lds > 64 * 1024) return QIMG_EUNSUPPORTED;
  const int tiles = a.tile_start[a.n_readers];
  dim3 grid((unsigned)((int64_t)tiles * units)), block(sh.NW * 64);
#define QIMG_MMVQ_CASE(L, NWM)                                                                \
  if (sh.LPR == L && sh.NW <= NWM) {                                                          \
    hipLaunchKernelGGL((mmvq_kernel<L, NWM>), grid, block, lds, s, a, max_cols);              \
    return launch_status();                                                                   \
  }
  QIMG_MMVQ_CASE(64, 8) QIMG_MMVQ_CASE(64, 16)
  QIMG_MMVQ_CASE(32, 8) QIMG_MMVQ_CASE(32, 16)
  QIMG_MMVQ_CASE(16, 8) QIMG_MMVQ_CASE(16, 16)
#undef QIMG_MMVQ_CASE
  return QIMG_EUNSUPPORTED;
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

static int emit_common(int op, const float* a, int64_t lda, const float* b, int64_t ldb,
                       int b_rows, float eps, int32_t rows, const int32_t* live_rows, int32_t K,
                       float* y, int64_t ldy, void* img, void* stream) {
  int st = check_k(K);
  if (st) return st;
  if (rows < 0) return QIMG_EINVAL;
  if (rows == 0) return QIMG_OK;
  if (!a || (op != OP_QUANT && !y) || (op == OP_QUANT && !img)) return QIMG_EINVAL;
  if ((op == OP_SWIGLU || op == OP_GEGLU) && !b) return QIMG_EINVAL;
  if (lda < K || (op != OP_QUANT && ldy < K) || (b && b_rows > 1 && ldb < K)) return QIMG_EINVAL;
  if (!al16(a) || lda % 4 || (b && (!al16(b) || (b_rows > 1 && ldb % 4))) ||
      (y && (!al16(y) || ldy % 4)) || (img && !al16(img)) || (live_rows && !al(live_rows, 4)))
    return QIMG_EALIGN;
  const int64_t ib = qimg_image_bytes(rows, K);
  const Span sa = span(a, rows_extent(rows, lda, K, 4));
  const Span sb = b ? span(b, b_rows > 1 ? rows_extent(rows, ldb, K, 4) : (int64_t)K * 4) : Span{0, 0};
  const Span sy = y ? span(y, rows_extent(rows, ldy, K, 4)) : Span{0, 0};
  const Span si = img ? span(img, ib) : Span{0, 0};
  const Span sl = live_rows ? span(live_rows, 4) : Span{0, 0};
  for (Span out : {sy, si}) {
    if (overlap(out, sa) || overlap(out, sb) || overlap(out, sl)) return QIMG_EALIAS;
  }
  if (overlap(sy, si)) return QIMG_EALIAS;

  EmitArgs e{};
  e.a = a; e.lda = lda; e.b = b; e.ldb = ldb; e.y = y; e.ldy = ldy;
  const int RB = row_blocks(K);
  e.codes = (uint8_t*)img;
  e.ds = img ? (uint32_t*)((uint8_t*)img + (size_t)rows * RB * 32) : nullptr;
  e.live_rows = live_rows; e.rows = rows; e.K = K; e.Kb = K / 32; e.RB = RB; e.eps = eps;
  return launch_emit(op, e, (hipStream_t)stream);
}

int qimg_emit_rmsnorm(const float* x, int64_t ldx, const float* gamma, float eps, int32_t rows,
                      const int32_t* live_rows, int32_t K, float* y, int64_t ldy, void* img,
                      void* stream) {
  return emit_common(OP_RMS, x, ldx, gamma, 0, 1, eps, rows, live_rows, K, y, ldy, img, stream);
}

int qimg_emit_glu(int32_t op, const float* gate, int64_t ldg, const float* up, int64_t ldu,
                  int32_t rows, const int32_t* live_rows, int32_t K, float* y, int64_t ldy,
                  void* img, void* stream) {
  if (op != QIMG_GLU_SWIGLU && op != QIMG_GLU_GEGLU_ERF) return QIMG_EINVAL;
  const int kop = op == QIMG_GLU_SWIGLU ? OP_SWIGLU : OP_GEGLU;
  // gate and up may be the two halves of one packed row (they must not overlap each other's
  // elements, which packed halves do not)
  return emit_common(kop, gate, ldg, up, ldu, 2, 0.0f, rows, live_rows, K, y, ldy, img, stream);
}

int qimg_quantize_q8_1(const float* y, int64_t ldy, int32_t rows, const int32_t* live_rows,
                       int32_t K, void* img, void* stream) {
  return emit_common(OP_QUANT, y, ldy, nullptr, 0, 0, 0.0f, rows, live_rows, K, nullptr, 0, img,
                     stream);
}

static int check_image(const void* img, int32_t rows, int32_t K) {
  if (!img) return QIMG_EINVAL;
  if (!al16(img)) return QIMG_EALIGN;
  (void)rows; (void)K;
  return QIMG_OK;
}

int mmvq_q4_0_q8_1(const qimg_q4_0_reader* readers, int32_t n_readers, const void* img,
                   int32_t rows, const int32_t* live_rows, int32_t K, void* stream) {
  int st = check_k(K);
  if (st) return st;
  if (!readers || n_readers < 1 || n_readers > QIMG_MAX_READERS || rows < 0) return QIMG_EINVAL;
  if (rows == 0) return QIMG_OK;
  if ((st = check_image(img, rows, K))) return st;
  if (live_rows && !al(live_rows, 4)) return QIMG_EALIGN;
  const int Kb = K / 32;
  const Span si = span(img, qimg_image_bytes(rows, K));
  const Span sl = live_rows ? span(live_rows, 4) : Span{0, 0};
  Span outs[QIMG_MAX_READERS];
  int64_t total_rows = 0;
  for (int i = 0; i < n_readers; ++i) {
    const qimg_q4_0_reader& r = readers[i];
    if (!r.qs || !r.d || !r.out || r.N <= 0 || r.ldo < r.N) return QIMG_EINVAL;
    if (!al16(r.qs) || !al(r.d, 4) || !al(r.out, 4)) return QIMG_EALIGN;
    outs[i] = span(r.out, rows_extent(rows, r.ldo, r.N, 4));
    const Span sq = span(r.qs, (int64_t)r.N * Kb * 16), sd = span(r.d, (int64_t)r.N * Kb * 2);
    total_rows += r.N;
    for (int j = 0; j < n_readers; ++j) {
      const Span oq = span(readers[j].qs, (int64_t)readers[j].N * Kb * 16);
      const Span od = span(readers[j].d, (int64_t)readers[j].N * Kb * 2);
      if (overlap(outs[i], oq) || overlap(outs[i], od)) return QIMG_EALIAS;
    }
    if (overlap(outs[i], si) || overlap(outs[i], sl) || overlap(outs[i], sq) || overlap(outs[i], sd))
      return QIMG_EALIAS;
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j])) return QIMG_EALIAS;
  }
  const ReaderShape sh = reader_shape(Kb, total_rows, 1);
  MmvqArgs a{};
  int tiles = 0;
  for (int i = 0; i < n_readers; ++i) {
    const qimg_q4_0_reader& r = readers[i];
    a.r[i] = ReaderDesc{(const uint8_t*)r.qs, (const uint16_t*)r.d, r.out, r.ldo, r.N, 0};
    a.tile_start[i] = tiles;
    tiles += (r.N + sh.TR - 1) / sh.TR;
  }
  a.tile_start[n_readers] = tiles;
  const int RB = row_blocks(K);
  a.codes = (const uint8_t*)img;
  a.ds = (const uint32_t*)((const uint8_t*)img + (size_t)rows * RB * 32);
  a.live_rows = live_rows;
  a.n_readers = n_readers; a.RB = RB; a.Kb = Kb; a.rows = rows; a.TR = sh.TR;
  a.top_k = 1; a.E = 0; a.routed = 0; a.ids = nullptr; a.ws = nullptr;
  return launch_mmvq(a, 1, rows, (hipStream_t)stream, sh);
}

size_t mmvq_id_workspace_bytes(int32_t bucket, int32_t top_k, int32_t E) {
  if (bucket < 0 || top_k <= 0 || E <= 0) return 0;
  const size_t words = 4 + (size_t)E + (size_t)E + 1 + (size_t)bucket * top_k;
  return (words * 4 + 255) & ~(size_t)255;
}

int mmvq_id_q4_0_q8_1(const qimg_q4_0_expert_reader* readers, int32_t n_readers, int32_t E,
                      const void* img, const int32_t* ids, int32_t bucket, int32_t top_k,
                      const int32_t* live_rows, int32_t K, void* workspace,
                      size_t workspace_bytes, void* stream) {
  int st = check_k(K);
  if (st) return st;
  if (!readers || n_readers < 1 || n_readers > QIMG_MAX_READERS || E <= 0 || bucket < 0 ||
      top_k <= 0 || !ids)
    return QIMG_EINVAL;
  if (bucket == 0) return QIMG_OK;
  if ((st = check_image(img, bucket, K))) return st;
  if (!workspace || workspace_bytes < mmvq_id_workspace_bytes(bucket, top_k, E))
    return QIMG_EWORKSPACE;
  if (!al16(workspace) || !al(ids, 4) || (live_rows && !al(live_rows, 4))) return QIMG_EALIGN;
  const int Kb = K / 32;
  const int64_t pairs = (int64_t)bucket * top_k;
  const Span si = span(img, qimg_image_bytes(bucket, K));
  const Span sids = span(ids, pairs * 4);
  const Span sl = live_rows ? span(live_rows, 4) : Span{0, 0};
  const Span sw = span(workspace, (int64_t)mmvq_id_workspace_bytes(bucket, top_k, E));
  if (overlap(sw, si) || overlap(sw, sids) || overlap(sw, sl)) return QIMG_EALIAS;
  Span outs[QIMG_MAX_READERS];
  int maxN = 0;
  for (int i = 0; i < n_readers; ++i) {
    const qimg_q4_0_expert_reader& r = readers[i];
    if (!r.qs || !r.d || !r.out || r.N <= 0 || r.ld_pair < r.N) return QIMG_EINVAL;
    if (!al16(r.qs) || !al(r.d, 4) || !al(r.out, 4)) return QIMG_EALIGN;
    outs[i] = span(r.out, rows_extent(pairs, r.ld_pair, r.N, 4));
    for (int j = 0; j < n_readers; ++j) {
      const Span oq = span(readers[j].qs, (int64_t)E * readers[j].N * Kb * 16);
      const Span od = span(readers[j].d, (int64_t)E * readers[j].N * Kb * 2);
      if (overlap(outs[i], oq) || overlap(outs[i], od)) return QIMG_EALIAS;
    }
    if (overlap(outs[i], si) || overlap(outs[i], sids) || overlap(outs[i], sl) ||
        overlap(outs[i], sw))
      return QIMG_EALIAS;
    for (int j = 0; j < i; ++j)
      if (overlap(outs[i], outs[j])) return QIMG_EALIAS;
    if (r.N > maxN) maxN = r.N;
  }
  const ReaderShape sh = reader_shape(Kb, maxN, E);
  MmvqArgs a{};
  int tiles = 0;
  for (int i = 0; i < n_readers; ++i) {
    const qimg_q4_0_expert_reader& r = readers[i];
    a.r[i] = ReaderDesc{(const uint8_t*)r.qs, (const uint16_t*)r.d, r.out, r.ld_pair, r.N, 0};
    a.tile_start[i] = tiles;
    tiles += (r.N + sh.TR - 1) / sh.TR;
  }
  a.tile_start[n_readers] = tiles;
  if ((int64_t)tiles * E > 0x7fffffff) return QIMG_EUNSUPPORTED;
  const int RB = row_blocks(K);
  a.codes = (const uint8_t*)img;
  a.ds = (const uint32_t*)((const uint8_t*)img + (size_t)bucket * RB * 32);
  a.live_rows = live_rows;
  a.ids = ids;
  a.ws = (int32_t*)workspace;
  a.n_readers = n_readers; a.RB = RB; a.Kb = Kb; a.rows = bucket; a.TR = sh.TR;
  a.top_k = top_k; a.E = E; a.routed = 1;
  return launch_mmvq(a, E, (int)pairs, (hipStream_t)stream, sh);
}

int mmvq_q4_0_q8_1_blockdots(const qimg_q4_0_reader* reader, const void* img, int32_t rows,
                             int32_t K, int32_t* sumi, void* stream) {
  int st = check_k(K);
  if (st) return st;
  if (!reader || !sumi || rows < 0 || !reader->qs || reader->N <= 0) return QIMG_EINVAL;
  if (rows == 0) return QIMG_OK;
  if ((st = check_image(img, rows, K))) return st;
  if (!al16(reader->qs) || !al(sumi, 4)) return QIMG_EALIGN;
  const int Kb = K / 32;
  const int64_t total = (int64_t)rows * reader->N * Kb;
  const Span ss = span(sumi, total * 4);
  if (overlap(ss, span(img, qimg_image_bytes(rows, K))) ||
      overlap(ss, span(reader->qs, (int64_t)reader->N * Kb * 16)))
    return QIMG_EALIAS;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(blockdots_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (const uint8_t*)reader->qs, reader->N, Kb, (const uint8_t*)img,
                     row_blocks(K), rows, sumi);
  return launch_status();
}

}  // extern "C"
