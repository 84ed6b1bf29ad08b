// KV-cache decode step of the block: one new token per sequence attends to
// its cached keys and values.  Inference with a KV cache (prefill, then one
// token per step) is named on the 7minutos.es page, section on midtraining,
// SFT and tool use, and in the launch thread on the same subject.
//
// The step reads every weight once (12 C^2 values) and each sequence's cache
// (2 x H x L x 128 values): it is bound by HBM bandwidth, not by MFMA.
//
//   skinny_gemm_kernel     part[s] = A W^T over K-split s           (x4)
//                          (the QKV one on x itself: rmsnorm(x) W^T =
//                          r1 (x W^T), with r1 = 1/rms(x) a row scale)
//   dec_qkv_epi_kernel     r1 of the row; rotary + QK-norm of q, k; k, v
//                          into slot p
//   dec_attn_kernel        per 256-key split: max, sum, sum p v
//   dec_combine_kernel     merge the splits -> o                    [B, C]
//   dec_resid_norm_kernel  y1 = x + o W_o^T; h2 = rmsnorm(y1)
//   skinny_gemm_relu2      a = relu(h2 W_fc^T)^2, unsplit, in one kernel
//   dec_out_kernel         y = y1 + a W_proj^T
#pragma once
#include "common.cuh"

namespace blk {
namespace dec {

constexpr int KEYS = 256;        // keys per attention workgroup (4 waves x 64)
constexpr int NBLK = 32;         // output columns per skinny-GEMM workgroup
constexpr int MBLK = 64;         // rows per skinny-GEMM workgroup
constexpr int KCH = 64;          // K elements per skinny-GEMM step (4 MFMAs)

__device__ __forceinline__ float block_sum256(float v, float* sh) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
  __syncthreads();
  v = sh[0] + sh[1] + sh[2] + sh[3];
  __syncthreads();
  return v;
}

// Skinny GEMM for a few rows: part[s][m][n] = sum over K-split s of
// A[m, k] W[n, k], fp32.  A [M, K] and W [N, K] row-major bf16; N % 32 == 0,
// K % 64 == 0.  Grid (N/32, S, ceil(M/64)); 4 waves share the workgroup's
// 64 x 32 tile and take its K-steps in turn, then add up through LDS.
//
// Within a 64-wide K-step, lane l (column/row l%32, half g = l/32) loads 32
// consecutive elements k0 + 32g .. k0 + 32g + 31 of its W row and of its A
// rows, and MFMA e (of 4) takes elements 8e..8e+7 of them: the contraction
// is over a permutation of the step's 64 k that both operands share.
__global__ __launch_bounds__(256) void skinny_gemm_kernel(const bf16* __restrict__ A, int M,
                                                          const bf16* __restrict__ W, int N, int K, int cps,
                                                          float* __restrict__ part) {
  __shared__ float red[4][MBLK * NBLK];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n0 = blockIdx.x * NBLK, s = blockIdx.y, m0 = blockIdx.z * MBLK;
  const int ksteps = K / KCH;
  const int c0 = s * cps, c1 = min(ksteps, c0 + cps);
  const int l32 = lane & 31, g = lane >> 5;
  const bf16* wrow = W + (long)(n0 + l32) * K + 32 * g;
  const int ra = m0 + l32, rb = m0 + 32 + l32;
  const bool oka = ra < M, okb = rb < M;
  const bf16* arow = A + (long)(oka ? ra : 0) * K + 32 * g;
  const bf16* brow = A + (long)(okb ? rb : 0) * K + 32 * g;
  f32x16 acc0 = {}, acc1 = {};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int c = c0 + wv; c < c1; c += 4) {
    const long k0 = (long)c * KCH;
    u32x4 wb[4], xa[4], xb[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wb[e] = ld16(wrow + k0 + 8 * e);
      xa[e] = oka ? ld16(arow + k0 + 8 * e) : zero;
      xb[e] = okb ? ld16(brow + k0 + 8 * e) : zero;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x8 w8 = __builtin_bit_cast(bf16x8, wb[e]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[e]), w8, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xb[e]), w8, acc1, 0, 0, 0);
    }
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = acc_row(j, lane);
    red[wv][r * NBLK + l32] = acc0[j];
    red[wv][(r + 32) * NBLK + l32] = acc1[j];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MBLK * NBLK / 256; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int r = e / NBLK, col = e % NBLK;
    if (m0 + r < M)
      part[((long)s * M + m0 + r) * N + n0 + col] = red[0][e] + red[1][e] + red[2][e] + red[3][e];
  }
}

// Sum of the S split partials of one output, in split order.  Loads are
// issued eight at a time so their latencies overlap.
__device__ __forceinline__ float sum_parts(const float* __restrict__ part, int S, long stride, long idx) {
  float v = 0.f;
  for (int s0 = 0; s0 < S; s0 += 8) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = s0 + i < S ? part[(s0 + i) * stride + idx] : 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) v += x[i];
  }
  return v;
}

// Position of sequence b's new token.  A length outside [0, S_max - 1] is
// an argument error of that sequence: the kernels that read the cache use
// the clamped value (every access stays inside the cache), the slot is not
// written, the status word counts the sequence and its output row is NaN.
__device__ __forceinline__ int clamp_pos(const int* __restrict__ cache_len, int b, int S_max) {
  return min(max(cache_len[b], 0), S_max - 1);
}
__device__ __forceinline__ bool pos_ok(const int* __restrict__ cache_len, int b, int S_max) {
  const int p = cache_len[b];
  return p >= 0 && p < S_max;
}

// The FC skinny GEMM with ReLU^2 in its own epilogue: a = bf16(relu(A W^T)^2)
// over the whole K range in one workgroup per 64 x 32 tile (no split, so no
// partials and no second kernel; with K = C the A rows a workgroup reads, 64
// x K, stay small).  Operand layout and MFMA use as in skinny_gemm_kernel;
// each wave takes the K-steps c = wave, wave + 4, ... and issues the loads
// of step c + 4 before the MFMAs of step c (two register stages), so its
// step loop waits about one memory latency instead of one per step.
// Grid (N/32, ceil(M/64)).
__global__ __launch_bounds__(256) void skinny_gemm_relu2_kernel(const bf16* __restrict__ A, int M,
                                                                const bf16* __restrict__ W, int N, int K,
                                                                bf16* __restrict__ out) {
  __shared__ float red[4][MBLK * NBLK];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int n0 = blockIdx.x * NBLK, m0 = blockIdx.y * MBLK;
  const int ksteps = K / KCH;
  const int l32 = lane & 31, g = lane >> 5;
  const bf16* wrow = W + (long)(n0 + l32) * K + 32 * g;
  const int ra = m0 + l32, rb = m0 + 32 + l32;
  const bool oka = ra < M, okb = rb < M;
  const bf16* arow = A + (long)(oka ? ra : 0) * K + 32 * g;
  const bf16* brow = A + (long)(okb ? rb : 0) * K + 32 * g;
  f32x16 acc0 = {}, acc1 = {};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  u32x4 w0[4], a0[4], b0[4], w1[4], a1[4], b1[4];
  auto load = [&](int c, u32x4* wb, u32x4* xa, u32x4* xb) {
    const long k0 = (long)c * KCH;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      wb[e] = ld16(wrow + k0 + 8 * e);
      xa[e] = oka ? ld16(arow + k0 + 8 * e) : zero;
      xb[e] = okb ? ld16(brow + k0 + 8 * e) : zero;
    }
  };
  auto mma = [&](const u32x4* wb, const u32x4* xa, const u32x4* xb) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x8 w8 = __builtin_bit_cast(bf16x8, wb[e]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xa[e]), w8, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, xb[e]), w8, acc1, 0, 0, 0);
    }
  };
  int c = wv;
  if (c < ksteps) load(c, w0, a0, b0);
  while (c < ksteps) {          // stage 0 holds step c
    const bool n1 = c + 4 < ksteps;
    if (n1) load(c + 4, w1, a1, b1);
    mma(w0, a0, b0);
    if (!n1) break;
    if (c + 8 < ksteps) load(c + 8, w0, a0, b0);
    mma(w1, a1, b1);
    c += 8;
  }
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int r = acc_row(j, lane);
    red[wv][r * NBLK + l32] = acc0[j];
    red[wv][(r + 32) * NBLK + l32] = acc1[j];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < MBLK * NBLK / 256; ++i) {
    const int e = threadIdx.x + 256 * i;
    const int r = e / NBLK, col = e % NBLK;
    if (m0 + r < M) {
      const float u = fmaxf(red[0][e] + red[1][e] + red[2][e] + red[3][e], 0.f);
      out[(long)(m0 + r) * N + n0 + col] = (bf16)(u * u);
    }
  }
}

// From the QKV partials of row b (products with x itself): times r1 =
// 1/rms(x[b]) they are rmsnorm(x) W^T; q and k rotated by the angle of
// position p = cache_len[b] and RMS-normalised per head (QK-norm); q
// (float32) into qbuf[b, h, :], k and v (bf16) into slot p of the caches of
// key/value head h (h < G).  Grid (H, B), 3 waves: q, k, v of head h; lane i
// owns the pair (i, i + 64); each wave computes r1 of the row itself.
__global__ __launch_bounds__(192) void dec_qkv_epi_kernel(const float* __restrict__ part, int S, int B, int H, int G,
                                                          const bf16* __restrict__ x, const int* __restrict__ cache_len,
                                                          int S_max, float eps, double rope_base,
                                                          float* __restrict__ qbuf, bf16* __restrict__ kc,
                                                          bf16* __restrict__ vc) {
  const int h = blockIdx.x, b = blockIdx.y, which = threadIdx.x >> 6, i = threadIdx.x & 63;
  if (which > 0 && (h >= G || !pos_ok(cache_len, b, S_max))) return;   // no cache write for an out-of-range length
  const int C = H * 128;
  float ss = 0.f;
  for (int c = 8 * i; c < C; c += 512) {
    float f[8];
    Chunk<bf16>::unpack(ld16(x + (long)b * C + c), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += f[e] * f[e];
  }
  const float r1 = 1.f / sqrtf(wave_sum(ss) / (float)C + eps);
  const long LD = C + 256L * G;                 // q | k | v columns
  const long stride = (long)B * LD;
  const long base = (long)b * LD + (which == 0 ? 0 : which == 1 ? C : C + 128L * G) + h * 128;
  float z1 = r1 * sum_parts(part, S, stride, base + i), z2 = r1 * sum_parts(part, S, stride, base + i + 64);
  const int p = clamp_pos(cache_len, b, S_max);
  const long slot = ((long)(b * G + h) * S_max + p) * 128;
  if (which == 2) {
    vc[slot + i] = (bf16)z1;
    vc[slot + i + 64] = (bf16)z2;
    return;
  }
  double sn, cs;
  sincos((double)p * pow(rope_base, -2.0 * i / 128.0), &sn, &cs);
  const float c = (float)cs, s = (float)sn;
  const float y1 = z1 * c - z2 * s, y2 = z1 * s + z2 * c;
  const float r = 1.f / sqrtf(wave_sum(y1 * y1 + y2 * y2) / 128.f + eps);
  if (which == 0) {
    float* q = qbuf + (long)(b * H + h) * 128;
    q[i] = y1 * r;
    q[i + 64] = y2 * r;
  } else {
    kc[slot + i] = (bf16)(y1 * r);
    kc[slot + i + 64] = (bf16)(y2 * r);
  }
}

// One split of KEYS keys of one (sequence, key/value head): keys j in
// [s*KEYS, min((s+1)*KEYS, L)), L = cache_len[b] + 1.  For each of the R =
// H/G query heads that share the key/value head it writes the split's running
// maximum m (log2 units), sum l = sum 2^(t_j - m) and unnormalised output
// sum 2^(t_j - m) v_j, t_j = log2(e) q.k_j / sqrt(128).  The keys and values
// are loaded once into registers and serve every query head of the group.
// Grid (NS, G, B), 4 waves of 64 keys, dynamic LDS dec_attn_lds(R).  Lane
// (g = lane/16, r = lane%16) holds dims 8r..8r+7 of keys base + 4i + g,
// i = 0..15.  With a window W only the keys j0 = max(0, L - W) .. L-1 are
// visible; splits wholly before j0 write nothing.
__device__ __forceinline__ int first_visible(int L, int W) { return L > W ? L - W : 0; }

__host__ __device__ constexpr size_t dec_attn_lds(int R) { return (size_t)R * (5 * 128 + 8) * sizeof(float); }

// GROUPED = false is the R = 1 instance (no head loop; K can be released
// while V is still in flight).
template <bool GROUPED>
__global__ __launch_bounds__(256) void dec_attn_kernel(const float* __restrict__ qbuf, const bf16* __restrict__ kc,
                                                       const bf16* __restrict__ vc, const int* __restrict__ cache_len,
                                                       int H, int G, int S_max, int NS, int W, float sl2,
                                                       float* __restrict__ opart, float2* __restrict__ ml) {
  extern __shared__ float dsm[];
  const int R = GROUPED ? H / G : 1;
  float* wo = dsm;                 // [R][4][128] per-wave output sums
  float* wm = dsm + R * 512;       // [R][4] per-wave maxima
  float* wl = wm + R * 4;          // [R][4] per-wave sums
  float* qs = wl + R * 4;          // [R][128] the group's q rows, scaled
  const int s = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int L = clamp_pos(cache_len, b, S_max) + 1;
  const int j0 = first_visible(L, W);
  if (s * KEYS >= L || (s + 1) * KEYS <= j0) return;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, r = lane & 15;
  const int kb = s * KEYS + wv * 64;
  const long head0 = (long)b * H + (long)kvh * R;   // first query head of the group
  if constexpr (GROUPED) {
    for (int e = threadIdx.x; e < R * 128; e += 256) qs[e] = qbuf[head0 * 128 + e] * sl2;
    __syncthreads();
  }
  if (kb < L && kb + 63 >= j0) {
    const long kvrow = (long)b * G + kvh;
    const bf16* kp = kc + kvrow * S_max * 128 + r * 8;
    const bf16* vp = vc + kvrow * S_max * 128 + r * 8;
    u32x4 kr[16], vr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const long j = min(kb + 4 * i + g, L - 1);   // past the end: a valid key, masked below
      kr[i] = ld16(kp + j * 128);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const long j = min(kb + 4 * i + g, L - 1);
      vr[i] = ld16(vp + j * 128);
    }
    const bool valid = kb + 4 * r + g < L && kb + 4 * r + g >= j0;
    for (int hr = 0; hr < R; ++hr) {
      // keep K and V packed across the head loop: unpacking them once for
      // every head would take 256 float registers
      if constexpr (GROUPED) {
#pragma unroll
        for (int i = 0; i < 16; ++i) asm volatile("" : "+v"(kr[i]), "+v"(vr[i]));
      }
      float q[8];
      if constexpr (GROUPED) {
        Chunk<float>::unpack(*reinterpret_cast<const u32x4*>(qs + hr * 128 + r * 8), q);
        Chunk<float>::unpack(*reinterpret_cast<const u32x4*>(qs + hr * 128 + r * 8 + 4), q + 4);
      } else {
        const float* qp = qbuf + (head0 + hr) * 128 + r * 8;
#pragma unroll
        for (int e = 0; e < 8; ++e) q[e] = qp[e] * sl2;
      }
      // partial dot products over this lane's 8 dims, then a transposing
      // butterfly over the 16 lanes of the key group: after the steps with
      // masks 8, 4, 2, 1 lane r holds the full score of key base + 4r + g
      float t[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float f[8];
        Chunk<bf16>::unpack(kr[i], f);
        float a = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) a += q[e] * f[e];
        t[i] = a;
      }
#pragma unroll
      for (int half = 8; half >= 1; half >>= 1) {
        const bool up = (r & half) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
          // the empty asm keeps the two picks selects of values: folded
          // into one load of t at a per-lane index, they would become a
          // compare-and-select chain over all 16 entries once unrolled
          float lo = t[i], hi = t[i + half];
          asm("" : "+v"(lo), "+v"(hi));
          const float send = up ? lo : hi;
          const float keep = up ? hi : lo;
          t[i] = keep + __shfl_xor(send, half, 64);
        }
      }
      const float sc = valid ? t[0] : -INFINITY;
      const float m = wave_max(sc);
      const float p = valid ? __builtin_amdgcn_exp2f(sc - m) : 0.f;
      const float l = wave_sum(p);
      float pk[16];   // p of the keys this lane multiplies: held by lanes 16g + i
#pragma unroll
      for (int i = 0; i < 16; ++i) pk[i] = __shfl(p, 16 * g + i, 64);
      float o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float f[8];
        Chunk<bf16>::unpack(vr[i], f);
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] += pk[i] * f[e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        o[e] += __shfl_xor(o[e], 16, 64);
        o[e] += __shfl_xor(o[e], 32, 64);
      }
      if (lane < 16) {
#pragma unroll
        for (int e = 0; e < 8; ++e) wo[(hr * 4 + wv) * 128 + lane * 8 + e] = o[e];
      }
      if (lane == 0) {
        wm[hr * 4 + wv] = m;
        wl[hr * 4 + wv] = l;
      }
    }
  } else {
    // a wave with no visible key contributes nothing to any head
    for (int e = lane; e < R * 128; e += 64) wo[(e / 128 * 4 + wv) * 128 + e % 128] = 0.f;
    for (int hr = lane; hr < R; hr += 64) {
      wm[hr * 4 + wv] = -INFINITY;
      wl[hr * 4 + wv] = 0.f;
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < R * 128; e += 256) {
    const int hr = e / 128, d = e % 128;
    const float* m4 = wm + hr * 4;
    const float* l4 = wl + hr * 4;
    const float M = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));   // finite: some wave has keys
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float f = m4[w] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m4[w] - M);
      acc += f * wo[(hr * 4 + w) * 128 + d];
      lsum += f * l4[w];
    }
    const long slot = (head0 + hr) * NS + s;
    opart[slot * 128 + d] = acc;
    if (d == 0) ml[slot] = make_float2(M, lsum);
  }
}

// o[b, h*128 + d] = sum_s 2^(m_s - M) o_s[d] / sum_s 2^(m_s - M) l_s over the
// splits that hold visible keys.  Grid (H, B), 128 threads.
__global__ __launch_bounds__(128) void dec_combine_kernel(const float* __restrict__ opart,
                                                          const float2* __restrict__ ml,
                                                          const int* __restrict__ cache_len, int H, int S_max,
                                                          int NS, int W, bf16* __restrict__ o) {
  const int h = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int L = clamp_pos(cache_len, b, S_max) + 1;
  const int nv = (L + KEYS - 1) / KEYS;
  const int s0 = first_visible(L, W) / KEYS;
  const long head = (long)(b * H + h);
  float M = -INFINITY;
  for (int s = s0; s < nv; ++s) M = fmaxf(M, ml[head * NS + s].x);
  float acc = 0.f, lsum = 0.f;
  for (int s = s0; s < nv; ++s) {
    const float2 v = ml[head * NS + s];
    const float f = __builtin_amdgcn_exp2f(v.x - M);
    acc += f * opart[(head * NS + s) * 128 + d];
    lsum += f * v.y;
  }
  o[(long)b * H * 128 + h * 128 + d] = (bf16)(acc / lsum);
}

// y1 = x + sum_s part[s] (float32), h2 = bf16(y1 / rms(y1)).  Grid B.
__global__ __launch_bounds__(256) void dec_resid_norm_kernel(const float* __restrict__ part, int S, int B, int C,
                                                             const bf16* __restrict__ x, float eps,
                                                             float* __restrict__ y1, bf16* __restrict__ h2) {
  __shared__ float sh[4];
  const long row = blockIdx.x;
  const long stride = (long)B * C;
  float v[8];
  float ss = 0.f;
  const int per = (C + 255) / 256;   // <= 8
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = threadIdx.x + 256 * u;
    v[u] = 0.f;
    if (u < per && c < C) {
      v[u] = (float)x[row * C + c] + sum_parts(part, S, stride, row * C + c);
      ss += v[u] * v[u];
    }
  }
  const float r = 1.f / sqrtf(block_sum256(ss, sh) / (float)C + eps);
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    const int c = threadIdx.x + 256 * u;
    if (u < per && c < C) {
      y1[row * C + c] = v[u];
      h2[row * C + c] = (bf16)(v[u] * r);
    }
  }
}

// y = bf16(y1 + sum_s part[s]) over n = B*C values; NaN in the rows of
// sequences whose length is out of range, whose count thread 0 writes to
// *status (when given).
__global__ __launch_bounds__(256) void dec_out_kernel(const float* __restrict__ part, int S, long n,
                                                      const float* __restrict__ y1, bf16* __restrict__ y,
                                                      const int* __restrict__ cache_len, int S_max, int C,
                                                      int* __restrict__ status) {
  const long i = (long)blockIdx.x * 256 + threadIdx.x;
  if (status && i == 0) {
    int bad = 0;
    for (int b = 0; b < (int)(n / C); ++b) bad += pos_ok(cache_len, b, S_max) ? 0 : 1;
    *status = bad;
  }
  if (i >= n) return;
  const float v = y1[i] + sum_parts(part, S, n, i);
  y[i] = (bf16)(pos_ok(cache_len, (int)(i / C), S_max) ? v : __builtin_nanf(""));
}

}  // namespace dec
}  // namespace blk
