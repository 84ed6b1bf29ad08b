// FP8 (OCP E4M3) support for the fp8 mode of the linear layers: per-tensor
// absolute maximum, quantisation to E4M3 codes (row-major and transposed
// copies) with current scaling s = amax/448, saturating at +-448, rounding to
// nearest even (the conversion instruction's default mode).
//
// FP8 training of the linear layers is named on the flicky.cc nanochat page
// (repository map, nanochat/fp8.py) and in the README mirror's leaderboard
// ("d26 ... +fp8"); the format and the scaling recipe are not on the pages.
#pragma once
#include "common.cuh"

namespace blk {

constexpr float E4M3_MAX = 448.f;

// Non-negative floats order like their bit patterns, so max is an integer max.
__device__ __forceinline__ float amax_value(const unsigned* a) { return __uint_as_float(*a); }
__device__ __forceinline__ float quant_inv(float amax) { return amax > 0.f ? E4M3_MAX / amax : 1.f; }
__device__ __forceinline__ float quant_scale(float amax) { return amax > 0.f ? amax / E4M3_MAX : 1.f; }

// Two floats (already scaled) -> two E4M3 codes in the low 16 bits.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -E4M3_MAX), E4M3_MAX);
  b = fminf(fmaxf(b, -E4M3_MAX), E4M3_MAX);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

__global__ void zero_u32_kernel(unsigned* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

// out = max(out, max |x|) over n elements (n % 8 == 0), bf16 input.  Every
// workgroup ends in one atomic on the same word, and those serialise: the
// host caps the grid (AMAX_GRID workgroups) and each thread keeps eight
// 16-byte loads in flight per iteration instead.
constexpr unsigned AMAX_GRID = 256;
__global__ __launch_bounds__(256) void amax_kernel(const bf16* __restrict__ x, long n, unsigned* __restrict__ out) {
  float m = 0.f;
  const long stride = (long)gridDim.x * 256 * 8;
  long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8;
  for (; i + 7 * stride < n; i += 8 * stride) {
    u32x4 c[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) c[u] = ld16(x + i + u * stride);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      float f[8];
      Chunk<bf16>::unpack(c[u], f);
#pragma unroll
      for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[e]));
    }
  }
  for (; i < n; i += stride) {
    float f[8];
    Chunk<bf16>::unpack(ld16(x + i), f);
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(f[e]));
  }
  m = wave_max(m);
  __shared__ float wm[4];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
    const unsigned cur = __hip_atomic_load(out, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__float_as_uint(m) > cur) atomicMax(out, __float_as_uint(m));
  }
}

// q[i] = e4m3(x[i] * 448/amax), n % 8 == 0.
__global__ __launch_bounds__(256) void quant_kernel(const bf16* __restrict__ x, long n, const unsigned* __restrict__ amax,
                                                    uint8_t* __restrict__ q) {
  const float inv = quant_inv(amax_value(amax));
  for (long i = ((long)blockIdx.x * 256 + threadIdx.x) * 8; i < n; i += (long)gridDim.x * 256 * 8) {
    float f[8];
    Chunk<bf16>::unpack(ld16(x + i), f);
    u32x2 o;
    o[0] = e4m3x2(f[0] * inv, f[1] * inv) | (e4m3x2(f[2] * inv, f[3] * inv) << 16);
    o[1] = e4m3x2(f[4] * inv, f[5] * inv) | (e4m3x2(f[6] * inv, f[7] * inv) << 16);
    st8(q + i, o);
  }
}

// qT[c][r] = e4m3(x[r][c] * 448/amax) for a rows x cols bf16 matrix (cols %
// 64 == 0); qT has leading dimension ldT >= rows (a multiple of 64) and the
// padding columns rows..ldT-1 are written as 0.  64 x 64 tiles through LDS.
// When q is given, the row-major codes q[r][c] are written in the same pass.
__global__ __launch_bounds__(256) void quant_trans_kernel(const bf16* __restrict__ x, int rows, int cols,
                                                          const unsigned* __restrict__ amax, uint8_t* __restrict__ qT,
                                                          int ldT, uint8_t* __restrict__ q) {
  __shared__ uint8_t t[64][65];
  const float inv = quant_inv(amax_value(amax));
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 7, ty = threadIdx.x >> 3;      // 8 chunks of 8 columns x 32 rows per pass
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = ty + 32 * p;
    float f[8];
    if (r0 + r < rows) {
      Chunk<bf16>::unpack(ld16(x + (long)(r0 + r) * cols + c0 + tx * 8), f);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = 0.f;
    }
    u32x2 row8;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t two = e4m3x2(f[e] * inv, f[e + 1] * inv);
      t[tx * 8 + e][r] = (uint8_t)(two & 0xff);
      t[tx * 8 + e + 1][r] = (uint8_t)(two >> 8);
      if (e < 4) row8[0] = e == 0 ? two : (row8[0] | (two << 16));
      else row8[1] = e == 4 ? two : (row8[1] | (two << 16));
    }
    if (q && r0 + r < rows) st8(q + (long)(r0 + r) * cols + c0 + tx * 8, row8);
  }
  __syncthreads();
  // write: row c of qT gets 64 bytes (r0..r0+63); 4 threads x 16 bytes per row
  const int wr = threadIdx.x >> 2, wq = threadIdx.x & 3;
  u32x4 v;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) word |= (uint32_t)t[wr][wq * 16 + w * 4 + b] << (8 * b);
    v[w] = word;
  }
  st16(qT + (long)(c0 + wr) * ldT + r0 + wq * 16, v);
}

// quant_trans_kernel on 128 x 128 tiles (cols % 128 == 0): each thread has
// 8 row chunks of 16 bytes in flight (rows 8*ty .. 8*ty+7 of its 8-column
// group), packs the 8 codes of one column into one 8-byte LDS store, and both
// outputs are written in whole 128-byte lines.  qT columns past ldT are not
// written (ldT is a multiple of 64).
__global__ __launch_bounds__(256) void quant_trans128_kernel(const bf16* __restrict__ x, int rows, int cols,
                                                             const unsigned* __restrict__ amax,
                                                             uint8_t* __restrict__ qT, int ldT,
                                                             uint8_t* __restrict__ q) {
  constexpr int P = 144;                      // LDS row pitch (bytes), a multiple of 16
  __shared__ __attribute__((aligned(16))) uint8_t t[128 * P];
  const float inv = quant_inv(amax_value(amax));
  const int r0 = blockIdx.y * 128, c0 = blockIdx.x * 128;
  const int tx = threadIdx.x & 15, ty = threadIdx.x >> 4;   // 16 chunks of 8 columns x 16 groups of 8 rows
  u32x4 raw[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    const int r = r0 + 8 * ty + p;
    raw[p] = r < rows ? ld16(x + (long)r * cols + c0 + tx * 8) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t col8[8][2];                        // codes of column tx*8 + e, rows 8*ty .. 8*ty+7
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    float f[8];
    Chunk<bf16>::unpack(raw[p], f);
    uint32_t two[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) two[e] = e4m3x2(f[2 * e] * inv, f[2 * e + 1] * inv);
    const int r = r0 + 8 * ty + p;
    if (q && r < rows) {
      u32x2 row8;
      row8[0] = two[0] | (two[1] << 16);
      row8[1] = two[2] | (two[3] << 16);
      st8(q + (long)r * cols + c0 + tx * 8, row8);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t b = (two[e >> 1] >> (8 * (e & 1))) & 0xffu;
      const int w = p >> 2, sh = 8 * (p & 3);
      col8[e][w] = (p & 3) == 0 ? b : (col8[e][w] | (b << sh));
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    u32x2 v;
    v[0] = col8[e][0];
    v[1] = col8[e][1];
    *reinterpret_cast<u32x2*>(t + (tx * 8 + e) * P + 8 * ty) = v;
  }
  __syncthreads();
  // row c0 + wr of qT gets bytes r0 + 64 h .. r0 + 64 h + 63: 4 x 16 bytes
  const int wr = threadIdx.x >> 1, h = threadIdx.x & 1;
  if (r0 + 64 * h < ldT) {
#pragma unroll
    for (int w = 0; w < 4; ++w)
      st16(qT + (long)(c0 + wr) * ldT + r0 + 64 * h + 16 * w,
           *reinterpret_cast<const u32x4*>(t + wr * P + 64 * h + 16 * w));
  }
}

}  // namespace blk
