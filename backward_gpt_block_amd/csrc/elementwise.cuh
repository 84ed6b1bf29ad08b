// Row-wise kernels of the block: RMSNorm forward/backward, the rotary angle
// table, rotary + QK-norm forward/backward, the attention-backward row dot
// product and the split-k reduction of weight gradients.  All are HBM-bound:
// one wave per row, 16-byte accesses along the row.
#pragma once
#include "common.cuh"

namespace blk {

constexpr int MAXCH = 8;   // 16-byte chunks per lane a row kernel keeps in registers

// The row kernels' absolute maximum (fp8 mode): reduced over the workgroup's
// four waves, then one atomic per workgroup.  A row kernel launched for an
// fp8 tensor walks its rows with a grid stride over at most amax_blocks
// workgroups, so a tensor costs a few hundred atomics on its one word instead
// of one per row.  Every thread of the workgroup must call it.
constexpr unsigned AMAX_BLOCKS = 1024;
template <typename T>
__device__ __forceinline__ void amax_publish_wg(unsigned* amax, float m) {
  __shared__ float wm[4];
  m = wave_max(m);
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    m = to_f32(from_f32<T>(fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]))));
    const unsigned cur = __hip_atomic_load(amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__float_as_uint(m) > cur) atomicMax(amax, __float_as_uint(m));
  }
}

// h = x * r, r = (mean(x^2) + eps)^-1/2 per row of C elements.
// Parameter-free RMSNorm (flicky.cc nanochat page, section on the model,
// and its glossary entry for RMSNorm, without the gain).
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const T* __restrict__ x, T* __restrict__ h,
                                                          float* __restrict__ r, int N, int C, float eps,
                                                          unsigned* __restrict__ amax = nullptr) {
  constexpr int EL = Chunk<T>::N;
  const int lane = threadIdx.x & 63;
  const int nch = C / EL;
  float mx = 0.f;
  // one row per wave; the grid covers all rows (one pass) unless it was
  // capped for an fp8 tensor
  for (long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6); row < N; row += (long)gridDim.x * 4) {
  const T* xr = x + row * C;
  u32x4 c[MAXCH];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    int ch = lane + i * 64;
    if (ch < nch) {
      c[i] = ld16(xr + ch * EL);
      float f[EL];
      Chunk<T>::unpack(c[i], f);
#pragma unroll
      for (int e = 0; e < EL; ++e) ss += f[e] * f[e];
    }
  }
  ss = wave_sum(ss);
  const float rr = 1.f / sqrtf(ss / (float)C + eps);
  if (lane == 0 && r) r[row] = rr;
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    int ch = lane + i * 64;
    if (ch < nch) {
      float f[EL];
      Chunk<T>::unpack(c[i], f);
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        f[e] *= rr;
        mx = fmaxf(mx, fabsf(f[e]));
      }
      st16(h + row * C + ch * EL, Chunk<T>::pack(f));
    }
  }
  }
  if (amax) amax_publish_wg<T>(amax, mx);   // fp8 mode: the tensor's absolute maximum
}

// out = resid + r * (dh - hn * mean(dh * hn)): RMSNorm backward (hn is the
// normalised output) plus the gradient arriving through the residual path.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const T* __restrict__ resid, const T* __restrict__ dh,
                                                          const T* __restrict__ hn, const float* __restrict__ r,
                                                          T* __restrict__ out, int N, int C,
                                                          unsigned* __restrict__ amax = nullptr) {
  constexpr int EL = Chunk<T>::N;
  const int lane = threadIdx.x & 63;
  const int nch = C / EL;
  float mx = 0.f;
  for (long row = (long)blockIdx.x * 4 + (threadIdx.x >> 6); row < N; row += (long)gridDim.x * 4) {
  u32x4 cd[MAXCH], ch_[MAXCH];
  float dot = 0.f;
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    int ch = lane + i * 64;
    if (ch < nch) {
      cd[i] = ld16(dh + row * C + ch * EL);
      ch_[i] = ld16(hn + row * C + ch * EL);
      float a[EL], b[EL];
      Chunk<T>::unpack(cd[i], a);
      Chunk<T>::unpack(ch_[i], b);
#pragma unroll
      for (int e = 0; e < EL; ++e) dot += a[e] * b[e];
    }
  }
  dot = wave_sum(dot);
  const float mean = dot / (float)C;
  const float rr = r[row];
#pragma unroll
  for (int i = 0; i < MAXCH; ++i) {
    int ch = lane + i * 64;
    if (ch < nch) {
      float a[EL], b[EL], g[EL];
      Chunk<T>::unpack(cd[i], a);
      Chunk<T>::unpack(ch_[i], b);
      if (resid) Chunk<T>::unpack(ld16(resid + row * C + ch * EL), g);
      else {
#pragma unroll
        for (int e = 0; e < EL; ++e) g[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        g[e] += rr * (a[e] - b[e] * mean);
        mx = fmaxf(mx, fabsf(g[e]));
      }
      st16(out + row * C + ch * EL, Chunk<T>::pack(g));
    }
  }
  }
  if (amax) amax_publish_wg<T>(amax, mx);   // fp8 mode: the tensor's absolute maximum
}

// cs[t][i] = (cos, sin) of t * base^(-2i/D), i < D/2, computed in double
// precision and rounded to float.
__global__ void rope_table_kernel(float2* __restrict__ cs, int T, int D, double base) {
  const int half = D / 2;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)T * half) return;
  const int t = idx / half, i = idx % half;
  const double inv = pow(base, -2.0 * i / (double)D);
  double s, c;
  sincos((double)t * inv, &s, &c);
  cs[idx] = make_float2((float)c, (float)s);
}

// In place on the dq, dk parts of dqkv [N, 3C]: QK-norm backward
// (dz' = rho * (dz'' - z'' * mean(dz'' * z''))) then the transpose rotation.
// zn = the saved normalised q'' | k'' (qkv layout).
// One wave per (row, head) of the H query heads then the G key heads; rows of
// qkv / dqkv are C + 2*128*G wide.
template <typename T>
__global__ __launch_bounds__(256) void qknorm_rope_bwd_kernel(T* __restrict__ dqkv, const T* __restrict__ zn,
                                                              const float* __restrict__ rho,
                                                              const float2* __restrict__ cs, int N, int Tlen,
                                                              int H, int C, int G) {
  const int lane = threadIdx.x & 63;
  const long w = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long total = (long)N * (H + G);
  if (w >= total) return;
  const int j = (int)(w % (H + G));
  const int which = j < H ? 0 : 1;
  const int head = which ? j - H : j;
  const long row = w / (H + G);
  const int t = row % Tlen;
  const long off = row * (C + 256L * G) + which * C + head * 128;
  T* g = dqkv + off;
  const T* z = zn + off;
  const float g1 = to_f32(g[lane]), g2 = to_f32(g[lane + 64]);
  const float z1 = to_f32(z[lane]), z2 = to_f32(z[lane + 64]);
  const float mean = wave_sum(g1 * z1 + g2 * z2) / 128.f;
  const float p = rho[((long)which * N + row) * H + head];
  const float d1 = p * (g1 - z1 * mean), d2 = p * (g2 - z2 * mean);
  const float2 a = cs[(long)t * 64 + lane];
  g[lane] = from_f32<T>(d1 * a.x + d2 * a.y);
  g[lane + 64] = from_f32<T>(-d1 * a.y + d2 * a.x);
}

// dst[c][r] = src[r][c] for a rows x cols matrix (both multiples of 64):
// 64 x 64 tiles through LDS, 256 threads.
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, T* __restrict__ dst, int rows,
                                                        int cols) {
  __shared__ T t[64][65];
  const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 16; ++i) t[ty + 4 * i][tx] = src[(long)(r0 + ty + 4 * i) * cols + c0 + tx];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 16; ++i) dst[(long)(c0 + ty + 4 * i) * rows + r0 + tx] = t[tx][ty + 4 * i];
}

// dst[i] = (accumulate ? dst[i] : 0) + sum_s part[s*n + i], in split order.
__global__ void splitk_reduce_kernel(float* __restrict__ dst, const float* __restrict__ part, long n, int splits,
                                     int accumulate) {
  const long i4 = ((long)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i4 >= n) return;
  f32x4 s = accumulate ? *reinterpret_cast<const f32x4*>(dst + i4) : f32x4{0, 0, 0, 0};
  for (int k = 0; k < splits; ++k) s += *reinterpret_cast<const f32x4*>(part + (long)k * n + i4);
  *reinterpret_cast<f32x4*>(dst + i4) = s;
}

}  // namespace blk
