// Language-model head and loss: the reductions around the head GEMMs.
//
// The logits z = h W^T of a row are never stored: the forward GEMM's
// epilogue reduces every 128-column segment of a row to (max, sum of
// exp(z - max)) and keeps the logit at the row's target; head_lse_kernel
// merges a row's segments into its log-sum-exp and its loss term
// lse - z[target]; head_loss_kernel sums the terms in a fixed order into the
// mean over the counted rows (targets in [0, V)).  The backward GEMM
// recomputes z and writes dz = dloss/count * (softmax(z) - onehot(target)).
//   (Cross-entropy of an untied lm_head: the flicky.cc course page, sections
//   on what changed since GPT-2 and on the bits-per-byte metric.)
#pragma once
#include "common.cuh"

namespace blk {
namespace head {

// One wave per row: lse[row] = M + log sum_j l_j exp(m_j - M) over the nseg
// segment pairs (m_j, l_j), M = max_j m_j; per workgroup, the sum of the
// loss terms of its counted rows and their number.  Grid ceil(N/4), 256 threads.
__global__ __launch_bounds__(256) void head_lse_kernel(const float2* __restrict__ part, int nseg,
                                                       const float* __restrict__ tgt_logit,
                                                       const int* __restrict__ tgt, int N, int V,
                                                       float* __restrict__ lse, float* __restrict__ nll_part,
                                                       int* __restrict__ cnt_part) {
  __shared__ float wn[4];
  __shared__ int wc[4];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const long row = (long)blockIdx.x * 4 + w;
  float nll = 0.f;
  int c = 0;
  if (row < N) {
    const float2* p = part + row * nseg;
    float M = -INFINITY;
    for (int j = lane; j < nseg; j += 64) M = fmaxf(M, p[j].x);
    M = wave_max(M);
    float L = 0.f;
    for (int j = lane; j < nseg; j += 64) {
      const float2 v = p[j];
      L += v.y * __builtin_amdgcn_exp2f((v.x - M) * 1.4426950408889634f);
    }
    L = wave_sum(L);
    const float ls = M + logf(L);
    if (lane == 0) {
      lse[row] = ls;
      const int t = tgt[row];
      if (t >= 0 && t < V) {
        nll = ls - tgt_logit[row];
        c = 1;
      }
    }
  }
  if (lane == 0) {
    wn[w] = nll;
    wc[w] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    nll_part[blockIdx.x] = (wn[0] + wn[1]) + (wn[2] + wn[3]);
    cnt_part[blockIdx.x] = wc[0] + wc[1] + wc[2] + wc[3];
  }
}

// Fixed-order sum of nb partial sums and counts (double accumulation):
// *loss = sum / count (0 with no counted row), *count.  One workgroup of 1024.
__global__ __launch_bounds__(1024) void head_loss_kernel(const float* __restrict__ nll_part,
                                                         const int* __restrict__ cnt_part, int nb,
                                                         float* __restrict__ loss, int* __restrict__ count) {
  __shared__ double sn[1024];
  __shared__ int sc[1024];
  const int tid = threadIdx.x;
  double a = 0.0;
  int c = 0;
  for (int i = tid; i < nb; i += 1024) {
    a += (double)nll_part[i];
    c += cnt_part[i];
  }
  sn[tid] = a;
  sc[tid] = c;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s) {
      sn[tid] += sn[tid + s];
      sc[tid] += sc[tid + s];
    }
    __syncthreads();
  }
  if (tid == 0) {
    *count = sc[0];
    if (loss) *loss = sc[0] > 0 ? (float)(sn[0] / sc[0]) : 0.f;
  }
}

// Number of counted rows (targets in [0, V)).  One workgroup of 1024.
__global__ __launch_bounds__(1024) void head_count_kernel(const int* __restrict__ tgt, int N, int V,
                                                          int* __restrict__ count) {
  __shared__ int sc[1024];
  const int tid = threadIdx.x;
  int c = 0;
  for (int i = tid; i < N; i += 1024) c += (tgt[i] >= 0 && tgt[i] < V) ? 1 : 0;
  sc[tid] = c;
  __syncthreads();
  for (int s = 512; s > 0; s >>= 1) {
    if (tid < s) sc[tid] += sc[tid + s];
    __syncthreads();
  }
  if (tid == 0) *count = sc[0];
}

}  // namespace head
}  // namespace blk
