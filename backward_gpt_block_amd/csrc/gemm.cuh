// MFMA GEMM for gfx950:  C[m, n] = sum_k A(m, k) * B(n, k)  (fp32 accumulate)
//
// A(m, k) is A[m*lda + k] when A is "k-contiguous" (KA = true), else
// A[k*lda + m]; likewise B.  Forward projections (y = x W^T) have both
// operands k-contiguous; input gradients (dx = dy W) have a k-contiguous A and
// an n-contiguous B; weight gradients (dW = dy^T x) have both operands
// contiguous along m/n with k (tokens) strided.
//
// Workgroup tile 256 x 256, four waves in a 2 x 2 grid, each wave 128 x 128
// as 4 x 4 MFMA 32x32 blocks.  Each k-step stages a 256-row x 128-byte slab of
// A and of B into LDS (double-buffered, next slab prefetched into registers
// while the current one feeds the MFMAs).  LDS always holds rows of the m (n)
// index with k contiguous, so fragment reads are single 16-byte loads; an
// operand that is contiguous along m (n) in memory is transposed in registers
// (8 x 8 element blocks) between the global load and the LDS store.
#pragma once
#include "common.cuh"

namespace blk {

enum EpiKind : int {
  EPI_STORE = 0,    // out = alpha*acc                         (element T)
  EPI_RESID = 1,    // out = aux + alpha*acc                   (T)
  EPI_RELU2 = 2,    // out = v, out2 = max(v,0)^2, v = alpha*acc (T)
  EPI_DRELU2 = 3,   // out = alpha*acc * 2*max(aux, 0)         (T)
  EPI_F32 = 4,      // out[split] = alpha*acc                  (float)
  EPI_F32_ADD = 5,  // out += alpha*acc                        (float)
};

struct GemmArgs {
  const void* A; long lda;
  const void* B; long ldb;
  int M, N, K;
  int k_split;          // k-range per split (multiple of BK); grid splits = ceil(K / k_split)
  int tiles_m, tiles_n;
  void* out; long ldo;  // EPI_F32: split s writes out + s*M*ldo
  void* out2; long ldo2;
  const void* aux; long ldaux;
  float alpha;
  const float* alpha_ptr;  // if non-null, alpha *= alpha_ptr[0] * alpha_ptr[1]
};

template <typename TI> struct GemmTile {
  static constexpr int ELEM = 16 / sizeof(TI);   // elements per 16-byte chunk
  static constexpr int BK = 8 * ELEM;            // 128 bytes of k per row
  static constexpr int BM = 256, BN = 256, NT = 256;
  static constexpr int ROWB = 128;               // LDS bytes per tile row
  static constexpr int SLAB = (BM + BN) * ROWB;  // one stage, A then B
  static constexpr int LDS = 2 * SLAB;           // 128 KiB
};

// Staging of one operand slab: R rows of the m (n) index x BK of k.
template <typename TI, bool KC, int R>
struct Stager {
  typedef GemmTile<TI> G;
  static constexpr int ELEM = G::ELEM;
  // k-contiguous: R*8 chunks, consecutive threads take consecutive chunks of a row.
  // m-contiguous: (BK/ELEM) x (R/ELEM) blocks of ELEM x ELEM elements.
  static constexpr int NCH = KC ? (R * 8) / G::NT : ((G::BK / ELEM) * (R / ELEM) * ELEM) / G::NT;
  u32x4 reg[NCH];

  // rows r0.. (< rows_valid), k in [k0, k_end)
  __device__ void load(const TI* P, long ld, int r0, int rows_valid, int k0, int k_end) {
    const int t = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        int idx = t + i * G::NT;
        int row = idx >> 3, ch = idx & 7;
        int gr = r0 + row, gk = k0 + ch * ELEM;
        if (gr < rows_valid && gk < k_end)
          reg[i] = ld16(P + (long)gr * ld + gk);
        else
          reg[i] = u32x4{0, 0, 0, 0};
      }
    } else {
      constexpr int RB = R / ELEM;                 // blocks along the row index
      constexpr int NB = NCH / ELEM;               // blocks per thread
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        int blkid = t + b * G::NT;
        int rb = blkid % RB, kb = blkid / RB;
        int gr = r0 + rb * ELEM;
#pragma unroll
        for (int i = 0; i < ELEM; ++i) {
          int gk = k0 + kb * ELEM + i;
          if (gr < rows_valid && gk < k_end)
            reg[b * ELEM + i] = ld16(P + (long)gk * ld + gr);
          else
            reg[b * ELEM + i] = u32x4{0, 0, 0, 0};
        }
      }
    }
  }

  __device__ void store(char* lds) {
    const int t = threadIdx.x;
    if constexpr (KC) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        int idx = t + i * G::NT;
        int row = idx >> 3, ch = idx & 7;
        st16(lds + tile_off(row, ch, 8), reg[i]);
      }
    } else {
      constexpr int RB = R / ELEM;
      constexpr int NB = NCH / ELEM;
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        int blkid = t + b * G::NT;
        int rb = blkid % RB, kb = blkid / RB;
        u32x4 tr[ELEM];
        transpose_chunks(&reg[b * ELEM], tr, (TI*)nullptr);
#pragma unroll
        for (int j = 0; j < ELEM; ++j) st16(lds + tile_off(rb * ELEM + j, kb, 8), tr[j]);
      }
    }
  }
};

// Fragment of a 32-row block at k-substep ks from an LDS slab.
template <typename TI>
__device__ __forceinline__ typename Mfma<TI>::frag load_frag(const char* lds, int row0, int ks, int lane) {
  typedef Mfma<TI> MM;
  constexpr int ELEM = GemmTile<TI>::ELEM;
  const int row = row0 + (lane & 31);
  const int kel = ks * MM::KI + (lane >> 5) * MM::E;   // element offset in the row
  if constexpr (sizeof(TI) == 2) {
    return __builtin_bit_cast(typename MM::frag, ld16(lds + tile_off(row, kel / ELEM, 8)));
  } else if constexpr (sizeof(TI) == 4) {
    const char* p = lds + tile_off(row, kel / ELEM, 8) + (kel % ELEM) * 4;
    return *reinterpret_cast<const float*>(p);
  } else {
    u32x4 lo = ld16(lds + tile_off(row, kel / ELEM, 8));
    u32x4 hi = ld16(lds + tile_off(row, kel / ELEM + 1, 8));
    i32x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) { f[i] = (int)lo[i]; f[4 + i] = (int)hi[i]; }
    return f;
  }
}

template <typename TO, int EPI>
__device__ __forceinline__ void epi_store(const GemmArgs& g, float alpha, int split, int row, int col, float v) {
  v *= alpha;
  if constexpr (EPI == EPI_STORE) {
    static_cast<TO*>(g.out)[(long)row * g.ldo + col] = from_f32<TO>(v);
  } else if constexpr (EPI == EPI_RESID) {
    float r = to_f32(static_cast<const TO*>(g.aux)[(long)row * g.ldaux + col]);
    static_cast<TO*>(g.out)[(long)row * g.ldo + col] = from_f32<TO>(r + v);
  } else if constexpr (EPI == EPI_RELU2) {
    static_cast<TO*>(g.out)[(long)row * g.ldo + col] = from_f32<TO>(v);
    float p = fmaxf(v, 0.f);
    static_cast<TO*>(g.out2)[(long)row * g.ldo2 + col] = from_f32<TO>(p * p);
  } else if constexpr (EPI == EPI_DRELU2) {
    float u = to_f32(static_cast<const TO*>(g.aux)[(long)row * g.ldaux + col]);
    static_cast<TO*>(g.out)[(long)row * g.ldo + col] = from_f32<TO>(v * 2.f * fmaxf(u, 0.f));
  } else if constexpr (EPI == EPI_F32) {
    static_cast<float*>(g.out)[(long)split * g.M * g.ldo + (long)row * g.ldo + col] = v;
  } else {
    float* p = static_cast<float*>(g.out) + (long)row * g.ldo + col;
    *p = *p + v;
  }
}

// Workgroup index -> (tile_m, tile_n, split).  Workgroups are dealt round
// robin to the 8 XCDs; the remap gives each XCD a contiguous run of logical
// tiles, and tiles are walked in groups of 8 m-tiles so that an XCD's
// concurrent tiles share A rows and B columns in its L2.
__device__ __forceinline__ void tile_coords(const GemmArgs& g, int& tm, int& tn, int& split) {
  const int per_split = g.tiles_m * g.tiles_n;
  const int total = per_split * gridDim.y;
  int pid = blockIdx.x + blockIdx.y * gridDim.x;
  if (total % 8 == 0) pid = (pid % 8) * (total / 8) + pid / 8;
  split = pid / per_split;
  int t = pid % per_split;
  const int GROUP = 8;
  int group = t / (GROUP * g.tiles_n);
  int first_m = group * GROUP;
  int gsize = min(g.tiles_m - first_m, GROUP);
  int in_group = t % (GROUP * g.tiles_n);
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

template <typename TI, typename TO, bool KA, bool KB, int EPI>
__device__ __forceinline__ void gemm_body(const GemmArgs& g) {
  typedef GemmTile<TI> G;
  typedef Mfma<TI> MM;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  int tm, tn, split;
  tile_coords(g, tm, tn, split);
  const int m0 = tm * G::BM, n0 = tn * G::BN;
  const int kbeg = split * g.k_split;
  const int kend = min(g.K, kbeg + g.k_split);
  const int nk = (kend - kbeg + G::BK - 1) / G::BK;

  const TI* A = static_cast<const TI*>(g.A);
  const TI* B = static_cast<const TI*>(g.B);
  Stager<TI, KA, G::BM> sa;
  Stager<TI, KB, G::BN> sb;

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  if (nk > 0) {
    sa.load(A, g.lda, m0, g.M, kbeg, kend);
    sb.load(B, g.ldb, n0, g.N, kbeg, kend);
    sa.store(smem);
    sb.store(smem + G::BM * G::ROWB);
  }
  __syncthreads();

  for (int kt = 0; kt < nk; ++kt) {
    const char* cur = smem + (kt & 1) * G::SLAB;
    if (kt + 1 < nk) {
      const int k0 = kbeg + (kt + 1) * G::BK;
      sa.load(A, g.lda, m0, g.M, k0, kend);
      sb.load(B, g.ldb, n0, g.N, k0, kend);
    }
#pragma unroll
    for (int ks = 0; ks < G::BK / MM::KI; ++ks) {
      typename MM::frag fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = load_frag<TI>(cur, wm * 128 + i * 32, ks, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j] = load_frag<TI>(cur + G::BM * G::ROWB, wn * 128 + j * 32, ks, lane);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = MM::mma(fa[i], fb[j], acc[i][j]);
    }
    if (kt + 1 < nk) {
      char* nxt = smem + ((kt + 1) & 1) * G::SLAB;
      sa.store(nxt);
      sb.store(nxt + G::BM * G::ROWB);
    }
    __syncthreads();
  }

  float alpha = g.alpha;
  if (g.alpha_ptr) alpha *= g.alpha_ptr[0] * g.alpha_ptr[1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + (lane & 31);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + acc_row(r, lane);
        if (row < g.M && col < g.N) epi_store<TO, EPI>(g, alpha, split, row, col, acc[i][j][r]);
      }
    }
  }
}

}  // namespace blk

// One kernel symbol per call site of the block, so that traces and timings
// name the projection and pass (the bodies are the template above).
#define BLK_GEMM_KERNEL(NAME, KA, KB, EPI, TO)                                    \
  template <typename T>                                                         \
  __global__ __launch_bounds__(256, 1) void NAME(GemmArgs g) {                   \
    gemm_body<T, TO, KA, KB, EPI>(g);                                           \
  }

namespace blk {
BLK_GEMM_KERNEL(gemm_qkv_fwd, true, true, EPI_STORE, T)
BLK_GEMM_KERNEL(gemm_o_fwd, true, true, EPI_RESID, T)
BLK_GEMM_KERNEL(gemm_fc_fwd, true, true, EPI_RELU2, T)
BLK_GEMM_KERNEL(gemm_proj_fwd, true, true, EPI_RESID, T)
BLK_GEMM_KERNEL(gemm_proj_dgrad, true, false, EPI_DRELU2, T)
BLK_GEMM_KERNEL(gemm_fc_dgrad, true, false, EPI_STORE, T)
BLK_GEMM_KERNEL(gemm_o_dgrad, true, false, EPI_STORE, T)
BLK_GEMM_KERNEL(gemm_qkv_dgrad, true, false, EPI_STORE, T)
BLK_GEMM_KERNEL(gemm_proj_wgrad, false, false, EPI_F32, float)
BLK_GEMM_KERNEL(gemm_fc_wgrad, false, false, EPI_F32, float)
BLK_GEMM_KERNEL(gemm_o_wgrad, false, false, EPI_F32, float)
BLK_GEMM_KERNEL(gemm_qkv_wgrad, false, false, EPI_F32, float)
BLK_GEMM_KERNEL(gemm_proj_wgrad_acc, false, false, EPI_F32_ADD, float)
BLK_GEMM_KERNEL(gemm_fc_wgrad_acc, false, false, EPI_F32_ADD, float)
BLK_GEMM_KERNEL(gemm_o_wgrad_acc, false, false, EPI_F32_ADD, float)
BLK_GEMM_KERNEL(gemm_qkv_wgrad_acc, false, false, EPI_F32_ADD, float)
}  // namespace blk
