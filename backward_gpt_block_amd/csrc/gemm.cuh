// MFMA GEMM for gfx950:  C[m, n] = sum_k A(m, k) * B(n, k)  (fp32 accumulate)
//
// A(m, k) is A[m*lda + k] when A is "k-contiguous" (KA = true), else
// A[k*lda + m]; likewise B.  Forward projections (y = x W^T) and input
// gradients (dx = dy W, with W passed transposed) have both operands
// k-contiguous; weight gradients (dW = dy^T x) have both operands contiguous
// along m/n with k (tokens) strided.
//
// Workgroup tile 256 x 256, four waves in a 2 x 2 grid, each wave 128 x 128
// as 4 x 4 MFMA 32x32 blocks; a k-step stages a 256-row x 128-byte slab of A
// and of B in LDS (two stages, 128 KiB).  LDS rows hold k contiguously, with
// an XOR swizzle of the 16-byte chunks, so every MFMA fragment is one LDS
// read.
//   k-contiguous operands: buffer loads straight into LDS (no registers),
//     issued one k-step ahead; each lane fetches the global chunk that
//     belongs at its LDS slot, so the swizzle costs nothing.  Rows and k past
//     the matrix edge are given an out-of-range offset and read as zero.
//   m/n-contiguous operands: buffer loads into registers one k-step ahead,
//     transposed in registers (8 x 8 element blocks), then written to LDS.
// Epilogue: each wave parks its 128 x 128 fp32 results in LDS (two halves of
// 64 rows), then every lane handles 8 consecutive columns of a row: 16-byte
// loads of the residual / pre-activation, 16-byte stores.
#pragma once
#include "common.cuh"
#include <type_traits>

namespace blk {

enum EpiKind : int {
  EPI_STORE = 0,    // out = alpha*acc                         (element TO)
  EPI_RESID = 1,    // out = aux + alpha*acc                   (TO)
  EPI_RELU2 = 2,    // out = max(v,0)^2, v = alpha*acc           (TO)
  EPI_DRELU2 = 3,   // out = alpha*acc * 2*sqrt(aux), aux = max(u,0)^2 (TO)
  EPI_F32 = 4,      // out[split] = alpha*acc                  (float)
  EPI_F32_ADD = 5,  // out += alpha*acc                        (float)
  EPI_ROPE = 6,     // q, k columns: rotary then QK-norm; v columns stored (TO)
  EPI_DELTA = 7,    // out = alpha*acc, and delta = per-head row dot of out with aux (TO)
  EPI_LSE = 8,      // head forward: per row and 128-column segment, max and sum of exp of
                    // the logits (lse_part), and the logit at the row's target (nothing stored)
  EPI_DZ = 9,       // head backward: out = dscale/count * (exp(z - lse) - [col == target]) (TO)
};

struct GemmArgs {
  const void* A; long lda;
  const void* B; long ldb;
  int M, N, K;
  int k_split;          // k-range per split (multiple of BK); grid splits = ceil(K / k_split)
  int tiles_m, tiles_n;
  int nsplit;           // splits (the persistent eight-wave kernels walk tiles_m * tiles_n * nsplit tiles)
  void* out; long ldo;  // EPI_F32: split s writes out + s*M*ldo
  void* out2; long ldo2;
  const void* aux; long ldaux;
  float alpha;
  // fp8 operands: per-tensor absolute maxima (float bits); the epilogue
  // multiplies by (amax_a/448) * (amax_b/448) (a zero amax counts as 448)
  const unsigned* amax_a;
  const unsigned* amax_b;
  // EPI_ROPE: angle table cs[t*64 + i] = (cos, sin), QK-norm factors
  // rho[(which*M + row)*H + head], tokens per sequence T, heads H, width C,
  // key/value heads G (columns [0, C) q, [C, C + 128G) k, then v).
  // EPI_DELTA: delta[(b*H + head)*T + t] for row = b*T + t.
  const float2* cs;
  float* rho;
  float* delta;
  unsigned* amax_out;   // fp8 mode: absolute maximum of the stored output (float bits), or null
  int T, H, C, G;
  float eps;
  // EPI_LSE / EPI_DZ (language-model head; rows = tokens, columns = vocabulary):
  // tgt[row] target id (counted when 0 <= tgt < N); lse_part[row*nseg + col/128]
  // = (max, sum exp(z - max)) of a 128-column segment; tgt_logit[row] = z at
  // the target; lse_in[row] the row's log-sum-exp; *count the counted rows;
  // dscale the upstream gradient of the mean loss.
  const int* tgt;
  float2* lse_part;
  int nseg;
  float* tgt_logit;
  const float* lse_in;
  const int* count;
  float dscale;
};

template <typename TI> struct GemmTile {
  static constexpr int ELEM = 16 / sizeof(TI);   // elements per 16-byte chunk
  static constexpr int BK = 8 * ELEM;            // 128 bytes of k per row
  static constexpr int BM = 256, BN = 256, NT = 256;
  static constexpr int ROWB = 128;               // LDS bytes per tile row
  static constexpr int SLAB = (BM + BN) * ROWB;  // one stage, A then B
  static constexpr int LDS = 2 * SLAB;           // 128 KiB
};

// buffer resources (i32x4, make_rsrc, raw_buffer_load_lds): common.cuh

// ---- staging ------------------------------------------------------------------
// k-contiguous slab of R rows: 8 chunks per row, R*8 chunks, 64 per wave issue.
// Each lane's LDS slot is fixed (slot = issue base + lane); the lane fetches
// the global chunk that the swizzle puts there.  The row part of the global
// offset is computed once; each k-step adds k0.
template <typename TI, int R>
struct DirectStager {
  static constexpr int ELEM = GemmTile<TI>::ELEM;
  static constexpr int PER_WAVE = R * 8 / 4;       // chunks per wave
  static constexpr int NI = PER_WAVE / 64;         // issues per wave
  uint32_t row_off[NI];                            // byte offset of (row, chunk) at k = 0
  int kel[NI];                                     // element offset of the chunk along k
  bool row_ok[NI];

  __device__ __forceinline__ void init(long ld, int r0, int rows_valid, int wave, int lane) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int p = wave * PER_WAVE + i * 64 + lane;
      const int row = p >> 3, c = (p & 7) ^ swz(row, 8);
      row_ok[i] = r0 + row < rows_valid;
      kel[i] = c * ELEM;
      row_off[i] = (uint32_t)(((long)(r0 + row) * ld + c * ELEM) * sizeof(TI));
    }
  }
  // k0 >= k_end (past the last k-step) reads nothing: every offset is out of range
  __device__ __forceinline__ void issue(char* lds, i32x4 rs, uint32_t oob, int k0, int k_end, int wave) const {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const bool ok = row_ok[i] && (k0 + kel[i] < k_end);
      const uint32_t off = ok ? row_off[i] + (uint32_t)(k0 * (int)sizeof(TI)) : oob;
      lds_u32* dst = (lds_u32*)(lds + __builtin_amdgcn_readfirstlane(wave * PER_WAVE + i * 64) * 16);
      raw_buffer_load_lds(rs, dst, 16, (int)off, 0, 0, 0);
    }
  }
};

// m-contiguous slab of R rows (of the m/n index) x BK of k: ELEM x ELEM blocks.
template <typename TI, int R>
struct StageTrans {
  static constexpr int ELEM = GemmTile<TI>::ELEM;
  static constexpr int RB = R / ELEM;
  static constexpr int NB = (GemmTile<TI>::BK / ELEM) * RB / GemmTile<TI>::NT;   // blocks per thread
  u32x4 reg[NB > 0 ? NB * ELEM : 1];

  __device__ __forceinline__ void load(i32x4 rs, uint32_t oob, long ld, int r0, int rows_valid, int k0, int k_end) {
    static_assert(NB >= 1, "slab too small for the transposing stager");
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int blkid = threadIdx.x + b * GemmTile<TI>::NT;
      const int rb = blkid % RB, kb = blkid / RB;
      const int gr = r0 + rb * ELEM;
#pragma unroll
      for (int i = 0; i < ELEM; ++i) {
        const int gk = k0 + kb * ELEM + i;
        const uint32_t off = (gr < rows_valid && gk < k_end) ? (uint32_t)(((long)gk * ld + gr) * sizeof(TI)) : oob;
        reg[b * ELEM + i] = raw_buffer_load_b128(rs, (int)off, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(char* lds) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int blkid = threadIdx.x + b * GemmTile<TI>::NT;
      const int rb = blkid % RB, kb = blkid / RB;
      u32x4 tr[ELEM];
      transpose_chunks(&reg[b * ELEM], tr, (TI*)nullptr);
#pragma unroll
      for (int j = 0; j < ELEM; ++j) st16(lds + tile_off(rb * ELEM + j, kb, 8), tr[j]);
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

// Index v of a workgroup (or of a persistent grid's tile walk) -> logical
// tile: workgroups are dealt round robin to the 8 XCDs, so index v runs on
// XCD v % 8; the remap gives XCD x the contiguous run of logical tiles that
// starts at x q + min(x, r) (q = total / 8, r = total % 8; the first r XCDs
// take q + 1), which is exactly the number of indices v < total with
// v % 8 = x, so the map is a bijection for any total.
__device__ __forceinline__ int xcd_run(int v, int total) {
  const int q = total / 8, r = total % 8, x = v % 8;
  return x * q + min(x, r) + v / 8;
}
// Workgroup index -> (tile_m, tile_n, split): the XCD remap, then tiles are
// walked in groups of GROUP m-tiles so that an XCD's concurrent tiles share A
// rows and B columns in its L2 (and, for split-K weight gradients, one
// k-slice).
__device__ __forceinline__ void tile_coords(const GemmArgs& g, int& tm, int& tn, int& split, int GROUP = 8) {
  const int per_split = g.tiles_m * g.tiles_n;
  const int total = per_split * gridDim.y;
  const int pid = xcd_run(blockIdx.x + blockIdx.y * gridDim.x, total);
  split = pid / per_split;
  int t = pid % per_split;
  int group = t / (GROUP * g.tiles_n);
  int first_m = group * GROUP;
  int gsize = min(g.tiles_m - first_m, GROUP);
  int in_group = t % (GROUP * g.tiles_n);
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}
// The same for tile v of a persistent grid of workgroups that walk the
// total tiles in steps of the grid size: workgroup b runs on XCD b % 8, so
// with a grid that is a multiple of 8 (or no larger than the tile count's
// one round) tile v = b + i * grid lands on the same XCD for every i, and
// the remap gives each XCD a contiguous run of logical tiles exactly as for
// one workgroup per tile.
__device__ __forceinline__ void tile_coords_v(const GemmArgs& g, int v, int total, bool persistent, int& tm, int& tn,
                                              int& split, int GROUP = 8) {
  const int per_split = g.tiles_m * g.tiles_n;
  int pid = v;
  if (!persistent || gridDim.x % 8 == 0 || total <= (int)gridDim.x) pid = xcd_run(v, total);
  split = pid / per_split;
  int t = pid % per_split;
  int group = t / (GROUP * g.tiles_n);
  int first_m = group * GROUP;
  int gsize = min(g.tiles_m - first_m, GROUP);
  int in_group = t % (GROUP * g.tiles_n);
  tm = first_m + in_group % gsize;
  tn = in_group / gsize;
}

// ---- epilogue ------------------------------------------------------------------
// Position of token row `row` in its sequence of T (a mask when T is a power of two).
__device__ __forceinline__ int seq_pos(int row, int T) { return (T & (T - 1)) == 0 ? (row & (T - 1)) : row % T; }

// Output stores; NT marks them non-temporal (streamed past the caches).
template <bool NT>
__device__ __forceinline__ void st16_out(void* p, u32x4 v) {
  if constexpr (NT) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
  else st16(p, v);
}

// 8 consecutive results of one row (fp32, already scaled) -> memory.
template <typename TO, int EPI, bool NT = false>
__device__ __forceinline__ void epi8(const GemmArgs& g, int split, int row, int col, float* f, float& mx,
                                     const u32x4* pre = nullptr) {
  if constexpr (EPI == EPI_F32 || EPI == EPI_F32_ADD) {
    float* p = static_cast<float*>(g.out) + (EPI == EPI_F32 ? (long)split * g.M * g.ldo : 0L) + (long)row * g.ldo + col;
    u32x4 a = Chunk<float>::pack(f), b = Chunk<float>::pack(f + 4);
    if constexpr (EPI == EPI_F32_ADD) {
      float o[8];
      Chunk<float>::unpack(ld16(p), o);
      Chunk<float>::unpack(ld16(p + 4), o + 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] += f[e];
      a = Chunk<float>::pack(o);
      b = Chunk<float>::pack(o + 4);
    }
    st16(p, a);
    st16(p + 4, b);
  } else if constexpr (EPI == EPI_DZ) {
    const int t = g.tgt[row];
    const bool counted = t >= 0 && t < g.N;
    const float sc = counted ? g.dscale / (float)max(*g.count, 1) : 0.f;
    const float ls = g.lse_in[row];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float p = __builtin_amdgcn_exp2f((f[e] - ls) * 1.4426950408889634f);
      if (col + e == t) p -= 1.f;
      f[e] = p * sc;
    }
    constexpr int EL = Chunk<TO>::N;
    TO* o = static_cast<TO*>(g.out) + (long)row * g.ldo + col;
#pragma unroll
    for (int h = 0; h < 8 / EL; ++h) st16_out<NT>(o + h * EL, Chunk<TO>::pack(f + h * EL));
  } else if constexpr (EPI == EPI_ROPE) {
    // 16 consecutive lanes (a DPP row) hold one 128-wide head of the row (8
    // columns each); rotary pairs (i, i + 64) sit 8 lanes apart.  pre, if
    // given, holds this lane's 16 floats of the angle table (cos, sin of its
    // 8 column pairs), loaded ahead by the caller.
    constexpr int EL = Chunk<TO>::N;
    TO* o = static_cast<TO*>(g.out) + (long)row * g.ldo + col;
    // 0 q, 1 k, 2 v (uniform over the 16 lanes); hd the head within its part
    const int which = col < g.C ? 0 : (col < g.C + 128 * g.G ? 1 : 2);
    const int hd = (col - (which == 0 ? 0 : g.C)) / 128;
    if (which < 2) {
      const int cg = (col % 128) >> 3;    // this lane's 8-column group in the head
      float c8[16];
      if (pre) {
#pragma unroll
        for (int h = 0; h < 4; ++h) Chunk<float>::unpack(pre[h], c8 + 4 * h);
      } else {
        const float* csp = reinterpret_cast<const float*>(g.cs + (long)seq_pos(row, g.T) * 64 + (cg & 7) * 8);
#pragma unroll
        for (int h = 0; h < 4; ++h) Chunk<float>::unpack(ld16(csp + 4 * h), c8 + 4 * h);
      }
      float ss = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float other = dpp_mov<DPP_XOR8>(f[e]);
        const float c = c8[2 * e], sn = c8[2 * e + 1];
        // first half: z1 = own, z2 = partner; second half: z1 = partner, z2 = own
        f[e] = cg < 8 ? f[e] * c - other * sn : other * sn + f[e] * c;
        ss += f[e] * f[e];
      }
      ss = row16_sum(ss);
      const float r = __builtin_amdgcn_rsqf(ss / 128.f + g.eps);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] *= r;
      if (cg == 0) g.rho[((long)which * g.M + row) * g.H + hd] = r;
    }
#pragma unroll
    for (int h = 0; h < 8 / EL; ++h) st16_out<NT>(o + h * EL, Chunk<TO>::pack(f + h * EL));
  } else {
    constexpr int EL = Chunk<TO>::N;     // 8 bf16 or 4 float per chunk
    TO* o = static_cast<TO*>(g.out) + (long)row * g.ldo + col;
    if constexpr (EPI == EPI_RESID || EPI == EPI_DRELU2) {
      const TO* x = static_cast<const TO*>(g.aux) + (long)row * g.ldaux + col;
      float xv[8];
#pragma unroll
      for (int h = 0; h < 8 / EL; ++h) Chunk<TO>::unpack(pre ? pre[h] : ld16(x + h * EL), xv + h * EL);
      // ReLU^2 derivative 2 max(u,0) recovered from the stored a = max(u,0)^2
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = (EPI == EPI_RESID) ? xv[e] + f[e] : f[e] * 2.f * __builtin_amdgcn_sqrtf(xv[e]);
    }
    if constexpr (EPI == EPI_RELU2) {
#pragma unroll
      for (int e = 0; e < 8; ++e) { const float p = fmaxf(f[e], 0.f); f[e] = p * p; }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(f[e]));
#pragma unroll
    for (int h = 0; h < 8 / EL; ++h) st16_out<NT>(o + h * EL, Chunk<TO>::pack(f + h * EL));
    if constexpr (EPI == EPI_DELTA) {
      // the dot uses the stored (rounded) values, as the attention kernels read them
      const TO* x = static_cast<const TO*>(g.aux) + (long)row * g.ldaux + col;
      float xv[8], rv[8];
#pragma unroll
      for (int h = 0; h < 8 / EL; ++h) {
        Chunk<TO>::unpack(pre ? pre[h] : ld16(x + h * EL), xv + h * EL);
        Chunk<TO>::unpack(Chunk<TO>::pack(f + h * EL), rv + h * EL);
      }
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) d += rv[e] * xv[e];
      d = row16_sum(d);
      if ((col & 127) == 0) {
        const long b = row / g.T, t = row % g.T;
        g.delta[(b * g.H + col / 128) * g.T + t] = d;
      }
    }
  }
}

// Staging area of one wave's half tile: 64 rows x 128 fp32 (32 KiB), rows of
// 32 chunks; chunk c of row r at c ^ (8 * bit 2 of r) so that the two
// half-waves (rows r and r + 4) write disjoint bank halves.
__device__ __forceinline__ int epi_off(int row, int chunk) { return row * 512 + ((chunk ^ (((row >> 2) & 1) << 3)) << 4); }

template <typename TO, int EPI>
__device__ __forceinline__ void epilogue(const GemmArgs& g, f32x16 (&acc)[4][4], char* smem, int m0, int n0,
                                         int split, int wave, int lane) {
  const int wm = wave >> 1, wn = wave & 1;
  float alpha = g.alpha;
  if (g.amax_a) {
    const float a = __uint_as_float(*g.amax_a), b = __uint_as_float(*g.amax_b);
    alpha *= (a > 0.f ? a / 448.f : 1.f) * (b > 0.f ? b / 448.f : 1.f);
  }
  char* wreg = smem + wave * 32768;
  float mx = 0.f;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = ii * 32 + acc_row(r, lane), col = j * 32 + (lane & 31);
          *reinterpret_cast<float*>(wreg + epi_off(row, col >> 2) + (col & 3) * 4) = acc[2 * pass + ii][j][r] * alpha;
        }
    __syncthreads();
#pragma unroll 4
    for (int it = 0; it < 16; ++it) {
      const int q = it * 64 + lane;
      const int row = q >> 4, cg = q & 15;
      float f[8];
      Chunk<float>::unpack(ld16(wreg + epi_off(row, 2 * cg)), f);
      Chunk<float>::unpack(ld16(wreg + epi_off(row, 2 * cg + 1)), f + 4);
      const int grow = m0 + wm * 128 + pass * 64 + row;
      const int gcol = n0 + wn * 128 + cg * 8;
      if (grow < g.M && gcol < g.N) epi8<TO, EPI>(g, split, grow, gcol, f, mx);
    }
  }
  if (g.amax_out) amax_publish<TO>(g.amax_out, mx);
}

// ---- main body -------------------------------------------------------------------
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

  const uint32_t bytesA = clamp_bytes((KA ? (long)g.M * g.lda : (long)g.K * g.lda) * (long)sizeof(TI));
  const uint32_t bytesB = clamp_bytes((KB ? (long)g.N * g.ldb : (long)g.K * g.ldb) * (long)sizeof(TI));
  const i32x4 rsA = make_rsrc(g.A, bytesA), rsB = make_rsrc(g.B, bytesB);

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  DirectStager<TI, G::BM> da;
  DirectStager<TI, G::BN> db;
  StageTrans<TI, G::BM> ta;
  StageTrans<TI, G::BN> tb;
  if constexpr (KA) da.init(g.lda, m0, g.M, wave, lane);
  if constexpr (KB) db.init(g.ldb, n0, g.N, wave, lane);
  auto issue = [&](int stage, int k0) {
    char* s = smem + stage * G::SLAB;
    if constexpr (KA) da.issue(s, rsA, bytesA, k0, kend, wave);
    else ta.load(rsA, bytesA, g.lda, m0, g.M, k0, kend);
    if constexpr (KB) db.issue(s + G::BM * G::ROWB, rsB, bytesB, k0, kend, wave);
    else tb.load(rsB, bytesB, g.ldb, n0, g.N, k0, kend);
  };
  auto commit = [&](int stage) {   // register-staged operands -> LDS
    char* s = smem + stage * G::SLAB;
    if constexpr (!KA) ta.store(s);
    if constexpr (!KB) tb.store(s + G::BM * G::ROWB);
  };

  constexpr int KS = G::BK / MM::KI;          // MFMA k-substeps per k-step
  if (nk > 0) {
    issue(0, kbeg);
    commit(0);
  }
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt is complete (own loads, then everyone's); stage kt-1 is free
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    // next stage (past the end: out-of-range offsets, nothing is read)
    issue((kt + 1) & 1, kbeg + (kt + 1) * G::BK);
    const char* cur = smem + (kt & 1) * G::SLAB;
    // fragments of substep ks+1 are read while the MFMAs of substep ks run
    typename MM::frag fa[2][4], fb[2][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[0][i] = load_frag<TI>(cur, wm * 128 + i * 32, 0, lane);
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[0][j] = load_frag<TI>(cur + G::BM * G::ROWB, wn * 128 + j * 32, 0, lane);
    __builtin_amdgcn_sched_group_barrier(0x020, 16, 0);      // next stage's 16 global loads first
    __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);       // then substep 0's LDS reads
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c = ks & 1, n = c ^ 1;
      if (ks + 1 < KS) {
#pragma unroll
        for (int i = 0; i < 4; ++i) fa[n][i] = load_frag<TI>(cur, wm * 128 + i * 32, ks + 1, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[n][j] = load_frag<TI>(cur + G::BM * G::ROWB, wn * 128 + j * 32, ks + 1, lane);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = MM::mma(fa[c][i], fb[c][j], acc[i][j]);
      if (ks + 1 < KS) {
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 2 MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // 1 LDS read
        }
      } else {
        __builtin_amdgcn_sched_group_barrier(0x008, 16, 0);
      }
    }
    if (kt + 1 < nk) commit((kt + 1) & 1);
  }
  // the past-the-end loads write zeros into LDS: let them land before the
  // epilogue reuses LDS
  __builtin_amdgcn_s_waitcnt(0);
  epilogue<TO, EPI>(g, acc, smem, m0, n0, split, wave, lane);
}

// ---- eight-wave ping-pong body (both operands k-contiguous) --------------------
// Same 256 x 256 workgroup tile and LDS slab layout as the four-wave body
// (two stages of 128-byte rows), eight waves.  Wave w = 4*grp + q computes
// rows (q>>1)*128 + grp*64 .. +64 and columns (q&1)*128 .. +128 (2 x 4 MFMA
// blocks).  The two groups (waves w and w+4 share a SIMD) take turns one
// phase apart: while one group runs the MFMAs of half a k-step from
// registers, the other reads its fragments of that half from LDS, so each
// SIMD's matrix pipe has a wave feeding it while the other waits on LDS.
// Per k-step kt (grp 0 | grp 1):
//   A0: issue half of kt+1's A rows, read (kt, half 0) | MFMAs (kt-1, 1), half of kt+1's B rows
//   B0: MFMAs (kt, 0), the other half of the A rows   | read (kt, 0)
//   A1: read (kt, 1)                                 | MFMAs (kt, 0), the other half of the B rows
//   B1: MFMAs (kt, 1), wait for kt+1                 | read (kt, 1), wait for kt+1
// Spreading each stage's loads over two phases keeps a phase from holding
// all 64 KiB of them: with every load in A0 the vector-memory path backed up
// and stalled the MFMAs interleaved with them (d20 step 9.47 -> 9.25 ms;
// fewer in the first part, or the reads ahead of the loads, were slower).
// Stage kt+1 goes global -> LDS (whole 128-byte rows: one load instruction
// covers 8 full cache lines) into the slot stage kt-1 vacated.  Requires K
// and the split length to be multiples of the k-step and both leading
// dimensions to be multiples of 128 bytes, so row offsets leave the chunk
// bits free.  Output tiles are stored non-temporally: they are not read
// again by this kernel and would only evict operand lines from L2.
template <typename TI>
struct PPStager {
  i32x4 rs;        // buffer resource from the tile's first row
  uint32_t x;      // byte offset (k = 0) of this lane's chunk in the wave's first 8-row group
  uint32_t step;   // bytes between consecutive 8-row groups
  // LDS row R = 64q + 8j + lane/8 holds at chunk position lane%8 the global
  // chunk (lane%8) ^ swz(R) = (lane%8) ^ (lane/8) ^ j
  __device__ __forceinline__ void init(const void* p, long ld, long rows, int r0, int q, int lane) {
    const char* base = static_cast<const char*>(p) + (long)r0 * ld * (long)sizeof(TI);
    const long left = rows > r0 ? (rows - r0) * ld * (long)sizeof(TI) : 0L;
    rs = make_rsrc(base, (uint32_t)min(left, 0x7fffffffL));
    x = (uint32_t)((64 * q + (lane >> 3)) * ld * (long)sizeof(TI)) + (uint32_t)(((lane & 7) ^ (lane >> 3)) << 4);
    step = (uint32_t)(8 * ld * (long)sizeof(TI));
  }
  // rows past the matrix edge have offsets >= the resource size and read
  // zero; so does a whole stage past the end of k (live = false)
  template <int J0 = 0, int J1 = 8>
  __device__ __forceinline__ void issue(char* sub, int k0_bytes, bool live, int q) const {
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const uint32_t off = (x ^ (uint32_t)(j << 4)) + (uint32_t)j * step + (uint32_t)k0_bytes;
      lds_u32* dst = (lds_u32*)(sub + __builtin_amdgcn_readfirstlane((8 * q + j) * 1024));
      raw_buffer_load_lds(rs, dst, 16, live ? (int)off : (int)0x80000000u, 0, 0, 0);
    }
  }
};

// m/n-contiguous bf16 operands (weight gradients: A(m, k) = G[k][m]): the
// LDS sub-slab holds the tile as 64 k-rows x 256 elements (512 bytes, 32
// chunks); chunk c of row r sits at c ^ (2 (r & 7)), so the 4 rows x 2
// chunks one 16-lane transpose read touches fall on distinct banks.
__device__ __forceinline__ int toff(int row, int chunk) { return row * 512 + ((chunk ^ ((row & 7) << 1)) << 4); }

// One operand's share of a stage for wave q: k-rows 16q .. 16q+15, two
// 512-byte rows (4 full cache lines each) per 1 KiB load.
struct PPStagerT {
  const char* base;  // (k = kbeg, first column of the tile)
  long left;         // bytes from base to the end of the matrix
  uint32_t x;        // byte offset of this lane's row in a stage, load 0
  uint32_t ldb;      // bytes per k-row
  uint32_t cl;       // this lane's chunk byte offset before the per-load swizzle term
  __device__ __forceinline__ void init(const void* p, long ld, long K, int c0, int kbeg, int q, int lane) {
    const long first = (long)kbeg * ld + c0;
    base = static_cast<const char*>(p) + first * 2;
    left = ((long)K * ld - first) * 2;
    ldb = (uint32_t)(ld * 2);
    x = (uint32_t)(16 * q + (lane >> 5)) * ldb;
    // LDS row R = 16q + 2j + lane/32 holds at chunk position lane%32 the
    // global chunk (lane%32) ^ 2 (R & 7), and R & 7 = (2j & 7) | lane/32
    cl = (uint32_t)(((lane & 31) ^ ((lane >> 5) << 1)) << 4);
  }
  // The buffer resource starts at the stage's first k-row, so offsets stay
  // below 64 rows whatever the matrix size.  Columns past the matrix edge
  // read in-bounds neighbours or zero; they only feed outputs the epilogue
  // drops.  k past the end (live = false) reads zero.  The loads are the
  // assembly form (dma16): the fragments of this operand come from the LDS
  // transpose read, and after a direct-to-LDS load the compiler knows of it
  // would make that read wait for the stage just issued; the body waits for
  // each stage explicitly.
  template <int J0 = 0, int J1 = 8>
  __device__ __forceinline__ void issue(char* sub, int krel, bool live, int q) const {
    const long adv = (long)krel * ldb;
    const i32x4 rs = make_rsrc(base + adv, (uint32_t)max(0L, min(left - adv, 0x7fffffffL)));
#pragma unroll
    for (int j = J0; j < J1; ++j) {
      const uint32_t off = x + (uint32_t)(2 * j) * ldb + (cl ^ (uint32_t)(((2 * j) & 7) << 5));
      lds_u32* dst = (lds_u32*)(sub + (8 * q + j) * 1024);
      dma16(rs, dst, live ? off : 0x80000000u);
    }
  }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// MFMA 32x32x16 fragment of 32 columns (col0..) at k-substep ks from a
// k-row sub-slab, by two LDS transpose reads: in each 16-lane group the
// lanes address a 4-row x 16-column block and lane s receives column s of
// it.  Lane l gets column col0 + l%32 and the k-slots 4h..4h+3, 8+4h..8+4h+3
// (h = l/32) of the substep: a fixed permutation of the MFMA's k order,
// the same for both operands, so the product is unchanged.
__device__ __forceinline__ bf16x8 frag_t(const char* sub, int col0, int ks, int lane) {
  const int g = (lane >> 4) & 3, s = lane & 15;
  const int row = ks * 16 + 4 * (g >> 1) + (s >> 2);
  const int col = col0 + 16 * (g & 1) + 4 * (s & 3);
  const char* p0 = sub + toff(row, col >> 3) + (col & 7) * 2;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p0);
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 8 * 512));   // rows + 8: same swizzle
  const s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// Workgroup barrier that is also a hard scheduling boundary: no instruction
// (MFMAs included) moves across it, and no memory wait is implied.
__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Head forward epilogue: the 16 lanes holding one 128-column segment of a
// row (8 logits each) reduce it to (max, sum exp(z - max)); the lane whose
// columns hold the row's target keeps that logit.  Every lane takes part in
// the shuffles; columns past the vocabulary count as -inf (the vocabulary
// is a multiple of 8, so a lane's 8 columns are all in or all out).
__device__ __forceinline__ void head_lse8(const GemmArgs& g, int row, int col, const float* f) {
  const bool ok = row < g.M && col < g.N;
  float m = -INFINITY;
  if (ok) {
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, f[e]);
  }
  m = row16_max(m);
  float l = 0.f;
  if (ok) {
#pragma unroll
    for (int e = 0; e < 8; ++e) l += __builtin_amdgcn_exp2f((f[e] - m) * 1.4426950408889634f);
    const int t = g.tgt[row];
    if (t >= col && t < col + 8) g.tgt_logit[row] = f[t - col];
  }
  l = row16_sum(l);
  if (ok && (col & 127) == 0) g.lse_part[(long)row * g.nseg + (col >> 7)] = make_float2(m, l);
}

// Epilogues that read a bf16 operand of their own (residual, stored
// activation, o for delta) take it from registers loaded before the
// epilogue starts: pre[pass][it] is the 16-byte chunk of the row segment
// that iteration it of pass pass handles (zero outside the matrix).
template <typename TO, int EPI>
struct EpiAux {
  static constexpr bool on = (EPI == EPI_RESID || EPI == EPI_DRELU2 || EPI == EPI_DELTA) && sizeof(TO) == 2;
};
template <typename TO, int EPI>
__device__ __forceinline__ void epi_prefetch(const GemmArgs& g, u32x4 (&pre)[2][8], int m0, int n0, int wave,
                                             int lane) {
  if constexpr (EpiAux<TO, EPI>::on) {
    const int grp = wave >> 2, q = wave & 3;
    const int rbase = m0 + (q >> 1) * 128 + grp * 64, cbase = n0 + (q & 1) * 128;
    const TO* aux = static_cast<const TO*>(g.aux);
#pragma unroll
    for (int pass = 0; pass < 2; ++pass)
#pragma unroll
      for (int it = 0; it < 8; ++it) {
        const int qq = it * 64 + lane;
        const int grow = rbase + pass * 32 + (qq >> 4), gcol = cbase + (qq & 15) * 8;
        pre[pass][it] = (grow < g.M && gcol < g.N) ? ld16(aux + (long)grow * g.ldaux + gcol) : u32x4{0u, 0u, 0u, 0u};
      }
  }
}

// stage: 64 KiB of LDS (one operand slot), 8 KiB per wave
template <typename TO, int EPI>
__device__ __forceinline__ void epilogue_pp(const GemmArgs& g, f32x16 (&acc)[2][4], char* stage, int m0, int n0,
                                            int split, int wave, int lane, const u32x4 (&pre)[2][8]) {
  const int grp = wave >> 2, q = wave & 3;
  float alpha = g.alpha;
  if (g.amax_a) {
    const float a = __uint_as_float(*g.amax_a), b = __uint_as_float(*g.amax_b);
    alpha *= (a > 0.f ? a / 448.f : 1.f) * (b > 0.f ? b / 448.f : 1.f);
  }
  // each wave parks 16 rows x 128 fp32 (8 KiB) at a time in its own region
  // (the other operand slot takes the next tile's first stage meanwhile);
  // LDS accesses of one wave complete in order, so no barrier is needed
  char* wreg = stage + wave * 8192;
  const int rbase = m0 + (q >> 1) * 128 + grp * 64, cbase = n0 + (q & 1) * 128;
  float mx = 0.f;
  // EPI_ROPE on a q or k head (the wave's 128 columns are one head): the
  // angle-table chunks of step s = 8 pass + it are loaded during step s - 2
  bool rot = false;
  if constexpr (EPI == EPI_ROPE) rot = cbase < g.C + 128 * g.G;
  u32x4 csr[2][4];
  auto cs_load = [&](int s) {
    const int qq = (s & 7) * 64 + lane;
    const int grow = rbase + (s >> 3) * 32 + (qq >> 4), cg = qq & 7;
    const float* p = reinterpret_cast<const float*>(g.cs + (long)seq_pos(grow, g.T) * 64 + cg * 8);
#pragma unroll
    for (int h = 0; h < 4; ++h) csr[s & 1][h] = ld16(p + 4 * h);
  };
  if (rot) {
    cs_load(0);
    cs_load(1);
  }
  // registers 8h .. 8h+7 of a 32-row block hold its rows 16h .. 16h+15
#pragma unroll
  for (int pass = 0; pass < 2; ++pass)
#pragma unroll
  for (int half = 0; half < 2; ++half) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 8 * half; r < 8 * half + 8; ++r) {
        const int row = acc_row(r, lane) - 16 * half, col = j * 32 + (lane & 31);
        *reinterpret_cast<float*>(wreg + epi_off(row, col >> 2) + (col & 3) * 4) = acc[pass][j][r] * alpha;
      }
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      const int it = 4 * half + i4;           // step of the pass: rows 4 it .. 4 it + 3
      const int qq = i4 * 64 + lane;
      const int row = qq >> 4, cg = qq & 15;
      float f[8];
      Chunk<float>::unpack(ld16(wreg + epi_off(row, 2 * cg)), f);
      Chunk<float>::unpack(ld16(wreg + epi_off(row, 2 * cg + 1)), f + 4);
      const int grow = rbase + pass * 32 + 16 * half + row, gcol = cbase + cg * 8;
      if constexpr (EPI == EPI_LSE) head_lse8(g, grow, gcol, f);
      else if (grow < g.M && gcol < g.N) {
        // (the v heads do not read the ring)
        if constexpr (EPI == EPI_ROPE) epi8<TO, EPI, true>(g, split, grow, gcol, f, mx, csr[it & 1]);
        else epi8<TO, EPI, true>(g, split, grow, gcol, f, mx, EpiAux<TO, EPI>::on ? &pre[pass][it] : nullptr);
      }
      if (rot && pass * 8 + it + 2 < 16) cs_load(pass * 8 + it + 2);
    }
  }
  if (g.amax_out) amax_publish<TO>(g.amax_out, mx);
}

// TR: both operands m/n-contiguous (bf16 weight gradients), staged as k-rows
// and read through the LDS transpose read.
template <typename TI, typename TO, int EPI, bool TR = false>
__device__ __forceinline__ void gemm_pp_body(const GemmArgs& g) {
  typedef GemmTile<TI> G;
  typedef Mfma<TI> MM;
  static_assert(!TR || sizeof(TI) == 2, "transposed staging is for 16-bit operands");
  constexpr int HS = G::BK / MM::KI / 2;                              // MFMA substeps per half k-step
  constexpr int RD = 6 * HS * (sizeof(TI) == 1 || TR ? 2 : 1);        // LDS reads per read phase
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63;
  // wave-uniform: the group's branch and its buffer resource live in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2, q = wave & 3;

  // Persistent: the grid walks the tiles (all splits) in steps of its size;
  // while a tile's epilogue runs through operand slot 1, the next tile's
  // first stage loads into slot 0.  Not for E4M3 operands with an epilogue
  // that loads an operand of its own: beside that operand's registers the
  // next tile's state made them spill (58 registers, 14-35% slower); they run
  // one workgroup per tile (grid tiles x splits).
  constexpr bool PERSIST = !EpiAux<TO, EPI>::on || sizeof(TI) == 2;
  static_assert(8 * 8192 <= G::SLAB, "the epilogue's staging fits one operand slot");
  const int total = g.tiles_m * g.tiles_n * g.nsplit;
  int v = PERSIST ? (int)blockIdx.x : (int)(blockIdx.x + blockIdx.y * gridDim.x);
  if (v >= total) return;
  int m0, n0, split, kbeg, nk;
  // grp 0 stages the A operand, grp 1 the B operand
  typename std::conditional<TR, PPStagerT, PPStager<TI>>::type st;
  auto setup = [&](int tile) {
    int tm, tn;
    tile_coords_v(g, tile, total, PERSIST, tm, tn, split, 4);
    m0 = tm * G::BM;
    n0 = tn * G::BN;
    kbeg = split * g.k_split;
    nk = (min(g.K, kbeg + g.k_split) - kbeg) / G::BK;
    if constexpr (TR) {
      if (grp == 0) st.init(g.A, g.lda, g.K, m0, kbeg, q, lane);
      else st.init(g.B, g.ldb, g.K, n0, kbeg, q, lane);
    } else {
      if (grp == 0) st.init(g.A, g.lda, g.M, m0, q, lane);
      else st.init(g.B, g.ldb, g.N, n0, q, lane);
    }
  };
  auto issue = [&](int kt) {
    char* sub = smem + (kt & 1) * G::SLAB + grp * (G::BM * G::ROWB);
    if constexpr (TR) st.issue(sub, kt * G::BK, kt < nk, q);
    else st.issue(sub, (kbeg + kt * G::BK) * (int)sizeof(TI), kt < nk, q);
  };
  // a stage's eight loads per wave in two parts of L0 and 8 - L0, issued in
  // different phases (see the schedule above)
  constexpr int L0 = 4;
  auto issue0 = [&](int kt) {
    char* sub = smem + (kt & 1) * G::SLAB + grp * (G::BM * G::ROWB);
    if constexpr (TR) st.template issue<0, L0>(sub, kt * G::BK, kt < nk, q);
    else st.template issue<0, L0>(sub, (kbeg + kt * G::BK) * (int)sizeof(TI), kt < nk, q);
  };
  auto issue1 = [&](int kt) {
    char* sub = smem + (kt & 1) * G::SLAB + grp * (G::BM * G::ROWB);
    if constexpr (TR) st.template issue<L0, 8>(sub, kt * G::BK, kt < nk, q);
    else st.template issue<L0, 8>(sub, (kbeg + kt * G::BK) * (int)sizeof(TI), kt < nk, q);
  };
  constexpr int NMF = 8 * HS;                 // MFMAs per phase
  constexpr int P0 = NMF / L0, P1 = NMF / (8 - L0);

  const int arow = (q >> 1) * 128 + grp * 64, brow = (q & 1) * 128;
  f32x16 acc[2][4];
  typename MM::frag fa[HS][2], fb[HS][4];
  u32x4 pre[2][8];   // the epilogue's own operand, loaded while the last MFMAs run
  auto read = [&](int kt, int h) {
    const char* cur = smem + (kt & 1) * G::SLAB;
#pragma unroll
    for (int s = 0; s < HS; ++s) {
      if constexpr (TR) {
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[s][i] = frag_t(cur, arow + 32 * i, h * HS + s, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[s][j] = frag_t(cur + G::BM * G::ROWB, brow + 32 * j, h * HS + s, lane);
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) fa[s][i] = load_frag<TI>(cur, arow + 32 * i, h * HS + s, lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) fb[s][j] = load_frag<TI>(cur + G::BM * G::ROWB, brow + 32 * j, h * HS + s, lane);
      }
    }
  };
  auto mfma = [&]() {
#pragma unroll
    for (int s = 0; s < HS; ++s)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = MM::mma(fa[s][i], fb[s][j], acc[i][j]);
  };

  setup(v);
  if (nk > 0) issue(0);
  for (;;) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    // A stage past the end (kt + 1 == nk) is issued with out-of-range offsets:
    // it writes zeros into the free slot and keeps the loop free of branches
    // that would split the instruction schedule.
    if (nk > 0) {
      __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): stage 0 (and the last epilogue's stores)
      wg_barrier();
      if (grp == 0) {
        for (int kt = 0; kt < nk; ++kt) {
          issue0(kt + 1);
          read(kt, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, L0, 0);   // the first loads, then the LDS reads
          __builtin_amdgcn_sched_group_barrier(0x100, RD, 0);
          wg_barrier();
          issue1(kt + 1);
          mfma();
#pragma unroll
          for (int i = 0; i < 8 - L0; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, P1, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
          wg_barrier();
          read(kt, 1);
          wg_barrier();
          mfma();
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0): stage kt+1's A rows have landed
          wg_barrier();
        }
        epi_prefetch<TO, EPI>(g, pre, m0, n0, wave, lane);   // in flight while grp 1 finishes
        wg_barrier();   // grp 1 runs the last half-step's MFMAs
      } else {
        // the slot is refilled after the stage's last barrier, so each read
        // phase ends with its fragments in registers
        auto tail = [&](int kt, bool more) {
          read(kt, 0);
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
          wg_barrier();
          if (more) {
            issue1(kt + 1);
            mfma();
#pragma unroll
            for (int i = 0; i < 8 - L0; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, P1, 0);
              __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
          } else {
            mfma();
          }
          wg_barrier();
          read(kt, 1);
          __builtin_amdgcn_sched_barrier(0);
          __builtin_amdgcn_s_waitcnt(0);        // fragments, and stage kt+1's B rows
          wg_barrier();
        };
        issue(1);
        wg_barrier();
        tail(0, false);
        for (int kt = 1; kt < nk; ++kt) {
          issue0(kt + 1);
          mfma();
#pragma unroll
          for (int i = 0; i < L0; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, P0, 0);
            __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
          }
          wg_barrier();
          tail(kt, true);
        }
        mfma();
        epi_prefetch<TO, EPI>(g, pre, m0, n0, wave, lane);
        wg_barrier();
      }
    } else {
      epi_prefetch<TO, EPI>(g, pre, m0, n0, wave, lane);
    }
    // every staging load (the past-the-end one included) was waited for
    // inside the loops; after the barrier both slots are free: the next
    // tile's first stage goes to slot 0, this tile's epilogue through slot 1
    wg_barrier();
    if constexpr (PERSIST) {
      const int cm0 = m0, cn0 = n0, csplit = split;
      const int vn = v + (int)gridDim.x;
      if (vn < total) {
        setup(vn);
        if (nk > 0) issue(0);
      }
      epilogue_pp<TO, EPI>(g, acc, smem + G::SLAB, cm0, cn0, csplit, wave, lane, pre);
      if (vn >= total) break;
      v = vn;
    } else {
      epilogue_pp<TO, EPI>(g, acc, smem + G::SLAB, m0, n0, split, wave, lane, pre);
      break;
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
#define BLK_GEMM_PP_KERNEL(NAME, EPI, TO)                                         \
  template <typename T>                                                         \
  __global__ __launch_bounds__(512, 1) void NAME(GemmArgs g) {                   \
    gemm_pp_body<T, TO, EPI>(g);                                                \
  }

namespace blk {
BLK_GEMM_PP_KERNEL(gemm_qkv_fwd, EPI_ROPE, T)
BLK_GEMM_PP_KERNEL(gemm_o_fwd, EPI_RESID, T)
BLK_GEMM_PP_KERNEL(gemm_fc_fwd, EPI_RELU2, T)
BLK_GEMM_PP_KERNEL(gemm_proj_fwd, EPI_RESID, T)
BLK_GEMM_PP_KERNEL(gemm_proj_dgrad, EPI_DRELU2, T)
BLK_GEMM_PP_KERNEL(gemm_fc_dgrad, EPI_STORE, T)
BLK_GEMM_PP_KERNEL(gemm_o_dgrad, EPI_DELTA, T)
BLK_GEMM_PP_KERNEL(gemm_qkv_dgrad, EPI_STORE, T)
BLK_GEMM_KERNEL(gemm_proj_wgrad, false, false, EPI_F32, float)
BLK_GEMM_KERNEL(gemm_fc_wgrad, false, false, EPI_F32, float)
BLK_GEMM_KERNEL(gemm_o_wgrad, false, false, EPI_F32, float)
BLK_GEMM_KERNEL(gemm_qkv_wgrad, false, false, EPI_F32, float)
BLK_GEMM_KERNEL(gemm_proj_wgrad_acc, false, false, EPI_F32_ADD, float)
BLK_GEMM_KERNEL(gemm_fc_wgrad_acc, false, false, EPI_F32_ADD, float)
BLK_GEMM_KERNEL(gemm_o_wgrad_acc, false, false, EPI_F32_ADD, float)
BLK_GEMM_KERNEL(gemm_qkv_wgrad_acc, false, false, EPI_F32_ADD, float)
BLK_GEMM_KERNEL(gemm_head_wgrad, false, false, EPI_F32, float)
BLK_GEMM_KERNEL(gemm_head_wgrad_acc, false, false, EPI_F32_ADD, float)
}  // namespace blk

// bf16 weight gradients on the eight-wave body (k = tokens a multiple of 64).
#define BLK_GEMM_PPT_KERNEL(NAME, EPI)                                            \
  __global__ __launch_bounds__(512, 1) void NAME(GemmArgs g) {                   \
    gemm_pp_body<bf16, float, EPI, true>(g);                                    \
  }

namespace blk {
// language-model head: logits with the log-sum-exp epilogue, logits again
// with the softmax-gradient epilogue, the input gradient and the weight
// gradient (token count a multiple of 64; else the four-wave body)
__global__ __launch_bounds__(512, 1) void gemm_head_fwd(GemmArgs g) { gemm_pp_body<bf16, bf16, EPI_LSE>(g); }
__global__ __launch_bounds__(512, 1) void gemm_head_dz(GemmArgs g) { gemm_pp_body<bf16, bf16, EPI_DZ>(g); }
__global__ __launch_bounds__(512, 1) void gemm_head_dgrad(GemmArgs g) { gemm_pp_body<bf16, bf16, EPI_STORE>(g); }
BLK_GEMM_PPT_KERNEL(gemm_head_wgrad_pp, EPI_F32)
BLK_GEMM_PPT_KERNEL(gemm_head_wgrad_acc_pp, EPI_F32_ADD)
BLK_GEMM_PPT_KERNEL(gemm_proj_wgrad_pp, EPI_F32)
BLK_GEMM_PPT_KERNEL(gemm_fc_wgrad_pp, EPI_F32)
BLK_GEMM_PPT_KERNEL(gemm_o_wgrad_pp, EPI_F32)
BLK_GEMM_PPT_KERNEL(gemm_qkv_wgrad_pp, EPI_F32)
BLK_GEMM_PPT_KERNEL(gemm_proj_wgrad_acc_pp, EPI_F32_ADD)
BLK_GEMM_PPT_KERNEL(gemm_fc_wgrad_acc_pp, EPI_F32_ADD)
BLK_GEMM_PPT_KERNEL(gemm_o_wgrad_acc_pp, EPI_F32_ADD)
BLK_GEMM_PPT_KERNEL(gemm_qkv_wgrad_acc_pp, EPI_F32_ADD)
}  // namespace blk

// FP8 (E4M3) linear layers: every GEMM takes k-contiguous operands (weights
// and activations quantised row-major, or transposed for weight gradients).
#define BLK_GEMM8_KERNEL(NAME, EPI, TO)                                           \
  __global__ __launch_bounds__(256, 1) void NAME(GemmArgs g) {                   \
    gemm_body<fp8e4, TO, true, true, EPI>(g);                                   \
  }
#define BLK_GEMM8_PP_KERNEL(NAME, EPI, TO)                                        \
  __global__ __launch_bounds__(512, 1) void NAME(GemmArgs g) {                   \
    gemm_pp_body<fp8e4, TO, EPI>(g);                                            \
  }

namespace blk {
BLK_GEMM8_PP_KERNEL(gemm8_qkv_fwd, EPI_ROPE, bf16)
BLK_GEMM8_PP_KERNEL(gemm8_o_fwd, EPI_RESID, bf16)
BLK_GEMM8_PP_KERNEL(gemm8_fc_fwd, EPI_RELU2, bf16)
BLK_GEMM8_PP_KERNEL(gemm8_proj_fwd, EPI_RESID, bf16)
BLK_GEMM8_PP_KERNEL(gemm8_proj_dgrad, EPI_DRELU2, bf16)
BLK_GEMM8_PP_KERNEL(gemm8_fc_dgrad, EPI_STORE, bf16)
BLK_GEMM8_PP_KERNEL(gemm8_o_dgrad, EPI_DELTA, bf16)
BLK_GEMM8_PP_KERNEL(gemm8_qkv_dgrad, EPI_STORE, bf16)
BLK_GEMM8_KERNEL(gemm8_proj_wgrad, EPI_F32, float)
BLK_GEMM8_KERNEL(gemm8_fc_wgrad, EPI_F32, float)
BLK_GEMM8_KERNEL(gemm8_o_wgrad, EPI_F32, float)
BLK_GEMM8_KERNEL(gemm8_qkv_wgrad, EPI_F32, float)
BLK_GEMM8_KERNEL(gemm8_proj_wgrad_acc, EPI_F32_ADD, float)
BLK_GEMM8_KERNEL(gemm8_fc_wgrad_acc, EPI_F32_ADD, float)
BLK_GEMM8_KERNEL(gemm8_o_wgrad_acc, EPI_F32_ADD, float)
BLK_GEMM8_KERNEL(gemm8_qkv_wgrad_acc, EPI_F32_ADD, float)
// the same on the eight-wave body (token count a multiple of 128)
BLK_GEMM8_PP_KERNEL(gemm8_proj_wgrad_pp, EPI_F32, float)
BLK_GEMM8_PP_KERNEL(gemm8_fc_wgrad_pp, EPI_F32, float)
BLK_GEMM8_PP_KERNEL(gemm8_o_wgrad_pp, EPI_F32, float)
BLK_GEMM8_PP_KERNEL(gemm8_qkv_wgrad_pp, EPI_F32, float)
BLK_GEMM8_PP_KERNEL(gemm8_proj_wgrad_acc_pp, EPI_F32_ADD, float)
BLK_GEMM8_PP_KERNEL(gemm8_fc_wgrad_acc_pp, EPI_F32_ADD, float)
BLK_GEMM8_PP_KERNEL(gemm8_o_wgrad_acc_pp, EPI_F32_ADD, float)
BLK_GEMM8_PP_KERNEL(gemm8_qkv_wgrad_acc_pp, EPI_F32_ADD, float)
}  // namespace blk
