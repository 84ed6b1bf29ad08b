// Causal multi-head attention, head size 128, for gfx950 (flash-style: the
// T x T score matrix never reaches HBM).
//
// Forward: each wave owns 32 queries and walks key tiles.  It computes the
// TRANSPOSED score block S^T = K Q^T with MFMA 32x32, so the lane that holds
// column l%32 of S^T holds every score of one query: the running maximum and
// denominator of the online softmax are per-lane scalars (plus one exchange
// with lane l^32), and the rescale of the output accumulator O^T (d x query)
// is a per-lane multiply.  P^T feeds O^T += V^T P^T straight from registers:
// the MFMA k-slots of P^T are the keys this lane already holds, and V^T is
// read from LDS with the same key order.
//
// Backward (no atomics, deterministic): a pass over key tiles per query tile
// for dQ, and a pass over query tiles per key tile for dK and dV, both
// recomputing P from the saved log-sum-exp.
//
// (Causal multi-head attention with 128-dim heads: 7minutos.es nanochat
// article, section "Modelo, escalado y objetivo de speedrun"; QK-norm and
// rotary precede it: flicky.cc nanochat page, section on the model.)
#pragma once
#include "common.cuh"

namespace blk {

constexpr int HD = 128;   // head size

template <typename T> struct AttnCfg {
  static constexpr int EL = 16 / sizeof(T);          // elements per chunk
  static constexpr int RT = (sizeof(T) == 2) ? 64 : 32;  // keys (queries) per LDS tile
  static constexpr int NB = RT / 32;                  // 32-wide MFMA blocks per tile
  static constexpr int RCH = HD * sizeof(T) / 16;     // chunks per row of a [rows][128] tile
  static constexpr int ROWT = RT * 128 * sizeof(T);   // bytes of a [RT][128] tile
  static constexpr int TCH = 8;                       // chunks per row of a [128][RT] tile (128 B)
  static constexpr int TRT = 128 * 128;               // bytes of a [128][RT] tile
};

// ---- staging helpers (256 threads) -----------------------------------------

// Rows r0..r0+RT-1 (valid < rvalid) of a [*, ld] matrix, 128 columns from src,
// into an LDS [RT][128] tile (row layout, swizzled).  Rows past rvalid are 0.
template <typename T>
__device__ __forceinline__ void stage_rows(char* lds, const T* src, long ld, int r0, int rvalid) {
  typedef AttnCfg<T> A;
  constexpr int NCH = A::RT * A::RCH / 256;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
    int idx = threadIdx.x + i * 256;
    int row = idx / A::RCH, ch = idx % A::RCH;
    u32x4 v = u32x4{0, 0, 0, 0};
    if (r0 + row < rvalid) v = ld16(src + (long)(r0 + row) * ld + ch * A::EL);
    st16(lds + tile_off(row, ch, A::RCH), v);
  }
}

// The same rows, transposed into an LDS [128][RT] tile (rows = the 128
// columns of src; each row holds the RT tile rows).  Each thread moves
// half-blocks of EL/2 rows x EL columns.
template <typename T>
__device__ __forceinline__ void stage_trans(char* lds, const T* src, long ld, int r0, int rvalid) {
  typedef AttnCfg<T> A;
  constexpr int HB = A::EL / 2;                 // rows per half block (4 bf16 / 2 f32)
  constexpr int NCB = HD / A::EL;               // column blocks (16 / 32)
  constexpr int NHB = (A::RT / HB) * NCB;       // half blocks (256 / 512)
#pragma unroll
  for (int i = 0; i < NHB / 256; ++i) {
    int idx = threadIdx.x + i * 256;
    int cb = idx % NCB, rq = idx / NCB;
    u32x4 in[HB];
#pragma unroll
    for (int r = 0; r < HB; ++r) {
      int gr = r0 + rq * HB + r;
      in[r] = (gr < rvalid) ? ld16(src + (long)gr * ld + cb * A::EL) : u32x4{0, 0, 0, 0};
    }
    // rq*HB rows start at byte rq*8 of each LDS row: chunk rq/2, half rq%2
#pragma unroll
    for (int c = 0; c < A::EL; ++c) {
      u32x2 o;
      if constexpr (sizeof(T) == 2) {
        uint32_t sh = (c & 1) ? 16 : 0;
        uint32_t e0 = (in[0][c >> 1] >> sh) & 0xffffu, e1 = (in[1][c >> 1] >> sh) & 0xffffu;
        uint32_t e2 = (in[2][c >> 1] >> sh) & 0xffffu, e3 = (in[3][c >> 1] >> sh) & 0xffffu;
        o = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
      } else {
        o = u32x2{in[0][c], in[1][c]};
      }
      int row = cb * A::EL + c;
      st8(lds + tile_off(row, rq >> 1, A::TCH) + (rq & 1) * 8, o);
    }
  }
}

// A-operand fragment from a row-layout tile: rows row0 + l%32, k-substep ks
// along the 128 columns.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_rows(const char* lds, int row0, int ks, int lane) {
  typedef Mfma<T> MM;
  typedef AttnCfg<T> A;
  const int row = row0 + (lane & 31);
  const int kel = ks * MM::KI + (lane >> 5) * MM::E;
  if constexpr (sizeof(T) == 2) {
    return __builtin_bit_cast(typename MM::frag, ld16(lds + tile_off(row, kel / A::EL, A::RCH)));
  } else {
    return *reinterpret_cast<const float*>(lds + tile_off(row, kel / A::EL, A::RCH) + (kel % A::EL) * 4);
  }
}

// A-operand fragment from a transposed tile [128][RT]: row d = row0 + l%32,
// k-slots = the tile rows (keys or queries) that the P/dS fragment of MFMA
// number mm holds in this lane: block blk = mm / (16/E), registers
// jj0 = (mm % (16/E)) * E ... jj0 + E - 1, index blk*32 + acc_row(j, lane).
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_trans(const char* lds, int row0, int mm, int lane) {
  typedef Mfma<T> MM;
  typedef AttnCfg<T> A;
  constexpr int PER = 16 / MM::E;
  const int row = row0 + (lane & 31);
  const int blk = mm / PER, jj0 = (mm % PER) * MM::E;
  const int idx0 = blk * 32 + acc_row(jj0, lane);
  if constexpr (sizeof(T) == 2) {
    // two runs of 4 consecutive indices: idx0 .. idx0+3 and idx0+8 .. idx0+11
    u32x2 a = ld8(lds + tile_off(row, idx0 >> 3, A::TCH) + ((idx0 >> 2) & 1) * 8);
    u32x2 b = ld8(lds + tile_off(row, (idx0 >> 3) + 1, A::TCH) + ((idx0 >> 2) & 1) * 8);
    return __builtin_bit_cast(typename MM::frag, u32x4{a[0], a[1], b[0], b[1]});
  } else {
    return *reinterpret_cast<const float*>(lds + tile_off(row, idx0 >> 2, A::TCH) + (idx0 & 3) * 4);
  }
}

// B-operand fragment from accumulator registers jj0 .. jj0+E-1.
template <typename T>
__device__ __forceinline__ typename Mfma<T>::frag frag_regs(const f32x16& p, int jj0) {
  if constexpr (sizeof(T) == 2) {
    bf16x8 f;
#pragma unroll
    for (int s = 0; s < 8; ++s) f[s] = (bf16)p[jj0 + s];
    return f;
  } else {
    return p[jj0];
  }
}

// Per-lane fragment of a row of 128 values (one query / key row), all ks.
template <typename T>
__device__ __forceinline__ void frag_row_global(typename Mfma<T>::frag* f, const T* rowp, bool valid, int lane) {
  typedef Mfma<T> MM;
#pragma unroll
  for (int ks = 0; ks < HD / MM::KI; ++ks) {
    const int kel = ks * MM::KI + (lane >> 5) * MM::E;
    if constexpr (sizeof(T) == 2) {
      f[ks] = valid ? __builtin_bit_cast(bf16x8, ld16(rowp + kel)) : bf16x8{};
    } else {
      f[ks] = valid ? rowp[kel] : 0.f;
    }
  }
}

// Store the 128 x 32 accumulator acc[4] (rows d, column = this lane's row r)
// times `scale` into dst row (128 contiguous values).
template <typename T>
__device__ __forceinline__ void store_acc_row(T* dst, const f32x16* acc, float scale, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + 8 * g + 4 * h;
      if constexpr (sizeof(T) == 2) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(acc[db][4 * g + e] * scale);
        st8(dst + d, __builtin_bit_cast(u32x2, v));
      } else {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(acc[db][4 * g + e] * scale);
        st16(dst + d, v);
      }
    }
  }
}

struct AttnArgs {
  const void* qkv;   // [B*T, 3C]: q'' | k'' | v, heads contiguous in each
  void* o;           // [B*T, C]
  float* lse;        // [B*H, T], log2-domain log-sum-exp of the scaled scores
  const void* dO;    // [B*T, C]
  const float* delta;  // [B*H, T] rowsum(dO * O)
  void* dqkv;        // [B*T, 3C]: dq'' | dk'' | dv
  int B, T, H, C;
  float sl2;         // log2(e) / sqrt(D)
  float rsd;         // 1 / sqrt(D)
};

// ---- forward ----------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(AttnArgs a) {
  typedef AttnCfg<T> A;
  typedef Mfma<T> MM;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int STAGE = A::ROWT + A::TRT;      // K rows + V^T
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
  const int BH = a.B * a.H;
  const int nqt = (a.T + 127) / 128;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);   // longest rows first
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H, head = bh % a.H;
  const long ld = 3L * a.C;
  const T* qkv = static_cast<const T*>(a.qkv);
  const T* Kg = qkv + (long)b * a.T * ld + a.C + head * HD;
  const T* Vg = Kg + a.C;
  const int qw0 = qt * 128 + wave * 32;
  const int q = qw0 + (lane & 31);

  typename MM::frag qf[HD / MM::KI];
  frag_row_global<T>(qf, qkv + ((long)b * a.T + q) * ld + head * HD, q < a.T, lane);

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int last_key = min(a.T - 1, qt * 128 + 127);
  const int nkt = last_key / A::RT + 1;
  stage_rows<T>(smem, Kg, ld, 0, a.T);
  stage_trans<T>(smem + A::ROWT, Vg, ld, 0, a.T);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const char* cur = smem + (kt & 1) * STAGE;
    char* nxt = smem + ((kt + 1) & 1) * STAGE;
    const int k0 = kt * A::RT;
    if (k0 <= qw0 + 31) {          // some key of this tile is visible to this wave
      f32x16 s[A::NB];
#pragma unroll
      for (int kb = 0; kb < A::NB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < HD / MM::KI; ++ks)
          s[kb] = MM::mma(frag_rows<T>(cur, kb * 32, ks, lane), qf[ks], s[kb]);
      }
      const bool need_mask = (k0 + A::RT - 1 > qw0) || (k0 + A::RT > a.T);
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < A::NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[kb][r] * a.sl2;
          if (need_mask) {
            const int key = k0 + kb * 32 + acc_row(r, lane);
            if (key > q || key >= a.T) v = -INFINITY;
          }
          s[kb][r] = v;
          mt = fmaxf(mt, v);
        }
      mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
      const float m_new = fmaxf(m_run, mt);
      const float ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m_run - ref);
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < A::NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2f(s[kb][r] - ref);
          s[kb][r] = p;
          ls += p;
        }
      l_run = l_run * alpha + ls;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] *= alpha;
#pragma unroll
      for (int mm = 0; mm < A::RT / MM::KI; ++mm) {
        constexpr int PER = 16 / MM::E;
        const auto pf = frag_regs<T>(s[mm / PER], (mm % PER) * MM::E);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = MM::mma(frag_trans<T>(cur + A::ROWT, db * 32, mm, lane), pf, acc[db]);
      }
    }
    if (kt + 1 < nkt) {
      // single-phase prefetch: the other buffer was last read before the
      // barrier that ended the previous iteration
      stage_rows<T>(nxt, Kg, ld, k0 + A::RT, a.T);
      stage_trans<T>(nxt + A::ROWT, Vg, ld, k0 + A::RT, a.T);
    }
    __syncthreads();
  }
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (q < a.T) {
    const float inv = 1.f / l_tot;
    store_acc_row<T>(static_cast<T*>(a.o) + ((long)b * a.T + q) * a.C + head * HD, acc, inv, lane);
    if (h == 0) a.lse[(long)bh * a.T + q] = m_run + log2f(l_tot);
  }
}

// ---- backward: dQ -------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_kernel(AttnArgs a) {
  typedef AttnCfg<T> A;
  typedef Mfma<T> MM;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int STAGE = 2 * A::ROWT + A::TRT;   // K rows, V rows, K^T
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int BH = a.B * a.H;
  const int nqt = (a.T + 127) / 128;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H, head = bh % a.H;
  const long ld = 3L * a.C;
  const T* qkv = static_cast<const T*>(a.qkv);
  const T* Kg = qkv + (long)b * a.T * ld + a.C + head * HD;
  const T* Vg = Kg + a.C;
  const int qw0 = qt * 128 + wave * 32;
  const int q = qw0 + (lane & 31);
  const bool qv = q < a.T;

  typename MM::frag qf[HD / MM::KI], df[HD / MM::KI];
  frag_row_global<T>(qf, qkv + ((long)b * a.T + q) * ld + head * HD, qv, lane);
  frag_row_global<T>(df, static_cast<const T*>(a.dO) + ((long)b * a.T + q) * a.C + head * HD, qv, lane);
  const float lse = qv ? a.lse[(long)bh * a.T + q] : 0.f;
  const float dlt = qv ? a.delta[(long)bh * a.T + q] : 0.f;

  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;

  const int last_key = min(a.T - 1, qt * 128 + 127);
  const int nkt = last_key / A::RT + 1;
  stage_rows<T>(smem, Kg, ld, 0, a.T);
  stage_rows<T>(smem + A::ROWT, Vg, ld, 0, a.T);
  stage_trans<T>(smem + 2 * A::ROWT, Kg, ld, 0, a.T);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const char* cur = smem + (kt & 1) * STAGE;
    char* nxt = smem + ((kt + 1) & 1) * STAGE;
    const int k0 = kt * A::RT;
    if (k0 <= qw0 + 31) {
      f32x16 s[A::NB], dp[A::NB];
#pragma unroll
      for (int kb = 0; kb < A::NB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[kb][r] = 0.f; dp[kb][r] = 0.f; }
#pragma unroll
        for (int ks = 0; ks < HD / MM::KI; ++ks) {
          s[kb] = MM::mma(frag_rows<T>(cur, kb * 32, ks, lane), qf[ks], s[kb]);
          dp[kb] = MM::mma(frag_rows<T>(cur + A::ROWT, kb * 32, ks, lane), df[ks], dp[kb]);
        }
      }
      const bool need_mask = (k0 + A::RT - 1 > qw0) || (k0 + A::RT > a.T);
#pragma unroll
      for (int kb = 0; kb < A::NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = exp2f(s[kb][r] * a.sl2 - lse);
          if (need_mask) {
            const int key = k0 + kb * 32 + acc_row(r, lane);
            if (key > q || key >= a.T) p = 0.f;
          }
          if (!qv) p = 0.f;
          s[kb][r] = p * (dp[kb][r] - dlt);   // dS^T
        }
#pragma unroll
      for (int mm = 0; mm < A::RT / MM::KI; ++mm) {
        constexpr int PER = 16 / MM::E;
        const auto sf = frag_regs<T>(s[mm / PER], (mm % PER) * MM::E);
#pragma unroll
        for (int db = 0; db < 4; ++db)
          acc[db] = MM::mma(frag_trans<T>(cur + 2 * A::ROWT, db * 32, mm, lane), sf, acc[db]);
      }
    }
    if (kt + 1 < nkt) {
      stage_rows<T>(nxt, Kg, ld, k0 + A::RT, a.T);
      stage_rows<T>(nxt + A::ROWT, Vg, ld, k0 + A::RT, a.T);
      stage_trans<T>(nxt + 2 * A::ROWT, Kg, ld, k0 + A::RT, a.T);
    }
    __syncthreads();
  }
  if (qv) store_acc_row<T>(static_cast<T*>(a.dqkv) + ((long)b * a.T + q) * ld + head * HD, acc, a.rsd, lane);
}

// ---- backward: dK, dV -----------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(AttnArgs a) {
  typedef AttnCfg<T> A;
  typedef Mfma<T> MM;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // Q rows, dO rows, Q^T, dO^T, lse[RT], delta[RT]
  constexpr int STAGE = 2 * A::ROWT + 2 * A::TRT + 2 * A::RT * 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int BH = a.B * a.H;
  const int kt = (int)(blockIdx.x / BH);          // first key tiles have the most queries
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H, head = bh % a.H;
  const long ld = 3L * a.C;
  const T* qkv = static_cast<const T*>(a.qkv);
  const T* Qg = qkv + (long)b * a.T * ld + head * HD;
  const T* dOg = static_cast<const T*>(a.dO) + (long)b * a.T * a.C + head * HD;
  const float* lseg = a.lse + (long)bh * a.T;
  const float* dlg = a.delta + (long)bh * a.T;
  const int kw0 = kt * 128 + wave * 32;
  const int key = kw0 + (lane & 31);
  const bool kv = key < a.T;

  typename MM::frag kf[HD / MM::KI], vf[HD / MM::KI];
  frag_row_global<T>(kf, qkv + ((long)b * a.T + key) * ld + a.C + head * HD, kv, lane);
  frag_row_global<T>(vf, qkv + ((long)b * a.T + key) * ld + 2 * a.C + head * HD, kv, lane);

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[i][r] = 0.f; dv[i][r] = 0.f; }

  auto stage = [&](char* dst, int q0) {
    stage_rows<T>(dst, Qg, ld, q0, a.T);
    stage_rows<T>(dst + A::ROWT, dOg, a.C, q0, a.T);
    stage_trans<T>(dst + 2 * A::ROWT, Qg, ld, q0, a.T);
    stage_trans<T>(dst + 2 * A::ROWT + A::TRT, dOg, a.C, q0, a.T);
    float* vec = reinterpret_cast<float*>(dst + 2 * A::ROWT + 2 * A::TRT);
    if (threadIdx.x < A::RT) {
      const int qq = q0 + threadIdx.x;
      vec[threadIdx.x] = (qq < a.T) ? lseg[qq] : INFINITY;      // exp2(s - inf) = 0
      vec[A::RT + threadIdx.x] = (qq < a.T) ? dlg[qq] : 0.f;
    }
  };

  const int qt0 = (kt * 128) / A::RT;
  const int nqt = (a.T + A::RT - 1) / A::RT;
  if (qt0 < nqt) stage(smem, qt0 * A::RT);
  __syncthreads();
  for (int qt = qt0; qt < nqt; ++qt) {
    const int it = qt - qt0;
    const char* cur = smem + (it & 1) * STAGE;
    char* nxt = smem + ((it + 1) & 1) * STAGE;
    const int q0 = qt * A::RT;
    const float* lsev = reinterpret_cast<const float*>(cur + 2 * A::ROWT + 2 * A::TRT);
    const float* dlv = lsev + A::RT;
    if (q0 + A::RT - 1 >= kw0) {      // some query of this tile sees a key of this wave
      const bool need_mask = q0 < kw0 + 31;
#pragma unroll
      for (int qb = 0; qb < A::NB; ++qb) {
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) { s[r] = 0.f; dp[r] = 0.f; }
#pragma unroll
        for (int ks = 0; ks < HD / MM::KI; ++ks) {
          s = MM::mma(frag_rows<T>(cur, qb * 32, ks, lane), kf[ks], s);               // S  (q x key)
          dp = MM::mma(frag_rows<T>(cur + A::ROWT, qb * 32, ks, lane), vf[ks], dp);   // dP (q x key)
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int qi = qb * 32 + 8 * g + 4 * (lane >> 5);
          const f32x4 lv = *reinterpret_cast<const f32x4*>(lsev + qi);
          const f32x4 dv4 = *reinterpret_cast<const f32x4*>(dlv + qi);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = 4 * g + e;
            float p = exp2f(s[r] * a.sl2 - lv[e]);
            if (need_mask && key > q0 + qi + e) p = 0.f;
            s[r] = p;
            dp[r] = p * (dp[r] - dv4[e]);    // dS
          }
        }
#pragma unroll
        for (int mm = 0; mm < 32 / MM::KI; ++mm) {
          const int mmt = qb * (32 / MM::KI) + mm;      // MFMA index within the tile
          const auto pf = frag_regs<T>(s, mm * MM::E);
          const auto sf = frag_regs<T>(dp, mm * MM::E);
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            dv[db] = MM::mma(frag_trans<T>(cur + 2 * A::ROWT + A::TRT, db * 32, mmt, lane), pf, dv[db]);
            dk[db] = MM::mma(frag_trans<T>(cur + 2 * A::ROWT, db * 32, mmt, lane), sf, dk[db]);
          }
        }
      }
    }
    if (qt + 1 < nqt) stage(nxt, q0 + A::RT);
    __syncthreads();
  }
  if (kv) {
    T* row = static_cast<T*>(a.dqkv) + ((long)b * a.T + key) * ld + head * HD;
    store_acc_row<T>(row + a.C, dk, a.rsd, lane);
    store_acc_row<T>(row + 2 * a.C, dv, 1.f, lane);
  }
}

template <typename T> constexpr int attn_fwd_lds() { return 2 * (AttnCfg<T>::ROWT + AttnCfg<T>::TRT); }
template <typename T> constexpr int attn_dq_lds() { return 2 * (2 * AttnCfg<T>::ROWT + AttnCfg<T>::TRT); }
template <typename T> constexpr int attn_dkdv_lds() {
  return 2 * (2 * AttnCfg<T>::ROWT + 2 * AttnCfg<T>::TRT + 2 * AttnCfg<T>::RT * 4);
}

}  // namespace blk
