// Causal multi-head attention, head size 128, for gfx950 (flash-style: the
// T x T score matrix never reaches HBM), with an optional sliding window and
// grouped key/value heads.
//
// Forward: each wave owns 32 queries (float32) or two blocks of 32 (bf16)
// and walks key tiles.  It computes the TRANSPOSED score block S^T = K Q^T
// with MFMA 32x32, so the lane that holds column l%32 of S^T holds every
// score of one query: the running maximum and denominator of the online
// softmax are per-lane scalars (plus one exchange with lane l^32), and the
// rescale of the output accumulator O^T (d x query) is a per-lane multiply.
// P^T feeds O^T += V^T P^T straight from registers: the MFMA k-slots of P^T
// are the keys this lane already holds, and V^T is read from LDS with the
// same key order.
//
// Backward (no atomics, deterministic): a pass over key tiles per query tile
// for dQ, and a pass over query tiles per key tile for dK and dV, both
// recomputing P from the saved log-sum-exp.  The bf16 backward loops are
// written as explicit steps of two MFMAs whose LDS reads are issued two
// steps ahead, with a scheduling fence per step.  The bf16 backward kernels
// are persistent (one workgroup per CU walking units of 128 rows), and their
// per-unit row operands and results pass through LDS so that every global
// access between units is row-contiguous.
//
// This header is compiled only in attn.hip, with MFMA results in vector
// registers (the softmax reads them after every MFMA chain).
//
// (Causal multi-head attention with 128-dim heads: 7minutos.es nanochat
// article, section "Modelo, escalado y objetivo de speedrun"; QK-norm and
// rotary precede it: flicky.cc nanochat page, section on the model.)
#pragma once
#include <type_traits>
#include "attn_args.cuh"
#include "common.cuh"

namespace blk {


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
__device__ __forceinline__ float store_acc_row(T* dst, const f32x16* acc, float scale, int lane) {
  const int h = lane >> 5;
  float mx = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d = db * 32 + 8 * g + 4 * h;
      if constexpr (sizeof(T) == 2) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float x = acc[db][4 * g + e] * scale;
          mx = fmaxf(mx, fabsf(x));
          v[e] = (bf16)x;
        }
        st8(dst + d, __builtin_bit_cast(u32x2, v));
      } else {
        u32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = __float_as_uint(acc[db][4 * g + e] * scale);
        st16(dst + d, v);
      }
    }
  }
  return mx;   // largest stored magnitude (bf16 rows), before rounding
}

// The operands the QK-norm / rotary backward of one row reads besides the
// accumulator: this lane's 64 values of the normalised row z (dims db*32 +
// 8i + 4h + e, h = lane/32) and the (cos, sin) pairs of its 32 first-half
// dims.  Loaded apart from the arithmetic so that a caller can put other
// loads in flight between the two.
struct QkRowIn {
  bf16x4 z[4][4];
  u32x4 c[2][4][2];
};
__device__ __forceinline__ void qk_row_load(QkRowIn& in, const bf16* z, const float2* cs, int lane) {
  const int h = lane >> 5;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) in.z[db][i] = __builtin_bit_cast(bf16x4, ld8(z + db * 32 + 8 * i + 4 * h));
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* cp = reinterpret_cast<const float*>(cs + db * 32 + 8 * i + 4 * h);
      in.c[db][i][0] = ld16(cp);
      in.c[db][i][1] = ld16(cp + 4);
    }
}

// Stores the gradient of q' or k' (before QK-norm and rotary) of one row:
// g = acc * scale is the gradient of the normalised row z (this lane holds
// dims db*32 + 8i + 4h + e, h = lane/32; lane ^ 32 the rest), p its QK-norm
// factor, in.c the row's angles.  QK-norm backward
// dz' = p (g - z mean(g z)), then the transposed rotation of each pair
// (d, d + 64).  (Rotary embedding and QK-norm: flicky.cc nanochat page,
// section on the model.)
__device__ __forceinline__ float store_acc_row_qk(bf16* dst, const QkRowIn& in, float p, const f32x16* acc,
                                                  float scale, int lane) {
  const int h = lane >> 5;
  float gv[4][16], zv[4][16];
  float dot = 0.f;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const bf16x4 zz = in.z[db][i];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        gv[db][4 * i + e] = acc[db][4 * i + e] * scale;
        zv[db][4 * i + e] = (float)zz[e];
        dot += gv[db][4 * i + e] * zv[db][4 * i + e];
      }
    }
  dot += __shfl_xor(dot, 32, 64);
  const float mean = dot * (1.f / 128.f);
  float mx = 0.f;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float c8[8];
      Chunk<float>::unpack(in.c[db][i][0], c8);
      Chunk<float>::unpack(in.c[db][i][1], c8 + 4);
      bf16x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int r = 4 * i + e;
        const float d1 = p * (gv[db][r] - zv[db][r] * mean);
        const float d2 = p * (gv[db + 2][r] - zv[db + 2][r] * mean);
        const float c = c8[2 * e], sn = c8[2 * e + 1];
        const float vlo = d1 * c + d2 * sn, vhi = d2 * c - d1 * sn;
        mx = fmaxf(mx, fmaxf(fabsf(vlo), fabsf(vhi)));
        lo[e] = (bf16)vlo;
        hi[e] = (bf16)vhi;
      }
      st8(dst + db * 32 + 8 * i + 4 * h, __builtin_bit_cast(u32x2, lo));
      st8(dst + (db + 2) * 32 + 8 * i + 4 * h, __builtin_bit_cast(u32x2, hi));
    }
  return mx;   // largest stored magnitude, before rounding
}
__device__ __forceinline__ float store_acc_row_qk(bf16* dst, const bf16* z, float p, const float2* cs,
                                                  const f32x16* acc, float scale, int lane) {
  QkRowIn in;
  qk_row_load(in, z, cs, lane);
  return store_acc_row_qk(dst, in, p, acc, scale, lane);
}



// ---- forward ----------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256, 1) void attn_fwd_kernel(AttnArgs a) {
  typedef AttnCfg<T> A;
  typedef Mfma<T> MM;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int STAGE = A::ROWT + A::TRT;      // K rows + V^T
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), h = lane >> 5;
  const int BH = a.B * a.H;
  const int nqt = (a.T + 127) / 128;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);   // longest rows first
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H, head = bh % a.H;
  const long ld = a.LD;
  const int kvh = head / (a.H / a.G);
  const T* qkv = static_cast<const T*>(a.qkv);
  const T* Kg = qkv + (long)b * a.T * ld + a.KO + kvh * HD;
  const T* Vg = qkv + (long)b * a.T * ld + a.VO + kvh * HD;
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
  const int kt_lo = max(0, qt * 128 - a.W + 1) / A::RT;   // first tile inside the window
  stage_rows<T>(smem, Kg, ld, kt_lo * A::RT, a.T);
  stage_trans<T>(smem + A::ROWT, Vg, ld, kt_lo * A::RT, a.T);
  __syncthreads();
  for (int kt = kt_lo; kt < nkt; ++kt) {
    const char* cur = smem + ((kt - kt_lo) & 1) * STAGE;
    char* nxt = smem + ((kt - kt_lo + 1) & 1) * STAGE;
    const int k0 = kt * A::RT;
    // some key of this tile is visible to some query of this wave
    if (k0 <= qw0 + 31 && k0 + A::RT - 1 > qw0 - a.W) {
      f32x16 s[A::NB];
#pragma unroll
      for (int kb = 0; kb < A::NB; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
#pragma unroll
        for (int ks = 0; ks < HD / MM::KI; ++ks)
          s[kb] = MM::mma(frag_rows<T>(cur, kb * 32, ks, lane), qf[ks], s[kb]);
      }
      const bool need_mask = (k0 + A::RT - 1 > qw0) || (k0 + A::RT > a.T) || (k0 <= qw0 + 31 - a.W);
      float mt = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < A::NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float v = s[kb][r] * a.sl2;
          if (need_mask) {
            const int key = k0 + kb * 32 + acc_row(r, lane);
            if (key > q || key >= a.T || key <= q - a.W) v = -INFINITY;
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
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int BH = a.B * a.H;
  const int nqt = (a.T + 127) / 128;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H, head = bh % a.H;
  const long ld = a.LD;
  const int kvh = head / (a.H / a.G);
  const T* qkv = static_cast<const T*>(a.qkv);
  const T* Kg = qkv + (long)b * a.T * ld + a.KO + kvh * HD;
  const T* Vg = qkv + (long)b * a.T * ld + a.VO + kvh * HD;
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
  const int kt_lo = max(0, qt * 128 - a.W + 1) / A::RT;   // first tile inside the window
  stage_rows<T>(smem, Kg, ld, kt_lo * A::RT, a.T);
  stage_rows<T>(smem + A::ROWT, Vg, ld, kt_lo * A::RT, a.T);
  stage_trans<T>(smem + 2 * A::ROWT, Kg, ld, kt_lo * A::RT, a.T);
  __syncthreads();
  for (int kt = kt_lo; kt < nkt; ++kt) {
    const char* cur = smem + ((kt - kt_lo) & 1) * STAGE;
    char* nxt = smem + ((kt - kt_lo + 1) & 1) * STAGE;
    const int k0 = kt * A::RT;
    if (k0 <= qw0 + 31 && k0 + A::RT - 1 > qw0 - a.W) {
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
      const bool need_mask = (k0 + A::RT - 1 > qw0) || (k0 + A::RT > a.T) || (k0 <= qw0 + 31 - a.W);
#pragma unroll
      for (int kb = 0; kb < A::NB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], a.sl2, -lse));
          if (need_mask) {
            const int key = k0 + kb * 32 + acc_row(r, lane);
            if (key > q || key >= a.T || key <= q - a.W) p = 0.f;
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
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // one workgroup = 128 keys of one (sequence, key/value head); it walks the
  // query tiles of every query head of the group
  const int BG = a.B * a.G, R = a.H / a.G;
  const int kt = (int)(blockIdx.x / BG);          // first key tiles have the most queries
  const int bg = blockIdx.x % BG;
  const int b = bg / a.G, kvh = bg % a.G;
  const long ld = a.LD;
  const T* qkv = static_cast<const T*>(a.qkv);
  const int kw0 = kt * 128 + wave * 32;
  const int key = kw0 + (lane & 31);
  const bool kv = key < a.T;

  typename MM::frag kf[HD / MM::KI], vf[HD / MM::KI];
  frag_row_global<T>(kf, qkv + ((long)b * a.T + key) * ld + a.KO + kvh * HD, kv, lane);
  frag_row_global<T>(vf, qkv + ((long)b * a.T + key) * ld + a.VO + kvh * HD, kv, lane);

  f32x16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) { dk[i][r] = 0.f; dv[i][r] = 0.f; }

  const int qt0 = (kt * 128) / A::RT;
  // the last query that sees a key of this workgroup is kt*128 + 127 + W - 1
  const int nqt = min((a.T + A::RT - 1) / A::RT, (int)(((long)kt * 128 + 127 + a.W - 1) / A::RT) + 1);
  const int nq = max(0, nqt - qt0);               // query tiles per head
  // iteration it: query head kvh*R + it/nq, query tile qt0 + it%nq
  auto stage = [&](char* dst, int it) {
    const int h = kvh * R + it / nq, q0 = (qt0 + it % nq) * A::RT;
    const T* Qg = qkv + (long)b * a.T * ld + h * HD;
    const T* dOg = static_cast<const T*>(a.dO) + (long)b * a.T * a.C + h * HD;
    const float* lseg = a.lse + ((long)b * a.H + h) * a.T;
    const float* dlg = a.delta + ((long)b * a.H + h) * a.T;
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

  const int niter = R * nq;
  if (niter > 0) stage(smem, 0);
  __syncthreads();
  for (int it = 0; it < niter; ++it) {
    const char* cur = smem + (it & 1) * STAGE;
    char* nxt = smem + ((it + 1) & 1) * STAGE;
    const int q0 = (qt0 + it % nq) * A::RT;
    const float* lsev = reinterpret_cast<const float*>(cur + 2 * A::ROWT + 2 * A::TRT);
    const float* dlv = lsev + A::RT;
    // some query of this tile sees a key of this wave
    if (q0 + A::RT - 1 >= kw0 && q0 <= kw0 + 31 + a.W - 1) {
      const bool need_mask = q0 < kw0 + 31 || q0 + A::RT - 1 >= kw0 + a.W;
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
            float p = __builtin_amdgcn_exp2f(fmaf(s[r], a.sl2, -lv[e]));
            if (need_mask && (key > q0 + qi + e || q0 + qi + e >= key + a.W)) p = 0.f;
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
    if (it + 1 < niter) stage(nxt, it + 1);
    __syncthreads();
  }
  if (kv) {
    T* row = static_cast<T*>(a.dqkv) + ((long)b * a.T + key) * ld;
    store_acc_row<T>(row + a.KO + kvh * HD, dk, a.rsd, lane);
    store_acc_row<T>(row + a.VO + kvh * HD, dv, 1.f, lane);
  }
}

// ---- forward, bf16, direct-to-LDS pipeline ------------------------------------------
// One workgroup = 256 queries of one (sequence, head): 4 waves x 64 queries
// (two 32-query MFMA blocks that share every K and V fragment read, halving
// LDS traffic per MFMA).  Key tiles of 64 rows, K and V row-major in LDS,
// staged by buffer loads straight into LDS in a three-slot ring (prefetch
// distance two tiles).  V^T fragments come from the row-major V tile through
// the LDS transpose read (ds_read_b64_tr_b16).  Row layout: 16 chunks of 16
// bytes per 128-wide row, swizzled by fa::sw.
namespace fa {
constexpr int QW = 64;                 // queries per wave
constexpr int QWG = 4 * QW;            // queries per workgroup
constexpr int KT = 64;                 // keys per tile
constexpr int TILE = KT * 256;         // bytes of one [64][128] bf16 tile
constexpr int SLOT = 2 * TILE;         // K + V
constexpr int NSLOT = 3;
constexpr int LDS = NSLOT * SLOT;      // 96 KiB

// Chunk c (16 bytes) of row r (256 bytes) is stored at c ^ sw(r),
// sw(r) = 4 (r & 3) ^ (r & 2) ^ ((r >> 2) & 3), a function of r & 15.  A
// 16-byte fragment read touches 8 (or 16) consecutive rows at one chunk per
// LDS cycle and a 16-lane (32-lane) transpose read 4 consecutive rows x 2 (4)
// adjacent chunks; with 32 banks (64 banks) of 4 bytes both land on distinct
// banks, whichever of the two groupings the hardware uses.  Rows r and r + 8
// differ by sw ^ 2, rows r and r + 16 not at all.
__device__ __forceinline__ int sw(int row) { return ((row & 3) << 2) ^ (row & 2) ^ ((row >> 2) & 3); }
__device__ __forceinline__ int off(int row, int chunk) { return row * 256 + ((chunk ^ sw(row)) << 4); }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Issue the direct-to-LDS loads of key rows k0.. of K and V (rows >= T read 0).
__device__ __forceinline__ void issue_kv(char* slot, i32x4 rs, int k0, long ldb, int koff, int voff, int wave,
                                         int lane) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {                 // K, then V
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int base = wave * 256 + i * 64;     // chunk index in the tile (64 per issue)
      const int p = base + lane;
      const int row = p >> 4, c = (p & 15) ^ sw(row);
      const uint32_t o = (uint32_t)((long)(k0 + row) * ldb + (t ? voff : koff) + c * 16);
      lds_u32* dst = (lds_u32*)(slot + t * TILE + __builtin_amdgcn_readfirstlane(base) * 16);
      dma16(rs, dst, o);
    }
  }
}

// Per-lane byte offsets of the row-tile fragment reads, k-substep ks (add
// kb*8192 for key block kb): row l%32, chunk 2ks + l/32, swizzled.
__device__ __forceinline__ void frag_k_offsets(int* o, int lane) {
#pragma unroll
  for (int ks = 0; ks < 8; ++ks) o[ks] = off(lane & 31, 2 * ks + (lane >> 5));
}

// Per-lane byte offsets of the V^T transpose reads, run (0, 1) and d-block db
// (add mm*4096 for MFMA chunk mm: 16 rows of 256 bytes, the swizzle only
// depends on row & 15).
__device__ __forceinline__ void frag_vt_offsets(int* o, int lane) {
  const int g = (lane >> 4) & 3, s = lane & 15;
#pragma unroll
  for (int run = 0; run < 2; ++run)
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int key = 4 * (g >> 1) + (s >> 2) + 8 * run;
      const int col = db * 32 + 16 * (g & 1) + 4 * (s & 3);
      o[run * 4 + db] = off(key, col >> 3) + (col & 7) * 2;
    }
}

typedef __attribute__((address_space(3))) char lds_char;

// A fragment of V^T for MFMA chunk mm (16 keys) and d-block db from the
// precomputed offsets: lane l holds d = db*32 + l%32 and keys 16mm + 4h +
// {0..3}, 16mm + 8 + 4h + {0..3} (h = l/32), the key order of the P^T
// fragment built from the score registers.
__device__ __forceinline__ bf16x8 frag_vt_at(const lds_char* tile, const int* vo, int mm, int db) {
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + mm * 4096 + vo[db]));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(tile + mm * 4096 + vo[4 + db]));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// frag_vt_at with the offsets rebuilt from one per-lane base (vbase = the
// run-0, d-block-0 offset): the d-block step is an XOR of bits 6-7, and the
// 8 rows of run 1 add 2048 with chunk bit 1 flipped, so offset(0, db) =
// vbase ^ (db << 6) and offset(1, db) = (vbase ^ 32 ^ (db << 6)) + 2048.
__device__ __forceinline__ bf16x8 frag_vt_x(const lds_char* tile, int vbase, int mm, int db) {
  const lds_char* p = tile + mm * 4096;
  const s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + (vbase ^ (db << 6))));
  const s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p + 2048 + (vbase ^ 32 ^ (db << 6))));
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  const s16x8 r = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, r);
}

// K and V tiles of 64 rows through an LDS slot, issued by eight waves (two
// 16-byte chunks per lane and tile; layout as in issue_kv).
__device__ __forceinline__ void issue_kv8(char* slot, i32x4 rs, int k0, long ldb, int koff, int voff, int wave,
                                          int lane) {
#pragma unroll
  for (int t = 0; t < 2; ++t) {                 // K, then V
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int base = wave * 128 + i * 64;     // chunk index in the tile (64 per issue)
      const int p = base + lane;
      const int row = p >> 4, c = (p & 15) ^ sw(row);
      const uint32_t o = (uint32_t)((long)(k0 + row) * ldb + (t ? voff : koff) + c * 16);
      lds_u32* dst = (lds_u32*)(slot + t * TILE + __builtin_amdgcn_readfirstlane(base) * 16);
      dma16(rs, dst, o);
    }
  }
}
typedef __attribute__((address_space(3))) const bf16x8 lds_bf16x8;

}  // namespace fa

// Forward: one workgroup = 256 queries of one (sequence, head), eight waves of
// 32 queries (two waves per SIMD: while one runs the softmax arithmetic of a
// key tile the other's MFMAs proceed); key tiles of 64 through a 3-slot LDS
// ring.
// WIN: a window shorter than the sequence (a.W < a.T); the causal instance
// carries none of the window's bounds, masks or guards.
template <bool WIN>
__global__ __launch_bounds__(512, 1) void attn_fwd_bf16_kernel(AttnArgs a) {
  using namespace fa;
  typedef Mfma<bf16> MM;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  constexpr int QW8 = 32;                              // queries per wave
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), h = lane >> 5;
  const int BH = a.B * a.H;
  const int nqt = (a.T + QWG - 1) / QWG;
  const int qt = nqt - 1 - (int)(blockIdx.x / BH);     // longest rows first
  const int bh = blockIdx.x % BH;
  const int b = bh / a.H, head = bh % a.H;
  const long ldb = (long)a.LD * 2;                     // row stride in bytes
  const int kvh = head / (a.H / a.G);
  const bf16* qkv = static_cast<const bf16*>(a.qkv);
  const i32x4 rs = make_rsrc(qkv + (long)b * a.T * a.LD, clamp_bytes((long)a.T * ldb));
  const int koff = (a.KO + kvh * HD) * 2, voff = (a.VO + kvh * HD) * 2;
  const int qw0 = qt * QWG + wave * QW8;
  const int q = qw0 + (lane & 31);

  bf16x8 qf[8];
  frag_row_global<bf16>(qf, qkv + ((long)b * a.T + q) * a.LD + head * HD, q < a.T, lane);
  // the q fragments have landed before any tile is in flight (a wait the
  // compiler placed at their first use inside the loop would, with the
  // ring's loads outstanding, drain the ring every tile)
  wait_vm<0>();
  f32x16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[i][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  int ko[8], vo[8];
  frag_k_offsets(ko, lane);
  frag_vt_offsets(vo, lane);

  const int last_key = min(a.T - 1, qt * QWG + QWG - 1);
  const int kt_lo = WIN ? max(0, qt * QWG - a.W + 1) / KT : 0;   // first tile inside the window
  const int n = last_key / KT + 1 - kt_lo;
  issue_kv8(smem, rs, kt_lo * KT, ldb, koff, voff, wave, lane);
  if (n > 1) issue_kv8(smem + SLOT, rs, (kt_lo + 1) * KT, ldb, koff, voff, wave, lane);
  for (int it = 0; it < n; ++it) {
    // tile it landed (own loads, then everyone's); slot of tile it-1 is free
    if (it + 1 < n) wait_vm<4>();   // the next tile may stay in flight
    else wait_vm<0>();
    ring_barrier();
    if (it + 2 < n) issue_kv8(smem + ((it + 2) % NSLOT) * SLOT, rs, (kt_lo + it + 2) * KT, ldb, koff, voff, wave, lane);
    const lds_char* kt_ = (const lds_char*)smem + (it % NSLOT) * SLOT;
    const lds_char* vt_ = kt_ + TILE;
    const int k0 = (kt_lo + it) * KT;
    if (k0 > qw0 + QW8 - 1) continue;                 // every key of this tile is in this wave's future
    if (WIN && k0 + KT - 1 <= qw0 - a.W) continue;    // every key is before this wave's windows
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
    // K fragments read two k-steps ahead of their MFMAs (read just before
    // them, every MFMA pair waited out the LDS latency)
    bf16x8 kf0[8], kf1[8];
    auto rdk = [&](int ks) {
      kf0[ks] = *(lds_bf16x8*)(kt_ + ko[ks]);
      kf1[ks] = *(lds_bf16x8*)(kt_ + 8192 + ko[ks]);
    };
    rdk(0);
    rdk(1);
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      if (ks + 2 < 8) rdk(ks + 2);
      s[0] = MM::mma(kf0[ks], qf[ks], s[0]);
      s[1] = MM::mma(kf1[ks], qf[ks], s[1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the first V^T fragments of the PV product, read while the softmax runs
    bf16x8 vf[16];
    auto rdv = [&](int i) { vf[i] = frag_vt_at(vt_, vo, i >> 2, i & 3); };
    rdv(0);
    rdv(1);
    // Online softmax with a lazily updated reference: scores are exponentiated
    // against m_run, which only moves (rescaling l and O) when some lane's tile
    // maximum exceeds it by more than 8 (a factor 256, far from overflow).
    // diagonal, ragged or window-edge tile
    if ((k0 + KT - 1 > qw0) || (k0 + KT > a.T) || (WIN && k0 <= qw0 + 31 - a.W)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + kb * 32 + acc_row(r, lane);
          if (key > q || key >= a.T || (WIN && key <= q - a.W)) s[kb][r] = -INFINITY;
        }
    }
    float mt = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64)) * a.sl2;
    // with a window a query can meet whole tiles of hidden keys before its
    // first visible one: its running maximum is still -inf (and l, O zero).
    // Causal: every query sees key 0 in the first tile, so m is finite.
    if (__ballot(mt > m_run + 8.f) != 0) {
      const float m_new = fmaxf(m_run, mt);
      const float alpha = (WIN && m_new == -INFINITY) ? 0.f : exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
      m_run = m_new;
    }
    const float ref = (WIN && m_run == -INFINITY) ? 0.f : m_run;
    float ls = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(s[kb][r], a.sl2, -ref));
        s[kb][r] = p;
        ls += p;
      }
    l_run += ls;
    // O^T += V^T P^T, the V^T fragments read two MFMAs ahead
    bf16x8 p0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i + 2 < 16) rdv(i + 2);
      const int mm = i >> 2, db = i & 3;
      if (db == 0) p0 = frag_regs<bf16>(s[mm >> 1], (mm & 1) * 8);
      o[db] = MM::mma(vf[i], p0, o[db]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  float mx = 0.f;
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  if (q < a.T) {
    mx = store_acc_row<bf16>(static_cast<bf16*>(a.o) + ((long)b * a.T + q) * a.C + head * HD, o, 1.f / l_tot, lane);
    if (h == 0) a.lse[(long)bh * a.T + q] = m_run + log2f(l_tot);
  }
  if (a.amax_o) amax_publish<bf16>(a.amax_o, mx);
}

// ---- backward, bf16, direct-to-LDS pipelines ----------------------------------------
namespace fa {
// Issue direct-to-LDS loads of 64 rows (r0..) x 128 bf16 of one matrix view:
// row stride ldb bytes, column offset coff bytes; rows past the buffer read 0.
__device__ __forceinline__ void issue_tile(char* dst, i32x4 rs, int r0, long ldb, int coff, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int base = wave * 256 + i * 64;
    const int p = base + lane;
    const int row = p >> 4, c = (p & 15) ^ sw(row);
    const uint32_t o = (uint32_t)((long)(r0 + row) * ldb + coff + c * 16);
    dma16(rs, (lds_u32*)(dst + base * 16), o);
  }
}
// 64 floats of a vector at index r0.. into dst[0..63] (one issue: lanes 0-15
// carry the data, the other lanes read past the end and write zeros to
// dst[64..255], so dst must hold 1 KiB).
__device__ __forceinline__ void issue_vec(char* dst, i32x4 rv, int r0, int lane) {
  const uint32_t o = lane < 16 ? (uint32_t)((r0 + lane * 4) * 4) : 0xffffffffu;
  dma16(rv, (lds_u32*)dst, o);
}
typedef __attribute__((address_space(3))) const f32x4 lds_f32x4;

// ---- row layout of a wave's 128 x 32 accumulator (backward kernels) ----------
// A wave's accumulator acc[4] holds a 128 x 32 block: rows d (acc[db] covers
// d = 32 db ..), column = one of the wave's 32 rows (lane & 31).  It is staged
// in LDS as 32 rows x 128 floats, 16-byte chunks XOR-swizzled by row (the 32
// rows one instruction writes fall in distinct chunks), and read back in
// passes: pass i gives this lane row 4i + lane/16 and dims 8 (lane & 15) .. +7.
__device__ __forceinline__ int stg_idx(int row, int d) { return row * 128 + ((((d >> 2) ^ row) & 31) << 2) + (d & 3); }
// (row: the staging row of this lane's column; lane & 31 unless permuted)
// (registers r .. r+3, r % 4 == 0, are 4 consecutive dims: one 16-byte chunk)
// The rows are read back by other lanes of the same wave (whose LDS accesses
// execute in order): the compiler fence keeps those reads after these writes,
// which the compiler, reasoning per lane, would see as independent.
__device__ __forceinline__ void stage_acc(float* stg, const f32x16* acc, float scale, int lane, int row = -1) {
  if (row < 0) row = lane & 31;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; r += 4) {
      const int d = db * 32 + acc_row(r, lane);
      *reinterpret_cast<f32x4*>(stg + stg_idx(row, d)) =
          f32x4{acc[db][r] * scale, acc[db][r + 1] * scale, acc[db][r + 2] * scale, acc[db][r + 3] * scale};
    }
  __asm volatile("" ::: "memory");
}
__device__ __forceinline__ void unstage_row(const float* stg, int i, int lane, float* f) {
  const int row = 4 * i + (lane >> 4), d = 8 * (lane & 15);
  Chunk<float>::unpack(*reinterpret_cast<const u32x4*>(stg + stg_idx(row, d)), f);
  Chunk<float>::unpack(*reinterpret_cast<const u32x4*>(stg + stg_idx(row, d + 4)), f + 4);
}
// The staged rows as bf16 to out (row r at out + r*ld), rows < nrows; returns
// the largest stored magnitude before rounding.
__device__ __forceinline__ float store_rows(const float* stg, bf16* out, long ld, int nrows, int lane) {
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float f[8];
    unstage_row(stg, i, lane, f);
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fabsf(f[e]));
    const int r = 4 * i + (lane >> 4);
    if (r < nrows) st16(out + r * ld + 8 * (lane & 15), Chunk<bf16>::pack(f));
  }
  return mx;
}
// Operands of the QK-norm backward of the wave's 32 rows: the normalised rows
// z (row r at z + r*ld) and their factors rho[r * rs], zero past nrows.
// Also the rotary angles (cs: [T][64]) of this lane's 8 angle indices at its
// first pass's position and at position 4: pass i + 1's rows sit 4
// positions after pass i's, so each pass turns the previous pass's angles by
// the angle at position 4 (angle addition) instead of loading its own.
struct QkRows {
  u32x4 z[8];
  float p[8];
  u32x4 cs0[4];
  u32x4 cs4[4];
};
// angle-table chunks of pass i (rows 4i + lane/16 of t0 ..; rows past nrows
// read a valid row, their results are not stored)
__device__ __forceinline__ void cs_rows_load(u32x4* c, const float2* cs, int t0, int i, int nrows, int lane) {
  const int t = nrows > 0 ? t0 + min(4 * i + (lane >> 4), nrows - 1) : 0;
  const float* cp = reinterpret_cast<const float*>(cs + (long)t * 64 + (lane & 7) * 8);
#pragma unroll
  for (int h = 0; h < 4; ++h) c[h] = ld16(cp + 4 * h);
}
__device__ __forceinline__ void qk_rows_load(QkRows& q, const bf16* z, long ld, const float* rho, long rs, int nrows,
                                             int lane, const float2* cs, int t0, int T) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = 4 * i + (lane >> 4);
    q.z[i] = r < nrows ? ld16(z + r * ld + 8 * (lane & 15)) : u32x4{0u, 0u, 0u, 0u};
    q.p[i] = r < nrows ? rho[r * rs] : 0.f;
  }
  cs_rows_load(q.cs0, cs, t0, 0, nrows, lane);
  // position 4 (T <= 4: any row; no row of a later pass is stored then)
  const float* cp = reinterpret_cast<const float*>(cs + (long)min(4, T - 1) * 64 + (lane & 7) * 8);
#pragma unroll
  for (int h = 0; h < 4; ++h) q.cs4[h] = ld16(cp + 4 * h);
}
// Gradient of q' or k' from the staged gradient g of the normalised rows:
// QK-norm backward dz' = p (g - z mean(g z)) over the row's 128 dims (16
// lanes), then the transposed rotation of each pair (d, d + 64), 8 lanes
// apart, with the angles of sequence position t0 + r (cs: [T][64]).  Row r to
// out + r*ld for r < nrows; returns the largest stored magnitude before
// rounding.  (Rotary embedding and QK-norm: flicky.cc nanochat page, section
// on the model.)
__device__ __forceinline__ float store_rows_qk(const float* stg, const QkRows& q, bf16* out, long ld, int nrows,
                                               int lane) {
  const int cg = lane & 15;
  float mx = 0.f;
  // (cos, sin) of this lane's 8 angles at the current pass's position, and at position 4
  float c8[16], c4[16];
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    Chunk<float>::unpack(q.cs0[h], c8 + 4 * h);
    Chunk<float>::unpack(q.cs4[h], c4 + 4 * h);
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float g[8], z[8];
    unstage_row(stg, i, lane, g);
    Chunk<bf16>::unpack(q.z[i], z);
    if (i > 0) {   // 4 positions on: cos(a + b), sin(a + b) from a and b = the angle at position 4
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float c = c8[2 * e], sn = c8[2 * e + 1];
        c8[2 * e] = fmaf(c, c4[2 * e], -sn * c4[2 * e + 1]);
        c8[2 * e + 1] = fmaf(sn, c4[2 * e], c * c4[2 * e + 1]);
      }
    }
    float dot = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) dot += g[e] * z[e];
    const float mean = row16_sum(dot) * (1.f / 128.f);
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = q.p[i] * (g[e] - z[e] * mean);
      const float other = dpp_mov<DPP_XOR8>(d);
      const float c = c8[2 * e], sn = c8[2 * e + 1];
      // first half: d1 = own, d2 = partner -> d1 c + d2 s; second half: d2 c - d1 s
      o[e] = cg < 8 ? d * c + other * sn : d * c - other * sn;
      mx = fmaxf(mx, fabsf(o[e]));
    }
    const int r = 4 * i + (lane >> 4);
    if (r < nrows) st16(out + r * ld + 8 * cg, Chunk<bf16>::pack(o));
  }
  return mx;
}
}  // namespace fa

// dK, dV: one unit of work = 128 keys of one (sequence, key/value head); it
// walks the 64-query tiles at and after the diagonal of every query head of
// the group.  Eight waves, two per SIMD, in pairs that share 32 keys and
// split the work of a tile between them:
// - the P wave (waves 0-3) holds the pair's K fragments, computes the scores
//   S = Q K^T, the probabilities P = exp2(S sl2 - lse) and dV^T += dO^T P;
// - the dS wave (waves 4-7) holds the V fragments, computes dP = dO V^T,
//   takes P from its partner through LDS (bf16, the operand dV takes too),
//   forms dS = P (dP - delta) and dK^T += Q^T dS.
// Each wave issues 32 MFMAs per tile (one wave of 32 keys issued all 64
// before and held too many registers to share its SIMD); while one wave of
// a SIMD runs its exponentials or dS arithmetic the other's MFMAs proceed.
// The exchange costs one barrier per tile between the two halves.  Q and dO
// tiles are row-major in LDS (3-slot ring, loaded by the P waves); the
// transposes for dV^T and dK^T come from transpose reads.
//
// The grid holds one workgroup per CU and each workgroup walks units (longest
// first, every other round in reverse so that the workgroups' totals even
// out).  Between units every global access is row-contiguous: the unit's K
// and V rows arrive as direct-to-LDS tiles and the fragments are read from
// LDS; dV and dK go through LDS to row layout and out in 16-byte pieces, the
// QK-norm and rotary backward of dK computed in that layout (a row's 128
// values on 16 lanes).
//
// DS: the dS waves also store the bf16 dS of every (query, key) pair into
// a.ds (layout in AttnArgs): each dS fragment the dK MFMAs take (16 bytes
// per lane) is one store of 1 KiB, whole cache lines; a pair whose keys all
// follow a query tile (the diagonal tile) stores zeros there, so that every
// block is complete.
// The body of one role (PW: the P waves, else the dS waves): the two roles
// run the same unit walk and barriers, each with its own loop and registers.
template <bool DS, bool PW>
__device__ __forceinline__ void dkdv_bf16_role(const AttnArgs& a, char* smem, int wave) {
  using namespace fa;
  typedef Mfma<bf16> MM;
  constexpr int QT = 64;
  constexpr int SLOTB = 2 * TILE + 2048;      // Q, dO, lse (1 KiB), delta (1 KiB)
  constexpr bool pw = PW;
  const int lane = threadIdx.x & 63;
  const int kw = wave & 3;                    // key group of the pair: keys 32 kw .. of the unit
  const int BG = a.B * a.G, R = a.H / a.G;
  const int units = ((a.T + 127) / 128) * BG;
  const long ldq = (long)a.LD * 2, ldo = (long)a.C * 2;
  const bf16* qkv = static_cast<const bf16*>(a.qkv);
  const int nqt_all = (a.T + QT - 1) / QT;

  // The units form one queue (key tile major: longest first), or, with the
  // grid and the (sequence, key/value head) pairs both multiples of the 8
  // XCDs (workgroups are dealt to them round robin), one queue per XCD: XCD
  // x takes the pairs x BG/8 .. (x+1) BG/8 - 1, pair by pair, each pair's
  // units longest first, so that the Q and dO tiles the units of a pair all
  // read are fetched into that XCD's L2 once.  Round j of a queue: its
  // workgroups take the next entries, every other round in reverse order.
  const int nku = (a.T + 127) / 128;
  const bool xcd = gridDim.x % 8 == 0 && BG % 8 == 0;
  const int qlen = xcd ? units / 8 : units;
  const int per = xcd ? (int)gridDim.x / 8 : (int)gridDim.x;
  const int wg = xcd ? (int)blockIdx.x / 8 : (int)blockIdx.x;
  auto unit_of = [&](int j) {   // queue entry of round j for this workgroup (>= qlen: none)
    const int i = (j & 1) ? per - 1 - wg : wg;
    return j * per + i;
  };
  // a unit: key tile kt (first key tiles have the most queries), sequence b,
  // key/value head kvh; n iterations = R query heads x nq query tiles
  struct Unit {
    int kt, b, kvh, qt0, nq, n;
  };
  auto make_unit = [&](int e) {
    Unit p;
    int bg;
    if (xcd) {
      bg = ((int)blockIdx.x % 8) * (BG / 8) + e / nku;
      p.kt = e % nku;
    } else {
      p.kt = e / BG;
      bg = e % BG;
    }
    p.b = bg / a.G;
    p.kvh = bg % a.G;
    p.qt0 = (p.kt * 128) / QT;
    // the last query that sees a key of the unit is kt*128 + 127 + W - 1
    const int nqt = min(nqt_all, (int)(((long)p.kt * 128 + 127 + a.W - 1) / QT) + 1);
    p.nq = nqt - p.qt0;
    p.n = R * p.nq;
    return p;
  };
  // iteration it of unit p: query head kvh*R + it/nq, query tile qt0 + it%nq
  // (issued by the P waves)
  auto issue = [&](const Unit& p, int slot, int it) {
    char* d = smem + slot * SLOTB;
    const int h = p.kvh * R + it / p.nq, q0 = (p.qt0 + it % p.nq) * QT;
    const int qoff = h * HD * 2;
    const i32x4 rsq = make_rsrc(qkv + (long)p.b * a.T * a.LD, clamp_bytes((long)a.T * ldq));
    const i32x4 rso = make_rsrc(static_cast<const bf16*>(a.dO) + (long)p.b * a.T * a.C, clamp_bytes((long)a.T * ldo));
    issue_tile(d, rsq, q0, ldq, qoff, wave, lane);
    issue_tile(d + TILE, rso, q0, ldo, qoff, wave, lane);
    if (wave == 0) {
      // lse, delta rows of all the sequence's query heads ([H][T] each)
      const i32x4 rsl = make_rsrc(a.lse + (long)p.b * a.H * a.T, (uint32_t)a.H * a.T * 4);
      const i32x4 rsd = make_rsrc(a.delta + (long)p.b * a.H * a.T, (uint32_t)a.H * a.T * 4);
      issue_vec(d + 2 * TILE, rsl, h * a.T + q0, lane);
      issue_vec(d + 2 * TILE + 1024, rsd, h * a.T + q0, lane);
    }
  };
  // LDS offsets of the fragment reads from one base each: row-fragment read
  // ks at kbase ^ (ks << 5), transpose reads as in frag_vt_x
  int kbase = off(lane & 31, lane >> 5);
  int vbase;
  {
    int vo[8];
    frag_vt_offsets(vo, lane);
    vbase = vo[0];
  }
  // K and V rows of a unit (k rows 0-63, 64-127, then v): ring slot 2 and
  // past the ring, used only between units; the P exchange past those
  char* const kvs = smem + 2 * SLOTB;
  // P of the pair kw, fragment f (half f/2, MFMA chunk f%2): 16 bytes per lane
  lds_char* const pex = (lds_char*)(smem + 2 * SLOTB + 4 * TILE) + kw * 4096 + lane * 16;
  auto issue_kv_rows = [&](const Unit& p) {
    const i32x4 rsq = make_rsrc(qkv + (long)p.b * a.T * a.LD, clamp_bytes((long)a.T * ldq));
    const int k0 = p.kt * 128, ko = (a.KO + p.kvh * HD) * 2, vo = (a.VO + p.kvh * HD) * 2;
    issue_tile(kvs, rsq, k0, ldq, ko, wave, lane);
    issue_tile(kvs + TILE, rsq, k0 + 64, ldq, ko, wave, lane);
    issue_tile(kvs + 2 * TILE, rsq, k0, ldq, vo, wave, lane);
    issue_tile(kvs + 3 * TILE, rsq, k0 + 64, ldq, vo, wave, lane);
  };
  // the pair's 32 key rows (rows 32 (kw & 1) .. of tile kw / 2): K fragments
  // on the P wave, V fragments on the dS wave
  bf16x8 kvf[8];
  auto read_kv = [&]() {
    const lds_char* kb = (const lds_char*)kvs + (pw ? 0 : 2 * TILE) + (kw >> 1) * TILE + (kw & 1) * 8192;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) kvf[ks] = *(lds_bf16x8*)(kb + (kbase ^ (ks << 5)));
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): read before the ring slot 2 is refilled
  };
  // workgroup barrier over LDS only (global accesses in flight stay in flight)
  auto lds_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
  };

  int j = 0;
  if (unit_of(0) >= qlen) return;
  Unit cur = make_unit(unit_of(0));
  if (pw) issue_kv_rows(cur);
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  lds_barrier();
  read_kv();
  if (pw) {
    issue(cur, 0, 0);
    if (cur.n > 1) issue(cur, 1, 1);
  }
  float mx = 0.f;
  for (;;) {
    const int kw0 = cur.kt * 128 + kw * 32;
    const int key = kw0 + (lane & 31);
    const int n = cur.n;
    // dV^T (P wave) or dK^T (dS wave): 128 dims x the pair's 32 keys
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    for (int it = 0; it < n; ++it) {
      // tile it landed: the P waves' loads issued after it (the next tile's:
      // 10 issues on wave 0, 8 on the others) may stay in flight.  The dS
      // waves issue no loads; they keep at most two tiles of dS stores (4
      // each) in flight.
      const bool next = it + 1 < n;
      if (pw) {
        if (!next) wait_vm<0>();
        else if (wave == 0) wait_vm<10>();
        else wait_vm<8>();
      } else if (DS) {
        wait_vm<8>();
      }
      ring_barrier();
      // the bases count as changed here, so that the eight offsets derived from
      // each are not hoisted out of the loop into sixteen live registers
      asm volatile("" : "+v"(kbase), "+v"(vbase));
      if (pw && it + 2 < n) issue(cur, (it + 2) % 3, it + 2);
      const int q0 = (cur.qt0 + it % cur.nq) * QT;
      const lds_char* qt_ = (const lds_char*)smem + (it % 3) * SLOTB;
      const lds_char* ot_ = qt_ + TILE;
      const lds_char* vec = qt_ + 2 * TILE;   // lse (P wave), delta at +1024 (dS wave)
      const bool zero = q0 + QT - 1 < kw0;              // all queries precede all keys of this pair
      const bool skip = zero || q0 > kw0 + 31 + a.W - 1;  // or are past the keys' windows
      // dS block of (query head, key unit, query tile): row = key in the unit
      bf16* dsb = nullptr;
      if constexpr (DS) {
        if (!pw) {
          const int qt = cur.qt0 + it % cur.nq;
          const long pair = (long)cur.kt * nqt_all - (long)cur.kt * (cur.kt - 1) + (qt - 2 * cur.kt);
          dsb = static_cast<bf16*>(a.ds) + (((long)cur.b * a.H + cur.kvh * R + it / cur.nq) * a.dsP + pair) * 8192 +
                kw * 2048 + lane * 8;   // chunk 4 kw, this lane's 16 bytes
          if (zero) {   // zeros, in 4 stores like the computed iterations
#pragma unroll
            for (int c = 0; c < 4; ++c) __builtin_nontemporal_store(u32x4{0u, 0u, 0u, 0u}, (u32x4*)(dsb + 512 * c));
          }
        }
      }
      const bool need_mask = (q0 < kw0 + 31) || (q0 + QT > a.T) || (q0 + QT - 1 >= kw0 + a.W);
      // s: S then P (P wave) or dP then dP - delta (dS wave), per 32-query
      // half qb: rows = queries, column = this lane's key (the first MFMA of
      // each half takes a zero accumulator operand, so no register clearing)
      f32x16 s[2];
      const f32x16 zero16 = {};
      bf16x8 f[16];    // fragments read ahead of their MFMAs
      bf16x8 op[4];    // bf16 P or dS fragments of half f/2, MFMA chunk f%2
      if (!skip) {
        if (pw) {
          // S in 16 steps of one MFMA (Q row fragments three steps ahead);
          // the exponentials of half 0 between the MFMAs of half 1
          auto phase1 = [&](auto maskc) {
            constexpr bool MASK = decltype(maskc)::value;
            f32x4 lv;
            auto pexp = [&](int qb, int g) {
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const int r = 4 * g + e;
                float p = __builtin_amdgcn_exp2f(fmaf(s[qb][r], a.sl2, -lv[e]));
                if constexpr (MASK) {
                  const int qq = q0 + qb * 32 + 8 * g + 4 * (lane >> 5) + e;
                  p = (key > qq || qq >= a.T || qq >= key + a.W) ? 0.f : p;
                }
                s[qb][r] = p;
              }
            };
            auto ldl = [&](int qb, int g) { lv = *(const lds_f32x4*)(vec + (qb * 32 + 8 * g + 4 * (lane >> 5)) * 4); };
            auto rd = [&](int i) { f[i] = *(lds_bf16x8*)(qt_ + (i >> 3) * 8192 + (kbase ^ ((i & 7) << 5))); };
            rd(0);
            rd(1);
            rd(2);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              if (i >= 8 && (i & 1) == 0) {   // lse ahead of this step's fragment read
                ldl(0, (i - 8) >> 1);
                __builtin_amdgcn_sched_barrier(0);
              }
              if (i + 3 < 16) rd(i + 3);
              s[i >> 3] = MM::mma(f[i], kvf[i & 7], (i & 7) ? s[i >> 3] : zero16);
              if (i >= 8 && (i & 1)) pexp(0, (i - 8) >> 1);
              __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              ldl(1, g);
              pexp(1, g);
            }
          };
          if (need_mask) phase1(std::true_type());
          else phase1(std::false_type());
          // P as bf16 fragments, kept for dV and written for the partner
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            op[q] = frag_regs<bf16>(s[q >> 1], (q & 1) * 8);
            *(__attribute__((address_space(3))) bf16x8*)(pex + q * 1024) = op[q];
          }
        } else {
          // dP in 16 steps of one MFMA (dO row fragments three steps ahead);
          // dP - delta of half 0 between the MFMAs of half 1
          f32x4 dl;
          auto sub = [&](int qb, int g) {
#pragma unroll
            for (int e = 0; e < 4; ++e) s[qb][4 * g + e] -= dl[e];
          };
          auto ldd = [&](int qb, int g) {
            dl = *(const lds_f32x4*)(vec + 1024 + (qb * 32 + 8 * g + 4 * (lane >> 5)) * 4);
          };
          auto rd = [&](int i) { f[i] = *(lds_bf16x8*)(ot_ + (i >> 3) * 8192 + (kbase ^ ((i & 7) << 5))); };
          rd(0);
          rd(1);
          rd(2);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            if (i >= 8 && (i & 1) == 0) {
              ldd(0, (i - 8) >> 1);
              __builtin_amdgcn_sched_barrier(0);
            }
            if (i + 3 < 16) rd(i + 3);
            s[i >> 3] = MM::mma(f[i], kvf[i & 7], (i & 7) ? s[i >> 3] : zero16);
            if (i >= 8 && (i & 1)) sub(0, (i - 8) >> 1);
            __builtin_amdgcn_sched_barrier(0);
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            ldd(1, g);
            sub(1, g);
          }
        }
      }
      // P written (the barrier waits for this wave's LDS accesses first)
      ring_barrier();
      if (!skip) {
        // 16 MFMAs over (half qb, MFMA chunk mm, d-block db) = (u >> 3,
        // (u >> 2) & 1, u & 3), transposed fragments three steps ahead
        if (pw) {
          // dV^T += dO^T P
          auto rd = [&](int u) { f[u] = frag_vt_x(ot_, vbase, 2 * (u >> 3) + ((u >> 2) & 1), u & 3); };
          rd(0);
          rd(1);
          rd(2);
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            if (u + 3 < 16) rd(u + 3);
            acc[u & 3] = MM::mma(f[u], op[u >> 2], acc[u & 3]);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
          // dS = P (dP - delta) from the partner's P, then dK^T += Q^T dS
          auto rd = [&](int u) { f[u] = frag_vt_x(qt_, vbase, 2 * (u >> 3) + ((u >> 2) & 1), u & 3); };
          bf16x8 pp[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) pp[q] = *(const lds_bf16x8*)(pex + q * 1024);
          rd(0);
          rd(1);
          rd(2);
          auto dsh = [&](int qb) {
#pragma unroll
            for (int m = 0; m < 2; ++m) {
#pragma unroll
              for (int e = 0; e < 8; ++e) s[qb][8 * m + e] *= (float)pp[2 * qb + m][e];
              op[2 * qb + m] = frag_regs<bf16>(s[qb], m * 8);
              // chunk 4 kw + 2 qb + m: queries qb*32 + 16m + 4(lane/32) + 0..3 and + 8
              if constexpr (DS)
                __builtin_nontemporal_store(__builtin_bit_cast(u32x4, op[2 * qb + m]),
                                            (u32x4*)(dsb + 512 * (2 * qb + m)));
            }
          };
          dsh(0);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int u = 0; u < 16; ++u) {
            if (u + 3 < 16) rd(u + 3);
            acc[u & 3] = MM::mma(f[u], op[u >> 2], acc[u & 3]);
            if (u == 1) dsh(1);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    }
    // ---- unit boundary
    ++j;
    const int un = unit_of(j);
    const bool more = un < qlen;
    const Unit nxt = more ? make_unit(un) : cur;
    lds_barrier();                       // the ring is free
    if (more && pw) issue_kv_rows(nxt);  // into slot 2 and past the ring
    // dV (P waves), then dK (dS waves), through the pair's staging rows in
    // ring slots 0-1, out in row layout; the QK-norm operands of dK's rows
    // are loaded while dV is stored
    float* stg = reinterpret_cast<float*>(smem) + kw * 32 * 128;
    const long row0 = (long)cur.b * a.T + kw0;   // global row of the pair's first key
    const int nrows = min(32, a.T - kw0);
    bf16* const drow = static_cast<bf16*>(a.dqkv) + row0 * a.LD;
    QkRows qk;
    if (pw) {
      stage_acc(stg, acc, 1.f, lane);
      mx = fmaxf(mx, store_rows(stg, drow + a.VO + cur.kvh * HD, a.LD, nrows, lane));
    } else {
      // key QK-norm factors: [N][H] after the query ones, head index kvh
      qk_rows_load(qk, qkv + row0 * a.LD + a.KO + cur.kvh * HD, a.LD,
                   a.rho + ((long)a.B * a.T + row0) * a.H + cur.kvh, a.H, nrows, lane, a.cs, kw0, a.T);
    }
    lds_barrier();                       // dV's staging rows read
    if (!pw) {
      stage_acc(stg, acc, a.rsd, lane);
      mx = fmaxf(mx, store_rows_qk(stg, qk, drow + a.KO + cur.kvh * HD, a.LD, nrows, lane));
    }
    if (!more) break;
    // the next unit's K, V rows have landed (the P waves wait for their
    // loads, the barrier for everyone's) and the staging rows are free
    if (pw) __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    lds_barrier();
    cur = nxt;
    read_kv();
    if (pw) {
      issue(cur, 0, 0);
      if (cur.n > 1) issue(cur, 1, 1);
    }
  }
  if (a.amax_dqkv) amax_publish<bf16>(a.amax_dqkv, mx);
}

template <bool DS>
__global__ __launch_bounds__(512, 1) void attn_bwd_dkdv_bf16_kernel(AttnArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // the wave index as a scalar: the role branch is uniform
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (wave < 4) dkdv_bf16_role<DS, true>(a, smem, wave);
  else dkdv_bf16_role<DS, false>(a, smem, wave);
}

// dQ: one unit of work = 128 queries of one (sequence, head), 4 waves x 32
// queries (Q and dO fragments in registers); it walks the 64-key tiles up to
// the diagonal.  K and V tiles row-major in LDS (3-slot ring); K^T for
// dQ^T += K^T dS^T comes from transpose reads.  Persistent like the dK/dV
// kernel: one workgroup per CU walks the units (longest first, alternate
// rounds reversed); between units the Q and dO rows arrive as direct-to-LDS
// tiles (Q past the ring, dO in ring slot 2) and dQ leaves through LDS
// staging (ring slots 0-1) in row layout, QK-norm and rotary backward
// included.
__global__ __launch_bounds__(256, 1) void attn_bwd_dq_bf16_kernel(AttnArgs a) {
  using namespace fa;
  typedef Mfma<bf16> MM;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int BH = a.B * a.H;
  const int nqt = (a.T + 127) / 128;
  const int units = nqt * BH;
  const long ldb = (long)a.LD * 2, ldo = (long)a.C * 2;
  const bf16* qkv = static_cast<const bf16*>(a.qkv);

  auto unit_of = [&](int j) {
    const int i = (j & 1) ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x;
    return j * (int)gridDim.x + i;
  };
  // a unit: query tile qt (last tiles have the most keys), sequence b, head;
  // n key tiles from kt_lo
  struct Unit {
    int qt, b, head, kvh, kt_lo, n;
  };
  auto make_unit = [&](int u) {
    Unit p;
    p.qt = nqt - 1 - u / BH;
    const int bh = u % BH;
    p.b = bh / a.H;
    p.head = bh % a.H;
    p.kvh = p.head / (a.H / a.G);
    const int last_key = min(a.T - 1, p.qt * 128 + 127);
    p.kt_lo = max(0, p.qt * 128 - a.W + 1) / KT;   // first tile inside the window
    p.n = last_key / KT + 1 - p.kt_lo;
    return p;
  };
  auto issue = [&](const Unit& p, int slot, int it) {   // K, V tile it of unit p
    const i32x4 rs = make_rsrc(qkv + (long)p.b * a.T * a.LD, clamp_bytes((long)a.T * ldb));
    issue_kv(smem + slot * SLOT, rs, (p.kt_lo + it) * KT, ldb, (a.KO + p.kvh * HD) * 2, (a.VO + p.kvh * HD) * 2, wave,
             lane);
  };
  // Q rows of a unit past the ring, dO rows in ring slot 2 (between units)
  char* const qrows = smem + NSLOT * SLOT;
  char* const orows = smem + 2 * SLOT;
  auto issue_rows = [&](const Unit& p) {
    const i32x4 rs = make_rsrc(qkv + (long)p.b * a.T * a.LD, clamp_bytes((long)a.T * ldb));
    const i32x4 ro = make_rsrc(static_cast<const bf16*>(a.dO) + (long)p.b * a.T * a.C, clamp_bytes((long)a.T * ldo));
    const int q0 = p.qt * 128, co = p.head * HD * 2;
    issue_tile(qrows, rs, q0, ldb, co, wave, lane);
    issue_tile(qrows + TILE, rs, q0 + 64, ldb, co, wave, lane);
    issue_tile(orows, ro, q0, ldo, co, wave, lane);
    issue_tile(orows + TILE, ro, q0 + 64, ldo, co, wave, lane);
  };
  // LDS offsets of the fragment reads from one base each (as in the dK/dV kernel)
  int kbase = off(lane & 31, lane >> 5);
  int vbase;
  {
    int vo[8];
    frag_vt_offsets(vo, lane);
    vbase = vo[0];
  }
  bf16x8 qf[8], df[8];
  auto read_rows = [&]() {   // this wave's 32 queries: rows 32 (wave & 1) .. of tile wave / 2
    const int o = (wave >> 1) * TILE + (wave & 1) * 8192;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qf[ks] = *(lds_bf16x8*)((const lds_char*)qrows + o + (kbase ^ (ks << 5)));
      df[ks] = *(lds_bf16x8*)((const lds_char*)orows + o + (kbase ^ (ks << 5)));
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0): read before ring slot 2 is refilled
  };
  auto lds_barrier = [&]() {
    __builtin_amdgcn_s_waitcnt(0xc07f);
    __builtin_amdgcn_s_barrier();
  };

  int j = 0;
  if (unit_of(0) >= units) return;
  Unit cur = make_unit(unit_of(0));
  issue_rows(cur);
  __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
  lds_barrier();
  read_rows();
  issue(cur, 0, 0);
  if (cur.n > 1) issue(cur, 1, 1);
  float mx = 0.f;
  for (;;) {
    const int qw0 = cur.qt * 128 + wave * 32;
    const int q = qw0 + (lane & 31);
    const bool qv = q < a.T;
    const long bhT = ((long)cur.b * a.H + cur.head) * a.T;
    const float lse = qv ? a.lse[bhT + q] : INFINITY;
    const float dlt = qv ? a.delta[bhT + q] : 0.f;
    // these two loads complete here, behind the unit's first two tiles (a
    // wait at their first use inside the loop would drain the ring there
    // every tile)
    wait_vm<0>();
    const int kt_lo = cur.kt_lo, n = cur.n;
    f32x16 acc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
    for (int it = 0; it < n; ++it) {
      if (it + 1 < n) wait_vm<8>();
      else wait_vm<0>();
      ring_barrier();
      asm volatile("" : "+v"(kbase), "+v"(vbase));   // keep the derived offsets in the loop
      if (it + 2 < n) issue(cur, (it + 2) % NSLOT, it + 2);
      const lds_char* kt_ = (const lds_char*)smem + (it % NSLOT) * SLOT;
      const lds_char* vt_ = kt_ + TILE;
      const int k0 = (kt_lo + it) * KT;
      if (k0 > qw0 + 31) continue;
      if (k0 + KT - 1 <= qw0 - a.W) continue;           // every key is before this wave's windows
      const bool need_mask = (k0 + KT - 1 > qw0) || (k0 + KT > a.T) || (k0 <= qw0 + 31 - a.W);
      // Two 32-key halves in 24 steps of two MFMAs: S^T/dP^T(0); S^T/dP^T(1)
      // with dS(0); dQ(0) with dS(1); dQ(1).  As in the dK/dV kernel, each step
      // issues the LDS reads of the step after next and ends with a scheduling
      // fence.  Masked and unmasked tiles are separate copies.
      auto body = [&](auto maskc) {
        constexpr bool MASK = decltype(maskc)::value;
        f32x16 sv[2] = {}, dp[2] = {};
        bf16x8 fa[24], fb[24];
        auto rd = [&](int i) {
          if (i < 16) {        // K and V rows of half i/8, k-step i%8
            const int kb = i >> 3, ks = i & 7;
            fa[i] = *(lds_bf16x8*)(kt_ + kb * 8192 + (kbase ^ (ks << 5)));
            fb[i] = *(lds_bf16x8*)(vt_ + kb * 8192 + (kbase ^ (ks << 5)));
          } else {             // K^T of half, MFMA chunk, d-blocks d2 and d2+1
            const int u = i - 16, kb = u >> 2, m2 = (u >> 1) & 1, d2 = 2 * (u & 1);
            fa[i] = frag_vt_x(kt_, vbase, 2 * kb + m2, d2);
            fb[i] = frag_vt_x(kt_, vbase, 2 * kb + m2, d2 + 1);
          }
        };
        auto dsr = [&](int kb, int r) {   // dS^T of score r of half kb
          float p = __builtin_amdgcn_exp2f(fmaf(sv[kb][r], a.sl2, -lse));
          if constexpr (MASK) {
            const int kk = k0 + kb * 32 + acc_row(r, lane);
            p = (kk > q || kk >= a.T || kk <= q - a.W) ? 0.f : p;
          }
          sv[kb][r] = p * (dp[kb][r] - dlt);
        };
        bf16x8 sf[2];          // bf16 dS^T of the half being multiplied
        rd(0);
        rd(1);
  #pragma unroll
        for (int i = 0; i < 24; ++i) {
          if (i + 2 < 24) rd(i + 2);
          if (i < 16) {
            const int kb = i >> 3, ks = i & 7;
            sv[kb] = MM::mma(fa[i], qf[ks], sv[kb]);   // S^T
            dp[kb] = MM::mma(fb[i], df[ks], dp[kb]);   // dP^T
            if (kb == 1) {
              dsr(0, 2 * ks);
              dsr(0, 2 * ks + 1);
            }
          } else {
            const int u = i - 16, kb = u >> 2, m2 = (u >> 1) & 1, d2 = 2 * (u & 1);
            if ((u & 3) == 0) {
              sf[0] = frag_regs<bf16>(sv[kb], 0);
              sf[1] = frag_regs<bf16>(sv[kb], 8);
            }
            acc[d2] = MM::mma(fa[i], sf[m2], acc[d2]);           // dQ^T += K^T dS^T
            acc[d2 + 1] = MM::mma(fb[i], sf[m2], acc[d2 + 1]);
            if (kb == 0) {
  #pragma unroll
              for (int e = 0; e < 4; ++e) dsr(1, 4 * u + e);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      };
      if (need_mask) body(std::true_type());
      else body(std::false_type());
    }
    // ---- unit boundary
    ++j;
    const int un = unit_of(j);
    const bool more = un < units;
    const Unit nxt = more ? make_unit(un) : cur;
    lds_barrier();                 // the ring is free
    if (more) issue_rows(nxt);     // past the ring and into slot 2
    float* stg = reinterpret_cast<float*>(smem) + wave * 32 * 128;   // slots 0-1
    const long row0 = (long)cur.b * a.T + qw0;
    const int nrows = min(32, a.T - qw0);
    QkRows qk;
    qk_rows_load(qk, qkv + row0 * a.LD + cur.head * HD, a.LD, a.rho + row0 * a.H + cur.head, a.H, nrows, lane, a.cs,
                 qw0, a.T);
    stage_acc(stg, acc, a.rsd, lane);
    mx = fmaxf(mx, store_rows_qk(stg, qk, static_cast<bf16*>(a.dqkv) + row0 * a.LD + cur.head * HD, a.LD, nrows,
                                 lane));
    if (!more) break;
    // the next unit's Q, dO rows have landed and the staging rows are free
    __builtin_amdgcn_s_waitcnt(0x0f70);   // vmcnt(0)
    lds_barrier();
    cur = nxt;
    read_rows();
    issue(cur, 0, 0);
    if (cur.n > 1) issue(cur, 1, 1);
  }
  if (a.amax_dqkv) amax_publish<bf16>(a.amax_dqkv, mx);
}

// dQ from the stored dS: dQ^T (d x query) = K^T dS^T per unit of 128
// queries of one (sequence, query head), over the 32-key tiles up to the
// diagonal.  Four waves of 32 queries; per key tile the K rows and the dS^T
// rows (keys x the unit's 128 queries, 4 KiB of each of its two 64-query
// blocks) arrive in LDS by direct-to-LDS loads, four tiles ahead in a
// five-slot ring (the kernel streams dS from HBM once: the bytes in flight
// set its speed); both fragments come from the LDS transpose read in the
// same key order.  A dS^T row in LDS holds the stored 16-byte pieces, so
// within each 16 queries its positions 4..7 and 8..11 hold queries 8..11 and
// 4..7: lane l of a wave accumulates query qperm(l % 32), and the epilogue
// (the dQ kernel's: QK-norm and rotary backward in row layout) stages it in
// that row.  One workgroup per unit, two per CU; the units of one (sequence,
// head) run on one XCD, longest first, so that its K rows stay in that L2.
namespace fa {
constexpr int DSQ_KT = 32;                       // keys per tile
constexpr int DSQ_TILE = DSQ_KT * 256;           // bytes of a [32][128] bf16 tile
constexpr int DSQ_SLOT = 2 * DSQ_TILE;           // K tile, dS^T tile
constexpr int DSQ_NSLOT = 5;
constexpr int DSQ_LDS = DSQ_NSLOT * DSQ_SLOT;    // 80 KiB: two workgroups fill a CU's LDS
// The dS^T tile is two sub-tiles (the unit's two 64-query blocks) of 32 key
// rows x 128 bytes; chunk c (16 bytes) of row r sits at c ^ dsq_sw(r).  A
// 16-lane transpose read touches 4 consecutive rows x 2 adjacent chunks: the
// 8 pieces fall in distinct 16-byte bank groups of a 128-byte (32-bank) line,
// and a 32-lane read's 16 pieces in distinct groups of a 256-byte (64-bank)
// line.
__device__ __forceinline__ int dsq_sw(int row) { return 2 * (row & 3); }
}  // namespace fa
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_ds_kernel(AttnArgs a) {
  using namespace fa;
  typedef Mfma<bf16> MM;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int BH = a.B * a.H;
  const int nu = (a.T + 127) / 128, nqt_all = (a.T + 63) / 64;
  // workgroups are dealt round robin to the 8 XCDs: XCD x walks the units
  // x * total/8 .. in order, (sequence, head) by (sequence, head)
  const int total = nu * BH;
  int pid = blockIdx.x;
  if (total % 8 == 0) pid = (pid % 8) * (total / 8) + pid / 8;
  const int bh = pid / nu;
  const int u = nu - 1 - pid % nu;                    // longest units first
  const int b = bh / a.H, head = bh % a.H, kvh = head / (a.H / a.G);
  const long ldb = (long)a.LD * 2;
  const bf16* qkv = static_cast<const bf16*>(a.qkv);
  const i32x4 rk = make_rsrc(qkv + (long)b * a.T * a.LD, clamp_bytes((long)a.T * ldb));
  const i32x4 rd = make_rsrc(static_cast<const bf16*>(a.ds) + (long)bh * a.dsP * 8192,
                             clamp_bytes((long)a.dsP * 16384));
  const int koff = (a.KO + kvh * HD) * 2;
  const int n = min(4 * u + 4, (a.T + DSQ_KT - 1) / DSQ_KT);   // key tiles 0 .. n-1
  // the QK-norm and rotary operands of the epilogue, loaded first: every
  // tile wait below also covers them (completion follows issue order), and
  // the epilogue finds them in registers
  const int qw0 = u * 128 + wave * 32;
  const long row0 = (long)b * a.T + qw0;
  const int nrows = min(32, a.T - qw0);
  QkRows qk;
  qk_rows_load(qk, qkv + row0 * a.LD + head * HD, a.LD, a.rho + row0 * a.H + head, a.H, nrows, lane, a.cs, qw0, a.T);
  // key tile t: K rows 32t..; the dS pieces of keys 32 (t & 3).. (1 KiB chunks
  // 4 (t & 3) .. 4 (t & 3) + 3) of blocks (t / 4, 2u) and (t / 4, 2u + 1)
  auto issue = [&](int slot, int t) {
    char* d = smem + slot * DSQ_SLOT;
    const int kt = t >> 2;
    const long pair = (long)kt * nqt_all - (long)kt * (kt - 1) + (2 * u - 2 * kt);
    const long row0 = pair * 16384 + (long)(t & 3) * 4096;   // bytes: block (kt, 2u), chunk 4 (t & 3)
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int base = wave * 128 + i * 64;
      const int p = base + lane;
      const int row = p >> 4, c = (p & 15) ^ sw(row);
      const uint32_t ok = (uint32_t)((long)(t * DSQ_KT + row) * ldb + koff + c * 16);
      dma16(rk, (lds_u32*)(d + base * 16), ok);
      // dS^T slot p: sub-tile blk (query block 2u + blk), key row r, chunk cd
      // (8 queries: 1 KiB chunk cd/2 of the block's stored fragments, piece
      // of key row r + 32 (cd & 1)); one issue covers 8 key rows of a
      // sub-tile, so it reads 8 whole 128-byte lines
      const int blk = p >> 8, r = (p >> 3) & 31, cd = (p & 7) ^ dsq_sw(r);
      const uint32_t od = (uint32_t)(row0 + blk * 16384 + (cd >> 1) * 1024 + (r + 32 * (cd & 1)) * 16);
      dma16_nt(rd, (lds_u32*)(d + DSQ_TILE + base * 16), od);
    }
  };
  int vbase;
  {
    int vo[8];
    frag_vt_offsets(vo, lane);
    vbase = vo[0];
  }
  // dS^T transpose read of this lane (as frag_vt_x: keys 4 (g/2) + s/4, the
  // 4 queries from 16 (g & 1) + 4 (s & 3) of the wave's 32); keys + 8 (the
  // second read) and + 16 (MFMA chunk 1) keep the swizzle
  int sbase;
  {
    const int g = (lane >> 4) & 3, s = lane & 15;
    const int key = 4 * (g >> 1) + (s >> 2), col = (wave & 1) * 32 + 16 * (g & 1) + 4 * (s & 3);
    sbase = (wave >> 1) * 4096 + key * 128 + (((col >> 3) ^ dsq_sw(key)) << 4) + (col & 7) * 2;
  }
  auto frag_ds = [&](const lds_char* st, int mm) {
    const lds_char* q = st + mm * 2048 + sbase;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)q);
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(q + 1024));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, r);
  };
  f32x16 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  for (int t = 0; t < DSQ_NSLOT - 1 && t < n; ++t) issue(t, t);
  for (int t = 0; t < n; ++t) {
    // tile t landed (own loads, then everyone's; each tile is 4 issues per
    // wave, tiles t+1 .. t+3 may stay in flight); the slot of tile t-1 is free
    if (t + 3 < n) wait_vm<12>();
    else if (t + 2 < n) wait_vm<8>();
    else if (t + 1 < n) wait_vm<4>();
    else wait_vm<0>();
    ring_barrier();
    if (t + 4 < n) issue((t + 4) % DSQ_NSLOT, t + 4);
    const lds_char* kt_ = (const lds_char*)smem + (t % DSQ_NSLOT) * DSQ_SLOT;
    const lds_char* st_ = kt_ + DSQ_TILE;
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const bf16x8 bf = frag_ds(st_, mm);   // dS^T: this wave's 32 queries
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] = MM::mma(frag_vt_x(kt_, vbase, mm, db), bf, acc[db]);
    }
  }
  __syncthreads();   // every wave is done with the slots: they become staging rows
  float* stg = reinterpret_cast<float*>(smem) + wave * 32 * 128;
  // lane l holds query qperm(l % 32): bits 2 and 3 of the position swapped
  const int l32 = lane & 31;
  stage_acc(stg, acc, a.rsd, lane, (l32 & 0x13) | ((l32 & 4) << 1) | ((l32 & 8) >> 1));
  const float mx =
      store_rows_qk(stg, qk, static_cast<bf16*>(a.dqkv) + row0 * a.LD + head * HD, a.LD, nrows, lane);
  if (a.amax_dqkv) amax_publish<bf16>(a.amax_dqkv, mx);
}

template <typename T> constexpr int attn_fwd_lds() { return 2 * (AttnCfg<T>::ROWT + AttnCfg<T>::TRT); }
template <typename T> constexpr int attn_dq_lds() { return 2 * (2 * AttnCfg<T>::ROWT + AttnCfg<T>::TRT); }
template <typename T> constexpr int attn_dkdv_lds() {
  return 2 * (2 * AttnCfg<T>::ROWT + 2 * AttnCfg<T>::TRT + 2 * AttnCfg<T>::RT * 4);
}

}  // namespace blk
