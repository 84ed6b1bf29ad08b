// Device-side basics shared by the gfx950 kernels: element types, 16-byte
// chunk moves, MFMA operand traits, wave reductions and the LDS tile swizzle.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace blk {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

// One E4M3 code (OCP FP8); a distinct type so templates can tell it apart.
struct fp8e4 { uint8_t v; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE (v_cvt_pk_bf16_f32)

// 16-byte global/LDS moves.
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }
__device__ __forceinline__ void st8(void* p, u32x2 v) { *reinterpret_cast<u32x2*>(p) = v; }

// Elements of one 16-byte chunk, as float.
template <typename T> struct Chunk;
template <> struct Chunk<bf16> {
  static constexpr int N = 8;
  __device__ static void unpack(u32x4 c, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(c[i] << 16);
      f[2 * i + 1] = __uint_as_float(c[i] & 0xffff0000u);
    }
  }
  __device__ static u32x4 pack(const float* f) {
    bf16x8 b;
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = (bf16)f[i];
    return __builtin_bit_cast(u32x4, b);
  }
};
template <> struct Chunk<float> {
  static constexpr int N = 4;
  __device__ static void unpack(u32x4 c, float* f) {
#pragma unroll
    for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(c[i]);
  }
  __device__ static u32x4 pack(const float* f) {
    u32x4 c;
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = __float_as_uint(f[i]);
    return c;
  }
};

// MFMA 32x32 operand traits.  One instruction: D[32x32] += A[32xKI] B[KIx32].
// Lane l holds, of A, row l%32 and E consecutive k-slots starting at
// (l/32)*E; of B, column l%32 and the same k-slots.  The float32 result: lane
// l, register j holds D[8*(j/4) + 4*(l/32) + j%4][l%32].
template <typename T> struct Mfma;
template <> struct Mfma<bf16> {
  static constexpr int KI = 16, E = 8;
  typedef bf16x8 frag;
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<float> {
  static constexpr int KI = 2, E = 1;
  typedef float frag;
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};
template <> struct Mfma<fp8e4> {
  static constexpr int KI = 64, E = 32;
  typedef i32x8 frag;
  __device__ static f32x16 mma(frag a, frag b, f32x16 c) {
    // format code 0 = E4M3 for both operands; unit (2^0) block scales
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// s_waitcnt vmcnt(N): wait until at most N vector memory operations of this
// wave are outstanding (loads and stores both count, and complete in issue
// order); the LDS and export counters are not waited for.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt has 6 bits");
  __builtin_amdgcn_s_waitcnt(0x0f70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ int acc_row(int j, int lane) { return 8 * (j >> 2) + 4 * (lane >> 5) + (j & 3); }

// Lane moves inside a row of 16 lanes through DPP (a VALU operand modifier;
// __shfl_xor goes through ds_bpermute, an LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;     // quad_perm [1,0,3,2]: lane i <- lane i^1
constexpr int DPP_XOR2 = 0x4E;     // quad_perm [2,3,0,1]: lane i <- lane i^2
constexpr int DPP_MIRROR = 0x140;  // row_mirror: lane i <- lane 15-i of the row
constexpr int DPP_XOR8 = 0x128;    // row_ror:8: lane i <- lane i^8 of the row

// Sum and maximum over each row of 16 lanes.  Every lane of the row ends
// with the same bits: each step combines two values that the partner lanes
// hold in swapped order (after the quad steps all four lanes of a quad agree;
// the mirror pairs quad k with quad 3-k, the rotation quad k with quad k^2).
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_mov<DPP_XOR1>(v);
  v += dpp_mov<DPP_XOR2>(v);
  v += dpp_mov<DPP_MIRROR>(v);
  return v + dpp_mov<DPP_XOR8>(v);
}
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, dpp_mov<DPP_XOR1>(v));
  v = fmaxf(v, dpp_mov<DPP_XOR2>(v));
  v = fmaxf(v, dpp_mov<DPP_MIRROR>(v));
  return fmaxf(v, dpp_mov<DPP_XOR8>(v));
}

// Wave-wide reductions (64 lanes, all of them active): the rows' results
// are read into scalar registers and combined in one order, so every lane
// returns the same bits.
__device__ __forceinline__ float lane_value(float v, int lane) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  return (lane_value(v, 0) + lane_value(v, 16)) + (lane_value(v, 32) + lane_value(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  return fmaxf(fmaxf(lane_value(v, 0), lane_value(v, 16)), fmaxf(lane_value(v, 32), lane_value(v, 48)));
}

// Folds the wave's largest stored magnitude into *amax (float bits; a zero
// word is the identity, and non-negative floats order like their bits).  m
// is this lane's max |v| before rounding to T: rounding is monotone, so the
// rounded maximum is the maximum of the rounded values.  Every lane of the
// wave must call it.
// Waves whose maximum does not exceed the word's current value (read at
// device scope, so not a stale L1 copy) skip the atomic: once the word holds
// the tensor's maximum almost no wave contends for it.  A stale, smaller read
// only costs an extra atomic; within a kernel the word never decreases.
template <typename T>
__device__ __forceinline__ void amax_publish(unsigned* amax, float m) {
  m = to_f32(from_f32<T>(wave_max(m)));
  if ((threadIdx.x & 63) == 0) {
    const unsigned cur = __hip_atomic_load(amax, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (__float_as_uint(m) > cur) atomicMax(amax, __float_as_uint(m));
  }
}

// LDS tiles are arrays of rows made of 16-byte chunks.  Chunk c of row r is
// stored at chunk position c ^ swz(r): rows that are read together by the
// 32 lanes of an MFMA fragment (consecutive rows) and rows written together
// by the transposing stagers (rows 8 apart) fall on different banks.
__device__ __forceinline__ int swz(int row, int nchunks) { return (row ^ (row >> 3)) & (nchunks - 1); }
__device__ __forceinline__ int tile_off(int row, int chunk, int nchunks) {
  return (row * nchunks + (chunk ^ swz(row, nchunks))) * 16;
}

// Transpose an n x n block of elements held as n 16-byte rows (n = 8 for
// 2-byte, 4 for 4-byte elements): out[c] element r = in[r] element c.
__device__ __forceinline__ void transpose_chunks(const u32x4* in, u32x4* out, bf16*) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t lo = in[2 * i][c >> 1], hi = in[2 * i + 1][c >> 1];
      lo = (c & 1) ? (lo >> 16) : (lo & 0xffffu);
      hi = (c & 1) ? (hi & 0xffff0000u) : (hi << 16);
      out[c][i] = lo | hi;
    }
  }
}
__device__ __forceinline__ void transpose_chunks(const u32x4* in, u32x4* out, float*) {
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) out[c][r] = in[r][c];
}
__device__ __forceinline__ void transpose_chunks(const u32x4* in, u32x4* out, fp8e4*) {
  // 16 x 16 bytes
#pragma unroll
  for (int c = 0; c < 16; ++c) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t w = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        uint32_t src = in[4 * i + b][c >> 2];
        w |= ((src >> (8 * (c & 3))) & 0xffu) << (8 * b);
      }
      out[c][i] = w;
    }
  }
}

// ---- buffer resources -------------------------------------------------------
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint32_t lds_u32;

__device__ void raw_buffer_load_lds(i32x4 rsrc, lds_u32* lds, int size, int voffset, int soffset, int offset,
                                    int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");
__device__ u32x4 raw_buffer_load_b128(i32x4 rsrc, int voffset, int soffset, int aux) __asm(
    "llvm.amdgcn.raw.buffer.load.v4i32");

// A direct-to-LDS load of 16 bytes per lane (the lanes write 16 consecutive
// bytes each from `lds`, the destination of lane 0, uniform), written in
// assembly: the compiler does not see it as a write to LDS.  After a write
// it does see, it makes the next LDS read wait for every vector memory
// operation in flight (vmcnt(0)), which empties a prefetch ring at every
// tile.  Kernels that use it wait for their loads with explicit counts
// (wait_vm) before the barrier (ring_barrier) that publishes a tile; the
// instruction writes no register, so nothing of the compiler's is in flight.
__device__ __forceinline__ void dma16(i32x4 rsrc, const lds_u32* lds, uint32_t voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

// dma16 with the non-temporal cache policy: for data read once (streamed
// through L2 without displacing what other workgroups still re-read).
__device__ __forceinline__ void dma16_nt(i32x4 rsrc, const lds_u32* lds, uint32_t voffset) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(m0), "v"(voffset), "s"(rsrc)
               : "memory", "m0");
}

// Workgroup barrier for LDS rings filled by dma16: waits for this wave's
// own LDS accesses, then for every wave; unlike __syncthreads (whose memory
// fence waits for all global loads in flight) it leaves the prefetched
// tiles in flight.  Also a hard scheduling and memory-ordering boundary.
__device__ __forceinline__ void ring_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
  __builtin_amdgcn_sched_barrier(0);
  __asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Buffer resource over [p, p + bytes): loads at offsets >= bytes return 0.
__device__ __forceinline__ i32x4 make_rsrc(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xffff), (int)bytes, 0x00020000};
}

__device__ __forceinline__ uint32_t clamp_bytes(long b) { return b > 0xffffffffL ? 0xffffffffu : (uint32_t)b; }

}  // namespace blk
