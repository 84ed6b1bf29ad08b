// Arguments of the attention kernels and their host launchers.  The kernels
// themselves (attention.cuh) are compiled in a translation unit of their own
// (attn.hip), with MFMA results kept in ordinary vector registers: the
// score and probability blocks feed vector arithmetic after every MFMA chain,
// and with the compiler's default placement of MFMA results in accumulation
// registers they were copied back and forth several times per MFMA.
#pragma once
#include "common.cuh"

namespace blk {

constexpr int HD = 128;   // head size

struct AttnArgs {
  const void* qkv;   // [B*T, LD]: q'' (H heads) | k'' (G) | v (G), heads contiguous in each
  void* o;           // [B*T, C]
  float* lse;        // [B*H, T], log2-domain log-sum-exp of the scaled scores
  const void* dO;    // [B*T, C]
  const float* delta;  // [B*H, T] rowsum(dO * O)
  void* dqkv;        // [B*T, LD]: dq'' | dk'' | dv; bf16 kernels: dq' | dk' | dv
  const float* rho;    // [2][B*T][H] QK-norm factors (bf16 backward kernels)
  const float2* cs;    // [T][64] rotary angles (bf16 backward kernels)
  unsigned* amax_o;    // fp8 mode: absolute maxima (float bits) of o and of
  unsigned* amax_dqkv; //   dq' | dk' | dv, or null
  // bf16 causal backward: the dK/dV kernel stores dS here and dQ = dS K is
  // computed from it (null: the dQ kernel recomputes dS).  Per (sequence,
  // query head) dsP blocks of 16 KiB, one per pair of a 128-key unit kt and a
  // 64-query tile qt >= 2 kt, in the order of kt, then qt; dsP = sum over kt
  // of (query tiles - 2 kt).  A block holds the 128 x 64 bf16 dS values as 16
  // chunks of 1 KiB, chunk 4w + 2qb + m for keys 32w .. 32w+31 and queries
  // 32qb + 16m .. +15; within a chunk, 16 bytes per key k and half h (at
  // byte 16 (k + 32h)): queries 4h + {0..3} and 8 + 4h + {0..3} of the 16.
  void* ds;
  int dsP;
  int B, T, H, C;
  int G;             // key/value heads (query head h uses key/value head h / (H/G))
  int LD;            // elements per row of qkv / dqkv: C + 2 G D
  int KO, VO;        // column of the first key / value head in a qkv row: C, C + G D
  int W;             // attention window: query i sees keys i - W < j <= i (W >= T: causal)
  float sl2;         // log2(e) / sqrt(D)
  float rsd;         // 1 / sqrt(D)
};

// Launchers (attn.hip).  bf16: the gfx950 pipelines (direct-to-LDS staging,
// QK-norm and rotary backward applied in the stores of dq and dk); otherwise
// the float32 kernels.  Grids, LDS sizes and kernel attributes are theirs.
void attn_fwd(const AttnArgs& a, bool bf16, hipStream_t st);
void attn_bwd_dkdv(const AttnArgs& a, bool bf16, hipStream_t st);
void attn_bwd_dq(const AttnArgs& a, bool bf16, hipStream_t st);
// Compute units of the current device (the grid of the persistent kernels;
// attn.hip, looked up once per device).
int cu_count();

}  // namespace blk
