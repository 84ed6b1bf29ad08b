// Attention kernels and their launchers, a translation unit of its own so
// that it can be compiled with MFMA results placed in vector registers (see
// attn_args.cuh).  Everything else in the library launches attention through
// the three functions below.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>
#include <set>

#include "attention.cuh"

namespace blk {
namespace {

std::mutex g_mu;
std::set<const void*> g_done;

// Raise a kernel's dynamic LDS limit once (past 64 KiB it must be raised).
void allow_lds(const void* kern, int bytes) {
  std::lock_guard<std::mutex> l(g_mu);
  if (g_done.insert(kern).second) hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

int tiles(int n, int t) { return (n + t - 1) / t; }

// dK/dV: three ring slots of Q, dO, lse, delta; between units the K, V rows
// of a unit take slot 2 and 30 KiB past it; then 16 KiB of P exchange
constexpr int DKDV_SLOT = 2 * fa::TILE + 2048;
constexpr int DKDV_LDS = 2 * DKDV_SLOT + 4 * fa::TILE + 16384;
static_assert(DKDV_LDS - 16384 >= 3 * DKDV_SLOT && DKDV_LDS <= 160 * 1024, "dK/dV LDS");
static_assert(4 * 32 * 128 * 4 <= 2 * DKDV_SLOT, "dK/dV staging rows fit in ring slots 0-1");
static_assert(4 * 32 * 128 * 4 <= fa::DSQ_LDS, "dQ-from-dS staging rows fit in its two slots");
// dQ: the K/V ring, then the Q rows of a unit (its dO rows use ring slot 2)
constexpr int DQ_LDS = fa::LDS + 2 * fa::TILE;
static_assert(DQ_LDS <= 160 * 1024 && 4 * 32 * 128 * 4 <= 2 * fa::SLOT && 2 * fa::TILE <= fa::SLOT, "dQ LDS");

}  // namespace

// Compute units of the current device (the grid of the persistent kernels:
// one workgroup per CU); looked up once per device.
int cu_count() {
  static std::mutex mu;
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  std::lock_guard<std::mutex> l(mu);
  if (cached[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}


void attn_fwd(const AttnArgs& a, bool bf16, hipStream_t st) {
  if (bf16) {
    // the windowed instance only when the window is shorter than the sequence
    auto kern = a.W < a.T ? attn_fwd_bf16_kernel<true> : attn_fwd_bf16_kernel<false>;
    allow_lds(reinterpret_cast<const void*>(kern), fa::LDS);
    hipLaunchKernelGGL(kern, dim3(tiles(a.T, fa::QWG) * a.B * a.H), dim3(512), fa::LDS, st, a);
  } else {
    allow_lds(reinterpret_cast<const void*>(attn_fwd_kernel<float>), attn_fwd_lds<float>());
    hipLaunchKernelGGL(attn_fwd_kernel<float>, dim3(tiles(a.T, 128) * a.B * a.H), dim3(256), attn_fwd_lds<float>(),
                       st, a);
  }
}

void attn_bwd_dkdv(const AttnArgs& a, bool bf16, hipStream_t st) {
  // a unit of work per 128 keys of a (sequence, key/value head)
  const int units = tiles(a.T, 128) * a.B * a.G;
  const dim3 grid(units);
  if (bf16) {
    // persistent: one workgroup per CU walks the units; with a.ds it also
    // stores dS for the dQ kernel
    auto kern = a.ds ? attn_bwd_dkdv_bf16_kernel<true> : attn_bwd_dkdv_bf16_kernel<false>;
    allow_lds(reinterpret_cast<const void*>(kern), DKDV_LDS);
    hipLaunchKernelGGL(kern, dim3(std::min(units, cu_count())), dim3(512), DKDV_LDS, st, a);
  } else {
    allow_lds(reinterpret_cast<const void*>(attn_bwd_dkdv_kernel<float>), attn_dkdv_lds<float>());
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<float>, grid, dim3(256), attn_dkdv_lds<float>(), st, a);
  }
}

void attn_bwd_dq(const AttnArgs& a, bool bf16, hipStream_t st) {
  // a unit of work per 128 queries of a (sequence, head)
  const int units = tiles(a.T, 128) * a.B * a.H;
  const dim3 grid(units);
  if (bf16 && a.ds) {
    // dQ = dS K from the dS the dK/dV kernel stored: a workgroup per unit
    allow_lds(reinterpret_cast<const void*>(attn_bwd_dq_ds_kernel), fa::DSQ_LDS);
    hipLaunchKernelGGL(attn_bwd_dq_ds_kernel, grid, dim3(256), fa::DSQ_LDS, st, a);
  } else if (bf16) {
    // persistent: one workgroup per CU walks the units
    allow_lds(reinterpret_cast<const void*>(attn_bwd_dq_bf16_kernel), DQ_LDS);
    hipLaunchKernelGGL(attn_bwd_dq_bf16_kernel, dim3(std::min(units, cu_count())), dim3(256), DQ_LDS, st, a);
  } else {
    allow_lds(reinterpret_cast<const void*>(attn_bwd_dq_kernel<float>), attn_dq_lds<float>());
    hipLaunchKernelGGL(attn_bwd_dq_kernel<float>, grid, dim3(256), attn_dq_lds<float>(), st, a);
  }
}

}  // namespace blk
