// C ABI of the decoder-block library (declared in include/blk.h): argument
// checks, carving of the caller's saved/scratch buffers, and the launch
// sequences of the forward and backward passes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstring>
#include <mutex>
#include <set>
#include <type_traits>
#include <vector>

#include "../../include/blk.h"
#include "attn_args.cuh"
#include "decode.cuh"
#include "elementwise.cuh"
#include "fp8.cuh"
#include "gemm.cuh"
#include "head.cuh"

using namespace blk;

// decode_step_noalloc's temporaries live in this array: each GPU the library
// runs on holds one copy of it, from the load of the library's code to the
// end of the process.  Host code never names it: its device address (per
// device) comes from hipGetSymbolAddress, taken once per device on the
// entry point's first call there, with that device current.
static __device__ __align__(256) char noalloc_scratch[BLK_NOALLOC_SCRATCH_BYTES];

namespace {

// ---------------------------------------------------------------- layout
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* p) : base(static_cast<char*>(p)) {}
  template <typename X> X* take(size_t count) {
    off = (off + 255) & ~size_t(255);
    X* p = base ? reinterpret_cast<X*>(base + off) : nullptr;
    off += count * sizeof(X);
    return p;
  }
};

// Activations block_fwd keeps for block_bwd (element type T).
template <typename T> struct Saved {
  float2* cs;    // [T][64] rotary (cos, sin)
  float* r1;     // [N]
  T* h1;         // [N, C]
  T* qkv;        // [N, 3C]  q'' | k'' | v
  float* rho;    // [2][N][H]
  T* o;          // [N, C]
  float* lse;    // [B*H][T]
  float* r2;     // [N]
  T* h2;         // [N, C]
  T* a;          // [N, F]
  // fp8 mode: transposed E4M3 copies of the weight-gradient operands, [*, Np]
  // with Np = N rounded up to 64 (zero padding), and the 16 amax slots
  uint8_t *h1_8t = nullptr, *o_8t = nullptr, *h2_8t = nullptr, *a_8t = nullptr;
  unsigned* amax = nullptr;
  size_t bytes;
};

long pad64(long n) { return (n + 63) / 64 * 64; }

// Key/value heads G (grouped-query attention; G = H without grouping) and
// the width of the fused projection's rows, q | k | v = (H + 2G) x 128.
int kv_heads(const blk_cfg& c) { return c.n_kv_head > 0 ? c.n_kv_head : c.H; }
int kv_heads(const blk_dcfg& c) { return c.n_kv_head > 0 ? c.n_kv_head : c.H; }
long qkv_width(const blk_cfg& c) { return (long)c.C + 256L * kv_heads(c); }
long qkv_width(const blk_dcfg& c) { return (long)c.C + 256L * kv_heads(c); }

template <typename T> Saved<T> carve_saved(const blk_cfg& c, void* p) {
  const long N = (long)c.B * c.T;
  Carver k(p);
  Saved<T> s;
  s.cs = k.take<float2>((size_t)c.T * 64);
  s.r1 = k.take<float>(N);
  s.h1 = k.take<T>(N * c.C);
  s.qkv = k.take<T>(N * qkv_width(c));
  s.rho = k.take<float>(2 * N * c.H);
  s.o = k.take<T>(N * c.C);
  s.lse = k.take<float>((size_t)c.B * c.H * c.T);
  s.r2 = k.take<float>(N);
  s.h2 = k.take<T>(N * c.C);
  s.a = k.take<T>(N * c.F);
  if (c.gemm == BLK_GEMM_FP8_E4M3) {
    const long Np = pad64(N);
    s.h1_8t = k.take<uint8_t>(c.C * Np);
    s.o_8t = k.take<uint8_t>(c.C * Np);
    s.h2_8t = k.take<uint8_t>(c.C * Np);
    s.a_8t = k.take<uint8_t>(c.F * Np);
    s.amax = k.take<unsigned>(16);
  }
  s.bytes = (k.off + 255) & ~size_t(255);
  return s;
}

// fp8-mode forward temporaries: row-major E4M3 operands and weights.
struct Fwd8 {
  uint8_t *h1, *o, *h2, *a, *wqkv, *wo, *wfc, *wproj;
  size_t bytes;
};
Fwd8 carve_fwd8(const blk_cfg& c, void* p) {
  const long N = (long)c.B * c.T, C = c.C, F = c.F;
  Carver k(p);
  Fwd8 f;
  f.h1 = k.take<uint8_t>(N * C);
  f.o = k.take<uint8_t>(N * C);
  f.h2 = k.take<uint8_t>(N * C);
  f.a = k.take<uint8_t>(N * F);
  f.wqkv = k.take<uint8_t>(qkv_width(c) * C);
  f.wo = k.take<uint8_t>(C * C);
  f.wfc = k.take<uint8_t>(F * C);
  f.wproj = k.take<uint8_t>(C * F);
  f.bytes = (k.off + 255) & ~size_t(255);
  return f;
}

// Split-K count of a weight gradient: the smallest split count whose
// workgroups fill at least 85% of their last wave over the 256 CUs (fewer
// splits, fewer fp32 partials to write and reduce), then the largest count
// with the same number of waves (each split's k-range, and so the wave,
// gets shorter), keeping >= 8 k-steps per split.
int wgrad_splits(int M, int N, long K, int BK) {
  const long tiles = (long)((M + 255) / 256) * ((N + 255) / 256);
  const long ksteps = (K + BK - 1) / BK;
  const long smax = std::max<long>(1, std::min<long>(32, ksteps / 8));
  auto waves = [&](long s) { return (tiles * s + 255) / 256; };
  for (long s = 1; s <= smax; ++s) {
    if (tiles * s * 100 >= 85 * waves(s) * 256) {
      while (s < smax && waves(s + 1) == waves(s)) ++s;
      return (int)s;
    }
  }
  return (int)smax;
}

// Stored-dS backward attention (bf16, causal, T <= 4096): the dK/dV kernel
// writes the bf16 dS of every visible (query, key) pair and dQ = dS K is a
// pass over it, instead of a pass that recomputes S and dP.  Per (sequence,
// query head): one [128 keys][64 queries] block per pair of a 128-key unit kt
// and a 64-query tile qt >= 2 kt, ds_pairs of them (about T^2 / 2 values).
// With a window, or past T = 4096 (where the store would outgrow the other
// activations many times), the dQ pass recomputes dS.
bool stored_ds(const blk_cfg& c) {
  const bool causal = c.window <= 0 || c.window >= c.T;
  return c.dtype == BLK_BF16 && causal && c.T <= 4096;
}
long ds_pairs(const blk_cfg& c) {
  const long nk = (c.T + 127) / 128, nq = (c.T + 63) / 64;
  return nk * nq - nk * (nk - 1);   // sum over kt < nk of (nq - 2 kt)
}

template <typename T> struct BwdScratch {
  T* du;        // [N, F]
  T* dh;        // [N, C] (dh2, later dh1)
  T* dy1;       // [N, C]
  T* dO;        // [N, C]
  T* dqkv;      // [N, 3C]
  T* wt;        // transposed weights: W_proj^T [F,C], W_fc^T [C,F], W_o^T [C,C], W_qkv^T [C,(H+2G)128]
  float* delta; // [B*H][T]
  bf16* ds = nullptr;   // stored dS ([B*H][ds_pairs][128][64]), or null
  float* part;  // split-k partial sums
  // fp8 mode: E4M3 copies of the gradients (row-major and transposed [*, Np])
  // and of the transposed weights
  uint8_t *g8 = nullptr, *g8t = nullptr, *du8 = nullptr, *du8t = nullptr, *dqkv8 = nullptr, *dqkv8t = nullptr,
          *wt8 = nullptr;
  size_t bytes;
};

template <typename T> BwdScratch<T> carve_bwd(const blk_cfg& c, void* p) {
  const long N = (long)c.B * c.T;
  Carver k(p);
  BwdScratch<T> s;
  s.du = k.take<T>(N * c.F);
  s.dh = k.take<T>(N * c.C);
  s.dy1 = k.take<T>(N * c.C);
  s.dO = k.take<T>(N * c.C);
  s.dqkv = k.take<T>(N * qkv_width(c));
  s.wt = k.take<T>(9L * c.C * c.C + (long)c.C * qkv_width(c));
  s.delta = k.take<float>((size_t)c.B * c.H * c.T);
  if (stored_ds(c)) s.ds = k.take<bf16>((size_t)c.B * c.H * ds_pairs(c) * 128 * 64);
  size_t part = 0;
  const int shapes[4][2] = {{c.C, c.F}, {c.F, c.C}, {c.C, c.C}, {(int)qkv_width(c), c.C}};
  for (int bk : {GemmTile<T>::BK, GemmTile<fp8e4>::BK})
    for (auto& sh : shapes) {
      int sp = wgrad_splits(sh[0], sh[1], N, bk);
      if (sp > 1) part = std::max(part, (size_t)sp * sh[0] * sh[1]);
    }
  s.part = k.take<float>(part);
  if (c.gemm == BLK_GEMM_FP8_E4M3) {
    const long Np = pad64(N);
    s.g8 = k.take<uint8_t>(N * c.C);
    s.g8t = k.take<uint8_t>(c.C * Np);
    s.du8 = k.take<uint8_t>(N * c.F);
    s.du8t = k.take<uint8_t>(c.F * Np);
    s.dqkv8 = k.take<uint8_t>(N * qkv_width(c));
    s.dqkv8t = k.take<uint8_t>(qkv_width(c) * Np);
    s.wt8 = k.take<uint8_t>(9L * c.C * c.C + (long)c.C * qkv_width(c));
  }
  s.bytes = (k.off + 255) & ~size_t(255);
  return s;
}

size_t elt_size(const blk_cfg& c) { return c.dtype == BLK_BF16 ? 2 : 4; }

// Weight gradients run on the four-wave GEMM body when the eight-wave one
// does not apply: always in float32, and when the token count is not a
// multiple of the eight-wave body's k-step (bf16 64 tokens, E4M3 128).  The
// four-wave body forms 32-bit byte offsets from each operand's base, so
// every operand it reads must stay below 4 GiB.
bool four_wave_wgrad(const blk_cfg& c) {
  const long N = (long)c.B * c.T;
  if (c.dtype != BLK_BF16) return true;
  if (c.gemm == BLK_GEMM_FP8_E4M3) return N % GemmTile<fp8e4>::BK != 0;
  return N % GemmTile<bf16>::BK != 0;
}

// Bytes of the largest weight-gradient operand: [N, F] tokens x MLP width
// (F = 4C is at least the fused projection's C + 256G); the fp8 mode reads
// transposed E4M3 copies [F, N rounded up to 64].
long wgrad_operand_bytes(const blk_cfg& c) {
  const long N = (long)c.B * c.T;
  const long wide = std::max<long>(c.F, qkv_width(c));
  if (c.gemm == BLK_GEMM_FP8_E4M3) return wide * pad64(N);
  return wide * N * (long)elt_size(c);
}

int check_cfg(const blk_cfg* c) {
  if (!c) return BLK_EINVAL;
  if (c->B < 1 || c->T < 1 || c->H < 1 || c->D != 128 || c->C != c->H * c->D || c->F != 4 * c->C) return BLK_EINVAL;
  if (!(c->eps >= 0.f) || !(c->rope_base > 0.f)) return BLK_EINVAL;
  if (c->dtype != BLK_F32 && c->dtype != BLK_BF16) return BLK_EINVAL;
  if (c->gemm != BLK_GEMM_NATIVE && c->gemm != BLK_GEMM_FP8_E4M3) return BLK_EINVAL;
  if (c->window < 0) return BLK_EINVAL;
  if (c->n_kv_head < 0 || (c->n_kv_head > 0 && c->H % c->n_kv_head != 0)) return BLK_EINVAL;
  if (c->gemm == BLK_GEMM_FP8_E4M3 && c->dtype != BLK_BF16) return BLK_EUNSUPPORTED;
  // row kernels keep a row in registers: 8 chunks of 16 bytes per lane
  if ((long)c->C * (c->dtype == BLK_BF16 ? 2 : 4) > 8L * 64 * 16) return BLK_EUNSUPPORTED;
  if ((long)c->B * c->T * qkv_width(*c) >= (1L << 31)) return BLK_EUNSUPPORTED;
  if (four_wave_wgrad(*c) && wgrad_operand_bytes(*c) >= (1L << 32)) return BLK_EUNSUPPORTED;
  return BLK_OK;
}

bool aligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int launch_status() { return hipGetLastError() == hipSuccess ? BLK_OK : BLK_ELAUNCH; }

// ---------------------------------------------------------------- MFMA rate probe
// Register-only MFMA loop: each wave runs `iters` rounds of four independent
// 32x32 MFMA chains (bf16 32x32x16, or E4M3 32x32x64 with unit scales) and
// writes one float per lane, so the loop is not removed.  Its rate is the
// matrix cores' achievable throughput at the clock the chip holds under this
// load, a yardstick for the kernels (not part of any computation).
template <int KIND>
__global__ __launch_bounds__(256) void mfma_probe_kernel(int iters, float* sink) {
  f32x16 c[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) c[j][r] = 0.f;
  const int t = threadIdx.x;
  if constexpr (KIND == 0) {
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = (bf16)(1e-3f * (float)((t + e) & 7));
      b[e] = (bf16)(1e-3f * (float)((t * 3 + e) & 7));
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = Mfma<bf16>::mma(a, b, c[j]);
  } else {
    i32x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] = 0x38383838 + ((t + e) & 3);
      b[e] = 0x30303030 + ((t * 3 + e) & 3);
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) c[j] = Mfma<fp8e4>::mma(a, b, c[j]);
  }
  float v = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) v += c[j][r];
  sink[(long)blockIdx.x * 256 + t] = v;
}

// ---------------------------------------------------------------- timing
// Optional per-launch timing: while enabled, every launch site records a
// pair of hipEvents around its kernel(s) on the call's stream.
struct TimingRec { const char* name; hipEvent_t a, b; };
std::mutex g_tmu;
bool g_timing = false;
std::vector<TimingRec> g_recs;
std::vector<hipEvent_t> g_pool;
size_t g_pool_used = 0;

hipEvent_t pool_event() {
  if (g_pool_used == g_pool.size()) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    g_pool.push_back(e);
  }
  return g_pool[g_pool_used++];
}

struct Timed {
  const char* name;
  hipStream_t st;
  hipEvent_t a = nullptr;
  Timed(const char* n, hipStream_t s) : name(n), st(s) {
    if (!g_timing) return;
    std::lock_guard<std::mutex> l(g_tmu);
    a = pool_event();
    if (a) hipEventRecord(a, st);
  }
  ~Timed() {
    if (!a) return;
    std::lock_guard<std::mutex> l(g_tmu);
    hipEvent_t b = pool_event();
    if (!b) return;
    hipEventRecord(b, st);
    g_recs.push_back({name, a, b});
  }
};

// ---------------------------------------------------------------- launchers
std::mutex g_attr_mu;
std::set<const void*> g_attr_done;

void need_lds(const void* kern, int bytes) {
  std::lock_guard<std::mutex> l(g_attr_mu);
  if (g_attr_done.insert(kern).second)
    hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

// threads: 256 for the four-wave GEMM body, 512 for the eight-wave one
template <typename TI>
void gemm(void (*kern)(GemmArgs), const char* name, GemmArgs g, int splits, hipStream_t st, int threads = 256) {
  constexpr int LDS = GemmTile<TI>::LDS;
  need_lds(reinterpret_cast<const void*>(kern), LDS);
  g.tiles_m = (g.M + 255) / 256;
  g.tiles_n = (g.N + 255) / 256;
  if (splits <= 1) {
    g.k_split = g.K;
    splits = 1;
  } else {
    constexpr int BK = GemmTile<TI>::BK;
    long per = ((long)g.K + splits - 1) / splits;
    g.k_split = (int)(((per + BK - 1) / BK) * BK);
    splits = (g.K + g.k_split - 1) / g.k_split;
  }
  g.nsplit = splits;
  Timed t(name, st);
  if (threads == 512 && (!g.aux || sizeof(TI) == 2)) {
    // the eight-wave kernels are persistent, one workgroup per CU walking the
    // tiles, except the E4M3 ones whose epilogue reads an operand of its own
    const int total = g.tiles_m * g.tiles_n * splits;
    hipLaunchKernelGGL(kern, dim3(std::min(total, cu_count())), dim3(threads), LDS, st, g);
  } else {
    hipLaunchKernelGGL(kern, dim3(g.tiles_m * g.tiles_n, splits), dim3(threads), LDS, st, g);
  }
}

// Forward and input-gradient GEMMs (eight-wave kernels, no split): K and both
// leading dimensions are multiples of 128 elements here (C = 128 H, F = 4 C),
// as the kernels' k-step of 128 bytes requires.
template <typename TI>
void gemm_pp(void (*kern)(GemmArgs), const char* name, GemmArgs g, hipStream_t st) {
  gemm<TI>(kern, name, g, 1, st, 512);
}

GemmArgs gargs(const void* A, long lda, const void* B, long ldb, int M, int N, int K) {
  GemmArgs g{};
  g.A = A; g.lda = lda; g.B = B; g.ldb = ldb;
  g.M = M; g.N = N; g.K = K;
  g.alpha = 1.f;
  return g;
}

// Epilogue parameters of the QKV projection (rotary + QK-norm) and of the
// attention-output input gradient (per-head row dot with o).
void rope_args(GemmArgs& g, const blk_cfg& c, const float2* cs, float* rho) {
  g.cs = cs; g.rho = rho; g.T = c.T; g.H = c.H; g.C = c.C; g.G = kv_heads(c); g.eps = c.eps;
}
void delta_args(GemmArgs& g, const blk_cfg& c, const void* o, float* delta) {
  g.aux = o; g.ldaux = c.C; g.delta = delta; g.T = c.T; g.H = c.H; g.C = c.C;
}

// Weight gradient dW[M, N] (+)= sum_t G[t, m] X[t, n]  (G: [K, M], X: [K, N]).
// bf16 operands with K a multiple of the k-step run on the eight-wave body
// (kernels kp / kp_acc), others on the four-wave one.
typedef void (*GemmKernel)(GemmArgs);
template <typename T>
void wgrad(GemmKernel kern, GemmKernel kern_acc, GemmKernel kp, GemmKernel kp_acc, const char* name, const T* G,
           const T* X, float* dW, int M, int N, int K, int accumulate, float* part, hipStream_t st) {
  GemmArgs g = gargs(G, M, X, N, M, N, K);
  const bool pp = std::is_same<T, bf16>::value && K % GemmTile<T>::BK == 0;
  const int threads = pp ? 512 : 256;
  if (pp) { kern = kp; kern_acc = kp_acc; }
  int sp = wgrad_splits(M, N, K, GemmTile<T>::BK);
  if (sp <= 1) {
    g.out = dW; g.ldo = N;
    gemm<T>(accumulate ? kern_acc : kern, name, g, 1, st, threads);
    return;
  }
  g.out = part; g.ldo = N;
  gemm<T>(kern, name, g, sp, st, threads);
  // the launcher may round the split count down; recompute it identically
  constexpr int BK = GemmTile<T>::BK;
  long per = ((long)K + sp - 1) / sp;
  int ks = (int)(((per + BK - 1) / BK) * BK);
  int real = (K + ks - 1) / ks;
  const long n = (long)M * N;
  Timed t("splitk_reduce", st);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st, dW,
                     (const float*)part, n, real, accumulate);
}

unsigned row_blocks(long rows) { return (unsigned)((rows + 3) / 4); }
// row kernels that publish an absolute maximum: a capped grid walking the rows
unsigned amax_row_blocks(long rows) { return std::min(row_blocks(rows), AMAX_BLOCKS); }

// ---------------------------------------------------------------- forward
template <typename T> AttnArgs attn_args(const blk_cfg& c) {
  AttnArgs a{};
  a.B = c.B; a.T = c.T; a.H = c.H; a.C = c.C;
  a.W = (c.window <= 0 || c.window >= c.T) ? c.T : c.window;   // W >= T: causal
  a.G = kv_heads(c);
  a.LD = (int)qkv_width(c);
  a.KO = c.C;
  a.VO = c.C + a.G * 128;
  a.sl2 = (float)(1.4426950408889634 / std::sqrt(128.0));   // log2(e) / sqrt(D)
  a.rsd = (float)(1.0 / std::sqrt(128.0));
  return a;
}

template <typename T>
int fwd_impl(const blk_cfg& c, const T* x, const T* wqkv, const T* wo, const T* wfc, const T* wproj, T* y,
             const Saved<T>& s, hipStream_t st) {
  const int N = c.B * c.T, C = c.C, F = c.F, H = c.H;
  {  // rotary angle table
    Timed t("rope_table", st);
    hipLaunchKernelGGL(rope_table_kernel, dim3((c.T * 64 + 255) / 256), dim3(256), 0, st, s.cs, c.T, 128,
                       (double)c.rope_base);
  }
  {  // 1 h1 = rmsnorm(x)
    Timed t("rmsnorm_fwd", st);
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<T>, dim3(row_blocks(N)), dim3(256), 0, st, x, s.h1, s.r1, N, C, c.eps);
  }
  {  // 2-4 qkv = h1 W_qkv^T; rotary and QK-norm of q, k in the epilogue
    GemmArgs g = gargs(s.h1, C, wqkv, C, N, (int)qkv_width(c), C);
    g.out = s.qkv; g.ldo = qkv_width(c);
    rope_args(g, c, s.cs, s.rho);
    gemm_pp<T>(gemm_qkv_fwd<T>, "gemm_qkv_fwd", g, st);
  }
  {  // 5 causal attention
    AttnArgs a = attn_args<T>(c);
    a.qkv = s.qkv; a.o = s.o; a.lse = s.lse;
    Timed t("attn_fwd", st);
    attn_fwd(a, sizeof(T) == 2, st);
  }
  {  // 6 y1 = x + o W_o^T   (y1 is kept in y)
    GemmArgs g = gargs(s.o, C, wo, C, N, C, C);
    g.out = y; g.ldo = C; g.aux = x; g.ldaux = C;
    gemm_pp<T>(gemm_o_fwd<T>, "gemm_o_fwd", g, st);
  }
  {  // 7 h2 = rmsnorm(y1)
    Timed t("rmsnorm_fwd", st);
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<T>, dim3(row_blocks(N)), dim3(256), 0, st, (const T*)y, s.h2, s.r2, N,
                       C, c.eps);
  }
  {  // 8 a = relu(h2 W_fc^T)^2 (u itself is not kept: the backward uses 2 sqrt(a))
    GemmArgs g = gargs(s.h2, C, wfc, C, N, F, C);
    g.out = s.a; g.ldo = F;
    gemm_pp<T>(gemm_fc_fwd<T>, "gemm_fc_fwd", g, st);
  }
  {  // 9 y = y1 + a W_proj^T   (in place on y)
    GemmArgs g = gargs(s.a, F, wproj, F, N, C, F);
    g.out = y; g.ldo = C; g.aux = y; g.ldaux = C;
    gemm_pp<T>(gemm_proj_fwd<T>, "gemm_proj_fwd", g, st);
  }
  return launch_status();
}

// ---------------------------------------------------------------- backward
template <typename T>
int bwd_impl(const blk_cfg& c, const T* dy, const T* x, const T* wqkv, const T* wo, const T* wfc, const T* wproj,
             const Saved<T>& s, T* dx, float* dwqkv, float* dwo, float* dwfc, float* dwproj, int acc,
             const BwdScratch<T>& w, hipStream_t st) {
  (void)x;
  const int N = c.B * c.T, C = c.C, F = c.F, H = c.H;
  // input-gradient GEMMs read the weights k-contiguous: W^T, made once per call
  T* wt_proj = w.wt;                       // [F, C]
  T* wt_fc = wt_proj + (long)F * C;        // [C, F]
  T* wt_o = wt_fc + (long)C * F;           // [C, C]
  T* wt_qkv = wt_o + (long)C * C;          // [C, (H+2G)128]
  {
    Timed t("transpose_weights", st);
    auto tr = [&](const T* src, T* dst, int rows, int cols) {
      hipLaunchKernelGGL(transpose_kernel<T>, dim3(cols / 64, rows / 64), dim3(256), 0, st, src, dst, rows, cols);
    };
    tr(wproj, wt_proj, C, F);
    tr(wfc, wt_fc, F, C);
    tr(wo, wt_o, C, C);
    tr(wqkv, wt_qkv, (int)qkv_width(c), C);
  }
  {  // 9: du = (dy W_proj) * 2 max(u, 0), with max(u, 0) = sqrt(a)
    GemmArgs g = gargs(dy, C, wt_proj, C, N, F, C);
    g.out = w.du; g.ldo = F; g.aux = s.a; g.ldaux = F;
    gemm_pp<T>(gemm_proj_dgrad<T>, "gemm_proj_dgrad", g, st);
  }
  //    dW_proj = dy^T a
  wgrad<T>(gemm_proj_wgrad<T>, gemm_proj_wgrad_acc<T>, gemm_proj_wgrad_pp, gemm_proj_wgrad_acc_pp, "gemm_proj_wgrad", dy, s.a, dwproj, C, F, N, acc, w.part,
           st);
  {  // 8: dh2 = du W_fc
    GemmArgs g = gargs(w.du, F, wt_fc, F, N, C, F);
    g.out = w.dh; g.ldo = C;
    gemm_pp<T>(gemm_fc_dgrad<T>, "gemm_fc_dgrad", g, st);
  }
  //    dW_fc = du^T h2
  wgrad<T>(gemm_fc_wgrad<T>, gemm_fc_wgrad_acc<T>, gemm_fc_wgrad_pp, gemm_fc_wgrad_acc_pp, "gemm_fc_wgrad", w.du, s.h2, dwfc, F, C, N, acc, w.part, st);
  {  // 7: dy1 = dy + rmsnorm backward
    Timed t("rmsnorm_bwd", st);
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<T>, dim3(row_blocks(N)), dim3(256), 0, st, dy, (const T*)w.dh,
                       (const T*)s.h2, (const float*)s.r2, w.dy1, N, C);
  }
  {  // 6: do = dy1 W_o; delta = rowsum(do * o) per head in the epilogue
    GemmArgs g = gargs(w.dy1, C, wt_o, C, N, C, C);
    g.out = w.dO; g.ldo = C;
    delta_args(g, c, s.o, w.delta);
    gemm_pp<T>(gemm_o_dgrad<T>, "gemm_o_dgrad", g, st);
  }
  //    dW_o = dy1^T o
  wgrad<T>(gemm_o_wgrad<T>, gemm_o_wgrad_acc<T>, gemm_o_wgrad_pp, gemm_o_wgrad_acc_pp, "gemm_o_wgrad", w.dy1, s.o, dwo, C, C, N, acc, w.part, st);
  {  // 5: attention backward
    AttnArgs a = attn_args<T>(c);
    a.qkv = s.qkv; a.lse = s.lse; a.dO = w.dO; a.delta = w.delta; a.dqkv = w.dqkv;
    a.rho = s.rho; a.cs = s.cs;
    a.ds = w.ds; a.dsP = (int)ds_pairs(c);
    // 5-3: the bf16 kernels also apply the QK-norm and rotary backward to dq, dk
    {
      Timed t("attn_bwd_dkdv", st);
      attn_bwd_dkdv(a, sizeof(T) == 2, st);
    }
    {
      Timed t("attn_bwd_dq", st);
      attn_bwd_dq(a, sizeof(T) == 2, st);
    }
    if constexpr (sizeof(T) != 2) {
      {  // 4-3: QK-norm and rotary backward (in place on dq, dk)
        Timed t("qknorm_rope_bwd", st);
        hipLaunchKernelGGL(qknorm_rope_bwd_kernel<T>, dim3(row_blocks((long)N * (H + a.G))), dim3(256), 0, st,
                           w.dqkv, (const T*)s.qkv, (const float*)s.rho, (const float2*)s.cs, N, c.T, H, C, a.G);
      }
    }
  }
  {  // 2: dh1 = dqkv W_qkv
    const int W3 = (int)qkv_width(c);
    GemmArgs g = gargs(w.dqkv, W3, wt_qkv, W3, N, C, W3);
    g.out = w.dh; g.ldo = C;
    gemm_pp<T>(gemm_qkv_dgrad<T>, "gemm_qkv_dgrad", g, st);
  }
  //    dW_qkv = dqkv^T h1
  wgrad<T>(gemm_qkv_wgrad<T>, gemm_qkv_wgrad_acc<T>, gemm_qkv_wgrad_pp, gemm_qkv_wgrad_acc_pp, "gemm_qkv_wgrad", w.dqkv, s.h1, dwqkv, (int)qkv_width(c), C, N, acc,
           w.part, st);
  {  // 1: dx = dy1 + rmsnorm backward
    Timed t("rmsnorm_bwd", st);
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<T>, dim3(row_blocks(N)), dim3(256), 0, st, (const T*)w.dy1,
                       (const T*)w.dh, (const T*)s.h1, (const float*)s.r1, dx, N, C);
  }
  return launch_status();
}

// ---------------------------------------------------------------- fp8 mode
unsigned elt_grid(long n) { return (unsigned)std::min<long>(std::max<long>((n / 8 + 255) / 256, 1), 4096); }

// amax of x (rows x cols bf16) max-accumulated into *am; then, if given, the
// row-major codes q and the transposed codes qt ([cols][ldt], zero padded).
void quantize(const bf16* x, long rows, long cols, unsigned* am, uint8_t* q, uint8_t* qt, long ldt, bool amax,
              hipStream_t st) {
  const long n = rows * cols;
  Timed t("fp8_quantize", st);
  if (amax) hipLaunchKernelGGL(amax_kernel, dim3(std::min(elt_grid(n), AMAX_GRID)), dim3(256), 0, st, x, n, am);
  if (qt && cols % 128 == 0)   // transposed codes, and the row-major ones in the same pass
    hipLaunchKernelGGL(quant_trans128_kernel, dim3((unsigned)(cols / 128), (unsigned)((ldt + 127) / 128)), dim3(256),
                       0, st, x, (int)rows, (int)cols, (const unsigned*)am, qt, (int)ldt, q);
  else if (qt)
    hipLaunchKernelGGL(quant_trans_kernel, dim3((unsigned)(cols / 64), (unsigned)(ldt / 64)), dim3(256), 0, st, x,
                       (int)rows, (int)cols, (const unsigned*)am, qt, (int)ldt, q);
  else if (q)
    hipLaunchKernelGGL(quant_kernel, dim3(elt_grid(n)), dim3(256), 0, st, x, n, (const unsigned*)am, q);
}

GemmArgs gargs8(const uint8_t* A, long lda, const unsigned* ama, const uint8_t* B, long ldb, const unsigned* amb,
                int M, int N, int K) {
  GemmArgs g = gargs(A, lda, B, ldb, M, N, K);
  g.amax_a = ama;
  g.amax_b = amb;
  return g;
}

// dW[M, N] (+)= sum_k GT[m, k] XT[n, k], E4M3 operands [*, ld], fp32 out.
// Token counts that are a multiple of the k-step (128) run on the eight-wave
// body (kernels kp / kp_acc).
void wgrad8(GemmKernel kern, GemmKernel kern_acc, GemmKernel kp, GemmKernel kp_acc, const char* name,
            const uint8_t* GT, const unsigned* ama, const uint8_t* XT, const unsigned* amb, long ld, float* dW, int M,
            int N, int K, int accumulate, float* part, hipStream_t st) {
  GemmArgs g = gargs8(GT, ld, ama, XT, ld, amb, M, N, K);
  constexpr int BK = GemmTile<fp8e4>::BK;
  const bool pp = K % BK == 0 && ld % BK == 0;
  const int threads = pp ? 512 : 256;
  if (pp) { kern = kp; kern_acc = kp_acc; }
  const int sp = wgrad_splits(M, N, K, BK);
  if (sp <= 1) {
    g.out = dW; g.ldo = N;
    gemm<fp8e4>(accumulate ? kern_acc : kern, name, g, 1, st, threads);
    return;
  }
  g.out = part; g.ldo = N;
  gemm<fp8e4>(kern, name, g, sp, st, threads);
  long per = ((long)K + sp - 1) / sp;
  int ks = (int)(((per + BK - 1) / BK) * BK);
  int real = (K + ks - 1) / ks;
  const long n = (long)M * N;
  Timed t("splitk_reduce", st);
  hipLaunchKernelGGL(splitk_reduce_kernel, dim3((unsigned)((n / 4 + 255) / 256)), dim3(256), 0, st, dW,
                     (const float*)part, n, real, accumulate);
}

// amax slots: forward h1 o h2 a | W_qkv W_o W_fc W_proj ; backward dy du dy1 dqkv
enum { AM_H1, AM_O, AM_H2, AM_A, AM_WQKV, AM_WO, AM_WFC, AM_WPROJ, AM_DY, AM_DU, AM_DY1, AM_DQKV };

int fwd_fp8(const blk_cfg& c, const bf16* x, const bf16* wqkv, const bf16* wo, const bf16* wfc, const bf16* wproj,
            bf16* y, const Saved<bf16>& s, const Fwd8& f, hipStream_t st) {
  const int N = c.B * c.T, C = c.C, F = c.F, H = c.H;
  const long Np = pad64(N);
  unsigned* am = s.amax;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, st, am, 16);
  {
    Timed t("rope_table", st);
    hipLaunchKernelGGL(rope_table_kernel, dim3((c.T * 64 + 255) / 256), dim3(256), 0, st, s.cs, c.T, 128,
                       (double)c.rope_base);
  }
  {
    Timed t("rmsnorm_fwd", st);
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<bf16>, dim3(amax_row_blocks(N)), dim3(256), 0, st, x, s.h1, s.r1, N, C,
                       c.eps, am + AM_H1);
  }
  quantize(wqkv, qkv_width(c), C, am + AM_WQKV, f.wqkv, nullptr, 0, true, st);
  quantize(wo, C, C, am + AM_WO, f.wo, nullptr, 0, true, st);
  quantize(wfc, F, C, am + AM_WFC, f.wfc, nullptr, 0, true, st);
  quantize(wproj, C, F, am + AM_WPROJ, f.wproj, nullptr, 0, true, st);
  quantize(s.h1, N, C, am + AM_H1, f.h1, s.h1_8t, Np, false, st);   // amax from rmsnorm_fwd
  {
    GemmArgs g = gargs8(f.h1, C, am + AM_H1, f.wqkv, C, am + AM_WQKV, N, (int)qkv_width(c), C);
    g.out = s.qkv; g.ldo = qkv_width(c);
    rope_args(g, c, s.cs, s.rho);
    gemm_pp<fp8e4>(gemm8_qkv_fwd, "gemm_qkv_fwd", g, st);
  }
  {
    AttnArgs a = attn_args<bf16>(c);
    a.qkv = s.qkv; a.o = s.o; a.lse = s.lse; a.amax_o = am + AM_O;
    Timed t("attn_fwd", st);
    attn_fwd(a, true, st);
  }
  quantize(s.o, N, C, am + AM_O, f.o, s.o_8t, Np, false, st);       // amax from attn_fwd
  {
    GemmArgs g = gargs8(f.o, C, am + AM_O, f.wo, C, am + AM_WO, N, C, C);
    g.out = y; g.ldo = C; g.aux = x; g.ldaux = C;
    gemm_pp<fp8e4>(gemm8_o_fwd, "gemm_o_fwd", g, st);
  }
  {
    Timed t("rmsnorm_fwd", st);
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<bf16>, dim3(amax_row_blocks(N)), dim3(256), 0, st, (const bf16*)y, s.h2,
                       s.r2, N, C, c.eps, am + AM_H2);
  }
  quantize(s.h2, N, C, am + AM_H2, f.h2, s.h2_8t, Np, false, st);   // amax from rmsnorm_fwd
  {
    GemmArgs g = gargs8(f.h2, C, am + AM_H2, f.wfc, C, am + AM_WFC, N, F, C);
    g.out = s.a; g.ldo = F; g.amax_out = am + AM_A;
    gemm_pp<fp8e4>(gemm8_fc_fwd, "gemm_fc_fwd", g, st);
  }
  quantize(s.a, N, F, am + AM_A, f.a, s.a_8t, Np, false, st);       // amax from gemm_fc_fwd
  {
    GemmArgs g = gargs8(f.a, F, am + AM_A, f.wproj, F, am + AM_WPROJ, N, C, F);
    g.out = y; g.ldo = C; g.aux = y; g.ldaux = C;
    gemm_pp<fp8e4>(gemm8_proj_fwd, "gemm_proj_fwd", g, st);
  }
  return launch_status();
}

int bwd_fp8(const blk_cfg& c, const bf16* dy, const bf16* wqkv, const bf16* wo, const bf16* wfc, const bf16* wproj,
            const Saved<bf16>& s, bf16* dx, float* dwqkv, float* dwo, float* dwfc, float* dwproj, int acc,
            const BwdScratch<bf16>& w, hipStream_t st) {
  const int N = c.B * c.T, C = c.C, F = c.F, H = c.H;
  const long Np = pad64(N);
  unsigned* am = s.amax;     // forward slots hold the weights' and activations' maxima
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, st, am + AM_DY, 4);
  // transposed E4M3 weights (same scales as the forward's row-major copies)
  uint8_t* wt_proj = w.wt8;                 // [F, C]
  uint8_t* wt_fc = wt_proj + (long)F * C;   // [C, F]
  uint8_t* wt_o = wt_fc + (long)C * F;      // [C, C]
  uint8_t* wt_qkv = wt_o + (long)C * C;     // [C, (H+2G)128]
  quantize(wproj, C, F, am + AM_WPROJ, nullptr, wt_proj, C, false, st);
  quantize(wfc, F, C, am + AM_WFC, nullptr, wt_fc, F, false, st);
  quantize(wo, C, C, am + AM_WO, nullptr, wt_o, C, false, st);
  quantize(wqkv, qkv_width(c), C, am + AM_WQKV, nullptr, wt_qkv, qkv_width(c), false, st);

  quantize(dy, N, C, am + AM_DY, w.g8, w.g8t, Np, true, st);
  {  // du = (dy W_proj) * 2 max(u, 0), with max(u, 0) = sqrt(a)
    GemmArgs g = gargs8(w.g8, C, am + AM_DY, wt_proj, C, am + AM_WPROJ, N, F, C);
    g.out = w.du; g.ldo = F; g.aux = s.a; g.ldaux = F; g.amax_out = am + AM_DU;
    gemm_pp<fp8e4>(gemm8_proj_dgrad, "gemm_proj_dgrad", g, st);
  }
  wgrad8(gemm8_proj_wgrad, gemm8_proj_wgrad_acc, gemm8_proj_wgrad_pp, gemm8_proj_wgrad_acc_pp, "gemm_proj_wgrad", w.g8t, am + AM_DY, s.a_8t, am + AM_A, Np, dwproj,
         C, F, N, acc, w.part, st);
  quantize(w.du, N, F, am + AM_DU, w.du8, w.du8t, Np, false, st);   // amax from gemm_proj_dgrad
  {  // dh2 = du W_fc
    GemmArgs g = gargs8(w.du8, F, am + AM_DU, wt_fc, F, am + AM_WFC, N, C, F);
    g.out = w.dh; g.ldo = C;
    gemm_pp<fp8e4>(gemm8_fc_dgrad, "gemm_fc_dgrad", g, st);
  }
  wgrad8(gemm8_fc_wgrad, gemm8_fc_wgrad_acc, gemm8_fc_wgrad_pp, gemm8_fc_wgrad_acc_pp, "gemm_fc_wgrad", w.du8t, am + AM_DU, s.h2_8t, am + AM_H2, Np, dwfc, F, C,
         N, acc, w.part, st);
  {
    Timed t("rmsnorm_bwd", st);
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<bf16>, dim3(amax_row_blocks(N)), dim3(256), 0, st, dy, (const bf16*)w.dh,
                       (const bf16*)s.h2, (const float*)s.r2, w.dy1, N, C, am + AM_DY1);
  }
  quantize(w.dy1, N, C, am + AM_DY1, w.g8, w.g8t, Np, false, st);   // amax from rmsnorm_bwd
  {  // do = dy1 W_o
    GemmArgs g = gargs8(w.g8, C, am + AM_DY1, wt_o, C, am + AM_WO, N, C, C);
    g.out = w.dO; g.ldo = C;
    delta_args(g, c, s.o, w.delta);
    gemm_pp<fp8e4>(gemm8_o_dgrad, "gemm_o_dgrad", g, st);
  }
  wgrad8(gemm8_o_wgrad, gemm8_o_wgrad_acc, gemm8_o_wgrad_pp, gemm8_o_wgrad_acc_pp, "gemm_o_wgrad", w.g8t, am + AM_DY1, s.o_8t, am + AM_O, Np, dwo, C, C, N,
         acc, w.part, st);
  {
    AttnArgs a = attn_args<bf16>(c);
    a.qkv = s.qkv; a.lse = s.lse; a.dO = w.dO; a.delta = w.delta; a.dqkv = w.dqkv;
    a.rho = s.rho; a.cs = s.cs;   // QK-norm and rotary backward in the stores
    a.amax_dqkv = am + AM_DQKV;
    a.ds = w.ds; a.dsP = (int)ds_pairs(c);
    {
      Timed t("attn_bwd_dkdv", st);
      attn_bwd_dkdv(a, true, st);
    }
    {
      Timed t("attn_bwd_dq", st);
      attn_bwd_dq(a, true, st);
    }
  }
  quantize(w.dqkv, N, qkv_width(c), am + AM_DQKV, w.dqkv8, w.dqkv8t, Np, false, st);   // amax from attention bwd
  {  // dh1 = dqkv W_qkv
    const int W3 = (int)qkv_width(c);
    GemmArgs g = gargs8(w.dqkv8, W3, am + AM_DQKV, wt_qkv, W3, am + AM_WQKV, N, C, W3);
    g.out = w.dh; g.ldo = C;
    gemm_pp<fp8e4>(gemm8_qkv_dgrad, "gemm_qkv_dgrad", g, st);
  }
  wgrad8(gemm8_qkv_wgrad, gemm8_qkv_wgrad_acc, gemm8_qkv_wgrad_pp, gemm8_qkv_wgrad_acc_pp, "gemm_qkv_wgrad", w.dqkv8t, am + AM_DQKV, s.h1_8t, am + AM_H1, Np,
         dwqkv, (int)qkv_width(c), C, N, acc, w.part, st);
  {
    Timed t("rmsnorm_bwd", st);
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<bf16>, dim3(row_blocks(N)), dim3(256), 0, st, (const bf16*)w.dy1,
                       (const bf16*)w.dh, (const bf16*)s.h1, (const float*)s.r1, dx, N, C);
  }
  return launch_status();
}

// ---------------------------------------------------------------- decode
int check_dcfg(const blk_dcfg* c) {
  if (!c) return BLK_EINVAL;
  if (c->B < 1 || c->H < 1 || c->D != 128 || c->C != c->H * c->D || c->F != 4 * c->C || c->S_max < 1)
    return BLK_EINVAL;
  if (!(c->eps >= 0.f) || !(c->rope_base > 0.f)) return BLK_EINVAL;
  if (c->dtype != BLK_F32 && c->dtype != BLK_BF16) return BLK_EINVAL;
  if (c->window < 0) return BLK_EINVAL;
  if (c->dtype != BLK_BF16) return BLK_EUNSUPPORTED;   // the decode kernels are bf16 only
  if (c->C > 2048 || c->B > 65535) return BLK_EUNSUPPORTED;
  if ((long)c->B * c->H * c->S_max * 128 >= (1L << 40)) return BLK_EUNSUPPORTED;
  if (c->n_kv_head < 0 || (c->n_kv_head > 0 && c->H % c->n_kv_head != 0)) return BLK_EINVAL;
  return BLK_OK;
}

struct DecSplit { int S, cps; };

// K-splits of a skinny GEMM: one 64-wide K-step per wave (4 per workgroup),
// so each wave issues all its loads at once; the splits' fp32 partials are
// summed by the row-wise epilogue kernels.
DecSplit dec_split(int M, int N, int K) {
  (void)M; (void)N;
  const int ks = K / dec::KCH;
  const int cps = std::min(4, ks);
  return {(ks + cps - 1) / cps, cps};
}

struct DecScratch {
  float* part;    // [S][B][N], the largest of the four GEMMs
  float* q;       // [B, H, 128]
  float* opart;   // [B, H, NS, 128]
  float2* ml;     // [B, H, NS]
  bf16* o;        // [B, C]
  float* y1;      // [B, C]
  bf16* h2;       // [B, C]
  bf16* a;        // [B, F]
  size_t bytes;
};

DecScratch carve_dec(const blk_dcfg& c, void* p) {
  const long B = c.B, C = c.C, F = c.F, H = c.H;
  const long NS = (c.S_max + dec::KEYS - 1) / dec::KEYS;
  long part = 0;
  const long nk[3][2] = {{qkv_width(c), C}, {C, C}, {C, F}};   // (N, K) of the split GEMMs (FC is unsplit)
  for (const auto& g : nk) part = std::max(part, (long)dec_split((int)B, (int)g[0], (int)g[1]).S * B * g[0]);
  Carver k(p);
  DecScratch d;
  d.part = k.take<float>(part);
  d.q = k.take<float>(B * H * 128);
  d.opart = k.take<float>(B * H * NS * 128);
  d.ml = k.take<float2>(B * H * NS);
  d.o = k.take<bf16>(B * C);
  d.y1 = k.take<float>(B * C);
  d.h2 = k.take<bf16>(B * C);
  d.a = k.take<bf16>(B * F);
  d.bytes = (k.off + 255) & ~size_t(255);
  return d;
}

void dec_gemm(const char* name, const bf16* A, int M, const bf16* W, int N, int K, DecSplit sp, float* part,
              hipStream_t st) {
  Timed t(name, st);
  hipLaunchKernelGGL(dec::skinny_gemm_kernel, dim3(N / dec::NBLK, sp.S, (M + dec::MBLK - 1) / dec::MBLK), dim3(256),
                     0, st, A, M, W, N, K, sp.cps, part);
}

// Arguments of a decode step other than its workspace.
int check_decode_args(const blk_dcfg* cfg, const void* x, const void* w_qkv, const void* w_o, const void* w_fc,
                      const void* w_proj, const void* k_cache, const void* v_cache, const int32_t* cache_len,
                      const int32_t* status, const void* y) {
  if (int e = check_dcfg(cfg)) return e;
  for (const void* p : {x, w_qkv, w_o, w_fc, w_proj, k_cache, v_cache, y})
    if (!p) return BLK_EINVAL;
  if (!cache_len || k_cache == v_cache) return BLK_EINVAL;
  for (const void* p : {x, w_qkv, w_o, w_fc, w_proj, k_cache, v_cache, y})
    if (!aligned(p)) return BLK_EALIGN;
  if ((reinterpret_cast<uintptr_t>(cache_len) | reinterpret_cast<uintptr_t>(status)) & 3) return BLK_EALIGN;
  return BLK_OK;
}

// The launch sequence of one decode step, its temporaries carved from
// `scratch` (decode_scratch_bytes(cfg) bytes of device memory).
int decode_run(const blk_dcfg& c, const void* x, const void* w_qkv, const void* w_o, const void* w_fc,
               const void* w_proj, void* k_cache, void* v_cache, const int32_t* cache_len, int32_t* status, void* y,
               void* scratch, hipStream_t st) {
  const DecScratch d = carve_dec(c, scratch);
  hipGetLastError();
  const int B = c.B, C = c.C, H = c.H, F = c.F;
  const bf16* xb = static_cast<const bf16*>(x);
  bf16* kc = static_cast<bf16*>(k_cache);
  bf16* vc = static_cast<bf16*>(v_cache);
  const int NS = (c.S_max + dec::KEYS - 1) / dec::KEYS;
  // x W_qkv^T (the row scale r1 of rmsnorm(x) is applied in the epilogue kernel)
  const DecSplit sq = dec_split(B, (int)qkv_width(c), C);
  dec_gemm("dec_gemm_qkv", xb, B, static_cast<const bf16*>(w_qkv), (int)qkv_width(c), C, sq, d.part, st);
  {  // r1; rotary + QK-norm at position cache_len[b]; k, v into the caches
    Timed t("dec_qkv_epi", st);
    hipLaunchKernelGGL(dec::dec_qkv_epi_kernel, dim3(H, B), dim3(192), 0, st, (const float*)d.part, sq.S, B, H,
                       kv_heads(c), xb, cache_len, c.S_max, c.eps, (double)c.rope_base, d.q, kc, vc);
  }
  const int dwin = c.window > 0 ? c.window : INT_MAX;
  {  // attention of the new token over slots 0..cache_len[b] (the last W with a window)
    Timed t("dec_attn", st);
    const int G = kv_heads(c);
    hipLaunchKernelGGL(G == H ? dec::dec_attn_kernel<false> : dec::dec_attn_kernel<true>, dim3(NS, G, B), dim3(256),
                       dec::dec_attn_lds(H / G), st, (const float*)d.q, (const bf16*)kc, (const bf16*)vc, cache_len,
                       H, G, c.S_max, NS, dwin, (float)(1.4426950408889634 / std::sqrt(128.0)), d.opart, d.ml);
  }
  {
    Timed t("dec_combine", st);
    hipLaunchKernelGGL(dec::dec_combine_kernel, dim3(H, B), dim3(128), 0, st, (const float*)d.opart,
                       (const float2*)d.ml, cache_len, H, c.S_max, NS, dwin, d.o);
  }
  const DecSplit so = dec_split(B, C, C);
  dec_gemm("dec_gemm_o", d.o, B, static_cast<const bf16*>(w_o), C, C, so, d.part, st);
  {  // y1 = x + o W_o^T; h2 = rmsnorm(y1)
    Timed t("dec_resid_norm", st);
    hipLaunchKernelGGL(dec::dec_resid_norm_kernel, dim3(B), dim3(256), 0, st, (const float*)d.part, so.S, B, C, xb,
                       c.eps, d.y1, d.h2);
  }
  {  // a = relu(h2 W_fc^T)^2 (unsplit: K = C)
    Timed t("dec_gemm_fc", st);
    hipLaunchKernelGGL(dec::skinny_gemm_relu2_kernel, dim3(F / dec::NBLK, (B + dec::MBLK - 1) / dec::MBLK), dim3(256),
                       0, st, (const bf16*)d.h2, B, static_cast<const bf16*>(w_fc), F, C, d.a);
  }
  const DecSplit sp = dec_split(B, C, F);
  dec_gemm("dec_gemm_proj", d.a, B, static_cast<const bf16*>(w_proj), C, F, sp, d.part, st);
  {
    Timed t("dec_out", st);
    const long n = (long)B * C;
    hipLaunchKernelGGL(dec::dec_out_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       (const float*)d.part, sp.S, n, (const float*)d.y1, static_cast<bf16*>(y), cache_len, c.S_max, C,
                       (int*)status);
  }
  return launch_status();
}

// ---------------------------------------------------------------- workspace without allocation
constexpr int MAX_DEVICES = 64;
std::mutex g_noalloc_mu;
void* g_noalloc_ptr[MAX_DEVICES] = {};

int noalloc_workspace(void** ws) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return BLK_ELAUNCH;
  std::lock_guard<std::mutex> l(g_noalloc_mu);
  if (!g_noalloc_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(noalloc_scratch)) != hipSuccess || !p) return BLK_ELAUNCH;
    g_noalloc_ptr[dev] = p;
  }
  *ws = g_noalloc_ptr[dev];
  return BLK_OK;
}

size_t saved_bytes(const blk_cfg& c) {
  return c.dtype == BLK_BF16 ? carve_saved<bf16>(c, nullptr).bytes : carve_saved<float>(c, nullptr).bytes;
}
size_t bwd_bytes(const blk_cfg& c) {
  return c.dtype == BLK_BF16 ? carve_bwd<bf16>(c, nullptr).bytes : carve_bwd<float>(c, nullptr).bytes;
}
// forward temporaries: the saved store itself when saved == NULL, then the
// fp8 operand copies in fp8 mode
size_t fwd_scratch_bytes(const blk_cfg& c, bool with_saved) {
  size_t b = with_saved ? saved_bytes(c) : 0;
  if (c.gemm == BLK_GEMM_FP8_E4M3) b += carve_fwd8(c, nullptr).bytes;
  return b;
}

// ---------------------------------------------------------------- language-model head
int check_hcfg(const blk_hcfg* c) {
  if (!c) return BLK_EINVAL;
  if (c->N < 1 || c->C < 128 || c->C % 128 != 0 || c->V < 64 || c->V % 64 != 0) return BLK_EINVAL;
  if (!(c->eps >= 0.f)) return BLK_EINVAL;
  if (c->dtype != BLK_F32 && c->dtype != BLK_BF16) return BLK_EINVAL;
  if (c->dtype != BLK_BF16) return BLK_EUNSUPPORTED;                 // the head kernels are bf16 only
  if ((long)c->C * 2 > 8L * 64 * 16) return BLK_EUNSUPPORTED;        // row kernels keep a row in registers
  // weight gradient with K = N tokens: the eight-wave body (N a multiple of
  // 64) handles any size; the four-wave fallback needs 32-bit offsets
  if (c->N % 64 != 0 && (long)c->N * c->V * 2 >= (1L << 31)) return BLK_EUNSUPPORTED;
  if ((long)c->N * c->V >= (1L << 40)) return BLK_EUNSUPPORTED;
  return BLK_OK;
}

struct HeadScratch {
  bf16* h; float* r;                                  // normalised rows, 1/rms
  float2* part; float* tgt_logit;                     // forward: segment pairs, target logits
  float* nll_part; int* cnt_part; int* count;         // loss reduction
  bf16* dz; bf16* wt; bf16* dh; float* wpart;         // backward
  size_t bytes;
};

int head_lse_blocks(const blk_hcfg& c) { return (c.N + 3) / 4; }

HeadScratch carve_head(const blk_hcfg& c, void* base, bool bwd) {
  Carver k(base);
  HeadScratch s{};
  const long N = c.N, C = c.C, V = c.V;
  s.h = k.take<bf16>(N * C);
  s.r = k.take<float>(N);
  s.nll_part = k.take<float>(head_lse_blocks(c));
  s.cnt_part = k.take<int>(head_lse_blocks(c));
  s.count = k.take<int>(1);
  if (!bwd) {
    s.part = k.take<float2>(N * ((V + 127) / 128));
    s.tgt_logit = k.take<float>(N);
  } else {
    s.dz = k.take<bf16>(N * V);
    s.wt = k.take<bf16>(C * V);
    s.dh = k.take<bf16>(N * C);
    const int sp = wgrad_splits((int)V, (int)C, N, GemmTile<bf16>::BK);
    if (sp > 1) s.wpart = k.take<float>((size_t)sp * V * C);
  }
  s.bytes = (k.off + 255) & ~size_t(255);
  return s;
}

}  // namespace

extern "C" {

size_t block_saved_bytes(const blk_cfg* cfg) {
  if (check_cfg(cfg) != BLK_OK) return 0;
  return saved_bytes(*cfg);
}

size_t block_scratch_bytes(const blk_cfg* cfg) {
  if (check_cfg(cfg) != BLK_OK) return 0;
  return std::max(fwd_scratch_bytes(*cfg, true), bwd_bytes(*cfg));
}

int block_fwd(const blk_cfg* cfg, const void* x, const void* w_qkv, const void* w_o, const void* w_fc,
              const void* w_proj, void* y, void* saved, size_t saved_sz, void* scratch, size_t scratch_sz,
              void* stream) {
  int e = check_cfg(cfg);
  if (e) return e;
  const blk_cfg& c = *cfg;
  if (!x || !w_qkv || !w_o || !w_fc || !w_proj || !y) return BLK_EINVAL;
  if (x == y) return BLK_EINVAL;
  for (const void* p : {x, w_qkv, w_o, w_fc, w_proj, (const void*)y})
    if (!aligned(p)) return BLK_EALIGN;
  const size_t need = saved_bytes(c);
  void* store = saved;
  if (saved) {
    if (!aligned(saved)) return BLK_EALIGN;
    if (saved_sz < need) return BLK_ENOSPC;
  }
  const size_t scratch_need = fwd_scratch_bytes(c, saved == nullptr);
  if (scratch_need > 0) {
    if (!scratch) return BLK_EINVAL;
    if (!aligned(scratch)) return BLK_EALIGN;
    if (scratch_sz < scratch_need) return BLK_ENOSPC;
  }
  if (!saved) store = scratch;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipGetLastError();
  if (c.gemm == BLK_GEMM_FP8_E4M3) {
    char* f8 = static_cast<char*>(scratch) + (saved ? 0 : need);
    return fwd_fp8(c, (const bf16*)x, (const bf16*)w_qkv, (const bf16*)w_o, (const bf16*)w_fc, (const bf16*)w_proj,
                   (bf16*)y, carve_saved<bf16>(c, store), carve_fwd8(c, f8), st);
  }
  if (c.dtype == BLK_BF16)
    return fwd_impl<bf16>(c, (const bf16*)x, (const bf16*)w_qkv, (const bf16*)w_o, (const bf16*)w_fc,
                          (const bf16*)w_proj, (bf16*)y, carve_saved<bf16>(c, store), st);
  return fwd_impl<float>(c, (const float*)x, (const float*)w_qkv, (const float*)w_o, (const float*)w_fc,
                         (const float*)w_proj, (float*)y, carve_saved<float>(c, store), st);
}

int block_bwd(const blk_cfg* cfg, const void* dy, const void* x, const void* w_qkv, const void* w_o,
              const void* w_fc, const void* w_proj, const void* saved, size_t saved_sz, void* dx, float* dw_qkv,
              float* dw_o, float* dw_fc, float* dw_proj, int accumulate, void* scratch, size_t scratch_sz,
              void* stream) {
  int e = check_cfg(cfg);
  if (e) return e;
  const blk_cfg& c = *cfg;
  if (!dy || !x || !w_qkv || !w_o || !w_fc || !w_proj || !saved || !dx || !dw_qkv || !dw_o || !dw_fc || !dw_proj ||
      !scratch)
    return BLK_EINVAL;
  if (accumulate != 0 && accumulate != 1) return BLK_EINVAL;
  for (const void* p : {dy, x, w_qkv, w_o, w_fc, w_proj, saved, (const void*)dx, (const void*)dw_qkv,
                        (const void*)dw_o, (const void*)dw_fc, (const void*)dw_proj, (const void*)scratch})
    if (!aligned(p)) return BLK_EALIGN;
  if (saved_sz < saved_bytes(c) || scratch_sz < bwd_bytes(c)) return BLK_ENOSPC;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipGetLastError();
  if (c.gemm == BLK_GEMM_FP8_E4M3)
    return bwd_fp8(c, (const bf16*)dy, (const bf16*)w_qkv, (const bf16*)w_o, (const bf16*)w_fc, (const bf16*)w_proj,
                   carve_saved<bf16>(c, const_cast<void*>(saved)), (bf16*)dx, dw_qkv, dw_o, dw_fc, dw_proj, accumulate,
                   carve_bwd<bf16>(c, scratch), st);
  if (c.dtype == BLK_BF16)
    return bwd_impl<bf16>(c, (const bf16*)dy, (const bf16*)x, (const bf16*)w_qkv, (const bf16*)w_o,
                          (const bf16*)w_fc, (const bf16*)w_proj, carve_saved<bf16>(c, const_cast<void*>(saved)),
                          (bf16*)dx, dw_qkv, dw_o, dw_fc, dw_proj, accumulate, carve_bwd<bf16>(c, scratch), st);
  return bwd_impl<float>(c, (const float*)dy, (const float*)x, (const float*)w_qkv, (const float*)w_o,
                         (const float*)w_fc, (const float*)w_proj, carve_saved<float>(c, const_cast<void*>(saved)),
                         (float*)dx, dw_qkv, dw_o, dw_fc, dw_proj, accumulate, carve_bwd<float>(c, scratch), st);
}

size_t decode_scratch_bytes(const blk_dcfg* cfg) {
  if (check_dcfg(cfg) != BLK_OK) return 0;
  return carve_dec(*cfg, nullptr).bytes;
}

int decode_step(const blk_dcfg* cfg, const void* x, const void* w_qkv, const void* w_o, const void* w_fc,
                const void* w_proj, void* k_cache, void* v_cache, const int32_t* cache_len, int32_t* status, void* y,
                void* scratch, size_t scratch_bytes, void* stream) {
  if (int e = check_decode_args(cfg, x, w_qkv, w_o, w_fc, w_proj, k_cache, v_cache, cache_len, status, y)) return e;
  if (!scratch) return BLK_EINVAL;
  if (!aligned(scratch)) return BLK_EALIGN;
  if (scratch_bytes < carve_dec(*cfg, nullptr).bytes) return BLK_ENOSPC;
  return decode_run(*cfg, x, w_qkv, w_o, w_fc, w_proj, k_cache, v_cache, cache_len, status, y, scratch,
                    static_cast<hipStream_t>(stream));
}

int decode_step_noalloc(const blk_dcfg* cfg, const void* x, const void* w_qkv, const void* w_o, const void* w_fc,
                        const void* w_proj, void* k_cache, void* v_cache, const int32_t* cache_len, int32_t* status,
                        void* y, void* stream) {
  if (int e = check_decode_args(cfg, x, w_qkv, w_o, w_fc, w_proj, k_cache, v_cache, cache_len, status, y)) return e;
  if (carve_dec(*cfg, nullptr).bytes > BLK_NOALLOC_SCRATCH_BYTES) return BLK_ELIMIT;
  void* ws = nullptr;
  if (int e = noalloc_workspace(&ws)) return e;
  return decode_run(*cfg, x, w_qkv, w_o, w_fc, w_proj, k_cache, v_cache, cache_len, status, y, ws,
                    static_cast<hipStream_t>(stream));
}

int block_fp8_quantize(const void* x, size_t n, void* codes, uint32_t* amax, void* stream) {
  if (!x || !codes || !amax) return BLK_EINVAL;
  if (n == 0 || n % 8 != 0) return BLK_EINVAL;
  if (!aligned(x) || !aligned(codes) || (reinterpret_cast<uintptr_t>(amax) & 3)) return BLK_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipGetLastError();
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, st, (unsigned*)amax, 1);
  quantize(static_cast<const bf16*>(x), 1, (long)n, (unsigned*)amax, static_cast<uint8_t*>(codes), nullptr, 0, true, st);
  return launch_status();
}

int block_fp8_quantize_2d(const void* x, int64_t rows, int64_t cols, void* codes, void* codes_t, int64_t ldt,
                          uint32_t* amax, void* stream) {
  if (!x || !codes_t || !amax) return BLK_EINVAL;
  if (rows < 1 || rows >= (1LL << 31) || cols < 64 || cols % 64 != 0 || cols >= (1LL << 31)) return BLK_EINVAL;
  if (ldt < rows || ldt % 64 != 0 || ldt >= (1LL << 31)) return BLK_EINVAL;
  if (!aligned(x) || !aligned(codes_t) || (codes && !aligned(codes)) || (reinterpret_cast<uintptr_t>(amax) & 3))
    return BLK_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipGetLastError();
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, st, (unsigned*)amax, 1);
  quantize(static_cast<const bf16*>(x), rows, cols, (unsigned*)amax, static_cast<uint8_t*>(codes),
           static_cast<uint8_t*>(codes_t), ldt, true, st);
  return launch_status();
}

int block_mfma_probe(int kind, int workgroups, int iters, float* sink, void* stream) {
  if ((kind != 0 && kind != 1) || workgroups < 1 || iters < 1 || !sink) return BLK_EINVAL;
  if (reinterpret_cast<uintptr_t>(sink) & 3) return BLK_EALIGN;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipGetLastError();
  hipLaunchKernelGGL(kind == 0 ? mfma_probe_kernel<0> : mfma_probe_kernel<1>, dim3(workgroups), dim3(256), 0, st,
                     iters, sink);
  return launch_status();
}

void block_timing_enable(int on) {
  std::lock_guard<std::mutex> l(g_tmu);
  g_timing = on != 0;
  g_recs.clear();
  g_pool_used = 0;
}

int block_timing_read(int max, const char** names, double* total_ms, int* counts) {
  std::lock_guard<std::mutex> l(g_tmu);
  int n = 0;
  for (const TimingRec& r : g_recs) {
    if (hipEventSynchronize(r.b) != hipSuccess) return -1;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return -1;
    int i = 0;
    while (i < n && std::strcmp(names[i], r.name) != 0) ++i;
    if (i == n) {
      if (n == max) continue;
      names[n] = r.name; total_ms[n] = 0.0; counts[n] = 0;
      ++n;
    }
    total_ms[i] += ms;
    counts[i] += 1;
  }
  g_recs.clear();
  g_pool_used = 0;
  return n;
}

size_t head_scratch_bytes(const blk_hcfg* cfg) {
  if (check_hcfg(cfg) != BLK_OK) return 0;
  return std::max(carve_head(*cfg, nullptr, false).bytes, carve_head(*cfg, nullptr, true).bytes);
}

int head_loss_fwd(const blk_hcfg* cfg, const void* x, const void* w_lm, const int32_t* targets, float* loss,
                  float* lse, void* scratch, size_t scratch_sz, void* stream) {
  int e = check_hcfg(cfg);
  if (e) return e;
  const blk_hcfg& c = *cfg;
  if (!x || !w_lm || !targets || !loss || !lse || !scratch) return BLK_EINVAL;
  for (const void* p : {x, w_lm, (const void*)scratch})
    if (!aligned(p)) return BLK_EALIGN;
  if ((reinterpret_cast<uintptr_t>(targets) | reinterpret_cast<uintptr_t>(loss) | reinterpret_cast<uintptr_t>(lse)) & 3)
    return BLK_EALIGN;
  const HeadScratch s = carve_head(c, scratch, false);
  if (scratch_sz < s.bytes) return BLK_ENOSPC;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int N = c.N, C = c.C, V = c.V;
  {
    Timed t("head_rmsnorm", st);
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<bf16>, dim3(row_blocks(N)), dim3(256), 0, st, (const bf16*)x, s.h, s.r, N,
                       C, c.eps, (unsigned*)nullptr);
  }
  {
    GemmArgs g = gargs(s.h, C, w_lm, C, N, V, C);
    g.tgt = targets; g.lse_part = s.part; g.nseg = (V + 127) / 128; g.tgt_logit = s.tgt_logit;
    gemm_pp<bf16>(gemm_head_fwd, "gemm_head_fwd", g, st);
  }
  {
    Timed t("head_lse", st);
    hipLaunchKernelGGL(head::head_lse_kernel, dim3(head_lse_blocks(c)), dim3(256), 0, st, (const float2*)s.part,
                       (V + 127) / 128, (const float*)s.tgt_logit, (const int*)targets, N, V, lse, s.nll_part,
                       s.cnt_part);
    hipLaunchKernelGGL(head::head_loss_kernel, dim3(1), dim3(1024), 0, st, (const float*)s.nll_part,
                       (const int*)s.cnt_part, head_lse_blocks(c), loss, s.count);
  }
  return launch_status();
}

int head_loss_bwd(const blk_hcfg* cfg, const void* x, const void* w_lm, const int32_t* targets, const float* lse,
                  float dloss, void* dx, float* dw_lm, int accumulate, void* scratch, size_t scratch_sz,
                  void* stream) {
  int e = check_hcfg(cfg);
  if (e) return e;
  const blk_hcfg& c = *cfg;
  if (!x || !w_lm || !targets || !lse || !dx || !dw_lm || !scratch) return BLK_EINVAL;
  if (accumulate != 0 && accumulate != 1) return BLK_EINVAL;
  if (x == dx) return BLK_EINVAL;
  for (const void* p : {x, w_lm, (const void*)dx, (const void*)dw_lm, (const void*)scratch})
    if (!aligned(p)) return BLK_EALIGN;
  if ((reinterpret_cast<uintptr_t>(targets) | reinterpret_cast<uintptr_t>(lse)) & 3) return BLK_EALIGN;
  const HeadScratch s = carve_head(c, scratch, true);
  if (scratch_sz < s.bytes) return BLK_ENOSPC;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int N = c.N, C = c.C, V = c.V;
  {
    Timed t("head_rmsnorm", st);
    hipLaunchKernelGGL(rmsnorm_fwd_kernel<bf16>, dim3(row_blocks(N)), dim3(256), 0, st, (const bf16*)x, s.h, s.r, N,
                       C, c.eps, (unsigned*)nullptr);
    hipLaunchKernelGGL(head::head_count_kernel, dim3(1), dim3(1024), 0, st, (const int*)targets, N, V, s.count);
  }
  {  // dz = dloss/count * (softmax(z) - onehot), z recomputed
    GemmArgs g = gargs(s.h, C, w_lm, C, N, V, C);
    g.out = s.dz; g.ldo = V;
    g.tgt = targets; g.lse_in = lse; g.count = s.count; g.dscale = dloss;
    gemm_pp<bf16>(gemm_head_dz, "gemm_head_dz", g, st);
  }
  {
    Timed t("transpose_head", st);
    hipLaunchKernelGGL(transpose_kernel<bf16>, dim3(C / 64, V / 64), dim3(256), 0, st, (const bf16*)w_lm, s.wt, V, C);
  }
  {  // dh = dz W
    GemmArgs g = gargs(s.dz, V, s.wt, V, N, C, V);
    g.out = s.dh; g.ldo = C;
    gemm_pp<bf16>(gemm_head_dgrad, "gemm_head_dgrad", g, st);
  }
  // dW = dz^T h  (fp32, overwrite or accumulate)
  wgrad<bf16>(gemm_head_wgrad<bf16>, gemm_head_wgrad_acc<bf16>, gemm_head_wgrad_pp, gemm_head_wgrad_acc_pp,
              "gemm_head_wgrad", s.dz, s.h, dw_lm, V, C, N, accumulate, s.wpart, st);
  {
    Timed t("head_rmsnorm_bwd", st);
    hipLaunchKernelGGL(rmsnorm_bwd_kernel<bf16>, dim3(row_blocks(N)), dim3(256), 0, st, (const bf16*)nullptr,
                       (const bf16*)s.dh, (const bf16*)s.h, (const float*)s.r, (bf16*)dx, N, C, (unsigned*)nullptr);
  }
  return launch_status();
}

const char* block_strerror(int code) {
  switch (code) {
    case BLK_OK: return "ok";
    case BLK_EINVAL: return "invalid argument (size, dtype, mode or null pointer)";
    case BLK_EALIGN: return "pointer not 16-byte aligned";
    case BLK_ENOSPC: return "saved or scratch buffer too small";
    case BLK_EUNSUPPORTED: return "configuration not supported";
    case BLK_ELAUNCH: return "kernel launch failed";
    case BLK_ELIMIT: return "workspace needed exceeds the library's static workspace (decode_step_noalloc)";
    default: return "unknown status";
  }
}

}  // extern "C"
