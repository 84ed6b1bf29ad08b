/*
 * blk.h -- C ABI of the MI355X (gfx950) decoder-block library.
 *
 * One training step (forward + backward) and one KV-cache decode step of the
 * dense GPT decoder block that nanochat trains:
 *
 *   h1 = rmsnorm(x)                       parameter-free RMSNorm
 *   [q|k|v] = h1 W_qkv^T                  fused QKV projection, no bias
 *   q, k <- rotary(q, k); q, k <- rmsnorm  rotary embedding, then QK-norm
 *   o = softmax(q k^T / sqrt(D), causal) v   multi-head attention, D = 128
 *   y1 = x + o W_o^T                      output projection + residual
 *   h2 = rmsnorm(y1)
 *   y = y1 + relu(h2 W_fc^T)^2 W_proj^T   4x MLP with ReLU^2 + residual
 *
 * Sources: the flicky.cc course page "nanochat: свой ChatGPT от токенизатора
 * до чата", section "Модель: что изменилось со времён GPT-2" (rotary, QK-norm,
 * ReLU^2, parameter-free RMSNorm, no biases); the CSDN article "4小时100美元！
 * Andrej Karpathy新开源项目nanochat..." section 一 item 1 (dense Llama-like
 * transformer, rotary, QK norm); the 7minutos.es article, section "Modelo,
 * escalado y objetivo de speedrun" (d20: 1280 channels, 10 heads of 128); the
 * README mirror "karpathy/nanochat", section "精度 / dtype" (weights kept in
 * fp32 and cast to the compute dtype inside the linear layer; bf16 compute).
 *
 * Conventions shared by every entry point
 *   - Every data pointer is a DEVICE pointer, 16-byte aligned, to a dense
 *     row-major array; the caller allocates and owns every buffer.  The
 *     library allocates no memory, keeps no pointer after returning, and
 *     holds no state between calls (except the lazily loaded kernels and
 *     the static device workspace of decode_step_noalloc).
 *   - Weights are [out, in] and act as y = x W^T (the PyTorch Linear layout).
 *   - Element type of activations and weights: cfg->dtype (BLK_F32 or
 *     BLK_BF16).  Weight gradients are always float32.  Statistics, softmax
 *     and every MFMA accumulation are float32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued on it, in order, with no host synchronisation; results are
 *     ready when the stream reaches that point.
 *   - Return value: BLK_OK, or an error code below.  Every argument is
 *     checked on the host before any launch; on an error nothing has been
 *     enqueued.  Device faults surface at the caller's next synchronisation.
 *     No C++ exception crosses this interface.
 *   - Sizes: D must be 128, C == H*D, F == 4*C; B, T >= 1.  Any T is
 *     accepted (ragged tiles are masked inside the kernels).  Limits
 *     (BLK_EUNSUPPORTED): B*T*(C + 256*G) < 2^31 elements; and when a weight
 *     gradient runs on the four-wave GEMM body (float32 always; bf16 when
 *     B*T is not a multiple of 64; fp8 when it is not a multiple of 128),
 *     its widest operand, B*T x max(F, C + 256*G) elements (fp8: the
 *     transposed E4M3 copy, B*T rounded up to 64), stays below 4 GiB.
 */
#ifndef BLK_H
#define BLK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum blk_status {
  BLK_OK = 0,
  BLK_EINVAL = 1,        /* bad size, dtype, mode or NULL pointer            */
  BLK_EALIGN = 2,        /* a pointer is not 16-byte aligned                 */
  BLK_ENOSPC = 3,        /* saved/scratch buffer smaller than required       */
  BLK_EUNSUPPORTED = 4,  /* valid but not provided (e.g. fp8 with float32)   */
  BLK_ELAUNCH = 5,       /* a kernel launch failed (hipGetLastError)          */
  BLK_ELIMIT = 6         /* the call needs more workspace than the library's
                          * static workspace holds (decode_step_noalloc)      */
};

enum blk_dtype { BLK_F32 = 0, BLK_BF16 = 1 };

/* GEMM mode of the four linear layers.  BLK_GEMM_FP8_E4M3: every GEMM of
 * every linear layer (forward, input gradient, weight gradient) takes OCP
 * E4M3 operands with per-tensor current scaling s = amax/448, accumulates in
 * float32 and applies s_A*s_B in its epilogue; attention, norms and rotary
 * stay in bf16.  Requires dtype == BLK_BF16.  (FP8 training of the linear
 * layers: the flicky.cc page's repository map row for nanochat/fp8.py and the
 * README mirror's leaderboard row "d26 ... +fp8".) */
enum blk_gemm_mode { BLK_GEMM_NATIVE = 0, BLK_GEMM_FP8_E4M3 = 1 };

typedef struct {
  int32_t B, T;        /* sequences, tokens per sequence                     */
  int32_t C, H, D, F;  /* width, heads, head size (128), MLP width (4C)     */
  float eps;           /* RMSNorm / QK-norm epsilon (1e-6 in the workloads) */
  float rope_base;     /* rotary base (10000)                                */
  int32_t dtype;       /* enum blk_dtype                                     */
  int32_t gemm;        /* enum blk_gemm_mode                                 */
  int32_t window;      /* attention window W: 0 = causal over the whole
                        * sequence; W >= 1: token i attends to tokens
                        * i-W < j <= i (W >= T is the same as 0).  The
                        * flicky.cc course page, section on what changed
                        * since GPT-2, alternates short windows of a quarter
                        * of the context with full ones across layers; the
                        * per-layer choice is the caller's.  < 0: EINVAL.   */
  int32_t n_kv_head;   /* key/value heads G (0 = H: multi-head attention);
                        * G must divide H.  Query heads form G groups that
                        * share one K/V pair (grouped-query attention, listed
                        * on the flicky.cc course page's model section):
                        * w_qkv is [(H + 2G) D, C], its output rows
                        * [q (H heads) | k (G heads) | v (G heads)], and
                        * query head h attends with key/value head
                        * h / (H / G).                                       */
} blk_cfg;

typedef struct {
  int32_t B;           /* sequences, one new token each                      */
  int32_t C, H, D, F;
  int32_t S_max;       /* cache capacity (slots) per sequence and head       */
  float eps, rope_base;
  int32_t dtype;       /* BLK_BF16 or BLK_F32                                */
  int32_t window;      /* as blk_cfg.window: the new token at position p
                        * attends to slots p-W < j <= p (0 = all 0..p)       */
  int32_t n_kv_head;   /* as blk_cfg.n_kv_head; the caches are
                        * [B, G, S_max, D]                                   */
} blk_dcfg;

/* Language-model head and loss, the step after the block stack.
 *   h = rmsnorm(x) (parameter-free, eps), z = h W^T with the untied head
 *   W [V, C] (no bias, no cap), loss = mean over the counted rows of
 *   lse(z_i) - z_i[t_i]; a row counts when its target t_i is in [0, V).
 *   (The flicky.cc course page: untied embedding and lm_head, norms without
 *   parameters, the loss behind the bits-per-byte metric; the CSDN page: a
 *   Llama-like stack, hence the final norm.)  bf16 only (BLK_EUNSUPPORTED
 *   for BLK_F32); V a multiple of 64 (the vocabulary is padded to one), C a
 *   multiple of 128.  The logits are never stored. */
typedef struct {
  int32_t N;           /* rows (tokens)                                      */
  int32_t C;           /* width                                              */
  int32_t V;           /* vocabulary                                         */
  float eps;           /* final RMSNorm epsilon (1e-6)                       */
  int32_t dtype;       /* BLK_BF16                                           */
} blk_hcfg;

/* Bytes of scratch head_loss_fwd / head_loss_bwd need (the larger of the
 * two; the backward holds the softmax gradient [N, V] in bf16).  0 for an
 * invalid cfg. */
size_t head_scratch_bytes(const blk_hcfg* cfg);

/* Forward: x [N, C] (bf16), w_lm [V, C] (bf16), targets [N] (int32, device);
 * writes *loss (one float, device) and lse [N] (float32, natural-log
 * log-sum-exp of each row's logits, kept for the backward).  With no
 * counted row *loss = 0.  BLK_EINVAL (bad cfg, NULL pointer), BLK_EALIGN
 * (x, w_lm, scratch not 16-byte, targets/loss/lse not 4-byte aligned),
 * BLK_ENOSPC (short scratch). */
int head_loss_fwd(const blk_hcfg* cfg, const void* x, const void* w_lm, const int32_t* targets,
                  float* loss, float* lse, void* scratch, size_t scratch_bytes, void* stream);

/* Backward of dloss * loss: dx [N, C] (bf16; may not alias x) and
 * dw_lm [V, C] (float32, overwritten, or added to with accumulate = 1), from
 * the lse the forward wrote.  Errors as head_loss_fwd, plus BLK_EINVAL for
 * accumulate not 0/1 or dx == x. */
int head_loss_bwd(const blk_hcfg* cfg, const void* x, const void* w_lm, const int32_t* targets,
                  const float* lse, float dloss, void* dx, float* dw_lm, int accumulate,
                  void* scratch, size_t scratch_bytes, void* stream);

/* Bytes of the activation store that block_fwd fills for block_bwd.
 * Returns 0 for an invalid cfg. */
size_t block_saved_bytes(const blk_cfg* cfg);

/* Bytes of temporary device memory block_fwd / block_bwd need (the larger
 * of the two; covers block_fwd with saved == NULL).  0 for an invalid cfg. */
size_t block_scratch_bytes(const blk_cfg* cfg);

/* Forward of the block.
 *   x      [B,T,C]   input rows (dtype)
 *   (fp8 mode: scratch is always required; it holds the E4M3 operand copies)
 *   w_qkv  [3C,C], w_o [C,C], w_fc [F,C], w_proj [C,F]   (dtype)
 *   y      [B,T,C]   output (dtype); may not alias x
 *   saved  activation store of block_saved_bytes(cfg) bytes, written here and
 *          read by block_bwd; NULL for inference only
 *   scratch            block_scratch_bytes(cfg) bytes
 * The rotary angle of token t of each sequence is t * rope_base^(-2i/D). */
int block_fwd(const blk_cfg* cfg, const void* x,
              const void* w_qkv, const void* w_o, const void* w_fc, const void* w_proj,
              void* y, void* saved, size_t saved_bytes,
              void* scratch, size_t scratch_bytes, void* stream);

/* Backward of the block: gradients of <dy, y>.
 *   dy     [B,T,C]   upstream gradient (dtype)
 *   x, weights: as passed to the block_fwd that filled `saved`
 *   dx     [B,T,C]   input gradient (dtype), written
 *   dw_*   float32 weight gradients, same shapes as the weights; overwritten
 *          when accumulate == 0, added to when accumulate == 1 (gradient
 *          accumulation over micro-batches)
 * Deterministic: the same inputs give bitwise the same outputs. */
int block_bwd(const blk_cfg* cfg, const void* dy, const void* x,
              const void* w_qkv, const void* w_o, const void* w_fc, const void* w_proj,
              const void* saved, size_t saved_bytes, void* dx,
              float* dw_qkv, float* dw_o, float* dw_fc, float* dw_proj, int accumulate,
              void* scratch, size_t scratch_bytes, void* stream);

/* Bytes of temporary device memory decode_step needs.  0 for invalid cfg. */
size_t decode_scratch_bytes(const blk_dcfg* cfg);

/* One decode step of the block: a new token per sequence at position
 * p_b = cache_len[b] attends to the cached keys and values of slots
 * 0..p_b (its own included).  Inference with a KV cache (prefill, then one
 * token per step) is named on the 7minutos.es page, section on midtraining,
 * SFT and tool use, and in the launch thread on the same subject; the block
 * computed for the new row is the one described at the top of this file.
 *   x       [B,C]               new rows (bf16)
 *   k_cache, v_cache [B,G,S_max,D]  (bf16; G = n_kv_head, or H when 0) keys
 *           after rotary and QK-norm,
 *           and values; slot p_b of each (b, h) is written here, slots
 *           0..p_b are attended, slots beyond p_b are neither read nor written
 *   cache_len [B] int32 DEVICE array, read only (the caller advances it);
 *           every entry must satisfy 0 <= cache_len[b] <= S_max-1.  The
 *           lengths live on the device, so the host cannot check them: a
 *           sequence whose entry is outside that range is an error of that
 *           sequence only: its cache slots are not written, its row of y is
 *           NaN, and the step counts it in *status
 *   status  one int32 DEVICE word, or NULL: set by the step to the number of
 *           sequences whose cache_len is out of range (0 when all are valid)
 *   y       [B,C] output (bf16); may be the same buffer as x
 *   scratch at least decode_scratch_bytes(cfg) bytes of device memory
 * Only cfg->dtype == BLK_BF16 and C <= 2048 are implemented (else
 * BLK_EUNSUPPORTED).  BLK_EINVAL for a bad cfg, a NULL pointer, or
 * k_cache == v_cache; BLK_EALIGN for a data pointer not 16-byte aligned or
 * cache_len / status not 4-byte aligned; BLK_ENOSPC for a short scratch. */
int decode_step(const blk_dcfg* cfg, const void* x,
                const void* w_qkv, const void* w_o, const void* w_fc, const void* w_proj,
                void* k_cache, void* v_cache, const int32_t* cache_len, int32_t* status, void* y,
                void* scratch, size_t scratch_bytes, void* stream);

/* Bytes of the static workspace decode_step_noalloc uses on each device. */
#define BLK_NOALLOC_SCRATCH_BYTES (32u << 20)

/* decode_step without a caller-supplied scratch buffer, for callers that
 * cannot allocate device memory on the call path (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, results and errors as decode_step, with the temporaries in a
 * static workspace of BLK_NOALLOC_SCRATCH_BYTES (32 MiB) that the library
 * keeps on each device for the life of the process (its address is looked
 * up on the first call on each device).  Returns BLK_ELIMIT, with nothing
 * enqueued, when decode_scratch_bytes(cfg) exceeds that size (d20 with 64
 * sequences and 2049 cache slots needs 10.7 MiB).  The call allocates
 * nothing.  Every call on one GPU uses that GPU's single workspace: calls
 * whose work overlaps on one GPU (other streams, other host threads) race
 * and give wrong results; calls enqueued in order on one stream do not. */
int decode_step_noalloc(const blk_dcfg* cfg, const void* x,
                        const void* w_qkv, const void* w_o, const void* w_fc, const void* w_proj,
                        void* k_cache, void* v_cache, const int32_t* cache_len, int32_t* status, void* y,
                        void* stream);

/* The quantiser of the fp8 mode as a standalone call: amax = max |x| over
 * the n bf16 values at x (n a multiple of 8), written as float bits to the
 * device word *amax, and codes[i] = E4M3(x[i] * 448/amax) rounded to nearest
 * even, saturating at +-448 (amax == 0 gives scale 1).  x and codes are
 * device pointers, 16-byte aligned; codes holds n bytes. */
int block_fp8_quantize(const void* x, size_t n, void* codes, uint32_t* amax, void* stream);

/* The same quantiser on a rows x cols bf16 matrix x (row-major, leading
 * dimension cols), in the form the fp8 mode applies it to the operands of
 * its weight-gradient GEMMs: amax = max |x| written to *amax as float bits;
 * codes[r][c] = E4M3(x[r][c] * 448/amax) when codes is not NULL; and the
 * transposed copy codes_t[c][r] with leading dimension ldt (>= rows, a
 * multiple of 64), whose padding columns rows .. ldt-1 are written as 0.
 * (OCP 8-bit E4M3, per-tensor scale from the current amax: fp8 training as
 * the flicky.cc nanochat page's repository map row for nanochat/fp8.py and
 * the leaderboard row "d26 ... +fp8" of the pigsec.cn README mirror name
 * it.)  rows in [1, 2^31), cols a positive multiple
 * of 64 below 2^31; device pointers 16-byte aligned (amax 4-byte aligned).
 * BLK_EINVAL for a NULL x, codes_t or amax, or a bad size; BLK_EALIGN for a
 * misaligned pointer. */
int block_fp8_quantize_2d(const void* x, int64_t rows, int64_t cols, void* codes, void* codes_t, int64_t ldt,
                          uint32_t* amax, void* stream);

/* Measurement hooks (for benchmarks; not needed to compute anything).
 * block_timing_enable(1) starts recording, for every kernel launch site of
 * the calls above, a pair of hipEvents around the launch on the call's
 * stream; block_timing_enable(0) stops.  Either call drops what was recorded.
 * block_timing_read waits for the recorded events, then fills up to `max`
 * entries: names[i] (static strings naming the launch site, e.g.
 * "gemm_fc_fwd", "attn_fwd"), total_ms[i] and counts[i] (launches), clears
 * the records, and returns the number of entries (-1 on a HIP error). */
void block_timing_enable(int on);
int block_timing_read(int max, const char** names, double* total_ms, int* counts);

/* Measurement hook: the matrix cores' achievable rate.  Launches
 * `workgroups` workgroups of four waves; each wave runs `iters` rounds of
 * four independent 32x32 MFMAs from registers (kind 0: bf16 32x32x16,
 * 2*32*32*16 FLOP each; kind 1: OCP E4M3 32x32x64, 2*32*32*64 FLOP each)
 * and writes one float per lane to sink (workgroups * 256 floats, device,
 * 4-byte aligned).  Time it with events on the stream.  BLK_EINVAL for a bad
 * kind, count or NULL sink. */
int block_mfma_probe(int kind, int workgroups, int iters, float* sink, void* stream);

/* Static, human-readable text of a status code. */
const char* block_strerror(int code);

#ifdef __cplusplus
}
#endif
#endif /* BLK_H */
