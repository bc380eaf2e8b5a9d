/*
 * dtb.h -- C ABI of libdtb.so: one pre-norm decoder-only transformer block,
 * forward and backward, and causal grouped-query flash attention, as
 * hand-written HIP kernels for AMD gfx950 (MI355X).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Problem statement (B, T, C, NH, NKV) as in the flash_attn_forward_kernel /
 *   flash_attn_backward_kernel declarations of the "nanoeuler — CUDA kernels"
 *   page: B sequences of T tokens, model width C, NH query heads of width
 *   hd = C / NH, NKV key/value heads; query head h reads kv head h / (NH/NKV).
 * - Activations are row-major [B, T, width].  The packed qkv row of token
 *   (b, t) is [q heads (NH*hd) | k heads (NKV*hd) | v heads (NKV*hd)], width
 *   QKV = C + 2*NKV*hd (that page's `qkvd`).
 * - Weights are row-major [out, in] (that page's parameter layout `W`, and
 *   llm.c's ParameterTensors): a linear layer computes y = x W^T + b.
 * - dtype DTB_F32: every activation, weight, gamma and bias is fp32.
 *   dtype DTB_BF16: they are bf16 (raw 16-bit storage, round-to-nearest-even
 *   on store); accumulation is fp32.  In both cases lse, the saved norm
 *   statistics and every parameter gradient are fp32.
 * - All pointers are DEVICE pointers (hipMalloc'd or torch CUDA tensors) except
 *   the cfg / weights / grads structs themselves, which are read on the host
 *   during the call.  Buffers must be 16-byte aligned.
 * - The caller owns every buffer.  The library never allocates, frees or
 *   synchronises: each call validates its arguments on the host, enqueues
 *   kernels on `stream` (a hipStream_t; NULL = the null stream) and returns.
 *   It keeps no state between calls apart from its kernels (the opt-in
 *   measurement timing and the per-device address of attn_backward_noalloc's
 *   scratch array aside); the one second stream, of block_backward_overlap,
 *   is a handle the caller creates and destroys.
 * - Errors: 0 on success, a negative DTB_E* code otherwise (no kernel is
 *   enqueued when validation fails; the library never calls exit()).
 *   dtb_strerror() gives a message; for DTB_ELAUNCH it includes the HIP error.
 * - Calls on the same stream are ordered; calls on different streams that
 *   touch the same buffers race.
 * - Graph capture: the block, attention, linear, norm and activation entry
 *   points enqueue kernels and (block_backward_overlap) event waits only,
 *   never a memset, copy or host wait, so a stream capture of them replays
 *   to the same results; not while timing or debug mode is on.
 */
#ifndef DTB_H
#define DTB_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- codes ------------------------------------------------------------- */
#define DTB_OK 0
#define DTB_EINVAL_SHAPE (-1) /* C % NH, NH % NKV, hd unsupported, odd hd with RoPE,
                                 C or H not a multiple of 8, negative sizes, overflow */
#define DTB_EINVAL_PTR (-2)   /* a required pointer is NULL or misaligned */
#define DTB_EDTYPE (-3)       /* dtype not DTB_F32 / DTB_BF16 */
#define DTB_EINVAL_ENUM (-4)  /* unknown norm / mlp / rope selector */
#define DTB_ELAUNCH (-5)      /* a kernel launch failed; see dtb_strerror */

#define DTB_F32 0
#define DTB_BF16 1

#define DTB_NORM_RMS 0         /* RMSNorm with gamma */
#define DTB_NORM_RMS_NOGAMMA 1 /* RMSNorm without gamma */
#define DTB_NORM_LAYER 2       /* LayerNorm with gamma and beta */

#define DTB_MLP_SWIGLU 0       /* h = silu(x Wg^T) * (x Wu^T) */
#define DTB_MLP_RELU 1         /* h = relu(x W1^T + b1) */
#define DTB_MLP_GELU_TANH 2    /* h = gelu_tanh(x W1^T + b1) */

#define DTB_ROPE_NONE 0
#define DTB_ROPE_NEOX 1        /* half-split pairs (i, i + hd/2) */

/* Supported head widths: hd in {4, 8, 16, 32, 64, 128} for DTB_F32 and
 * {8, 16, 32, 64, 128} for DTB_BF16 (hd * element size a multiple of 16 bytes). */

/* ---- causal GQA flash attention ----------------------------------------
 * attn_forward: "nanoeuler — CUDA kernels", flash_attn_forward_kernel
 * declaration (packed qkv in; out and lse out), with the softmax of
 * attention_cpu_fwd on the same page:
 *   s_tj = (q_t . k_j) / sqrt(hd) for j <= t, o_t = sum_j softmax_j(s_t) v_j,
 *   lse_t = max_j s_tj + ln sum_j exp(s_tj - max_j s_tj)  (natural log).
 *   qkv  [B, T, QKV]  input, dtype
 *   out  [B, T, C]    output, dtype; head h at columns h*hd .. h*hd+hd-1
 *   lse  [B, NH, T]   output, fp32
 * B == 0 or T == 0 is a no-op.  No workspace.
 * One sequence must stay below 2^31 bytes of qkv: T * QKV * sizeof(dtype)
 * < 2^31 (rows are addressed by 32-bit offsets from the sequence's first
 * row), else DTB_EINVAL_SHAPE; the same limit holds for attn_backward and
 * for the block calls. */
int attn_forward(void *out, float *lse, const void *qkv, int B, int T, int C, int NH, int NKV,
                 int dtype, void *stream);

/* attn_backward: the same page's flash_attn_backward_kernel declaration
 * (dqkv from qkv, out, dout, lse); the gradient is the softmax backward of
 * attention_cpu_bwd there and of attention_backward on the "microgpt.cu" page:
 *   P_tj = exp(s_tj - lse_t), D_t = sum_d dO_td O_td, dS_tj = P_tj (dO_t.v_j - D_t),
 *   dq_t = sum_j dS_tj k_j / sqrt(hd), dk_j = sum_{t, h in group} dS_tj q_t / sqrt(hd),
 *   dv_j = sum_{t, h in group} P_tj dO_t.
 *   dqkv [B, T, QKV]  output, dtype, OVERWRITTEN (every element written)
 *   qkv, out, dout    inputs as in attn_forward (out and lse from attn_forward)
 *   workspace attn_workspace_bytes(B, T, NH) bytes of device scratch (holds
 *             -D = -rowsum(dO o) and -lse / scale, each [B, NH, T]
 *             fp32, written and read by the backward's own kernels);
 *             contents on entry are ignored
 * Deterministic (no atomics). */
int attn_backward(void *dqkv, const void *qkv, const void *out, const void *dout,
                  const float *lse, int B, int T, int C, int NH, int NKV, int dtype,
                  void *workspace, void *stream);
size_t attn_workspace_bytes(int B, int T, int NH);

/* attn_backward_noalloc: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as attn_backward (the same
 * kernels), without the workspace argument: its scratch (-D and -lse / scale,
 * 8 * B * NH * T bytes) lives in a device array inside the library,
 * DTB_NOALLOC_SCRATCH_BYTES (8 MiB) on each device it runs on, held until the
 * process ends.  8 * B * NH * T above that size is DTB_EINVAL_SHAPE (B * NH * T
 * up to 2^20: one 16384-token sequence of 64 heads, say).  The call allocates
 * and frees nothing (the array's device address is looked up once per device,
 * on the first call there) and clears nothing: every scratch value the
 * kernels read, they have written in the same call.  Every call on one
 * device shares that device's array, which keeps the last call's contents:
 * calls on one stream are ordered, but calls that can overlap in time on one
 * device (other streams, other host threads) race on it. */
#define DTB_NOALLOC_SCRATCH_BYTES (8u << 20)
int attn_backward_noalloc(void *dqkv, const void *qkv, const void *out, const void *dout,
                          const float *lse, int B, int T, int C, int NH, int NKV, int dtype,
                          void *stream);

/* ---- decode attention ---------------------------------------------------
 * One new query per sequence against that sequence's KV cache, forward only
 * ("microgpt.cu": attention_forward_kernel as forward_position calls it, the
 * newest position's query reading the cached keys and values of positions
 * 0 .. pos_id):
 *   out[b, h] = sum_{j < lens[b]} softmax_j(q[b, h] . k[b, j, kh] / sqrt(hd)) v[b, j, kh]
 *   lse[b, h] = natural-log logsumexp_j of the same scores,  kh = h / (NH/NKV)
 * The caller has already rotated q (RoPE at position lens[b]-1) and written
 * the newest position's key and value into row lens[b]-1 of the caches.
 *   out      [B][NH*hd] of dtype (written)
 *   lse      [B][NH] fp32 (written)
 *   q        [B][NH*hd] of dtype
 *   k_cache, v_cache  [B][Tmax][NKV*hd] of dtype: row t of sequence b holds
 *            kv head kh at columns kh*hd (a row holds every kv head of one
 *            position, as the microgpt cache rows do).  Rows at or past
 *            lens[b] are never read and may hold anything.
 *   lens     [B] int32 in device memory: cache rows in use, 0 .. Tmax.
 *            lens[b] = 0 gives out = 0 and lse = -inf (an empty softmax);
 *            a length outside [0, Tmax] gives NaN in that sequence's out and
 *            lse (the lengths are not visible to the host; nothing outside
 *            the caches is read)
 *   chunk    cache positions per workgroup, a multiple of 32, or 0 for the
 *            library's choice (sized from B, NKV and Tmax)
 *   workspace  attn_decode_workspace_bytes(...) bytes of device scratch
 *            (per-chunk partial results); contents on entry are ignored
 * dtype DTB_F32 or DTB_BF16 for q, the caches and out; hd as for
 * attn_forward; Tmax * NKV * hd * sizeof(dtype) below 2^31.  Deterministic. */
size_t attn_decode_workspace_bytes(int B, int NH, int NKV, int hd, int Tmax, int chunk, int dtype);
int attn_decode(void *out, float *lse, const void *q, const void *k_cache, const void *v_cache,
                const int *lens, int B, int NH, int NKV, int hd, int Tmax, int chunk, int dtype,
                void *workspace, void *stream);

/* attn_decode over caches in another arrangement of head rows (the same
 * computation, the same chunks and the same results bit for bit as attn_decode
 * on the same values): the hd contiguous elements of kv head kh at position t
 * of sequence b start at element
 *   b * stride_b + t * stride_t + kh * stride_h
 * of each cache (K and V share the strides).  attn_decode is the case
 * stride_b = Tmax*NKV*hd, stride_t = NKV*hd, stride_h = hd; the head-major
 * cache [B][NKV][Tmax][hd] is stride_b = NKV*Tmax*hd, stride_t = hd,
 * stride_h = Tmax*hd, in which one kv head's positions are contiguous and
 * stream from HBM in whole pages.  Requires stride_t >= hd, stride_b and
 * stride_h >= 0, and ((Tmax-1)*stride_t + hd) * sizeof(dtype) below 2^31
 * (DTB_EINVAL_SHAPE otherwise); the other arguments, the workspace and the
 * errors are those of attn_decode. */
int attn_decode_strided(void *out, float *lse, const void *q, const void *k_cache, const void *v_cache,
                        const int *lens, int B, int NH, int NKV, int hd, int Tmax, long long stride_b,
                        long long stride_t, long long stride_h, int chunk, int dtype, void *workspace,
                        void *stream);

/* ---- the block --------------------------------------------------------- */
typedef struct {
    int B, T, C, NH, NKV, H; /* H = MLP hidden width */
    int norm;                /* DTB_NORM_* (both norms of the block) */
    int mlp;                 /* DTB_MLP_* */
    int rope;                /* DTB_ROPE_* */
    float rope_base;         /* theta_i = rope_base^(-2i/hd) */
    float eps;               /* inside the square root of both norms */
    int qkv_bias, o_bias, mlp_bias; /* 0/1: which linear layers carry a bias */
    int dtype;               /* DTB_F32 / DTB_BF16 */
} dtb_block_cfg;

/* Block parameters (dtype storage).  Unused entries may be NULL.
 *   g1, b1   [C]      norm1 gamma / beta (beta: LayerNorm only)
 *   wqkv     [QKV, C] packed q, k, v projection; bqkv [QKV]
 *   wo       [C, C]   output projection; bo [C]
 *   g2, b2   [C]      norm2 gamma / beta
 *   w_up     SwiGLU: [2H, C], rows 0..H-1 the gate, rows H..2H-1 the up
 *            projection; ReLU / GELU: [H, C].  b_up [2H] or [H]
 *   w_down   [C, H];  b_down [C]
 *   rope_cs  optional, DTB_ROPE_NEOX only: the (cos, sin) table that
 *            rope_table_build writes for this config's T, head width C/NH
 *            and rope_base (its contents are not checked).
 *            NULL: block_forward and block_backward compute it in their
 *            workspace on every call; a table built once serves every layer
 *            of a stack and every step. */
typedef struct {
    const void *g1, *b1, *wqkv, *bqkv, *wo, *bo, *g2, *b2, *w_up, *b_up, *w_down, *b_down;
    const float *rope_cs;
} dtb_block_weights;

/* rope_table_build: the NeoX rotation table of "nx_f32_qwen2_train_gate.nx
 * source" build_rope / "nanoeuler — CUDA kernels" rope_kernel:
 *   cs[2 (t hd/2 + i)] = cos(t theta_i),  cs[2 (t hd/2 + i) + 1] = sin(t theta_i),
 *   theta_i = base^(-2i/hd),  0 <= t < T, 0 <= i < hd/2,
 * the angle and its cosine and sine in fp64, rounded to fp32.  cs: T*hd
 * floats, OVERWRITTEN.  T >= 0; hd even in [2, 256]; base > 0
 * (DTB_EINVAL_SHAPE otherwise; DTB_EINVAL_PTR for a null or misaligned cs
 * when T > 0). */
int rope_table_build(float *cs, int T, int hd, float base, void *stream);

/* Parameter gradients, fp32, same shapes as dtb_block_weights, ACCUMULATED
 * (+=): the caller zeroes them before the first backward of a step (cuBLAS
 * beta = 1 in nanoeuler's matmul_backward_*_cuda; += in llm.c's backward).
 * Entries for parameters the config does not use are ignored. */
typedef struct {
    float *g1, *b1, *wqkv, *bqkv, *wo, *bo, *g2, *b2, *w_up, *b_up, *w_down, *b_down;
} dtb_block_grads;

/* Byte offsets of the activations block_forward stores in `saved` (each
 * 256-byte aligned; -1 where the config has no such tensor).
 *   n1 [BT, C] dtype        norm1 output
 *   r1, mu1 [BT] fp32       norm1 rstd and mean (mean: LayerNorm only)
 *   qkv [BT, QKV] dtype     projection + bias, after RoPE on q and k
 *   o [BT, C] dtype         attention output;  lse [B, NH, T] fp32
 *   x2 [BT, C] dtype        x + attention branch
 *   n2, r2, mu2             as n1, r1, mu1 for norm2
 *   up [BT, 2H or H] dtype  MLP pre-activation ([gate | up] for SwiGLU)
 *   h [BT, H] dtype         MLP activation output */
typedef struct {
    long long n1, r1, mu1, qkv, o, lse, x2, n2, r2, mu2, up, h, total;
} dtb_saved_layout;

/* Sizes (bytes) of the caller-provided `saved` and `workspace` buffers for a
 * config; 0 if the config is invalid.  One workspace serves both calls. */
size_t block_saved_bytes(const dtb_block_cfg *cfg);
size_t block_workspace_bytes(const dtb_block_cfg *cfg);
int block_saved_layout(const dtb_block_cfg *cfg, dtb_saved_layout *layout);

/* Byte offsets, inside `workspace`, of the intermediate gradients that
 * block_backward leaves there (valid once its work on the stream has
 * completed, until the next call that uses the same workspace), for
 * inspection and testing; all dtype, row-major:
 *   dh [BT, H]          dy Wdown                       (activation output)
 *   dup [BT, 2H or H]   gradient of the MLP pre-activation ([gate | up])
 *   dn2 [BT, C]         dup Wup                        (norm2 output)
 *   dx2 [BT, C]         dy + Norm2^T(dn2)              (residual stream)
 *   dO [BT, C]          dx2 Wo                         (attention output)
 *   dqkv [BT, QKV]      attention backward, after the inverse RoPE of dq, dk
 *   dn1 [BT, C]         dqkv Wqkv                      (norm1 output) */
typedef struct {
    long long dh, dup, dn2, dx2, dO, dqkv, dn1, total;
} dtb_workspace_layout;
int block_workspace_layout(const dtb_block_cfg *cfg, dtb_workspace_layout *layout);

/* block_forward: the pre-norm block of "nanoeuler — CUDA kernels" run_train /
 * forward_gpu (RMSNorm, QKV GEMM, RoPE, flash attention, O GEMM + residual,
 * RMSNorm, MLP GEMMs, down GEMM + residual), generalised by the mini-Qwen2
 * trainer (QKV bias before NeoX RoPE), llm.c's gpt2_forward (LayerNorm, GELU,
 * biases) and microgpt.cu's forward_position (RMSNorm without gamma, ReLU):
 *   n1 = Norm1(x); qkv = n1 Wqkv^T + bqkv; RoPE(q, k); o, lse = attention(qkv);
 *   x2 = x + o Wo^T + bo; n2 = Norm2(x2); up = n2 Wup^T + bup; h = act(up);
 *   x_out = x2 + h Wdown^T + bdown.
 *   x_in  [B, T, C] dtype input;  x_out [B, T, C] dtype output (must not alias x_in)
 *   saved block_saved_bytes(cfg) bytes, written (read later by block_backward)
 *   workspace block_workspace_bytes(cfg) bytes, scratch */
int block_forward(const dtb_block_cfg *cfg, const dtb_block_weights *w, const void *x_in,
                  void *x_out, void *saved, void *workspace, void *stream);

/* block_backward: the backward of block_forward (nanoeuler run_train's
 * backward sequence; llm.c gpt2_backward):
 *   dh = dy Wdown (+dWdown, dbdown); dup = act'(dh); dn2 = dup Wup (+dWup, dbup);
 *   dx2 = dy + Norm2^T(dn2) (+dg2, db2); do = dx2 Wo (+dWo, dbo);
 *   dqkv = attention^T(do); inverse RoPE on dq, dk; dn1 = dqkv Wqkv (+dWqkv, dbqkv);
 *   dx = dx2 + Norm1^T(dn1) (+dg1, db1).
 *   x_in   the block input given to block_forward
 *   saved  as written by block_forward for the same x_in and weights
 *   dx_out [B, T, C] dtype: gradient of the loss w.r.t. x_out (input)
 *   dx_in  [B, T, C] dtype: gradient w.r.t. x_in (output, OVERWRITTEN);
 *          may alias dx_out (the residual gradient is updated in place)
 *   g      parameter gradients, fp32, ACCUMULATED
 *   workspace block_workspace_bytes(cfg) bytes, scratch
 * Every kernel runs on `stream`, one after another. */
int block_backward(const dtb_block_cfg *cfg, const dtb_block_weights *w, const void *x_in,
                   const void *saved, const void *dx_out, void *dx_in,
                   const dtb_block_grads *g, void *workspace, void *stream);

/* block_backward_overlap: block_backward with its four weight-gradient GEMMs
 * (dWdown, dWup, dWo, dWqkv) on a second stream that the caller owns: each
 * forks from `stream` once its output gradient exists and runs beside the
 * input-gradient GEMM of the same projection (the pages run them one after
 * another; both only read that gradient).  The second stream joins `stream`
 * before the call's last kernel, so all of the call's work is ordered before
 * anything enqueued on `stream` afterwards.  Results are bit-identical to
 * block_backward.  Arguments as block_backward, plus
 *   side  a handle from dtb_overlap_create on the current device
 *         (DTB_EINVAL_PTR if NULL or made on another device).
 * One handle holds one stream and two events: calls that share a handle
 * must be issued from one host thread at a time; calls with separate handles
 * are independent.  While a backward kernel class is timed
 * (dtb_timing_enable) everything runs on `stream`. */
typedef struct dtb_overlap_s *dtb_overlap;
int dtb_overlap_create(dtb_overlap *out); /* on the current device: a non-blocking stream of
                                             default priority and two events without timing */
int dtb_overlap_destroy(dtb_overlap h);   /* NULL is a no-op; pending work still completes */
int block_backward_overlap(const dtb_block_cfg *cfg, const dtb_block_weights *w, const void *x_in,
                           const void *saved, const void *dx_out, void *dx_in,
                           const dtb_block_grads *g, void *workspace, void *stream,
                           dtb_overlap side);

/* ---- component: one linear layer ------------------------------------------
 * The GEMMs block_forward / block_backward run, exposed on their own
 * ("nanoeuler — CUDA kernels": matmul_forward_cuda, matmul_backward_dinp_cuda,
 * matmul_backward_dw_cuda; llm.c matmul_forward / matmul_backward with bias).
 * linear_forward:  out[R, N] = inp[R, K] W[N, K]^T (+ bias[N]) (+ res[R, N])
 *   out, inp, w, bias, res: dtype; bias and res may be NULL; res may alias out.
 * linear_backward: dinp[R, K] = dout W (OVERWRITTEN);  dw[N, K] += dout^T inp;
 *   db[N] += sum_r dout[r, :]   (dw, db fp32, ACCUMULATED; dinp, dw or db may be
 *   NULL to skip that product).  workspace: linear_workspace_bytes(R, K, N, dtype)
 *   bytes (split-K partial sums of dw and column partials of db).
 * K and N must be multiples of 8; R >= 0. */
int linear_forward(void *out, const void *inp, const void *w, const void *bias, const void *res, int R,
                   int K, int N, int dtype, void *stream);
int linear_backward(void *dinp, float *dw, float *db, const void *dout, const void *inp, const void *w,
                    int R, int K, int N, int dtype, void *workspace, void *stream);
size_t linear_workspace_bytes(int R, int K, int N, int dtype);

/* ---- model harness ----------------------------------------------------------
 * The steps around the block stack that turn token ids into a loss and back:
 * embedding, a norm on its own (the final norm; the embedding RMSNorm of the
 * "microgpt.cu" forward_position), the LM head and the softmax cross-entropy.
 * ids / targets are int32 device arrays (4-byte aligned).
 *
 * encoder_forward: x[b, t, :] = wte[ids[b, t], :] (+ wpe[t, :])   ("nanoeuler —
 *   CUDA kernels" encoder_forward_kernel; llm.c encoder_forward with wpe).
 *   x [B, T, C], wte [V, C], wpe [T, C] or NULL: dtype.  An id outside [0, V)
 *   reads as a zero row.  C must be a multiple of 8.
 * encoder_backward: dwte[ids[b, t], :] += dx[b, t, :];  dwpe[t, :] += sum_b dx[b, t, :]
 *   (nanoeuler encoder_backward_kernel; llm.c encoder_backward).  dwte [V, C]
 *   and dwpe [T, C] fp32, ACCUMULATED; either may be NULL.  Repeated ids add
 *   into dwte by fp32 atomics, so the summation order (not the set of terms)
 *   varies from run to run; dwpe sums the B sequences in order. */
int encoder_forward(void *x, const int *ids, const void *wte, const void *wpe, int B, int T, int C, int V,
                    int dtype, void *stream);
int encoder_backward(float *dwte, float *dwpe, const int *ids, const void *dx, int B, int T, int C, int V,
                     int dtype, void *stream);

/* norm_forward / norm_backward: the block's norms on their own (DTB_NORM_*;
 * nanoeuler rmsnorm_forward_kernel / rmsnorm_backward_kernel, llm.c
 * layernorm_forward / layernorm_backward).
 *   out = Norm(x) [R, C] dtype; rstd [R] fp32; mean [R] fp32 (LayerNorm only,
 *   else may be NULL).  g, b [C] dtype (g unused for RMS_NOGAMMA, b LayerNorm only).
 *   norm_backward: dx = dres + Norm^T(dy) (OVERWRITTEN; dres may be NULL, may
 *   alias dx);  dg, db [C] fp32 ACCUMULATED.  workspace norm_workspace_bytes(R, C)
 *   bytes (per-workgroup partial sums, and for rows wider than a wave holds in
 *   registers (C above 4096 bf16 / 2048 fp32) the per-row statistics of a
 *   first pass; deterministic).  C a multiple of
 *   8, at most 8192 (bf16) / 4096 (fp32). */
int norm_forward(void *out, float *rstd, float *mean, const void *x, const void *g, const void *b, int R, int C,
                 int norm, float eps, int dtype, void *stream);
int norm_backward(void *dx, float *dg, float *db, const void *dy, const void *x, const void *g, const float *rstd,
                  const float *mean, const void *dres, int R, int C, int norm, int dtype, void *workspace,
                  void *stream);
size_t norm_workspace_bytes(int R, int C);

/* activation_forward / activation_backward: the block's MLP activation on its
 * own (DTB_MLP_*; "nanoeuler — CUDA kernels" swiglu_forward_kernel /
 * swiglu_backward_kernel, "microgpt.cu" relu_forward_kernel /
 * relu_backward_kernel, llm.c gelu_forward / gelu_backward, tanh form).
 *   up  [R, 2H] for SwiGLU (gate columns 0..H-1, then up columns), else [R, H]
 *   h   [R, H]  = silu(gate) * up, relu(up) or gelu_tanh(up)  (OVERWRITTEN)
 *   dup [R, 2H or H] = gradient of up from dh [R, H]         (OVERWRITTEN)
 * All dtype; H a multiple of 8.  (In block_forward the SwiGLU forward runs in
 * the up projection's GEMM epilogue where the tiling allows.) */
int activation_forward(void *h, const void *up, int R, int H, int mlp, int dtype, void *stream);
int activation_backward(void *dup, const void *dh, const void *up, int R, int H, int mlp, int dtype,
                        void *stream);

/* lm_head_forward: logits[R, :V] = inp[R, C] W[V, C]^T ("nanoeuler — CUDA
 *   kernels" forward_gpu's head matmul; llm.c gpt2_forward, where W is wte when
 *   the head is tied).  logits rows have stride ldl >= V, ldl a multiple of 8
 *   (llm.c pads the vocabulary the same way); columns V..ldl-1 are not part
 *   of the result (unspecified on return; softmax_ce never reads them).
 * lm_head_backward: dinp[R, C] = dlogits[:, :V] W (OVERWRITTEN);
 *   dw[V, C] += dlogits[:, :V]^T inp (fp32, ACCUMULATED).  dlogits' padded
 *   columns must hold zeros (softmax_ce writes them so).  dinp or dw may be
 *   NULL.  workspace lm_head_workspace_bytes(R, C, V, dtype) bytes. */
int lm_head_forward(void *logits, int ldl, const void *inp, const void *w, int R, int C, int V, int dtype,
                    void *stream);
int lm_head_backward(void *dinp, float *dw, const void *dlogits, int ldl, const void *inp, const void *w, int R,
                     int C, int V, int dtype, void *workspace, void *stream);
size_t lm_head_workspace_bytes(int R, int C, int V, int dtype);

/* softmax_ce: softmax cross-entropy of R rows of logits [R, ldl] (V valid
 * columns) against targets [R] ("nanoeuler — CUDA kernels" softmax_ce_kernel
 * with one head; llm.c crossentropy_forward / crossentropy_softmax_backward):
 *   lse_r = max + ln sum_v exp(l_rv - max);  row_loss[r] = lse_r - l_r,target
 *   dlogits[r, v] = scale * (exp(l_rv - lse_r) - [v == target_r]),  v < V
 *   loss[0] = scale * sum_r row_loss[r]   (fixed-order reduction)
 * A target outside [0, V) (e.g. -1, a masked position) gives row_loss 0 and a
 * zero gradient row.  dlogits [R, ldl] dtype is OVERWRITTEN, its padded columns
 * with zeros, and may alias logits.  row_loss [R] and loss [1] fp32,
 * OVERWRITTEN.  Probabilities are not stored. */
int softmax_ce(float *loss, float *row_loss, void *dlogits, const void *logits, int ldl, const int *targets, int R,
               int V, float scale, int dtype, void *stream);

/* lm_head_ce: the LM head and the softmax cross-entropy fused and chunked over
 * the vocabulary, forward and backward in one call: the logits of the whole
 * vocabulary never exist at once, nor do probabilities.  Chunks of vchunk
 * vocabulary rows (a multiple of 256; 0 = 4096): pass 1 computes each chunk's
 * logits = inp W_chunk^T and folds them into running per-row max / sum of exp
 * (catching the target logit); pass 2 recomputes each chunk, forms
 * dlogits = scale (exp(l - lse) - onehot) in place and applies it:
 *   dinp[R, C] = sum over chunks of dlogits W_chunk   (dtype, OVERWRITTEN)
 *   dw[V, C]  += dlogits^T inp                         (fp32, ACCUMULATED)
 * loss, row_loss as softmax_ce (targets outside [0, V) masked).  dinp or dw
 * may be NULL (both NULL: loss only, one pass).  inp [R, C], w [V, C]: dtype.
 * Cost against lm_head_forward + softmax_ce + lm_head_backward: one more
 * GEMM of the head's forward size, for a workspace of R * vchunk logits
 * instead of R * V.  workspace: lm_head_ce_workspace_bytes(R, C, V, vchunk, dtype). */
int lm_head_ce(float *loss, float *row_loss, void *dinp, float *dw, const void *inp, const void *w, const int *targets,
               int R, int C, int V, int vchunk, float scale, int dtype, void *workspace, void *stream);
size_t lm_head_ce_workspace_bytes(int R, int C, int V, int vchunk, int dtype);

/* lm_head_mtp_ce: lm_head_ce with K prediction heads ("nanoeuler — CUDA
 * kernels": the head GEMM with K*V output columns and softmax_ce_kernel over
 * every (position, head) row; its batches give head j at position t the token
 * t+1+j as target, and supervised fine-tuning masks targets with -1):
 *   w [K*V, C] dtype, head j = rows j*V .. j*V+V-1
 *   targets [R][K] int32 (outside [0, V): masked), row_loss [R][K] fp32
 *   loss[0] = scale * sum over (r, j) of row_loss   (1/(R K) for pretraining,
 *             1/(number of unmasked targets) for fine-tuning)
 *   dinp [R, C] = sum over heads of dlogits_j W_j   (dtype, OVERWRITTEN)
 *   dw [K*V, C] += dlogits_j^T inp per head         (fp32, ACCUMULATED)
 * The heads run one after another through the same workspace, so
 * lm_head_ce_workspace_bytes(R, C, V, vchunk, dtype) sizes it for any K.
 * K = 1 is lm_head_ce. */
int lm_head_mtp_ce(float *loss, float *row_loss, void *dinp, float *dw, const void *inp, const void *w,
                   const int *targets, int R, int C, int V, int K, int vchunk, float scale, int dtype,
                   void *workspace, void *stream);

/* ---- optimizer ----------------------------------------------------------------
 * adamw_update: one AdamW step over a flat buffer of n parameters ("nanoeuler —
 * CUDA kernels" adamw_kernel; llm.c gpt2_update; microgpt adam_update_param):
 *   m = beta1 m + (1 - beta1) g;  v = beta2 v + (1 - beta2) g^2
 *   p -= lr (m / (1 - beta1^step) / (sqrt(v / (1 - beta2^step)) + eps) + weight_decay p)
 * params (the fp32 master values), grads, m, v: fp32 [n], updated in place
 * (grads only read, then set to zero when zero_grads != 0, ready for the next
 * accumulation).  params_lowp: NULL, or [n] of lowp_dtype (DTB_BF16 only)
 * receiving the rounded parameters (the storage copy the kernels read).
 * step >= 1 is the 1-based step number; 0 <= beta < 1.  Any n >= 0. */
int adamw_update(float *params, float *grads, float *m, float *v, void *params_lowp, long long n, float lr,
                 float beta1, float beta2, float eps, float weight_decay, int step, int lowp_dtype, int zero_grads,
                 void *stream);

/* ---- misc ---------------------------------------------------------------- */
const char *dtb_strerror(int code);
const char *dtb_version(void);

/* Opt-in debugging, in the spirit of the CHECK_CUDA discipline of "nanoeuler —
 * CUDA kernels" (every call checked): level 1 makes the library check each
 * kernel launch and wait for its stream right after it, so a failing kernel
 * is caught at once; the entry point that launched it returns DTB_ELAUNCH and
 * dtb_strerror names that kernel.  Level 2 also prints one line per kernel to
 * stderr as it completes.  0 (the default) turns it off.  Process-wide; it
 * slows every call and must not be on under graph capture.  A level outside
 * 0..2 gives DTB_EINVAL_ENUM. */
int dtb_debug_enable(int level);

/* Optional per-kernel timing for measurement: while enabled, every kernel the
 * library enqueues in an enabled class carries HIP start / stop events on its
 * own dispatch packet (hipExtLaunchKernelGGL, so no marker packets are added
 * between kernels), grouped by kernel
 * class (0 forward-projection GEMMs, 1 attn_fwd, 2 attn_bwd, 3 elementwise,
 * 4 input-gradient GEMMs, 5 weight-gradient GEMMs, 6 the decode-attention
 * kernel, 7 its chunk merge), together with the algorithmic flops / bytes of
 * each launch (0 for the decode-attention kernel, whose bytes depend on the
 * cache lengths in device memory).  dtb_timing_collect() waits for
 * the recorded events, adds the elapsed times to the running totals and
 * returns the number of classes filled (at most max_classes).  Not for use
 * under graph capture. */
typedef struct {
    double ms;          /* summed kernel time */
    double flops;       /* summed algorithmic flops */
    double bytes;       /* summed algorithmic HBM bytes */
    long long launches; /* number of launches */
} dtb_timing;
/* class_mask: bit c enables class c; a negative value enables every class,
 * 0 disables timing. */
int dtb_timing_enable(int class_mask);
int dtb_timing_collect(dtb_timing *out, int max_classes);

#ifdef __cplusplus
}
#endif
#endif
