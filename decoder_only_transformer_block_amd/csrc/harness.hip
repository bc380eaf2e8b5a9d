// Model harness around the block stack: token / position embedding and its
// backward, and the softmax cross-entropy of the LM head (forward and
// backward in one pass pair), with a deterministic mean-loss reduction.
//
// Sources (page title, section):
//   "nanoeuler — CUDA kernels": encoder_forward_kernel (a row of the token
//     table per position), encoder_backward_kernel (atomic scatter-add into
//     the table, ids repeat), softmax_ce_kernel (max, sum of exp, normalised
//     probabilities, dlogits = (p - onehot) * scale, a negative target masks
//     the row).
//   "microgpt.cu": forward_position (token row + position row).
//   llm.c train_gpt2.c: encoder_forward / encoder_backward (wte and wpe),
//     crossentropy_forward / crossentropy_softmax_backward (vocabulary rows
//     padded to a wider stride, padded columns not part of the softmax).
//
// Design: one wave64 per embedding row with 16-byte vectors; one 256-thread
// workgroup per logits row for the cross-entropy (an online max / sum pass,
// then the gradient pass; probabilities are never stored, and the gradient may
// overwrite the logits in place).  The position-table gradient sums the B
// sequences in order; the token-table gradient uses fp32 atomics (repeated ids
// add in an unspecified order).
#include <math.h>

#include "common.h"

namespace dtb {

// x[bt, :] = wte[ids[bt], :] (+ wpe[bt % T, :]); an id outside [0, V) gives wpe only
template <typename T>
__global__ __launch_bounds__(256) void embed_fwd_kernel(const int *ids, const T *wte, const T *wpe, long BT, int Tn,
                                                        int C, int V, T *x) {
    constexpr int EPC = 16 / sizeof(T);
    const long row = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= BT) return;
    const int lane = threadIdx.x & 63;
    const int id = ids[row];
    const bool ok = id >= 0 && id < V;
    const long t = row % Tn;
    const int nch = C / EPC;
    for (int c = lane; c < nch; c += 64) {
        float a[EPC], b[EPC];
        if (ok) {
            unpack16<T>(ld16(wte + (long)id * C + c * EPC), a);
        } else {
#pragma unroll
            for (int e = 0; e < EPC; e++) a[e] = 0.f;
        }
        if (wpe) {
            unpack16<T>(ld16(wpe + t * C + c * EPC), b);
#pragma unroll
            for (int e = 0; e < EPC; e++) a[e] += b[e];
        }
        st16(x + row * C + c * EPC, pack16<T>(a));
    }
}

// dwte[ids[bt], :] += dx[bt, :]   (fp32 atomics; ids outside [0, V) skipped)
template <typename T>
__global__ __launch_bounds__(256) void embed_bwd_kernel(const int *ids, const T *dx, long BT, int C, int V,
                                                        float *dwte) {
    constexpr int EPC = 16 / sizeof(T);
    const long row = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= BT) return;
    const int lane = threadIdx.x & 63;
    const int id = ids[row];
    if (id < 0 || id >= V) return;
    const int nch = C / EPC;
    float *dst = dwte + (long)id * C;
    for (int c = lane; c < nch; c += 64) {
        float d[EPC];
        unpack16<T>(ld16(dx + row * C + c * EPC), d);
#pragma unroll
        for (int e = 0; e < EPC; e++) unsafeAtomicAdd(dst + c * EPC + e, d[e]);
    }
}

// dwpe[t, c] += sum_b dx[b, t, c]   (b in order)
template <typename T>
__global__ __launch_bounds__(256) void embed_pos_bwd_kernel(const T *dx, int B, int Tn, int C, float *dwpe) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)Tn * C) return;
    float s = 0.f;
    for (int b = 0; b < B; b++) s += to_f32(dx[(long)b * Tn * C + i]);
    dwpe[i] += s;
}

// ---- softmax cross-entropy --------------------------------------------------
// combine two (max, sum-of-exp relative to that max) pairs
__device__ __forceinline__ void lse_merge(float &m, float &s, float m2, float s2) {
    const float M = fmaxf(m, m2);
    if (M == -INFINITY) {
        s = 0.f;
    } else {
        s = s * __expf(m - M) + s2 * __expf(m2 - M);
    }
    m = M;
}

// One workgroup per row r of logits [R, ldl] (V valid columns):
//   lse = max + ln sum exp(l - max);  row_loss[r] = lse - l[target]
//   dlogits[r, v] = scale * (exp(l_v - lse) - [v == target]) for v < V, 0 for
//   the padded columns V <= v < ldl.  target < 0: row_loss 0, zero gradient.
// dlogits may alias logits (each vector is read before the same thread writes it).
template <typename T>
__global__ __launch_bounds__(256) void softmax_xent_kernel(const T *logits, long ldl, const int *targets, int V,
                                                           float scale, float *row_loss, T *dlogits) {
    constexpr int EPC = 16 / sizeof(T);
    const long r = blockIdx.x;
    const T *l = logits + r * ldl;
    T *dl = dlogits + r * ldl;
    const int tg = targets[r];
    const int nv = (V + EPC - 1) / EPC;  // vectors holding valid columns
    const int nvl = (int)(ldl / EPC);    // vectors of the padded row
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ float sm[4], ss[4];
    if (tg < 0 || tg >= V) {  // masked row
        float z[EPC];
#pragma unroll
        for (int e = 0; e < EPC; e++) z[e] = 0.f;
        for (int c = tid; c < nvl; c += 256) st16(dl + c * EPC, pack16<T>(z));
        if (tid == 0) row_loss[r] = 0.f;
        return;
    }
    // pass 1: running max and sum of exp
    float m = -INFINITY, s = 0.f;
    for (int c = tid; c < nv; c += 256) {
        float v[EPC];
        unpack16<T>(ld16(l + c * EPC), v);
        float mv = -INFINITY;
#pragma unroll
        for (int e = 0; e < EPC; e++)
            if (c * EPC + e < V) mv = fmaxf(mv, v[e]);
        if (mv > m) {
            s = (m == -INFINITY) ? 0.f : s * __expf(m - mv);
            m = mv;
        }
#pragma unroll
        for (int e = 0; e < EPC; e++)
            if (c * EPC + e < V) s += __expf(v[e] - m);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
        lse_merge(m, s, m2, s2);
    }
    if (lane == 0) {
        sm[wave] = m;
        ss[wave] = s;
    }
    __syncthreads();
    m = sm[0];
    s = ss[0];
#pragma unroll
    for (int w = 1; w < 4; w++) lse_merge(m, s, sm[w], ss[w]);
    const float lse = m + logf(s);
    if (tid == 0) row_loss[r] = lse - to_f32(l[tg]);
    // pass 2: the gradient (and zeros in the padded columns)
    for (int c = tid; c < nvl; c += 256) {
        float v[EPC], o[EPC];
        if (c < nv) unpack16<T>(ld16(l + c * EPC), v);
#pragma unroll
        for (int e = 0; e < EPC; e++) {
            const int idx = c * EPC + e;
            o[e] = (c < nv && idx < V) ? scale * (__expf(v[e] - lse) - (idx == tg ? 1.f : 0.f)) : 0.f;
        }
        st16(dl + c * EPC, pack16<T>(o));
    }
}

// loss = scale * sum_r row_loss[r], one workgroup, fixed order (double sums)
__global__ __launch_bounds__(256) void loss_sum_kernel(const float *rows, long R, float scale, float *loss) {
    __shared__ double part[256];
    double acc = 0.0;
    for (long i = threadIdx.x; i < R; i += 256) acc += rows[i];
    part[threadIdx.x] = acc;
    __syncthreads();
    for (int w = 128; w >= 1; w >>= 1) {
        if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
        __syncthreads();
    }
    if (threadIdx.x == 0) loss[0] = (float)(scale * part[0]);
}

// ---- vocabulary-chunked cross-entropy ------------------------------------------
// The head's logits are produced chunk by chunk ([R, ldc] for vocabulary
// columns v0 .. v0+vc-1) and never exist for the whole vocabulary at once.
// Pass 1 folds each chunk into running per-row (max, sum of exp) and catches
// the target logit; pass 2 recomputes each chunk and turns it into the scaled
// gradient in place.

// pass 1: one workgroup per row
template <typename T>
__global__ __launch_bounds__(256) void ce_chunk_stats_kernel(const T *lg, long ldc, int vc, int v0, const int *targets,
                                                             int ts, float *rm, float *rs, float *tl, int first) {
    constexpr int EPC = 16 / sizeof(T);
    const long r = blockIdx.x;
    const T *l = lg + r * ldc;
    const int nv = (vc + EPC - 1) / EPC;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    __shared__ float sm[4], ss[4];
    float m = -INFINITY, s = 0.f;
    for (int c = tid; c < nv; c += 256) {
        float v[EPC];
        unpack16<T>(ld16(l + c * EPC), v);
        float mv = -INFINITY;
#pragma unroll
        for (int e = 0; e < EPC; e++)
            if (c * EPC + e < vc) mv = fmaxf(mv, v[e]);
        if (mv > m) {
            s = (m == -INFINITY) ? 0.f : s * __expf(m - mv);
            m = mv;
        }
#pragma unroll
        for (int e = 0; e < EPC; e++)
            if (c * EPC + e < vc) s += __expf(v[e] - m);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        const float m2 = __shfl_xor(m, o, 64), s2 = __shfl_xor(s, o, 64);
        lse_merge(m, s, m2, s2);
    }
    if (lane == 0) {
        sm[wave] = m;
        ss[wave] = s;
    }
    __syncthreads();
    if (tid == 0) {
        m = sm[0];
        s = ss[0];
#pragma unroll
        for (int w = 1; w < 4; w++) lse_merge(m, s, sm[w], ss[w]);
        if (!first) lse_merge(m, s, rm[r], rs[r]);
        rm[r] = m;
        rs[r] = s;
        const int tg = targets[r * ts];
        if (tg >= v0 && tg < v0 + vc) tl[r] = to_f32(l[tg - v0]);
    }
}

// after pass 1: lse (+inf for a masked row, so its gradient comes out zero)
// and the row losses (targets and row losses at stride ts: one prediction
// head of several)
__global__ __launch_bounds__(256) void ce_finish_kernel(const float *rm, const float *rs, const float *tl,
                                                        const int *targets, int ts, long R, int V, float *lse,
                                                        float *row_loss) {
    const long r = (long)blockIdx.x * 256 + threadIdx.x;
    if (r >= R) return;
    const int tg = targets[r * ts];
    const bool masked = tg < 0 || tg >= V;
    const float l = rm[r] + logf(rs[r]);
    lse[r] = masked ? INFINITY : l;
    row_loss[r * ts] = masked ? 0.f : l - tl[r];
}

// pass 2: the chunk's logits become scale * (exp(l - lse) - onehot) in place,
// zeros in the padded columns; one workgroup per row
template <typename T>
__global__ __launch_bounds__(256) void ce_chunk_grad_kernel(T *lg, long ldc, int vc, int v0, const int *targets,
                                                            int ts, const float *lse, float scale) {
    constexpr int EPC = 16 / sizeof(T);
    const long r = blockIdx.x;
    T *l = lg + r * ldc;
    const float ls = lse[r];
    const int tg = targets[r * ts] - v0;
    const int nvl = (int)(ldc / EPC);
    for (int c = threadIdx.x; c < nvl; c += 256) {
        float v[EPC], o[EPC];
        unpack16<T>(ld16(l + c * EPC), v);
#pragma unroll
        for (int e = 0; e < EPC; e++) {
            const int idx = c * EPC + e;
            o[e] = idx < vc ? scale * (__expf(v[e] - ls) - (idx == tg ? 1.f : 0.f)) : 0.f;
        }
        st16(l + c * EPC, pack16<T>(o));
    }
}

// x = 0 (fp32) / out = in (fp32 -> dtype), 4 elements per thread (n % 4 == 0)
__global__ __launch_bounds__(256) void zero4_kernel(float *x, long long n4) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i < n4) reinterpret_cast<f32x4 *>(x)[i] = f32x4{0.f, 0.f, 0.f, 0.f};
}
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float *in, bf16 *out, long long n4) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const f32x4 v = reinterpret_cast<const f32x4 *>(in)[i];
    reinterpret_cast<u32x2 *>(out)[i] = u32x2{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
}

// ---- AdamW over a flat parameter buffer --------------------------------------
// ("nanoeuler — CUDA kernels" adamw_kernel; llm.c gpt2_update.)  fp32 master
// p, gradient g, moments m and v; optionally the bf16 storage copy of p and the
// gradient cleared for the next accumulation.  ic1 = 1 / (1 - b1^t),
// ic2 = 1 / (1 - b2^t).  16-byte vectors for the first 4*n4 elements, one
// element per thread for the tail.  Nothing is reused, so every access is
// non-temporal, and the grid covers the buffer (a capped grid-stride loop and
// cached accesses measured 4.5 instead of 5.9 TB/s).
struct AdamArgs {
    float *p, *g, *m, *v;
    bf16 *lowp;
    long long n;
    float lr, b1, b2, eps, wd, ic1, ic2;
    int zero_g;
};
__device__ __forceinline__ void adam_one(float &p, float g, float &m, float &v, const AdamArgs &a) {
    m = a.b1 * m + (1.f - a.b1) * g;
    v = a.b2 * v + (1.f - a.b2) * g * g;
    const float mh = m * a.ic1, vh = v * a.ic2;
    p -= a.lr * (mh / (sqrtf(vh) + a.eps) + a.wd * p);
}
__global__ __launch_bounds__(256) void adamw_kernel(AdamArgs a) {
    const long long n4 = a.n / 4, stride = (long long)gridDim.x * 256;
    const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
    for (long long i = tid; i < n4; i += stride) {
        f32x4 p = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.p) + i);
        f32x4 g = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.g) + i);
        f32x4 m = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.m) + i);
        f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(a.v) + i);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            float pe = p[e], me = m[e], ve = v[e];
            adam_one(pe, g[e], me, ve, a);
            p[e] = pe;
            m[e] = me;
            v[e] = ve;
        }
        __builtin_nontemporal_store(p, reinterpret_cast<f32x4 *>(a.p) + i);
        __builtin_nontemporal_store(m, reinterpret_cast<f32x4 *>(a.m) + i);
        __builtin_nontemporal_store(v, reinterpret_cast<f32x4 *>(a.v) + i);
        if (a.lowp) __builtin_nontemporal_store(u32x2{pack2_bf16(p[0], p[1]), pack2_bf16(p[2], p[3])}, reinterpret_cast<u32x2 *>(a.lowp) + i);
        if (a.zero_g) __builtin_nontemporal_store(f32x4{0.f, 0.f, 0.f, 0.f}, reinterpret_cast<f32x4 *>(a.g) + i);
    }
    const long long j = 4 * n4 + tid;  // tail
    if (j < a.n) {
        float p = a.p[j], m = a.m[j], v = a.v[j];
        adam_one(p, a.g[j], m, v, a);
        a.p[j] = p;
        a.m[j] = m;
        a.v[j] = v;
        if (a.lowp) a.lowp[j] = (bf16)p;
        if (a.zero_g) a.g[j] = 0.f;
    }
}

// ---- host side ----------------------------------------------------------------
int embed_fwd(int dtype, const int *ids, const void *wte, const void *wpe, long BT, int Tn, int C, int V, void *x,
              hipStream_t s) {
    if (BT <= 0) return DTB_OK;
    if (g_timing_on) timing_begin(s, K_ELEM);
    dim3 grid((unsigned)((BT + 3) / 4));
    if (dtype == DTB_BF16)
        DTB_LAUNCH(embed_fwd_kernel<bf16>, grid, dim3(256), 0, s, ids, (const bf16 *)wte, (const bf16 *)wpe,
                           BT, Tn, C, V, (bf16 *)x);
    else
        DTB_LAUNCH(embed_fwd_kernel<float>, grid, dim3(256), 0, s, ids, (const float *)wte,
                           (const float *)wpe, BT, Tn, C, V, (float *)x);
    DTB_LAUNCH_CHECK("encoder_forward");
    if (g_timing_on) {
        const double es = dtype == DTB_BF16 ? 2 : 4;
        timing_end(s, K_ELEM, 0, (double)BT * (4 + es * C * (wpe ? 3 : 2)));
    }
    return DTB_OK;
}

int embed_bwd(int dtype, const int *ids, const void *dx, int B, int Tn, int C, int V, float *dwte, float *dwpe,
              hipStream_t s) {
    const long BT = (long)B * Tn;
    if (BT <= 0) return DTB_OK;
    if (g_timing_on) timing_begin(s, K_ELEM);
    if (dwte) {
        dim3 grid((unsigned)((BT + 3) / 4));
        if (dtype == DTB_BF16)
            DTB_LAUNCH(embed_bwd_kernel<bf16>, grid, dim3(256), 0, s, ids, (const bf16 *)dx, BT, C, V, dwte);
        else
            DTB_LAUNCH(embed_bwd_kernel<float>, grid, dim3(256), 0, s, ids, (const float *)dx, BT, C, V,
                               dwte);
        DTB_LAUNCH_CHECK("encoder_backward");
    }
    if (dwpe) {
        dim3 grid((unsigned)(((long)Tn * C + 255) / 256));
        if (dtype == DTB_BF16)
            DTB_LAUNCH(embed_pos_bwd_kernel<bf16>, grid, dim3(256), 0, s, (const bf16 *)dx, B, Tn, C, dwpe);
        else
            DTB_LAUNCH(embed_pos_bwd_kernel<float>, grid, dim3(256), 0, s, (const float *)dx, B, Tn, C,
                               dwpe);
        DTB_LAUNCH_CHECK("encoder_backward (positions)");
    }
    if (g_timing_on) {
        const double es = dtype == DTB_BF16 ? 2 : 4;
        timing_end(s, K_ELEM, 0, (double)BT * C * (es + (dwte ? 8 : 0)) + (dwpe ? 8.0 * Tn * C : 0));
    }
    return DTB_OK;
}

int softmax_xent_rows(int dtype, const void *logits, long ldl, const int *targets, long R, int V, float scale,
                      float *row_loss, void *dlogits, float *loss, hipStream_t s) {
    if (g_timing_on) timing_begin(s, K_ELEM);
    if (R > 0) {
        if (dtype == DTB_BF16)
            DTB_LAUNCH(softmax_xent_kernel<bf16>, dim3((unsigned)R), dim3(256), 0, s, (const bf16 *)logits,
                               ldl, targets, V, scale, row_loss, (bf16 *)dlogits);
        else
            DTB_LAUNCH(softmax_xent_kernel<float>, dim3((unsigned)R), dim3(256), 0, s,
                               (const float *)logits, ldl, targets, V, scale, row_loss, (float *)dlogits);
        DTB_LAUNCH_CHECK("softmax_ce");
    }
    DTB_LAUNCH(loss_sum_kernel, dim3(1), dim3(256), 0, s, row_loss, R, scale, loss);
    DTB_LAUNCH_CHECK("softmax_ce loss");
    if (g_timing_on) {
        const double es = dtype == DTB_BF16 ? 2 : 4;
        timing_end(s, K_ELEM, 0, (double)R * (3.0 * es * ldl + 12));
    }
    return DTB_OK;
}

// ---- chunked head + cross-entropy: orchestration -------------------------------
static size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t head_ce_ws_bytes(int R, int C, int V, int vc, int dtype) {
    const size_t es = dtype == DTB_BF16 ? 2 : 4;
    const size_t ldc = ((size_t)vc + 7) / 8 * 8;
    size_t g1 = gemm_ws_bytes(vc, C, R, dtype), g2 = gemm_ws_bytes(R, C, vc, dtype);
    return al256((size_t)R * ldc * es) + 5 * al256((size_t)R * 4) + (dtype == DTB_BF16 ? al256((size_t)R * C * 4) : 0) +
           al256(g1 > g2 ? g1 : g2) + 256;
}

int head_ce(float *loss, float *row_loss, void *dinp, float *dw, const void *inp, const void *w, const int *targets,
            int R, int C, int V, int K, int vc, float scale, int dtype, void *workspace, hipStream_t s) {
    const size_t es = dtype == DTB_BF16 ? 2 : 4;
    const long ldc = ((long)vc + 7) / 8 * 8;
    char *ws = static_cast<char *>(workspace);
    void *chunk = ws;
    ws += al256((size_t)R * ldc * es);
    float *rm = reinterpret_cast<float *>(ws); ws += al256((size_t)R * 4);
    float *rs = reinterpret_cast<float *>(ws); ws += al256((size_t)R * 4);
    float *tl = reinterpret_cast<float *>(ws); ws += al256((size_t)R * 4);
    float *lse = reinterpret_cast<float *>(ws); ws += al256((size_t)R * 4);
    ws += al256((size_t)R * 4);
    float *dacc = nullptr;
    if (dinp) dacc = dtype == DTB_BF16 ? reinterpret_cast<float *>(ws) : reinterpret_cast<float *>(dinp);
    if (dtype == DTB_BF16) ws += al256((size_t)R * C * 4);
    void *gws = ws;
    size_t g1 = gemm_ws_bytes(vc, C, R, dtype), g2 = gemm_ws_bytes(R, C, vc, dtype);
    const size_t gws_bytes = g1 > g2 ? g1 : g2;
    if (R <= 0) {  // no rows: the loss is zero
        DTB_LAUNCH(loss_sum_kernel, dim3(1), dim3(256), 0, s, row_loss, 0L, scale, loss);
        DTB_LAUNCH_CHECK("lm_head_ce loss");
        return DTB_OK;
    }
    const bool grads = dinp || dw;
    if (dacc) {
        const long long n4 = (long long)R * C / 4;
        DTB_LAUNCH(zero4_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, dacc, n4);
        DTB_LAUNCH_CHECK("lm_head_ce zero");
    }
    // head j: vocabulary rows j*V .. j*V+V-1 of w, targets[r*K + j], row_loss[r*K + j]
    for (int j = 0; j < K; j++) {
        const long long w0 = (long long)j * V;
        const int *tj = targets + j;
        auto wchunk = [&](int v0) -> const void * {
            const long long off = (w0 + v0) * C;
            return dtype == DTB_BF16 ? static_cast<const void *>(static_cast<const bf16 *>(w) + off)
                                     : static_cast<const void *>(static_cast<const float *>(w) + off);
        };
        auto logits = [&](int v0, int n) {
            GemmArgs g{};
            g.dtype = dtype;
            g.a_kmajor = g.b_kmajor = true;
            g.A = inp; g.lda = C; g.B = wchunk(v0); g.ldb = C; g.M = R; g.N = n; g.K = C;
            g.out = chunk; g.ldo = ldc;
            return gemm(g, nullptr, 0, s);
        };
        // pass 1: running max / sum of exp over the head's vocabulary chunks
        for (int v0 = 0, i = 0; v0 < V; v0 += vc, i++) {
            const int n = V - v0 < vc ? V - v0 : vc;
            int r = logits(v0, n);
            if (r) return r;
            if (dtype == DTB_BF16)
                DTB_LAUNCH(ce_chunk_stats_kernel<bf16>, dim3((unsigned)R), dim3(256), 0, s, (const bf16 *)chunk,
                                   ldc, n, v0, tj, K, rm, rs, tl, i == 0);
            else
                DTB_LAUNCH(ce_chunk_stats_kernel<float>, dim3((unsigned)R), dim3(256), 0, s,
                                   (const float *)chunk, ldc, n, v0, tj, K, rm, rs, tl, i == 0);
            DTB_LAUNCH_CHECK("lm_head_ce stats");
        }
        DTB_LAUNCH(ce_finish_kernel, dim3((unsigned)((R + 255) / 256)), dim3(256), 0, s, rm, rs, tl, tj, K,
                           (long)R, V, lse, row_loss + j);
        DTB_LAUNCH_CHECK("lm_head_ce finish");
        if (!grads) continue;
        // pass 2: recompute each chunk, turn it into the gradient, apply it
        for (int v0 = 0; v0 < V; v0 += vc) {
            const int n = V - v0 < vc ? V - v0 : vc;
            int r = logits(v0, n);
            if (r) return r;
            if (dtype == DTB_BF16)
                DTB_LAUNCH(ce_chunk_grad_kernel<bf16>, dim3((unsigned)R), dim3(256), 0, s, (bf16 *)chunk, ldc,
                                   n, v0, tj, K, lse, scale);
            else
                DTB_LAUNCH(ce_chunk_grad_kernel<float>, dim3((unsigned)R), dim3(256), 0, s, (float *)chunk,
                                   ldc, n, v0, tj, K, lse, scale);
            DTB_LAUNCH_CHECK("lm_head_ce gradient");
            if (dacc) {  // dinp += dlogits_chunk W_chunk
                GemmArgs g{};
                g.dtype = dtype;
                g.a_kmajor = true;
                g.b_kmajor = false;
                g.A = chunk; g.lda = ldc; g.B = wchunk(v0); g.ldb = C; g.M = R; g.N = C; g.K = n;
                g.out = dacc; g.ldo = C; g.out_f32 = g.accumulate = true;
                r = gemm(g, gws, gws_bytes, s);
                if (r) return r;
            }
            if (dw) {  // dw[j*V + v0 ..) += dlogits_chunk^T inp
                GemmArgs g{};
                g.dtype = dtype;
                g.a_kmajor = g.b_kmajor = false;
                g.A = chunk; g.lda = ldc; g.B = inp; g.ldb = C; g.M = n; g.N = C; g.K = R;
                g.out = dw + (w0 + v0) * C; g.ldo = C; g.out_f32 = g.accumulate = true;
                r = gemm(g, gws, gws_bytes, s);
                if (r) return r;
            }
        }
    }
    DTB_LAUNCH(loss_sum_kernel, dim3(1), dim3(256), 0, s, row_loss, (long)R * K, scale, loss);
    DTB_LAUNCH_CHECK("lm_head_ce loss");
    if (dinp && dtype == DTB_BF16) {
        const long long n4 = (long long)R * C / 4;
        DTB_LAUNCH(f32_to_bf16_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, dacc,
                           (bf16 *)dinp, n4);
        DTB_LAUNCH_CHECK("lm_head_ce convert");
    }
    return DTB_OK;
}

int adamw(float *p, float *g, float *m, float *v, void *lowp, long long n, float lr, float b1, float b2, float eps,
          float wd, int t, int zero_g, hipStream_t s) {
    if (n <= 0) return DTB_OK;
    AdamArgs a{};
    a.p = p; a.g = g; a.m = m; a.v = v;
    a.lowp = reinterpret_cast<bf16 *>(lowp);
    a.n = n;
    a.lr = lr; a.b1 = b1; a.b2 = b2; a.eps = eps; a.wd = wd;
    a.ic1 = (float)(1.0 / (1.0 - pow((double)b1, t)));
    a.ic2 = (float)(1.0 / (1.0 - pow((double)b2, t)));
    a.zero_g = zero_g;
    const long long n4 = n / 4;
    long long blocks = (n4 + 255) / 256;
    if (blocks > (1LL << 20)) blocks = 1LL << 20;
    if (blocks < 1) blocks = 1;
    if (g_timing_on) timing_begin(s, K_ELEM);
    DTB_LAUNCH(adamw_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    DTB_LAUNCH_CHECK("adamw_update");
    if (g_timing_on) timing_end(s, K_ELEM, 0, (double)n * (28 + (lowp ? 2 : 0) + (zero_g ? 4 : 0)));
    return DTB_OK;
}

}  // namespace dtb
