// Bandwidth-bound kernels of the block: RMSNorm / LayerNorm forward and
// backward, NeoX RoPE, the MLP activations and the bias-gradient reductions.
//
// Sources (page title, section):
//   "nanoeuler — CUDA kernels": rmsnorm_forward_kernel / rmsnorm_backward_kernel
//     (r = (mean x^2 + eps)^-1/2; dx += g dy r - x (sum dy g x) r^3 / C),
//     swiglu_forward_kernel / swiglu_backward_kernel, residual_add_kernel.
//   "microgpt.cu": RMSNorm without gamma, relu_forward/backward_kernel.
//   llm.c train_gpt2.c: layernorm_forward / layernorm_backward, gelu_forward /
//     gelu_backward (tanh approximation), matmul_backward's bias gradient.
//   "nx_f32_qwen2_train_gate.nx source": build_rope (NeoX half-split pairs,
//     theta_i = base^(-2i/hd)).
//
// Layout and design: one wave64 per row for the norms, 16-byte vector loads
// and stores, the row held in registers between the reduction and the write;
// gamma/beta/bias gradients are reduced deterministically (per-workgroup
// partial sums in fp32, then a second kernel adds them into the gradient).
#include <type_traits>

#include "common.h"

namespace dtb {

// ---------------------------------------------------------------- norms ---
// NPL: 16-byte chunks per lane (row width C <= 64 * NPL * EPC)
template <typename T, int NPL, int MODE>
__global__ __launch_bounds__(256) void norm_fwd_kernel(const T *x, const T *g, const T *bta, float eps, long R,
                                                        int C, T *out, float *rstd, float *mean) {
    constexpr int EPC = 16 / sizeof(T);
    const long row = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= R) return;
    const int nch = C / EPC;
    const Buf bx(x + row * C);
    float v[NPL][EPC];
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < NPL; k++) {
        int c = lane + 64 * k;
        unpack16<T>(bx.ld16(c * 16, c < nch), v[k]);
#pragma unroll
        for (int e = 0; e < EPC; e++) s += (MODE == DTB_NORM_LAYER) ? v[k][e] : v[k][e] * v[k][e];
    }
    float mu = 0.f, ms;
    if (MODE == DTB_NORM_LAYER) {
        mu = wave_sum(s) / C;
        float q = 0.f;
#pragma unroll
        for (int k = 0; k < NPL; k++) {
            int c = lane + 64 * k;
            if (c < nch)
#pragma unroll
                for (int e = 0; e < EPC; e++) {
                    float d = v[k][e] - mu;
                    q += d * d;
                }
        }
        ms = wave_sum(q) / C;
    } else {
        ms = wave_sum(s) / C;
    }
    const float r = rsqrtf(ms + eps);
    T *orow = out + row * C;
#pragma unroll
    for (int k = 0; k < NPL; k++) {
        int c = lane + 64 * k;
        if (c >= nch) continue;
        float gv[EPC], bv[EPC], o[EPC];
        if (MODE != DTB_NORM_RMS_NOGAMMA) unpack16<T>(ld16(g + c * EPC), gv);
        if (MODE == DTB_NORM_LAYER) unpack16<T>(ld16(bta + c * EPC), bv);
#pragma unroll
        for (int e = 0; e < EPC; e++) {
            float n = (v[k][e] - mu) * r;
            if (MODE != DTB_NORM_RMS_NOGAMMA) n *= gv[e];
            if (MODE == DTB_NORM_LAYER) n += bv[e];
            o[e] = n;
        }
        st16(orow + c * EPC, pack16<T>(o));
    }
    if (lane == 0) {
        rstd[row] = r;
        if (MODE == DTB_NORM_LAYER) mean[row] = mu;
    }
}

// Row statistics of the norm backward for rows too wide to hold in a wave's
// registers: st[2 row] = mean over the row of dn (LayerNorm; 0 otherwise),
// st[2 row + 1] = mean of dn xhat, with dn = dy gamma and xhat the normalised
// input.  One wave per row streams it in 16-byte chunks; each lane adds its
// chunks in the order the register-resident kernel does.
template <typename T, int MODE>
__global__ __launch_bounds__(256) void norm_bwd_stats_kernel(const T *dy, const T *x, const T *g, const float *rstd,
                                                              const float *mean, long R, int C, float *st) {
    constexpr int EPC = 16 / sizeof(T);
    constexpr bool HAS_G = MODE != DTB_NORM_RMS_NOGAMMA;
    constexpr bool LN = MODE == DTB_NORM_LAYER;
    const int lane = threadIdx.x & 63;
    const long row = (long)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (row >= R) return;
    const int nch = C / EPC;
    const float r = rstd[row];
    const float mu = LN ? mean[row] : 0.f;
    float s1 = 0.f, s2 = 0.f;
    for (int c = lane; c < nch; c += 64) {
        float xv[EPC], d[EPC], gv[EPC];
        unpack16<T>(ld16(x + row * C + c * EPC), xv);
        unpack16<T>(ld16(dy + row * C + c * EPC), d);
#pragma unroll
        for (int e = 0; e < EPC; e++) gv[e] = 1.f;
        if (HAS_G) unpack16<T>(ld16(g + c * EPC), gv);
#pragma unroll
        for (int e = 0; e < EPC; e++) {
            const float xh = (xv[e] - mu) * r;
            const float dn = d[e] * gv[e];
            s1 += dn;
            s2 += dn * xh;
        }
    }
    s2 = wave_sum(s2) / C;
    if (LN) s1 = wave_sum(s1) / C;
    if (lane == 0) {
        st[2 * row] = LN ? s1 : 0.f;
        st[2 * row + 1] = s2;
    }
}

// dx = dres + Norm^T(dy).  Each wave handles rows wave_id, wave_id + nwaves, ...;
// gamma/beta partials per workgroup -> part[blockIdx.x][0..C) and [C..2C).
// WIN: the workgroup covers the column window blockIdx.y (64 NPL chunks) of
// its rows and takes the row statistics from st (norm_bwd_stats_kernel);
// otherwise one wave holds a whole row and reduces it itself.
template <typename T, int NPL, int MODE, bool WIN>
__global__ __launch_bounds__(256) void norm_bwd_kernel(const T *dy, const T *x, const T *g, const float *rstd,
                                                        const float *mean, const T *dres, long R, int C, T *dx,
                                                        float *part, const float *st) {
    constexpr int EPC = 16 / sizeof(T);
    constexpr bool HAS_G = MODE != DTB_NORM_RMS_NOGAMMA;
    constexpr bool LN = MODE == DTB_NORM_LAYER;
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nch = C / EPC;
    const int c0 = WIN ? (int)blockIdx.y * 64 * NPL : 0;  // first chunk of the window
    const long nwaves = (long)gridDim.x * 4;
    float ag[NPL][EPC], ab[NPL][EPC];
#pragma unroll
    for (int k = 0; k < NPL; k++)
#pragma unroll
        for (int e = 0; e < EPC; e++) ag[k][e] = ab[k][e] = 0.f;
    float gv[NPL][EPC];
#pragma unroll
    for (int k = 0; k < NPL; k++) {
        int c = c0 + lane + 64 * k;
#pragma unroll
        for (int e = 0; e < EPC; e++) gv[k][e] = 1.f;
        if (HAS_G && c < nch) unpack16<T>(ld16(g + c * EPC), gv[k]);
    }
    // Each wave walks its rows with the next row's x, dy and residual
    // gradient already loading while it reduces and stores the current one
    // (two waves per SIMD leave no other latency hiding).
    u32x4 qx[NPL], qd[NPL], qr[NPL];
    auto fetch = [&](long rw) {
        const bool live = rw < R;
        const long rr = live ? rw : 0;
        const Buf bx(x + rr * C), bd(dy + rr * C), br(dres ? dres + rr * C : dy + rr * C);
#pragma unroll
        for (int k = 0; k < NPL; k++) {
            const int c = c0 + lane + 64 * k;
            qx[k] = bx.ld16(c * 16, live && c < nch);
            qd[k] = bd.ld16(c * 16, live && c < nch);
            qr[k] = br.ld16(c * 16, live && dres != nullptr && c < nch);
        }
    };
    long row = (long)blockIdx.x * 4 + wave;
    fetch(row);
    for (; row < R; row += nwaves) {
        const float r = rstd[row];
        const float mu = LN ? mean[row] : 0.f;
        float xh[NPL][EPC], d[NPL][EPC];
        u32x4 rsv[NPL];
#pragma unroll
        for (int k = 0; k < NPL; k++) {
            unpack16<T>(qx[k], xh[k]);
            unpack16<T>(qd[k], d[k]);
            rsv[k] = qr[k];
        }
        fetch(row + nwaves);
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int k = 0; k < NPL; k++) {
#pragma unroll
            for (int e = 0; e < EPC; e++) {
                xh[k][e] = (xh[k][e] - mu) * r;        // normalised input
                float dn = d[k][e] * gv[k][e];
                s1 += dn;
                s2 += dn * xh[k][e];
            }
        }
        if constexpr (WIN) {
            s1 = st[2 * row];
            s2 = st[2 * row + 1];
        } else {
            s2 = wave_sum(s2) / C;
            if (LN) s1 = wave_sum(s1) / C;
        }
        // residual gradient (rsv) added to the result (zeros when dres is null)
#pragma unroll
        for (int k = 0; k < NPL; k++) {
            int c = c0 + lane + 64 * k;
            if (c >= nch) continue;
            float rs[EPC], o[EPC];
            unpack16<T>(rsv[k], rs);
#pragma unroll
            for (int e = 0; e < EPC; e++) {
                float dn = d[k][e] * gv[k][e];
                // RMS: r (dn - xhat * mean(dn xhat));  LN: r (dn - mean(dn) - xhat mean(dn xhat))
                float v = r * (dn - (LN ? s1 : 0.f) - xh[k][e] * s2);
                o[e] = rs[e] + v;
                ag[k][e] += d[k][e] * xh[k][e];
                ab[k][e] += d[k][e];
            }
            st16(dx + row * C + c * EPC, pack16<T>(o));
        }
    }
    if (!HAS_G) return;
    // combine the 4 waves through LDS, chunk by chunk, then write the partial
    __shared__ float buf[4][64 * 4];
#pragma unroll
    for (int k = 0; k < NPL; k++) {
        for (int half = 0; half < (LN ? 2 : 1); half++) {
#pragma unroll
            for (int e0 = 0; e0 < EPC; e0 += 4) {
                __syncthreads();
#pragma unroll
                for (int e = 0; e < 4; e++) buf[wave][lane * 4 + e] = half ? ab[k][e0 + e] : ag[k][e0 + e];
                __syncthreads();
                // thread i (of 256) owns element i of the 64*4 slice
                int i = threadIdx.x;
                float sum = buf[0][i] + buf[1][i] + buf[2][i] + buf[3][i];
                int ln = i >> 2, e = i & 3;
                int c = c0 + ln + 64 * k;
                if (c < nch) part[(long)blockIdx.x * 2 * C + half * C + c * EPC + e0 + e] = sum;
            }
        }
    }
}

// dst[i] += sum over p of part[p][i] for the n columns of part (row stride
// ld); with dst1, columns n .. 2n-1 of part go to dst1 (the gamma and beta
// partials of a LayerNorm, side by side in part, in one launch).  A workgroup
// covers 32 columns with 32 groups of 32 threads: group pg sums the parts
// pg, pg + 32, ... (a few independent loads, issued back to back: the partials
// are few hundred rows, so the latency of one batch is the kernel's time),
// then the 32 group sums meet in a fixed tree.  Deterministic.
__global__ __launch_bounds__(1024) void reduce_parts_kernel(const float *part, int np, long ld, int n, float *dst,
                                                            float *dst1) {
    __shared__ float red[32][33];
    const int c = threadIdx.x & 31, pg = threadIdx.x >> 5;
    const int i = blockIdx.x * 32 + c;
    const int ncols = dst1 ? 2 * n : n;
    float s = 0.f;
    if (i < ncols) {
#pragma unroll 8
        for (int p = pg; p < np; p += 32) s += part[(long)p * ld + i];
    }
    red[pg][c] = s;
    __syncthreads();
    // pairwise tree over the 32 groups: after the step of width w, group g < w
    // holds the sum of groups g, g + w, g + 2w, ... (a fixed order)
#pragma unroll
    for (int w = 16; w >= 1; w >>= 1) {
        if (pg < w) red[pg][c] += red[pg + w][c];
        __syncthreads();
    }
    if (pg == 0 && i < ncols) {
        const float t = red[0][c];
        if (i < n) dst[i] += t;
        else dst1[i - n] += t;
    }
}

static int npl_for(int C, int dtype) {
    int epc = dtype == DTB_BF16 ? 8 : 4;
    int nch = C / epc;
    int npl = 1;
    while (64 * npl < nch) npl <<= 1;
    return npl;
}

template <typename T, int NPL>
static hipError_t norm_fwd_t(int mode, const void *x, const void *g, const void *b, float eps, long R, int C,
                             void *out, float *rstd, float *mean, hipStream_t s) {
    dim3 grid((unsigned)((R + 3) / 4));
    const T *xx = (const T *)x, *gg = (const T *)g, *bb = (const T *)b;
    T *oo = (T *)out;
    if (mode == DTB_NORM_RMS)
        DTB_LAUNCH((norm_fwd_kernel<T, NPL, DTB_NORM_RMS>), grid, dim3(256), 0, s, xx, gg, bb, eps, R, C, oo,
                           rstd, mean);
    else if (mode == DTB_NORM_RMS_NOGAMMA)
        DTB_LAUNCH((norm_fwd_kernel<T, NPL, DTB_NORM_RMS_NOGAMMA>), grid, dim3(256), 0, s, xx, gg, bb, eps,
                           R, C, oo, rstd, mean);
    else
        DTB_LAUNCH((norm_fwd_kernel<T, NPL, DTB_NORM_LAYER>), grid, dim3(256), 0, s, xx, gg, bb, eps, R, C,
                           oo, rstd, mean);
    return last_error();
}

#define NPL_DISPATCH(FN, T, npl, ...)                                                   \
    (npl == 1   ? FN<T, 1>(__VA_ARGS__)                                                \
     : npl == 2 ? FN<T, 2>(__VA_ARGS__)                                                \
     : npl == 4 ? FN<T, 4>(__VA_ARGS__)                                                \
     : npl == 8 ? FN<T, 8>(__VA_ARGS__)                                                \
                : FN<T, 16>(__VA_ARGS__))

int norm_forward(int mode, int dtype, const void *x, const void *g, const void *b, float eps, long R, int C,
                 void *out, float *rstd, float *mean, hipStream_t s) {
    if (R <= 0) return DTB_OK;
    int npl = npl_for(C, dtype);
    if (g_timing_on) timing_begin(s, K_ELEM);
    hipError_t e = dtype == DTB_BF16 ? NPL_DISPATCH(norm_fwd_t, bf16, npl, mode, x, g, b, eps, R, C, out, rstd, mean, s)
                                     : NPL_DISPATCH(norm_fwd_t, float, npl, mode, x, g, b, eps, R, C, out, rstd, mean, s);
    if (e != hipSuccess) return set_launch_error(e, "norm_forward");
    if (g_timing_on) {
        double es = dtype == DTB_BF16 ? 2 : 4;
        timing_end(s, K_ELEM, 0, (double)R * (2 * es * C + (mode == DTB_NORM_LAYER ? 8 : 4)));
    }
    return DTB_OK;
}

int norm_backward_parts(long R) {
    long waves = (R + 3) / 4;
    return (int)(waves < 512 ? (waves > 0 ? waves : 1) : 512);
}

// Rows of 16 chunks per lane (bf16 C > 4096, fp32 C > 2048), whose chunks and
// gamma / beta partial sums no longer fit a wave's registers (the whole-row
// kernel spilled hundreds of registers there), take the windowed path: a
// statistics pass over each row, then workgroups of 4-chunk column windows.
// R = 16384: bf16 C = 8192 RMS 1393 -> 271 us, LayerNorm 1635 -> 288 us; fp32
// C = 4096 RMS 264 -> 262 us, LayerNorm 365 -> 272 us.  (The bf16 LayerNorm at
// 8 chunks spills 67 registers but measured 112 us against 128-137 windowed.)
template <typename T, int MODE, int NPL> constexpr bool norm_bwd_windowed() { return NPL >= 16; }

template <typename T, int MODE, int NPL, bool WIN>
static void norm_bwd_launch(dim3 grid, const T *a, const T *xx, const T *gg, const float *rstd, const float *mean,
                            const T *rr, long R, int C, T *o, float *part, const float *st, hipStream_t s) {
    DTB_LAUNCH((norm_bwd_kernel<T, NPL, MODE, WIN>), grid, dim3(256), 0, s, a, xx, gg, rstd, mean, rr, R, C, o, part,
               st);
}

template <typename T, int MODE, int NPL>
static hipError_t norm_bwd_mode(const T *a, const T *xx, const T *gg, const float *rstd, const float *mean,
                                const T *rr, long R, int C, T *o, float *part, int np, float *st, hipStream_t s) {
    if constexpr (norm_bwd_windowed<T, MODE, NPL>()) {
        DTB_LAUNCH((norm_bwd_stats_kernel<T, MODE>), dim3((unsigned)((R + 3) / 4)), dim3(256), 0, s, a, xx, gg, rstd,
                   mean, R, C, st);
        hipError_t e = last_error();
        if (e != hipSuccess) return e;
        norm_bwd_launch<T, MODE, 4, true>(dim3(np, NPL / 4), a, xx, gg, rstd, mean, rr, R, C, o, part, st, s);
    } else {
        norm_bwd_launch<T, MODE, NPL, false>(dim3(np), a, xx, gg, rstd, mean, rr, R, C, o, part, nullptr, s);
    }
    return last_error();
}

template <typename T, int NPL>
static hipError_t norm_bwd_t(int mode, const void *dy, const void *x, const void *g, const float *rstd,
                             const float *mean, const void *dres, long R, int C, void *dx, float *part, int np,
                             hipStream_t s) {
    const T *a = (const T *)dy, *xx = (const T *)x, *gg = (const T *)g, *rr = (const T *)dres;
    T *o = (T *)dx;
    float *st = part + norm_backward_stats_offset(np, C);
    if (mode == DTB_NORM_RMS)
        return norm_bwd_mode<T, DTB_NORM_RMS, NPL>(a, xx, gg, rstd, mean, rr, R, C, o, part, np, st, s);
    if (mode == DTB_NORM_RMS_NOGAMMA)
        return norm_bwd_mode<T, DTB_NORM_RMS_NOGAMMA, NPL>(a, xx, gg, rstd, mean, rr, R, C, o, part, np, st, s);
    return norm_bwd_mode<T, DTB_NORM_LAYER, NPL>(a, xx, gg, rstd, mean, rr, R, C, o, part, np, st, s);
}

int norm_backward(int mode, int dtype, const void *dy, const void *x, const void *g, const float *rstd,
                  const float *mean, const void *dres, long R, int C, void *dx, float *dg, float *db, float *part,
                  int npart, hipStream_t s) {
    if (R <= 0) return DTB_OK;
    int npl = npl_for(C, dtype);
    if (g_timing_on) timing_begin(s, K_ELEM);
    hipError_t e = dtype == DTB_BF16
                       ? NPL_DISPATCH(norm_bwd_t, bf16, npl, mode, dy, x, g, rstd, mean, dres, R, C, dx, part, npart, s)
                       : NPL_DISPATCH(norm_bwd_t, float, npl, mode, dy, x, g, rstd, mean, dres, R, C, dx, part, npart, s);
    if (e != hipSuccess) return set_launch_error(e, "norm_backward");
    if (mode != DTB_NORM_RMS_NOGAMMA) {
        // LayerNorm: the gamma (columns 0 .. C-1) and beta (C .. 2C-1) partials in one launch
        const bool ln = mode == DTB_NORM_LAYER;
        DTB_LAUNCH(reduce_parts_kernel, dim3(((ln ? 2 : 1) * C + 31) / 32), dim3(1024), 0, s, part, npart, 2L * C, C,
                   dg, ln ? db : (float *)nullptr);
        e = last_error();
        if (e != hipSuccess) return set_launch_error(e, "norm_backward reduce");
    }
    if (g_timing_on) {
        double es = dtype == DTB_BF16 ? 2 : 4;
        timing_end(s, K_ELEM, 0, (double)R * (4 * es * C + (mode == DTB_NORM_LAYER ? 8 : 4)));
    }
    return DTB_OK;
}

// ------------------------------------------------------------------ RoPE ---
// cs[t][i] = (cos(t theta_i), sin(t theta_i)), theta_i = base^(-2i/hd), computed
// in double and rounded to fp32 (fp32 angles lose ~1e-4 rad at t ~ 1e3-1e4)
// cos / sin of the angle t * base^(-2k/hd), in fp64, rounded to fp32.  The
// angle (up to T radians) is first reduced by whole turns, a - n 2pi with 2pi
// split into two doubles (Cody-Waite; each fma is exact up to one rounding of
// a result below pi, so the reduced angle is good to ~1e-15), which keeps
// cos and sin on their short-argument path.
__global__ void rope_table_kernel(float2 *cs, int T, int half, int hd, double base) {
    long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)T * half) return;
    int t = (int)(i / half), k = (int)(i % half);
    const double theta = pow(base, -2.0 * k / hd);
    const double a = t * theta;
    constexpr double TWO_PI_HI = 6.283185307179586232e+00;   // 2pi rounded to double
    constexpr double TWO_PI_LO = 2.449293598294706354e-16;   // 2pi - TWO_PI_HI
    constexpr double INV_TWO_PI = 1.591549430918953358e-01;
    const double n = rint(a * INV_TWO_PI);
    const double r = fma(-n, TWO_PI_LO, fma(-n, TWO_PI_HI, a));
    double sn, c;
    sincos(r, &sn, &c);
    cs[i] = make_float2((float)c, (float)sn);
}

int rope_table(float *cs, int T, int hd, float base, hipStream_t s) {
    int half = hd / 2;
    long n = (long)T * half;
    if (n <= 0) return DTB_OK;
    DTB_LAUNCH(rope_table_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, (float2 *)cs, T, half,
                       hd, (double)base);
    DTB_LAUNCH_CHECK("rope_table");
    return DTB_OK;
}

// one thread per (row, head, pair i); heads 0..NH-1 are q (offset 0), NH.. are k (offset C)
template <typename T>
__global__ __launch_bounds__(256) void rope_kernel(T *qkv, const float2 *cs, long BT, int T_, int QKV, int NH,
                                                    int NKV, int hd, int inverse) {
    const int half = hd / 2;
    const int nheads = NH + NKV;
    long i = (long)blockIdx.x * 256 + threadIdx.x;
    long total = BT * nheads * half;
    if (i >= total) return;
    int k = (int)(i % half);
    long rh = i / half;
    int head = (int)(rh % nheads);
    long row = rh / nheads;
    int t = (int)(row % T_);
    T *v = qkv + row * QKV + (long)head * hd;   // k heads follow the q heads contiguously
    float2 c = cs[(long)t * half + k];
    float x = to_f32(v[k]), y = to_f32(v[k + half]);
    float sn = inverse ? -c.y : c.y;
    v[k] = from_f32<T>(x * c.x - y * sn);
    v[k + half] = from_f32<T>(y * c.x + x * sn);
}

int rope_apply(int dtype, void *qkv, const float *cs, int B, int T, int QKV, int NH, int NKV, int hd, int inverse,
               hipStream_t s) {
    long BT = (long)B * T;
    long total = BT * (NH + NKV) * (hd / 2);
    if (total <= 0) return DTB_OK;
    if (g_timing_on) timing_begin(s, K_ELEM);
    dim3 grid((unsigned)((total + 255) / 256));
    if (dtype == DTB_BF16)
        DTB_LAUNCH(rope_kernel<bf16>, grid, dim3(256), 0, s, (bf16 *)qkv, (const float2 *)cs, BT, T, QKV, NH,
                           NKV, hd, inverse);
    else
        DTB_LAUNCH(rope_kernel<float>, grid, dim3(256), 0, s, (float *)qkv, (const float2 *)cs, BT, T, QKV,
                           NH, NKV, hd, inverse);
    DTB_LAUNCH_CHECK("rope");
    if (g_timing_on) timing_end(s, K_ELEM, 0, 2.0 * (dtype == DTB_BF16 ? 2 : 4) * total * 2);
    return DTB_OK;
}

// ------------------------------------------------------------ activations ---
// logistic sigmoid with the hardware reciprocal (1 ulp; an IEEE division
// here is a ten-instruction sequence); 1 + e^-x = inf gives 0
__device__ __forceinline__ float sigm(float x) { return __builtin_amdgcn_rcpf(1.f + __expf(-x)); }
template <typename T, int MLP>
__global__ __launch_bounds__(256) void act_fwd_kernel(const T *up, long R, int H, T *h) {
    constexpr int EPC = 16 / sizeof(T);
    const int W = MLP == DTB_MLP_SWIGLU ? 2 * H : H;
    const int hc = H / EPC;
    long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= R * hc) return;
    long r = i / hc;
    int c = (int)(i % hc);
    float a[EPC], o[EPC];
    unpack16<T>(ld16(up + r * W + c * EPC), a);
    if (MLP == DTB_MLP_SWIGLU) {
        float u[EPC];
        unpack16<T>(ld16(up + r * W + H + c * EPC), u);
#pragma unroll
        for (int e = 0; e < EPC; e++) o[e] = a[e] * sigm(a[e]) * u[e];
    } else if (MLP == DTB_MLP_RELU) {
#pragma unroll
        for (int e = 0; e < EPC; e++) o[e] = a[e] > 0.f ? a[e] : 0.f;
    } else {
#pragma unroll
        for (int e = 0; e < EPC; e++) {
            float f = a[e];
            o[e] = 0.5f * f * (1.f + tanhf(GELU_K * (f + GELU_C * f * f * f)));
        }
    }
    st16(h + r * H + c * EPC, pack16<T>(o));
}

template <typename T, int MLP>
__global__ __launch_bounds__(256) void act_bwd_kernel(const T *dh, const T *up, long R, int H, T *dup) {
    constexpr int EPC = 16 / sizeof(T);
    const int W = MLP == DTB_MLP_SWIGLU ? 2 * H : H;
    const int hc = H / EPC;
    long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= R * hc) return;
    long r = i / hc;
    int c = (int)(i % hc);
    float d[EPC], a[EPC], u[EPC], o[EPC], du[EPC];
    unpack16<T>(ld16(dh + r * H + c * EPC), d);
    unpack16<T>(ld16(up + r * W + c * EPC), a);
    if (MLP == DTB_MLP_SWIGLU) unpack16<T>(ld16(up + r * W + H + c * EPC), u);
#pragma unroll
    for (int e = 0; e < EPC; e++) o[e] = act_grad(MLP, d[e], a[e], MLP == DTB_MLP_SWIGLU ? u[e] : 0.f, &du[e]);
    if (MLP == DTB_MLP_SWIGLU) st16(dup + r * W + H + c * EPC, pack16<T>(du));
    st16(dup + r * W + c * EPC, pack16<T>(o));
}

template <typename T>
static hipError_t act_fwd_t(int mlp, const void *up, long R, int H, void *h, hipStream_t s) {
    constexpr int EPC = 16 / sizeof(T);
    long n = R * (H / EPC);
    dim3 grid((unsigned)((n + 255) / 256));
    if (mlp == DTB_MLP_SWIGLU)
        DTB_LAUNCH((act_fwd_kernel<T, DTB_MLP_SWIGLU>), grid, dim3(256), 0, s, (const T *)up, R, H, (T *)h);
    else if (mlp == DTB_MLP_RELU)
        DTB_LAUNCH((act_fwd_kernel<T, DTB_MLP_RELU>), grid, dim3(256), 0, s, (const T *)up, R, H, (T *)h);
    else
        DTB_LAUNCH((act_fwd_kernel<T, DTB_MLP_GELU_TANH>), grid, dim3(256), 0, s, (const T *)up, R, H, (T *)h);
    return last_error();
}
template <typename T>
static hipError_t act_bwd_t(int mlp, const void *dh, const void *up, long R, int H, void *dup, hipStream_t s) {
    constexpr int EPC = 16 / sizeof(T);
    long n = R * (H / EPC);
    dim3 grid((unsigned)((n + 255) / 256));
    if (mlp == DTB_MLP_SWIGLU)
        DTB_LAUNCH((act_bwd_kernel<T, DTB_MLP_SWIGLU>), grid, dim3(256), 0, s, (const T *)dh, (const T *)up, R,
                           H, (T *)dup);
    else if (mlp == DTB_MLP_RELU)
        DTB_LAUNCH((act_bwd_kernel<T, DTB_MLP_RELU>), grid, dim3(256), 0, s, (const T *)dh, (const T *)up, R, H,
                           (T *)dup);
    else
        DTB_LAUNCH((act_bwd_kernel<T, DTB_MLP_GELU_TANH>), grid, dim3(256), 0, s, (const T *)dh,
                           (const T *)up, R, H, (T *)dup);
    return last_error();
}

int act_forward(int mlp, int dtype, const void *up, long R, int H, void *h, hipStream_t s) {
    if (R <= 0) return DTB_OK;
    if (g_timing_on) timing_begin(s, K_ELEM);
    hipError_t e = dtype == DTB_BF16 ? act_fwd_t<bf16>(mlp, up, R, H, h, s) : act_fwd_t<float>(mlp, up, R, H, h, s);
    if (e != hipSuccess) return set_launch_error(e, "act_forward");
    if (g_timing_on) {
        double es = dtype == DTB_BF16 ? 2 : 4;
        timing_end(s, K_ELEM, 0, es * R * H * (mlp == DTB_MLP_SWIGLU ? 3 : 2));
    }
    return DTB_OK;
}

int act_backward(int mlp, int dtype, const void *dh, const void *up, long R, int H, void *dup, hipStream_t s) {
    if (R <= 0) return DTB_OK;
    if (g_timing_on) timing_begin(s, K_ELEM);
    hipError_t e = dtype == DTB_BF16 ? act_bwd_t<bf16>(mlp, dh, up, R, H, dup, s)
                                     : act_bwd_t<float>(mlp, dh, up, R, H, dup, s);
    if (e != hipSuccess) return set_launch_error(e, "act_backward");
    if (g_timing_on) {
        double es = dtype == DTB_BF16 ? 2 : 4;
        timing_end(s, K_ELEM, 0, es * R * H * (mlp == DTB_MLP_SWIGLU ? 5 : 3));
    }
    return DTB_OK;
}

// --------------------------------------------------------- bias gradient ---
// part[p][n] = sum over the p-th range of rows of dy[r][n].  A workgroup owns
// 64 column chunks of 16 bytes (one per lane) and one row range; its four
// waves take every fourth row of the range, and their sums are combined in
// LDS in a fixed order (deterministic).
template <typename T>
__global__ __launch_bounds__(256) void colsum_kernel(const T *dy, long R, int N, long rows_per, float *part) {
    constexpr int EPV = 16 / sizeof(T);
    __shared__ float red[3][64 * EPV];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int n0 = (blockIdx.x * 64 + lane) * EPV;
    const long r0 = (long)blockIdx.y * rows_per, r1 = min(R, r0 + rows_per);
    const bool ok = n0 < N;
    float acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; e++) acc[e] = 0.f;
    if (ok) {
#pragma unroll 4
        for (long r = r0 + wv; r < r1; r += 4) {
            float f[EPV];
            unpack16<T>(ld16(dy + r * N + n0), f);
#pragma unroll
            for (int e = 0; e < EPV; e++) acc[e] += f[e];
        }
    }
    if (wv > 0) {
#pragma unroll
        for (int e = 0; e < EPV; e++) red[wv - 1][lane * EPV + e] = acc[e];
    }
    __syncthreads();
    if (wv == 0 && ok) {
        float *dst = part + (long)blockIdx.y * N + n0;
#pragma unroll
        for (int e4 = 0; e4 < EPV; e4 += 4) {
            f32x4 v;
#pragma unroll
            for (int e = 0; e < 4; e++)
                v[e] = (acc[e4 + e] + red[0][lane * EPV + e4 + e]) +
                       (red[1][lane * EPV + e4 + e] + red[2][lane * EPV + e4 + e]);
            *reinterpret_cast<f32x4 *>(dst + e4) = v;
        }
    }
}

// the most row ranges a bias gradient of R rows uses (sizes the partials)
int bias_grad_parts(long R) {
    long p = (R + 15) / 16;
    return (int)(p < 512 ? (p > 0 ? p : 1) : 512);
}

int bias_grad(int dtype, const void *dy, long R, int N, float *db, float *part, int npart, hipStream_t s) {
    if (R <= 0 || N <= 0) return DTB_OK;
    if (g_timing_on) timing_begin(s, K_ELEM);
    // about 1024 workgroups: the column blocks times as many row ranges as
    // that takes (at most npart, at least 16 rows each)
    const int epv = dtype == DTB_BF16 ? 8 : 4;
    const int cblocks = (N / epv + 63) / 64;
    int np = (1024 + cblocks - 1) / cblocks;
    if (np > npart) np = npart;
    if (np < 1) np = 1;
    const long rows_per = (R + np - 1) / np;
    np = (int)((R + rows_per - 1) / rows_per);
    dim3 grid(cblocks, np);
    if (dtype == DTB_BF16)
        DTB_LAUNCH(colsum_kernel<bf16>, grid, dim3(256), 0, s, (const bf16 *)dy, R, N, rows_per, part);
    else
        DTB_LAUNCH(colsum_kernel<float>, grid, dim3(256), 0, s, (const float *)dy, R, N, rows_per, part);
    DTB_LAUNCH(reduce_parts_kernel, dim3((N + 31) / 32), dim3(1024), 0, s, part, np, (long)N, N, db,
               (float *)nullptr);
    DTB_LAUNCH_CHECK("bias_grad");
    if (g_timing_on) timing_end(s, K_ELEM, 0, (double)R * N * (dtype == DTB_BF16 ? 2 : 4));
    return DTB_OK;
}

}  // namespace dtb
