// Internal header of libdtb: element types, vector loads, MFMA wrappers and
// the launch bookkeeping shared by the kernel files.  gfx950 (CDNA4) only.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/dtb.h"

namespace dtb {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr int WAVE = 64;

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

// 16-byte vector of T: 4 floats or 8 bf16
template <typename T> struct Vec;
template <> struct Vec<float> {
    static constexpr int N = 4;
    typedef f32x4 type;
};
template <> struct Vec<bf16> {
    static constexpr int N = 8;
    typedef bf16x8 type;
};

template <typename T> __device__ __forceinline__ u32x4 ld16(const T *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
template <typename T> __device__ __forceinline__ void st16(T *p, u32x4 v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}

// Branch-free masked 16-byte loads: a raw buffer resource over a base pointer;
// an invalid lane passes an offset past num_records and the hardware returns
// zeros (no divergent branch, so no wait is forced before the next load).
// Byte offsets must stay below 2^31 from the base.
struct Buf {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ explicit Buf(const void *p)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, 0x7fffffff, 0x00020000)) {}
    __device__ __forceinline__ u32x4 ld16(int byte_off, bool ok) const {
        return __builtin_amdgcn_raw_buffer_load_b128(r, ok ? byte_off : (int)0x80000000, 0, 0);
    }
    __device__ __forceinline__ u32x4 ld16(int byte_off) const {
        return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
    }
};

typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// unpack / pack a 16-byte vector into floats
template <typename T> __device__ __forceinline__ void unpack16(u32x4 v, float *f);
template <> __device__ __forceinline__ void unpack16<float>(u32x4 v, float *f) {
#pragma unroll
    for (int i = 0; i < 4; i++) f[i] = __uint_as_float(v[i]);
}
template <> __device__ __forceinline__ void unpack16<bf16>(u32x4 v, float *f) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        f[2 * i] = __uint_as_float(v[i] << 16);
        f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
    }
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) { return pack2_bf16(lo, hi); }
template <typename T> __device__ __forceinline__ u32x4 pack16(const float *f);
template <> __device__ __forceinline__ u32x4 pack16<float>(const float *f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = __float_as_uint(f[i]);
    return v;
}
template <> __device__ __forceinline__ u32x4 pack16<bf16>(const float *f) {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; i++) v[i] = pack_bf16x2(f[2 * i], f[2 * i + 1]);
    return v;
}

// wave-wide reductions (64 lanes)
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// max / sum of the lane's value and that of lane l ^ 32.  v_permlane32_swap
// exchanges the upper 32 lanes of one register with the lower 32 of another:
// swapping x with itself leaves the lower half's values in one result and the
// upper half's in the other, in every lane, so no LDS round trip is needed.
__device__ __forceinline__ float max_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// maximum of N values as a balanced tree of 3-input maxima (dependency depth
// log3 N instead of a serial chain of N/2)
template <int N> __device__ __forceinline__ float tree_max(const float *v) {
    if constexpr (N == 1) {
        return v[0];
    } else if constexpr (N == 2) {
        return fmaxf(v[0], v[1]);
    } else {
        constexpr int M = (N + 2) / 3;
        float w[M];
#pragma unroll
        for (int i = 0; i < M; i++) {
            const int a = 3 * i;
            w[i] = a + 2 < N ? fmaxf(fmaxf(v[a], v[a + 1]), v[a + 2]) : a + 1 < N ? fmaxf(v[a], v[a + 1]) : v[a];
        }
        return tree_max<M>(w);
    }
}

// ---------------------------------------------------------------- MFMA ---
// 32x32 output block: lane l, accumulator r holds row 8*(r/4) + 4*(l/32) + r%4,
// column l%32.  The A operand lane l supplies row l%32, the B operand lane l
// column l%32; both supply the same k positions for the same lane half l/32.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---- activation backward, per element --------------------------------------
// d: gradient of the activation output; a: its input (SwiGLU: the gate g);
// u: the SwiGLU up value.  Returns the gradient of a; *du receives the SwiGLU
// gradient of u.  ("nanoeuler — CUDA kernels": swiglu_backward_kernel;
// "microgpt.cu": relu_backward_kernel; llm.c gelu_backward, tanh form.)
constexpr float GELU_K = 0.7978845608028654f;  // sqrt(2/pi)
constexpr float GELU_C = 0.044715f;
__device__ __forceinline__ float act_grad(int mlp, float d, float a, float u, float *du) {
    if (mlp == DTB_MLP_SWIGLU) {
        const float sg = 1.f / (1.f + __expf(-a));
        *du = d * a * sg;
        return d * u * sg * (1.f + a * (1.f - sg));
    } else if (mlp == DTB_MLP_RELU) {
        return a > 0.f ? d : 0.f;
    } else {
        const float t = GELU_K * (a + GELU_C * a * a * a);
        const float th = tanhf(t);
        return d * (0.5f * (1.f + th) + 0.5f * a * (1.f - th * th) * GELU_K * (1.f + 3.f * GELU_C * a * a));
    }
}

// ---- MFMA on one 16-byte chunk of A and B ---------------------------------
__device__ __forceinline__ void mma_chunk(f32x16 &acc, u32x4 a, u32x4 b, bf16) {
    acc = mfma32(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc);
}
__device__ __forceinline__ void mma_chunk(f32x16 &acc, u32x4 a, u32x4 b, float) {
#pragma unroll
    for (int e = 0; e < 4; e++) acc = mfma32(__uint_as_float(a[e]), __uint_as_float(b[e]), acc);
}

// ---- transposes of register blocks ---------------------------------------
// bf16 8x8: in[i] holds row k=i (8 consecutive m); out[j] holds m=j (8 consecutive k)
__device__ __forceinline__ void transpose8x8(const u32x4 *in, u32x4 *out) {
#pragma unroll
    for (int j = 0; j < 8; j++) {
#pragma unroll
        for (int p = 0; p < 4; p++) {
            uint32_t a = in[2 * p][j >> 1], b = in[2 * p + 1][j >> 1];
            out[j][p] = (j & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
    }
}
// fp32 4x4
__device__ __forceinline__ void transpose4x4(const u32x4 *in, u32x4 *out) {
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
        for (int p = 0; p < 4; p++) out[j][p] = in[p][j];
}

// ----------------------------------------------------------- host side ---
struct Launch {
    hipStream_t stream;
};

// per-kernel-class timing (measurement only)
// timing classes: GEMMs by role (forward projections: both operands k-major,
// output in the storage dtype; input gradients: B m/n-major; weight gradients:
// fp32 accumulation), attention, everything else
enum KClass {
    K_GEMM_FWD = 0, K_ATTN_FWD = 1, K_ATTN_BWD = 2, K_ELEM = 3, K_GEMM_DINP = 4, K_GEMM_DW = 5,
    K_ATTN_DEC = 6, K_DEC_MERGE = 7, K_NCLASS = 8
};
void timing_begin(hipStream_t s, int cls);  // opens a unit only if cls is enabled
void timing_end(hipStream_t s, int cls, double flops, double bytes);
void timing_launch_events(hipEvent_t *start, hipEvent_t *stop);
extern bool g_timing_on;

// Every kernel launch of the library.  While a timed unit is open (between
// timing_begin and timing_end) the launch carries the unit's start event (on
// its first launch) and a stop event on its own dispatch packet, so timing
// adds no marker packets, and no idle time, between kernels.
// Opt-in debugging (dtb_debug_enable): with a level above 0, every launch is
// followed by a check of the launch and a wait for the stream, and the first
// failure of the calling thread is kept for last_error() with the kernel's name.
extern int g_debug_level;
void debug_after_launch(hipStream_t s, const char *kernel);

#define DTB_LAUNCH(kernel, grid, block, shmem, stream, ...)                                        \
    do {                                                                                           \
        hipEvent_t dtb_ev0_ = nullptr, dtb_ev1_ = nullptr;                                         \
        if (g_timing_on) timing_launch_events(&dtb_ev0_, &dtb_ev1_);                               \
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, dtb_ev0_, dtb_ev1_, 0u, __VA_ARGS__); \
        if (g_debug_level) ::dtb::debug_after_launch(stream, #kernel);                             \
    } while (0)

int set_launch_error(hipError_t e, const char *what);
// hipGetLastError(), or (debug mode) the first failure a debug check saw
hipError_t last_error();

#define DTB_LAUNCH_CHECK(what)                                           \
    do {                                                                  \
        hipError_t _e = ::dtb::last_error();                              \
        if (_e != hipSuccess) return ::dtb::set_launch_error(_e, what);   \
    } while (0)

// ---------------------------------------------------------- internal ops ---
// GEMM: C[m, n] = sum_k A(m, k) B(n, k) over a K range, with
//   A(m, k) = a_kmajor ? A[m*lda + k] : A[k*lda + m]
//   B(n, k) = b_kmajor ? B[n*ldb + k] : B[k*ldb + n]
// Epilogue: out = acc (+ bias[n]) (+ res[m*ldr + n]) stored as out_dtype, or
// (accumulate) out_f32 += acc.
struct GemmArgs {
    const void *A, *B;
    long long lda, ldb;
    int M, N, K;
    bool a_kmajor, b_kmajor;
    int dtype;            // operand dtype
    void *out;            // dtype (or fp32 when out_f32)
    long long ldo;
    bool out_f32;         // out is fp32
    bool accumulate;      // out_f32 += acc
    const void *bias;     // [N] dtype, may be NULL
    const void *res;      // [M, ldr] dtype, may be NULL (may alias out)
    long long ldr;
    // NeoX RoPE of the output (after the bias): columns [0, rope_cols) are
    // heads of rope_hd, row m is position m % rope_T; table [rope_T][rope_hd/2]
    // of (cos, sin).  Null rope_cs: none.  Only with the plain dtype output.
    const float *rope_cs;
    int rope_T, rope_hd, rope_cols;
    // activation forward: out = [M][ldo] activation input (ldo = N = 2 act_H for
    // SwiGLU, gate columns then up columns) and act_h [M][act_H] = activation
    // output (fused into the GEMM where the tiling allows, else a second pass).
    // Null: none.
    void *act_h;
    int act_mode, act_H;
};
// ws: fp32 scratch for split-K partials (may be NULL -> no split)
int gemm(const GemmArgs &g, void *ws, size_t ws_bytes, hipStream_t s);
size_t gemm_ws_bytes(int M, int N, int K, int dtype);

int launch_attn_forward(void *out, float *lse, const void *qkv, int B, int T, int C, int NH, int NKV,
                        int dtype, hipStream_t s);
// D: fp32 scratch [B][NH][T]
// rope_cs: NeoX (cos, sin) table [T][hd/2] -> dq and dk are rotated back
// (transposed rotation) before they are stored; null for plain attention
int launch_attn_backward(void *dqkv, const void *qkv, const void *out, const void *dout,
                         const float *lse, int B, int T, int C, int NH, int NKV, int dtype,
                         float *D, const float *rope_cs, hipStream_t s);

// decode attention: chunking of the cache and the workspace it needs
struct DecodeGeom {
    int chunk, nsplit, ngrp;
    size_t ws_bytes;
};
DecodeGeom decode_geometry(int B, int NH, int NKV, int hd, int Tmax, int chunk, int dtype);
// cache head row (b, t, kv head) at element b*sb + t*st + kh*sh of each cache
hipError_t attn_decode_launch(void *out, float *lse, const void *q, const void *kc, const void *vc, const int *lens,
                              int B, int NH, int NKV, int hd, int Tmax, long long sb, long long st, long long sh,
                              const DecodeGeom &g, int dtype, void *workspace, hipStream_t s);

// elementwise / reductions
int norm_forward(int mode, int dtype, const void *x, const void *g, const void *b, float eps, long R, int C,
                 void *out, float *rstd, float *mean, hipStream_t s);
// dx = dres + Norm^T(dy); partial sums of dgamma/dbeta into part[npart][2][C]
int norm_backward(int mode, int dtype, const void *dy, const void *x, const void *g, const float *rstd,
                  const float *mean, const void *dres, long R, int C, void *dx, float *dg, float *db,
                  float *part, int npart, hipStream_t s);
int norm_backward_parts(long R);
// the norm backward's workspace: np x 2C fp32 partials, then (wide rows) the
// row statistics, 2 fp32 per row, from this float offset (64-float aligned)
inline long norm_backward_stats_offset(int np, int C) { return ((long)np * 2 * C + 63) / 64 * 64; }
inline size_t norm_backward_ws_bytes(long R, int C) {
    return (size_t)(norm_backward_stats_offset(norm_backward_parts(R), C) + 2 * R) * 4;
}
int rope_table(float *cs, int T, int hd, float base, hipStream_t s);
int rope_apply(int dtype, void *qkv, const float *cs, int B, int T, int QKV, int NH, int NKV, int hd,
               int inverse, hipStream_t s);
int act_forward(int mlp, int dtype, const void *up, long R, int H, void *h, hipStream_t s);
int act_backward(int mlp, int dtype, const void *dh, const void *up, long R, int H, void *dup,
                 hipStream_t s);
// db[n] += sum_r dy[r*N + n]
int bias_grad(int dtype, const void *dy, long R, int N, float *db, float *part, int npart, hipStream_t s);
int bias_grad_parts(long R);

// model harness
int embed_fwd(int dtype, const int *ids, const void *wte, const void *wpe, long BT, int T, int C, int V, void *x,
              hipStream_t s);
int embed_bwd(int dtype, const int *ids, const void *dx, int B, int T, int C, int V, float *dwte, float *dwpe,
              hipStream_t s);
size_t head_ce_ws_bytes(int R, int C, int V, int vc, int dtype);
// K prediction heads: w [K*V, C], targets and row_loss [R][K]
int head_ce(float *loss, float *row_loss, void *dinp, float *dw, const void *inp, const void *w, const int *targets,
            int R, int C, int V, int K, int vc, float scale, int dtype, void *workspace, hipStream_t s);
int adamw(float *p, float *g, float *m, float *v, void *lowp, long long n, float lr, float b1, float b2, float eps,
          float wd, int t, int zero_g, hipStream_t s);
int softmax_xent_rows(int dtype, const void *logits, long ldl, const int *targets, long R, int V, float scale,
                      float *row_loss, void *dlogits, float *loss, hipStream_t s);

}  // namespace dtb
