// MFMA GEMM for gfx950: the linear layers of the block and their backward
// products ("nanoeuler — CUDA kernels": matmul_forward_cuda, out = inp w^T;
// matmul_backward_dinp_cuda, dinp += dout w; matmul_backward_dw_cuda,
// dw += dout^T inp; llm.c matmul_forward / matmul_backward with bias).
//
// One kernel template computes C[m, n] = sum_k A(m, k) B(n, k) for any of the
// three operand layouts:
//   forward  out = x W^T      A = x    [M][K] (k-major)  B = W  [N][K] (k-major)
//   dinp     dx  = dy W       A = dy   [M][K] (k-major)  B = W  [K][N] (n-major)
//   dW       dW += dy^T x     A = dy   [K][M] (m-major)  B = x  [K][N] (n-major)
//
// Design (CDNA4):
// * 256 threads = 4 wave64s in a 2 x 2 grid; each wave owns a (BM/2) x (BN/2)
//   sub-tile made of 32 x 32 MFMA blocks (v_mfma_f32_32x32x16_bf16 for bf16,
//   v_mfma_f32_32x32x2_f32 for fp32) accumulated in fp32.
// * A K-slab of the A and B tiles is staged in LDS as rows of 128 bytes
//   (64 bf16 or 32 fp32 along k) split into eight 16-byte chunks whose
//   position is XOR-swizzled with (row & 7), so the 16-byte fragment reads of
//   32 consecutive rows are spread over all banks.  Two LDS stages: the global
//   loads of slab k+1 are issued before the MFMAs of slab k and written to the
//   other stage afterwards, one barrier per slab.
// * k-major operands are copied with 16-byte loads; m/n-major operands are
//   loaded as 8x8 (bf16) or 4x4 (fp32) blocks and transposed in registers so
//   that LDS always holds k-contiguous rows.
// * Lane half g = lane/32 of both operands reads chunk 2c+g of a slab for
//   c = 0..3; that fixes one common k order for A and B, which is all the MFMA
//   contraction needs.
// * Weight gradients accumulate into fp32 (+=).  When there are too few output
//   tiles to fill 256 CUs, K is split over gridDim.z into fp32 partials that a
//   second kernel adds into the gradient (deterministic, no atomics).
// * Workgroup ids are remapped so that each XCD (ids are dealt round-robin to
//   the 8 XCDs) works on a contiguous, row-grouped range of tiles and shares
//   operand panels in its own L2.
#include <type_traits>

#include "common.h"

namespace dtb {

template <typename T> struct GT;
template <> struct GT<bf16> {
    static constexpr int EPC = 8;   // elements per 16-byte chunk
    static constexpr int BK = 64;   // k per slab (8 chunks)
};
template <> struct GT<float> {
    static constexpr int EPC = 4;
    static constexpr int BK = 32;
};

struct KParams {
    const void *A, *B;
    long long lda, ldb;
    int M, N, K;
    int kchunk;  // k range per split (multiple of BK)
    void *out;
    long long ldo;
    int out_mode;  // 0 store dtype, 1 store fp32, 2 accumulate fp32, 3 split partial fp32,
                   // 5 SwiGLU forward
    const void *bias;
    const void *res;
    long long ldr;
    float *part;   // split partials of splits 1 .. S-1: [S-1][M][N] (split 0 accumulates into out)
    const float2 *rope_cs;  // NeoX RoPE of the output columns [0, rope_cols) (mode 0), or null
    int rope_T, rope_hd, rope_cols;
    // mode 5: SwiGLU forward (256 x 256 kernel) -- tile column block tn holds
    // gate columns tn*128 .. +127 and the matching up columns act_H + tn*128 ..;
    // out receives [g | u] and act_h [M][act_H] receives silu(g) u.
    void *act_h;
    int act_mode, act_H;
};

// 128-byte LDS rows, 16-byte chunk XOR-ed with (row ^ row/8) & 7: conflict-free for
// the 16-byte fragment reads of consecutive rows, the 16-byte k-major row
// stores, and the transposed m/n-major stores whose lanes write rows 8 apart.
__device__ __forceinline__ int swz(int row, int chunk) {
    return row * 128 + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// ---- slab loaders ---------------------------------------------------------
// rows R of an operand tile starting at row0 (< nrows valid), k in [k0, kend)
template <typename T, int R, bool KMAJOR> struct Loader;

template <typename T, int R> struct Loader<T, R, true> {
    static constexpr int P = R / 32;  // rows per thread
    u32x4 reg[P];
    __device__ __forceinline__ void load(const T *base, long long ld, int row0, int nrows, int k0, int kend) {
        const int t = threadIdx.x, c = t & 7;
        const int kk = k0 + c * GT<T>::EPC;
        const Buf buf(base + (long long)row0 * ld + k0);
#pragma unroll
        for (int p = 0; p < P; p++) {
            int r = (t >> 3) + 32 * p, gr = row0 + r;
            reg[p] = buf.ld16((int)(((long long)r * ld + c * GT<T>::EPC) * (int)sizeof(T)), gr < nrows && kk < kend);
        }
    }
    __device__ __forceinline__ void store(char *lds) const {
        const int t = threadIdx.x, c = t & 7;
#pragma unroll
        for (int p = 0; p < P; p++) {
            int r = (t >> 3) + 32 * p;
            *reinterpret_cast<u32x4 *>(lds + swz(r, c)) = reg[p];
        }
    }
};

// m/n-major: global element (k, r) at base[k*ld + r]
template <int R> struct Loader<bf16, R, false> {
    static constexpr int NB = R;                  // (64/8) * (R/8) 8x8 blocks
    static constexpr int P = (NB + 255) / 256;
    u32x4 reg[P][8];
    __device__ __forceinline__ void load(const bf16 *base, long long ld, int row0, int nrows, int k0, int kend) {
        const int t = threadIdx.x;
        const Buf buf(base + (long long)k0 * ld + row0);
#pragma unroll
        for (int p = 0; p < P; p++) {
            int blk = t + 256 * p;
            int rb = blk % (R / 8), kb = blk / (R / 8);
            int gr = row0 + rb * 8;
            bool live = blk < NB && gr < nrows;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                int k = kb * 8 + i;
                reg[p][i] = buf.ld16((int)(((long long)k * ld + rb * 8) * 2), live && k0 + k < kend);
            }
        }
    }
    __device__ __forceinline__ void store(char *lds) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int p = 0; p < P; p++) {
            int blk = t + 256 * p;
            if (blk >= NB) continue;
            int rb = blk % (R / 8), kb = blk / (R / 8);
            u32x4 o[8];
            transpose8x8(reg[p], o);
#pragma unroll
            for (int j = 0; j < 8; j++) {
                int r = rb * 8 + j;
                *reinterpret_cast<u32x4 *>(lds + swz(r, kb)) = o[j];
            }
        }
    }
};

template <int R> struct Loader<float, R, false> {
    static constexpr int NB = 2 * R;              // (32/4) * (R/4) 4x4 blocks
    static constexpr int P = (NB + 255) / 256;
    u32x4 reg[P][4];
    __device__ __forceinline__ void load(const float *base, long long ld, int row0, int nrows, int k0, int kend) {
        const int t = threadIdx.x;
        const Buf buf(base + (long long)k0 * ld + row0);
#pragma unroll
        for (int p = 0; p < P; p++) {
            int blk = t + 256 * p;
            int rb = blk % (R / 4), kb = blk / (R / 4);
            int gr = row0 + rb * 4;
            bool live = blk < NB && gr < nrows;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                int k = kb * 4 + i;
                reg[p][i] = buf.ld16((int)(((long long)k * ld + rb * 4) * 4), live && k0 + k < kend);
            }
        }
    }
    __device__ __forceinline__ void store(char *lds) const {
        const int t = threadIdx.x;
#pragma unroll
        for (int p = 0; p < P; p++) {
            int blk = t + 256 * p;
            if (blk >= NB) continue;
            int rb = blk % (R / 4), kb = blk / (R / 4);
            u32x4 o[4];
            transpose4x4(reg[p], o);
#pragma unroll
            for (int j = 0; j < 4; j++) {
                int r = rb * 4 + j;
                *reinterpret_cast<u32x4 *>(lds + swz(r, kb)) = o[j];
            }
        }
    }
};

// ---- tile id remap ---------------------------------------------------------
__device__ __forceinline__ void tile_coords(int nm, int nn, int &tm, int &tn) {
    int nt = nm * nn;
    int pid = blockIdx.x;
    if ((nt & 7) == 0) pid = (pid & 7) * (nt >> 3) + (pid >> 3);  // contiguous range per XCD
    // groups of 2 tile rows: an XCD's 32 concurrent tiles span 2 rows x 16
    // columns, so each A slab is read by 16 neighbouring workgroups at once
    // (measured against groups of 1, 4, 8 and 16 on the block's shapes: 8 cost
    // the Llama-GQA step 1.7% and 1 cost more)
    const int GM = 2;
    int per_group = GM * nn;
    int group = pid / per_group;
    int first_m = group * GM;
    int gsize = min(nm - first_m, GM);
    int in_group = pid - group * per_group;
    tm = first_m + in_group % gsize;
    tn = in_group / gsize;
}

// four consecutive elements of a row-major T array as floats (zeros if !ok),
// and the store of four floats as T
template <typename T> __device__ __forceinline__ f32x4 load_row4(const void *base, long long idx, bool ok) {
    const Buf b(base);
    if constexpr (std::is_same<T, bf16>::value) {
        u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(b.r, ok ? (int)(idx * 2) : (int)0x80000000, 0, 0);
        return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u), __uint_as_float(w[1] << 16),
                     __uint_as_float(w[1] & 0xffff0000u)};
    } else {
        return __builtin_bit_cast(f32x4, b.ld16(ok ? (int)(idx * 4) : (int)0x80000000, true));
    }
}
template <typename T> __device__ __forceinline__ void store_row4(void *base, long long idx, f32x4 v) {
    if constexpr (std::is_same<T, bf16>::value) {
        u32x2 w{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
        *reinterpret_cast<u32x2 *>(reinterpret_cast<bf16 *>(base) + idx) = w;
    } else {
        *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(base) + idx) = v;
    }
}

// ---- epilogue through LDS ----------------------------------------------------
// One wave writes a 32-row block of its accumulators (NI blocks of 32 columns,
// fp32) to its private LDS region, then reads it back as rows of float4 so
// that the bias / residual reads and the output writes are contiguous vector
// accesses (8 bytes of bf16 or 16 bytes of fp32 per lane) issued without
// intervening waits.  Requires that no other wave still reads that LDS region.
// mode: 0 store dtype (+bias, +res), 1 store fp32 (+bias), 2 fp32 +=, 3 fp32 partial
template <typename T, int NI, bool ROPE_AHEAD = false>
__device__ __forceinline__ void epilogue_block(const f32x16 *acc, float *lw, int m_base, int n_base,
                                               const KParams &p, int mode, int lane, bool staged = false) {
    constexpr int W = NI * 32;          // floats per row
    constexpr int CPR = W / 4;          // float4 chunks per row
    constexpr int RPP = 64 / CPR;       // rows per pass
    constexpr int PASSES = 32 / RPP;
    const int g = lane >> 5, l32 = lane & 31;
    if (!staged) {  // else the caller has already written the block into lw
#pragma unroll
        for (int j = 0; j < NI; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) lw[(8 * (r >> 2) + 4 * g + (r & 3)) * W + j * 32 + l32] = acc[j][r];
    }
    const int cc = lane % CPR, rr = lane / CPR;
    const int n = n_base + cc * 4;
    const bool nok = n < p.N;
    auto load_bias = [&](int col, bool ok) -> f32x4 {
        const Buf bb(p.bias);
        if constexpr (std::is_same<T, bf16>::value) {
            u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(bb.r, ok ? col * 2 : (int)0x80000000, 0, 0);
            return f32x4{__uint_as_float(w[0] << 16), __uint_as_float(w[0] & 0xffff0000u),
                         __uint_as_float(w[1] << 16), __uint_as_float(w[1] & 0xffff0000u)};
        } else {
            return __builtin_bit_cast(f32x4, bb.ld16(col * 4, ok));
        }
    };
    f32x4 bv = {0.f, 0.f, 0.f, 0.f};
    if ((mode == 0 || mode == 1) && p.bias) bv = load_bias(n, nok);
    // RoPE: the rotation partner of column n is n +- hd/2, in this wave's LDS
    // rows (the host only asks for it when a wave's columns hold whole heads)
    const bool rope = mode == 0 && p.rope_cs && n < p.rope_cols;
    const int rhalf = p.rope_hd / 2;
    const int ri = n % (p.rope_hd > 0 ? p.rope_hd : 1);
    const bool rlow = ri < rhalf;
    const int rk = rlow ? ri : ri - rhalf, roff = rlow ? rhalf : -rhalf;
    f32x4 bvp = {0.f, 0.f, 0.f, 0.f};
    if (rope && rhalf >= 4 && p.bias) bvp = load_bias(n + roff, nok);
    // residual / accumulate inputs for all passes first (uniform
    // branches outside the loops, so the loads issue back to back and are
    // waited for at first use).  Buffer offsets are taken from the first row of
    // this 32-row block, so they stay far below 2^31 bytes.
    f32x4 in[PASSES];
#pragma unroll
    for (int q = 0; q < PASSES; q++) in[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    const long long es = std::is_same<T, bf16>::value ? 2 : 4;
    if (mode == 0 && p.res) {
        const char *rb = static_cast<const char *>(p.res) + (long long)m_base * p.ldr * es;
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const int row = q * RPP + rr;
            in[q] = load_row4<T>(rb, (long long)row * p.ldr + n, nok && m_base + row < p.M);
        }
    } else if (mode == 2 || (mode == 3 && blockIdx.z == 0)) {
        // accumulate (split 0 of a split-K launch adds its partial into the
        // output here; the reduction adds splits 1 .. S-1 afterwards)
        const char *ob = static_cast<const char *>(p.out) + (long long)m_base * p.ldo * 4;
#pragma unroll
        for (int q = 0; q < PASSES; q++) {
            const int row = q * RPP + rr;
            in[q] = load_row4<float>(ob, (long long)row * p.ldo + n, nok && m_base + row < p.M);
        }
    }
    // RoPE table row of pass q: one modulo per call (a 32-row block wraps past
    // T at most once when T >= 32; rows past M still index a valid table row)
    const int rT = p.rope_T > 0 ? p.rope_T : 1;
    const int pos0 = rope ? (m_base + rr) % rT : 0;
    auto rpos = [&](int q) {
        const int x = pos0 + q * RPP;
        return rT >= 32 ? (x >= rT ? x - rT : x) : x % rT;
    };
    // ROPE_AHEAD: the (cos, sin) pairs of a batch of RB passes are loaded
    // before any of them is used (the output stores in between keep the
    // compiler from hoisting them itself)
    constexpr int RB = !ROPE_AHEAD ? PASSES : PASSES < 4 ? PASSES : 4;
#pragma unroll
    for (int qb = 0; qb < PASSES; qb += RB) {
    float2 rc[ROPE_AHEAD ? RB : 1][4];
    if constexpr (ROPE_AHEAD) {
        if (rope && rhalf >= 4) {
#pragma unroll
            for (int q = 0; q < RB; q++) {
                const float2 *cs = p.rope_cs + (long long)rpos(qb + q) * rhalf + rk;
#pragma unroll
                for (int e = 0; e < 4; e++) rc[q][e] = cs[e];
            }
        }
    }
#pragma unroll
    for (int q = qb; q < qb + RB; q++) {
        const int row = q * RPP + rr;
        const int m = m_base + row;
        f32x4 v = *reinterpret_cast<const f32x4 *>(lw + row * W + cc * 4);
        if (!(nok && m < p.M)) continue;
        if (mode == 0) {
            v = v + bv + in[q];
            if (rope) {
                const float2 *cs = p.rope_cs + (long long)rpos(q) * rhalf;
                if (rhalf >= 4) {
                    const f32x4 w = *reinterpret_cast<const f32x4 *>(lw + row * W + cc * 4 + roff) + bvp;
                    const float sg = rlow ? -1.f : 1.f;
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const float2 c = ROPE_AHEAD ? rc[ROPE_AHEAD ? q - qb : 0][e] : cs[rk + e];
                        v[e] = v[e] * c.x + sg * w[e] * c.y;
                    }
                } else {  // head width 4: pairs (0, 2), (1, 3) of the vector
                    const float2 c0 = cs[0], c1 = cs[1];
                    const f32x4 x = v;
                    v[0] = x[0] * c0.x - x[2] * c0.y;
                    v[2] = x[2] * c0.x + x[0] * c0.y;
                    v[1] = x[1] * c1.x - x[3] * c1.y;
                    v[3] = x[3] * c1.x + x[1] * c1.y;
                }
            }
            if constexpr (std::is_same<T, bf16>::value) {
                u32x2 w{pack2_bf16(v[0], v[1]), pack2_bf16(v[2], v[3])};
                *reinterpret_cast<u32x2 *>(reinterpret_cast<bf16 *>(p.out) + (long long)m * p.ldo + n) = w;
            } else {
                *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.out) + (long long)m * p.ldo + n) = v;
            }
        } else if (mode == 1) {
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.out) + (long long)m * p.ldo + n) = v + bv;
        } else if (mode == 2 || blockIdx.z == 0) {
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.out) + (long long)m * p.ldo + n) = v + in[q];
        } else {
            *reinterpret_cast<f32x4 *>(p.part + ((long long)(blockIdx.z - 1) * p.M + m) * p.N + n) = v;
        }
    }
    }
}

// SwiGLU forward epilogue of the 256 x 256 kernel (mode 5).  The two waves of
// a pair (same rows, wn = 0 and 1) hold the gate and the up columns of the same
// 128 hidden units; after a workgroup barrier each reads its partner's block
// from LDS.  Each wave stores its own values into out ([g | u] layout) and
// computes h = silu(g) u for half of the rows.  Every wave of the workgroup
// must call this the same number of times (two barriers per call).
__device__ __forceinline__ void epilogue_swiglu(const f32x16 *acc, float *lw, const float *lw_partner, int m_base,
                                                int col_base, bool gate_wave, const KParams &p, int lane,
                                                bool staged = false) {
    constexpr int W = 128, CPR = 32, RPP = 2, PASSES = 16;
    const int g = lane >> 5, l32 = lane & 31;
    if (!staged) {
#pragma unroll
        for (int j = 0; j < 4; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) lw[(8 * (r >> 2) + 4 * g + (r & 3)) * W + j * 32 + l32] = acc[j][r];
    }
    __syncthreads();
    const int cc = lane % CPR, rr = lane / CPR;
    const int n = col_base + cc * 4;  // hidden unit (gate column n, up column act_H + n)
    f32x4 bg = {0.f, 0.f, 0.f, 0.f}, bu = bg;
    if (p.bias) {
        bg = load_row4<bf16>(p.bias, n, true);
        bu = load_row4<bf16>(p.bias, (long long)p.act_H + n, true);
    }
    const f32x4 b_own = gate_wave ? bg : bu, b_par = gate_wave ? bu : bg;
    const int own_col = gate_wave ? n : p.act_H + n;
    const int q0 = gate_wave ? 0 : PASSES / 2;
#pragma unroll
    for (int q = 0; q < PASSES; q++) {
        const int row = q * RPP + rr;
        const int m = m_base + row;
        if (m >= p.M) continue;
        const f32x4 v = *reinterpret_cast<const f32x4 *>(lw + row * W + cc * 4) + b_own;
        store_row4<bf16>(p.out, (long long)m * p.ldo + own_col, v);
        if (q >= q0 && q < q0 + PASSES / 2) {
            const f32x4 w = *reinterpret_cast<const f32x4 *>(lw_partner + row * W + cc * 4) + b_par;
            const f32x4 gv = gate_wave ? v : w, uv = gate_wave ? w : v;
            f32x4 h;
#pragma unroll
            for (int e = 0; e < 4; e++)  // silu(g) u, sigmoid by the hardware reciprocal (1 ulp)
                h[e] = gv[e] * __builtin_amdgcn_rcpf(1.f + __expf(-gv[e])) * uv[e];
            store_row4<bf16>(p.act_h, (long long)m * p.act_H + n, h);
        }
    }
    __syncthreads();
}

template <typename T, int BM, int BN, bool AK, bool BKM>
__global__ __launch_bounds__(256) void gemm_kernel(KParams p) {
    constexpr int BK = GT<T>::BK;
    constexpr int MI = BM / 64, NI = BN / 64;
    constexpr int STAGE = (BM + BN) * 128;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int nm = (p.M + BM - 1) / BM, nn = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(nm, nn, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = blockIdx.z * p.kchunk;
    const int kend = min(p.K, kbeg + p.kchunk);
    const int nk = (kend - kbeg + BK - 1) / BK;

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1, g = lane >> 5, l32 = lane & 31;

    const T *A = reinterpret_cast<const T *>(p.A);
    const T *B = reinterpret_cast<const T *>(p.B);
    Loader<T, BM, AK> la;
    Loader<T, BN, BKM> lb;

    f32x16 acc[MI][NI];
#pragma unroll
    for (int i = 0; i < MI; i++)
#pragma unroll
        for (int j = 0; j < NI; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    if (nk > 0) {
        la.load(A, p.lda, m0, p.M, kbeg, kend);
        lb.load(B, p.ldb, n0, p.N, kbeg, kend);
        la.store(smem);
        lb.store(smem + BM * 128);
    }
    __syncthreads();

    for (int kt = 0; kt < nk; kt++) {
        const bool more = kt + 1 < nk;
        if (more) {
            int k0 = kbeg + (kt + 1) * BK;
            la.load(A, p.lda, m0, p.M, k0, kend);
            lb.load(B, p.ldb, n0, p.N, k0, kend);
        }
        const char *As = smem + (kt & 1) * STAGE;
        const char *Bs = As + BM * 128;
#pragma unroll
        for (int c = 0; c < 4; c++) {
            u32x4 af[MI], bfr[NI];
#pragma unroll
            for (int i = 0; i < MI; i++)
                af[i] = *reinterpret_cast<const u32x4 *>(As + swz(wm * (BM / 2) + i * 32 + l32, 2 * c + g));
#pragma unroll
            for (int j = 0; j < NI; j++)
                bfr[j] = *reinterpret_cast<const u32x4 *>(Bs + swz(wn * (BN / 2) + j * 32 + l32, 2 * c + g));
#pragma unroll
            for (int i = 0; i < MI; i++)
#pragma unroll
                for (int j = 0; j < NI; j++) mma_chunk(acc[i][j], af[i], bfr[j], T());
        }
        if (more) {
            char *nx = smem + ((kt + 1) & 1) * STAGE;
            la.store(nx);
            lb.store(nx + BM * 128);
        }
        __syncthreads();
    }

    // ---- epilogue (LDS is free after the last barrier) ----
    {
        constexpr int W = NI * 32;
        float *lw = reinterpret_cast<float *>(smem) + wave * 32 * W;
#pragma unroll
        for (int i = 0; i < MI; i++) {
            epilogue_block<T, NI>(acc[i], lw, m0 + wm * (BM / 2) + i * 32, n0 + wn * (BN / 2), p, p.out_mode, lane);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 256x256 kernel, direct-to-LDS pipeline.  8 waves (4 x 2), wave tile
// 64 x 128 (2 x 4 MFMA blocks), two waves per SIMD.  Every operand slab (32 k)
// is moved from global memory into LDS by buffer loads with the LDS bit (no
// VGPR staging), into a ring of four stages; slab k+3 is issued, spread over
// the MFMAs, while slab k is multiplied, and must have landed two steps later.
// The 16-byte chunk swizzles below were chosen by measurement (the LDS
// bank-conflict counter over the whole kernel reads zero with them; the
// unswizzled k-major layout, or a swizzle on row bits 0-1, conflicts).
// Permuting 16-byte chunks inside a row does not split the global requests.
// * k-major tiles: 256 rows x 64 B; chunk c of row r at c ^ ((r>>3)&3);
//   MFMA fragments are ds_read_b128 (16 B = 8 k of one row).
// * m/n-major tiles stay in their global orientation: 32 k-rows x 512 B;
//   chunk c of k-row r at c ^ (2(r&3) | 8(r&1)).  Fragments use the gfx950 transposing
//   read ds_read_b64_tr_b16: within each 16-lane group, lane l receives
//   elements l, l+16, l+32, l+48 of the 4x16 block the group reads, so with
//   lane i pointing at (k0 + i/4, m0 + 4(i%4)) each lane gets 4 consecutive k
//   of its own m; two such reads give the 8 k an MFMA lane needs.
// * The swizzles are applied by permuting which global chunk each lane DMAs.
// * Stages are four distinct __shared__ objects and the loop is unrolled by 4
//   so that the compiler's alias analysis keeps its LDS-DMA waits per stage;
//   the barrier is issued as a bare s_barrier after an explicit wait for this
//   wave's DMAs of the stage about to be read (a compiler barrier would also
//   wait for the slabs still in flight).
// ---------------------------------------------------------------------------
__shared__ __attribute__((aligned(16))) char g_dma_st0[32768];
__shared__ __attribute__((aligned(16))) char g_dma_st1[32768];
__shared__ __attribute__((aligned(16))) char g_dma_st2[32768];
__shared__ __attribute__((aligned(16))) char g_dma_st3[32768];

template <int S> __device__ __forceinline__ char *dma_stage() {
    if constexpr (S == 0) return g_dma_st0;
    else if constexpr (S == 1) return g_dma_st1;
    else if constexpr (S == 2) return g_dma_st2;
    else return g_dma_st3;
}

typedef __attribute__((address_space(3))) void *lds_vptr;
typedef short __attribute__((ext_vector_type(4))) s16x4;

__device__ __forceinline__ int kmaj_swz(int r) { return (r >> 3) & 3; }
__device__ __forceinline__ int mmaj_swz(int kr) { return ((kr & 3) << 1) | ((kr & 1) << 3); }
__device__ __forceinline__ int kmaj_off(int r, int c) { return r * 64 + ((c ^ kmaj_swz(r)) << 4); }
__device__ __forceinline__ int mmaj_off(int kr, int c) { return kr * 512 + ((c ^ mmaj_swz(kr)) << 4); }

// issue this wave's BPW 1 KB DMA instructions for one operand slab; the
// buffer resource is rebased on the slab so offsets stay small
template <bool KMAJOR, int BPW>
__device__ __forceinline__ void dma_slab(char *region, const bf16 *base, long long ld, int row0, int nrows, int k0,
                                         int kend, int wave, int lane) {
    const Buf buf(KMAJOR ? base + (long long)row0 * ld + k0 : base + (long long)k0 * ld + row0);
#pragma unroll
    for (int q = 0; q < BPW; q++) {
        const int blk = wave * BPW + q;  // 16 blocks of 1 KB, BPW per wave
        int off;
        bool ok;
        if constexpr (KMAJOR) {
            const int r = blk * 16 + (lane >> 2), pc = lane & 3;
            const int c = pc ^ kmaj_swz(r);
            ok = row0 + r < nrows && k0 + c * 8 < kend;
            off = (r * (int)ld + c * 8) * 2;
        } else {
            const int kr = blk * 2 + (lane >> 5), pc = lane & 31;
            const int c = pc ^ mmaj_swz(kr);
            ok = k0 + kr < kend && row0 + c * 8 < nrows;
            off = (kr * (int)ld + c * 8) * 2;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(buf.r, (lds_vptr)(region + blk * 1024), 16,
                                                 ok ? off : (int)0x80000000, 0, 0, 0);
    }
}

// MFMA fragment (8 bf16 along k) of row `r` of a tile, k16 step s (0..1), lane half g
template <bool KMAJOR>
__device__ __forceinline__ bf16x8 dma_frag(const char *region, int r, int s, int lane) {
    if constexpr (KMAJOR) {
        const int g = lane >> 5;
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(region + kmaj_off(r, 2 * s + g)));
    } else {
        // lane i16 of each 16-lane group reads (k = kb + i16/4, m = mb + 4 (i16%4))
        const int g = lane >> 5, i16 = lane & 15;
        const int mb = (r & ~15);                 // first row of this lane's 16-row group
        const int m = mb + 4 * (i16 & 3);
        const int kb = 16 * s + 8 * g + (i16 >> 2);
        const char *p0 = region + mmaj_off(kb, m >> 3) + (m & 7) * 2;
        const char *p1 = region + mmaj_off(kb + 4, m >> 3) + (m & 7) * 2;
        s16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p0);
        s16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p1);
        typedef short __attribute__((ext_vector_type(8))) s16x8;
        s16x8 v = __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(bf16x8, v);
    }
}

// s_waitcnt immediate for vmcnt(n) lgkmcnt(0) (vmcnt bits [3:0] and [15:14],
// expcnt [6:4] left at its maximum, lgkmcnt [11:8])
constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }
// the same with lgkmcnt(l) (l <= 15)
constexpr int wait_vm_lgkm(int n, int l) { return wait_vm_lgkm0(n) | ((l & 15) << 8); }

// NW waves: 8 -> 4 x 2 waves of 64 x 128, 4 -> 2 x 2 waves of 128 x 128.
template <bool AK, bool BKM, int MODE, int NW>
__global__ __launch_bounds__(NW * 64) void gemm_dma_kernel(KParams p) {
    constexpr int BM = 256, BN = 256, BK = 32;
    constexpr int WGN = 2, WGM = NW / WGN, TM = BM / WGM, FI = TM / 32, FJ = 4;
    constexpr int NDW = NW / 2;           // waves that issue the DMA (one per SIMD)
    constexpr int BPD = 16 / NDW;         // DMA blocks per operand per DMA wave
    const int nm = (p.M + BM - 1) / BM, nn = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(nm, nn, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = blockIdx.z * p.kchunk;
    const int kend = min(p.K, kbeg + p.kchunk);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WGN, wn = wave % WGN, l32 = lane & 31;
    const bf16 *gA = static_cast<const bf16 *>(p.A), *gB = static_cast<const bf16 *>(p.B);

    f32x16 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; i++)
#pragma unroll
        for (int j = 0; j < FJ; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    // mode 5: B rows 0..127 of the tile are gate rows tn*128.., rows 128..255
    // the up rows act_H + tn*128.. (each wave's DMA blocks lie in one half)
    const bool dmaw = wave < NDW;
    const int nb0 = MODE == 5 ? (wave < NDW / 2 ? tn * 128 : p.act_H + tn * 128 - 128) : n0;
    auto issue = [&](char *st, int k0) {
        if (dmaw) {
            dma_slab<AK, BPD>(st, gA, p.lda, m0, p.M, k0, kend, wave, lane);
            dma_slab<BKM, BPD>(st + 16384, gB, p.ldb, nb0, p.N, k0, kend, wave, lane);
        }
    };
    auto frags = [&](const char *st, int sidx, bf16x8 *af, bf16x8 *bfr) {
        const char *As = st, *Bs = st + 16384;
#pragma unroll
        for (int i = 0; i < FI; i++) af[i] = dma_frag<AK>(As, wm * TM + i * 32 + l32, sidx, lane);
#pragma unroll
        for (int j = 0; j < FJ; j++) bfr[j] = dma_frag<BKM>(Bs, wn * 128 + j * 32 + l32, sidx, lane);
    };
    auto mma = [&](const bf16x8 *af, const bf16x8 *bfr) {
#pragma unroll
        for (int i = 0; i < FI; i++)
#pragma unroll
            for (int j = 0; j < FJ; j++) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    };
    auto compute = [&](const char *st) {
        bf16x8 af[FI], bfr[FJ];
        frags(st, 0, af, bfr);
        mma(af, bfr);
        frags(st, 1, af, bfr);
        mma(af, bfr);
    };
    // Main loop: whole groups of four slabs.  One wave per SIMD (waves
    // 0 .. NW/2-1) issues the whole operand DMA and the other wave of the SIMD
    // none, so that one never stalls on a full texture-address FIFO and keeps
    // the MFMAs fed (measured 1-3 % faster than every wave issuing a share).
    // Step k waits until the DMA of slab k+1 has landed (only slab k+2 may
    // still be in flight), and
    // the barrier makes that true for every wave and retires every wave's
    // reads of slab k-1, whose stage the step then refills with slab k+3.
    // The fragments of slab k's first k16 step were read during step k-1, so
    // no LDS latency follows the barrier.  Inside the step the DMA
    // instructions and the next fragment reads are spread evenly over the
    // MFMAs (issuing the DMA as one burst after the barrier filled the
    // texture-address FIFO and stalled the issuing waves: measured 5-13 %
    // slower).  Past the end of K the loads are out of range and write zeros
    // into a stage that is no longer read, so every step has the same count.
    bf16x8 fa[FI], fb[FJ];
    // LDS reads of one k16 step and DMA instructions of one operand slab,
    // spread evenly over the 8 MFMAs of the other fragment set
    constexpr int NRD = FI * (AK ? 1 : 2) + FJ * (BKM ? 1 : 2);
    constexpr int NMM = FI * FJ;
    // one younger slab in flight; the last NRD LDS reads (the next slab's
    // first fragments, issued at the end of the previous step) may still be in
    // flight: the barrier only needs the reads of the stage it frees
    static_assert(NRD <= 15, "lgkmcnt field");
    constexpr int WAIT1 = wait_vm_lgkm(2 * BPD, NRD);
#define PIPE_PATTERN(NVM)                                                       \
    {                                                                           \
        _Pragma("unroll") for (int q = 0; q < NMM; q++) {                       \
            const int nr = ((q + 1) * NRD) / NMM - (q * NRD) / NMM;              \
            if (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      \
            if (nr > 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      \
            const int nv = ((q + 1) * (NVM)) / NMM - (q * (NVM)) / NMM;          \
            if (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  \
        }                                                                       \
    }
#define DMA_STEP(S, D)                                                          \
    {                                                                           \
        __builtin_amdgcn_s_waitcnt(WAIT1);                                      \
        asm volatile("s_barrier" ::: "memory");                                 \
        __builtin_amdgcn_sched_barrier(0);                                      \
        bf16x8 ga[FI], gb[FJ];                                                  \
        const int k3 = kbeg + (kt + S + 3) * BK;                                \
        if (D) dma_slab<AK, BPD>(dma_stage<(S + 3) & 3>(), gA, p.lda, m0, p.M, k3, kend, wave, lane); \
        frags(dma_stage<S>(), 1, ga, gb);                                       \
        mma(fa, fb);                                                            \
        PIPE_PATTERN((D) ? BPD : 0)                                             \
        __builtin_amdgcn_sched_barrier(0);                                      \
        if (D) dma_slab<BKM, BPD>(dma_stage<(S + 3) & 3>() + 16384, gB, p.ldb, nb0, p.N, k3, kend, wave, lane); \
        frags(dma_stage<(S + 1) & 3>(), 0, fa, fb);                             \
        mma(ga, gb);                                                            \
        PIPE_PATTERN((D) ? BPD : 0)                                             \
        __builtin_amdgcn_sched_barrier(0);                                      \
    }
    issue(dma_stage<0>(), kbeg);
    issue(dma_stage<1>(), kbeg + BK);
    issue(dma_stage<2>(), kbeg + 2 * BK);
    __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(4 * BPD));
    asm volatile("s_barrier" ::: "memory");
    frags(dma_stage<0>(), 0, fa, fb);
    // one wave per SIMD issues the whole DMA, so the other wave of the SIMD
    // never stalls on the texture-address FIFO and keeps the MFMAs fed
    int kt = 0;
    if (dmaw) {
        for (; kt + 4 <= nk; kt += 4) {
            DMA_STEP(0, true)
            DMA_STEP(1, true)
            DMA_STEP(2, true)
            DMA_STEP(3, true)
        }
    } else {
        for (; kt + 4 <= nk; kt += 4) {
            DMA_STEP(0, false)
            DMA_STEP(1, false)
            DMA_STEP(2, false)
            DMA_STEP(3, false)
        }
    }
#undef DMA_STEP
#undef PIPE_PATTERN
    // tail of 0..3 slabs, all already issued; the first k16 step of slab kt is in fa/fb
    if (kt < nk) {
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(0));
        asm volatile("s_barrier" ::: "memory");
        mma(fa, fb);
        frags(dma_stage<0>(), 1, fa, fb);
        mma(fa, fb);
        if (kt + 1 < nk) compute(dma_stage<1>());
        if (kt + 2 < nk) compute(dma_stage<2>());
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- epilogue through LDS (16 KB per wave; all DMA has landed and all reads are done)
    {
        constexpr int PER_STAGE = NW / 4;  // waves sharing one 32 KB stage
        auto region = [&](int w) {
            const int sidx = w / PER_STAGE;
            char *reg = sidx == 0 ? dma_stage<0>() : sidx == 1 ? dma_stage<1>() : sidx == 2 ? dma_stage<2>() : dma_stage<3>();
            return reinterpret_cast<float *>(reg + (w % PER_STAGE) * 16384);
        };
        float *lw = region(wave);
        if constexpr (MODE == 5) {
            const float *lp = region(wave ^ 1);
#pragma unroll
            for (int i = 0; i < FI; i++)
                epilogue_swiglu(acc[i], lw, lp, m0 + wm * TM + i * 32, tn * 128, wn == 0, p, lane);
        } else {
#pragma unroll
            for (int i = 0; i < FI; i++)
                epilogue_block<bf16, 4>(acc[i], lw, m0 + wm * TM + i * 32, n0 + wn * 128, p, MODE, lane);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 256x256 kernel on 64-k slabs.  The same 8-wave tiling, fragments and
// epilogue as gemm_dma_kernel, but every operand slab is 64 k deep, so a
// k-major tile row is 128 bytes: one DMA instruction moves 8 whole 128-byte
// rows (every lane's 16 bytes in a fully used cache line) instead of 16
// half-filled ones.  A stream of such slabs alone runs 23-31 % faster than the
// 64-byte-row stream of the 32-k kernel, and that stream is what bounds the
// 32-k main loop.  m/n-major tiles hold 64 k-rows x 512 bytes (2 k-rows per
// instruction, as before).
// LDS: a ring of five 32 KB units (the whole 160 KB), each one operand of one
// slab: slab j has A in unit 2j mod 5 and B in unit 2j+1 mod 5.  At the
// barrier that opens step j (slab j landed, every wave done reading slab
// j-1) the two units of slab j-1 are free: B of slab j+1 goes into one and A
// of slab j+2 into the other, so B is issued one step (64 k) and A two steps
// ahead of their use.  The last k16 fragments of slab j-1 are read before the
// barrier and multiplied after it, while slab j's first fragments load.
// ---------------------------------------------------------------------------
__shared__ __attribute__((aligned(16))) char g_k64_u0[32768];
__shared__ __attribute__((aligned(16))) char g_k64_u1[32768];
__shared__ __attribute__((aligned(16))) char g_k64_u2[32768];
__shared__ __attribute__((aligned(16))) char g_k64_u3[32768];
__shared__ __attribute__((aligned(16))) char g_k64_u4[32768];

template <int U> __device__ __forceinline__ char *k64_unit() {
    if constexpr (U == 0) return g_k64_u0;
    else if constexpr (U == 1) return g_k64_u1;
    else if constexpr (U == 2) return g_k64_u2;
    else if constexpr (U == 3) return g_k64_u3;
    else return g_k64_u4;
}

// 128-byte k-major rows: chunk c of row r at c ^ ((r >> 1) & 7) (the 16-byte
// fragment reads of one access group then hit distinct banks)
__device__ __forceinline__ int k64_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int k64_off(int r, int c) { return r * 128 + ((c ^ k64_swz(r)) << 4); }

// this wave's BPW 1 KB DMA instructions of one 64-k operand slab (32 KB)
template <bool KMAJOR, int BPW>
__device__ __forceinline__ void dma_slab64(char *unit, const bf16 *base, long long ld, int row0, int nrows, int k0,
                                           int kend, int wave, int lane) {
    const Buf buf(KMAJOR ? base + (long long)row0 * ld + k0 : base + (long long)k0 * ld + row0);
#pragma unroll
    for (int q = 0; q < BPW; q++) {
        const int blk = wave * BPW + q;  // 32 blocks of 1 KB
        int off;
        bool ok;
        if constexpr (KMAJOR) {
            const int r = blk * 8 + (lane >> 3), pc = lane & 7;
            const int c = pc ^ k64_swz(r);
            ok = row0 + r < nrows && k0 + c * 8 < kend;
            off = (r * (int)ld + c * 8) * 2;
        } else {
            const int kr = blk * 2 + (lane >> 5), pc = lane & 31;
            const int c = pc ^ mmaj_swz(kr);
            ok = k0 + kr < kend && row0 + c * 8 < nrows;
            off = (kr * (int)ld + c * 8) * 2;
        }
        __builtin_amdgcn_raw_ptr_buffer_load_lds(buf.r, (lds_vptr)(unit + blk * 1024), 16,
                                                 ok ? off : (int)0x80000000, 0, 0, 0);
    }
}

// The same DMA with the per-lane offsets computed once per tile.  When K is a
// multiple of 64 no slab is cut short in k, so a lane's offset from its slab
// base depends only on its row (validity included) and never changes from
// slab to slab; the k limit is left to the buffer's record count: slabs past
// kend get a record of 0 bytes (every load reads zeros), and for m/n-major
// operands, whose rows are k, a record of the (kend - k0) rows still in range.
// Issuing a slab is then scalar work (base, record, LDS address) only.
template <bool KMAJOR>
__device__ __forceinline__ void slab64_offsets(int *voff, long long ld, int row0, int nrows, int wave, int lane) {
#pragma unroll
    for (int q = 0; q < 8; q++) {
        const int blk = wave * 8 + q;
        int off;
        bool ok;
        if constexpr (KMAJOR) {
            const int r = blk * 8 + (lane >> 3), c = (lane & 7) ^ k64_swz(r);
            ok = row0 + r < nrows;
            off = (r * (int)ld + c * 8) * 2;
        } else {
            const int kr = blk * 2 + (lane >> 5), c = (lane & 31) ^ mmaj_swz(kr);
            ok = row0 + c * 8 < nrows;
            off = (kr * (int)ld + c * 8) * 2;
        }
        voff[q] = ok ? off : (int)0x80000000;
    }
}
template <bool KMAJOR, int N>
__device__ __forceinline__ void dma_slab64_pre(char *unit, const bf16 *base, long long ld, int row0, int k0, int kend,
                                               const int *voff, int q0, int wave) {
    const bf16 *g = KMAJOR ? base + (long long)row0 * ld + k0 : base + (long long)k0 * ld + row0;
    long long nb = 0;
    if (k0 < kend) nb = KMAJOR ? 0x7fffffffLL : (long long)(kend - k0) * ld * 2;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16 *>(g), (short)0, (int)(nb < 0x7fffffffLL ? nb : 0x7fffffffLL), 0x00020000);
#pragma unroll
    for (int i = 0; i < N; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(unit + (wave * 8 + q0 + i) * 1024), 16, voff[q0 + i], 0,
                                                 0, 0);
}

// MFMA fragment of row r, k16 step s (0..3) of a 64-k unit
template <bool KMAJOR>
__device__ __forceinline__ bf16x8 k64_frag(const char *unit, int r, int s, int lane) {
    if constexpr (KMAJOR) {
        return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(unit + k64_off(r, 2 * s + (lane >> 5))));
    } else {
        return dma_frag<false>(unit, r, s, lane);  // k-rows 16 s .. 16 s + 15 of the 64
    }
}

// PRE: K is a multiple of 64 and the DMA offsets are computed once per tile
template <bool AK, bool BKM, int MODE, bool PRE>
__global__ __launch_bounds__(512) void gemm_k64_kernel(KParams p) {
    constexpr int NW = 8, BM = 256, BN = 256, BK = 64;
    constexpr int WGN = 2, TM = 64, FI = 2, FJ = 4;
    constexpr int NDW = 4;               // waves that issue the DMA (one per SIMD)
    constexpr int BPD = 32 / NDW;        // 1 KB blocks per operand slab per DMA wave
    const int nm = (p.M + BM - 1) / BM, nn = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(nm, nn, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = blockIdx.z * p.kchunk;
    const int kend = min(p.K, kbeg + p.kchunk);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WGN, wn = wave % WGN, l32 = lane & 31;
    const bf16 *gA = static_cast<const bf16 *>(p.A), *gB = static_cast<const bf16 *>(p.B);

    f32x16 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; i++)
#pragma unroll
        for (int j = 0; j < FJ; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) acc[i][j][r] = 0.f;

    const bool dmaw = wave < NDW;
    // mode 5: B rows 0..127 are gate rows tn*128.., rows 128..255 the up rows
    // act_H + tn*128.. (DMA waves 0-1 load the first half, 2-3 the second)
    const int nb0 = MODE == 5 ? (wave < NDW / 2 ? tn * 128 : p.act_H + tn * 128 - 128) : n0;
    auto frags = [&](const char *ua, const char *ub, int sidx, bf16x8 *af, bf16x8 *bfr) {
#pragma unroll
        for (int i = 0; i < FI; i++) af[i] = k64_frag<AK>(ua, wm * TM + i * 32 + l32, sidx, lane);
#pragma unroll
        for (int j = 0; j < FJ; j++) bfr[j] = k64_frag<BKM>(ub, wn * 128 + j * 32 + l32, sidx, lane);
    };
    auto mma = [&](const bf16x8 *af, const bf16x8 *bfr) {
#pragma unroll
        for (int i = 0; i < FI; i++)
#pragma unroll
            for (int j = 0; j < FJ; j++) acc[i][j] = mfma32(af[i], bfr[j], acc[i][j]);
    };
    constexpr int NRD = FI * (AK ? 1 : 2) + FJ * (BKM ? 1 : 2);
    constexpr int NMM = FI * FJ;
    constexpr int NV = BPD / 2;  // DMA instructions per k16 group (one operand over two groups)
    // LDS reads of one k16 step and NVM DMA instructions spread evenly over 8 MFMAs
#define K64_PATTERN(NVM, FRONT)                                                 \
    {                                                                           \
        _Pragma("unroll") for (int q = 0; q < NMM; q++) {                       \
            const int nr = (FRONT) ? (2 * q < NRD ? (2 * q + 1 < NRD ? 2 : 1) : 0) \
                                   : ((q + 1) * NRD) / NMM - (q * NRD) / NMM;     \
            if (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      \
            if (nr > 1) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      \
            const int nv = ((q + 1) * (NVM)) / NMM - (q * (NVM)) / NMM;          \
            if (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);      \
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                  \
        }                                                                       \
    }
    // this DMA wave's per-lane slab offsets (PRE: once per tile)
    int voffA[PRE ? 8 : 1], voffB[PRE ? 8 : 1];
    if constexpr (PRE) {
        slab64_offsets<AK>(voffA, p.lda, m0, p.M, wave, lane);
        slab64_offsets<BKM>(voffB, p.ldb, nb0, p.N, wave, lane);
    }
    // half h of this wave's NV-instruction shares of the B (A) slab at k
#define DMA_B(unit, k, h)                                                                                        \
    {                                                                                                            \
        if constexpr (PRE) dma_slab64_pre<BKM, NV>(unit, gB, p.ldb, nb0, k, kend, voffB, (h) * NV, wave);        \
        else dma_slab64<BKM, NV>(unit, gB, p.ldb, nb0, p.N, k, kend, 2 * wave + (h), lane);                      \
    }
#define DMA_A(unit, k, h)                                                                                        \
    {                                                                                                            \
        if constexpr (PRE) dma_slab64_pre<AK, NV>(unit, gA, p.lda, m0, k, kend, voffA, (h) * NV, wave);          \
        else dma_slab64<AK, NV>(unit, gA, p.lda, m0, p.M, k, kend, 2 * wave + (h), lane);                        \
    }
    // one 64-k step: J = j mod 5 picks the units at compile time
#define K64_STEP(J, D)                                                          \
    {                                                                           \
        constexpr int UA = (2 * (J)) % 5, UB = (2 * (J) + 1) % 5;               \
        constexpr int NB = (2 * (J) + 3) % 5, NA = (2 * (J) + 4) % 5;           \
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(BPD));                         \
        asm volatile("s_barrier" ::: "memory");                                 \
        __builtin_amdgcn_sched_barrier(0);                                      \
        const int kb1 = kbeg + (j + 1) * BK, ka2 = kbeg + (j + 2) * BK;          \
        bf16x8 ga[FI], gb[FJ];                                                  \
        if (D) DMA_B(k64_unit<NB>(), kb1, 0)                                    \
        frags(k64_unit<UA>(), k64_unit<UB>(), 0, ga, gb);                       \
        mma(fa, fb);                                                            \
        K64_PATTERN((D) ? NV : 0, false)                                               \
        __builtin_amdgcn_sched_barrier(0);                                      \
        if (D) DMA_B(k64_unit<NB>(), kb1, 1)                                    \
        frags(k64_unit<UA>(), k64_unit<UB>(), 1, fa, fb);                       \
        mma(ga, gb);                                                            \
        K64_PATTERN((D) ? NV : 0, false)                                               \
        __builtin_amdgcn_sched_barrier(0);                                      \
        if (D) DMA_A(k64_unit<NA>(), ka2, 0)                                    \
        frags(k64_unit<UA>(), k64_unit<UB>(), 2, ga, gb);                       \
        mma(fa, fb);                                                            \
        K64_PATTERN((D) ? NV : 0, false)                                               \
        __builtin_amdgcn_sched_barrier(0);                                      \
        if (D) DMA_A(k64_unit<NA>(), ka2, 1)                                    \
        frags(k64_unit<UA>(), k64_unit<UB>(), 3, fa, fb);                       \
        mma(ga, gb);                                                            \
        K64_PATTERN((D) ? NV : 0, true)                                                \
        __builtin_amdgcn_sched_barrier(0);                                      \
        ++j;                                                                    \
    }
    // prologue: A of slabs 0 and 1, B of slab 0 (B of slab 1 and A of slab 2
    // go out in step 0).  The k16 fragments multiplied first in step 0
    // belong to no slab and are zero.
    if (dmaw) {
        if constexpr (PRE) {
            dma_slab64_pre<AK, BPD>(k64_unit<0>(), gA, p.lda, m0, kbeg, kend, voffA, 0, wave);
            dma_slab64_pre<BKM, BPD>(k64_unit<1>(), gB, p.ldb, nb0, kbeg, kend, voffB, 0, wave);
            dma_slab64_pre<AK, BPD>(k64_unit<2>(), gA, p.lda, m0, kbeg + BK, kend, voffA, 0, wave);
        } else {
            dma_slab64<AK, BPD>(k64_unit<0>(), gA, p.lda, m0, p.M, kbeg, kend, wave, lane);
            dma_slab64<BKM, BPD>(k64_unit<1>(), gB, p.ldb, nb0, p.N, kbeg, kend, wave, lane);
            dma_slab64<AK, BPD>(k64_unit<2>(), gA, p.lda, m0, p.M, kbeg + BK, kend, wave, lane);
        }
    }
    bf16x8 fa[FI], fb[FJ];
#pragma unroll
    for (int i = 0; i < FI; i++) fa[i] = bf16x8{};
#pragma unroll
    for (int j = 0; j < FJ; j++) fb[j] = bf16x8{};
    int j = 0;
    if (nk > 0) {
        // every step issues the same number of DMA instructions (past the end
        // of K they load zeros into free units), so the wait count is uniform.
        // Whole groups of five steps, then up to four more (a loop with an
        // exit after every step made the compiler spill the accumulators).
        if (dmaw) {
            for (; j + 5 <= nk;) {
                K64_STEP(0, true)
                K64_STEP(1, true)
                K64_STEP(2, true)
                K64_STEP(3, true)
                K64_STEP(4, true)
            }
            if (j < nk) K64_STEP(0, true)
            if (j < nk) K64_STEP(1, true)
            if (j < nk) K64_STEP(2, true)
            if (j < nk) K64_STEP(3, true)
        } else {
            for (; j + 5 <= nk;) {
                K64_STEP(0, false)
                K64_STEP(1, false)
                K64_STEP(2, false)
                K64_STEP(3, false)
                K64_STEP(4, false)
            }
            if (j < nk) K64_STEP(0, false)
            if (j < nk) K64_STEP(1, false)
            if (j < nk) K64_STEP(2, false)
            if (j < nk) K64_STEP(3, false)
        }
        mma(fa, fb);  // last k16 step of the last slab
    }
#undef K64_STEP
#undef DMA_A
#undef DMA_B
#undef K64_PATTERN
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- epilogue through LDS (16 KB per wave in units 0-3)
    {
        auto region = [&](int w) {
            const int u = w >> 1;
            char *reg = u == 0 ? k64_unit<0>() : u == 1 ? k64_unit<1>() : u == 2 ? k64_unit<2>() : k64_unit<3>();
            return reinterpret_cast<float *>(reg + (w & 1) * 16384);
        };
        float *lw = region(wave);
        if constexpr (MODE == 5) {
            const float *lp = region(wave ^ 1);
#pragma unroll
            for (int i = 0; i < FI; i++)
                epilogue_swiglu(acc[i], lw, lp, m0 + wm * TM + i * 32, tn * 128, wn == 0, p, lane);
        } else {
#pragma unroll
            for (int i = 0; i < FI; i++)
                epilogue_block<bf16, 4>(acc[i], lw, m0 + wm * TM + i * 32, n0 + wn * 128, p, MODE, lane);
        }
    }
}

// ---------------------------------------------------------------------------
// bf16 256x256 kernel for two k-major operands (the forward projections) on
// v_mfma_f32_16x16x32_bf16.  The tiles, 64-k slabs, five-unit LDS ring, DMA
// schedule and epilogue are those of gemm_k64_kernel; each wave's 64 x 128
// block is 4 x 8 MFMA blocks of 16 x 16 and a slab is two k32 steps (12
// fragment reads, 32 MFMAs).  Measured on the MLP-up shape, the 16x16x32 form
// lets the chip hold a higher clock under its power limit (the 32x32x16 form
// moves twice the accumulator registers per flop): sustained 1305-1324
// against 1248-1260 TFLOP/s, about 1880 against 1690-1730 MHz, and the sums
// come out bit-identical (each output is the same fp32 chain of 64-k dot
// products).
// * Register budget (two waves per SIMD: 256 per wave): 128 accumulators;
//   fragments of the next k32 step are read while the current one is
//   multiplied, column pair by column pair (A blocks double-buffered, the B
//   blocks of the next step only after the same blocks of the current step are
//   done), 18 fragments at most; the DMA offsets are per-lane pattern values.
// ---------------------------------------------------------------------------
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Lane offsets of the 16x16x32 fragments of a k-major 64-k unit: the A (B)
// operand lane l supplies row (column) l % 16 of a 16-row block and k
// 8 (l / 16) .. + 7 of the k32 step.  Row block b sits at + 2048 b (16 rows of
// 128 bytes; the chunk swizzle depends on row bits 1-3 only), so a lane needs
// one offset per k32 step: lc0 for k 0..31, lc1 for k 32..63.
__device__ __forceinline__ void frag16_lane(int row0, int lane, int &lc0, int &lc1) {
    const int r = row0 + (lane & 15);  // row0 a multiple of 16
    lc0 = k64_off(r, lane >> 4);
    lc1 = k64_off(r, 4 + (lane >> 4));
}
__device__ __forceinline__ bf16x8 frag16(const char *unit, int s, int b, int lc0, int lc1) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(unit + b * 2048 + (s ? lc1 : lc0)));
}

// DMA of one k-major 64-k slab (32 KB, 32 blocks of 1 KB: 8 rows x 128 bytes)
// by one of four DMA waves (8 blocks each), K a multiple of 64.  A lane's
// offset in block q is its row-in-block and swizzled chunk, which depend on q
// only through q mod 2 (the swizzle takes row bits 1-3), plus q's first row:
// the two pattern values vpat[] are computed once per tile.  Rows past the
// tile's last valid row (nrows) and slabs past kend are cut off by the
// buffer's record count (zeros land in LDS).
__device__ __forceinline__ void slab16_pattern(int *vpat, long long ld, int lane) {
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int r = q * 8 + (lane >> 3), c = (lane & 7) ^ k64_swz(r);
        vpat[q] = ((lane >> 3) * (int)ld + c * 8) * 2;
    }
}
__device__ __forceinline__ void dma_slab16(char *unit, const bf16 *base, long long ld, int row0, int nrows, int k0,
                                           int kend, const int *vpat, int wave) {
    const bf16 *g = base + (long long)row0 * ld + k0;
    // last valid byte: row (min(nrows - row0, 256) - 1), chunk 7, when k0 + 64 <= ld
    long long nb = 0;
    if (k0 < kend) nb = (long long)(min(nrows - row0, 256) - 1) * ld * 2 + 128;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16 *>(g), (short)0, (int)(nb < 0x7fffffffLL ? nb : 0x7fffffffLL), 0x00020000);
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const int blk = wave * 8 + i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(unit + blk * 1024), 16,
                                                 vpat[i & 1] + blk * 16 * (int)ld, 0, 0, 0);
    }
}

// rows 0..31 x columns 0..127 of a wave's 16x16 accumulators acc[2][8]
// (lane l, element e: row 4 (l / 16) + e, column l % 16 of its block) into lw [32][128]
__device__ __forceinline__ void stage16(const f32x4 *acc, float *lw, int lane) {
    const int g = lane >> 4, c = lane & 15;
#pragma unroll
    for (int bi = 0; bi < 2; bi++)
#pragma unroll
        for (int bj = 0; bj < 8; bj++)
#pragma unroll
            for (int e = 0; e < 4; e++) lw[(bi * 16 + 4 * g + e) * 128 + bj * 16 + c] = acc[bi * 8 + bj][e];
}

// K a multiple of 64 and one split (kbeg = 0, kend = K)
template <int MODE>
__global__ __launch_bounds__(512) void gemm_k64m16_kernel(KParams p) {
    constexpr int BM = 256, BN = 256, BK = 64;
    constexpr int WGN = 2, TM = 64, FI = 4, FJ = 8;
    constexpr int NDW = 4;   // waves that issue the DMA (one per SIMD)
    constexpr int BPD = 8;   // 1 KB blocks per operand slab per DMA wave
    const int nm = (p.M + BM - 1) / BM, nn = (p.N + BN - 1) / BN;
    int tm, tn;
    tile_coords(nm, nn, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int kbeg = blockIdx.z * p.kchunk;
    const int kend = min(p.K, kbeg + p.kchunk);
    const int nk = kend > kbeg ? (kend - kbeg + BK - 1) / BK : 0;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave / WGN, wn = wave % WGN;
    const bf16 *gA = static_cast<const bf16 *>(p.A), *gB = static_cast<const bf16 *>(p.B);

    f32x4 acc[FI][FJ];
#pragma unroll
    for (int i = 0; i < FI; i++)
#pragma unroll
        for (int j = 0; j < FJ; j++) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const bool dmaw = wave < NDW;
    // mode 5: B rows 0..127 are gate rows tn*128.., rows 128..255 the up rows
    // act_H + tn*128.. (DMA waves 0-1 load the first half, 2-3 the second)
    const int nb0 = MODE == 5 ? (wave < NDW / 2 ? tn * 128 : p.act_H + tn * 128 - 128) : n0;
    int la0, la1, lb0, lb1;
    frag16_lane(wm * TM, lane, la0, la1);
    frag16_lane(wn * 128, lane, lb0, lb1);
    // the 8 MFMAs of column pair g (B blocks 2g, 2g+1)
    auto mma_pair = [&](const bf16x8 *af, const bf16x8 *bfr, int g) {
#pragma unroll
        for (int i = 0; i < FI; i++) {
            acc[i][2 * g] = mfma16(af[i], bfr[2 * g], acc[i][2 * g]);
            acc[i][2 * g + 1] = mfma16(af[i], bfr[2 * g + 1], acc[i][2 * g + 1]);
        }
    };
    // multiply the current k32 step (ca, cb) column pair by column pair while
    // the next step's fragments (na, nb) are read from units ua / ub
    auto phase = [&](const bf16x8 *ca, const bf16x8 *cb, bf16x8 *na, bf16x8 *nb, const char *ua, const char *ub,
                     int sidx) {
        // the lane offsets pass through an empty asm, so the addresses of the
        // five units (beyond the 64 KB reach of a read's immediate offset) are
        // formed here instead of being hoisted out of the loop as live registers
        asm volatile("" : "+v"(la0), "+v"(la1), "+v"(lb0), "+v"(lb1));
        na[0] = frag16(ua, sidx, 0, la0, la1);
        na[1] = frag16(ua, sidx, 1, la0, la1);
        mma_pair(ca, cb, 0);
        nb[0] = frag16(ub, sidx, 0, lb0, lb1);
        nb[1] = frag16(ub, sidx, 1, lb0, lb1);
        na[2] = frag16(ua, sidx, 2, la0, la1);
        mma_pair(ca, cb, 1);
        nb[2] = frag16(ub, sidx, 2, lb0, lb1);
        nb[3] = frag16(ub, sidx, 3, lb0, lb1);
        na[3] = frag16(ua, sidx, 3, la0, la1);
        if (sidx) {  // before the barrier: the last pair is read one group early
            nb[6] = frag16(ub, sidx, 6, lb0, lb1);
            nb[7] = frag16(ub, sidx, 7, lb0, lb1);
        }
        mma_pair(ca, cb, 2);
        nb[4] = frag16(ub, sidx, 4, lb0, lb1);
        nb[5] = frag16(ub, sidx, 5, lb0, lb1);
        if (!sidx) {
            nb[6] = frag16(ub, sidx, 6, lb0, lb1);
            nb[7] = frag16(ub, sidx, 7, lb0, lb1);
        }
        mma_pair(ca, cb, 3);
    };
    // fragment reads per column-pair group (2, 3, 3, 4) and NVM DMA
    // instructions spread over the 32 MFMAs of a phase
#define M16_PATTERN(NVM, LATE)                                                  \
    {                                                                           \
        _Pragma("unroll") for (int g = 0; g < 4; g++) {                         \
            const int nrg = g == 0 ? 2 : g == 1 ? 3 : g == 2 ? ((LATE) ? 3 : 5) : ((LATE) ? 4 : 2); \
            _Pragma("unroll") for (int q = 0; q < 8; q++) {                     \
                const int nr = (!(LATE) && g == 3) ? (q < nrg ? 1 : 0)          \
                                                   : ((q + 1) * nrg) / 8 - (q * nrg) / 8; \
                if (nr > 0) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  \
                const int qq = g * 8 + q;                                       \
                const int nv = ((qq + 1) * (NVM)) / 32 - (qq * (NVM)) / 32;     \
                if (nv > 0) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  \
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              \
            }                                                                   \
        }                                                                       \
    }
    int vpA[2], vpB[2];
    slab16_pattern(vpA, p.lda, lane);
    slab16_pattern(vpB, p.ldb, lane);
    // one 64-k step: J = j mod 5 picks the units at compile time (the same
    // ring as gemm_k64_kernel: B of slab j+1 and A of slab j+2 go into the
    // units of slab j-1, freed at the barrier that opens step j)
#define M16_STEP(J, D)                                                                          \
    {                                                                                           \
        constexpr int UA = (2 * (J)) % 5, UB = (2 * (J) + 1) % 5;                               \
        constexpr int NB = (2 * (J) + 3) % 5, NA = (2 * (J) + 4) % 5;                           \
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0(BPD));                                         \
        asm volatile("s_barrier" ::: "memory");                                                 \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        const int kb1 = kbeg + (j + 1) * BK, ka2 = kbeg + (j + 2) * BK;                          \
        bf16x8 ga[FI], gb[FJ];                                                                  \
        if (D) dma_slab16(k64_unit<NB>(), gB, p.ldb, nb0, p.N, kb1, kend, vpB, wave);           \
        phase(fa, fb, ga, gb, k64_unit<UA>(), k64_unit<UB>(), 0);                               \
        M16_PATTERN((D) ? BPD : 0, true)                                                        \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        if (D) dma_slab16(k64_unit<NA>(), gA, p.lda, m0, p.M, ka2, kend, vpA, wave);            \
        phase(ga, gb, fa, fb, k64_unit<UA>(), k64_unit<UB>(), 1);                               \
        M16_PATTERN((D) ? BPD : 0, false)                                                              \
        __builtin_amdgcn_sched_barrier(0);                                                      \
        ++j;                                                                                    \
    }
    // prologue: A of slabs 0 and 1, B of slab 0.  The k32 fragments
    // multiplied first in step 0 belong to no slab and are zero.
    if (dmaw) {
        dma_slab16(k64_unit<0>(), gA, p.lda, m0, p.M, kbeg, kend, vpA, wave);
        dma_slab16(k64_unit<1>(), gB, p.ldb, nb0, p.N, kbeg, kend, vpB, wave);
        dma_slab16(k64_unit<2>(), gA, p.lda, m0, p.M, kbeg + BK, kend, vpA, wave);
    }
    bf16x8 fa[FI], fb[FJ];
#pragma unroll
    for (int i = 0; i < FI; i++) fa[i] = bf16x8{};
#pragma unroll
    for (int j = 0; j < FJ; j++) fb[j] = bf16x8{};
    int j = 0;
    if (nk > 0) {
        // every step issues the same number of DMA instructions (past the end
        // of K they load zeros into free units), so the wait count is uniform
        if (dmaw) {
            for (; j + 5 <= nk;) {
                M16_STEP(0, true)
                M16_STEP(1, true)
                M16_STEP(2, true)
                M16_STEP(3, true)
                M16_STEP(4, true)
            }
            if (j < nk) M16_STEP(0, true)
            if (j < nk) M16_STEP(1, true)
            if (j < nk) M16_STEP(2, true)
            if (j < nk) M16_STEP(3, true)
        } else {
            for (; j + 5 <= nk;) {
                M16_STEP(0, false)
                M16_STEP(1, false)
                M16_STEP(2, false)
                M16_STEP(3, false)
                M16_STEP(4, false)
            }
            if (j < nk) M16_STEP(0, false)
            if (j < nk) M16_STEP(1, false)
            if (j < nk) M16_STEP(2, false)
            if (j < nk) M16_STEP(3, false)
        }
#pragma unroll
        for (int g = 0; g < 4; g++) mma_pair(fa, fb, g);  // last k32 step of the last slab
    }
#undef M16_STEP
#undef M16_PATTERN
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    // ---- epilogue through LDS (16 KB per wave in units 0-3), 32 rows at a time
    {
        auto region = [&](int w) {
            const int u = w >> 1;
            char *reg = u == 0 ? k64_unit<0>() : u == 1 ? k64_unit<1>() : u == 2 ? k64_unit<2>() : k64_unit<3>();
            return reinterpret_cast<float *>(reg + (w & 1) * 16384);
        };
        float *lw = region(wave);
        if constexpr (MODE == 5) {
            const float *lp = region(wave ^ 1);
#pragma unroll
            for (int i = 0; i < 2; i++) {
                stage16(&acc[2 * i][0], lw, lane);
                epilogue_swiglu(nullptr, lw, lp, m0 + wm * TM + i * 32, tn * 128, wn == 0, p, lane, true);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; i++) {
                stage16(&acc[2 * i][0], lw, lane);
                epilogue_block<bf16, 4, MODE == 0>(nullptr, lw, m0 + wm * TM + i * 32, n0 + wn * 128, p, MODE, lane,
                                                   true);
            }
        }
    }
}

// out[m*ldo + n] += sum_z part[z][m][n]   (N % 4 == 0), z in order: the
// partials of splits 1 .. S-1 (split 0 has already added its own into out).
// The count is a template argument so that every partial's load is issued
// before the first add; partials are read exactly once (non-temporal).
template <int S>
__global__ __launch_bounds__(256) void splitk_reduce(const float *part, float *out, long long ldo, int M, int N) {
    const long long i4 = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long total4 = (long long)M * N / 4;
    if (i4 >= total4) return;
    const long long e = i4 * 4;
    const int m = (int)(e / N), n = (int)(e % N);
    const long long MN = (long long)M * N;
    f32x4 v[S];
#pragma unroll
    for (int z = 0; z < S; z++) v[z] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(part + z * MN + e));
    f32x4 *o = reinterpret_cast<f32x4 *>(out + (long long)m * ldo + n);
    f32x4 acc = v[0];
#pragma unroll
    for (int z = 1; z < S; z++) acc += v[z];
    *o = *o + acc;
}
static hipError_t launch_reduce(const float *part, float *out, long long ldo, int M, int N, int splits, hipStream_t s) {
    const long long total4 = (long long)M * N / 4;
    const dim3 grid((unsigned)((total4 + 255) / 256));
    switch (splits - 1) {  // partial slots (splits is in [2, 16])
#define DTB_REDUCE_CASE(n) \
    case n: DTB_LAUNCH(splitk_reduce<n>, grid, dim3(256), 0, s, part, out, ldo, M, N); break;
    DTB_REDUCE_CASE(1) DTB_REDUCE_CASE(2) DTB_REDUCE_CASE(3) DTB_REDUCE_CASE(4) DTB_REDUCE_CASE(5)
    DTB_REDUCE_CASE(6) DTB_REDUCE_CASE(7) DTB_REDUCE_CASE(8) DTB_REDUCE_CASE(9) DTB_REDUCE_CASE(10)
    DTB_REDUCE_CASE(11) DTB_REDUCE_CASE(12) DTB_REDUCE_CASE(13) DTB_REDUCE_CASE(14) DTB_REDUCE_CASE(15)
#undef DTB_REDUCE_CASE
    default: return hipErrorInvalidValue;
    }
    return last_error();
}

// ---- host side ---------------------------------------------------------------
template <typename T, int BM, int BN, bool AK, bool BKM>
static hipError_t launch_t(const KParams &p, int splits, hipStream_t s) {
    constexpr int STAGE = (BM + BN) * 128;
    // set on every launch (a host-side attribute, per device): no flag that
    // would only remember the first device is kept
    hipError_t e = hipFuncSetAttribute((const void *)gemm_kernel<T, BM, BN, AK, BKM>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 2 * STAGE);
    if (e != hipSuccess) return e;
    int nm = (p.M + BM - 1) / BM, nn = (p.N + BN - 1) / BN;
    dim3 grid(nm * nn, 1, splits);
    DTB_LAUNCH((gemm_kernel<T, BM, BN, AK, BKM>), grid, dim3(256), 2 * STAGE, s, p);
    return last_error();
}

template <typename T, int BM, int BN>
static hipError_t launch_layout(const KParams &p, bool ak, bool bk, int splits, hipStream_t s) {
    if (ak && bk) return launch_t<T, BM, BN, true, true>(p, splits, s);
    if (ak && !bk) return launch_t<T, BM, BN, true, false>(p, splits, s);
    if (!ak && !bk) return launch_t<T, BM, BN, false, false>(p, splits, s);
    return launch_t<T, BM, BN, false, true>(p, splits, s);
}

template <bool AK, bool BKM, int MODE>
static hipError_t launch256_t(const KParams &p, int splits, hipStream_t s) {
    int nm = (p.M + 255) / 256, nn = (p.N + 255) / 256;
    const dim3 grid(nm * nn, 1, splits);
    // 64-k slabs whenever an operand is k-major (its rows then fill whole
    // cache lines); both operands m/n-major (the weight gradients) already
    // stream whole lines on 32-k slabs, and the 32-k ring measured the same
    // K a multiple of 64 (one split: kbeg = 0, kend = K): every slab is whole in k
    const bool whole = p.K % 64 == 0 && splits == 1;
    if constexpr (AK && BKM) {
        if (whole) DTB_LAUNCH((gemm_k64m16_kernel<MODE>), grid, dim3(512), 0, s, p);
        else DTB_LAUNCH((gemm_k64_kernel<AK, BKM, MODE, false>), grid, dim3(512), 0, s, p);
    } else if constexpr (AK || BKM) {
        if (whole) DTB_LAUNCH((gemm_k64_kernel<AK, BKM, MODE, true>), grid, dim3(512), 0, s, p);
        else DTB_LAUNCH((gemm_k64_kernel<AK, BKM, MODE, false>), grid, dim3(512), 0, s, p);
    } else {
        DTB_LAUNCH((gemm_dma_kernel<AK, BKM, MODE, 8>), grid, dim3(512), 0, s, p);
    }
    return last_error();
}

template <int MODE>
static hipError_t launch256_mode(const KParams &p, bool ak, bool bk, int splits, hipStream_t s) {
    if (ak && bk) return launch256_t<true, true, MODE>(p, splits, s);
    if (ak && !bk) return launch256_t<true, false, MODE>(p, splits, s);
    if (!ak && !bk) return launch256_t<false, false, MODE>(p, splits, s);
    return launch256_t<false, true, MODE>(p, splits, s);
}

static hipError_t launch256(const KParams &p, bool ak, bool bk, int splits, hipStream_t s) {
    if (p.out_mode == 0) return launch256_mode<0>(p, ak, bk, splits, s);
    if (p.out_mode == 2) return launch256_mode<2>(p, ak, bk, splits, s);
    if (p.out_mode == 5) return launch256_t<true, true, 5>(p, splits, s);  // the host checks the layout
    return launch256_mode<3>(p, ak, bk, splits, s);
}

// compute units of the current device (asked each time: the answer depends
// on the device, and the runtime answers from its own cache)
static int device_cus() {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
        return cus;
    return 256;
}

struct TileChoice {
    int bm, bn;
};
static TileChoice choose_tile(int M, int N, int dtype, bool splittable) {
    auto tiles = [&](int bm, int bn) { return (long long)((M + bm - 1) / bm) * ((N + bn - 1) / bn); };
    if (dtype == DTB_BF16) {
        if (M >= 256 && N >= 256 && (tiles(256, 256) >= 120 || splittable)) return {256, 256};
        if (tiles(256, 128) >= 512) return {256, 128};
        if (tiles(128, 128) >= 256) return {128, 128};
        return {64, 64};
    }
    // fp32: weight gradients (split over K, see choose_splits) on 128 x 128
    // tiles.  The forward and input-gradient GEMMs take 64 x 128 tiles when
    // there are at least four per CU and 64 x 64 otherwise: on the GPT-2-small
    // projection shapes 64 x 128 ran 101-122 TFLOP/s against 82-97 for
    // 128 x 128 (two workgroups per CU by LDS against three), and with fewer
    // tiles 64 x 64 keeps the CUs evenly loaded (384 tiles of 64 x 128 leave
    // half the CUs with twice the work).
    if (splittable && M >= 128 && N >= 128) return {128, 128};
    if (tiles(64, 128) >= 4LL * device_cus()) return {64, 128};
    return {64, 64};
}

static int choose_splits(const GemmArgs &g, TileChoice tc) {
    if (!(g.out_f32 && g.accumulate) || g.bias || g.res) return 1;
    const int BK = g.dtype == DTB_BF16 ? 64 : 32;
    long long tiles = (long long)((g.M + tc.bm - 1) / tc.bm) * ((g.N + tc.bn - 1) / tc.bn);
    if (g.dtype == DTB_BF16 && tc.bm == 256 && tc.bn == 256) {
        // bf16 256 x 256 tiles: the split count with the least estimated time,
        // rounds of workgroups x (per-round cost + k range x per-k cost) plus
        // the reduction's traffic ((S + 2) M N fp32 values), with constants
        // measured on this kernel: 9 us per round, 27.5 ns per k with every CU
        // busy, 6 TB/s.  A round that leaves CUs idle runs its k range faster
        // (the busy ones share L2, HBM and power with fewer others): per-k cost
        // x (0.45 + 0.55 x busy fraction), fitted to the Llama-GQA
        // weight-gradient shapes (e.g. the QKV one ran 1061 TFLOP/s on 2 splits,
        // one round of 192 workgroups, against 908 on 8, three full rounds).
        const int cus = device_cus();
        int best = 1;
        double best_t = 0.0;
        for (int sp = 1; sp <= 16; sp *= 2) {
            if (sp > 1 && (long long)g.K / sp < 8 * BK) break;
            const long long units = tiles * sp, full = units / cus, rest = units % cus;
            const double kcost = (double)g.K / sp * 0.0275;
            double t = (double)full * (9.0 + kcost);
            if (rest) t += 9.0 + kcost * (0.45 + 0.55 * (double)rest / cus);
            if (sp > 1) t += (sp + 2) * 4.0 * g.M * g.N / 6e6;
            if (sp == 1 || t < best_t) {
                best = sp;
                best_t = t;
            }
        }
        return best;
    }
    if (g.dtype == DTB_BF16) {  // bf16 tiles below 256 x 256 (a side under 256)
        int splits = 1;
        while (tiles * splits < 512 && (long long)g.K / (splits * 2) >= 8 * BK && splits < 16) splits *= 2;
        return splits;
    }
    // fp32 128 x 128 tiles: the split count with the least estimated time.
    // The workgroups of S splits x tiles are dealt to the CUs in turn, so the
    // busiest CU runs ceil(tiles S / CUs) of them, each a fixed cost plus its
    // k range; the reduction streams (S + 2) M N fp32 values.  Constants
    // measured on the GPT-2-small weight-gradient shapes: 3 us per workgroup,
    // 70 ns per k, 6 TB/s.  Any S (not only powers of two): there, 7 splits
    // of 108, 36 or 144 tiles ran 80-104 TFLOP/s against 65-91 for 4-16.
    const int cus = device_cus();
    int best = 1;
    double best_t = 0.0;
    for (int sp = 1; sp <= 16; sp++) {
        const long long kc = ((long long)g.K + sp - 1) / sp;
        if (sp > 1 && kc < 4 * BK) break;
        const long long per_cu = (tiles * sp + cus - 1) / cus;
        double t = (double)per_cu * (3.0 + (double)kc * 0.07 * (tc.bm * tc.bn) / (128.0 * 128.0));
        if (sp > 1) t += (sp + 2) * 4.0 * g.M * g.N / 6e6;
        if (sp == 1 || t < best_t) {
            best = sp;
            best_t = t;
        }
    }
    return best;
}

size_t gemm_ws_bytes(int M, int N, int K, int dtype) {
    GemmArgs g{};
    g.M = M; g.N = N; g.K = K; g.dtype = dtype; g.out_f32 = true; g.accumulate = true;
    TileChoice tc = choose_tile(M, N, dtype, true);
    int sp = choose_splits(g, tc);
    return sp > 1 ? (size_t)(sp - 1) * M * N * sizeof(float) : 0;  // split 0 needs no partial
}

int gemm(const GemmArgs &g, void *ws, size_t ws_bytes, hipStream_t s) {
    if (g.M <= 0 || g.N <= 0) return DTB_OK;
    const bool splittable = g.out_f32 && g.accumulate && !g.bias && !g.res;
    TileChoice tc = choose_tile(g.M, g.N, g.dtype, splittable);
    if (tc.bm == 256 && tc.bn == 256 && g.out_f32 && !g.accumulate) tc = {128, 128};
    int splits = choose_splits(g, tc);
    if (splits > 1 && (!ws || ws_bytes < (size_t)(splits - 1) * g.M * g.N * sizeof(float))) splits = 1;
    const int BK = g.dtype == DTB_BF16 ? 64 : 32;
    KParams p{};
    p.A = g.A; p.B = g.B; p.lda = g.lda; p.ldb = g.ldb;
    p.M = g.M; p.N = g.N; p.K = g.K;
    int kchunk = (g.K + splits - 1) / splits;
    kchunk = (kchunk + BK - 1) / BK * BK;
    p.kchunk = kchunk > 0 ? kchunk : BK;
    p.out = g.out; p.ldo = g.ldo;
    p.out_mode = splits > 1 ? 3 : (g.out_f32 ? (g.accumulate ? 2 : 1) : 0);
    p.bias = g.bias; p.res = g.res; p.ldr = g.ldr;
    p.part = splits > 1 ? reinterpret_cast<float *>(ws) : nullptr;
    // RoPE in the epilogue needs whole heads inside one wave's columns
    const int wave_cols = (g.dtype == DTB_BF16 && tc.bm == 256 && tc.bn == 256) ? 128 : tc.bn / 2;
    const bool rope_fused = g.rope_cs && splits == 1 && !g.out_f32 && g.rope_hd <= wave_cols;
    p.rope_cs = rope_fused ? reinterpret_cast<const float2 *>(g.rope_cs) : nullptr;
    p.rope_T = g.rope_T; p.rope_hd = g.rope_hd; p.rope_cols = g.rope_cols;
    p.act_h = g.act_h; p.act_mode = g.act_mode; p.act_H = g.act_H;
    const bool swiglu_fused = g.act_h && g.act_mode == DTB_MLP_SWIGLU && g.dtype == DTB_BF16 && tc.bm == 256 &&
                              tc.bn == 256 && g.act_H % 128 == 0 && g.N == 2 * g.act_H && g.ldo == g.N &&
                              g.a_kmajor && g.b_kmajor && splits == 1 && !g.out_f32 && !g.res && !g.rope_cs;
    if (swiglu_fused) p.out_mode = 5;
    double flops = 2.0 * g.M * g.N * (double)g.K;
    const int cls = g.out_f32 ? K_GEMM_DW : (g.b_kmajor ? K_GEMM_FWD : K_GEMM_DINP);
    if (g_timing_on) timing_begin(s, cls);
    hipError_t e;
    if (g.dtype == DTB_BF16) {
        if (tc.bm == 256 && tc.bn == 256) e = launch256(p, g.a_kmajor, g.b_kmajor, splits, s);
        else if (tc.bm == 256) e = launch_layout<bf16, 256, 128>(p, g.a_kmajor, g.b_kmajor, splits, s);
        else if (tc.bm == 128) e = launch_layout<bf16, 128, 128>(p, g.a_kmajor, g.b_kmajor, splits, s);
        else e = launch_layout<bf16, 64, 64>(p, g.a_kmajor, g.b_kmajor, splits, s);
    } else {
        if (tc.bm == 128) e = launch_layout<float, 128, 128>(p, g.a_kmajor, g.b_kmajor, splits, s);
        else if (tc.bn == 128) e = launch_layout<float, 64, 128>(p, g.a_kmajor, g.b_kmajor, splits, s);
        else e = launch_layout<float, 64, 64>(p, g.a_kmajor, g.b_kmajor, splits, s);
    }
    if (e != hipSuccess) return set_launch_error(e, "gemm");
    if (splits > 1) {  // splits is in [2, 16] (choose_splits)
        e = launch_reduce(reinterpret_cast<const float *>(ws), reinterpret_cast<float *>(g.out), g.ldo, g.M, g.N,
                          splits, s);
        if (e != hipSuccess) return set_launch_error(e, "splitk_reduce");
    }
    if (g_timing_on) {
        const double es = g.dtype == DTB_BF16 ? 2.0 : 4.0;
        double bytes = es * ((double)g.M * g.K + (double)g.N * g.K) +
                       (g.out_f32 ? 4.0 * (g.accumulate ? 2.0 : 1.0) : es) * g.M * g.N;
        if (swiglu_fused) bytes += es * (double)g.M * g.act_H;          // write the activation output
        timing_end(s, cls, flops, bytes);
    }
    // passes the epilogue could not take (timed as their own launches)
    if (g.act_h && !swiglu_fused) {
        const int r = act_forward(g.act_mode, g.dtype, g.out, g.M, g.act_H, g.act_h, s);
        if (r) return r;
    }
    if (g.rope_cs && !rope_fused) {  // heads wider than a wave's columns: separate pass
        const int r = rope_apply(g.dtype, g.out, g.rope_cs, g.M / g.rope_T, g.rope_T, (int)g.ldo,
                                 g.rope_cols / g.rope_hd, 0, g.rope_hd, 0, s);
        if (r) return r;
    }
    return DTB_OK;
}

}  // namespace dtb
