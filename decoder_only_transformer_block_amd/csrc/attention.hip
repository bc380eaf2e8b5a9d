// Causal grouped-query flash attention, forward and backward, for gfx950.
//
// What is computed ("nanoeuler — CUDA kernels": the flash_attn_forward_kernel /
// flash_attn_backward_kernel declarations and the attention_cpu_fwd/bwd
// definitions; "microgpt.cu": attention_backward's dS = P (dP - sum P dP)):
//   s_tj = q_t.k_j / sqrt(hd) (j <= t), o_t = softmax(s_t) V, lse_t = logsumexp_j s_tj,
//   backward with P_tj = exp(s_tj - lse_t), D_t = dO_t.o_t, dS = P (dO V^T - D).
// Query head h reads kv head h / (NH/NKV).
//
// This file holds the fp32 path (bf16 has its own kernels): fp32 operands
// use the 32x32x2 fp32 MFMA.
// * Scores are computed transposed, S^T = K Q^T, so a lane owns one query
//   (column l%32) and 16 keys (rows) of each 32x32 block: the running max and
//   sum of the online softmax are in-register reductions plus one exchange
//   with the partner lane l^32.  The same layout makes P^T (and dS^T) usable
//   directly as the B operand of the next product.
// * The A operand of those products needs one element of a natural tile per
//   lane and k step (V^T, K^T, Q^T, dO^T), read straight from LDS.
// * Natural tiles are rows of hd elements in 16-byte chunks, XOR-swizzled
//   with (row & 7).  Two LDS stages; the next tile's global loads are issued
//   before the current tile's MFMAs (one barrier per tile).  Half of the
//   threads stage one tensor, the other half the other.
// * forward: one workgroup = 64 queries of one (b, h), key tiles of 64 whose
//   two 32-key halves go to two waves per 32-query slice (merged at the end),
//   last query blocks launched first (causal load balance).
// * backward: D = rowsum(dO o) by a small kernel; dQ by a query-owning kernel
//   (like the forward: S^T, dP^T = V dO^T, dQ^T += K^T dS^T); dK and dV by a
//   key-owning kernel (64 keys of one (b, kv head)) that loops over
//   the group's query heads and the query tiles at or after its keys
//   (S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS), so dK/dV are
//   summed over the group in registers -- no atomics, deterministic.  In both
//   backward kernels a workgroup holds two 32-row slices of its own rows and
//   gives each slice two waves that take alternate 32-row halves of the other
//   side's tiles; the halves' partial sums meet in LDS at the end.
#include <type_traits>

#include "attention.h"

namespace dtb {

template <typename T, int HD> struct AT {
    static constexpr int ES = sizeof(T);
    static constexpr int EPC = 16 / ES;                 // elements per 16-byte chunk
    static constexpr int NCH = HD * ES / 16;            // chunks per natural row
    static constexpr int NC = NCH / 2;                  // chunk pairs (MFMA steps)
    static constexpr int RB = HD * ES;                  // natural row bytes
    static constexpr int XM = (NCH < 8 ? NCH : 8) - 1;  // swizzle mask
    static constexpr int ND = HD >= 32 ? HD / 32 : 1;   // 32-row blocks over hd
};

template <typename T, int HD> __device__ __forceinline__ int nat_off(int row, int chunk) {
    return row * AT<T, HD>::RB + ((chunk ^ (row & AT<T, HD>::XM)) << 4);
}
// ---------------------------------------------------------------------------
// staging helpers (a subset of NT threads, local id tl)
// ---------------------------------------------------------------------------
// natural [ROWS][HD] tile: chunk items
template <typename T, int HD, int ROWS, int NT> struct Nat {
    static constexpr int ITEMS = ROWS * AT<T, HD>::NCH;
    static constexpr int P = (ITEMS + NT - 1) / NT;
    __device__ static __forceinline__ void load(u32x4 *reg, const T *g, long long stride, int row0, int nrows,
                                                int hd, int tl) {
        constexpr int NCH = AT<T, HD>::NCH, EPC = AT<T, HD>::EPC;
        const Buf buf(g + (long long)row0 * stride);
#pragma unroll
        for (int p = 0; p < P; p++) {
            int idx = tl + NT * p;
            int r = idx / NCH, c = idx % NCH;
            bool ok = idx < ITEMS && row0 + r < nrows && c * EPC < hd;
            reg[p] = buf.ld16((int)(((long long)r * stride + c * EPC) * (int)sizeof(T)), ok);
        }
    }
    __device__ static __forceinline__ void store(const u32x4 *reg, char *lds, int tl) {
        constexpr int NCH = AT<T, HD>::NCH;
#pragma unroll
        for (int p = 0; p < P; p++) {
            int idx = tl + NT * p;
            if (idx < ITEMS) *reinterpret_cast<u32x4 *>(lds + nat_off<T, HD>(idx / NCH, idx % NCH)) = reg[p];
        }
    }
};

// ---------------------------------------------------------------------------
// fragment helpers
// ---------------------------------------------------------------------------
// fp32: element (row, d) of a natural tile
template <int HD> __device__ __forceinline__ float nat_elem(const char *nat, int row, int d) {
    if (HD < 32 && d >= HD) return 0.f;
    return *reinterpret_cast<const float *>(nat + nat_off<float, HD>(row, d >> 2) + ((d & 3) << 2));
}

// acc_o (ND blocks over head dim, columns = the lane's query/key) +=
//   A^T (HD x 32 positions of block j) * X (32 positions x 32 columns), with X in
// S^T-layout registers x (one 32x32 block) and A^T read from LDS.
template <typename T, int HD, int ROWS>
__device__ __forceinline__ void mma_trans(f32x16 *acc, const f32x16 &x, const char *tile, int j, int lane) {
    const int l32 = lane & 31;
#pragma unroll
    for (int r = 0; r < 16; r++) {
        const int row = j * 32 + acc_row(r, lane);
#pragma unroll
        for (int db = 0; db < AT<T, HD>::ND; db++)
            acc[db] = mfma32(nat_elem<HD>(tile, row, db * 32 + l32), x[r], acc[db]);
    }
}

// S-block (32 rows of `tile` x 32 columns given by per-lane fragments frag[c]):
// acc += tile[rows j*32 .. +32] . frag^T over the head dimension
template <typename T, int HD>
__device__ __forceinline__ void mma_rows(f32x16 &acc, const char *tile, int rowbase, const u32x4 *frag, int lane) {
    const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int c = 0; c < AT<T, HD>::NC; c++) {
        u32x4 a = *reinterpret_cast<const u32x4 *>(tile + nat_off<T, HD>(rowbase + l32, 2 * c + g));
        mma_chunk(acc, a, frag[c], T());
    }
}

// per-lane fragments of row `row` of a uniform base (row stride `stride`
// elements): chunks 2c+g of the head slice
template <typename T, int HD>
__device__ __forceinline__ void load_row_frag(u32x4 *f, const T *base, long long stride, int row, bool valid,
                                              int hd, int g) {
    const Buf buf(base);
#pragma unroll
    for (int c = 0; c < AT<T, HD>::NC; c++) {
        int ch = 2 * c + g;
        f[c] = buf.ld16((int)(((long long)row * stride + ch * AT<T, HD>::EPC) * (int)sizeof(T)),
                        valid && ch * AT<T, HD>::EPC < hd);
    }
}

// write ND accumulator blocks (lane = row position, regs = head dim) scaled by s
template <typename T, int HD>
__device__ __forceinline__ void store_rows(T *row, const f32x16 *acc, float s, int hd, int lane) {
#pragma unroll
    for (int db = 0; db < AT<T, HD>::ND; db++)
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
            int d = db * 32 + 8 * r4 + 4 * (lane >> 5);
            if (d < hd) {
                f32x4 v{acc[db][4 * r4] * s, acc[db][4 * r4 + 1] * s, acc[db][4 * r4 + 2] * s,
                            acc[db][4 * r4 + 3] * s};
                    *reinterpret_cast<f32x4 *>(row + d) = v;
            }
        }
}

// ---------------------------------------------------------------------------
// transposed fp32 tiles (head widths >= 32): a natural [64][HD] tile staged as
// its transpose [HD][64], so that the A operand of a product over positions
// (V^T, K^T, ...) comes as one 16-byte read of four consecutive positions per
// lane, i.e. one read per four MFMAs, instead of one 4-byte read per MFMA.
// Row d holds the 64 positions of column d in 16 chunks; chunk kc (positions
// 4 kc .. 4 kc + 3) sits at kc ^ (d & 15), so the 16 lanes of a read group
// (16 consecutive d, one chunk) hit 16 different bank quads.
// Staging items are 4 x 4 blocks (4 positions x 4 columns): four 16-byte row
// pieces loaded, transposed in registers, stored as four 16-byte column pieces.
// ---------------------------------------------------------------------------
template <int HD, int NT> struct NatT {
    static constexpr int CB = HD / 4;              // column blocks
    static constexpr int ITEMS = 16 * CB;          // 16 position blocks of 4
    static constexpr int P = (ITEMS + NT - 1) / NT;
    static constexpr int REGS = 4 * P;             // 16-byte registers per thread
    __device__ static __forceinline__ void load(u32x4 *reg, const float *g, long long stride, int row0, int nrows,
                                                int hd, int tl) {
        const Buf buf(g + (long long)row0 * stride);
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int idx = tl + NT * p;
            const int cb = idx % CB, pb = idx / CB;   // neighbouring threads: neighbouring 16-byte pieces of a row
            const bool live = idx < ITEMS && cb * 4 < hd;
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int r = pb * 4 + i;
                reg[4 * p + i] = buf.ld16((int)(((long long)r * stride + cb * 4) * 4), live && row0 + r < nrows);
            }
        }
    }
    __device__ static __forceinline__ void store(const u32x4 *reg, char *lds, int tl) {
#pragma unroll
        for (int p = 0; p < P; p++) {
            const int idx = tl + NT * p;
            if (idx >= ITEMS) continue;
            const int cb = idx % CB, pb = idx / CB;
            u32x4 o[4];
            transpose4x4(reg + 4 * p, o);   // o[e]: column cb*4+e, positions 4 pb .. 4 pb + 3
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int d = cb * 4 + e;
                *reinterpret_cast<u32x4 *>(lds + d * 256 + ((pb ^ (d & 15)) << 4)) = o[e];
            }
        }
    }
};

// acc (ND blocks over the head dimension, columns = the lane's query or key)
// += A^T (HD x 32 positions of block j) * X (32 positions x 32 columns, the
// S^T-layout registers x), A^T read from a transposed tile: chunk
// j*8 + 2q + g of row d holds positions 32 j + 8 q + 4 g + e, the rows that
// registers 4q + e of lane half g hold in x
template <int HD>
__device__ __forceinline__ void mma_trans_t(f32x16 *acc, const f32x16 &x, const char *tt, int j, int lane) {
    const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int db = 0; db < HD / 32; db++) {
        const int d = db * 32 + l32;
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const int kc = j * 8 + 2 * q + g;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(tt + d * 256 + ((kc ^ (d & 15)) << 4));
#pragma unroll
            for (int e = 0; e < 4; e++) acc[db] = mfma32(__uint_as_float(v[e]), x[4 * q + e], acc[db]);
        }
    }
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------
template <typename T, int HD> struct FwdCfg {
    static constexpr int BQ = 64, BKV = 64;
    static constexpr int KB = BKV * HD * (int)sizeof(T);  // K natural tile bytes (= V tile bytes)
    static constexpr int STAGE = 2 * KB;
    // staging: threads [0, 128) load V, [128, 256) load K with the same loader
    static constexpr int PREG = Nat<T, HD, BKV, 128>::P;
    // end of the kernel: the two slices' (O, m, l) hand-over, in the same LDS
    static constexpr int MERGE = 2 * (AT<T, HD>::ND * 16 * 64 + 128) * 4;
    static constexpr int LDS = 2 * STAGE > MERGE ? 2 * STAGE : MERGE;
};

// V staged transposed (fp32, HD >= 32): the same register count as the natural loader
template <typename T, int HD> constexpr bool fwd_vt() { return std::is_same<T, float>::value && HD >= 32; }

template <typename T, int HD>
__device__ __forceinline__ void fwd_stage_load(u32x4 *reg, const T *kb, const T *vb, long long stride, int kv0,
                                               int T_, int hd) {
    const int t = threadIdx.x;
    const bool lo = __builtin_amdgcn_readfirstlane(t >> 6) < 2;
    if constexpr (fwd_vt<T, HD>()) {
        static_assert(NatT<HD, 128>::REGS == Nat<T, HD, 64, 128>::P, "transposed staging must fit the registers");
        if (lo) NatT<HD, 128>::load(reg, vb, stride, kv0, T_, hd, t & 127);
        else Nat<T, HD, 64, 128>::load(reg, kb, stride, kv0, T_, hd, t & 127);
    } else {
        const T *g = lo ? vb : kb;
        Nat<T, HD, 64, 128>::load(reg, g, stride, kv0, T_, hd, t & 127);
    }
}
template <typename T, int HD> __device__ __forceinline__ void fwd_stage_store(const u32x4 *reg, char *st) {
    const int t = threadIdx.x;
    constexpr int KB = FwdCfg<T, HD>::KB;
    const bool lo = __builtin_amdgcn_readfirstlane(t >> 6) < 2;
    if constexpr (fwd_vt<T, HD>()) {
        if (lo) NatT<HD, 128>::store(reg, st + KB, t & 127);
        else Nat<T, HD, 64, 128>::store(reg, st, t & 127);
    } else {
        Nat<T, HD, 64, 128>::store(reg, lo ? st + KB : st, t & 127);
    }
}

// One workgroup: 64 queries of one (b, h) as two slices of 32, each slice
// shared by two waves that split every 64-key tile into its two 32-key halves
// (wave = slice + 2 * half).  Each wave keeps its own online-softmax state over
// its keys; at the end the half-1 waves hand (m, l, O) to their half-0
// partners through LDS, which merge and store.  Splitting the keys halves the
// serial chain of the slices next to the diagonal's end (the last 32 queries
// see every key): with one wave per slice that chain alone took longer than
// the average CU's share of the whole launch.
template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_fwd_kernel(AttnP p) {
    using A = AT<T, HD>;
    using FC = FwdCfg<T, HD>;
    constexpr int BQ = FC::BQ, BKV = FC::BKV;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int nqb = (p.T + BQ - 1) / BQ;
    const int BH = p.B * p.NH;
    const int qb = nqb - 1 - (int)(blockIdx.x / BH);
    const int bh = blockIdx.x % BH;
    const int b = bh / p.NH, h = bh % p.NH, kh = h / (p.NH / p.NKV);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, l32 = lane & 31;
    const int slice = wave & 1, half = wave >> 1;
    const int q0 = qb * BQ, qw0 = q0 + slice * 32, qi = qw0 + l32;
    // last key this slice can see (none if the slice starts past the sequence)
    const int klast = qw0 < p.T ? min(qw0 + 31, p.T - 1) : -1;

    const long long stride = p.QKV;
    const T *base = reinterpret_cast<const T *>(p.qkv) + (long long)b * p.T * stride;
    const T *kbase = base + p.C + kh * p.hd;
    const T *vbase = kbase + p.NKV * p.hd;

    u32x4 qf[A::NC];
    load_row_frag<T, HD>(qf, base + h * p.hd, stride, qi, qi < p.T, p.hd, g);

    f32x16 O[A::ND];
#pragma unroll
    for (int d = 0; d < A::ND; d++)
#pragma unroll
        for (int r = 0; r < 16; r++) O[d][r] = 0.f;
    float m = -1e30f, lsum = 0.f;

    const int kv_end = min(p.T, q0 + BQ);
    const int ntiles = (kv_end + BKV - 1) / BKV;

    u32x4 reg[FC::PREG];
    fwd_stage_load<T, HD>(reg, kbase, vbase, stride, 0, p.T, p.hd);
    fwd_stage_store<T, HD>(reg, smem);
    // the per-lane fragments loaded above are complete before the loop, so the
    // loop body never waits on them (nor, by extension, on the prefetch it issues)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = 0; kt < ntiles; kt++) {
        const bool more = kt + 1 < ntiles;
        if (more) fwd_stage_load<T, HD>(reg, kbase, vbase, stride, (kt + 1) * BKV, p.T, p.hd);
        const char *Ks = smem + (kt & 1) * FC::STAGE;
        const char *Vs = Ks + FC::KB;
        const int kb0 = kt * BKV + half * 32;   // this wave's 32 keys
        if (kb0 <= klast) {
            f32x16 S;
#pragma unroll
            for (int r = 0; r < 16; r++) S[r] = 0.f;
            mma_rows<T, HD>(S, Ks, half * 32, qf, lane);
            // keys above the diagonal only occur in the last blocks of a slice
            if (kb0 + 31 > qw0) {
#pragma unroll
                for (int r = 0; r < 16; r++)
                    if (kb0 + acc_row(r, lane) > qi) S[r] = -INFINITY;
            }
            float sv[16];
#pragma unroll
            for (int r = 0; r < 16; r++) sv[r] = S[r];
            const float mt = max_xor32(tree_max<16>(sv)) * p.sl2;   // tile max in log2 units
            const float mn = fmaxf(m, mt);
            if (!__all(mn == m)) {
                const float alpha = exp2f(m - mn);
                lsum *= alpha;
#pragma unroll
                for (int d = 0; d < A::ND; d++)
#pragma unroll
                    for (int r = 0; r < 16; r++) O[d][r] *= alpha;
            }
            m = mn;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                float e = exp2f(fmaf(S[r], p.sl2, -mn));
                S[r] = e;
                lsum += e;
            }
            if constexpr (fwd_vt<T, HD>()) mma_trans_t<HD>(O, S, Vs, half, lane);
            else mma_trans<T, HD, BKV>(O, S, Vs, half, lane);
        }
        if (more) fwd_stage_store<T, HD>(reg, smem + ((kt + 1) & 1) * FC::STAGE);
        __syncthreads();
    }

    // merge the two halves of each slice (the stages are free after the last barrier):
    // per slice, O as [ND][16][64 lanes] floats, then m and the lane's partial sum
    float *xo = reinterpret_cast<float *>(smem) + slice * (A::ND * 16 * 64 + 128);
    if (half == 1) {
#pragma unroll
        for (int d = 0; d < A::ND; d++)
#pragma unroll
            for (int r = 0; r < 16; r++) xo[(d * 16 + r) * 64 + lane] = O[d][r];
        xo[A::ND * 16 * 64 + lane] = m;
        xo[A::ND * 16 * 64 + 64 + lane] = lsum;
    }
    __syncthreads();
    if (half == 1) return;
    {
        const float m1 = xo[A::ND * 16 * 64 + lane], l1 = xo[A::ND * 16 * 64 + 64 + lane];
        const float mm = fmaxf(m, m1);
        const float a0 = exp2f(m - mm), a1 = exp2f(m1 - mm);
#pragma unroll
        for (int d = 0; d < A::ND; d++)
#pragma unroll
            for (int r = 0; r < 16; r++) O[d][r] = O[d][r] * a0 + xo[(d * 16 + r) * 64 + lane] * a1;
        lsum = lsum * a0 + l1 * a1;
        m = mm;
    }
    const float ltot = sum_xor32(lsum);
    if (qi < p.T) {
        T *orow = reinterpret_cast<T *>(p.o) + ((long long)b * p.T + qi) * p.C + h * p.hd;
        store_rows<T, HD>(orow, O, 1.f / ltot, p.hd, lane);
        if (g == 0) p.lse[((long long)b * p.NH + h) * p.T + qi] = (m + log2f(ltot)) * LN2;
    }
}

// ---------------------------------------------------------------------------
// backward of the fp32 kernels: D = rowsum(dO * O)   [B][NH][T] fp32, one wave
// per (b, t) row (the bf16 dQ kernel computes its own D)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void attn_bwd_dot_kernel(AttnP p, float *D) {
    const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= (long long)p.B * p.T) return;
    const int b = (int)(row / p.T), tq = (int)(row % p.T);
    const T *o = reinterpret_cast<const T *>(p.out) + row * p.C;
    const T *d = reinterpret_cast<const T *>(p.dout) + row * p.C;
    constexpr int EPC = 16 / sizeof(T);
    const int hd = p.hd;
    // lanes sweep the row in 16-byte chunks; a head spans hd/EPC chunks
    const int nch = p.C / EPC, hch = hd / EPC;
    // four sweeps of loads in flight before any reduction (a row is 4 sweeps
    // at C = 2048 in bf16)
    const Buf bo(o), bdd(d);
    for (int c00 = 0; c00 < nch; c00 += 4 * 64) {
        u32x4 ov[4], dv[4];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int c = c00 + 64 * u + lane;
            ov[u] = bo.ld16(c * 16, c < nch);
            dv[u] = bdd.ld16(c * 16, c < nch);
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int c = c00 + 64 * u + lane;
            if (c00 + 64 * u >= nch) break;  // uniform
            float fo[EPC], fd[EPC], s = 0.f;
            unpack16<T>(ov[u], fo);
            unpack16<T>(dv[u], fd);
#pragma unroll
            for (int e = 0; e < EPC; e++) s += fo[e] * fd[e];
            // reduce over the hch consecutive lanes of each head (hch is a
            // power of 2, at most 32 for hd <= 128)
            for (int off = 1; off < hch && off < 64; off <<= 1) s += __shfl_xor(s, off, 64);
            if (c < nch && (c % hch) == 0) {
                int h = c / hch;
                const long long i = ((long long)b * p.NH + h) * p.T + tq;
                D[i] = s;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// backward: dQ (query-owning)
// ---------------------------------------------------------------------------
template <typename T, int HD> struct DqCfg {
    static constexpr int BQ = 64, BKV = 64;
    static constexpr int KB = BKV * HD * (int)sizeof(T);
    // LDS stage: K natural, V natural.  Threads [0, 128) load K, [128, 256)
    // load V with the same loader.
    static constexpr int STAGE = 2 * KB;
    static constexpr int PREG = Nat<T, HD, BKV, 128>::P;
    // end of the kernel: the half-1 waves' dQ partials, in the same LDS
    static constexpr int MERGE = 2 * AT<T, HD>::ND * 16 * 64 * 4;
    static constexpr int LDS = 2 * STAGE > MERGE ? 2 * STAGE : MERGE;
};

template <typename T, int HD>
__device__ __forceinline__ void dq_stage_load(u32x4 *reg, const T *kb, const T *vb, long long stride, int kv0,
                                              int T_, int hd) {
    const int t = threadIdx.x;
    const bool lo = __builtin_amdgcn_readfirstlane(t >> 6) < 2;
    const T *g = lo ? kb : vb;
    Nat<T, HD, 64, 128>::load(reg, g, stride, kv0, T_, hd, t & 127);
}
template <typename T, int HD> __device__ __forceinline__ void dq_stage_store(const u32x4 *reg, char *st) {
    const int t = threadIdx.x;
    constexpr int KB = DqCfg<T, HD>::KB;
    const bool lo = __builtin_amdgcn_readfirstlane(t >> 6) < 2;
    Nat<T, HD, 64, 128>::store(reg, lo ? st : st + KB, t & 127);
}

template <typename T, int HD>
__global__ __launch_bounds__(256) void attn_bwd_dq_kernel(AttnP p) {
    using A = AT<T, HD>;
    using FC = DqCfg<T, HD>;
    constexpr int BQ = FC::BQ, BKV = FC::BKV;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int nqb = (p.T + BQ - 1) / BQ;
    const int BH = p.B * p.NH;
    const int qb = nqb - 1 - (int)(blockIdx.x / BH);
    const int bh = blockIdx.x % BH;
    const int b = bh / p.NH, h = bh % p.NH, kh = h / (p.NH / p.NKV);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, l32 = lane & 31;
    // two 32-query slices; each 64-key tile's two 32-key halves go to two
    // waves (wave = slice + 2 * half), whose dQ partials are summed at the end
    const int slice = wave & 1, half = wave >> 1;
    const int q0 = qb * BQ, qw0 = q0 + slice * 32, qi = qw0 + l32;
    const int klast = qw0 < p.T ? min(qw0 + 31, p.T - 1) : -1;

    const long long stride = p.QKV;
    const T *base = reinterpret_cast<const T *>(p.qkv) + (long long)b * p.T * stride;
    const T *kbase = base + p.C + kh * p.hd;
    const T *vbase = kbase + p.NKV * p.hd;

    u32x4 qf[A::NC], df[A::NC];
    load_row_frag<T, HD>(qf, base + h * p.hd, stride, qi, qi < p.T, p.hd, g);
    load_row_frag<T, HD>(df, reinterpret_cast<const T *>(p.dout) + (long long)b * p.T * p.C + h * p.hd, p.C, qi,
                         qi < p.T, p.hd, g);
    const long long li = ((long long)b * p.NH + h) * p.T + qi;
    const float lse2 = qi < p.T ? p.lse_in[li] * LOG2E : INFINITY;
    const float Dq = qi < p.T ? p.D[li] : 0.f;

    f32x16 dQ[A::ND];
#pragma unroll
    for (int d = 0; d < A::ND; d++)
#pragma unroll
        for (int r = 0; r < 16; r++) dQ[d][r] = 0.f;

    const int kv_end = min(p.T, q0 + BQ);
    const int ntiles = (kv_end + BKV - 1) / BKV;

    u32x4 reg[FC::PREG];
    dq_stage_load<T, HD>(reg, kbase, vbase, stride, 0, p.T, p.hd);
    dq_stage_store<T, HD>(reg, smem);
    // the per-lane fragments loaded above are complete before the loop, so the
    // loop body never waits on them (nor, by extension, on the prefetch it issues)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int kt = 0; kt < ntiles; kt++) {
        const bool more = kt + 1 < ntiles;
        if (more) dq_stage_load<T, HD>(reg, kbase, vbase, stride, (kt + 1) * BKV, p.T, p.hd);
        const char *Ks = smem + (kt & 1) * FC::STAGE;
        const char *Vs = Ks + FC::KB;
        const char *Kt = Ks;
        const int kb0 = kt * BKV + half * 32;   // this wave's 32 keys
        if (kb0 <= klast) {
            f32x16 S, dP;
#pragma unroll
            for (int r = 0; r < 16; r++) S[r] = dP[r] = 0.f;
            mma_rows<T, HD>(S, Ks, half * 32, qf, lane);
            mma_rows<T, HD>(dP, Vs, half * 32, df, lane);
            const bool diag = kb0 + 31 > qw0;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                float pr = exp2f(fmaf(S[r], p.sl2, -lse2));
                if (diag && kb0 + acc_row(r, lane) > qi) pr = 0.f;
                S[r] = pr * (dP[r] - Dq);
            }
            mma_trans<T, HD, BKV>(dQ, S, Kt, half, lane);
        }
        if (more) dq_stage_store<T, HD>(reg, smem + ((kt + 1) & 1) * FC::STAGE);
        __syncthreads();
    }
    // sum the two halves of each slice (the stages are free after the last barrier)
    {
        float *xq = reinterpret_cast<float *>(smem) + slice * (A::ND * 16 * 64);
        if (half == 1) {
#pragma unroll
            for (int d = 0; d < A::ND; d++)
#pragma unroll
                for (int r = 0; r < 16; r++) xq[(d * 16 + r) * 64 + lane] = dQ[d][r];
        }
        __syncthreads();
        if (half == 1) return;
#pragma unroll
        for (int d = 0; d < A::ND; d++)
#pragma unroll
            for (int r = 0; r < 16; r++) dQ[d][r] += xq[(d * 16 + r) * 64 + lane];
    }
    if (p.rope_cs) rope_rotate_acc<A::ND>(dQ, p.rope_cs + (long long)min(qi, p.T - 1) * (p.hd / 2), p.hd, -1.f, lane);
    if (qi < p.T) {
        T *row = reinterpret_cast<T *>(p.o) + ((long long)b * p.T + qi) * p.QKV + h * p.hd;
        store_rows<T, HD>(row, dQ, p.scale, p.hd, lane);
    }
}

// ---------------------------------------------------------------------------
// backward: dK, dV (key-owning, summed over the query heads of the group)
// ---------------------------------------------------------------------------
template <typename T, int HD> struct DkvCfg {
    static constexpr int BK = 64;    // keys per workgroup (2 slices of 32, two waves each)
    static constexpr int BQ = 64;    // queries per tile
    static constexpr int QB = BQ * HD * (int)sizeof(T);
    // LDS stage: Q natural, dO natural, then lse2[BQ], D[BQ]
    static constexpr int STAGE = 2 * QB + 2 * BQ * 4;
    static constexpr int PQ = Nat<T, HD, BQ, 128>::P;
    static constexpr int PREG = PQ;
    // end of the kernel: the half-1 waves' dK and dV partials, in the same LDS
    static constexpr int MERGE = 2 * 2 * AT<T, HD>::ND * 16 * 64 * 4;
    static constexpr int LDS = 2 * STAGE > MERGE ? 2 * STAGE : MERGE;
};

template <typename T, int HD>
__device__ __forceinline__ void dkv_stage_load(u32x4 *reg, float &aux, const T *qb, const T *db, long long qstride,
                                               long long dstride, const float *lse, const float *D, int q0, int T_,
                                               int hd) {
    const int t = threadIdx.x;
    constexpr int BQ = DkvCfg<T, HD>::BQ;
    const bool lo = __builtin_amdgcn_readfirstlane(t >> 6) < 2;
    const T *g = lo ? qb : db;
    const long long st = lo ? qstride : dstride;
    const int tl = t & 127;
    Nat<T, HD, BQ, 128>::load(reg, g, st, q0, T_, hd, tl);
    // threads 0..BQ-1: lse of query q0+t; threads 128..128+BQ-1: D (raw; the
    // transform to log2 units happens at the LDS store, away from the load)
    {
        const int q = q0 + tl;
        const bool ok = tl < BQ && q < T_;
        const Buf bl(lo ? lse : D);
        aux = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bl.r, ok ? q * 4 : (int)0x80000000, 0, 0));
    }
}
template <typename T, int HD>
__device__ __forceinline__ void dkv_stage_store(const u32x4 *reg, float aux, char *st, int q0, int T_) {
    using FC = DkvCfg<T, HD>;
    const int t = threadIdx.x, tl = t & 127;
    char *nat = st + (t < 128 ? 0 : FC::QB);
    Nat<T, HD, FC::BQ, 128>::store(reg, nat, tl);
    float *f = reinterpret_cast<float *>(st + 2 * FC::QB);
    if (tl < FC::BQ) {
        const bool lo = t < 128;
        const bool ok = q0 + tl < T_;
        f[(lo ? 0 : FC::BQ) + tl] = lo ? (ok ? aux * LOG2E : INFINITY) : aux;
    }
}

template <typename T, int HD>
__global__ __launch_bounds__(256, HD == 64 ? 2 : 1) void attn_bwd_dkv_kernel(AttnP p) {
    using A = AT<T, HD>;
    using FC = DkvCfg<T, HD>;
    constexpr int BK = FC::BK, BQ = FC::BQ;
    extern __shared__ __attribute__((aligned(16))) char smem[];

    const int nkb = (p.T + BK - 1) / BK;
    const int BKVH = p.B * p.NKV;
    const int kb = (int)(blockIdx.x / BKVH);   // low key blocks (most work) first
    const int bk = blockIdx.x % BKVH;
    const int b = bk / p.NKV, kh = bk % p.NKV;
    const int grp = p.NH / p.NKV;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, g = lane >> 5, l32 = lane & 31;
    // two 32-key slices; each 64-query tile's two 32-query halves go to two
    // waves (wave = slice + 2 * half), whose dK and dV partials are summed at the end
    const int slice = wave & 1, half = wave >> 1;
    const int k0 = kb * BK, kw0 = k0 + slice * 32, ki = kw0 + l32;
    (void)nkb;

    const long long stride = p.QKV;
    const T *base = reinterpret_cast<const T *>(p.qkv) + (long long)b * p.T * stride;
    u32x4 kf[A::NC], vf[A::NC];
    load_row_frag<T, HD>(kf, base + p.C + kh * p.hd, stride, ki, ki < p.T, p.hd, g);
    load_row_frag<T, HD>(vf, base + p.C + (p.NKV + kh) * p.hd, stride, ki, ki < p.T, p.hd, g);

    f32x16 dK[A::ND], dV[A::ND];
#pragma unroll
    for (int d = 0; d < A::ND; d++)
#pragma unroll
        for (int r = 0; r < 16; r++) dK[d][r] = dV[d][r] = 0.f;

    const int qt0 = k0 / BQ;                       // first query tile touching these keys
    const int nqt = (p.T + BQ - 1) / BQ - qt0;     // query tiles per head
    const int niter = nqt * grp;

    auto srcs = [&](int it, const T *&qb, const T *&db, const float *&lse, const float *&D, int &q0) {
        int hh = it / nqt, qt = qt0 + it % nqt;
        int h = kh * grp + hh;
        q0 = qt * BQ;
        qb = base + h * p.hd;
        db = reinterpret_cast<const T *>(p.dout) + (long long)b * p.T * p.C + h * p.hd;
        lse = p.lse_in + ((long long)b * p.NH + h) * p.T;
        D = p.D + ((long long)b * p.NH + h) * p.T;
    };

    u32x4 reg[FC::PREG];
    float aux = 0.f;
    if (niter > 0) {
        const T *qb, *db;
        const float *lse, *D;
        int q0;
        srcs(0, qb, db, lse, D, q0);
        dkv_stage_load<T, HD>(reg, aux, qb, db, stride, p.C, lse, D, q0, p.T, p.hd);
        dkv_stage_store<T, HD>(reg, aux, smem, q0, p.T);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    for (int it = 0; it < niter; it++) {
        const bool more = it + 1 < niter;
        if (more) {
            const T *qb, *db;
            const float *lse, *D;
            int q0;
            srcs(it + 1, qb, db, lse, D, q0);
            dkv_stage_load<T, HD>(reg, aux, qb, db, stride, p.C, lse, D, q0, p.T, p.hd);
        }
        const char *st = smem + (it & 1) * FC::STAGE;
        const char *Qs = st, *dOs = st + FC::QB;
        const char *Qt = Qs;
        const char *dOt = dOs;
        const float *lse2 = reinterpret_cast<const float *>(st + 2 * FC::QB);
        const float *Dt = lse2 + BQ;
        const int q0 = (qt0 + it % nqt) * BQ;
        const int j = half;   // this wave's 32 queries of the tile
        if (q0 + j * 32 + 31 >= kw0 && kw0 < p.T) {
            {
                f32x16 S, dP;
#pragma unroll
                for (int r = 0; r < 16; r++) S[r] = dP[r] = 0.f;
                mma_rows<T, HD>(S, Qs, j * 32, kf, lane);
                mma_rows<T, HD>(dP, dOs, j * 32, vf, lane);
                const bool diag = q0 + j * 32 < kw0 + 31;
                // the 16 query rows of this lane: 4 groups of 4 consecutive rows
#pragma unroll
                for (int r4 = 0; r4 < 4; r4++) {
                    const int qg = j * 32 + 8 * r4 + 4 * g;
                    const f32x4 lq = *reinterpret_cast<const f32x4 *>(lse2 + qg);
                    const f32x4 dq4 = *reinterpret_cast<const f32x4 *>(Dt + qg);
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        const int r = 4 * r4 + e;
                        float pr = exp2f(fmaf(S[r], p.sl2, -lq[e]));
                        if (diag && q0 + qg + e < ki) pr = 0.f;
                        S[r] = pr;
                        dP[r] = pr * (dP[r] - dq4[e]);
                    }
                }
                mma_trans<T, HD, BQ>(dV, S, dOt, j, lane);
                mma_trans<T, HD, BQ>(dK, dP, Qt, j, lane);
            }
        }
        if (more) dkv_stage_store<T, HD>(reg, aux, smem + ((it + 1) & 1) * FC::STAGE, (qt0 + (it + 1) % nqt) * BQ, p.T);
        __syncthreads();
    }
    // sum the two halves of each slice (the stages are free after the last barrier)
    {
        float *xk = reinterpret_cast<float *>(smem) + slice * (2 * A::ND * 16 * 64);
        float *xv = xk + A::ND * 16 * 64;
        if (half == 1) {
#pragma unroll
            for (int d = 0; d < A::ND; d++)
#pragma unroll
                for (int r = 0; r < 16; r++) {
                    xk[(d * 16 + r) * 64 + lane] = dK[d][r];
                    xv[(d * 16 + r) * 64 + lane] = dV[d][r];
                }
        }
        __syncthreads();
        if (half == 1) return;
#pragma unroll
        for (int d = 0; d < A::ND; d++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                dK[d][r] += xk[(d * 16 + r) * 64 + lane];
                dV[d][r] += xv[(d * 16 + r) * 64 + lane];
            }
    }
    if (p.rope_cs) rope_rotate_acc<A::ND>(dK, p.rope_cs + (long long)min(ki, p.T - 1) * (p.hd / 2), p.hd, -1.f, lane);
    if (ki < p.T) {
        T *row = reinterpret_cast<T *>(p.o) + ((long long)b * p.T + ki) * p.QKV + p.C + kh * p.hd;
        store_rows<T, HD>(row, dK, p.scale, p.hd, lane);
        store_rows<T, HD>(row + p.NKV * p.hd, dV, 1.f, p.hd, lane);
    }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
template <typename K> static hipError_t set_lds(K kernel, int bytes) {
    return hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
}

static int pad_hd(int hd, int dtype) {
    int m = dtype == DTB_BF16 ? 16 : 8;
    int p = m;
    while (p < hd) p <<= 1;
    return p;
}

template <typename T, int HD> static hipError_t fwd_t(const AttnP &p, hipStream_t s) {
    using FC = FwdCfg<T, HD>;
    // set on every launch (per device), no first-device-only flag
    hipError_t e = set_lds(attn_fwd_kernel<T, HD>, FC::LDS);
    if (e != hipSuccess) return e;
    int nqb = (p.T + FC::BQ - 1) / FC::BQ;
    DTB_LAUNCH((attn_fwd_kernel<T, HD>), dim3(nqb * p.B * p.NH), dim3(256), FC::LDS, s, p);
    return last_error();
}

template <typename T, int HD> static hipError_t bwd_t(const AttnP &p, float *D, hipStream_t s) {
    using QC = DqCfg<T, HD>;
    using KC = DkvCfg<T, HD>;
    hipError_t e = set_lds(attn_bwd_dq_kernel<T, HD>, QC::LDS);
    if (e != hipSuccess) return e;
    e = set_lds(attn_bwd_dkv_kernel<T, HD>, KC::LDS);
    if (e != hipSuccess) return e;
    long long rows = (long long)p.B * p.T;
    DTB_LAUNCH((attn_bwd_dot_kernel<T>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, p, D);
    e = last_error();
    if (e != hipSuccess) return e;
    AttnP q = p;
    q.D = D;
    int nqb = (p.T + QC::BQ - 1) / QC::BQ;
    DTB_LAUNCH((attn_bwd_dq_kernel<T, HD>), dim3(nqb * p.B * p.NH), dim3(256), QC::LDS, s, q);
    e = last_error();
    if (e != hipSuccess) return e;
    int nkb = (p.T + KC::BK - 1) / KC::BK;
    DTB_LAUNCH((attn_bwd_dkv_kernel<T, HD>), dim3(nkb * p.B * p.NKV), dim3(256), KC::LDS, s, q);
    return last_error();
}

// bf16: the dQ kernel computes -D and -lse / scale per query (it holds the
// query's dO row) and stores them for the dK/dV kernel
static hipError_t bwd_bf16(const AttnP &p, int hdp, float *D, hipStream_t s) {
    float *lsn = D + (long long)p.B * p.NH * p.T;
    AttnP q = p;
    q.D = D;
    q.lsn = lsn;
    return attn_bwd_bf16(q, hdp, s);
}

static AttnP make_params(const void *qkv, int B, int T, int C, int NH, int NKV) {
    AttnP p{};
    p.qkv = qkv;
    p.B = B; p.T = T; p.C = C; p.NH = NH; p.NKV = NKV;
    p.hd = C / NH;
    p.QKV = C + 2 * NKV * p.hd;
    p.scale = 1.f / sqrtf((float)p.hd);
    p.sl2 = p.scale * LOG2E;
    return p;
}

#define DTB_HD_DISPATCH(FN, T, hdp, ...)                 \
    (hdp == 8     ? FN<T, 8>(__VA_ARGS__)                \
     : hdp == 16  ? FN<T, 16>(__VA_ARGS__)               \
     : hdp == 32  ? FN<T, 32>(__VA_ARGS__)               \
     : hdp == 64  ? FN<T, 64>(__VA_ARGS__)               \
                  : FN<T, 128>(__VA_ARGS__))

int launch_attn_forward(void *out, float *lse, const void *qkv, int B, int T, int C, int NH, int NKV, int dtype,
                        hipStream_t s) {
    if (B == 0 || T == 0) return DTB_OK;
    AttnP p = make_params(qkv, B, T, C, NH, NKV);
    p.o = out;
    p.lse = lse;
    int hdp = pad_hd(p.hd, dtype);
    if (g_timing_on) timing_begin(s, K_ATTN_FWD);
    hipError_t e = dtype == DTB_BF16 ? attn_fwd_bf16(p, hdp, s) : DTB_HD_DISPATCH(fwd_t, float, hdp, p, s);
    if (e != hipSuccess) return set_launch_error(e, "attn_forward");
    if (g_timing_on) {
        double es = dtype == DTB_BF16 ? 2 : 4;
        double flops = 4.0 * p.hd * (double)NH * B * (double)T * (T + 1) / 2;
        double bytes = es * (double)B * T * (p.QKV + C) + 4.0 * B * NH * T;
        timing_end(s, K_ATTN_FWD, flops, bytes);
    }
    return DTB_OK;
}

int launch_attn_backward(void *dqkv, const void *qkv, const void *out, const void *dout, const float *lse, int B,
                         int T, int C, int NH, int NKV, int dtype, float *D, const float *rope_cs, hipStream_t s) {
    if (B == 0 || T == 0) return DTB_OK;
    AttnP p = make_params(qkv, B, T, C, NH, NKV);
    p.rope_cs = reinterpret_cast<const float2 *>(rope_cs);
    p.o = dqkv;
    p.out = out;
    p.dout = dout;
    p.lse_in = lse;
    int hdp = pad_hd(p.hd, dtype);
    if (g_timing_on) timing_begin(s, K_ATTN_BWD);
    hipError_t e = dtype == DTB_BF16 ? bwd_bf16(p, hdp, D, s) : DTB_HD_DISPATCH(bwd_t, float, hdp, p, D, s);
    if (e != hipSuccess) return set_launch_error(e, "attn_backward");
    if (g_timing_on) {
        double es = dtype == DTB_BF16 ? 2 : 4;
        double flops = 2.5 * 4.0 * p.hd * (double)NH * B * (double)T * (T + 1) / 2;
        double bytes = es * (double)B * T * (2.0 * p.QKV + 2.0 * C) + 4.0 * B * NH * T;
        timing_end(s, K_ATTN_BWD, flops, bytes);
    }
    return DTB_OK;
}

}  // namespace dtb
