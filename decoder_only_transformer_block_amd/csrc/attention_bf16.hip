// Causal grouped-query flash attention in bf16 for gfx950.
//
// What is computed ("nanoeuler — CUDA kernels": the flash attention forward /
// backward declarations and the CPU attention definitions): s_tj = q_t.k_j /
// sqrt(hd) for j <= t, o_t = softmax(s_t) V, lse_t = logsumexp_j s_tj; query
// head h reads kv head h / (NH / NKV).
//
// Design:
// * Tiles of 64 positions x HD (the head width padded to 16/32/64/128) are
//   staged in LDS in their natural row-major form only, by buffer loads that
//   write LDS directly (no VGPR staging), into a ring of NS stages: the tile
//   NS-1 steps ahead is issued while the current one is multiplied.  The
//   16-byte chunk index of a row is XOR-ed with a function of the row; the
//   permutation is applied by choosing which global chunk each lane loads, so
//   every row is still fetched as whole contiguous segments.
// * Scores are computed transposed, S^T = K Q^T, so a lane owns one query
//   (column l%32) and 16 keys of each 32x32 block; K is read as rows
//   (ds_read_b128).  The product O^T += V^T P^T takes P^T from the score
//   registers as its B operand (the k order of an MFMA is free as long as both
//   operands follow it: lane half g holds keys 4g..4g+3 and 8+4g..8+4g+3 of
//   each 16-key step), and V^T fragments come from the natural V tile through
//   the transposing read ds_read_b64_tr_b16: within a 16-lane group, lane i
//   addresses (key kb + i/4, head dims d0 + 4(i%4) .. +3) and lane l receives
//   keys kb..kb+3 of head dim d0 + l.
// * Every lane's LDS addresses are a per-lane base plus compile-time offsets.
// * The online softmax runs in base 2 with the hardware exp2.
#include "attention.h"
#include "attn_tiles.h"

namespace dtb {
namespace {

// A wave's DMA instructions qsub .. qsub+N-1 of every 64-row tile of one
// row-major tensor.  The per-lane byte offsets within a tile do not change
// from tile to tile, so they are computed once (tile_dma_offsets); the rows
// past the valid range are zero-filled by the buffer's record count (a tile at
// row0 gets a record of (nrows - row0) rows), and head dims past hd by an
// out-of-range offset.  Issuing a tile (tile_dma_issue) then costs scalar work
// only.
enum { SWZ_ROWS, SWZ_COLS, SWZ_DUAL };  // which chunk swizzle a tile is stored with
template <int HD, int MODE, int N>
__device__ __forceinline__ void tile_dma_offsets(int (&voff)[N], long long stride, int hd, int qsub, int lane) {
    constexpr int RB = TL<HD>::RB;
#pragma unroll
    for (int i = 0; i < N; i++) {
        const int off = (qsub + i) * 1024 + lane * 16;
        const int r = off / RB, pc = (off % RB) >> 4;
        const int c = pc ^ (MODE == SWZ_COLS ? swz_cols<HD>(r) : MODE == SWZ_DUAL ? swz_dual<HD>(r) : swz_rows<HD>(r));
        voff[i] = c * 8 < hd ? (int)((r * stride + c * 8) * 2) : (int)0x80000000;
    }
}
template <int N>
__device__ __forceinline__ void tile_dma_issue(char *lds, const bf16 *g, long long stride, int row0, int nrows,
                                               const int *voff, int qsub) {
    const long long rows = nrows > row0 ? nrows - row0 : 0;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16 *>(g + (long long)row0 * stride), (short)0, (int)(rows * stride * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < N; i++)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_vptr)(lds + (qsub + i) * 1024), 16, voff[i], 0, 0, 0);
}

// 64 fp32 values (4 bytes per lane) of a row of a [rows][T] array into LDS
__device__ __forceinline__ void dma_vec64(char *lds, const float *g, int q0, int n, bool live, int lane) {
    const Buf buf(g);
    const bool ok = live && q0 + lane < n;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(buf.r, (lds_vptr)lds, 4, ok ? (q0 + lane) * 4 : (int)0x80000000, 0, 0, 0);
}

// write ND accumulator blocks (lane = position, registers = head dim) scaled by s
template <int HD>
__device__ __forceinline__ void store_rows_bf16(bf16 *row, const f32x16 *acc, float s, int hd, int lane) {
#pragma unroll
    for (int db = 0; db < TL<HD>::ND; db++)
#pragma unroll
        for (int r4 = 0; r4 < 4; r4++) {
            const int d = db * 32 + 8 * r4 + 4 * (lane >> 5);
            if (d < hd) {
                u32x2 v{pack2_bf16(acc[db][4 * r4] * s, acc[db][4 * r4 + 1] * s),
                        pack2_bf16(acc[db][4 * r4 + 2] * s, acc[db][4 * r4 + 3] * s)};
                *reinterpret_cast<u32x2 *>(row + d) = v;
            }
        }
}

// ---------------------------------------------------------------------------
// forward: one workgroup = 4 waves x 32 queries of one (b, h); key tiles of 64;
// last query blocks launched first (causal load balance)
// ---------------------------------------------------------------------------
// (query block, b*NH + h) of a query-owning workgroup.  Workgroups go to the
// eight XCDs round robin; when the B*NKV head groups split evenly over them,
// the G = NH/NKV query heads of a group (which read the same K / V tiles) are
// placed on one XCD one after another, so that XCD's L2 serves all of them.
// Heaviest query blocks still come first.
__device__ __forceinline__ void qowner_coords(int x, int nqb, int B, int NH, int NKV, int &qb, int &bh) {
    const int BH = B * NH, NG = B * NKV, G = NH / NKV;
    if (NG % 8 != 0) {
        qb = nqb - 1 - x / BH;
        bh = x % BH;
        return;
    }
    const int xcd = x & 7, r = x >> 3;
    const int hg = r % G, t = r / G;
    const int g = (t % (NG / 8)) * 8 + xcd;
    qb = nqb - 1 - t / (NG / 8);
    bh = g * G + hg;
}

// Head width 64 runs a two-stage ring (32 KB of LDS, five workgroups' worth
// per CU) held to 128 VGPRs: four waves per SIMD.  One register spills, kept
// across the loop only.
template <int HD, int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HD == 64 && NS == 2 ? 4 : 1, 8))) void
fwd_bf16_kernel(AttnP p) {
    using L = TL<HD>;
    constexpr int BQ = 128, BKV = 64, RB = L::RB;
    constexpr int DPW = L::NDMA / 2;  // DMA instructions per wave per tile (waves 0-1: K, 2-3: V)
    constexpr int STB = 2 * L::TILE;
    __shared__ __attribute__((aligned(1024))) char s0[STB];
    __shared__ __attribute__((aligned(1024))) char s1[STB];
    __shared__ __attribute__((aligned(1024))) char s2[NS > 2 ? STB : 16];
#define STG(S) ((S) == 0 ? s0 : (S) == 1 ? s1 : s2)

    const int nqb = (p.T + BQ - 1) / BQ, BH = p.B * p.NH;
    int qb, bh;
    qowner_coords((int)blockIdx.x, nqb, p.B, p.NH, p.NKV, qb, bh);
    const int b = bh / p.NH, h = bh % p.NH, kh = h / (p.NH / p.NKV);
    const int t = threadIdx.x, lane = t & 63, g = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int q0 = qb * BQ, qw0 = q0 + wave * 32, qi = qw0 + l32;
    const long long stride = p.QKV;
    const bf16 *base = reinterpret_cast<const bf16 *>(p.qkv) + (long long)b * p.T * stride;
    const bf16 *kbase = base + p.C + kh * p.hd;
    const bf16 *vbase = kbase + p.NKV * p.hd;
    const int kv_end = min(p.T, q0 + BQ);
    const int ntiles = (kv_end + BKV - 1) / BKV;
    const int wtiles = qw0 < p.T ? min(qw0 + 31, p.T - 1) / BKV + 1 : 0;

    const bool isK = wave < 2;
    const bf16 *src = isK ? kbase : vbase;
    const int qsub = (wave & 1) * DPW;
    int voff[DPW];   // K rows and V columns use different swizzles
    if (isK) tile_dma_offsets<HD, SWZ_ROWS>(voff, stride, p.hd, qsub, lane);
    else tile_dma_offsets<HD, SWZ_COLS>(voff, stride, p.hd, qsub, lane);
    auto issue = [&](char *st, int kt) {
        tile_dma_issue<DPW>(st + (isK ? 0 : L::TILE), src, stride, kt * BKV, kv_end, voff, qsub);
    };

    // query fragments (chunks 2c+g of row qi), then the first NS-1 tiles
    u32x4 qf[L::NC];
    {
        const Buf bq(base + h * p.hd);
#pragma unroll
        for (int c = 0; c < L::NC; c++) {
            const int ch = 2 * c + g;
            qf[c] = bq.ld16((int)(((long long)qi * stride + ch * 8) * 2), qi < p.T && ch * 8 < p.hd);
        }
    }
    issue(s0, 0);
    if (NS > 2) issue(s1, 1);

    int kofs[L::NC];
#pragma unroll
    for (int c = 0; c < L::NC; c++) kofs[c] = l32 * RB + (((2 * c + g) ^ swz_rows<HD>(l32)) << 4);
    int vofs[L::ND];
    {
        const int i16 = lane & 15, vr = 4 * g + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < L::ND; db++) {
            const int d = 32 * db + (l32 & 16) + 4 * (i16 & 3);
            const int ch = (d >> 3) & (L::NCH - 1);
            vofs[db] = vr * RB + ((ch ^ swz_cols<HD>(vr)) << 4) + 8 * (i16 & 1);
        }
    }

    f32x16 O[L::ND];
#pragma unroll
    for (int d = 0; d < L::ND; d++)
#pragma unroll
        for (int r = 0; r < 16; r++) O[d][r] = 0.f;
    float m = -1e30f;
    // the softmax row sums ride on the P V product: an A operand that is 1 in
    // row 0 and 0 elsewhere gives row 0 of Ls = sum over keys of the (bf16) P
    // of each query column, in the accumulator of lanes 0..31 (no VALU adds)
    f32x16 Ls;
#pragma unroll
    for (int r = 0; r < 16; r++) Ls[r] = 0.f;
    const bf16x8 ones = __builtin_bit_cast(
        bf16x8, (l32 == 0) ? u32x4{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u} : u32x4{0u, 0u, 0u, 0u});

    auto compute = [&](const char *st, int kt) {
        const char *Ks = st, *Vs = st + L::TILE;
        const int kv0 = kt * BKV;
        f32x16 S[2];
#pragma unroll
        for (int j = 0; j < 2; j++) {
#pragma unroll
            for (int r = 0; r < 16; r++) S[j][r] = 0.f;
#pragma unroll
            for (int c = 0; c < L::NC; c++)
                S[j] = mfma32(lds_row16(Ks + kofs[c] + j * 32 * RB), __builtin_bit_cast(bf16x8, qf[c]), S[j]);
        }
        if (kv0 + BKV - 1 > qw0) {  // diagonal tile
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int r = 0; r < 16; r++)
                    if (kv0 + j * 32 + acc_row(r, lane) > qi) S[j][r] = -INFINITY;
        }
        float sv[32];
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) sv[16 * j + r] = S[j][r];
        const float mt = max_xor32(tree_max<32>(sv)) * p.sl2;  // tile max in log2 units
        // the reference max m moves only when a column's scores exceed it by
        // more than 2^8 (then O and the sums are rescaled); otherwise the
        // exponentials below stay under 256 and no rescale is spent
        if (!__all(mt <= m + 8.f)) {
            const float mn = fmaxf(m, mt);
            const float alpha = fast_exp2(m - mn);
            Ls[0] *= alpha;
#pragma unroll
            for (int d = 0; d < L::ND; d++)
#pragma unroll
                for (int r = 0; r < 16; r++) O[d][r] *= alpha;
            m = mn;
        }
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int r = 0; r < 16; r++) S[j][r] = fast_exp2(fmaf(S[j][r], p.sl2, -m));
#pragma unroll
        for (int j = 0; j < 2; j++)
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                u32x4 xw;
#pragma unroll
                for (int e = 0; e < 4; e++) xw[e] = pack2_bf16(S[j][8 * hh + 2 * e], S[j][8 * hh + 2 * e + 1]);
                const bf16x8 xb = __builtin_bit_cast(bf16x8, xw);
#pragma unroll
                for (int db = 0; db < L::ND; db++)
                    O[db] = mfma32(lds_tr8<RB>(Vs + vofs[db] + (32 * j + 16 * hh) * RB), xb, O[db]);
                Ls = mfma32(ones, xb, Ls);
            }
    };

    // all fragment and prologue loads complete before the loop
    __builtin_amdgcn_s_waitcnt(0);
#define FWD_STEP(S)                                                              \
    {                                                                            \
        const int kt = kt0 + (S);                                                \
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NS - 2) * DPW));               \
        asm volatile("s_barrier" ::: "memory");                                  \
        issue(STG(((S) + NS - 1) % NS), kt + NS - 1);                            \
        if (kt < wtiles) compute(STG(S), kt);                                    \
    }
    for (int kt0 = 0; kt0 < ntiles; kt0 += NS) {
        FWD_STEP(0)
        FWD_STEP(1)
        if constexpr (NS > 2) FWD_STEP(2)
    }
#undef FWD_STEP
#undef STG
    __builtin_amdgcn_s_waitcnt(0);

    // row 0 of Ls sits in register 0 of lanes 0..31; lanes 32..63 take it from their partner
    const float ltot = __shfl(Ls[0], l32, 64);
    if (qi < p.T) {
        bf16 *orow = reinterpret_cast<bf16 *>(p.o) + ((long long)b * p.T + qi) * p.C + h * p.hd;
        store_rows_bf16<HD>(orow, O, 1.f / ltot, p.hd, lane);
        if (g == 0) p.lse[((long long)b * p.NH + h) * p.T + qi] = (m + log2f(ltot)) * LN2;
    }
}

template <int HD> hipError_t fwd_launch(const AttnP &p, hipStream_t s) {
    constexpr int NS = HD >= 64 ? 2 : 3;
    const int nqb = (p.T + 127) / 128;
    DTB_LAUNCH((fwd_bf16_kernel<HD, NS>), dim3(nqb * p.B * p.NH), dim3(256), 0, s, p);
    return last_error();
}


// ---------------------------------------------------------------------------
// backward dQ: one workgroup = 4 waves x 32 queries of one (b, h), key tiles of
// 64 (K and V, natural).  S^T = K Q^T and dP^T = V dO^T from the tile rows,
// dS^T = P^T (dP^T - D), dQ^T += K^T dS^T with K^T through transposing reads.
// ---------------------------------------------------------------------------
template <int HD, int NS>
__global__ __launch_bounds__(256) void dq_bf16_kernel(AttnP p) {
    using L = TL<HD>;
    constexpr int BQ = 128, BKV = 64, RB = L::RB;
    constexpr int DPW = L::NDMA / 2;
    constexpr int STB = 2 * L::TILE;
    __shared__ __attribute__((aligned(1024))) char s0[STB];
    __shared__ __attribute__((aligned(1024))) char s1[STB];
    __shared__ __attribute__((aligned(1024))) char s2[NS > 2 ? STB : 16];
#define STG(S) ((S) == 0 ? s0 : (S) == 1 ? s1 : s2)

    const int nqb = (p.T + BQ - 1) / BQ, BH = p.B * p.NH;
    int qb, bh;
    qowner_coords((int)blockIdx.x, nqb, p.B, p.NH, p.NKV, qb, bh);
    const int b = bh / p.NH, h = bh % p.NH, kh = h / (p.NH / p.NKV);
    const int t = threadIdx.x, lane = t & 63, g = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int q0 = qb * BQ, qw0 = q0 + wave * 32, qi = qw0 + l32;
    const long long stride = p.QKV;
    const bf16 *base = reinterpret_cast<const bf16 *>(p.qkv) + (long long)b * p.T * stride;
    const bf16 *kbase = base + p.C + kh * p.hd;
    const bf16 *vbase = kbase + p.NKV * p.hd;
    const int kv_end = min(p.T, q0 + BQ);
    const int ntiles = (kv_end + BKV - 1) / BKV;
    const int wtiles = qw0 < p.T ? min(qw0 + 31, p.T - 1) / BKV + 1 : 0;

    const bool isK = wave < 2;
    const bf16 *src = isK ? kbase : vbase;
    const int qsub = (wave & 1) * DPW;
    int voff[DPW];
    tile_dma_offsets<HD, SWZ_DUAL>(voff, stride, p.hd, qsub, lane);
    auto issue = [&](char *st, int kt) {
        tile_dma_issue<DPW>(st + (isK ? 0 : L::TILE), src, stride, kt * BKV, kv_end, voff, qsub);
    };

    u32x4 qf[L::NC], df[L::NC];
    const long long li = ((long long)b * p.NH + h) * p.T + qi;
    float nls = 0.f, nDq = 0.f;  // -lse / scale and -D of this lane's query
    {
        const Buf bq(base + h * p.hd);
        const Buf bd(reinterpret_cast<const bf16 *>(p.dout) + (long long)b * p.T * p.C + h * p.hd);
        const Buf bo(reinterpret_cast<const bf16 *>(p.out) + (long long)b * p.T * p.C + h * p.hd);
        // D = rowsum(dO o) of this lane's query: the lane holds chunks 2c + g
        // of the row, its partner (lane ^ 32) the others
        float dot = 0.f;
#pragma unroll
        for (int c = 0; c < L::NC; c++) {
            const int ch = 2 * c + g;
            const bool ok = qi < p.T && ch * 8 < p.hd;
            qf[c] = bq.ld16((int)(((long long)qi * stride + ch * 8) * 2), ok);
            df[c] = bd.ld16((int)(((long long)qi * p.C + ch * 8) * 2), ok);
            const u32x4 of = bo.ld16((int)(((long long)qi * p.C + ch * 8) * 2), ok);
#pragma unroll
            for (int e = 0; e < 4; e++)
                dot += __uint_as_float(df[c][e] << 16) * __uint_as_float(of[e] << 16) +
                       __uint_as_float(df[c][e] & 0xffff0000u) * __uint_as_float(of[e] & 0xffff0000u);
        }
        dot = sum_xor32(dot);
        if (qi < p.T) {
            // also kept for the dK/dV kernel, which runs after this one
            nls = -p.lse_in[li] / p.scale;
            nDq = -dot;
            if (g == 0) {
                p.lsn[li] = nls;
                p.D[li] = nDq;
            }
        }
    }
    issue(s0, 0);
    if (NS > 2) issue(s1, 1);

    int kofs[L::NC];
#pragma unroll
    for (int c = 0; c < L::NC; c++) kofs[c] = l32 * RB + (((2 * c + g) ^ swz_dual<HD>(l32)) << 4);
    int tofs[L::ND];
    {
        const int i16 = lane & 15, xr = 4 * g + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < L::ND; db++) {
            const int d = 32 * db + (l32 & 16) + 4 * (i16 & 3);
            const int ch = (d >> 3) & (L::NCH - 1);
            tofs[db] = xr * RB + ((ch ^ swz_dual<HD>(xr)) << 4) + 8 * (i16 & 1);
        }
    }
    int tofs8[L::ND];  // the transposing reads' second 8 rows
#pragma unroll
    for (int db = 0; db < L::ND; db++) tofs8[db] = tofs[db] ^ dual_x8<HD>();

    f32x16 dQ[L::ND];
#pragma unroll
    for (int d = 0; d < L::ND; d++)
#pragma unroll
        for (int r = 0; r < 16; r++) dQ[d][r] = 0.f;

    auto compute = [&](const char *st, int kt) {
        const char *Ks = st, *Vs = st + L::TILE;
        const int kv0 = kt * BKV;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            // S starts from -lse / scale and dP from -D of this lane's query
            // (every element of the lane's column shares them): P = 2^(S sl2)
            // is one multiply and an exp, dS = P * dP one multiply
            f32x16 S, dP;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                S[r] = nls;
                dP[r] = nDq;
            }
#pragma unroll
            for (int c = 0; c < L::NC; c++) {
                S = mfma32(lds_row16(Ks + kofs[c] + j * 32 * RB), __builtin_bit_cast(bf16x8, qf[c]), S);
                dP = mfma32(lds_row16(Vs + kofs[c] + j * 32 * RB), __builtin_bit_cast(bf16x8, df[c]), dP);
            }
            // causal mask on diagonal blocks only: a real (uniform) branch, kept
            // from being flattened into per-element selects on every block
            if (kv0 + j * 32 + 31 > qw0) {
                asm volatile("");
#pragma unroll
                for (int r = 0; r < 16; r++)
                    if (kv0 + j * 32 + acc_row(r, lane) > qi) S[r] = -INFINITY;
            }
#pragma unroll
            for (int r = 0; r < 16; r++) S[r] = fast_exp2(S[r] * p.sl2) * dP[r];
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                u32x4 xw;
#pragma unroll
                for (int e = 0; e < 4; e++) xw[e] = pack2_bf16(S[8 * hh + 2 * e], S[8 * hh + 2 * e + 1]);
                const bf16x8 xb = __builtin_bit_cast(bf16x8, xw);
#pragma unroll
                for (int db = 0; db < L::ND; db++)
                    dQ[db] = mfma32(lds_tr8x<RB>(Ks + tofs[db] + (32 * j + 16 * hh) * RB,
                                                 Ks + tofs8[db] + (32 * j + 16 * hh) * RB), xb, dQ[db]);
            }
        }
    };

    __builtin_amdgcn_s_waitcnt(0);
#define BWD_STEP(S)                                                              \
    {                                                                            \
        const int kt = kt0 + (S);                                                \
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NS - 2) * DPW));               \
        asm volatile("s_barrier" ::: "memory");                                  \
        issue(STG(((S) + NS - 1) % NS), kt + NS - 1);                            \
        if (kt < wtiles) compute(STG(S), kt);                                    \
    }
    for (int kt0 = 0; kt0 < ntiles; kt0 += NS) {
        BWD_STEP(0)
        BWD_STEP(1)
        if constexpr (NS > 2) BWD_STEP(2)
    }
#undef BWD_STEP
#undef STG
    __builtin_amdgcn_s_waitcnt(0);
    if (p.rope_cs) rope_rotate_acc<L::ND>(dQ, p.rope_cs + (long long)min(qi, p.T - 1) * (p.hd / 2), p.hd, -1.f, lane);
    if (qi < p.T) {
        bf16 *row = reinterpret_cast<bf16 *>(p.o) + ((long long)b * p.T + qi) * p.QKV + h * p.hd;
        store_rows_bf16<HD>(row, dQ, p.scale, p.hd, lane);
    }
}

// ---------------------------------------------------------------------------
// backward dK, dV: one workgroup = 4 waves x 32 keys of one (b, kv head),
// looping over the group's query heads and the query tiles (64) at or after
// its keys, so dK / dV are summed over the group in registers (no atomics).
// S = Q K^T and dP = dO V^T from the tile rows, dV^T += dO^T P and
// dK^T += Q^T dS with dO^T and Q^T through transposing reads.  A stage holds
// the Q tile, the dO tile and the 64 lse*log2(e) and D values of its queries.
// ---------------------------------------------------------------------------
// Register target: 3 waves per SIMD at HD <= 64 (the LDS of three workgroups
// fits), 2 at HD = 128, where the compiler alone chose 268 registers (one
// wave) and 2 waves with 13 spilled registers measured 6 % faster.
template <int HD, int NS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(HD >= 128 ? 2 : 3, 8))) void dkv_bf16_kernel(
    AttnP p) {
    using L = TL<HD>;
    constexpr int BK = 128, BQ = 64, RB = L::RB;
    constexpr int DPW = L::NDMA / 2 + 1;   // tile share plus one 256-byte vector
    constexpr int AUX = 2 * L::TILE;       // [-lse/scale 64][-D 64][unused 128 floats]
    constexpr int STB = 2 * L::TILE + 1024;
    __shared__ __attribute__((aligned(1024))) char s0[STB];
    __shared__ __attribute__((aligned(1024))) char s1[STB];
    __shared__ __attribute__((aligned(1024))) char s2[NS > 2 ? STB : 16];
#define STG(S) ((S) == 0 ? s0 : (S) == 1 ? s1 : s2)

    const int BKVH = p.B * p.NKV;
    const int kb = (int)(blockIdx.x / BKVH);  // low key blocks (most work) first
    const int bk = blockIdx.x % BKVH;
    const int b = bk / p.NKV, kh = bk % p.NKV;
    const int grp = p.NH / p.NKV;
    const int t = threadIdx.x, lane = t & 63, g = lane >> 5, l32 = lane & 31;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int k0 = kb * BK, kw0 = k0 + wave * 32, ki = kw0 + l32;
    const long long stride = p.QKV;
    const bf16 *base = reinterpret_cast<const bf16 *>(p.qkv) + (long long)b * p.T * stride;
    const bf16 *dbase = reinterpret_cast<const bf16 *>(p.dout) + (long long)b * p.T * p.C;

    const int qt0 = k0 / BQ;                    // first query tile touching these keys
    const int nqt = (p.T + BQ - 1) / BQ - qt0;  // query tiles per head
    const int niter = nqt * grp;

    const bool isQ = wave < 2;
    const int qsub = (wave & 1) * (DPW - 1);
    const long long st_ = isQ ? stride : (long long)p.C;
    int voff[DPW - 1];
    tile_dma_offsets<HD, SWZ_DUAL>(voff, st_, p.hd, qsub, lane);
    auto issue = [&](char *st, int it) {
        const bool live = it < niter;
        const int hh = live ? it / nqt : 0, q0 = (qt0 + (live ? it % nqt : 0)) * BQ;
        const int h = kh * grp + hh;
        const bf16 *src = isQ ? base + h * p.hd : dbase + h * p.hd;
        tile_dma_issue<DPW - 1>(st + (isQ ? 0 : L::TILE), src, st_, q0, live ? p.T : 0, voff, qsub);
        const float *vec = (wave == 0 ? p.lsn : p.D) + ((long long)b * p.NH + h) * p.T;
        dma_vec64(st + AUX + wave * 256, vec, q0, p.T, live && wave < 2, lane);
    };

    u32x4 kf[L::NC], vf[L::NC];
    {
        const Buf bkk(base + p.C + kh * p.hd);
        const Buf bvv(base + p.C + (p.NKV + kh) * p.hd);
#pragma unroll
        for (int c = 0; c < L::NC; c++) {
            const int ch = 2 * c + g;
            const bool ok = ki < p.T && ch * 8 < p.hd;
            kf[c] = bkk.ld16((int)(((long long)ki * stride + ch * 8) * 2), ok);
            vf[c] = bvv.ld16((int)(((long long)ki * stride + ch * 8) * 2), ok);
        }
    }
    issue(s0, 0);
    if (NS > 2) issue(s1, 1);

    int kofs[L::NC];
#pragma unroll
    for (int c = 0; c < L::NC; c++) kofs[c] = l32 * RB + (((2 * c + g) ^ swz_dual<HD>(l32)) << 4);
    int tofs[L::ND];
    {
        const int i16 = lane & 15, xr = 4 * g + (i16 >> 2);
#pragma unroll
        for (int db = 0; db < L::ND; db++) {
            const int d = 32 * db + (l32 & 16) + 4 * (i16 & 3);
            const int ch = (d >> 3) & (L::NCH - 1);
            tofs[db] = xr * RB + ((ch ^ swz_dual<HD>(xr)) << 4) + 8 * (i16 & 1);
        }
    }
    int tofs8[L::ND];  // the transposing reads' second 8 rows
#pragma unroll
    for (int db = 0; db < L::ND; db++) tofs8[db] = tofs[db] ^ dual_x8<HD>();

    f32x16 dK[L::ND], dV[L::ND];
#pragma unroll
    for (int d = 0; d < L::ND; d++)
#pragma unroll
        for (int r = 0; r < 16; r++) dK[d][r] = dV[d][r] = 0.f;

    auto compute = [&](const char *st, int it) {
        const char *Qs = st, *dOs = st + L::TILE;
        const float *lss = reinterpret_cast<const float *>(st + AUX), *Ds = lss + BQ;
        const int q0 = (qt0 + it % nqt) * BQ;
#pragma unroll
        for (int j = 0; j < 2; j++) {
            // the 16 query rows of this lane: 4 groups of 4 consecutive rows;
            // lss holds -lse / scale and Ds -D, read in the accumulator's row
            // order, so S = Q K^T accumulates from the first (P = 2^(S sl2))
            // and dP = dO V^T from the second (it ends as dP - D); no per-row
            // value stays live across the MFMAs
            f32x16 S, dP;
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++) {
                const int ql = j * 32 + 8 * r4 + 4 * g;
                const f32x4 ls = *reinterpret_cast<const f32x4 *>(lss + ql);
                const f32x4 nd = *reinterpret_cast<const f32x4 *>(Ds + ql);
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    S[4 * r4 + e] = ls[e];
                    dP[4 * r4 + e] = nd[e];
                }
            }
#pragma unroll
            for (int c = 0; c < L::NC; c++) {
                S = mfma32(lds_row16(Qs + kofs[c] + j * 32 * RB), __builtin_bit_cast(bf16x8, kf[c]), S);
                dP = mfma32(lds_row16(dOs + kofs[c] + j * 32 * RB), __builtin_bit_cast(bf16x8, vf[c]), dP);
            }
            const bool diag = q0 + j * 32 < kw0 + 31;
            // causal mask on diagonal blocks only (a real uniform branch, as in dQ)
            if (diag) {
                asm volatile("");
#pragma unroll
                for (int r = 0; r < 16; r++)
                    if (q0 + j * 32 + acc_row(r, lane) < ki) S[r] = -INFINITY;
            }
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const float pr = fast_exp2(S[r] * p.sl2);
                S[r] = pr;
                dP[r] = pr * dP[r];
            }
#pragma unroll
            for (int hh = 0; hh < 2; hh++) {
                u32x4 xs, xd;
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    xs[e] = pack2_bf16(S[8 * hh + 2 * e], S[8 * hh + 2 * e + 1]);
                    xd[e] = pack2_bf16(dP[8 * hh + 2 * e], dP[8 * hh + 2 * e + 1]);
                }
#pragma unroll
                for (int db = 0; db < L::ND; db++) {
                    const int o = tofs[db] + (32 * j + 16 * hh) * RB, o8 = tofs8[db] + (32 * j + 16 * hh) * RB;
                    dV[db] = mfma32(lds_tr8x<RB>(dOs + o, dOs + o8), __builtin_bit_cast(bf16x8, xs), dV[db]);
                    dK[db] = mfma32(lds_tr8x<RB>(Qs + o, Qs + o8), __builtin_bit_cast(bf16x8, xd), dK[db]);
                }
            }
        }
    };

    __builtin_amdgcn_s_waitcnt(0);
#define BWD_STEP(S)                                                              \
    {                                                                            \
        const int it = it0 + (S);                                                \
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NS - 2) * DPW));               \
        asm volatile("s_barrier" ::: "memory");                                  \
        issue(STG(((S) + NS - 1) % NS), it + NS - 1);                            \
        if (it < niter && (qt0 + it % nqt) * BQ + BQ - 1 >= kw0 && kw0 < p.T) compute(STG(S), it); \
    }
    for (int it0 = 0; it0 < niter; it0 += NS) {
        BWD_STEP(0)
        BWD_STEP(1)
        if constexpr (NS > 2) BWD_STEP(2)
    }
#undef BWD_STEP
#undef STG
    __builtin_amdgcn_s_waitcnt(0);
    if (p.rope_cs) rope_rotate_acc<L::ND>(dK, p.rope_cs + (long long)min(ki, p.T - 1) * (p.hd / 2), p.hd, -1.f, lane);
    if (ki < p.T) {
        bf16 *row = reinterpret_cast<bf16 *>(p.o) + ((long long)b * p.T + ki) * p.QKV + p.C + kh * p.hd;
        store_rows_bf16<HD>(row, dK, p.scale, p.hd, lane);
        store_rows_bf16<HD>(row + p.NKV * p.hd, dV, 1.f, p.hd, lane);
    }
}

template <int HD> hipError_t bwd_launch(const AttnP &p, hipStream_t s) {
    constexpr int NS = HD >= 128 ? 2 : 3;
    const int nqb = (p.T + 127) / 128;
    DTB_LAUNCH((dq_bf16_kernel<HD, NS>), dim3(nqb * p.B * p.NH), dim3(256), 0, s, p);
    hipError_t e = last_error();
    if (e != hipSuccess) return e;
    const int nkb = (p.T + 127) / 128;
    DTB_LAUNCH((dkv_bf16_kernel<HD, NS>), dim3(nkb * p.B * p.NKV), dim3(256), 0, s, p);
    return last_error();
}

}  // namespace

hipError_t attn_fwd_bf16(const AttnP &p, int HD, hipStream_t s) {
    switch (HD) {
    case 16: return fwd_launch<16>(p, s);
    case 32: return fwd_launch<32>(p, s);
    case 64: return fwd_launch<64>(p, s);
    case 128: return fwd_launch<128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t attn_bwd_bf16(const AttnP &p, int HD, hipStream_t s) {
    switch (HD) {
    case 16: return bwd_launch<16>(p, s);
    case 32: return bwd_launch<32>(p, s);
    case 64: return bwd_launch<64>(p, s);
    case 128: return bwd_launch<128>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace dtb
