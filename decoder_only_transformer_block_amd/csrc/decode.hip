// Decode attention: one new query per sequence against its KV cache, forward
// only ("microgpt.cu": attention_forward_kernel as forward_position calls it,
// the newest position's query reading the cached keys and values of
// positions 0 .. pos_id).
//
//   out[b, h] = sum_{j < len_b} softmax_j(q_{b,h} . k_{b,j,kh} / sqrt(hd)) v_{b,j,kh}
//   lse[b, h] = natural-log logsumexp_j of the same scores,   kh = h / (NH/NKV)
//
// Layout: q and out [B][NH*hd]; k_cache and v_cache addressed by element
// strides (b, t, kv head): position-major [B][Tmax][NKV*hd] (a cache row holds
// every kv head of one position, as the microgpt cache rows do) or any other
// arrangement of hd-contiguous head rows, e.g. head-major [B][NKV][Tmax][hd];
// lens [B] int32 in device memory; lse [B][NH] fp32.
//
// Design.  The work is bound by HBM: every cached byte is read once and meets
// 2 * (NH/NKV) flops per element.
// * Each sequence's cache is cut into chunks of `chunk` positions.  One wave64
//   workgroup owns (chunk, sequence, kv head, group of query heads); the heads
//   of a group share every K/V tile, so the cache is read once whatever the
//   group size.  The chunk index runs slowest in the grid, so the workgroups
//   of chunks past a sequence's length (which exit at once) gather at the end
//   of the dispatch.
// * bf16: 32-position K and V tiles stream into a private LDS ring by buffer
//   loads that write LDS directly, NS-1 tiles ahead of the MFMAs.  Scores are
//   computed transposed, S^T = K Q^T on 32x32x16 MFMAs whose 32 columns are the
//   group's query heads, and O^T += V^T P^T takes P^T from the score registers
//   and V^T from the tile through the transposing LDS read (the arrangement of
//   the training forward kernel, with heads in place of query positions).
// * fp32: at this intensity no MFMA is needed.  A lane holds 4 head dims of one
//   cached position, scores are summed across the position's lanes, and every
//   lane keeps its own running max / sum / output over the positions it saw;
//   the lanes are merged at the end.
// * A chunk's result is stored unnormalised with its running max (log2 units)
//   and sum; decode_merge_kernel combines the chunks of each (sequence, head)
//   with weights 2^(m_c - M).  A sequence that fits in one chunk is finished by
//   its only workgroup.
#include "attention.h"
#include "attn_tiles.h"

namespace dtb {

struct DecP {
    void *o;            // [B][NH*hd]
    float *lse;         // [B][NH]
    const void *q;      // [B][NH*hd]
    const void *kc;     // head row (b, t, kh) at b*sb + t*st + kh*sh elements
    const void *vc;
    long long sb, st, sh;
    const int *lens;    // [B]
    float *po;          // [nsplit][B][NH][hd] unnormalised chunk outputs
    float2 *pml;        // [nsplit][B][NH] (running max in log2 units, sum)
    int B, NH, NKV, hd, Tmax, chunk, ngrp;
    float sl2;          // log2(e) / sqrt(hd)
};

namespace {

__device__ __forceinline__ bool decode_range(const DecP &p, int b, int split, int &len, int &kv0, int &kv1) {
    len = p.lens[b];
    if (len < 0 || len > p.Tmax) return false;  // reported as NaN by the merge kernel
    kv0 = split * p.chunk;
    kv1 = min(len, kv0 + p.chunk);
    return kv0 < kv1;
}

// one 32-position K tile and V tile at row r0 into LDS (st, st + KT): the
// lanes' offsets within a tile are given, and the rows at or past kv1 are
// zero-filled by the record count of the tile's buffers
template <int NDQ, int KT>
__device__ __forceinline__ void decode_tile_dma(char *st, const bf16 *kc, const bf16 *vc, long long stride, int r0,
                                                int kv1, const int *okof, const int *ovof) {
    const long long nb = r0 < kv1 ? (long long)(kv1 - r0) * stride * 2 : 0;
    const int nrec = (int)(nb < 0x7fffffffLL ? nb : 0x7fffffffLL);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16 *>(kc + (long long)r0 * stride), (short)0, nrec, 0x00020000);
    const __amdgpu_buffer_rsrc_t rv =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<bf16 *>(vc + (long long)r0 * stride), (short)0, nrec, 0x00020000);
#pragma unroll
    for (int i = 0; i < NDQ; i++) {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_vptr)(st + i * 1024), 16, okof[i], 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_vptr)(st + KT + i * 1024), 16, ovof[i], 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// bf16: one wave = (chunk, b, kv head, up to 32 query heads); a workgroup holds
// the waves of W consecutive kv heads of the same positions, so that the
// heads' 128-byte pieces of each cache row (one position's kv heads are
// contiguous) are requested together.  The waves share nothing: each has its
// own LDS ring and never waits for another.
// ---------------------------------------------------------------------------
template <int HD, int NS, int W>
__global__ __launch_bounds__(64 * W) void decode_bf16_kernel(DecP p) {
    using L = TL<HD>;
    constexpr int RB = L::RB, KT = 32 * RB;  // bytes of a 32-position K (or V) tile
    constexpr int NDQ = KT / 1024;           // 1 KB DMA instructions per tile
    __shared__ __attribute__((aligned(1024))) char rings[W][NS * 2 * KT];
    const int wv = W > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6) : 0;
    char *ring = rings[wv];

    int x = blockIdx.x;
    const int hg = x % p.ngrp;
    x /= p.ngrp;
    const int nkg = (p.NKV + W - 1) / W;
    const int kh = (x % nkg) * W + wv;
    x /= nkg;
    if (kh >= p.NKV) return;
    const int b = x % p.B, split = x / p.B;
    int len, kv0, kv1;
    if (!decode_range(p, b, split, len, kv0, kv1)) return;
    const int ntile = (kv1 - kv0 + 31) / 32;

    const int lane = threadIdx.x & 63, g = lane >> 5, l32 = lane & 31;
    const int grp = p.NH / p.NKV, hl = hg * 32 + l32, h = kh * grp + hl;
    const bool hv = hl < grp;
    const long long stride = p.st;

    // query fragments: chunks 2c+g of head h (zero for lanes past the group)
    u32x4 qf[L::NC];
    {
        const Buf bq(reinterpret_cast<const bf16 *>(p.q) + (long long)b * p.NH * p.hd);
#pragma unroll
        for (int c = 0; c < L::NC; c++) {
            const int ch = 2 * c + g;
            qf[c] = bq.ld16((h * p.hd + ch * 8) * 2, hv && ch * 8 < p.hd);
        }
    }

    const long long cbase = (long long)b * p.sb + (long long)kh * p.sh;
    const bf16 *kc = reinterpret_cast<const bf16 *>(p.kc) + cbase;
    const bf16 *vc = reinterpret_cast<const bf16 *>(p.vc) + cbase;
    // K tiles are read as rows, V tiles transposed: each has its own swizzle.
    // A lane's byte offsets within a tile are the same for every tile (head
    // dims past hd: out of range); positions at or past kv1 are zero-filled by
    // the record count of the tile's buffer, (kv1 - r0) rows of the row stride.
    int okof[NDQ], ovof[NDQ];
#pragma unroll
    for (int i = 0; i < NDQ; i++) {
        const int off = i * 1024 + lane * 16;
        const int r = off / RB, pc = (off % RB) >> 4;
        const int ck = pc ^ swz_rows<HD>(r), cv = pc ^ swz_cols<HD>(r);
        okof[i] = ck * 8 < p.hd ? (int)((r * stride + ck * 8) * 2) : (int)0x80000000;
        ovof[i] = cv * 8 < p.hd ? (int)((r * stride + cv * 8) * 2) : (int)0x80000000;
    }
    auto issue = [&](char *st, int t) {
        decode_tile_dma<NDQ, KT>(st, kc, vc, stride, kv0 + t * 32, kv1, okof, ovof);
    };

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
    float m = -1e30f, lsum = 0.f;

    auto compute = [&](const char *st, int t) {
        const char *Ks = st, *Vs = st + KT;
        f32x16 S;
#pragma unroll
        for (int r = 0; r < 16; r++) S[r] = 0.f;
#pragma unroll
        for (int c = 0; c < L::NC; c++) S = mfma32(lds_row16(Ks + kofs[c]), __builtin_bit_cast(bf16x8, qf[c]), S);
        const int kb0 = kv0 + t * 32;
        if (kb0 + 32 > kv1) {  // the chunk's ragged last tile
            asm volatile("");
#pragma unroll
            for (int r = 0; r < 16; r++)
                if (kb0 + acc_row(r, lane) >= kv1) S[r] = -INFINITY;
        }
        float sv[16];
#pragma unroll
        for (int r = 0; r < 16; r++) sv[r] = S[r];
        const float mt = max_xor32(tree_max<16>(sv)) * p.sl2;
        const float mn = fmaxf(m, mt);
        if (!__all(mn == m)) {
            const float alpha = fast_exp2(m - mn);
            lsum *= alpha;
#pragma unroll
            for (int d = 0; d < L::ND; d++)
#pragma unroll
                for (int r = 0; r < 16; r++) O[d][r] *= alpha;
        }
        m = mn;
#pragma unroll
        for (int r = 0; r < 16; r++) {
            const float e = fast_exp2(fmaf(S[r], p.sl2, -mn));
            S[r] = e;
            lsum += e;
        }
#pragma unroll
        for (int hh = 0; hh < 2; hh++) {
            u32x4 xw;
#pragma unroll
            for (int e = 0; e < 4; e++) xw[e] = pack2_bf16(S[8 * hh + 2 * e], S[8 * hh + 2 * e + 1]);
            const bf16x8 xb = __builtin_bit_cast(bf16x8, xw);
#pragma unroll
            for (int db = 0; db < L::ND; db++)
                O[db] = mfma32(lds_tr8<RB>(Vs + vofs[db] + 16 * hh * RB), xb, O[db]);
        }
    };

    __builtin_amdgcn_s_waitcnt(0);  // query fragments
#pragma unroll
    for (int s = 0; s < NS - 1; s++) issue(ring + s * 2 * KT, s);
    for (int t = 0; t < ntile; t++) {
        // tile t has landed once at most NS-2 younger tiles are in flight; the
        // LDS reads of the stage about to be refilled (tile t-1) are complete
        __builtin_amdgcn_s_waitcnt(wait_vm_lgkm0((NS - 2) * 2 * NDQ));
        issue(ring + ((t + NS - 1) % NS) * 2 * KT, t + NS - 1);
        compute(ring + (t % NS) * 2 * KT, t);
    }
    __builtin_amdgcn_s_waitcnt(0);

    const float ltot = sum_xor32(lsum);
    if (!hv) return;
    // lane column l32 = head h; accumulator rows = head dims 32 db + 8 (r/4) + 4 g + r%4
    if (kv0 == 0 && kv1 == len) {
        bf16 *orow = reinterpret_cast<bf16 *>(p.o) + ((long long)b * p.NH + h) * p.hd;
        const float s = 1.f / ltot;
#pragma unroll
        for (int db = 0; db < L::ND; db++)
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++) {
                const int d = db * 32 + 8 * r4 + 4 * g;
                if (d < p.hd)
                    *reinterpret_cast<u32x2 *>(orow + d) =
                        u32x2{pack2_bf16(O[db][4 * r4] * s, O[db][4 * r4 + 1] * s),
                              pack2_bf16(O[db][4 * r4 + 2] * s, O[db][4 * r4 + 3] * s)};
            }
        if (g == 0) p.lse[(long long)b * p.NH + h] = (m + log2f(ltot)) * LN2;
    } else {
        const long long row = ((long long)split * p.B + b) * p.NH + h;
        float *prow = p.po + row * p.hd;
#pragma unroll
        for (int db = 0; db < L::ND; db++)
#pragma unroll
            for (int r4 = 0; r4 < 4; r4++) {
                const int d = db * 32 + 8 * r4 + 4 * g;
                if (d < p.hd)
                    *reinterpret_cast<f32x4 *>(prow + d) =
                        f32x4{O[db][4 * r4], O[db][4 * r4 + 1], O[db][4 * r4 + 2], O[db][4 * r4 + 3]};
            }
        if (g == 0) p.pml[row] = float2{m, ltot};
    }
}

// ---------------------------------------------------------------------------
// fp32: one wave = (chunk, b, kv head, up to HG query heads)
// ---------------------------------------------------------------------------
template <int HD, int HG>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecP p) {
    constexpr int LPK = HD / 4;    // lanes per cached position (4 head dims each)
    constexpr int KPS = 64 / LPK;  // positions per wave step
    constexpr int U = 4;           // steps whose loads are in flight together

    int x = blockIdx.x;
    const int hg = x % p.ngrp;
    x /= p.ngrp;
    const int kh = x % p.NKV;
    x /= p.NKV;
    const int b = x % p.B, split = x / p.B;
    int len, kv0, kv1;
    if (!decode_range(p, b, split, len, kv0, kv1)) return;

    const int lane = threadIdx.x, slot = lane / LPK, dl = (lane % LPK) * 4;
    const int grp = p.NH / p.NKV;
    const bool dv = dl < p.hd;
    const long long stride = p.st;

    // the group's queries, pre-scaled so that scores come out in log2 units
    float qv[HG][4];
    {
        const Buf bq(reinterpret_cast<const float *>(p.q) + (long long)b * p.NH * p.hd);
#pragma unroll
        for (int i = 0; i < HG; i++) {
            const int hl = hg * HG + i;
            const u32x4 v = bq.ld16(((kh * grp + hl) * p.hd + dl) * 4, hl < grp && dv);
#pragma unroll
            for (int k = 0; k < 4; k++) qv[i][k] = __uint_as_float(v[k]) * p.sl2;
        }
    }
    const long long cbase = (long long)b * p.sb + (long long)kh * p.sh;
    const Buf bk(reinterpret_cast<const float *>(p.kc) + cbase);
    const Buf bv(reinterpret_cast<const float *>(p.vc) + cbase);

    float m[HG], l[HG], o[HG][4];
#pragma unroll
    for (int i = 0; i < HG; i++) {
        m[i] = -1e30f;
        l[i] = 0.f;
#pragma unroll
        for (int k = 0; k < 4; k++) o[i][k] = 0.f;
    }

    for (int j0 = kv0; j0 < kv1; j0 += U * KPS) {
        u32x4 kx[U], vx[U];
#pragma unroll
        for (int u = 0; u < U; u++) {
            const int j = j0 + u * KPS + slot;
            const bool ok = j < kv1 && dv;
            const int off = (int)(((long long)j * stride + dl) * 4);
            kx[u] = bk.ld16(off, ok);
            vx[u] = bv.ld16(off, ok);
        }
#pragma unroll
        for (int u = 0; u < U; u++) {
            const bool live = j0 + u * KPS + slot < kv1;
#pragma unroll
            for (int i = 0; i < HG; i++) {
                float s = 0.f;
#pragma unroll
                for (int k = 0; k < 4; k++) s = fmaf(qv[i][k], __uint_as_float(kx[u][k]), s);
#pragma unroll
                for (int off = 1; off < LPK; off <<= 1) s += __shfl_xor(s, off, 64);
                s = live ? s : -INFINITY;
                const float mn = fmaxf(m[i], s);
                const float a = fast_exp2(m[i] - mn), e = fast_exp2(s - mn);
                l[i] = fmaf(l[i], a, e);
#pragma unroll
                for (int k = 0; k < 4; k++) o[i][k] = fmaf(o[i][k], a, e * __uint_as_float(vx[u][k]));
                m[i] = mn;
            }
        }
    }
    // merge the position slots (lanes lane % LPK equal, slot different)
#pragma unroll
    for (int off = LPK; off < 64; off <<= 1)
#pragma unroll
        for (int i = 0; i < HG; i++) {
            const float m2 = __shfl_xor(m[i], off, 64), l2 = __shfl_xor(l[i], off, 64);
            const float mn = fmaxf(m[i], m2), a = fast_exp2(m[i] - mn), c = fast_exp2(m2 - mn);
            l[i] = l[i] * a + l2 * c;
#pragma unroll
            for (int k = 0; k < 4; k++) o[i][k] = o[i][k] * a + __shfl_xor(o[i][k], off, 64) * c;
            m[i] = mn;
        }
    if (slot != 0 || !dv) return;
    const bool whole = kv0 == 0 && kv1 == len;
#pragma unroll
    for (int i = 0; i < HG; i++) {
        const int hl = hg * HG + i;
        if (hl >= grp) break;
        const int h = kh * grp + hl;
        if (whole) {
            const float s = 1.f / l[i];
            *reinterpret_cast<f32x4 *>(reinterpret_cast<float *>(p.o) + ((long long)b * p.NH + h) * p.hd + dl) =
                f32x4{o[i][0] * s, o[i][1] * s, o[i][2] * s, o[i][3] * s};
            if (dl == 0) p.lse[(long long)b * p.NH + h] = (m[i] + log2f(l[i])) * LN2;
        } else {
            const long long row = ((long long)split * p.B + b) * p.NH + h;
            *reinterpret_cast<f32x4 *>(p.po + row * p.hd + dl) = f32x4{o[i][0], o[i][1], o[i][2], o[i][3]};
            if (dl == 0) p.pml[row] = float2{m[i], l[i]};
        }
    }
}

// ---------------------------------------------------------------------------
// merge the chunks of each (sequence, head); one wave per (b, h)
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void decode_merge_kernel(DecP p) {
    const int w = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
    if (w >= p.B * p.NH) return;
    const int b = w / p.NH;
    const int len = p.lens[b];
    const bool bad = len < 0 || len > p.Tmax;
    const int nc = bad ? 0 : (len + p.chunk - 1) / p.chunk;
    if (nc == 1) return;  // finished by the sequence's only chunk
    T *orow = reinterpret_cast<T *>(p.o) + (long long)w * p.hd;
    if (nc == 0) {  // empty cache: zero output and lse = -inf; invalid length: NaN
        const float v = bad ? __builtin_nanf("") : 0.f;
        for (int d = lane; d < p.hd; d += 64) orow[d] = from_f32<T>(v);
        if (lane == 0) p.lse[w] = bad ? __builtin_nanf("") : -INFINITY;
        return;
    }
    const long long cs = (long long)p.B * p.NH;  // chunk stride in rows
    float M = -INFINITY;
    for (int c = 0; c < nc; c++) M = fmaxf(M, p.pml[c * cs + w].x);
    float Ls = 0.f, acc0 = 0.f, acc1 = 0.f;
    const bool d0 = lane < p.hd, d1 = lane + 64 < p.hd;
    for (int c = 0; c < nc; c++) {
        const float2 ml = p.pml[c * cs + w];
        const float wt = fast_exp2(ml.x - M);
        Ls = fmaf(wt, ml.y, Ls);
        const float *prow = p.po + (c * cs + w) * p.hd;
        if (d0) acc0 = fmaf(wt, prow[lane], acc0);
        if (d1) acc1 = fmaf(wt, prow[lane + 64], acc1);
    }
    const float s = 1.f / Ls;
    if (d0) orow[lane] = from_f32<T>(acc0 * s);
    if (d1) orow[lane + 64] = from_f32<T>(acc1 * s);
    if (lane == 0) p.lse[w] = (M + log2f(Ls)) * LN2;
}

int pow2_at_least(int v, int lo) {
    int p = lo;
    while (p < v) p <<= 1;
    return p;
}

// waves (kv heads) per workgroup and ring depth of the bf16 kernel.  With the
// Llama-GQA heads (hd 64, 8 kv heads) eight waves per workgroup, i.e. whole
// 1 KB cache rows, with two stages each (the LDS holds no more) measured 3-4 %
// faster than one-wave workgroups with four stages; 4 or 2 heads per
// workgroup gained nothing.  hd 128 keeps one wave and three stages.
template <int HD> struct DecCfg {
    static constexpr int W = HD >= 128 ? 1 : 8;
    static constexpr int NS = HD >= 128 ? 3 : HD >= 64 ? 2 : 4;
};
template <int HD, int W, int NS> hipError_t bf16_launch_t(const DecP &p, long long nwave, hipStream_t s) {
    // nwave counts (split, b, kv head, head group) waves; a workgroup takes W kv heads
    const long long nblk = nwave / p.NKV * ((p.NKV + W - 1) / W);
    DTB_LAUNCH((decode_bf16_kernel<HD, NS, W>), dim3((unsigned)nblk), dim3(64 * W), 0, s, p);
    return last_error();
}
template <int HD> hipError_t bf16_launch(const DecP &p, long long nwave, hipStream_t s) {
    // rows of one kv head contiguous (head-major caches): nothing to gain from
    // grouping a position's heads, so one wave per workgroup (more resident
    // waves); on the 256-sequence workload at hd 64 two stages measured best
    // (5.0-5.1 TB/s with the merge, against 4.5-5.1 for 3, 4 or 6 stages or
    // workgroups of 2 or 4 waves, and 4.6-4.8 for the position-major caches)
    if (HD == 64 && p.st == p.hd) return bf16_launch_t<HD, 1, 2>(p, nwave, s);
    if (HD < 64 && p.st == p.hd) return bf16_launch_t<HD, 1, 4>(p, nwave, s);
    return bf16_launch_t<HD, DecCfg<HD>::W, DecCfg<HD>::NS>(p, nwave, s);
}
template <int HD> hipError_t f32_launch(const DecP &p, int HG, int nblk, hipStream_t s) {
    switch (HG) {
    case 1: DTB_LAUNCH((decode_f32_kernel<HD, 1>), dim3(nblk), dim3(64), 0, s, p); break;
    case 2: DTB_LAUNCH((decode_f32_kernel<HD, 2>), dim3(nblk), dim3(64), 0, s, p); break;
    case 4: DTB_LAUNCH((decode_f32_kernel<HD, 4>), dim3(nblk), dim3(64), 0, s, p); break;
    default: DTB_LAUNCH((decode_f32_kernel<HD, 8>), dim3(nblk), dim3(64), 0, s, p); break;
    }
    return last_error();
}

}  // namespace

// query heads per workgroup for the fp32 kernel
static int f32_heads_per_wave(int grp) { return grp >= 8 ? 8 : pow2_at_least(grp, 1); }

DecodeGeom decode_geometry(int B, int NH, int NKV, int hd, int Tmax, int chunk, int dtype) {
    DecodeGeom g{};
    const int grp = NH / NKV;
    g.ngrp = dtype == DTB_BF16 ? (grp + 31) / 32 : (grp + f32_heads_per_wave(grp) - 1) / f32_heads_per_wave(grp);
    if (chunk <= 0) {
        // about 8192 workgroups over the cache capacity (32 per CU), chunks of
        // at least 64 positions so that a chunk's set-up and merge stay small
        const long long pairs = (long long)B * NKV * g.ngrp;
        long long ns = pairs > 0 ? (8192 + pairs - 1) / pairs : 1;
        long long c = (Tmax + ns - 1) / (ns > 0 ? ns : 1);
        c = (c + 31) / 32 * 32;
        chunk = (int)(c < 64 ? 64 : c);
    }
    g.chunk = chunk;
    g.nsplit = Tmax > 0 ? (Tmax + chunk - 1) / chunk : 0;
    g.ws_bytes = (size_t)g.nsplit * B * NH * ((size_t)hd * 4 + 8);
    return g;
}

hipError_t attn_decode_launch(void *out, float *lse, const void *q, const void *kc, const void *vc, const int *lens,
                              int B, int NH, int NKV, int hd, int Tmax, long long sb, long long st, long long sh,
                              const DecodeGeom &g, int dtype, void *workspace, hipStream_t s) {
    DecP p{};
    p.o = out;
    p.lse = lse;
    p.q = q;
    p.kc = kc;
    p.vc = vc;
    p.sb = sb;
    p.st = st;
    p.sh = sh;
    p.lens = lens;
    p.po = reinterpret_cast<float *>(workspace);
    p.pml = reinterpret_cast<float2 *>(reinterpret_cast<char *>(workspace) + (size_t)g.nsplit * B * NH * hd * 4);
    p.B = B;
    p.NH = NH;
    p.NKV = NKV;
    p.hd = hd;
    p.Tmax = Tmax;
    p.chunk = g.chunk;
    p.ngrp = g.ngrp;
    p.sl2 = LOG2E / sqrtf((float)hd);
    const long long nblk = (long long)g.nsplit * B * NKV * g.ngrp;
    hipError_t e = hipSuccess;
    if (nblk > 0) {
        if (g_timing_on) timing_begin(s, K_ATTN_DEC);
        if (dtype == DTB_BF16) {
            switch (pow2_at_least(hd, 16)) {
            case 16: e = bf16_launch<16>(p, nblk, s); break;
            case 32: e = bf16_launch<32>(p, nblk, s); break;
            case 64: e = bf16_launch<64>(p, nblk, s); break;
            default: e = bf16_launch<128>(p, nblk, s); break;
            }
        } else {
            const int HG = f32_heads_per_wave(NH / NKV);
            switch (pow2_at_least(hd, 4)) {
            case 4: e = f32_launch<4>(p, HG, (int)nblk, s); break;
            case 8: e = f32_launch<8>(p, HG, (int)nblk, s); break;
            case 16: e = f32_launch<16>(p, HG, (int)nblk, s); break;
            case 32: e = f32_launch<32>(p, HG, (int)nblk, s); break;
            case 64: e = f32_launch<64>(p, HG, (int)nblk, s); break;
            default: e = f32_launch<128>(p, HG, (int)nblk, s); break;
            }
        }
        if (e != hipSuccess) return e;
        // the bytes read depend on the cache lengths, which live on the device
        if (g_timing_on) timing_end(s, K_ATTN_DEC, 0.0, 0.0);
    }
    const int mblk = (B * NH + 3) / 4;
    if (mblk > 0) {
        if (g_timing_on) timing_begin(s, K_DEC_MERGE);
        if (dtype == DTB_BF16) DTB_LAUNCH(decode_merge_kernel<bf16>, dim3(mblk), dim3(256), 0, s, p);
        else DTB_LAUNCH(decode_merge_kernel<float>, dim3(mblk), dim3(256), 0, s, p);
        e = last_error();
        if (e != hipSuccess) return e;
        if (g_timing_on) timing_end(s, K_DEC_MERGE, 0.0, (double)B * NH * (hd * 2 + 4));
    }
    return hipSuccess;
}

}  // namespace dtb
