// Internal declarations shared by the attention translation units.
#pragma once
#include "common.h"

namespace dtb {

struct AttnP {
    const void *qkv;
    const void *out;
    const void *dout;
    void *o;        // forward output / dqkv for the backward
    float *lse;     // forward output
    const float *lse_in;
    float *D;           // backward: -rowsum(dO o)   [B][NH][T]
    float *lsn;         // backward: -lse / scale, lse in raw score units  [B][NH][T]
    const float2 *rope_cs;  // backward: NeoX (cos, sin) table [T][hd/2] to rotate dq, dk back, or null
    int B, T, C, NH, NKV, hd, QKV;
    float sl2;      // log2(e) / sqrt(hd)
    float scale;    // 1 / sqrt(hd)
};

// In-register NeoX rotation of the ND accumulator blocks of one position (the
// lane's column): registers hold head dims d = 32 db + 8 (r/4) + 4 g + r%4
// (g = lane/32).  Pair (k, k + hd/2) turns by the angle in cs_t[k]; sgn = -1
// applies the transposed (inverse) rotation, which the backward needs
// ("nx_f32_qwen2_train_gate.nx source": rope_node; "nanoeuler — CUDA kernels":
// rope_kernel with inverse = 1).  hd is the real head width (hd = 32 ND when
// ND > 1).
template <int ND>
__device__ __forceinline__ void rope_rotate_acc(f32x16 *acc, const float2 *cs_t, int hd, float sgn, int lane) {
    const int g = lane >> 5;
    // rotate registers (a of block da, b of block db) as the pair (x, y) of index k
#define DTB_TURN(da, ra, dbk, rb, k)                                     \
    {                                                                   \
        const float2 c_ = cs_t[k];                                      \
        const float sn_ = sgn * c_.y, x_ = acc[da][ra], y_ = acc[dbk][rb]; \
        acc[da][ra] = x_ * c_.x - y_ * sn_;                             \
        acc[dbk][rb] = y_ * c_.x + x_ * sn_;                            \
    }
    if constexpr (ND > 1) {
        constexpr int PB = ND / 2;  // partner block: hd/2 = 32 PB
#pragma unroll
        for (int db = 0; db < PB; db++)
#pragma unroll
            for (int r = 0; r < 16; r++) DTB_TURN(db, r, db + PB, r, 32 * db + 8 * (r >> 2) + 4 * g + (r & 3))
    } else {
        const int half = hd / 2;
        if (half == 16) {
#pragma unroll
            for (int r = 0; r < 8; r++) DTB_TURN(0, r, 0, r + 8, 8 * (r >> 2) + 4 * g + (r & 3))
        } else if (half == 8) {
#pragma unroll
            for (int r = 0; r < 4; r++) DTB_TURN(0, r, 0, r + 4, 4 * g + r)
        } else if (half == 4) {  // partner in lane l ^ 32 (g = 0 holds the lower half)
#pragma unroll
            for (int r = 0; r < 4; r++) {
                const float other = __shfl_xor(acc[0][r], 32, 64);
                const float x = g ? other : acc[0][r], y = g ? acc[0][r] : other;
                const float2 c = cs_t[r];
                const float sn = sgn * c.y;
                acc[0][r] = g ? y * c.x + x * sn : x * c.x - y * sn;
            }
        } else if (half == 2) {
#pragma unroll
            for (int r = 0; r < 2; r++) DTB_TURN(0, r, 0, r + 2, r)
        }
    }
#undef DTB_TURN
}

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// bf16 kernels (head width padded to HD in {16, 32, 64, 128})
hipError_t attn_fwd_bf16(const AttnP &p, int HD, hipStream_t s);
// dQ and dK/dV; the dQ kernel writes p.D = -rowsum(dO o) and p.lsn = -lse / scale
// (from p.out, p.dout and p.lse_in) for the dK/dV kernel that follows it
hipError_t attn_bwd_bf16(const AttnP &p, int HD, hipStream_t s);

}  // namespace dtb
