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
    const float *D;     // backward: rowsum(dO o)   [B][NH][T]
    const float *L2;    // backward: lse * log2(e)  [B][NH][T]
    int B, T, C, NH, NKV, hd, QKV;
    float sl2;      // log2(e) / sqrt(hd)
    float scale;    // 1 / sqrt(hd)
};

constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// bf16 kernels (head width padded to HD in {16, 32, 64, 128})
hipError_t attn_fwd_bf16(const AttnP &p, int HD, hipStream_t s);
// dQ and dK/dV; p.D and p.L2 must already hold rowsum(dO o) and lse * log2(e)
hipError_t attn_bwd_bf16(const AttnP &p, int HD, hipStream_t s);

}  // namespace dtb
