// LDS tile helpers shared by the bf16 attention kernels (training flash
// attention and decode attention): tile geometry over a head width padded to
// HD, the 16-byte-chunk swizzles that keep LDS reads free of bank conflicts,
// the row and transposing LDS reads that feed the 32x32x16 MFMA, and the
// wait-count encoding.
#pragma once
#include "common.h"

namespace dtb {

typedef short __attribute__((ext_vector_type(4))) short4_t;
typedef __attribute__((address_space(3))) void *lds_vptr;
typedef __attribute__((address_space(3))) short4_t *lds_s4ptr;

template <int HD> struct TL {
    static constexpr int RB = HD * 2;          // row bytes
    static constexpr int NCH = HD / 8;         // 16-byte chunks per row
    static constexpr int TILE = 64 * RB;       // 64-row tile bytes
    static constexpr int NDMA = TILE / 1024;   // 1 KB DMA instructions per tile
    static constexpr int NC = HD / 16;         // 16-wide MFMA k steps over the head
    static constexpr int ND = HD >= 32 ? HD / 32 : 1;  // 32-row output blocks over the head
};

// chunk swizzle of tiles read as rows (32 consecutive rows, one chunk)
template <int HD> __device__ __forceinline__ int swz_rows(int r) {
    constexpr int M = TL<HD>::NCH - 1;
    r &= 31;
    if constexpr (HD <= 32) return (r >> 3) & M;
    else return (r ^ (r >> 3)) & M;
}
// chunk swizzle of tiles read transposed (groups of 4 rows).  It depends on the
// row modulo 8 only, so row offsets that are multiples of 8 stay immediates;
// this permutation was chosen with the LDS bank-conflict counter (none left in
// the forward; half of the identity's in the backward, whose tiles are also
// read as rows).
template <int HD> __device__ __forceinline__ int swz_cols(int r) {
    r &= 7;
    return (((r & 3) << 1) | ((r >> 2) & 1)) & (TL<HD>::NCH - 1);
}

// tiles read both ways (backward): the transposed reads need the row-mod-8
// form, which the row reads then share
template <int HD> __device__ __forceinline__ int swz_dual(int r) { return swz_cols<HD>(r); }

constexpr int wait_vm_lgkm0(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0070; }

__device__ __forceinline__ bf16x8 lds_row16(const char *p) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p));
}
// two transposing reads 8 rows apart: 8 consecutive k of the lane's column
template <int RB> __device__ __forceinline__ bf16x8 lds_tr8(const char *p) {
    short4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)p);
    short4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)(p + 8 * RB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace dtb
