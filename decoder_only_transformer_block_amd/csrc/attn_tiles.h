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

// Chunk swizzles.  Bank model (it reproduces the LDS bank-conflict counter
// on every layout measured): 64 banks of 4 bytes, i.e. 16 groups of 16 bytes;
// ds_read_b128 serves 16 lanes per pass, ds_read_b64_tr_b16 32 lanes, and a
// pass is conflict-free when its lanes hit distinct 16-byte groups (two lanes
// share a group in the transposing read, one 8-byte half each).  A row read of
// an MFMA operand takes 16 consecutive rows at one logical chunk per pass; a
// transposing read 4 consecutive rows x 4 chunks.

// tiles read as rows (32 consecutive rows, one chunk)
template <int HD> __device__ __forceinline__ int swz_rows(int r) {
    constexpr int M = TL<HD>::NCH - 1;
    r &= 31;
    if constexpr (HD <= 32) return (r >> 3) & M;
    else return (r ^ (r >> 3)) & M;
}
// tiles read transposed only (groups of 4 rows).  It depends on the row
// modulo 8 only, so row offsets that are multiples of 8 stay immediates.  At
// head width 128 (256-byte rows, every row starting at bank 0) the 4 rows of
// a pass take distinct chunk quarters.
template <int HD> __device__ __forceinline__ int swz_cols(int r) {
    if constexpr (HD >= 128) return (r & 3) << 2;
    r &= 7;
    return (((r & 3) << 1) | ((r >> 2) & 1)) & (TL<HD>::NCH - 1);
}

// tiles read both ways (backward).  At head width 64 the 16 rows of a row-read
// pass need 16 distinct groups, so the swizzle also takes row bit 3 (even and
// odd rows fall in different bank halves; bits 1-3 pick the chunk), and the
// transposing reads then find their second 8 rows at logical chunk ^ 2, i.e.
// byte offset ^ dual_x8 within the row.  At head width 128 a swizzle of row
// bits 0-2 keeps the transposing reads conflict-free (row reads stay 2-way:
// another 2 registers per fragment address did not fit that kernel's budget).
template <int HD> __device__ __forceinline__ int swz_dual(int r) {
    if constexpr (HD == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 1) | (((r >> 3) & 1) << 1);
    r &= 7;
    if constexpr (HD == 128) return ((r & 3) << 2) | ((r >> 2) & 1);
    return (((r & 3) << 1) | ((r >> 2) & 1)) & (TL<HD>::NCH - 1);
}
template <int HD> constexpr int dual_x8() { return HD == 64 ? 32 : 0; }

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
// the same with the second 8 rows addressed from p8 (tiles whose swizzle
// depends on row bit 3)
template <int RB> __device__ __forceinline__ bf16x8 lds_tr8x(const char *p, const char *p8) {
    short4_t a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)p);
    short4_t b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4ptr)(p8 + 8 * RB));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace dtb
