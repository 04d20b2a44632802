// Chunk-level helpers shared by the chunked forward, the state rebuild and the
// adjoint: LDS "frag slot" addressing, the row-owner input loads and the
// column-layout pair stores.  Frag conventions are those of kda_common.hpp.
#pragma once

#include "kda_common.hpp"
#include "kda_kernels.h"

namespace kda {

constexpr int FS = 264;  // frag slot stride in bf16 (256 + 8 padding)

// Operand "frag slots" in LDS (64 lanes x 4 bf16 each, padded):
//   RF(X)[kb]: lane (gq, c) holds X[c][16kb + 4gq + i]   (rows = tokens)
//   CF(X)[kb]: lane (gq, k) holds X[4gq + i][16kb + k]   (tokens along i)
__device__ __forceinline__ int rf_off(int c, int k) {  // (token c, channel k) in an RF slot set
    return (k >> 4) * FS + ((((k >> 2) & 3) << 4) + c) * 4 + (k & 3);
}
__device__ __forceinline__ int cf_off(int c, int k) {  // (token c, channel k) in a CF slot set
    return (k >> 4) * FS + (((c >> 2) << 4) + (k & 15)) * 4 + (c & 3);
}
__device__ __forceinline__ bf16x4 ld4(const bf16* slot, int lane) {
    return *(const bf16x4*)(slot + lane * 4);
}

struct RowIn {   // one token row, 8 channels (row-owner mapping)
    bf16x8 q, k, g;
    bf16 b;
};
// Loads are unconditional (the row is clamped into the sequence by the
// caller): a load in a conditional block tends to be sunk next to its use.
__device__ __forceinline__ void load_rows(RowIn& x, const FwdArgs& a, int64_t tok, int hq, int h,
                                          int c8) {
    const int64_t qo = tok * a.Hqk * D + hq * D + c8;
    x.q = *(const bf16x8*)((const bf16*)a.q + qo);
    x.k = *(const bf16x8*)((const bf16*)a.k + qo);
    x.g = *(const bf16x8*)((const bf16*)a.g + tok * a.Hv * D + h * D + c8);
    x.b = ((const bf16*)a.beta)[tok * a.Hv + h];
}
// Column-layout stores of one token row's 8 channels (c8..c8+7, one 16-channel
// block) as single BF16 values: channel c8 + j sits 4j elements after c8.
__device__ __forceinline__ void store_cf16(bf16* slots, int r, int c8, bf16x4 lo, bf16x4 hi) {
    bf16* dst = &slots[cf_off(r, c8)];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        dst[4 * j] = lo[j];
        dst[4 * (j + 4)] = hi[j];
    }
}

// Broadcast lane q of every quad to the whole quad (DPP quad_perm [q,q,q,q]);
// q must fold to a constant.
__device__ __forceinline__ float quad_bcast(float x, int q) {
    const int xi = __float_as_int(x);
    switch (q) {
        case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(xi, 0x00, 0xF, 0xF, false));
        case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(xi, 0x55, 0xF, 0xF, false));
        case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(xi, 0xAA, 0xF, 0xF, false));
        default: return __int_as_float(__builtin_amdgcn_mov_dpp(xi, 0xFF, 0xF, 0xF, false));
    }
}

__device__ __forceinline__ void set_prio_by_remaining(int left, int total) {
    const int p = (4 * left - 1) / total;  // 3 for the first quarter, 0 for the last
    switch (p) {
        case 3: __builtin_amdgcn_s_setprio(3); break;
        case 2: __builtin_amdgcn_s_setprio(2); break;
        case 1: __builtin_amdgcn_s_setprio(1); break;
        default: __builtin_amdgcn_s_setprio(0); break;
    }
}

}  // namespace kda
