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

struct ColIn {   // V for the wave's 16-column blocks: CF(V)[vb0], CF(V)[vb0+1]
    bf16x4 v[2];
};

// Per-task base pointers (uniform, so they live in scalar registers) and
// element strides; a token row inside the sequence is then a 32-bit offset
// (the host rejects sequences whose span exceeds 2^31 elements).
struct SeqPtrs {
    const bf16* q;   // q[tok0][hq][0]; k likewise
    const bf16* k;
    const bf16* g;   // g[tok0][h][0]; v and o likewise
    const bf16* v;
    bf16* o;
    const bf16* beta;  // beta[tok0][h]
    unsigned sq, sv, sb;  // per-token strides: Hqk*128, Hv*128, Hv
};

__device__ __forceinline__ void load_rows_s(RowIn& x, const SeqPtrs& p, unsigned t, unsigned c8) {
    const unsigned oq = __umul24(t, p.sq) + c8;
    x.q = *(const bf16x8*)at(p.q, oq);
    x.k = *(const bf16x8*)at(p.k, oq);
    x.g = *(const bf16x8*)at(p.g, __umul24(t, p.sv) + c8);
    x.b = *at(p.beta, __umul24(t, p.sb));
}
// CF(V) straight from memory: lane (gq, n) takes tokens t4 .. t4+3 (t4 =
// t0 + 4gq, each clamped to the sequence's last token, whose rows the
// chunk's zero beta then masks) of channels ch, ch + 16, ...: 2-byte loads
// into the halves of four registers per block, no transpose.
template <int NVB>
__device__ __forceinline__ void load_cols_cf(ColIn& x, const SeqPtrs& p, int t4, int last, unsigned ch) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const unsigned o = __umul24((unsigned)min(t4 + i, last), p.sv) + ch;
#pragma unroll
        for (int j = 0; j < NVB; ++j) x.v[j][i] = *at(p.v, o + 16 * j);
    }
}

template <int NVB>
__device__ __forceinline__ void store_state(float* dst, const f32x4 (&S)[8][NVB], int vb0, int gq,
                                            int cl) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int j = 0; j < NVB; ++j) {
            const int vcol = 16 * (vb0 + j) + cl;
            *(float4*)(dst + (int64_t)vcol * D + 16 * kb + 4 * gq) =
                make_float4(S[kb][j][0], S[kb][j][1], S[kb][j][2], S[kb][j][3]);
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

// XCD-aware order of the work items: the hardware hands blocks to the 8 XCDs
// round robin (block b to XCD b mod 8), so the G value heads of a q/k head,
// adjacent in the task list, go to blocks 8 apart (one XCD) and read that
// head's q and k rows through one L2.  Each window of 8G blocks holds the same
// items as before (the list's longest-first order at that granularity); a
// trailing partial window keeps its order.  A bijection on [0, n).
__device__ __forceinline__ int xcd_order(int b, int n, int G) {
    const int win = 8 * G;
    if (G > 1 && b < n / win * win) {
        const int x = b & 7, y = b >> 3;
        return G * (8 * (y / G) + x) + y % G;
    }
    return b;
}

}  // namespace kda
