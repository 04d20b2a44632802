// Row-split recurrent forward: the per-token recurrence in FP32 on the vector
// ALUs, for problems with few (sequence, value head) tasks.
//
// Given the normalised key kn, query qn, decay alpha and beta of a token, the
// rows S[v][:] of the value-first state evolve independently:
//     S[v][:] *= alpha;   e = beta (v_t[v] - S[v][:].kn);   S[v][:] += e kn;
//     o[v] = scale S[v][:].qn
// (recurrence of page "flashinfer.kda_backward.recurrent_kda_backward",
// description; state layout of page "flashinfer.kda_training.recurrent_kda_
// training_forward", parameter initial_state).  So each task's 128 rows are
// split over 8 workgroups of 16 rows; 16 lanes share a row, 8 keys each, and
// the two dot products per token are 16-lane butterfly sums.
//
// Tokens are staged 16 at a time: the workgroup first computes the prologue
// (L2 norms, gate, beta) of the block into LDS, then walks the block.
#include "kda_common.hpp"
#include "kda_kernels.h"

namespace kda {

namespace {
constexpr int RS_ROWS = 16;   // state rows per workgroup
constexpr int RS_TPR = 16;    // lanes per state row
constexpr int RS_KPT = 8;     // keys per lane
constexpr int RS_SPLIT = D / RS_ROWS;
constexpr int RS_TB = 16;     // tokens staged per block
constexpr int RS_THREADS = RS_ROWS * RS_TPR;
static_assert(RS_THREADS == 256, "one 256-lane workgroup");
static_assert(RS_TPR * RS_KPT == D, "a row's lanes cover all keys");
}  // namespace

__global__ __launch_bounds__(RS_THREADS) void fwd_rowsplit_kernel(FwdArgs a) {
    __shared__ float s_kn[RS_TB][D];
    __shared__ float s_qn[RS_TB][D];
    __shared__ float s_al[RS_TB][D];
    __shared__ float s_v[RS_TB][RS_ROWS];
    __shared__ float s_o[RS_TB][RS_ROWS];
    __shared__ float s_b[RS_TB];

    const int tid = threadIdx.x;
    const int ti = blockIdx.x / RS_SPLIT;
    const int r0 = (blockIdx.x % RS_SPLIT) * RS_ROWS;
    const int code = a.plan.task[ti];
    const int n = code / a.Hv;
    const int h = code - n * a.Hv;
    const int hq = h / a.G;
    const int64_t tok0 = a.plan.seq_start[n];
    const int L = a.plan.seq_len[n];

    const bf16* __restrict__ q = (const bf16*)a.q;
    const bf16* __restrict__ k = (const bf16*)a.k;
    const bf16* __restrict__ v = (const bf16*)a.v;
    const bf16* __restrict__ g = (const bf16*)a.g;
    const bf16* __restrict__ beta = (const bf16*)a.beta;
    bf16* __restrict__ o = (bf16*)a.o;

    // recurrence mapping: state row `row`, keys [kofs, kofs+8)
    const int row = tid / RS_TPR;
    const int kofs = (tid % RS_TPR) * RS_KPT;
    // prologue mapping: token pt of the block, keys [pc, pc+8)
    const int pt = tid / 16;
    const int pc = (tid % 16) * 8;

    const int64_t slab = ((int64_t)n * a.Hv + h) * D * D;
    float S[RS_KPT];
    {
        const float4* p = (const float4*)(a.s0 + slab + (int64_t)(r0 + row) * D + kofs);
        float4 x0 = p[0], x1 = p[1];
        S[0] = x0.x; S[1] = x0.y; S[2] = x0.z; S[3] = x0.w;
        S[4] = x1.x; S[5] = x1.y; S[6] = x1.z; S[7] = x1.w;
    }
    const float eA = __expf(a.A_log[h]);
    float dtb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) dtb[i] = a.dt_bias[h * D + pc + i];

    const int64_t qstride = (int64_t)a.Hqk * D;
    const int64_t vstride = (int64_t)a.Hv * D;

    for (int t0 = 0; t0 < L; t0 += RS_TB) {
        const int nv = min(RS_TB, L - t0);
        // ---- prologue of the block ----
        {
            float qf[8], kf[8], gf[8];
            if (pt < nv) {
                const int64_t tok = tok0 + t0 + pt;
                bf16x8 qv = *(const bf16x8*)(q + tok * qstride + hq * D + pc);
                bf16x8 kv = *(const bf16x8*)(k + tok * qstride + hq * D + pc);
                bf16x8 gv = *(const bf16x8*)(g + tok * vstride + h * D + pc);
#pragma unroll
                for (int i = 0; i < 8; ++i) { qf[i] = (float)qv[i]; kf[i] = (float)kv[i]; gf[i] = (float)gv[i]; }
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) { qf[i] = 0.f; kf[i] = 0.f; gf[i] = 0.f; }
            }
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) { sq += qf[i] * qf[i]; sk += kf[i] * kf[i]; }
            sq = group_sum<16>(sq);
            sk = group_sum<16>(sk);
            const float rq = 1.0f / sqrtf(sq + 1e-6f);
            const float rk = 1.0f / sqrtf(sk + 1e-6f);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                s_qn[pt][pc + i] = qf[i] * rq;
                s_kn[pt][pc + i] = kf[i] * rk;
                const float z = eA * (gf[i] + dtb[i]);
                s_al[pt][pc + i] = fast_exp(-5.0f * sigmoidf_(z));
            }
            if (tid < RS_TB) {
                s_b[tid] = (tid < nv) ? sigmoidf_((float)beta[(tok0 + t0 + tid) * a.Hv + h]) : 0.f;
            }
            if (tid < 2 * RS_TB) {
                const int tt = tid >> 1, half = tid & 1;
                if (tt < nv) {
                    bf16x8 vv = *(const bf16x8*)(v + (tok0 + t0 + tt) * vstride + h * D + r0 + half * 8);
#pragma unroll
                    for (int i = 0; i < 8; ++i) s_v[tt][half * 8 + i] = (float)vv[i];
                }
            }
        }
        __syncthreads();
        // ---- sequential walk over the block ----
        for (int tt = 0; tt < nv; ++tt) {
            float pk = 0.f;
#pragma unroll
            for (int i = 0; i < RS_KPT; ++i) {
                S[i] *= s_al[tt][kofs + i];
                pk += S[i] * s_kn[tt][kofs + i];
            }
            pk = group_sum<RS_TPR>(pk);
            const float e = (s_v[tt][row] - pk) * s_b[tt];
            float oq = 0.f;
#pragma unroll
            for (int i = 0; i < RS_KPT; ++i) {
                S[i] += e * s_kn[tt][kofs + i];
                oq += S[i] * s_qn[tt][kofs + i];
            }
            oq = group_sum<RS_TPR>(oq);
            if ((tid % RS_TPR) == 0) s_o[tt][row] = oq * a.scale;
        }
        __syncthreads();
        if (tid < nv * RS_ROWS) {
            const int tt = tid / RS_ROWS, r = tid % RS_ROWS;
            o[(tok0 + t0 + tt) * vstride + h * D + r0 + r] = (bf16)s_o[tt][r];
        }
        const int tend = t0 + nv;
        if (a.tape != nullptr && tend < L && (tend % a.ck_every) == 0) {
            const int64_t j = tend / a.ck_every;
            float* p = a.tape + ((a.plan.tape_off[n] + j - 1) * a.Hv + h) * D * D
                       + (int64_t)(r0 + row) * D + kofs;
            ((float4*)p)[0] = make_float4(S[0], S[1], S[2], S[3]);
            ((float4*)p)[1] = make_float4(S[4], S[5], S[6], S[7]);
        }
    }
    if (a.s_final != nullptr) {
        float* p = a.s_final + slab + (int64_t)(r0 + row) * D + kofs;
        ((float4*)p)[0] = make_float4(S[0], S[1], S[2], S[3]);
        ((float4*)p)[1] = make_float4(S[4], S[5], S[6], S[7]);
    }
}

hipError_t launch_fwd_rowsplit(const FwdArgs& a, hipStream_t s) {
    if (a.num_tasks == 0) return hipSuccess;
    dim3 grid((unsigned)(a.num_tasks * RS_SPLIT));
    hipLaunchKernelGGL(fwd_rowsplit_kernel, grid, dim3(RS_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
