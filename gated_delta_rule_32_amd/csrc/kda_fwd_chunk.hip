// Chunked forward on the MFMA units.
//
// The recurrence of page "flashinfer.kda_backward.recurrent_kda_backward"
// (description) is evaluated 16 tokens at a time in its WY / UT form.  For a
// chunk with start state S0 (value-first, [v][k]) and per-token log-decays
// lam (the prologue's lower_bound * sigmoid(z)):
//
//   gc = cumsum(lam) over the chunk's tokens,  Gam = exp(gc),  gC = gc[last]
//   Qg = qn*Gam,  Kg = kn*Gam,  Ki = kn/Gam,  Kt = kn*exp(gC - gc)
//   Akk = strictly-lower(Kg Ki^T),  Aqk = lower(Qg Ki^T)
//   Tb  = (I + diag(beta) Akk)^-1 diag(beta)        (forward substitution)
//   W   = Tb Kg,   Ut = Tb V,   U = Ut - W S0^T
//   O   = scale (Qg S0^T + Aqk U)
//   S_C = S0 diag(exp(gC)) + U^T Kt
//
// Within a chunk the log-decay sums stay above 16 * (-5) = -80, so the factors
// exp(+-gc) stay inside the FP32/BF16 exponent range (e^80 < 3.4e38).
//
// Work split.  One workgroup (4 waves) owns one (sequence, value head) task
// for its whole length; wave w owns state columns v in [32w, 32w+32) of S
// (held as transposed 16x16 frags S^T[kb][vb] in FP32 registers).  The state
// path (U, O, S update) is column-local, so each wave runs it without
// exchanging state; only the chunk's shared quantities (Qg, Kg, Ki, Kt, V
// frags, W, Tb, Aqk) pass through LDS.
//
// Precision.  Products that feed the carried state (W = Tb Kg, Ut = Tb V,
// W S0^T, U^T Kt) use BF16 hi/lo operand pairs, three MFMAs per product, which
// keeps them FP32-accurate; Akk/Aqk and the output product use plain BF16.
#include "kda_common.hpp"
#include "kda_kernels.h"

namespace kda {

namespace {

constexpr int FC_THREADS = 256;
constexpr int FRAG = 256;  // bf16 elements in one frag slot (64 lanes x 4)

struct FwdLds {
    bf16 rf_qg[8][FRAG];     // RF(Qg)[kb]: lane (gq,c) holds Qg[c][16kb+4gq+i]
    bf16 rf_kg[8][FRAG];
    bf16 rf_ki[8][FRAG];
    bf16 cf_kg_hi[8][FRAG];  // CF(Kg)[kb]: lane (gq,k) holds Kg[4gq+i][16kb+k]
    bf16 cf_kg_lo[8][FRAG];
    bf16 cf_kt_hi[8][FRAG];
    bf16 cf_kt_lo[8][FRAG];
    bf16 cf_v[8][FRAG];      // CF(V)[vb]
    bf16 rf_w_hi[8][FRAG];   // RF(-W)[kb]
    bf16 rf_w_lo[8][FRAG];
    bf16 tb_hi[FRAG];        // RF16(Tb): lane (gq,c) holds Tb[c][4gq+i]
    bf16 tb_lo[FRAG];
    bf16 aqk_rf[FRAG];       // RF16(Aqk)
    float akk[16][17];
    float aqk[16][17];
    float lam[16][D];        // log-decays, then their in-chunk prefix sums
    float gamc[D];           // exp(gC)
    float beta[16];
    bf16 o[16][D];           // output staging
};

// element (row c, col k) of a 16 x 128 matrix -> RF slot offset
__device__ __forceinline__ int rf_off(int c, int k) {
    return (k >> 4) * FRAG + ((((k >> 2) & 3) << 4) + c) * 4 + (k & 3);
}
// element (row c, col k) of a 16 x 128 matrix -> CF slot offset
__device__ __forceinline__ int cf_off(int c, int k) {
    return (k >> 4) * FRAG + (((c >> 2) << 4) + (k & 15)) * 4 + (c & 3);
}

__device__ __forceinline__ bf16x4 ld4(const bf16* base, int lane) {
    return *(const bf16x4*)(base + lane * 4);
}
__device__ __forceinline__ void st4(bf16* base, int lane, bf16x4 x) {
    *(bf16x4*)(base + lane * 4) = x;
}

struct ChunkIn {
    bf16x8 q, k, g, v;
    float b;
};

__device__ __forceinline__ void load_chunk(ChunkIn& x, const FwdArgs& a, int64_t tok, bool valid,
                                           int hq, int h, int c8, bool lead) {
    if (valid) {
        const int64_t qo = tok * a.Hqk * D + hq * D + c8;
        const int64_t vo = tok * a.Hv * D + h * D + c8;
        x.q = *(const bf16x8*)((const bf16*)a.q + qo);
        x.k = *(const bf16x8*)((const bf16*)a.k + qo);
        x.g = *(const bf16x8*)((const bf16*)a.g + vo);
        x.v = *(const bf16x8*)((const bf16*)a.v + vo);
        x.b = lead ? (float)((const bf16*)a.beta)[tok * a.Hv + h] : 0.f;
    }
}

}  // namespace

__global__ __launch_bounds__(FC_THREADS, 2) void fwd_chunk_kernel(FwdArgs a) {
    __shared__ FwdLds sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int gq = lane >> 4;
    const int cl = lane & 15;

    const int code = a.plan.task[blockIdx.x];
    const int n = code / a.Hv;
    const int h = code - n * a.Hv;
    const int hq = h / a.G;
    const int64_t tok0 = a.plan.seq_start[n];
    const int L = a.plan.seq_len[n];
    const int64_t slab = ((int64_t)n * a.Hv + h) * D * D;

    // ---- state: S^T frags for kb = 0..7, vb = 2*wave + {0,1} ----
    f32x4 S[8][2];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int vcol = 16 * (2 * wave + j) + cl;
            const float4 x = *(const float4*)(a.s0 + slab + (int64_t)vcol * D + 16 * kb + 4 * gq);
            S[kb][j] = f32x4{x.x, x.y, x.z, x.w};
        }

    // prologue mapping: token row r, channels [c8, c8+8)
    const int r = tid >> 4;
    const int c8 = (tid & 15) * 8;
    const float eA = __expf(a.A_log[h]);
    float dtb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) dtb[i] = a.dt_bias[h * D + c8 + i];

    ChunkIn cur{}, nxt{};
    load_chunk(cur, a, tok0 + r, r < L, hq, h, c8, (tid & 15) == 0);

    const int nchunks = (L + CH - 1) / CH;
    for (int ci = 0; ci < nchunks; ++ci) {
        const int t0 = ci * CH;
        const int nv = min(CH, L - t0);
        const bool valid = r < nv;
        // prefetch the next chunk
        if (ci + 1 < nchunks) {
            const int nr = t0 + CH + r;
            load_chunk(nxt, a, tok0 + nr, nr < L, hq, h, c8, (tid & 15) == 0);
        }

        // ---- phase A: prologue ----
        float qf[8], kf[8];
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            qf[i] = valid ? (float)cur.q[i] : 0.f;
            kf[i] = valid ? (float)cur.k[i] : 0.f;
            sq += qf[i] * qf[i];
            sk += kf[i] * kf[i];
        }
        sq = group_sum<16>(sq);
        sk = group_sum<16>(sk);
        const float rq = 1.0f / sqrtf(sq + 1e-6f);
        const float rk = 1.0f / sqrtf(sk + 1e-6f);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            qf[i] *= rq;
            kf[i] *= rk;
            const float z = eA * ((float)cur.g[i] + dtb[i]);
            sm.lam[r][c8 + i] = valid ? -5.0f * sigmoidf_(z) : 0.f;
        }
        if ((tid & 15) == 0) sm.beta[r] = valid ? sigmoidf_(cur.b) : 0.f;
        __syncthreads();
        if (tid < D) {
            float acc = 0.f;
#pragma unroll
            for (int rr = 0; rr < CH; ++rr) {
                acc += sm.lam[rr][tid];
                sm.lam[rr][tid] = acc;
            }
            sm.gamc[tid] = fast_exp(acc);
        }
        __syncthreads();
        {
            bf16x4 q4[2], kg4[2], ki4[2];
            float kgv[8], ktv[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float gc = sm.lam[r][c8 + i];
                const float gC = sm.lam[CH - 1][c8 + i];
                const float gam = fast_exp(gc);
                const float gin = fast_exp(-gc);
                const float gt = fast_exp(gC - gc);
                const float qg = qf[i] * gam;
                kgv[i] = kf[i] * gam;
                ktv[i] = kf[i] * gt;
                q4[i >> 2][i & 3] = (bf16)qg;
                kg4[i >> 2][i & 3] = (bf16)kgv[i];
                ki4[i >> 2][i & 3] = (bf16)(kf[i] * gin);
            }
            // RF slots: two groups of four consecutive channels
#pragma unroll
            for (int hgrp = 0; hgrp < 2; ++hgrp) {
                const int o = rf_off(r, c8 + 4 * hgrp);
                *(bf16x4*)(&sm.rf_qg[0][0] + o) = q4[hgrp];
                *(bf16x4*)(&sm.rf_kg[0][0] + o) = kg4[hgrp];
                *(bf16x4*)(&sm.rf_ki[0][0] + o) = ki4[hgrp];
            }
            // CF slots: one element per channel
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int o = cf_off(r, c8 + i);
                const bf16 kh = (bf16)kgv[i];
                (&sm.cf_kg_hi[0][0])[o] = kh;
                (&sm.cf_kg_lo[0][0])[o] = (bf16)(kgv[i] - (float)kh);
                const bf16 th = (bf16)ktv[i];
                (&sm.cf_kt_hi[0][0])[o] = th;
                (&sm.cf_kt_lo[0][0])[o] = (bf16)(ktv[i] - (float)th);
                (&sm.cf_v[0][0])[o] = valid ? cur.v[i] : (bf16)0.f;
            }
        }
        // store the previous chunk's output (staged in LDS before the last sync)
        if (ci > 0) {
            const int pr = tid >> 4;  // row of the previous chunk (always full)
            const int64_t tok = tok0 + t0 - CH + pr;
            *(bf16x8*)((bf16*)a.o + tok * a.Hv * D + h * D + c8) = *(const bf16x8*)(&sm.o[pr][c8]);
        }
        __syncthreads();

        // ---- phase B: Akk (wave 0) and Aqk (wave 1) ----
        if (wave < 2) {
            const bf16* lhs = wave == 0 ? &sm.rf_kg[0][0] : &sm.rf_qg[0][0];
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                bf16x8 x = cat8(ld4(lhs + (2 * j) * FRAG, lane), ld4(lhs + (2 * j + 1) * FRAG, lane));
                bf16x8 y = cat8(ld4(&sm.rf_ki[2 * j][0], lane), ld4(&sm.rf_ki[2 * j + 1][0], lane));
                acc = mma32(x, y, acc);
            }
            // lane (gq, cl) holds A[4gq+i][cl]; keep the causal part
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 4 * gq + i;
                if (wave == 0) sm.akk[row][cl] = (cl < row) ? acc[i] : 0.f;
                else sm.aqk[row][cl] = (cl <= row) ? acc[i] : 0.f;
            }
        }
        __syncthreads();

        // ---- phase C: Tb = (I + diag(beta) Akk)^-1 diag(beta) (wave 0), RF16(Aqk) (wave 1) ----
        if (wave == 0 && lane < 16) {
            const int col = lane;
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float s = 0.f;
#pragma unroll
                for (int m = 0; m < i; ++m) s += sm.akk[i][m] * t[m];
                t[i] = (i == col ? 1.0f : 0.0f) - sm.beta[i] * s;
            }
            const float bc = sm.beta[col];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float x = t[i] * bc;  // Tb[i][col]
                const bf16 xh = (bf16)x;
                const int o = (((col >> 2) << 4) + i) * 4 + (col & 3);
                sm.tb_hi[o] = xh;
                sm.tb_lo[o] = (bf16)(x - (float)xh);
            }
        } else if (wave == 1) {
            bf16x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (bf16)sm.aqk[cl][4 * gq + i];
            st4(sm.aqk_rf, lane, x);
        }
        __syncthreads();

        // ---- phase D1: -W frags for kb = 2w, 2w+1;  D2: Ut for own vb ----
        const bf16x4 tbh = ld4(sm.tb_hi, lane);
        const bf16x4 tbl = ld4(sm.tb_lo, lane);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int kb = 2 * wave + j;
            const bf16x4 kh = ld4(&sm.cf_kg_hi[kb][0], lane);
            const bf16x4 kl = ld4(&sm.cf_kg_lo[kb][0], lane);
            f32x4 w = mma16(kh, tbh, zero4());
            w = mma16(kh, tbl, w);
            w = mma16(kl, tbh, w);
            bf16x4 wh, wl;
            split4(-w, wh, wl);
            st4(&sm.rf_w_hi[kb][0], lane, wh);
            st4(&sm.rf_w_lo[kb][0], lane, wl);
        }
        f32x4 U[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const bf16x4 vv = ld4(&sm.cf_v[2 * wave + j][0], lane);
            U[j] = mma16(tbh, vv, zero4());
            U[j] = mma16(tbl, vv, U[j]);
        }
        __syncthreads();

        // ---- phase D3: U = Ut - W S0^T,  O = Qg S0^T + Aqk U,  S update ----
        f32x4 O[2] = {zero4(), zero4()};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 wh = cat8(ld4(&sm.rf_w_hi[2 * j][0], lane), ld4(&sm.rf_w_hi[2 * j + 1][0], lane));
            const bf16x8 wl = cat8(ld4(&sm.rf_w_lo[2 * j][0], lane), ld4(&sm.rf_w_lo[2 * j + 1][0], lane));
            const bf16x8 qg = cat8(ld4(&sm.rf_qg[2 * j][0], lane), ld4(&sm.rf_qg[2 * j + 1][0], lane));
#pragma unroll
            for (int vb = 0; vb < 2; ++vb) {
                bf16x4 h0, l0, h1, l1;
                split4(S[2 * j][vb], h0, l0);
                split4(S[2 * j + 1][vb], h1, l1);
                const bf16x8 sh = cat8(h0, h1);
                const bf16x8 sl = cat8(l0, l1);
                U[vb] = mma32(wh, sh, U[vb]);
                U[vb] = mma32(wh, sl, U[vb]);
                U[vb] = mma32(wl, sh, U[vb]);
                O[vb] = mma32(qg, sh, O[vb]);
            }
        }
        const bf16x4 aq = ld4(sm.aqk_rf, lane);
        bf16x4 uh[2], ul[2];
#pragma unroll
        for (int vb = 0; vb < 2; ++vb) {
            split4(U[vb], uh[vb], ul[vb]);
            O[vb] = mma16(aq, uh[vb], O[vb]);
            // lane (gq, cl) holds O[4gq+i][v]
#pragma unroll
            for (int i = 0; i < 4; ++i)
                sm.o[4 * gq + i][16 * (2 * wave + vb) + cl] = (bf16)(O[vb][i] * a.scale);
        }
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const bf16x4 th = ld4(&sm.cf_kt_hi[kb][0], lane);
            const bf16x4 tl = ld4(&sm.cf_kt_lo[kb][0], lane);
            const float4 gd = *(const float4*)(&sm.gamc[16 * kb + 4 * gq]);
#pragma unroll
            for (int vb = 0; vb < 2; ++vb) {
                f32x4 s = S[kb][vb];
                s[0] *= gd.x; s[1] *= gd.y; s[2] *= gd.z; s[3] *= gd.w;
                s = mma16(th, uh[vb], s);
                s = mma16(th, ul[vb], s);
                s = mma16(tl, uh[vb], s);
                S[kb][vb] = s;
            }
        }
        // tape: state after t0 + 16 tokens
        const int tend = t0 + nv;
        if (a.tape != nullptr && tend < L && (tend % a.ck_every) == 0) {
            const int64_t jck = tend / a.ck_every;
            float* base = a.tape + ((a.plan.tape_off[n] + jck - 1) * a.Hv + h) * (int64_t)D * D;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int vcol = 16 * (2 * wave + j) + cl;
                    *(float4*)(base + (int64_t)vcol * D + 16 * kb + 4 * gq) =
                        make_float4(S[kb][j][0], S[kb][j][1], S[kb][j][2], S[kb][j][3]);
                }
        }
        cur = nxt;
        __syncthreads();
    }
    // last chunk's output
    {
        const int t0 = (nchunks - 1) * CH;
        const int nv = L - t0;
        const int pr = tid >> 4;
        if (pr < nv) {
            const int64_t tok = tok0 + t0 + pr;
            *(bf16x8*)((bf16*)a.o + tok * a.Hv * D + h * D + c8) = *(const bf16x8*)(&sm.o[pr][c8]);
        }
    }
    if (a.s_final != nullptr) {
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int vcol = 16 * (2 * wave + j) + cl;
                *(float4*)(a.s_final + slab + (int64_t)vcol * D + 16 * kb + 4 * gq) =
                    make_float4(S[kb][j][0], S[kb][j][1], S[kb][j][2], S[kb][j][3]);
            }
    }
}

hipError_t launch_fwd_chunk(const FwdArgs& a, hipStream_t s) {
    if (a.num_tasks == 0) return hipSuccess;
    hipLaunchKernelGGL(fwd_chunk_kernel, dim3((unsigned)a.num_tasks), dim3(FC_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
