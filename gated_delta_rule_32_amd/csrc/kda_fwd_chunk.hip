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
// for its whole length; wave w owns state columns v in [32w, 32w+32), held as
// transposed 16x16 frags S^T[kb][vb] in FP32 registers.  The state path is
// column-local, so no state crosses waves; the chunk's shared operands pass
// through LDS in "frag slots" (64 lanes x 4 bf16, padded against bank
// conflicts):
//   RF(X)[kb]: lane (gq, c) holds X[c][16kb + 4gq + i]   (rows = tokens)
//   CF(X)[kb]: lane (gq, k) holds X[4gq + i][16kb + k]   (tokens along i)
// Products that contract over tokens take CF operands, those that contract
// over channels take RF operands.  The output is formed transposed,
// O^T = S0 Qg^T + U^T Aqk^T, whose accumulator layout gives each lane four
// consecutive channels of one token, stored straight to global memory.
//
// Precision.  Only the products that add new information to the carried state
// need FP32-accurate operands: Ut = Tb V (Tb as a BF16 hi/lo pair, V exact)
// and U^T Kt (both operands as hi/lo pairs, three products).  W, W S0^T, the
// A matrices and the output product use plain BF16 operands: the delta rule
// re-measures the state against each key, so rounding in the prediction
// W S0^T does not accumulate (checked against the FP64 definition over
// 1024-4096-token sequences: final-state error ~2e-5 to 5e-5).
//
// Latency.  The next chunk's inputs are loaded into the same registers right
// after their last use (end of phase C), so they arrive during the rest of the
// chunk without a second register buffer or a register copy; vector-memory
// waits then fall only on the first use, at the start of the next chunk.
#include "kda_common.hpp"
#include "kda_kernels.h"

namespace kda {

namespace {

constexpr int FC_THREADS = 256;
constexpr int FS = 264;  // frag slot stride in bf16 (256 + 8 padding)

struct FwdLds {
    float lam[CH][D];        // log2-domain decays, then their in-chunk prefix sums
    float gamc[D];           // exp(gC) per channel
    float dtz[D];            // dt_bias * exp(A_log) * log2(e)
    float beta[CH];
    float akkT[CH][CH];      // akkT[m][i] = Akk[i][m] (strictly lower part)
    bf16 rf_qg[8 * FS];
    bf16 rf_kg[8 * FS];
    bf16 rf_ki[8 * FS];
    bf16 cf_kg[8 * FS];
    bf16 cf_kth[8 * FS];
    bf16 cf_ktl[8 * FS];
    bf16 rf_w[8 * FS];       // RF(-W)
    bf16 tbh[FS];            // RF16(Tb): lane (gq, c) holds Tb[c][4gq+i]
    bf16 tbl[FS];
    bf16 aqk[FS];            // RF16(Aqk)
};

__device__ __forceinline__ int rf_off(int c, int k) {  // (token c, channel k) in an RF slot set
    return (k >> 4) * FS + ((((k >> 2) & 3) << 4) + c) * 4 + (k & 3);
}
__device__ __forceinline__ int cf_off(int c, int k) {  // (token c, channel k) in a CF slot set
    return (k >> 4) * FS + (((c >> 2) << 4) + (k & 15)) * 4 + (c & 3);
}
__device__ __forceinline__ bf16x4 ld4(const bf16* slot, int lane) {
    return *(const bf16x4*)(slot + lane * 4);
}
__device__ __forceinline__ void st4(bf16* slot, int lane, bf16x4 x) {
    *(bf16x4*)(slot + lane * 4) = x;
}

struct RowIn {   // one token row, 8 channels (row-owner mapping)
    bf16x8 q, k, g;
    bf16 b;
};
struct ColIn {   // V for the wave's 32 columns: RF(V)[2w], RF(V)[2w+1]
    bf16x4 v0, v1;
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
__device__ __forceinline__ void load_cols(ColIn& x, const FwdArgs& a, int64_t tok, int h,
                                          int ch0) {
    const bf16* p = (const bf16*)a.v + tok * a.Hv * D + h * D + ch0;
    x.v0 = *(const bf16x4*)p;
    x.v1 = *(const bf16x4*)(p + 16);
}

__device__ __forceinline__ void store_state(float* dst, const f32x4 (&S)[8][2], int wave, int gq,
                                            int cl) {
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int vcol = 16 * (2 * wave + j) + cl;
            *(float4*)(dst + (int64_t)vcol * D + 16 * kb + 4 * gq) =
                make_float4(S[kb][j][0], S[kb][j][1], S[kb][j][2], S[kb][j][3]);
        }
}

}  // namespace

__global__ __launch_bounds__(FC_THREADS, 3) void fwd_chunk_kernel(FwdArgs a) {
    __shared__ FwdLds sm;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;

    const int code = a.plan.task[blockIdx.x];
    const int n = code / a.Hv;
    const int h = code - n * a.Hv;
    const int hq = h / a.G;
    const int64_t tok0 = a.plan.seq_start[n];
    const int L = a.plan.seq_len[n];
    const int64_t slab = ((int64_t)n * a.Hv + h) * D * D;
    const int64_t tape_base = a.tape != nullptr ? a.plan.tape_off[n] : 0;

    // state: S^T frags for kb = 0..7 and vb = 2*wave + {0, 1}
    f32x4 S[8][2];
    {
        const int lane = tid & 63, gq = lane >> 4, cl = lane & 15;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int vcol = 16 * (2 * wave + j) + cl;
                const float4 x =
                    *(const float4*)(a.s0 + slab + (int64_t)vcol * D + 16 * kb + 4 * gq);
                S[kb][j] = f32x4{x.x, x.y, x.z, x.w};
            }
    }

    const float eA = __expf(a.A_log[h]);
    // z*log2(e) = g*(eA log2e) + dt*(eA log2e); the log2-domain decay is
    // -5 log2(e) sigmoid(z)
    const float zs = eA * LOG2E;
    if (tid < D) sm.dtz[tid] = a.dt_bias[h * D + tid] * zs;

    RowIn cur;
    ColIn vcur;
    {
        const int lane = tid & 63;
        load_rows(cur, a, tok0 + min(tid >> 4, L - 1), hq, h, (tid & 15) * 8);
        load_cols(vcur, a, tok0 + min(lane & 15, L - 1), h, 32 * wave + 4 * (lane >> 4));
    }
    __syncthreads();

    const int nchunks = (L + CH - 1) / CH;
    for (int ci = 0; ci < nchunks; ++ci) {
        // Per-lane index arithmetic is recomputed every iteration from an
        // opaque copy of the thread id; hoisted out of the loop it would keep
        // ~20 address registers alive and push the kernel into scratch spills.
        int tix = tid;
        asm volatile("" : "+v"(tix));
        const int lane = tix & 63;
        const int gq = lane >> 4;
        const int cl = lane & 15;
        const int r = tix >> 4;          // row-owner mapping: token row r,
        const int c8 = (tix & 15) * 8;   // channels [c8, c8 + 8)
        const int t0 = ci * CH;
        const int nv = min(CH, L - t0);
        const bool valid = r < nv;

        // ---- A: norms, gate, beta ----
        float rq, rk;
        {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float qv = (float)cur.q[i], kv = (float)cur.k[i];
                sq += qv * qv;
                sk += kv * kv;
            }
            sq = group_sum<16>(sq);
            sk = group_sum<16>(sk);
            rq = valid ? fast_rsqrt(sq + 1e-6f) : 0.f;
            rk = valid ? fast_rsqrt(sk + 1e-6f) : 0.f;
            float lv[8], dz[8];
            *(float4*)&dz[0] = *(const float4*)&sm.dtz[c8];
            *(float4*)&dz[4] = *(const float4*)&sm.dtz[c8 + 4];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float e = __builtin_amdgcn_exp2f(-((float)cur.g[i] * zs + dz[i]));
                lv[i] = valid ? (-5.0f * LOG2E) * __builtin_amdgcn_rcpf(1.0f + e) : 0.f;
            }
            *(float4*)&sm.lam[r][c8] = make_float4(lv[0], lv[1], lv[2], lv[3]);
            *(float4*)&sm.lam[r][c8 + 4] = make_float4(lv[4], lv[5], lv[6], lv[7]);
            if ((tix & 15) == 0) sm.beta[r] = valid ? sigmoidf_((float)cur.b) : 0.f;
        }
        __syncthreads();
        // ---- B: prefix sums over the chunk's tokens, per channel ----
        if (tix < D) {
            float acc = 0.f;
#pragma unroll
            for (int rr = 0; rr < CH; ++rr) {
                acc += sm.lam[rr][tix];
                sm.lam[rr][tix] = acc;
            }
            sm.gamc[tix] = __builtin_amdgcn_exp2f(acc);
        }
        __syncthreads();
        // ---- C: decay factors and the chunk's operands ----
        {
            float gc[8], gC[8];
            *(float4*)&gc[0] = *(const float4*)&sm.lam[r][c8];
            *(float4*)&gc[4] = *(const float4*)&sm.lam[r][c8 + 4];
            *(float4*)&gC[0] = *(const float4*)&sm.gamc[c8];
            *(float4*)&gC[4] = *(const float4*)&sm.gamc[c8 + 4];
            bf16x4 qg4[2], kg4[2], ki4[2];
            const int ocf = cf_off(r, c8);  // channel c8 + i sits at ocf + 4i
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float qn = (float)cur.q[i] * rq;
                const float kn = (float)cur.k[i] * rk;
                const float gam = __builtin_amdgcn_exp2f(gc[i]);
                const float gin = __builtin_amdgcn_exp2f(-gc[i]);
                const float kg = kn * gam;
                const float kt = kn * gin * gC[i];
                qg4[i >> 2][i & 3] = (bf16)(qn * gam);
                const bf16 kgb = (bf16)kg;
                kg4[i >> 2][i & 3] = kgb;
                ki4[i >> 2][i & 3] = (bf16)(kn * gin);
                const bf16 kth = (bf16)kt;
                sm.cf_kg[ocf + 4 * i] = kgb;
                sm.cf_kth[ocf + 4 * i] = kth;
                sm.cf_ktl[ocf + 4 * i] = (bf16)(kt - (float)kth);
            }
            const int orf = rf_off(r, c8);  // channels c8+4.. sit one lane group later
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                *(bf16x4*)&sm.rf_qg[orf + 64 * s] = qg4[s];
                *(bf16x4*)&sm.rf_kg[orf + 64 * s] = kg4[s];
                *(bf16x4*)&sm.rf_ki[orf + 64 * s] = ki4[s];
            }
        }
        // the row inputs are dead: fetch the next chunk's into the same registers
        load_rows(cur, a, tok0 + min(t0 + CH + r, L - 1), hq, h, c8);
        __syncthreads();
        // ---- D: V to CF (all); Akk and the substitution (wave 0); Aqk (wave 1) ----
        bf16x4 cfv[2];
        {
            bf16x4 ident;  // frag of the 16x16 identity: lane (gq, n) holds I[4gq+i][n]
#pragma unroll
            for (int i = 0; i < 4; ++i) ident[i] = (bf16)((4 * gq + i == cl) ? 1.0f : 0.0f);
            // CF(V)[vb] = RF(V)[vb] * I, exact
            cfv[0] = to_bf4(mma16(vcur.v0, ident, zero4()));
            cfv[1] = to_bf4(mma16(vcur.v1, ident, zero4()));
        }
        load_cols(vcur, a, tok0 + min(t0 + CH + cl, L - 1), h, 32 * wave + 4 * gq);
        if (wave == 0) {
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 x = cat8(ld4(&sm.rf_kg[(2 * j) * FS], lane), ld4(&sm.rf_kg[(2 * j + 1) * FS], lane));
                const bf16x8 y = cat8(ld4(&sm.rf_ki[(2 * j) * FS], lane), ld4(&sm.rf_ki[(2 * j + 1) * FS], lane));
                acc = mma32(x, y, acc);
            }
            // lane (gq, cl) holds Akk[4gq+i][cl]: store column cl, rows 4gq..4gq+3
            {
                float4 col;
                col.x = (cl < 4 * gq + 0) ? acc[0] : 0.f;
                col.y = (cl < 4 * gq + 1) ? acc[1] : 0.f;
                col.z = (cl < 4 * gq + 2) ? acc[2] : 0.f;
                col.w = (cl < 4 * gq + 3) ? acc[3] : 0.f;
                *(float4*)&sm.akkT[cl][4 * gq] = col;
            }
            if (lane < 16) {
                // Column `lane` of T by right-looking substitution: once t[m]
                // is final, every later row takes its share of it.
                //   t[i] = [i == col] - beta_i * sum_{m<i} Akk[i][m] t[m]
                const int col = lane;
                float acc_t[CH];
#pragma unroll
                for (int i = 0; i < CH; ++i) acc_t[i] = 0.f;
                float t[CH];
#pragma unroll
                for (int m = 0; m < CH; ++m) {
                    const float tm = (m == col) ? 1.0f : -sm.beta[m] * acc_t[m];
                    t[m] = tm;
                    if (m + 1 < CH) {
                        float ac[CH];
#pragma unroll
                        for (int q4 = 0; q4 < 4; ++q4)
                            if (4 * q4 + 3 > m) *(float4*)&ac[4 * q4] = *(const float4*)&sm.akkT[m][4 * q4];
#pragma unroll
                        for (int i = m + 1; i < CH; ++i) acc_t[i] += ac[i] * tm;
                    }
                }
                const float bc = sm.beta[col];
#pragma unroll
                for (int i = 0; i < CH; ++i) {
                    const float x = t[i] * bc;  // Tb[i][col]
                    const bf16 xh = (bf16)x;
                    const int o = (((col >> 2) << 4) + i) * 4 + (col & 3);
                    sm.tbh[o] = xh;
                    sm.tbl[o] = (bf16)(x - (float)xh);
                }
            }
        } else if (wave == 1) {
            // Aqk^T = Ki Qg^T: lane (gq, c) holds Aqk[c][4gq+i] = RF16(Aqk)
            f32x4 acc = zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 x = cat8(ld4(&sm.rf_ki[(2 * j) * FS], lane), ld4(&sm.rf_ki[(2 * j + 1) * FS], lane));
                const bf16x8 y = cat8(ld4(&sm.rf_qg[(2 * j) * FS], lane), ld4(&sm.rf_qg[(2 * j + 1) * FS], lane));
                acc = mma32(x, y, acc);
            }
            bf16x4 x;
#pragma unroll
            for (int i = 0; i < 4; ++i) x[i] = (bf16)((4 * gq + i <= cl) ? acc[i] : 0.f);
            st4(sm.aqk, lane, x);
        }
        __syncthreads();
        // ---- E: -W frags (kb = 2w, 2w+1) and Ut for the wave's columns ----
        f32x4 U[2];
        {
            const bf16x4 tbh = ld4(sm.tbh, lane);
            const bf16x4 tbl = ld4(sm.tbl, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kb = 2 * wave + j;
                // W^T[kb] = Kg^T Tb^T: A = CF(Kg)[kb], B = RF16(Tb)
                const f32x4 w = mma16(ld4(&sm.cf_kg[kb * FS], lane), tbh, zero4());
                st4(&sm.rf_w[kb * FS], lane, to_bf4(-w));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                U[j] = mma16(tbh, cfv[j], zero4());
                U[j] = mma16(tbl, cfv[j], U[j]);
            }
        }
        __syncthreads();
        // ---- F: U = Ut - W S0^T;  O^T = S0 Qg^T + U^T Aqk^T;  S update ----
        f32x4 OT[2] = {zero4(), zero4()};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8 w8 = cat8(ld4(&sm.rf_w[(2 * j) * FS], lane), ld4(&sm.rf_w[(2 * j + 1) * FS], lane));
            const bf16x8 q8 = cat8(ld4(&sm.rf_qg[(2 * j) * FS], lane), ld4(&sm.rf_qg[(2 * j + 1) * FS], lane));
#pragma unroll
            for (int vb = 0; vb < 2; ++vb) {
                const bf16x8 s8 = cat8(to_bf4(S[2 * j][vb]), to_bf4(S[2 * j + 1][vb]));
                U[vb] = mma32(w8, s8, U[vb]);
                OT[vb] = mma32(s8, q8, OT[vb]);
            }
        }
        const bf16x4 aq = ld4(sm.aqk, lane);
        bf16x4 uh[2], ul[2];
#pragma unroll
        for (int vb = 0; vb < 2; ++vb) {
            split4(U[vb], uh[vb], ul[vb]);
            OT[vb] = mma16(uh[vb], aq, OT[vb]);
            // lane (gq, c) holds O[c][32w + 16vb + 4gq + i]
            if (cl < nv) {
                bf16x4 ob;
#pragma unroll
                for (int i = 0; i < 4; ++i) ob[i] = (bf16)(OT[vb][i] * a.scale);
                *(bf16x4*)((bf16*)a.o + (tok0 + t0 + cl) * a.Hv * D + h * D + 32 * wave + 16 * vb + 4 * gq) = ob;
            }
        }
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const bf16x4 th = ld4(&sm.cf_kth[kb * FS], lane);
            const bf16x4 tl = ld4(&sm.cf_ktl[kb * FS], lane);
            const bf16x8 thh = cat8(th, th);
            const float4 gd = *(const float4*)&sm.gamc[16 * kb + 4 * gq];
#pragma unroll
            for (int vb = 0; vb < 2; ++vb) {
                f32x4 s = S[kb][vb];
                s[0] *= gd.x; s[1] *= gd.y; s[2] *= gd.z; s[3] *= gd.w;
                s = mma32(thh, cat8(uh[vb], ul[vb]), s);
                s = mma16(tl, uh[vb], s);
                S[kb][vb] = s;
            }
        }
        const int tend = t0 + nv;
        if (a.tape != nullptr && tend < L && (tend % a.ck_every) == 0) {
            const int64_t jck = tend / a.ck_every;
            store_state(a.tape + ((tape_base + jck - 1) * a.Hv + h) * (int64_t)D * D, S, wave, gq, cl);
        }
    }
    {
        const int lane = tid & 63;
        if (a.s_final != nullptr) store_state(a.s_final + slab, S, wave, lane >> 4, lane & 15);
    }
}

hipError_t launch_fwd_chunk(const FwdArgs& a, hipStream_t s) {
    if (a.num_tasks == 0) return hipSuccess;
    hipLaunchKernelGGL(fwd_chunk_kernel, dim3((unsigned)a.num_tasks), dim3(FC_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
