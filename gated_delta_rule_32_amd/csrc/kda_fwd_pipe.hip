// Column-split training forward for calls with few tasks: producer waves
// prepare whole chunks ahead of the state path.
//
// The chunk form is the chunked forward's (page
// "flashinfer.kda_backward.recurrent_kda_backward", description; the steps
// are listed at the top of kda_fwd_chunk.hip): for each 16-token chunk,
// gc = cumsum(lam), Qg = qn exp(gc), Kg = kn exp(gc), Ki = kn exp(-gc),
// Kt = Ki exp(gC); Akk = strict-lower(Kg Ki^T), Aqk = lower(Qg Ki^T);
// Tb = (I + diag(beta) Akk)^-1 diag(beta); Y = Kg S0^T, U = Tb V - Tb Y;
// O = scale (Qg S0^T + Aqk U); S_C = S0 diag(exp(gC)) + U^T Kt.  The products
// and their precision are the chunked kernel's.
//
// With at most 128 tasks each column half of a task (two workgroups per task,
// 8 blocks apart so that both sit on one XCD) runs alone on its compute unit,
// and the call lasts as long as one task's chain of chunks.  Only Y, U, the
// output and the update depend on the carried state; the rest of a chunk
// (norms, gate, beta, decay prefix sums, the operands, Akk, the substitution
// for Tb, Aqk) can run ahead.  Eight waves:
//   - waves 0-3 (consumers) own one 16-column block of the state each and
//     run the state path of chunk s in step s, from LDS only;
//   - wave 4 + j (producer j) prepares chunks j, j+4, j+8, ..., each alone
//     and in four stages, one per step: stage k of chunk c runs in step
//     c - 4 + k, so four chunks are in flight and chunk c's operands are
//     complete when step c begins.  Its results go to LDS slot c mod 4.
// One barrier per step.  The two groups run separate loops with the same
// number of steps and one barrier each, so every wave meets every barrier.
//
// A producer lane (gq, t) holds token t of the chunk and channels 16kb + 4gq
// + i (kb = 0..7, i = 0..3): the operands' RF frag layout, so that Akk and
// Aqk multiply straight from registers and the RF slots are plain 8-byte
// stores.  The decay prefix sums over tokens run along each 16-lane row by
// DPP shifts; CF(Kt) (tokens along the register) is the RF frag transposed
// exactly through the matrix unit.
#include "kda_chunk.hpp"

namespace kda {

namespace {

constexpr int PP_THREADS = 512;
constexpr int PP_FS2 = 520;  // CF(Kt) slot stride: 8 halves per lane (512 + 8 padding)
constexpr int PP_VS = 136;   // V row stride in a slot, halves (128 + 8 padding)

struct PipeSlot {  // one chunk's operands, written by its producer
    alignas(16) bf16 rf_qg[8 * FS];     // RF(Qg), the output scale included
    alignas(16) bf16 rf_kg[8 * FS];     // RF(Kg)
    alignas(16) bf16 rf_kg_lo[8 * FS];  // precise chunks: Kg's lo part
    alignas(16) f16 cf_kt[8 * PP_FS2];  // CF(Kt) as [hi | lo] FP16 pairs
    alignas(16) bf16 vrow[CH * PP_VS];  // the chunk's rows of v
    alignas(16) bf16x8 tb2[64];         // [Tb_hi | Tb_lo], lane (gq, c) holding Tb[c][4gq+i]
    alignas(16) bf16x8 aq[64];          // [Aqk/2 | Aqk/2], lane (gq, c) holding Aqk[c][4gq+i]
    alignas(16) float gamc[D];          // exp(gC) per channel
    alignas(16) float glog[D];          // gC (log2 domain) per channel
    int precise;                        // the chunk runs precise
};

struct ProdScratch {  // one producer's
    alignas(16) float nT[CH][CH];   // nT[m][i] = beta_i Akk[i][m] for i > m
    alignas(16) float tb[CH][20];   // Tb[i][j] (16-byte rows)
    alignas(16) float beta[CH];
};

struct PipeLds {
    PipeSlot slot[4];   // by chunk mod 4 (= its producer)
    ProdScratch scr[4];
    alignas(16) float dtz[D];  // dt_bias * exp(A_log) * log2(e)
};

// Sum over the 4 lane rows (gq) of a wave, on every row.
__device__ __forceinline__ float sum_rows(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Inclusive prefix sum along each 16-lane row (lane t gets lanes 0..t of its
// row): DPP row shifts toward higher lanes, zero-filled.
__device__ __forceinline__ float row16_prefix(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xF, 0xF, true));
    return x;
}

// Exact transpose of an FP16 frag (lane (gq, m) holding X[m][4gq+i]) into
// the accumulator layout (lane (gq, n) holding X[4gq+i][n]).
__device__ __forceinline__ f16x4 transpose_frag_h(f16x4 x, f16x4 ident) {
    return to_f16x4(__builtin_amdgcn_mfma_f32_16x16x16f16(x, ident, zero4(), 0, 0, 0));
}

struct ProdRows {  // one producer lane's inputs of a chunk
    bf16x4 q[8], k[8], g[8];  // token t, channels 16kb + 4gq + i
    bf16 b;
    bf16x8 v[4];              // v rows: token lane/4, channels 32 (lane%4) + 8m + 0..7
};

}  // namespace

__global__ __launch_bounds__(PP_THREADS, 1) void fwd_pipe_kernel(FwdArgs a) {
    __shared__ PipeLds sm;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool prod = wave >= 4;
    const int b = blockIdx.x;
    const int ti = (b >> 4) * 8 + (b & 7);
    if (ti >= a.num_tasks) return;  // uniform over the workgroup: before any barrier
    const int code = a.plan.task[ti];
    const int n = code / a.Hv;
    const int h = code - n * a.Hv;
    const int hq = h / a.G;
    const int64_t tok0 = a.plan.seq_start[n];
    const int L = a.plan.seq_len[n];
    const int64_t slab = ((int64_t)n * a.Hv + h) * D * D;
    const int nch = (L + CH - 1) / CH;

    SeqPtrs sp;
    sp.q = (const bf16*)a.q + (tok0 * a.Hqk + hq) * D;
    sp.k = (const bf16*)a.k + (tok0 * a.Hqk + hq) * D;
    sp.g = (const bf16*)a.g + (tok0 * a.Hv + h) * D;
    sp.v = (const bf16*)a.v + (tok0 * a.Hv + h) * D;
    sp.o = (bf16*)a.o + (tok0 * a.Hv + h) * D;
    sp.beta = (const bf16*)a.beta + tok0 * a.Hv + h;
    sp.sq = (unsigned)(a.Hqk * D);
    sp.sv = (unsigned)(a.Hv * D);
    sp.sb = (unsigned)a.Hv;

    const float zs = __expf(a.A_log[h]) * LOG2E;
    if (tid < D) sm.dtz[tid] = a.dt_bias != nullptr ? a.dt_bias[h * D + tid] * zs : 0.f;
    __syncthreads();

    if (prod) {
        // ================= producer j: chunks j, j+4, ... =================
        // (issue priority over the consumer on the same SIMD: the producers
        // set the step, the consumers have slack in it)
        __builtin_amdgcn_s_setprio(3);
        const int j = wave - 4;
        const int lane = tid & 63;
        const int gq = lane >> 4;
        const int t = lane & 15;
        PipeSlot& sl = sm.slot[j];
        ProdScratch& sc = sm.scr[j];
        const float lb2 = -5.0f * LOG2E;  // log2-domain lower bound of the decay
        ProdRows in;
        auto load_rows = [&](const int ci) __attribute__((always_inline)) {
            const unsigned tk = (unsigned)min(ci * CH + t, L - 1);
            const unsigned oq = __umul24(tk, sp.sq) + 4 * gq, og = __umul24(tk, sp.sv) + 4 * gq;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                in.q[kb] = *(const bf16x4*)at(sp.q, oq + 16 * kb);
                in.k[kb] = *(const bf16x4*)at(sp.k, oq + 16 * kb);
                in.g[kb] = *(const bf16x4*)at(sp.g, og + 16 * kb);
            }
            in.b = *at(sp.beta, __umul24(tk, sp.sb));
            const unsigned tv = (unsigned)min(ci * CH + (lane >> 2), L - 1);
            const unsigned ov = __umul24(tv, sp.sv) + 32 * (lane & 3);
#pragma unroll
            for (int m = 0; m < 4; ++m) in.v[m] = *(const bf16x8*)at(sp.v, ov + 8 * m);
        };
        float rq = 0.f, rk = 0.f;
        f32x4 lam[8];             // decays, then their prefix sums gc, then exp(-gc)
        f32x4 gam[8];             // exp(gc) in stages 1-2, then Kt for stage 3
        f32x4 akk, aqkT;          // Akk (lane (gq, c): Akk[4gq+i][c]) and Aqk^T
        bool precise = false;
        const f16x4 identh = [&] {
            f32x4 id;
#pragma unroll
            for (int i = 0; i < 4; ++i) id[i] = (4 * gq + i == t) ? 1.0f : 0.0f;
            return to_f16x4(id);
        }();

        if (j < nch) load_rows(j);
        for (int s = -4; s < nch; ++s) {
            const int d = (j - s - 1) & 3;
            const int ci = s + 1 + d;       // this producer's chunk in this step
            const int stage = 3 - d;
            if (ci >= 0 && ci < nch) {
                const float vm = t < L - ci * CH ? 1.0f : 0.0f;
                if (stage == 0) {
                    // norms (BF16 pair dot products, FP32 sums over the row's
                    // four lanes), gate and beta
                    float sq = 0.f, sk = 0.f;
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) {
                        const bf16x4 q4 = in.q[kb], k4 = in.k[kb];
                        sq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q4, q4, 0, 1),
                                                             __builtin_shufflevector(q4, q4, 0, 1), sq, false);
                        sq = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q4, q4, 2, 3),
                                                             __builtin_shufflevector(q4, q4, 2, 3), sq, false);
                        sk = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(k4, k4, 0, 1),
                                                             __builtin_shufflevector(k4, k4, 0, 1), sk, false);
                        sk = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(k4, k4, 2, 3),
                                                             __builtin_shufflevector(k4, k4, 2, 3), sk, false);
                    }
                    sq = sum_rows(sq);
                    sk = sum_rows(sk);
                    rq = (a.scale * vm) * fast_rsqrt(sq + 1e-6f);  // the output scale rides on Qg
                    rk = vm * fast_rsqrt(sk + 1e-6f);
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) {
                        const float4 dz = *(const float4*)&sm.dtz[16 * kb + 4 * gq];
                        const float dzi[4] = {dz.x, dz.y, dz.z, dz.w};
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float e = __builtin_amdgcn_exp2f(-((float)in.g[kb][i] * zs + dzi[i]));
                            lam[kb][i] = (lb2 * vm) * __builtin_amdgcn_rcpf(1.0f + e);
                        }
                    }
                    if (gq == 0) sc.beta[t] = vm * sigmoidf_((float)in.b);
                    // prefix sums over the chunk's tokens, channel blocks 0-3
#pragma unroll
                    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) lam[kb][i] = row16_prefix(lam[kb][i]);
                } else if (stage == 1) {
                    // prefix sums of channel blocks 4-7; gC and the precision
                    // flag from the row's last token; exp(gc) and exp(-gc) (the
                    // latter in place of gc); exp(gC) two channels per lane
#pragma unroll
                    for (int kb = 4; kb < 8; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) lam[kb][i] = row16_prefix(lam[kb][i]);
                    bool hot = false;
                    if (t == 15) {
#pragma unroll
                        for (int kb = 0; kb < 8; ++kb) {
                            *(float4*)&sl.glog[16 * kb + 4 * gq] =
                                make_float4(lam[kb][0], lam[kb][1], lam[kb][2], lam[kb][3]);
#pragma unroll
                            for (int i = 0; i < 4; ++i) hot = hot || lam[kb][i] > a.precise_log2;
                        }
                    }
                    precise = __builtin_amdgcn_ballot_w64(hot) != 0;
                    if (lane == 0) sl.precise = precise ? 1 : 0;
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            gam[kb][i] = __builtin_amdgcn_exp2f(lam[kb][i]);
                            lam[kb][i] = __builtin_amdgcn_exp2f(-lam[kb][i]);
                        }
                    // (this wave's own stores above: LDS keeps one wave's
                    // accesses in order)
                    const float2 gl = *(const float2*)&sl.glog[2 * lane];
                    *(float2*)&sl.gamc[2 * lane] =
                        make_float2(__builtin_amdgcn_exp2f(gl.x), __builtin_amdgcn_exp2f(gl.y));
                } else if (stage == 2) {
                    // the operands: RF(Qg), RF(Kg) (+ lo) to the slot, CF(Kt)
                    // as transposed FP16 pairs, v rows; then Akk and Aqk
                    // (two channel blocks at a time, so that few operands are live)
                    akk = zero4();
                    aqkT = zero4();
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        bf16x4 qg4[2], kg4[2], ki4[2], kgl4[2], kil4[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int kb = 2 * jj + e;
                            const float4 gC = *(const float4*)&sl.gamc[16 * kb + 4 * gq];
                            const float gCi[4] = {gC.x, gC.y, gC.z, gC.w};
                            f32x4 qg, kg, ki, kt;
#pragma unroll
                            for (int i = 0; i < 4; ++i) {
                                const float qn = (float)in.q[kb][i] * rq;
                                const float kn = (float)in.k[kb][i] * rk;
                                const float gi = lam[kb][i];   // exp(-gc)
                                qg[i] = qn * gam[kb][i];
                                kg[i] = kn * gam[kb][i];
                                ki[i] = kn * gi;
                                kt[i] = ki[i] * gCi[i];
                            }
                            qg4[e] = to_bf4(qg);
                            if (precise) {
                                split4(kg, kg4[e], kgl4[e]);
                                split4(ki, ki4[e], kil4[e]);
                                *(bf16x4*)&sl.rf_kg_lo[kb * FS + lane * 4] = kgl4[e];
                            } else {
                                kg4[e] = to_bf4(kg);
                                ki4[e] = to_bf4(ki);
                            }
                            *(bf16x4*)&sl.rf_qg[kb * FS + lane * 4] = qg4[e];
                            *(bf16x4*)&sl.rf_kg[kb * FS + lane * 4] = kg4[e];
                            gam[kb] = kt;
                        }
                        const bf16x8 kg8 = cat8(kg4[0], kg4[1]);
                        const bf16x8 ki8 = cat8(ki4[0], ki4[1]);
                        akk = mma32(kg8, ki8, akk);   // lane (gq, c) holds Akk[4gq+i][c]
                        if (precise) {   // + Kg_hi Ki_lo + Kg_lo Ki_hi
                            akk = mma32(kg8, cat8(kil4[0], kil4[1]), akk);
                            akk = mma32(cat8(kgl4[0], kgl4[1]), ki8, akk);
                        }
                        aqkT = mma32(ki8, cat8(qg4[0], qg4[1]), aqkT);  // Aqk^T
                    }
                    {
                        bf16* vr = &sl.vrow[(lane >> 2) * PP_VS + 32 * (lane & 3)];
#pragma unroll
                        for (int m = 0; m < 4; ++m) *(bf16x8*)(vr + 8 * m) = in.v[m];
                    }
                    // the rows are dead: fetch those of this producer's next chunk
                    if (ci + 4 < nch) load_rows(ci + 4);
                } else {
                    // CF(Kt) as FP16 pairs (about 22 bits: Kt lies in [0, 1]),
                    // transposed; the substitution for Tb; Aqk to the slot
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) {
                        f16x4 hh, ll;
                        split4_f16(gam[kb], hh, ll);
                        *(f16x8*)&sl.cf_kt[kb * PP_FS2 + lane * 8] =
                            cat8h(transpose_frag_h(hh, identh), transpose_frag_h(ll, identh));
                    }
                    {
                        // RF16(Aqk), causal part, halved and stored twice:
                        // [Aqk/2 | Aqk/2] against [U_hi | U_hi] is U_hi Aqk
                        f32x4 am;
#pragma unroll
                        for (int i = 0; i < 4; ++i) am[i] = (4 * gq + i <= t) ? aqkT[i] * 0.5f : 0.f;
                        const bf16x4 ah = to_bf4(am);
                        sl.aq[lane] = cat8(ah, ah);
                    }
                    const float4 b4 = *(const float4*)&sc.beta[4 * gq];
                    float4 col;  // column t of N = diag(beta) Akk, rows 4gq..4gq+3
                    col.x = (t < 4 * gq + 0) ? b4.x * akk[0] : 0.f;
                    col.y = (t < 4 * gq + 1) ? b4.y * akk[1] : 0.f;
                    col.z = (t < 4 * gq + 2) ? b4.z * akk[2] : 0.f;
                    col.w = (t < 4 * gq + 3) ? b4.w * akk[3] : 0.f;
                    *(float4*)&sc.nT[t][4 * gq] = col;
                    // T = (I + N)^-1 by right-looking substitution on all 64
                    // lanes: lane (col = lane/4, q = lane%4) keeps rows
                    // 4q..4q+3 of column col and loses N[row][m] t[m] at step m
                    const int colx = lane >> 2;
                    const int qd = lane & 3;
                    float y[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) y[jj] = (4 * qd + jj == colx) ? 1.0f : 0.0f;
                    float4 nxt = *(const float4*)&sc.nT[0][4 * qd];
#pragma unroll
                    for (int m = 0; m < CH - 1; ++m) {
                        const float4 nm = nxt;
                        if (m + 1 < CH - 1) nxt = *(const float4*)&sc.nT[m + 1][4 * qd];
                        const float tm = quad_bcast(y[m & 3], m >> 2);
                        if (m < 12) y[0] -= nm.x * tm;
                        if (m < 13) y[1] -= nm.y * tm;
                        if (m < 14) y[2] -= nm.z * tm;
                        y[3] -= nm.w * tm;
                    }
                    const float bc = sc.beta[colx];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) sc.tb[4 * qd + jj][colx] = y[jj] * bc;
                    // RF16(Tb) as a hi/lo pair: lane (gq, c) holds Tb[c][4gq+i]
                    const float4 t4 = *(const float4*)&sc.tb[t][4 * gq];
                    bf16x4 tbh, tbl;
                    split4(f32x4{t4.x, t4.y, t4.z, t4.w}, tbh, tbl);
                    sl.tb2[lane] = cat8(tbh, tbl);
                }
            }
            __syncthreads();
        }
    } else {
        // ================= consumers: the state path =================
        int tix = tid;
        asm volatile("" : "+v"(tix));
        const int lane = tix & 63, gq = lane >> 4, cl = lane & 15;
        const int vb0 = 4 * ((b >> 3) & 1) + wave;  // this wave's 16-column block
        const int64_t tape_base = a.tape != nullptr ? a.plan.tape_off[n] : 0;
        f32x4 S[8];  // S^T frags: lane (gq, cl) holds S[16vb0 + cl][16kb + 4gq + i]
        {
            const float* src = a.s0 + slab + (int64_t)(16 * vb0 + cl) * D + 4 * gq;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const float4 x = *(const float4*)(src + 16 * kb);
                S[kb] = f32x4{x.x, x.y, x.z, x.w};
            }
        }
        for (int s = -4; s < nch; ++s) {
            if (s >= 0) {
                const PipeSlot& sl = sm.slot[s & 3];
                const int t0 = s * CH;
                const bool precise = __builtin_amdgcn_readfirstlane(sl.precise) != 0;
                // U starts from Tb V (state-independent, off the chain)
                const bf16x8 tb2 = sl.tb2[lane];
                bf16x4 vv;
#pragma unroll
                for (int i = 0; i < 4; ++i) vv[i] = sl.vrow[(4 * gq + i) * PP_VS + 16 * vb0 + cl];
                f32x4 U = mma32(tb2, cat8(vv, vv), zero4());
                // Y = Kg S0^T, O^T = S0 Qg^T
                f32x4 Y = zero4(), OT = zero4();
                if (precise) {
                    // Y = Kg_hi S0_hi + Kg_hi S0_lo + Kg_lo S0_hi, O^T from S0_hi
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const bf16x8 kg8 = cat8(ld4(&sl.rf_kg[(2 * jj) * FS], lane), ld4(&sl.rf_kg[(2 * jj + 1) * FS], lane));
                        const bf16x8 kl8 = cat8(ld4(&sl.rf_kg_lo[(2 * jj) * FS], lane),
                                                ld4(&sl.rf_kg_lo[(2 * jj + 1) * FS], lane));
                        const bf16x8 q8 = cat8(ld4(&sl.rf_qg[(2 * jj) * FS], lane), ld4(&sl.rf_qg[(2 * jj + 1) * FS], lane));
                        bf16x4 h0, l0, h1, l1;
                        split4(S[2 * jj], h0, l0);
                        split4(S[2 * jj + 1], h1, l1);
                        const bf16x8 sh = cat8(h0, h1);
                        Y = mma32(kg8, sh, Y);
                        Y = mma32(kg8, cat8(l0, l1), Y);
                        Y = mma32(kl8, sh, Y);
                        OT = mma32(sh, q8, OT);
                    }
                    bf16x4 yh, yl;
                    split4(-Y, yh, yl);
                    U = mma32(tb2, cat8(yh, yh), U);
                    U = mma32(tb2, cat8(yl, yl), U);
                } else {
                    bf16x8 sb[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const bf16x8 kg8 = cat8(ld4(&sl.rf_kg[(2 * jj) * FS], lane), ld4(&sl.rf_kg[(2 * jj + 1) * FS], lane));
                        sb[jj] = cat8(to_bf4(S[2 * jj]), to_bf4(S[2 * jj + 1]));
                        Y = mma32(kg8, sb[jj], Y);    // lane (gq, v) holds Y[4gq+i][v]
                    }
                    U = mma32(tb2, cat8(to_bf4_neg(Y), to_bf4_neg(Y)), U);
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        const bf16x8 q8 = cat8(ld4(&sl.rf_qg[(2 * jj) * FS], lane), ld4(&sl.rf_qg[(2 * jj + 1) * FS], lane));
                        OT = mma32(sb[jj], q8, OT);   // lane (gq, c): O[c][v=4gq+i]
                    }
                }
                // O^T += U^T Aqk^T; lane (gq, c) holds O[c][16vb0 + 4gq + i]
                {
                    const bf16x4 uh = to_bf4(U);
                    OT = mma32(cat8(uh, uh), sl.aq[lane], OT);
                    if (cl < L - t0) {
                        const bf16x4 ob = to_bf4(OT);
                        *(bf16x4*)at(sp.o, __umul24((unsigned)(t0 + cl), sp.sv) + 16 * vb0 + 4 * gq) = ob;
                    }
                }
                // the decay and S^T += Kt^T U in FP16 ([Kt_hi|Kt_lo] against
                // [U;U], precise chunks add [U_lo;U_lo]); U beyond FP16's
                // range is scaled by a power of two around the product, the
                // state with it
                float um = fmaxf(fmaxf(fabsf(U[0]), fabsf(U[1])), fmaxf(fabsf(U[2]), fabsf(U[3])));
                const bool big = __builtin_amdgcn_ballot_w64(!(um < 16384.f)) != 0;
                float isc = 1.f;
                if (big) {
#pragma unroll
                    for (int o = 1; o < 64; o <<= 1) um = fmaxf(um, __shfl_xor(um, o, 64));
                    const int e = __builtin_amdgcn_readfirstlane(um < 3.0e38f ? max(ilogbf(um) - 12, 0) : 116);
                    const float scl = ldexpf(1.f, -e);
                    isc = ldexpf(1.f, e);
                    U *= scl;
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) S[kb] *= scl;
                }
                f16x4 uhh, ull;
                if (precise)
                    split4_f16(U, uhh, ull);
                else
                    uhh = to_f16x4(U);
                const f16x8 uh8 = cat8h(uhh, uhh);
#pragma unroll
                for (int kb = 0; kb < 8; ++kb) {
                    const f16x8 t2 = *(const f16x8*)&sl.cf_kt[kb * PP_FS2 + lane * 8];
                    const float4 gd = *(const float4*)&sl.gamc[16 * kb + 4 * gq];
                    f32x4 sv = S[kb];
                    sv[0] *= gd.x; sv[1] *= gd.y; sv[2] *= gd.z; sv[3] *= gd.w;
                    S[kb] = mma32h(t2, uh8, sv);
                }
                if (precise) {
                    const f16x8 ul8 = cat8h(ull, ull);
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) {
                        const f16x8 t2 = *(const f16x8*)&sl.cf_kt[kb * PP_FS2 + lane * 8];
                        S[kb] = mma32h(t2, ul8, S[kb]);
                    }
                }
                if (big) {
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb) S[kb] *= isc;
                }
                const int tend = min(t0 + CH, L);
                if (a.tape != nullptr && tend < L && (tend % a.ck_every) == 0) {
                    float* dst = a.tape + ((tape_base + tend / a.ck_every - 1) * a.Hv + h) * (int64_t)D * D +
                                 (int64_t)(16 * vb0 + cl) * D + 4 * gq;
#pragma unroll
                    for (int kb = 0; kb < 8; ++kb)
                        *(float4*)(dst + 16 * kb) = make_float4(S[kb][0], S[kb][1], S[kb][2], S[kb][3]);
                }
            }
            __syncthreads();
        }
        if (a.s_final != nullptr) {
            float* dst = a.s_final + slab + (int64_t)(16 * vb0 + cl) * D + 4 * gq;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
                *(float4*)(dst + 16 * kb) = make_float4(S[kb][0], S[kb][1], S[kb][2], S[kb][3]);
        }
    }
}

hipError_t launch_fwd_pipe(const FwdArgs& a, hipStream_t s) {
    if (a.num_tasks == 0) return hipSuccess;
    hipLaunchKernelGGL(fwd_pipe_kernel, dim3((unsigned)(16 * ((a.num_tasks + 7) / 8))), dim3(PP_THREADS), 0,
                       s, a);
    return hipGetLastError();
}

}  // namespace kda
