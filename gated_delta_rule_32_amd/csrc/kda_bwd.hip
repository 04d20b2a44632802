// Backward of the KDA training recurrence: the chunk adjoint and the ordered
// reductions.
//
// The loss is <do, o> + <dfinal_state, S_L> (page
// "flashinfer.kda_backward.recurrent_kda_backward", description); its
// gradients are taken through the chunked (WY / UT) form of the recurrence
// that the forward evaluates.  For a chunk with start state S0, end state S_C
// and the quantities of the forward (Qg' = scale*Qg, Kg, Ki, Kt, T, Tb = T
// diag(beta), Akk, Aqk' = scale*Aqk, U, W = Tb Kg), the adjoint dS of S_C
// gives, in this order:
//
//   dS0  = dS diag(exp(gC)) + dO^T Qg' - dU^T W        (carried to the chunk before)
//   dU   = Kt dS^T + Aqk'^T dO
//   dKt  = U dS,   dQg' = dO S0 + dAqk' Ki,   dAqk' = lower(dO U^T)
//   dW   = -dU S0
//   dT   = dU (beta V)^T + dW (beta Kg)^T,   dM = -T^T dT T^T
//   dAkk = strictly-lower(diag(beta) dM)
//   dv   = beta (T^T dU),   dbeta_chunk = rows of (T^T dU).V + (T^T dW).Kg + dM.Akk
//   dKg  = beta (T^T dW) + dAkk Ki,   dKi = dAkk^T Kg + dAqk'^T Qg'
//   dg_c = -dKt Kt + dKg Kg - dKi Ki + dQg' Qg'   (per token and channel)
//   dgC  = sum_v dS * S0 * exp(gC) + sum_c dKt Kt   (added at the last token)
//   dlam = reverse cumulative sum of dg over the chunk's tokens, plus dgC
//
// then the prologue's chain rule (gate sigmoid, beta sigmoid, L2 norms).
//
// Work split.  One workgroup (4 waves) owns one (sequence, value head) task
// and walks its chunks from last to first; wave w owns state channels
// k in [32w, 32w+32), holding dS as 16x16 frags with v along the MFMA
// accumulator rows (lane (gq, k) holds dS[16vb + 4gq + i][16kb + k]).  In that
// layout every product that contracts over v (dKt, dQg', dW, dgC) is local to
// the wave; the one product that contracts over k (dU = Kt dS^T) is formed
// per wave over its channels and reduced through LDS.  The chunk-start state,
// U, T, Akk and Aqk' come from the records the state rebuild wrote.
//
// Precision.  Every product uses BF16 operands with FP32 accumulation except
// the two pairs whose contributions to dg cancel exactly for every token pair
// on the same side of t in the reverse cumulative sum: dAqk' Ki and
// dAqk'^T Qg' (three-product hi/lo splits, FP32-accurate), and dAkk Ki and
// dAkk^T Kg (Ki and Kg as hi/lo pairs against the same BF16 dAkk, so that
// the two terms of each pair are the same product).  With single BF16
// operands the uncancelled rounding residue dominates dlam, the more so the
// weaker the decay (Akk's entries are then O(1)).  W = Tb Kg takes Kg's lo
// part as well.
#include <type_traits>

#include "kda_chunk.hpp"

namespace kda {

namespace {

constexpr int BW_THREADS = 256;
constexpr float LN2 = 0.6931471805599453f;

// Record layouts (per record = (chunk, value head); per pair record =
// (pair of chunks 2p, 2p+1, value head)); see the state rebuild.
constexpr int REC_S0 = D * D;       // bf16 per pair: [8 kb][8 vb][64 lanes][4], chunk 2p's S0
constexpr int REC_X = REC_X_ELEMS;  // bf16 per pair: CF(U) [8 vb][64][4], CF(Kt) [8 kb][64][4]
                                    // of chunk 2p, then exp(gC) [128] as FP32
constexpr int REC_U = CH * D;       // bf16: [8 vb][64 lanes][4], RF(U)
constexpr int REC_TA = 3 * CH * CH; // f32:  T^T, Akk^T, Aqk'

struct BwdLds {
    alignas(16) float lam[CH][D];     // log2-domain decays, then their in-chunk prefix sums
    alignas(16) float gamc[D];        // exp(gC) per channel
    alignas(16) float dtz[D];         // dt_bias * exp(A_log) * log2(e)
    alignas(16) float beta[2][CH];    // by chunk parity: the next chunk's are formed
    alignas(16) float rqn[2][CH];     // during this one's last phase; 1/|q| and 1/|k|
    alignas(16) float rkn[2][CH];     // per token (0 past the end)
    alignas(16) float dba[CH];        // dbeta contribution of dM.Akk
    alignas(16) float ta[3][CH][CH];  // T^T, Akk^T, Aqk'
    alignas(16) float dgc[D];         // dgC from the state part, per channel
    alignas(16) float dbp[2][4][CH];  // per-wave dbeta partials (V part, Kg part)
    alignas(16) float dots[4][2][CH]; // per-wave partial row dots qn.dqn, kn.dkn
    alignas(16) bf16 cf_qh[8 * FS];   // CF(Qg') hi / lo
    alignas(16) bf16 cf_ql[8 * FS];
    alignas(16) bf16 cf_kg[8 * FS];   // CF(Kg) hi / lo
    alignas(16) bf16 cf_kgl[8 * FS];
    alignas(16) bf16 cf_kih[8 * FS];  // CF(Ki) hi / lo
    alignas(16) bf16 cf_kil[8 * FS];
    alignas(16) bf16 rf_kt[8 * FS];   // RF(Kt)
    alignas(16) bf16 rf_kg[8 * FS];   // RF(Kg)
    alignas(16) bf16 rf_du[8 * FS];   // RF(dU), CF(dU)
    alignas(16) bf16 cf_du[8 * FS];
    // dU partials: part[dst wave][slot][2 v-blocks][64 lanes] (slot 0..2 =
    // the three other source waves); afterwards the dT partials [4][16][16]
    alignas(16) f32x4 part[4][3][2][64];
};

// Sum over the 4 lane rows (gq) of a wave, broadcast to all rows.  A swap of
// rows 2p <-> 2p+1 (then of halves) returns each lane's own value in one
// result and its partner's in the other, so their sum is the pair sum.
__device__ __forceinline__ float xor_sum_gq(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Inclusive suffix sum over the 16 lanes of each row (lane c gets sum of
// lanes c..15 of its row): DPP row shifts toward lower lanes, zero-filled
// (bound_ctrl: a lane with no source reads 0, which also lets the compiler
// fold each shift into its add).
__device__ __forceinline__ float row16_suffix(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x101, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x102, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x104, 0xF, 0xF, true));
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x108, 0xF, 0xF, true));
    return x;
}

__device__ __forceinline__ f32x4 ld4f(const float* p) {
    const float4 x = *(const float4*)p;
    return f32x4{x.x, x.y, x.z, x.w};
}

// x ~= a * b with FP32-accurate operands: three products of hi/lo pairs.
__device__ __forceinline__ f32x4 mma16_split(bf16x4 ah, bf16x4 al, bf16x4 bh, bf16x4 bl, f32x4 c) {
    c = mma16(ah, bh, c);
    c = mma16(ah, bl, c);
    return mma16(al, bh, c);
}

}  // namespace

// kSeg: the segment-parallel passes (b.seg_pass 1 or 2), a separate instance
// so that the whole-task one keeps its code.  kPairs: pair records (the
// start states of even chunks only; b.f.rec_pairs), also an instance of its
// own, since forming the odd chunks' states costs the other one registers.
template <bool kSeg, bool kPairs>
__global__ __launch_bounds__(BW_THREADS, 2) void bwd_chunk_kernel(BwdArgs b) {
    __shared__ BwdLds sm;
    const FwdArgs& a = b.f;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: scalar registers

    int n, h, seg = 0, code;
    int64_t segidx = 0;
    if constexpr (kSeg) {  // item = segment list index * Hv + h
        const int sidx = blockIdx.x / a.Hv;
        h = blockIdx.x - sidx * a.Hv;
        n = a.plan.task[2 * sidx];
        seg = a.plan.task[2 * sidx + 1];
        segidx = a.plan.tape_off[n] + n + seg;
        code = (int)segidx * a.Hv + h;  // parameter-partial slot
    } else {
        code = a.plan.task[xcd_order(blockIdx.x, a.num_tasks, a.G)];
        n = code / a.Hv;
        h = code - n * a.Hv;
    }
    const int hq = h / a.G;
    const int64_t tok0 = a.plan.seq_start[n];
    const int L = a.plan.seq_len[n];
    const int64_t slab = ((int64_t)n * a.Hv + h) * D * D;
    const int64_t rec0 = a.plan.chunk_off[n];
    const int nchunks = (L + CH - 1) / CH;
    const int nfull = L / CH;
    // chunks [cb, ce): the whole task, or one tape segment
    int cb = 0, ce = nchunks;
    if constexpr (kSeg) {
        cb = seg * (a.ck_every / CH);
        ce = min(cb + a.ck_every / CH, nchunks);
    }
    const bool last_seg = ce == nchunks;
    const float eA = __expf(a.A_log[h]);
    const float zs = eA * LOG2E;
    const float scale = a.scale;
    // Per-task base pointers (uniform, so they live in scalar registers) and
    // per-token element strides: a token inside the sequence is then a 32-bit
    // row offset (the host rejects sequences spanning 2^31 elements or more).
    const unsigned sq = (unsigned)(a.Hqk * D), sv = (unsigned)(a.Hv * D), sb = (unsigned)a.Hv;
    const int64_t qk0 = (tok0 * a.Hqk + hq) * D, vh0 = (tok0 * a.Hv + h) * D, bh0 = tok0 * a.Hv + h;
    const bf16* const qp = (const bf16*)a.q + qk0;
    const bf16* const kp = (const bf16*)a.k + qk0;
    const bf16* const gp = (const bf16*)a.g + vh0;
    const bf16* const vp0 = (const bf16*)a.v + vh0;
    const bf16* const dop0 = (const bf16*)b.d_o + vh0;
    const bf16* const betap = (const bf16*)a.beta + bh0;
    bf16* const dvp = (bf16*)b.dv + vh0;
    bf16* const dgp = (bf16*)b.dg + vh0;
    bf16* const dqp = (bf16*)b.dq + qk0;
    bf16* const dkp = (bf16*)b.dk + qk0;
    bf16* const dbetap = (bf16*)b.dbeta + bh0;
    bf16* const dqkp = b.dqk_part != nullptr ? (bf16*)b.dqk_part + vh0 * 2 : nullptr;
    // one token row (8 channels at c8) of q, k, g and its beta logit
    auto load_row = [&](RowIn& x, int t, int c8) __attribute__((always_inline)) {
        const unsigned oq = __umul24((unsigned)t, sq) + c8;
        x.q = *(const bf16x8*)at(qp, oq);
        x.k = *(const bf16x8*)at(kp, oq);
        x.g = *(const bf16x8*)at(gp, __umul24((unsigned)t, sv) + c8);
        x.b = *at(betap, __umul24((unsigned)t, sb));
    };

    // dS frags: dS[vb][j] for kb = 2*wave + j, lane (gq, k) holds
    // dS[16vb + 4gq + i][16kb + k]; starts at dfinal_state (the last segment),
    // zero (pass 1) or the chained segment end (pass 2)
    const float* ds_src = b.dfinal + slab;
    bool ds_zero = false;
    if constexpr (kSeg) {
        if (b.seg_pass == 2 && !last_seg) ds_src = b.seg_e + (segidx * a.Hv + h) * (int64_t)D * D;
        ds_zero = b.seg_pass == 1;
    }
    f32x4 dS[8][2];
    {
        // addresses from an opaque copy of the thread id: the epilogue's
        // dinitial_state stores use the same addresses, and the compiler
        // would otherwise keep all 64 of them alive (spilled) through the loop
        int tix = tid;
        asm volatile("" : "+v"(tix));
        const int lane = tix & 63, gq = lane >> 4, cl = lane & 15;
#pragma unroll
        for (int vb = 0; vb < 8; ++vb)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    dS[vb][j][i] = ds_zero ? 0.f : ds_src[(int64_t)(16 * vb + 4 * gq + i) * D + 16 * (2 * wave + j) + cl];
    }
    if (tid < D) sm.dtz[tid] = a.dt_bias[h * D + tid] * zs;
    float ddt_acc[2][4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int i = 0; i < 4; ++i) ddt_acc[j][i] = 0.f;
    float dA_acc = 0.f;

    RowIn cur;
    load_row(cur, min((ce - 1) * CH + (tid >> 4), L - 1), (tid & 15) * 8);
    __syncthreads();
    // ---- P1 of chunk ci: norms, gate, beta (row-owner mapping) from the
    // rows in `cur`.  Run for chunk ci-1 in chunk ci's last phase (it writes
    // only lam, which that phase no longer reads, and the other parity's
    // beta and norms), and for the first chunk before the loop. ----
    auto p1 = [&](const int ci) __attribute__((always_inline)) {
        int tix = tid;
        asm volatile("" : "+v"(tix));
        const int r = tix >> 4;
        const int c8 = (tix & 15) * 8;
        const bool valid_r = r < L - ci * CH;
        {
            float sq = 0.f, sk = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {  // BF16 pair dot products, FP32 sums
                const bf16x2 q2 = {cur.q[i], cur.q[i + 1]}, k2 = {cur.k[i], cur.k[i + 1]};
                sq = __builtin_amdgcn_fdot2_f32_bf16(q2, q2, sq, false);
                sk = __builtin_amdgcn_fdot2_f32_bf16(k2, k2, sk, false);
            }
            sq = row16_sum(sq);
            sk = row16_sum(sk);
            float lv[8], dz[8];
            *(float4*)&dz[0] = *(const float4*)&sm.dtz[c8];
            *(float4*)&dz[4] = *(const float4*)&sm.dtz[c8 + 4];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float e = __builtin_amdgcn_exp2f(-((float)cur.g[i] * zs + dz[i]));
                lv[i] = valid_r ? (-5.0f * LOG2E) * __builtin_amdgcn_rcpf(1.0f + e) : 0.f;
            }
            *(float4*)&sm.lam[r][c8] = make_float4(lv[0], lv[1], lv[2], lv[3]);
            *(float4*)&sm.lam[r][c8 + 4] = make_float4(lv[4], lv[5], lv[6], lv[7]);
            if ((tix & 15) == 0) {
                sm.beta[ci & 1][r] = valid_r ? sigmoidf_((float)cur.b) : 0.f;
                sm.rqn[ci & 1][r] = valid_r ? fast_rsqrt(sq + 1e-6f) : 0.f;
                sm.rkn[ci & 1][r] = valid_r ? fast_rsqrt(sk + 1e-6f) : 0.f;
            }
        }
    };
    p1(ce - 1);
    __syncthreads();

    auto chunk = [&](const int ci, auto tail_tag) __attribute__((always_inline)) {
        constexpr bool kTail = decltype(tail_tag)::value;
        int tix = tid;
        asm volatile("" : "+v"(tix));
        const int lane = tix & 63;
        const int gq = lane >> 4;
        const int cl = lane & 15;
        const int r = tix >> 4;
        const int c8 = (tix & 15) * 8;
        const int t0 = ci * CH;
        const int nv = kTail ? L - t0 : CH;
        const bool valid_r = !kTail || r < nv;
        const bool valid_c = !kTail || cl < nv;
        const int64_t rec = (rec0 + ci) * a.Hv + h;
        // with pair records (chunks 2p, 2p+1; rec0 is even) the pair holds
        // chunk 2p's start state, and an odd chunk steps it forward by chunk
        // 2p's update; otherwise every chunk holds its own
        const int64_t prec = kPairs ? ((rec0 + ci) >> 1) * a.Hv + h : rec;
        const bool odd = kPairs && (ci & 1) != 0;
        const int kb0 = 2 * wave;

        // Global operands of the state-side products, issued in the prologue
        // so that their latency hides behind it: this wave's chunk-start
        // state frags, RF(U) and RF(dO) (zero past the end); S0 and dO stay
        // in registers until the state update.
        const unsigned tc = (unsigned)(t0 + (kTail ? min(cl, nv - 1) : cl));  // RF row token
        const unsigned ov = __umul24(tc, sv), oq = __umul24(tc, sq);          // its row offsets
        // the chunk's T^T, Akk^T, Aqk' record first (its LDS copy is made at
        // the end of the prologue; loads complete in issue order)
        float4 ta4 = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tix < REC_TA / 4) ta4 = *(const float4*)at(a.rec_ta + rec * REC_TA, 4 * tix);
        bf16x4 s0f[8][2], ru[8], rdo[8];

        // The state-side loads are spread over the chunk's first two phases
        // (a wave's loads queue at the memory pipeline and would otherwise
        // hold back the in-order issue of later work).  The chunk's P1 ran in
        // the previous chunk's last phase; its barrier published it.
        {
            const bf16* s0p = (const bf16*)a.rec_s0 + prec * REC_S0;  // uniform record base
#pragma unroll
            for (int vb = 0; vb < 8; ++vb)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    s0f[vb][j] = *(const bf16x4*)at(s0p, ((kb0 + j) * 8 + vb) * 256 + lane * 4);
        }
        // odd chunk: chunk 2p's CF(U), this wave's CF(Kt) blocks and exp(gC)
        bf16x4 xu[8], xk[2];
        float xg[2];
        if (odd) {
            const bf16* xp = (const bf16*)a.rec_x + prec * REC_X;
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) xu[vb] = *(const bf16x4*)at(xp, vb * 256 + lane * 4);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                xk[j] = *(const bf16x4*)at(xp, 2048 + (kb0 + j) * 256 + lane * 4);
                xg[j] = *(const float*)at(xp, 4096 + 2 * (16 * (kb0 + j) + cl));
            }
        }
        // ---- P2: prefix sums over the chunk's tokens.  Every wave takes 32
        // channels: lanes 0-31 sum rows 0-7, lanes 32-63 rows 8-15 and add the
        // lower half's total, swapped across the wave's halves. ----
        {
            const int ch = 32 * wave + (lane & 31);
            const bool upper = lane >= 32;
            const int r0 = upper ? 8 : 0;
            float x[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = sm.lam[r0 + i][ch];
#pragma unroll
            for (int i = 1; i < 8; ++i) x[i] += x[i - 1];
            // upper lanes receive the lower half's total in [0], lower lanes
            // the upper half's in [1]
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[7]), __float_as_uint(x[7]),
                                                             false, false);
            const float other = __uint_as_float(upper ? sw[0] : sw[1]);
            const float off = upper ? other : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) sm.lam[r0 + i][ch] = x[i] + off;
            // both halves hold the chunk total: the pair stores the same value
            sm.gamc[ch] = __builtin_amdgcn_exp2f(x[7] + other);
        }
        {
            const bf16* up = (const bf16*)a.rec_u + rec * REC_U;
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) {
                ru[vb] = *(const bf16x4*)at(up, vb * 256 + lane * 4);
                rdo[vb] = *(const bf16x4*)at(dop0, ov + 16 * vb + 4 * gq);
            }
        }
        __syncthreads();
        // ---- P3: the chunk's operands into LDS ----
        {
            float gc[8], gC[8];
            *(float4*)&gc[0] = *(const float4*)&sm.lam[r][c8];
            *(float4*)&gc[4] = *(const float4*)&sm.lam[r][c8 + 4];
            *(float4*)&gC[0] = *(const float4*)&sm.gamc[c8];
            *(float4*)&gC[4] = *(const float4*)&sm.gamc[c8 + 4];
            const float rq = sm.rqn[ci & 1][r] * scale;
            const float rk = sm.rkn[ci & 1][r];
            bf16x4 qh4[2], ql4[2], kg4[2], kgh4[2], kgl4[2], kih4[2], kil4[2], kt4[2];
#pragma unroll
            for (int s4 = 0; s4 < 2; ++s4) {
                f32x4 qg, kg, ki, kt;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int i = 4 * s4 + j;
                    const float qn = (float)cur.q[i] * rq;
                    const float kn = (float)cur.k[i] * rk;
                    const float gam = __builtin_amdgcn_exp2f(gc[i]);
                    const float gin = __builtin_amdgcn_exp2f(-gc[i]);
                    qg[j] = qn * gam;
                    kg[j] = kn * gam;
                    ki[j] = kn * gin;
                    kt[j] = ki[j] * gC[i];
                }
                // rounded hi: the dS update uses it alone (a truncated hi
                // would shrink dO^T Qg' by 2^-10 on average, and the shrink
                // accumulates in dS as long as the decay keeps it)
                split4_rne(qg, qh4[s4], ql4[s4]);
                kg4[s4] = to_bf4(kg);
                split4(kg, kgh4[s4], kgl4[s4]);
                split4(ki, kih4[s4], kil4[s4]);
                kt4[s4] = to_bf4(kt);
            }
            const int orf = rf_off(r, c8);
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                *(bf16x4*)&sm.rf_kt[orf + 64 * s] = kt4[s];
                *(bf16x4*)&sm.rf_kg[orf + 64 * s] = kg4[s];
            }
            store_cf16(sm.cf_qh, r, c8, qh4[0], qh4[1]);
            store_cf16(sm.cf_ql, r, c8, ql4[0], ql4[1]);
            store_cf16(sm.cf_kg, r, c8, kgh4[0], kgh4[1]);
            store_cf16(sm.cf_kgl, r, c8, kgl4[0], kgl4[1]);
            store_cf16(sm.cf_kih, r, c8, kih4[0], kih4[1]);
            store_cf16(sm.cf_kil, r, c8, kil4[0], kil4[1]);
        }
        if (tix < REC_TA / 4) ((float4*)&sm.ta[0][0][0])[tix] = ta4;
        // the row inputs are dead: fetch the previous chunk's
        load_row(cur, max(t0 - CH + r, 0), c8);
        // odd chunk: its start state from chunk 2p's, S0 = S0(2p)
        // diag(exp(gC(2p))) + U(2p)^T Kt(2p), frag by frag in the layout of s0f
        // (A = CF(U) frag vb, B = CF(Kt) block kb0 + j); after the prologue,
        // so that its loads have arrived
        if (odd) {
#pragma unroll
            for (int vg = 0; vg < 8; vg += 2) {
                f32x4 c[2][2];
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
#pragma unroll
                        for (int i = 0; i < 4; ++i) c[e][j][i] = (float)s0f[vg + e][j][i] * xg[j];
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int j = 0; j < 2; ++j) c[e][j] = mma16(xu[vg + e], xk[j], c[e][j]);
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int j = 0; j < 2; ++j) s0f[vg + e][j] = to_bf4(c[e][j]);
            }
        }
        __syncthreads();

        // ---- M1 (per wave): state-side products with the incoming dS ----
        const bf16x4 ident = identity_frag(lane);
        if (kTail && !valid_c) {
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) rdo[vb] = to_bf4(zero4());
        }
        f32x4 dKtT[2] = {zero4(), zero4()};  // RF orientation: lane (gq, c) holds X[c][16kb + 4gq + i]
        f32x4 dQgT[2] = {zero4(), zero4()};
        f32x4 duOwn[2];
        f32x4 daq = zero4();  // dO U^T: lane (gq, j) holds (dO U^T)[4gq + i][j]
        {
            const bf16x8 kt8 = cat8(ld4(&sm.rf_kt[kb0 * FS], lane), ld4(&sm.rf_kt[(kb0 + 1) * FS], lane));
            float dgcacc[2] = {0.f, 0.f};
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                bf16x4 dsb[2][2];
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const int vb = 2 * p + e;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        dsb[e][j] = to_bf4(dS[vb][j]);
                        // sum over v of dS * S0 as BF16 pair dot products
                        const bf16x4 d = dsb[e][j], z = s0f[vb][j];
                        dgcacc[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(d, d, 0, 1),
                                                                    __builtin_shufflevector(z, z, 0, 1),
                                                                    dgcacc[j], false);
                        dgcacc[j] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(d, d, 2, 3),
                                                                    __builtin_shufflevector(z, z, 2, 3),
                                                                    dgcacc[j], false);
                    }
                    // dU over this wave's channels (RF orientation): A = dS with
                    // k along the rows (transposed frags), B = RF(Kt)
                    const bf16x4 t0b = to_bf4(transpose_frag(dsb[e][0], ident));
                    const bf16x4 t1b = to_bf4(transpose_frag(dsb[e][1], ident));
                    const f32x4 du = mma32(cat8(t0b, t1b), kt8, zero4());
                    const int dst = vb >> 1;
                    if (dst == wave) {
                        duOwn[e] = du;
                    } else {
                        sm.part[dst][(wave - dst - 1) & 3][e][lane] = du;
                    }
                }
                // dKt^T = dS^T U^T and dQg'^T = S0^T dO^T, contracting over v
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    dKtT[j] = mma32(cat8(dsb[0][j], dsb[1][j]), cat8(ru[2 * p], ru[2 * p + 1]), dKtT[j]);
                    dQgT[j] = mma32(cat8(s0f[2 * p][j], s0f[2 * p + 1][j]), cat8(rdo[2 * p], rdo[2 * p + 1]), dQgT[j]);
                }
                daq = mma32(cat8(rdo[2 * p], rdo[2 * p + 1]), cat8(ru[2 * p], ru[2 * p + 1]), daq);
            }
            // dgC from the state: sum over v of dS * S0, times exp(gC)
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float acc = xor_sum_gq(dgcacc[j]);
                const int k = 16 * (kb0 + j) + cl;
                if (gq == 0) sm.dgc[k] = acc * sm.gamc[k];
            }
        }
        // dAqk' = lower(dO U^T): lane (gq, j) holds dAqk'[4gq + i][j]
        bf16x4 daqh, daql, daqTh, daqTl;
        {
#pragma unroll
            for (int i = 0; i < 4; ++i) daq[i] = (4 * gq + i >= cl) ? daq[i] : 0.f;
            split4(daq, daqh, daql);
            // transposed (exactly, part by part): lane (gq, c) holds dAqk'[c][4gq + i]
            daqTh = to_bf4(transpose_frag(daqh, ident));
            daqTl = to_bf4(transpose_frag(daql, ident));
        }
        __syncthreads();

        // ---- R1 (per wave): finish dU for v-blocks 2w, 2w+1 ----
        // V for this phase and raw q, k, g for the per-channel gradients
        // (issued here, used after the dU reduction and two barriers later)
        bf16x4 vv[2], qraw[2], kraw[2], graw[2];
        {
            vv[0] = *(const bf16x4*)at(vp0, ov + 32 * wave + 4 * gq);
            vv[1] = *(const bf16x4*)at(vp0, ov + 32 * wave + 16 + 4 * gq);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                qraw[j] = *(const bf16x4*)at(qp, oq + 16 * (kb0 + j) + 4 * gq);
                kraw[j] = *(const bf16x4*)at(kp, oq + 16 * (kb0 + j) + 4 * gq);
                graw[j] = *(const bf16x4*)at(gp, ov + 16 * (kb0 + j) + 4 * gq);
            }
        }
        const f32x4 tB = ld4f(&sm.ta[0][cl][4 * gq]);  // frag(T): lane (gq, c) holds T[4gq+i][c]
        const bf16x4 tBb = to_bf4(tB);
        f32x4 dT;  // lane (gq, j) holds dT[4gq + i][j] (partial)
        {
            // frag(Aqk'): lane (gq, c) holds Aqk'[4gq + i][c]
            f32x4 aqB;
#pragma unroll
            for (int i = 0; i < 4; ++i) aqB[i] = sm.ta[2][4 * gq + i][cl];
            const bf16x4 aqBb = to_bf4(aqB);
            bf16x4 rfdu[2], bv[2];
            float dbv = 0.f;
#pragma unroll
            for (int jj = 0; jj < 2; ++jj) {
                const int vbo = 2 * wave + jj;
                f32x4 du = duOwn[jj];
#pragma unroll
                for (int s = 0; s < 3; ++s) du += sm.part[wave][s][jj][lane];
                bf16x4 rdv = rdo[0];  // RF(dO)[vbo], picked without dynamic indexing
#pragma unroll
                for (int v = 1; v < 8; ++v)
                    if (v == vbo) rdv = rdo[v];
                const bf16x4 cfdo = to_bf4(transpose_frag(rdv, ident));
                du = mma16(cfdo, aqBb, du);  // + Aqk'^T dO
                rfdu[jj] = to_bf4(du);
                const bf16x4 cfdu = to_bf4(transpose_frag(rfdu[jj], ident));
                *(bf16x4*)&sm.rf_du[vbo * FS + lane * 4] = rfdu[jj];
                *(bf16x4*)&sm.cf_du[vbo * FS + lane * 4] = cfdu;
                // dBv^T = dU^T T (RF orientation): lane (gq, c) holds (T^T dU)[c][16vbo + 4gq + i]
                const f32x4 dbvT = mma16(cfdu, tBb, zero4());
                const float bc = sm.beta[ci & 1][cl];
                const f32x4 vvf = from_bf4(vv[jj]);
                if (valid_c)
                    *(bf16x4*)at(dvp, ov + 16 * vbo + 4 * gq) = to_bf4(dbvT * bc);
#pragma unroll
                for (int i = 0; i < 4; ++i) dbv += dbvT[i] * vvf[i];
                bv[jj] = to_bf4(vvf * bc);  // RF(beta V): lane (gq, j) holds beta_j V[j][..]
            }
            dbv = xor_sum_gq(dbv);
            if (gq == 0) sm.dbp[0][wave][cl] = dbv;
            // dT += dU (beta V)^T over this wave's value columns
            dT = mma32(cat8(rfdu[0], rfdu[1]), cat8(bv[0], bv[1]), zero4());
        }
        __syncthreads();

        // ---- M4 (per wave): dW, dT, dKg part, dS update ----
        f32x4 dKgT[2];
        {
            bf16x4 rfduA[8];
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) rfduA[vb] = ld4(&sm.rf_du[vb * FS], lane);
            bf16x4 dWb[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                f32x4 x = zero4();
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const bf16x8 s8 = cat8(s0f[2 * p][j], s0f[2 * p + 1][j]);
                    x = mma32(s8, cat8(rfduA[2 * p], rfduA[2 * p + 1]), x);
                }
                dWb[j] = to_bf4_neg(x);  // RF(dW): lane (gq, c) holds dW[c][16kb + 4gq + i]
            }
            // dT += dW (beta Kg)^T over this wave's channels
            bf16x4 bk[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) bk[j] = to_bf4(from_bf4(ld4(&sm.rf_kg[(kb0 + j) * FS], lane)) * sm.beta[ci & 1][cl]);
            dT = mma32(cat8(dWb[0], dWb[1]), cat8(bk[0], bk[1]), dT);
            float* dTp = (float*)&sm.part[0][0][0][0];  // [4 waves][16 c][16 j]
#pragma unroll
            for (int i = 0; i < 4; ++i) dTp[wave * 256 + (4 * gq + i) * 16 + cl] = dT[i];
            // dBk^T = dW^T T; dKg = beta dBk; dbeta part sum_k dBk Kg
            float dbk = 0.f;
            f32x4 wcf[2];
            f32x4 tbA;  // frag(Tb^T): lane (gq, c) holds T[c][4gq+i] beta_{4gq+i}
#pragma unroll
            for (int i = 0; i < 4; ++i) tbA[i] = sm.ta[0][4 * gq + i][cl] * sm.beta[ci & 1][4 * gq + i];
            const bf16x4 tbAb = to_bf4(tbA);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x4 cfdw = to_bf4(transpose_frag(dWb[j], ident));
                const f32x4 dbkT = mma16(cfdw, tBb, zero4());
                const f32x4 kgr = from_bf4(ld4(&sm.rf_kg[(kb0 + j) * FS], lane));
#pragma unroll
                for (int i = 0; i < 4; ++i) dbk += dbkT[i] * kgr[i];
                dKgT[j] = dbkT * sm.beta[ci & 1][cl];
                // W = Tb Kg (CF): lane (gq, k) holds W[4gq + i][k]
                wcf[j] = mma16(tbAb, ld4(&sm.cf_kgl[(kb0 + j) * FS], lane),
                               mma16(tbAb, ld4(&sm.cf_kg[(kb0 + j) * FS], lane), zero4()));
            }
            dbk = xor_sum_gq(dbk);
            if (gq == 0) sm.dbp[1][wave][cl] = dbk;
            // dS <- dS exp(gC) + dO^T Qg' - dU^T W
            bf16x4 nw[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) nw[j] = to_bf4_neg(wcf[j]);
#pragma unroll
            for (int vb = 0; vb < 8; ++vb) {
                const bf16x4 cfdo = to_bf4(transpose_frag(rdo[vb], ident));
                const bf16x4 cfdu = ld4(&sm.cf_du[vb * FS], lane);
                const bf16x8 a8 = cat8(cfdo, cfdu);
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float ec = sm.gamc[16 * (kb0 + j) + cl];
                    const bf16x8 b8 = cat8(ld4(&sm.cf_qh[(kb0 + j) * FS], lane), nw[j]);
                    dS[vb][j] = mma32(a8, b8, dS[vb][j] * ec);
                }
            }
        }
        __syncthreads();

        // ---- A1 (per wave): dM, dAkk and the per-channel gradients ----
        f32x4 dKiT[2];
        {
            const float* dTp = (const float*)&sm.part[0][0][0][0];
            f32x4 dTa = zero4();  // frag(dT^T): lane (gq, c) holds dT[c][4gq + i]
#pragma unroll
            for (int w = 0; w < 4; ++w) dTa += ld4f(&dTp[w * 256 + cl * 16 + 4 * gq]);
            f32x4 tTB;  // frag(T^T): lane (gq, b) holds T[b][4gq + i]
#pragma unroll
            for (int i = 0; i < 4; ++i) tTB[i] = sm.ta[0][4 * gq + i][cl];
            const f32x4 P = mma16(to_bf4(dTa), to_bf4(tTB), zero4());  // P = dT T^T
            const f32x4 dM = -mma16(tBb, to_bf4(P), zero4());            // lane (gq, b): dM[4gq + i][b]
            const f32x4 akk = ld4f(&sm.ta[1][cl][4 * gq]);               // Akk[4gq + i][b]
            f32x4 dAkk;
            float dba[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                dAkk[i] = (4 * gq + i > cl) ? sm.beta[ci & 1][4 * gq + i] * dM[i] : 0.f;
                dba[i] = row16_sum(dM[i] * akk[i]);
            }
            if (wave == 0 && cl == 0) {
#pragma unroll
                for (int i = 0; i < 4; ++i) sm.dba[4 * gq + i] = dba[i];
            }
            const bf16x4 dAkkB = to_bf4(dAkk);                              // lane (gq, j): dAkk[4gq+i][j]
            const bf16x4 dAkkT = to_bf4(transpose_frag(dAkkB, ident));     // lane (gq, c): dAkk[c][4gq+i]
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const bf16x4 kih = ld4(&sm.cf_kih[(kb0 + j) * FS], lane);
                const bf16x4 kil = ld4(&sm.cf_kil[(kb0 + j) * FS], lane);
                const bf16x4 qh = ld4(&sm.cf_qh[(kb0 + j) * FS], lane);
                const bf16x4 ql = ld4(&sm.cf_ql[(kb0 + j) * FS], lane);
                dKgT[j] = mma16(kil, dAkkT, mma16(kih, dAkkT, dKgT[j]));  // + dAkk Ki
                // dAkk^T Kg with Kg as a hi/lo pair: its dg terms cancel those of
                // dAkk Ki (Ki hi/lo) pair by pair in the reverse sum
                f32x4 x = mma16(ld4(&sm.cf_kgl[(kb0 + j) * FS], lane), dAkkB,
                                mma16(ld4(&sm.cf_kg[(kb0 + j) * FS], lane), dAkkB, zero4()));
                dKiT[j] = mma16_split(qh, ql, daqh, daql, x);             // + dAqk'^T Qg'
                dQgT[j] = mma16_split(kih, kil, daqTh, daqTl, dQgT[j]);   // + dAqk' Ki
            }
        }
        // per-element gradients (lane (gq, c), channels k = 16kb + 4gq + i)
        f32x4 qn4[2], kn4[2], dqn4[2], dkn4[2], dlam4[2], zl4[2];
        {
            const float rq = sm.rqn[ci & 1][cl], rk = sm.rkn[ci & 1][cl];
            float dotq = 0.f, dotk = 0.f;
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int kbase = 16 * (kb0 + j) + 4 * gq;
                const f32x4 qr = from_bf4(qraw[j]);
                const f32x4 kr = from_bf4(kraw[j]);
                const f32x4 gr = from_bf4(graw[j]);
                const f32x4 gc = ld4f(&sm.lam[cl][kbase]);
                const f32x4 gC = ld4f(&sm.gamc[kbase]);
                const f32x4 dz4 = ld4f(&sm.dtz[kbase]);
                f32x4 dge, ktkt;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    // with Kg = kn G, Ki = kn Gi, Kt = kn et and Qg' = scale qn G:
                    //   dg_c = kn (dKg G - dKi Gi - dKt et) + qn dqn,  dqn = scale G dQg'
                    const float qn = qr[i] * rq, kn = kr[i] * rk;
                    const float G = __builtin_amdgcn_exp2f(gc[i]);
                    const float Gi = __builtin_amdgcn_exp2f(-gc[i]);
                    const float et = gC[i] * Gi;
                    const float ta = dKtT[j][i] * et, tb = dKgT[j][i] * G, tc = dKiT[j][i] * Gi;
                    dkn4[j][i] = ta + tb + tc;
                    dqn4[j][i] = (scale * dQgT[j][i]) * G;
                    const float pq = qn * dqn4[j][i];
                    dge[i] = kn * (tb - ta - tc) + pq;
                    ktkt[i] = kn * ta;
                    qn4[j][i] = qn;
                    kn4[j][i] = kn;
                    zl4[j][i] = gr[i] * zs + dz4[i];
                    dotq += pq;
                    dotk += kn * dkn4[j][i];
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float dgC = sm.dgc[kbase + i] + row16_sum(ktkt[i]);
                    dlam4[j][i] = row16_suffix(dge[i]) + dgC;
                }
            }
            dotq = xor_sum_gq(dotq);
            dotk = xor_sum_gq(dotk);
            if (gq == 0) {
                sm.dots[wave][0][cl] = dotq;
                sm.dots[wave][1][cl] = dotk;
            }
        }
        __syncthreads();

        // ---- A3: prologue chain rule and stores ----
        {
            const float rq = sm.rqn[ci & 1][cl], rk = sm.rkn[ci & 1][cl];
            const float dotq = sm.dots[0][0][cl] + sm.dots[1][0][cl] + sm.dots[2][0][cl] + sm.dots[3][0][cl];
            const float dotk = sm.dots[0][1][cl] + sm.dots[1][1][cl] + sm.dots[2][1][cl] + sm.dots[3][1][cl];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int koff = 16 * (kb0 + j) + 4 * gq;
                f32x4 dgo, dq, dk;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float sg = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zl4[j][i]));
                    const float dz = -5.0f * dlam4[j][i] * sg * (1.0f - sg);
                    dgo[i] = eA * dz;
                    dq[i] = rq * (dqn4[j][i] - qn4[j][i] * dotq);
                    dk[i] = rk * (dkn4[j][i] - kn4[j][i] * dotk);
                    if (valid_c) {
                        ddt_acc[j][i] += dgo[i];
                        dA_acc += dz * zl4[j][i] * LN2;
                    }
                }
                if (valid_c) {
                    *(bf16x4*)at(dgp, ov + koff) = to_bf4(dgo);
                    if (dqkp == nullptr) {
                        *(bf16x4*)at(dqp, oq + koff) = to_bf4(dq);
                        *(bf16x4*)at(dkp, oq + koff) = to_bf4(dk);
                    } else {
                        bf16* pp = dqkp + 2 * ov + koff;
                        *(bf16x4*)pp = to_bf4(dq);
                        *(bf16x4*)(pp + D) = to_bf4(dk);
                    }
                }
            }
            if (wave == 0 && gq == 0 && valid_c) {
                const float db = sm.dbp[0][0][cl] + sm.dbp[0][1][cl] + sm.dbp[0][2][cl] + sm.dbp[0][3][cl] +
                                 sm.dbp[1][0][cl] + sm.dbp[1][1][cl] + sm.dbp[1][2][cl] + sm.dbp[1][3][cl] +
                                 sm.dba[cl];
                const float bt = sm.beta[ci & 1][cl];
                // dbeta on the logit: db * sigma'(x) = db * beta (1 - beta)
                *at(dbetap, __umul24(tc, sb)) = (bf16)(db * bt * (1.0f - bt));
            }
        }
        if (ci > cb) p1(ci - 1);
        __syncthreads();
    };
    if (last_seg && nfull < nchunks) chunk(nfull, std::true_type{});
    for (int ci = min(nfull, ce) - 1; ci >= cb; --ci) chunk(ci, std::false_type{});

    // dinitial_state, parameter partials
    {
        int tix = tid;
        asm volatile("" : "+v"(tix));
        const int lane = tix & 63, gq = lane >> 4, cl = lane & 15;
#pragma unroll
        for (int vb = 0; vb < 8; ++vb)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int64_t e = (int64_t)(16 * vb + 4 * gq + i) * D + 16 * (2 * wave + j) + cl;
                    if (kSeg && b.seg_pass == 1)  // R: the segment's start dS from zero
                        b.seg_r[(segidx * a.Hv + h) * (int64_t)D * D + e] = dS[vb][j][i];
                    else if (cb == 0)
                        b.dinit[slab + e] = dS[vb][j][i];
                }
        if (kSeg && b.seg_pass == 1) return;  // no parameter partials from pass 1
        float* pp = b.dparam_part + (int64_t)code * 2 * D;
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = row16_sum(ddt_acc[j][i]);
                if (cl == 0) pp[16 * (2 * wave + j) + 4 * gq + i] = x;
            }
        float x = xor_sum_gq(row16_sum(dA_acc));
        if (lane == 0) pp[D + wave] = x;
    }
}

// dA_log[h] and ddt_bias[h][:] from the per-task partials, in sequence order;
// dq, dk summed over the G value heads of each q/k head, in head order.
__global__ void bwd_param_reduce_kernel(BwdArgs b, int N) {
    const FwdArgs& a = b.f;
    const int h = blockIdx.x;
    const int k = threadIdx.x;
    float s = 0.f, sa = 0.f;
    for (int n = 0; n < N; ++n) {
        const float* pp = b.dparam_part + ((int64_t)n * a.Hv + h) * 2 * D;
        s += pp[k];
        if (k == 0) sa += (pp[D] + pp[D + 1]) + (pp[D + 2] + pp[D + 3]);
    }
    b.ddt_bias[h * D + k] = s;
    if (k == 0) b.dA_log[h] = sa;
}

__global__ void bwd_dqk_reduce_kernel(BwdArgs b, int64_t items) {
    const FwdArgs& a = b.f;
    const int64_t it = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (token, hq, which, 4-channel group)
    if (it >= items) return;
    const int grp = (int)(it % (D / 4));
    int64_t rest = it / (D / 4);
    const int which = (int)(rest % 2);
    rest /= 2;
    const int hq = (int)(rest % a.Hqk);
    const int64_t tok = rest / a.Hqk;
    f32x4 s = zero4();
    for (int g = 0; g < a.G; ++g) {
        const bf16* pp = (const bf16*)b.dqk_part + (tok * a.Hv + hq * a.G + g) * (2 * D) + which * D + 4 * grp;
        s += from_bf4(*(const bf16x4*)pp);
    }
    bf16* out = (bf16*)(which == 0 ? b.dq : b.dk);
    *(bf16x4*)(out + (tok * a.Hqk + hq) * D + 4 * grp) = to_bf4(s);
}

hipError_t launch_bwd_chunk(const BwdArgs& b, hipStream_t s) {
    if (b.f.num_tasks == 0) return hipSuccess;
    if (b.f.rec_pairs)
        hipLaunchKernelGGL((bwd_chunk_kernel<false, true>), dim3((unsigned)b.f.num_tasks), dim3(BW_THREADS), 0,
                           s, b);
    else
        hipLaunchKernelGGL((bwd_chunk_kernel<false, false>), dim3((unsigned)b.f.num_tasks), dim3(BW_THREADS), 0,
                           s, b);
    return hipGetLastError();
}

// dS_end(j-1) = dS_end(j) P(j)^T + R(j), from dfinal at the last segment, for
// 16 value rows of one task per workgroup (value rows are independent): the
// forward's combine run backward with P transposed.
__global__ __launch_bounds__(256) void seg_combine_bwd_kernel(BwdArgs b) {
    const FwdArgs& a = b.f;
    constexpr int SP = D + 1;
    __shared__ float sr[16 * SP];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, gq = lane >> 4, cl = lane & 15;
    const int rb = blockIdx.x & 7;
    const int nh = blockIdx.x >> 3;
    const int n = nh / a.Hv, h = nh - n * a.Hv;
    const int L = a.plan.seq_len[n];
    const int nseg = (L + a.ck_every - 1) / a.ck_every;
    if (nseg < 2) return;  // uniform over the workgroup: before any barrier
    const int64_t base = a.plan.tape_off[n] + n;  // segment index of segment 0
    const int64_t DD = (int64_t)D * D;
    {
        const float* df = b.dfinal + ((int64_t)n * a.Hv + h) * DD + (int64_t)(16 * rb) * D;
        for (int e = tid; e < 16 * D; e += 256) sr[(e / D) * SP + (e % D)] = df[e];
    }
    for (int j = nseg - 1; j >= 1; --j) {
        const float* P = b.seg_p + ((base + j) * a.Hv + h) * DD;
        const float* R = b.seg_r + ((base + j) * a.Hv + h) * DD;
        __syncthreads();  // rows of dS_end(j) in LDS
        f32x4 acc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = 16 * (2 * wave + t) + cl;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] = R[(int64_t)(16 * rb + 4 * gq + i) * D + col];
        }
#pragma unroll 8
        for (int kk = 0; kk < D; kk += 4) {
            const float x = sr[cl * SP + kk + gq];  // A[row cl][k = kk + gq]
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                // B[k][col] = P^T[k][col], stored row-major
                const float y = P[(int64_t)(kk + gq) * D + 16 * (2 * wave + t) + cl];
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, acc[t], 0, 0, 0);
            }
        }
        __syncthreads();  // every wave has read dS_end(j)
        float* dst = b.seg_e + ((base + j - 1) * a.Hv + h) * DD + (int64_t)(16 * rb) * D;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = 16 * (2 * wave + t) + cl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sr[(4 * gq + i) * SP + col] = acc[t][i];
                dst[(4 * gq + i) * D + col] = acc[t][i];
            }
        }
    }
}

// The segment-parallel adjoint (after the state rebuild): pass 1 over every
// segment, the chain, pass 2 over every segment.  b.f.plan.task must be the
// segment list and b.f.seg_items its length times Hv.
hipError_t launch_bwd_segments(const BwdArgs& b, int N, hipStream_t s) {
    if (b.f.seg_items == 0) return hipSuccess;
    BwdArgs p1 = b;
    p1.seg_pass = 1;
    hipLaunchKernelGGL((bwd_chunk_kernel<true, false>), dim3((unsigned)b.f.seg_items), dim3(BW_THREADS), 0, s, p1);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(seg_combine_bwd_kernel, dim3((unsigned)(N * b.f.Hv * 8)), dim3(256), 0, s, b);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    BwdArgs p2 = b;
    p2.seg_pass = 2;
    hipLaunchKernelGGL((bwd_chunk_kernel<true, false>), dim3((unsigned)b.f.seg_items), dim3(BW_THREADS), 0, s, p2);
    return hipGetLastError();
}

hipError_t launch_bwd_reduce(const BwdArgs& b, int N, hipStream_t s) {
    hipLaunchKernelGGL(bwd_param_reduce_kernel, dim3((unsigned)b.f.Hv), dim3(D), 0, s, b, N);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || b.dqk_part == nullptr) return e;
    const int64_t items = b.total_tokens * b.f.Hqk * 2 * (D / 4);
    if (items == 0) return hipSuccess;
    hipLaunchKernelGGL(bwd_dqk_reduce_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, s, b,
                       items);
    return hipGetLastError();
}

}  // namespace kda
