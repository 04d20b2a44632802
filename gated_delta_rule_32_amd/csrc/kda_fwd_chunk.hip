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
//   Tb  = (I + diag(beta) Akk)^-1 diag(beta)        (substitution)
//   Y   = Kg S0^T,   U = Tb V - Tb Y
//   O   = scale (Qg S0^T + Aqk U)
//   S_C = S0 diag(exp(gC)) + U^T Kt
//
// (U = Tb (V - Kg S0^T) is the chunk's delta-rule correction; forming Kg S0^T
// first keeps it independent of the substitution, so its MFMAs overlap it.)
// Within a chunk the log-decay sums stay above 16 * (-5) = -80, so the factors
// exp(+-gc) stay inside the FP32/BF16 exponent range (e^80 < 3.4e38).
//
// Work split.  One workgroup (4 waves) owns one (sequence, value head) task
// for its whole length; wave w owns state columns v in [32w, 32w+32), held as
// transposed 16x16 frags S^T[kb][vb] in FP32 registers.  The state path is
// column-local, so no state crosses waves.  Three barriers per chunk: at its
// start (its decay prefix sums, exp(gC) and beta are in LDS), after its shared
// operands are in LDS, and after its 16x16 algebra (Akk and the substitution
// on wave 0, Aqk on wave 1, shared through LDS).  The next chunk's norms and
// gate run inside the algebra phase, its prefix sums inside the state update.
// Shared operands sit in LDS "frag slots" (64 lanes x 4 bf16, padded):
//   RF(X)[kb]: lane (gq, c) holds X[c][16kb + 4gq + i]   (rows = tokens)
//   CF(X)[kb]: lane (gq, k) holds X[4gq + i][16kb + k]   (tokens along i)
// Products that contract over tokens take CF operands, those that contract
// over channels take RF operands.  The output is formed transposed,
// O^T = S0 Qg^T + U^T Aqk^T, whose accumulator layout gives each lane four
// consecutive channels of one token, stored straight to global memory.
//
// Precision.  The products that write new information into the carried
// state need FP32-like operands: Tb V (Tb as a BF16 hi/lo pair, V exact in
// BF16) and U^T Kt, done in FP16 as [Kt_hi|Kt_lo] [U;U] in one 16x16x32 per
// state frag (Kt lies in [0, 1] and keeps about 22 bits as an FP16 pair; U
// keeps 11; U of 16384 or more is scaled by a power of two around the
// product).  The products that predict the state (Kg S0^T, Tb Y, Akk) and the
// output use single BF16 operands: under decay the delta rule re-measures the
// state against each key and the prediction's rounding fades within a few
// tokens (final-state error 5e-5 to 3e-4 against the FP64 definition over
// 1024-4096 tokens for chunk decays up to exp(-2)).  A channel that decays
// less keeps that rounding: a chunk in which some channel keeps more than
// exp(-2) of its state ("precise") takes Kg, Ki, S0 and Y as BF16 hi/lo pairs
// too (three products each) and U as an FP16 hi/lo pair, which holds the
// final state within about 3e-5 without any decay.
#include <type_traits>

#include "kda_chunk.hpp"

namespace kda {

namespace {

constexpr int FC_THREADS = 256;
constexpr int TBS = 20;  // row stride of the per-wave Tb scratch (16-byte rows)
constexpr int FS2 = 520;  // stride of a slot that holds 8 bf16 per lane (512 + 8 padding)

struct SolveScratch {
    alignas(16) float nT[CH][CH];   // nT[m][i] = beta_i Akk[i][m] for i > m, else 0 (wave 0 only)
    alignas(16) float tb[CH][TBS];  // Tb[i][j], written by wave 0, read by all after a barrier
};

struct FwdLds {
    alignas(16) float lam[CH][D];   // log2-domain decays, then their in-chunk prefix sums
    alignas(16) float gamc[2][D];   // exp(gC) per channel, by chunk parity
    alignas(16) float dtz[D];       // dt_bias * exp(A_log) * log2(e)
    alignas(16) float beta[2][CH];  // double-buffered: a wave may start the next
                                    // chunk while another still solves with this one's
    SolveScratch sv;
    alignas(16) bf16 sh_aq[512];    // [Aqk/2 | Aqk/2] frag pair (RF16 layout), written by wave 1
    alignas(16) bf16 rf_qg[8 * FS];
    alignas(16) bf16 rf_kg[8 * FS];
    alignas(16) bf16 rf_ki[8 * FS];
    alignas(16) bf16 rf_kg_lo[8 * FS];  // precise chunks: lo parts of Kg, Ki
    alignas(16) bf16 rf_ki_lo[8 * FS];
    alignas(16) bf16 cf_kt[8 * FS2];  // CF(Kt) as [hi | lo] pairs, 8 bf16 per lane
    alignas(16) f16x4 ulo[4][2][64];  // precise chunks: each wave's FP16 lo part of U
    int precise[2];                   // by chunk parity: the chunk runs precise
};

}  // namespace

// kMode = kFwdTape: the training forward over whole tasks (o, final state, the
// FP32 state tape).  kMode = kFwdRebuild: the backward's state rebuild over one
// tape segment of one task: it starts from the segment's checkpoint, writes no
// output, and stores for every chunk the records the adjoint reads
// (chunk-start state, U, T, Akk, Aqk).  kMode = kFwdRecords: the training
// forward that stores those records for every chunk instead of the tape, so
// that the backward reruns nothing.  kMode = kFwdInfer: the inference forward
// of page "flashinfer.kda.recurrent_kda" (no tape): the state comes from a
// BF16 pool slot and goes back to it, and the prologue follows the call's
// options (L2 norm on or off, the in-kernel gate with its lower bound, beta as
// a logit or as given).  The chunk form needs every per-token log-decay at or
// above -5 (so that the factors exp(+-gc) stay in range), so the host sends
// only the in-kernel gate with lower_bound >= -5 here; log-space gates run
// token by token.
// kFwdRebuildPairs and kFwdRecordsPairs store the records with the
// chunk-start state of even chunks only, and with what steps it to the odd
// chunk after (pair records, for calls with many tasks).
// kFwdInferCkpt is the same with state checkpoints (a separate instance, so
// that the plain one keeps its registers).  kFwdSegPQ and kFwdSegOut make the
// segment-parallel training forward for calls with few tasks: each tape
// segment's end state is affine in its start state, S_out = S_in P + Q, so
// kFwdSegPQ runs every segment at once from the identity with v = 0 (giving
// P) and from zero (giving Q), a combine kernel chains S_in through the
// segments into the tape, and kFwdSegOut reruns every segment from its tape
// state for o and the final state.
constexpr int kFwdTape = 0, kFwdRebuild = 1, kFwdRecords = 2, kFwdInfer = 3, kFwdInferCkpt = 4,
              kFwdSegPQ = 5, kFwdSegOut = 6, kFwdRebuildPairs = 7, kFwdRecordsPairs = 8;

template <int kMode>
__global__ __launch_bounds__(FC_THREADS, 3) void fwd_chunk_kernel(FwdArgs a) {
    constexpr int kNVB = 2;  // 16-column blocks per wave
    constexpr bool kPairs = kMode == kFwdRebuildPairs || kMode == kFwdRecordsPairs;  // pair records
    constexpr bool kRebuild = kMode == kFwdRebuild || kMode == kFwdRebuildPairs;  // one segment, no output
    constexpr bool kSegPQ = kMode == kFwdSegPQ;
    constexpr bool kSegTask = kRebuild || kSegPQ || kMode == kFwdSegOut;  // one tape segment per task
    constexpr bool kOut = !kRebuild && !kSegPQ;      // o and the final state
    constexpr bool kRec = kRebuild || kMode == kFwdRecords || kMode == kFwdRecordsPairs;  // records
    constexpr bool kInfer = kMode == kFwdInfer || kMode == kFwdInferCkpt;  // BF16 pool state, options
    constexpr bool kCkpt = kMode == kFwdInferCkpt;   // state checkpoints
    __shared__ FwdLds sm;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;

    int n, h, seg = 0;
    // (from a scalar copy of the wave index: with the vector one the state
    // rebuild spills)
    int vb0 = 2 * __builtin_amdgcn_readfirstlane(wave);  // this wave's first 16-column block
    bool segQ = false;  // kFwdSegPQ: the second half of the grid forms Q, the first P
    if constexpr (kSegTask) {
        // item = segment index * Hv + h; the segment list holds (n, j) pairs
        int64_t item = blockIdx.x;
        if constexpr (kRebuild) item = xcd_order((int)item, (int)(gridDim.x), a.G);  // items = segments * Hv
        if constexpr (kSegPQ) {
            segQ = item >= a.seg_items;
            if (segQ) item -= a.seg_items;
        }
        const int sidx = (int)(item / a.Hv);
        h = (int)(item - (int64_t)sidx * a.Hv);
        n = a.plan.task[2 * sidx];
        seg = a.plan.task[2 * sidx + 1];
    } else {
        const int code = a.plan.task[xcd_order(blockIdx.x, a.num_tasks, a.G)];
        n = code / a.Hv;
        h = code - n * a.Hv;
    }
    const int hq = h / a.G;
    const int64_t tok0 = a.plan.seq_start[n];
    const int L = a.plan.seq_len[n];
    const int64_t slab = ((int64_t)n * a.Hv + h) * D * D;
    const int64_t tape_base = a.tape != nullptr ? a.plan.tape_off[n] : 0;
    const int nchunks = (L + CH - 1) / CH;
    const int nfull = L / CH;
    int cb = 0, ce = nchunks;
    const float* src = a.s0 + slab;
    int64_t rec0 = 0;
    if constexpr (kSegTask) {
        const int per = a.ck_every / CH;
        cb = seg * per;
        ce = min(cb + per, nchunks);
        if (!kSegPQ && seg > 0) src = a.tape + ((tape_base + seg - 1) * a.Hv + h) * (int64_t)D * D;
    }
    if constexpr (kRec) rec0 = a.plan.chunk_off[n];
    // inference: the pool slot of sequence n (checked on the host; a slot
    // out of range ends the workgroup before any access or barrier)
    bf16* pslab = nullptr;
    const bf16* pinit = nullptr;  // initial state: the source pool's slot when given
    if constexpr (kInfer) {
        const int64_t slot = a.pool_index != nullptr ? a.pool_index[n] : n;
        if (slot < 0 || slot >= a.pool_slots) return;
        pslab = (bf16*)a.pool + (slot * a.Hv + h) * (int64_t)D * D;
        pinit = pslab;
        if (a.src_pool != nullptr) {
            const int64_t ss = a.src_index[n];
            if (ss < 0 || ss >= a.src_slots) return;
            pinit = (const bf16*)a.src_pool + (ss * a.Hv + h) * (int64_t)D * D;
        }
    }

    // state: S^T frags for kb = 0..7 and the wave's column blocks vb0 + j
    f32x4 S[8][kNVB];
    {
        const int lane = tid & 63, gq = lane >> 4, cl = lane & 15;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int j = 0; j < kNVB; ++j) {
                const int vcol = 16 * (vb0 + j) + cl;
                if constexpr (kInfer) {
                    S[kb][j] = from_bf4(*(const bf16x4*)(pinit + vcol * D + 16 * kb + 4 * gq));
                } else if constexpr (kSegPQ) {
                    // P: the identity (row vcol, key 16kb + 4gq + i); Q: zero
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        S[kb][j][i] = (!segQ && vcol == 16 * kb + 4 * gq + i) ? 1.0f : 0.0f;
                } else {
                    const float4 x = *(const float4*)(src + (int64_t)vcol * D + 16 * kb + 4 * gq);
                    S[kb][j] = f32x4{x.x, x.y, x.z, x.w};
                }
            }
    }

    // prologue options (inference only; the training modes fix them)
    const bool l2norm = !kInfer || a.use_qk_l2norm != 0;
    const bool beta_logit = !kInfer || a.beta_is_logit != 0;
    const float lb2 = (kInfer ? a.lower_bound : -5.0f) * LOG2E;  // log2-domain lower bound
    const float eA = __expf(a.A_log[h]);
    // z*log2(e) = g*(eA log2e) + dt*(eA log2e); the log2-domain decay is
    // -5 log2(e) sigmoid(z)
    const float zs = eA * LOG2E;
    if (tid < D) sm.dtz[tid] = a.dt_bias != nullptr ? a.dt_bias[h * D + tid] * zs : 0.f;

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

    RowIn cur;
    ColIn vcur;
    {
        const int lane = tid & 63;
        load_rows_s(cur, sp, min(cb * CH + (tid >> 4), L - 1), (tid & 15) * 8);
        load_cols_cf<kNVB>(vcur, sp, cb * CH + 4 * (lane >> 4), L - 1, 16 * vb0 + (lane & 15));
    }
    __syncthreads();

    // ---- A: norms, gate and beta of chunk ci into LDS, 1/|q| and 1/|k| into
    // registers; rows past the end of the sequence get zero operands and no
    // decay.  Run for chunk ci+1 at the end of chunk ci's D1 phase (it
    // touches nothing that phase reads), so its arithmetic overlaps the
    // substitution and the MFMAs there; the D1 barrier publishes it.
    auto phase_a = [&](const int ci, float& rq, float& rk) __attribute__((always_inline)) {
        int tix = tid;
        asm volatile("" : "+v"(tix));
        const int r = tix >> 4;
        const int c8 = (tix & 15) * 8;
        // 1 for rows inside the sequence, else 0: multiplied in rather than
        // selected, so that no branch splits the phase this runs inside
        const float vm = r < L - ci * CH ? 1.0f : 0.0f;
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {  // BF16 pair dot products, FP32 sums
            const bf16x2 q2 = {cur.q[i], cur.q[i + 1]}, k2 = {cur.k[i], cur.k[i + 1]};
            sq = __builtin_amdgcn_fdot2_f32_bf16(q2, q2, sq, false);
            sk = __builtin_amdgcn_fdot2_f32_bf16(k2, k2, sk, false);
        }
        sq = row16_sum(sq);
        sk = row16_sum(sk);
        // the output scale rides on the query norm: O = (s Qg) S0^T + (s Aqk) U
        rq = (a.scale * vm) * (l2norm ? fast_rsqrt(sq + 1e-6f) : 1.0f);
        rk = vm * (l2norm ? fast_rsqrt(sk + 1e-6f) : 1.0f);
        float lv[8], dz[8];
        *(float4*)&dz[0] = *(const float4*)&sm.dtz[c8];
        *(float4*)&dz[4] = *(const float4*)&sm.dtz[c8 + 4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float e = __builtin_amdgcn_exp2f(-((float)cur.g[i] * zs + dz[i]));
            lv[i] = (lb2 * vm) * __builtin_amdgcn_rcpf(1.0f + e);
        }
        *(float4*)&sm.lam[r][c8] = make_float4(lv[0], lv[1], lv[2], lv[3]);
        *(float4*)&sm.lam[r][c8 + 4] = make_float4(lv[4], lv[5], lv[6], lv[7]);
        // the row's 16 lanes store the same value (no branch)
        sm.beta[ci & 1][r] = vm * (beta_logit ? sigmoidf_((float)cur.b) : (float)cur.b);
        // chunk ci's precision flag, set by phase B after the next barrier
        // (its slot last served chunk ci-2, which every wave has finished)
        if (tix == 0) sm.precise[ci & 1] = 0;
    };
    // ---- B: in-place prefix sums of chunk ci's decays over its tokens, and
    // exp(gC).  Every wave takes 32 channels: lanes 0-31 sum rows 0-7, lanes
    // 32-63 rows 8-15 and add the lower half's total, swapped across the
    // wave's halves.  Run for chunk ci+1 inside chunk ci's last phase, after
    // the barrier that publishes phase A. ----
    auto phase_b = [&](const int ci) __attribute__((always_inline)) {
        int tix = tid;
        asm volatile("" : "+v"(tix));
        const int lane = tix & 63;
        const int ch = 32 * wave + (lane & 31);
        const bool upper = lane >= 32;
        const int r0 = upper ? 8 : 0;
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = sm.lam[r0 + i][ch];
#pragma unroll
        for (int i = 1; i < 8; ++i) x[i] += x[i - 1];
        // upper lanes receive the lower half's total in [0], lower lanes the
        // upper half's in [1]
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x[7]), __float_as_uint(x[7]),
                                                         false, false);
        const float other = __uint_as_float(upper ? sw[0] : sw[1]);
        const float off = upper ? other : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) sm.lam[r0 + i][ch] = x[i] + off;
        // both halves hold the chunk total: the pair stores the same value
        sm.gamc[ci & 1][ch] = __builtin_amdgcn_exp2f(x[7] + other);
        // a channel that keeps more than exp(-2) of its state over the chunk
        // makes the chunk precise (every lane that sees one stores the same 1)
        if (x[7] + other > a.precise_log2) sm.precise[ci & 1] = 1;
    };
    float rq, rk;   // 1/sqrt(128)/|q| and 1/|k| of the chunk's row
    phase_a(cb, rq, rk);
    __syncthreads();
    phase_b(cb);

    // One chunk; full chunks are compiled without the tail masks.
    auto chunk = [&](const int ci, auto tail_tag) __attribute__((always_inline)) {
        constexpr bool kTail = decltype(tail_tag)::value;
        // Per-lane index arithmetic is recomputed every chunk from an opaque
        // copy of the thread id; hoisted out of the loop it would keep ~20
        // address registers alive and push the kernel into scratch spills.
        int tix = tid;
        asm volatile("" : "+v"(tix));
        const int lane = tix & 63;
        const int gq = lane >> 4;
        const int cl = lane & 15;
        const int r = tix >> 4;          // row-owner mapping: token row r,
        const int c8 = (tix & 15) * 8;   // channels [c8, c8 + 8)
        const int t0 = ci * CH;
        const int nv = kTail ? L - t0 : CH;
        const bool valid = !kTail || r < nv;
        // Issue priority by work left: the wave scheduler favours older
        // waves, so without this the first workgroup on a CU races ahead and
        // the last one finishes alone; raising the priority of those with
        // more chunks left keeps co-resident tasks abreast.
        set_prio_by_remaining(ce - ci, ce - cb);
        const int64_t rec = (rec0 + ci) * a.Hv + h;  // record index (records only)
        // with pair records (chunks 2p, 2p+1; rec0 is even) the even chunk
        // stores its start state and what steps it to the odd one (CF(U),
        // CF(Kt), exp(gC)), from which the adjoint forms the odd chunk's
        // start state; otherwise every chunk stores its start state
        const int64_t prec = kPairs ? ((rec0 + ci) >> 1) * a.Hv + h : rec;
        const bool rec_even = !kPairs || (ci & 1) == 0;   // stores S0
        const bool rec_step = kPairs && (ci & 1) == 0;    // stores the step
        if constexpr (kCkpt) {
            // state checkpoint before token t0 (E is a multiple of the chunk)
            // (the row comes from the caller's device copy of the starts, which
            // the host checked only through its mirror: a row out of range is
            // skipped rather than stored)
            const int64_t row = a.ckpt_start[n] + (ci * CH) / a.ckpt_every;
            if ((ci * CH) % a.ckpt_every == 0 && row >= 0 && row < a.ckpt_rows) {
                bf16* dst = (bf16*)a.ckpt + (row * a.Hv + h) * (int64_t)D * D;
#pragma unroll
                for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                    for (int j = 0; j < kNVB; ++j) {
                        const int vcol = 16 * (vb0 + j) + cl;
                        *(bf16x4*)(dst + vcol * D + 16 * kb + 4 * gq) = to_bf4(S[kb][j]);
                    }
            }
        }

        __syncthreads();   // chunk ci's prefix sums, exp(gC) and beta are in LDS
        // Precise chunk (some channel keeps more than exp(-2) of its state
        // over it): the operands that predict the state, Kg, Ki and S0, and Y
        // in Tb Y, become BF16 hi/lo pairs as well (three products each), so
        // that with weak decay the rounding of the prediction does not pile
        // up in the carried state.  The flag is uniform over the workgroup,
        // and the backward's rebuild takes the same decisions as the forward,
        // so it reproduces the forward's chunk states exactly.
        const bool precise = __builtin_amdgcn_readfirstlane(sm.precise[ci & 1]) != 0;
        // ---- C: decay factors and the chunk's operands (one branch for the
        // whole phase, so that each variant is scheduled on its own) ----
        auto phase_c = [&](auto prec_tag) __attribute__((always_inline)) {
            constexpr bool kPrecise = decltype(prec_tag)::value;
            float gc[8], gC[8];
            *(float4*)&gc[0] = *(const float4*)&sm.lam[r][c8];
            *(float4*)&gc[4] = *(const float4*)&sm.lam[r][c8 + 4];
            *(float4*)&gC[0] = *(const float4*)&sm.gamc[ci & 1][c8];
            *(float4*)&gC[4] = *(const float4*)&sm.gamc[ci & 1][c8 + 4];
            bf16x4 qg4[2], kg4[2], ki4[2], th4[2], tl4[2];
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
                qg4[s4] = to_bf4(qg);
                if constexpr (kPrecise) {
                    bf16x4 kl, il;
                    split4(kg, kg4[s4], kl);
                    split4(ki, ki4[s4], il);
                    const int o = rf_off(r, c8) + 64 * s4;
                    *(bf16x4*)&sm.rf_kg_lo[o] = kl;
                    *(bf16x4*)&sm.rf_ki_lo[o] = il;
                } else {
                    kg4[s4] = to_bf4(kg);
                    ki4[s4] = to_bf4(ki);
                }
                {
                    // FP16 pair (about 22 bits): Kt lies in [0, 1]; what falls
                    // below FP16's range is a contribution under 1e-7 of |U|
                    f16x4 h, l;
                    split4_f16(kt, h, l);
                    th4[s4] = __builtin_bit_cast(bf16x4, h);
                    tl4[s4] = __builtin_bit_cast(bf16x4, l);
                }
            }
            const int orf = rf_off(r, c8);  // channels c8+4.. sit one lane group later
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                *(bf16x4*)&sm.rf_qg[orf + 64 * s] = qg4[s];
                *(bf16x4*)&sm.rf_kg[orf + 64 * s] = kg4[s];
                *(bf16x4*)&sm.rf_ki[orf + 64 * s] = ki4[s];
            }
            // CF(Kt) hi / lo FP16 pairs: lane slot (gq, k) holds the hi parts of tokens
            // 4gq..4gq+3, then their lo parts; channel c8 + j of row r sits 8j
            // elements after channel c8 (one 16-channel block)
            const int ocf = (c8 >> 4) * FS2 + (((r >> 2) << 4) + (c8 & 15)) * 8 + (r & 3);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                sm.cf_kt[ocf + 8 * j] = th4[0][j];
                sm.cf_kt[ocf + 8 * (j + 4)] = th4[1][j];
                sm.cf_kt[ocf + 8 * j + 4] = tl4[0][j];
                sm.cf_kt[ocf + 8 * (j + 4) + 4] = tl4[1][j];
            }
        };
        if (precise)
            phase_c(std::true_type{});
        else
            phase_c(std::false_type{});
        // the row inputs are dead: fetch the next chunk's into the same registers
        load_rows_s(cur, sp, min(t0 + CH + r, L - 1), c8);
        __syncthreads();

        // ---- D1: the chunk's 16x16 algebra once (wave 0: Akk and the
        // substitution; wave 1: Aqk), Y and O^T on every wave ----
        // Y = Kg S0^T and O^T = S0 Qg^T (S0 converted once for both); every
        // wave forms its own, waves 0 and 1 inside their branches so that
        // these MFMAs fill the latency of the substitution
        f32x4 Y[kNVB], OT[kNVB];
#pragma unroll
        for (int vb = 0; vb < kNVB; ++vb) Y[vb] = OT[vb] = zero4();
        auto y_ot = [&]() __attribute__((always_inline)) {
            if (precise) {
                // Y = Kg_hi S0_hi + Kg_hi S0_lo + Kg_lo S0_hi, O^T from S0_hi
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 kg8 = cat8(ld4(&sm.rf_kg[(2 * j) * FS], lane), ld4(&sm.rf_kg[(2 * j + 1) * FS], lane));
                    const bf16x8 kl8 = cat8(ld4(&sm.rf_kg_lo[(2 * j) * FS], lane),
                                            ld4(&sm.rf_kg_lo[(2 * j + 1) * FS], lane));
                    bf16x8 q8;
                    if constexpr (kOut)
                        q8 = cat8(ld4(&sm.rf_qg[(2 * j) * FS], lane), ld4(&sm.rf_qg[(2 * j + 1) * FS], lane));
#pragma unroll
                    for (int vb = 0; vb < kNVB; ++vb) {
                        if constexpr (kRec) {
                            if (rec_even) {
                                const bf16x4 ident = identity_frag(lane);
                                const int vbg = vb0 + vb;
                                bf16* dst = (bf16*)a.rec_s0 + prec * (D * D) + lane * 4;
                                *(bf16x4*)(dst + ((2 * j) * 8 + vbg) * 256) =
                                    to_bf4(transpose_frag(to_bf4(S[2 * j][vb]), ident));
                                *(bf16x4*)(dst + ((2 * j + 1) * 8 + vbg) * 256) =
                                    to_bf4(transpose_frag(to_bf4(S[2 * j + 1][vb]), ident));
                            }
                        }
                        bf16x4 h0, l0, h1, l1;
                        split4(S[2 * j][vb], h0, l0);
                        split4(S[2 * j + 1][vb], h1, l1);
                        const bf16x8 sh = cat8(h0, h1);
                        Y[vb] = mma32(kg8, sh, Y[vb]);
                        Y[vb] = mma32(kg8, cat8(l0, l1), Y[vb]);
                        Y[vb] = mma32(kl8, sh, Y[vb]);
                        if constexpr (kOut) OT[vb] = mma32(sh, q8, OT[vb]);
                    }
                }
                return;
            }
            bf16x8 sb[4][kNVB];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 kg8 = cat8(ld4(&sm.rf_kg[(2 * j) * FS], lane), ld4(&sm.rf_kg[(2 * j + 1) * FS], lane));
#pragma unroll
                for (int vb = 0; vb < kNVB; ++vb) {
                    const bf16x4 s0 = to_bf4(S[2 * j][vb]);
                    const bf16x4 s1 = to_bf4(S[2 * j + 1][vb]);
                    sb[j][vb] = cat8(s0, s1);
                    Y[vb] = mma32(kg8, sb[j][vb], Y[vb]);    // lane (gq, v) holds Y[4gq+i][v]
                    if constexpr (kRec) {
                        // chunk-start state record (even chunks): frag (kb, vb)
                        // with lane (gq, k) holding S0[16vb + 4gq + i][16kb + k]
                        if (rec_even) {
                            const bf16x4 ident = identity_frag(lane);
                            const int vbg = vb0 + vb;
                            bf16* dst = (bf16*)a.rec_s0 + prec * (D * D) + lane * 4;
                            *(bf16x4*)(dst + ((2 * j) * 8 + vbg) * 256) = to_bf4(transpose_frag(s0, ident));
                            *(bf16x4*)(dst + ((2 * j + 1) * 8 + vbg) * 256) = to_bf4(transpose_frag(s1, ident));
                        }
                    }
                }
            }
            if constexpr (kOut) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 q8 = cat8(ld4(&sm.rf_qg[(2 * j) * FS], lane), ld4(&sm.rf_qg[(2 * j + 1) * FS], lane));
#pragma unroll
                    for (int vb = 0; vb < kNVB; ++vb) OT[vb] = mma32(sb[j][vb], q8, OT[vb]);   // lane (gq, c): O[c][v=4gq+i]
                }
            }
        };
        float rq_next, rk_next;
        if (wave == 0) {
            // the substitution is the phase's longest chain: top issue
            // priority until the next chunk resets it
            __builtin_amdgcn_s_setprio(3);
            SolveScratch& ws = sm.sv;
            f32x4 akk = zero4();
            if (precise) {   // Kg_hi Ki_hi + Kg_hi Ki_lo + Kg_lo Ki_hi
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 kg8 = cat8(ld4(&sm.rf_kg[(2 * j) * FS], lane), ld4(&sm.rf_kg[(2 * j + 1) * FS], lane));
                    const bf16x8 ki8 = cat8(ld4(&sm.rf_ki[(2 * j) * FS], lane), ld4(&sm.rf_ki[(2 * j + 1) * FS], lane));
                    akk = mma32(kg8, ki8, akk);
                    akk = mma32(kg8, cat8(ld4(&sm.rf_ki_lo[(2 * j) * FS], lane),
                                          ld4(&sm.rf_ki_lo[(2 * j + 1) * FS], lane)), akk);
                    akk = mma32(cat8(ld4(&sm.rf_kg_lo[(2 * j) * FS], lane),
                                     ld4(&sm.rf_kg_lo[(2 * j + 1) * FS], lane)), ki8, akk);
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const bf16x8 kg8 = cat8(ld4(&sm.rf_kg[(2 * j) * FS], lane), ld4(&sm.rf_kg[(2 * j + 1) * FS], lane));
                    const bf16x8 ki8 = cat8(ld4(&sm.rf_ki[(2 * j) * FS], lane), ld4(&sm.rf_ki[(2 * j + 1) * FS], lane));
                    akk = mma32(kg8, ki8, akk);     // lane (gq, c) holds Akk[4gq+i][c]
                }
            }
            y_ot();
            const float4 b4 = *(const float4*)&sm.beta[ci & 1][4 * gq];
            float4 col;  // column cl of N, rows 4gq..4gq+3
            col.x = (cl < 4 * gq + 0) ? b4.x * akk[0] : 0.f;
            col.y = (cl < 4 * gq + 1) ? b4.y * akk[1] : 0.f;
            col.z = (cl < 4 * gq + 2) ? b4.z * akk[2] : 0.f;
            col.w = (cl < 4 * gq + 3) ? b4.w * akk[3] : 0.f;
            *(float4*)&ws.nT[cl][4 * gq] = col;
            if constexpr (kRec) {
                // Akk^T[col][row] = Akk[row][col] for row > col
                float4 m;
                m.x = (cl < 4 * gq + 0) ? akk[0] : 0.f;
                m.y = (cl < 4 * gq + 1) ? akk[1] : 0.f;
                m.z = (cl < 4 * gq + 2) ? akk[2] : 0.f;
                m.w = (cl < 4 * gq + 3) ? akk[3] : 0.f;
                *(float4*)at(a.rec_ta + rec * 768, 256 + cl * 16 + 4 * gq) = m;
            }
            // T = (I + N)^-1 by right-looking substitution on all 64 lanes:
            // lane (col = lane/4, q = lane%4) keeps rows 4q..4q+3 of column
            // col; N is zero on and above the diagonal, so no masking is
            // needed.  y[j] (row 4q+j of column col) starts at [row == col]
            // and loses N[row][m] t[m] at every step m; row m is final when
            // step m begins, so t[m] = y of the quad lane that holds row m.
            const int colx = lane >> 2;
            const int qd = lane & 3;
            float y[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) y[j] = (4 * qd + j == colx) ? 1.0f : 0.0f;
            // (step m changes only rows below m: the last step is empty, and
            // element j, the rows 4q+j, is done once m reaches 12+j)
            float4 nxt = *(const float4*)&ws.nT[0][4 * qd];
#pragma unroll
            for (int m = 0; m < CH - 1; ++m) {
                const float4 nm = nxt;
                if (m + 1 < CH - 1) nxt = *(const float4*)&ws.nT[m + 1][4 * qd];
                const float tm = quad_bcast(y[m & 3], m >> 2);
                if (m < 12) y[0] -= nm.x * tm;
                if (m < 13) y[1] -= nm.y * tm;
                if (m < 14) y[2] -= nm.z * tm;
                y[3] -= nm.w * tm;
            }
            if constexpr (kRec)   // T^T[col][row]
                *(float4*)at(a.rec_ta + rec * 768, colx * 16 + 4 * qd) = make_float4(y[0], y[1], y[2], y[3]);
            // Tb[i][col] = T[i][col] beta_col
            const float bc = sm.beta[ci & 1][colx];
#pragma unroll
            for (int j = 0; j < 4; ++j) ws.tb[4 * qd + j][colx] = y[j] * bc;
            phase_a(ci + 1, rq_next, rk_next);
        } else if (wave == 1) {
            // RF16(Aqk) = frag of Aqk^T = Ki Qg^T, causal part
            f32x4 aqkT = zero4();
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bf16x8 ki8 = cat8(ld4(&sm.rf_ki[(2 * j) * FS], lane), ld4(&sm.rf_ki[(2 * j + 1) * FS], lane));
                const bf16x8 qg8 = cat8(ld4(&sm.rf_qg[(2 * j) * FS], lane), ld4(&sm.rf_qg[(2 * j + 1) * FS], lane));
                aqkT = mma32(ki8, qg8, aqkT);
            }
            y_ot();
            f32x4 am;
#pragma unroll
            for (int i = 0; i < 4; ++i) am[i] = (4 * gq + i <= cl) ? aqkT[i] : 0.f;
            if constexpr (kRec)   // Aqk[row = cl][col = 4gq + i], scale included
                *(float4*)at(a.rec_ta + rec * 768, 512 + cl * 16 + 4 * gq) = make_float4(am[0], am[1], am[2], am[3]);
            if constexpr (kOut) {
                // halved and stored twice: [Aqk/2 | Aqk/2] against [U_hi | U_hi]
                // is U_hi Aqk in one 16x16x32 (halving is exact)
                const bf16x4 h = to_bf4(am * 0.5f);
                *(bf16x8*)&sm.sh_aq[lane * 8] = cat8(h, h);
            }
            phase_a(ci + 1, rq_next, rk_next);
        } else {
            y_ot();
            phase_a(ci + 1, rq_next, rk_next);
        }
        __syncthreads();
        // ---- D2 (per wave): U, output, state update ----
        // RF16(Tb) as a hi/lo pair, split by every wave from wave 0's FP32 Tb
        // (off the substitution's critical path): lane (gq, c) holds Tb[c][4gq+i]
        bf16x4 tbh, tbl;
        {
            const float4 t4 = *(const float4*)&sm.sv.tb[cl][4 * gq];
            split4(f32x4{t4.x, t4.y, t4.z, t4.w}, tbh, tbl);
        }
        bf16x8 aq2;
        if constexpr (kOut) aq2 = *(const bf16x8*)&sm.sh_aq[lane * 8];
        // U = Tb V - Tb Y (CF(V) loaded directly)
        f32x4 U[kNVB];
        {
            if constexpr (kSegPQ) {
                if (!segQ) {  // P runs with v = 0
#pragma unroll
                    for (int vb = 0; vb < kNVB; ++vb) vcur.v[vb] = to_bf4(zero4());
                }
            }
            // a 16x16x32 costs about what a 16x16x16 does, so the hi/lo
            // products take two: [Tb_hi|Tb_lo] [V;V] and [Tb_hi|Tb_lo] [-Y;-Y]
            // (every operand tuple is formed where it is produced, no copies)
            const bf16x8 tb2 = cat8(tbh, tbl);
#pragma unroll
            for (int vb = 0; vb < kNVB; ++vb) U[vb] = mma32(tb2, cat8(vcur.v[vb], vcur.v[vb]), zero4());
            if (precise) {   // Y as a hi/lo pair as well: [Tb_hi|Tb_lo] [-Y_hi;-Y_hi] + [-Y_lo;-Y_lo]
#pragma unroll
                for (int vb = 0; vb < kNVB; ++vb) {
                    bf16x4 yh, yl;
                    split4(-Y[vb], yh, yl);
                    U[vb] = mma32(tb2, cat8(yh, yh), U[vb]);
                    U[vb] = mma32(tb2, cat8(yl, yl), U[vb]);
                }
            } else {
#pragma unroll
                for (int vb = 0; vb < kNVB; ++vb)
                    U[vb] = mma32(tb2, cat8(to_bf4_neg(Y[vb]), to_bf4_neg(Y[vb])), U[vb]);
            }
        }
        load_cols_cf<kNVB>(vcur, sp, t0 + CH + 4 * gq, L - 1, 16 * vb0 + cl);
        // O^T += U^T Aqk^T, store; then the state update S^T += Kt^T U
        auto out_term = [&](int vb, bf16x4 uh) __attribute__((always_inline)) {
            if constexpr (kRec) {
                // U record, RF layout: lane (gq, c) holds U[c][16vb + 4gq + i]
                const bf16x4 ub = to_bf4(U[vb]);
                const bf16x4 ut = to_bf4(transpose_frag(ub, identity_frag(lane)));
                *(bf16x4*)at((bf16*)a.rec_u + rec * (CH * D), ((vb0 + vb) * 64 + lane) * 4) = ut;
                // even chunks: CF(U) as well (lane (gq, c) holds U[4gq + i][16vb + c])
                if (rec_step) *(bf16x4*)((bf16*)a.rec_x + prec * REC_X_ELEMS + ((vb0 + vb) * 64 + lane) * 4) = ub;
            }
            if constexpr (kOut) {
                // [U_hi|U_hi] against [Aqk/2;Aqk/2]: the chain's last step is a
                // 16x16x32 as well; lane (gq, c) holds O[c][16(vb0 + vb) + 4gq + i]
                OT[vb] = mma32(cat8(uh, uh), aq2, OT[vb]);
                if (cl < nv) {
                    const bf16x4 ob = to_bf4(OT[vb]);
                    *(bf16x4*)at(sp.o, __umul24((unsigned)(t0 + cl), sp.sv) + 16 * (vb0 + vb) + 4 * gq) = ob;
                }
            }
        };
#pragma unroll
        for (int vb = 0; vb < kNVB; ++vb) out_term(vb, to_bf4(U[vb]));
        phase_b(ci + 1);
        // S^T += Kt^T U in FP16, [Kt_hi|Kt_lo] (about 22 bits) against [U;U]
        // (11 bits) in one 16x16x32 per state frag; precise chunks add
        // [Kt_hi|Kt_lo] [U_lo;U_lo] (U to about 22 bits as well).  (One
        // accumulation chain keeps one MFMA shape: a 16x16x16 that reads the
        // accumulator of a 16x16x32 issued just before it has been seen to
        // miss that product.)
        // U beyond FP16's range (|U| of 16384 or more somewhere in the wave,
        // or not finite) is scaled by 2^-e for the product, and the state
        // with it (powers of two: exact), and both are scaled back after.
        float um = 0.f;
#pragma unroll
        for (int vb = 0; vb < kNVB; ++vb)
            um = fmaxf(um, fmaxf(fmaxf(fabsf(U[vb][0]), fabsf(U[vb][1])),
                                 fmaxf(fabsf(U[vb][2]), fabsf(U[vb][3]))));
        const bool big = __builtin_amdgcn_ballot_w64(!(um < 16384.f)) != 0;
        float isc = 1.f;
        if (big) {
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) um = fmaxf(um, __shfl_xor(um, o, 64));
            const int e = __builtin_amdgcn_readfirstlane(um < 3.0e38f ? max(ilogbf(um) - 12, 0) : 116);
            const float sc = ldexpf(1.f, -e);
            isc = ldexpf(1.f, e);
#pragma unroll
            for (int vb = 0; vb < kNVB; ++vb) U[vb] *= sc;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                for (int vb = 0; vb < kNVB; ++vb) S[kb][vb] *= sc;
        }
        // (a precise chunk parks U's lo part in LDS over the main loop, which
        // then holds no value that only precise chunks need)
        f16x8 uh8[kNVB];
#pragma unroll
        for (int vb = 0; vb < kNVB; ++vb) {
            f16x4 h, l;
            if (precise) {
                split4_f16(U[vb], h, l);
                sm.ulo[wave][vb][lane] = l;
            } else {
                h = to_f16x4(U[vb]);
            }
            uh8[vb] = cat8h(h, h);
        }
#pragma unroll
        for (int kb = 0; kb < 8; ++kb) {
            const f16x8 t2 = *(const f16x8*)&sm.cf_kt[kb * FS2 + lane * 8];
            const float4 gd = *(const float4*)&sm.gamc[ci & 1][16 * kb + 4 * gq];
#pragma unroll
            for (int vb = 0; vb < kNVB; ++vb) {
                f32x4 s = S[kb][vb];
                s[0] *= gd.x; s[1] *= gd.y; s[2] *= gd.z; s[3] *= gd.w;
                S[kb][vb] = mma32h(t2, uh8[vb], s);
            }
        }
        if (precise) {   // + [Kt_hi|Kt_lo] [U_lo;U_lo]
            f16x8 ul8[kNVB];
#pragma unroll
            for (int vb = 0; vb < kNVB; ++vb) {
                const f16x4 l = sm.ulo[wave][vb][lane];
                ul8[vb] = cat8h(l, l);
            }
#pragma unroll
            for (int kb = 0; kb < 8; ++kb) {
                const f16x8 t2 = *(const f16x8*)&sm.cf_kt[kb * FS2 + lane * 8];
#pragma unroll
                for (int vb = 0; vb < kNVB; ++vb) S[kb][vb] = mma32h(t2, ul8[vb], S[kb][vb]);
            }
        }
        if (big) {
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                for (int vb = 0; vb < kNVB; ++vb) S[kb][vb] *= isc;
        }
        if constexpr (kRec) {
            // even chunks of pair records: this wave's CF(Kt) blocks vb0,
            // vb0 + 1 in BF16 (hi + lo of the FP16 pair) and, from wave 0, exp(gC)
            if (rec_step) {
                bf16* xp = (bf16*)a.rec_x + prec * REC_X_ELEMS;
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int kb = vb0 + j;
                    const f16x8 t2 = *(const f16x8*)&sm.cf_kt[kb * FS2 + lane * 8];
                    f32x4 kt;
#pragma unroll
                    for (int i = 0; i < 4; ++i) kt[i] = (float)t2[i] + (float)t2[i + 4];
                    *(bf16x4*)(xp + 2048 + (kb * 64 + lane) * 4) = to_bf4(kt);
                }
                if (vb0 == 0)
                    *(float2*)((float*)(xp + 4096) + 2 * lane) = *(const float2*)&sm.gamc[ci & 1][2 * lane];
            }
        }
        const int tend = t0 + nv;
        if (kMode == kFwdTape && a.tape != nullptr && tend < L && (tend % a.ck_every) == 0) {
            const int64_t jck = tend / a.ck_every;
            store_state<kNVB>(a.tape + ((tape_base + jck - 1) * a.Hv + h) * (int64_t)D * D, S, vb0, gq, cl);
        }
        rq = rq_next;
        rk = rk_next;
    };
    const int cfull = min(ce, nfull);
    for (int ci = cb; ci < cfull; ++ci) chunk(ci, std::false_type{});
    if (nfull < ce) chunk(nfull, std::true_type{});
    if constexpr (kInfer) {
        const int lane = tid & 63, gq = lane >> 4, cl = lane & 15;
#pragma unroll
        for (int kb = 0; kb < 8; ++kb)
#pragma unroll
            for (int j = 0; j < kNVB; ++j) {
                const int vcol = 16 * (vb0 + j) + cl;
                *(bf16x4*)(pslab + vcol * D + 16 * kb + 4 * gq) = to_bf4(S[kb][j]);
            }
    } else if constexpr (kSegPQ) {
        const int64_t segs = a.seg_items / a.Hv;
        const int64_t sj = a.plan.tape_off[n] + n + seg;
        const int64_t si = (segQ ? segs : 0) + sj;
        store_state<kNVB>(a.seg_out + (si * a.Hv + h) * (int64_t)D * D, S, vb0, (tid & 63) >> 4, tid & 15);
        if (!segQ) {
            // P transposed as well (third slab), for the adjoint's chain:
            // lane (gq, cl) holds P[vcol][16kb + 4gq + i]; adjacent lanes
            // write adjacent columns of row 16kb + 4gq + i
            float* pt = a.seg_out + ((2 * segs + sj) * a.Hv + h) * (int64_t)D * D;
            const int lane = tid & 63, gq = lane >> 4, cl = lane & 15;
#pragma unroll
            for (int kb = 0; kb < 8; ++kb)
#pragma unroll
                for (int j = 0; j < kNVB; ++j)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        pt[(16 * kb + 4 * gq + i) * D + 16 * (vb0 + j) + cl] = S[kb][j][i];
        }
    } else if (kOut && a.s_final != nullptr && ce == nchunks) {
        store_state<kNVB>(a.s_final + slab, S, vb0, (tid & 63) >> 4, tid & 15);
    }
}

hipError_t launch_fwd_chunk(const FwdArgs& a, hipStream_t s) {
    if (a.num_tasks == 0) return hipSuccess;
    if (a.infer && a.ckpt != nullptr)
        hipLaunchKernelGGL(fwd_chunk_kernel<kFwdInferCkpt>, dim3((unsigned)a.num_tasks), dim3(FC_THREADS),
                           0, s, a);
    else if (a.infer)
        hipLaunchKernelGGL(fwd_chunk_kernel<kFwdInfer>, dim3((unsigned)a.num_tasks), dim3(FC_THREADS), 0,
                           s, a);
    else if (a.rec_s0 != nullptr && a.rec_pairs)
        hipLaunchKernelGGL(fwd_chunk_kernel<kFwdRecordsPairs>, dim3((unsigned)a.num_tasks), dim3(FC_THREADS),
                           0, s, a);
    else if (a.rec_s0 != nullptr)
        hipLaunchKernelGGL(fwd_chunk_kernel<kFwdRecords>, dim3((unsigned)a.num_tasks), dim3(FC_THREADS), 0,
                           s, a);
    else if (a.vsplit)  // two workgroups per task, producer and consumer waves
        return launch_fwd_pipe(a, s);
    else
        hipLaunchKernelGGL(fwd_chunk_kernel<kFwdTape>, dim3((unsigned)a.num_tasks), dim3(FC_THREADS), 0, s,
                           a);
    return hipGetLastError();
}

// One workgroup per (tape segment, value head): num_items = segments * Hv.
hipError_t launch_state_rebuild(const FwdArgs& a, int64_t num_items, hipStream_t s) {
    if (num_items == 0) return hipSuccess;
    if (a.rec_pairs)
        hipLaunchKernelGGL(fwd_chunk_kernel<kFwdRebuildPairs>, dim3((unsigned)num_items), dim3(FC_THREADS), 0,
                           s, a);
    else
        hipLaunchKernelGGL(fwd_chunk_kernel<kFwdRebuild>, dim3((unsigned)num_items), dim3(FC_THREADS), 0, s,
                           a);
    return hipGetLastError();
}

// Chains the start states through the segments of every (sequence, value
// head): S_in(j) = S_in(j-1) P(j-1) + Q(j-1), written to tape row j-1.  Value
// rows are independent, so each workgroup takes 16 rows of one task (8 per
// task) and keeps them in LDS; wave w forms output columns 32w..32w+31 with
// FP32 16x16x4 MFMAs (FP32 products and sums), P read from L2.
__global__ __launch_bounds__(256) void seg_combine_kernel(FwdArgs a) {
    constexpr int SP = D + 1;  // padded row: the 16 rows of a K-step sit in distinct banks
    __shared__ float sr[16 * SP];
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6, gq = lane >> 4, cl = lane & 15;
    const int rb = blockIdx.x & 7;
    const int nh = blockIdx.x >> 3;
    const int n = nh / a.Hv, h = nh - n * a.Hv;
    const int L = a.plan.seq_len[n];
    const int nseg = (L + a.ck_every - 1) / a.ck_every;
    if (nseg < 2) return;  // uniform over the workgroup: before any barrier
    const int64_t toff = a.plan.tape_off[n];
    const int64_t DD = (int64_t)D * D;
    const int64_t segs = a.seg_items / a.Hv;
    {
        const float* s0 = a.s0 + ((int64_t)n * a.Hv + h) * DD + (int64_t)(16 * rb) * D;
        for (int e = tid; e < 16 * D; e += 256) sr[(e / D) * SP + (e % D)] = s0[e];
    }
    for (int j = 1; j < nseg; ++j) {
        const int64_t sj = toff + n + (j - 1);  // segment j-1 of sequence n
        const float* P = a.seg_out + (sj * a.Hv + h) * DD;
        const float* Q = a.seg_out + ((segs + sj) * a.Hv + h) * DD;
        __syncthreads();  // rows of S_in(j-1) in LDS
        f32x4 acc[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = 16 * (2 * wave + t) + cl;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[t][i] = Q[(int64_t)(16 * rb + 4 * gq + i) * D + col];
        }
#pragma unroll 8
        for (int kk = 0; kk < D; kk += 4) {
            const float x = sr[cl * SP + kk + gq];  // A[row cl][k = kk + gq]
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const float y = P[(int64_t)(kk + gq) * D + 16 * (2 * wave + t) + cl];  // B[k][col]
                acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(x, y, acc[t], 0, 0, 0);
            }
        }
        __syncthreads();  // every wave has read S_in(j-1)
        float* dst = a.tape + ((toff + j - 1) * a.Hv + h) * DD + (int64_t)(16 * rb) * D;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int col = 16 * (2 * wave + t) + cl;
#pragma unroll
            for (int i = 0; i < 4; ++i) {  // lane (gq, cl) holds rows 4gq+i, column col
                sr[(4 * gq + i) * SP + col] = acc[t][i];
                dst[(4 * gq + i) * D + col] = acc[t][i];
            }
        }
    }
}

// The segment-parallel forward (needs a.tape, a.seg_out and a.seg_items):
// P and Q of every segment, the chain through the tape, then every segment
// again for o and the final state.  The plan's task list must be the segment
// list; N is the number of sequences.
hipError_t launch_fwd_segments(const FwdArgs& a, int N, hipStream_t s) {
    if (a.seg_items == 0) return hipSuccess;
    hipLaunchKernelGGL(fwd_chunk_kernel<kFwdSegPQ>, dim3((unsigned)(2 * a.seg_items)), dim3(FC_THREADS), 0,
                       s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(seg_combine_kernel, dim3((unsigned)(N * a.Hv * 8)), dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(fwd_chunk_kernel<kFwdSegOut>, dim3((unsigned)a.seg_items), dim3(FC_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
