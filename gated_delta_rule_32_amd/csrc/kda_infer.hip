// Inference forward of page "flashinfer.kda.recurrent_kda": decode and
// prefill on a BF16 state pool updated in place, with the page's gate, beta
// and norm options (parameters use_qk_l2norm_in_kernel, use_gate_in_kernel,
// lower_bound, beta_is_logit, initial_state with ssm_state_indices).
//
// Token-serial recurrence in FP32, one workgroup (4 waves) per (sequence,
// value head), no LDS and no barriers.  A lane owns 8 keys of 8 state rows:
// lanes 16m..16m+15 of wave w cover all 128 keys of rows 16j + 4w + m
// (j = 0..7), so each of the 8 row loads and stores of a wave moves 1 KiB of
// contiguous state, and every per-row dot product is a sum over one 16-lane
// DPP row.  Per token, every lane forms the prologue of its own 8 keys (the
// norms' sums over 128 keys are also DPP-row sums), then for each row:
//     S[v][:] *= alpha;   e = beta (v_t[v] - S[v][:].kn);   S[v][:] += e kn;
//     o[v] = scale S[v][:].qn
// (recurrence of page "flashinfer.kda_backward.recurrent_kda_backward",
// description).  The next token's inputs are fetched while the current one
// is processed.  With one token per sequence (decode) the kernel moves each
// state slot once in and once out.  With state checkpoints every E tokens the
// state before token j*E is also stored, rounded to BF16, to row j of the
// sequence's checkpoint rows (parameter state_checkpoints).  Speculative
// decode (parameters num_spec_tokens, num_accepted_tokens): the state starts
// from the slot of the last accepted token of the previous round and is
// written after every token to that token's own slot, so that the next round
// can resume from any accepted prefix.
#include "kda_common.hpp"
#include "kda_kernels.h"

namespace kda {

namespace {
constexpr int IT_THREADS = 256;

struct TokIn {
    bf16x8 q, k, g;
    bf16 b;
    bf16 v[8];   // value of rows 16j + 4w + m
};
}  // namespace

__global__ __launch_bounds__(IT_THREADS) void infer_token_kernel(FwdArgs a) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int rbase = 4 * (tid >> 6) + (lane >> 4);  // row of j = 0
    const int kofs = (lane & 15) * 8;                // this lane's 8 keys
    const int code = a.plan.task[blockIdx.x];
    const int n = code / a.Hv;
    const int h = code - n * a.Hv;
    const int hq = h / a.G;
    const int64_t tok0 = a.plan.seq_start[n];
    const int L = a.plan.seq_len[n];
    // pool slot of sequence n (checked on the host; a slot out of range ends
    // the workgroup before any access)
    const int spec = a.spec_tokens;
    int64_t slot;
    if (spec > 0) {
        const int acc = a.spec_accepted != nullptr ? a.spec_accepted[n] : 1;
        slot = a.pool_index[(int64_t)n * (spec + 1) + min(max(acc, 1), spec + 1) - 1];
    } else {
        slot = a.pool_index != nullptr ? a.pool_index[n] : n;
    }
    if (slot < 0 || slot >= a.pool_slots) return;
    bf16* pool = (bf16*)a.pool + (slot * a.Hv + h) * (int64_t)D * D;
    const int64_t slab_elems = (int64_t)a.Hv * D * D;
    // initial state: the source pool's slot when one is given
    const bf16* init = pool;
    if (a.src_pool != nullptr) {
        const int64_t ss = a.src_index[n];
        if (ss < 0 || ss >= a.src_slots) return;
        init = (const bf16*)a.src_pool + (ss * a.Hv + h) * (int64_t)D * D;
    }

    float S[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const bf16x8 x = *(const bf16x8*)(init + (16 * j + rbase) * D + kofs);
#pragma unroll
        for (int i = 0; i < 8; ++i) S[j][i] = (float)x[i];
    }
    const bool gate_in = a.use_gate_in_kernel != 0;
    const bool l2norm = a.use_qk_l2norm != 0;
    const bool beta_logit = a.beta_is_logit != 0;
    const float eA = gate_in ? __expf(a.A_log[h]) : 0.f;
    float dtb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
        dtb[i] = (gate_in && a.dt_bias != nullptr) ? a.dt_bias[h * D + kofs + i] : 0.f;

    const bf16* qp = (const bf16*)a.q + (tok0 * a.Hqk + hq) * D + kofs;
    const bf16* kp = (const bf16*)a.k + (tok0 * a.Hqk + hq) * D + kofs;
    const bf16* gp = (const bf16*)a.g + (tok0 * a.Hv + h) * D + kofs;
    const bf16* vp = (const bf16*)a.v + (tok0 * a.Hv + h) * D + rbase;
    const bf16* bp = (const bf16*)a.beta + tok0 * a.Hv + h;
    bf16* op = (bf16*)a.o + (tok0 * a.Hv + h) * D + rbase;
    const int64_t sq = (int64_t)a.Hqk * D, sv = (int64_t)a.Hv * D, sb = a.Hv;

    auto load = [&](TokIn& x, int t) __attribute__((always_inline)) {
        x.q = *(const bf16x8*)(qp + t * sq);
        x.k = *(const bf16x8*)(kp + t * sq);
        x.g = *(const bf16x8*)(gp + t * sv);
        x.b = bp[t * sb];
#pragma unroll
        for (int j = 0; j < 8; ++j) x.v[j] = vp[t * sv + 16 * j];
    };
    TokIn nxt;
    load(nxt, 0);
    // checkpoint rows start at the caller's device copy of the starts, which
    // the host checked only through its mirror: rows out of range are skipped
    const int64_t ck_row0 = a.ckpt != nullptr ? a.ckpt_start[n] : 0;
    bf16* ck = a.ckpt != nullptr && ck_row0 >= 0 ? (bf16*)a.ckpt + (ck_row0 * a.Hv + h) * (int64_t)D * D : nullptr;
    const int64_t ck_stride = (int64_t)a.Hv * D * D;
    for (int t = 0; t < L; ++t) {
        const TokIn cur = nxt;
        load(nxt, min(t + 1, L - 1));
        if (ck != nullptr && t % a.ckpt_every == 0 && ck_row0 + t / a.ckpt_every < a.ckpt_rows) {
            bf16* dst = ck + (t / a.ckpt_every) * ck_stride;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                bf16x8 x;
#pragma unroll
                for (int i = 0; i < 8; ++i) x[i] = (bf16)S[j][i];
                *(bf16x8*)(dst + (16 * j + rbase) * D + kofs) = x;
            }
        }
        float qn[8], kn[8], al[8];
        float ssq = 0.f, ssk = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            qn[i] = (float)cur.q[i];
            kn[i] = (float)cur.k[i];
            ssq += qn[i] * qn[i];
            ssk += kn[i] * kn[i];
        }
        if (l2norm) {
            const float rq = fast_rsqrt(row16_sum(ssq) + 1e-6f);
            const float rk = fast_rsqrt(row16_sum(ssk) + 1e-6f);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                qn[i] *= rq;
                kn[i] *= rk;
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float gv = (float)cur.g[i];
            al[i] = fast_exp(gate_in ? a.lower_bound * sigmoidf_(eA * (gv + dtb[i])) : gv);
        }
        const float bv = (float)cur.b;
        const float b = beta_logit ? sigmoidf_(bv) : bv;
        float ov[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float pk = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                S[j][i] *= al[i];
                pk += S[j][i] * kn[i];
            }
            const float e = b * ((float)cur.v[j] - row16_sum(pk));
            float oq = 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                S[j][i] += e * kn[i];
                oq += S[j][i] * qn[i];
            }
            ov[j] = row16_sum(oq);
        }
        if ((lane & 15) == 0) {
#pragma unroll
            for (int j = 0; j < 8; ++j) op[t * sv + 16 * j] = (bf16)(a.scale * ov[j]);
        }
        if (spec > 0) {  // the state after token t, to token t's slot
            const int64_t st = a.pool_index[(int64_t)n * (spec + 1) + t];
            if (st >= 0 && st < a.pool_slots) {
                bf16* dst = (bf16*)a.pool + st * slab_elems + h * (int64_t)D * D;
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    bf16x8 x;
#pragma unroll
                    for (int i = 0; i < 8; ++i) x[i] = (bf16)S[j][i];
                    *(bf16x8*)(dst + (16 * j + rbase) * D + kofs) = x;
                }
            }
        }
    }
    if (spec == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            bf16x8 x;
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = (bf16)S[j][i];
            *(bf16x8*)(pool + (16 * j + rbase) * D + kofs) = x;
        }
    }
}

hipError_t launch_infer_token(const FwdArgs& a, hipStream_t s) {
    if (a.num_tasks == 0) return hipSuccess;
    hipLaunchKernelGGL(infer_token_kernel, dim3((unsigned)a.num_tasks), dim3(IT_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace kda
