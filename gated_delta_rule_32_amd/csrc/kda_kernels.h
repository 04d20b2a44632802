// Internal launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef unsigned short bf16_t;  // BF16 bits in memory

// 16-bit elements of one pair record of rec_x: CF(U) and CF(Kt) of the pair's
// even chunk (2048 BF16 each), then exp(gC) (128 FP32).
constexpr int REC_X_ELEMS = 2 * 2048 + 2 * 128;

// Device-side schedule built on the host from the sequence lengths.  Task i
// (0 <= i < num_tasks, longest sequence first) is (n, h) = (task[i] / Hv,
// task[i] % Hv).  Sequence n occupies flattened tokens [seq_start[n],
// seq_start[n] + seq_len[n]) of the [B*T] token axis.  tape_off[n] counts the
// stored checkpoints of the sequences before n (ceil(L/C_ck) - 1 each) and
// chunk_off[n] the 16-token chunks (ceil(L/16) each, rounded up to even, so
// that every sequence's chunk pairs start at an even index).
struct DevPlan {
    const int32_t* task;
    const int64_t* seq_start;
    const int32_t* seq_len;
    const int64_t* tape_off;
    const int64_t* chunk_off;
};

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* g;
    const void* beta;
    const float* A_log;
    const float* dt_bias;
    const float* s0;        // [N][Hv][128][128]
    void* o;
    float* s_final;         // [N][Hv][128][128]; may be null (state rebuild)
    float* tape;            // [ck][Hv][128][128]; may be null
    // Records written by the state rebuild and read by the adjoint (layouts:
    // kda_bwd.hip).  Per chunk, rec = (chunk_off[n] + chunk) * Hv + h.  With
    // rec_pairs the chunk-start state is stored for even chunks only, per
    // pair of chunks (2p, 2p+1) at prec = ((chunk_off[n] + chunk) / 2) * Hv
    // + h (chunk_off[n] is even), with what steps it to the odd chunk after;
    // otherwise for every chunk, at prec = rec, and rec_x is unused.
    bf16_t* rec_s0;         // [prec][8 kb][8 vb][64][4] chunk-start state, BF16
    bf16_t* rec_x;          // [prec][REC_X] the even chunk's CF(U), CF(Kt) (BF16) and exp(gC) (FP32)
    bf16_t* rec_u;          // [rec][8 vb][64][4] U, BF16
    float* rec_ta;          // [rec][3][16][16] T^T, Akk^T, scale*Aqk
    int rec_pairs;
    DevPlan plan;
    int Hqk, Hv, G;
    int num_tasks;
    int ck_every;           // tape interval (tokens), multiple of 16
    float scale;
    // Chunked kernels: a chunk in which some channel's log2-domain decay sum
    // exceeds precise_log2 runs with hi/lo operands on its whole state path
    // (-inf: every chunk; above 0: none).
    float precise_log2;
    // Training forward (tape or none): split each task's value columns over
    // two workgroups (for calls with few tasks)
    int vsplit;
    // Inference (infer_token_kernel): prologue options and the BF16 state
    // pool [pool_slots][Hv][128][128] read and written in place at slot
    // pool_index[n] (slot n when pool_index is null); s0, s_final and tape
    // are unused.
    int infer;
    int use_qk_l2norm, use_gate_in_kernel, beta_is_logit;
    float lower_bound;
    bf16_t* pool;
    const int32_t* pool_index;
    int64_t pool_slots;
    // inference state checkpoints: the BF16 state before token j*ckpt_every
    // of sequence n goes to row ckpt_start[n] + j of ckpt [rows][Hv][128][128]
    bf16_t* ckpt;           // null: none
    const int64_t* ckpt_start;
    int64_t ckpt_rows;      // rows of ckpt; a row outside [0, ckpt_rows) is not stored
    // Segment-parallel forward: seg_out is [3][segments][Hv][128][128] FP32,
    // the transfer P, offset Q and P transposed of every tape segment
    // (segment index tape_off[n] + n + j), and seg_items = segments * Hv.
    float* seg_out;
    int64_t seg_items;
    int ckpt_every;
    // speculative decode (spec_tokens = S > 0): pool_index is [N][1+S]; the
    // state is read from slot [n][a-1] (a = spec_accepted[n] clamped to
    // [1, 1+S], 1 if null) and written after token s to slot [n][s]
    int spec_tokens;
    const int32_t* spec_accepted;
    // read-only source pool: when set, sequence n starts from its slot
    // src_index[n] instead of its state-pool slot
    const bf16_t* src_pool;
    const int32_t* src_index;
    int64_t src_slots;
};

struct BwdArgs {
    FwdArgs f;              // inputs and plan (o, s_final unused)
    const void* d_o;
    const float* dfinal;
    void* dq; void* dk; void* dv; void* dg; void* dbeta;
    float* dA_log; float* ddt_bias; float* dinit;
    bf16_t* dqk_part;       // [tokens][Hv][2][128] BF16 partial dq,dk when G > 1; else null
    float* dparam_part;     // [tasks][2][128]: per-task ddt_bias and dA_log partial sums
    int64_t total_tokens;
    // Segment-parallel adjoint (seg_pass 1 or 2; 0: whole tasks).  Tasks are
    // tape segments (f.plan.task is the segment list, f.seg_items = segments
    // * Hv; segment index tape_off[n] + n + j).  Pass 1 runs each segment
    // from dS = 0 and stores its start dS to seg_r; a combine chains
    // dS_end(j-1) = dS_end(j) P(j)^T + R(j) into seg_e; pass 2 runs each
    // segment from dfinal (last segment) or seg_e for the gradients, with
    // the parameter partials per segment.  seg_p is the forward's P
    // transposed (row-major P^T).
    int seg_pass;
    const float* seg_p;
    float* seg_r;
    float* seg_e;
};

hipError_t launch_fwd_rowsplit(const FwdArgs& a, hipStream_t s);
hipError_t launch_infer_token(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_chunk(const FwdArgs& a, hipStream_t s);
hipError_t launch_fwd_pipe(const FwdArgs& a, hipStream_t s);
hipError_t launch_state_rebuild(const FwdArgs& a, int64_t num_items, hipStream_t s);
hipError_t launch_fwd_segments(const FwdArgs& a, int N, hipStream_t s);
hipError_t launch_bwd_chunk(const BwdArgs& a, hipStream_t s);
hipError_t launch_bwd_reduce(const BwdArgs& a, int N, hipStream_t s);
hipError_t launch_bwd_segments(const BwdArgs& a, int N, hipStream_t s);

// The static device scratch of kda_fwd_noalloc (KDA_NOALLOC_SCRATCH_BYTES per
// device): its address on device `dev` (found once per device, with `dev`
// current), and a stream-ordered copy of `bytes` (a multiple of 4) of host
// data into it by kernel launches that carry the data as arguments.
hipError_t noalloc_scratch(int dev, void** ptr);
hipError_t upload_to_scratch(void* scratch, const void* host, size_t bytes, hipStream_t s);

}  // namespace kda
