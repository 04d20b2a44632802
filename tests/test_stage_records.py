"""Stage parity: the per-chunk quantities of the chunked forward against the
FP64 chunk form of the oracle (oracle.chunk_quantities / chunk_recurrence).

The records context stores, for every 16-token chunk and value head, U
(BF16) and T, Akk, scale*Aqk (FP32), and the chunk-start state S0 (BF16): for
every chunk with up to 256 tasks, otherwise for every pair of chunks (2p,
2p+1) the start state of chunk 2p with what steps it to chunk 2p+1 (U and Kt
of chunk 2p in the column layout, BF16, and exp(gC)).  They are decoded here
from their MFMA fragment layouts and compared stage by stage with the
oracle's FP64 chunk form on the same inputs, so that a mistake in one stage
(the triangular solve, the decay factors of Akk or Aqk, the correction U, the
carried state) shows up where it is made rather than only in o.  The odd
chunks' start states are formed from the pair record as the adjoint forms
them, S0(2p+1) = S0(2p) diag(exp(gC)) + U^T Kt (here in FP64 from the stored
values), and compared with the oracle's.

Record layouts (per chunk record = (chunk, value head); per pair record =
(chunk pair, value head); each sequence has an even number of chunk records):
  S0: bf16 [8 kb][8 vb][64 lanes][4] per chunk or per pair: lane 16gq + k of
      frag (kb, vb) holds S0[16vb + 4gq + i][16kb + k];
  X:  per pair (pair records only): bf16 CF(U) [8 vb][64 lanes][4] (lane 16gq + c holds
      U[4gq + i][16vb + c]), bf16 CF(Kt) [8 kb][64 lanes][4] (lane 16gq + k
      holds Kt[4gq + i][16kb + k]), then f32 exp(gC) [128];
  U:  bf16 [8 vb][64 lanes][4] per chunk: lane 16gq + c holds U[c][16vb + 4gq + i];
  TA: f32 [3][16][16] per chunk: T^T, Akk^T, and Aqk' = scale*Aqk (row-major).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from oracle import kda_oracle as ko
from tests import parity_util as pu

pytestmark = pytest.mark.gpu

P = workloads.Problem
D, C = 128, 16


def _align256(x):
    return (x + 255) & ~255


def _decode_s0(raw):  # raw: bf16 [8*8*64*4] -> S0 [128 v][128 k]
    x = raw.reshape(8, 8, 4, 16, 4)       # kb, vb, gq, k, i
    s = np.empty((D, D), np.float32)
    for kb in range(8):
        for vb in range(8):
            # rows v = 16vb + 4gq + i, columns k = 16kb + k
            blk = x[kb, vb].transpose(0, 2, 1).reshape(16, 16)  # (gq, i) x k
            s[16 * vb:16 * vb + 16, 16 * kb:16 * kb + 16] = blk
    return s


def _decode_cf(raw):  # raw: bf16 [8*64*4] -> X [16 tokens][128] from CF frags
    x = raw.reshape(8, 4, 16, 4)           # block, gq, column, i
    out = np.empty((C, D), np.float32)
    for b in range(8):
        # rows 4gq + i, columns 16b + column
        out[:, 16 * b:16 * b + 16] = x[b].transpose(0, 2, 1).reshape(16, 16)
    return out


def _decode_u(raw):  # raw: bf16 [8*64*4] -> U [16 tokens][128 v]
    x = raw.reshape(8, 4, 16, 4)           # vb, gq, c, i
    u = np.empty((C, D), np.float32)
    for vb in range(8):
        u[:, 16 * vb:16 * vb + 16] = x[vb].transpose(1, 0, 2).reshape(16, 16)
    return u


# (problem, sequences checked): up to 256 tasks every chunk stores its start
# state; beyond, pair records (the 20-token sequences end in an odd tail chunk,
# whose start state comes from its pair)
LAYOUTS = {
    "chunk_records": (P([70, 37], 1, 2, packed=True), [0, 1]),
    "pair_records": (P([70, 37] + [20] * 127, 1, 2, packed=True), [0, 1, 2, 128]),
}


@pytest.mark.parametrize("precision", [0, 1], ids=["auto", "full"])
@pytest.mark.parametrize("layout", list(LAYOUTS.keys()))
def test_records_match_oracle_chunk_form(layout, precision):
    import gated_delta_rule_32_amd as kda
    problem, checked = LAYOUTS[layout]
    inp = workloads.make_inputs(problem, 310, with_adjoints=False)
    d = inp.to("cuda")
    print(f"[stage] {layout} precision={precision} sequences={problem.N}", flush=True)
    o, fs, ctx = kda.recurrent_kda_training_forward(
        d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
        cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=inp.cu_seqlens, context=kda.CONTEXT_RECORDS,
        precision=precision)
    torch.cuda.synchronize()
    raw = ctx.ctx.cpu().numpy()
    Hv = problem.Hv
    chunks = [-(-L // C) for L in problem.lengths]
    padded = [c + (c & 1) for c in chunks]
    recs = sum(padded) * Hv
    use_pairs = problem.N * Hv > 256
    assert use_pairs == (layout == "pair_records")
    s0_recs = recs // 2 if use_pairs else recs
    X_BYTES = (2 * 2048 + 2 * 128) * 2
    off_s0 = 256
    off_x = _align256(off_s0 + s0_recs * D * D * 2)
    off_u = _align256(off_x + (recs // 2 if use_pairs else 0) * X_BYTES)
    off_ta = _align256(off_u + recs * C * D * 2)
    as_bf16 = lambda b: torch.from_numpy(b.copy()).view(torch.bfloat16).float().numpy()
    worst = {}
    chunk_off = np.concatenate([[0], np.cumsum(padded)])
    for (n, b, t0, L) in workloads.sequence_slices(problem):
        if n not in checked:
            continue
        for h in range(Hv):
            hq = h // (Hv // problem.Hqk)
            s = slice(t0, t0 + L)
            qn, kn, lam, alpha, bb, z = ko.prologue(
                inp.q[b, s, hq].double().numpy(), inp.k[b, s, hq].double().numpy(),
                inp.g[b, s, h].double().numpy(), inp.beta[b, s, h].double().numpy(),
                float(inp.A_log[h]), inp.dt_bias[h].double().numpy())
            v = inp.v[b, s, h].double().numpy()
            _, _, states = ko.chunk_recurrence(qn, kn, v, lam, bb,
                                               inp.initial_state[n, h].double().numpy(), C,
                                               keep_states=True)
            for c in range(chunks[n]):
                rec = (int(chunk_off[n]) + c) * Hv + h
                prec = ((int(chunk_off[n]) + c) // 2) * Hv + h if use_pairs else rec
                cs = slice(c * C, min(L, c * C + C))
                m = cs.stop - cs.start
                cq = ko.chunk_quantities(qn[cs], kn[cs], v[cs], lam[cs], bb[cs])
                S0 = states[c]
                U = cq["Ut"] - cq["W"] @ S0.T
                s0p = _decode_s0(as_bf16(raw[off_s0 + prec * D * D * 2:
                                             off_s0 + (prec + 1) * D * D * 2])).astype(np.float64)
                s0, extra = s0p, {}
                if use_pairs:
                    xr = raw[off_x + prec * X_BYTES:off_x + (prec + 1) * X_BYTES]
                    xu = _decode_cf(as_bf16(xr[:4096])).astype(np.float64)
                    xk = _decode_cf(as_bf16(xr[4096:8192])).astype(np.float64)
                    xg = xr[8192:].view(np.float32).astype(np.float64)
                    if c % 2 == 0:
                        # what steps the state to the odd chunk after this one
                        extra = {"U (column layout)": (xu[:m], U), "Kt": (xk[:m], cq["Kt"]),
                                 "exp(gC)": (xg, np.exp(cq["gC"]))}
                        assert np.all(xu[m:] == 0.0) and np.all(xk[m:] == 0.0)
                    else:
                        # the odd chunk's start state as the adjoint forms it
                        s0 = s0p * xg[None, :] + xu.T @ xk
                u = _decode_u(as_bf16(raw[off_u + rec * C * D * 2:off_u + (rec + 1) * C * D * 2]))
                ta = raw[off_ta + rec * 3 * C * C * 4:off_ta + (rec + 1) * 3 * C * C * 4].view(np.float32)
                ta = ta.reshape(3, C, C)
                T_gpu = ta[0].T[:m, :m]
                Akk_gpu = ta[1].T[:m, :m]
                Aqk_gpu = ta[2][:m, :m]
                stages = {"S0": (s0, S0), "U": (u[:m], U), "T": (T_gpu, cq["T"]),
                          "Akk": (Akk_gpu, cq["Akk"]), "Aqk": (Aqk_gpu, ko.SCALE * cq["Aqk"]), **extra}
                for name, (x, ref) in stages.items():
                    viol, fr, mx, fviol = pu.errors(x, ref)
                    worst[name] = max(worst.get(name, 0.0), viol)
                    assert viol <= 1.0 and fviol <= 1.0, \
                        f"{name} of chunk {c} (n={n}, h={h}): worst ratio {viol:.3g}, rel-frob {fr:.3g}"
                # padding rows of a tail chunk's U are zero
                assert np.all(u[m:] == 0.0)
    print("  worst elementwise ratios: " + ", ".join(f"{k} {v:.3g}" for k, v in worst.items()),
          flush=True)
    # the records forward's own outputs
    ref_o, ref_s = pu.oracle_forward(inp)
    pu.assert_close("o", o.float().cpu().numpy(), ref_o)
    pu.assert_state_close("final_state", fs.cpu().numpy(), ref_s)
