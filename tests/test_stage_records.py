"""Stage parity: the per-chunk quantities of the chunked forward against the
FP64 chunk form of the oracle (oracle.chunk_quantities / chunk_recurrence).

The records context stores, for every 16-token chunk and value head, the
chunk-start state S0 (BF16), U (BF16), and T, Akk, scale*Aqk (FP32).  They are
decoded here from their MFMA fragment layouts and compared stage by stage
with the oracle's chunk form on the same inputs, so that a mistake in one
stage (the triangular solve, the decay factors of Akk or Aqk, the correction
U, the carried state) shows up where it is made rather than only in o.

Record layouts (one record = one (chunk, value head)):
  S0: bf16 [8 kb][8 vb][64 lanes][4]: lane 16gq + k of frag (kb, vb) holds
      S0[16vb + 4gq + i][16kb + k];
  U:  bf16 [8 vb][64 lanes][4]: lane 16gq + c holds U[c][16vb + 4gq + i];
  TA: f32 [3][16][16]: T^T, Akk^T, and Aqk' = scale*Aqk (row-major).
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


def _decode_u(raw):  # raw: bf16 [8*64*4] -> U [16 tokens][128 v]
    x = raw.reshape(8, 4, 16, 4)           # vb, gq, c, i
    u = np.empty((C, D), np.float32)
    for vb in range(8):
        u[:, 16 * vb:16 * vb + 16] = x[vb].transpose(1, 0, 2).reshape(16, 16)
    return u


@pytest.mark.parametrize("precision", [0, 1], ids=["auto", "full"])
def test_records_match_oracle_chunk_form(precision):
    import gated_delta_rule_32_amd as kda
    problem = P([70, 37], 1, 2, packed=True)
    inp = workloads.make_inputs(problem, 310, with_adjoints=False)
    d = inp.to("cuda")
    print(f"[stage] records precision={precision} lengths={problem.lengths}", flush=True)
    o, fs, ctx = kda.recurrent_kda_training_forward(
        d.q, d.k, d.v, d.g, d.beta, d.A_log, d.dt_bias, d.initial_state,
        cu_seqlens=d.cu_seqlens, cu_seqlens_cpu=inp.cu_seqlens, context=kda.CONTEXT_RECORDS,
        precision=precision)
    torch.cuda.synchronize()
    raw = ctx.ctx.cpu().numpy()
    Hv = problem.Hv
    chunks = [-(-L // C) for L in problem.lengths]
    recs = sum(chunks) * Hv
    off_s0 = 256
    off_u = _align256(off_s0 + recs * D * D * 2)
    off_ta = _align256(off_u + recs * C * D * 2)
    as_bf16 = lambda b: torch.from_numpy(b.copy()).view(torch.bfloat16).float().numpy()
    worst = {}
    chunk_off = np.concatenate([[0], np.cumsum(chunks)])
    for (n, b, t0, L) in workloads.sequence_slices(problem):
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
                cs = slice(c * C, min(L, c * C + C))
                m = cs.stop - cs.start
                cq = ko.chunk_quantities(qn[cs], kn[cs], v[cs], lam[cs], bb[cs])
                S0 = states[c]
                U = cq["Ut"] - cq["W"] @ S0.T
                s0 = _decode_s0(as_bf16(raw[off_s0 + rec * D * D * 2:off_s0 + (rec + 1) * D * D * 2]))
                u = _decode_u(as_bf16(raw[off_u + rec * C * D * 2:off_u + (rec + 1) * C * D * 2]))
                ta = raw[off_ta + rec * 3 * C * C * 4:off_ta + (rec + 1) * 3 * C * C * 4].view(np.float32)
                ta = ta.reshape(3, C, C)
                T_gpu = ta[0].T[:m, :m]
                Akk_gpu = ta[1].T[:m, :m]
                Aqk_gpu = ta[2][:m, :m]
                pairs = {"S0": (s0, S0), "U": (u[:m], U), "T": (T_gpu, cq["T"]),
                         "Akk": (Akk_gpu, cq["Akk"]), "Aqk": (Aqk_gpu, ko.SCALE * cq["Aqk"])}
                for name, (x, ref) in pairs.items():
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
