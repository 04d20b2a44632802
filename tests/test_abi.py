"""CPU tests of the C ABI: the library loads, exports every declared entry point,
and rejects malformed calls on the host before any device work (page
"flashinfer.kda_training", paragraphs 1-4, for the rules checked)."""
import ctypes
import math
import os
import re

import pytest
import torch

import gated_delta_rule_32_amd as kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "libkda.h")).read()
    declared = set(re.findall(r"\b(kda_[a-z_]+)\s*\(", hdr))
    assert declared, "no declarations found"
    lib = ctypes.CDLL(kda.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), f"libkda.so does not export {name}"
    assert set(kda.EXPORTED) == declared
    assert kda.kda_version() == 1


def _fixed(**kw):
    base = dict(B=2, T=40, Hqk=2, Hv=4, N=2)
    base.update(kw)
    return kda.make_problem(**base)


def _status(fn, *a):
    with pytest.raises(ValueError) as ei:
        fn(*a)
    return ei.value.status


def test_shape_and_grouping_rejections():
    assert _status(kda.kda_fwd_ctx_bytes, _fixed(Hv=3)) == 3        # grouping
    assert _status(kda.kda_fwd_ctx_bytes, _fixed(T=0)) == 2         # shape
    assert _status(kda.kda_fwd_ctx_bytes, _fixed(N=3)) == 2         # fixed needs N == B


def test_scale_and_lower_bound_rejections():
    assert _status(kda.kda_fwd_ctx_bytes, _fixed(scale=0.1)) == 5
    assert _status(kda.kda_fwd_ctx_bytes, _fixed(lower_bound=-4.0)) == 6
    # None / exact value accepted
    kda.kda_fwd_ctx_bytes(_fixed(scale=1.0 / math.sqrt(128.0)))


def test_route_and_checkpoint_rejections():
    assert _status(kda.kda_fwd_ctx_bytes, _fixed(route=7)) == 11
    assert _status(kda.kda_fwd_ctx_bytes, _fixed(checkpoint_every=24)) == 11


def _packed(cu, Hqk=1, Hv=2):
    cu_cpu = torch.tensor(cu, dtype=torch.int64)
    # a dummy non-null "device" pointer: validation never dereferences it
    p = kda.make_problem(1, cu[-1], Hqk, Hv, len(cu) - 1, None, cu_cpu)
    p.cu_seqlens = 0x1000
    return p, cu_cpu


def test_seqlens_rejections():
    for cu in ([1, 5, 9], [0, 5, 5, 9], [0, 6, 4, 9], [0, 4, 8]):
        p, keep = _packed(cu)
        if cu == [0, 4, 8]:
            p.T = 9  # does not end at T
        assert _status(kda.kda_fwd_ctx_bytes, p) == 4
    p, keep = _packed([0, 4, 9])
    p.B = 2
    assert _status(kda.kda_fwd_ctx_bytes, p) == 2
    p, keep = _packed([0, 4, 9])
    p.cu_seqlens = None
    assert _status(kda.kda_fwd_ctx_bytes, p) == 1


def test_context_and_workspace_sizes():
    cu = [0, 300, 301, 812]
    p, keep = _packed(cu, Hqk=1, Hv=2)
    # checkpoints strictly inside each sequence every 256 tokens:
    # 300 -> 1, 1 -> 0, 511 -> 1
    assert kda.kda_fwd_ctx_bytes(p) == 256 + 2 * 2 * 128 * 128 * 4
    p.checkpoint_every = 64
    p.route = kda.ROUTE_CHUNK
    n_ck = (300 + 63) // 64 - 1 + 0 + (511 + 63) // 64 - 1
    tape = n_ck * 2 * 128 * 128 * 4
    assert kda.kda_fwd_ctx_bytes(p) == 256 + tape
    # with 5 + 1 + 8 segments (2 x 14 x 2 <= 768) and the longest sequence
    # spanning 8 of them, AUTO takes the segment-parallel route, whose context
    # adds P, Q and P transposed of every segment after the tape (256-byte aligned)
    p.route = kda.ROUTE_AUTO
    assert kda.kda_plan_query(p)[0] == kda.ROUTE_SEGMENTS
    segs = 5 + 1 + 8
    assert kda.kda_fwd_ctx_bytes(p) == (256 + tape + 255) // 256 * 256 + 3 * segs * 2 * 128 * 128 * 4
    p.route = kda.ROUTE_CHUNK
    # chunk records per sequence, rounded up to even: 19 -> 20, 1 -> 2, 32
    chunks = sum(((L + 15) // 16 + 1) // 2 * 2 for L in (300, 1, 511))
    assert chunks == 54
    ws = kda.kda_bwd_workspace_bytes(p)
    # per (chunk, value head): BF16 chunk-start state, BF16 U, FP32 T/Akk/Aqk
    # (6 tasks: no pair records); BF16 dq/dk partials per token and value
    # head (G = 2); per-task partials
    rec = 128 * 128 * 2 + 16 * 128 * 2 + 3 * 16 * 16 * 4
    tasks = 3 * 2
    need = chunks * 2 * rec + 812 * 2 * 2 * 128 * 2 + tasks * 2 * 128 * 4
    assert need <= ws <= need + 16 * 256


def test_longest_first_order():
    """Tasks of longer sequences come first; within a sequence, heads in order
    (page "flashinfer.kda.recurrent_kda", parameter cu_seqlens)."""
    cu = [0, 5, 105, 108, 300]
    p, keep = _packed(cu, Hqk=1, Hv=2)
    route, nt, order = kda.kda_plan_query(p, with_order=True)
    assert nt == 8
    lens = [5, 100, 3, 192]
    seqs = [o // 2 for o in order]
    assert [lens[s] for s in seqs] == sorted([lens[s] for s in seqs], reverse=True)
    assert order == [6, 7, 2, 3, 0, 1, 4, 5]
    # sequence order on request (for measuring what longest-first buys)
    p.schedule = kda.SCHEDULE_SEQUENCE
    assert kda.kda_plan_query(p, with_order=True)[2] == list(range(8))
    p.schedule = 2
    assert _status(kda.kda_fwd_ctx_bytes, p) == 11


def test_route_choice():
    # the chunked kernel at every task count, its column split for 128 tasks
    # or fewer (two workgroups each); the row-split one on request
    assert kda.kda_plan_query(_fixed())[0] == kda.ROUTE_CHUNK_SPLIT
    assert kda.kda_plan_query(kda.make_problem(8, 64, 16, 16, 8))[0] == kda.ROUTE_CHUNK_SPLIT
    assert kda.kda_plan_query(kda.make_problem(8, 64, 16, 32, 8))[0] == kda.ROUTE_CHUNK
    # few tasks with long sequences: the segment-parallel route once the
    # longest sequence spans more than 4 tape segments, the column split
    # up to that
    assert kda.kda_plan_query(kda.make_problem(2, 2048, 16, 16, 2))[0] == kda.ROUTE_SEGMENTS
    assert kda.kda_plan_query(kda.make_problem(8, 1024, 12, 12, 8))[0] == kda.ROUTE_CHUNK_SPLIT
    assert kda.kda_plan_query(kda.make_problem(8, 1024, 24, 24, 8))[0] == kda.ROUTE_CHUNK
    assert kda.kda_plan_query(_fixed(route=2))[0] == kda.ROUTE_ROWSPLIT
    assert kda.kda_plan_query(_fixed(route=1))[0] == kda.ROUTE_CHUNK
    assert kda.kda_plan_query(_fixed(route=4))[0] == kda.ROUTE_CHUNK_SPLIT
    # the per-chunk records need the unsplit kernel
    p = _fixed(context=kda.CONTEXT_RECORDS)
    assert kda.kda_plan_query(p)[0] == kda.ROUTE_CHUNK
    assert _status(kda.kda_plan_query, _fixed(context=kda.CONTEXT_RECORDS, route=4)) == 11
    assert _status(kda.kda_plan_query, _fixed(route=5)) == 11


def test_forward_rejects_overlap_and_null_before_device_work():
    p = _fixed(B=1, T=16, Hqk=1, Hv=1, N=1)
    nb = 16 * 128 * 2
    base = 0x10000000
    q, k, v, g = base, base + nb, base + 2 * nb, base + 3 * nb
    beta, A, dtb = base + 4 * nb, base + 5 * nb, base + 6 * nb
    s0 = base + 8 * nb
    fs = base + 8 * nb + 65536
    o_ok = base + 100 * nb
    lib = kda._lib
    pr = ctypes.byref(p)
    # o overlaps v
    st = lib.kda_fwd(pr, q, k, v, g, beta, A, dtb, s0, v + 64, fs, None, 0, None)
    assert st == 7
    # final state overlaps initial state
    st = lib.kda_fwd(pr, q, k, v, g, beta, A, dtb, s0, o_ok, s0 + 4, None, 0, None)
    assert st == 7
    # null input
    st = lib.kda_fwd(pr, None, k, v, g, beta, A, dtb, s0, o_ok, fs, None, 0, None)
    assert st == 1
    # context too small
    st = lib.kda_fwd(pr, q, k, v, g, beta, A, dtb, s0, o_ok, fs, base + 400 * nb, 16, None)
    assert st == 8
    assert "context" in kda.kda_last_error()


def test_backward_rejects_unknown_context():
    p = _fixed(B=1, T=16, Hqk=1, Hv=1, N=1)
    ws = kda.kda_bwd_workspace_bytes(p)
    args = [0x10000000 + i * 0x100000 for i in range(22)]
    lib = kda._lib
    st = lib.kda_bwd(ctypes.byref(p), *args[:8], args[8], 1 << 20, args[9], args[10],
                     *args[11:19], args[19], ws, None)
    # no forward recorded this context: rejected (after no device work besides
    # querying the current device, which may itself fail on a GPU-less host)
    assert st in (9, 12)


def test_sequence_span_limit():
    """Kernels address a sequence's rows with 32-bit element offsets: a
    sequence of L tokens over Hv heads needs L * Hv * 128 < 2^31."""
    p, keep = _packed([0, 1 << 18], Hqk=64, Hv=64)   # 2^18 * 64 * 128 = 2^31
    assert _status(kda.kda_fwd_ctx_bytes, p) == 2
    p, keep = _packed([0, (1 << 18) - 1], Hqk=64, Hv=64)
    kda.kda_fwd_ctx_bytes(p)
    p = _fixed(T=1 << 18, Hqk=64, Hv=64)
    assert _status(kda.kda_fwd_ctx_bytes, p) == 2


def test_records_context_sizes_and_rejections():
    """Records context: one record per (16-token chunk, value head), each
    sequence's chunks rounded up to an even count, after a 256-byte header;
    with more than 256 tasks the chunk-start state only per (chunk pair,
    value head), with the even chunk's column-layout U and Kt and exp(gC).
    The backward workspace then holds no records."""
    cu = [0, 300, 301, 812]
    chunks = sum(((L + 15) // 16 + 1) // 2 * 2 for L in (300, 1, 511))
    per_chunk = 16 * 128 * 2 + 3 * 16 * 16 * 4          # U, T/Akk/Aqk
    s0 = 128 * 128 * 2
    step = 2 * 16 * 128 * 2 + 128 * 4                    # CF(U), CF(Kt), exp(gC)
    for Hv, pairs in ((2, False), (96, True)):           # 6 and 288 tasks
        p, keep = _packed(cu, Hqk=Hv // 2, Hv=Hv)
        ws_tape = kda.kda_bwd_workspace_bytes(p)
        p.context = kda.CONTEXT_RECORDS
        recs = chunks * Hv
        rec_bytes = recs * per_chunk + (recs // 2 * (s0 + step) if pairs else recs * s0)
        ctx = kda.kda_fwd_ctx_bytes(p)
        need = 256 + rec_bytes
        assert need <= ctx <= need + 4 * 256
        ws_rec = kda.kda_bwd_workspace_bytes(p)
        assert ws_rec + rec_bytes <= ws_tape <= ws_rec + rec_bytes + 4 * 256
    p, keep = _packed(cu, Hqk=1, Hv=2)
    p.context = kda.CONTEXT_RECORDS
    p.route = 2
    assert _status(kda.kda_fwd_ctx_bytes, p) == 11      # records need the chunked route
    p.route = 0
    p.context = 5
    assert _status(kda.kda_fwd_ctx_bytes, p) == 11      # unknown context kind


def test_pair_records_threshold():
    """Pair records (the start state of every other chunk) from 257 tasks on,
    on the chunked routes; a start state per chunk up to 256 tasks and on the
    segment-parallel route, for any task count."""
    per_chunk = 16 * 128 * 2 + 3 * 16 * 16 * 4
    s0 = 128 * 128 * 2
    step = 2 * 16 * 128 * 2 + 128 * 4

    def records(N, Hv, pairs, chunks=2):
        recs = N * chunks * Hv
        return recs * per_chunk + (recs // 2 * (s0 + step) if pairs else recs * s0)

    for Hv, pairs in ((64, False), (128, True)):        # 4 x 64 = 256, 4 x 128 = 512 tasks
        p = kda.make_problem(4, 32, Hv, Hv, 4, context=kda.CONTEXT_RECORDS, route=kda.ROUTE_CHUNK)
        need = 256 + records(4, Hv, pairs)
        assert need <= kda.kda_fwd_ctx_bytes(p) <= need + 4 * 256
    # tape context with 512 tasks: the rebuilt records in the workspace are
    # pair records on the chunked route (G = 1: no dq/dk partials; per-task
    # parameter partials) ...
    p1 = kda.make_problem(4, 32, 128, 128, 4, route=kda.ROUTE_CHUNK)
    need = records(4, 128, True) + 512 * 2 * 128 * 4
    assert need <= kda.kda_bwd_workspace_bytes(p1) <= need + 8 * 256
    # ... and a start state per chunk on the segment-parallel route (16-token
    # segments: 8 segments x 128 heads of parameter partials, R and dS_end)
    p3 = kda.make_problem(4, 32, 128, 128, 4, route=kda.ROUTE_SEGMENTS, checkpoint_every=16)
    need = records(4, 128, False) + 1024 * 2 * 128 * 4 + 2 * 1024 * 128 * 128 * 4
    assert need <= kda.kda_bwd_workspace_bytes(p3) <= need + 8 * 256


def test_status_strings_cover_every_code():
    hdr = open(os.path.join(ROOT, "include", "libkda.h")).read()
    codes = {name: int(val) for name, val in re.findall(r"\b(KDA_(?:OK|ERR_[A-Z_]+))\s*=\s*(\d+)", hdr)}
    assert codes["KDA_ERR_CAPTURE"] == kda.KDA_ERR_CAPTURE and codes["KDA_ERR_HIP"] == kda.KDA_ERR_HIP
    texts = {kda.kda_status_string(c) for c in codes.values()}
    assert len(texts) == len(codes), "two status codes share a description"
    assert kda.kda_status_string(max(codes.values()) + 1) not in texts


def test_infer_rejections_before_device_work():
    """kda_infer checks its options, pool indices and buffers on the host
    (page "flashinfer.kda.recurrent_kda", parameters)."""
    lib = kda._lib
    nb = 16 * 128 * 2
    base = 0x10000000
    q, k, v, g, beta = (base + i * nb for i in range(5))
    A, dtb = base + 6 * nb, base + 7 * nb
    pool = base + 64 * nb
    o = base + 2000 * nb

    def call(p, A_ptr=A, o_ptr=o, pool_ptr=pool):
        return lib.kda_infer(ctypes.byref(p), q, k, v, g, beta, A_ptr, dtb, pool_ptr, o_ptr, None)

    def prob(**kw):
        base_kw = dict(B=1, T=16, Hqk=1, Hv=1, N=1, pool_slots=1)
        base_kw.update(kw)
        return kda.make_infer_problem(**base_kw)

    # in-kernel gate needs a lower bound (softplus form not implemented) and A_log
    assert call(prob(use_gate_in_kernel=True)) == 6
    assert call(prob(use_gate_in_kernel=True, lower_bound=2.0)) == 6
    assert call(prob(use_gate_in_kernel=True, lower_bound=-3.0), A_ptr=None) == 1
    # routes: unknown, or the chunked one with a gate it cannot bound
    assert call(prob(route=3)) == 11
    assert call(prob(use_gate_in_kernel=True, lower_bound=-6.0, route=1)) == 11
    # a log-space gate (no bound the host can check) on the chunked route
    assert call(prob(route=1)) == 11
    assert call(prob(use_gate_in_kernel=False, route=1)) == 11
    # scale must be positive
    assert call(prob(scale=-1.0)) == 5
    # option flags are 0 or 1
    p = prob()
    p.beta_is_logit = 2
    assert call(p) == 2
    # pool too small for slot n without indices
    assert call(kda.make_infer_problem(B=2, T=16, Hqk=1, Hv=1, N=2, pool_slots=1)) == 2
    # indices: out of range, repeated, or without their host mirror
    cu = torch.tensor([0, 5, 16], dtype=torch.int64)
    for bad in ([0, 3], [1, 1], [-1, 0]):
        idx = torch.tensor(bad, dtype=torch.int32)
        p = kda.make_infer_problem(1, 16, 1, 1, 2, 3, cu, cu, state_indices=idx,
                                   state_indices_cpu=idx)
        assert call(p) == 2, bad
    idx = torch.tensor([2, 0], dtype=torch.int32)
    p = kda.make_infer_problem(1, 16, 1, 1, 2, 3, cu, cu, state_indices=idx)
    assert call(p) == 1
    # output overlapping the pool or an input
    assert call(prob(), o_ptr=pool + 64) == 7
    assert call(prob(), o_ptr=v) == 7
    assert call(prob(), pool_ptr=q + 2) == 7


def test_infer_checkpoint_rejections():
    """State checkpoints: interval, per-sequence counts and capacity are
    checked on the host (page "flashinfer.kda.recurrent_kda", parameters
    state_checkpoints, checkpoint_cu_starts, checkpoint_every_n_tokens)."""
    lib = kda._lib
    nb = 16 * 128 * 2
    base = 0x10000000
    q, k, v, g, beta = (base + i * nb for i in range(5))
    pool, o = base + 64 * nb, base + 2000 * nb
    ckbuf = torch.empty((3, 1, 128, 128), dtype=torch.bfloat16)   # host memory: never touched
    cu = torch.tensor([0, 5, 40], dtype=torch.int64)             # lengths 5 and 35

    def call(every, starts, rows=3):
        p = kda.make_infer_problem(1, 40, 1, 1, 2, 2, cu, cu, checkpoint_every=every,
                                   state_checkpoints=ckbuf[:rows] if rows else None,
                                   checkpoint_cu_starts=starts, checkpoint_cu_starts_cpu=starts)
        return lib.kda_infer(ctypes.byref(p), q, k, v, g, beta, None, None, pool, o, None)

    good = torch.tensor([0, 1, 4], dtype=torch.int64)           # ceil(5/16)=1, ceil(35/16)=3
    assert call(24, good) == 11                                  # not a multiple of 16
    assert call(16, torch.tensor([0, 1, 3], dtype=torch.int64)) == 4   # wrong count
    assert call(16, torch.tensor([1, 2, 5], dtype=torch.int64)) == 4   # not starting at 0
    assert call(16, good, rows=3) == 2                           # 4 rows needed, 3 given
    # checkpoint fields without an interval
    p = kda.make_infer_problem(1, 40, 1, 1, 2, 2, cu, cu, state_checkpoints=ckbuf)
    assert lib.kda_infer(ctypes.byref(p), q, k, v, g, beta, None, None, pool, o, None) == 11


def test_infer_spec_decode_rejections():
    """Speculative decode needs 1+S tokens and 1+S distinct slots per
    sequence, the token-serial route and no checkpoints."""
    lib = kda._lib
    nb = 16 * 128 * 2
    base = 0x10000000
    q, k, v, g, beta = (base + i * nb for i in range(5))
    pool, o = base + 64 * nb, base + 2000 * nb
    cu = torch.tensor([0, 3, 6], dtype=torch.int64)              # two sequences of 3 tokens
    idx = torch.tensor([0, 1, 2, 3, 4, 5], dtype=torch.int32)

    def call(**kw):
        base_kw = dict(state_indices=idx, state_indices_cpu=idx, num_spec_tokens=2)
        base_kw.update(kw)
        p = kda.make_infer_problem(1, 6, 1, 1, 2, 8, cu, cu, **base_kw)
        return lib.kda_infer(ctypes.byref(p), q, k, v, g, beta, None, None, pool, o, None)

    assert call(num_spec_tokens=3) == 4                          # sequences are not 1+S long
    assert call(state_indices=None, state_indices_cpu=None) == 1
    assert call(route=1) == 11
    dup = torch.tensor([0, 1, 2, 3, 4, 0], dtype=torch.int32)
    assert call(state_indices=dup, state_indices_cpu=dup) == 2
    acc = torch.zeros(2, dtype=torch.int32)
    assert call(num_spec_tokens=0, num_accepted_tokens=acc, state_indices=idx[:2],
                state_indices_cpu=idx[:2]) == 2


def test_infer_source_pool_rejections():
    lib = kda._lib
    nb = 16 * 128 * 2
    base = 0x10000000
    q, k, v, g, beta = (base + i * nb for i in range(5))
    pool, o, srcp = base + 64 * nb, base + 2000 * nb, base + 3000 * nb
    sidx = torch.tensor([0, 3], dtype=torch.int32)
    cu = torch.tensor([0, 5, 16], dtype=torch.int64)

    def call(src, idx_dev, idx_host, slots=2):
        p = kda.make_infer_problem(1, 16, 1, 1, 2, 2, cu, cu)
        p.state_source, p.source_slots = src, slots
        p.source_indices = None if idx_dev is None else idx_dev.data_ptr()
        p.source_indices_host = None if idx_host is None else idx_host.data_ptr()
        return lib.kda_infer(ctypes.byref(p), q, k, v, g, beta, None, None, pool, o, None)

    assert call(srcp, sidx, sidx) == 2                     # slot 3 outside 2 slots
    assert call(srcp, None, None) == 1                     # source without indices
    assert call(None, sidx, sidx) == 1                     # indices without source
    assert call(pool + 16, sidx, sidx, slots=4) == 7      # source overlaps the state pool


def test_problem_keeps_its_offsets_alive():
    """The problem structs hold raw pointers to cu_seqlens and the other index
    tensors: they keep those tensors alive, so a problem made in a helper is
    still valid after the helper's tensors went out of scope."""
    import gc

    def make():
        cu = torch.tensor([0, 3, 40, 41], dtype=torch.int64)
        return kda.make_problem(1, 41, 1, 2, 3, cu, cu.clone())

    p = make()
    gc.collect()
    junk = [torch.full((4,), -7, dtype=torch.int64) for _ in range(256)]  # reuse freed memory
    route, ntasks, order = kda.kda_plan_query(p, with_order=True)
    assert ntasks == 6 and order[:2] == [2, 3]   # sequence 1 (37 tokens) first
    del junk
    ip = kda.make_infer_problem(1, 41, 1, 2, 3, 8, torch.tensor([0, 3, 40, 41], dtype=torch.int64),
                                torch.tensor([0, 3, 40, 41], dtype=torch.int64),
                                state_indices=torch.tensor([5, 1, 2], dtype=torch.int32),
                                state_indices_cpu=torch.tensor([5, 1, 2], dtype=torch.int32))
    gc.collect()
    assert all(t is not None for t in ip._keep[:4])
