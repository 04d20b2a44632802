"""Python binding of libkda, the MI355X (gfx950) KDA training recurrence.

Argument marshalling only: every step of the computation runs in the HIP
kernels of libkda.so, called through its C ABI (include/libkda.h).  PyTorch
supplies device memory and the current stream.

Low-level functions carry the C names (kda_fwd, kda_bwd, kda_fwd_ctx_bytes,
kda_bwd_workspace_bytes, kda_plan_query, kda_status_string, kda_last_error,
kda_version, kda_infer).  The paired training API mirrors the FlashInfer pages
"flashinfer.kda_training.recurrent_kda_training_forward" and
"flashinfer.kda_training" (recurrent_kda_training_backward); recurrent_kda
covers the decode/prefill subset of page "flashinfer.kda.recurrent_kda"
(gate, beta and norm options; a BF16 state pool updated in place).

The library must be built first (``python -m gated_delta_rule_32_amd.build_lib``);
importing this package without it raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkda.so")
HEAD_DIM = 128
SCALE = 1.0 / math.sqrt(128.0)

KDA_OK = 0
KDA_ERR_HIP = 12
KDA_ERR_CAPTURE = 13
ROUTE_AUTO, ROUTE_CHUNK, ROUTE_ROWSPLIT, ROUTE_SEGMENTS, ROUTE_CHUNK_SPLIT = 0, 1, 2, 3, 4
CONTEXT_TAPE, CONTEXT_RECORDS = 0, 1
PRECISION_AUTO, PRECISION_FULL, PRECISION_FAST = 0, 1, 2
SCHEDULE_LONGEST_FIRST, SCHEDULE_SEQUENCE = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libkda.so not found at {LIB_PATH}; build it with "
        "`python gated_delta_rule_32_amd/build_lib.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)


class KdaProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hqk", ctypes.c_int32),
        ("Hv", ctypes.c_int32), ("N", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
        ("scale", ctypes.c_float), ("lower_bound", ctypes.c_float),
        ("route", ctypes.c_int32), ("checkpoint_every", ctypes.c_int32),
        ("context", ctypes.c_int32), ("precision", ctypes.c_int32),
        ("schedule", ctypes.c_int32),
    ]


class KdaInferProblem(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32), ("T", ctypes.c_int32), ("Hqk", ctypes.c_int32),
        ("Hv", ctypes.c_int32), ("N", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p), ("cu_seqlens_host", ctypes.c_void_p),
        ("scale", ctypes.c_float), ("use_qk_l2norm", ctypes.c_int32),
        ("use_gate_in_kernel", ctypes.c_int32), ("lower_bound", ctypes.c_float),
        ("beta_is_logit", ctypes.c_int32), ("route", ctypes.c_int32),
        ("pool_slots", ctypes.c_int64),
        ("state_indices", ctypes.c_void_p), ("state_indices_host", ctypes.c_void_p),
        ("checkpoint_every", ctypes.c_int32), ("state_checkpoints", ctypes.c_void_p),
        ("checkpoint_rows", ctypes.c_int64), ("checkpoint_cu_starts", ctypes.c_void_p),
        ("checkpoint_cu_starts_host", ctypes.c_void_p),
        ("num_spec_tokens", ctypes.c_int32), ("num_accepted_tokens", ctypes.c_void_p),
        ("state_source", ctypes.c_void_p), ("source_slots", ctypes.c_int64),
        ("source_indices", ctypes.c_void_p), ("source_indices_host", ctypes.c_void_p),
    ]


_P = ctypes.POINTER(KdaProblem)
_vp = ctypes.c_void_p
_lib.kda_version.restype = ctypes.c_int
_lib.kda_status_string.restype = ctypes.c_char_p
_lib.kda_status_string.argtypes = [ctypes.c_int]
_lib.kda_last_error.restype = ctypes.c_char_p
_lib.kda_fwd_ctx_bytes.restype = ctypes.c_int
_lib.kda_fwd_ctx_bytes.argtypes = [_P, ctypes.POINTER(ctypes.c_size_t)]
_lib.kda_bwd_workspace_bytes.restype = ctypes.c_int
_lib.kda_bwd_workspace_bytes.argtypes = [_P, ctypes.POINTER(ctypes.c_size_t)]
_lib.kda_plan_query.restype = ctypes.c_int
_lib.kda_plan_query.argtypes = [_P, ctypes.POINTER(ctypes.c_int32),
                                ctypes.POINTER(ctypes.c_int64), _vp, ctypes.c_int64]
_lib.kda_fwd.restype = ctypes.c_int
_lib.kda_fwd.argtypes = [_P] + [_vp] * 10 + [_vp, ctypes.c_size_t, _vp]
_lib.kda_fwd_noalloc.restype = ctypes.c_int
_lib.kda_fwd_noalloc.argtypes = [_P] + [_vp] * 10 + [_vp, ctypes.c_size_t, _vp]
_lib.kda_bwd.restype = ctypes.c_int
_lib.kda_bwd.argtypes = ([_P] + [_vp] * 8 + [_vp, ctypes.c_size_t] + [_vp] * 2 + [_vp] * 8
                         + [_vp, ctypes.c_size_t, _vp])

_lib.kda_infer.restype = ctypes.c_int
_lib.kda_infer.argtypes = [ctypes.POINTER(KdaInferProblem)] + [_vp] * 10

EXPORTED = ("kda_version", "kda_status_string", "kda_last_error", "kda_fwd_ctx_bytes",
            "kda_bwd_workspace_bytes", "kda_plan_query", "kda_fwd", "kda_bwd", "kda_infer",
            "kda_fwd_noalloc")
NOALLOC_SCRATCH_BYTES = 4 << 20  # KDA_NOALLOC_SCRATCH_BYTES


class KdaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{kda_status_string(status)}: {msg}")
        self.status = status


class KdaValueError(ValueError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{kda_status_string(status)}: {msg}")
        self.status = status


def kda_version() -> int:
    return int(_lib.kda_version())


def kda_status_string(status: int) -> str:
    return _lib.kda_status_string(int(status)).decode()


def kda_last_error() -> str:
    return _lib.kda_last_error().decode()


def _check(status: int):
    if status == KDA_OK:
        return
    msg = kda_last_error()
    if status == KDA_ERR_HIP:
        raise KdaError(status, msg)
    raise KdaValueError(status, msg)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def make_problem(B: int, T: int, Hqk: int, Hv: int, N: int,
                 cu_seqlens: Optional[torch.Tensor] = None,
                 cu_seqlens_cpu: Optional[torch.Tensor] = None,
                 scale: Optional[float] = None, lower_bound: float = -5.0,
                 route: int = ROUTE_AUTO, checkpoint_every: int = 0,
                 context: int = CONTEXT_TAPE, precision: int = PRECISION_AUTO,
                 schedule: int = SCHEDULE_LONGEST_FIRST) -> KdaProblem:
    p = KdaProblem()
    p.B, p.T, p.Hqk, p.Hv, p.N = int(B), int(T), int(Hqk), int(Hv), int(N)
    p.cu_seqlens = _ptr(cu_seqlens)
    p.cu_seqlens_host = _ptr(cu_seqlens_cpu)
    p.scale = 0.0 if scale is None else float(scale)
    p.lower_bound = float(lower_bound)
    p.route = int(route)
    p.checkpoint_every = int(checkpoint_every)
    p.context = int(context)
    p.precision = int(precision)
    p.schedule = int(schedule)
    # the struct holds raw pointers: keep the tensors alive with it
    p._keep = (cu_seqlens, cu_seqlens_cpu)
    return p


def kda_fwd_ctx_bytes(p: KdaProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.kda_fwd_ctx_bytes(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def kda_bwd_workspace_bytes(p: KdaProblem) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.kda_bwd_workspace_bytes(ctypes.byref(p), ctypes.byref(n)))
    return int(n.value)


def kda_plan_query(p: KdaProblem, with_order: bool = False):
    """(route, num_tasks, order or None): host planning only."""
    route = ctypes.c_int32(0)
    nt = ctypes.c_int64(0)
    _check(_lib.kda_plan_query(ctypes.byref(p), ctypes.byref(route), ctypes.byref(nt), None, 0))
    order = None
    if with_order:
        buf = (ctypes.c_int32 * int(nt.value))()
        _check(_lib.kda_plan_query(ctypes.byref(p), None, None, ctypes.cast(buf, _vp),
                                   int(nt.value)))
        order = list(buf)
    return int(route.value), int(nt.value), order


def _stream_handle(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def kda_fwd(p: KdaProblem, q, k, v, g, beta, A_log, dt_bias, initial_state, o, final_state,
            ctx: Optional[torch.Tensor], stream: Optional[int] = None) -> None:
    """C kda_fwd on torch tensors (no shape checks beyond the library's)."""
    if stream is None:
        stream = _stream_handle(q.device)
    ctx_bytes = 0 if ctx is None else ctx.numel() * ctx.element_size()
    _check(_lib.kda_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                        _ptr(A_log), _ptr(dt_bias), _ptr(initial_state), _ptr(o),
                        _ptr(final_state), _ptr(ctx), ctx_bytes, stream))


def kda_fwd_noalloc(p: KdaProblem, q, k, v, g, beta, A_log, dt_bias, initial_state, o,
                    final_state, ctx: Optional[torch.Tensor], stream: Optional[int] = None) -> None:
    """C kda_fwd_noalloc (the schedule in the library's static device scratch;
    no device allocation) on torch tensors."""
    if stream is None:
        stream = _stream_handle(q.device)
    ctx_bytes = 0 if ctx is None else ctx.numel() * ctx.element_size()
    _check(_lib.kda_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                _ptr(A_log), _ptr(dt_bias), _ptr(initial_state), _ptr(o),
                                _ptr(final_state), _ptr(ctx), ctx_bytes, stream))


def kda_bwd(p: KdaProblem, q, k, v, g, beta, A_log, dt_bias, initial_state, ctx, d_o,
            dfinal_state, dq, dk, dv, dg, dbeta, dA_log, ddt_bias, dinitial_state,
            workspace: torch.Tensor, stream: Optional[int] = None) -> None:
    """C kda_bwd on torch tensors."""
    if stream is None:
        stream = _stream_handle(q.device)
    _check(_lib.kda_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                        _ptr(A_log), _ptr(dt_bias), _ptr(initial_state), _ptr(ctx),
                        ctx.numel() * ctx.element_size(), _ptr(d_o), _ptr(dfinal_state),
                        _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dg), _ptr(dbeta), _ptr(dA_log),
                        _ptr(ddt_bias), _ptr(dinitial_state), _ptr(workspace),
                        workspace.numel() * workspace.element_size(), stream))


def make_infer_problem(B: int, T: int, Hqk: int, Hv: int, N: int, pool_slots: int,
                       cu_seqlens: Optional[torch.Tensor] = None,
                       cu_seqlens_cpu: Optional[torch.Tensor] = None,
                       scale: Optional[float] = None, use_qk_l2norm: bool = True,
                       use_gate_in_kernel: bool = False, lower_bound: Optional[float] = None,
                       beta_is_logit: bool = False,
                       state_indices: Optional[torch.Tensor] = None,
                       state_indices_cpu: Optional[torch.Tensor] = None,
                       route: int = ROUTE_AUTO, checkpoint_every: int = 0,
                       state_checkpoints: Optional[torch.Tensor] = None,
                       checkpoint_cu_starts: Optional[torch.Tensor] = None,
                       checkpoint_cu_starts_cpu: Optional[torch.Tensor] = None,
                       num_spec_tokens: int = 0,
                       num_accepted_tokens: Optional[torch.Tensor] = None,
                       state_source: Optional[torch.Tensor] = None,
                       source_indices: Optional[torch.Tensor] = None,
                       source_indices_cpu: Optional[torch.Tensor] = None) -> KdaInferProblem:
    p = KdaInferProblem()
    p.B, p.T, p.Hqk, p.Hv, p.N = int(B), int(T), int(Hqk), int(Hv), int(N)
    p.cu_seqlens = _ptr(cu_seqlens)
    p.cu_seqlens_host = _ptr(cu_seqlens_cpu)
    p.scale = 0.0 if scale is None else float(scale)
    p.use_qk_l2norm = int(bool(use_qk_l2norm))
    p.use_gate_in_kernel = int(bool(use_gate_in_kernel))
    p.lower_bound = 0.0 if lower_bound is None else float(lower_bound)
    p.beta_is_logit = int(bool(beta_is_logit))
    p.route = int(route)
    p.pool_slots = int(pool_slots)
    p.state_indices = _ptr(state_indices)
    p.state_indices_host = _ptr(state_indices_cpu)
    p.checkpoint_every = int(checkpoint_every)
    p.state_checkpoints = _ptr(state_checkpoints)
    p.checkpoint_rows = 0 if state_checkpoints is None else int(state_checkpoints.shape[0])
    p.checkpoint_cu_starts = _ptr(checkpoint_cu_starts)
    p.checkpoint_cu_starts_host = _ptr(checkpoint_cu_starts_cpu)
    p.num_spec_tokens = int(num_spec_tokens)
    p.num_accepted_tokens = _ptr(num_accepted_tokens)
    p.state_source = _ptr(state_source)
    p.source_slots = 0 if state_source is None else int(state_source.shape[0])
    p.source_indices = _ptr(source_indices)
    p.source_indices_host = _ptr(source_indices_cpu)
    # the struct holds raw pointers: keep the tensors alive with it
    p._keep = (cu_seqlens, cu_seqlens_cpu, state_indices, state_indices_cpu, state_checkpoints,
               checkpoint_cu_starts, checkpoint_cu_starts_cpu, num_accepted_tokens, state_source,
               source_indices, source_indices_cpu)
    return p


def kda_infer(p: KdaInferProblem, q, k, v, g, beta, A_log, dt_bias, state_pool, o,
              stream: Optional[int] = None) -> None:
    """C kda_infer on torch tensors."""
    if stream is None:
        stream = _stream_handle(q.device)
    _check(_lib.kda_infer(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                          _ptr(A_log), _ptr(dt_bias), _ptr(state_pool), _ptr(o), stream))


# ---------------------------------------------------------------------------
# paired training API
# ---------------------------------------------------------------------------
def _require(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _check_tensor(name, t, dtype, shape, device):
    _require(isinstance(t, torch.Tensor), f"{name} must be a tensor")
    _require(t.dtype == dtype, f"{name} must be {dtype}, got {t.dtype}")
    _require(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    _require(t.is_contiguous(), f"{name} must be contiguous")
    _require(t.device == device, f"{name} must be on {device}, got {t.device}")


@dataclass
class RecurrentKDATrainingContext:
    """What the forward saved for the backward: the problem, the state tape
    (a byte tensor on the device) and the inputs with their versions."""
    problem: KdaProblem
    ctx: torch.Tensor
    inputs: tuple
    versions: tuple
    cu_seqlens: Optional[torch.Tensor]
    cu_seqlens_cpu: Optional[torch.Tensor]
    stream: int


def _problem_from(q, v, cu_seqlens, cu_seqlens_cpu, scale, lower_bound, route, checkpoint_every,
                  context=CONTEXT_TAPE, precision=PRECISION_AUTO):
    _require(q.dim() == 4 and v.dim() == 4, "q and v must be [B, T, H, 128]")
    B, T, Hqk, Dq = q.shape
    Hv = v.shape[2]
    _require(Dq == HEAD_DIM and v.shape[3] == HEAD_DIM, "head dimensions must be 128")
    if cu_seqlens is not None:
        _require(cu_seqlens_cpu is not None, "packed calls need cu_seqlens_cpu")
        _require(cu_seqlens.dtype == torch.int64 and cu_seqlens_cpu.dtype == torch.int64,
                 "cu_seqlens must be int64")
        _require(cu_seqlens_cpu.device.type == "cpu" and cu_seqlens_cpu.is_contiguous(),
                 "cu_seqlens_cpu must be a contiguous CPU tensor")
        _require(cu_seqlens.is_contiguous() and cu_seqlens.device == q.device,
                 "cu_seqlens must be contiguous on the device of q")
        N = cu_seqlens.numel() - 1
    else:
        _require(cu_seqlens_cpu is None, "cu_seqlens_cpu must be omitted for fixed layout")
        N = B
    return make_problem(B, T, Hqk, Hv, N, cu_seqlens, cu_seqlens_cpu, scale, lower_bound,
                        route, checkpoint_every, context, precision)


def recurrent_kda_training_forward(q, k, v, g, beta, A_log, dt_bias, initial_state,
                                   cu_seqlens=None, scale=None, lower_bound=-5.0, out=None,
                                   final_state_out=None, context_out=None, *,
                                   cu_seqlens_cpu=None, route: int = ROUTE_AUTO,
                                   checkpoint_every: int = 0, save_context: bool = True,
                                   context: int = CONTEXT_TAPE, precision: int = PRECISION_AUTO):
    """Forward of the KDA training recurrence: returns (o, final_state, ctx).
    context: CONTEXT_TAPE (FP32 state tape; the backward rebuilds chunk
    states) or CONTEXT_RECORDS (every chunk's records; the backward reruns
    nothing, the context is about 39 KiB per 16 tokens and value head)."""
    dev = q.device
    p = _problem_from(q, v, cu_seqlens, cu_seqlens_cpu, scale, lower_bound, route,
                      checkpoint_every, context, precision)
    B, T, Hqk, Hv, N = p.B, p.T, p.Hqk, p.Hv, p.N
    bf = torch.bfloat16
    _check_tensor("q", q, bf, (B, T, Hqk, 128), dev)
    _check_tensor("k", k, bf, (B, T, Hqk, 128), dev)
    _check_tensor("v", v, bf, (B, T, Hv, 128), dev)
    _check_tensor("g", g, bf, (B, T, Hv, 128), dev)
    _check_tensor("beta", beta, bf, (B, T, Hv), dev)
    _check_tensor("A_log", A_log, torch.float32, (Hv,), dev)
    _check_tensor("dt_bias", dt_bias, torch.float32, (Hv, 128), dev)
    _check_tensor("initial_state", initial_state, torch.float32, (N, Hv, 128, 128), dev)
    o = out if out is not None else torch.empty((B, T, Hv, 128), dtype=bf, device=dev)
    _check_tensor("out", o, bf, (B, T, Hv, 128), dev)
    fs = final_state_out if final_state_out is not None else torch.empty_like(initial_state)
    _check_tensor("final_state_out", fs, torch.float32, (N, Hv, 128, 128), dev)
    ctx_t = None
    if save_context:
        need = kda_fwd_ctx_bytes(p)
        if context_out is not None:
            _require(context_out.ctx.numel() >= need and context_out.ctx.device == dev,
                     "context_out does not fit this call")
            _require(context_out.stream == _stream_handle(dev),
                     "a context is reused only on the stream that created it")
            ctx_t = context_out.ctx
        else:
            ctx_t = torch.empty(need, dtype=torch.uint8, device=dev)
    stream = _stream_handle(dev)
    kda_fwd(p, q, k, v, g, beta, A_log, dt_bias, initial_state, o, fs, ctx_t, stream)
    ctx = None
    if save_context:
        inputs = (q, k, v, g, beta, A_log, dt_bias, initial_state)
        ctx = RecurrentKDATrainingContext(p, ctx_t, inputs, tuple(t._version for t in inputs),
                                          cu_seqlens, cu_seqlens_cpu, stream)
    return o, fs, ctx


def recurrent_kda_training_backward(context: RecurrentKDATrainingContext, do, dfinal_state,
                                    out: Optional[Sequence[torch.Tensor]] = None,
                                    workspace: Optional[torch.Tensor] = None):
    """Gradients (dq, dk, dv, dg, dbeta, dA_log, ddt_bias, dinitial_state)."""
    _require(context is not None, "context is required")
    inputs = context.inputs
    now = tuple(t._version for t in inputs)
    _require(now == context.versions, "an input changed after the forward (tensor version)")
    q, k, v, g, beta, A_log, dt_bias, s0 = inputs
    p = context.problem
    dev = q.device
    _check_tensor("do", do, torch.bfloat16, tuple(v.shape), dev)
    _check_tensor("dfinal_state", dfinal_state, torch.float32, tuple(s0.shape), dev)
    if out is None:
        out = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v), torch.empty_like(g),
               torch.empty_like(beta), torch.empty_like(A_log), torch.empty_like(dt_bias),
               torch.empty_like(s0))
    _require(len(out) == 8, "out must hold eight tensors")
    for name, t, ref in zip(("dq", "dk", "dv", "dg", "dbeta", "dA_log", "ddt_bias",
                             "dinitial_state"), out, inputs):
        _check_tensor(name, t, ref.dtype, tuple(ref.shape), dev)
    need = kda_bwd_workspace_bytes(p)
    if workspace is None or workspace.numel() * workspace.element_size() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    kda_bwd(p, q, k, v, g, beta, A_log, dt_bias, s0, context.ctx, do, dfinal_state, *out,
            workspace, _stream_handle(dev))
    return tuple(out)


# ---------------------------------------------------------------------------
# inference API (decode and prefill on a state pool)
# ---------------------------------------------------------------------------
def recurrent_kda(q, k, v, g, beta, A_log=None, dt_bias=None, scale=None, initial_state=None,
                  output_final_state: bool = False, use_qk_l2norm_in_kernel: bool = True, use_gate_in_kernel: bool = False,
                  lower_bound=None, cu_seqlens=None, ssm_state_indices=None,
                  num_spec_tokens: Optional[int] = None, num_accepted_tokens=None,
                  output=None, initial_state_source=None, initial_state_indices=None,
                  beta_is_logit: bool = False, state_checkpoints=None,
                  checkpoint_cu_starts=None, checkpoint_every_n_tokens: int = 0, *,
                  cu_seqlens_cpu=None, ssm_state_indices_cpu=None, checkpoint_cu_starts_cpu=None,
                  initial_state_indices_cpu=None, route: int = ROUTE_AUTO):
    """Decode / prefill subset of page "flashinfer.kda.recurrent_kda": returns
    (output, final_state).  initial_state is a BF16 state pool
    [P, Hv, 128, 128], updated in place (slot ssm_state_indices[n] for sequence
    n, or slot n); None starts every sequence from zero in a new pool of N
    slots (not with ssm_state_indices or speculative decode).  final_state is
    that pool when output_final_state is set, else None.  Packed calls pass cu_seqlens (int64) with its CPU mirror,
    and indices with theirs.  route: ROUTE_AUTO, ROUTE_CHUNK (needs every
    per-token log-decay >= -5) or ROUTE_ROWSPLIT (token-serial, any gate).
    With checkpoint_every_n_tokens = E > 0, state_checkpoints (BF16
    [C, Hv, 128, 128]) receives, from row checkpoint_cu_starts[n] on, the
    states of sequence n before tokens 0, E, 2E, ... and the call returns
    (output, final_state, state_checkpoints).  Speculative decode
    (num_spec_tokens = S): every sequence has 1+S tokens, ssm_state_indices is
    [N, 1+S]; the state starts from slot [n, a-1] with a =
    num_accepted_tokens[n] clamped to [1, 1+S] (1 when omitted) and the state
    after token s goes to slot [n, s].  initial_state_source (a read-only BF16
    pool) with initial_state_indices [N] (and their CPU mirror) replaces the
    state each sequence starts from.  The softplus gate is not supported."""
    dev = q.device
    _require(q.dim() == 4 and v.dim() == 4, "q and v must be [B, T, H, 128]")
    B, T, Hqk, Dq = q.shape
    Hv = v.shape[2]
    _require(Dq == HEAD_DIM and v.shape[3] == HEAD_DIM, "head dimensions must be 128")
    if cu_seqlens is not None:
        _require(cu_seqlens_cpu is not None, "packed calls need cu_seqlens_cpu")
        _require(cu_seqlens.dtype == torch.int64 and cu_seqlens_cpu.dtype == torch.int64,
                 "cu_seqlens must be int64")
        _require(cu_seqlens.is_contiguous() and cu_seqlens.device == dev,
                 "cu_seqlens must be contiguous on the device of q")
        _require(cu_seqlens_cpu.device.type == "cpu" and cu_seqlens_cpu.is_contiguous(),
                 "cu_seqlens_cpu must be a contiguous CPU tensor")
        N = cu_seqlens.numel() - 1
    else:
        N = B
    S = int(num_spec_tokens or 0)
    if initial_state is None:
        _require(ssm_state_indices is None and S == 0,
                 "ssm_state_indices and speculative decode need an initial_state pool")
        initial_state = torch.zeros((N, Hv, 128, 128), dtype=torch.bfloat16, device=dev)
    _require(initial_state.dim() == 4 and tuple(initial_state.shape[1:]) == (Hv, 128, 128),
             "initial_state must be [P, Hv, 128, 128]")
    P = initial_state.shape[0]
    bf = torch.bfloat16
    _check_tensor("initial_state", initial_state, bf, (P, Hv, 128, 128), dev)
    _check_tensor("q", q, bf, (B, T, Hqk, 128), dev)
    _check_tensor("k", k, bf, (B, T, Hqk, 128), dev)
    _check_tensor("v", v, bf, (B, T, Hv, 128), dev)
    _check_tensor("g", g, bf, (B, T, Hv, 128), dev)
    _check_tensor("beta", beta, bf, (B, T, Hv), dev)
    if A_log is not None:
        _check_tensor("A_log", A_log, torch.float32, (Hv,), dev)
    if dt_bias is not None:
        dt_bias = dt_bias.reshape(Hv, 128) if dt_bias.dim() == 1 else dt_bias
        _check_tensor("dt_bias", dt_bias, torch.float32, (Hv, 128), dev)
    if ssm_state_indices is not None:
        _require(ssm_state_indices_cpu is not None, "ssm_state_indices needs its CPU mirror")
        _check_tensor("ssm_state_indices", ssm_state_indices, torch.int32,
                      (N, 1 + S) if S else (N,), dev)
        _require(ssm_state_indices_cpu.dtype == torch.int32 and
                 ssm_state_indices_cpu.device.type == "cpu" and ssm_state_indices_cpu.is_contiguous(),
                 "ssm_state_indices_cpu must be a contiguous int32 CPU tensor")
    o = output if output is not None else torch.empty((B, T, Hv, 128), dtype=bf, device=dev)
    _check_tensor("output", o, bf, (B, T, Hv, 128), dev)
    if checkpoint_every_n_tokens:
        _require(state_checkpoints is not None and checkpoint_cu_starts is not None and
                 checkpoint_cu_starts_cpu is not None,
                 "checkpoints need state_checkpoints and checkpoint_cu_starts with its CPU mirror")
        _require(state_checkpoints.dim() == 4, "state_checkpoints must be [C, Hv, 128, 128]")
        _check_tensor("state_checkpoints", state_checkpoints, bf,
                      (state_checkpoints.shape[0], Hv, 128, 128), dev)
        _check_tensor("checkpoint_cu_starts", checkpoint_cu_starts, torch.int64, (N + 1,), dev)
    p = make_infer_problem(B, T, Hqk, Hv, N, P, cu_seqlens, cu_seqlens_cpu, scale,
                           use_qk_l2norm_in_kernel, use_gate_in_kernel, lower_bound, beta_is_logit,
                           ssm_state_indices, ssm_state_indices_cpu, route,
                           checkpoint_every_n_tokens,
                           state_checkpoints if checkpoint_every_n_tokens else None,
                           checkpoint_cu_starts if checkpoint_every_n_tokens else None,
                           checkpoint_cu_starts_cpu if checkpoint_every_n_tokens else None,
                           S, num_accepted_tokens)
    if num_accepted_tokens is not None:
        _check_tensor("num_accepted_tokens", num_accepted_tokens, torch.int32, (N,), dev)
    if initial_state_source is not None:
        _require(initial_state_indices is not None and initial_state_indices_cpu is not None,
                 "initial_state_source needs initial_state_indices and their CPU mirror")
        _require(initial_state_source.dim() == 4, "initial_state_source must be [P0, Hv, 128, 128]")
        _check_tensor("initial_state_source", initial_state_source, bf,
                      (initial_state_source.shape[0], Hv, 128, 128), dev)
        _check_tensor("initial_state_indices", initial_state_indices, torch.int32, (N,), dev)
        p.state_source = _ptr(initial_state_source)
        p.source_slots = int(initial_state_source.shape[0])
        p.source_indices = _ptr(initial_state_indices)
        p.source_indices_host = _ptr(initial_state_indices_cpu)
    kda_infer(p, q, k, v, g, beta, A_log, dt_bias, initial_state, o)
    final = initial_state if output_final_state else None
    if checkpoint_every_n_tokens:
        return o, final, state_checkpoints
    return o, final
