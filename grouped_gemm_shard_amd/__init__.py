"""Python binding of libmoe_shard.so, the one-shard expert-parallel MoE layer.

Argument marshalling only: every step of the layer runs in the library's
HIP kernels.  Tensors are torch tensors on the GPU (torch provides device
memory and the current stream); the names mirror the C ABI in
include/moe_shard.h.  The library is loaded on first use, and that use fails
loudly when it has not been built (``python -m grouped_gemm_shard_amd.build``);
there is no fallback.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

__all__ = [
    "MOE_OK", "MOE_EINVAL", "MOE_EUNSUPPORTED", "MOE_ECAPACITY", "MOE_EHIP",
    "MODE_LAYER", "MODE_FORCE_DROPLESS", "MODE_CAPPED_ONLY", "MODE_FORCE_CHUNKED",
    "EXPORTED", "MoeError", "Problem", "lib", "lib_path", "workspace_bytes",
    "layer_workspace_bytes", "pass_max_rows", "moe_route", "moe_count_overflow",
    "moe_permute", "moe_gmm_swiglu", "moe_combine", "moe_combine_partial",
    "moe_combine_from_partials", "moe_layer_dropless_chunked", "status_string", "LayerRunner",
    "bwd_workspace_bytes", "moe_combine_bwd", "moe_gmm_swiglu_bwd",
    "moe_permute_bwd", "moe_route_bwd", "layer_bwd_workspace_bytes", "moe_layer_bwd",
    "LayerBackwardRunner", "testing_set_gemm_wait_limit", "moe_gmm_swiglu_noalloc",
    "calib_copy", "calib_mfma", "ERR_BAD_INDEX", "ERR_BAD_OFFSETS",
    "ERR_GEMM_WAIT",
]

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ECAPACITY, MOE_EHIP = 0, -1, -2, -3, -4
MODE_LAYER, MODE_FORCE_DROPLESS, MODE_CAPPED_ONLY, MODE_FORCE_CHUNKED = 0, 1, 2, 3
GATES = {"softmax": 0, "sigmoid": 1}

EXPORTED = ["moe_workspace_bytes", "moe_pass_max_rows", "moe_layer_workspace_bytes",
            "moe_layer_chunks_per_pass",
            "moe_route", "moe_count_overflow", "moe_permute", "moe_gmm_swiglu",
            "moe_combine", "moe_combine_partial", "moe_combine_from_partials",
            "moe_layer_dropless_chunked", "moe_bwd_workspace_bytes", "moe_combine_bwd",
            "moe_gmm_swiglu_bwd", "moe_permute_bwd", "moe_route_bwd",
            "moe_layer_bwd_workspace_bytes", "moe_layer_bwd", "moe_status_string",
            "moe_testing_set_gemm_wait_limit", "moe_gmm_swiglu_noalloc", "moe_calib_copy",
            "moe_calib_mfma"]

# Device-side error bits (include/moe_shard.h)
ERR_BAD_INDEX, ERR_BAD_OFFSETS, ERR_GEMM_WAIT = 1, 2, 4

lib_path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_shard.so")


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {status_string(status)} ({status})")
        self.status = status


class _CProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "tokens", "seq_len", "hidden", "ffn", "num_experts", "top_k", "num_shards",
        "res_shard_lo", "res_shard_hi")] + [("buffer_factor", ctypes.c_float)] + [
        (n, ctypes.c_int32) for n in ("num_chunks", "gate", "dtype", "dedup",
                                      "slots_per_shard", "num_replicas")]


@dataclass(frozen=True)
class Problem:
    """Statement of one layer call (the fields of moe_problem)."""

    tokens: int
    seq_len: int
    hidden: int
    ffn: int
    num_experts: int
    top_k: int
    num_shards: int
    res_lo: int
    res_hi: int
    factor: float
    num_chunks: int = 0
    gate: str = "softmax"
    bf16: bool = True
    dedup: bool = False
    slots_per_shard: int = 0
    num_replicas: int = 0

    def c(self) -> _CProblem:
        return _CProblem(self.tokens, self.seq_len, self.hidden, self.ffn, self.num_experts,
                         self.top_k, self.num_shards, self.res_lo, self.res_hi,
                         float(self.factor), self.num_chunks, GATES[self.gate],
                         1 if self.bf16 else 0, int(self.dedup), self.slots_per_shard,
                         self.num_replicas)

    @property
    def e_loc(self):
        return self.num_experts // self.num_shards

    @property
    def spd(self):
        return self.e_loc + self.slots_per_shard

    @property
    def num_slots(self):
        return self.num_shards * self.spd

    @property
    def g_res(self):
        return (self.res_hi - self.res_lo) * self.spd

    @property
    def s_res(self):
        return self.res_hi - self.res_lo

    @property
    def dtype(self):
        return torch.bfloat16 if self.bf16 else torch.float32


def _load():
    if not os.path.exists(lib_path):
        raise ImportError(f"{lib_path} is not built; run `python -m grouped_gemm_shard_amd.build`")
    L = ctypes.CDLL(lib_path)
    P = ctypes.POINTER(_CProblem)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    sig = {
        "moe_workspace_bytes": [P, ctypes.POINTER(sz)],
        "moe_pass_max_rows": [P, i32, i32, ctypes.POINTER(i64), ctypes.POINTER(i64)],
        "moe_layer_workspace_bytes": [P, i32, ctypes.POINTER(sz)],
        "moe_layer_chunks_per_pass": [P, i32, ctypes.POINTER(i32)],
        "moe_route": [P, vp, vp, vp, vp],
        "moe_count_overflow": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_permute": [P, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp,
                        sz, vp],
        "moe_gmm_swiglu": [P, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp, sz, vp],
        "moe_combine": [P, i32, i32, vp, vp, vp, vp, vp],
        "moe_combine_partial": [P, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, i64, vp],
        "moe_combine_from_partials": [P, i32, i32, i32, vp, vp, vp, vp, i64, i64, vp],
        "moe_layer_dropless_chunked": [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_bwd_workspace_bytes": [P, i64, ctypes.POINTER(sz)],
        "moe_combine_bwd": [P, i32, i32, vp, vp, vp, vp, vp, vp, i64, vp],
        "moe_gmm_swiglu_bwd": [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, i64, vp, sz,
                               vp],
        "moe_permute_bwd": [P, i32, i32, vp, vp, vp, i64, vp],
        "moe_route_bwd": [P, vp, vp, vp, vp, vp],
        "moe_layer_bwd_workspace_bytes": [P, i32, ctypes.POINTER(sz)],
        "moe_layer_bwd": [P, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp],
        "moe_testing_set_gemm_wait_limit": [i32],
        "moe_gmm_swiglu_noalloc": [P, vp, vp, vp, vp, vp, vp, vp, vp, i64, vp, vp],
        "moe_calib_copy": [vp, vp, i64, i32, vp],
        "moe_calib_mfma": [i32, i32, vp, ctypes.POINTER(i64), vp],
    }
    for name, args in sig.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    L.moe_status_string.argtypes = [ctypes.c_int]
    L.moe_status_string.restype = ctypes.c_char_p
    return L


_LIB = None


def _lib():
    """The loaded library (loaded on first use, so that the build module can
    run before a library exists)."""
    global _LIB
    if _LIB is None:
        _LIB = _load()
    return _LIB


def __getattr__(name):
    if name == "lib":
        return _lib()
    raise AttributeError(name)


def testing_set_gemm_wait_limit(spins: int):
    """Test hook (include/moe_testing.h): bound of the grouped GEMM's wait in
    sleeps for every later call; 0 restores the default, < 0 gives up at
    once."""
    _check("moe_testing_set_gemm_wait_limit", _lib().moe_testing_set_gemm_wait_limit(spins))


def calib_copy(src, dst, blocks=8192, stream=None):
    """Streaming copy kernel (include/moe_calib.h): src and dst are byte
    tensors of the same size."""
    _check("moe_calib_copy", _lib().moe_calib_copy(_ptr(src, torch.uint8, "src"),
                                                   _ptr(dst, torch.uint8, "dst"), src.numel(),
                                                   blocks, _stream(stream)))


def calib_mfma(blocks, iters, sink, stream=None) -> int:
    """Matrix-core peak loop (include/moe_calib.h); returns its bf16 flops."""
    flops = ctypes.c_int64()
    _check("moe_calib_mfma", _lib().moe_calib_mfma(blocks, iters,
                                                   _ptr(sink, torch.float32, "sink"),
                                                   ctypes.byref(flops), _stream(stream)))
    return flops.value


def status_string(status: int) -> str:
    return _lib().moe_status_string(status).decode()


def _check(fn: str, status: int):
    if status != MOE_OK:
        raise MoeError(fn, status)


def _ptr(t, dtype=None, name="tensor"):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def workspace_bytes(p: Problem) -> int:
    out = ctypes.c_size_t()
    _check("moe_workspace_bytes", _lib().moe_workspace_bytes(ctypes.byref(p.c()), ctypes.byref(out)))
    return out.value


def layer_workspace_bytes(p: Problem, mode: int) -> int:
    out = ctypes.c_size_t()
    _check("moe_layer_workspace_bytes",
           _lib().moe_layer_workspace_bytes(ctypes.byref(p.c()), mode, ctypes.byref(out)))
    return out.value


def layer_chunks_per_pass(p: Problem, mode: int) -> int:
    out = ctypes.c_int32()
    _check("moe_layer_chunks_per_pass",
           _lib().moe_layer_chunks_per_pass(ctypes.byref(p.c()), mode, ctypes.byref(out)))
    return out.value


def pass_max_rows(p: Problem, num_chunks: int, capped: int):
    r, u = ctypes.c_int64(), ctypes.c_int64()
    _check("moe_pass_max_rows", _lib().moe_pass_max_rows(ctypes.byref(p.c()), num_chunks, capped,
                                                      ctypes.byref(r), ctypes.byref(u)))
    return r.value, u.value


def _ws(ws):
    t = _ptr(ws, torch.uint8, "ws")
    return t, ws.numel()


def moe_route(p: Problem, logits, topk_idx, topk_gate, stream=None):
    _check("moe_route", _lib().moe_route(ctypes.byref(p.c()), _ptr(logits, torch.float32, "logits"),
                                      _ptr(topk_idx, torch.int32, "topk_idx"),
                                      _ptr(topk_gate, torch.float32, "topk_gate"), _stream(stream)))


def moe_count_overflow(p: Problem, topk_idx, expert_counts, slot_expert, ndiv, slot_of_assign,
                       shard_counts, status, ws, stream=None, required_factor=None):
    """required_factor: a float32 tensor of one element, or None."""
    w, nb = _ws(ws)
    i32 = torch.int32
    _check("moe_count_overflow", _lib().moe_count_overflow(
        ctypes.byref(p.c()), _ptr(topk_idx, i32, "topk_idx"),
        _ptr(expert_counts, i32, "expert_counts"), _ptr(slot_expert, i32, "slot_expert"),
        _ptr(ndiv, i32, "ndiv"), _ptr(slot_of_assign, i32, "slot_of_assign"),
        _ptr(shard_counts, i32, "shard_counts"), _ptr(status, i32, "status"),
        _ptr(required_factor, torch.float32, "required_factor"), w, nb, _stream(stream)))


def moe_permute(p: Problem, num_chunks, chunk, capped, x, slot_of_assign, group_offsets,
                row_of_assign, sorted_assign, dedup_offsets, dedup_token, expand_idx, x_dedup,
                x_sorted, ws, stream=None):
    w, nb = _ws(ws)
    i32 = torch.int32
    max_rows = x_sorted.shape[0]
    max_dedup = x_dedup.shape[0] if x_dedup is not None else 0
    _check("moe_permute", _lib().moe_permute(
        ctypes.byref(p.c()), num_chunks, chunk, capped, _ptr(x, p.dtype, "x"),
        _ptr(slot_of_assign, i32, "slot_of_assign"), _ptr(group_offsets, i32, "group_offsets"),
        _ptr(row_of_assign, i32, "row_of_assign"), _ptr(sorted_assign, i32, "sorted_assign"),
        _ptr(dedup_offsets, i32, "dedup_offsets"), _ptr(dedup_token, i32, "dedup_token"),
        _ptr(expand_idx, i32, "expand_idx"), _ptr(x_dedup, p.dtype, "x_dedup"),
        _ptr(x_sorted, p.dtype, "x_sorted"), max_rows, max_dedup, w, nb, _stream(stream)))


def moe_gmm_swiglu(p: Problem, x_sorted, group_offsets, slot_expert, w_gate, w_up, w_down, act,
                   expert_out, ws, stream=None, status=None):
    """status: an int32 tensor of one element (receives the MOE_ERR_* bits),
    or None."""
    w, nb = _ws(ws)
    i32 = torch.int32
    max_rows = min(x_sorted.shape[0], act.shape[0], expert_out.shape[0])
    _check("moe_gmm_swiglu", _lib().moe_gmm_swiglu(
        ctypes.byref(p.c()), _ptr(x_sorted, p.dtype, "x_sorted"),
        _ptr(group_offsets, i32, "group_offsets"), _ptr(slot_expert, i32, "slot_expert"),
        _ptr(w_gate, p.dtype, "w_gate"), _ptr(w_up, p.dtype, "w_up"),
        _ptr(w_down, p.dtype, "w_down"), _ptr(act, p.dtype, "act"),
        _ptr(expert_out, p.dtype, "expert_out"), max_rows, _ptr(status, i32, "status"), w, nb,
        _stream(stream)))


def moe_gmm_swiglu_noalloc(p: Problem, x_sorted, group_offsets, slot_expert, w_gate, w_up,
                           w_down, act, expert_out, stream=None, status=None):
    """moe_gmm_swiglu without a workspace: its scratch is the library's own
    fixed device array (for callers that cannot allocate)."""
    i32 = torch.int32
    max_rows = min(x_sorted.shape[0], act.shape[0], expert_out.shape[0])
    _check("moe_gmm_swiglu_noalloc", _lib().moe_gmm_swiglu_noalloc(
        ctypes.byref(p.c()), _ptr(x_sorted, p.dtype, "x_sorted"),
        _ptr(group_offsets, i32, "group_offsets"), _ptr(slot_expert, i32, "slot_expert"),
        _ptr(w_gate, p.dtype, "w_gate"), _ptr(w_up, p.dtype, "w_up"),
        _ptr(w_down, p.dtype, "w_down"), _ptr(act, p.dtype, "act"),
        _ptr(expert_out, p.dtype, "expert_out"), max_rows, _ptr(status, i32, "status"),
        _stream(stream)))


def moe_combine(p: Problem, num_chunks, chunk, expert_out, row_of_assign, topk_gate, y,
                stream=None):
    _check("moe_combine", _lib().moe_combine(
        ctypes.byref(p.c()), num_chunks, chunk, _ptr(expert_out, p.dtype, "expert_out"),
        _ptr(row_of_assign, torch.int32, "row_of_assign"),
        _ptr(topk_gate, torch.float32, "topk_gate"), _ptr(y, p.dtype, "y"), _stream(stream)))


def moe_combine_partial(p: Problem, num_chunks, chunk, capped, expert_out, row_of_assign,
                        topk_gate, dedup_offsets, dedup_token, expand_idx, partial, stream=None):
    """Return-path dedup, receiving side: one float32 partial row per (token,
    shard) of the pass (chunk of num_chunks, capped or not).  max_rows /
    max_dedup_rows are the row counts of expert_out / partial."""
    _check("moe_combine_partial", _lib().moe_combine_partial(
        ctypes.byref(p.c()), num_chunks, chunk, capped, _ptr(expert_out, p.dtype, "expert_out"),
        _ptr(row_of_assign, torch.int32, "row_of_assign"),
        _ptr(topk_gate, torch.float32, "topk_gate"),
        _ptr(dedup_offsets, torch.int32, "dedup_offsets"),
        _ptr(dedup_token, torch.int32, "dedup_token"), _ptr(expand_idx, torch.int32, "expand_idx"),
        _ptr(partial, torch.float32, "partial"), expert_out.shape[0], partial.shape[0],
        _stream(stream)))


def moe_combine_from_partials(p: Problem, num_chunks, chunk, capped, partial, row_of_assign,
                              expand_idx, y, max_rows, stream=None):
    """Return-path dedup, source side: y of the pass's tokens from the partial
    rows.  max_rows is the row count behind row_of_assign (the length of
    expand_idx)."""
    _check("moe_combine_from_partials", _lib().moe_combine_from_partials(
        ctypes.byref(p.c()), num_chunks, chunk, capped, _ptr(partial, torch.float32, "partial"),
        _ptr(row_of_assign, torch.int32, "row_of_assign"),
        _ptr(expand_idx, torch.int32, "expand_idx"), _ptr(y, p.dtype, "y"), max_rows,
        partial.shape[0], _stream(stream)))


def moe_layer_dropless_chunked(p: Problem, mode, x, logits, w_gate, w_up, w_down, y, info, ws,
                               stream=None):
    w, nb = _ws(ws)
    _check("moe_layer_dropless_chunked", _lib().moe_layer_dropless_chunked(
        ctypes.byref(p.c()), mode, _ptr(x, p.dtype, "x"), _ptr(logits, torch.float32, "logits"),
        _ptr(w_gate, p.dtype, "w_gate"), _ptr(w_up, p.dtype, "w_up"),
        _ptr(w_down, p.dtype, "w_down"), _ptr(y, p.dtype, "y"),
        _ptr(info, torch.int32, "info"), w, nb, _stream(stream)))


# ---- backward ---------------------------------------------------------------

def bwd_workspace_bytes(p: Problem, max_rows: int) -> int:
    out = ctypes.c_size_t()
    _check("moe_bwd_workspace_bytes",
           _lib().moe_bwd_workspace_bytes(ctypes.byref(p.c()), max_rows, ctypes.byref(out)))
    return out.value


def moe_combine_bwd(p: Problem, num_chunks, chunk, dy, expert_out, row_of_assign, topk_gate,
                    d_out, d_gate, stream=None):
    """max_rows is the row count of expert_out and d_out (the smaller)."""
    _check("moe_combine_bwd", _lib().moe_combine_bwd(
        ctypes.byref(p.c()), num_chunks, chunk, _ptr(dy, p.dtype, "dy"),
        _ptr(expert_out, p.dtype, "expert_out"), _ptr(row_of_assign, torch.int32, "row_of_assign"),
        _ptr(topk_gate, torch.float32, "topk_gate"), _ptr(d_out, p.dtype, "d_out"),
        _ptr(d_gate, torch.float32, "d_gate"), min(expert_out.shape[0], d_out.shape[0]),
        _stream(stream)))


def moe_gmm_swiglu_bwd(p: Problem, x_sorted, group_offsets, slot_expert, w_gate, w_up, w_down,
                       d_out, dx_sorted, dw_gate, dw_up, dw_down, accumulate, ws, stream=None):
    """max_rows is the row count of x_sorted, d_out and dx_sorted (the
    smallest)."""
    w, nb = _ws(ws)
    i32, f32 = torch.int32, torch.float32
    max_rows = min(x_sorted.shape[0], d_out.shape[0], dx_sorted.shape[0])
    _check("moe_gmm_swiglu_bwd", _lib().moe_gmm_swiglu_bwd(
        ctypes.byref(p.c()), _ptr(x_sorted, p.dtype, "x_sorted"),
        _ptr(group_offsets, i32, "group_offsets"), _ptr(slot_expert, i32, "slot_expert"),
        _ptr(w_gate, p.dtype, "w_gate"), _ptr(w_up, p.dtype, "w_up"),
        _ptr(w_down, p.dtype, "w_down"), _ptr(d_out, p.dtype, "d_out"),
        _ptr(dx_sorted, p.dtype, "dx_sorted"), _ptr(dw_gate, f32, "dw_gate"),
        _ptr(dw_up, f32, "dw_up"), _ptr(dw_down, f32, "dw_down"), int(accumulate), max_rows, w,
        nb, _stream(stream)))


def moe_permute_bwd(p: Problem, num_chunks, chunk, dx_sorted, row_of_assign, dx, stream=None):
    _check("moe_permute_bwd", _lib().moe_permute_bwd(
        ctypes.byref(p.c()), num_chunks, chunk, _ptr(dx_sorted, p.dtype, "dx_sorted"),
        _ptr(row_of_assign, torch.int32, "row_of_assign"), _ptr(dx, p.dtype, "dx"),
        dx_sorted.shape[0], _stream(stream)))


def moe_route_bwd(p: Problem, topk_idx, topk_gate, d_gate, d_logits, stream=None):
    _check("moe_route_bwd", _lib().moe_route_bwd(
        ctypes.byref(p.c()), _ptr(topk_idx, torch.int32, "topk_idx"),
        _ptr(topk_gate, torch.float32, "topk_gate"), _ptr(d_gate, torch.float32, "d_gate"),
        _ptr(d_logits, torch.float32, "d_logits"), _stream(stream)))


def layer_bwd_workspace_bytes(p: Problem, mode: int) -> int:
    out = ctypes.c_size_t()
    _check("moe_layer_bwd_workspace_bytes",
           _lib().moe_layer_bwd_workspace_bytes(ctypes.byref(p.c()), mode, ctypes.byref(out)))
    return out.value


def moe_layer_bwd(p: Problem, mode, x, logits, w_gate, w_up, w_down, dy, dx, d_logits, dw_gate,
                  dw_up, dw_down, ws, stream=None):
    w, nb = _ws(ws)
    f32 = torch.float32
    _check("moe_layer_bwd", _lib().moe_layer_bwd(
        ctypes.byref(p.c()), mode, _ptr(x, p.dtype, "x"), _ptr(logits, f32, "logits"),
        _ptr(w_gate, p.dtype, "w_gate"), _ptr(w_up, p.dtype, "w_up"),
        _ptr(w_down, p.dtype, "w_down"), _ptr(dy, p.dtype, "dy"), _ptr(dx, p.dtype, "dx"),
        _ptr(d_logits, f32, "d_logits"), _ptr(dw_gate, f32, "dw_gate"),
        _ptr(dw_up, f32, "dw_up"), _ptr(dw_down, f32, "dw_down"), w, nb, _stream(stream)))


class LayerBackwardRunner:
    """Owns the gradient and workspace tensors of repeated layer backward
    calls."""

    def __init__(self, p: Problem, mode: int, device="cuda"):
        self.p, self.mode = p, mode
        e_res = p.s_res * p.e_loc
        f32 = torch.float32
        self.ws = torch.empty(layer_bwd_workspace_bytes(p, mode), dtype=torch.uint8,
                              device=device)
        self.dx = torch.empty((p.tokens, p.hidden), dtype=p.dtype, device=device)
        self.d_logits = torch.empty((p.tokens, p.num_experts), dtype=f32, device=device)
        self.dw_gate = torch.empty((e_res, p.ffn, p.hidden), dtype=f32, device=device)
        self.dw_up = torch.empty_like(self.dw_gate)
        self.dw_down = torch.empty((e_res, p.hidden, p.ffn), dtype=f32, device=device)

    def __call__(self, x, logits, w_gate, w_up, w_down, dy, stream=None):
        moe_layer_bwd(self.p, self.mode, x, logits, w_gate, w_up, w_down, dy, self.dx,
                      self.d_logits, self.dw_gate, self.dw_up, self.dw_down, self.ws, stream)
        return dict(dx=self.dx, d_logits=self.d_logits, dw_gate=self.dw_gate,
                    dw_up=self.dw_up, dw_down=self.dw_down)


class LayerRunner:
    """Owns the output, info and workspace tensors of repeated layer calls."""

    def __init__(self, p: Problem, mode: int, device="cuda"):
        self.p, self.mode = p, mode
        self.ws = torch.empty(layer_workspace_bytes(p, mode), dtype=torch.uint8, device=device)
        self.y = torch.empty((p.tokens, p.hidden), dtype=p.dtype, device=device)
        # [overflow, fallback_ran, cap, max shard count, MOE_ERR_* bits]
        self.info = torch.zeros(5, dtype=torch.int32, device=device)

    def __call__(self, x, logits, w_gate, w_up, w_down, stream=None):
        moe_layer_dropless_chunked(self.p, self.mode, x, logits, w_gate, w_up, w_down, self.y,
                                   self.info, self.ws, stream)
        return self.y
