"""Python binding of libmoe.so (include/moe.h).

Argument marshalling only: tensors become device pointers, the current torch
stream becomes the hipStream_t, and a negative status raises MoeError. Every
step of the layer runs in the library's HIP kernels. Importing this module
fails loudly if libmoe.so has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loads torch's HIP runtime first; libmoe.so then shares it

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe.so")

MOE_OK = 0
STATUS = {0: "MOE_OK", -1: "MOE_ERR_INVALID_ARG", -2: "MOE_ERR_UNSUPPORTED",
          -3: "MOE_ERR_WORKSPACE", -4: "MOE_ERR_HIP"}
MOE_F32, MOE_BF16 = 0, 1
MOE_ACT_RELU, MOE_ACT_GELU_TANH = 0, 1
MOE_PRIORITY_TOKEN, MOE_PRIORITY_RANK = 0, 1
MOE_NUM_STAGES = 5
STAGE_NAMES = ["route", "dispatch", "gemm1", "gemm2", "combine"]

EXPORTED = ["moe_capacity", "moe_candidates", "moe_max_rows", "moe_workspace_size", "moe_route",
            "moe_dispatch", "moe_dispatch_reroute", "moe_expert_ffn", "moe_combine",
            "moe_layer_forward", "moe_layer_forward_noalloc", "moe_load_stats", "moe_backward_workspace_size",
            "moe_layer_backward", "moe_set_gemm_max_blocks", "moe_status_string"]
STAT_NAMES = ["dropped", "overflow_ratio", "max_over_mean_load", "padding_ratio", "load_entropy",
              "kept_variance", "aux_loss", "kept_rows"]


class MoeError(RuntimeError):
    def __init__(self, fn, status, lib):
        self.status = status
        msg = lib.moe_status_string(status).decode() if lib is not None else ""
        super().__init__(f"{fn} returned {STATUS.get(status, status)}: {msg}")


class MoeConfig(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int64), ("d", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("capacity", ctypes.c_int32),
                ("renormalize", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32),
                ("priority", ctypes.c_int32), ("reroute", ctypes.c_int32)]


class MoeRouteInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("topk_ids", "topk_gates", "prob_sum", "expert_counts", "expert_offsets", "slot",
                 "row_of", "row_token", "served_ids", "combine_gates", "h")]


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        CFG = ctypes.POINTER(MoeConfig)
        L.moe_capacity.argtypes = [I64, I32, I32, ctypes.c_double, ctypes.POINTER(I32)]
        L.moe_candidates.argtypes = [CFG, ctypes.POINTER(I32)]
        L.moe_max_rows.argtypes = [CFG, ctypes.POINTER(I64)]
        L.moe_workspace_size.argtypes = [CFG, ctypes.POINTER(SZ)]
        L.moe_route.argtypes = [CFG, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_dispatch.argtypes = [CFG, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_dispatch_reroute.argtypes = [CFG, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_expert_ffn.argtypes = [CFG, P, P, P, P, P, P, P, P, P, SZ, P]
        L.moe_combine.argtypes = [CFG, P, P, P, P, P]
        L.moe_layer_forward.argtypes = [CFG, P, P, P, P, P, P, P, P, ctypes.POINTER(MoeRouteInfo),
                                        P, SZ, P, P, P]
        L.moe_layer_forward_noalloc.argtypes = [CFG, P, P, P, P, P, P, P, P,
                                                ctypes.POINTER(MoeRouteInfo), P]
        L.moe_load_stats.argtypes = [CFG, P, P, P, ctypes.c_double, P, P, P, P]
        L.moe_backward_workspace_size.argtypes = [CFG, ctypes.POINTER(SZ)]
        L.moe_layer_backward.argtypes = [CFG, P, P, P, P, P, P, P, ctypes.POINTER(MoeRouteInfo), P,
                                         ctypes.c_float, P, P, P, P, P, P, P, P, SZ, P, P]
        L.moe_set_gemm_max_blocks.argtypes = [I32]
        L.moe_status_string.argtypes = [I32]
        L.moe_status_string.restype = ctypes.c_char_p
        for n in EXPORTED[:-1]:
            getattr(L, n).restype = I32
        _lib = L
    return _lib


def _check(fn, status):
    if status != MOE_OK:
        raise MoeError(fn, status, lib())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"expected a tensor, got {type(t)}")
    if t.numel() > 0 and not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    return t.data_ptr() or None


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def config(T, d, d_ff, E, k, capacity, renormalize, dtype, act, priority="token",
           reroute=0) -> MoeConfig:
    dt = {"f32": MOE_F32, "bf16": MOE_BF16}.get(dtype, dtype)
    ac = {"relu": MOE_ACT_RELU, "gelu_tanh": MOE_ACT_GELU_TANH}.get(act, act)
    pr = {"token": MOE_PRIORITY_TOKEN, "rank": MOE_PRIORITY_RANK}.get(priority, priority)
    return MoeConfig(int(T), int(d), int(d_ff), int(E), int(k), int(capacity),
                     int(bool(renormalize)), int(dt), int(ac), int(pr), int(reroute))


# ------------------------------------------------------------------ host-only calls

def capacity(T: int, k: int, E: int, c: float) -> int:
    out = ctypes.c_int32(0)
    _check("moe_capacity", lib().moe_capacity(int(T), int(k), int(E), float(c), ctypes.byref(out)))
    return out.value


def candidates(cfg: MoeConfig) -> int:
    out = ctypes.c_int32(0)
    _check("moe_candidates", lib().moe_candidates(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def max_rows(cfg: MoeConfig) -> int:
    out = ctypes.c_int64(0)
    _check("moe_max_rows", lib().moe_max_rows(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def workspace_size(cfg: MoeConfig) -> int:
    out = ctypes.c_size_t(0)
    _check("moe_workspace_size", lib().moe_workspace_size(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def set_gemm_max_blocks(blocks: int) -> None:
    """Cap the persistent expert GEMMs' grid (0: one block per CU)."""
    _check("moe_set_gemm_max_blocks", lib().moe_set_gemm_max_blocks(int(blocks)))


def alloc_workspace(cfg: MoeConfig, device="cuda") -> torch.Tensor:
    return torch.empty(max(1, workspace_size(cfg)), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------ stage calls

def route(cfg, x, W_r, b_r, topk_ids, topk_gates, prob_sum=None, logits=None, ws=None,
          stream=None):
    ws = alloc_workspace(cfg, x.device) if ws is None else ws
    _check("moe_route", lib().moe_route(ctypes.byref(cfg), _ptr(x), _ptr(W_r), _ptr(b_r),
                                        _ptr(topk_ids), _ptr(topk_gates), _ptr(prob_sum),
                                        _ptr(logits), _ptr(ws), ws.numel(), _stream(stream)))


def dispatch(cfg, x, topk_ids, expert_counts, expert_offsets, slot, row_of, row_token, x_perm,
             ws=None, stream=None):
    ws = alloc_workspace(cfg, x.device) if ws is None else ws
    _check("moe_dispatch", lib().moe_dispatch(ctypes.byref(cfg), _ptr(x), _ptr(topk_ids),
                                              _ptr(expert_counts), _ptr(expert_offsets),
                                              _ptr(slot), _ptr(row_of), _ptr(row_token),
                                              _ptr(x_perm), _ptr(ws), ws.numel(),
                                              _stream(stream)))


def dispatch_reroute(cfg, x, cand_ids, cand_gates, expert_counts, expert_offsets, slot, row_of,
                     row_token, served_ids, combine_gates, x_perm=None, ws=None, stream=None):
    ws = alloc_workspace(cfg, cand_ids.device) if ws is None else ws
    _check("moe_dispatch_reroute", lib().moe_dispatch_reroute(
        ctypes.byref(cfg), _ptr(x), _ptr(cand_ids), _ptr(cand_gates), _ptr(expert_counts),
        _ptr(expert_offsets), _ptr(slot), _ptr(row_of), _ptr(row_token), _ptr(served_ids),
        _ptr(combine_gates), _ptr(x_perm), _ptr(ws), ws.numel(), _stream(stream)))


def expert_ffn(cfg, x_perm, expert_offsets, W1, b1, W2, b2, h, y_perm, ws=None, stream=None):
    ws = alloc_workspace(cfg, x_perm.device) if ws is None else ws
    _check("moe_expert_ffn", lib().moe_expert_ffn(ctypes.byref(cfg), _ptr(x_perm),
                                                  _ptr(expert_offsets), _ptr(W1), _ptr(b1),
                                                  _ptr(W2), _ptr(b2), _ptr(h), _ptr(y_perm),
                                                  _ptr(ws), ws.numel(), _stream(stream)))


def combine(cfg, y_perm, row_of, topk_gates, y, stream=None):
    _check("moe_combine", lib().moe_combine(ctypes.byref(cfg), _ptr(y_perm), _ptr(row_of),
                                            _ptr(topk_gates), _ptr(y), _stream(stream)))


def layer_forward(cfg, x, W_r, b_r, W1, b1, W2, b2, y, info: dict | None = None, ws=None,
                  stage_events=None, kernel_events=None, stream=None):
    """info: optional dict of output tensors keyed like moe_route_info's fields.
    stage_events: optional HipEvents with MOE_NUM_STAGES + 1 events.
    kernel_events: optional HipEvents with 2 * MOE_NUM_STAGES events (start of
    each stage's first kernel, end of its last)."""
    ws = alloc_workspace(cfg, x.device) if ws is None else ws
    ri = None
    if info:
        ri = MoeRouteInfo(**{k: _ptr(v) for k, v in info.items()})
    ev = stage_events.array if stage_events is not None else None
    gev = kernel_events.array if kernel_events is not None else None
    _check("moe_layer_forward", lib().moe_layer_forward(
        ctypes.byref(cfg), _ptr(x), _ptr(W_r), _ptr(b_r), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
        _ptr(y), ctypes.byref(ri) if ri is not None else None, _ptr(ws), ws.numel(), ev, gev,
        _stream(stream)))


def load_stats(cfg, expert_counts, expert_offsets, prob_sum, aux_alpha, stats, kept=None,
               dropped=None, stream=None):
    """stats: a float64 tensor of len(STAT_NAMES) (filled on the device)."""
    _check("moe_load_stats", lib().moe_load_stats(
        ctypes.byref(cfg), _ptr(expert_counts), _ptr(expert_offsets), _ptr(prob_sum),
        float(aux_alpha), _ptr(kept), _ptr(dropped), _ptr(stats), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 268435456


def layer_forward_noalloc(cfg, x, W_r, b_r, W1, b1, W2, b2, y, info: dict | None = None,
                          stream=None):
    """moe_layer_forward in the library's own fixed device array (no workspace)."""
    ri = MoeRouteInfo(**{k: _ptr(v) for k, v in info.items()}) if info else None
    _check("moe_layer_forward_noalloc", lib().moe_layer_forward_noalloc(
        ctypes.byref(cfg), _ptr(x), _ptr(W_r), _ptr(b_r), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
        _ptr(y), ctypes.byref(ri) if ri is not None else None, _stream(stream)))


def backward_workspace_size(cfg: MoeConfig) -> int:
    out = ctypes.c_size_t(0)
    _check("moe_backward_workspace_size",
           lib().moe_backward_workspace_size(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


MOE_BWD_NUM_STAGES = 5
BWD_STAGE_NAMES = ["recompute", "rows", "dgrad", "wgrad", "router"]


def layer_backward(cfg, x, W_r, b_r, W1, b1, W2, b2, fwd: dict, dy, aux_alpha, grads: dict,
                   ws=None, stage_events=None, stream=None):
    """fwd: the forward's routing outputs (topk_ids, topk_gates, expert_counts,
    expert_offsets, row_of, row_token). grads: output tensors dx, dW_r, dW1,
    dW2 and optionally db_r, db1, db2. stage_events: optional HipEvents with
    MOE_BWD_NUM_STAGES + 1 events."""
    if ws is None:
        ws = torch.empty(max(1, backward_workspace_size(cfg)), dtype=torch.uint8, device=x.device)
    ri = MoeRouteInfo(**{k: _ptr(v) for k, v in fwd.items()})
    gp = {k: _ptr(grads.get(k)) for k in ("dx", "dW_r", "db_r", "dW1", "db1", "dW2", "db2")}
    _check("moe_layer_backward", lib().moe_layer_backward(
        ctypes.byref(cfg), _ptr(x), _ptr(W_r), _ptr(b_r), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
        ctypes.byref(ri), _ptr(dy), float(aux_alpha), gp["dx"], gp["dW_r"], gp["db_r"], gp["dW1"],
        gp["db1"], gp["dW2"], gp["db2"], _ptr(ws), ws.numel(),
        stage_events.array if stage_events is not None else None, _stream(stream)))


# ------------------------------------------------------------------ HIP events (timing)

class HipEvents:
    """n raw hipEvent_t handles from the HIP runtime torch already loaded, for
    the stage boundaries of moe_layer_forward (recorded on its stream)."""

    def __init__(self, n: int):
        self._rt = ctypes.CDLL("libamdhip64.so.7")
        self._rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._rt.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.array = (ctypes.c_void_p * n)()
        for i in range(n):
            h = ctypes.c_void_p()
            if self._rt.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.array[i] = h
        self.n = n

    def elapsed_ms(self, i: int, j: int) -> float:
        out = ctypes.c_float(0)
        self._rt.hipEventSynchronize(self.array[j])
        if self._rt.hipEventElapsedTime(ctypes.byref(out), self.array[i], self.array[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for i in range(self.n):
            if self.array[i]:
                self._rt.hipEventDestroy(self.array[i])
                self.array[i] = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
