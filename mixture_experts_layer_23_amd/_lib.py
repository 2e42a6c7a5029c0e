"""ctypes binding of ``libmoe_mi355x.so`` (the C ABI in ``include/moe.h``).

Argument marshalling only: torch tensors supply device pointers and the
stream handle; every step of the layer runs in the HIP kernels of the
library.  There is no fallback: if the library is missing, importing a
function raises.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_mi355x.so")

MOE_OK, MOE_EINVAL, MOE_EALIGN, MOE_EDTYPE, MOE_ELAUNCH, MOE_EWORKSPACE = 0, -1, -2, -3, -4, -5
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_GATE_TRUNCATED, MOE_GATE_RENORM = 0, 1
MOE_F32, MOE_BF16 = 0, 1
MOE_ROUTE_LOGITS_GIVEN = 1
MOE_TOKEN_CHOICE, MOE_EXPERT_CHOICE = 0, 1

EXPORTS = ["moe_capacity", "moe_rows_max", "moe_workspace_size", "moe_route", "moe_permute",
           "moe_expert_ffn", "moe_combine", "aux_balance_loss", "moe_backward",
           "moe_error_string", "moe_timing_enable", "moe_timing_report",
           "moe_timing_select", "moe_bias_update", "aux_seq_loss", "moe_route_ex",
           "moe_backward_ex", "moe_route_expert_choice", "moe_permute_noalloc",
           "moe_route_permute"]


class MoeConfig(C.Structure):
    _fields_ = [("T", C.c_int32), ("D", C.c_int32), ("E", C.c_int32), ("K", C.c_int32),
                ("F", C.c_int32), ("expert_lo", C.c_int32), ("expert_hi", C.c_int32),
                ("n_shared", C.c_int32), ("score_fn", C.c_int32), ("gating", C.c_int32),
                ("dtype", C.c_int32), ("capacity_factor", C.c_double),
                ("routing", C.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, code: int, text: str):
        super().__init__(f"{fn} failed: {code} ({text})")
        self.code = code


_lib = None


def lib():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m "
                              "mixture_experts_layer_23_amd.build` (no CPU fallback exists)")
        L = C.CDLL(LIB_PATH)
        P, I, S = C.c_void_p, C.c_int32, C.c_size_t
        cfg = C.POINTER(MoeConfig)
        sig = {
            "moe_capacity": [cfg, C.POINTER(C.c_int32)],
            "moe_rows_max": [cfg, C.POINTER(C.c_int64)],
            "moe_workspace_size": [cfg, C.POINTER(C.c_size_t)],
            "moe_route": [cfg, P, P, P, P, P, P, P, P, I, P],
            "moe_permute": [cfg, P, P, P, P, P, P, P, P, P, P, S, P],
            "moe_permute_noalloc": [cfg, P, P, P, P, P, P, P, P, P, P],
            "moe_expert_ffn": [cfg, P, P, P, P, P, P, P, P, P, P],
            "moe_combine": [cfg, P, P, P, P, P, P],
            "aux_balance_loss": [cfg, P, P, C.c_float, C.c_float, P, P, P, S, P],
            "moe_backward": [cfg] + [P] * 24 + [S, P],
            "moe_error_string": [C.c_int],
            "moe_timing_enable": [I],
            "moe_timing_report": [C.c_char_p, S],
            "moe_timing_select": [C.c_char_p],
            "moe_bias_update": [cfg, P, C.c_float, P, P],
            "moe_route_ex": [cfg, P, P, P, P, P, P, P, P, P, P, P, P, I, P],
            "moe_backward_ex": [cfg] + [P] * 25 + [S, P],
            "aux_seq_loss": [cfg, P, P, I, C.c_float, P, P, I, P, S, P],
            "moe_route_expert_choice": [cfg] + [P] * 12 + [I, P, S, P],
            # x, w_r, r_bias, sel_bias, logits, idx, w, lse, counts_all,
            # offsets, slot_row, row_token, row_slot, n_dropped, x_perm, ws
            "moe_route_permute": [cfg] + [P] * 16 + [S, P],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = C.c_char_p if name == "moe_error_string" else C.c_int
        _lib = L
    return _lib


def error_string(code: int) -> str:
    s = lib().moe_error_string(int(code))
    return s.decode() if s else ""


def _check(name: str, rc: int) -> None:
    if rc != MOE_OK:
        raise MoeError(name, rc, error_string(rc))


def ptr(t) -> int | None:
    """Device (or host) address of a tensor / int / None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def stream_handle(stream=None) -> int | None:
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def make_config(T, D, E, K, F, expert_lo=0, expert_hi=None, n_shared=0, score_fn=0, gating=1,
                dtype=MOE_BF16, capacity_factor=0.0, routing=MOE_TOKEN_CHOICE) -> MoeConfig:
    return MoeConfig(T, D, E, K, F, expert_lo, E if expert_hi is None else expert_hi, n_shared,
                     score_fn, gating, dtype, float(capacity_factor), int(routing))


# ---- host-only queries ------------------------------------------------------
def capacity(cfg: MoeConfig) -> int:
    v = C.c_int32()
    _check("moe_capacity", lib().moe_capacity(C.byref(cfg), C.byref(v)))
    return int(v.value)


def rows_max(cfg: MoeConfig) -> int:
    v = C.c_int64()
    _check("moe_rows_max", lib().moe_rows_max(C.byref(cfg), C.byref(v)))
    return int(v.value)


def workspace_size(cfg: MoeConfig) -> int:
    v = C.c_size_t()
    _check("moe_workspace_size", lib().moe_workspace_size(C.byref(cfg), C.byref(v)))
    return int(v.value)


# ---- entry points (same names as the C ABI) -----------------------------------
def moe_route(cfg, x, w_r, r_bias, sel_bias, logits, topk_idx, topk_w, lse, flags=0, stream=None):
    rc = lib().moe_route(C.byref(cfg), ptr(x), ptr(w_r), ptr(r_bias), ptr(sel_bias), ptr(logits),
                         ptr(topk_idx), ptr(topk_w), ptr(lse), int(flags), stream_handle(stream))
    _check("moe_route", rc)


def moe_permute(cfg, topk_idx, x, counts_all, offsets, slot_row, row_token, row_slot, n_dropped,
                x_perm, ws, stream=None):
    rc = lib().moe_permute(C.byref(cfg), ptr(topk_idx), ptr(x), ptr(counts_all), ptr(offsets),
                           ptr(slot_row), ptr(row_token), ptr(row_slot), ptr(n_dropped),
                           ptr(x_perm), ptr(ws), ws.numel() * ws.element_size(),
                           stream_handle(stream))
    _check("moe_permute", rc)


def moe_route_permute(cfg, x, w_r, r_bias, sel_bias, logits, topk_idx, topk_w, lse, counts_all,
                      offsets, slot_row, row_token, row_slot, n_dropped, x_perm, ws, stream=None):
    rc = lib().moe_route_permute(C.byref(cfg), ptr(x), ptr(w_r), ptr(r_bias), ptr(sel_bias),
                                 ptr(logits), ptr(topk_idx), ptr(topk_w), ptr(lse),
                                 ptr(counts_all), ptr(offsets), ptr(slot_row), ptr(row_token),
                                 ptr(row_slot), ptr(n_dropped), ptr(x_perm), ptr(ws),
                                 ws.numel() * ws.element_size(), stream_handle(stream))
    _check("moe_route_permute", rc)


def moe_permute_noalloc(cfg, topk_idx, x, counts_all, offsets, slot_row, row_token, row_slot,
                        n_dropped, x_perm, stream=None):
    rc = lib().moe_permute_noalloc(C.byref(cfg), ptr(topk_idx), ptr(x), ptr(counts_all),
                                   ptr(offsets), ptr(slot_row), ptr(row_token), ptr(row_slot),
                                   ptr(n_dropped), ptr(x_perm), stream_handle(stream))
    _check("moe_permute_noalloc", rc)


def moe_expert_ffn(cfg, x, x_perm, offsets, w_gate, w_up, w_down, act, h, o_perm, stream=None):
    rc = lib().moe_expert_ffn(C.byref(cfg), ptr(x), ptr(x_perm), ptr(offsets), ptr(w_gate),
                              ptr(w_up), ptr(w_down), ptr(act), ptr(h), ptr(o_perm),
                              stream_handle(stream))
    _check("moe_expert_ffn", rc)


def moe_combine(cfg, o_perm, offsets, slot_row, topk_w, y, stream=None):
    rc = lib().moe_combine(C.byref(cfg), ptr(o_perm), ptr(offsets), ptr(slot_row), ptr(topk_w),
                           ptr(y), stream_handle(stream))
    _check("moe_combine", rc)


def aux_balance_loss(cfg, logits, counts_all, alpha, z_lambda, losses, d_logits, ws, stream=None):
    rc = lib().aux_balance_loss(C.byref(cfg), ptr(logits), ptr(counts_all), float(alpha),
                                float(z_lambda), ptr(losses), ptr(d_logits), ptr(ws),
                                ws.numel() * ws.element_size(), stream_handle(stream))
    _check("aux_balance_loss", rc)


def moe_backward(cfg, x, w_r, logits, topk_idx, topk_w, offsets, slot_row, x_perm, act, h, o_perm,
                 w_gate, w_up, w_down, dy, d_logits_extra, dx, dw_r, d_rbias, dw_gate, dw_up,
                 dw_down, d_logits_out, ws, stream=None):
    rc = lib().moe_backward(C.byref(cfg), ptr(x), ptr(w_r), ptr(logits), ptr(topk_idx),
                            ptr(topk_w), ptr(offsets), ptr(slot_row), ptr(x_perm), ptr(act),
                            ptr(h), ptr(o_perm), ptr(w_gate), ptr(w_up), ptr(w_down), ptr(dy),
                            ptr(d_logits_extra), ptr(dx), ptr(dw_r), ptr(d_rbias), ptr(dw_gate),
                            ptr(dw_up), ptr(dw_down), ptr(d_logits_out), ptr(ws),
                            ws.numel() * ws.element_size(), stream_handle(stream))
    _check("moe_backward", rc)


def timing_enable(on: bool) -> None:
    _check("moe_timing_enable", lib().moe_timing_enable(1 if on else 0))


def moe_route_ex(cfg, x, w_r, r_bias, sel_bias, jitter, w_noise, noise_eps, noise_logits, logits,
                 topk_idx, topk_w, lse, flags=0, stream=None):
    _check("moe_route_ex",
           lib().moe_route_ex(C.byref(cfg), ptr(x), ptr(w_r), ptr(r_bias), ptr(sel_bias),
                              ptr(jitter), ptr(w_noise), ptr(noise_eps), ptr(noise_logits),
                              ptr(logits), ptr(topk_idx), ptr(topk_w), ptr(lse), int(flags),
                              stream_handle(stream)))


def moe_backward_ex(cfg, x, w_r, logits, topk_idx, topk_w, offsets, slot_row, x_perm, act, h,
                    o_perm, w_gate, w_up, w_down, dy, d_logits_extra, jitter, dx, dw_r, d_rbias,
                    dw_gate, dw_up, dw_down, d_logits_out, ws, stream=None):
    args = [x, w_r, logits, topk_idx, topk_w, offsets, slot_row, x_perm, act, h, o_perm, w_gate,
            w_up, w_down, dy, d_logits_extra, jitter, dx, dw_r, d_rbias, dw_gate, dw_up, dw_down,
            d_logits_out, ws]
    _check("moe_backward_ex",
           lib().moe_backward_ex(C.byref(cfg), *[ptr(a) for a in args],
                                 ws.numel() * ws.element_size(), stream_handle(stream)))


def moe_route_expert_choice(cfg, x, w_r, r_bias, logits, gate_w, lse, counts_all, offsets,
                            slot_row, row_token, row_slot, x_perm, ws, flags=0, stream=None):
    args = [x, w_r, r_bias, logits, gate_w, lse, counts_all, offsets, slot_row, row_token,
            row_slot, x_perm]
    _check("moe_route_expert_choice",
           lib().moe_route_expert_choice(C.byref(cfg), *[ptr(a) for a in args], int(flags),
                                         ptr(ws), ws.numel() * ws.element_size(),
                                         stream_handle(stream)))


def moe_bias_update(cfg, counts_all, gamma, sel_bias, stream=None):
    _check("moe_bias_update",
           lib().moe_bias_update(C.byref(cfg), ptr(counts_all), float(gamma), ptr(sel_bias),
                                 stream_handle(stream)))


def aux_seq_loss(cfg, logits, topk_idx, seq_len, alpha, loss, d_logits, accumulate, ws,
                 stream=None):
    _check("aux_seq_loss",
           lib().aux_seq_loss(C.byref(cfg), ptr(logits), ptr(topk_idx), int(seq_len),
                              float(alpha), ptr(loss), ptr(d_logits), 1 if accumulate else 0,
                              ptr(ws), ws.numel() * ws.element_size(), stream_handle(stream)))


def timing_select(name: str | None) -> None:
    _check("moe_timing_select", lib().moe_timing_select(name.encode() if name else None))


def timing_report() -> dict:
    buf = C.create_string_buffer(1 << 16)
    _check("moe_timing_report", lib().moe_timing_report(buf, len(buf)))
    out = {}
    for line in buf.value.decode().splitlines():
        name, n, ms = line.split("\t")
        out[name] = (int(n), float(ms))
    return out
