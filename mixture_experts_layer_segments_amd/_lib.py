"""ctypes binding of libmoe.so (argument marshalling only)."""
from __future__ import annotations

import ctypes
import os

# torch first: its HIP runtime must be the one libmoe.so binds to.  Loading
# libmoe.so first would pull in a second copy of libamdhip64 (same soname,
# different file) that does not share torch's device state.
import torch  # noqa: F401

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_DT_F32, MOE_DT_BF16 = 0, 1
MOE_SCORE_SOFTMAX, MOE_SCORE_SIGMOID = 0, 1
MOE_SPLIT_PARITY, MOE_SPLIT_BOUNDED = 0, 1

EXPORTED_SYMBOLS = (
    "moe_status_string", "moe_num_segments", "moe_workspace_size", "moe_route_topk",
    "moe_permute", "moe_grouped_ffn", "moe_unpermute_combine", "moe_layer_forward",
    "moe_quantize_fp8", "moe_grouped_ffn_fp8w", "moe_layer_forward_fp8w",
    "moe_layer_plan_offsets", "moe_num_rows", "moe_quantize_act_fp8", "moe_grouped_ffn_w8a8",
    "moe_layer_forward_w8a8", "moe_layer_forward_static",
)
MOE_STATIC_WORKSPACE_BYTES = 64 * 1024 * 1024   # include/moe.h


class MoEConfig(ctypes.Structure):
    """Mirror of ``moe_config`` in include/moe.h."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "T", "H", "E", "k", "I", "score", "n_group", "topk_group", "group_score_topn",
        "renormalize", "n_hot_split", "split_ways", "shared_I", "act_dtype", "split_mode",
        "split_c_permille", "capacity_factor_permille")]


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {moe_status_string(status)} ({status})")
        self.status = status


if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_cfgp = ctypes.POINTER(MoEConfig)
lib.moe_status_string.restype = ctypes.c_char_p
lib.moe_status_string.argtypes = [ctypes.c_int]
lib.moe_num_segments.restype = ctypes.c_int32
lib.moe_num_segments.argtypes = [_cfgp]
lib.moe_workspace_size.restype = ctypes.c_size_t
lib.moe_workspace_size.argtypes = [_cfgp]
lib.moe_num_rows.restype = ctypes.c_int32
lib.moe_num_rows.argtypes = [_cfgp]
lib.moe_layer_plan_offsets.restype = ctypes.c_int
lib.moe_layer_plan_offsets.argtypes = [_cfgp, ctypes.POINTER(ctypes.c_size_t)]
lib.moe_route_topk.restype = ctypes.c_int
lib.moe_route_topk.argtypes = [_cfgp, _p, _p, _p, _p]
lib.moe_permute.restype = ctypes.c_int
lib.moe_permute.argtypes = [_cfgp] + [_p] * 10 + [ctypes.c_size_t, _p]
lib.moe_grouped_ffn.restype = ctypes.c_int
lib.moe_grouped_ffn.argtypes = [_cfgp] + [_p] * 8 + [ctypes.c_size_t, _p]
lib.moe_unpermute_combine.restype = ctypes.c_int
lib.moe_unpermute_combine.argtypes = [_cfgp] + [_p] * 6
lib.moe_layer_forward.restype = ctypes.c_int
lib.moe_layer_forward.argtypes = [_cfgp] + [_p] * 12 + [ctypes.c_size_t, _p]
lib.moe_quantize_fp8.restype = ctypes.c_int
lib.moe_quantize_fp8.argtypes = [ctypes.c_int32] * 3 + [_p] * 4
lib.moe_grouped_ffn_fp8w.restype = ctypes.c_int
lib.moe_grouped_ffn_fp8w.argtypes = [_cfgp] + [_p] * 10 + [ctypes.c_size_t, _p]
lib.moe_layer_forward_fp8w.restype = ctypes.c_int
lib.moe_layer_forward_fp8w.argtypes = [_cfgp] + [_p] * 16 + [ctypes.c_size_t, _p]
lib.moe_quantize_act_fp8.restype = ctypes.c_int
lib.moe_quantize_act_fp8.argtypes = [ctypes.c_int32] * 2 + [_p] * 4
lib.moe_grouped_ffn_w8a8.restype = ctypes.c_int
lib.moe_grouped_ffn_w8a8.argtypes = [_cfgp] + [_p] * 11 + [ctypes.c_size_t, _p]
lib.moe_layer_forward_w8a8.restype = ctypes.c_int
lib.moe_layer_forward_w8a8.argtypes = [_cfgp] + [_p] * 16 + [ctypes.c_size_t, _p]
lib.moe_layer_forward_static.restype = ctypes.c_int
lib.moe_layer_forward_static.argtypes = [_cfgp] + [_p] * 12


def make_config(shape) -> MoEConfig:
    """MoEConfig from any object with the layer's fields (T, H, E, k, I,
    dtype 'f32'|'bf16', score 'softmax'|'sigmoid', n_group, topk_group,
    group_score_topn, renormalize, n_hot_split, split_ways, split_mode
    'parity'|'bounded', split_c_permille, shared_I, capacity_factor_permille)."""
    g = lambda n, d: getattr(shape, n, d)  # noqa: E731
    return MoEConfig(
        T=shape.T, H=shape.H, E=shape.E, k=shape.k, I=shape.I,
        score=MOE_SCORE_SIGMOID if g("score", "softmax") == "sigmoid" else MOE_SCORE_SOFTMAX,
        n_group=g("n_group", 1), topk_group=g("topk_group", 1),
        group_score_topn=g("group_score_topn", 2), renormalize=int(g("renormalize", 1)),
        n_hot_split=g("n_hot_split", 0), split_ways=g("split_ways", 1),
        shared_I=g("shared_I", 0),
        act_dtype=MOE_DT_F32 if g("dtype", "bf16") == "f32" else MOE_DT_BF16,
        split_mode=MOE_SPLIT_BOUNDED if g("split_mode", "parity") == "bounded" else MOE_SPLIT_PARITY,
        split_c_permille=g("split_c_permille", 0),
        capacity_factor_permille=g("capacity_factor_permille", 0))


def moe_status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def _cfg(cfg) -> MoEConfig:
    return cfg if isinstance(cfg, MoEConfig) else make_config(cfg)


def moe_num_segments(cfg) -> int:
    return int(lib.moe_num_segments(ctypes.byref(_cfg(cfg))))


def moe_num_rows(cfg) -> int:
    return int(lib.moe_num_rows(ctypes.byref(_cfg(cfg))))


def moe_workspace_size(cfg) -> int:
    return int(lib.moe_workspace_size(ctypes.byref(_cfg(cfg))))


def moe_layer_plan_offsets(cfg) -> dict:
    """Byte offsets of seg_offsets, seg_expert, assign_to_row and
    row_to_token inside the layer call's workspace."""
    off = (ctypes.c_size_t * 4)()
    _check(lib.moe_layer_plan_offsets(ctypes.byref(_cfg(cfg)), off), "moe_layer_plan_offsets")
    return dict(zip(("seg_offsets", "seg_expert", "assign_to_row", "row_to_token"), off))


def _ptr(t):
    """Device address of a tensor (or an int address / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to libmoe must be contiguous")
    if t.device.type != "cuda":
        raise ValueError("tensors passed to libmoe must be on the GPU")
    return t.data_ptr()


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != MOE_OK:
        raise MoEError(status, where)


def moe_route_topk(cfg, logits, topk_ids, topk_w, stream=None):
    _check(lib.moe_route_topk(ctypes.byref(_cfg(cfg)), _ptr(logits), _ptr(topk_ids),
                              _ptr(topk_w), _stream(stream)), "moe_route_topk")


def moe_permute(cfg, x, topk_ids, x_perm, seg_offsets, seg_expert, assign_to_row,
                row_to_token, counts, balancedness, workspace, stream=None):
    _check(lib.moe_permute(ctypes.byref(_cfg(cfg)), _ptr(x), _ptr(topk_ids), _ptr(x_perm),
                           _ptr(seg_offsets), _ptr(seg_expert), _ptr(assign_to_row),
                           _ptr(row_to_token), _ptr(counts), _ptr(balancedness),
                           _ptr(workspace), _nbytes(workspace), _stream(stream)), "moe_permute")


def moe_grouped_ffn(cfg, x_perm, seg_offsets, seg_expert, w13, w2, row_scale, y_perm,
                    workspace, stream=None):
    _check(lib.moe_grouped_ffn(ctypes.byref(_cfg(cfg)), _ptr(x_perm), _ptr(seg_offsets),
                               _ptr(seg_expert), _ptr(w13), _ptr(w2), _ptr(row_scale),
                               _ptr(y_perm), _ptr(workspace), _nbytes(workspace),
                               _stream(stream)), "moe_grouped_ffn")


def moe_unpermute_combine(cfg, y_perm, assign_to_row, topk_w, shared_y, out, stream=None):
    _check(lib.moe_unpermute_combine(ctypes.byref(_cfg(cfg)), _ptr(y_perm), _ptr(assign_to_row),
                                     _ptr(topk_w), _ptr(shared_y), _ptr(out), _stream(stream)),
           "moe_unpermute_combine")


def moe_layer_forward(cfg, logits, x, w13, w2, shared_w13, shared_w2, out, topk_ids, topk_w,
                      counts, balancedness, workspace, stream=None):
    _check(lib.moe_layer_forward(ctypes.byref(_cfg(cfg)), _ptr(logits), _ptr(x), _ptr(w13),
                                 _ptr(w2), _ptr(shared_w13), _ptr(shared_w2), _ptr(out),
                                 _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(balancedness),
                                 _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_static(cfg, logits, x, w13, w2, shared_w13, shared_w2, out, topk_ids,
                             topk_w, counts, balancedness, stream=None):
    """moe_layer_forward on the library's own per-GPU workspace (allocates
    nothing; overlapping calls on one GPU race)."""
    _check(lib.moe_layer_forward_static(ctypes.byref(_cfg(cfg)), _ptr(logits), _ptr(x), _ptr(w13),
                                        _ptr(w2), _ptr(shared_w13), _ptr(shared_w2), _ptr(out),
                                        _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
                                        _ptr(balancedness), _stream(stream)),
           "moe_layer_forward_static")


def moe_quantize_fp8(src, q, scale, stream=None):
    """src [n, rows, cols] (or [rows, cols]) bf16 -> q uint8 same shape, scale
    fp32 [n, rows/128, cols/128]."""
    shape = tuple(src.shape)
    n, rows, cols = (1,) + shape if len(shape) == 2 else shape
    _check(lib.moe_quantize_fp8(n, rows, cols, _ptr(src), _ptr(q), _ptr(scale), _stream(stream)),
           "moe_quantize_fp8")


def moe_grouped_ffn_fp8w(cfg, x_perm, seg_offsets, seg_expert, w13_q, w13_scale, w2_q, w2_scale,
                         row_scale, y_perm, workspace, stream=None):
    _check(lib.moe_grouped_ffn_fp8w(ctypes.byref(_cfg(cfg)), _ptr(x_perm), _ptr(seg_offsets),
                                    _ptr(seg_expert), _ptr(w13_q), _ptr(w13_scale), _ptr(w2_q),
                                    _ptr(w2_scale), _ptr(row_scale), _ptr(y_perm),
                                    _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "moe_grouped_ffn_fp8w")


def moe_layer_forward_fp8w(cfg, logits, x, w13_q, w13_scale, w2_q, w2_scale, shared_w13_q,
                           shared_w13_scale, shared_w2_q, shared_w2_scale, out, topk_ids, topk_w,
                           counts, balancedness, workspace, stream=None):
    _check(lib.moe_layer_forward_fp8w(
        ctypes.byref(_cfg(cfg)), _ptr(logits), _ptr(x), _ptr(w13_q), _ptr(w13_scale), _ptr(w2_q),
        _ptr(w2_scale), _ptr(shared_w13_q), _ptr(shared_w13_scale), _ptr(shared_w2_q),
        _ptr(shared_w2_scale), _ptr(out), _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
        _ptr(balancedness), _ptr(workspace), _nbytes(workspace), _stream(stream)),
        "moe_layer_forward_fp8w")


def moe_quantize_act_fp8(src, q, scale, stream=None):
    """src [rows, cols] bf16 -> q uint8 [rows, cols], scale fp32 [rows, cols/128]."""
    rows, cols = tuple(src.shape)
    _check(lib.moe_quantize_act_fp8(rows, cols, _ptr(src), _ptr(q), _ptr(scale), _stream(stream)),
           "moe_quantize_act_fp8")


def moe_grouped_ffn_w8a8(cfg, x_perm_q, x_perm_scale, seg_offsets, seg_expert, w13_q, w13_scale,
                         w2_q, w2_scale, row_scale, y_perm, workspace, stream=None):
    _check(lib.moe_grouped_ffn_w8a8(ctypes.byref(_cfg(cfg)), _ptr(x_perm_q), _ptr(x_perm_scale),
                                    _ptr(seg_offsets), _ptr(seg_expert), _ptr(w13_q),
                                    _ptr(w13_scale), _ptr(w2_q), _ptr(w2_scale), _ptr(row_scale),
                                    _ptr(y_perm), _ptr(workspace), _nbytes(workspace),
                                    _stream(stream)),
           "moe_grouped_ffn_w8a8")


def moe_layer_forward_w8a8(cfg, logits, x, w13_q, w13_scale, w2_q, w2_scale, shared_w13_q,
                           shared_w13_scale, shared_w2_q, shared_w2_scale, out, topk_ids, topk_w,
                           counts, balancedness, workspace, stream=None):
    _check(lib.moe_layer_forward_w8a8(
        ctypes.byref(_cfg(cfg)), _ptr(logits), _ptr(x), _ptr(w13_q), _ptr(w13_scale), _ptr(w2_q),
        _ptr(w2_scale), _ptr(shared_w13_q), _ptr(shared_w13_scale), _ptr(shared_w2_q),
        _ptr(shared_w2_scale), _ptr(out), _ptr(topk_ids), _ptr(topk_w), _ptr(counts),
        _ptr(balancedness), _ptr(workspace), _nbytes(workspace), _stream(stream)),
        "moe_layer_forward_w8a8")
