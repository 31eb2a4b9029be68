"""The C-ABI library on a host without a GPU: it loads, exports every symbol
that include/moe.h declares, and rejects bad arguments synchronously with a
status code before launching anything (every call here fails validation, so
no kernel is ever launched)."""
import ctypes
import os
import re

import pytest

import moe_inputs as mi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def moe():
    import mixture_experts_layer_segments_amd as m
    return m


def _declared():
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\S.*?\b(moe_[a-z0-9_]+)\(", text, flags=re.M)))


def test_exports_every_declared_symbol(moe):
    names = _declared()
    assert set(names) == set(moe.EXPORTED_SYMBOLS), names
    for n in names:
        assert hasattr(moe.lib, n), n


def test_status_strings(moe):
    for s in (0, -1, -2, -3, -4):
        assert moe.moe_status_string(s)
    assert moe.moe_status_string(-99) == "unknown status"


def test_segments_and_workspace_of_the_workloads(moe):
    expect = {"tiny_fp32": 64, "decode_bf16": 64, "prefill_skew_bf16": 64,
              "deepseek_v3_bf16": 256, "ragged_stress_bf16": 136}
    for name, S in expect.items():
        cfg = mi.WORKLOADS[name]
        assert moe.moe_num_segments(cfg) == S == cfg.S
        ws = moe.moe_workspace_size(cfg)
        eb = cfg.elem_bytes
        # at least y_perm and h of every assignment (the layer reads x rows
        # through row_to_token, so it needs no x_perm)
        assert ws >= cfg.A * (cfg.H + cfg.I) * eb


def test_capacity_rows_follow_the_book(moe):
    """The library's slot arithmetic on the book's example ("Capacity,
    padding, and the drop decision"): 64 assignments over 8 experts at
    1.25 x the mean give 80 slots; sizing for the busiest expert (22, factor
    2.75) gives 176; S = 2E segments (kept rows and padding per expert)."""
    book = mi.MoEShape("book", T=32, H=64, E=8, k=2, I=64, capacity_factor_permille=1250)
    assert moe.moe_num_rows(book) == 80 and moe.moe_num_segments(book) == 16 == book.S
    assert moe.moe_num_rows(book.replace(capacity_factor_permille=2750)) == 176
    assert moe.moe_num_rows(book.replace(capacity_factor_permille=0)) == 64
    dec = mi.WORKLOADS["decode_capacity_bf16"]
    assert moe.moe_num_rows(dec) == 64 * 3          # ceil(1.25 * 128 / 64) = 3 slots
    assert moe.moe_workspace_size(dec) >= 192 * (dec.H + dec.I) * 2
    # a fixed capacity with replica segments is not supported
    rag = moe.make_config(mi.WORKLOADS["ragged_stress_bf16"])
    rag.capacity_factor_permille = 1250
    assert moe.lib.moe_num_rows(ctypes.byref(rag)) == -1
    assert moe.lib.moe_route_topk(ctypes.byref(rag), FAKE, FAKE, FAKE, None) == -2


FAKE = 1 << 20          # 256-byte aligned non-null address, never dereferenced


def _layer(moe, cfg, ws_bytes=None, **override):
    c = moe.make_config(cfg)
    args = dict(logits=FAKE, x=FAKE, w13=FAKE, w2=FAKE, sw13=None, sw2=None, out=FAKE,
                ids=FAKE, w=FAKE, counts=FAKE, bal=FAKE, ws=FAKE)
    args.update(override)
    wsb = moe.moe_workspace_size(cfg) if ws_bytes is None else ws_bytes
    return moe.lib.moe_layer_forward(ctypes.byref(c), args["logits"], args["x"], args["w13"],
                                     args["w2"], args["sw13"], args["sw2"], args["out"],
                                     args["ids"], args["w"], args["counts"], args["bal"],
                                     args["ws"], wsb, None)


@pytest.mark.parametrize("field,value,status", [
    ("E", 0, -1), ("k", 0, -1), ("H", -8, -1), ("I", 0, -1), ("T", -1, -1),
    ("k", 65, -2), ("E", 2048, -2), ("act_dtype", 7, -1), ("score", 3, -1),
    ("n_group", 3, -1), ("split_ways", 9, -2), ("H", 100, -2), ("I", 100, -2),
    ("shared_I", 36, -2), ("renormalize", 2, -1), ("split_mode", 2, -1),
    ("split_c_permille", -1, -1), ("split_c_permille", 100001, -1),
    ("capacity_factor_permille", -1, -1), ("capacity_factor_permille", 1000001, -1),
    ("H", 1 << 24, -2),   # T*k*H reaches 2^31 elements: beyond 32-bit byte offsets
])
def test_bad_config_is_rejected(moe, field, value, status):
    c = moe.make_config(mi.WORKLOADS["decode_bf16"])
    setattr(c, field, value)
    assert moe.lib.moe_route_topk(ctypes.byref(c), FAKE, FAKE, FAKE, None) == status
    assert moe.lib.moe_workspace_size(ctypes.byref(c)) == 0
    assert moe.lib.moe_num_segments(ctypes.byref(c)) == -1


@pytest.mark.parametrize("H,I", [(200, 72), (8, 8), (4104, 1544)])
def test_bf16_sizes_in_multiples_of_8_are_accepted(moe, H, I):
    """bf16 rows are moved in 16-byte chunks, so H and I need only be
    multiples of 8 (the GEMM tiles zero the K tail of their last stage)."""
    c = moe.make_config(mi.WORKLOADS["decode_bf16"].replace(H=H, I=I))
    assert moe.lib.moe_workspace_size(ctypes.byref(c)) > 0


def test_grouped_softmax_and_bad_groups_are_rejected(moe):
    base = mi.WORKLOADS["deepseek_v3_bf16"]
    for kw, st in [(dict(score="softmax"), -2), (dict(topk_group=0), -1),
                   (dict(topk_group=9), -1), (dict(group_score_topn=33), -1),
                   (dict(k=8, topk_group=1, n_group=64), -1)]:
        c = moe.make_config(base.replace(**kw))
        assert moe.lib.moe_route_topk(ctypes.byref(c), FAKE, FAKE, FAKE, None) == st, kw


def test_null_misaligned_and_small_workspace(moe):
    cfg = mi.WORKLOADS["decode_bf16"]
    assert _layer(moe, cfg, out=None) == -1
    assert _layer(moe, cfg, x=FAKE + 8) == -1             # 16-byte alignment
    assert _layer(moe, cfg, ws=FAKE + 64) == -1           # 256-byte alignment
    assert _layer(moe, cfg, ws_bytes=moe.moe_workspace_size(cfg) - 1) == -3
    shared = mi.WORKLOADS["deepseek_v3_bf16"]
    assert _layer(moe, shared) == -1                       # shared weights missing
    c = moe.make_config(cfg)
    assert moe.lib.moe_permute(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                               FAKE, FAKE, 16, None) == -3
    assert moe.lib.moe_grouped_ffn(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, None, FAKE,
                                   FAKE, 16, None) == -3
    assert moe.lib.moe_unpermute_combine(ctypes.byref(c), FAKE, None, None, None, FAKE,
                                         None) == -1


def test_static_workspace_limit_is_checked_on_the_host(moe):
    """moe_layer_forward_static refuses, before any HIP call, a layer whose
    workspace exceeds the library's static array, and invalid configs; the
    limit in the binding is the header's."""
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        m = re.search(r"#define MOE_STATIC_WORKSPACE_BYTES \((\d+)u \* 1024u \* 1024u\)", f.read())
    assert m and int(m.group(1)) * 1024 * 1024 == moe.MOE_STATIC_WORKSPACE_BYTES
    big = mi.WORKLOADS["prefill_skew_bf16"]
    assert moe.moe_workspace_size(big) > moe.MOE_STATIC_WORKSPACE_BYTES
    assert moe.moe_workspace_size(mi.WORKLOADS["decode_bf16"]) <= moe.MOE_STATIC_WORKSPACE_BYTES
    args = [FAKE] * 4 + [None, None] + [FAKE] * 5 + [None]
    c = moe.make_config(big)
    assert moe.lib.moe_layer_forward_static(ctypes.byref(c), *args) == -3
    c = moe.make_config(mi.WORKLOADS["decode_bf16"])
    c.E = 0
    assert moe.lib.moe_layer_forward_static(ctypes.byref(c), *args) == -1
    c = moe.make_config(mi.WORKLOADS["decode_bf16"].replace(T=0))
    assert moe.lib.moe_layer_forward_static(ctypes.byref(c), *args) == 0


def test_empty_batch_returns_ok_without_launching(moe):
    cfg = mi.WORKLOADS["decode_bf16"].replace(T=0)
    c = moe.make_config(cfg)
    assert moe.lib.moe_route_topk(ctypes.byref(c), None, None, None, None) == 0
    assert _layer(moe, cfg, out=None) == 0


def test_config_struct_matches_header(moe):
    with open(os.path.join(ROOT, "include", "moe.h")) as f:
        text = f.read()
    body = text[text.index("typedef struct moe_config"):text.index("} moe_config;")]
    fields = re.findall(r"int32_t\s+([^;]+);", body)
    names = [n.strip() for grp in fields for n in grp.split(",")]
    assert names == [f for f, _ in moe.MoEConfig._fields_]


def test_fp8_calls_validate_before_launching(moe):
    """The FP8 entry points reject bad sizes and pointers on the host."""
    bf = mi.WORKLOADS["decode_bf16"]
    lib = moe.lib
    c = moe.make_config(bf)
    ws = moe.moe_workspace_size(c)
    args = [FAKE] * 8 + [None] + [FAKE, FAKE, ws, None]
    # quantizer: sizes must be positive multiples of 128
    assert lib.moe_quantize_fp8(1, 100, 128, FAKE, FAKE, FAKE, None) == -1
    assert lib.moe_quantize_fp8(1, 128, 0, FAKE, FAKE, FAKE, None) == -1
    assert lib.moe_quantize_fp8(-1, 128, 128, FAKE, FAKE, FAKE, None) == -1
    assert lib.moe_quantize_fp8(0, 128, 128, None, None, None, None) == 0
    assert lib.moe_quantize_fp8(1, 128, 128, None, FAKE, FAKE, None) == -1
    # grouped FFN: bf16 activations only, 128-multiples, scales required
    f32 = moe.make_config(bf.replace(dtype="f32"))
    assert lib.moe_grouped_ffn_fp8w(ctypes.byref(f32), *args[:3], FAKE, FAKE, FAKE, FAKE,
                                    None, FAKE, FAKE, ws, None) == -2
    odd = moe.make_config(bf.replace(I=192))
    assert lib.moe_grouped_ffn_fp8w(ctypes.byref(odd), *args[:3], FAKE, FAKE, FAKE, FAKE,
                                    None, FAKE, FAKE, ws, None) == -2
    assert lib.moe_grouped_ffn_fp8w(ctypes.byref(c), *args[:3], FAKE, None, FAKE, FAKE,
                                    None, FAKE, FAKE, ws, None) == -1
    assert lib.moe_layer_forward_fp8w(ctypes.byref(c), FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                      None, None, None, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, ws, None) == -1
