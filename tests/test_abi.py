"""The C ABI of libmonolayer without a GPU: the library loads, exports every function that
include/mono.h declares, and its host-side argument checks reject bad calls, listing every
reason, before anything is enqueued. No call here reaches a kernel launch: every call either
fails its checks or has rows == 0, which returns before touching the device."""

import ctypes
import os
import re

import pytest

import moe_decode_layer_amd as mono
from moe_decode_layer_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mono.h")

# fake device addresses: never dereferenced, because every call below returns on the host
P16 = 0x100000
P256 = 0x200000


def declared_functions():
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    return sorted(set(re.findall(r"\b(mono_[a-z_0-9]+)\s*\(", text)))


def shape(**kw):
    base = dict(rows=1, hidden=5120, n_experts=256, top_k=8, inter=2048, shared_inter=2048,
                act="bf16", routed_scale=2.5)
    base.update(kw)
    return B.make_shape(**base)


def experts(fmt="bf16"):
    q = fmt in ("q8_0", "mxfp4")
    return B.make_experts(fmt, P16, P16, P16, P16 if q else None, P16 if q else None,
                          P16 if q else None)


def layer(rfmt="bf16", sfmt="bf16"):
    return B.make_layer(P16, P16, P16, P16, P16, P16, experts(rfmt), experts(sfmt))


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(B.LIB_PATH)
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(B.EXPORTS) == names


def test_binding_loads_the_in_tree_library():
    L = mono.lib()
    assert os.path.samefile(L._name, B.LIB_PATH)


def test_workspace_bytes_grows_with_rows_and_is_aligned():
    a = B.mono_workspace_bytes(shape(rows=1))
    b = B.mono_workspace_bytes(shape(rows=8, hidden=4096))
    assert a > 0 and b > 0 and a % 256 == 0 and b % 256 == 0
    assert B.mono_workspace_bytes(shape(rows=6)) > a


def test_invalid_shape_lists_every_reason():
    s = shape(rows=9, hidden=100, top_k=0, inter=48)
    s.n_streams = 3
    with pytest.raises(B.MonoError) as e:
        B.mono_workspace_bytes(s)
    msg = e.value.message
    for part in ("rows=9", "n_streams=3", "hidden=100", "top_k=0", "inter=48"):
        assert part in msg, (part, msg)


@pytest.mark.parametrize("kw,needle", [
    (dict(n_experts=513), "n_experts=513"),
    (dict(top_k=17), "top_k=17"),
    (dict(top_k=8, n_experts=4), "n_experts=4"),
    (dict(act="q8_0"), "act="),
    (dict(shared_inter=-32), "shared_inter=-32"),
    (dict(sinkhorn_iters=-1), "sinkhorn_iters=-1"),
    (dict(eps_norm=-1.0), "eps_hc / eps_norm"),
    (dict(act_quant=7), "act_quant=7"),
])
def test_each_shape_limit(kw, needle):
    with pytest.raises(B.MonoError) as e:
        B.mono_workspace_bytes(shape(**kw))
    assert needle in e.value.message
    assert e.value.status == B.MONO_E_INVAL


def test_on_chip_limits_are_unsupported_not_invalid():
    with pytest.raises(B.MonoError) as e:
        B.mono_ffn_layer(shape(rows=8, hidden=8192), layer(), None, P16, None, P16, None, P256)
    assert e.value.status == B.MONO_E_UNSUPPORTED
    assert "activation buffer" in e.value.message
    with pytest.raises(B.MonoError) as e:
        B.mono_ffn_layer(shape(rows=8, inter=8192, shared_inter=0), layer(), None, P16, None, P16,
                         None, P256)
    assert e.value.status == B.MONO_E_UNSUPPORTED
    assert "hidden-row buffer" in e.value.message


def test_mxfp8_activations_need_mxfp4_routed_experts():
    s = shape(rows=8, act_quant="mxfp8")
    for call in (lambda L: B.mono_ffn_layer(s, L, None, P16, None, P16, None, P256),
                 lambda L: B.mono_moe_experts(s, P16, P16, P16, L, P16, P16, P16, P256)):
        with pytest.raises(B.MonoError) as e:
            call(layer("q8_0", "mxfp4"))
        assert e.value.status == B.MONO_E_UNSUPPORTED
        assert "act_quant MONO_AQ_MXFP8 needs routed.fmt MONO_MXFP4" in e.value.message
    # with MXFP4 routed experts the mode passes the checks (rows == 0: nothing is enqueued)
    s0 = shape(rows=0, act_quant="mxfp8")
    B.mono_ffn_layer(s0, layer("mxfp4", "bf16"), None, P16, None, P16, None, P256)
    B.mono_moe_experts(s0, P16, P16, P16, layer("mxfp4", "mxfp4"), P16, P16, P16, P256)


def test_rows_zero_is_ok_and_enqueues_nothing():
    s = shape(rows=0)
    L = layer()
    B.mono_ffn_layer(s, L, P16, P16, None, P16, P16, P256)
    B.mono_hc_mix_collapse(s, P16, L, None, P16, P16, P16, P16, P16, P16, P256)
    B.mono_router_select(s, P16, L, P16, P16, P16, P256)
    B.mono_moe_experts(s, P16, P16, P16, L, P16, P16, P16, P256)
    B.mono_hc_expand(s, P16, P16, P16, P16, P16, P256, P16, P256)


def test_null_and_misaligned_pointers_are_all_reported():
    s = shape()
    L = layer()
    L.w_router = None
    with pytest.raises(B.MonoError) as e:
        B.mono_ffn_layer(s, L, P16, None, None, P16 + 2, None, P256 + 16)
    msg = e.value.message
    for part in ("state_in is NULL", "state_out is not 16-byte aligned", "layer.w_router is NULL",
                 "carry_out is NULL", "ws is not 256-byte aligned"):
        assert part in msg, (part, msg)


def test_quantised_experts_need_their_scales():
    s = shape(rows=6)
    L = layer("q8_0", "q8_0")
    L.routed.down_s = None
    with pytest.raises(B.MonoError) as e:
        B.mono_ffn_layer(s, L, None, P16, None, P16, None, P256)
    assert "routed.down_s is NULL" in e.value.message


def test_f32_activations_need_f32_experts():
    s = shape(act="f32", hidden=256, n_experts=8, top_k=2, inter=128, shared_inter=128)
    with pytest.raises(B.MonoError) as e:
        B.mono_ffn_layer(s, layer("bf16", "bf16"), None, P16, None, P16, None, P256)
    assert e.value.status == B.MONO_E_UNSUPPORTED


def test_unfused_expand_refuses_aliasing():
    s = shape()
    with pytest.raises(B.MonoError) as e:
        B.mono_hc_expand(s, P16, P16, P16, P16, None, P16, None, P256)
    assert "aliases" in e.value.message


def test_workspace_tensor_offsets_stay_inside_the_workspace():
    s = shape(rows=8, hidden=4096)
    total = B.mono_workspace_bytes(s)
    for which in range(B.MONO_T_TRACE + 1):
        p, n = B.mono_workspace_tensor(s, P256, which)
        assert p >= P256 and p + n <= P256 + total, which


def test_static_workspace_refuses_shapes_beyond_its_size():
    """mono_ffn_layer_static checks the shape's workspace size on the host before any device
    work: 8 rows with top-16 need more than MONO_STATIC_WS_BYTES."""
    s = shape(rows=8, top_k=16)
    assert B.mono_workspace_bytes(s) > B.MONO_STATIC_WS_BYTES
    with pytest.raises(B.MonoError) as e:
        B.mono_ffn_layer_static(s, layer(), None, P16, None, P16, None)
    assert e.value.status == B.MONO_E_UNSUPPORTED
    assert "static workspace" in e.value.message


def test_race_shaker_limit_is_checked_before_any_device_work():
    with pytest.raises(B.MonoError) as e:
        B.mono_workspace_set_jitter(P256, B.MONO_JITTER_MAX_TICKS + 1, 7)
    assert e.value.status == B.MONO_E_INVAL
    assert "MONO_JITTER_MAX_TICKS" in e.value.message
    with pytest.raises(B.MonoError) as e:
        B.mono_workspace_set_jitter(P256 + 16, 100, 7)
    assert "ws is not 256-byte aligned" in e.value.message


def test_model_tail_checks_every_pointer():
    s = shape(rows=2)
    head = B.make_head(None, P16, None, P16 + 2)
    with pytest.raises(B.MonoError) as e:
        B.mono_hc_head(s, P16 + 4, head, None, None, None)
    msg = e.value.message
    for part in ("state is not 16-byte aligned", "head.w_head is NULL", "head.head_base is NULL",
                 "head.w_norm is not 16-byte aligned", "norm is NULL"):
        assert part in msg, (part, msg)
    B.mono_hc_head(shape(rows=0), P16, B.make_head(P16, P16, P16, P16), None, None, P16)
