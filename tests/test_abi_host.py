"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every
symbol include/moe.h declares, sizes its workspace, and rejects bad arguments
with the documented status codes before anything reaches the GPU."""
import ctypes
import os
import re

import pytest

import mixture_experts_layer_48_amd as M

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return M.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert {"moe_route", "moe_permute", "moe_expert_ffn", "moe_combine", "moe_layer_forward"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert b"gfx950" in lib.moe_version()
    assert lib.moe_status_str(M.MOE_ERR_WORKSPACE) == b"MOE_ERR_WORKSPACE"
    assert lib.moe_status_str(M.MOE_OK) == b"MOE_OK"


def _desc(**kw):
    base = dict(T=64, d=128, N=8, k=2, d_ff=256, dtype="bf16", ffn="swiglu", gating="topk_softmax")
    base.update(kw)
    return M.make_desc(**base)


def test_workspace_size_grows_with_tokens_and_is_zero_when_invalid():
    # both above the decode regime (> 16 routed rows per expert)
    a = M.moe_workspace_size(_desc(T=128))
    b = M.moe_workspace_size(_desc(T=256))
    assert 0 < a < b
    assert M.moe_workspace_size(_desc(k=9)) == 0
    # hidden state and per-row outputs dominate: (T*k rows) x (d_ff + d) x 2 bytes at least
    assert a >= 128 * 2 * (256 + 128) * 2
    cap = M.moe_workspace_size(_desc(T=128, capacity_factor=2.0))
    assert cap >= a + 128 * 8           # ranked expert lists


def test_x_size_limit_applies_to_bf16_only():
    # the grouped GEMM addresses x with 32-bit byte offsets: bf16 x must stay below 4 GiB
    assert M.moe_workspace_size(_desc(T=(1 << 19) - 1, d=4096)) > 0
    assert M.moe_workspace_size(_desc(T=1 << 19, d=4096)) == 0
    assert M.moe_workspace_size(_desc(T=1 << 19, d=4096, dtype="f32")) > 0


def test_expert_matrix_size_limit_applies_to_bf16_only():
    # one expert's weight matrix is read through 32-bit byte offsets: d * d_ff * 2 < 2^32 on bf16
    assert M.moe_workspace_size(_desc(T=16, d=65536, d_ff=32768 - 64)) > 0
    assert M.moe_workspace_size(_desc(T=16, d=65536, d_ff=32768)) == 0
    assert M.moe_workspace_size(_desc(T=16, d=32768, d_ff=65536)) == 0
    assert M.moe_workspace_size(_desc(T=16, d=65536, d_ff=32768, dtype="f32")) > 0


FAKE = 0x1000   # never dereferenced: every call below fails validation on the host


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), M.MOE_ERR_INVALID_ARG),
    (dict(k=9), M.MOE_ERR_INVALID_ARG),
    (dict(N=0, k=1), M.MOE_ERR_INVALID_ARG),
    (dict(T=-1), M.MOE_ERR_INVALID_ARG),
    (dict(d=0), M.MOE_ERR_INVALID_ARG),
    (dict(dtype=7), M.MOE_ERR_INVALID_ARG),
    (dict(ffn=5), M.MOE_ERR_INVALID_ARG),
    (dict(gating=3), M.MOE_ERR_INVALID_ARG),
    (dict(capacity_factor=float("nan")), M.MOE_ERR_INVALID_ARG),
    (dict(N=300, k=2), M.MOE_ERR_UNSUPPORTED),
    (dict(d=100), M.MOE_ERR_UNSUPPORTED),
    (dict(d_ff=200), M.MOE_ERR_UNSUPPORTED),
    (dict(T=1 << 19, d=4096), M.MOE_ERR_UNSUPPORTED),     # bf16 x of exactly 4 GiB
    (dict(d=65536, d_ff=32768), M.MOE_ERR_UNSUPPORTED),   # bf16 expert matrix of exactly 4 GiB
])
def test_descriptor_errors(lib, kw, status):
    desc = _desc(**kw)
    wt = M.moe_weights(FAKE, None, FAKE, FAKE, FAKE, None, None, None)
    r = M.moe_routing()
    st = lib.moe_layer_forward(ctypes.byref(desc), ctypes.byref(wt), FAKE, FAKE, ctypes.byref(r), FAKE,
                               1 << 40, None)
    assert st == status
    assert lib.moe_last_error() != b""


def test_fp32_layer_has_no_divisibility_requirement(lib):
    assert M.moe_workspace_size(_desc(dtype="f32", d=100, d_ff=37)) > 0


def test_missing_pointers_and_small_workspace(lib):
    desc = _desc()
    r = M.moe_routing()
    good = M.moe_weights(FAKE, None, FAKE, FAKE, FAKE, None, None, None)
    need = M.moe_workspace_size(desc)
    # x missing
    assert lib.moe_layer_forward(ctypes.byref(desc), ctypes.byref(good), None, FAKE, ctypes.byref(r), FAKE,
                                 need, None) == M.MOE_ERR_INVALID_ARG
    # SwiGLU without w_gate
    nogate = M.moe_weights(FAKE, None, None, FAKE, FAKE, None, None, None)
    assert lib.moe_layer_forward(ctypes.byref(desc), ctypes.byref(nogate), FAKE, FAKE, ctypes.byref(r), FAKE,
                                 need, None) == M.MOE_ERR_INVALID_ARG
    # shared expert requested but absent
    dsh = _desc(has_shared=True)
    assert lib.moe_layer_forward(ctypes.byref(dsh), ctypes.byref(good), FAKE, FAKE, ctypes.byref(r), FAKE,
                                 M.moe_workspace_size(dsh), None) == M.MOE_ERR_INVALID_ARG
    # workspace one byte short, or absent
    assert lib.moe_layer_forward(ctypes.byref(desc), ctypes.byref(good), FAKE, FAKE, ctypes.byref(r), FAKE,
                                 need - 1, None) == M.MOE_ERR_WORKSPACE
    assert lib.moe_layer_forward(ctypes.byref(desc), ctypes.byref(good), FAKE, FAKE, ctypes.byref(r), None,
                                 need, None) == M.MOE_ERR_WORKSPACE
    # stage entry points
    assert lib.moe_route(ctypes.byref(desc), FAKE, FAKE, None, None, None, FAKE, FAKE, need, None) \
        == M.MOE_ERR_INVALID_ARG
    assert lib.moe_route(ctypes.byref(desc), FAKE, FAKE, None, None, FAKE, FAKE, None, 0, None) \
        == M.MOE_ERR_WORKSPACE
    assert lib.moe_permute(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, None, None, None, None) \
        == M.MOE_ERR_INVALID_ARG
    assert lib.moe_permute(ctypes.byref(desc), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None) \
        == M.MOE_ERR_INVALID_ARG
    assert lib.moe_expert_ffn(ctypes.byref(desc), ctypes.byref(good), FAKE, FAKE, FAKE, None, FAKE, FAKE, 16,
                              None) == M.MOE_ERR_WORKSPACE
    assert lib.moe_combine(ctypes.byref(desc), None, FAKE, None, FAKE, None) == M.MOE_ERR_INVALID_ARG
    # NULL entries in the events array are allowed (no event at that boundary); the timed entry
    # point validates the rest like the plain one
    events = (ctypes.c_void_p * (M.MOE_NUM_STAGES + 1))(*([None] * 3 + [FAKE, FAKE] + [None] * (M.MOE_NUM_STAGES - 4)))
    assert lib.moe_layer_forward_timed(ctypes.byref(desc), ctypes.byref(good), FAKE, FAKE, ctypes.byref(r), FAKE,
                                       need - 1, None, events) == M.MOE_ERR_WORKSPACE
    assert lib.moe_layer_forward_timed(ctypes.byref(desc), ctypes.byref(good), None, FAKE, ctypes.byref(r), FAKE,
                                       need, None, events) == M.MOE_ERR_INVALID_ARG


def test_routing_stats_argument_errors(lib):
    desc = _desc(T=300, N=64, k=4)
    need = M.moe_workspace_size(desc)
    call = lambda d, z, i, c, alpha, st, t3, ws, nb: lib.moe_routing_stats(  # noqa: E731
        ctypes.byref(d), z, i, c, alpha, st, t3, None, ws, nb, None)
    assert call(desc, None, FAKE, FAKE, 0.01, FAKE, FAKE, FAKE, need) == M.MOE_ERR_INVALID_ARG
    assert call(desc, FAKE, FAKE, FAKE, 0.01, FAKE, None, FAKE, need) == M.MOE_ERR_INVALID_ARG
    assert call(desc, FAKE, FAKE, FAKE, float("inf"), FAKE, FAKE, FAKE, need) == M.MOE_ERR_INVALID_ARG
    assert call(_desc(T=0), FAKE, FAKE, FAKE, 0.01, FAKE, FAKE, FAKE, need) == M.MOE_ERR_INVALID_ARG
    assert call(desc, FAKE, FAKE, FAKE, 0.01, FAKE, FAKE, None, need) == M.MOE_ERR_WORKSPACE
    assert call(desc, FAKE, FAKE, FAKE, 0.01, FAKE, FAKE, FAKE, 64) == M.MOE_ERR_WORKSPACE
    assert call(_desc(k=0), FAKE, FAKE, FAKE, 0.01, FAKE, FAKE, FAKE, need) == M.MOE_ERR_INVALID_ARG
    assert b"workspace" in lib.moe_last_error() or b"k must" in lib.moe_last_error()


def test_ep_argument_errors(lib):
    desc = _desc(T=100, N=8, k=2)
    own = lambda v: (ctypes.c_int32 * len(v))(*v)  # noqa: E731
    ok = own([0, 0, 1, 1, 2, 2, 3, 3])
    F = [FAKE] * 6
    # owner out of range, G out of range, missing outputs, x without send_buf
    assert lib.moe_ep_dispatch(ctypes.byref(desc), FAKE, own([0, 0, 1, 1, 2, 2, 3, 4]), 4, *F, None, None,
                               None) == M.MOE_ERR_INVALID_ARG
    assert b"owner[7]" in lib.moe_last_error()
    assert lib.moe_ep_dispatch(ctypes.byref(desc), FAKE, ok, 0, *F, None, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_ep_dispatch(ctypes.byref(desc), FAKE, ok, 65, *F, None, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_ep_dispatch(ctypes.byref(desc), FAKE, None, 4, *F, None, None, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_ep_dispatch(ctypes.byref(desc), FAKE, ok, 4, FAKE, None, FAKE, FAKE, FAKE, FAKE, None, None,
                               None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_ep_dispatch(ctypes.byref(desc), FAKE, ok, 4, *F, FAKE, None, None) == M.MOE_ERR_INVALID_ARG
    # receive layout: rank outside [0, G), too many (source, local expert) pairs, missing outputs
    assert lib.moe_ep_receive_layout(8, 4, ok, 4, FAKE, 10, FAKE, FAKE, FAKE, FAKE, None) == M.MOE_ERR_INVALID_ARG
    big = own([0] * 256)
    assert lib.moe_ep_receive_layout(256, 64, big, 0, FAKE, 10, FAKE, FAKE, FAKE, FAKE, None) \
        == M.MOE_ERR_UNSUPPORTED
    assert lib.moe_ep_receive_layout(8, 4, ok, 1, FAKE, 10, FAKE, None, FAKE, FAKE, None) == M.MOE_ERR_INVALID_ARG
    # unpack: row size not a multiple of 16, missing buffers
    assert lib.moe_ep_unpack(4, 10, 24, FAKE, FAKE, FAKE, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_ep_unpack(4, 10, 32, FAKE, None, FAKE, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_ep_unpack(4, 0, 32, None, None, None, None, None) == M.MOE_OK


def test_q4_argument_errors(lib):
    assert lib.moe_quantize_q4(FAKE, 2, 16, 192, FAKE, FAKE, None) == M.MOE_ERR_UNSUPPORTED
    assert lib.moe_quantize_q4(FAKE, 2, 16, 256, None, FAKE, None) == M.MOE_ERR_INVALID_ARG
    assert lib.moe_quantize_q4(None, 0, 16, 256, None, None, None) == M.MOE_OK
    m = M.moe_q4_matrix(FAKE, FAKE)
    none = M.moe_q4_matrix(None, None)
    q = M.moe_weights_q4(FAKE, None, m, m, m, none, none, none)
    r = M.moe_routing()
    desc = _desc(d=128, d_ff=256)
    need = M.moe_workspace_size(desc)
    fwd = lambda d, w, ws: lib.moe_layer_forward_q4(ctypes.byref(d), ctypes.byref(w), FAKE, FAKE,  # noqa: E731
                                                    ctypes.byref(r), FAKE, ws, None, None)
    assert fwd(_desc(dtype="f32", d=128, d_ff=256), q, 1 << 40) == M.MOE_ERR_UNSUPPORTED
    assert fwd(_desc(d=192, d_ff=256), q, 1 << 40) == M.MOE_ERR_UNSUPPORTED
    assert fwd(_desc(d=128, d_ff=320), q, 1 << 40) == M.MOE_ERR_UNSUPPORTED
    nogate = M.moe_weights_q4(FAKE, None, none, m, m, none, none, none)
    assert fwd(desc, nogate, need) == M.MOE_ERR_INVALID_ARG
    half = M.moe_weights_q4(FAKE, None, m, M.moe_q4_matrix(FAKE, None), m, none, none, none)
    assert fwd(desc, half, need) == M.MOE_ERR_INVALID_ARG
    assert fwd(_desc(d=128, d_ff=256, has_shared=True), q, 1 << 40) == M.MOE_ERR_INVALID_ARG
    assert fwd(desc, q, need - 1) == M.MOE_ERR_WORKSPACE
    assert lib.moe_expert_ffn_q4(ctypes.byref(desc), ctypes.byref(q), FAKE, FAKE, FAKE, None, FAKE, FAKE, 16,
                                 None) == M.MOE_ERR_WORKSPACE


def test_header_constants_match_binding():
    text = open(HEADER).read()
    assert int(re.search(r"#define MOE_NUM_STATS (\d+)", text).group(1)) == M.MOE_NUM_STATS == len(M.STAT_NAMES)
    assert int(re.search(r"#define MOE_NUM_STAGES (\d+)", text).group(1)) == M.MOE_NUM_STAGES
    assert int(re.search(r"#define MOE_EP_MAX_RANKS (\d+)", text).group(1)) == M.MOE_EP_MAX_RANKS
    block = text[text.index("#define MOE_NUM_STATS") - 1200:text.index("#define MOE_NUM_STATS")]
    listed = re.findall(r"\*\s+\d\s+([a-z0-9_]+)", block)
    assert tuple(listed) == M.STAT_NAMES


def test_empty_batch_is_a_no_op(lib):
    desc = _desc(T=0)
    good = M.moe_weights(FAKE, None, FAKE, FAKE, FAKE, None, None, None)
    r = M.moe_routing()
    assert lib.moe_layer_forward(ctypes.byref(desc), ctypes.byref(good), FAKE, FAKE, ctypes.byref(r), FAKE,
                                 M.moe_workspace_size(desc), None) == M.MOE_OK


def test_binding_raises_with_detail():
    with pytest.raises(M.MoeError) as ei:
        M.moe_combine(_desc(k=0), None, None, None, None, stream=0)
    assert ei.value.status == M.MOE_ERR_INVALID_ARG
    assert "k must satisfy" in str(ei.value)
