"""Host-side checks of the C ABI: the library loads, exports every function
include/moe_experts.h declares, sizes workspaces, and rejects bad arguments
before touching the GPU (no compute calls here)."""
import ctypes
import math
import os
import re

import pytest

from mixture_experts_expert_02_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_experts.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = B.lib()
    names = header_functions()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), f"{n} declared in the header but not exported"
    assert set(names) == set(B.EXPORTED)


def test_strerror():
    assert B.strerror(0) == "success"
    assert "workspace" in B.strerror(B.MOE_ENOSPC)
    assert B.strerror(12345) == "unknown status"


def test_workspace_bytes_monotone_and_aligned():
    prev = 0
    for T in (1, 7, 64, 513, 4096, 9000):
        p = B.problem(T, 4096, 14336, 8, 2)
        n = B.moe_experts_workspace_bytes(p)
        assert n % 256 == 0 and n > prev
        prev = n
    # act and y dominate: 2 bytes per element each
    p = B.problem(4096, 4096, 14336, 8, 2)
    assert B.moe_experts_workspace_bytes(p) >= 8192 * (4096 + 14336) * 2
    lay = B.moe_experts_workspace_layout(p)
    assert lay.status == 0 and lay.total == B.moe_experts_workspace_bytes(p)
    assert lay.act % 256 == 0 and lay.y % 256 == 0 and lay.y >= lay.act + 8192 * 14336 * 2


def test_workspace_room_for_split_down_projection(monkeypatch):
    # Few tiles (Mixtral-shaped prefill): y holds up to four partial outputs of
    # the down projection; MOE_EXPERTS_MAX_SPLIT_K caps that. Many tiles
    # (256 experts): no split, one output.
    p = B.problem(4096, 4096, 14336, 8, 2)
    full = B.moe_experts_workspace_bytes(p)
    monkeypatch.setenv("MOE_EXPERTS_MAX_SPLIT_K", "1")
    one = B.moe_experts_workspace_bytes(p)
    assert full - one == 3 * 8192 * 4096 * 2
    lay = B.moe_experts_workspace_layout(p)
    assert lay.total == lay.y + 8192 * 4096 * 2
    monkeypatch.delenv("MOE_EXPERTS_MAX_SPLIT_K")
    q = B.problem(8192, 7168, 2048, 256, 8)
    lay = B.moe_experts_workspace_layout(q)
    assert lay.total == lay.y + 65536 * 7168 * 2


@pytest.mark.parametrize("kw,code", [
    (dict(H=100), B.MOE_ENOTSUP),                 # not a multiple of 64
    (dict(I=96), B.MOE_ENOTSUP),
    (dict(E=0), B.MOE_EINVAL),
    (dict(k=9), B.MOE_EINVAL),                    # k > E
    (dict(k=0), B.MOE_EINVAL),
    (dict(T=-1), B.MOE_EINVAL),
    (dict(E=5000, k=2), B.MOE_ENOTSUP),           # beyond the LDS histogram
    (dict(act="swiglu_oai", limit=0.0), B.MOE_ENOTSUP),
    (dict(act="swiglu_oai", limit=-1.0), B.MOE_ENOTSUP),
    (dict(act="swiglu_oai", alpha=math.nan, limit=7.0), B.MOE_EINVAL),
    (dict(wfmt="mxfp4", H=16448), B.MOE_ENOTSUP),  # MXFP4 scale rows beyond the LDS staging limit
    (dict(wfmt="mxfp4", I=16448), B.MOE_ENOTSUP),
    (dict(T=1 << 20, H=2048, I=256), B.MOE_ENOTSUP),  # T*H = 2^31: beyond 32-bit row offsets
    (dict(T=1 << 18, k=2, H=128, I=4096), B.MOE_ENOTSUP),  # rows*I = 2^31
    (dict(H=32768, I=32832), B.MOE_ENOTSUP),      # one expert's I*H above 2^30
    (dict(act="situ", alpha=0.0, beta=1.0), B.MOE_ENOTSUP),   # SiTu needs alpha > 0 and beta > 0
    (dict(act="situ", alpha=1.0, beta=-1.0), B.MOE_ENOTSUP),
    (dict(act="situ", alpha=math.inf, beta=1.0), B.MOE_EINVAL),
    (dict(act=3), B.MOE_EINVAL),
    (dict(weight_on_input=2), B.MOE_EINVAL),
    (dict(act_fmt="mxfp8"), B.MOE_ENOTSUP),        # MXFP8 activations need MXFP4 weights
    (dict(act_fmt=2), B.MOE_EINVAL),
    (dict(wfmt="mxfp4", act_fmt=-1), B.MOE_EINVAL),
])
def test_invalid_problems_rejected(kw, code):
    base = dict(T=16, H=128, I=256, E=8, k=2)
    base.update(kw)
    p = B.problem(**base)
    assert B.moe_experts_workspace_bytes(p) == 0
    lay = B.MoeWsLayout()
    assert B.lib().moe_experts_workspace_layout(ctypes.byref(p), ctypes.byref(lay)) == B.MOE_EINVAL
    fake = ctypes.c_void_p(1 << 20)                # never dereferenced: validation fails first
    rc = B.lib().moe_experts_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None, None,
                                     fake, fake, 1 << 40, None)
    assert rc == code


def test_bad_enum_and_pointers_rejected():
    L = B.lib()
    fake = ctypes.c_void_p(1 << 20)
    p = B.problem(16, 128, 256, 8, 2)
    p.wfmt = 7
    assert L.moe_experts_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None, None, fake, fake,
                                 1 << 40, None) == B.MOE_EINVAL
    p = B.problem(16, 128, 256, 8, 2)
    for i in range(12):                            # each required pointer null in turn
        args = [fake] * 6 + [None, None, None] + [fake, fake]
        req = [0, 1, 2, 3, 4, 5, 9, 10]
        if i >= len(req):
            break
        args[req[i]] = None
        assert L.moe_experts_forward(ctypes.byref(p), *args, 1 << 40, None) == B.MOE_EINVAL
    # misaligned x
    odd = ctypes.c_void_p((1 << 20) + 2)
    assert L.moe_experts_forward(ctypes.byref(p), odd, fake, fake, fake, fake, fake, None, None, None, fake, fake,
                                 1 << 40, None) == B.MOE_EINVAL
    # MXFP4 needs scales
    p = B.problem(16, 128, 256, 8, 2, wfmt="mxfp4")
    assert L.moe_experts_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None, None, fake, fake,
                                 1 << 40, None) == B.MOE_EINVAL
    # MXFP4 scale arrays must be 16-byte aligned (the decode GEMM copies them in 16-byte pieces)
    odd_s = ctypes.c_void_p((1 << 20) + 4)
    for i in range(3):
        sc = [fake, fake, fake]
        sc[i] = odd_s
        assert L.moe_experts_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, *sc, fake, fake,
                                     1 << 40, None) == B.MOE_EINVAL
    # timed variant: event count must be 0 or 5
    p = B.problem(16, 128, 256, 8, 2)
    ev = (ctypes.c_void_p * 3)()
    assert L.moe_experts_forward_timed(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None, None, fake,
                                       fake, 1 << 40, None, ev, 3) == B.MOE_EINVAL


def test_short_workspace_rejected():
    L = B.lib()
    fake = ctypes.c_void_p(1 << 20)
    p = B.problem(64, 128, 256, 8, 2)
    need = B.moe_experts_workspace_bytes(p)
    assert L.moe_experts_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None, None, fake, fake,
                                 need - 1, None) == B.MOE_ENOSPC
    g = B.problem(100, 128, 256, 5)
    needg = B.moe_experts_grouped_workspace_bytes(g)
    assert needg > 0
    assert L.moe_experts_forward_grouped(ctypes.byref(g), fake, fake, fake, fake, fake, fake, None, None, None, fake,
                                         fake, needg - 1, None) == B.MOE_ENOSPC
    na = B.moe_align_workspace_bytes(64, 2, 8)
    assert na > 0
    assert L.moe_align(fake, 64, 2, 8, fake, fake, fake, fake, fake, na - 1, None) == B.MOE_ENOSPC
    assert L.moe_align(fake, 64, 9, 8, fake, fake, fake, fake, fake, 1 << 30, None) == B.MOE_EINVAL


def test_empty_input_is_a_noop():
    L = B.lib()
    fake = ctypes.c_void_p(1 << 20)
    p = B.problem(0, 128, 256, 8, 2)
    assert L.moe_experts_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None, None, fake, fake,
                                 B.moe_experts_workspace_bytes(p), None) == B.MOE_OK


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1, E=8, k=2), B.MOE_EINVAL),
    (dict(T=4, E=0, k=1), B.MOE_EINVAL),
    (dict(T=4, E=8, k=0), B.MOE_EINVAL),
    (dict(T=4, E=8, k=9), B.MOE_EINVAL),
    (dict(T=4, E=2048, k=2), B.MOE_ENOTSUP),
    (dict(T=4, E=64, k=33), B.MOE_ENOTSUP),
    (dict(T=4, E=8, k=2, method=5), B.MOE_EINVAL),
    (dict(T=4, E=12, k=2, method="deepseek_v3", n_group=5, topk_group=1), B.MOE_EINVAL),   # E % n_group
    (dict(T=4, E=8, k=2, method="deepseek_v3", n_group=8, topk_group=1), B.MOE_EINVAL),    # one expert per group
    (dict(T=4, E=16, k=2, method="deepseek_v3", n_group=4, topk_group=0), B.MOE_EINVAL),
    (dict(T=4, E=16, k=2, method="deepseek_v3", n_group=4, topk_group=5), B.MOE_EINVAL),
    (dict(T=4, E=16, k=9, method="deepseek_v3", n_group=4, topk_group=2), B.MOE_EINVAL),   # k > kept experts
    (dict(T=4, E=256, k=8, method="deepseek_v3", n_group=128, topk_group=4), B.MOE_EINVAL),  # > 64 groups
    (dict(T=4, E=8, k=2, method="deepseek_v3", routed_scaling_factor=math.inf), B.MOE_EINVAL),
])
def test_route_invalid_problems_rejected(kw, code):
    L = B.lib()
    fake = ctypes.c_void_p(1 << 20)
    p = B.route_problem(**kw)
    assert L.moe_route(ctypes.byref(p), fake, None, fake, fake, None) == code


def test_route_pointers_and_empty_input():
    L = B.lib()
    fake = ctypes.c_void_p(1 << 20)
    odd = ctypes.c_void_p((1 << 20) + 2)
    p = B.route_problem(4, 8, 2)
    for args in ([None, None, fake, fake], [fake, None, None, fake], [fake, None, fake, None],
                 [odd, None, fake, fake], [fake, odd, fake, fake]):
        assert L.moe_route(ctypes.byref(p), *args, None) == B.MOE_EINVAL
    assert L.moe_route(ctypes.byref(B.route_problem(0, 8, 2)), fake, None, fake, fake, None) == B.MOE_OK


def test_weight_on_input_workspace_holds_scaled_rows():
    p0 = B.problem(64, 128, 256, 8, 2)
    p1 = B.problem(64, 128, 256, 8, 2, weight_on_input=True)
    # p0 (a decode-shaped problem) may run as one launch after the align and
    # reserves 256 bytes of counters for it; p1 cannot (its rows are weighted first)
    assert B.moe_experts_workspace_layout(p1).single_launch == 0
    assert B.moe_experts_workspace_bytes(p1) >= B.moe_experts_workspace_bytes(p0) - 256 + 64 * 2 * 128 * 2
    g0 = B.problem(100, 128, 256, 5)
    g1 = B.problem(100, 128, 256, 5, weight_on_input=True)
    assert B.moe_experts_grouped_workspace_bytes(g1) >= B.moe_experts_grouped_workspace_bytes(g0) + 100 * 128 * 2


def test_grouped_timed_event_count_checked():
    L = B.lib()
    fake = ctypes.c_void_p(1 << 20)
    g = B.problem(100, 128, 256, 5)
    ev = (ctypes.c_void_p * 3)()
    assert L.moe_experts_forward_grouped_timed(ctypes.byref(g), fake, fake, fake, fake, fake, fake, None, None, None,
                                               fake, fake, 1 << 40, None, ev, 3) == B.MOE_EINVAL


def test_mxfp8_activations_need_mxfp4_weights():
    # checked on the host: no device needed
    ok = B.problem(32, 256, 256, 8, 2, wfmt="mxfp4", act_fmt="mxfp8")
    assert B.moe_experts_workspace_bytes(ok) > 0
    assert B.moe_experts_workspace_bytes(B.problem(32, 256, 256, 8, 2, wfmt="bf16", act_fmt="mxfp8")) == 0
    assert B.moe_experts_workspace_bytes(B.problem(32, 256, 256, 8, 2, wfmt="mxfp4", act_fmt=7)) == 0
    lay = B.moe_experts_workspace_layout(ok)
    assert lay.xq > 0 and lay.aq > lay.xq and lay.xq_rows == 32


# ------------------------------------------------------------------ per-expert parameters
def test_check_expert_params_host_rules():
    E = 4
    ok = [1.0, 0.5, 2.0, 3.0]
    silu = B.problem(8, 128, 256, E, 2)
    assert B.moe_check_expert_params(silu, fc1_alpha=ok, fc2_alpha=ok) == B.MOE_OK
    for bad, code in (([1.0, math.nan, 1.0, 1.0], B.MOE_EINVAL), ([1.0, math.inf, 1.0, 1.0], B.MOE_EINVAL),
                      ([1.0, 0.0, 1.0, 1.0], B.MOE_ENOTSUP), ([1.0, -2.0, 1.0, 1.0], B.MOE_ENOTSUP)):
        assert B.moe_check_expert_params(silu, fc1_alpha=bad) == code
        assert B.moe_check_expert_params(silu, fc2_alpha=bad) == code
    oai = B.problem(8, 128, 256, E, 2, act="swiglu_oai", alpha=1.702, beta=1.0, limit=7.0)
    assert B.moe_check_expert_params(oai, alpha_e=[1.7, -1.0, 0.0, 2.0], beta_e=[1.0, 0.0, -1.0, 1.0],
                                     limit_e=[7.0, math.inf, 1.0, 3.0]) == B.MOE_OK
    assert B.moe_check_expert_params(oai, limit_e=[7.0, math.nan, 1.0, 3.0]) == B.MOE_EINVAL
    assert B.moe_check_expert_params(oai, limit_e=[7.0, 0.0, 1.0, 3.0]) == B.MOE_ENOTSUP
    assert B.moe_check_expert_params(oai, alpha_e=[7.0, math.inf, 1.0, 3.0]) == B.MOE_EINVAL
    situ = B.problem(8, 128, 256, E, 2, act="situ", alpha=1.5, beta=0.8)
    assert B.moe_check_expert_params(situ, alpha_e=ok, beta_e=ok) == B.MOE_OK
    assert B.moe_check_expert_params(situ, alpha_e=[1.0, 1.0, 0.0, 1.0]) == B.MOE_ENOTSUP
    assert B.moe_check_expert_params(situ, beta_e=[1.0, 1.0, math.nan, 1.0]) == B.MOE_EINVAL
    # a problem the scalar checks reject is rejected here too
    assert B.moe_check_expert_params(B.problem(8, 128, 256, 0, 1)) == B.MOE_EINVAL


def test_misaligned_expert_param_pointer_rejected():
    for name in B.EXPERT_PARAMS:
        p = B.problem(64, 128, 256, 8, 2)
        setattr(p, name, (1 << 20) + 2)          # not 4-byte aligned; never dereferenced
        assert B.moe_experts_workspace_bytes(p) == 0
        fake = ctypes.c_void_p(1 << 20)
        assert B.lib().moe_experts_forward(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None, None,
                                           fake, fake, 1 << 40, None) == B.MOE_EINVAL


def test_mx_packed_bytes_and_pack_errors():
    """moe_mx_packed_bytes: one 17408-byte block per expert, column tile and
    128-K stage of each GEMM (MXFP4 weights, either activation format: the
    decode kernels read the codes too); moe_mx_pack_weights and
    moe_problem.mx_packed reject what the header says before any launch."""
    L = B.lib()
    T, H, I, E = 64, 2880, 2880, 4
    p = B.problem(T, H, I, E, 2, "mxfp4", "swiglu_oai", 1.702, 1.0, 7.0, act_fmt="mxfp8")
    blocks = E * (math.ceil(I / 128) * math.ceil(H / 128) + math.ceil(H / 256) * math.ceil(I / 128))
    assert B.moe_mx_packed_bytes(p) == blocks * 17408
    assert B.moe_mx_packed_bytes(B.problem(T, H, I, E, 2, "mxfp4", act_fmt="bf16")) == blocks * 17408
    assert B.moe_mx_packed_bytes(B.problem(T, H, I, E, 2)) == 0
    fake = ctypes.c_void_p(1 << 20)
    need = B.moe_mx_packed_bytes(p)
    args = [fake] * 7
    assert L.moe_mx_pack_weights(ctypes.byref(p), *args, need - 1, None) == B.MOE_ENOSPC
    for i in range(7):
        bad = list(args)
        bad[i] = None
        assert L.moe_mx_pack_weights(ctypes.byref(p), *bad, need, None) == B.MOE_EINVAL
        bad[i] = ctypes.c_void_p((1 << 20) + 8)
        assert L.moe_mx_pack_weights(ctypes.byref(p), *bad, need, None) == B.MOE_EINVAL
    q = B.problem(T, H, I, E, 2)
    assert L.moe_mx_pack_weights(ctypes.byref(q), *args, need, None) == B.MOE_EINVAL
    # packed weights with bf16 weights, or misaligned: the problem is invalid
    for wfmt, afmt, ptr in (("bf16", "bf16", 1 << 20), ("mxfp4", "bf16", (1 << 20) + 4),
                            ("mxfp4", "mxfp8", (1 << 20) + 4)):
        r = B.problem(T, H, I, E, 2, wfmt, act_fmt=afmt)
        r.mx_packed = ptr
        assert B.moe_experts_workspace_bytes(r) == 0
        assert B.moe_experts_grouped_workspace_bytes(r) == 0
    for afmt in ("bf16", "mxfp8"):
        r = B.problem(T, H, I, E, 2, "mxfp4", act_fmt=afmt)
        r.mx_packed = 1 << 20
        assert B.moe_experts_workspace_bytes(r) > 0


def test_bf16_packed_bytes_and_pack_errors():
    """moe_bf16_packed_bytes: the three weight sets at 2 E I H bytes each (bf16
    only); moe_bf16_pack_weights and moe_problem.bf16_packed reject what the
    header says before any launch."""
    L = B.lib()
    T, H, I, E = 64, 320, 192, 3
    p = B.problem(T, H, I, E, 2)
    assert B.moe_bf16_packed_bytes(p) == 3 * 2 * E * I * H
    assert B.moe_bf16_packed_bytes(B.problem(T, H, I, E, 2, "mxfp4")) == 0
    assert B.moe_bf16_packed_bytes(B.problem(T, H, I, 0, 2)) == 0
    assert B.moe_bf16_packed_bytes(B.problem(T, H, I, E, 0)) == 3 * 2 * E * I * H  # k is not looked at
    fake = ctypes.c_void_p(1 << 20)
    need = B.moe_bf16_packed_bytes(p)
    args = [fake] * 4
    assert L.moe_bf16_pack_weights(ctypes.byref(p), *args, need - 1, None) == B.MOE_ENOSPC
    for i in range(4):
        bad = list(args)
        bad[i] = None
        assert L.moe_bf16_pack_weights(ctypes.byref(p), *bad, need, None) == B.MOE_EINVAL
        bad[i] = ctypes.c_void_p((1 << 20) + 8)
        assert L.moe_bf16_pack_weights(ctypes.byref(p), *bad, need, None) == B.MOE_EINVAL
    q = B.problem(T, H, I, E, 2, "mxfp4")
    assert L.moe_bf16_pack_weights(ctypes.byref(q), *args, need, None) == B.MOE_EINVAL
    # operand-block weights with MXFP4 weights, or misaligned: the problem is invalid (both entries)
    for wfmt, ptr in (("mxfp4", 1 << 20), ("bf16", (1 << 20) + 4)):
        r = B.problem(T, H, I, E, 2, wfmt)
        r.bf16_packed = ptr
        assert B.moe_experts_workspace_bytes(r) == 0
        assert B.moe_experts_grouped_workspace_bytes(r) == 0
    r = B.problem(T, H, I, E, 2)
    r.bf16_packed = 1 << 20
    assert B.moe_experts_workspace_bytes(r) > 0
    assert B.moe_experts_grouped_workspace_bytes(r) > 0
