"""The C ABI on the host, without a GPU: the library loads, exports every
function include/acceptmoe.h declares, and rejects bad arguments with the
documented codes before anything reaches the device.  No call here launches
a kernel: every call fails validation first."""

import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "acceptmoe.h")


@pytest.fixture(scope="module")
def m():
    import moe_speculative_decoding_gemm_amd as m
    return m


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\**\s+\**([a-z_0-9]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_exports_every_declared_symbol(m):
    names = declared_functions()
    assert len(names) >= 11, names
    lib = C.CDLL(m.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), f"{n} not exported"
    assert set(m.EXPORTED) == set(names)


def test_version_and_messages(m):
    assert "gfx950" in m.version()
    lib = m.raw()
    assert lib.acceptmoe_strerror(0) == b"success"
    assert lib.acceptmoe_strerror(-1) == b"invalid argument"
    assert lib.acceptmoe_strerror(-2) == b"unsupported dtype or flag"
    assert lib.acceptmoe_strerror(-3) == b"HIP launch failure"


FAKE = C.c_void_p(0x1000)  # never dereferenced: every call below fails validation


def _shape(m, **kw):
    base = dict(N=64, H=2048, I=768, E=128, k=8, n_depth=6)
    base.update(kw)
    return m.make_shape(base.pop("N"), base.pop("H"), base.pop("I"), base.pop("E"),
                        base.pop("k"), base.pop("n_depth"), **base)


@pytest.mark.parametrize("kw,code", [
    (dict(N=0), -1), (dict(N=4097), -1), (dict(k=0), -1), (dict(k=17), -1),
    (dict(E=4, k=8), -1), (dict(E=257), -1), (dict(H=100), -1), (dict(I=96), -1),
    (dict(n_depth=0), -1), (dict(min_set=129), -1), (dict(fixed_budget=-1), -1),
    (dict(reroute_budget=-2), -1), (dict(act_dtype=0, w_dtype=1), -2),
    (dict(act_dtype=2, w_dtype=2), -2), (dict(w_dtype=2, H=2048 + 64), -1),
    (dict(flags=64), -2),
])
def test_shape_validation(m, kw, code):
    lib = m.raw()
    s = _shape(m, **kw)
    assert lib.acceptmoe_workspace_size(C.byref(s)) == 0
    inp = m.Inputs(*([FAKE.value] * 16))
    out = m.Outputs(*([FAKE.value] * 8))
    rc = lib.verify_block(C.byref(s), C.byref(inp), C.byref(out), FAKE, 1 << 40, None)
    assert rc == code, lib.acceptmoe_last_error()


def test_workspace_sizes_and_small_workspace(m):
    lib = m.raw()
    s = _shape(m)
    need = lib.acceptmoe_workspace_size(C.byref(s))
    # h_perm (bf16) and y_perm (fp32) dominate: N*k*(2I + 4H) bytes
    assert need >= 64 * 8 * (2 * 768 + 4 * 2048)
    inp = m.Inputs(*([FAKE.value] * 16))
    inp.w13_shared = None
    out = m.Outputs(*([FAKE.value] * 8))
    rc = lib.verify_block(C.byref(s), C.byref(inp), C.byref(out), FAKE, need - 1, None)
    assert rc == -1 and b"workspace" in lib.acceptmoe_last_error()
    sel = lib.acceptmoe_select_workspace_size(C.byref(s))
    assert 0 < sel < need
    args = [FAKE] * 13
    rc = lib.acceptmoe_select(C.byref(s), *args, FAKE, sel - 1, None)
    assert rc == -1
    assert lib.moe_grouped_swiglu_workspace_size(64, 8, 768, 1) >= 64 * 8 * 768 * 2


def test_null_pointers_rejected(m):
    lib = m.raw()
    s = _shape(m)
    inp = m.Inputs(*([FAKE.value] * 16))
    inp.parent = None
    out = m.Outputs(*([FAKE.value] * 8))
    assert lib.verify_block(C.byref(s), C.byref(inp), C.byref(out), FAKE, 1 << 40, None) == -1
    inp = m.Inputs(*([FAKE.value] * 16))
    out.y = None
    assert lib.verify_block(C.byref(s), C.byref(inp), C.byref(out), FAKE, 1 << 40, None) == -1
    assert lib.verify_block(None, C.byref(inp), C.byref(out), FAKE, 1 << 40, None) == -1
    # fp8 without scales
    s8 = _shape(m, w_dtype=2)
    inp = m.Inputs(*([FAKE.value] * 16))
    inp.s13 = None
    out = m.Outputs(*([FAKE.value] * 8))
    assert lib.verify_block(C.byref(s8), C.byref(inp), C.byref(out), FAKE, 1 << 40, None) == -1
    # shared expert half given
    inp = m.Inputs(*([FAKE.value] * 16))
    inp.w2_shared = None
    assert lib.verify_block(C.byref(s), C.byref(inp), C.byref(out), FAKE, 1 << 40, None) == -1
    # permute / combine / grouped argument checks
    P = [FAKE] * 7
    assert lib.moe_route_permute(0, 8, 128, *P, None) == -1
    assert lib.moe_route_permute(64, 8, 4, *P, None) == -1
    assert lib.moe_route_permute(64, 8, 128, FAKE, None, *P[2:], None) == -1
    assert lib.moe_combine(64, 8, 2048, 2, *([FAKE] * 5), None) == -2
    assert lib.moe_combine(64, 8, 100, 1, *([FAKE] * 5), None) == -1
    assert lib.moe_combine(64, 8, 2048, 1, None, FAKE, FAKE, None, FAKE, None) == -1
    G = [FAKE] * 10
    assert lib.moe_grouped_swiglu(64, 8, 128, 2048, 768, 0, 1, 0, *G, FAKE, 1 << 40, None) == -2
    assert lib.moe_grouped_swiglu(64, 8, 128, 2000, 768, 1, 1, 0, *G, FAKE, 1 << 40, None) == -1
    G8 = [FAKE] * 3 + [None] + [FAKE] * 6
    assert lib.moe_grouped_swiglu(64, 8, 128, 2048, 768, 1, 2, 0, *G8, FAKE, 1 << 40, None) == -1
    assert lib.moe_grouped_swiglu(64, 8, 128, 2048, 768, 1, 1, 0, *G, FAKE, 10, None) == -1
    assert lib.moe_grouped_swiglu(64, 8, 128, 2048, 768, 0, 0, 1, *G, FAKE, 1 << 40, None) == -2
    assert lib.moe_grouped_swiglu(64, 8, 128, 2048, 768, 1, 1, 7, *G, FAKE, 1 << 40, None) == -2


def test_packed_layout_rules(m):
    """The packed layout: sizes, and the cases it does not support."""
    lib = m.raw()
    s = _shape(m, w_layout=1)
    n13 = lib.acceptmoe_packed_size(C.byref(s), 0, 128)
    n2 = lib.acceptmoe_packed_size(C.byref(s), 1, 128)
    # same bytes as row-major (K = 2048 and 768 are whole 128-chunks)
    assert n13 == 128 * 2 * 768 * 2048 * 2 and n2 == 128 * 2048 * 768 * 2
    s_odd = _shape(m, H=2880, I=2880)        # reduction padded to 2944
    assert lib.acceptmoe_packed_size(C.byref(s_odd), 0, 1) == 2 * 2880 * 2944 * 2
    s8 = _shape(m, w_dtype=2, H=7168, I=2048)
    assert lib.acceptmoe_packed_size(C.byref(s8), 1, 256) == 256 * 7168 * 2048
    f32 = _shape(m, act_dtype=0, w_dtype=0, w_layout=1)
    assert lib.acceptmoe_packed_size(C.byref(f32), 0, 1) == 0
    inp = m.Inputs(*([FAKE.value] * 16))
    out = m.Outputs(*([FAKE.value] * 8))
    assert lib.verify_block(C.byref(f32), C.byref(inp), C.byref(out), FAKE, 1 << 40, None) == -2
    bad = _shape(m, w_layout=5)
    assert lib.verify_block(C.byref(bad), C.byref(inp), C.byref(out), FAKE, 1 << 40, None) == -2
    assert lib.acceptmoe_pack_experts(C.byref(s), 0, FAKE, FAKE, FAKE, FAKE, None) == -1
    assert lib.acceptmoe_pack_experts(C.byref(s), 4, FAKE, None, FAKE, FAKE, None) == -1
    assert lib.acceptmoe_pack_experts(C.byref(s), 4, None, None, None, None, None) == -1
    assert lib.acceptmoe_pack_experts(C.byref(f32), 4, FAKE, FAKE, FAKE, FAKE, None) == -2


def test_logits_in_requires_logits(m):
    lib = m.raw()
    s = _shape(m, flags=m.F_LOGITS_IN)
    inp = m.Inputs(*([FAKE.value] * 16))
    inp.logits_in = None
    out = m.Outputs(*([FAKE.value] * 8))
    assert lib.verify_block(C.byref(s), C.byref(inp), C.byref(out), FAKE, 1 << 40, None) == -1
    assert b"logits_in" in lib.acceptmoe_last_error()


def test_python_wrappers_reject_host_tensors(m):
    import torch
    s = _shape(m, N=4, H=64, I=64, E=16, k=2, n_depth=4)
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        m.acceptmoe_select(s, x, x, None, None, None, None, None, None, None, None, None,
                           None, None, None)


def test_noalloc_rejects_a_block_beyond_its_workspace(m):
    """verify_block_noalloc holds a fixed device workspace: a block that
    needs more (256 nodes of hidden size 7168) is refused before any launch."""
    lib = m.raw()
    sh = _shape(m, N=256, H=7168, I=2048, E=256, k=8, n_depth=8, w_dtype=m.FP8_E4M3FN)
    assert m.acceptmoe_workspace_size(sh) > m.NOALLOC_WORKSPACE_BYTES
    inp = m.Inputs(*([FAKE.value] * 16))
    out = m.Outputs(*([FAKE.value] * 8))
    assert lib.verify_block_noalloc(C.byref(sh), C.byref(inp), C.byref(out), None) == m.EINVAL
    assert b"NOALLOC_WORKSPACE_BYTES" in lib.acceptmoe_last_error()
    # and argument errors come first, as for verify_block
    assert lib.verify_block_noalloc(None, C.byref(inp), C.byref(out), None) == m.EINVAL
    sh64 = _shape(m)
    assert m.acceptmoe_workspace_size(sh64) <= m.NOALLOC_WORKSPACE_BYTES
    assert lib.verify_block_noalloc(C.byref(sh64), None, C.byref(out), None) == m.EINVAL


def test_overlap_argument_checks(m):
    """verify_block_overlap refuses a missing side stream or event, and a side
    stream equal to the call's stream, before anything is enqueued."""
    lib = m.raw()
    sh = _shape(m, w_layout=m.LAYOUT_PACKED)
    inp = m.Inputs(*([FAKE.value] * 16))
    out = m.Outputs(*([FAKE.value] * 8))
    ws_bytes = m.acceptmoe_workspace_size(sh)
    stream = C.c_void_p(0x2000)
    ok = m.Overlap(0x3000, 0x4000, 0x5000)
    cases = [None, m.Overlap(None, 0x4000, 0x5000), m.Overlap(0x3000, None, 0x5000),
             m.Overlap(0x3000, 0x4000, None), m.Overlap(0x2000, 0x4000, 0x5000)]
    for ov in cases:
        ref = C.byref(ov) if ov is not None else None
        rc = lib.verify_block_overlap(C.byref(sh), C.byref(inp), C.byref(out), ref, FAKE,
                                      ws_bytes, stream)
        assert rc == m.EINVAL, ov
    # a valid overlap descriptor still fails the workspace check first
    rc = lib.verify_block_overlap(C.byref(sh), C.byref(inp), C.byref(out), C.byref(ok), FAKE,
                                  ws_bytes - 1, stream)
    assert rc == m.EINVAL and b"workspace" in lib.acceptmoe_last_error()
