"""C ABI checks that need no GPU: the library loads, exports every symbol include/moe.h declares,
computes sizes on the host, and rejects invalid arguments before any HIP call.

Also checks that the oracle and the HIP path stay independent (neither imports the other).
"""
import ctypes
import os
import re

import pytest

import combine_router_gemm_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED = -1, -2
FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: validation fails before any use


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(moe.library_path()):
        pytest.skip("HIP library not built (python -m combine_router_gemm_amd.build)")
    return moe.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = _declared_functions()
    assert set(names) == set(moe.EXPORTED_SYMBOLS)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    assert moe.moe_status_string(0) == "ok"
    assert moe.moe_status_string(-1) == "invalid argument"
    assert moe.moe_status_string(-2) == "unsupported shape or dtype"
    assert moe.moe_status_string(-3) == "HIP launch error"


def test_rows_max(lib):
    assert moe.moe_rows_max(4096, 8, 256, 128) == 32768
    assert moe.moe_rows_max(128, 8, 384, 4) == 1024
    assert moe.moe_rows_max(16384, 8, 256, 512) == 131072
    assert moe.moe_rows_max(256, 2, 8, 80) == 512
    assert moe.moe_rows_max(10, 2, 3, 2) == 6
    assert moe.moe_rows_max(0, 2, 8, 5) == 0
    assert moe.moe_rows_max(10, 2, 8, 0) == 0


def test_workspace_sizes(lib):
    assert moe.moe_dispatch_workspace_bytes(4096, 8, 256) >= (16 * 256 + 4096 * 8) * 4
    assert moe.moe_dispatch_workspace_bytes(0, 8, 256) == 0
    # h [rows_max, F] bf16 dominates the MLP workspace
    assert moe.moe_expert_mlp_workspace_bytes(4096, 8, 256, 8, 128, 2048, moe.MOE_BF16) >= 32768 * 2048 * 2
    assert moe.moe_expert_mlp_workspace_bytes(256, 2, 8, 1, 80, 256, moe.MOE_F32) >= 512 * 256 * 4
    # the router's scratch: whole [T, E] fp32 partials when the H reduction is split, after (bf16, 2048+
    # tokens, H % 64 == 0) the router weight's three bf16 planes, 256-byte aligned
    for T, H, E in ((16384, 7168, 256), (128, 4096, 8), (256, 128, 8), (4096, 7168, 256)):
        for xdt in (moe.MOE_BF16, moe.MOE_F32):
            n = moe.moe_route_workspace_bytes(T, H, E, xdt)
            planes = ((3 * E * H * 2 + 255) // 256) * 256 if (xdt == moe.MOE_BF16 and T >= 2048) else 0
            assert n >= planes and (n - planes) % (T * E * 4) == 0 and n - planes != T * E * 4
    # few experts and tokens: one fused kernel, no scratch; many experts: split-K partials
    assert moe.moe_route_workspace_bytes(128, 4096, 8, moe.MOE_BF16) == 0
    assert moe.moe_route_workspace_bytes(4096, 4096, 16, moe.MOE_F32) == 0
    assert moe.moe_route_workspace_bytes(128, 7168, 384, moe.MOE_BF16) > 0
    assert moe.moe_route_workspace_bytes(128, 4096, 8, 9) == 0


def _route(lib, **kw):
    a = dict(x=FAKE, xdt=moe.MOE_BF16, w=FAKE, bias=None, stride=0, T=16, H=64, E=8, k=2, logits=FAKE,
             ids=FAKE, wts=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.moe_route(a["x"], a["xdt"], a["w"], a["bias"], a["stride"], a["T"], a["H"], a["E"], a["k"],
                         a["logits"], a["ids"], a["wts"], a["ws"], a["wsb"], None)


def test_route_rejects_invalid_arguments(lib):
    assert _route(lib, k=0) == MOE_ERR_INVALID
    assert _route(lib, k=9, E=16) == MOE_ERR_INVALID
    assert _route(lib, k=4, E=3) == MOE_ERR_INVALID
    assert _route(lib, E=513) == MOE_ERR_INVALID
    assert _route(lib, T=-1) == MOE_ERR_INVALID
    assert _route(lib, H=12) == MOE_ERR_UNSUPPORTED
    assert _route(lib, xdt=7) == MOE_ERR_UNSUPPORTED
    assert _route(lib, x=None) == MOE_ERR_INVALID
    assert _route(lib, ids=None) == MOE_ERR_INVALID
    assert _route(lib, bias=FAKE, stride=-1) == MOE_ERR_INVALID
    # needs scratch (split reduction) but none given
    assert _route(lib, T=128, H=7168, E=384, k=8, ws=None, wsb=0) == MOE_ERR_INVALID
    # T == 0 is a no-op that succeeds without touching anything
    assert _route(lib, T=0, x=None, logits=None, ids=None, wts=None) == 0


def _layout(**kw):
    d = dict(T=16, k=2, E=8, R=1, C=4, H=64)
    d.update(kw)
    arr = [FAKE.value] * 7
    for name in kw.get("null", ()):
        arr[["expert_count", "expert_kept", "expert_overflow", "expert_offset", "row_token", "row_slot",
             "pair_row"].index(name)] = None
    d.pop("null", None)
    return moe._CLayout(d["T"], d["k"], d["E"], d["R"], d["C"], d["H"], *arr)


def test_dispatch_rejects_invalid_arguments(lib):
    def call(L, xdt=moe.MOE_BF16, x=FAKE, ids=FAKE, sb=FAKE, ws=FAKE, wsb=1 << 30):
        return lib.moe_dispatch(x, xdt, ids, ctypes.byref(L), sb, ws, wsb, None)
    assert lib.moe_dispatch(FAKE, moe.MOE_BF16, FAKE, None, FAKE, FAKE, 1 << 30, None) == MOE_ERR_INVALID
    assert call(_layout(E=10, R=3)) == MOE_ERR_INVALID          # E % R != 0
    assert call(_layout(k=9, E=16)) == MOE_ERR_INVALID
    assert call(_layout(C=-1)) == MOE_ERR_INVALID
    assert call(_layout(H=60)) == MOE_ERR_UNSUPPORTED
    assert call(_layout(), xdt=3) == MOE_ERR_UNSUPPORTED
    assert call(_layout(null=("pair_row",))) == MOE_ERR_INVALID
    assert call(_layout(null=("expert_offset",))) == MOE_ERR_INVALID
    assert call(_layout(), sb=None) == MOE_ERR_INVALID
    assert call(_layout(), ws=None) == MOE_ERR_INVALID
    assert call(_layout(), wsb=16) == MOE_ERR_INVALID


def test_dispatch_noalloc_rejects_invalid_arguments_and_sizes_beyond_its_scratch(lib):
    def call(L, xdt=moe.MOE_BF16, x=FAKE, ids=FAKE, sb=FAKE):
        return lib.moe_dispatch_noalloc(x, xdt, ids, ctypes.byref(L), sb, None)
    assert lib.moe_dispatch_noalloc(FAKE, moe.MOE_BF16, FAKE, None, FAKE, None) == MOE_ERR_INVALID
    assert call(_layout(E=10, R=3)) == MOE_ERR_INVALID
    assert call(_layout(H=60)) == MOE_ERR_UNSUPPORTED
    assert call(_layout(), xdt=3) == MOE_ERR_UNSUPPORTED
    assert call(_layout(), sb=None) == MOE_ERR_INVALID
    assert call(_layout(), x=ctypes.c_void_p(0x1008)) == MOE_ERR_INVALID
    # the static scratch holds (T / 256 blocks) x E counts and T * k ranks: 65536 x 8 x 512 fits, more does not
    cap = moe.MOE_DISPATCH_NOALLOC_MAX_WORKSPACE
    assert lib.moe_dispatch_workspace_bytes(65536, 8, 512) <= cap
    assert lib.moe_dispatch_workspace_bytes(131072, 8, 512) > cap
    assert call(_layout(T=131072, k=8, E=512, C=2048)) == MOE_ERR_UNSUPPORTED


def test_mlp_and_combine_reject_invalid_arguments(lib):
    L = _layout()
    assert lib.moe_expert_mlp(FAKE, moe.MOE_BF16, ctypes.byref(L), FAKE, FAKE, 0, FAKE, FAKE, 1 << 30,
                              None) == MOE_ERR_INVALID
    assert lib.moe_expert_mlp(FAKE, moe.MOE_BF16, ctypes.byref(L), FAKE, FAKE, 12, FAKE, FAKE, 1 << 30,
                              None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_expert_mlp(FAKE, moe.MOE_BF16, ctypes.byref(L), None, FAKE, 64, FAKE, FAKE, 1 << 30,
                              None) == MOE_ERR_INVALID
    assert lib.moe_expert_mlp(FAKE, moe.MOE_BF16, ctypes.byref(L), FAKE, FAKE, 64, FAKE, FAKE, 8,
                              None) == MOE_ERR_INVALID
    assert lib.moe_combine(FAKE, moe.MOE_BF16, ctypes.byref(L), None, FAKE, None) == MOE_ERR_INVALID
    assert lib.moe_combine(FAKE, 5, ctypes.byref(L), FAKE, FAKE, None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_combine(FAKE, moe.MOE_BF16, ctypes.byref(_layout(E=0)), FAKE, FAKE, None) == MOE_ERR_INVALID


def test_fused_combine_rejects_invalid_arguments_and_sizes_its_workspace(lib):
    L = _layout(T=16, k=2, E=8, R=1, C=4, H=64)
    base = lib.moe_expert_mlp_workspace_bytes(16, 2, 8, 1, 4, 64, moe.MOE_BF16)
    fused = lib.moe_expert_mlp_combine_workspace_bytes(16, 2, 8, 1, 4, 64, 64, moe.MOE_BF16)
    assert fused > base                          # plus one counter per (token, column band)
    assert lib.moe_expert_mlp_combine_workspace_bytes(16, 2, 8, 3, 4, 64, 64, moe.MOE_BF16) == 0  # E % R != 0

    def call(L, topk_w=FAKE, y=FAKE, ws=FAKE, wsb=1 << 30, F=64):
        return lib.moe_expert_mlp_combine(FAKE, moe.MOE_BF16, ctypes.byref(L), FAKE, FAKE, F, topk_w, FAKE, y, ws,
                                          wsb, None)
    assert call(L, topk_w=None) == MOE_ERR_INVALID
    assert call(L, y=None) == MOE_ERR_INVALID
    assert call(L, ws=None) == MOE_ERR_INVALID
    assert call(L, wsb=base) == MOE_ERR_INVALID   # the plain expert-MLP workspace is too small
    assert call(L, F=12) == MOE_ERR_UNSUPPORTED
    assert call(_layout(R=3)) == MOE_ERR_INVALID


def test_misaligned_pointers_are_rejected(lib):
    ODD16 = ctypes.c_void_p(0x1008)   # 8-byte aligned, not 16
    ODD4 = ctypes.c_void_p(0x1002)    # 2-byte aligned
    L = _layout()
    # activations and rows need 16 bytes, int / fp32 arrays 4
    assert lib.moe_dispatch(ODD16, moe.MOE_BF16, FAKE, ctypes.byref(L), FAKE, FAKE, 1 << 30, None) == MOE_ERR_INVALID
    assert lib.moe_dispatch(FAKE, moe.MOE_BF16, ODD4, ctypes.byref(L), FAKE, FAKE, 1 << 30, None) == MOE_ERR_INVALID
    assert lib.moe_combine(FAKE, moe.MOE_BF16, ctypes.byref(L), FAKE, ODD16, None) == MOE_ERR_INVALID
    assert lib.moe_combine(FAKE, moe.MOE_BF16, ctypes.byref(L), ODD4, FAKE, None) == MOE_ERR_INVALID
    assert lib.moe_expert_mlp(FAKE, moe.MOE_BF16, ctypes.byref(L), ODD16, FAKE, 64, FAKE, FAKE, 1 << 30, None) == \
        MOE_ERR_INVALID
    assert lib.moe_route(ODD16, moe.MOE_BF16, FAKE, None, 0, 16, 64, 8, 2, FAKE, FAKE, FAKE, FAKE, 1 << 30, None) == \
        MOE_ERR_INVALID
    assert lib.moe_combine_recv(ODD16, moe.MOE_BF16, ctypes.byref(L), FAKE, None) == MOE_ERR_INVALID
    # a misaligned layout array
    arr = [FAKE.value] * 7
    arr[6] = ODD4.value
    bad = moe._CLayout(16, 2, 8, 1, 4, 64, *arr)
    assert lib.moe_combine(FAKE, moe.MOE_BF16, ctypes.byref(bad), FAKE, FAKE, None) == MOE_ERR_INVALID


def test_sender_side_combine_rejects_invalid_arguments(lib):
    L = _layout(R=2)
    assert lib.moe_combine_send(FAKE, moe.MOE_BF16, ctypes.byref(L), FAKE, None, None) == MOE_ERR_INVALID
    assert lib.moe_combine_send(None, moe.MOE_BF16, ctypes.byref(L), FAKE, FAKE, None) == MOE_ERR_INVALID
    assert lib.moe_combine_send(FAKE, moe.MOE_BF16, ctypes.byref(L), None, FAKE, None) == MOE_ERR_INVALID
    assert lib.moe_combine_send(FAKE, 7, ctypes.byref(L), FAKE, FAKE, None) == MOE_ERR_UNSUPPORTED
    assert lib.moe_combine_recv(None, moe.MOE_BF16, ctypes.byref(L), FAKE, None) == MOE_ERR_INVALID
    assert lib.moe_combine_recv(FAKE, moe.MOE_BF16, ctypes.byref(L), None, None) == MOE_ERR_INVALID
    assert lib.moe_combine_recv(FAKE, moe.MOE_BF16, ctypes.byref(_layout(R=3)), FAKE, None) == MOE_ERR_INVALID
    assert lib.moe_combine_recv(FAKE, moe.MOE_F32, ctypes.byref(_layout(null=("pair_row",))), FAKE, None) == \
        MOE_ERR_INVALID
    # no tokens: nothing to do, nothing dereferenced
    assert lib.moe_combine_send(None, moe.MOE_BF16, ctypes.byref(_layout(T=0)), None, None, None) == 0
    assert lib.moe_combine_recv(None, moe.MOE_BF16, ctypes.byref(_layout(T=0)), None, None) == 0


def test_fp8_entry_points_reject_invalid_arguments(lib):
    def disp(L, xdt=moe.MOE_BF16, q=FAKE, sc=FAKE, ws=FAKE, wsb=1 << 30):
        return lib.moe_dispatch_fp8(FAKE, xdt, FAKE, ctypes.byref(L), q, sc, ws, wsb, None)
    assert disp(_layout(H=128), xdt=moe.MOE_F32) == MOE_ERR_UNSUPPORTED   # fp8 rows come from bf16 x
    assert disp(_layout(H=64)) == MOE_ERR_UNSUPPORTED                     # H not a multiple of the block
    assert disp(_layout(H=128), q=None) == MOE_ERR_INVALID
    assert disp(_layout(H=128), sc=None) == MOE_ERR_INVALID
    assert disp(_layout(H=128), ws=None) == MOE_ERR_INVALID
    assert disp(_layout(H=128, k=9, E=16)) == MOE_ERR_INVALID

    def mlp(L, sc=FAKE, F=64, wgu=FAKE, ws=FAKE, wsb=1 << 30):
        return lib.moe_expert_mlp_fp8(FAKE, sc, ctypes.byref(L), wgu, FAKE, F, FAKE, ws, wsb, None)
    assert mlp(_layout(H=64)) == MOE_ERR_UNSUPPORTED
    assert mlp(_layout(H=128), sc=None) == MOE_ERR_INVALID
    assert mlp(_layout(H=128), F=12) == MOE_ERR_UNSUPPORTED
    assert mlp(_layout(H=128), wgu=None) == MOE_ERR_INVALID
    assert mlp(_layout(H=128), wsb=8) == MOE_ERR_INVALID


def _py_sources(folder):
    for dirpath, _, files in os.walk(os.path.join(ROOT, folder)):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                yield os.path.join(dirpath, f)


def test_oracle_and_hip_path_are_independent():
    for path in _py_sources("oracle"):
        assert "combine_router_gemm_amd" not in open(path).read(), path
    for path in _py_sources("combine_router_gemm_amd"):
        text = open(path).read()
        assert not re.search(r"^\s*(import|from)\s+oracle\b", text, flags=re.M), path
    for path in _py_sources("moe_workloads"):
        text = open(path).read()
        assert not re.search(r"^\s*(import|from)\s+(oracle|combine_router_gemm_amd)\b", text, flags=re.M), path


def test_library_missing_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(moe, "_lib", None)
    monkeypatch.setattr(moe, "_PKG", str(tmp_path))
    with pytest.raises(moe.MoeError, match="missing"):
        moe.load_library()
