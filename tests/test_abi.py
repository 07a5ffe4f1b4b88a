"""CPU tests of the C-ABI boundary: the library loads, exports every entry
point include/na_attn.h declares, and rejects bad arguments on the host before
any HIP call (so these run without a GPU).  No compute call is made here."""
import ctypes
import os
import re
import subprocess

import pytest

import causal_self_attention_mha_amd as na

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "na_attn.h")

OK, INVALID, UNSUPPORTED, HIP = 0, 1, 2, 3


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(na_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    """The library, only where no GPU is visible: the calls below pass fake
    device addresses and rely on the host checks rejecting every one of them,
    so a regression in a check must never reach a real device."""
    if not os.path.exists(na.library_path()):
        pytest.skip("library not built")
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a GPU is visible: the fake-address calls run on CPU-only hosts")
    return na.load_library()


def test_header_declares_the_entry_points():
    syms = declared_symbols()
    for s in ("na_attn_fwd", "na_attn_bwd", "na_attn_decode", "na_attn_decode_workspace_bytes",
              "na_attn_bwd_workspace_bytes", "na_attn_bwd_timed", "na_attn_decode_timed",
              "na_attn_fwd_f32", "na_attn_bwd_f32", "na_status_string", "na_last_error",
              "na_attn_fwd_window", "na_attn_bwd_window", "na_attn_decode_window",
              "na_attn_fwd_gqa", "na_attn_bwd_gqa", "na_attn_decode_gqa", "na_attn_prefill",
              "na_qk_norm_rope_fwd", "na_qk_norm_rope_bwd", "na_value_gate_fwd",
              "na_value_gate_bwd", "na_attn_prefill_rope", "na_attn_decode_append",
              "na_attn_bwd_rope", "na_attn_fwd_rope"):
        assert s in syms


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", na.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)", out))
    for s in declared_symbols():
        assert s in exported, s
        assert hasattr(lib, s)


def test_status_strings(lib):
    for code, word in ((OK, b"NA_OK"), (INVALID, b"INVALID"), (UNSUPPORTED, b"UNSUPPORTED"),
                       (HIP, b"HIP")):
        assert word in lib.na_status_string(code)
    assert b"unknown" in lib.na_status_string(99)


A = 0x10000  # a fake, 16-byte aligned "device" address; never dereferenced.
# Every call below must fail a host-side check: a call that passed them would
# launch kernels on these addresses.


def fwd(lib, q=A, k=A + 0x100, v=A + 0x200, o=A + 0x300, lse=A + 0x400, B=1, T=8, H=1, D=128):
    return lib.na_attn_fwd(q, k, v, o, lse, B, T, H, D, None)


def test_fwd_rejects_bad_arguments(lib):
    assert fwd(lib, q=0) == INVALID and b"q is NULL" in lib.na_last_error()
    assert fwd(lib, lse=0) == INVALID
    assert fwd(lib, B=0) == INVALID
    assert fwd(lib, T=-1) == INVALID
    assert fwd(lib, H=0) == INVALID
    assert fwd(lib, D=64) == UNSUPPORTED and b"head dim" in lib.na_last_error()
    assert fwd(lib, k=A + 0x108) == INVALID and b"aligned" in lib.na_last_error()
    assert fwd(lib, o=A) == INVALID and b"aliases" in lib.na_last_error()
    assert fwd(lib, B=1, T=1 << 20, H=1 << 10) == UNSUPPORTED    # T*H*D >= 2^31 per batch
    assert fwd(lib, B=1 << 20, T=1 << 12, H=1) == INVALID        # B*H*T over the grid limit
    assert lib.na_attn_fwd_f32(A, A + 16, A + 32, A + 48, A, 1, 8, 1, 128, None) == INVALID


def test_bwd_rejects_bad_arguments(lib):
    p = [A + 0x100 * i for i in range(11)]   # q k v o dout lse dq dk dv delta workspace
    need = lib.na_attn_bwd_workspace_bytes(1, 8, 1, 128)

    def bwd(ptrs, ws_bytes=need, D=128, T=8):
        return lib.na_attn_bwd(*ptrs[:10], ptrs[10], ws_bytes, 1, T, 1, D, None)

    bad = list(p)
    bad[3] = 0                     # o
    assert bwd(bad) == INVALID
    bad = list(p)
    bad[7] = bad[6]                # dk == dq
    assert bwd(bad) == INVALID and b"alias" in lib.na_last_error()
    bad = list(p)
    bad[10] = bad[0]               # workspace == q
    assert bwd(bad) == INVALID
    assert bwd(p, ws_bytes=need - 1) == INVALID and b"workspace" in lib.na_last_error()
    assert bwd(p, D=96) == UNSUPPORTED
    bad = list(p)
    bad[10] = 0                    # no workspace: recompute path, still checks the rest
    bad[9] = 0                     # delta scratch
    assert bwd(bad) == INVALID
    assert lib.na_attn_bwd_f32(*bad[:5], bad[5], *bad[6:9], bad[9], 1, 8, 1, 128, None) == INVALID


def test_window_entry_points_check_their_arguments(lib):
    assert lib.na_attn_fwd_window(0, A, A + 0x100, A + 0x200, A + 0x300, 1, 8, 1, 128, 3,
                                  None) == INVALID
    assert lib.na_attn_fwd_window(A, A + 0x100, A + 0x200, A + 0x300, A + 0x400, 1, 8, 1, 64, 3,
                                  None) == UNSUPPORTED
    p = [A + 0x100 * i for i in range(11)]
    need = lib.na_attn_bwd_workspace_bytes(1, 8, 1, 128)
    # without a workspace (the recompute path) the usual checks apply ...
    bad = list(p)
    bad[9] = bad[0]                # delta == q
    assert lib.na_attn_bwd_window(*bad[:10], None, 0, 1, 8, 1, 128, 3, None, None) == INVALID
    assert lib.na_attn_bwd_window(*p[:10], None, 0, 1, 8, 1, 96, 3, None, None) == UNSUPPORTED
    # ... and with one
    bad = list(p)
    bad[7] = bad[6]
    assert lib.na_attn_bwd_window(*bad[:10], bad[10], need, 1, 8, 1, 128, 3, None,
                                  None) == INVALID
    d = [A + 0x100 * i for i in range(7)]   # q k v seqlens o lse workspace
    wneed = lib.na_attn_decode_workspace_bytes(4, 2, 128, 64)
    assert lib.na_attn_decode_window(d[0], d[1], d[2], 0, d[4], d[5], 4, 2, 128, 64, 5, d[6],
                                     wneed, None, None) == INVALID
    assert lib.na_attn_decode_window(*d[:6], 4, 2, 128, 64, 5, d[6], wneed - 1, None,
                                     None) == INVALID


def test_gqa_entry_points_check_the_head_counts(lib):
    f = lambda H, Hk: lib.na_attn_fwd_gqa(A, A + 0x100, A + 0x200, A + 0x300, A + 0x400,  # noqa
                                          1, 8, H, Hk, 128, -1, None)
    for H, Hk in ((4, 3), (4, 0), (4, 8), (6, -2)):
        assert f(H, Hk) == INVALID and b"H_kv" in lib.na_last_error()
    p = [A + 0x100 * i for i in range(11)]
    need = lib.na_attn_bwd_workspace_bytes(1, 8, 4, 128)
    assert lib.na_attn_bwd_gqa(*p[:10], p[10], need, 1, 8, 4, 3, 128, -1, None,
                               None) == INVALID
    bad = list(p)
    bad[7] = bad[6]  # dk aliases dq
    assert lib.na_attn_bwd_gqa(*bad[:10], bad[10], need, 1, 8, 4, 2, 128, -1, None,
                               None) == INVALID
    d = [A + 0x100 * i for i in range(7)]
    wneed = lib.na_attn_decode_workspace_bytes(4, 6, 128, 64)
    assert lib.na_attn_decode_gqa(*d[:6], 4, 6, 4, 128, 64, -1, d[6], wneed, None,
                                  None) == INVALID


def test_prefill_checks_its_arguments(lib):
    p = [A + 0x100 * i for i in range(8)]  # q k_new v_new k_cache v_cache lens o lse
    call = lambda ptrs, T_q=8, H=2, Hk=2, T_cap=64: lib.na_attn_prefill(  # noqa: E731
        *ptrs, 1, T_q, H, Hk, 128, T_cap, -1, None)
    assert call(p, T_cap=4) == INVALID and b"T_cap" in lib.na_last_error()
    assert call(p, H=4, Hk=3) == INVALID
    bad = list(p)
    bad[6] = bad[0]              # o aliases q
    assert call(bad) == INVALID
    bad = list(p)
    bad[5] = 0                   # no cache_lens
    assert call(bad) == INVALID


def test_prologue_checks_its_arguments(lib):
    p = [A + 0x100 * i for i in range(7)]  # q k q_out k_out cos sin pos_offset
    fwd = lambda ptrs, T=8, H=2, Hk=2, D=128, T_tab=16, eps=1e-6: lib.na_qk_norm_rope_fwd(  # noqa
        *ptrs, 1, T, H, Hk, D, T_tab, eps, None)
    assert fwd(p, T_tab=4) == INVALID and b"T_tab" in lib.na_last_error()
    assert fwd(p, D=64) == UNSUPPORTED
    assert fwd(p, Hk=0) == INVALID
    assert fwd(p, eps=-1.0) == INVALID and b"eps" in lib.na_last_error()
    assert fwd(p, eps=float("nan")) == INVALID
    bad = list(p)
    bad[2] = bad[0]              # q_out aliases q
    assert fwd(bad) == INVALID
    bad = list(p)
    bad[4] = 0                   # no cos table
    assert fwd(bad) == INVALID
    bad = list(p)
    bad[5] = A + 8               # sin table not 16-byte aligned
    assert fwd(bad) == INVALID
    g = [A + 0x100 * i for i in range(9)]  # q k dq_rot dk_rot dq dk cos sin pos_offset
    assert lib.na_qk_norm_rope_bwd(*g, 1, 8, 2, 2, 128, 4, 1e-6, None) == INVALID
    g[4] = g[2]                  # dq aliases dq_rot
    assert lib.na_qk_norm_rope_bwd(*g, 1, 8, 2, 2, 128, 16, 1e-6, None) == INVALID


def test_prefill_rope_checks_its_arguments(lib):
    p = [A + 0x100 * i for i in range(12)]  # q k_new v_new k_cache v_cache lens cos sin o lse ve g
    call = lambda ptrs, T_tab=64, eps=1e-6, T_cap=64, ve=None, g=None: (  # noqa: E731
        lib.na_attn_prefill_rope(*ptrs[:8], T_tab, eps, ve, g, ptrs[8], ptrs[9], 1, 8, 2, 2, 128,
                                 T_cap, -1, None))
    assert call(p, ve=p[10]) == INVALID and b"together" in lib.na_last_error()
    assert call(p, ve=p[10], g=A + 2) == INVALID       # misaligned gate
    assert call(p, T_tab=32) == INVALID and b"T_tab" in lib.na_last_error()
    assert call(p, eps=-1.0) == INVALID
    bad = list(p)
    bad[6] = 0                   # no cos table
    assert call(bad) == INVALID
    bad = list(p)
    bad[8] = bad[0]              # o aliases q
    assert call(bad) == INVALID


def test_decode_append_checks_its_arguments(lib):
    p = [A + 0x100 * i for i in range(14)]
    need = lib.na_attn_decode_workspace_bytes(4, 6, 128, 64)
    # q k_new v_new k_cache v_cache seqlens cos sin T_tab eps ve gate o lse ... ws
    call = lambda cos=p[6], sin=p[7], T_tab=64, ve=None, g=None, ws=need: (  # noqa: E731
        lib.na_attn_decode_append(p[0], p[1], p[2], p[3], p[4], p[5], cos, sin, T_tab, 1e-6, ve, g,
                                  p[8], p[9], 4, 6, 3, 128, 64, -1, p[13], ws, None))
    assert call(T_tab=32) == INVALID and b"T_tab" in lib.na_last_error()
    assert call(sin=None) == INVALID and b"together" in lib.na_last_error()
    assert call(ve=p[10]) == INVALID
    assert call(ws=need - 4) == INVALID and b"workspace" in lib.na_last_error()
    assert lib.na_attn_decode_append(p[0], p[1], p[2], p[3], p[4], p[5], None, None, 0, 0.0, None,
                                     None, p[8], p[9], 4, 6, 4, 128, 64, -1, p[13], need,
                                     None) == INVALID  # H not a multiple of H_kv


def test_bwd_rope_checks_its_arguments(lib):
    p = [A + 0x100 * i for i in range(17)]
    need = lib.na_attn_bwd_workspace_bytes(1, 64, 2, 128)
    # q k v o dout lse q_raw k_raw cos sin | dq dk dv delta ws | ve gate dve dgate
    call = lambda ptrs=p, T_tab=64, ws=need, Hk=2, g=(None,) * 4: lib.na_attn_bwd_rope(  # noqa
        *ptrs[:10], T_tab, 1e-6, g[0], g[1], ptrs[10], ptrs[11], ptrs[12], g[2], g[3], ptrs[13],
        ptrs[14], ws, 1, 64, 2, Hk, 128, -1, None)
    assert call(T_tab=32) == INVALID and b"T_tab" in lib.na_last_error()
    assert call(ws=need - 1) == INVALID and b"workspace" in lib.na_last_error()
    bad = list(p)
    bad[14] = 0                  # no workspace
    assert call(bad) == INVALID
    bad = list(p)
    bad[10] = bad[6]             # dq aliases q_raw
    assert call(bad) == INVALID
    assert call(Hk=3) == INVALID
    gate = (A + 0x3000, A + 0x3100, A + 0x3200, A + 0x3300)
    for j in range(4):           # the gate's four pointers: all or none
        part = list(gate)
        part[j] = None
        assert call(g=tuple(part)) == INVALID and b"all four" in lib.na_last_error()
    assert call(g=gate[:2] + (p[12], gate[3])) == INVALID  # dve aliases dv
    assert call(g=gate[:3] + (gate[2],)) == INVALID       # dgate aliases dve


def test_fwd_rope_checks_its_arguments(lib):
    p = [A + 0x100 * i for i in range(9)]  # q_raw k_raw v cos sin | q_rot k_rot o lse
    call = lambda ptrs=p, T_tab=64, eps=1e-6, H=2, Hk=2, D=128, win=-1: (  # noqa: E731
        lib.na_attn_fwd_rope(*ptrs[:5], T_tab, eps, *ptrs[5:], 1, 64, H, Hk, D, win, None))
    assert call(T_tab=32) == INVALID and b"T_tab" in lib.na_last_error()
    assert call(eps=-1.0) == INVALID and b"eps" in lib.na_last_error()
    assert call(eps=float("inf")) == INVALID
    assert call(D=64) == UNSUPPORTED
    assert call(Hk=3) == INVALID
    assert call(H=4, Hk=3) == INVALID
    bad = list(p)
    bad[5] = bad[0]              # q_rot aliases q_raw
    assert call(bad) == INVALID and b"alias" in lib.na_last_error()
    bad = list(p)
    bad[6] = bad[7]              # k_rot aliases o
    assert call(bad) == INVALID
    bad = list(p)
    bad[8] = A + 4               # lse not 16-byte aligned
    assert call(bad) == INVALID


def test_value_gate_checks_its_arguments(lib):
    p = [A + 0x100 * i for i in range(5)]
    assert lib.na_value_gate_fwd(*p[:4], 1, 8, 2, 64, None) == UNSUPPORTED
    assert lib.na_value_gate_fwd(*p[:4], 1, 8, 0, 128, None) == INVALID
    assert lib.na_value_gate_fwd(p[0], p[1], p[2], p[0], 1, 8, 2, 128, None) == INVALID  # alias
    assert lib.na_value_gate_fwd(p[0], p[1], 0, p[3], 1, 8, 2, 128, None) == INVALID
    assert lib.na_value_gate_bwd(p[0], p[1], p[2], p[3], p[3], 1, 8, 2, 128, None) == INVALID
    assert lib.na_value_gate_bwd(p[0], p[1], p[2], p[3], A + 2, 1, 8, 2, 128, None) == INVALID


def test_bwd_workspace_bytes(lib):
    # lower-triangular 32 x 32 bf16 blocks per (b, h)
    for B, T, H in ((1, 1, 1), (2, 33, 3), (32, 2048, 10)):
        nblk = (T + 31) // 32
        assert lib.na_attn_bwd_workspace_bytes(B, T, H, 128) == B * H * nblk * (nblk + 1) // 2 * 2048
    assert lib.na_attn_bwd_workspace_bytes(1, 8, 1, 64) == 0
    assert lib.na_attn_bwd_workspace_bytes(0, 8, 1, 128) == 0


def test_decode_workspace_and_checks(lib):
    need = lib.na_attn_decode_workspace_bytes(64, 10, 128, 2048)
    assert need > 0 and need % 4 == 0
    assert lib.na_attn_decode_workspace_bytes(64, 10, 64, 2048) == 0
    assert lib.na_attn_decode_workspace_bytes(0, 10, 128, 2048) == 0
    # grows with the cache capacity, never shrinks
    assert lib.na_attn_decode_workspace_bytes(64, 10, 128, 4096) >= need
    p = [A + 0x100 * i for i in range(7)]
    call = lambda ws_bytes, D=128, lse=p[5]: lib.na_attn_decode(  # noqa: E731
        p[0], p[1], p[2], p[3], p[4], lse, 64, 10, D, 2048, p[6], ws_bytes, None)
    assert call(need - 4) == INVALID and b"workspace" in lib.na_last_error()
    assert call(need, D=256) == UNSUPPORTED
    q_alias = lib.na_attn_decode(p[0], p[1], p[2], p[3], p[0], p[5], 64, 10, 128, 2048, p[6],
                                 need, None)
    assert q_alias == INVALID
    no_seqlens = lib.na_attn_decode(p[0], p[1], p[2], 0, p[4], p[5], 64, 10, 128, 2048, p[6],
                                    need, None)
    assert no_seqlens == INVALID


def test_binding_has_no_cpu_path():
    torch = pytest.importorskip("torch")
    if not os.path.exists(na.library_path()):
        pytest.skip("library not built")
    x = torch.zeros(1, 4, 1, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        na.attn_fwd(x, x, x)


def test_product_and_oracle_share_no_code():
    """Neither side imports the other; the library sources name no oracle."""
    pkg = os.path.join(ROOT, "causal_self_attention_mha_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".hpp", ".h")):
                src = open(os.path.join(dirpath, f), encoding="utf-8").read()
                assert not re.search(r"^\s*(from|import)\s+oracle\b", src, re.M), f
                assert "#include" not in src or "oracle" not in " ".join(
                    re.findall(r"#include\s*[<\"]([^>\"]+)", src)), f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            src = open(os.path.join(ROOT, "oracle", f), encoding="utf-8").read()
            assert "causal_self_attention_mha_amd" not in src
            assert not re.search(r"^\s*(from|import)\s+workloads\b", src, re.M)


def _p(i):
    return A + 0x100 * i


# entry point, argument list builder (pointers by index), indices of required pointers
_NULL_CASES = [
    ("na_attn_fwd", lambda p: (*p[:4], p[4], 1, 8, 2, 128, None), range(5)),
    ("na_attn_bwd", lambda p: (*p[:10], p[10], 1 << 20, 1, 8, 2, 128, None), range(10)),
    ("na_attn_prefill", lambda p: (*p[:8], 1, 8, 2, 2, 128, 64, -1, None), range(7)),
    ("na_qk_norm_rope_fwd", lambda p: (*p[:6], None, 1, 8, 2, 2, 128, 16, 1e-6, None), range(6)),
    ("na_qk_norm_rope_bwd", lambda p: (*p[:8], None, 1, 8, 2, 2, 128, 16, 1e-6, None), range(8)),
    ("na_value_gate_fwd", lambda p: (*p[:4], 1, 8, 2, 128, None), range(4)),
    ("na_value_gate_bwd", lambda p: (*p[:5], 1, 8, 2, 128, None), range(5)),
    ("na_attn_bwd_rope", lambda p: (*p[:10], 64, 1e-6, None, None, *p[10:13], None, None,
                                    *p[13:15], 1 << 26, 1, 64, 2, 2, 128, -1, None), range(15)),
    ("na_attn_fwd_rope", lambda p: (*p[:5], 64, 1e-6, *p[5:9], 1, 64, 2, 2, 128, -1, None),
     range(9)),
]


@pytest.mark.parametrize("name,args,required", _NULL_CASES, ids=[c[0] for c in _NULL_CASES])
def test_every_required_pointer_is_checked(lib, name, args, required):
    """Each required pointer, set to NULL alone, is rejected on the host (so
    no kernel ever sees it)."""
    fn = getattr(lib, name)
    for i in required:
        p = [_p(j) for j in range(16)]
        p[i] = 0
        assert fn(*args(p)) == INVALID, (name, i)
        assert b"NULL" in lib.na_last_error(), (name, i, lib.na_last_error())


def test_decode_noalloc_rejects_sizes_beyond_its_scratch(lib):
    """na_attn_decode_noalloc refuses, on the host, sizes whose split-KV
    partials would not fit its fixed 16 MiB scratch."""
    need = lib.na_attn_decode_workspace_bytes(512, 16, 128, 4096)
    assert need > 16 << 20
    st = lib.na_attn_decode_noalloc(A, A + 0x100, A + 0x200, A + 0x300, A + 0x400, A + 0x500,
                                    512, 16, 128, 4096, None)
    assert st == INVALID and b"scratch" in lib.na_last_error()
    assert lib.na_attn_decode_noalloc(0, A, A, A, A, A, 4, 2, 128, 64, None) == INVALID
    assert lib.na_attn_decode_noalloc(A, A + 0x100, A + 0x200, A + 0x300, A + 0x400, A + 0x500,
                                      4, 2, 64, 64, None) == UNSUPPORTED
