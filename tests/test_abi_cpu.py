"""The C ABI library on the CPU: it loads, exports every symbol include/fa.h
declares, and rejects bad arguments before touching any device.  No kernel is
launched here (there is no GPU in this environment)."""

import os
import re
import subprocess

import pytest

import tiled_attention_fa_amd as fa
from tiled_attention_fa_amd._lib import EXPORTS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return fa.load_library()


def test_exports_match_header(lib):
    names = declared_functions()
    assert names == sorted(EXPORTS)
    out = subprocess.run(["nm", "-D", "--defined-only", fa.library_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    for n in names:
        assert n in exported, f"{n} declared in fa.h but not exported"
        assert hasattr(lib, n)


def test_library_targets_gfx950_only():
    out = subprocess.run(["/opt/rocm/lib/llvm/bin/clang-offload-bundler", "--list", "--type=o",
                          f"--input={fa.library_path()}"], capture_output=True, text=True)
    if out.returncode == 0 and out.stdout.strip():
        targets = [t for t in out.stdout.split() if "amdgcn" in t]
        assert targets and all("gfx950" in t for t in targets), out.stdout


def test_version_and_status_strings(lib):
    assert "gfx950" in fa.fa_version()
    texts = {c: fa.fa_status_string(c) for c in fa.STATUS_NAMES}
    assert texts[0] == "ok"
    assert len(set(texts.values())) == len(texts)
    assert fa.fa_status_string(12345) == "unknown status"


# Fake, well-aligned, non-overlapping addresses: validation never dereferences.
A, B_, C, O = 0x100000, 0x200000, 0x300000, 0x400000


@pytest.mark.parametrize("args,status", [
    (dict(dtype=7), "FA_ERR_DTYPE"),
    (dict(B=0), "FA_ERR_DIM"),
    (dict(H=-1), "FA_ERR_DIM"),
    (dict(N=-5), "FA_ERR_DIM"),
    (dict(D=0), "FA_ERR_DIM"),
    (dict(D=80), "FA_ERR_UNSUPPORTED_D"),
    (dict(D=256), "FA_ERR_UNSUPPORTED_D"),
    (dict(scale=float("nan")), "FA_ERR_SCALE"),
    (dict(scale=float("inf")), "FA_ERR_SCALE"),
    (dict(N=0, q=0, k=0, v=0, o=0), "FA_OK"),
    (dict(q=0), "FA_ERR_NULL"),
    (dict(o=0), "FA_ERR_NULL"),
    (dict(k=A + 8), "FA_ERR_ALIGN"),
    (dict(o=A), "FA_ERR_ALIAS"),
    (dict(o=B_ + 64 * 64 * 2 - 16), "FA_ERR_ALIAS"),
    (dict(N=1 << 25, D=64), "FA_ERR_TOO_LARGE"),
    (dict(B=1 << 20, H=1 << 20), "FA_ERR_TOO_LARGE"),
    (dict(), "FA_ERR_DEVICE"),
])
def test_validation(lib, args, status):
    kw = dict(q=A, k=B_, v=C, o=O, B=1, H=1, N=64, D=64, scale=0.125, causal=False, dtype=1)
    kw.update(args)
    got = fa.fa_forward_raw(kw["q"], kw["k"], kw["v"], kw["o"], kw["B"], kw["H"], kw["N"], kw["D"],
                            kw["scale"], kw["causal"], kw["dtype"])
    if status == "FA_ERR_DEVICE" and got == 0:
        pytest.skip("a gfx950 device is present; the no-device path is not reachable")
    assert fa.STATUS_NAMES[got] == status


def test_device_info_without_device(lib):
    import ctypes
    cus, clk = ctypes.c_int(-7), ctypes.c_int(-7)
    got = lib.fa_device_info(ctypes.byref(cus), ctypes.byref(clk))
    if got == 0:
        pytest.skip("a device is present; the no-device path is not reachable")
    assert fa.STATUS_NAMES[got] == "FA_ERR_DEVICE"
    assert (cus.value, clk.value) == (-7, -7)  # outputs untouched on error


# ------------------------------------------------- three-pass entry points

def _ws(B, H, N, dt):
    NP = (N + 63) // 64 * 64
    up = lambda x: (x + 255) // 256 * 256
    s = B * H * N * NP * 4
    p = B * H * N * NP * 2
    p_off = up(s)
    plo_off = up(p_off + p)
    return up(plo_off + p) if dt == fa.FA_BF16 else plo_off


@pytest.mark.parametrize("B,H,N", [(1, 1, 0), (1, 1, 1), (1, 32, 2048), (4, 32, 2048), (2, 8, 1000),
                                   (1, 16, 8192), (3, 5, 77)])
@pytest.mark.parametrize("dt", [1, 2])
def test_naive_workspace_bytes(lib, B, H, N, dt):
    assert fa.fa_naive_workspace_bytes(B, H, N, dt) == _ws(B, H, N, dt)


@pytest.mark.parametrize("args,status", [
    (dict(dtype=0), "FA_ERR_DTYPE"),
    (dict(dtype=9), "FA_ERR_DTYPE"),
    (dict(B=0), "FA_ERR_DIM"),
    (dict(N=-1), "FA_ERR_DIM"),
    (dict(B=1 << 40, H=1 << 40), "FA_ERR_TOO_LARGE"),
    (dict(B=1 << 20, N=1 << 20), "FA_ERR_TOO_LARGE"),
])
def test_naive_workspace_bytes_rejects(lib, args, status):
    kw = dict(B=1, H=1, N=64, dtype=1)
    kw.update(args)
    got = fa.fa_naive_workspace_bytes(kw["B"], kw["H"], kw["N"], kw["dtype"])
    assert fa.STATUS_NAMES[got] == status


W = 0x10000000  # fake 256-byte aligned workspace, clear of the tensors


@pytest.mark.parametrize("args,status", [
    (dict(dtype=0), "FA_ERR_DTYPE"),
    (dict(dtype=5), "FA_ERR_DTYPE"),
    (dict(B=0), "FA_ERR_DIM"),
    (dict(D=80), "FA_ERR_UNSUPPORTED_D"),
    (dict(scale=float("nan")), "FA_ERR_SCALE"),
    (dict(N=0, q=0, k=0, v=0, o=0, ws=0, ws_bytes=0), "FA_OK"),
    (dict(v=0), "FA_ERR_NULL"),
    (dict(o=O + 4), "FA_ERR_ALIGN"),
    (dict(o=C), "FA_ERR_ALIAS"),
    (dict(N=1 << 25, D=64), "FA_ERR_TOO_LARGE"),
    (dict(N=(1 << 20) + 1, D=64, q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40, ws=5 << 40,
          ws_bytes=1 << 62), "FA_ERR_TOO_LARGE"),
    (dict(ws=0), "FA_ERR_WORKSPACE"),
    (dict(ws=W + 128), "FA_ERR_WORKSPACE"),
    (dict(ws_bytes=-1), "FA_ERR_WORKSPACE"),
    (dict(ws_bytes="short"), "FA_ERR_WORKSPACE"),
    (dict(ws=O - 256), "FA_ERR_WORKSPACE"),
    (dict(ws=A + 4096), "FA_ERR_WORKSPACE"),
    (dict(ws=A - 8192), "FA_ERR_WORKSPACE"),
    (dict(), "FA_ERR_DEVICE"),
    (dict(dtype=2), "FA_ERR_DEVICE"),
])
def test_naive_validation(lib, args, status):
    kw = dict(q=A, k=B_, v=C, o=O, B=1, H=1, N=64, D=64, scale=0.125, causal=False, dtype=1, ws=W)
    kw.update(args)
    need = fa.fa_naive_workspace_bytes(kw["B"], kw["H"], max(kw["N"], 0), kw["dtype"]) \
        if kw["dtype"] in (1, 2) and kw["B"] >= 1 and kw["N"] >= 0 else 1 << 20
    if "ws_bytes" not in kw:
        kw["ws_bytes"] = need
    elif kw["ws_bytes"] == "short":
        kw["ws_bytes"] = need - 1
    got = fa.fa_naive_forward_raw(kw["q"], kw["k"], kw["v"], kw["o"], kw["B"], kw["H"], kw["N"],
                                  kw["D"], kw["scale"], kw["causal"], kw["dtype"], kw["ws"],
                                  kw["ws_bytes"])
    if status == "FA_ERR_DEVICE" and got == 0:
        pytest.skip("a gfx950 device is present; the no-device path is not reachable")
    assert fa.STATUS_NAMES[got] == status


# ----------------------------------------- fa_forward_ex (LSE, split-KV)

def _ex_ws(B, H, N, D, S):
    if S <= 1 or N == 0:
        return 0
    up = lambda x: (x + 255) // 256 * 256
    lse_off = up(S * B * H * N * D * 4)
    return up(lse_off + S * B * H * N * 4)


@pytest.mark.parametrize("B,H,N,D,S", [(1, 1, 64, 64, 1), (1, 1, 64, 64, 2), (2, 8, 1000, 96, 2),
                                       (1, 32, 2048, 64, 3), (1, 1, 0, 128, 4), (3, 5, 77, 128, 64)])
def test_ex_workspace_bytes(lib, B, H, N, D, S):
    for dt in (0, 1, 2):
        assert fa.fa_forward_ex_workspace_bytes(B, H, N, D, dt, False, S) == _ex_ws(B, H, N, D, S)


@pytest.mark.parametrize("args,status", [
    (dict(S=-1), "FA_ERR_SPLITS"),
    (dict(S=65), "FA_ERR_SPLITS"),
    (dict(dtype=7), "FA_ERR_DTYPE"),
    (dict(B=0), "FA_ERR_DIM"),
    (dict(D=80), "FA_ERR_UNSUPPORTED_D"),
])
def test_ex_workspace_bytes_rejects(lib, args, status):
    kw = dict(B=1, H=1, N=64, D=64, dtype=1, S=2)
    kw.update(args)
    got = fa.fa_forward_ex_workspace_bytes(kw["B"], kw["H"], kw["N"], kw["D"], kw["dtype"], False, kw["S"])
    assert fa.STATUS_NAMES[got] == status


L_ = 0x500000  # fake lse address, clear of the tensors and the workspace


@pytest.mark.parametrize("args,status", [
    (dict(dtype=9), "FA_ERR_DTYPE"),
    (dict(H=0), "FA_ERR_DIM"),
    (dict(D=32), "FA_ERR_UNSUPPORTED_D"),
    (dict(scale=float("-inf")), "FA_ERR_SCALE"),
    (dict(N=0, q=0, k=0, v=0, o=0, ws=0, S=7), "FA_OK"),
    (dict(k=0), "FA_ERR_NULL"),
    (dict(v=C + 2), "FA_ERR_ALIGN"),
    (dict(o=B_), "FA_ERR_ALIAS"),
    (dict(S=-2), "FA_ERR_SPLITS"),
    (dict(S=65), "FA_ERR_SPLITS"),
    (dict(lse=L_ + 2), "FA_ERR_ALIGN"),
    (dict(lse=O + 64), "FA_ERR_ALIAS"),
    (dict(lse=A), "FA_ERR_ALIAS"),
    (dict(ws=0), "FA_ERR_WORKSPACE"),
    (dict(ws=W + 64), "FA_ERR_WORKSPACE"),
    (dict(ws_bytes="short"), "FA_ERR_WORKSPACE"),
    (dict(ws=C - 256), "FA_ERR_WORKSPACE"),
    (dict(ws=L_ - 256), "FA_ERR_WORKSPACE"),
    (dict(B=1 << 12, H=1 << 12, N=64, D=64, S=64, q=1 << 40, k=2 << 40, v=3 << 40, o=4 << 40,
          lse=0, ws=5 << 40, ws_bytes=1 << 60), "FA_ERR_TOO_LARGE"),
    (dict(S=1, ws=0, ws_bytes=0), "FA_ERR_DEVICE"),
    (dict(), "FA_ERR_DEVICE"),
    (dict(dtype=0), "FA_ERR_DEVICE"),
    (dict(S=0), "FA_ERR_DEVICE"),
])
def test_ex_validation(lib, args, status):
    kw = dict(q=A, k=B_, v=C, o=O, lse=L_, B=1, H=1, N=64, D=64, scale=0.125, causal=False, dtype=1,
              S=2, ws=W)
    kw.update(args)
    if "ws_bytes" not in kw or kw["ws_bytes"] == "short":
        need = _ex_ws(kw["B"], kw["H"], kw["N"], kw["D"], max(kw["S"], 1)) if kw["S"] >= 0 else 1 << 20
        kw["ws_bytes"] = need - 1 if kw.get("ws_bytes") == "short" else need
    got = fa.fa_forward_ex_raw(kw["q"], kw["k"], kw["v"], kw["o"], kw["lse"], kw["B"], kw["H"], kw["N"],
                               kw["D"], kw["scale"], kw["causal"], kw["dtype"], kw["S"], kw["ws"],
                               kw["ws_bytes"])
    if status == "FA_ERR_DEVICE" and got == 0:
        pytest.skip("a gfx950 device is present; the no-device path is not reachable")
    assert fa.STATUS_NAMES[got] == status


def test_splitkv_suggest_without_device(lib):
    got = fa.fa_splitkv_suggest(1, 32, 2048, 64, 1, False)
    if got >= 1:
        pytest.skip("a device is present")
    assert fa.STATUS_NAMES[got] == "FA_ERR_DEVICE"
    assert fa.STATUS_NAMES[fa.fa_splitkv_suggest(1, 32, 2048, 80, 1, False)] == "FA_ERR_UNSUPPORTED_D"


def test_key_groups_suggest_without_device(lib):
    got = fa.fa_key_groups_suggest(1, 8, 1000, 96, 1, False)
    if got >= 1:
        pytest.skip("a device is present")
    assert fa.STATUS_NAMES[got] == "FA_ERR_DEVICE"
    assert fa.STATUS_NAMES[fa.fa_key_groups_suggest(1, 8, 1000, 80, 1, False)] == "FA_ERR_UNSUPPORTED_D"
    assert fa.STATUS_NAMES[fa.fa_key_groups_suggest(1, 8, 1000, 64, 7, False)] == "FA_ERR_DTYPE"
    assert fa.STATUS_NAMES[fa.fa_key_groups_suggest(0, 8, 1000, 64, 1, False)] == "FA_ERR_DIM"


def test_workgroup_shape_without_device(lib):
    got = fa.fa_workgroup_shape(1, 8, 1000, 96, 1, False)
    if isinstance(got, tuple):
        pytest.skip("a device is present")
    assert fa.STATUS_NAMES[got] == "FA_ERR_DEVICE"
    assert fa.STATUS_NAMES[fa.fa_workgroup_shape(1, 8, 1000, 80, 1, False)] == "FA_ERR_UNSUPPORTED_D"
    assert fa.STATUS_NAMES[fa.fa_workgroup_shape(1, 8, 1000, 64, 7, False)] == "FA_ERR_DTYPE"
    assert fa.STATUS_NAMES[fa.fa_workgroup_shape(1, 8, 1000, 64, fa.FA_F32, False)] == "FA_ERR_DEVICE"
    assert fa.STATUS_NAMES[fa.fa_workgroup_shape(1, 0, 1000, 64, 2, True)] == "FA_ERR_DIM"


# ------------------------------------------------------ fa_forward_strided

DENSE = (4 * 64 * 64, 64 * 64, 64)          # [B, H=4, N=64, D=64]
BNHD = (64 * 4 * 64, 64, 4 * 64)            # [B, N, H=4, D]
KV2 = (2 * 64 * 64, 64 * 64, 64)            # [B, H_kv=2, N, D]
BIG = 1 << 24                               # spacing of the fake bases


@pytest.mark.parametrize("args,status", [
    (dict(dtype=3), "FA_ERR_DTYPE"),
    (dict(Hkv=3), "FA_ERR_DIM"),
    (dict(Hkv=0), "FA_ERR_DIM"),
    (dict(D=48), "FA_ERR_UNSUPPORTED_D"),
    (dict(scale=float("nan")), "FA_ERR_SCALE"),
    (dict(N=0, q=0, qs=None), "FA_OK"),
    (dict(qs=None), "FA_ERR_NULL"),
    (dict(v=0), "FA_ERR_NULL"),
    (dict(ks=(KV2[0], -64, 64)), "FA_ERR_STRIDE"),
    (dict(q=BIG + 8), "FA_ERR_ALIGN"),
    (dict(vs=(KV2[0], KV2[1], 68)), "FA_ERR_ALIGN"),
    (dict(qs=(DENSE[0], DENSE[1], 56)), "FA_ERR_STRIDE"),
    (dict(os=(DENSE[0], 64, 64)), "FA_ERR_STRIDE"),
    (dict(os=(0, DENSE[1], 64), B=2), "FA_ERR_STRIDE"),
    (dict(os=BNHD), "FA_ERR_DEVICE"),
    (dict(os=(DENSE[0], 64 * 64 * 2, 128)), "FA_ERR_DEVICE"),
    (dict(ks=(0, 0, 64)), "FA_ERR_DEVICE"),
    (dict(ks=(KV2[0], KV2[1], 1 << 26)), "FA_ERR_TOO_LARGE"),
    (dict(N=1 << 25, H=1, Hkv=1, qs=(64 << 25, 64 << 25, 64), ks=(64 << 25, 64 << 25, 64),
          vs=(64 << 25, 64 << 25, 64), os=(64 << 25, 64 << 25, 64), q=1 << 40, k=2 << 40, v=3 << 40,
          o=4 << 40), "FA_ERR_TOO_LARGE"),
    (dict(o=1 * BIG + 4096), "FA_ERR_ALIAS"),
    (dict(o=3 * BIG - 1024, os=BNHD), "FA_ERR_ALIAS"),
    (dict(), "FA_ERR_DEVICE"),
    (dict(dtype=0), "FA_ERR_DEVICE"),
])
def test_strided_validation(lib, args, status):
    kw = dict(q=1 * BIG, k=2 * BIG, v=3 * BIG, o=4 * BIG, qs=DENSE, ks=KV2, vs=KV2, os=DENSE,
              B=1, H=4, Hkv=2, N=64, D=64, scale=0.125, causal=False, dtype=1)
    kw.update(args)
    got = fa.fa_forward_strided_raw(kw["q"], kw["qs"], kw["k"], kw["ks"], kw["v"], kw["vs"], kw["o"],
                                    kw["os"], kw["B"], kw["H"], kw["Hkv"], kw["N"], kw["D"],
                                    kw["scale"], kw["causal"], kw["dtype"])
    if status == "FA_ERR_DEVICE" and got == 0:
        pytest.skip("a gfx950 device is present; the no-device path is not reachable")
    assert fa.STATUS_NAMES[got] == status


# ------------------------------------------- tile-calibration library

TUNE_HEADER = os.path.join(ROOT, "include", "fa_tune.h")


def test_tune_library_exports_its_header():
    from tiled_attention_fa_amd import tile_sweep
    lib = tile_sweep.load_tune()
    text = re.sub(r"/\*.*?\*/", "", open(TUNE_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))
    assert names == ["fa_tune_f32_shapes", "fa_tune_forward", "fa_tune_forward_f32", "fa_tune_shapes",
                     "fa_tune_split_merge"]
    out = subprocess.run(["nm", "-D", "--defined-only", tile_sweep.TUNE_LIB], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT (fa_\w+)", out))
    for n in names + list(EXPORTS):
        assert n in exported, n
    assert tile_sweep.shapes(lib, 64) == [
        (2, 1, 1, 64), (4, 1, 1, 64), (4, 2, 1, 64), (8, 1, 1, 64), (4, 1, 2, 64), (4, 2, 2, 64), (8, 1, 2, 64),
        (2, 1, 1, 32), (4, 1, 1, 32), (4, 2, 1, 32), (8, 1, 1, 32), (2, 1, 1, 128), (4, 1, 1, 128),
        (8, 1, 1, 128), (8, 1, 4, 32)]
    wide = [(2, 1, 1, 64), (4, 1, 1, 64), (8, 1, 1, 64), (4, 1, 2, 64), (8, 1, 2, 64), (2, 1, 1, 32),
            (4, 1, 1, 32), (8, 1, 1, 32), (8, 1, 4, 32)]
    assert tile_sweep.shapes(lib, 96) == wide
    assert tile_sweep.shapes(lib, 128) == wide
    assert lib.fa_tune_shapes(80, None, None, None, None, 0) == -3
    f32 = [(4, 1), (4, 2), (2, 2), (2, 4), (1, 4)]
    assert tile_sweep.f32_shapes(lib, 64) == f32
    assert tile_sweep.f32_shapes(lib, 96) == f32
    assert tile_sweep.f32_shapes(lib, 128) == f32
    assert lib.fa_tune_f32_shapes(80, None, None, 0) == -3


@pytest.mark.parametrize("args,status", [
    (dict(dtype=5), "FA_ERR_DTYPE"),
    (dict(rows=-1), "FA_ERR_DIM"),
    (dict(D=80), "FA_ERR_DIM"),
    (dict(S=0), "FA_ERR_SPLITS"),
    (dict(S=65), "FA_ERR_SPLITS"),
    (dict(rows=0, po=0, pl=0, o=0), "FA_OK"),
    (dict(po=0), "FA_ERR_NULL"),
    (dict(o=O + 8), "FA_ERR_ALIGN"),
    (dict(), "FA_ERR_DEVICE"),
])
def test_tune_split_merge_validation(args, status):
    from tiled_attention_fa_amd import tile_sweep
    lib = tile_sweep.load_tune()
    kw = dict(po=A, pl=B_, o=O, lse=0, rows=4, D=64, S=2, dtype=1)
    kw.update(args)
    got = lib.fa_tune_split_merge(kw["po"] or None, kw["pl"] or None, kw["o"] or None, kw["lse"] or None,
                                  kw["rows"], kw["D"], kw["S"], kw["dtype"], None)
    if status == "FA_ERR_DEVICE" and got == 0:
        pytest.skip("a gfx950 device is present; the no-device path is not reachable")
    assert fa.STATUS_NAMES[got] == status


@pytest.mark.parametrize("args,status", [
    (dict(B=0), "FA_ERR_DIM"),
    (dict(D=80), "FA_ERR_UNSUPPORTED_D"),
    (dict(rw=1, kg=1), "FA_ERR_UNSUPPORTED_D"),
    (dict(D=128, rw=4, kg=4), "FA_ERR_UNSUPPORTED_D"),
    (dict(D=96, rw=8, kg=2), "FA_ERR_UNSUPPORTED_D"),
    (dict(q=0), "FA_ERR_NULL"),
    (dict(o=A), "FA_ERR_ALIAS"),
    (dict(N=0, q=0, k=0, v=0, o=0), "FA_OK"),
    (dict(), "FA_ERR_DEVICE"),
    (dict(D=128, rw=4, kg=1), "FA_ERR_DEVICE"),
    (dict(rw=1, kg=4), "FA_ERR_DEVICE"),
    (dict(D=96, rw=2, kg=2), "FA_ERR_DEVICE"),
])
def test_tune_forward_f32_validation(args, status):
    from tiled_attention_fa_amd import tile_sweep
    lib = tile_sweep.load_tune()
    kw = dict(q=A, k=B_, v=C, o=O, B=1, H=1, N=64, D=64, rw=4, kg=2)
    kw.update(args)
    got = lib.fa_tune_forward_f32(kw["q"] or None, kw["k"] or None, kw["v"] or None, kw["o"] or None, kw["B"],
                                  kw["H"], kw["N"], kw["D"], 0.125, 0, kw["rw"], kw["kg"], None)
    if status == "FA_ERR_DEVICE" and got == 0:
        pytest.skip("a gfx950 device is present; the no-device path is not reachable")
    assert fa.STATUS_NAMES[got] == status


@pytest.mark.parametrize("args,status", [
    (dict(dtype=0), "FA_ERR_DTYPE"),
    (dict(B=0), "FA_ERR_DIM"),
    (dict(waves=3), "FA_ERR_UNSUPPORTED_D"),
    (dict(D=128, waves=4, occ=2), "FA_ERR_UNSUPPORTED_D"),
    (dict(D=128, waves=4, occ=2, ks=2), "FA_ERR_UNSUPPORTED_D"),
    (dict(waves=2, occ=1, ks=2), "FA_ERR_UNSUPPORTED_D"),
    (dict(ks=3), "FA_ERR_UNSUPPORTED_D"),
    (dict(bn=96), "FA_ERR_UNSUPPORTED_D"),
    (dict(bn=128, occ=2), "FA_ERR_UNSUPPORTED_D"),
    (dict(D=128, waves=8, occ=1, bn=128), "FA_ERR_UNSUPPORTED_D"),
    (dict(waves=4, occ=1, ks=2, bn=32), "FA_ERR_UNSUPPORTED_D"),
    (dict(waves=8, occ=1, ks=4, bn=64), "FA_ERR_UNSUPPORTED_D"),
    (dict(waves=4, occ=1, ks=4, bn=32), "FA_ERR_UNSUPPORTED_D"),
    (dict(o=A), "FA_ERR_ALIAS"),
    (dict(), "FA_ERR_DEVICE"),
    (dict(waves=8, occ=1, bn=128), "FA_ERR_DEVICE"),
])
def test_tune_forward_validation(args, status):
    from tiled_attention_fa_amd import tile_sweep
    lib = tile_sweep.load_tune()
    kw = dict(q=A, k=B_, v=C, o=O, B=1, H=1, N=64, D=64, dtype=1, waves=4, occ=2, ks=1, bn=64)
    kw.update(args)
    got = lib.fa_tune_forward(kw["q"], kw["k"], kw["v"], kw["o"], kw["B"], kw["H"], kw["N"], kw["D"],
                              0.125, 0, kw["dtype"], kw["waves"], kw["occ"], kw["ks"], kw["bn"], None)
    if status == "FA_ERR_DEVICE" and got == 0:
        pytest.skip("a gfx950 device is present; the no-device path is not reachable")
    assert fa.STATUS_NAMES[got] == status
