"""The C ABI library on the host: it loads, exports every declared symbol,
and rejects bad arguments before touching the GPU (no compute call here)."""
import ctypes as C
import os
import re

import pytest

from sparse_moe_layer_03_amd import moe
from tests.tiling_rule import tiles_per_expert

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return moe.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), f"{n} declared in include/moe.h but not exported"
    assert set(names) == set(moe.EXPORTS)


def test_status_strings(L):
    for code, name in ((0, "MOE_OK"), (-1, "MOE_ERR_NULL"), (-2, "MOE_ERR_SHAPE"), (-3, "MOE_ERR_ALIGN"),
                       (-4, "MOE_ERR_WORKSPACE"), (-5, "MOE_ERR_ARCH"), (-6, "MOE_ERR_HIP")):
        assert moe.status_str(code) == name


def test_tile_rows_policy():
    # mean rows per expert T*k/E (integer): >= 64 -> 256, >= 32 -> 64, else 32
    assert moe.moe_align_tile_rows(8192, 256, 8) == 256
    assert moe.moe_align_tile_rows(32768, 256, 8) == 256
    assert moe.moe_align_tile_rows(6144, 256, 8) == 256
    assert moe.moe_align_tile_rows(4096, 256, 8) == 256
    assert moe.moe_align_tile_rows(2048, 256, 8) == 256
    assert moe.moe_align_tile_rows(2047, 256, 8) == 64
    assert moe.moe_align_tile_rows(1024, 256, 8) == 64
    assert moe.moe_align_tile_rows(1023, 256, 8) == 32
    for T, E, k in ((8192, 256, 8), (4096, 256, 8), (2048, 256, 8), (1024, 256, 8), (16, 8, 2), (5, 3, 3)):
        assert moe.moe_align_small_tile_rows(T, E, k) == moe.moe_align_tile_rows(T, E, k)
    # padding is at most BIG - 1 rows per used expert
    assert moe.moe_align_max_rows(8192, 256, 8) == 8192 * 8 + 256 * 255
    assert moe.moe_align_max_rows(4096, 256, 8) == 4096 * 8 + 256 * 255
    assert moe.moe_align_max_rows(2048, 256, 8) == 2048 * 8 + 256 * 255
    assert moe.moe_align_max_rows(2047, 256, 8) == 2047 * 8 + 256 * 63
    assert moe.moe_align_max_rows(2, 256, 8) == 16 + 16 * 31
    assert moe.moe_align_max_big_tiles(8192, 256, 8) == (65536 + 256 * 255) // 256
    assert moe.moe_align_max_tiles(8192, 256, 8) == (65536 + 256 * 255) // 256
    # BIG == SMALL == 32: one tile class, ceil(count / 32) tiles per expert
    assert moe.moe_align_max_big_tiles(16, 8, 2) == (32 + 8 * 31) // 32
    assert moe.moe_align_max_tiles(16, 8, 2) == (32 + 8 * 31) // 32


def test_tile_capacity_is_worst_case():
    """Brute force over small histograms: the capacities bound every possible tiling."""
    import itertools
    import numpy as np
    for E, k, T in ((3, 2, 40), (4, 1, 70), (2, 2, 100)):
        B, S = moe.moe_align_tile_rows(T, E, k), moe.moe_align_small_tile_rows(T, E, k)
        n = T * k
        worst = [0, 0, 0]
        for c in itertools.product(range(T + 1), repeat=E - 1):
            last = n - sum(c)
            if not 0 <= last <= T:
                continue
            cnt = np.array(list(c) + [last])
            nb, ns = tiles_per_expert(cnt, B, S)
            worst = [max(worst[0], int((nb * B + ns * S).sum())), max(worst[1], int(nb.sum())),
                     max(worst[2], int(nb.sum() + ns.sum()))]
        assert worst[0] <= moe.moe_align_max_rows(T, E, k)
        assert worst[1] <= moe.moe_align_max_big_tiles(T, E, k)
        assert worst[2] <= moe.moe_align_max_tiles(T, E, k)


def test_workspace_sizes():
    big = moe.moe_workspace_size(8192, 2048, 256, 8, 512, 512)
    small = moe.moe_workspace_size(1024, 2048, 256, 8, 512, 512)
    dec = moe.moe_workspace_size(1, 2048, 256, 8, 512, 512)
    assert big > small > dec > 0
    assert dec < (1 << 20)
    # h of every padded row and o of every assignment must fit
    rows = moe.moe_align_max_rows(8192, 256, 8)
    assert big >= rows * 512 * 2 + 8192 * 8 * 2048 * 2
    for bad in ((16, 255, 8, 2, 128, 0), (16, 256, 0, 1, 128, 0), (16, 256, 8, 9, 128, 0), (16, 256, 8, 2, 100, 0),
                (16, 256, 8, 2, 128, 64), (16, 256, 300, 2, 128, 0), (16, 256, 8, 17, 128, 0), (-1, 256, 8, 2, 128, 0)):
        assert moe.moe_workspace_size(*bad) == 0, bad


def fwd(L, x=1 << 12, wr=1 << 12, b=None, wg=1 << 12, wu=1 << 12, wd=1 << 12, sg=None, su=None, sd=None, wsg=None,
        T=16, H=256, E=8, k=2, I=128, I_s=0, y=1 << 12, ws=1 << 12, nbytes=1 << 40):
    return L.moe_forward(x, wr, b, wg, wu, wd, sg, su, sd, wsg, T, H, E, k, I, I_s, y, ws, nbytes, None)


def test_forward_argument_errors(L):
    assert fwd(L, T=0) == moe.MOE_OK  # no-op
    assert fwd(L, x=None) == moe.MOE_ERR_NULL
    assert fwd(L, y=None) == moe.MOE_ERR_NULL
    assert fwd(L, ws=None) == moe.MOE_ERR_NULL
    assert fwd(L, k=9) == moe.MOE_ERR_SHAPE
    assert fwd(L, k=0) == moe.MOE_ERR_SHAPE
    assert fwd(L, E=257, k=2) == moe.MOE_ERR_SHAPE
    assert fwd(L, H=320) == moe.MOE_ERR_SHAPE
    assert fwd(L, I=96) == moe.MOE_ERR_SHAPE
    assert fwd(L, T=-3) == moe.MOE_ERR_SHAPE
    # shared-expert pointers: all or none
    assert fwd(L, sg=1 << 12) == moe.MOE_ERR_SHAPE
    assert fwd(L, I_s=128, sg=1 << 12, su=1 << 12, sd=1 << 12) == moe.MOE_ERR_NULL
    # alignment and workspace size
    assert fwd(L, x=(1 << 12) + 2) == moe.MOE_ERR_ALIGN
    assert fwd(L, ws=(1 << 12) + 16) == moe.MOE_ERR_ALIGN
    assert fwd(L, nbytes=100) == moe.MOE_ERR_WORKSPACE
    assert "workspace" in moe.last_error()


def test_stage_argument_errors(L):
    p = 1 << 12
    assert L.moe_route(None, p, None, None, 16, 256, 8, 2, p, p, None, p, None, 0, None) == moe.MOE_ERR_NULL
    assert L.moe_route(p, p, None, None, 16, 256, 8, 2, None, p, None, p, None, 0, None) == moe.MOE_ERR_NULL  # ids
    assert L.moe_route(p, p, None, p, 16, 256, 8, 2, p, p, None, p, None, 0, None) == moe.MOE_ERR_NULL  # s missing
    assert L.moe_route(p, p, None, None, 16, 256, 8, 20, p, p, None, p, None, 0, None) == moe.MOE_ERR_SHAPE
    # streamed form: scratch (W_router in operand order: 32-expert groups x H x 64 bytes) too
    # small, then misaligned
    need = L.moe_route_scratch_size(16, 256, 8)
    assert need == 1 * 256 * 64 and L.moe_route_scratch_size(1, 2048, 256) == 8 * 2048 * 64
    assert L.moe_route(p, p, None, None, 16, 256, 8, 2, p, p, None, p, p, need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert "scratch" in moe.last_error()
    assert L.moe_route(p, p, None, None, 16, 256, 8, 2, p, p, None, p, p + 4, need, None) == moe.MOE_ERR_ALIGN
    assert L.moe_route_scratch_size(16, 100, 8) == 0
    assert L.moe_route_from_logits(p, 16, 300, 2, p, p, None) == moe.MOE_ERR_SHAPE
    assert L.moe_route_from_logits(None, 16, 8, 2, p, p, None) == moe.MOE_ERR_NULL
    assert L.moe_align(p, 16, 8, 2, p, p, p, p, p, p, p, 1, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_align(p, 16, 8, 2, p, p, None, p, p, p, p, 1 << 20, None) == moe.MOE_ERR_NULL
    assert L.moe_grouped_gate_up(p, p, p, None, None, p, p, p, 16, 256, 8, 2, 128, 128, p, None, None) == \
        moe.MOE_ERR_NULL
    assert L.moe_grouped_down(p, p, p, p, p, 16, 256, 8, 2, 100, p, None) == moe.MOE_ERR_SHAPE
    assert L.moe_combine(p, p, p, None, None, 16, 256, 2, 0, p, None) == moe.MOE_ERR_SHAPE
    assert L.moe_combine(p, p, None, None, None, 16, 256, 2, 0, None, None) == moe.MOE_ERR_NULL
    for f, args in ((L.moe_route, (p, p, None, None, 0, 256, 8, 2, None, None, None, None, None, 0, None)),
                    (L.moe_align, (None, 0, 8, 2, None, None, None, None, None, None, None, 0, None))):
        assert f(*args) == moe.MOE_OK  # T = 0 is a no-op


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host without a GPU only")
def test_valid_call_without_gpu_reports_arch(L):
    assert fwd(L) == moe.MOE_ERR_ARCH


def fwd8(L, **kw):
    """moe_forward_fp8 with fake (never dereferenced) aligned pointers; overrides by name."""
    p = 1 << 12
    a = dict(x=p, wr=p, b=None, qg=p, sg=p, qu=p, su=p, qd=p, sd=p, qsg=None, ssg=None, qsu=None, ssu=None,
             qsd=None, ssd=None, wsg=None, T=4, H=256, E=8, k=2, I=128, I_s=0, y=p, ws=p, nbytes=1 << 30)
    a.update(kw)
    return L.moe_forward_fp8(a["x"], a["wr"], a["b"], a["qg"], a["sg"], a["qu"], a["su"], a["qd"], a["sd"],
                             a["qsg"], a["ssg"], a["qsu"], a["ssu"], a["qsd"], a["ssd"], a["wsg"],
                             a["T"], a["H"], a["E"], a["k"], a["I"], a["I_s"], a["y"], a["ws"], a["nbytes"], None)


def test_forward_fp8_argument_errors(L):
    p = 1 << 12
    assert fwd8(L, T=0) == moe.MOE_OK
    assert fwd8(L, qg=None) == moe.MOE_ERR_NULL
    assert fwd8(L, sd=None) == moe.MOE_ERR_NULL  # a scale is missing
    assert fwd8(L, k=0) == moe.MOE_ERR_SHAPE
    assert fwd8(L, qsg=p) == moe.MOE_ERR_SHAPE  # shared tensors with I_s = 0
    assert fwd8(L, I_s=128, qsg=p, ssg=p, qsu=p, ssu=p, qsd=p, ssd=p) == moe.MOE_ERR_NULL  # w_sg missing
    assert fwd8(L, sg=p + 4) == moe.MOE_ERR_ALIGN
    assert fwd8(L, nbytes=100) == moe.MOE_ERR_WORKSPACE
    assert L.moe_e4m3_to_f32(p, p, -1, None) == moe.MOE_ERR_SHAPE
    assert L.moe_e4m3_to_f32(None, p, 8, None) == moe.MOE_ERR_NULL
    assert L.moe_e4m3_to_f32(None, None, 0, None) == moe.MOE_OK


@pytest.mark.skipif(os.path.exists("/dev/kfd"), reason="host without a GPU only")
def test_valid_fp8_call_without_gpu_reports_arch(L):
    assert fwd8(L) == moe.MOE_ERR_ARCH
    assert fwd8(L, T=1) == moe.MOE_ERR_ARCH
    assert fwd8(L, T=100) == moe.MOE_ERR_ARCH


def test_forward_q4_argument_errors(L):
    p = 1 << 12
    a = dict(x=p, wr=p, b=None, qg=p, sg=p, qu=p, su=p, qd=p, sd=p, qsg=None, ssg=None, qsu=None, ssu=None,
             qsd=None, ssd=None, wsg=None, T=4, H=256, E=8, k=2, I=128, I_s=0, y=p, ws=p, nbytes=1 << 30)

    def q4(**kw):
        b = dict(a)
        b.update(kw)
        return L.moe_forward_q4(b["x"], b["wr"], b["b"], b["qg"], b["sg"], b["qu"], b["su"], b["qd"], b["sd"],
                                b["qsg"], b["ssg"], b["qsu"], b["ssu"], b["qsd"], b["ssd"], b["wsg"],
                                b["T"], b["H"], b["E"], b["k"], b["I"], b["I_s"], b["y"], b["ws"], b["nbytes"], None)
    assert q4(T=0) == moe.MOE_OK
    assert q4(qd=None) == moe.MOE_ERR_NULL
    assert q4(T=moe.Q4_MAX_T + 1) == moe.MOE_ERR_SHAPE
    assert "4-bit" in moe.last_error()
    assert q4(qsg=p) == moe.MOE_ERR_SHAPE
    assert q4(I_s=128, qsg=p, ssg=p, qsu=p, ssu=p, qsd=p, ssd=p) == moe.MOE_ERR_NULL
    assert q4(su=p + 2) == moe.MOE_ERR_ALIGN
    assert q4(nbytes=100) == moe.MOE_ERR_WORKSPACE
    if not os.path.exists("/dev/kfd"):
        assert q4() == moe.MOE_ERR_ARCH


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built library every call raises."""
    monkeypatch.setattr(moe, "LIB_PATH", str(tmp_path / "libmoe355.so"))
    monkeypatch.setattr(moe, "_lib", None)
    with pytest.raises(ImportError):
        moe.lib()
    with pytest.raises(ImportError):
        moe.moe_workspace_size(16, 256, 8, 2, 128, 0)
