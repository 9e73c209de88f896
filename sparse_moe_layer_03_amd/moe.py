"""Thin Python binding of libmoe355 (include/moe.h).

Argument marshalling only: every function takes PyTorch tensors that live on
the GPU, passes their data pointers and the current HIP stream to the C ABI
function of the same name, and raises ``MoEError`` on a non-zero status.
All arithmetic happens in the HIP kernels.  There is no fallback: if the
library has not been built, importing and calling fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
# MOE355_LIB names another build of this library to load (the sanitizer build of the CPU tests)
LIB_PATH = os.environ.get("MOE355_LIB") or os.path.join(_PKG, "libmoe355.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_SHAPE = -2
MOE_ERR_ALIGN = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_ARCH = -5
MOE_ERR_HIP = -6
SMALL_BATCH_MAX_T = 32  # MOE_SMALL_BATCH_MAX_T: moe_forward's small-batch path covers 2 <= T <= this
Q4_MAX_T = 32  # MOE_Q4_MAX_T: moe_forward_q4 covers 1 <= T <= this

EXPORTS = (
    "moe_status_str", "moe_last_error", "moe_align_tile_rows", "moe_align_small_tile_rows", "moe_align_max_rows",
    "moe_align_max_big_tiles", "moe_align_max_tiles", "moe_workspace_size", "moe_forward_ids_offset", "moe_forward", "moe_route", "moe_route_scratch_size", "moe_route_from_logits", "moe_align_scratch_size",
    "moe_align", "moe_grouped_gate_up", "moe_grouped_down", "moe_combine", "moe_forward_fp8", "moe_e4m3_to_f32", "moe_forward_q4",
    "moe_bucket_plan", "moe_prefill_runner_create", "moe_prefill_runner_create_fp8", "moe_prefill_runner_run", "moe_prefill_runner_destroy",
    "moe_forward_noalloc", "moe_workspace_sections",
)
NOALLOC_WS_BYTES = 64 << 20  # MOE_NOALLOC_WS_BYTES: the fixed workspace of moe_forward_noalloc


class MoEError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_str(status)}: {message}")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sparse_moe_layer_03_amd.build`")
        L = C.CDLL(LIB_PATH)
        p, i, z, i64 = C.c_void_p, C.c_int, C.c_size_t, C.c_int64
        sig = {
            "moe_status_str": ([i], C.c_char_p),
            "moe_last_error": ([], C.c_char_p),
            "moe_align_tile_rows": ([i, i, i], i),
            "moe_align_small_tile_rows": ([i, i, i], i),
            "moe_align_max_rows": ([i, i, i], i64),
            "moe_align_max_big_tiles": ([i, i, i], i64),
            "moe_align_max_tiles": ([i, i, i], i64),
            "moe_workspace_size": ([i, i, i, i, i, i], z),
            "moe_forward_ids_offset": ([i, i, i, i, i, i], z),
            "moe_workspace_sections": ([i, i, i, i, i, i, p, p, i], i),
            "moe_forward": ([p] * 10 + [i] * 6 + [p, p, z, p], i),
            "moe_forward_noalloc": ([p] * 10 + [i] * 6 + [p, p], i),
            "moe_route": ([p, p, p, p, i, i, i, i, p, p, p, p, p, z, p], i),
            "moe_route_scratch_size": ([i, i, i], z),
            "moe_route_from_logits": ([p, i, i, i, p, p, p], i),
            "moe_align_scratch_size": ([i, i, i], z),
            "moe_align": ([p, i, i, i, p, p, p, p, p, p, p, z, p], i),
            "moe_grouped_gate_up": ([p] * 8 + [i] * 6 + [p, p, p], i),
            "moe_grouped_down": ([p] * 5 + [i] * 5 + [p, p], i),
            "moe_combine": ([p] * 5 + [i] * 4 + [p, p], i),
            "moe_forward_fp8": ([p] * 16 + [i] * 6 + [p, p, z, p], i),
            "moe_e4m3_to_f32": ([p, p, i64, p], i),
            "moe_forward_q4": ([p] * 16 + [i] * 6 + [p, p, z, p], i),
            "moe_bucket_plan": ([i, p, i, p, p, i, p], i),
            "moe_prefill_runner_create": ([p] * 9 + [i] * 5 + [p, i, p], i),
            "moe_prefill_runner_create_fp8": ([p] * 15 + [i] * 5 + [p, i, p], i),
            "moe_prefill_runner_run": ([p, p, i, p, p], i),
            "moe_prefill_runner_destroy": ([p], i),
        }
        for name, (args, res) in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def last_error() -> str:
    return lib().moe_last_error().decode()


def _check(rc: int):
    if rc != MOE_OK:
        raise MoEError(rc, last_error())


def _p(t) -> Optional[int]:
    """Device pointer of a tensor (None stays NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream=None) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------------------- sizes
def moe_align_tile_rows(T: int, E: int, k: int) -> int:
    return lib().moe_align_tile_rows(T, E, k)


def moe_align_small_tile_rows(T: int, E: int, k: int) -> int:
    return lib().moe_align_small_tile_rows(T, E, k)


def moe_align_max_rows(T: int, E: int, k: int) -> int:
    return lib().moe_align_max_rows(T, E, k)


def moe_align_max_big_tiles(T: int, E: int, k: int) -> int:
    return lib().moe_align_max_big_tiles(T, E, k)


def moe_align_max_tiles(T: int, E: int, k: int) -> int:
    return lib().moe_align_max_tiles(T, E, k)


def moe_workspace_size(T: int, H: int, E: int, k: int, I: int, I_s: int) -> int:
    return lib().moe_workspace_size(T, H, E, k, I, I_s)


def moe_forward_ids_offset(T: int, H: int, E: int, k: int, I: int, I_s: int) -> int:
    return lib().moe_forward_ids_offset(T, H, E, k, I, I_s)


def moe_workspace_sections(T: int, H: int, E: int, k: int, I: int, I_s: int):
    """[(offset, bytes)] of the workspace sections moe_forward carves for these sizes (host only)."""
    L = lib()
    n = L.moe_workspace_sections(T, H, E, k, I, I_s, None, None, 0)
    if n <= 0:
        return []
    off = (C.c_size_t * n)()
    nb = (C.c_size_t * n)()
    L.moe_workspace_sections(T, H, E, k, I, I_s, off, nb, n)
    return [(int(off[i]), int(nb[i])) for i in range(n)]


def moe_align_scratch_size(T: int, E: int, k: int) -> int:
    return lib().moe_align_scratch_size(T, E, k)


# ------------------------------------------------------------- stages
def moe_forward(x, w_router, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, w_sg,
                T, H, E, k, I, I_s, y, workspace, ws_bytes: int, stream=None):
    _check(lib().moe_forward(_p(x), _p(w_router), _p(router_bias), _p(w_gate), _p(w_up), _p(w_down),
                             _p(ws_gate), _p(ws_up), _p(ws_down), _p(w_sg), T, H, E, k, I, I_s,
                             _p(y), _p(workspace), ws_bytes, _stream(stream)))


def moe_forward_noalloc(x, w_router, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, w_sg,
                        T, H, E, k, I, I_s, y, stream=None):
    _check(lib().moe_forward_noalloc(_p(x), _p(w_router), _p(router_bias), _p(w_gate), _p(w_up), _p(w_down),
                                     _p(ws_gate), _p(ws_up), _p(ws_down), _p(w_sg), T, H, E, k, I, I_s,
                                     _p(y), _stream(stream)))


def moe_forward_fp8(x, w_router, router_bias, q_gate, sc_gate, q_up, sc_up, q_down, sc_down,
                    qs_gate, ssc_gate, qs_up, ssc_up, qs_down, ssc_down, w_sg,
                    T, H, E, k, I, I_s, y, workspace, ws_bytes: int, stream=None):
    _check(lib().moe_forward_fp8(_p(x), _p(w_router), _p(router_bias), _p(q_gate), _p(sc_gate), _p(q_up),
                                 _p(sc_up), _p(q_down), _p(sc_down), _p(qs_gate), _p(ssc_gate), _p(qs_up),
                                 _p(ssc_up), _p(qs_down), _p(ssc_down), _p(w_sg), T, H, E, k, I, I_s,
                                 _p(y), _p(workspace), ws_bytes, _stream(stream)))


def moe_forward_q4(x, w_router, router_bias, q_gate, s_gate, q_up, s_up, q_down, s_down,
                   qs_gate, ss_gate, qs_up, ss_up, qs_down, ss_down, w_sg,
                   T, H, E, k, I, I_s, y, workspace, ws_bytes: int, stream=None):
    _check(lib().moe_forward_q4(_p(x), _p(w_router), _p(router_bias), _p(q_gate), _p(s_gate), _p(q_up),
                                _p(s_up), _p(q_down), _p(s_down), _p(qs_gate), _p(ss_gate), _p(qs_up),
                                _p(ss_up), _p(qs_down), _p(ss_down), _p(w_sg), T, H, E, k, I, I_s,
                                _p(y), _p(workspace), ws_bytes, _stream(stream)))


def moe_e4m3_to_f32(codes, out, n: int, stream=None):
    _check(lib().moe_e4m3_to_f32(_p(codes), _p(out), n, _stream(stream)))


def moe_bucket_plan(T: int, buckets):
    """(segment bucket sizes, real tokens per segment) covering T tokens (host only)."""
    nb = len(buckets)
    barr = (C.c_int * max(nb, 1))(*buckets)
    n = C.c_int(0)
    cap = 64
    while True:
        sb, sl = (C.c_int * cap)(), (C.c_int * cap)()
        rc = lib().moe_bucket_plan(T, barr, nb, sb, sl, cap, C.byref(n))
        if rc == MOE_ERR_SHAPE and n.value > cap:
            cap = n.value
            continue
        _check(rc)
        return list(sb[:n.value]), list(sl[:n.value])


def moe_prefill_runner_create(w_router, router_bias, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, w_sg,
                              H, E, k, I, I_s, buckets) -> int:
    """Opaque runner handle (an int); free it with moe_prefill_runner_destroy."""
    nb = len(buckets)
    barr = (C.c_int * max(nb, 1))(*buckets)
    out = C.c_void_p()
    _check(lib().moe_prefill_runner_create(_p(w_router), _p(router_bias), _p(w_gate), _p(w_up), _p(w_down),
                                           _p(ws_gate), _p(ws_up), _p(ws_down), _p(w_sg), H, E, k, I, I_s,
                                           barr, nb, C.byref(out)))
    return out.value


def moe_prefill_runner_create_fp8(w_router, router_bias, q_gate, sc_gate, q_up, sc_up, q_down, sc_down,
                                  qs_gate, ssc_gate, qs_up, ssc_up, qs_down, ssc_down, w_sg,
                                  H, E, k, I, I_s, buckets) -> int:
    """Runner over FP8 expert weights (codes and row scales as moe_forward_fp8)."""
    nb = len(buckets)
    barr = (C.c_int * max(nb, 1))(*buckets)
    out = C.c_void_p()
    _check(lib().moe_prefill_runner_create_fp8(_p(w_router), _p(router_bias), _p(q_gate), _p(sc_gate), _p(q_up),
                                               _p(sc_up), _p(q_down), _p(sc_down), _p(qs_gate), _p(ssc_gate),
                                               _p(qs_up), _p(ssc_up), _p(qs_down), _p(ssc_down), _p(w_sg),
                                               H, E, k, I, I_s, barr, nb, C.byref(out)))
    return out.value


def moe_prefill_runner_run(runner: int, x, T: int, y, stream=None):
    _check(lib().moe_prefill_runner_run(runner, _p(x), T, _p(y), _stream(stream)))


def moe_prefill_runner_destroy(runner: Optional[int]):
    _check(lib().moe_prefill_runner_destroy(runner))


def moe_route_scratch_size(T, H, E):
    return lib().moe_route_scratch_size(T, H, E)


def moe_route(x, w_router, router_bias, w_sg, T, H, E, k, ids, w, s, logits, stream=None, scratch=None):
    """scratch (a device tensor of moe_route_scratch_size bytes or more) selects the streamed form."""
    nbytes = scratch.numel() * scratch.element_size() if scratch is not None else 0
    _check(lib().moe_route(_p(x), _p(w_router), _p(router_bias), _p(w_sg), T, H, E, k,
                           _p(ids), _p(w), _p(s), _p(logits), _p(scratch), nbytes, _stream(stream)))


def moe_route_from_logits(logits, T, E, k, ids, w, stream=None):
    _check(lib().moe_route_from_logits(_p(logits), T, E, k, _p(ids), _p(w), _stream(stream)))


def moe_align(ids, T, E, k, counts, pad_off, sorted_rows, inv, tiles, n_tiles, scratch, scratch_bytes,
              stream=None):
    _check(lib().moe_align(_p(ids), T, E, k, _p(counts), _p(pad_off), _p(sorted_rows),
                           _p(inv), _p(tiles), _p(n_tiles), _p(scratch), scratch_bytes, _stream(stream)))


def moe_grouped_gate_up(x, w_gate, w_up, ws_gate, ws_up, sorted_rows, tiles, n_tiles, T, H, E, k, I, I_s,
                        h, h_s, stream=None):
    _check(lib().moe_grouped_gate_up(_p(x), _p(w_gate), _p(w_up), _p(ws_gate), _p(ws_up), _p(sorted_rows),
                                     _p(tiles), _p(n_tiles), T, H, E, k, I, I_s, _p(h), _p(h_s),
                                     _stream(stream)))


def moe_grouped_down(h, w_down, sorted_rows, tiles, n_tiles, T, H, E, k, I, o, stream=None):
    _check(lib().moe_grouped_down(_p(h), _p(w_down), _p(sorted_rows), _p(tiles), _p(n_tiles), T, H, E, k, I,
                                  _p(o), _stream(stream)))


def moe_combine(o, w, h_s, ws_down, s, T, H, k, I_s, y, stream=None):
    _check(lib().moe_combine(_p(o), _p(w), _p(h_s), _p(ws_down), _p(s), T, H, k, I_s, _p(y),
                             _stream(stream)))
