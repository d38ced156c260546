"""Thin ctypes binding of libconvt3d (include/convt3d.h).

The functions keep the C names and only marshal arguments: torch tensors (or
raw integers) become device pointers, a torch stream becomes a hipStream_t.
All computation happens in the library's HIP kernels; if the library is not
built, every call raises instead of falling back to anything else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libconvt3d.so")

EPI_NONE = 0
EPI_RELU_GROUPNORM = 1
EPI_SOFTMAX_SIGMOID = 2
EPI_SCALE_BN_TRAIN_AVGPOOL = 3
EPI_SCALE_BN_EVAL_AVGPOOL = 4
POOLED = (EPI_SCALE_BN_TRAIN_AVGPOOL, EPI_SCALE_BN_EVAL_AVGPOOL)

STATUS = {
    0: "OK", 1: "ERR_NULL", 2: "ERR_GEOMETRY", 3: "ERR_GROUPS", 4: "ERR_ALIGNMENT",
    5: "ERR_WORKSPACE", 6: "ERR_UNSUPPORTED", 7: "ERR_LAUNCH", 8: "ERR_TOO_LARGE", 9: "ERR_ALIAS",
    10: "ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 32 << 20  # CONVT3D_NOALLOC_SCRATCH_BYTES


class Geom(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int32) for f in ("n", "cin", "cout", "d", "h", "w")] + \
               [(f, ctypes.c_int32 * 3) for f in ("k", "stride", "pad", "out_pad", "dilation")] + \
               [("groups", ctypes.c_int32)]


class Epilogue(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("groups", ctypes.c_int32), ("eps", ctypes.c_float),
                ("scale", ctypes.c_float), ("gamma", ctypes.c_void_p), ("beta", ctypes.c_void_p),
                ("stats_out", ctypes.c_void_p), ("momentum", ctypes.c_float),
                ("running_mean", ctypes.c_void_p), ("running_var", ctypes.c_void_p)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("variant", ctypes.c_int32), ("co_blocks_per_wave", ctypes.c_int32),
                ("pos_blocks_per_wave", ctypes.c_int32), ("w_phases_per_wave", ctypes.c_int32),
                ("waves_co", ctypes.c_int32), ("waves_pos", ctypes.c_int32),
                ("tile_q", ctypes.c_int32 * 3), ("ci_chunk", ctypes.c_int32),
                ("lds_bytes", ctypes.c_int32), ("workgroups", ctypes.c_int64),
                ("issued_macs", ctypes.c_int64), ("valid_macs", ctypes.c_int64),
                ("phase_loop", ctypes.c_int32),
                ("tuned", ctypes.c_int32), ("border_split", ctypes.c_int32), ("xcd_order", ctypes.c_int32),
                ("softmax_pass", ctypes.c_int32), ("eval_bins", ctypes.c_int32),
                ("conv_launches", ctypes.c_int32)]


class TuneResult(ctypes.Structure):
    _fields_ = [("candidates", ctypes.c_int32), ("chosen", ctypes.c_int32), ("chosen_ms", ctypes.c_float),
                ("model_choice_ms", ctypes.c_float)]


class Profile(ctypes.Structure):
    _fields_ = [("calls", ctypes.c_int32), ("conv_ms", ctypes.c_double), ("finalize_ms", ctypes.c_double),
                ("normalize_ms", ctypes.c_double), ("reduce_ms", ctypes.c_double),
                ("prepack_ms", ctypes.c_double)]


class Convt3dError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({status_string(status)})")


_lib = None


def _hip_runtimes():
    """Paths of the HIP runtime libraries mapped into this process (Linux)."""
    try:
        with open("/proc/self/maps") as f:
            return sorted({ln.split()[-1] for ln in f if "libamdhip64" in ln and "/" in ln})
    except OSError:
        return []


def lib():
    """Load libconvt3d.so (built in-tree by activation_epilogues_amd.build).

    torch is imported first: its ROCm build carries its own HIP runtime, and
    the library must bind to that one (the runtime that owns the caller's
    device memory and streams).  Loaded before torch, the library would pull
    in the system HIP runtime and torch would then load its own beside it:
    two runtimes in one process, with torch's stream handles handed to the
    other one.  That state is refused here."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libconvt3d is not built ({LIB_PATH} missing); run "
                               "python -m activation_epilogues_amd.build")
        import torch  # noqa: F401  (binds the process to torch's HIP runtime first)
        L = ctypes.CDLL(LIB_PATH)
        rts = _hip_runtimes()
        if len(rts) > 1:
            raise RuntimeError("more than one HIP runtime is loaded in this process (" + ", ".join(rts) +
                               "); load libconvt3d through this module, after torch")
        P = ctypes.POINTER
        vp, sz = ctypes.c_void_p, ctypes.c_size_t
        L.convt3d_status_string.restype = ctypes.c_char_p
        L.convt3d_status_string.argtypes = [ctypes.c_int]
        L.convt3d_output_dims.restype = ctypes.c_int
        L.convt3d_output_dims.argtypes = [P(Geom), P(ctypes.c_int32)]
        L.convt3d_output_elems.restype = ctypes.c_int64
        L.convt3d_output_elems.argtypes = [P(Geom), P(Epilogue)]
        L.convt3d_packed_weight_bytes.restype = sz
        L.convt3d_packed_weight_bytes.argtypes = [P(Geom)]
        L.convt3d_prepack_weights.restype = ctypes.c_int
        L.convt3d_prepack_weights.argtypes = [P(Geom), vp, vp, vp]
        L.convt3d_eval_weight_bytes.restype = sz
        L.convt3d_eval_weight_bytes.argtypes = [P(Geom)]
        L.convt3d_prepack_eval_weights.restype = ctypes.c_int
        L.convt3d_prepack_eval_weights.argtypes = [P(Geom), vp, vp, vp]
        L.convt3d_epilogue_workspace_size.restype = sz
        L.convt3d_epilogue_workspace_size.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, P(Epilogue)]
        L.convt3d_epilogue_only.restype = ctypes.c_int
        L.convt3d_epilogue_only.argtypes = [vp, ctypes.c_int32, ctypes.c_int32, ctypes.c_int64, P(Epilogue), vp,
                                            vp, sz, vp]
        L.convt3d_workspace_size.restype = sz
        L.convt3d_workspace_size.argtypes = [P(Geom), P(Epilogue)]
        L.convt3d_fused.restype = ctypes.c_int
        L.convt3d_fused.argtypes = [vp, vp, vp, P(Geom), P(Epilogue), vp, vp, sz, vp]
        L.convt3d_fused_noalloc.restype = ctypes.c_int
        L.convt3d_fused_noalloc.argtypes = [vp, vp, vp, P(Geom), P(Epilogue), vp, vp]
        L.convt3d_autotune.restype = ctypes.c_int
        L.convt3d_autotune.argtypes = [vp, vp, vp, P(Geom), P(Epilogue), vp, vp, sz, vp, P(TuneResult)]
        L.convt3d_get_plan_info.restype = ctypes.c_int
        L.convt3d_get_plan_info.argtypes = [P(Geom), P(Epilogue), P(PlanInfo)]
        L.convt3d_profile_begin.restype = ctypes.c_int
        L.convt3d_profile_begin.argtypes = []
        L.convt3d_profile_begin_kinds.restype = ctypes.c_int
        L.convt3d_profile_begin_kinds.argtypes = [ctypes.c_uint32]
        L.convt3d_profile_end.restype = ctypes.c_int
        L.convt3d_profile_end.argtypes = [P(Profile)]
        _lib = L
    return _lib


EXPORTED = ["convt3d_status_string", "convt3d_output_dims", "convt3d_output_elems",
            "convt3d_packed_weight_bytes", "convt3d_prepack_weights", "convt3d_eval_weight_bytes",
            "convt3d_prepack_eval_weights", "convt3d_workspace_size", "convt3d_fused", "convt3d_fused_noalloc",
            "convt3d_autotune",
            "convt3d_epilogue_workspace_size", "convt3d_epilogue_only", "convt3d_get_plan_info",
            "convt3d_profile_begin", "convt3d_profile_begin_kinds", "convt3d_profile_end"]


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or an int / None)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _triple(v):
    t = tuple(int(a) for a in v) if isinstance(v, (tuple, list)) else (int(v),) * 3
    return (ctypes.c_int32 * 3)(*t)


def make_geom(n, cin, cout, d, h, w, k, stride=1, pad=0, out_pad=0, dilation=1, groups=1) -> Geom:
    """k, stride, pad, out_pad and dilation: an int (every dim) or a (d, h, w) triple."""
    return Geom(n, cin, cout, d, h, w, _triple(k), _triple(stride), _triple(pad), _triple(out_pad),
                _triple(dilation), groups)


def make_epilogue(kind, groups=1, eps=1e-5, scale=1.0, gamma=None, beta=None, stats_out=None,
                  momentum=0.1, running_mean=None, running_var=None) -> Epilogue:
    return Epilogue(kind, groups, eps, scale, _ptr(gamma), _ptr(beta), _ptr(stats_out), momentum,
                    _ptr(running_mean), _ptr(running_var))


def status_string(status: int) -> str:
    return lib().convt3d_status_string(status).decode()


def convt3d_status_string(status: int) -> str:
    return status_string(status)


def convt3d_output_dims(geom: Geom):
    arr = (ctypes.c_int32 * 3)()
    st = lib().convt3d_output_dims(ctypes.byref(geom), arr)
    if st:
        raise Convt3dError(st, "convt3d_output_dims")
    return tuple(arr)


def convt3d_output_elems(geom: Geom, epi: Epilogue) -> int:
    return int(lib().convt3d_output_elems(ctypes.byref(geom), ctypes.byref(epi)))


def convt3d_packed_weight_bytes(geom: Geom) -> int:
    return int(lib().convt3d_packed_weight_bytes(ctypes.byref(geom)))


def convt3d_workspace_size(geom: Geom, epi: Epilogue) -> int:
    return int(lib().convt3d_workspace_size(ctypes.byref(geom), ctypes.byref(epi)))


def convt3d_prepack_weights(geom: Geom, w, w_packed, stream=None, check=True) -> int:
    st = lib().convt3d_prepack_weights(ctypes.byref(geom), _ptr(w), _ptr(w_packed), _stream(stream))
    if check and st:
        raise Convt3dError(st, "convt3d_prepack_weights")
    return st


def convt3d_eval_weight_bytes(geom: Geom) -> int:
    return int(lib().convt3d_eval_weight_bytes(ctypes.byref(geom)))


def convt3d_prepack_eval_weights(geom: Geom, w, w_eval, stream=None, check=True) -> int:
    st = lib().convt3d_prepack_eval_weights(ctypes.byref(geom), _ptr(w), _ptr(w_eval), _stream(stream))
    if check and st:
        raise Convt3dError(st, "convt3d_prepack_eval_weights")
    return st


def convt3d_epilogue_workspace_size(n: int, c: int, spatial: int, epi: Epilogue) -> int:
    return int(lib().convt3d_epilogue_workspace_size(n, c, spatial, ctypes.byref(epi)))


def convt3d_epilogue_only(y, n: int, c: int, spatial: int, epi: Epilogue, out, workspace, workspace_bytes: int,
                          stream=None, check=True) -> int:
    st = lib().convt3d_epilogue_only(_ptr(y), n, c, spatial, ctypes.byref(epi), _ptr(out), _ptr(workspace),
                                     workspace_bytes, _stream(stream))
    if check and st:
        raise Convt3dError(st, "convt3d_epilogue_only")
    return st


def convt3d_fused(x, w_packed, bias, geom: Geom, epi: Epilogue, out, workspace, workspace_bytes: int,
                  stream=None, check=True) -> int:
    st = lib().convt3d_fused(_ptr(x), _ptr(w_packed), _ptr(bias), ctypes.byref(geom), ctypes.byref(epi),
                             _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream))
    if check and st:
        raise Convt3dError(st, "convt3d_fused")
    return st


def convt3d_fused_noalloc(x, w_packed, bias, geom: Geom, epi: Epilogue, out, stream=None, check=True) -> int:
    st = lib().convt3d_fused_noalloc(_ptr(x), _ptr(w_packed), _ptr(bias), ctypes.byref(geom), ctypes.byref(epi),
                                     _ptr(out), _stream(stream))
    if check and st:
        raise Convt3dError(st, "convt3d_fused_noalloc")
    return st


def convt3d_autotune(x, w_packed, bias, geom: Geom, epi: Epilogue, out, workspace, workspace_bytes: int,
                     stream=None) -> dict:
    res = TuneResult()
    st = lib().convt3d_autotune(_ptr(x), _ptr(w_packed), _ptr(bias), ctypes.byref(geom), ctypes.byref(epi),
                                _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream), ctypes.byref(res))
    if st:
        raise Convt3dError(st, "convt3d_autotune")
    return {f: getattr(res, f) for f, _ in TuneResult._fields_}


def convt3d_get_plan_info(geom: Geom, epi: Epilogue) -> dict:
    info = PlanInfo()
    st = lib().convt3d_get_plan_info(ctypes.byref(geom), ctypes.byref(epi), ctypes.byref(info))
    if st:
        raise Convt3dError(st, "convt3d_get_plan_info")
    d = {f: getattr(info, f) for f, _ in PlanInfo._fields_}
    d["tile_q"] = tuple(info.tile_q)
    return d


def plan_string(info: dict) -> str:
    """CONVT3D_PLAN value that selects this plan again (with CONVT3D_PHASE_LOOP
    set to info["phase_loop"])."""
    t = info["tile_q"]
    return (f"{info['variant']},{info['waves_co']},{t[0]},{t[1]},{t[2]},{info['ci_chunk']},"
            f"{info['border_split']}")


def convt3d_profile_begin() -> None:
    st = lib().convt3d_profile_begin()
    if st:
        raise Convt3dError(st, "convt3d_profile_begin")


PROFILE_CONV, PROFILE_FINALIZE, PROFILE_NORMALIZE, PROFILE_REDUCE, PROFILE_PREPACK = 0x1, 0x2, 0x4, 0x8, 0x10
PROFILE_ALL = 0x1F


def convt3d_profile_begin_kinds(kinds: int) -> None:
    st = lib().convt3d_profile_begin_kinds(kinds)
    if st:
        raise Convt3dError(st, "convt3d_profile_begin_kinds")


def convt3d_profile_end() -> dict:
    p = Profile()
    st = lib().convt3d_profile_end(ctypes.byref(p))
    if st:
        raise Convt3dError(st, "convt3d_profile_end")
    return {f: getattr(p, f) for f, _ in Profile._fields_}


# ----------------------------------------------------------------------------
# Device-memory plumbing with torch (allocation only; no arithmetic).

class FusedCall:
    """Holds the device buffers of one geometry/epilogue and calls the library.

    Allocates with torch (packed weights, workspace, output, stats); every step
    of the computation runs in libconvt3d.
    """

    def __init__(self, geom: Geom, kind: int, groups: int = 1, eps: float = 1e-5, scale: float = 1.0,
                 device="cuda", want_stats: bool = False, momentum: float = 0.1):
        import torch
        self.geom = geom
        self.kind = kind
        self.groups, self.eps, self.scale, self.momentum = groups, eps, scale, momentum
        probe = make_epilogue(kind, groups, eps, scale)
        self.out_dims = convt3d_output_dims(geom)
        self.out_elems = convt3d_output_elems(geom, probe)
        if self.out_elems < 0:
            raise Convt3dError(2, "convt3d_output_elems")
        self.ws_bytes = convt3d_workspace_size(geom, probe)
        if kind == EPI_SCALE_BN_EVAL_AVGPOOL:  # tap-summed weights, no conv operand
            self.packed_bytes = convt3d_eval_weight_bytes(geom)
        else:
            self.packed_bytes = convt3d_packed_weight_bytes(geom)
        if self.packed_bytes == 0:
            raise Convt3dError(6, "weight buffer size")
        self.w_packed = torch.empty(max(1, self.packed_bytes // 4), dtype=torch.float32, device=device)
        self.workspace = torch.empty(max(1, self.ws_bytes // 4), dtype=torch.float32, device=device)
        if kind in POOLED:
            self.out = torch.empty((geom.n, geom.cout, 1, 1, 1), dtype=torch.float32, device=device)
        else:
            self.out = torch.empty((geom.n, geom.cout) + tuple(self.out_dims), dtype=torch.float32,
                                   device=device)
        self.stats = None
        if want_stats:
            if kind == EPI_RELU_GROUPNORM:
                self.stats = torch.empty((geom.n, groups, 2), dtype=torch.float32, device=device)
            elif kind == EPI_SCALE_BN_TRAIN_AVGPOOL:
                self.stats = torch.empty((geom.cout, 2), dtype=torch.float32, device=device)

    def epilogue(self, gamma=None, beta=None, running_mean=None, running_var=None) -> Epilogue:
        return make_epilogue(self.kind, self.groups, self.eps, self.scale, gamma, beta, self.stats,
                             self.momentum, running_mean, running_var)

    def prepack(self, w, stream=None):
        if self.kind == EPI_SCALE_BN_EVAL_AVGPOOL:
            convt3d_prepack_eval_weights(self.geom, w, self.w_packed, stream)
        else:
            convt3d_prepack_weights(self.geom, w, self.w_packed, stream)

    def __call__(self, x, bias=None, gamma=None, beta=None, stream=None, running_mean=None, running_var=None):
        convt3d_fused(x, self.w_packed, bias, self.geom, self.epilogue(gamma, beta, running_mean, running_var),
                      self.out, self.workspace, self.ws_bytes, stream)
        return self.out

    def autotune(self, x, bias=None, gamma=None, beta=None, stream=None) -> dict:
        """Time the candidate plans on these buffers and keep the fastest."""
        return convt3d_autotune(x, self.w_packed, bias, self.geom, self.epilogue(gamma, beta), self.out,
                                self.workspace, self.ws_bytes, stream)

    def plan_info(self) -> dict:
        return convt3d_get_plan_info(self.geom, self.epilogue())
