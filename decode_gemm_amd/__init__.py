"""Python binding of libuw (include/uw.h): argument marshalling only.

Every step of the method runs in libuw.so (host encoder in C++, everything else in HIP
kernels for gfx950). PyTorch tensors supply device memory and streams; a "d_" argument
may be a torch tensor on the GPU or a raw device address (int). Host arrays are NumPy.

Importing this package loads libuw.so and raises ImportError if it has not been built
(`python -m decode_gemm_amd.build`); there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import importlib.util
import os

import numpy as np

__all__ = [
    "UwError", "Header", "Plan", "lib", "encode", "inspect", "validate_header", "decode_full",
    "decode_exponent", "transcode_palette", "prepare_direct", "recon_gemm", "run_pipeline", "autotune", "swiglu",
    "workspace_bytes", "direct_plane_bytes", "variant_count", "variant_name", "variant_supports", "version",
    "W_BF16", "W_EXP", "W_IDX", "W_DIRECT", "PIPE_FULL", "PIPE_EXP", "PIPE_TRANSCODE", "PIPE_DIRECT", "PIPE_EXPAND",
    "expand_direct", "split_count", "run_pipeline_noalloc", "noalloc_scratch_bytes", "bundle_write", "bundle_open",
    "bundle_items", "bundle_plans", "load_bundle", "variant_by_name",
    "DERR_BADCODE", "DERR_CHUNKLEN", "DERR_RAWINDEX", "STATUS", "Proj", "MlpLayer", "proj", "mlp_layers", "mlp_stack_workspace",
    "mlp_stack_forward",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libuw.so")

STATUS = {0: "UW_OK", 1: "UW_EINVAL", 2: "UW_ESHAPE", 3: "UW_EFORMAT", 4: "UW_ERANGE", 5: "UW_ENOSPACE",
          6: "UW_EHIP", 7: "UW_EUNSUPPORTED", 8: "UW_EINTERNAL"}
OK, EINVAL, ESHAPE, EFORMAT, ERANGE, ENOSPACE, EHIP, EUNSUPPORTED, EINTERNAL = range(9)
W_BF16, W_EXP, W_IDX, W_DIRECT = 0, 1, 2, 3
PIPE_FULL, PIPE_EXP, PIPE_TRANSCODE, PIPE_DIRECT, PIPE_EXPAND = 0, 1, 2, 3, 4
PIPELINE_NAMES = {0: "full", 1: "exp", 2: "transcode", 3: "direct", 4: "expand"}
DERR_BADCODE, DERR_CHUNKLEN, DERR_RAWINDEX = 1, 2, 4


class UwError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


class Header(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint32), ("N", ctypes.c_int64), ("K", ctypes.c_int64),
        ("chunk", ctypes.c_uint32), ("lmax", ctypes.c_uint32), ("n_pal", ctypes.c_uint32),
        ("n_chunks", ctypes.c_uint32), ("palette", ctypes.c_uint8 * 16), ("code_len", ctypes.c_uint8 * 16),
        ("n_raw", ctypes.c_int64), ("total_bits", ctypes.c_uint64), ("off_sm", ctypes.c_uint64),
        ("off_bitmap", ctypes.c_uint64), ("off_rowbase", ctypes.c_uint64), ("off_raw", ctypes.c_uint64),
        ("off_chunk", ctypes.c_uint64), ("off_stream", ctypes.c_uint64), ("bytes_stream", ctypes.c_uint64),
        ("total_bytes", ctypes.c_uint64), ("bitmap_words", ctypes.c_uint32), ("reserved", ctypes.c_uint32 * 25),
    ]


class EncodeOpts(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_uint32), ("lmax", ctypes.c_uint32)]


class GemmArgs(ctypes.Structure):
    _fields_ = [
        ("M", ctypes.c_int64), ("d_x", ctypes.c_void_p), ("ldx", ctypes.c_int64), ("h", ctypes.POINTER(Header)),
        ("d_blob", ctypes.c_void_p), ("src", ctypes.c_int32), ("d_wplane", ctypes.c_void_p),
        ("d_y", ctypes.c_void_p), ("ldy", ctypes.c_int64), ("variant", ctypes.c_int32), ("split_k", ctypes.c_int32),
    ]


class Plan(ctypes.Structure):
    _fields_ = [("pipeline", ctypes.c_int32), ("variant", ctypes.c_int32), ("t_ms", ctypes.c_float),
                ("split_k", ctypes.c_int32)]

    def __repr__(self):
        return (f"Plan(pipeline={PIPELINE_NAMES.get(self.pipeline, self.pipeline)}, variant={self.variant}, "
                f"split_k={self.split_k}, t_ms={self.t_ms:.4f})")


class Proj(ctypes.Structure):
    """uw_proj: one projection of a model and the pipeline / variant / K split it runs with."""
    _fields_ = [("h", ctypes.POINTER(Header)), ("d_blob", ctypes.c_void_p), ("d_direct", ctypes.c_void_p),
                ("pipeline", ctypes.c_int32), ("variant", ctypes.c_int32), ("split_k", ctypes.c_int32)]


class MlpLayer(ctypes.Structure):
    _fields_ = [("gate", Proj), ("up", Proj), ("down", Proj)]


class StackOpts(ctypes.Structure):
    """uw_stack_opts: decode slots and decode order of a stack forward."""
    _fields_ = [("slots", ctypes.c_int32), ("down_first", ctypes.c_int32)]


class StackTuneArgs(ctypes.Structure):
    _fields_ = [
        ("layers", ctypes.POINTER(MlpLayer)), ("n_layers", ctypes.c_int32), ("M", ctypes.c_int64),
        ("d_x", ctypes.c_void_p), ("d_y", ctypes.c_void_p), ("d_ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
        ("decode_stream", ctypes.c_void_p), ("opts", StackOpts), ("pipeline_mask", ctypes.c_uint32),
        ("reps", ctypes.c_int32), ("warmup", ctypes.c_int32), ("max_passes", ctypes.c_int32),
        ("t_start_ms", ctypes.c_float), ("t_ms", ctypes.c_float), ("passes", ctypes.c_int32), ("trials", ctypes.c_int32),
    ]


class TuneArgs(ctypes.Structure):
    _fields_ = [
        ("h", ctypes.POINTER(Header)), ("d_blob", ctypes.c_void_p), ("d_direct", ctypes.c_void_p),
        ("d_x", ctypes.c_void_p), ("d_y", ctypes.c_void_p), ("d_ws", ctypes.c_void_p), ("ws_bytes", ctypes.c_size_t),
        ("reps", ctypes.c_int32), ("warmup", ctypes.c_int32), ("pipeline_mask", ctypes.c_uint32),
        ("variant_mask", ctypes.c_int32), ("d_scrub", ctypes.c_void_p), ("scrub_bytes", ctypes.c_size_t),
        ("rot", ctypes.POINTER(Proj)), ("n_rot", ctypes.c_int32), ("trials", ctypes.c_int32),
        ("tune_split", ctypes.c_int32),
    ]


class BundleItem(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("blob", ctypes.c_void_p), ("blob_bytes", ctypes.c_size_t)]


class BundlePlan(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("K", ctypes.c_int64), ("M", ctypes.c_int64), ("pipeline", ctypes.c_int32),
                ("split_k", ctypes.c_int32), ("t_ms", ctypes.c_float), ("variant", ctypes.c_char * 48)]


class BundleInfo(ctypes.Structure):
    _fields_ = [("n_items", ctypes.c_uint32), ("n_plans", ctypes.c_uint32), ("total_bytes", ctypes.c_uint64)]


class BundleEntry(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 64), ("offset", ctypes.c_uint64), ("blob_bytes", ctypes.c_uint64),
                ("header", Header)]


def _preload_torch_hip():
    """Load the HIP runtime that PyTorch ships, if PyTorch is installed, before libuw.so.

    A process can drive the GPU through one HIP runtime only, and the tensors handed to
    libuw come from PyTorch's. With PyTorch's copy already loaded, libuw's dependency on
    libamdhip64 resolves to it whatever the import order; otherwise the system copy would
    be loaded first and the second runtime to start would find no device."""
    spec = importlib.util.find_spec("torch")
    for d in (spec.submodule_search_locations or []) if spec else []:
        path = os.path.join(d, "lib", "libamdhip64.so")
        if os.path.exists(path):
            ctypes.CDLL(path, mode=ctypes.RTLD_GLOBAL)
            return


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libuw.so not built at {LIB_PATH}; run `python decode_gemm_amd/build.py` "
                          "or __graft_entry__.build()")
    _preload_torch_hip()
    L = ctypes.CDLL(LIB_PATH)
    P, i32, i64, u32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_size_t
    H = ctypes.POINTER(Header)
    sigs = {
        "uw_status_string": ([ctypes.c_int], ctypes.c_char_p),
        "uw_last_error": ([], ctypes.c_char_p),
        "uw_version": ([], ctypes.c_int),
        "uw_encode": ([P, i64, i64, ctypes.POINTER(EncodeOpts), P, ctypes.POINTER(sz)], ctypes.c_int),
        "uw_inspect": ([P, sz, H], ctypes.c_int),
        "uw_validate_header": ([H, sz], ctypes.c_int),
        "uw_decode_full": ([H, P, P, P, P], ctypes.c_int),
        "uw_decode_exponent": ([H, P, P, P, P], ctypes.c_int),
        "uw_transcode_palette": ([H, P, P, P, P], ctypes.c_int),
        "uw_prepare_direct": ([H, P, P, P, P], ctypes.c_int),
        "uw_direct_plane_bytes": ([H, ctypes.POINTER(sz)], ctypes.c_int),
        "uw_recon_gemm": ([ctypes.POINTER(GemmArgs), P], ctypes.c_int),
        "uw_recon_gemm_gate_up": ([ctypes.POINTER(GemmArgs), ctypes.POINTER(GemmArgs), P, i64, P], ctypes.c_int),
        "uw_variant_count": ([], ctypes.c_int),
        "uw_variant_name": ([ctypes.c_int], ctypes.c_char_p),
        "uw_variant_supports": ([ctypes.c_int, i64, i64, i64, i32], ctypes.c_int),
        "uw_workspace_bytes": ([H, i32, ctypes.POINTER(sz)], ctypes.c_int),
        "uw_run_pipeline": ([i32, i32, i32, H, P, P, i64, P, i64, P, i64, P, sz, P, P], ctypes.c_int),
        "uw_split_count": ([ctypes.c_int, i64, i64, i64, i32], ctypes.c_int),
        "uw_run_pipeline_noalloc": ([i32, i32, i32, H, P, P, i64, P, i64, P, i64, P, P], ctypes.c_int),
        "uw_noalloc_scratch_bytes": ([], sz),
        "uw_bundle_write": ([ctypes.POINTER(BundleItem), ctypes.c_int, ctypes.POINTER(BundlePlan), ctypes.c_int, P,
                             ctypes.POINTER(sz)], ctypes.c_int),
        "uw_bundle_open": ([P, sz, ctypes.c_int, ctypes.POINTER(BundleInfo)], ctypes.c_int),
        "uw_bundle_item_at": ([P, sz, u32, ctypes.POINTER(BundleEntry)], ctypes.c_int),
        "uw_bundle_plan_at": ([P, sz, u32, ctypes.POINTER(BundlePlan)], ctypes.c_int),
        "uw_variant_by_name": ([ctypes.c_char_p], ctypes.c_int),
        "uw_autotune": ([ctypes.POINTER(TuneArgs), ctypes.POINTER(i64), ctypes.c_int, P, ctypes.POINTER(Plan)],
                        ctypes.c_int),
        "uw_swiglu": ([P, P, i64, P, P], ctypes.c_int),
        "uw_mlp_stack_workspace": ([ctypes.POINTER(MlpLayer), ctypes.c_int, i64, ctypes.c_int, ctypes.POINTER(sz)],
                                   ctypes.c_int),
        "uw_mlp_stack_forward": ([ctypes.POINTER(MlpLayer), ctypes.c_int, i64, P, P, P, sz, P, P], ctypes.c_int),
        "uw_mlp_stack_workspace_ex": ([ctypes.POINTER(MlpLayer), ctypes.c_int, i64, ctypes.POINTER(StackOpts),
                                       ctypes.POINTER(sz)], ctypes.c_int),
        "uw_mlp_stack_forward_ex": ([ctypes.POINTER(MlpLayer), ctypes.c_int, i64, P, P, P, sz, P, P,
                                     ctypes.POINTER(StackOpts)], ctypes.c_int),
        "uw_mlp_stack_autotune": ([ctypes.POINTER(StackTuneArgs), P], ctypes.c_int),
        "uw_stream_pair_create": ([ctypes.c_int, ctypes.POINTER(P), ctypes.POINTER(P)], ctypes.c_int),
        "uw_stream_destroy": ([P], ctypes.c_int),
        "uw_stream_cu_count": ([P, ctypes.POINTER(ctypes.c_int)], ctypes.c_int),
        "uw_stream_read": ([P, ctypes.c_size_t, P, P], ctypes.c_int),
        "uw_expand_direct": ([H, P, P, P], ctypes.c_int),
    }
    for name, (args, res) in sigs.items():
        f = getattr(L, name)
        f.argtypes = args
        f.restype = res
    return L


lib = _load()


def _check(status: int):
    if status != OK:
        raise UwError(status, lib.uw_last_error().decode())


def _ptr(t):
    """Device address of a torch tensor, an int address, or None."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def version() -> int:
    return lib.uw_version()


# ---------------------------------------------------------------- host
def encode(w: np.ndarray, chunk: int = 0, lmax: int = 0) -> np.ndarray:
    """uw_encode: W [N][K] bf16 bit patterns (uint16, host) -> blob (uint8, host)."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    if w.ndim != 2:
        raise ValueError("w must be 2-D [N][K]")
    N, K = w.shape
    opts = EncodeOpts(chunk, lmax)
    need = ctypes.c_size_t(0)
    st = lib.uw_encode(w.ctypes.data, N, K, ctypes.byref(opts), None, ctypes.byref(need))
    if st != ENOSPACE:
        _check(st)
    blob = np.empty(need.value, np.uint8)
    _check(lib.uw_encode(w.ctypes.data, N, K, ctypes.byref(opts), blob.ctypes.data, ctypes.byref(need)))
    return blob


def inspect(blob: np.ndarray) -> Header:
    """uw_inspect: validate a host blob and return its header."""
    b = np.ascontiguousarray(blob, dtype=np.uint8)
    h = Header()
    _check(lib.uw_inspect(b.ctypes.data, b.size, ctypes.byref(h)))
    return h


def validate_header(h: Header, blob_bytes: int) -> None:
    _check(lib.uw_validate_header(ctypes.byref(h), blob_bytes))


def workspace_bytes(h: Header, pipeline: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.uw_workspace_bytes(ctypes.byref(h), pipeline, ctypes.byref(out)))
    return out.value


def variant_count() -> int:
    return lib.uw_variant_count()


def variant_name(v: int) -> str:
    return lib.uw_variant_name(v).decode()


def variant_supports(v: int, N: int, K: int, M: int, src: int) -> bool:
    return bool(lib.uw_variant_supports(v, N, K, M, src))


# ---------------------------------------------------------------- device
def decode_full(h: Header, d_blob, d_w, d_err=None, stream=None) -> None:
    _check(lib.uw_decode_full(ctypes.byref(h), _ptr(d_blob), _ptr(d_w), _ptr(d_err), _stream(stream)))


def decode_exponent(h: Header, d_blob, d_exp, d_err=None, stream=None) -> None:
    _check(lib.uw_decode_exponent(ctypes.byref(h), _ptr(d_blob), _ptr(d_exp), _ptr(d_err), _stream(stream)))


def transcode_palette(h: Header, d_blob, d_idx, d_err=None, stream=None) -> None:
    _check(lib.uw_transcode_palette(ctypes.byref(h), _ptr(d_blob), _ptr(d_idx), _ptr(d_err), _stream(stream)))


def prepare_direct(h: Header, d_blob, d_direct, d_err=None, stream=None) -> None:
    """uw_prepare_direct: the direct-palette plane (direct_plane_bytes(h) bytes), made once at load."""
    _check(lib.uw_prepare_direct(ctypes.byref(h), _ptr(d_blob), _ptr(d_direct), _ptr(d_err), _stream(stream)))


def expand_direct(h: Header, d_direct, d_w, stream=None) -> None:
    """uw_expand_direct: bf16 W[N][K] (2*N*K bytes at d_w) rebuilt from a direct plane."""
    _check(lib.uw_expand_direct(ctypes.byref(h), _ptr(d_direct), _ptr(d_w), _stream(stream)))


def direct_plane_bytes(h: Header) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.uw_direct_plane_bytes(ctypes.byref(h), ctypes.byref(out)))
    return out.value


def split_count(v: int, N: int, K: int, M: int, split_k: int = 0) -> int:
    """uw_split_count: K slices a launch of variant v (-1 = default) with split_k uses."""
    return lib.uw_split_count(v, N, K, M, split_k)


def recon_gemm(h: Header, d_blob, src: int, d_wplane, d_x, d_y, M: int, ldx: int | None = None,
               ldy: int | None = None, variant: int = -1, stream=None, split_k: int = 0) -> None:
    a = GemmArgs(M, _ptr(d_x), h.K if ldx is None else ldx, ctypes.pointer(h), _ptr(d_blob), src, _ptr(d_wplane),
                 _ptr(d_y), h.N if ldy is None else ldy, variant, split_k)
    _check(lib.uw_recon_gemm(ctypes.byref(a), _stream(stream)))


def recon_gemm_gate_up(hg: Header, d_blob_g, d_direct_g, hu: Header, d_blob_u, d_direct_u, d_x, d_yg, d_yu, d_h,
                       M: int, ldx: int | None = None, ldf: int | None = None, variant: int = -1,
                       stream=None, split_k: int = 0) -> None:
    """uw_recon_gemm_gate_up: gate and up (direct planes, same X) and h = bf16(silu(g) * u)
    in one launch; raises UwError(EUNSUPPORTED) where the fused form does not apply."""
    lx = hg.K if ldx is None else ldx
    lf = hg.N if ldf is None else ldf
    ag = GemmArgs(M, _ptr(d_x), lx, ctypes.pointer(hg), _ptr(d_blob_g), W_DIRECT, _ptr(d_direct_g), _ptr(d_yg), lf,
                  variant, split_k)
    au = GemmArgs(M, _ptr(d_x), lx, ctypes.pointer(hu), _ptr(d_blob_u), W_DIRECT, _ptr(d_direct_u), _ptr(d_yu), lf,
                  variant, split_k)
    _check(lib.uw_recon_gemm_gate_up(ctypes.byref(ag), ctypes.byref(au), _ptr(d_h), lf, _stream(stream)))


def run_pipeline(pipeline: int, h: Header, d_blob, d_x, d_y, M: int, d_direct=None, d_ws=None, ws_bytes: int = 0,
                 variant: int = -1, d_err=None, ldx: int | None = None, ldy: int | None = None, stream=None,
                 split_k: int = 0) -> None:
    _check(lib.uw_run_pipeline(pipeline, variant, split_k, ctypes.byref(h), _ptr(d_blob), _ptr(d_direct), M, _ptr(d_x),
                               h.K if ldx is None else ldx, _ptr(d_y), h.N if ldy is None else ldy, _ptr(d_ws),
                               ws_bytes, _ptr(d_err), _stream(stream)))


def run_pipeline_noalloc(pipeline: int, h: Header, d_blob, d_x, d_y, M: int, d_direct=None, variant: int = -1,
                         split_k: int = 0, d_err=None, ldx: int | None = None, ldy: int | None = None,
                         stream=None) -> None:
    """uw_run_pipeline_noalloc: the pipeline with its preprocessing slot in the library's
    scratch array (noalloc_scratch_bytes()); calls that overlap on one GPU race on it."""
    _check(lib.uw_run_pipeline_noalloc(pipeline, variant, split_k, ctypes.byref(h), _ptr(d_blob), _ptr(d_direct), M,
                                       _ptr(d_x), h.K if ldx is None else ldx, _ptr(d_y), h.N if ldy is None else ldy,
                                       _ptr(d_err), _stream(stream)))


def noalloc_scratch_bytes() -> int:
    return lib.uw_noalloc_scratch_bytes()


def autotune(h: Header, d_blob, d_x, d_y, Ms, d_direct=None, d_ws=None, ws_bytes: int = 0, reps: int = 0,
             warmup: int = 0, pipeline_mask: int = 0, variant_mask: int = 0, d_scrub=None, scrub_bytes: int = 0,
             stream=None, rot=None, trials: int = 0, tune_split: bool = False) -> list:
    """uw_autotune. rot: optional list of Proj (same N, K) cycled through by every timed
    forward, as a model's layers are; without it the one matrix (h, d_blob, d_direct)."""
    rarr = None
    if rot:
        rarr = (Proj * len(rot))(*rot)
    a = TuneArgs(ctypes.pointer(h), _ptr(d_blob), _ptr(d_direct), _ptr(d_x), _ptr(d_y), _ptr(d_ws), ws_bytes, reps,
                 warmup, pipeline_mask, variant_mask, _ptr(d_scrub), scrub_bytes,
                 ctypes.cast(rarr, ctypes.POINTER(Proj)) if rarr is not None else None, len(rot) if rot else 0,
                 trials, int(tune_split))
    ms = (ctypes.c_int64 * len(Ms))(*Ms)
    out = (Plan * len(Ms))()
    _check(lib.uw_autotune(ctypes.byref(a), ms, len(Ms), _stream(stream), out))
    return list(out)


def swiglu(d_g, d_u, d_h, n: int, stream=None) -> None:
    _check(lib.uw_swiglu(_ptr(d_g), _ptr(d_u), n, _ptr(d_h), _stream(stream)))


def proj(h: Header, d_blob, pipeline: int = PIPE_DIRECT, d_direct=None, variant: int = -1, split_k: int = 0) -> Proj:
    """A uw_proj; keep `h` alive as long as the layer array is used."""
    return Proj(ctypes.pointer(h), _ptr(d_blob), _ptr(d_direct), pipeline, variant, split_k)


def mlp_layers(layers) -> ctypes.Array:
    """uw_mlp_layer array from (gate, up, down) Proj triples."""
    arr = (MlpLayer * len(layers))()
    for i, (g, u, d) in enumerate(layers):
        arr[i] = MlpLayer(g, u, d)
    return arr


def mlp_stack_workspace(layers: ctypes.Array, M: int, two_slots: bool = False) -> int:
    out = ctypes.c_size_t(0)
    _check(lib.uw_mlp_stack_workspace(layers, len(layers), M, int(two_slots), ctypes.byref(out)))
    return out.value


def mlp_stack_forward(layers: ctypes.Array, M: int, d_x, d_y, d_ws, ws_bytes: int, stream=None,
                      decode_stream=None) -> None:
    """uw_mlp_stack_forward: every layer's SwiGLU MLP on the same X; d_y ends as the last
    layer's output. decode_stream (optional) decodes one projection ahead."""
    _check(lib.uw_mlp_stack_forward(layers, len(layers), M, _ptr(d_x), _ptr(d_y), _ptr(d_ws), ws_bytes,
                                    _stream(stream), None if decode_stream is None else _stream(decode_stream)))


def mlp_stack_workspace_ex(layers: ctypes.Array, M: int, slots: int = 2, down_first: bool = False) -> int:
    out = ctypes.c_size_t(0)
    opts = StackOpts(slots, int(down_first))
    _check(lib.uw_mlp_stack_workspace_ex(layers, len(layers), M, ctypes.byref(opts), ctypes.byref(out)))
    return out.value


def mlp_stack_forward_ex(layers: ctypes.Array, M: int, d_x, d_y, d_ws, ws_bytes: int, stream=None, decode_stream=None,
                         slots: int = 2, down_first: bool = False) -> None:
    """uw_mlp_stack_forward_ex: the stack forward with `slots` decode slots and, optionally,
    each layer's down projection decoded before its gate and up."""
    opts = StackOpts(slots, int(down_first))
    _check(lib.uw_mlp_stack_forward_ex(layers, len(layers), M, _ptr(d_x), _ptr(d_y), _ptr(d_ws), ws_bytes,
                                       _stream(stream), None if decode_stream is None else _stream(decode_stream),
                                       ctypes.byref(opts)))


def mlp_stack_autotune(layers: ctypes.Array, M: int, d_x, d_y, d_ws, ws_bytes: int, stream=None, decode_stream=None,
                       slots: int = 2, down_first: bool = False, pipeline_mask: int = 0, reps: int = 0,
                       warmup: int = 0, max_passes: int = 0) -> StackTuneArgs:
    """uw_mlp_stack_autotune: coordinate descent over the layers' plans (written back into
    `layers`); returns the argument struct with opts, t_start_ms, t_ms, passes and trials."""
    a = StackTuneArgs(ctypes.cast(layers, ctypes.POINTER(MlpLayer)), len(layers), M, _ptr(d_x), _ptr(d_y), _ptr(d_ws),
                      ws_bytes, None if decode_stream is None else _stream(decode_stream),
                      StackOpts(slots, int(down_first)), pipeline_mask, reps, warmup, max_passes, 0.0, 0.0, 0, 0)
    _check(lib.uw_mlp_stack_autotune(ctypes.byref(a), _stream(stream)))
    return a


def stream_pair_create(decode_cus: int):
    """uw_stream_pair_create: (gemm_stream, decode_stream) handles on disjoint compute units,
    decode_cus of them for the decode stream. Wrap with torch.cuda.ExternalStream to use them
    from torch; release with stream_destroy."""
    g, d = ctypes.c_void_p(), ctypes.c_void_p()
    _check(lib.uw_stream_pair_create(decode_cus, ctypes.byref(g), ctypes.byref(d)))
    return g.value, d.value


def stream_destroy(handle: int) -> None:
    _check(lib.uw_stream_destroy(handle))


def stream_read(src, sink, nbytes: int | None = None, stream=None) -> None:
    """uw_stream_read: read the device tensor src (its first nbytes, default all) once with
    a plain streaming kernel; sink is a device tensor of at least 4 bytes it may modify."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    _check(lib.uw_stream_read(_ptr(src), n, _ptr(sink), _stream(stream)))


def stream_cu_count(stream=None) -> int:
    out = ctypes.c_int(0)
    _check(lib.uw_stream_cu_count(_stream(stream), ctypes.byref(out)))
    return out.value


# ---------------------------------------------------------------- bundle
def variant_by_name(name: str) -> int:
    return lib.uw_variant_by_name(name.encode())


def bundle_write(items, plans=()) -> np.ndarray:
    """uw_bundle_write: items = [(name, host blob)], plans = [dict(N, K, M, pipeline,
    split_k, t_ms, variant=<index or name, -1 / "" = default>)] -> the bundle bytes."""
    blobs = [np.ascontiguousarray(b, dtype=np.uint8) for _, b in items]
    arr = (BundleItem * max(1, len(items)))()
    for i, ((name, _), b) in enumerate(zip(items, blobs)):
        arr[i] = BundleItem(name.encode(), b.ctypes.data, b.size)
    parr = (BundlePlan * max(1, len(plans)))()
    for i, p in enumerate(plans):
        v = p.get("variant", "")
        vname = v if isinstance(v, str) else ("" if v < 0 else variant_name(v))
        parr[i] = BundlePlan(p["N"], p["K"], p["M"], p["pipeline"], p.get("split_k", 0), p.get("t_ms", 0.0),
                             vname.encode())
    need = ctypes.c_size_t(0)
    st = lib.uw_bundle_write(arr, len(items), parr, len(plans), None, ctypes.byref(need))
    if st != ENOSPACE:
        _check(st)
    out = np.empty(need.value, np.uint8)
    _check(lib.uw_bundle_write(arr, len(items), parr, len(plans), out.ctypes.data, ctypes.byref(need)))
    return out


def bundle_open(buf: np.ndarray, verify: bool = True) -> BundleInfo:
    info = BundleInfo()
    _check(lib.uw_bundle_open(buf.ctypes.data, buf.size, int(verify), ctypes.byref(info)))
    return info


def bundle_items(buf: np.ndarray) -> list:
    """[(name, offset, blob_bytes, Header)] of a bundle in host memory."""
    info = bundle_open(buf, verify=False)
    out = []
    for i in range(info.n_items):
        e = BundleEntry()
        _check(lib.uw_bundle_item_at(buf.ctypes.data, buf.size, i, ctypes.byref(e)))
        out.append((e.name.decode(), e.offset, e.blob_bytes, e.header))
    return out


def bundle_plans(buf: np.ndarray) -> list:
    """[dict(N, K, M, pipeline, split_k, t_ms, variant_name, variant)] of a bundle; variant
    is the index in this build (-1 for the default or a name it lacks)."""
    info = bundle_open(buf, verify=False)
    out = []
    for i in range(info.n_plans):
        p = BundlePlan()
        _check(lib.uw_bundle_plan_at(buf.ctypes.data, buf.size, i, ctypes.byref(p)))
        name = p.variant.decode()
        out.append({"N": p.N, "K": p.K, "M": p.M, "pipeline": p.pipeline, "split_k": p.split_k, "t_ms": p.t_ms,
                    "variant_name": name, "variant": variant_by_name(name) if name else -1})
    return out


def load_bundle(buf: np.ndarray, device="cuda", direct=True, verify: bool = True) -> dict:
    """Load every blob of a bundle into device memory (torch tensors) and, with direct,
    transcode each into its direct-palette plane with uw_prepare_direct (the load-time
    step of the direct pipeline). Returns {name: (Header, d_blob, d_direct or None)}."""
    import torch

    bundle_open(buf, verify=verify)
    out = {}
    for name, off, nbytes, h in bundle_items(buf):
        d_blob = torch.from_numpy(buf[off: off + nbytes]).to(device)
        d_direct = None
        if direct:
            d_direct = torch.empty(direct_plane_bytes(h), dtype=torch.uint8, device=device)
            prepare_direct(h, d_blob, d_direct)
        out[name] = (h, d_blob, d_direct)
    return out

