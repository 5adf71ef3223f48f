"""Python binding of librq.so, the MI355X (gfx950) KV-vector codec.

The functions below have the names and argument lists of include/rq.h and
only marshal arguments: device pointers may be given as torch tensors or
integers; every step of the codec runs in the HIP library.  The `Codec`
class adds record allocation with torch (device memory and streams only).

The library is loaded on first use, so importing the package (or its
CPU-only `workloads` module) touches no HIP code.  There is no fallback: if
librq.so is missing it is built in-tree (and the first call raises if that
fails); if it was built from other sources than those in csrc/ and include/
the first call raises instead of running stale code.
"""
import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librq.so")

RQ_OK, RQ_EINVAL, RQ_EUNSUPPORTED, RQ_ENOMEM, RQ_EHIP = 0, 1, 2, 3, 4
RQ_MSE, RQ_QJL, RQ_DENSE, RQ_POLAR = 0, 1, 2, 4
RQ_F32, RQ_F16 = 0, 1
RQ_SCORE_CHUNK = 4096

STATUS_NAMES = {0: "RQ_OK", 1: "RQ_EINVAL", 2: "RQ_EUNSUPPORTED", 3: "RQ_ENOMEM", 4: "RQ_EHIP"}

EXPORTS = ("rq_layout", "rq_host_params", "rq_host_quantizer", "rq_init", "rq_free", "rq_get_layout", "rq_get_params",
           "rq_quantize", "rq_dequantize", "rq_roundtrip", "rq_score", "rq_attend_workspace", "rq_attend",
           "rq_attend_noalloc",
           "tq_quantize", "tq_dequantize", "tq_roundtrip", "rq_cache_create", "rq_cache_free", "rq_cache_open",
           "rq_cache_close", "rq_cache_length", "rq_cache_free_pages", "rq_cache_append", "rq_cache_read",
           "rq_cache_attend_workspace", "rq_cache_attend",
           "rq_cache_append_layers", "rq_cache_attend_layers_workspace", "rq_cache_attend_layers", "pq_quantize", "pq_dequantize", "pq_roundtrip", "pq_score",
           "rq_outlier_channels", "rq_quantize_outliers", "rq_dequantize_outliers", "rq_score_outliers",
           "rq_bench_copy", "rq_last_error", "rq_version")


class RQError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class Layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("d", "bits", "mse_bits", "mode", "n_coords", "n_groups", "levels",
                                                "code_words", "sign_words", "record_bytes")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class ParamsHost(ctypes.Structure):
    _fields_ = [("rotors", ctypes.c_void_p), ("rotmats", ctypes.c_void_p), ("centroids", ctypes.c_void_p),
                ("boundaries", ctypes.c_void_p), ("pi", ctypes.c_void_p), ("s", ctypes.c_void_p)]


def _load():
    from .build import build, hip_runtime_dir, source_digest, stamp_path
    if not os.path.exists(LIB_PATH):
        build()
    try:
        with open(stamp_path()) as f:
            built_from = f.read().strip()
    except OSError:
        built_from = None
    if built_from != source_digest():
        raise ImportError(f"{LIB_PATH} was built from other sources than those in csrc/ and include/ "
                          "(or carries no source stamp); rebuild it (__graft_entry__.build())")
    # One HIP runtime per process: load the libamdhip64 that torch uses before
    # librq.so, so that librq.so's dependency resolves to that same runtime
    # (torch owns the device memory and streams handed to the library).
    hip = os.path.join(hip_runtime_dir(), "libamdhip64.so")
    if os.path.exists(hip):
        ctypes.CDLL(hip, mode=ctypes.RTLD_GLOBAL)
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64, U64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_uint64
    sig = {
        "rq_layout": ([I, I, I, ctypes.POINTER(Layout)], I),
        "rq_host_params": ([I, I, U64, I, ctypes.POINTER(ParamsHost)], I),
        "rq_host_quantizer": ([I, I, I, P, P], I),
        "rq_init": ([I, I, U64, I, ctypes.POINTER(P)], I),
        "rq_free": ([P], None),
        "rq_get_layout": ([P, ctypes.POINTER(Layout)], I),
        "rq_get_params": ([P, ctypes.POINTER(ParamsHost)], I),
        "rq_quantize": ([P, P, I, I64, I64, P, P, P, P, P], I),
        "rq_dequantize": ([P, P, P, P, P, I64, P, I, I64, P], I),
        "rq_roundtrip": ([P, P, I, I64, I64, P, P, P, P, P, I, I64, P], I),
        "rq_score": ([P, P, I, I, P, P, P, P, I64, I64, P, I64, P], I),
        "rq_attend_workspace": ([I, I, I64], I64),
        "rq_attend": ([P, P, P, I, I, P, P, P, P, P, P, P, P, I64, I64, ctypes.c_float, P, I64, P, I64, P], I),
        "rq_attend_noalloc": ([P, P, P, I, I, P, P, P, P, P, P, P, P, I64, I64, ctypes.c_float, P, I64, P], I),
        "rq_cache_create": ([P, P, I, I, I, I64, I64, ctypes.POINTER(P)], I),
        "rq_cache_free": ([P], None),
        "rq_cache_open": ([P, I64, ctypes.POINTER(I)], I),
        "rq_cache_close": ([P, I], I),
        "rq_cache_length": ([P, I, I], I64),
        "rq_cache_free_pages": ([P], I64),
        "rq_cache_append": ([P, I, I, P, P, I, I64, I64, P], I),
        "rq_cache_read": ([P, I, I, I, P, P, P, P, P], I),
        "rq_cache_attend_workspace": ([P, I, I64], I64),
        "rq_cache_attend": ([P, I, I, P, I, ctypes.c_float, P, P, P, I64, P, I64, P], I),
        "rq_cache_append_layers": ([P, I, I, I, P, P, I, I64, I64, P], I),
        "rq_cache_attend_layers_workspace": ([P, I, I, I64], I64),
        "rq_cache_attend_layers": ([P, I, I, I, P, I, ctypes.c_float, P, P, P, I64, P, I64, P], I),
        "tq_quantize": ([P, P, I, I64, I64, P, P, P, P, P], I),
        "tq_dequantize": ([P, P, P, P, P, I64, P, I, I64, P], I),
        "tq_roundtrip": ([P, P, I, I64, I64, P, P, P, P, P, I, I64, P], I),
        "pq_quantize": ([P, P, I, I64, I64, P, P], I),
        "pq_dequantize": ([P, P, I64, P, I, I64, P], I),
        "pq_roundtrip": ([P, P, I, I64, I64, P, P, I, I64, P], I),
        "pq_score": ([P, P, I, I, P, I64, I64, P, I64, P], I),
        "rq_outlier_channels": ([P, I, I64, I64, I64, I, P, P], I),
        "rq_quantize_outliers": ([P, P, I, I64, I64, I64, I, P, P, P, P, P, P], I),
        "rq_dequantize_outliers": ([P, P, P, P, P, I64, I64, I, P, P, I, I64, P], I),
        "rq_score_outliers": ([P, P, I, I, P, P, P, P, I, P, I64, I64, P, I64, P], I),
        "rq_bench_copy": ([P, P, I64, P], I),
        "rq_last_error": ([], ctypes.c_char_p),
        "rq_version": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        try:
            f = getattr(lib, name)
        except AttributeError:
            raise ImportError(f"{LIB_PATH} does not export {name}: the library is older than its sources; "
                              "rebuild it (__graft_entry__.build())") from None
        f.argtypes = args
        f.restype = res
    return lib


class _LazyLib:
    """The ctypes handle of librq.so, loaded (and checked) on first use."""
    _handle = None

    def __getattr__(self, name):
        if _LazyLib._handle is None:
            _LazyLib._handle = _load()
        return getattr(_LazyLib._handle, name)


_lib = _LazyLib()


def lib():
    """The loaded librq.so (ctypes.CDLL), loading it on the first call."""
    if _LazyLib._handle is None:
        _LazyLib._handle = _load()
    return _LazyLib._handle


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _stream(stream):
    if stream is None:
        try:
            import torch
            if torch.cuda.is_available():
                return torch.cuda.current_stream().cuda_stream
        except ImportError:
            pass
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc):
    if rc != RQ_OK:
        raise RQError(rc, rq_last_error())
    return rc


# ----------------------------------------------------------------- C ABI --
def rq_last_error():
    return _lib.rq_last_error().decode()


def rq_version():
    return _lib.rq_version().decode()


def rq_layout(d, bits, mode):
    out = Layout()
    _check(_lib.rq_layout(d, bits, mode, ctypes.byref(out)))
    return out.as_dict()


def rq_host_params(d, bits, seed, mode):
    """Host parameter tables as numpy arrays (no GPU involved)."""
    lay = rq_layout(d, bits, mode)
    arrays = _param_arrays(lay, mode)
    p = ParamsHost(*[arrays[k].ctypes.data if k in arrays else None for k in
                     ("rotors", "rotmats", "centroids", "boundaries", "pi", "s")])
    _check(_lib.rq_host_params(d, bits, seed, mode, ctypes.byref(p)))
    return arrays


def rq_host_quantizer(d, bits, mode):
    """(bias, table [256, 4] uint32) of the kernels' slot lookup (host only)."""
    bias = ctypes.c_float()
    table = np.zeros((256, 4), np.uint32)
    _check(_lib.rq_host_quantizer(d, bits, mode, ctypes.byref(bias), table.ctypes.data))
    return float(bias.value), table


def _param_arrays(lay, mode):
    d, g, levels = lay["d"], lay["n_groups"], lay["levels"]
    if mode & RQ_POLAR:
        return {"centroids": np.zeros(28, np.float32), "boundaries": np.zeros(24, np.float32),
                "pi": np.zeros((d, d), np.float32)}
    a = {"centroids": np.zeros(levels, np.float32), "boundaries": np.zeros(levels - 1, np.float32)}
    if not mode & RQ_DENSE:
        a["rotors"] = np.zeros((g, 4), np.float32)
        a["rotmats"] = np.zeros((g, 3, 3), np.float32)
    else:
        a["pi"] = np.zeros((d, d), np.float32)
    if mode & RQ_QJL:
        a["s"] = np.zeros((d, d), np.uint16)
    return a


def rq_init(d, bits, seed, mode):
    h = ctypes.c_void_p()
    _check(_lib.rq_init(d, bits, seed, mode, ctypes.byref(h)))
    return h.value


def rq_free(ctx):
    _lib.rq_free(ctx)


def rq_get_layout(ctx):
    out = Layout()
    _check(_lib.rq_get_layout(ctx, ctypes.byref(out)))
    return out.as_dict()


def rq_get_params(ctx):
    lay = rq_get_layout(ctx)
    arrays = _param_arrays(lay, lay["mode"])
    p = ParamsHost(*[arrays[k].ctypes.data if k in arrays else None for k in
                     ("rotors", "rotmats", "centroids", "boundaries", "pi", "s")])
    _check(_lib.rq_get_params(ctx, ctypes.byref(p)))
    return arrays


def _quant(fn, ctx, x, x_dtype, n, ldx, codes, norms, signs, rnorms, stream):
    return _check(fn(ctx, _ptr(x), x_dtype, n, ldx, _ptr(codes), _ptr(norms), _ptr(signs), _ptr(rnorms),
                     _stream(stream)))


def _dequant(fn, ctx, codes, norms, signs, rnorms, n, y, y_dtype, ldy, stream):
    return _check(fn(ctx, _ptr(codes), _ptr(norms), _ptr(signs), _ptr(rnorms), n, _ptr(y), y_dtype, ldy,
                     _stream(stream)))


def _round(fn, ctx, x, x_dtype, n, ldx, codes, norms, signs, rnorms, y, y_dtype, ldy, stream):
    return _check(fn(ctx, _ptr(x), x_dtype, n, ldx, _ptr(codes), _ptr(norms), _ptr(signs), _ptr(rnorms), _ptr(y),
                     y_dtype, ldy, _stream(stream)))


def rq_quantize(ctx, x, x_dtype, n, ldx, codes, norms, signs=None, rnorms=None, stream=None):
    return _quant(_lib.rq_quantize, ctx, x, x_dtype, n, ldx, codes, norms, signs, rnorms, stream)


def tq_quantize(ctx, x, x_dtype, n, ldx, codes, norms, signs=None, rnorms=None, stream=None):
    return _quant(_lib.tq_quantize, ctx, x, x_dtype, n, ldx, codes, norms, signs, rnorms, stream)


def rq_dequantize(ctx, codes, norms, signs, rnorms, n, y, y_dtype, ldy, stream=None):
    return _dequant(_lib.rq_dequantize, ctx, codes, norms, signs, rnorms, n, y, y_dtype, ldy, stream)


def tq_dequantize(ctx, codes, norms, signs, rnorms, n, y, y_dtype, ldy, stream=None):
    return _dequant(_lib.tq_dequantize, ctx, codes, norms, signs, rnorms, n, y, y_dtype, ldy, stream)


def rq_roundtrip(ctx, x, x_dtype, n, ldx, codes, norms, signs, rnorms, y, y_dtype, ldy, stream=None):
    return _round(_lib.rq_roundtrip, ctx, x, x_dtype, n, ldx, codes, norms, signs, rnorms, y, y_dtype, ldy, stream)


def tq_roundtrip(ctx, x, x_dtype, n, ldx, codes, norms, signs, rnorms, y, y_dtype, ldy, stream=None):
    return _round(_lib.tq_roundtrip, ctx, x, x_dtype, n, ldx, codes, norms, signs, rnorms, y, y_dtype, ldy, stream)


def rq_score(ctx, q, hq, group, codes, norms, signs, rnorms, t, kv_stride, scores, ld_scores, stream=None):
    return _check(_lib.rq_score(ctx, _ptr(q), hq, group, _ptr(codes), _ptr(norms), _ptr(signs), _ptr(rnorms), t,
                                kv_stride, _ptr(scores), ld_scores, _stream(stream)))


def rq_attend_workspace(hq, group, t):
    return _lib.rq_attend_workspace(hq, group, t)


def rq_attend(kctx, vctx, q, hq, group, kcodes, knorms, ksigns, krnorms, vcodes, vnorms, vsigns, vrnorms, t,
              kv_stride, scale, workspace, workspace_bytes, out, ld_out, stream=None):
    return _check(_lib.rq_attend(kctx, vctx, _ptr(q), hq, group, _ptr(kcodes), _ptr(knorms), _ptr(ksigns),
                                 _ptr(krnorms), _ptr(vcodes), _ptr(vnorms), _ptr(vsigns), _ptr(vrnorms), t, kv_stride,
                                 float(scale), _ptr(workspace), workspace_bytes, _ptr(out), ld_out, _stream(stream)))


RQ_MAX_OUTLIERS = 16


def rq_outlier_channels(x, x_dtype, heads, head_rows, ldx, k, chans, stream=None):
    return _check(_lib.rq_outlier_channels(_ptr(x), x_dtype, heads, head_rows, ldx, k, _ptr(chans), _stream(stream)))


def rq_quantize_outliers(ctx, x, x_dtype, n, ldx, head_rows, k, chans, norms, signs, rnorms, outliers, stream=None):
    return _check(_lib.rq_quantize_outliers(ctx, _ptr(x), x_dtype, n, ldx, head_rows, k, _ptr(chans), _ptr(norms),
                                            _ptr(signs), _ptr(rnorms), _ptr(outliers), _stream(stream)))


def rq_dequantize_outliers(ctx, norms, signs, rnorms, outliers, n, head_rows, k, chans, y, y_dtype, ldy, stream=None):
    return _check(_lib.rq_dequantize_outliers(ctx, _ptr(norms), _ptr(signs), _ptr(rnorms), _ptr(outliers), n,
                                              head_rows, k, _ptr(chans), _ptr(y), y_dtype, ldy, _stream(stream)))


def rq_score_outliers(ctx, q, hq, group, norms, signs, rnorms, outliers, k, chans, t, kv_stride, scores, ld_scores,
                      stream=None):
    return _check(_lib.rq_score_outliers(ctx, _ptr(q), hq, group, _ptr(norms), _ptr(signs), _ptr(rnorms),
                                         _ptr(outliers), k, _ptr(chans), t, kv_stride, _ptr(scores), ld_scores,
                                         _stream(stream)))


def rq_bench_copy(src, dst, nbytes, stream=None):
    return _check(_lib.rq_bench_copy(_ptr(src), _ptr(dst), nbytes, _stream(stream)))


RQ_ATTEND_NOALLOC_BYTES = 64 << 20


def rq_attend_noalloc(kctx, vctx, q, hq, group, kcodes, knorms, ksigns, krnorms, vcodes, vnorms, vsigns, vrnorms, t,
                      kv_stride, scale, out, ld_out, stream=None):
    return _check(_lib.rq_attend_noalloc(kctx, vctx, _ptr(q), hq, group, _ptr(kcodes), _ptr(knorms), _ptr(ksigns),
                                         _ptr(krnorms), _ptr(vcodes), _ptr(vnorms), _ptr(vsigns), _ptr(vrnorms), t,
                                         kv_stride, float(scale), _ptr(out), ld_out, _stream(stream)))


def pq_quantize(ctx, x, x_dtype, n, ldx, words, stream=None):
    return _check(_lib.pq_quantize(ctx, _ptr(x), x_dtype, n, ldx, _ptr(words), _stream(stream)))


def pq_dequantize(ctx, words, n, y, y_dtype, ldy, stream=None):
    return _check(_lib.pq_dequantize(ctx, _ptr(words), n, _ptr(y), y_dtype, ldy, _stream(stream)))


def pq_roundtrip(ctx, x, x_dtype, n, ldx, words, y, y_dtype, ldy, stream=None):
    return _check(_lib.pq_roundtrip(ctx, _ptr(x), x_dtype, n, ldx, _ptr(words), _ptr(y), y_dtype, ldy,
                                    _stream(stream)))


def pq_score(ctx, q, hq, group, words, t, kv_stride, scores, ld_scores, stream=None):
    return _check(_lib.pq_score(ctx, _ptr(q), hq, group, _ptr(words), t, kv_stride, _ptr(scores), ld_scores,
                                _stream(stream)))


# ----------------------------------------------------------- convenience --
class Record:
    """Device record arrays of n vectors (torch tensors)."""

    def __init__(self, codes, norms, signs=None, rnorms=None):
        self.codes, self.norms, self.signs, self.rnorms = codes, norms, signs, rnorms

    @property
    def n(self):
        return self.codes.shape[0]

    def host(self):
        """(codes uint32, norms uint16, signs uint32 | None, rnorms uint16 | None) as numpy."""
        def u(t, dt):
            return None if t is None else t.cpu().numpy().view(dt)
        return u(self.codes, np.uint32), u(self.norms, np.uint16), u(self.signs, np.uint32), u(self.rnorms, np.uint16)


class Codec:
    """A session plus torch-allocated outputs.  `dense` selects TurboQuant."""

    def __init__(self, bits=3, seed=0, mode=RQ_MSE, d=128):
        import torch
        self.torch = torch
        self.mode = mode
        self.dense = bool(mode & RQ_DENSE)
        self.ctx = rq_init(d, bits, seed, mode)
        self.layout = rq_get_layout(self.ctx)

    def close(self):
        if self.ctx:
            rq_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def params(self):
        return rq_get_params(self.ctx)

    def alloc_record(self, n, device="cuda"):
        t = self.torch
        lay = self.layout
        codes = t.zeros((n, lay["code_words"]), dtype=t.int32, device=device)
        norms = t.zeros((n,), dtype=t.int16, device=device)
        signs = rnorms = None
        if lay["sign_words"]:
            signs = t.zeros((n, lay["sign_words"]), dtype=t.int32, device=device)
            rnorms = t.zeros((n,), dtype=t.int16, device=device)
        return Record(codes, norms, signs, rnorms)

    def _dt(self, tensor):
        t = self.torch
        if tensor.dtype == t.float16:
            return RQ_F16
        if tensor.dtype == t.float32:
            return RQ_F32
        raise TypeError("vectors must be float16 or float32")

    def quantize(self, x, rec=None, stream=None):
        n = x.shape[0]
        rec = rec or self.alloc_record(n, x.device)
        fn = tq_quantize if self.dense else rq_quantize
        fn(self.ctx, x, self._dt(x), n, x.stride(0), rec.codes, rec.norms, rec.signs, rec.rnorms, stream)
        return rec

    def dequantize(self, rec, dtype=None, out=None, stream=None):
        t = self.torch
        n = rec.n
        if out is None:
            out = t.empty((n, self.layout["d"]), dtype=dtype or t.float32, device=rec.codes.device)
        fn = tq_dequantize if self.dense else rq_dequantize
        fn(self.ctx, rec.codes, rec.norms, rec.signs, rec.rnorms, n, out, self._dt(out), out.stride(0), stream)
        return out

    def roundtrip(self, x, dtype=None, rec=None, out=None, stream=None):
        t = self.torch
        n = x.shape[0]
        rec = rec or self.alloc_record(n, x.device)
        if out is None:
            out = t.empty((n, self.layout["d"]), dtype=dtype or x.dtype, device=x.device)
        fn = tq_roundtrip if self.dense else rq_roundtrip
        fn(self.ctx, x, self._dt(x), n, x.stride(0), rec.codes, rec.norms, rec.signs, rec.rnorms, out,
           self._dt(out), out.stride(0), stream)
        return rec, out

    def score(self, q, rec, group, t, kv_stride=None, out=None, stream=None):
        th = self.torch
        hq = q.shape[0]
        kv_stride = t if kv_stride is None else kv_stride
        if out is None:
            out = th.empty((hq, t), dtype=th.float32, device=q.device)
        rq_score(self.ctx, q, hq, group, rec.codes, rec.norms, rec.signs, rec.rnorms, t, kv_stride, out,
                 out.stride(0), stream)
        return out


class PolarCodec:
    """A PolarQuant session (RQ_POLAR, bits = 4) plus torch-allocated
    outputs.  Records are [n, 16] int32 tensors (16 u32 words per vector)."""

    def __init__(self, seed=0, d=128):
        import torch
        self.torch = torch
        self.ctx = rq_init(d, 4, seed, RQ_POLAR)
        self.layout = rq_get_layout(self.ctx)

    def close(self):
        if self.ctx:
            rq_free(self.ctx)
            self.ctx = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def params(self):
        return rq_get_params(self.ctx)

    def alloc_words(self, n, device="cuda"):
        return self.torch.zeros((n, self.layout["code_words"]), dtype=self.torch.int32, device=device)

    def _dt(self, tensor):
        t = self.torch
        if tensor.dtype == t.float16:
            return RQ_F16
        if tensor.dtype == t.float32:
            return RQ_F32
        raise TypeError("vectors must be float16 or float32")

    def quantize(self, x, words=None, stream=None):
        n = x.shape[0]
        words = self.alloc_words(n, x.device) if words is None else words
        pq_quantize(self.ctx, x, self._dt(x), n, x.stride(0), words, stream)
        return words

    def dequantize(self, words, dtype=None, out=None, stream=None):
        n = words.shape[0]
        if out is None:
            out = self.torch.empty((n, self.layout["d"]), dtype=dtype or self.torch.float32, device=words.device)
        pq_dequantize(self.ctx, words, n, out, self._dt(out), out.stride(0), stream)
        return out

    def roundtrip(self, x, dtype=None, words=None, out=None, stream=None):
        n = x.shape[0]
        words = self.alloc_words(n, x.device) if words is None else words
        if out is None:
            out = self.torch.empty((n, self.layout["d"]), dtype=dtype or x.dtype, device=x.device)
        pq_roundtrip(self.ctx, x, self._dt(x), n, x.stride(0), words, out, self._dt(out), out.stride(0), stream)
        return words, out

    def score(self, q, words, group, t, kv_stride=None, out=None, stream=None):
        hq = q.shape[0]
        kv_stride = t if kv_stride is None else kv_stride
        if out is None:
            out = self.torch.empty((hq, t), dtype=self.torch.float32, device=q.device)
        pq_score(self.ctx, q, hq, group, words, t, kv_stride, out, out.stride(0), stream)
        return out


def attend(kcodec, vcodec, q, krec, vrec, group, t, kv_stride=None, scale=None, out=None, workspace=None,
           stream=None):
    """softmax(scale * q.k) . V over compressed keys (kcodec's records, or a
    PolarCodec's word tensor) and values (vcodec's records, or a PolarCodec's
    word tensor); scale defaults
    to 1/sqrt(128).  Returns
    [hq, 128] fp32.  The workspace (torch uint8 tensor) is allocated when not
    given; pass one of rq_attend_workspace(hq, group, t) bytes to avoid that."""
    import torch
    hq = q.shape[0]
    kv_stride = t if kv_stride is None else kv_stride
    scale = 1.0 / math.sqrt(kcodec.layout["d"]) if scale is None else scale
    need = rq_attend_workspace(hq, group, t)
    if need < 0:
        raise RQError(RQ_EINVAL, "rq_attend_workspace: invalid sizes")
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    base = workspace.data_ptr()
    ws = base + ((-base) % 256)
    avail = workspace.numel() - (ws - base)
    if out is None:
        out = torch.empty((hq, kcodec.layout["d"]), dtype=torch.float32, device=q.device)
    if isinstance(kcodec, PolarCodec):          # krec: the [n, 16] word records
        kparts = (krec, None, None, None)
    else:
        kparts = (krec.codes, krec.norms, krec.signs, krec.rnorms)
    if isinstance(vcodec, PolarCodec):          # vrec: the [n, 16] word records
        vparts = (vrec, None, None, None)
    else:
        vparts = (vrec.codes, vrec.norms, vrec.signs, vrec.rnorms)
    rq_attend(kcodec.ctx, vcodec.ctx, q, hq, group, *kparts, *vparts, t, kv_stride, scale, ws, avail, out,
              out.stride(0), stream)
    return out


class Cache:
    """Paged compressed KV cache (rq_cache_*): keys in kcodec's format, values
    in vcodec's, pages of `page_tokens` tokens per (layer, KV head)."""

    def __init__(self, kcodec, vcodec, layers, kv_heads, page_tokens=256, max_pages=1024, stage_tokens=65536):
        self.kc, self.vc = kcodec, vcodec
        self.layers, self.kv_heads = layers, kv_heads
        h = ctypes.c_void_p()
        _check(_lib.rq_cache_create(kcodec.ctx, vcodec.ctx, layers, kv_heads, page_tokens, max_pages, stage_tokens,
                                    ctypes.byref(h)))
        self.h = h

    def close_cache(self):
        if self.h:
            _lib.rq_cache_free(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close_cache()
        except Exception:
            pass

    def open(self, max_tokens):
        sid = ctypes.c_int()
        _check(_lib.rq_cache_open(self.h, max_tokens, ctypes.byref(sid)))
        return sid.value

    def close(self, seq):
        _check(_lib.rq_cache_close(self.h, seq))

    def length(self, seq, layer):
        return _lib.rq_cache_length(self.h, seq, layer)

    def free_pages(self):
        return _lib.rq_cache_free_pages(self.h)

    def append(self, seq, layer, k, v, stream=None):
        """k, v: [kv_heads, n, 128] fp16 or fp32 (rows of pitch stride(1))."""
        dt = self.kc._dt(k)
        _check(_lib.rq_cache_append(self.h, seq, layer, _ptr(k), _ptr(v), dt, k.shape[1], k.stride(1),
                                    _stream(stream)))

    def read(self, seq, layer, which, stream=None):
        """Dense copy [kv_heads * length] of the cached key (0) or value (1) records."""
        codec = self.vc if which else self.kc
        rec = codec.alloc_record(self.kv_heads * self.length(seq, layer))
        _check(_lib.rq_cache_read(self.h, seq, layer, which, _ptr(rec.codes), _ptr(rec.norms), _ptr(rec.signs),
                                  _ptr(rec.rnorms), _stream(stream)))
        return rec

    def append_layers(self, seq, layer0, k, v, stream=None):
        """k, v: [nlayers, kv_heads, n, 128] fp16 or fp32 (rows of pitch stride(2)) for
        layers layer0 .. layer0 + nlayers - 1, in one call."""
        dt = self.kc._dt(k)
        _check(_lib.rq_cache_append_layers(self.h, seq, layer0, k.shape[0], _ptr(k), _ptr(v), dt, k.shape[2],
                                           k.stride(2), _stream(stream)))

    def attend_layers(self, seq, layer0, q, scale=None, k_cur=None, v_cur=None, out=None, workspace=None,
                      stream=None):
        """q: [nlayers, hq, 128] fp32; k_cur, v_cur: [nlayers, kv_heads, 128] fp32.
        Returns [nlayers * hq, 128] fp32."""
        import torch
        nl, hq = q.shape[0], q.shape[1]
        scale = 1.0 / math.sqrt(128) if scale is None else scale
        t = self.length(seq, layer0)
        need = _lib.rq_cache_attend_layers_workspace(self.h, nl, hq, t)
        if need < 0:
            raise RQError(RQ_EINVAL, "rq_cache_attend_layers_workspace: invalid sizes")
        if workspace is None:
            workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
        base = workspace.data_ptr()
        ws = base + ((-base) % 256)
        if out is None:
            out = torch.empty((nl * hq, 128), dtype=torch.float32, device=q.device)
        _check(_lib.rq_cache_attend_layers(self.h, seq, layer0, nl, _ptr(q), hq, float(scale), _ptr(k_cur),
                                           _ptr(v_cur), ws, workspace.numel() - (ws - base), _ptr(out),
                                           out.stride(0), _stream(stream)))
        return out

    def attend(self, seq, layer, q, scale=None, k_cur=None, v_cur=None, out=None, workspace=None, stream=None):
        import torch
        hq = q.shape[0]
        scale = 1.0 / math.sqrt(128) if scale is None else scale
        t = self.length(seq, layer)
        need = _lib.rq_cache_attend_workspace(self.h, hq, t)
        if need < 0:
            raise RQError(RQ_EINVAL, "rq_cache_attend_workspace: invalid sizes")
        if workspace is None:
            workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
        base = workspace.data_ptr()
        ws = base + ((-base) % 256)
        if out is None:
            out = torch.empty((hq, 128), dtype=torch.float32, device=q.device)
        _check(_lib.rq_cache_attend(self.h, seq, layer, _ptr(q), hq, float(scale), _ptr(k_cur), _ptr(v_cur), ws,
                                    workspace.numel() - (ws - base), _ptr(out), out.stride(0), _stream(stream)))
        return out
