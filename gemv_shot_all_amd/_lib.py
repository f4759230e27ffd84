"""ctypes binding of libgsa.  Argument marshalling only: every step of the
operation runs in the library's HIP kernels.  Names mirror include/gsa.h."""
import ctypes
import os

LIBRARY = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgsa.so")

# Values of include/gsa.h (tests check that these agree with the header).
GSA_OK = 0
GSA_EINVAL = -1
GSA_ENOMEM = -2
GSA_EHIP = -3
GSA_ETIMEOUT = -4
GSA_ESTATE = -5
GSA_ESPLIT = -6
GSA_FLAG_PUBLISHED = 0xFFFFFFFF
GSA_FLAG_TILE_ROWS = 4
GSA_FLAG_GROUP_TILES = 4
GSA_FLAG_GROUP_WORDS = 32
GSA_MOE_TILE_ROWS = 16
GSA_PAD_HEADER_WORDS = 16
GSA_MAX_W = 8
GSA_MAX_B = 16
GSA_MAX_X_LDS_BYTES = 128 * 1024
GSA_DTYPE_F32 = 0
GSA_DTYPE_BF16 = 1
GSA_MOE_MAX_TOKENS = 256
GSA_MOE_MAX_F = 4088

EXPORTS = ("gsa_symm_alloc", "gsa_symm_alloc_dtype", "gsa_symm_free", "gsa_symm_slots", "gsa_symm_signal_pad",
           "gsa_symm_gathered", "gsa_signal_pad_row_stride", "gsa_signal_pad_reset",
           "gsa_gemv_allreduce", "gsa_gemv_allreduce_dtype", "gsa_gemv_allreduce_two_shot",
           "gsa_gemv_allreduce_rmsnorm", "gsa_gemv_allreduce_rmsnorm_noalloc", "gsa_bias_rmsnorm",
           "gsa_peer_publish", "gsa_signal_pad_status", "gsa_set_wait_timeout_us",
           "gsa_strerror",
           "gsa_a2a_pad_words", "gsa_a2a_alloc", "gsa_a2a_free", "gsa_a2a_buffers",
           "gsa_a2a_signal_pads", "gsa_a2a_reset", "gsa_moe_gemm_all_to_all", "gsa_a2a_status")


class gsa_epilogue(ctypes.Structure):
    """struct gsa_epilogue of include/gsa.h."""
    _fields_ = [("bias", ctypes.c_void_p), ("rms_weight", ctypes.c_void_p),
                ("eps", ctypes.c_float), ("y_dtype", ctypes.c_int), ("y", ctypes.c_void_p),
                ("inv_rms", ctypes.c_void_p)]


class GsaError(RuntimeError):
    """A GSA_E* code returned by the library."""

    def __init__(self, code, what):
        self.code = code
        super().__init__(f"{what}: {_strerror(code)} ({code})")


_lib = None


def lib():
    """The loaded library.  Raises if it has not been built: there is no
    fallback implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIBRARY):
            raise ImportError(
                f"{LIBRARY} is missing; build it with gemv_shot_all_amd.build.build() "
                "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIBRARY)
        vp, i64, u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
        ci = ctypes.c_int
        L.gsa_symm_alloc.argtypes = [ci, i64, ci, ctypes.POINTER(vp)]
        L.gsa_symm_alloc.restype = ci
        L.gsa_symm_alloc_dtype.argtypes = [ci, i64, ci, ci, ctypes.POINTER(vp)]
        L.gsa_symm_alloc_dtype.restype = ci
        L.gsa_symm_free.argtypes = [vp]
        L.gsa_symm_free.restype = ci
        L.gsa_symm_slots.argtypes = [vp]
        L.gsa_symm_slots.restype = vp
        L.gsa_symm_signal_pad.argtypes = [vp]
        L.gsa_symm_signal_pad.restype = vp
        L.gsa_symm_gathered.argtypes = [vp]
        L.gsa_symm_gathered.restype = vp
        L.gsa_signal_pad_row_stride.argtypes = [i64]
        L.gsa_signal_pad_row_stride.restype = i64
        L.gsa_signal_pad_reset.argtypes = [vp, ci, i64, u32, vp]
        L.gsa_signal_pad_reset.restype = ci
        L.gsa_gemv_allreduce.argtypes = [vp, vp, vp, vp, vp, ci, ci, i64, i64, ci, vp]
        L.gsa_gemv_allreduce.restype = ci
        L.gsa_gemv_allreduce_dtype.argtypes = [vp, vp, vp, vp, vp, ci, ci, ci, i64, i64, ci, vp]
        L.gsa_gemv_allreduce_dtype.restype = ci
        L.gsa_gemv_allreduce_two_shot.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, i64, i64, ci,
                                                  vp]
        L.gsa_gemv_allreduce_two_shot.restype = ci
        L.gsa_gemv_allreduce_rmsnorm.argtypes = [vp, vp, vp, vp, vp, ci, ci, i64, i64, ci,
                                                 ctypes.POINTER(gsa_epilogue), vp]
        L.gsa_gemv_allreduce_rmsnorm.restype = ci
        L.gsa_gemv_allreduce_rmsnorm_noalloc.argtypes = L.gsa_gemv_allreduce_rmsnorm.argtypes
        L.gsa_gemv_allreduce_rmsnorm_noalloc.restype = ci
        L.gsa_bias_rmsnorm.argtypes = [vp, i64, ci, ctypes.POINTER(gsa_epilogue), vp]
        L.gsa_bias_rmsnorm.restype = ci
        L.gsa_peer_publish.argtypes = [vp, vp, vp, ci, ci, i64, ci, u32, u32, vp]
        L.gsa_peer_publish.restype = ci
        L.gsa_signal_pad_status.argtypes = [vp, vp, ctypes.POINTER(ci),
                                            ctypes.POINTER(i64), ctypes.POINTER(ci)]
        L.gsa_signal_pad_status.restype = ci
        L.gsa_set_wait_timeout_us.argtypes = [u32]
        L.gsa_set_wait_timeout_us.restype = ci
        L.gsa_strerror.argtypes = [ci]
        L.gsa_strerror.restype = ctypes.c_char_p
        L.gsa_a2a_pad_words.argtypes = [ci, ci, i64]
        L.gsa_a2a_pad_words.restype = i64
        L.gsa_a2a_alloc.argtypes = [ci, ci, i64, i64, ctypes.POINTER(vp)]
        L.gsa_a2a_alloc.restype = ci
        L.gsa_a2a_free.argtypes = [vp]
        L.gsa_a2a_free.restype = ci
        L.gsa_a2a_buffers.argtypes = [vp]
        L.gsa_a2a_buffers.restype = vp
        L.gsa_a2a_signal_pads.argtypes = [vp]
        L.gsa_a2a_signal_pads.restype = vp
        L.gsa_a2a_reset.argtypes = [vp, ci, ci, i64, u32, vp]
        L.gsa_a2a_reset.restype = ci
        L.gsa_moe_gemm_all_to_all.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, i64, i64, i64,
                                              i64, vp]
        L.gsa_moe_gemm_all_to_all.restype = ci
        L.gsa_a2a_status.argtypes = [vp, ci, vp, ctypes.POINTER(ci), ctypes.POINTER(i64),
                                     ctypes.POINTER(ci)]
        L.gsa_a2a_status.restype = ci
        _lib = L
    return _lib


def _strerror(code):
    try:
        return lib().gsa_strerror(code).decode()
    except ImportError:
        return "library not loaded"


def _check(rc, what):
    if rc != GSA_OK:
        raise GsaError(rc, what)


def _ptr(t):
    """Device address of a torch tensor (must be contiguous) or a raw int."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream):
    """hipStream_t of `stream`: None means torch's current stream."""
    if isinstance(stream, int):
        return stream
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def gsa_symm_alloc(W, N, B):
    h = ctypes.c_void_p()
    _check(lib().gsa_symm_alloc(W, N, B, ctypes.byref(h)), "gsa_symm_alloc")
    return h.value


def gsa_symm_alloc_dtype(W, N, B, slot_dtype):
    h = ctypes.c_void_p()
    _check(lib().gsa_symm_alloc_dtype(W, N, B, slot_dtype, ctypes.byref(h)),
           "gsa_symm_alloc_dtype")
    return h.value


def gsa_symm_free(h):
    _check(lib().gsa_symm_free(h), "gsa_symm_free")


def gsa_symm_slots(h):
    p = lib().gsa_symm_slots(h)
    if not p:
        raise GsaError(GSA_EINVAL, "gsa_symm_slots")
    return p


def gsa_symm_signal_pad(h):
    p = lib().gsa_symm_signal_pad(h)
    if not p:
        raise GsaError(GSA_EINVAL, "gsa_symm_signal_pad")
    return p


def gsa_symm_gathered(h):
    p = lib().gsa_symm_gathered(h)
    if not p:
        raise GsaError(GSA_EINVAL, "gsa_symm_gathered")
    return p


def gsa_signal_pad_row_stride(N):
    return lib().gsa_signal_pad_row_stride(N)


def flag_word(t):
    """Word of flag tile t (int or numpy array) within a rank's row of the
    pad: groups of GSA_FLAG_GROUP_TILES flags, GSA_FLAG_GROUP_WORDS apart."""
    return (t // GSA_FLAG_GROUP_TILES) * GSA_FLAG_GROUP_WORDS + t % GSA_FLAG_GROUP_TILES


def gsa_signal_pad_reset(pad, W, N, published_mask, stream=None):
    _check(lib().gsa_signal_pad_reset(_ptr(pad), W, N, published_mask, _stream(stream)),
           "gsa_signal_pad_reset")


def gsa_gemv_allreduce(A_r, x, slots, pad, out, W, rank, N, K, B, stream=None):
    _check(lib().gsa_gemv_allreduce(_ptr(A_r), _ptr(x), _ptr(slots), _ptr(pad), _ptr(out),
                                    W, rank, N, K, B, _stream(stream)),
           "gsa_gemv_allreduce")


def gsa_gemv_allreduce_dtype(A_r, x, slots, pad, out, out_dtype, W, rank, N, K, B, stream=None):
    _check(lib().gsa_gemv_allreduce_dtype(_ptr(A_r), _ptr(x), _ptr(slots), _ptr(pad), _ptr(out),
                                          out_dtype, W, rank, N, K, B, _stream(stream)),
           "gsa_gemv_allreduce_dtype")


def gsa_gemv_allreduce_two_shot(A_r, x, slots, pad, gathered, out, W, rank, N, K, B,
                                stream=None):
    _check(lib().gsa_gemv_allreduce_two_shot(_ptr(A_r), _ptr(x), _ptr(slots), _ptr(pad),
                                             _ptr(gathered), _ptr(out), W, rank, N, K, B,
                                             _stream(stream)),
           "gsa_gemv_allreduce_two_shot")


def make_epilogue(y, bias=None, rms_weight=None, eps=1e-5, inv_rms=None):
    """A gsa_epilogue for device tensors: y (N x B, float32 or bfloat16),
    optional bias / rms_weight (N float32) and inv_rms (B float32)."""
    import torch
    if y.dtype == torch.float32:
        dt = GSA_DTYPE_F32
    elif y.dtype == torch.bfloat16:
        dt = GSA_DTYPE_BF16
    else:
        raise ValueError("y must be float32 or bfloat16")
    return gsa_epilogue(_ptr(bias), _ptr(rms_weight), float(eps), dt, _ptr(y), _ptr(inv_rms))


def gsa_gemv_allreduce_rmsnorm(A_r, x, slots, pad, out, W, rank, N, K, B, ep, stream=None):
    """ep: a gsa_epilogue (see make_epilogue), or None (rejected by the library)."""
    _check(lib().gsa_gemv_allreduce_rmsnorm(_ptr(A_r), _ptr(x), _ptr(slots), _ptr(pad),
                                            _ptr(out), W, rank, N, K, B,
                                            None if ep is None else ctypes.byref(ep),
                                            _stream(stream)),
           "gsa_gemv_allreduce_rmsnorm")


def gsa_peer_publish(slots, pad, values, W, peer, N, B, epoch, delay_us, stream=None):
    _check(lib().gsa_peer_publish(_ptr(slots), _ptr(pad), _ptr(values), W, peer, N, B, epoch,
                                  delay_us, _stream(stream)), "gsa_peer_publish")


def gsa_gemv_allreduce_rmsnorm_noalloc(A_r, x, slots, pad, out, W, rank, N, K, B, ep,
                                       stream=None):
    """As gsa_gemv_allreduce_rmsnorm, with the epilogue's scratch in the
    library's static device array (no allocation)."""
    _check(lib().gsa_gemv_allreduce_rmsnorm_noalloc(_ptr(A_r), _ptr(x), _ptr(slots), _ptr(pad),
                                                    _ptr(out), W, rank, N, K, B,
                                                    None if ep is None else ctypes.byref(ep),
                                                    _stream(stream)),
           "gsa_gemv_allreduce_rmsnorm_noalloc")


def gsa_bias_rmsnorm(out, N, B, ep, stream=None):
    """The epilogue of gsa_gemv_allreduce_rmsnorm as a kernel of its own,
    over an out (N x B float32) already written; ep: a gsa_epilogue."""
    _check(lib().gsa_bias_rmsnorm(_ptr(out), N, B, ctypes.byref(ep) if ep is not None else None,
                                  _stream(stream)),
           "gsa_bias_rmsnorm")


def gsa_signal_pad_status(pad, stream=None):
    code, tile, peer = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int()
    _check(lib().gsa_signal_pad_status(_ptr(pad), _stream(stream), ctypes.byref(code),
                                       ctypes.byref(tile), ctypes.byref(peer)),
           "gsa_signal_pad_status")
    return code.value, tile.value, peer.value


def gsa_set_wait_timeout_us(us):
    _check(lib().gsa_set_wait_timeout_us(us), "gsa_set_wait_timeout_us")


def gsa_strerror(code):
    return lib().gsa_strerror(code).decode()


class _DeviceArray:
    """Minimal __cuda_array_interface__ exporter for library-owned memory."""

    def __init__(self, ptr, shape, typestr):
        self.__cuda_array_interface__ = {
            "shape": tuple(int(s) for s in shape), "typestr": typestr,
            "data": (int(ptr), False), "version": 2, "strides": None}


def device_view(ptr, shape, dtype):
    """A torch tensor aliasing device memory at `ptr` (no copy, no ownership).
    Used to fill and read the library-owned slots and signal pad."""
    import numpy as np
    import torch
    typestr = {torch.float32: "<f4", torch.int32: "<i4", torch.uint8: "|u1",
               torch.int64: "<i8", torch.int16: "<i2"}[dtype]
    del np
    return torch.as_tensor(_DeviceArray(ptr, shape, typestr), device="cuda")


class SymmBuffer:
    """One symmetric buffer (W slots of N x B fp32, signal pad, the two-shot
    variant's gathered chunks), freed on close().  Convenience wrapper over
    gsa_symm_alloc / gsa_symm_free."""

    def __init__(self, W, N, B, slot_dtype=GSA_DTYPE_F32):
        self.W, self.N, self.B = W, N, B
        self.slot_dtype = slot_dtype
        self.handle = gsa_symm_alloc_dtype(W, N, B, slot_dtype)
        self.slots = gsa_symm_slots(self.handle)
        self.pad = gsa_symm_signal_pad(self.handle)
        self.gathered = gsa_symm_gathered(self.handle)
        self.row_stride = gsa_signal_pad_row_stride(N)
        self.tiles = (N + GSA_FLAG_TILE_ROWS - 1) // GSA_FLAG_TILE_ROWS

    def slots_view(self):
        """torch view (W, N, B) of the slots: float32, or int16 holding the
        bf16 bits for a buffer with bf16 slots."""
        import torch
        dt = torch.int16 if self.slot_dtype == GSA_DTYPE_BF16 else torch.float32
        return device_view(self.slots, (self.W, self.N, self.B), dt)

    def gathered_view(self):
        """torch float32 view (N, B) of the gathered chunks."""
        import torch
        return device_view(self.gathered, (self.N, self.B), torch.float32)

    def pad_view(self):
        """torch int32 view of the whole signal pad (header + 2W flag rows)."""
        import torch
        return device_view(self.pad, (GSA_PAD_HEADER_WORDS + 2 * self.W * self.row_stride,),
                           torch.int32)

    def _flag_rows(self, first):
        import numpy as np
        raw = self.pad_view().cpu().numpy().view(np.uint32)
        rows = raw[GSA_PAD_HEADER_WORDS:].reshape(2 * self.W, self.row_stride)
        return rows[first:first + self.W, flag_word(np.arange(self.tiles))].copy()

    def flags(self):
        """Host copy (numpy uint32, W x T) of the slot flags."""
        return self._flag_rows(0)

    def flags2(self):
        """Host copy (numpy uint32, W x T) of the reduced-chunk flags."""
        return self._flag_rows(self.W)

    def reset(self, published_mask, stream=None):
        gsa_signal_pad_reset(self.pad, self.W, self.N, published_mask, stream)

    def status(self, stream=None):
        return gsa_signal_pad_status(self.pad, stream)

    def close(self):
        if self.handle:
            gsa_symm_free(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


# --- mixture of experts: expert GEMM fused with the combine all-to-all ---

def gsa_a2a_pad_words(W, ne, H):
    return lib().gsa_a2a_pad_words(W, ne, H)


def gsa_a2a_alloc(W, ne, H, rows_out):
    h = ctypes.c_void_p()
    _check(lib().gsa_a2a_alloc(W, ne, H, rows_out, ctypes.byref(h)), "gsa_a2a_alloc")
    return h.value


def gsa_a2a_free(h):
    _check(lib().gsa_a2a_free(h), "gsa_a2a_free")


def gsa_a2a_buffers(h):
    p = lib().gsa_a2a_buffers(h)
    if not p:
        raise GsaError(GSA_EINVAL, "gsa_a2a_buffers")
    return p


def gsa_a2a_signal_pads(h):
    p = lib().gsa_a2a_signal_pads(h)
    if not p:
        raise GsaError(GSA_EINVAL, "gsa_a2a_signal_pads")
    return p


def gsa_a2a_reset(pads, W, ne, H, published_mask, stream=None):
    _check(lib().gsa_a2a_reset(_ptr(pads), W, ne, H, published_mask, _stream(stream)),
           "gsa_a2a_reset")


def gsa_moe_gemm_all_to_all(X, Wd, splits, dst_off, bufs, pads, W, rank, ne, H, F, rows_in,
                            rows_out, stream=None):
    _check(lib().gsa_moe_gemm_all_to_all(_ptr(X), _ptr(Wd), _ptr(splits), _ptr(dst_off),
                                         _ptr(bufs), _ptr(pads), W, rank, ne, H, F, rows_in,
                                         rows_out, _stream(stream)),
           "gsa_moe_gemm_all_to_all")


def gsa_a2a_status(pads, rank, stream=None):
    """(code, tile, peer) of rank `rank`'s pad; synchronizes the stream."""
    c, t, p = ctypes.c_int(), ctypes.c_int64(), ctypes.c_int()
    _check(lib().gsa_a2a_status(_ptr(pads), rank, _stream(stream), ctypes.byref(c),
                                ctypes.byref(t), ctypes.byref(p)), "gsa_a2a_status")
    return c.value, t.value, p.value


class A2ABuffer:
    """W combine buffers (rows_out x H fp32 each) and W signal pads, freed on
    close().  Convenience wrapper over gsa_a2a_alloc / gsa_a2a_free."""

    def __init__(self, W, ne, H, rows_out):
        self.W, self.ne, self.H, self.rows_out = W, ne, H, rows_out
        self.handle = gsa_a2a_alloc(W, ne, H, rows_out)
        self.bufs = gsa_a2a_buffers(self.handle)
        self.pads = gsa_a2a_signal_pads(self.handle)
        self.pad_words = gsa_a2a_pad_words(W, ne, H)
        self.row_stride = (self.pad_words - GSA_PAD_HEADER_WORDS) // (W * ne)
        self.tiles = (H + GSA_MOE_TILE_ROWS - 1) // GSA_MOE_TILE_ROWS

    def bufs_view(self):
        """torch float32 view (W, rows_out, H) of the combine buffers."""
        import torch
        return device_view(self.bufs, (self.W, self.rows_out, self.H), torch.float32)

    def pads_view(self):
        """torch int32 view (W, pad_words) of the signal pads."""
        import torch
        return device_view(self.pads, (self.W, self.pad_words), torch.int32)

    def flags(self):
        """Host copy (numpy uint32, W pads x W sources x ne x tiles)."""
        import numpy as np
        raw = self.pads_view().cpu().numpy().view(np.uint32)
        rows = raw[:, GSA_PAD_HEADER_WORDS:].reshape(self.W, self.W, self.ne, self.row_stride)
        return rows[..., :self.tiles].copy()

    def reset(self, published_mask, stream=None):
        gsa_a2a_reset(self.pads, self.W, self.ne, self.H, published_mask, stream)

    def status(self, rank, stream=None):
        return gsa_a2a_status(self.pads, rank, stream)

    def close(self):
        if self.handle:
            gsa_a2a_free(self.handle)
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()
