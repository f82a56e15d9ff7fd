"""ctypes binding of librssm.so (C ABI in include/rssm.h).

Argument marshalling only: every step of the decode path runs in the HIP
kernels behind the C ABI.  PyTorch provides device memory and the current
stream; there is no fallback of any kind -- if the library is missing, every
entry point raises.

Entry points keep the C names: :func:`rssm_mamba2_step`, :func:`rssm_gdn_step`,
:func:`rssm_commit`, :func:`rssm_verify`, :func:`rssm_rollback`,
:func:`rssm_eager_step`, :func:`rssm_status`, :func:`rssm_strerror`,
:func:`rssm_abi_version`.  :class:`Layer` allocates one layer's state tensors
and fills the ``rssm_layer`` descriptor.
"""
import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "librssm.so")

RSSM_OK, RSSM_EINVAL, RSSM_EUNSUPPORTED, RSSM_EALIGN, RSSM_ERANGE, RSSM_EHIP = 0, -1, -2, -3, -4, -5
STATUS_OVERFLOW, STATUS_ROLLBACK, STATUS_NONFINITE, STATUS_INDEX = 1, 2, 4, 8
RSSM_MAMBA2, RSSM_GDN = 1, 2
RSSM_F32, RSSM_DUAL, RSSM_SHARED = 0, 1, 2
RSSM_LP_NONE, RSSM_BF16, RSSM_E4M3 = 0, 1, 2
RSSM_ABI_VERSION = 11
RSSM_ARRIVE_STRIDE = 32   # uint32 elements between two sequences' arrival counters
RSSM_NOALLOC_MAX_BATCH = 4096   # sequences rssm_mamba2_step_noalloc serves
RSSM_LAYER_INDEX_READONLY = 1   # rssm_layer.flags: indices read, never written

_vp = ctypes.c_void_p
_i32 = ctypes.c_int32


class rssm_layer(ctypes.Structure):
    _fields_ = [("kind", _i32), ("scheme", _i32), ("lp_dtype", _i32),
                ("batch", _i32), ("nheads", _i32), ("ngroups", _i32),
                ("dim_v", _i32), ("dim_k", _i32), ("capacity", _i32),
                ("flags", _i32),
                ("ckpt", _vp), ("ckpt_lp", _vp), ("lp_scale", _vp),
                ("A", _vp), ("D", _vp), ("ring", _vp * 4),
                ("ckpt_pos", _vp), ("len", _vp), ("arrive", _vp), ("status", _vp)]


class rssm_inputs(ctypes.Structure):
    _fields_ = [("x", _vp), ("B", _vp), ("C", _vp), ("dt", _vp),
                ("q", _vp), ("k", _vp), ("v", _vp), ("alpha", _vp), ("beta", _vp)]


class RssmError(RuntimeError):
    def __init__(self, code, where):
        super().__init__(f"{where}: {rssm_strerror(code)} (code {code})")
        self.code = code


_lib = None


def lib():
    """Open librssm.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with "
                "`python -m linear_attention_decode_replayssm_amd.build` "
                "(or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.rssm_abi_version.restype = ctypes.c_int
        if L.rssm_abi_version() != RSSM_ABI_VERSION:   # before any other symbol is looked up
            raise RuntimeError(f"{LIB_PATH} implements ABI {L.rssm_abi_version()}, this binding "
                               f"{RSSM_ABI_VERSION}: rebuild the library")
        P = ctypes.POINTER
        L.rssm_mamba2_step.argtypes = [P(rssm_layer), _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp]
        L.rssm_mamba2_step_noalloc.argtypes = [P(rssm_layer), _vp, _vp, _vp, _vp, _vp,
                                               ctypes.c_int, _vp]
        L.rssm_gdn_step.argtypes = [P(rssm_layer), _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_int, _vp]
        L.rssm_commit.argtypes = [P(rssm_layer), _vp, ctypes.c_int, _vp]
        L.rssm_verify.argtypes = [P(rssm_layer), ctypes.c_int, P(rssm_inputs), _vp, _vp]
        L.rssm_verify_commit.argtypes = [P(rssm_layer), ctypes.c_int, P(rssm_inputs), _vp,
                                         ctypes.c_int, _vp]
        L.rssm_rollback.argtypes = [P(rssm_layer), _vp, _vp]
        L.rssm_rollback_verify_commit.argtypes = [P(rssm_layer), _vp, ctypes.c_int,
                                                  P(rssm_inputs), _vp, ctypes.c_int, _vp]
        L.rssm_verify_tree.argtypes = [P(rssm_layer), ctypes.c_int, P(ctypes.c_int32),
                                       P(rssm_inputs), _vp, _vp]
        L.rssm_verify_tree_commit.argtypes = [P(rssm_layer), ctypes.c_int, P(ctypes.c_int32),
                                              P(rssm_inputs), _vp, ctypes.c_int, _vp]
        L.rssm_append_path.argtypes = [P(rssm_layer), ctypes.c_int, _vp, _vp, ctypes.c_int,
                                       P(rssm_inputs), _vp]
        L.rssm_prefill.argtypes = [P(rssm_layer), ctypes.c_int, P(rssm_inputs), _vp, _vp, _vp]
        L.rssm_eager_step.argtypes = [P(rssm_layer), P(rssm_inputs), _vp, _vp]
        L.rssm_eager_spec_round.argtypes = [P(rssm_layer), ctypes.c_int, P(rssm_inputs), _vp, _vp,
                                            _vp, _vp]
        L.rssm_eager_spec_accept.argtypes = [P(rssm_layer), ctypes.c_int, _vp, _vp, _vp]
        L.rssm_probe_stream.argtypes = [_vp, _vp, _vp, ctypes.c_int64, _vp]
        L.rssm_probe_stream_tiles.argtypes = [_vp, _vp, _vp, ctypes.c_int64, ctypes.c_int32,
                                              ctypes.c_int32, _vp]
        L.rssm_status.argtypes = [P(rssm_layer), P(ctypes.c_uint32), _vp]
        L.rssm_strerror.argtypes = [ctypes.c_int]
        L.rssm_strerror.restype = ctypes.c_char_p
        for f in ("rssm_mamba2_step", "rssm_gdn_step", "rssm_commit", "rssm_verify",
                  "rssm_rollback", "rssm_eager_step", "rssm_status", "rssm_verify_tree",
                  "rssm_append_path", "rssm_prefill", "rssm_eager_spec_round",
                  "rssm_eager_spec_accept", "rssm_probe_stream", "rssm_probe_stream_tiles",
                  "rssm_verify_commit", "rssm_verify_tree_commit", "rssm_mamba2_step_noalloc",
                  "rssm_rollback_verify_commit"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(t):
    """Device address of a tensor (or None / an int address)."""
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


def _check(rc, where):
    if rc != RSSM_OK:
        raise RssmError(rc, where)
    return rc


def _desc(layer):
    return layer.desc if isinstance(layer, Layer) else layer


def rssm_abi_version() -> int:
    return lib().rssm_abi_version()


def rssm_strerror(code: int) -> str:
    return lib().rssm_strerror(int(code)).decode()


def rssm_mamba2_step(layer, x, B, C, dt, y, commit_after=False, stream=None, check=True):
    rc = lib().rssm_mamba2_step(ctypes.byref(_desc(layer)), _ptr(x), _ptr(B), _ptr(C), _ptr(dt),
                                _ptr(y), int(bool(commit_after)), _stream(stream))
    return _check(rc, "rssm_mamba2_step") if check else rc


def rssm_mamba2_step_noalloc(layer, x, B, C, dt, y, commit_after=False, stream=None, check=True):
    rc = lib().rssm_mamba2_step_noalloc(ctypes.byref(_desc(layer)), _ptr(x), _ptr(B), _ptr(C),
                                        _ptr(dt), _ptr(y), int(bool(commit_after)),
                                        _stream(stream))
    return _check(rc, "rssm_mamba2_step_noalloc") if check else rc


def rssm_gdn_step(layer, q, k, v, alpha, beta, o, commit_after=False, stream=None, check=True):
    rc = lib().rssm_gdn_step(ctypes.byref(_desc(layer)), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha),
                             _ptr(beta), _ptr(o), int(bool(commit_after)), _stream(stream))
    return _check(rc, "rssm_gdn_step") if check else rc


def rssm_commit(layer, mask=None, min_len=0, stream=None, check=True):
    rc = lib().rssm_commit(ctypes.byref(_desc(layer)), _ptr(mask), int(min_len), _stream(stream))
    return _check(rc, "rssm_commit") if check else rc


def make_inputs(x=None, B=None, C=None, dt=None, q=None, k=None, v=None, alpha=None, beta=None):
    return rssm_inputs(_ptr(x), _ptr(B), _ptr(C), _ptr(dt), _ptr(q), _ptr(k), _ptr(v),
                       _ptr(alpha), _ptr(beta))


def rssm_verify(layer, n_pos, inputs, out, stream=None, check=True):
    if isinstance(inputs, dict):
        inputs = make_inputs(**inputs)
    rc = lib().rssm_verify(ctypes.byref(_desc(layer)), int(n_pos), ctypes.byref(inputs), _ptr(out),
                           _stream(stream))
    return _check(rc, "rssm_verify") if check else rc


def rssm_verify_commit(layer, n_pos, inputs, out, min_len, stream=None, check=True):
    """rssm_verify, first folding the buffer of every sequence with len >= min_len
    into its checkpoint from the same state read (fp32 checkpoints)."""
    if isinstance(inputs, dict):
        inputs = make_inputs(**inputs)
    rc = lib().rssm_verify_commit(ctypes.byref(_desc(layer)), int(n_pos), ctypes.byref(inputs),
                                  _ptr(out), int(min_len), _stream(stream))
    return _check(rc, "rssm_verify_commit") if check else rc


def rssm_rollback_verify_commit(layer, n_reject, n_pos, inputs, out, min_len, stream=None,
                                check=True):
    """rssm_rollback(layer, n_reject) then rssm_verify_commit, in one launch;
    n_reject: device int32 [batch]."""
    if isinstance(inputs, dict):
        inputs = make_inputs(**inputs)
    rc = lib().rssm_rollback_verify_commit(ctypes.byref(_desc(layer)), _ptr(n_reject), int(n_pos),
                                           ctypes.byref(inputs), _ptr(out), int(min_len),
                                           _stream(stream))
    return _check(rc, "rssm_rollback_verify_commit") if check else rc


def rssm_verify_tree(layer, parent, inputs, out, stream=None, check=True):
    """parent: host sequence of int (parent[j] < j, -1 = below the buffer tail)."""
    if isinstance(inputs, dict):
        inputs = make_inputs(**inputs)
    n = len(parent)
    arr = (ctypes.c_int32 * max(n, 1))(*[int(p) for p in parent])
    rc = lib().rssm_verify_tree(ctypes.byref(_desc(layer)), n, arr, ctypes.byref(inputs),
                                _ptr(out), _stream(stream))
    return _check(rc, "rssm_verify_tree") if check else rc


def rssm_verify_tree_commit(layer, parent, inputs, out, min_len, stream=None, check=True):
    """rssm_verify_tree, first folding the buffer of every sequence with
    len >= min_len into its checkpoint from the same state read (fp32
    checkpoints); nothing is appended."""
    if isinstance(inputs, dict):
        inputs = make_inputs(**inputs)
    n = len(parent)
    arr = (ctypes.c_int32 * max(n, 1))(*[int(p) for p in parent])
    rc = lib().rssm_verify_tree_commit(ctypes.byref(_desc(layer)), n, arr, ctypes.byref(inputs),
                                       _ptr(out), int(min_len), _stream(stream))
    return _check(rc, "rssm_verify_tree_commit") if check else rc


def rssm_append_path(layer, n_nodes, path, path_len, inputs, stream=None, check=True):
    """path: device int32 [batch][depth]; path_len: device int32 [batch]."""
    if isinstance(inputs, dict):
        inputs = make_inputs(**inputs)
    depth = int(path.shape[1]) if hasattr(path, "shape") else int(path[1])
    rc = lib().rssm_append_path(ctypes.byref(_desc(layer)), int(n_nodes), _ptr(path),
                                _ptr(path_len), depth, ctypes.byref(inputs), _stream(stream))
    return _check(rc, "rssm_append_path") if check else rc


def rssm_prefill(layer, n_tok, inputs, out=None, mask=None, stream=None, check=True):
    """inputs: leading [n_tok]; out: [n_tok][batch][H][dim_v] or None; mask:
    device uint8 [batch] or None."""
    if isinstance(inputs, dict):
        inputs = make_inputs(**inputs)
    rc = lib().rssm_prefill(ctypes.byref(_desc(layer)), int(n_tok), ctypes.byref(inputs),
                            _ptr(out), _ptr(mask), _stream(stream))
    return _check(rc, "rssm_prefill") if check else rc


def rssm_rollback(layer, n_reject, stream=None, check=True):
    rc = lib().rssm_rollback(ctypes.byref(_desc(layer)), _ptr(n_reject), _stream(stream))
    return _check(rc, "rssm_rollback") if check else rc


def rssm_eager_step(layer, inputs, out, stream=None, check=True):
    if isinstance(inputs, dict):
        inputs = make_inputs(**inputs)
    rc = lib().rssm_eager_step(ctypes.byref(_desc(layer)), ctypes.byref(inputs), _ptr(out),
                               _stream(stream))
    return _check(rc, "rssm_eager_step") if check else rc


def rssm_eager_spec_round(layer, n_pos, inputs, out, slots, cur, stream=None, check=True):
    """slots: device fp32 [n_pos + 1][batch][H][dim_v][dim_k]; cur: device int32 [batch]."""
    if isinstance(inputs, dict):
        inputs = make_inputs(**inputs)
    rc = lib().rssm_eager_spec_round(ctypes.byref(_desc(layer)), int(n_pos), ctypes.byref(inputs),
                                     _ptr(out), _ptr(slots), _ptr(cur), _stream(stream))
    return _check(rc, "rssm_eager_spec_round") if check else rc


def rssm_eager_spec_accept(layer, n_pos, cur, n_accept, stream=None, check=True):
    rc = lib().rssm_eager_spec_accept(ctypes.byref(_desc(layer)), int(n_pos), _ptr(cur),
                                      _ptr(n_accept), _stream(stream))
    return _check(rc, "rssm_eager_spec_accept") if check else rc


def rssm_probe_stream(src, dst, sink, nbytes, stream=None, check=True):
    """Streaming probe (measurement utility): copy src -> dst, or read src and
    write one float per wave to sink when dst is None."""
    rc = lib().rssm_probe_stream(_ptr(src), _ptr(dst), _ptr(sink), int(nbytes), _stream(stream))
    return _check(rc, "rssm_probe_stream") if check else rc


def rssm_probe_stream_tiles(src, dst, sink, nbytes, tile_bytes, write_all=True, stream=None,
                            check=True):
    """As rssm_probe_stream with a workgroup tile of tile_bytes (32768 or 4096).
    The read-only pass writes each wave's XOR fold to sink (nbytes /
    (tile_bytes / 4) floats) when write_all, else (timing) almost never."""
    rc = lib().rssm_probe_stream_tiles(_ptr(src), _ptr(dst), _ptr(sink), int(nbytes),
                                       int(tile_bytes), int(bool(write_all)), _stream(stream))
    return _check(rc, "rssm_probe_stream_tiles") if check else rc


def rssm_status(layer, stream=None) -> int:
    bits = ctypes.c_uint32(0)
    _check(lib().rssm_status(ctypes.byref(_desc(layer)), ctypes.byref(bits), _stream(stream)),
           "rssm_status")
    return bits.value


class Layer:
    """One layer's caller-owned device state, plus its ``rssm_layer`` descriptor.

    Tensors (torch, on ``device``): ``ckpt`` fp32 [b,H,dv,dk] (None under
    SHARED), ``ckpt_lp`` (uint16 bf16 bits / uint8 E4M3 codes, None under F32),
    ``lp_scale`` fp32 [b,H] (E4M3), ``A``/``D`` fp32 [H] (Mamba-2), ``rings``,
    ``ckpt_pos`` int64 [b], ``len`` int32 [b], ``arrive`` int32 [b * RSSM_ARRIVE_STRIDE] (zero),
    ``status`` int32 [1].
    """

    def __init__(self, kind, batch, nheads, dim_v, dim_k, capacity, ngroups=1,
                 scheme=RSSM_F32, lp_dtype=RSSM_LP_NONE, device="cuda"):
        import torch
        self.kind, self.scheme, self.lp_dtype = kind, scheme, lp_dtype
        self.flags = 0
        self.batch, self.nheads, self.ngroups = batch, nheads, ngroups
        self.dim_v, self.dim_k, self.capacity = dim_v, dim_k, capacity
        f32 = dict(dtype=torch.float32, device=device)
        shape = (batch, nheads, dim_v, dim_k)
        self.ckpt = torch.zeros(shape, **f32) if scheme != RSSM_SHARED else None
        self.ckpt_lp = None
        self.lp_scale = None
        if scheme != RSSM_F32:
            dt = torch.int16 if lp_dtype == RSSM_BF16 else torch.uint8
            self.ckpt_lp = torch.zeros(shape, dtype=dt, device=device)
            if lp_dtype == RSSM_E4M3:
                self.lp_scale = torch.ones((batch, nheads), **f32)
        self.A = self.D = None
        if kind == RSSM_MAMBA2:
            self.A = torch.zeros(nheads, **f32)
            self.D = torch.zeros(nheads, **f32)
            self.rings = [torch.zeros((batch, nheads, capacity, dim_v), **f32),
                          torch.zeros((batch, ngroups, capacity, dim_k), **f32),
                          torch.zeros((batch, nheads, capacity), **f32)]
        else:
            self.rings = [torch.zeros((batch, nheads, capacity, dim_k), **f32),
                          torch.zeros((batch, nheads, capacity, dim_v), **f32),
                          torch.zeros((batch, nheads, capacity), **f32),
                          torch.zeros((batch, nheads, capacity), **f32)]
        self.ckpt_pos = torch.zeros(batch, dtype=torch.int64, device=device)
        self.len = torch.zeros(batch, dtype=torch.int32, device=device)
        self.arrive = torch.zeros(max(batch, 1) * RSSM_ARRIVE_STRIDE, dtype=torch.int32,
                                  device=device)
        self.status = torch.zeros(1, dtype=torch.int32, device=device)
        self.refresh()

    def refresh(self):
        """(Re)build the descriptor from the current tensors."""
        rings = (_vp * 4)(*([_ptr(r) for r in self.rings] + [None] * (4 - len(self.rings))))
        self.desc = rssm_layer(self.kind, self.scheme, self.lp_dtype, self.batch, self.nheads,
                               self.ngroups, self.dim_v, self.dim_k, self.capacity, self.flags,
                               _ptr(self.ckpt), _ptr(self.ckpt_lp), _ptr(self.lp_scale),
                               _ptr(self.A), _ptr(self.D), rings, _ptr(self.ckpt_pos),
                               _ptr(self.len), _ptr(self.arrive), _ptr(self.status))
        return self.desc

    def share_indices(self, owner, readonly=True):
        """Use `owner`'s ckpt_pos / len arrays: one set of buffer indices for
        layers that advance together.  readonly sets RSSM_LAYER_INDEX_READONLY
        (every layer of the stack but the one whose calls move the indices)."""
        self.ckpt_pos, self.len = owner.ckpt_pos, owner.len
        self.flags = RSSM_LAYER_INDEX_READONLY if readonly else 0
        return self.refresh()

    @classmethod
    def mamba2(cls, batch, nheads, ngroups, headdim, dstate, capacity, scheme=RSSM_F32,
               lp_dtype=RSSM_LP_NONE, device="cuda"):
        return cls(RSSM_MAMBA2, batch, nheads, headdim, dstate, capacity, ngroups=ngroups,
                   scheme=scheme, lp_dtype=lp_dtype, device=device)

    @classmethod
    def gdn(cls, batch, nheads, dk, dv, capacity, scheme=RSSM_F32, lp_dtype=RSSM_LP_NONE,
            device="cuda"):
        return cls(RSSM_GDN, batch, nheads, dv, dk, capacity, scheme=scheme, lp_dtype=lp_dtype,
                   device=device)
